"""Shared helpers for the parity tests: tolerances derived from the arithmetic.

Output tolerance (the reference value y64 is the oracle's fp64 dequantization):
  * fp16 / bf16 outputs: |y - y64| <= 1 ulp of the output format at y64, plus the
    worst-case error of an fp32 evaluation, (G + 2) * 2^-24 * mag, where mag is the
    sum of the magnitudes of the terms (mag = |y64| for per-channel, G = 1).
  * fp32 outputs: |y - y64| <= 1e-5 * max(|y64|, mag).
Codes, scales and int32 accumulators are compared bit for bit.
"""
import numpy as np

F16_MIN_NORMAL = 2.0 ** -14
BF16_MIN_NORMAL = 2.0 ** -126


def ulp(y64: np.ndarray, fmt: str) -> np.ndarray:
    a = np.abs(y64)
    if fmt == "f16":
        e = np.floor(np.log2(np.maximum(a, F16_MIN_NORMAL)))
        return np.exp2(e - 10)
    if fmt == "bf16":
        e = np.floor(np.log2(np.maximum(a, BF16_MIN_NORMAL)))
        return np.exp2(e - 7)
    raise ValueError(fmt)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_output(y_gpu: np.ndarray, fmt: str, y64: np.ndarray, mag: np.ndarray, G: int = 1,
                 what: str = ""):
    """y_gpu: float16 array (fmt f16), uint16 bf16 bits (fmt bf16) or float32 (fmt f32)."""
    if fmt == "f16":
        yg = y_gpu.astype(np.float64)
    elif fmt == "bf16":
        yg = bf16_bits_to_f64(y_gpu)
    else:
        yg = y_gpu.astype(np.float64)
    err = np.abs(yg - y64)
    if fmt == "f32":
        tol = 1e-5 * np.maximum(np.abs(y64), mag)
    else:
        tol = ulp(y64, fmt) + (G + 2) * 2.0 ** -24 * mag
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outputs out of tolerance; first at {tuple(i)}: "
            f"gpu={yg[tuple(i)]!r} ref={y64[tuple(i)]!r} tol={tol[tuple(i)]!r}")
    if fmt == "f16":
        # rounding mode: almost every output must equal the correctly rounded reference (an
        # fp32 evaluation rounds differently from the fp64 value at a few outputs; on small
        # outputs one or two of them are more than 1 %)
        miss = int((y_gpu != y64.astype(np.float16)).sum())
        assert miss <= max(2, 0.01 * y_gpu.size), f"{what}: {miss} of {y_gpu.size} fp16 outputs are not RNE(y64)"
    return float(err.max()) if err.size else 0.0


def bf16_rne_bits(f32: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def check_exact(y_gpu: np.ndarray, fmt: str, y32: np.ndarray, what: str = ""):
    """Bit-for-bit equality with the oracle's fp32 evaluation rounded once to the output
    format (fp16 by numpy's round-to-nearest-even conversion, bf16 by bf16_rne_bits, fp32
    as is). y_gpu: float16 (f16), uint16 bf16 bits (bf16) or float32 (f32)."""
    if fmt == "f16":
        got, ref = y_gpu.view(np.uint16), y32.astype(np.float16).view(np.uint16)
    elif fmt == "bf16":
        got, ref = y_gpu.view(np.uint16), bf16_rne_bits(y32)
    elif fmt == "f32":
        got, ref = y_gpu.view(np.uint32), np.ascontiguousarray(y32, dtype=np.float32).view(np.uint32)
    else:
        raise ValueError(fmt)
    bad = got != ref
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs differ from the oracle's fp32 "
                             f"evaluation; first at {i}: gpu bits {int(got[i]):#x}, oracle {int(ref[i]):#x}")
