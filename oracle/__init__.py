"""CPU oracle for the fused per-token-quantize -> int8 GEMM -> dequant linear layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The GPU library never
imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C loops, compiled with gcc at
``-O2 -fno-fast-math -ffp-contract=off``, OpenMP over rows only); this module
builds it, loads it with ctypes and wraps it for numpy arrays. Every function
cites the passage of the pages it follows in ``oracle.c``.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, exact rational arithmetic, brute force on tiny inputs and
hand-worked fixtures under ``tests/golden/``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc). Returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # W8A8_ORACLE_LIB: another build of oracle.c (the sanitizer tests load one built
        # with AddressSanitizer and UndefinedBehaviorSanitizer)
        path = os.environ.get("W8A8_ORACLE_LIB")
        if not path:
            path = build(force=False)
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_quantize_per_token.argtypes = [vp, i32, i64, i64, i64, vp, vp]
        lib.oracle_quantize_weight.argtypes = [vp, i64, i64, i32, i32, vp, vp]
        lib.oracle_unpack_int4.argtypes = [vp, i64, i64, vp]
        lib.oracle_gemm_i32.argtypes = [vp, vp, i64, i64, i64, vp]
        lib.oracle_group_acc.argtypes = [vp, vp, i64, i64, i64, i32, vp]
        lib.oracle_dequant_pc.argtypes = [vp, vp, vp, i64, i64, vp]
        lib.oracle_dequant_pg.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp]
        lib.oracle_dequant_pc_f32.argtypes = [vp, vp, vp, i64, i64, vp]
        lib.oracle_dequant_pg_f32.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        lib.oracle_mv.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, i32, vp, vp]
        lib.oracle_quantize_weight_clipped.argtypes = [vp, i64, i64, i32, i32, ctypes.c_float, vp, vp]
        lib.oracle_sdpa_decode.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, ctypes.c_double, vp, vp, vp]
        lib.oracle_rmsnorm_quantize.argtypes = [vp, i32, vp, i32, ctypes.c_double, i64, i64, i64, vp, vp, vp]
        lib.oracle_swiglu_quantize.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, vp]
        lib.oracle_exp_steps.argtypes = [vp, i64, vp]
        for f in (lib.oracle_quantize_per_token, lib.oracle_quantize_weight, lib.oracle_unpack_int4,
                  lib.oracle_gemm_i32, lib.oracle_group_acc, lib.oracle_dequant_pc,
                  lib.oracle_dequant_pg, lib.oracle_dequant_pc_f32, lib.oracle_dequant_pg_f32, lib.oracle_mv, lib.oracle_quantize_weight_clipped,
                  lib.oracle_sdpa_decode, lib.oracle_rmsnorm_quantize, lib.oracle_swiglu_quantize,
                  lib.oracle_exp_steps):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc == 1:
        raise ValueError(f"oracle {what}: bad argument")
    if rc == 2:
        raise OverflowError(f"oracle {what}: int32 accumulator overflow")
    if rc != 0:
        raise RuntimeError(f"oracle {what}: status {rc}")


def quantize_per_token(x: np.ndarray):
    """x: float16 (or a bf16 bit pattern array tagged via ``bf16=True`` wrapper) [M, K].

    Returns (x_q int8 [M, K], s_x float32 [M]).
    """
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        bits, is_bf16 = x.view(np.uint16), 0
    else:
        raise TypeError("quantize_per_token expects float16; use quantize_per_token_bf16 for bf16 bits")
    return _qpt(bits, is_bf16)


def quantize_per_token_bf16(bits: np.ndarray):
    """Like quantize_per_token, for a uint16 array holding bfloat16 bit patterns."""
    return _qpt(np.ascontiguousarray(bits, dtype=np.uint16), 1)


def _qpt(bits: np.ndarray, is_bf16: int):
    M, K = bits.shape
    xq = np.empty((M, K), np.int8)
    sx = np.empty((M,), np.float32)
    _check(_load().oracle_quantize_per_token(_p(bits), is_bf16, M, K, K, _p(xq), _p(sx)),
           "quantize_per_token")
    return xq, sx


def rmsnorm_quantize(x: np.ndarray, g: np.ndarray, eps: float, x_bf16: bool = False, g_bf16: bool = False):
    """RMSNorm with the per-token quantization folded in (oracle.c cites the passages).

    x [M, K] and g [K]: float16 arrays, or uint16 arrays of bfloat16 bit patterns with the
    matching flag set. Returns (x_q int8 [M, K], s_u float32 [M], s_x float64 [M]): x_q and
    s_u are the symmetric quantization of u = x * g (one fp32 multiply per element), and
    s_x = s_u / sqrt(mean(x^2) + eps), so s_x * x_q approximates the normalized row.
    """
    xb = np.ascontiguousarray(x).view(np.uint16)
    gb = np.ascontiguousarray(g).view(np.uint16)
    M, K = xb.shape
    assert gb.shape == (K,)
    xq = np.empty((M, K), np.int8)
    su = np.empty((M,), np.float32)
    sx = np.empty((M,), np.float64)
    _check(_load().oracle_rmsnorm_quantize(_p(xb), int(x_bf16), _p(gb), int(g_bf16), float(eps), M, K, K,
                                           _p(xq), _p(su), _p(sx)), "rmsnorm_quantize")
    return xq, su, sx


def swiglu_quantize(gate: np.ndarray, up: np.ndarray, bf16: bool = False):
    """SwiGLU with the per-token quantization folded in (oracle.c cites the passages).

    gate, up [M, I]: float16 arrays, or (bf16=True) uint16 arrays of bfloat16 bit patterns
    (row strides may differ: views into one wider array work). Returns (x_q int8 [M, I],
    s_x float32 [M], h float32 [M, I]) with h = silu(gate) * up evaluated in the specified
    fp32 steps and x_q, s_x its per-token quantization."""
    gb = np.asarray(gate).view(np.uint16)
    ub = np.asarray(up).view(np.uint16)
    if gb.strides[1] != 2 or ub.strides[1] != 2:
        gb, ub = np.ascontiguousarray(gb), np.ascontiguousarray(ub)
    M, I = gb.shape
    assert ub.shape == (M, I)
    xq = np.empty((M, I), np.int8)
    sx = np.empty((M,), np.float32)
    h = np.empty((M, I), np.float32)
    _check(_load().oracle_swiglu_quantize(_p(gb), _p(ub), int(bf16), M, I, gb.strides[0] // 2, ub.strides[0] // 2,
                                          _p(xq), _p(sx), _p(h)), "swiglu_quantize")
    return xq, sx, h


def exp_steps(x: np.ndarray) -> np.ndarray:
    """The fp32 exp evaluation the SwiGLU producer specifies (oracle.c, exp_steps)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    _check(_load().oracle_exp_steps(_p(x), x.size, _p(y)), "exp_steps")
    return y


def quantize_weight(W: np.ndarray, bits: int = 8, group_size: int = 0):
    """W float32 [N, K] -> (w_q, s_w).

    bits 8: w_q int8 [N, K]; bits 4: w_q uint8 [N, K/2] (even k in low nibble).
    s_w float32 [N] (group_size 0) or [N, K/group_size].
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    wq = np.empty((N, K) if bits == 8 else (N, K // 2), np.int8 if bits == 8 else np.uint8)
    sw = np.empty((N,) if group_size == 0 else (N, K // group_size), np.float32)
    _check(_load().oracle_quantize_weight(_p(W), N, K, bits, group_size, _p(wq), _p(sw)),
           "quantize_weight")
    return wq, sw


def quantize_weight_clipped(W: np.ndarray, bits: int, group_size: int, pct: float):
    """quantize_weight with each run's scale taken from the pct-th percentile of |W| (linear
    interpolation between order statistics) instead of the maximum; pct in (0, 100]."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    wq = np.empty((N, K) if bits == 8 else (N, K // 2), np.int8 if bits == 8 else np.uint8)
    sw = np.empty((N,) if group_size == 0 else (N, K // group_size), np.float32)
    _check(_load().oracle_quantize_weight_clipped(_p(W), N, K, bits, group_size, float(pct), _p(wq), _p(sw)),
           "quantize_weight_clipped")
    return wq, sw


def unpack_int4(packed: np.ndarray, K: int):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    wq = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack_int4(_p(packed), N, K, _p(wq)), "unpack_int4")
    return wq


def gemm_i32(x_q: np.ndarray, w_q: np.ndarray):
    """acc int32 [M, N] = x_q [M, K] . w_q [N, K]^T, exact."""
    x_q = np.ascontiguousarray(x_q, dtype=np.int8)
    w_q = np.ascontiguousarray(w_q, dtype=np.int8)
    M, K = x_q.shape
    N = w_q.shape[0]
    assert w_q.shape[1] == K
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_gemm_i32(_p(x_q), _p(w_q), M, N, K, _p(acc)), "gemm_i32")
    return acc


def group_acc(x_q: np.ndarray, w_q: np.ndarray, group_size: int):
    """acc_g int32 [M, N, G]: the integer product restricted to each K-group."""
    x_q = np.ascontiguousarray(x_q, dtype=np.int8)
    w_q = np.ascontiguousarray(w_q, dtype=np.int8)
    M, K = x_q.shape
    N = w_q.shape[0]
    G = K // group_size
    acc = np.empty((M, N, G), np.int32)
    _check(_load().oracle_group_acc(_p(x_q), _p(w_q), M, N, K, group_size, _p(acc)), "group_acc")
    return acc


def dequant_pc(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray):
    """fp64 y [M, N] = (acc * s_x[m]) * s_w[n]."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _check(_load().oracle_dequant_pc(_p(acc), _p(s_x), _p(s_w), M, N, _p(y)), "dequant_pc")
    return y


def dequant_pg(acc_g: np.ndarray, s_x: np.ndarray, s_w: np.ndarray):
    """fp64 (y, mag) [M, N]: y = s_x * sum_g s_w[n,g] * acc_g; mag = sum of |terms|."""
    acc_g = np.ascontiguousarray(acc_g, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    M, N, G = acc_g.shape
    y = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    _check(_load().oracle_dequant_pg(_p(acc_g), _p(s_x), _p(s_w), M, N, G, _p(y), _p(mag)),
           "dequant_pg")
    return y, mag


def dequant_pc_f32(acc: np.ndarray, s_x: np.ndarray, s_w: np.ndarray):
    """fp32 y32 [M, N] = ((float)acc * s_x[m]) * s_w[n], each product rounded to fp32."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    _check(_load().oracle_dequant_pc_f32(_p(acc), _p(s_x), _p(s_w), M, N, _p(y)), "dequant_pc_f32")
    return y


def dequant_pg_f32(acc_g: np.ndarray, s_x: np.ndarray, s_w: np.ndarray):
    """fp32 y32 [M, N]: t = fmaf((float)acc_g, s_w[n, g], t) over g ascending from +0, then t * s_x[m]."""
    acc_g = np.ascontiguousarray(acc_g, dtype=np.int32)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    M, N, G = acc_g.shape
    y = np.empty((M, N), np.float32)
    _check(_load().oracle_dequant_pg_f32(_p(acc_g), _p(s_x), _p(s_w), M, N, G, _p(y)), "dequant_pg_f32")
    return y


# ---- whole-path conveniences (the steps above, in the pages' order) --------------------

def linear_pc(x: np.ndarray, w_q: np.ndarray, s_w: np.ndarray):
    """Per-channel W8A8 linear: quantize x per token, int GEMM, dequant.

    Returns dict with x_q, s_x, acc (int32), y (fp64) and y32 (the fp32 evaluation the
    output format is rounded from).
    """
    x_q, s_x = quantize_per_token(x)
    acc = gemm_i32(x_q, w_q)
    return {"x_q": x_q, "s_x": s_x, "acc": acc, "y": dequant_pc(acc, s_x, s_w),
            "y32": dequant_pc_f32(acc, s_x, s_w)}


def linear_pg(x: np.ndarray, w_q: np.ndarray, s_w: np.ndarray, group_size: int):
    """Per-group W8A8 linear. Returns x_q, s_x, acc (sum of group accumulators), y (fp64),
    mag and y32 (the fp32 fold in K order the output format is rounded from)."""
    x_q, s_x = quantize_per_token(x)
    acc_g = group_acc(x_q, w_q, group_size)
    y, mag = dequant_pg(acc_g, s_x, s_w)
    acc = acc_g.astype(np.int64).sum(axis=2).astype(np.int32)
    return {"x_q": x_q, "s_x": s_x, "acc": acc, "acc_g": acc_g, "y": y, "mag": mag,
            "y32": dequant_pg_f32(acc_g, s_x, s_w)}


def linear_w4(x: np.ndarray, w_packed: np.ndarray, s_w: np.ndarray, group_size: int):
    """W4A8 linear: unpack the int4 codes, then the per-group path (group_size 64 / 128) or,
    for group_size 0 (one scale per output channel), the per-channel path."""
    K = x.shape[1]
    if group_size == 0:
        return linear_pc(x, unpack_int4(w_packed, K), s_w)
    return linear_pg(x, unpack_int4(w_packed, K), s_w, group_size)


def linear_mv(x: np.ndarray, w_q: np.ndarray, s_w: np.ndarray, group_size: int = 0, bf16: bool = False):
    """Decode matrix-vector product without activation quantization: fp64
    y[m, n] = sum_k x[m, k] * w_q[n, k] * s_w[n, k // group_size] (s_w[n] for group_size 0).

    x: float16 [M, K], or (bf16=True) a uint16 array of bfloat16 bit patterns.
    Returns dict with y and mag (the sum of the terms' magnitudes), both fp64 [M, N].
    """
    bits = np.ascontiguousarray(x.view(np.uint16) if x.dtype == np.float16 else x, dtype=np.uint16)
    if x.dtype == np.float16 and bf16:
        raise TypeError("bf16=True expects bfloat16 bit patterns (uint16), not float16")
    w_q = np.ascontiguousarray(w_q, dtype=np.int8)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    M, K = bits.shape
    N = w_q.shape[0]
    assert w_q.shape[1] == K
    y = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    _check(_load().oracle_mv(_p(bits), 1 if bf16 else 0, M, K, K, _p(w_q), _p(s_w), N, group_size, _p(y), _p(mag)),
           "mv")
    return {"y": y, "mag": mag}


def sdpa_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, N: int = None, scale: float = None,
                bf16: bool = False):
    """Decode-step attention in fp64. q [B, Hq, D]; k, v [B, Hkv, Ncap, D] (first N rows used),
    float16 arrays, or (bf16=True) uint16 bfloat16 bit patterns. scale defaults to 1/sqrt(D).
    Returns dict with o [B, Hq, D], vmag [B, Hq, D] and smag [B, Hq] (fp64)."""
    def bits(a):
        return np.ascontiguousarray(a.view(np.uint16) if a.dtype == np.float16 else a, dtype=np.uint16)
    qb, kb, vb = bits(q), bits(k), bits(v)
    B, Hq, D = qb.shape
    _, Hkv, Ncap, _ = kb.shape
    N = Ncap if N is None else N
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    o = np.empty((B, Hq, D), np.float64)
    vmag = np.empty((B, Hq, D), np.float64)
    smag = np.empty((B, Hq), np.float64)
    _check(_load().oracle_sdpa_decode(_p(qb), _p(kb), _p(vb), 1 if bf16 else 0, B, Hq, Hkv, N, Ncap, D, float(scale),
                                      _p(o), _p(vmag), _p(smag)), "sdpa_decode")
    return {"o": o, "vmag": vmag, "smag": smag}
