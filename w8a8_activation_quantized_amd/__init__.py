"""Python binding of libw8a8 (fused per-token quantize -> int8 GEMM -> dequant on MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels
of ``libw8a8.so``; PyTorch provides device memory and the current stream. The
functions keep the C names of ``include/w8a8.h``.

Importing this package loads the built library and raises ImportError when it is
missing (build it with ``python -m w8a8_activation_quantized_amd.build``). There is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# W8A8_LIB names another build of the same library (the sanitizer tests load a build whose
# host code carries AddressSanitizer and UndefinedBehaviorSanitizer)
LIB_PATH = os.environ.get("W8A8_LIB") or os.path.join(_HERE, "libw8a8.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libw8a8.so not found at {LIB_PATH}; build it with "
        "`python -m w8a8_activation_quantized_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_i64, _int, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
_SIGNATURES = {
    "w8a8_is_available": ([_int], _int),
    "w8a8_status_string": ([_int], ctypes.c_char_p),
    "w8a8_last_error": ([], ctypes.c_char_p),
    "w8a8_abi_version": ([], _int),
    "w8a8_debug_force_config": ([_int], _int),
    "quantize_per_token": ([_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp], _int),
    "quantize_weight": ([_vp, _i64, _i64, _int, _int, _vp, _vp, _vp], _int),
    "rmsnorm_quantize": ([_vp, _int, _i64, _i64, _i64, _vp, _int, ctypes.c_float, _vp, _vp, _vp], _int),
    "swiglu_quantize": ([_vp, _vp, _int, _i64, _i64, _i64, _i64, _vp, _vp, _vp], _int),
    "w8a8_gemm_pc": ([_vp, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _i64, _vp], _int),
    "w8a8_gemm_pg": ([_vp, _vp, _vp, _vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _vp], _int),
    "w4a8_gemm_pg": ([_vp, _vp, _vp, _vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _vp], _int),
    "w4a8_gemm_pc": ([_vp, _vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _i64, _vp], _int),
    "w8a8_linear": ([_vp, _int, _i64, _vp, _vp, _int, _int, _vp, _vp, _vp, _int, _i64, _i64, _i64, _i64, _vp],
                    _int),
    "w8a8_gemm_splitk_workspace": ([_int, _int, _int, _i64, _i64, _i64], _i64),
    "w8a8_gemm_splitk": ([_vp, _vp, _vp, _vp, _int, _int, _vp, _int, _i64, _i64, _i64, _i64, _vp, _i64, _vp],
                         _int),
    "w8a8_debug_force_splitk": ([_int], _int),
    "w8a8_debug_clock_probe": ([_vp, _vp], _int),
    "w8a8_gemm_splitk_noalloc": ([_vp, _vp, _vp, _vp, _int, _int, _vp, _int, _i64, _i64, _i64, _i64, _vp], _int),
    "int8_mv": ([_vp, _int, _i64, _vp, _vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _vp], _int),
    "quantize_weight_clipped": ([_vp, _i64, _i64, _int, _int, ctypes.c_float, _vp, _vp, _vp], _int),
    "sdpa_decode_workspace": ([_i64, _i64, _i64, _i64, _i64], _i64),
    "sdpa_decode": ([_vp, _vp, _vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp, _i64,
                     _vp], _int),
    "sdpa_decode_autotune": ([_vp, _vp, _vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_float, _vp,
                              _i64, _vp, ctypes.POINTER(ctypes.c_int)], _int),
    "sdpa_decode_tuned_slices": ([_int, _i64, _i64, _i64, _i64, _i64], _int),
}
for _name, (_args, _res) in _SIGNATURES.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

# dtype enum of the C ABI
F16, BF16, F32, I32 = 0, 1, 2, 3
_DTYPE_CODE = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32, torch.int32: I32}
STATUS = {0: "W8A8_OK", 1: "W8A8_ERR_INVALID_ARGUMENT", 2: "W8A8_ERR_UNSUPPORTED_DEVICE",
          3: "W8A8_ERR_UNSUPPORTED_SHAPE", 4: "W8A8_ERR_HIP"}


class W8A8Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _check(rc: int):
    if rc != 0:
        raise W8A8Error(rc, _lib.w8a8_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def lib():
    """The ctypes handle of libw8a8.so (raw C entry points)."""
    return _lib


def w8a8_is_available(device: int = 0) -> bool:
    return bool(_lib.w8a8_is_available(device))


def w8a8_last_error() -> str:
    return _lib.w8a8_last_error().decode()


def w8a8_debug_force_config(config_id: int) -> int:
    n = _lib.w8a8_debug_force_config(config_id)
    if n < 0:
        raise W8A8Error(-n, f"unknown config id {config_id}")
    return n


def w8a8_debug_force_splitk(slices: int) -> None:
    rc = _lib.w8a8_debug_force_splitk(slices)
    if rc != 0:
        raise W8A8Error(-rc, f"bad slice count {slices}")


def w8a8_debug_clock_probe(out: torch.Tensor, stream=None) -> None:
    """Enqueue the clock probe: out (int64 [4096], device) receives per workgroup b its location
    (XCC_ID << 32 | HW_ID), shader-clock and 100 MHz counters at out[4 b .. 4 b + 2]."""
    if out.dtype != torch.int64 or out.numel() < 4096 or not out.is_cuda:
        raise ValueError("out must be a device int64 tensor of at least 4096 elements")
    _check(_lib.w8a8_debug_clock_probe(_ptr(out), _stream(stream)))


def quantize_per_token(x: torch.Tensor, x_q: torch.Tensor | None = None,
                       s_x: torch.Tensor | None = None, stream=None):
    """x [M, K] fp16/bf16 (row stride x.stride(0)) -> (x_q int8 [M, K], s_x fp32 [M])."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with a contiguous last dimension")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    M, K = x.shape
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_x is None:
        s_x = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(_lib.quantize_per_token(_ptr(x), _DTYPE_CODE[x.dtype], M, K, x.stride(0), _ptr(x_q),
                                   _ptr(s_x), _stream(stream)))
    return x_q, s_x


def rmsnorm_quantize(x: torch.Tensor, gamma: torch.Tensor, eps: float, x_q: torch.Tensor | None = None,
                     s_x: torch.Tensor | None = None, stream=None):
    """x [M, K] fp16/bf16 (row stride x.stride(0)), gamma [K] fp16/bf16 -> (x_q int8 [M, K],
    s_x fp32 [M]): the per-token codes of x * gamma, and s_x = (max|x * gamma| / 127) /
    sqrt(mean(x^2) + eps), so s_x * x_q approximates RMSNorm(x) * gamma."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with a contiguous last dimension")
    if x.dtype not in (torch.float16, torch.bfloat16) or gamma.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x and gamma must be float16 or bfloat16")
    M, K = x.shape
    if gamma.shape != (K,) or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous [K] tensor")
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_x is None:
        s_x = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(_lib.rmsnorm_quantize(_ptr(x), _DTYPE_CODE[x.dtype], M, K, x.stride(0), _ptr(gamma),
                                 _DTYPE_CODE[gamma.dtype], float(eps), _ptr(x_q), _ptr(s_x), _stream(stream)))
    return x_q, s_x


def swiglu_quantize(gate: torch.Tensor, up: torch.Tensor, x_q: torch.Tensor | None = None,
                    s_x: torch.Tensor | None = None, stream=None):
    """Codes and per-token scale of h = silu(gate) * up: gate, up [M, I] fp16/bf16 with a
    contiguous last dimension (they may be the two halves of one [M, 2 I] tensor).
    Returns (x_q int8 [M, I], s_x fp32 [M])."""
    for t in (gate, up):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("gate and up must be 2-D with a contiguous last dimension")
    if gate.dtype != up.dtype or gate.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("gate and up must both be float16 or both bfloat16")
    if gate.shape != up.shape:
        raise ValueError("gate and up must have the same shape")
    M, I = gate.shape
    if x_q is None:
        x_q = torch.empty((M, I), dtype=torch.int8, device=gate.device)
    if s_x is None:
        s_x = torch.empty((M,), dtype=torch.float32, device=gate.device)
    _check(_lib.swiglu_quantize(_ptr(gate), _ptr(up), _DTYPE_CODE[gate.dtype], M, I, gate.stride(0), up.stride(0),
                                _ptr(x_q), _ptr(s_x), _stream(stream)))
    return x_q, s_x


def quantize_weight(W: torch.Tensor, bits: int = 8, group_size: int = 0, stream=None):
    """W fp32 [N, K] -> (w_q, s_w); int8 [N, K] or packed uint8 [N, K/2]."""
    if W.dtype != torch.float32 or W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous fp32 [N, K] tensor")
    N, K = W.shape
    if bits == 8:
        w_q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    else:
        w_q = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    s_w = torch.empty((N,) if group_size == 0 else (N, K // max(group_size, 1)), dtype=torch.float32,
                      device=W.device)
    _check(_lib.quantize_weight(_ptr(W), N, K, bits, group_size, _ptr(w_q), _ptr(s_w), _stream(stream)))
    return w_q, s_w


def quantize_weight_clipped(W: torch.Tensor, bits: int = 8, group_size: int = 0, clip_percentile: float = 99.9,
                            stream=None):
    """quantize_weight with each run's scale from the clip_percentile-th percentile of |W|."""
    if W.dtype != torch.float32 or W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous fp32 [N, K] tensor")
    N, K = W.shape
    if bits == 8:
        w_q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    else:
        w_q = torch.empty((N, K // 2), dtype=torch.uint8, device=W.device)
    s_w = torch.empty((N,) if group_size == 0 else (N, K // max(group_size, 1)), dtype=torch.float32,
                      device=W.device)
    _check(_lib.quantize_weight_clipped(_ptr(W), N, K, bits, group_size, clip_percentile, _ptr(w_q), _ptr(s_w),
                                        _stream(stream)))
    return w_q, s_w


def _out(y, M, N, out_dtype, device):
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=device)
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be 2-D with a contiguous last dimension")
    return y


def w8a8_gemm_pc(x_q, s_x, w_q, s_w, out_dtype=torch.float16, y=None, stream=None):
    """y [M, N] = (acc * s_x[m]) * s_w[n], acc = x_q . w_q^T (int32)."""
    M, K = x_q.shape
    N = w_q.shape[0]
    y = _out(y, M, N, out_dtype, x_q.device)
    _check(_lib.w8a8_gemm_pc(_ptr(x_q), _ptr(s_x), _ptr(w_q), _ptr(s_w), _ptr(y), _DTYPE_CODE[y.dtype],
                             M, N, K, y.stride(0), _stream(stream)))
    return y


def w8a8_gemm_pg(x_q, s_x, w_q, s_w, group_size, out_dtype=torch.float16, y=None, stream=None):
    """Per-group dequant: y = s_x[m] * sum_g s_w[n, g] * acc_g."""
    M, K = x_q.shape
    N = w_q.shape[0]
    y = _out(y, M, N, out_dtype, x_q.device)
    _check(_lib.w8a8_gemm_pg(_ptr(x_q), _ptr(s_x), _ptr(w_q), _ptr(s_w), group_size, _ptr(y),
                             _DTYPE_CODE[y.dtype], M, N, K, y.stride(0), _stream(stream)))
    return y


def w4a8_gemm_pg(x_q, s_x, w_packed, s_w, group_size, out_dtype=torch.float16, y=None, stream=None):
    """W4A8: int4 weights packed two per byte, unpacked in-kernel; per-group dequant."""
    M, K = x_q.shape
    N = w_packed.shape[0]
    y = _out(y, M, N, out_dtype, x_q.device)
    _check(_lib.w4a8_gemm_pg(_ptr(x_q), _ptr(s_x), _ptr(w_packed), _ptr(s_w), group_size, _ptr(y),
                             _DTYPE_CODE[y.dtype], M, N, K, y.stride(0), _stream(stream)))
    return y


def w4a8_gemm_pc(x_q, s_x, w_packed, s_w, out_dtype=torch.float16, y=None, stream=None):
    """W4A8 with per-column int4 weights: one scale per output channel, s_w [N]."""
    M, K = x_q.shape
    N = w_packed.shape[0]
    y = _out(y, M, N, out_dtype, x_q.device)
    _check(_lib.w4a8_gemm_pc(_ptr(x_q), _ptr(s_x), _ptr(w_packed), _ptr(s_w), _ptr(y), _DTYPE_CODE[y.dtype], M, N, K,
                             y.stride(0), _stream(stream)))
    return y


def w8a8_linear(x, w, s_w, weight_bits=8, group_size=0, out_dtype=torch.float16, y=None, x_q=None, s_x=None,
                stream=None):
    """The whole layer: y = dequant(quantize_per_token(x) . w^T) in one call.

    x [M, K] fp16/bf16; w int8 [N, K] (weight_bits 8) or packed uint8 [N, K/2] (4);
    s_w [N] (group_size 0) or [N, K/group_size]. Returns (y, x_q, s_x); x_q and s_x hold
    the activation codes and scales as quantize_per_token computes them."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with a contiguous last dimension")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    M, K = x.shape
    N = w.shape[0]
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_x is None:
        s_x = torch.empty((M,), dtype=torch.float32, device=x.device)
    y = _out(y, M, N, out_dtype, x.device)
    _check(_lib.w8a8_linear(_ptr(x), _DTYPE_CODE[x.dtype], x.stride(0), _ptr(w), _ptr(s_w), weight_bits,
                            group_size, _ptr(x_q), _ptr(s_x), _ptr(y), _DTYPE_CODE[y.dtype], M, N, K,
                            y.stride(0), _stream(stream)))
    return y, x_q, s_x


def w8a8_gemm_splitk_workspace(M, N, K, weight_bits=8, group_size=0, out_dtype=torch.float16) -> int:
    """Workspace bytes w8a8_gemm_splitk uses for this problem (0: it runs the single pass)."""
    n = _lib.w8a8_gemm_splitk_workspace(weight_bits, group_size, _DTYPE_CODE[out_dtype], M, N, K)
    if n < 0:
        raise W8A8Error(-n, _lib.w8a8_last_error().decode())
    return n


def w8a8_gemm_splitk(x_q, s_x, w, s_w, weight_bits=8, group_size=0, out_dtype=torch.float16, y=None,
                     workspace=None, stream=None):
    """The GEMM selected by (weight_bits, group_size) as in w8a8_linear, with K cut into slices
    whose partial results go to `workspace` (a device tensor of at least
    w8a8_gemm_splitk_workspace(...) bytes; None or smaller: the single-pass kernels)."""
    M, K = x_q.shape
    N = w.shape[0]
    y = _out(y, M, N, out_dtype, x_q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.w8a8_gemm_splitk(_ptr(x_q), _ptr(s_x), _ptr(w), _ptr(s_w), weight_bits, group_size, _ptr(y),
                                 _DTYPE_CODE[y.dtype], M, N, K, y.stride(0), _ptr(workspace), ws_bytes,
                                 _stream(stream)))
    return y


def w8a8_gemm_splitk_noalloc(x_q, s_x, w, s_w, weight_bits=8, group_size=0, out_dtype=torch.float16, y=None,
                             stream=None):
    """w8a8_gemm_splitk with the partial results in the library's per-device scratch array
    (allocates nothing; raises W8A8Error when the split plan needs more scratch than it holds).
    Pass `y` to keep the call free of allocations on the Python side too."""
    M, K = x_q.shape
    N = w.shape[0]
    y = _out(y, M, N, out_dtype, x_q.device)
    _check(_lib.w8a8_gemm_splitk_noalloc(_ptr(x_q), _ptr(s_x), _ptr(w), _ptr(s_w), weight_bits, group_size, _ptr(y),
                                         _DTYPE_CODE[y.dtype], M, N, K, y.stride(0), _stream(stream)))
    return y


def int8_mv(x, w_q, s_w, group_size=0, out_dtype=torch.float16, y=None, stream=None):
    """Decode path without activation quantization: y = x . (w_q * s_w)^T in fp32.

    x [M, K] fp16/bf16 with 1 <= M <= 16; w_q int8 [N, K]; s_w [N] or [N, K/group_size]."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with a contiguous last dimension")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    M, K = x.shape
    N = w_q.shape[0]
    y = _out(y, M, N, out_dtype, x.device)
    _check(_lib.int8_mv(_ptr(x), _DTYPE_CODE[x.dtype], x.stride(0), _ptr(w_q), _ptr(s_w), group_size, _ptr(y),
                        _DTYPE_CODE[y.dtype], M, N, K, y.stride(0), _stream(stream)))
    return y


def sdpa_decode_workspace(B, Hq, Hkv, N, D) -> int:
    n = _lib.sdpa_decode_workspace(B, Hq, Hkv, N, D)
    if n < 0:
        raise W8A8Error(-n, _lib.w8a8_last_error().decode())
    return n


def sdpa_decode(q, k, v, N=None, scale=None, out_dtype=None, o=None, workspace=None, stream=None):
    """Attention for one decode step: q [B, Hq, D]; k, v [B, Hkv, Ncap, D] (contiguous, fp16 or
    bf16, first N rows used). Returns o [B, Hq, D]. workspace: a device tensor of at least
    sdpa_decode_workspace(...) bytes for the split-KV pass (None: one slice per KV head)."""
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("q, k, v must be contiguous fp16 / bf16 tensors")
    if not (q.dtype == k.dtype == v.dtype) or k.shape != v.shape or q.dim() != 3 or k.dim() != 4:
        raise ValueError("q [B, Hq, D] and k, v [B, Hkv, Ncap, D] of one dtype")
    B, Hq, D = q.shape
    _, Hkv, Ncap, _ = k.shape
    N = Ncap if N is None else N
    scale = 1.0 / (D ** 0.5) if scale is None else scale
    if o is None:
        o = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.sdpa_decode(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[q.dtype], _ptr(o), _DTYPE_CODE[o.dtype], B, Hq, Hkv,
                            N, Ncap, D, scale, _ptr(workspace), ws_bytes, _stream(stream)))
    return o


def sdpa_decode_autotune(q, k, v, N=None, scale=None, out_dtype=None, o=None, workspace=None, stream=None) -> int:
    """Time sdpa_decode on these tensors for each candidate slice count and record the fastest
    for their size class (later sdpa_decode calls use it). Returns the count chosen. Waits for
    the stream; arguments as sdpa_decode."""
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("q, k, v must be contiguous fp16 / bf16 tensors")
    B, Hq, D = q.shape
    _, Hkv, Ncap, _ = k.shape
    N = Ncap if N is None else N
    scale = 1.0 / (D ** 0.5) if scale is None else scale
    if o is None:
        o = torch.empty((B, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    best = ctypes.c_int(0)
    _check(_lib.sdpa_decode_autotune(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[q.dtype], _ptr(o), _DTYPE_CODE[o.dtype], B, Hq,
                                     Hkv, N, Ncap, D, scale, _ptr(workspace), ws_bytes, _stream(stream),
                                     ctypes.byref(best)))
    return best.value


def sdpa_decode_tuned_slices(dtype, B, Hq, Hkv, N, D) -> int:
    """The autotuned slice count for this size class on the current device (0: none)."""
    n = _lib.sdpa_decode_tuned_slices(_DTYPE_CODE[dtype], B, Hq, Hkv, N, D)
    if n < 0:
        raise W8A8Error(-n, _lib.w8a8_last_error().decode())
    return n
