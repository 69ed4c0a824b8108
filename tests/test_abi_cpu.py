"""Host-side tests of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status codes BEFORE touching a device.

No compute call is made here: every call either fails argument validation or runs
with W8A8_FORCE_UNAVAILABLE=1, so nothing can be launched on any machine.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

OK, INVALID, UNSUPPORTED_DEVICE, UNSUPPORTED_SHAPE = 0, 1, 2, 3
F16, BF16, F32, I32 = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x100000)  # 16-byte aligned, never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def w8a8():
    import w8a8_activation_quantized_amd as pkg
    return pkg


@pytest.fixture
def unavailable(monkeypatch):
    monkeypatch.setenv("W8A8_FORCE_UNAVAILABLE", "1")


def test_header_declares_the_hot_path():
    names = declared_functions()
    for required in ("quantize_per_token", "quantize_weight", "w8a8_gemm_pc", "w8a8_gemm_pg",
                     "w4a8_gemm_pg", "w4a8_gemm_pc", "w8a8_linear", "w8a8_is_available", "w8a8_last_error",
                     "w8a8_status_string", "int8_mv", "w8a8_gemm_splitk", "w8a8_gemm_splitk_workspace",
                     "rmsnorm_quantize", "sdpa_decode", "sdpa_decode_autotune", "sdpa_decode_tuned_slices",
                     "quantize_weight_clipped"):
        assert required in names, names


def test_library_exports_every_declared_symbol(w8a8):
    lib = ctypes.CDLL(w8a8.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"libw8a8.so does not export {name}"


def test_status_strings(w8a8):
    lib = w8a8.lib()
    assert lib.w8a8_status_string(OK) == b"ok"
    assert lib.w8a8_status_string(INVALID) == b"invalid argument"
    assert lib.w8a8_status_string(99) == b"unknown status"
    assert lib.w8a8_abi_version() >= 1


def test_forced_unavailable(w8a8, unavailable):
    lib = w8a8.lib()
    assert lib.w8a8_is_available(0) == 0
    rc = lib.w8a8_gemm_pc(FAKE, FAKE, FAKE, FAKE, FAKE, F16, 128, 256, 256, 256, None)
    assert rc == UNSUPPORTED_DEVICE
    assert b"W8A8_FORCE_UNAVAILABLE" in lib.w8a8_last_error()
    rc = lib.quantize_per_token(FAKE, F16, 4, 64, 64, FAKE, FAKE, None)
    assert rc == UNSUPPORTED_DEVICE


@pytest.mark.parametrize("args,status,needle", [
    # (M, N, K, ldy, y_dtype)
    ((-1, 256, 256, 256, F16), INVALID, "M"),
    ((8, 250, 256, 256, F16), UNSUPPORTED_SHAPE, "N"),
    ((8, 0, 256, 256, F16), UNSUPPORTED_SHAPE, "N"),
    ((8, 256, 100, 256, F16), UNSUPPORTED_SHAPE, "K"),
    ((8, 256, 0, 256, F16), UNSUPPORTED_SHAPE, "K"),
    ((8, 256, 256, 255, F16), INVALID, "ldy"),
    ((8, 256, 256, 128, F16), INVALID, "ldy"),
    ((8, 256, 256, 256, 7), INVALID, "y_dtype"),
])
def test_gemm_pc_validation(w8a8, args, status, needle):
    lib = w8a8.lib()
    M, N, K, ldy, dt = args
    rc = lib.w8a8_gemm_pc(FAKE, FAKE, FAKE, FAKE, FAKE, dt, M, N, K, ldy, None)
    assert rc == status
    assert needle in lib.w8a8_last_error().decode()


def test_gemm_null_and_misaligned_pointers(w8a8):
    lib = w8a8.lib()
    rc = lib.w8a8_gemm_pc(None, FAKE, FAKE, FAKE, FAKE, F16, 8, 256, 256, 256, None)
    assert rc == INVALID and b"null" in lib.w8a8_last_error()
    odd = ctypes.c_void_p(0x100004)
    rc = lib.w8a8_gemm_pc(FAKE, FAKE, odd, FAKE, FAKE, F16, 8, 256, 256, 256, None)
    assert rc == INVALID and b"aligned" in lib.w8a8_last_error()


def test_group_size_validation(w8a8):
    lib = w8a8.lib()
    for gs in (0, 32, 96, 256):
        rc = lib.w8a8_gemm_pg(FAKE, FAKE, FAKE, FAKE, gs, FAKE, F16, 8, 256, 256, 256, None)
        assert rc == INVALID, gs
        rc = lib.w4a8_gemm_pg(FAKE, FAKE, FAKE, FAKE, gs, FAKE, F16, 8, 256, 256, 256, None)
        assert rc == INVALID, gs
    rc = lib.w8a8_gemm_pg(FAKE, FAKE, FAKE, FAKE, 128, FAKE, F16, 8, 256, 192, 256, None)
    assert rc == UNSUPPORTED_SHAPE  # K not a multiple of the group size


def test_quantize_validation(w8a8):
    lib = w8a8.lib()
    assert lib.quantize_per_token(FAKE, F32, 4, 64, 64, FAKE, FAKE, None) == INVALID
    assert lib.quantize_per_token(FAKE, F16, 4, 60, 64, FAKE, FAKE, None) == UNSUPPORTED_SHAPE
    assert lib.quantize_per_token(FAKE, F16, 4, 64, 60, FAKE, FAKE, None) == INVALID
    assert lib.quantize_per_token(FAKE, F16, 4, 64, 68, FAKE, FAKE, None) == INVALID
    assert lib.quantize_per_token(None, F16, 4, 64, 64, FAKE, FAKE, None) == INVALID
    assert lib.quantize_weight(FAKE, 16, 256, 3, 0, FAKE, FAKE, None) == INVALID
    assert lib.quantize_weight(FAKE, 16, 256, 8, 32, FAKE, FAKE, None) == INVALID
    assert lib.quantize_weight(FAKE, 16, 200, 8, 0, FAKE, FAKE, None) == UNSUPPORTED_SHAPE
    assert lib.quantize_weight(FAKE, 0, 256, 8, 0, FAKE, FAKE, None) == INVALID


def test_rmsnorm_quantize_validation(w8a8):
    """Argument checks run on the host before anything is enqueued (no GPU here)."""
    lib = w8a8.lib()
    f = lambda *a: lib.rmsnorm_quantize(*a)
    assert f(FAKE, F32, 4, 64, 64, FAKE, F16, 1e-6, FAKE, FAKE, None) == INVALID      # x dtype
    assert f(FAKE, F16, 4, 64, 64, FAKE, F32, 1e-6, FAKE, FAKE, None) == INVALID      # gamma dtype
    assert f(FAKE, F16, 4, 64, 64, FAKE, F16, -1.0, FAKE, FAKE, None) == INVALID      # eps < 0
    assert f(FAKE, F16, 4, 64, 64, FAKE, F16, float("nan"), FAKE, FAKE, None) == INVALID
    assert f(FAKE, F16, 4, 64, 64, FAKE, F16, float("inf"), FAKE, FAKE, None) == INVALID
    assert f(FAKE, F16, -1, 64, 64, FAKE, F16, 1e-6, FAKE, FAKE, None) == INVALID
    assert f(FAKE, F16, 4, 60, 64, FAKE, F16, 1e-6, FAKE, FAKE, None) == UNSUPPORTED_SHAPE
    assert f(FAKE, F16, 4, 64, 60, FAKE, F16, 1e-6, FAKE, FAKE, None) == INVALID      # ldx < K
    assert f(FAKE, F16, 4, 64, 68, FAKE, F16, 1e-6, FAKE, FAKE, None) == INVALID      # ldx % 8
    assert f(FAKE, F16, 4, 64, 64, None, F16, 1e-6, FAKE, FAKE, None) == INVALID      # null gamma
    assert f(FAKE, F16, 4, 64, 64, ctypes.c_void_p(0x100002), F16, 1e-6, FAKE, FAKE, None) == INVALID  # misaligned


def test_debug_force_config_bounds(w8a8):
    lib = w8a8.lib()
    n = lib.w8a8_debug_force_config(-1)
    assert n >= 1
    assert lib.w8a8_debug_force_config(n) < 0
    assert lib.w8a8_debug_force_config(-2) < 0
    assert lib.w8a8_debug_force_config(-1) == n


def test_binding_raises_on_bad_input(w8a8):
    import torch
    x = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        w8a8.quantize_per_token(x)


def _linear(lib, x=FAKE, x_dtype=F16, ldx=256, bits=8, gs=0, x_q=FAKE, y_dtype=F16, M=8, N=256, K=256, ldy=256):
    return lib.w8a8_linear(x, x_dtype, ldx, FAKE, FAKE, bits, gs, x_q, FAKE, FAKE, y_dtype, M, N, K, ldy, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x_dtype=F32), INVALID, "x_dtype"),
    (dict(bits=2), INVALID, "weight_bits"),
    (dict(gs=32), INVALID, "group_size"),
    (dict(y_dtype=I32), INVALID, "y_dtype"),
    (dict(ldx=200), INVALID, "ldx"),
    (dict(ldx=260), INVALID, "ldx"),
    (dict(N=250), UNSUPPORTED_SHAPE, "N"),
    (dict(K=100, ldx=104), UNSUPPORTED_SHAPE, "K"),
    (dict(gs=128, K=192, ldx=192), UNSUPPORTED_SHAPE, "group_size"),
    (dict(ldy=250), INVALID, "ldy"),
    (dict(x=None), INVALID, "x"),
    (dict(x=ctypes.c_void_p(0x100008)), INVALID, "x"),
    (dict(x_q=None), INVALID, "null"),
])
def test_linear_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    assert _linear(lib, **kw) == status
    assert needle in lib.w8a8_last_error().decode()


def test_linear_forced_unavailable(w8a8, unavailable):
    lib = w8a8.lib()
    assert _linear(lib) == UNSUPPORTED_DEVICE


def _splitk(lib, x_q=FAKE, bits=8, gs=0, y_dtype=F16, M=128, N=2560, K=10240, ldy=2560, ws=FAKE,
            ws_bytes=1 << 30):
    return lib.w8a8_gemm_splitk(x_q, FAKE, FAKE, FAKE, bits, gs, FAKE, y_dtype, M, N, K, ldy, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(bits=2), INVALID, "weight_bits"),
    (dict(gs=32), INVALID, "group_size"),
    (dict(y_dtype=7), INVALID, "y_dtype"),
    (dict(N=250, ldy=256), UNSUPPORTED_SHAPE, "N"),
    (dict(K=100), UNSUPPORTED_SHAPE, "K"),
    (dict(gs=128, K=192), UNSUPPORTED_SHAPE, "group_size"),
    (dict(ldy=2500), INVALID, "ldy"),
    (dict(x_q=None), INVALID, "null"),
    (dict(ws_bytes=-1), INVALID, "workspace_bytes"),
    (dict(ws=ctypes.c_void_p(0x100008)), INVALID, "workspace"),
])
def test_splitk_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    assert _splitk(lib, **kw) == status
    assert needle in lib.w8a8_last_error().decode()


def test_splitk_forced_unavailable(w8a8, unavailable):
    lib = w8a8.lib()
    assert _splitk(lib) == UNSUPPORTED_DEVICE
    assert _splitk(lib, ws=None, ws_bytes=0) == UNSUPPORTED_DEVICE


def _noalloc(lib, x_q=FAKE, bits=8, gs=0, y_dtype=F16, M=128, N=2560, K=10240, ldy=2560):
    return lib.w8a8_gemm_splitk_noalloc(x_q, FAKE, FAKE, FAKE, bits, gs, FAKE, y_dtype, M, N, K, ldy, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(bits=2), INVALID, "weight_bits"),
    (dict(gs=32), INVALID, "group_size"),
    (dict(y_dtype=7), INVALID, "y_dtype"),
    (dict(N=250, ldy=256), UNSUPPORTED_SHAPE, "N"),
    (dict(K=100), UNSUPPORTED_SHAPE, "K"),
    (dict(ldy=2500), INVALID, "ldy"),
    (dict(x_q=None), INVALID, "null"),
])
def test_splitk_noalloc_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    assert _noalloc(lib, **kw) == status
    assert needle in lib.w8a8_last_error().decode()


def test_splitk_noalloc_forced_unavailable(w8a8, unavailable):
    lib = w8a8.lib()
    assert _noalloc(lib) == UNSUPPORTED_DEVICE
    assert _noalloc(lib, M=0) == UNSUPPORTED_DEVICE


def test_splitk_workspace_query(w8a8):
    """The query is host-only arithmetic: slices * M * N * 4 bytes, or 0 where no split runs."""
    lib = w8a8.lib()
    q = lib.w8a8_gemm_splitk_workspace
    assert lib.w8a8_debug_force_splitk(0) < 0 and lib.w8a8_debug_force_splitk(-2) < 0
    try:
        # forced slice counts, per-channel and per-group, capped at K / 128
        assert lib.w8a8_debug_force_splitk(4) == OK
        assert q(8, 0, F16, 128, 2560, 10240) == 4 * 128 * 2560 * 4
        assert q(8, 128, BF16, 100, 2560, 10240) == 4 * 100 * 2560 * 4
        assert q(4, 64, F32, 64, 512, 10240) == 4 * 64 * 512 * 4
        assert lib.w8a8_debug_force_splitk(100) == OK
        assert q(8, 0, F16, 128, 2560, 1024) == 8 * 128 * 2560 * 4
        # never split: GEMV range, K not a whole number of 128-value tiles, int4 with I32 out,
        # per-column int4
        assert q(8, 0, F16, 16, 2560, 10240) == 0
        assert q(8, 0, F16, 128, 2560, 10240 + 64) == 0
        assert q(4, 128, I32, 128, 2560, 10240) == 0
        assert q(4, 0, F16, 128, 2560, 10240) == 0
        assert q(8, 0, F16, 0, 2560, 10240) == 0
        # a forced configuration without a split form runs the single pass
        lib.w8a8_debug_force_config(13)
        assert q(8, 0, F16, 128, 2560, 10240) == 0
        lib.w8a8_debug_force_config(-1)
        assert lib.w8a8_debug_force_splitk(1) == OK
        assert q(8, 0, F16, 128, 2560, 10240) == 0
        # automatic: a narrow-N long-K problem splits, a large square-ish one does not
        assert lib.w8a8_debug_force_splitk(-1) == OK
        n = q(8, 0, F16, 128, 2560, 10240)
        assert n > 0 and n % (128 * 2560 * 4) == 0
        assert q(8, 0, F16, 4096, 10240, 2560) == 0
        # invalid shapes: -status
        assert q(8, 0, F16, 128, 250, 10240) == -UNSUPPORTED_SHAPE
        assert q(8, 32, F16, 128, 256, 1024) == -INVALID
        assert q(8, 0, F16, -1, 256, 1024) == -INVALID
    finally:
        lib.w8a8_debug_force_config(-1)
        lib.w8a8_debug_force_splitk(-1)


def _mv(lib, x=FAKE, x_dtype=F16, ldx=256, w=FAKE, gs=0, y_dtype=F16, M=1, N=256, K=256, ldy=256):
    return lib.int8_mv(x, x_dtype, ldx, w, FAKE, gs, FAKE, y_dtype, M, N, K, ldy, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x_dtype=F32), INVALID, "x_dtype"),
    (dict(gs=32), INVALID, "group_size"),
    (dict(y_dtype=I32), INVALID, "y_dtype"),
    (dict(M=-1), INVALID, "M"),
    (dict(M=17), UNSUPPORTED_SHAPE, "M"),
    (dict(N=250), UNSUPPORTED_SHAPE, "N"),
    (dict(K=192, ldx=192), UNSUPPORTED_SHAPE, "K"),
    (dict(ldx=200), INVALID, "ldx"),
    (dict(ldx=260), INVALID, "ldx"),
    (dict(ldy=250), INVALID, "ldy"),
    (dict(x=None), INVALID, "null"),
    (dict(w=None), INVALID, "null"),
    (dict(x=ctypes.c_void_p(0x100008)), INVALID, "aligned"),
])
def test_mv_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    assert _mv(lib, **kw) == status
    assert needle in lib.w8a8_last_error().decode()


def test_mv_forced_unavailable(w8a8, unavailable):
    lib = w8a8.lib()
    assert _mv(lib) == UNSUPPORTED_DEVICE
    assert _mv(lib, M=0, x=None) == UNSUPPORTED_DEVICE


@pytest.mark.parametrize("kw,status,needle", [
    (dict(pct=0.0), INVALID, "clip_percentile"),
    (dict(pct=100.5), INVALID, "clip_percentile"),
    (dict(pct=float("nan")), INVALID, "clip_percentile"),
    (dict(bits=3), INVALID, "bits"),
    (dict(gs=32), INVALID, "group_size"),
    (dict(K=200), UNSUPPORTED_SHAPE, "K"),
    (dict(N=0), INVALID, "N"),
])
def test_quantize_weight_clipped_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    a = dict(N=16, K=256, bits=8, gs=0, pct=99.9)
    a.update(kw)
    assert lib.quantize_weight_clipped(FAKE, a["N"], a["K"], a["bits"], a["gs"], a["pct"], FAKE, FAKE, None) == status
    assert needle in lib.w8a8_last_error().decode()


def test_quantize_weight_clipped_forced_unavailable(w8a8, unavailable):
    assert w8a8.lib().quantize_weight_clipped(FAKE, 16, 256, 8, 0, 99.0, FAKE, FAKE, None) == UNSUPPORTED_DEVICE


def _sdpa(lib, q=FAKE, dtype=F16, o_dtype=F16, B=1, Hq=8, Hkv=2, N=64, Ncap=64, D=128, scale=0.088, ws=None,
          ws_bytes=0):
    return lib.sdpa_decode(q, FAKE, FAKE, dtype, FAKE, o_dtype, B, Hq, Hkv, N, Ncap, D, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=F32), INVALID, "dtype"),
    (dict(o_dtype=I32), INVALID, "o_dtype"),
    (dict(B=-1), INVALID, "B"),
    (dict(Hq=6, Hkv=4), INVALID, "Hkv"),
    (dict(Hq=34, Hkv=2), UNSUPPORTED_SHAPE, "16"),
    (dict(D=96), UNSUPPORTED_SHAPE, "D"),
    (dict(N=0), INVALID, "N"),
    (dict(N=65, Ncap=64), INVALID, "N"),
    (dict(scale=0.0), INVALID, "scale"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(q=None), INVALID, "null"),
    (dict(ws_bytes=-1), INVALID, "workspace_bytes"),
    (dict(ws=ctypes.c_void_p(0x100008), ws_bytes=4096), INVALID, "workspace"),
])
def test_sdpa_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    assert _sdpa(lib, **kw) == status
    assert needle in lib.w8a8_last_error().decode()


def test_sdpa_forced_unavailable_and_workspace_query(w8a8, unavailable):
    lib = w8a8.lib()
    assert _sdpa(lib) == UNSUPPORTED_DEVICE
    # the size query is host arithmetic: slices * B * Hq * (D + 4) * 4 bytes for the most
    # slices the autotuner may pick (4 x the rule's count, at least 128 keys each), 0 for one
    # slice; with no GPU the rule takes 256 compute units: 64 slices for 4 KV heads
    assert lib.sdpa_decode_workspace(1, 32, 8, 64, 128) == 0
    assert lib.sdpa_decode_workspace(1, 32, 4, 32768, 128) == 32 * 132 * 4 * 256
    assert lib.sdpa_decode_workspace(1, 32, 4, 4096, 128) == 32 * 132 * 4 * 32  # N / 128 caps it
    assert lib.sdpa_decode_workspace(1, 32, 3, 1024, 128) < 0


def _tune(lib, q=FAKE, dtype=F16, o_dtype=F16, B=1, Hq=8, Hkv=2, N=64, Ncap=64, D=128, scale=0.088, ws=None,
          ws_bytes=0, out=None):
    return lib.sdpa_decode_autotune(q, FAKE, FAKE, dtype, FAKE, o_dtype, B, Hq, Hkv, N, Ncap, D, scale, ws, ws_bytes,
                                    None, out)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=F32), INVALID, "dtype"),
    (dict(B=0), INVALID, "B"),
    (dict(Hq=6, Hkv=4), INVALID, "Hkv"),
    (dict(D=96), UNSUPPORTED_SHAPE, "D"),
    (dict(N=65, Ncap=64), INVALID, "N"),
    (dict(q=None), INVALID, "null"),
    (dict(ws_bytes=-1), INVALID, "workspace_bytes"),
])
def test_sdpa_autotune_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    assert _tune(lib, **kw) == status
    assert needle in lib.w8a8_last_error().decode()


def test_sdpa_autotune_unavailable_and_empty_table(w8a8, unavailable):
    lib = w8a8.lib()
    best = ctypes.c_int(-7)
    assert _tune(lib, out=ctypes.byref(best)) == UNSUPPORTED_DEVICE
    assert best.value == -7  # nothing written
    assert lib.sdpa_decode_tuned_slices(F16, 1, 32, 8, 4096, 128) == 0
    assert lib.sdpa_decode_tuned_slices(F16, 1, 32, 3, 4096, 128) == -INVALID


def test_clock_probe_validation(w8a8, unavailable):
    lib = w8a8.lib()
    assert lib.w8a8_debug_clock_probe(None, None) == INVALID
    assert lib.w8a8_debug_clock_probe(ctypes.c_void_p(0x100008), None) == INVALID
    assert lib.w8a8_debug_clock_probe(FAKE, None) == UNSUPPORTED_DEVICE


def test_per_column_int4_validation(w8a8, unavailable):
    """Per-column int4 weights (group size 0) pass argument validation (W8A8_FORCE_UNAVAILABLE
    then stops the call before any launch); a bad shape still fails first."""
    lib = w8a8.lib()
    assert lib.quantize_weight(FAKE, 16, 256, 4, 0, FAKE, FAKE, None) == UNSUPPORTED_DEVICE
    assert lib.w4a8_gemm_pc(FAKE, FAKE, FAKE, FAKE, FAKE, F16, 4, 256, 512, 256, None) == UNSUPPORTED_DEVICE
    assert lib.w4a8_gemm_pc(FAKE, FAKE, FAKE, FAKE, FAKE, F16, 4, 250, 512, 256, None) == UNSUPPORTED_SHAPE
    assert lib.w4a8_gemm_pc(None, FAKE, FAKE, FAKE, FAKE, F16, 4, 256, 512, 256, None) == INVALID
    assert lib.w8a8_linear(FAKE, F16, 512, FAKE, FAKE, 4, 0, FAKE, FAKE, FAKE, F16, 4, 256, 512, 256,
                           None) == UNSUPPORTED_DEVICE


def _swiglu(lib, g=FAKE, dtype=F16, M=4, I=512, ldg=1024, ldu=1024, xq=FAKE):
    return lib.swiglu_quantize(g, FAKE, dtype, M, I, ldg, ldu, xq, FAKE, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=F32), INVALID, "dtype"),
    (dict(M=-1), INVALID, "M"),
    (dict(I=500, ldg=504, ldu=504), UNSUPPORTED_SHAPE, "I"),
    (dict(ldg=500), INVALID, "ldg"),
    (dict(ldu=1020), INVALID, "ldu"),
    (dict(g=None), INVALID, "null"),
    (dict(xq=ctypes.c_void_p(0x100008)), INVALID, "aligned"),
])
def test_swiglu_quantize_validation(w8a8, kw, status, needle):
    lib = w8a8.lib()
    assert _swiglu(lib, **kw) == status
    assert needle in lib.w8a8_last_error().decode()


def test_swiglu_quantize_forced_unavailable(w8a8, unavailable):
    lib = w8a8.lib()
    assert _swiglu(lib) == UNSUPPORTED_DEVICE
