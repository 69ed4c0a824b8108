"""GPU tests of w8a8_linear, the one-call layer (quantize -> GEMM -> dequant).

For M <= 16 it runs one kernel that quantizes the activations itself; larger M runs
quantize_per_token and the GEMM. Both must give the codes and scales of
quantize_per_token bit for bit, and outputs within the oracle tolerance; per-channel
outputs must equal the two-step GPU path bit for bit (the same arithmetic).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import linear_inputs
from _parity import check_output

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def w8a8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_activation_quantized_amd as w
    assert w.w8a8_is_available(0), w.w8a8_last_error()
    w.w8a8_debug_force_config(-1)
    return w


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def weights(w8a8, W, mode):
    Wd = dev(W)
    if mode == "pc":
        return (*w8a8.quantize_weight(Wd, 8, 0), 8, 0)
    if mode.startswith("pg"):
        gs = int(mode[2:])
        return (*w8a8.quantize_weight(Wd, 8, gs), 8, gs)
    gs = int(mode[3:])
    return (*w8a8.quantize_weight(Wd, 4, gs), 4, gs)


def two_step(w8a8, xd, wq, sw, bits, gs, out):
    xq, sx = w8a8.quantize_per_token(xd)
    if bits == 4 and gs == 0:
        y = w8a8.w4a8_gemm_pc(xq, sx, wq, sw, out)
    elif bits == 4:
        y = w8a8.w4a8_gemm_pg(xq, sx, wq, sw, gs, out)
    elif gs:
        y = w8a8.w8a8_gemm_pg(xq, sx, wq, sw, gs, out)
    else:
        y = w8a8.w8a8_gemm_pc(xq, sx, wq, sw, out)
    return y, xq, sx


def oracle_y(x, W, mode):
    if mode == "pc":
        wq, sw = oracle.quantize_weight(W, 8, 0)
        r = oracle.linear_pc(x, wq, sw)
        return r["y"], np.abs(r["y"]), 1
    if mode.startswith("pg"):
        gs = int(mode[2:])
        wq, sw = oracle.quantize_weight(W, 8, gs)
        r = oracle.linear_pg(x, wq, sw, gs)
    else:
        gs = int(mode[3:])
        wq, sw = oracle.quantize_weight(W, 4, gs)
        r = oracle.linear_w4(x, wq, sw, gs)
        if gs == 0:
            return r["y"], np.abs(r["y"]), 1
    return r["y"], r["mag"], W.shape[1] // gs


def with_edge_rows(x):
    """Row 1 all zero (scale 0); the rest as generated."""
    x = x.copy()
    if x.shape[0] > 1:
        x[1] = 0
    return x


@pytest.mark.parametrize("mode", ["pc", "pg64", "pg128", "w4_128", "w4_64", "w4_0"])
@pytest.mark.parametrize("M,N,K", [(1, 272, 2560), (2, 48, 10240), (3, 1040, 640), (5, 16, 4096), (8, 272, 1280),
                                   (16, 528, 2560), (1, 10240, 2560), (17, 272, 640), (40, 48, 1280)])
def test_linear_fp16(w8a8, mode, M, N, K):
    x, W = linear_inputs(M, N, K, seed=M * 3 + N + K)
    x = with_edge_rows(x)
    xd = dev(x)
    wq, sw, bits, gs = weights(w8a8, W, mode)
    oq, osx = oracle.quantize_per_token(x)
    y64, mag, G = oracle_y(x, W, mode)
    for out, fmt in ((torch.float16, "f16"), (torch.bfloat16, "bf16"), (torch.float32, "f32")):
        note(f"linear {mode} M={M} N={N} K={K} {fmt}")
        y, xq, sx = w8a8.w8a8_linear(xd, wq, sw, bits, gs, out)
        torch.cuda.synchronize()
        assert (host(xq) == oq).all(), "activation codes differ from the oracle"
        assert (host(sx).view(np.uint32) == osx.view(np.uint32)).all(), "activation scales differ"
        check_output(host(y), fmt, y64, mag, G, f"linear {mode} {M}x{N}x{K} {fmt}")
        if gs == 0:
            y2, _, _ = two_step(w8a8, xd, wq, sw, bits, gs, out)
            assert (host(y) == host(y2)).all(), "per-channel output differs from the two-step path"


@pytest.mark.parametrize("mode", ["pc", "pg128", "w4_128", "w4_0"])
@pytest.mark.parametrize("M", [1, 4, 16, 33])
def test_linear_bf16_input_and_tiny_rows(w8a8, mode, M):
    """bf16 activations, including a row whose scale is below 2^-100 (exact-division path)."""
    N, K = 272, 2560
    x16, W = linear_inputs(M, N, K, seed=90 + M)
    xb = torch.from_numpy(x16.astype(np.float32)).to(torch.bfloat16)
    if M > 2:
        xb[2] = xb[2] * 1e-33  # scale ~ 1e-33 < 2^-100
    xd = xb.cuda()
    wq, sw, bits, gs = weights(w8a8, W, mode)
    note(f"linear bf16 {mode} M={M}")
    y, xq, sx = w8a8.w8a8_linear(xd, wq, sw, bits, gs, torch.float16)
    y2, xq2, sx2 = two_step(w8a8, xd, wq, sw, bits, gs, torch.float16)
    torch.cuda.synchronize()
    assert (host(xq) == host(xq2)).all() and (host(sx).view(np.uint32) == host(sx2).view(np.uint32)).all()
    oq, osx = oracle.quantize_per_token_bf16(xb.view(torch.int16).numpy().view(np.uint16))
    assert (host(xq) == oq).all() and (host(sx).view(np.uint32) == osx.view(np.uint32)).all()
    # the oracle's dequantization of the oracle's codes (equal to the GPU's, checked above)
    K_ = x16.shape[1]
    owq, osw = oracle.quantize_weight(W, bits, gs)
    codes = oracle.unpack_int4(owq, K_) if bits == 4 else owq
    if gs == 0:
        y64 = oracle.dequant_pc(oracle.gemm_i32(oq, codes), osx, osw)
        mag, G = np.abs(y64), 1
        assert (host(y) == host(y2)).all()
    else:
        y64, mag = oracle.dequant_pg(oracle.group_acc(oq, codes, gs), osx, osw)
        G = K_ // gs
    check_output(host(y), "f16", y64, mag, G, f"linear bf16 {mode} M={M}")
    check_output(host(y2), "f16", y64, mag, G, f"two-step bf16 {mode} M={M}")


def test_linear_strided_x_and_empty(w8a8):
    M, N, K = 5, 272, 1280
    x, W = linear_inputs(M, N, K, seed=4)
    big = np.zeros((M, K + 64), np.float16)
    big[:, :K] = x
    xd = dev(big)[:, :K]
    wq, sw, bits, gs = weights(w8a8, W, "pc")
    note("linear strided x")
    y, xq, sx = w8a8.w8a8_linear(xd, wq, sw, bits, gs, torch.float16)
    y2, _, _ = two_step(w8a8, xd, wq, sw, bits, gs, torch.float16)
    torch.cuda.synchronize()
    oq, _ = oracle.quantize_per_token(x)
    assert (host(xq) == oq).all() and (host(y) == host(y2)).all()
    xe = torch.zeros((0, K), dtype=torch.float16, device="cuda")
    ye, _, _ = w8a8.w8a8_linear(xe, wq, sw, bits, gs, torch.float16)
    torch.cuda.synchronize()
    assert ye.shape == (0, N)


def test_linear_forced_config_runs_two_steps(w8a8):
    """With a forced GEMM configuration the call takes the two-launch path; same results."""
    M, N, K = 4, 272, 1280
    x, W = linear_inputs(M, N, K, seed=8)
    xd = dev(x)
    wq, sw, bits, gs = weights(w8a8, W, "pc")
    y, _, _ = w8a8.w8a8_linear(xd, wq, sw, bits, gs, torch.float16)
    try:
        w8a8.w8a8_debug_force_config(10)
        y2, xq2, _ = w8a8.w8a8_linear(xd, wq, sw, bits, gs, torch.float16)
    finally:
        w8a8.w8a8_debug_force_config(-1)
    torch.cuda.synchronize()
    assert (host(y) == host(y2)).all()
