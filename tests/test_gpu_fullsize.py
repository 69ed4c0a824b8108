"""Full-size parity at every point of the workload definitions, every output row.

The points: per-channel W8A8 at M in {1, 128, 1024, 4096, 8192} on [N=10240, K=2560] and
[N=2560, K=10240] (the first workload is per-channel M=128 on the first shape, included);
per-group gs 128 and 64 at M in {128, 1024, 4096, 8192} on both shapes; W4A8 gs=128 at
M in {1, 1024, 4096} on [10240, 2560]; and one Qwen3-8B-shaped block's linears at M=2048
(bf16 output). Inputs are the benchmark's (synth_inputs, seed 0); each point runs the
launch configuration the benchmark times (quantize_per_token, then the GEMM call with the
automatic tile choice; for M <= 16 also the one-kernel w8a8_linear).

Bit-exact against the oracle (computed from x and W on the CPU, independently of the GPU):
the int8 codes and scales of every row, the int32 sums (W8A8_I32) of every output, and the
fp16 / bf16 outputs of every kernel that folds in the pages' fp32 order (every per-channel
kernel; the single-pass per-group kernels). The per-group GEMV (M <= 16) splits each row's
K range over waves and adds the partial folds afterwards: its outputs are held to the
fp32 evaluation bound of tests/_parity.py instead. Every output also meets that bound
against the fp64 value.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import linear_inputs, qwen3_8b_block_inputs
from _parity import check_exact, check_output

pytestmark = pytest.mark.gpu

SHAPES = [(10240, 2560), (2560, 10240)]
POINTS = ([("pc", M, N, K) for M in (1, 128, 1024, 4096, 8192) for N, K in SHAPES]
          + [(mode, M, N, K) for mode in ("pg128", "pg64") for M in (128, 1024, 4096, 8192) for N, K in SHAPES]
          + [("w4_128", M, 10240, 2560) for M in (1, 1024, 4096)]
          # per-column int4 weights (the README's W4A8 weight format), the W4A8 sizes
          + [("w4_0", M, 10240, 2560) for M in (1, 1024, 4096)])
KIND = {"pc": (8, 0), "pg128": (8, 128), "pg64": (8, 64), "w4_128": (4, 128), "w4_0": (4, 0)}


def note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def w8a8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_activation_quantized_amd as w
    assert w.w8a8_is_available(0), w.w8a8_last_error()
    w.w8a8_debug_force_config(-1)
    w.w8a8_debug_force_splitk(-1)
    return w


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_gemm(w8a8, mode, xq, sx, wq, sw, out):
    bits, gs = KIND[mode]
    if mode == "pc":
        y = w8a8.w8a8_gemm_pc(xq, sx, wq, sw, out)
    elif bits == 8:
        y = w8a8.w8a8_gemm_pg(xq, sx, wq, sw, gs, out)
    elif gs == 0:
        y = w8a8.w4a8_gemm_pc(xq, sx, wq, sw, out)
    else:
        y = w8a8.w4a8_gemm_pg(xq, sx, wq, sw, gs, out)
    torch.cuda.synchronize()
    return host(y)


def oracle_rows(mode, x_rows, owq, osw):
    bits, gs = KIND[mode]
    if mode == "pc":
        r = oracle.linear_pc(x_rows, owq, osw)
        r["mag"], r["G"] = np.abs(r["y"]), 1
    elif bits == 8:
        r = oracle.linear_pg(x_rows, owq, osw, gs)
        r["G"] = owq.shape[1] // gs
    elif gs == 0:
        r = oracle.linear_w4(x_rows, owq, osw, 0)
        r["mag"], r["G"] = np.abs(r["y"]), 1
    else:
        r = oracle.linear_w4(x_rows, owq, osw, gs)
        r["G"] = x_rows.shape[1] // gs
    return r


@pytest.mark.parametrize("mode,M,N,K", POINTS)
def test_every_row(w8a8, mode, M, N, K):
    bits, gs = KIND[mode]
    note(f"full size, every row: {mode} M={M} N={N} K={K}")
    x, W = linear_inputs(M, N, K, seed=0)
    xq, sx = w8a8.quantize_per_token(torch.from_numpy(x).cuda())
    wq, sw = w8a8.quantize_weight(torch.from_numpy(W).cuda(), bits, gs)
    torch.cuda.synchronize()
    owq, osw = oracle.quantize_weight(W, bits, gs)
    assert (host(wq) == owq).all() and (host(sw).view(np.uint32) == osw.view(np.uint32)).all(), "weight codes"
    oxq, osx = oracle.quantize_per_token(x)
    assert (host(xq) == oxq).all() and (host(sx).view(np.uint32) == osx.view(np.uint32)).all(), "token codes"
    y16 = gpu_gemm(w8a8, mode, xq, sx, wq, sw, torch.float16)
    acc = gpu_gemm(w8a8, mode, xq, sx, wq, sw, torch.int32)
    fused = None
    if M <= 16:
        xq2 = torch.empty_like(xq)
        sx2 = torch.empty_like(sx)
        fused = host(w8a8.w8a8_linear(torch.from_numpy(x).cuda(), wq, sw, bits, gs, torch.float16, x_q=xq2, s_x=sx2)[0])
        torch.cuda.synchronize()
        assert (host(xq2) == oxq).all() and (host(sx2).view(np.uint32) == osx.view(np.uint32)).all(), "fused codes"
    canonical = gs == 0 or M > 16  # the fp32 fold in K order (see the module docstring)
    chunk = 2048 if mode == "pc" else 512
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        r = oracle_rows(mode, x[r0:r1], owq, osw)
        what = f"{mode} {M}x{N}x{K} rows {r0}:{r1}"
        assert (acc[r0:r1] == r["acc"]).all(), f"{what}: int32 sums differ"
        check_output(y16[r0:r1], "f16", r["y"], r["mag"], r["G"], what)
        if canonical:
            check_exact(y16[r0:r1], "f16", r["y32"], what)
        if fused is not None:
            check_output(fused[r0:r1], "f16", r["y"], r["mag"], r["G"], what + " (w8a8_linear)")
            if gs == 0:
                check_exact(fused[r0:r1], "f16", r["y32"], what + " (w8a8_linear)")


# the block as the benchmark runs it: one GEMM per input, projections that share an input
# concatenated along N (per-channel scales belong to output rows)
BLOCK = (("attn_in", ("q", "k", "v")), ("o_in", ("o",)), ("mlp_in", ("gate", "up")), ("down_in", ("down",)))


@pytest.mark.parametrize("in_name,projs", BLOCK)
def test_qwen3_block_every_row(w8a8, in_name, projs):
    note(f"qwen3 block, every row: {in_name} -> {'+'.join(projs)}")
    inputs, weights = qwen3_8b_block_inputs(M=2048, seed=0)
    x = inputs[in_name]
    W = np.concatenate([weights[n] for n in projs])
    del inputs, weights
    xq, sx = w8a8.quantize_per_token(torch.from_numpy(x).cuda())
    wq, sw = w8a8.quantize_weight(torch.from_numpy(W).cuda(), 8, 0)
    y = host(w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.bfloat16))
    acc = host(w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.int32))
    torch.cuda.synchronize()
    owq, osw = oracle.quantize_weight(W, 8, 0)
    oxq, osx = oracle.quantize_per_token(x)
    assert (host(xq) == oxq).all() and (host(sx).view(np.uint32) == osx.view(np.uint32)).all()
    r = oracle.linear_pc(x, owq, osw)
    what = f"qwen3 {in_name} 2048x{W.shape[0]}x{W.shape[1]}"
    assert (acc == r["acc"]).all(), f"{what}: int32 sums differ"
    check_output(y, "bf16", r["y"], np.abs(r["y"]), 1, what)
    check_exact(y, "bf16", r["y32"], what)
