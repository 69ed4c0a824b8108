"""GPU parity of rmsnorm_quantize (RMSNorm with the per-token quantization folded into its
scale) against the CPU oracle, through the C ABI.

Codes: bit-exact (both sides quantize u = x * g, one fp32 multiply per element, with the
same fp32 scale and correctly rounded quotient). Scale: s_x = s_u / sqrt(mean x^2 + eps)
carries the GPU's fp32 rounding of the sum of K squares (any order: relative error
<= (K - 1) 2^-24), halved by the square root, plus a few roundings (mean, + eps, square
root, reciprocal, product), so
    |s_x - s_x64| <= ((K + 1) / 2 + 8) * 2^-24 * s_x64   (x 1.01 for second-order terms).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import rmsnorm_inputs
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
    return w


def bf16_bits(a16: np.ndarray) -> np.ndarray:
    """fp16 values -> bf16 bit patterns, round to nearest even (the test's own bf16 inputs)."""
    u = a16.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def to_dev(a16: np.ndarray, bf16: bool):
    if bf16:
        return torch.from_numpy(bf16_bits(a16).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a16)).cuda()


def check(w8a8, x, g, eps, x_bf16, g_bf16, what, ldx_pad=0):
    M, K = x.shape
    xd, gd = to_dev(x, x_bf16), to_dev(g, g_bf16)
    if ldx_pad:
        big = torch.zeros((M, K + ldx_pad), dtype=xd.dtype, device="cuda")
        big[:, :K] = xd
        xd = big[:, :K]
    note(what)
    xq, sx = w8a8.rmsnorm_quantize(xd, gd, eps)
    torch.cuda.synchronize()
    xo = bf16_bits(x) if x_bf16 else x
    go = bf16_bits(g) if g_bf16 else g
    rq, _, rs = oracle.rmsnorm_quantize(xo, go, eps, x_bf16=x_bf16, g_bf16=g_bf16)
    got_q, got_s = xq.cpu().numpy(), sx.cpu().numpy().astype(np.float64)
    bad = np.argwhere(got_q != rq)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[0]}: {got_q[tuple(bad[0])]} vs {rq[tuple(bad[0])]}"
    bound = 1.01 * ((K + 1) / 2 + 8) * 2.0 ** -24 * rs
    err = np.abs(got_s - rs)
    assert (err <= bound).all(), f"{what}: scale off by {np.max(err / np.maximum(rs, 1e-300))} relative"
    return xq, sx


@pytest.mark.parametrize("M,K", [(1, 8), (3, 64), (5, 520), (37, 4096), (7, 12288), (2, 40960), (2048, 4096)])
def test_rmsnorm_quantize_parity(w8a8, M, K):
    x, g = rmsnorm_inputs(M, K, seed=M + K)
    for x_bf16 in (False, True):
        for g_bf16 in (False, True):
            for eps in (1e-6, 0.0):
                check(w8a8, x, g, eps, x_bf16, g_bf16, f"rmsnorm_quantize {M}x{K} bf16x={x_bf16} bf16g={g_bf16} eps={eps}")


def test_rmsnorm_quantize_benchmark_size(w8a8):
    """The benchmark's workload (M = 4096 rows of K = 10240, fp16, eps 1e-6), every row."""
    x, g = rmsnorm_inputs(4096, 10240, seed=0)
    check(w8a8, x, g, 1e-6, False, False, "rmsnorm_quantize 4096x10240 (benchmark workload)")


def test_rmsnorm_quantize_special_rows_and_stride(w8a8):
    K = 1024
    x, g = rmsnorm_inputs(8, K, seed=5)
    x[0] = 0                                   # zero row: zero codes, zero scale (also at eps = 0)
    x[1] = 0
    x[1, 333] = -3                             # one-hot row: one code -127
    x[2] = np.float16(65504) * np.where(np.arange(K) % 3 == 0, -1, 1)  # fp16 maxima
    x[3] = np.ldexp(np.arange(K) % 7 - 3, -24).astype(np.float16)  # subnormal halves
    x[4] = 1                                   # constant row: codes follow g alone
    for eps in (0.0, 1e-6):
        xq, sx = check(w8a8, x, g, eps, False, False, f"special rows eps={eps}", ldx_pad=24)
        q = xq.cpu().numpy()
        assert (q[0] == 0).all() and sx[0].item() == 0
        assert q[1, 333] == -127 and (np.delete(q[1], 333) == 0).all()


def test_rmsnorm_quantize_bf16_extreme_rows(w8a8):
    """bf16 rows whose squares leave the fp32 range (|x| ~ 1e30: x^2 ~ 1e60; |x| ~ 2^-100 and
    the subnormal 2^-130: x^2 ~ 2^-200 .. 2^-260) and rows near the fp32 overflow of x^2
    (|x| ~ 1e19). The kernel sums the squares of bf16 rows in fp64, as the oracle does, so the
    scale stays finite and nonzero at eps = 0 and equals the oracle's to the sum's bound."""
    K = 512
    rng = np.random.default_rng(9)
    x32 = np.stack([rng.standard_normal(K) * 1e30,
                    rng.standard_normal(K) * 2.0 ** -100,
                    np.where(np.arange(K) % 5 == 0, 2.0 ** -130, 0.0) * np.where(np.arange(K) % 2 == 0, 1, -1),
                    rng.standard_normal(K) * 1e19]).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    xb = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # RNE to bf16 bit patterns
    g = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    gd = torch.from_numpy(g).cuda()
    for eps in (0.0, 1e-6):
        note(f"rmsnorm_quantize bf16 extreme rows eps={eps}")
        xq, sx = w8a8.rmsnorm_quantize(xd, gd, eps)
        torch.cuda.synchronize()
        rq, _, rs = oracle.rmsnorm_quantize(xb, g, eps, x_bf16=True, g_bf16=False)
        got_q, got_s = xq.cpu().numpy(), sx.cpu().numpy().astype(np.float64)
        assert (got_q == rq).all(), f"eps={eps}: codes differ"
        assert np.isfinite(got_s).all() and (got_s > 0).all(), f"eps={eps}: scales {got_s}"
        bound = 1.01 * ((K + 1) / 2 + 8) * 2.0 ** -24 * rs
        assert (np.abs(got_s - rs) <= bound).all(), f"eps={eps}: scales {got_s} against {rs}"


def test_rmsnorm_quantize_feeds_the_gemm(w8a8):
    """The codes and scale go into w8a8_gemm_pc unchanged; the GEMM output matches the oracle's
    linear layer applied to the same codes (fp32 bound of the per-channel epilogue)."""
    M, N, K = 64, 256, 2048
    x, g = rmsnorm_inputs(M, K, seed=7)
    W = (np.random.default_rng(8).standard_normal((N, K)) * 0.02).astype(np.float32)
    xq, sx = check(w8a8, x, g, 1e-6, False, False, "rmsnorm_quantize -> gemm")
    wq, sw = w8a8.quantize_weight(torch.from_numpy(W).cuda(), 8, 0)
    y = w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.float32)
    torch.cuda.synchronize()
    acc = oracle.gemm_i32(xq.cpu().numpy(), wq.cpu().numpy())
    ref = oracle.dequant_pc(acc, sx.cpu().numpy(), sw.cpu().numpy())
    check_output(y.cpu().numpy(), "f32", ref, np.abs(ref), 1, "rmsnorm_quantize -> gemm_pc")
