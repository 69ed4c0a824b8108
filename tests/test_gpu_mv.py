"""GPU parity of int8_mv (decode path, activations not quantized) against the CPU oracle.

Tolerance from the arithmetic: every product x * q is exact in fp32 (fp16: 11 significant
bits, bf16: 8, a code: 8), the K products are summed in fp32 in an unspecified order and
scaled by s_w (per channel) or folded per group with one fma each, so
    |y - y64| <= (K + G + 2) * 2^-24 * mag,   mag = sum_k |x * q * s_w|,
plus the rounding to the output format (1 ulp for fp16 / bf16, 2^-24 |y| for fp32).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import linear_inputs
from _parity import ulp, bf16_bits_to_f64

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


def to_bf16_bits(x16: np.ndarray) -> np.ndarray:
    """fp16 values -> bf16 bit patterns, round to nearest even (the test's own bf16 inputs)."""
    u = x16.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def check_mv(y_t: torch.Tensor, y64: np.ndarray, mag: np.ndarray, K: int, G: int, what: str):
    if y_t.dtype == torch.bfloat16:
        got, fmt = bf16_bits_to_f64(y_t.view(torch.int16).cpu().numpy().view(np.uint16)), "bf16"
    else:
        got, fmt = y_t.cpu().numpy().astype(np.float64), ("f16" if y_t.dtype == torch.float16 else "f32")
    bound = (K + G + 2) * 2.0 ** -24 * mag
    out = 2.0 ** -24 * np.abs(y64) if fmt == "f32" else ulp(y64, fmt)
    err = np.abs(got - y64)
    bad = ~(err <= bound + out)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} out of tolerance; first {np.argwhere(bad)[0]}: "
                           f"got {got[tuple(np.argwhere(bad)[0])]} ref {y64[tuple(np.argwhere(bad)[0])]}")
    return float(err.max()) if err.size else 0.0


def run(w8a8, x16, W, gs, x_bf16, out, y=None, ldx_pad=0):
    M, K = x16.shape
    wq, sw = w8a8.quantize_weight(torch.from_numpy(W).cuda(), 8, gs)
    if x_bf16:
        xb = torch.from_numpy(to_bf16_bits(x16).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xb = torch.from_numpy(x16).cuda()
    if ldx_pad:
        big = torch.zeros((M, K + ldx_pad), dtype=xb.dtype, device="cuda")
        big[:, :K] = xb
        xb = big[:, :K]
    yt = w8a8.int8_mv(xb, wq, sw, gs, out, y=y)
    torch.cuda.synchronize()
    return yt, wq.cpu().numpy(), sw.cpu().numpy()


def reference(x16, wq, sw, gs, x_bf16):
    if x_bf16:
        return oracle.linear_mv(to_bf16_bits(x16), wq, sw, gs, bf16=True)
    return oracle.linear_mv(x16, wq, sw, gs)


@pytest.mark.parametrize("gs", [0, 64, 128])
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (1, 272, 2560), (2, 1040, 640), (3, 48, 1280), (5, 272, 384),
                                   (8, 528, 2560), (13, 16, 256), (16, 1040, 1280), (1, 2560, 10240),
                                   (4, 32, 12288)])
def test_mv_parity(w8a8, gs, M, N, K):
    x, W = linear_inputs(M, N, K, seed=M * 31 + N + K + gs)
    for x_bf16 in (False, True):
        for out in (torch.float16, torch.bfloat16, torch.float32):
            note(f"int8_mv gs={gs} M={M} N={N} K={K} bf16x={x_bf16} out={out}")
            yt, wq, sw = run(w8a8, x, W, gs, x_bf16, out)
            # the weights the GPU used are the oracle's (bit-exact quantization, tested elsewhere)
            rq, rs = oracle.quantize_weight(W, 8, gs)
            assert (wq == rq).all() and (sw.view(np.uint32) == rs.view(np.uint32)).all()
            r = reference(x, wq, sw, gs, x_bf16)
            check_mv(yt, r["y"], r["mag"], K, K // gs if gs else 1, f"mv gs={gs} {M}x{N}x{K} {out}")


def test_mv_strided_and_empty(w8a8):
    M, N, K = 6, 272, 1280
    x, W = linear_inputs(M, N, K, seed=3)
    ybig = torch.full((M, N + 20), 9.0, dtype=torch.float16, device="cuda")
    note("int8_mv strided x and y")
    yt, wq, sw = run(w8a8, x, W, 128, False, torch.float16, y=ybig[:, :N], ldx_pad=24)
    r = reference(x, wq, sw, 128, False)
    check_mv(ybig[:, :N], r["y"], r["mag"], K, K // 128, "strided")
    assert (ybig[:, N:].cpu().numpy() == np.float16(9.0)).all()
    note("int8_mv M=0")
    x0 = torch.zeros((0, K), dtype=torch.float16, device="cuda")
    wq0 = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    sw0 = torch.ones((N,), dtype=torch.float32, device="cuda")
    assert w8a8.int8_mv(x0, wq0, sw0).shape == (0, N)


def test_mv_special_inputs(w8a8):
    """Zero rows, one-hot rows (each output is one dequantized weight, exactly), extreme codes
    and a row of fp16 maxima."""
    N, K = 48, 256
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0, :] = 0.0  # zero row: scale 0
    W[1, :64] = 1.0  # one group of equal weights: codes 127
    x = np.zeros((5, K), np.float16)
    x[1, 17] = 1.0
    x[2, 200] = -2.0
    x[3, :] = 65504.0 * np.where(np.arange(K) % 2 == 0, 1, -1)
    x[4, :] = rng.standard_normal(K) * 1e-3
    for gs in (0, 64):
        note(f"int8_mv special inputs gs={gs}")
        yt, wq, sw = run(w8a8, x, W, gs, False, torch.float32)
        r = reference(x, wq, sw, gs, False)
        check_mv(yt, r["y"], r["mag"], K, K // gs if gs else 1, f"special gs={gs}")
        got = yt.cpu().numpy()
        assert (got[0] == 0).all()
        # one-hot rows: one exact product x * q, then one fp32 rounding by the scale (per
        # channel) or by the fold's fma (per group): the fp32 rounding of the exact value
        assert (got[1] == r["y"][1].astype(np.float32)).all() and (got[2] == r["y"][2].astype(np.float32)).all()


def test_mv_graph_replay(w8a8):
    x, W = linear_inputs(1, 2560, 10240, seed=5)
    xd = torch.from_numpy(x).cuda()
    wq, sw = w8a8.quantize_weight(torch.from_numpy(W).cuda(), 8, 128)
    y = torch.empty((1, 2560), dtype=torch.float16, device="cuda")
    w8a8.int8_mv(xd, wq, sw, 128, y=y)
    torch.cuda.synchronize()
    eager = y.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        w8a8.int8_mv(xd, wq, sw, 128, y=y, stream=torch.cuda.current_stream())
    for i in range(4):
        note(f"int8_mv graph replay {i}")
        y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
