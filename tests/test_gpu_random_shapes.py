"""Parity at seeded random shapes: every weight format and output type against the oracle
(160 cases), the split-K call at random forced configurations and slice counts (40),
decode attention at random head counts, cache lengths and formats (40), and the decode
matrix-vector product, the RMSNorm and SwiGLU producers and the clipped weight quantizer
(24 each),
on shapes that no fixed test picks (ragged M, N and K, small M that runs the GEMV, the tile
configurations the automatic choice reaches at those shapes).

Each case draws a mode (per channel, per group 64 / 128, int4 per group 64 / 128 or per
column), M in [1, 700] (a third of the cases at M <= 16), N a multiple of 16 up to 3200, K a
multiple of 64 (of the group size for per-group weights) up to 4096, and an output type.
The bar is the one of the fixed parity tests: int32 sums bit-exact, outputs bit-exact against
the oracle's fp32 evaluation wherever the kernel folds in that order, and within the fp32
evaluation bound of the fp64 value everywhere; the one-call layer at the same shape gives
the codes and scales of the oracle and outputs within the same bound.
"""
import numpy as np
import pytest
import torch

import oracle
import test_gpu_parity as tp
from _parity import check_output
from synth_inputs import linear_inputs

pytestmark = pytest.mark.gpu

MODES = ["pc", "pg64", "pg128", "w4_64", "w4_128", "w4_0"]
OUTS = [torch.float16, torch.bfloat16, torch.float32, torch.int32]


def draw_cases(n, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        mode = MODES[rng.integers(len(MODES))]
        gs = int(mode[2:]) if mode.startswith("pg") else int(mode[3:]) if mode.startswith("w4_") else 0
        M = int(rng.integers(1, 17)) if i % 3 == 0 else int(rng.integers(17, 701))
        N = 16 * int(rng.integers(1, 201))
        unit = gs if gs else 64
        K = unit * int(rng.integers(1, 4096 // unit + 1))
        out = OUTS[rng.integers(len(OUTS))]
        cases.append((mode, M, N, K, out))
    return cases


CASES = draw_cases(160)


@pytest.fixture(scope="module")
def w8a8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_activation_quantized_amd as w
    assert w.w8a8_is_available(0), w.w8a8_last_error()
    w.w8a8_debug_force_config(-1)
    return w


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shape(w8a8, i):
    mode, M, N, K, out = CASES[i]
    what = f"case {i}: {mode} M={M} N={N} K={K} {out}"
    tp.note(what)
    x, W = linear_inputs(M, N, K, seed=1000 + i)
    r = tp.oracle_mode(mode, x, W)
    tp.compare(tp.run_mode(w8a8, mode, x, W, out), r, what)
    if out == torch.int32 or M > 64:
        return
    # the one-call layer (quantization inside the kernel for M <= 16)
    bits = 4 if mode.startswith("w4") else 8
    gs = int(mode[2:]) if mode.startswith("pg") else int(mode[3:]) if bits == 4 else 0
    wq, sw = w8a8.quantize_weight(tp.dev(W), bits, gs)
    y, xq, sx = w8a8.w8a8_linear(tp.dev(x), wq, sw, bits, gs, out)
    torch.cuda.synchronize()
    oq, osx = oracle.quantize_per_token(x)
    assert (tp.host(xq) == oq).all() and (tp.host(sx).view(np.uint32) == osx.view(np.uint32)).all(), what
    check_output(tp.host(y), tp.OUT_FMT[out], r["y"], r["mag"], r["G"], "linear " + what)


# ---- split-K at random shapes, configurations and slice counts ------------------------

def draw_split_cases(n, seed=2027):
    import test_gpu_splitk as tk
    rng = np.random.default_rng(seed)
    modes = list(tk.KIND)
    cases = []
    for _ in range(n):
        mode = modes[rng.integers(len(modes))]
        cfgs = tk.SPLIT_CFGS[mode]
        cfg = int(cfgs[rng.integers(len(cfgs))])
        M = int(rng.integers(17, 401))
        N = 16 * int(rng.integers(1, 101))
        K = 128 * int(rng.integers(2, 81))
        slices = int(rng.integers(2, min(32, K // 128) + 1))
        out = OUTS[rng.integers(len(OUTS))]
        cases.append((mode, cfg, M, N, K, slices, out))
    return cases


SPLIT_CASES = draw_split_cases(40)


@pytest.mark.parametrize("i", range(len(SPLIT_CASES)))
def test_random_splitk(w8a8, i):
    """The split-K call with a forced tile configuration and slice count: within the fp32
    bound of the oracle; per-channel (and int32) results identical to the single pass."""
    import test_gpu_splitk as tk
    mode, cfg, M, N, K, slices, out = SPLIT_CASES[i]
    what = f"split case {i}: {mode} cfg {cfg} M={M} N={N} K={K} slices {slices} {out}"
    tp.note(what)
    prob = tk.Problem(w8a8, mode, M, N, K, seed=3000 + i)
    ref = tk.host(prob.single(w8a8, out))
    try:
        tk.forced(w8a8, cfg, slices)
        if not tk.has_split(mode, cfg, out):
            assert prob.workspace_bytes(w8a8, out) == 0
            return
        assert prob.workspace_bytes(w8a8, out) == slices * M * N * 4
        yt = prob.split(w8a8, out)
    finally:
        tk.reset(w8a8)
    prob.check(yt, what)
    if mode == "pc" or out == torch.int32:
        assert (tk.host(yt).view(np.uint8) == ref.view(np.uint8)).all(), f"{what}: differs from the single pass"


# ---- decode attention at random head counts, cache lengths and formats -----------------

def draw_sdpa_cases(n, seed=2028):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        N = int(rng.integers(1, 9001))
        Ncap = N + int(rng.integers(0, 64))
        D = int(rng.choice([64, 128]))
        bf16 = bool(rng.integers(2))
        out = [torch.float16, torch.bfloat16, torch.float32][rng.integers(3)]
        cases.append((B, Hkv * G, Hkv, N, Ncap, D, bf16, out))
    return cases


SDPA_CASES = draw_sdpa_cases(40)


@pytest.mark.parametrize("i", range(len(SDPA_CASES)))
def test_random_sdpa(w8a8, i):
    """sdpa_decode against the oracle within the fp32 evaluation bound of the attention
    tests, with and without a workspace."""
    import test_gpu_sdpa as ts
    B, Hq, Hkv, N, Ncap, D, bf16, out = SDPA_CASES[i]
    q, k, v = ts.inputs(B, Hq, Hkv, N, Ncap, D, seed=5000 + i)
    r = oracle.sdpa_decode(*((ts.to_bf16_bits(a) for a in (q, k, v)) if bf16 else (q, k, v)), N=N, bf16=bf16)
    qd, kd, vd = ts.dev(q, bf16), ts.dev(k, bf16), ts.dev(v, bf16)
    ws_n = w8a8.sdpa_decode_workspace(B, Hq, Hkv, N, D)
    ws = torch.full((max(ws_n, 16) // 4,), 777, dtype=torch.int32, device="cuda")
    for w in ((ws, None) if ws_n > 0 else (None,)):
        what = f"sdpa case {i}: B={B} Hq={Hq} Hkv={Hkv} N={N} Ncap={Ncap} D={D} bf16={bf16} {out} ws={w is not None}"
        tp.note(what)
        o = w8a8.sdpa_decode(qd, kd, vd, N=N, out_dtype=out, workspace=w)
        torch.cuda.synchronize()
        ts.check(o, r, N, D, what)


# ---- the other entry points at random shapes -------------------------------------------

def _rng_cases(seed, n, draw):
    rng = np.random.default_rng(seed)
    return [draw(rng) for _ in range(n)]


MV_CASES = _rng_cases(2029, 24, lambda r: (int(r.integers(1, 17)), 16 * int(r.integers(1, 201)),
                                           128 * int(r.integers(1, 49)), int(r.choice([0, 64, 128])),
                                           bool(r.integers(2)), int(r.integers(3))))


@pytest.mark.parametrize("i", range(len(MV_CASES)))
def test_random_int8_mv(w8a8, i):
    """The decode path (no activation quantization) within the fp32 evaluation bound."""
    import test_gpu_mv as tm
    M, N, K, gs, x_bf16, o = MV_CASES[i]
    out = [torch.float16, torch.bfloat16, torch.float32][o]
    what = f"mv case {i}: M={M} N={N} K={K} gs={gs} bf16x={x_bf16} {out}"
    tp.note(what)
    x, W = linear_inputs(M, N, K, seed=6000 + i)
    yt, wq, sw = tm.run(w8a8, x, W, gs, x_bf16, out)
    r = tm.reference(x, wq, sw, gs, x_bf16)
    tm.check_mv(yt, r["y"], r["mag"], K, K // gs if gs else 1, what)


RMS_CASES = _rng_cases(2030, 24, lambda r: (int(r.integers(1, 301)), 8 * int(r.integers(1, 2049)),
                                            bool(r.integers(2)), bool(r.integers(2)), float(r.choice([0.0, 1e-6, 1e-5]))))


@pytest.mark.parametrize("i", range(len(RMS_CASES)))
def test_random_rmsnorm_quantize(w8a8, i):
    """The RMSNorm producer: codes bit-exact, scale within the fp32 sum bound."""
    import test_gpu_rmsnorm_quant as tr
    from synth_inputs import rmsnorm_inputs
    M, K, x_bf16, g_bf16, eps = RMS_CASES[i]
    x, g = rmsnorm_inputs(M, K, seed=7000 + i)
    tr.check(w8a8, x, g, eps, x_bf16, g_bf16, f"rmsnorm case {i}: M={M} K={K} bf16x={x_bf16} bf16g={g_bf16} eps={eps}")


SWIGLU_CASES = _rng_cases(2031, 24, lambda r: (int(r.integers(1, 201)), 8 * int(r.integers(1, 2049)), bool(r.integers(2))))


@pytest.mark.parametrize("i", range(len(SWIGLU_CASES)))
def test_random_swiglu_quantize(w8a8, i):
    """The SwiGLU producer: codes and scales bit-exact."""
    import test_gpu_swiglu as tw
    M, I, bf16 = SWIGLU_CASES[i]
    dtype = torch.bfloat16 if bf16 else torch.float16
    tp.note(f"swiglu case {i}: M={M} I={I} {dtype}")
    tw.check(w8a8, tw.inputs(M, I, seed=8000 + i, dtype=dtype), I, f"swiglu case {i}: {M}x{I} {dtype}")


CLIP_CASES = _rng_cases(2032, 24, lambda r: (int(r.choice([8, 4])), int(r.choice([0, 64, 128])), 16 * int(r.integers(1, 41)),
                                             int(r.integers(1, 33)), float(r.choice([99.9, 99.0, 97.5, 50.0, 100.0]))))


@pytest.mark.parametrize("i", range(len(CLIP_CASES)))
def test_random_quantize_weight_clipped(w8a8, i):
    """Percentile-clipped weight quantization: codes and scales bit-exact."""
    import test_gpu_clip as tc
    bits, gs, N, kk, pct = CLIP_CASES[i]
    K = kk * 128
    W = tc.weights(N, K, seed=9000 + i)
    tp.note(f"clip case {i}: bits={bits} gs={gs} N={N} K={K} pct={pct}")
    wq, sw = w8a8.quantize_weight_clipped(torch.from_numpy(W).cuda(), bits, gs, pct)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_weight_clipped(W, bits, gs, pct)
    assert (sw.cpu().numpy().view(np.uint32) == rs.view(np.uint32)).all(), f"clip case {i}: scales differ"
    assert (wq.cpu().numpy() == rq).all(), f"clip case {i}: codes differ"
