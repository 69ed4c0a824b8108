"""Parity at seeded random shapes: every weight format and output type against the oracle,
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
