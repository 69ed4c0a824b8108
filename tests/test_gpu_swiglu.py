"""GPU parity of swiglu_quantize (the gated MLP's producer of the down projection's int8
input) through the C ABI: int8 codes and fp32 scales bit-exact against the oracle, which
evaluates h = silu(gate) * up in the same specified fp32 steps. Ragged and full sizes
(the Qwen3-8B block's down input: M = 2048, I = 12288), fp16 and bf16, gate and up as the
two halves of one [M, 2 I] array (the gate/up GEMM's output), zero rows and clamped
arguments."""
import sys

import numpy as np
import pytest
import torch

import oracle

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


def inputs(M, I, seed, dtype):
    """gate / up as an [M, 2 I] array (gate first), the distribution of a gate/up projection's
    output at prefill: roughly normal, a few large gate channels."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((M, I)) * 2.0
    u = rng.standard_normal((M, I))
    g[:, rng.choice(I, max(1, I // 256), replace=False)] *= 20
    both = torch.from_numpy(np.concatenate([g, u], axis=1).astype(np.float32)).to(dtype)
    return both


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check(w8a8, both, I, what):
    gate, up = both[:, :I], both[:, I:]
    bits = host_bits(both)
    ox, os_, _ = oracle.swiglu_quantize(bits[:, :I], bits[:, I:], bf16=both.dtype == torch.bfloat16)
    d = both.cuda()
    xq, sx = w8a8.swiglu_quantize(d[:, :I], d[:, I:])
    torch.cuda.synchronize()
    got_q, got_s = xq.cpu().numpy(), sx.cpu().numpy()
    assert (got_s.view(np.uint32) == os_.view(np.uint32)).all(), f"{what}: scales differ"
    bad = np.argwhere(got_q != ox)
    assert len(bad) == 0, f"{what}: {len(bad)} codes differ, first at {bad[0].tolist()}"


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,I", [(1, 8), (3, 64), (37, 384), (5, 2056), (130, 2560), (64, 12288), (9, 20480)])
def test_swiglu_quantize_parity(w8a8, dtype, M, I):
    note(f"swiglu_quantize {dtype} M={M} I={I}")
    check(w8a8, inputs(M, I, seed=M + I, dtype=dtype), I, f"{dtype} {M}x{I}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_swiglu_quantize_full_size(w8a8, dtype):
    """The Qwen3-8B block's down-projection input at prefill: M = 2048, I = 12288, every row."""
    note(f"swiglu_quantize full size {dtype}")
    check(w8a8, inputs(2048, 12288, seed=0, dtype=dtype), 12288, f"full size {dtype}")


def test_swiglu_quantize_special_rows_and_empty(w8a8):
    I = 512
    both = inputs(8, I, seed=7, dtype=torch.bfloat16)
    both[0, :I] = 0.0           # silu(0) = 0: zero row
    both[1, I:] = 0.0           # up = 0: zero row
    both[2, :I] = -200.0        # clamped exp argument: silu tiny, codes of a near-zero row
    both[3, :I] = 100.0         # silu(g) = g
    both[4, :I // 2] = -1e30    # huge negative gates next to normal ones
    both[5] = both[5] * 1e-30   # a row whose scale is below 2^-100 (exact-division path)
    check(w8a8, both, I, "special rows")
    xq, sx = w8a8.swiglu_quantize(torch.zeros((0, 64), dtype=torch.float16, device="cuda"),
                                  torch.zeros((0, 64), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert xq.shape == (0, 64) and sx.shape == (0,)
