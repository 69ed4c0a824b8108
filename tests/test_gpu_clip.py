"""GPU parity of quantize_weight_clipped (percentile-clipped weight scales) against the CPU
oracle: codes and scales bit for bit, including percentile 100 (min-max), ties, zero and
one-sided runs, outliers, int8 and int4, per channel and per group."""
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


def weights(N, K, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[:, rng.choice(K, max(1, K // 100), replace=False)] *= 40.0  # outlier columns
    W[0, :] = 0.0                                                 # zero run(s)
    W[1, :] = -np.abs(W[1, :])                                    # one-sided
    W[2, :] = np.round(W[2, :] * 200) / 200                       # many ties
    W[3, : K // 2] = 0.0                                          # half zeros
    return W


@pytest.mark.parametrize("bits,gs", [(8, 0), (8, 64), (8, 128), (4, 64), (4, 128), (4, 0)])
@pytest.mark.parametrize("N,K", [(272, 2560), (48, 384), (16, 10240)])
def test_clipped_bit_exact(w8a8, bits, gs, N, K):
    W = weights(N, K, seed=N + K + gs + bits)
    Wd = torch.from_numpy(W).cuda()
    for pct in (99.9, 99.0, 50.0, 0.5, 100.0, 1e-3, 99.99):
        note(f"quantize_weight_clipped bits={bits} gs={gs} N={N} K={K} pct={pct}")
        wq, sw = w8a8.quantize_weight_clipped(Wd, bits, gs, pct)
        torch.cuda.synchronize()
        rq, rs = oracle.quantize_weight_clipped(W, bits, gs, pct)
        got_s = sw.cpu().numpy()
        assert (got_s.view(np.uint32) == rs.view(np.uint32)).all(), \
            f"scales differ at {np.argwhere(got_s.view(np.uint32) != rs.view(np.uint32))[:4].tolist()}"
        assert (wq.cpu().numpy() == rq).all(), "codes differ"


def test_clipped_100_equals_min_max_on_gpu(w8a8):
    W = torch.from_numpy(weights(64, 1280, seed=7)).cuda()
    for bits, gs in ((8, 0), (8, 128), (4, 64)):
        a = w8a8.quantize_weight(W, bits, gs)
        b = w8a8.quantize_weight_clipped(W, bits, gs, 100.0)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))
