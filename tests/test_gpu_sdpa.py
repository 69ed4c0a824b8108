"""GPU parity of sdpa_decode (decode-step attention) against the CPU oracle.

Tolerance from the arithmetic (u = 2^-24): a score is an fp32 sum of D exact products,
scaled once (error <= (D + 4) u smag, smag = max_n scale sum_d |q_d k_nd|, natural units),
so each probability is off by a relative 2 (D + 4) u smag at most after the max shift,
exp2 adds a few ulps, and the fp32 sums over N keys add (N + 16) u relative; the output
moves by at most twice the largest relative weight error times vmag = sum_n p_n |v_nd|:
    |o - o64| <= ulp_out(o64) + (4 (D + 4) u smag + 2 (N + 16) u + 16 * 2^-23) vmag
(ulp_out: 1 ulp for fp16 / bf16, 2^-24 |o64| for fp32). fp16 runs also require 90 % of the
outputs to equal the correctly rounded reference.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from _parity import ulp, bf16_bits_to_f64

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def w8a8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_activation_quantized_amd as w
    assert w.w8a8_is_available(0), w.w8a8_last_error()
    return w


def to_bf16_bits(x16):
    u = x16.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def inputs(B, Hq, Hkv, N, Ncap, D, seed):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, Hq, D)) * 1.5).astype(np.float16)
    k = rng.standard_normal((B, Hkv, Ncap, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, Ncap, D)).astype(np.float16)
    k[:, :, N:] = np.float16(250.0)  # rows past N: must not count
    v[:, :, N:] = np.float16(-9.0)
    return q, k, v


def dev(a, bf16):
    if bf16:
        return torch.from_numpy(to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def check(o_t, r, N, D, what):
    if o_t.dtype == torch.bfloat16:
        got, fmt = bf16_bits_to_f64(o_t.view(torch.int16).cpu().numpy().view(np.uint16)), "bf16"
    else:
        got, fmt = o_t.cpu().numpy().astype(np.float64), ("f16" if o_t.dtype == torch.float16 else "f32")
    o64 = r["o"]
    E = 4 * (D + 4) * U * r["smag"][:, :, None] + 2 * (N + 16) * U + 16 * 2.0 ** -23
    tol = (U * np.abs(o64) if fmt == "f32" else ulp(o64, fmt)) + E * r["vmag"]
    err = np.abs(got - o64)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of tolerance, max err {err.max():.3g}"
    if fmt == "f16":
        exact = (o_t.cpu().numpy() == o64.astype(np.float16)).mean()
        assert exact >= 0.9, f"{what}: only {exact:.3f} of fp16 outputs equal RNE(o64)"


@pytest.mark.parametrize("B,Hq,Hkv,N,Ncap,D", [
    (1, 32, 8, 1, 1, 128), (1, 32, 8, 17, 40, 128), (1, 32, 8, 1000, 1000, 128), (1, 32, 4, 4096, 4100, 128),
    (2, 8, 8, 300, 300, 64), (1, 16, 1, 777, 800, 128), (3, 12, 4, 2049, 2049, 64), (1, 32, 32, 1024, 1024, 128),
    (1, 32, 4, 32768, 32768, 128),
])
def test_sdpa_parity(w8a8, B, Hq, Hkv, N, Ncap, D):
    q, k, v = inputs(B, Hq, Hkv, N, Ncap, D, seed=B * 7 + Hq + Hkv + N + D)
    ws_n = w8a8.sdpa_decode_workspace(B, Hq, Hkv, N, D)
    ws = torch.full((max(ws_n, 16) // 4,), 12345, dtype=torch.int32, device="cuda")
    for bf16 in (False, True):
        r = oracle.sdpa_decode(*((to_bf16_bits(a) for a in (q, k, v)) if bf16 else (q, k, v)), N=N, bf16=bf16)
        qd, kd, vd = dev(q, bf16), dev(k, bf16), dev(v, bf16)
        for out in (torch.float16, torch.bfloat16, torch.float32):
            for w in ((ws, None) if ws_n > 0 else (None,)):
                what = f"sdpa B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} bf16={bf16} out={out} ws={w is not None}"
                note(what)
                o = w8a8.sdpa_decode(qd, kd, vd, N=N, out_dtype=out, workspace=w)
                torch.cuda.synchronize()
                check(o, r, N, D, what)


@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(1, 32, 8, 4096, 128), (1, 32, 4, 32768, 128), (2, 8, 8, 3000, 64)])
def test_sdpa_autotune(w8a8, B, Hq, Hkv, N, D):
    """The autotuner picks one of its candidate slice counts, records it for the size class
    (N rounded up to a power of two), and later calls in that class (here N and a shorter
    cache) use it and still match the oracle; without a workspace only one slice is tried."""
    q, k, v = inputs(B, Hq, Hkv, N, N, D, seed=B + Hq + Hkv + N)
    qd, kd, vd = dev(q, False), dev(k, False), dev(v, False)
    ws = torch.zeros(max(w8a8.sdpa_decode_workspace(B, Hq, Hkv, N, D), 16) // 4, dtype=torch.int32, device="cuda")
    note(f"sdpa autotune B={B} Hq={Hq} Hkv={Hkv} N={N} D={D}")
    best = w8a8.sdpa_decode_autotune(qd, kd, vd, workspace=ws)
    assert 1 <= best <= max(1, N // 128), best
    N2 = (1 << (N - 1).bit_length()) // 2 + 1  # the shortest cache of the same power-of-two class
    assert w8a8.sdpa_decode_tuned_slices(torch.float16, B, Hq, Hkv, N, D) == best
    assert w8a8.sdpa_decode_tuned_slices(torch.float16, B, Hq, Hkv, N2, D) == best
    for n in (N, N2):
        r = oracle.sdpa_decode(q, k, v, N=n, bf16=False)
        o = w8a8.sdpa_decode(qd, kd, vd, N=n, workspace=ws)
        torch.cuda.synchronize()
        check(o, r, n, D, f"after autotune (best {best}) N={n}")
    assert w8a8.sdpa_decode_autotune(qd, kd, vd, workspace=None) == 1
    w8a8.sdpa_decode_autotune(qd, kd, vd, workspace=ws)  # leave the class tuned with a workspace


def test_sdpa_graph_replay(w8a8):
    B, Hq, Hkv, N, D = 1, 32, 8, 8192, 128
    q, k, v = inputs(B, Hq, Hkv, N, N, D, seed=3)
    qd, kd, vd = dev(q, False), dev(k, False), dev(v, False)
    ws = torch.empty(w8a8.sdpa_decode_workspace(B, Hq, Hkv, N, D) // 4, dtype=torch.int32, device="cuda")
    o = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    w8a8.sdpa_decode(qd, kd, vd, o=o, workspace=ws)
    torch.cuda.synchronize()
    eager = o.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        w8a8.sdpa_decode(qd, kd, vd, o=o, workspace=ws, stream=torch.cuda.current_stream())
    for i in range(4):
        note(f"sdpa graph replay {i}")
        o.zero_()
        ws.fill_(7)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
