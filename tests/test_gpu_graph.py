"""Graph capture of the entry points (the benchmark replays its steps as a captured graph).

Every entry point is captured on a side stream, and the graph is replayed several times
with unrelated eager work and synchronizations between replays. Each replay must give
outputs identical, bit for bit, to the same calls issued eagerly. The library enqueues
kernels only (no allocation, no memset), so nothing in it depends on capture state.
"""
import sys

import numpy as np
import pytest
import torch

from synth_inputs import linear_inputs

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


def test_graph_replays_equal_eager(w8a8):
    # shapes that take the alternating-groups per-channel kernel, the per-group and W4A8
    # kernels, and the fused small-M kernel
    xl, Wl = linear_inputs(600, 1280, 2560, seed=41)
    xs, Ws = linear_inputs(3, 1040, 2560, seed=42)
    x = torch.from_numpy(xl).cuda()
    x1 = torch.from_numpy(xs).cuda()
    wq, sw = w8a8.quantize_weight(torch.from_numpy(Wl).cuda(), 8, 0)
    wg, sg = w8a8.quantize_weight(torch.from_numpy(Wl).cuda(), 8, 128)
    w4, s4 = w8a8.quantize_weight(torch.from_numpy(Wl).cuda(), 4, 64)
    ws1, ss1 = w8a8.quantize_weight(torch.from_numpy(Ws).cuda(), 8, 0)
    xq = torch.empty((600, 2560), dtype=torch.int8, device="cuda")
    sx = torch.empty((600,), dtype=torch.float32, device="cuda")
    outs = [torch.empty((600, 1280), dtype=dt, device="cuda") for dt in (torch.float16, torch.bfloat16, torch.float16)]
    y1 = torch.empty((3, 1040), dtype=torch.float16, device="cuda")
    xq1 = torch.empty((3, 2560), dtype=torch.int8, device="cuda")
    sx1 = torch.empty((3,), dtype=torch.float32, device="cuda")

    def step():
        s = torch.cuda.current_stream()
        w8a8.quantize_per_token(x, xq, sx, stream=s)
        w8a8.w8a8_debug_force_config(13)  # the alternating-groups kernel (chosen at large M)
        try:
            w8a8.w8a8_gemm_pc(xq, sx, wq, sw, y=outs[0], stream=s)
        finally:
            w8a8.w8a8_debug_force_config(-1)
        w8a8.w8a8_gemm_pg(xq, sx, wg, sg, 128, y=outs[1], stream=s)
        w8a8.w4a8_gemm_pg(xq, sx, w4, s4, 64, y=outs[2], stream=s)
        w8a8.w8a8_linear(x1, ws1, ss1, 8, 0, y=y1, x_q=xq1, s_x=sx1, stream=s)

    tensors = [xq, sx, *outs, y1, xq1, sx1]
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in tensors]
    for t in tensors:
        t.zero_()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    junk = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        note(f"graph replay {rep}")
        for t in tensors:
            t.zero_()
        junk.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("x_q", "s_x", "pc", "pg128", "w4", "linear y", "linear x_q", "linear s_x"),
                                  tensors, eager):
            assert torch.equal(got.view(torch.uint8) if got.dtype != torch.uint8 else got,
                               ref.view(torch.uint8) if ref.dtype != torch.uint8 else ref), \
                f"replay {rep}: {name} differs from the eager result"
