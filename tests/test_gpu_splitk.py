"""GPU parity of the split-K calls (w8a8_gemm_splitk) through the C ABI.

Per-channel and I32 results must be bit-identical to the single-pass GEMM calls (int32
slice sums are exact in any order) and match the oracle; per-group and W4A8 results must
match the oracle within the fp32 tolerance of tests/_parity.py. Every configuration with a
split form is run with slice counts that divide the K-tiles evenly and unevenly, at ragged
M and N.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import linear_inputs
from _parity import check_exact, check_output

pytestmark = pytest.mark.gpu

OUT_FMT = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
KIND = {"pc": (8, 0), "pg64": (8, 64), "pg128": (8, 128), "w4_64": (4, 64), "w4_128": (4, 128)}
SPLIT_CFGS = {"pc": (7, 12, 14), "pg64": (11, 12), "pg128": (11, 12), "w4_64": (11, 12), "w4_128": (11, 12)}


def has_split(mode, cfg, out):
    """I32 output is the plain integer product: the per-channel slice kernels (int8 weights)."""
    if out == torch.int32:
        return KIND[mode][0] == 8 and cfg in SPLIT_CFGS["pc"]
    return cfg in SPLIT_CFGS[mode]


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
    yield w
    w.w8a8_debug_force_config(-1)
    w.w8a8_debug_force_splitk(-1)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class Problem:
    """Operands on the device (quantized by the library) and the oracle's results."""

    def __init__(self, w8a8, mode, M, N, K, seed, rows=None):
        self.mode, self.M, self.N, self.K = mode, M, N, K
        self.bits, self.gs = KIND[mode]
        x, W = linear_inputs(M, N, K, seed=seed)
        self.xq, self.sx = w8a8.quantize_per_token(dev(x))
        self.wq, self.sw = w8a8.quantize_weight(dev(W), self.bits, self.gs)
        torch.cuda.synchronize()
        xr = x if rows is None else x[rows]
        wq, sw = oracle.quantize_weight(W, self.bits, self.gs)
        if mode == "pc":
            self.r = oracle.linear_pc(xr, wq, sw)
            self.r["mag"], self.G = np.abs(self.r["y"]), 1
        elif self.bits == 8:
            self.r, self.G = oracle.linear_pg(xr, wq, sw, self.gs), K // self.gs
        else:
            self.r, self.G = oracle.linear_w4(xr, wq, sw, self.gs), K // self.gs

    def single(self, w8a8, out, y=None):
        if self.mode == "pc":
            yt = w8a8.w8a8_gemm_pc(self.xq, self.sx, self.wq, self.sw, out, y=y)
        elif self.bits == 8:
            yt = w8a8.w8a8_gemm_pg(self.xq, self.sx, self.wq, self.sw, self.gs, out, y=y)
        else:
            yt = w8a8.w4a8_gemm_pg(self.xq, self.sx, self.wq, self.sw, self.gs, out, y=y)
        torch.cuda.synchronize()
        return yt

    def workspace_bytes(self, w8a8, out):
        return w8a8.w8a8_gemm_splitk_workspace(self.M, self.N, self.K, self.bits, self.gs, out)

    def split(self, w8a8, out, y=None, ws=None):
        if ws is None:
            n = self.workspace_bytes(w8a8, out)
            assert n > 0, "expected a split plan"
            # garbage in the workspace: the slices overwrite every element they use
            ws = torch.full((n // 4,), -123456789, dtype=torch.int32, device="cuda")
        yt = w8a8.w8a8_gemm_splitk(self.xq, self.sx, self.wq, self.sw, self.bits, self.gs, out, y=y,
                                   workspace=ws)
        torch.cuda.synchronize()
        return yt

    def check(self, yt, what, rows=None):
        got = host(yt) if rows is None else host(yt)[rows]
        if yt.dtype == torch.int32:
            assert (got == self.r["acc"]).all(), f"{what}: int32 accumulators differ"
        else:
            check_output(got, OUT_FMT[yt.dtype], self.r["y"], self.r["mag"], self.G, what)


def forced(w8a8, cfg, slices):
    w8a8.w8a8_debug_force_config(cfg)
    w8a8.w8a8_debug_force_splitk(slices)


def reset(w8a8):
    w8a8.w8a8_debug_force_config(-1)
    w8a8.w8a8_debug_force_splitk(-1)


# (M, N, K, slice counts): K-tiles 10, 20 and 80; even and uneven deals, up to one K-tile
# per slice; ragged M (17, 37, 300) and N (272, 1040 against 64 / 128-wide tiles)
CASES = [(300, 528, 1280, (2, 3, 10)), (37, 272, 2560, (4, 7, 20)), (17, 1040, 1280, (5,)),
         (130, 1040, 10240, (3, 16))]


@pytest.mark.parametrize("mode", list(KIND))
@pytest.mark.parametrize("M,N,K,slices", CASES)
def test_splitk_every_config(w8a8, mode, M, N, K, slices):
    prob = Problem(w8a8, mode, M, N, K, seed=M + N + K)
    outs = (torch.float16, torch.bfloat16, torch.float32, torch.int32)
    ref = {out: host(prob.single(w8a8, out)) for out in outs}
    try:
        for cfg in SPLIT_CFGS[mode]:
            for s in slices:
                forced(w8a8, cfg, s)
                for out in outs:
                    if not has_split(mode, cfg, out):
                        assert prob.workspace_bytes(w8a8, out) == 0  # the single pass runs
                        continue
                    what = f"splitk {mode} {M}x{N}x{K} cfg {cfg} slices {s} {out}"
                    note(what)
                    assert prob.workspace_bytes(w8a8, out) == s * M * N * 4
                    yt = prob.split(w8a8, out)
                    prob.check(yt, what)
                    got = host(yt)
                    if mode == "pc" or out == torch.int32:
                        assert (got.view(np.uint8) == ref[out].view(np.uint8)).all(), \
                            f"{what}: differs from the single-pass result"
                    # repeatable: the same plan gives the same bits
                    assert (host(prob.split(w8a8, out)).view(np.uint8) == got.view(np.uint8)).all()
    finally:
        reset(w8a8)


def test_splitk_fallback_and_strided_output(w8a8):
    """No workspace, or one byte short: the single pass runs. A row stride above N leaves the
    padding columns alone."""
    prob = Problem(w8a8, "pc", 200, 1040, 2560, seed=5)
    ref = host(prob.single(w8a8, torch.float16))
    try:
        forced(w8a8, 12, 4)
        n = prob.workspace_bytes(w8a8, torch.float16)
        assert n == 4 * 200 * 1040 * 4
        short = torch.zeros((n - 16) // 4, dtype=torch.int32, device="cuda")
        for ws in (None, short):
            note(f"splitk fallback ws={'none' if ws is None else 'short'}")
            y = w8a8.w8a8_gemm_splitk(prob.xq, prob.sx, prob.wq, prob.sw, 8, 0, torch.float16, workspace=ws)
            torch.cuda.synchronize()
            assert (host(y) == ref).all()
        for cfg in (7, 12, 14):
            forced(w8a8, cfg, 3)
            for out in (torch.float16, torch.bfloat16, torch.float32, torch.int32):
                note(f"splitk strided y cfg {cfg} {out}")
                ybig = torch.zeros((200, 1040 + 24), dtype=out, device="cuda")
                prob.split(w8a8, out, y=ybig[:, :1040])
                got = host(ybig)
                prob.check(ybig[:, :1040], f"strided cfg {cfg} {out}")
                assert (got[:, 1040:] == 0).all(), "padding columns written"
    finally:
        reset(w8a8)


@pytest.mark.parametrize("mode,M,N,K", [("pc", 128, 2560, 10240), ("pc", 1024, 2560, 10240),
                                        ("pg128", 128, 2560, 10240), ("pg64", 1024, 2560, 10240),
                                        ("w4_128", 128, 2560, 10240)])
def test_splitk_automatic_full_size(w8a8, mode, M, N, K):
    """The automatic plan at the narrow-N, long-K workload sizes: every row of the split and
    of the single-pass result against the oracle (the fp32 evaluation bound; the single pass
    also bit-exact against the oracle's fp32 fold), and per-channel split == single pass bit
    for bit."""
    reset(w8a8)
    prob = Problem(w8a8, mode, M, N, K, seed=0)
    note(f"splitk automatic {mode} {M}x{N}x{K}: {prob.workspace_bytes(w8a8, torch.float16)} workspace bytes")
    y = prob.split(w8a8, torch.float16)
    prob.check(y, f"splitk auto {mode} {M}x{N}x{K}")
    single = prob.single(w8a8, torch.float16)
    prob.check(single, f"single pass {mode} {M}x{N}x{K}")
    check_exact(host(single), "f16", prob.r["y32"], f"single pass {mode} {M}x{N}x{K}")
    if mode == "pc":
        assert (host(y) == host(single)).all()


def test_splitk_graph_replay(w8a8):
    """The split call (slice kernel + finish kernel, no memsets) captured in a HIP graph and
    replayed, with eager work between replays: every replay equals the eager result."""
    reset(w8a8)
    prob = Problem(w8a8, "pc", 128, 2560, 10240, seed=9)
    n = prob.workspace_bytes(w8a8, torch.float16)
    assert n > 0
    ws = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    eager = host(prob.split(w8a8, torch.float16, ws=ws))
    y = torch.empty((128, 2560), dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        w8a8.w8a8_gemm_splitk(prob.xq, prob.sx, prob.wq, prob.sw, 8, 0, torch.float16, y=y, workspace=ws,
                              stream=torch.cuda.current_stream())
    for i in range(4):
        note(f"splitk graph replay {i}")
        y.zero_()
        ws.fill_(7)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            g.replay()
        torch.cuda.synchronize()
        assert (host(y) == eager).all(), f"replay {i} differs"
        prob.split(w8a8, torch.float16)  # eager work between replays
