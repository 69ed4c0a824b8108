"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: int8 codes, fp32 scales, int32 accumulators. Outputs: within the
tolerance of tests/_parity.py (1 ulp for fp16/bf16, 1e-5 relative for fp32, plus
the fp32 evaluation bound for per-group sums). Inputs come from synth_inputs (the
same seeded generator for both sides); every expected value comes from the oracle.
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


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_quantize(w8a8, x_np):
    xq, sx = w8a8.quantize_per_token(dev(x_np))
    torch.cuda.synchronize()
    return host(xq), host(sx)


# ---- activation quantization -----------------------------------------------------------

@pytest.mark.parametrize("M,K", [(1, 2560), (3, 64), (65, 2560), (128, 2560), (300, 10240), (129, 4096),
                                 (17, 12288), (5, 8), (7, 24), (2, 20000), (1000, 2560)])
def test_quantize_per_token(w8a8, M, K):
    note(f"quantize_per_token M={M} K={K}")
    x, _ = linear_inputs(M, 16, K, seed=M * 7 + K)
    xq, sx = gpu_quantize(w8a8, x)
    rq, rs = oracle.quantize_per_token(x)
    assert (sx.view(np.uint32) == rs.view(np.uint32)).all()
    assert (xq == rq).all()


def edge_rows(K=256):
    rng = np.random.default_rng(99)
    rows = [np.zeros(K), np.full(K, 3.0), np.full(K, -7.25), np.full(K, 65504.0),
            np.where(np.arange(K) % 2 == 0, 65504.0, -65504.0),
            np.ldexp(rng.integers(-1023, 1024, K).astype(np.float64), -24),  # subnormals
            np.eye(1, K, 17)[0] * 1000.0,  # one-hot outlier
            -np.abs(rng.standard_normal(K)),  # all negative
            rng.standard_normal(K) * 1e-3]
    ties = np.zeros(K)  # max 127 -> scale 1 exactly; half-integers are exact ties
    ties[:8] = [127.0, 2.5, -2.5, 3.5, -3.5, 0.5, -0.5, 126.5]
    ties[8:] = (rng.integers(-254, 255, K - 8) / 2.0)
    rows.append(ties)
    return np.stack(rows).astype(np.float16)


def test_quantize_edge_rows(w8a8):
    note("quantize edge rows")
    x = edge_rows()
    xq, sx = gpu_quantize(w8a8, x)
    rq, rs = oracle.quantize_per_token(x)
    assert (sx.view(np.uint32) == rs.view(np.uint32)).all()
    assert (xq == rq).all()
    assert sx[0] == 0 and (xq[0] == 0).all()
    assert xq[-1, :8].tolist() == [127, 2, -2, 4, -4, 0, 0, 126]


def test_quantize_strided_and_bf16(w8a8):
    note("quantize strided + bf16")
    x, _ = linear_inputs(70, 16, 2560, seed=5)
    wide = np.zeros((70, 2560 + 64), np.float16)
    wide[:, :2560] = x
    t = dev(wide)[:, :2560]
    xq, sx = w8a8.quantize_per_token(t)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_per_token(x)
    assert (host(xq) == rq).all() and (host(sx) == rs).all()
    # bf16 input
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    xq, sx = w8a8.quantize_per_token(xb.cuda())
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_per_token_bf16(bits)
    assert (host(xq) == rq).all() and (host(sx).view(np.uint32) == rs.view(np.uint32)).all()


@pytest.mark.parametrize("K", [256, 2560, 4096])
def test_quantize_ties_and_magnitudes_each_row_kernel(w8a8, K):
    """Exact ties (row maximum 127 * 2^j, so s = 2^j and half-integer multiples of s are
    ties) and a spread of every magnitude below sampled maxima, for fp16 and bf16, at row
    lengths taken by the wave-per-row (K=256), wave-pair (K=2560) and workgroup-per-row
    (K=4096) kernels: codes and scales bit-exact against the oracle."""
    note(f"quantize ties + magnitudes K={K}")
    rng = np.random.default_rng(K)
    rows = []
    for j in (-20, -3, 0, 5, 9):
        r = rng.integers(-254, 255, K) / 2.0  # half-integers: ties at s = 1
        r[0] = 127.0
        rows.append(np.ldexp(r, j))
    x16 = np.stack(rows).astype(np.float16)
    assert (np.abs(x16.astype(np.float64)).max(axis=1) == np.ldexp(127.0, np.array([-20, -3, 0, 5, 9]))).all()
    # fp16: sampled maxima, each row a spread of the magnitudes up to the maximum, both signs
    maxima = np.concatenate([[0x7BFF, 0x3C00, 0x0400, 0x03FF], rng.integers(1, 0x7C00, 12)]).astype(np.uint16)
    spread = np.zeros((len(maxima), K), np.uint16)
    for i, mb in enumerate(maxima):
        mags = np.sort(rng.integers(0, int(mb) + 1, K // 2).astype(np.uint16))
        mags[-1] = mb
        v = np.concatenate([mags, mags | 0x8000])
        spread[i] = rng.permutation(v)
    x = np.concatenate([x16, spread.view(np.float16)])
    xq, sx = gpu_quantize(w8a8, x)
    rq, rs = oracle.quantize_per_token(x)
    assert (sx.view(np.uint32) == rs.view(np.uint32)).all()
    assert (xq == rq).all()
    # bf16: the same tie rows (exact in bf16) and spreads of bf16 magnitudes down to 2^-100
    # (the fast path's lower limit) and below it
    b16 = x16.astype(np.float32).view(np.uint32) >> 16
    assert ((b16.astype(np.uint32) << 16).view(np.float32) == x16.astype(np.float32)).all()
    # 0x10FE = 127 * 2^-100 (s = 2^-100, the fast path's smallest scale), 0x10FD just below
    bmax = np.concatenate([[0x7F7F, 0x3F80, 0x10FF, 0x10FE, 0x10FD, 0x0D80, 0x0080],
                           rng.integers(0x0100, 0x7F80, 9)]).astype(np.uint16)
    bspread = np.zeros((len(bmax), K), np.uint16)
    for i, mb in enumerate(bmax):
        mags = np.sort(rng.integers(0, int(mb) + 1, K // 2).astype(np.uint16))
        mags[-1] = mb
        bspread[i] = rng.permutation(np.concatenate([mags, mags | 0x8000]))
    bits = np.concatenate([b16.astype(np.uint16), bspread])
    xb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    xq, sx = w8a8.quantize_per_token(xb.cuda())
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_per_token_bf16(bits)
    assert (host(sx).view(np.uint32) == rs.view(np.uint32)).all()
    assert (host(xq) == rq).all()


def test_quantize_empty_batch(w8a8):
    xq, sx = w8a8.quantize_per_token(torch.zeros((0, 256), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert xq.shape == (0, 256) and sx.shape == (0,)


# ---- weight quantization ---------------------------------------------------------------

@pytest.mark.parametrize("bits,gs,N,K", [(8, 0, 272, 2560), (8, 64, 272, 2560), (8, 128, 48, 384),
                                         (4, 128, 272, 2560), (4, 64, 48, 384),
                                         (8, 0, 10240, 2560), (4, 128, 10240, 2560), (4, 0, 272, 2560),
                                         (4, 0, 10240, 2560)])
def test_quantize_weight(w8a8, bits, gs, N, K):
    note(f"quantize_weight bits={bits} gs={gs} N={N} K={K}")
    _, W = linear_inputs(0, N, K, seed=N + K + gs)
    W[3, :gs or K] = 0.0  # an all-zero group / row
    wq, sw = w8a8.quantize_weight(dev(W), bits, gs)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_weight(W, bits, gs)
    assert (host(sw).view(np.uint32) == rs.view(np.uint32)).all()
    assert (host(wq) == rq).all()


# ---- GEMM + dequant ----------------------------------------------------------------------

MODES = ["pc", "pg64", "pg128", "w4_128", "w4_64", "w4_0"]


def run_mode(w8a8, mode, x, W, out_dtype, y=None):
    """GPU path end to end from raw x and W. Returns (y, x_q, s_x)."""
    xq, sx = w8a8.quantize_per_token(dev(x))
    Wd = dev(W)
    if mode == "pc":
        wq, sw = w8a8.quantize_weight(Wd, 8, 0)
        yt = w8a8.w8a8_gemm_pc(xq, sx, wq, sw, out_dtype, y=y)
    elif mode.startswith("pg"):
        gs = int(mode[2:])
        wq, sw = w8a8.quantize_weight(Wd, 8, gs)
        yt = w8a8.w8a8_gemm_pg(xq, sx, wq, sw, gs, out_dtype, y=y)
    else:
        gs = int(mode[3:])
        wq, sw = w8a8.quantize_weight(Wd, 4, gs)
        if gs:
            yt = w8a8.w4a8_gemm_pg(xq, sx, wq, sw, gs, out_dtype, y=y)
        else:
            yt = w8a8.w4a8_gemm_pc(xq, sx, wq, sw, out_dtype, y=y)
    torch.cuda.synchronize()
    return yt


def oracle_mode(mode, x, W):
    if mode == "pc":
        wq, sw = oracle.quantize_weight(W, 8, 0)
        r = oracle.linear_pc(x, wq, sw)
        r["mag"], r["G"] = np.abs(r["y"]), 1
    elif mode.startswith("pg"):
        gs = int(mode[2:])
        wq, sw = oracle.quantize_weight(W, 8, gs)
        r = oracle.linear_pg(x, wq, sw, gs)
        r["G"] = W.shape[1] // gs
    else:
        gs = int(mode[3:])
        wq, sw = oracle.quantize_weight(W, 4, gs)
        r = oracle.linear_w4(x, wq, sw, gs)
        if gs:
            r["G"] = W.shape[1] // gs
        else:
            r["mag"], r["G"] = np.abs(r["y"]), 1
    return r


def compare(yt, r, what):
    """int32 sums bit-exact; outputs within the fp32 evaluation bound of the fp64 value and,
    for every kernel that folds in the pages' fp32 order (all but the per-group GEMV that
    M <= 16 runs, which splits a row's K range over waves), bit-exact against the oracle's
    fp32 evaluation rounded once to the output format."""
    if yt.dtype == torch.int32:
        got = host(yt)
        assert (got == r["acc"]).all(), f"{what}: int32 accumulators differ"
        return
    got = host(yt)
    check_output(got, OUT_FMT[yt.dtype], r["y"], r["mag"], r["G"], what)
    if r["G"] == 1 or got.shape[0] > 16:
        check_exact(got, OUT_FMT[yt.dtype], r["y32"], what)


SHAPES = [(37, 272, 384), (300, 1040, 2560), (128, 512, 640), (1, 16, 128), (65, 48, 256), (513, 272, 1280),
          (16, 272, 1280), (7, 1040, 640), (2, 48, 10240), (9, 16, 12288), (3, 32, 4096)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_parity(w8a8, mode, M, N, K):
    x, W = linear_inputs(M, N, K, seed=M + N + K)
    r = oracle_mode(mode, x, W)
    for out in (torch.float16, torch.bfloat16, torch.float32, torch.int32):
        note(f"gemm {mode} M={M} N={N} K={K} out={out}")
        compare(run_mode(w8a8, mode, x, W, out), r, f"{mode} {M}x{N}x{K} {out}")


def test_gemm_strided_output_and_empty(w8a8):
    note("gemm strided y, M=0")
    x, W = linear_inputs(50, 272, 512, seed=3)
    r = oracle_mode("pc", x, W)
    ybig = torch.full((50, 272 + 32), 7.0, dtype=torch.float16, device="cuda")
    run_mode(w8a8, "pc", x, W, torch.float16, y=ybig[:, :272])
    got = host(ybig)
    check_output(got[:, :272], "f16", r["y"], r["mag"], 1, "strided y")
    assert (got[:, 272:] == np.float16(7.0)).all()  # padding columns untouched
    # row strides of 304 (16-byte rows: staged stores) and 276 (8-byte rows: direct
    # stores), both 16-bit types, in the automatic choice and the DMA-pipeline kernels
    try:
        for cfg in (-1, 6, 7, 13, 16, 17, 18, 19, 20):
            w8a8.w8a8_debug_force_config(cfg)
            for ldy in (304, 276):
                for out, fmt in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
                    note(f"gemm strided y: config {cfg} ldy={ldy} {fmt}")
                    ybig = torch.zeros((50, ldy), dtype=out, device="cuda")
                    run_mode(w8a8, "pc", x, W, out, y=ybig[:, :272])
                    got = host(ybig)
                    check_output(got[:, :272], fmt, r["y"], r["mag"], 1, f"cfg {cfg} ldy={ldy} {fmt}")
                    assert (got[:, 272:] == 0).all()
    finally:
        w8a8.w8a8_debug_force_config(-1)
    xq = torch.zeros((0, 512), dtype=torch.int8, device="cuda")
    sx = torch.zeros((0,), dtype=torch.float32, device="cuda")
    wq = torch.zeros((272, 512), dtype=torch.int8, device="cuda")
    sw = torch.zeros((272,), dtype=torch.float32, device="cuda")
    y = w8a8.w8a8_gemm_pc(xq, sx, wq, sw)
    torch.cuda.synchronize()
    assert y.shape == (0, 272)


@pytest.mark.parametrize("M,N,K,pad", [(4000, 10000, 512, 0), (2100, 12000, 256, 8)])
def test_pc_several_rounds_of_tiles(w8a8, M, N, K, pad):
    """More output tiles than compute units (several rounds of workgroups) in the ping-pong
    configurations 16, 18, 19 and 20 with 16-bit outputs staged in LDS: partial tiles in M and N,
    contiguous and strided output rows; bit-exact against the oracle's fp32 evaluation, and
    the padding columns untouched."""
    x, W = linear_inputs(M, N, K, seed=M + N)
    r = oracle_mode("pc", x, W)
    try:
        for cfg in (-1, 16, 18, 19, 20):
            w8a8.w8a8_debug_force_config(cfg)
            for out, fmt in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
                note(f"several rounds: config {cfg} M={M} N={N} K={K} ldy={N + pad} {fmt}")
                ybig = torch.zeros((M, N + pad), dtype=out, device="cuda")
                run_mode(w8a8, "pc", x, W, out, y=ybig[:, :N])
                got = host(ybig)
                check_exact(got[:, :N], fmt, r["y32"], f"cfg {cfg} {M}x{N}x{K} {fmt}")
                assert (got[:, N:] == 0).all()
    finally:
        w8a8.w8a8_debug_force_config(-1)


@pytest.mark.parametrize("K", [128, 256, 384, 640])
def test_pp_split_dma_stage_counts(w8a8, K):
    """The ping-pong configurations with each stage's DMA split over two memory phases (19,
    20) and their one-phase forms (16, 18) at one, two, three and five 128-value stages: the
    first stage issued in the prologue only, group 1's share of stage 1 issued before its
    late start, the last stage with no DMA after it, an odd stage count; partial tiles in M
    and N. Bit-exact against the oracle's fp32 evaluation (fp16) and its int32 sums, and
    identical across the four configurations."""
    M, N = 300, 704
    x, W = linear_inputs(M, N, K, seed=K)
    r = oracle_mode("pc", x, W)
    outs = {}
    try:
        for cfg in (16, 18, 19, 20):
            w8a8.w8a8_debug_force_config(cfg)
            for out, fmt in ((torch.float16, "f16"), (torch.int32, "i32")):
                note(f"split DMA: config {cfg} K={K} {fmt}")
                y = host(run_mode(w8a8, "pc", x, W, out))
                if fmt == "f16":
                    check_exact(y, fmt, r["y32"], f"cfg {cfg} K={K}")
                else:
                    assert (y.astype(np.int64) == r["acc"]).all(), f"cfg {cfg} K={K}: int32 sums differ"
                outs.setdefault(fmt, []).append(y)
    finally:
        w8a8.w8a8_debug_force_config(-1)
    for fmt, ys in outs.items():
        for y in ys[1:]:
            assert (y.view(np.uint8) == ys[0].view(np.uint8)).all(), f"configurations differ ({fmt}, K={K})"


@pytest.mark.parametrize("mode", ["pc", "pg64", "w4_128", "w4_0"])
def test_every_config_identical(w8a8, mode):
    """Every tile configuration gives bit-identical results (catches edge-mask and LDS races)."""
    M, N, K = 300, 528, 1280
    x, W = linear_inputs(M, N, K, seed=11)
    r = oracle_mode(mode, x, W)
    n_cfg = w8a8.w8a8_debug_force_config(-1)
    outs = {}
    try:
        for cfg in range(-1, n_cfg):
            w8a8.w8a8_debug_force_config(cfg)
            for out in (torch.float16, torch.int32):
                note(f"config {cfg} {mode} {out}")
                y = run_mode(w8a8, mode, x, W, out)
                compare(y, r, f"cfg {cfg} {mode}")
                outs.setdefault(out, []).append(host(y))
                y2 = run_mode(w8a8, mode, x, W, out)
                assert (host(y2) == outs[out][-1]).all(), "non-deterministic"
    finally:
        w8a8.w8a8_debug_force_config(-1)
    for out, ys in outs.items():
        for y in ys[1:]:
            assert (y.view(np.uint8) == ys[0].view(np.uint8)).all(), f"configs differ ({out})"


# ---- shapes that route to specific tile configurations, at full size, every row --------
# (the points of the workload definitions themselves are in test_gpu_fullsize.py)

@pytest.mark.parametrize("mode,M,N,K", [
    ("pc", 2048, 1024, 4096),     # 64 x 128 tiles, one round (Qwen3 k/v shape)
    ("pc", 1536, 2560, 10240),    # 128 x 128 tiles, one round
    ("pg128", 768, 2560, 10240),  # 64 x 64 per-group DMA tiles
    ("w4_0", 1, 10240, 2560),     # per-column int4: GEMV
    ("w4_0", 1024, 10240, 2560),  # 320 x 256 ping-pong tiles, int4 unpacked in the memory phase
    ("w4_0", 4096, 10240, 2560),
    ("w4_0", 2048, 2560, 10240),  # 128 x 256 DMA tiles without the fold
    ("w4_0", 768, 2560, 10240),   # 64 x 64 DMA tiles without the fold
])
def test_full_size_config_shapes(w8a8, mode, M, N, K):
    note(f"full size {mode} M={M} N={N} K={K}")
    x, W = linear_inputs(M, N, K, seed=0)
    xq, sx = gpu_quantize(w8a8, x)
    rq, rs = oracle.quantize_per_token(x)
    assert (xq == rq).all() and (sx.view(np.uint32) == rs.view(np.uint32)).all()
    r = oracle_mode(mode, x, W)
    for out in (torch.float16, torch.int32):
        compare(run_mode(w8a8, mode, x, W, out), r, f"{mode} {M}x{N}x{K} {out}")


@pytest.mark.parametrize("mode", ["pg128", "w4_128", "pg64"])
@pytest.mark.parametrize("M,N,K", [(300, 528, 128), (300, 528, 256), (513, 272, 384)])
def test_grouped_few_k_tiles(w8a8, mode, M, N, K):
    """The per-group DMA kernels (128 x 256 and 64 x 64 forms) with one, two and three
    128-value K-tiles: the first group's fold of zeros, the loop with no barrier inside, and
    (gs = 128) the two halves of the workgroup that fold half a K-tile apart; ragged M and N."""
    x, W = linear_inputs(M, N, K, seed=M + K)
    r = oracle_mode(mode, x, W)
    try:
        for cfg in (11, 12):
            w8a8.w8a8_debug_force_config(cfg)
            for out in (torch.float16, torch.int32):
                note(f"few K-tiles {mode} {M}x{N}x{K} config {cfg} {out}")
                compare(run_mode(w8a8, mode, x, W, out), r, f"cfg {cfg} {mode} {M}x{N}x{K} {out}")
    finally:
        w8a8.w8a8_debug_force_config(-1)


@pytest.mark.parametrize("K", [130816, 130944, 131072])
@pytest.mark.parametrize("M", [2, 300])
def test_int4_per_channel_extreme_sums(w8a8, M, K):
    """int4 weights with per-channel scales, raw int32 sums at their largest: every activation
    code -128 and every weight -8 (stored nibble 0), so each sum is K * 1024 (closed form).
    The paths that sum 16 q in int32 (16 K 1024 < 2^31) take K up to 130944 in whole
    128-value K-tiles (M > 16; 130816 is the last that the DMA GEMV, K % 256 == 0, takes at
    M <= 16); K = 131072 must take the kernels that sum q."""
    N = 64
    xq = torch.full((M, K), -128, dtype=torch.int8, device="cuda")
    sx = torch.ones((M,), dtype=torch.float32, device="cuda")
    wq = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.ones((N,), dtype=torch.float32, device="cuda")
    cfgs = (-1, 17) if M > 16 else (-1,)
    try:
        for cfg in cfgs:
            w8a8.w8a8_debug_force_config(cfg)
            note(f"int4 extreme sums M={M} K={K} config {cfg}")
            y = w8a8.w4a8_gemm_pc(xq, sx, wq, sw, torch.int32)
            torch.cuda.synchronize()
            got = host(y)
            assert (got == K * 1024).all(), f"M={M} K={K} cfg {cfg}: {np.unique(got)[:4]} against {K * 1024}"
    finally:
        w8a8.w8a8_debug_force_config(-1)


def _bf16_rne_bits(f32: np.ndarray) -> np.ndarray:
    u = f32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("M,N,K,cfgs", [(300, 528, 1280, (-1, 0, 1, 4, 5, 6, 7, 13, 16, 18)), (9, 1040, 640, (-1, 10, 4)),
                                        (2000, 5280, 384, (-1, 6, 7, 13, 16, 18))])
def test_pc_epilogue_rounding_exact(w8a8, M, N, K, cfgs):
    """Per-channel outputs are RNE of the fp32 value ((fp32)acc * s_x) * s_w, two fp32
    roundings and then one to fp16/bf16, in every tile configuration: checked exactly
    (not to a tolerance) from the GPU's own int32 accumulators and scales, which the
    other tests hold bit-exact against the oracle. Catches a multiply fused into the
    fp16 conversion (one rounding), which differs at fp16 ties only."""
    x, W = linear_inputs(M, N, K, seed=17)
    xq, sx = w8a8.quantize_per_token(dev(x))
    wq, sw = w8a8.quantize_weight(dev(W), 8, 0)
    try:
        for cfg in cfgs:
            w8a8.w8a8_debug_force_config(cfg)
            note(f"epilogue rounding: config {cfg} M={M} N={N} K={K}")
            acc = host(w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.int32))
            y32 = (acc.astype(np.float32) * host(sx)[:, None]) * host(sw)[None, :]
            y16 = host(w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.float16))
            bad = np.argwhere(y16.view(np.uint16) != y32.astype(np.float16).view(np.uint16))
            assert len(bad) == 0, f"config {cfg}: fp16 rounding differs at {bad[:4].tolist()}"
            yb = host(w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.bfloat16))
            assert (yb == _bf16_rne_bits(y32)).all(), f"config {cfg}: bf16 rounding differs"
            yf = host(w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.float32))
            assert (yf.view(np.uint32) == y32.view(np.uint32)).all(), f"config {cfg}: fp32 output differs"
    finally:
        w8a8.w8a8_debug_force_config(-1)


def test_concatenated_projections_equal_separate(w8a8):
    """Projections that share an input (q, k, v; gate, up) run as one GEMM over their
    concatenated weights in the block benchmark: per-channel scales belong to output rows,
    so each column block is bit-identical to the projection's own GEMM (which the tests
    above hold against the oracle), whatever tile configuration each shape selects."""
    note("concatenated projections")
    x, W = linear_inputs(520, 1024 + 256 + 256, 1024, seed=23)
    xq, sx = w8a8.quantize_per_token(dev(x))
    wq, sw = w8a8.quantize_weight(dev(W), 8, 0)
    y = host(w8a8.w8a8_gemm_pc(xq, sx, wq, sw, torch.bfloat16))
    for a, b in ((0, 1024), (1024, 1280), (1280, 1536)):
        wq_i, sw_i = w8a8.quantize_weight(dev(W[a:b]), 8, 0)
        y_i = host(w8a8.w8a8_gemm_pc(xq, sx, wq_i, sw_i, torch.bfloat16))
        assert (y[:, a:b] == y_i).all(), f"columns {a}:{b} differ"


def test_quantize_all_fp16_values_sampled_maxima(w8a8):
    """For 96 row maxima (extremes + random), a row holding every fp16 value of magnitude
    <= the maximum, both signs: codes and scales bit-exact against the oracle's IEEE
    division (covers every quotient the per-row reciprocal path can meet for those rows)."""
    note("quantize: all fp16 element values under sampled maxima")
    rng = np.random.default_rng(31)
    maxima = np.concatenate([[1, 2, 0x3C00, 0x7BFF, 0x7BFE, 0x0400, 0x03FF, 0x5BF0],
                             rng.integers(1, 0x7C00, 88)]).astype(np.uint16)
    K = 2 * 0x7C00  # room for every magnitude of both signs
    rows = np.zeros((len(maxima), K), np.uint16)
    for i, mb in enumerate(maxima):
        mags = np.arange(0, int(mb) + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | 0x8000])
        rows[i, :len(vals)] = vals
    x = rows.view(np.float16)
    xq, sx = gpu_quantize(w8a8, x)
    rq, rs = oracle.quantize_per_token(x)
    assert (sx.view(np.uint32) == rs.view(np.uint32)).all()
    assert (xq == rq).all()


@pytest.mark.parametrize("mode", ["pg64", "w4_64"])
@pytest.mark.parametrize("M,N,K", [(300, 272, 320), (257, 48, 64)])
def test_grouped_k_not_multiple_of_128(w8a8, mode, M, N, K):
    """Per-group shapes whose K is a multiple of 64 but not 128 (the register-staged kernel)."""
    note(f"grouped K%128 != 0 {mode} M={M} N={N} K={K}")
    x, W = linear_inputs(M, N, K, seed=M + K)
    r = oracle_mode(mode, x, W)
    for out in (torch.float16, torch.float32, torch.int32):
        compare(run_mode(w8a8, mode, x, W, out), r, f"{mode} {M}x{N}x{K} {out}")
