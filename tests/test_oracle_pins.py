"""Pins for the CPU oracle: checks it against what the pages and mathematics fix.

None of these tests re-derives a value with the oracle's own code path. They use
hand-worked fixtures (tests/golden/), exact rational arithmetic with an
independent correctly-rounded fp32 routine, closed-form invariants, brute force
on tiny inputs and independent library routines (numpy int64/fp64 matmul).

Which plausible oracle mistake each group of pins catches:
  * wrong divisor (not 127 / 7), reciprocal-multiply instead of division,
    round-half-away instead of half-even, missing clamp  -> golden rows, exact
    rational brute force, exhaustive max -> +-127;
  * dropped or transposed GEMM operand, wrong index     -> brute-force loops,
    numpy int64 matmul on non-square shapes, golden linear;
  * wrong dequant factor / order                         -> golden linear, exact
    rational dequant, fake-quant identity;
  * wrong group boundaries or scale indexing             -> per-group scales vs
    per-slice brute force, gs = K equals per-channel;
  * nibble order or offset in int4 packing               -> golden w4 bytes.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---- an independent, exact model of IEEE binary32 round-to-nearest-even ----------------

def round_to_f32(fr: Fraction) -> Fraction:
    """Correctly round a rational to the nearest binary32 value, ties to even."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q_exp = max(e - 23, -149)  # 24-bit significand; subnormal quantum 2^-149
    scaled = a / Fraction(2) ** q_exp
    n, rem = divmod(scaled.numerator, scaled.denominator)
    rem = Fraction(rem, scaled.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * Fraction(n) * Fraction(2) ** q_exp


def exact_quantize(values, qdiv=127, lo=-128, hi=127):
    """Quantize one run with exact arithmetic + correct fp32 rounding of each step."""
    a = max((abs(Fraction(float(v))) for v in values), default=Fraction(0))
    s = round_to_f32(a / qdiv)
    codes = []
    for v in values:
        if s == 0:
            codes.append(0)
            continue
        t = round_to_f32(Fraction(float(v)) / s)
        q = round(t)  # Python's round on a Fraction: nearest, ties to even
        codes.append(int(min(max(q, lo), hi)))
    return float(s), codes


# ---- activation quantization -------------------------------------------------------------

def test_golden_quantize_rows():
    for case in _golden("quantize_rows.json")["cases"]:
        x = np.array([case["x"]], np.float16)
        q, s = oracle.quantize_per_token(x)
        assert s[0] == np.float32(case["scale"]), case["why"]
        assert q[0].tolist() == case["codes"], case["why"]


def test_exhaustive_fp16_max_maps_to_127():
    """Every positive finite fp16 maximum a: codes of [a, -a] are [127, -127] and
    the scale equals the correctly rounded a/127 (so -128 is never produced)."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)  # all positive finite halves
    a = bits.view(np.float16)
    x = np.stack([a, -a, (a / 3).astype(np.float16)], axis=1)
    q, s = oracle.quantize_per_token(x)
    assert (q[:, 0] == 127).all() and (q[:, 1] == -127).all()
    assert (np.abs(q[:, 2]) <= 127).all()
    # scale against exact rational rounding on an evenly spaced subset (all 31743 is slow)
    for i in range(0, len(a), 97):
        assert Fraction(float(s[i])) == round_to_f32(Fraction(float(a[i])) / 127)


def test_exact_rational_brute_force_rows():
    rng = np.random.default_rng(1)
    rows = []
    for r in range(40):
        v = rng.standard_normal(48).astype(np.float32)
        v[rng.integers(0, 48, 2)] *= 50
        if r % 5 == 1:
            v *= 1e-3  # small magnitudes
        if r % 5 == 2:
            v[:] = np.ldexp(rng.integers(-20, 21, 48), -24).astype(np.float32)  # subnormals
        rows.append(v.astype(np.float16))
    x = np.stack(rows)
    q, s = oracle.quantize_per_token(x)
    for i in range(x.shape[0]):
        es, ec = exact_quantize(x[i])
        assert float(s[i]) == es
        assert q[i].tolist() == ec


def test_quantize_invariants():
    rng = np.random.default_rng(2)
    # values in [2^-6, 2^6] so that scaling by 2^j, |j| <= 4, stays exact in fp16
    mag = np.ldexp(1.0 + rng.random((16, 64)), rng.integers(-6, 6, (16, 64)))
    x = (mag * rng.choice([-1.0, 1.0], (16, 64))).astype(np.float16)
    q, s = oracle.quantize_per_token(x)
    for j in (-4, -1, 1, 3):
        qj, sj = oracle.quantize_per_token((x.astype(np.float32) * 2.0 ** j).astype(np.float16))
        assert (qj == q).all()
        assert (sj == s * np.float32(2.0 ** j)).all()
    qn, sn = oracle.quantize_per_token(-x)
    assert (qn == -q).all() and (sn == s).all()
    # reconstruction error: |x - s q| <= s (1/2 + 2^-17), checked exactly
    for i in range(x.shape[0]):
        si = Fraction(float(s[i]))
        for k in range(x.shape[1]):
            err = abs(Fraction(float(x[i, k])) - si * int(q[i, k]))
            assert err <= si * (Fraction(1, 2) + Fraction(1, 2 ** 17))


def test_zero_and_degenerate_rows():
    x = np.zeros((3, 64), np.float16)
    x[1, 5] = -0.0
    x[2, 7] = np.float16(2.0 ** -24)  # smallest subnormal as the only nonzero
    q, s = oracle.quantize_per_token(x)
    assert s[0] == 0 and s[1] == 0 and (q[:2] == 0).all()
    assert q[2, 7] == 127 and (np.delete(q[2], 7) == 0).all()
    # empty batch
    q0, s0 = oracle.quantize_per_token(np.zeros((0, 64), np.float16))
    assert q0.shape == (0, 64) and s0.shape == (0,)


def test_bf16_input_matches_exact():
    rng = np.random.default_rng(3)
    f = rng.standard_normal((8, 32)).astype(np.float32) * 10
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16 (any bf16 values do)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    q, s = oracle.quantize_per_token_bf16(bits)
    for i in range(8):
        es, ec = exact_quantize(vals[i])
        assert float(s[i]) == es and q[i].tolist() == ec


# ---- weight quantization -----------------------------------------------------------------

@pytest.mark.parametrize("gs", [0, 64, 128])
def test_weight_quantize_against_exact_slices(gs):
    rng = np.random.default_rng(4)
    K = 256
    W = (rng.standard_normal((6, K)) * 0.02).astype(np.float32)
    W[2, 70] = 0.5  # one large weight affects only its own group
    W[3, 128:192] = 0.0  # an all-zero group
    wq, sw = oracle.quantize_weight(W, 8, gs)
    run = gs or K
    for n in range(6):
        for g in range(K // run):
            es, ec = exact_quantize(W[n, g * run:(g + 1) * run])
            got_s = sw[n] if gs == 0 else sw[n, g]
            assert float(got_s) == es
            assert wq[n, g * run:(g + 1) * run].tolist() == ec


def test_golden_w4_pack():
    d = _golden("w4_pack.json")
    W = np.array(d["W"], np.float32)
    packed, s = oracle.quantize_weight(W, 4, d["group_size"])
    assert s.tolist() == d["scale"]
    assert packed.tolist() == d["packed"]
    assert oracle.unpack_int4(packed, W.shape[1]).tolist() == d["codes"]


def test_w4_against_exact_and_range():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((5, 256)) * 0.02).astype(np.float32)
    packed, sw = oracle.quantize_weight(W, 4, 128)
    codes = oracle.unpack_int4(packed, 256)
    assert codes.min() >= -7 and codes.max() <= 7  # -8 unreachable: max maps to +-7
    for n in range(5):
        for g in range(2):
            es, ec = exact_quantize(W[n, g * 128:(g + 1) * 128], qdiv=7, lo=-8, hi=7)
            assert float(sw[n, g]) == es
            assert codes[n, g * 128:(g + 1) * 128].tolist() == ec
    # nibble arithmetic: unpack inverts the documented packing for every code pair
    q = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], np.int8).reshape(1, -1)
    byte = ((q[0, 0::2].astype(np.int32) + 8) | ((q[0, 1::2].astype(np.int32) + 8) << 4)).astype(np.uint8)
    assert (oracle.unpack_int4(byte.reshape(1, -1), q.shape[1]) == q).all()


# ---- integer GEMM ------------------------------------------------------------------------

def test_gemm_brute_force_tiny():
    rng = np.random.default_rng(6)
    xq = rng.integers(-128, 128, (3, 64), dtype=np.int8)
    wq = rng.integers(-128, 128, (5, 64), dtype=np.int8)
    acc = oracle.gemm_i32(xq, wq)
    for m in range(3):
        for n in range(5):
            assert acc[m, n] == sum(int(xq[m, k]) * int(wq[n, k]) for k in range(64))


def test_gemm_vs_numpy_int64():
    rng = np.random.default_rng(7)
    xq = rng.integers(-127, 128, (37, 320), dtype=np.int8)
    wq = rng.integers(-127, 128, (53, 320), dtype=np.int8)
    ref = xq.astype(np.int64) @ wq.astype(np.int64).T
    assert (oracle.gemm_i32(xq, wq) == ref).all()


def test_gemm_overflow_is_detected():
    K = 140000  # 128*128*K > 2^31
    xq = np.full((1, K), -128, np.int8)
    wq = np.full((1, K), -128, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i32(xq, wq)


def test_group_acc_sums_to_full():
    rng = np.random.default_rng(8)
    xq = rng.integers(-127, 128, (9, 256), dtype=np.int8)
    wq = rng.integers(-127, 128, (11, 256), dtype=np.int8)
    accg = oracle.group_acc(xq, wq, 64)
    for g in range(4):
        ref = xq[:, g * 64:(g + 1) * 64].astype(np.int64) @ wq[:, g * 64:(g + 1) * 64].astype(np.int64).T
        assert (accg[:, :, g] == ref).all()


# ---- dequantization ----------------------------------------------------------------------

def test_golden_linear():
    d = _golden("linear_small.json")
    x = np.array(d["x"], np.float16)
    W = np.array(d["W"], np.float32)
    wq, sw = oracle.quantize_weight(W, 8, 0)
    assert wq.tolist() == d["w_codes"] and sw.tolist() == d["w_scale"]
    r = oracle.linear_pc(x, wq, sw)
    assert r["x_q"].tolist() == d["x_codes"] and r["s_x"].tolist() == d["x_scale"]
    assert r["acc"].tolist() == d["acc"]
    assert r["y"].tolist() == d["y"]


def test_dequant_pc_exact_rational():
    rng = np.random.default_rng(9)
    acc = rng.integers(-2 ** 26, 2 ** 26, (7, 9)).astype(np.int32)
    sx = (rng.random(7) * 2).astype(np.float32)
    sw = (rng.random(9) * 1e-3).astype(np.float32)
    y = oracle.dequant_pc(acc, sx, sw)
    for m in range(7):
        for n in range(9):
            exact = Fraction(int(acc[m, n])) * Fraction(float(sx[m])) * Fraction(float(sw[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 51)


def test_dequant_pg_exact_rational_and_mag():
    rng = np.random.default_rng(10)
    G = 5
    accg = rng.integers(-2 ** 20, 2 ** 20, (4, 6, G)).astype(np.int32)
    sx = (rng.random(4) + 0.1).astype(np.float32)
    sw = (rng.random((6, G)) * 1e-3).astype(np.float32)
    y, mag = oracle.dequant_pg(accg, sx, sw)
    for m in range(4):
        for n in range(6):
            terms = [Fraction(float(sw[n, g])) * int(accg[m, n, g]) for g in range(G)]
            exact = Fraction(float(sx[m])) * sum(terms)
            amag = Fraction(float(sx[m])) * sum(abs(t) for t in terms)
            assert abs(Fraction(float(y[m, n])) - exact) <= amag * (G + 2) * Fraction(1, 2 ** 53)
            assert abs(Fraction(float(mag[m, n])) - amag) <= amag * (G + 2) * Fraction(1, 2 ** 53)


def test_pg_with_one_group_equals_pc_and_fake_quant_identity():
    rng = np.random.default_rng(11)
    M, N, K = 20, 24, 256
    x = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, sw = oracle.quantize_weight(W, 8, 0)
    wq1, sw1 = oracle.quantize_weight(W, 8, K)
    assert (wq1 == wq).all() and (sw1[:, 0] == sw).all()
    pc = oracle.linear_pc(x, wq, sw)
    pg = oracle.linear_pg(x, wq1, sw1, K)
    assert (pg["acc"] == pc["acc"]).all()
    np.testing.assert_allclose(pg["y"], pc["y"], rtol=1e-15, atol=0)
    # fake-quant identity: y = (s_x x_q)(s_w w_q)^T, in an independent fp64 matmul
    fq = (pc["s_x"][:, None].astype(np.float64) * pc["x_q"]) @ (sw[:, None].astype(np.float64) * wq).T
    np.testing.assert_allclose(pc["y"], fq, rtol=1e-12, atol=1e-12)
    # per-group fake-quant identity at gs = 64
    wq64, sw64 = oracle.quantize_weight(W, 8, 64)
    r = oracle.linear_pg(x, wq64, sw64, 64)
    wdq = (np.repeat(sw64, 64, axis=1).astype(np.float64) * wq64)
    fq64 = (r["s_x"][:, None].astype(np.float64) * r["x_q"]) @ wdq.T
    np.testing.assert_allclose(r["y"], fq64, rtol=1e-12, atol=1e-12)


def test_w4_path_equals_pg_on_unpacked_codes():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((5, 256)).astype(np.float16)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    packed, sw = oracle.quantize_weight(W, 4, 128)
    r4 = oracle.linear_w4(x, packed, sw, 128)
    r8 = oracle.linear_pg(x, oracle.unpack_int4(packed, 256), sw, 128)
    assert (r4["acc"] == r8["acc"]).all() and (r4["y"] == r8["y"]).all()


def test_golden_w4_per_column():
    """Per-column int4 (group size 0): one scale per output channel, the same nibble packing."""
    d = _golden("w4_per_column.json")
    W = np.array(d["W"], np.float32)
    packed, s = oracle.quantize_weight(W, 4, 0)
    assert s.tolist() == d["scale"]
    assert packed.tolist() == d["packed"]
    assert oracle.unpack_int4(packed, W.shape[1]).tolist() == d["codes"]


def test_w4_per_column_against_exact_rows_and_pc_path():
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((6, 320)) * 0.02).astype(np.float32)
    W[2, 17] = 0.3  # an outlier sets its whole row's scale
    W[4] = 0.0      # an all-zero row: scale 0, codes 0
    packed, sw = oracle.quantize_weight(W, 4, 0)
    codes = oracle.unpack_int4(packed, 320)
    assert sw.shape == (6,) and codes.min() >= -7 and codes.max() <= 7
    for n in range(6):
        es, ec = exact_quantize(W[n], qdiv=7, lo=-8, hi=7)
        assert float(sw[n]) == es and codes[n].tolist() == ec
    # the per-column W4 linear is the per-channel path on the unpacked codes: integer sums
    # against numpy's int64 product, outputs against an fp64 fake-quant matmul
    x = rng.standard_normal((5, 320)).astype(np.float16)
    r = oracle.linear_w4(x, packed, sw, 0)
    assert (r["acc"] == r["x_q"].astype(np.int64) @ codes.astype(np.int64).T).all()
    fq = (r["s_x"][:, None].astype(np.float64) * r["x_q"]) @ (sw[:, None].astype(np.float64) * codes).T
    np.testing.assert_allclose(r["y"], fq, rtol=1e-12, atol=1e-12)


# ---- dequantization in the pages' fp32 arithmetic ---------------------------------------
# Plausible mistakes caught: a swapped multiply order or a fused (single-rounding) product
# in the per-channel epilogue, an int32 -> fp32 conversion that truncates, a per-group fold
# in another order or with separate multiply and add roundings, a missing token scale.

def test_dequant_pc_f32_exact_rational_model():
    rng = np.random.default_rng(21)
    acc = rng.integers(-2 ** 30, 2 ** 30, (9, 11)).astype(np.int32)  # most need rounding to fp32
    acc[0, :4] = [0, 1, -(2 ** 24) - 1, 2 ** 24 + 3]
    sx = (rng.random(9) * np.exp2(rng.integers(-20, 4, 9))).astype(np.float32)
    sw = (rng.random(11) * np.exp2(rng.integers(-12, 2, 11))).astype(np.float32)
    y32 = oracle.dequant_pc_f32(acc, sx, sw)
    assert y32.dtype == np.float32
    swapped = 0
    for m in range(9):
        for n in range(11):
            a = round_to_f32(Fraction(int(acc[m, n])))
            t = round_to_f32(a * Fraction(float(sx[m])))
            ref = round_to_f32(t * Fraction(float(sw[n])))
            assert Fraction(float(y32[m, n])) == ref, (m, n)
            swapped += round_to_f32(round_to_f32(a * Fraction(float(sw[n]))) * Fraction(float(sx[m]))) != ref
    assert swapped > 0  # the inputs tell the two multiply orders apart


def _fma_chain_exact(accs, scales, sx):
    t = Fraction(0)
    for a, s in zip(accs, scales):
        t = round_to_f32(round_to_f32(Fraction(int(a))) * Fraction(float(s)) + t)  # one rounding per fma
    return round_to_f32(t * Fraction(float(sx)))


def test_dequant_pg_f32_exact_rational_chain():
    rng = np.random.default_rng(22)
    G = 7
    accg = rng.integers(-2 ** 27, 2 ** 27, (4, 5, G)).astype(np.int32)
    sx = (rng.random(4) + 0.05).astype(np.float32)
    sw = (rng.random((5, G)) * 1e-3).astype(np.float32)
    sw[1, 3] = 0.0  # an all-zero group's scale
    y32 = oracle.dequant_pg_f32(accg, sx, sw)
    for m in range(4):
        for n in range(5):
            assert Fraction(float(y32[m, n])) == _fma_chain_exact(accg[m, n], sw[n], sx[m]), (m, n)


def test_dequant_pg_f32_folds_in_k_order_and_stays_in_the_fp32_bound():
    # groups [2^24, 1, -2^24] at unit scales: ascending, 2^24 + 1 rounds to 2^24 (ties to even)
    # and the last group cancels it (0); descending would give -2^24 + 1 + 2^24 = 1
    accg = np.array([[[2 ** 24, 1, -(2 ** 24)]]], np.int32)
    assert oracle.dequant_pg_f32(accg, np.ones(1, np.float32), np.ones((1, 3), np.float32))[0, 0] == 0.0
    # on the workload's distributions: within the fp32 evaluation bound (G fmas and one
    # multiply, each a relative 2^-24 of the running magnitude) of the fp64 value
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((16, 512)) * 2).astype(np.float16)
    W = (rng.standard_normal((24, 512)) * 0.02).astype(np.float32)
    for gs in (64, 128):
        wq, sw = oracle.quantize_weight(W, 8, gs)
        r = oracle.linear_pg(x, wq, sw, gs)
        G = 512 // gs
        assert (np.abs(r["y32"].astype(np.float64) - r["y"]) <= (G + 1) * 2.0 ** -24 * r["mag"] + 1e-300).all()
    # per channel: three roundings (conversion and two products) of the exact value
    wq, sw = oracle.quantize_weight(W, 8, 0)
    r = oracle.linear_pc(x, wq, sw)
    assert (np.abs(r["y32"].astype(np.float64) - r["y"]) <= 3 * 2.0 ** -24 * np.abs(r["y"])).all()


# ---- decode matrix-vector product without activation quantization (linear_mv) ----------
# Plausible mistakes caught: a quantized activation slipping in (one-hot and exact
# rational sums), a wrong group index for the weight scale (per-slice rational brute
# force at gs 64 / 128 with distinct scales per group), transposed operands (non-square
# shapes), a dropped scale (one-hot), the bf16 path reading the wrong half of the bits.

def _mv_exact(x16, wq, sw, gs):
    M, K = x16.shape
    N = wq.shape[0]
    y = np.zeros((M, N), dtype=object)
    for m in range(M):
        xs = [Fraction(float(v)) for v in x16[m].astype(np.float64)]
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                s = Fraction(float(sw[n] if gs == 0 else sw[n, k // gs]))
                acc += xs[k] * int(wq[n, k]) * s
            y[m, n] = acc
    return y


@pytest.mark.parametrize("gs", [0, 64, 128])
def test_mv_exact_rational_brute_force(gs):
    rng = np.random.default_rng(5 + gs)
    M, N, K = 3, 5, 256
    x = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    wq = rng.integers(-128, 128, (N, K)).astype(np.int8)
    sw = (rng.random(N if gs == 0 else (N, K // gs)) * 0.01 + 1e-3).astype(np.float32)
    r = oracle.linear_mv(x, wq, sw, gs)
    ex = _mv_exact(x, wq, sw, gs)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(r["y"][m, n])) - ex[m, n]) <= abs(ex[m, n]) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)
    # mag is the sum of |terms|: at least |y|, equal when all terms share a sign
    assert (r["mag"] >= np.abs(r["y"]) * (1 - 1e-15)).all()


def test_mv_one_hot_picks_dequantized_weight():
    rng = np.random.default_rng(6)
    N, K, gs = 16, 256, 64
    wq = rng.integers(-128, 128, (N, K)).astype(np.int8)
    sw = (rng.random((N, K // gs)) + 0.5).astype(np.float32)
    for j in (0, 63, 64, 200, 255):
        x = np.zeros((1, K), np.float16)
        x[0, j] = 2.0
        y = oracle.linear_mv(x, wq, sw, gs)["y"][0]
        assert (y == 2.0 * wq[:, j].astype(np.float64) * sw[:, j // gs].astype(np.float64)).all()


def test_mv_equals_w8a8_on_exactly_quantizable_activations():
    """x = c * 2^-e with integer |c| <= 127 and max |c| = 127 per row: per-token quantization
    gives s_x = 2^-e and x_q = c exactly, so the W8A8 result and the matrix-vector result are
    the same real number (and both are exact in fp64 here)."""
    rng = np.random.default_rng(7)
    M, N, K = 4, 24, 384
    c = rng.integers(-127, 128, (M, K))
    c[:, 5] = 127
    x = (c * 2.0 ** -6).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, sw = oracle.quantize_weight(W, 8, 0)
    pc = oracle.linear_pc(x, wq, sw)
    assert (pc["x_q"] == c).all() and (pc["s_x"] == np.float32(2.0 ** -6)).all()
    assert (oracle.linear_mv(x, wq, sw, 0)["y"] == pc["y"]).all()
    wq, sw = oracle.quantize_weight(W, 8, 128)
    pg = oracle.linear_pg(x, wq, sw, 128)
    assert np.allclose(oracle.linear_mv(x, wq, sw, 128)["y"], pg["y"], rtol=1e-13, atol=0)


def test_mv_group_scales_equal_channel_scale_and_bf16_bits():
    rng = np.random.default_rng(8)
    M, N, K = 2, 16, 256
    x = rng.standard_normal((M, K)).astype(np.float16)
    wq = rng.integers(-128, 128, (N, K)).astype(np.int8)
    s = (rng.random(N) + 0.1).astype(np.float32)
    y0 = oracle.linear_mv(x, wq, s, 0)["y"]
    assert (oracle.linear_mv(x, wq, np.repeat(s[:, None], K // 64, 1), 64)["y"] == y0).all()
    # values exact in both formats (8 significant bits, normal range): same result from bf16 bits
    xb = np.round(rng.standard_normal((M, K)) * 64).astype(np.float32) / 64
    bits = (xb.view(np.uint32) >> 16).astype(np.uint16)
    assert (bits.astype(np.uint32) << 16).view(np.float32).tolist() == xb.tolist()
    assert (oracle.linear_mv(bits, wq, s, 0, bf16=True)["y"] ==
            oracle.linear_mv(xb.astype(np.float16), wq, s, 0)["y"]).all()


# ---- clipped weight scales (quantize_weight_clipped) --------------------------------------
# Mistakes caught: an off-by-one order statistic or a missing interpolation (closed forms at
# integer and half positions), percentile applied to signed values instead of magnitudes
# (random signs), percentile in percent vs fraction (numpy comparison), a clamp that does
# not saturate the clipped tail, pct = 100 not reducing to min-max.

@pytest.mark.parametrize("bits,gs", [(8, 0), (8, 64), (8, 128), (4, 64), (4, 128)])
def test_clipped_at_100_is_min_max(bits, gs):
    rng = np.random.default_rng(21 + gs + bits)
    W = (rng.standard_normal((9, 256)) * 0.03).astype(np.float32)
    a = oracle.quantize_weight(W, bits, gs)
    b = oracle.quantize_weight_clipped(W, bits, gs, 100.0)
    assert (a[0] == b[0]).all() and (a[1].view(np.uint32) == b[1].view(np.uint32)).all()


@pytest.mark.parametrize("n,pct,pos", [(101, 99.0, 99.0), (101, 50.0, 50.0), (101, 1.0, 1.0), (11, 25.0, 2.5),
                                       (11, 95.0, 9.5), (5, 100.0, 4.0), (5, 10.0, 0.4)])
def test_clipped_closed_form(n, pct, pos):
    """Magnitudes j * 2^-7 (j = 0 .. n-1, shuffled, random signs): the percentile is pos * 2^-7
    (pos = pct (n - 1) / 100, exact here), s = that / 127, and every weight beyond it saturates."""
    rng = np.random.default_rng(n * 7 + int(pct * 10))
    mags = rng.permutation(np.arange(n)) * 2.0 ** -7
    W = (mags * rng.choice([-1.0, 1.0], n)).astype(np.float32)[None, :]
    wq, sw = oracle.quantize_weight_clipped(W, 8, 0, pct)
    a = np.float32(pos * 2.0 ** -7)
    assert sw[0] == a / np.float32(127.0)
    big = np.abs(W[0]) >= a
    assert (np.abs(wq[0][big].astype(int)) >= 127).all()  # saturated (+127, or -128 past -127.5)
    assert (np.abs(wq[0]).astype(int) <= 128).all()


def test_clipped_against_numpy_percentile():
    rng = np.random.default_rng(33)
    for n, gs in ((2560, 0), (128, 128), (64, 64)):
        W = (rng.standard_normal((40, 2560 if gs == 0 else 1024)) * 0.02).astype(np.float32)
        W[:, ::97] *= 30.0  # outliers
        for pct in (99.9, 99.0, 50.0, 0.5):
            _, sw = oracle.quantize_weight_clipped(W, 8, gs, pct)
            runs = np.abs(W).reshape(W.shape[0], -1, n)
            # the percentile travels as an fp32 argument: numpy gets the same value
            p32 = float(np.float32(pct))
            ref = (np.percentile(runs.astype(np.float64), p32, axis=2).astype(np.float32) / np.float32(127)).ravel()
            got = sw.ravel()
            ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
            assert ulps.max() <= 1 and (ulps == 0).mean() >= 0.95, (n, pct, ulps.max())


# ---- decode-step attention (sdpa_decode) --------------------------------------------------
# Mistakes caught: a missing scale or max subtraction (scipy softmax comparison, large scores),
# a wrong GQA head mapping (per-head comparison with repeated KV heads), rows past N read
# (garbage in the unused cache rows), a transposed q . k (non-square D / N).

def _sdpa_ref(q, k, v, N, scale):
    from scipy.special import softmax
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    o = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            kk = k[b, h // (Hq // Hkv), :N].astype(np.float64)
            vv = v[b, h // (Hq // Hkv), :N].astype(np.float64)
            p = softmax(scale * (kk @ q[b, h].astype(np.float64)))
            o[b, h] = p @ vv
    return o


def test_sdpa_against_scipy_softmax_gqa_and_cache_rows():
    rng = np.random.default_rng(41)
    B, Hq, Hkv, D, N, Ncap = 2, 8, 2, 64, 37, 50
    q = (rng.standard_normal((B, Hq, D)) * 2).astype(np.float16)
    k = rng.standard_normal((B, Hkv, Ncap, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, Ncap, D)).astype(np.float16)
    k[:, :, N:] = np.float16(300.0)  # rows past N must not count
    v[:, :, N:] = np.float16(-7.0)
    r = oracle.sdpa_decode(q, k, v, N=N)
    ref = _sdpa_ref(q, k, v, N, 1 / np.sqrt(D))
    assert np.allclose(r["o"], ref, rtol=1e-12, atol=1e-13)
    assert (r["vmag"] >= np.abs(r["o"]) - 1e-12).all()


def test_sdpa_closed_forms():
    rng = np.random.default_rng(42)
    D = 128
    v = rng.standard_normal((1, 1, 9, D)).astype(np.float16)
    k = rng.standard_normal((1, 1, 9, D)).astype(np.float16)
    q = rng.standard_normal((1, 4, D)).astype(np.float16)
    # one key: the output is that value row
    r = oracle.sdpa_decode(q, k, v, N=1)
    assert (r["o"][0] == v[0, 0, 0].astype(np.float64)).all()
    # q = 0 (all scores equal): the mean of the value rows
    r = oracle.sdpa_decode(np.zeros_like(q), k, v)
    assert np.allclose(r["o"][0], v[0, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)
    # one score far above the rest (about 80 after the scale): that value row
    kk = np.zeros_like(k)
    kk[0, 0, 5, 0] = np.float16(30.0)
    qq = np.zeros_like(q)
    qq[0, :, 0] = np.float16(30.0)
    r = oracle.sdpa_decode(qq, kk, v)
    assert np.allclose(r["o"][0], v[0, 0, 5].astype(np.float64), rtol=0, atol=1e-30)


def test_sdpa_gqa_equals_mha_with_repeated_heads_and_bf16():
    rng = np.random.default_rng(43)
    B, Hq, Hkv, D, N = 1, 8, 2, 64, 20
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float16)
    gqa = oracle.sdpa_decode(q, k, v)["o"]
    mha = oracle.sdpa_decode(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1))["o"]
    assert (gqa == mha).all()
    # bf16 bit patterns of values exact in both formats give the fp16 result
    r16 = [np.round(a.astype(np.float32) * 8) / 8 for a in (q, k, v)]
    bits = [(a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for a in r16]
    assert (oracle.sdpa_decode(*[a.astype(np.float16) for a in r16])["o"] ==
            oracle.sdpa_decode(*bits, bf16=True)["o"]).all()


# ---- RMSNorm with the per-token quantization folded in ------------------------------------

def _exact_rmsnorm_quantize(xrow, grow, eps):
    """Exact rationals: u = RN32(x g), the exact quantization of u, and s_x from a 40-digit
    square root of the exact mean of squares."""
    from decimal import Decimal, getcontext
    getcontext().prec = 40
    u = [float(round_to_f32(Fraction(float(a)) * Fraction(float(b)))) for a, b in zip(xrow, grow)]
    s, codes = exact_quantize(np.array(u, np.float32))
    ms = sum(Fraction(float(a)) ** 2 for a in xrow) / len(xrow) + Fraction(eps)
    d = Decimal(ms.numerator) / Decimal(ms.denominator)
    sx = float(Decimal(s) / d.sqrt()) if ms > 0 else float("inf")
    return s, codes, sx


def test_rmsnorm_quantize_hand_worked():
    """x = [3, 4], g = 1, eps = 0: mean square 12.5; s_u = RN32(4 / 127); 3 / s_u = 95.25 -> 95."""
    q, su, sx = oracle.rmsnorm_quantize(np.array([[3, 4]], np.float16), np.ones(2, np.float16), 0.0)
    assert q.tolist() == [[95, 127]]
    assert Fraction(float(su[0])) == round_to_f32(Fraction(4, 127))
    assert abs(sx[0] - float(su[0]) / 12.5 ** 0.5) <= 1e-16
    # an all-zero row: zero codes and zero scales, with or without eps
    for eps in (1e-6, 0.0):
        q, su, sx = oracle.rmsnorm_quantize(np.zeros((1, 8), np.float16), np.ones(8, np.float16), eps)
        assert (q == 0).all() and su[0] == 0 and sx[0] == 0


def test_rmsnorm_quantize_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    for r in range(12):
        K = int(rng.integers(2, 40))
        x = (rng.standard_normal(K) * (50 if r % 3 == 0 else 1)).astype(np.float16)
        g = (1 + 0.3 * rng.standard_normal(K)).astype(np.float16)
        if r % 4 == 1:
            x = (x * np.float16(1e-3)).astype(np.float16)
        eps = [0.0, 1e-6, 1e-2][r % 3]
        q, su, sx = oracle.rmsnorm_quantize(x[None, :], g, eps)
        es, ec, esx = _exact_rmsnorm_quantize(x, g, eps)
        assert q[0].tolist() == ec and float(su[0]) == es, r
        assert abs(sx[0] - esx) <= 1e-15 * esx, r


def test_rmsnorm_quantize_bf16_inputs_brute_force():
    rng = np.random.default_rng(12)
    K = 24
    xf = (rng.standard_normal((3, K)) * 4).astype(np.float32)
    xb = (xf.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 bits will do
    gb = ((1 + 0.2 * rng.standard_normal(K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, su, sx = oracle.rmsnorm_quantize(xb, gb, 1e-5, x_bf16=True, g_bf16=True)
    to32 = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    for m in range(3):
        es, ec, esx = _exact_rmsnorm_quantize(to32(xb[m]), to32(gb), 1e-5)
        assert q[m].tolist() == ec and float(su[m]) == es
        assert abs(sx[m] - esx) <= 1e-15 * esx


def test_rmsnorm_quantize_reduces_to_quantize_and_is_scale_invariant():
    from synth_inputs import linear_inputs
    x, _ = linear_inputs(6, 16, 512, seed=13)
    q0, s0 = oracle.quantize_per_token(x)
    q, su, sx = oracle.rmsnorm_quantize(x, np.ones(512, np.float16), 1e-6)
    assert (q == q0).all() and (su.view(np.uint32) == s0.view(np.uint32)).all()  # g = 1: u = x exactly
    # eps = 0: the norm of 2^j x is the norm of x (the power of two is exact in every step)
    g = (1 + 0.1 * np.random.default_rng(3).standard_normal(512)).astype(np.float16)
    qa, _, sa = oracle.rmsnorm_quantize(x, g, 0.0)
    qb, _, sb = oracle.rmsnorm_quantize((x.astype(np.float32) / 4).astype(np.float16), g, 0.0)
    assert (qa == qb).all() and np.allclose(sa, sb, rtol=1e-15, atol=0)


def test_rmsnorm_quantize_reconstructs_the_normalized_row():
    """s_x * q is the RMSNorm output (numpy fp64) within half a quantization step."""
    from synth_inputs import linear_inputs
    x, _ = linear_inputs(8, 16, 1024, seed=14)
    g = (1 + 0.1 * np.random.default_rng(4).standard_normal(1024)).astype(np.float16)
    eps = 1e-6
    q, su, sx = oracle.rmsnorm_quantize(x, g, eps)
    xf, gf = x.astype(np.float64), g.astype(np.float64)
    n = xf / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + eps) * gf
    err = np.abs(sx[:, None] * q - n)
    # half a step, plus the fp32 roundings of x g and of the quotient (each <= 127 * 2^-24 steps)
    assert (err <= sx[:, None] * (0.5 + 2 * 127 * 2.0 ** -24)).all()
    assert (np.abs(q).max(axis=1) == 127).all()


def test_rmsnorm_quantize_codes_equal_quantize_of_the_fp64_norm():
    """Pins the fold itself against the unfolded definition: numpy's fp64 RMSNorm
    n = x g / sqrt(mean x^2 + eps), quantized per token in fp64 (s = max|n| / 127,
    q = rint(n / s)), gives the oracle's codes on every row where no quotient n / s lies
    within 2^-13 of a half-integer. The oracle's quotient u / s_u (u = x g is exact in fp32
    for fp16 or bf16 factors: at most 22 significant bits) carries two fp32 roundings of
    relative size 2^-24 each, so it moves a quotient of magnitude <= 127 by less than
    2^-16; outside the band both round to the same integer."""
    rng = np.random.default_rng(41)
    M, K = 300, 256
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, 3, replace=False)] *= 50  # outlier channels
    x = (x * np.exp2(rng.integers(-6, 6, (M, 1)))).astype(np.float16)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    for eps in (0.0, 1e-6, 0.5):
        xq, su, sx = oracle.rmsnorm_quantize(x, g, eps)
        xf = x.astype(np.float64)
        n = xf * g.astype(np.float64) / np.sqrt((xf * xf).mean(axis=1, keepdims=True) + eps)
        s = np.abs(n).max(axis=1) / 127.0
        t = n / s[:, None]
        near = np.abs(np.abs(t - np.floor(t)) - 0.5) < 2.0 ** -13
        ok = ~near.any(axis=1)
        assert ok.sum() >= 0.8 * M
        assert (xq[ok] == np.rint(t[ok])).all()
        np.testing.assert_allclose(sx, s, rtol=2.0 ** -20)


# ---- SwiGLU with the per-token quantization folded in (swiglu_quantize) -----------------
# Plausible mistakes caught: a wrong exp (range reduction, a dropped Taylor term, a wrong
# clamp) -> fp64 exp bound and the fixed points; silu with a wrong sign or without the gate
# factor -> fp64 silu * up bound; quantization of something other than h -> numpy's fp32
# quantization of the returned h and the fp64 quantization away from near-ties; gate and up
# swapped -> the asymmetric fp64 check.

def test_exp_steps_against_fp64_exp():
    x = np.concatenate([np.linspace(-87.0, 88.0, 400001), [0.0, -0.0, 1e-30, -1e-30, 0.34657359, -0.34657359]])
    x = x.astype(np.float32)
    y = oracle.exp_steps(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert (np.abs(y - ref) <= 2.0 ** -22 * ref).all()
    assert oracle.exp_steps(np.zeros(1, np.float32))[0] == 1.0
    # clamped arguments: finite, and equal to the value at the clamp
    big = oracle.exp_steps(np.array([88.0, 100.0, 1e30, -87.0, -200.0, -1e30], np.float32))
    assert big[0] == big[1] == big[2] and np.isfinite(big[0]) and big[3] == big[4] == big[5] > 0


def _silu64(g):
    return g / (1.0 + np.exp(-g))


def _swiglu_inputs(M, I, seed, bf16=False):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((M, I)) * 2.0
    u = rng.standard_normal((M, I))
    g[:, rng.choice(I, 3, replace=False)] *= 20  # large gate values (silu ~ g and ~ 0)
    if bf16:
        import torch
        gb = torch.from_numpy(g.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        ub = torch.from_numpy(u.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return gb, ub, (gb.astype(np.uint32) << 16).view(np.float32), (ub.astype(np.uint32) << 16).view(np.float32)
    g16, u16 = g.astype(np.float16), u.astype(np.float16)
    return g16, u16, g16.astype(np.float32), u16.astype(np.float32)


@pytest.mark.parametrize("bf16", [False, True])
def test_swiglu_quantize_h_codes_and_scale(bf16):
    M, I = 120, 384
    ga, ua, gf, uf = _swiglu_inputs(M, I, seed=51, bf16=bf16)
    xq, sx, h = oracle.swiglu_quantize(ga, ua, bf16=bf16)
    # h against fp64 silu(g) * u: exp within 2^-22, then one add, one division, one product;
    # below g = -87 the exp argument is clamped and h is only bounded (|h| <= |g u| 2^-125,
    # since 1 + e^87 > 2^125): those values quantize to 0 next to any normal entry of the row
    h64 = _silu64(gf.astype(np.float64)) * uf.astype(np.float64)
    hd = h.astype(np.float64)
    live = gf >= -87.0
    assert (np.abs(hd - h64) <= 2.0 ** -20 * np.abs(h64) + 1e-37)[live].all()
    assert (np.abs(hd) <= np.abs(gf.astype(np.float64) * uf) * 2.0 ** -125)[~live].all()
    # the quantization of the returned h, recomputed with numpy's IEEE fp32 division
    s_np = (np.abs(h).max(axis=1) / np.float32(127.0)).astype(np.float32)
    assert (sx.view(np.uint32) == s_np.view(np.uint32)).all()
    q_np = np.clip(np.rint(h / s_np[:, None]), -128, 127).astype(np.int8)
    assert (xq == q_np).all()
    # and against the fp64 definition, away from near-ties: the fp32 evaluation moves a
    # quotient of magnitude <= 127 by less than 127 * 2^-21 < 2^-14
    s64 = np.abs(h64).max(axis=1) / 127.0
    t = h64 / s64[:, None]
    ok = ~(np.abs(np.abs(t - np.floor(t)) - 0.5) < 2.0 ** -13).any(axis=1)
    assert ok.sum() >= 0.8 * M
    assert (xq[ok] == np.rint(t[ok])).all()


def test_swiglu_quantize_closed_forms_and_strided_halves():
    M, I = 6, 64
    ga, ua, _, _ = _swiglu_inputs(M, I, seed=52)
    ga[0] = 0          # silu(0) = 0: a zero row
    ua[1] = 0          # up = 0: a zero row
    ga[2] = 60.0       # silu(g) = g / (1 + e^-60) = g in fp32: h = g * u exactly
    ua[2] = np.float16(-1.5)
    xq, sx, h = oracle.swiglu_quantize(ga, ua)
    assert sx[0] == 0 and sx[1] == 0 and (xq[:2] == 0).all()
    assert (h[2] == np.float32(60.0) * np.float32(-1.5)).all() and (xq[2] == -127).all()
    # gate and up as the two halves of one [M, 2I] array (the gate/up projection's output)
    both = np.concatenate([ga, ua], axis=1)
    xq2, sx2, h2 = oracle.swiglu_quantize(both[:, :I], both[:, I:])
    assert (xq2 == xq).all() and (sx2 == sx).all() and (h2 == h).all()
    # swapping gate and up changes the result (silu applies to the gate only)
    xq3, _, _ = oracle.swiglu_quantize(ua, ga)
    assert (xq3[3:] != xq[3:]).any()
