"""The activation-quantization kernel replaces the per-element IEEE division x / s with a
per-row reciprocal r = 1/s and Markstein's corrected quotient
    q0 = x*r;  e = fma(-q0, s, x);  q = fma(e, r, q0).
These host-side tests check, exhaustively, that this changes no code:
  * fp16: for every positive finite fp16 maximum a (s = a/127) and every fp16 x with
    |x| <= a, q equals x / s exactly (about 1.0e9 pairs);
  * bf16: for every bf16 maximum with s >= 2^-100 (smaller scales keep the division in the
    kernel) and every bf16 |x| <= a, rint(q) equals rint(x / s).
  * products of two halves (the RMSNorm producer quantizes u = x * g): on 2.5e8 random
    (u, s) pairs (of 4e8 drawn), s = a / 127 for a product a of two halves and |u| <= a, a quarter of them
    placed at and next to every half-integer quotient, q equals u / s (up to the sign of a
    zero quotient). Markstein's theorem says so for any fp32 u when r is the correctly
    rounded reciprocal and nothing underflows; the sample checks the implementation.
The check is plain C (gcc, -ffp-contract=off, libm fmaf); it shares nothing with the
GPU library or the oracle.
"""
import os
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <stdlib.h>
#include <omp.h>
static float h2f(uint32_t h) {
    uint32_t e = (h >> 10) & 31, m = h & 1023; float v;
    if (e == 0) v = ldexpf((float)m, -24); else v = ldexpf((float)(1024 + m), (int)e - 25);
    return (h >> 15) ? -v : v;
}
static float b2f(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static float mq(float x, float s, float r) { float q0 = x * r; float e = fmaf(-q0, s, x); return fmaf(e, r, q0); }
static uint32_t rh(uint64_t *st) {  /* a random finite half, magnitude bits only */
    for (;;) {
        *st ^= *st << 13; *st ^= *st >> 7; *st ^= *st << 17;
        uint32_t h = (uint32_t)(*st & 0x7fff);
        if (((h >> 10) & 31) != 31) return h;
    }
}
static int products(long long n) {
    long long done = 0, bad = 0;
#pragma omp parallel reduction(+:done, bad)
    {
        uint64_t st = 0x9E3779B97F4A7C15ull ^ (uint64_t)(omp_get_thread_num() + 1) * 0xBF58476D1CE4E5B9ull;
#pragma omp for schedule(static)
        for (long long i = 0; i < n; ++i) {
            float a = h2f(rh(&st)) * h2f(rh(&st));
            float s = a / 127.0f;
            if (!(s >= 0x1p-100f)) continue;
            float r = 1.0f / s, u;
            if (i & 3) {
                u = h2f(rh(&st)) * h2f(rh(&st));
                if (fabsf(u) > a) continue;
            } else {  /* at and next to the half-integer quotient k + 1/2 */
                uint32_t b;
                u = ((float)(rh(&st) % 127) + 0.5f) * s;
                memcpy(&b, &u, 4); b += (int)(rh(&st) % 5) - 2; memcpy(&u, &b, 4);
                if (fabsf(u) > a) continue;
            }
            if (rh(&st) & 1) u = -u;
            float t = u / s, q = mq(u, s, r);
            done++;
            if (u != 0.0f && q != t) bad++;
        }
    }
    printf("%lld %lld\n", done, bad);
    return 0;
}
int main(int argc, char **argv) {
    if (argc > 2) return products(atoll(argv[2]));
    int bf = argc > 1;
    long long pairs = 0, bad = 0;
    const int top = bf ? 0x7F80 : 0x7C00;
#pragma omp parallel for schedule(dynamic, 64) reduction(+:pairs, bad)
    for (int ab = 1; ab < top; ++ab) {
        float a = bf ? b2f(ab) : h2f(ab);
        float s = a / 127.0f;
        if (bf && !(s >= 0x1p-100f)) continue;
        float r = 1.0f / s;
        for (int xb = 0; xb <= ab; ++xb)
            for (int sg = 0; sg < 2; ++sg) {
                uint32_t bits = xb | (sg << 15);
                float x = bf ? b2f(bits) : h2f(bits);
                float t = x / s, q = mq(x, s, r);
                pairs++;
                if (bf ? (rintf(q) != rintf(t)) : (q != t)) bad++;
            }
    }
    printf("%lld %lld\n", pairs, bad);
    return 0;
}
"""


@pytest.fixture(scope="module")
def checker():
    d = tempfile.mkdtemp()
    src = os.path.join(d, "q.c")
    exe = os.path.join(d, "q")
    open(src, "w").write(SRC)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, src, "-lm"])
    return exe


def test_fp16_corrected_quotient_equals_division(checker):
    pairs, bad = map(int, subprocess.check_output([checker]).split())
    assert pairs > 1_000_000_000 and bad == 0


def test_bf16_corrected_quotient_gives_same_codes(checker):
    pairs, bad = map(int, subprocess.check_output([checker, "bf16"]).split())
    assert pairs > 1_000_000_000 and bad == 0


def test_products_of_halves_corrected_quotient_equals_division(checker):
    done, bad = map(int, subprocess.check_output([checker, "products", "400000000"]).split())
    assert done > 200_000_000 and bad == 0
