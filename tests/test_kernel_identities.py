"""CPU checks of the floating-point identities the gfx950 kernels rely on to
compute the documented semantics with fewer instructions.  Each identity is
exact IEEE-754 binary32 arithmetic, so a C program with correctly rounded
fmaf (no contraction) checks it exhaustively or on large random samples:

1. s = m / r for r in {7, 127, 448}: with c = RN(1/r), q = m*c, e = fma(-q, r, m),
   fma(e, c, q) == RN(m / r) for every float mantissa (three exponent ranges),
   and for r in {7, 127} also for every m below 2^-117: the subnormals and the
   lowest binades, where q or the result is subnormal (above them every
   quantity is normal and the check of one binade carries over by exact
   power-of-two scaling), so these widths need no separate path for tiny
   groups.
2. Offset-binary dequantization: fma(c + 2^(b-1), sa, -2^(b-1)*sa) == RN(c*sa)
   for every code c and random (incl. subnormal) sa below 2^120, the library's
   supported state magnitude (beyond it 2^(b-1)*sa itself may overflow).
3. Stochastic rounding by integer addition: with y = fma(x, inv*2^f, 1.5*2^23)
   (or fma(x*2^f, inv, 1.5*2^23) for huge inv), byte 2 of bits(y) + R (4-bit,
   f = 16; low nibble) or of 2 bits(y) + R + 2^23 (8-bit, f = 15) is the code
   floor((rint(x*inv*2^f) * 2^(16-f) + R) / 2^16), computed here in double.
4. Round-to-nearest via the 1.5*2^23 constant: the low bits of
   fma(x, inv, 1.5*2^23) hold rint(x*inv) of the exact product when |x*inv| <= r.
5. INT4 widening through FP8: a byte b in [0, 15] read as OCP E4M3 (decoded
   here from the format's definition) is b * 2^-9, and
   fma(b * 2^-9, s * 2^9, -8 s) == RN((b - 8) * s) for s below 2^118.
"""

import os
import subprocess
import tempfile

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float f_of(uint32_t u){float f; memcpy(&f,&u,4); return f;}
static uint32_t u_of(float f){uint32_t u; memcpy(&u,&f,4); return u;}
static uint64_t s = 88172645463325252ull;
static uint32_t rnd(void){ s ^= s << 13; s ^= s >> 7; s ^= s << 17; return (uint32_t)(s >> 11); }
/* largest float v with v*m <= r */
static float inv_rz(float m, float r){ float v = (float)((double)r / (double)m);
  while ((double)v * (double)m > (double)r) v = nextafterf(v, 0.0f); return v; }
int main(void){
  long bad = 0;
  /* 1 */
  const float rs[3] = {7.0f, 127.0f, 448.0f};  /* INT4, INT8, FP8 (E4M3) vector scales */
  for (int t = 0; t < 3; ++t) {
    const float r = rs[t], c = 1.0f / r;
    for (uint32_t mant = 0; mant < (1u << 23); ++mant)
      for (int ex = 0; ex < 3; ++ex) {
        const uint32_t e8 = ex == 0 ? 127 : (ex == 1 ? 28 : 200);
        const float m = f_of((e8 << 23) | mant);
        const float q = m * c;
        const float got = fmaf(fmaf(-q, r, m), c, q);
        if (got != m / r) { if (bad < 5) printf("div r=%g m=%a\n", r, m); ++bad; }
      }
  }
  for (int t = 0; t < 2; ++t) {
    const float r = rs[t], c = 1.0f / r;
    for (uint32_t u = 1; u < (10u << 23); ++u) {
      const float m = f_of(u);
      const float q = m * c;
      const float got = fmaf(fmaf(-q, r, m), c, q);
      if (got != m / r) { if (bad < 5) printf("div-tiny r=%g m=%a\n", r, m); ++bad; }
    }
  }
  printf("identity1 %ld\n", bad);
  /* 2 */
  long bad2 = 0;
  for (int bits = 4; bits <= 8; bits += 4) {
    const int r = (1 << (bits - 1)) - 1; const float bias = (float)(1 << (bits - 1));
    for (int it = 0; it < 200000; ++it) {
      uint32_t u = rnd() & 0x7fffffffu;
      if ((u >> 23) >= 247) u &= 0x3fffffffu;  /* supported range: |sa| < 2^120 */
      const float sa = f_of(u);
      for (int c = -r; c <= r; ++c) {
        const float got = fmaf((float)(c + (1 << (bits - 1))), sa, -bias * sa);
        const float want = (float)c * sa;
        if (u_of(got) != u_of(want) && !(got == 0.0f && want == 0.0f)) { if (bad2 < 5) printf("deq c=%d sa=%a\n", c, sa); ++bad2; }
      }
    }
  }
  printf("identity2 %ld\n", bad2);
  /* 3 and 4 */
  long bad3 = 0, bad4 = 0;
  for (int bits = 4; bits <= 8; bits += 4) {
    const float r = (float)((1 << (bits - 1)) - 1);
    for (int it = 0; it < 3000000; ++it) {
      const float m = f_of(((uint32_t)(97 + rnd() % 60) << 23) | (rnd() & 0x7fffffu));
      const float inv = inv_rz(m, r);
      const float x = (rnd() & 1 ? -1.0f : 1.0f) * m * (float)(rnd() & 0xffffff) / 16777216.0f;
      const uint32_t R = rnd() & 0xffffu;
      const int f = bits == 4 ? 16 : 15;
      const float sf = (float)(1 << f);
      const double nr = nearbyint(ldexp((double)x * (double)inv, f));
      const int want = (int)floor((ldexp(nr, 16 - f) + (double)R) / 65536.0);
      const uint32_t yb = u_of(fmaf(x, inv * sf, 12582912.0f));
      const uint32_t yb2 = u_of(fmaf(x * sf, inv, 12582912.0f));
      const uint32_t t = bits == 4 ? yb + R : yb + (yb + R) + 0x00800000u;
      const int code = bits == 4 ? (int)(((t >> 16) & 0xFu) ^ 8u) - 8 : (int)(int8_t)(t >> 16);
      if (code != want || yb != yb2 || abs(want) > (int)r) {
        if (bad3 < 5) printf("sr x=%a inv=%a R=%u\n", x, inv, R); ++bad3; }
      const int n = (int)(u_of(fmaf(x, inv, 12582912.0f)) - 0x4B400000u);
      const int w = (int)rint((double)x * (double)inv);
      if (n != w || abs(w) > (int)r) { if (bad4 < 5) printf("rtn x=%a inv=%a\n", x, inv); ++bad4; }
    }
  }
  /* 3 for tiny groups (inv above 2^100): the scaled-x form */
  for (int bits = 4; bits <= 8; bits += 4) {
    const float r = (float)((1 << (bits - 1)) - 1);
    const int f = bits == 4 ? 16 : 15;
    const float sf = (float)(1 << f);
    for (int it = 0; it < 1000000; ++it) {
      const uint32_t e8 = rnd() % 24;  /* m from subnormal up to 2^-104 */
      const float m = f_of((e8 << 23) | (rnd() & 0x7fffffu));
      if (m == 0.0f) continue;
      const float inv = inv_rz(m, r);
      const uint32_t back = rnd() % 4096u;  /* |x| <= m, x stays a float below m */
      const float x = (rnd() & 1 ? -1.0f : 1.0f) * f_of(u_of(m) - (back < u_of(m) ? back : 0u));
      const uint32_t R = rnd() & 0xffffu;
      const double nr = nearbyint(ldexp((double)x * (double)inv, f));
      const int want = (int)floor((ldexp(nr, 16 - f) + (double)R) / 65536.0);
      const uint32_t yb = u_of(fmaf(x * sf, inv, 12582912.0f));
      const uint32_t t = bits == 4 ? yb + R : yb + (yb + R) + 0x00800000u;
      const int code = bits == 4 ? (int)(((t >> 16) & 0xFu) ^ 8u) - 8 : (int)(int8_t)(t >> 16);
      if (code != want || abs(want) > (int)r) {
        if (bad3 < 10) printf("sr-tiny x=%a inv=%a R=%u\n", x, inv, R); ++bad3; }
    }
  }
  /* 5 */
  long bad5 = 0;
  for (int b = 0; b < 16; ++b) {
    const int e = b >> 3, mm = b & 7;
    const double dec = e == 0 ? ldexp(mm, -9) : ldexp(1.0 + mm / 8.0, e - 7);
    if (dec != ldexp(b, -9)) { printf("e4m3 b=%d\n", b); ++bad5; }
  }
  for (int it = 0; it < 200000; ++it) {
    uint32_t u = rnd() & 0x7fffffffu;
    if ((u >> 23) >= 245) u &= 0x3fffffffu;  /* s < 2^118 */
    const float sa = f_of(u);
    for (int b = 0; b < 16; ++b) {
      const float got = fmaf(ldexpf((float)b, -9), sa * 512.0f, -8.0f * sa);
      const float want = (float)(b - 8) * sa;
      if (u_of(got) != u_of(want) && !(got == 0.0f && want == 0.0f)) {
        if (bad5 < 5) printf("fp8deq b=%d sa=%a\n", b, sa); ++bad5; }
    }
  }
  printf("identity3 %ld\nidentity4 %ld\nidentity5 %ld\n", bad3, bad4, bad5);
  return (bad || bad2 || bad3 || bad4 || bad5) ? 1 : 0;
}
"""


def test_kernel_float_identities():
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "ident.c")
        exe = os.path.join(d, "ident")
        open(c, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe, c, "-lm"],
                       check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        lines = dict(l.split() for l in r.stdout.splitlines() if l.startswith("identity"))
        assert r.returncode == 0, r.stdout
        assert lines == {"identity1": "0", "identity2": "0", "identity3": "0", "identity4": "0",
                         "identity5": "0"}


def test_one_stochastic_rounding_form_for_both_widths():
    """Lanes whose width is chosen at run time compute the stochastic-rounding
    word as (bits(y) << sh) + (R16 | add), sh = 1 and add = 2^23 for 8 bits,
    0 and 0 for 4 bits, with R16 | add formed by one byte permute.  That equals
    the one-width forms 2 bits(y) + R16 + 2^23 and bits(y) + R16 modulo 2^32
    (R16 < 2^16 leaves bit 23 free), checked here over every R16 for sampled
    y of the constant's binade, byte 2 and its low nibble."""
    import numpy as np
    rng = np.random.default_rng(11)
    magic = 0x4B400000
    ys = np.concatenate([magic + rng.integers(-(1 << 22), 1 << 22, 2000),
                         magic + np.array([-(1 << 22), (1 << 22) - 1, 0, 1, -1])]).astype(np.int64)
    r16 = np.arange(1 << 16, dtype=np.int64)
    m32 = (1 << 32) - 1
    for y in ys:
        one8 = ((2 * y + r16 + (1 << 23)) & m32) >> 16 & 0xFF
        rt8 = (((y << 1) + (r16 | (1 << 23))) & m32) >> 16 & 0xFF
        assert np.array_equal(one8, rt8), hex(y)
        one4 = ((y + r16) & m32) >> 16 & 0xF
        rt4 = (((y << 0) + (r16 | 0)) & m32) >> 16 & 0xF
        assert np.array_equal(one4, rt4), hex(y)


BDR_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f_of(uint32_t u){float f; memcpy(&f,&u,4); return f;}
static uint32_t u_of(float f){uint32_t u; memcpy(&u,&f,4); return u;}
static uint64_t s = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void){ s ^= s << 13; s ^= s >> 7; s ^= s << 17; return (uint32_t)(s >> 11); }
static float med3f(float a, float b, float c){ return fmaxf(fminf(a, b), fminf(fmaxf(a, b), c)); }
static int med3i(int a, int b, int c){ int lo = a < b ? a : b, hi = a < b ? b : a;
  return c < lo ? lo : (c > hi ? hi : c); }
static float inv_rz(float m, float r){ float v = (float)((double)r / (double)m);
  while ((double)v * (double)m > (double)r) v = nextafterf(v, 0.0f); return v; }
int main(void){
  long bad1 = 0, bad2 = 0, steps = 0;
  const float rs[2] = {7.0f, 127.0f};
  /* 1: RN(r * RN(m / r)) is m or a float neighbour of m, every mantissa of [1, 2) */
  for (int t = 0; t < 2; ++t)
    for (uint32_t mant = 0; mant < (1u << 23); ++mant) {
      const float m = f_of((127u << 23) | mant), r = rs[t];
      const float tr = r * (m / r);
      if (tr != m && tr != nextafterf(m, 0.0f) && tr != nextafterf(m, 1e30f)) {
        if (bad1 < 5) printf("neighbour r=%g m=%a\n", r, m); ++bad1; }
    }
  /* 2: the definition (round to nearest, one step toward the update where the
     stored value p lies strictly between n*s_new and x, clamp to [-r, r])
     against the unclamped branch-free form (y - med3_i32(bits(med3(p - x,
     n*s_new - p, 0)), -1, 1)) for groups with absmax m >= 2^-100, x drawn
     near the group's edges and p near the grid values around x */
  for (int t = 0; t < 2; ++t)
    for (int it = 0; it < 4000000; ++it) {
      const float r = rs[t];
      const float m = f_of(((uint32_t)(27 + rnd() % 200) << 23) | (rnd() & 0x7fffffu));
      const float s_new = m / r, inv = inv_rz(m, r);
      const uint32_t k = rnd() % 4;
      float x = k == 0 ? m : (k == 1 ? -m : m * ((float)(rnd() & 0xffffff) / 8388608.0f - 1.0f));
      if (rnd() & 1) x = nextafterf(x, 0.0f);
      const float y = fmaf(x, inv, 12582912.0f);
      const int n = (int)(u_of(y) - 0x4B400000u);
      const float grid = (float)n * s_new;
      float p;
      const uint32_t c = rnd() % 6;
      if (c == 0) p = nextafterf(grid, 1e30f); else if (c == 1) p = nextafterf(grid, -1e30f);
      else if (c == 2) p = nextafterf(x, 1e30f); else if (c == 3) p = nextafterf(x, -1e30f);
      else p = grid + (x - grid) * ((float)(rnd() & 0xffff) / 65536.0f) * (c == 4 ? 1.0f : 2.0f);
      int want = n;
      if (x > p && grid < p) want += 1;
      if (x < p && grid > p) want -= 1;
      want = want < -(int)r ? -(int)r : (want > (int)r ? (int)r : want);
      const float mm = med3f(p - x, (y - 12582912.0f) * s_new - p, 0.0f);
      int sm; memcpy(&sm, &mm, 4);
      const int got = (int)u_of(y) - med3i(sm, -1, 1) - 0x4B400000;
      if (got != n) ++steps;
      if (got != want) { if (bad2 < 5) printf("bdr r=%g m=%a x=%a p=%a\n", r, m, x, p); ++bad2; }
    }
  printf("bdr1 %ld\nbdr2 %ld\nsteps %ld\n", bad1, bad2, steps);
  return (bad1 || bad2) ? 1 : 0;
}
"""


def test_bdr_unclamped_step_for_normal_groups():
    """The persistent step's INT4 BDR leaves out the clamp to [-r, r] unless
    some group of the wave has an absmax below 2^-100: RN(r * RN(m / r)) is m
    or a float neighbour of m for every mantissa (so, by exact power-of-two
    scaling, for every m >= 2^-100, where m / r stays normal), which leaves no
    stored value strictly between the value of code +-r and an |x| <= m; and
    on sampled groups the branch-free unclamped form equals the definition
    (round to nearest, one step toward the update, clamp)."""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "bdr.c")
        exe = os.path.join(d, "bdr")
        open(c, "w").write(BDR_SRC)
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe, c, "-lm"],
                       check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        lines = dict(l.split() for l in r.stdout.splitlines())
        assert r.returncode == 0, r.stdout
        assert lines["bdr1"] == "0" and lines["bdr2"] == "0"
        assert int(lines["steps"]) > 100000  # the samples do exercise the directional step
