/* Host model of the library's E4M3-scaled FP4 encoding arithmetic, checked
 * against the encoding rule it must reproduce (the scale byte: the smallest
 * E4M3 code with 6 * value >= the group maximum; the code: the nearest E2M1
 * value of x / s, ties to the even code, saturating, zero magnitude +0, NaN 0;
 * jokeuncle.pages.dev, "两张架构图里藏着 890 字节", section 三).
 *
 *   scale_closed: amax * RN(1/6) rounded up to the E4M3 grid through its
 *                 bit pattern, then one code up if 6 * value < amax;
 *   code_quot:    q = RN(x / sig) as q0 = x * RN(1/sig) plus one residual
 *                 step, then the rule at the power of two 2^E (what the
 *                 hardware convert applies), s = 2^E * sig.
 *
 * Checked: every fp32 within +-N ulps of 6 * value(b) for each scale code,
 * and of M * s for every midpoint and grid value M at every scale code, both
 * signs, plus seeded random values and the non-finite and zero inputs.
 * Usage: e4m3_encoder_check N_ULPS N_RANDOM SEED; prints the counts, exit 1
 * on any mismatch.  -DWITHOUT_RESIDUAL_STEP builds the encoder without its
 * residual step (q = q0), which must fail.  Build with -ffp-contract=off (the products and fmaf are
 * written out as the kernel rounds them).  */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E4M3FN byte -> value: e >= 1: 2^(e-7) (1 + m/8); e = 0: m 2^-9; 0x7F NaN */
static float e4m3(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if ((b & 0x7Fu) == 0x7Fu) return NAN;
  const float v = e ? ldexpf(1.0f + m / 8.0f, (int)e - 7) : ldexpf((float)m, -9);
  return (b & 0x80u) ? -v : v;
}

static uint32_t scale_search(float amax) {
  if (!(amax > 0.0f)) return 0u;
  for (uint32_t b = 0; b < 0x7Eu; ++b)
    if (6.0f * e4m3(b) >= amax) return b;
  return 0x7Eu;
}

static uint32_t scale_closed(float amax) {
  if (!(amax > 0.0f)) return 0u;
  const float t = amax * (1.0f / 6.0f);
  int b = t < 0x1p-6f ? (int)ceilf(t * 512.0f) : (int)((f2u(t) - (120u << 23) + 0xFFFFFu) >> 20);
  b = b < 0x7E ? b : 0x7E;
  if (6.0f * e4m3((uint32_t)b) < amax) b = b + 1 < 0x7E ? b + 1 : 0x7E;
  return (uint32_t)b;
}

/* the rule, by exact comparison with the midpoints (products exact here) */
static uint32_t code_rule(float x, float s) {
  const float a = fabsf(x);
  if (!(a > 0.0f)) return 0u;
  uint32_t c = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) +
               (a > 2.5f * s) + (a >= 3.5f * s) + (a > 5.0f * s);
  return (c && (f2u(x) >> 31)) ? c | 8u : c;
}

static uint32_t code_quot(float x, float s) {
  const uint32_t su = f2u(s);
  const float sig = u2f((su & 0x007FFFFFu) | 0x3F800000u);
  const float r = 1.0f / sig;
  const float pow2 = s == 0.0f ? 1.0f : u2f(su & 0x7F800000u);
  float xc = x == x ? x : 0.0f;
  xc = fminf(fmaxf(xc, -0x1p100f), 0x1p100f);
  const float q0 = xc * r;
#ifdef WITHOUT_RESIDUAL_STEP  /* a planted mistake the check must catch */
  const float q = q0;
#else
  const float q = fmaf(fmaf(-q0, sig, xc), r, q0);
#endif
  return code_rule(q, pow2);
}

static uint64_t rng_state;
static uint32_t rnd(void) {  /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

int main(int argc, char** argv) {
  const int64_t N = argc > 1 ? atoll(argv[1]) : 4096;
  const int64_t R = argc > 2 ? atoll(argv[2]) : 1000000;
  rng_state = argc > 3 ? strtoull(argv[3], 0, 10) : 1;
  uint64_t ns = 0, nc = 0, bad = 0;
  const float M[] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  for (uint32_t b = 0; b <= 0x7Eu; ++b) {
    const float s = e4m3(b);
    const uint32_t u6 = f2u(6.0f * s);
    for (int64_t d = -N; d <= N; ++d) {
      const float a = u2f((uint32_t)((int64_t)u6 + d));
      ++ns;
      if (scale_search(a) != scale_closed(a)) {
        if (bad < 10) printf("scale mismatch at %a: %u vs %u\n", a, scale_search(a), scale_closed(a));
        ++bad;
      }
    }
    if (b == 0) continue;  /* scale code 0 only for a group of zeros */
    for (int i = 0; i < 14; ++i) {
      const uint32_t up = f2u(M[i] * s);
      for (int64_t d = -N; d <= N; ++d)
        for (int sg = 0; sg < 2; ++sg) {
          const float x = u2f((uint32_t)((int64_t)up + d) | (sg ? 0x80000000u : 0u));
          ++nc;
          if (code_rule(x, s) != code_quot(x, s)) {
            if (bad < 10) printf("code mismatch b=%u x=%a: %u vs %u\n", b, x, code_rule(x, s), code_quot(x, s));
            ++bad;
          }
        }
    }
  }
  const float sp[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 0x1p-149f, -0x1p-149f, 0x1p-126f, 3.4e38f, -3.4e38f};
  for (int64_t i = 0; i < R; ++i) {
    const uint32_t b = 1u + rnd() % 0x7Eu;
    const float s = e4m3(b);
    float x;
    if (i < 10 * 0x7E) x = sp[i % 10];
    else x = u2f((rnd() & 0x807FFFFFu) | ((uint32_t)(f2u(s) >> 23) - 8u + rnd() % 14u) << 23);
    ++nc;
    if (code_rule(x, s) != code_quot(x, s)) {
      if (bad < 10) printf("code mismatch b=%u x=%a: %u vs %u\n", b, x, code_rule(x, s), code_quot(x, s));
      ++bad;
    }
    const float a = u2f(rnd() & 0x7FFFFFFFu);
    if (a == a) {
      ++ns;
      if (scale_search(a) != scale_closed(a)) {
        if (bad < 10) printf("scale mismatch at %a\n", a);
        ++bad;
      }
    }
  }
  printf("scales %llu codes %llu mismatches %llu\n", (unsigned long long)ns, (unsigned long long)nc,
         (unsigned long long)bad);
  return bad ? 1 : 0;
}
