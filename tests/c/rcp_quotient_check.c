/* The block encoder forms |x| / b as q0 = |x|*y, q = fma(fma(-q0, b, |x|), y, q0)
 * with y = RN(1/b) (b = E4M3 block scale times the per-tensor scale).  This
 * program compares the E2M1 code of q with the code of the correctly rounded
 * quotient RN(|x|/b) for every positive finite bfloat16 |x|, every positive
 * E4M3 scale and a set of per-tensor scales, plus random float32 |x|.
 * Prints "cases <n> code_diffs <d> largest_missed_quotient <a>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E4M3 (bias 7, subnormals m * 2^-9) */
static float e4m3(int c) {
  const int e = (c >> 3) & 15, m = c & 7;
  return e ? ldexpf(1.0f + m / 8.0f, e - 7) : ldexpf((float)m, -9);
}

/* E2M1 magnitude code of a non-negative value, round to nearest, ties to the
 * even code, saturating at 6 */
static int e2m1_code(float v) {
  static const float bound[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  int c = 0;
  for (int i = 0; i < 7; ++i)
    if (v > bound[i] || (v == bound[i] && (i & 1))) c = i + 1;
  return c;
}

static float via_reciprocal(float a, float b, float y) {
  const float q0 = a * y;
  const float q = fmaf(fmaf(-q0, b, a), y, q0);
  return q0 < INFINITY ? q : q0;
}

int main(void) {
  long long cases = 0, diffs = 0;
  float missed = 0.0f;
  float gs[12];
  int ng = 0;
  for (int i = -30; i <= 30; i += 10) gs[ng++] = ldexpf(1.0f, i) / 2688.0f;
  const float odd[5] = {0.0371f, 1.0f / 3.0f, 7.77e-5f, 123.456f, 0.9999999f};
  for (int i = 0; i < 5; ++i) gs[ng++] = odd[i];
  for (int gi = 0; gi < ng; ++gi)
    for (int sc = 1; sc <= 126; ++sc) {
      const float b = e4m3(sc) * gs[gi];
      const float y = 1.0f / b;
      if (!(b > 0.0f) || !(y < INFINITY)) continue;   /* the encoder divides there */
      for (uint32_t h = 1; h < 0x7F80u; ++h) {
        const float a = from_bits(h << 16);
        const float qr = a / b, q = via_reciprocal(a, b, y);
        ++cases;
        if (to_bits(q) != to_bits(qr) && qr > missed) missed = qr;
        if (e2m1_code(q) != e2m1_code(qr)) ++diffs;
      }
    }
  uint64_t st = 0x9E3779B97F4A7C15ull;
  for (long long it = 0; it < 20000000LL; ++it) {
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    const float a = from_bits((uint32_t)(st & 0x7F7FFFFFu));
    const float b = e4m3(1 + (int)((st >> 40) % 126)) * gs[(st >> 52) % ng];
    const float y = 1.0f / b;
    if (!(b > 0.0f) || !(y < INFINITY)) continue;
    const float qr = a / b, q = via_reciprocal(a, b, y);
    ++cases;
    if (to_bits(q) != to_bits(qr) && !(isinf(q) && isinf(qr)) && qr > missed) missed = qr;
    if (e2m1_code(q) != e2m1_code(qr)) ++diffs;
  }
  printf("cases %lld code_diffs %lld largest_missed_quotient %a\n", cases, diffs, missed);
  return 0;
}
