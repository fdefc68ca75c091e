/* The block-fp8 quantiser's shortcut, checked exhaustively on the CPU.
 *
 * The sender's scale is s = RN(amax / 448) (IEEE fp32). Its codes are those
 * of the IEEE quotient q = RN(|x| / s), rounded to e4m3 (nearest, ties to
 * even) after clamping to 448. Instead of one division per value the kernel
 * computes y = RN(1 / s) once per block and, per value,
 *     q0 = RN(|x| * y),  r = fma(-s, q0, |x|),  q1 = fma(r, y, q0).
 * This program runs those operations for every pair of a positive finite
 * bf16 amax and a bf16 magnitude |x| <= amax, and counts, for amax of at
 * least 2^-96 (the kernel's limit for the shortcut), the pairs whose e4m3
 * code from q1 differs from the code from q. It prints the pair count and
 * the mismatch count; exit status 0 iff there is no mismatch.
 *
 * The e4m3 encoder here is written from the format (1 sign, 4 exponent bits
 * of bias 7, 3 fraction bits, largest finite 448). Needs hardware fma
 * (fmaf), round to nearest and no flush of subnormals, which x86-64 gives. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static uint32_t e4m3(float q) { /* 0 <= q <= 448 */
  uint32_t u; memcpy(&u, &q, 4);
  if (q < 0.015625f) return (uint32_t)rintf(q * 512.0f); /* subnormal step 2^-9 */
  const int e = (int)((u >> 23) & 0xff) - 127;           /* 2^e <= q < 2^(e+1) */
  return (uint32_t)((e + 6) * 8) + (uint32_t)rintf(q * from_bits((uint32_t)(127 + 3 - e) << 23));
}

typedef struct { uint32_t lo, hi; unsigned long long pairs, bad; } Job;

static void* run(void* arg) {
  Job* j = (Job*)arg;
  volatile float k448 = 448.0f, one = 1.0f; /* keep the divisions as written */
  for (uint32_t ha = j->lo; ha < j->hi; ++ha) {
    const float amax = from_bits(ha << 16);
    if (!(amax >= 0x1p-96f)) continue;
    const float s = amax / k448;
    const float y = one / s;
    for (uint32_t hx = 0; hx <= ha; ++hx) {
      const float a = from_bits(hx << 16);
      const float q = a / s;
      const float q0 = a * y;
      const float q1 = fmaf(fmaf(-s, q0, a), y, q0);
      j->pairs++;
      if (e4m3(q < 448.0f ? q : 448.0f) != e4m3(q1 < 448.0f ? q1 : 448.0f)) j->bad++;
    }
  }
  return 0;
}

int main(void) {
  enum { kThreads = 8 };
  const uint32_t lo = 1, hi = 0x7f80; /* positive finite bf16 patterns */
  pthread_t t[kThreads];
  Job jobs[kThreads];
  for (int i = 0; i < kThreads; ++i) { /* work grows with ha: split by sqrt */
    jobs[i].lo = lo + (uint32_t)((hi - lo) * sqrt((double)i / kThreads));
    jobs[i].hi = lo + (uint32_t)((hi - lo) * sqrt((double)(i + 1) / kThreads));
    jobs[i].pairs = jobs[i].bad = 0;
    pthread_create(&t[i], 0, run, &jobs[i]);
  }
  unsigned long long pairs = 0, bad = 0;
  for (int i = 0; i < kThreads; ++i) {
    pthread_join(t[i], 0);
    pairs += jobs[i].pairs;
    bad += jobs[i].bad;
  }
  printf("pairs %llu mismatches %llu\n", pairs, bad);
  return bad == 0 ? 0 : 1;
}
