/* Seeded synthetic-input generator: counter-based, integer-exact.
 *
 * Test and benchmark infrastructure only.  It holds none of the MoE method's
 * arithmetic; it only produces the seeded bf16 (and fp8 code) tensors that both the CPU
 * oracle and the GPU path consume.  The same element is produced bit-for-bit
 * on the host (dg_host.c, gcc) and on the device (dg_device.hip, hipcc)
 * because every step is integer arithmetic followed by exactly one IEEE fp32
 * multiply and one round-to-nearest-even to bf16.
 *
 * Generator: the SplitMix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014, with the
 * 64-bit finaliser constants of Vigna's public-domain splitmix64.c) applied to
 * key + GAMMA * counter, i.e. SplitMix64 used as a counter-based generator.
 *
 * Distribution: the classic twelve-uniform sum (Irwin-Hall with n = 12):
 * s = sum of twelve 16-bit uniforms minus 6 * 65535 has mean 0 and variance
 * 65536^2 - 1, so s / 65536 has unit variance and a near-normal shape
 * (excess kurtosis -0.1, support +-6 sigma).  Value = bf16(float(s) * scale)
 * with scale = sigma / 65536 rounded once to fp32 on the host.
 */
#ifndef MOE_DATAGEN_CORE_H
#define MOE_DATAGEN_CORE_H
#include <stdint.h>

#ifndef DG_FN
#define DG_FN static inline
#endif

#define DG_GAMMA 0x9E3779B97F4A7C15ULL

DG_FN uint64_t dg_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of one tensor slice: absorbs each field in turn. */
DG_FN uint64_t dg_key(uint64_t seed, uint32_t family, uint32_t layer, uint32_t tensor,
                      uint32_t expert, uint32_t attempt) {
  uint64_t k = dg_mix64(seed ^ 0x6D6F652D6465636FULL);
  k = dg_mix64(k + DG_GAMMA * (1ULL + family));
  k = dg_mix64(k + DG_GAMMA * (1ULL + layer));
  k = dg_mix64(k + DG_GAMMA * (1ULL + tensor));
  k = dg_mix64(k + DG_GAMMA * (1ULL + expert));
  k = dg_mix64(k + DG_GAMMA * (1ULL + attempt));
  return k;
}

/* Integer Irwin-Hall(12) sample for flat element index n of the keyed tensor. */
DG_FN int32_t dg_ih12(uint64_t key, uint64_t n) {
  int32_t s = 0;
  for (int t = 0; t < 3; ++t) {
    uint64_t r = dg_mix64(key + DG_GAMMA * (3ULL * n + (uint64_t)t + 1ULL));
    s += (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
         (int32_t)((r >> 32) & 0xFFFF) + (int32_t)((r >> 48) & 0xFFFF);
  }
  return s - 6 * 65535;
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are always finite). */
DG_FN uint16_t dg_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

DG_FN uint16_t dg_value(uint64_t key, uint64_t n, float scale) {
  float x = (float)dg_ih12(key, n);  /* exact: |s| < 2^24 */
  return dg_f32_to_bf16(x * scale);
}

/* fp8 e4m3 (OCP "e4m3fn") code of v = s * mul / 65536, rounded to nearest
 * (ties to even) and saturated at +-448; integer arithmetic only, so host and
 * device agree.  Used to draw synthetic block-quantised expert weights
 * directly in the code domain (s: an Irwin-Hall(12) sample, mul: the code-unit
 * standard deviation).  Values are q * 2^p with q < 16; exponent field p + 10
 * for q >= 8, field 0 (subnormal, p = -9) for q < 8. */
DG_FN uint8_t dg_e4m3_code(int32_t s, int32_t mul) {
  const uint8_t sign = s < 0 ? 0x80u : 0u;
  const uint64_t a = (uint64_t)(s < 0 ? -(int64_t)s : (int64_t)s) * (uint64_t)mul;
  if (a == 0) return sign;
  int lg = 0;
  for (uint64_t t = a; t > 1; t >>= 1) ++lg;
  int e = lg - 16;
  if (e < -6) e = -6;
  int p = e - 3;
  const int sh = 16 + p;
  uint64_t q;
  if (sh <= 0) {
    q = a << (-sh);
  } else {
    q = a >> sh;
    const uint64_t rem = a & ((1ULL << sh) - 1ULL), half = 1ULL << (sh - 1);
    if (rem > half || (rem == half && (q & 1ULL))) ++q;
  }
  if (q >= 16) {
    q >>= 1;
    ++p;
  }
  const int ef = p + 10;
  if (ef > 15 || (ef == 15 && q > 14)) return (uint8_t)(sign | 0x7Eu);
  if (q < 8) return (uint8_t)(sign | (uint8_t)q);
  return (uint8_t)(sign | (uint8_t)((ef << 3) | (int)(q - 8)));
}

DG_FN uint8_t dg_value_fp8(uint64_t key, uint64_t n, int32_t mul) {
  return dg_e4m3_code(dg_ih12(key, n), mul);
}

#endif
