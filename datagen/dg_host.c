/* Host side of the seeded input generator (test/benchmark infrastructure). */
#include <stdint.h>
#include "dg_core.h"

uint64_t dg_key_c(uint64_t seed, uint32_t family, uint32_t layer, uint32_t tensor,
                  uint32_t expert, uint32_t attempt) {
  return dg_key(seed, family, layer, tensor, expert, attempt);
}

int32_t dg_ih12_c(uint64_t key, uint64_t n) { return dg_ih12(key, n); }

/* out[r][c] = value(key, (row0 + r) * ld_full + col0 + c), r < rows, c < cols. */
void dg_fill_bf16(uint16_t* out, uint64_t key, int64_t row0, int64_t col0, int64_t rows,
                  int64_t cols, int64_t ld_full, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint64_t base = (uint64_t)(row0 + r) * (uint64_t)ld_full + (uint64_t)col0;
    uint16_t* o = out + r * cols;
    for (int64_t c = 0; c < cols; ++c) o[c] = dg_value(key, base + (uint64_t)c, scale);
  }
}

/* fp8 codes: out[r][c] = dg_value_fp8(key, (row0 + r) * ld_full + col0 + c, mul). */
void dg_fill_fp8(uint8_t* out, uint64_t key, int64_t row0, int64_t col0, int64_t rows,
                 int64_t cols, int64_t ld_full, int32_t mul) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint64_t base = (uint64_t)(row0 + r) * (uint64_t)ld_full + (uint64_t)col0;
    uint8_t* o = out + r * cols;
    for (int64_t c = 0; c < cols; ++c) o[c] = dg_value_fp8(key, base + (uint64_t)c, mul);
  }
}

uint8_t dg_e4m3_code_c(int32_t s, int32_t mul) { return dg_e4m3_code(s, mul); }

/* Block scales: out[i] = fp32(base * (1 + ih12(key, i) / 2^19)), i < n (a spread of
 * about 1/8 around base). */
void dg_fill_scales(float* out, uint64_t key, int64_t n, double base) {
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(base * (1.0 + (double)dg_ih12(key, (uint64_t)i) / 524288.0));
}
