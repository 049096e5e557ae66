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
