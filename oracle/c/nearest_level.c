/* Brute-force nearest-level search (oracle; test infrastructure only).
 *
 * The NF4 code of a normalized weight x is the first index j that minimises
 * the fp32 distance |fl32(x - L_j)| over all levels (paperclase lesson
 * "QLoRA", Parte 4: argmin of the distance to the NF4 levels; ultralytics
 * glossary "QLoRA": nearest of the 16 levels).  This is that definition in
 * plain C, for tensors too large for the NumPy version of the same loop.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (SSE scalar float arithmetic: every subtraction is IEEE fp32, correctly
 * rounded; fabsf is exact).
 */
#include <math.h>
#include <stdint.h>

void oracle_nearest_level(const float* x, int64_t n, const float* levels, int n_levels,
                          uint8_t* codes_out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const float xi = x[i];
    int best = 0;
    float best_d = fabsf(xi - levels[0]);
    for (int j = 1; j < n_levels; ++j) {
      const float d = fabsf(xi - levels[j]);
      if (d < best_d) { /* strict: the first minimum wins ties */
        best_d = d;
        best = j;
      }
    }
    codes_out[i] = (uint8_t)best;
  }
}

/* Every fp32 value whose bit pattern lies in [first_bits, first_bits + n):
 * helper that lets a test walk all fp32 numbers of an interval without
 * materialising them in Python. */
void oracle_nearest_level_bits(uint32_t first_bits, int64_t n, const float* levels,
                               int n_levels, uint8_t* codes_out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    union { uint32_t u; float f; } v;
    v.u = first_bits + (uint32_t)i;
    const float xi = v.f;
    int best = 0;
    float best_d = fabsf(xi - levels[0]);
    for (int j = 1; j < n_levels; ++j) {
      const float d = fabsf(xi - levels[j]);
      if (d < best_d) {
        best_d = d;
        best = j;
      }
    }
    codes_out[i] = (uint8_t)best;
  }
}
