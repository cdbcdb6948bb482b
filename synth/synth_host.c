/*
 * Seeded synthetic inputs, host side (gcc, OpenMP).  Produces the same bytes
 * as synth_dev.hip for every (seed, stream, index); see philox.h.
 * Inputs only: nothing here belongs to the shard step being tested.
 */
#include <math.h>
#include <stdint.h>

#define SYNTH_FN static inline
#include "philox.h"

/* c = sigma / sd(D), D the centred Irwin-Hall integer of philox.h:
 * Var(one 16-bit half) = (65536^2 - 1)/12, eight halves, D = 2*sum - const. */
double synth_ih8_scale(double sigma) {
  double var_half = (65536.0 * 65536.0 - 1.0) / 12.0;
  return sigma / sqrt(4.0 * 8.0 * var_half);
}

void synth_philox(uint32_t out[4], uint32_t c0, uint32_t c1, uint32_t c2,
                  uint32_t c3, uint32_t k0, uint32_t k1) {
  synth_u32x4 r = synth_philox4x32_10(c0, c1, c2, c3, k0, k1);
  for (int q = 0; q < 4; ++q) out[q] = r.v[q];
}

uint32_t synth_stream_word_a(uint32_t kind, uint32_t t) {
  return synth_stream_a(kind, t);
}
uint32_t synth_stream_word_b(uint32_t k, uint32_t r, uint32_t id) {
  return synth_stream_b(k, r, id);
}

void synth_fill_bf16(uint16_t* out, int64_t n, uint64_t seed, uint32_t sa,
                     uint32_t sb, uint64_t i0, double c) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = synth_normal_bf16(seed, sa, sb, i0 + (uint64_t)j, c);
}

void synth_fill_f32(float* out, int64_t n, uint64_t seed, uint32_t sa,
                    uint32_t sb, uint64_t i0, double c) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = synth_normal_f32(seed, sa, sb, i0 + (uint64_t)j, c);
}

void synth_gather_bf16(uint16_t* out, const int64_t* idx, int64_t count,
                       uint64_t seed, uint32_t sa, uint32_t sb, double c) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j)
    out[j] = synth_normal_bf16(seed, sa, sb, (uint64_t)idx[j], c);
}

void synth_gather_f32(float* out, const int64_t* idx, int64_t count,
                      uint64_t seed, uint32_t sa, uint32_t sb, double c) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j)
    out[j] = synth_normal_f32(seed, sa, sb, (uint64_t)idx[j], c);
}

/* Valid-token count of rank r at step t: uniform integer on [lo, hi]. */
int64_t synth_tokens(uint64_t seed, uint32_t t, uint32_t r, int64_t lo,
                     int64_t hi) {
  synth_u32x4 w = synth_philox4x32_10(0u, 0u,
                                      synth_stream_a(SYNTH_KIND_TOKENS, t),
                                      synth_stream_b(0u, r, 0u),
                                      (uint32_t)seed, (uint32_t)(seed >> 32));
  uint64_t span = (uint64_t)(hi - lo + 1);
  uint64_t x = ((uint64_t)w.v[1] << 32) | w.v[0];
  return lo + (int64_t)(x % span);
}
