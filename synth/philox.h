/*
 * Seeded synthetic inputs: the counter-based generator shared by the host
 * generator (synth_host.c, gcc) and the device generator (synth_dev.hip).
 *
 * This module produces INPUTS only (peer gradient chunks, per-tensor
 * gradients, initial fp32 master weights, per-rank valid-token counts).  It
 * holds none of the shard step's arithmetic: no reduction, no normalisation,
 * no optimizer update, and not the round-to-nearest-even bf16 cast of the
 * step (generated bf16 values are truncated, a different rounding on purpose).
 *
 * Generator: Philox4x32-10, as published by Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 4x32-bit counter,
 * a 2x32-bit key, ten rounds of two 32x32->64 multiplies, the key bumped by
 * two Weyl constants between rounds.
 *
 * Normal deviates: Irwin-Hall sum of the eight 16-bit halves of one Philox
 * block.  The centred sum D = 2*sum - 8*65535 is an exact even integer in
 * [-524280, 524280]; the value is (float)((double)D * c) with c = sigma/sd(D)
 * computed once on the host.  Every step (integer ops, exact int->double,
 * one correctly rounded double multiply, one RNE double->float conversion) is
 * bit-reproducible on x86 and on gfx950, so both sides see identical bytes.
 *
 * Include with SYNTH_FN defined to the qualifiers wanted (e.g.
 * "static inline" for C, "__host__ __device__ static inline" for HIP).
 */
#ifndef SBP_SYNTH_PHILOX_H
#define SBP_SYNTH_PHILOX_H

#include <stdint.h>

#ifndef SYNTH_FN
#define SYNTH_FN static inline
#endif

#define SYNTH_PHILOX_M0 0xD2511F53u
#define SYNTH_PHILOX_M1 0xCD9E8D57u
#define SYNTH_PHILOX_W0 0x9E3779B9u
#define SYNTH_PHILOX_W1 0xBB67AE85u

/* stream kinds (top 4 bits of counter word 2) */
#define SYNTH_KIND_PEER 1u    /* peer gradient chunk, shard layout          */
#define SYNTH_KIND_TENSOR 2u  /* per-tensor gradient of one rank            */
#define SYNTH_KIND_MASTER 3u  /* initial fp32 master weights, shard layout  */
#define SYNTH_KIND_TOKENS 4u  /* valid-token count of one rank              */

typedef struct {
  uint32_t v[4];
} synth_u32x4;

SYNTH_FN synth_u32x4 synth_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                         uint32_t c3, uint32_t k0,
                                         uint32_t k1) {
  for (int round = 0; round < 10; ++round) {
    uint64_t p0 = (uint64_t)SYNTH_PHILOX_M0 * (uint64_t)c0;
    uint64_t p1 = (uint64_t)SYNTH_PHILOX_M1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += SYNTH_PHILOX_W0;
    k1 += SYNTH_PHILOX_W1;
  }
  synth_u32x4 r;
  r.v[0] = c0;
  r.v[1] = c1;
  r.v[2] = c2;
  r.v[3] = c3;
  return r;
}

/* Stream words: word 2 = kind<<28 | t (t < 2^28); word 3 = k<<24 | r<<16 | id */
SYNTH_FN uint32_t synth_stream_a(uint32_t kind, uint32_t t) {
  return (kind << 28) | (t & 0x0FFFFFFFu);
}
SYNTH_FN uint32_t synth_stream_b(uint32_t k, uint32_t r, uint32_t id) {
  return ((k & 0xFFu) << 24) | ((r & 0xFFu) << 16) | (id & 0xFFFFu);
}

/* Centred Irwin-Hall integer of element i of a stream. */
SYNTH_FN int32_t synth_ih8(uint64_t seed, uint32_t sa, uint32_t sb,
                           uint64_t i) {
  synth_u32x4 w = synth_philox4x32_10((uint32_t)i, (uint32_t)(i >> 32), sa, sb,
                                      (uint32_t)seed, (uint32_t)(seed >> 32));
  int32_t s = 0;
  for (int q = 0; q < 4; ++q) s += (int32_t)(w.v[q] & 0xFFFFu) + (int32_t)(w.v[q] >> 16);
  return 2 * s - 8 * 65535;
}

/* N(0, sigma)-shaped fp32 value; c = sigma / sd(D) from synth_ih8_scale(). */
SYNTH_FN float synth_normal_f32(uint64_t seed, uint32_t sa, uint32_t sb,
                                uint64_t i, double c) {
  double d = (double)synth_ih8(seed, sa, sb, i);
  return (float)(d * c);
}

/* Same value as bf16 bits, by truncation of the fp32 value. */
SYNTH_FN uint16_t synth_normal_bf16(uint64_t seed, uint32_t sa, uint32_t sb,
                                    uint64_t i, double c) {
  union {
    float f;
    uint32_t u;
  } x;
  x.f = synth_normal_f32(seed, sa, sb, i, c);
  return (uint16_t)(x.u >> 16);
}

#endif
