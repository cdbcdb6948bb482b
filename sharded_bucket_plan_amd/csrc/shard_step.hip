// Streaming kernels of the shard step on CDNA4 (gfx950): the ascending-rank
// reduce of R bf16 peer chunks, microbatch accumulation, and the fused
// reduce + normalise + AdamW + bf16-emit kernel.
//
// The reduce-scatter share and the owned-shard update follow "Parallelisms"
// (vladislavkruglikov.com), sections ZeRO-1 and ZeRO-2, and "Parallelism
// Starts With the Bottleneck" (rajdeepmondal.com), section "ZeRO removes the
// copies without adding bandwidth"; the normalisation follows "Distributed
// Training and Parallelism" (naatyu.github.io), section "Data parallelism and
// the global gradient".  Exact semantics are in include/sbp.h.
//
// Design.  Every kernel here is a single pass over HBM with no reuse, so it
// is bandwidth-bound (about 0.5 flop per byte against a ridge near 20):
//   - each lane owns 8 elements of its tile, and issues all its loads before
//     any arithmetic.  Mostly they are 8 consecutive elements: one 16-byte
//     load per bf16 peer, two 16-byte loads per fp32 stream, 16-byte stores.
//     The fused step with at most 2 peers splits them into two runs of 4, a
//     wave's 64 lanes covering 256 consecutive elements with each run (each
//     fp32 instruction of the wave one contiguous kilobyte; see
//     fused_split_tile);
//   - R is a template parameter so the peer loop unrolls and the peer
//     pointers stay in scalar registers (passed by value in the kernel
//     arguments);
//   - one pass: one 256-lane block per tile of 2048 elements.  The hardware
//     hands blocks to the 8 XCDs round-robin; the tiles are dealt back in
//     chunks of C consecutive tiles per XCD (block b, the k-th block of XCD
//     x = b mod 8, works on tile ((k / C) * 8 + x) * C + k mod C), so each
//     XCD sweeps runs of C * 2048 elements while all eight advance together
//     through every stream.  C = 64 measured on MI355X against one
//     contiguous eighth per XCD: fused step 68.3% -> 70.3% of 8 TB/s,
//     accumulate 67.8% -> 71.0%, norm pass 69.3% -> 75.0%; single tiles
//     round-robin (the hardware order) are slower than either.  The fused
//     step gains another 0.2-0.35 points at C = 32, where the reduce and
//     accumulate passes lose 0.3-1 point, so it has its own C;
//   - the mix of 11-15 read and write streams runs fastest on MI355X when
//     each CU keeps about 56 KB of loads in flight; more outstanding
//     requests congest HBM.  The launch reserves LDS (unused by the kernels)
//     to hold each CU to the number of blocks that gives that depth for the
//     kernel's bytes per lane -- a persistent grid measured slower than
//     letting the dispatcher refill CUs tile by tile;
//   - the n % 8 tail is done element-wise by the first block;
//   - binary32 arithmetic with no contraction (also compiled with
//     -ffp-contract=off): peer sums in ascending order seeded by peer 0,
//     correctly rounded sqrt and divide, so results match a scalar
//     one-rounding-per-operation evaluation bit for bit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <type_traits>
#include <utility>

#include "internal.h"

#pragma clang fp contract(off)

// Build-time tuning knobs (defaults measured best on MI355X): loads in
// flight per CU that the occupancy cap aims at (KiB; 0 = no cap), tiles per
// chunk dealt to one XCD (0 = one contiguous eighth per XCD), and
// nontemporal hints on streaming loads/stores.
#ifndef SBP_INFLIGHT_KB
#define SBP_INFLIGHT_KB 56
#endif
// The reduce and accumulate passes (no state arrays) have their own cap.
#ifndef SBP_REDUCE_INFLIGHT_KB
#define SBP_REDUCE_INFLIGHT_KB SBP_INFLIGHT_KB
#endif
// The squared-norm pass ends every block with a block-wide reduction (a
// barrier); with one block per CU the CU idles through it, so that pass aims
// at more loads in flight: four blocks per CU at R = 8, three with an
// accumulator (at R = 8 on pages spread over the HBM, 74% -> 78% of 8 TB/s
// against three blocks; 72.6% -> 73.8% with the G write).
#ifndef SBP_NORM_INFLIGHT_KB
#define SBP_NORM_INFLIGHT_KB 112
#endif
#ifndef SBP_XCD_CHUNK
#define SBP_XCD_CHUNK 64
#endif
// The fused step's own chunk (its 15 streams per element favour shorter
// runs per XCD than the reduce and accumulate passes).
#ifndef SBP_FUSED_XCD_CHUNK
#define SBP_FUSED_XCD_CHUNK 32
#endif
#ifndef SBP_NT_LOAD
#define SBP_NT_LOAD 0
#endif
#ifndef SBP_NT_STORE
#define SBP_NT_STORE 0
#endif

namespace {

constexpr int kBlock = 256;
constexpr int kXcds = 8;
constexpr bool kNtLoad = SBP_NT_LOAD != 0;
constexpr bool kNtStore = SBP_NT_STORE != 0;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  if constexpr (kNtLoad) return __builtin_nontemporal_load(p);
  else return *p;
}
template <typename T>
__device__ __forceinline__ void stg(T* p, T v) {
  if constexpr (kNtStore) __builtin_nontemporal_store(v, p);
  else *p = v;
}

struct Peers {
  const uint16_t* p[SBP_MAX_PEERS];
};

// Per-call AdamW scalars, each already rounded to binary32 on the host.
struct Scalars {
  float b1, b2, omb1, omb2, eps, step_size, c2, decay;
};

// Parameter groups of the grouped step: the shard's run table (device) and
// each group's step size and decay (binary32, unused slots hold group 0's).
struct GroupArgs {
  const int64_t* run_start;
  const int32_t* run_group;
  int64_t n_runs;
  float step_size[SBP_MAX_GROUPS];
  float decay[SBP_MAX_GROUPS];
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_one(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// binary32 -> bf16 bits: nearest, ties to even; NaN kept (quiet bit set).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return __builtin_isnan(x) ? quiet : rounded;  // a select, not a branch
}

__device__ __forceinline__ void adamw_one(float g, float& th, float& m, float& v,
                                          const Scalars& s) {
  float m1 = s.b1 * m + s.omb1 * g;
  float v1 = s.b2 * v + s.omb2 * (g * g);
  float d = sqrtf(v1) * s.c2 + s.eps;
  th = th * s.decay - s.step_size * (m1 / d);
  m = m1;
  v = v1;
}

// Last run whose start is <= x (run 0 if none is).  Uniform when x is.
__device__ __forceinline__ int64_t find_run(const int64_t* __restrict__ rs, int64_t nr,
                                            int64_t x) {
  int64_t a = 0, b = nr;
  while (b - a > 1) {
    const int64_t mid = a + ((b - a) >> 1);
    if (rs[mid] <= x) a = mid;
    else b = mid;
  }
  return a;
}

// Step size and decay of group g (a chain of selects: the table stays in
// kernel arguments, no indexed private copy); ids outside 1..7 take group 0.
__device__ __forceinline__ void group_pick(const GroupArgs& ga, int32_t g, float& step_size,
                                           float& decay) {
  step_size = ga.step_size[0];
  decay = ga.decay[0];
#pragma unroll
  for (int k = 1; k < SBP_MAX_GROUPS; ++k) {
    step_size = g == k ? ga.step_size[k] : step_size;
    decay = g == k ? ga.decay[k] : decay;
  }
}

// Per-element step size and decay of the lane's 8 elements [e0, e0+8) in a
// tile [lo, lo + 2048).  One search per block (block-uniform, in scalar
// loads); only a tile that holds a run boundary looks elements up one by one.
__device__ __forceinline__ void group_scalars8(const GroupArgs& ga, int64_t lo, int64_t e0,
                                               float (&ss)[8], float (&dc)[8]) {
  const int64_t nr = ga.n_runs;
  const int64_t k = find_run(ga.run_start, nr, lo);
  if (k + 1 >= nr || ga.run_start[k + 1] >= lo + static_cast<int64_t>(kBlock) * 8) {
    float a, b;
    group_pick(ga, ga.run_group[k], a, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ss[j] = a;
      dc[j] = b;
    }
  } else {
    int64_t kk = k;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      while (kk + 1 < nr && ga.run_start[kk + 1] <= e0 + j) ++kk;
      group_pick(ga, ga.run_group[kk], ss[j], dc[j]);
    }
  }
}

// This block's tile in the chunked XCD order (C tiles per chunk).  A
// bijection on [0, gridDim.x): blocks past the last whole round of 8 chunks
// keep their own tile.
template <unsigned C = SBP_XCD_CHUNK>
__device__ __forceinline__ unsigned my_tile() {
  unsigned b = blockIdx.x;
  if constexpr (C > 0) {
    const unsigned full = gridDim.x / (kXcds * C) * (kXcds * C);
    if (b < full) {
      const unsigned x = b % kXcds, k = b / kXcds;
      b = ((k / C) * kXcds + x) * C + k % C;
    }
  } else {
    const unsigned per = gridDim.x / kXcds;
    if (b < per * kXcds) b = (b % kXcds) * per + b / kXcds;
  }
  return b;
}

// Group (8 elements) handled by this lane.
template <unsigned C = SBP_XCD_CHUNK>
__device__ __forceinline__ int64_t my_group() {
  return static_cast<int64_t>(my_tile<C>()) * kBlock + threadIdx.x;
}

// Widen peer 0's 8 bf16 values and add peers 1..R-1 in ascending order.
template <int R>
__device__ __forceinline__ void peer_sum8(const u32x4 (&w)[R], float (&S)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    S[2 * q] = bf16_lo(w[0][q]);
    S[2 * q + 1] = bf16_hi(w[0][q]);
  }
#pragma unroll
  for (int r = 1; r < R; ++r) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      S[2 * q] = S[2 * q] + bf16_lo(w[r][q]);
      S[2 * q + 1] = S[2 * q + 1] + bf16_hi(w[r][q]);
    }
  }
}

template <int R>
__device__ __forceinline__ float peer_sum1(const Peers& P, int64_t i) {
  float s = bf16_one(P.p[0][i]);
#pragma unroll
  for (int r = 1; r < R; ++r) s = s + bf16_one(P.p[r][i]);
  return s;
}

__device__ __forceinline__ void load8(const float* p, int64_t gi, float (&x)[8]) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p) + 2 * gi;
  f32x4 a = ldg(q), b = ldg(q + 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}

__device__ __forceinline__ void store8(float* p, int64_t gi, const float (&x)[8]) {
  f32x4* q = reinterpret_cast<f32x4*>(p) + 2 * gi;
  stg(q, f32x4{x[0], x[1], x[2], x[3]});
  stg(q + 1, f32x4{x[4], x[5], x[6], x[7]});
}

template <int R>
__device__ __forceinline__ void load_peers(const Peers& P, int64_t gi, u32x4 (&w)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) w[r] = ldg(reinterpret_cast<const u32x4*>(P.p[r]) + gi);
}

// ---- reduce: out = fl(S * scale) ------------------------------------------
template <int R>
__global__ void __launch_bounds__(kBlock)
reduce_kernel(Peers P, float scale, float* __restrict__ out, int64_t n) {
  const int64_t groups = n >> 3;
  const int64_t gi = my_group();
  if (gi < groups) {
    u32x4 w[R];
    load_peers<R>(P, gi, w);
    float S[8];
    peer_sum8<R>(w, S);
#pragma unroll
    for (int j = 0; j < 8; ++j) S[j] = S[j] * scale;
    store8(out, gi, S);
  }
  if (blockIdx.x == 0) {
    const int64_t i = (groups << 3) + threadIdx.x;
    if (i < n) out[i] = peer_sum1<R>(P, i) * scale;
  }
}

// ---- accumulate: acc = S (first) or acc + S --------------------------------
template <int R, bool FIRST>
__global__ void __launch_bounds__(kBlock)
accumulate_kernel(Peers P, float* __restrict__ acc, int64_t n) {
  const int64_t groups = n >> 3;
  const int64_t gi = my_group();
  if (gi < groups) {
    u32x4 w[R];
    load_peers<R>(P, gi, w);
    float A[8];
    if (!FIRST) load8(acc, gi, A);
    float S[8];
    peer_sum8<R>(w, S);
    if (!FIRST) {
#pragma unroll
      for (int j = 0; j < 8; ++j) S[j] = A[j] + S[j];
    }
    store8(acc, gi, S);
  }
  if (blockIdx.x == 0) {
    const int64_t i = (groups << 3) + threadIdx.x;
    if (i < n) {
      float s = peer_sum1<R>(P, i);
      acc[i] = FIRST ? s : acc[i] + s;
    }
  }
}

// ---- fused: G = [acc +] S, g = G*scale, AdamW, bf16 emit --------------------
// Plain step with R <= 2 (one parameter group): the lane-to-element map is
// "split" -- lane l of wave w takes elements [w*512 + 4l, +4) and
// [w*512 + 256 + 4l, +4) of its tile -- so each 16-byte fp32 load or store
// instruction of a wave covers one contiguous kilobyte (with 8 consecutive
// elements per lane, an instruction touches every other 16 bytes of 2 KB),
// and each 8-byte bf16 one covers 512 contiguous bytes.  Measured on the
// 1.0B shard, round-robin in two processes against 8 consecutive elements
// per lane: R = 2 +1.0 / +2.1 points of 8 TB/s, the update from G (R = 0)
// +0.9 / +1.4.  With R = 8 the same map needs twice the peer load
// instructions and measured 0.5 points slower; loading each peer's 8
// elements with one 16-byte load and swapping halves between the two lanes
// of a pair with a lane shuffle measured -0.55 points (+0.15 with the
// accumulator), so R >= 3 keeps 8 consecutive elements per lane.
__device__ __forceinline__ void bf16x4(u32x2 u, float (&x)[4]) {
  x[0] = bf16_lo(u.x);
  x[1] = bf16_hi(u.x);
  x[2] = bf16_lo(u.y);
  x[3] = bf16_hi(u.y);
}

template <int R, bool ACC>
__device__ __forceinline__ void fused_split_tile(const Peers& P, const float* __restrict__ acc,
                                                 float scale, float* __restrict__ master,
                                                 float* __restrict__ mom1,
                                                 float* __restrict__ mom2,
                                                 uint16_t* __restrict__ pout, int64_t n,
                                                 const Scalars& s) {
  static_assert(R <= 2, "the split map is for light peer counts");
  const int64_t full = (n >> 3) << 3;  // elements in whole groups of 8
  const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
  const int64_t tile0 = static_cast<int64_t>(my_tile<SBP_FUSED_XCD_CHUNK>()) * (kBlock * 8);
  const int64_t e[2] = {tile0 + wv * 512 + ln * 4, tile0 + wv * 512 + 256 + ln * 4};
  // a run of 4 lies wholly inside or outside [0, full): full is a multiple of 8
  const bool ok[2] = {e[0] < full, e[1] < full};
  u32x2 w[2][R > 0 ? R : 1];
  f32x4 A[2], T[2], M[2], V[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (ok[c]) {
      if constexpr (R > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) w[c][r] = ldg(reinterpret_cast<const u32x2*>(P.p[r] + e[c]));
      }
      if (ACC) A[c] = ldg(reinterpret_cast<const f32x4*>(acc + e[c]));
      T[c] = ldg(reinterpret_cast<const f32x4*>(master + e[c]));
      M[c] = ldg(reinterpret_cast<const f32x4*>(mom1 + e[c]));
      V[c] = ldg(reinterpret_cast<const f32x4*>(mom2 + e[c]));
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (ok[c]) {
      float G[4];
      if constexpr (R > 0) {
        bf16x4(w[c][0], G);
#pragma unroll
        for (int r = 1; r < R; ++r) {
          float x[4];
          bf16x4(w[c][r], x);
#pragma unroll
          for (int j = 0; j < 4; ++j) G[j] = G[j] + x[j];
        }
        if (ACC) {
#pragma unroll
          for (int j = 0; j < 4; ++j) G[j] = A[c][j] + G[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) G[j] = A[c][j];
      }
      float th[4], m[4], v[4];
      uint32_t pb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        th[j] = T[c][j];
        m[j] = M[c][j];
        v[j] = V[c][j];
        adamw_one(G[j] * scale, th[j], m[j], v[j], s);
        pb[j] = bf16_rne(th[j]);
      }
      stg(reinterpret_cast<f32x4*>(master + e[c]), f32x4{th[0], th[1], th[2], th[3]});
      stg(reinterpret_cast<f32x4*>(mom1 + e[c]), f32x4{m[0], m[1], m[2], m[3]});
      stg(reinterpret_cast<f32x4*>(mom2 + e[c]), f32x4{v[0], v[1], v[2], v[3]});
      stg(reinterpret_cast<u32x2*>(pout + e[c]), u32x2{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)});
    }
  }
}

// R >= 3 or GROUPED: 8 consecutive elements per lane.  GROUPED: step size
// and decay per element from the run table in `ga`.
template <int R, bool ACC, bool GROUPED>
__global__ void __launch_bounds__(kBlock)
fused_adamw_kernel(Peers P, const float* __restrict__ acc, float scale,
                   float* __restrict__ master, float* __restrict__ mom1,
                   float* __restrict__ mom2, uint16_t* __restrict__ pout, int64_t n,
                   Scalars s, GroupArgs ga) {
  static_assert(R > 0 || ACC, "R == 0 needs the accumulator");
  const int64_t groups = n >> 3;
  if constexpr (!GROUPED && R <= 2) {
    fused_split_tile<R, ACC>(P, acc, scale, master, mom1, mom2, pout, n, s);
  } else {
    const int64_t gi = my_group<SBP_FUSED_XCD_CHUNK>();
    if (gi < groups) {
      u32x4 w[R > 0 ? R : 1];
      if constexpr (R > 0) load_peers<R>(P, gi, w);
      float A[8], th[8], m[8], v[8];
      if (ACC) load8(acc, gi, A);
      load8(master, gi, th);
      load8(mom1, gi, m);
      load8(mom2, gi, v);
      float G[8];
      if constexpr (R > 0) {
        peer_sum8<R>(w, G);
        if (ACC) {
#pragma unroll
          for (int j = 0; j < 8; ++j) G[j] = A[j] + G[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) G[j] = A[j];
      }
      uint32_t pb[8];
      if constexpr (GROUPED) {
        float ss[8], dc[8];
        group_scalars8(ga, (gi - threadIdx.x) * 8, gi * 8, ss, dc);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          Scalars sj = s;
          sj.step_size = ss[j];
          sj.decay = dc[j];
          adamw_one(G[j] * scale, th[j], m[j], v[j], sj);
          pb[j] = bf16_rne(th[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          adamw_one(G[j] * scale, th[j], m[j], v[j], s);
          pb[j] = bf16_rne(th[j]);
        }
      }
      store8(master, gi, th);
      store8(mom1, gi, m);
      store8(mom2, gi, v);
      stg(reinterpret_cast<u32x4*>(pout) + gi,
          u32x4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                pb[6] | (pb[7] << 16)});
    }
  }  // GROUPED
  if (blockIdx.x == 0) {  // the n % 8 tail, element by element
    const int64_t i = (groups << 3) + threadIdx.x;
    if (i < n) {
      float G;
      if constexpr (R > 0) {
        G = peer_sum1<R>(P, i);
        if (ACC) G = acc[i] + G;
      } else {
        G = acc[i];
      }
      float th = master[i], m = mom1[i], v = mom2[i];
      Scalars si = s;
      if constexpr (GROUPED)
        group_pick(ga, ga.run_group[find_run(ga.run_start, ga.n_runs, i)], si.step_size,
                   si.decay);
      adamw_one(G * scale, th, m, v, si);
      master[i] = th;
      mom1[i] = m;
      mom2[i] = v;
      pout[i] = static_cast<uint16_t>(bf16_rne(th));
    }
  }
}

// ---- squared norm of g = fl(G*scale) in fp64 (for global-norm clipping) -----
// Deterministic: a fixed order within a lane, a fixed shuffle tree within a
// wave, waves in order within a block, one partial per tile, and the tile
// partials summed by a tree of fixed shape (partials_sum_kernel levels).

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = x + __shfl_xor(x, off, 64);
  return x;
}

// Sum of x over the block, in a fixed order; valid in thread 0.
__device__ __forceinline__ double block_sum(double x) {
  __shared__ double per_wave[kBlock / 64];
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) per_wave[threadIdx.x >> 6] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) t = t + per_wave[w];
  }
  return t;
}

// GPL groups of 8 per lane (a tile of 2048 * GPL elements): the light
// configurations (16 or 32 bytes of loads per group) take 4 or 2 so a CU can
// keep enough loads in flight; all of a lane's loads are issued first, and
// its groups are summed in order.
template <int R, bool ACC, bool WRITE, int GPL>
__global__ void __launch_bounds__(kBlock)
sq_norm_kernel(Peers P, const float* __restrict__ acc, float scale, float* __restrict__ gsum,
               int64_t n, double* __restrict__ partial) {
  static_assert(R > 0 || ACC, "R == 0 needs the accumulator");
  const int64_t groups = n >> 3;
  const int64_t g0 = static_cast<int64_t>(my_tile()) * kBlock * GPL + threadIdx.x;
  double local = 0.0;
  u32x4 w[GPL][R > 0 ? R : 1];
  float A[GPL][8];
#pragma unroll
  for (int q = 0; q < GPL; ++q) {
    const int64_t gi = g0 + static_cast<int64_t>(q) * kBlock;
    if (gi < groups) {
      if constexpr (R > 0) load_peers<R>(P, gi, w[q]);
      if (ACC) load8(acc, gi, A[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < GPL; ++q) {
    const int64_t gi = g0 + static_cast<int64_t>(q) * kBlock;
    if (gi < groups) {
      float G[8];
      if constexpr (R > 0) {
        peer_sum8<R>(w[q], G);
        if (ACC) {
#pragma unroll
          for (int j = 0; j < 8; ++j) G[j] = A[q][j] + G[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) G[j] = A[q][j];
      }
      if (WRITE) store8(gsum, gi, G);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double g = static_cast<double>(G[j] * scale);
        local = local + g * g;
      }
    }
  }
  if (blockIdx.x == 0) {
    const int64_t i = (groups << 3) + threadIdx.x;
    if (i < n) {
      float G;
      if constexpr (R > 0) {
        G = peer_sum1<R>(P, i);
        if (ACC) G = acc[i] + G;
      } else {
        G = acc[i];
      }
      if (WRITE) gsum[i] = G;
      const double g = static_cast<double>(G * scale);
      local = local + g * g;
    }
  }
  const double t = block_sum(local);
  if (threadIdx.x == 0) partial[my_tile()] = t;  // one partial per tile, in tile order
}

// One level of the fixed-shape tree over the partials: block b sums
// in[b*kFanIn, (b+1)*kFanIn) -- 8 consecutive values per lane in order, then
// the block sum -- into out[b].
constexpr int kFanIn = kBlock * 8;

__global__ void __launch_bounds__(kBlock)
partials_sum_kernel(const double* __restrict__ in, int64_t count, double* __restrict__ out) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kFanIn + threadIdx.x * 8;
  double t = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (base + j < count) t = t + in[base + j];
  t = block_sum(t);
  if (threadIdx.x == 0) out[blockIdx.x] = t;
}

// ---- launch helpers ---------------------------------------------------------

struct DeviceInfo {
  int cus = 0;
  int lds_per_cu = 0;
};

DeviceInfo device_info() {
  static std::mutex mu;
  static DeviceInfo cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceInfo{256, 0};
  std::lock_guard<std::mutex> lock(mu);
  DeviceInfo& d = cached[dev];
  if (d.cus == 0) {
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        lds < 0)
      lds = 0;
    d.cus = cus;
    d.lds_per_cu = lds;
  }
  return d;
}

struct Launch {
  unsigned grid;
  unsigned lds;  // dynamic LDS reserved per block to cap blocks per CU
};

// Tiles (one 256-lane block each) covering n elements; at least one.
int64_t tiles_for(int64_t n) {
  const int64_t tiles = ((n >> 3) + kBlock - 1) / kBlock;
  return tiles < 1 ? 1 : tiles;
}

// One block per 2048-element tile; `lane_bytes` = bytes one lane loads;
// blocks per CU capped to keep about `inflight_kb` KiB of loads in flight.
Launch launch_for(int64_t n, int lane_bytes, int inflight_kb, int gpl = 1) {
  Launch L{static_cast<unsigned>((tiles_for(n) + gpl - 1) / gpl), 0};
  const DeviceInfo d = device_info();
  if (inflight_kb > 0 && d.lds_per_cu > 0) {
    const int64_t per_block = static_cast<int64_t>(lane_bytes) * kBlock;
    int64_t blocks_per_cu =
        (static_cast<int64_t>(inflight_kb) * 1024 + per_block / 2) / per_block;
    if (blocks_per_cu < 1) blocks_per_cu = 1;
    if (blocks_per_cu < 8)  // beyond that the cap no longer binds
      // 512 bytes of slack so exactly blocks_per_cu reservations fit a CU,
      // together with the few bytes of static LDS the norm kernels use
      L.lds = static_cast<unsigned>(d.lds_per_cu / blocks_per_cu - 512);
  }
  return L;
}

// Large dynamic LDS needs the kernel's limit raised.  A kernel always asks
// for the same reservation on a given device (it depends on its bytes per
// lane and the device's LDS), so this is done once per kernel and device and
// later launches -- also inside a captured graph -- only enqueue.
template <typename K>
sbp_status allow_lds(K kernel, unsigned lds) {
  if (lds <= 65536) return SBP_OK;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const void* key = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({key, dev})) return SBP_OK;
  hipError_t e = hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) {
    (void)hipGetLastError();  // reported through the status, not left for the next check
    return sbp::fail(SBP_EHIP,
                     std::string("raising the kernel's LDS limit failed: ") + hipGetErrorString(e));
  }
  done.insert({key, dev});
  return SBP_OK;
}

sbp_status launched(const char* who) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return sbp::fail(SBP_EHIP, std::string(who) + ": launch failed: " + hipGetErrorString(e));
  return sbp::ok();
}

// Validates R peer pointers (non-null, 16-B aligned) into P.
sbp_status collect_peers(const char* who, const void* const* peers, int32_t R, Peers& P) {
  if (R < 0 || R > SBP_MAX_PEERS)
    return sbp::fail(SBP_EINVAL, std::string(who) + ": R must be in 0..16");
  if (R > 0 && peers == nullptr)
    return sbp::fail(SBP_EINVAL, std::string(who) + ": peers is null");
  for (int r = 0; r < SBP_MAX_PEERS; ++r) P.p[r] = nullptr;
  for (int32_t r = 0; r < R; ++r) {
    if (peers[r] == nullptr)
      return sbp::fail(SBP_EINVAL, std::string(who) + ": a peer pointer is null");
    if (!sbp::aligned(peers[r], 16))
      return sbp::fail(SBP_EALIGN, std::string(who) + ": peer pointers must be 16-byte aligned");
    P.p[r] = static_cast<const uint16_t*>(peers[r]);
  }
  return SBP_OK;
}

// Calls f(std::integral_constant<int, R>) for the runtime R in 0..16.
template <typename F>
sbp_status dispatch_r(int32_t R, F&& f) {
  switch (R) {
#define SBP_CASE(k) \
  case k:           \
    return f(std::integral_constant<int, k>{});
    SBP_CASE(0) SBP_CASE(1) SBP_CASE(2) SBP_CASE(3) SBP_CASE(4) SBP_CASE(5) SBP_CASE(6)
    SBP_CASE(7) SBP_CASE(8) SBP_CASE(9) SBP_CASE(10) SBP_CASE(11) SBP_CASE(12) SBP_CASE(13)
    SBP_CASE(14) SBP_CASE(15) SBP_CASE(16)
#undef SBP_CASE
    default:
      return sbp::fail(SBP_EINVAL, "R must be in 0..16");
  }
}

// Bias corrections 1 - b1^t and 1 - b2^t in float64 from the binary32 betas;
// beta^t by t multiplications.  A training run calls with t = 1, 2, 3, ...,
// so the powers of the last call are kept per thread (with the betas they
// belong to) and extended by the missing multiplications: the same sequence
// of products, hence the same bits, at O(1) cost per step instead of O(t)
// (about a millisecond at t = 10^6).  Any other call starts again from 1.
//
// The products need not run to t.  1 - x rounds to 1 in float64 for every
// 0 <= x <= 2^-54 (at 2^-54 exactly, the tie goes to the even 1.0), and the
// powers never grow (0 <= beta < 1), so once both are that small both
// corrections are exactly 1 at this and every later step.  Waiting for them
// to reach 0 instead would not end: a subnormal power can be a fixed point of
// the rounded product (0.9 times 4 x 2^-1074 rounds back to 4 x 2^-1074).
// Reaching 2^-54 takes about 37.4 / -ln(beta) products: 730 for 0.95, 37,400
// for 0.999, and 6.3 x 10^8 (of the order of a second) for the largest
// binary32 below 1.
struct BetaPowers {
  float b1 = 0.0f, b2 = 0.0f;
  int64_t t = -1;  // no powers kept yet
  double b1t = 1.0, b2t = 1.0;
};
thread_local BetaPowers g_beta_powers;

void bias_corrections(const sbp_adamw_hparams& hp, double& bc1, double& bc2) {
  BetaPowers& c = g_beta_powers;
  const bool same_betas = std::memcmp(&c.b1, &hp.beta1, sizeof(float)) == 0 &&
                          std::memcmp(&c.b2, &hp.beta2, sizeof(float)) == 0;
  if (c.t < 0 || !same_betas || c.t > hp.step) {
    c.b1 = hp.beta1;
    c.b2 = hp.beta2;
    c.t = 0;
    c.b1t = 1.0;
    c.b2t = 1.0;
  }
  const double b1 = hp.beta1, b2 = hp.beta2;
  constexpr double kOneMinusRoundsToOne = 0x1p-54;
  for (; c.t < hp.step; ++c.t) {
    if (c.b1t <= kOneMinusRoundsToOne && c.b2t <= kOneMinusRoundsToOne) {
      c.t = hp.step;  // both corrections are 1 from here on
      break;
    }
    c.b1t *= b1;
    c.b2t *= b2;
  }
  bc1 = 1.0 - c.b1t;
  bc2 = 1.0 - c.b2t;
}

// Host scalars of one AdamW step: float64 from the binary32 hyperparameters,
// each rounded once to binary32.  step_size and decay use (lr, wd).
Scalars adamw_scalars(const sbp_adamw_hparams& hp, double bc1, double bc2, float lr_f,
                      float wd_f) {
  const double lr = lr_f, wd = wd_f, b1 = hp.beta1, b2 = hp.beta2;
  Scalars s;
  s.b1 = hp.beta1;
  s.b2 = hp.beta2;
  s.omb1 = static_cast<float>(1.0 - b1);
  s.omb2 = static_cast<float>(1.0 - b2);
  s.eps = hp.eps;
  s.step_size = static_cast<float>(lr / bc1);
  s.c2 = static_cast<float>(1.0 / sqrt(bc2));
  s.decay = static_cast<float>(1.0 - lr * wd);
  return s;
}

// Launches kernel K with the tile grid and the occupancy cap for
// `lane_bytes` and `inflight_kb`.
template <typename K, typename... Args>
sbp_status launch_capped(const char* who, K kernel, int64_t n, int lane_bytes, int inflight_kb,
                         int gpl, hipStream_t stream, Args... args) {
  const Launch L = launch_for(n, lane_bytes * gpl, inflight_kb, gpl);
  sbp_status st = allow_lds(kernel, L.lds);
  if (st != SBP_OK) return st;
  hipLaunchKernelGGL(kernel, dim3(L.grid), dim3(kBlock), L.lds, stream, args...);
  return launched(who);
}

template <typename K, typename... Args>
sbp_status launch(const char* who, K kernel, int64_t n, int lane_bytes, hipStream_t stream,
                  Args... args) {
  return launch_capped(who, kernel, n, lane_bytes, SBP_INFLIGHT_KB, 1, stream, args...);
}

}  // namespace

extern "C" {

sbp_status sbp_reduce_shard(const void* const* peers, int32_t R, int64_t n, float scale,
                            float* out, hipStream_t stream) {
  const char* who = "sbp_reduce_shard";
  if (R < 1 || R > SBP_MAX_PEERS)
    return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: R must be in 1..16");
  if (n < 0) return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: n < 0");
  if (n == 0) return sbp::ok();  // nothing is read or written
  Peers P;
  sbp_status st = collect_peers(who, peers, R, P);
  if (st != SBP_OK) return st;
  if (out == nullptr) return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: out is null");
  if (!sbp::aligned(out, 16))
    return sbp::fail(SBP_EALIGN, "sbp_reduce_shard: out not 16-B aligned");
  if (n > SBP_MAX_SHARD_NUMEL)
    return sbp::fail(SBP_ERANGE, "sbp_reduce_shard: n above SBP_MAX_SHARD_NUMEL");
  for (int32_t r = 0; r < R; ++r)
    if (sbp::overlaps(out, 4 * n, peers[r], 2 * n))
      return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: out overlaps a peer");
  (void)hipGetLastError();
  return dispatch_r(R, [&](auto rc) -> sbp_status {
    constexpr int RR = decltype(rc)::value;
    if constexpr (RR == 0) {
      return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: R must be >= 1");
    } else {
      return launch_capped(who, reduce_kernel<RR>, n, 16 * RR, SBP_REDUCE_INFLIGHT_KB, 1, stream, P,
                           scale, out, n);
    }
  });
}

sbp_status sbp_accumulate_grads(float* acc, const void* const* peers, int32_t R, int64_t n,
                                int32_t first, hipStream_t stream) {
  const char* who = "sbp_accumulate_grads";
  if (R < 1 || R > SBP_MAX_PEERS)
    return sbp::fail(SBP_EINVAL, "sbp_accumulate_grads: R must be in 1..16");
  if (n < 0) return sbp::fail(SBP_EINVAL, "sbp_accumulate_grads: n < 0");
  if (n == 0) return sbp::ok();
  Peers P;
  sbp_status st = collect_peers(who, peers, R, P);
  if (st != SBP_OK) return st;
  if (acc == nullptr) return sbp::fail(SBP_EINVAL, "sbp_accumulate_grads: acc is null");
  if (!sbp::aligned(acc, 16))
    return sbp::fail(SBP_EALIGN, "sbp_accumulate_grads: acc not 16-B aligned");
  if (n > SBP_MAX_SHARD_NUMEL)
    return sbp::fail(SBP_ERANGE, "sbp_accumulate_grads: n above SBP_MAX_SHARD_NUMEL");
  for (int32_t r = 0; r < R; ++r)
    if (sbp::overlaps(acc, 4 * n, peers[r], 2 * n))
      return sbp::fail(SBP_EINVAL, "sbp_accumulate_grads: acc overlaps a peer");
  (void)hipGetLastError();
  return dispatch_r(R, [&](auto rc) -> sbp_status {
    constexpr int RR = decltype(rc)::value;
    if constexpr (RR == 0) {
      return sbp::fail(SBP_EINVAL, "sbp_accumulate_grads: R must be >= 1");
    } else if (first) {
      return launch_capped(who, accumulate_kernel<RR, true>, n, 16 * RR, SBP_REDUCE_INFLIGHT_KB, 1,
                           stream, P, acc, n);
    } else {
      return launch_capped(who, accumulate_kernel<RR, false>, n, 16 * RR + 32,
                           SBP_REDUCE_INFLIGHT_KB, 1, stream, P, acc, n);
    }
  });
}

}  // extern "C"

namespace {

// Hyperparameter ranges, as torch.optim.AdamW checks them (a NaN fails every
// comparison): betas in [0, 1) keep the bias corrections positive, and lr,
// eps and weight decay are finite and >= 0.
bool valid_betas_eps(const sbp_adamw_hparams& hp) {
  return hp.beta1 >= 0.0f && hp.beta1 < 1.0f && hp.beta2 >= 0.0f && hp.beta2 < 1.0f &&
         hp.eps >= 0.0f && std::isfinite(hp.eps);
}
bool valid_lr_wd(float lr, float wd) {
  return lr >= 0.0f && std::isfinite(lr) && wd >= 0.0f && std::isfinite(wd);
}

// Checks shared by the fused entry points; fills P.
sbp_status check_fused(const char* who, const void* const* peers, int32_t R, const float* acc,
                       float* master, float* m, float* v, void* param_out, int64_t n,
                       const sbp_adamw_hparams* hp, Peers& P) {
  const std::string w(who);
  if (R < 0 || R > SBP_MAX_PEERS) return sbp::fail(SBP_EINVAL, w + ": R must be in 0..16");
  if (n < 0) return sbp::fail(SBP_EINVAL, w + ": n < 0");
  if (hp == nullptr) return sbp::fail(SBP_EINVAL, w + ": hp is null");
  if (hp->step < 1) return sbp::fail(SBP_EINVAL, w + ": step must be >= 1");
  if (!valid_betas_eps(*hp))
    return sbp::fail(SBP_EINVAL, w + ": beta1 and beta2 must be in [0, 1), eps finite and >= 0");
  if (n == 0) return SBP_OK;
  sbp_status st = collect_peers(who, peers, R, P);
  if (st != SBP_OK) return st;
  if (R == 0 && acc == nullptr)
    return sbp::fail(SBP_EINVAL, w + ": R == 0 needs an accumulator");
  if (master == nullptr || m == nullptr || v == nullptr || param_out == nullptr)
    return sbp::fail(SBP_EINVAL, w + ": null state or output pointer");
  const void* dev[5] = {acc, master, m, v, param_out};
  for (const void* p : dev)
    if (p != nullptr && !sbp::aligned(p, 16))
      return sbp::fail(SBP_EALIGN, w + ": device pointers must be 16-byte aligned");
  if (n > SBP_MAX_SHARD_NUMEL) return sbp::fail(SBP_ERANGE, w + ": n above SBP_MAX_SHARD_NUMEL");
  // pairwise disjoint: acc, master, m, v, param_out and the peers
  const void* ptr[5 + SBP_MAX_PEERS];
  int64_t len[5 + SBP_MAX_PEERS];
  int k = 0;
  ptr[k] = acc; len[k++] = acc ? 4 * n : 0;
  ptr[k] = master; len[k++] = 4 * n;
  ptr[k] = m; len[k++] = 4 * n;
  ptr[k] = v; len[k++] = 4 * n;
  ptr[k] = param_out; len[k++] = 2 * n;
  for (int32_t r = 0; r < R; ++r) { ptr[k] = peers[r]; len[k++] = 2 * n; }
  for (int a = 0; a < 5; ++a)  // outputs (and acc) against everything else
    for (int b = a + 1; b < k; ++b)
      if (sbp::overlaps(ptr[a], len[a], ptr[b], len[b]))
        return sbp::fail(SBP_EINVAL, w + ": buffers overlap");
  return SBP_OK;
}

// Launches the fused kernel for the runtime R and accumulator presence.
template <bool GROUPED>
sbp_status launch_fused(const char* who, const Peers& P, int32_t R, const float* acc, float scale,
                        float* master, float* m, float* v, void* param_out, int64_t n,
                        const Scalars& s, const GroupArgs& ga, hipStream_t stream) {
  uint16_t* pout = static_cast<uint16_t*>(param_out);
  const int lane_bytes = 16 * R + 96 + (acc ? 32 : 0);
  (void)hipGetLastError();
  return dispatch_r(R, [&](auto rc) -> sbp_status {
    constexpr int RR = decltype(rc)::value;
    auto go = [&](auto kernel) {
      return launch(who, kernel, n, lane_bytes, stream, P, acc, scale, master, m, v, pout, n, s,
                    ga);
    };
    if constexpr (RR == 0) {
      return go(fused_adamw_kernel<0, true, GROUPED>);
    } else if (acc) {
      return go(fused_adamw_kernel<RR, true, GROUPED>);
    } else {
      return go(fused_adamw_kernel<RR, false, GROUPED>);
    }
  });
}

}  // namespace

extern "C" {

sbp_status sbp_adamw_shard(const void* const* peers, int32_t R, const float* acc, float scale,
                           float* master, float* m, float* v, void* param_out, int64_t n,
                           const sbp_adamw_hparams* hp, hipStream_t stream) {
  const char* who = "sbp_adamw_shard";
  Peers P;
  sbp_status st = check_fused(who, peers, R, acc, master, m, v, param_out, n, hp, P);
  if (st != SBP_OK) return st;
  if (!valid_lr_wd(hp->lr, hp->weight_decay))
    return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: lr and weight_decay must be finite and >= 0");
  if (n == 0) return sbp::ok();  // nothing is read or written
  const GroupArgs none{};
  double bc1, bc2;
  bias_corrections(*hp, bc1, bc2);
  return launch_fused<false>(who, P, R, acc, scale, master, m, v, param_out, n,
                             adamw_scalars(*hp, bc1, bc2, hp->lr, hp->weight_decay), none,
                             stream);
}

sbp_status sbp_adamw_shard_grouped(const void* const* peers, int32_t R, const float* acc,
                                   float scale, float* master, float* m, float* v,
                                   void* param_out, int64_t n, const sbp_adamw_hparams* hp,
                                   const sbp_group_hparams* groups, int32_t n_groups,
                                   const int64_t* run_start, const int32_t* run_group,
                                   int64_t n_runs, hipStream_t stream) {
  const char* who = "sbp_adamw_shard_grouped";
  Peers P;
  sbp_status st = check_fused(who, peers, R, acc, master, m, v, param_out, n, hp, P);
  if (st != SBP_OK) return st;
  if (groups == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_adamw_shard_grouped: groups is null");
  if (n_groups < 1 || n_groups > SBP_MAX_GROUPS)
    return sbp::fail(SBP_EINVAL, "sbp_adamw_shard_grouped: n_groups must be in 1..8");
  for (int32_t k = 0; k < n_groups; ++k)
    if (!valid_lr_wd(groups[k].lr, groups[k].weight_decay))
      return sbp::fail(SBP_EINVAL,
                       "sbp_adamw_shard_grouped: each group's lr and weight_decay must be "
                       "finite and >= 0");
  if (n_runs < 1) return sbp::fail(SBP_EINVAL, "sbp_adamw_shard_grouped: n_runs must be >= 1");
  if (n == 0) return sbp::ok();  // nothing is read or written
  if (run_start == nullptr || run_group == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_adamw_shard_grouped: run table is null");
  if (!sbp::aligned(run_start, 8) || !sbp::aligned(run_group, 4))
    return sbp::fail(SBP_EALIGN, "sbp_adamw_shard_grouped: run table misaligned");
  if (n_runs > INT64_MAX / 8)
    return sbp::fail(SBP_ERANGE, "sbp_adamw_shard_grouped: n_runs too large");
  // the run table is read while the outputs are written
  const void* outs[4] = {master, m, v, param_out};
  const int64_t out_len[4] = {4 * n, 4 * n, 4 * n, 2 * n};
  for (int a = 0; a < 4; ++a)
    if (sbp::overlaps(outs[a], out_len[a], run_start, 8 * n_runs) ||
        sbp::overlaps(outs[a], out_len[a], run_group, 4 * n_runs))
      return sbp::fail(SBP_EINVAL, "sbp_adamw_shard_grouped: run table overlaps an output");
  double bc1, bc2;
  bias_corrections(*hp, bc1, bc2);
  const Scalars s = adamw_scalars(*hp, bc1, bc2, groups[0].lr, groups[0].weight_decay);
  GroupArgs ga{};
  ga.run_start = run_start;
  ga.run_group = run_group;
  ga.n_runs = n_runs;
  for (int k = 0; k < SBP_MAX_GROUPS; ++k) {
    const sbp_group_hparams& g = groups[k < n_groups ? k : 0];
    const Scalars sk = adamw_scalars(*hp, bc1, bc2, g.lr, g.weight_decay);
    ga.step_size[k] = sk.step_size;
    ga.decay[k] = sk.decay;
  }
  return launch_fused<true>(who, P, R, acc, scale, master, m, v, param_out, n, s, ga, stream);
}

// Groups of 8 per lane of the squared-norm pass for `lane_bytes` of loads per
// group: 4 at 16 bytes (one bf16 peer), 2 at 32 bytes (two peers, or the
// accumulator alone), else 1 -- the same choice as the dispatch below.
static int norm_groups_per_lane(int lane_bytes) {
  return lane_bytes == 16 ? 4 : lane_bytes == 32 ? 2 : 1;
}

// Workspace of the squared norm: the tile partials, then each tree level.
static int64_t sq_norm_workspace(int64_t n) {
  int64_t count = tiles_for(n), total = count;
  while (count > kFanIn) {
    count = (count + kFanIn - 1) / kFanIn;
    total += count;
  }
  return total;
}

// Sums `count` partials at `ws` into *out with the fixed-shape tree; the
// levels' outputs go to the workspace right after the partials.
static sbp_status sum_partials(const char* who, double* ws, int64_t count, double* out,
                               hipStream_t stream) {
  double* in = ws;
  double* next = ws + count;
  while (count > kFanIn) {
    const int64_t blocks = (count + kFanIn - 1) / kFanIn;
    hipLaunchKernelGGL(partials_sum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                       stream, in, count, next);
    sbp_status st = launched(who);
    if (st != SBP_OK) return st;
    in = next;
    next += blocks;
    count = blocks;
  }
  hipLaunchKernelGGL(partials_sum_kernel, dim3(1), dim3(kBlock), 0, stream, in, count, out);
  return launched(who);
}

int64_t sbp_grad_sq_norm_workspace(int64_t n) { return n < 0 ? -1 : sq_norm_workspace(n); }

}  // extern "C"

// Validation and launches shared by sbp_grad_sq_norm and its allocation-free
// variant.  `workspace` may be null only when `scratch_ws` supplies it: then
// the arguments are checked first and the workspace is fetched afterwards, so
// a bad argument is reported without touching a device.
static sbp_status grad_sq_norm_on(const char* who, const void* const* peers, int32_t R,
                                  const float* acc, float scale, int64_t n, float* g_sum_out,
                                  double* workspace, int64_t workspace_len, double* sq_out,
                                  hipStream_t stream, sbp_status (*scratch_ws)(double**, int64_t)) {
  const std::string w(who);
  if (R < 0 || R > SBP_MAX_PEERS) return sbp::fail(SBP_EINVAL, w + ": R must be in 0..16");
  if (n < 0) return sbp::fail(SBP_EINVAL, w + ": n < 0");
  if (sq_out == nullptr || (workspace == nullptr && scratch_ws == nullptr))
    return sbp::fail(SBP_EINVAL, w + ": null workspace or result pointer");
  if (!sbp::aligned(sq_out, 8) || !sbp::aligned(workspace, 8))
    return sbp::fail(SBP_EALIGN, w + ": workspace and result must be 8-byte aligned");
  if (n > SBP_MAX_SHARD_NUMEL) return sbp::fail(SBP_ERANGE, w + ": n above SBP_MAX_SHARD_NUMEL");
  const int64_t need = sq_norm_workspace(n);
  if (scratch_ws == nullptr && workspace_len < need)
    return sbp::fail(SBP_EINVAL, w + ": workspace too small (see sbp_grad_sq_norm_workspace)");
  Peers P;
  if (n > 0) {
    sbp_status st = collect_peers(who, peers, R, P);
    if (st != SBP_OK) return st;
    if (R == 0 && acc == nullptr) return sbp::fail(SBP_EINVAL, w + ": R == 0 needs an accumulator");
    if ((acc && !sbp::aligned(acc, 16)) || (g_sum_out && !sbp::aligned(g_sum_out, 16)))
      return sbp::fail(SBP_EALIGN, w + ": device arrays must be 16-byte aligned");
  }
  // outputs (g_sum_out, sq_out, and the workspace) must not overlap any other
  // buffer; the workspace is checked once known
  const void* ptr[4 + SBP_MAX_PEERS];
  int64_t len[4 + SBP_MAX_PEERS];
  int k = 0;
  ptr[k] = g_sum_out; len[k++] = (g_sum_out && n > 0) ? 4 * n : 0;
  ptr[k] = sq_out; len[k++] = 8;
  ptr[k] = acc; len[k++] = (acc && n > 0) ? 4 * n : 0;
  for (int32_t r = 0; n > 0 && r < R; ++r) { ptr[k] = peers[r]; len[k++] = 2 * n; }
  for (int a = 0; a < 2; ++a)
    for (int b = a + 1; b < k; ++b)
      if (sbp::overlaps(ptr[a], len[a], ptr[b], len[b]))
        return sbp::fail(SBP_EINVAL, w + ": buffers overlap");
  if (scratch_ws != nullptr) {
    sbp_status st = scratch_ws(&workspace, need);
    if (st != SBP_OK) return st;
  }
  for (int b = 0; b < k; ++b)
    if (sbp::overlaps(workspace, 8 * need, ptr[b], len[b]))
      return sbp::fail(SBP_EINVAL, w + (b == 1 ? ": result overlaps the workspace"
                                               : ": buffers overlap"));
  (void)hipGetLastError();
  if (n == 0)  // the squared norm of nothing is 0
    return sum_partials(who, workspace, 0, sq_out, stream);
  const int lane_bytes = 16 * R + (acc ? 32 : 0);  // per group of 8
  const int gpl = norm_groups_per_lane(lane_bytes);
  constexpr int kNormInflight = SBP_NORM_INFLIGHT_KB;
  sbp_status st = dispatch_r(R, [&](auto rc) -> sbp_status {
    constexpr int RR = decltype(rc)::value;
    const bool wr = g_sum_out != nullptr;
    auto go = [&](auto kernel, int g) {
      return launch_capped(who, kernel, n, lane_bytes, kNormInflight, g, stream, P, acc, scale,
                           g_sum_out, n, workspace);
    };
    if constexpr (RR == 0) {  // 32 bytes per group
      return wr ? go(sq_norm_kernel<0, true, true, 2>, 2) : go(sq_norm_kernel<0, true, false, 2>, 2);
    } else if (acc) {
      return wr ? go(sq_norm_kernel<RR, true, true, 1>, 1)
                : go(sq_norm_kernel<RR, true, false, 1>, 1);
    } else {
      constexpr int G = RR == 1 ? 4 : RR == 2 ? 2 : 1;  // 16, 32 bytes per group
      return wr ? go(sq_norm_kernel<RR, false, true, G>, G)
                : go(sq_norm_kernel<RR, false, false, G>, G);
    }
  });
  if (st != SBP_OK) return st;
  return sum_partials(who, workspace, (tiles_for(n) + gpl - 1) / gpl, sq_out, stream);
}

// ---- the squared norm without a caller workspace ------------------------------
// The tile partials and tree levels live in one file-scope device array per
// GPU.  Its host-side name is not a device address: the address is looked up
// once per device (with that device current) and only that pointer is passed
// to kernels.  Every slot the tree reads was written earlier in the same call
// (one partial per tile, then each level from the one below), so the array is
// never cleared; calls that overlap on one GPU share it and race.
static __device__ __align__(256) double scratch[SBP_NOALLOC_SCRATCH_DOUBLES];

static sbp_status scratch_workspace(double** ws, int64_t need) {
  if (need > SBP_NOALLOC_SCRATCH_DOUBLES)
    return sbp::fail(SBP_ERANGE, "sbp_grad_sq_norm_noalloc: n needs " + std::to_string(need) +
                                     " workspace doubles, above the " +
                                     std::to_string(SBP_NOALLOC_SCRATCH_DOUBLES) +
                                     " of the static scratch (SBP_NOALLOC_MAX_NUMEL)");
  static std::mutex mu;
  static double* addr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // reported through the status, not left for the next check
    return sbp::fail(SBP_EHIP, std::string("sbp_grad_sq_norm_noalloc: hipGetDevice failed: ") +
                                   hipGetErrorString(e));
  }
  if (dev < 0 || dev >= 64)
    return sbp::fail(SBP_EINVAL, "sbp_grad_sq_norm_noalloc: device id outside 0..63");
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return sbp::fail(SBP_EHIP,
                       std::string("sbp_grad_sq_norm_noalloc: looking up the scratch array "
                                   "failed: ") + hipGetErrorString(e));
    }
    addr[dev] = static_cast<double*>(p);
  }
  *ws = addr[dev];
  return SBP_OK;
}

extern "C" {

sbp_status sbp_grad_sq_norm(const void* const* peers, int32_t R, const float* acc, float scale,
                            int64_t n, float* g_sum_out, double* workspace,
                            int64_t workspace_len, double* sq_out, hipStream_t stream) {
  return grad_sq_norm_on("sbp_grad_sq_norm", peers, R, acc, scale, n, g_sum_out, workspace,
                         workspace_len, sq_out, stream, nullptr);
}

sbp_status sbp_grad_sq_norm_noalloc(const void* const* peers, int32_t R, const float* acc,
                                    float scale, int64_t n, float* g_sum_out, double* sq_out,
                                    hipStream_t stream) {
  return grad_sq_norm_on("sbp_grad_sq_norm_noalloc", peers, R, acc, scale, n, g_sum_out,
                         nullptr, 0, sq_out, stream, scratch_workspace);
}

sbp_status sbp_clip_scale(double total_sq, float max_norm, float scale, float* clipped_scale,
                          double* coef) {
  if (clipped_scale == nullptr) return sbp::fail(SBP_EINVAL, "sbp_clip_scale: null output");
  if (!(max_norm >= 0.0f))  // also rejects NaN
    return sbp::fail(SBP_EINVAL, "sbp_clip_scale: max_norm must be >= 0");
  if (total_sq < 0.0)  // a sum of squares; NaN is let through and propagates
    return sbp::fail(SBP_EINVAL, "sbp_clip_scale: total_sq must be >= 0");
  const double q = static_cast<double>(max_norm) / (sqrt(total_sq) + 1e-6);
  const double c = (q < 1.0 || q != q) ? q : 1.0;  // NaN propagates
  *clipped_scale = static_cast<float>(static_cast<double>(scale) * c);
  if (coef) *coef = c;
  return sbp::ok();
}

}  // extern "C"
