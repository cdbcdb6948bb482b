// Measurement kernels (not part of the shard-step library): passes that move
// exactly the fused R-peer step's traffic -- R bf16 peer reads, the fp32
// master / m / v read and written in place, one bf16 output write -- with no
// arithmetic beyond integer bit operations, so every store depends on every
// load.  The best of them on the caller's arrays is the ceiling of that
// access mix on that placement, against which the fused kernel's rate is
// read; the others and the read-only / write-only halves of the mix map the
// design space around it.
//
// With mask = 0 the state arrays are written back unchanged and the output
// array is zeroed, so a probe can run between real steps (the write-only
// variant does overwrite the state).
//
// Launch shape as in the library's streaming kernels: one 256-lane block per
// tile, tiles dealt to the 8 XCDs in chunks of `xcd_chunk` consecutive tiles
// (0: one contiguous eighth per XCD; 1: the hardware's round-robin), and
// `blocks_per_cu` blocks per CU at most (LDS reserved to cap occupancy; 0:
// no cap).  Variants (tile = 2048 elements unless stated):
//   0  each lane owns 8 consecutive elements, stores at the end
//   1  as 0; the results go through LDS and wave w stores stream w (master,
//      m, v, output) for the whole tile
//   2  lane l of wave w owns [w*512 + 4l, +4) and [w*512 + 256 + 4l, +4)
//   3  read-only: the R + 3 read streams of variant 0, no stores
//   4  write-only: the 4 write streams of variant 0, no loads
//   5  16 consecutive elements per lane (tile 4096)
//   6  two groups of 8 per lane, 256 groups apart (tile 4096)
//   7  as 1, and the loads too go through LDS: wave w loads whole streams of
//      the tile (peers 2w and 2w+1, and master / m / v for w < 3); R = 8 only
// Only whole tiles are covered.
//
// sbp_probe_streams moves the traffic of each of the library's other
// streaming kernels the same way (reduce, accumulate, the squared-norm
// pass, the pack's copy, the fused step from G or with an accumulator), so
// each kernel's rate can be read against the ceiling of its own mix.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kMaxPeers = 16;

struct Arrays {
  const uint16_t* p[kMaxPeers];
  uint32_t* th;
  uint32_t* m;
  uint32_t* v;
  uint16_t* out;
  uint32_t* sink;
};

__device__ __forceinline__ unsigned dealt_tile(unsigned C) {
  unsigned b = blockIdx.x;
  if (C > 0) {
    const unsigned full = gridDim.x / (8 * C) * (8 * C);
    if (b < full) {
      const unsigned x = b % 8, k = b / 8;
      b = ((k / C) * 8 + x) * C + k % C;
    }
  } else {
    const unsigned per = gridDim.x / 8;
    if (b < per * 8) b = (b % 8) * per + b / 8;
  }
  return b;
}

// Groups of 8 (u32x4 of bf16, two u32x4 of fp32) at group index g.
template <int R>
__device__ __forceinline__ u32x4 peers_x(const Arrays& A, int64_t g) {
  u32x4 x = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < R; ++r) x ^= reinterpret_cast<const u32x4*>(A.p[r])[g];
  return x;
}

template <int R, int VARIANT>
__global__ void __launch_bounds__(256) mix_probe(Arrays A, uint32_t mask, unsigned C) {
  extern __shared__ u32x4 lds[];
  const unsigned tile = dealt_tile(C);
  const int t = threadIdx.x, wv = t >> 6, ln = t & 63;
  if constexpr (VARIANT == 2) {
    const int64_t e0 = (int64_t)tile * 2048 + wv * 512 + ln * 4, e1 = e0 + 256;
    u32x2 x0 = {0, 0}, x1 = {0, 0};
#pragma unroll
    for (int r = 0; r < R; ++r) {
      x0 ^= *reinterpret_cast<const u32x2*>(A.p[r] + e0);
      x1 ^= *reinterpret_cast<const u32x2*>(A.p[r] + e1);
    }
    u32x4 t0 = *reinterpret_cast<const u32x4*>(A.th + e0);
    u32x4 t1 = *reinterpret_cast<const u32x4*>(A.th + e1);
    u32x4 m0 = *reinterpret_cast<const u32x4*>(A.m + e0);
    u32x4 m1 = *reinterpret_cast<const u32x4*>(A.m + e1);
    u32x4 v0 = *reinterpret_cast<const u32x4*>(A.v + e0);
    u32x4 v1 = *reinterpret_cast<const u32x4*>(A.v + e1);
    x0 &= mask;
    x1 &= mask;
    const u32x4 y0 = {x0.x, x0.y, x0.x, x0.y}, y1 = {x1.x, x1.y, x1.x, x1.y};
    *reinterpret_cast<u32x4*>(A.th + e0) = t0 ^ y0;
    *reinterpret_cast<u32x4*>(A.th + e1) = t1 ^ y1;
    *reinterpret_cast<u32x4*>(A.m + e0) = m0 ^ y0;
    *reinterpret_cast<u32x4*>(A.m + e1) = m1 ^ y1;
    *reinterpret_cast<u32x4*>(A.v + e0) = v0 ^ y0;
    *reinterpret_cast<u32x4*>(A.v + e1) = v1 ^ y1;
    *reinterpret_cast<u32x2*>(A.out + e0) = x0;
    *reinterpret_cast<u32x2*>(A.out + e1) = x1;
  } else if constexpr (VARIANT == 5 || VARIANT == 6) {
    // two groups per lane: adjacent (5) or 256 groups apart (6)
    const int64_t ga = VARIANT == 5 ? ((int64_t)tile * 256 + t) * 2 : (int64_t)tile * 512 + t;
    const int64_t gb = VARIANT == 5 ? ga + 1 : ga + 256;
    u32x4 xa = peers_x<R>(A, ga), xb = peers_x<R>(A, gb);
    u32x4 T[4], M[4], V[4];
    const int64_t gg[2] = {ga, gb};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        T[2 * h + j] = reinterpret_cast<const u32x4*>(A.th)[2 * gg[h] + j];
        M[2 * h + j] = reinterpret_cast<const u32x4*>(A.m)[2 * gg[h] + j];
        V[2 * h + j] = reinterpret_cast<const u32x4*>(A.v)[2 * gg[h] + j];
      }
    xa &= mask;
    xb &= mask;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 x = h ? xb : xa;
        reinterpret_cast<u32x4*>(A.th)[2 * gg[h] + j] = T[2 * h + j] ^ x;
        reinterpret_cast<u32x4*>(A.m)[2 * gg[h] + j] = M[2 * h + j] ^ x;
        reinterpret_cast<u32x4*>(A.v)[2 * gg[h] + j] = V[2 * h + j] ^ x;
      }
    reinterpret_cast<u32x4*>(A.out)[ga] = xa;
    reinterpret_cast<u32x4*>(A.out)[gb] = xb;
  } else if constexpr (VARIANT == 4) {
    const int64_t gi = (int64_t)tile * 256 + t;
    const u32x4 x = {(uint32_t)gi & mask, mask, mask, mask};
    reinterpret_cast<u32x4*>(A.th)[2 * gi] = x;
    reinterpret_cast<u32x4*>(A.th)[2 * gi + 1] = x;
    reinterpret_cast<u32x4*>(A.m)[2 * gi] = x;
    reinterpret_cast<u32x4*>(A.m)[2 * gi + 1] = x;
    reinterpret_cast<u32x4*>(A.v)[2 * gi] = x;
    reinterpret_cast<u32x4*>(A.v)[2 * gi + 1] = x;
    reinterpret_cast<u32x4*>(A.out)[gi] = x;
  } else {
    const int64_t gi = (int64_t)tile * 256 + t;
    u32x4 x, t0, t1, m0, m1, v0, v1;
    if constexpr (VARIANT == 7) {
      // LDS (u32x4 units): peers [8][256], master [512], m [512], v [512]
      const int64_t tg = (int64_t)tile * 256;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4* src = reinterpret_cast<const u32x4*>(A.p[2 * wv + q]) + tg;
#pragma unroll
        for (int j = 0; j < 4; ++j) lds[(2 * wv + q) * 256 + j * 64 + ln] = src[j * 64 + ln];
      }
      if (wv < 3) {
        const u32x4* src =
            reinterpret_cast<const u32x4*>(wv == 0 ? A.th : wv == 1 ? A.m : A.v) + 2 * tg;
#pragma unroll
        for (int j = 0; j < 8; ++j) lds[2048 + wv * 512 + j * 64 + ln] = src[j * 64 + ln];
      }
      __syncthreads();
      x = lds[t];
#pragma unroll
      for (int r = 1; r < 8; ++r) x ^= lds[r * 256 + t];
      t0 = lds[2048 + 2 * t]; t1 = lds[2048 + 2 * t + 1];
      m0 = lds[2560 + 2 * t]; m1 = lds[2560 + 2 * t + 1];
      v0 = lds[3072 + 2 * t]; v1 = lds[3072 + 2 * t + 1];
      __syncthreads();
    } else {
      x = peers_x<R>(A, gi);
      t0 = reinterpret_cast<const u32x4*>(A.th)[2 * gi];
      t1 = reinterpret_cast<const u32x4*>(A.th)[2 * gi + 1];
      m0 = reinterpret_cast<const u32x4*>(A.m)[2 * gi];
      m1 = reinterpret_cast<const u32x4*>(A.m)[2 * gi + 1];
      v0 = reinterpret_cast<const u32x4*>(A.v)[2 * gi];
      v1 = reinterpret_cast<const u32x4*>(A.v)[2 * gi + 1];
    }
    if constexpr (VARIANT == 3) {
      const u32x4 y = x ^ t0 ^ t1 ^ m0 ^ m1 ^ v0 ^ v1;
      if ((y.x ^ y.y ^ y.z ^ y.w) == (0x9E3779B9u | ~mask)) A.sink[0] = y.x;  // never with mask 0
      return;
    }
    x &= mask;
    t0 ^= x; t1 ^= x; m0 ^= x; m1 ^= x; v0 ^= x; v1 ^= x;
    if constexpr (VARIANT == 0) {
      reinterpret_cast<u32x4*>(A.th)[2 * gi] = t0;
      reinterpret_cast<u32x4*>(A.th)[2 * gi + 1] = t1;
      reinterpret_cast<u32x4*>(A.m)[2 * gi] = m0;
      reinterpret_cast<u32x4*>(A.m)[2 * gi + 1] = m1;
      reinterpret_cast<u32x4*>(A.v)[2 * gi] = v0;
      reinterpret_cast<u32x4*>(A.v)[2 * gi + 1] = v1;
      reinterpret_cast<u32x4*>(A.out)[gi] = x;
    } else {
      // LDS (u32x4 units): master [512], m [512], v [512], output [256]
      lds[2 * t] = t0; lds[2 * t + 1] = t1;
      lds[512 + 2 * t] = m0; lds[512 + 2 * t + 1] = m1;
      lds[1024 + 2 * t] = v0; lds[1024 + 2 * t + 1] = v1;
      lds[1536 + t] = x;
      __syncthreads();
      const int64_t tg = (int64_t)tile * 256;
      if (wv < 3) {
        u32x4* dst = reinterpret_cast<u32x4*>(wv == 0 ? A.th : wv == 1 ? A.m : A.v) + 2 * tg;
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[j * 64 + ln] = lds[wv * 512 + j * 64 + ln];
      } else {
        u32x4* dst = reinterpret_cast<u32x4*>(A.out) + tg;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j * 64 + ln] = lds[1536 + j * 64 + ln];
      }
    }
  }
}

// Plain copy, 16 bytes per lane, four per lane 256 lanes apart (tile 16 KiB).
__global__ void __launch_bounds__(256) copy_probe(const u32x4* __restrict__ a,
                                                  u32x4* __restrict__ b, unsigned C) {
  const unsigned tile = dealt_tile(C);
  const int64_t base = (int64_t)tile * 1024 + threadIdx.x;
  u32x4 x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = a[base + j * 256];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[base + j * 256] = x[j];
}

// ---- the traffic of any of the library's streaming kernels ------------------
// RB bf16 read streams, RF fp32 read streams of which the first WF are
// written back in place, WG fp32 write-only streams (0 or 1), WB bf16
// write-only streams (0 or 1).  GPL groups of 8 consecutive elements per
// lane, the groups of a lane 256 apart (tile = 2048 * GPL elements); every
// load of a lane before its stores.  Every store depends on every load of its
// group; with mask = 0 in-place streams are written back unchanged and the
// write-only streams get zeros.
struct StreamArrays {
  const u32x4* b[8];
  u32x4* f[4];
  u32x4* g;
  u32x4* o;
  uint32_t* sink;
};

template <int RB, int RF, int WF, int WG, int WB, int GPL>
__global__ void __launch_bounds__(256) streams_probe(StreamArrays A, uint32_t mask, unsigned C) {
  static_assert(WF <= RF && RB <= 8 && RF <= 4, "stream counts");
  const int64_t g0 = (int64_t)dealt_tile(C) * 256 * GPL + threadIdx.x;
  u32x4 x[GPL];
  u32x4 F[GPL][RF > 0 ? RF : 1][2];
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
    const int64_t gi = g0 + j * 256;
    x[j] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < RB; ++r) x[j] ^= A.b[r][gi];
#pragma unroll
    for (int q = 0; q < RF; ++q) {
      F[j][q][0] = A.f[q][2 * gi];
      F[j][q][1] = A.f[q][2 * gi + 1];
    }
  }
#pragma unroll
  for (int j = 0; j < GPL; ++j) {
#pragma unroll
    for (int q = WF; q < RF; ++q) x[j] ^= F[j][q][0] ^ F[j][q][1];
  }
  if constexpr (WF + WG + WB == 0) {
    u32x4 y = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < GPL; ++j) y ^= x[j];
    if ((y.x ^ y.y ^ y.z ^ y.w) == (0x9E3779B9u | ~mask)) A.sink[0] = y.x;  // never with mask 0
  } else {
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int64_t gi = g0 + j * 256;
      const u32x4 y = x[j] & mask;
#pragma unroll
      for (int q = 0; q < WF; ++q) {
        A.f[q][2 * gi] = F[j][q][0] ^ y;
        A.f[q][2 * gi + 1] = F[j][q][1] ^ y;
      }
      if constexpr (WG) {
        A.g[2 * gi] = y;
        A.g[2 * gi + 1] = y;
      }
      if constexpr (WB) A.o[gi] = y;
    }
  }
}

constexpr unsigned kLdsNeed[8] = {0, 1792 * 16, 0, 0, 0, 0, 0, 3584 * 16};

int lds_cap(int blocks_per_cu, unsigned need, unsigned* out) {
  int dev = 0, lds_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
      hipSuccess)
    return -1;
  unsigned lds = blocks_per_cu > 0 ? static_cast<unsigned>(lds_cu / blocks_per_cu - 512) : 0;
  *out = lds < need ? need : lds;
  return 0;
}

template <typename K, typename... Args>
int go(K kernel, unsigned grid, unsigned lds, hipStream_t stream, Args... args) {
  if (lds > 65536 && hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds)) != hipSuccess)
    return -1;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), lds, stream, args...);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int R>
int launch_r(int variant, const Arrays& A, unsigned tiles, uint32_t mask, unsigned lds,
             unsigned C, hipStream_t stream) {
  const unsigned wide = tiles / 2;  // 4096-element tiles of variants 5 and 6
  switch (variant) {
    case 0: return go(mix_probe<R, 0>, tiles, lds, stream, A, mask, C);
    case 1: return go(mix_probe<R, 1>, tiles, lds, stream, A, mask, C);
    case 2: return go(mix_probe<R, 2>, tiles, lds, stream, A, mask, C);
    case 3: return go(mix_probe<R, 3>, tiles, lds, stream, A, mask, C);
    case 4: return go(mix_probe<R, 4>, tiles, lds, stream, A, mask, C);
    case 5: return wide ? go(mix_probe<R, 5>, wide, lds, stream, A, mask, C) : -1;
    case 6: return wide ? go(mix_probe<R, 6>, wide, lds, stream, A, mask, C) : -1;
    case 7: return R == 8 ? go(mix_probe<R, 7>, tiles, lds, stream, A, mask, C) : -1;
    default: return -1;
  }
}

// The shapes (RB, RF, WF, WG, WB) of the library's kernels: the squared-norm
// pass at R = 1, 2, 8, of the accumulator, and at R = 8 with it; the pack
// (a bf16 copy); reduce at R = 1 and R = 8 (also the norm pass writing G and
// the first accumulate); the later accumulate; the fused step from G, at
// R = 2, at R = 8 and at R = 8 with the accumulator.
#define SBP_PROBE_SHAPES(X) \
  X(1, 0, 0, 0, 0) X(2, 0, 0, 0, 0) X(0, 1, 0, 0, 0) X(8, 0, 0, 0, 0) X(8, 1, 0, 0, 0) \
  X(1, 0, 0, 0, 1) X(1, 0, 0, 1, 0) X(8, 0, 0, 1, 0) X(8, 1, 1, 0, 0) X(0, 4, 3, 0, 1) \
  X(2, 3, 3, 0, 1) X(8, 3, 3, 0, 1) X(8, 4, 3, 0, 1)

int launch_streams(const int* sh, int gpl, const StreamArrays& A, unsigned grid, uint32_t mask,
                   unsigned lds, unsigned C, hipStream_t stream) {
#define SBP_PROBE_TRY(rb, rf, wf, wg, wb)                                                  \
  if (sh[0] == rb && sh[1] == rf && sh[2] == wf && sh[3] == wg && sh[4] == wb) {           \
    if (gpl == 1) return go(streams_probe<rb, rf, wf, wg, wb, 1>, grid, lds, stream, A, mask, C); \
    if (gpl == 2) return go(streams_probe<rb, rf, wf, wg, wb, 2>, grid, lds, stream, A, mask, C); \
    if (gpl == 4) return go(streams_probe<rb, rf, wf, wg, wb, 4>, grid, lds, stream, A, mask, C); \
    return -1;                                                                             \
  }
  SBP_PROBE_SHAPES(SBP_PROBE_TRY)
#undef SBP_PROBE_TRY
  return -1;
}

}  // namespace

extern "C" {

// One zero-arithmetic pass of shape sh = {RB, RF, WF, WG, WB} (one of the
// shapes listed above) over n_tiles whole tiles of 2048 * gpl elements (gpl
// 1, 2 or 4).  b: host array of RB device pointers to bf16 arrays; f: host
// array of RF device pointers to fp32 arrays (the first WF written back in
// place); g: fp32 array (WG = 1) or null; o: bf16 array (WB = 1) or null;
// sink: one device uint32 (read-only shapes).  Every array 16-byte aligned
// and at least n_tiles * 2048 * gpl elements; the written ones disjoint from
// the others.  blocks_per_cu: 0 = no cap.  Returns 0, or -1 on a bad
// argument or a launch failure.
int sbp_probe_streams(const int* sh, int gpl, const void* const* b, void* const* f, void* g,
                      void* o, void* sink, int64_t n_tiles, uint32_t mask, int blocks_per_cu,
                      unsigned xcd_chunk, hipStream_t stream) {
  if (sh == nullptr || sh[0] < 0 || sh[0] > 8 || sh[1] < 0 || sh[1] > 4 || sh[2] < 0 ||
      sh[2] > sh[1] || sh[3] < 0 || sh[3] > 1 || sh[4] < 0 || sh[4] > 1 ||
      (gpl != 1 && gpl != 2 && gpl != 4) || n_tiles < 1 || n_tiles > (int64_t{1} << 24) - 1 ||
      sink == nullptr || blocks_per_cu < 0 || blocks_per_cu > 8 ||
      (sh[0] > 0 && b == nullptr) || (sh[1] > 0 && f == nullptr) ||
      (sh[3] && g == nullptr) || (sh[4] && o == nullptr))
    return -1;
  StreamArrays A{};
  for (int r = 0; r < sh[0]; ++r) {
    if (b[r] == nullptr) return -1;
    A.b[r] = static_cast<const u32x4*>(b[r]);
  }
  for (int q = 0; q < sh[1]; ++q) {
    if (f[q] == nullptr) return -1;
    A.f[q] = static_cast<u32x4*>(f[q]);
  }
  A.g = static_cast<u32x4*>(g);
  A.o = static_cast<u32x4*>(o);
  A.sink = static_cast<uint32_t*>(sink);
  unsigned lds = 0;
  if (lds_cap(blocks_per_cu, 0, &lds)) return -1;
  return launch_streams(sh, gpl, A, static_cast<unsigned>(n_tiles), mask, lds, xcd_chunk, stream);
}

// One probe pass over n_tiles whole 2048-element tiles (variants 5 and 6
// cover the whole 4096-element tiles inside them).  peers: host array of R
// (1, 2 or 8) device pointers to bf16 arrays; master, m, v: fp32; out: bf16;
// sink: one device uint32 (read-only variant); all 16-byte aligned, each
// array at least n_tiles * 2048 elements.  blocks_per_cu: 0 = no cap.
// Returns 0, or -1 on a launch failure or a bad argument.
int sbp_probe_stream_mix(int variant, const void* const* peers, int R, void* master, void* m,
                         void* v, void* out, void* sink, int64_t n_tiles, uint32_t mask,
                         int blocks_per_cu, unsigned xcd_chunk, hipStream_t stream) {
  if (variant < 0 || variant > 7 || n_tiles < 1 || n_tiles > (int64_t{1} << 24) - 1 ||
      peers == nullptr || master == nullptr || m == nullptr || v == nullptr || out == nullptr ||
      sink == nullptr || blocks_per_cu < 0 || blocks_per_cu > 8)
    return -1;
  Arrays A{};
  for (int r = 0; r < R && r < kMaxPeers; ++r) {
    if (peers[r] == nullptr) return -1;
    A.p[r] = static_cast<const uint16_t*>(peers[r]);
  }
  A.th = static_cast<uint32_t*>(master);
  A.m = static_cast<uint32_t*>(m);
  A.v = static_cast<uint32_t*>(v);
  A.out = static_cast<uint16_t*>(out);
  A.sink = static_cast<uint32_t*>(sink);
  unsigned lds = 0;
  if (lds_cap(blocks_per_cu, kLdsNeed[variant], &lds)) return -1;
  const unsigned tiles = static_cast<unsigned>(n_tiles);
  switch (R) {
    case 1: return launch_r<1>(variant, A, tiles, mask, lds, xcd_chunk, stream);
    case 2: return launch_r<2>(variant, A, tiles, mask, lds, xcd_chunk, stream);
    case 8: return launch_r<8>(variant, A, tiles, mask, lds, xcd_chunk, stream);
    default: return -1;
  }
}

// Copy of `bytes` (a multiple of 16 KiB, at most 2^24 - 1 tiles) from a to
// b, 16-byte aligned and disjoint.
int sbp_probe_copy(const void* a, void* b, int64_t bytes, int blocks_per_cu, unsigned xcd_chunk,
                   hipStream_t stream) {
  if (a == nullptr || b == nullptr || bytes <= 0 || bytes % 16384 != 0 ||
      bytes / 16384 > (int64_t{1} << 24) - 1 || blocks_per_cu < 0 || blocks_per_cu > 8)
    return -1;
  unsigned lds = 0;
  if (lds_cap(blocks_per_cu, 0, &lds)) return -1;
  return go(copy_probe, static_cast<unsigned>(bytes / 16384), lds, stream,
            static_cast<const u32x4*>(a), static_cast<u32x4*>(b), xcd_chunk);
}

}  // extern "C"
