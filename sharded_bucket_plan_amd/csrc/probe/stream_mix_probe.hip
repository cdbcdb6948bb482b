// Measurement kernels (not part of the shard-step library): passes that move
// exactly the fused R-peer step's traffic -- R bf16 peer reads, the fp32
// master / m / v read and written in place, one bf16 output write -- with no
// arithmetic beyond integer bit operations, so every store depends on every
// load.  The rate of the best of them on the caller's arrays is the ceiling
// of that access mix on that placement, against which the fused kernel's
// rate is read.
//
// With mask = 0 the state arrays are written back unchanged and the output
// array is zeroed, so a probe can run between real steps.
//
// Launch shape as in the library's streaming kernels: one 256-lane block per
// 2048-element tile, tiles dealt to the 8 XCDs in chunks of 64, one block
// per CU (LDS reserved to cap occupancy).  Variants:
//   0  each lane owns 8 consecutive elements, stores at the end
//   1  the same loads; the results go through LDS and wave w stores stream w
//      (master, m, v, output) for the whole tile
//   2  lane l of wave w owns [w*512 + 4l, +4) and [w*512 + 256 + 4l, +4)
// Only whole tiles are covered (n_tiles * 2048 elements).
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
};

__device__ __forceinline__ unsigned chunked_tile() {
  constexpr unsigned C = 64;
  unsigned b = blockIdx.x;
  const unsigned full = gridDim.x / (8 * C) * (8 * C);
  if (b < full) {
    const unsigned x = b % 8, k = b / 8;
    b = ((k / C) * 8 + x) * C + k % C;
  }
  return b;
}

template <int R, int VARIANT>
__global__ void __launch_bounds__(256) mix_probe(Arrays A, uint32_t mask) {
  extern __shared__ u32x4 lds[];
  const unsigned tile = chunked_tile();
  if (VARIANT == 2) {
    const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
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
    return;
  }
  const int64_t gi = (int64_t)tile * 256 + threadIdx.x;
  u32x4 x = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < R; ++r) x ^= reinterpret_cast<const u32x4*>(A.p[r])[gi];
  u32x4 t0 = reinterpret_cast<const u32x4*>(A.th)[2 * gi];
  u32x4 t1 = reinterpret_cast<const u32x4*>(A.th)[2 * gi + 1];
  u32x4 m0 = reinterpret_cast<const u32x4*>(A.m)[2 * gi];
  u32x4 m1 = reinterpret_cast<const u32x4*>(A.m)[2 * gi + 1];
  u32x4 v0 = reinterpret_cast<const u32x4*>(A.v)[2 * gi];
  u32x4 v1 = reinterpret_cast<const u32x4*>(A.v)[2 * gi + 1];
  x &= mask;
  t0 ^= x; t1 ^= x; m0 ^= x; m1 ^= x; v0 ^= x; v1 ^= x;
  if (VARIANT == 0) {
    reinterpret_cast<u32x4*>(A.th)[2 * gi] = t0;
    reinterpret_cast<u32x4*>(A.th)[2 * gi + 1] = t1;
    reinterpret_cast<u32x4*>(A.m)[2 * gi] = m0;
    reinterpret_cast<u32x4*>(A.m)[2 * gi + 1] = m1;
    reinterpret_cast<u32x4*>(A.v)[2 * gi] = v0;
    reinterpret_cast<u32x4*>(A.v)[2 * gi + 1] = v1;
    reinterpret_cast<u32x4*>(A.out)[gi] = x;
  } else {
    // LDS (u32x4 units): master [512], m [512], v [512], output [256]
    const int t = threadIdx.x, wv = t >> 6, ln = t & 63;
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

template <int R>
int launch_r(int variant, const Arrays& A, unsigned tiles, uint32_t mask, hipStream_t stream) {
  int dev = 0, lds_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
      hipSuccess)
    return -1;
  const unsigned lds = static_cast<unsigned>(lds_cu - 512);  // one block per CU (>= 28 KB)
  const void* k = variant == 0 ? (const void*)mix_probe<R, 0>
                  : variant == 1 ? (const void*)mix_probe<R, 1>
                                 : (const void*)mix_probe<R, 2>;
  if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return -1;
  if (variant == 0)
    hipLaunchKernelGGL((mix_probe<R, 0>), dim3(tiles), dim3(256), lds, stream, A, mask);
  else if (variant == 1)
    hipLaunchKernelGGL((mix_probe<R, 1>), dim3(tiles), dim3(256), lds, stream, A, mask);
  else
    hipLaunchKernelGGL((mix_probe<R, 2>), dim3(tiles), dim3(256), lds, stream, A, mask);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

extern "C" {

// One probe pass over n_tiles whole 2048-element tiles.  peers: host array
// of R (1, 2 or 8) device pointers to bf16 arrays; master, m, v: fp32;
// out: bf16; all 16-byte aligned, each at least n_tiles * 2048 elements.
// Returns 0, or -1 on a launch failure / bad argument.
int sbp_probe_stream_mix(int variant, const void* const* peers, int R, void* master, void* m,
                         void* v, void* out, int64_t n_tiles, uint32_t mask, hipStream_t stream) {
  if (variant < 0 || variant > 2 || n_tiles < 1 || n_tiles > (int64_t{1} << 24) - 1 ||
      peers == nullptr || master == nullptr || m == nullptr || v == nullptr || out == nullptr)
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
  const unsigned tiles = static_cast<unsigned>(n_tiles);
  switch (R) {
    case 1: return launch_r<1>(variant, A, tiles, mask, stream);
    case 2: return launch_r<2>(variant, A, tiles, mask, stream);
    case 8: return launch_r<8>(variant, A, tiles, mask, stream);
    default: return -1;
  }
}

}  // extern "C"
