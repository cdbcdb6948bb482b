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
//   - each lane owns 8 consecutive elements: one 16-byte load per bf16 peer,
//     two 16-byte loads per fp32 stream, 16-byte stores;
//   - all loads of a group are issued before any arithmetic, so a lane has
//     R + 6 (fused) independent 16-byte requests in flight;
//   - R is a template parameter so the peer loop unrolls and the peer
//     pointers stay in scalar registers (passed by value in the kernel
//     arguments); no LDS is needed;
//   - grid-stride over 8-element groups with a grid sized from the CU count;
//     the n % 8 tail is done element-wise by the first block;
//   - binary32 arithmetic with no contraction (also compiled with
//     -ffp-contract=off): peer sums in ascending order seeded by peer 0,
//     correctly rounded sqrt and divide, so results match a scalar
//     one-rounding-per-operation evaluation bit for bit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <string>

#include "internal.h"

#pragma clang fp contract(off)

namespace {

constexpr int kBlock = 256;

struct Peers {
  const uint16_t* p[SBP_MAX_PEERS];
};

// Per-call AdamW scalars, each already rounded to binary32 on the host.
struct Scalars {
  float b1, b2, omb1, omb2, eps, step_size, c2, decay;
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

// Widen peer 0's 8 bf16 values and add peers 1..R-1 in ascending order.
template <int R>
__device__ __forceinline__ void peer_sum8(const uint4 (&w)[R], float (&S)[8]) {
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&w[0]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    S[2 * q] = bf16_lo(w0[q]);
    S[2 * q + 1] = bf16_hi(w0[q]);
  }
#pragma unroll
  for (int r = 1; r < R; ++r) {
    const uint32_t* wr = reinterpret_cast<const uint32_t*>(&w[r]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      S[2 * q] = S[2 * q] + bf16_lo(wr[q]);
      S[2 * q + 1] = S[2 * q + 1] + bf16_hi(wr[q]);
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
  const float4* q = reinterpret_cast<const float4*>(p) + 2 * gi;
  float4 a = q[0], b = q[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(float* p, int64_t gi, const float (&x)[8]) {
  float4* q = reinterpret_cast<float4*>(p) + 2 * gi;
  q[0] = make_float4(x[0], x[1], x[2], x[3]);
  q[1] = make_float4(x[4], x[5], x[6], x[7]);
}

template <int R>
__device__ __forceinline__ void load_peers(const Peers& P, int64_t gi, uint4 (&w)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) w[r] = reinterpret_cast<const uint4*>(P.p[r])[gi];
}

// ---- reduce: out = fl(S * scale) ------------------------------------------
template <int R>
__global__ void __launch_bounds__(kBlock)
reduce_kernel(Peers P, float scale, float* __restrict__ out, int64_t n) {
  const int64_t groups = n >> 3;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; gi < groups;
       gi += stride) {
    uint4 w[R];
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
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; gi < groups;
       gi += stride) {
    uint4 w[R];
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
template <int R, bool ACC>
__global__ void __launch_bounds__(kBlock)
fused_adamw_kernel(Peers P, const float* __restrict__ acc, float scale,
                   float* __restrict__ master, float* __restrict__ mom1,
                   float* __restrict__ mom2, uint16_t* __restrict__ pout, int64_t n,
                   Scalars s) {
  static_assert(R > 0 || ACC, "R == 0 needs the accumulator");
  const int64_t groups = n >> 3;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; gi < groups;
       gi += stride) {
    uint4 w[R > 0 ? R : 1];
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
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      adamw_one(G[j] * scale, th[j], m[j], v[j], s);
      pb[j] = bf16_rne(th[j]);
    }
    store8(master, gi, th);
    store8(mom1, gi, m);
    store8(mom2, gi, v);
    reinterpret_cast<uint4*>(pout)[gi] =
        make_uint4(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                   pb[6] | (pb[7] << 16));
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
      float th = master[i], m = mom1[i], v = mom2[i];
      adamw_one(G * scale, th, m, v, s);
      master[i] = th;
      mom1[i] = m;
      mom2[i] = v;
      pout[i] = static_cast<uint16_t>(bf16_rne(th));
    }
  }
}

// ---- launch helpers ---------------------------------------------------------

int cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Blocks for a grid-stride pass over `groups` 8-element groups.
unsigned grid_for(int64_t groups) {
  const int64_t want = (groups + kBlock - 1) / kBlock;
  const int64_t cap = static_cast<int64_t>(cu_count()) * 32;
  int64_t g = want < cap ? want : cap;
  return static_cast<unsigned>(g < 1 ? 1 : g);
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

// Host scalars of one AdamW step: float64 from the binary32 hyperparameters,
// each rounded once to binary32; beta^t by t multiplications.
Scalars adamw_scalars(const sbp_adamw_hparams& hp) {
  const double lr = hp.lr, b1 = hp.beta1, b2 = hp.beta2, wd = hp.weight_decay;
  double b1t = 1.0, b2t = 1.0;
  for (int64_t k = 0; k < hp.step; ++k) {
    b1t *= b1;
    b2t *= b2;
    if (b1t == 0.0 && b2t == 0.0) break;  // both powers have underflowed for good
  }
  const double bc1 = 1.0 - b1t, bc2 = 1.0 - b2t;
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

}  // namespace

extern "C" {

sbp_status sbp_reduce_shard(const void* const* peers, int32_t R, int64_t n, float scale,
                            float* out, hipStream_t stream) {
  const char* who = "sbp_reduce_shard";
  if (R < 1 || R > SBP_MAX_PEERS) return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: R must be in 1..16");
  if (n < 0) return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: n < 0");
  if (n == 0) return sbp::ok();  // nothing is read or written
  Peers P;
  sbp_status st = collect_peers(who, peers, R, P);
  if (st != SBP_OK) return st;
  if (out == nullptr) return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: out is null");
  if (!sbp::aligned(out, 16)) return sbp::fail(SBP_EALIGN, "sbp_reduce_shard: out not 16-B aligned");
  if (n > INT64_MAX / 4) return sbp::fail(SBP_ERANGE, "sbp_reduce_shard: n too large");
  for (int32_t r = 0; r < R; ++r)
    if (sbp::overlaps(out, 4 * n, peers[r], 2 * n))
      return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: out overlaps a peer");
  (void)hipGetLastError();
  return dispatch_r(R, [&](auto rc) -> sbp_status {
    constexpr int RR = decltype(rc)::value;
    if constexpr (RR == 0) {
      return sbp::fail(SBP_EINVAL, "sbp_reduce_shard: R must be >= 1");
    } else {
      hipLaunchKernelGGL(reduce_kernel<RR>, dim3(grid_for(n >> 3)), dim3(kBlock), 0, stream, P,
                         scale, out, n);
      return launched(who);
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
  if (n > INT64_MAX / 4) return sbp::fail(SBP_ERANGE, "sbp_accumulate_grads: n too large");
  for (int32_t r = 0; r < R; ++r)
    if (sbp::overlaps(acc, 4 * n, peers[r], 2 * n))
      return sbp::fail(SBP_EINVAL, "sbp_accumulate_grads: acc overlaps a peer");
  (void)hipGetLastError();
  return dispatch_r(R, [&](auto rc) -> sbp_status {
    constexpr int RR = decltype(rc)::value;
    if constexpr (RR == 0) {
      return sbp::fail(SBP_EINVAL, "sbp_accumulate_grads: R must be >= 1");
    } else {
      if (first)
        hipLaunchKernelGGL((accumulate_kernel<RR, true>), dim3(grid_for(n >> 3)), dim3(kBlock), 0,
                           stream, P, acc, n);
      else
        hipLaunchKernelGGL((accumulate_kernel<RR, false>), dim3(grid_for(n >> 3)), dim3(kBlock),
                           0, stream, P, acc, n);
      return launched(who);
    }
  });
}

sbp_status sbp_adamw_shard(const void* const* peers, int32_t R, const float* acc, float scale,
                           float* master, float* m, float* v, void* param_out, int64_t n,
                           const sbp_adamw_hparams* hp, hipStream_t stream) {
  const char* who = "sbp_adamw_shard";
  if (R < 0 || R > SBP_MAX_PEERS)
    return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: R must be in 0..16");
  if (n < 0) return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: n < 0");
  if (hp == nullptr) return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: hp is null");
  if (hp->step < 1) return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: step must be >= 1");
  if (n == 0) return sbp::ok();  // nothing is read or written
  Peers P;
  sbp_status st = collect_peers(who, peers, R, P);
  if (st != SBP_OK) return st;
  if (R == 0 && acc == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: R == 0 needs an accumulator");
  if (master == nullptr || m == nullptr || v == nullptr || param_out == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: null state or output pointer");
  const void* dev[5] = {acc, master, m, v, param_out};
  for (const void* p : dev)
    if (p != nullptr && !sbp::aligned(p, 16))
      return sbp::fail(SBP_EALIGN, "sbp_adamw_shard: device pointers must be 16-byte aligned");
  if (n > INT64_MAX / 4) return sbp::fail(SBP_ERANGE, "sbp_adamw_shard: n too large");
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
        return sbp::fail(SBP_EINVAL, "sbp_adamw_shard: buffers overlap");
  const Scalars s = adamw_scalars(*hp);
  uint16_t* pout = static_cast<uint16_t*>(param_out);
  (void)hipGetLastError();
  const unsigned grid = grid_for(n >> 3);
  return dispatch_r(R, [&](auto rc) -> sbp_status {
    constexpr int RR = decltype(rc)::value;
    if constexpr (RR == 0) {
      hipLaunchKernelGGL((fused_adamw_kernel<0, true>), dim3(grid), dim3(kBlock), 0, stream, P,
                         acc, scale, master, m, v, pout, n, s);
    } else {
      if (acc)
        hipLaunchKernelGGL((fused_adamw_kernel<RR, true>), dim3(grid), dim3(kBlock), 0, stream,
                           P, acc, scale, master, m, v, pout, n, s);
      else
        hipLaunchKernelGGL((fused_adamw_kernel<RR, false>), dim3(grid), dim3(kBlock), 0, stream,
                           P, acc, scale, master, m, v, pout, n, s);
    }
    return launched(who);
  });
}

}  // extern "C"
