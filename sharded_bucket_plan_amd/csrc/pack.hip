// Multi-tensor pack of per-parameter bf16 gradients into flat buckets
// ("Parallelisms" (vladislavkruglikov.com), Gradient bucketing: gradients
// gathered into buffers at fixed offsets; FSDP / Flat parameter: one
// contiguous buffer concatenating parameters; YaFSDP writes gradients
// straight into the communication buffers, which is what the bucket here
// is: a persistent, caller-owned buffer written in place).
//
// Design (CDNA4).  A bucket mixes 4096-element norm vectors with matrices
// of half a billion elements, so work is cut into equal chunks of
// 2048 * kRounds elements, not per tensor:
//   - the host lists the bucket(s) as segments -- a tensor copy, or a run of
//     zero padding -- each with the index of its first chunk; up to
//     kMaxSegs segments travel by value in the kernel arguments (no device
//     allocation, nothing to upload), longer lists take several launches;
//   - one pass: one block per chunk, in XCD-contiguous order (as the
//     streaming kernels), and it finds its segment by binary search over
//     the chunk starts (uniform per block, so it runs on scalar loads of the
//     kernel arguments);
//   - a chunk is kRounds rounds of 256 lanes x 16 bytes: fully coalesced
//     16-byte loads and stores when the source is 16-byte aligned and the
//     destination offset a multiple of 8 elements; otherwise element-wise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "internal.h"

namespace {

#ifndef SBP_PACK_ROUNDS
#define SBP_PACK_ROUNDS 1
#endif

constexpr int kBlock = 256;
constexpr int kRounds = SBP_PACK_ROUNDS;
constexpr int kXcds = 8;
constexpr int64_t kChunk = static_cast<int64_t>(kBlock) * 8 * kRounds;  // elements
constexpr int kMaxSegs = 96;

struct Seg {
  const uint16_t* src;  // null: zero fill
  int64_t dst;          // element offset in the flat buffer
  int64_t len;          // elements
  int64_t first_chunk;  // chunk index (within this launch) of the segment's start
};

struct SegList {
  Seg seg[kMaxSegs];
  int32_t count;
  int64_t chunks;  // total chunks of this launch
};

__device__ __forceinline__ int find_seg(const SegList& L, int64_t c) {
  int lo = 0, hi = L.count - 1;  // last segment whose first_chunk <= c
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (L.seg[mid].first_chunk <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kBlock) pack_kernel(SegList L, uint16_t* __restrict__ flat) {
  // one block per chunk (gridDim.x == L.chunks), XCD-contiguous order
  unsigned b = blockIdx.x;
  const unsigned per = gridDim.x / kXcds;
  if (b < per * kXcds) b = (b % kXcds) * per + b / kXcds;
  {
    const int64_t c = b;
    const Seg sg = L.seg[find_seg(L, c)];
    const int64_t start = (c - sg.first_chunk) * kChunk;
    const int64_t rem = sg.len - start;
    const int64_t cnt = rem < kChunk ? rem : kChunk;
    uint16_t* d = flat + sg.dst + start;
    const uint16_t* s = sg.src ? sg.src + start : nullptr;
    const bool vec = ((sg.dst & 7) == 0) &&
                     (s == nullptr || (reinterpret_cast<uintptr_t>(sg.src) & 15) == 0);
    if (vec) {
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
        const int64_t e = static_cast<int64_t>(k) * kBlock * 8 + threadIdx.x * 8;
        if (e + 8 <= cnt) {
          uint4 x = s ? *reinterpret_cast<const uint4*>(s + e) : make_uint4(0, 0, 0, 0);
          *reinterpret_cast<uint4*>(d + e) = x;
        } else {
          for (int64_t j = e; j < cnt; ++j) d[j] = s ? s[j] : 0;
        }
      }
    } else {
      for (int64_t j = threadIdx.x; j < cnt; j += kBlock) d[j] = s ? s[j] : 0;
    }
  }
}

}  // namespace

extern "C" sbp_status sbp_pack_grads(const sbp_plan* plan, int32_t bucket,
                                     const void* const* tensor_grads, void* flat,
                                     hipStream_t stream) {
  if (plan == nullptr) return sbp::fail(SBP_EINVAL, "sbp_pack_grads: plan is null");
  if (tensor_grads == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_pack_grads: tensor_grads is null");
  if (flat == nullptr) return sbp::fail(SBP_EINVAL, "sbp_pack_grads: flat is null");
  if (!sbp::aligned(flat, 16))
    return sbp::fail(SBP_EALIGN, "sbp_pack_grads: flat must be 16-byte aligned");
  const int32_t nb = static_cast<int32_t>(plan->buckets.size());
  if (bucket < -1 || bucket >= nb)
    return sbp::fail(SBP_EINVAL, "sbp_pack_grads: bucket out of range");
  const int32_t b0 = bucket < 0 ? 0 : bucket, b1 = bucket < 0 ? nb : bucket + 1;

  // segments in flat order: each tensor, and the zero runs around them
  std::vector<Seg> segs;
  try {
    for (int32_t b = b0; b < b1; ++b) {
      const sbp::Bucket& k = plan->buckets[b];
      // tensors were placed at increasing offsets in visit order
      int64_t pos = 0;
      for (int32_t t : k.tensors) {
        const int64_t off = plan->tensor_offset[t], len = plan->numel[t];
        if (len == 0) continue;
        const void* src = tensor_grads[t];
        if (src == nullptr)
          return sbp::fail(SBP_EINVAL, "sbp_pack_grads: gradient pointer of a tensor is null");
        if (!sbp::aligned(src, 2))
          return sbp::fail(SBP_EALIGN, "sbp_pack_grads: gradients must be 2-byte aligned");
        if (sbp::overlaps(src, 2 * len, flat, 2 * plan->flat_numel))
          return sbp::fail(SBP_EINVAL, "sbp_pack_grads: a gradient overlaps the flat buffer");
        if (off > pos) segs.push_back(Seg{nullptr, k.flat_offset + pos, off - pos, 0});
        segs.push_back(Seg{static_cast<const uint16_t*>(src), k.flat_offset + off, len, 0});
        pos = off + len;
      }
      if (k.padded > pos) segs.push_back(Seg{nullptr, k.flat_offset + pos, k.padded - pos, 0});
    }
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, "sbp_pack_grads: out of host memory");
  }

  (void)hipGetLastError();
  for (size_t i = 0; i < segs.size(); i += kMaxSegs) {
    SegList L;
    L.count = 0;
    L.chunks = 0;
    for (size_t j = i; j < segs.size() && j < i + kMaxSegs; ++j) {
      Seg s = segs[j];
      s.first_chunk = L.chunks;
      L.chunks += (s.len + kChunk - 1) / kChunk;
      L.seg[L.count++] = s;
    }
    if (L.chunks > 0x7FFFFFFF)
      return sbp::fail(SBP_ERANGE, "sbp_pack_grads: too many chunks for one launch");
    hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(L.chunks)), dim3(kBlock), 0, stream,
                       L, static_cast<uint16_t*>(flat));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return sbp::fail(SBP_EHIP, std::string("sbp_pack_grads: launch failed: ") +
                                     hipGetErrorString(e));
  }
  return sbp::ok();
}
