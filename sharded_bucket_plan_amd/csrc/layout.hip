// Layout moves between per-tensor buffers, flat buckets and shards:
//   pack    per-tensor bf16 gradients -> flat buckets (+0 elsewhere)
//   unpack  flat buckets -> per-tensor bf16 parameters (the all-gather side)
//   shard_of  one rank's chunk of every bucket -> its shard layout (what that
//             rank contributes to each owner in the reduce-scatter)
//   gather    the N ranks' shards -> flat buckets (what the all-gather
//             assembles on every rank)
// ("Parallelisms" (vladislavkruglikov.com), Gradient bucketing: gradients
// gathered into buffers at fixed offsets; FSDP / Flat parameter: one
// contiguous buffer concatenating parameters, the originals being views into
// it; YaFSDP writes gradients straight into communication buffers, which is
// what the bucket here is: a persistent, caller-owned buffer written in place;
// ZeRO-1: reduce-scatter to owners, all-gather of the updated shards.)
//
// Design (CDNA4).  Every call is a list of copy segments (source, destination,
// length; a null source writes zeros), cut into equal chunks of 2048
// elements rather than per tensor, because a bucket mixes 4096-element norm
// vectors with matrices of half a billion elements:
//   - up to 160 segments (24 bytes each) travel by value in the kernel
//     arguments (no device allocation, nothing to upload, so the calls can be
//     captured in a graph); longer lists take several launches of 64;
//   - one pass: one block per chunk, in XCD-contiguous order (the order the
//     streaming kernels use); a block finds its segment by binary search over
//     the chunk starts, uniform per block, so it runs on scalar loads of the
//     kernel arguments;
//   - a chunk is 256 lanes x 16 bytes, fully coalesced, when source and
//     destination are 16-byte aligned; otherwise element by element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <string>
#include <utility>
#include <vector>

#include "internal.h"
#include "layout.h"

#ifndef SBP_PACK_ROUNDS
#define SBP_PACK_ROUNDS 1
#endif

namespace {

using sbp::Seg;

constexpr int kBlock = 256;
constexpr int kRounds = SBP_PACK_ROUNDS;
constexpr int kXcds = 8;
constexpr int64_t kChunk = static_cast<int64_t>(kBlock) * 8 * kRounds;  // elements
constexpr int kMaxSegs = 160;
// A list that does not fit one launch goes out in several.  A launch is cut
// at this many segments once it holds kBigLaunchChunks chunks: a shorter list
// per launch keeps each block's segment search shallow (measured: Llama-3-8B
// pack 79.2% of 8 TB/s with 64 per launch, 78.0% with 160).  A launch of
// small segments is filled up to kMaxSegs instead, since each launch's ramp
// and drain cost a few microseconds; likewise a list that fits one launch
// goes out in one (GPT-2-small pack: 70.3% in one launch against 65.8% in two).
constexpr int kSegsPerLaunchWhenSplit = 64;
constexpr int32_t kBigLaunchChunks = 1 << 15;  // 64M elements, ~40 us of copying
constexpr int64_t kMaxPiece = int64_t{1} << 30;  // longer segments are split (a multiple of kChunk)
// One block per chunk, and a launch holds at most 2^32 - 1 work-items.
constexpr int64_t kMaxLaunchChunks = (int64_t{1} << 32) / kBlock - 1;

// A copy segment as the kernel sees it: 24 bytes, so 160 fit in the kernel
// arguments (a 32-bit length; the host splits longer segments).
struct DevSeg {
  const uint16_t* src;  // null: +0
  uint16_t* dst;
  int32_t len;          // elements, at most kMaxPiece
  int32_t first_chunk;  // chunk index (within this launch) of the segment's start
};

struct SegList {
  DevSeg seg[kMaxSegs];
  int32_t count;
  int32_t chunks;  // total chunks of this launch
};
static_assert(sizeof(SegList) <= 4096, "the segment list must fit the kernel arguments");
static_assert(kMaxPiece % kChunk == 0, "pieces are whole chunks");
static_assert(kMaxPiece / kChunk <= kMaxLaunchChunks, "a piece fits one launch");

__device__ __forceinline__ int find_seg(const SegList& L, int64_t c) {
  int lo = 0, hi = L.count - 1;  // last segment whose first_chunk <= c
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (L.seg[mid].first_chunk <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kBlock) copy_kernel(SegList L) {
  // one block per chunk (gridDim.x == L.chunks), XCD-contiguous order
  unsigned b = blockIdx.x;
  const unsigned per = gridDim.x / kXcds;
  if (b < per * kXcds) b = (b % kXcds) * per + b / kXcds;
  const int64_t c = b;
  const DevSeg sg = L.seg[find_seg(L, c)];
  const int64_t start = (c - sg.first_chunk) * kChunk;
  const int64_t rem = static_cast<int64_t>(sg.len) - start;
  const int64_t cnt = rem < kChunk ? rem : kChunk;
  uint16_t* d = sg.dst + start;
  const uint16_t* s = sg.src ? sg.src + start : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(sg.dst) & 15) == 0 &&
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

sbp_status launch_segments(const char* who, const std::vector<Seg>& segs, hipStream_t stream) {
  (void)hipGetLastError();
  SegList L;
  L.count = 0;
  L.chunks = 0;
  auto flush = [&]() -> sbp_status {
    if (L.count == 0) return SBP_OK;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(L.chunks)), dim3(kBlock), 0,
                       stream, L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return sbp::fail(SBP_EHIP, std::string(who) + ": launch failed: " + hipGetErrorString(e));
    L.count = 0;
    L.chunks = 0;
    return SBP_OK;
  };
  int64_t pieces = 0;
  for (const Seg& s : segs) pieces += (s.len + kMaxPiece - 1) / kMaxPiece;
  const bool one_launch = pieces <= kMaxSegs;
  for (const Seg& s : segs) {
    for (int64_t off = 0; off < s.len; off += kMaxPiece) {
      const int64_t len = std::min(kMaxPiece, s.len - off);
      const int64_t ch = (len + kChunk - 1) / kChunk;
      const bool cut_early =
          !one_launch && L.count >= kSegsPerLaunchWhenSplit && L.chunks >= kBigLaunchChunks;
      if (L.count == kMaxSegs || cut_early || L.chunks + ch > kMaxLaunchChunks) {
        sbp_status st = flush();
        if (st != SBP_OK) return st;
      }
      L.seg[L.count++] = DevSeg{s.src ? s.src + off : nullptr, s.dst + off,
                                static_cast<int32_t>(len), L.chunks};
      L.chunks += static_cast<int32_t>(ch);
    }
  }
  sbp_status st = flush();
  return st != SBP_OK ? st : sbp::ok();
}

}  // namespace

extern "C" {

sbp_status sbp_pack_grads(const sbp_plan* plan, int32_t bucket, const void* const* tensor_grads,
                          void* flat, hipStream_t stream) {
  std::vector<Seg> segs;
  sbp_status st = sbp::pack_segments(plan, bucket, tensor_grads, flat, segs);
  return st != SBP_OK ? st : launch_segments("sbp_pack_grads", segs, stream);
}

sbp_status sbp_unpack_params(const sbp_plan* plan, int32_t bucket, const void* flat,
                             void* const* tensor_params, hipStream_t stream) {
  std::vector<Seg> segs;
  sbp_status st = sbp::unpack_segments(plan, bucket, flat, tensor_params, segs);
  return st != SBP_OK ? st : launch_segments("sbp_unpack_params", segs, stream);
}

sbp_status sbp_shard_of(const sbp_plan* plan, int32_t bucket, int32_t rank, const void* flat,
                        void* shard, hipStream_t stream) {
  std::vector<Seg> segs;
  sbp_status st = sbp::shard_of_segments(plan, bucket, rank, flat, shard, segs);
  return st != SBP_OK ? st : launch_segments("sbp_shard_of", segs, stream);
}

sbp_status sbp_gather_shards(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                             void* flat, hipStream_t stream) {
  std::vector<Seg> segs;
  sbp_status st = sbp::gather_segments(plan, bucket, shards, flat, segs);
  return st != SBP_OK ? st : launch_segments("sbp_gather_shards", segs, stream);
}

sbp_status sbp_unpack_shards(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                             void* const* tensor_params, hipStream_t stream) {
  std::vector<Seg> segs;
  sbp_status st = sbp::unpack_shards_segments(plan, bucket, shards, tensor_params, segs);
  return st != SBP_OK ? st : launch_segments("sbp_unpack_shards", segs, stream);
}

}  // extern "C"
