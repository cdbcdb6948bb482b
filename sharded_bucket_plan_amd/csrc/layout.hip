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
//     destination are 16-byte aligned; otherwise the destination's unaligned
//     head and tail go element by element and the body in aligned 16-byte
//     stores, its source read as aligned words and realigned in registers
//     (a tensor at an odd element offset, as align = 1 and split plans make,
//     or a view into a larger buffer).
// gather and unpack_shards read across the N shards, which as segments is one
// per rank for every bucket or tensor piece (GPT-2 small under the per-tensor
// plan: 1,184 segments, eight launches).  They go out as fans instead: the N
// shard pointers once in the arguments, then one 40-byte piece per bucket or
// tensor piece naming the bucket positions it covers.  A block whose 2048
// elements lie in one rank's chunk (every block, when chunks are long) copies
// as above; otherwise each lane finds its rank from its own position.
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

// 16 bytes of a byte stream that starts `sh` bytes (even, 2..14) into the
// aligned word a, continuing into the aligned word b: v_alignbyte takes 4
// bytes at a byte offset out of two concatenated dwords.  sh is uniform
// across the block, so the switch does not diverge.
__device__ __forceinline__ uint4 realign16(uint4 a, uint4 b, uint32_t sh) {
  const uint32_t r = sh & 3;  // 0 or 2: bytes into the dword
  uint32_t D[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  switch (sh >> 2) {
    case 0:
      return make_uint4(__builtin_amdgcn_alignbyte(D[1], D[0], r),
                        __builtin_amdgcn_alignbyte(D[2], D[1], r),
                        __builtin_amdgcn_alignbyte(D[3], D[2], r),
                        __builtin_amdgcn_alignbyte(D[4], D[3], r));
    case 1:
      return make_uint4(__builtin_amdgcn_alignbyte(D[2], D[1], r),
                        __builtin_amdgcn_alignbyte(D[3], D[2], r),
                        __builtin_amdgcn_alignbyte(D[4], D[3], r),
                        __builtin_amdgcn_alignbyte(D[5], D[4], r));
    case 2:
      return make_uint4(__builtin_amdgcn_alignbyte(D[3], D[2], r),
                        __builtin_amdgcn_alignbyte(D[4], D[3], r),
                        __builtin_amdgcn_alignbyte(D[5], D[4], r),
                        __builtin_amdgcn_alignbyte(D[6], D[5], r));
    default:
      return make_uint4(__builtin_amdgcn_alignbyte(D[4], D[3], r),
                        __builtin_amdgcn_alignbyte(D[5], D[4], r),
                        __builtin_amdgcn_alignbyte(D[6], D[5], r),
                        __builtin_amdgcn_alignbyte(D[7], D[6], r));
  }
}

// `cnt` (at most kChunk) elements from s (null: +0) to d, by one block.
// Both 16-byte aligned: 16-byte loads and stores.  Otherwise the elements
// before d's first 16-byte boundary and after its last are copied one by
// one, and the body between goes out in aligned 16-byte stores; its source,
// `sh` bytes past a 16-byte boundary, is read as whole aligned 16-byte words
// and realigned in registers.  The last word read ends inside the aligned
// 16 bytes that hold the body's last source byte, so it never touches a page
// the source does not.
__device__ __forceinline__ void copy_chunk(uint16_t* d, const uint16_t* s, int64_t cnt) {
  const uint32_t dmis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(d) & 15);
  const uint32_t smis = s ? static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s) & 15) : 0;
  const int t = threadIdx.x;
  if (dmis == 0 && smis == 0) {
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const int64_t e = static_cast<int64_t>(k) * kBlock * 8 + t * 8;
      if (e + 8 <= cnt) {
        uint4 x = s ? *reinterpret_cast<const uint4*>(s + e) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(d + e) = x;
      } else {
        for (int64_t j = e; j < cnt; ++j) d[j] = s ? s[j] : 0;
      }
    }
    return;
  }
  // every load of the lane (its head element, body words and tail element)
  // goes out before any store: one memory round trip per block
  const int64_t head0 = static_cast<int64_t>(((16 - dmis) & 15) >> 1);
  const int64_t head = head0 < cnt ? head0 : cnt;
  const int64_t words = (cnt - head) >> 3;  // at most kRounds * kBlock
  const int64_t tail0 = head + (words << 3);
  const bool in_head = t < head, in_tail = tail0 + t < cnt;
  uint16_t hv = 0, tv = 0;
  uint4 x[kRounds];
  uint4* db = reinterpret_cast<uint4*>(d + head);
  if (s == nullptr) {
#pragma unroll
    for (int k = 0; k < kRounds; ++k) x[k] = make_uint4(0, 0, 0, 0);
  } else {
    if (in_head) hv = s[t];
    if (in_tail) tv = s[tail0 + t];
    const uintptr_t sb = reinterpret_cast<uintptr_t>(s + head);
    const uint32_t sh = static_cast<uint32_t>(sb & 15);
    const uint4* sa = reinterpret_cast<const uint4*>(sb - sh);
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const int64_t w = t + static_cast<int64_t>(k) * kBlock;
      if (w < words) x[k] = sh == 0 ? sa[w] : realign16(sa[w], sa[w + 1], sh);
    }
  }
  if (in_head) d[t] = hv;
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    const int64_t w = t + static_cast<int64_t>(k) * kBlock;
    if (w < words) db[w] = x[k];
  }
  if (in_tail) d[tail0 + t] = tv;
}

// Block ci of a segment of `len` elements whose destination is not 16-byte
// aligned (or whose source is not): the destination's aligned 16-byte words
// are numbered from its first 16-byte boundary, and block ci writes words
// [ci * W, (ci + 1) * W), W = kRounds * kBlock, so every word is written
// whole by one block; the elements before the first boundary (block 0) and
// after the last whole word (the last block) go one by one.  No word is left
// half-written by two blocks at every chunk boundary, as cutting at element
// chunks would.  Sources as in copy_chunk (aligned words, realigned).
__device__ __forceinline__ void copy_words(uint16_t* d, const uint16_t* s, int64_t len,
                                           int64_t ci) {
  constexpr int64_t W = static_cast<int64_t>(kRounds) * kBlock;
  const int t = threadIdx.x;
  const uint32_t dmis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(d) & 15);
  const int64_t head0 = static_cast<int64_t>(((16 - dmis) & 15) >> 1);
  const int64_t head = head0 < len ? head0 : len;
  const int64_t words = (len - head) >> 3;
  const int64_t tail0 = head + (words << 3);
  const int64_t last_ci = (len - 1) / kChunk;
  const bool in_head = ci == 0 && t < head;
  const bool in_tail = ci == last_ci && tail0 + t < len;
  uint16_t hv = 0, tv = 0;
  uint4 x[kRounds];
  uint4* db = reinterpret_cast<uint4*>(d + head);
  if (s == nullptr) {
#pragma unroll
    for (int k = 0; k < kRounds; ++k) x[k] = make_uint4(0, 0, 0, 0);
  } else {
    if (in_head) hv = s[t];
    if (in_tail) tv = s[tail0 + t];
    const uintptr_t sb = reinterpret_cast<uintptr_t>(s + head);
    const uint32_t sh = static_cast<uint32_t>(sb & 15);
    const uint4* sa = reinterpret_cast<const uint4*>(sb - sh);
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const int64_t w = ci * W + t + static_cast<int64_t>(k) * kBlock;
      if (w < words) x[k] = sh == 0 ? sa[w] : realign16(sa[w], sa[w + 1], sh);
    }
  }
  if (in_head) d[t] = hv;
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    const int64_t w = ci * W + t + static_cast<int64_t>(k) * kBlock;
    if (w < words) db[w] = x[k];
  }
  if (in_tail) d[tail0 + t] = tv;
}

__global__ void __launch_bounds__(kBlock) copy_kernel(SegList L) {
  // one block per chunk (gridDim.x == L.chunks), XCD-contiguous order
  unsigned b = blockIdx.x;
  const unsigned per = gridDim.x / kXcds;
  if (b < per * kXcds) b = (b % kXcds) * per + b / kXcds;
  const int64_t c = b;
  const DevSeg sg = L.seg[find_seg(L, c)];
  const int64_t ci = c - sg.first_chunk;
  const bool aligned = (reinterpret_cast<uintptr_t>(sg.dst) & 15) == 0 &&
                       (sg.src == nullptr || (reinterpret_cast<uintptr_t>(sg.src) & 15) == 0);
  if (!aligned) {
    copy_words(sg.dst, sg.src, sg.len, ci);
    return;
  }
  const int64_t start = ci * kChunk;
  const int64_t rem = static_cast<int64_t>(sg.len) - start;
  const int64_t cnt = rem < kChunk ? rem : kChunk;
  copy_chunk(sg.dst + start, sg.src ? sg.src + start : nullptr, cnt);
}

// Fans (the all-gather side): the shard pointers once, then up to kMaxFans
// pieces, within the argument size the segment list above already uses.
constexpr int kMaxFans = 83;
using sbp::FanPiece;
using sbp::kMaxFanRanks;

struct FanList {
  const uint16_t* shard[kMaxFanRanks];
  FanPiece fan[kMaxFans];
  int32_t count;
  int32_t chunks;  // total chunks of this launch
};
static_assert(sizeof(FanPiece) == 40, "a fan piece is 40 bytes");
static_assert(sizeof(FanList) <= sizeof(SegList), "fans take no more argument space than segments");
static_assert(sbp::kFanPiece % kChunk == 0, "pieces are whole chunks");
static_assert(sbp::kFanPiece / kChunk <= kMaxLaunchChunks, "a piece fits one launch");

__device__ __forceinline__ int find_fan(const FanList& L, int64_t c) {
  int lo = 0, hi = L.count - 1;  // last piece whose first_chunk <= c
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (L.fan[mid].first_chunk <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Block ci of a fan piece whose destination is not 16-byte aligned: as
// copy_words, the destination's whole 16-byte words by word index, each
// word's 8 sources found from its position -- one shard's contiguous run
// (aligned words, realigned) unless a rank boundary falls inside the word,
// which then goes element by element, like the piece's unaligned ends.
__device__ __forceinline__ void fan_words(const FanList& L, const FanPiece& f, uint32_t ci) {
  constexpr uint32_t W = static_cast<uint32_t>(kRounds) * kBlock;
  const uint32_t t = threadIdx.x;
  const uint32_t len = static_cast<uint32_t>(f.len), chunk = static_cast<uint32_t>(f.chunk);
  const uint32_t j0 = static_cast<uint32_t>(f.j0);
  auto src = [&](uint32_t o) {
    const uint32_t x = j0 + o;
    const uint32_t q = x / chunk;
    return L.shard[f.s0 + static_cast<int32_t>(q)] + f.shard_off + (x - q * chunk);
  };
  const uint32_t dmis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(f.dst) & 15);
  const uint32_t head0 = ((16 - dmis) & 15) >> 1;
  const uint32_t head = head0 < len ? head0 : len;
  const uint32_t words = (len - head) >> 3;
  const uint32_t tail0 = head + (words << 3);
  const uint32_t last_ci = (len - 1) / static_cast<uint32_t>(kChunk);
  const bool in_head = ci == 0 && t < head;
  const bool in_tail = ci == last_ci && tail0 + t < len;
  const uint16_t hv = in_head ? *src(t) : 0;
  const uint16_t tv = in_tail ? *src(tail0 + t) : 0;
  uint4 x[kRounds];
  // the block's words [w_lo, w_hi): when they all lie in one rank's chunk
  // (every block but those at a rank boundary) the shard pointer and the
  // source's misalignment are block-uniform
  const uint32_t w_lo = ci * W;
  const uint32_t w_hi = words < w_lo + W ? words : w_lo + W;
  uint32_t q_lo = 0, q_hi = 1;
  if (w_lo < w_hi) {
    q_lo = (j0 + head + (w_lo << 3)) / chunk;
    q_hi = (j0 + head + ((w_hi - 1) << 3) + 7) / chunk;
  }
  if (q_lo == q_hi) {
    const uint32_t off_lo = j0 + head + (w_lo << 3) - q_lo * chunk;
    const uintptr_t p_lo = reinterpret_cast<uintptr_t>(
        L.shard[f.s0 + static_cast<int32_t>(q_lo)] + f.shard_off + off_lo);
    const uint32_t sh = static_cast<uint32_t>(p_lo & 15);
    const uint4* sa = reinterpret_cast<const uint4*>(p_lo - sh);  // word w: sa[w - w_lo]
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const uint32_t i = t + static_cast<uint32_t>(k) * kBlock;
      if (w_lo + i < w_hi) x[k] = sh == 0 ? sa[i] : realign16(sa[i], sa[i + 1], sh);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const uint32_t w = ci * W + t + static_cast<uint32_t>(k) * kBlock;
      if (w >= words) continue;
      const uint32_t o0 = head + (w << 3);
      const uint32_t x0 = j0 + o0;
      if (x0 / chunk == (x0 + 7) / chunk) {
        const uintptr_t p = reinterpret_cast<uintptr_t>(src(o0));
        const uint32_t sh = static_cast<uint32_t>(p & 15);
        const uint4* sa = reinterpret_cast<const uint4*>(p - sh);
        x[k] = sh == 0 ? sa[0] : realign16(sa[0], sa[1], sh);
      } else {
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = static_cast<uint32_t>(*src(o0 + 2 * e)) |
                 (static_cast<uint32_t>(*src(o0 + 2 * e + 1)) << 16);
        x[k] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  }
  uint16_t* d = f.dst;
  uint4* db = reinterpret_cast<uint4*>(d + head);
  if (in_head) d[t] = hv;
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    const uint32_t w = ci * W + t + static_cast<uint32_t>(k) * kBlock;
    if (w < words) db[w] = x[k];
  }
  if (in_tail) d[tail0 + t] = tv;
}

__global__ void __launch_bounds__(kBlock) fan_copy_kernel(FanList L) {
  // one block per chunk (gridDim.x == L.chunks), XCD-contiguous order
  unsigned b = blockIdx.x;
  const unsigned per = gridDim.x / kXcds;
  if (b < per * kXcds) b = (b % kXcds) * per + b / kXcds;
  const int64_t c = b;
  const FanPiece f = L.fan[find_fan(L, c)];
  if ((reinterpret_cast<uintptr_t>(f.dst) & 15) != 0) {
    fan_words(L, f, static_cast<uint32_t>(c - f.first_chunk));
    return;
  }
  const uint32_t start = static_cast<uint32_t>(c - f.first_chunk) * static_cast<uint32_t>(kChunk);
  const uint32_t rem = static_cast<uint32_t>(f.len) - start;
  const uint32_t cnt = rem < static_cast<uint32_t>(kChunk) ? rem : static_cast<uint32_t>(kChunk);
  uint16_t* d = f.dst + start;
  // offset o of the piece: position t = j0 + o past the start of rank s0's chunk
  const uint32_t base = static_cast<uint32_t>(f.j0) + start;
  const uint32_t chunk = static_cast<uint32_t>(f.chunk);
  const uint32_t q0 = base / chunk;
  if ((base + cnt - 1) / chunk == q0) {
    // the block's elements lie in one rank's chunk (every block, when chunks
    // are long): one shard pointer for the block, a plain copy
    const uint16_t* s = L.shard[f.s0 + static_cast<int32_t>(q0)] + f.shard_off + (base - q0 * chunk);
    copy_chunk(d, s, cnt);
    return;
  }
  auto src = [&](uint32_t o) {
    const uint32_t t = base + o;
    const uint32_t q = t / chunk;
    return L.shard[f.s0 + static_cast<int32_t>(q)] + f.shard_off + (t - q * chunk);
  };
  if (f.vec) {
    // j0, chunk and the start are multiples of 8: a lane's 8 elements lie in one rank's chunk
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const uint32_t e = static_cast<uint32_t>(k * kBlock * 8) + threadIdx.x * 8;
      if (e + 8 <= cnt) {
        *reinterpret_cast<uint4*>(d + e) = *reinterpret_cast<const uint4*>(src(e));
      } else {
        for (uint32_t j = e; j < cnt; ++j) d[j] = *src(j);
      }
    }
  } else {
    for (uint32_t j = threadIdx.x; j < cnt; j += kBlock) d[j] = *src(j);
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

// The fans in as few launches as their pieces allow, or, when they cannot be
// expressed as pieces, as plain segments.
sbp_status launch_fans(const char* who, const sbp_plan* plan, const void* const* shards,
                       const std::vector<sbp::Fan>& fans, hipStream_t stream) {
  std::vector<FanPiece> pieces;
  std::vector<Seg> segs;
  try {
    if (!sbp::fan_pieces(fans, plan->world_n, pieces)) {
      sbp::fans_to_segments(fans, shards, segs);
      return launch_segments(who, segs, stream);
    }
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, std::string(who) + ": out of host memory");
  }
  (void)hipGetLastError();
  FanList L;
  for (int32_t r = 0; r < kMaxFanRanks; ++r)
    L.shard[r] = r < plan->world_n ? static_cast<const uint16_t*>(shards[r]) : nullptr;
  L.count = 0;
  L.chunks = 0;
  auto flush = [&]() -> sbp_status {
    if (L.count == 0) return SBP_OK;
    hipLaunchKernelGGL(fan_copy_kernel, dim3(static_cast<unsigned>(L.chunks)), dim3(kBlock), 0,
                       stream, L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return sbp::fail(SBP_EHIP, std::string(who) + ": launch failed: " + hipGetErrorString(e));
    L.count = 0;
    L.chunks = 0;
    return SBP_OK;
  };
  for (FanPiece p : pieces) {
    const int64_t ch = (p.len + kChunk - 1) / kChunk;
    if (L.count == kMaxFans || L.chunks + ch > kMaxLaunchChunks) {
      sbp_status st = flush();
      if (st != SBP_OK) return st;
    }
    p.first_chunk = L.chunks;
    L.fan[L.count++] = p;
    L.chunks += static_cast<int32_t>(ch);
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
  std::vector<sbp::Fan> fans;
  sbp_status st = sbp::gather_fans(plan, bucket, shards, flat, fans);
  return st != SBP_OK ? st : launch_fans("sbp_gather_shards", plan, shards, fans, stream);
}

sbp_status sbp_unpack_shards(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                             void* const* tensor_params, hipStream_t stream) {
  std::vector<sbp::Fan> fans;
  sbp_status st = sbp::unpack_shards_fans(plan, bucket, shards, tensor_params, fans);
  return st != SBP_OK ? st : launch_fans("sbp_unpack_shards", plan, shards, fans, stream);
}

}  // extern "C"
