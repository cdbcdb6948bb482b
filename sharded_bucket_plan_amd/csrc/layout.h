// Copy segments of the layout calls, shared by the host builders
// (layout_host.cpp) and the copy kernel (layout.hip).
#pragma once

#include <stdint.h>

#include <vector>

#include "internal.h"

namespace sbp {

// `len` bf16 elements from src to dst; a null src writes +0.
struct Seg {
  const uint16_t* src;
  uint16_t* dst;
  int64_t len;  // elements
};

// Validate one layout call's arguments and list its copies in `segs`
// (cleared first).  On error `segs` stays empty and the status is returned
// with the message set, exactly as the C entry points report it.
sbp_status pack_segments(const sbp_plan* plan, int32_t bucket, const void* const* tensor_grads,
                         void* flat, std::vector<Seg>& segs);
sbp_status unpack_segments(const sbp_plan* plan, int32_t bucket, const void* flat,
                           void* const* tensor_params, std::vector<Seg>& segs);
sbp_status shard_of_segments(const sbp_plan* plan, int32_t bucket, int32_t rank, const void* flat,
                             void* shard, std::vector<Seg>& segs);
sbp_status gather_segments(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                           void* flat, std::vector<Seg>& segs);
sbp_status unpack_shards_segments(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                                  void* const* tensor_params, std::vector<Seg>& segs);

// The all-gather side reads across the N shards.  A fan is `len` consecutive
// positions of one bucket from position x0, written to dst[0, len): position
// x lies in the chunk of rank x / chunk, which that rank's shard holds at
// shard_off + x % chunk.  One fan covers what would be one segment per rank.
struct Fan {
  int64_t shard_off;  // the bucket's offset in every shard
  int64_t chunk;      // the bucket's per-rank chunk (> 0)
  int64_t x0;         // first position in the bucket
  int64_t len;        // positions (> 0)
  uint16_t* dst;
};

// Fan lists of sbp_gather_shards and sbp_unpack_shards, validated exactly as
// the segment builders above, which are these fans cut into segments.
sbp_status gather_fans(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                       void* flat, std::vector<Fan>& fans);
sbp_status unpack_shards_fans(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                              void* const* tensor_params, std::vector<Fan>& fans);
// Each fan as plain segments, cut where rank chunks meet (appended to segs).
void fans_to_segments(const std::vector<Fan>& fans, const void* const* shards,
                      std::vector<Seg>& segs);

// A fan as the fan copy kernel takes it: at most kFanPiece positions, 32-bit
// fields, its first element's rank s0 and chunk position j0 worked out.  For
// the element at offset o the kernel takes t = j0 + o (unsigned 32-bit: below
// 2^31 + 2^30), rank s0 + t / chunk, shard position shard_off + t % chunk.
constexpr int32_t kMaxFanRanks = 64;             // shard pointers in the kernel arguments
constexpr int64_t kFanPiece = int64_t{1} << 30;  // longer fans are cut
struct FanPiece {
  uint16_t* dst;
  int64_t shard_off;
  int32_t len;          // elements, 1..kFanPiece
  int32_t chunk;        // 1..INT32_MAX
  int32_t s0, j0;
  int32_t first_chunk;  // set by the launcher: the piece's first block in its launch
  int32_t vec;          // 1: dst 16-byte aligned and shard_off, chunk, j0 multiples of 8
};
// Cuts the fans into pieces (pieces cleared first).  False, with no pieces,
// when world_n exceeds kMaxFanRanks or a chunk exceeds INT32_MAX: the caller
// then copies the fans as segments.
bool fan_pieces(const std::vector<Fan>& fans, int32_t world_n, std::vector<FanPiece>& pieces);

}  // namespace sbp
