// Internal declarations shared by the library's translation units.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "sbp.h"

namespace sbp {

// Records `msg` as this thread's last error and returns `code`.
sbp_status fail(sbp_status code, const std::string& msg);
// Clears this thread's last error and returns SBP_OK.
sbp_status ok();

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// [a, a+na) and [b, b+nb) overlap (byte ranges; empty ranges never do).
inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (na <= 0 || nb <= 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + static_cast<uintptr_t>(nb) && b0 < a0 + static_cast<uintptr_t>(na);
}

// Host-side plan (the opaque sbp_plan).
struct Bucket {
  std::vector<int32_t> tensors;  // in placement order
  int64_t used, padded, chunk, shard_offset, flat_offset;
};

}  // namespace sbp

struct sbp_plan;

namespace sbp {
// plan.cpp: fixed-size split plan, and the per-tensor flat positions.
sbp_status split_plan(sbp_plan* p, int64_t cap_bytes, bool reverse);
void finish_flat_positions(sbp_plan* p);
}  // namespace sbp

struct sbp_plan {
  std::vector<int64_t> numel;
  std::vector<int32_t> tensor_bucket;  // bucket of the tensor's first element
  std::vector<int64_t> tensor_offset;  // offset of that element in the bucket
  std::vector<int64_t> tensor_flat;    // position of the tensor in the flat buffer
  std::vector<int32_t> flat_order;     // non-empty tensors by flat position
  std::vector<sbp::Bucket> buckets;
  int32_t world_n;
  int32_t align;
  bool split;                          // fixed-size buckets, tensors may straddle
  int64_t shard_numel;
  int64_t flat_numel;
};
