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

}  // namespace sbp
