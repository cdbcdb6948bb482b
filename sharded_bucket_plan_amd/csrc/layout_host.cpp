// Host side of the layout calls: validation, the copy-segment lists the copy
// kernel executes, and the fan lists (with their kernel-argument pieces) of
// the calls that read across the N shards (layout.hip).  Pure host code, so
// it also builds with g++ for the sanitizer tests; the kernels trust these
// lists, so every segment and every fan must lie inside the buffers it names.
//
// Segments follow the plan ("Parallelisms", Gradient bucketing: gradients at
// fixed offsets in flat buffers; FSDP / Flat parameter: the originals are
// views into the flat buffer; ZeRO-1: rank s owns chunk s of every bucket).
#include <stdint.h>

#include <algorithm>
#include <string>
#include <utility>
#include <vector>

#include "internal.h"
#include "layout.h"

namespace sbp {

namespace {

// Flat range [lo, hi) of bucket `bucket` (-1: all buckets).
sbp_status bucket_range(const char* who, const sbp_plan* plan, int32_t bucket, int32_t* b0,
                        int32_t* b1, int64_t* lo, int64_t* hi) {
  const int32_t nb = static_cast<int32_t>(plan->buckets.size());
  if (bucket < -1 || bucket >= nb)
    return sbp::fail(SBP_EINVAL, std::string(who) + ": bucket out of range");
  *b0 = bucket < 0 ? 0 : bucket;
  *b1 = bucket < 0 ? nb : bucket + 1;
  if (*b0 >= *b1) {
    *lo = *hi = 0;
  } else {
    *lo = plan->buckets[*b0].flat_offset;
    *hi = plan->buckets[*b1 - 1].flat_offset + plan->buckets[*b1 - 1].padded;
  }
  return SBP_OK;
}

// Pieces of the non-empty tensors inside flat [lo, hi): (tensor, first
// element of the tensor in the piece, flat position, length), in flat order.
struct Piece {
  int32_t t;
  int64_t elem, flat, len;
};

std::vector<Piece> pieces_in(const sbp_plan* plan, int64_t lo, int64_t hi) {
  std::vector<Piece> out;
  const auto& order = plan->flat_order;
  // first tensor that ends after lo
  auto it = std::lower_bound(order.begin(), order.end(), lo, [&](int32_t t, int64_t x) {
    return plan->tensor_flat[t] + plan->numel[t] <= x;
  });
  for (; it != order.end(); ++it) {
    const int32_t t = *it;
    const int64_t a = plan->tensor_flat[t], e = a + plan->numel[t];
    if (a >= hi) break;
    const int64_t s = a > lo ? a : lo, f = e < hi ? e : hi;
    if (f > s) out.push_back(Piece{t, s - a, s, f - s});
  }
  return out;
}

// Device pointers in `ptrs` (lengths in bytes) pairwise disjoint?
bool disjoint(std::vector<std::pair<uintptr_t, int64_t>> ranges) {
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].first + static_cast<uintptr_t>(ranges[i - 1].second))
      return false;
  return true;
}

}  // namespace

sbp_status pack_segments(const sbp_plan* plan, int32_t bucket, const void* const* tensor_grads,
                         void* flat, std::vector<Seg>& out) {
  out.clear();
  const char* who = "sbp_pack_grads";
  if (plan == nullptr) return sbp::fail(SBP_EINVAL, "sbp_pack_grads: plan is null");
  if (tensor_grads == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_pack_grads: tensor_grads is null");
  if (flat == nullptr) return sbp::fail(SBP_EINVAL, "sbp_pack_grads: flat is null");
  if (!sbp::aligned(flat, 16))
    return sbp::fail(SBP_EALIGN, "sbp_pack_grads: flat must be 16-byte aligned");
  int32_t b0, b1;
  int64_t lo, hi;
  sbp_status st = bucket_range(who, plan, bucket, &b0, &b1, &lo, &hi);
  if (st != SBP_OK) return st;
  uint16_t* F = static_cast<uint16_t*>(flat);
  std::vector<Seg> segs;
  try {
    int64_t pos = lo;
    for (const Piece& pc : pieces_in(plan, lo, hi)) {
      const void* src = tensor_grads[pc.t];
      if (src == nullptr)
        return sbp::fail(SBP_EINVAL, "sbp_pack_grads: gradient pointer of a tensor is null");
      if (!sbp::aligned(src, 2))
        return sbp::fail(SBP_EALIGN, "sbp_pack_grads: gradients must be 2-byte aligned");
      if (sbp::overlaps(src, 2 * plan->numel[pc.t], flat, 2 * plan->flat_numel))
        return sbp::fail(SBP_EINVAL, "sbp_pack_grads: a gradient overlaps the flat buffer");
      if (pc.flat > pos) segs.push_back(Seg{nullptr, F + pos, pc.flat - pos});
      segs.push_back(Seg{static_cast<const uint16_t*>(src) + pc.elem, F + pc.flat, pc.len});
      pos = pc.flat + pc.len;
    }
    if (hi > pos) segs.push_back(Seg{nullptr, F + pos, hi - pos});
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, "sbp_pack_grads: out of host memory");
  }
  out.swap(segs);
  return sbp::ok();
}

sbp_status unpack_segments(const sbp_plan* plan, int32_t bucket, const void* flat,
                           void* const* tensor_params, std::vector<Seg>& out) {
  out.clear();
  const char* who = "sbp_unpack_params";
  if (plan == nullptr) return sbp::fail(SBP_EINVAL, "sbp_unpack_params: plan is null");
  if (tensor_params == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_unpack_params: tensor_params is null");
  if (flat == nullptr) return sbp::fail(SBP_EINVAL, "sbp_unpack_params: flat is null");
  if (!sbp::aligned(flat, 16))
    return sbp::fail(SBP_EALIGN, "sbp_unpack_params: flat must be 16-byte aligned");
  int32_t b0, b1;
  int64_t lo, hi;
  sbp_status st = bucket_range(who, plan, bucket, &b0, &b1, &lo, &hi);
  if (st != SBP_OK) return st;
  const uint16_t* F = static_cast<const uint16_t*>(flat);
  std::vector<Seg> segs;
  try {
    std::vector<std::pair<uintptr_t, int64_t>> outs;
    int32_t last = -1;
    for (const Piece& pc : pieces_in(plan, lo, hi)) {
      void* dst = tensor_params[pc.t];
      if (dst == nullptr)
        return sbp::fail(SBP_EINVAL, "sbp_unpack_params: parameter pointer of a tensor is null");
      if (!sbp::aligned(dst, 2))
        return sbp::fail(SBP_EALIGN, "sbp_unpack_params: parameters must be 2-byte aligned");
      if (sbp::overlaps(dst, 2 * plan->numel[pc.t], flat, 2 * plan->flat_numel))
        return sbp::fail(SBP_EINVAL, "sbp_unpack_params: a parameter overlaps the flat buffer");
      if (pc.t != last)
        outs.push_back({reinterpret_cast<uintptr_t>(dst), 2 * plan->numel[pc.t]});
      last = pc.t;
      segs.push_back(Seg{F + pc.flat, static_cast<uint16_t*>(dst) + pc.elem, pc.len});
    }
    if (!disjoint(outs))
      return sbp::fail(SBP_EINVAL, "sbp_unpack_params: parameter buffers overlap");
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, "sbp_unpack_params: out of host memory");
  }
  out.swap(segs);
  return sbp::ok();
}

sbp_status shard_of_segments(const sbp_plan* plan, int32_t bucket, int32_t rank, const void* flat,
                             void* shard, std::vector<Seg>& out) {
  out.clear();
  const char* who = "sbp_shard_of";
  if (plan == nullptr || flat == nullptr || shard == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_shard_of: null argument");
  if (rank < 0 || rank >= plan->world_n)
    return sbp::fail(SBP_EINVAL, "sbp_shard_of: rank out of range");
  if (!sbp::aligned(flat, 16) || !sbp::aligned(shard, 16))
    return sbp::fail(SBP_EALIGN, "sbp_shard_of: buffers must be 16-byte aligned");
  if (sbp::overlaps(flat, 2 * plan->flat_numel, shard, 2 * plan->shard_numel))
    return sbp::fail(SBP_EINVAL, "sbp_shard_of: the shard overlaps the flat buffer");
  int32_t b0, b1;
  int64_t lo, hi;
  sbp_status st = bucket_range(who, plan, bucket, &b0, &b1, &lo, &hi);
  if (st != SBP_OK) return st;
  const uint16_t* F = static_cast<const uint16_t*>(flat);
  uint16_t* S = static_cast<uint16_t*>(shard);
  std::vector<Seg> segs;
  try {
    for (int32_t b = b0; b < b1; ++b) {
      const sbp::Bucket& k = plan->buckets[b];
      if (k.chunk > 0)
        segs.push_back(Seg{F + k.flat_offset + rank * k.chunk, S + k.shard_offset, k.chunk});
    }
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, "sbp_shard_of: out of host memory");
  }
  out.swap(segs);
  return sbp::ok();
}

sbp_status gather_fans(const sbp_plan* plan, int32_t bucket, const void* const* shards, void* flat,
                       std::vector<Fan>& out) {
  out.clear();
  const char* who = "sbp_gather_shards";
  if (plan == nullptr || shards == nullptr || flat == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_gather_shards: null argument");
  if (!sbp::aligned(flat, 16))
    return sbp::fail(SBP_EALIGN, "sbp_gather_shards: flat must be 16-byte aligned");
  for (int32_t s = 0; s < plan->world_n; ++s) {
    if (shards[s] == nullptr) return sbp::fail(SBP_EINVAL, "sbp_gather_shards: a shard is null");
    if (!sbp::aligned(shards[s], 16))
      return sbp::fail(SBP_EALIGN, "sbp_gather_shards: shards must be 16-byte aligned");
    if (sbp::overlaps(shards[s], 2 * plan->shard_numel, flat, 2 * plan->flat_numel))
      return sbp::fail(SBP_EINVAL, "sbp_gather_shards: a shard overlaps the flat buffer");
  }
  int32_t b0, b1;
  int64_t lo, hi;
  sbp_status st = bucket_range(who, plan, bucket, &b0, &b1, &lo, &hi);
  if (st != SBP_OK) return st;
  uint16_t* F = static_cast<uint16_t*>(flat);
  std::vector<Fan> fans;
  try {
    for (int32_t b = b0; b < b1; ++b) {
      const sbp::Bucket& k = plan->buckets[b];
      if (k.chunk > 0) fans.push_back(Fan{k.shard_offset, k.chunk, 0, k.padded, F + k.flat_offset});
    }
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, "sbp_gather_shards: out of host memory");
  }
  out.swap(fans);
  return sbp::ok();
}

sbp_status gather_segments(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                           void* flat, std::vector<Seg>& out) {
  out.clear();
  std::vector<Fan> fans;
  sbp_status st = gather_fans(plan, bucket, shards, flat, fans);
  if (st != SBP_OK) return st;
  try {
    fans_to_segments(fans, shards, out);
  } catch (...) {
    out.clear();
    return sbp::fail(SBP_ENOMEM, "sbp_gather_shards: out of host memory");
  }
  return sbp::ok();
}

// Each tensor piece of a selected bucket is cut where the bucket's rank
// chunks meet; each cut part is read from the shard of the rank that owns it.
sbp_status unpack_shards_fans(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                              void* const* tensor_params, std::vector<Fan>& out) {
  out.clear();
  const char* who = "sbp_unpack_shards";
  if (plan == nullptr || shards == nullptr || tensor_params == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_unpack_shards: null argument");
  for (int32_t s = 0; s < plan->world_n; ++s) {
    if (shards[s] == nullptr) return sbp::fail(SBP_EINVAL, "sbp_unpack_shards: a shard is null");
    if (!sbp::aligned(shards[s], 16))
      return sbp::fail(SBP_EALIGN, "sbp_unpack_shards: shards must be 16-byte aligned");
  }
  int32_t b0, b1;
  int64_t lo, hi;
  sbp_status st = bucket_range(who, plan, bucket, &b0, &b1, &lo, &hi);
  if (st != SBP_OK) return st;
  std::vector<Fan> fans;
  try {
    std::vector<std::pair<uintptr_t, int64_t>> outs;
    std::vector<char> seen(plan->numel.size(), 0);
    for (int32_t b = b0; b < b1; ++b) {
      const sbp::Bucket& k = plan->buckets[b];
      if (k.chunk == 0) continue;
      for (const Piece& pc : pieces_in(plan, k.flat_offset, k.flat_offset + k.padded)) {
        void* dst = tensor_params[pc.t];
        if (dst == nullptr)
          return sbp::fail(SBP_EINVAL, "sbp_unpack_shards: parameter pointer of a tensor is null");
        if (!sbp::aligned(dst, 2))
          return sbp::fail(SBP_EALIGN, "sbp_unpack_shards: parameters must be 2-byte aligned");
        if (!seen[pc.t]) {
          const int64_t bytes = 2 * plan->numel[pc.t];
          for (int32_t s = 0; s < plan->world_n; ++s)
            if (sbp::overlaps(dst, bytes, shards[s], 2 * plan->shard_numel))
              return sbp::fail(SBP_EINVAL, "sbp_unpack_shards: a parameter overlaps a shard");
          outs.push_back({reinterpret_cast<uintptr_t>(dst), bytes});
          seen[pc.t] = 1;
        }
        // the piece's positions in the bucket, read from the ranks that own them
        fans.push_back(Fan{k.shard_offset, k.chunk, pc.flat - k.flat_offset, pc.len,
                           static_cast<uint16_t*>(dst) + pc.elem});
      }
    }
    if (!disjoint(outs))
      return sbp::fail(SBP_EINVAL, "sbp_unpack_shards: parameter buffers overlap");
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, "sbp_unpack_shards: out of host memory");
  }
  out.swap(fans);
  return sbp::ok();
}

sbp_status unpack_shards_segments(const sbp_plan* plan, int32_t bucket, const void* const* shards,
                                  void* const* tensor_params, std::vector<Seg>& out) {
  out.clear();
  std::vector<Fan> fans;
  sbp_status st = unpack_shards_fans(plan, bucket, shards, tensor_params, fans);
  if (st != SBP_OK) return st;
  try {
    fans_to_segments(fans, shards, out);
  } catch (...) {
    out.clear();
    return sbp::fail(SBP_ENOMEM, "sbp_unpack_shards: out of host memory");
  }
  return sbp::ok();
}

void fans_to_segments(const std::vector<Fan>& fans, const void* const* shards,
                      std::vector<Seg>& segs) {
  for (const Fan& f : fans) {
    for (int64_t x = f.x0; x < f.x0 + f.len;) {
      const int64_t s = x / f.chunk, j = x - s * f.chunk;
      const int64_t n = std::min(f.x0 + f.len, (s + 1) * f.chunk) - x;
      segs.push_back(Seg{static_cast<const uint16_t*>(shards[s]) + f.shard_off + j,
                         f.dst + (x - f.x0), n});
      x += n;
    }
  }
}

bool fan_pieces(const std::vector<Fan>& fans, int32_t world_n, std::vector<FanPiece>& pieces) {
  pieces.clear();
  if (world_n > kMaxFanRanks) return false;
  for (const Fan& f : fans)
    if (f.chunk > INT32_MAX) return false;
  for (const Fan& f : fans) {
    for (int64_t off = 0; off < f.len; off += kFanPiece) {
      const int64_t x = f.x0 + off;
      FanPiece p;
      p.dst = f.dst + off;
      p.shard_off = f.shard_off;
      p.len = static_cast<int32_t>(std::min(kFanPiece, f.len - off));
      p.chunk = static_cast<int32_t>(f.chunk);
      p.s0 = static_cast<int32_t>(x / f.chunk);
      p.j0 = static_cast<int32_t>(x % f.chunk);
      p.first_chunk = 0;
      p.vec = sbp::aligned(p.dst, 16) && f.shard_off % 8 == 0 && f.chunk % 8 == 0 && p.j0 % 8 == 0;
      pieces.push_back(p);
    }
  }
  return true;
}


}  // namespace sbp

using sbp::Piece;
using sbp::pieces_in;

extern "C" {

sbp_status sbp_group_runs(const sbp_plan* plan, int32_t rank, const int32_t* tensor_group,
                          int64_t* run_start, int32_t* run_group, int64_t cap, int64_t* count) {
  if (plan == nullptr || tensor_group == nullptr || count == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_group_runs: null argument");
  if (cap > 0 && (run_start == nullptr || run_group == nullptr))
    return sbp::fail(SBP_EINVAL, "sbp_group_runs: null output arrays");
  if (rank < 0 || rank >= plan->world_n)
    return sbp::fail(SBP_EINVAL, "sbp_group_runs: rank out of range");
  const int32_t T = static_cast<int32_t>(plan->numel.size());
  for (int32_t t = 0; t < T; ++t)
    if (tensor_group[t] < 0 || tensor_group[t] >= SBP_MAX_GROUPS)
      return sbp::fail(SBP_EINVAL, "sbp_group_runs: group ids must be in 0..7");
  // Leading padding is group 0; later padding extends the run before it;
  // neighbouring pieces of the same group merge.
  std::vector<std::pair<int64_t, int32_t>> runs;
  try {
    runs.push_back({0, 0});
    for (const sbp::Bucket& b : plan->buckets) {
      const int64_t lo = b.flat_offset + rank * b.chunk, hi = lo + b.chunk;
      for (const Piece& pc : pieces_in(plan, lo, hi)) {
        const int64_t at = b.shard_offset + (pc.flat - lo);
        const int32_t g = tensor_group[pc.t];
        if (g == runs.back().second) continue;
        if (at == runs.back().first)
          runs.back().second = g;  // the run before had no elements of its own
        else
          runs.push_back({at, g});
        if (runs.size() >= 2 && runs[runs.size() - 2].second == runs.back().second)
          runs.pop_back();  // merged with the one before
      }
    }
  } catch (...) {
    return sbp::fail(SBP_ENOMEM, "sbp_group_runs: out of host memory");
  }
  for (size_t i = 0; i < runs.size() && static_cast<int64_t>(i) < cap; ++i) {
    run_start[i] = runs[i].first;
    run_group[i] = runs[i].second;
  }
  *count = static_cast<int64_t>(runs.size());
  return sbp::ok();
}

}  // extern "C"
