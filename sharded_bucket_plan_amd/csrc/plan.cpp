// Host side of the library: error state, the bucket planner and its
// queries, model-state accounting and the normalisation factors.
//
// Planner: "Parallelisms" (vladislavkruglikov.com), sections Data parallel
// (later layers' gradients are ready first), Gradient bucketing (gradients
// gathered into buffers communicated when ready), FSDP / Flat parameter
// (parameters concatenated into one contiguous buffer) and ZeRO-2 (each ready
// bucket reduce-scattered; every rank keeps its 1/N shard).  The closing
// rule, alignment and shard layout are stated in sbp.h.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

namespace sbp {

namespace {
thread_local std::string g_last_error;
}

sbp_status fail(sbp_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

sbp_status ok() {
  g_last_error.clear();
  return SBP_OK;
}

namespace {

// A plan with more buckets than this is a caller error (a cap far below the
// model size); refusing it keeps the host tables bounded.
constexpr int64_t kMaxBuckets = int64_t{1} << 24;

bool add_ok(int64_t a, int64_t b, int64_t* out) {
  return !__builtin_add_overflow(a, b, out);
}

// Smallest multiple of m (> 0) that is >= x (>= 0), or -1 on overflow.
int64_t round_up(int64_t x, int64_t m) {
  int64_t r = x % m;
  if (r == 0) return x;
  int64_t y;
  if (!add_ok(x, m - r, &y)) return -1;
  return y;
}

}  // namespace

// Flat position of every tensor, and the non-empty tensors in flat order.
void finish_flat_positions(sbp_plan* p) {
  const int32_t T = static_cast<int32_t>(p->numel.size());
  p->tensor_flat.assign(T, 0);
  for (int32_t t = 0; t < T; ++t)
    p->tensor_flat[t] = p->buckets.empty()
                            ? 0
                            : p->buckets[p->tensor_bucket[t]].flat_offset + p->tensor_offset[t];
  p->flat_order.clear();
  for (int32_t t = 0; t < T; ++t)
    if (p->numel[t] > 0) p->flat_order.push_back(t);
  std::sort(p->flat_order.begin(), p->flat_order.end(),
            [&](int32_t a, int32_t b) { return p->tensor_flat[a] < p->tensor_flat[b]; });
}

// Fixed-size buckets over the concatenated tensors: the flat buffer (each
// tensor at the first multiple of align after the previous one, in visit
// order) is cut into buckets of cap/2 elements rounded down to a multiple of
// align*N (at least align*N); tensors may straddle buckets and only the last
// bucket can be short (then padded to align*N).  Flat parameters cut into
// equal communication pieces ("Parallelisms", FSDP / Flat parameter).
sbp_status split_plan(sbp_plan* p, int64_t cap_bytes, bool reverse) {
  const int32_t T = static_cast<int32_t>(p->numel.size());
  const int64_t unit = static_cast<int64_t>(p->align) * p->world_n;
  int64_t size = (cap_bytes / 2) / unit * unit;
  if (size < unit) size = unit;
  std::vector<int64_t> pos(T, 0);
  int64_t end = 0;
  for (int32_t i = 0; i < T; ++i) {
    const int32_t t = reverse ? T - 1 - i : i;
    const int64_t start = end == 0 ? 0 : round_up(end, p->align);
    int64_t e;
    if (start < 0 || !add_ok(start, p->numel[t], &e))
      return fail(SBP_ERANGE, "sbp_bucket_plan: flat size overflows");
    pos[t] = start;
    end = e;
  }
  if (end > INT64_MAX / 4) return fail(SBP_ERANGE, "sbp_bucket_plan: flat size overflows");
  const int64_t nb = end > 0 ? (end + size - 1) / size : (T > 0 ? 1 : 0);
  if (nb > kMaxBuckets) return fail(SBP_ERANGE, "sbp_bucket_plan: more than 2^24 buckets");
  p->tensor_bucket.assign(T, 0);
  p->tensor_offset.assign(T, 0);
  for (int32_t t = 0; t < T; ++t) {
    int64_t b = pos[t] / size;
    if (b > nb - 1) b = nb - 1;
    p->tensor_bucket[t] = static_cast<int32_t>(b);
    p->tensor_offset[t] = pos[t] - b * size;
  }
  p->buckets.assign(static_cast<size_t>(nb), Bucket{{}, 0, 0, 0, 0, 0});
  int64_t shard = 0, flat = 0;
  for (int64_t b = 0; b < nb; ++b) {
    Bucket& k = p->buckets[b];
    const int64_t lo = b * size, hi = lo + size;
    k.used = (end < hi ? end : hi) - lo;
    if (k.used < 0) k.used = 0;
    k.padded = round_up(k.used, unit);
    if (k.padded < 0) return fail(SBP_ERANGE, "sbp_bucket_plan: padding overflows");
    k.chunk = k.padded / p->world_n;
    k.shard_offset = shard;
    k.flat_offset = lo;
    if (!add_ok(shard, k.chunk, &shard) || !add_ok(flat, k.padded, &flat))
      return fail(SBP_ERANGE, "sbp_bucket_plan: total size overflows");
  }
  // members of each bucket, in visit order
  for (int32_t i = 0; i < T; ++i) {
    const int32_t t = reverse ? T - 1 - i : i;
    if (p->numel[t] == 0) {
      p->buckets[p->tensor_bucket[t]].tensors.push_back(t);
      continue;
    }
    const int64_t b0 = pos[t] / size, b1 = (pos[t] + p->numel[t] - 1) / size;
    for (int64_t b = b0; b <= b1; ++b) p->buckets[b].tensors.push_back(t);
  }
  p->shard_numel = shard;
  p->flat_numel = flat;
  finish_flat_positions(p);
  return SBP_OK;
}

}  // namespace sbp

using sbp::fail;
using sbp::ok;

extern "C" {

const char* sbp_last_error(void) { return sbp::g_last_error.c_str(); }

const char* sbp_version(void) { return "sbp 0.1.0 (gfx950)"; }

sbp_status sbp_bucket_plan(const int64_t* numel, int32_t n_tensors,
                           int64_t bucket_cap_bytes, int32_t world_n,
                           int32_t align_elems, uint32_t flags,
                           sbp_plan** out) {
  if (out == nullptr) return fail(SBP_EINVAL, "sbp_bucket_plan: out is null");
  *out = nullptr;
  if (n_tensors < 0) return fail(SBP_EINVAL, "sbp_bucket_plan: n_tensors < 0");
  if (n_tensors > 0 && numel == nullptr)
    return fail(SBP_EINVAL, "sbp_bucket_plan: numel is null");
  if (bucket_cap_bytes <= 0)
    return fail(SBP_EINVAL, "sbp_bucket_plan: bucket_cap_bytes must be > 0");
  if (world_n <= 0) return fail(SBP_EINVAL, "sbp_bucket_plan: world_n must be > 0");
  if (align_elems <= 0 || align_elems > 4096 || (align_elems & (align_elems - 1)))
    return fail(SBP_EINVAL, "sbp_bucket_plan: align_elems must be a power of two in 1..4096");
  if (flags & ~(SBP_ORDER_FORWARD | SBP_SPLIT_TENSORS))
    return fail(SBP_EINVAL, "sbp_bucket_plan: unknown flags");
  for (int32_t t = 0; t < n_tensors; ++t)
    if (numel[t] < 0) return fail(SBP_EINVAL, "sbp_bucket_plan: negative numel");

  sbp_plan* p = new (std::nothrow) sbp_plan();
  if (p == nullptr) return fail(SBP_ENOMEM, "sbp_bucket_plan: out of host memory");
  try {
    p->numel.assign(numel, numel + n_tensors);
    p->tensor_bucket.assign(n_tensors, -1);
    p->tensor_offset.assign(n_tensors, 0);
    p->world_n = world_n;
    p->align = align_elems;
    p->split = (flags & SBP_SPLIT_TENSORS) != 0;
    const bool reverse = (flags & SBP_ORDER_FORWARD) == 0;
    if (p->split) {
      sbp_status st = sbp::split_plan(p, bucket_cap_bytes, reverse);
      if (st != SBP_OK) {
        delete p;
        return st;
      }
      *out = p;
      return ok();
    }

    sbp::Bucket cur{{}, 0, 0, 0, 0, 0};
    auto close = [&]() { p->buckets.push_back(cur); cur = sbp::Bucket{{}, 0, 0, 0, 0, 0}; };
    for (int32_t i = 0; i < n_tensors; ++i) {
      int32_t t = reverse ? n_tensors - 1 - i : i;
      int64_t off = cur.used == 0 ? 0 : sbp::round_up(cur.used, align_elems);
      int64_t end;
      if (off < 0 || !sbp::add_ok(off, p->numel[t], &end) || end > INT64_MAX / 2) {
        delete p;
        return fail(SBP_ERANGE, "sbp_bucket_plan: bucket size overflows");
      }
      cur.tensors.push_back(t);
      p->tensor_bucket[t] = static_cast<int32_t>(p->buckets.size());
      p->tensor_offset[t] = off;
      cur.used = end;
      if (2 * end >= bucket_cap_bytes) close();
    }
    if (!cur.tensors.empty()) close();

    const int64_t unit = static_cast<int64_t>(align_elems) * world_n;
    int64_t shard = 0, flat = 0;
    for (auto& b : p->buckets) {
      b.padded = sbp::round_up(b.used, unit);
      if (b.padded < 0) { delete p; return fail(SBP_ERANGE, "sbp_bucket_plan: padding overflows"); }
      b.chunk = b.padded / world_n;
      b.shard_offset = shard;
      b.flat_offset = flat;
      if (!sbp::add_ok(shard, b.chunk, &shard) || !sbp::add_ok(flat, b.padded, &flat)) {
        delete p;
        return fail(SBP_ERANGE, "sbp_bucket_plan: total size overflows");
      }
    }
    p->shard_numel = shard;
    p->flat_numel = flat;
    sbp::finish_flat_positions(p);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(SBP_ENOMEM, "sbp_bucket_plan: out of host memory");
  }
  *out = p;
  return ok();
}

sbp_status sbp_bucket_plan_per_tensor(const int64_t* numel, const int64_t* row_elems,
                                      int32_t n_tensors, int32_t world_n, int32_t align_elems,
                                      uint32_t flags, sbp_plan** out) {
  if (out == nullptr) return fail(SBP_EINVAL, "sbp_bucket_plan_per_tensor: out is null");
  *out = nullptr;
  if (n_tensors < 0) return fail(SBP_EINVAL, "sbp_bucket_plan_per_tensor: n_tensors < 0");
  if (n_tensors > 0 && numel == nullptr)
    return fail(SBP_EINVAL, "sbp_bucket_plan_per_tensor: numel is null");
  if (world_n <= 0) return fail(SBP_EINVAL, "sbp_bucket_plan_per_tensor: world_n must be > 0");
  if (align_elems <= 0 || align_elems > 4096 || (align_elems & (align_elems - 1)))
    return fail(SBP_EINVAL,
                "sbp_bucket_plan_per_tensor: align_elems must be a power of two in 1..4096");
  if (flags & ~SBP_ORDER_FORWARD)
    return fail(SBP_EINVAL, "sbp_bucket_plan_per_tensor: unknown flags");
  for (int32_t t = 0; t < n_tensors; ++t) {
    const int64_t row = row_elems ? row_elems[t] : 1;
    if (numel[t] < 0 || row <= 0 || numel[t] % row != 0)
      return fail(SBP_EINVAL,
                  "sbp_bucket_plan_per_tensor: numel must be >= 0 and a multiple of its row size");
  }
  sbp_plan* p = new (std::nothrow) sbp_plan();
  if (p == nullptr) return fail(SBP_ENOMEM, "sbp_bucket_plan_per_tensor: out of host memory");
  try {
    p->numel.assign(numel, numel + n_tensors);
    p->tensor_bucket.assign(n_tensors, -1);
    p->tensor_offset.assign(n_tensors, 0);
    p->world_n = world_n;
    p->align = align_elems;
    p->split = false;
    const bool reverse = (flags & SBP_ORDER_FORWARD) == 0;
    int64_t shard = 0, flat = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
      const int32_t t = reverse ? n_tensors - 1 - i : i;
      const int64_t row = row_elems ? row_elems[t] : 1;
      // whole, aligned rows per rank: pad to N * lcm(align, row)
      const int64_t a = align_elems;
      int64_t g = a, r = row;
      while (r) { const int64_t q = g % r; g = r; r = q; }
      int64_t unit, step;
      if (__builtin_mul_overflow(a / g, row, &unit) ||
          __builtin_mul_overflow(unit, static_cast<int64_t>(world_n), &step)) {
        delete p;
        return fail(SBP_ERANGE, "sbp_bucket_plan_per_tensor: row unit overflows");
      }
      sbp::Bucket k{{t}, numel[t], 0, 0, shard, flat};
      k.padded = sbp::round_up(numel[t], step);
      if (k.padded < 0) {
        delete p;
        return fail(SBP_ERANGE, "sbp_bucket_plan_per_tensor: padding overflows");
      }
      k.chunk = k.padded / world_n;
      p->tensor_bucket[t] = static_cast<int32_t>(p->buckets.size());
      p->buckets.push_back(k);
      if (!sbp::add_ok(shard, k.chunk, &shard) || !sbp::add_ok(flat, k.padded, &flat)) {
        delete p;
        return fail(SBP_ERANGE, "sbp_bucket_plan_per_tensor: total size overflows");
      }
    }
    p->shard_numel = shard;
    p->flat_numel = flat;
    sbp::finish_flat_positions(p);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(SBP_ENOMEM, "sbp_bucket_plan_per_tensor: out of host memory");
  }
  *out = p;
  return ok();
}

void sbp_plan_free(sbp_plan* plan) { delete plan; }

int32_t sbp_plan_num_tensors(const sbp_plan* plan) {
  return plan ? static_cast<int32_t>(plan->numel.size()) : -1;
}
int32_t sbp_plan_num_buckets(const sbp_plan* plan) {
  return plan ? static_cast<int32_t>(plan->buckets.size()) : -1;
}
int32_t sbp_plan_world_n(const sbp_plan* plan) { return plan ? plan->world_n : -1; }
int64_t sbp_plan_shard_numel(const sbp_plan* plan) { return plan ? plan->shard_numel : -1; }
int64_t sbp_plan_flat_numel(const sbp_plan* plan) { return plan ? plan->flat_numel : -1; }

sbp_status sbp_plan_tensor(const sbp_plan* plan, int32_t t, int32_t* bucket,
                           int64_t* offset) {
  if (plan == nullptr) return fail(SBP_EINVAL, "sbp_plan_tensor: plan is null");
  if (t < 0 || t >= static_cast<int32_t>(plan->numel.size()))
    return fail(SBP_EINVAL, "sbp_plan_tensor: tensor index out of range");
  if (bucket) *bucket = plan->tensor_bucket[t];
  if (offset) *offset = plan->tensor_offset[t];
  return ok();
}

sbp_status sbp_plan_bucket(const sbp_plan* plan, int32_t b, int64_t* used,
                           int64_t* padded, int64_t* chunk,
                           int64_t* shard_offset, int64_t* flat_offset) {
  if (plan == nullptr) return fail(SBP_EINVAL, "sbp_plan_bucket: plan is null");
  if (b < 0 || b >= static_cast<int32_t>(plan->buckets.size()))
    return fail(SBP_EINVAL, "sbp_plan_bucket: bucket index out of range");
  const sbp::Bucket& k = plan->buckets[b];
  if (used) *used = k.used;
  if (padded) *padded = k.padded;
  if (chunk) *chunk = k.chunk;
  if (shard_offset) *shard_offset = k.shard_offset;
  if (flat_offset) *flat_offset = k.flat_offset;
  return ok();
}

sbp_status sbp_plan_bucket_tensors(const sbp_plan* plan, int32_t b, int32_t* ids,
                                   int32_t cap, int32_t* count) {
  if (plan == nullptr || count == nullptr)
    return fail(SBP_EINVAL, "sbp_plan_bucket_tensors: null argument");
  if (b < 0 || b >= static_cast<int32_t>(plan->buckets.size()))
    return fail(SBP_EINVAL, "sbp_plan_bucket_tensors: bucket index out of range");
  if (cap > 0 && ids == nullptr)
    return fail(SBP_EINVAL, "sbp_plan_bucket_tensors: ids is null");
  const auto& ts = plan->buckets[b].tensors;
  *count = static_cast<int32_t>(ts.size());
  for (int32_t i = 0; i < cap && i < *count; ++i) ids[i] = ts[i];
  return ok();
}

sbp_status sbp_plan_state_bytes(const sbp_plan* plan, int32_t zero_stage,
                                int64_t* per_rank_bytes) {
  if (plan == nullptr || per_rank_bytes == nullptr)
    return fail(SBP_EINVAL, "sbp_plan_state_bytes: null argument");
  // bf16 param 2 + bf16 grad 2 + fp32 master 4 + m 4 + v 4 bytes a parameter
  const int64_t full = plan->flat_numel, shard = plan->shard_numel;
  __int128 bytes;
  switch (zero_stage) {
    case 0: bytes = (__int128)16 * full; break;
    case 1: bytes = (__int128)4 * full + (__int128)12 * shard; break;
    case 2: bytes = (__int128)2 * full + (__int128)14 * shard; break;
    case 3: bytes = (__int128)16 * shard; break;
    default: return fail(SBP_EINVAL, "sbp_plan_state_bytes: zero_stage must be 0..3");
  }
  if (bytes > INT64_MAX) return fail(SBP_ERANGE, "sbp_plan_state_bytes: overflows int64");
  *per_rank_bytes = static_cast<int64_t>(bytes);
  return ok();
}

sbp_status sbp_mean_scale(int32_t R, int32_t K, float* scale) {
  if (scale == nullptr) return fail(SBP_EINVAL, "sbp_mean_scale: scale is null");
  if (R < 1 || K < 1) return fail(SBP_EINVAL, "sbp_mean_scale: R and K must be >= 1");
  *scale = static_cast<float>(1.0 / (static_cast<double>(R) * static_cast<double>(K)));
  return ok();
}

sbp_status sbp_tokens_scale(const int64_t* counts, int32_t R, float* scale) {
  if (scale == nullptr || counts == nullptr)
    return fail(SBP_EINVAL, "sbp_tokens_scale: null argument");
  if (R < 1) return fail(SBP_EINVAL, "sbp_tokens_scale: R must be >= 1");
  int64_t total = 0;
  for (int32_t r = 0; r < R; ++r) {
    if (counts[r] < 0) return fail(SBP_EINVAL, "sbp_tokens_scale: negative count");
    if (!sbp::add_ok(total, counts[r], &total))
      return fail(SBP_ERANGE, "sbp_tokens_scale: total overflows");
  }
  if (total == 0) return fail(SBP_EINVAL, "sbp_tokens_scale: zero valid tokens");
  *scale = static_cast<float>(1.0 / static_cast<double>(total));
  return ok();
}

}  // extern "C"
