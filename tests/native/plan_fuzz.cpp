// Host fuzz driver for the bucket planners and plan queries, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_native_sanitize.py.
// Random and hostile arguments (huge counts, overflowing sizes, bad indices,
// short output arrays); every call must return a status without a sanitizer
// report, and every plan that is made must satisfy the layout invariants.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "sbp.h"

namespace {

std::mt19937_64 rng(20260101);

int64_t pick(const std::vector<int64_t>& xs) { return xs[rng() % xs.size()]; }

int64_t random_numel() {
  switch (rng() % 6) {
    case 0: return 0;
    case 1: return static_cast<int64_t>(rng() % 16);
    case 2: return static_cast<int64_t>(rng() % 5000);
    case 3: return static_cast<int64_t>(rng() % (int64_t{1} << 30));
    case 4: return pick({INT64_MAX, INT64_MAX / 2, INT64_MAX / 4 + 1, int64_t{1} << 40, -1});
    default: return static_cast<int64_t>(rng() % 100000);
  }
}

#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "invariant failed at line %d: %s\n", __LINE__, #cond); \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

void check_plan(const sbp_plan* p, const std::vector<int64_t>& numel, int32_t N, bool split) {
  const int32_t T = sbp_plan_num_tensors(p), nb = sbp_plan_num_buckets(p);
  CHECK(T == static_cast<int32_t>(numel.size()));
  CHECK(sbp_plan_world_n(p) == N);
  int64_t shard = 0, flat = 0;
  for (int32_t b = 0; b < nb; ++b) {
    int64_t used, padded, chunk, so, fo;
    CHECK(sbp_plan_bucket(p, b, &used, &padded, &chunk, &so, &fo) == SBP_OK);
    CHECK(used >= 0 && used <= padded && chunk * N == padded);
    CHECK(so == shard && fo == flat);
    shard += chunk;
    flat += padded;
    int32_t count = -1;
    CHECK(sbp_plan_bucket_tensors(p, b, nullptr, 0, &count) == SBP_OK && count >= 0);
    std::vector<int32_t> ids(count > 1 ? count - 1 : 1, -7);  // short on purpose
    int32_t count2 = -1;
    CHECK(sbp_plan_bucket_tensors(p, b, ids.data(), static_cast<int32_t>(ids.size()),
                                  &count2) == SBP_OK);
    CHECK(count2 == count);
    for (int32_t i = 0; i < count && i < static_cast<int32_t>(ids.size()); ++i)
      CHECK(ids[i] >= 0 && ids[i] < T);
  }
  CHECK(shard == sbp_plan_shard_numel(p) && flat == sbp_plan_flat_numel(p));
  CHECK(flat == shard * N);
  for (int32_t t = 0; t < T; ++t) {
    int32_t b;
    int64_t off;
    CHECK(sbp_plan_tensor(p, t, &b, &off) == SBP_OK);
    CHECK(b >= 0 && b < nb && off >= 0);
    int64_t used;
    CHECK(sbp_plan_bucket(p, b, &used, nullptr, nullptr, nullptr, nullptr) == SBP_OK);
    if (!split) CHECK(off + numel[t] <= used);
  }
  int32_t b;
  int64_t off;
  CHECK(sbp_plan_tensor(p, -1, &b, &off) == SBP_EINVAL);
  CHECK(sbp_plan_tensor(p, T, &b, &off) == SBP_EINVAL);
  CHECK(sbp_plan_bucket(p, -1, nullptr, nullptr, nullptr, nullptr, nullptr) == SBP_EINVAL);
  CHECK(sbp_plan_bucket(p, nb, nullptr, nullptr, nullptr, nullptr, nullptr) == SBP_EINVAL);
  for (int32_t stage = -1; stage <= 4; ++stage) {
    int64_t bytes = -1;
    const sbp_status st = sbp_plan_state_bytes(p, stage, &bytes);
    CHECK(st == SBP_OK || st == SBP_EINVAL || st == SBP_ERANGE);
    if (stage < 0 || stage > 3) CHECK(st == SBP_EINVAL);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  int made = 0, refused = 0;
  for (int it = 0; it < iters; ++it) {
    const int32_t T = static_cast<int32_t>(rng() % 12);
    std::vector<int64_t> numel(T), rows(T);
    for (int32_t t = 0; t < T; ++t) {
      numel[t] = random_numel();
      rows[t] = pick({1, 2, 3, 7, 8, 768, 4096, INT64_MAX / 3});
      if (rng() % 2 && numel[t] > 0 && rows[t] > 0) numel[t] -= numel[t] % rows[t];
    }
    const int64_t cap = pick({1, 2, 16, 100, 4096, int64_t{25} << 20, INT64_MAX, 0, -5});
    if (cap > 0 && cap < 4096)  // keep split plans to a few thousand buckets
      for (int64_t& x : numel)
        if (x > 0 && x < (int64_t{1} << 31)) x %= 4096;
    const int32_t N = static_cast<int32_t>(pick({1, 2, 3, 8, 64, 1 << 20, INT32_MAX, 0, -1}));
    const int32_t align = static_cast<int32_t>(pick({1, 2, 8, 16, 4096, 3, 0, 8192}));
    const uint32_t flags = static_cast<uint32_t>(pick({0, 1, 2, 3, 4}));
    sbp_plan* p = nullptr;
    sbp_status st;
    const bool per_tensor = rng() % 3 == 0;
    if (per_tensor)
      st = sbp_bucket_plan_per_tensor(numel.data(), rng() % 4 ? rows.data() : nullptr, T, N,
                                      align, flags & 1u, &p);
    else
      st = sbp_bucket_plan(numel.data(), T, cap, N, align, flags, &p);
    if (st == SBP_OK) {
      CHECK(p != nullptr);
      check_plan(p, numel, N, !per_tensor && (flags & SBP_SPLIT_TENSORS));
      sbp_plan_free(p);
      ++made;
    } else {
      CHECK(p == nullptr);
      CHECK(st == SBP_EINVAL || st == SBP_ERANGE || st == SBP_ENOMEM);
      CHECK(sbp_last_error()[0] != '\0');
      ++refused;
    }
  }
  // a split plan of a huge model with a tiny cap is refused, not built
  {
    const int64_t big[2] = {int64_t{1} << 40, 5};
    sbp_plan* p = nullptr;
    CHECK(sbp_bucket_plan(big, 2, 16, 8, 8, SBP_SPLIT_TENSORS, &p) == SBP_ERANGE && !p);
    CHECK(sbp_bucket_plan(big, 2, 16, 8, 8, 0, &p) == SBP_OK && p);
    check_plan(p, std::vector<int64_t>(big, big + 2), 8, false);
    sbp_plan_free(p);
  }
  // the scale helpers on edge values
  float s;
  CHECK(sbp_mean_scale(0, 1, &s) == SBP_EINVAL);
  const sbp_status ms = sbp_mean_scale(INT32_MAX, INT32_MAX, &s);
  CHECK(ms == SBP_OK || ms == SBP_ERANGE);
  int64_t counts[3] = {INT64_MAX, INT64_MAX, 1};
  CHECK(sbp_tokens_scale(counts, 3, &s) == SBP_ERANGE);
  CHECK(sbp_tokens_scale(nullptr, 3, &s) == SBP_EINVAL);
  printf("plans made %d, refused %d\n", made, refused);
  return made > 0 && refused > 0 ? 0 : 1;
}
