// Host fuzz driver for the copy-segment builders of the layout calls (pack,
// unpack, shard_of, gather, unpack_shards) and the fan pieces of the last two, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_native_sanitize.py.  The GPU copy
// kernel executes these segment lists as they are, so a segment outside its
// buffers would be an out-of-bounds device write.  Here every list is
// executed on host buffers with guard bands: every destination element must be
// written exactly once, nothing outside the selected buckets may change, and
// the values must land where the plan queries say.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "layout.h"
#include "sbp.h"

namespace {

std::mt19937_64 rng(20260102);
constexpr int64_t kGuard = 64;
constexpr uint16_t kSentinel = 0xA5A5;

#define CHECK(cond)                                                            \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);      \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

// A host buffer with guard bands; `p` is the usable part.
struct Buf {
  std::vector<uint16_t> mem;
  uint16_t* p;
  int64_t n;
  explicit Buf(int64_t n_, uint16_t fill = kSentinel) : mem(n_ + 2 * kGuard, fill), n(n_) {
    p = mem.data() + kGuard;
    for (int64_t i = 0; i < kGuard; ++i) mem[i] = mem[kGuard + n + i] = 0xBEEF;
  }
  bool guards_ok() const {
    for (int64_t i = 0; i < kGuard; ++i)
      if (mem[i] != 0xBEEF || mem[kGuard + n + i] != 0xBEEF) return false;
    return true;
  }
  bool holds(const uint16_t* q, int64_t len) const { return q >= p && len >= 0 && q + len <= p + n; }
};

// Executes the segments; every write must stay in one of `dsts`, every read in
// one of `srcs`; `written` counts writes per element of each destination.
void run(const std::vector<sbp::Seg>& segs, std::vector<Buf*> dsts, std::vector<Buf*> srcs,
         std::vector<std::vector<int>>& written) {
  written.assign(dsts.size(), {});
  for (size_t d = 0; d < dsts.size(); ++d) written[d].assign(dsts[d]->n, 0);
  for (const sbp::Seg& s : segs) {
    CHECK(s.len > 0);
    int d = -1;
    for (size_t k = 0; k < dsts.size(); ++k)
      if (dsts[k]->holds(s.dst, s.len)) d = static_cast<int>(k);
    CHECK(d >= 0);  // inside a destination buffer
    if (s.src) {
      bool in = false;
      for (Buf* b : srcs) in = in || b->holds(s.src, s.len);
      CHECK(in);  // inside a source buffer
    }
    for (int64_t i = 0; i < s.len; ++i) {
      s.dst[i] = s.src ? s.src[i] : 0;
      written[d][s.dst + i - dsts[d]->p] += 1;
    }
  }
  for (Buf* b : dsts) CHECK(b->guards_ok());
}

// Executes fan pieces element by element with the fan copy kernel's index
// arithmetic (t = j0 + o in unsigned 32 bits, rank s0 + t / chunk, shard
// position shard_off + t % chunk), checking that every read stays inside its
// shard, every write inside a destination, and that a piece marked for
// 16-byte copies keeps each group of 8 elements in one rank's chunk, aligned.
void run_pieces(const std::vector<sbp::FanPiece>& pieces, const std::vector<const void*>& shards,
                int64_t shard_numel, std::vector<Buf*> dsts, std::vector<std::vector<int>>& written) {
  written.assign(dsts.size(), {});
  for (size_t d = 0; d < dsts.size(); ++d) written[d].assign(dsts[d]->n, 0);
  const int32_t N = static_cast<int32_t>(shards.size());
  for (const sbp::FanPiece& f : pieces) {
    CHECK(f.len >= 1 && f.len <= sbp::kFanPiece && f.chunk >= 1);
    CHECK(f.s0 >= 0 && f.s0 < N && f.j0 >= 0 && f.j0 < f.chunk && f.first_chunk == 0);
    CHECK(static_cast<uint64_t>(f.j0) + static_cast<uint64_t>(f.len) < (uint64_t{1} << 32));
    int d = -1;
    for (size_t k = 0; k < dsts.size(); ++k)
      if (dsts[k]->holds(f.dst, f.len)) d = static_cast<int>(k);
    CHECK(d >= 0);
    if (f.vec) CHECK((reinterpret_cast<uintptr_t>(f.dst) & 15) == 0);
    for (int64_t o = 0; o < f.len; ++o) {
      const uint32_t t = static_cast<uint32_t>(f.j0) + static_cast<uint32_t>(o);
      const uint32_t q = t / static_cast<uint32_t>(f.chunk);
      const int64_t s = f.s0 + static_cast<int64_t>(q);
      const int64_t pos = f.shard_off + (t - q * static_cast<uint32_t>(f.chunk));
      CHECK(s < N && pos >= 0 && pos < shard_numel);
      if (f.vec && o % 8 == 0 && o + 8 <= f.len) {
        CHECK((t + 7) / static_cast<uint32_t>(f.chunk) == q);  // one rank's chunk
        CHECK(pos % 8 == 0);                                    // 16-byte aligned read
      }
      f.dst[o] = static_cast<const uint16_t*>(shards[s])[pos];
      written[d][f.dst + o - dsts[d]->p] += 1;
    }
  }
  for (Buf* b : dsts) CHECK(b->guards_ok());
}

struct Case {
  std::vector<int64_t> numel, rows;
  int32_t N = 1, align = 8;
  int kind = 0;  // 0 whole, 1 split, 2 per-tensor
  int64_t cap = 64;
};

sbp_plan* make(const Case& c) {
  sbp_plan* p = nullptr;
  sbp_status st;
  if (c.kind == 2)
    st = sbp_bucket_plan_per_tensor(c.numel.data(), c.rows.data(),
                                    static_cast<int32_t>(c.numel.size()), c.N, c.align, 0, &p);
  else
    st = sbp_bucket_plan(c.numel.data(), static_cast<int32_t>(c.numel.size()), c.cap, c.N,
                         c.align, c.kind == 1 ? SBP_SPLIT_TENSORS : 0, &p);
  CHECK(st == SBP_OK && p);
  return p;
}

int64_t tensor_flat(const sbp_plan* p, int32_t t) {
  int32_t b;
  int64_t off, fo;
  CHECK(sbp_plan_tensor(p, t, &b, &off) == SBP_OK);
  CHECK(sbp_plan_bucket(p, b, nullptr, nullptr, nullptr, nullptr, &fo) == SBP_OK);
  return fo + off;
}

void one_case(const Case& c) {
  sbp_plan* p = make(c);
  const int32_t T = static_cast<int32_t>(c.numel.size()), nb = sbp_plan_num_buckets(p);
  const int64_t F = sbp_plan_flat_numel(p), S = sbp_plan_shard_numel(p);
  const int32_t bucket = nb > 0 && rng() % 2 ? static_cast<int32_t>(rng() % nb) : -1;
  int64_t lo = 0, hi = 0;  // selected flat range
  if (nb > 0) {
    const int32_t b0 = bucket < 0 ? 0 : bucket, b1 = bucket < 0 ? nb - 1 : bucket;
    int64_t padded;
    CHECK(sbp_plan_bucket(p, b0, nullptr, nullptr, nullptr, nullptr, &lo) == SBP_OK);
    CHECK(sbp_plan_bucket(p, b1, nullptr, &padded, nullptr, nullptr, &hi) == SBP_OK);
    hi += padded;
  }
  std::vector<Buf> tens;
  for (int32_t t = 0; t < T; ++t) {
    tens.emplace_back(c.numel[t]);
    for (int64_t i = 0; i < c.numel[t]; ++i) tens[t].p[i] = static_cast<uint16_t>(t * 977 + i + 1);
  }
  std::vector<const void*> src_ptrs(T);
  std::vector<void*> dst_ptrs(T);
  std::vector<Buf*> tens_bufs;
  for (int32_t t = 0; t < T; ++t) {
    src_ptrs[t] = dst_ptrs[t] = tens[t].p;
    tens_bufs.push_back(&tens[t]);
  }
  std::vector<sbp::Seg> segs;
  std::vector<std::vector<int>> written;

  // pack: the selected range of flat gets tensor elements at their places, +0 elsewhere
  Buf flat(F);
  CHECK(sbp::pack_segments(p, bucket, T ? src_ptrs.data() : nullptr, flat.p, segs) == SBP_OK ||
        T == 0);
  if (T > 0) {
    run(segs, {&flat}, tens_bufs, written);
    std::vector<uint16_t> want(F, kSentinel);
    for (int64_t i = lo; i < hi; ++i) want[i] = 0;
    for (int32_t t = 0; t < T; ++t) {
      const int64_t a = tensor_flat(p, t);
      for (int64_t i = 0; i < c.numel[t]; ++i)
        if (a + i >= lo && a + i < hi) want[a + i] = tens[t].p[i];
    }
    for (int64_t i = 0; i < F; ++i) {
      CHECK(flat.p[i] == want[i]);
      CHECK(written[0][i] == (i >= lo && i < hi ? 1 : 0));
    }
  }

  // unpack: tensor elements inside the selected range come back from flat
  if (T > 0) {
    std::vector<Buf> outs;
    std::vector<void*> out_ptrs(T);
    std::vector<Buf*> out_bufs;
    for (int32_t t = 0; t < T; ++t) outs.emplace_back(c.numel[t]);
    for (int32_t t = 0; t < T; ++t) {
      out_ptrs[t] = outs[t].p;
      out_bufs.push_back(&outs[t]);
    }
    CHECK(sbp::unpack_segments(p, bucket, flat.p, out_ptrs.data(), segs) == SBP_OK);
    run(segs, out_bufs, {&flat}, written);
    for (int32_t t = 0; t < T; ++t) {
      const int64_t a = tensor_flat(p, t);
      for (int64_t i = 0; i < c.numel[t]; ++i) {
        const bool sel = a + i >= lo && a + i < hi;
        CHECK(written[t][i] == (sel ? 1 : 0));
        CHECK(outs[t].p[i] == (sel ? tens[t].p[i] : kSentinel));
      }
    }
  }

  // shard_of and gather: chunk s of every selected bucket <-> shard s
  std::vector<Buf> shards;
  for (int32_t s = 0; s < c.N; ++s) shards.emplace_back(S);
  std::vector<Buf*> shard_bufs;
  std::vector<const void*> shard_ptrs(c.N);
  for (int32_t s = 0; s < c.N; ++s) {
    shard_bufs.push_back(&shards[s]);
    shard_ptrs[s] = shards[s].p;
  }
  for (int64_t i = 0; i < F; ++i) flat.p[i] = static_cast<uint16_t>(i * 31 + 7);
  for (int32_t s = 0; s < c.N; ++s) {
    CHECK(sbp::shard_of_segments(p, bucket, s, flat.p, shards[s].p, segs) == SBP_OK);
    run(segs, {&shards[s]}, {&flat}, written);
  }
  Buf back(F);
  CHECK(sbp::gather_segments(p, bucket, shard_ptrs.data(), back.p, segs) == SBP_OK);
  run(segs, {&back}, shard_bufs, written);
  for (int64_t i = 0; i < F; ++i) {
    const bool sel = i >= lo && i < hi;
    CHECK(written[0][i] == (sel ? 1 : 0));
    CHECK(back.p[i] == (sel ? flat.p[i] : kSentinel));  // gather(shard_of(x)) = x
  }
  {  // the same gather as fan pieces, the way the fan copy kernel reads them
    std::vector<sbp::Fan> fans;
    std::vector<sbp::FanPiece> pieces;
    CHECK(sbp::gather_fans(p, bucket, shard_ptrs.data(), back.p, fans) == SBP_OK);
    if (sbp::fan_pieces(fans, c.N, pieces)) {
      CHECK(c.N <= sbp::kMaxFanRanks);
      Buf via(F);
      for (sbp::FanPiece& f : pieces) f.dst = via.p + (f.dst - back.p);
      run_pieces(pieces, shard_ptrs, S, {&via}, written);
      for (int64_t i = 0; i < F; ++i) {
        CHECK(written[0][i] == ((i >= lo && i < hi) ? 1 : 0));
        CHECK(via.p[i] == back.p[i]);
      }
    } else {
      CHECK(c.N > sbp::kMaxFanRanks && pieces.empty());
    }
  }
  for (int32_t b = 0; b < nb; ++b) {  // shard s holds chunk s of each selected bucket
    int64_t chunk, so, fo;
    CHECK(sbp_plan_bucket(p, b, nullptr, nullptr, &chunk, &so, &fo) == SBP_OK);
    const bool sel = bucket < 0 || bucket == b;
    for (int32_t s = 0; s < c.N; ++s)
      for (int64_t j = 0; j < chunk; ++j)
        CHECK(shards[s].p[so + j] == (sel ? flat.p[fo + s * chunk + j] : kSentinel));
  }

  // unpack_shards: what gather followed by unpack gives, in one list, from
  // shards whose every slot (padding included) holds data
  for (int32_t s = 0; s < c.N; ++s)
    for (int64_t j = 0; j < S; ++j) shards[s].p[j] = static_cast<uint16_t>(s * 7919 + j * 13 + 3);
  if (T > 0) {
    Buf ref(F);
    CHECK(sbp::gather_segments(p, bucket, shard_ptrs.data(), ref.p, segs) == SBP_OK);
    run(segs, {&ref}, shard_bufs, written);
    std::vector<Buf> outs;
    std::vector<void*> out_ptrs(T);
    std::vector<Buf*> out_bufs;
    for (int32_t t = 0; t < T; ++t) outs.emplace_back(c.numel[t]);
    for (int32_t t = 0; t < T; ++t) {
      out_ptrs[t] = outs[t].p;
      out_bufs.push_back(&outs[t]);
    }
    CHECK(sbp::unpack_shards_segments(p, bucket, shard_ptrs.data(), out_ptrs.data(), segs) ==
          SBP_OK);
    run(segs, out_bufs, shard_bufs, written);
    for (int32_t t = 0; t < T; ++t) {
      const int64_t a = tensor_flat(p, t);
      for (int64_t i = 0; i < c.numel[t]; ++i) {
        const bool sel = a + i >= lo && a + i < hi;
        CHECK(written[t][i] == (sel ? 1 : 0));
        CHECK(outs[t].p[i] == (sel ? ref.p[a + i] : kSentinel));
      }
    }
    // the same list as fan pieces, into fresh buffers, must give the same bits
    std::vector<sbp::Fan> fans;
    std::vector<sbp::FanPiece> pieces;
    CHECK(sbp::unpack_shards_fans(p, bucket, shard_ptrs.data(), out_ptrs.data(), fans) == SBP_OK);
    if (sbp::fan_pieces(fans, c.N, pieces)) {
      std::vector<Buf> again;
      std::vector<Buf*> again_bufs;
      for (int32_t t = 0; t < T; ++t) again.emplace_back(c.numel[t]);
      for (int32_t t = 0; t < T; ++t) again_bufs.push_back(&again[t]);
      for (sbp::FanPiece& f : pieces) {
        int32_t owner = -1;
        for (int32_t t = 0; t < T; ++t)
          if (outs[t].holds(f.dst, f.len)) owner = t;
        CHECK(owner >= 0);
        f.dst = again[owner].p + (f.dst - outs[owner].p);
      }
      run_pieces(pieces, shard_ptrs, S, again_bufs, written);
      for (int32_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < c.numel[t]; ++i) CHECK(again[t].p[i] == outs[t].p[i]);
    }
  }

  // run tables: the groups over each shard start at 0, ascend, and fit
  std::vector<int32_t> tg(T > 0 ? T : 1);
  for (int32_t t = 0; t < T; ++t) tg[t] = static_cast<int32_t>(rng() % SBP_MAX_GROUPS);
  for (int32_t s = 0; s < c.N; ++s) {
    int64_t count = -1;
    CHECK(sbp_group_runs(p, s, tg.data(), nullptr, nullptr, 0, &count) == SBP_OK && count >= 1);
    std::vector<int64_t> starts(count);
    std::vector<int32_t> groups(count);
    const int64_t cap = count > 1 && rng() % 3 == 0 ? count - 1 : count;  // short on purpose
    CHECK(sbp_group_runs(p, s, tg.data(), starts.data(), groups.data(), cap, &count) == SBP_OK);
    CHECK(starts[0] == 0);
    for (int64_t k = 1; k < cap; ++k) CHECK(starts[k] > starts[k - 1] && starts[k] < S);
  }
  sbp_plan_free(p);
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 3000;
  for (int it = 0; it < iters; ++it) {
    Case c;
    c.kind = static_cast<int>(rng() % 3);
    c.N = rng() % 8 == 0 ? static_cast<int32_t>(std::vector<int>{8, 17, 64}[rng() % 3])
                         : 1 + static_cast<int32_t>(rng() % 5);
    c.align = static_cast<int32_t>(std::vector<int>{1, 2, 8}[rng() % 3]);
    c.cap = static_cast<int64_t>(std::vector<int>{2, 16, 64, 200, 1 << 20}[rng() % 5]);
    const int32_t T = static_cast<int32_t>(rng() % 9);
    for (int32_t t = 0; t < T; ++t) {
      const int64_t row = std::vector<int>{1, 2, 3, 7, 8}[rng() % 5];
      c.rows.push_back(row);
      c.numel.push_back(row * static_cast<int64_t>(rng() % 40));
    }
    one_case(c);
  }
  // invalid calls list nothing
  {
    Case c;
    c.numel = {10, 20};
    c.rows = {1, 1};
    sbp_plan* p = make(c);
    std::vector<sbp::Seg> segs(3);
    alignas(16) uint16_t buf[256];
    // tensor 1 comes first in flat order and is listed before tensor 0's
    // null pointer is found: the partial list must not come back
    const void* srcs[2] = {nullptr, buf + 128};
    CHECK(sbp::pack_segments(p, -1, srcs, buf, segs) == SBP_EINVAL && segs.empty());
    segs.resize(2);
    CHECK(sbp::shard_of_segments(p, 5, 0, buf, buf + 128, segs) == SBP_EINVAL && segs.empty());
    // tensor 1's segments are listed before tensor 0's null parameter is found
    const void* shard_list[1] = {buf};
    void* params[2] = {nullptr, buf + 128};
    segs.resize(2);
    CHECK(sbp::unpack_shards_segments(p, -1, shard_list, params, segs) == SBP_EINVAL &&
          segs.empty());
    // a parameter on top of a shard
    void* clash[2] = {buf + 200, buf + 8};
    CHECK(sbp::unpack_shards_segments(p, -1, shard_list, clash, segs) == SBP_EINVAL &&
          segs.empty());
    sbp_plan_free(p);
  }
  // long fans are cut into pieces of at most kFanPiece positions that resume
  // where the one before stopped; a chunk beyond 32 bits, or more ranks than
  // the kernel arguments hold, makes no pieces (nothing is executed here)
  {
    uint16_t* far = reinterpret_cast<uint16_t*>(uintptr_t{1} << 40);
    const int64_t chunk = (int64_t{3} << 29) + 8, len = 5 * chunk + 100;
    std::vector<sbp::Fan> fans = {sbp::Fan{64, chunk, 8, len, far}};
    std::vector<sbp::FanPiece> pieces;
    CHECK(sbp::fan_pieces(fans, 8, pieces));
    int64_t off = 0;
    for (const sbp::FanPiece& f : pieces) {
      const int64_t x = 8 + off;
      CHECK(f.dst == far + off && f.shard_off == 64 && f.chunk == chunk);
      CHECK(f.s0 == x / chunk && f.j0 == x % chunk && f.len <= sbp::kFanPiece && f.len > 0);
      CHECK(f.vec == 1 && static_cast<uint64_t>(f.j0) + f.len < (uint64_t{1} << 32));
      off += f.len;
    }
    CHECK(off == len && pieces.size() == static_cast<size_t>((len + sbp::kFanPiece - 1) / sbp::kFanPiece));
    CHECK(!sbp::fan_pieces(fans, sbp::kMaxFanRanks + 1, pieces) && pieces.empty());
    fans[0].chunk = int64_t{1} << 31;
    CHECK(!sbp::fan_pieces(fans, 8, pieces) && pieces.empty());
    fans[0].chunk = 12;  // not a multiple of 8: element by element
    fans[0].len = 30;
    CHECK(sbp::fan_pieces(fans, 8, pieces) && pieces.size() == 1 && pieces[0].vec == 0);
  }
  printf("layout cases %d ok\n", iters);
  return 0;
}
