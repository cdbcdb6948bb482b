// Spread arena: device arrays for one rank's shard step (the optimizer state
// and the peer receive buffers) whose physical pages are spread evenly over
// the device memory, built on HIP's virtual-memory calls.
//
// Why.  The fused step streams 12 arrays at the same element offset at
// once.  On MI355X the rate of that mix depends on where the arrays sit
// physically: with the arrays packed into one region of HBM it runs near 69%
// of 8 TB/s, while the same kernel on arrays whose pages are spread over the
// whole HBM runs near 76% (and a write-only pass 78% -> 92%).  Measured with
// a zero-arithmetic probe of the same traffic, over 40+ placements: the
// layout inside a region does not matter, only how widely the pages are
// spread.  A caller can build its state the ordinary way; this arena is the
// placement the library recommends for it.
//
// How.  Every array gets its own virtual range.  Physical chunks of
// `chunk_bytes` are then created one after another over `spread_bytes` of
// device memory (the driver hands them out in address order), every k-th is
// kept so the kept ones are evenly spaced over that span, and they are mapped
// to the arrays' chunk slots in a seeded random order; the chunks not kept
// are released at once.  No timing is involved: the policy is fixed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <string>
#include <vector>

#include "internal.h"

struct sbp_arena {
  int device = -1;
  int64_t chunk = 0;
  int64_t spread_chunks = 0;
  std::vector<void*> base;
  std::vector<int64_t> reserved;  // bytes of each virtual range (0: none)
  std::vector<std::pair<void*, int64_t>> mapped;  // mapped pieces
  std::vector<hipMemGenericAllocationHandle_t> kept;
};

namespace {

constexpr int64_t kTwoMiB = int64_t{2} << 20;
constexpr int64_t kDefaultChunk = int64_t{64} << 20;
// Chunks one arena may create while spreading (and hold): the driver's
// per-process mapping budget is of the order of 40,000 chunks.
constexpr int64_t kMaxSpreadChunks = 8192;
constexpr int64_t kMaxKeptChunks = 16384;

// splitmix64 (Steele, Lea and Flood, OOPSLA 2014): a seeded stream of 64-bit
// values for the shuffle below.
uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Uniform integer in [0, m) (m >= 1) by rejection, so every permutation of
// the Fisher-Yates shuffle is equally likely.
uint64_t below(uint64_t& s, uint64_t m) {
  const uint64_t limit = UINT64_MAX - UINT64_MAX % m;
  uint64_t x;
  do x = splitmix64(s);
  while (x >= limit);
  return x % m;
}

// HIP keeps a failed call's error as the thread's last error, where the next
// unrelated launch check (the library's, or the caller's own) would report
// it.  The arena reports its failures through its status and message, so it
// clears that state after a failed call it has handled.
void clear_hip_error() { (void)hipGetLastError(); }

void release_all(sbp_arena* a, std::vector<hipMemGenericAllocationHandle_t>& loose) {
  for (auto& p : a->mapped) (void)hipMemUnmap(p.first, static_cast<size_t>(p.second));
  a->mapped.clear();
  for (auto h : a->kept) (void)hipMemRelease(h);
  a->kept.clear();
  for (auto h : loose) (void)hipMemRelease(h);
  loose.clear();
  for (size_t i = 0; i < a->base.size(); ++i)
    if (a->base[i] != nullptr)
      (void)hipMemAddressFree(a->base[i], static_cast<size_t>(a->reserved[i]));
  a->base.clear();
  a->reserved.clear();
  clear_hip_error();
}

sbp_status hip_fail(const char* what, hipError_t e) {
  return sbp::fail(e == hipErrorOutOfMemory ? SBP_ENOMEM : SBP_EHIP,
                   std::string("sbp_arena_create: ") + what + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

sbp_status sbp_arena_create(const int64_t* bytes, int32_t n_arrays, int64_t chunk_bytes,
                            int64_t spread_bytes, uint64_t seed, void** ptrs, sbp_arena** out) {
  if (bytes == nullptr || ptrs == nullptr || out == nullptr)
    return sbp::fail(SBP_EINVAL, "sbp_arena_create: null argument");
  if (n_arrays < 1 || n_arrays > SBP_ARENA_MAX_ARRAYS)
    return sbp::fail(SBP_EINVAL, "sbp_arena_create: n_arrays must be in 1..64");
  if (chunk_bytes == 0) chunk_bytes = kDefaultChunk;
  if (chunk_bytes < 0 || chunk_bytes % kTwoMiB != 0)
    return sbp::fail(SBP_EINVAL, "sbp_arena_create: chunk_bytes must be a multiple of 2 MiB");
  if (spread_bytes < 0) return sbp::fail(SBP_EINVAL, "sbp_arena_create: spread_bytes < 0");
  int64_t need = 0;
  for (int32_t i = 0; i < n_arrays; ++i) {
    if (bytes[i] < 0) return sbp::fail(SBP_EINVAL, "sbp_arena_create: negative array size");
    const int64_t c = bytes[i] / chunk_bytes + (bytes[i] % chunk_bytes != 0);
    if (c > kMaxKeptChunks || (need += c) > kMaxKeptChunks)
      return sbp::fail(SBP_ERANGE, "sbp_arena_create: more than 16384 chunks; use a larger "
                                   "chunk_bytes");
  }
  *out = nullptr;

  sbp_arena* a = new (std::nothrow) sbp_arena;
  if (a == nullptr) return sbp::fail(SBP_ENOMEM, "sbp_arena_create: host allocation failed");
  std::vector<hipMemGenericAllocationHandle_t> loose;
  auto bail = [&](sbp_status st) {
    release_all(a, loose);
    delete a;
    return st;
  };
  hipError_t e = hipGetDevice(&a->device);
  if (e != hipSuccess) return bail(hip_fail("hipGetDevice", e));
  int vmm = 0;
  e = hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, a->device);
  if (e != hipSuccess || vmm == 0)
    return bail(sbp::fail(SBP_EHIP, "sbp_arena_create: the device has no virtual memory "
                                    "management"));
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = a->device;
  size_t gran = 0;
  e = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum);
  if (e != hipSuccess) return bail(hip_fail("hipMemGetAllocationGranularity", e));
  if (gran == 0 || chunk_bytes % static_cast<int64_t>(gran) != 0)
    return bail(sbp::fail(SBP_EINVAL, "sbp_arena_create: chunk_bytes is not a multiple of the "
                                      "device's allocation granularity"));
  a->chunk = chunk_bytes;

  // the span to spread over, in chunks: all free memory less a reserve of
  // 1/32 (at least 1 GiB) unless the caller names it; never below the need
  int64_t avail = 0;
  if (spread_bytes > 0) {
    avail = spread_bytes / chunk_bytes;
  } else {
    size_t fr = 0, tot = 0;
    e = hipMemGetInfo(&fr, &tot);
    if (e != hipSuccess) return bail(hip_fail("hipMemGetInfo", e));
    int64_t reserve = static_cast<int64_t>(tot / 32);
    if (reserve < (int64_t{1} << 30)) reserve = int64_t{1} << 30;
    const int64_t usable = static_cast<int64_t>(fr) - reserve;
    avail = usable > 0 ? usable / chunk_bytes : 0;
  }
  if (avail > kMaxSpreadChunks) avail = kMaxSpreadChunks;
  if (avail < need) avail = need;
  if (need == 0) avail = 0;

  // virtual ranges, one per array
  a->base.assign(n_arrays, nullptr);
  a->reserved.assign(n_arrays, 0);
  std::vector<std::pair<int32_t, int64_t>> slots;  // (array, chunk index)
  slots.reserve(static_cast<size_t>(need));
  for (int32_t i = 0; i < n_arrays; ++i) {
    const int64_t c = bytes[i] / chunk_bytes + (bytes[i] % chunk_bytes != 0);
    ptrs[i] = nullptr;
    if (c == 0) continue;
    void* b = nullptr;
    e = hipMemAddressReserve(&b, static_cast<size_t>(c * chunk_bytes),
                             static_cast<size_t>(chunk_bytes), nullptr, 0);
    if (e != hipSuccess) return bail(hip_fail("hipMemAddressReserve", e));
    a->base[i] = b;
    a->reserved[i] = c * chunk_bytes;
    for (int64_t s = 0; s < c; ++s) slots.push_back({i, s});
  }

  // physical chunks in creation order; stop early (keeping what exists) if
  // the memory runs out after enough chunks for the arrays
  loose.reserve(static_cast<size_t>(avail));
  for (int64_t k = 0; k < avail; ++k) {
    hipMemGenericAllocationHandle_t h;
    e = hipMemCreate(&h, static_cast<size_t>(chunk_bytes), &prop, 0);
    if (e != hipSuccess) {
      if (k >= need) {  // enough for the arrays: spread over what exists
        clear_hip_error();
        break;
      }
      return bail(hip_fail("hipMemCreate", e));
    }
    loose.push_back(h);
  }
  a->spread_chunks = static_cast<int64_t>(loose.size());

  // seeded Fisher-Yates shuffle of the slots
  uint64_t st = seed;
  for (size_t i = slots.size(); i > 1; --i) {
    const size_t j = static_cast<size_t>(below(st, i));
    std::swap(slots[i - 1], slots[j]);
  }
  // kept chunk k = created chunk floor(k * created / need), mapped to slots[k]
  const int64_t created = a->spread_chunks;
  std::vector<char> is_kept(static_cast<size_t>(created), 0);
  for (int64_t k = 0; k < need; ++k) {
    const int64_t idx = static_cast<int64_t>((static_cast<unsigned __int128>(k) * created) /
                                             static_cast<unsigned __int128>(need));
    is_kept[idx] = 1;
    char* at = static_cast<char*>(a->base[slots[k].first]) + slots[k].second * chunk_bytes;
    e = hipMemMap(at, static_cast<size_t>(chunk_bytes), 0, loose[idx], 0);
    if (e != hipSuccess) return bail(hip_fail("hipMemMap", e));
    a->mapped.push_back({at, chunk_bytes});
  }
  std::vector<hipMemGenericAllocationHandle_t> rest;
  for (int64_t i = 0; i < created; ++i) {
    if (is_kept[i]) a->kept.push_back(loose[i]);
    else rest.push_back(loose[i]);
  }
  loose.swap(rest);
  for (auto h : loose) (void)hipMemRelease(h);
  loose.clear();

  hipMemAccessDesc acc = {};
  acc.location.type = hipMemLocationTypeDevice;
  acc.location.id = a->device;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  for (int32_t i = 0; i < n_arrays; ++i) {
    if (a->base[i] == nullptr) continue;
    e = hipMemSetAccess(a->base[i], static_cast<size_t>(a->reserved[i]), &acc, 1);
    if (e != hipSuccess) return bail(hip_fail("hipMemSetAccess", e));
  }
  for (int32_t i = 0; i < n_arrays; ++i) ptrs[i] = a->base[i];
  *out = a;
  return sbp::ok();
}

sbp_status sbp_arena_info(const sbp_arena* a, int64_t* chunk_bytes, int64_t* chunks_kept,
                          int64_t* chunks_spread) {
  if (a == nullptr) return sbp::fail(SBP_EINVAL, "sbp_arena_info: null arena");
  if (chunk_bytes) *chunk_bytes = a->chunk;
  if (chunks_kept) *chunks_kept = static_cast<int64_t>(a->kept.size());
  if (chunks_spread) *chunks_spread = a->spread_chunks;
  return sbp::ok();
}

sbp_status sbp_arena_free(sbp_arena* a) {
  if (a == nullptr) return sbp::ok();
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess && cur != a->device) e = hipSetDevice(a->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();  // no kernel may still use the memory
  std::vector<hipMemGenericAllocationHandle_t> none;
  release_all(a, none);
  delete a;
  if (cur >= 0) (void)hipSetDevice(cur);
  if (e != hipSuccess)
    return sbp::fail(SBP_EHIP, std::string("sbp_arena_free: ") + hipGetErrorString(e));
  return sbp::ok();
}

}  // extern "C"
