/* A plain C99 client of libsbp: no Python, no torch, only include/sbp.h and
 * the HIP runtime's C API.  It shows the boundary stands on its own.
 *
 *   abi_c plan CAP N ALIGN FLAGS NUMEL...
 *       Host only.  Builds a plan and prints every query's answer, one
 *       record per line, then checks that a bad argument comes back as
 *       SBP_EINVAL with a message.
 *
 *   abi_c step IN OUT
 *       One fused step on the GPU.  IN holds, little-endian and packed:
 *         int64 n, int32 R, int32 with_acc, float scale,
 *         float lr, beta1, beta2, eps, weight_decay, int64 step,
 *         R x n uint16 peers, [n float acc], n float master, m, v.
 *       OUT receives n float master, m, v, then n uint16 params.
 *
 * Exit status 0 on success; any failure prints its reason and exits 1. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sbp.h"

static int fail(const char* what) {
  fprintf(stderr, "abi_c: %s\n", what);
  return 1;
}

static int run_plan(int argc, char** argv) {
  if (argc < 7) return fail("plan needs CAP N ALIGN FLAGS and at least one numel");
  const int64_t cap = strtoll(argv[2], NULL, 10);
  const int32_t world_n = (int32_t)strtol(argv[3], NULL, 10);
  const int32_t align = (int32_t)strtol(argv[4], NULL, 10);
  const uint32_t flags = (uint32_t)strtoul(argv[5], NULL, 10);
  const int32_t T = argc - 6;
  int64_t* numel = (int64_t*)malloc(sizeof(int64_t) * (size_t)T);
  if (!numel) return fail("out of host memory");
  for (int32_t t = 0; t < T; ++t) numel[t] = strtoll(argv[6 + t], NULL, 10);

  sbp_plan* plan = NULL;
  sbp_status st = sbp_bucket_plan(numel, T, cap, world_n, align, flags, &plan);
  if (st != SBP_OK) {
    fprintf(stderr, "abi_c: sbp_bucket_plan: %d %s\n", st, sbp_last_error());
    free(numel);
    return 1;
  }
  const int32_t B = sbp_plan_num_buckets(plan);
  printf("plan %d %d %d %lld %lld\n", sbp_plan_num_tensors(plan), B, sbp_plan_world_n(plan),
         (long long)sbp_plan_shard_numel(plan), (long long)sbp_plan_flat_numel(plan));
  for (int32_t t = 0; t < T; ++t) {
    int32_t b = -1;
    int64_t off = -1;
    if (sbp_plan_tensor(plan, t, &b, &off) != SBP_OK) return fail("sbp_plan_tensor");
    printf("tensor %d %d %lld\n", t, b, (long long)off);
  }
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
  if (!ids) return fail("out of host memory");
  for (int32_t b = 0; b < B; ++b) {
    int64_t used, padded, chunk, shard_off, flat_off;
    if (sbp_plan_bucket(plan, b, &used, &padded, &chunk, &shard_off, &flat_off) != SBP_OK)
      return fail("sbp_plan_bucket");
    int32_t count = 0;
    if (sbp_plan_bucket_tensors(plan, b, ids, T, &count) != SBP_OK || count > T)
      return fail("sbp_plan_bucket_tensors");
    printf("bucket %d %lld %lld %lld %lld %lld", b, (long long)used, (long long)padded,
           (long long)chunk, (long long)shard_off, (long long)flat_off);
    for (int32_t i = 0; i < count; ++i) printf(" %d", ids[i]);
    printf("\n");
  }
  for (int32_t stage = 0; stage < 4; ++stage) {
    int64_t bytes = -1;
    if (sbp_plan_state_bytes(plan, stage, &bytes) != SBP_OK) return fail("sbp_plan_state_bytes");
    printf("state %d %lld\n", stage, (long long)bytes);
  }
  sbp_plan_free(plan);
  free(ids);

  /* errors come back as codes with a message, and leave *out null */
  sbp_plan* bad = (sbp_plan*)&st; /* any non-null value */
  st = sbp_bucket_plan(numel, T, 0, world_n, align, flags, &bad);
  free(numel);
  if (st != SBP_EINVAL || bad != NULL || sbp_last_error()[0] == '\0')
    return fail("a zero bucket cap was not reported as SBP_EINVAL");
  printf("einval %s\n", sbp_last_error()[0] ? "message" : "none");
  return 0;
}

static int read_all(FILE* f, void* dst, size_t bytes) {
  return fread(dst, 1, bytes, f) == bytes ? 0 : 1;
}

#define HIP_OK(call)                                                         \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "abi_c: %s: %s\n", #call, hipGetErrorString(e_));      \
      return 1;                                                              \
    }                                                                        \
  } while (0)

/* One fused step on the input file's arrays.  use_arena: every device array
 * from one spread arena (sbp_arena_create) instead of hipMalloc, and this
 * rank's squared norm of the step's gradient taken first with the
 * allocation-free call (appended to the output). */
static int run_step(const char* in_path, const char* out_path, int use_arena) {
  FILE* f = fopen(in_path, "rb");
  if (!f) return fail("cannot open the input file");
  int64_t n = 0;
  int32_t R = 0, with_acc = 0;
  float scale = 0.0f;
  sbp_adamw_hparams hp;
  memset(&hp, 0, sizeof hp);
  if (read_all(f, &n, 8) || read_all(f, &R, 4) || read_all(f, &with_acc, 4) ||
      read_all(f, &scale, 4) || read_all(f, &hp.lr, 4) || read_all(f, &hp.beta1, 4) ||
      read_all(f, &hp.beta2, 4) || read_all(f, &hp.eps, 4) || read_all(f, &hp.weight_decay, 4) ||
      read_all(f, &hp.step, 8))
    return fail("short header");
  if (n < 1 || n > ((int64_t)1 << 28) || R < 0 || R > SBP_MAX_PEERS) return fail("bad header");

  const size_t nb2 = (size_t)n * 2, nb4 = (size_t)n * 4;
  /* host: peers, acc, master, m, v, params */
  unsigned char* host = (unsigned char*)malloc(nb2 * (size_t)R + nb4 * 4 + nb2);
  if (!host) return fail("out of host memory");
  unsigned char* h_peers = host;
  unsigned char* h_acc = h_peers + nb2 * (size_t)R;
  unsigned char* h_state = h_acc + nb4;   /* master, m, v */
  unsigned char* h_param = h_state + 3 * nb4;
  if (read_all(f, h_peers, nb2 * (size_t)R) || (with_acc && read_all(f, h_acc, nb4)) ||
      read_all(f, h_state, 3 * nb4))
    return fail("short body");
  fclose(f);

  void* d_peer[SBP_MAX_PEERS] = {0};
  void *d_acc = NULL, *d_master = NULL, *d_m = NULL, *d_v = NULL, *d_param = NULL, *d_sq = NULL;
  sbp_arena* arena = NULL;
  if (use_arena) {
    /* peers, acc (maybe empty), master, m, v, param, the squared norm */
    int64_t bytes[SBP_MAX_PEERS + 6];
    void* ptr[SBP_MAX_PEERS + 6];
    int32_t k = 0;
    for (int32_t r = 0; r < R; ++r) bytes[k++] = (int64_t)nb2;
    bytes[k++] = with_acc ? (int64_t)nb4 : 0;
    bytes[k++] = (int64_t)nb4;
    bytes[k++] = (int64_t)nb4;
    bytes[k++] = (int64_t)nb4;
    bytes[k++] = (int64_t)nb2;
    bytes[k++] = 8;
    const sbp_status st = sbp_arena_create(bytes, k, (int64_t)2 << 20, (int64_t)512 << 20, 7,
                                           ptr, &arena);
    if (st != SBP_OK) {
      fprintf(stderr, "abi_c: sbp_arena_create: %d %s\n", st, sbp_last_error());
      return 1;
    }
    for (int32_t r = 0; r < R; ++r) d_peer[r] = ptr[r];
    d_acc = ptr[R];
    d_master = ptr[R + 1];
    d_m = ptr[R + 2];
    d_v = ptr[R + 3];
    d_param = ptr[R + 4];
    d_sq = ptr[R + 5];
  } else {
    for (int32_t r = 0; r < R; ++r) HIP_OK(hipMalloc(&d_peer[r], nb2));
    if (with_acc) HIP_OK(hipMalloc(&d_acc, nb4));
    HIP_OK(hipMalloc(&d_master, nb4));
    HIP_OK(hipMalloc(&d_m, nb4));
    HIP_OK(hipMalloc(&d_v, nb4));
    HIP_OK(hipMalloc(&d_param, nb2));
  }
  for (int32_t r = 0; r < R; ++r)
    HIP_OK(hipMemcpy(d_peer[r], h_peers + nb2 * (size_t)r, nb2, hipMemcpyHostToDevice));
  if (with_acc) HIP_OK(hipMemcpy(d_acc, h_acc, nb4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_master, h_state, nb4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_m, h_state + nb4, nb4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_v, h_state + 2 * nb4, nb4, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  if (use_arena) {
    const sbp_status sn = sbp_grad_sq_norm_noalloc((const void* const*)d_peer, R,
                                                   (const float*)d_acc, scale, n, NULL,
                                                   (double*)d_sq, stream);
    if (sn != SBP_OK) {
      fprintf(stderr, "abi_c: sbp_grad_sq_norm_noalloc: %d %s\n", sn, sbp_last_error());
      return 1;
    }
  }
  const sbp_status st = sbp_adamw_shard((const void* const*)d_peer, R, (const float*)d_acc, scale,
                                        (float*)d_master, (float*)d_m, (float*)d_v, d_param, n,
                                        &hp, stream);
  if (st != SBP_OK) {
    fprintf(stderr, "abi_c: sbp_adamw_shard: %d %s\n", st, sbp_last_error());
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipStreamDestroy(stream));

  HIP_OK(hipMemcpy(h_state, d_master, nb4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_state + nb4, d_m, nb4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_state + 2 * nb4, d_v, nb4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_param, d_param, nb2, hipMemcpyDeviceToHost));
  double sq = 0.0;
  if (use_arena) {
    HIP_OK(hipMemcpy(&sq, d_sq, 8, hipMemcpyDeviceToHost));
    const sbp_status sf = sbp_arena_free(arena);
    if (sf != SBP_OK) {
      fprintf(stderr, "abi_c: sbp_arena_free: %d %s\n", sf, sbp_last_error());
      return 1;
    }
  } else {
    for (int32_t r = 0; r < R; ++r) HIP_OK(hipFree(d_peer[r]));
    if (d_acc) HIP_OK(hipFree(d_acc));
    HIP_OK(hipFree(d_master));
    HIP_OK(hipFree(d_m));
    HIP_OK(hipFree(d_v));
    HIP_OK(hipFree(d_param));
  }

  FILE* o = fopen(out_path, "wb");
  if (!o) return fail("cannot open the output file");
  if (fwrite(h_state, 1, 3 * nb4 + nb2, o) != 3 * nb4 + nb2) return fail("short write");
  if (use_arena && fwrite(&sq, 1, 8, o) != 8) return fail("short write");
  fclose(o);
  free(host);
  printf("step %lld done\n", (long long)n);
  return 0;
}

int main(int argc, char** argv) {
  printf("%s\n", sbp_version());
  if (argc >= 2 && strcmp(argv[1], "plan") == 0) return run_plan(argc, argv);
  if (argc == 4 && strcmp(argv[1], "step") == 0) return run_step(argv[2], argv[3], 0);
  if (argc == 4 && strcmp(argv[1], "arena_step") == 0) return run_step(argv[2], argv[3], 1);
  return fail("usage: abi_c plan CAP N ALIGN FLAGS NUMEL... | abi_c step|arena_step IN OUT");
}
