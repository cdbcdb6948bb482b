/*
 * sbp.h -- one data-parallel rank's gradient-sync and sharded-optimizer hot
 * path on an AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The path, per optimizer step:
 *   1. bucket plan      per-parameter offsets in flat gradient buckets, each
 *                       bucket split into N equal chunks, one per rank
 *   2. pack             per-tensor bf16 gradients copied into the buckets
 *   3. reduce           this rank's reduce-scatter share: R peer bf16 chunks
 *                       summed in fp32 in ascending rank order
 *   4. normalise        one fp32 multiply by 1/(R*K) or 1/global_token_count
 *   5. accumulate       fp32 accumulation over microbatches
 *   6. AdamW + emit     mixed-precision AdamW on the owned shard (fp32 master,
 *                       m, v) and the updated bf16 parameter shard written
 *                       out for the all-gather
 * Steps 3-6 of the last microbatch run as one fused streaming kernel.
 *
 * Sources (public pages on data-parallel training):
 *   "Parallelisms" (vladislavkruglikov.com/articles/parallelisms), sections
 *     Data parallel, Gradient bucketing, ZeRO-1, ZeRO-2, ZeRO-3, FSDP /
 *     Flat parameter;
 *   "Distributed Training and Parallelism" (naatyu.github.io/atlas/training/
 *     parallelism), sections "Data parallelism and the global gradient",
 *     "ZeRO and sharded state";
 *   "Parallelism Starts With the Bottleneck" (rajdeepmondal.com), sections
 *     "Allreduce equals reducescatter plus allgather", "Data parallelism is
 *     simple and pays for it in memory", "ZeRO removes the copies without
 *     adding bandwidth".
 *
 * Conventions for every call below:
 *   - Return value: SBP_OK or a negative status; sbp_last_error() then holds
 *     a message for the calling thread.  Invalid arguments are reported
 *     before anything is enqueued; nothing is written on error.
 *   - n == 0 (after the count and hyperparameter checks) returns SBP_OK
 *     without reading any pointer or launching anything.
 *   - Device pointers are caller-owned device (HBM) memory.  No call
 *     allocates or frees device memory, except the spread arena's
 *     (sbp_arena_create / sbp_arena_free), whose purpose that is.  Host
 *     arrays are read during the call only.
 *   - Device calls validate on the host, enqueue on `stream` and return;
 *     a fault in a kernel surfaces at the caller's next synchronisation.
 *   - Before it launches, a device call reads and clears the calling
 *     thread's last HIP error (hipGetLastError), so that SBP_EHIP reports a
 *     launch of its own.  A caller that checks hipGetLastError for its own
 *     earlier launches does so before calling into the library.
 *   - bf16 values are passed as their 16-bit patterns (uint16 storage).
 *   - Arithmetic is IEEE binary32 with one round-to-nearest-even rounding per
 *     operation (no fused multiply-add), subnormals kept; a sum over peers
 *     starts from peer 0's value and adds peers 1..R-1 in that order.  Results
 *     are therefore fully determined by the inputs.
 */
#ifndef SBP_H
#define SBP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sbp_status;
#define SBP_OK 0
#define SBP_EINVAL (-1) /* bad argument: null pointer, bad size/count/index  */
#define SBP_EALIGN (-2) /* a pointer lacks the alignment the call requires   */
#define SBP_ERANGE (-3) /* a size overflows int64 or a documented maximum    */
#define SBP_EHIP (-4)   /* the HIP runtime refused a launch                  */
#define SBP_ENOMEM (-5) /* host allocation failed                            */

#define SBP_MAX_PEERS 16 /* largest R accepted by the reduce-type calls */
/* Largest n of one reduce, accumulate, fused-step or squared-norm call:
 * one launch covers the whole range with one 256-lane block per 2048
 * elements, and a launch holds at most 2^32 - 1 work-items, so at most
 * 2^24 - 1 blocks.  Larger shards are stepped in ranges (the calls are
 * elementwise; a range's pointers are the shard's plus its offset). */
#define SBP_MAX_SHARD_NUMEL 34359736320LL /* (2^24 - 1) * 2048 */
#define SBP_MAX_GROUPS 8 /* parameter groups of the grouped AdamW step    */

/* Message for the last failed call on this thread ("" if none). */
const char* sbp_last_error(void);
/* Library version string. */
const char* sbp_version(void);

/* ------------------------------------------------------------------------
 * Bucket plan (host only).
 *
 * "Parallelisms", Gradient bucketing: gradients are collected into buffers
 * that are communicated once ready; Data parallel: buckets for later layers
 * are ready first during backward; FSDP / Flat parameter: a bucket is one
 * contiguous buffer that concatenates parameters; ZeRO-2: each ready bucket
 * is reduce-scattered and each rank keeps the 1/N shard it owns.
 *
 * Rule (readings where the pages are silent):
 *   - tensors are visited in reverse registration order (SBP_ORDER_REVERSE,
 *     the default) or in registration order (SBP_ORDER_FORWARD);
 *   - a tensor is added to the open bucket at the first multiple of
 *     align_elems at or after the bucket's used length (the first tensor at
 *     0); the bucket closes once 2*used >= bucket_cap_bytes (the cap counts
 *     bf16 gradient bytes); tensors are never split, so a bucket may exceed
 *     the cap by its last tensor and a tensor larger than the cap forms its
 *     own bucket; the last open bucket closes at the end;
 *   - each bucket is zero-padded to a multiple of align_elems * world_n
 *     elements and split into world_n equal chunks; rank s owns chunk s of
 *     every bucket, and its shard is those chunks in bucket order.
 *
 * With SBP_SPLIT_TENSORS the buckets are instead fixed-size pieces of the
 * flat buffer: tensors are concatenated (each at the first multiple of
 * align_elems after the previous one, in visit order) and cut into buckets
 * of bucket_cap_bytes/2 elements rounded down to a multiple of
 * align_elems * world_n (at least that); a tensor may straddle buckets, and
 * only the last bucket can be short (then padded as above).
 *
 * numel[n_tensors]   element counts in registration order (>= 0 each)
 * bucket_cap_bytes   > 0
 * world_n            shard divisor N, > 0
 * align_elems        power of two, 1..4096 (8 keeps every chunk 16-B aligned)
 * flags              SBP_ORDER_REVERSE (0) or SBP_ORDER_FORWARD, optionally
 *                    | SBP_SPLIT_TENSORS
 * out                receives an immutable plan; free with sbp_plan_free.
 *                    A plan is read-only after creation and may be shared
 *                    between threads.
 * Errors: SBP_EINVAL (null, n_tensors < 0, negative numel, bad cap/N/align/
 * flags), SBP_ERANGE (a flat size beyond 2^62 elements (2^61 split), or a
 * split plan of more than 2^24 buckets), SBP_ENOMEM.
 * ---------------------------------------------------------------------- */
typedef struct sbp_plan sbp_plan;

#define SBP_ORDER_REVERSE 0u
#define SBP_ORDER_FORWARD 1u
#define SBP_SPLIT_TENSORS 2u

sbp_status sbp_bucket_plan(const int64_t* numel, int32_t n_tensors,
                           int64_t bucket_cap_bytes, int32_t world_n,
                           int32_t align_elems, uint32_t flags,
                           sbp_plan** out);
void sbp_plan_free(sbp_plan* plan);

/* One bucket per tensor, every rank owning whole rows of it ("Parallelisms",
 * FSDP: FSDP2 shards each parameter in place on dim 0, keeping parameter
 * identities).  Tensor t (visit order per flags: SBP_ORDER_REVERSE or
 * SBP_ORDER_FORWARD) is its own bucket, padded to a multiple of
 * world_n * lcm(align_elems, row_elems[t]); rank s's chunk is then
 * ceil(numel / (N * unit)) * unit elements -- whole rows, aligned.
 * row_elems: elements per dim-0 row, or null for 1 (a 1-D view); numel[t]
 * must be a multiple of it.  Queries and every other call work on the
 * result as on any plan.  Errors: SBP_EINVAL, SBP_ERANGE, SBP_ENOMEM. */
sbp_status sbp_bucket_plan_per_tensor(const int64_t* numel,
                                      const int64_t* row_elems,
                                      int32_t n_tensors, int32_t world_n,
                                      int32_t align_elems, uint32_t flags,
                                      sbp_plan** out);

/* Plan queries.  Counts and offsets are in elements. */
int32_t sbp_plan_num_tensors(const sbp_plan* plan);
int32_t sbp_plan_num_buckets(const sbp_plan* plan);
int32_t sbp_plan_world_n(const sbp_plan* plan);
/* Elements of one rank's shard (the same for every rank). */
int64_t sbp_plan_shard_numel(const sbp_plan* plan);
/* Elements of the flat buffer holding all buckets (= N * shard numel). */
int64_t sbp_plan_flat_numel(const sbp_plan* plan);
/* Tensor t's bucket and its offset inside the bucket (for a split plan: the
 * bucket holding its first element). */
sbp_status sbp_plan_tensor(const sbp_plan* plan, int32_t t, int32_t* bucket,
                           int64_t* offset);
/* Bucket b: used length, padded length, chunk (= padded / N), start of its
 * chunk in a rank's shard, start of the bucket in the flat buffer.  Any of
 * the output pointers may be null. */
sbp_status sbp_plan_bucket(const sbp_plan* plan, int32_t b, int64_t* used,
                           int64_t* padded, int64_t* chunk,
                           int64_t* shard_offset, int64_t* flat_offset);
/* Tensor ids of bucket b in the order they were placed (for a split plan:
 * every tensor with an element in the bucket); writes up to `cap` ids and
 * returns the bucket's tensor count in *count. */
sbp_status sbp_plan_bucket_tensors(const sbp_plan* plan, int32_t b,
                                   int32_t* ids, int32_t cap, int32_t* count);
/* Persistent model-state bytes per rank: bf16 params (2) + bf16 grads (2) +
 * fp32 master, m, v (12) per parameter, with stage 0 = plain DP (all
 * replicated), 1 = optimizer state sharded, 2 = + gradients, 3 = + params
 * ("Parallelism Strategies in Distributed Computing", Cost per strategy and
 * ZeRO and FSDP; "Parallelism Starts With the Bottleneck", memory section).
 * Counted over the padded flat buffer; activations and temporary buckets
 * are excluded.  Errors: SBP_EINVAL (null, stage outside 0..3). */
sbp_status sbp_plan_state_bytes(const sbp_plan* plan, int32_t zero_stage,
                                int64_t* per_rank_bytes);

/* ------------------------------------------------------------------------
 * Normalisation factors ("Distributed Training and Parallelism", Data
 * parallelism and the global gradient: average over R ranks, or scale by
 * R / global valid-token count; with the 1/R average that is 1/C).
 * Computed in float64 and rounded once to binary32.
 * ---------------------------------------------------------------------- */
/* *scale = fl32(1 / (R * K)).  Errors: SBP_EINVAL (null, R < 1, K < 1). */
sbp_status sbp_mean_scale(int32_t R, int32_t K, float* scale);
/* *scale = fl32(1 / sum(counts[0..R-1])).  Errors: SBP_EINVAL (null, R < 1,
 * a negative count, a zero total), SBP_ERANGE (the total overflows). */
sbp_status sbp_tokens_scale(const int64_t* counts, int32_t R, float* scale);

/* ------------------------------------------------------------------------
 * Pack ("Parallelisms", Gradient bucketing and FSDP: gradients gathered
 * into flat communication buffers at fixed offsets).
 *
 * Copies every tensor of bucket `bucket` (or of all buckets if bucket == -1)
 * bit for bit from tensor_grads[t] to flat[flat_offset_b + offset_t ...],
 * and writes +0 (0x0000) into every other element of those buckets.  With a
 * split plan only the part of a straddling tensor inside the selected
 * bucket(s) is copied.
 *
 * tensor_grads  host array of plan->n_tensors device pointers to bf16
 *               gradients (2-byte aligned); entries of tensors outside the
 *               selected bucket(s) are not read and may be null.  Sources
 *               that are 16-byte aligned take the vector path.
 * flat          device bf16 buffer of sbp_plan_flat_numel elements,
 *               16-byte aligned; must not overlap any source.
 * Errors: SBP_EINVAL (null plan/array/buffer, null source of a selected
 * tensor, bucket out of range), SBP_EALIGN (flat not 16-B aligned, a source
 * not 2-B aligned), SBP_EHIP.
 * ---------------------------------------------------------------------- */
sbp_status sbp_pack_grads(const sbp_plan* plan, int32_t bucket,
                          const void* const* tensor_grads, void* flat,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * The all-gather side and the local halves of the collectives
 * ("Parallelisms", ZeRO-1: a rank receives its owned shard of the summed
 * gradient from the reduce-scatter, and all-gathering the updated shards
 * gives every rank the whole model back; FSDP / Flat parameter: each
 * original parameter is a view into the flat buffer).  Same copy engine and conventions as pack (16-byte
 * vector path when both sides are 16-B aligned, element-wise otherwise; no
 * device allocation; bucket = -1 for all buckets).
 *
 * sbp_unpack_params: flat bf16 buckets -> per-tensor bf16 parameters: every
 *   tensor element inside the selected bucket(s) is copied to
 *   tensor_params[t]; padding is not read.  tensor_params is a host array of
 *   plan->n_tensors device pointers (2-B aligned; entries of tensors outside
 *   the selection are not read); they must not overlap each other or flat.
 * sbp_shard_of: chunk `rank` of every selected bucket of a flat buffer ->
 *   shard[shard_offset_b ...] (what rank `rank` owns; each rank's flat
 *   gradient buckets reduce into these shards).  flat: flat_numel elements,
 *   shard: shard_numel elements, both 16-B aligned, disjoint.
 * sbp_gather_shards: the N ranks' shards -> flat[flat_offset_b + s*chunk_b
 *   ...] for every selected bucket: the layout an all-gather of the bf16
 *   parameter shards produces.  shards: host array of N device pointers
 *   (16-B aligned, shard_numel elements each), disjoint from flat.
 * sbp_unpack_shards: the N ranks' shards -> per-tensor bf16 parameters in
 *   one pass: the same result as sbp_gather_shards into a flat buffer
 *   followed by sbp_unpack_params, without the flat buffer and its extra
 *   write and read ("Parallelisms", ZeRO-3: a layer's parameter shards are
 *   all-gathered just before it runs; YaFSDP: fewer memory operations
 *   around the collectives).  Each tensor element inside the selected
 *   bucket(s) is read from the shard of the rank that owns it; padding is
 *   not read.  shards as for sbp_gather_shards; tensor_params as for
 *   sbp_unpack_params, disjoint from each other and from every shard.
 * Errors: SBP_EINVAL (null, rank or bucket out of range, overlap),
 * SBP_EALIGN, SBP_ERANGE, SBP_EHIP.
 * ---------------------------------------------------------------------- */
sbp_status sbp_unpack_params(const sbp_plan* plan, int32_t bucket,
                             const void* flat, void* const* tensor_params,
                             hipStream_t stream);
sbp_status sbp_shard_of(const sbp_plan* plan, int32_t bucket, int32_t rank,
                        const void* flat, void* shard, hipStream_t stream);
sbp_status sbp_gather_shards(const sbp_plan* plan, int32_t bucket,
                             const void* const* shards, void* flat,
                             hipStream_t stream);
sbp_status sbp_unpack_shards(const sbp_plan* plan, int32_t bucket,
                             const void* const* shards,
                             void* const* tensor_params, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Reduce ("Parallelisms", ZeRO-1: reduce-scatter leaves each worker the
 * reduced gradient shard of the parameters it owns; "Distributed Training
 * and Parallelism": the reduction order changes the bits, so it is fixed).
 *
 * out[i] = fl( S[i] * scale ),  S[i] = fp32(p0[i]) + fp32(p1[i]) + ... in
 * ascending peer order, one rounding per addition.
 *
 * peers  host array of R device pointers to bf16 chunks of n elements
 * R      1..SBP_MAX_PEERS
 * out    device fp32[n]
 * All device pointers 16-byte aligned; out must not overlap a peer.
 * Errors: SBP_EINVAL, SBP_EALIGN, SBP_ERANGE (n > SBP_MAX_SHARD_NUMEL),
 * SBP_EHIP.
 * ---------------------------------------------------------------------- */
sbp_status sbp_reduce_shard(const void* const* peers, int32_t R, int64_t n,
                            float scale, float* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Accumulate ("Distributed Training and Parallelism": intermediate
 * reductions suppressed over microbatches, the last pass synchronises;
 * "Parallelisms", ZeRO-2: accumulation adds later microbatches' shards).
 *
 * acc[i] = S[i] if first != 0, else fl(acc[i] + S[i]); S as in reduce, no
 * scaling (the scale is applied once, in the fused step).  R = 1 is a
 * rank's local (no_sync) accumulation; R > 1 accumulates reduce-scattered
 * shards.  acc is read and written in place.
 * Errors: SBP_EINVAL, SBP_EALIGN, SBP_ERANGE (n > SBP_MAX_SHARD_NUMEL),
 * SBP_EHIP.
 * ---------------------------------------------------------------------- */
sbp_status sbp_accumulate_grads(float* acc, const void* const* peers,
                                int32_t R, int64_t n, int32_t first,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * Fused shard step: reduce + normalise + AdamW + bf16 emit, one pass.
 *
 * ("Parallelisms", ZeRO-1: each worker updates its owned shard with its
 * local optimizer state -- first and second moments, a step counter and an
 * fp32 master copy -- then the updated shards are all-gathered; ZeRO-3: the
 * same update on a persistent 1/N shard.)
 *
 * Per element i:
 *   G = acc[i] + S[i]   (acc given, R >= 1)   S = ascending peer sum
 *   G = S[i]            (acc null)
 *   G = acc[i]          (R == 0)
 *   g = fl(G * scale)
 *   m'  = b1*m + (1-b1)*g
 *   v'  = b2*v + (1-b2)*(g*g)
 *   d   = sqrt(v')*c2 + eps                  (sqrt correctly rounded)
 *   th' = th*decay - step_size*(m'/d)        (divide correctly rounded)
 *   master[i] = th', m[i] = m', v[i] = v', param_out[i] = bf16_rne(th')
 * with, per call, from the binary32 hyperparameters in float64, each rounded
 * once to binary32: bc1 = 1 - b1^t, bc2 = 1 - b2^t (powers by repeated
 * multiplication), step_size = lr/bc1, c2 = 1/sqrt(bc2), decay = 1 - lr*wd,
 * 1-b1 and 1-b2.  bf16_rne: nearest, ties to even; NaN stays NaN (sign
 * kept, quiet bit set); overflow to +-inf.
 *
 * peers      host array of R device bf16 pointers (unused if R == 0)
 * R          0..SBP_MAX_PEERS; 0 requires acc
 * acc        device fp32[n] or null
 * master,m,v device fp32[n], updated in place
 * param_out  device bf16[n] (the all-gather send buffer)
 * hp         hyperparameters; hp->step = t >= 1 (1-based, once per
 *            optimizer step, not per microbatch); beta1 and beta2 in
 *            [0, 1); lr, eps and weight_decay finite and >= 0 (the ranges
 *            torch.optim.AdamW accepts); SBP_EINVAL otherwise
 * All device pointers 16-byte aligned and pairwise non-overlapping.
 * Errors: SBP_EINVAL, SBP_EALIGN, SBP_ERANGE (n > SBP_MAX_SHARD_NUMEL),
 * SBP_EHIP.
 * Host cost: beta^t is formed by repeated float64 multiplication.  Each
 * host thread keeps the powers of its last call and extends them when t
 * grows, so consecutive steps cost one multiplication.  A call at a smaller
 * t or with other betas starts again from 1, at up to min(t, 37.4 /
 * -ln(beta)) multiplications per beta (past that 1 - beta^t is exactly 1).
 * ---------------------------------------------------------------------- */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} sbp_adamw_hparams;

sbp_status sbp_adamw_shard(const void* const* peers, int32_t R,
                           const float* acc, float scale, float* master,
                           float* m, float* v, void* param_out, int64_t n,
                           const sbp_adamw_hparams* hp, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Parameter groups: per-group learning rate and weight decay on one shard
 * ("Parallelisms", ZeRO-1 and ZeRO-3: a rank updates the owned shard with
 * the optimizer's usual per-parameter update; an optimizer's parameter
 * groups -- decay on weight matrices, none on norms and biases -- are part
 * of that update.  beta1, beta2, eps and the step stay shared.)
 *
 * sbp_group_runs (host): the run table of rank `rank`'s shard -- maximal
 *   runs of shard elements with one group.  tensor_group: host int32[n_tensors],
 *   each in 0..SBP_MAX_GROUPS-1.  An element of a tensor takes that tensor's
 *   group; a padding element takes the group of the element before it in
 *   the shard, or group 0 at the shard's start (padding is +0 with +0 state,
 *   so it stays +0 under any group).  Runs are written as run_start[k]
 *   (ascending, run_start[0] == 0) and run_group[k]; at most `cap` entries
 *   are written and *count receives the number of runs (call with cap == 0
 *   to size the arrays).  A shard of 0 elements has one run (0, 0).
 *   Errors: SBP_EINVAL (null, rank out of range, group id out of range),
 *   SBP_ENOMEM.
 *
 * sbp_adamw_shard_grouped: sbp_adamw_shard where element i takes step_size
 *   and decay from group k's lr and weight_decay (groups[k], same rounding
 *   rules), k = run_group[j] of the last run j with run_start[j] <= i; hp
 *   supplies beta1, beta2, eps and step (its lr and weight_decay are not
 *   used).  A group id outside 0..n_groups-1 in the table uses group 0.
 *   Other arguments, layout and errors as in sbp_adamw_shard, plus:
 *   groups      host array of n_groups (1..SBP_MAX_GROUPS) entries, each
 *               lr and weight_decay finite and >= 0
 *   run_start   device int64[n_runs], 8-B aligned, ascending, starting at 0
 *   run_group   device int32[n_runs], 4-B aligned
 *   n_runs      >= 1 (the table from sbp_group_runs, copied to the device)
 *   The tables are only read; the extra traffic is a few bytes per 2048
 *   elements (one search of the table per tile).
 * ---------------------------------------------------------------------- */
typedef struct {
  float lr, weight_decay;
} sbp_group_hparams;

sbp_status sbp_group_runs(const sbp_plan* plan, int32_t rank,
                          const int32_t* tensor_group, int64_t* run_start,
                          int32_t* run_group, int64_t cap, int64_t* count);
sbp_status sbp_adamw_shard_grouped(const void* const* peers, int32_t R,
                                   const float* acc, float scale,
                                   float* master, float* m, float* v,
                                   void* param_out, int64_t n,
                                   const sbp_adamw_hparams* hp,
                                   const sbp_group_hparams* groups,
                                   int32_t n_groups, const int64_t* run_start,
                                   const int32_t* run_group, int64_t n_runs,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Global gradient-norm clipping ("Parallelisms", ZeRO-2: the clip norm is
 * the all-reduced sum of the ranks' local squared norms, known before the
 * update).
 *
 * sbp_grad_sq_norm: this rank's squared norm of the normalised gradient,
 *   sum_i (double) g_i^2 with g_i = fl(G_i * scale), G as in sbp_adamw_shard
 *   (G = acc + S, S, or acc when R == 0), accumulated in float64 (each square
 *   is exact) in a fixed order: one partial per tile of 2048 * gpl elements
 *   in `workspace` (gpl = 4 when a group of 8 elements loads 16 bytes: R = 1
 *   without acc; 2 when it loads 32: R = 2 without acc, or acc alone; else
 *   1), then a tree of fixed shape over those partials (groups of 2048
 *   consecutive partials, level by level, the levels also kept in
 *   `workspace`) into *sq_out (device).  Within a tile, each of the 256
 *   lanes adds its 8 * gpl squares in element order (its groups 256 groups
 *   apart; in the first tile lane l then adds tail element 8 * (n / 8) + l,
 *   if any), and the lanes' sums meet in a fixed tree.
 *   Results are deterministic run to run.  If g_sum_out is given, G (fp32,
 *   unscaled) is also written there, so the update can follow as
 *   sbp_adamw_shard(R = 0, acc = g_sum_out, scale = clipped scale) without
 *   reading the peers again.  Without g_sum_out the update is
 *   sbp_adamw_shard(the same peers and acc, scale = clipped scale), which
 *   recomputes G; both give the same bits.  Per element, writing G moves
 *   2R + 34 bytes in the two calls (+4 with acc) and recomputing 4R + 26
 *   (+8 with acc): recomputing moves less below R = 4 (R = 2 with acc).
 *   peers, R, acc, scale, n   as in sbp_adamw_shard (R may be 0 with acc)
 *   g_sum_out                 device fp32[n], 16-B aligned, or null
 *   workspace                 device double[workspace_len], 8-B aligned,
 *                             workspace_len >= sbp_grad_sq_norm_workspace(n)
 *   sq_out                    device double, 8-B aligned (n == 0 writes 0)
 *   Outputs must not overlap any other buffer.
 *   Errors: SBP_EINVAL (also a workspace shorter than needed), SBP_EALIGN,
 *   SBP_ERANGE (n > SBP_MAX_SHARD_NUMEL), SBP_EHIP.
 *
 * sbp_clip_scale (host): with total_sq the sum of all ranks' squared norms,
 *   coef = min(1, max_norm / (sqrt(total_sq) + 1e-6)) in float64 (a NaN norm
 *   gives a NaN coefficient), *clipped_scale = fl32(scale * coef), and
 *   *coef (optional) receives coef.  Errors: SBP_EINVAL (null output,
 *   max_norm negative or NaN, total_sq negative).
 * ---------------------------------------------------------------------- */
int64_t sbp_grad_sq_norm_workspace(int64_t n);
sbp_status sbp_grad_sq_norm(const void* const* peers, int32_t R,
                            const float* acc, float scale, int64_t n,
                            float* g_sum_out, double* workspace,
                            int64_t workspace_len, double* sq_out,
                            hipStream_t stream);
sbp_status sbp_clip_scale(double total_sq, float max_norm, float scale,
                          float* clipped_scale, double* coef);

/* ------------------------------------------------------------------------
 * Spread arena: device memory for a rank's shard state and receive buffers
 * ("Parallelisms", ZeRO-1 and ZeRO-3: each rank keeps its shard's fp32
 * master copy, first and second moments and parameter shard, and receives
 * its peers' gradient chunks of that shard).  Unlike every call above, these
 * calls allocate and free device memory; they exist for placement.
 *
 * The fused step streams all its arrays at the same offset at once, and on
 * MI355X that mix runs measurably faster when the arrays' physical pages are
 * spread over the whole HBM instead of packed into one region.
 * sbp_arena_create gives each array its own virtual range and backs it with
 * physical chunks of chunk_bytes taken evenly spaced from a run of chunks
 * created over spread_bytes of device memory (the chunks in between are
 * released before the call returns), mapped to the arrays' chunk slots in a
 * seeded random order.  The policy is fixed (no timing, no search); only the
 * device's allocator decides where the run lies.
 *
 * bytes[n_arrays]  size of each array in bytes (>= 0; 0 gives a null pointer)
 * n_arrays         1..SBP_ARENA_MAX_ARRAYS
 * chunk_bytes      physical chunk size: 0 for the default 64 MiB, else a
 *                  positive multiple of 2 MiB (and of the device's
 *                  allocation granularity); each array is rounded up to a
 *                  whole number of chunks, at most 16384 in all
 * spread_bytes     memory to spread over: 0 for all free device memory less
 *                  a reserve of 1/32 of the total (at least 1 GiB); at most
 *                  8192 chunks are created to spread, never fewer than the
 *                  arrays need
 * seed             seed of the slot order (splitmix64 + Fisher-Yates)
 * ptrs[n_arrays]   receive the arrays' device addresses (chunk_bytes-aligned;
 *                  contents undefined until written)
 * out              receives the arena; free with sbp_arena_free
 * The arrays belong to the device current at the call and are readable and
 * writable from it.  sbp_arena_free synchronises that device, then unmaps
 * and releases everything; a null arena is a no-op.  sbp_arena_info reports
 * the chunk size, the chunks kept and the chunks created to spread over
 * (any output pointer may be null).
 * Errors: SBP_EINVAL (null, bad count, negative size, bad chunk size),
 * SBP_ERANGE (more than 16384 chunks), SBP_ENOMEM (device memory), SBP_EHIP
 * (no virtual memory management, or another runtime failure).  On error
 * nothing stays allocated.
 * ---------------------------------------------------------------------- */
#define SBP_ARENA_MAX_ARRAYS 64
typedef struct sbp_arena sbp_arena;
sbp_status sbp_arena_create(const int64_t* bytes, int32_t n_arrays,
                            int64_t chunk_bytes, int64_t spread_bytes,
                            uint64_t seed, void** ptrs, sbp_arena** out);
sbp_status sbp_arena_info(const sbp_arena* arena, int64_t* chunk_bytes,
                          int64_t* chunks_kept, int64_t* chunks_spread);
sbp_status sbp_arena_free(sbp_arena* arena);

/* ------------------------------------------------------------------------
 * The squared norm for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops and harnesses that forbid
 * hipMalloc.
 *
 * sbp_grad_sq_norm_noalloc: the same computation, result bits and argument
 *   rules as sbp_grad_sq_norm, with the workspace taken from a static
 *   device array inside the library instead of from the caller.  Each GPU
 *   the library runs on holds one such array of
 *   SBP_NOALLOC_SCRATCH_DOUBLES doubles (8 MiB) until the process ends; its
 *   address is looked up once per device, on that device's first call.  The
 *   call allocates and frees nothing.
 *   n is limited to SBP_NOALLOC_MAX_NUMEL (the largest n whose tile
 *   partials and tree levels fit the array); a larger n is SBP_ERANGE.
 *   Every workspace slot is written before it is read within one call, so
 *   nothing needs clearing between calls.  All calls on one GPU share its
 *   array: calls that overlap in time on one GPU (two streams, or two
 *   threads) race and must be ordered by the caller.
 *   Errors: as sbp_grad_sq_norm (less the workspace checks), SBP_ERANGE
 *   also for n > SBP_NOALLOC_MAX_NUMEL, SBP_EHIP if the array's device
 *   address cannot be looked up.
 * ---------------------------------------------------------------------- */
#define SBP_NOALLOC_SCRATCH_DOUBLES 1048576 /* 2^20 doubles per GPU       */
#define SBP_NOALLOC_MAX_NUMEL 2146435079LL   /* 2048 * 1048064 + 7         */
sbp_status sbp_grad_sq_norm_noalloc(const void* const* peers, int32_t R,
                                    const float* acc, float scale, int64_t n,
                                    float* g_sum_out, double* sq_out,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SBP_H */
