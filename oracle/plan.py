"""Oracle bucket plan (test infrastructure only; see oracle/__init__.py).

What it follows:
  * "Parallelisms" (vladislavkruglikov.com), section "Gradient bucketing":
    parameter gradients are collected into buffers, each communicated once
    ready; a bigger bucket means fewer collectives but a later start.
  * same page, section "Data parallel": buckets for later layers are ready
    first, during backward -> tensors are visited in reverse registration
    order.
  * same page, section "FSDP" / "Flat parameter": one contiguous buffer that
    concatenates parameters, the originals being views into its slices.
  * same page, sections "ZeRO-1" and "ZeRO-2": each ready bucket is
    reduce-scattered and each worker keeps the reduced shard of the
    parameters it owns, roughly 1/N of the model.

Readings where the pages are silent:
  * the cap counts bf16 gradient bytes (the communication buffer); a tensor
    is added, then the bucket closes once 2*used >= cap; tensors are never
    split, so a bucket may exceed the cap by its last tensor;
  * each tensor starts at a multiple of `align` elements (first one at 0);
    a bucket is padded with zeros to a multiple of align*N elements, so each
    of its N equal chunks keeps that alignment;
  * rank s owns chunk s of every bucket; its shard is those chunks
    concatenated in bucket order.
"""

import math
from dataclasses import dataclass


def _round_up(x, m):
    return (x + m - 1) // m * m


@dataclass
class Bucket:
    tensors: list  # tensor ids in visit order
    used: int  # elements up to the end of the last tensor
    padded: int  # used rounded up to align * N
    chunk: int  # padded / N: elements each rank owns of this bucket
    shard_offset: int  # where this bucket's chunk starts in a rank's shard
    flat_offset: int  # where this bucket starts in the flat buffer


@dataclass
class Plan:
    numels: list
    cap_bytes: int
    world_n: int
    align: int
    order: str
    tensor_bucket: list  # per tensor id
    tensor_offset: list  # per tensor id, element offset inside its bucket
    buckets: list
    shard_numel: int  # n: elements of one rank's shard (same for all ranks)
    flat_numel: int  # sum of padded bucket sizes

    def tensor_flat_offset(self, t):
        return self.buckets[self.tensor_bucket[t]].flat_offset + self.tensor_offset[t]


def bucket_plan(numels, cap_bytes, world_n, align=8, order="reverse", split=False):
    """Assign tensors to flat bf16 buckets and split each bucket into N chunks.

    split=False: whole tensors per bucket (the closing rule above).
    split=True: the tensors are concatenated (each at the first multiple of
    `align` after the previous one, in visit order) and the result is cut
    into fixed-size buckets of cap_bytes / 2 elements rounded down to a
    multiple of align * N (at least align * N); a tensor may then straddle
    buckets, as when a flat parameter is cut into equal communication
    pieces.  Only the last bucket can be shorter; it is padded as before.
    """
    if cap_bytes <= 0 or world_n <= 0 or align <= 0 or (align & (align - 1)):
        raise ValueError("cap_bytes, world_n > 0 and align a power of two required")
    if any(int(x) < 0 for x in numels):
        raise ValueError("negative numel")
    T = len(numels)
    visit = list(range(T - 1, -1, -1)) if order == "reverse" else list(range(T))
    if split:
        return _split_plan(numels, cap_bytes, world_n, align, order, visit)

    groups = []  # (tensor ids, offsets, used)
    cur, offs, used = [], [], 0
    for t in visit:
        off = 0 if used == 0 else _round_up(used, align)
        cur.append(t)
        offs.append(off)
        used = off + int(numels[t])
        if 2 * used >= cap_bytes:
            groups.append((cur, offs, used))
            cur, offs, used = [], [], 0
    if cur:
        groups.append((cur, offs, used))

    tensor_bucket = [None] * T
    tensor_offset = [None] * T
    buckets = []
    shard_off = flat_off = 0
    for b, (ids, offsets, used) in enumerate(groups):
        padded = _round_up(used, align * world_n)
        chunk = padded // world_n
        buckets.append(Bucket(list(ids), used, padded, chunk, shard_off, flat_off))
        for t, o in zip(ids, offsets):
            tensor_bucket[t] = b
            tensor_offset[t] = o
        shard_off += chunk
        flat_off += padded
    return Plan([int(x) for x in numels], cap_bytes, world_n, align, order,
                tensor_bucket, tensor_offset, buckets, shard_off, flat_off)


def _split_plan(numels, cap_bytes, world_n, align, order, visit):
    T = len(numels)
    unit = align * world_n
    size = max(unit, (cap_bytes // 2) // unit * unit)  # elements per bucket
    # concatenate in visit order, each tensor at the first aligned slot
    flat_pos = [None] * T
    end = 0
    for t in visit:
        flat_pos[t] = 0 if end == 0 else _round_up(end, align)
        end = flat_pos[t] + int(numels[t])
    nb = -(-end // size) if end > 0 else (1 if T else 0)
    # a tensor's bucket is the one its first element falls in (the last one
    # for an empty tensor at the very end)
    tensor_bucket = [min(flat_pos[t] // size, nb - 1) for t in range(T)]
    tensor_offset = [flat_pos[t] - tensor_bucket[t] * size for t in range(T)]
    buckets = []
    shard_off = 0
    for b in range(nb):
        lo, hi = b * size, (b + 1) * size
        used = max(0, min(hi, end) - lo)
        padded = _round_up(used, unit)
        members = [t for t in visit
                   if (int(numels[t]) > 0 and flat_pos[t] < hi and flat_pos[t] + int(numels[t]) > lo)
                   or (int(numels[t]) == 0 and tensor_bucket[t] == b)]
        buckets.append(Bucket(members, used, padded, padded // world_n, shard_off, lo))
        shard_off += padded // world_n
    flat = sum(b.padded for b in buckets)
    return Plan([int(x) for x in numels], cap_bytes, world_n, align, order, tensor_bucket,
                tensor_offset, buckets, shard_off, flat)


def per_tensor_plan(numels, world_n, rows=None, align=8, order="reverse"):
    """One bucket per tensor, each rank owning whole rows of it.

    "Parallelisms", section FSDP: FSDP2 shards each parameter in place
    (dim 0), keeping parameter identities instead of a flat parameter.  Here
    tensor t (visit order as before) is its own bucket, padded to a multiple
    of N * unit_t with unit_t = lcm(align, row_t), row_t = elements per dim-0
    row (1 for a 1-D view); so every rank's chunk is ceil(numel / (N unit_t))
    * unit_t elements: whole rows, aligned.
    """
    if world_n <= 0 or align <= 0 or (align & (align - 1)):
        raise ValueError("world_n > 0 and align a power of two required")
    T = len(numels)
    rows = [1] * T if rows is None else [int(r) for r in rows]
    if len(rows) != T or any(r <= 0 for r in rows):
        raise ValueError("one positive row size per tensor")
    if any(int(n) < 0 or int(n) % r for n, r in zip(numels, rows)):
        raise ValueError("numel must be >= 0 and a multiple of its row size")
    visit = list(range(T - 1, -1, -1)) if order == "reverse" else list(range(T))
    buckets = []
    tensor_bucket = [None] * T
    tensor_offset = [0] * T
    shard_off = flat_off = 0
    for t in visit:
        unit = align * rows[t] // math.gcd(align, rows[t])
        padded = _round_up(int(numels[t]), world_n * unit)
        b = len(buckets)
        buckets.append(Bucket([t], int(numels[t]), padded, padded // world_n, shard_off, flat_off))
        tensor_bucket[t] = b
        shard_off += padded // world_n
        flat_off += padded
    return Plan([int(x) for x in numels], 0, world_n, align, order, tensor_bucket, tensor_offset,
                buckets, shard_off, flat_off)


# Bytes per parameter of the model state with bf16 params and grads, an fp32
# master copy and two fp32 Adam moments: 2 + 2 + 4 + 4 + 4 = 16
# ("Parallelism Strategies in Distributed Computing", Comparison / Cost per
# strategy; "Parallelism Starts With the Bottleneck", section "Data
# parallelism is simple and pays for it in memory").
PARAM_BYTES, GRAD_BYTES, OPT_BYTES = 2, 2, 12


def state_bytes(flat_numel, shard_numel, zero_stage):
    """Persistent model-state bytes one rank holds.

    Stage 0 is plain DP (everything replicated); stage 1 shards the optimizer
    state (master, m, v), stage 2 also the gradients, stage 3 also the
    parameters ("Distributed Training and Parallelism", section "ZeRO and
    sharded state"; "Parallelisms", sections ZeRO-1/2/3).  Activations,
    temporary buckets and gathers are excluded, as that page says its totals
    exclude them.
    """
    full, shard = flat_numel, shard_numel
    if zero_stage == 0:
        return (PARAM_BYTES + GRAD_BYTES + OPT_BYTES) * full
    if zero_stage == 1:
        return (PARAM_BYTES + GRAD_BYTES) * full + OPT_BYTES * shard
    if zero_stage == 2:
        return PARAM_BYTES * full + (GRAD_BYTES + OPT_BYTES) * shard
    if zero_stage == 3:
        return (PARAM_BYTES + GRAD_BYTES + OPT_BYTES) * shard
    raise ValueError("zero_stage must be 0..3")
