"""Full-size parity at model scale: the oracle on many host cores at once.

Test infrastructure (imports the oracle; nothing in the product imports this).
The shard step is elementwise once the plan is fixed, and every input element
can be regenerated on its own, so a shard splits into independent slices.
Spawned worker processes (which never touch the GPU) each compute the
oracle's state for one slice after the workload's steps and return 128-bit
xxh3 digests of the expected master, m, v and bf16 parameter bytes; the test
process digests the GPU's copy of the same slice and compares.  A slice whose
digest differs is recomputed in the test process for an element-level report.
"""

import os

import numpy as np

import synth
from oracle import plan as OP
from oracle import step as OS

SLICE = 1 << 24  # elements per job


def _worker_init():
    # one host thread per worker process: the pool already spans the cores
    os.environ["OMP_NUM_THREADS"] = "1"


def shard_state(job):
    """The oracle's (master, m, v, param bits) for elements [i0, i1) of shard 0
    of workload `name` after optimizer steps 1..steps, from seeded inputs:
    R peers per microbatch, K microbatches (all but the last accumulated),
    MEAN 1/(R*K) or TOKENS 1/C scaling."""
    name, seed, i0, i1, steps = job
    w = synth.WORKLOADS[name]
    n = i1 - i0
    th = synth.normal_f32(seed, synth.master_stream(0), n, w.master_sigma, i0)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = None
    for t in range(1, steps + 1):
        if w.norm == "tokens":
            scale = OS.tokens_scale([synth.tokens(seed, t, r) for r in range(w.R)])
        else:
            scale = OS.mean_scale(w.R, w.K)
        A = None
        for k in range(w.K):
            peers = [synth.normal_bf16(seed, synth.peer_stream(t, k, r), n, w.grad_sigma, i0)
                     for r in range(w.R)]
            if k < w.K - 1:
                A = OS.accumulate(A, OS.reduce_peers(peers))
            else:
                th, m, v, p = OS.shard_step(peers, A, scale, th, m, v, w.adamw, t)
    return th, m, v, p


def dp_rank0_packed(seed, plan, numels, grad_sigma, a, b, t=1):
    """Rank 0's packed bf16 gradient over flat positions [a, b) of a whole-
    tensor plan: each tensor's seeded gradient at its plan offset, +0 in
    padding (the oracle's pack, restricted to the range)."""
    out = np.zeros(b - a, np.uint16)
    for tid, k in enumerate(numels):
        lo = plan.tensor_flat_offset(tid)
        hi = lo + k
        s, e = max(a, lo), min(b, hi)
        if s < e:
            out[s - a:e - a] = synth.normal_bf16(seed, synth.tensor_stream(t, 0, 0, tid), e - s,
                                                 grad_sigma, s - lo)
    return out


_DP_PLAN = {}


def _dp_peers(name, seed, a, b):
    """The DP replica's two contributions over flat positions [a, b): rank
    0's per-tensor gradients packed, and rank 1's bucket-layout gradient."""
    w = synth.WORKLOADS[name]
    if name not in _DP_PLAN:
        _DP_PLAN[name] = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    p0 = dp_rank0_packed(seed, _DP_PLAN[name], w.numels, w.grad_sigma, a, b)
    p1 = synth.normal_bf16(seed, synth.peer_stream(1, 0, 1), b - a, w.grad_sigma, a)
    return p0, p1


def dp_state(job):
    """The oracle's state for flat positions [a, b) of the DP replica (N = 1,
    R = 2) after one step, and rank 0's packed gradient there.  The scale is
    MEAN 1/2, or the clipped scale given as a fifth job entry (the step then
    sums the peers again, as a norm pass that stores no G leaves it)."""
    name, seed, a, b = job[:4]
    w = synth.WORKLOADS[name]
    p0, p1 = _dp_peers(name, seed, a, b)
    scale = OS.mean_scale(w.R) if len(job) == 4 else np.float32(job[4])
    th = synth.normal_f32(seed, synth.master_stream(0), b - a, w.master_sigma, a)
    z = np.zeros(b - a, np.float32)
    return OS.shard_step([p0, p1], None, scale, th, z, z, w.adamw, 1) + (p0,)


def dp_norm_partial(job):
    """The DP replica's part of the squared norm over [a, b) (MEAN 1/2): the
    oracle's grad_sq_norm, correctly rounded."""
    name, seed, a, b = job
    w = synth.WORKLOADS[name]
    return job, OS.grad_sq_norm(OS.reduce_peers(list(_dp_peers(name, seed, a, b))),
                                OS.mean_scale(w.R))


_SHARD_MAP = {}


def shard0_groups(name, i0, i1):
    """Parameter group of each element [i0, i1) of rank 0's shard under the
    benchmark's two groups (0: weight decay, for matrices; 1: none, for 1-D
    tensors), found through the oracle's plan: shard position -> bucket ->
    flat position of rank 0's chunk -> the tensor holding it (the plan has no
    padding)."""
    w = synth.WORKLOADS[name]
    if name not in _SHARD_MAP:
        plan = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
        so = np.array([b.shard_offset for b in plan.buckets], np.int64)
        fo = np.array([b.flat_offset for b in plan.buckets], np.int64)
        starts = np.array([plan.tensor_flat_offset(t) for t in range(len(w.numels))], np.int64)
        order = np.argsort(starts)
        tg = np.array([1 if len(shape) == 1 else 0 for _, shape in w.params], np.int64)
        _SHARD_MAP[name] = (so, fo, starts, order, tg)
    so, fo, starts, order, tg = _SHARD_MAP[name]
    idx = np.arange(i0, i1, dtype=np.int64)
    bk = np.searchsorted(so, idx, side="right") - 1
    flat = fo[bk] + (idx - so[bk])
    tids = order[np.searchsorted(starts[order], flat, side="right") - 1]
    return tg[tids]


def grouped_state(job):
    """shard_state() for the grouped step: the benchmark's two parameter
    groups (lr and weight decay; none on 1-D tensors)."""
    name, seed, i0, i1, steps = job
    w = synth.WORKLOADS[name]
    n = i1 - i0
    groups = [(w.adamw.lr, w.adamw.weight_decay), (w.adamw.lr, 0.0)]
    eg = shard0_groups(name, i0, i1)
    th = synth.normal_f32(seed, synth.master_stream(0), n, w.master_sigma, i0)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = None
    for t in range(1, steps + 1):
        peers = [synth.normal_bf16(seed, synth.peer_stream(t, 0, r), n, w.grad_sigma, i0)
                 for r in range(w.R)]
        th, m, v, p = OS.shard_step_grouped(peers, None, OS.mean_scale(w.R), th, m, v, w.adamw,
                                            groups, eg, t)
    return th, m, v, p


def _step1_scale(w, seed):
    """The oracle's normalisation of step 1: 1/C over the ranks' valid-token
    counts, or the mean 1/(R*K)."""
    if w.norm == "tokens":
        return OS.tokens_scale([synth.tokens(seed, 1, r) for r in range(w.R)])
    return OS.mean_scale(w.R, w.K)


def _step1_g(w, seed, i0, i1):
    """G of step 1 over [i0, i1): the first K - 1 microbatches' peer sums
    accumulated, plus the last one's (the sum the norm pass stores)."""
    A = None
    for k in range(w.K):
        peers = [synth.normal_bf16(seed, synth.peer_stream(1, k, r), i1 - i0, w.grad_sigma, i0)
                 for r in range(w.R)]
        A = OS.accumulate(A, OS.reduce_peers(peers))
    return A


def clip_norm_partial(job):
    """This slice's part of the squared norm of g = fl(G * scale) at step 1:
    the oracle's grad_sq_norm (correctly rounded)."""
    name, seed, i0, i1 = job
    w = synth.WORKLOADS[name]
    return job, OS.grad_sq_norm(_step1_g(w, seed, i0, i1), _step1_scale(w, seed))


def clipped_state(job):
    """The oracle's state for [i0, i1) after one clipped step taken the way
    the benchmark's --clip step takes it: G stored by the norm pass, then the
    update from G alone (no peers, G as the accumulator) with the clipped
    scale cs (the oracle's)."""
    name, seed, i0, i1, cs = job
    w = synth.WORKLOADS[name]
    n = i1 - i0
    G = _step1_g(w, seed, i0, i1)
    th = synth.normal_f32(seed, synth.master_stream(0), n, w.master_sigma, i0)
    z = np.zeros(n, np.float32)
    return OS.shard_step([], G, np.float32(cs), th, z, z, w.adamw, 1)


def digests(arrays):
    import xxhash
    return tuple(xxhash.xxh3_128_digest(np.ascontiguousarray(x).view(np.uint8)) for x in arrays)


def shard_digests(job):
    return job, digests(shard_state(job))


def dp_digests(job):
    return job, digests(dp_state(job))


def grouped_digests(job):
    return job, digests(grouped_state(job))


def clipped_digests(job):
    return job, digests(clipped_state(job))


def workers():
    """Worker processes for this host: the cores this process may use,
    capped by OMP_NUM_THREADS where set (this process's share of a shared host)
    and at 16."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def pool(procs=None):
    import multiprocessing as mp
    return mp.get_context("spawn").Pool(procs or workers(), initializer=_worker_init)
