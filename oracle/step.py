"""Oracle shard step (test infrastructure only; see oracle/__init__.py).

All floating point is IEEE binary32, one round-to-nearest-even rounding per
operation (numpy float32 ufuncs; no fused multiply-add), except host scalars,
computed in float64 from the binary32 hyperparameters and rounded once.
bf16 values travel as their 16-bit patterns (np.uint16).
"""

import math
from dataclasses import dataclass

import numpy as np

F32 = np.float32


# ---- bf16 <-> fp32 -------------------------------------------------------------

def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns: they are the top half of a binary32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x):
    """Round binary32 to bf16, to nearest, ties to even (the bf16 parameter copy).

    The pages keep bf16 model weights next to an fp32 master ("Distributed
    Training and Parallelism", section "ZeRO and sharded state"); the rounding
    rule is the reading taken here: nearest, ties to the even upper half;
    overflow goes to +-inf; a NaN stays a NaN of the same sign (quiet bit set).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    quiet = (u >> 16) | 0x0040
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


# ---- layout: pack, chunks, gather ------------------------------------------------

def pack(plan, grads):
    """Copy per-tensor bf16 gradients into the flat buckets; other slots are +0.

    "Parallelisms", section "Gradient bucketing" (gradients collected into
    buffers) and section "FSDP" (flat parameter: parameters concatenated into
    one contiguous tensor; YaFSDP writes gradients directly into the
    communication buffers).
    """
    flat = np.zeros(plan.flat_numel, dtype=np.uint16)
    for t, g in enumerate(grads):
        g = np.asarray(g, dtype=np.uint16).reshape(-1)
        if g.size != plan.numels[t]:
            raise ValueError(f"tensor {t}: {g.size} elements, plan says {plan.numels[t]}")
        o = plan.tensor_flat_offset(t)
        flat[o:o + g.size] = g
    return flat


def unpack(plan, flat):
    """Per-tensor views of a flat buffer (the inverse of pack)."""
    return [flat[plan.tensor_flat_offset(t):plan.tensor_flat_offset(t) + n]
            for t, n in enumerate(plan.numels)]


def chunk(plan, flat, s):
    """Rank s's share of a flat buffer: chunk s of every bucket, in bucket order.

    "Parallelisms", section ZeRO-2: each bucket is reduce-scattered as it
    becomes ready and each worker keeps the reduced gradients of its 1/N
    shard.  This is the layout of every peer contribution the shard step
    reads, and of the shard state.
    """
    parts = [flat[b.flat_offset + s * b.chunk: b.flat_offset + (s + 1) * b.chunk]
             for b in plan.buckets]
    return np.concatenate(parts) if parts else flat[:0].copy()


def gather(plan, shards):
    """All-gather: put every rank's shard back into the flat bucket layout.

    "Parallelisms", section ZeRO-1: after the update each rank's parameter
    shard is all-gathered, so every rank again holds the whole model.
    """
    if len(shards) != plan.world_n:
        raise ValueError("one shard per rank")
    flat = np.empty(plan.flat_numel, dtype=np.asarray(shards[0]).dtype)
    for b in plan.buckets:
        for s in range(plan.world_n):
            flat[b.flat_offset + s * b.chunk: b.flat_offset + (s + 1) * b.chunk] = \
                shards[s][b.shard_offset: b.shard_offset + b.chunk]
    return flat


# ---- reduce, accumulate, normalise -------------------------------------------------

def reduce_peers(peers):
    """S = sum of the R peer contributions, in fp32, in ascending rank order.

    The reduce-scatter sums every worker's contribution to the shard a worker
    owns ("Parallelisms", section ZeRO-1; "Parallelism Starts With the
    Bottleneck", section "Allreduce equals reducescatter plus allgather").
    The order is fixed because the reduction order changes the bits
    ("Distributed Training and Parallelism", section "Data parallelism and
    the global gradient"); the sum starts from peer 0 itself (not from 0, which
    would turn a -0 into +0), then adds peers 1..R-1 one at a time.
    """
    if len(peers) < 1:
        raise ValueError("at least one peer")
    s = bf16_to_f32(peers[0]).copy()
    for p in peers[1:]:
        s = s + bf16_to_f32(p)
    return s


def accumulate(acc, s):
    """Gradient accumulation over microbatches: A = S for the first, else A + S.

    "Distributed Training and Parallelism", section "Data parallelism and the
    global gradient": intermediate reductions are suppressed (no_sync) and the
    final pass synchronises the accumulated gradients; "Parallelisms",
    section ZeRO-2: accumulation adds contributions from later microbatches.
    """
    if acc is None:
        return np.array(s, dtype=np.float32, copy=True)
    return np.asarray(acc, dtype=np.float32) + np.asarray(s, dtype=np.float32)


def mean_scale(R, K=1):
    """DDP average over R contributions and K accumulated microbatches: fl32(1/(R*K))."""
    return F32(1.0 / (R * K))


def tokens_scale(counts):
    """Valid-token normalisation: fl32(1/C), C the global valid-token count.

    "Distributed Training and Parallelism", section "Data parallelism and the
    global gradient": with unequal valid-token counts a rank's summed loss is
    scaled by R/global_count when the framework averages over the R ranks;
    that average's 1/R composed with R/C is 1/C, applied once after the sum
    (the page's adjoint remark asks for that scaling to be accounted for
    explicitly).
    """
    C = int(sum(int(c) for c in counts))
    if C <= 0:
        raise ValueError("global valid-token count must be positive")
    return F32(1.0 / C)


def normalise(G, scale):
    """g = fl(G * scale): one fp32 multiply after the sum."""
    return np.asarray(G, dtype=np.float32) * F32(scale)


# ---- AdamW -----------------------------------------------------------------------

@dataclass(frozen=True)
class AdamWScalars:
    beta1: np.float32
    beta2: np.float32
    omb1: np.float32  # 1 - beta1
    omb2: np.float32  # 1 - beta2
    eps: np.float32
    step_size: np.float32  # lr / (1 - beta1^t)
    c2: np.float32  # 1 / sqrt(1 - beta2^t)
    decay: np.float32  # 1 - lr * weight_decay


def adamw_scalars(lr, beta1, beta2, eps, weight_decay, t):
    """Per-step host scalars: float64 from the binary32 hyperparameters, rounded once.

    beta^t is formed by t multiplications in float64.
    """
    if t < 1:
        raise ValueError("optimizer step t is 1-based")
    lr, b1, b2, eps, wd = (float(F32(x)) for x in (lr, beta1, beta2, eps, weight_decay))
    b1t = b2t = 1.0
    for _ in range(int(t)):
        b1t *= b1
        b2t *= b2
    bc1 = 1.0 - b1t
    bc2 = 1.0 - b2t
    return AdamWScalars(
        beta1=F32(b1), beta2=F32(b2), omb1=F32(1.0 - b1), omb2=F32(1.0 - b2), eps=F32(eps),
        step_size=F32(lr / bc1), c2=F32(1.0 / math.sqrt(bc2)), decay=F32(1.0 - lr * wd))


def adamw(theta, m, v, g, sc):
    """One decoupled-weight-decay Adam step on the owned shard (fp32 state).

    The pages name the state: first and second moment buffers, a small step
    counter and an fp32 master copy, held only for the owned 1/N shard
    ("Parallelisms", section ZeRO-1; "Parallelism Starts With the
    Bottleneck", section "Data parallelism is simple and pays for it in
    memory").  The update rule is the reading taken here (bias-corrected
    moments, eps outside the square root, decay theta*(1 - lr*wd) applied to
    the old weight), in this operation order:
        m' = b1*m + (1-b1)*g
        v' = b2*v + (1-b2)*(g*g)
        d  = sqrt(v')*c2 + eps
        theta' = theta*decay - step_size*(m'/d)
    """
    theta = np.asarray(theta, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    m1 = sc.beta1 * m + sc.omb1 * g
    v1 = sc.beta2 * v + sc.omb2 * (g * g)
    d = np.sqrt(v1) * sc.c2 + sc.eps
    theta1 = theta * sc.decay - sc.step_size * (m1 / d)
    return theta1, m1, v1


# ---- parameter groups --------------------------------------------------------------

def shard_groups(plan, s, tensor_group):
    """Group of every element of rank s's shard: its tensor's group; a padding
    element takes the group of the element before it in the shard (group 0 at
    the very start) -- padding stays +0 under any group."""
    spans = sorted((plan.tensor_flat_offset(t), plan.tensor_flat_offset(t) + n, t)
                   for t, n in enumerate(plan.numels) if n)
    flat_group = np.full(plan.flat_numel, -1, dtype=np.int64)
    for a, e, t in spans:
        flat_group[a:e] = tensor_group[t]
    g = chunk(plan, flat_group, s)
    prev = 0
    for j in range(g.size):  # plain loop: padding inherits the group before it
        if g[j] < 0:
            g[j] = prev
        prev = g[j]
    return g.astype(np.int32)


def adamw_grouped(theta, m, v, g, sc, step_size, decay):
    """adamw() with per-element step_size and decay (binary32 arrays)."""
    theta = np.asarray(theta, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    m1 = sc.beta1 * m + sc.omb1 * g
    v1 = sc.beta2 * v + sc.omb2 * (g * g)
    d = np.sqrt(v1) * sc.c2 + sc.eps
    theta1 = theta * decay - step_size * (m1 / d)
    return theta1, m1, v1


def shard_step_grouped(peers, acc, scale, theta, m, v, hp, groups, elem_group, t):
    """shard_step() with per-group lr and weight decay (betas, eps and t shared).

    groups: list of (lr, weight_decay); elem_group: group of each element.
    Each group's step size and decay are that group's host scalars (same
    rules as adamw_scalars); the element takes its group's pair.
    """
    if peers:
        S = reduce_peers(peers)
        G = S if acc is None else np.asarray(acc, dtype=np.float32) + S
    else:
        G = np.asarray(acc, dtype=np.float32)
    g = normalise(G, scale)
    per = [adamw_scalars(lr, hp.beta1, hp.beta2, hp.eps, wd, t) for lr, wd in groups]
    sc = per[0]
    step_size = np.array([p.step_size for p in per], dtype=np.float32)[elem_group]
    decay = np.array([p.decay for p in per], dtype=np.float32)[elem_group]
    theta1, m1, v1 = adamw_grouped(theta, m, v, g, sc, step_size, decay)
    return theta1, m1, v1, f32_to_bf16(theta1)


# ---- global gradient-norm clipping -------------------------------------------------

CLIP_EPS = 1e-6  # added to the norm before dividing (the common convention)


def grad_sq_norm(G, scale):
    """Sum over this rank's shard of g*g, g = fl(G*scale), in float64.

    "Parallelisms", section ZeRO-2: the clip norm is the all-reduced sum of
    the ranks' local squared norms, known before the update.  Each square of
    a binary32 value is exact in float64; math.fsum gives the correctly
    rounded float64 sum.
    """
    g = normalise(G, scale).astype(np.float64)
    return math.fsum((g * g).tolist())


def clip_coef(total_sq, max_norm):
    """min(1, max_norm / (||g|| + eps)), in float64; ||g|| = sqrt(total of the
    ranks' squared norms).  max_norm is a binary32 hyperparameter, like lr.
    A NaN norm gives a NaN coefficient (no skip policy: NaN propagates)."""
    q = float(F32(max_norm)) / (math.sqrt(total_sq) + CLIP_EPS)
    return q if (q < 1.0 or math.isnan(q)) else 1.0


def clipped_scale(scale, coef):
    """The clip coefficient folded into the normalisation: fl32(scale * coef)."""
    return F32(float(F32(scale)) * coef)


# ---- the whole shard step ----------------------------------------------------------

def shard_step(peers, acc, scale, theta, m, v, hp, t):
    """Reduce (+ accumulated microbatches) -> normalise -> AdamW -> bf16 emit.

    peers: list of R bf16 arrays (R may be 0 when acc carries the whole
    gradient); acc: fp32 accumulator of earlier microbatches or None.
    G = acc + S (or S, or acc), g = G*scale; returns (theta', m', v', bf16
    parameter shard for the all-gather).
    """
    if peers:
        S = reduce_peers(peers)
        G = S if acc is None else np.asarray(acc, dtype=np.float32) + S
    else:
        if acc is None:
            raise ValueError("need peers or an accumulator")
        G = np.asarray(acc, dtype=np.float32)
    g = normalise(G, scale)
    sc = adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t)
    theta1, m1, v1 = adamw(theta, m, v, g, sc)
    return theta1, m1, v1, f32_to_bf16(theta1)
