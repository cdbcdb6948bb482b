"""Pins of the oracle's shard step (CPU only).

Each part is checked against something other than itself: hand-worked
values, closed forms (the AdamW first step, the valid-token mean), exact
rational arithmetic and floating-point error bounds, invariants of the
collectives (reduce-scatter then all-gather equals all-reduce; the union of
shard updates equals the unsharded update), and library routines (torch's
bf16 conversion, torch.optim.AdamW).
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import plan as P
from oracle import step as S
from tests.conftest import read_golden

U = 2.0 ** -24  # unit roundoff of binary32


def f32(x):
    return np.asarray(x, dtype=np.float32)


def bits(x):
    return f32(x).view(np.uint32)


def ulp32(x):
    """Spacing of binary32 at |x| (the gap to the next larger magnitude)."""
    x = np.abs(f32(x))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def bf16(x):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    u = bits(x)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


# ---- bf16 cast ---------------------------------------------------------------

def test_bf16_cast_golden():
    for ln in read_golden("bf16_rne.txt"):
        src, want = ln.split()[:2]
        got = S.f32_to_bf16(np.array([int(src, 16)], dtype=np.uint32).view(np.float32))[0]
        assert got == int(want, 16), (src, hex(got), want)


def test_bf16_cast_matches_torch_structured_sweep():
    highs = np.arange(65536, dtype=np.uint32) << 16
    rng = np.random.default_rng(7)
    lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF], np.uint32),
                           rng.integers(0, 65536, 16, dtype=np.uint32)])
    u = (highs[:, None] | lows[None, :]).reshape(-1)
    x = u.view(np.float32)
    ours = S.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN compared by class and sign (torch returns one canonical NaN)
    o32 = (ours[nan].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(o32))
    assert np.array_equal(ours[nan] >> 15, (u[nan] >> 31).astype(np.uint16))


def test_bf16_cast_exhaustive():
    """Every one of the 2^32 fp32 bit patterns: the oracle's cast equals
    torch's round-to-nearest-even conversion, NaNs compared by class and
    sign (torch returns one canonical NaN).  256 blocks of 2^24 patterns in
    spawned worker processes (about half a minute on 8 cores)."""
    import multiprocessing as mp
    import os
    from tests import cast_sweep
    workers = max(1, min(8, os.cpu_count() or 1))
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(cast_sweep.check_block, range((1 << 32) // cast_sweep.BLOCK))
    assert sum(r[0] for r in res) == 0, "non-NaN patterns that round differently"
    assert sum(r[1] for r in res) == 0, "NaN patterns that lose their class or sign"


def test_bf16_widen_exact():
    b = np.arange(65536, dtype=np.uint16)
    w = S.bf16_to_f32(b)
    assert np.array_equal(w.view(np.uint32) >> 16, b.astype(np.uint32))
    assert np.all(w.view(np.uint32) & 0xFFFF == 0)
    fin = np.isfinite(w)
    assert np.array_equal(S.f32_to_bf16(w[fin]), b[fin])


# ---- pack / chunk / gather -----------------------------------------------------

def _ragged_plan(N=4, cap=600):
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3]
    return numels, P.bucket_plan(numels, cap, N)


def test_pack_roundtrip_and_padding():
    numels, pl = _ragged_plan()
    rng = np.random.default_rng(1)
    grads = [rng.integers(1, 65536, n, dtype=np.uint16) for n in numels]
    flat = S.pack(pl, grads)
    for g, back in zip(grads, S.unpack(pl, flat)):
        assert np.array_equal(g, back)
    owned = np.zeros(pl.flat_numel, bool)
    for t, n in enumerate(numels):
        owned[pl.tensor_flat_offset(t):pl.tensor_flat_offset(t) + n] = True
    assert np.all(flat[~owned] == 0) and np.all(flat[owned] != 0)
    assert (~owned).sum() > 0  # this plan does pad
    for b in pl.buckets:  # a bucket's gradient bytes = its tensors' bytes
        assert 2 * np.count_nonzero(flat[b.flat_offset:b.flat_offset + b.padded]) == \
            2 * sum(numels[t] for t in b.tensors)


def test_chunk_gather_partition():
    numels, pl = _ragged_plan()
    flat = np.arange(pl.flat_numel, dtype=np.int64)
    shards = [S.chunk(pl, flat, s) for s in range(pl.world_n)]
    assert all(len(sh) == pl.shard_numel for sh in shards)
    allidx = np.sort(np.concatenate(shards))
    assert np.array_equal(allidx, flat)  # the N shards partition the buffer
    assert np.array_equal(S.gather(pl, shards), flat)
    b = pl.buckets[-1]
    assert shards[1][b.shard_offset] == b.flat_offset + b.chunk


# ---- reduce ------------------------------------------------------------------

def test_reduce_ascending_order_by_hand():
    # 2^24 + 1 rounds back to 2^24 (tie, even), so ascending order gives 2^24
    # while adding the two ones first would give 2^24 + 2.
    big, one = bf16([2.0 ** 24])[0], bf16([1.0])[0]
    peers = [np.array([big]), np.array([one]), np.array([one])]
    assert S.reduce_peers(peers)[0] == 2.0 ** 24
    assert S.reduce_peers(peers[::-1])[0] == 2.0 ** 24 + 2


def test_reduce_keeps_negative_zero():
    nz = np.array([0x8000], np.uint16)
    s = S.reduce_peers([nz, nz, nz])
    assert s.view(np.uint32)[0] == 0x80000000


def test_reduce_error_bound_and_exact_pairs():
    rng = np.random.default_rng(3)
    n = 1 << 16
    for R in (1, 2, 3, 8, 16):
        peers = [synth.normal_bf16(9, synth.peer_stream(1, 0, r), n, 1e-3) for r in range(R)]
        s = S.reduce_peers(peers).astype(np.float64)
        vals = np.stack([S.bf16_to_f32(p).astype(np.float64) for p in peers])
        exact = vals.sum(0)  # exact: 8-bit significands within a narrow exponent range
        gamma = (R - 1) * U / (1 - (R - 1) * U)
        assert np.all(np.abs(s - exact) <= gamma * np.abs(vals).sum(0))
        if R == 1:
            assert np.array_equal(s, exact)
    # two bf16 values whose exponents differ by <= 15 add exactly in binary32
    a = rng.normal(size=n).astype(np.float32)
    b = (rng.normal(size=n) * 2.0 ** rng.integers(-15, 16, n)).astype(np.float32)
    pa, pb = S.f32_to_bf16(a), S.f32_to_bf16(b)
    ea, eb = (pa.astype(np.int32) >> 7) & 0xFF, (pb.astype(np.int32) >> 7) & 0xFF
    ok = (np.abs(ea - eb) <= 15) & (ea > 0) & (eb > 0)
    got = S.reduce_peers([pa[ok], pb[ok]]).astype(np.float64)
    want = S.bf16_to_f32(pa[ok]).astype(np.float64) + S.bf16_to_f32(pb[ok]).astype(np.float64)
    assert ok.sum() > n // 2 and np.array_equal(got, want)


def test_reduce_scatter_then_all_gather_equals_all_reduce():
    """Ring all-reduce = reduce-scatter + all-gather ("Parallelism Starts With the
    Bottleneck", section "Allreduce equals reducescatter plus allgather")."""
    numels, pl = _ragged_plan(N=4)
    R = pl.world_n
    flats = [S.pack(pl, [synth.normal_bf16(5, synth.tensor_stream(1, 0, r, t), n, 1e-2)
                         for t, n in enumerate(numels)]) for r in range(R)]
    all_reduce = S.reduce_peers(flats)
    rs = [S.reduce_peers([S.chunk(pl, f, s) for f in flats]) for s in range(R)]
    ag = S.gather(pl, rs)
    assert np.array_equal(ag.view(np.uint32), all_reduce.view(np.uint32))


# ---- normalise / accumulate ----------------------------------------------------

def test_mean_scale_values():
    assert S.mean_scale(2) == np.float32(0.5) and S.mean_scale(8) == np.float32(0.125)
    assert S.mean_scale(8, 4) == np.float32(1 / 32)
    assert S.mean_scale(3) == np.float32(1 / 3)


def test_token_normalisation_equals_global_token_mean():
    """Scaling each rank's summed loss by R/C under a 1/R average gives the mean
    over all C valid tokens ("Distributed Training and Parallelism", section
    "Data parallelism and the global gradient")."""
    rng = np.random.default_rng(11)
    counts = [1000, 1500, 1596]  # unequal, C = 4096 = 2^12
    C = sum(counts)
    n = 512
    # per-token gradient contributions: small dyadic values, so every rank's
    # summed gradient is a bf16 value and every sum is exact
    x = [rng.choice([-1, 0, 0, 0, 1], size=(c, n)).astype(np.float64) * 2.0 ** -12 for c in counts]
    P_r = [xi.sum(0) for xi in x]
    peers = [bf16(p) for p in P_r]
    g = S.normalise(S.reduce_peers(peers), S.tokens_scale(counts))
    global_mean = np.concatenate(x).sum(0) / C
    assert np.array_equal(g.astype(np.float64), global_mean)  # exact: C is a power of two
    # the naive mean of per-rank means is a different quantity here
    naive = np.mean([p / c for p, c in zip(P_r, counts)], axis=0)
    assert np.max(np.abs(naive - global_mean)) > 1e-6


def test_token_normalisation_general_counts_one_ulp():
    n = 4096
    R = 8
    for t in range(1, 6):
        counts = [synth.tokens(3, t, r) for r in range(R)]
        peers = [synth.normal_bf16(3, synth.peer_stream(t, 0, r), n, 1e-3) for r in range(R)]
        G = S.reduce_peers(peers)
        g = S.normalise(G, S.tokens_scale(counts))
        C = sum(counts)
        exact = np.array([float(Fraction(float(v)) / C) for v in G])
        assert np.all(np.abs(g - exact) <= ulp32(exact) * 1.0 + 1e-45)


def test_accumulate_microbatches():
    n, R, K = 4096, 4, 4
    acc = None
    contributions = []
    for k in range(K):
        peers = [synth.normal_bf16(2, synth.peer_stream(1, k, r), n, 1e-3) for r in range(R)]
        contributions += [S.bf16_to_f32(p).astype(np.float64) for p in peers]
        s_k = S.reduce_peers(peers)
        if k < K - 1:
            acc = S.accumulate(acc, s_k)
        else:
            G = s_k if acc is None else acc + s_k
    vals = np.stack(contributions)
    exact = vals.sum(0)
    m = R * K
    gamma = (m - 1) * U / (1 - (m - 1) * U)
    assert np.all(np.abs(G.astype(np.float64) - exact) <= gamma * np.abs(vals).sum(0))
    # first microbatch copies; identical microbatches of a power-of-two count
    # average back exactly
    s = S.reduce_peers([synth.normal_bf16(2, synth.peer_stream(9, 0, 0), n, 1e-3)])
    a = S.accumulate(None, s)
    assert a is not s and np.array_equal(a, s)
    for _ in range(3):
        a = S.accumulate(a, s)
    assert np.array_equal(S.normalise(a, S.mean_scale(1, 4)), s)


# ---- AdamW -------------------------------------------------------------------

def test_adamw_dyadic_golden():
    for ln in read_golden("adamw_dyadic.txt"):
        kv = dict(tok.split("=") for tok in ln.split()[1:])
        kv = {k: float(v) for k, v in kv.items()}
        sc = S.adamw_scalars(kv["lr"], kv["beta1"], kv["beta2"], kv["eps"], kv["wd"], int(kv["t"]))
        th, m, v = S.adamw(f32([kv["theta"]]), f32([kv["m"]]), f32([kv["v"]]), f32([kv["g"]]), sc)
        assert (th[0], m[0], v[0]) == (kv["theta1"], kv["m1"], kv["v1"]), ln


def test_adamw_step_one_closed_form():
    """At t = 1 with zero moments the update is lr*g/(|g|+eps) after the decay."""
    hp = synth.AdamW()
    n = 1 << 18
    theta = synth.normal_f32(4, synth.master_stream(0), n, 0.02)
    g = S.bf16_to_f32(synth.normal_bf16(4, synth.peer_stream(1, 0, 0), n, 1e-2))
    sc = S.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1)
    th1, m1, v1 = S.adamw(theta, np.zeros(n, np.float32), np.zeros(n, np.float32), g, sc)
    lr, wd, eps = (float(np.float32(x)) for x in (hp.lr, hp.weight_decay, hp.eps))
    gd, td = g.astype(np.float64), theta.astype(np.float64)
    decayed = td * (1 - lr * wd)
    update = lr * gd / (np.abs(gd) + eps)
    closed = decayed - update
    scale = np.maximum(np.abs(decayed), np.abs(update))
    err = np.abs(th1.astype(np.float64) - closed) / ulp32(scale)
    assert err.max() <= 4.0, err.max()
    assert np.array_equal(m1, sc.omb1 * g)
    assert np.array_equal(v1, sc.omb2 * (g * g))


def test_adamw_matches_torch_adamw():
    """torch.optim.AdamW (CPU, fp32) orders some operations differently (a lerp
    for m, a divide by sqrt(bc2)), so agreement is within a few ulp, not
    bitwise.  Each of ten steps starts the oracle from torch's own state, so
    differences do not accumulate; they are measured in ulp of the larger term
    of each update (m and theta can cancel towards 0)."""
    hp = synth.AdamW()
    n = 1 << 15
    theta0 = synth.normal_f32(6, synth.master_stream(0), n, 0.02)
    p = torch.nn.Parameter(torch.from_numpy(theta0.copy()))
    # the hyperparameters are binary32 values; hand torch exactly those
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in
                           (hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False, fused=False)
    th, m, v = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 11):
        g = S.bf16_to_f32(synth.normal_bf16(6, synth.peer_stream(t, 0, 0), n, 1e-2))
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        sc = S.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t)
        th1, m1, v1 = S.adamw(th, m, v, g, sc)
        st = opt.state[p]
        tt, tm, tv = (p.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
                      st["exp_avg_sq"].numpy().copy())
        m_scale = np.maximum(np.abs(sc.beta1 * m), np.abs(sc.omb1 * g))
        v_scale = np.maximum(np.abs(sc.beta2 * v), np.abs(sc.omb2 * g * g))
        # m's rounding (at m_scale) reaches theta through step_size/d, so the
        # update's scale is step_size*m_scale/d even when m itself cancels
        d = np.sqrt(v1) * sc.c2 + sc.eps
        upd_scale = sc.step_size * m_scale.astype(np.float64) / d
        th_scale = np.maximum.reduce([np.abs(th * sc.decay), np.abs(th1),
                                      np.abs(th * sc.decay - th1), upd_scale])
        assert np.max(np.abs(m1 - tm) / ulp32(m_scale)) <= 2
        assert np.max(np.abs(v1 - tv) / ulp32(v_scale)) <= 2
        # each side rounds d (sqrt, bias-correction constant, product or
        # quotient, + eps), the quotient and the step product differently:
        # about 7u relative on the update, plus the final rounding
        assert np.max(np.abs(th1 - tt) / ulp32(th_scale)) <= 8
        th, m, v = tt, tm, tv


def test_adamw_float64_step_bound():
    """Each fp32 step against the same step in float64 from the same fp32 state.

    Rounding count per element: m' two products and a sum (half an ulp of
    each product's term, and half an ulp of a sum that can reach twice the
    larger term: <= 2 ulp of that term), v' three products and a sum
    (<= 2.5), theta' the decay
    product, the update (sqrt, two rounded constants, the product with c2,
    + eps, the quotient, the step product: about 3.5u relative, plus m's
    own rounding carried through step_size/d) and the final difference."""
    hp = synth.AdamW()
    n = 1 << 15
    th = synth.normal_f32(8, synth.master_stream(0), n, 0.02)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in
                           (hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay))
    for t in range(1, 11):
        g = S.bf16_to_f32(synth.normal_bf16(8, synth.peer_stream(t, 0, 0), n, 1e-2))
        sc = S.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t)
        th1, m1, v1 = S.adamw(th, m, v, g, sc)
        gd, md, vd, td = (a.astype(np.float64) for a in (g, m, v, th))
        m64 = b1 * md + (1 - b1) * gd
        v64 = b2 * vd + (1 - b2) * gd * gd
        upd64 = lr * (m64 / (1 - b1 ** t)) / (np.sqrt(v64 / (1 - b2 ** t)) + eps)
        th64 = td * (1 - lr * wd) - upd64
        m_scale = np.maximum(np.abs(b1 * md), np.abs((1 - b1) * gd))
        v_scale = np.maximum(np.abs(b2 * vd), np.abs((1 - b2) * gd * gd))
        d = np.sqrt(v64 / (1 - b2 ** t)) + eps
        th_scale = np.maximum.reduce([np.abs(td * (1 - lr * wd)), np.abs(th64), np.abs(upd64),
                                      lr / (1 - b1 ** t) * m_scale / d])
        assert np.max(np.abs(m1 - m64) / ulp32(m_scale)) <= 2
        assert np.max(np.abs(v1 - v64) / ulp32(v_scale)) <= 2.5
        assert np.max(np.abs(th1 - th64) / ulp32(th_scale)) <= 6
        th, m, v = th1, m1, v1


def test_adamw_zero_gradient_and_padding():
    hp = synth.AdamW()
    theta = synth.normal_f32(1, synth.master_stream(0), 1000, 0.02)
    theta[:10] = 0
    th, m, v = theta.copy(), np.zeros(1000, np.float32), np.zeros(1000, np.float32)
    for t in range(1, 11):
        sc = S.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t)
        prev = th
        th, m, v = S.adamw(th, m, v, np.zeros(1000, np.float32), sc)
        assert np.array_equal(th, prev * sc.decay)  # only the decay acts
        assert not m.any() and not v.any()
    assert np.all(th[:10].view(np.uint32) == 0)  # padding slots stay +0


def test_adamw_nan_propagates_elementwise():
    hp = synth.AdamW()
    sc = S.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1)
    g = f32([np.nan, 1e-3, np.inf, -1e-3])
    with np.errstate(invalid="ignore"):
        th, m, v = S.adamw(f32([0.1] * 4), np.zeros(4, np.float32), np.zeros(4, np.float32), g, sc)
    assert np.isnan(th[0]) and np.isfinite(th[1]) and np.isnan(th[2]) and np.isfinite(th[3])
    p = S.f32_to_bf16(th)
    assert np.isnan(S.bf16_to_f32(p[[0, 2]])).all()


def test_adamw_scalars():
    sc = S.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    b1, b2 = float(np.float32(0.9)), float(np.float32(0.999))
    assert float(sc.omb1) == 1 - b1 and float(sc.omb2) == 1 - b2  # exact (Sterbenz)
    assert sc.step_size == np.float32(float(np.float32(1e-3)) / (1 - b1))
    with pytest.raises(ValueError):
        S.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 0)


# ---- the composed step: sharding invariants --------------------------------------

def _full_model_run(numels, N, steps, seed=21, cap=600, hp=None, reshard_at=None):
    """Run `steps` shard steps for every rank of an N-way sharded ragged model.

    Returns per-tensor fp32 masters after the last step.  With reshard_at, the
    run switches from N shards to one (N=1) after that many steps.
    """
    hp = hp or synth.AdamW()
    pl = P.bucket_plan(numels, cap, N)
    R = 4  # data-parallel contributions (independent of N)
    masters = [synth.normal_f32(seed, synth.tensor_stream(0, 0, 0, t), n, 0.02)
               for t, n in enumerate(numels)]
    flat_master = np.zeros(pl.flat_numel, np.float32)
    for t, mt in enumerate(masters):
        flat_master[pl.tensor_flat_offset(t):pl.tensor_flat_offset(t) + len(mt)] = mt
    state = [[S.chunk(pl, flat_master, s), np.zeros(pl.shard_numel, np.float32),
              np.zeros(pl.shard_numel, np.float32)] for s in range(N)]
    for t in range(1, steps + 1):
        if reshard_at is not None and t == reshard_at + 1:
            full = [S.unpack(pl, S.gather(pl, [st[i] for st in state])) for i in range(3)]
            pl = P.bucket_plan(numels, cap, 1)
            N = 1
            state = [[np.zeros(pl.flat_numel, np.float32) for _ in range(3)]]
            for i in range(3):
                for tt in range(len(numels)):
                    o = pl.tensor_flat_offset(tt)
                    state[0][i][o:o + numels[tt]] = full[i][tt]
        flats = [S.pack(pl, [synth.normal_bf16(seed, synth.tensor_stream(t, 0, r, tt), n, 1e-2)
                             for tt, n in enumerate(numels)]) for r in range(R)]
        for s in range(N):
            peers = [S.chunk(pl, f, s) for f in flats]
            th, m, v, _ = S.shard_step(peers, None, S.mean_scale(R), *state[s], hp, t)
            state[s] = [th, m, v]
    return S.unpack(pl, S.gather(pl, [st[0] for st in state])), pl, state


def test_union_of_shard_updates_equals_unsharded_update():
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3]
    ref, _, _ = _full_model_run(numels, 1, 3)
    for N in (2, 3, 4):
        got, _, _ = _full_model_run(numels, N, 3)
        for a, b in zip(got, ref):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_padding_state_stays_zero():
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3]
    _, pl, state = _full_model_run(numels, 4, 4)
    owned = np.zeros(pl.flat_numel, bool)
    for t, n in enumerate(numels):
        owned[pl.tensor_flat_offset(t):pl.tensor_flat_offset(t) + n] = True
    for i in range(3):
        flat = S.gather(pl, [st[i] for st in state])
        assert np.all(flat[~owned].view(np.uint32) == 0)
    assert (~owned).any()


def test_resume_and_reshard_equal_continuous_run():
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3]
    ref, _, _ = _full_model_run(numels, 1, 6)
    resharded, _, _ = _full_model_run(numels, 2, 6, reshard_at=3)
    for a, b in zip(resharded, ref):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_shard_step_composition_and_bf16_emit():
    hp = synth.AdamW()
    n, R = 3000, 3
    peers = [synth.normal_bf16(1, synth.peer_stream(1, 0, r), n, 1e-3) for r in range(R)]
    theta = synth.normal_f32(1, synth.master_stream(0), n, 0.02)
    z = np.zeros(n, np.float32)
    th, m, v, p = S.shard_step(peers, None, S.mean_scale(R), theta, z, z, hp, 1)
    assert np.array_equal(p, S.f32_to_bf16(th))
    # an accumulator alone (R = 0) gives the same as reducing the same values
    acc = S.reduce_peers(peers)
    th2, _, _, _ = S.shard_step([], acc, S.mean_scale(R), theta, z, z, hp, 1)
    assert np.array_equal(th, th2)
    # emitted bf16 differs from the master by at most half a bf16 ulp
    back = S.bf16_to_f32(p).astype(np.float64)
    assert np.all(np.abs(back - th) <= ulp32(th) * 2 ** 15 * 1.0000001 + 1e-45)


# ---- global gradient-norm clipping ----------------------------------------------

def test_grad_sq_norm_exact_and_sharded():
    """The squared norm is the correctly rounded float64 sum of exact squares;
    summing the shards' squared norms (the all-reduce the page asks for)
    gives the unsharded norm."""
    numels, pl = _ragged_plan(N=4)
    R = 3
    flats = [S.pack(pl, [synth.normal_bf16(6, synth.tensor_stream(1, 0, r, t), n, 1e-2)
                         for t, n in enumerate(numels)]) for r in range(R)]
    scale = S.mean_scale(R)
    G_full = S.reduce_peers(flats)
    full = S.grad_sq_norm(G_full, scale)
    g = S.normalise(G_full, scale)
    exact = sum(Fraction(float(x)) ** 2 for x in g)
    assert full == float(exact)  # fsum rounds the exact sum once
    parts = [S.grad_sq_norm(S.reduce_peers([S.chunk(pl, f, s) for f in flats]), scale)
             for s in range(pl.world_n)]
    assert abs(sum(parts) - full) <= 4 * 2.0 ** -53 * full
    # padding contributes nothing; zero gradient has zero norm
    assert S.grad_sq_norm(np.zeros(10, np.float32), scale) == 0.0


def test_clip_coefficient_and_clipped_norm():
    n = 4096
    G = S.reduce_peers([synth.normal_bf16(8, synth.peer_stream(1, 0, r), n, 1e-1)
                        for r in range(2)])
    scale = S.mean_scale(2)
    sq = S.grad_sq_norm(G, scale)
    norm = math.sqrt(sq)
    assert S.clip_coef(sq, 10 * norm) == 1.0  # below the threshold: untouched
    assert S.clipped_scale(scale, 1.0) == scale
    max_norm = float(np.float32(norm / 4))  # a binary32 hyperparameter
    c = S.clip_coef(sq, max_norm)
    assert 0.24 < c < 0.26  # a quarter, less the 1e-6 in the denominator
    cs = S.clipped_scale(scale, c)
    clipped = math.sqrt(S.grad_sq_norm(G, cs))
    assert abs(clipped / max_norm - 1) < 1e-6  # the clipped gradient has the target norm
    assert math.isnan(S.clip_coef(float("nan"), 1.0))  # NaN propagates
    assert S.clip_coef(float("inf"), 1.0) == 0.0


def test_clip_coefficient_golden():
    """Hand-worked coefficients and clipped scales (tests/golden/clip_coef.txt):
    dyadic norms where the 1e-6 rounds away, a zero norm, the binary32
    reading of max_norm, and a tiny norm the 1e-6 dominates."""
    rows = 0
    for ln in read_golden("clip_coef.txt"):
        f = ln.split()
        if f[0] == "coef":
            got = S.clip_coef(float.fromhex(f[1]), float(f[2]))
            assert got == float.fromhex(f[3]), ln
        elif f[0] == "bound":
            got = S.clip_coef(float.fromhex(f[1]), float(f[2]))
            assert float(f[3]) < got < float(f[4]), (ln, got)
        else:
            got = S.clipped_scale(np.float32(float.fromhex(f[1])), float.fromhex(f[2]))
            assert float(got) == float.fromhex(f[3]), ln
        rows += 1
    assert rows == 10


def test_clip_matches_torch_clip_grad_norm():
    """torch.nn.utils.clip_grad_norm_ (fp32 norm, same coefficient rule)."""
    n = 1 << 14
    G = S.reduce_peers([synth.normal_bf16(9, synth.peer_stream(1, 0, r), n, 1e-1)
                        for r in range(4)])
    scale = S.mean_scale(4)
    g = S.normalise(G, scale)
    for max_norm in (0.05, 0.5, 50.0):
        p = torch.nn.Parameter(torch.zeros(n))
        p.grad = torch.from_numpy(g.copy())
        total = torch.nn.utils.clip_grad_norm_([p], max_norm)
        sq = S.grad_sq_norm(G, scale)
        assert abs(float(total) - math.sqrt(sq)) <= 1e-6 * math.sqrt(sq)
        ref = p.grad.numpy().astype(np.float64)
        ours = S.normalise(G, S.clipped_scale(scale, S.clip_coef(sq, max_norm)))
        # torch's norm is an fp32 reduction (about 1e-6 relative), ours exact
        assert np.all(np.abs(ours - ref) <= 2e-6 * np.abs(ref) + 1e-30)
        if max_norm == 50.0:  # no clipping: identical to the unclipped gradient
            assert np.array_equal(ours, g)



# ---- parameter groups --------------------------------------------------------------

def test_grouped_step_reduces_to_plain_and_zero_decay_group():
    n, R = 5000, 3
    hp = synth.AdamW()
    peers = [synth.normal_bf16(12, synth.peer_stream(1, 0, r), n, 1e-2) for r in range(R)]
    theta = synth.normal_f32(12, synth.master_stream(0), n, 0.02)
    z = np.zeros(n, np.float32)
    eg = (np.arange(n) // 700 % 2).astype(np.int32)
    same = [(hp.lr, hp.weight_decay)] * 2
    a = S.shard_step_grouped(peers, None, S.mean_scale(R), theta, z, z, hp, same, eg, 1)
    b = S.shard_step(peers, None, S.mean_scale(R), theta, z, z, hp, 1)
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x).view(np.uint32 if x.dtype == np.float32 else np.uint16),
                              np.asarray(y).view(np.uint32 if y.dtype == np.float32 else np.uint16))
    # group 1 without decay: theta' = theta - step*(m'/d) exactly (decay is 1)
    two = [(hp.lr, hp.weight_decay), (hp.lr, 0.0)]
    th, m1, v1, _ = S.shard_step_grouped(peers, None, S.mean_scale(R), theta, z, z, hp, two, eg, 1)
    sc = S.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, 0.0, 1)
    assert sc.decay == 1
    g = S.normalise(S.reduce_peers(peers), S.mean_scale(R))
    want = theta - sc.step_size * (m1 / (np.sqrt(v1) * sc.c2 + sc.eps))
    sel = eg == 1
    assert np.array_equal(th[sel], want[sel]) and not np.array_equal(th[~sel], want[~sel])
    assert np.array_equal(m1, sc.omb1 * g)


def test_grouped_matches_torch_param_groups():
    """torch.optim.AdamW with two parameter groups (decay / no decay), one step
    from the same state, within the per-step bound of the plain comparison."""
    hp = synth.AdamW()
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in
                           (hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay))
    n1, n2 = 3000, 500
    th0 = synth.normal_f32(13, synth.master_stream(0), n1 + n2, 0.02)
    g = S.bf16_to_f32(synth.normal_bf16(13, synth.peer_stream(1, 0, 0), n1 + n2, 1e-2))
    p1 = torch.nn.Parameter(torch.from_numpy(th0[:n1].copy()))
    p2 = torch.nn.Parameter(torch.from_numpy(th0[n1:].copy()))
    opt = torch.optim.AdamW([{"params": [p1], "weight_decay": wd},
                             {"params": [p2], "weight_decay": 0.0, "lr": lr * 2}],
                            lr=lr, betas=(b1, b2), eps=eps, foreach=False, fused=False)
    p1.grad = torch.from_numpy(g[:n1].copy())
    p2.grad = torch.from_numpy(g[n1:].copy())
    opt.step()
    eg = np.r_[np.zeros(n1, np.int32), np.ones(n2, np.int32)]
    z = np.zeros(n1 + n2, np.float32)
    th, _, _, _ = S.shard_step_grouped([S.f32_to_bf16(g)], None, np.float32(1.0), th0, z, z, hp,
                                       [(lr, wd), (lr * 2, 0.0)], eg, 1)
    ref = np.r_[p1.detach().numpy(), p2.detach().numpy()]
    upd = np.abs(th0 - ref) + np.abs(th0)
    assert np.max(np.abs(th - ref) / ulp32(upd)) <= 8


def test_shard_groups_follow_tensors_and_padding():
    # the second and third plans leave whole shards of padding (tensor 0
    # alone in a 32-element bucket), so a shard can start with padding
    for numels, cap, tg in (([37, 8, 1, 130, 0, 64, 9, 250, 3], 600, None),
                            ([3, 5], 2, [2, 1]), ([3], 1 << 20, [1])):
        _check_shard_groups(numels, cap, tg)


def _check_shard_groups(numels, cap, tg):
    pl = P.bucket_plan(numels, cap, 4)
    tg = tg or [t % 3 for t in range(len(numels))]
    for s in range(4):
        g = S.shard_groups(pl, s, tg)
        flat_ids = S.chunk(pl, np.arange(pl.flat_numel), s)
        prev = 0
        for j, fpos in enumerate(flat_ids):
            owner = [t for t in range(len(numels)) if numels[t] and
                     pl.tensor_flat_offset(t) <= fpos < pl.tensor_flat_offset(t) + numels[t]]
            want = tg[owner[0]] if owner else prev
            assert g[j] == want
            prev = want


def test_bias_corrections_settle_at_one():
    """Facts of float64 arithmetic that let a caller stop forming beta^t early.
    1 - x rounds to 1 exactly when 0 <= x <= 2^-54 (the tie at 2^-54 goes to
    the even 1.0); a subnormal power can be a fixed point of the rounded
    product, so waiting for 0 may never end; and once both powers are at most
    2^-54 the oracle's scalars no longer change with t."""
    tiny = 2.0 ** -54
    assert 1.0 - tiny == 1.0
    assert 1.0 - math.nextafter(tiny, 1.0) < 1.0
    b = float(np.float32(0.9))
    x = 4 * 2.0 ** -1074
    assert x * b == x and x > 0.0
    for beta1, beta2 in [(0.9, 0.95), (0.8, 0.99), (0.5, 0.5)]:
        b1, b2 = float(np.float32(beta1)), float(np.float32(beta2))
        t = 1
        while b1 ** t > tiny or b2 ** t > tiny:
            t += 1
        base = S.adamw_scalars(1e-3, beta1, beta2, 1e-8, 0.1, t + 2)
        for later in (t + 3, 2 * t + 50, 5 * t):
            assert S.adamw_scalars(1e-3, beta1, beta2, 1e-8, 0.1, later) == base
        assert base.c2 == 1.0 and base.step_size == np.float32(1e-3)
