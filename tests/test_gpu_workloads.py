"""GPU parity on the five synthetic workloads, in the launch configuration and
placement the benchmark times.  The comparison is over every element, at
model scale too: there the oracle runs slice by slice in worker processes on
the host's cores (tests/oracle_pool.py; the step is elementwise once the plan
is fixed, and the inputs of any element can be regenerated on their own).
The all-gather side at full scale is compared over sampled elements, which the
oracle computes one by one."""

import numpy as np
import pytest

import sharded_bucket_plan_amd as sbp
import synth
from oracle import plan as OP
from oracle import step as OS
from tests import helpers as H

pytestmark = pytest.mark.gpu

SEED = synth.SEED


@pytest.fixture(autouse=True)
def _gpu():
    H.need_gpu()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _hp(w):
    return sbp.AdamW(w.adamw.lr, w.adamw.beta1, w.adamw.beta2, w.adamw.eps, w.adamw.weight_decay)


@pytest.mark.parametrize("s", [0, 1])
def test_tiny_mlp_all_steps(s):
    """2-layer MLP, N=2, R=2: each rank packs its per-tensor gradients, this
    rank's chunk of each is reduced, 10 optimizer steps, every element."""
    import torch
    w = synth.WORKLOADS["tiny_mlp"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    opl = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    th = synth.normal_f32(SEED, synth.master_stream(s), n, w.master_sigma)
    z = np.zeros(n, np.float32)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(z), H.from_np_f32(z)
    dp = H.empty_u16(n)
    flats = [H.empty_u16(pl.flat_numel) for _ in range(w.R)]
    grads = [[H.empty_u16(k) for k in w.numels] for _ in range(w.R)]
    peers = [H.empty_u16(n) for _ in range(w.R)]
    want = (th, z, z, None)
    for t in range(1, w.steps + 1):
        host_flats = []
        for r in range(w.R):
            gh = []
            for tid, k in enumerate(w.numels):
                st = synth.tensor_stream(t, 0, r, tid)
                synth.dev_normal_bf16(grads[r][tid], SEED, st, w.grad_sigma)
                gh.append(synth.normal_bf16(SEED, st, k, w.grad_sigma))
            sbp.pack_grads(pl, grads[r], flats[r])
            host_flats.append(OS.pack(opl, gh))
        for r in range(w.R):  # rank r's contribution to this rank's shard
            sbp.shard_of(pl, s, flats[r], peers[r])
        scale = sbp.mean_scale(w.R)
        sbp.adamw_shard(peers, None, scale, dth, dm, dv, dp, hp, t)
        want = OS.shard_step([OS.chunk(opl, f, s) for f in host_flats], None,
                             OS.mean_scale(w.R), want[0], want[1], want[2], hp, t)
        torch.cuda.synchronize()
        for r in range(w.R):
            H.assert_bits_equal(H.to_np_u16(flats[r]), host_flats[r], f"pack rank {r} step {t}")
        got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
        for a, b, name in zip(got, want, ("master", "m", "v", "param")):
            H.assert_bits_equal(a, b, f"tiny_mlp s={s} step {t} {name}")


@pytest.mark.parametrize("s", range(8))
def test_gpt2_small_full(s):
    """GPT-2-small ZeRO-2 shard (N=8, R=8, 15.5M elements), every shard index:
    every element after every step -- ten steps (the workloads' AdamW run)
    for shard 0, two for the others (whose master weights differ)."""
    import torch
    w = synth.WORKLOADS["gpt2_small"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 15554976
    th = synth.normal_f32(SEED, synth.master_stream(s), n, w.master_sigma)
    z = np.zeros(n, np.float32)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(z), H.from_np_f32(z)
    dp = H.empty_u16(n)
    bufs = None
    want = (th, z, z, None)
    for t in range(1, (10 if s == 0 else 2) + 1):
        bufs = H.dev_peers(SEED, t, 0, w.R, n, w.grad_sigma, bufs)
        sbp.adamw_shard(bufs, None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t)
        want = OS.shard_step(H.host_peers(SEED, t, 0, w.R, n, w.grad_sigma), None,
                             OS.mean_scale(w.R), want[0], want[1], want[2], hp, t)
        torch.cuda.synchronize()
        got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
        for a_, b_, name in zip(got, want, ("master", "m", "v", "param")):
            H.assert_bits_equal(a_, b_, f"gpt2_small shard {s} step {t} {name}")


@pytest.mark.parametrize("s", range(8))
def test_gpt2_small_grouped_full(s):
    """GPT-2-small shard with the usual two parameter groups -- weight decay
    on matrices, none on biases, norm gains and other 1-D tensors -- plus a
    lower lr on the embeddings (a third group); every shard index (each has
    its own run table from the plan), two steps, every element."""
    import torch
    w = synth.WORKLOADS["gpt2_small"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    opl = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    groups = [(hp.lr, hp.weight_decay), (hp.lr, 0.0), (hp.lr * 0.5, hp.weight_decay)]
    tg = [1 if len(shape) == 1 else (2 if "wte" in name or "wpe" in name else 0)
          for name, shape in w.params]
    assert set(tg) == {0, 1, 2}
    rs, rg = sbp.group_table(pl, s, tg, H.dev())
    eg = OS.shard_groups(opl, s, tg)
    th = synth.normal_f32(SEED, synth.master_stream(s), n, w.master_sigma)
    z = np.zeros(n, np.float32)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(z), H.from_np_f32(z)
    dp = H.empty_u16(n)
    bufs = None
    want = (th, z, z, None)
    for t in (1, 2):
        bufs = H.dev_peers(SEED, t, 0, w.R, n, w.grad_sigma, bufs)
        sbp.adamw_shard_grouped(bufs, None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t,
                                groups, rs, rg)
        want = OS.shard_step_grouped(H.host_peers(SEED, t, 0, w.R, n, w.grad_sigma), None,
                                     OS.mean_scale(w.R), want[0], want[1], want[2], hp,
                                     groups, eg, t)
    torch.cuda.synchronize()
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    for a, b, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(a, b, f"gpt2_small grouped {name}")


def _sample_index(plan, n, count, seed):
    """Random elements plus the first and last element of every bucket's chunk
    and the shard's last 16 elements (ragged ends of each launch range)."""
    rng = np.random.default_rng(seed)
    idx = [rng.integers(0, n, count)]
    for b in range(plan.num_buckets):
        info = plan.bucket(b)
        o, c = info["shard_offset"], info["chunk"]
        idx.append(np.array([o, o + 1, o + c - 1, o + c - 2]))
    idx.append(np.arange(max(0, n - 16), n))
    idx = np.unique(np.concatenate(idx))
    return idx[(idx >= 0) & (idx < n)].astype(np.int64)


def _gather(t, idx_d):
    return t.index_select(0, idx_d)


def _sampled_state(dth, dm, dv, dp, idx):
    import torch
    idx_d = torch.from_numpy(idx).to(H.dev())
    return (H.to_np_f32(_gather(dth, idx_d)), H.to_np_f32(_gather(dm, idx_d)),
            H.to_np_f32(_gather(dv, idx_d)), H.to_np_u16(_gather(dp, idx_d)))


def _compare_slices(results, arrays, recompute, what, every=8):
    """Compares the oracle workers' digests of each slice with digests of the
    GPU's copy of the same slice; a differing slice is recomputed here and
    compared element by element (the assertion then names the element)."""
    from tests import oracle_pool as OPL
    done = 0
    for job, want in results:
        i0, i1 = job[2], job[3]
        got_arrays = [H.to_np_f32(a[i0:i1]) for a in arrays[:3]] + [H.to_np_u16(arrays[3][i0:i1])]
        if OPL.digests(got_arrays) != want:
            exp = recompute(job)
            for x, y, name in zip(got_arrays, exp, ("master", "m", "v", "param")):
                H.assert_bits_equal(x, y, f"{what} {name} in [{i0}, {i1})")
            raise AssertionError(f"{what}: digests of [{i0}, {i1}) differ but the arrays agree")
        done += 1
        if done % every == 0:
            print(f"{what}: {done} slices equal (through element {i1})", flush=True)
    return done


def _arena_state(n, R, K=1, with_acc=False, with_g=False):
    """The step's arrays in one spread arena, as bench.py places them:
    master, m, v, param shard, then K microbatches of R peers (+ acc, + the
    stored G of a clipped step)."""
    import torch
    sizes = ([4 * n] * 3 + [2 * n] + [2 * n] * (R * K) + ([4 * n] if with_acc else [])
             + ([4 * n] if with_g else []))
    a = sbp.Arena(sizes)
    th, m, v = (a.tensor(j, torch.float32, n) for j in range(3))
    p = a.tensor(3, torch.int16, n)
    mb = [[a.tensor(4 + k * R + r, torch.int16, n) for r in range(R)] for k in range(K)]
    acc = a.tensor(4 + R * K, torch.float32, n) if with_acc else None
    if with_g:
        return a, th, m, v, p, mb, acc, a.tensor(len(sizes) - 1, torch.float32, n)
    return a, th, m, v, p, mb, acc


def test_llama3_8b_shard_full():
    """Llama-3-8B ZeRO-3 shard (N=8, R=8, 1,003,782,656 elements): the
    benchmark's workload, launch and placement (a spread arena), two steps,
    every element of master, m, v and the bf16 shard against the oracle run
    slice by slice on the host's cores."""
    from tests import oracle_pool as OPL
    import torch
    w = synth.WORKLOADS["llama3_8b"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 1003782656
    jobs = [("llama3_8b", SEED, i0, min(n, i0 + OPL.SLICE), 2) for i0 in range(0, n, OPL.SLICE)]
    with OPL.pool() as pool:
        results = pool.imap(OPL.shard_digests, jobs)  # the host works while the GPU does
        arena, dth, dm, dv, dp, mb, _ = _arena_state(n, w.R)
        synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
        dm.zero_()
        dv.zero_()
        for t in (1, 2):
            H.dev_peers(SEED, t, 0, w.R, n, w.grad_sigma, mb[0])
            sbp.adamw_shard(mb[0], None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t)
        torch.cuda.synchronize()
        print(f"llama3_8b: GPU steps done; comparing {len(jobs)} slices", flush=True)
        done = _compare_slices(results, (dth, dm, dv, dp),
                               lambda job: OPL.shard_state(job), "llama3_8b")
    assert done == len(jobs)


def _clipped_full(name, max_norm, slice_len, recompute=False):
    """One clipped step of workload `name` at full size, as bench.py --clip
    takes it: the first K - 1 microbatches accumulated over the whole shard,
    the norm pass over the accumulator and the last microbatch writing G and
    this rank's float64 squared norm, the clip coefficient folded into the
    scale, and the update reading G alone (recompute: as --clip-recompute
    takes it, the norm pass stores no G and the fused step sums the peers and
    the accumulator again, which gives the same bits).  The squared norm is checked
    against the oracle's (per-slice correctly rounded sums, then their
    correctly rounded sum) within the fixed tree's derived bound plus that
    extra rounding, the clipped scale must be the oracle's, and every element
    of the updated state is compared with the oracle's clipped step, slice by
    slice on the host's cores.  Returns the clip coefficient."""
    import math
    from tests import oracle_pool as OPL
    import torch
    w = synth.WORKLOADS[name]
    hp = _hp(w)
    n = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n).shard_numel
    accum = w.K > 1
    spans = [(i0, min(n, i0 + slice_len)) for i0 in range(0, n, slice_len)]
    with OPL.pool() as pool:
        parts = pool.imap(OPL.clip_norm_partial, [(name, SEED, i0, i1) for i0, i1 in spans])
        arena, dth, dm, dv, dp, mb, acc, dg = _arena_state(n, w.R, w.K, with_acc=accum,
                                                             with_g=True)
        synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
        dm.zero_()
        dv.zero_()
        if w.norm == "tokens":
            scale = sbp.tokens_scale([synth.tokens(SEED, 1, r) for r in range(w.R)])
        else:
            scale = sbp.mean_scale(w.R, w.K)
        for k in range(w.K):
            H.dev_peers(SEED, 1, k, w.R, n, w.grad_sigma, mb[k])
            if k < w.K - 1:
                sbp.accumulate_grads(acc, mb[k], first=(k == 0))
        sq = sbp.grad_sq_norm(mb[w.K - 1], acc, scale, n,
                              g_sum_out=None if recompute else dg).item()
        cs, coef = sbp.clip_scale(sq, max_norm, scale)
        if recompute:
            sbp.adamw_shard(mb[w.K - 1], acc, cs, dth, dm, dv, dp, hp, 1)
        else:
            sbp.adamw_shard([], dg, cs, dth, dm, dv, dp, hp, 1)
        torch.cuda.synchronize()
        want_total = math.fsum(p for _, p in parts)
        u = 2.0 ** -53
        d = H.sq_norm_depth(n, H.norm_gpl(w.R, accum))
        bound = (d * u / (1 - d * u) + 2 * u) * want_total * (1 + 1e-9)
        assert abs(sq - want_total) <= bound, (sq, want_total, bound)
        want_cs = float(OS.clipped_scale(OPL._step1_scale(w, SEED),
                                         OS.clip_coef(want_total, max_norm)))
        assert cs == want_cs, (cs, want_cs)
        print(f"{name} clipped: norm {math.sqrt(sq):.6g}, coefficient {coef:.6g}; "
              f"comparing {len(spans)} slices", flush=True)
        jobs = [(name, SEED, i0, i1, want_cs) for i0, i1 in spans]
        done = _compare_slices(pool.imap(OPL.clipped_digests, jobs), (dth, dm, dv, dp),
                               lambda job: OPL.clipped_state(job), f"{name} clipped")
    assert done == len(jobs)
    return coef


def test_llama3_8b_clipped_full():
    """The Llama-3-8B shard (R = 8, 1,003,782,656 elements) clipped at
    max_norm 1.0 (bench.py --clip 1.0): every element against the oracle."""
    from tests import oracle_pool as OPL
    assert _clipped_full("llama3_8b", 1.0, OPL.SLICE) < 1.0  # clipping is active


def test_llama3_8b_clipped_recompute_full():
    """The same clipped Llama step as --clip 1.0 --clip-recompute takes it:
    the norm pass reads the 8 peers only, then the fused step from the peers
    under the clipped scale; every element against the oracle."""
    from tests import oracle_pool as OPL
    assert _clipped_full("llama3_8b", 1.0, OPL.SLICE, recompute=True) < 1.0


def test_gpt_7b5_clipped_full():
    """The '7.5B' shard (R = 8, K = 4, 1/C, 103,890,048 elements) clipped: the
    norm pass reads the accumulator of three microbatches and the last one's
    peers.  max_norm 1e-3 (this shard's norm is about 3e-3, so bench.py's
    1.0 would not clip): every element against the oracle."""
    from tests import oracle_pool as OPL
    assert _clipped_full("gpt_7b5", 1e-3, OPL.SLICE // 4) < 1.0


def test_llama3_8b_grouped_full():
    """The Llama-3-8B shard with the benchmark's two parameter groups (decay on
    matrices, none on the 1-D tensors; bench.py --groups): two grouped steps,
    every element against the oracle's grouped step run slice by slice on the
    host's cores (each element's group found through the oracle's plan)."""
    from tests import oracle_pool as OPL
    import torch
    w = synth.WORKLOADS["llama3_8b"]
    hp = _hp(w)
    tg = [1 if len(shape) == 1 else 0 for _, shape in w.params]
    groups = [(hp.lr, hp.weight_decay), (hp.lr, 0.0)]
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    jobs = [("llama3_8b", SEED, i0, min(n, i0 + OPL.SLICE), 2) for i0 in range(0, n, OPL.SLICE)]
    # both groups occur (a slice holding a 1-D tensor's piece and a matrix's)
    g = OPL.shard0_groups("llama3_8b", 0, n)
    assert set(np.unique(g)) == {0, 1}
    with OPL.pool() as pool:
        results = pool.imap(OPL.grouped_digests, jobs)
        rs, rg = sbp.group_table(pl, 0, tg, H.dev())
        arena, dth, dm, dv, dp, mb, _ = _arena_state(n, w.R)
        synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
        dm.zero_()
        dv.zero_()
        for t in (1, 2):
            H.dev_peers(SEED, t, 0, w.R, n, w.grad_sigma, mb[0])
            sbp.adamw_shard_grouped(mb[0], None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t,
                                    groups, rs, rg)
        torch.cuda.synchronize()
        print(f"llama3_8b grouped: GPU steps done; comparing {len(jobs)} slices", flush=True)
        done = _compare_slices(results, (dth, dm, dv, dp),
                               lambda job: OPL.grouped_state(job), "llama3_8b grouped")
    assert done == len(jobs)


def test_gpt_7b5_accumulate_tokens_full():
    """'7.5B'-labelled GPT shard (N=64, R=8, 103,890,048 elements): 4
    microbatches, the first three accumulated bucket by bucket, the last
    fused; 1/C valid-token scaling; two steps; every element against the
    oracle run slice by slice on the host's cores."""
    from tests import oracle_pool as OPL
    import torch
    w = synth.WORKLOADS["gpt_7b5"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 103890048
    step = OPL.SLICE // 4
    jobs = [("gpt_7b5", SEED, i0, min(n, i0 + step), 2) for i0 in range(0, n, step)]
    with OPL.pool() as pool:
        results = pool.imap(OPL.shard_digests, jobs)
        arena, dth, dm, dv, dp, mb, acc = _arena_state(n, w.R, w.K, with_acc=True)
        synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
        dm.zero_()
        dv.zero_()
        ranges = [(pl.bucket(b)["shard_offset"], pl.bucket(b)["chunk"])
                  for b in range(pl.num_buckets)]
        for t in (1, 2):
            scale = sbp.tokens_scale([synth.tokens(SEED, t, r) for r in range(w.R)])
            for k in range(w.K):
                H.dev_peers(SEED, t, k, w.R, n, w.grad_sigma, mb[k])
                if k < w.K - 1:
                    for o, c in ranges:
                        sbp.accumulate_grads(acc[o:o + c], [x[o:o + c] for x in mb[k]],
                                             first=(k == 0))
                else:
                    sbp.adamw_shard(mb[k], acc, scale, dth, dm, dv, dp, hp, t)
        torch.cuda.synchronize()
        print(f"gpt_7b5: GPU steps done; comparing {len(jobs)} slices", flush=True)
        done = _compare_slices(results, (dth, dm, dv, dp),
                               lambda job: OPL.shard_state(job), "gpt_7b5")
    assert done == len(jobs)


def _dp_full(max_norm=None):
    """Llama-3-8B as a full DP replica (N=1, R=2, 8.03B elements): rank 0's
    291 per-tensor gradients packed into the 162 buckets, rank 1's
    bucket-layout gradient as the other contribution, one fused step -- with
    max_norm, clipped as bench.py --clip --clip-recompute takes it (the norm
    pass reads the two contributions and stores nothing; the fused step sums
    them again under the clipped scale).  Every element of every bucket (the
    packed gradient, master, m, v and the bf16 parameters) against the oracle
    run slice by slice on the host's cores; the first, the last and the
    largest bucket and 8 seeded random others are compared first."""
    import math
    from tests import oracle_pool as OPL
    import torch
    w = synth.WORKLOADS["llama3_8b_dp"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 8030261248 == pl.flat_numel
    B = pl.num_buckets
    info = [pl.bucket(b) for b in range(B)]
    largest = max(range(B), key=lambda b: info[b]["padded"])
    rng = np.random.default_rng(11)
    others = [b for b in range(B) if b not in (0, B - 1, largest)]
    chosen = sorted({0, B - 1, largest} | set(int(x) for x in rng.choice(others, 8, replace=False)))
    spans = []
    for b in chosen + [b for b in range(B) if b not in chosen]:
        o, c = info[b]["shard_offset"], info[b]["chunk"]
        spans += [(i0, min(o + c, i0 + OPL.SLICE)) for i0 in range(o, o + c, OPL.SLICE)]
    what = "llama3_8b_dp" + (" clipped" if max_norm else "")
    t = 1
    with OPL.pool() as pool:
        if max_norm:
            parts = pool.imap(OPL.dp_norm_partial,
                              [("llama3_8b_dp", SEED, i0, i1) for i0, i1 in spans])
        else:
            jobs = [("llama3_8b_dp", SEED, i0, i1) for i0, i1 in spans]
            results = pool.imap(OPL.dp_digests, jobs)
        sizes = [4 * n] * 3 + [2 * n] * 3  # master, m, v, param, rank 0 flat, rank 1
        arena = sbp.Arena(sizes)
        dth, dm, dv = (arena.tensor(j, torch.float32, n) for j in range(3))
        dp, flat0, peer1 = (arena.tensor(j, torch.int16, n) for j in range(3, 6))
        grads = []
        for tid, k in enumerate(w.numels):
            g = H.empty_u16(k)
            synth.dev_normal_bf16(g, SEED, synth.tensor_stream(t, 0, 0, tid), w.grad_sigma)
            grads.append(g)
        sbp.pack_grads(pl, grads, flat0)
        del grads
        synth.dev_normal_bf16(peer1, SEED, synth.peer_stream(t, 0, 1), w.grad_sigma)
        synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
        dm.zero_()
        dv.zero_()
        scale = sbp.mean_scale(w.R)
        if max_norm:
            sq = sbp.grad_sq_norm([flat0, peer1], None, scale, n).item()
            scale, coef = sbp.clip_scale(sq, max_norm, scale)
        sbp.adamw_shard([flat0, peer1], None, scale, dth, dm, dv, dp, hp, t)
        torch.cuda.synchronize()
        if max_norm:
            want_total = math.fsum(p for _, p in parts)
            u = 2.0 ** -53
            d = H.sq_norm_depth(n, H.norm_gpl(w.R, False))
            bound = (d * u / (1 - d * u) + 2 * u) * want_total * (1 + 1e-9)
            assert abs(sq - want_total) <= bound, (sq, want_total, bound)
            want_cs = float(OS.clipped_scale(OS.mean_scale(w.R),
                                             OS.clip_coef(want_total, max_norm)))
            assert scale == want_cs, (scale, want_cs)
            assert coef < 1.0
            print(f"{what}: norm {math.sqrt(sq):.6g}, coefficient {coef:.6g}", flush=True)
            jobs = [("llama3_8b_dp", SEED, i0, i1, want_cs) for i0, i1 in spans]
            results = pool.imap(OPL.dp_digests, jobs)
        print(f"{what}: GPU step done; comparing all {B} buckets ({chosen} first) in "
              f"{len(jobs)} slices", flush=True)
        done = 0
        for job, want in results:
            i0, i1 = job[2], job[3]
            got = ([H.to_np_f32(x[i0:i1]) for x in (dth, dm, dv)]
                   + [H.to_np_u16(dp[i0:i1]), H.to_np_u16(flat0[i0:i1])])
            if OPL.digests(got) != want:
                exp = OPL.dp_state(job)
                for x, y, name in zip(got, exp, ("master", "m", "v", "param", "packed rank 0")):
                    H.assert_bits_equal(x, y, f"{what} {name} in [{i0}, {i1})")
                raise AssertionError(f"{what}: digests of [{i0}, {i1}) differ")
            done += 1
            if done % 32 == 0:
                print(f"{what}: {done} slices equal (through element {i1})", flush=True)
    assert done == len(jobs)
    assert sum(j[3] - j[2] for j in jobs) == n


def test_llama3_8b_dp_pack_and_step_full():
    """The DP replica's pack and fused step, every element."""
    _dp_full()


def test_llama3_8b_dp_clip_recompute_full():
    """The DP replica clipped at max_norm 1.0 without a stored G: the norm
    pass over 8.03B elements (positions beyond 2^32, two groups of 8 per
    lane), then the fused step from the two contributions; every element."""
    _dp_full(max_norm=1.0)


@pytest.mark.parametrize("kind", ["whole", "per_tensor"])
def test_llama3_8b_all_gather_side_sampled(kind):
    """The all-gather side at full Llama-3-8B scale (N = 8, 8.03B parameter
    elements, flat positions beyond 2^32): the eight bf16 parameter shards go
    straight into the 291 per-tensor parameters (unpack_shards).  Sampled
    elements of every tensor (its first, its last and random ones) against the
    oracle plan's all-gather layout, element by element: element i of tensor t
    sits at flat position a = offset(t) + i of its bucket, which the gather
    fills from shard s = (a - bucket start) // chunk at the bucket's shard
    offset plus (a - bucket start - s * chunk)."""
    import torch
    w = synth.WORKLOADS["llama3_8b"]
    rows = [x[1] if len(x) == 2 else 1 for _, x in w.params]
    if kind == "per_tensor":
        pl = sbp.bucket_plan_per_tensor(w.numels, w.world_n, rows)
        opl = OP.per_tensor_plan(w.numels, w.world_n, rows)
    else:
        pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
        opl = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    N, n = w.world_n, pl.shard_numel
    assert n == opl.shard_numel and pl.flat_numel > 1 << 32
    shards = []
    for s in range(N):
        x = H.empty_u16(n)
        synth.dev_normal_bf16(x, SEED, synth.peer_stream(1, 0, s), 1.0)
        shards.append(x)
    params = [H.empty_u16(k) for k in w.numels]
    sbp.unpack_shards(pl, shards, params)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    fo_all = np.array([b.flat_offset for b in opl.buckets], np.int64)
    ch_all = np.array([b.chunk for b in opl.buckets], np.int64)
    so_all = np.array([b.shard_offset for b in opl.buckets], np.int64)
    for t, k in enumerate(w.numels):
        i = np.unique(np.concatenate([[0, k - 1], rng.integers(0, k, 64)])).astype(np.int64)
        a = opl.tensor_flat_offset(t) + i
        b = np.searchsorted(fo_all, a, side="right") - 1
        rel = a - fo_all[b]
        s = rel // ch_all[b]
        j = so_all[b] + rel - s * ch_all[b]
        want = np.empty(i.size, np.uint16)
        for r in np.unique(s):
            sel = s == r
            want[sel] = synth.normal_bf16_at(SEED, synth.peer_stream(1, 0, int(r)), j[sel], 1.0)
        got = H.to_np_u16(params[t].index_select(0, torch.from_numpy(i).to(H.dev())))
        H.assert_bits_equal(got, want, f"{kind} plan, tensor {t}")


@pytest.mark.parametrize("split", [False, True])
def test_tiny_mlp_zero_round_trip(split):
    """Both ranks of the 2-layer MLP on one GPU, each step: every rank packs its
    per-tensor gradients, each owner takes its chunk of every rank's buckets
    (shard_of), reduces and updates its shard, the bf16 shards are gathered
    and unpacked into per-tensor parameters (in two calls, and in one with
    unpack_shards) -- the reduce-scatter / update /
    all-gather round trip, all in the library's kernels, against the oracle."""
    import torch
    w = synth.WORKLOADS["tiny_mlp"]
    hp = _hp(w)
    cap = w.bucket_cap_bytes if not split else 256 << 10  # several split buckets
    pl = sbp.bucket_plan(w.numels, cap, w.world_n, split=split)
    opl = OP.bucket_plan(w.numels, cap, w.world_n, split=split)
    N, R, n = w.world_n, w.R, pl.shard_numel
    state = []
    ostate = []
    for s in range(N):
        th = synth.normal_f32(SEED, synth.master_stream(s), n, w.master_sigma)
        z = np.zeros(n, np.float32)
        state.append([H.from_np_f32(th), H.from_np_f32(z), H.from_np_f32(z), H.empty_u16(n)])
        ostate.append((th, z, z))
    grads = [[H.empty_u16(k) for k in w.numels] for _ in range(R)]
    flats = [H.empty_u16(pl.flat_numel) for _ in range(R)]
    recv = [[H.empty_u16(n) for _ in range(R)] for _ in range(N)]
    gathered = H.empty_u16(pl.flat_numel)
    params = [H.empty_u16(k) for k in w.numels]
    params1 = [H.empty_u16(k) for k in w.numels]  # the one-pass all-gather side
    for t in range(1, 4):
        host_flats = []
        for r in range(R):
            gh = []
            for tid, k in enumerate(w.numels):
                st = synth.tensor_stream(t, 0, r, tid)
                synth.dev_normal_bf16(grads[r][tid], SEED, st, w.grad_sigma)
                gh.append(synth.normal_bf16(SEED, st, k, w.grad_sigma))
            sbp.pack_grads(pl, grads[r], flats[r])
            host_flats.append(OS.pack(opl, gh))
        oshards = []
        for s in range(N):
            for r in range(R):
                sbp.shard_of(pl, s, flats[r], recv[s][r])
            sbp.adamw_shard(recv[s], None, sbp.mean_scale(R), *state[s][:3], state[s][3], hp, t)
            th, m, v, p = OS.shard_step([OS.chunk(opl, f, s) for f in host_flats], None,
                                        OS.mean_scale(R), *ostate[s], hp, t)
            ostate[s] = (th, m, v)
            oshards.append(p)
        sbp.gather_shards(pl, [state[s][3] for s in range(N)], gathered)
        sbp.unpack_params(pl, gathered, params)
        sbp.unpack_shards(pl, [state[s][3] for s in range(N)], params1)
        torch.cuda.synchronize()
        want = OS.unpack(opl, OS.gather(opl, oshards))
        for tid in range(len(w.numels)):
            H.assert_bits_equal(H.to_np_u16(params[tid]), want[tid], f"step {t} tensor {tid}")
            H.assert_bits_equal(H.to_np_u16(params1[tid]), want[tid],
                                f"step {t} tensor {tid}, unpack_shards")


def test_shard_union_resume_and_reshard():
    """The invariants that make sharding safe, on the GPU path, bit for bit:
    the union of the N = 4 shard updates equals the unsharded (N = 1) update,
    resuming from a host copy of the shard state equals running on, and
    resharding N = 4 -> 1 mid-run equals the unsharded run ("Distributed
    Training and Parallelism", "Reproduction and debugging": resumability and
    mesh reconfiguration).  A ragged model, so buckets carry padding; the
    unsharded run is also checked against the oracle."""
    import torch
    numels = [1000, 37, 4096, 130, 8, 513, 2]
    R, hp, sig = 3, sbp.AdamW(), 1e-2
    scale = sbp.mean_scale(R)
    theta = [synth.normal_f32(SEED, synth.master_stream(100 + t), k, 0.02)
             for t, k in enumerate(numels)]

    def layout(N):
        return (sbp.bucket_plan(numels, 2048, N), OP.bucket_plan(numels, 2048, N))

    def to_shards(opl, per_tensor):
        """Per-tensor fp32 arrays -> each rank's shard (host), padding +0."""
        flat = np.zeros(opl.flat_numel, np.float32)
        for t, x in enumerate(per_tensor):
            flat[opl.tensor_flat_offset(t):opl.tensor_flat_offset(t) + x.size] = x
        return [OS.chunk(opl, flat, s) for s in range(opl.world_n)]

    def to_tensors(opl, shards):
        return [x.copy() for x in OS.unpack(opl, OS.gather(opl, shards))]

    def upload(opl, tensors_th, tensors_m, tensors_v):
        cols = [to_shards(opl, x) for x in (tensors_th, tensors_m, tensors_v)]
        return [[H.from_np_f32(cols[i][s]) for i in range(3)] for s in range(opl.world_n)]

    def download(opl, state):
        return [to_tensors(opl, [H.to_np_f32(state[s][i]) for s in range(opl.world_n)])
                for i in range(3)]

    grads = [[H.empty_u16(k) for k in numels] for _ in range(R)]

    def step(pl, state, t):
        for r in range(R):
            for tid in range(len(numels)):
                synth.dev_normal_bf16(grads[r][tid], SEED, synth.tensor_stream(t, 0, r, tid), sig)
        flats = [H.empty_u16(pl.flat_numel) for _ in range(R)]
        for r in range(R):
            sbp.pack_grads(pl, grads[r], flats[r])
        for s in range(pl.world_n):
            recv = [H.empty_u16(pl.shard_numel) for _ in range(R)]
            for r in range(R):
                sbp.shard_of(pl, s, flats[r], recv[r])
            sbp.adamw_shard(recv, None, scale, *state[s], H.empty_u16(pl.shard_numel), hp, t)

    zeros = [np.zeros(k, np.float32) for k in numels]
    pl4, opl4 = layout(4)
    pl1, opl1 = layout(1)
    assert pl4.shard_numel * 4 > sum(numels)  # padding present
    # unsharded: 6 steps
    full = upload(opl1, theta, zeros, zeros)
    for t in range(1, 7):
        step(pl1, full, t)
    torch.cuda.synchronize()
    want = download(opl1, full)
    # N = 4: 3 steps, state to the host and back (checkpoint), 3 more steps
    sh = upload(opl4, theta, zeros, zeros)
    for t in range(1, 4):
        step(pl4, sh, t)
    torch.cuda.synchronize()
    ckpt = download(opl4, sh)
    del sh
    sh = upload(opl4, *ckpt)
    for t in range(4, 7):
        step(pl4, sh, t)
    torch.cuda.synchronize()
    got_resume = download(opl4, sh)
    # N = 4 for 3 steps, resharded to N = 1 for the last 3
    re = upload(opl1, *ckpt)
    for t in range(4, 7):
        step(pl1, re, t)
    torch.cuda.synchronize()
    got_reshard = download(opl1, re)
    for name, got in (("resume", got_resume), ("reshard", got_reshard)):
        for i, what in enumerate(("master", "m", "v")):
            for t in range(len(numels)):
                H.assert_bits_equal(got[i][t], want[i][t], f"{name} {what} tensor {t}")
    # the unsharded GPU run against the oracle
    th1 = to_shards(opl1, theta)[0]
    m1 = np.zeros(pl1.shard_numel, np.float32)
    v1 = m1.copy()
    for t in range(1, 7):
        gh = [[synth.normal_bf16(SEED, synth.tensor_stream(t, 0, r, tid), k, sig)
               for tid, k in enumerate(numels)] for r in range(R)]
        peers = [OS.chunk(opl1, OS.pack(opl1, g), 0) for g in gh]
        th1, m1, v1, _ = OS.shard_step(peers, None, OS.mean_scale(R), th1, m1, v1, hp, t)
    for i, x in enumerate((th1, m1, v1)):
        for t, y in enumerate(to_tensors(opl1, [x])):
            H.assert_bits_equal(want[i][t], y, f"unsharded vs oracle {i} tensor {t}")
