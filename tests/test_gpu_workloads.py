"""GPU parity on the five synthetic workloads, in the launch configuration the
benchmark times.  Where the oracle finishes in seconds the comparison is over
every element; at full model scale it is over sampled elements, which the
oracle computes one by one (the step is elementwise once the plan is fixed,
and the inputs of any element can be regenerated on their own)."""

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


def test_gpt2_small_full():
    """GPT-2-small ZeRO-2 shard (N=8, R=8, 15.5M elements), two steps, every element."""
    import torch
    w = synth.WORKLOADS["gpt2_small"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 15554976
    th = synth.normal_f32(SEED, synth.master_stream(0), n, w.master_sigma)
    z = np.zeros(n, np.float32)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(z), H.from_np_f32(z)
    dp = H.empty_u16(n)
    bufs = None
    want = (th, z, z, None)
    for t in (1, 2):
        bufs = H.dev_peers(SEED, t, 0, w.R, n, w.grad_sigma, bufs)
        sbp.adamw_shard(bufs, None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t)
        want = OS.shard_step(H.host_peers(SEED, t, 0, w.R, n, w.grad_sigma), None,
                             OS.mean_scale(w.R), want[0], want[1], want[2], hp, t)
    torch.cuda.synchronize()
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    for a, b, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(a, b, f"gpt2_small {name}")


def test_gpt2_small_grouped_full():
    """GPT-2-small shard with the usual two parameter groups -- weight decay
    on matrices, none on biases, norm gains and other 1-D tensors -- plus a
    lower lr on the embeddings (a third group); run table from the plan,
    two steps, every element."""
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
    s = 3
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


def test_llama3_8b_shard_sampled():
    """Llama-3-8B ZeRO-3 shard (N=8, R=8, 1.0B elements): the benchmark's
    workload and launch, two steps, sampled elements."""
    import torch
    w = synth.WORKLOADS["llama3_8b"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 1003782656
    f32 = lambda: torch.empty(n, dtype=torch.float32, device=H.dev())
    dth, dm, dv = f32(), f32(), f32()
    synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
    dm.zero_()
    dv.zero_()
    dp = H.empty_u16(n)
    idx = _sample_index(pl, n, 1 << 18, 1)
    th = synth.normal_f32_at(SEED, synth.master_stream(0), idx, w.master_sigma)
    want = (th, np.zeros_like(th), np.zeros_like(th), None)
    bufs = None
    for t in (1, 2):
        bufs = H.dev_peers(SEED, t, 0, w.R, n, w.grad_sigma, bufs)
        sbp.adamw_shard(bufs, None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t)
        peers_h = [synth.normal_bf16_at(SEED, synth.peer_stream(t, 0, r), idx, w.grad_sigma)
                   for r in range(w.R)]
        want = OS.shard_step(peers_h, None, OS.mean_scale(w.R), want[0], want[1], want[2], hp, t)
    torch.cuda.synchronize()
    got = _sampled_state(dth, dm, dv, dp, idx)
    for a, b, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(a, b, f"llama3_8b {name}")


def test_gpt_7b5_accumulate_tokens_sampled():
    """'7.5B'-labelled GPT shard (N=64, R=8): 4 microbatches, the first three
    accumulated bucket by bucket, the last fused; 1/C valid-token scaling."""
    import torch
    w = synth.WORKLOADS["gpt_7b5"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 103890048
    f32 = lambda: torch.empty(n, dtype=torch.float32, device=H.dev())
    dth, dm, dv, acc = f32(), f32(), f32(), f32()
    synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
    dm.zero_()
    dv.zero_()
    dp = H.empty_u16(n)
    idx = _sample_index(pl, n, 1 << 18, 2)
    th = synth.normal_f32_at(SEED, synth.master_stream(0), idx, w.master_sigma)
    want = (th, np.zeros_like(th), np.zeros_like(th), None)
    bufs = None
    ranges = [(pl.bucket(b)["shard_offset"], pl.bucket(b)["chunk"]) for b in range(pl.num_buckets)]
    for t in (1, 2):
        counts = [synth.tokens(SEED, t, r) for r in range(w.R)]
        scale = sbp.tokens_scale(counts)
        A = None
        for k in range(w.K):
            bufs = H.dev_peers(SEED, t, k, w.R, n, w.grad_sigma, bufs)
            peers_h = [synth.normal_bf16_at(SEED, synth.peer_stream(t, k, r), idx, w.grad_sigma)
                       for r in range(w.R)]
            if k < w.K - 1:
                for o, c in ranges:
                    sbp.accumulate_grads(acc[o:o + c], [b[o:o + c] for b in bufs], first=(k == 0))
                A = OS.accumulate(A, OS.reduce_peers(peers_h))
            else:
                sbp.adamw_shard(bufs, acc, scale, dth, dm, dv, dp, hp, t)
                want = OS.shard_step(peers_h, A, OS.tokens_scale(counts), want[0], want[1],
                                     want[2], hp, t)
    torch.cuda.synchronize()
    got = _sampled_state(dth, dm, dv, dp, idx)
    for a, b, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(a, b, f"gpt_7b5 {name}")


def test_llama3_8b_dp_pack_and_step_sampled():
    """Llama-3-8B as a full DP replica (N=1, R=2, 8.03B elements): rank 0's 291
    per-tensor gradients packed into the 162 buckets, rank 1's bucket-layout
    gradient as the other contribution, one fused step; sampled elements."""
    import torch
    w = synth.WORKLOADS["llama3_8b_dp"]
    hp = _hp(w)
    pl = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    opl = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    n = pl.shard_numel
    assert n == 8030261248 == pl.flat_numel
    t = 1
    grads = []
    for tid, k in enumerate(w.numels):
        g = H.empty_u16(k)
        synth.dev_normal_bf16(g, SEED, synth.tensor_stream(t, 0, 0, tid), w.grad_sigma)
        grads.append(g)
    flat0 = H.empty_u16(n)
    sbp.pack_grads(pl, grads, flat0)
    del grads
    peer1 = H.empty_u16(n)
    synth.dev_normal_bf16(peer1, SEED, synth.peer_stream(t, 0, 1), w.grad_sigma)
    f32 = lambda: torch.empty(n, dtype=torch.float32, device=H.dev())
    dth, dm, dv = f32(), f32(), f32()
    synth.dev_normal_f32(dth, SEED, synth.master_stream(0), w.master_sigma)
    dm.zero_()
    dv.zero_()
    dp = H.empty_u16(n)
    sbp.adamw_shard([flat0, peer1], None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t)
    torch.cuda.synchronize()
    idx = _sample_index(pl, n, 1 << 18, 3)
    # oracle side: rank 0's packed value at each sampled flat index, element by element
    starts = np.array([opl.tensor_flat_offset(x) for x in range(len(w.numels))])
    order = np.argsort(starts)
    pos = np.searchsorted(starts[order], idx, side="right") - 1
    tids = order[pos]
    within = idx - starts[tids]
    assert np.all(within < np.array(w.numels)[tids])  # this plan has no padding
    p0 = np.empty(idx.size, np.uint16)
    for tid in np.unique(tids):
        sel = tids == tid
        p0[sel] = synth.normal_bf16_at(SEED, synth.tensor_stream(t, 0, 0, int(tid)), within[sel],
                                       w.grad_sigma)
    idx_d = torch.from_numpy(idx).to(H.dev())
    H.assert_bits_equal(H.to_np_u16(flat0.index_select(0, idx_d)), p0, "packed rank-0 grads")
    p1 = synth.normal_bf16_at(SEED, synth.peer_stream(t, 0, 1), idx, w.grad_sigma)
    th = synth.normal_f32_at(SEED, synth.master_stream(0), idx, w.master_sigma)
    z = np.zeros_like(th)
    want = OS.shard_step([p0, p1], None, OS.mean_scale(w.R), th, z, z, hp, t)
    got = _sampled_state(dth, dm, dv, dp, idx)
    for a, b, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(a, b, f"llama3_8b_dp {name}")


@pytest.mark.parametrize("split", [False, True])
def test_tiny_mlp_zero_round_trip(split):
    """Both ranks of the 2-layer MLP on one GPU, each step: every rank packs its
    per-tensor gradients, each owner takes its chunk of every rank's buckets
    (shard_of), reduces and updates its shard, the bf16 shards are gathered
    and unpacked into per-tensor parameters -- the reduce-scatter / update /
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
        torch.cuda.synchronize()
        want = OS.unpack(opl, OS.gather(opl, oshards))
        for tid in range(len(w.numels)):
            H.assert_bits_equal(H.to_np_u16(params[tid]), want[tid], f"step {t} tensor {tid}")
