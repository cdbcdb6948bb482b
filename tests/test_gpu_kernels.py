"""GPU parity of each kernel against the oracle, element by element, on the
same seeded inputs (HIP path called through the C ABI).  Sizes span several
tiles and grid-stride passes with ragged tails; edge cases cover empty and
tiny inputs, every peer count, special values and out-of-bounds writes."""

import numpy as np
import pytest

import sharded_bucket_plan_amd as sbp
import synth
from oracle import plan as OP
from oracle import step as OS
from tests import helpers as H

pytestmark = pytest.mark.gpu

HP = sbp.AdamW()
SIZES = [1, 7, 8, 9, 2047, 256 * 8 * 3 + 5]
# 16.8M elements make one grid-stride pass of the largest grid; this spans 2+
BIG = 256 * 32 * 256 * 8 * 2 + 13
# sizes whose tile grids end in a partial round of the XCD deal: 301 and 522
# tiles of 2048 (one full round of 8 chunks of 32 tiles, or of 64, then a rest)
ROUNDS = [300 * 2048 + 5, 521 * 2048 + 3]


@pytest.fixture(autouse=True)
def _gpu():
    H.need_gpu()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_device_generator_matches_host():
    import torch
    for n, st, sigma in [(12345, synth.peer_stream(3, 1, 7), 1e-3),
                         (1 << 20, synth.tensor_stream(2, 0, 1, 9), 1e-2)]:
        d = H.empty_u16(n)
        synth.dev_normal_bf16(d, 42, st, sigma)
        H.assert_bits_equal(H.to_np_u16(d), synth.normal_bf16(42, st, n, sigma), "bf16 gen")
    f = torch.empty(99991, dtype=torch.float32, device=H.dev())
    synth.dev_normal_f32(f, 42, synth.master_stream(1), 0.02)
    H.assert_bits_equal(H.to_np_f32(f), synth.normal_f32(42, synth.master_stream(1), 99991, 0.02),
                        "f32 gen")


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("n", SIZES + ROUNDS)
def test_reduce_shard(R, n):
    import torch
    peers = H.dev_peers(11, 1, 0, R, n, 1e-3)
    scale = sbp.mean_scale(R)
    whole, out, g = H.guarded(n, 4)
    sbp.reduce_shard(peers, scale, out)
    torch.cuda.synchronize()
    want = OS.normalise(OS.reduce_peers(H.host_peers(11, 1, 0, R, n, 1e-3)), OS.mean_scale(R))
    H.assert_bits_equal(H.to_np_f32(out), want, f"reduce R={R} n={n}")
    assert H.canaries_intact(whole, g)


def test_reduce_shard_big_multi_pass():
    import torch
    R, n = 8, BIG
    peers = H.dev_peers(12, 1, 0, R, n, 1e-3)
    out = torch.empty(n, dtype=torch.float32, device=H.dev())
    sbp.reduce_shard(peers, 0.125, out)
    torch.cuda.synchronize()
    want = OS.normalise(OS.reduce_peers(H.host_peers(12, 1, 0, R, n, 1e-3)), np.float32(0.125))
    H.assert_bits_equal(H.to_np_f32(out), want, "reduce big")


@pytest.mark.parametrize("R", [1, 3, 8])
@pytest.mark.parametrize("n", [1, 9, 256 * 8 * 3 + 5, BIG] + ROUNDS)
def test_accumulate_grads(R, n):
    import torch
    K = 3
    whole, acc, g = H.guarded(n, 4)
    bufs = None
    A = None
    for k in range(K):
        bufs = H.dev_peers(13, 2, k, R, n, 1e-3, bufs)
        sbp.accumulate_grads(acc, bufs, first=(k == 0))
        A = OS.accumulate(A, OS.reduce_peers(H.host_peers(13, 2, k, R, n, 1e-3)))
    torch.cuda.synchronize()
    H.assert_bits_equal(H.to_np_f32(acc), A, f"accumulate R={R} n={n}")
    assert H.canaries_intact(whole, g)


def _state(seed, n):
    th = synth.normal_f32(seed, synth.master_stream(0), n, 0.02)
    return th, np.zeros(n, np.float32), np.zeros(n, np.float32)


# every peer count at the small sizes; the multi-pass size at R = 8
@pytest.mark.parametrize("R,n", [(R, n) for R in [1, 2, 4, 7, 8, 16] for n in SIZES] + [(8, BIG)]
                         + [(R, n) for R in [2, 8] for n in ROUNDS])
@pytest.mark.parametrize("with_acc", [False, True])
def test_adamw_shard(R, n, with_acc):
    import torch
    steps = 3
    th, m, v = _state(14, n)
    gs = [H.guarded_from(x) for x in (th, m, v)]
    dth, dm, dv = (x[1] for x in gs)
    pw, dp, g = H.guarded(n, 2)
    bufs = None
    acc_d = torch.empty(n, dtype=torch.float32, device=H.dev()) if with_acc else None
    scale = sbp.mean_scale(R, 2 if with_acc else 1)
    want = (th, m, v, None)
    for t in range(1, steps + 1):
        acc_h = None
        if with_acc:  # one earlier microbatch accumulated, the last one fused
            bufs = H.dev_peers(14, t, 0, R, n, 1e-3, bufs)
            sbp.accumulate_grads(acc_d, bufs, first=True)
            acc_h = OS.reduce_peers(H.host_peers(14, t, 0, R, n, 1e-3))
        bufs = H.dev_peers(14, t, 1, R, n, 1e-3, bufs)
        sbp.adamw_shard(bufs, acc_d, scale, dth, dm, dv, dp, HP, t)
        want = OS.shard_step(H.host_peers(14, t, 1, R, n, 1e-3), acc_h, np.float32(scale),
                             want[0], want[1], want[2], HP, t)
    torch.cuda.synchronize()
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    worst = H.assert_state_close(got, want, f"adamw R={R} n={n} acc={with_acc}")
    assert worst == 0, f"expected bit-exact, worst {worst} ulp"
    assert H.canaries_intact(pw, g)
    assert all(H.canaries_intact(w, gg) for w, _, gg in gs)


def test_adamw_shard_acc_only():
    """R = 0: the accumulator carries the whole gradient."""
    import torch
    n = 5003
    th, m, v = _state(15, n)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(m), H.from_np_f32(v)
    dp = H.empty_u16(n)
    acc = torch.empty(n, dtype=torch.float32, device=H.dev())
    sbp.accumulate_grads(acc, H.dev_peers(15, 1, 0, 4, n, 1e-3), first=True)
    sbp.adamw_shard([], acc, 0.25, dth, dm, dv, dp, HP, 1)
    torch.cuda.synchronize()
    A = OS.reduce_peers(H.host_peers(15, 1, 0, 4, n, 1e-3))
    want = OS.shard_step([], A, np.float32(0.25), th, m, v, HP, 1)
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    assert H.assert_state_close(got, want, "acc only") == 0


GROUPS = [(1e-3, 0.1), (5e-4, 0.0), (2e-3, 0.01)]


def _random_runs(n, rng):
    """A run table over n elements: runs of 1 element to several tiles, starts
    off the 8-element grid, and ids outside 0..len(GROUPS)-1 (which take
    group 0)."""
    starts, pos = [0], 0
    while True:
        pos += int(rng.choice([1, 3, 8, 17, 100, 2048, 5000, 40000]))
        if pos >= n:
            break
        starts.append(pos)
    groups = rng.integers(-1, len(GROUPS) + 6, len(starts)).astype(np.int32)
    return np.array(starts, np.int64), groups


def _elem_groups(starts, groups, n):
    g = np.empty(n, np.int64)
    ends = list(starts[1:]) + [n]
    for a, e, k in zip(starts, ends, groups):
        g[a:e] = k if 0 <= k < len(GROUPS) else 0
    return g


@pytest.mark.parametrize("R,n,with_acc",
                         [(R, n, R == 0) for R in [0, 1, 2, 8] for n in SIZES]
                         + [(R, n, True) for R in [3, 8] for n in SIZES]
                         + [(8, BIG, False), (8, BIG, True)]
                         + [(8, n, a) for n in ROUNDS for a in (False, True)])
def test_adamw_shard_grouped(R, n, with_acc):
    """Per-group lr and weight decay from a run table, every element: the
    peers alone, an accumulator of an earlier microbatch alone (R = 0), or
    both."""
    import torch
    rng = np.random.default_rng(n * 31 + R + (7 if with_acc else 0))
    starts, groups = _random_runs(n, rng)
    eg = _elem_groups(starts, groups, n)
    rs, rg = torch.from_numpy(starts).to(H.dev()), torch.from_numpy(groups).to(H.dev())
    th, m, v = _state(16, n)
    gs = [H.guarded_from(x) for x in (th, m, v)]
    dth, dm, dv = (x[1] for x in gs)
    pw, dp, g = H.guarded(n, 2)
    acc_d = torch.empty(n, dtype=torch.float32, device=H.dev()) if with_acc else None
    want = (th, m, v, None)
    bufs = None
    for t in (1, 2):
        acc_h = None
        if with_acc:
            sbp.accumulate_grads(acc_d, H.dev_peers(16, t, 0, 3, n, 1e-3), first=True)
            acc_h = OS.reduce_peers(H.host_peers(16, t, 0, 3, n, 1e-3))
        if R:
            bufs = H.dev_peers(16, t, 1, R, n, 1e-3, bufs)
        scale = sbp.mean_scale(max(R, 3))
        sbp.adamw_shard_grouped(bufs or [], acc_d, scale, dth, dm, dv, dp, HP, t, GROUPS, rs, rg)
        peers_h = H.host_peers(16, t, 1, R, n, 1e-3) if R else []
        want = OS.shard_step_grouped(peers_h, acc_h, np.float32(scale), want[0], want[1],
                                     want[2], HP, GROUPS, eg, t)
    torch.cuda.synchronize()
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    for a, b, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(a, b, f"grouped R={R} n={n} acc={with_acc} {name}")
    assert H.canaries_intact(pw, g)
    assert all(H.canaries_intact(w, gg) for w, _, gg in gs)


def test_adamw_shard_grouped_eight_groups():
    """All SBP_MAX_GROUPS groups in use, each with its own lr and decay;
    runs of every length from 1 element to several tiles."""
    import torch
    groups = [(1e-3 * (k + 1), 0.01 * k) for k in range(sbp.MAX_GROUPS)]
    n = 9 * 2048 + 5
    rng = np.random.default_rng(19)
    cuts = np.unique(rng.integers(1, n, 60))
    starts = np.r_[0, cuts].astype(np.int64)
    ids = (np.arange(starts.size) % sbp.MAX_GROUPS).astype(np.int32)
    eg = np.repeat(ids, np.diff(np.r_[starts, n])).astype(np.int64)
    th, m, v = _state(19, n)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(m), H.from_np_f32(v)
    dp = H.empty_u16(n)
    rs, rg = torch.from_numpy(starts).to(H.dev()), torch.from_numpy(ids).to(H.dev())
    peers = H.dev_peers(19, 1, 0, 4, n, 1e-3)
    sbp.adamw_shard_grouped(peers, None, 0.25, dth, dm, dv, dp, HP, 1, groups, rs, rg)
    torch.cuda.synchronize()
    want = OS.shard_step_grouped(H.host_peers(19, 1, 0, 4, n, 1e-3), None, np.float32(0.25),
                                 th, m, v, HP, groups, eg, 1)
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    for a, b, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(a, b, f"eight groups {name}")
    with pytest.raises(ValueError):
        sbp.adamw_shard_grouped(peers, None, 0.25, dth, dm, dv, dp, HP, 1, groups * 2, rs, rg)


def test_adamw_shard_grouped_one_group_is_plain():
    """One run of one group: the grouped step equals the plain step."""
    import torch
    n = 256 * 8 * 5 + 3
    th, m, v = _state(17, n)
    outs = []
    for grouped in (False, True):
        dth, dm, dv = H.from_np_f32(th), H.from_np_f32(m), H.from_np_f32(v)
        dp = H.empty_u16(n)
        peers = H.dev_peers(17, 1, 0, 4, n, 1e-3)
        if grouped:
            rs = torch.zeros(1, dtype=torch.int64, device=H.dev())
            rg = torch.zeros(1, dtype=torch.int32, device=H.dev())
            sbp.adamw_shard_grouped(peers, None, 0.25, dth, dm, dv, dp, HP, 1,
                                    [(HP.lr, HP.weight_decay)], rs, rg)
        else:
            sbp.adamw_shard(peers, None, 0.25, dth, dm, dv, dp, HP, 1)
        torch.cuda.synchronize()
        outs.append((H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp)))
    for a, b, name in zip(outs[0], outs[1], ("master", "m", "v", "param")):
        H.assert_bits_equal(b, a, f"one group {name}")


def test_empty_inputs_touch_nothing():
    import torch
    whole, out, g = H.guarded(0, 4)
    p = [H.empty_u16(8)]
    sbp.reduce_shard([x[:0] for x in p], 1.0, out)
    st = [torch.zeros(0, dtype=torch.float32, device=H.dev()) for _ in range(3)]
    sbp.adamw_shard([x[:0] for x in p], None, 1.0, *st, H.empty_u16(0), HP, 1)
    torch.cuda.synchronize()
    assert H.canaries_intact(whole, g)


def _special_bf16(n, rng):
    """bf16 patterns with zeros of both signs, subnormals, the largest finite
    values, infinities and NaNs mixed into ordinary values."""
    base = rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x7F7F,
                         0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x3F80, 0x3F81, 0x4B80],
                        dtype=np.uint16)
    pick = rng.random(n) < 0.3
    base[pick] = rng.choice(specials, pick.sum())
    return base


def test_special_values():
    import torch
    rng = np.random.default_rng(5)
    n, R = 4099, 3
    hp = [_special_bf16(n, rng) for _ in range(R)]
    th = (rng.normal(size=n) * 0.02).astype(np.float32)
    th[:50] = np.array([0.0, -0.0, 1e-40, -1e-40, 3e38] * 10, dtype=np.float32)
    m = (rng.normal(size=n) * 1e-3).astype(np.float32)
    v = np.abs(rng.normal(size=n) * 1e-6).astype(np.float32)
    v[::7] = 0.0
    v[1::11] = 1e-42  # subnormal second moment
    dpe = [H.from_np_u16(x) for x in hp]
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(m), H.from_np_f32(v)
    dp = H.empty_u16(n)
    out = torch.empty(n, dtype=torch.float32, device=H.dev())
    sbp.reduce_shard(dpe, 0.5, out)
    sbp.adamw_shard(dpe, None, 0.5, dth, dm, dv, dp, HP, 7)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        S = OS.normalise(OS.reduce_peers(hp), np.float32(0.5))
        want = OS.shard_step(hp, None, np.float32(0.5), th, m, v, HP, 7)
    d = H.ulp_f32(H.to_np_f32(out), S)
    assert d.max() == 0
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    assert H.assert_state_close(got, want, "special values") == 0
    # finite results are bit-identical; NaN results agree by class
    fin = np.isfinite(want[0])
    H.assert_bits_equal(got[0][fin], want[0][fin], "finite master")
    H.assert_bits_equal(got[3][fin], want[3][fin], "finite params")
    assert np.array_equal(np.isnan(got[0]), np.isnan(want[0]))
    assert np.array_equal(np.isnan(H.to_np_f32(out)), np.isnan(S))


HP_EDGES = [
    ("lr 0", sbp.AdamW(0.0, 0.9, 0.999, 1e-8, 0.01), (1, 2)),
    ("wd 0", sbp.AdamW(1e-3, 0.9, 0.999, 1e-8, 0.0), (1, 2)),
    ("betas 0", sbp.AdamW(1e-3, 0.0, 0.0, 1e-8, 0.01), (1, 2)),
    ("big lr and wd", sbp.AdamW(1.0, 0.9, 0.999, 1e-8, 2.0), (1, 2)),
    ("late steps", sbp.AdamW(), (1000, 1001)),
    ("very late steps", sbp.AdamW(), (10 ** 6, 10 ** 6 + 1)),
    ("eps 0, zero grads", sbp.AdamW(1e-3, 0.9, 0.999, 0.0, 0.01), (1, 2)),
]


@pytest.mark.parametrize("name,hp,steps", HP_EDGES, ids=[e[0] for e in HP_EDGES])
def test_adamw_hyperparameter_edges(name, hp, steps):
    """Edge hyperparameters (learning rate or decay 0, betas 0, decay factor
    below 0, bias corrections saturated at late steps, eps 0 over zero
    gradients, which makes 0/0) through two steps, against the oracle."""
    import torch
    n, R = 2 * 2048 + 13, 3
    th, m, v = _state(18, n)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(m), H.from_np_f32(v)
    dp = H.empty_u16(n)
    zero = name.startswith("eps 0")
    want = (th, m, v, None)
    for t in steps:
        if zero:
            ph = [np.zeros(n, np.uint16) for _ in range(R)]
            dpe = [H.from_np_u16(x) for x in ph]
        else:
            ph = H.host_peers(18, t, 0, R, n, 1e-3)
            dpe = H.dev_peers(18, t, 0, R, n, 1e-3)
        sbp.adamw_shard(dpe, None, sbp.mean_scale(R), dth, dm, dv, dp, hp, t)
        with np.errstate(all="ignore"):
            want = OS.shard_step(ph, None, OS.mean_scale(R), want[0], want[1], want[2], hp, t)
    torch.cuda.synchronize()
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    if zero:  # every update is 0/0: NaN on both sides (payload signs may differ)
        assert np.all(np.isnan(got[0])) and np.all(np.isnan(want[0]))
        assert H.assert_state_close(got, want, name) == 0
    else:
        for a, b, what in zip(got, want, ("master", "m", "v", "param")):
            H.assert_bits_equal(a, b, f"{name} {what}")


# ---- pack --------------------------------------------------------------------

def _pack_case(numels, cap, N, align=8, misalign=False, seed=3):
    import torch
    pl = sbp.bucket_plan(numels, cap, N, align)
    opl = OP.bucket_plan(numels, cap, N, align)
    grads_h = [synth.normal_bf16(seed, synth.tensor_stream(1, 0, 0, t), n, 1e-2)
               for t, n in enumerate(numels)]
    grads_d = []
    keep = []
    for gh in grads_h:
        if misalign and gh.size:
            base = torch.empty(gh.size + 3, dtype=torch.int16, device=H.dev())
            view = base[3:]  # 6 bytes past a 16-byte boundary
            view.copy_(H.from_np_u16(gh))
            keep.append(base)
            grads_d.append(view)
        else:
            grads_d.append(H.from_np_u16(gh) if gh.size else H.empty_u16(0))
    return pl, opl, grads_h, grads_d, keep


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("align", [8, 1])
def test_pack_ragged(misalign, align):
    import torch
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3, 20000, 8192 * 3 + 1]
    pl, opl, gh, gd, keep = _pack_case(numels, 600, 4, align, misalign)
    whole, flat, g = H.guarded(pl.flat_numel, 2)
    flat.fill_(0x7777)  # stale contents the pack must overwrite, padding included
    sbp.pack_grads(pl, gd, flat)
    torch.cuda.synchronize()
    H.assert_bits_equal(H.to_np_u16(flat), OS.pack(opl, gh), "pack all")
    assert H.canaries_intact(whole, g)


@pytest.mark.parametrize("length", [1, 7, 8, 9, 15, 17, 2040, 2047, 2049, 4103, 20003])
def test_copy_every_alignment(length):
    """Pack and unpack of one tensor at every pair of source and destination
    misalignments (0..7 elements past a 16-byte boundary each): the tensor is
    a view `o` elements into its buffer, and a k-element tensor ahead of it
    in the bucket (align 1) puts its flat offset at k.  Lengths straddle the
    unaligned head, the 8-element words, the tail and the 2048-element chunk.
    Bit-exact against the oracle's pack, guard bands intact."""
    import torch
    for k in range(8):
        numels = [length, k]  # visited in reverse: the k-element tensor first
        pl = sbp.bucket_plan(numels, 1 << 30, 1, align=1)
        opl = OP.bucket_plan(numels, 1 << 30, 1, align=1)
        assert pl.tensor(0) == (0, k)
        gh = [synth.normal_bf16(60 + k, synth.tensor_stream(1, 0, 0, t), n, 1e-2)
              for t, n in enumerate(numels)]
        want = OS.pack(opl, gh)
        for o in range(8):
            base = torch.full((length + o + 24,), 0x5A5A, dtype=torch.int16, device=H.dev())
            view = base[o:o + length]
            view.copy_(H.from_np_u16(gh[0]))
            other = H.from_np_u16(gh[1]) if k else H.empty_u16(0)
            whole, flat, g = H.guarded(pl.flat_numel, 2)
            flat.fill_(0x7777)
            sbp.pack_grads(pl, [view, other], flat)
            back_base = torch.full((length + o + 24,), 0x5A5A, dtype=torch.int16,
                                   device=H.dev())
            back = back_base[o + 1:o + 1 + length]  # another misalignment on the way back
            other_back = H.empty_u16(k)
            sbp.unpack_params(pl, flat, [back, other_back])
            torch.cuda.synchronize()
            what = f"length {length}, flat offset {k}, view offset {o}"
            H.assert_bits_equal(H.to_np_u16(flat), want, f"pack ({what})")
            assert H.canaries_intact(whole, g), what
            H.assert_bits_equal(H.to_np_u16(back), gh[0], f"unpack ({what})")
            b = H.to_np_u16(back_base)
            assert np.all(b[:o + 1] == 0x5A5A) and np.all(b[o + 1 + length:] == 0x5A5A), what


def test_pack_one_bucket_at_a_time():
    import torch
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3, 20000, 8192 * 3 + 1]
    pl, opl, gh, gd, keep = _pack_case(numels, 600, 4)
    flat = H.empty_u16(pl.flat_numel)
    flat.fill_(0x7777)
    want = OS.pack(opl, gh)
    for b in range(pl.num_buckets):
        sbp.pack_grads(pl, [gd[t] if t in pl.bucket_tensors(b) else None
                            for t in range(len(numels))], flat, bucket=b)
        torch.cuda.synchronize()
        got = H.to_np_u16(flat)
        info = pl.bucket(b)
        end = info["flat_offset"] + info["padded"]
        H.assert_bits_equal(got[:end], want[:end], f"bucket {b}")
        assert np.all(got[end:] == 0x7777)  # later buckets untouched


def test_pack_big_tensors_many_launches():
    """More segments than one launch carries (160), and chunks of multi-MB tensors."""
    import torch
    numels = [4096, 3 * 2 ** 20 + 8, 1000] * 60 + [5]
    pl, opl, gh, gd, keep = _pack_case(numels, 1 << 20, 8)
    flat = H.empty_u16(pl.flat_numel)
    sbp.pack_grads(pl, gd, flat)
    torch.cuda.synchronize()
    H.assert_bits_equal(H.to_np_u16(flat), OS.pack(opl, gh), "pack big")


@pytest.mark.parametrize("align", [8, 1])
def test_many_small_tensors(align):
    """5,000 small tensors (0-300 elements) at N = 8: thousands of copy
    segments, so many launches filled up to 160 small segments each; pack,
    then the shards straight into per-tensor buffers and back into the flat
    buckets, against the oracle."""
    import torch
    rng = np.random.default_rng(align)
    numels = [int(x) for x in rng.integers(0, 301, 5000)]
    N = 8
    pl = sbp.bucket_plan(numels, 64 << 10, N, align)
    opl = OP.bucket_plan(numels, 64 << 10, N, align)
    gh = [synth.normal_bf16(35, synth.tensor_stream(1, 0, 0, t), k, 1e-2)
          for t, k in enumerate(numels)]
    gd = [H.from_np_u16(h) if h.size else H.empty_u16(0) for h in gh]
    flat = H.empty_u16(pl.flat_numel)
    sbp.pack_grads(pl, gd, flat)
    want = OS.pack(opl, gh)
    shards = [H.empty_u16(pl.shard_numel) for _ in range(N)]
    for s in range(N):
        sbp.shard_of(pl, s, flat, shards[s])
    outs = [H.empty_u16(k) for k in numels]
    sbp.unpack_shards(pl, shards, outs)
    back = H.empty_u16(pl.flat_numel)
    back.fill_(0x1234)
    sbp.gather_shards(pl, shards, back)  # with align = 1, chunks that are not multiples of 8
    torch.cuda.synchronize()
    H.assert_bits_equal(H.to_np_u16(flat), want, "pack of 5,000 tensors")
    H.assert_bits_equal(H.to_np_u16(back), want, "gather_shards of 5,000 tensors")
    for t, h in enumerate(gh):
        if h.size:
            H.assert_bits_equal(H.to_np_u16(outs[t]), h, f"unpack_shards tensor {t}")


def test_layout_segment_longer_than_2_30():
    """A tensor of more than 2^30 elements: its copy segment is split into
    pieces for the kernel (whose segment length is 32-bit), and so are the
    fans of gather and unpack_shards.  Pack, unpack, shard_of, gather and
    unpack_shards are checked at sampled positions around every piece and
    rank-chunk boundary and at random, against the generator's values
    recomputed on the host."""
    import torch
    big = (1 << 30) + 12345
    numels = [7, big, 3]
    pl = sbp.bucket_plan(numels, 1 << 20, 2)
    opl = OP.bucket_plan(numels, 1 << 20, 2)
    dev = H.dev()
    st = [synth.tensor_stream(1, 0, 0, t) for t in range(3)]
    grads = [synth.dev_normal_bf16(torch.empty(k, dtype=torch.int16, device=dev), 42, st[t], 1e-2)
             for t, k in enumerate(numels)]
    flat = torch.full((pl.flat_numel,), 0x3333, dtype=torch.int16, device=dev)
    sbp.pack_grads(pl, grads, flat)
    rng = np.random.default_rng(43)
    b1 = opl.buckets[opl.tensor_bucket[1]]
    o1 = opl.tensor_flat_offset(1) - b1.flat_offset  # tensor 1's offset in its bucket
    # piece cuts of segments and fans, and where rank 1's chunk starts
    edges = [0, 1, (1 << 30) - 1, 1 << 30, (1 << 30) + 1, big - 2, big - 1,
             (1 << 30) - o1 - 1, (1 << 30) - o1, b1.chunk - o1 - 1, b1.chunk - o1]
    idx = np.unique(np.r_[edges, rng.integers(0, big, 1 << 14)]).astype(np.int64)
    want = synth.normal_bf16_at(42, st[1], idx, 1e-2)

    def at(t, i):
        return H.to_np_u16(t.index_select(0, torch.from_numpy(i).to(dev)))

    off = opl.tensor_flat_offset(1)
    H.assert_bits_equal(at(flat, off + idx), want, "pack of the big tensor")
    for t in (0, 2):  # the small tensors land whole
        o = opl.tensor_flat_offset(t)
        H.assert_bits_equal(at(flat, np.arange(o, o + numels[t])),
                            synth.normal_bf16(42, st[t], numels[t], 1e-2), f"pack tensor {t}")
    pad = np.array([b.flat_offset + b.used + j for b in opl.buckets
                    for j in range(min(16, b.padded - b.used))], dtype=np.int64)
    if pad.size:
        assert np.all(at(flat, pad) == 0), "padding not +0"
    out = torch.full((big,), 0x1111, dtype=torch.int16, device=dev)
    out2 = torch.full((3,), 0x1111, dtype=torch.int16, device=dev)  # shares the bucket
    sbp.unpack_params(pl, flat, [None, out, out2], bucket=opl.tensor_bucket[1])
    H.assert_bits_equal(at(out, idx), want, "unpack of the big tensor")
    H.assert_bits_equal(H.to_np_u16(out2), synth.normal_bf16(42, st[2], 3, 1e-2), "unpack tensor 2")
    shards = []
    for s in range(2):  # rank s's chunk of the big tensor's bucket
        shard = torch.empty(pl.shard_numel, dtype=torch.int16, device=dev)
        sbp.shard_of(pl, s, flat, shard)
        b = opl.buckets[opl.tensor_bucket[1]]
        j = np.unique(np.r_[0, b.chunk - 1, rng.integers(0, b.chunk, 4096)]).astype(np.int64)
        H.assert_bits_equal(at(shard, b.shard_offset + j), at(flat, b.flat_offset + s * b.chunk + j),
                            f"shard_of rank {s}")
        shards.append(shard)
    del out
    back = torch.full((pl.flat_numel,), 0x2222, dtype=torch.int16, device=dev)
    sbp.gather_shards(pl, shards, back, bucket=opl.tensor_bucket[1])
    H.assert_bits_equal(at(back, off + idx), want, "gather of the big tensor's bucket")
    H.assert_bits_equal(at(back, np.arange(b1.flat_offset, b1.flat_offset + b1.padded, 1 << 20)),
                        at(flat, np.arange(b1.flat_offset, b1.flat_offset + b1.padded, 1 << 20)),
                        "gather, every 2^20th position")
    del back
    out3 = torch.full((big,), 0x1111, dtype=torch.int16, device=dev)
    out4 = torch.full((3,), 0x1111, dtype=torch.int16, device=dev)  # shares the bucket
    sbp.unpack_shards(pl, shards, [None, out3, out4], bucket=opl.tensor_bucket[1])
    H.assert_bits_equal(at(out3, idx), want, "unpack_shards of the big tensor")
    H.assert_bits_equal(H.to_np_u16(out4), synth.normal_bf16(42, st[2], 3, 1e-2),
                        "unpack_shards tensor 2")
    torch.cuda.synchronize()


# ---- global gradient-norm clipping ---------------------------------------------

# R = 1 and R = 2 without an accumulator, and R = 0, take 4 / 2 / 2 groups per lane
@pytest.mark.parametrize("R,n", [(R, n) for R in [0, 1, 2, 3, 8]
                                  for n in [1, 9, 2047, 256 * 8 * 3 + 5, 256 * 8 * 9 + 3]]
                         + [(8, BIG), (1, BIG), (2, BIG), (0, BIG)]
                         + [(R, n) for R in [3, 8] for n in ROUNDS])
@pytest.mark.parametrize("write", [False, True])
def test_grad_sq_norm(R, n, write):
    import torch
    bufs = H.dev_peers(21, 1, 0, R, n, 1e-3) if R else []
    acc_d = None
    acc_h = None
    if R == 0 or R == 3:  # with an accumulator of an earlier microbatch
        acc_d = torch.empty(n, dtype=torch.float32, device=H.dev())
        sbp.accumulate_grads(acc_d, H.dev_peers(21, 1, 1, 2, n, 1e-3), first=True)
        acc_h = OS.reduce_peers(H.host_peers(21, 1, 1, 2, n, 1e-3))
    scale = sbp.mean_scale(max(R, 1), 2)
    whole, gsum, g = H.guarded(n, 4)
    ws_whole, ws, ws_g = H.guarded(sbp.grad_sq_norm_workspace(n), 8)
    sq_whole, sq_out, sq_g = H.guarded(1, 8)
    sq = sbp.grad_sq_norm(bufs, acc_d, scale, n, g_sum_out=gsum if write else None,
                          workspace=ws, sq_out=sq_out)
    sq2 = sbp.grad_sq_norm(bufs, acc_d, scale, n)
    torch.cuda.synchronize()
    assert H.canaries_intact(ws_whole, ws_g) and H.canaries_intact(sq_whole, sq_g)
    if R:
        S = OS.reduce_peers(H.host_peers(21, 1, 0, R, n, 1e-3))
        G = S if acc_h is None else acc_h + S
    else:
        G = acc_h
    want = OS.grad_sq_norm(G, np.float32(scale))
    got = float(sq.item())
    bound = H.sq_norm_bound(G, scale, n, H.norm_gpl(R, acc_h is not None))
    assert abs(got - want) <= bound, (got, want, bound)
    assert got == float(sq2.item())  # deterministic run to run
    if write:
        H.assert_bits_equal(H.to_np_f32(gsum), G, "g_sum_out")
        assert H.canaries_intact(whole, g)


def test_grad_sq_norm_empty():
    import torch
    sq = torch.full((1,), 7.0, dtype=torch.float64, device=H.dev())
    sbp.grad_sq_norm([H.empty_u16(0)], None, 1.0, 0, sq_out=sq)
    torch.cuda.synchronize()
    assert sq.item() == 0.0


@pytest.mark.parametrize("max_norm", [1e-3, 1e3])
def test_clipped_step_two_shards(max_norm):
    """Two ranks' shards: local squared norms (the all-reduce is their sum), a
    clip scale from the total, then the update from the stored G with R = 0.
    Compared with the oracle's clipping of the same gradients."""
    import torch
    R, n, hp = 4, 40000 + 3, HP
    scale = sbp.mean_scale(R)
    shards = []
    total = 0.0
    for s in range(2):
        peers = H.dev_peers(22 + s, 1, 0, R, n, 1e-2)
        G = torch.empty(n, dtype=torch.float32, device=H.dev())
        total += sbp.grad_sq_norm(peers, None, scale, n, g_sum_out=G).item()
        shards.append(G)
    cs, coef = sbp.clip_scale(total, max_norm, scale)
    Gh = [OS.reduce_peers(H.host_peers(22 + s, 1, 0, R, n, 1e-2)) for s in range(2)]
    want_total = sum(OS.grad_sq_norm(x, np.float32(scale)) for x in Gh)
    # each shard's fixed tree, plus the one host addition of the two totals
    bound = sum(H.sq_norm_bound(x, scale, n, H.norm_gpl(R, False)) for x in Gh)
    assert abs(total - want_total) <= bound + 2.0 ** -53 * want_total
    want_cs = OS.clipped_scale(scale, OS.clip_coef(want_total, max_norm))
    assert cs == float(want_cs)
    assert (coef < 1.0) == (max_norm < 1.0)
    for s in range(2):
        th, m, v = _state(30 + s, n)
        dth, dm, dv = H.from_np_f32(th), H.from_np_f32(m), H.from_np_f32(v)
        dp = H.empty_u16(n)
        sbp.adamw_shard([], shards[s], cs, dth, dm, dv, dp, hp, 1)
        torch.cuda.synchronize()
        want = OS.shard_step([], Gh[s], want_cs, th, m, v, hp, 1)
        got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
        assert H.assert_state_close(got, want, f"clipped shard {s}") == 0


@pytest.mark.parametrize("R", [2, 8])
@pytest.mark.parametrize("with_acc", [False, True])
def test_clipped_step_recompute_equals_stored_g(R, with_acc):
    """The two ways of clipping give the same bits: the norm pass writing G
    and the update reading it (R = 0), or the norm pass writing nothing and
    the update summing the peers (and accumulator) again.  Both against the
    oracle's clipped step."""
    import torch
    n, hp, max_norm = 256 * 8 * 5 + 3, HP, 1e-2
    scale = sbp.mean_scale(R, 2 if with_acc else 1)
    peers_h = H.host_peers(91, 1, 0, R, n, 1e-2)
    peers = [H.from_np_u16(x) for x in peers_h]
    acc_h = (np.asarray(OS.reduce_peers(H.host_peers(91, 1, 1, R, n, 1e-2)), np.float32)
             if with_acc else None)
    acc = H.from_np_f32(acc_h) if with_acc else None
    G = torch.empty(n, dtype=torch.float32, device=H.dev())
    sq_a = sbp.grad_sq_norm(peers, acc, scale, n, g_sum_out=G).item()
    sq_b = sbp.grad_sq_norm(peers, acc, scale, n).item()
    assert sq_a == sq_b
    cs, coef = sbp.clip_scale(sq_a, max_norm, scale)
    assert coef < 1.0
    th, m, v = _state(92, n)
    a = [H.from_np_f32(x) for x in (th, m, v)] + [H.empty_u16(n)]
    b = [H.from_np_f32(x) for x in (th, m, v)] + [H.empty_u16(n)]
    sbp.adamw_shard([], G, cs, *a, hp, 1)
    sbp.adamw_shard(peers, acc, cs, *b, hp, 1)
    torch.cuda.synchronize()
    for x, y, what in zip(a, b, ("master", "m", "v", "param")):
        assert torch.equal(x, y), f"recompute and stored G differ in {what}"
    S = OS.reduce_peers(peers_h)
    Gh = S if acc_h is None else OS.accumulate(acc_h, S)
    want_total = OS.grad_sq_norm(Gh, np.float32(scale))
    assert abs(sq_a - want_total) <= H.sq_norm_bound(Gh, scale, n, H.norm_gpl(R, with_acc))
    want_cs = OS.clipped_scale(scale, OS.clip_coef(want_total, max_norm))
    assert cs == float(want_cs)
    want = OS.shard_step(peers_h, acc_h, want_cs, th, m, v, hp, 1)
    got = (H.to_np_f32(b[0]), H.to_np_f32(b[1]), H.to_np_f32(b[2]), H.to_np_u16(b[3]))
    assert H.assert_state_close(got, want, f"recomputed clipped step R={R}") == 0


# ---- layout moves: pack / unpack / shard_of / gather on both plan kinds ---------

# N = 64 is the most ranks gather and unpack_shards take as fans; at N = 80
# they go out as plain segments
@pytest.mark.parametrize("kind,N", [("whole", 4), ("split", 4), ("per_tensor", 4),
                                    ("whole", 64), ("split", 64), ("per_tensor", 64),
                                    ("whole", 80), ("per_tensor", 80)])
@pytest.mark.parametrize("misalign", [False, True])
def test_layout_moves(kind, N, misalign):
    import torch
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3, 20000, 8192 * 3 + 1]
    if kind == "per_tensor":
        rows = [37, 8, 1, 13, 1, 16, 9, 25, 3, 400, 1]
        pl = sbp.bucket_plan_per_tensor(numels, N, rows)
        opl = OP.per_tensor_plan(numels, N, rows)
    else:
        pl = sbp.bucket_plan(numels, 600, N, split=kind == "split")
        opl = OP.bucket_plan(numels, 600, N, split=kind == "split")
    grads_h = [synth.normal_bf16(31, synth.tensor_stream(1, 0, 0, t), n, 1e-2)
               for t, n in enumerate(numels)]
    bases = []  # (base, view start, length): everything outside the view must stay 0x5A5A

    def dev_tensor(h):
        lead = 5 if misalign else 8
        base = torch.full((h.size + lead + 64,), 0x5A5A, dtype=torch.int16, device=H.dev())
        v = base[lead:lead + h.size]
        if h.size:
            v.copy_(H.from_np_u16(h))
        bases.append((base, lead, h.size))
        return v

    def guards_ok():
        for base, lead, k in bases:
            b = H.to_np_u16(base)
            if not (np.all(b[:lead] == 0x5A5A) and np.all(b[lead + k:] == 0x5A5A)):
                return False
        return True

    gd = [dev_tensor(h) for h in grads_h]
    flat = H.empty_u16(pl.flat_numel)
    flat.fill_(0x7777)
    sbp.pack_grads(pl, gd, flat)
    want_flat = OS.pack(opl, grads_h)
    torch.cuda.synchronize()
    H.assert_bits_equal(H.to_np_u16(flat), want_flat, "pack")
    # per-bucket pack of a second buffer
    flat2 = H.empty_u16(pl.flat_numel)
    flat2.fill_(0x7777)
    for b in range(pl.num_buckets):
        members = set(pl.bucket_tensors(b))
        sbp.pack_grads(pl, [gd[t] if t in members else None for t in range(len(numels))],
                       flat2, bucket=b)
    torch.cuda.synchronize()
    H.assert_bits_equal(H.to_np_u16(flat2), want_flat, "pack by bucket")
    # shard_of each rank, then gather back
    shard_g = [H.guarded(pl.shard_numel, 2) for _ in range(N)]
    shards = [x[1] for x in shard_g]
    for s in range(N):
        sbp.shard_of(pl, s, flat, shards[s])
    torch.cuda.synchronize()
    for s in range(N):
        H.assert_bits_equal(H.to_np_u16(shards[s]), OS.chunk(opl, want_flat, s), f"shard {s}")
    assert all(H.canaries_intact(w, gg) for w, _, gg in shard_g)
    back_whole, back, back_g = H.guarded(pl.flat_numel, 2)
    back.fill_(0x1234)
    sbp.gather_shards(pl, shards, back)
    torch.cuda.synchronize()
    H.assert_bits_equal(H.to_np_u16(back), want_flat, "gather")
    assert H.canaries_intact(back_whole, back_g)
    # unpack into per-tensor buffers (all at once, and bucket by bucket)
    outs = [dev_tensor(np.zeros(n, np.uint16)) for n in numels]
    sbp.unpack_params(pl, back, outs)
    outs2 = [dev_tensor(np.zeros(n, np.uint16)) for n in numels]
    for b in range(pl.num_buckets):
        members = set(pl.bucket_tensors(b))
        sbp.unpack_params(pl, back, [outs2[t] if t in members else None
                                     for t in range(len(numels))], bucket=b)
    torch.cuda.synchronize()
    for t, h in enumerate(grads_h):
        H.assert_bits_equal(H.to_np_u16(outs[t]), h, f"unpack tensor {t}")
        H.assert_bits_equal(H.to_np_u16(outs2[t]), h, f"unpack by bucket, tensor {t}")
    # shards -> per-tensor parameters in one pass (the oracle's gather, then its
    # unpack), from shards with nonzero padding slots, which must not be read
    rnd = [synth.normal_bf16(32, synth.peer_stream(1, 0, s), pl.shard_numel, 1.0)
           for s in range(N)]
    dsh = [x[1] for x in shard_g]  # 16-byte aligned, as the call requires
    for d, x in zip(dsh, rnd):
        d.copy_(H.from_np_u16(x))
    want_t = OS.unpack(opl, OS.gather(opl, rnd))
    outs3 = [dev_tensor(np.zeros(n, np.uint16)) for n in numels]
    sbp.unpack_shards(pl, dsh, outs3)
    outs4 = [dev_tensor(np.zeros(n, np.uint16)) for n in numels]
    for b in range(pl.num_buckets):
        members = set(pl.bucket_tensors(b))
        sbp.unpack_shards(pl, dsh, [outs4[t] if t in members else None
                                    for t in range(len(numels))], bucket=b)
    torch.cuda.synchronize()
    for t, h in enumerate(want_t):
        H.assert_bits_equal(H.to_np_u16(outs3[t]), h, f"unpack_shards tensor {t}")
        H.assert_bits_equal(H.to_np_u16(outs4[t]), h, f"unpack_shards by bucket, tensor {t}")
    assert guards_ok(), "a write outside a per-tensor buffer"


def test_graph_capture_replays():
    """The calls allocate nothing and pass their tables by value, so a step can
    be captured in a HIP graph.  The captured step uses every device entry
    point: pack, shard_of, accumulate, reduce, the squared norm, the fused
    step from G, the grouped fused step, gather, unpack and unpack_shards.  Each replay
    starts from the same saved state (restored by eager copies between
    replays) and must equal the eager run."""
    import torch
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3, 20000, 8192 * 3 + 1]
    pl = sbp.bucket_plan(numels, 600, 1)
    n = pl.shard_numel
    R = 2
    grads = [H.from_np_u16(synth.normal_bf16(41, synth.tensor_stream(1, 0, 0, t), k, 1e-2))
             if k else H.empty_u16(0) for t, k in enumerate(numels)]
    flat = H.empty_u16(n)
    shard = H.empty_u16(n)
    other = H.from_np_u16(synth.normal_bf16(41, synth.peer_stream(1, 0, 1), n, 1e-2))
    mb0 = [H.from_np_u16(synth.normal_bf16(41, synth.peer_stream(1, 1, r), n, 1e-2))
           for r in range(R)]
    th0 = synth.normal_f32(41, synth.master_stream(0), n, 0.02)
    init = [H.from_np_f32(th0), H.from_np_f32(np.zeros(n, np.float32)),
            H.from_np_f32(np.zeros(n, np.float32))]
    work = [x.clone() for x in init]
    work2 = [x.clone() for x in init]
    acc = torch.empty(n, dtype=torch.float32, device=H.dev())
    gsum = torch.empty(n, dtype=torch.float32, device=H.dev())
    red = torch.empty(n, dtype=torch.float32, device=H.dev())
    p = H.empty_u16(n)
    p2 = H.empty_u16(n)
    gathered = H.empty_u16(n)
    params = [H.empty_u16(k) for k in numels]
    params2 = [H.empty_u16(k) for k in numels]
    ws = torch.empty(sbp.grad_sq_norm_workspace(n), dtype=torch.float64, device=H.dev())
    sq = torch.empty(1, dtype=torch.float64, device=H.dev())
    scale = sbp.mean_scale(R, 2)
    groups = [(1e-3, 0.1), (5e-4, 0.0)]
    rs, rg = sbp.group_table(pl, 0, [t % 2 for t in range(len(numels))], H.dev())

    def step():
        sbp.pack_grads(pl, grads, flat)
        sbp.shard_of(pl, 0, flat, shard)
        sbp.accumulate_grads(acc, mb0, first=True)
        sbp.reduce_shard([shard, other], scale, red)
        sbp.grad_sq_norm([shard, other], acc, scale, n, g_sum_out=gsum, workspace=ws, sq_out=sq)
        sbp.adamw_shard([], gsum, scale, *work, p, HP, 1)
        sbp.adamw_shard_grouped([shard, other], acc, scale, *work2, p2, HP, 1, groups, rs, rg)
        sbp.gather_shards(pl, [p2], gathered)
        sbp.unpack_params(pl, gathered, params)
        sbp.unpack_shards(pl, [p], params2)

    outs = lambda: work + work2 + [p, p2, sq, red, gathered] + params + params2
    names = (["master", "m", "v", "grouped master", "grouped m", "grouped v", "param",
              "grouped param", "sq", "reduced", "gathered"] +
             [f"param tensor {t}" for t in range(len(numels))] +
             [f"unpack_shards tensor {t}" for t in range(len(numels))])
    step()
    torch.cuda.synchronize()
    eager = [x.clone() for x in outs()]

    def reset():
        for x, y in zip(work + work2, init + init):
            x.copy_(y)
        for x in (p, p2, gathered, *params, *params2):
            x.fill_(0)
        for x in (sq, red):
            x.fill_(-1.0)

    reset()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the side stream, as capture expects
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(outs(), eager, names):
            assert torch.equal(a, b), f"graph replay differs in {name}"


@pytest.mark.parametrize("with_acc", [False, True])
@pytest.mark.parametrize("mode", ["step", "arena_step"])
def test_c_client_fused_step(tmp_path, with_acc, mode):
    """A C99 program using only include/sbp.h and the HIP runtime's C API
    (its own buffers and stream, no torch) runs one fused step; its outputs
    equal the oracle's bit for bit.  "step": buffers from hipMalloc;
    "arena_step": every buffer from one spread arena, and the gradient's
    squared norm taken first with the allocation-free call."""
    import struct
    import subprocess
    exe = H.build_c_client(tmp_path)
    n, R, t = 256 * 8 * 3 + 37, 3, 3
    rng = np.random.default_rng(11)
    peers = H.host_peers(31, t, 1, R, n, 1e-3)
    acc = (rng.normal(size=n) * 1e-3).astype(np.float32) if with_acc else None
    th, _, _ = _state(31, n)
    m = (rng.normal(size=n) * 1e-3).astype(np.float32)
    v = np.abs(rng.normal(size=n) * 1e-6).astype(np.float32)
    scale = np.float32(sbp.mean_scale(R, 2 if with_acc else 1))
    hdr = struct.pack("<qiif5fq", n, R, int(with_acc), float(scale), HP.lr, HP.beta1, HP.beta2,
                      HP.eps, HP.weight_decay, t)
    body = b"".join(np.ascontiguousarray(p, np.uint16).tobytes() for p in peers)
    if with_acc:
        body += acc.tobytes()
    body += th.tobytes() + m.tobytes() + v.tobytes()
    (tmp_path / "in.bin").write_bytes(hdr + body)
    print(f"c client {mode} n={n} R={R} acc={with_acc}", flush=True)
    r = subprocess.run([exe, mode, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = (tmp_path / "out.bin").read_bytes()
    assert len(out) == 14 * n + (8 if mode == "arena_step" else 0)
    if mode == "arena_step":
        S = OS.reduce_peers(peers)
        G = S if acc is None else OS.accumulate(acc, S)
        sq = np.frombuffer(out, np.float64, 1, 14 * n)[0]
        want_sq = OS.grad_sq_norm(G, scale)
        gpl = H.norm_gpl(R, with_acc)
        assert abs(sq - want_sq) <= H.sq_norm_bound(G, scale, n, gpl), (sq, want_sq)
    got = (np.frombuffer(out, np.float32, n, 0), np.frombuffer(out, np.float32, n, 4 * n),
           np.frombuffer(out, np.float32, n, 8 * n), np.frombuffer(out, np.uint16, n, 12 * n))
    want = OS.shard_step(peers, acc, scale, th, m, v, HP, t)
    worst = H.assert_state_close(got, want, f"C client acc={with_acc}")
    assert worst == 0, f"expected bit-exact, worst {worst} ulp"


def test_bf16_emit_structured_sweep():
    """The fused kernel's bf16 emit over every upper half-word of an fp32
    pattern (all signs, exponents and high mantissas, NaN and inf included)
    times 23 lower half-words (the rounding boundaries 0x7FFF / 0x8000 /
    0x8001, the extremes and 16 random ones).  With lr = 0 and zero gradients
    the update leaves every master value unchanged (decay = 1, step = 0), so
    the emitted parameter is the cast of the input pattern; it equals the
    oracle's cast bit for bit, NaN by class."""
    import torch
    highs = np.arange(65536, dtype=np.uint32) << 16
    rng = np.random.default_rng(17)
    lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF], np.uint32),
                           rng.integers(0, 65536, 16, dtype=np.uint32)])
    th = (highs[:, None] | lows[None, :]).reshape(-1).view(np.float32)
    n = th.size
    hp = sbp.AdamW(0.0, 0.9, 0.999, 1e-8, 0.01)
    zero = np.zeros(n, np.uint16)
    dz = H.from_np_u16(zero)
    dth, dm, dv = H.from_np_f32(th), H.from_np_f32(np.zeros(n, np.float32)), \
        H.from_np_f32(np.zeros(n, np.float32))
    dp = H.empty_u16(n)
    sbp.adamw_shard([dz], None, 1.0, dth, dm, dv, dp, hp, 1)
    torch.cuda.synchronize()
    with np.errstate(all="ignore"):
        want = OS.shard_step([zero], None, np.float32(1.0), th, np.zeros(n, np.float32),
                             np.zeros(n, np.float32), hp, 1)
    got_th, got_p = H.to_np_f32(dth), H.to_np_u16(dp)
    nan = np.isnan(th)
    assert np.array_equal(np.isnan(want[0]), nan) and np.array_equal(np.isnan(got_th), nan)
    H.assert_bits_equal(got_th[~nan], th[~nan], "master passes through")
    H.assert_bits_equal(got_p[~nan], want[3][~nan], "bf16 emit")
    H.assert_bits_equal(want[3][~nan], OS.f32_to_bf16(th[~nan]), "oracle emit is the cast")
    pn = got_p[nan].astype(np.uint32) << 16
    assert np.all(np.isnan(pn.view(np.float32))), "NaN emits a NaN"


def test_two_threads_two_streams():
    """Two host threads, each on its own stream (default priority), step their
    own shards at the same time.  The kernel configuration is one no other
    test uses (R = 11 with an accumulator), so its first launches, which raise
    the kernel's LDS limit, also race.  Each thread's result equals the
    oracle's bit for bit."""
    import threading
    import torch
    n, R, steps = 256 * 8 * 37 + 5, 11, 4
    jobs = []
    for k in range(2):
        th, m, v = _state(60 + k, n)
        dev = [H.from_np_f32(x) for x in (th, m, v)] + [H.empty_u16(n)]
        acc_h = (np.random.default_rng(k).normal(size=n) * 1e-3).astype(np.float32)
        jobs.append(dict(seed=60 + k, host=(th, m, v), dev=dev, acc_h=acc_h,
                         acc=H.from_np_f32(acc_h), stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []
    barrier = threading.Barrier(2)

    def work(j):
        try:
            with torch.cuda.stream(j["stream"]):
                bufs = None
                barrier.wait()
                for t in range(1, steps + 1):
                    bufs = H.dev_peers(j["seed"], t, 0, R, n, 1e-3, bufs)
                    sbp.adamw_shard(bufs, j["acc"], 0.05, *j["dev"], HP, t)
                j["stream"].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    ts = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j in jobs:
        want = j["host"] + (None,)
        for t in range(1, steps + 1):
            want = OS.shard_step(H.host_peers(j["seed"], t, 0, R, n, 1e-3), j["acc_h"],
                                 np.float32(0.05), want[0], want[1], want[2], HP, t)
        got = tuple(H.to_np_f32(x) for x in j["dev"][:3]) + (H.to_np_u16(j["dev"][3]),)
        worst = H.assert_state_close(got, want, f"thread seed {j['seed']}")
        assert worst == 0, f"expected bit-exact, worst {worst} ulp"


def test_tensor_set_paths():
    """Per-tensor buffers marshalled once (TensorSet) give the same bytes as
    the list form in pack_grads, unpack_params and unpack_shards, whole and
    bucket by bucket, over repeated calls; a set built for another plan or
    with a wrongly sized tensor is refused."""
    import torch
    numels = [37, 8, 1, 130, 0, 64, 9, 250, 3, 20000, 8192 * 3 + 1]
    N = 4
    pl = sbp.bucket_plan(numels, 600, N)
    grads_h = [synth.normal_bf16(33, synth.tensor_stream(1, 0, 0, t), k, 1e-2)
               for t, k in enumerate(numels)]
    gd = [H.from_np_u16(h) if h.size else H.empty_u16(0) for h in grads_h]
    gs = sbp.TensorSet(pl, gd)
    want_flat = OS.pack(OP.bucket_plan(numels, 600, N), grads_h)
    for rep in range(2):
        flat = H.empty_u16(pl.flat_numel)
        flat.fill_(0x1111)
        if rep == 0:
            sbp.pack_grads(pl, gs, flat)
        else:
            for b in range(pl.num_buckets):
                sbp.pack_grads(pl, gs, flat, bucket=b)
        torch.cuda.synchronize()
        H.assert_bits_equal(H.to_np_u16(flat), want_flat, f"pack with a TensorSet, pass {rep}")
    outs = [H.empty_u16(k) for k in numels]
    os_ = sbp.TensorSet(pl, outs)
    sbp.unpack_params(pl, flat, os_)
    torch.cuda.synchronize()
    for t, h in enumerate(grads_h):
        H.assert_bits_equal(H.to_np_u16(outs[t]), h, f"unpack with a TensorSet, tensor {t}")
    shards = [H.empty_u16(pl.shard_numel) for _ in range(N)]
    for s in range(N):
        sbp.shard_of(pl, s, flat, shards[s])
    for x in outs:
        x.fill_(0)
    sbp.unpack_shards(pl, shards, os_)
    torch.cuda.synchronize()
    for t, h in enumerate(grads_h):
        H.assert_bits_equal(H.to_np_u16(outs[t]), h, f"unpack_shards with a TensorSet, tensor {t}")
    other = sbp.bucket_plan(numels, 600, N)
    with pytest.raises(ValueError):
        sbp.pack_grads(other, gs, flat)
    with pytest.raises(ValueError):
        sbp.TensorSet(pl, gd[:-1])
    with pytest.raises(ValueError):
        sbp.TensorSet(pl, gd[:-1] + [H.empty_u16(5)])


def test_step_counts_in_any_order():
    """The bias corrections depend only on the step passed, whatever steps
    earlier calls used (forwards, backwards, repeated, far ahead, another
    beta), each call checked against the oracle on fresh state.

    Steps of 2^40 and 2^62 are beyond what the oracle's t multiplications
    can reach; there both powers are far below 2^-54, where 1 - beta^t is
    exactly 1, so the oracle's result at t = 10^6 (checked to have both
    corrections exactly 1) is the result at those steps too."""
    import torch
    n, R = 256 * 8 * 2 + 7, 3
    th0, m0, v0 = _state(71, n)
    m0 = (np.random.default_rng(1).normal(size=n) * 1e-3).astype(np.float32)
    v0 = np.abs(np.random.default_rng(2).normal(size=n) * 1e-6).astype(np.float32)
    peers_h = H.host_peers(71, 1, 0, R, n, 1e-3)
    peers_d = [H.from_np_u16(x) for x in peers_h]
    other = sbp.AdamW(1e-3, 0.8, 0.99, 1e-8, 0.01)
    far = 10 ** 6
    for hp in (HP, other):
        sc_far = OS.adamw_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, far)
        sc_one = OS.adamw_scalars(hp.lr, 0.0, 0.0, hp.eps, hp.weight_decay, 1)  # corrections 1
        assert sc_far.step_size == sc_one.step_size and sc_far.c2 == sc_one.c2 == 1
    for t, hp in [(5, HP), (6, HP), (3, HP), (3, HP), (4, HP), (1000, HP), (7, HP),
                  (7, other), (8, other), (2, HP), (10 ** 6, HP), (10 ** 6 + 1, HP), (1, HP),
                  (1 << 40, HP), (1 << 62, other), ((1 << 62) + 1, other), (1 << 40, HP)]:
        dth, dm, dv = H.from_np_f32(th0), H.from_np_f32(m0), H.from_np_f32(v0)
        dp = H.empty_u16(n)
        sbp.adamw_shard(peers_d, None, 0.25, dth, dm, dv, dp, hp, t)
        torch.cuda.synchronize()
        want = OS.shard_step(peers_h, None, np.float32(0.25), th0, m0, v0, hp, min(t, far))
        got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
        worst = H.assert_state_close(got, want, f"step {t} betas {hp.beta1}/{hp.beta2}")
        assert worst == 0, f"step {t}: expected bit-exact, worst {worst} ulp"


def test_shard_step_object_matches_the_call():
    """ShardStep (buffers marshalled once) makes the same C call as
    adamw_shard: three steps each way, with and without an accumulator,
    bit-identical, and against the oracle."""
    import torch
    n, R = 256 * 8 * 3 + 5, 3
    peers_h = H.host_peers(81, 1, 0, R, n, 1e-3)
    acc_h = np.asarray(OS.reduce_peers(H.host_peers(81, 1, 1, 2, n, 1e-3)), np.float32)
    th0, m0, v0 = _state(82, n)
    for with_acc in (False, True):
        peers = [H.from_np_u16(x) for x in peers_h]
        acc = H.from_np_f32(acc_h) if with_acc else None
        a = [H.from_np_f32(x) for x in (th0, m0, v0)] + [H.empty_u16(n)]
        b = [H.from_np_f32(x) for x in (th0, m0, v0)] + [H.empty_u16(n)]
        step = sbp.ShardStep(peers, acc, *b)
        want = (th0, m0, v0, None)
        for t in (1, 2, 3):
            sbp.adamw_shard(peers, acc, 0.25, *a, HP, t)
            step(0.25, HP, t)
            want = OS.shard_step(peers_h, acc_h if with_acc else None, np.float32(0.25),
                                 want[0], want[1], want[2], HP, t)
        torch.cuda.synchronize()
        for x, y, what in zip(a, b, ("master", "m", "v", "param")):
            assert torch.equal(x, y), f"ShardStep {what} differs (acc={with_acc})"
        got = (H.to_np_f32(b[0]), H.to_np_f32(b[1]), H.to_np_f32(b[2]), H.to_np_u16(b[3]))
        assert H.assert_state_close(got, want, f"ShardStep acc={with_acc}") == 0
    # a stream given at construction is the one every call launches on
    side = torch.cuda.Stream()
    c = [H.from_np_f32(x) for x in (th0, m0, v0)] + [H.empty_u16(n)]
    torch.cuda.synchronize()
    on_side = sbp.ShardStep(peers, acc, *c, stream=side)
    assert on_side._stream.value == side.cuda_stream
    for t in (1, 2, 3):
        on_side(0.25, HP, t)
    side.synchronize()
    for x, y, what in zip(c, b, ("master", "m", "v", "param")):
        assert torch.equal(x, y), f"ShardStep on a side stream: {what} differs"
    with pytest.raises(ValueError, match="wrong size"):
        sbp.ShardStep(peers, None, a[0], a[1][:-1], a[2], a[3])
