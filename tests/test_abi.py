"""The C-ABI library on the host (CPU only): it loads, exports every function
include/sbp.h declares, its planner agrees with the oracle's independent
planner, and bad arguments come back as error codes before any device work
(no call here reaches the GPU)."""

import ctypes
import os
import random
import re

import pytest

import sharded_bucket_plan_amd as sbp
import synth
from oracle import plan as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "sbp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sbp_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert sorted(sbp.EXPORTS) == _declared()
    src = open(os.path.join(ROOT, "include", "sbp.h")).read()
    defs = dict(re.findall(r"#define (SBP_[A-Z_]+) \(?(-?\d+)(?:LL|u)?\)?", src))
    assert int(defs["SBP_MAX_SHARD_NUMEL"]) == sbp.MAX_SHARD_NUMEL
    assert int(defs["SBP_MAX_PEERS"]) == sbp.SBP_MAX_PEERS
    assert int(defs["SBP_MAX_GROUPS"]) == sbp.MAX_GROUPS
    for name in ("SBP_OK", "SBP_EINVAL", "SBP_EALIGN", "SBP_ERANGE", "SBP_EHIP", "SBP_ENOMEM"):
        assert int(defs[name]) == getattr(sbp, name), name
    assert int(defs["SBP_NOALLOC_SCRATCH_DOUBLES"]) == sbp.NOALLOC_SCRATCH_DOUBLES
    assert int(defs["SBP_NOALLOC_MAX_NUMEL"]) == sbp.NOALLOC_MAX_NUMEL
    assert int(defs["SBP_ARENA_MAX_ARRAYS"]) == sbp.ARENA_MAX_ARRAYS


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(sbp.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name
    assert sbp.version().startswith("sbp ")


def _same_plan(numels, cap, N, align=8, order="reverse"):
    p = sbp.bucket_plan(numels, cap, N, align, order)
    o = OP.bucket_plan(numels, cap, N, align, order)
    assert p.num_buckets == len(o.buckets)
    assert p.shard_numel == o.shard_numel and p.flat_numel == o.flat_numel
    for b, ob in enumerate(o.buckets):
        assert p.bucket(b) == dict(used=ob.used, padded=ob.padded, chunk=ob.chunk,
                                   shard_offset=ob.shard_offset, flat_offset=ob.flat_offset)
        assert p.bucket_tensors(b) == ob.tensors
    for t in range(len(numels)):
        assert p.tensor(t) == (o.tensor_bucket[t], o.tensor_offset[t])
    for stage in range(4):
        assert p.state_bytes(stage) == OP.state_bytes(o.flat_numel, o.shard_numel, stage)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_plan_matches_oracle_on_workloads(name):
    w = synth.WORKLOADS[name]
    _same_plan(w.numels, w.bucket_cap_bytes, w.world_n)


def test_plan_matches_oracle_on_cap_sweep():
    w = synth.WORKLOADS["gpt_7b5"]
    for mib in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        _same_plan(w.numels, mib << 20, w.world_n)


def test_plan_matches_oracle_random():
    rng = random.Random(99)
    for _ in range(400):
        T = rng.randint(0, 12)
        numels = [rng.choice([0, 1, 3, 7, 8, 9, 17, 64, 100, 1000]) for _ in range(T)]
        _same_plan(numels, rng.randint(1, 3000), rng.choice([1, 2, 3, 4, 8, 64]),
                   rng.choice([1, 2, 4, 8, 16]), rng.choice(["reverse", "forward"]))


def test_plan_rejects_bad_arguments():
    bad = [([8], 0, 1, 8), ([8], 64, 0, 8), ([8], 64, 1, 3), ([8], 64, 1, 8192), ([-1], 64, 1, 8)]
    for numels, cap, N, align in bad:
        with pytest.raises(sbp.SbpError) as e:
            sbp.bucket_plan(numels, cap, N, align)
        assert e.value.status == sbp.SBP_EINVAL
    with pytest.raises(sbp.SbpError):
        sbp.bucket_plan([8], 64, 1, 8, order="sideways")
    with pytest.raises(sbp.SbpError) as e:
        sbp.bucket_plan([2 ** 62, 2 ** 62], 64, 1)
    assert e.value.status == sbp.SBP_ERANGE
    p = sbp.bucket_plan([8, 8], 64, 1)
    with pytest.raises(sbp.SbpError):
        p.tensor(2)
    with pytest.raises(sbp.SbpError):
        p.bucket(-1)
    with pytest.raises(sbp.SbpError):
        p.state_bytes(4)


def test_scales_match_oracle():
    from oracle import step as OS
    for R in (1, 2, 3, 7, 8, 64):
        for K in (1, 3, 4):
            assert sbp.mean_scale(R, K) == float(OS.mean_scale(R, K))
    for t in range(1, 30):
        counts = [synth.tokens(17, t, r) for r in range(8)]
        assert sbp.tokens_scale(counts) == float(OS.tokens_scale(counts))
    for bad in ([0], [], [-1, 5]):
        with pytest.raises(sbp.SbpError):
            sbp.tokens_scale(bad)
    with pytest.raises(sbp.SbpError):
        sbp.mean_scale(0, 1)


def _raw(L, name, *args):
    return getattr(L, name)(*args)


def test_device_calls_validate_before_launch():
    """Null, misaligned, overlapping and out-of-range arguments are rejected on
    the host; the fake addresses below are never dereferenced."""
    L = sbp.lib()
    V = ctypes.c_void_p
    peers = (V * 2)(0x100000, 0x200000)
    hp = sbp.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    adam = L.sbp_adamw_shard
    ok_args = dict(peers=peers, R=2, acc=None, scale=0.5, master=V(0x300000), m=V(0x400000),
                   v=V(0x500000), p=V(0x600000), n=1024, hp=ctypes.byref(hp))

    def call(**kw):
        a = dict(ok_args, **kw)
        return adam(a["peers"], a["R"], a["acc"], a["scale"], a["master"], a["m"], a["v"],
                    a["p"], a["n"], a["hp"], None)

    assert call(R=17) == sbp.SBP_EINVAL
    assert call(R=-1) == sbp.SBP_EINVAL
    assert call(R=0) == sbp.SBP_EINVAL  # R == 0 needs acc
    assert call(R=0, n=0) == sbp.SBP_OK
    assert call(peers=(V * 2)(0x100000, None)) == sbp.SBP_EINVAL
    assert call(peers=(V * 2)(0x100008, 0x200000)) == sbp.SBP_EALIGN
    assert call(master=V(0x300004)) == sbp.SBP_EALIGN
    assert call(p=V(0x600002)) == sbp.SBP_EALIGN
    assert call(master=None) == sbp.SBP_EINVAL
    assert call(n=-1) == sbp.SBP_EINVAL
    bad_hp = sbp.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0)
    assert call(hp=ctypes.byref(bad_hp)) == sbp.SBP_EINVAL
    assert call(hp=None) == sbp.SBP_EINVAL
    # hyperparameter ranges: betas in [0, 1), lr, eps and weight decay finite and >= 0
    inf, nan = float("inf"), float("nan")
    for fields in [(1e-3, 1.0, 0.999, 1e-8, 0.01), (1e-3, 0.9, 1.0, 1e-8, 0.01),
                   (1e-3, -0.1, 0.999, 1e-8, 0.01), (1e-3, nan, 0.999, 1e-8, 0.01),
                   (1e-3, 0.9, 0.999, -1e-8, 0.01), (1e-3, 0.9, 0.999, inf, 0.01),
                   (-1e-3, 0.9, 0.999, 1e-8, 0.01), (inf, 0.9, 0.999, 1e-8, 0.01),
                   (1e-3, 0.9, 0.999, 1e-8, -0.01), (1e-3, 0.9, 0.999, 1e-8, nan)]:
        h = sbp.AdamWHParams(*fields, 1)
        assert call(hp=ctypes.byref(h)) == sbp.SBP_EINVAL, fields
        assert call(hp=ctypes.byref(h), n=0) == sbp.SBP_EINVAL, fields
    edge = sbp.AdamWHParams(0.0, 0.0, 0.0, 0.0, 0.0, 1)  # the low ends are allowed
    assert call(hp=ctypes.byref(edge), n=0) == sbp.SBP_OK
    assert call(m=V(0x300000 + 1024)) == sbp.SBP_EINVAL  # overlaps master
    assert call(p=V(0x100000 + 512)) == sbp.SBP_EINVAL  # overlaps a peer
    assert call(n=0) == sbp.SBP_OK  # nothing to do, nothing launched
    assert call(n=0, master=None, peers=None) == sbp.SBP_OK
    assert call(p=V(0x100000 + 512)) == sbp.SBP_EINVAL
    assert "overlap" in sbp.lib().sbp_last_error().decode()

    red = L.sbp_reduce_shard
    assert red(peers, 0, 16, 1.0, V(0x300000), None) == sbp.SBP_EINVAL
    assert red(peers, 2, 16, 1.0, V(0x300004), None) == sbp.SBP_EALIGN
    assert red(peers, 2, 16, 1.0, V(0x100000), None) == sbp.SBP_EINVAL  # out overlaps peer 0
    assert red(peers, 2, 0, 1.0, V(0x300000), None) == sbp.SBP_OK
    acc = L.sbp_accumulate_grads
    assert acc(None, peers, 2, 16, 1, None) == sbp.SBP_EINVAL
    assert acc(V(0x300008), peers, 2, 16, 1, None) == sbp.SBP_EALIGN
    assert acc(V(0x300000), peers, 2, 0, 0, None) == sbp.SBP_OK
    # one launch covers at most 2^24 - 1 tiles of 2048 elements
    big = sbp.MAX_SHARD_NUMEL
    assert big == (2 ** 24 - 1) * 2048
    assert call(n=big + 1) == sbp.SBP_ERANGE
    assert call(n=big) == sbp.SBP_EINVAL  # in range; the fake buffers then overlap
    assert red(peers, 2, big + 1, 1.0, V(0x300000), None) == sbp.SBP_ERANGE
    assert acc(V(0x300000), peers, 2, big + 1, 1, None) == sbp.SBP_ERANGE

    plan = sbp.bucket_plan([10, 20], 1 << 20, 1)
    grads = (V * 2)(0x100000, 0x200000)
    pack = L.sbp_pack_grads
    assert pack(None, -1, grads, V(0x300000), None) == sbp.SBP_EINVAL
    assert pack(plan.handle, 5, grads, V(0x300000), None) == sbp.SBP_EINVAL
    assert pack(plan.handle, -1, grads, V(0x300008), None) == sbp.SBP_EALIGN
    assert pack(plan.handle, -1, (V * 2)(0x100001, 0x200000), V(0x300000), None) == sbp.SBP_EALIGN
    assert pack(plan.handle, -1, (V * 2)(None, 0x200000), V(0x300000), None) == sbp.SBP_EINVAL
    assert pack(plan.handle, -1, grads, V(0x100000 + 16), None) == sbp.SBP_EINVAL  # overlap


def test_binding_refuses_steps_beyond_int64():
    """ctypes would wrap a step of 2^64 + 5 to 5 without a word; the binding
    refuses what does not fit the C struct's int64, and the library refuses
    steps below 1."""
    hp = sbp.AdamW()
    assert sbp.AdamWHParams.of(hp, (1 << 63) - 1, "t").step == (1 << 63) - 1
    for step in (1 << 63, (1 << 64) + 5, -(1 << 63) - 1):
        with pytest.raises(ValueError, match="does not fit int64"):
            sbp.AdamWHParams.of(hp, step, "t")
    V = ctypes.c_void_p
    peers = (V * 1)(0x100000)
    for step in (0, -1, -(1 << 63)):
        h = sbp.AdamWHParams.of(hp, step, "t")
        assert sbp.lib().sbp_adamw_shard(peers, 1, None, 1.0, V(0x300000), V(0x400000),
                                         V(0x500000), V(0x600000), 16, ctypes.byref(h),
                                         None) == sbp.SBP_EINVAL


def test_grad_sq_norm_needs_an_input():
    with pytest.raises(ValueError, match="needs peers or an accumulator"):
        sbp.grad_sq_norm([], None, 1.0, 0)


def test_clip_scale_matches_oracle():
    import math
    from oracle import step as OS
    import numpy as np
    rng = np.random.default_rng(4)
    for _ in range(2000):
        sq = float(rng.choice([0.0, 1e-30, 1e-6, 1.0, 123.4, 1e12])) * float(rng.random())
        mx = float(np.float32(rng.choice([1e-3, 0.5, 1.0, 5.0])))
        sc = float(OS.mean_scale(int(rng.integers(1, 9))))
        got, coef = sbp.clip_scale(sq, mx, sc)
        want_coef = OS.clip_coef(sq, mx)
        assert coef == want_coef
        assert got == float(OS.clipped_scale(sc, want_coef))
    got, coef = sbp.clip_scale(float("nan"), 1.0, 0.5)
    assert math.isnan(coef) and math.isnan(got)
    assert sbp.clip_scale(float("inf"), 1.0, 0.5) == (0.0, 0.0)
    assert sbp.clip_scale(4.0, 0.0, 0.5) == (0.0, 0.0)  # max_norm 0 zeroes the update
    for bad in ((1.0, -1.0), (1.0, float("nan")), (-1.0, 1.0)):
        with pytest.raises(sbp.SbpError):
            sbp.clip_scale(bad[0], bad[1], 0.5)


def test_grad_sq_norm_validates_before_launch():
    L = sbp.lib()
    V = ctypes.c_void_p
    peers = (V * 2)(0x100000, 0x200000)
    n = 10000
    need = sbp.grad_sq_norm_workspace(n)
    assert need == (n // 8 + 255) // 256 and sbp.grad_sq_norm_workspace(0) == 1
    tiles = (10 ** 10 // 8 + 255) // 256  # 4882813 tile partials, then 2385, then 2
    assert sbp.grad_sq_norm_workspace(10 ** 10) == tiles + 2385 + 2
    f = L.sbp_grad_sq_norm
    ws, sq = V(0x800000), V(0x900000)
    assert f(peers, 2, None, 1.0, n, None, None, need, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, n, None, ws, need - 1, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, n, None, ws, need, V(0x900004), None) == sbp.SBP_EALIGN
    assert f(peers, 0, None, 1.0, n, None, ws, need, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 17, None, 1.0, n, None, ws, need, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, n, V(0x300008), ws, need, sq, None) == sbp.SBP_EALIGN
    assert f(peers, 2, None, 1.0, n, V(0x100000), ws, need, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, n, None, ws, need, V(0x800000), None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, -1, None, ws, need, sq, None) == sbp.SBP_EINVAL
    big = sbp.MAX_SHARD_NUMEL + 1
    assert f(peers, 2, None, 1.0, big, None, ws, sbp.grad_sq_norm_workspace(big), sq,
             None) == sbp.SBP_ERANGE


def test_grad_sq_norm_noalloc_limit_and_validation():
    """The static scratch holds exactly the workspace of NOALLOC_MAX_NUMEL
    elements; bad arguments and a larger n are refused on the host, before the
    scratch's device address is looked up (no call here reaches a device)."""
    cap, top = sbp.NOALLOC_SCRATCH_DOUBLES, sbp.NOALLOC_MAX_NUMEL
    assert sbp.grad_sq_norm_workspace(top) == cap
    assert sbp.grad_sq_norm_workspace(top + 1) == cap + 1
    assert top >= 1003782656  # the Llama-3-8B 1/8 shard fits
    L = sbp.lib()
    V = ctypes.c_void_p
    f = L.sbp_grad_sq_norm_noalloc
    peers = (V * 2)(0x100000, 0x200000)
    sq = V(0x900000)
    n = 10000
    assert f(peers, 2, None, 1.0, n, None, None, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, n, None, V(0x900004), None) == sbp.SBP_EALIGN
    assert f(peers, 0, None, 1.0, n, None, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 17, None, 1.0, n, None, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, -1, None, sq, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, n, V(0x300008), sq, None) == sbp.SBP_EALIGN
    assert f(peers, 2, None, 1.0, n, V(0x100000), sq, None) == sbp.SBP_EINVAL
    assert f(peers, 2, None, 1.0, top + 1, None, V(1 << 40), None) == sbp.SBP_ERANGE
    assert "SBP_NOALLOC_MAX_NUMEL" in sbp.lib().sbp_last_error().decode()
    big = sbp.MAX_SHARD_NUMEL + 1
    assert f(peers, 2, None, 1.0, big, None, sq, None) == sbp.SBP_ERANGE


def test_arena_validates_before_touching_a_device():
    """Bad arena arguments come back as error codes before any HIP call (no
    device here: a valid request then fails at the device lookup)."""
    L = sbp.lib()
    V = ctypes.c_void_p
    I = ctypes.c_int64
    p, h = (V * 2)(), V()
    two = (I * 2)(100, 200)
    assert L.sbp_arena_create(None, 2, 0, 0, 1, p, ctypes.byref(h)) == sbp.SBP_EINVAL
    assert L.sbp_arena_create(two, 2, 0, 0, 1, None, ctypes.byref(h)) == sbp.SBP_EINVAL
    assert L.sbp_arena_create(two, 2, 0, 0, 1, p, None) == sbp.SBP_EINVAL
    assert L.sbp_arena_create(two, 0, 0, 0, 1, p, ctypes.byref(h)) == sbp.SBP_EINVAL
    assert L.sbp_arena_create(two, 65, 0, 0, 1, p, ctypes.byref(h)) == sbp.SBP_EINVAL
    for chunk in (-(2 << 20), 3 << 20, 1 << 20, 4096):
        assert L.sbp_arena_create(two, 2, chunk, 0, 1, p, ctypes.byref(h)) == sbp.SBP_EINVAL
    assert L.sbp_arena_create(two, 2, 0, -1, 1, p, ctypes.byref(h)) == sbp.SBP_EINVAL
    assert L.sbp_arena_create((I * 2)(-1, 5), 2, 0, 0, 1, p, ctypes.byref(h)) == sbp.SBP_EINVAL
    # 16384 chunks at most: 32 GiB of 2 MiB chunks fit, one byte more does not
    assert L.sbp_arena_create((I * 1)((32 << 30) + 1), 1, 2 << 20, 0, 1, p,
                              ctypes.byref(h)) == sbp.SBP_ERANGE
    assert L.sbp_arena_create((I * 2)(1 << 62, 1 << 62), 2, 0, 0, 1, p,
                              ctypes.byref(h)) == sbp.SBP_ERANGE
    assert L.sbp_arena_free(None) == sbp.SBP_OK
    assert L.sbp_arena_info(None, None, None, None) == sbp.SBP_EINVAL


def _same_split_plan(numels, cap, N, align=8, order="reverse"):
    p = sbp.bucket_plan(numels, cap, N, align, order, split=True)
    o = OP.bucket_plan(numels, cap, N, align, order, split=True)
    assert p.num_buckets == len(o.buckets)
    assert p.shard_numel == o.shard_numel and p.flat_numel == o.flat_numel
    for b, ob in enumerate(o.buckets):
        assert p.bucket(b) == dict(used=ob.used, padded=ob.padded, chunk=ob.chunk,
                                   shard_offset=ob.shard_offset, flat_offset=ob.flat_offset)
        assert p.bucket_tensors(b) == ob.tensors
    for t in range(len(numels)):
        assert p.tensor(t) == (o.tensor_bucket[t], o.tensor_offset[t])


def test_split_plan_matches_oracle():
    rng = random.Random(5)
    for _ in range(400):
        T = rng.randint(0, 10)
        numels = [rng.choice([0, 1, 3, 7, 8, 9, 17, 64, 100, 1000]) for _ in range(T)]
        _same_split_plan(numels, rng.randint(1, 3000), rng.choice([1, 2, 3, 4, 8]),
                         rng.choice([1, 2, 4, 8, 16]), rng.choice(["reverse", "forward"]))
    w = synth.WORKLOADS["gpt_7b5"]
    for mib in (1, 25, 256):
        _same_split_plan(w.numels, mib << 20, w.world_n)
    for name in ("tiny_mlp", "gpt2_small"):
        w = synth.WORKLOADS[name]
        _same_split_plan(w.numels, w.bucket_cap_bytes, w.world_n)


def test_layout_calls_validate_before_launch():
    L = sbp.lib()
    V = ctypes.c_void_p
    plan = sbp.bucket_plan([10, 20], 1 << 20, 2)
    two = (V * 2)(0x100000, 0x200000)
    assert L.sbp_unpack_params(None, -1, V(0x300000), two, None) == sbp.SBP_EINVAL
    assert L.sbp_unpack_params(plan.handle, -1, V(0x300008), two, None) == sbp.SBP_EALIGN
    assert L.sbp_unpack_params(plan.handle, 3, V(0x300000), two, None) == sbp.SBP_EINVAL
    assert L.sbp_unpack_params(plan.handle, -1, V(0x300000), (V * 2)(0x100001, 0x200000),
                               None) == sbp.SBP_EALIGN
    assert L.sbp_unpack_params(plan.handle, -1, V(0x300000), (V * 2)(0x100000, 0x100010),
                               None) == sbp.SBP_EINVAL  # the two outputs overlap
    assert L.sbp_unpack_params(plan.handle, -1, V(0x100000), two, None) == sbp.SBP_EINVAL
    assert L.sbp_shard_of(plan.handle, -1, 2, V(0x300000), V(0x400000), None) == sbp.SBP_EINVAL
    assert L.sbp_shard_of(plan.handle, -1, 0, V(0x300000), V(0x400008), None) == sbp.SBP_EALIGN
    assert L.sbp_shard_of(plan.handle, -1, 0, V(0x300000), V(0x300010), None) == sbp.SBP_EINVAL
    assert L.sbp_gather_shards(plan.handle, -1, (V * 2)(0x100000, None), V(0x300000),
                               None) == sbp.SBP_EINVAL
    assert L.sbp_gather_shards(plan.handle, -1, two, V(0x100000), None) == sbp.SBP_EINVAL
    assert L.sbp_gather_shards(plan.handle, -1, (V * 2)(0x100004, 0x200000), V(0x300000),
                               None) == sbp.SBP_EALIGN
    shards = (V * 2)(0x500000, 0x600000)
    assert L.sbp_unpack_shards(None, -1, shards, two, None) == sbp.SBP_EINVAL
    assert L.sbp_unpack_shards(plan.handle, 3, shards, two, None) == sbp.SBP_EINVAL
    assert L.sbp_unpack_shards(plan.handle, -1, (V * 2)(0x500000, None), two,
                               None) == sbp.SBP_EINVAL
    assert L.sbp_unpack_shards(plan.handle, -1, (V * 2)(0x500008, 0x600000), two,
                               None) == sbp.SBP_EALIGN
    assert L.sbp_unpack_shards(plan.handle, -1, shards, (V * 2)(0x100001, 0x200000),
                               None) == sbp.SBP_EALIGN
    assert L.sbp_unpack_shards(plan.handle, -1, shards, (V * 2)(0x100000, 0x100010),
                               None) == sbp.SBP_EINVAL  # the two outputs overlap
    assert L.sbp_unpack_shards(plan.handle, -1, shards, (V * 2)(0x100000, 0x600004),
                               None) == sbp.SBP_EINVAL  # an output inside a shard
    assert b"overlaps a shard" in L.sbp_last_error()


def test_per_tensor_plan_matches_oracle():
    rng = random.Random(8)
    for _ in range(300):
        T = rng.randint(0, 8)
        rows = [rng.choice([1, 2, 3, 7, 8, 768]) for _ in range(T)]
        numels = [r * rng.choice([0, 1, 2, 5, 13]) for r in rows]
        N, align = rng.choice([1, 2, 3, 8]), rng.choice([1, 2, 8])
        order = rng.choice(["reverse", "forward"])
        use_rows = rng.random() < 0.8
        p = sbp.bucket_plan_per_tensor(numels, N, rows if use_rows else None, align, order)
        o = OP.per_tensor_plan(numels, N, rows if use_rows else None, align, order)
        assert p.num_buckets == len(o.buckets) and p.flat_numel == o.flat_numel
        for b, ob in enumerate(o.buckets):
            assert p.bucket(b) == dict(used=ob.used, padded=ob.padded, chunk=ob.chunk,
                                       shard_offset=ob.shard_offset, flat_offset=ob.flat_offset)
            assert p.bucket_tensors(b) == ob.tensors
        for t in range(T):
            assert p.tensor(t) == (o.tensor_bucket[t], o.tensor_offset[t])
    with pytest.raises(sbp.SbpError):
        sbp.bucket_plan_per_tensor([31], 4, [3])
    with pytest.raises(sbp.SbpError):
        sbp.bucket_plan_per_tensor([30], 0, [3])


def _expand_runs(starts, groups, n):
    import numpy as np
    out = np.empty(n, dtype=np.int32)
    ends = list(starts[1:]) + [n]
    for a, e, g in zip(starts, ends, groups):
        out[a:e] = g
    return out


def _check_runs(p, o, T, rng):
    """group_runs() of every rank equals the run-length encoding of the
    oracle's per-element groups (starts ascending from 0, neighbours differ)."""
    import numpy as np
    from oracle import step as OS
    tg = [rng.randrange(sbp.MAX_GROUPS) if rng.random() < 0.7 else rng.randrange(2)
          for _ in range(T)]
    for s in range(p.world_n):
        starts, groups = sbp.group_runs(p, s, tg)
        assert starts[0] == 0 and len(starts) == len(groups) >= 1
        assert np.all(np.diff(starts) > 0) and np.all(groups[1:] != groups[:-1])
        assert (p.shard_numel == 0) == (starts[-1] >= p.shard_numel)
        want = OS.shard_groups(o, s, tg)
        assert np.array_equal(_expand_runs(starts, groups, p.shard_numel), want)


def test_group_runs_match_oracle():
    rng = random.Random(11)
    for _ in range(150):
        T = rng.randint(0, 9)
        numels = [rng.choice([0, 1, 3, 8, 13, 40, 257]) for _ in range(T)]
        N = rng.choice([1, 2, 3, 8])
        cap = rng.choice([16, 64, 200, 1 << 20])
        kind = rng.choice(["whole", "split", "per_tensor"])
        if kind == "per_tensor":
            align = rng.choice([1, 2, 8])
            p = sbp.bucket_plan_per_tensor(numels, N, None, align)
            o = OP.per_tensor_plan(numels, N, None, align)
        else:
            split = kind == "split"
            p = sbp.bucket_plan(numels, cap, N, split=split)
            o = OP.bucket_plan(numels, cap, N, split=split)
        _check_runs(p, o, T, rng)


def test_group_runs_on_workloads():
    rng = random.Random(12)
    for name in ("tiny_mlp", "gpt2_small"):
        w = synth.WORKLOADS[name]
        p = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
        o = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
        _check_runs(p, o, len(w.numels), rng)


def test_group_runs_validate():
    L = sbp.lib()
    plan = sbp.bucket_plan([10, 20], 1 << 20, 2)
    G = ctypes.c_int32 * 2
    cnt = ctypes.c_int64()
    assert L.sbp_group_runs(plan.handle, 0, G(0, 8), None, None, 0, ctypes.byref(cnt)) \
        == sbp.SBP_EINVAL
    assert L.sbp_group_runs(plan.handle, 0, G(-1, 0), None, None, 0, ctypes.byref(cnt)) \
        == sbp.SBP_EINVAL
    assert L.sbp_group_runs(plan.handle, 2, G(0, 1), None, None, 0, ctypes.byref(cnt)) \
        == sbp.SBP_EINVAL
    assert L.sbp_group_runs(None, 0, G(0, 1), None, None, 0, ctypes.byref(cnt)) == sbp.SBP_EINVAL
    assert L.sbp_group_runs(plan.handle, 0, G(0, 1), None, None, 1, ctypes.byref(cnt)) \
        == sbp.SBP_EINVAL
    assert L.sbp_group_runs(plan.handle, 0, G(0, 1), None, None, 0, ctypes.byref(cnt)) \
        == sbp.SBP_OK and cnt.value >= 1
    # a short output array gets the first `cap` runs and the full count
    starts = (ctypes.c_int64 * 1)()
    groups = (ctypes.c_int32 * 1)()
    assert L.sbp_group_runs(plan.handle, 0, G(3, 5), starts, groups, 1, ctypes.byref(cnt)) \
        == sbp.SBP_OK
    full_s, full_g = sbp.group_runs(plan, 0, [3, 5])
    assert cnt.value == len(full_s) and starts[0] == full_s[0] and groups[0] == full_g[0]


def test_grouped_step_validates_before_launch():
    L = sbp.lib()
    V = ctypes.c_void_p
    peers = (V * 2)(0x100000, 0x200000)
    hp = sbp.AdamWHParams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    gs = (sbp.GroupHParams * 2)(sbp.GroupHParams(1e-3, 0.1), sbp.GroupHParams(1e-3, 0.0))
    ok = dict(peers=peers, R=2, acc=None, scale=0.5, master=V(0x300000), m=V(0x400000),
              v=V(0x500000), p=V(0x600000), n=1024, hp=ctypes.byref(hp), groups=gs, ng=2,
              rs=V(0x700000), rg=V(0x800000), nr=3)

    def call(**kw):
        a = dict(ok, **kw)
        return L.sbp_adamw_shard_grouped(a["peers"], a["R"], a["acc"], a["scale"], a["master"],
                                         a["m"], a["v"], a["p"], a["n"], a["hp"], a["groups"],
                                         a["ng"], a["rs"], a["rg"], a["nr"], None)

    assert call(R=17) == sbp.SBP_EINVAL
    assert call(groups=None) == sbp.SBP_EINVAL
    assert call(ng=0) == sbp.SBP_EINVAL
    assert call(ng=9) == sbp.SBP_EINVAL
    assert call(nr=0) == sbp.SBP_EINVAL
    assert call(rs=None) == sbp.SBP_EINVAL
    assert call(rs=V(0x700004)) == sbp.SBP_EALIGN
    assert call(rg=V(0x800002)) == sbp.SBP_EALIGN
    assert call(rs=V(0x300000 + 64)) == sbp.SBP_EINVAL  # inside master
    assert call(rg=V(0x600000 + 64)) == sbp.SBP_EINVAL  # inside param_out
    assert call(master=V(0x300004)) == sbp.SBP_EALIGN
    assert call(m=V(0x300000 + 1024)) == sbp.SBP_EINVAL
    assert call(n=0) == sbp.SBP_OK
    assert call(n=0, rs=None, rg=None) == sbp.SBP_OK
    # each group's lr and weight decay finite and >= 0 (hp's own are not used)
    bad = (sbp.GroupHParams * 2)(sbp.GroupHParams(1e-3, 0.1), sbp.GroupHParams(-1e-3, 0.0))
    assert call(groups=bad) == sbp.SBP_EINVAL
    bad = (sbp.GroupHParams * 2)(sbp.GroupHParams(1e-3, float("nan")), sbp.GroupHParams(1e-3, 0))
    assert call(groups=bad) == sbp.SBP_EINVAL
    assert call(groups=bad, ng=1) == sbp.SBP_EINVAL
    unused = sbp.AdamWHParams(-1.0, 0.9, 0.999, 1e-8, -5.0, 1)
    assert call(hp=ctypes.byref(unused), n=0) == sbp.SBP_OK


@pytest.mark.parametrize("name,flags", [("tiny_mlp", 0), ("gpt2_small", 0), ("gpt2_small", 1),
                                        ("gpt2_small", 2)])
def test_c_client_plan_matches_oracle(tmp_path, name, flags):
    """A C99 program using only include/sbp.h builds the plan and reads every
    query back; the answers equal the oracle's planner."""
    import subprocess
    from tests import helpers as H
    exe = H.build_c_client(tmp_path)
    w = synth.WORKLOADS[name]
    cap = w.bucket_cap_bytes if flags != 2 else 1 << 20
    r = subprocess.run([exe, "plan", str(cap), str(w.world_n), "8", str(flags)]
                       + [str(x) for x in w.numels], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.split("\n")
    assert lines[0] == sbp.version()
    order = "forward" if flags & 1 else "reverse"
    o = OP.bucket_plan(w.numels, cap, w.world_n, 8, order, split=bool(flags & 2))
    want = [f"plan {len(w.numels)} {len(o.buckets)} {w.world_n} {o.shard_numel} {o.flat_numel}"]
    want += [f"tensor {t} {o.tensor_bucket[t]} {o.tensor_offset[t]}" for t in range(len(w.numels))]
    want += [" ".join(["bucket", str(b), str(ob.used), str(ob.padded), str(ob.chunk),
                       str(ob.shard_offset), str(ob.flat_offset)] + [str(i) for i in ob.tensors])
             for b, ob in enumerate(o.buckets)]
    want += [f"state {s} {OP.state_bytes(o.flat_numel, o.shard_numel, s)}" for s in range(4)]
    want += ["einval message", ""]
    assert lines[1:] == want


def test_threads_plan_and_keep_their_own_errors():
    """Plans are built and queried from several threads at once (ctypes
    releases the GIL, so the calls overlap in the library); each thread reads
    back the error message of its own last failing call."""
    import threading
    w = synth.WORKLOADS["gpt2_small"]
    want = OP.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    L = sbp.lib()
    errors = []
    barrier = threading.Barrier(8)

    def work(k):
        try:
            barrier.wait()
            for it in range(40):
                p = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
                assert p.num_buckets == len(want.buckets) and p.shard_numel == want.shard_numel
                assert p.bucket(it % p.num_buckets)["chunk"] == want.buckets[it % p.num_buckets].chunk
                out = ctypes.c_void_p()
                if k % 2:  # odd threads fail on the cap, even threads on the world size
                    st = L.sbp_bucket_plan(None, 0, 0, 1, 8, 0, ctypes.byref(out))
                    assert st == sbp.SBP_EINVAL and b"bucket_cap_bytes" in L.sbp_last_error()
                else:
                    st = L.sbp_bucket_plan(None, 0, 1, 0, 8, 0, ctypes.byref(out))
                    assert st == sbp.SBP_EINVAL and b"world_n" in L.sbp_last_error()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    ts = [threading.Thread(target=work, args=(k,)) for k in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors[:3]
