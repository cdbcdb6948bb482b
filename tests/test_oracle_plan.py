"""Pins of the oracle's bucket plan and state accounting (CPU only).

Brute force over random tiny tensor lists checks every property the planning
rule implies; hand-derived plans of the five workloads check the rule's
concrete outcome; the pages' byte counts check the state accounting.
"""

import math
import random

import pytest

import synth
from oracle import plan as P
from tests.conftest import read_golden


def _check_plan_properties(numels, cap, N, align, order):
    pl = P.bucket_plan(numels, cap, N, align, order)
    T = len(numels)
    visit = list(range(T - 1, -1, -1)) if order == "reverse" else list(range(T))
    # visit order kept, every tensor in exactly one bucket, none split
    assert [t for b in pl.buckets for t in b.tensors] == visit
    for bi, b in enumerate(pl.buckets):
        assert b.tensors, "no empty bucket"
        end = 0
        for j, t in enumerate(b.tensors):
            assert pl.tensor_bucket[t] == bi
            off = pl.tensor_offset[t]
            assert off % align == 0
            if j == 0:
                assert off == 0
            else:
                # the first aligned slot at or after the previous tensor's end
                assert end <= off < end + align or (end == 0 and off == 0)
            end = off + numels[t]
            # closing rule: no bucket reached the cap before its last tensor
            if j < len(b.tensors) - 1:
                assert 2 * end < cap
        assert b.used == end
        if bi < len(pl.buckets) - 1:
            assert 2 * b.used >= cap
        # padding: smallest multiple of align*N, split into N equal chunks
        assert b.padded % (align * N) == 0 and b.used <= b.padded < b.used + align * N
        assert b.chunk * N == b.padded
    # offsets are running sums; n is the same for every rank
    so = fo = 0
    for b in pl.buckets:
        assert b.shard_offset == so and b.flat_offset == fo
        so += b.chunk
        fo += b.padded
    assert pl.shard_numel == so and pl.flat_numel == fo == N * so
    # tensors never overlap in the flat buffer
    spans = sorted((pl.tensor_flat_offset(t), pl.tensor_flat_offset(t) + numels[t])
                   for t in range(T) if numels[t])
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    return pl


def test_plan_properties_brute_force():
    rng = random.Random(1234)
    for _ in range(3000):
        T = rng.randint(1, 10)
        numels = [rng.choice([0, 1, 3, 7, 8, 9, 16, 31, 64, 100]) for _ in range(T)]
        cap = rng.randint(1, 400)
        N = rng.choice([1, 2, 3, 4, 8])
        align = rng.choice([1, 2, 4, 8])
        order = rng.choice(["reverse", "forward"])
        _check_plan_properties(numels, cap, N, align, order)


def test_plan_exhaustive_tiny():
    """Every list of up to 4 tensors from a small size set, every cap up to 80 bytes."""
    sizes = [0, 1, 5, 8, 13]
    import itertools
    for T in range(1, 5):
        for numels in itertools.product(sizes, repeat=T):
            for cap in range(1, 81, 3):
                for N in (1, 2, 3):
                    _check_plan_properties(list(numels), cap, N, 8, "reverse")


def test_plan_rejects_bad_args():
    for args in [([1], 0, 1), ([1], 8, 0), ([1], 8, 1, 3), ([-1], 8, 1)]:
        with pytest.raises(ValueError):
            P.bucket_plan(*args)


def test_tiny_mlp_plan_by_hand():
    # reverse order b2, W2, b1, W1; cap 1 MiB = 2^20 bytes = 524288 bf16 elements.
    # b2 [256] @0; W2 [1024x256] @256 (used 262400); b1 [1024] @262400 (used
    # 263424); W1 [256x1024] @263424 -> used 525568, 2*used = 1051136 >= 2^20:
    # one bucket, padded to a multiple of 8*2 (already), chunk 262784.
    w = synth.WORKLOADS["tiny_mlp"]
    pl = P.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    assert len(pl.buckets) == 1
    b = pl.buckets[0]
    names = w.names
    assert [names[t] for t in b.tensors] == ["b2", "W2", "b1", "W1"]
    assert [pl.tensor_offset[names.index(x)] for x in ["b2", "W2", "b1", "W1"]] == [0, 256, 262400, 263424]
    assert (b.used, b.padded, b.chunk) == (525568, 525568, 262784)
    assert pl.shard_numel == 262784
    # rank 0 owns b2, W2 and the first 384 elements of b1 (a tensor split between ranks)
    assert 262784 - 262400 == 384


def test_gpt2_small_plan_by_hand():
    # Reverse order opens with ln_f.b, ln_f.w (1536 elements), then each layer
    # backwards from mlp.c_proj.b to ln_1.w: 7087872 elements a layer, 1536 of
    # them in the ln_1 pair.  The cap (25 MiB = 13107200 bf16 elements) is
    # first reached at the c_attn.w of every second layer, so each bucket is
    # a 1536-element norm pair + one whole layer + the next layer without its
    # ln_1 pair = 2*7087872 = 14175744.  The last bucket is
    # [h0.ln_1.b, h0.ln_1.w, wpe, wte] = 1536 + 786432 + 38597376 = 39385344.
    w = synth.WORKLOADS["gpt2_small"]
    pl = P.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    sizes = [b.used for b in pl.buckets]
    assert len(pl.buckets) == 7
    assert sizes[:6] == [14175744] * 6
    assert sizes[6] == 39385344
    assert [w.names[t] for t in pl.buckets[6].tensors] == ["h0.ln_1.b", "h0.ln_1.w", "wpe", "wte"]
    assert all(b.padded == b.used for b in pl.buckets)
    assert pl.shard_numel == 15554976


def test_llama3_8b_plan_by_hand():
    # Every Llama matrix except k/v is >= the 25 MiB cap (13107200 elements),
    # so buckets close at each big matrix: lm_head alone, then
    # [final_norm, l31.down], [l31.up], [l31.gate], [l31.mlp_norm, l31.o],
    # [l31.v, l31.k, l31.q], [l31.attn_norm, l30.down], ... [l0.attn_norm, embed]:
    # 1 + 32*5 + 1 = 162 buckets.
    w = synth.WORKLOADS["llama3_8b"]
    pl = P.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    nm = lambda b: [w.names[t] for t in b.tensors]
    assert len(pl.buckets) == 162
    assert [nm(b) for b in pl.buckets[:6]] == [
        ["lm_head"], ["final_norm", "l31.down"], ["l31.up"], ["l31.gate"],
        ["l31.mlp_norm", "l31.o"], ["l31.v", "l31.k", "l31.q"]]
    assert nm(pl.buckets[6]) == ["l31.attn_norm", "l30.down"]
    assert nm(pl.buckets[-1]) == ["l0.attn_norm", "embed"]
    sizes = [b.used for b in pl.buckets]
    assert min(sizes) == 4096 + 16777216 and max(sizes) == 4096 + 525336576
    assert pl.shard_numel == 1003782656 and pl.flat_numel == 8030261248
    dp = P.bucket_plan(w.numels, w.bucket_cap_bytes, 1)
    assert dp.shard_numel == 8030261248 and len(dp.buckets) == 162


def test_gpt_7b5_plan_by_hand():
    # Per layer in reverse: [.. fc2.b, fc2.w] [fc1.b, fc1.w]
    # [ln2.b, ln2.w, proj.b, proj.w] [qkv.b, qkv.w] and the ln1 pair opens the
    # next bucket: 4 buckets a layer + the final [l0.ln1.b, l0.ln1.w, wte].
    w = synth.WORKLOADS["gpt_7b5"]
    nm = lambda pl, b: [w.names[t] for t in b.tensors]
    pl = P.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    assert len(pl.buckets) == 129
    assert nm(pl, pl.buckets[0]) == ["ln_f.b", "ln_f.w", "l31.fc2.b", "l31.fc2.w"]
    assert nm(pl, pl.buckets[1]) == ["l31.fc1.b", "l31.fc1.w"]
    assert nm(pl, pl.buckets[-1]) == ["l0.ln1.b", "l0.ln1.w", "wte"]
    sizes = [b.used for b in pl.buckets]
    assert min(sizes) == 3 * 4096 + 16777216 and max(sizes) == 2 * 4096 + 50000 * 4096
    assert pl.shard_numel == 103890048
    MiB = 1 << 20
    # caps up to 32 MiB close at the same tensors; 64 and 128 MiB merge the
    # [ln2.., proj] group with qkv; 256 MiB packs about two layers a bucket.
    counts = {c: len(P.bucket_plan(w.numels, c * MiB, 64).buckets) for c in (1, 32, 64, 128, 256)}
    assert counts == {1: 129, 32: 129, 64: 97, 128: 97, 256: 49}


def test_state_bytes_pages_numbers():
    g = dict(ln.split(" = ") for ln in read_golden("state_bytes.txt"))
    g = {k: int(v) for k, v in g.items()}
    assert P.PARAM_BYTES == g["param_bytes"] and P.GRAD_BYTES == g["grad_bytes"]
    assert P.OPT_BYTES == g["optimizer_bytes"] == g["master_bytes"] + g["moments_bytes"]
    assert g["moments_bytes"] == g["m_bytes"] + g["v_bytes"]
    psi = g["example_params"]
    assert P.state_bytes(psi, psi, 0) == g["example_state_bytes"]  # 7.5B -> 120 GB
    assert P.state_bytes(psi, psi, 0) == g["total_bytes_per_param"] * psi


def test_state_bytes_zero_stages():
    psi = 7_500_000_000
    N = 64
    n = psi // N  # 7.5e9 is not divisible by 64; use exact rational arithmetic instead
    from fractions import Fraction
    sh = Fraction(psi, N)
    want = {1: 4 * psi + 12 * sh, 2: 2 * psi + 14 * sh, 3: 16 * sh}
    assert float(want[1]) == 31.40625e9 and float(want[2]) == 16.640625e9 and float(want[3]) == 1.875e9
    for stage in (1, 2, 3):
        assert P.state_bytes(psi * 64, psi, stage) == int(want[stage] * 64)
    # "ZeRO-1 ... 4x less memory", "ZeRO-2 ... 8x less" relative to DP's 16 bytes,
    # reached as N grows ("Parallelism Strategies in Distributed Computing", ZeRO and FSDP)
    big = 1 << 40
    full = 16 * big
    assert abs(full / P.state_bytes(big, big >> 20, 1) - 4) < 1e-4
    assert abs(full / P.state_bytes(big, big >> 20, 2) - 8) < 1e-4
    # ZeRO-3: falls linearly with N
    assert P.state_bytes(big, big // 8, 3) * 8 == P.state_bytes(big, big, 3) == full
    assert n > 0


def test_state_bytes_workload_plans():
    w = synth.WORKLOADS["llama3_8b"]
    pl = P.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
    assert P.state_bytes(pl.flat_numel, pl.shard_numel, 0) == 16 * 8030261248
    assert P.state_bytes(pl.flat_numel, pl.shard_numel, 3) == 16 * 1003782656


# ---- fixed-size buckets with tensors split across them ----------------------------

def _check_split_plan(numels, cap, N, align, order):
    pl = P.bucket_plan(numels, cap, N, align, order, split=True)
    T = len(numels)
    unit = align * N
    size = max(unit, (cap // 2) // unit * unit)
    visit = list(range(T - 1, -1, -1)) if order == "reverse" else list(range(T))
    pos = {t: pl.tensor_flat_offset(t) for t in range(T)}
    # concatenation in visit order at the first aligned slot
    end = 0
    for t in visit:
        want = 0 if end == 0 else -(-end // align) * align
        assert pos[t] == want
        end = want + numels[t]
    total = end
    # equal buckets of `size` elements, only the last one short (and padded)
    nb = len(pl.buckets)
    assert nb == (-(-total // size) if total else (1 if T else 0))
    for b, bk in enumerate(pl.buckets):
        assert bk.flat_offset == b * size
        if b < nb - 1:
            assert bk.used == bk.padded == size
        assert bk.padded % unit == 0 and bk.used <= bk.padded < bk.used + unit or bk.used == 0
        assert bk.chunk * N == bk.padded
    # every element of a tensor lies in exactly one bucket listing the tensor
    for t in range(T):
        for e in range(pos[t], pos[t] + numels[t]):
            b = e // size
            assert t in pl.buckets[b].tensors
        if numels[t]:
            assert pl.tensor_bucket[t] == pos[t] // size
    so = 0
    for bk in pl.buckets:
        assert bk.shard_offset == so
        so += bk.chunk
    assert pl.shard_numel == so and pl.flat_numel == N * so == sum(b.padded for b in pl.buckets)
    return pl


def test_split_plan_properties_brute_force():
    rng = random.Random(77)
    for _ in range(1500):
        T = rng.randint(0, 8)
        numels = [rng.choice([0, 1, 3, 8, 9, 31, 64, 100]) for _ in range(T)]
        _check_split_plan(numels, rng.randint(1, 300), rng.choice([1, 2, 3, 4]),
                          rng.choice([1, 2, 4, 8]), rng.choice(["reverse", "forward"]))


def test_split_plan_gpt_7b5_cap_sweep():
    # every numel of this model is a multiple of 8, so the flat buffer is the plain
    # concatenation of 6,648,963,072 elements; a c MiB cap gives buckets of
    # c * 2^19 elements (a multiple of 8 * 64): ceil(6648963072 / (c * 2^19)).
    w = synth.WORKLOADS["gpt_7b5"]
    got = {c: len(P.bucket_plan(w.numels, c << 20, 64, split=True).buckets)
           for c in (1, 2, 4, 8, 16, 32, 64, 128, 256)}
    assert got == {1: 12682, 2: 6341, 4: 3171, 8: 1586, 16: 793, 32: 397, 64: 199, 128: 100,
                   256: 50}
    pl = P.bucket_plan(w.numels, 25 << 20, 64, split=True)
    assert pl.shard_numel == 103890048  # same shard size as whole-tensor buckets (no padding)


# ---- one bucket per tensor, dim-0 row shards -----------------------------------

def test_per_tensor_plan_rows():
    # a [10, 3] matrix on N = 4 ranks with align 1: torch.chunk-style dim-0 split
    # gives ceil(10/4) = 3 rows per rank (the last rank 1 row + 2 padding rows)
    pl = P.per_tensor_plan([30], 4, rows=[3], align=1)
    b = pl.buckets[0]
    assert (b.used, b.padded, b.chunk) == (30, 36, 9)
    # with align 8: unit lcm(8, 3) = 24 elements (8 rows), chunk = 24
    pl = P.per_tensor_plan([30], 4, rows=[3], align=8)
    assert (pl.buckets[0].padded, pl.buckets[0].chunk) == (96, 24)
    with pytest.raises(ValueError):
        P.per_tensor_plan([31], 4, rows=[3])


def test_per_tensor_plan_properties():
    rng = random.Random(3)
    for _ in range(1000):
        T = rng.randint(0, 8)
        rows = [rng.choice([1, 2, 3, 7, 8, 768]) for _ in range(T)]
        numels = [r * rng.choice([0, 1, 2, 5, 13]) for r in rows]
        N = rng.choice([1, 2, 3, 8])
        align = rng.choice([1, 2, 8])
        order = rng.choice(["reverse", "forward"])
        pl = P.per_tensor_plan(numels, N, rows, align, order)
        visit = list(range(T - 1, -1, -1)) if order == "reverse" else list(range(T))
        assert [b.tensors for b in pl.buckets] == [[t] for t in visit]
        for b in pl.buckets:
            t = b.tensors[0]
            assert b.used == numels[t] and pl.tensor_offset[t] == 0
            assert b.chunk % rows[t] == 0 and b.chunk % align == 0  # whole, aligned rows
            assert b.chunk * N == b.padded >= b.used
            assert b.padded - b.used < N * (align * rows[t] // math.gcd(align, rows[t]))
        assert pl.flat_numel == N * pl.shard_numel


def test_per_tensor_plan_llama_rows():
    # Llama-3-8B, N = 8: every matrix's dim 0 (4096, 1024, 14336, 128256) is a
    # multiple of 8 and rows are multiples of 8, so no padding at all
    w = synth.WORKLOADS["llama3_8b"]
    rows = [s[1] if len(s) == 2 else 1 for _, s in w.params]
    pl = P.per_tensor_plan(w.numels, 8, rows)
    assert len(pl.buckets) == 291 and pl.flat_numel == w.psi and pl.shard_numel == w.psi // 8
