"""The spread arena on the GPU: its arrays hold what is written to them, do
not overlap, are chunk-aligned, and the chunks it spread over but did not
keep go back to the device; the fused step on arena arrays is bit-exact
against the oracle (GPT-2-small shard, every element, two steps)."""

import numpy as np
import pytest

import sharded_bucket_plan_amd as sbp
import synth
from oracle import step as OS
from tests import helpers as H

pytestmark = pytest.mark.gpu

MiB = 1 << 20


@pytest.fixture(autouse=True)
def _gpu():
    H.need_gpu()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_arena_arrays_hold_data_and_do_not_overlap():
    import torch
    sizes = [3 * MiB + 5 * 4, 70 * MiB, 0, 64 * MiB, 4]
    a = sbp.Arena(sizes, chunk=2 * MiB, spread=8 << 30, seed=7)
    info = a.info()
    kept = sum((b + 2 * MiB - 1) // (2 * MiB) for b in sizes)
    assert info["chunk_bytes"] == 2 * MiB and info["chunks_kept"] == kept
    assert info["chunks_spread"] == 4096  # 8 GiB of 2 MiB chunks
    assert a.ptrs[2] == 0
    spans = sorted((p, p + b) for p, b in zip(a.ptrs, sizes) if b)
    assert all(p % (2 * MiB) == 0 for p, _ in spans)
    assert all(e1 <= p2 for (_, e1), (p2, _) in zip(spans, spans[1:]))
    ts = [a.tensor(i, torch.float32) for i in (0, 1, 3, 4)]
    for k, t in enumerate(ts):
        t.copy_(torch.arange(t.numel(), dtype=torch.float32, device=H.dev()) * 3 + k)
    torch.cuda.synchronize()
    for k, t in enumerate(ts):
        want = np.arange(t.numel(), dtype=np.float32) * 3 + k
        H.assert_bits_equal(H.to_np_f32(t), want, f"arena array {k}")
    del ts, a


def test_arena_releases_what_it_does_not_keep():
    import torch
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    a = sbp.Arena([100 * MiB] * 4, chunk=64 * MiB, spread=16 << 30, seed=1)
    free1, _ = torch.cuda.mem_get_info()
    info = a.info()
    assert info["chunks_kept"] == 8 and info["chunks_spread"] == 256
    # the 8 kept chunks stay (give or take the driver's own accounting); the
    # other 248 of the 16 GiB spread over are back
    used = free0 - free1
    assert 8 * 64 * MiB - 64 * MiB <= used <= 8 * 64 * MiB + 256 * MiB, used
    del a
    import gc
    gc.collect()
    torch.cuda.synchronize()
    free2, _ = torch.cuda.mem_get_info()
    assert free2 >= free0 - 256 * MiB


def test_arena_tensor_keeps_the_arena_alive():
    import gc
    import torch
    a = sbp.Arena([8 * MiB], chunk=2 * MiB, spread=64 * MiB)
    t = a.tensor(0, torch.int32)
    del a
    gc.collect()
    t.fill_(5)  # the arena must still be mapped
    torch.cuda.synchronize()
    assert int(t.sum().item()) == 5 * t.numel()


def test_fused_step_on_arena_arrays_gpt2_small_full():
    """GPT-2-small ZeRO-2 shard (N=8, R=8, 15.5M elements) with the peers,
    master, m, v and the parameter shard in one spread arena: two steps,
    every element against the oracle."""
    import torch
    w = synth.WORKLOADS["gpt2_small"]
    hp = sbp.AdamW(w.adamw.lr, w.adamw.beta1, w.adamw.beta2, w.adamw.eps, w.adamw.weight_decay)
    n = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n).shard_numel
    assert n == 15554976
    a = sbp.Arena([2 * n] * w.R + [4 * n] * 3 + [2 * n], chunk=2 * MiB, seed=3)
    bufs = [a.tensor(r, torch.int16, n) for r in range(w.R)]
    dth, dm, dv = (a.tensor(w.R + j, torch.float32, n) for j in range(3))
    dp = a.tensor(w.R + 3, torch.int16, n)
    th = synth.normal_f32(synth.SEED, synth.master_stream(0), n, w.master_sigma)
    dth.copy_(torch.from_numpy(th).to(H.dev()))
    dm.zero_()
    dv.zero_()
    z = np.zeros(n, np.float32)
    want = (th, z, z, None)
    for t in (1, 2):
        H.dev_peers(synth.SEED, t, 0, w.R, n, w.grad_sigma, bufs)
        sbp.adamw_shard(bufs, None, sbp.mean_scale(w.R), dth, dm, dv, dp, hp, t)
        want = OS.shard_step(H.host_peers(synth.SEED, t, 0, w.R, n, w.grad_sigma), None,
                             OS.mean_scale(w.R), want[0], want[1], want[2], hp, t)
    torch.cuda.synchronize()
    got = (H.to_np_f32(dth), H.to_np_f32(dm), H.to_np_f32(dv), H.to_np_u16(dp))
    for x, y, name in zip(got, want, ("master", "m", "v", "param")):
        H.assert_bits_equal(x, y, f"gpt2_small on the arena {name}")


def test_failed_arena_leaves_no_hip_error():
    """An arena larger than the whole device fails (out of memory part way
    through creating its chunks).  The chunks it did create go back, and the
    HIP error it handled is not left as the thread's last error, where the
    next launch check (torch's, here) would report it."""
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0, total = torch.cuda.mem_get_info()
    with pytest.raises(sbp.SbpError) as err:
        sbp.Arena([total + (16 << 30)], chunk=64 * MiB)
    assert err.value.status in (sbp.SBP_ENOMEM, sbp.SBP_EHIP), err.value
    x = torch.arange(1 << 20, dtype=torch.float64, device=H.dev())
    assert float(x.sum().item()) == float((1 << 20) * ((1 << 20) - 1) // 2)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 >= free0 - 256 * MiB
    a = sbp.Arena([4 * MiB], chunk=2 * MiB, spread=64 * MiB)
    t = a.tensor(0, torch.int32)
    t.fill_(3)
    torch.cuda.synchronize()
    assert int(t.sum().item()) == 3 * t.numel()
