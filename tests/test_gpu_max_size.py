"""The largest shard the calls accept, SBP_MAX_SHARD_NUMEL = (2^24 - 1) * 2048
elements: the grid of 2^24 - 1 tiles and its XCD deal at full size.  The
one-peer reduce and the one-peer squared norm fit in HBM there (206 GB with
their fp32 output); the fused step (42 B per element) does not.

- reduce: seeded bf16 input, the fp32 sum compared with the oracle in 64
  windows of 256 elements spread over the shard, the last one ending at its
  end;
- squared norm over a shard of ones, writing G: every square is 1, so every
  float64 partial sum is an exact integer and the result must be n exactly
  -- a tile dropped or counted twice anywhere in the grid changes it -- and G
  must be 1 everywhere."""

import numpy as np
import pytest

import sharded_bucket_plan_amd as sbp
import synth
from oracle import step as OS
from tests import helpers as H

pytestmark = pytest.mark.gpu

N = sbp.MAX_SHARD_NUMEL
NEED = 6 * N + (8 << 30)  # bf16 peer + fp32 output, and room for the rest


@pytest.fixture(autouse=True)
def _gpu():
    H.need_gpu()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _windows(n, count=64, width=256, seed=5):
    rng = np.random.default_rng(seed)
    starts = sorted(set(int(x) for x in rng.integers(0, n - width, count - 2)) | {0, n - width})
    return [(s, s + width) for s in starts]


def test_max_shard_reduce_and_norm():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < NEED:
        pytest.skip(f"{free / 2**30:.0f} GiB free, {NEED / 2**30:.0f} GiB needed")
    assert N == (2**24 - 1) * 2048
    arena = sbp.Arena([2 * N, 4 * N])
    peer = arena.tensor(0, torch.int16, N)
    out = arena.tensor(1, torch.float32, N)
    sigma = 1e-3
    stream = synth.peer_stream(1, 0, 0)
    synth.dev_normal_bf16(peer, synth.SEED, stream, sigma)
    sbp.reduce_shard([peer], 1.0, out)
    torch.cuda.synchronize()
    for a, b in _windows(N):
        want = OS.reduce_peers([synth.normal_bf16(synth.SEED, stream, b - a, sigma, a)])
        H.assert_bits_equal(H.to_np_f32(out[a:b]), want, f"max-size reduce [{a}, {b})")
    peer.fill_(0x3F80)  # bf16 1.0
    out.fill_(0.0)
    sq = sbp.grad_sq_norm([peer], None, 1.0, N, g_sum_out=out).item()
    assert sq == float(N), (sq, N)
    step = 1 << 31  # compare in slices: a whole-shard mask would take 34 GB
    for i in range(0, N, step):
        assert bool(torch.all(out[i:i + step] == 1.0).item()), f"G differs from 1 in [{i}, {i + step})"
    del peer, out, arena
    gc.collect()
