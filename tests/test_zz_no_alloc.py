"""The allocation-free squared norm (sbp_grad_sq_norm_noalloc) against the
entry point it varies, sbp_grad_sq_norm with a caller workspace, through the
C ABI: the same squared norm bits and the same G, on calls in a row that
reuse the library's static per-GPU scratch with a smaller input each time
(the scratch keeps the previous call's partials; nothing may leak into the
next result).  Both are also held to the oracle's squared norm within the
float64 summation bound."""

import numpy as np
import pytest

import sharded_bucket_plan_amd as sbp
from oracle import step as OS
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    H.need_gpu()
    yield
    import torch
    torch.cuda.synchronize()

# (R, with accumulator, n, write G): large first, each call smaller than the
# one before; ragged n (tails of 5, 3 and 1 elements past a whole group)
CALLS = [
    (8, False, 256 * 32 * 256 * 8 + 5, True),  # 16.8M elements, 8192 tiles
    (2, False, 256 * 8 * 9 + 3, False),  # 9 tiles
    (0, True, 256 * 8 * 3 + 1, True),  # accumulator only, 3 tiles (2 per lane group)
    (3, True, 9, False),  # one tile
]


def _inputs(R, with_acc, n, seed):
    import torch
    bufs = H.dev_peers(seed, 1, 0, R, n, 1e-3) if R else []
    acc_d = acc_h = None
    if with_acc:
        acc_d = torch.empty(n, dtype=torch.float32, device=H.dev())
        sbp.accumulate_grads(acc_d, H.dev_peers(seed, 1, 1, 2, n, 1e-3), first=True)
        acc_h = OS.reduce_peers(H.host_peers(seed, 1, 1, 2, n, 1e-3))
    if R:
        S = OS.reduce_peers(H.host_peers(seed, 1, 0, R, n, 1e-3))
        G = S if acc_h is None else acc_h + S
    else:
        G = acc_h
    return bufs, acc_d, G


def test_noalloc_matches_workspace_variant_on_calls_in_a_row():
    import torch
    for i, (R, with_acc, n, write) in enumerate(CALLS):
        print(f"noalloc call {i}: R={R} acc={with_acc} n={n} write_G={write}", flush=True)
        bufs, acc_d, G = _inputs(R, with_acc, n, 40 + i)
        scale = sbp.mean_scale(max(R, 1), 2)
        sq_a = torch.full((1,), -1.0, dtype=torch.float64, device=H.dev())
        sq_b = torch.full((1,), -2.0, dtype=torch.float64, device=H.dev())
        g_a = g_b = None
        if write:
            g_a = torch.full((n,), float("nan"), dtype=torch.float32, device=H.dev())
            g_b = torch.full((n,), float("inf"), dtype=torch.float32, device=H.dev())
        sbp.grad_sq_norm_noalloc(bufs, acc_d, scale, n, sq_a, g_sum_out=g_a)
        sbp.grad_sq_norm(bufs, acc_d, scale, n, g_sum_out=g_b, sq_out=sq_b)
        torch.cuda.synchronize()
        a, b = float(sq_a.item()), float(sq_b.item())
        assert np.float64(a).view(np.uint64) == np.float64(b).view(np.uint64), (i, a, b)
        want = OS.grad_sq_norm(G, np.float32(scale))
        bound = H.sq_norm_bound(G, scale, n, H.norm_gpl(R, with_acc))
        assert abs(a - want) <= bound, (i, a, want, bound)
        if write:
            H.assert_bits_equal(H.to_np_f32(g_a), H.to_np_f32(g_b), f"call {i} G")
            H.assert_bits_equal(H.to_np_f32(g_a), G, f"call {i} G vs oracle")


def test_noalloc_empty_and_refusals():
    import torch
    sq = torch.full((1,), 7.0, dtype=torch.float64, device=H.dev())
    sbp.grad_sq_norm_noalloc([H.empty_u16(0)], None, 1.0, 0, sq)
    torch.cuda.synchronize()
    assert sq.item() == 0.0
    # a size beyond the scratch is refused on the host, before any launch
    import ctypes
    x = H.empty_u16(16)
    V = ctypes.c_void_p
    st = sbp.lib().sbp_grad_sq_norm_noalloc((V * 1)(x.data_ptr()), 1, None, 1.0,
                                            sbp.NOALLOC_MAX_NUMEL + 1, None, sq.data_ptr(), None)
    assert st == sbp.SBP_ERANGE
    torch.cuda.synchronize()
    assert sq.item() == 0.0  # untouched


def test_noalloc_in_a_captured_graph():
    """What the call is for: captured in a HIP graph with no allocation in or
    around it.  Four replays, each after eager calls of other sizes that
    overwrite the shared scratch; every replay's squared norm and G must
    equal the eager result (each call writes every scratch slot it reads)."""
    import torch
    R, n = 4, 256 * 8 * 40 + 3
    bufs, acc_d, G = _inputs(R, True, n, 77)
    scale = sbp.mean_scale(R, 2)
    sq = torch.empty(1, dtype=torch.float64, device=H.dev())
    g_out = torch.empty(n, dtype=torch.float32, device=H.dev())
    sbp.grad_sq_norm_noalloc(bufs, acc_d, scale, n, sq, g_sum_out=g_out)  # eager (and first) call
    torch.cuda.synchronize()
    want_sq, want_g = sq.clone(), g_out.clone()
    other_bufs, _, _ = _inputs(8, False, 256 * 8 * 1000 + 1, 78)  # a larger call, other data
    other_sq = torch.empty(1, dtype=torch.float64, device=H.dev())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream, as capture expects
        sbp.grad_sq_norm_noalloc(bufs, acc_d, scale, n, sq, g_sum_out=g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sbp.grad_sq_norm_noalloc(bufs, acc_d, scale, n, sq, g_sum_out=g_out)
    for rep in range(4):
        # eager work between replays: other sizes through the same scratch
        sbp.grad_sq_norm_noalloc(other_bufs, None, 0.125, 256 * 8 * 1000 + 1, other_sq)
        sbp.grad_sq_norm_noalloc(bufs[:1], None, 1.0, n, other_sq)
        sq.fill_(-1.0)
        g_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sq, want_sq), f"replay {rep}: squared norm differs"
        assert torch.equal(g_out, want_g), f"replay {rep}: G differs"
