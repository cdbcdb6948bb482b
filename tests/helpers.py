"""Shared helpers of the GPU tests: device buffers, seeded inputs on both
sides, ordered-bit ulp distances, guard bands."""

import numpy as np
import pytest

import synth


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")


def dev():
    import torch
    return torch.device("cuda:0")


def empty_u16(n, guard=0):
    """2-byte device tensor (int16 storage for bf16 bits)."""
    import torch
    return torch.empty(n + 2 * guard, dtype=torch.int16, device=dev())


def to_np_u16(t):
    return t.cpu().numpy().view(np.uint16)


def to_np_f32(t):
    return t.cpu().numpy()


def from_np_u16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev())


def from_np_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


# ---- ulp distances on ordered bit patterns ------------------------------------

def _ordered32(a):
    i = np.ascontiguousarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(i < 0, -(i & 0x7FFFFFFF), i)


def ulp_f32(a, b):
    """Distance in binary32 ulps (+0 and -0 coincide; two NaNs are 0 apart,
    a NaN against a number is infinitely far)."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    d = np.abs(_ordered32(a) - _ordered32(b)).astype(np.float64)
    na, nb = np.isnan(a), np.isnan(b)
    d[na & nb] = 0
    d[na ^ nb] = np.inf
    return d


def ulp_bf16(a, b):
    a = np.asarray(a, np.uint16).astype(np.uint32) << 16
    b = np.asarray(b, np.uint16).astype(np.uint32) << 16
    return ulp_f32(a.view(np.float32), b.view(np.float32)) / 65536.0


def assert_bits_equal(got, want, what):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, what
    if got.dtype == np.float32:
        g, w = got.view(np.uint32), want.view(np.uint32)
    else:
        g, w = got, want
    bad = np.flatnonzero(g != w)
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ; first at {bad[:5]}: "
                           f"got {got.ravel()[bad[:5]]} want {want.ravel()[bad[:5]]}")


def assert_state_close(got, want, what, f32_ulps=4, bf16_ulps=1):
    """Tolerance for the state: master/m/v within 4 fp32 ulp, params within 1 bf16 ulp.
    Returns the largest distance seen (expected 0: the path is bit-exact)."""
    th, m, v, p = got
    wth, wm, wv, wp = want
    worst = 0.0
    for a, b, name in ((th, wth, "master"), (m, wm, "m"), (v, wv, "v")):
        d = ulp_f32(a, b)
        mx = float(d.max()) if d.size else 0.0
        assert mx <= f32_ulps, f"{what}: {name} off by {mx} ulp"
        worst = max(worst, mx)
    d = ulp_bf16(p, wp)
    mx = float(d.max()) if d.size else 0.0
    assert mx <= bf16_ulps, f"{what}: param off by {mx} bf16 ulp"
    return max(worst, mx)


# ---- the squared norm's summation bound ---------------------------------------

def sq_norm_depth(n, gpl):
    """Longest chain of float64 additions any term of sbp_grad_sq_norm passes
    through, from the documented fixed shape: a lane adds its 8*gpl squares
    in order (plus one tail element in the first block), the wave adds by a
    6-level shuffle tree, the block adds its 4 wave sums in order; each level
    of the tree over the tile partials adds 8 per lane in order, then the
    same wave and block steps; levels run while more than 2048 partials are
    left, and a last one sums what remains."""
    tiles = max(1, ((n >> 3) + 255) // 256)
    count = (tiles + gpl - 1) // gpl
    levels = 1
    while count > 2048:
        count = (count + 2047) // 2048
        levels += 1
    return 8 * gpl + 1 + 6 + 4 + levels * (8 + 6 + 4)


def sq_norm_bound(G, scale, n, gpl):
    """Bound on |library - oracle| for the squared norm of g = fl(G*scale):
    the squares are exact in float64 and all terms are >= 0, so a sum whose
    terms each pass through at most d roundings is within gamma_d * sum
    (gamma_d = d*u / (1 - d*u), u = 2^-53) of the exact sum; the oracle's
    correctly rounded sum is within u * sum of it."""
    g = (np.asarray(G, np.float32) * np.float32(scale)).astype(np.float64)
    total = float(np.sum(g * g))
    u = 2.0 ** -53
    d = sq_norm_depth(n, gpl)
    return (d * u / (1 - d * u) + u) * total * (1 + 1e-9)  # np.sum's own slack


def norm_gpl(R, with_acc):
    """Groups of 8 per lane the norm pass takes (16 or 32 bytes of loads per
    group take 4 or 2), as the header's launch description states."""
    lane_bytes = 16 * R + (32 if with_acc else 0)
    return 4 if lane_bytes == 16 else 2 if lane_bytes == 32 else 1


# ---- seeded inputs on both sides --------------------------------------------

def host_peers(seed, t, k, R, n, sigma, i0=0):
    return [synth.normal_bf16(seed, synth.peer_stream(t, k, r), n, sigma, i0) for r in range(R)]


def dev_peers(seed, t, k, R, n, sigma, bufs=None):
    out = bufs if bufs is not None else [empty_u16(n) for _ in range(R)]
    for r in range(R):
        synth.dev_normal_bf16(out[r], seed, synth.peer_stream(t, k, r), sigma)
    return out


def guarded(n, itemsize, guard=64, fill=0x5A):
    """A device buffer with `guard` canary bytes on each side; returns
    (whole buffer as uint8, the inner view of n elements as a typed tensor)."""
    import torch
    g = max(guard, 16)
    whole = torch.full((n * itemsize + 2 * g,), fill, dtype=torch.uint8, device=dev())
    inner = whole[g:g + n * itemsize]
    dt = {2: torch.int16, 4: torch.float32, 8: torch.float64}[itemsize]
    return whole, inner.view(dt), g


def guarded_from(a):
    """guarded() holding a copy of the numpy array `a` (float32, or uint16 bf16
    bits)."""
    import torch
    a = np.ascontiguousarray(a)
    whole, inner, g = guarded(a.size, a.dtype.itemsize)
    if a.size:
        src = a.view(np.int16) if a.dtype.itemsize == 2 else a
        inner.copy_(torch.from_numpy(src).to(dev()))
    return whole, inner, g


def canaries_intact(whole, g, fill=0x5A):
    w = whole.cpu().numpy()
    return bool(np.all(w[:g] == fill) and np.all(w[-g:] == fill))


def build_c_client(out_dir):
    """Compile tests/native/abi_c.c, a plain C99 client of include/sbp.h, with
    gcc and link it against the in-tree libsbp.so; returns the executable."""
    import os
    import shutil
    import subprocess

    import sharded_bucket_plan_amd as sbp
    if shutil.which("gcc") is None:
        pytest.skip("needs gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(os.path.abspath(sbp.LIB_PATH))
    exe = os.path.join(str(out_dir), "abi_c")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
           os.path.join(root, "tests", "native", "abi_c.c"), "-o", exe,
           "-L", libdir, "-lsbp", "-Wl,-rpath," + libdir,
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe
