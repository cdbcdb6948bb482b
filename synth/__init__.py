"""Seeded synthetic inputs for the shard step (shared by both sides).

Every input the tests and the benchmark feed to the shard step comes from
here: peer gradient chunks (bf16, shard layout), per-tensor gradients of one
rank (bf16), initial fp32 master weights, and per-rank valid-token counts.
Values are a pure function of (seed, stream, index) (Philox4x32-10, see
philox.h), so the host generator (numpy arrays, for the oracle) and the
device generator (HBM buffers, for the HIP path) give identical bytes, and
any single element can be regenerated on its own for sampled checks.

This module holds none of the step's arithmetic.
"""

import ctypes
import os

import numpy as np

from .workloads import SEED, TOKENS_HI, TOKENS_LO, WORKLOADS, AdamW, Workload

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsbpsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsbpsynth_dev.so")

KIND_PEER, KIND_TENSOR, KIND_MASTER, KIND_TOKENS = 1, 2, 3, 4

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            from .build import build_host
            build_host()
        L = ctypes.CDLL(HOST_LIB)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.synth_ih8_scale.argtypes = [ctypes.c_double]
        L.synth_ih8_scale.restype = ctypes.c_double
        L.synth_stream_word_a.argtypes = [ctypes.c_uint32] * 2
        L.synth_stream_word_a.restype = ctypes.c_uint32
        L.synth_stream_word_b.argtypes = [ctypes.c_uint32] * 3
        L.synth_stream_word_b.restype = ctypes.c_uint32
        common = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        L.synth_fill_bf16.argtypes = [u16p, ctypes.c_int64] + common + [ctypes.c_uint64, ctypes.c_double]
        L.synth_fill_f32.argtypes = [f32p, ctypes.c_int64] + common + [ctypes.c_uint64, ctypes.c_double]
        L.synth_gather_bf16.argtypes = [u16p, i64p, ctypes.c_int64] + common + [ctypes.c_double]
        L.synth_gather_f32.argtypes = [f32p, i64p, ctypes.c_int64] + common + [ctypes.c_double]
        L.synth_tokens.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                   ctypes.c_int64, ctypes.c_int64]
        L.synth_tokens.restype = ctypes.c_int64
        L.synth_philox.argtypes = [ctypes.POINTER(ctypes.c_uint32)] + [ctypes.c_uint32] * 6
        for f in (L.synth_fill_bf16, L.synth_fill_f32, L.synth_gather_bf16, L.synth_gather_f32,
                  L.synth_philox):
            f.restype = None
        _host = L
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(DEV_LIB)
        for name in ("synth_dev_fill_bf16", "synth_dev_fill_f32"):
            f = getattr(L, name)
            f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                          ctypes.c_uint32, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p]
            f.restype = ctypes.c_int
        _dev = L
    return _dev


def philox4x32_10(counter, key):
    """Raw Philox4x32-10 block (for the generator's own known-answer tests)."""
    out = (ctypes.c_uint32 * 4)()
    _load_host().synth_philox(out, *[ctypes.c_uint32(x) for x in tuple(counter) + tuple(key)])
    return tuple(out)


def ih8_scale(sigma):
    return _load_host().synth_ih8_scale(float(sigma))


# ---- stream keys -----------------------------------------------------------

def _words(kind, t, k, r, ident):
    L = _load_host()
    return L.synth_stream_word_a(kind, t), L.synth_stream_word_b(k, r, ident)


def peer_stream(t, k, r):
    """Peer r's gradient chunk at optimizer step t, microbatch k (shard layout)."""
    return _words(KIND_PEER, t, k, r, 0)


def tensor_stream(t, k, r, tensor_id):
    """Rank r's gradient of tensor `tensor_id` at step t, microbatch k."""
    return _words(KIND_TENSOR, t, k, r, tensor_id)


def master_stream(shard_index):
    """Initial fp32 master weights of shard `shard_index` (shard layout)."""
    return _words(KIND_MASTER, 0, 0, shard_index, 0)


# ---- host generation (numpy) -----------------------------------------------

def _u16p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _f32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _i64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def normal_bf16(seed, stream, n, sigma, i0=0):
    """bf16 bits (np.uint16) of elements i0 .. i0+n-1 of a stream."""
    out = np.empty(int(n), dtype=np.uint16)
    _load_host().synth_fill_bf16(_u16p(out), int(n), seed, stream[0], stream[1], int(i0),
                                 ih8_scale(sigma))
    return out


def normal_f32(seed, stream, n, sigma, i0=0):
    out = np.empty(int(n), dtype=np.float32)
    _load_host().synth_fill_f32(_f32p(out), int(n), seed, stream[0], stream[1], int(i0),
                                ih8_scale(sigma))
    return out


def normal_bf16_at(seed, stream, idx, sigma):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    _load_host().synth_gather_bf16(_u16p(out), _i64p(idx), idx.size, seed, stream[0],
                                   stream[1], ih8_scale(sigma))
    return out


def normal_f32_at(seed, stream, idx, sigma):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    _load_host().synth_gather_f32(_f32p(out), _i64p(idx), idx.size, seed, stream[0],
                                  stream[1], ih8_scale(sigma))
    return out


def tokens(seed, t, r, lo=TOKENS_LO, hi=TOKENS_HI):
    """Valid-token count of rank r at optimizer step t (uniform on [lo, hi])."""
    return int(_load_host().synth_tokens(seed, t, r, lo, hi))


# ---- device generation (torch tensors in HBM) --------------------------------

def _dev_fill(fn, tensor, seed, stream, sigma, i0, stream_handle):
    if not tensor.is_cuda or not tensor.is_contiguous():
        raise ValueError("device generator needs a contiguous device tensor")
    if stream_handle is None:
        import torch
        stream_handle = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = fn(ctypes.c_void_p(tensor.data_ptr()), tensor.numel(), seed, stream[0], stream[1],
            int(i0), ih8_scale(sigma), ctypes.c_void_p(stream_handle))
    if rc != 0:
        raise RuntimeError(f"device generator failed ({rc})")
    return tensor


def dev_normal_bf16(tensor, seed, stream, sigma, i0=0, stream_handle=None):
    """Fill a 2-byte device tensor (bf16 or int16/uint16 view) with bf16 bits."""
    if tensor.element_size() != 2:
        raise ValueError("bf16 fill needs a 2-byte tensor")
    return _dev_fill(_load_dev().synth_dev_fill_bf16, tensor, seed, stream, sigma, i0,
                     stream_handle)


def dev_normal_f32(tensor, seed, stream, sigma, i0=0, stream_handle=None):
    import torch
    if tensor.dtype != torch.float32:
        raise ValueError("f32 fill needs a float32 tensor")
    return _dev_fill(_load_dev().synth_dev_fill_f32, tensor, seed, stream, sigma, i0,
                     stream_handle)


__all__ = [
    "SEED", "TOKENS_LO", "TOKENS_HI", "WORKLOADS", "AdamW", "Workload",
    "philox4x32_10", "ih8_scale", "peer_stream", "tensor_stream", "master_stream",
    "normal_bf16", "normal_f32", "normal_bf16_at", "normal_f32_at", "tokens",
    "dev_normal_bf16", "dev_normal_f32",
]
