"""Python binding of libsbp.so, the shard-step C ABI (include/sbp.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Device buffers are torch tensors on a ROCm device (PyTorch supplies
device memory and streams); they are passed as raw pointers together with
the current HIP stream.  There is no fallback: if libsbp.so is missing, or a
call fails, an error is raised.

Functions (same names as the C calls without the "sbp_" prefix):
  plans        bucket_plan (whole-tensor or split buckets), bucket_plan_per_tensor
               (one bucket per tensor, dim-0 row shards), Plan queries
  layout       pack_grads, unpack_params, shard_of, gather_shards, unpack_shards
               (+ TensorSet: a plan's per-tensor buffers marshalled once)
  scales       mean_scale, tokens_scale, clip_scale
  shard step   reduce_shard, accumulate_grads, adamw_shard, grad_sq_norm
               (+ grad_sq_norm_workspace), grad_sq_norm_noalloc (no workspace
               argument: the library's static per-GPU scratch)
  groups       group_runs (+ group_table: the run table on a device),
               adamw_shard_grouped
  placement    Arena (sbp_arena_create / _info / _free): device arrays whose
               physical pages are spread over the whole device memory
"""

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsbp.so")

SBP_OK, SBP_EINVAL, SBP_EALIGN, SBP_ERANGE, SBP_EHIP, SBP_ENOMEM = 0, -1, -2, -3, -4, -5
SBP_MAX_PEERS = 16
MAX_SHARD_NUMEL = (2 ** 24 - 1) * 2048  # SBP_MAX_SHARD_NUMEL: n of one step call
ORDER_REVERSE, ORDER_FORWARD, SPLIT_TENSORS = 0, 1, 2

# every function include/sbp.h declares
EXPORTS = (
    "sbp_last_error", "sbp_version", "sbp_bucket_plan", "sbp_plan_free",
    "sbp_plan_num_tensors", "sbp_plan_num_buckets", "sbp_plan_world_n",
    "sbp_plan_shard_numel", "sbp_plan_flat_numel", "sbp_plan_tensor", "sbp_plan_bucket",
    "sbp_plan_bucket_tensors", "sbp_plan_state_bytes", "sbp_mean_scale", "sbp_tokens_scale",
    "sbp_pack_grads", "sbp_reduce_shard", "sbp_accumulate_grads", "sbp_adamw_shard",
    "sbp_grad_sq_norm_workspace", "sbp_grad_sq_norm", "sbp_clip_scale",
    "sbp_unpack_params", "sbp_shard_of", "sbp_gather_shards", "sbp_bucket_plan_per_tensor",
    "sbp_group_runs", "sbp_adamw_shard_grouped", "sbp_unpack_shards",
    "sbp_grad_sq_norm_noalloc", "sbp_arena_create", "sbp_arena_info", "sbp_arena_free",
)

MAX_GROUPS = 8
NOALLOC_SCRATCH_DOUBLES = 1 << 20  # SBP_NOALLOC_SCRATCH_DOUBLES
NOALLOC_MAX_NUMEL = 2146435079  # SBP_NOALLOC_MAX_NUMEL
ARENA_MAX_ARRAYS = 64  # SBP_ARENA_MAX_ARRAYS


class SbpError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"sbp status {status}: {message}")
        self.status = status


class AdamWHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("step", ctypes.c_int64)]

    @classmethod
    def of(cls, hp, step, what):
        """The C struct of an AdamW and a step; a step outside int64 would
        wrap silently in ctypes, so it is refused here (the library checks
        step >= 1 itself)."""
        step = int(step)
        if not -(1 << 63) <= step < (1 << 63):
            raise ValueError(f"{what}: step {step} does not fit int64")
        return cls(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, step)


class GroupHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("weight_decay", ctypes.c_float)]


_lib = None
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_vpp = ctypes.POINTER(ctypes.c_void_p)


def lib():
    """The loaded C library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int32
    sig = {
        "sbp_last_error": ([], ctypes.c_char_p),
        "sbp_version": ([], ctypes.c_char_p),
        "sbp_bucket_plan": ([_i64p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                             ctypes.c_int32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_void_p)], st),
        "sbp_plan_free": ([ctypes.c_void_p], None),
        "sbp_plan_num_tensors": ([ctypes.c_void_p], ctypes.c_int32),
        "sbp_plan_num_buckets": ([ctypes.c_void_p], ctypes.c_int32),
        "sbp_plan_world_n": ([ctypes.c_void_p], ctypes.c_int32),
        "sbp_plan_shard_numel": ([ctypes.c_void_p], ctypes.c_int64),
        "sbp_plan_flat_numel": ([ctypes.c_void_p], ctypes.c_int64),
        "sbp_plan_tensor": ([ctypes.c_void_p, ctypes.c_int32, _i32p, _i64p], st),
        "sbp_plan_bucket": ([ctypes.c_void_p, ctypes.c_int32] + [_i64p] * 5, st),
        "sbp_plan_bucket_tensors": ([ctypes.c_void_p, ctypes.c_int32, _i32p, ctypes.c_int32,
                                     _i32p], st),
        "sbp_plan_state_bytes": ([ctypes.c_void_p, ctypes.c_int32, _i64p], st),
        "sbp_mean_scale": ([ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_float)], st),
        "sbp_tokens_scale": ([_i64p, ctypes.c_int32, ctypes.POINTER(ctypes.c_float)], st),
        "sbp_pack_grads": ([ctypes.c_void_p, ctypes.c_int32, _vpp, ctypes.c_void_p,
                            ctypes.c_void_p], st),
        "sbp_reduce_shard": ([_vpp, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_void_p, ctypes.c_void_p], st),
        "sbp_accumulate_grads": ([ctypes.c_void_p, _vpp, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_void_p], st),
        "sbp_adamw_shard": ([_vpp, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_int64, ctypes.POINTER(AdamWHParams), ctypes.c_void_p], st),
        "sbp_grad_sq_norm_workspace": ([ctypes.c_int64], ctypes.c_int64),
        "sbp_grad_sq_norm": ([_vpp, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                              ctypes.c_void_p, ctypes.c_void_p], st),
        "sbp_grad_sq_norm_noalloc": ([_vpp, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p], st),
        "sbp_arena_create": ([_i64p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                              ctypes.c_uint64, _vpp, ctypes.POINTER(ctypes.c_void_p)], st),
        "sbp_arena_info": ([ctypes.c_void_p, _i64p, _i64p, _i64p], st),
        "sbp_arena_free": ([ctypes.c_void_p], st),
        "sbp_clip_scale": ([ctypes.c_double, ctypes.c_float, ctypes.c_float,
                            ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)], st),
        "sbp_bucket_plan_per_tensor": ([_i64p, _i64p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_uint32,
                                        ctypes.POINTER(ctypes.c_void_p)], st),
        "sbp_unpack_params": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, _vpp,
                               ctypes.c_void_p], st),
        "sbp_shard_of": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_void_p], st),
        "sbp_gather_shards": ([ctypes.c_void_p, ctypes.c_int32, _vpp, ctypes.c_void_p,
                               ctypes.c_void_p], st),
        "sbp_unpack_shards": ([ctypes.c_void_p, ctypes.c_int32, _vpp, _vpp, ctypes.c_void_p], st),
        "sbp_group_runs": ([ctypes.c_void_p, ctypes.c_int32, _i32p, _i64p, _i32p,
                            ctypes.c_int64, _i64p], st),
        "sbp_adamw_shard_grouped": ([_vpp, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.POINTER(AdamWHParams),
                                     ctypes.POINTER(GroupHParams), ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p], st),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(status):
    if status != SBP_OK:
        raise SbpError(status, lib().sbp_last_error().decode())


def version():
    return lib().sbp_version().decode()


# ---- plan ------------------------------------------------------------------

class Plan:
    """An immutable bucket plan (owns the C handle)."""

    def __init__(self, handle, numels):
        self._h = ctypes.c_void_p(handle)
        self.numels = [int(x) for x in numels]
        self._sizes = None  # (num_tensors, flat_numel, shard_numel), read once
        self._members = {}  # bucket -> tensor ids with an element in it

    def _cached_sizes(self):
        if self._sizes is None:
            L = lib()
            self._sizes = (L.sbp_plan_num_tensors(self._h), L.sbp_plan_flat_numel(self._h),
                           L.sbp_plan_shard_numel(self._h))
        return self._sizes

    def _tensors_of(self, bucket):
        """Tensor ids a call on `bucket` reads (every tensor for bucket -1)."""
        if bucket < 0:
            return range(len(self.numels))
        ids = self._members.get(bucket)
        if ids is None:
            ids = self._members[bucket] = self.bucket_tensors(bucket)
        return ids

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None and self._h.value:
            _lib.sbp_plan_free(self._h)
            self._h = ctypes.c_void_p(None)

    @property
    def handle(self):
        return self._h

    @property
    def num_tensors(self):
        return lib().sbp_plan_num_tensors(self._h)

    @property
    def num_buckets(self):
        return lib().sbp_plan_num_buckets(self._h)

    @property
    def world_n(self):
        return lib().sbp_plan_world_n(self._h)

    @property
    def shard_numel(self):
        return lib().sbp_plan_shard_numel(self._h)

    @property
    def flat_numel(self):
        return lib().sbp_plan_flat_numel(self._h)

    def tensor(self, t):
        b, o = ctypes.c_int32(), ctypes.c_int64()
        _check(lib().sbp_plan_tensor(self._h, t, ctypes.byref(b), ctypes.byref(o)))
        return b.value, o.value

    def bucket(self, b):
        vals = [ctypes.c_int64() for _ in range(5)]
        _check(lib().sbp_plan_bucket(self._h, b, *[ctypes.byref(v) for v in vals]))
        return dict(zip(("used", "padded", "chunk", "shard_offset", "flat_offset"),
                        (v.value for v in vals)))

    def bucket_tensors(self, b):
        cnt = ctypes.c_int32()
        _check(lib().sbp_plan_bucket_tensors(self._h, b, None, 0, ctypes.byref(cnt)))
        ids = (ctypes.c_int32 * max(cnt.value, 1))()
        _check(lib().sbp_plan_bucket_tensors(self._h, b, ids, cnt.value, ctypes.byref(cnt)))
        return list(ids[:cnt.value])

    def state_bytes(self, zero_stage):
        out = ctypes.c_int64()
        _check(lib().sbp_plan_state_bytes(self._h, zero_stage, ctypes.byref(out)))
        return out.value


def bucket_plan(numels, bucket_cap_bytes, world_n, align=8, order="reverse", split=False):
    """sbp_bucket_plan: flat-bucket layout of a parameter list (host only).

    split=True: fixed-size buckets with tensors split across them."""
    arr = (ctypes.c_int64 * max(len(numels), 1))(*[int(x) for x in numels])
    h = ctypes.c_void_p()
    flags = ORDER_REVERSE if order == "reverse" else ORDER_FORWARD
    if order not in ("reverse", "forward"):
        flags = 0xFF  # rejected by the library
    if split:
        flags |= SPLIT_TENSORS
    _check(lib().sbp_bucket_plan(arr, len(numels), int(bucket_cap_bytes), int(world_n),
                                 int(align), flags, ctypes.byref(h)))
    return Plan(h.value, numels)


def bucket_plan_per_tensor(numels, world_n, rows=None, align=8, order="reverse"):
    """sbp_bucket_plan_per_tensor: one bucket per tensor, dim-0 row shards."""
    arr = (ctypes.c_int64 * max(len(numels), 1))(*[int(x) for x in numels])
    rarr = None
    if rows is not None:
        if len(rows) != len(numels):
            raise ValueError("bucket_plan_per_tensor: one row size per tensor")
        rarr = (ctypes.c_int64 * max(len(rows), 1))(*[int(r) for r in rows])
    flags = ORDER_REVERSE if order == "reverse" else ORDER_FORWARD
    if order not in ("reverse", "forward"):
        flags = 0xFF
    h = ctypes.c_void_p()
    _check(lib().sbp_bucket_plan_per_tensor(arr, rarr, len(numels), int(world_n), int(align),
                                            flags, ctypes.byref(h)))
    return Plan(h.value, numels)


def mean_scale(R, K=1):
    out = ctypes.c_float()
    _check(lib().sbp_mean_scale(int(R), int(K), ctypes.byref(out)))
    return out.value


def tokens_scale(counts):
    arr = (ctypes.c_int64 * max(len(counts), 1))(*[int(c) for c in counts])
    out = ctypes.c_float()
    _check(lib().sbp_tokens_scale(arr, len(counts), ctypes.byref(out)))
    return out.value


# ---- device calls ------------------------------------------------------------

def _stream(stream, tensor):
    """The HIP stream of a call: the given one, else the current stream of the
    current device.  The library launches on the current HIP device, so the
    call's tensors must live there."""
    import torch
    if tensor.device.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {tensor.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}; select it with torch.cuda.device")
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream(tensor.device).cuda_stream)


def _dev(t, itemsize, what):
    if not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")
    if t.element_size() != itemsize:
        raise ValueError(f"{what}: expected {itemsize}-byte elements, got {t.dtype}")
    return t.data_ptr()


def _f32(t, what):
    import torch
    if t.dtype != torch.float32:
        raise ValueError(f"{what}: expected float32, got {t.dtype}")
    return _dev(t, 4, what)


def _ptrs(tensors, what):
    return (ctypes.c_void_p * max(len(tensors), 1))(*[_dev(t, 2, what) for t in tensors])


class TensorSet:
    """One 2-byte device tensor per plan tensor, marshalled once.

    Gradient and parameter buffers usually live for the whole run: building
    their pointer array once takes the per-call work (a size check and a
    data pointer per tensor) out of pack_grads, unpack_params and
    unpack_shards, which accept a TensorSet wherever they take a list.  The
    set holds references to its tensors.  None entries stay null and may only
    stand for tensors outside the buckets a call selects."""

    def __init__(self, plan, tensors):
        T, _, _ = plan._cached_sizes()
        if len(tensors) != T:
            raise ValueError("TensorSet: one tensor per plan tensor")
        self.plan = plan
        self.tensors = list(tensors)
        self.array = (ctypes.c_void_p * max(T, 1))()
        for t, x in enumerate(self.tensors):
            if x is None:
                continue
            if x.numel() != plan.numels[t]:
                raise ValueError(f"TensorSet: tensor {t} has {x.numel()} elements")
            if x.numel():
                self.array[t] = _dev(x, 2, "TensorSet")


def _tensor_array(plan, tensors, bucket, what):
    """Host array of per-tensor device pointers for a layout call on `bucket`:
    a TensorSet's own array, or one marshalled from a list (only the tensors
    the call touches are read; None allowed for the others)."""
    if isinstance(tensors, TensorSet):
        if tensors.plan is not plan:
            raise ValueError(f"{what}: the TensorSet was built for another plan")
        return tensors.array
    T, _, _ = plan._cached_sizes()
    if len(tensors) != T:
        raise ValueError(f"{what}: one tensor per plan tensor")
    arr = (ctypes.c_void_p * max(T, 1))()
    for t in plan._tensors_of(int(bucket)):
        x = tensors[t]
        if x is None:
            continue
        if x.numel() != plan.numels[t]:
            raise ValueError(f"{what}: tensor {t} has {x.numel()} elements")
        if x.numel():
            arr[t] = _dev(x, 2, what)
    return arr


def pack_grads(plan, grads, flat, bucket=-1, stream=None):
    """sbp_pack_grads: copy per-tensor bf16 grads into the flat buckets (+0 elsewhere).

    grads: one 2-byte device tensor per plan tensor (None allowed for tensors
    outside the selected bucket), or a TensorSet; flat: 2-byte device tensor
    of plan.flat_numel.
    """
    _, F, _ = plan._cached_sizes()
    if flat.numel() != F:
        raise ValueError("pack_grads: flat has the wrong size")
    if bucket >= plan.num_buckets:
        raise SbpError(SBP_EINVAL, "pack_grads: bucket out of range")
    arr = _tensor_array(plan, grads, bucket, "pack_grads grads")
    _check(lib().sbp_pack_grads(plan.handle, int(bucket), arr, _dev(flat, 2, "pack_grads flat"),
                                _stream(stream, flat)))


def reduce_shard(peers, scale, out, stream=None):
    """sbp_reduce_shard: out = (ascending fp32 sum of the bf16 peers) * scale."""
    n = out.numel()
    if any(p.numel() != n for p in peers):
        raise ValueError("reduce_shard: peers and out differ in size")
    _check(lib().sbp_reduce_shard(_ptrs(peers, "reduce_shard peers"), len(peers), n,
                                  float(scale), _f32(out, "reduce_shard out"),
                                  _stream(stream, out)))


def accumulate_grads(acc, peers, first, stream=None):
    """sbp_accumulate_grads: acc = S (first) or acc + S."""
    n = acc.numel()
    if any(p.numel() != n for p in peers):
        raise ValueError("accumulate_grads: peers and acc differ in size")
    _check(lib().sbp_accumulate_grads(_f32(acc, "accumulate_grads acc"),
                                      _ptrs(peers, "accumulate_grads peers"), len(peers), n,
                                      1 if first else 0, _stream(stream, acc)))


@dataclass
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


def adamw_shard(peers, acc, scale, master, m, v, param_out, hp, step, stream=None):
    """sbp_adamw_shard: fused reduce (+acc) -> *scale -> AdamW -> bf16 emit."""
    n = master.numel()
    for t, what in ((m, "m"), (v, "v"), (param_out, "param_out")):
        if t.numel() != n:
            raise ValueError(f"adamw_shard: {what} has the wrong size")
    if any(p.numel() != n for p in peers) or (acc is not None and acc.numel() != n):
        raise ValueError("adamw_shard: peers/acc differ in size")
    h = AdamWHParams.of(hp, step, "adamw_shard")
    _check(lib().sbp_adamw_shard(
        _ptrs(peers, "adamw_shard peers"), len(peers),
        None if acc is None else _f32(acc, "adamw_shard acc"), float(scale),
        _f32(master, "adamw_shard master"), _f32(m, "adamw_shard m"), _f32(v, "adamw_shard v"),
        _dev(param_out, 2, "adamw_shard param_out"), n, ctypes.byref(h),
        _stream(stream, master)))


class ShardStep:
    """sbp_adamw_shard with its buffers marshalled once.

    A training loop steps the same shard buffers every iteration.  Building
    the peer pointer array, checking sizes and dtypes and looking up the
    stream once leaves each call with the hyperparameter struct and the C
    call, which is what a small shard's step rate is bound by.  The launch
    stream is the one given, else the current stream at construction.  The
    object holds references to its tensors.

        step = sbp.ShardStep(peers, acc, master, m, v, param_out)
        step(scale, hp, t)   # = adamw_shard(peers, acc, scale, ..., hp, t)
    """

    def __init__(self, peers, acc, master, m, v, param_out, stream=None):
        n = master.numel()
        for t, what in ((m, "m"), (v, "v"), (param_out, "param_out")):
            if t.numel() != n:
                raise ValueError(f"ShardStep: {what} has the wrong size")
        if any(p.numel() != n for p in peers) or (acc is not None and acc.numel() != n):
            raise ValueError("ShardStep: peers/acc differ in size")
        self.tensors = (list(peers), acc, master, m, v, param_out)
        self.n = n
        self.R = len(peers)
        self._args = (_ptrs(peers, "ShardStep peers"), self.R,
                      None if acc is None else _f32(acc, "ShardStep acc"))
        self._state = (_f32(master, "ShardStep master"), _f32(m, "ShardStep m"),
                       _f32(v, "ShardStep v"), _dev(param_out, 2, "ShardStep param_out"), n)
        self._stream = _stream(stream, master)

    def __call__(self, scale, hp, step):
        h = AdamWHParams.of(hp, step, "ShardStep")
        peers, R, acc = self._args
        _check(lib().sbp_adamw_shard(peers, R, acc, float(scale), *self._state, ctypes.byref(h),
                                     self._stream))


def group_runs(plan, rank, tensor_group):
    """sbp_group_runs: rank's shard as runs of one parameter group.

    tensor_group: a group id (0..7) per plan tensor.  Returns numpy arrays
    (run_start int64, run_group int32); run_start[0] == 0.
    """
    import numpy as np
    g = np.ascontiguousarray(tensor_group, dtype=np.int32)
    if g.shape != (plan.num_tensors,):
        raise ValueError("group_runs: one group id per plan tensor")
    gp = g.ctypes.data_as(_i32p)
    count = ctypes.c_int64()
    _check(lib().sbp_group_runs(plan.handle, int(rank), gp, None, None, 0, ctypes.byref(count)))
    starts = np.zeros(count.value, dtype=np.int64)
    groups = np.zeros(count.value, dtype=np.int32)
    _check(lib().sbp_group_runs(plan.handle, int(rank), gp, starts.ctypes.data_as(_i64p),
                                groups.ctypes.data_as(_i32p), count.value, ctypes.byref(count)))
    return starts, groups


def group_table(plan, rank, tensor_group, device):
    """group_runs() copied to `device`: (run_start, run_group) device tensors."""
    import torch
    starts, groups = group_runs(plan, rank, tensor_group)
    return (torch.from_numpy(starts).to(device), torch.from_numpy(groups).to(device))


def adamw_shard_grouped(peers, acc, scale, master, m, v, param_out, hp, step, groups,
                        run_start, run_group, stream=None):
    """sbp_adamw_shard_grouped: adamw_shard() with per-group lr and weight decay.

    groups: list of (lr, weight_decay), at most MAX_GROUPS; run_start/run_group:
    the rank's run table as device tensors (int64, int32; see group_table).
    hp supplies beta1, beta2 and eps.
    """
    import torch
    n = master.numel()
    for t, what in ((m, "m"), (v, "v"), (param_out, "param_out")):
        if t.numel() != n:
            raise ValueError(f"adamw_shard_grouped: {what} has the wrong size")
    if any(p.numel() != n for p in peers) or (acc is not None and acc.numel() != n):
        raise ValueError("adamw_shard_grouped: peers/acc differ in size")
    if run_start.dtype != torch.int64 or run_group.dtype != torch.int32:
        raise ValueError("adamw_shard_grouped: run_start must be int64, run_group int32")
    if run_start.numel() != run_group.numel():
        raise ValueError("adamw_shard_grouped: run tables differ in length")
    if not 1 <= len(groups) <= MAX_GROUPS:
        raise ValueError(f"adamw_shard_grouped: 1..{MAX_GROUPS} groups")
    h = AdamWHParams.of(hp, step, "adamw_shard_grouped")
    gs = (GroupHParams * len(groups))(*[GroupHParams(lr, wd) for lr, wd in groups])
    _check(lib().sbp_adamw_shard_grouped(
        _ptrs(peers, "adamw_shard_grouped peers"), len(peers),
        None if acc is None else _f32(acc, "adamw_shard_grouped acc"), float(scale),
        _f32(master, "adamw_shard_grouped master"), _f32(m, "adamw_shard_grouped m"),
        _f32(v, "adamw_shard_grouped v"), _dev(param_out, 2, "adamw_shard_grouped param_out"), n,
        ctypes.byref(h), gs, len(groups), _dev(run_start, 8, "adamw_shard_grouped run_start"),
        _dev(run_group, 4, "adamw_shard_grouped run_group"), run_start.numel(),
        _stream(stream, master)))


def grad_sq_norm_workspace(n):
    """Doubles of workspace sbp_grad_sq_norm needs for n elements."""
    return int(lib().sbp_grad_sq_norm_workspace(int(n)))


def grad_sq_norm(peers, acc, scale, n, g_sum_out=None, workspace=None, sq_out=None,
                 stream=None):
    """sbp_grad_sq_norm: this rank's squared norm of g = fl(G*scale) (float64).

    Returns the device tensor holding it (float64[1]); workspace and sq_out are
    allocated with torch when not given.  With g_sum_out, G is written too.
    """
    import torch
    ref = peers[0] if peers else acc
    if ref is None:
        raise ValueError("grad_sq_norm: needs peers or an accumulator")
    dev = ref.device
    if any(p.numel() != n for p in peers) or (acc is not None and acc.numel() != n):
        raise ValueError("grad_sq_norm: peers/acc differ in size")
    if g_sum_out is not None and g_sum_out.numel() != n:
        raise ValueError("grad_sq_norm: g_sum_out has the wrong size")
    if workspace is None:
        workspace = torch.empty(grad_sq_norm_workspace(n), dtype=torch.float64, device=dev)
    if sq_out is None:
        sq_out = torch.empty(1, dtype=torch.float64, device=dev)
    for t, what in ((workspace, "workspace"), (sq_out, "sq_out")):
        if t.dtype != torch.float64 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"grad_sq_norm: {what} must be a contiguous float64 device tensor")
    _check(lib().sbp_grad_sq_norm(
        _ptrs(peers, "grad_sq_norm peers"), len(peers),
        None if acc is None else _f32(acc, "grad_sq_norm acc"), float(scale), int(n),
        None if g_sum_out is None else _f32(g_sum_out, "grad_sq_norm g_sum_out"),
        workspace.data_ptr(), workspace.numel(), sq_out.data_ptr(), _stream(stream, ref)))
    return sq_out


def grad_sq_norm_noalloc(peers, acc, scale, n, sq_out, g_sum_out=None, stream=None):
    """sbp_grad_sq_norm_noalloc: grad_sq_norm with the library's static
    per-GPU scratch as the workspace (n <= NOALLOC_MAX_NUMEL).  The caller
    passes every output, sq_out included: nothing is allocated here either.
    Calls that overlap on one GPU share the scratch and race."""
    import torch
    ref = peers[0] if peers else acc
    if ref is None:
        raise ValueError("grad_sq_norm_noalloc: needs peers or an accumulator")
    if any(p.numel() != n for p in peers) or (acc is not None and acc.numel() != n):
        raise ValueError("grad_sq_norm_noalloc: peers/acc differ in size")
    if g_sum_out is not None and g_sum_out.numel() != n:
        raise ValueError("grad_sq_norm_noalloc: g_sum_out has the wrong size")
    if sq_out.dtype != torch.float64 or not sq_out.is_cuda or not sq_out.is_contiguous():
        raise ValueError("grad_sq_norm_noalloc: sq_out must be a contiguous float64 device "
                         "tensor")
    _check(lib().sbp_grad_sq_norm_noalloc(
        _ptrs(peers, "grad_sq_norm_noalloc peers"), len(peers),
        None if acc is None else _f32(acc, "grad_sq_norm_noalloc acc"), float(scale), int(n),
        None if g_sum_out is None else _f32(g_sum_out, "grad_sq_norm_noalloc g_sum_out"),
        sq_out.data_ptr(), _stream(stream, ref)))
    return sq_out


def clip_scale(total_sq, max_norm, scale):
    """sbp_clip_scale: (fl32(scale * coef), coef), coef = min(1, max/(||g||+1e-6))."""
    out = ctypes.c_float()
    coef = ctypes.c_double()
    _check(lib().sbp_clip_scale(float(total_sq), float(max_norm), float(scale),
                                ctypes.byref(out), ctypes.byref(coef)))
    return out.value, coef.value


def unpack_params(plan, flat, params, bucket=-1, stream=None):
    """sbp_unpack_params: flat bf16 buckets -> per-tensor bf16 parameters.

    params: one 2-byte device tensor per plan tensor (None allowed outside the
    selected bucket), or a TensorSet."""
    _, F, _ = plan._cached_sizes()
    if flat.numel() != F:
        raise ValueError("unpack_params: flat has the wrong size")
    if bucket >= plan.num_buckets:
        raise SbpError(SBP_EINVAL, "unpack_params: bucket out of range")
    arr = _tensor_array(plan, params, bucket, "unpack_params params")
    _check(lib().sbp_unpack_params(plan.handle, int(bucket), _dev(flat, 2, "unpack_params flat"),
                                   arr, _stream(stream, flat)))


def shard_of(plan, rank, flat, shard, bucket=-1, stream=None):
    """sbp_shard_of: rank's chunk of every bucket of `flat` -> shard layout."""
    if flat.numel() != plan.flat_numel or shard.numel() != plan.shard_numel:
        raise ValueError("shard_of: flat or shard has the wrong size")
    _check(lib().sbp_shard_of(plan.handle, int(bucket), int(rank), _dev(flat, 2, "shard_of flat"),
                              _dev(shard, 2, "shard_of shard"), _stream(stream, flat)))


def gather_shards(plan, shards, flat, bucket=-1, stream=None):
    """sbp_gather_shards: the N ranks' shards -> flat bucket layout (all-gather layout)."""
    if len(shards) != plan.world_n:
        raise ValueError("gather_shards: one shard per rank")
    if flat.numel() != plan.flat_numel or any(s.numel() != plan.shard_numel for s in shards):
        raise ValueError("gather_shards: flat or a shard has the wrong size")
    _check(lib().sbp_gather_shards(plan.handle, int(bucket), _ptrs(shards, "gather_shards shards"),
                                   _dev(flat, 2, "gather_shards flat"), _stream(stream, flat)))


def unpack_shards(plan, shards, params, bucket=-1, stream=None):
    """sbp_unpack_shards: the N ranks' shards -> per-tensor bf16 parameters in
    one pass (gather_shards followed by unpack_params, without the flat buffer).

    params: one 2-byte device tensor per plan tensor (None allowed outside the
    selected bucket), or a TensorSet."""
    if len(shards) != plan.world_n:
        raise ValueError("unpack_shards: one shard per rank")
    if any(x.numel() != plan.shard_numel for x in shards):
        raise ValueError("unpack_shards: a shard has the wrong size")
    if bucket >= plan.num_buckets:
        raise SbpError(SBP_EINVAL, "unpack_shards: bucket out of range")
    arr = _tensor_array(plan, params, bucket, "unpack_shards params")
    _check(lib().sbp_unpack_shards(plan.handle, int(bucket), _ptrs(shards, "unpack_shards shards"),
                                   arr, _stream(stream, shards[0])))


# ---- spread arena ---------------------------------------------------------------

_TYPESTR = {"float32": "<f4", "float64": "<f8", "int16": "<i2", "int32": "<i4", "int64": "<i8",
            "uint8": "|u1", "bfloat16": "<i2"}


class _DeviceView:
    """A __cuda_array_interface__ view of arena memory; it holds the arena,
    and torch holds it for as long as a tensor made from it lives."""

    def __init__(self, arena, ptr, numel, typestr):
        self._arena = arena
        self.__cuda_array_interface__ = {"shape": (int(numel),), "typestr": typestr,
                                         "data": (int(ptr), False), "version": 3,
                                         "strides": None}


class Arena:
    """sbp_arena_create: device arrays of the given byte sizes whose physical
    chunks are spread evenly over the device memory (chunk 0 = 64 MiB,
    spread 0 = all free memory less a reserve).  tensor(i, dtype, numel)
    returns a torch tensor aliasing array i; the arena stays allocated while
    any such tensor (or this object) is alive, and is freed after the last
    (sbp_arena_free synchronises the device first)."""

    def __init__(self, nbytes, chunk=0, spread=0, seed=0x5EED):
        nbytes = [int(b) for b in nbytes]
        k = len(nbytes)
        arr = (ctypes.c_int64 * max(k, 1))(*nbytes)
        ptrs = (ctypes.c_void_p * max(k, 1))()
        h = ctypes.c_void_p()
        _check(lib().sbp_arena_create(arr, k, int(chunk), int(spread), int(seed) & (2**64 - 1),
                                      ptrs, ctypes.byref(h)))
        self._h = h
        self.nbytes = nbytes
        self.ptrs = [ptrs[i] or 0 for i in range(k)]

    def info(self):
        c, kept, spread = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().sbp_arena_info(self._h, ctypes.byref(c), ctypes.byref(kept),
                                    ctypes.byref(spread)))
        return {"chunk_bytes": c.value, "chunks_kept": kept.value, "chunks_spread": spread.value}

    def tensor(self, i, dtype, numel=None):
        import torch
        name = str(dtype).replace("torch.", "")
        item = torch.empty(0, dtype=dtype).element_size()
        if numel is None:
            numel = self.nbytes[i] // item
        if numel * item > self.nbytes[i]:
            raise ValueError(f"Arena.tensor: {numel} x {item} bytes exceed array {i}")
        if name not in _TYPESTR:
            raise ValueError(f"Arena.tensor: unsupported dtype {dtype}")
        t = torch.as_tensor(_DeviceView(self, self.ptrs[i], numel, _TYPESTR[name]),
                            device=torch.device("cuda", torch.cuda.current_device()))
        return t.view(dtype) if name == "bfloat16" else t

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.sbp_arena_free(h)
            self._h = None
