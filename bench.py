#!/usr/bin/env python3
"""Benchmark of the one-rank shard step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line on stdout (diagnostics go to stderr).  A step is one
pass of the workload's whole per-step path over inputs already resident in
HBM:
  llama3_8b     (default) Llama-3-8B-shaped ZeRO-3 shard, N=8, R=8,
                n = 1,003,782,656: one fused reduce + 1/R + AdamW + bf16
                emit launch over the shard (the plan is made once, before)
  gpt2_small    GPT-2-small ZeRO-2 shard, N=8, R=8 (two buffer sets rotate so
                the working set exceeds the 256 MB last-level cache twice over)
  tiny_mlp      2-layer MLP shard, R=2 (cache-resident; many rotating sets)
  gpt_7b5       "7.5B" GPT shard, N=64, R=8, 4 microbatches: 3 accumulate
                launches + the fused step with acc, 1/C token scaling
  llama3_8b_dp  Llama-3-8B full DP replica (N=1, R=2): pack of 291 tensors
                into 162 buckets + the fused step over 8.03B elements
value = shard elements updated per second (whole job = the one GPU).

The roofline object is for the fused kernel: algorithmic bytes per launch
((26 + 2R) bytes per element, +4 with an fp32 accumulator) over its average
launch time, measured with HIP events on the stream it is launched on.
HBM traffic comes from a committed rocprofv3 counter summary when that
summary was taken on the current kernel source, else null.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("params updated/sec and HBM GB/s (% of 8 TB/s roofline), fused shard step")
PEAK_GBS = 8000.0  # MI355X HBM3E
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fused_adamw_llama3_8b_pmc.json")
KERNEL_SRC = os.path.join(ROOT, "sharded_bucket_plan_amd", "csrc", "shard_step.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    with open(KERNEL_SRC, "rb") as f:
        h.update(f.read())
    from sharded_bucket_plan_amd.build import FLAGS
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def fused_bytes_per_elem(R, acc):
    return 2 * R + 12 + 12 + 2 + (4 if acc else 0)


class Workload:
    """Device buffers and the per-step launches of one workload."""

    def __init__(self, name, seed):
        import torch
        import sharded_bucket_plan_amd as sbp
        import synth

        self.sbp, self.synth, self.torch = sbp, synth, torch
        self.name = name
        self.w = w = synth.WORKLOADS[name]
        self.seed = seed
        self.dev = torch.device("cuda:0")
        self.hp = sbp.AdamW(w.adamw.lr, w.adamw.beta1, w.adamw.beta2, w.adamw.eps,
                            w.adamw.weight_decay)
        self.plan = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)
        self.n = self.plan.shard_numel
        self.acc = w.K > 1
        self.bytes_fused = fused_bytes_per_elem(w.R, self.acc) * self.n
        mall = 256 << 20
        set_bytes = self.bytes_fused
        self.nsets = 1 if set_bytes >= 4 * mall else max(2, -(-4 * mall // set_bytes))
        self.sets = [self._alloc_set(i) for i in range(self.nsets)]
        self.i = 0
        torch.cuda.synchronize()

    def _u16(self, n):
        return self.torch.empty(n, dtype=self.torch.int16, device=self.dev)

    def _f32(self, n):
        return self.torch.empty(n, dtype=self.torch.float32, device=self.dev)

    def _alloc_set(self, i):
        w, n, synth = self.w, self.n, self.synth
        s = {}
        s["master"] = synth.dev_normal_f32(self._f32(n), self.seed + i, synth.master_stream(0),
                                           w.master_sigma)
        s["m"] = self._f32(n).zero_()
        s["v"] = self._f32(n).zero_()
        s["p"] = self._u16(n)
        if w.pack:
            # rank 0 packs its per-tensor gradients; rank 1's contribution is
            # already in bucket layout (N = 1: bucket layout = shard layout)
            s["grads"] = [synth.dev_normal_bf16(self._u16(k), self.seed + i,
                                                synth.tensor_stream(1, 0, 0, t), w.grad_sigma)
                          for t, k in enumerate(w.numels)]
            s["flat0"] = self._u16(n)
            s["peers"] = [s["flat0"]] + [
                synth.dev_normal_bf16(self._u16(n), self.seed + i, synth.peer_stream(1, 0, r),
                                      w.grad_sigma) for r in range(1, w.R)]
        else:
            nmb = w.K
            s["mb"] = [[synth.dev_normal_bf16(self._u16(n), self.seed + i,
                                              synth.peer_stream(1, k, r), w.grad_sigma)
                        for r in range(w.R)] for k in range(nmb)]
            s["peers"] = s["mb"][-1]
        if self.acc:
            s["acc"] = self._f32(n)
        return s

    def scale(self, t):
        w = self.w
        if w.norm == "tokens":
            return self.sbp.tokens_scale([self.synth.tokens(self.seed, t, r) for r in range(w.R)])
        return self.sbp.mean_scale(w.R, w.K)

    def step(self, t, ev=None):
        """One whole per-step path; ev = (start, end) events around the fused launch."""
        s = self.sets[self.i]
        self.i = (self.i + 1) % self.nsets
        sbp, w = self.sbp, self.w
        if w.pack:
            sbp.pack_grads(self.plan, s["grads"], s["flat0"])
        if self.acc:
            for k in range(w.K - 1):
                sbp.accumulate_grads(s["acc"], s["mb"][k], first=(k == 0))
        scale = self.scale(t)
        if ev:
            ev[0].record()
        sbp.adamw_shard(s["peers"], s.get("acc"), scale, s["master"], s["m"], s["v"], s["p"],
                        self.hp, t)
        if ev:
            ev[1].record()

    def config(self):
        w = self.w
        return {"workload": self.name, "params": w.psi, "shard_numel": self.n, "R": w.R,
                "N": w.world_n, "K": w.K, "norm": w.norm,
                "bucket_cap_MiB": w.bucket_cap_bytes >> 20, "buckets": self.plan.num_buckets,
                "pack": w.pack, "rotating_buffer_sets": self.nsets,
                "fused_bytes_per_elem": fused_bytes_per_elem(w.R, self.acc)}


def traffic_from_profile(nbytes_per_launch):
    """HBM bytes per fused launch from the committed counter summary, if it was
    taken on the current kernel source and the same workload size."""
    try:
        with open(PMC_SUMMARY) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != kernel_source_hash():
        return None
    if d.get("algorithmic_bytes_per_launch") != nbytes_per_launch:
        return None
    return d.get("traffic_bytes_per_launch")


def cpu_baseline(workload_name, seed, target_s):
    """The oracle as it stands, on a bounded contiguous sample of the same
    workload's shard (inputs generated on the host), single-threaded numpy."""
    import numpy as np
    import synth
    from oracle import step as OS

    w = synth.WORKLOADS[workload_name]
    hp = w.adamw
    chunk = 1 << 22
    done = 0
    spent = 0.0
    i0 = 0
    while spent < target_s:
        peers = [synth.normal_bf16(seed, synth.peer_stream(1, 0, r), chunk, w.grad_sigma, i0)
                 for r in range(w.R)]
        th = synth.normal_f32(seed, synth.master_stream(0), chunk, w.master_sigma, i0)
        z = np.zeros(chunk, np.float32)
        acc = OS.reduce_peers(peers) if w.K > 1 else None
        scale = OS.mean_scale(w.R, w.K)
        t0 = time.perf_counter()
        OS.shard_step(peers, acc, scale, th, z, z, hp, 1)
        spent += time.perf_counter() - t0
        done += chunk
        i0 += chunk
    b = fused_bytes_per_elem(w.R, w.K > 1)
    return {"value": done / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "gbs": done * b / spent / 1e9,
            "sample": (f"{done} elements ({done // chunk} contiguous slices of {chunk}) of the "
                       f"{workload_name} shard, one fused step (R={w.R}"
                       f"{', with accumulator' if w.K > 1 else ''}), numpy binary32 oracle, "
                       f"{spent:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "shard step is per rank and nothing here crosses GPUs", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth

    seed = synth.SEED if args.seed is None else args.seed
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    log(f"bench: workload {args.workload}, allocating and generating inputs on cuda:0")
    W = Workload(args.workload, seed)
    log(f"bench: n={W.n} R={W.w.R} sets={W.nsets}; warmup {args.warmup}")
    t = 0
    for _ in range(args.warmup):
        t += 1
        W.step(t)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        t += 1
        W.step(t, evs[k])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_avg = sum(kern_ms) / len(kern_ms)
    achieved = W.bytes_fused / (kern_avg * 1e-3) / 1e9
    value = W.n / (ms_per_step * 1e-3)
    log(f"bench: {ms_per_step:.4f} ms/step, fused kernel {kern_avg:.4f} ms avg "
        f"(min {min(kern_ms):.4f}), {achieved:.1f} GB/s algorithmic")

    traffic = traffic_from_profile(W.bytes_fused)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"bench: CPU baseline (~{args.cpu_seconds:.0f} s of oracle work)")
        cpu = cpu_baseline(args.workload, seed, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": W.config(),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBS, "traffic": traffic,
                     "kernel": "fused_adamw_kernel", "kernel_ms_avg": kern_avg,
                     "algorithmic_bytes_per_launch": W.bytes_fused},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
