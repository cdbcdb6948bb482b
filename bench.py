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

Variants of the step (same JSON line): --clip MAX_NORM adds global-norm
clipping (the norm pass writing G, then the update from G; with
--clip-recompute the norm pass writes nothing and the update sums the peers
again); --groups uses
two parameter groups (no weight decay on 1-D tensors) and the grouped step.
Other modes print their own JSON: --layout times pack / shard_of /
gather_shards / unpack_params / unpack_shards and the plan builds on the workload's model
(--plan whole | split | per_tensor picks the layout); --bucket-sweep times one
accumulate pass per bucket for caps of 1..256 MiB on the 7.5B shard;
--stream-mix times the library's kernels against their mix of read and
write streams on the Llama shard; --calibrate-copy and --summarize-pmc make
the HBM-counter summary.

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
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("params updated/sec and HBM GB/s (% of 8 TB/s roofline), fused shard step")
PEAK_GBS = 8000.0  # MI355X HBM3E
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fused_adamw_llama3_8b_pmc.md")
COPY_BYTES = 1 << 32  # the calibration copy moves 4 GiB in and 4 GiB out
CALIBRATION_CALLS = 4  # --calibrate-copy: one warm-up copy + 3 timed ones
KERNEL_SRC = os.path.join(ROOT, "sharded_bucket_plan_amd", "csrc", "shard_step.hip")
LAYOUT_SRC = os.path.join(ROOT, "sharded_bucket_plan_amd", "csrc", "layout.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(path=KERNEL_SRC):
    h = hashlib.sha256()
    with open(path, "rb") as f:
        h.update(f.read())
    from sharded_bucket_plan_amd.build import FLAGS
    # the flags minus absolute paths (the tree lives elsewhere on other machines)
    h.update(" ".join(f for f in FLAGS if not os.path.isabs(f)).encode())
    return h.hexdigest()


def fused_bytes_per_elem(R, acc):
    return 2 * R + 12 + 12 + 2 + (4 if acc else 0)


class Workload:
    """Device buffers and the per-step launches of one workload."""

    def __init__(self, name, seed, clip=None, groups=False, recompute=False, placement="spread"):
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
        self.clip = clip
        # clipping without G: the norm pass only reads, the update reads the peers again
        self.recompute = bool(clip) and recompute
        self.groups = None
        if groups:
            # the usual two parameter groups: decay on matrices, none on 1-D
            # tensors (biases, norm gains); run table of this rank's shard
            tg = [1 if len(shape) == 1 else 0 for _, shape in w.params]
            self.groups = [(self.hp.lr, self.hp.weight_decay), (self.hp.lr, 0.0)]
            self.runs = sbp.group_table(self.plan, w.shard_index, tg, self.dev)
        # with clipping the update reads G (fp32) written by the norm pass
        self.bytes_fused = (fused_bytes_per_elem(0, True) if clip and not self.recompute else
                            fused_bytes_per_elem(w.R, self.acc)) * self.n
        mall = 256 << 20
        set_bytes = self.bytes_fused
        self.nsets = 1 if set_bytes >= 4 * mall else max(2, -(-4 * mall // set_bytes))
        # the step's arrays in spread arenas (one per buffer set) unless the
        # sets are many small cache-resident ones, where placement is moot
        self.placement = placement if self.nsets <= 4 else "torch"
        self.arenas = []
        self.sets = [self._alloc_set(i) for i in range(self.nsets)]
        self.i = 0
        torch.cuda.synchronize()

    def _u16(self, n):
        return self.torch.empty(n, dtype=self.torch.int16, device=self.dev)

    def _f32(self, n):
        return self.torch.empty(n, dtype=self.torch.float32, device=self.dev)

    def _arrays(self):
        """(name, dtype, numel) of the step's arrays in one buffer set."""
        w, n, torch = self.w, self.n, self.torch
        a = [("master", torch.float32, n), ("m", torch.float32, n), ("v", torch.float32, n),
             ("p", torch.int16, n)]
        if w.pack:
            a += [("flat0", torch.int16, n)] + [(f"peer{r}", torch.int16, n)
                                                 for r in range(1, w.R)]
        else:
            a += [(f"mb{k}_{r}", torch.int16, n) for k in range(w.K) for r in range(w.R)]
        if self.acc:
            a.append(("acc", torch.float32, n))
        if self.clip:
            a.append(("gsum", torch.float32, n))
        return a

    def _alloc_set(self, i):
        w, n, synth = self.w, self.n, self.synth
        spec = self._arrays()
        buf = None
        if self.placement == "spread":
            try:
                ar = self.sbp.Arena([k * self.torch.empty(0, dtype=dt).element_size()
                                     for _, dt, k in spec], seed=0x5EED + i)
            except self.sbp.SbpError as e:
                # no virtual memory management, or no room to spread: the
                # line then says where its arrays really were
                if i > 0:
                    raise
                log(f"bench: spread arena unavailable ({e}); ordinary torch allocations instead")
                self.placement = "torch"
            else:
                self.arenas.append(ar)
                buf = {nm: ar.tensor(j, dt, k) for j, (nm, dt, k) in enumerate(spec)}
        if buf is None:
            buf = {nm: self.torch.empty(k, dtype=dt, device=self.dev) for nm, dt, k in spec}
        s = {}
        s["master"] = synth.dev_normal_f32(buf["master"], self.seed + i, synth.master_stream(0),
                                           w.master_sigma)
        s["m"] = buf["m"].zero_()
        s["v"] = buf["v"].zero_()
        s["p"] = buf["p"]
        if w.pack:
            # rank 0 packs its per-tensor gradients (the backward's outputs,
            # ordinary allocations); rank 1's contribution is already in
            # bucket layout (N = 1: bucket layout = shard layout)
            s["grads"] = [synth.dev_normal_bf16(self._u16(k), self.seed + i,
                                                synth.tensor_stream(1, 0, 0, t), w.grad_sigma)
                          for t, k in enumerate(w.numels)]
            s["flat0"] = buf["flat0"]
            s["peers"] = [s["flat0"]] + [
                synth.dev_normal_bf16(buf[f"peer{r}"], self.seed + i, synth.peer_stream(1, 0, r),
                                      w.grad_sigma) for r in range(1, w.R)]
        else:
            s["mb"] = [[synth.dev_normal_bf16(buf[f"mb{k}_{r}"], self.seed + i,
                                              synth.peer_stream(1, k, r), w.grad_sigma)
                        for r in range(w.R)] for k in range(w.K)]
            s["peers"] = s["mb"][-1]
        if self.acc:
            s["acc"] = buf["acc"]
        # the plain step's buffers marshalled once (the step the timed loop makes)
        s["step"] = self.sbp.ShardStep(s["peers"], s.get("acc"), s["master"], s["m"], s["v"],
                                       s["p"])
        if self.clip:
            s["gsum"] = buf["gsum"]
            s["ws"] = self.torch.empty(self.sbp.grad_sq_norm_workspace(n),
                                       dtype=self.torch.float64, device=self.dev)
            s["sq"] = self.torch.empty(1, dtype=self.torch.float64, device=self.dev)
        return s

    def scale(self, t):
        w = self.w
        if w.norm == "tokens":
            return self.sbp.tokens_scale([self.synth.tokens(self.seed, t, r) for r in range(w.R)])
        return self.sbp.mean_scale(w.R, w.K)

    def parts(self):
        """Kernel groups of one step with their algorithmic bytes."""
        w, n = self.w, self.n
        out = []
        if w.pack:
            out.append(("copy_kernel", 4 * sum(w.numels) + 2 * (self.plan.flat_numel - sum(w.numels))))
        if self.acc:
            out.append(("accumulate_kernel", (2 * w.R + 4) * n + (2 * w.R + 8) * n * (w.K - 2)))
        if self.clip:
            out.append(("sq_norm_kernel", (2 * w.R + (4 if self.acc else 0)
                                           + (0 if self.recompute else 4)) * n))
        out.append(("fused_adamw_kernel", self.bytes_fused))
        return out

    def step(self, t, ev=None):
        """One whole per-step path; ev = {part: (start, end)} events around each
        kernel group (on the stream the kernels are launched on)."""
        s = self.sets[self.i]
        self.i = (self.i + 1) % self.nsets
        sbp, w = self.sbp, self.w

        def mark(part, k):
            if ev:
                ev[part][k].record()

        if w.pack:
            mark("copy_kernel", 0)
            sbp.pack_grads(self.plan, s["grads"], s["flat0"])
            mark("copy_kernel", 1)
        if self.acc:
            mark("accumulate_kernel", 0)
            for k in range(w.K - 1):
                sbp.accumulate_grads(s["acc"], s["mb"][k], first=(k == 0))
            mark("accumulate_kernel", 1)
        scale = self.scale(t)
        if self.clip:
            # this rank's squared norm; with more ranks its all-reduce goes here
            mark("sq_norm_kernel", 0)
            sbp.grad_sq_norm(s["peers"], s.get("acc"), scale, self.n,
                             g_sum_out=None if self.recompute else s["gsum"],
                             workspace=s["ws"], sq_out=s["sq"])
            mark("sq_norm_kernel", 1)
            scale, _ = sbp.clip_scale(s["sq"].item(), self.clip, scale)
            mark("fused_adamw_kernel", 0)
            if self.recompute:
                s["step"](scale, self.hp, t)
            else:
                sbp.adamw_shard([], s["gsum"], scale, s["master"], s["m"], s["v"], s["p"],
                                self.hp, t)
            mark("fused_adamw_kernel", 1)
            return
        mark("fused_adamw_kernel", 0)
        if self.groups:
            sbp.adamw_shard_grouped(s["peers"], s.get("acc"), scale, s["master"], s["m"], s["v"],
                                    s["p"], self.hp, t, self.groups, *self.runs)
        else:
            s["step"](scale, self.hp, t)
        mark("fused_adamw_kernel", 1)

    def config(self):
        w = self.w
        return {"workload": self.name, "params": w.psi, "shard_numel": self.n, "R": w.R,
                "N": w.world_n, "K": w.K, "norm": w.norm,
                "bucket_cap_MiB": w.bucket_cap_bytes >> 20, "buckets": self.plan.num_buckets,
                "pack": w.pack, "rotating_buffer_sets": self.nsets,
                "clip_max_norm": self.clip,
                "clip_recompute": self.recompute,
                "param_groups": len(self.groups) if self.groups else 1,
                "group_runs": int(self.runs[0].numel()) if self.groups else 1,
                "fused_bytes_per_elem": self.bytes_fused // self.n,
                "placement": self.placement}

    def release(self):
        """Drops the buffer sets (and frees the arenas once nothing uses them)."""
        self.sets = []
        self.arenas = []
        import gc
        gc.collect()
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def _summary_fields(path):
    """`key: value` lines of a profile summary."""
    out = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith(("#", "|", " ")):
                k, v = ln.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def traffic_from_profile(nbytes_per_launch):
    """HBM bytes per fused launch from the committed counter summary, if it was
    taken on the current kernel source and the same workload size."""
    try:
        d = _summary_fields(PMC_SUMMARY)
    except OSError:
        return None
    if d.get("source_sha256") != kernel_source_hash():
        return None
    if d.get("algorithmic_bytes_per_launch") != str(nbytes_per_launch):
        return None
    try:
        return int(d["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_ceiling_gbs(reps=5):
    """A plain streaming copy of 4 GiB on this GPU (bytes read + written / time).

    An elementwise kernel (dst = -src) rather than copy_(), which torch hands
    to the runtime's memcpy; it is the only dispatch here, so the same call
    under rocprofv3 --pmc calibrates the byte counters."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def footprint_copy_gbs(nbytes, nsets, reps=20):
    """A plain streaming copy on the same footprint as a small workload's
    step: nbytes moved per launch (nbytes/2 read, nbytes/2 written), nsets
    rotating buffer pairs as the step rotates its sets; HIP events around
    every launch, average."""
    import torch
    half = max(4, nbytes // 2 // 4 * 4)
    pairs = [(torch.empty(half // 4, dtype=torch.float32, device="cuda:0"),
              torch.empty(half // 4, dtype=torch.float32, device="cuda:0")) for _ in range(nsets)]
    for src, dst in pairs:
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for k, (a, b) in enumerate(ev):
        src, dst = pairs[k % nsets]
        a.record()
        torch.neg(src, out=dst)
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / reps
    del pairs
    torch.cuda.empty_cache()
    return 2 * half / (ms * 1e-3) / 1e9


def _pmc_rows(d, counter):
    """(kernel name, value) of every dispatch in rocprofv3 counter CSVs under d."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    return rows


def _pmc_dispatches(d):
    """[(kernel name, {counter: value})] of every dispatch in rocprofv3 counter
    CSVs under d, in dispatch order."""
    import csv
    import glob
    by = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                k = int(r["Dispatch_Id"])
                name, ctr = by.setdefault(k, (r.get("Kernel_Name", ""), {}))
                ctr[r["Counter_Name"]] = ctr.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [by[k] for k in sorted(by)]


def summarize_sweep_pmc(pmc_dir, sweep_json, rates_json, command):
    """Markdown table of the DRAM credit stalls per launch of --placement-sweep
    --sweep-quick under rocprofv3 --pmc (the sweep's launch log names each
    dispatch), beside the rates of a plain --placement-sweep run."""
    sw = json.loads(open(sweep_json).read().strip().splitlines()[-1])
    rates = json.loads(open(rates_json).read().strip().splitlines()[-1]) if rates_json else None
    keep = ("fused_adamw_kernel", "mix_probe", "copy_probe")
    disp = [d for d in _pmc_dispatches(pmc_dir) if any(k in d[0] for k in keep)]
    log_ = [tuple(x) for x in sw["launches"]]
    if len(disp) != len(log_):
        raise SystemExit(f"{len(disp)} dispatches against {len(log_)} logged launches")
    last = {}
    for (sname, label), (_, ctr) in zip(log_, disp):
        if label != "touch":
            last[(sname, label)] = ctr  # the timed launch follows the warm one
    counters = sorted({c for ctr in last.values() for c in ctr})
    labels = list(dict.fromkeys(label for (_, label) in last))
    sets = sw["phase_a_sets"]
    lines = ["Command (repository root R on the measuring machine, TMPDIR=/tmp, cwd /tmp):", "",
             "```", command, "```", "",
             f"Box: {sw.get('box')}" + (f"; rates from a separate `--placement-sweep` run on "
                                        f"box {rates.get('box')}" if rates else ""), ""]
    for label in labels:
        lines += [f"**{label}** (counters per launch, millions)", "",
                  "| set | " + " | ".join(c.replace("TCC_EA0_", "").replace("_sum", "")
                                        for c in counters)
                  + (" | % of 8 TB/s |" if rates else " |"),
                  "|---|" + "---|" * (len(counters) + (1 if rates else 0))]
        for sname in sets:
            ctr = last.get((sname, label), {})
            row = [f"{ctr.get(c, float('nan')) / 1e6:.2f}" for c in counters]
            if rates:
                row.append(f"{rates['phase_a'].get(label, {}).get(sname, float('nan')):.2f}")
            lines.append(f"| {sname} | " + " | ".join(row) + " |")
        lines.append("")
    return "\n".join(lines) + "\n"


def summarize_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, command):
    """Write the committed HBM-traffic summary of the fused kernel from four
    rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE, on the benchmark and on
    the 4 GiB calibration copy).  Counter values are KiB per dispatch."""
    import statistics

    def per(rows, key):
        v = [x for k, x in rows if key in k]
        if not v:
            raise SystemExit(f"no dispatch of {key} in the counter files")
        return statistics.median(v), len(v)

    f_k, nf = per(_pmc_rows(fetch_dir, "FETCH_SIZE"), "fused_adamw_kernel")
    w_k, nw = per(_pmc_rows(write_dir, "WRITE_SIZE"), "fused_adamw_kernel")
    # calibration: --calibrate-copy makes CALIBRATION_CALLS copies that each read
    # and write COPY_BYTES (torch may split one copy into several dispatches, so
    # counters are summed over all of them)
    cf = sum(x for _, x in _pmc_rows(copy_fetch_dir, "FETCH_SIZE"))
    cw = sum(x for _, x in _pmc_rows(copy_write_dir, "WRITE_SIZE"))
    if cf <= 0 or cw <= 0:
        raise SystemExit("no calibration dispatches in the counter files")
    known = CALIBRATION_CALLS * COPY_BYTES
    f_scale = known / (cf * 1024)
    w_scale = known / (cw * 1024)
    fetch_b = f_k * 1024 * f_scale
    write_b = w_k * 1024 * w_scale
    import synth
    import sharded_bucket_plan_amd as sbp
    w = synth.WORKLOADS["llama3_8b"]
    n = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n).shard_numel
    alg = fused_bytes_per_elem(w.R, False) * n
    alg_read = (2 * w.R + 12) * n
    alg_write = 14 * n
    lines = [
        "# fused_adamw_kernel, llama3_8b shard (n = %d, R = %d): HBM traffic" % (n, w.R),
        "",
        "Commands (rocprofv3, one counter per run):",
        "",
        "```",
        command,
        "```",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| FETCH_SIZE per fused dispatch (KiB, median of {nf}) | {f_k:.0f} |",
        f"| WRITE_SIZE per fused dispatch (KiB, median of {nw}) | {w_k:.0f} |",
        f"| calibration: {CALIBRATION_CALLS} copies of {COPY_BYTES} B each way; summed FETCH_SIZE / WRITE_SIZE (KiB) | {cf:.0f} / {cw:.0f} |",
        f"| scale factors (known bytes / counted bytes) fetch, write | {f_scale:.4f}, {w_scale:.4f} |",
        f"| fused reads: counted x scale / algorithmic | {fetch_b:.4g} / {alg_read} = {fetch_b / alg_read:.4f} |",
        f"| fused writes: counted x scale / algorithmic | {write_b:.4g} / {alg_write} = {write_b / alg_write:.4f} |",
        "",
        f"source_sha256: {kernel_source_hash()}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_bytes_per_launch: {int(round(fetch_b + write_b))}",
        f"traffic_over_algorithmic: {(fetch_b + write_b) / alg:.4f}",
    ]
    os.makedirs(os.path.dirname(PMC_SUMMARY), exist_ok=True)
    with open(PMC_SUMMARY, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Workloads of the per-kernel counter summary: (run name, workload, bench flags)
PMC_KERNEL_RUNS = (
    ("dp", "llama3_8b_dp", "--workload llama3_8b_dp --steps 2 --warmup 1"),
    ("clip", "llama3_8b", "--clip 1.0 --steps 3 --warmup 1"),
    ("b7", "gpt_7b5", "--workload gpt_7b5 --steps 3 --warmup 1"),
    ("gather", "llama3_8b", "--layout-call gather_shards --steps 3 --warmup 1"),
    ("ushards", "llama3_8b", "--layout-call unpack_shards --steps 3 --warmup 1"),
    ("gather_pt", "gpt2_small",
     "--layout-call gather_shards --plan per_tensor --workload gpt2_small --steps 3 --warmup 1"),
)


def _kernel_read_write(name, R):
    """Algorithmic (read, write) bytes per element of a kernel, from the
    template arguments in its rocprofv3 name, or None for a kernel that is
    not the library's (input generators, torch fills)."""
    import re
    m = re.search(r"(fused_adamw_kernel|accumulate_kernel|sq_norm_kernel|reduce_kernel)"
                  r"<(\d+)(?:, (true|false))?(?:, (true|false))?(?:, \d+)?>", name)
    if not m:
        return None
    kind, r = m.group(1), int(m.group(2))
    a = m.group(3) == "true"
    b = m.group(4) == "true"
    if kind == "fused_adamw_kernel":  # <R, acc, grouped>
        return 2 * r + 12 + (4 if a else 0), 14
    if kind == "accumulate_kernel":  # <R, first>
        return 2 * r + (0 if a else 4), 4
    if kind == "sq_norm_kernel":  # <R, acc, write>; the tile partials are left out
        return 2 * r + (4 if a else 0), 4 if b else 0
    return 2 * r, 4  # reduce_kernel<R>


def summarize_pmc_kernels(base, command):
    """Counted HBM traffic of every library kernel in three workloads against
    its algorithmic bytes, from rocprofv3 --pmc runs under `base`
    ({run}_FETCH_SIZE and {run}_WRITE_SIZE per entry of PMC_KERNEL_RUNS, and
    cal_FETCH_SIZE / cal_WRITE_SIZE of --calibrate-copy).  Dispatches of one
    kernel are summed and divided by the steps the run made (warm-up
    included); copy_kernel's algorithmic bytes are the pack's 4 per element."""
    import synth
    import sharded_bucket_plan_amd as sbp

    cf = sum(x for _, x in _pmc_rows(os.path.join(base, "cal_FETCH_SIZE"), "FETCH_SIZE"))
    cw = sum(x for _, x in _pmc_rows(os.path.join(base, "cal_WRITE_SIZE"), "WRITE_SIZE"))
    known = CALIBRATION_CALLS * COPY_BYTES
    fs, ws = known / (cf * 1024), known / (cw * 1024)
    lines = ["# HBM traffic of every library kernel against its algorithmic bytes", "",
             "Commands (rocprofv3, one counter per run; R is the repository root where they ran):",
             "", "```", command, "```", "",
             f"Calibration (4 GiB copies, {CALIBRATION_CALLS} calls): bytes read = 1024 x "
             f"FETCH_SIZE x {fs:.4f}, bytes written = 1024 x WRITE_SIZE x {ws:.4f}.  "
             "Per step: the kernel's dispatches "
             "summed over the run, divided by its steps (warm-up included); a step of a "
             "--layout-call run is one call of that layout call.  The squared-norm "
             "pass also writes one 8-byte partial per 2048-element tile, which its algorithmic "
             "bytes leave out.", "",
             "| workload | kernel | dispatches | read GB counted / algorithmic | "
             "written GB counted / algorithmic |", "|---|---|---|---|---|"]
    for run, wl, flags in PMC_KERNEL_RUNS:
        w = synth.WORKLOADS[wl]
        n = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n).shard_numel
        steps = int(flags.split("--steps ")[1].split()[0]) + int(flags.split("--warmup ")[1].split()[0])
        F, W = {}, {}
        for k, x in _pmc_rows(os.path.join(base, f"{run}_FETCH_SIZE"), "FETCH_SIZE"):
            F.setdefault(k, []).append(x)
        for k, x in _pmc_rows(os.path.join(base, f"{run}_WRITE_SIZE"), "WRITE_SIZE"):
            W.setdefault(k, []).append(x)
        call = flags.split("--layout-call ")[1].split()[0] if "--layout-call" in flags else None
        if call:  # one layout call per step: its bytes from the plan
            kind = flags.split("--plan ")[1].split()[0] if "--plan " in flags else "whole"
            pl = layout_plan(w, kind)
            call_bytes = LAYOUT_CALL_BYTES[call](sum(w.numels), pl.flat_numel, pl.shard_numel)
        for k in sorted(F):
            if call:
                if "copy_kernel" not in k:
                    continue
                base_name = "fan_copy_kernel" if "fan_copy_kernel" in k else "copy_kernel"
                short = f"{base_name} ({call}, {kind} plan)"
                alg_r, alg_w = call_bytes
            elif "copy_kernel" in k:
                # a pack covers the flat buffer once per step, in however many launches
                short = "copy_kernel (pack)"
                alg_r, alg_w = 2 * n, 2 * n
            else:
                rw = _kernel_read_write(k, w.R)
                if rw is None:
                    continue
                short = k.split("(anonymous namespace)::")[1].split("(")[0] if \
                    "(anonymous namespace)::" in k else k
                launches = len(F[k]) / steps
                alg_r, alg_w = rw[0] * n * launches, rw[1] * n * launches
            per = 1.0 / steps
            got_r = sum(F[k]) * 1024 * fs * per
            got_w = sum(W.get(k, [0.0])) * 1024 * ws * per
            wcell = f"{got_w / 1e9:.3f} / {alg_w / 1e9:.3f} = {got_w / alg_w:.4f}" if alg_w \
                else f"{got_w / 1e9:.4f} / 0"
            lines.append(f"| {wl} | `{short}` | {len(F[k])} | {got_r / 1e9:.3f} / {alg_r / 1e9:.3f}"
                         f" = {got_r / alg_r:.4f} | {wcell} |")
    lines += ["", f"source_sha256 (shard_step.hip and its build flags): {kernel_source_hash()}",
              "", f"source_sha256 (layout.hip and its build flags): "
              f"{kernel_source_hash(LAYOUT_SRC)}"]
    return "\n".join(lines) + "\n"


def box_identity():
    """Which machine and GPU a measurement ran on (MI355X boxes differ)."""
    import socket
    out = {"host": socket.gethostname()}
    try:
        import torch
        prop = torch.cuda.get_device_properties(0)
        out["gpu"] = prop.name
        uuid = getattr(prop, "uuid", None)
        if uuid is not None:
            out["gpu_uuid"] = str(uuid)
    except Exception:  # identity is informative only
        pass
    return out


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_slices(workload_name, seed, first, stride, target_s, chunk=1 << 22):
    """Runs the oracle's fused step over contiguous slices of `chunk` elements
    of the workload's shard (slices first, first + stride, ...; inputs
    generated on the host, outside the timing) until `target_s` seconds of
    oracle work.  Returns (elements done, seconds spent in the oracle)."""
    import numpy as np
    import synth
    from oracle import step as OS

    w = synth.WORKLOADS[workload_name]
    hp = w.adamw
    done = 0
    spent = 0.0
    k = first
    while spent < target_s:
        i0 = k * chunk
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
        k += stride
    return done, spent


def cpu_baseline(workload_name, seed, target_s):
    """The oracle as it stands, on a bounded contiguous sample of the same
    workload's shard (inputs generated on the host), single-threaded numpy."""
    import synth

    w = synth.WORKLOADS[workload_name]
    chunk = 1 << 22
    done, spent = _oracle_slices(workload_name, seed, 0, 1, target_s, chunk)
    b = fused_bytes_per_elem(w.R, w.K > 1)
    return {"value": done / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "gbs": done * b / spent / 1e9, "host_cpu": host_cpu_model(),
            "host_threads_available": os.cpu_count(),
            "sample": (f"{done} elements ({done // chunk} contiguous slices of {chunk}) of the "
                       f"{workload_name} shard, one fused step (R={w.R}"
                       f"{', with accumulator' if w.K > 1 else ''}), numpy binary32 oracle, "
                       f"{spent:.1f} s")}


def _oracle_core_worker(workload_name, seed, k, target_s, chunk, ready, go, results):
    """One core's share of OracleCores: slice k of the shard generated first,
    then, once every worker is ready and the parent says go, the oracle's
    fused step on it over and over for `target_s` seconds (its time does not
    depend on the values)."""
    import numpy as np
    import synth
    from oracle import step as OS

    w = synth.WORKLOADS[workload_name]
    i0 = k * chunk
    peers = [synth.normal_bf16(seed, synth.peer_stream(1, 0, r), chunk, w.grad_sigma, i0)
             for r in range(w.R)]
    th = synth.normal_f32(seed, synth.master_stream(0), chunk, w.master_sigma, i0)
    z = np.zeros(chunk, np.float32)
    acc = OS.reduce_peers(peers) if w.K > 1 else None
    scale = OS.mean_scale(w.R, w.K)
    ready.wait()
    go.wait()
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < target_s:
        OS.shard_step(peers, acc, scale, th, z, z, w.adamw, 1)
        done += chunk
    results.put((k, done, time.perf_counter() - t0))


def host_cores():
    """Host cores this process may use: the affinity mask, capped by
    OMP_NUM_THREADS where that is set (this process's share of a shared host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


class OracleCores:
    """The oracle on `procs` host cores at once: one worker process per core,
    each on its own slice of the shard (the step is elementwise, so the slices
    are independent).  The workers are spawned (not forked) at construction,
    which the bench does before it touches the GPU; they generate their
    inputs and wait.  run() starts them together, each runs only the oracle
    for about `target_s` seconds, and throughput is all elements done over
    the longest worker's time."""

    def __init__(self, workload_name, seed, procs, target_s, chunk=1 << 22):
        import multiprocessing as mp
        self.workload_name, self.procs, self.target_s, self.chunk = (workload_name, procs,
                                                                     target_s, chunk)
        ctx = mp.get_context("spawn")
        self.ready, self.go = ctx.Barrier(procs + 1), ctx.Barrier(procs + 1)
        self.results = ctx.Queue()
        self.workers = [ctx.Process(target=_oracle_core_worker, daemon=True,
                                    args=(workload_name, seed, k, target_s, chunk, self.ready,
                                          self.go, self.results))
                        for k in range(procs)]
        for p in self.workers:
            p.start()

    def wait_ready(self):
        self.ready.wait(timeout=600)

    def run(self):
        import synth
        self.go.wait(timeout=600)
        res = [self.results.get(timeout=600) for _ in range(self.procs)]
        for p in self.workers:
            p.join(timeout=60)
        if any(p.exitcode != 0 for p in self.workers):
            raise RuntimeError("OracleCores: a worker failed")
        w = synth.WORKLOADS[self.workload_name]
        done = sum(d for _, d, _ in res)
        wall = max(t for _, _, t in res)
        b = fused_bytes_per_elem(w.R, w.K > 1)
        return {"value": done / wall, "unit": "params/s", "cores": self.procs, "kind": "oracle",
                "gbs": done * b / wall / 1e9, "wall_s": wall,
                "per_core_params_per_s": [d / t for _, d, t in sorted(res)],
                "host_cpu": host_cpu_model(), "host_threads_available": os.cpu_count(),
                "sample": (f"{self.procs} slices of {self.chunk} elements of the "
                           f"{self.workload_name} shard, one per worker process, each stepped "
                           f"repeatedly for {self.target_s:.0f} s (one fused step, R={w.R}), "
                           "numpy binary32 oracle")}


def cpu_oracle_cores(workload_name, seed, procs, target_s):
    """OracleCores on its own (no GPU work in this process)."""
    pool = OracleCores(workload_name, seed, procs, target_s)
    pool.wait_ready()
    return pool.run()


def _probe_lib():
    import ctypes
    from sharded_bucket_plan_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built: run __graft_entry__.build()")
    L = ctypes.CDLL(PROBE_LIB)
    L.sbp_probe_stream_mix.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_uint32, ctypes.c_int,
                                       ctypes.c_uint, ctypes.c_void_p]
    L.sbp_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_uint, ctypes.c_void_p]
    L.sbp_probe_streams.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_void_p),
                                    ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_uint32, ctypes.c_int, ctypes.c_uint,
                                    ctypes.c_void_p]
    return L


PROBE_VARIANTS = ("8 consecutive per lane", "stores by stream through LDS", "split 4+4")


def mix_ceiling(W, t, rounds=3, reps=3):
    """The ceiling of the fused step's access mix on W's arrays: three
    zero-arithmetic passes of the same traffic (the measurement kernels of
    libsbp_probe.so, mask 0: the state is written back unchanged) timed
    round-robin with the fused step itself, `reps` launches each per round.
    Returns the best probe rate and the fused step's rate in the same rounds;
    None where the step is not a plain fused step with R in {1, 2, 8}."""
    import ctypes
    import torch
    w = W.w
    if W.acc or W.clip or W.groups or w.R not in (1, 2, 8):
        return None
    L = _probe_lib()
    s = W.sets[0]
    tiles = W.n // 2048
    peers = (ctypes.c_void_p * w.R)(*[x.data_ptr() for x in s["peers"]])
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(4, dtype=torch.int32, device=W.dev)
    scale = W.scale(t)
    probe_bytes = fused_bytes_per_elem(w.R, False) * tiles * 2048
    ms = {k: [] for k in range(len(PROBE_VARIANTS))}
    fused_ms = []
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for _ in range(rounds):
        for k in range(-1, len(PROBE_VARIANTS)):
            def launch():
                if k < 0:
                    s["step"](scale, W.hp, t)
                else:
                    rc = L.sbp_probe_stream_mix(k, peers, w.R, s["master"].data_ptr(),
                                                s["m"].data_ptr(), s["v"].data_ptr(),
                                                s["p"].data_ptr(), sink.data_ptr(), tiles, 0,
                                                1, 64, stream)
                    if rc != 0:
                        raise RuntimeError("sbp_probe_stream_mix failed")
            launch()
            for a, b in ev:
                a.record()
                launch()
                b.record()
            torch.cuda.synchronize()
            (fused_ms if k < 0 else ms[k]).extend(a.elapsed_time(b) for a, b in ev)
    rates = {PROBE_VARIANTS[k]: probe_bytes / (statistics.median(v) * 1e-3) / 1e9
             for k, v in ms.items()}
    best = max(rates.values())
    fused = W.bytes_fused / (statistics.median(fused_ms) * 1e-3) / 1e9
    return {"mix_ceiling_gbs": best, "probe_gbs": rates, "fused_gbs_same_rounds": fused,
            "frac_of_mix_ceiling": fused / best, "rounds": rounds, "launches_per_round": reps}


# The probe family of --placement-sweep: (label, kind, variant, blocks per
# CU, XCD chunk, bytes per element of the Llama shard's traffic mix)
SWEEP = ([("fused step (library kernel)", "fused", None, None, None, 42)]
         + [(f"8/lane, stores at end, {b} blk/CU, C64", "probe", 0, b, 64, 42)
            for b in (1, 2, 3, 4)]
         + [("8/lane, stores at end, uncapped, C64", "probe", 0, 0, 64, 42)]
         + [(f"8/lane, stores at end, 1 blk/CU, C{c}", "probe", 0, 1, c, 42)
            for c in (1, 16, 32, 256)]
         + [("8/lane, stores at end, 1 blk/CU, one eighth per XCD", "probe", 0, 1, 0, 42)]
         + [(f"stores by stream through LDS, {b} blk/CU", "probe", 1, b, 64, 42) for b in (1, 2)]
         + [(f"loads and stores by stream through LDS, {b} blk/CU", "probe", 7, b, 64, 42)
            for b in (1, 2)]
         + [(f"split 4+4, {b} blk/CU", "probe", 2, b, 64, 42) for b in (1, 2, 4)]
         + [(f"16 consecutive/lane, {b} blk/CU", "probe", 5, b, 64, 42) for b in (1, 2)]
         + [(f"2 x 8, 256 groups apart, {b} blk/CU", "probe", 6, b, 64, 42) for b in (1, 2)]
         + [(f"read-only (11 streams), {b or 'uncapped'} blk/CU", "probe", 3, b, 64, 28)
            for b in (1, 2, 0)]
         + [(f"write-only (4 streams), {b or 'uncapped'} blk/CU", "probe", 4, b, 64, 14)
            for b in (1, 2, 4, 0)]
         + [(f"copy 4 GiB, {b or 'uncapped'} blk/CU", "copy", None, b, 64, None)
            for b in (2, 4, 8, 0)])
SWEEP_QUICK = (0, 1, 22, 26)  # fused, 8/lane at 1 blk/CU, read-only at 1, write-only at 2


def placement_sweep(seed, passes=3, reps=3, quick=False, compact_sets=9, spread_sets=3):
    """The stream-mix probe family (libsbp_probe.so) and the library's fused
    R = 8 step on the Llama-3-8B shard's 12 arrays (n rounded down to whole
    tiles), on many physical placements held at once, timed round-robin:
      phase A  `compact_sets` arenas made with no spread (each array's chunks
               created one after another), allocated in sequence, so together
               they walk through the HBM; the fused step, the 8/lane probe
               and the read-only and write-only halves of the mix;
      phase B  (after A's arenas are freed) `spread_sets` spread arenas, then
               one set of torch allocations; every variant of the family.
    Rates are % of 8 TB/s from the median of `reps` launches per pass."""
    import ctypes
    import torch
    import sharded_bucket_plan_amd as sbp
    import synth

    L = _probe_lib()
    w = synth.WORKLOADS["llama3_8b"]
    n_shard = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n).shard_numel
    tiles = n_shard // 2048
    n = tiles * 2048
    R = w.R
    sizes = [4 * n] * 3 + [2 * n] + [2 * n] * R  # master, m, v, out, peers
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    hp = sbp.AdamW(w.adamw.lr, w.adamw.beta1, w.adamw.beta2, w.adamw.eps, w.adamw.weight_decay)
    copy_a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    copy_b = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)

    def arrays_of(ptrs):
        return {"master": ptrs[0], "m": ptrs[1], "v": ptrs[2], "out": ptrs[3],
                "peers": (ctypes.c_void_p * R)(*ptrs[4:4 + R])}

    launches = []  # (set, label) of every kernel launch, in order

    def launch(item, a, t, sname=""):
        label, kind, var, bpc, C, _ = item
        launches.append((sname, label))
        if kind == "fused":
            h = sbp.AdamWHParams.of(hp, t, "sweep")
            rc = sbp.lib().sbp_adamw_shard(a["peers"], R, None, 0.125, a["master"], a["m"],
                                           a["v"], a["out"], n, ctypes.byref(h), stream)
        elif kind == "copy":
            rc = L.sbp_probe_copy(copy_a.data_ptr(), copy_b.data_ptr(), COPY_BYTES, bpc, C,
                                  stream)
        else:
            rc = L.sbp_probe_stream_mix(var, a["peers"], R, a["master"], a["m"], a["v"],
                                        a["out"], sink.data_ptr(), tiles, 0, bpc, C, stream)
        if rc != 0:
            raise RuntimeError(f"sweep launch failed: {label}")

    def nbytes(item):
        return 2 * COPY_BYTES if item[1] == "copy" else item[5] * n

    def run(sets, items, tag):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        ms = {}
        for p in range(passes):
            for sname, a in sets:
                for item in items:
                    if item[1] == "copy" and sname != sets[0][0]:
                        continue
                    launch(item, a, 1, sname)
                    for x, y in ev:
                        x.record()
                        launch(item, a, 1, sname)
                        y.record()
                    torch.cuda.synchronize()
                    ms.setdefault((item[0], sname), []).extend(x.elapsed_time(y) for x, y in ev)
            log(f"sweep {tag}: pass {p + 1}/{passes}")
        table = {}
        for item in items:
            row = {}
            for sname, _ in sets:
                v = ms.get((item[0], sname))
                if v:
                    row[sname] = round(nbytes(item) / (statistics.median(v) * 1e-3) / 1e9
                                       / PEAK_GBS * 100, 2)
            table[item[0]] = row
        return table

    def touch(a, sname):  # write every page once (the write-only probe, no cap)
        launches.append((sname, "touch"))
        if L.sbp_probe_stream_mix(4, a["peers"], R, a["master"], a["m"], a["v"], a["out"],
                                  sink.data_ptr(), tiles, 0, 0, 64, stream) != 0:
            raise RuntimeError("sweep: touch failed")
        for k in range(R):  # peers: a copy over each of them
            p = a["peers"][k]
            launches.append((sname, "touch"))
            if L.sbp_probe_copy(copy_a.data_ptr(), p, (2 * n) // 16384 * 16384, 0, 64,
                                stream) != 0:
                raise RuntimeError("sweep: touch failed")

    out = {"n": n, "R": R, "passes": passes, "launches_per_pass": reps,
           "unit": "% of 8 TB/s (algorithmic bytes / median launch time)",
           "box": box_identity()}
    log(f"sweep: box {out['box']}")
    # phase A: compact arenas, allocated in sequence through the HBM
    items_a = [SWEEP[i] for i in SWEEP_QUICK]
    arenas, sets = [], []
    for k in range(compact_sets):
        ar = sbp.Arena(sizes, spread=sum(-(-b // (64 << 20)) for b in sizes) * (64 << 20),
                       seed=k)
        free, _ = torch.cuda.mem_get_info()
        log(f"sweep: compact set {k} allocated; {free / 1e9:.1f} GB free")
        arenas.append(ar)
        sets.append((f"compact{k}", arrays_of(ar.ptrs)))
        touch(sets[-1][1], sets[-1][0])
    torch.cuda.synchronize()
    out["phase_a"] = run(sets, items_a, "A")
    out["phase_a_sets"] = [s for s, _ in sets]
    del arenas, sets
    import gc
    gc.collect()
    torch.cuda.synchronize()
    if quick:
        out["launches"] = launches
        return out
    # phase B: spread arenas, then torch allocations
    arenas, sets, keep = [], [], []
    for k in range(spread_sets):
        ar = sbp.Arena(sizes, seed=100 + k)
        arenas.append(ar)
        sets.append((f"spread{k}", arrays_of(ar.ptrs)))
        touch(sets[-1][1], sets[-1][0])
        log(f"sweep: spread set {k} allocated ({ar.info()['chunks_spread']} chunks spread over)")
    ts = [torch.empty(b, dtype=torch.uint8, device=dev) for b in sizes]
    keep.append(ts)
    sets.append(("torch", arrays_of([t.data_ptr() for t in ts])))
    touch(sets[-1][1], sets[-1][0])
    torch.cuda.synchronize()
    out["phase_b"] = run(sets, SWEEP, "B")
    out["phase_b_sets"] = [s for s, _ in sets]
    return out


def fused_rate_on(args, seed, placement, warmup, steps):
    """The workload's fused kernel on buffers of the given placement, in this
    process: `warmup` steps, then the average of `steps` launches."""
    import torch
    W = Workload(args.workload, seed, args.clip, args.groups, args.clip_recompute, placement)
    t = 0
    for _ in range(warmup):
        t += 1
        W.step(t)
    torch.cuda.synchronize()
    evs = [{p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for p, _ in W.parts()} for _ in range(steps)]
    for k in range(steps):
        t += 1
        W.step(t, evs[k])
    torch.cuda.synchronize()
    ms = [e["fused_adamw_kernel"][0].elapsed_time(e["fused_adamw_kernel"][1]) for e in evs]
    avg = sum(ms) / len(ms)
    gbs = W.bytes_fused / (avg * 1e-3) / 1e9
    out = {"placement": W.placement, "kernel_ms_avg": avg, "gbs": gbs, "frac": gbs / PEAK_GBS}
    W.release()
    return out


def bucket_sweep(seed, reps=5):
    """Bucket-size sweep on the "7.5B" shard (n = 103,890,048, R = 8): one later
    microbatch accumulated bucket by bucket -- one launch per bucket, as each
    bucket's reduce-scatter share arrives -- for caps of 1..256 MiB, with
    whole-tensor and split-tensor plans.  The per-bucket launches of one pass
    are captured in a HIP graph and replayed, so host launch cost is left out.
    Fits the alpha-beta model of "Parallelisms" (Gradient bucketing):
    T(K buckets) = K * alpha + beta * M, M = (2R + 8) * n bytes."""
    import numpy as np
    import torch
    import sharded_bucket_plan_amd as sbp
    import synth

    w = synth.WORKLOADS["gpt_7b5"]
    dev = torch.device("cuda:0")
    n = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n).shard_numel
    peers = [synth.dev_normal_bf16(torch.empty(n, dtype=torch.int16, device=dev), seed,
                                   synth.peer_stream(1, 1, r), w.grad_sigma) for r in range(w.R)]
    acc = torch.zeros(n, dtype=torch.float32, device=dev)
    M = (2 * w.R + 8) * n
    rows = []
    for split in (False, True):
        for cap in (1, 2, 4, 8, 16, 32, 64, 128, 256):
            pl = sbp.bucket_plan(w.numels, cap << 20, w.world_n, split=split)
            if pl.shard_numel != n:
                raise SystemExit("bucket sweep: shard size changed with the cap")
            views = []
            for b in range(pl.num_buckets):
                info = pl.bucket(b)
                o, c = info["shard_offset"], info["chunk"]
                views.append((acc[o:o + c], [x[o:o + c] for x in peers]))

            def one_pass():
                for a, ps in views:
                    sbp.accumulate_grads(a, ps, first=False)

            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                one_pass()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_pass()
            g.replay()
            torch.cuda.synchronize()
            ms = []
            for _ in range(reps):
                a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b2.record()
                torch.cuda.synchronize()
                ms.append(a.elapsed_time(b2))
            med = sorted(ms)[len(ms) // 2]
            rows.append({"split": split, "cap_MiB": cap, "buckets": pl.num_buckets, "ms": med,
                         "gbs": M / (med * 1e-3) / 1e9})
            log(f"bucket sweep: split={split} cap={cap} MiB buckets={pl.num_buckets} "
                f"{med:.3f} ms {M / (med * 1e-3) / 1e9:.0f} GB/s")
            del g, views
    fit = {}
    for split in (False, True):
        K = np.array([r["buckets"] for r in rows if r["split"] == split], dtype=np.float64)
        T = np.array([r["ms"] for r in rows if r["split"] == split], dtype=np.float64)
        alpha, c = np.polyfit(K, T, 1)
        fit["split" if split else "whole_tensor"] = {
            "alpha_us_per_bucket": alpha * 1e3, "beta_M_ms": c,
            "bandwidth_gbs_at_one_bucket": M / (c * 1e-3) / 1e9}
    return {"bucket_sweep": rows, "fit": fit, "bytes_per_pass": M, "shard_numel": n}


def layout_plan(w, plan_kind):
    """The plan of a workload's model under one plan kind (whole, split or
    per_tensor)."""
    import sharded_bucket_plan_amd as sbp
    if plan_kind == "split":
        return sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n, split=True)
    if plan_kind == "per_tensor":
        rows = [s[1] if len(s) == 2 else 1 for _, s in w.params]
        return sbp.bucket_plan_per_tensor(w.numels, w.world_n, rows)
    return sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n)


# Algorithmic bytes of one layout call (read, written), from the plan:
# per-tensor element counts P, flat (padded) numel F, shard numel n.
LAYOUT_CALL_BYTES = {
    "pack_grads": lambda P, F, n: (2 * P, 2 * F),
    "shard_of": lambda P, F, n: (2 * n, 2 * n),
    "gather_shards": lambda P, F, n: (2 * F, 2 * F),
    "unpack_params": lambda P, F, n: (2 * P, 2 * P),
    "unpack_shards": lambda P, F, n: (2 * P, 2 * P),
}


def layout_call(seed, workload, plan_kind, call, warmup, steps, misalign=0):
    """One layout call made eagerly warmup + steps times on a workload's model,
    nothing else launched on the GPU after the inputs are generated: the run a
    counter pass divides by its number of calls.  Returns the calls made and
    the median time of the timed ones (HIP events on the launch stream)."""
    import statistics as st
    import torch
    import sharded_bucket_plan_amd as sbp
    import synth

    w = synth.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    pl = layout_plan(w, plan_kind)
    n, F, P = pl.shard_numel, pl.flat_numel, sum(w.numels)
    flat = torch.empty(F, dtype=torch.int16, device=dev)
    shards = [synth.dev_normal_bf16(torch.empty(n, dtype=torch.int16, device=dev), seed,
                                    synth.peer_stream(1, 0, r), w.grad_sigma)
              for r in range(w.world_n)]
    tensors = [torch.empty(k + 8, dtype=torch.int16, device=dev)[misalign:misalign + k]
               for k in w.numels]
    for t, x in enumerate(tensors):
        synth.dev_normal_bf16(x, seed, synth.tensor_stream(1, 0, 0, t), w.grad_sigma)
    tset = sbp.TensorSet(pl, tensors)
    run = {
        "pack_grads": lambda: sbp.pack_grads(pl, tset, flat),
        "shard_of": lambda: sbp.shard_of(pl, 0, flat, shards[0]),
        "gather_shards": lambda: sbp.gather_shards(pl, shards, flat),
        "unpack_params": lambda: sbp.unpack_params(pl, flat, tset),
        "unpack_shards": lambda: sbp.unpack_shards(pl, shards, tset),
    }[call]
    torch.cuda.synchronize()
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    rd, wr = LAYOUT_CALL_BYTES[call](P, F, n)
    med = st.median(ms)
    log(f"layout call: {call} ({plan_kind}, {workload}) x {warmup + steps}, {med:.3f} ms median")
    return {"call": call, "plan": plan_kind, "workload": workload, "calls": warmup + steps,
            "ms_median": med, "algorithmic_bytes": rd + wr,
            "gbs": (rd + wr) / (med * 1e-3) / 1e9}


def layout_moves(seed, workload="llama3_8b", plan_kind="whole", reps=5, misalign=0):
    """The layout calls on a workload's model (default Llama-3-8B at N = 8:
    162 buckets of 291 tensors, 8,030,261,248 elements) under one plan kind
    (whole: tensors whole in capped buckets; split: fixed-size buckets with
    tensors split across them; per_tensor: one bucket per tensor, dim-0 row
    shards): rank 0's chunks of one rank's flat buckets
    (shard_of: what that rank contributes to owner 0 in the reduce-scatter),
    the 8 shards into the flat buckets (gather_shards: the all-gather's
    layout), and the flat buckets into the 291 per-tensor parameters
    (unpack_params), the 8 shards straight into the per-tensor parameters
    (unpack_shards: gather and unpack in one pass), as well as pack_grads
    (per-tensor gradients into the buckets).  Each call is timed with events on the launch stream, median of
    `reps`, twice: as a Python call (host marshalling included) and as a
    replay of a graph holding the call's launches k times (GPU time, which
    the roofline figures use; k spreads the graph's own launch cost); algorithmic bytes are one read and one write per element
    moved (a zero-filled padding element is a write only).  misalign = E > 0
    makes every per-tensor buffer a view E elements into a larger
    allocation, so pack reads and unpack writes 2E bytes off 16-byte
    alignment (as views into a larger parameter buffer are)."""
    import statistics as st
    import torch
    import sharded_bucket_plan_amd as sbp
    import synth

    w = synth.WORKLOADS[workload]
    dev = torch.device("cuda:0")
    rows = [s[1] if len(s) == 2 else 1 for _, s in w.params]
    pl = layout_plan(w, plan_kind)
    n, F, P = pl.shard_numel, pl.flat_numel, sum(w.numels)
    flat = torch.empty(F, dtype=torch.int16, device=dev)
    shards = [synth.dev_normal_bf16(torch.empty(n, dtype=torch.int16, device=dev), seed,
                                    synth.peer_stream(1, 0, r), w.grad_sigma)
              for r in range(w.world_n)]
    tensors = [torch.empty(k + 8, dtype=torch.int16, device=dev)[misalign:misalign + k]
               for k in w.numels]
    for t, x in enumerate(tensors):
        synth.dev_normal_bf16(x, seed, synth.tensor_stream(1, 0, 0, t), w.grad_sigma)
    tset = sbp.TensorSet(pl, tensors)  # the same buffers, marshalled once
    one_pass = {
        "pack_grads": lambda: sbp.pack_grads(pl, tset, flat),
        "unpack_params": lambda: sbp.unpack_params(pl, flat, tset),
        "unpack_shards": lambda: sbp.unpack_shards(pl, shards, tset),
    }
    calls = {
        "pack_grads": (lambda: sbp.pack_grads(pl, tensors, flat), 4 * P + 2 * (F - P)),
        "shard_of": (lambda: sbp.shard_of(pl, 0, flat, shards[0]), 4 * n),
        "gather_shards": (lambda: sbp.gather_shards(pl, shards, flat), 4 * F),
        "unpack_params": (lambda: sbp.unpack_params(pl, flat, tensors), 4 * P),
        "unpack_shards": (lambda: sbp.unpack_shards(pl, shards, tensors), 4 * P),
    }
    def timed(run):
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return st.median(ms)

    out = {}
    for name, (f, nbytes) in calls.items():
        f()
        torch.cuda.synchronize()
        call = timed(f)  # the Python call as a user makes it, host marshalling included
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        # the same launches captured k times in one graph and replayed: GPU time,
        # with the graph's own launch cost spread over k calls
        k = max(1, min(50, int(2.0 / max(call, 1e-3))))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(k):
                f()
        g.replay()
        torch.cuda.synchronize()
        med = timed(g.replay) / k
        del g
        out[name] = {"ms_median": med, "call_ms_median": call, "algorithmic_bytes": nbytes,
                     "gbs": nbytes / (med * 1e-3) / 1e9,
                     "frac": nbytes / (med * 1e-3) / 1e9 / PEAK_GBS}
        if name in one_pass:  # the per-tensor pointers from a TensorSet
            one_pass[name]()
            torch.cuda.synchronize()
            out[name]["call_ms_median_tensorset"] = timed(one_pass[name])
        log(f"layout: {name} {med:.3f} ms on the GPU ({out[name]['gbs']:.0f} GB/s), "
            f"{call:.3f} ms per Python call"
            + (f", {out[name]['call_ms_median_tensorset']:.3f} ms with a TensorSet"
               if name in one_pass else ""))
    # the plans themselves (host only, made once per model): microseconds per build
    plans = {}
    for name, make in (("bucket_plan", lambda: sbp.bucket_plan(w.numels, w.bucket_cap_bytes,
                                                                w.world_n)),
                       ("bucket_plan split", lambda: sbp.bucket_plan(w.numels, w.bucket_cap_bytes,
                                                                      w.world_n, split=True)),
                       ("bucket_plan_per_tensor", lambda: sbp.bucket_plan_per_tensor(
                           w.numels, w.world_n, rows))):
        make()
        t0 = time.perf_counter()
        for _ in range(200):
            make()
        plans[name] = {"us_per_plan": (time.perf_counter() - t0) / 200 * 1e6}
        log(f"layout: {name} {plans[name]['us_per_plan']:.1f} us per plan")
    return {"layout_moves": out, "plans": plans, "workload": workload, "plan": plan_kind,
            "misalign_elements": misalign, "N": w.world_n,
            "shard_numel": n, "flat_numel": F, "tensors": len(w.numels),
            "buckets": pl.num_buckets}


def stream_mix(seed, passes=4, reps=5):
    """Achieved HBM bandwidth of the library's own kernels against their mix of
    read and write streams, on the Llama-3-8B shard (n = 1,003,782,656): the
    squared-norm pass (reads only), one-tensor pack (a plain copy), reduce,
    accumulate and the fused step at several R.  Beside each kernel, the
    ceiling of its own mix: the best of zero-arithmetic passes of exactly its
    traffic (libsbp_probe.so's sbp_probe_streams, mask 0) over 1 to 4 groups
    of 8 per lane, 1 to 4 blocks per CU or no cap, and tiles dealt to the XCDs
    in chunks of 32 or 64.  Every configuration is timed round-robin in one
    process (`passes` rounds of `reps` launches each, HIP events on the launch
    stream, median), so all share one placement of the arrays (a spread
    arena).  Algorithmic bytes per element as in the roofline table."""
    import ctypes
    import statistics as st
    import torch
    import sharded_bucket_plan_amd as sbp
    import synth

    w = synth.WORKLOADS["llama3_8b"]
    n = sbp.bucket_plan(w.numels, w.bucket_cap_bytes, w.world_n).shard_numel
    dev = torch.device("cuda:0")
    # every array in one spread arena, as the benchmark's step places them
    arena = sbp.Arena([2 * n] * 8 + [4 * n] * 5 + [2 * n] * 2)
    peers = [synth.dev_normal_bf16(arena.tensor(r, torch.int16, n), seed,
                                   synth.peer_stream(1, 0, r), 1e-3) for r in range(8)]
    acc, m, v, out = (arena.tensor(8 + j, torch.float32, n).zero_() for j in range(4))
    master = synth.dev_normal_f32(arena.tensor(12, torch.float32, n), seed,
                                  synth.master_stream(0), 0.02)
    p = arena.tensor(13, torch.int16, n)
    flat = arena.tensor(14, torch.int16, n)
    one = sbp.bucket_plan([n], 4 * n, 1)  # one tensor, one bucket: pack is a plain copy
    ws = torch.empty(sbp.grad_sq_norm_workspace(n), dtype=torch.float64, device=dev)
    sq = torch.empty(1, dtype=torch.float64, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    hp = sbp.AdamW()
    t = [0]
    L = _probe_lib()
    stream = torch.cuda.current_stream()

    def fused(R, with_acc):
        def f():
            t[0] += 1
            sbp.adamw_shard(peers[:R], acc if with_acc else None, 0.125, master, m, v, p, hp, t[0])
        return f

    def probe(shape, b, f, g, o, gpl, bpc, C):
        """One zero-arithmetic pass of `shape` = (RB, RF, WF, WG, WB) on the
        given arrays; returns (call, elements it covers)."""
        tiles = n // (2048 * gpl)
        sh = (ctypes.c_int * 5)(*shape)
        bp = (ctypes.c_void_p * 8)(*[x.data_ptr() for x in b])
        fp = (ctypes.c_void_p * 4)(*[x.data_ptr() for x in f])
        args = (sh, gpl, bp, fp, g.data_ptr() if g is not None else None,
                o.data_ptr() if o is not None else None, sink.data_ptr(), tiles, 0, bpc, C)

        def call():
            if L.sbp_probe_streams(*args, ctypes.c_void_p(stream.cuda_stream)) != 0:
                raise RuntimeError(f"sbp_probe_streams failed for {shape}")
        return call, tiles * 2048 * gpl

    # (name, read streams, write streams, bytes per element, call,
    #  probe shape (RB, RF, WF, WG, WB), its bf16 / fp32 / G / bf16-out arrays)
    kinds = [
        ("squared norm, R=1", 1, 0, 2, lambda: sbp.grad_sq_norm(peers[:1], None, 1.0, n,
                                                                workspace=ws, sq_out=sq),
         (1, 0, 0, 0, 0), peers[:1], [], None, None),
        ("squared norm, R=2", 2, 0, 4, lambda: sbp.grad_sq_norm(peers[:2], None, 0.5, n,
                                                                workspace=ws, sq_out=sq),
         (2, 0, 0, 0, 0), peers[:2], [], None, None),
        ("squared norm of the accumulator (R=0)", 1, 0, 4,
         lambda: sbp.grad_sq_norm([], acc, 0.125, n, workspace=ws, sq_out=sq),
         (0, 1, 0, 0, 0), [], [acc], None, None),
        ("squared norm, R=8", 8, 0, 16, lambda: sbp.grad_sq_norm(peers, None, 0.125, n,
                                                                 workspace=ws, sq_out=sq),
         (8, 0, 0, 0, 0), peers, [], None, None),
        ("squared norm, R=8 + accumulator", 9, 0, 20,
         lambda: sbp.grad_sq_norm(peers, acc, 0.125, n, workspace=ws, sq_out=sq),
         (8, 1, 0, 0, 0), peers, [acc], None, None),
        ("pack of one tensor (copy)", 1, 1, 4, lambda: sbp.pack_grads(one, [peers[0]], flat),
         (1, 0, 0, 0, 1), peers[:1], [], None, flat),
        ("reduce, R=1", 1, 1, 6, lambda: sbp.reduce_shard(peers[:1], 1.0, out),
         (1, 0, 0, 1, 0), peers[:1], [], out, None),
        ("reduce, R=8", 8, 1, 20, lambda: sbp.reduce_shard(peers, 0.125, out),
         (8, 0, 0, 1, 0), peers, [], out, None),
        ("squared norm, R=8, writing G", 8, 1, 20,
         lambda: sbp.grad_sq_norm(peers, None, 0.125, n, g_sum_out=out, workspace=ws, sq_out=sq),
         (8, 0, 0, 1, 0), peers, [], out, None),
        ("accumulate, R=8, first", 8, 1, 20,
         lambda: sbp.accumulate_grads(acc, peers, first=True),
         (8, 0, 0, 1, 0), peers, [], acc, None),
        ("accumulate, R=8, later", 9, 1, 24,
         lambda: sbp.accumulate_grads(acc, peers, first=False),
         (8, 1, 1, 0, 0), peers, [acc], None, None),
        ("fused step from G (R=0)", 4, 4, 30, fused(0, True),
         (0, 4, 3, 0, 1), [], [master, m, v, acc], None, p),
        ("fused step, R=2", 5, 4, 30, fused(2, False),
         (2, 3, 3, 0, 1), peers[:2], [master, m, v], None, p),
        ("fused step, R=8 (the headline)", 11, 4, 42, fused(8, False),
         (8, 3, 3, 0, 1), peers, [master, m, v], None, p),
        ("fused step, R=8 + accumulator", 12, 4, 46, fused(8, True),
         (8, 4, 3, 0, 1), peers, [master, m, v, acc], None, p),
    ]
    # every configuration to time: the kernels, then each kernel's probes
    calls = {}
    for name, _, _, bpe, f, shape, b, fa, g, o in kinds:
        calls[name] = (f, n, bpe, None)
        lane = 16 * shape[0] + 32 * shape[1]
        for gpl in ((1, 2, 4) if lane <= 32 else (1, 2)):
            for bpc in (1, 2, 3, 4, 0):
                for C in (32, 64):
                    call, cover = probe(shape, b, fa, g, o, gpl, bpc, C)
                    calls[(name, gpl, bpc, C)] = (call, cover, bpe, (gpl, bpc, C))
    times = {k: [] for k in calls}
    torch.cuda.synchronize()
    for ps in range(passes):
        for key, (f, _, _, _) in calls.items():
            for _ in range(2):
                f()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps)]
            for a, b in evs:
                a.record(stream)
                f()
                b.record(stream)
            torch.cuda.synchronize()
            times[key] += [a.elapsed_time(b) for a, b in evs]
        log(f"stream mix: pass {ps + 1} of {passes} done")

    def rate(key):
        _, cover, bpe, _ = calls[key]
        return bpe * cover / (st.median(times[key]) * 1e-3) / 1e9

    rows = []
    for name, rd, wr, bpe, _, shape, _, _, _, _ in kinds:
        ms = st.median(times[name])
        gbs = rate(name)
        best = max((k for k in calls if isinstance(k, tuple) and k[0] == name), key=rate)
        pg = rate(best)
        gpl, bpc, C = calls[best][3]
        rows.append({"kind": name, "read_streams": rd, "write_streams": wr,
                     "bytes_per_elem": bpe, "ms_median": ms, "gbs": gbs, "frac": gbs / PEAK_GBS,
                     "probe_shape": list(shape),
                     "probe_best": {"gbs": pg, "frac": pg / PEAK_GBS, "groups_per_lane": gpl,
                                    "blocks_per_cu": bpc, "xcd_chunk": C},
                     "frac_of_probe": gbs / pg})
        log(f"stream mix: {name:38s} {rd:2d}R+{wr}W {bpe:2d} B {ms:.3f} ms {gbs:.0f} GB/s "
            f"{100 * gbs / PEAK_GBS:.1f}%; its mix's probe {pg:.0f} GB/s "
            f"(gpl {gpl}, {bpc or 'no cap'} blocks/CU, C={C}): {gbs / pg:.3f}")
    return {"stream_mix": rows, "n": n, "passes": passes, "reps": reps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-oracle-cores", type=int, metavar="P",
                    help="only time the oracle on P host cores at once (about --cpu-seconds "
                         "of oracle work per core, --workload's shard) and print its JSON; "
                         "the GPU is not used")
    ap.add_argument("--clip", type=float, default=None, metavar="MAX_NORM",
                    help="add global gradient-norm clipping to the step")
    ap.add_argument("--clip-recompute", action="store_true",
                    help="with --clip: the norm pass writes no G and the update sums the "
                         "peers again (fewer bytes when R < 4, or R < 2 with an accumulator)")
    ap.add_argument("--groups", action="store_true",
                    help="two parameter groups (no weight decay on 1-D tensors): the grouped "
                         "fused step")
    ap.add_argument("--placement", choices=["spread", "torch"], default="spread",
                    help="where the step's arrays live: a spread arena (the library's "
                         "sbp_arena, pages spread over the whole HBM; the default) or "
                         "ordinary torch allocations")
    ap.add_argument("--no-compare-placement", action="store_true",
                    help="skip timing the fused kernel on torch allocations after the "
                         "spread-arena run")
    ap.add_argument("--no-mix-ceiling", action="store_true",
                    help="skip the zero-arithmetic probes of the fused step's access mix")
    ap.add_argument("--oracle-cores", type=int, default=None, metavar="P",
                    help="host cores for the all-core oracle baseline (default: this "
                         "process's share, capped by OMP_NUM_THREADS)")
    ap.add_argument("--placement-sweep", action="store_true",
                    help="only run the stream-mix probe family and the fused step over many "
                         "physical placements of the Llama shard's arrays and print its JSON")
    ap.add_argument("--sweep-quick", action="store_true",
                    help="with --placement-sweep: phase A only, one pass, one launch each "
                         "(for counter runs)")
    ap.add_argument("--summarize-sweep-pmc", nargs=4,
                    metavar=("PMC_DIR", "SWEEP_QUICK_JSON", "RATES_JSON", "CMD"),
                    help="print the DRAM credit-stall table of a counter run of "
                         "--placement-sweep --sweep-quick (RATES_JSON: a plain sweep's output, "
                         "or '')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--bucket-sweep", action="store_true",
                    help="only run the bucket-size sweep (7.5B shard) and print its JSON")
    ap.add_argument("--layout", action="store_true",
                    help="only time the layout calls (pack, shard_of, gather, unpack) and the "
                         "plan builds on --workload's model and print their JSON")
    ap.add_argument("--plan", choices=["whole", "split", "per_tensor"], default="whole",
                    help="with --layout: the plan whose layout is timed (whole-tensor buckets, "
                         "fixed-size split buckets, or one bucket per tensor with row shards)")
    ap.add_argument("--misalign", type=int, default=0, metavar="E",
                    help="with --layout: every per-tensor buffer a view E (0..7) elements into "
                         "a larger allocation")
    ap.add_argument("--layout-call", choices=sorted(LAYOUT_CALL_BYTES),
                    help="only make this layout call --warmup + --steps times, eagerly, on "
                         "--workload's model under --plan (a counter pass of one kernel)")
    ap.add_argument("--stream-mix", action="store_true",
                    help="only time the library's kernels against their read/write stream mix "
                         "on the Llama-3-8B shard and print their JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the 4 GiB device copy (for counter calibration)")
    ap.add_argument("--summarize-pmc-kernels", nargs=2, metavar=("BASE_DIR", "CMD"),
                    help="print the per-kernel HBM-traffic summary from the counter runs "
                         "under BASE_DIR")
    ap.add_argument("--summarize-pmc", nargs=5,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "CMD"),
                    help="write the HBM-traffic summary from rocprofv3 counter runs")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_sweep_pmc:
        print(summarize_sweep_pmc(*args.summarize_sweep_pmc), end="")
        return
    if args.summarize_pmc_kernels:
        print(summarize_pmc_kernels(*args.summarize_pmc_kernels), end="")
        return

    if args.cpu_oracle_cores:
        import synth
        seed = synth.SEED if args.seed is None else args.seed
        print(json.dumps(cpu_oracle_cores(args.workload, seed, args.cpu_oracle_cores,
                                          args.cpu_seconds)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the "
              "shard step is per rank and nothing here crosses GPUs", file=sys.stderr)
        sys.exit(2)

    # the all-core oracle's workers are spawned before anything touches the
    # GPU; they generate their inputs now and run after the GPU timing
    import synth
    seed = synth.SEED if args.seed is None else args.seed
    modes = (args.bucket_sweep or args.layout or args.layout_call or args.stream_mix
             or args.calibrate_copy or args.placement_sweep)
    pool = None
    cores = args.oracle_cores or host_cores()
    if not modes and not args.no_cpu_baseline and cores > 1:
        pool = OracleCores(args.workload, seed, cores, args.cpu_seconds)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.bucket_sweep:
        print(json.dumps(bucket_sweep(seed)), flush=True)
        return
    if args.layout:
        if not 0 <= args.misalign <= 7:
            raise SystemExit("bench.py: --misalign takes 0..7 elements")
        print(json.dumps(layout_moves(seed, args.workload, args.plan, misalign=args.misalign)),
              flush=True)
        return
    if args.layout_call:
        print(json.dumps(layout_call(seed, args.workload, args.plan, args.layout_call,
                                     args.warmup, args.steps, args.misalign)), flush=True)
        return
    if args.stream_mix:
        print(json.dumps(stream_mix(seed)), flush=True)
        return
    if args.placement_sweep:
        if args.sweep_quick:
            res = placement_sweep(seed, passes=1, reps=1, quick=True, compact_sets=9)
        else:
            res = placement_sweep(seed)
        print(json.dumps(res), flush=True)
        return
    if args.calibrate_copy:
        print(json.dumps({"copy_gbs": copy_ceiling_gbs(CALIBRATION_CALLS - 1),
                          "bytes_each_way": COPY_BYTES, "calls": CALIBRATION_CALLS}))
        return
    log(f"bench: workload {args.workload}, allocating and generating inputs on cuda:0")
    if args.groups and args.clip:
        raise SystemExit("bench.py: --groups and --clip are separate measurements")
    if args.clip_recompute and not args.clip:
        raise SystemExit("bench.py: --clip-recompute goes with --clip")
    W = Workload(args.workload, seed, args.clip, args.groups, args.clip_recompute,
                 args.placement)
    log(f"bench: n={W.n} R={W.w.R} sets={W.nsets} placement={W.placement}; "
        f"warmup {args.warmup}")
    t = 0
    for _ in range(args.warmup):
        t += 1
        W.step(t)
    torch.cuda.synchronize()
    if pool:
        pool.wait_ready()  # the oracle workers have their inputs and are idle
    parts = W.parts()
    evs = [{p: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for p, _ in parts} for _ in range(args.steps)]
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
    kernels = {}
    for p, nbytes in parts:
        ms = [e[p][0].elapsed_time(e[p][1]) for e in evs]
        avg = sum(ms) / len(ms)
        gbs = nbytes / (avg * 1e-3) / 1e9
        kernels[p] = {"ms_avg": avg, "ms_median": statistics.median(ms), "ms_min": min(ms),
                      "algorithmic_bytes": nbytes,
                      "gbs": gbs, "frac": gbs / PEAK_GBS}
    kern_ms = [e["fused_adamw_kernel"][0].elapsed_time(e["fused_adamw_kernel"][1]) for e in evs]
    kern_avg = sum(kern_ms) / len(kern_ms)
    achieved = W.bytes_fused / (kern_avg * 1e-3) / 1e9
    value = W.n / (ms_per_step * 1e-3)
    config = W.config()
    bytes_fused = W.bytes_fused
    log(f"bench: {ms_per_step:.4f} ms/step, fused kernel {kern_avg:.4f} ms avg "
        f"(min {min(kern_ms):.4f}), {achieved:.1f} GB/s algorithmic")

    # the committed counters are of the plain fused kernel
    traffic = None if args.groups else traffic_from_profile(bytes_fused)
    ceiling = None
    if not args.no_mix_ceiling:
        ceiling = mix_ceiling(W, t + 1)
        if ceiling:
            log(f"bench: access-mix ceiling {ceiling['mix_ceiling_gbs']:.0f} GB/s "
                f"(zero-arithmetic probes); fused step {ceiling['fused_gbs_same_rounds']:.0f} "
                f"GB/s in the same rounds = {ceiling['frac_of_mix_ceiling']:.3f} of it")
    placement = W.placement
    nsets = W.nsets
    W.release()
    del W
    other = None
    if placement == "spread" and not args.no_compare_placement:
        other = fused_rate_on(args, seed, "torch", args.warmup, args.steps)
        log(f"bench: the same kernel on torch allocations: {other['kernel_ms_avg']:.4f} ms, "
            f"{other['frac']:.3f} of 8 TB/s")
    copy_gbs = copy_fp = None
    if not args.no_copy_ceiling:
        torch.cuda.empty_cache()
        copy_gbs = copy_ceiling_gbs()
        log(f"bench: 4 GiB device copy on this GPU: {copy_gbs:.0f} GB/s")
        if nsets > 1:  # a small workload: also a copy of its own footprint
            copy_fp = footprint_copy_gbs(bytes_fused, nsets)
            log(f"bench: copy of the same footprint ({bytes_fused / 1e6:.0f} MB per launch, "
                f"{nsets} rotating sets): {copy_fp:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"bench: CPU baseline (~{args.cpu_seconds:.0f} s of oracle work on 1 core"
            + (f", then on {cores} cores)" if pool else ")"))
        one = cpu_baseline(args.workload, seed, args.cpu_seconds)
        if pool:
            cpu = pool.run()
            cpu["one_core"] = one
        else:
            cpu = one

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
        "config": config,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBS, "traffic": traffic,
                     "kernel": "fused_adamw_kernel", "kernel_ms_avg": kern_avg,
                     "algorithmic_bytes_per_launch": bytes_fused,
                     "copy_gbs_this_gpu": copy_gbs,
                     "frac_of_copy": (achieved / copy_gbs) if copy_gbs else None,
                     "copy_gbs_same_footprint": copy_fp,
                     "frac_of_copy_same_footprint": (achieved / copy_fp) if copy_fp else None,
                     "placement": placement,
                     "mix_ceiling_gbs": ceiling["mix_ceiling_gbs"] if ceiling else None,
                     "frac_of_mix_ceiling": (achieved / ceiling["mix_ceiling_gbs"]
                                             if ceiling else None),
                     "mix_ceiling": ceiling,
                     "torch_placement": other},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "box": box_identity(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
