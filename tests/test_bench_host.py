"""Host-side logic of bench.py (CPU): algorithmic bytes per kernel and per
layout call, the one-GPU refusal, and the per-kernel traffic summary run end
to end on synthetic rocprofv3 counter files."""
import csv
import os
import subprocess
import sys

import pytest

import bench
import sharded_bucket_plan_amd as sbp
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,R,want", [
    ("(anonymous namespace)::fused_adamw_kernel<8, false, false>(...)", 8, (28, 14)),
    ("(anonymous namespace)::fused_adamw_kernel<2, false, true>(...)", 2, (16, 14)),
    ("(anonymous namespace)::fused_adamw_kernel<0, true, false>(...)", 8, (16, 14)),
    ("(anonymous namespace)::fused_adamw_kernel<8, true, false>(...)", 8, (32, 14)),
    ("(anonymous namespace)::accumulate_kernel<8, true>(...)", 8, (16, 4)),
    ("(anonymous namespace)::accumulate_kernel<8, false>(...)", 8, (20, 4)),
    ("(anonymous namespace)::sq_norm_kernel<8, false, true, 1>(...)", 8, (16, 4)),
    ("(anonymous namespace)::sq_norm_kernel<1, false, false, 4>(...)", 1, (2, 0)),
    ("(anonymous namespace)::sq_norm_kernel<0, true, false, 2>(...)", 8, (4, 0)),
    ("(anonymous namespace)::reduce_kernel<8>(...)", 8, (16, 4)),
    ("(anonymous namespace)::fill_bf16_kernel(unsigned short*, long)", 8, None),
])
def test_kernel_bytes_per_element(name, R, want):
    """The per-element bytes each kernel must move (reads, writes)."""
    assert bench._kernel_read_write(name, R) == want
    if want and "fused_adamw_kernel" in name and "<0," not in name:
        acc = "true, " in name.split("<")[1].split(">")[0][3:]
        assert sum(want) == bench.fused_bytes_per_elem(R, acc)


def test_fused_bytes_per_element():
    assert bench.fused_bytes_per_elem(8, False) == 42
    assert bench.fused_bytes_per_elem(2, False) == 30
    assert bench.fused_bytes_per_elem(8, True) == 46


def test_layout_call_bytes_follow_the_plan():
    w = synth.WORKLOADS["gpt2_small"]
    for kind in ("whole", "split", "per_tensor"):
        pl = bench.layout_plan(w, kind)
        P, F, n = sum(w.numels), pl.flat_numel, pl.shard_numel
        assert F == n * w.world_n and F >= P
        got = {k: f(P, F, n) for k, f in bench.LAYOUT_CALL_BYTES.items()}
        assert got["gather_shards"] == (2 * F, 2 * F)  # padding read and written
        assert got["unpack_shards"] == got["unpack_params"] == (2 * P, 2 * P)
        assert got["pack_grads"] == (2 * P, 2 * F)  # padding is written as +0
        assert got["shard_of"] == (2 * n, 2 * n)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        out = csv.writer(f)
        out.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (kernel, value) in enumerate(rows):
            out.writerow([i + 1, kernel, counter, repr(value)])


def test_traffic_summary_of_a_layout_call(tmp_path):
    """Synthetic counter files: a calibration copy read twice as many bytes as
    FETCH_SIZE counts (and written once), and a gather whose counted bytes are
    exactly its algorithmic ones in 2 launches per call over 4 calls; the
    summary must divide by the calls, scale by the calibration and land on
    1.0000 both ways.  Kernels that are not the library's are left out."""
    base = str(tmp_path)
    calls = bench.CALIBRATION_CALLS
    _write_counters(os.path.join(base, "cal_FETCH_SIZE"), "FETCH_SIZE",
                    [("copy", bench.COPY_BYTES / 1024 / 2)] * calls)
    _write_counters(os.path.join(base, "cal_WRITE_SIZE"), "WRITE_SIZE",
                    [("copy", bench.COPY_BYTES / 1024)] * calls)
    for run, _, _ in bench.PMC_KERNEL_RUNS:
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            _write_counters(os.path.join(base, f"{run}_{c}"), c, [])
    pl = bench.layout_plan(synth.WORKLOADS["llama3_8b"], "whole")
    F = pl.flat_numel
    fan = "(anonymous namespace)::fan_copy_kernel((anonymous namespace)::FanList)"
    gen = "(anonymous namespace)::fill_bf16_kernel(unsigned short*, long)"
    n_calls, per_call = 4, 2
    dispatches = n_calls * per_call
    read_each = 2 * F * n_calls / dispatches / 1024 / 2.0  # counted units per dispatch
    write_each = 2 * F * n_calls / dispatches / 1024 / 1.0
    _write_counters(os.path.join(base, "gather_FETCH_SIZE"), "FETCH_SIZE",
                    [(gen, 123.0)] + [(fan, read_each)] * dispatches)
    _write_counters(os.path.join(base, "gather_WRITE_SIZE"), "WRITE_SIZE",
                    [(gen, 456.0)] + [(fan, write_each)] * dispatches)
    text = bench.summarize_pmc_kernels(base, "the commands")
    assert "FETCH_SIZE x 2.0000" in text and "WRITE_SIZE x 1.0000" in text
    rows = [ln for ln in text.splitlines() if "fan_copy_kernel" in ln]
    assert len(rows) == 1
    cells = [c.strip() for c in rows[0].strip("|").split("|")]
    assert cells[0] == "llama3_8b"
    assert cells[1] == "`fan_copy_kernel (gather_shards, whole plan)`"
    assert cells[2] == str(dispatches)
    gb = f"{2 * F / 1e9:.3f}"
    assert cells[3] == f"{gb} / {gb} = 1.0000" and cells[4] == f"{gb} / {gb} = 1.0000"
    assert "fill_bf16_kernel" not in text
    assert f"source_sha256 (layout.hip and its build flags): " \
           f"{bench.kernel_source_hash(bench.LAYOUT_SRC)}" in text


def _undefined_globals(path):
    """Names that some function of `path` reads as globals although neither the
    module nor the builtins define them (a stdlib symtable walk)."""
    import builtins
    import symtable
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    defined = {s.get_name() for s in top.get_symbols()
               if s.is_assigned() or s.is_imported() or s.is_namespace()}
    defined |= set(dir(builtins)) | {"__file__", "__name__"}
    bad = set()

    def walk(t):
        for child in t.get_children():
            for sym in child.get_symbols():
                if sym.is_referenced() and sym.is_global() and sym.get_name() not in defined:
                    bad.add((child.get_name(), sym.get_name()))
            walk(child)
    walk(top)
    return sorted(bad)


def test_no_undefined_names():
    """Every Python file of the repository, the GPU tests included (they only
    run on a GPU, so a misspelt name there would otherwise surface there)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = sorted(set(glob.glob(os.path.join(root, "*.py"))
                       + glob.glob(os.path.join(root, "tests", "**", "*.py"), recursive=True)
                       + glob.glob(os.path.join(root, "oracle", "**", "*.py"), recursive=True)
                       + glob.glob(os.path.join(root, "synth", "*.py"))
                       + glob.glob(os.path.join(root, "sharded_bucket_plan_amd", "*.py"))))
    assert len(files) >= 20
    for path in files:
        assert _undefined_globals(path) == [], os.path.relpath(path, root)
