"""Benchmark of the structured-mask attention forward on one MI355X.

One step = one pass of the hot path over the 128K-token block-sparse causal
prefill (L = 131072, batch 1, 32 heads, head dim 128, bf16, block 128; every
block row keeps the diagonal block, the first block and the top half of the
remaining causal blocks by a seeded score): one launch of the HIP kernel over
the plan compiled from the block matrix, on resident Q, K, V.  The plan is
compiled and uploaded before the timed region.  `--workload` selects another
workload of the catalogue for the headline (its masks then run as one grouped
launch per step).

Metric: effective attention TFLOP/s = 4 * d * (unmasked query-key pairs) per
head divided by the step time (2d flops for the score and 2d for the value mix
per allowed pair; padding, masked pairs inside partial tiles and the
exponentials are not counted), and the same as a fraction of the bf16 dense
MFMA peak.  Launch durations come from HIP events attached to the kernel's own
dispatch; the median and minimum of the launches are reported beside the mean.

Timing protocol of the per-mask figures (headline workload and `extra`): 3
warm-up launches, then every launch timed alone by its events, with a 512 MiB
scratch buffer rewritten between launches for every workload whose inputs and
outputs fit in the 256 MB last-level cache (so no launch starts from a warm
cache); median and minimum reported.  The 128K-token inputs (4.3 GB) exceed
that cache by far and run back to back.

CPU baseline: the float64 oracle on 512 seeded query rows per head of the same
workload (the sampled-row protocol of the largest configs), on as many heads
as fit in about 20 s of host time, with the BLAS thread count; the full-config
oracle time is extrapolated from the per-row time and labelled so.

Extra workloads (skipped with --quick): the 896-px ViT layer (L = 4096, d = 80:
full, chunk 256, window radius 128, one grouped launch), the 1792-px layer
(L = 16384: full and window radius 512), causal LM prefill with per-head
windows and sinks (L = 4096, d = 128), RRAttention's block-pattern search on
the 128K-token Q and K, the token re-permutation, the backward pass of the
896-px and per-head-window masks, and one-query decode steps over key/value
caches, reported in GB/s against HBM.

GPU clocks: sampled with amd-smi by a helper process started before this
process touches the GPU (the helper never does), skipped under a profiler.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
LLC_BYTES = 256 * 2**20       # MI355X last-level (Infinity) cache
FLUSH_BYTES = 512 * 2**20     # scratch rewritten between launches to evict it
CSRC = os.path.join(ROOT, "block_sparse_softmax_amd", "csrc")
# source of each head dim's forward kernel, the headers every forward kernel includes, and the
# scheduler (which work-group runs which tiles decides what the L2s share, hence the traffic)
KERNEL_SRC = {"swizzled": "attn_fwd.hip", "pingpong": "attn_fwd_pp.hip", "single": "attn_fwd_sg.hip"}
KERNEL_HEADERS = ("fwd_common.hpp", "tile_common.hpp", "kernels.hpp", "plan.cpp")
DEFAULT_WORKLOAD = "blocksparse128k"


def _kernel_hash(kind: str) -> str:
    """Hash of a forward kernel's source (its file, the shared headers and the scheduler); kind as
    Plan.kernel()."""
    h = hashlib.sha256()
    for f in (KERNEL_SRC[kind], *KERNEL_HEADERS):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def _traffic_from_profile(workload: str, mask: str, kind: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_{mask}_traffic.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not b or m.group(1) != _kernel_hash(kind):
        return None
    return float(b.group(1))


WORKLOADS = {
    "tiny_chunk": "Tiny chunk-window attention: L=256 tokens, batch 1, 2 heads, head dim 64; chunks of 64",
    "vit896": "ViT layer at 896 px: L=4096 tokens, batch 1, 16 heads, head dim 80; "
              "masks full + chunk 256 + sliding window radius 128",
    "vit1792": "ViT layer at 1792 px: L=16384 tokens, batch 1, 16 heads, head dim 80; "
               "masks full + sliding window radius 512",
    "lm_headwin": "Causal LM prefill: L=4096, batch 1, 16 heads, head dim 128; per-head causal windows "
                  "{512, 1024, 2048, 4096} and a sink logit per head",
    "blocksparse128k": "Block-sparse causal prefill: L=131072, batch 1, 32 heads, head dim 128; block 128, "
                       "diagonal + first block + top half of the remaining causal blocks per block row",
    "swa576_d256": "Sliding-window causal prefill: L=131072, batch 1, 16 query heads on 4 K/V heads, head dim "
                   "256; window of 576 keys and a sink logit per head",
}


def under_profiler() -> bool:
    """True when a profiler's tool library is loaded into this process (rocprofv3 exports its settings
    as ROCPROF* variables): a child started now would inherit it."""
    return any(k.startswith("ROCPROF") for k in os.environ)


# The clock sampler: a helper process started before this process touches the GPU.  It never
# initialises the GPU itself; on each request line it runs amd-smi (its own child) and answers with
# one JSON line.  So no process that holds the GPU ever starts another program.
_SAMPLER = r"""
import json, subprocess, sys
for line in sys.stdin:
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "-p", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        g0 = (d["gpu_data"] if isinstance(d, dict) else d)[0]
        c = g0["clock"]
        gfx = [float(v["clk"]["value"]) for k, v in c.items() if k.startswith("gfx") and isinstance(v, dict)]
        mem = [float(v["clk"]["value"]) for k, v in c.items() if k.startswith("mem") and isinstance(v, dict)]
        try:
            watts = float(g0["power"]["socket_power"]["value"])
        except (KeyError, TypeError, ValueError):
            watts = None
        out = dict(gfx_mhz_mean=sum(gfx) / len(gfx) if gfx else None, gfx_mhz_min=min(gfx) if gfx else None,
                   gfx_mhz_max=max(gfx) if gfx else None, mem_mhz=mem[0] if mem else None, socket_watts=watts)
    except Exception:
        out = None
    sys.stdout.write(json.dumps(out) + "\n")
    sys.stdout.flush()
"""


class ClockSampler:
    """GPU clocks and socket power from amd-smi through the helper process (best effort; None when
    unavailable)."""

    def __init__(self, enabled: bool):
        self.proc = None
        if enabled and not under_profiler():
            try:
                self.proc = subprocess.Popen([sys.executable, "-c", _SAMPLER], stdin=subprocess.PIPE,
                                             stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
            except OSError:
                self.proc = None

    def __call__(self):
        if self.proc is None:
            return None
        try:
            self.proc.stdin.write("sample\n")
            self.proc.stdin.flush()
            return json.loads(self.proc.stdout.readline() or "null")
        except (OSError, ValueError):
            return None

    def close(self):
        if self.proc is not None:
            try:
                self.proc.stdin.close()
                self.proc.wait(timeout=30)
            except Exception:  # noqa: BLE001 - shutting down a best-effort helper
                self.proc.kill()
            self.proc = None


def calibrate_copy(mib: int, steps: int, device: str) -> dict:
    """A plain device copy of `mib` MiB, `steps` times: the reference the HBM counters are scaled by."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    if src.is_cuda:
        torch.cuda.synchronize()
    return {"calibrate_copy_bytes": n, "copies": steps}


def _kernel_name(kind: str, D: int) -> str:
    """Name (prefix) of the forward kernel of this kind and head dim in profiler output."""
    return {"pingpong": "attn_fwd_pp_kernel", "single": f"attn_fwd_sg_kernel<{D}"}.get(kind, f"attn_fwd_kernel<{D}")


def _workload_kernel(w) -> tuple:
    """(kind, name) of the forward kernel that runs the workload's launch (host-side plan only)."""
    from block_sparse_softmax_amd._lib import Plan
    m = next(iter(w["masks"].values()))
    kind = Plan(m, w["L"], w["H"], w["D"]).kernel()
    return kind, _kernel_name(kind, w["D"])


def _counter_values(run_dir: str, counter: str, kernel: str):
    """Per-dispatch values of `counter` for kernels whose name contains `kernel`, in dispatch order,
    from the counter_collection.csv files rocprofv3 wrote under run_dir."""
    import csv
    import glob
    vals = []
    for path in sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
                    vals.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    if not vals:
        raise SystemExit(f"no {counter} values for {kernel} under {run_dir}")
    return [v for _, v in sorted(vals)]


# the counter passes run bench.py with --steps 3 --warmup 1: the kernel's first four dispatches are the
# grouped launch (one dispatch for all masks of the workload); the per-mask launches follow
TRAFFIC_RUN_ARGS = "--quick --no-cpu-baseline --no-clocks --steps 3 --warmup 1 --reps 3"
GROUPED_DISPATCHES = slice(1, 4)   # the timed steps (the warm-up dispatch is left out)


def traffic_summary(workload: str, pmc_dir: str, copy_mib: int = 1024, out_dir: str | None = None) -> str:
    """Write profiles/attn_fwd_<workload>_<masks>_traffic.txt from four rocprofv3 counter passes under
    pmc_dir (FETCH_SIZE and WRITE_SIZE of the workload's launches and of a plain copy of copy_mib MiB,
    each scaled so that the copy reads as its known size): HBM bytes of the workload's grouped launch
    (median of its timed dispatches)."""
    import statistics
    from block_sparse_softmax_amd import inputs as gen
    w = gen.workload(workload)
    label = "+".join(w["masks"])
    kind, kern = _workload_kernel(w)
    run = f"python3 bench.py --workload {workload} {TRAFFIC_RUN_ARGS}"
    copy = f"python3 bench.py --calibrate-copy {copy_mib} --steps 3"
    kib = copy_mib * 1024.0
    fc = statistics.median(_counter_values(os.path.join(pmc_dir, "FETCH_SIZE_copy"), "FETCH_SIZE", "copyBuffer"))
    wc = statistics.median(_counter_values(os.path.join(pmc_dir, "WRITE_SIZE_copy"), "WRITE_SIZE", "copyBuffer"))
    fs, ws = kib / fc, kib / wc
    fv = _counter_values(os.path.join(pmc_dir, f"FETCH_SIZE_{workload}"), "FETCH_SIZE", kern)[GROUPED_DISPATCHES]
    wv = _counter_values(os.path.join(pmc_dir, f"WRITE_SIZE_{workload}"), "WRITE_SIZE", kern)[GROUPED_DISPATCHES]
    f, wr = statistics.median(fv), statistics.median(wv)
    hbm = (f * fs + wr * ws) * 1024
    alg = _io_bytes(w) * len(w["masks"])
    cmds = "\n".join(
        f"rocprofv3 --pmc {c} --output-format csv -d {pmc_dir}/{c}_{tag} -o run -- {cmd}"
        for tag, cmd in ((workload, run), ("copy", copy)) for c in ("FETCH_SIZE", "WRITE_SIZE"))
    shown = kern + (">" if "<" in kern else "")
    txt = f"""# {shown}, {workload} grouped launch ({label}) — HBM traffic per launch

{WORKLOADS[workload]}.

Commands (from the repository root, one MI355X; each counter in its own pass), then
`python3 bench.py --traffic-summary {pmc_dir} --workload {workload}`:

```
{cmds}
```

kernel_source_sha256_16: {_kernel_hash(kind)}

Calibration with a plain {copy_mib} MiB device copy ({kib:,.0f} KiB read and written):

- FETCH_SIZE reads {fc:.1f} KiB per copy -> scale {fs:.4f}
- WRITE_SIZE reads {wc:.1f} KiB per copy -> scale {ws:.4f}

The grouped launch (one dispatch of {shown} for all masks; median of the {len(fv)} timed dispatches):

- FETCH_SIZE {f:.1f} KiB raw -> {f * 1024 * fs / 1e6:.2f} MB
- WRITE_SIZE {wr:.1f} KiB raw -> {wr * 1024 * ws / 1e6:.2f} MB

hbm_bytes_per_launch: {hbm:.0f}
algorithmic_bytes_per_launch: {alg}  (per mask: Q, K, V read once and O written once, bf16)
ratio: {hbm / alg:.3f}
"""
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"attn_fwd_{workload}_{label}_traffic.txt")
    with open(path, "w") as fh:
        fh.write(txt)
    return path


TRACE_RUN_ARGS = "--quick --no-cpu-baseline --no-clocks --steps 10 --warmup 2 --reps 10"
TRACE_GROUPED = slice(2, 12)   # the timed grouped launches of a TRACE_RUN_ARGS run
TRACE_REPS, TRACE_MASK_WARMUP = 10, 3   # then per mask: 3 untimed and 10 timed launches alone


def _kernel_rows(path_glob: str, kernel: str):
    """(dispatch id, kernel name, duration ms) of kernels whose name contains `kernel`, dispatch order."""
    import csv
    import glob
    out = []
    for path in glob.glob(path_glob, recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6))
    return sorted(out)


def trace_summary(workload: str, trace_dir: str, out_dir: str | None = None) -> str:
    """Write profiles/<kernel>_<workload>_stats.md from a rocprofv3 --kernel-trace --stats run of this
    workload under trace_dir (the command below): the grouped launch's timed dispatches of the forward
    kernel (all masks of the workload in one dispatch) and the throughput at their average duration."""
    import statistics
    from block_sparse_softmax_amd import inputs as gen
    from block_sparse_softmax_amd._lib import Plan
    w = gen.workload(workload)
    kind, kern = _workload_kernel(w)
    rows = _kernel_rows(os.path.join(trace_dir, "**", "*kernel_trace.csv"), kern)
    if not rows:
        raise SystemExit(f"no {kern} dispatches under {trace_dir}")
    name = rows[0][1]
    durs = [d for _, _, d in rows[TRACE_GROUPED]]
    merges = [d for _, _, d in _kernel_rows(os.path.join(trace_dir, "**", "*kernel_trace.csv"),
                                           "attn_merge_kernel")]
    pairs = sum(int(Plan(m, w["L"], w["H"], w["D"]).pairs()[1]) for m in w["masks"].values())
    flops = 4.0 * w["D"] * pairs * w["B"]
    avg, med = statistics.mean(durs), statistics.median(durs)
    tf = flops / (avg * 1e-3) / 1e12
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o run -- python3 bench.py "
           f"--workload {workload} {TRACE_RUN_ARGS}")
    merge_line = ""
    if merges:
        merge_line = (f"\nThe run also holds {len(merges)} dispatches of the split-row merge "
                      f"(attn_merge_kernel), {statistics.mean(merges) * 1e3:.1f} us on average.\n")
    # each mask alone: its timed dispatches of the per-launch protocol (kernel durations, so without
    # the dispatch latency that the event-timed figures of the bench line include)
    io = _io_bytes(w)
    alone = ["", "Each mask alone (the per-launch protocol's timed dispatches; kernel durations):", "",
             "| mask | dispatches | median | min | TFLOP/s at the median | algorithmic GB/s at the median | of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    for mi, (label, m) in enumerate(w["masks"].items()):
        s0 = TRACE_GROUPED.stop + mi * (TRACE_MASK_WARMUP + TRACE_REPS) + TRACE_MASK_WARMUP
        ds = [d for _, _, d in rows[s0:s0 + TRACE_REPS]]
        if len(ds) < TRACE_REPS:
            continue
        md = statistics.median(ds)
        f_m = 4.0 * w["D"] * int(Plan(m, w["L"], w["H"], w["D"]).pairs()[1]) * w["B"]
        alone.append(f"| {label} | {len(ds)} | {md * 1e3:.1f} us | {min(ds) * 1e3:.1f} us | "
                     f"{f_m / (md * 1e-3) / 1e12:.1f} | {io / (md * 1e-3) / 1e9:.0f} | "
                     f"{io / (md * 1e-3) / 1e9 / PEAK_HBM_GBS:.3f} |")
    alone_txt = "\n".join(alone) + "\n" if len(alone) > 5 else ""
    shown = kern + (">" if "<" in kern else "")
    txt = f"""# {shown}, {workload} — kernel trace

{WORKLOADS[workload]}; masks {", ".join(w["masks"])} in one grouped launch.

Command (from the repository root, one MI355X), then
`python3 bench.py --trace-summary {trace_dir} --workload {workload}`:

```
{cmd}
```

kernel_source_sha256_16: {_kernel_hash(kind)}

| kernel | timed grouped dispatches | average | median | min | max |
|---|---|---|---|---|---|
| {name} | {len(durs)} | {avg:.4f} ms | {med:.4f} ms | {min(durs):.4f} ms | {max(durs):.4f} ms |

Effective throughput at the average duration: {flops / 1e12:.4f} TFLOP (4 d per allowed pair) / {avg:.4f} ms =
{tf:.1f} TFLOP/s = {tf / PEAK_BF16_TFLOPS:.3f} of the {PEAK_BF16_TFLOPS} TFLOP/s bf16 peak.  The kernel's
{len(rows)} dispatches of the run are 2 warm-up and 10 timed grouped launches (summarised here), then the
per-launch protocol (each mask alone, with a cache flush between launches when the working set fits the
last-level cache).
{alone_txt}{merge_line}"""
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"{kern.split('<')[0]}_{workload}_stats.md")
    with open(path, "w") as fh:
        fh.write(txt)
    return path


def kernels_summary(trace_dir: str, name: str, run_args: str, out_dir: str | None = None) -> str:
    """Write profiles/<name>_kernels.md: every kernel of a rocprofv3 --kernel-trace run of
    `python3 bench.py <run_args>` under trace_dir, with its dispatch count and durations."""
    import statistics
    rows = _kernel_rows(os.path.join(trace_dir, "**", "*kernel_trace.csv"), "")
    by = {}
    for _, kname, d in rows:
        by.setdefault(kname, []).append(d)
    cmd = f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o run -- python3 bench.py {run_args}"
    lines = [f"# Kernels of `bench.py {run_args}` — kernel trace", "",
             "Command (from the repository root, one MI355X), then",
             f"`python3 bench.py --kernels-summary {trace_dir} --summary-name {name} --run-args \"{run_args}\"`:",
             "", "```", cmd, "```", "",
             "Source hashes (sha256[:16]): " + ", ".join(
                 f"{k} {_kernel_hash(k)}" for k in KERNEL_SRC), "",
             "| kernel | calls | average (us) | median (us) | min (us) | max (us) | total (ms) |",
             "|---|---|---|---|---|---|---|"]
    for kname, ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        short = kname.replace("void ", "").replace("(anonymous namespace)::", "")
        short = short.split("(bss::")[0].split("(")[0] if "bss::" in short else short[:90]
        lines.append(f"| {short} | {len(ds)} | {statistics.mean(ds) * 1e3:.1f} | {statistics.median(ds) * 1e3:.1f} "
                     f"| {min(ds) * 1e3:.1f} | {max(ds) * 1e3:.1f} | {sum(ds):.2f} |")
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"{name}_kernels.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def counters_summary(workload: str, pmc_dir: str, out_dir: str | None = None) -> str:
    """Write profiles/<kernel>_<workload>_counters.md from two rocprofv3 passes under pmc_dir: MFMA
    utilisation and counted bf16 MFMA work (MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16), L2 hits and misses
    (TCC_HIT_sum, TCC_MISS_sum), each the median over the grouped launch's timed dispatches."""
    import statistics
    from block_sparse_softmax_amd import inputs as gen
    from block_sparse_softmax_amd._lib import Plan
    w = gen.workload(workload)
    kind, kern = _workload_kernel(w)

    def med(tag, counter):
        return statistics.median(_counter_values(os.path.join(pmc_dir, f"{tag}_{workload}"), counter,
                                                 kern)[GROUPED_DISPATCHES])
    util = med("mfma", "MfmaUtil")
    mops = med("mfma", "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
    hit, miss = med("l2", "TCC_HIT_sum"), med("l2", "TCC_MISS_sum")
    listed = 0
    pairs = 0
    for m in w["masks"].values():
        plan = Plan(m, w["L"], w["H"], w["D"])
        bm, bn, _, kv_tile, _ = plan.tiles()
        listed += len(kv_tile) * bm * bn
        pairs += int(plan.pairs()[1])
    # per listed pair: 2 d for the score, 2 d' for the value mix, d' = d rounded up to 32 (the
    # output tiles of the value MFMAs; d = 80 runs 96 rows)
    d_out = 32 * ((w["D"] + 31) // 32)
    listed_flops = 2.0 * (w["D"] + d_out) * listed * w["B"]
    alg = 4.0 * w["D"] * pairs * w["B"]
    run = f"python3 bench.py --workload {workload} {TRAFFIC_RUN_ARGS}"
    shown = kern + (">" if "<" in kern else "")
    txt = f"""# {shown}, {workload} grouped launch — MFMA utilisation, MFMA work, L2 hit rate

{WORKLOADS[workload]}.

Commands (from the repository root, one MI355X; one pass each), then
`python3 bench.py --counters-summary {pmc_dir} --workload {workload}`:

```
rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv -d {pmc_dir}/mfma_{workload} -o run -- {run}
rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv -d {pmc_dir}/l2_{workload} -o run -- {run}
```

kernel_source_sha256_16: {_kernel_hash(kind)}

Per grouped launch (median of the timed dispatches):

| measure | value |
|---|---|
| MfmaUtil (rocprofv3's derived metric: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) | {util:.1f} % |
| MFMA work counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) | {mops / 1e12:.4f} TFLOP |
| MFMA work of the listed 128 x 64 tiles (2 d + 2 d' per pair, d' = {d_out}) | {listed_flops / 1e12:.4f} TFLOP |
| algorithmic work (4 d per allowed pair) | {alg / 1e12:.4f} TFLOP |
| L2 hits / misses (TCC_HIT_sum, TCC_MISS_sum) | {hit / 1e9:.3f} G / {miss / 1e9:.3f} G |
| L2 hit rate | {100 * hit / max(hit + miss, 1):.1f} % |
"""
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"{kern.split('<')[0]}_{workload}_counters.md")
    with open(path, "w") as fh:
        fh.write(txt)
    return path


def _clocks_under_load(setup, layout, sampler, seconds=3.0):
    """Sample the clocks and power while about `seconds` of the workload's launches are queued on
    the GPU (the sample is taken two thirds of the way in, once power and clocks have settled)."""
    import torch
    from block_sparse_softmax_amd import bind_group
    q, k, v = setup["dev"]
    ms = setup["masks"]
    n = len(ms)
    group = bind_group([m["pm"] for m in ms], [q] * n, [k] * n, [v] * n, [m["o"] for m in ms],
                       sinks=[setup["sink"]] * n, layout=layout)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    group()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-4)
    for _ in range(max(1, int(seconds / one))):
        group()
    time.sleep(2.0 * seconds / 3)
    c = sampler()
    torch.cuda.synchronize()
    return c


def _bits_to_dev(u16, device, layout):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)
    if layout == "blhd":
        t = t.permute(0, 2, 1, 3).contiguous()
    return t.to(device)


def _setup(name, device, layout):
    import torch
    from block_sparse_softmax_amd import inputs as gen
    from block_sparse_softmax_amd import prepare
    w = gen.workload(name)
    q, k, v = gen.qkv_bf16(0, w["cfg"], w["B"], w["H"], w["L"], w["D"], w["Hkv"])
    dev = [_bits_to_dev(x, device, layout) for x in (q, k, v)]
    sink = None if w["sink"] is None else torch.from_numpy(w["sink"]).to(device)
    masks = []
    for label, mask in w["masks"].items():
        pm = prepare(mask, w["L"], w["H"], w["D"], device)
        _, pairs = pm.plan.pairs()
        bm, bn, _, kv_tile, _ = pm.plan.tiles()
        masks.append(dict(label=label, mask=mask, pm=pm, pairs=int(pairs), tiles=int(len(kv_tile)), tile_pairs=bm * bn,
                          o=torch.empty_like(dev[0])))
    # bytes a launch of one mask touches: Q, K, V read and O written (bf16)
    ws_bytes = _io_bytes(w)
    return dict(w=w, host=(q, k, v), dev=dev, sink=sink, masks=masks, name=name,
                flush=ws_bytes * len(masks) < LLC_BYTES)


def _io_bytes(w) -> int:
    """Algorithmic bytes of one launch: Q, K, V read once and O written once (bf16)."""
    return 2 * w["B"] * w["L"] * w["D"] * (2 * w["H"] + 2 * w["Hkv"])


def _events(n):
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:             # a torch event exists once it has been recorded
        a.record()
        b.record()
    return ev


class _Flusher:
    """Rewrites a 512 MiB scratch buffer (read and write of every byte), evicting the last-level cache
    and the L2s before the next launch."""

    def __init__(self, device):
        import torch
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=device)

    def __call__(self):
        self.buf.add_(1)


def _stats(t):
    import numpy as np
    t = np.asarray(t, dtype=np.float64)
    return dict(avg_ms=float(t.mean()), median_ms=float(np.median(t)), min_ms=float(t.min()), n=int(t.size))


def _time(setup, steps, warmup, layout, flusher=None, warm_s=0.0, reps=20):
    """Time `steps` steps back to back.  A step is ONE grouped launch (attn_masked_fwd_group) of every
    mask of the workload, each mask writing its own output; the step time is the host wall clock
    between two device synchronisations, and the launch durations come from HIP events that the
    launch attaches to its own dispatch (nothing is recorded between the kernels).

    Then the per-launch protocol: each mask alone, `reps` launches each timed by its events; with a
    flusher (workloads that fit in the last-level cache) the scratch buffer is rewritten before every
    launch, so every launch starts from cold caches."""
    import torch
    from block_sparse_softmax_amd import bind_group
    q, k, v = setup["dev"]
    sink = setup["sink"]
    ms = setup["masks"]
    stream = torch.cuda.current_stream()
    n = len(ms)
    group = bind_group([m["pm"] for m in ms], [q] * n, [k] * n, [v] * n, [m["o"] for m in ms],
                       sinks=[sink] * n, layout=layout, stream=stream)
    for _ in range(warmup):
        group()
    if warm_s > 0:   # keep launching until the clocks have settled
        torch.cuda.synchronize()
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < warm_s:
            group()
            torch.cuda.synchronize()
    ev = _events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        group(*ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_group = [a.elapsed_time(b) for a, b in ev]  # ms

    def protocol(f):
        for _ in range(3):
            f()
        e1 = _events(reps)
        for a, b in e1:
            if flusher is not None:
                flusher()
            f(a, b)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in e1]

    per_mask = [protocol(m["pm"].bind(q, k, v, m["o"], sink=sink, layout=layout, stream=stream)) for m in ms]
    grouped_cold = protocol(group) if (flusher is not None and n > 1) else None
    return wall, per_group, per_mask, grouped_cold


def _summarise(setup, wall, per_group, per_mask, steps, grouped_cold=None):
    w = setup["w"]
    D = w["D"]
    rows = []
    for m, t in zip(setup["masks"], per_mask):
        flops = 4.0 * D * m["pairs"] * w["B"]
        st = _stats(t)
        med = st["median_ms"] * 1e-3
        computed = float(m["tiles"]) * m["tile_pairs"] * w["B"]   # pairs inside listed tiles: one exp each
        rows.append(dict(mask=m["label"], pairs=m["pairs"], **st, cold_caches=setup["flush"],
                         tflops=flops / med / 1e12, frac_bf16_peak=flops / med / 1e12 / PEAK_BF16_TFLOPS,
                         alg_gbs=_io_bytes(w) / med / 1e9,
                         frac_hbm=_io_bytes(w) / med / 1e9 / PEAK_HBM_GBS,
                         listed_tiles=m["tiles"], tile_efficiency=m["pairs"] * w["B"] / computed,
                         exp_per_s=computed / med))
    total_flops = sum(4.0 * D * m["pairs"] * w["B"] for m in setup["masks"])
    ms_per_step = wall / steps * 1e3
    group = dict(**_stats(per_group), masks=[m["label"] for m in setup["masks"]], back_to_back=True)
    if grouped_cold is not None:
        group["cold_caches"] = _stats(grouped_cold)
    return rows, total_flops, ms_per_step, group


def _roofline(setup, group, total_flops, workload):
    """Roofline object for the step's kernel (the launch of all masks of the workload): achieved =
    algorithmic flops / the mean event duration of the timed launches."""
    w = setup["w"]
    achieved = total_flops / (group["avg_ms"] * 1e-3) / 1e12
    label = "+".join(group["masks"])
    # a grouped launch runs the ping-pong kernel only when every plan picks it
    kinds = [m["pm"].plan.kernel() for m in setup["masks"]]
    kind = kinds[0] if all(k == kinds[0] for k in kinds) else "single"
    return dict(bound="mfma", achieved=achieved, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=achieved / PEAK_BF16_TFLOPS, traffic=_traffic_from_profile(workload, label, kind),
                kernel=(_kernel_name(kind, w["D"]) + (">" if kind != "pingpong" else "") +
                        f" ({workload}: {', '.join(group['masks'])})"),
                avg_launch_ms=group["avg_ms"], median_launch_ms=group["median_ms"],
                frac_at_median=total_flops / (group["median_ms"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def _cpu_baseline(setup, budget_s=20.0, rows_per_head=512):
    """The float64 oracle on `rows_per_head` seeded query rows per head (the sampled rows of the
    largest configs), head after head until about `budget_s` of host time, through every mask of the
    workload.  Reports the useful rate (4 d flops per allowed pair in the evaluated rows), the
    performed rate (the oracle is dense-then-mask: 4 d L flops per row), the cores, and the
    full-config time extrapolated from the per-row time."""
    import numpy as np
    from block_sparse_softmax_amd import inputs as gen
    from oracle.attention import attention
    w = setup["w"]
    q, k, v = setup["host"]
    D, H, L, B = w["D"], w["H"], w["L"], w["B"]
    n = min(rows_per_head, L)
    rows_all = gen.sampled_rows(0, w["cfg"], H, L, n)
    useful = performed = 0.0
    done_s, heads = 0.0, 0
    for h in range(H):
        t0 = time.perf_counter()
        for m in setup["masks"]:
            mask = dict(m["mask"])
            if mask.get("kind") == "block":
                mask["block_mask"] = np.asarray(mask["block_mask"])[h:h + 1]
            if mask.get("head_left") is not None:
                mask["head_left"] = np.asarray(mask["head_left"])[h:h + 1]
            hk = h // (H // w["Hkv"])          # the K/V head of query head h
            r = attention(q[:, h:h + 1], k[:, hk:hk + 1], v[:, hk:hk + 1], mask,
                          sink=None if w["sink"] is None else w["sink"][h:h + 1], rows=rows_all[h:h + 1],
                          row_chunk=64)
            useful += 4.0 * D * float(r["pairs"].sum()) * B
            performed += 4.0 * D * L * n * B
        done_s += time.perf_counter() - t0
        heads += 1
        if done_s >= budget_s:
            break
    rows_done = heads * n
    full_s = done_s / rows_done * (H * L)
    return dict(value=useful / done_s / 1e12, unit="TFLOP/s (effective, unmasked pairs)",
                cores=int(_blas_threads()), kind="oracle",
                sample=f"{n} seeded query rows per head on {heads} of {H} heads ({rows_done} rows) through "
                       f"{'every mask' if len(setup['masks']) > 1 else 'the mask'} of the {L}-token workload, "
                       f"float64 numpy, {done_s:.1f} s",
                performed_gflops=performed / done_s / 1e9, seconds=done_s,
                full_config_seconds_extrapolated=full_s)


def _bench_rr(q, k, steps, warmup, layout, stride=8, block=128, tau=0.9):
    """RRAttention's block-pattern search on the 128K-token Q, K (all heads): events around its
    kernels (prep, key-norm maximum, single pass with the block scores, recompute of flagged tiles,
    select).  Algorithmic work: the stride importance GEMM of Eq. 8 once over the causal stride pairs
    (2 d flops per pair); bytes: Q's sampled rows and K read once, the block scores and block matrix
    written once."""
    import numpy as np
    import torch
    from block_sparse_softmax_amd import RrSearch
    srch = RrSearch(q, stride, block, tau, layout=layout)
    for _ in range(max(1, warmup)):
        srch(q, k)
    ev = _events(steps)
    torch.cuda.synchronize()
    for a, b in ev:
        srch(q, k, start_event=a, stop_event=b)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    B, H, L, D = (q.shape[0], q.shape[1], q.shape[2], q.shape[3]) if layout == "bhld" else \
        (q.shape[0], q.shape[2], q.shape[1], q.shape[3])
    ns = L // stride
    nb = -(-L // block)
    flops = 2.0 * D * B * H * ns * (ns + 1) / 2
    nbytes = B * H * (ns * D * 2 + L * D * 2 + nb * nb * 5)
    avg = float(np.mean(t))
    med = float(np.median(t))
    density = float(srch.block_mask.float().mean().item() * 2)
    return dict(workload=f"RRAttention block-pattern search (Eq. 6-12): L={L}, {H} heads, d={D}, stride {stride}, "
                         f"block {block}, tau {tau}; synthetic Q, K of the 128K block-sparse workload",
                avg_ms=avg, median_ms=med, min_ms=float(np.min(t)), n=len(t), tflops=flops / (avg * 1e-3) / 1e12,
                frac_at_median=flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                frac_bf16_peak=flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                alg_gbs=nbytes / (avg * 1e-3) / 1e9, kept_causal_fraction=density,
                roofline=dict(bound="mfma", achieved=flops / (avg * 1e-3) / 1e12, peak=PEAK_BF16_TFLOPS,
                              unit="TFLOP/s", frac=flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, traffic=None,
                              kernel="rr_prep + rr_kmax + rr_scores1p + rr_scores (flagged tiles) + rr_select",
                              avg_launch_ms=avg, median_launch_ms=med))


def _bench_reorder(xs, gh, gw, steps, layout):
    """Re-permute the layer's Q, K and V from the 2 x 2-block row-major to the column-major order
    (Ariadne's switch between layer orders): algorithmic bytes = every token row read and written
    once, per tensor."""
    import numpy as np
    import torch
    from block_sparse_softmax_amd import reorder_tokens
    outs = [torch.empty_like(x) for x in xs]
    for x, o in zip(xs, outs):
        reorder_tokens(x, "block_row", "block_col", gh, gw, out=o, layout=layout)
    ev = _events(steps * len(xs))
    torch.cuda.synchronize()
    for s in range(steps):
        for i, (x, o) in enumerate(zip(xs, outs)):
            a, b = ev[s * len(xs) + i]
            reorder_tokens(x, "block_row", "block_col", gh, gw, out=o, layout=layout, start_event=a, stop_event=b)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    avg = float(np.mean(per))
    nbytes = 2 * xs[0].numel() * xs[0].element_size()
    gbs = nbytes / (avg * 1e-3) / 1e9
    return dict(workload=f"token re-permutation 2x2-block row-major -> column-major, {gh}x{gw} grid, "
                         f"tensor {tuple(xs[0].shape)} bf16 ({layout}), Q, K and V",
                avg_ms=avg, min_ms=float(np.min(per)), alg_gbs=gbs,
                roofline=dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s", frac=gbs / PEAK_HBM_GBS,
                              traffic=None, kernel="reorder_kernel", avg_launch_ms=avg))


def _bench_bwd(name, device, steps, layout):
    """Backward of every mask of a workload (the masks the pages train): attn_masked_fwd_lse once, then
    attn_masked_bwd timed with events attached to its first and last kernel.  Algorithmic work per allowed
    pair: 10 d flops (five products of 2 d: the scores, dP = dO V^T, dV, dK and dQ); the kernels
    recompute the scores and dP once more each (14 d performed).  Bytes: Q, K, V, O, dO read and dQ,
    dK, dV written once (bf16), the row statistics are negligible."""
    import numpy as np
    import torch
    from block_sparse_softmax_amd import inputs as gen
    from block_sparse_softmax_amd import prepare_backward
    w = gen.workload(name)
    B, H, L, D = w["B"], w["H"], w["L"], w["D"]
    q, k, v = (_bits_to_dev(x, device, layout) for x in gen.qkv_bf16(0, w["cfg"], B, H, L, D))
    g = torch.Generator(device="cpu").manual_seed(7)
    dout = (torch.randn(q.shape, generator=g) * 0.05).to(torch.bfloat16).to(device)
    sink = None if w["sink"] is None else torch.from_numpy(w["sink"]).to(device)
    rows, tot_flops, tot_ms = [], 0.0, 0.0
    for label, mask in w["masks"].items():
        pb = prepare_backward(mask, L, H, D, B, H, device)
        _, pairs = pb.plan.pairs()
        o, lse = torch.empty_like(q), torch.empty((B, H, L), dtype=torch.float32, device=device)
        pb.bind_forward(q, k, v, o, lse, sink=sink, layout=layout)()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dsink = None if sink is None else torch.empty(H, dtype=torch.float32, device=device)
        f = pb.bind_backward(q, k, v, o, dout, lse, dq, dk, dv, sink=sink, dsink=dsink, layout=layout)
        f()
        ev = _events(steps)
        torch.cuda.synchronize()
        for a, b in ev:
            f(a, b)
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in ev]
        avg = float(np.mean(t))
        flops = 10.0 * D * float(pairs) * B
        tot_flops += flops
        tot_ms += avg
        rows.append(dict(mask=label, pairs=int(pairs), avg_ms=avg, min_ms=float(np.min(t)),
                         tflops=flops / (avg * 1e-3) / 1e12,
                         frac_bf16_peak=flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         alg_gbs=(8 * B * H * L * D * 2) / (avg * 1e-3) / 1e9))
        del pb, o, lse, dq, dk, dv
    ach = tot_flops / (tot_ms * 1e-3) / 1e12
    return dict(workload=WORKLOADS[name] + " -- backward (dQ, dK, dV, sink gradient), 10 d flops per allowed pair",
                masks=rows, tflops=ach, frac_bf16_peak=ach / PEAK_BF16_TFLOPS,
                roofline=dict(bound="mfma", achieved=ach, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=ach / PEAK_BF16_TFLOPS, traffic=None,
                              kernel=f"bwd_prep + bwd_dq + bwd_dkdv + bwd_sink, d = {D}, masks run one after another",
                              avg_launch_ms=tot_ms / len(rows)))


def _bench_decode(name, device, steps, layout="blhd"):
    """One decode step (attn_decode_fwd) over the sequences of a decode workload: caches resident on the
    device (every row outside the filled window / prefix holds NaN), events on the launch.  Algorithmic
    bytes: the K and V rows of every allowed key of every sequence read once, the queries read and the
    outputs written once (bf16)."""
    import numpy as np
    import torch
    from block_sparse_softmax_amd import PreparedDecode
    from block_sparse_softmax_amd import inputs as gen
    w = gen.decode_workload(name)
    B, H, Hkv, D, L, W, P = w["B"], w["H"], w["Hkv"], w["D"], w["Lmax"], w["window"], w["prefix"]
    # caches [B, Lmax, Hkv, D] ('blhd', a token's heads side by side) or [B, Hkv, Lmax, D] ('bhld')
    shape = (B, L, Hkv, D) if layout == "blhd" else (B, Hkv, L, D)
    kc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)
    vc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)
    for b in range(B):
        pos, kr, vr = gen.decode_cache_rows(0, w["cfg"], b, int(w["lens"][b]), Hkv, D, P, W if W > 0 else L)
        idx = torch.as_tensor(pos, device=device)
        if layout == "blhd":
            kc[b].index_copy_(0, idx, _bits_to_dev(kr.transpose(1, 0, 2)[None], device, "bhld")[0])
            vc[b].index_copy_(0, idx, _bits_to_dev(vr.transpose(1, 0, 2)[None], device, "bhld")[0])
        else:
            kc[b].index_copy_(1, idx, _bits_to_dev(kr[None], device, "bhld")[0])
            vc[b].index_copy_(1, idx, _bits_to_dev(vr[None], device, "bhld")[0])
    q = _bits_to_dev(gen.decode_queries(0, w["cfg"], B, H, D)[None], device, "bhld")[0]
    lens = torch.as_tensor(w["lens"], device=device)
    sink = None if w["sink"] is None else torch.as_tensor(w["sink"], device=device)
    out = torch.empty_like(q)
    pd = PreparedDecode(q, kc, L, W, P, layout=layout)
    f = pd.bind(q, kc, vc, lens, out, sink=sink)
    for _ in range(3):
        f()
    ev = _events(steps)
    torch.cuda.synchronize()
    for a, b in ev:
        f(a, b)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    n = w["lens"].astype(np.int64)
    lo = np.maximum(0, n - W) if W > 0 else np.zeros_like(n)
    keys = np.minimum(np.minimum(P, n), lo) + (n - lo)            # window plus the prefix keys outside it
    nbytes = float(keys.sum()) * Hkv * D * 2 * 2 + 2.0 * B * H * D * 2
    avg = float(np.mean(t))
    gbs = nbytes / (avg * 1e-3) / 1e9
    del kc, vc
    torch.cuda.empty_cache()
    win = f"window {W}" if W > 0 else "full causal"
    return dict(workload=f"decode step: {B} sequences of {int(n.min())}..{int(n.max())} cached tokens, {H} query heads "
                         f"on {Hkv} K/V heads, d={D}, {win}, cache {layout}" + (f" + {P} prefix tokens" if P else "")
                         + (", sink per head" if sink is not None else ""),
                avg_ms=avg, min_ms=float(np.min(t)), alg_bytes=nbytes, alg_gbs=gbs,
                sequences_per_s=B / (avg * 1e-3), splits=None if pd.workspace_bytes == 0 else "split keys + merge",
                roofline=dict(bound="hbm", achieved=gbs, peak=PEAK_HBM_GBS, unit="GB/s", frac=gbs / PEAK_HBM_GBS,
                              traffic=None, kernel=f"decode_kernel<{D}>" + (" + decode_combine_kernel"
                                                                           if pd.workspace_bytes else ""),
                              avg_launch_ms=avg))


def _workload_block(name, device, layout, steps, warmup, flusher, warm_s):
    """Time one workload of the catalogue (back-to-back steps and the per-launch protocol)."""
    setup = _setup(name, device, layout)
    wall, pg, pm, gc = _time(setup, steps, warmup, layout, flusher=flusher if setup["flush"] else None,
                             warm_s=warm_s)
    rows, flops, ms, group = _summarise(setup, wall, pg, pm, steps, gc)
    return setup, rows, flops, ms, group


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layout", default="bhld", choices=["blhd", "bhld"],
                    help="bhld = [B, H, L, D] (each head contiguous), blhd = [B, L, H, D]")
    ap.add_argument("--quick", action="store_true", help="skip the extra workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--only", default=None, help="time only this mask of the workload (profiling)")
    ap.add_argument("--decode-only", action="store_true", help="run only the decode workloads (profiling)")
    ap.add_argument("--no-clocks", action="store_true", help="do not sample the GPU clocks")
    ap.add_argument("--decode-layout", default="blhd", choices=["blhd", "bhld"],
                    help="K/V cache layout of the decode workloads")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run only a plain device copy of MIB mebibytes (counter calibration)")
    ap.add_argument("--reps", type=int, default=20, help="launches per mask in the per-launch protocol")
    ap.add_argument("--kernels-summary", default=None, metavar="DIR",
                    help="summarise every kernel of a rocprofv3 kernel trace under DIR into profiles/ (no GPU)")
    ap.add_argument("--summary-name", default="bench", help=argparse.SUPPRESS)
    ap.add_argument("--run-args", default="", help=argparse.SUPPRESS)
    ap.add_argument("--counters-summary", default=None, metavar="DIR",
                    help="summarise rocprofv3 MFMA and L2 counter passes under DIR into profiles/ (no GPU)")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="summarise a rocprofv3 kernel trace of the workload under DIR into profiles/ (no GPU)")
    ap.add_argument("--traffic-summary", default=None, metavar="DIR",
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE passes under DIR into profiles/ (no GPU)")
    ap.add_argument("--device", default="cuda:0", help=argparse.SUPPRESS)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the kernel shards by head with no exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if args.kernels_summary:
        print(kernels_summary(args.kernels_summary, args.summary_name, args.run_args))
        return
    if args.counters_summary:
        print(counters_summary(args.workload, args.counters_summary))
        return
    if args.trace_summary:
        print(trace_summary(args.workload, args.trace_summary))
        return
    if args.traffic_summary:
        print(traffic_summary(args.workload, args.traffic_summary))
        return
    if args.calibrate_copy:
        # counter calibration under a profiler: nothing else runs and no other process is started
        print(json.dumps(calibrate_copy(args.calibrate_copy, args.steps, args.device)))
        return

    sampler = ClockSampler(enabled=not args.no_clocks)   # before anything touches the GPU
    try:
        _run(args, sampler)
    finally:
        sampler.close()


def _progress(msg: str):
    """One line per phase on stderr (the JSON result goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _run(args, sampler):
    import torch
    device = torch.device(args.device)
    clocks = dict(idle_before=sampler())
    from block_sparse_softmax_amd import load_library
    load_library()

    if args.decode_only:
        from block_sparse_softmax_amd.inputs import DECODE_WORKLOADS
        print(json.dumps({name: _bench_decode(name, device, args.steps, args.decode_layout)
                          for name in DECODE_WORKLOADS}))
        return

    flusher = _Flusher(device)
    _progress(f"setting up {args.workload}")
    setup = _setup(args.workload, device, args.layout)
    _progress(f"timing {args.workload}")
    if args.only:
        setup["masks"] = [m for m in setup["masks"] if m["label"] == args.only]
    wall, per_group, per_mask, gc = _time(setup, args.steps, args.warmup, args.layout,
                                          flusher=flusher if setup["flush"] else None, reps=args.reps)
    rows, total_flops, ms_per_step, group = _summarise(setup, wall, per_group, per_mask, args.steps, gc)
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    roof = _roofline(setup, group, total_flops, args.workload)
    if args.workload == "blocksparse128k" and not args.no_clocks:
        c = clocks["under_load_blocksparse128k"] = _clocks_under_load(setup, args.layout, sampler)
        if c and c.get("gfx_mhz_mean"):
            # context only: the bf16 peak at the clock the chip sustains under this load
            pk = PEAK_BF16_TFLOPS * c["gfx_mhz_mean"] / 2400.0
            roof["peak_at_load_clock"] = pk
            roof["frac_at_load_clock"] = roof["achieved"] / pk
            roof["socket_watts_under_load"] = c.get("socket_watts")

    if not args.no_cpu_baseline:
        _progress("cpu baseline (oracle on sampled rows)")
    cpu = None if args.no_cpu_baseline else _cpu_baseline(setup)

    extra = {}
    if not args.quick:
        if args.workload == "blocksparse128k":
            q, k, _ = setup["dev"]
            _progress("pattern search")
            extra["rr_search128k"] = _bench_rr(q, k, 10, 3, args.layout)
            del q, k
        del setup
        torch.cuda.empty_cache()
        for name in ("vit896", "vit1792", "lm_headwin", "blocksparse128k", "swa576_d256"):
            if name == args.workload:
                continue
            _progress(f"extra workload {name}")
            s2, r2, tf2, ms2, g2 = _workload_block(name, device, args.layout, max(5, args.steps // 2),
                                                   args.warmup, flusher, warm_s=0.2)
            extra[name] = dict(workload=WORKLOADS[name], ms_per_step=ms2, tflops=tf2 / (ms2 * 1e-3) / 1e12,
                               frac_bf16_peak=tf2 / (ms2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, masks=r2,
                               grouped_launch=g2, roofline=_roofline(s2, g2, tf2, name))
            if name == "vit1792":
                extra["reorder_vit1792"] = _bench_reorder(list(s2["dev"]), 128, 128, 5, args.layout)
            del s2
            torch.cuda.empty_cache()
        for name in ("vit896", "lm_headwin"):
            _progress(f"backward {name}")
            extra[f"backward_{name}"] = _bench_bwd(name, device, 5, args.layout)
        _progress("decode workloads")
        from block_sparse_softmax_amd.inputs import DECODE_WORKLOADS
        for name in DECODE_WORKLOADS:
            extra[name] = _bench_decode(name, device, 10)

    out = {
        "metric": "effective attention TFLOP/s (unmasked pairs) and % bf16 MFMA peak, 1 MI355X",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q, K, V rounded to bf16)",
        "config": {"workload": WORKLOADS[args.workload] + (f" (mask {args.only} only)" if args.only else ""),
                   "layout": args.layout, "frac_bf16_peak": value / PEAK_BF16_TFLOPS},
        "grouped_launch": group,
        "per_mask": rows,
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
        "gpu_clocks": dict(clocks, after=sampler()),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
