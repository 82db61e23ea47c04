#!/usr/bin/env python3
"""Throughput of the fused causal GQA attention path (forward + backward) on one MI355X.

One *step* is one pass of the whole hot path over one batch of synthetic input:
attn_fwd, then attn_bwd_preprocess and attn_bwd_dkdv_dq (dK/dV and dQ
co-launched in one grid) -- the launches attn_bwd makes -- on the stream torch
treats as current.  The separate attn_bwd_dkdv and attn_bwd_dq are timed in the
per-kernel pass and reported too.
The default workload is one layer of the 101.7M decoder of "Training a 100M
transformer in pure Rust: RustingBrain vs PyTorch and TensorFlow" (section
"The setup": GQA 12/4, head_dim 64) at the 4 x 1024 batch shape.

Timing protocol: the correctness gate runs first (finite outputs, bitwise-equal
hashes over repeated runs, exact-math invariants of the gradients), then each
kernel alone (back-to-back launches between two HIP events) to find the
dominant one, then ``--warmup`` untimed steps right before the timed region (the
step time falls by a few percent over the first ~10 ms of continuous load as
the GPU's clocks settle, so the default warmup covers 18 ms), then exactly ``--steps`` steps between
two device synchronisations, with HIP events around the dominant kernel in every
8th step, so its average duration inside the steps gives the roofline figure
without serialising the other launches (an event pair costs its step ~2 us);
then 5 trials of 10 steps, each between two HIP events, for the spread
(``trials``: per-trial us per step, mean, min, max).  ``value`` is algorithmic
TFLOP/s (4*D forward + 10*D backward flops per unmasked (query, key) pair and
query head) over the wall-clock time of the timed steps, inputs resident in HBM.

The cpu_baseline leg times the fp64 numpy oracle on a bounded sample of
(batch, KV-group) units of the same workload on the host cores, and compares
its outputs with the GPU's on those units.

With ``--rope`` the step is the rotary variant instead: attn_fwd_rope, then
attn_bwd_rope (its preparation kernel -- delta and the rotated q', k' -- and the
co-launched dK/dV + dQ grid on q', k'), with cos / sin tables of base 10000.

With ``--unfused`` the step is the unfused baseline of libattn_unfused.so
(attn_unfused_fwd + attn_unfused_bwd: float32 [T, T] scores from rocBLAS GEMMs
and the three softmax row kernels); its roofline object covers the dominant
row kernel against HBM bandwidth, each row kernel timed alone by HIP events
around back-to-back launches on the step's buffers.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rope | --unfused]
Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 4096 bf16 flop/clk/CU (dense MFMA) x 2.4 GHz
PEAK_HBM_GBS = 8000.0      # HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_sources_digest() -> str:
    """SHA-256 over the kernel sources (not the C-ABI validation layer) with their
    comments removed and white space collapsed: identifies the kernels whose
    counters were taken, and stays the same when only a comment or the layout of
    the text changes."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "reproducible_causal_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")) and name != "attn_api.hip":
            text = open(os.path.join(csrc, name), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = " ".join(re.sub(r"//[^\n]*", "", text).split())
            h.update(name.encode())
            h.update(text.encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, if current."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("sources_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


def load_kernel_time(kernel: str, workload: str, digest: str):
    """Average rocprofv3 duration (us) of one launch of ``kernel`` on ``workload`` from
    the committed kernel-trace summaries, if taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("sources_digest") != digest:
        return None
    return rec.get("avg_us")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Samples the GPU's current graphics (shader) clock through amdsmi from a host
    thread while the GPU runs; reports the median of the samples in MHz, or None
    where amdsmi is unavailable."""

    def __init__(self, period_s: float = 0.004):
        import threading
        self.period_s, self.samples, self._stop = period_s, [], threading.Event()
        self._thread, self._handle, self._amdsmi = None, None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if handles:
                self._amdsmi, self._handle = amdsmi, handles[0]
                self._read()
        except Exception as e:  # amdsmi missing, no permission, or no device
            log("clock sampling unavailable:", repr(e)[:120])
            self._amdsmi = None

    def _read(self):
        info = self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)
        return float(info["clk"])

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                return
            self._stop.wait(self.period_s)

    def __enter__(self):
        import threading
        if self._amdsmi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self):
        """Median, min and max over the second half of the samples (the reading lags
        the load by tens of milliseconds); `steady` is False when the readings moved by
        more than 20% of their maximum (normal DPM steps move them ~12%), in which case no
        single clock describes the run."""
        if not self.samples:
            return None
        import statistics
        late = self.samples[len(self.samples) // 2:]
        lo, hi = min(late), max(late)
        return {"median_mhz": statistics.median(late), "min_mhz": lo,
                "max_mhz": hi, "samples": len(late), "steady": hi - lo <= 0.2 * hi,
                "source": "amdsmi GFX clock, sampled every ~4 ms while the step runs back "
                          "to back for --clock-seconds after the timed region (second half "
                          "of the samples)"}


def summarize_rocprof(stats_csv: str, workload: str, command: str, digest: str | None) -> int:
    """Write profiles/kernels_<workload>.md from a rocprofv3 --kernel-trace --stats
    kernel_stats.csv and record the hot-path kernels' average durations, with the
    digest of the kernel sources they ran (the profiled bench line's
    ``sources_digest``; default: the current tree's), in profiles/kernel_times.json."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    digest = digest or kernel_sources_digest()
    names = {"attn_fwd64_kernel": "fwd", "attn_fwd_kernel": "fwd", "attn_bwd_pre_kernel": "bwd_preprocess",
             "attn_bwd_dkdv_dq_kernel": "bwd_dkdv_dq", "attn_bwd_dkdv_kernel": "bwd_dkdv",
             "attn_bwd_dq_kernel": "bwd_dq", "attn_bwd_rope_prep_kernel": "bwd_rope_prep"}
    lines = [f"# rocprofv3 kernel statistics: {workload}", "",
             "Command (from the repository root on one MI355X; TMPDIR=/tmp):", "", "```",
             command, "```", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    times = {}
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("void ", "").replace("rca::(anonymous namespace)::", "")
        name = name.replace("rca::", "").replace("(anonymous namespace)::", "")
        avg, mn, mx = (float(r[c]) / 1e3 for c in ("AverageNs", "MinNs", "MaxNs"))
        share = 100.0 * float(r["TotalDurationNs"]) / total
        if share < 0.05:
            continue
        lines.append(f"| {name[:72]} | {r['Calls']} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {share:.1f}% |")
        for prefix, key in names.items():
            if name.startswith(prefix + "<") and key not in times:
                times[key] = {"avg_us": round(avg, 3), "calls": int(r["Calls"]), "kernel": name,
                              "sources_digest": digest}
    lines += ["", f"Kernel sources digest: `{digest}` (bench.py's `sources_digest`)."]
    out_md = os.path.join(ROOT, "profiles", f"kernels_{workload}.md")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        data = {"_note": "average rocprofv3 kernel-trace durations per launch, by workload and "
                         "kernel, with the digest of the kernel sources they were taken on"}
    data[workload] = times
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    log(f"wrote {out_md} and {path} ({len(times)} hot-path kernels)")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="gqa-4x1024")
    ap.add_argument("--layers", type=int, default=None,
                    help="also time a stack of this many independent layers (0: skip; "
                         "default 16 for gqa-4x1024, else 0)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle cpu_baseline sample (0: skip)")
    ap.add_argument("--kernel-only", default=None,
                    choices=("fwd", "bwd_preprocess", "bwd_dkdv_dq", "bwd_dkdv", "bwd_dq",
                             "fwd_rope", "bwd_rope"),
                    help="counter runs: launch only this kernel --launches times and exit")
    ap.add_argument("--launches", type=int, default=3)
    ap.add_argument("--clock-seconds", type=float, default=1.0,
                    help="seconds of back-to-back steps during which the GPU clock is sampled")
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused baseline (libattn_unfused.so) instead")
    ap.add_argument("--rope", action="store_true",
                    help="time the rotary-embedding variant (attn_fwd_rope + attn_bwd_rope)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="counter calibration: copy this many bytes device to device "
                         "--launches times and exit")
    ap.add_argument("--summarize-rocprof", default=None, metavar="KERNEL_STATS_CSV",
                    help="write profiles/kernels_<workload>.md and profiles/kernel_times.json "
                         "from a rocprofv3 --stats kernel_stats.csv, then exit")
    ap.add_argument("--command", default="",
                    help="with --summarize-rocprof: the profiled command, quoted in the summary")
    ap.add_argument("--sources-digest", default=None,
                    help="with --summarize-rocprof: sources_digest of the profiled run")
    args = ap.parse_args()
    if args.summarize_rocprof:
        return summarize_rocprof(args.summarize_rocprof, args.workload, args.command,
                                 args.sources_digest)
    if args.layers is None:
        args.layers = 16 if args.workload == "gqa-4x1024" else 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the attention path has no cross-GPU step and "
              "the benchmark runs on a single GPU; run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from reproducible_causal_attention_amd import attn as A
    from reproducible_causal_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_bytes > 0:
        # A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it
        # calibrates the counters to bytes.
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.launches):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_bytes} bytes x {args.launches}")
        return 0
    if args.unfused:
        return main_unfused(args)
    lib = A.load_library()
    w = W.WORKLOADS[args.workload]
    if w.dtype not in ("bf16", "f16"):
        print("bench.py times bf16 and f16 workloads", file=sys.stderr)
        return 2
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
    dev = torch.device("cuda:0")
    log("workload", w.name, w.label(), "|", lib.attn_build_info().decode())

    inp = W.generate(w)
    q, k, v, dO = (torch.from_numpy(getattr(inp, n).view(np.int16)).view(tdt).to(dev)
                   for n in ("q", "k", "v", "dO"))

    def buffers():
        return dict(o=torch.empty_like(q), lse=torch.empty((B, Hq, T), device=dev),
                    delta=torch.empty((B, Hq, T), device=dev), dq=torch.empty_like(q),
                    dk=torch.empty_like(k), dv=torch.empty_like(v))

    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    bf = A.ATTN_BF16 if w.dtype == "bf16" else A.ATTN_F16
    causal = int(w.causal)

    def launch(fn_name, *a):
        st = getattr(lib, fn_name)(*a)
        if st != 0:
            raise RuntimeError(f"{fn_name}: {lib.attn_status_string(st).decode()}")

    names = ("fwd", "bwd_preprocess", "bwd_dkdv_dq")  # one step, in order
    all_names = names + ("bwd_dkdv", "bwd_dq")
    rope = None
    if args.rope:
        names = all_names = ("fwd_rope", "bwd_rope")
        c_np, s_np = W.rope_tables(T, D)
        ws_bytes = int(lib.attn_bwd_rope_workspace_bytes(B, T, Hq, Hkv, D, bf))
        rope = {"cos": torch.from_numpy(c_np).to(dev), "sin": torch.from_numpy(s_np).to(dev),
                "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev), "np": (c_np, s_np)}

    def kernel(name, x, b):
        qq, kk, vv, dd = x
        if name == "fwd":
            launch("attn_fwd", qq.data_ptr(), kk.data_ptr(), vv.data_ptr(), b["o"].data_ptr(),
                   b["lse"].data_ptr(), B, T, Hq, Hkv, D, w.scale, causal, bf, s)
        elif name == "bwd_preprocess":
            launch("attn_bwd_preprocess", b["o"].data_ptr(), dd.data_ptr(), b["delta"].data_ptr(),
                   B, T, Hq, D, bf, s)
        elif name == "bwd_dkdv_dq":
            launch("attn_bwd_dkdv_dq", qq.data_ptr(), kk.data_ptr(), vv.data_ptr(), dd.data_ptr(),
                   b["lse"].data_ptr(), b["delta"].data_ptr(), b["dq"].data_ptr(),
                   b["dk"].data_ptr(), b["dv"].data_ptr(), B, T, Hq, Hkv, D, w.scale, causal,
                   bf, s)
        elif name == "bwd_dkdv":
            launch("attn_bwd_dkdv", qq.data_ptr(), kk.data_ptr(), vv.data_ptr(), dd.data_ptr(),
                   b["lse"].data_ptr(), b["delta"].data_ptr(), b["dk"].data_ptr(),
                   b["dv"].data_ptr(), B, T, Hq, Hkv, D, w.scale, causal, bf, s)
        elif name == "bwd_dq":
            launch("attn_bwd_dq", qq.data_ptr(), kk.data_ptr(), vv.data_ptr(), dd.data_ptr(),
                   b["lse"].data_ptr(), b["delta"].data_ptr(), b["dq"].data_ptr(),
                   B, T, Hq, Hkv, D, w.scale, causal, bf, s)
        elif name == "fwd_rope":
            launch("attn_fwd_rope", qq.data_ptr(), kk.data_ptr(), vv.data_ptr(),
                   rope["cos"].data_ptr(), rope["sin"].data_ptr(), b["o"].data_ptr(),
                   b["lse"].data_ptr(), B, T, Hq, Hkv, D, w.scale, causal, bf, s)
        else:  # bwd_rope: preparation kernel, then the co-launched dK/dV + dQ grid
            launch("attn_bwd_rope", qq.data_ptr(), kk.data_ptr(), vv.data_ptr(),
                   b["o"].data_ptr(), b["lse"].data_ptr(), dd.data_ptr(), rope["cos"].data_ptr(),
                   rope["sin"].data_ptr(), b["dq"].data_ptr(), b["dk"].data_ptr(),
                   b["dv"].data_ptr(), B, T, Hq, Hkv, D, w.scale, causal, bf,
                   rope["ws"].data_ptr(), rope["ws"].numel(), s)

    def step(x, bufs, mark=None, ev=None):
        """One fwd+bwd step; with mark set, events ev[0], ev[1] bracket that kernel."""
        for n in names:
            if n == mark:
                ev[0].record(stream)
            kernel(n, x, bufs)
            if n == mark:
                ev[1].record(stream)

    def digest(b):
        h = hashlib.sha256()
        for n in ("o", "lse", "dq", "dk", "dv"):
            h.update(b[n].contiguous().view(torch.uint8).cpu().numpy().tobytes())
        return h.hexdigest()

    if args.kernel_only:
        # Counter runs: inputs and the forward's outputs in place, then only the
        # named kernel.
        bufs = buffers()
        step((q, k, v, dO), bufs)
        torch.cuda.synchronize()
        for _ in range(args.launches):
            kernel(args.kernel_only, (q, k, v, dO), bufs)
        torch.cuda.synchronize()
        log(f"{args.kernel_only} x {args.launches} on {w.name}")
        return 0

    # ---- correctness gate (no oracle): finite, reproducible, invariants ----
    bufs = buffers()
    hashes = []
    for _ in range(3):
        step((q, k, v, dO), bufs)
        torch.cuda.synchronize()
        hashes.append(digest(bufs))
    outs = ("o", "lse", "dq", "dk", "dv") + (() if rope else ("delta",))  # rotary: delta in the workspace
    gate = {"finite": all(bool(torch.isfinite(bufs[n].float()).all()) for n in outs),
            "hash_repeats_equal": len(set(hashes)) == 1}
    G = Hq // Hkv
    dv32, dk32, dO32 = bufs["dv"].float(), bufs["dk"].float(), dO.float()
    # Rows of P sum to one: sum_j dv_j equals the sum of dO over the group's query rows.
    want = dO32.view(B, T, Hkv, G, D).sum(dim=(1, 3))
    got = dv32.sum(dim=1)
    gate["dv_column_sum_rel_err"] = float((got - want).abs().max() / want.abs().max())
    # Key-translation invariance: sum_j dk_j = 0, relative to the column sums of |dk|
    # (with rotary positions it holds for the gradients of the rotated keys, so
    # each dk_j is rotated forward by its position's angles first).
    if rope is not None:
        cs, sn = rope["cos"][None, :, None, :], rope["sin"][None, :, None, :]
        a, b_ = dk32[..., 0::2], dk32[..., 1::2]
        dk32 = torch.stack((a * cs - b_ * sn, a * sn + b_ * cs), dim=-1).flatten(-2)
    gate["dk_sum_rel"] = float(dk32.sum(dim=1).abs().max() / dk32.abs().sum(dim=1).max())
    gate["ok"] = (gate["finite"] and gate["hash_repeats_equal"]
                  and gate["dv_column_sum_rel_err"] < 2e-2 and gate["dk_sum_rel"] < 2e-2)
    log("gate", gate)
    if not gate["ok"]:
        print(json.dumps({"metric": "gate failed", "gate": gate}), flush=True)
        return 1

    # ---- per-kernel durations: back-to-back launches of one kernel, GPU events ----
    # (picks the dominant kernel; the timed region below re-measures that one in place)
    per_kernel_us = {}
    n_rep = max(5, min(50, args.steps // 4))
    for n in all_names:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # Queue the launches behind a ~1 ms GPU sleep so the host enqueues them
        # faster than the short kernels run: the events then time the kernels,
        # not the host's launch rate.
        torch.cuda._sleep(int(2e6))
        e0.record(stream)
        for _ in range(n_rep):
            kernel(n, (q, k, v, dO), bufs)
        e1.record(stream)
        torch.cuda.synchronize()
        per_kernel_us[n] = 1e3 * e0.elapsed_time(e1) / n_rep
    dom = max(names, key=per_kernel_us.get)

    for _ in range(args.warmup):
        step((q, k, v, dO), bufs)
    torch.cuda.synchronize()

    # ---- timed region: whole steps; the dominant kernel is bracketed by events in
    # every 8th step (each event pair adds ~2 us to its step) ----
    sampled = list(range(0, args.steps, 8))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for i in sampled}
    e_all = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_all[0].record(stream)
    for i in range(args.steps):
        if i in evs:
            step((q, k, v, dO), bufs, dom, evs[i])
        else:
            step((q, k, v, dO), bufs)
    e_all[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_us = 1e3 * float(np.mean([e[0].elapsed_time(e[1]) for e in evs.values()]))
    event_step_us = 1e3 * e_all[0].elapsed_time(e_all[1]) / args.steps
    ms_per_step = 1e3 * wall / args.steps
    flops = w.fwd_flops + w.bwd_flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    log(f"step {ms_per_step * 1e3:.1f} us wall, {event_step_us:.1f} us by events; "
        f"{tflops:.1f} TFLOP/s; kernels alone {per_kernel_us}; {dom} in the steps {dom_us:.2f} us")

    # ---- spread: 5 trials of 10 steps each, HIP events around each trial (after
    # the timed region; reported beside `value`, which the region above gives) ----
    trial_us = []
    for _ in range(5):
        et = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        et[0].record(stream)
        for _ in range(10):
            step((q, k, v, dO), bufs)
        et[1].record(stream)
        torch.cuda.synchronize()
        trial_us.append(1e3 * et[0].elapsed_time(et[1]) / 10)
    # ---- observed shader clock: the driver's GFX clock reading is refreshed too slowly
    # for a timed region of tens of milliseconds, so it is sampled while the same steps
    # run back to back for about a second (after the trials; not timed) ----
    with ClockSampler() as clock:
        t_end = time.perf_counter() + args.clock_seconds
        while time.perf_counter() < t_end:
            for _ in range(20):
                step((q, k, v, dO), bufs)
            torch.cuda.synchronize()
    trials = {"trials": 5, "steps_each": 10, "us_per_step": [round(t, 2) for t in trial_us],
              "mean": round(float(np.mean(trial_us)), 2), "min": round(min(trial_us), 2),
              "max": round(max(trial_us), 2)}
    log(f"trials (5 x 10 steps) us per step: {trials['us_per_step']}")

    # ---- roofline of the dominant kernel ----
    pairs = w.causal_pairs
    algo = {  # algorithmic work of one launch (flops, or bytes for the preprocess)
        "fwd": 4.0 * D * pairs,
        "bwd_dkdv_dq": 10.0 * D * pairs,  # the backward's own work, not the 14*D executed
        "bwd_dkdv": 8.0 * D * pairs,   # S, dP, dV, dK
        "bwd_dq": 6.0 * D * pairs,     # S and dP recomputed, dQ
        "bwd_preprocess": 2.0 * B * T * Hq * D * 2 + 4.0 * B * Hq * T,
        "fwd_rope": 4.0 * D * pairs,
        "bwd_rope": 10.0 * D * pairs,  # two launches: preparation + dK/dV + dQ grid
    }
    sec = dom_us * 1e-6
    src_digest = kernel_sources_digest()
    traffic = load_traffic(dom, w.name, src_digest)
    if dom == "bwd_preprocess":
        achieved = algo[dom] / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = algo[dom] / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["avg_launch_us"] = round(dom_us, 2)
    roof["timing"] = ("frac from HIP events around the kernel inside the timed steps "
                      "(includes one dispatch latency per launch)")
    prof_us = load_kernel_time(dom, w.name + ("+rope" if rope else ""), src_digest)
    if prof_us:
        prof_sec = prof_us * 1e-6
        if dom == "bwd_preprocess":
            prof_ach = algo[dom] / prof_sec / 1e9
            roof["frac_rocprof"] = round(prof_ach / PEAK_HBM_GBS, 4)
        else:
            prof_ach = algo[dom] / prof_sec / 1e12
            roof["frac_rocprof"] = round(prof_ach / PEAK_BF16_TFLOPS, 4)
        roof["rocprof_avg_us"] = prof_us
        roof["achieved_rocprof"] = round(prof_ach, 1)
    else:
        roof["frac_rocprof"] = None
    roof["per_kernel_frac_rocprof"] = {}
    for kname in ("fwd", "bwd_dkdv_dq", "bwd_preprocess"):
        kus = load_kernel_time(kname, w.name, src_digest) if not rope else None
        if kus:
            peak = PEAK_HBM_GBS if kname == "bwd_preprocess" else PEAK_BF16_TFLOPS
            scale_ = 1e9 if kname == "bwd_preprocess" else 1e12
            roof["per_kernel_frac_rocprof"][kname] = round(algo[kname] / (kus * 1e-6) / scale_ / peak, 4)
    if dom in ("bwd_dkdv_dq", "bwd_rope"):  # matrix work the split design executes (S and dP twice)
        roof["executed_tflops"] = round(14.0 * D * pairs / sec / 1e12, 1)
    if dom == "bwd_rope":
        roof["note"] = ("attn_bwd_rope as a whole: its preparation kernel and the co-launched "
                        "dK/dV + dQ grid, between one pair of events")
    pre_gbs = (algo["bwd_preprocess"] / (per_kernel_us["bwd_preprocess"] * 1e-6) / 1e9
               if "bwd_preprocess" in per_kernel_us else None)

    # ---- a stack of independent layers (forward 0..L-1, backward L-1..0) ----
    layers = None
    if args.layers > 0 and rope is None:
        L = args.layers
        xs = [(torch.randn_like(q, dtype=torch.float32).to(tdt),
               torch.randn_like(k, dtype=torch.float32).to(tdt),
               torch.randn_like(v, dtype=torch.float32).to(tdt),
               torch.randn_like(dO, dtype=torch.float32).to(tdt)) for _ in range(L)]
        ws_bytes_stack = int(lib.attn_bwd_workspace_bytes(B, T, Hq, Hkv, D, bf))
        bs = [dict(buffers(), ws=torch.empty(ws_bytes_stack, dtype=torch.uint8, device=dev))
              for _ in range(L)]

        def stack_step():
            for i in range(L):
                x, b = xs[i], bs[i]
                launch("attn_fwd", x[0].data_ptr(), x[1].data_ptr(), x[2].data_ptr(),
                       b["o"].data_ptr(), b["lse"].data_ptr(), B, T, Hq, Hkv, D, w.scale,
                       causal, bf, s)
            for i in reversed(range(L)):
                x, b = xs[i], bs[i]
                # attn_bwd itself: the preprocess into the workspace (this layer's
                # delta buffer), then the co-launched dK/dV + dQ grid
                launch("attn_bwd", x[0].data_ptr(), x[1].data_ptr(), x[2].data_ptr(),
                       b["o"].data_ptr(), b["lse"].data_ptr(), x[3].data_ptr(),
                       b["dq"].data_ptr(), b["dk"].data_ptr(), b["dv"].data_ptr(), B, T, Hq,
                       Hkv, D, w.scale, causal, bf, b["ws"].data_ptr(), b["ws"].numel(), s)

        for _ in range(3):
            stack_step()
        n_stack = max(3, args.steps // L)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_stack):
            stack_step()
        torch.cuda.synchronize()
        st = (time.perf_counter() - t0) / n_stack
        layers = {"layers": L, "steps": n_stack, "ms_per_step": round(st * 1e3, 4),
                  "tflops": round(L * flops / st / 1e12, 1),
                  "pct_peak": round(100 * L * flops / st / 1e12 / PEAK_BF16_TFLOPS, 2)}
        log("layer stack", layers)
        del xs, bs

    # ---- cpu_baseline: the oracle on a bounded sample of the same workload ----
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, inp, bufs, args.cpu_seconds, rope["np"] if rope else None)
        log("cpu_baseline", cpu)

    out = {
        "metric": "attn fwd+bwd TFLOP/s & % bf16 MFMA peak, B4·T1024 GQA12/4 d64",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name + ("+rope" if rope else ""), "B": B, "T": T, "Hq": Hq,
                   "Hkv": Hkv, "D": D, "causal": bool(w.causal), "scale": w.scale,
                   "gflop_per_step": round(flops / 1e9, 4),
                   **({"rope": {"pairs": "adjacent", "base": 10000.0}} if rope else {})},
        "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "per_kernel_us": {n: round(u, 2) for n, u in per_kernel_us.items()},
        "event_step_us": round(event_step_us, 2),
        "trials": trials,
        "clock": clock.summary(),
        "pct_peak_at_observed_clock": (
            round(100 * tflops / (PEAK_BF16_TFLOPS * clock.summary()["median_mhz"] / 2400.0), 2)
            if clock.summary() and clock.summary()["steady"] else None),
        "preprocess_gbs": round(pre_gbs, 1) if pre_gbs is not None else None,
        "roofline": roof,
        "cpu_baseline": cpu,
        "layers": layers,
        "gate": gate,
        "output_sha256": hashes[0],
        "sources_digest": src_digest,
        "build": lib.attn_build_info().decode(),
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)
    if cpu is not None and not cpu.get("parity_ok", True):
        return 1
    return 0


def row_kernel_bytes(name, B, T, Hq, causal):
    """Algorithmic HBM bytes of one launch of an unfused row kernel: the visible
    part of each row read (float32 scores / dP, 16-bit P), every column of the
    16-bit output written, float32 lse read or written."""
    vis = B * Hq * (T * (T + 1) // 2 if causal else T * T)
    full = B * Hq * T * T
    rows = B * Hq * T
    return {"softmax_lse": 4 * vis + 2 * full + 4 * rows,
            "probs_from_lse": 4 * vis + 4 * rows + 2 * full,
            "softmax_bwd": (2 + 4) * vis + 2 * full}[name]


def main_unfused(args) -> int:
    """The unfused baseline's step: attn_unfused_fwd + attn_unfused_bwd."""
    import numpy as np
    import torch

    from reproducible_causal_attention_amd import attn as A
    from reproducible_causal_attention_amd import unfused as U
    from reproducible_causal_attention_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    if w.dtype not in ("bf16", "f16"):
        print("the unfused baseline runs bf16 and f16 workloads", file=sys.stderr)
        return 2
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
    dev = torch.device("cuda:0")
    lib = U.load_library()
    code = A.ATTN_BF16 if w.dtype == "bf16" else A.ATTN_F16
    log("unfused baseline", w.name, w.label())
    inp = W.generate(w)
    q, k, v, dO = (torch.from_numpy(getattr(inp, n).view(np.int16)).view(tdt).to(dev)
                   for n in ("q", "k", "v", "dO"))
    ws = torch.empty(int(lib.attn_unfused_workspace_bytes(B, T, Hq, Hkv, D, code)),
                     dtype=torch.uint8, device=dev)
    bufs = dict(o=torch.empty_like(q), lse=torch.empty((B, Hq, T), device=dev),
                dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v))
    # row-kernel operands of their own, [B, Hq, T, T]
    n = B * Hq * T * T
    rows = dict(s=torch.randn(n, device=dev), dp=torch.randn(n, device=dev),
                p=torch.empty(n, dtype=tdt, device=dev), ds=torch.empty(n, dtype=tdt, device=dev),
                lse=torch.empty(B * Hq * T, device=dev))
    ctx = U.Context()
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    causal = int(w.causal)

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {A.load_library().attn_status_string(st).decode()}")

    def kernel(name):
        if name == "unfused_fwd":
            check(lib.attn_unfused_fwd(ctx.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       bufs["o"].data_ptr(), bufs["lse"].data_ptr(), B, T, Hq, Hkv,
                                       D, w.scale, causal, code, ws.data_ptr(), ws.numel(), s), name)
        elif name == "unfused_bwd":
            check(lib.attn_unfused_bwd(ctx.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       bufs["lse"].data_ptr(), dO.data_ptr(), bufs["dq"].data_ptr(),
                                       bufs["dk"].data_ptr(), bufs["dv"].data_ptr(), B, T, Hq, Hkv,
                                       D, w.scale, causal, code, ws.data_ptr(), ws.numel(), s), name)
        elif name == "softmax_lse":
            check(lib.attn_unfused_softmax_lse(rows["s"].data_ptr(), rows["p"].data_ptr(),
                                               rows["lse"].data_ptr(), B * Hq * T, T, w.scale,
                                               causal, code, s), name)
        elif name == "probs_from_lse":
            check(lib.attn_unfused_probs_from_lse(rows["s"].data_ptr(), rows["lse"].data_ptr(),
                                                  rows["p"].data_ptr(), B * Hq * T, T, w.scale,
                                                  causal, code, s), name)
        else:
            check(lib.attn_unfused_softmax_bwd(rows["p"].data_ptr(), rows["dp"].data_ptr(),
                                               rows["ds"].data_ptr(), B * Hq * T, T, causal, code,
                                               s), name)

    names = ("unfused_fwd", "unfused_bwd")
    row_names = ("softmax_lse", "probs_from_lse", "softmax_bwd")

    def digest():
        h = hashlib.sha256()
        for nme in ("o", "lse", "dq", "dk", "dv"):
            h.update(bufs[nme].contiguous().view(torch.uint8).cpu().numpy().tobytes())
        return h.hexdigest()

    hashes = []
    for _ in range(3):
        for nme in names:
            kernel(nme)
        torch.cuda.synchronize()
        hashes.append(digest())
    gate = {"finite": all(bool(torch.isfinite(bufs[nme].float()).all()) for nme in bufs),
            "hash_repeats_equal": len(set(hashes)) == 1}
    gate["ok"] = gate["finite"] and gate["hash_repeats_equal"]
    log("gate", gate)
    if not gate["ok"]:
        print(json.dumps({"metric": "gate failed", "gate": gate}), flush=True)
        return 1
    for nme in row_names:  # warm the row operands (p from s, etc.)
        kernel(nme)
    for _ in range(args.warmup):
        for nme in names:
            kernel(nme)
    torch.cuda.synchronize()

    per_kernel_us = {}
    n_rep = max(5, min(20, args.steps // 4))
    for nme in names + row_names:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(2e6))
        e0.record(stream)
        for _ in range(n_rep):
            kernel(nme)
        e1.record(stream)
        torch.cuda.synchronize()
        per_kernel_us[nme] = 1e3 * e0.elapsed_time(e1) / n_rep

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for nme in names:
            kernel(nme)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    flops = w.fwd_flops + w.bwd_flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    dom = max(row_names, key=per_kernel_us.get)
    nbytes = row_kernel_bytes(dom, B, T, Hq, bool(causal))
    achieved = nbytes / (per_kernel_us[dom] * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None, "kernel": dom,
            "avg_launch_us": round(per_kernel_us[dom], 2), "bytes_per_launch": nbytes,
            "timing": "back-to-back launches of the row kernel alone between HIP events"}
    row_gbs = {nme: round(row_kernel_bytes(nme, B, T, Hq, bool(causal)) / (per_kernel_us[nme] * 1e-6) / 1e9, 1)
               for nme in row_names}
    log(f"unfused step {ms_per_step * 1e3:.1f} us, {tflops:.1f} TFLOP/s; kernels {per_kernel_us}; "
        f"row kernels GB/s {row_gbs}")
    ctx.close()
    out = {
        "metric": "attn fwd+bwd TFLOP/s & % bf16 MFMA peak, B4·T1024 GQA12/4 d64",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name + "+unfused", "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "D": D,
                   "causal": bool(w.causal), "scale": w.scale,
                   "gflop_per_step": round(flops / 1e9, 4),
                   "path": "unfused baseline: [T,T] float32 scores in HBM, rocBLAS GEMMs"},
        "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "per_kernel_us": {nme: round(u, 2) for nme, u in per_kernel_us.items()},
        "row_kernel_gbs": row_gbs,
        "roofline": roof,
        "cpu_baseline": None,
        "gate": gate,
        "output_sha256": hashes[0],
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(w, inp, bufs, budget_s, tables=None):
    """Time the fp64 oracle on (batch, KV-group) units until ``budget_s`` is spent,
    and compare the GPU outputs of those units with it.  With rotary ``tables``
    (cos, sin) the oracle rotates q and k first (timed) and maps dq, dk back."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing or unusable
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    q, k, v, dO = (inp.as_float64(n) for n in ("q", "k", "v", "dO"))
    rot_secs = 0.0
    if tables is not None:
        t0 = time.perf_counter()
        q, k = oracle.apply_rope(q, *tables), oracle.apply_rope(k, *tables)
        rot_secs = time.perf_counter() - t0
    gpu = {n: bufs[n].float().cpu().numpy().astype(np.float64) for n in ("o", "lse", "dq", "dk", "dv")}
    units = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    G = w.G
    # Passes over the units (the first one also compared with the GPU) until the
    # budget is spent, so a small workload is still timed over seconds.
    done, secs, worst, passes = 0, 0.0, {}, 0
    while secs < budget_s:
        passes += 1
        for b, g in units:
            t0 = time.perf_counter()
            o_r, lse_r = oracle.ref_fwd_group(q, k, v, w.scale, w.causal, b, g)
            dq_r, dk_r, dv_r, _ = oracle.ref_bwd_group(q, k, v, dO, w.scale, w.causal, b, g)
            if tables is not None:
                dq_r = oracle.apply_rope_transpose(dq_r[None], *tables)[0]
                dk_r = oracle.apply_rope_transpose(dk_r[None, :, None], *tables)[0, :, 0]
            secs += time.perf_counter() - t0
            done += 1
            if passes == 1:
                hs = slice(g * G, (g + 1) * G)
                pairs = (("o", gpu["o"][b, :, hs], o_r), ("dq", gpu["dq"][b, :, hs], dq_r),
                         ("dk", gpu["dk"][b, :, g], dk_r), ("dv", gpu["dv"][b, :, g], dv_r))
                for n, a, r in pairs:
                    worst[n] = max(worst.get(n, 0.0), float(np.max(np.abs(a - r)) / np.max(np.abs(r))))
                worst["lse"] = max(worst.get("lse", 0.0), float(np.max(np.abs(gpu["lse"][b, hs] - lse_r))))
            if secs >= budget_s:
                break
    secs += rot_secs * done / len(units)  # this sample's share of the rotation
    pairs_per_unit = G * (w.T * (w.T + 1) // 2 if w.causal else w.T * w.T)
    flops = done * pairs_per_unit * (4.0 + 10.0) * w.D
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} unit computations ({passes} pass{'es' if passes > 1 else ''} over the "
                      f"{len(units)} (batch, KV-group) units of {w.name}"
                      f"{' with rotary positions' if tables is not None else ''}), fwd+bwd, "
                      f"{secs:.2f} s",
            "seconds": round(secs, 3),
            "max_err_vs_gpu": {n: float(f"{e:.3g}") for n, e in worst.items()},
            "parity_ok": all(e <= 2e-2 for e in worst.values())}


if __name__ == "__main__":
    sys.exit(main())
