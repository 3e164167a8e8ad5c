#!/usr/bin/env python3
"""RelayAttention decode-attention benchmark on one MI355X.

One step = one relay_attn_decode call (system attention, context attention and the
relay merge) over one batch of the Llama2-7B-shaped decode-attention layer: batch 32,
32 MHA heads, head_dim 128, bf16 in / fp32 accumulation, system prompt 2048 tokens,
per-request contexts uniform in [16, 512] (paged, block 16, shuffled block tables),
synthetic seeded inputs.  Inputs are resident in HBM before timing starts.  Each real
layer has its own KV cache, so the timed loop rotates over several copies of the
inputs whose total exceeds the 256 MB Infinity Cache; a step therefore reads its K/V
from HBM, not from the last-level cache.

Prints one JSON line:
  value          query-tokens/s/layer (T_q / step time)
  roofline       dominant kernel: algorithmic bytes (or flops) per launch over its
                 kernel-execution time (HIP events the runtime stamps at the kernel's
                 start and end), against the published peak and the measured ceiling
                 (librelay_probes.so); with the committed rocprofv3 figure beside it
  cpu_baseline   the fp64 oracle on the host cores over a bounded sample
  sweep          query-tokens/s and HBM fraction vs system length (Llama-30B shape)
  batch_sweep, context_dilution   relay against the prefix-shared baseline
  oracle_single_thread   the oracle on one host thread, configs 1-3

Other modes (one JSON line per case, for rocprofv3 runs): --sys-scaling,
--batch-sweep, --copy-calibration; --summarize turns rocprofv3 CSV output into the
text summaries under profiles/.
"""
import argparse
import csv
import ctypes
import glob
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 * 2**20
COPY_BYTES = 512 * 2**20
READ_PROBE_BYTES = 2**30

BATCH_POINTS = (1, 4, 16, 64, 256)       # Llama2-7B shape, relay against the baseline
CTX_POINTS = (64, 256, 1024, 4096)       # every request's own context length, batch 32
ORACLE_1T = ((1, 0), (2, 0), (3, 0), (3, 5))
BATCH_SWEEP = (1, 2, 4, 8, 16, 32, 64, 128, 256)
SYS_SCALING = (("llama2_7b_mha", 2, (1, 4, 8, 16, 32)), ("llama3_8b_gqa", 4, (1, 4, 16, 64, 256)))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload config 1..5 (default 2)")
    ap.add_argument("--sweep-index", type=int, default=0, help="config-3 system-length index")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="only the main line (no sweeps, probes, extras)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the oracle sample in CPU-seconds (wall time x threads)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (for counter runs, which serialise dispatches)")
    ap.add_argument("--sys-scaling", action="store_true",
                    help="only run the system-attention step over batch sweeps of the Llama2-7B and "
                         "Llama-3-8B shapes (for counters: system-KV bytes read vs batch size)")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="only run relay vs the no-relay baseline over more batch sizes of the Llama2-7B "
                         "shape, then over request context lengths at batch 32 (one JSON line per point)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run torch's device copy of COPY_BYTES, 10 times (scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes)")
    ap.add_argument("--summarize", choices=("stats", "traffic", "mfma", "sysbytes"),
                    help="write a profiles/ summary from rocprofv3 --output-format csv directories")
    ap.add_argument("--workload", default="", help="--summarize: workload name of the profiled run(s)")
    ap.add_argument("--dirs", nargs="*", default=[],
                    help="--summarize: rocprofv3 -d directories (stats: 1; traffic: fetch, write, copy "
                         "fetch, copy write; mfma: one per workload, --workload lists them comma-separated; "
                         "sysbytes: the --sys-scaling FETCH_SIZE run, its stdout, the copy-calibration fetch run)")
    ap.add_argument("--commands", nargs="*", default=[], help="--summarize: the commands that made --dirs")
    ap.add_argument("--timed-steps", type=int, default=0,
                    help="--summarize stats: also report the mean of each kernel's last N dispatches")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------
# kernels by short name, and the rocprofv3 summaries under profiles/

# stream_sys_kernel is the streaming launch that also holds the matrix-core system
# workgroups (sys_mode 4): it is the step's streaming launch, named like the other one;
# sys_attn_mfma_pp_kernel is the eight-wave form of the matrix-core system kernel
KERNELS = (("stream_attn_kernel", "stream_attn"), ("stream_sys_kernel", "stream_attn"),
           ("sys_attn_mfma_kernel", "sys_attn_mfma"), ("sys_attn_mfma_pp_kernel", "sys_attn_mfma"),
           ("sys_attn_tiled_kernel", "sys_attn_tiled"), ("relay_merge_kernel", "relay_merge"),
           ("relay_fuse_kernel", "relay_fuse"), ("rope_append_kernel", "rope_append"),
           ("read_probe_kernel", "read_probe"), ("mfma_probe_kernel", "mfma_probe"))


def short_name(full):
    for k, s in KERNELS:
        if k in full:
            return s
    return None


def source_digest():
    from shared_prompt_kv_amd import build as B
    return B.source_digest()


def _csv(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def _counters(d):
    """{(short kernel, counter): [value per dispatch]} from a counter_collection.csv."""
    per = {}
    for row in _csv(d, "counter_collection.csv"):
        k = short_name(row["Kernel_Name"]) or ("copy" if "copyBuffer" in row["Kernel_Name"] else None)
        if k is None:
            continue
        key = (k, row["Counter_Name"], row["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (k, c, _), v in per.items():
        out.setdefault((k, c), []).append(v)
    return out


def summarize(args):
    """profiles/ text summary of rocprofv3 CSV output: kernel statistics, HBM traffic
    per launch (FETCH_SIZE / WRITE_SIZE scaled by a device copy of known size), or
    matrix-core utilisation."""
    dig = source_digest()
    head = [f"library_sources_sha256: {dig}"]
    cmds = ["# commands:"] + [f"#   {c}" for c in args.commands]
    if args.summarize == "stats":
        rows = []
        for r in _csv(args.dirs[0], "kernel_stats.csv"):
            rows.append((short_name(r["Name"]) or "-", int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"]), r["Name"]))
        named = [r for r in rows if r[0] != "-"]
        dom = max(named, key=lambda r: r[1] * r[2])[0]
        # the mean over each kernel's last --timed-steps dispatches: the eager pass whose
        # kernels bench.py times with start/end events (the graph replays before it can
        # run at another clock)
        last = {}
        if args.timed_steps > 0:
            per = {}
            for r in _csv(args.dirs[0], "kernel_trace.csv"):
                per.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            for k, v in per.items():
                v = [d for _, d in sorted(v)][-args.timed_steps:]
                last[k] = sum(v) / len(v) / 1e3
        path = os.path.join(ROOT, "profiles", f"{dom}_{args.workload}_kernel_stats.txt")
        lines = [f"# rocprofv3 kernel-trace statistics: {args.workload} (kernels timed by dispatch start/end);",
                 f"# timed_avg_us: mean of each kernel's last {args.timed_steps} dispatches (the eager pass "
                 "that bench.py times with kernel start/end events)"]
        lines += cmds + head
        lines.append(f"{'kernel':16s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} "
                     f"{'timed_avg_us':>12s} {'pct':>6s}  full name")
        for s, c, a, mn, mx, pct, full in sorted(rows, key=lambda r: -r[5]):
            ta = f"{last[full]:12.3f}" if full in last else f"{'-':>12s}"
            lines.append(f"{s:16s} {c:6d} {a:9.3f} {mn:9.3f} {mx:9.3f} {ta} {pct:6.2f}  {full[:90]}")
    elif args.summarize == "traffic":
        fetch, write, cfetch, cwrite = (_counters(d) for d in args.dirs[:4])
        cf = sum(cfetch[("copy", "FETCH_SIZE")]) / len(cfetch[("copy", "FETCH_SIZE")])
        cw = sum(cwrite[("copy", "WRITE_SIZE")]) / len(cwrite[("copy", "WRITE_SIZE")])
        fscale, wscale = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
        lines = [f"# HBM traffic per launch on {args.workload}: rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per "
                 "dispatch), scaled by what the same counters read for torch's device copy of 512 MiB "
                 "(one read + one write of 512 MiB)"]
        lines += cmds + head
        lines += [f"copy_bytes: {COPY_BYTES}", f"copy_fetch_kib_per_dispatch: {cf:.1f}",
                  f"copy_write_kib_per_dispatch: {cw:.1f}", f"fetch_scale: {fscale:.4f}",
                  f"write_scale: {wscale:.4f}"]
        kernels = sorted({k for k, c in fetch if k not in ("copy",)})
        best = None
        for k in kernels:
            f = fetch.get((k, "FETCH_SIZE"), [])
            w = write.get((k, "WRITE_SIZE"), [])
            if not f or not w:
                continue
            fk, wk = sum(f) / len(f), sum(w) / len(w)
            t = int(round(fk * 1024 * fscale + wk * 1024 * wscale))
            lines += [f"{k}.dispatches: {len(f)}", f"{k}.fetch_kib_per_dispatch: {fk:.1f}",
                      f"{k}.write_kib_per_dispatch: {wk:.1f}", f"{k}.traffic_bytes_per_launch: {t}"]
            if best is None or t > best[1]:
                best = (k, t)
        path = os.path.join(ROOT, "profiles", f"{best[0]}_{args.workload}_traffic.txt")
    elif args.summarize == "sysbytes":
        # dispatches of the system step in order; the cases of the --sys-scaling run in
        # the order of its JSON lines, `dispatches` each
        rows = [r for r in _csv(args.dirs[0], "counter_collection.csv")
                if r["Counter_Name"] == "FETCH_SIZE" and short_name(r["Kernel_Name"]) in
                ("stream_attn", "sys_attn_mfma", "sys_attn_tiled")]
        per = {}
        for r in rows:
            per[int(r["Dispatch_Id"])] = per.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
        fetch = [per[k] for k in sorted(per)]
        cases = [json.loads(l) for l in open(args.dirs[1]) if l.startswith("{")]
        cfetch = _counters(args.dirs[2])[("copy", "FETCH_SIZE")]
        fscale = COPY_BYTES / (sum(cfetch) / len(cfetch) * 1024)
        lines = ["# System-KV bytes read from HBM by the system step vs batch size (RelayAttention reads the",
                 "# shared system K/V once per batch).  FETCH_SIZE (KiB per dispatch) of the system step's",
                 f"# kernel, scaled by {fscale:.4f} (what FETCH_SIZE reads for torch's 512 MiB device copy);",
                 "# per case: 3 untimed + the timed calls of relay_sys_attn, the merge launch excluded;",
                 "# sys_kv_bytes = 2 * H_kv * d * 2 B * L_s."]
        lines += cmds + head
        lines.append(f"{'shape':16s} {'batch':>6s} {'rows/kvh':>8s} {'kernel':15s} {'sys_kv_MB':>9s} "
                     f"{'fetch_MB':>9s} {'fetch/kv':>8s}")
        i = 0
        for c in cases:
            n = c["dispatches"]
            f = fetch[i:i + n]
            i += n
            mb = sum(f) / len(f) * 1024 * fscale / 1e6
            kv = c["sys_kv_bytes"] / 1e6
            lines.append(f"{c['shape']:16s} {c['batch']:6d} {c['rows_per_kv_head']:8d} {c['kernel']:15s} "
                         f"{kv:9.2f} {mb:9.2f} {mb / kv:8.3f}")
        path = os.path.join(ROOT, "profiles", "sys_attn_kv_bytes_vs_batch.txt")
    else:
        lines = ["# Matrix-core utilisation: SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / "
                 "(GRBM_GUI_ACTIVE per XCD * 1024 SIMDs); GRBM_GUI_ACTIVE is reported summed over "
                 "the 8 XCDs, so per-XCD active cycles = value / 8"]
        lines += cmds + head
        lines.append(f"{'workload':26s} {'kernel':16s} {'dispatches':>10s} {'mfma_busy':>14s} "
                     f"{'active/xcd':>12s} {'mfma_util':>9s}")
        for wl, d in zip(args.workload.split(","), args.dirs):
            cnt = _counters(d)
            for k in sorted({k for k, c in cnt}):
                busy = cnt.get((k, "SQ_VALU_MFMA_BUSY_CYCLES"))
                act = cnt.get((k, "GRBM_GUI_ACTIVE"))
                if not busy or not act:
                    continue
                b, a = sum(busy) / len(busy), sum(act) / len(act) / 8
                lines.append(f"{wl:26s} {k:16s} {len(busy):10d} {b:14.0f} {a:12.0f} {b / (a * 1024):9.3f}")
        path = os.path.join(ROOT, "profiles", "sys_attn_mfma_mfma_util.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def read_profile(kind, workload):
    """A committed summary of this workload taken from the current library sources:
    {kernel: (avg_us, timed_avg_us or None)} (kind "stats") or {kernel: traffic bytes per
    launch} ("traffic"),
    with the file it came from; None when there is none or it is stale."""
    pat = os.path.join(ROOT, "profiles", f"*_{workload}_{'kernel_stats' if kind == 'stats' else 'traffic'}.txt")
    dig = source_digest()
    for path in sorted(glob.glob(pat)):
        with open(path) as f:
            text = f.read().splitlines()
        if f"library_sources_sha256: {dig}" not in text:
            continue
        out = {}
        for line in text:
            if line.startswith("#"):
                continue
            if kind == "stats":
                parts = line.split()
                if len(parts) >= 7 and parts[0] in dict((s, 1) for _, s in KERNELS):
                    out[parts[0]] = (float(parts[2]), None if parts[5] == "-" else float(parts[5]))
            elif ".traffic_bytes_per_launch:" in line:
                k, v = line.split(":", 1)
                out[k.split(".")[0]] = int(v)
        if out:
            return out, os.path.relpath(path, ROOT)
    return None


# ---------------------------------------------------------------------------------------
# algorithmic work (what the method must move / compute) and the partials' overhead


def work_of(w, plan=None):
    s = w.spec
    E = 2 if s.dtype == "bf16" else 4
    d, Hq, Hkv = s.head_dim, s.num_q_heads, s.num_kv_heads
    Tq, B = w.total_q, s.batch
    sum_ctx = int(w.ctx_lens.sum())
    mb = w.max_blocks_per_seq
    rows = Tq * Hq
    kv_sys = 2 * Hkv * d * E * s.sys_len
    kv_ctx = 2 * Hkv * d * E * sum_ctx
    q_bytes = rows * d * E
    out_bytes = rows * d * 4
    part_row = rows * (d + 1) * 4          # one fp32 output row + LSE per query row
    tables = 4 * B * (mb + 2) + (4 * (B + 1) if int(w.q_lens.max()) > 1 else 0)
    ql, cl = w.q_lens.astype(int), w.ctx_lens.astype(int)
    vis = int((ql * cl - ql * (ql - 1) // 2).sum())      # visible context keys over all query tokens
    # the system K/V are read by the streaming launch (system streams, or the matrix-core
    # system workgroups inside it)
    sys_in_stream = plan is None or plan["sys_mode"] in (1, 4)
    work = {
        "step_bytes": kv_sys + kv_ctx + q_bytes + out_bytes + tables,
        "step_flops": 4 * Hq * d * (Tq * s.sys_len + vis),
        "sys_flops": 4 * Hq * d * Tq * s.sys_len,
        "ctx_flops": 4 * Hq * d * vis,
        "sys_attn_mfma": kv_sys + q_bytes,
        "sys_attn_tiled": kv_sys + q_bytes,
        # the streaming launch: context (and, at <= 64 stacked rows per KV head, system) K/V
        "stream_attn": (kv_sys if sys_in_stream else 0) + kv_ctx + q_bytes + tables,
        # relay fusion as the method states it: two partials in, the output out
        "relay_merge": 2 * part_row + out_bytes,
    }
    if plan is not None:
        work["overhead"] = partial_overhead(w, plan)
    return work


def partial_overhead(w, plan):
    """Bytes of partial results beyond the method's two per row: what the kernels write
    (each piece of a stream writes its rows' O and LSE) and what the merge reads back
    beyond two partials per row (every place fixed in advance, sys_row_slots per KV head
    and ctx_row_slots per row, whether a piece went there or not, and the pieces past
    them).  Follows the streaming launch's static partition (single request group); the
    system kernel writes every run slot of every row."""
    import numpy as np
    s = w.spec
    d, g, Hkv = s.head_dim, s.group, s.num_kv_heads
    row_b = (d + 1) * 4
    rows = w.total_q * s.num_q_heads
    if plan["stream_launches"] != 1:
        return None
    rtc, rbmax = plan["ctx_row_tiles"], plan["ctx_row_blocks"]
    nq = w.q_lens.astype(np.int64)
    c = np.minimum(w.ctx_lens.astype(np.int64), w.max_blocks_per_seq * 16)
    steps = np.maximum(1, -(-c // 32))
    rbs = np.minimum(-(-(nq * g) // (16 * rtc)), rbmax)
    # streams in (request, head, row block) order
    req = np.repeat(np.arange(len(c)), rbs * Hkv)
    rb = np.concatenate([np.tile(np.arange(r), Hkv) for r in rbs]) if len(c) else np.zeros(0, np.int64)
    st = steps[req]
    rows_in = np.minimum(nq[req] * g - rb * 16 * rtc, 16 * rtc)
    M = w.total_q * g
    sys_mode = plan["sys_mode"]
    S = -(-s.sys_len // 32) if sys_mode == 1 else 0
    Ts = Hkv * S
    T = Ts + int(st.sum())
    W = min(plan["stream_waves"], T)
    part_of = lambda x: ((x + 1) * W + T - 1) // T - 1
    p0 = Ts + np.concatenate([[0], np.cumsum(st)[:-1]]) if len(st) else np.zeros(0, np.int64)
    ctx_pieces = part_of(p0 + st - 1) - part_of(p0) + 1
    written = int((ctx_pieces * rows_in).sum()) * row_b
    ks, kc = plan.get("sys_row_slots", 0), plan.get("ctx_row_slots", 0)
    read = int((np.maximum(ctx_pieces, kc) * rows_in).sum()) * row_b
    if sys_mode == 1 and S > 0:
        h = np.arange(Hkv)
        sys_pieces = part_of(h * S + S - 1) // 4 - part_of(h * S) // 4 + 1
        written_sys = int(sys_pieces.sum()) * M * row_b
        read += int(np.maximum(sys_pieces, ks).sum()) * M * row_b
    elif sys_mode >= 2:
        written_sys = plan["sys_runs"] * rows * row_b
        read += written_sys
    else:
        written_sys = 0
    in_stream = sys_mode in (1, 4)
    return {"stream_attn_partials_written": written + (written_sys if in_stream else 0),
            "sys_kernel_partials_written": 0 if in_stream else written_sys,
            "merge_extra_partial_reads": max(0, read - 2 * rows * row_b)}


# ---------------------------------------------------------------------------------------


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self, torch):
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def clone_set(torch, t):
    return {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in t.items()}


def sys_kernel_name(plan):
    return {2: "sys_attn_mfma", 3: "sys_attn_tiled"}.get(plan["sys_mode"])


def measure(torch, relay, w, steps, warmup, per_kernel=True, graph=True, prep=None):
    """Times decode steps over rotating input copies.

    graph: the steps captured in one HIP graph (a full rotation over the copies) and
    replayed, as a served model replays its decode step; the timed region holds `steps`
    steps.  eager: the same steps launched one by one through the prepared C-ABI call.
    Per-kernel durations: the timed entry point's events, which the runtime stamps at
    each kernel's own start and end (eager steps, `steps` of them).
    """
    t0 = relay.to_device(w, "cuda")
    if prep is not None:  # e.g. the no-relay baseline's inputs
        t0 = prep(t0)
    dims = relay.dims_of(t0)
    plan = relay.relay_get_plan(dims, t0["sys_len"])
    work = work_of(w, plan)
    n_sets = max(2, math.ceil(3 * MALL_BYTES / max(work["step_bytes"], 1)))
    n_sets = min(n_sets, 16)
    sets = [t0] + [clone_set(torch, t0) for _ in range(n_sets - 1)]
    ws = relay.workspace(dims, t0["sys_len"], "cuda")
    outs = [torch.empty(t0["q"].shape, dtype=torch.float32, device="cuda") for _ in range(n_sets)]
    calls = [relay.DecodeCall(sets[i], outs[i], ws) for i in range(n_sets)]
    res = {"n_sets": n_sets, "work": work, "plan": plan}

    for i in range(warmup):
        calls[i % n_sets]()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        calls[i % n_sets]()
    e1.record()
    torch.cuda.synchronize()
    res["eager_ms_per_step"] = e0.elapsed_time(e1) / steps

    res["ms_per_step"] = res["eager_ms_per_step"]
    if graph:
        _time_graph(torch, calls, n_sets, steps, res)

    if per_kernel:
        he = HipEvents(torch)
        evs = he.create(6 * steps)
        for i in range(steps):
            calls[i % n_sets].timed(evs[6 * i:6 * i + 6])
        torch.cuda.synchronize()
        names = [sys_kernel_name(plan), "stream_attn", "relay_merge"]
        acc = {}
        for i in range(steps):
            e = evs[6 * i:6 * i + 6]
            for j, k in enumerate(names):
                if k is not None:
                    acc[k] = acc.get(k, 0.0) + he.elapsed_ms(e[2 * j], e[2 * j + 1])
        he.destroy(evs)
        res["kernel_us"] = {k: 1000.0 * v / steps for k, v in acc.items()}
    del calls, sets, outs, ws
    torch.cuda.empty_cache()
    return res


def _time_graph(torch, calls, n_sets, steps, res):
    """HIP graphs of the decode step, replayed for exactly `steps` steps: one graph
    holds a full rotation over the input copies, a second the first steps % n_sets
    calls of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    reps, rest = divmod(steps, n_sets)
    full = torch.cuda.CUDAGraph()
    with torch.cuda.graph(full):
        for c in calls:
            c()
    part = None
    if rest:
        part = torch.cuda.CUDAGraph()
        with torch.cuda.graph(part):
            for c in calls[:rest]:
                c()
    for _ in range(2):
        full.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        full.replay()
    if part is not None:
        part.replay()
    e1.record()
    torch.cuda.synchronize()
    res["graph_ms_per_step"] = e0.elapsed_time(e1) / steps
    res["ms_per_step"] = res["graph_ms_per_step"]
    del full, part


# ---------------------------------------------------------------------------------------
# measured ceilings: librelay_probes.so


def probes_lib():
    from shared_prompt_kv_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        raise RuntimeError(f"{B.PROBE_LIB} is not built: run `python -m shared_prompt_kv_amd.build`")
    lib = ctypes.CDLL(B.PROBE_LIB)
    vp = ctypes.c_void_p
    lib.relay_probe_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int32, vp]
    lib.relay_probe_mfma.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
    return lib


def measured_ceilings(torch):
    """What this GPU reaches at all: a hand-written streaming read of 1 GiB (best over
    a few grid sizes) and bf16 matrix-core products on register operands (one
    v_mfma_f32_32x32x16_bf16 stream per wave, two waves per SIMD)."""
    lib = probes_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.ones(READ_PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(16 * cus * 256, dtype=torch.float32, device="cuda")

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    best = (0.0, 0)
    for per_cu in (1, 2, 4, 8):
        grid = per_cu * cus
        t = timed(lambda: lib.relay_probe_read(ctypes.c_void_p(buf.data_ptr()), READ_PROBE_BYTES,
                                               ctypes.c_void_p(sink.data_ptr()), grid, stream))
        best = max(best, (READ_PROBE_BYTES / t / 1e9, grid))
    iters, grid = 512, 2 * cus
    flops = grid * 4 * iters * 4 * 32768
    t = timed(lambda: lib.relay_probe_mfma(ctypes.c_void_p(sink.data_ptr()), iters, grid, stream), n=5)
    out = {"read_GBps": round(best[0], 1), "read_grid": best[1],
           "read_frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4),
           "mfma_bf16_TFLOPs": round(flops / t / 1e12, 1),
           "mfma_frac_of_peak": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4),
           "note": "librelay_probes.so: relay_probe_read over 1 GiB (16-byte loads, 8 in flight per thread, "
                   "one contiguous slab per workgroup, best grid), relay_probe_mfma (register operands, 4 "
                   "independent accumulators per wave, 2 workgroups of 4 waves per CU)"}
    del buf, sink
    torch.cuda.empty_cache()
    return out


def copy_calibration(torch):
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "dispatches": 10}), flush=True)


# ---------------------------------------------------------------------------------------
# the oracle on the host


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip() + f" ({os.cpu_count()} logical CPUs visible)"
    except OSError:
        pass
    return "unknown"


def _oracle_rate(w, budget_wall):
    """Query tokens per second of the oracle (exact fp64 attention over all heads),
    request by request through the workload (cycling) for about budget_wall seconds."""
    import numpy as np
    import oracle
    P = oracle.Problem(w)
    Hq = w.spec.num_q_heads
    tokens, elapsed, n = 0, 0.0, 0
    start = time.perf_counter()
    while elapsed < budget_wall:
        b = n % w.spec.batch
        lo, hi = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
        P.attention(np.arange(lo * Hq, hi * Hq, dtype=np.int64))
        tokens += hi - lo
        n += 1
        elapsed = time.perf_counter() - start
    return tokens / elapsed, n, tokens, elapsed


def cpu_baseline(w, budget_cpu_s):
    """The oracle (unchanged) on all host cores, until about budget_cpu_s CPU-seconds
    have been spent."""
    import oracle
    cores = oracle.num_threads()
    rate, n, tokens, elapsed = _oracle_rate(w, budget_cpu_s / max(cores, 1))
    return {"value": round(rate, 3), "unit": "query-tokens/s/layer", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"exact fp64 causal attention (all {w.spec.num_q_heads} heads) for {n} requests taken in "
                      f"order, cycling over the {w.spec.batch} requests of the same workload: {tokens} query "
                      f"tokens in {elapsed:.2f} s wall on {cores} threads"}


def oracle_single_thread(budget_s=1.5):
    """The oracle on one host thread for configs 1-3 (config 3 at its shortest and
    longest system prompt), about budget_s seconds each."""
    import oracle
    import workloads
    before = oracle.num_threads()
    oracle.set_num_threads(1)
    out = []
    try:
        for cfg, sweep in ORACLE_1T:
            w = workloads.generate(workloads.config_spec(cfg, sweep))
            rate, n, tokens, elapsed = _oracle_rate(w, budget_s)
            out.append({"workload": w.spec.name, "qtok_s": round(rate, 2), "requests": n, "query_tokens": tokens,
                        "seconds": round(elapsed, 2)})
    finally:
        oracle.set_num_threads(before)
    return {"unit": "query-tokens/s/layer", "threads": 1, "points": out}


# ---------------------------------------------------------------------------------------
# points, sweeps and the steps around the path


def point(torch, relay, spec, args, with_baseline=False, steps=50):
    """One workload measured like the main line (fewer steps): throughput and
    roofline fractions; with_baseline adds the no-relay baseline's step time."""
    w = workloads_generate(spec)
    rr = measure(torch, relay, w, min(args.steps, steps), min(args.warmup, 10))
    print(f"[bench] {spec.name}: {1000 * rr['ms_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    m = rr["ms_per_step"]
    work = rr["work"]
    peak = (BF16_PEAK_TFLOPS if spec.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12
    out = {"workload": spec.name, "qtok_s": round(w.total_q / (m * 1e-3), 1),
           "us_per_step": round(1000 * m, 2), "eager_us_per_step": round(1000 * rr["eager_ms_per_step"], 2),
           "hbm_frac": round(work["step_bytes"] / (m * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
           "mfma_frac": round(work["step_flops"] / (m * 1e-3) / peak, 4),
           "kernel_us": {k: round(v, 2) for k, v in rr["kernel_us"].items()},
           "sys_mode": rr["plan"]["sys_mode"]}
    ov = work.get("overhead")
    if ov:
        out["partial_bytes_frac"] = round((ov["stream_attn_partials_written"] + ov["sys_kernel_partials_written"])
                                          / work["step_bytes"], 4)
    sk = sys_kernel_name(rr["plan"])
    if sk == "sys_attn_mfma" and sk in rr["kernel_us"]:
        out["sys_attn_mfma_frac"] = round(work["sys_flops"] / (rr["kernel_us"][sk] * 1e-6) / peak, 4)
    if rr["plan"]["sys_mode"] == 4:  # system flops over the launch that holds them
        out["stream_attn_mfma_frac"] = round(work["sys_flops"] / (rr["kernel_us"]["stream_attn"] * 1e-6) / peak, 4)
        out["stream_attn_hbm_frac"] = round(work["stream_attn"] / (rr["kernel_us"]["stream_attn"] * 1e-6)
                                            / (HBM_PEAK_GBS * 1e9), 4)
    if with_baseline:
        out.update(no_relay_baseline(torch, relay, w, args, m))
    return out


def no_relay_baseline(torch, relay, w, args, relay_ms, steps=50):
    """The same decode step without relay: every request's block table starts with
    the shared system pages and the context step reads them once per request."""
    from shared_prompt_kv_amd import baseline
    rb = measure(torch, relay, w, min(args.steps, steps), min(args.warmup, 10), per_kernel=False,
                 prep=baseline.prefix_shared)
    bm = rb["ms_per_step"]
    print(f"[bench] {w.spec.name} no-relay baseline: {1000 * bm:.2f} us/step", file=sys.stderr, flush=True)
    return {"no_relay_us_per_step": round(1000 * bm, 2), "relay_speedup": round(bm / relay_ms, 3)}


def batch_points(torch, relay, args, batches, steps=30):
    """Relay against the prefix-shared baseline over batch sizes of the Llama2-7B shape:
    the gain grows with the batch and a single request gains nothing."""
    import workloads
    out = []
    for B in batches:
        r = point(torch, relay, workloads.config_spec(2, 0).replace(batch=B), args, with_baseline=True, steps=steps)
        out.append({"batch": B, "relay_us": r["us_per_step"], "no_relay_us": r["no_relay_us_per_step"],
                    "speedup": r["relay_speedup"], "qtok_s": r["qtok_s"]})
    return out


def ctx_points(torch, relay, args, lens, steps=30):
    """Relay against the baseline at batch 32 when every request has its own context of
    C tokens: long request contexts dilute the gain (the system share of the bytes
    shrinks; kv_bytes_ratio = baseline K/V bytes over relay K/V bytes)."""
    import workloads
    out = []
    for C in lens:
        spec = workloads.config_spec(2, 0).replace(ctx_len_dist="fixed", ctx_lo=C, ctx_hi=C)
        r = point(torch, relay, spec, args, with_baseline=True, steps=steps)
        L, B = spec.sys_len, spec.batch
        out.append({"ctx_len": C, "relay_us": r["us_per_step"], "no_relay_us": r["no_relay_us_per_step"],
                    "speedup": r["relay_speedup"], "kv_bytes_ratio": round(B * (L + C) / (L + B * C), 3)})
    return out


def rope_append_time(torch, relay, w, args):
    """The step before the path on the same workload: position embedding of the new
    tokens' q and k at sys_len + context position and their K/V appended to the pages
    (relay_rope_append), through a pre-marshalled call, back to back, timed with HIP
    events; also the same calls replayed from a HIP graph."""
    t = relay.to_device(w, "cuda")
    s = w.spec
    dt = t["q"].dtype
    tab = relay.relay_rope_table(s.sys_len + int(w.ctx_lens.max()), s.head_dim)
    g = torch.Generator(device="cuda").manual_seed(1)
    q_new = torch.randn(t["q"].shape, generator=g, device="cuda").to(dt)
    k_new = torch.randn((w.total_q, s.num_kv_heads, s.head_dim), generator=g, device="cuda").to(dt)
    v_new = torch.randn((w.total_q, s.num_kv_heads, s.head_dim), generator=g, device="cuda").to(dt)
    q_out = torch.empty_like(q_new)
    dims = relay.dims_of(t)
    call = relay.RopeAppendCall(dims, s.sys_len, q_new, k_new, v_new, tab, t["block_tables"], t["ctx_lens"],
                                t["cu_q_lens"], t["ctx_k_pages"], t["ctx_v_pages"], q_out)
    n = min(args.steps, 200)

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    for _ in range(10):
        call()
    us = 1000 * timed(call, n) / n
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(20):
            call()
    graph.replay()
    reps = max(1, n // 20)
    us_graph = 1000 * timed(graph.replay, reps) / (20 * reps)
    E = 2 if s.dtype == "bf16" else 4
    nbytes = (2 * w.total_q * s.num_q_heads * s.head_dim * E      # q in and out
              + 4 * w.total_q * s.num_kv_heads * s.head_dim * E   # k, v in; k, v pages out
              + w.total_q * s.head_dim * 4)                       # one table row per token
    return {"us_per_call": round(us, 2), "us_per_call_graph": round(us_graph, 2), "bytes_alg": nbytes,
            "hbm_frac": round(nbytes / (us_graph * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "note": "pre-marshalled calls back to back (eager), and 20 calls per HIP graph replay; a few MB "
                    "per call, so launch-latency bound"}


def prefill_time(torch, relay, spec, args):
    """The offline step before serving on a workload's shapes: the system prompt's cache
    fill (position embedding, layouts) and its causal attention
    (shared_prompt_kv_amd.prefill), timed over repeated calls on synthetic projections;
    the causal attention call (relay_prefill_attn) also alone."""
    from shared_prompt_kv_amd import prefill
    s = spec
    L = s.sys_len
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(2)
    q = torch.randn((L, s.num_q_heads, s.head_dim), generator=g, device="cuda").to(dt)
    k = torch.randn((L, s.num_kv_heads, s.head_dim), generator=g, device="cuda").to(dt)
    v = torch.randn((L, s.num_kv_heads, s.head_dim), generator=g, device="cuda").to(dt)
    tab = relay.relay_rope_table(L, s.head_dim)
    flops = 4 * s.num_q_heads * s.head_dim * (L * (L + 1) // 2)   # causal: token j sees j + 1 keys
    peak = (BF16_PEAK_TFLOPS if s.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12

    def timed(fn, n=5):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1000 * e0.elapsed_time(e1) / n

    us = timed(lambda: prefill.prefill_system(q, k, v, tab, s.scale))
    out = {"workload": s.name, "sys_len": L, "us_per_call": round(us, 1),
           "attn_tflops": round(flops / (us * 1e-6) / 1e12, 2)}
    if prefill.uses_matrix_cores(q, k, s.scale):
        sk, sv, _ = prefill.prefill_system(q, k, v, tab, s.scale)
        dims = relay.prefill_dims(q, sk, s.scale)
        ws = relay.prefill_workspace(dims, L, "cuda")
        ua = timed(lambda: relay.relay_prefill_attn(q, sk, sv, L, s.scale, workspace_buf=ws))
        out.update(attn_us=round(ua, 1), attn_kernel_tflops=round(flops / (ua * 1e-6) / 1e12, 2),
                   attn_mfma_frac=round(flops / (ua * 1e-6) / peak, 4))
    out["note"] = ("cache fill + the prompt's causal attention (matrix-core system kernel with a causal mask "
                   "when bf16 / head_dim 128, else the decode path), its allocations included; attn_*: "
                   "relay_prefill_attn alone (causal system kernel + merge)")
    print(f"[bench] {s.name} system prefill L={L}: {us:.1f} us", file=sys.stderr, flush=True)
    return out


def sys_scaling(torch, relay, steps):
    """relay_sys_attn alone (system kernel + merge) for each batch size: 3 untimed
    calls then `steps` timed ones.  Prints one JSON line per case; under rocprofv3 the
    system kernel's dispatches come in the same order, 3 + steps per case."""
    import workloads
    for name, cfg, batches in SYS_SCALING:
        for B in batches:
            spec = workloads.config_spec(cfg, 0).replace(batch=B)
            w = workloads.generate(spec)
            t = relay.to_device(w, "cuda")
            dims = relay.dims_of(t)
            ws = relay.workspace(dims, t["sys_len"], "cuda")
            call = lambda: relay.relay_sys_attn(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], dims,
                                                workspace_buf=ws)
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                call()
            e1.record()
            torch.cuda.synchronize()
            plan = relay.relay_get_plan(dims, t["sys_len"])
            E = 2 if spec.dtype == "bf16" else 4
            print(json.dumps({"shape": name, "batch": B, "sys_len": spec.sys_len,
                              "rows_per_kv_head": w.total_q * spec.group,
                              # relay_sys_attn: the system streams at <= 64 rows per KV
                              # head, else the system kernel as a launch of its own
                              "kernel": {1: "stream_attn", 3: "sys_attn_tiled"}.get(plan["sys_mode"],
                                                                                    "sys_attn_mfma"),
                              "dispatches": 3 + steps,
                              "sys_kv_bytes": 2 * spec.num_kv_heads * spec.head_dim * E * spec.sys_len,
                              "us_per_call": round(1000 * e0.elapsed_time(e1) / steps, 2)}), flush=True)
            del t, ws, w
            torch.cuda.empty_cache()


def workloads_generate(spec):
    import workloads
    return workloads.generate(spec)


# ---------------------------------------------------------------------------------------


def roofline(r, spec, ceilings):
    """The dominant kernel's roofline: algorithmic work per launch over its
    kernel-execution time (live HIP events), against the published peak and the
    measured ceiling, with the committed rocprofv3 figure of the same workload (when it
    was taken from the current library sources) beside it."""
    kus, work, plan = r["kernel_us"], r["work"], r["plan"]
    dom = max(kus, key=kus.get)
    us = kus[dom]
    mfma = dom == "sys_attn_mfma"
    if dom == "stream_attn" and plan["sys_mode"] == 4:
        # the matrix-core system workgroups and the context streams in one launch: the
        # roofline is whichever of the two bounds takes longer
        mfma = work["sys_flops"] / (BF16_PEAK_TFLOPS * 1e12) > work["stream_attn"] / (HBM_PEAK_GBS * 1e9)
    if mfma:
        alg, unit, peak = work["sys_flops"], "TFLOP/s", BF16_PEAK_TFLOPS
        achieved = alg / (us * 1e-6) / 1e12
    else:
        alg, unit, peak = work[dom], "GB/s", HBM_PEAK_GBS
        achieved = alg / (us * 1e-6) / 1e9
    out = {"kernel": dom, "bound": "mfma" if mfma else "hbm", "achieved": round(achieved, 1), "peak": peak,
           "unit": unit, "frac": round(achieved / peak, 4), "traffic": None, "avg_us": round(us, 3),
           "timing": "kernel start/end events (hipExtLaunchKernelGGL), eager steps"}
    out["flops_alg_per_launch" if mfma else "bytes_alg_per_launch"] = alg
    ov = work.get("overhead")
    if ov:
        out["overhead_bytes_per_launch"] = (ov["sys_kernel_partials_written"] if mfma
                                            else ov["stream_attn_partials_written"] if dom == "stream_attn"
                                            else ov["merge_extra_partial_reads"])
    if ceilings:
        c = ceilings["mfma_bf16_TFLOPs"] if mfma else ceilings["read_GBps"]
        out["measured_ceiling"] = {"value": c, "unit": unit, "frac": round(achieved / c, 4),
                                   "probe": "relay_probe_mfma" if mfma else "relay_probe_read"}
    tr = read_profile("traffic", spec.name)
    if tr and dom in tr[0]:
        out["traffic"] = tr[0][dom]
        out["traffic_source"] = tr[1]
    st = read_profile("stats", spec.name)
    if st and dom in st[0]:
        avg, timed = st[0][dom]
        ru = timed if timed is not None else avg
        out["rocprof"] = {"avg_us": avg, "timed_avg_us": timed,
                          "frac": round(alg / (ru * 1e-6) / (1e12 if mfma else 1e9) / peak, 4),
                          "source": st[1]}
    return out


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the decode-attention path runs on a single MI355X; DESIGN.md says how it would shard)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    from shared_prompt_kv_amd import relay

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch)
        return
    relay.load_library()
    if args.sys_scaling:
        sys_scaling(torch, relay, min(args.steps, 20))
        return
    if args.batch_sweep:
        for p in batch_points(torch, relay, args, BATCH_SWEEP):
            print(json.dumps(dict(shape="llama2_7b_mha", **p)), flush=True)
        for p in ctx_points(torch, relay, args, CTX_POINTS):
            print(json.dumps(dict(shape="llama2_7b_mha", batch=32, **p)), flush=True)
        return
    spec = workloads.config_spec(args.config, args.sweep_index)
    w = workloads.generate(spec)
    r = measure(torch, relay, w, args.steps, args.warmup, graph=not args.no_graph)
    print(f"[bench] {spec.name}: {1000 * r['ms_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    ceilings = None if args.no_sweep else measured_ceilings(torch)
    work = r["work"]
    ms = r["ms_per_step"]
    value = w.total_q / (ms * 1e-3)
    peak_flops = (BF16_PEAK_TFLOPS if spec.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12
    line = {
        "metric": "decode-attn query-tokens/s/layer + % HBM roofline vs system-prompt length",
        "value": round(value, 1),
        "unit": "query-tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "timing": ("eager launches" if args.no_graph else
                   "HIP graph replay of the decode step (eager launch: %.5f ms/step)" % r["eager_ms_per_step"]),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "num_q_heads": spec.num_q_heads,
                   "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
                   "sys_len": spec.sys_len, "total_q": w.total_q, "sum_ctx_len": int(w.ctx_lens.sum()),
                   "ctx_len_range": [int(w.ctx_lens.min()), int(w.ctx_lens.max())],
                   "parallelism": "single-gpu", "input_copies_rotated": r["n_sets"]},
        "step_hbm_roofline_frac": round(work["step_bytes"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "step_mfma_roofline_frac": round(work["step_flops"] / (ms * 1e-3) / peak_flops, 5),
        "step_bytes_alg": work["step_bytes"],
        "partial_overhead_bytes": work.get("overhead"),
        "kernel_us": {k: round(v, 3) for k, v in r["kernel_us"].items()},
        "plan": r["plan"],
        "roofline": roofline(r, spec, ceilings),
    }
    if ceilings:
        line["step_hbm_frac_of_measured_read"] = round(work["step_bytes"] / (ms * 1e-3) / (ceilings["read_GBps"] * 1e9),
                                                       4)
    if not args.no_sweep and args.config == 2:
        line["sweep"] = {"workload": "llama30b_mha (batch 32, 52 heads, ctx 128)",
                         "points": [dict(sys_len=Ls, **point(torch, relay, workloads.config_spec(3, i), args,
                                                             with_baseline=True))
                                    for i, Ls in enumerate(workloads.CONFIG3_SYS_LENS)]}
        line["other_configs"] = [point(torch, relay, workloads.config_spec(c, 0), args, with_baseline=True)
                                 for c in (1, 4, 5)]
        line["batch_sweep"] = {"workload": "llama2_7b_mha shape, system 2048, contexts U[16, 512]",
                               "points": batch_points(torch, relay, args, BATCH_POINTS)}
        line["context_dilution"] = {"workload": "llama2_7b_mha shape, batch 32, system 2048, every context C",
                                    "points": ctx_points(torch, relay, args, CTX_POINTS)}
    if not args.no_sweep:
        line["no_relay_baseline"] = no_relay_baseline(torch, relay, w, args, ms)
        line["rope_append"] = rope_append_time(torch, relay, w, args)
        line["system_prefill"] = [prefill_time(torch, relay, workloads.config_spec(c, 0), args) for c in (2, 4)]
        line["hbm_measured"] = ceilings
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        if not args.no_sweep:
            line["oracle_single_thread"] = oracle_single_thread()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
