#!/usr/bin/env python3
"""RelayAttention decode-attention benchmark on one MI355X.

One step = one relay_attn_decode call (sys_attn + ctx_attn + relay_fuse) over one
batch of the Llama2-7B-shaped decode-attention layer: batch 32, 32 MHA heads,
head_dim 128, bf16 in / fp32 accumulation, system prompt 2048 tokens, per-request
contexts uniform in [16, 512] (paged, block 16, shuffled block tables), synthetic
seeded inputs.  Inputs are resident in HBM before timing starts.  Each real layer
has its own KV cache, so the timed loop rotates over several copies of the inputs
whose total exceeds the 256 MB Infinity Cache; a step therefore reads its K/V from
HBM, not from the last-level cache.

Prints one JSON line:
  value          query-tokens/s/layer (T_q / step time)
  roofline       dominant kernel: algorithmic bytes / HIP-event duration vs 8 TB/s
  cpu_baseline   the fp64 oracle on the host cores over a bounded sample
  sweep          query-tokens/s and HBM fraction vs system length (Llama-30B shape)
"""
import argparse
import ctypes
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload config 1..5 (default 2)")
    ap.add_argument("--sweep-index", type=int, default=0, help="config-3 system-length index")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the oracle sample in CPU-seconds (wall time x threads)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (for counter runs, which serialise dispatches)")
    ap.add_argument("--sys-scaling", action="store_true",
                    help="only run the system-attention step over batch sweeps of the Llama2-7B and "
                         "Llama-3-8B shapes (for counters: system-KV bytes read vs batch size)")
    ap.add_argument("--batch-sweep", action="store_true",
                    help="only run relay vs the no-relay baseline (prefix-shared system pages) over "
                         "batch sizes of the Llama2-7B shape, then over request context lengths at batch 32 "
                         "(one JSON line per point)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run torch's device copy of COPY_BYTES, 10 times (scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


COPY_BYTES = 512 * 2**20


def copy_calibration(torch):
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "dispatches": 10}), flush=True)


BATCH_SWEEP = (1, 2, 4, 8, 16, 32, 64, 128, 256)
CTX_SWEEP = (64, 256, 1024, 4096)  # every request's own context length, Llama2-7B shape, batch 32
SYS_SCALING = (("llama2_7b_mha", 2, (1, 4, 8, 16, 32)), ("llama3_8b_gqa", 4, (1, 4, 16, 64, 256)))


def sys_scaling(torch, relay, steps):
    """relay_sys_attn alone (system kernel + chunk merge) for each batch size: 3
    untimed calls then `steps` timed ones.  Prints one JSON line per case; under
    rocprofv3 the system kernel's dispatches come in the same order, 3 + steps per
    case."""
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
                              "kernel": ("sys_attn" if plan["sys_mode"] == 1 else
                                         "sys_attn_mfma" if (spec.dtype == "bf16" and spec.head_dim == 128)
                                         else "sys_attn_tiled"),
                              "dispatches": 3 + steps,
                              "sys_kv_bytes": 2 * spec.num_kv_heads * spec.head_dim * E * spec.sys_len,
                              "us_per_call": round(1000 * e0.elapsed_time(e1) / steps, 2)}), flush=True)
            del t, ws, w
            torch.cuda.empty_cache()


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3
    counter summary, or None when there is none or the library's sources have
    changed since it was taken."""
    from shared_prompt_kv_amd import build as B
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("library_sources_sha256") != B.source_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------------------
# algorithmic work (what the method must move / compute, not implementation overhead)


def work_of(w):
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
    part_row = rows * (d + 1) * 4          # one fp32 output row + LSE per query row
    tables = 4 * B * (mb + 2) + (4 * (B + 1) if int(w.q_lens.max()) > 1 else 0)
    vis = 0
    for b in range(B):
        n, c = int(w.q_lens[b]), int(w.ctx_lens[b])
        vis += sum(c - n + t + 1 for t in range(n))
    return {
        "step_bytes": kv_sys + kv_ctx + rows * d * (E + 4) + tables,
        "step_flops": 4 * Hq * d * (Tq * s.sys_len + vis),
        "sys_attn": kv_sys + q_bytes,
        # the streaming launch: context (and, at <= 64 stacked rows per KV head, system) K/V
        "stream_attn": (kv_sys if w.total_q * s.group <= 64 else 0) + kv_ctx + q_bytes + tables,
        "relay_merge": 2 * part_row + rows * d * 4,
        "sys_flops": 4 * Hq * d * Tq * s.sys_len,
        "ctx_flops": 4 * Hq * d * vis,
    }


# ---------------------------------------------------------------------------------------


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self, torch):
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

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


def measure(torch, relay, w, steps, warmup, per_kernel=True, graph=True, prep=None):
    """Times decode steps over rotating input copies.

    graph: the steps captured in one HIP graph (a full rotation over the copies)
    and replayed, as a served model replays its decode step; the timed region holds
    `steps` steps.  eager: the same steps launched one by one through the prepared
    C-ABI call.  Per-kernel durations come from HIP events recorded by the library
    between its launches (eager).
    """
    t0 = relay.to_device(w, "cuda")
    if prep is not None:  # e.g. the no-relay baseline's inputs
        t0 = prep(t0)
    work = work_of(w)
    n_sets = max(2, math.ceil(3 * MALL_BYTES / max(work["step_bytes"], 1)))
    n_sets = min(n_sets, 16)
    sets = [t0] + [clone_set(torch, t0) for _ in range(n_sets - 1)]
    dims = relay.dims_of(t0)
    ws = relay.workspace(dims, t0["sys_len"], "cuda")
    outs = [torch.empty(t0["q"].shape, dtype=torch.float32, device="cuda") for _ in range(n_sets)]
    calls = [relay.DecodeCall(sets[i], outs[i], ws) for i in range(n_sets)]
    res = {"n_sets": n_sets, "work": work, "plan": relay.relay_get_plan(dims, t0["sys_len"])}

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
        evs = he.create(4 * steps)
        for i in range(steps):
            calls[i % n_sets].timed(evs[4 * i:4 * i + 4])
        torch.cuda.synchronize()
        # launch names: a separate (tiled) system launch, then the attention launch
        # (both steps together when sys_mode == 1), then relay_fuse
        mode = res["plan"]["sys_mode"]
        names = ("sys_attn", "stream_attn", "relay_merge")
        acc = dict.fromkeys(names, 0.0)
        for i in range(steps):
            e = evs[4 * i:4 * i + 4]
            for j, k in enumerate(names):
                acc[k] += he.elapsed_ms(e[j], e[j + 1])
        he.destroy(evs)
        res["kernel_us"] = {k: 1000.0 * v / steps for k, v in acc.items() if mode >= 2 or k != "sys_attn"}
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


def measured_hbm(torch):
    """What plain torch kernels reach on this GPU: a 1 GiB read (sum of a bf16 tensor)
    and a 512 MiB device copy (read + write), GB/s.  Context for the roofline fraction
    (the 8 TB/s peak is a spec figure); not part of the decode step."""
    x = torch.ones(2**29, dtype=torch.bfloat16, device="cuda")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def rate(fn, nbytes, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(nbytes / (e0.elapsed_time(e1) / n * 1e-3) / 1e9, 1)

    out = {"read_GBps": rate(lambda: x.sum(), x.numel() * 2),
           "copy_GBps": rate(lambda: dst.copy_(src), 2 * COPY_BYTES),
           "note": "torch sum over 1 GiB bf16 (read) and device copy of 512 MiB (read + write)"}
    del x, src, dst
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip() + f" ({os.cpu_count()} logical CPUs visible)"
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_cpu_s):
    """The oracle (unchanged) on the host cores, request by request through the
    workload (cycling), until about budget_cpu_s CPU-seconds have been spent."""
    import oracle
    import numpy as np

    P = oracle.Problem(w)
    Hq = w.spec.num_q_heads
    cores = oracle.num_threads()
    budget_wall = budget_cpu_s / max(cores, 1)
    tokens, elapsed, n = 0, 0.0, 0
    start = time.perf_counter()
    while elapsed < budget_wall:
        b = n % w.spec.batch
        lo, hi = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
        P.attention(np.arange(lo * Hq, hi * Hq, dtype=np.int64))
        tokens += hi - lo
        n += 1
        elapsed = time.perf_counter() - start
    return {"value": round(tokens / elapsed, 3), "unit": "query-tokens/s/layer", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"exact fp64 causal attention (all {Hq} heads) for {n} requests taken in order, "
                      f"cycling over the {w.spec.batch} requests of the same workload: {tokens} query "
                      f"tokens in {elapsed:.2f} s wall on {cores} threads"}


def point(torch, relay, spec, args, with_baseline=False):
    """One workload measured like the main line (fewer steps): throughput and
    roofline fractions; with_baseline adds the no-relay baseline's step time."""
    w = workloads_generate(spec)
    rr = measure(torch, relay, w, min(args.steps, 50), min(args.warmup, 10))
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
    if with_baseline:
        out.update(no_relay_baseline(torch, relay, w, args, m))
    return out


def no_relay_baseline(torch, relay, w, args, relay_ms):
    """The same decode step without relay: every request's block table starts with
    the shared system pages and the context step reads them once per request."""
    from shared_prompt_kv_amd import baseline
    rb = measure(torch, relay, w, min(args.steps, 50), min(args.warmup, 10), per_kernel=False,
                 prep=baseline.prefix_shared)
    bm = rb["ms_per_step"]
    print(f"[bench] {w.spec.name} no-relay baseline: {1000 * bm:.2f} us/step", file=sys.stderr, flush=True)
    return {"no_relay_us_per_step": round(1000 * bm, 2), "relay_speedup": round(bm / relay_ms, 3)}


def rope_append_time(torch, relay, w, args):
    """The step before the path on the same workload: position embedding of the new
    tokens' q and k at sys_len + context position and their K/V appended to the pages
    (relay_rope_append), timed alone with HIP events over back-to-back calls."""
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
    call = lambda: relay.relay_rope_append(dims, s.sys_len, q_new, k_new, v_new, tab, t["block_tables"],
                                           t["ctx_lens"], t["cu_q_lens"], t["ctx_k_pages"], t["ctx_v_pages"],
                                           q_out=q_out)
    for _ in range(10):
        call()
    torch.cuda.synchronize()
    n = min(args.steps, 200)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = 1000 * e0.elapsed_time(e1) / n
    E = 2 if s.dtype == "bf16" else 4
    nbytes = (2 * w.total_q * s.num_q_heads * s.head_dim * E      # q in and out
              + 4 * w.total_q * s.num_kv_heads * s.head_dim * E   # k, v in; k, v pages out
              + w.total_q * s.head_dim * 4)                       # one table row per token
    return {"us_per_call": round(us, 2), "bytes_alg": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "note": "back-to-back eager launches; a few MB per call, launch-latency bound"}


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


def workloads_generate(spec):
    import workloads
    return workloads.generate(spec)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the decode-attention path runs on a single MI355X; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    from shared_prompt_kv_amd import relay

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.sys_scaling:
        relay.load_library()
        sys_scaling(torch, relay, min(args.steps, 20))
        return
    if args.batch_sweep:
        relay.load_library()
        for B in BATCH_SWEEP:
            spec = workloads.config_spec(2, 0).replace(batch=B)
            r = point(torch, relay, spec, args, with_baseline=True)
            print(json.dumps({"shape": "llama2_7b_mha", "batch": B, "sys_len": spec.sys_len,
                              "relay_us_per_step": r["us_per_step"], "qtok_s": r["qtok_s"],
                              "no_relay_us_per_step": r["no_relay_us_per_step"],
                              "relay_speedup": r["relay_speedup"]}), flush=True)
        # long request contexts dilute the gain: the system share of the bytes shrinks
        for C in CTX_SWEEP:
            spec = workloads.config_spec(2, 0).replace(ctx_len_dist="fixed", ctx_lo=C, ctx_hi=C)
            r = point(torch, relay, spec, args, with_baseline=True)
            L, B = spec.sys_len, spec.batch
            print(json.dumps({"shape": "llama2_7b_mha", "batch": B, "sys_len": L, "ctx_len": C,
                              "relay_us_per_step": r["us_per_step"], "qtok_s": r["qtok_s"],
                              "no_relay_us_per_step": r["no_relay_us_per_step"],
                              "relay_speedup": r["relay_speedup"],
                              "kv_bytes_ratio": round(B * (L + C) / (L + B * C), 3)}), flush=True)
        return
    relay.load_library()
    spec = workloads.config_spec(args.config, args.sweep_index)
    w = workloads.generate(spec)
    r = measure(torch, relay, w, args.steps, args.warmup, graph=not args.no_graph)
    print(f"[bench] {spec.name}: {1000 * r['ms_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    work = r["work"]
    ms = r["ms_per_step"]
    value = w.total_q / (ms * 1e-3)
    kus = r["kernel_us"]
    dom = max(kus, key=kus.get)
    achieved = work[dom] / (kus[dom] * 1e-6) / 1e9
    step_hbm_frac = work["step_bytes"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)
    peak_flops = (BF16_PEAK_TFLOPS if spec.dtype == "bf16" else FP32_PEAK_TFLOPS) * 1e12
    step_mfma_frac = work["step_flops"] / (ms * 1e-3) / peak_flops
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
        "step_hbm_roofline_frac": round(step_hbm_frac, 4),
        "step_mfma_roofline_frac": round(step_mfma_frac, 5),
        "step_bytes_alg": work["step_bytes"],
        "kernel_us": {k: round(v, 3) for k, v in kus.items()},
        "plan": r["plan"],
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_alg_per_launch": work[dom], "traffic": stored_traffic(dom, spec.name)},
    }
    if not args.no_sweep and args.config == 2:
        line["sweep"] = {"workload": "llama30b_mha (batch 32, 52 heads, ctx 128)",
                         "points": [dict(sys_len=Ls, **point(torch, relay, workloads.config_spec(3, i), args,
                                                             with_baseline=True))
                                    for i, Ls in enumerate(workloads.CONFIG3_SYS_LENS)]}
        line["other_configs"] = [point(torch, relay, workloads.config_spec(c, 0), args, with_baseline=True)
                                 for c in (1, 4, 5)]
    if not args.no_sweep:
        line["no_relay_baseline"] = no_relay_baseline(torch, relay, w, args, ms)
        line["rope_append"] = rope_append_time(torch, relay, w, args)
        line["system_prefill"] = [prefill_time(torch, relay, workloads.config_spec(c, 0), args) for c in (2, 4)]
    if not args.no_sweep:
        line["hbm_measured"] = measured_hbm(torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
