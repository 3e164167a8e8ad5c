"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: fp32 inputs max|gpu - oracle| <= 1e-5; bf16 inputs (fp32 accumulation)
max|gpu - oracle| <= 2e-3 and ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2 over the
whole output.  Integer-valued properties (page relabelling, batch permutation,
poison, determinism) are checked bitwise.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
from shared_prompt_kv_amd import relay as R
import workloads as W

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16_ABS = 2e-3
TOL_BF16_REL = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    R.load_library()
    yield
    torch.cuda.synchronize()


def check(gpu, ref, dtype, what=""):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    gi, ri = np.isneginf(g), np.isneginf(r)
    np.testing.assert_array_equal(gi, ri, err_msg=f"{what}: -inf pattern")
    assert np.all(np.isfinite(g[~gi])), f"{what}: non-finite values"
    diff = np.abs(g[~gi] - r[~ri])
    err = float(diff.max()) if diff.size else 0.0
    if dtype == "f32":
        assert err <= TOL_F32, f"{what}: max abs {err:.3e} > {TOL_F32}"
    else:
        rel = float(np.linalg.norm(g[~gi] - r[~ri]) / max(np.linalg.norm(r[~ri]), 1e-30))
        assert err <= TOL_BF16_ABS, f"{what}: max abs {err:.3e} > {TOL_BF16_ABS}"
        assert rel <= TOL_BF16_REL, f"{what}: rel L2 {rel:.3e} > {TOL_BF16_REL}"
    return err


@functools.lru_cache(maxsize=4)
def workload(spec):
    return W.generate(spec)


def upload(w):
    return R.to_device(w, "cuda")


# ------------------------------------------------------------------------------------------
# small and medium cases: several tiles, ragged tails, every row checked

SMALL = [
    W.config_spec(1),
    W.config_spec(1).replace(name="c1-d128", head_dim=128, sys_len=77, ctx_lo=1, ctx_hi=70),
    W.config_spec(2).replace(batch=5, sys_len=333, ctx_lo=16, ctx_hi=100),
    W.config_spec(2).replace(name="c2-d64", head_dim=64, batch=3, sys_len=100, ctx_lo=1, ctx_hi=50),
    W.config_spec(3, 0).replace(batch=3, num_q_heads=6, num_kv_heads=6, sys_len=200),
    W.config_spec(4).replace(batch=9, sys_len=515, ctx_median=60, ctx_cap=200),
    W.config_spec(5).replace(batch=5, sys_len=290, ctx_lo=64, ctx_hi=300),
    W.config_spec(5).replace(name="c5-f32", dtype="f32", batch=3, sys_len=40, ctx_lo=17, ctx_hi=99),
    W.config_spec(5).replace(name="c5-g8", batch=3, num_q_heads=32, num_kv_heads=4, sys_len=64,
                             ctx_lo=20, ctx_hi=90),
    # 17..32 stacked rows over >= 384 (head, chunk) groups: system units of two row tiles
    # (the second one ragged), a ragged last chunk
    W.config_spec(3, 0).replace(name="c3-two-tile", batch=24, num_q_heads=16, num_kv_heads=16,
                                sys_len=12000, ctx_lo=40, ctx_hi=40),
    W.config_spec(1).replace(name="c1-two-tile-f32", batch=20, num_q_heads=24, num_kv_heads=24,
                             sys_len=8200, ctx_lo=1, ctx_hi=40),
    # a single request (one stacked row per KV head), MHA and GQA
    W.config_spec(2).replace(name="c2-B1", batch=1),
    W.config_spec(4).replace(name="c4-B1", batch=1, sys_len=3000),
    # 33..64 stacked rows: system streams of four row tiles
    W.config_spec(2).replace(name="c2-B48", batch=48, sys_len=700, ctx_lo=16, ctx_hi=200),
    # more than 64 stacked rows per KV head at head_dim 64 or fp32: the tiled system kernel
    W.config_spec(4).replace(name="c4-d64-bf16", head_dim=64, batch=20, sys_len=333, ctx_median=60, ctx_cap=200),
    W.config_spec(4).replace(name="c4-d64-f32", dtype="f32", head_dim=64, batch=20, sys_len=333,
                             ctx_median=60, ctx_cap=200),
    W.config_spec(4).replace(name="c4-d128-f32", dtype="f32", batch=20, sys_len=150, ctx_median=40, ctx_cap=100),
    # MHA with more than 64 stacked rows (g = 1): the matrix-core system kernel at batch 128
    W.config_spec(2).replace(name="c2-B128", batch=128),
]
SMALL_IDS = [f"{s.name}-B{s.batch}-L{s.sys_len}-d{s.head_dim}" for s in SMALL]


@pytest.mark.parametrize("spec", SMALL, ids=SMALL_IDS)
def test_decode_matches_oracle_small(spec):
    say(f"[parity] relay_attn_decode {spec}")
    w = workload(spec)
    t = upload(w)
    out = R.decode_workload(t)
    torch.cuda.synchronize()
    ref, _ = oracle.Problem(w).attention()
    check(out.cpu().numpy(), ref, spec.dtype, "out")


@pytest.mark.parametrize("spec", SMALL, ids=SMALL_IDS)
def test_system_step_matches_oracle(spec):
    say(f"[parity] relay_sys_attn {spec}")
    w = workload(spec)
    t = upload(w)
    o, lse = R.relay_sys_attn(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], R.dims_of(t))
    torch.cuda.synchronize()
    ro, rl = oracle.Problem(w).system_part()
    check(o.cpu().numpy(), ro, spec.dtype, "o_sys")
    check(lse.cpu().numpy(), rl, spec.dtype, "lse_sys")


@pytest.mark.parametrize("spec", SMALL, ids=SMALL_IDS)
def test_context_step_matches_oracle(spec):
    say(f"[parity] relay_ctx_attn {spec}")
    w = workload(spec)
    t = upload(w)
    o, lse = R.relay_ctx_attn(t["q"], t["ctx_k_pages"], t["ctx_v_pages"], t["block_tables"],
                              t["ctx_lens"], t["cu_q_lens"], R.dims_of(t))
    torch.cuda.synchronize()
    ro, rl = oracle.Problem(w).context_part()
    check(o.cpu().numpy(), ro, spec.dtype, "o_ctx")
    check(lse.cpu().numpy(), rl, spec.dtype, "lse_ctx")


def test_fuse_on_oracle_partials():
    say("[parity] relay_fuse on oracle partials")
    w = workload(W.config_spec(5).replace(batch=4, sys_len=150, ctx_lo=64, ctx_hi=200))
    P = oracle.Problem(w)
    o_s, l_s = P.system_part()
    o_c, l_c = P.context_part()
    ref, ref_lse, _ = oracle.relay_fuse(o_s, l_s, o_c, l_c)
    # force empty parts on some rows: a -inf LSE carries weight 0
    l_s = l_s.copy()
    l_s[0, :] = -np.inf
    o_s = o_s.copy()
    o_s[0, :] = 0.0
    ref[0], ref_lse[0] = o_c[0], l_c[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    out, lse = R.relay_fuse(dev(o_s), dev(l_s), dev(o_c), dev(l_c))
    torch.cuda.synchronize()
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-6
    assert np.max(np.abs(lse.cpu().numpy() - ref_lse)) <= 1e-5
    out16, _ = R.relay_fuse(dev(o_s), dev(l_s), dev(o_c), dev(l_c), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # bf16 output: within one bf16 ulp of the fp64 result
    o16 = out16.float().cpu().numpy().astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(o16 - ref) <= ulp + 1e-6)


# ------------------------------------------------------------------------------------------
# edge cases


def test_zero_system_length_equals_context_attention():
    spec = W.config_spec(2).replace(batch=4, sys_len=0, ctx_lo=1, ctx_hi=90)
    say(f"[parity] sys_len=0 {spec}")
    w = workload(spec)
    t = upload(w)
    out = R.decode_workload(t)
    o, lse = R.relay_sys_attn(t["q"], t["sys_k"], t["sys_v"], 0, R.dims_of(t))
    torch.cuda.synchronize()
    ref, _ = oracle.Problem(w).attention()
    check(out.cpu().numpy(), ref, "bf16", "out")
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_single_token_contexts_and_tiny_system():
    spec = W.config_spec(1).replace(batch=7, sys_len=1, ctx_lo=1, ctx_hi=1)
    say(f"[parity] ctx_len=1 {spec}")
    w = workload(spec)
    out = R.decode_workload(upload(w))
    torch.cuda.synchronize()
    check(out.cpu().numpy(), oracle.Problem(w).attention()[0], "f32", "out")


def test_nan_poison_never_reaches_output():
    spec = W.config_spec(5).replace(batch=4, sys_len=45, ctx_lo=20, ctx_hi=75)
    say(f"[parity] NaN poison {spec}")
    a = R.decode_workload(upload(workload(spec)))
    b = R.decode_workload(upload(workload(spec.replace(poison="nan"))))
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(b))
    assert torch.equal(a, b)


def test_page_relabelling_is_bitwise_invariant():
    spec = W.config_spec(4).replace(batch=6, sys_len=100, ctx_median=50, ctx_cap=150)
    say(f"[parity] relabel {spec}")
    w = workload(spec)
    a = R.decode_workload(upload(w))
    b = R.decode_workload(upload(W.relabel_pages(w, 11)))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_batch_permutation_permutes_output():
    import dataclasses
    spec = W.config_spec(5).replace(batch=4, sys_len=70, ctx_lo=20, ctx_hi=60)
    say(f"[parity] batch permutation {spec}")
    w = workload(spec)
    perm = np.array([3, 1, 0, 2])
    cu = w.cu_q_lens
    q2 = np.concatenate([w.q[cu[b]:cu[b + 1]] for b in perm])
    ql = w.q_lens[perm]
    w2 = dataclasses.replace(w, q=np.ascontiguousarray(q2), block_tables=np.ascontiguousarray(w.block_tables[perm]),
                             ctx_lens=np.ascontiguousarray(w.ctx_lens[perm]), q_lens=ql,
                             cu_q_lens=np.concatenate([[0], np.cumsum(ql)]).astype(np.int32))
    a = R.decode_workload(upload(w)).cpu()
    b = R.decode_workload(upload(w2)).cpu()
    assert torch.equal(b, torch.cat([a[cu[i]:cu[i + 1]] for i in perm]))


def test_run_to_run_determinism():
    spec = W.config_spec(2).replace(batch=8, sys_len=700, ctx_lo=16, ctx_hi=300)
    say(f"[parity] determinism {spec}")
    t = upload(workload(spec))
    a = R.decode_workload(t)
    b = R.decode_workload(t)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bf16_output():
    spec = W.config_spec(2).replace(batch=4, sys_len=260, ctx_lo=16, ctx_hi=90)
    say(f"[parity] bf16 out {spec}")
    w = workload(spec)
    out = R.decode_workload(upload(w), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, _ = oracle.Problem(w).attention()
    g = out.float().cpu().numpy().astype(np.float64)
    # fp32 tolerance plus one bf16 ulp of the value
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(g - ref) <= TOL_BF16_ABS + ulp)


# ------------------------------------------------------------------------------------------
# full configuration sizes: every row, except the long-prompt multi-token workload (about
# 40 s of oracle per row block of rows), where 2000 sampled rows are checked

FULL = [(1, 0, None), (2, 0, None)] + [(3, i, None) for i in range(len(W.CONFIG3_SYS_LENS))] + \
    [(4, 0, None), (5, 0, 2000)]


@pytest.mark.parametrize("cfg,sweep,n_rows", FULL, ids=[f"c{c}s{s}" for c, s, _ in FULL])
def test_decode_matches_oracle_full_size(cfg, sweep, n_rows):
    spec = W.config_spec(cfg, sweep)
    say(f"[parity] full size {spec} rows={n_rows or 'all'}")
    w = W.generate(spec)
    t = upload(w)
    out = R.decode_workload(t)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(-1, spec.head_dim)
    P = oracle.Problem(w)
    if n_rows is None:
        ref, _ = P.attention()
        check(out, ref.reshape(-1, spec.head_dim), spec.dtype, "out")
    else:
        n_all = w.total_q * spec.num_q_heads
        rng = np.random.default_rng(1000 + cfg)
        rows = np.unique(np.concatenate([[0, n_all - 1], rng.integers(0, n_all, n_rows)]))
        ref, _ = P.attention(rows)
        check(out[rows], ref, spec.dtype, "out")
    del t
    torch.cuda.empty_cache()


def test_graph_replay_matches_eager():
    """The decode call captured in a HIP graph: every replay (with eager work and
    synchronisations between replays) equals the eager result bitwise."""
    spec = W.config_spec(2).replace(batch=6, sys_len=300, ctx_lo=16, ctx_hi=140)
    say(f"[parity] graph replay {spec}")
    w = workload(spec)
    t = upload(w)
    dims = R.dims_of(t)
    ws = R.workspace(dims, t["sys_len"], "cuda")
    ref = R.decode_workload(t, workspace_buf=ws).clone()
    out = torch.empty_like(ref)
    call = R.DecodeCall(t, out, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    other = upload(workload(W.config_spec(1)))
    for rep in range(4):
        out.fill_(float("nan"))
        R.decode_workload(other)            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs"
    expect, _ = oracle.Problem(w).attention()
    check(out.cpu().numpy(), expect, "bf16", "graph out")


# ------------------------------------------------------------------------------------------
# the unit schedule at other shapes; a workspace full of garbage

SCHED_SPECS = [
    W.config_spec(2).replace(batch=12, sys_len=1100, ctx_lo=16, ctx_hi=700),
    W.config_spec(4).replace(batch=40, sys_len=700, ctx_median=200, ctx_cap=1500),
    W.config_spec(5).replace(batch=6, sys_len=900, ctx_lo=64, ctx_hi=1200),
]


@pytest.mark.parametrize("spec", SCHED_SPECS, ids=[s.name for s in SCHED_SPECS])
def test_multi_split_shapes(spec):
    """Several context splits and row blocks per request, grids smaller than the unit
    count: every unit runs once (oracle parity, deterministic bits)."""
    say(f"[parity] multi-split {spec}")
    w = workload(spec)
    t = upload(w)
    a = R.decode_workload(t).cpu()
    b = R.decode_workload(t).cpu()
    assert torch.equal(a, b)
    expect, _ = oracle.Problem(w).attention()
    check(a.numpy(), expect, spec.dtype, "multi-split")


# shapes whose matrix-core system runs cross KV-head boundaries: (batch, sys_len); 1 query
# token per request, 32 / 8 heads, so M = 4 B stacked rows per KV head in row blocks of
# the plan's rows per workgroup and slots // row_blocks runs over the 8 heads' 64-key
# steps (slots: one workgroup per CU, or two for 128-row blocks in a launch of their own)
CROSSING = [(75, 1920), (150, 2560), (200, 1000)]


def _runs_cross_heads(batch, sys_len, plan, hkv=8, g=4):
    rows = plan["sys_rows_per_wg"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if plan["sys_mode"] == 2 and rows == 128:
        cus *= 2
    rb = -(-batch * g // rows)
    sph = -(-sys_len // 64)
    S = hkv * sph
    parts = min(max(cus // rb, 1), S)
    return any((p * S // parts) % sph for p in range(1, parts))


@pytest.mark.parametrize("batch,sys_len", CROSSING, ids=[f"B{b}-L{l}" for b, l in CROSSING])
def test_system_runs_across_heads(batch, sys_len):
    """Matrix-core system step whose key runs cross KV-head boundaries (each run one
    partial per head it touches, unused slots empty), step alone and whole decode."""
    spec = W.config_spec(4).replace(batch=batch, sys_len=sys_len, ctx_median=60, ctx_cap=300)
    say(f"[parity] system runs across heads {spec}")
    w = workload(spec)
    t = upload(w)
    plan = R.relay_get_plan(R.dims_of(t), t["sys_len"])
    assert plan["sys_mode"] in (2, 4) and plan["sys_runs"] >= 2
    assert _runs_cross_heads(batch, sys_len, plan)
    o, lse = R.relay_sys_attn(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], R.dims_of(t))
    out = R.decode_workload(t)
    torch.cuda.synchronize()
    P = oracle.Problem(w)
    ro, rl = P.system_part()
    check(o.cpu().numpy(), ro, spec.dtype, "o_sys")
    check(lse.cpu().numpy(), rl, spec.dtype, "lse_sys")
    ref, _ = P.attention()
    check(out.cpu().numpy(), ref, spec.dtype, "out")


# the system step alone on the eight-wave two-group kernel (256 rows per workgroup, one
# workgroup per CU): (batch, sys_len, sign of the scale).  M = 4 B stacked rows per KV
# head; B = 120 leaves the last row block partly padded; sys_len 3000 and 1000 end inside
# a 64-key step and inside a 16-key tile; the runs of 64-key steps cross KV heads
TWO_GROUP = [(64, 3000, 1), (120, 1000, 1), (64, 1000, -1)]


@pytest.mark.parametrize("batch,sys_len,sign", TWO_GROUP,
                         ids=[f"B{b}-L{l}-{'neg' if g < 0 else 'pos'}" for b, l, g in TWO_GROUP])
def test_system_two_group_kernel(batch, sys_len, sign):
    """relay_sys_attn on the two-group matrix-core kernel: every row's system-part output
    and log-sum-exp against the oracle (a negative scale included: its sign is folded
    into the query)."""
    spec = W.config_spec(4).replace(batch=batch, sys_len=sys_len, ctx_median=60, ctx_cap=300)
    say(f"[parity] two-group system kernel {spec} sign {sign}")
    w = workload(spec)
    t = upload(w)
    t["scale"] = sign * spec.scale
    d = R.dims_of(t)
    M = batch * spec.group
    assert 10 * 256 * -(-M // 256) <= 11 * 128 * -(-M // 128)  # the plan's rule for 256 rows
    o, lse = R.relay_sys_attn(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], d)
    torch.cuda.synchronize()
    ro, rl = oracle.Problem(w, scale=sign * spec.scale).system_part()
    check(o.cpu().numpy(), ro, spec.dtype, "o_sys")
    check(lse.cpu().numpy(), rl, spec.dtype, "lse_sys")


def test_steps_full_size_gqa():
    """System step and context step alone at the full Llama-3-8B GQA size (256 requests,
    8192 system keys, lognormal contexts): every row against the oracle's parts."""
    spec = W.config_spec(4)
    say(f"[parity] per-step full size {spec}")
    w = W.generate(spec)
    t = upload(w)
    dims = R.dims_of(t)
    o_s, l_s = R.relay_sys_attn(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], dims)
    o_c, l_c = R.relay_ctx_attn(t["q"], t["ctx_k_pages"], t["ctx_v_pages"], t["block_tables"], t["ctx_lens"],
                                t["cu_q_lens"], dims)
    torch.cuda.synchronize()
    P = oracle.Problem(w)
    ro, rl = P.system_part()
    check(o_s.cpu().numpy(), ro, spec.dtype, "o_sys")
    check(l_s.cpu().numpy(), rl, spec.dtype, "lse_sys")
    ro, rl = P.context_part()
    check(o_c.cpu().numpy(), ro, spec.dtype, "o_ctx")
    check(l_c.cpu().numpy(), rl, spec.dtype, "lse_ctx")
    del t
    torch.cuda.empty_cache()


def test_many_requests_in_several_streaming_launches():
    """More requests than one streaming launch takes (2880): the context streams run as
    several launches over request groups; every row against the oracle."""
    spec = W.config_spec(4).replace(name="c4-B4100", batch=4100, sys_len=100, ctx_median=20, ctx_cap=40)
    say(f"[parity] request groups {spec}")
    w = workload(spec)
    t = upload(w)
    plan = R.relay_get_plan(R.dims_of(t), t["sys_len"])
    assert plan["stream_launches"] == 2
    out = R.decode_workload(t)
    torch.cuda.synchronize()
    ref, _ = oracle.Problem(w).attention()
    check(out.cpu().numpy(), ref, spec.dtype, "out")


# ------------------------------------------------------------------------------------------
# pieces past the places fixed in advance: the plan sizes the fixed places from an
# estimate (the context lengths are device data); pieces past them take the stream slots

def _piece_counts(w, plan):
    """Most pieces of one KV head's system stream and of one context stream, from the
    equal split of the launch's 32-key steps over its waves (the partition the header
    documents for relay_plan.stream_waves), for one query token per request."""
    spec = w.spec
    H, ss = spec.num_kv_heads, -(-spec.sys_len // 32)
    steps = [max(1, -(-int(c) // 32)) for c in w.ctx_lens]
    T = H * ss + H * sum(steps)
    Wv = min(T, plan["stream_waves"])
    part = lambda x: ((x + 1) * Wv + T - 1) // T - 1
    n_sys = max(part(h * ss + ss - 1) // 4 - part(h * ss) // 4 + 1 for h in range(H)) if ss else 0
    n_ctx, p0 = 0, H * ss
    for s in steps:
        for _ in range(H):
            n_ctx = max(n_ctx, part(p0 + s - 1) - part(p0) + 1)
            p0 += s
    return n_sys, n_ctx


OVERFLOW = [
    # contexts far shorter than the declared longest one: the step estimate is too high,
    # so system streams fall into more workgroups than their fixed slots
    ("sys", W.config_spec(2).replace(name="c2-short-ctx", batch=24, sys_len=3000, ctx_lo=8, ctx_hi=40), 4096),
    ("sys", W.config_spec(1).replace(name="c1-short-ctx", batch=16, num_q_heads=4, num_kv_heads=4,
                                      sys_len=900, ctx_lo=1, ctx_hi=20), 8192),
    # one long context over many waves: more context pieces than the row's own slots
    ("ctx", W.config_spec(2).replace(name="c2-long-ctx", batch=2, num_q_heads=4, num_kv_heads=4,
                                      sys_len=64, ctx_lo=2500, ctx_hi=3000), None),
]


@pytest.mark.parametrize("kind,spec,declared", OVERFLOW, ids=[s.name for _, s, _ in OVERFLOW])
def test_pieces_past_the_fixed_places(kind, spec, declared):
    say(f"[parity] pieces past the fixed places ({kind}) {spec} declared max_ctx_len {declared}")
    w = workload(spec)
    t = upload(w)
    if declared:
        # a larger declared bound, with block tables wide enough for it (padding entries
        # are never read)
        cols = -(-declared // 16)
        bt = t["block_tables"]
        t = dict(t, max_ctx_len=declared,
                 block_tables=torch.nn.functional.pad(bt, (0, cols - bt.shape[1])).contiguous())
    plan = R.relay_get_plan(R.dims_of(t), t["sys_len"])
    n_sys, n_ctx = _piece_counts(w, plan)
    if kind == "sys":
        assert plan["sys_mode"] == 1 and n_sys > plan["sys_row_slots"] >= 1, (plan, n_sys)
    else:
        assert n_ctx > plan["ctx_row_slots"] >= 1, (plan, n_ctx)
    out = R.decode_workload(t)
    torch.cuda.synchronize()
    ref, _ = oracle.Problem(w).attention()
    check(out.cpu().numpy(), ref, spec.dtype, f"pieces past the fixed places ({kind})")


def test_garbage_workspace():
    """Whatever the workspace held (here random bytes), a call gives the same bits."""
    spec = SCHED_SPECS[0]
    say(f"[parity] garbage workspace {spec}")
    t = upload(workload(spec))
    dims = R.dims_of(t)
    ws = R.workspace(dims, t["sys_len"], "cuda")
    ref = R.decode_workload(t, workspace_buf=ws).clone()
    g = torch.Generator(device="cuda").manual_seed(7)
    for _ in range(3):
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=g).view(ws.dtype))
        assert torch.equal(R.decode_workload(t, workspace_buf=ws), ref)
