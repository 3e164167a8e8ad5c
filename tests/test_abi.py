"""C-ABI library checks that need no GPU: exported symbols, argument validation,
the work plan and relay_validate.  No call here enqueues device work."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

from shared_prompt_kv_amd import relay as R
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relay_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(R.LIB_PATH):
        from shared_prompt_kv_amd import build
        build.build()
    return R.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(relay_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(R.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", R.LIB_PATH]).decode()
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_noalloc_scratch_size_matches_the_header():
    m = re.search(r"#define RELAY_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == R.NOALLOC_SCRATCH_BYTES


def test_library_is_gfx950_only(lib):
    # the device code objects are embedded for gfx950 alone
    blob = open(R.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in blob


def test_abi_version_and_strerror(lib):
    assert R.relay_abi_version() == 6
    assert lib.relay_strerror(0) == b"ok"
    assert lib.relay_strerror(-3) == b"workspace too small"


def base_dims(**kw):
    d = dict(batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
             max_blocks_per_seq=8, num_blocks=40, total_q=4, max_q_len=1, max_ctx_len=128,
             scale=0.088, in_dtype=1, out_dtype=0)
    d.update(kw)
    return R.relay_dims(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -1),
    (dict(num_q_heads=6, num_kv_heads=4), -1),
    (dict(num_kv_heads=0), -1),
    (dict(head_dim=96), -2),
    (dict(block_size=32), -2),
    (dict(in_dtype=7), -2),
    (dict(out_dtype=3), -2),
    (dict(total_q=0), -1),
    (dict(max_q_len=5), -1),
    (dict(max_ctx_len=0), -1),
    (dict(max_blocks_per_seq=7), -1),
    (dict(num_blocks=0), -1),
    (dict(scale=math.inf), -1),
])
def test_invalid_dims_rejected_before_any_device_work(lib, kw, code):
    d = base_dims(**kw)
    rc = lib.relay_attn_decode(ctypes.byref(d), *([ctypes.c_void_p(16)] * 3), 100,
                               *([ctypes.c_void_p(16)] * 6), ctypes.c_void_p(256), 1 << 30, None)
    assert rc == code, lib.relay_last_error()
    assert lib.relay_last_error()
    assert lib.relay_workspace_size(ctypes.byref(d), 100) == 0


def test_pointer_and_workspace_errors(lib):
    d = base_dims()
    p = ctypes.c_void_p(4096)
    args = lambda **o: [o.get("q", p), p, p, 100, p, p, p, p, None, o.get("out", p),
                        o.get("ws", ctypes.c_void_p(4096)), o.get("n", 1 << 30), None]
    assert lib.relay_attn_decode(ctypes.byref(d), *args(q=None)) == -1
    assert lib.relay_attn_decode(ctypes.byref(d), *args(out=ctypes.c_void_p(4100))) == -1   # misaligned
    assert lib.relay_attn_decode(ctypes.byref(d), *args(ws=ctypes.c_void_p(4096 + 16))) == -1
    need = lib.relay_workspace_size(ctypes.byref(d), 100)
    assert need > 0
    assert lib.relay_attn_decode(ctypes.byref(d), *args(n=need - 1)) == -3
    # cu_q_lens == NULL requires one query per request
    d2 = base_dims(total_q=6, max_q_len=2)
    assert lib.relay_attn_decode(ctypes.byref(d2), *args()) == -1
    assert lib.relay_fuse(10, 96, p, p, p, p, p, 0, None, None) == -2
    assert lib.relay_fuse(-1, 128, p, p, p, p, p, 0, None, None) == -1
    assert lib.relay_fuse(0, 128, None, None, None, None, None, 0, None, None) == 0


CUS = 256          # no GPU here: the library plans for 256 compute units


def corun(d, sys_len):
    """The plan's choice for the decode step's matrix-core system workgroups (bf16, d = 128,
    > 64 rows per KV head): inside the streaming launch unless the system step's
    matrix-core time (at 0.9 PFLOP/s) exceeds twice the context step's memory time (at
    4.5 TB/s, half of max_ctx_len per request)."""
    t_sys = 4.0 * d.num_q_heads * d.head_dim * d.total_q * sys_len / 0.9e15
    t_ctx = 4.0 * d.num_kv_heads * d.head_dim * d.batch * (d.max_ctx_len / 2.0 + 16.0) / 4.5e12
    return t_ctx > 0.5 * t_sys


def stream_grid(bf16, D, rts, rtc):
    """Workgroups of a streaming launch: two per CU where the instantiation's registers
    fit two waves per SIMD (the header's plan contract), else one."""
    if bf16:
        per_cu = 1 if (D == 128 and rts == 4) else 2
    elif D == 128:
        per_cu = 1 if (rts >= 2 or rtc == 2) else 2
    else:
        per_cu = 1 if rts == 4 else 2
    return CUS * per_cu


def a256(x):
    return -(-x // 256) * 256


def row_slots(d, sys_len, sys_mode, waves, ctx=True):
    """The rows' own piece slots the plan reserves (the header's relay_plan contract):
    context, the most waves the longest stream (S 32-key steps) falls into when each wave
    holds at least (system steps + one per stream) // waves steps, at most min(4, S);
    system streams, the most workgroups of four waves one KV head's steps fall into when
    the launch holds the system steps plus, per context stream, half the longest
    context's steps (all W waves share the steps equally), plus one when the launch also
    holds context streams; capped so that both fit 16.  None with the system kernel's runs
    or more than 4096 output rows."""
    if sys_mode > 1 or d.total_q * d.num_q_heads > 4096:
        return 0, 0
    cap = min(d.max_ctx_len, d.max_blocks_per_seq * 16)
    max_steps = max(1, -(-cap // 32))
    ss = -(-sys_len // 32) if sys_mode == 1 else 0
    Ts = d.num_kv_heads * ss
    kc = 0
    if ctx:
        per_wave = max(1, (Ts + d.batch * d.num_kv_heads) // waves)
        kc = min(4, max_steps, -(-(max_steps - 1) // per_wave) + 1)
    ks = 0
    if sys_mode == 1:
        T = Ts + (d.batch * d.num_kv_heads * ((max_steps + 1) // 2) if ctx else 0)
        W = min(T, waves)
        part = lambda x: ((x + 1) * W + T - 1) // T - 1
        most = max(part(h * ss + ss - 1) // 4 - part(h * ss) // 4 + 1 for h in range(d.num_kv_heads))
        ks = min(most + (1 if ctx else 0), 16 - kc)
    return ks, kc


def test_workspace_covers_the_plan(lib):
    """Workspace = the partial regions of the streaming launch, laid out as the header says:
    system pieces (H_kv (sys_row_slots + 1) + workgroups slots of 16 * sys_row_tiles rows),
    their descriptors, context pieces (B H_kv row_blocks + waves slots per request group),
    row descriptors and every row's ctx_row_slots own slots."""
    d = base_dims()               # B 4, H_q 8 / H_kv 2 -> M = 16 stacked rows per KV head
    plan = R.relay_get_plan(d, 1000)
    assert plan["sys_mode"] == 1 and plan["sys_row_tiles"] == 1
    assert plan["ctx_row_tiles"] == 1 and plan["ctx_row_blocks"] == 1
    grid = stream_grid(True, 128, 1, 1)
    assert plan["stream_waves"] == 4 * grid and plan["stream_launches"] == 1 and plan["launches"] == 2
    rows, D, H = 4 * 8, 128, 2
    ks, kc = row_slots(d, 1000, 1, 4 * grid)
    assert (plan["sys_row_slots"], plan["ctx_row_slots"]) == (ks, kc) and ks >= 1 and kc == 4
    sys_slots, ctx_slots = H * (ks + 1) + grid, 4 * H * 1 + 4 * grid
    expect = (a256(sys_slots * 16 * D * 4) + a256(sys_slots * 16 * 4) + a256(H * 2 * 4)
              + a256(ctx_slots * 16 * D * 4) + a256(ctx_slots * 16 * 4) + a256(rows * 16)
              + a256(rows * kc * D * 4) + a256(rows * kc * 4))
    assert R.relay_workspace_size(d, 1000) == expect
    p0 = R.relay_get_plan(d, 0)
    assert p0["sys_mode"] == 0 and p0["launches"] == 2
    assert (p0["sys_row_slots"], p0["ctx_row_slots"]) == (0, 4)
    ctx0 = 4 * H + 4 * stream_grid(True, 128, 0, 1)
    assert R.relay_workspace_size(d, 0) == (a256(ctx0 * 16 * D * 4) + a256(ctx0 * 16 * 4) + a256(rows * 16)
                                            + a256(rows * 4 * D * 4) + a256(rows * 4 * 4))


@pytest.mark.parametrize("cfg,sweep", [(1, 0), (2, 0), (3, 0), (3, 5), (4, 0), (5, 0)])
def test_plan_for_each_config(lib, cfg, sweep):
    spec = W.config_spec(cfg, sweep)
    s = W.expected_sizes(spec)
    d = R.relay_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, 16,
                     -(-s["max_ctx"] // 16), 1000, s["total_q"], int(s["q_lens"].max()), s["max_ctx"],
                     spec.scale, 1 if spec.dtype == "bf16" else 0, 0)
    plan = R.relay_get_plan(d, spec.sys_len)
    M = s["total_q"] * spec.group
    if M <= 64:   # system streams (all M rows of a KV head) in the streaming launch
        assert plan["sys_mode"] == 1 and plan["launches"] == 2
        tiles = -(-M // 16)
        assert plan["sys_row_tiles"] == (tiles if tiles <= 2 else 4)
        assert plan["sys_runs"] == 0 and plan["sys_wgs"] == 0
    else:         # matrix-core system workgroups, (row block, run of 64-key steps)
        co = corun(d, spec.sys_len)
        if co:    # inside the streaming launch, one per CU
            assert plan["sys_mode"] == 4 and plan["launches"] == 2
        else:     # a launch of their own first, one workgroup per CU: 256 rows where the
            # 256-row blocks pad at most 10 % more rows than 128-row ones, else 128
            assert plan["sys_mode"] == 2 and plan["launches"] == 3
        pp = not co and 10 * 256 * -(-M // 256) <= 11 * 128 * -(-M // 128)
        assert plan["sys_rows_per_wg"] == (256 if pp else 128)
        row_blocks = -(-M // plan["sys_rows_per_wg"])
        steps = spec.num_kv_heads * -(-spec.sys_len // 64)
        parts = min(max((CUS if co or pp else 2 * CUS) // row_blocks, 1), steps)
        assert plan["sys_wgs"] == -(-row_blocks * parts // 8) * 8
        # slots: the most runs one head's steps fall into
        part_of = lambda x: ((x + 1) * parts + steps - 1) // steps - 1
        sph = steps // spec.num_kv_heads
        assert plan["sys_runs"] == max(part_of(h * sph + sph - 1) - part_of(h * sph) + 1
                                       for h in range(spec.num_kv_heads))
    R_ = int(s["q_lens"].max()) * spec.group      # query rows per (request, KV head)
    assert plan["ctx_row_tiles"] == (1 if R_ <= 16 else 2)
    assert plan["ctx_row_blocks"] == -(-R_ // (16 * plan["ctx_row_tiles"]))
    rts = plan["sys_row_tiles"] if plan["sys_mode"] == 1 else 0
    # beside the system workgroups: one context workgroup per CU
    grid = CUS if plan["sys_mode"] == 4 else stream_grid(spec.dtype == "bf16", spec.head_dim, rts,
                                                         plan["ctx_row_tiles"])
    assert plan["stream_waves"] == 4 * grid and plan["stream_launches"] == 1
    assert plan["stream_max_requests"] == spec.batch
    assert (plan["sys_row_slots"], plan["ctx_row_slots"]) == row_slots(d, spec.sys_len, plan["sys_mode"],
                                                                       plan["stream_waves"])


def test_requests_in_groups_of_one_streaming_launch(lib):
    """More requests than one launch's tables hold: the context streams run as several
    launches over request groups (2880 requests each)."""
    d = base_dims(batch=9000, total_q=9000, num_blocks=90000, max_ctx_len=100, max_blocks_per_seq=7)
    plan = R.relay_get_plan(d, 500)
    assert corun(d, 500) and plan["sys_mode"] == 4 and plan["stream_max_requests"] == 2880
    assert plan["stream_launches"] == 4 and plan["launches"] == 5   # system workgroups in the first
    ws = R.relay_workspace_size(d, 500)
    assert ws >= 4 * (2880 * 2 + 4 * stream_grid(True, 128, 0, 1)) * 16 * 129 * 4


def test_key_tile_layout_matches_the_header_formula():
    """The key layout the header documents (element c of key r at ((c/G)*16 + slot(r))*G
    + c%G, slot() read from the header text) is the layout the generator writes."""
    text = open(HEADER).read()
    m = re.search(r"slot\(r\) = ([\d, ]+) for\s*\n?\s*\*?\s*r = 0\.\.15", text)
    assert m, "slot() table not found in the header"
    slot = [int(x) for x in m.group(1).replace(" ", "").split(",") if x]
    assert sorted(slot) == list(range(16)) and all(slot[slot[r]] == r for r in range(16))
    rng = np.random.default_rng(5)
    for dtype, G, d in (("bf16", 8, 128), ("f32", 4, 128), ("bf16", 8, 64), ("f32", 4, 64)):
        tile = rng.integers(0, 60000, size=(16, d)).astype(np.uint16 if dtype == "bf16" else np.float32)
        flat = np.empty(16 * d, tile.dtype)
        for r in range(16):
            for c in range(d):
                flat[((c // G) * 16 + slot[r]) * G + c % G] = tile[r, c]
        assert np.array_equal(W.k_tiles(tile[None], dtype).reshape(-1), flat), dtype
        assert np.array_equal(W.k_untile(W.k_tiles(tile[None], dtype))[0], tile)


def test_prefill_workspace_holds_only_the_system_runs(lib):
    """The offline prefill's workspace is its causal system runs (at most a few per row),
    not the decode plan's context partials: bounded at the long-prompt shape."""
    L, Hq, Hkv, D = 65536, 32, 8, 128
    d = R.relay_dims(1, Hq, Hkv, D, 16, L // 16, L // 16, L, L, L, D ** -0.5, 1, 0)
    n = R.load_library().relay_prefill_workspace_size(ctypes.byref(d), L)
    rows = L * Hq
    assert 0 < n <= 4 * rows * (D + 1) * 4 + 4096
    d2 = R.relay_dims(1, 32, 32, D, 16, 512, 512, 8192, 8192, 8192, D ** -0.5, 1, 0)
    n2 = R.load_library().relay_prefill_workspace_size(ctypes.byref(d2), 8192)
    assert 0 < n2 <= 8 * 8192 * 32 * (D + 1) * 4


def meta(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="meta")


def decode_args(**o):
    """Well-formed relay_attn_decode tensors (meta: shapes and dtypes only): B 3, H_q 8,
    H_kv 2, d 128, bf16, sys_len 40 (3 tiles), 10 pages."""
    import torch
    bf = torch.bfloat16
    a = dict(q=meta((3, 8, 128), bf), sys_k=meta((2, 3, 16, 16, 8), bf), sys_v=meta((2, 3, 128, 16), bf),
             sys_len=40, ctx_k_pages=meta((10, 2, 16, 16, 8), bf), ctx_v_pages=meta((10, 2, 128, 16), bf),
             block_tables=meta((3, 4), torch.int32), ctx_lens=meta((3,), torch.int32), cu_q_lens=None,
             out=meta((3, 8, 128), torch.float32), out_dtype=torch.float32)
    a.update(o)
    return a


def test_binding_accepts_well_formed_decode_arguments():
    R.check_decode_args(**decode_args())
    import torch
    R.check_decode_args(**decode_args(out=meta((3, 8, 128), torch.bfloat16), out_dtype=torch.bfloat16))
    R.check_decode_args(**decode_args(sys_len=0, sys_k=meta((16,), torch.bfloat16), sys_v=meta((16,), torch.bfloat16)))
    R.check_decode_args(**decode_args(cu_q_lens=meta((4,), torch.int32)))


@pytest.mark.parametrize("bad,match", [
    (dict(out="bf16"), "out dtype"),                       # bf16 buffer for a float32 output
    (dict(out="short"), "shape"),
    (dict(sys_len=49), "sys_k must be"),                   # longer than the cache's 3 tiles
    (dict(sys_k="f32"), "sys_k dtype"),
    (dict(ctx_v_pages="f32"), "ctx_v_pages dtype"),
    (dict(ctx_v_pages="shape"), "ctx_v_pages must be"),
    (dict(block_tables="i64"), "block_tables"),
    (dict(ctx_lens="short"), "ctx_lens"),
    (dict(cu_q_lens="short"), "cu_q_lens"),
    (dict(q="rows"), "one query token"),
])
def test_binding_refuses_inconsistent_decode_arguments(bad, match):
    """The C library cannot see extents: the binding refuses what would be read or written
    out of bounds (a bf16 out with a float32 out_dtype, a sys_len past the cache, ...)."""
    import torch
    subst = {"bf16": meta((3, 8, 128), torch.bfloat16), "short": None, "f32": None, "shape": None,
             "i64": meta((3, 4), torch.int64), "rows": meta((4, 8, 128), torch.bfloat16)}
    kw = {}
    for k, v in bad.items():
        if k == "out" and v == "short":
            kw[k] = meta((3, 8, 64), torch.float32)
        elif k == "sys_k" and v == "f32":
            kw[k] = meta((2, 3, 32, 16, 4), torch.float32)
        elif k == "ctx_v_pages" and v == "f32":
            kw[k] = meta((10, 2, 128, 16), torch.float32)
        elif k == "ctx_v_pages" and v == "shape":
            kw[k] = meta((10, 2, 16, 128), torch.bfloat16)
        elif k == "ctx_lens":
            kw[k] = meta((2,), torch.int32)
        elif k == "cu_q_lens":
            kw[k] = meta((3,), torch.int32)
        elif k == "sys_len":
            kw[k] = v
        else:
            kw[k] = subst[v]
    with pytest.raises(ValueError, match=match):
        R.check_decode_args(**decode_args(**kw))


def test_validate_accepts_generated_workloads_and_rejects_bad_data(lib):
    w = W.generate(W.config_spec(5).replace(batch=4, sys_len=50, ctx_lo=20, ctx_hi=80))
    spec = w.spec
    d = R.relay_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, 16,
                     w.max_blocks_per_seq, w.num_blocks, w.total_q, int(w.q_lens.max()),
                     w.max_ctx_len, spec.scale, 1, 0)
    R.relay_validate(d, w.block_tables, w.ctx_lens, w.cu_q_lens, spec.sys_len)
    bt = w.block_tables.copy(); bt[1, 0] = w.num_blocks
    with pytest.raises(R.RelayError, match="block_tables"):
        R.relay_validate(d, bt, w.ctx_lens, w.cu_q_lens, spec.sys_len)
    cl = w.ctx_lens.copy(); cl[2] = 0
    with pytest.raises(R.RelayError, match="ctx_len"):
        R.relay_validate(d, w.block_tables, cl, w.cu_q_lens, spec.sys_len)
    cu = w.cu_q_lens.copy(); cu[-1] += 1
    with pytest.raises(R.RelayError, match="total_q"):
        R.relay_validate(d, w.block_tables, w.ctx_lens, cu, spec.sys_len)
    cu = w.cu_q_lens.copy(); cu[1] = cu[0]
    with pytest.raises(R.RelayError, match="n_b"):
        R.relay_validate(d, w.block_tables, w.ctx_lens, cu, spec.sys_len)


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        R.relay_fuse(q.float(), q[..., 0].float(), q.float(), q[..., 0].float())


def test_prefill_entry_rejects_what_it_does_not_run(lib):
    """relay_prefill_attn runs only on the matrix-core system kernel; everything else
    is refused with an error code before any device work (fake pointers here)."""
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)

    def call(d, sys_len=300, out_dtype=0, n=1 << 30):
        return lib.relay_prefill_attn(ctypes.byref(d), p, p, p, sys_len, p, out_dtype, None, ws, n, None)

    big = dict(batch=1, total_q=300, max_q_len=300, max_ctx_len=300, max_blocks_per_seq=19, num_blocks=1)
    assert call(base_dims(**big, in_dtype=0)) == -2                        # fp32: not on matrix cores
    assert call(base_dims(**big, head_dim=64)) == -2                        # head_dim 64
    assert call(base_dims(**dict(big, total_q=16, max_q_len=16))) == -2     # 16 x 4 = 64 rows per KV head
    assert call(base_dims(**big, scale=-0.1)) == -1                         # masked scores need scale > 0
    assert call(base_dims(**big), sys_len=0) == -1
    assert call(base_dims(**big), out_dtype=5) == -2
    d = base_dims(**big)
    need = lib.relay_prefill_workspace_size(ctypes.byref(d), 300)
    assert need > 0
    assert call(d, n=need - 1) == -3


@pytest.mark.parametrize("L,Hq,Hkv", [(37, 8, 2), (2048, 32, 32), (8192, 32, 8)])
def test_prefill_dims_pass_the_checks(lib, L, Hq, Hkv):
    """The binding's dims for relay_prefill_attn are valid and get a workspace."""
    import torch
    q = torch.empty((L, Hq, 128), dtype=torch.bfloat16)
    sk = torch.empty((Hkv, L, 128), dtype=torch.bfloat16)
    d = R.prefill_dims(q, sk, 128 ** -0.5)
    assert lib.relay_prefill_workspace_size(ctypes.byref(d), L) > 0, lib.relay_last_error()
