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
from shared_prompt_kv_amd import workloads as W

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


def test_library_is_gfx950_only(lib):
    # the device code objects are embedded for gfx950 alone
    blob = open(R.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in blob


def test_abi_version_and_strerror(lib):
    assert R.relay_abi_version() == 2
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


def test_workspace_covers_the_plan(lib):
    d = base_dims()
    plan = R.relay_get_plan(d, 1000)
    rows = 4 * 8
    need = R.relay_workspace_size(d, 1000)
    parts = (plan["sys_chunks"] + plan["ctx_max_splits"]) * rows * (128 + 1) * 4
    assert need >= parts and need <= parts + 4 * 256
    assert plan["sys_chunks"] * plan["sys_chunk_len"] >= 1000
    assert plan["sys_chunk_len"] % 32 == 0 and plan["ctx_split_len"] % 32 == 0
    assert plan["ctx_max_splits"] * plan["ctx_split_len"] >= 128
    assert R.relay_get_plan(d, 0)["sys_chunks"] == 0


@pytest.mark.parametrize("cfg,sweep", [(1, 0), (2, 0), (3, 0), (3, 5), (4, 0), (5, 0)])
def test_plan_for_each_config(lib, cfg, sweep):
    spec = W.config_spec(cfg, sweep)
    s = W.expected_sizes(spec)
    d = R.relay_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, 16,
                     -(-s["max_ctx"] // 16), 1000, s["total_q"], int(s["q_lens"].max()), s["max_ctx"],
                     spec.scale, 1 if spec.dtype == "bf16" else 0, 0)
    plan = R.relay_get_plan(d, spec.sys_len)
    M = s["total_q"] * spec.group
    if M <= 64:   # single-wave system units, launched together with the context units
        assert plan["sys_chunks"] * plan["sys_chunk_len"] >= spec.sys_len
        assert (plan["sys_chunks"] - 1) * plan["sys_chunk_len"] < spec.sys_len
        assert plan["sys_mode"] == 1 and plan["launches"] == 2
        groups = spec.num_kv_heads * plan["sys_chunks"]
        # units of two 16-row tiles when M <= 32 and there are >= 384 (head, chunk) groups
        rt = 2 if 16 < M <= 32 and groups >= 384 else 1
        assert plan["sys_row_blocks"] == -(-M // (16 * rt))
        assert plan["sys_wgs"] == 8 * plan["sys_row_blocks"] * (-(-groups // 8))
    else:         # matrix-core system kernel: (row block, run of 64-key steps) workgroups
        assert plan["sys_mode"] == 2 and plan["launches"] == 3
        assert plan["sys_row_blocks"] * 128 >= M
        steps = spec.num_kv_heads * -(-spec.sys_len // 64)
        parts = min(max(512 // plan["sys_row_blocks"], 1), steps)
        assert plan["sys_wgs"] == -(-plan["sys_row_blocks"] * parts // 8) * 8 <= max(512, plan["sys_wgs"])
        assert plan["sys_chunk_len"] == -(-steps // parts) * 64
        # slots: the most runs one head's steps fall into
        part_of = lambda x: ((x + 1) * parts + steps - 1) // steps - 1
        sph = steps // spec.num_kv_heads
        assert plan["sys_chunks"] == max(part_of(h * sph + sph - 1) - part_of(h * sph) + 1
                                         for h in range(spec.num_kv_heads))
    # context split: 512 keys while every context fits one, else 768
    assert plan["ctx_split_len"] == (768 if s["max_ctx"] > 512 else 512)
    assert plan["ctx_max_splits"] == -(-s["max_ctx"] // plan["ctx_split_len"])
    assert 0 < plan["ctx_wgs"] < 2**31 and 0 < plan["sys_wgs"] < 2**31


@pytest.mark.parametrize("env,rows", [({}, 2), ({"RELAY_SYS_ROW_TILES": "2"}, 1),
                                      ({"RELAY_SYS_ROW_TILES": "2", "RELAY_KEY_LANES": "8"}, 2),
                                      ({"RELAY_CTX_SPLIT": "256"}, 2)])
def test_plan_tuning_knobs(lib, monkeypatch, env, rows):
    """The environment knobs the plan reads: two-tile system units on request (never with
    eight key lanes), and the context split."""
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    spec = W.config_spec(2, 0)
    s = W.expected_sizes(spec)
    d = R.relay_dims(spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, 16,
                     -(-s["max_ctx"] // 16), 1000, s["total_q"], 1, s["max_ctx"], spec.scale, 1, 0)
    plan = R.relay_get_plan(d, spec.sys_len)
    assert plan["sys_row_blocks"] == rows          # M = 32 rows: two one-tile units or one two-tile unit
    assert plan["ctx_split_len"] == int(env.get("RELAY_CTX_SPLIT", 512))


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
    assert need >= lib.relay_workspace_size(ctypes.byref(d), 300) > 0
    assert call(d, n=need - 1) == -3


@pytest.mark.parametrize("L,Hq,Hkv", [(37, 8, 2), (2048, 32, 32), (8192, 32, 8)])
def test_prefill_dims_pass_the_checks(lib, L, Hq, Hkv):
    """The binding's dims for relay_prefill_attn are valid and get a workspace."""
    import torch
    q = torch.empty((L, Hq, 128), dtype=torch.bfloat16)
    sk = torch.empty((Hkv, L, 128), dtype=torch.bfloat16)
    d = R.prefill_dims(q, sk, 128 ** -0.5)
    assert lib.relay_prefill_workspace_size(ctypes.byref(d), L) > 0, lib.relay_last_error()
