"""The allocation-free decode entry point (relay_attn_decode_noalloc) against
relay_attn_decode on the same inputs, through the C ABI.

Both run the same plan and kernels; the allocation-free one keeps its partials in the
library's static per-device scratch instead of a caller workspace.  Two calls in a row
(the second one smaller, so it runs on the first call's leftovers), then a call on the
matrix-core system path; each output is held to the parity bar of its input dtype
(fp32: max abs 1e-5; bf16: max abs 2e-3 and relative L2 1e-2), and sampled rows to the
fp64 oracle.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from shared_prompt_kv_amd import relay as R
import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def within_bar(a, b, dtype, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape and np.all(np.isfinite(a)) and np.all(np.isfinite(b)), what
    err = float(np.abs(a - b).max())
    if dtype == "f32":
        assert err <= 1e-5, f"{what}: max abs {err:.3e}"
    else:
        rel = float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
        assert err <= 2e-3 and rel <= 1e-2, f"{what}: max abs {err:.3e}, rel L2 {rel:.3e}"
    return err


def noalloc(t, out):
    return R.relay_attn_decode_noalloc(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], t["ctx_k_pages"],
                                       t["ctx_v_pages"], t["block_tables"], t["ctx_lens"], t["cu_q_lens"], out,
                                       scale=t["scale"], max_ctx_len=t["max_ctx_len"],
                                       max_q_len=t["max_q_len"])


CASES = [
    ("llama2-7b shape, batch 32", W.config_spec(2)),
    ("smaller: batch 6, system 300", W.config_spec(2).replace(name="c2-small", batch=6, sys_len=300,
                                                              ctx_lo=16, ctx_hi=120)),
    ("gqa, matrix-core system step", W.config_spec(4).replace(name="c4-mid", batch=40, sys_len=1500,
                                                              ctx_median=200, ctx_cap=700)),
    ("fp32, tiny", W.config_spec(1)),
]


def test_noalloc_matches_the_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    R.load_library()
    rng = np.random.default_rng(11)
    for what, spec in CASES:
        say(f"[noalloc] {what}: {spec.name} batch {spec.batch} sys_len {spec.sys_len}")
        w = W.generate(spec)
        t = R.to_device(w, "cuda")
        dims = R.dims_of(t)
        assert R.relay_workspace_size(dims, t["sys_len"]) <= R.NOALLOC_SCRATCH_BYTES
        out_n = torch.full(t["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
        noalloc(t, out_n)
        torch.cuda.synchronize()
        ref = R.decode_workload(t).cpu().numpy()
        got = out_n.cpu().numpy()
        err = within_bar(got, ref, spec.dtype, what)
        # a few rows against the oracle as well (the two entry points could share a bug)
        rows = rng.choice(w.total_q * spec.num_q_heads, size=min(24, w.total_q * spec.num_q_heads), replace=False)
        o_ref, _ = oracle.Problem(w).attention(np.sort(rows))
        within_bar(got.reshape(-1, spec.head_dim)[np.sort(rows)], o_ref, spec.dtype, what + " (oracle rows)")
        say(f"[noalloc] {what}: max |noalloc - decode| = {err:.3e}")
        del t
        torch.cuda.empty_cache()


def test_noalloc_refuses_a_workspace_past_the_scratch():
    """Sizes whose workspace exceeds the static scratch are refused before any launch."""
    spec = W.config_spec(4)
    big = R.relay_dims(8192, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, 16, 128, 10000, 8192, 1, 2048,
                       spec.scale, 1, 0)
    assert R.relay_workspace_size(big, spec.sys_len) > R.NOALLOC_SCRATCH_BYTES
    rc = R.load_library().relay_attn_decode_noalloc(ctypes.byref(big), None, None, None, spec.sys_len, None,
                                                   None, None, None, None, None, None)
    assert rc == R.RELAY_ERR_WORKSPACE
