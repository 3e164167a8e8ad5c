"""The no-relay baseline's inputs (prefix-shared pages): host-side layout checks.

Gathering each request's keys and values through the baseline's block tables must
give exactly [system; own context] in order, with the system pages stored once."""
import numpy as np
import pytest
import torch

from shared_prompt_kv_amd import baseline, relay as R
import workloads as W

SPECS = [
    W.config_spec(2).replace(batch=3, sys_len=48, ctx_lo=5, ctx_hi=40),
    W.config_spec(5).replace(batch=3, sys_len=32, ctx_lo=20, ctx_hi=70),
    W.config_spec(4).replace(batch=4, sys_len=16, ctx_median=30, ctx_cap=64),
    W.config_spec(1).replace(sys_len=0),
]


def untile(k):
    """Key tiles [..., d/G, 16, G] -> key-major [..., 16, d]."""
    return k.transpose(-3, -2).reshape(*k.shape[:-3], k.shape[-2], -1)


def gather(pool_k, pool_v, bt, n):
    """K [H_kv, n, d] and V [H_kv, n, d] of positions 0..n-1 through one block-table row."""
    pool_k = untile(pool_k)
    ks, vs = [], []
    for j in range(n):
        p = int(bt[j // 16])
        ks.append(pool_k[p, :, j % 16, :])
        vs.append(pool_v[p, :, :, j % 16])
    return torch.stack(ks, 1), torch.stack(vs, 1)


@pytest.mark.parametrize("spec", SPECS, ids=[s.name for s in SPECS])
def test_prefix_shared_pages_reproduce_system_then_context(spec):
    w = W.generate(spec)
    t = R.to_device(w, "cpu")
    b = baseline.prefix_shared(t)
    L = spec.sys_len
    assert b["sys_len"] == 0 and b["max_ctx_len"] == t["max_ctx_len"] + L
    assert b["ctx_k_pages"].shape[0] == t["ctx_k_pages"].shape[0] + L // 16   # system pages once
    H_kv, d = spec.num_kv_heads, spec.head_dim
    sys_v = t["sys_v"].reshape(H_kv, -1, d, 16).permute(0, 1, 3, 2).reshape(H_kv, -1, d)[:, :L] if L else None
    for r in range(spec.batch):
        c = int(t["ctx_lens"][r])
        assert int(b["ctx_lens"][r]) == c + L
        kb, vb = gather(b["ctx_k_pages"], b["ctx_v_pages"], b["block_tables"][r], c + L)
        kc, vc = gather(t["ctx_k_pages"], t["ctx_v_pages"], t["block_tables"][r], c)
        if L:
            kc = torch.cat([untile(t["sys_k"]).reshape(H_kv, -1, d)[:, :L], kc], 1)
            vc = torch.cat([sys_v, vc], 1)
        assert torch.equal(kb, kc) and torch.equal(vb, vc)
        # every request's table starts with the same shared page ids
        assert torch.equal(b["block_tables"][r, :L // 16], torch.arange(L // 16, dtype=torch.int32))


def test_unaligned_system_length_is_rejected():
    w = W.generate(W.config_spec(2).replace(batch=2, sys_len=20, ctx_lo=5, ctx_hi=9))
    with pytest.raises(ValueError):
        baseline.prefix_shared(R.to_device(w, "cpu"))
