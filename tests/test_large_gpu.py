"""GPU: a system cache, and a context page pool, larger than 4 GiB per tensor (byte
offsets past 2^32), on the single-wave unit path (at most 64 stacked rows) and on the
matrix-core path.

The system K/V are drawn on the device (torch's seeded generator; 2^31+ values are too
many to draw on the host in a test).  The oracle checks sampled rows one by one: for a
(request, KV head) pair it gets that head's keys and values copied back and the
request's own context, and computes exact attention for the head's query rows in
fp64.  Head 7 of 8 lies partly past the 4 GiB boundary of both tensors.
"""
import numpy as np
import pytest
import torch

import oracle
from shared_prompt_kv_amd import relay as R
import workloads as W
from tests.test_parity_gpu import check, say

pytestmark = pytest.mark.gpu

H_KV, H_Q, D = 8, 32, 128
L_SYS = (1 << 21) + (1 << 18) + 37   # 2,359,333 keys: K is 8 * L * 256 B = 4.83 GB


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("batch", [4, 40])
def test_system_cache_past_4_gib(batch):
    spec = W.config_spec(5).replace(batch=batch, sys_len=0, ctx_lo=16, ctx_hi=64, q_lo=1, q_hi=1)
    say(f"[parity] system cache past 4 GiB: L_s={L_SYS} H_kv={H_KV} batch={batch}")
    w = W.generate(spec)   # queries and context only
    t = R.to_device(w)
    g = torch.Generator(device="cuda").manual_seed(11)
    ntile = -(-L_SYS // 16)
    sys_k = torch.randn(R.key_tile_shape((H_KV, ntile), D, torch.bfloat16), generator=g,
                        device="cuda").to(torch.bfloat16)   # key tiles (padding keys never read)
    sys_v = torch.randn((H_KV, ntile, D, 16), generator=g, device="cuda").to(torch.bfloat16)
    sys_v[:, -1, :, L_SYS % 16:] = 0   # the tail tile's padding keys
    assert sys_k.numel() * 2 > 2**32 and sys_v.numel() * 2 > 2**32
    t.update(sys_k=sys_k, sys_v=sys_v, sys_len=L_SYS)
    plan = R.relay_get_plan(R.dims_of(t), L_SYS)
    assert plan["sys_mode"] in ((1,) if batch * H_Q // H_KV <= 64 else (2, 4))
    out = R.decode_workload(t).cpu().numpy()
    torch.cuda.synchronize()

    g_ = H_Q // H_KV
    for b, hk in ((batch - 1, H_KV - 1), (0, 3)):
        say(f"  sample request {b} KV head {hk}")
        tok = int(w.cu_q_lens[b])
        rows = slice(hk * g_, (hk + 1) * g_)
        sub = W.Workload(spec.replace(batch=1, num_q_heads=g_, num_kv_heads=1, sys_len=L_SYS),
                         np.ascontiguousarray(w.q[tok:tok + 1, rows]), bits(sys_k[hk:hk + 1]), bits(sys_v[hk:hk + 1]),
                         np.ascontiguousarray(w.ctx_k_pages[:, hk:hk + 1]),
                         np.ascontiguousarray(w.ctx_v_pages[:, hk:hk + 1]),
                         np.ascontiguousarray(w.block_tables[b:b + 1]), w.ctx_lens[b:b + 1].copy(),
                         np.array([1], np.int32), np.array([0, 1], np.int32))
        ref, _ = oracle.Problem(sub).attention()
        check(out[tok:tok + 1, rows], ref, "bf16", f"request {b} head {hk}")


@pytest.mark.parametrize("batch", [4, 40])
def test_context_pages_past_4_gib(batch):
    """The same requests with their pages moved to the end of a page pool larger than
    4 GiB per tensor (block ids relabelled; the rest of the pool is random): every
    output against the oracle on the original workload (relabelling pages leaves
    attention unchanged)."""
    spec = W.config_spec(5).replace(batch=batch, sys_len=100, ctx_lo=16, ctx_hi=700, q_lo=1, q_hi=3)
    say(f"[parity] context pages past 4 GiB: batch={batch}")
    w = W.generate(spec)
    t = R.to_device(w)
    nb, hkv = t["ctx_k_pages"].shape[:2]
    d = t["ctx_v_pages"].shape[2]
    big = (2**32 // (hkv * 16 * d * 2)) + 4096   # pages: each tensor > 4 GiB
    g = torch.Generator(device="cuda").manual_seed(5)
    pool_k = torch.randn(R.key_tile_shape((big, hkv), d, torch.bfloat16), generator=g, device="cuda").to(torch.bfloat16)
    pool_v = torch.randn((big, hkv, d, 16), generator=g, device="cuda").to(torch.bfloat16)
    off = big - nb
    pool_k[off:] = t["ctx_k_pages"]
    pool_v[off:] = t["ctx_v_pages"]
    bt = t["block_tables"]
    t.update(ctx_k_pages=pool_k, ctx_v_pages=pool_v, block_tables=torch.where(bt >= 0, bt + off, bt).contiguous())
    assert pool_k.numel() * 2 > 2**32 and int(t["block_tables"].max()) * hkv * 16 * d * 2 > 2**32
    out = R.decode_workload(t).cpu().numpy()
    torch.cuda.synchronize()
    ref, _ = oracle.Problem(w).attention()
    check(out, ref, "bf16", "decode over relabelled pages")
