"""GPU: position embedding with context positions offset by the system length, and the
append of new tokens' K/V to the pages, against the oracle (oracle/rope.py); then the
relay decode on the embedded cache against exact attention over the rotated
[system; context].  Stored values: bf16 within one unit in the last place of the
oracle's rounded value, or 2e-6 where the rotation cancels to near zero (most are
bit-identical), fp32 within 2e-6 relative; the decode
output with the parity tolerances of test_parity_gpu."""
import numpy as np
import pytest
import torch

from oracle import Problem, rope
from shared_prompt_kv_amd import relay as R
import workloads as W
from tests.test_parity_gpu import check, say

pytestmark = pytest.mark.gpu

SPECS = [
    W.config_spec(5).replace(batch=4, sys_len=100, ctx_lo=20, ctx_hi=90),
    W.config_spec(2).replace(batch=5, sys_len=333, ctx_lo=16, ctx_hi=100),
    W.config_spec(4).replace(batch=6, sys_len=64, ctx_median=40, ctx_cap=120),
    W.config_spec(1).replace(sys_len=40),
]


def values(spec, a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if spec.dtype == "bf16" else np.asarray(a, np.float64)


def assert_stored_close(spec, got, want, what):
    g, e = values(spec, got), values(spec, want)
    if spec.dtype == "bf16":
        # one bf16 unit in the last place, plus the fp32 arithmetic and table rounding
        # (about 2^-22 of the operands) where the rotation cancels to near zero
        ulp = np.abs(e) * 2.0 ** -7 + 2e-6
        assert np.all(np.abs(g - e) <= ulp), f"{what}: more than one bf16 ulp"
        assert np.mean(g == e) > 0.99, f"{what}: too few bit-identical values"
    else:
        np.testing.assert_allclose(g, e, rtol=2e-6, atol=1e-7, err_msg=what)


def gather_tokens(w, positions_of):
    """Raw K and V [T, H_kv, d] (storage dtype) of the listed (request, position) pairs."""
    ks, vs = [], []
    ck = w.ctx_k_keys()
    for b, j in positions_of:
        p = int(w.block_tables[b, j // 16])
        ks.append(ck[p, :, j % 16, :])
        vs.append(w.ctx_v_pages[p, :, :, j % 16])
    return np.stack(ks), np.stack(vs)


def upload(spec, a):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if spec.dtype == "bf16" else torch.from_numpy(a)
    return t.to("cuda")


def test_table_matches_fp64_angles():
    say("[parity] rope table")
    for d in (64, 128):
        tab = R.relay_rope_table(70000, d).cpu().numpy().astype(np.float64)
        a = rope.angles(np.arange(70000), d)
        np.testing.assert_allclose(tab[:, : d // 2], np.cos(a), rtol=0, atol=1.2e-7)
        np.testing.assert_allclose(tab[:, d // 2:], np.sin(a), rtol=0, atol=1.2e-7)


@pytest.mark.parametrize("spec", SPECS, ids=[f"{s.name}-B{s.batch}-L{s.sys_len}" for s in SPECS])
def test_append_then_relay_decode(spec):
    say(f"[parity] rope + append + decode {spec}")
    w = W.generate(spec)                 # raw (pre-embedding) values
    wr = rope.rotated_workload(w)        # the oracle's embedded workload
    L, B = spec.sys_len, spec.batch
    t = R.to_device(w, "cuda")
    tab = R.relay_rope_table(L + int(w.ctx_lens.max()), spec.head_dim)
    # offline prefill of the system keys
    R.relay_rope_system(t["sys_k"], L, tab)
    # each request's earlier tokens, appended as one multi-token step (positions 0 .. c_b - 1)
    hist = [(b, j) for b in range(B) for j in range(int(w.ctx_lens[b]))]
    k_all, v_all = gather_tokens(w, hist)
    cu_all = np.concatenate([[0], np.cumsum(w.ctx_lens)]).astype(np.int32)
    q_dummy = torch.zeros((len(hist), spec.num_q_heads, spec.head_dim), dtype=t["q"].dtype, device="cuda")
    cu_all_t = torch.from_numpy(cu_all).to("cuda")
    dims_all = R.make_dims(q_dummy, t["ctx_k_pages"], t["block_tables"], scale=spec.scale,
                           max_ctx_len=t["max_ctx_len"], max_q_len=int(w.ctx_lens.max()))
    R.relay_rope_append(dims_all, L, q_dummy, upload(spec, k_all), upload(spec, v_all), tab, t["block_tables"],
                        t["ctx_lens"], cu_all_t, t["ctx_k_pages"], t["ctx_v_pages"])
    # the decode step's new tokens: q embedded, their K/V (re)appended
    new = [(b, int(w.ctx_lens[b]) - int(w.q_lens[b]) + i) for b in range(B) for i in range(int(w.q_lens[b]))]
    k_new, v_new = gather_tokens(w, new)
    dims = R.dims_of(t)
    q_rot = R.relay_rope_append(dims, L, t["q"], upload(spec, k_new), upload(spec, v_new), tab, t["block_tables"],
                                t["ctx_lens"], t["cu_q_lens"], t["ctx_k_pages"], t["ctx_v_pages"])
    t2 = dict(t, q=q_rot)
    out = R.decode_workload(t2)
    torch.cuda.synchronize()

    def host(x):
        x = x.cpu()
        return x.view(torch.int16).numpy().view(np.uint16) if spec.dtype == "bf16" else x.numpy()

    assert_stored_close(spec, host(q_rot), wr.q, "q")
    if L:
        assert_stored_close(spec, host(t["sys_k"]).reshape(wr.sys_k.shape), wr.sys_k, "system keys")
    ck = W.k_untile(host(t["ctx_k_pages"]))                  # key-major [page, H_kv, slot, d]
    live = np.zeros(ck.shape[:1] + ck.shape[2:3], bool)       # [page, slot]
    for b, j in hist:
        live[int(w.block_tables[b, j // 16]), j % 16] = True
    want = W.k_untile(wr.ctx_k_pages)
    assert_stored_close(spec, ck[live.nonzero()[0], :, live.nonzero()[1]],
                        want[live.nonzero()[0], :, live.nonzero()[1]], "context keys")
    assert np.array_equal(ck[~live.any(1)], w.ctx_k_keys()[~live.any(1)]), "pages nobody owns were written"
    assert np.array_equal(host(t["ctx_v_pages"]), w.ctx_v_pages), "values must be stored unchanged"
    ref, _ = Problem(wr).attention()
    check(out.cpu().numpy(), ref, spec.dtype, "decode on the embedded cache")
