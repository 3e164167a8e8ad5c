"""Pins for the fp64 oracle, against things other than itself.

* brute force: pure-Python loops written from the definition of causal attention,
  over the generator's dense (pre-paging) K/V, on tiny inputs;
* a library routine: torch's scaled_dot_product_attention and logsumexp in fp64 on
  the CPU over the dense gathered [K_s; K_c] with an explicit causal mask;
* closed forms: q = 0, one key, two keys, constant V, V shifted by a constant;
* the relay identity (RelayAttention abstract: exact reformulation; atyun.com
  article, section "RelayAttention": the output is a weighted average of the two
  intermediate outputs): weights non-negative and summing to 1, split == unsplit, split-point
  invariance, k-way == 2-way, sys_len = 0 and empty-context reductions;
* paging invariances: page relabelling, GQA->MHA expansion, batch permutation,
  poison never reaching an output.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_spec(idx, *, B=2, Hq=2, Hkv=1, d=4, Ls=3, lo=1, hi=9, qlo=1, qhi=1, dtype=W.F32,
              poison="sentinel", kscale=False):
    return W.WorkloadSpec(f"tiny{idx}", 100 + idx, 0, dtype, B, Hq, Hkv, d, Ls, "uniform", lo, hi,
                          q_lo=qlo, q_hi=qhi, poison=poison, k_channel_scale=kscale)


# ----------------------------------------------------------------------------------------
# brute force: pure Python, from the definition


def dense_rows(w):
    """Yield (t, h, keys, values) with the visible [system; context] K/V rows as float lists."""
    s = w.spec
    g = s.num_q_heads // s.num_kv_heads
    q = w.values(w.q).astype(np.float64)
    sk = w.values(w.sys_k_keys()).astype(np.float64)
    sv = w.values(w.sys_v_dense).astype(np.float64)
    for b in range(s.batch):
        n_b = int(w.q_lens[b])
        kc = w.values(w.ctx_k_dense[b]).astype(np.float64)
        vc = w.values(w.ctx_v_dense[b]).astype(np.float64)
        for tl in range(n_b):
            t = int(w.cu_q_lens[b]) + tl
            p = int(w.ctx_lens[b]) - n_b + tl
            for h in range(s.num_q_heads):
                hk = h // g
                keys = [list(sk[hk, j]) for j in range(s.sys_len)] + [list(kc[j, hk]) for j in range(p + 1)]
                vals = [list(sv[hk, j]) for j in range(s.sys_len)] + [list(vc[j, hk]) for j in range(p + 1)]
                yield t, h, list(q[t, h]), keys, vals


def brute_attention(qrow, keys, vals, scale):
    if not keys:
        return [0.0] * len(qrow), -math.inf
    scores = [scale * math.fsum(a * b for a, b in zip(qrow, k)) for k in keys]
    m = max(scores)
    e = [math.exp(x - m) for x in scores]
    z = math.fsum(e)
    out = [math.fsum(e[j] * vals[j][c] for j in range(len(keys))) / z for c in range(len(qrow))]
    return out, m + math.log(z)


TINY = [
    dict(B=1, Hq=1, Hkv=1, d=1, Ls=0, lo=1, hi=1),
    dict(B=2, Hq=2, Hkv=1, d=2, Ls=1, lo=1, hi=5),
    dict(B=3, Hq=4, Hkv=2, d=4, Ls=2, lo=1, hi=33),
    dict(B=2, Hq=4, Hkv=1, d=4, Ls=17, lo=3, hi=20, qlo=1, qhi=3),
    dict(B=3, Hq=2, Hkv=2, d=64, Ls=3, lo=16, hi=33, qlo=1, qhi=4),
    dict(B=2, Hq=4, Hkv=4, d=2, Ls=0, lo=1, hi=17, qlo=1, qhi=2),
]


@pytest.mark.parametrize("i,kw", list(enumerate(TINY)))
def test_oracle_matches_bruteforce(oracle_lib, i, kw):
    w = W.generate(tiny_spec(i, **kw), keep_dense=True)
    P = oracle_lib.Problem(w)
    out, lse = P.attention()
    o_s, l_s = P.system_part()
    o_c, l_c = P.context_part()
    Ls = w.spec.sys_len
    for t, h, qrow, keys, vals in dense_rows(w):
        ref, ref_lse = brute_attention(qrow, keys, vals, w.spec.scale)
        np.testing.assert_allclose(out[t, h], ref, rtol=0, atol=1e-13)
        assert abs(lse[t, h] - ref_lse) <= 1e-13
        rs, rls = brute_attention(qrow, keys[:Ls], vals[:Ls], w.spec.scale)
        rc, rlc = brute_attention(qrow, keys[Ls:], vals[Ls:], w.spec.scale)
        np.testing.assert_allclose(o_s[t, h], rs, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o_c[t, h], rc, rtol=0, atol=1e-13)
        assert (l_s[t, h] == rls) if math.isinf(rls) else abs(l_s[t, h] - rls) <= 1e-13
        assert abs(l_c[t, h] - rlc) <= 1e-13


# ----------------------------------------------------------------------------------------
# library routine: torch SDPA / logsumexp in fp64 on the CPU


def sdpa_reference(w):
    s = w.spec
    g = s.group
    q = torch.from_numpy(w.values(w.q).astype(np.float64))
    sk = torch.from_numpy(w.values(w.sys_k_keys()).astype(np.float64))   # [Hkv, Ls, d]
    sv = torch.from_numpy(w.values(w.sys_v_dense).astype(np.float64))    # [Hkv, Ls, d]
    outs, lses = [], []
    for b in range(s.batch):
        n_b = int(w.q_lens[b])
        c = int(w.ctx_lens[b])
        kc = torch.from_numpy(w.values(w.ctx_k_dense[b]).astype(np.float64)).transpose(0, 1)
        vc = torch.from_numpy(w.values(w.ctx_v_dense[b]).astype(np.float64)).transpose(0, 1)
        K = torch.cat([sk, kc], 1).repeat_interleave(g, 0).contiguous()  # [Hq, Ls+c, d]
        V = torch.cat([sv, vc], 1).repeat_interleave(g, 0).contiguous()
        t0 = int(w.cu_q_lens[b])
        Q = q[t0:t0 + n_b].transpose(0, 1).contiguous()                    # [Hq, n_b, d]
        j = torch.arange(s.sys_len + c)
        pos = c - n_b + torch.arange(n_b)
        mask = j[None, :] <= (s.sys_len + pos)[:, None]                    # [n_b, Ls+c]
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=mask, scale=s.scale)
        scores = torch.matmul(Q, K.transpose(1, 2).contiguous()) * s.scale
        scores = scores.masked_fill(~mask, -math.inf)
        lses.append(torch.logsumexp(scores, -1).transpose(0, 1))
        outs.append(o.transpose(0, 1))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


@pytest.mark.parametrize("spec", [
    W.config_spec(1),
    W.config_spec(2).replace(batch=3, sys_len=300, ctx_lo=16, ctx_hi=80),
    W.config_spec(4).replace(batch=5, sys_len=200, ctx_median=40, ctx_cap=100),
    W.config_spec(5).replace(batch=4, sys_len=130, ctx_lo=20, ctx_hi=70),
], ids=["c1", "c2-small", "c4-small", "c5-small"])
def test_oracle_matches_torch_sdpa(oracle_lib, spec):
    w = W.generate(spec, keep_dense=True)
    out, lse = oracle_lib.Problem(w).attention()
    ref, ref_lse = sdpa_reference(w)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------------
# closed forms


def test_zero_query_gives_mean_of_visible_values(oracle_lib):
    w = W.generate(tiny_spec(20, B=3, Hq=2, Hkv=1, d=8, Ls=5, lo=1, hi=12, qlo=1, qhi=2), keep_dense=True)
    w.q[...] = 0.0
    out, lse = oracle_lib.Problem(w).attention()
    for t, h, _, keys, vals in dense_rows(w):
        np.testing.assert_allclose(out[t, h], np.mean(np.array(vals), 0), rtol=0, atol=1e-14)
        assert abs(lse[t, h] - math.log(len(keys))) <= 1e-14


def test_single_key(oracle_lib):
    # No system prompt, a context of one token: out = v, LSE = scale * q.k.
    w = W.generate(tiny_spec(21, B=2, Hq=2, Hkv=2, d=16, Ls=0, lo=1, hi=1), keep_dense=True)
    out, lse = oracle_lib.Problem(w).attention()
    for b in range(2):
        for h in range(2):
            q = w.q[b, h].astype(np.float64)
            k = w.ctx_k_dense[b][0, h].astype(np.float64)
            v = w.ctx_v_dense[b][0, h].astype(np.float64)
            np.testing.assert_array_equal(out[b, h], v)
            assert abs(lse[b, h] - w.spec.scale * math.fsum(q * k)) <= 1e-15


def _hand_workload(q, sys_kv, ctx_kv, scale_dim):
    """One request, one head, fp32; explicit keys/values."""
    d = len(q)
    Ls = len(sys_kv)
    c = len(ctx_kv)
    spec = tiny_spec(30, B=1, Hq=1, Hkv=1, d=d, Ls=Ls, lo=c, hi=c)
    w = W.generate(spec, keep_dense=True)
    w.q[0, 0, :] = q
    G = W.k_chunk(spec.dtype, d)
    for j, (k, v) in enumerate(sys_kv):
        w.sys_k[0, j // 16, :, W.KEY_SLOTS[j % 16], :] = np.reshape(k, (d // G, G))
        w.sys_v[0, j // 16, :, j % 16] = v
    for j, (k, v) in enumerate(ctx_kv):
        blk = w.block_tables[0, j // 16]
        w.ctx_k_pages[blk, 0, :, W.KEY_SLOTS[j % 16], :] = np.reshape(k, (d // G, G))
        w.ctx_v_pages[blk, 0, :, j % 16] = v
    return w


def test_golden_closed_form_cases(oracle_lib):
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        w = _hand_workload(case["q"], case["system"], case["context"], None)
        P = oracle_lib.Problem(w, scale=case["scale"])
        out, lse = P.attention()
        np.testing.assert_allclose(out[0, 0], case["out"], rtol=0, atol=1e-14, err_msg=case["name"])
        assert abs(lse[0, 0] - case["lse"]) <= 1e-14, case["name"]
        if "alpha_s" in case:
            o_s, l_s = P.system_part()
            o_c, l_c = P.context_part()
            _, _, alpha = oracle_lib.relay_fuse(o_s, l_s, o_c, l_c)
            assert abs(alpha[0, 0, 0] - case["alpha_s"]) <= 1e-15, case["name"]


def test_constant_values_and_shift(oracle_lib):
    w = W.generate(tiny_spec(22, B=3, Hq=4, Hkv=2, d=8, Ls=9, lo=2, hi=30, qlo=1, qhi=3))
    # values on a 2^-10 grid so that V + 0.75 is exact in float32
    for arr in (w.sys_v, w.ctx_v_pages):
        arr[...] = np.round(arr * 1024) / 1024
    out0, lse0 = oracle_lib.Problem(w).attention()
    # V -> V + 0.75: every output shifts by 0.75 (the weights sum to 1), LSE unchanged
    for arr in (w.sys_v, w.ctx_v_pages):
        arr += np.float32(0.75)
    out1, lse1 = oracle_lib.Problem(w).attention()
    np.testing.assert_allclose(out1 - out0, 0.75, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(lse1, lse0)
    # V == const: out == const
    w.sys_v[...] = np.float32(-2.5)
    w.ctx_v_pages[...] = np.float32(-2.5)
    out2, _ = oracle_lib.Problem(w).attention()
    np.testing.assert_allclose(out2, -2.5, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------------------
# relay identity


SPLIT_SPECS = [
    W.config_spec(1),
    W.config_spec(2).replace(batch=4, sys_len=257, ctx_lo=16, ctx_hi=100),
    W.config_spec(3, 0).replace(batch=3, num_q_heads=4, num_kv_heads=4),
    W.config_spec(4).replace(batch=6, sys_len=300, ctx_median=50, ctx_cap=120),
    W.config_spec(5).replace(batch=4, sys_len=500, ctx_lo=64, ctx_hi=200),
]


@pytest.mark.parametrize("spec", SPLIT_SPECS, ids=lambda s: s.name)
def test_relay_split_equals_unsplit(oracle_lib, spec):
    w = W.generate(spec)
    P = oracle_lib.Problem(w)
    out, lse = P.attention()
    o_s, l_s = P.system_part()
    o_c, l_c = P.context_part()
    fused, fl, alpha = oracle_lib.relay_fuse(o_s, l_s, o_c, l_c)
    assert np.all(alpha >= 0)
    np.testing.assert_allclose(alpha.sum(-1), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(fused, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fl, lse, rtol=0, atol=1e-12)


def test_relay_split_equals_unsplit_long_system(oracle_lib):
    """Configuration-5 lengths (65536 system keys, up to 4096 context keys) on sampled rows."""
    spec = W.config_spec(5).replace(batch=3)
    w = W.generate(spec)
    P = oracle_lib.Problem(w)
    Tq = w.total_q
    rows = np.unique(np.random.default_rng(5).integers(0, Tq * spec.num_q_heads, 6))
    out, lse = P.attention(rows)
    out2, lse2 = P.relay(rows)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def test_split_point_invariance_and_kway_merge(oracle_lib):
    w = W.generate(tiny_spec(23, B=3, Hq=4, Hkv=2, d=8, Ls=40, lo=5, hi=60, qlo=1, qhi=4))
    P = oracle_lib.Problem(w)
    out, lse = P.attention()
    big = 1 << 30
    for x in (0, 1, 7, 40, 41, 63, 99):
        a, la = P.attention_range(0, x)
        b, lb = P.attention_range(x, big)
        f, fl, _ = oracle_lib.relay_fuse(a, la, b, lb)
        np.testing.assert_allclose(f, out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(fl, lse, rtol=0, atol=1e-12)
    cuts = [0, 3, 17, 40, 52, big]
    parts = [P.attention_range(cuts[i], cuts[i + 1]) for i in range(len(cuts) - 1)]
    m, ml = oracle_lib.merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(m, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-12)


def test_zero_system_length_reduces_to_context_attention(oracle_lib):
    w = W.generate(tiny_spec(24, B=3, Hq=4, Hkv=2, d=8, Ls=0, lo=1, hi=40, qlo=1, qhi=3))
    P = oracle_lib.Problem(w)
    out, lse = P.attention()
    o_s, l_s = P.system_part()
    o_c, l_c = P.context_part()
    assert np.all(np.isneginf(l_s)) and np.all(o_s == 0)
    np.testing.assert_array_equal(o_c, out)
    fused, fl, alpha = oracle_lib.relay_fuse(o_s, l_s, o_c, l_c)
    assert np.all(alpha[..., 0] == 0) and np.all(alpha[..., 1] == 1)
    np.testing.assert_array_equal(fused, out)


def test_empty_context_reduces_to_system_attention(oracle_lib):
    # The relay fusion with an empty context part returns the system part unchanged.
    w = W.generate(tiny_spec(25, B=2, Hq=2, Hkv=1, d=8, Ls=20, lo=3, hi=9))
    P = oracle_lib.Problem(w)
    o_s, l_s = P.system_part()
    empty = np.zeros_like(o_s)
    fused, fl, alpha = oracle_lib.relay_fuse(o_s, l_s, empty, np.full_like(l_s, -np.inf))
    np.testing.assert_array_equal(fused, o_s)
    np.testing.assert_array_equal(fl, l_s)
    np.testing.assert_array_equal(alpha[..., 0], 1.0)


# ----------------------------------------------------------------------------------------
# paging invariances


def test_page_relabelling_is_bitwise_invariant(oracle_lib):
    w = W.generate(W.config_spec(5).replace(batch=3, sys_len=70, ctx_lo=20, ctx_hi=90))
    out, lse = oracle_lib.Problem(w).attention()
    w2 = W.relabel_pages(w, 3)
    assert not np.array_equal(w2.block_tables, w.block_tables)
    out2, lse2 = oracle_lib.Problem(w2).attention()
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_gqa_equals_expanded_mha(oracle_lib):
    spec = W.config_spec(4).replace(batch=3, sys_len=33, ctx_median=20, ctx_cap=50)
    w = W.generate(spec)
    out, lse = oracle_lib.Problem(w).attention()
    g = spec.group
    import dataclasses
    w2 = dataclasses.replace(
        w, spec=spec.replace(num_kv_heads=spec.num_q_heads),
        sys_k=np.ascontiguousarray(np.repeat(w.sys_k, g, 0)),
        sys_v=np.ascontiguousarray(np.repeat(w.sys_v, g, 0)),
        ctx_k_pages=np.ascontiguousarray(np.repeat(w.ctx_k_pages, g, 1)),
        ctx_v_pages=np.ascontiguousarray(np.repeat(w.ctx_v_pages, g, 1)))
    out2, lse2 = oracle_lib.Problem(w2).attention()
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_batch_permutation_permutes_output(oracle_lib):
    import dataclasses
    w = W.generate(tiny_spec(26, B=4, Hq=2, Hkv=1, d=8, Ls=10, lo=1, hi=40, qlo=1, qhi=3))
    out, _ = oracle_lib.Problem(w).attention()
    perm = np.array([2, 0, 3, 1])
    qs = [w.q[w.cu_q_lens[b]:w.cu_q_lens[b + 1]] for b in range(4)]
    os_ = [out[w.cu_q_lens[b]:w.cu_q_lens[b + 1]] for b in range(4)]
    ql = w.q_lens[perm]
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    w2 = dataclasses.replace(w, q=np.ascontiguousarray(np.concatenate([qs[b] for b in perm])),
                             block_tables=np.ascontiguousarray(w.block_tables[perm]),
                             ctx_lens=np.ascontiguousarray(w.ctx_lens[perm]),
                             q_lens=ql, cu_q_lens=cu)
    out2, _ = oracle_lib.Problem(w2).attention()
    np.testing.assert_array_equal(out2, np.concatenate([os_[b] for b in perm]))


def test_poison_never_reaches_output(oracle_lib):
    spec = tiny_spec(27, B=3, Hq=4, Hkv=2, d=16, Ls=21, lo=1, hi=45, qlo=1, qhi=3)
    a, la = oracle_lib.Problem(W.generate(spec)).attention()
    b, lb = oracle_lib.Problem(W.generate(spec.replace(poison="nan"))).attention()
    assert np.all(np.isfinite(b))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
