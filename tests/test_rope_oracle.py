"""Pins of the oracle's position embedding (oracle/rope.py) against facts that do not
come from its own formula: the complex-number form of a rotation, the identity at
position 0, norm preservation, the relative-position property, and the position
contract (context keys after the system prompt) against a brute-force attention over
the concatenated, rotated sequence."""
import numpy as np
import pytest

from oracle import rope, Problem
import workloads as W


def rng(seed=0):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_rotation_is_complex_multiplication(d):
    x = rng(d).standard_normal((5, d))
    pos = np.array([0, 1, 7, 1000, 65535])
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * 10000.0 ** (-np.arange(d // 2) * 2.0 / d))
    expect = np.concatenate([z.real, z.imag], axis=1)
    np.testing.assert_allclose(rope.rotate(x, pos[:, None][:, 0]), expect, rtol=0, atol=1e-12)


def test_position_zero_is_identity_and_norms_are_kept():
    x = rng(1).standard_normal((3, 4, 128))
    np.testing.assert_array_equal(rope.rotate(x, 0), x)
    y = rope.rotate(x, 12345)
    pair = lambda a: a[..., :64] ** 2 + a[..., 64:] ** 2
    np.testing.assert_allclose(pair(y), pair(x), rtol=1e-12)


def test_scores_depend_on_relative_position_only():
    q, k = rng(2).standard_normal((2, 128))
    s = lambda p, pk: float(rope.rotate(q, p) @ rope.rotate(k, pk))
    for p, pk, shift in [(10, 3, 100), (5000, 4990, 777), (0, 0, 65000)]:
        assert abs(s(p, pk) - s(p + shift, pk + shift)) < 1e-9
        assert abs(s(p, pk) - float(q @ rope.rotate(k, pk - p))) < 1e-9


def brute_force(w, rows):
    """Exact attention over each request's [system; context] keys, both rotated by their
    index in the concatenated sequence, the query at the index of its own key."""
    spec = w.spec
    L, d, g = spec.sys_len, spec.head_dim, spec.group
    vals = lambda a: np.asarray(a, np.float64)
    out = {}
    for b in range(spec.batch):
        c = int(w.ctx_lens[b])
        lo, hi = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
        n = hi - lo
        sk, ck = w.sys_k_keys(), w.ctx_k_keys()
        for hk in range(spec.num_kv_heads):
            ks = [vals(sk[hk, j]) for j in range(L)]
            vs = [vals(w.sys_v[hk, j // 16, :, j % 16]) for j in range(L)]
            for j in range(c):
                p = int(w.block_tables[b, j // 16])
                ks.append(vals(ck[p, hk, j % 16]))
                vs.append(vals(w.ctx_v_pages[p, hk, :, j % 16]))
            K = np.stack([np.asarray(rope.rotate(k, i), np.float32).astype(np.float64) for i, k in enumerate(ks)])
            V = np.stack(vs)
            for t in range(n):
                pos = L + c - n + t
                for gi in range(g):
                    h = hk * g + gi
                    if (lo + t, h) not in rows:
                        continue
                    qv = np.asarray(rope.rotate(vals(w.q[lo + t, h]), pos), np.float32).astype(np.float64)
                    s = spec.scale * (K[: pos + 1] @ qv)
                    p_ = np.exp(s - s.max())
                    out[(lo + t, h)] = (p_ @ V[: pos + 1]) / p_.sum()
    return out


def test_relay_with_offset_positions_equals_unsplit_rotated_attention():
    spec = W.config_spec(5).replace(name="rope-f32", dtype="f32", batch=3, sys_len=20, ctx_lo=5, ctx_hi=40,
                                    num_q_heads=4, num_kv_heads=2, head_dim=64)
    w = W.generate(spec)
    rows = {(t, h) for t in range(int(w.cu_q_lens[-1])) for h in range(spec.num_q_heads)}
    expect = brute_force(w, rows)
    pr = Problem(rope.rotated_workload(w))
    relay_out, _ = pr.relay()
    for (t, h), e in expect.items():
        np.testing.assert_allclose(relay_out[t, h], e, rtol=0, atol=1e-12)
    # a planted mistake: context positions restarting at 0 instead of after the system prompt
    wrong, _ = Problem(rope.rotated_workload(w, ctx_offset=0)).relay()
    assert max(float(np.abs(wrong[t, h] - e).max()) for (t, h), e in expect.items()) > 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_oracle_against_brute_force(dtype):
    r = rng(5)
    L, Hq, Hkv, d = 37, 4, 2, 64
    conv = (lambda x: W.f32_to_bf16_bits(x.astype(np.float32))) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    back = (lambda a: W.bf16_bits_to_f32(a).astype(np.float64)) if dtype == "bf16" else (lambda a: a.astype(np.float64))
    q, k, v = (conv(r.standard_normal(s)) for s in ((L, Hq, d), (L, Hkv, d), (L, Hkv, d)))
    sk, sv, out = rope.prefill_expect(q, k, v, dtype)
    # cache layouts: keys embedded at their positions, values tiled, padding zero
    np.testing.assert_array_equal(back(sv).transpose(0, 1, 3, 2).reshape(Hkv, -1, d)[:, :L], back(v).transpose(1, 0, 2))
    assert not back(sv).transpose(0, 1, 3, 2).reshape(Hkv, -1, d)[:, L:].any()
    qv = back(conv(rope.rotate(back(q), np.arange(L)[:, None])))
    kv = back(conv(rope.rotate(back(k), np.arange(L)[:, None])))
    np.testing.assert_array_equal(back(W.sys_k_dense(sk, L)), kv.transpose(1, 0, 2))
    assert not back(W.k_untile(sk)).reshape(Hkv, -1, d)[:, L:].any()
    G = W.k_chunk(dtype, d)
    for j, c, slot in ((0, 0, 0), (5, G - 1, 9), (17, G, 1), (25, 3, 5), (36, d - 1, 8)):   # key tiles by index arithmetic
        assert back(sk[1, j // 16, c // G, slot, c % G]) == kv[j, 1, c]
    for t in (0, 1, 15, 16, 36):
        for h in range(Hq):
            s = kv[: t + 1, h // 2] @ qv[t, h] / np.sqrt(d)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(out[t, h], p @ back(v)[: t + 1, h // 2] / p.sum(), rtol=0, atol=1e-13)
