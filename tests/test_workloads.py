"""The seeded input generator: determinism, ranges and paging structure."""
import json
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_same_seed_same_bytes_and_recorded_hashes():
    with open(os.path.join(GOLDEN, "workload_sha256.json")) as f:
        rec = json.load(f)
    for name, spec in _hash_specs().items():
        a = W.generate(spec).sha256()
        assert a == W.generate(spec).sha256()
        assert a == rec[name], name


def _hash_specs():
    return {
        "c1": W.config_spec(1),
        "c2_small": W.config_spec(2).replace(batch=3, sys_len=100, ctx_hi=70),
        "c4_small": W.config_spec(4).replace(batch=4, sys_len=50, ctx_median=30, ctx_cap=64),
        "c5_small": W.config_spec(5).replace(batch=3, sys_len=77, ctx_lo=20, ctx_hi=60),
    }


@pytest.mark.parametrize("cfg,sweep", [(1, 0), (2, 0), (3, 0), (3, 5), (4, 0), (5, 0)])
def test_length_distributions(cfg, sweep):
    spec = W.config_spec(cfg, sweep)
    s = W.expected_sizes(spec)
    ctx, ql = s["ctx_lens"], s["q_lens"]
    assert len(ctx) == spec.batch and np.all(ql <= ctx) and np.all(ql >= 1)
    if spec.ctx_len_dist == "uniform":
        assert ctx.min() >= spec.ctx_lo and ctx.max() <= spec.ctx_hi
    elif spec.ctx_len_dist == "fixed":
        assert np.all(ctx == spec.ctx_lo)
    else:
        assert ctx.min() >= 1 and ctx.max() <= spec.ctx_cap
        assert 150 < np.median(ctx) < 600
    assert ql.min() >= spec.q_lo and ql.max() <= spec.q_hi


def test_paging_structure_and_poison():
    spec = W.config_spec(5).replace(batch=5, sys_len=37, ctx_lo=20, ctx_hi=70, poison="nan")
    w = W.generate(spec, keep_dense=True)
    used = w.block_tables[w.block_tables >= 0]
    assert len(np.unique(used)) == len(used)                  # pages are not shared
    assert w.num_blocks == len(used) + spec.batch             # one spare page per request
    ck = w.ctx_k_keys()
    vals_k = w.values(ck)
    vals_v = w.values(w.ctx_v_pages)
    G = W.k_chunk(spec.dtype, spec.head_dim)
    for b in range(spec.batch):
        c = int(w.ctx_lens[b])
        n = -(-c // 16)
        assert np.all(w.block_tables[b, :n] >= 0) and np.all(w.block_tables[b, n:] == -1)
        for j in range(c):
            blk = w.block_tables[b, j // 16]
            np.testing.assert_array_equal(ck[blk, :, j % 16, :], w.ctx_k_dense[b][j])
            slot = (j % 16) ^ 12 if 4 <= j % 16 < 12 else j % 16   # keys 4..7 and 8..11 exchanged
            for c in (0, G - 1, G, spec.head_dim - 1):   # key tiles: chunk-major, G per chunk, slot order
                np.testing.assert_array_equal(w.ctx_k_pages[blk, :, c // G, slot, c % G], w.ctx_k_dense[b][j][:, c])
            np.testing.assert_array_equal(w.ctx_v_pages[blk, :, :, j % 16], w.ctx_v_dense[b][j])
        tail = w.block_tables[b, n - 1]
        assert np.all(np.isnan(vals_k[tail, :, c - (n - 1) * 16:, :]))
        assert np.all(np.isnan(vals_v[tail, :, :, c - (n - 1) * 16:]))
    spare = np.setdiff1d(np.arange(w.num_blocks), used)
    assert np.all(np.isnan(vals_k[spare])) and np.all(np.isnan(vals_v[spare]))
    # system V: dim-major 16-key tiles, poison in the tail tile's padding
    sv = w.values(w.sys_v)
    for j in (0, 15, 16, 36):
        np.testing.assert_array_equal(w.sys_v[:, j // 16, :, j % 16], w.sys_v_dense[:, j, :])
    assert np.all(np.isnan(sv[:, 2, :, 37 - 32:]))
    # system K: the same tiles as the pages, poison in the tail tile's padding keys
    sk = w.values(W.k_untile(w.sys_k))
    assert sk.shape == (spec.num_kv_heads, 3, 16, spec.head_dim)
    np.testing.assert_array_equal(w.sys_k_keys(), W.k_untile(w.sys_k).reshape(spec.num_kv_heads, 48, -1)[:, :37])
    assert np.all(np.isnan(sk[:, 2, 37 - 32:, :]))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, -2.5, 1.0 + 2**-9, 1.0 + 3 * 2**-8], np.float32)
    got = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    # bf16 keeps 7 fraction bits (ulp(1) = 2^-7): 1+2^-8 and 1+3*2^-8 are ties -> even
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2**-7, -2.5, 1.0,
                                                  1.0 + 2**-6], np.float32))


def test_gqa_k_channel_scale_applied():
    spec = W.config_spec(4).replace(batch=2, sys_len=64, ctx_median=20, ctx_cap=40)
    w = W.generate(spec)
    ks = W.bf16_bits_to_f32(w.sys_k_keys()).astype(np.float64)
    std = ks.reshape(-1, spec.head_dim).std(0)
    assert std.max() / std.min() > 2.0  # per-channel scale in [0.5, 2]
