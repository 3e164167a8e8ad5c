"""fp64 CPU oracle for the step before the relay path: rotary position embedding with
context positions offset by the system length, and the append of new tokens' K/V to
the paged context cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): only ``tests/``, the smoke check
and the benchmark's CPU leg use it; it imports nothing from the product.

The pages fix the position contract only: the system K/V are prefilled offline at
positions 0 .. L_s - 1, so every request's own tokens are placed after them, at
positions offset by the system length (atyun.com article, section "RelayAttention";
linnk.ai summary, section "Deeper Inquiries": position embeddings adjusted when the
system KV cache is prefilled).  They do not fix the embedding.  The reading taken is rotary position
embedding (RoPE) as the Llama family of the pages' models uses it, in "rotate half"
form: with i < d/2 and inverse frequency f_i = base^(-2i/d),

    out[i]       = x[i] cos(p f_i) - x[i + d/2] sin(p f_i)
    out[i + d/2] = x[i + d/2] cos(p f_i) + x[i] sin(p f_i)

applied to queries and keys (not values) at their absolute position p.  Context token
j of request b is at absolute position L_s + j; new query token t at L_s + c_b - n_b + t.

Everything here is fp64 numpy; results stored in a bf16 cache are rounded to bf16 (via
float32, round to nearest even), as the cache stores them.
"""
from __future__ import annotations

import copy

import numpy as np

import workloads as W  # the seeded generator only (no arithmetic)

ROPE_BASE = 10000.0


def angles(pos, d: int, base: float = ROPE_BASE) -> np.ndarray:
    """p * f_i for every position in `pos` and i < d/2 (fp64): shape pos.shape + (d/2,)."""
    inv = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv


def rotate(x: np.ndarray, pos, base: float = ROPE_BASE) -> np.ndarray:
    """RoPE of vectors x[..., d] (fp64) at positions `pos` (broadcast over x's leading dims
    except the last): the rotate-half form above."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = angles(pos, d, base)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _values(w, a: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(a).astype(np.float64) if w.spec.dtype == "bf16" else np.asarray(a, np.float64)


def _store(w, x: np.ndarray) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float32)
    return W.f32_to_bf16_bits(x32) if w.spec.dtype == "bf16" else x32


def token_positions(w) -> np.ndarray:
    """Absolute position of every new query token (row t of q): L_s + c_b - n_b + t_local."""
    pos = np.zeros(int(w.cu_q_lens[-1]), np.int64)
    for b in range(w.spec.batch):
        lo, hi = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
        n, c = hi - lo, int(w.ctx_lens[b])
        pos[lo:hi] = w.spec.sys_len + c - n + np.arange(n)
    return pos


def rotated_workload(w, base: float = ROPE_BASE, ctx_offset=None):
    """The workload as the relay path sees it after RoPE: q at its tokens' absolute
    positions, system keys at 0 .. L_s - 1, context keys of request b at
    ctx_offset + j (ctx_offset = L_s, the pages' contract; another value only for
    tests that plant a mistake), values unchanged.  Stored in the workload's dtype."""
    spec = w.spec
    L = spec.sys_len
    off = L if ctx_offset is None else ctx_offset
    H_kv, d = spec.num_kv_heads, spec.head_dim
    r = copy.copy(w)
    # queries [T_q, H_q, d]
    q = _values(w, w.q)
    r.q = _store(w, rotate(q, token_positions(w)[:, None]))
    # system keys: key tiles -> [H_kv, padded L_s, d], first L_s rotated, back to tiles
    if L > 0:
        sk = W.k_untile(w.sys_k)
        sk = sk.reshape(sk.shape[0], -1, d)
        rot = _store(w, rotate(_values(w, sk[:, :L]), np.arange(L)[None, :]))
        sk = sk.copy()
        sk[:, :L] = rot
        r.sys_k = W.k_tiles(sk.reshape(H_kv, -1, 16, d), spec.dtype)
    # context keys through the block tables: key tiles -> [num_blocks, H_kv, 16, d]
    ck = _values(w, W.k_untile(w.ctx_k_pages)).copy()
    for b in range(spec.batch):
        for j in range(int(w.ctx_lens[b])):
            p = int(w.block_tables[b, j // 16])
            ck[p, :, j % 16, :] = rotate(ck[p, :, j % 16, :], off + j)
    r.ctx_k_pages = W.k_tiles(_store(w, ck), spec.dtype)
    r.ctx_k_dense = r.ctx_v_dense = None
    return r


def append_expect(w, q_new, k_new, v_new, base: float = ROPE_BASE):
    """What appending the new tokens does, as values: (q_rot [T_q, H_q, d],
    k_rot [T_q, H_kv, d], v [T_q, H_kv, d]) in fp64 before storage rounding.  Token t
    (row t, request b) goes to context position c_b - n_b + t_local, absolute position
    L_s + that; its K/V land at page block_tables[b][p / 16], slot p % 16."""
    pos = token_positions(w)
    return rotate(q_new, pos[:, None], base), rotate(k_new, pos[:, None], base), np.asarray(v_new, np.float64)


def prefill_expect(q_raw, k_raw, v_raw, dtype: str, base: float = ROPE_BASE):
    """The offline prefill of a system prompt, as values: queries q_raw [L, H_q, d] and
    keys / values k_raw, v_raw [L, H_kv, d] in storage form (bf16 bit patterns or
    float32), before position embedding.  Returns (sys_k [H_kv, ceil(L/16), d/G, 16, G]
    and sys_v [H_kv, ceil(L/16), d, 16] in storage form, out [L, H_q, d] fp64): the
    system cache (keys embedded at positions 0..L-1 in 16-key chunk-major tiles, values
    in 16-key dimension-major tiles, tail padding 0 in both) and every prompt token's causal attention over keys 0..its own position
    (computed by the fp64 C oracle on a one-request workload whose L tokens are new)."""
    from . import Problem
    L, H_q, d = q_raw.shape
    H_kv = k_raw.shape[1]
    vals = (lambda a: W.bf16_bits_to_f32(a).astype(np.float64)) if dtype == "bf16" else \
        (lambda a: np.asarray(a, np.float64))
    store = (lambda x: W.f32_to_bf16_bits(np.asarray(x, np.float32))) if dtype == "bf16" else \
        (lambda x: np.asarray(x, np.float32))
    pos = np.arange(L)
    k_rot = store(rotate(vals(k_raw), pos[:, None]))          # [L, H_kv, d]
    q_rot = store(rotate(vals(q_raw), pos[:, None]))          # [L, H_q, d]
    ntile = (L + 15) // 16
    sys_k = np.zeros((H_kv, ntile * 16, d), dtype=k_rot.dtype)
    sys_k[:, :L] = k_rot.transpose(1, 0, 2)
    sys_k = W.k_tiles(sys_k.reshape(H_kv, ntile, 16, d), dtype)
    sys_v = np.zeros((H_kv, ntile * 16, d), dtype=np.asarray(v_raw).dtype)
    sys_v[:, :L] = np.asarray(v_raw).transpose(1, 0, 2)
    sys_v = np.ascontiguousarray(sys_v.reshape(H_kv, ntile, 16, d).transpose(0, 1, 3, 2))
    # the prompt as one request: pages 0..ntile-1 in order, every token new
    kp = np.zeros((ntile * 16, H_kv, d), dtype=k_rot.dtype)
    kp[:L] = k_rot
    kp = W.k_tiles(kp.reshape(ntile, 16, H_kv, d).transpose(0, 2, 1, 3), dtype)
    vp = np.ascontiguousarray(sys_v.transpose(1, 0, 2, 3))     # [ntile, H_kv, d, 16]
    spec = W.WorkloadSpec("prefill", 0, 0, dtype, 1, H_q, H_kv, d, 0, "fixed", L, L, q_lo=L, q_hi=L)
    G = W.k_chunk(dtype, d)
    empty = np.zeros((H_kv, 0, d // G, 16, G), dtype=k_rot.dtype)
    w = W.Workload(spec, q_rot, empty, np.zeros((H_kv, 0, d, 16), dtype=k_rot.dtype), kp, vp,
                   np.arange(ntile, dtype=np.int32)[None, :], np.array([L], np.int32),
                   np.array([L], np.int32), np.array([0, L], np.int32))
    out, _ = Problem(w).attention()
    return sys_k, sys_v, out
