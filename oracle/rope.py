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

from shared_prompt_kv_amd import workloads as W  # the seeded generator only (no arithmetic)

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
    # system keys [H_kv, L_s, d]
    if L > 0:
        sk = _values(w, w.sys_k)
        r.sys_k = _store(w, rotate(sk, np.arange(L)[None, :]))
    # context keys through the block tables: [num_blocks, H_kv, 16, d]
    ck = _values(w, w.ctx_k_pages).copy()
    for b in range(spec.batch):
        for j in range(int(w.ctx_lens[b])):
            p = int(w.block_tables[b, j // 16])
            ck[p, :, j % 16, :] = rotate(ck[p, :, j % 16, :], off + j)
    r.ctx_k_pages = _store(w, ck)
    r.ctx_k_dense = r.ctx_v_dense = None
    return r


def append_expect(w, q_new, k_new, v_new, base: float = ROPE_BASE):
    """What appending the new tokens does, as values: (q_rot [T_q, H_q, d],
    k_rot [T_q, H_kv, d], v [T_q, H_kv, d]) in fp64 before storage rounding.  Token t
    (row t, request b) goes to context position c_b - n_b + t_local, absolute position
    L_s + that; its K/V land at page block_tables[b][p / 16], slot p % 16."""
    pos = token_positions(w)
    return rotate(q_new, pos[:, None], base), rotate(k_new, pos[:, None], base), np.asarray(v_new, np.float64)
