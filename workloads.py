"""Seeded synthetic decode-attention workloads.

This module only draws random numbers and lays them out in the storage layouts of
the C ABI (see ``include/relay_attn.h``).  It holds no attention arithmetic: no
scores, no softmax, no fusion.  Both the fp64 oracle (``oracle/``) and the HIP path
consume the arrays it produces, so it is the one piece of code they share.

Shapes and distributions follow the five synthetic decode-attention configurations
of the RelayAttention decode path (Llama2-7B-, Llama-30B- and Llama-3-8B-shaped
layers).  They stand in for the ShareGPT / MMLU serving workloads of the
RelayAttention paper (atyun.com article, section "RelayAttention in practice"),
which are not used here.

Recipe (all integer ranges inclusive):

* Generator per stream: ``numpy.random.Generator(PCG64(SeedSequence([cfg, sweep,
  stream])))``.  Streams: 0 q, 1 sys_k, 2 sys_v, 3 ctx_k, 4 ctx_v, 5 ctx_lens,
  6 q_lens, 7 page permutation, 8 K channel scale.
* Q/K/V values: ``standard_normal(dtype=float32)``; for bf16 storage they are then
  rounded to nearest-even bfloat16 (bit arithmetic below) and stored as uint16 bit
  patterns.  The oracle reads those exact values.
* K channel scale (GQA config only): one vector ``s[H_kv, d] ~ U(0.5, 2)`` multiplies
  every key (system and context) before the bf16 rounding.
* Context lengths ``c_b`` include the ``n_b`` new query tokens, whose K/V are
  already in the pages.  Query t of request b sits at context-local position
  ``c_b - n_b + t``.
* Paging: block size 16; ``num_blocks = sum(ceil(c_b/16)) + B`` (one spare page per
  request); a seeded permutation of page ids is handed out to the requests in order;
  ``block_tables`` rows are padded with -1.  Unused slots of tail pages and spare
  pages are filled with a poison value (finite sentinel K=+1e4, V=-1e4 by default, or
  NaN), which must never reach an output.
* System V padding: the tail 16-key tile of ``sys_v`` is filled with the same poison;
  so are the padding keys of the tail tile of ``sys_k``.
* Key layout: keys are stored in 16-key tiles, each tile as ``[d/G, 16, G]`` with G the
  elements of one 16-byte chunk (8 bf16, 4 fp32; d itself when d is smaller): chunk c
  of every key of the tile, then chunk c + 1; inside a chunk the keys are in slot order
  (``KEY_SLOTS``: keys 4..7 and 8..11 exchanged).  ``k_tiles`` / ``k_untile`` convert from / to ``[..., 16, d]``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BLOCK_SIZE = 16
SYS_TILE = 16  # keys per dim-major tile of the system V cache

F32 = "f32"
BF16 = "bf16"

# Stream ids of the seed sequence.
S_Q, S_SYS_K, S_SYS_V, S_CTX_K, S_CTX_V, S_CTX_LENS, S_Q_LENS, S_PERM, S_KSCALE = range(9)

CONFIG3_SYS_LENS = (512, 1024, 2048, 4096, 8192, 16384)


@dataclass(frozen=True)
class WorkloadSpec:
    """Shape and distribution of one decode-attention layer call."""

    name: str
    cfg: int                 # 1..5, the seed-sequence config id
    sweep: int               # index into a sweep (config 3), else 0
    dtype: str               # "f32" or "bf16"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sys_len: int
    ctx_len_dist: str        # "uniform" | "fixed" | "lognormal"
    ctx_lo: int = 1          # uniform: inclusive range; fixed: ctx_lo
    ctx_hi: int = 1
    ctx_median: float = 0.0  # lognormal median
    ctx_sigma: float = 1.0   # lognormal sigma
    ctx_cap: int = 0         # lognormal cap
    q_lo: int = 1            # new query tokens per request, inclusive range
    q_hi: int = 1
    k_channel_scale: bool = False
    poison: str = "sentinel"  # "sentinel" | "nan"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


def config_spec(cfg: int, sweep: int = 0) -> WorkloadSpec:
    """The five synthetic decode-attention configurations at full size."""
    if cfg == 1:
        return WorkloadSpec("tiny_f32", 1, 0, F32, 4, 2, 2, 64, 128, "uniform", 1, 32)
    if cfg == 2:
        return WorkloadSpec("llama2_7b_mha", 2, 0, BF16, 32, 32, 32, 128, 2048,
                            "uniform", 16, 512)
    if cfg == 3:
        return WorkloadSpec(f"llama30b_mha_sys{CONFIG3_SYS_LENS[sweep]}", 3, sweep, BF16,
                            32, 52, 52, 128, CONFIG3_SYS_LENS[sweep], "fixed", 128, 128)
    if cfg == 4:
        return WorkloadSpec("llama3_8b_gqa", 4, 0, BF16, 256, 32, 8, 128, 8192,
                            "lognormal", ctx_median=300.0, ctx_sigma=1.0, ctx_cap=2048,
                            k_channel_scale=True)
    if cfg == 5:
        return WorkloadSpec("long_sys_multitok_gqa", 5, 0, BF16, 64, 32, 8, 128, 65536,
                            "uniform", 64, 4096, q_lo=1, q_hi=16)
    raise ValueError(f"unknown config {cfg}")


def all_config_specs() -> List[WorkloadSpec]:
    out = [config_spec(1), config_spec(2)]
    out += [config_spec(3, i) for i in range(len(CONFIG3_SYS_LENS))]
    out += [config_spec(4), config_spec(5)]
    return out


def _rng(spec: WorkloadSpec, stream: int, salt: int = 0) -> np.random.Generator:
    key = [spec.cfg, spec.sweep, stream] + ([salt] if salt else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even bfloat16; return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """Arrays in the C-ABI storage layouts (host numpy).

    ``q`` etc. hold float32 values for dtype f32 and uint16 bf16 bit patterns for
    dtype bf16.
    """

    spec: WorkloadSpec
    q: np.ndarray              # [T_q, H_q, d]
    sys_k: np.ndarray          # [H_kv, ceil(L_s/16), d/G, 16, G]  (key tiles)
    sys_v: np.ndarray          # [H_kv, ceil(L_s/16), d, 16]
    ctx_k_pages: np.ndarray    # [num_blocks, H_kv, d/G, 16, G]    (key tiles)
    ctx_v_pages: np.ndarray    # [num_blocks, H_kv, d, 16]
    block_tables: np.ndarray   # int32 [B, max_blocks]
    ctx_lens: np.ndarray       # int32 [B]
    q_lens: np.ndarray         # int32 [B]
    cu_q_lens: np.ndarray      # int32 [B+1]
    # dense per-request context K/V as drawn, before paging: list of [c_b, H_kv, d]
    ctx_k_dense: Optional[List[np.ndarray]] = field(default=None, repr=False)
    ctx_v_dense: Optional[List[np.ndarray]] = field(default=None, repr=False)
    sys_v_dense: Optional[np.ndarray] = field(default=None, repr=False)  # [H_kv, L_s, d]

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_lens.max()) if len(self.ctx_lens) else 0

    @property
    def num_blocks(self) -> int:
        return int(self.ctx_k_pages.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def sys_k_keys(self) -> np.ndarray:
        """System keys in storage form, key-major ``[H_kv, L_s, d]``."""
        return sys_k_dense(self.sys_k, self.spec.sys_len)

    def ctx_k_keys(self) -> np.ndarray:
        """Context key pages in storage form, key-major ``[num_blocks, H_kv, 16, d]``."""
        return k_untile(self.ctx_k_pages)

    def values(self, a: np.ndarray) -> np.ndarray:
        """Exact float32 values of a storage array."""
        return bf16_bits_to_f32(a) if self.spec.dtype == BF16 else a

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.sys_k, self.sys_v, self.ctx_k_pages, self.ctx_v_pages,
                  self.block_tables, self.ctx_lens, self.cu_q_lens):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def _draw_lens(spec: WorkloadSpec) -> tuple:
    B = spec.batch
    r = _rng(spec, S_Q_LENS)
    q_lens = r.integers(spec.q_lo, spec.q_hi + 1, size=B).astype(np.int32)
    r = _rng(spec, S_CTX_LENS)
    if spec.ctx_len_dist == "uniform":
        ctx = r.integers(spec.ctx_lo, spec.ctx_hi + 1, size=B)
    elif spec.ctx_len_dist == "fixed":
        ctx = np.full(B, spec.ctx_lo)
    elif spec.ctx_len_dist == "lognormal":
        x = r.lognormal(mean=math.log(spec.ctx_median), sigma=spec.ctx_sigma, size=B)
        ctx = np.clip(np.rint(x), 1, spec.ctx_cap)
    else:
        raise ValueError(spec.ctx_len_dist)
    ctx = np.maximum(ctx.astype(np.int64), q_lens).astype(np.int32)
    return q_lens, ctx


def k_chunk(dtype: str, d: int) -> int:
    """Elements of one 16-byte chunk of a key row (a whole row when d is below it)."""
    return min(8 if dtype == BF16 else 4, d)


# Slot order of the keys inside a key tile: slot s holds key KEY_SLOTS[s] (keys 4..7
# and 8..11 exchanged; the permutation is its own inverse).
KEY_SLOTS = np.array([0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15])


def k_tiles(k: np.ndarray, dtype: str) -> np.ndarray:
    """Key-major 16-key tiles ``[..., 16, d]`` -> the cache's key layout ``[..., d/G, 16, G]``
    (slot s of every chunk holds key ``KEY_SLOTS[s]``)."""
    *lead, t, d = k.shape
    G = k_chunk(dtype, d)
    return np.ascontiguousarray(k[..., KEY_SLOTS, :].reshape(*lead, t, d // G, G).swapaxes(-3, -2))


def k_untile(k: np.ndarray) -> np.ndarray:
    """The cache's key layout ``[..., d/G, 16, G]`` -> key-major ``[..., 16, d]``."""
    *lead, c, t, g = k.shape
    return np.ascontiguousarray(k.swapaxes(-3, -2).reshape(*lead, t, c * g)[..., KEY_SLOTS, :])


def sys_k_dense(sys_k: np.ndarray, sys_len: int) -> np.ndarray:
    """The system key cache ``[H_kv, ceil(L_s/16), d/G, 16, G]`` as ``[H_kv, L_s, d]``."""
    t = k_untile(sys_k)
    return t.reshape(t.shape[0], -1, t.shape[-1])[:, :sys_len]


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, np.float32)


def _poison_values(spec: WorkloadSpec) -> tuple:
    if spec.poison == "nan":
        pk = pv = np.float32(np.nan)
    else:
        pk, pv = np.float32(1.0e4), np.float32(-1.0e4)
    return _to_storage(np.array([pk]), spec.dtype)[0], _to_storage(np.array([pv]), spec.dtype)[0]


def generate(spec: WorkloadSpec, keep_dense: bool = False) -> Workload:
    """Draw one seeded workload in the C-ABI layouts."""
    B, Hq, Hkv, d, Ls = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.sys_len
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    store = np.uint16 if spec.dtype == BF16 else np.float32
    q_lens, ctx_lens = _draw_lens(spec)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(q_lens)
    Tq = int(cu[-1])

    kscale = None
    if spec.k_channel_scale:
        kscale = _rng(spec, S_KSCALE).uniform(0.5, 2.0, size=(Hkv, d)).astype(np.float32)

    q = _to_storage(_rng(spec, S_Q).standard_normal((Tq, Hq, d), dtype=np.float32), spec.dtype)

    sk = _rng(spec, S_SYS_K).standard_normal((Hkv, Ls, d), dtype=np.float32)
    if kscale is not None:
        sk *= kscale[:, None, :]
    pk, pv = _poison_values(spec)
    nbs = -(-Ls // SYS_TILE)
    sys_k = np.full((Hkv, nbs * SYS_TILE, d), pk, dtype=store)
    sys_k[:, :Ls, :] = _to_storage(sk, spec.dtype)
    del sk
    sys_k = k_tiles(sys_k.reshape(Hkv, nbs, SYS_TILE, d), spec.dtype)
    sv = _to_storage(_rng(spec, S_SYS_V).standard_normal((Hkv, Ls, d), dtype=np.float32), spec.dtype)
    sys_v = np.full((Hkv, nbs * SYS_TILE, d), pv, dtype=store)
    sys_v[:, :Ls, :] = sv
    # [H_kv, nbs, 16, d] -> dim-major tiles [H_kv, nbs, d, 16]
    sys_v = np.ascontiguousarray(sys_v.reshape(Hkv, nbs, SYS_TILE, d).transpose(0, 1, 3, 2))

    # paging
    pages_per = [-(-int(c) // BLOCK_SIZE) for c in ctx_lens]
    num_blocks = int(sum(pages_per)) + B
    max_blocks = max(pages_per) if pages_per else 0
    perm = _rng(spec, S_PERM).permutation(num_blocks).astype(np.int32)
    block_tables = np.full((B, max(max_blocks, 1)), -1, dtype=np.int32)
    kp = np.full((num_blocks, Hkv, BLOCK_SIZE, d), pk, dtype=store)
    vp = np.full((num_blocks, Hkv, d, BLOCK_SIZE), pv, dtype=store)
    rk, rv = _rng(spec, S_CTX_K), _rng(spec, S_CTX_V)
    k_dense, v_dense = [], []
    pos = 0
    for b in range(B):
        c = int(ctx_lens[b])
        ids = perm[pos:pos + pages_per[b]]
        pos += pages_per[b]
        block_tables[b, :len(ids)] = ids
        kb = rk.standard_normal((c, Hkv, d), dtype=np.float32)
        if kscale is not None:
            kb *= kscale[None, :, :]
        kb = _to_storage(kb, spec.dtype)
        vb = _to_storage(rv.standard_normal((c, Hkv, d), dtype=np.float32), spec.dtype)
        for i, blk in enumerate(ids):
            lo, hi = i * BLOCK_SIZE, min(c, (i + 1) * BLOCK_SIZE)
            kp[blk, :, : hi - lo, :] = kb[lo:hi].transpose(1, 0, 2)
            vp[blk, :, :, : hi - lo] = vb[lo:hi].transpose(1, 2, 0)
        if keep_dense:
            k_dense.append(kb)
            v_dense.append(vb)
    kp = k_tiles(kp, spec.dtype)
    return Workload(spec, q, sys_k, sys_v, kp, vp, block_tables, ctx_lens, q_lens, cu,
                    k_dense if keep_dense else None, v_dense if keep_dense else None,
                    sv if keep_dense else None)


def relabel_pages(w: Workload, seed: int) -> Workload:
    """Same logical workload with the physical page ids permuted (for invariance tests)."""
    nb = w.num_blocks
    perm = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77]))).permutation(nb)
    kp = np.empty_like(w.ctx_k_pages)
    vp = np.empty_like(w.ctx_v_pages)
    kp[perm] = w.ctx_k_pages
    vp[perm] = w.ctx_v_pages
    bt = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    return dataclasses.replace(w, ctx_k_pages=kp, ctx_v_pages=vp, block_tables=bt)


def expected_sizes(spec: WorkloadSpec) -> dict:
    """Element counts of the drawn arrays (cheap; no generation)."""
    q_lens, ctx = _draw_lens(spec)
    return {"total_q": int(q_lens.sum()), "sum_ctx": int(ctx.sum()), "max_ctx": int(ctx.max()),
            "ctx_lens": ctx, "q_lens": q_lens}
