"""Offline system-prompt prefill: fill the contiguous system KV cache before serving,
and save / load it.

RelayAttention keeps the system prompt's K/V in a cache of its own, filled once,
offline, before the model serves (atyun.com article, section "RelayAttention": a
separate system KV cache prefilled offline; prefix sharing plus prompt caching).  The
prefill here takes the system prompt's queries, keys and values as a projection
produces them (token-major, before position embedding; the projection weights are a
model's and are out of scope) and

* writes the system cache (``relay_system_fill``): keys with RoPE at positions
  0 .. L_s - 1, values in 16-key dimension-major tiles;
* computes the prompt's own causal attention outputs, which a model's next layer
  consumes.  On the matrix-core path (bf16, head_dim 128, more than 64 query rows per
  KV head) that is ``relay_prefill_attn``: the system kernel with a causal mask, run
  over the cache just filled, with the queries embedded by ``relay_rope_append``.
  Otherwise the library's decode path runs the prompt as one request whose L_s tokens
  are all new (``relay_rope_append`` also builds that request's pages,
  ``relay_attn_decode`` with ``sys_len = 0`` is the causal attention);
* saves and loads the cache (safetensors: data only, nothing executed on load).

Every computation runs in the library's kernels; this module allocates tensors and
calls them.
"""
from __future__ import annotations

import json

import torch

from . import relay

PAGE = 16


def uses_matrix_cores(q_raw: torch.Tensor, k_raw: torch.Tensor, scale: float) -> bool:
    """Whether prefill_system's attention runs on relay_prefill_attn."""
    L, H_q, d = q_raw.shape
    return q_raw.dtype == torch.bfloat16 and d == 128 and L * (H_q // k_raw.shape[1]) > 64 and scale > 0


def prefill_system(q_raw: torch.Tensor, k_raw: torch.Tensor, v_raw: torch.Tensor, cos_sin: torch.Tensor,
                   scale: float, *, out_dtype=torch.float32, method: str = "auto", stream=None):
    """(sys_k [H_kv, ceil(L_s/16), d/G, 16, G], sys_v [H_kv, ceil(L_s/16), d, 16], out [L_s, H_q, d]).

    q_raw [L_s, H_q, d], k_raw / v_raw [L_s, H_kv, d]: the prompt's projections before
    position embedding (bf16 or fp32, one dtype).  cos_sin: ``relay.relay_rope_table``
    with at least L_s rows.  ``out[j]`` is token j's causal attention over keys 0..j.
    method: "auto" (matrix cores when they apply), "mfma" or "decode".
    """
    L, H_q, d = q_raw.shape
    if k_raw.shape[0] != L or v_raw.shape != k_raw.shape:
        raise ValueError("q_raw [L, H_q, d], k_raw and v_raw [L, H_kv, d] expected")
    if method not in ("auto", "mfma", "decode"):
        raise ValueError(f"unknown method {method!r}")
    sys_k, sys_v = relay.relay_system_fill(k_raw, v_raw, cos_sin, stream=stream)
    H_kv = k_raw.shape[1]
    dev = q_raw.device
    npages = (L + PAGE - 1) // PAGE
    if method == "mfma" or (method == "auto" and uses_matrix_cores(q_raw, k_raw, scale)):
        # queries only: a block table of -1 makes relay_rope_append write no K/V
        bt = torch.full((1, npages), -1, dtype=torch.int32, device=dev)
        ctx_lens = torch.tensor([L], dtype=torch.int32, device=dev)
        cu = torch.tensor([0, L], dtype=torch.int32, device=dev)
        no_page = torch.empty(relay.key_tile_shape((1, H_kv), d, k_raw.dtype), dtype=k_raw.dtype, device=dev)
        dims = relay.make_dims(q_raw, no_page, bt, scale=scale, max_ctx_len=L, max_q_len=L)
        q_rot = relay.relay_rope_append(dims, 0, q_raw, k_raw, v_raw, cos_sin, bt, ctx_lens, cu, no_page,
                                        torch.empty((1, H_kv, d, PAGE), dtype=k_raw.dtype, device=dev),
                                        stream=stream)
        out, _ = relay.relay_prefill_attn(q_rot, sys_k, sys_v, L, scale, out_dtype=out_dtype, stream=stream)
        return sys_k, sys_v, out
    pages_k = torch.empty(relay.key_tile_shape((npages, H_kv), d, k_raw.dtype), dtype=k_raw.dtype, device=dev)
    pages_v = torch.empty((npages, H_kv, d, PAGE), dtype=k_raw.dtype, device=dev)
    bt = torch.arange(npages, dtype=torch.int32, device=dev).view(1, npages)
    ctx_lens = torch.tensor([L], dtype=torch.int32, device=dev)
    cu = torch.tensor([0, L], dtype=torch.int32, device=dev)
    dims = relay.make_dims(q_raw, pages_k, bt, scale=scale, max_ctx_len=L, max_q_len=L)
    q_rot = relay.relay_rope_append(dims, 0, q_raw, k_raw, v_raw, cos_sin, bt, ctx_lens, cu, pages_k, pages_v,
                                    stream=stream)
    out = relay.relay_attn_decode(q_rot, sys_k, sys_v, 0, pages_k, pages_v, bt, ctx_lens, cu, scale=scale,
                                  max_ctx_len=L, max_q_len=L, out_dtype=out_dtype, stream=stream)
    return sys_k, sys_v, out


def save_system_cache(path: str, sys_k: torch.Tensor, sys_v: torch.Tensor, sys_len: int,
                      rope_base: float = 10000.0) -> None:
    """Write the system cache to a safetensors file (tensors and a small JSON header)."""
    from safetensors.torch import save_file
    meta = {"format": "relay-system-kv/2", "sys_len": str(int(sys_len)), "rope_base": repr(float(rope_base)),
            "layout": json.dumps({"sys_k": "[H_kv, ceil(L_s/16), d/G, 16, G]", "sys_v": "[H_kv, ceil(L_s/16), d, 16]"})}
    save_file({"sys_k": sys_k.contiguous().cpu(), "sys_v": sys_v.contiguous().cpu()}, path, metadata=meta)


def load_system_cache(path: str, device="cuda"):
    """(sys_k, sys_v, sys_len, rope_base) from a file written by save_system_cache."""
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        meta = f.metadata() or {}
        if meta.get("format") != "relay-system-kv/2":
            raise ValueError(f"{path}: not a system KV cache file")
        sys_k = f.get_tensor("sys_k").to(device)
        sys_v = f.get_tensor("sys_v").to(device)
    return sys_k, sys_v, int(meta["sys_len"]), float(meta["rope_base"])
