"""The no-relay baseline: the same decode step over a paged cache whose block tables
start with the system prompt's pages, shared by every request (prefix sharing of a
paged KV cache).

This is what RelayAttention replaces (RelayAttention paper page, Abstract; atyun.com
article, section "RelayAttention"): with shared system pages the system K/V occupy
memory once, but attention still reads them once per request, because every request's
attention runs over its own [system; context] key sequence.  Here that sequence is
served by the library's context step alone (sys_len = 0): the system tokens become
context positions 0 .. L_s - 1 of every request, its own context follows at L_s.  The
result is the same exact attention, so the two paths are compared on time only.

Input preparation only (torch tensor ops on whatever device the inputs are on); the
attention itself runs in the library's kernels.
"""
from __future__ import annotations

import torch

PAGE = 16


def prefix_shared(t: dict) -> dict:
    """The baseline's inputs from a relay input dict (as ``relay.to_device`` returns).

    The system prompt's K/V become ceil(L_s / 16) pages placed before the context
    pool (one copy, shared); every block table gets those page ids in front of its
    own, shifted past them; context lengths grow by L_s.  L_s must be a multiple of
    16, so that each request's own pages keep their slots.
    """
    L = int(t["sys_len"])
    if L % PAGE:
        raise ValueError(f"system length {L} is not a multiple of {PAGE}: no whole shared pages")
    ck, cv, bt = t["ctx_k_pages"], t["ctx_v_pages"], t["block_tables"]
    nb, H_kv = ck.shape[:2]
    d = cv.shape[2]
    ns = L // PAGE
    if ns:
        # the system caches are already 16-key tiles of the page layouts:
        # sys_k [H_kv, ns, d/G, 16, G] -> [ns, H_kv, d/G, 16, G]; sys_v [H_kv, ns, d, 16] -> [ns, H_kv, d, 16]
        sk = t["sys_k"].reshape(H_kv, ns, *ck.shape[2:]).transpose(0, 1)
        sv = t["sys_v"].reshape(H_kv, ns, d, PAGE).transpose(0, 1)
        pool_k = torch.cat([sk, ck], 0).contiguous()
        pool_v = torch.cat([sv, cv], 0).contiguous()
    else:
        pool_k, pool_v = ck, cv
    B = bt.shape[0]
    front = torch.arange(ns, dtype=bt.dtype, device=bt.device).expand(B, ns)
    own = torch.where(bt >= 0, bt + ns, bt)
    out = dict(t)
    out.update(
        sys_len=0,
        ctx_k_pages=pool_k, ctx_v_pages=pool_v,
        block_tables=torch.cat([front, own], 1).contiguous(),
        ctx_lens=(t["ctx_lens"] + L).contiguous(),
        max_ctx_len=int(t["max_ctx_len"]) + L,
    )
    return out
