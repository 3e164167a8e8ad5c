"""Python binding of librelay_attn.so (ctypes; argument marshalling only).

Every function has the name of the C entry point it calls (see
``include/relay_attn.h`` for the contract).  Tensors are torch device tensors;
PyTorch supplies the device memory and the current stream, nothing else: every
step of the computation runs in the library's HIP kernels.  There is no fallback:
if the library is missing or the device is not a GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librelay_attn.so")

RELAY_F32, RELAY_BF16 = 0, 1
RELAY_OK = 0
RELAY_ERR_WORKSPACE = -3
NOALLOC_SCRATCH_BYTES = 128 << 20  # the header's RELAY_NOALLOC_SCRATCH_BYTES


class relay_dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


class relay_plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "sys_mode", "sys_row_tiles", "sys_runs", "sys_wgs", "ctx_row_tiles", "ctx_row_blocks",
        "stream_waves", "stream_launches", "stream_max_requests", "merge_wgs", "launches", "sys_rows_per_wg",
        "sys_row_slots", "ctx_row_slots")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class RelayError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"relay error {code}: {msg}")
        self.code = code


EXPORTS = ("relay_abi_version", "relay_strerror", "relay_last_error", "relay_workspace_size",
           "relay_get_plan", "relay_attn_decode", "relay_attn_decode_timed", "relay_attn_decode_noalloc",
           "relay_sys_attn",
           "relay_ctx_attn", "relay_fuse", "relay_validate", "relay_rope_table", "relay_rope_append",
           "relay_rope_system", "relay_system_fill", "relay_prefill_workspace_size", "relay_prefill_attn")

_lib = None


def load_library(path: str = LIB_PATH):
    """Load librelay_attn.so and declare its signatures (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m shared_prompt_kv_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(relay_dims)
    lib.relay_abi_version.argtypes, lib.relay_abi_version.restype = [], ctypes.c_int
    lib.relay_strerror.argtypes, lib.relay_strerror.restype = [ctypes.c_int], ctypes.c_char_p
    lib.relay_last_error.argtypes, lib.relay_last_error.restype = [], ctypes.c_char_p
    lib.relay_workspace_size.argtypes, lib.relay_workspace_size.restype = [D, i32], sz
    lib.relay_get_plan.argtypes = [D, i32, ctypes.POINTER(relay_plan)]
    lib.relay_get_plan.restype = ctypes.c_int
    lib.relay_attn_decode.argtypes = [D, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.relay_attn_decode.restype = ctypes.c_int
    lib.relay_attn_decode_noalloc.argtypes = [D, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.relay_attn_decode_noalloc.restype = ctypes.c_int
    lib.relay_attn_decode_timed.argtypes = [D, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                            ctypes.POINTER(vp)]
    lib.relay_attn_decode_timed.restype = ctypes.c_int
    lib.relay_sys_attn.argtypes = [D, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.relay_sys_attn.restype = ctypes.c_int
    lib.relay_prefill_workspace_size.argtypes = [D, i32]
    lib.relay_prefill_workspace_size.restype = sz
    lib.relay_prefill_attn.argtypes = [D, vp, vp, vp, i32, vp, i32, vp, vp, sz, vp]
    lib.relay_prefill_attn.restype = ctypes.c_int
    lib.relay_ctx_attn.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.relay_ctx_attn.restype = ctypes.c_int
    lib.relay_fuse.argtypes = [ctypes.c_int64, i32, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.relay_fuse.restype = ctypes.c_int
    lib.relay_validate.argtypes = [D, vp, vp, vp, i32]
    lib.relay_validate.restype = ctypes.c_int
    lib.relay_rope_table.argtypes = [vp, i32, i32, ctypes.c_float, vp]
    lib.relay_rope_table.restype = ctypes.c_int
    lib.relay_rope_append.argtypes = [D, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.relay_rope_append.restype = ctypes.c_int
    lib.relay_rope_system.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp]
    lib.relay_rope_system.restype = ctypes.c_int
    lib.relay_system_fill.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp]
    lib.relay_system_fill.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != RELAY_OK:
        lib = load_library()
        raise RelayError(rc, f"{lib.relay_strerror(rc).decode()}: {lib.relay_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return RELAY_F32
    if dt == torch.bfloat16:
        return RELAY_BF16
    raise ValueError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _stream(stream) -> ctypes.c_void_p:
    """hipStream_t of a torch stream, a raw handle (int), or the current stream."""
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require_device(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be GPU tensors")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _elems16(dt: torch.dtype) -> int:
    return 8 if dt == torch.bfloat16 else 4


def _check_system_cache(q, sys_k, sys_v, sys_len: int, num_kv_heads: int):
    """sys_k / sys_v must be the system cache layouts of q's dtype covering sys_len keys."""
    if sys_len < 0:
        raise ValueError(f"sys_len must be >= 0 (got {sys_len})")
    if sys_len == 0:
        return
    d = q.shape[-1]
    g = min(_elems16(q.dtype), d)
    tiles = -(-sys_len // 16)
    for name, x in (("sys_k", sys_k), ("sys_v", sys_v)):
        if x is None:
            raise ValueError(f"{name} is required when sys_len > 0")
        if x.dtype != q.dtype:
            raise ValueError(f"{name} dtype {x.dtype} differs from q's {q.dtype}")
    want_k = (num_kv_heads, tiles, d // g, 16, g)
    want_v = (num_kv_heads, tiles, d, 16)
    # the kernels step from one KV head's tiles to the next by ceil(sys_len / 16) tiles
    if tuple(sys_k.shape) != want_k:
        raise ValueError(f"sys_k must be key tiles {want_k} for sys_len {sys_len}, got {tuple(sys_k.shape)}")
    if tuple(sys_v.shape) != want_v:
        raise ValueError(f"sys_v must be value tiles {want_v} for sys_len {sys_len}, got {tuple(sys_v.shape)}")


def _check_context(q, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens):
    """Paged context cache, block tables and lengths: layouts, dtypes and batch size."""
    if q.dim() != 3:
        raise ValueError("q must be [T_q, H_q, d]")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"unsupported dtype {q.dtype} (float32 or bfloat16)")
    Tq, Hq, d = q.shape
    g = min(_elems16(q.dtype), d)
    if ctx_k_pages.dim() != 5 or ctx_k_pages.shape[2] * ctx_k_pages.shape[4] != d or ctx_k_pages.shape[3] != 16 \
            or ctx_k_pages.shape[4] != g:
        raise ValueError(f"ctx_k_pages must be key tiles [num_blocks, H_kv, {d // g}, 16, {g}], "
                         f"got {tuple(ctx_k_pages.shape)}")
    nb, Hkv = ctx_k_pages.shape[:2]
    if tuple(ctx_v_pages.shape) != (nb, Hkv, d, 16):
        raise ValueError(f"ctx_v_pages must be [{nb}, {Hkv}, {d}, 16], got {tuple(ctx_v_pages.shape)}")
    for name, x in (("ctx_k_pages", ctx_k_pages), ("ctx_v_pages", ctx_v_pages)):
        if x.dtype != q.dtype:
            raise ValueError(f"{name} dtype {x.dtype} differs from q's {q.dtype}")
    if Hq % Hkv:
        raise ValueError(f"H_q ({Hq}) must be a multiple of H_kv ({Hkv})")
    if block_tables.dim() != 2 or block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32 [B, max_blocks_per_seq]")
    B = block_tables.shape[0]
    if ctx_lens.dtype != torch.int32 or tuple(ctx_lens.shape) != (B,):
        raise ValueError(f"ctx_lens must be int32 [{B}]")
    if cu_q_lens is None:
        if Tq != B:
            raise ValueError(f"without cu_q_lens every request has one query token: q has {Tq} rows, batch {B}")
    elif cu_q_lens.dtype != torch.int32 or tuple(cu_q_lens.shape) != (B + 1,):
        raise ValueError(f"cu_q_lens must be int32 [{B + 1}]")


def _check_out(q, out, out_dtype):
    if out is None:
        return
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    if out.dtype != out_dtype:
        raise ValueError(f"out dtype {out.dtype} differs from out_dtype {out_dtype}")


def check_decode_args(q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens,
                      cu_q_lens=None, out=None, out_dtype=torch.float32):
    """Shapes, dtypes and sizes of a relay_attn_decode call (no device needed; raises
    ValueError).  The C library cannot see tensor extents, so an output or cache too
    small for the dims would be written or read out of bounds: the binding refuses it."""
    _check_context(q, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens)
    _check_system_cache(q, sys_k, sys_v, int(sys_len), ctx_k_pages.shape[1])
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"unsupported out_dtype {out_dtype}")
    _check_out(q, out, out_dtype)


def make_dims(q: torch.Tensor, ctx_k_pages: torch.Tensor, block_tables: torch.Tensor, *,
              scale: float, max_ctx_len: int, max_q_len: int = 1,
              out_dtype: torch.dtype = torch.float32) -> relay_dims:
    """relay_dims from tensor shapes plus the host-known maxima."""
    Tq, Hq, d = q.shape
    if ctx_k_pages.dim() != 5:
        raise ValueError("ctx_k_pages must be key tiles [num_blocks, H_kv, d/G, 16, G]")
    nb, Hkv, nc, bs, g = ctx_k_pages.shape
    if nc * g != d:
        raise ValueError("head_dim mismatch between q and ctx_k_pages")
    B, mb = block_tables.shape
    return relay_dims(B, Hq, Hkv, d, bs, mb, nb, Tq, max_q_len, max_ctx_len, float(scale),
                      _dtype_code(q.dtype), _dtype_code(out_dtype))


def relay_abi_version() -> int:
    return load_library().relay_abi_version()


def relay_workspace_size(dims: relay_dims, sys_len: int) -> int:
    n = load_library().relay_workspace_size(ctypes.byref(dims), sys_len)
    if n == 0:
        lib = load_library()
        msg = lib.relay_last_error().decode()
        if msg:
            raise RelayError(-1, msg)
    return int(n)


def relay_get_plan(dims: relay_dims, sys_len: int) -> dict:
    p = relay_plan()
    _check(load_library().relay_get_plan(ctypes.byref(dims), sys_len, ctypes.byref(p)))
    return p.as_dict()


def workspace(dims: relay_dims, sys_len: int, device) -> torch.Tensor:
    n = max(relay_workspace_size(dims, sys_len), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def relay_attn_decode(q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens,
                      cu_q_lens=None, out=None, *, scale: float, max_ctx_len: int,
                      max_q_len: int = 1, out_dtype=torch.float32, workspace_buf=None,
                      stream=None) -> torch.Tensor:
    """RelayAttention decode step (system + context attention + relay fusion)."""
    _require_device(q, sys_k, sys_v, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens, out)
    check_decode_args(q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens,
                      out, out_dtype)
    dims = make_dims(q, ctx_k_pages, block_tables, scale=scale, max_ctx_len=max_ctx_len,
                     max_q_len=max_q_len, out_dtype=out_dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    ws = workspace_buf if workspace_buf is not None else workspace(dims, sys_len, q.device)
    _check(load_library().relay_attn_decode(
        ctypes.byref(dims), _ptr(q), _ptr(sys_k), _ptr(sys_v), int(sys_len), _ptr(ctx_k_pages),
        _ptr(ctx_v_pages), _ptr(block_tables), _ptr(ctx_lens), _ptr(cu_q_lens), _ptr(out), _ptr(ws),
        ws.numel(), _stream(stream)))
    return out


def relay_attn_decode_noalloc(q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens,
                              cu_q_lens=None, out=None, *, scale: float, max_ctx_len: int,
                              max_q_len: int = 1, out_dtype=torch.float32, stream=None) -> torch.Tensor:
    """relay_attn_decode on the library's static per-device scratch (no workspace
    argument, no device allocation inside the call; ``out`` is allocated here only when
    it is not given).  Calls that overlap on one device race."""
    _require_device(q, sys_k, sys_v, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens, out)
    check_decode_args(q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens,
                      out, out_dtype)
    dims = make_dims(q, ctx_k_pages, block_tables, scale=scale, max_ctx_len=max_ctx_len,
                     max_q_len=max_q_len, out_dtype=out_dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _check(load_library().relay_attn_decode_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(sys_k), _ptr(sys_v), int(sys_len), _ptr(ctx_k_pages),
        _ptr(ctx_v_pages), _ptr(block_tables), _ptr(ctx_lens), _ptr(cu_q_lens), _ptr(out), _stream(stream)))
    return out


def relay_attn_decode_timed(t: dict, out, workspace_buf, events, out_dtype=torch.float32,
                            stream=None):
    """relay_attn_decode on a ``to_device`` dict; ``events`` holds 6 raw hipEvent_t
    handles (ints or None) stamped with the start and end of the system kernel, the
    streaming launch and the merge."""
    _require_device(t["q"], t["sys_k"], t["sys_v"], t["ctx_k_pages"], t["ctx_v_pages"], t["block_tables"],
                    t["ctx_lens"], t["cu_q_lens"], out, workspace_buf)
    check_decode_args(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], t["ctx_k_pages"], t["ctx_v_pages"],
                      t["block_tables"], t["ctx_lens"], t["cu_q_lens"], out, out_dtype)
    dims = dims_of(t, out_dtype)
    ev = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e) if e else None for e in events])
    _check(load_library().relay_attn_decode_timed(
        ctypes.byref(dims), _ptr(t["q"]), _ptr(t["sys_k"]), _ptr(t["sys_v"]), int(t["sys_len"]),
        _ptr(t["ctx_k_pages"]), _ptr(t["ctx_v_pages"]), _ptr(t["block_tables"]), _ptr(t["ctx_lens"]),
        _ptr(t["cu_q_lens"]), _ptr(out), _ptr(workspace_buf), workspace_buf.numel(), _stream(stream), ev))
    return out


def relay_sys_attn(q, sys_k, sys_v, sys_len, dims: relay_dims, *, workspace_buf=None, stream=None):
    """System-attention step alone -> (o_sys float32 [T_q,H_q,d], lse_sys float32 [T_q,H_q])."""
    _require_device(q, sys_k, sys_v)
    if q.dim() != 3 or tuple(q.shape) != (dims.total_q, dims.num_q_heads, dims.head_dim) \
            or _dtype_code(q.dtype) != dims.in_dtype:
        raise ValueError("q does not match dims")
    _check_system_cache(q, sys_k, sys_v, int(sys_len), dims.num_kv_heads)
    o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    ws = workspace_buf if workspace_buf is not None else workspace(dims, sys_len, q.device)
    _check(load_library().relay_sys_attn(ctypes.byref(dims), _ptr(q), _ptr(sys_k), _ptr(sys_v),
                                         int(sys_len), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                         _stream(stream)))
    return o, lse


def prefill_dims(q, sys_k, scale: float, out_dtype=torch.float32) -> relay_dims:
    """relay_dims for relay_prefill_attn: the prompt's L tokens as one request."""
    L, Hq, d = q.shape
    Hkv = sys_k.shape[0]
    nb = -(-L // 16)
    return relay_dims(1, Hq, Hkv, d, 16, nb, nb, L, L, L, float(scale), _dtype_code(q.dtype), _dtype_code(out_dtype))


def prefill_workspace(dims: relay_dims, sys_len: int, device) -> torch.Tensor:
    """A workspace of relay_prefill_workspace_size bytes."""
    lib = load_library()
    n = lib.relay_prefill_workspace_size(ctypes.byref(dims), int(sys_len))
    if n == 0 and lib.relay_last_error():
        raise RelayError(-1, lib.relay_last_error().decode())
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def relay_prefill_attn(q, sys_k, sys_v, sys_len, scale: float, *, out_dtype=torch.float32, with_lse=False,
                       workspace_buf=None, stream=None):
    """Causal attention of the system prompt's tokens over the system cache -> (out, lse or None).

    q [L, H_q, d] (position-embedded); sys_k / sys_v the system cache.  Row (t, h) sees
    system keys 0..t.  Raises RelayError(RELAY_ERR_UNSUPPORTED) off the matrix-core
    path (bf16, head_dim 128, more than 64 rows per KV head)."""
    _require_device(q, sys_k, sys_v)
    dims = prefill_dims(q, sys_k, scale, out_dtype)
    lib = load_library()
    out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if with_lse else None
    if workspace_buf is None:
        workspace_buf = prefill_workspace(dims, sys_len, q.device)
    _check(lib.relay_prefill_attn(ctypes.byref(dims), _ptr(q), _ptr(sys_k), _ptr(sys_v), int(sys_len), _ptr(out),
                                  _dtype_code(out_dtype), _ptr(lse) if lse is not None else None,
                                  _ptr(workspace_buf), workspace_buf.numel(), _stream(stream)))
    return out, lse


def relay_ctx_attn(q, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens, dims: relay_dims,
                   *, workspace_buf=None, stream=None):
    """Context-attention step alone -> (o_ctx, lse_ctx)."""
    _require_device(q, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens)
    _check_context(q, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens)
    o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    ws = workspace_buf if workspace_buf is not None else workspace(dims, 0, q.device)
    _check(load_library().relay_ctx_attn(ctypes.byref(dims), _ptr(q), _ptr(ctx_k_pages),
                                         _ptr(ctx_v_pages), _ptr(block_tables), _ptr(ctx_lens),
                                         _ptr(cu_q_lens), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                         _stream(stream)))
    return o, lse


def relay_fuse(o_sys, lse_sys, o_ctx, lse_ctx, *, out_dtype=torch.float32, with_lse=True,
               stream=None):
    """Relay fusion alone -> (out, lse or None)."""
    _require_device(o_sys, lse_sys, o_ctx, lse_ctx)
    for x in (o_sys, lse_sys, o_ctx, lse_ctx):
        if x.dtype != torch.float32:
            raise ValueError("relay_fuse partials are float32")
    if o_ctx.shape != o_sys.shape or lse_sys.shape != lse_ctx.shape or tuple(o_sys.shape[:-1]) != tuple(lse_sys.shape):
        raise ValueError("o_sys / o_ctx must be [..., d] and lse_sys / lse_ctx the matching [...]")
    d = o_sys.shape[-1]
    n = lse_sys.numel()
    out = torch.empty(o_sys.shape, dtype=out_dtype, device=o_sys.device)
    lse = torch.empty(lse_sys.shape, dtype=torch.float32, device=o_sys.device) if with_lse else None
    _check(load_library().relay_fuse(n, d, _ptr(o_sys), _ptr(lse_sys), _ptr(o_ctx), _ptr(lse_ctx),
                                     _ptr(out), _dtype_code(out_dtype), _ptr(lse), _stream(stream)))
    return out, lse


def relay_validate(dims: relay_dims, block_tables, ctx_lens, cu_q_lens, sys_len: int) -> None:
    """Host-side data check on CPU int32 tensors / numpy arrays; raises RelayError."""
    import numpy as np

    def host(a):
        if a is None:
            return None
        if isinstance(a, torch.Tensor):
            a = a.cpu().numpy()
        return np.ascontiguousarray(a, dtype=np.int32)

    bt, cl, cu = host(block_tables), host(ctx_lens), host(cu_q_lens)
    _check(load_library().relay_validate(
        ctypes.byref(dims), bt.ctypes.data_as(ctypes.c_void_p), cl.ctypes.data_as(ctypes.c_void_p),
        None if cu is None else cu.ctypes.data_as(ctypes.c_void_p), int(sys_len)))


def relay_rope_table(max_pos: int, head_dim: int, base: float = 10000.0, device="cuda", stream=None):
    """The cos/sin table [max_pos, head_dim] float32 the position-embedding entries read."""
    t = torch.empty((max_pos, head_dim), dtype=torch.float32, device=device)
    _require_device(t)
    _check(load_library().relay_rope_table(_ptr(t), int(max_pos), int(head_dim), float(base), _stream(stream)))
    return t


def relay_rope_append(dims: relay_dims, sys_len: int, q_new, k_new, v_new, cos_sin, block_tables, ctx_lens,
                      cu_q_lens, ctx_k_pages, ctx_v_pages, *, q_out=None, stream=None):
    """Position embedding of a decode step's new tokens at sys_len + context position,
    and their K/V appended to the pages (in place).  Returns q_out."""
    if q_out is None:
        q_out = torch.empty_like(q_new)
    _require_device(q_new, k_new, v_new, cos_sin, block_tables, ctx_lens, cu_q_lens, ctx_k_pages, ctx_v_pages, q_out)
    for x in (q_new, k_new, v_new, ctx_k_pages, ctx_v_pages, q_out):
        if x.dtype != q_new.dtype or not x.is_contiguous():
            raise ValueError("q/k/v/pages must be contiguous and of one dtype")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != q_new.shape[-1]:
        raise ValueError("cos_sin must be float32 [max_pos, head_dim]")
    _check(load_library().relay_rope_append(
        ctypes.byref(dims), int(sys_len), _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(cos_sin), cos_sin.shape[0],
        _ptr(block_tables), _ptr(ctx_lens), _ptr(cu_q_lens), _ptr(q_out), _ptr(ctx_k_pages), _ptr(ctx_v_pages),
        _stream(stream)))
    return q_out


class RopeAppendCall:
    """A relay_rope_append call with its arguments checked and marshalled once (as
    ``DecodeCall`` for the decode step): calling it is one ctypes call, so a serving
    loop, or a benchmark, sees the kernel rather than the argument handling."""

    def __init__(self, dims: relay_dims, sys_len: int, q_new, k_new, v_new, cos_sin, block_tables, ctx_lens,
                 cu_q_lens, ctx_k_pages, ctx_v_pages, q_out):
        _require_device(q_new, k_new, v_new, cos_sin, block_tables, ctx_lens, cu_q_lens, ctx_k_pages, ctx_v_pages,
                        q_out)
        for x in (q_new, k_new, v_new, ctx_k_pages, ctx_v_pages, q_out):
            if x.dtype != q_new.dtype or not x.is_contiguous():
                raise ValueError("q/k/v/pages must be contiguous and of one dtype")
        if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != q_new.shape[-1]:
            raise ValueError("cos_sin must be float32 [max_pos, head_dim]")
        self._keep = (dims, q_new, k_new, v_new, cos_sin, block_tables, ctx_lens, cu_q_lens, ctx_k_pages,
                      ctx_v_pages, q_out)
        self._fn = load_library().relay_rope_append
        self._args = (ctypes.byref(dims), int(sys_len), _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(cos_sin),
                      cos_sin.shape[0], _ptr(block_tables), _ptr(ctx_lens), _ptr(cu_q_lens), _ptr(q_out),
                      _ptr(ctx_k_pages), _ptr(ctx_v_pages))
        self.q_out = q_out

    def __call__(self, stream=None):
        rc = self._fn(*self._args, _stream(stream))
        if rc != RELAY_OK:
            _check(rc)
        return self.q_out


def key_tile_shape(lead: tuple, d: int, dtype: torch.dtype) -> tuple:
    """Shape of key tiles: lead + (d/G, 16, G), G the elements of 16 bytes."""
    g = 8 if dtype == torch.bfloat16 else 4
    return (*lead, d // g, 16, g)


def relay_rope_system(sys_k, sys_len: int, cos_sin, *, stream=None):
    """The system keys (key tiles [H_kv, ceil(L_s/16), d/G, 16, G]) rotated in place at
    positions 0 .. sys_len - 1."""
    _require_device(sys_k, cos_sin)
    if not sys_k.is_contiguous() or sys_k.dim() != 5 or sys_k.shape[1] * 16 < sys_len:
        raise ValueError("sys_k must be contiguous key tiles [H_kv, ceil(L_s/16), d/G, 16, G]")
    d = sys_k.shape[2] * sys_k.shape[4]
    _check(load_library().relay_rope_system(sys_k.shape[0], d, int(sys_len), _dtype_code(sys_k.dtype),
                                            _ptr(sys_k), _ptr(cos_sin), cos_sin.shape[0], _stream(stream)))
    return sys_k


def relay_system_fill(k_raw, v_raw, cos_sin, *, sys_k=None, sys_v=None, stream=None):
    """The system cache from token-major k_raw / v_raw [L_s, H_kv, d]: returns
    (sys_k [H_kv, ceil(L_s/16), d/G, 16, G] with RoPE at 0 .. L_s - 1, sys_v
    [H_kv, ceil(L_s/16), d, 16]); the tail tiles' padding keys are 0."""
    L, H_kv, d = k_raw.shape
    if sys_k is None:
        sys_k = torch.empty(key_tile_shape((H_kv, (L + 15) // 16), d, k_raw.dtype), dtype=k_raw.dtype,
                            device=k_raw.device)
    if sys_v is None:
        sys_v = torch.empty((H_kv, (L + 15) // 16, d, 16), dtype=k_raw.dtype, device=k_raw.device)
    _require_device(k_raw, v_raw, cos_sin, sys_k, sys_v)
    if v_raw.shape != k_raw.shape or v_raw.dtype != k_raw.dtype:
        raise ValueError("k_raw and v_raw must have one shape and dtype")
    _check(load_library().relay_system_fill(H_kv, d, L, _dtype_code(k_raw.dtype), _ptr(k_raw), _ptr(v_raw),
                                            _ptr(cos_sin), cos_sin.shape[0], _ptr(sys_k), _ptr(sys_v),
                                            _stream(stream)))
    return sys_k, sys_v


# ---- marshalling of generator workloads -------------------------------------------------


def to_device(w, device="cuda", single_query_null_cu: bool = True) -> dict:
    """Upload a ``workloads.Workload`` to ``device`` in the C-ABI layouts."""
    import numpy as np

    def arr(a):
        if w.spec.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return t.to(device)

    ints = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    multi = int(w.q_lens.max()) > 1
    dt = torch.bfloat16 if w.spec.dtype == "bf16" else torch.float32
    sys_k = arr(w.sys_k) if w.spec.sys_len > 0 else torch.zeros(16, dtype=dt, device=device)
    sys_v = arr(w.sys_v) if w.spec.sys_len > 0 else torch.zeros(16, dtype=dt, device=device)
    return dict(
        q=arr(w.q), sys_k=sys_k, sys_v=sys_v, sys_len=w.spec.sys_len,
        ctx_k_pages=arr(w.ctx_k_pages), ctx_v_pages=arr(w.ctx_v_pages),
        block_tables=ints(w.block_tables), ctx_lens=ints(w.ctx_lens),
        cu_q_lens=ints(w.cu_q_lens) if (multi or not single_query_null_cu) else None,
        scale=w.spec.scale, max_ctx_len=int(w.ctx_lens.max()), max_q_len=int(w.q_lens.max()))


def decode_workload(t: dict, out_dtype=torch.float32, workspace_buf=None, stream=None, out=None):
    """relay_attn_decode on the dict returned by ``to_device``."""
    return relay_attn_decode(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], t["ctx_k_pages"],
                             t["ctx_v_pages"], t["block_tables"], t["ctx_lens"], t["cu_q_lens"], out,
                             scale=t["scale"], max_ctx_len=t["max_ctx_len"], max_q_len=t["max_q_len"],
                             out_dtype=out_dtype, workspace_buf=workspace_buf, stream=stream)


class DecodeCall:
    """A relay_attn_decode call with its arguments marshalled once.

    Checks and converts every argument at construction; calling it is one ctypes
    call (on ``stream``, or on the stream current at call time when stream is None),
    cheap enough that the host keeps ahead of the GPU and usable inside HIP graph
    capture.  The tensors must stay alive and unmoved while the object is used.
    """

    def __init__(self, t: dict, out: torch.Tensor, workspace_buf: torch.Tensor, out_dtype=torch.float32,
                 timed_events=None):
        _require_device(t["q"], t["sys_k"], t["sys_v"], t["ctx_k_pages"], t["ctx_v_pages"],
                        t["block_tables"], t["ctx_lens"], t["cu_q_lens"], out, workspace_buf)
        check_decode_args(t["q"], t["sys_k"], t["sys_v"], t["sys_len"], t["ctx_k_pages"], t["ctx_v_pages"],
                          t["block_tables"], t["ctx_lens"], t["cu_q_lens"], out, out_dtype)
        self.dims = dims_of(t, out_dtype)
        need = relay_workspace_size(self.dims, t["sys_len"])
        if workspace_buf.numel() < need:
            raise ValueError(f"workspace has {workspace_buf.numel()} bytes, needs {need}")
        lib = load_library()
        self._keep = (t, out, workspace_buf)
        self._args = [ctypes.byref(self.dims), _ptr(t["q"]), _ptr(t["sys_k"]), _ptr(t["sys_v"]),
                      int(t["sys_len"]), _ptr(t["ctx_k_pages"]), _ptr(t["ctx_v_pages"]),
                      _ptr(t["block_tables"]), _ptr(t["ctx_lens"]), _ptr(t["cu_q_lens"]), _ptr(out),
                      _ptr(workspace_buf), workspace_buf.numel()]
        self._fn = lib.relay_attn_decode
        self._timed = lib.relay_attn_decode_timed
        self.out = out

    def __call__(self, stream=None):
        rc = self._fn(*self._args, _stream(stream))
        if rc != RELAY_OK:
            _check(rc)
        return self.out

    def timed(self, events, stream=None):
        """The same call; ``events``: 6 raw hipEvent_t handles, start and end of the system
        kernel, the streaming launch and the merge."""
        ev = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e) if e else None for e in events])
        rc = self._timed(*self._args, _stream(stream), ev)
        if rc != RELAY_OK:
            _check(rc)
        return self.out


def dims_of(t: dict, out_dtype=torch.float32) -> relay_dims:
    return make_dims(t["q"], t["ctx_k_pages"], t["block_tables"], scale=t["scale"],
                     max_ctx_len=t["max_ctx_len"], max_q_len=t["max_q_len"], out_dtype=out_dtype)
