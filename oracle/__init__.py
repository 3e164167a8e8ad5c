"""fp64 CPU oracle for RelayAttention decode attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``shared_prompt_kv_amd``) never imports it, and it imports nothing from the
product: the two share only the seeded input generator, which holds no attention
arithmetic.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows, built -O2
without fast-math).  This wrapper only marshals numpy arrays.  What each function
computes, and the passage of the RelayAttention pages it follows, is documented
in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("sys_len", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("q", ctypes.c_void_p),
        ("sys_k", ctypes.c_void_p),
        ("sys_v", ctypes.c_void_p),
        ("ctx_k", ctypes.c_void_p),
        ("ctx_v", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("ctx_lens", ctypes.c_void_p),
        ("cu_q_lens", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str):
    """Load an oracle build from ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = load_library(_LIB_PATH)
    return _lib


def _declare(lib):
    P = ctypes.POINTER(_Problem)
    dp = ctypes.c_void_p
    for name in ("oracle_attention", "oracle_system_part", "oracle_context_part"):
        f = getattr(lib, name)
        f.argtypes = [P, dp, ctypes.c_long, dp, dp]
        f.restype = ctypes.c_int
    lib.oracle_attention_range.argtypes = [P, ctypes.c_long, ctypes.c_long, dp, ctypes.c_long, dp, dp]
    lib.oracle_attention_range.restype = ctypes.c_int
    lib.oracle_relay_fuse.argtypes = [ctypes.c_long, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_relay_fuse.restype = None
    lib.oracle_merge.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_int, dp, dp, dp, dp]
    lib.oracle_merge.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Problem:
    """Holds a workload's arrays (kept alive) and the C struct that points at them."""

    def __init__(self, w, scale: Optional[float] = None, lib=None):
        spec = w.spec
        self.w = w
        self.lib = lib
        self._keep = [np.ascontiguousarray(a) for a in (
            w.q, w.sys_k, w.sys_v, w.ctx_k_pages, w.ctx_v_pages)]
        self._ints = [np.ascontiguousarray(a, dtype=np.int32) for a in (
            w.block_tables, w.ctx_lens, w.cu_q_lens)]
        self.num_q_heads = spec.num_q_heads
        self.head_dim = spec.head_dim
        self.total_q = int(w.cu_q_lens[-1])
        self.c = _Problem(
            BF16 if spec.dtype == "bf16" else F32,
            spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
            int(w.block_tables.shape[1]), spec.sys_len,
            float(spec.scale if scale is None else scale),
            *[a.ctypes.data for a in self._keep], *[a.ctypes.data for a in self._ints])

    def _call(self, fn, rows, *extra):
        lib = self.lib or _load()
        if rows is None:
            n = self.total_q * self.num_q_heads
            rows_arr = None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            n = len(rows_arr)
        out = np.zeros((n, self.head_dim), np.float64)
        lse = np.zeros(n, np.float64)
        rc = getattr(lib, fn)(ctypes.byref(self.c), *extra, _ptr(rows_arr), n, _ptr(out), _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"{fn} failed with {rc}")
        return out, lse

    def _shape(self, out, lse, rows):
        if rows is None:
            return (out.reshape(self.total_q, self.num_q_heads, self.head_dim),
                    lse.reshape(self.total_q, self.num_q_heads))
        return out, lse

    def attention(self, rows=None):
        """Exact causal attention over [system; context]: (out, lse)."""
        return self._shape(*self._call("oracle_attention", rows), rows)

    def system_part(self, rows=None):
        """System-attention step output (O_s, LSE_s)."""
        return self._shape(*self._call("oracle_system_part", rows), rows)

    def context_part(self, rows=None):
        """Context-attention step output (O_c, LSE_c)."""
        return self._shape(*self._call("oracle_context_part", rows), rows)

    def attention_range(self, lo: int, hi: int, rows=None):
        """Attention over keys [lo, hi) of each row's concatenated visible sequence."""
        return self._shape(*self._call("oracle_attention_range", rows, lo, hi), rows)

    def relay(self, rows=None):
        """The three relay steps on the oracle: system part, context part, fusion."""
        o_s, l_s = self.system_part(rows)
        o_c, l_c = self.context_part(rows)
        out, lse, _ = relay_fuse(o_s, l_s, o_c, l_c, lib=self.lib)
        return out, lse


def relay_fuse(o_s, lse_s, o_c, lse_c, lib=None):
    """Relay fusion (convex combination by LSE).  Returns (out, lse, alpha[...,2])."""
    o_s = np.ascontiguousarray(o_s, np.float64)
    o_c = np.ascontiguousarray(o_c, np.float64)
    lse_s = np.ascontiguousarray(lse_s, np.float64)
    lse_c = np.ascontiguousarray(lse_c, np.float64)
    d = o_s.shape[-1]
    n = lse_s.size
    out = np.zeros_like(o_s)
    lse = np.zeros_like(lse_s)
    alpha = np.zeros(lse_s.shape + (2,), np.float64)
    (lib or _load()).oracle_relay_fuse(n, d, _ptr(o_s), _ptr(lse_s), _ptr(o_c), _ptr(lse_c), _ptr(out),
                              _ptr(lse), _ptr(alpha))
    return out, lse, alpha


def merge(os_: Sequence[np.ndarray], lses: Sequence[np.ndarray], lib=None):
    """k-way LSE merge of partial results over disjoint key sets."""
    o = np.ascontiguousarray(np.stack([np.asarray(x, np.float64) for x in os_]))
    l = np.ascontiguousarray(np.stack([np.asarray(x, np.float64) for x in lses]))
    k = o.shape[0]
    d = o.shape[-1]
    n = l[0].size
    out = np.zeros(o.shape[1:], np.float64)
    lse = np.zeros(l.shape[1:], np.float64)
    (lib or _load()).oracle_merge(k, n, d, _ptr(o), _ptr(l), _ptr(out), _ptr(lse))
    return out, lse


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the following oracle calls (timing only: results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))
