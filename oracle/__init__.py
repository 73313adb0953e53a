"""fp64 CPU oracle for the attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and the
product path has no CPU fallback.

``liboracle.so`` is built from ``fa_oracle.c`` with gcc (see ``build()``);
``brute.py`` is an independent whole-matrix numpy evaluation for tiny shapes.
The definitions each function follows are cited in ``fa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation tests point this at a deliberately broken build of fa_oracle.c.
_LIB_OVERRIDE = os.environ.get("FA_ORACLE_LIB")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile fa_oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("QN", ctypes.c_int64), ("KVN", ctypes.c_int64),
                ("QS", ctypes.c_int64), ("KVS", ctypes.c_int64), ("D", ctypes.c_int64),
                ("layout", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_double),
                ("lens", ctypes.POINTER(ctypes.c_int64)),
                ("mask_mode", ctypes.c_int32),
                ("mask", ctypes.POINTER(ctypes.c_uint8)),
                ("mask_stride", ctypes.c_int64 * 4),
                ("kv_layout", ctypes.c_int32),
                ("block_table", ctypes.POINTER(ctypes.c_int32)),
                ("block_size", ctypes.c_int64), ("max_blocks", ctypes.c_int64),
                ("win_left", ctypes.c_int64), ("win_right", ctypes.c_int64),
                ("cu_q", ctypes.POINTER(ctypes.c_int32)), ("cu_kv", ctypes.POINTER(ctypes.c_int32)),
                ("used_q", ctypes.POINTER(ctypes.c_int32))]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB_OVERRIDE:
                lib = ctypes.CDLL(_LIB_OVERRIDE)
            else:
                if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                    build(force=True)  # missing or older than its source
                lib = ctypes.CDLL(_LIB)
            P = ctypes.POINTER
            u16p, f64p, i64p = P(ctypes.c_uint16), P(ctypes.c_double), P(ctypes.c_int64)
            lib.orc_attention.argtypes = [P(_Problem), u16p, u16p, u16p, ctypes.c_int64, i64p,
                                          f64p, f64p, ctypes.c_int]
            lib.orc_split_partials.argtypes = [P(_Problem), u16p, u16p, u16p, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, i64p,
                                               f64p, f64p, f64p, ctypes.c_int]
            lib.orc_merge.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      f64p, f64p, f64p, f64p, f64p]
            for f in (lib.orc_attention, lib.orc_split_partials, lib.orc_merge):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct)) if a is not None else None


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


class Problem:
    """Shapes and options of one attention-forward call, as the oracle sees them."""

    def __init__(self, B, QN, KVN, QS, KVS, D, layout="BNSD", dtype="bf16", scale=1.0,
                 lens=None, mask_mode="none", mask=None, mask_strides=(0, 0, 0, 0),
                 kv_layout="contiguous", block_table=None, block_size=0, window=(-1, -1),
                 cu_seqlens_q=None, cu_seqlens_kv=None, seqused_q=None):
        self.B, self.QN, self.KVN, self.QS, self.KVS, self.D = B, QN, KVN, QS, KVS, D
        self.layout, self.dtype, self.scale = layout, dtype, float(scale)
        self.lens = None if lens is None else np.ascontiguousarray(lens, dtype=np.int64)
        self.mask_mode = mask_mode
        self.mask = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
        self.mask_strides = tuple(int(s) for s in mask_strides)
        self.kv_layout = kv_layout          # "contiguous", "PA_BBND" or "PA_BNBD"
        self.block_table = (None if block_table is None
                            else np.ascontiguousarray(block_table, dtype=np.int32))
        self.block_size = int(block_size)
        self.window = (int(window[0]), int(window[1]))  # mask_mode "window": (win_left, win_right)
        # layout "TND": QS / KVS are the packed totals Q_T / KV_T; sequence b spans
        # cu_seqlens[b] .. cu_seqlens[b+1].  seqused_q ([B], any layout) truncates
        # each batch's query rows: rows past it keep the initial output (0, +inf).
        i32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.int32)
        self.cu_seqlens_q, self.cu_seqlens_kv = i32(cu_seqlens_q), i32(cu_seqlens_kv)
        self.seqused_q = i32(seqused_q)

    @classmethod
    def from_inputs(cls, inp, mask_mode: Optional[str] = None):
        s = inp.spec
        mode = mask_mode
        if mode is None:
            mode = {"none": "none", "causal": "causal", "bool_causal": "bool"}[s.mask]
        return cls(s.B, s.QN, s.KVN, s.QS, s.KVS, s.D, s.layout, s.dtype, s.softmax_scale,
                   inp.lens, mode, inp.mask if mode == "bool" else None, inp.mask_strides)

    def _c(self):
        p = _Problem()
        p.B, p.QN, p.KVN, p.QS, p.KVS, p.D = self.B, self.QN, self.KVN, self.QS, self.KVS, self.D
        p.layout = {"BNSD": 0, "BSND": 1, "TND": 2}[self.layout]
        p.cu_q = _ptr(self.cu_seqlens_q, ctypes.c_int32)
        p.cu_kv = _ptr(self.cu_seqlens_kv, ctypes.c_int32)
        p.used_q = _ptr(self.seqused_q, ctypes.c_int32)
        p.dtype = 1 if self.dtype == "bf16" else 0
        p.scale = self.scale
        p.lens = _ptr(self.lens, ctypes.c_int64)
        p.mask_mode = {"none": 0, "causal": 1, "bool": 2, "window": 3}[self.mask_mode]
        p.win_left, p.win_right = self.window
        p.mask = _ptr(self.mask, ctypes.c_uint8)
        for i in range(4):
            p.mask_stride[i] = self.mask_strides[i]
        p.kv_layout = {"contiguous": 0, "PA_BBND": 1, "PA_BNBD": 2}[self.kv_layout]
        p.block_table = _ptr(self.block_table, ctypes.c_int32)
        p.block_size = self.block_size
        p.max_blocks = 0 if self.block_table is None else self.block_table.shape[-1]
        return p

    def nrows(self) -> int:
        return self.QN * self.QS if self.layout == "TND" else self.B * self.QN * self.QS


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def attention_rows(prob: Problem, q, k, v, rows=None, threads: Optional[int] = None):
    """fp64 out [nrows, D] and lse [nrows] for the given flat row ids (None = every row)."""
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = prob.nrows() if rows_a is None else rows_a.size
    out = np.empty((n, prob.D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    pc = prob._c()
    rc = lib.orc_attention(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                           _ptr(v, ctypes.c_uint16), n, _ptr(rows_a, ctypes.c_int64),
                           _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double),
                           threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return out, lse


def rows_to_layout(prob: Problem, out_rows, lse_rows):
    """Flat-row results (every row) -> out in the q layout and lse [B, QN, QS] ([Q_T, QN] for TND)."""
    B, QN, QS, D = prob.B, prob.QN, prob.QS, prob.D
    if prob.layout == "TND":
        return np.ascontiguousarray(out_rows.reshape(QS, QN, D)), lse_rows.reshape(QS, QN)
    o = out_rows.reshape(B, QN, QS, D)
    if prob.layout == "BSND":
        o = o.transpose(0, 2, 1, 3)
    return np.ascontiguousarray(o), lse_rows.reshape(B, QN, QS)


def attention(prob: Problem, q, k, v, threads: Optional[int] = None):
    """Every row: out in the q layout (fp64) and lse [B, QN, QS] (fp64)."""
    o, l = attention_rows(prob, q, k, v, None, threads)
    return rows_to_layout(prob, o, l)


def split_partials(prob: Problem, q, k, v, splits: int, chunk: int, rows=None,
                   threads: Optional[int] = None):
    """Per-chunk unnormalised O [nrows, splits, D], m and l [nrows, splits] (fp64)."""
    lib = _load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = prob.nrows() if rows_a is None else rows_a.size
    o = np.empty((n, splits, prob.D), dtype=np.float64)
    m = np.empty((n, splits), dtype=np.float64)
    l = np.empty((n, splits), dtype=np.float64)
    pc = prob._c()
    rc = lib.orc_split_partials(ctypes.byref(pc), _ptr(q, ctypes.c_uint16),
                                _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
                                int(splits), int(chunk), n, _ptr(rows_a, ctypes.c_int64),
                                _ptr(o, ctypes.c_double), _ptr(m, ctypes.c_double),
                                _ptr(l, ctypes.c_double), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return o, m, l


def merge(o_part, m_part, l_part):
    """FD reduction of per-chunk partials -> out [nrows, D], lse [nrows] (fp64)."""
    lib = _load()
    o = np.ascontiguousarray(o_part, dtype=np.float64)
    m = np.ascontiguousarray(m_part, dtype=np.float64)
    l = np.ascontiguousarray(l_part, dtype=np.float64)
    n, splits, D = o.shape
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.orc_merge(n, splits, D, _ptr(o, ctypes.c_double), _ptr(m, ctypes.c_double),
                       _ptr(l, ctypes.c_double), _ptr(out, ctypes.c_double),
                       _ptr(lse, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle merge rejected its input (code {rc})")
    return out, lse


def decode16(bits, dtype: str):
    """Exact fp64 value of 16-bit storage (used by tests to read stored inputs)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)
