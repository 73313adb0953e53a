"""Python binding of the gfx950 attention-forward library (include/fa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa_mi355x.so``.  The low-level functions carry the C names
(``fa_fwd``, ``fa_fwd_noalloc``, ``fa_workspace_size``, ``fa_splitkv_plan``,
``fa_decode_splitkv``, ``fa_decode_fused``, ``fa_combine``, ``fa_last_error``) and take device pointers as ints or torch
tensors; ``fwd`` is a convenience wrapper that allocates the outputs and the
workspace with torch on the current stream.  There is no CPU fallback: if the
shared library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")

FA_OK, FA_ERR_NULLPTR, FA_ERR_PARAM_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_RUNTIME = range(5)
FA_BNSD, FA_BSND, FA_TND = 0, 1, 2
LAYOUTS = {"BNSD": FA_BNSD, "BSND": FA_BSND, "TND": FA_TND}
FA_F16, FA_BF16 = 0, 1
FA_MASK_NONE, FA_MASK_CAUSAL, FA_MASK_BOOL, FA_MASK_WINDOW = 0, 1, 2, 3
MASK_MODES = {"none": FA_MASK_NONE, "causal": FA_MASK_CAUSAL, "bool": FA_MASK_BOOL,
              "window": FA_MASK_WINDOW}
FA_KV_CONTIGUOUS, FA_KV_PAGED_BBND, FA_KV_PAGED_BNBD = 0, 1, 2
KV_LAYOUTS = {"contiguous": FA_KV_CONTIGUOUS, "PA_BBND": FA_KV_PAGED_BBND, "PA_BNBD": FA_KV_PAGED_BNBD}

EXPORTS = ("fa_workspace_size", "fa_fwd", "fa_fwd_noalloc", "fa_splitkv_plan", "fa_decode_fused_plan",
           "fa_decode_splitkv", "fa_decode_fused", "fa_combine", "fa_describe", "fa_last_error")


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fa status {status}: {message}")
        self.status = status


class FaParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("num_heads", ctypes.c_int64),
                ("num_kv_heads", ctypes.c_int64), ("q_seq", ctypes.c_int64),
                ("kv_seq", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("layout", ctypes.c_int), ("dtype", ctypes.c_int), ("scale", ctypes.c_double),
                ("actual_seq_lengths", ctypes.c_void_p), ("mask_mode", ctypes.c_int),
                ("mask", ctypes.c_void_p), ("mask_stride", ctypes.c_int64 * 4),
                ("kv_layout", ctypes.c_int), ("block_table", ctypes.c_void_p),
                ("block_size", ctypes.c_int64), ("max_blocks_per_seq", ctypes.c_int64),
                ("num_blocks", ctypes.c_int64), ("win_left", ctypes.c_int64),
                ("win_right", ctypes.c_int64), ("cu_seqlens_q", ctypes.c_void_p),
                ("cu_seqlens_kv", ctypes.c_void_p), ("seqused_q", ctypes.c_void_p)]


_lock = threading.Lock()
_lib = None


def load(path: Optional[str] = None):
    """Load (once) and return the ctypes handle of the HIP library."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or LIB_PATH
            if not os.path.exists(p):
                raise RuntimeError(f"HIP library {p} is not built; run __graft_entry__.build() "
                                   "(there is no CPU fallback)")
            lib = ctypes.CDLL(p)
            P = ctypes.POINTER
            vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
            lib.fa_workspace_size.argtypes = [P(FaParams), P(sz)]
            lib.fa_fwd.argtypes = [P(FaParams), vp, vp, vp, vp, vp, vp, sz, vp]
            lib.fa_fwd_noalloc.argtypes = [P(FaParams), vp, vp, vp, vp, vp, vp]
            lib.fa_splitkv_plan.argtypes = [P(FaParams), ctypes.c_int, i64, P(i64), P(i64), P(sz)]
            lib.fa_decode_fused_plan.argtypes = [P(FaParams), ctypes.c_int, P(i64), P(i64), P(sz)]
            lib.fa_decode_splitkv.argtypes = [P(FaParams), i64, i64, vp, vp, vp, vp, vp, vp, vp]
            lib.fa_combine.argtypes = [P(FaParams), i64, vp, vp, vp, vp, vp, vp]
            lib.fa_decode_fused.argtypes = [P(FaParams), i64, i64, vp, vp, vp, vp, sz, vp, vp, vp]
            lib.fa_describe.argtypes = [P(FaParams), ctypes.c_char_p, sz]
            for f in (lib.fa_workspace_size, lib.fa_fwd, lib.fa_fwd_noalloc, lib.fa_splitkv_plan,
                      lib.fa_decode_fused_plan, lib.fa_decode_splitkv, lib.fa_combine, lib.fa_decode_fused,
                      lib.fa_describe):
                f.restype = ctypes.c_int
            lib.fa_last_error.argtypes = []
            lib.fa_last_error.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream  # torch.cuda.Stream -> hipStream_t


def fa_last_error() -> str:
    return load().fa_last_error().decode()


def _check(st: int):
    if st != FA_OK:
        raise FaError(st, fa_last_error())


def make_params(batch, num_heads, q_seq, kv_seq, head_dim, *, num_kv_heads=0, layout="BNSD",
                dtype="bf16", scale=1.0, actual_seq_lengths=None, mask_mode="none", mask=None,
                mask_stride: Sequence[int] = (0, 0, 0, 0), kv_layout="contiguous", block_table=None,
                block_size=0, max_blocks_per_seq=0, num_blocks=0, win_left=-1,
                win_right=-1, cu_seqlens_q=None, cu_seqlens_kv=None, seqused_q=None) -> FaParams:
    p = FaParams()
    p.batch, p.num_heads, p.num_kv_heads = batch, num_heads, num_kv_heads
    p.q_seq, p.kv_seq, p.head_dim = q_seq, kv_seq, head_dim
    p.layout = LAYOUTS[layout] if isinstance(layout, str) else layout
    p.cu_seqlens_q, p.cu_seqlens_kv = _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv)
    p.seqused_q = _ptr(seqused_q)
    p.dtype = {"f16": FA_F16, "bf16": FA_BF16}[dtype] if isinstance(dtype, str) else dtype
    p.scale = float(scale)
    p.actual_seq_lengths = _ptr(actual_seq_lengths)
    p.mask_mode = MASK_MODES[mask_mode] if isinstance(mask_mode, str) else mask_mode
    p.win_left, p.win_right = int(win_left), int(win_right)
    p.mask = _ptr(mask)
    for i in range(4):
        p.mask_stride[i] = int(mask_stride[i])
    p.kv_layout = KV_LAYOUTS[kv_layout] if isinstance(kv_layout, str) else kv_layout
    p.block_table = _ptr(block_table)
    p.block_size, p.max_blocks_per_seq, p.num_blocks = block_size, max_blocks_per_seq, num_blocks
    # The struct holds raw device addresses: keep the objects they came from
    # alive as long as the struct, so a temporary tensor passed here is not
    # freed (and its memory handed to the next allocation) before the call.
    p._keep = (actual_seq_lengths, mask, block_table, cu_seqlens_q, cu_seqlens_kv, seqused_q)
    return p


def fa_describe(params: FaParams) -> str:
    """The line fa_fwd would log (FA_LOG=1) for these parameters: path, kernels, plan."""
    buf = ctypes.create_string_buffer(1024)
    _check(load().fa_describe(ctypes.byref(params), buf, len(buf)))
    return buf.value.decode()


def fa_workspace_size(params: FaParams) -> int:
    n = ctypes.c_size_t(0)
    _check(load().fa_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def fa_fwd(params: FaParams, q, k, v, out, lse=None, workspace=None, workspace_bytes=0, stream=None):
    _check(load().fa_fwd(ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                         _ptr(workspace), int(workspace_bytes), _stream(stream)))


def fa_fwd_noalloc(params: FaParams, q, k, v, out, lse=None, stream=None):
    _check(load().fa_fwd_noalloc(ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _stream(stream)))


def fa_splitkv_plan(params: FaParams, num_cus: int = 0, chunk_hint: int = 0):
    sp, ch, ws = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_size_t(0)
    _check(load().fa_splitkv_plan(ctypes.byref(params), int(num_cus), int(chunk_hint),
                                  ctypes.byref(sp), ctypes.byref(ch), ctypes.byref(ws)))
    return sp.value, ch.value, ws.value


def fa_decode_fused_plan(params: FaParams, num_cus: int = 0):
    sp, ch, ws = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_size_t(0)
    _check(load().fa_decode_fused_plan(ctypes.byref(params), int(num_cus), ctypes.byref(sp), ctypes.byref(ch),
                                       ctypes.byref(ws)))
    return sp.value, ch.value, ws.value


def fa_decode_splitkv(params: FaParams, num_splits, chunk, q, k, v, o_part, m_part, l_part,
                      stream=None):
    _check(load().fa_decode_splitkv(ctypes.byref(params), int(num_splits), int(chunk), _ptr(q),
                                    _ptr(k), _ptr(v), _ptr(o_part), _ptr(m_part), _ptr(l_part),
                                    _stream(stream)))


def fa_decode_fused(params: FaParams, num_splits, chunk, q, k, v, workspace, workspace_bytes, out,
                    lse=None, stream=None):
    _check(load().fa_decode_fused(ctypes.byref(params), int(num_splits), int(chunk), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(workspace), int(workspace_bytes), _ptr(out), _ptr(lse),
                                  _stream(stream)))


def fa_combine(params: FaParams, num_splits, o_part, m_part, l_part, out, lse=None, stream=None):
    _check(load().fa_combine(ctypes.byref(params), int(num_splits), _ptr(o_part), _ptr(m_part),
                             _ptr(l_part), _ptr(out), _ptr(lse), _stream(stream)))


# ----------------------------------------------------------------- torch conveniences

def params_for(q, k, *, layout="BNSD", num_kv_heads=0, scale=1.0, actual_seq_lengths=None,
               mask=None, mask_stride=(0, 0, 0, 0), causal=False, kv_layout="contiguous",
               block_table=None, window=None, cu_seqlens_q=None, cu_seqlens_kv=None,
               seqused_q=None) -> FaParams:
    """FaParams from torch tensors q, k in ``layout`` (shapes as in include/fa.h).

    With a paged ``kv_layout`` k is [num_blocks, block_size, KV_N, D] (PA_BBND) or
    [num_blocks, KV_N, block_size, D] (PA_BNBD), block_table is int32
    [B, max_blocks_per_seq], and kv_seq is max_blocks_per_seq * block_size.
    ``window=(win_left, win_right)`` selects the window mask (-1 = unbounded side).
    With ``layout="TND"`` q is [Q_T, N, D], k is [KV_T, KV_N, D] and the int32
    cu_seqlens_q / cu_seqlens_kv ([B + 1]) and seqused_q ([B]) are device tensors.
    """
    import torch
    extra = dict(seqused_q=seqused_q) if seqused_q is not None else {}
    if layout == "TND":
        QS, N, D = q.shape
        B = cu_seqlens_q.shape[0] - 1
        extra = dict(cu_seqlens_q=cu_seqlens_q, cu_seqlens_kv=cu_seqlens_kv, seqused_q=seqused_q)
    elif layout == "BNSD":
        B, N, QS, D = q.shape
    else:
        B, QS, N, D = q.shape
    if layout == "TND":
        KVS, KVN = k.shape[0], k.shape[1]
    elif kv_layout == "contiguous":
        KVN, KVS = (k.shape[1], k.shape[2]) if layout == "BNSD" else (k.shape[2], k.shape[1])
    else:
        nb, bs, KVN = ((k.shape[0], k.shape[1], k.shape[2]) if kv_layout == "PA_BBND"
                       else (k.shape[0], k.shape[2], k.shape[1]))
        KVS = block_table.shape[1] * bs
        extra.update(kv_layout=kv_layout, block_table=block_table, block_size=bs,
                     max_blocks_per_seq=block_table.shape[1], num_blocks=nb)
    dtype = {torch.bfloat16: "bf16", torch.float16: "f16"}[q.dtype]
    mode = "bool" if mask is not None else ("causal" if causal else "none")
    if window is not None:
        mode = "window"
        extra.update(win_left=window[0], win_right=window[1])
    return make_params(B, N, QS, KVS, D, num_kv_heads=num_kv_heads or KVN, layout=layout,
                       dtype=dtype, scale=scale, actual_seq_lengths=actual_seq_lengths,
                       mask_mode=mode, mask=mask, mask_stride=mask_stride, **extra)


def fwd(q, k, v, *, layout="BNSD", scale=1.0, actual_seq_lengths=None, mask=None,
        mask_stride=(0, 0, 0, 0), causal=False, return_lse=False, stream=None,
        kv_layout="contiguous", block_table=None, window=None, cu_seqlens_q=None,
        cu_seqlens_kv=None, seqused_q=None):
    """Attention forward on device tensors; allocates out (and lse, workspace) with torch.
    scale defaults to 1.0, the default of the softmax scale in the attention
    formula of the FlashAttn developer guide's introduction; pass 1/sqrt(D) for
    the usual attention scale."""
    import torch
    p = params_for(q, k, layout=layout, scale=scale, actual_seq_lengths=actual_seq_lengths,
                   mask=mask, mask_stride=mask_stride, causal=causal, kv_layout=kv_layout,
                   block_table=block_table, window=window, cu_seqlens_q=cu_seqlens_q,
                   cu_seqlens_kv=cu_seqlens_kv, seqused_q=seqused_q)
    out = torch.empty_like(q)
    lse_shape = (p.q_seq, p.num_heads) if layout == "TND" else (p.batch, p.num_heads, p.q_seq)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device) if return_lse else None
    nbytes = fa_workspace_size(p)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=q.device) if nbytes else None
    s = stream if stream is not None else torch.cuda.current_stream()
    if ws is not None and isinstance(s, torch.cuda.Stream):
        ws.record_stream(s)
    fa_fwd(p, q, k, v, out, lse, ws, nbytes, s)
    return (out, lse) if return_lse else out
