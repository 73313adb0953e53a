"""Seeded synthetic inputs for the attention forward workloads.

This module only *generates data*: Gaussian Q/K/V rounded to 16-bit storage,
per-batch KV lengths and boolean masks.  It holds none of the attention
arithmetic, so both sides of a parity check (the fp64 oracle and the HIP
library) can take their inputs from here without sharing any of the method.

Draw order for every workload (fixed so any run can be reproduced from its
seed): ``rng = numpy.random.default_rng(seed)``; Q, then K, then V as
``standard_normal(float32) * std`` rounded to the storage type with
round-to-nearest-even; then the per-batch lengths as inclusive-bound integers.

The shapes, dtypes, scales and length mixes follow the workloads the pages
describe: the FlashAttn operator guide (function description: Q of shape
(Q_S, Q_N, D), K/V of shape (KV_S, KV_N, D), scale usually 1/sqrt(D)), the
aclnnIncreFlashAttention guide (section 1.1: query S fixed at 1 against a
padded KV cache with a real length per batch) and the FlashDecoding tutorial
(preface: B=1, 32 heads, a context of about 100k tokens).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

BNSD = "BNSD"
BSND = "BSND"

_CHUNK = 1 << 24  # elements rounded per pass, bounds temporary memory


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even) and return the raw bits.

    Inputs here are finite Gaussian draws; NaN/Inf are not produced by the
    generators (tests that need NaN padding write the NaN bit pattern directly).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf = x.reshape(-1)
    of = out.reshape(-1)
    for s in range(0, xf.size, _CHUNK):
        u = xf[s:s + _CHUNK].view(np.uint32)
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        of[s:s + _CHUNK] = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (numpy rounds to nearest even) and return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf = x.reshape(-1)
    of = out.reshape(-1)
    for s in range(0, xf.size, _CHUNK):
        of[s:s + _CHUNK] = xf[s:s + _CHUNK].astype(np.float16).view(np.uint16)
    return out


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00}


@dataclass(frozen=True)
class Spec:
    """One attention-forward workload (shapes, storage type, scale, masking, lengths)."""

    name: str
    layout: str            # "BNSD" or "BSND" for q, k, v and out
    B: int
    QN: int
    KVN: int
    QS: int
    KVS: int
    D: int
    dtype: str             # "bf16" or "f16"
    std: float = 1.0
    scale: Optional[float] = None      # None -> 1/sqrt(D)
    mask: str = "none"     # "none", "causal" (mask mode) or "bool_causal" (explicit tensor)
    lens: Optional[tuple] = None       # inclusive (lo, hi) for per-batch KV lengths
    seed: int = 0
    doc: str = ""

    @property
    def g(self) -> int:
        return self.QN // self.KVN

    @property
    def softmax_scale(self) -> float:
        return (1.0 / math.sqrt(self.D)) if self.scale is None else float(self.scale)

    def q_shape(self):
        if self.layout == BNSD:
            return (self.B, self.QN, self.QS, self.D)
        return (self.B, self.QS, self.QN, self.D)

    def kv_shape(self):
        if self.layout == BNSD:
            return (self.B, self.KVN, self.KVS, self.D)
        return (self.B, self.KVS, self.KVN, self.D)

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


# The five workloads, plus the mask-free variant of the causal one, with the
# seeds 1000 + index.
WORKLOADS = {
    "prefill_small": Spec(
        "prefill_small", BNSD, B=1, QN=2, KVN=2, QS=128, KVS=128, D=64, dtype="bf16",
        scale=1.0 / 8.0, seed=1001,
        doc="prefill, BNSD, B=1, N=2, S=128, D=64, bf16 N(0,1), no mask"),
    "decode_gqa": Spec(
        "decode_gqa", BSND, B=8, QN=32, KVN=8, QS=1, KVS=4096, D=128, dtype="bf16",
        lens=(1, 4096), seed=1002,
        doc="incremental decode, BSND, B=8, Q_N=32, KV_N=8, padded KV_S=4096, D=128, "
            "bf16 N(0,1), per-batch lengths U{1..4096}"),
    "decode_128k": Spec(
        "decode_128k", BNSD, B=1, QN=32, KVN=32, QS=1, KVS=131072, D=128, dtype="bf16",
        seed=1003,
        doc="split-KV decode, BNSD, B=1, N=32, KV_S=131072, D=128, bf16 N(0,1)"),
    "prefill_causal": Spec(
        "prefill_causal", BSND, B=2, QN=32, KVN=32, QS=4096, KVS=4096, D=128, dtype="bf16",
        mask="bool_causal", seed=1004,
        doc="causal prefill, BSND, B=2, N=32, S=4096, D=128, bf16 N(0,1), "
            "boolean upper-triangular mask"),
    "prefill_gqa_long": Spec(
        "prefill_gqa_long", BNSD, B=4, QN=64, KVN=8, QS=8192, KVS=8192, D=128, dtype="f16",
        std=0.5, mask="causal", lens=(4096, 8192), seed=1005,
        doc="large GQA causal prefill, BNSD, B=4, Q_N=64, KV_N=8, S=8192, D=128, "
            "fp16 N(0,0.5), per-batch KV lengths U{4096..8192}"),
}
WORKLOADS["prefill_4k"] = WORKLOADS["prefill_causal"].with_(
    name="prefill_4k", mask="none", seed=1004,
    doc="mask-free prefill, BSND, B=2, N=32, S=4096, D=128, bf16 N(0,1)")
# The same flop count with the head dimension of the 256-wide rows of the
# FlashAttn guide's configuration table.
WORKLOADS["prefill_4k_d256"] = WORKLOADS["prefill_4k"].with_(
    name="prefill_4k_d256", QN=16, KVN=16, D=256, seed=1007,
    doc="mask-free prefill, BSND, B=2, N=16, S=4096, D=256, bf16 N(0,1)")


@dataclass
class Inputs:
    spec: Spec
    q: np.ndarray                      # uint16 bits, spec.q_shape()
    k: np.ndarray                      # uint16 bits, spec.kv_shape()
    v: np.ndarray
    lens: Optional[np.ndarray] = None  # int64 [B] or None
    mask: Optional[np.ndarray] = None  # uint8, nonzero = excluded
    mask_strides: tuple = (0, 0, 0, 0)  # element strides for (b, n, i, j); 0 broadcasts
    extra: dict = field(default_factory=dict)


def causal_bool_mask(QS: int, KVS: int) -> np.ndarray:
    """Upper-triangular boolean mask: entry (i, j) is 1 (excluded) when key j > query i."""
    return np.triu(np.ones((QS, KVS), dtype=np.uint8), k=1)


def make(spec: Spec, seed: Optional[int] = None) -> Inputs:
    """Draw the inputs of ``spec`` from ``seed`` (default: the workload's own seed)."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if spec.std != 1.0:
            x *= np.float32(spec.std)
        return round_bits(x, spec.dtype)

    q = draw(spec.q_shape())
    k = draw(spec.kv_shape())
    v = draw(spec.kv_shape())
    lens = None
    if spec.lens is not None:
        lo, hi = spec.lens
        lens = rng.integers(lo, hi, endpoint=True, size=spec.B).astype(np.int64)
    mask = None
    strides = (0, 0, 0, 0)
    if spec.mask == "bool_causal":
        mask = causal_bool_mask(spec.QS, spec.KVS)
        strides = (0, 0, spec.KVS, 1)
    return Inputs(spec, q, k, v, lens, mask, strides)


def fill_padding(inp: Inputs, value_bits: int) -> Inputs:
    """Overwrite every K/V row at or beyond each batch's length with ``value_bits``.

    The padded region of a KV cache may hold anything; the attention result
    must not depend on it.
    """
    s = inp.spec
    if inp.lens is None:
        return inp
    k = inp.k.copy()
    v = inp.v.copy()
    for b in range(s.B):
        L = int(min(max(inp.lens[b], 0), s.KVS))
        if s.layout == BNSD:
            k[b, :, L:, :] = value_bits
            v[b, :, L:, :] = value_bits
        else:
            k[b, L:, :, :] = value_bits
            v[b, L:, :, :] = value_bits
    return Inputs(s, inp.q, k, v, inp.lens, inp.mask, inp.mask_strides, dict(inp.extra))


def sample_rows(spec: Spec, n: int, seed: int = 7, lens: Optional[np.ndarray] = None) -> np.ndarray:
    """A seeded sample of flat query-row ids r = (b*QN + n1)*QS + i.

    Always contains, for every batch: the first and last query position, the
    positions around that batch's length (L-1, L) and one full 128-row block.
    """
    rng = np.random.default_rng(seed)
    B, QN, QS = spec.B, spec.QN, spec.QS
    picks = set()
    for b in range(B):
        L = spec.KVS if lens is None else int(min(max(lens[b], 0), spec.KVS))
        n1 = int(rng.integers(0, QN))
        base = (b * QN + n1) * QS
        for i in (0, QS - 1, L - 1, L, min(QS - 1, 127)):
            if 0 <= i < QS:
                picks.add(base + i)
        blk = int(rng.integers(0, max(1, QS // 128))) * 128
        for i in range(blk, min(QS, blk + 128)):
            picks.add(base + i)
    total = B * QN * QS
    extra = rng.integers(0, total, size=max(0, n - len(picks)))
    picks.update(int(x) for x in extra)
    return np.array(sorted(picks), dtype=np.int64)


def to_paged(inp: Inputs, block_size: int, kv_layout: str = "PA_BBND", seed: int = 0,
             spare_blocks: int = 3):
    """Store the K/V cache of ``inp`` as a paged cache (FlashAttn developer guide 1.2).

    Token j of batch b goes to row j % block_size of physical block
    block_table[b][j // block_size]; physical blocks are a seeded permutation
    with ``spare_blocks`` unused ones filled with NaN (they must never be read).
    PA_BBND blocks are [block_size][KV_N][D]; PA_BNBD blocks [KV_N][block_size][D].
    Returns (k_paged, v_paged, block_table int32 [B, max_blocks], num_blocks).
    """
    s = inp.spec
    max_blocks = -(-s.KVS // block_size)
    nb = s.B * max_blocks + spare_blocks
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)
    table = perm[: s.B * max_blocks].reshape(s.B, max_blocks).astype(np.int32)
    nan = NAN_BITS[s.dtype]
    out = []
    for x in (inp.k, inp.v):
        xb = x if s.layout == BNSD else x.transpose(0, 2, 1, 3)  # -> [B, KVN, KVS, D]
        pad = np.full((s.B, s.KVN, max_blocks * block_size, s.D), nan, np.uint16)
        pad[:, :, : s.KVS] = xb
        blocks = pad.reshape(s.B, s.KVN, max_blocks, block_size, s.D)
        if kv_layout == "PA_BBND":
            phys = np.full((nb, block_size, s.KVN, s.D), nan, np.uint16)
            src = blocks.transpose(0, 2, 3, 1, 4)                      # [B, blk, bs, KVN, D]
        else:
            phys = np.full((nb, s.KVN, block_size, s.D), nan, np.uint16)
            src = blocks.transpose(0, 2, 1, 3, 4)                      # [B, blk, KVN, bs, D]
        phys[table.reshape(-1)] = src.reshape((s.B * max_blocks,) + phys.shape[1:])
        out.append(np.ascontiguousarray(phys))
    return out[0], out[1], table, nb


@dataclass
class PackedInputs:
    """Packed variable-length (TND) inputs: sequences laid end to end."""
    q: np.ndarray                 # uint16 [Q_T, QN, D]
    k: np.ndarray                 # uint16 [KV_T, KVN, D]
    v: np.ndarray
    cu_q: np.ndarray              # int32 [B + 1]
    cu_kv: np.ndarray             # int32 [B + 1]
    q_lens: np.ndarray            # int64 [B]
    kv_lens: np.ndarray           # int64 [B]
    QN: int
    KVN: int
    D: int
    dtype: str
    scale: float


def make_packed(B: int, QN: int, KVN: int, D: int, dtype: str = "bf16", q_lens=(1, 512),
                kv_lens=None, std: float = 1.0, scale: Optional[float] = None,
                seed: int = 0) -> PackedInputs:
    """Seeded TND inputs (FlashAttn developer guide 1.3, Packed Sequence).

    Draw order: rng = default_rng(seed); the B query lengths as inclusive
    integers in q_lens; the B KV lengths likewise in kv_lens (None: equal to the
    query lengths, self-attention prefill); then Q, K, V as standard_normal *
    std rounded to the storage type.
    """
    rng = np.random.default_rng(seed)
    ql = rng.integers(q_lens[0], q_lens[1], endpoint=True, size=B).astype(np.int64)
    kl = ql.copy() if kv_lens is None else rng.integers(kv_lens[0], kv_lens[1], endpoint=True,
                                                         size=B).astype(np.int64)
    cu_q = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    cu_kv = np.concatenate([[0], np.cumsum(kl)]).astype(np.int32)

    def draw(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return round_bits(x, dtype)

    q = draw((int(cu_q[-1]), QN, D))
    k = draw((int(cu_kv[-1]), KVN, D))
    v = draw((int(cu_kv[-1]), KVN, D))
    sc = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    return PackedInputs(q, k, v, cu_q, cu_kv, ql, kl, QN, KVN, D, dtype, sc)


# Ragged self-attention prefill in the packed layout: 16 sequences of 256..8192
# tokens, GQA 32/8, causal (the length mix of the ragged long-prefill workload,
# without the padding).
PACKED_WORKLOADS = {
    "prefill_varlen": dict(B=16, QN=32, KVN=8, D=128, dtype="bf16", q_lens=(256, 8192), seed=1006),
}
