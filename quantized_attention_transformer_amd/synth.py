"""Seeded synthetic attention inputs (shared by the oracle tests, the GPU parity
tests and the benchmark).

This module draws random fp16 tensors and nothing else: it holds none of the
attention method's arithmetic (no mean, no quantisation, no softmax), so the
CPU oracle and the HIP path can both consume its output without sharing any
of the computation under test.

Workloads stand in for the models the SageAttention pages measure on
(text LLMs, video diffusion transformers, long context); no dataset or model
weight is used.  Each workload fixes shapes and value distributions:

* Q, V ~ N(0, 1); K ~ N(0, 1) plus a per-(sequence, head, channel) bias that
  is shared by every token of that sequence and head.  The bias gives K the
  channel-wise outliers that smoothing K is meant to remove (SageAttention
  article, "技术方案", first item, smoothing K).
* The video-DiT workload puts a N(0, 8^2) bias on 4 randomly chosen channels
  per (batch, head) and N(0, 1) on the rest.
* The varlen workload packs 8 sequences whose lengths are uniform integers in
  [512, 8192], redrawn (whole draw) until their sum is at most 40 960.

Draw order for one workload: (varlen lengths), Q, K noise, K bias (outlier
channel choice first when there is one), V.  Samples are drawn in float32 by
numpy's PCG64 generator and rounded to fp16 (round-to-nearest-even).
Tensors are returned in the packed token-major layout [T, H, d] for varlen
and [B, N, H, d] for dense problems.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    heads: int
    head_dim: int
    batch: int = 1             # dense batch (ignored when varlen)
    seqlen: int = 0            # dense sequence length
    varlen_nseq: int = 0       # >0: packed variable-length sequences
    varlen_min: int = 512
    varlen_max: int = 8192
    varlen_total_max: int = 40960
    bias_std: float = 1.0      # std of the per-channel K bias
    outlier_channels: int = 0  # >0: bias only on this many channels (std bias_std), N(0,1) elsewhere
    causal: bool = False
    blk_q: int = 128
    blk_k: int = 64
    pv_fp8: bool = False

    @property
    def is_varlen(self) -> bool:
        return self.varlen_nseq > 0


# The workloads, in the order the method's benchmark list states them.
TINY = Workload("tiny B1 H2 N256 d64", 1001, heads=2, head_dim=64, batch=1, seqlen=256,
                bias_std=5.0, blk_q=64, blk_k=64)
TEXT = Workload("text B1 H8 N4096 d128", 1002, heads=8, head_dim=128, batch=1, seqlen=4096,
                bias_std=2.0, blk_q=128, blk_k=64)
TEXT_CAUSAL = dataclasses.replace(TEXT, name="text causal B1 H8 N4096 d128", causal=True)
VIDEO = Workload("video B2 H24 N16384 d64", 1003, heads=24, head_dim=64, batch=2, seqlen=16384,
                 bias_std=8.0, outlier_channels=4, blk_q=128, blk_k=64)
VARLEN = Workload("varlen H32 d128 8 seqs <=40960 tok", 1004, heads=32, head_dim=128,
                  varlen_nseq=8, bias_std=3.0, causal=True, blk_q=128, blk_k=64)
LONG = Workload("long causal B1 H32 N32768 d128", 1014, heads=32, head_dim=128, batch=1,
                seqlen=32768, bias_std=3.0, causal=True, blk_q=128, blk_k=64)
FP8 = Workload("fp8-PV B4 H16 N8192 d128", 1005, heads=16, head_dim=128, batch=4, seqlen=8192,
               bias_std=4.0, blk_q=128, blk_k=64, pv_fp8=True)

ALL = [TINY, TEXT, TEXT_CAUSAL, VIDEO, VARLEN, LONG, FP8]


@dataclasses.dataclass
class Inputs:
    wl: Workload
    q: np.ndarray            # fp16, [B, N, H, d] dense or [T, H, d] varlen
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: Optional[np.ndarray]  # int32 [nseq+1] (varlen) else None
    seqlens: np.ndarray      # int64 [nseq]

    @property
    def nseq(self) -> int:
        return len(self.seqlens)

    @property
    def max_seqlen(self) -> int:
        return int(self.seqlens.max()) if len(self.seqlens) else 0

    def digest(self) -> dict:
        return {n: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
                for n, a in (("q", self.q), ("k", self.k), ("v", self.v))}


def draw_varlen_lengths(rng: np.random.Generator, n: int, lo: int, hi: int, total_max: int) -> np.ndarray:
    """Lengths uniform in [lo, hi] (inclusive); the whole draw is repeated until the sum fits."""
    while True:
        lens = rng.integers(lo, hi, size=n, endpoint=True)
        if lens.sum() <= total_max:
            return lens.astype(np.int64)


def _normal16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x.astype(np.float16)


def generate(wl: Workload, seed: Optional[int] = None, *, seqlens=None, seqlen: Optional[int] = None,
             batch: Optional[int] = None, heads: Optional[int] = None) -> Inputs:
    """Draw one workload's Q, K, V.  Keyword overrides shrink a workload while
    keeping its distributions (used for small parity cases)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    H = wl.heads if heads is None else heads
    d = wl.head_dim
    if wl.is_varlen or seqlens is not None:
        if seqlens is None:
            seqlens = draw_varlen_lengths(rng, wl.varlen_nseq, wl.varlen_min, wl.varlen_max,
                                          wl.varlen_total_max)
        seqlens = np.asarray(seqlens, dtype=np.int64)
        T = int(seqlens.sum())
        cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(seqlens)
        tok_shape = (T, H, d)
        nseq = len(seqlens)
    else:
        B = wl.batch if batch is None else batch
        N = wl.seqlen if seqlen is None else seqlen
        seqlens = np.full(B, N, dtype=np.int64)
        cu = None
        tok_shape = (B, N, H, d)
        nseq = B

    q = _normal16(rng, tok_shape)
    knoise = rng.standard_normal(size=tok_shape, dtype=np.float32)
    if wl.outlier_channels:
        bias = rng.standard_normal(size=(nseq, H, d), dtype=np.float32)
        for s in range(nseq):
            for h in range(H):
                ch = rng.choice(d, size=wl.outlier_channels, replace=False)
                bias[s, h, ch] *= np.float32(wl.bias_std)
    else:
        bias = rng.standard_normal(size=(nseq, H, d), dtype=np.float32) * np.float32(wl.bias_std)
    if cu is None:
        knoise += bias[:, None, :, :]
    else:
        for s in range(nseq):
            knoise[cu[s]:cu[s + 1]] += bias[s][None, :, :]
    k = knoise.astype(np.float16)
    del knoise
    v = _normal16(rng, tok_shape)
    return Inputs(wl, q, k, v, cu, seqlens)


def per_sequence(x: np.ndarray, inp: Inputs, s: int) -> np.ndarray:
    """View of sequence s as [L, H, d] (token-major), for either layout."""
    if inp.cu_seqlens is None:
        return x[s]
    return x[inp.cu_seqlens[s]:inp.cu_seqlens[s + 1]]
