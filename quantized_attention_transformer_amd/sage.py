"""Python binding of libsage (include/sage.h): argument marshalling only.

Every computation runs in the HIP library; this module turns torch tensors
(device memory) and torch's current stream into the C ABI's pointers,
strides and stream handle.  It raises if libsage.so is missing or a call
returns a non-OK status.

Tensor layouts accepted: dense "bnhd" [B, N, H, d] (default) or "bhnd"
[B, H, N, d]; packed variable-length [T, H, d] with cu_seqlens (int32,
device).  The channel dimension must be contiguous.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsage.so")
_lib = None

SAGE_PV_FP16 = 0
SAGE_PV_FP8 = 1
SAGE_PV_FP8_SMOOTH_V = 2

EXPORTED = ("sage_workspace_bytes", "sage_quantize_workspace_bytes", "sage_quantize", "sage_quantize_v_fp8",
            "sage_quantize_v_fp8_smooth_workspace_bytes", "sage_quantize_v_fp8_smooth",
            "sage_quantize_smooth_q_workspace_bytes", "sage_quantize_smooth_q",
            "sage_quantize_mxfp4_workspace_bytes", "sage_quantize_mxfp4",
            "sage_attn_quantized", "sage_attn", "sage_attn_noalloc", "sage_debug_qk_i32", "sage_debug_fp8_mfma",
            "sage_debug_mxfp4_mfma", "sage_last_error")


class Strides(ctypes.Structure):
    _fields_ = [("s", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class Problem(ctypes.Structure):
    _fields_ = [("nseq", ctypes.c_int32), ("heads", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("total_tokens", ctypes.c_int64), ("cu_seqlens", ctypes.c_void_p),
                ("blk_q", ctypes.c_int32), ("blk_k", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("smooth_q", ctypes.c_int32), ("qk_fp4", ctypes.c_int32)]


class SageError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """Load libsage.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with quantized_attention_transformer_amd/build_lib.py")
        L = ctypes.CDLL(_LIB_PATH)
        P, S, vp, i32, f32, sz = (ctypes.POINTER(Problem), Strides, ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                  ctypes.c_size_t)
        L.sage_workspace_bytes.argtypes = [P, i32, ctypes.POINTER(sz)]
        L.sage_quantize_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
        L.sage_quantize.argtypes = [P, vp, S, vp, S, f32, vp, S, vp, S, vp, vp, vp, vp, sz, vp]
        L.sage_quantize_smooth_q_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
        L.sage_quantize_smooth_q.argtypes = [P, vp, S, vp, S, f32, vp, S, vp, S, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sage_quantize_mxfp4_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
        L.sage_quantize_mxfp4.argtypes = [P, vp, S, vp, S, f32, vp, S, vp, S, vp, S, vp, S, vp, vp, vp, vp, sz, vp]
        L.sage_quantize_v_fp8.argtypes = [P, vp, S, vp, S, vp, vp]
        L.sage_quantize_v_fp8_smooth_workspace_bytes.argtypes = [P, ctypes.POINTER(sz)]
        L.sage_quantize_v_fp8_smooth.argtypes = [P, vp, S, vp, S, vp, vp, sz, vp]
        L.sage_attn_quantized.argtypes = [P, vp, S, vp, S, vp, vp, vp, S, vp, vp, S, i32, i32, vp]
        L.sage_attn.argtypes = [P, vp, S, vp, S, vp, S, vp, S, i32, f32, i32, vp, sz, vp]
        L.sage_attn_noalloc.argtypes = [P, vp, S, vp, S, vp, S, vp, S, i32, f32, i32, vp]
        L.sage_debug_qk_i32.argtypes = [P, vp, S, vp, S, vp, vp]
        L.sage_debug_fp8_mfma.argtypes = [vp, vp, vp, i32, i32, vp, vp]
        L.sage_debug_mxfp4_mfma.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.sage_last_error.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name != "sage_last_error":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise SageError(fn, rc, lib().sage_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def strides_of(t: torch.Tensor, layout: str) -> Strides:
    if t.stride(-1) != 1:
        raise ValueError("the channel dimension must be contiguous")
    if t.dim() == 3:                          # packed [T, H, d]
        return Strides(0, t.stride(1), t.stride(0))
    if layout == "bnhd":
        return Strides(t.stride(0), t.stride(2), t.stride(1))
    if layout == "bhnd":
        return Strides(t.stride(0), t.stride(1), t.stride(2))
    raise ValueError(f"unknown layout {layout!r}")


def heads_of(t: torch.Tensor, layout: str = "bnhd", packed: bool = False) -> int:
    """Number of heads of a [B, N, H, d] ("bnhd"), [B, H, N, d] ("bhnd") or packed [T, H, d] tensor."""
    if packed:
        return t.shape[1]
    return t.shape[2] if layout == "bnhd" else t.shape[1]


def make_problem(q: torch.Tensor, layout: str = "bnhd", cu_seqlens: Optional[torch.Tensor] = None,
                 max_seqlen: Optional[int] = None, blk_q: int = 128, blk_k: int = 64,
                 k: Optional[torch.Tensor] = None) -> Problem:
    """The sage_problem of q (and, for grouped-query attention, kv_heads from k's head count)."""
    prob = _make_problem(q, layout, cu_seqlens, max_seqlen, blk_q, blk_k)
    if k is not None:
        hk = heads_of(k, layout, cu_seqlens is not None)
        prob.kv_heads = 0 if hk == prob.heads else hk
    return prob


def _make_problem(q, layout, cu_seqlens, max_seqlen, blk_q, blk_k) -> Problem:
    if cu_seqlens is not None:
        if q.dim() != 3:
            raise ValueError("packed inputs are [T, H, d]")
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens (the library never reads cu_seqlens on the host)")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be an int32 device tensor")
        return Problem(cu_seqlens.numel() - 1, q.shape[1], int(max_seqlen), q.shape[2], q.shape[0],
                       cu_seqlens.data_ptr(), blk_q, blk_k)
    if q.dim() != 4:
        raise ValueError("dense inputs are 4-D")
    B = q.shape[0]
    N, H = (q.shape[1], q.shape[2]) if layout == "bnhd" else (q.shape[2], q.shape[1])
    return Problem(B, H, N, q.shape[3], 0, None, blk_q, blk_k)


def workspace_bytes(prob: Problem, pv_mode: int = SAGE_PV_FP16) -> int:
    n = ctypes.c_size_t(0)
    _check("sage_workspace_bytes", lib().sage_workspace_bytes(ctypes.byref(prob), pv_mode, ctypes.byref(n)))
    return n.value


def quantize_workspace_bytes(prob: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check("sage_quantize_workspace_bytes", lib().sage_quantize_workspace_bytes(ctypes.byref(prob), ctypes.byref(n)))
    return n.value


def _nblocks(n, b):
    return (n + b - 1) // b


def quantize(q, k, *, sm_scale: Optional[float] = None, layout="bnhd", cu_seqlens=None, max_seqlen=None,
             blk_q=128, blk_k=64, workspace=None):
    """sage_quantize: returns dict(q8, k8 (int8, the shapes and layout of q and k), q_scale,
    k_scale, k_mean).  k may have fewer heads than q (grouped-query attention)."""
    prob = make_problem(q, layout, cu_seqlens, max_seqlen, blk_q, blk_k, k=k)
    q8 = torch.empty(q.shape, dtype=torch.int8, device=q.device)
    k8 = torch.empty(k.shape, dtype=torch.int8, device=q.device)
    nseq, H, N, d = prob.nseq, prob.heads, prob.max_seqlen, prob.head_dim
    Hk = prob.kv_heads or H
    sq = torch.zeros((nseq, H, _nblocks(N, blk_q)), dtype=torch.float32, device=q.device)
    sk = torch.zeros((nseq, Hk, _nblocks(N, blk_k)), dtype=torch.float32, device=q.device)
    km = torch.zeros((nseq, Hk, d), dtype=torch.float32, device=q.device)
    nws = quantize_workspace_bytes(prob)
    if workspace is None:
        workspace = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    rc = lib().sage_quantize(ctypes.byref(prob), _ptr(q), strides_of(q, layout), _ptr(k), strides_of(k, layout),
                             0.0 if sm_scale is None else float(sm_scale), _ptr(q8), strides_of(q8, layout),
                             _ptr(k8), strides_of(k8, layout), _ptr(sq), _ptr(sk), _ptr(km), _ptr(workspace),
                             workspace.numel(), _stream())
    _check("sage_quantize", rc)
    return dict(q8=q8, k8=k8, q_scale=sq, k_scale=sk, k_mean=km)


def quantize_smooth_q(q, k, *, sm_scale: Optional[float] = None, layout="bnhd", cu_seqlens=None, max_seqlen=None,
                      blk_q=128, blk_k=64):
    """sage_quantize_smooth_q: quantize() with Q smoothed by its mean; returns the same dict
    plus q_mean [nseq, H, d] and q_delta (the per-key compensation; dense [nseq, H, N],
    packed [H, T])."""
    prob = make_problem(q, layout, cu_seqlens, max_seqlen, blk_q, blk_k, k=k)
    prob.smooth_q = 1
    q8 = torch.empty(q.shape, dtype=torch.int8, device=q.device)
    k8 = torch.empty(k.shape, dtype=torch.int8, device=q.device)
    nseq, H, N, d = prob.nseq, prob.heads, prob.max_seqlen, prob.head_dim
    Hk = prob.kv_heads or H
    sq = torch.zeros((nseq, H, _nblocks(N, blk_q)), dtype=torch.float32, device=q.device)
    sk = torch.zeros((nseq, Hk, _nblocks(N, blk_k)), dtype=torch.float32, device=q.device)
    km = torch.zeros((nseq, Hk, d), dtype=torch.float32, device=q.device)
    qm = torch.zeros((nseq, H, d), dtype=torch.float32, device=q.device)
    qdel = torch.zeros((H, prob.total_tokens) if cu_seqlens is not None else (nseq, H, N), dtype=torch.float32,
                       device=q.device)
    n = ctypes.c_size_t(0)
    _check("sage_quantize_smooth_q_workspace_bytes",
           lib().sage_quantize_smooth_q_workspace_bytes(ctypes.byref(prob), ctypes.byref(n)))
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=q.device)
    rc = lib().sage_quantize_smooth_q(ctypes.byref(prob), _ptr(q), strides_of(q, layout), _ptr(k),
                                      strides_of(k, layout), 0.0 if sm_scale is None else float(sm_scale), _ptr(q8),
                                      strides_of(q8, layout), _ptr(k8), strides_of(k8, layout), _ptr(sq), _ptr(sk),
                                      _ptr(km), _ptr(qm), _ptr(qdel), _ptr(ws), ws.numel(), _stream())
    _check("sage_quantize_smooth_q", rc)
    return dict(q8=q8, k8=k8, q_scale=sq, k_scale=sk, k_mean=km, q_mean=qm, q_delta=qdel)


def quantize_mxfp4(q, k, *, sm_scale: Optional[float] = None, layout="bnhd", cu_seqlens=None, max_seqlen=None,
                   smooth_q=False):
    """sage_quantize_mxfp4: 4-bit (MXFP4) Q and K.  Returns dict(q4, k4 (uint8, two E2M1
    codes per byte, the shapes of q and k with d/2 channels), q_scale, k_scale (uint8 E8M0
    codes, d/32 per row), k_mean, and with smooth_q q_mean and q_delta)."""
    prob = make_problem(q, layout, cu_seqlens, max_seqlen, k=k)
    prob.smooth_q = int(bool(smooth_q))
    d = prob.head_dim
    q4 = torch.empty(q.shape[:-1] + (d // 2,), dtype=torch.uint8, device=q.device)
    k4 = torch.empty(k.shape[:-1] + (d // 2,), dtype=torch.uint8, device=q.device)
    qsc = torch.zeros(q.shape[:-1] + (d // 32,), dtype=torch.uint8, device=q.device)
    ksc = torch.zeros(k.shape[:-1] + (d // 32,), dtype=torch.uint8, device=q.device)
    nseq, H, N = prob.nseq, prob.heads, prob.max_seqlen
    Hk = prob.kv_heads or H
    km = torch.zeros((nseq, Hk, d), dtype=torch.float32, device=q.device)
    qm = torch.zeros((nseq, H, d), dtype=torch.float32, device=q.device)
    qdel = torch.zeros((H, prob.total_tokens) if cu_seqlens is not None else (nseq, H, N), dtype=torch.float32,
                       device=q.device)
    n = ctypes.c_size_t(0)
    _check("sage_quantize_mxfp4_workspace_bytes",
           lib().sage_quantize_mxfp4_workspace_bytes(ctypes.byref(prob), ctypes.byref(n)))
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=q.device)
    rc = lib().sage_quantize_mxfp4(ctypes.byref(prob), _ptr(q), strides_of(q, layout), _ptr(k), strides_of(k, layout),
                                   0.0 if sm_scale is None else float(sm_scale), _ptr(q4), strides_of(q4, layout),
                                   _ptr(qsc), strides_of(qsc, layout), _ptr(k4), strides_of(k4, layout), _ptr(ksc),
                                   strides_of(ksc, layout), _ptr(km), _ptr(qm), _ptr(qdel), _ptr(ws), ws.numel(),
                                   _stream())
    _check("sage_quantize_mxfp4", rc)
    out = dict(q4=q4, k4=k4, q_scale=qsc, k_scale=ksc, k_mean=km)
    if smooth_q:
        out.update(q_mean=qm, q_delta=qdel)
    return out


def quantize_v_fp8(v, *, layout="bnhd", cu_seqlens=None, max_seqlen=None, smooth=False):
    """sage_quantize_v_fp8: returns (v8 uint8 E4M3 codes in v's shape, v_scale [nseq, H, d]).
    smooth=True: sage_quantize_v_fp8_smooth, returns (v8 of the smoothed V, v_scale_mean
    [2, nseq, H, d]: the scales, then the means), for pv_mode SAGE_PV_FP8_SMOOTH_V."""
    prob = make_problem(v, layout, cu_seqlens, max_seqlen)
    v8 = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    if smooth:
        n = ctypes.c_size_t(0)
        _check("sage_quantize_v_fp8_smooth_workspace_bytes",
               lib().sage_quantize_v_fp8_smooth_workspace_bytes(ctypes.byref(prob), ctypes.byref(n)))
        ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=v.device)
        svm = torch.zeros((2, prob.nseq, prob.heads, prob.head_dim), dtype=torch.float32, device=v.device)
        rc = lib().sage_quantize_v_fp8_smooth(ctypes.byref(prob), _ptr(v), strides_of(v, layout), _ptr(v8),
                                              strides_of(v8, layout), _ptr(svm), _ptr(ws), ws.numel(), _stream())
        _check("sage_quantize_v_fp8_smooth", rc)
        return v8, svm
    sv = torch.zeros((prob.nseq, prob.heads, prob.head_dim), dtype=torch.float32, device=v.device)
    rc = lib().sage_quantize_v_fp8(ctypes.byref(prob), _ptr(v), strides_of(v, layout), _ptr(v8),
                                   strides_of(v8, layout), _ptr(sv), _stream())
    _check("sage_quantize_v_fp8", rc)
    return v8, sv


def attn_quantized(q8, k8, q_scale, k_scale, v, *, v_scale=None, causal=False, pv_mode=SAGE_PV_FP16,
                   layout="bnhd", cu_seqlens=None, max_seqlen=None, blk_q=128, blk_k=64, out=None):
    """sage_attn_quantized: fused attention over quantised inputs; returns O (fp16, q8's shape).
    k8 and v may have fewer heads than q8 (grouped-query attention)."""
    prob = make_problem(q8, layout, cu_seqlens, max_seqlen, blk_q, blk_k, k=k8)
    if out is None:
        out = torch.empty(q8.shape, dtype=torch.float16, device=q8.device)
    rc = lib().sage_attn_quantized(ctypes.byref(prob), _ptr(q8), strides_of(q8, layout), _ptr(k8),
                                   strides_of(k8, layout), _ptr(q_scale), _ptr(k_scale), _ptr(v),
                                   strides_of(v, layout), _ptr(v_scale), _ptr(out), strides_of(out, layout),
                                   int(bool(causal)), pv_mode, _stream())
    _check("sage_attn_quantized", rc)
    return out


def attn(q, k, v, *, causal=False, sm_scale: Optional[float] = None, pv_mode=SAGE_PV_FP16, layout="bnhd",
         cu_seqlens=None, max_seqlen=None, blk_q=128, blk_k=64, out=None, workspace=None, smooth_q=False,
         qk_fp4=False):
    """sage_attn: the whole forward pass; returns O (fp16, q's shape).  k and v may have
    fewer heads than q (grouped-query attention).  smooth_q: smooth Q as well (blk_k a
    multiple of 64).  qk_fp4: 4-bit (MXFP4) Q and K (head_dim 128 or 96)."""
    prob = make_problem(q, layout, cu_seqlens, max_seqlen, blk_q, blk_k, k=k)
    prob.smooth_q = int(bool(smooth_q))
    prob.qk_fp4 = int(bool(qk_fp4))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float16, device=q.device)
    nws = workspace_bytes(prob, pv_mode)
    if workspace is None:
        workspace = torch.empty(max(nws, 16), dtype=torch.uint8, device=q.device)
    rc = lib().sage_attn(ctypes.byref(prob), _ptr(q), strides_of(q, layout), _ptr(k), strides_of(k, layout),
                         _ptr(v), strides_of(v, layout), _ptr(out), strides_of(out, layout), int(bool(causal)),
                         0.0 if sm_scale is None else float(sm_scale), pv_mode, _ptr(workspace),
                         workspace.numel(), _stream())
    _check("sage_attn", rc)
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # SAGE_NOALLOC_SCRATCH_BYTES


def attn_noalloc(q, k, v, out, *, causal=False, sm_scale: Optional[float] = None, pv_mode=SAGE_PV_FP16,
                 layout="bnhd", cu_seqlens=None, max_seqlen=None, blk_q=128, blk_k=64, smooth_q=False,
                 qk_fp4=False):
    """sage_attn_noalloc: sage_attn with the library's fixed scratch array as its
    workspace (no device allocation by the library; `out` is the caller's).
    Calls on one GPU share the array: they must not overlap."""
    prob = make_problem(q, layout, cu_seqlens, max_seqlen, blk_q, blk_k, k=k)
    prob.smooth_q = int(bool(smooth_q))
    prob.qk_fp4 = int(bool(qk_fp4))
    rc = lib().sage_attn_noalloc(ctypes.byref(prob), _ptr(q), strides_of(q, layout), _ptr(k), strides_of(k, layout),
                                 _ptr(v), strides_of(v, layout), _ptr(out), strides_of(out, layout),
                                 int(bool(causal)), 0.0 if sm_scale is None else float(sm_scale), pv_mode, _stream())
    _check("sage_attn_noalloc", rc)
    return out


def debug_qk_i32(q8, k8, *, layout="bnhd"):
    """sage_debug_qk_i32: INT32 scores [B, H, N, N] from the fused kernel's integer stage
    (k8 may have fewer heads than q8)."""
    prob = make_problem(q8, layout, k=k8)
    s = torch.empty((prob.nseq, prob.heads, prob.max_seqlen, prob.max_seqlen), dtype=torch.int32,
                    device=q8.device)
    rc = lib().sage_debug_qk_i32(ctypes.byref(prob), _ptr(q8), strides_of(q8, layout), _ptr(k8),
                                 strides_of(k8, layout), _ptr(s), _stream())
    _check("sage_debug_qk_i32", rc)
    return s


def attention_ops(seqlens, heads: int, head_dim: int, causal: bool) -> float:
    """Attention operation count used for TOPS: 4 * H * L^2 * d per sequence, halved when causal."""
    tot = sum(4.0 * heads * float(L) * float(L) * head_dim for L in seqlens)
    return tot / 2 if causal else tot


def default_sm_scale(d: int) -> float:
    return float(1.0 / math.sqrt(d))


def debug_fp8_mfma(a8: torch.Tensor, b8: torch.Tensor, c: torch.Tensor, scale_a: int = 127, scale_b: int = 127):
    """sage_debug_fp8_mfma: D = A . B * 2^(scale_a-127) * 2^(scale_b-127) + C on the
    FP8 P.V instruction.  a8 uint8 [32, 64], b8 uint8 [64, 32] (E4M3 codes), c fp32
    [32, 32], all contiguous on the device; returns D fp32 [32, 32]."""
    if a8.shape != (32, 64) or b8.shape != (64, 32) or c.shape != (32, 32):
        raise ValueError("shapes must be A [32, 64], B [64, 32], C [32, 32]")
    if a8.dtype != torch.uint8 or b8.dtype != torch.uint8 or c.dtype != torch.float32:
        raise ValueError("A and B are uint8 E4M3 codes, C is float32")
    a8, b8, c = a8.contiguous(), b8.contiguous(), c.contiguous()
    d = torch.empty((32, 32), dtype=torch.float32, device=c.device)
    _check("sage_debug_fp8_mfma", lib().sage_debug_fp8_mfma(_ptr(a8), _ptr(b8), _ptr(c), int(scale_a), int(scale_b),
                                                           _ptr(d), _stream()))
    return d


def debug_mxfp4_mfma(a4: torch.Tensor, b4: torch.Tensor, sa: torch.Tensor, sb: torch.Tensor, c: torch.Tensor):
    """sage_debug_mxfp4_mfma: D = C + sum_k A[m][k] 2^(sa[m][k/32]-127) B[k][n] 2^(sb[k/32][n]-127)
    on the MXFP4 form of the scaled MFMA.  a4 uint8 [32, 64], b4 uint8 [64, 32] (one E2M1
    code per byte), sa uint8 [32, 2], sb uint8 [2, 32] (E8M0), c fp32 [32, 32]; returns D."""
    if a4.shape != (32, 64) or b4.shape != (64, 32) or sa.shape != (32, 2) or sb.shape != (2, 32) \
            or c.shape != (32, 32):
        raise ValueError("shapes must be A [32, 64], B [64, 32], sa [32, 2], sb [2, 32], C [32, 32]")
    if any(t.dtype != torch.uint8 for t in (a4, b4, sa, sb)) or c.dtype != torch.float32:
        raise ValueError("A, B and the scales are uint8 codes, C is float32")
    a4, b4, sa, sb, c = (t.contiguous() for t in (a4, b4, sa, sb, c))
    d = torch.empty((32, 32), dtype=torch.float32, device=c.device)
    _check("sage_debug_mxfp4_mfma", lib().sage_debug_mxfp4_mfma(_ptr(a4), _ptr(b4), _ptr(sa), _ptr(sb), _ptr(c),
                                                               _ptr(d), _stream()))
    return d


def scaled_dot_product_attention(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
                                 enable_gqa=False, *, pv_mode=SAGE_PV_FP16, blk_q=128, blk_k=64, smooth_q=False,
                                 qk_fp4=False):
    """Drop-in for torch.nn.functional.scaled_dot_product_attention on [B, H, N, d]
    fp16 tensors (the interface the SageAttention pages replace in one line):
    softmax(Q K^T * scale) V through sage_attn, with scale = 1/sqrt(d) when None
    and is_causal masking.  key and value may have fewer heads than query when
    enable_gqa is set (query head h reads K/V head h / (H / H_kv)), as in
    torch's function.  No attn_mask and no dropout (they raise).  Returns O in
    query's shape."""
    if attn_mask is not None:
        raise NotImplementedError("attn_mask is not supported (is_causal is)")
    if dropout_p:
        raise NotImplementedError("dropout is not supported (inference forward pass)")
    if query.dim() != 4 or key.dim() != 4 or value.dim() != 4:
        raise ValueError("query, key and value are [B, H, N, d]")
    hq, hk = query.shape[1], key.shape[1]
    if value.shape[1] != hk:
        raise ValueError("key and value must have the same number of heads")
    if hk != hq and not enable_gqa:
        raise ValueError("key/value with fewer heads than query need enable_gqa=True")
    if hq % hk:
        raise ValueError(f"query heads ({hq}) must be a multiple of key/value heads ({hk})")
    if key.shape[2] != query.shape[2]:
        raise NotImplementedError("self-attention only: query and key have the same length")
    to16 = lambda t: t if (t.dtype == torch.float16 and t.stride(-1) == 1) else t.to(torch.float16).contiguous()  # noqa: E731
    q, k, v = to16(query), to16(key), to16(value)
    return attn(q, k, v, causal=bool(is_causal), sm_scale=None if scale is None else float(scale), pv_mode=pv_mode,
                layout="bhnd", blk_q=blk_q, blk_k=blk_k, smooth_q=smooth_q, qk_fp4=qk_fp4)
