"""CPU oracle for SageAttention's 8-bit attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library (no kernels, headers, tables or helpers); the only thing both
sides consume is the seeded input generator, which holds none of the method's
arithmetic.

What is computed, and where the pages state it
----------------------------------------------
Pages cited (by title):

[SA]   "SageAttention：低比特量化Attention，实现推理加速" (xinfinite.net repost of
       the 机器之心 article on SageAttention).  Section "技术方案" (technical
       approach) has three items: (1) smoothing K, (2) per-block INT8
       quantisation of Q and K, (3) an FP16 accumulator for P·V.
[SA2]  "4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级"
       (17aitech.com).  Section "即插即用举例" (input Q, K, V, get O);
       section "技术方案" item (4): P and V quantised to FP8 E4M3.
[ABS]  "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
       Acceleration" (ai-search.io), abstract.
[GUIDE] "如何将SageAttention量化注意力机制集成到你的AI项目中获得2-5倍速度提升"
       (maplevalley.com.cn), section "针对不同AI任务的优化建议", causal mode and
       the variable-length (varlen) kernels.

Steps, in the pages' order:
 1. mean(K) per channel, taken over the tokens of one (sequence, head)
    ([SA] 技术方案 item 1).  Sum exactly in fp64, one fp64 divide, round to
    fp32.  Every fp16 value is a multiple of 2^-24, so while the running
    |sum| stays below 2^29 every partial sum is exact and the result does not
    depend on summation order.
 2. K_s = fp32(K) - mean(K), rounded to fp32 ([SA] 技术方案 item 1).
 3. Q' = fp32(Q) * sm_scale rounded to fp32 (the softmax scale is folded into
    Q before quantisation; default sm_scale = fp32(1/sqrt(d))).
 4. Per block of rows of one (sequence, head) -- the block is the tile size of
    the fused attention kernel ([SA] 技术方案 item 2): a = max|x|; scale =
    fp32(a / 127) (IEEE division); code = clamp(round_half_even(fp32(x /
    scale)), -127, 127); an all-zero block gets scale 0 and codes 0.
 5. S_int = q8 . k8^T exactly ([SA] 技术方案 item 2: INT8 product with an INT32
    accumulator).
 6. S = S_int * sq[row block] * sk[key block] in fp64; keys of other
    sequences are excluded; causal keeps key j <= query i.
 7. Softmax in fp64 (plain two-pass; the fused kernel's online softmax is an
    exact reformulation of it).
 8. fp16 P.V path: O = P V / l in fp64 ([SA] 技术方案 item 3 states that the
    FP16 accumulator loses no accuracy, so the oracle's fp16-path result is
    the exact product).
 8'. FP8 P.V path ([SA2] 技术方案 item 4): V per (sequence, head, channel)
    scale sv = fp32(max|V| / 448), v8 = E4M3(fp32(V / sv)); P (in (0, 1],
    taken relative to the row maximum rounded up to a power of two, see
    fp8_probs) is encoded as E4M3(p * 448); O = sum_j dec(p8) dec(v8) * sv /
    448 / l with l from the unquantised p.  E4M3 is the OCP format (bias 7, max 448, no
    infinities), round-to-nearest-even, saturating at 448.

Smooth Q ([SA2] 技术方案 item 1, optional here as on the page's INT8
kernel): mean(Q') per channel over the tokens of the sequence (the same
reading as mean(K)), taken from the exact fp64 sum of the fp16 Q as
fp32((sum / L) * sm_scale); Q_s = fp32(Q' - mean(Q')) is quantised in place
of Q'; the product of mean(Q') with K_s^T, one value per key (delta_j =
mean(Q') . K_s[j] in fp64), is added to every row of S in step 6, which
makes S equal to Q' K_s^T again up to quantisation.

4-bit Q and K ([SA2] 技术方案, its INT4 kernel): gfx950 has no INT4 matrix
instruction; its 4-bit one takes OCP MXFP4, so the 4-bit variant here
quantises Q' (or Q_s) and the smoothed K to MXFP4 instead: per row, per block
of 32 channels, one power-of-two scale 2^e with e = floor(log2(max|x|)) - 2
(E2M1's largest power of two is 2^2; E8M0 code e + 127, clamped to [-127,
127]; an all-zero block gets code 0), and elements E2M1(x / 2^e), round to
nearest even, saturating at 6.  S is then exact from the codes: sum over the
blocks of 2^(eq + ek) times the E2M1 dot product (mx_* functions).

K and V may have fewer heads than Q (grouped-query attention, which the
scaled-dot-product-attention interface the pages' drop-in replaces accepts):
query head h reads K/V head h // (Hq / Hk), and K's mean is per K head.

Readings of points the pages leave open are listed with the design notes
(mean over tokens per channel; fp32 smoothed K fed to the quantiser; IEEE
division rather than a reciprocal multiply; symmetric [-127, 127]; scale 0 for
an all-zero block; the mean of a causal or varlen sequence taken over the
whole sequence; the FP8 scale of P fixed at 448 with P taken relative to
the row maximum rounded up to a power of two).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

LOG2E = math.log2(math.e)


# --------------------------------------------------------------------------
# step 1-4: smoothing and block quantisation
# --------------------------------------------------------------------------

def default_sm_scale(d: int) -> np.float32:
    """Softmax scale 1/sqrt(d) (the scaled-dot-product-attention convention
    the pages' drop-in interface replaces; [SA] "即插即用举例"), computed in
    fp64 and rounded once to fp32."""
    return np.float32(1.0 / math.sqrt(d))


def k_mean(k_seq: np.ndarray) -> np.ndarray:
    """mean(K) over the tokens of one sequence, per channel ([SA] 技术方案,
    smoothing K).  k_seq: fp16 [L, d].  Exact fp64 sum, fp64 divide by L,
    one rounding to fp32."""
    L = k_seq.shape[0]
    if L == 0:
        return np.zeros(k_seq.shape[1], np.float32)
    s = np.sum(k_seq.astype(np.float64), axis=0)
    return (s / np.float64(L)).astype(np.float32)


def smooth_k(k_seq: np.ndarray, km: np.ndarray) -> np.ndarray:
    """K - mean(K) in fp32 ([SA] 技术方案, smoothing K)."""
    return k_seq.astype(np.float32) - km.astype(np.float32)[None, :]


def fold_sm_scale(q_seq: np.ndarray, sm_scale) -> np.ndarray:
    """Q' = fp32(Q) * sm_scale, one fp32 rounding."""
    return q_seq.astype(np.float32) * np.float32(sm_scale)


def q_mean(q_seq: np.ndarray, sm_scale) -> np.ndarray:
    """mean(Q') over the tokens of one sequence, per channel, for smoothing Q
    ([SA2] 技术方案 item 1).  q_seq: fp16 [L, d].  Exact fp64 sum of the fp16
    values, then fp32((sum / L) * sm_scale) with fp64 operations (mean(Q * s)
    = mean(Q) * s, taken so that the sum stays exact)."""
    L = q_seq.shape[0]
    if L == 0:
        return np.zeros(q_seq.shape[1], np.float32)
    s = np.sum(q_seq.astype(np.float64), axis=0)
    return ((s / np.float64(L)) * np.float64(np.float32(sm_scale))).astype(np.float32)


def smooth_q_values(q_fold: np.ndarray, qm: np.ndarray) -> np.ndarray:
    """Q_s = fp32(Q' - mean(Q')) for Q' = fold_sm_scale(Q) ([SA2] 技术方案 item 1)."""
    return (q_fold.astype(np.float32) - qm.astype(np.float32)[None, :]).astype(np.float32)


def q_delta(qm: np.ndarray, k_s: np.ndarray) -> np.ndarray:
    """The compensation of smoothing Q: mean(Q') . K_s^T, one value per key
    ([SA2] 技术方案 item 1: a vector-matrix product added to S).  fp64 [L]."""
    return k_s.astype(np.float64) @ qm.astype(np.float64)


def quant_block(x: np.ndarray):
    """INT8 quantisation of one block with one scale ([SA] 技术方案, per-block
    INT8 quantisation of Q and K).  x: fp32 [rows, d].  Returns (int8 codes,
    fp32 scale)."""
    a = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if a == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    scale = np.float32(a / np.float32(127))          # IEEE binary32 division
    r = np.rint((x / scale).astype(np.float32))      # fp32 quotient, ties to even
    return np.clip(r, -127, 127).astype(np.int8), scale


def quant_rows(x: np.ndarray, blk: int):
    """Blocks of `blk` rows starting at the sequence's first token; the last
    block holds the remaining rows.  x: fp32 [L, d] -> (int8 [L, d], fp32
    [ceil(L/blk)]).  blk = 1 is one scale per token, the finest of the
    granularities finer than per-block that [SA2] 技术方案 item 2 argues for."""
    L = x.shape[0]
    nb = -(-L // blk)
    codes = np.zeros(x.shape, np.int8)
    scales = np.zeros(nb, np.float32)
    for b in range(nb):
        sl = slice(b * blk, min((b + 1) * blk, L))
        codes[sl], scales[b] = quant_block(x[sl])
    return codes, scales


def _seq_views(x: np.ndarray, cu: Optional[np.ndarray], nseq: int):
    """Per-sequence [L, H, d] views of a [B, N, H, d] or packed [T, H, d] array."""
    if cu is None:
        return [x[s] for s in range(nseq)]
    return [x[cu[s]:cu[s + 1]] for s in range(nseq)]


def quantize_qk(q: np.ndarray, k: np.ndarray, seqlens: Sequence[int], cu: Optional[np.ndarray],
                blk_q: int, blk_k: int, sm_scale=None, smooth: bool = True, smooth_q: bool = False):
    """Steps 1-4 for every (sequence, head).

    q, k: fp16 in [B, N, H, d] (dense, cu None) or [T, H, d] (packed, cu int32
    prefix offsets); k may have fewer heads Hk than q (grouped-query
    attention: Hq a multiple of Hk).  Returns a dict with q8, k8 (int8, same
    layout as the input), sq [nseq, Hq, ceil(maxL/blk_q)], sk [nseq, Hk,
    ceil(maxL/blk_k)] (entries past a sequence's last block are 0) and km
    [nseq, Hk, d] fp32 (the mean is per K head).  smooth=False is the ablation
    without mean subtraction (km is then 0).  smooth_q: Q is smoothed too;
    adds qm [nseq, Hq, d] fp32 (mean(Q')) and qdelta [nseq, Hq, maxL] fp64
    (mean(Q') . K_s^T per key; 0 past a sequence's end), and q8/sq are those
    of Q_s."""
    nseq = len(seqlens)
    H, d = q.shape[-2], q.shape[-1]
    Hk = k.shape[-2]
    maxL = int(max(seqlens)) if nseq else 0
    sm = default_sm_scale(d) if sm_scale is None else np.float32(sm_scale)
    q8 = np.zeros(q.shape, np.int8)
    k8 = np.zeros(k.shape, np.int8)
    sq = np.zeros((nseq, H, -(-maxL // blk_q)), np.float32)
    sk = np.zeros((nseq, Hk, -(-maxL // blk_k)), np.float32)
    km = np.zeros((nseq, Hk, d), np.float32)
    qm = np.zeros((nseq, H, d), np.float32)
    qdel = np.zeros((nseq, H, maxL), np.float64)
    grp = H // Hk
    qv, kv = _seq_views(q, cu, nseq), _seq_views(k, cu, nseq)
    q8v, k8v = _seq_views(q8, cu, nseq), _seq_views(k8, cu, nseq)
    for s in range(nseq):
        L = int(seqlens[s])
        k_s = []
        for h in range(Hk):
            kh = kv[s][:L, h, :]
            if smooth:
                km[s, h] = k_mean(kh)
                ks = smooth_k(kh, km[s, h])
            else:
                ks = kh.astype(np.float32)
            k_s.append(ks)
            c, sc = quant_rows(ks, blk_k)
            k8v[s][:L, h, :] = c
            sk[s, h, :len(sc)] = sc
        for h in range(H):
            qf = fold_sm_scale(qv[s][:L, h, :], sm)
            if smooth_q:
                qm[s, h] = q_mean(qv[s][:L, h, :], sm)
                qf = smooth_q_values(qf, qm[s, h])
                qdel[s, h, :L] = q_delta(qm[s, h], k_s[h // grp])
            c, sc = quant_rows(qf, blk_q)
            q8v[s][:L, h, :] = c
            sq[s, h, :len(sc)] = sc
    out = dict(q8=q8, k8=k8, sq=sq, sk=sk, km=km, sm_scale=sm)
    if smooth_q:
        out.update(qm=qm, qdelta=qdel)
    return out


# --------------------------------------------------------------------------
# step 5: integer scores
# --------------------------------------------------------------------------

def scores_int(q8_rows: np.ndarray, k8_rows: np.ndarray) -> np.ndarray:
    """S_int = q8 . k8^T, exact ([SA] 技术方案, INT8 matmul with INT32
    accumulator).  Uses an fp64 matrix product: every product is an integer
    of magnitude <= 127^2 and every partial sum of a d <= 256 contraction is
    below 2^22, far inside fp64's 2^53 exact-integer range, so the result is
    exact whatever order the library sums in.  Returns int64."""
    assert q8_rows.shape[-1] <= 256
    return np.rint(q8_rows.astype(np.float64) @ k8_rows.astype(np.float64).T).astype(np.int64)


# --------------------------------------------------------------------------
# FP8 E4M3 (OCP) encoder, written from the format's definition
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code (sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 is subnormal; 0x7F/0xFF are NaN)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_POS = np.array([e4m3_value(c) for c in range(0x7F)], np.float64)   # codes 0..126, increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    table = np.array([e4m3_value(c) for c in range(256)], np.float64)
    return table[np.asarray(codes, np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to nearest OCP E4M3 value, ties to the even code, saturating at
    448 and never producing NaN; the sign is kept (so -0 and negative values
    that round to zero give 0x80)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1      # largest code with value <= a
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= 448.0, 126, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quant_v_fp8_seq(v_seq: np.ndarray, smooth: bool = False):
    """V of one (sequence, head) -> (e4m3 codes [L, d], fp32 scale [d], fp32
    mean [d]).  Without smoothing: scale = fp32(max_n |V| / 448) per channel
    ([SA2] 技术方案 item 4), codes = E4M3(fp32(V / scale)), mean 0.  With
    smoothing (the optional smooth-V step described after 技术方案 on the same
    page): mean = mean(V) over the tokens per channel (exact, as for K), V' =
    fp32(V - mean), then the same scale and codes on V'.  A channel that is
    all zero (after smoothing: constant) gets scale 0 and codes 0."""
    vf = v_seq.astype(np.float32)
    vm = k_mean(v_seq) if smooth else np.zeros(vf.shape[1], np.float32)
    if smooth:
        vf = (vf - vm[None, :]).astype(np.float32)
    a = np.max(np.abs(vf), axis=0) if vf.shape[0] else np.zeros(vf.shape[1], np.float32)
    sv = (a / np.float32(448)).astype(np.float32)
    safe = np.where(sv == 0, np.float32(1), sv)
    r = (vf / safe[None, :]).astype(np.float32)
    codes = e4m3_encode(r)
    codes[:, sv == 0] = 0
    return codes, sv, vm


def quant_v_fp8(v: np.ndarray, seqlens, cu, smooth: bool = False):
    """quant_v_fp8_seq for every (sequence, head); returns codes in V's layout,
    scales [nseq, H, d] and means [nseq, H, d] (zero without smoothing)."""
    nseq = len(seqlens)
    H, d = v.shape[-2], v.shape[-1]
    v8 = np.zeros(v.shape, np.uint8)
    sv = np.zeros((nseq, H, d), np.float32)
    vm = np.zeros((nseq, H, d), np.float32)
    vv, v8v = _seq_views(v, cu, nseq), _seq_views(v8, cu, nseq)
    for s in range(nseq):
        L = int(seqlens[s])
        for h in range(H):
            v8v[s][:L, h, :], sv[s, h], vm[s, h] = quant_v_fp8_seq(vv[s][:L, h, :], smooth)
    return v8, sv, vm


# --------------------------------------------------------------------------
# 4-bit Q and K: OCP MXFP4 (E2M1 elements, one E8M0 scale per 32 channels of a row)
# --------------------------------------------------------------------------

MX_BLOCK = 32


def e2m1_value(code: int) -> float:
    """Value of an E2M1 code (bit 3 sign, bits 2-1 exponent with bias 1, bit 0
    mantissa; exponent 0 is subnormal: 0 or 0.5).  Magnitudes: 0, 0.5, 1, 1.5,
    2, 3, 4, 6."""
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return sign * mag


_E2M1_POS = np.array([e2m1_value(c) for c in range(8)], np.float64)   # codes 0..7, increasing


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    table = np.array([e2m1_value(c) for c in range(16)], np.float64)
    return table[np.asarray(codes, np.uint8) & 0xF]


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E2M1 value, ties to the even code, saturating at 6;
    the sign bit is the input's (so negative values that round to 0 give 0x8)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    lo = np.clip(np.searchsorted(_E2M1_POS, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    dlo = a - _E2M1_POS[lo]
    dhi = _E2M1_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(a >= 6.0, 7, np.where(pick_hi, hi, lo))
    return (code | np.where(np.signbit(x), 0x8, 0)).astype(np.uint8)


def mx_scale_code(amax: float) -> int:
    """E8M0 code of a block whose largest magnitude is amax: 127 + floor(log2
    amax) - 2, clamped to [0, 254]; 0 for an all-zero block."""
    if amax == 0:
        return 0
    k = math.frexp(float(amax))[1] - 1          # floor(log2 amax), exact
    return int(min(254, max(0, 127 + k - 2)))


def mx_quant_rows(x: np.ndarray):
    """MXFP4 of every row of x (fp32 [L, d], d a multiple of 32): returns
    (E2M1 codes uint8 [L, d], one per element; E8M0 scale codes uint8
    [L, d/32])."""
    L, d = x.shape
    xb = np.asarray(x, np.float64).reshape(L, d // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    sc = np.array([[mx_scale_code(a) for a in row] for row in amax], np.uint8).reshape(L, d // MX_BLOCK)
    codes = e2m1_encode(xb / np.exp2(sc.astype(np.float64) - 127.0)[:, :, None])
    codes[np.broadcast_to((amax == 0)[:, :, None], codes.shape)] = 0
    return codes.reshape(L, d), sc


def mx_dequant(codes: np.ndarray, sc: np.ndarray) -> np.ndarray:
    """Values of MXFP4 rows (fp64 [L, d])."""
    L, d = codes.shape
    v = e2m1_decode(codes).reshape(L, d // MX_BLOCK, MX_BLOCK)
    return (v * np.exp2(sc.astype(np.float64) - 127.0)[:, :, None]).reshape(L, d)


def quantize_qk_fp4(q: np.ndarray, k: np.ndarray, seqlens: Sequence[int], cu: Optional[np.ndarray],
                    sm_scale=None, smooth_q: bool = False):
    """The 4-bit variant of quantize_qk: Q' (or, smooth_q, Q_s) and the smoothed
    K quantised to MXFP4.  Returns q4, k4 (E2M1 codes, one per element, in the
    inputs' layouts), qsc [nseq, Hq, maxL, d/32] and ksc [nseq, Hk, maxL, d/32]
    (E8M0 codes, 0 past a sequence's end), km, and with smooth_q qm and qdelta
    as in quantize_qk."""
    nseq = len(seqlens)
    H, d = q.shape[-2], q.shape[-1]
    Hk = k.shape[-2]
    grp = H // Hk
    maxL = int(max(seqlens)) if nseq else 0
    sm = default_sm_scale(d) if sm_scale is None else np.float32(sm_scale)
    q4 = np.zeros(q.shape, np.uint8)
    k4 = np.zeros(k.shape, np.uint8)
    qsc = np.zeros((nseq, H, maxL, d // MX_BLOCK), np.uint8)
    ksc = np.zeros((nseq, Hk, maxL, d // MX_BLOCK), np.uint8)
    km = np.zeros((nseq, Hk, d), np.float32)
    qm = np.zeros((nseq, H, d), np.float32)
    qdel = np.zeros((nseq, H, maxL), np.float64)
    qv, kv = _seq_views(q, cu, nseq), _seq_views(k, cu, nseq)
    q4v, k4v = _seq_views(q4, cu, nseq), _seq_views(k4, cu, nseq)
    for s in range(nseq):
        L = int(seqlens[s])
        k_s = []
        for h in range(Hk):
            km[s, h] = k_mean(kv[s][:L, h, :])
            ks = smooth_k(kv[s][:L, h, :], km[s, h])
            k_s.append(ks)
            k4v[s][:L, h, :], ksc[s, h, :L] = mx_quant_rows(ks)
        for h in range(H):
            qf = fold_sm_scale(qv[s][:L, h, :], sm)
            if smooth_q:
                qm[s, h] = q_mean(qv[s][:L, h, :], sm)
                qf = smooth_q_values(qf, qm[s, h])
                qdel[s, h, :L] = q_delta(qm[s, h], k_s[h // grp])
            q4v[s][:L, h, :], qsc[s, h, :L] = mx_quant_rows(qf)
    out = dict(q4=q4, k4=k4, qsc=qsc, ksc=ksc, km=km, sm_scale=sm)
    if smooth_q:
        out.update(qm=qm, qdelta=qdel)
    return out


def scores_fp4(q4h, qsch, k4h, ksch) -> np.ndarray:
    """S = (MXFP4 Q) (MXFP4 K)^T in fp64 for one (sequence, head): every product
    of two E2M1 values times two powers of two is exact."""
    return mx_dequant(q4h, qsch) @ mx_dequant(k4h, ksch).T


# --------------------------------------------------------------------------
# steps 6-8: dequantise, mask, softmax, P.V
# --------------------------------------------------------------------------

def fp8_probs(S):
    """Unnormalised probabilities for the FP8 P.V path.  The pages fix P's
    FP8 scale as one constant for values in [0, 1] ([SA2] 技术方案 item 4)
    but not the maximum P is taken relative to; here it is the row maximum
    in base-2 units rounded up to an integer, m2 = ceil(max_j S_ij log2 e),
    and p = 2^(S log2 e - m2) lies in (0, 1].  With that choice the E4M3 code
    of a weight does not depend on the order keys are visited in (a
    power-of-two shift of the reference commutes with E4M3 rounding away
    from its subnormal range).  Returns (p, l = sum p)."""
    x = S * LOG2E
    m2 = np.ceil(np.max(x, axis=1, keepdims=True))
    P = np.exp2(x - m2)
    return P, np.sum(P, axis=1, keepdims=True)


def attention_head(q8h, k8h, sqh, skh, vh, blk_q, blk_k, causal, rows=None,
                   pv_fp8=False, v8h=None, svh=None, return_lse=False, vmh=None, qdel=None, fp4=None):
    """One (sequence, head).  q8h, k8h: int8 [L, d]; sqh, skh: per-block scales;
    vh: fp16 [L, d]; rows: query indices to compute (default all); FP8 path:
    v8h, svh and, with smooth V, vmh (the mean added back to O: every row of
    P sums to 1, so P V = P (V - mean) + mean); smooth Q: qdel [L], the
    per-key compensation mean(Q') . K_s^T added to every row of S; 4-bit Q and
    K: fp4 = (q4h, qsch, k4h, ksch) in place of q8h ... skh (S from scores_fp4).
    Returns O fp64 [len(rows), d]."""
    L = vh.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    if len(rows) == 0 or L == 0:
        return np.zeros((len(rows), vh.shape[1]), np.float64)
    if fp4 is not None:
        q4h, qsch, k4h, ksch = fp4
        S = scores_fp4(q4h[rows], qsch[rows], k4h, ksch)
    else:
        s_int = scores_int(q8h[rows], k8h)                           # step 5
        rs = sqh[rows // blk_q].astype(np.float64)
        cs = skh[np.arange(L) // blk_k].astype(np.float64)
        S = s_int.astype(np.float64) * rs[:, None] * cs[None, :]     # step 6
    if qdel is not None:
        S = S + np.asarray(qdel, np.float64)[None, :L]
    if causal:
        S = np.where(np.arange(L)[None, :] <= rows[:, None], S, -np.inf)
    m = np.max(S, axis=1, keepdims=True)                             # step 7
    P = np.exp(S - m)
    l = np.sum(P, axis=1, keepdims=True)
    if not pv_fp8:                                                   # step 8
        O = (P @ vh.astype(np.float64)) / l
    else:                                                            # step 8'
        P, l = fp8_probs(S)
        p8 = e4m3_decode(e4m3_encode(P * 448.0))
        vd = e4m3_decode(v8h)
        O = (p8 @ vd) * (svh.astype(np.float64)[None, :] / 448.0) / l
        if vmh is not None:
            O = O + vmh.astype(np.float64)[None, :]
    if return_lse:
        return O, (m[:, 0] + np.log(l[:, 0]))
    return O


def sage_attn(q, k, v, seqlens, cu, causal, blk_q, blk_k, sm_scale=None, pv_fp8=False,
              rows_by_seq=None, smooth=True, quant=None, smooth_v=False, smooth_q=False, qk_fp4=False):
    """The whole forward pass.  Layouts as in quantize_qk.  rows_by_seq
    optionally maps a sequence index to the query rows to compute (the rest
    of O is left NaN).  smooth_v (FP8 path): subtract mean(V) before the E4M3
    quantisation and add it to O.  smooth_q: smooth Q as well (quantize_qk).
    qk_fp4: 4-bit (MXFP4) Q and K (quantize_qk_fp4; blk_q and blk_k unused).
    Returns (O fp64 in Q's layout, quantisation dict)."""
    nseq = len(seqlens)
    H = q.shape[-2]
    grp = H // k.shape[-2]  # query heads per K/V head (grouped-query attention)
    if quant is not None:
        qd = quant
    elif qk_fp4:
        qd = quantize_qk_fp4(q, k, seqlens, cu, sm_scale, smooth_q=smooth_q)
    else:
        qd = quantize_qk(q, k, seqlens, cu, blk_q, blk_k, sm_scale, smooth=smooth, smooth_q=smooth_q)
    if pv_fp8:
        v8, sv, vm = quant_v_fp8(v, seqlens, cu, smooth_v)
        qd = dict(qd, v8=v8, sv=sv, vm=vm)
    O = np.full(q.shape, np.nan, np.float64)
    ov = _seq_views(O, cu, nseq)
    fp4 = "q4" in qd
    q8v, k8v = (_seq_views(qd[a], cu, nseq) for a in (("q4", "k4") if fp4 else ("q8", "k8")))
    vv = _seq_views(v, cu, nseq)
    v8v = _seq_views(qd["v8"], cu, nseq) if pv_fp8 else None
    for s in range(nseq):
        L = int(seqlens[s])
        rows = None if rows_by_seq is None else rows_by_seq.get(s)
        if rows_by_seq is not None and rows is None:
            continue
        for h in range(H):
            kh = h // grp
            f4 = (q8v[s][:L, h], qd["qsc"][s, h, :L], k8v[s][:L, kh], qd["ksc"][s, kh, :L]) if fp4 else None
            o = attention_head(None if fp4 else q8v[s][:L, h], None if fp4 else k8v[s][:L, kh],
                               None if fp4 else qd["sq"][s, h], None if fp4 else qd["sk"][s, kh],
                               vv[s][:L, kh], blk_q, blk_k, causal, rows=rows, pv_fp8=pv_fp8, fp4=f4,
                               v8h=None if v8v is None else v8v[s][:L, kh],
                               svh=None if v8v is None else qd["sv"][s, kh],
                               vmh=qd["vm"][s, kh] if (pv_fp8 and smooth_v) else None,
                               qdel=qd["qdelta"][s, h, :L] if "qdelta" in qd else None)
            if rows is None:
                ov[s][:L, h] = o
            else:
                ov[s][np.asarray(rows), h] = o
    return O, qd


def exact_attention(q, k, v, seqlens, cu, causal, sm_scale=None, rows_by_seq=None):
    """Unquantised attention softmax(Q K^T * sm_scale) V in fp64, no smoothing
    (the result the quantised method approximates; [SA2] "即插即用举例")."""
    nseq = len(seqlens)
    H, d = q.shape[-2], q.shape[-1]
    grp = H // k.shape[-2]
    sm = float(default_sm_scale(d) if sm_scale is None else np.float32(sm_scale))
    O = np.full(q.shape, np.nan, np.float64)
    ov = _seq_views(O, cu, nseq)
    qv, kv, vv = (_seq_views(a, cu, nseq) for a in (q, k, v))
    for s in range(nseq):
        L = int(seqlens[s])
        rows = np.arange(L) if rows_by_seq is None else rows_by_seq.get(s)
        if rows is None or L == 0:
            continue
        rows = np.asarray(rows)
        for h in range(H):
            S = (qv[s][rows, h].astype(np.float64) @ kv[s][:L, h // grp].astype(np.float64).T) * sm
            if causal:
                S = np.where(np.arange(L)[None, :] <= rows[:, None], S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            ov[s][rows, h] = (P @ vv[s][:L, h // grp].astype(np.float64)) / P.sum(axis=1, keepdims=True)
    return O
