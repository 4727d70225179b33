/*
 * sage.h -- C ABI of libsage, SageAttention's 8-bit attention forward pass
 * for AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (cited by title and section):
 *   [SA]  "SageAttention：低比特量化Attention，实现推理加速" -- section 技术方案:
 *         item 1 smooth K (subtract its per-channel mean), item 2 per-block
 *         INT8 quantisation of Q and K (INT32 accumulation of Q K^T), item 3
 *         P.V kept in FP16 with an FP16 accumulator.
 *   [SA2] "4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级" --
 *         section 即插即用举例 (input Q, K, V; output O) and section 技术方案
 *         item 2 (quantisation finer than per block) and item 4 (P and V
 *         quantised to FP8 E4M3).
 *         The same page, after 技术方案: the optional smoothing of V (subtract
 *         mean(V) per channel, add it back to the output).
 *   [GUIDE] "如何将SageAttention量化注意力机制集成到你的AI项目中获得2-5倍速度提升"
 *         -- section 针对不同AI任务的优化建议 (causal mode; varlen kernels).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Problem.  `nseq` sequences, `heads` heads, head dimension `head_dim` (64 or
 *   128; sage_attn and sage_workspace_bytes also take 96, see there; every
 *   other entry returns SAGE_ERR_UNSUPPORTED for it).  Dense problems (cu_seqlens == NULL) have nseq = batch and every
 *   sequence of length max_seqlen.  Packed variable-length problems pass
 *   `cu_seqlens`, a DEVICE array of nseq+1 int32 prefix offsets (cu[0] = 0,
 *   non-decreasing, cu[nseq] = total_tokens); sequence s is tokens
 *   [cu[s], cu[s+1]).  `max_seqlen` must be >= every length (the library
 *   never reads cu_seqlens on the host); total_tokens < 2^31.  A cu_seqlens
 *   that breaks these rules gives wrong results, not out-of-bounds
 *   accesses: the kernels clamp every offset to [0, total_tokens] and every
 *   length to max_seqlen.  Queries and keys are the same tokens
 *   (self-attention).
 * Tensors.  Element strides in a sage_strides {s, h, n}: element (seq s,
 *   head h, token n, channel c) of a dense tensor is at s*S.s + h*S.h +
 *   n*S.n + c; in a packed tensor it is at (cu[s] + n)*S.n + h*S.h + c
 *   (S.s is ignored).  The channel stride is 1.  Base pointers must be
 *   16-byte aligned and S.h, S.n multiples of 8 elements (fp16) / 16 (8-bit).
 *   Q, K, V, O are fp16.  q8/k8 are int8; v8 is OCP FP8 E4M3 (uint8).
 * Heads.  Q and O have `heads` heads; K, V, k8, v8 have kv_heads (0: the
 *   same).  A problem that describes V alone (sage_quantize_v_fp8*) uses
 *   `heads` for V's heads.
 * Scales.  q_scale [nseq][heads][ceil(max_seqlen/blk_q)] and k_scale
 *   [nseq][kv_heads][ceil(max_seqlen/blk_k)] fp32, contiguous; entries past a
 *   sequence's last block are left unspecified.  k_mean and v_scale are
 *   [nseq][kv_heads][head_dim] fp32, contiguous.
 * Blocks.  blk_q and blk_k: quantisation block lengths in tokens, multiples
 *   of 16 in [16, 256]; blk_q may also be 1, one Q scale per token (finer
 *   than per-block, as [SA2] 技术方案 item 2 argues; in the fused kernel each
 *   lane holds one query row, so a per-token scale costs nothing there).
 *   Blocks restart at each sequence's first token; the last block of a
 *   sequence holds its remaining tokens.
 * Ownership.  The caller allocates every buffer (device memory) including
 *   the workspace; the library allocates and frees nothing on the device and
 *   keeps no pointer after returning.
 * Aliasing.  No output of a call (O, codes, scales, means, the workspace)
 *   may overlap any of its inputs or another of its outputs: the kernels
 *   read and write them concurrently, and the library does not check.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  All work
 *   is enqueued asynchronously; nothing synchronises.  Buffers must stay
 *   valid until the stream has executed the work.
 * Errors.  Every entry point returns a sage_status.  Arguments are checked
 *   before anything is enqueued; on a non-OK status nothing was enqueued,
 *   except SAGE_ERR_HIP, which reports a failed launch.  sage_last_error()
 *   returns a thread-local message describing the last non-OK status.
 *   Non-finite inputs are outside the contract.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARG = -1,
  SAGE_ERR_UNSUPPORTED = -2,
  SAGE_ERR_WORKSPACE = -3,
  SAGE_ERR_HIP = -4
} sage_status;

/* P.V precision: fp16 P and V; E4M3 P and V; E4M3 P and smoothed V (V minus
 * its per-channel mean, the mean added to O: the optional V smoothing the
 * [SA2] page describes after 技术方案). */
typedef enum { SAGE_PV_FP16 = 0, SAGE_PV_FP8 = 1, SAGE_PV_FP8_SMOOTH_V = 2 } sage_pv_mode;

typedef struct {
  int64_t s, h, n;
} sage_strides;

typedef struct {
  int32_t nseq;               /* dense: batch; varlen: number of packed sequences */
  int32_t heads;
  int32_t max_seqlen;         /* dense: N; varlen: upper bound of every length    */
  int32_t head_dim;           /* 64 or 128 (96: sage_attn only)                    */
  int64_t total_tokens;       /* varlen: cu_seqlens[nseq]; dense: ignored          */
  const int32_t* cu_seqlens;  /* device pointer, nseq+1 entries; NULL = dense      */
  int32_t blk_q;              /* Q quantisation block (tokens)                     */
  int32_t blk_k;              /* K quantisation block (tokens)                     */
  int32_t kv_heads;           /* heads of K and V; 0 = heads.  Fewer (a divisor of
                                 heads): grouped-query attention, query head h
                                 reads K/V head h / (heads / kv_heads)            */
  int32_t smooth_q;           /* 1: smooth Q as well (sage_attn and
                                 sage_quantize_smooth_q; blk_k a multiple of 64);
                                 0: not                                           */
  int32_t qk_fp4;             /* 1: 4-bit Q and K (OCP MXFP4; sage_attn with
                                 head_dim 128 or 96, sage_quantize_mxfp4); 0: INT8 */
} sage_problem;

/* Bytes of workspace sage_attn and sage_quantize need for this problem
 * (sage_attn: int8 Q/K, their scales, mean(K), column-sum partials and, for
 * the FP8 modes, the E4M3 V, its scales (and means and column statistics
 * for SAGE_PV_FP8_SMOOTH_V); with smooth_q also Q's column-sum partials,
 * mean(Q') and the per-key compensation; sage_quantize: the column-sum
 * partials only).  Writes *bytes; returns SAGE_OK or SAGE_ERR_INVALID_ARG. */
int sage_workspace_bytes(const sage_problem* p, int pv_mode, size_t* bytes);
int sage_quantize_workspace_bytes(const sage_problem* p, size_t* bytes);

/* Smooth K and quantise Q and K to INT8 per block ([SA] 技术方案 items 1-2).
 *   k_mean[s][h][c] = fp32( (sum over the sequence's tokens of K, exact) / L )
 *   Q' = fp32(Q * sm_scale); K' = fp32(K - k_mean)
 *   per block: scale = fp32(absmax / 127); code = round-half-even(fp32(x / scale)),
 *   in [-127, 127]; an all-zero block has scale 0 and codes 0.
 * sm_scale <= 0 selects fp32(1/sqrt(head_dim)).  q8 and k8 use the strides
 * q8s, k8s (any layout, same indexing rules as the inputs).  `workspace`
 * holds sage_quantize_workspace_bytes() bytes of scratch. */
int sage_quantize(const sage_problem* p,
                  const void* Q, sage_strides qs, const void* K, sage_strides ks, float sm_scale,
                  int8_t* q8, sage_strides q8s, int8_t* k8, sage_strides k8s,
                  float* q_scale, float* k_scale, float* k_mean,
                  void* workspace, size_t workspace_bytes, void* stream);

/* sage_quantize with Q smoothed as well ([SA2] 技术方案 item 1; p->smooth_q
 * must be 1, blk_k a multiple of 64):
 *   q_mean[s][h][c] = fp32( ((sum over the sequence's tokens of Q, exact) / L)
 *                           * sm_scale )                       (fp64 operations)
 *   Q_s = fp32(fp32(Q * sm_scale) - q_mean), quantised per block (or per
 *   token) in place of Q' as above; K as in sage_quantize;
 *   q_delta[s][h][n] = fp32( sum_c q_mean[s][h][c] * K'[s][h'][n][c] ), the
 *   sum in fp64 (h' = the K head of query head h), which sage_attn adds to
 *   every row of S: S = q8 . k8 * q_scale * k_scale + q_delta.
 * q_mean: [nseq][heads][head_dim] fp32.  q_delta: fp32, dense
 * [nseq][heads][max_seqlen], packed [heads][total_tokens] (entries past a
 * sequence's end unspecified).  `workspace` holds
 * sage_quantize_smooth_q_workspace_bytes() bytes (column-sum partials of Q
 * and K). */
int sage_quantize_smooth_q_workspace_bytes(const sage_problem* p, size_t* bytes);

/* 4-bit Q and K ([SA2] 技术方案: the INT4 kernel; gfx950 has no INT4 matrix
 * instruction, its 4-bit one takes OCP MXFP4):
 *   K' = fp32(K - k_mean) as in sage_quantize; Q' = fp32(Q * sm_scale), or with
 *   p->smooth_q Q_s as in sage_quantize_smooth_q (then q_mean and q_delta are
 *   written as there; otherwise they may be NULL);
 *   per row and block of 32 channels: e = floor(log2 max|x|) - 2, E8M0 code
 *   e + 127 (clamped to [0, 254]; 0 for an all-zero block), and E2M1 codes of
 *   x / 2^e, round to nearest even, saturating at 6, sign bit from x.
 * q4/k4: the codes two per byte (channel 2c in the low nibble of byte c), rows
 * of head_dim/2 bytes at the strides q4s/k4s (counted in bytes, multiples of
 * 16); q_sc/k_sc: one E8M0 byte per block, rows of head_dim/32 bytes at the
 * strides q_scs/k_scs (bytes).  head_dim 64 or 128.
 * `workspace` holds sage_quantize_mxfp4_workspace_bytes() bytes. */
int sage_quantize_mxfp4_workspace_bytes(const sage_problem* p, size_t* bytes);
int sage_quantize_mxfp4(const sage_problem* p,
                        const void* Q, sage_strides qs, const void* K, sage_strides ks, float sm_scale,
                        uint8_t* q4, sage_strides q4s, uint8_t* q_sc, sage_strides q_scs,
                        uint8_t* k4, sage_strides k4s, uint8_t* k_sc, sage_strides k_scs,
                        float* k_mean, float* q_mean, float* q_delta,
                        void* workspace, size_t workspace_bytes, void* stream);
int sage_quantize_smooth_q(const sage_problem* p,
                           const void* Q, sage_strides qs, const void* K, sage_strides ks, float sm_scale,
                           int8_t* q8, sage_strides q8s, int8_t* k8, sage_strides k8s,
                           float* q_scale, float* k_scale, float* k_mean, float* q_mean, float* q_delta,
                           void* workspace, size_t workspace_bytes, void* stream);

/* FP8 E4M3 V for the FP8 P.V path ([SA2] 技术方案 item 4):
 *   v_scale[s][h][c] = fp32(max over the sequence's tokens of |V| / 448)
 *   v8 = E4M3(fp32(V / v_scale)), round to nearest even, saturating at 448;
 *   a channel that is all zero gets scale 0 and codes 0. */
int sage_quantize_v_fp8(const sage_problem* p, const void* V, sage_strides vs,
                        uint8_t* v8, sage_strides v8s, float* v_scale, void* stream);

/* Smoothed FP8 E4M3 V for pv_mode SAGE_PV_FP8_SMOOTH_V ([SA2], V smoothing):
 *   v_mean[s][h][c] = fp32( (sum over the sequence's tokens of V, exact) / L )
 *   V' = fp32(V - v_mean); v_scale = fp32(max |V'| / 448) per channel;
 *   v8 = E4M3(fp32(V' / v_scale)) (a constant channel: scale 0, codes 0).
 * v_scale_mean holds 2 * nseq*heads*head_dim floats: v_scale [nseq][heads][head_dim]
 * followed by v_mean in the same layout.  `workspace` holds
 * sage_quantize_v_fp8_smooth_workspace_bytes() bytes of scratch (column
 * statistics per chunk of tokens). */
int sage_quantize_v_fp8_smooth_workspace_bytes(const sage_problem* p, size_t* bytes);
int sage_quantize_v_fp8_smooth(const sage_problem* p, const void* V, sage_strides vs,
                               uint8_t* v8, sage_strides v8s, float* v_scale_mean,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Fused attention over already-quantised inputs ([SA] 技术方案; [SA2] 即插即用举例):
 *   S = (q8 . k8^T) * q_scale[block(i)] * k_scale[block(j)]   (INT32 accumulation)
 *   keys of other sequences never count; causal keeps key j <= query i;
 *   O = softmax(S) V, online softmax in fp32 (exp2), P.V on fp16 MFMA with
 *   fp32 accumulation (pv_mode SAGE_PV_FP16, V fp16, v_scale unused) or on
 *   FP8 MFMA with P as E4M3(448 * 2^(S log2e - m)), m the running row maximum
 *   rounded up to an integer, and V = v8 with per-channel v_scale applied in
 *   the epilogue (pv_mode SAGE_PV_FP8).  pv_mode SAGE_PV_FP8_SMOOTH_V: V = v8
 *   of the smoothed V and v_scale points to the scales followed by the means
 *   (as written by sage_quantize_v_fp8_smooth); the epilogue adds the mean,
 *   exact since every row of softmax(S) sums to 1.  O is written as fp16 with
 *   strides os; rows of a sequence of length 0 are not written.  Problems
 *   with smooth_q set go through sage_attn (SAGE_ERR_UNSUPPORTED here).
 *   In the FP8 modes v_scale must be 16-byte aligned. */
int sage_attn_quantized(const sage_problem* p,
                        const int8_t* q8, sage_strides q8s, const int8_t* k8, sage_strides k8s,
                        const float* q_scale, const float* k_scale,
                        const void* V, sage_strides vs, const float* v_scale,
                        void* out, sage_strides os, int causal, int pv_mode, void* stream);

/* The whole forward pass: sage_quantize (+ sage_quantize_v_fp8 or
 * sage_quantize_v_fp8_smooth in the FP8 modes) into the workspace, then
 * sage_attn_quantized.  O = softmax(Q K^T * sm_scale) V
 * computed as described above.  `workspace` holds sage_workspace_bytes() bytes.
 * head_dim 96 (models with 96-channel heads, [SA2] 即插即用举例): Q, K, V and
 * O hold 96 channels per row; the intermediates in the workspace take the
 * 128-channel layout with channels 96..127 zero (which changes no block
 * maximum, K mean or Q.K), sm_scale <= 0 still selects 1/sqrt(96), and only
 * channels 0..95 of O are written.
 * smooth_q = 1: sage_quantize_smooth_q in place of sage_quantize, and the
 * fused kernel adds q_delta to S (a block whose scale is 0 has all codes 0;
 * its S is then the compensation alone).
 * qk_fp4 = 1: sage_quantize_mxfp4 in place of sage_quantize and the fused
 * kernel forms S = Q4 . K4^T on the MXFP4 matrix instruction (the E8M0 scales
 * applied inside it, fp32 result); blk_q and blk_k are not used. */
int sage_attn(const sage_problem* p,
              const void* Q, sage_strides qs, const void* K, sage_strides ks,
              const void* V, sage_strides vs, void* out, sage_strides os,
              int causal, float sm_scale, int pv_mode,
              void* workspace, size_t workspace_bytes, void* stream);

/* sage_attn for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation as sage_attn (same kernels, same results), with the
 * workspace taken from a fixed array of SAGE_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds on each GPU it runs on until the process ends (its
 * device address is looked up on the entry's first call on a device; the
 * entry calls no hipMalloc/hipFree and no allocating routine).  Problems
 * whose sage_workspace_bytes exceed it are refused with SAGE_ERR_WORKSPACE.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or host threads) race and must not be issued;
 * calls in one stream are ordered.  The stream must belong to the current
 * device.  Nothing in the array must start zeroed (every byte read is
 * written earlier in the same call). */
#define SAGE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sage_attn_noalloc(const sage_problem* p,
                      const void* Q, sage_strides qs, const void* K, sage_strides ks,
                      const void* V, sage_strides vs, void* out, sage_strides os,
                      int causal, float sm_scale, int pv_mode, void* stream);

/* Debug: the INT32 scores S_int = q8 . k8^T of the fused kernel's integer
 * stage ("SageAttention：低比特量化Attention，实现推理加速", 技术方案 item 2:
 * INT8 product, INT32 accumulator), taken from the fused kernel itself: a
 * dump instantiation of it runs the same K tile ring, the same steady-state
 * and edge-phase INT8 MFMA code and the same phase schedule, and writes every
 * tile's sums at the start of its softmax, before dequantisation (V is not
 * read, no scale is read, no O is written).  Dense problems only, with
 * max_seqlen <= 1024 and a multiple of 4; q8/k8 as for sage_attn_quantized
 * (k8 with kv_heads heads); s_out is int32 [nseq][heads][max_seqlen]
 * [max_seqlen] (query-major), every entry written. */
int sage_debug_qk_i32(const sage_problem* p,
                      const int8_t* q8, sage_strides q8s, const int8_t* k8, sage_strides k8s,
                      int32_t* s_out, void* stream);

/* Debug: one issue of the FP8 P.V instruction (v_mfma_scale_f32_32x32x64_f8f6f4)
 * on given operands, to check its arithmetic, e.g. the accumulator precision
 * ([SA2] 技术方案 item 3 reports an accumulator narrower than FP32 for the
 * FP8 matrix instruction of other hardware):
 *   D = (A . B) * 2^(scale_a - 127) * 2^(scale_b - 127) + C
 * A [32][64] and B [64][32] are OCP E4M3 codes, C and D fp32 [32][32], all
 * row-major device arrays (D may not alias the inputs); scale_a, scale_b are
 * E8M0 exponents in [0, 254].  One wave; asynchronous on `stream`. */
int sage_debug_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, int scale_a, int scale_b, float* d,
                        void* stream);

/* Debug: one issue of the same instruction in its MXFP4 form, the 4-bit Q.K^T
 * product of the 4-bit variant ([SA2] 技术方案, the INT4 kernel; gfx950's
 * 4-bit matrix format is OCP MXFP4):
 *   D[m][n] = C[m][n] + sum_k A[m][k] 2^(scale_a[m][k/32] - 127)
 *                             * B[k][n] 2^(scale_b[k/32][n] - 127)
 * A [32][64] and B [64][32] hold one E2M1 code per byte (low nibble);
 * scale_a [32][2] and scale_b [2][32] are E8M0 codes; C and D fp32 [32][32];
 * all row-major device arrays (D may not alias the inputs).  One wave;
 * asynchronous on `stream`. */
int sage_debug_mxfp4_mfma(const uint8_t* a, const uint8_t* b, const uint8_t* scale_a, const uint8_t* scale_b,
                          const float* c, float* d, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* sage_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H */
