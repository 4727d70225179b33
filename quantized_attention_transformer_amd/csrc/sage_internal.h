// Internal declarations shared by the libsage translation units (not part of
// the C ABI).  Addressing follows sage.h: element (s, h, n, c) of a dense
// tensor is at s*S.s + h*S.h + n*S.n + c, of a packed tensor at
// (cu[s] + n)*S.n + h*S.h + c.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace sage {

struct Str {
  int64_t s, h, n;
};

// Tokens per partial of the V column statistics.
constexpr int kColChunk = 512;
// Tokens per partial of the K (and Q) column sums; the workspace holds ceil(max_seqlen /
// kKSumRows) partials per (sequence, head).
constexpr int kKSumRows = 128;
// Tokens per partial of the K column sums in the INT8 pre-pass (sage_quantize, sage_attn):
// fewer partials for the K quantisation to add up.
constexpr int kKChunkRows = 512;

// Packed sequences: sequence s holds tokens [cu[s], cu[s+1]) of `total`.  The
// offsets are clamped so that every token range stays inside [0, total) and
// no length exceeds max_seqlen, whatever cu_seqlens holds: a malformed array
// gives wrong sequences, never an access outside the caller's buffers or the
// per-sequence scale, workspace and output rows sized from max_seqlen.
__host__ __device__ __forceinline__ int seq_start(const int32_t* cu, int s, int total) {
  return min(max(cu[s], 0), total);
}
__host__ __device__ __forceinline__ int seq_len(const int32_t* cu, int s, int max_seqlen, int total) {
  if (!cu) return max_seqlen;
  const int a = seq_start(cu, s, total);
  return min(min(max(cu[s + 1], a), total) - a, max_seqlen);
}

// Offset of token 0 of (sequence s, head h).
__device__ __forceinline__ int64_t seq_head_base(const int32_t* cu, Str st, int s, int h, int total) {
  return (cu ? (int64_t)seq_start(cu, s, total) * st.n : (int64_t)s * st.s) + (int64_t)h * st.h;
}

struct Problem {
  const int32_t* cu;
  int nseq, heads, max_seqlen, head_dim, blk_q, blk_k;
  int total;             // packed sequences: total_tokens (< 2^31); dense: unused
  int kv_heads;          // heads of K and V (grouped-query attention: heads % kv_heads == 0)
  int dv;                // channels of the fp16 inputs and of O: head_dim, or 96 with head_dim 128
                         // (head dimension 96 runs on the 128-channel kernels, channels 96..127 zero)
  int nbq, nbk, nchunk;  // ceil(max_seqlen/blk_q), ceil(max_seqlen/blk_k), ceil(max_seqlen/kColChunk)
  int nks;               // ceil(max_seqlen/kKSumRows): K column-sum partials per (sequence, head)
  int smooth_q;          // Q smoothed by its mean; S compensated by q_delta (key blocks: multiples of 64)
  int qk_fp4;            // 4-bit (MXFP4) Q and K
};

// ---- pre-pass (prepass.hip) ----
// INT8 Q blocks (blk_q == 1: one scale per token), plus fp64 column sums of K over chunks of
// kKChunkRows tokens (partial: room for nseq*kv_heads*nks*head_dim).
hipError_t launch_quant_q_colsum(const Problem& p, const void* Q, Str qs, const void* K, Str ks, float sm_scale,
                                 int8_t* q8, Str q8s, float* q_scale, double* partial, hipStream_t st);
// k_mean = fp32(sum of the partials / L) per (sequence, head, channel), and INT8 K blocks of K - k_mean;
// the partials cover `chunk` tokens each (kKChunkRows after launch_quant_q_colsum, kKSumRows after
// launch_quant_q_smooth).
hipError_t launch_quant_k(const Problem& p, const void* K, Str ks, const double* partial, int chunk, float* k_mean, int8_t* k8,
                          Str k8s, float* k_scale, hipStream_t st);
// Smooth Q: fp64 column sums of Q (qpart: nseq*heads*nks*head_dim) and of K (kpart, as
// launch_quant_q_colsum's partial), q_mean = fp32((sum / L) * sm_scale) per (sequence, query
// head, channel), and INT8 blocks of Q_s = fp32(fp32(Q * sm_scale) - q_mean).
hipError_t launch_quant_q_smooth(const Problem& p, const void* Q, Str qs, const void* K, Str ks, float sm_scale,
                                 int8_t* q8, Str q8s, float* q_scale, float* q_mean, double* qpart, double* kpart,
                                 hipStream_t st);
// 4-bit Q and K (MXFP4): column sums of K (and, smooth_q, of Q; partials as above), k_mean
// (q_mean) finalised, then per row and block of 32 channels an E8M0 code (byte cg/4 of the row
// in qsc/ksc, row stride .n bytes) and the E2M1 codes packed two per byte, low nibble first
// (q4/k4, row stride .n bytes), of Q' = fp32(Q * sm_scale) (- q_mean) and K' = fp32(K - k_mean).
hipError_t launch_quant_mxfp4(const Problem& p, const void* Q, Str qs, const void* K, Str ks, float sm_scale,
                              uint8_t* q4, Str q4s, uint8_t* qsc, Str qss, uint8_t* k4, Str k4s, uint8_t* ksc, Str kss,
                              float* k_mean, float* q_mean, double* kpart, double* qpart, hipStream_t st);
// q_delta[s, h, n] = q_mean[s, h] . fp32(K[s, kvh(h), n] - k_mean[s, kvh(h)]) (fp64 sum, fp32 result);
// element (s, h, n) at seq_head_base(cu, qds, s, h) + n.
hipError_t launch_q_delta(const Problem& p, const void* K, Str ks, const float* q_mean, const float* k_mean,
                          float* q_delta, Str qds, hipStream_t st);
// v_scale = max|V| / 448 per (sequence, head, channel): zero fill, atomic column max, divide in place.
hipError_t launch_v_colmax(const Problem& p, const void* V, Str vs, float* v_scale, hipStream_t st);
hipError_t launch_v_scale(const Problem& p, float* v_scale, hipStream_t st);
// E4M3 codes of V (v_mean != nullptr: of fp32(V - v_mean)) with the per-channel v_scale.
hipError_t launch_quant_v(const Problem& p, const void* V, Str vs, const float* v_scale, const float* v_mean,
                          uint8_t* v8, Str v8s, hipStream_t st);
// Smoothed V: per chunk of kColChunk tokens the exact fp64 column sums and the fp16 column
// max/min (psum, pmax, pmin: nseq*heads*nchunk*head_dim each), then per (sequence, head,
// channel) v_mean = fp32(sum / L) and v_scale = max|fp32(V - v_mean)| / 448.
hipError_t launch_v_smooth_stats(const Problem& p, const void* V, Str vs, double* psum, float* pmax, float* pmin,
                                 float* v_scale, float* v_mean, hipStream_t st);

// ---- fused attention (attn_fwd.hip) ----
struct AttnArgs {
  const int8_t* q8;
  Str q8s;
  const int8_t* k8;
  Str k8s;
  const float* q_scale;
  const float* k_scale;
  const void* v;  // fp16 or E4M3
  Str vs;
  const float* v_scale;
  void* out;  // fp16
  Str os;
  int32_t* dump;  // debug i32 scores or nullptr
  const float* v_mean;  // FP8 with smoothed V: per-channel mean added to O, else nullptr
  const float* q_delta;  // smooth Q: per (sequence, query head, key) compensation added to S, else nullptr
  Str qds;               // its strides (n = 1)
  // 4-bit Q.K^T (MXFP4; head_dim 128): q8/k8 then hold E2M1 codes, two per byte (rows of
  // head_dim/2 bytes), and these the E8M0 codes, 4 bytes per row (strides in bytes); else nullptr
  const uint8_t* qsc4;
  Str qss4;
  const uint8_t* ksc4;
  Str kss4;
};
hipError_t launch_attn(const Problem& p, const AttnArgs& a, bool causal, bool fp8, hipStream_t st);
// One FP8 P.V MFMA on given operands (debug; one wave).
hipError_t launch_debug_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, int sa, int sb, float* d,
                                 hipStream_t st);
// One MXFP4 MFMA with per-lane E8M0 scales (debug; one wave).
hipError_t launch_debug_mxfp4_mfma(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                   const float* c, float* d, hipStream_t st);

}  // namespace sage
