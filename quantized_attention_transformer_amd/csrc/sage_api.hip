// Host side of libsage: the C ABI declared in include/sage.h.
//
// Every entry point validates its arguments before anything is enqueued,
// carves the caller's workspace, sizes the grids and enqueues the kernels on
// the caller's stream.  Nothing here allocates device memory, synchronises or
// reads device memory.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "sage.h"
#include "sage_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SAGE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// head_dim 96 runs on the 128-channel kernels with channels 96..127 zero; it is
// accepted by the entries that own their int8/E4M3 intermediates (sage_attn and
// its workspace query), whose layout then stays internal.
int check_problem(const sage_problem* p, bool allow_d96 = false) {
  if (!p) return fail(SAGE_ERR_INVALID_ARG, "problem is NULL");
  if (p->nseq < 0 || p->heads <= 0 || p->max_seqlen < 0)
    return fail(SAGE_ERR_INVALID_ARG, "nseq (%d) must be >= 0, heads (%d) > 0, max_seqlen (%d) >= 0", p->nseq,
                p->heads, p->max_seqlen);
  if (p->head_dim == 96 && !allow_d96)
    return fail(SAGE_ERR_UNSUPPORTED, "head_dim 96 is supported by sage_attn only (this entry: 64 or 128)");
  if (p->head_dim != 64 && p->head_dim != 96 && p->head_dim != 128)
    return fail(SAGE_ERR_UNSUPPORTED, "head_dim %d not supported (64, 96 or 128)", p->head_dim);
  auto block_ok = [](int b) { return b >= 16 && b <= 256 && b % 16 == 0; };
  if (!(block_ok(p->blk_q) || p->blk_q == 1) || !block_ok(p->blk_k))
    return fail(SAGE_ERR_INVALID_ARG,
                "blk_q/blk_k (%d, %d) must be multiples of 16 in [16, 256] (blk_q may also be 1: per token)",
                p->blk_q, p->blk_k);
  if (p->cu_seqlens && (p->total_tokens < 0 || p->total_tokens > INT32_MAX))
    return fail(SAGE_ERR_INVALID_ARG, "total_tokens (%lld) must be in [0, 2^31) (cu_seqlens is int32)",
                (long long)p->total_tokens);
  if (p->heads > 65535 || p->nseq > 65535) return fail(SAGE_ERR_UNSUPPORTED, "heads and nseq must be <= 65535");
  if (p->kv_heads < 0 || (p->kv_heads > 0 && p->heads % p->kv_heads != 0))
    return fail(SAGE_ERR_INVALID_ARG, "kv_heads (%d) must divide heads (%d) (0: same as heads)", p->kv_heads,
                p->heads);
  if (p->smooth_q != 0 && p->smooth_q != 1) return fail(SAGE_ERR_INVALID_ARG, "smooth_q must be 0 or 1");
  if (p->qk_fp4 != 0 && p->qk_fp4 != 1) return fail(SAGE_ERR_INVALID_ARG, "qk_fp4 must be 0 or 1");
  if (p->smooth_q && !p->qk_fp4 && p->blk_k % 64 != 0)
    return fail(SAGE_ERR_UNSUPPORTED, "smooth_q needs blk_k to be a multiple of 64 (got %d)", p->blk_k);
  return SAGE_OK;
}

// Entries that take INT8 Q and K only.
int no_qk_fp4(const sage_problem* p, const char* name) {
  if (p->qk_fp4)
    return fail(SAGE_ERR_UNSUPPORTED, "%s does not take qk_fp4 (use sage_quantize_mxfp4 / sage_attn)", name);
  return SAGE_OK;
}

// Entries that take caller-laid-out int8 Q without the smooth-Q compensation.
int no_smooth_q(const sage_problem* p, const char* name) {
  if (p->smooth_q)
    return fail(SAGE_ERR_UNSUPPORTED, "%s does not take smooth_q (use sage_quantize_smooth_q / sage_attn)", name);
  return SAGE_OK;
}

bool empty(const sage_problem* p) { return p->nseq == 0 || p->max_seqlen == 0; }

sage::Problem to_internal(const sage_problem* p) {
  sage::Problem q;
  q.cu = p->cu_seqlens;
  q.nseq = p->nseq;
  q.heads = p->heads;
  q.kv_heads = p->kv_heads > 0 ? p->kv_heads : p->heads;
  q.max_seqlen = p->max_seqlen;
  q.total = p->cu_seqlens ? (int)p->total_tokens : 0;
  q.head_dim = p->head_dim == 96 ? 128 : p->head_dim;
  q.dv = p->head_dim;
  q.blk_q = p->blk_q;
  q.blk_k = p->blk_k;
  q.nbq = (int)cdiv(p->max_seqlen, p->blk_q);
  q.nbk = (int)cdiv(p->max_seqlen, p->blk_k);
  q.nchunk = (int)cdiv(p->max_seqlen, sage::kColChunk);
  q.nks = (int)cdiv(p->max_seqlen, sage::kKSumRows);
  q.smooth_q = p->smooth_q;
  q.qk_fp4 = p->qk_fp4;
  return q;
}

// Tensor check: non-null, 16-byte aligned, head and token strides multiples of `mult` elements.
int check_tensor(const char* name, const void* ptr, sage_strides st, int mult, const sage_problem* p) {
  if (!ptr) return fail(SAGE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(SAGE_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  if (st.h % mult || st.n % mult || (!p->cu_seqlens && st.s % mult))
    return fail(SAGE_ERR_INVALID_ARG, "%s strides (s=%lld h=%lld n=%lld) must be multiples of %d elements", name,
                (long long)st.s, (long long)st.h, (long long)st.n, mult);
  if (st.h < 0 || st.n < 0 || st.s < 0) return fail(SAGE_ERR_INVALID_ARG, "%s strides must be non-negative", name);
  return SAGE_OK;
}

sage::Str S(sage_strides s) { return sage::Str{s.s, s.h, s.n}; }

// The attention kernel addresses one (sequence, head) of K and V through a
// buffer resource with 32-bit offsets: max_seqlen rows must span < 2 GiB.
int check_row_span(const char* name, sage_strides st, int elem_bytes, const sage_problem* p) {
  if ((int64_t)p->max_seqlen * st.n * elem_bytes >= (int64_t)1 << 31)
    return fail(SAGE_ERR_UNSUPPORTED, "%s: max_seqlen * token stride must stay below 2 GiB", name);
  return SAGE_OK;
}

int64_t tokens(const sage_problem* p) {
  return p->cu_seqlens ? p->total_tokens : (int64_t)p->nseq * p->max_seqlen;
}

int kv_heads_of(const sage_problem* p) { return p->kv_heads > 0 ? p->kv_heads : p->heads; }

// Workspace layout of sage_attn (offsets in bytes).  int8 Q/K (and E4M3 V)
// are stored head-major: dense [nseq][heads][max_seqlen][d], packed
// [heads][total_tokens][d] (K and V with kv_heads heads).
struct WsLayout {
  size_t q8, k8, sq, sk, km, colsum, v8, sv, vpsum, vpmax, vpmin, qpart, qm, qdelta, total;
  sage_strides s8q, s8kv, sqd;
  // 4-bit Q and K: q8/k8 hold the packed codes (rows of d/2 bytes, strides s4q/s4kv in
  // bytes) and sq/sk the E8M0 codes (rows of d/32 bytes, strides ssq/sskv)
  sage_strides s4q, s4kv, ssq, sskv;
};

// Strides of q_delta (one fp32 per (sequence, query head, token)): dense
// [nseq][heads][max_seqlen], packed [heads][total_tokens].
sage_strides qdelta_strides(const sage_problem* p) {
  const int64_t T = p->cu_seqlens ? p->total_tokens : (int64_t)p->max_seqlen;
  return p->cu_seqlens ? sage_strides{0, T, 1} : sage_strides{(int64_t)p->heads * T, T, 1};
}
int64_t tokens(const sage_problem* p);
size_t qdelta_count(const sage_problem* p) {
  return (size_t)(p->cu_seqlens ? tokens(p) : (int64_t)p->nseq * p->max_seqlen) * p->heads;
}

bool valid_pv_mode(int m) { return m == SAGE_PV_FP16 || m == SAGE_PV_FP8 || m == SAGE_PV_FP8_SMOOTH_V; }

// Partials of the smoothed-V statistics (sum, max, min per chunk and channel).
struct VSmoothWs {
  size_t psum, pmax, pmin, total;
};

VSmoothWs v_smooth_ws(const sage_problem* p, size_t base) {
  const sage::Problem q = to_internal(p);
  const size_t n = (size_t)p->nseq * q.kv_heads * q.nchunk * q.head_dim;
  VSmoothWs w{};
  w.psum = base;
  w.pmax = w.psum + align_up(n * 8);
  w.pmin = w.pmax + align_up(n * 4);
  w.total = w.pmin + align_up(n * 4) - base;
  return w;
}

WsLayout ws_layout(const sage_problem* p, int pv_mode) {
  const sage::Problem q = to_internal(p);
  const int64_t T = tokens(p);
  const int64_t d = q.head_dim, H = p->heads, Hk = q.kv_heads;
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  if (p->qk_fp4) {
    w.q8 = take((size_t)(T * H * d / 2));
    w.k8 = take((size_t)(T * Hk * d / 2));
    w.sq = take((size_t)(T * H * d / 32));
    w.sk = take((size_t)(T * Hk * d / 32));
  } else {
    w.q8 = take((size_t)(T * H * d));
    w.k8 = take((size_t)(T * Hk * d));
    w.sq = take((size_t)p->nseq * H * q.nbq * 4);
    w.sk = take((size_t)p->nseq * Hk * q.nbk * 4);
  }
  w.km = take((size_t)p->nseq * Hk * d * 4);
  w.colsum = take((size_t)p->nseq * Hk * q.nks * d * 8);
  if (pv_mode == SAGE_PV_FP8 || pv_mode == SAGE_PV_FP8_SMOOTH_V) {
    w.v8 = take((size_t)(T * Hk * d));
    // scales (then, smoothed V: the means)
    w.sv = take((size_t)p->nseq * Hk * d * 4 * (pv_mode == SAGE_PV_FP8_SMOOTH_V ? 2 : 1));
  }
  if (pv_mode == SAGE_PV_FP8_SMOOTH_V) {
    const VSmoothWs v = v_smooth_ws(p, off);
    w.vpsum = v.psum;
    w.vpmax = v.pmax;
    w.vpmin = v.pmin;
    off += v.total;
  }
  if (p->smooth_q) {
    w.qpart = take((size_t)p->nseq * H * q.nks * d * 8);
    w.qm = take((size_t)p->nseq * H * d * 4);
    w.qdelta = take(qdelta_count(p) * 4);
  }
  w.sqd = qdelta_strides(p);
  w.total = off;
  // head-major rows of `row` bytes: dense [nseq][heads][max_seqlen], packed [heads][T]
  auto rows = [&](int64_t heads, int64_t row) {
    return p->cu_seqlens ? sage_strides{0, T * row, row}
                         : sage_strides{heads * p->max_seqlen * row, p->max_seqlen * row, row};
  };
  w.s8q = rows(H, d);
  w.s8kv = rows(Hk, d);
  w.s4q = rows(H, d / 2);
  w.s4kv = rows(Hk, d / 2);
  w.ssq = rows(H, d / 32);
  w.sskv = rows(Hk, d / 32);
  return w;
}

size_t quantize_ws_bytes(const sage_problem* p) {
  const sage::Problem q = to_internal(p);
  return align_up((size_t)p->nseq * q.kv_heads * q.nks * q.head_dim * 8);
}

// sage_quantize_smooth_q: K column-sum partials, then Q's.
size_t quantize_sq_ws_bytes(const sage_problem* p) {
  const sage::Problem q = to_internal(p);
  return quantize_ws_bytes(p) + align_up((size_t)p->nseq * p->heads * q.nks * q.head_dim * 8);
}

// sage_quantize_mxfp4: K column-sum partials, then (smooth Q) Q's.
size_t quantize_fp4_ws_bytes(const sage_problem* p) {
  return p->smooth_q ? quantize_sq_ws_bytes(p) : quantize_ws_bytes(p);
}

int run_quantize_mxfp4(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                       float sm_scale, uint8_t* q4, sage_strides q4s, uint8_t* qsc, sage_strides qss, uint8_t* k4,
                       sage_strides k4s, uint8_t* ksc, sage_strides kss, float* k_mean, float* q_mean,
                       float* q_delta, sage_strides qds, double* kpart, double* qpart, hipStream_t st) {
  const sage::Problem q = to_internal(p);
  if (sm_scale <= 0.0f || !std::isfinite(sm_scale)) sm_scale = (float)(1.0 / std::sqrt((double)p->head_dim));
  hipError_t e;
  if ((e = sage::launch_quant_mxfp4(q, Q, S(qs), K, S(ks), sm_scale, q4, S(q4s), qsc, S(qss), k4, S(k4s), ksc,
                                    S(kss), k_mean, q_mean, kpart, qpart, st)) != hipSuccess)
    return hip_fail(e, "mxfp4 quantisation launch");
  if (p->smooth_q && (e = sage::launch_q_delta(q, K, S(ks), q_mean, k_mean, q_delta, S(qds), st)) != hipSuccess)
    return hip_fail(e, "q_delta launch");
  return SAGE_OK;
}

int run_quantize_smooth_q(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                          float sm_scale, int8_t* q8, sage_strides q8s, int8_t* k8, sage_strides k8s, float* q_scale,
                          float* k_scale, float* k_mean, float* q_mean, float* q_delta, sage_strides qds,
                          double* kpart, double* qpart, hipStream_t st) {
  const sage::Problem q = to_internal(p);
  if (sm_scale <= 0.0f || !std::isfinite(sm_scale)) sm_scale = (float)(1.0 / std::sqrt((double)p->head_dim));
  hipError_t e;
  if ((e = sage::launch_quant_q_smooth(q, Q, S(qs), K, S(ks), sm_scale, q8, S(q8s), q_scale, q_mean, qpart, kpart,
                                       st)) != hipSuccess)
    return hip_fail(e, "smooth-Q quantisation launch");
  if ((e = sage::launch_quant_k(q, K, S(ks), kpart, sage::kKSumRows, k_mean, k8, S(k8s), k_scale, st)) != hipSuccess)
    return hip_fail(e, "quant_k launch");
  if ((e = sage::launch_q_delta(q, K, S(ks), q_mean, k_mean, q_delta, S(qds), st)) != hipSuccess)
    return hip_fail(e, "q_delta launch");
  return SAGE_OK;
}

int run_quantize(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                 float sm_scale, int8_t* q8, sage_strides q8s, int8_t* k8, sage_strides k8s, float* q_scale,
                 float* k_scale, float* k_mean, double* colsum, hipStream_t st) {
  const sage::Problem q = to_internal(p);
  if (sm_scale <= 0.0f || !std::isfinite(sm_scale)) sm_scale = (float)(1.0 / std::sqrt((double)p->head_dim));
  hipError_t e;
  if ((e = sage::launch_quant_q_colsum(q, Q, S(qs), K, S(ks), sm_scale, q8, S(q8s), q_scale, colsum, st)) !=
      hipSuccess)
    return hip_fail(e, "quant_q_colsum launch");
  if ((e = sage::launch_quant_k(q, K, S(ks), colsum, sage::kKChunkRows, k_mean, k8, S(k8s), k_scale, st)) !=
      hipSuccess)
    return hip_fail(e, "quant_k launch");
  return SAGE_OK;
}

int run_quantize_v(const sage_problem* p, const void* V, sage_strides vs, uint8_t* v8, sage_strides v8s,
                   float* v_scale, hipStream_t st) {
  const sage::Problem q = to_internal(p);
  hipError_t e;
  if ((e = sage::launch_v_colmax(q, V, S(vs), v_scale, st)) != hipSuccess) return hip_fail(e, "v_colmax launch");
  if ((e = sage::launch_v_scale(q, v_scale, st)) != hipSuccess) return hip_fail(e, "v_scale launch");
  if ((e = sage::launch_quant_v(q, V, S(vs), v_scale, nullptr, v8, S(v8s), st)) != hipSuccess)
    return hip_fail(e, "quant_v launch");
  return SAGE_OK;
}

// v_scale_mean: nseq*heads*head_dim scales, then as many means.
int run_quantize_v_smooth(const sage_problem* p, const void* V, sage_strides vs, uint8_t* v8, sage_strides v8s,
                          float* v_scale_mean, char* ws, const VSmoothWs& w, hipStream_t st) {
  const sage::Problem q = to_internal(p);
  float* const vmean = v_scale_mean + (size_t)p->nseq * q.kv_heads * q.head_dim;
  hipError_t e;
  if ((e = sage::launch_v_smooth_stats(q, V, S(vs), (double*)(ws + w.psum), (float*)(ws + w.pmax),
                                       (float*)(ws + w.pmin), v_scale_mean, vmean, st)) != hipSuccess)
    return hip_fail(e, "v smooth stats launch");
  if ((e = sage::launch_quant_v(q, V, S(vs), v_scale_mean, vmean, v8, S(v8s), st)) != hipSuccess)
    return hip_fail(e, "quant_v launch");
  return SAGE_OK;
}

}  // namespace

extern "C" {

const char* sage_last_error(void) { return g_last_error.c_str(); }

// The fused kernel's 4-bit Q.K^T runs on 128-channel heads (96: padded).
int fp4_head_dim(const sage_problem* p) {
  if (p->qk_fp4 && p->head_dim == 64)
    return fail(SAGE_ERR_UNSUPPORTED, "qk_fp4 attention needs head_dim 128 or 96 (got 64)");
  return SAGE_OK;
}

int sage_workspace_bytes(const sage_problem* p, int pv_mode, size_t* bytes) {
  int rc = check_problem(p, true);
  if (rc || (rc = fp4_head_dim(p))) return rc;
  if (!valid_pv_mode(pv_mode)) return fail(SAGE_ERR_INVALID_ARG, "bad pv_mode %d", pv_mode);
  if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(p, pv_mode).total;
  return SAGE_OK;
}

int sage_quantize_workspace_bytes(const sage_problem* p, size_t* bytes) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = quantize_ws_bytes(p);
  return SAGE_OK;
}

int sage_quantize(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                  float sm_scale, int8_t* q8, sage_strides q8s, int8_t* k8, sage_strides k8s, float* q_scale,
                  float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc || (rc = no_smooth_q(p, "sage_quantize")) || (rc = no_qk_fp4(p, "sage_quantize"))) return rc;
  if (empty(p)) return SAGE_OK;
  if ((rc = check_tensor("Q", Q, qs, 8, p)) || (rc = check_tensor("K", K, ks, 8, p)) ||
      (rc = check_tensor("q8", q8, q8s, 16, p)) || (rc = check_tensor("k8", k8, k8s, 16, p)))
    return rc;
  if (!q_scale || !k_scale || !k_mean) return fail(SAGE_ERR_INVALID_ARG, "scale/mean outputs must not be NULL");
  if (!workspace || workspace_bytes < quantize_ws_bytes(p))
    return fail(SAGE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, quantize_ws_bytes(p));
  if (!aligned16(workspace)) return fail(SAGE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return run_quantize(p, Q, qs, K, ks, sm_scale, q8, q8s, k8, k8s, q_scale, k_scale, k_mean, (double*)workspace,
                      (hipStream_t)stream);
}

int sage_quantize_smooth_q_workspace_bytes(const sage_problem* p, size_t* bytes) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = quantize_sq_ws_bytes(p);
  return SAGE_OK;
}

int sage_quantize_smooth_q(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                           float sm_scale, int8_t* q8, sage_strides q8s, int8_t* k8, sage_strides k8s, float* q_scale,
                           float* k_scale, float* k_mean, float* q_mean, float* q_delta, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc || (rc = no_qk_fp4(p, "sage_quantize_smooth_q"))) return rc;
  if (!p->smooth_q) return fail(SAGE_ERR_INVALID_ARG, "sage_quantize_smooth_q needs p->smooth_q = 1");
  if (empty(p)) return SAGE_OK;
  if ((rc = check_tensor("Q", Q, qs, 8, p)) || (rc = check_tensor("K", K, ks, 8, p)) ||
      (rc = check_tensor("q8", q8, q8s, 16, p)) || (rc = check_tensor("k8", k8, k8s, 16, p)))
    return rc;
  if (!q_scale || !k_scale || !k_mean || !q_mean || !q_delta)
    return fail(SAGE_ERR_INVALID_ARG, "scale/mean/delta outputs must not be NULL");
  const size_t need = quantize_sq_ws_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(SAGE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(SAGE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = (char*)workspace;
  return run_quantize_smooth_q(p, Q, qs, K, ks, sm_scale, q8, q8s, k8, k8s, q_scale, k_scale, k_mean, q_mean, q_delta,
                               qdelta_strides(p), (double*)ws, (double*)(ws + quantize_ws_bytes(p)),
                               (hipStream_t)stream);
}

int sage_quantize_mxfp4_workspace_bytes(const sage_problem* p, size_t* bytes) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = quantize_fp4_ws_bytes(p);
  return SAGE_OK;
}

int sage_quantize_mxfp4(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                        float sm_scale, uint8_t* q4, sage_strides q4s, uint8_t* q_sc, sage_strides q_scs, uint8_t* k4,
                        sage_strides k4s, uint8_t* k_sc, sage_strides k_scs, float* k_mean, float* q_mean,
                        float* q_delta, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (empty(p)) return SAGE_OK;
  if ((rc = check_tensor("Q", Q, qs, 8, p)) || (rc = check_tensor("K", K, ks, 8, p)) ||
      (rc = check_tensor("q4", q4, q4s, 16, p)) || (rc = check_tensor("k4", k4, k4s, 16, p)))
    return rc;
  if (!q_sc || !k_sc || q_scs.h < 0 || q_scs.n < 0 || q_scs.s < 0 || k_scs.h < 0 || k_scs.n < 0 || k_scs.s < 0)
    return fail(SAGE_ERR_INVALID_ARG, "q_sc/k_sc must be non-NULL with non-negative strides");
  if (!k_mean || (p->smooth_q && (!q_mean || !q_delta)))
    return fail(SAGE_ERR_INVALID_ARG, "k_mean (and with smooth_q q_mean, q_delta) must not be NULL");
  const size_t need = quantize_fp4_ws_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(SAGE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(SAGE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = (char*)workspace;
  return run_quantize_mxfp4(p, Q, qs, K, ks, sm_scale, q4, q4s, q_sc, q_scs, k4, k4s, k_sc, k_scs, k_mean, q_mean,
                            q_delta, qdelta_strides(p), (double*)ws,
                            p->smooth_q ? (double*)(ws + quantize_ws_bytes(p)) : nullptr, (hipStream_t)stream);
}

int sage_quantize_v_fp8_smooth_workspace_bytes(const sage_problem* p, size_t* bytes) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!bytes) return fail(SAGE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = v_smooth_ws(p, 0).total;
  return SAGE_OK;
}

int sage_quantize_v_fp8_smooth(const sage_problem* p, const void* V, sage_strides vs, uint8_t* v8, sage_strides v8s,
                               float* v_scale_mean, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (empty(p)) return SAGE_OK;
  if ((rc = check_tensor("V", V, vs, 8, p)) || (rc = check_tensor("v8", v8, v8s, 16, p))) return rc;
  if (!v_scale_mean) return fail(SAGE_ERR_INVALID_ARG, "v_scale_mean is NULL");
  const VSmoothWs w = v_smooth_ws(p, 0);
  if (!workspace || workspace_bytes < w.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, w.total);
  if (!aligned16(workspace)) return fail(SAGE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return run_quantize_v_smooth(p, V, vs, v8, v8s, v_scale_mean, (char*)workspace, w, (hipStream_t)stream);
}

int sage_quantize_v_fp8(const sage_problem* p, const void* V, sage_strides vs, uint8_t* v8, sage_strides v8s,
                        float* v_scale, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (empty(p)) return SAGE_OK;
  if ((rc = check_tensor("V", V, vs, 8, p)) || (rc = check_tensor("v8", v8, v8s, 16, p))) return rc;
  if (!v_scale) return fail(SAGE_ERR_INVALID_ARG, "v_scale is NULL");
  return run_quantize_v(p, V, vs, v8, v8s, v_scale, (hipStream_t)stream);
}

int sage_attn_quantized(const sage_problem* p, const int8_t* q8, sage_strides q8s, const int8_t* k8,
                        sage_strides k8s, const float* q_scale, const float* k_scale, const void* V, sage_strides vs,
                        const float* v_scale, void* out, sage_strides os, int causal, int pv_mode, void* stream) {
  int rc = check_problem(p);
  if (rc || (rc = no_smooth_q(p, "sage_attn_quantized")) || (rc = no_qk_fp4(p, "sage_attn_quantized"))) return rc;
  if (!valid_pv_mode(pv_mode)) return fail(SAGE_ERR_INVALID_ARG, "bad pv_mode %d", pv_mode);
  if (empty(p)) return SAGE_OK;
  const bool fp8 = pv_mode != SAGE_PV_FP16;
  if ((rc = check_tensor("q8", q8, q8s, 16, p)) || (rc = check_tensor("k8", k8, k8s, 16, p)) ||
      (rc = check_tensor("V", V, vs, fp8 ? 16 : 8, p)) || (rc = check_tensor("out", out, os, 8, p)))
    return rc;
  if (!q_scale || !k_scale || (fp8 && !v_scale)) return fail(SAGE_ERR_INVALID_ARG, "scales must not be NULL");
  if (fp8 && !aligned16(v_scale)) return fail(SAGE_ERR_INVALID_ARG, "v_scale must be 16-byte aligned");
  if ((rc = check_row_span("k8", k8s, 1, p)) || (rc = check_row_span("V", vs, fp8 ? 1 : 2, p))) return rc;
  const float* v_mean =
      pv_mode == SAGE_PV_FP8_SMOOTH_V ? v_scale + (size_t)p->nseq * kv_heads_of(p) * p->head_dim : nullptr;
  sage::AttnArgs a{q8, S(q8s), k8, S(k8s), q_scale, k_scale, V, S(vs), v_scale, out, S(os), nullptr, v_mean, nullptr,
                   sage::Str{0, 0, 0}};
  hipError_t e = sage::launch_attn(to_internal(p), a, causal != 0, fp8, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return SAGE_OK;
}

// Arguments of sage_attn / sage_attn_noalloc checked; the workspace is the
// caller's or the library's scratch array.
static int check_attn_args(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                           const void* V, sage_strides vs, void* out, sage_strides os, int pv_mode) {
  int rc = check_problem(p, true);
  if (rc || (rc = fp4_head_dim(p))) return rc;
  if (!valid_pv_mode(pv_mode)) return fail(SAGE_ERR_INVALID_ARG, "bad pv_mode %d", pv_mode);
  if (empty(p)) return SAGE_OK;
  if ((rc = check_tensor("Q", Q, qs, 8, p)) || (rc = check_tensor("K", K, ks, 8, p)) ||
      (rc = check_tensor("V", V, vs, 8, p)) || (rc = check_tensor("out", out, os, 8, p)))
    return rc;
  return check_row_span("V", vs, 2, p);
}

static int run_attn(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                    const void* V, sage_strides vs, void* out, sage_strides os, int causal, float sm_scale,
                    int pv_mode, char* ws, hipStream_t st);

int sage_attn(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks, const void* V,
              sage_strides vs, void* out, sage_strides os, int causal, float sm_scale, int pv_mode, void* workspace,
              size_t workspace_bytes, void* stream) {
  int rc = check_attn_args(p, Q, qs, K, ks, V, vs, out, os, pv_mode);
  if (rc || empty(p)) return rc;
  const WsLayout w = ws_layout(p, pv_mode);
  if (!workspace || workspace_bytes < w.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, w.total);
  if (!aligned16(workspace)) return fail(SAGE_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return run_attn(p, Q, qs, K, ks, V, vs, out, os, causal, sm_scale, pv_mode, (char*)workspace,
                  (hipStream_t)stream);
}

static int run_attn(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                    const void* V, sage_strides vs, void* out, sage_strides os, int causal, float sm_scale,
                    int pv_mode, char* ws, hipStream_t st) {
  int rc;
  const WsLayout w = ws_layout(p, pv_mode);
  int8_t* q8 = (int8_t*)(ws + w.q8);
  int8_t* k8 = (int8_t*)(ws + w.k8);
  float* sq = (float*)(ws + w.sq);
  float* sk = (float*)(ws + w.sk);
  if (p->qk_fp4) {
    if ((rc = run_quantize_mxfp4(p, Q, qs, K, ks, sm_scale, (uint8_t*)q8, w.s4q, (uint8_t*)sq, w.ssq, (uint8_t*)k8,
                                 w.s4kv, (uint8_t*)sk, w.sskv, (float*)(ws + w.km), (float*)(ws + w.qm),
                                 (float*)(ws + w.qdelta), w.sqd, (double*)(ws + w.colsum), (double*)(ws + w.qpart),
                                 st)))
      return rc;
  } else if (p->smooth_q) {
    if ((rc = run_quantize_smooth_q(p, Q, qs, K, ks, sm_scale, q8, w.s8q, k8, w.s8kv, sq, sk, (float*)(ws + w.km),
                                    (float*)(ws + w.qm), (float*)(ws + w.qdelta), w.sqd, (double*)(ws + w.colsum),
                                    (double*)(ws + w.qpart), st)))
      return rc;
  } else if ((rc = run_quantize(p, Q, qs, K, ks, sm_scale, q8, w.s8q, k8, w.s8kv, sq, sk, (float*)(ws + w.km),
                                (double*)(ws + w.colsum), st))) {
    return rc;
  }
  const void* vin = V;
  sage_strides vin_s = vs;
  const float* sv = nullptr;
  const float* vmean = nullptr;
  if (pv_mode == SAGE_PV_FP8) {
    if ((rc = run_quantize_v(p, V, vs, (uint8_t*)(ws + w.v8), w.s8kv, (float*)(ws + w.sv), st)))
      return rc;
  } else if (pv_mode == SAGE_PV_FP8_SMOOTH_V) {
    const VSmoothWs vw{w.vpsum, w.vpmax, w.vpmin, 0};
    if ((rc = run_quantize_v_smooth(p, V, vs, (uint8_t*)(ws + w.v8), w.s8kv, (float*)(ws + w.sv), ws, vw, st)))
      return rc;
    vmean = (const float*)(ws + w.sv) + (size_t)p->nseq * kv_heads_of(p) * to_internal(p).head_dim;
  }
  if (pv_mode != SAGE_PV_FP16) {
    vin = ws + w.v8;
    vin_s = w.s8kv;
    sv = (const float*)(ws + w.sv);
  }
  sage::AttnArgs a{q8, S(p->qk_fp4 ? w.s4q : w.s8q), k8, S(p->qk_fp4 ? w.s4kv : w.s8kv), sq, sk, vin, S(vin_s), sv,
                   out, S(os), nullptr, vmean, p->smooth_q ? (const float*)(ws + w.qdelta) : nullptr, S(w.sqd),
                   p->qk_fp4 ? (const uint8_t*)sq : nullptr, S(w.ssq), p->qk_fp4 ? (const uint8_t*)sk : nullptr,
                   S(w.sskv)};
  hipError_t e = sage::launch_attn(to_internal(p), a, causal != 0, pv_mode != SAGE_PV_FP16, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return SAGE_OK;
}

// ---- sage_attn_noalloc: the workspace in a file-scope device array.  Its
// name is a host-side stand-in, not a device address: host code uses only the
// address hipGetSymbolAddress returns for the current device, fetched at the
// entry's first call on that device and kept per device.
static __device__ __align__(256) unsigned char scratch[SAGE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SAGE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return SAGE_OK;
}
}  // namespace

int sage_attn_noalloc(const sage_problem* p, const void* Q, sage_strides qs, const void* K, sage_strides ks,
                      const void* V, sage_strides vs, void* out, sage_strides os, int causal, float sm_scale,
                      int pv_mode, void* stream) {
  int rc = check_attn_args(p, Q, qs, K, ks, V, vs, out, os, pv_mode);
  if (rc || empty(p)) return rc;
  const size_t need = ws_layout(p, pv_mode).total;
  if (need > SAGE_NOALLOC_SCRATCH_BYTES)
    return fail(SAGE_ERR_WORKSPACE,
                "sage_attn_noalloc: this problem needs %zu bytes of scratch, above the library's fixed %zu-byte "
                "array (use sage_attn with a workspace)",
                need, (size_t)SAGE_NOALLOC_SCRATCH_BYTES);
  char* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws))) return rc;
  return run_attn(p, Q, qs, K, ks, V, vs, out, os, causal, sm_scale, pv_mode, ws, (hipStream_t)stream);
}

int sage_debug_qk_i32(const sage_problem* p, const int8_t* q8, sage_strides q8s, const int8_t* k8, sage_strides k8s,
                      int32_t* s_out, void* stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->cu_seqlens) return fail(SAGE_ERR_UNSUPPORTED, "sage_debug_qk_i32 supports dense problems only");
  if (p->max_seqlen > 1024) return fail(SAGE_ERR_UNSUPPORTED, "sage_debug_qk_i32 supports max_seqlen <= 1024");
  if (empty(p)) return SAGE_OK;
  if ((rc = check_tensor("q8", q8, q8s, 16, p)) || (rc = check_tensor("k8", k8, k8s, 16, p))) return rc;
  if (!s_out || !aligned16(s_out)) return fail(SAGE_ERR_INVALID_ARG, "s_out must be non-NULL and 16-byte aligned");
  if (p->max_seqlen % 4) return fail(SAGE_ERR_UNSUPPORTED, "sage_debug_qk_i32 needs max_seqlen % 4 == 0");
  // scales are not read on the integer path
  sage::AttnArgs a{q8,      S(q8s),  k8,      S(k8s),  nullptr, nullptr, nullptr, sage::Str{0, 0, 0},
                   nullptr, nullptr, sage::Str{0, 0, 0}, s_out, nullptr};
  hipError_t e = sage::launch_attn(to_internal(p), a, false, false, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug qk launch");
  return SAGE_OK;
}

int sage_debug_mxfp4_mfma(const uint8_t* a, const uint8_t* b, const uint8_t* scale_a, const uint8_t* scale_b,
                          const float* c, float* d, void* stream) {
  if (!a || !b || !scale_a || !scale_b || !c || !d) return fail(SAGE_ERR_INVALID_ARG, "operands must not be NULL");
  hipError_t e = sage::launch_debug_mxfp4_mfma(a, b, scale_a, scale_b, c, d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug mxfp4 mfma launch");
  return SAGE_OK;
}

int sage_debug_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, int scale_a, int scale_b, float* d,
                        void* stream) {
  if (!a || !b || !c || !d) return fail(SAGE_ERR_INVALID_ARG, "operands must not be NULL");
  if (scale_a < 0 || scale_a > 254 || scale_b < 0 || scale_b > 254)
    return fail(SAGE_ERR_INVALID_ARG, "E8M0 scales must be in [0, 254] (%d, %d)", scale_a, scale_b);
  hipError_t e = sage::launch_debug_fp8_mfma(a, b, c, scale_a, scale_b, d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "debug fp8 mfma launch");
  return SAGE_OK;
}

}  // extern "C"
