// Pre-pass kernels of SageAttention's forward: smooth K, per-block INT8
// quantisation of Q and K, and the E4M3 V of the FP8 P.V path.
//
// Pages followed:
//   "SageAttention：低比特量化Attention，实现推理加速", section 技术方案,
//     item 1: K minus its mean over tokens, one mean per channel;
//     item 2: INT8 Q and K with one scale per block of rows (the attention
//     kernel's tile size).
//   "4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级", section
//     技术方案 item 4: V quantised to FP8 E4M3; item 1: smoothing Q (Q minus
//     its per-channel mean, the mean's product with K^T added to S).
//
// All of these are HBM-bound streaming passes.  Rounding is fixed so that the
// results are bit-exact against a plain CPU implementation:
//   * K column sums are taken in fp64 (one partial per chunk of tokens, fused with
//     the Q quantisation, then a small reduction); every fp16 value is a
//     multiple of 2^-24 and the sums stay far below 2^29, so each partial sum
//     is exact and the result is independent of the reduction order.  mean =
//     fp32(sum / L) with one IEEE fp64 division.
//   * Q' = fp32(Q * sm_scale), K' = fp32(K - mean): one rounding each.
//   * scale = fp32(absmax / 127) (IEEE fp32 division) and code =
//     rint(fp32(x / scale)) with round-half-to-even; the quotient is taken
//     through the hardware reciprocal except within 2^-13 of a half-integer,
//     where the IEEE division decides (see quant_block); absmax is exact in
//     any order.
//   * E4M3 codes come from the hardware convert (round to nearest even).
#include "sage_internal.h"

namespace sage {
namespace {

constexpr int kThreads = 256;  // E4M3 V kernels

// Cross-lane moves without LDS: DPP within a row of 16 lanes, then gfx950's
// row swaps (permlane16/32_swap).  A chain of LDS permutes instead costs an
// LDS round trip per step.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // lane i^1 (quad_perm [1,0,3,2])
  v = fmaxf(v, dpp_f<0x4E>(v));   // lane i^2 (quad_perm [2,3,0,1])
  v = fmaxf(v, dpp_f<0x141>(v));  // lane 7-i of its 8 (row_half_mirror): max over 8
  v = fmaxf(v, dpp_f<0x140>(v));  // lane 15-i of its 16 (row_mirror): max over the row
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));  // rows 0|1, 2|3
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));  // halves
}

// Block-wide max of a non-negative value (NTH threads).
template <int NTH>
__device__ __forceinline__ float block_max(float v) {
  __shared__ float wm[NTH / 64];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = wm[0];
#pragma unroll
  for (int i = 1; i < NTH / 64; ++i) r = fmaxf(r, wm[i]);
  return r;
}

struct H8 {
  _Float16 v[8];
};

__device__ __forceinline__ H8 load_h8(const _Float16* p) {
  H8 r;
  *reinterpret_cast<uint4*>(&r) = *reinterpret_cast<const uint4*>(p);
  return r;
}

// 8 channels of a row, or zeros for channels past the valid ones (head_dim 96
// runs on the 128-channel kernels with channels 96..127 zero).
__device__ __forceinline__ H8 load_h8_or_zero(const _Float16* p, bool valid) {
  if (valid) return load_h8(p);
  H8 r;
  *reinterpret_cast<uint4*>(&r) = make_uint4(0u, 0u, 0u, 0u);
  return r;
}

// ---------------------------------------------------------------- INT8 blocks
// The INT8 kernels run 512 threads (8 waves, two per SIMD): a text-sized head
// gives one block per CU, and the per-element work then spreads over twice
// the waves.
constexpr int kQThreads = 512;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: M + r for an integer |r| < 2^22 is exact,
                                       // and its bit pattern's low byte is r as int8

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Rows of a block of up to 128 rows held in registers: thread (r, cg) holds
// rows n0 + r + RPP*j, j < R, channels 8cg .. 8cg+7 (n0 < n1).  All loads are
// issued before any is used, so the block costs one memory round trip: a
// slot past the block's end re-reads row n1 - 1 (callers skip those slots).
// Branching around such loads instead puts a wait for each load at the end
// of its branch (the compiler settles pending loads where paths join), which
// turns the R loads into R round trips.
template <int D>
struct BlockRows {
  static constexpr int TPR = D / 8, RPP = kQThreads / TPR, R = 128 / RPP;
  H8 x[R];
  __device__ __forceinline__ void load(const _Float16* __restrict__ src, int64_t sn, int n0, int n1, bool cgv) {
    const int r = threadIdx.x / TPR;
    if (cgv) {
#pragma unroll
      for (int j = 0; j < R; ++j) x[j] = load_h8(src + (int64_t)min(n0 + r + RPP * j, n1 - 1) * sn);
    } else {
#pragma unroll
      for (int j = 0; j < R; ++j) *reinterpret_cast<uint4*>(&x[j]) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
};

// Per-channel maximum and minimum of rows, in fp16 (packed pairs: exact).
struct Extremes {
  v2h hi[4], lo[4];
  __device__ __forceinline__ Extremes() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hi[i] = v2h{(_Float16)-INFINITY, (_Float16)-INFINITY};
      lo[i] = v2h{(_Float16)INFINITY, (_Float16)INFINITY};
    }
  }
  __device__ __forceinline__ void add(const H8& x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v2h p = {x.v[2 * i], x.v[2 * i + 1]};
      hi[i] = __builtin_elementwise_max(hi[i], p);
      lo[i] = __builtin_elementwise_min(lo[i], p);
    }
  }
  // max over the 8 channels of |T(x)| for T monotone non-decreasing: the
  // extremes of T(x) over the rows are T(max) and T(min)
  template <typename F>
  __device__ __forceinline__ float absmax(F transform) const {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float h = transform((float)hi[i >> 1][i & 1], i), l = transform((float)lo[i >> 1][i & 1], i);
      a = fmaxf(a, fmaxf(fabsf(h), fabsf(l)));
    }
    return a;
  }
};

// INT8 codes of one row chunk (8 channels): x' = transform(x) (one fp32
// rounding), code = rint(fp32(x' / scale)) with round-half-to-even.  With y =
// rcp(scale) (at most 1 ulp off) the exact product x' * y is within 2^-16 of
// x' / scale, and fp32(x' / scale) within 2^-17 of it (|x' / scale| < 127.5):
// when x' * y is more than 2^-15 from every half-integer, all of them round
// to the same integer.  fma(x', y, M) with M = 1.5 * 2^23 rounds x' * y to
// that integer r (ties to even; M is even), and fma(x', y, -r) gives the
// residual to within 2^-25; lanes with |residual| > 1/2 - 2^-13 (about 1
// element in 4000) take the IEEE division instead.  |r| <= 127 always (x' <=
// absmax and the errors above stay far below 1/2), so the code is the low
// byte of M + r.
template <typename F>
__device__ __forceinline__ uint2 codes8(const H8& x, F transform, float scale, float y) {
  float xv[8], tv[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xv[i] = transform((float)x.v[i], i);
    tv[i] = __builtin_fmaf(xv[i], y, kMagic);
    near |= fabsf(__builtin_fmaf(xv[i], y, kMagic - tv[i])) > 0.5f - 0x1p-13f;
  }
  if (__builtin_expect(__any(near), 0)) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (fabsf(__builtin_fmaf(xv[i], y, kMagic - tv[i])) > 0.5f - 0x1p-13f)
        tv[i] = __builtin_rintf(xv[i] / scale) + kMagic;
  }
  uint32_t t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = __float_as_uint(tv[i]);
  // low bytes: [t0 t1 t2 t3], [t4 t5 t6 t7]
  const uint32_t w0 = __builtin_amdgcn_perm(t[1], t[0], 0x0c0c0400u) | __builtin_amdgcn_perm(t[3], t[2], 0x04000c0cu);
  const uint32_t w1 = __builtin_amdgcn_perm(t[5], t[4], 0x0c0c0400u) | __builtin_amdgcn_perm(t[7], t[6], 0x04000c0cu);
  return make_uint2(w0, w1);
}

// One quantisation block, rows [n0, n1) of one (sequence, head): thread (r,
// cg) handles rows n0 + r + RPP*j, channels 8cg .. 8cg+7 (16-byte loads).
// transform must be monotone non-decreasing (x * sm_scale with sm_scale > 0,
// or x - mean): the block's absmax of x' then comes from the per-channel fp16
// maximum and minimum.  scale = fp32(absmax / 127); codes as in codes8 (0 when
// the block is all zero).  Blocks of up to 128 rows stay in registers between
// the absmax and the codes (one read of HBM; `pre`: already loaded); longer
// ones are read twice.  Returns the scale.
template <int D, typename F>
__device__ __forceinline__ float quant_block(const _Float16* __restrict__ src, int64_t sn, int n0, int n1,
                                             F transform, int8_t* __restrict__ dst, int64_t dn, bool cgv,
                                             const BlockRows<D>* pre = nullptr) {
  constexpr int TPR = D / 8, RPP = kQThreads / TPR, R = 128 / RPP;
  const int r = threadIdx.x / TPR;
  Extremes ex;
  if (n1 - n0 <= RPP * R) {
    BlockRows<D> rows;
    if (pre)
      rows = *pre;
    else
      rows.load(src, sn, n0, n1, cgv);
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (n0 + r + RPP * j < n1) ex.add(rows.x[j]);
    const float a = block_max<kQThreads>(n0 + r < n1 ? ex.absmax(transform) : 0.0f);
    const float scale = a > 0.0f ? a / 127.0f : 0.0f;
    const float y = __builtin_amdgcn_rcpf(scale);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int n = n0 + r + RPP * j;
      if (n < n1)
        *reinterpret_cast<uint2*>(dst + (int64_t)n * dn) =
            a > 0.0f ? codes8(rows.x[j], transform, scale, y) : make_uint2(0u, 0u);
    }
    return scale;
  }
#pragma unroll 2
  for (int n = n0 + r; n < n1; n += RPP) ex.add(load_h8_or_zero(src + (int64_t)n * sn, cgv));
  const float a = block_max<kQThreads>(n0 + r < n1 ? ex.absmax(transform) : 0.0f);
  const float scale = a > 0.0f ? a / 127.0f : 0.0f;
  const float y = __builtin_amdgcn_rcpf(scale);
#pragma unroll 2
  for (int n = n0 + r; n < n1; n += RPP)
    *reinterpret_cast<uint2*>(dst + (int64_t)n * dn) =
        a > 0.0f ? codes8(load_h8_or_zero(src + (int64_t)n * sn, cgv), transform, scale, y) : make_uint2(0u, 0u);
  return scale;
}

// Exact fp64 column sums of rows [n0, n1) (n1 - n0 <= 128 * NSB) of one
// (sequence, head): thread (r, cg) adds rows n0 + r + RPP*j of channels 8cg ..
// 8cg+7 (base points at channel 8cg of token 0), then the RPP partials of a
// channel are added in LDS and written to out[0 .. D-1].  Every fp16 value is a
// multiple of 2^-24 and |sum| < 2^29, so the sums are exact in any order.
template <int D, int NSB = 1>
__device__ __forceinline__ void colsum_chunk(const _Float16* __restrict__ base, int64_t sn, int n0, int n1, bool cgv,
                                             double* __restrict__ out) {
  constexpr int TPR = D / 8, RPP = kQThreads / TPR;
  const int tid = threadIdx.x, cg = tid % TPR, r = tid / TPR;
  double acc[8] = {};
  {
    // up to NSB blocks of 128 rows; the next block's loads are in flight while a
    // block is added (a block wholly past n1 re-reads row n1 - 1 and adds nothing)
    auto add = [&](const BlockRows<D>& rows, int sb) {
#pragma unroll
      for (int j = 0; j < BlockRows<D>::R; ++j)
        if (n0 + 128 * sb + r + RPP * j < n1)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += (double)(float)rows.x[j].v[i];
    };
    auto blk = [&](int sb) { return min(n0 + 128 * sb, n1 - 1); };
    BlockRows<D> ra, rb;
    ra.load(base, sn, n0, n1, cgv);
    if constexpr (NSB == 1) {
      add(ra, 0);
    } else {
      static_assert(NSB % 2 == 0, "blocks go in pairs");
#pragma unroll 1
      for (int sb = 0; sb < NSB; sb += 2) {
        rb.load(base, sn, blk(sb + 1), n1, cgv);
        add(ra, sb);
        if (sb + 2 < NSB) ra.load(base, sn, blk(sb + 2), n1, cgv);
        add(rb, sb + 1);
      }
    }
  }
  __shared__ double red[RPP][D];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[r][cg * 8 + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < RPP; ++i) t += red[i][tid];
    out[tid] = t;
  }
}

// grid (nkc + nqw, heads, nseq), kQThreads (heads: of Q).  Workgroups x < nkc
// with a K head (y < kv_heads) take the fp64 column sums of K over the tokens
// of chunk x (kKChunkRows tokens), one partial per chunk -- the longest work,
// dispatched first.  Workgroups x >= nkc quantise Q (INT8 Q' = Q * sm_scale):
// block x - nkc of blk_q rows, or for blk_q == 1 (one scale per token) the RPP
// rows (x - nkc)*RPP .. + RPP - 1, TPR threads per row.
template <int D>
__global__ __launch_bounds__(kQThreads) void k_quant_q_colsum(
    const _Float16* __restrict__ Q, Str qs, const _Float16* __restrict__ K, Str ks, const int32_t* __restrict__ cu,
    int max_seqlen, int total, int blk_q, int nbq, int nkc, int nks, int kv_heads, int dv, float sm_scale,
    int8_t* __restrict__ q8, Str q8s,
    float* __restrict__ sq, double* __restrict__ part) {
  constexpr int TPR = D / 8, RPP = kQThreads / TPR;
  const int h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  // x < nqw: Q work; x >= nqw: K chunk x - nqw (dispatched first: blockIdx.x < nkc)
  const int nqw = gridDim.x - nkc;
  const int x = (int)blockIdx.x < nkc ? nqw + (int)blockIdx.x : (int)blockIdx.x - nkc;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int tid = threadIdx.x, cg = tid % TPR, r = tid / TPR;
  const bool cgv = 8 * cg < dv;  // this thread's 8 channels are real (not head_dim 96 padding)
  const int64_t sh = (int64_t)s * H + h;
  // fp32(Q * sm_scale), one rounding of the exact product (as an FMA with a
  // zero addend the fp16 operand is read directly: v_fma_mix_f32)
  auto scale_q = [&](float v, int) { return __builtin_fmaf(v, sm_scale, 0.0f); };
  if (x < nqw && blk_q == 1) {
    // one scale per token: absmax of the row = fp32(max |Q| * sm_scale) (monotone)
    if (x * RPP >= L) return;
    const int n = x * RPP + r;
    const bool valid = n < L;
    H8 row;
    float a = 0.0f;
    if (valid) {
      row = load_h8_or_zero(Q + seq_head_base(cu, qs, s, h, total) + (int64_t)n * qs.n + cg * 8, cgv);
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf((float)row.v[i]));
      a *= sm_scale;
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 64));  // the row's TPR lanes
    if (valid) {
      const float scale = a > 0.0f ? a / 127.0f : 0.0f;
      *reinterpret_cast<uint2*>(q8 + seq_head_base(cu, q8s, s, h, total) + (int64_t)n * q8s.n + cg * 8) =
          a > 0.0f ? codes8(row, scale_q, scale, __builtin_amdgcn_rcpf(scale)) : make_uint2(0u, 0u);
      if (cg == 0) sq[sh * nbq + n] = scale;
    }
    return;
  }
  if (x < nqw) {
    const int n0 = x * blk_q;
    if (n0 >= L) return;
    const int n1 = min(L, n0 + blk_q);
    const float scale = quant_block<D>(Q + seq_head_base(cu, qs, s, h, total) + cg * 8, qs.n, n0, n1, scale_q,
                                       q8 + seq_head_base(cu, q8s, s, h, total) + cg * 8, q8s.n, cgv);
    if (tid == 0) sq[sh * nbq + x] = scale;
    return;
  }
  // K column sums (exact in fp64, in any order), over the K heads only
  if (h >= kv_heads) return;
  const int64_t skv = (int64_t)s * kv_heads + h;
  const int ci = x - nqw;
  const int n0 = ci * kKChunkRows;
  if (n0 >= L) return;
  colsum_chunk<D, kKChunkRows / 128>(K + seq_head_base(cu, ks, s, h, total) + cg * 8, ks.n, n0, min(L, n0 + kKChunkRows),
                                     cgv, part + (skv * nks + ci) * D);
}

// grid (nks, heads, nseq), kQThreads (heads: of Q).  Smooth Q: the fp64 column sums of
// Q (every query head) and of K (the K heads) over chunk x of kKSumRows tokens.
template <int D>
__global__ __launch_bounds__(kQThreads) void k_colsums_qk(const _Float16* __restrict__ Q, Str qs,
                                                          const _Float16* __restrict__ K, Str ks,
                                                          const int32_t* __restrict__ cu, int max_seqlen, int total, int nks,
                                                          int kv_heads, int dv, double* __restrict__ qpart,
                                                          double* __restrict__ kpart) {
  const int ci = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int n0 = ci * kKSumRows;
  if (n0 >= L) return;
  const int n1 = min(L, n0 + kKSumRows);
  const int cg = threadIdx.x % (D / 8);
  const bool cgv = 8 * cg < dv;
  if (qpart)
    colsum_chunk<D>(Q + seq_head_base(cu, qs, s, h, total) + cg * 8, qs.n, n0, n1, cgv,
                    qpart + (((int64_t)s * H + h) * nks + ci) * D);
  if (h < kv_heads) {
    __syncthreads();  // (colsum_chunk's LDS is reused)
    colsum_chunk<D>(K + seq_head_base(cu, ks, s, h, total) + cg * 8, ks.n, n0, n1, cgv,
                    kpart + (((int64_t)s * kv_heads + h) * nks + ci) * D);
  }
}

// Sum of the nb = ceil(L / kKSumRows) partials of channel c of (s, h), by the
// kQThreads / D threads of c (16 independent loads per round), combined in LDS.
template <int D>
__device__ __forceinline__ double sum_partials(const double* __restrict__ pp, int nb, int c, int g) {
  constexpr int G = kQThreads / D;
  double tot = 0.0;
  for (int k0 = g; k0 < nb; k0 += 16 * G) {
    double t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int k = k0 + u * G;
      t[u] = k < nb ? pp[(int64_t)k * D] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) tot += t[u];
  }
  __shared__ double red[G][D];
  red[g][c] = tot;
  __syncthreads();
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < G; ++i) sum += red[i][c];
  return sum;
}

// grid (heads, nseq), kQThreads: mean = fp32((sum / L) * scale) from the
// partials (scale 1: K's mean; sm_scale: the mean of Q' = Q * sm_scale); long
// sequences (shorter ones fold this into the quantisation kernel).
template <int D>
__global__ __launch_bounds__(kQThreads) void k_mean_finalize(const double* __restrict__ part,
                                                             const int32_t* __restrict__ cu, int max_seqlen, int total,
                                                             int nks, int chunk, double scale,
                                                             float* __restrict__ km) {
  const int h = blockIdx.x, s = blockIdx.y, H = gridDim.x, c = threadIdx.x % D, g = threadIdx.x / D;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int nb = (L + chunk - 1) / chunk;
  const double sum = sum_partials<D>(part + ((int64_t)s * H + h) * nks * D + c, nb, c, g);
  if (g == 0) km[((int64_t)s * H + h) * D + c] = L > 0 ? (float)((sum / (double)L) * scale) : 0.0f;
}

// grid (nqw, heads, nseq), kQThreads: INT8 Q_s = fp32(fp32(Q * sm_scale) - qm)
// with qm = mean(Q') (smooth Q), per block of blk_q rows or, blk_q == 1, per
// token (RPP rows per workgroup).  FOLD: every workgroup sums its head's
// column partials itself (the first stores q_mean); otherwise q_mean comes
// from k_mean_finalize.
template <int D, bool FOLD>
__global__ __launch_bounds__(kQThreads) void k_quant_q_smooth(const _Float16* __restrict__ Q, Str qs,
                                                              const int32_t* __restrict__ cu, int max_seqlen, int total,
                                                              int blk_q, int nbq, int nks, int dv, float sm_scale,
                                                              const double* __restrict__ qpart,
                                                              float* __restrict__ qmean, int8_t* __restrict__ q8,
                                                              Str q8s, float* __restrict__ sq) {
  constexpr int TPR = D / 8, RPP = kQThreads / TPR;
  const int x = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int tid = threadIdx.x, cg = tid % TPR, r = tid / TPR;
  const bool cgv = 8 * cg < dv;
  const int64_t sh = (int64_t)s * H + h;
  const int n0 = blk_q == 1 ? x * RPP : x * blk_q;
  if (n0 >= L) return;
  float mean[8];
  if constexpr (FOLD) {
    __shared__ float qm[D];
    const int c = tid % D, g = tid / D;
    const double sum = sum_partials<D>(qpart + sh * nks * D + c, (L + kKSumRows - 1) / kKSumRows, c, g);
    if (g == 0) {
      const float mv = (float)((sum / (double)L) * (double)sm_scale);
      qm[c] = mv;
      if (x == 0) qmean[sh * D + c] = mv;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) mean[i] = qm[cg * 8 + i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) mean[i] = qmean[sh * D + cg * 8 + i];
  }
  // two roundings: the product is not contracted with the subtraction into one
  // fma (device code contracts by default); monotone non-decreasing in x
  auto smooth = [&](float v, int i) {
#pragma clang fp contract(off)
    return v * sm_scale - mean[i];
  };
  if (blk_q == 1) {
    const int n = n0 + r;
    const bool valid = n < L;
    H8 row;
    float a = 0.0f;
    if (valid) {
      row = load_h8_or_zero(Q + seq_head_base(cu, qs, s, h, total) + (int64_t)n * qs.n + cg * 8, cgv);
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(smooth((float)row.v[i], i)));
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 64));  // the row's TPR lanes
    if (valid) {
      const float scale = a > 0.0f ? a / 127.0f : 0.0f;
      *reinterpret_cast<uint2*>(q8 + seq_head_base(cu, q8s, s, h, total) + (int64_t)n * q8s.n + cg * 8) =
          a > 0.0f ? codes8(row, smooth, scale, __builtin_amdgcn_rcpf(scale)) : make_uint2(0u, 0u);
      if (cg == 0) sq[sh * nbq + n] = scale;
    }
    return;
  }
  const float scale = quant_block<D>(Q + seq_head_base(cu, qs, s, h, total) + cg * 8, qs.n, n0, min(L, n0 + blk_q), smooth,
                                     q8 + seq_head_base(cu, q8s, s, h, total) + cg * 8, q8s.n, cgv);
  if (tid == 0) sq[sh * nbq + x] = scale;
}

// grid (ceil(max_seqlen / 128), heads, nseq), kQThreads (heads: of Q).  The
// compensation of smoothing Q for 128 keys of one (sequence, query head):
// delta_j = sum_c qm_c * fp32(K_jc - km_c), products exact in fp64, added in
// fp64 (channels in order within a thread, then a butterfly over the row's
// TPR lanes), rounded once to fp32.
template <int D>
__global__ __launch_bounds__(kQThreads) void k_q_delta(const _Float16* __restrict__ K, Str ks,
                                                       const int32_t* __restrict__ cu, int max_seqlen, int total, int kv_heads,
                                                       int dv, const float* __restrict__ qmean,
                                                       const float* __restrict__ kmean, float* __restrict__ qdelta,
                                                       Str qds) {
  constexpr int TPR = D / 8, RPP = kQThreads / TPR, R = 128 / RPP;
  const int h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int kvh = h / (H / kv_heads);
  const int L = seq_len(cu, s, max_seqlen, total);
  const int n0 = blockIdx.x * 128;
  if (n0 >= L) return;
  const int tid = threadIdx.x, cg = tid % TPR, r = tid / TPR;
  const bool cgv = 8 * cg < dv;
  float qm[8], km[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    qm[i] = qmean[((int64_t)s * H + h) * D + cg * 8 + i];
    km[i] = kmean[((int64_t)s * kv_heads + kvh) * D + cg * 8 + i];
  }
  BlockRows<D> rows;
  rows.load(K + seq_head_base(cu, ks, s, kvh, total) + cg * 8, ks.n, n0, min(L, n0 + 128), cgv);
  float* const out = qdelta + seq_head_base(cu, qds, s, h, total);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int n = n0 + r + RPP * j;
    double t = 0.0;
    if (n < L)
#pragma unroll
      for (int i = 0; i < 8; ++i) t += (double)qm[i] * (double)((float)rows.x[j].v[i] - km[i]);
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) t += __shfl_xor(t, m, 64);
    if (n < L && cg == 0) out[n] = (float)t;
  }
}

// grid (nbk, kv heads, nseq), kQThreads: K block bi -> INT8 K' = K - mean(K).
// FOLD: the workgroup sums the column partials itself (every block of the
// head does; block 0 stores k_mean), with the block's K rows already in
// flight; otherwise k_mean comes from k_mean_finalize.
template <int D, bool FOLD>
__global__ __launch_bounds__(kQThreads) void k_quant_k(const _Float16* __restrict__ K, Str ks,
                                                       const int32_t* __restrict__ cu, int max_seqlen, int total, int blk_k,
                                                       int nbk, int nks, int chunk, int dv,
                                                       const double* __restrict__ part,
                                                       float* __restrict__ km, int8_t* __restrict__ k8, Str k8s,
                                                       float* __restrict__ sk) {
  constexpr int TPR = D / 8;
  // heads and sequences in the reverse of k_quant_q_colsum's order: the K rows
  // that pass read last are read again first, while the memory-side cache may
  // still hold them
  const int bi = blockIdx.x, H = gridDim.y, h = H - 1 - blockIdx.y, s = gridDim.z - 1 - blockIdx.z;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int n0 = bi * blk_k;
  if (n0 >= L) return;
  const int n1 = min(L, n0 + blk_k);
  const int cg = threadIdx.x % TPR;
  const int64_t sh = (int64_t)s * H + h;
  const _Float16* kb = K + seq_head_base(cu, ks, s, h, total) + cg * 8;
  const bool cgv = 8 * cg < dv;
  BlockRows<D> krows;
  const bool pre = n1 - n0 <= 128;
  if (pre) krows.load(kb, ks.n, n0, n1, cgv);
  float mean[8];
  if constexpr (FOLD) {
    __shared__ float kmean[D];
    const int c = threadIdx.x % D, g = threadIdx.x / D;
    const double sum = sum_partials<D>(part + sh * nks * D + c, (L + chunk - 1) / chunk, c, g);
    if (g == 0) {
      const float mv = (float)(sum / (double)L);
      kmean[c] = mv;
      if (bi == 0) km[sh * D + c] = mv;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) mean[i] = kmean[cg * 8 + i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) mean[i] = km[sh * D + cg * 8 + i];
  }
  const float scale = quant_block<D>(kb, ks.n, n0, n1, [&](float v, int i) { return v - mean[i]; },
                                     k8 + seq_head_base(cu, k8s, s, h, total) + cg * 8, k8s.n, cgv, pre ? &krows : nullptr);
  if (threadIdx.x == 0) sk[sh * nbk + bi] = scale;
}

// ---------------------------------------------------------------- MXFP4 Q and K
// 4-bit Q and K ("4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级",
// 技术方案: the INT4 kernel) in the 4-bit matrix format of gfx950, OCP MXFP4:
// per row, per block of 32 channels, an E8M0 exponent e = floor(log2 max|x|) - 2
// (code e + 127, clamped to [0, 254]; 0 for an all-zero block) and E2M1
// elements RNE(x / 2^e), ties to the even code, saturating at 6, sign bit from
// x.  x / 2^e is exact (a power-of-two scaling whose result is either normal
// or far below the smallest E2M1 step).

// E2M1 code of y (|y| compared with the midpoints of 0, 0.5, 1, 1.5, 2, 3, 4, 6;
// a midpoint goes to the even code).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t mag = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return mag | ((__float_as_uint(y) >> 28) & 0x8u);
}

// grid (ceil(max_seqlen / RPP), heads, nseq), kQThreads: thread (r, cg) quantises
// channels 8cg .. 8cg+7 of row x*RPP + r of x' = transform(x) (Q: fp32(Q *
// sm_scale), minus q_mean when smoothing Q; K: fp32(K - k_mean)); a block of 32
// channels is 4 neighbouring threads.  Writes the 8 codes as one dword (element
// c at nibble c) at byte 4cg of the row in x4 (row stride x4s.n bytes) and the
// block's E8M0 code at byte cg/4 of the row in xsc (row stride xss.n bytes).
template <int D, bool IS_Q>
__global__ __launch_bounds__(kQThreads) void k_quant_mxfp4(const _Float16* __restrict__ X, Str xs,
                                                           const int32_t* __restrict__ cu, int max_seqlen, int total, int dv,
                                                           float sm_scale, const float* __restrict__ mean,
                                                           uint8_t* __restrict__ x4, Str x4s, uint8_t* __restrict__ xsc,
                                                           Str xss) {
  constexpr int TPR = D / 8, RPP = kQThreads / TPR;
  const int h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int tid = threadIdx.x, cg = tid % TPR, n = blockIdx.x * RPP + tid / TPR;
  if (blockIdx.x * RPP >= L) return;
  const bool valid = n < L;
  float mu[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mu[i] = mean ? mean[((int64_t)s * H + h) * D + cg * 8 + i] : 0.0f;
  float xv[8] = {};
  float a = 0.0f;
  if (valid) {
    const H8 row = load_h8_or_zero(X + seq_head_base(cu, xs, s, h, total) + (int64_t)n * xs.n + cg * 8, 8 * cg < dv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
      const float v = (float)row.v[i];
      xv[i] = IS_Q ? (v * sm_scale - mu[i]) : (v - mu[i]);
      a = fmaxf(a, fabsf(xv[i]));
    }
  }
  a = fmaxf(a, __shfl_xor(a, 1, 64));  // the block's 4 threads
  a = fmaxf(a, __shfl_xor(a, 2, 64));
  if (!valid) return;
  int code = 0;
  if (a > 0.0f) {
    int k;
    (void)frexpf(a, &k);  // a = m 2^k, m in [0.5, 1): floor(log2 a) = k - 1
    code = min(254, max(0, 127 + (k - 1) - 2));
  }
  uint32_t w = 0;
  if (code > 0 || a > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= e2m1_code(ldexpf(xv[i], 127 - code)) << (4 * i);
  }
  *reinterpret_cast<uint32_t*>(x4 + seq_head_base(cu, x4s, s, h, total) + (int64_t)n * x4s.n + 4 * cg) = w;
  if ((cg & 3) == 0) xsc[seq_head_base(cu, xss, s, h, total) + (int64_t)n * xss.n + cg / 4] = (uint8_t)code;
}

// ---------------------------------------------------------------- E4M3 V
// v_scale is first filled with 0, then each chunk folds its per-channel
// max|V| in with an unsigned atomic max on the float bit pattern (for
// non-negative floats the bit patterns order like the values, and max is
// exact, so the result does not depend on the order), then k_v_scale divides
// by 448 in place.
__global__ void k_fill_zero(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0.0f;
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_v_colmax(const _Float16* __restrict__ V, Str vs,
                                                        const int32_t* __restrict__ cu, int max_seqlen, int total, int dv,
                                                        float* __restrict__ vmax) {
  constexpr int TPR = D / 8, RPP = kThreads / TPR;
  const int chunk = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int n0 = chunk * kColChunk;
  if (n0 >= L) return;
  const int n1 = min(L, n0 + kColChunk);
  const int tid = threadIdx.x, cg = tid % TPR, r = tid / TPR;
  const _Float16* base = V + seq_head_base(cu, vs, s, h, total) + cg * 8;
  float m[8] = {};
  if (8 * cg < dv) {  // padding channels (head_dim 96) keep 0; the test stays outside the loop so that
                      // the unrolled loads issue together
#pragma unroll 4
    for (int n = n0 + r; n < n1; n += RPP) {
      const H8 x = load_h8(base + (int64_t)n * vs.n);
#pragma unroll
      for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf((float)x.v[i]));
    }
  }
  __shared__ float red[RPP][D];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[r][cg * 8 + i] = m[i];
  __syncthreads();
  if (tid < D) {
    float t = 0.0f;
    for (int i = 0; i < RPP; ++i) t = fmaxf(t, red[i][tid]);
    atomicMax(reinterpret_cast<unsigned int*>(vmax + ((int64_t)s * H + h) * D + tid), __float_as_uint(t));
  }
}

__global__ void k_v_scale(float* __restrict__ sv, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) sv[i] = sv[i] / 448.0f;
}

// grid (nchunk, kv heads, nseq): E4M3 codes of V (vmean != nullptr: of V' =
// fp32(V - vmean), the smoothed V) with the per-channel scales sv.
template <int D>
__global__ __launch_bounds__(kThreads) void k_quant_v(const _Float16* __restrict__ V, Str vs,
                                                       const int32_t* __restrict__ cu, int max_seqlen, int total, int dv,
                                                       const float* __restrict__ sv,
                                                       const float* __restrict__ vmean, uint8_t* __restrict__ v8,
                                                       Str v8s) {
  constexpr int TPR = D / 8, RPP = kThreads / TPR;
  const int chunk = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int n0 = chunk * kColChunk;
  if (n0 >= L) return;
  const int n1 = min(L, n0 + kColChunk);
  const int tid = threadIdx.x, cg = tid % TPR, r = tid / TPR;
  const _Float16* src = V + seq_head_base(cu, vs, s, h, total) + cg * 8;
  uint8_t* dst = v8 + seq_head_base(cu, v8s, s, h, total) + cg * 8;
  float scale[8], mean[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    scale[i] = sv[((int64_t)s * H + h) * D + cg * 8 + i];
    mean[i] = vmean ? vmean[((int64_t)s * H + h) * D + cg * 8 + i] : 0.0f;
  }
  auto codes = [&](const H8& x) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = scale[i] > 0.0f ? ((float)x.v[i] - mean[i]) / scale[i] : 0.0f;
    uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    return make_uint2(w0, w1);
  };
  if (8 * cg < dv) {  // the channel test stays outside the loop so that the unrolled loads issue together
#pragma unroll 2
    for (int n = n0 + r; n < n1; n += RPP)
      *reinterpret_cast<uint2*>(dst + (int64_t)n * v8s.n) = codes(load_h8(src + (int64_t)n * vs.n));
  } else {  // padding channels (head_dim 96): the codes of zeros
    H8 z;
    *reinterpret_cast<uint4*>(&z) = make_uint4(0u, 0u, 0u, 0u);
    const uint2 c = codes(z);
    for (int n = n0 + r; n < n1; n += RPP) *reinterpret_cast<uint2*>(dst + (int64_t)n * v8s.n) = c;
  }
}

// ---------------------------------------------------------------- smoothed E4M3 V
// Smooth V (the optional V smoothing described after 技术方案 on the
// SageAttention2 page): mean(V) per channel as for K (exact fp64 sums, one
// fp64 divide, fp32), V' = fp32(V - mean), then the per-channel E4M3 scale
// of V'.  x -> fp32(x - mean) is monotone, so max|V'| of a channel comes from
// its fp16 maximum and minimum.

// grid (nchunk, kv heads, nseq), kThreads: per chunk of kColChunk tokens and
// channel, the exact fp64 sum and the fp16 maximum and minimum (as float).
template <int D>
__global__ __launch_bounds__(kThreads) void k_v_colstats(const _Float16* __restrict__ V, Str vs,
                                                          const int32_t* __restrict__ cu, int max_seqlen, int total, int dv,
                                                          int nchunk,
                                                          double* __restrict__ psum, float* __restrict__ pmax,
                                                          float* __restrict__ pmin) {
  constexpr int TPR = D / 8, RPP = kThreads / TPR;
  const int chunk = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int n0 = chunk * kColChunk;
  if (n0 >= L) return;
  const int n1 = min(L, n0 + kColChunk);
  const int tid = threadIdx.x, cg = tid % TPR, r = tid / TPR;
  const _Float16* base = V + seq_head_base(cu, vs, s, h, total) + cg * 8;
  double acc[8] = {};
  Extremes ex;
  if (8 * cg < dv) {  // the channel test stays outside the loop so that the unrolled loads issue together
#pragma unroll 4
    for (int n = n0 + r; n < n1; n += RPP) {
      const H8 x = load_h8(base + (int64_t)n * vs.n);
      ex.add(x);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += (double)(float)x.v[i];
    }
  } else if (n0 + r < n1) {  // padding channels (head_dim 96): sums 0, maximum and minimum 0
    H8 z;
    *reinterpret_cast<uint4*>(&z) = make_uint4(0u, 0u, 0u, 0u);
    ex.add(z);
  }
  __shared__ double rsum[RPP][D];
  __shared__ float rmax[RPP][D], rmin[RPP][D];
  const bool any = n0 + r < n1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    rsum[r][cg * 8 + i] = acc[i];
    rmax[r][cg * 8 + i] = any ? (float)ex.hi[i >> 1][i & 1] : -INFINITY;
    rmin[r][cg * 8 + i] = any ? (float)ex.lo[i >> 1][i & 1] : INFINITY;
  }
  __syncthreads();
  if (tid < D) {
    double t = 0.0;
    float hi = -INFINITY, lo = INFINITY;
#pragma unroll
    for (int i = 0; i < RPP; ++i) {
      t += rsum[i][tid];
      hi = fmaxf(hi, rmax[i][tid]);
      lo = fminf(lo, rmin[i][tid]);
    }
    const int64_t o = (((int64_t)s * H + h) * nchunk + chunk) * D + tid;
    psum[o] = t;
    pmax[o] = hi;
    pmin[o] = lo;
  }
}

// grid (kv heads, nseq), D threads: mean = fp32(sum / L); scale = fp32(max(|fp32(max -
// mean)|, |fp32(min - mean)|) / 448) per channel (0 for an empty sequence).
template <int D>
__global__ __launch_bounds__(D) void k_v_finalize(const double* __restrict__ psum, const float* __restrict__ pmax,
                                                  const float* __restrict__ pmin, const int32_t* __restrict__ cu,
                                                  int max_seqlen, int total, int nchunk, float* __restrict__ sv,
                                                  float* __restrict__ vmean) {
  const int h = blockIdx.x, s = blockIdx.y, H = gridDim.x, c = threadIdx.x;
  const int L = seq_len(cu, s, max_seqlen, total);
  const int64_t sh = (int64_t)s * H + h;
  if (L <= 0) {
    sv[sh * D + c] = 0.0f;
    vmean[sh * D + c] = 0.0f;
    return;
  }
  const int nc = (L + kColChunk - 1) / kColChunk;
  double t = 0.0;
  float hi = -INFINITY, lo = INFINITY;
  for (int k = 0; k < nc; ++k) {
    const int64_t o = (sh * nchunk + k) * D + c;
    t += psum[o];
    hi = fmaxf(hi, pmax[o]);
    lo = fminf(lo, pmin[o]);
  }
  const float mean = (float)(t / (double)L);
  const float a = fmaxf(fabsf(hi - mean), fabsf(lo - mean));
  sv[sh * D + c] = a / 448.0f;
  vmean[sh * D + c] = mean;
}

}  // namespace

// ---------------------------------------------------------------- launchers

#define SAGE_DISPATCH_D(D_, ...)         \
  do {                                   \
    if ((D_) == 64) {                    \
      constexpr int D = 64;              \
      __VA_ARGS__;                       \
    } else {                             \
      constexpr int D = 128;             \
      __VA_ARGS__;                       \
    }                                    \
  } while (0)

// Heads with at most this many K column-sum partials fold the mean into k_quant_k.
constexpr int kFoldMaxBlocks = 64;
// Sequences up to this many tokens fold the K mean into k_quant_k (each of its workgroups
// adds at most 64 partials of kKSumRows tokens, or 16 of kKChunkRows).
constexpr int kFoldMaxTokens = kFoldMaxBlocks * kKSumRows;

hipError_t launch_quant_q_colsum(const Problem& p, const void* Q, Str qs, const void* K, Str ks, float sm_scale,
                                 int8_t* q8, Str q8s, float* q_scale, double* partial, hipStream_t st) {
  SAGE_DISPATCH_D(p.head_dim, {
    constexpr int RPP = kQThreads / (D / 8);  // rows per workgroup of the per-token path
    const int nqw = p.blk_q == 1 ? (p.max_seqlen + RPP - 1) / RPP : p.nbq;
    const int nkc = (p.max_seqlen + kKChunkRows - 1) / kKChunkRows;  // K column-sum chunks per head
    hipLaunchKernelGGL((k_quant_q_colsum<D>), dim3(nkc + nqw, p.heads, p.nseq), dim3(kQThreads), 0, st,
                       (const _Float16*)Q, qs, (const _Float16*)K, ks, p.cu, p.max_seqlen, p.total, p.blk_q, p.nbq, nkc,
                       p.nks, p.kv_heads, p.dv, sm_scale, q8, q8s, q_scale, partial);
  });
  return hipGetLastError();
}

hipError_t launch_quant_k(const Problem& p, const void* K, Str ks, const double* partial, int chunk, float* k_mean,
                          int8_t* k8, Str k8s, float* k_scale, hipStream_t st) {
  dim3 grid(p.nbk, p.kv_heads, p.nseq);
  if (p.max_seqlen <= kFoldMaxTokens) {
    SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_quant_k<D, true>), grid, dim3(kQThreads), 0, st,
                                                   (const _Float16*)K, ks, p.cu, p.max_seqlen, p.total, p.blk_k, p.nbk, p.nks,
                                                   chunk, p.dv, partial, k_mean, k8, k8s, k_scale));
    return hipGetLastError();
  }
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_mean_finalize<D>), dim3(p.kv_heads, p.nseq), dim3(kQThreads), 0, st,
                                                 partial, p.cu, p.max_seqlen, p.total, p.nks, chunk, 1.0, k_mean));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_quant_k<D, false>), grid, dim3(kQThreads), 0, st,
                                                 (const _Float16*)K, ks, p.cu, p.max_seqlen, p.total, p.blk_k, p.nbk, p.nks,
                                                 chunk, p.dv, partial, k_mean, k8, k8s, k_scale));
  return hipGetLastError();
}

hipError_t launch_quant_q_smooth(const Problem& p, const void* Q, Str qs, const void* K, Str ks, float sm_scale,
                                 int8_t* q8, Str q8s, float* q_scale, float* q_mean, double* qpart, double* kpart,
                                 hipStream_t st) {
  hipError_t e;
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_colsums_qk<D>), dim3(p.nks, p.heads, p.nseq), dim3(kQThreads), 0,
                                                 st, (const _Float16*)Q, qs, (const _Float16*)K, ks, p.cu,
                                                 p.max_seqlen, p.total, p.nks, p.kv_heads, p.dv, qpart, kpart));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  SAGE_DISPATCH_D(p.head_dim, {
    constexpr int RPP = kQThreads / (D / 8);
    const int nqw = p.blk_q == 1 ? (p.max_seqlen + RPP - 1) / RPP : p.nbq;
    const dim3 grid(nqw, p.heads, p.nseq);
    if (p.nks <= kFoldMaxBlocks) {
      hipLaunchKernelGGL((k_quant_q_smooth<D, true>), grid, dim3(kQThreads), 0, st, (const _Float16*)Q, qs, p.cu,
                         p.max_seqlen, p.total, p.blk_q, p.nbq, p.nks, p.dv, sm_scale, qpart, q_mean, q8, q8s, q_scale);
    } else {
      hipLaunchKernelGGL((k_mean_finalize<D>), dim3(p.heads, p.nseq), dim3(kQThreads), 0, st, qpart, p.cu,
                         p.max_seqlen, p.total, p.nks, kKSumRows, (double)sm_scale, q_mean);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL((k_quant_q_smooth<D, false>), grid, dim3(kQThreads), 0, st, (const _Float16*)Q, qs, p.cu,
                         p.max_seqlen, p.total, p.blk_q, p.nbq, p.nks, p.dv, sm_scale, qpart, q_mean, q8, q8s, q_scale);
    }
  });
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4(const Problem& p, const void* Q, Str qs, const void* K, Str ks, float sm_scale,
                              uint8_t* q4, Str q4s, uint8_t* qsc, Str qss, uint8_t* k4, Str k4s, uint8_t* ksc, Str kss,
                              float* k_mean, float* q_mean, double* kpart, double* qpart, hipStream_t st) {
  hipError_t e;
  SAGE_DISPATCH_D(p.head_dim, {
    constexpr int RPP = kQThreads / (D / 8);
    const int nx = (p.max_seqlen + RPP - 1) / RPP;
    hipLaunchKernelGGL((k_colsums_qk<D>), dim3(p.nks, p.heads, p.nseq), dim3(kQThreads), 0, st, (const _Float16*)Q, qs,
                       (const _Float16*)K, ks, p.cu, p.max_seqlen, p.total, p.nks, p.kv_heads, p.dv,
                       p.smooth_q ? qpart : nullptr, kpart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_mean_finalize<D>), dim3(p.kv_heads, p.nseq), dim3(kQThreads), 0, st, kpart, p.cu,
                       p.max_seqlen, p.total, p.nks, kKSumRows, 1.0, k_mean);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.smooth_q) {
      hipLaunchKernelGGL((k_mean_finalize<D>), dim3(p.heads, p.nseq), dim3(kQThreads), 0, st, qpart, p.cu,
                         p.max_seqlen, p.total, p.nks, kKSumRows, (double)sm_scale, q_mean);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_quant_mxfp4<D, true>), dim3(nx, p.heads, p.nseq), dim3(kQThreads), 0, st,
                       (const _Float16*)Q, qs, p.cu, p.max_seqlen, p.total, p.dv, sm_scale, p.smooth_q ? q_mean : nullptr, q4,
                       q4s, qsc, qss);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_quant_mxfp4<D, false>), dim3(nx, p.kv_heads, p.nseq), dim3(kQThreads), 0, st,
                       (const _Float16*)K, ks, p.cu, p.max_seqlen, p.total, p.dv, 1.0f, k_mean, k4, k4s, ksc, kss);
  });
  return hipGetLastError();
}

hipError_t launch_q_delta(const Problem& p, const void* K, Str ks, const float* q_mean, const float* k_mean,
                          float* q_delta, Str qds, hipStream_t st) {
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_q_delta<D>), dim3((p.max_seqlen + 127) / 128, p.heads, p.nseq),
                                                 dim3(kQThreads), 0, st, (const _Float16*)K, ks, p.cu, p.max_seqlen, p.total,
                                                 p.kv_heads, p.dv, q_mean, k_mean, q_delta, qds));
  return hipGetLastError();
}

hipError_t launch_v_colmax(const Problem& p, const void* V, Str vs, float* vmax, hipStream_t st) {
  const int64_t n = (int64_t)p.nseq * p.kv_heads * p.head_dim;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, vmax, n);
  dim3 grid(p.nchunk, p.kv_heads, p.nseq);
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_v_colmax<D>), grid, dim3(kThreads), 0, st,
                                                 (const _Float16*)V, vs, p.cu, p.max_seqlen, p.total, p.dv, vmax));
  return hipGetLastError();
}

hipError_t launch_v_scale(const Problem& p, float* v_scale, hipStream_t st) {
  const int64_t n = (int64_t)p.nseq * p.kv_heads * p.head_dim;
  hipLaunchKernelGGL(k_v_scale, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, v_scale, n);
  return hipGetLastError();
}

hipError_t launch_quant_v(const Problem& p, const void* V, Str vs, const float* v_scale, const float* v_mean,
                          uint8_t* v8, Str v8s, hipStream_t st) {
  dim3 grid(p.nchunk, p.kv_heads, p.nseq);
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_quant_v<D>), grid, dim3(kThreads), 0, st,
                                                 (const _Float16*)V, vs, p.cu, p.max_seqlen, p.total, p.dv, v_scale, v_mean,
                                                 v8, v8s));
  return hipGetLastError();
}

hipError_t launch_v_smooth_stats(const Problem& p, const void* V, Str vs, double* psum, float* pmax, float* pmin,
                                 float* v_scale, float* v_mean, hipStream_t st) {
  dim3 grid(p.nchunk, p.kv_heads, p.nseq);
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_v_colstats<D>), grid, dim3(kThreads), 0, st,
                                                 (const _Float16*)V, vs, p.cu, p.max_seqlen, p.total, p.dv, p.nchunk, psum,
                                                 pmax, pmin));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SAGE_DISPATCH_D(p.head_dim, hipLaunchKernelGGL((k_v_finalize<D>), dim3(p.kv_heads, p.nseq), dim3(D), 0, st, psum,
                                                 pmax, pmin, p.cu, p.max_seqlen, p.total, p.nchunk, v_scale, v_mean));
  return hipGetLastError();
}

}  // namespace sage
