// Fused SageAttention forward kernel for gfx950 (MI355X).
//
// Pages followed:
//   "SageAttention：低比特量化Attention，实现推理加速", section 技术方案: INT8
//     Q K^T with an INT32 accumulator on per-block quantised Q and smoothed K
//     (item 2); P.V kept at 16 bits (item 3: the pages use an FP16
//     accumulator; CDNA4's fp16 MFMA accumulates in fp32, which is used here).
//   "4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级", section
//     技术方案 item 4: FP8 E4M3 P and V for the P.V product.
//   "如何将SageAttention量化注意力机制集成到你的AI项目中获得2-5倍速度提升",
//     section 针对不同AI任务的优化建议: causal mode and packed varlen sequences.
//
// One workgroup = NW waves, each owning RG groups of 32 query rows of one
// (sequence, head); the workgroup walks 64-key tiles of K and V staged in LDS.
//
// Per 64-key tile and 32-row group, on the matrix cores:
//   S^T[key][query] += K[key][c] . Q[query][c]   v_mfma_i32_32x32x32_i8
//   O^T[c][query]   += V^T[c][key] . P^T[key][query]
//                      v_mfma_f32_32x32x16_f16 (fp16 P, V) or
//                      v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 P, V; unit scales)
// Computing the transposes puts one query row in each lane (lanes l and l+32
// share row l%32), so the online-softmax state (m, l) and the rescale of O
// are lane-local, and P leaves the i32 accumulator layout already in the
// B-operand layout of the P.V instruction: no LDS round trip for P.
//
// Key order inside an MFMA: for S^T tile jt (32 keys), lane (row i, half g =
// lane/32) holds accumulator r = 0..15 for key 32jt + 8(r/4) + 4g + r%4.
// Both contraction operands of the P.V instruction only need the SAME key for
// the same (lane half, k slot); V's operand is read to match:
//   fp16: V stays row-major in LDS ([key][channel]) and ds_read_b64_tr_b16
//         transposes 4x16 blocks on the read (two reads per operand).
//   fp8:  V is written to LDS transposed ([channel][permuted key]) so each
//         lane's 32 key bytes are contiguous.
//
// Softmax: x = S_int * (q_scale * k_scale * log2 e) in fp32; m = running row
// max; p = exp2(x - m); alpha = exp2(m_old - m_new); l and O rescaled by
// alpha.  FP8 path: m is rounded up to an integer so alpha is a power of two
// and E4M3(448 p) does not depend on the tile order.
#include "sage_internal.h"

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int BN = 64;  // keys per tile

template <int D, int RG, int NW, bool FP8, bool CAUSAL, bool DUMP>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * RG * 32;
  static constexpr int KROW = D + 16;                       // bytes per K row in LDS
  static constexpr int VROW = FP8 ? (BN + 16) : (2 * D + 32);  // fp8: channel rows; fp16: key rows
  static constexpr int VROWS = FP8 ? D : BN;
  static constexpr int KCH = BN * D / 16;                   // 16-byte chunks per K tile
  static constexpr int KPT = (KCH + NT - 1) / NT;
  // V tile: fp16 = 16-byte chunks of key rows; fp8 = items of 4 keys x 8 channels
  static constexpr int VITEMS = FP8 ? (BN / 4) * (D / 8) : BN * D * 2 / 16;
  static constexpr int VPT = (VITEMS + NT - 1) / NT;
  static constexpr int VLOADS = FP8 ? 4 : 1;                // loads per item
};

__device__ __forceinline__ int pos8(int kq) {  // LDS position of key quad kq in an fp8 V^T row
  return 32 * (kq & 1) + 16 * (kq >> 3) + 4 * ((kq & 7) >> 1);
}

template <int D, int RG, int NW, bool FP8, bool CAUSAL, bool DUMP>
__global__ __launch_bounds__(NW * 64) void k_attn(Problem p, AttnArgs a) {
  using C = Cfg<D, RG, NW, FP8, CAUSAL, DUMP>;
  constexpr int NT = C::NT, BM = C::BM, KROW = C::KROW, VROW = C::VROW;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[BN * KROW];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[DUMP ? 16 : C::VROWS * VROW];

  const int h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int qt = CAUSAL ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int L = seq_len(p.cu, s, p.max_seqlen);
  const int q0 = qt * BM;
  if (q0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 31, g = lane >> 5;
  const int64_t sh = (int64_t)s * H + h;

  const int8_t* __restrict__ qbase = a.q8 + seq_head_base(p.cu, a.q8s, s, h);
  const int8_t* __restrict__ kbase = a.k8 + seq_head_base(p.cu, a.k8s, s, h);
  const uint8_t* __restrict__ vbase =
      DUMP ? nullptr : (const uint8_t*)a.v + seq_head_base(p.cu, a.vs, s, h) * (FP8 ? 1 : 2);
  const int64_t kn = a.k8s.n, vn = a.vs.n * (FP8 ? 1 : 2);  // row strides in bytes
  const float* __restrict__ ksc = a.k_scale + sh * p.nbk;

  // ---- Q fragments (B operand of S^T): lane holds row i, channels 32kk + 16g .. +16
  v4i qf[RG][D / 32];
  float qsc[RG];
  int row0[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    row0[rg] = q0 + (w * RG + rg) * 32;
    const int i = row0[rg] + li;
    if (i < L) {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        qf[rg][kk] = *reinterpret_cast<const v4i*>(qbase + (int64_t)i * a.q8s.n + 32 * kk + 16 * g);
      qsc[rg] = DUMP ? 0.0f : a.q_scale[sh * p.nbq + i / p.blk_q] * kLog2e;
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qf[rg][kk] = v4i{0, 0, 0, 0};
      qsc[rg] = 0.0f;
    }
  }

  const int kv_end = CAUSAL ? min(L, q0 + BM) : L;
  const int ntiles = (kv_end + BN - 1) / BN;

  float m[RG], lsum[RG];
  v16f o[RG][D / 32];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m[rg] = -INFINITY;
    lsum[rg] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) o[rg][ct] = v16f{};
  }

  // ---- global -> register prefetch of one K/V tile
  uint4 kreg[C::KPT];
  uint4 vreg16[FP8 || DUMP ? 1 : C::VPT];
  uint2 vreg8[FP8 ? C::VPT * 4 : 1];
  auto gload = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int x = 0; x < C::KPT; ++x) {
      const int idx = tid + x * NT;
      const int r = idx / (D / 16), c = idx % (D / 16);
      uint4 val = make_uint4(0, 0, 0, 0);
      if (idx < C::KCH && j0 + r < L)
        val = *reinterpret_cast<const uint4*>(kbase + (int64_t)(j0 + r) * kn + 16 * c);
      kreg[x] = val;
    }
    if constexpr (!DUMP) {
      if constexpr (!FP8) {
#pragma unroll
        for (int x = 0; x < C::VPT; ++x) {
          const int idx = tid + x * NT;
          const int r = idx / (D / 8), c = idx % (D / 8);
          uint4 val = make_uint4(0, 0, 0, 0);
          if (idx < C::VITEMS && j0 + r < L)
            val = *reinterpret_cast<const uint4*>(vbase + (int64_t)(j0 + r) * vn + 16 * c);
          vreg16[x] = val;
        }
      } else {
#pragma unroll
        for (int x = 0; x < C::VPT; ++x) {
          const int idx = tid + x * NT;
          const int kq = idx % (BN / 4), cg = idx / (BN / 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint2 val = make_uint2(0, 0);
            const int j = j0 + 4 * kq + e;
            if (idx < C::VITEMS && j < L) val = *reinterpret_cast<const uint2*>(vbase + (int64_t)j * vn + 8 * cg);
            vreg8[x * 4 + e] = val;
          }
        }
      }
    }
  };
  auto lds_store = [&]() {
#pragma unroll
    for (int x = 0; x < C::KPT; ++x) {
      const int idx = tid + x * NT;
      const int r = idx / (D / 16), c = idx % (D / 16);
      if (idx < C::KCH) *reinterpret_cast<uint4*>(k_lds + r * KROW + 16 * c) = kreg[x];
    }
    if constexpr (!DUMP) {
      if constexpr (!FP8) {
#pragma unroll
        for (int x = 0; x < C::VPT; ++x) {
          const int idx = tid + x * NT;
          const int r = idx / (D / 8), c = idx % (D / 8);
          if (idx < C::VITEMS) *reinterpret_cast<uint4*>(v_lds + r * VROW + 16 * c) = vreg16[x];
        }
      } else {
#pragma unroll
        for (int x = 0; x < C::VPT; ++x) {
          const int idx = tid + x * NT;
          const int kq = idx % (BN / 4), cg = idx / (BN / 4);
          if (idx < C::VITEMS) {
            const int pos = pos8(kq);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const uint32_t r0 = half ? vreg8[x * 4 + 0].y : vreg8[x * 4 + 0].x;
              const uint32_t r1 = half ? vreg8[x * 4 + 1].y : vreg8[x * 4 + 1].x;
              const uint32_t r2 = half ? vreg8[x * 4 + 2].y : vreg8[x * 4 + 2].x;
              const uint32_t r3 = half ? vreg8[x * 4 + 3].y : vreg8[x * 4 + 3].x;
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                const uint32_t t = ((r0 >> (8 * b)) & 0xffu) | (((r1 >> (8 * b)) & 0xffu) << 8) |
                                   (((r2 >> (8 * b)) & 0xffu) << 16) | (((r3 >> (8 * b)) & 0xffu) << 24);
                *reinterpret_cast<uint32_t*>(v_lds + (8 * cg + 4 * half + b) * VROW + pos) = t;
              }
            }
          }
        }
      }
    }
  };

  gload(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    lds_store();
    __syncthreads();
    if (t + 1 < ntiles) gload(t + 1);
    const int j0 = t * BN;

    // rows of this wave that can see any key of the tile
    bool active[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) active[rg] = !CAUSAL || j0 <= row0[rg] + 31;

    // ---- S^T = K . Q^T (INT8 MFMA, INT32 accumulation)
    v16i sacc[RG][BN / 32];
#pragma unroll
    for (int jt = 0; jt < BN / 32; ++jt) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) sacc[rg][jt] = v16i{};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const v4i kf = *reinterpret_cast<const v4i*>(k_lds + (32 * jt + li) * KROW + 32 * kk + 16 * g);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          if (active[rg]) sacc[rg][jt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, qf[rg][kk], sacc[rg][jt], 0, 0, 0);
      }
    }

    if constexpr (DUMP) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const int i = row0[rg] + li;
        if (i >= L) continue;
        int32_t* drow = a.dump + (sh * p.max_seqlen + i) * p.max_seqlen;
#pragma unroll
        for (int jt = 0; jt < BN / 32; ++jt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = j0 + 32 * jt + 8 * q + 4 * g;
            if (j < L)
              *reinterpret_cast<v4i*>(drow + j) =
                  v4i{sacc[rg][jt][4 * q], sacc[rg][jt][4 * q + 1], sacc[rg][jt][4 * q + 2], sacc[rg][jt][4 * q + 3]};
          }
      }
      continue;
    } else {
      // ---- key scales of this lane's keys (one per aligned group of 4 keys)
      float kscale[BN / 32][4];
#pragma unroll
      for (int jt = 0; jt < BN / 32; ++jt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + 32 * jt + 8 * q + 4 * g;
          kscale[jt][q] = j < L ? ksc[j / p.blk_k] : 0.0f;
        }

      const bool tail = j0 + BN > L;
      v8h pf[RG][BN / 16];
      v8i pf8[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        if (!active[rg]) continue;
        const int i = row0[rg] + li;
        float x[BN / 32][16];
#pragma unroll
        for (int jt = 0; jt < BN / 32; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r) x[jt][r] = (float)sacc[rg][jt][r] * (qsc[rg] * kscale[jt][r >> 2]);
        const bool need_mask = tail || (CAUSAL && j0 + BN - 1 > row0[rg]);
        if (need_mask) {
#pragma unroll
          for (int jt = 0; jt < BN / 32; ++jt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = j0 + 32 * jt + 8 * (r >> 2) + 4 * g + (r & 3);
              if (j >= L || (CAUSAL && j > i)) x[jt][r] = -INFINITY;
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < BN / 32; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, x[jt][r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        if constexpr (FP8) mt = ceilf(mt);
        const float mnew = fmaxf(m[rg], mt);
        const float mref = mnew == -INFINITY ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m[rg] - mref);
        m[rg] = mnew;
        float ps = 0.0f;
#pragma unroll
        for (int jt = 0; jt < BN / 32; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(x[jt][r] - mref);
            ps += pv;
            x[jt][r] = pv;
          }
        lsum[rg] = lsum[rg] * alpha + ps;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) o[rg][ct] *= alpha;
        if constexpr (!FP8) {
#pragma unroll
          for (int u = 0; u < BN / 16; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[rg][u][e] = (_Float16)x[u >> 1][8 * (u & 1) + e];
        } else {
#pragma unroll
          for (int jt = 0; jt < BN / 32; ++jt)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
              uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(x[jt][r] * 448.0f, x[jt][r + 1] * 448.0f, 0, false);
              wv = __builtin_amdgcn_cvt_pk_fp8_f32(x[jt][r + 2] * 448.0f, x[jt][r + 3] * 448.0f, wv, true);
              pf8[rg][4 * jt + r / 4] = (int)wv;
            }
        }
      }

      // ---- O^T += V^T . P^T
      if constexpr (!FP8) {
        const int b = lane >> 4, tl = lane & 15;
#pragma unroll
        for (int u = 0; u < BN / 16; ++u) {
#pragma unroll
          for (int ct = 0; ct < D / 32; ++ct) {
            const int col = 32 * ct + 16 * (b & 1) + 4 * (tl & 3);
            const uint8_t* pa = v_lds + (16 * u + 4 * g + (tl >> 2)) * VROW + 2 * col;
            const v4s ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)pa);
            const v4s rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(pa + 8 * VROW));
            const v4h ha = __builtin_bit_cast(v4h, ra), hb = __builtin_bit_cast(v4h, rb);
            const v8h vf = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
              if (active[rg]) o[rg][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[rg][u], o[rg][ct], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const uint8_t* pa = v_lds + (32 * ct + li) * VROW + 32 * g;
          const v4i va = *reinterpret_cast<const v4i*>(pa);
          const v4i vb = *reinterpret_cast<const v4i*>(pa + 16);
          const v8i vf = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            if (active[rg])
              o[rg][ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf8[rg], o[rg][ct], 0, 0, 0, 127, 0, 127);
        }
      }
    }
  }

  if constexpr (!DUMP) {
    _Float16* __restrict__ obase = (_Float16*)a.out + seq_head_base(p.cu, a.os, s, h);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const float lt = lsum[rg] + __shfl_xor(lsum[rg], 32, 64);
      const float inv = 1.0f / lt;
      const int i = row0[rg] + li;
      if (i >= L) continue;
      _Float16* orow = obase + (int64_t)i * a.os.n;
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 32 * ct + 8 * q + 4 * g;
          float f[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f[e] = o[rg][ct][4 * q + e] * inv;
            if constexpr (FP8) f[e] *= a.v_scale[sh * D + c + e] * (1.0f / 448.0f);
          }
          const v4h hv = {(_Float16)f[0], (_Float16)f[1], (_Float16)f[2], (_Float16)f[3]};
          *reinterpret_cast<v4h*>(orow + c) = hv;
        }
    }
  }
}

template <int D, int RG, int NW, bool FP8, bool CAUSAL, bool DUMP>
hipError_t launch_cfg(const Problem& p, const AttnArgs& a, hipStream_t st) {
  using C = Cfg<D, RG, NW, FP8, CAUSAL, DUMP>;
  const int nqt = (p.max_seqlen + C::BM - 1) / C::BM;
  dim3 grid(nqt, p.heads, p.nseq);
  hipLaunchKernelGGL((k_attn<D, RG, NW, FP8, CAUSAL, DUMP>), grid, dim3(C::NT), 0, st, p, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem& p, const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  if (a.dump) return launch_cfg<D, 1, 4, false, false, true>(p, a, st);
  if (fp8) return causal ? launch_cfg<D, 1, 4, true, true, false>(p, a, st) : launch_cfg<D, 1, 4, true, false, false>(p, a, st);
  return causal ? launch_cfg<D, 1, 4, false, true, false>(p, a, st) : launch_cfg<D, 1, 4, false, false, false>(p, a, st);
}

}  // namespace

hipError_t launch_attn(const Problem& p, const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  return p.head_dim == 64 ? launch_d<64>(p, a, causal, fp8, st) : launch_d<128>(p, a, causal, fp8, st);
}

}  // namespace sage
