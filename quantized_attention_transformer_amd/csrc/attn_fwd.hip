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
// Work decomposition.  One workgroup = 4 waves x 32 query rows of one
// (sequence, head); it walks 64-key tiles of K and V through three LDS
// stages, filled straight from global memory by buffer_load ... lds.
// (Sequence, head) pairs are dealt round-robin over the 8 XCDs and each XCD
// runs all query tiles of a pair back to back (longest causal rows first), so
// a pair's K/V re-reads stay in one L2 and the work spreads evenly.
//
// Per 64-key tile, on the matrix cores (one wave, 32 rows):
//   S^T[key][query] += K[key][c] . Q[query][c]   v_mfma_i32_32x32x32_i8 (8x)
//   O^T[c][query]   += V^T[c][key] . P^T[key][query]
//                      v_mfma_f32_32x32x16_f16 (16x, fp16 P and V) or
//                      v_mfma_scale_f32_32x32x64_f8f6f4 (4x, E4M3 P and V)
// Computing the transposes puts one query row in each lane (lanes l and l+32
// share row l%32), so the online-softmax state and the rescale of O are
// lane-local, and P leaves the i32 accumulator layout already in the operand
// layout of the P.V instruction (no LDS round trip for P).
//
// Key order inside an MFMA: in S^T tile jt (32 keys), lane (row i, half g =
// lane/32) holds accumulator r = 0..15 for key 32jt + 8(r/4) + 4g + r%4.  The
// two contraction operands of the P.V instruction only need the same key in
// the same (lane half, k slot); V's operand is read to match:
//   fp16: V stays row-major in LDS and ds_read_b64_tr_b16 transposes it on the
//         read (two reads per operand);
//   fp8:  V is written to LDS transposed ([channel][permuted key]).
//
// Software pipeline (per wave, step t): the P.V MFMAs of tile t-1 run while
// the VALU computes the softmax of tile t; one barrier; the loads of tile t+2
// are issued and the INT8 MFMAs of tile t+1.  The matrix cores see QK(t+1)
// then PV(t) back to back while the softmax of tile t+1 overlaps PV(t).
//
// Softmax.  The i32 accumulator starts at the bit pattern of 1.5*2^23, so the
// MFMA leaves the float 1.5*2^23 + S exactly (|S| <= 127^2*128 < 2^22): no
// conversion instruction.  With c = q_scale*k_scale*log2(e) the exponent is
// one FMA, x*c - (1.5*2^23*c + m).  m is the running row maximum in base-2
// units; O and l are rescaled (wave-uniform branch) only when some row's
// maximum grows: by more than 8 on the fp16 path (P stays <= 2^8, exact in
// fp16), by any amount on the FP8 path, where m is kept rounded up to an
// integer so rescales are exact powers of two and E4M3(448 p) does not depend
// on the order keys are visited.  l sums the fp16-rounded P fed to the MFMA
// (v_dot2) on the fp16 path, and the unquantised P on the FP8 path.
#include <type_traits>

#include "sage_internal.h"

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))
typedef LDS uint8_t lds_u8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;
constexpr int kMagicBits = 0x4B400000;  // float 1.5 * 2^23
constexpr float kMagic = 12582912.0f;
constexpr int BN = 64;                  // keys per tile
constexpr int NW = 4;                   // waves per workgroup
constexpr int NT = NW * 64;
constexpr int BM = NW * 32;             // query rows per workgroup
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3 for gfx9 (raw, 32-bit format)

// LDS stage of one 64-key tile.  K rows (D bytes) and fp16 V rows (2D bytes)
// are stored without padding; 16-byte chunks are XOR-swizzled by row so that
// every 256-byte LDS pass of the fragment reads (64 banks x 4 B) hits each
// bank once:
//   K:  chunk c of row r at c ^ ((r / (256/D)) % (D/16))   (ds_read_b128, 16 lanes = 16 rows)
//   V:  chunk c of row r at c ^ 4*(r % 4)       (D = 128)  (ds_read_b64_tr_b16, 32 lanes =
//                           c ^ 4*((r / 2) % 2) (D = 64)    4 rows x 64 bytes)
// The E4M3 V is stored transposed ([channel][permuted key], rows of BN+16 bytes).
template <int D, bool FP8>
struct Lds {
  static constexpr int KBYTES = BN * D;
  static constexpr int VROW = FP8 ? (BN + 16) : 2 * D;
  static constexpr int VBYTES = (FP8 ? D : BN) * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NSTAGE = 3;
  static constexpr int KBLK = KBYTES / 1024 / NW;             // 1 KiB DMA blocks per wave (K)
  static constexpr int VBLK = FP8 ? 0 : VBYTES / 1024 / NW;   // (fp16 V)
  __device__ static constexpr int kswz(int r) { return (r / (256 / D)) % (D / 16); }
  __device__ static constexpr int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

__device__ __forceinline__ int pos8(int kq) {  // byte position of key quad kq in an fp8 V^T row
  return 32 * (kq & 1) + 16 * (kq >> 3) + 4 * ((kq & 7) >> 1);
}

// Per-lane constants of the direct-to-LDS tile loads.  Wave w fills 1 KiB
// blocks w*NBLK .. w*NBLK+NBLK-1 of a region; lane l lands at block + 16 l and
// fetches the global 16-byte chunk the swizzle assigns there, at byte offset
// (row within the tile) * row_stride + 16 * chunk.
template <int D, bool FP8>
struct DmaPlan {
  using S = Lds<D, FP8>;
  int koff[S::KBLK];
  int voff[S::VBLK > 0 ? S::VBLK : 1];
  __device__ void init(int w, int lane, int64_t kn, int64_t vn) {
#pragma unroll
    for (int x = 0; x < S::KBLK; ++x) {
      const int byte = (w * S::KBLK + x) * 1024 + 16 * lane;
      const int r = byte / D, c = ((byte % D) / 16) ^ S::kswz(r);
      koff[x] = (int)(r * kn) + 16 * c;
    }
#pragma unroll
    for (int x = 0; x < S::VBLK; ++x) {
      const int byte = (w * S::VBLK + x) * 1024 + 16 * lane;
      const int r = byte / (2 * D), c = ((byte % (2 * D)) / 16) ^ S::vswz(r);
      voff[x] = (int)(r * vn) + 16 * c;
    }
  }
  // One tile: the descriptors start at the tile's first row and end at the
  // sequence's last byte, so rows past the sequence fall outside them (their
  // LDS bytes keep older, finite, data; those keys are masked).
  __device__ __forceinline__ void issue(const int8_t* kseq, int64_t kn, const uint8_t* vseq, int64_t vn, int j0,
                                        int L, lds_u8* stage, int w) const {
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kseq + (int64_t)j0 * kn), 0, (int)((L - 1 - j0) * kn + D), kRsrcWord3);
#pragma unroll
    for (int x = 0; x < S::KBLK; ++x)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (LDS void*)(stage + (w * S::KBLK + x) * 1024), 16, koff[x], 0, 0, 0);
    if constexpr (S::VBLK > 0) {
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vseq + (int64_t)j0 * vn), 0, (int)((L - 1 - j0) * vn + 2 * D), kRsrcWord3);
#pragma unroll
      for (int x = 0; x < S::VBLK; ++x)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (LDS void*)(stage + S::KBYTES + (w * S::VBLK + x) * 1024), 16,
                                                 voff[x], 0, 0, 0);
    }
  }
};

// E4M3 V tile through registers: 4 keys x 8 channels per item, written to LDS
// transposed.  Rows past the sequence are clamped to its last row.
template <int D>
struct V8Stager {
  static constexpr int VITEMS = (BN / 4) * (D / 8);
  static constexpr int VPT = (VITEMS + NT - 1) / NT;
  uint2 v8[VPT * 4];
  __device__ __forceinline__ void load(const uint8_t* vseq, int64_t vn, int j0, int L, int tid) {
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)vseq, 0, (int)((L - 1) * vn + D), kRsrcWord3);
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
      const int idx = tid + x * NT;
      const int kq = idx % (BN / 4), cg = idx / (BN / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = min(j0 + 4 * kq + e, L - 1);
        if (VITEMS % NT == 0 || idx < VITEMS)
          v8[x * 4 + e] =
              __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(vr, (int)(row * vn) + 8 * cg, 0, 0));
      }
    }
  }
  __device__ __forceinline__ void store(lds_u8* vl, int tid) const {
    constexpr int VROW = Lds<D, true>::VROW;
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
      const int idx = tid + x * NT;
      const int kq = idx % (BN / 4), cg = idx / (BN / 4);
      if (VITEMS % NT == 0 || idx < VITEMS) {
        const int pos = pos8(kq);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint32_t r0 = hf ? v8[x * 4 + 0].y : v8[x * 4 + 0].x;
          const uint32_t r1 = hf ? v8[x * 4 + 1].y : v8[x * 4 + 1].x;
          const uint32_t r2 = hf ? v8[x * 4 + 2].y : v8[x * 4 + 2].x;
          const uint32_t r3 = hf ? v8[x * 4 + 3].y : v8[x * 4 + 3].x;
          // byte b of the four key rows -> one dword per channel
          const uint32_t lo01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
          const uint32_t hi01 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
          const uint32_t lo23 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
          const uint32_t hi23 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
          lds_u8* row = vl + (8 * cg + 4 * hf) * VROW + pos;
          *(LDS uint32_t*)(row) = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
          *(LDS uint32_t*)(row + VROW) = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
          *(LDS uint32_t*)(row + 2 * VROW) = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
          *(LDS uint32_t*)(row + 3 * VROW) = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
        }
      }
    }
  }
};

// S^T for one 64-key tile: s[jt] (keys 32jt..32jt+31) = 1.5*2^23 + K . Q^T (as int
// bits); `magic` (all lanes 0x4B400000) is the first MFMA's accumulator input.
// kl: this lane's K row li; kx[kk]: swizzled byte offset of chunk 2kk+g in it.
template <int D>
__device__ __forceinline__ void qk_tile(const lds_u8* kl, const int (&kx)[D / 32], const v4i (&qf)[D / 32],
                                        const v16i& magic, v16i (&s)[2]) {
  v4i kf[2][D / 32];
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) kf[jt][kk] = *(const LDS v4i*)(kl + 32 * jt * D + kx[kk]);
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    v16i acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[jt][0], qf[0], magic, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < D / 32; ++kk) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[jt][kk], qf[kk], acc, 0, 0, 0);
    s[jt] = acc;
  }
}

__device__ __forceinline__ float xhalf_max(float v) {  // max over lanes l and l^32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x *= a in place (a tied register operand keeps the accumulator where the
// MFMAs expect it on both sides of the rescale branch).
__device__ __forceinline__ void scale_inplace(v16f& x, float a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float t = x[r];
    asm volatile("v_mul_f32 %0, %1, %0" : "+v"(t) : "v"(a));
    x[r] = t;
  }
}

template <int D, bool FP8, bool CAUSAL, bool KSU>
__device__ __forceinline__ void attn_body(const Problem& p, const AttnArgs& a, lds_u8* const lds) {
  using S = Lds<D, FP8>;

  // ---- workgroup -> (sequence, head, query tile): pair = 8 * slot + xcd
  const int nqt = (p.max_seqlen + BM - 1) / BM;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int sh_i = (kx / nqt) * 8 + xcd;
  if (sh_i >= p.nseq * p.heads) return;
  const int qt = CAUSAL ? nqt - 1 - kx % nqt : kx % nqt;
  const int s = sh_i / p.heads, h = sh_i % p.heads;
  const int64_t sh = sh_i;

  const int L = seq_len(p.cu, s, p.max_seqlen);
  const int q0 = qt * BM;
  if (q0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int8_t* __restrict__ qbase = a.q8 + seq_head_base(p.cu, a.q8s, s, h);
  const int8_t* kseq = a.k8 + seq_head_base(p.cu, a.k8s, s, h);
  const uint8_t* vseq = (const uint8_t*)a.v + seq_head_base(p.cu, a.vs, s, h) * (FP8 ? 1 : 2);
  const int64_t kn = a.k8s.n, vn = a.vs.n * (FP8 ? 1 : 2);  // row strides in bytes
  const float* __restrict__ ksc = a.k_scale + sh * p.nbk;

  // ---- this lane's query row and its Q fragments (B operand of S^T)
  const int row0 = q0 + w * 32;
  const int i = row0 + li;
  v4i qf[D / 32];
  float qsc = 0.0f;
  if (i < L) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qf[kk] = *reinterpret_cast<const v4i*>(qbase + (int64_t)i * a.q8s.n + 32 * kk + 16 * g);
    qsc = a.q_scale[sh * p.nbq + i / p.blk_q] * kLog2e;
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf[kk] = v4i{0, 0, 0, 0};
  }
  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = kMagicBits;

  const int kv_end = CAUSAL ? min(L, q0 + BM) : L;
  const int ntiles = (kv_end + BN - 1) / BN;
  // tiles this wave needs (causal: keys beyond its last row are never visible)
  const int wtiles = CAUSAL ? min(ntiles, (row0 + 31) / BN + 1) : ntiles;

  // LDS fragment offsets of this lane: K row li, chunk 2kk+g (swizzled) ...
  int kx_off[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) kx_off[kk] = 16 * ((2 * kk + g) ^ S::kswz(li));
  const int krow = li * D;
  // ... and the transposed fp16 V reads: rows 4g + tl/4 (+8), chunk 4ct + 2(b&1) + (tl&3)/2
  const int vb = lane >> 4, tl = lane & 15;
  int vaddr[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) {
    const int vr = 4 * g + (tl >> 2);
    vaddr[ct] = S::KBYTES + vr * S::VROW + 16 * ((4 * ct + 2 * (vb & 1) + ((tl & 3) >> 1)) ^ S::vswz(vr)) + 8 * (tl & 1);
  }

  // LDS starts zeroed so bytes the tail tiles leave untouched are finite.
  for (int x = tid; x < S::NSTAGE * S::STAGE / 16; x += NT) *(LDS v4i*)(lds + 16 * x) = v4i{0, 0, 0, 0};
  __syncthreads();

  DmaPlan<D, FP8> dma;
  dma.init(w, lane, kn, vn);
  V8Stager<D> v8s;

  float m = -INFINITY, lsum = 0.0f;
  v16f o[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) o[ct] = v16f{};
  v16i sc[2];        // S of the tile being softmaxed
  v8h pf[4], pfp[4];  // fp16 P of this tile / of the previous tile
  v8i pf8, pf8p;      // E4M3 P of this tile / of the previous tile

  // O^T += V^T . P^T for the tile in stage `st` (P from the previous step)
  auto pv = [&](const lds_u8* st) {
    if constexpr (!FP8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const lds_u8* pa = st + vaddr[ct] + 16 * u * S::VROW;
          const v4h ha = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)pa));
          const v4h hb = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)(pa + 8 * S::VROW)));
          const v8h vf = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pfp[u], o[ct], 0, 0, 0);
        }
      }
    } else {
      const lds_u8* vl = st + S::KBYTES + li * S::VROW + 32 * g;  // V^T rows = channels
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) {
        const lds_u8* pa = vl + 32 * ct * S::VROW;
        const v4i va = *(const LDS v4i*)(pa);
        const v4i vb2 = *(const LDS v4i*)(pa + 16);
        const v8i vf = __builtin_shufflevector(va, vb2, 0, 1, 2, 3, 4, 5, 6, 7);
        o[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf8p, o[ct], 0, 0, 0, 127, 0, 127);
      }
    }
  };

  // softmax of tile t from sc -> pf / pf8 (lane: row i, keys j(jt, r)).
  // MASKED tiles (sequence tail, causal diagonal) take a separate instantiation.
  auto softmax = [&](int t, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int j0 = t * BN;
    float c[2][4];  // q_scale * k_scale * log2(e) per (jt, group of 4 keys)
    if constexpr (KSU) {
      const float ck = qsc * ksc[j0 / p.blk_k];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int q = 0; q < 4; ++q) c[jt][q] = ck;
    } else {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + 32 * jt + 8 * q + 4 * g;
          c[jt][q] = j < L ? qsc * ksc[j / p.blk_k] : 0.0f;
        }
    }
    bool valid[2][16];
    if constexpr (MASKED) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * jt + 8 * (r >> 2) + 4 * g + (r & 3);
          valid[jt][r] = j < L && (!CAUSAL || j <= i);
        }
    }
    // row maximum of this tile, in base-2 units
    float mt;
    float y[2][16];  // general key-block size: S * c per element
    if constexpr (KSU) {
      auto xv = [&](int jt, int r) {
        const float xx = __int_as_float(sc[jt][r]);
        if constexpr (MASKED) return valid[jt][r] ? xx : 0.0f;
        return xx;
      };
      float mx = fmaxf(xv(0, 0), xv(0, 1));
#pragma unroll
      for (int r = 2; r < 32; r += 2) mx = fmaxf(fmaxf(mx, xv(r >> 4, r & 15)), xv((r + 1) >> 4, (r + 1) & 15));
      mx = xhalf_max(mx);
      // every real x is >= 1.5*2^23 - 2^21 > 0, so 0 means "all masked": leave m alone
      mt = (MASKED && mx == 0.0f) ? -INFINITY : (mx - kMagic) * c[0][0];
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          y[jt][r] = (__int_as_float(sc[jt][r]) - kMagic) * c[jt][r >> 2];
          if constexpr (MASKED) y[jt][r] = valid[jt][r] ? y[jt][r] : -INFINITY;
          mx = fmaxf(mx, y[jt][r]);
        }
      mt = xhalf_max(mx);
    }
    if constexpr (FP8) mt = ceilf(mt);
    const bool grow = FP8 ? (mt > m) : (mt > m + 8.0f);
    if (__any(grow)) {  // rare after the first tiles; O waits for the previous P.V here
      const float mn = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) o[ct] *= alpha;
    }
    const float mref = FP8 ? m - kLog2_448 : m;  // FP8: P scaled by 448 inside the exponent
    const float bias = __builtin_fmaf(kMagic, c[0][0], mref);
    auto prob = [&](int jt, int r) {
      float arg = KSU ? __builtin_fmaf(__int_as_float(sc[jt][r]), c[0][0], -bias) : y[jt][r] - mref;
      if constexpr (MASKED) arg = valid[jt][r] ? arg : -INFINITY;
      return __builtin_amdgcn_exp2f(arg);
    };
    if constexpr (!FP8) {
      const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const v2h hp = {(_Float16)prob(u >> 1, 8 * (u & 1) + e), (_Float16)prob(u >> 1, 8 * (u & 1) + e + 1)};
          lsum = __builtin_amdgcn_fdot2(hp, ones, lsum, false);
          pf[u][e] = hp[0];
          pf[u][e + 1] = hp[1];
        }
    } else {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float p0 = prob(jt, r), p1 = prob(jt, r + 1), p2 = prob(jt, r + 2), p3 = prob(jt, r + 3);
          lsum += (p0 + p1) + (p2 + p3);
          uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          wv = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wv, true);
          pf8[4 * jt + r / 4] = (int)wv;
        }
    }
  };

  // prologue: tile 0 in stage 0 and its S; tile 1 in flight to stage 1
  dma.issue(kseq, kn, vseq, vn, 0, L, lds, w);
  if constexpr (FP8) {
    v8s.load(vseq, vn, 0, L, tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    v8s.store(lds + S::KBYTES, tid);
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  if (ntiles > 1) {
    dma.issue(kseq, kn, vseq, vn, BN, L, lds + S::STAGE, w);
    if constexpr (FP8) v8s.load(vseq, vn, BN, L, tid);
  }
  qk_tile<D>(lds + krow, kx_off, qf, magic, sc);

  // Step t (stage t%3 holds tile t, (t+1)%3 tile t+1 in flight or landed):
  // P.V of tile t-1 on the matrix cores while the VALU computes the softmax
  // of tile t; then one barrier (tile t+1 has landed everywhere and every
  // wave has finished reading stage (t-1)%3), the loads of tile t+2 into that
  // stage, and the INT8 MFMAs of tile t+1 into sc.
  for (int t = 0; t <= ntiles; ++t) {
    if (t >= 1 && t - 1 < wtiles) pv(lds + ((t - 1) % 3) * S::STAGE);
    if (t < wtiles) {
      const int j0 = t * BN;
      if ((j0 + BN > L) || (CAUSAL && j0 + BN - 1 > row0))
        softmax(t, std::true_type{});
      else
        softmax(t, std::false_type{});
    }
    if (t + 1 < ntiles) {
      lds_u8* nx1 = lds + ((t + 1) % 3) * S::STAGE;
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // own loads of tile t+1 landed, own V reads done
      if constexpr (FP8) v8s.store(nx1 + S::KBYTES, tid);
      __syncthreads();
      if (t + 2 < ntiles) {
        lds_u8* nx2 = lds + ((t + 2) % 3) * S::STAGE;
        dma.issue(kseq, kn, vseq, vn, (t + 2) * BN, L, nx2, w);
        if constexpr (FP8) v8s.load(vseq, vn, (t + 2) * BN, L, tid);
      }
      if (t + 1 < wtiles) qk_tile<D>(nx1 + krow, kx_off, qf, magic, sc);
    }
    if constexpr (!FP8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) pfp[u] = pf[u];
    } else {
      pf8p = pf8;
    }
  }

  // ---- epilogue: O = O^T / l (FP8: l and O both carry the factor 448; times v_scale)
  _Float16* __restrict__ obase = (_Float16*)a.out + seq_head_base(p.cu, a.os, s, h);
  const float inv = 1.0f / xhalf_sum(lsum);
  if (i < L) {
    _Float16* orow = obase + (int64_t)i * a.os.n;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = 32 * ct + 8 * q + 4 * g;
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = o[ct][4 * q + e] * inv;
          if constexpr (FP8) f[e] *= a.v_scale[sh * D + cc + e];
        }
        const v4h hv = {(_Float16)f[0], (_Float16)f[1], (_Float16)f[2], (_Float16)f[3]};
        *reinterpret_cast<v4h*>(orow + cc) = hv;
      }
  }
}

template <int D, bool FP8, bool CAUSAL, bool KSU>
__global__ __launch_bounds__(NT) void k_attn(Problem p, AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[Lds<D, FP8>::NSTAGE * Lds<D, FP8>::STAGE];
  attn_body<D, FP8, CAUSAL, KSU>(p, a, (lds_u8*)lds_raw);
}

// Debug: the INT32 scores of the same staging (DmaPlan) and MFMA path
// (qk_tile), before any dequantisation.  Dense problems, every query row and
// key written.
template <int D>
__global__ __launch_bounds__(NT) void k_qk_dump(Problem p, AttnArgs a) {
  using S = Lds<D, true>;  // K part only (the FP8 plan has no V DMA)
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[S::KBYTES];
  lds_u8* const lds = (lds_u8*)lds_raw;
  const int qt = blockIdx.x, h = blockIdx.y, s = blockIdx.z, H = gridDim.y;
  const int L = seq_len(p.cu, s, p.max_seqlen);
  const int q0 = qt * BM;
  if (q0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t sh = (int64_t)s * H + h;
  const int8_t* qbase = a.q8 + seq_head_base(p.cu, a.q8s, s, h);
  const int8_t* kseq = a.k8 + seq_head_base(p.cu, a.k8s, s, h);
  const int i = q0 + w * 32 + li;
  v4i qf[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = i < L ? *reinterpret_cast<const v4i*>(qbase + (int64_t)i * a.q8s.n + 32 * kk + 16 * g) : v4i{0, 0, 0, 0};
  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = kMagicBits;
  int kx_off[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) kx_off[kk] = 16 * ((2 * kk + g) ^ S::kswz(li));
  for (int x = tid; x < S::KBYTES / 16; x += NT) *(LDS v4i*)(lds + 16 * x) = v4i{0, 0, 0, 0};
  DmaPlan<D, true> dma;
  dma.init(w, lane, a.k8s.n, 0);
  for (int j0 = 0; j0 < L; j0 += BN) {
    __syncthreads();  // everyone is done reading the previous tile
    dma.issue(kseq, a.k8s.n, nullptr, 0, j0, L, lds, w);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    v16i sc[2];
    qk_tile<D>(lds + li * D, kx_off, qf, magic, sc);
    if (i < L) {
      int32_t* drow = a.dump + (sh * p.max_seqlen + i) * p.max_seqlen;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + 32 * jt + 8 * q + 4 * g;
          if (j < L)
            *reinterpret_cast<v4i*>(drow + j) =
                v4i{sc[jt][4 * q] - kMagicBits, sc[jt][4 * q + 1] - kMagicBits, sc[jt][4 * q + 2] - kMagicBits,
                    sc[jt][4 * q + 3] - kMagicBits};
        }
    }
  }
}

template <int D, bool FP8, bool CAUSAL, bool KSU>
hipError_t launch_cfg(const Problem& p, const AttnArgs& a, hipStream_t st) {
  const int nqt = (p.max_seqlen + BM - 1) / BM;
  const int64_t P8 = ((int64_t)p.nseq * p.heads + 7) / 8 * 8;
  const int64_t G = (int64_t)nqt * P8;
  if (G >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_attn<D, FP8, CAUSAL, KSU>), dim3((unsigned)G), dim3(NT), 0, st, p, a);
  return hipGetLastError();
}

template <int D, bool FP8, bool CAUSAL>
hipError_t launch_ks(const Problem& p, const AttnArgs& a, hipStream_t st) {
  return (p.blk_k % BN == 0) ? launch_cfg<D, FP8, CAUSAL, true>(p, a, st) : launch_cfg<D, FP8, CAUSAL, false>(p, a, st);
}

template <int D>
hipError_t launch_d(const Problem& p, const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  if (a.dump) {
    const int nqt = (p.max_seqlen + BM - 1) / BM;
    hipLaunchKernelGGL((k_qk_dump<D>), dim3(nqt, p.heads, p.nseq), dim3(NT), 0, st, p, a);
    return hipGetLastError();
  }
  if (fp8) return causal ? launch_ks<D, true, true>(p, a, st) : launch_ks<D, true, false>(p, a, st);
  return causal ? launch_ks<D, false, true>(p, a, st) : launch_ks<D, false, false>(p, a, st);
}

}  // namespace

hipError_t launch_attn(const Problem& p, const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  return p.head_dim == 64 ? launch_d<64>(p, a, causal, fp8, st) : launch_d<128>(p, a, causal, fp8, st);
}

}  // namespace sage
