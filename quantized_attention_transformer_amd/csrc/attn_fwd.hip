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
// Work decomposition.  One workgroup = 128 query rows of one (sequence,
// head), 8 waves in two halves of 4.  Wave w of half h owns rows 32(w%4) ..
// 32(w%4)+31 and the 64-key tiles t = h, h+2, h+4, ...: the halves split the
// keys and merge their partial (O, l, m) through LDS at the end.  The two
// waves a SIMD hosts (w and w+4) belong to different halves.  (Sequence,
// head) pairs are dealt round-robin over the 8 XCDs and each XCD runs all
// query tiles of a pair back to back (longest causal rows first), so a pair's
// K/V re-reads stay in one L2 and the work spreads evenly.
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
//   fp8:  V stays row-major in LDS too and ds_read_b64_tr_b8 transposes it
//         (four reads per operand).
//
// Ping-pong schedule.  Time is cut into phases b = 0, 1, ..., ntiles+1, one
// workgroup barrier after each.  In phase b the half with h = b mod 2 is in
// its matrix phase: INT8 S of tile b and the P.V of tile b-2; the other half
// is in its vector phase: the softmax of tile b-1.  So at any time one wave
// of every SIMD feeds the matrix core while the other keeps the VALU busy,
// and S and P need one register set each.  The half in its matrix phase b
// also issues the loads of the tiles it will use next: V(b+2) and K(b+4),
// straight into LDS with buffer_load ... lds, and waits for them at the end
// of its vector phase b+3, ~3.5 phases later.  K and V tiles live in rings of
// 5 LDS slots.
//
// Softmax.  The i32 accumulator starts at the bit pattern of 1.5*2^23, so the
// MFMA leaves the float 1.5*2^23 + S exactly (|S| <= 127^2*128 < 2^22): no
// conversion instruction.  With c = q_scale*k_scale*log2(e) the exponent is
// one FMA, x*c - (1.5*2^23*c + m).  fp16 path: m is a lazy running row
// maximum in base-2 units (moved only when the tile maximum exceeds it by
// more than 8; P <= 2^8 is exact in fp16), O rescaled by 2^(m_old - m_new)
// when it moves (rare).  FP8 path: m is kept rounded up to an integer
// (E4M3(448 p) then does not depend on the order keys are visited) and O is
// not rescaled: it keeps the first tile's maximum m0 as reference and each
// tile's P enters the P.V MFMA with the exact per-lane E8M0 scale
// 2^(m - m0).  l sums the fp32 P before rounding (fp32 adds), except on the
// fp16 path at D = 64, where it sums the fp16-rounded P fed to the MFMA
// (v_dot2).
//
// Smooth Q ("4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级",
// section 技术方案 item 1; key blocks that are multiples of 64): S gains the
// per-key compensation delta_j = mean(Q') . K_s[j].  The half that loads K(t)
// also loads delta(t) (256 bytes) into a ring of 6 LDS slots, read by the
// softmax of tile t; there x' = fma(delta_j, 1/(qs ks), x) puts delta_j in
// units of the integer scores (x stays the exact float 1.5*2^23 + S, and
// x' c = S c + delta_j log2(e)), before the row maximum.  A zero Q or K block
// scale (all codes 0: S is the compensation alone) is replaced by a positive
// one (2^-40 for Q, so that delta keeps fp32 precision in x'; 1 for K, where
// delta is 0).
#include <type_traits>

#include "sage_internal.h"

namespace sage {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
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
constexpr int NW = 8;                   // waves per workgroup (two halves of 4)
constexpr int NT = NW * 64;
constexpr int BM = 128;                 // query rows per workgroup (32 per wave of a half)
constexpr int NSK = 5;                  // K ring slots
constexpr int NSV = 5;                  // V ring slots
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3 for gfx9 (raw, 32-bit format)

// LDS of one workgroup.  K rows (D bytes), fp16 V rows (2D bytes) and E4M3
// V rows (D bytes) are stored without padding, one key per row, straight from
// the tile loads; 16-byte chunks are XOR-swizzled by row so that every
// 256-byte LDS pass of the fragment reads (64 banks x 4 B) hits each bank
// once:
//   K:     chunk c of row r at c ^ ((r / (256/D)) % (D/16))   (ds_read_b128, 16 lanes = 16 rows)
//   fp16 V: chunk c of row r at c ^ 4*(r % 4)       (D = 128)  (ds_read_b64_tr_b16, 32 lanes =
//                              c ^ 4*((r / 2) % 2) (D = 64)    4 rows x 64 bytes)
//   E4M3 V: chunk c of row r at c ^ (2*(r/2 % 2) + 4*(r/8 % 2))  (D = 128)  (ds_read_b64_tr_b8,
//                              c ^ 2*(r/8 % 2)                  (D = 64)   32 lanes = 8 rows x
//                                                                          32 bytes)
// After the key loop the same bytes hold the second half's partial results.
template <int D, bool FP8, bool QK4 = false>
struct Lds {
  static constexpr int KROW = QK4 ? D / 2 : D;  // bytes of a K row (INT8, or MXFP4 codes)
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VROW = FP8 ? D : 2 * D;
  static constexpr int VBYTES = BN * VROW;
  static constexpr int VRING = NSK * KBYTES;  // offset of the V ring
  static constexpr int RING = VRING + NSV * VBYTES;
  static constexpr int MSTRIDE = D / 2 + 2;   // floats per lane of a partial result: O^T, m, l
  static constexpr int MERGE = 4 * MSTRIDE * 64 * 4;
  static constexpr int KSTAB = RING > MERGE ? RING : MERGE;  // per-tile k_scale table (key blocks of 64k keys)
  static constexpr int KSCAP = 4096;                          // its capacity in tiles
  // (the O staging area after the merge must fit as well: with the 4-bit K tile
  // and E4M3 V the rings are smaller than it)
  static constexpr int BYTES0 = KSTAB + 4 * KSCAP;
  // fp16 O rows staged for the stores (after the merge, past the merge area);
  // rows padded by 16 bytes against bank conflicts on the writes
  static constexpr int OROW = 2 * D + 16;
  static constexpr int OSTAGE = MERGE;
  static constexpr int BYTES = BYTES0 > OSTAGE + BM * OROW ? BYTES0 : OSTAGE + BM * OROW;
  // smooth Q: ring of NSD slots of 1 KiB past BYTES, each holding 4 copies of
  // one tile's 64 fp32 compensations
  static constexpr int NSD = 6;
  static constexpr int DRING = BYTES;
  static constexpr int DBYTES = NSD * 1024;
  static constexpr int KCH = KBYTES / 1024;             // 1 KiB DMA blocks per K tile
  static constexpr int VCH = VBYTES / 1024;            // 1 KiB DMA blocks per V tile
  __device__ static constexpr int kswz(int r) { return (r / (256 / KROW)) % (KROW / 16); }
  __device__ static constexpr int vswz(int r) {
    if constexpr (FP8) return D == 128 ? 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1) : 2 * ((r >> 3) & 1);
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
  }
};


// Buffer descriptor (gfx9 raw buffer): base, num_records bytes, stride 0.
__device__ __forceinline__ v4i make_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), bytes, kRsrcWord3};
}

// 16 bytes per lane from buffer offset voff straight into LDS at lds_addr +
// 16 * lane (buffer_load_dwordx4 ... lds).  Written as inline asm: these loads
// write no register, and hiding them from the compiler keeps it from waiting
// for every one of them before each later LDS read.  The caller orders them
// with explicit s_waitcnt vmcnt and a barrier before the data is read.  M0
// (the LDS base of the load) is saved and restored around it.
__device__ __forceinline__ void dma_b128(const v4i& rsrc, int voff, uint32_t lds_addr) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %1, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(rsrc), "v"(voff), "s"(lds_addr)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// Per-lane constants of the direct-to-LDS tile loads, issued by the 4 waves of
// one half.  Wave w (0..3 within its half) fills the 1 KiB blocks w, w+4, ...
// of a tile; lane l lands at block + 16 l and fetches the global 16-byte chunk
// the swizzle assigns there, at byte offset (row within the tile) *
// row_stride + 16 * chunk.
constexpr int NWH = 4;  // waves per half
template <int D, bool FP8, bool QK4 = false>
struct DmaPlan {
  using S = Lds<D, FP8, QK4>;
  static constexpr int KPW = S::KCH / NWH;  // K blocks per wave
  static constexpr int VPW = S::VCH / NWH;  // V blocks per wave
  static_assert(S::KCH % NWH == 0 && S::VCH % NWH == 0, "tile blocks split over a half");
  int koff[KPW];
  int voff[VPW > 0 ? VPW : 1];
  int doff;  // smooth Q: byte offset of this lane's 4 compensations in a tile (4 copies per 1 KiB)
  __device__ void init(int w, int lane, int64_t kn, int64_t vn) {
    doff = 16 * (lane & 15);
#pragma unroll
    for (int x = 0; x < KPW; ++x) {
      const int byte = (w + NWH * x) * 1024 + 16 * lane;
      const int r = byte / S::KROW, c = ((byte % S::KROW) / 16) ^ S::kswz(r);
      koff[x] = (int)(r * kn) + 16 * c;
    }
#pragma unroll
    for (int x = 0; x < VPW; ++x) {
      const int byte = (w + NWH * x) * 1024 + 16 * lane;
      const int r = byte / S::VROW, c = ((byte % S::VROW) / 16) ^ S::vswz(r);
      voff[x] = (int)(r * vn) + 16 * c;
    }
  }
  // One tile: the descriptors start at the tile's first row and end at the
  // sequence's last byte, so rows past the sequence fall outside them (their
  // LDS bytes keep older, finite, data; those keys are masked).
  __device__ __forceinline__ void issue_k(const v4i& kr, lds_u8* slot, int w) const {
#pragma unroll
    for (int x = 0; x < KPW; ++x) dma_b128(kr, koff[x], lds_addr(slot + (w + NWH * x) * 1024));
  }
  __device__ __forceinline__ void issue_k1(const v4i& kr, lds_u8* slot, int w, int x) const {
    dma_b128(kr, koff[x], lds_addr(slot + (w + NWH * x) * 1024));
  }
  // smooth Q: the compensations of one tile into a 1 KiB slot (every wave of the
  // half writes the same bytes)
  __device__ __forceinline__ void issue_d(const v4i& dr, lds_u8* slot) const { dma_b128(dr, doff, lds_addr(slot)); }
  __device__ __forceinline__ void issue_v1(const v4i& vr, lds_u8* slot, int w, int x) const {
    if constexpr (VPW > 0) dma_b128(vr, voff[x], lds_addr(slot + (w + NWH * x) * 1024));
  }
  __device__ __forceinline__ void issue_v(const v4i& vr, lds_u8* slot, int w) const {
    if constexpr (VPW > 0) {
#pragma unroll
      for (int x = 0; x < VPW; ++x) dma_b128(vr, voff[x], lds_addr(slot + (w + NWH * x) * 1024));
    }
  }
};

// S^T for one 64-key tile: s[jt] (keys 32jt..32jt+31) = 1.5*2^23 + K . Q^T (as int
// bits); `magic` (0x4B400000 in every lane) is the first MFMA's accumulator input.
// kx[kk]: byte offset in a K slot of chunk 2kk+g (swizzled) of this lane's row li.
template <int D>
__device__ __forceinline__ void qk_tile(const lds_u8* kslot, const uint32_t (&kx)[D / 32], const v4i (&qf)[D / 32],
                                        const v16i& magic, v16i (&s)[2]) {
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    v4i kf[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) kf[kk] = *(const LDS v4i*)(kslot + kx[kk] + 32 * jt * D);
    v16i acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[0], qf[0], magic, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < D / 32; ++kk) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[kk], qf[kk], acc, 0, 0, 0);
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

// DUMP (debug, INT8 fp16-path only): the same kernel writes each tile's raw
// INT32 scores to a.dump at the start of its softmax -- after the steady-state
// (qk_pv) or edge-phase (qk_tile) matrix phase that produced them, through the
// same K ring -- and stores no O; V is not read (empty descriptors) and no
// scale is loaded (the softmax runs on scale 1, its result unused).
template <int D, bool FP8, bool CAUSAL, bool KSU, bool SQ, bool QK4, bool DUMP = false>
__device__ __forceinline__ void attn_body(const Problem& p, const AttnArgs& a, lds_u8* const lds) {
  static_assert(!DUMP || (!FP8 && !CAUSAL && KSU && !SQ && !QK4), "dump: the plain INT8 kernel");
  using S = Lds<D, FP8, QK4>;
  static_assert(!SQ || KSU, "smooth Q needs key blocks that are multiples of the tile");
  static_assert(!QK4 || (D == 128 && KSU), "4-bit Q.K^T: head_dim 128, no per-block k-scale table");
  // The softmax's score x: INT8 without smooth Q, the float 1.5*2^23 + S read
  // straight from the MFMA; smooth Q, S + delta/(qs ks) (the seed subtracted
  // exactly first); 4-bit, S itself (fp32 from the MFMA).
  constexpr float MAG = (QK4 || SQ) ? 0.0f : kMagic;
  constexpr bool NEGX = SQ || QK4;  // scores may be <= 0: a masked key is -inf
  constexpr bool BIASED = KSU && !NEGX;  // x carries the seed into the exponent's FMA
  // Smooth Q: a zero block scale (all codes 0) is replaced.  x' = x + delta /
  // (qs ks) is rounded to fp32, so the unit qs ks must not be coarse next to
  // delta: a zero Q scale becomes 2^-40 (x' then holds delta at fp32 relative
  // precision); a zero K scale means K_s = 0 in the block, hence delta = 0,
  // and becomes 1.
  auto qeff = [](float v) { return (SQ && !(v > 0.0f)) ? 0x1p-40f : v; };
  auto keff = [](float v) { return (SQ && !(v > 0.0f)) ? 1.0f : v; };

  // ---- workgroup -> (sequence, head, query tile).  (sequence, K/V head)
  // groups are dealt round-robin over the 8 XCDs, group = 8 * (slot / grp) +
  // xcd, and an XCD runs the grp query heads of a group (grouped-query
  // attention; grp = 1 otherwise) and all their query tiles back to back, so
  // a K/V head is read into one L2.
  const int nqt = (p.max_seqlen + BM - 1) / BM;
  const int grp = p.heads / p.kv_heads;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int slot = kx / nqt;
  const int kvg = (slot / grp) * 8 + xcd;
  if (kvg >= p.nseq * p.kv_heads) return;
  const int qt = CAUSAL ? nqt - 1 - kx % nqt : kx % nqt;
  const int s = kvg / p.kv_heads, kvh = kvg % p.kv_heads, h = kvh * grp + slot % grp;
  const int64_t sh = (int64_t)s * p.heads + h;  // (sequence, query head)
  const int64_t skv = kvg;                       // (sequence, K/V head)

  const int L = seq_len(p.cu, s, p.max_seqlen, p.total);
  const int q0 = qt * BM;
  if (q0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = w >> 2;  // half: key tiles t = hf (mod 2)

  const int8_t* __restrict__ qbase = a.q8 + seq_head_base(p.cu, a.q8s, s, h, p.total);
  const int8_t* kseq = a.k8 + seq_head_base(p.cu, a.k8s, s, kvh, p.total);
  const uint8_t* vseq = (const uint8_t*)a.v + seq_head_base(p.cu, a.vs, s, kvh, p.total) * (FP8 ? 1 : 2);
  const int64_t kn = a.k8s.n, vn = a.vs.n * (FP8 ? 1 : 2);  // row strides in bytes
  const float* __restrict__ ksc = a.k_scale + skv * p.nbk;
  const __attribute__((address_space(4))) float* ksc_c = (const __attribute__((address_space(4))) float*)ksc;

  // ---- this lane's query row and its Q fragments (B operand of S^T)
  const int row0 = q0 + (w & 3) * 32;
  const int i = row0 + li;
  v4i qf[D / 32];
  float qsc = (SQ || QK4) ? kLog2e : 0.0f;  // (rows past the sequence: never stored; kept finite)
  // 4-bit: qf[kk] (kk < D/64) = this lane's 32 E2M1 codes of channels 64kk + 32g .., and
  // qsb[kk] its block's E8M0 code
  int qsb[D / 64] = {};
  // The Q scale (word) is loaded here and only used after the prologue's wait,
  // so that its latency and the fragments' overlap the first tile loads.
  float qraw = 0.0f;
  uint32_t wq = 0;
  if constexpr (QK4) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf[kk] = v4i{0, 0, 0, 0};
    if (i < L) {
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk)
        qf[kk] = *reinterpret_cast<const v4i*>(qbase + (int64_t)i * a.q8s.n + 32 * kk + 16 * g);
      wq = *reinterpret_cast<const uint32_t*>(a.qsc4 + seq_head_base(p.cu, a.qss4, s, h, p.total) + (int64_t)i * a.qss4.n);
    }
  } else if (i < L) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qf[kk] = *reinterpret_cast<const v4i*>(qbase + (int64_t)i * a.q8s.n + 32 * kk + 16 * g);
    qraw = DUMP ? 1.0f : a.q_scale[sh * p.nbq + i / p.blk_q];
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
  uint32_t kofs[D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) kofs[kk] = li * S::KROW + 16 * ((2 * kk + g) ^ S::kswz(li));
  // ... and the transposed fp16 V reads: rows 4g + tl/4 (+8), chunk 4ct + 2(b&1) + (tl&3)/2
  const int vb = lane >> 4, tl = lane & 15;
  int vaddr[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) {
    const int vr = 4 * g + (tl >> 2);
    vaddr[ct] = vr * S::VROW + 16 * ((4 * ct + 2 * (vb & 1) + ((tl & 3) >> 1)) ^ S::vswz(vr)) + 8 * (tl & 1);
  }
  // ... and the transposed E4M3 V reads (ds_read_b64_tr_b8: in each group of 16
  // lanes, lane t receives byte t%8 of the 8 bytes named by lanes t/8, t/8+2,
  // .., t/8+14).  Lanes 2k and 2k+1 of a group name the two 8-channel halves
  // of 16-channel chunk 2ct + (group%2) in key row k of the P.V contraction's
  // slot order (rows 8(k/4) + 4g + k%4 of each 16 keys), so lane (m, g) gets 8
  // keys of channel 32ct + m, in the order P holds them.
  uint32_t vaddr8[D / 32];
  {
    const int t = lane & 15, k = t >> 1;
    const int vr = 8 * (k >> 2) + 4 * g + (k & 3);
    const int fh = S::vswz(vr) >> 1;  // (the swizzle of row 16 rr + vr is that of vr)
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) vaddr8[ct] = vr * S::VROW + 16 * ((lane >> 4) & 1) + 8 * (t & 1) + 32 * (ct ^ fh);
  }

  const bool ks_in_lds = KSU && !QK4 && !DUMP && ntiles <= S::KSCAP;

  DmaPlan<D, FP8, QK4> dma;
  dma.init(w & 3, lane, kn, vn);  // the plan covers a tile with the 4 waves of one half

  float m = -INFINITY, lsum = 0.0f;
  // FP8: O and l accumulate relative to the first tile's maximum m0; tile t's
  // P (E4M3, relative to the running integer maximum m) enters the P.V MFMA
  // with the exact per-lane E8M0 factor 2^(m - m0), so O is rarely rescaled.
  float m0 = 0.0f;
  int pscale = 127;
  v16f o[D / 32];
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) o[ct] = v16f{};
  v16i sc[2];   // S of the tile between its matrix and vector phases
  v8h pf[4];    // fp16 P (between the vector phase and the next matrix phase)
  v8i pf8 = {};  // E4M3 P
  // FP8: the tile's fp32 P, from its softmax (vector phase) to the next matrix
  // phase, which packs it to E4M3 and adds it into l in the shadow of its
  // Q.K^T MFMAs (the vector phase is the longer one on this path)
  float pr8[FP8 ? 32 : 1];

  // E4M3 V^T operand of channels 32ct .. 32ct+31 of the tile at LDS byte
  // offset vso: four transposed reads of 8 keys (16 keys apart in the tile)
  auto vread8 = [&](uint32_t vso, int ct) {
    v2i r[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      r[rr] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS v2i*)(lds + vso + vaddr8[ct] + 16 * rr * S::VROW));
    return v8i{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };
  // O^T += V^T . P^T for the tile at LDS byte offset vso
  auto pv = [&](uint32_t vso) {
    if constexpr (!FP8) {
      uint32_t va[D / 32];
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) va[ct] = vso + vaddr[ct];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const lds_u8* pa = lds + va[ct] + 16 * u * S::VROW;
          const v4h ha = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)pa));
          const v4h hb = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)(pa + 8 * S::VROW)));
          const v8h vf = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[u], o[ct], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct)
        o[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vread8(vso, ct), pf8, o[ct], 0, 0, 0, 127, 0, pscale);
    }
  };

  // k_scale * q_scale * log2(e) for the keys of tile t this lane handles
  // (per (jt, group of 4 keys); one value when key blocks are multiples of
  // the tile).  Loaded before the phase's tile loads are issued so that waiting
  // for it does not wait for them.
  struct Ck {
    float c[2][4];
  };
  auto load_ck = [&](int t) {
    Ck ck;
    const int j0 = t * BN;
    if constexpr (KSU) {
      // one value per tile, from the LDS table (longer sequences: a scalar
      // load, counted by lgkmcnt rather than by the tile loads' vmcnt); 4-bit:
      // the scales are inside S
      float v = (QK4 || DUMP) ? qsc
                              : qsc * (ks_in_lds ? *(const LDS float*)(lds + S::KSTAB + 4 * t)
                                                 : keff(ksc_c[min(j0, L - 1) / p.blk_k]));
      // 22 significant bits: 1.5*2^23 * c is then exact in fp32 (3 times a
      // 22-bit integer fits 24 bits), which the exponent's FMA relies on
      if constexpr (!QK4) v = __uint_as_float((__float_as_uint(v) + 2u) & ~3u);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int q = 0; q < 4; ++q) ck.c[jt][q] = v;
    } else {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + 32 * jt + 8 * q + 4 * g;
          const float v = ksc[min(j, L - 1) / p.blk_k];  // unconditional: one batch of loads, one wait
          ck.c[jt][q] = j < L ? qsc * v : 0.0f;
        }
    }
    return ck;
  };

  // softmax of tile t from sc -> pf / pf8 (lane: row i, keys j(jt, r)).
  // MASKED tiles (sequence tail, causal diagonal) take a separate instantiation.
  auto softmax = [&](int t, const Ck& ck, uint32_t dslot, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int j0 = t * BN;
    const auto& c = ck.c;
    // smooth Q: x' = S + delta_j / (qs ks), in place of the raw scores.  The
    // INT8 seed goes first (exact: S is an integer below 2^22), so the sum is
    // rounded at the size of the score, not of 1.5*2^23 (4-bit: S has none).
    if constexpr (SQ) {
      const float f = __builtin_amdgcn_rcpf(c[0][0]) * kLog2e;
      const lds_u8* dl = lds + dslot + 16 * g;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4f d4 = *(const LDS v4f*)(dl + 4 * (32 * jt + 8 * q));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sc[jt][4 * q + e] = __float_as_int(
                __builtin_fmaf(d4[e], f, __int_as_float(sc[jt][4 * q + e]) - (QK4 ? 0.0f : kMagic)));
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
      // (without smooth Q every real x is > 0, so 0 stands for a masked key)
      auto xv = [&](int jt, int r) {
        const float xx = __int_as_float(sc[jt][r]);
        if constexpr (MASKED) return valid[jt][r] ? xx : (NEGX ? -INFINITY : 0.0f);
        return xx;
      };
      // four independent max3 chains (one wave does all the VALU work of a
      // phase, so a single chain would leave the VALU waiting on its latency)
      float mx;
      if constexpr (!NEGX) {
        // every x is a positive float, or 0 for a masked key, so its bits order
        // as integers: v_max3_i32 on the raw sums, with none of the
        // canonicalising v_max_f32 that a float maximum of them costs
        auto xi = [&](int jt, int r) {
          if constexpr (MASKED) return valid[jt][r] ? sc[jt][r] : 0;
          return sc[jt][r];
        };
        int mc[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) mc[c4] = max(xi(c4 >> 1, 8 * (c4 & 1)), xi(c4 >> 1, 8 * (c4 & 1) + 1));
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int r = 2; r < 8; r += 2)
            mc[c4] = max(max(mc[c4], xi(c4 >> 1, 8 * (c4 & 1) + r)), xi(c4 >> 1, 8 * (c4 & 1) + r + 1));
        mx = __int_as_float(max(max(mc[0], mc[1]), max(mc[2], mc[3])));
      } else {
        float mc[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) mc[c4] = fmaxf(xv(c4 >> 1, 8 * (c4 & 1)), xv(c4 >> 1, 8 * (c4 & 1) + 1));
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int r = 2; r < 8; r += 2)
            mc[c4] = fmaxf(fmaxf(mc[c4], xv(c4 >> 1, 8 * (c4 & 1) + r)), xv(c4 >> 1, 8 * (c4 & 1) + r + 1));
        mx = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
      }
      mx = xhalf_max(mx);
      // every real x is >= 1.5*2^23 - 2^21 > 0, so 0 means "all masked": leave m alone
      // (smooth Q: a masked x is -inf, and so is mt)
      mt = (MASKED && !NEGX && mx == 0.0f) ? -INFINITY : (mx - MAG) * c[0][0];
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
    // O and l move to a new reference only in a rare, wave-uniform branch
    // (its test is the only work the common case does for it)
    auto rescale = [&](float alpha) {
      lsum *= alpha;
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) o[ct] *= alpha;
    };
    if constexpr (FP8) {
      // integer running maximum; the first finite one becomes the reference m0
      mt = ceilf(mt);
      if (m == -INFINITY) m0 = mt;
      m = fmaxf(m, mt);
      // O keeps the reference m0 unless m runs more than 100 past it; then O
      // and l move to the new reference m0 = m.
      if (__builtin_expect(__any(m - m0 > 100.0f), 0)) {
        const float mn0 = (m - m0 > 100.0f) ? m : m0;
        rescale(mn0 == m0 ? 1.0f : __builtin_amdgcn_exp2f(m0 - mn0));
        m0 = mn0;
      }
      pscale = 127 + (int)(m - m0);
    } else {
      // lazy running maximum: a row moves its reference m only when the tile
      // maximum exceeds it by more than 8 (P <= 2^8 stays exact in fp16 and
      // far from overflow)
      // (kept an integer: with c below 1 the bias below is then exact, and
      // every rescale factor 2^(m_old - m_new) is a power of two)
      if (__builtin_expect(__any(mt > m + 8.0f), 0)) {
        const float mn = mt > m + 8.0f ? ceilf(mt) : m;
        rescale(mn == m ? 1.0f : __builtin_amdgcn_exp2f(m - mn));
        m = mn;
      }
    }
    const float mref = FP8 ? m - kLog2_448 : m;  // FP8: P scaled by 448 inside the exponent
    // Exponent x c - (MAG c + mref), one FMA per score.  The FMA rounds once,
    // at the size of the result; what remains is the rounding of the bias
    // MAG c + mref, the same for every key of the tile but not from tile to
    // tile.  fp16 P.V: c has 22 significant bits, so MAG c = 3 * 2^22 * c is
    // an exact multiple of twice c's last bit, and m is an integer; while c <
    // 1 that unit divides m too and the sum stays below 2^24 of them (|m| <=
    // 2^21 c + 9), so the bias is exact (for c below 2^-18, where m is the
    // larger term, it is rounded at the size of m only).  FP8: mref = m -
    // log2(448) is not an integer; the bias is rounded up (by at least its
    // rounding error), so 448 P never exceeds 448, and its error, at most an
    // ulp of MAG c, stays below 2^-10 log2 units while c < 2^-9 (scores of
    // unit-scale Q and K have c ~ 2^-12).  Larger c (any lane) take the slow
    // form: the seed subtracted first, exactly, one more instruction per
    // score.
    bool slow = false;
    if constexpr (BIASED) slow = __builtin_expect(__any(c[0][0] >= (FP8 ? 0x1p-9f : 1.0f)), 0);
    float bias = __builtin_fmaf(MAG, c[0][0], mref);
    if constexpr (BIASED && FP8) bias = __builtin_fmaf(__builtin_fabsf(bias), 0x1p-23f, bias);
    auto prob = [&](int jt, int r, auto slow_tag) {
      constexpr bool SLOW = decltype(slow_tag)::value;
      float arg;
      if constexpr (!KSU)
        arg = y[jt][r] - mref;
      else if constexpr (SLOW)
        arg = __builtin_fmaf(__int_as_float(sc[jt][r]) - kMagic, c[0][0], -mref);
      else
        arg = __builtin_fmaf(__int_as_float(sc[jt][r]), c[0][0], -bias);
      if constexpr (MASKED) arg = valid[jt][r] ? arg : -INFINITY;
      return __builtin_amdgcn_exp2f(arg);
    };
    if constexpr (!FP8) {
      // Row sums.  On gfx950 v_dot2_f32_f16 barely advances while the other
      // wave of the SIMD streams MFMAs (measured: ~4% of its rate; plain VALU
      // ops keep ~80%), so at D = 128, where the matrix phase is as long as
      // this one, the sums are fp32 adds over the unrounded P (four chains).
      // At D = 64 the matrix phase is short and this phase is the longer one:
      // the 16 dot2 over the fp16 P (two chains) cost less than 32 adds.
      auto emit = [&](auto slow_tag) {
        float ls[4];
        const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = prob(u >> 1, 8 * (u & 1) + e, slow_tag), p1 = prob(u >> 1, 8 * (u & 1) + e + 1, slow_tag);
            const v2h hp = {(_Float16)p0, (_Float16)p1};
            if constexpr (D == 128) {
              ls[e >> 1] = u == 0 ? p0 + p1 : ls[e >> 1] + (p0 + p1);
            } else {
              const int a = (e >> 1) & 1;
              ls[a] = __builtin_amdgcn_fdot2(hp, ones, (u == 0 && e < 4) ? 0.0f : ls[a], false);
            }
            pf[u][e] = hp[0];
            pf[u][e + 1] = hp[1];
          }
        lsum += D == 128 ? (ls[0] + ls[1]) + (ls[2] + ls[3]) : ls[0] + ls[1];
      };
      if (BIASED && slow)
        emit(std::true_type{});
      else
        emit(std::false_type{});
      // P is complete here, in this (vector) phase: otherwise the compiler
      // sinks the exponentials into the next matrix phase, next to their use
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v4i x = __builtin_bit_cast(v4i, pf[u]);
        asm volatile("" : "+v"(x));
        pf[u] = __builtin_bit_cast(v8h, x);
      }
      asm volatile("" : "+v"(lsum));
    } else {
      auto emit = [&](auto slow_tag) {
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r) pr8[16 * jt + r] = prob(jt, r, slow_tag);
      };
      if (BIASED && slow)
        emit(std::true_type{});
      else
        emit(std::false_type{});
      // P is complete here, in this (vector) phase
#pragma unroll
      for (int j = 0; j < 32; ++j) asm volatile("" : "+v"(pr8[j]));
    }
  };
  // FP8: E4M3 P for the P.V MFMA and l += sum of P (relative to m0, at this
  // tile's scale 2^(pscale - 127)), in 8 pieces of 4 keys (word w of pf8):
  // pieces 0-3 at the end of the vector phase, 4-7 spread over the next
  // matrix phase's Q.K^T MFMAs (the split that balances the two phases best:
  // 1-2% faster than all eight in the matrix phase); fin() adds the sum to l.
  // Packing is idempotent, so the edge matrix phases simply pack all eight.
  float ps8[4];
  auto pack8 = [&](int w) {
    const float p0 = pr8[4 * w], p1 = pr8[4 * w + 1], p2 = pr8[4 * w + 2], p3 = pr8[4 * w + 3];
    // (the conversion writes one half of the word and keeps the other: the
    // previous tile's bits stand in for the half written next)
    uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, (uint32_t)pf8[w], false);
    wv = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wv, true);
    pf8[w] = (int)wv;
    const float q = (p0 + p1) + (p2 + p3);
    ps8[w & 3] = w < 4 ? q : ps8[w & 3] + q;
  };
  auto pack8_fin = [&] { lsum += __builtin_ldexpf((ps8[0] + ps8[1]) + (ps8[2] + ps8[3]), pscale - 127); };

  // Ring slots: tile t lives in K slot t % NSK and V slot t % NSV (NSK = NSV =
  // 5); ph = b % 5 is advanced at the end of every phase.
  static_assert(NSK == 5 && NSV == 5, "slot arithmetic below");
  int ph = 0;
  int pd = 0;  // smooth Q / 4-bit: b % 6, the rings of per-key data (tile t in slot t % 6)
  auto wrap = [](int x) { return x >= 5 ? x - 5 : x; };
  auto wrap6 = [](int x) { return x >= 6 ? x - 6 : x; };
  auto doffs = [](int slot) { return (uint32_t)(S::DRING + slot * 1024); };
  // 4-bit: ring of K's per-row E8M0 words (4 copies of a tile's 64 words per slot)
  auto ksoffs = [](int slot) { return (uint32_t)(S::DRING + (SQ ? S::DBYTES : 0) + slot * 1024); };
  auto koff = [](int slot) { return (uint32_t)(slot * S::KBYTES); };
  auto voff = [](int slot) { return (uint32_t)(S::VRING + slot * S::VBYTES); };
  // Tile loads.  The half that owns tile t (t = hf mod 2) loads K(t) in its
  // matrix phase t-4 and V(t) in its matrix phase t-2 (V is first read in
  // phase t+2), and waits for both at the end of its vector phase t-1, with
  // the loads of its matrix phase t-2 still in flight: ~3.5 phases of latency
  // hidden.  The barrier after that publishes them for the matrix phases t
  // (K) and t+2 (V), run by the same half.  K and V go straight to LDS.
  // Descriptors of this half's next K and V tiles: base at the tile's first
  // row, size up to the sequence's end.
  const int8_t* knext = kseq + (int64_t)hf * BN * kn;
  const uint8_t* vnext = vseq + (int64_t)hf * BN * vn;
  // (fp16 V rows hold dv channels: the last row is read up to them only; E4M3
  // V rows are the pre-pass's, of D channels)
  int krec = (int)((L - 1 - hf * BN) * kn + S::KROW);
  int vrec = DUMP ? -(1 << 30) : (int)((L - 1 - hf * BN) * vn + (FP8 ? D : 2 * p.dv));
  const int kstep = (int)(2 * BN * kn), vstep = (int)(2 * BN * vn);
  // smooth Q: this half's next compensation tile, with K (fp32 per key of this query head)
  const float* dnext = SQ ? a.q_delta + seq_head_base(p.cu, a.qds, s, h, p.total) + hf * BN : nullptr;
  int drec = (L - hf * BN) * 4;
  constexpr int dstep = 2 * BN * 4;
  // 4-bit: this half's next tile of K's E8M0 words (one 32-bit word per key, head kvh)
  const uint8_t* ksnext = QK4 ? a.ksc4 + seq_head_base(p.cu, a.kss4, s, kvh, p.total) + (int64_t)hf * BN * a.kss4.n : nullptr;
  int ksrec = (L - hf * BN) * 4;
  const int ksstep = QK4 ? (int)(2 * BN * a.kss4.n) : 0;
  const int wh = w & 3, tidh = tid & (NWH * 64 - 1);  // wave and thread within the half
  constexpr int KL = DmaPlan<D, FP8, QK4>::KPW, VL = DmaPlan<D, FP8, QK4>::VPW;
  constexpr int NOPS = KL + VL + (SQ ? 1 : 0) + (QK4 ? 1 : 0);  // DMA loads per wave per matrix phase
  constexpr int QKM = 2 * (QK4 ? D / 64 : D / 32);              // Q.K^T MFMAs per tile
  static_assert(8 % QKM == 0, "FP8 packing pieces per Q.K^T MFMA");
  // Every matrix phase issues NOPS DMA loads per wave: VL for V, then KL for
  // K, then (smooth Q, 4-bit) one for the per-key words.  At the end of a
  // vector phase the loads of the previous matrix phase may stay in flight:
  // s_waitcnt vmcnt(NOPS).
  auto wait_older = [&] {
    constexpr int n = NOPS;
    static_assert(n >= 1 && n <= 7, "wait counts below");
    if constexpr (n == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else if constexpr (n == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (n == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if constexpr (n == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (n == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else if constexpr (n == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  };

  // ---- prologue.  With a partial last tile the V ring starts zeroed: the
  // rows of that tile past the sequence are never loaded, and their (masked,
  // P = 0) keys must still meet finite V (fp16, or an E4M3 code that is not
  // NaN; later tiles leave codes of the pre-pass there, all finite).
  // Everything else a masked key reads may be anything: K codes are finite
  // by construction, and scores of masked keys are replaced, not scaled.  Then, in one batch of loads in
  // flight together with the Q fragments: half h's tiles K(h), K(h+2) and V(h)
  // (empty descriptors past the end) and the per-tile k_scale table.
  if ((L % BN) != 0) {
    for (int x = tid; x < NSV * S::VBYTES / 16; x += NT) *(LDS v4i*)(lds + S::VRING + 16 * x) = v4i{0, 0, 0, 0};
    // The zeroes are in place before any tile lands: this wave's LDS stores
    // are complete, then the barrier (the branch is the same for the whole
    // workgroup).  Not __syncthreads: its fence would also wait for the Q
    // fragments and Q scale loaded above, whose latency should overlap the
    // tile loads below; the wait at the end of the prologue drains them.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  {
    constexpr int KSPT = S::KSCAP / NT;  // k_scale table entries per thread
    float ksv[KSPT];
    if (ks_in_lds)
#pragma unroll
      for (int j = 0; j < KSPT; ++j) {
        const int t = tid + j * NT;
        ksv[j] = t < ntiles ? keff(ksc[(t * BN) / p.blk_k]) : 0.0f;
      }
    dma.issue_v(make_rsrc(vnext, max(vrec, 0)), lds + voff(hf), wh);
    vnext += vstep;
    vrec -= vstep;
    dma.issue_k(make_rsrc(knext, max(krec, 0)), lds + koff(hf), wh);
    dma.issue_k(make_rsrc(knext + kstep, max(krec - kstep, 0)), lds + koff(hf + 2), wh);
    knext += 2 * kstep;
    krec -= 2 * kstep;
    if constexpr (SQ) {
      dma.issue_d(make_rsrc(dnext, max(drec, 0)), lds + doffs(hf));
      dma.issue_d(make_rsrc(dnext + 2 * BN, max(drec - dstep, 0)), lds + doffs(hf + 2));
      dnext += 4 * BN;
      drec -= 2 * dstep;
    }
    if constexpr (QK4) {
      dma.issue_d(make_rsrc(ksnext, max(ksrec, 0)), lds + ksoffs(hf));
      dma.issue_d(make_rsrc(ksnext + ksstep, max(ksrec - dstep, 0)), lds + ksoffs(hf + 2));
      ksnext += 2 * ksstep;
      ksrec -= 2 * dstep;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (ks_in_lds)
#pragma unroll
      for (int j = 0; j < KSPT; ++j) {
        const int t = tid + j * NT;
        if (t < ntiles) *(LDS float*)(lds + S::KSTAB + 4 * t) = ksv[j];
      }
  }
  // The compiler's own bookkeeping of outstanding loads (Q, the k_scale
  // table) ends here: it must not add waits for them inside the loop, where
  // they would also wait for the tile loads it does not see.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  asm volatile("" : "+v"(qraw), "+v"(wq));
  if constexpr (QK4) {
    qsc = kLog2e;
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) qsb[kk] = (int)((wq >> (8 * (2 * kk + g))) & 0xFFu);
  } else if (i < L) {
    qsc = qeff(qraw) * kLog2e;
  }

  // ---- phases b = 0 .. ntiles+1, in pairs.  Matrix phase b: S of tile b and
  // P.V of tile b-2, and the loads V(b+2), K(b+4); vector phase b: softmax of
  // tile b-1, then wait for K(b+1), V(b-1).  Half 0 runs (matrix, vector) in
  // each pair, half 1 (vector, matrix).  FULL pairs have every step valid and
  // unmasked for this wave and run without checks.
  const int nph = ntiles + 2;
  auto end_phase = [&](int b, bool vector_phase) {
    if (vector_phase) {
      // K(b+1) and V(b-1) must have landed; in flight from matrix phase b-1
      // may stay: V(b+1), then K(b+3)
      wait_older();
    }
    // nothing moves across the phase boundary (the other half's work of the
    // next phase must not start in this one)
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    ph = wrap(ph + 1);
    if constexpr (SQ || QK4) pd = wrap6(pd + 1);
  };
  // Matrix phase with every LDS operand read well ahead of its MFMA: all K
  // fragments and the first V group; then the INT8 MFMAs with this phase's
  // tile loads (op(0) .. op(NOPS-1)) issued one per MFMA, in their shadow;
  // then per group of D/32 P.V MFMAs the V reads of the next group.
  // 4-bit S^T of one tile (edge phases): K codes from the K slot, K's E8M0 words
  // from the ring slot kss
  auto qk4_tile = [&](uint32_t kso, uint32_t kss) {
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const uint32_t wk = *(const LDS uint32_t*)(lds + kss + 4 * (32 * jt + li));
      v16f acc = {};
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk) {
        const v4i kv = *(const LDS v4i*)(lds + kso + kofs[kk] + 32 * jt * S::KROW);
        const v8i ka = __builtin_shufflevector(kv, kv, 0, 1, 2, 3, 4, 5, 6, 7);
        const v8i qb = __builtin_shufflevector(qf[kk], qf[kk], 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qb, acc, 4, 4, 0,
                                                              (int)((wk >> (8 * (2 * kk + g))) & 0xFFu), 0, qsb[kk]);
      }
      sc[jt] = __builtin_bit_cast(v16i, acc);
    }
  };
  auto qk_pv = [&](uint32_t kso, uint32_t vso, uint32_t kss, auto&& op) {
    constexpr int KK = QK4 ? D / 64 : D / 32;  // Q.K^T MFMAs per 32-key block
    v4i kf[2][D / 32];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kf[jt][kk] = *(const LDS v4i*)(lds + kso + kofs[kk] + 32 * jt * S::KROW);
    // 4-bit: the E8M0 code of key 32jt + li, channel block 2kk + g
    int ksb[2][D / 64] = {};
    if constexpr (QK4) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const uint32_t wk = *(const LDS uint32_t*)(lds + kss + 4 * (32 * jt + li));
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) ksb[jt][kk] = (int)((wk >> (8 * (2 * kk + g))) & 0xFFu);
      }
    }
    // FP8: the previous tile's P packed and summed, pieces 4-7 (the vector
    // phase did 0-3), 8 / QKM pieces per Q.K^T MFMA
    auto fill = [&](int x) {
      if constexpr (FP8) {
#pragma unroll
        for (int y = 0; y < 8 / QKM; ++y)
          if (x * (8 / QKM) + y >= 4) pack8(x * (8 / QKM) + y);
      }
    };
    // (sched_barrier(0): the instruction order below is the schedule)
    auto qk_mfmas = [&] {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        if constexpr (QK4) {
          v16f acc = {};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const v8i ka = __builtin_shufflevector(kf[jt][kk], kf[jt][kk], 0, 1, 2, 3, 4, 5, 6, 7);
            const v8i qb = __builtin_shufflevector(qf[kk], qf[kk], 0, 1, 2, 3, 4, 5, 6, 7);
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qb, acc, 4, 4, 0, ksb[jt][kk], 0, qsb[kk]);
            if (jt * KK + kk < NOPS) op(jt * KK + kk);
            fill(jt * KK + kk);
            __builtin_amdgcn_sched_barrier(0);
          }
          sc[jt] = __builtin_bit_cast(v16i, acc);
        } else {
          v16i acc = magic;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[jt][kk], qf[kk], acc, 0, 0, 0);
            if (jt * KK + kk < NOPS) op(jt * KK + kk);
            fill(jt * KK + kk);
            __builtin_amdgcn_sched_barrier(0);
          }
          sc[jt] = acc;
        }
      }
    };
    // tile loads beyond the Q.K^T MFMAs go with the P.V MFMAs
    auto spill = [&](int x) {
      if (QKM + x < NOPS) op(QKM + x);
    };
    if constexpr (!FP8) {
      uint32_t va[D / 32];
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) va[ct] = vso + vaddr[ct];
      v8h vf[4][D / 32];
      auto vread = [&](int u) {
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          const lds_u8* pa = lds + va[ct] + 16 * u * S::VROW;
          const v4h ha = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)pa));
          const v4h hb = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4s*)(pa + 8 * S::VROW)));
          vf[u][ct] = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      vread(0);
      __builtin_amdgcn_sched_barrier(0);
      qk_mfmas();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u + 1 < 4) vread(u + 1);
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct) {
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[u][ct], pf[u], o[ct], 0, 0, 0);
          spill(u * (D / 32) + ct);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      v8i vf[D / 32];
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) vf[ct] = vread8(vso, ct);
      __builtin_amdgcn_sched_barrier(0);
      qk_mfmas();
      pack8_fin();
#pragma unroll
      for (int ct = 0; ct < D / 32; ++ct) {
        o[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[ct], pf8, o[ct], 0, 0, 0, 127, 0, pscale);
        spill(ct);
      }
    }
    static_assert(NOPS <= QKM + (FP8 ? D / 32 : D / 8), "every tile load has an MFMA to go with");
  };
  auto mphase = [&](int b, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
    // Loads V(b+2), then K(b+4), of tiles owned by this half, as NOPS single
    // loads.  They are issued whether or not the tile exists (past the end
    // the descriptor is empty: nothing is read, the slot written holds a
    // consumed tile), so every matrix phase has the same count in flight.
    const v4i vr = make_rsrc(vnext, max(vrec, 0)), kr = make_rsrc(knext, max(krec, 0));
    lds_u8* const vsl = lds + voff(wrap(ph + 2));
    lds_u8* const ksl = lds + koff(wrap(ph + 4));
    v4i dr{}, ksr{};
    lds_u8* dsl = nullptr;
    lds_u8* kssl = nullptr;
    if constexpr (SQ) {
      dr = make_rsrc(dnext, max(drec, 0));
      dsl = lds + doffs(wrap6(pd + 4));  // delta(b+4), with K(b+4)
    }
    if constexpr (QK4) {
      ksr = make_rsrc(ksnext, max(ksrec, 0));
      kssl = lds + ksoffs(wrap6(pd + 4));  // K's E8M0 words of tile b+4, with K(b+4)
    }
    auto op = [&](int x) {
      if (x < VL)
        dma.issue_v1(vr, vsl, wh, x);
      else if (x < VL + KL)
        dma.issue_k1(kr, ksl, wh, x - VL);
      else if (SQ && x == VL + KL)
        dma.issue_d(dr, dsl);
      else if constexpr (QK4)
        dma.issue_d(ksr, kssl);
    };
    if (FULL) {
      qk_pv(koff(ph), voff(wrap(ph + 3)), ksoffs(pd), op);
    } else {
#pragma unroll
      for (int x = 0; x < NOPS; ++x) op(x);
      if (b >= 2 && b - 2 < wtiles) {
        if constexpr (FP8) {
#pragma unroll
          for (int w8 = 0; w8 < 8; ++w8) pack8(w8);
          pack8_fin();
        }
        pv(voff(wrap(ph + 3)));
      }
      if (b < wtiles) {
        if constexpr (QK4)
          qk4_tile(koff(ph), ksoffs(pd));
        else
          qk_tile<D>(lds + koff(ph), kofs, qf, magic, sc);
      }
    }
    knext += kstep;
    krec -= kstep;
    vnext += vstep;
    vrec -= vstep;
    if constexpr (SQ) {
      dnext += 2 * BN;
      drec -= dstep;
    }
    if constexpr (QK4) {
      ksnext += ksstep;
      ksrec -= dstep;
    }
    end_phase(b, false);
  };
  auto vphase = [&](int b, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    // D = 128: the softmax wave gets the higher issue priority on its SIMD
    // (about 1% on these kernels, 0.1-1.2% with FP8 P.V; at D = 64 it is not
    // faster, and giving the matrix wave the priority is 1-3% slower, 11%
    // with FP8 P.V)
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
    const int t = b - 1;
    const Ck ck = load_ck(min(max(t, 0), ntiles - 1));  // (t outside the tiles: value unused)
    const uint32_t dslot = doffs(wrap6(pd + 5));         // tile t = b - 1 (smooth Q)
    if constexpr (DUMP) {
      if ((FULL || (t >= 0 && t < wtiles)) && i < L) {
        int32_t* drow = a.dump + (sh * p.max_seqlen + i) * p.max_seqlen;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = t * BN + 32 * jt + 8 * q + 4 * g;
            if (j < L)
              *reinterpret_cast<v4i*>(drow + j) =
                  v4i{sc[jt][4 * q] - kMagicBits, sc[jt][4 * q + 1] - kMagicBits, sc[jt][4 * q + 2] - kMagicBits,
                      sc[jt][4 * q + 3] - kMagicBits};
          }
      }
    }
    if (FULL) {
      softmax(t, ck, dslot, std::false_type{});
    } else if (t >= 0 && t < wtiles) {
      const bool masked = (t * BN + BN > L) || (CAUSAL && t * BN + BN - 1 > row0);
      if (masked)
        softmax(t, ck, dslot, std::true_type{});
      else
        softmax(t, ck, dslot, std::false_type{});
    }
    if constexpr (FP8) {
      // pieces 0-3 of this tile's E4M3 P (whatever pr8 holds when no tile was
      // processed: the matrix phase that uses P repacks or never reads it)
#pragma unroll
      for (int w8 = 0; w8 < 4; ++w8) pack8(w8);
    }
    end_phase(b, true);
  };
  // tiles every key of which this wave sees (unmasked)
  const int tu = CAUSAL ? min(L / BN, (row0 + 1) / BN) : L / BN;
  auto run = [&](auto hf_tag) {
    constexpr int HF = decltype(hf_tag)::value;
    // FULL pair b0 (even): half 0: S(b0), P.V(b0-2), softmax(b0);
    //                      half 1: softmax(b0-1), P.V(b0-1), S(b0+1)
    const int bend = HF == 0 ? tu : min(tu + 1, wtiles - 1);
    auto pair = [&](int b0, auto full_tag) {
      if constexpr (HF == 0) {
        mphase(b0, full_tag);
        vphase(b0 + 1, full_tag);
      } else {
        vphase(b0, full_tag);
        mphase(b0 + 1, full_tag);
      }
    };
    pair(0, std::false_type{});
    int b0 = 2;
    for (; b0 < bend; b0 += 2) pair(b0, std::true_type{});
    for (; b0 < nph; b0 += 2) pair(b0, std::false_type{});
  };
  if (hf == 0)
    run(std::integral_constant<int, 0>{});
  else
    run(std::integral_constant<int, 1>{});

  // ---- merge the halves: half 1 leaves (O^T, m_ref, l) in LDS, half 0 combines.
  // m_ref is the exponent O and l are relative to (fp16: m; FP8: m0), -inf
  // if this half saw no key of the row.  O^T goes as 16-byte pieces: piece j
  // (accumulators 4j .. 4j+3) of lane l at float (4j * 64 + 4l) of the wave's
  // area (a wave's 64 lanes cover 1 KiB per piece: conflict-free).
  float* const mgw = (float*)lds + (w & 3) * S::MSTRIDE * 64;
  float* const mg = mgw + lane;
  const float mref_own = m == -INFINITY ? -INFINITY : (FP8 ? m0 : m);
  // FP8: the channel scales (and means) of this lane's pieces, loaded now so
  // that their latency overlaps the merge
  v4f vsc[FP8 ? D / 8 : 1], vmu[FP8 ? D / 8 : 1];
  if constexpr (FP8) {
    if (hf == 0) {
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const int cc = 32 * (j / 4) + 8 * (j % 4) + 4 * g;
        vsc[j] = *reinterpret_cast<const v4f*>(a.v_scale + skv * D + cc);
        vmu[j] = a.v_mean ? *reinterpret_cast<const v4f*>(a.v_mean + skv * D + cc) : v4f{0, 0, 0, 0};
      }
    }
  }
  // the last matrix phases' loads (past the last tile) are still in flight and
  // write into the ring, which the partial results reuse
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (hf == 1) {
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(LDS v4f*)(mgw + (4 * ct + q) * 256 + 4 * lane) =
            v4f{o[ct][4 * q], o[ct][4 * q + 1], o[ct][4 * q + 2], o[ct][4 * q + 3]};
    mg[(D / 2) * 64] = mref_own;
    mg[(D / 2 + 1) * 64] = lsum;
  }
  __syncthreads();
  if (hf == 1) return;
  const float mref_b = mg[(D / 2) * 64], lsum_b = mg[(D / 2 + 1) * 64];
  const float mmax = fmaxf(mref_own, mref_b);
  const float wa = mref_own == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mref_own - mmax);
  const float wb = mref_b == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mref_b - mmax);

  // ---- epilogue: O = O^T / l (FP8: l and O both carry the factor 448; times
  // v_scale).  A lane holds 4-channel pieces of its row; the fp16 rows go
  // through LDS so that the stores write whole rows (16 lanes per row).
  const float inv = 1.0f / xhalf_sum(lsum * wa + lsum_b * wb);
  const float ca = wa * inv, cb = wb * inv;
  lds_u8* const ostage = lds + S::OSTAGE;
  // all of half 1's pieces first (the O staging writes below could alias them
  // as far as the compiler knows, which would serialise read, wait and write)
  v4f ob[D / 8];
#pragma unroll
  for (int j = 0; j < D / 8; ++j) ob[j] = *(const LDS v4f*)(mgw + j * 256 + 4 * lane);
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q + e;
        f[e] = o[ct][r] * ca + ob[4 * ct + q][e] * cb;
        if constexpr (FP8) f[e] = f[e] * vsc[4 * ct + q][e] + vmu[4 * ct + q][e];  // smoothed V: P (V - mean) + mean
      }
      const int cc = 32 * ct + 8 * q + 4 * g;
      const v4h hv = {(_Float16)f[0], (_Float16)f[1], (_Float16)f[2], (_Float16)f[3]};
      *(LDS v4h*)(ostage + (i - q0) * S::OROW + 2 * cc) = hv;
    }
  __syncthreads();  // (half 1 has ended: the barrier waits for half 0's waves)
  _Float16* __restrict__ obase = (_Float16*)a.out + seq_head_base(p.cu, a.os, s, h, p.total);
  constexpr int CPR = D / 8;  // 16-byte pieces per row
  constexpr int NPC = BM * CPR / (NT / 2);
  v4i opc[NPC];  // (all LDS reads first, then the stores)
#pragma unroll
  for (int x = 0; x < NPC; ++x) {
    const int c = tid + x * (NT / 2), rr = c / CPR, cp = c % CPR;
    opc[x] = *(const LDS v4i*)(ostage + rr * S::OROW + 16 * cp);
  }
#pragma unroll
  for (int x = 0; x < NPC; ++x) {
    const int c = tid + x * (NT / 2), rr = c / CPR, cp = c % CPR;
    if (!DUMP && q0 + rr < L && 8 * cp < p.dv)
      *reinterpret_cast<v4i*>(obase + (int64_t)(q0 + rr) * a.os.n + 8 * cp) = opc[x];
  }
}

template <int D, bool FP8, bool CAUSAL, bool KSU, bool SQ, bool QK4, bool DUMP = false>
__global__ __launch_bounds__(NT) void k_attn(Problem p, AttnArgs a) {
  using S = Lds<D, FP8, QK4>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[S::BYTES + (SQ ? S::DBYTES : 0) + (QK4 ? S::DBYTES : 0)];
  attn_body<D, FP8, CAUSAL, KSU, SQ, QK4, DUMP>(p, a, (lds_u8*)lds_raw);
}

template <int D, bool FP8, bool CAUSAL, bool KSU, bool SQ, bool QK4 = false, bool DUMP = false>
hipError_t launch_cfg(const Problem& p, const AttnArgs& a, hipStream_t st) {
  const int nqt = (p.max_seqlen + BM - 1) / BM;
  // slots per XCD: ceil(groups / 8) groups of heads/kv_heads query heads
  const int64_t P8 = ((int64_t)p.nseq * p.kv_heads + 7) / 8 * 8 * (p.heads / p.kv_heads);
  const int64_t G = (int64_t)nqt * P8;
  if (G >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_attn<D, FP8, CAUSAL, KSU, SQ, QK4, DUMP>), dim3((unsigned)G), dim3(NT), 0, st, p, a);
  return hipGetLastError();
}

template <int D, bool FP8, bool CAUSAL>
hipError_t launch_ks(const Problem& p, const AttnArgs& a, hipStream_t st) {
  if constexpr (D == 128) {
    if (a.qsc4) {  // 4-bit Q.K^T (MXFP4), with or without smooth Q
      return a.q_delta ? launch_cfg<D, FP8, CAUSAL, true, true, true>(p, a, st)
                       : launch_cfg<D, FP8, CAUSAL, true, false, true>(p, a, st);
    }
  } else if (a.qsc4) {
    return hipErrorInvalidValue;
  }
  if (a.q_delta) {  // smooth Q (key blocks that are multiples of the tile: checked by the caller)
    if (p.blk_k % BN != 0) return hipErrorInvalidValue;
    return launch_cfg<D, FP8, CAUSAL, true, true>(p, a, st);
  }
  return (p.blk_k % BN == 0) ? launch_cfg<D, FP8, CAUSAL, true, false>(p, a, st)
                             : launch_cfg<D, FP8, CAUSAL, false, false>(p, a, st);
}

template <int D>
hipError_t launch_d(const Problem& p, const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  if (a.dump) return launch_cfg<D, false, false, true, false, false, true>(p, a, st);
  if (fp8) return causal ? launch_ks<D, true, true>(p, a, st) : launch_ks<D, true, false>(p, a, st);
  return causal ? launch_ks<D, false, true>(p, a, st) : launch_ks<D, false, false>(p, a, st);
}

// One wave: D = A . B * 2^(sa - 127) * 2^(sb - 127) + C with the FP8 P.V
// instruction, operands in the fused kernel's layout: lane (m, g = lane/32)
// holds A[m][32g .. 32g+31] and B[32g .. 32g+31][m]; accumulator r of lane
// (n, g) is D[8(r/4) + 4g + r%4][n].  A [32][64] and B [64][32] E4M3 codes, C
// and D fp32 [32][32], all row-major.
__global__ __launch_bounds__(64) void k_debug_fp8_mfma(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                       const float* __restrict__ C, int sa, int sb,
                                                       float* __restrict__ Dout) {
  const int lane = threadIdx.x, m = lane & 31, g = lane >> 5;
  v8i av, bv;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t wa = 0, wb = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int k = 32 * g + 4 * j + t;
      wa |= (uint32_t)A[m * 64 + k] << (8 * t);
      wb |= (uint32_t)B[k * 32 + m] << (8 * t);
    }
    av[j] = (int)wa;
    bv[j] = (int)wb;
  }
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = C[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + m];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, sb);
#pragma unroll
  for (int r = 0; r < 16; ++r) Dout[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + m] = acc[r];
}

// One wave: D = A . B + C with the instruction's MXFP4 form (E2M1 operands,
// format code 4): lane (m, g) holds A[m][32g .. 32g+31] as 16 bytes, element
// k in byte k/2 (low nibble first), with its E8M0 scale sa[m][g]; likewise
// B[32g .. 32g+31][n] with sb[g][n]; each lane's scale applies to its own 32
// products.  A [32][64] and B [64][32]: one E2M1 code per byte; sa [32][2], sb
// [2][32] E8M0 codes; C and D fp32 [32][32], all row-major.
__global__ __launch_bounds__(64) void k_debug_mxfp4_mfma(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                         const uint8_t* __restrict__ SA, const uint8_t* __restrict__ SB,
                                                         const float* __restrict__ C, float* __restrict__ Dout) {
  const int lane = threadIdx.x, m = lane & 31, g = lane >> 5;
  v8i av = {}, bv = {};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t wa = 0, wb = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int k = 32 * g + 8 * j + t;
      wa |= (uint32_t)(A[m * 64 + k] & 0xF) << (4 * t);
      wb |= (uint32_t)(B[k * 32 + m] & 0xF) << (4 * t);
    }
    av[j] = (int)wa;
    bv[j] = (int)wb;
  }
  const int sa = SA[m * 2 + g], sb = SB[g * 32 + m];
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = C[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + m];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, sa, 0, sb);
#pragma unroll
  for (int r = 0; r < 16; ++r) Dout[(8 * (r >> 2) + 4 * g + (r & 3)) * 32 + m] = acc[r];
}

}  // namespace

hipError_t launch_debug_mxfp4_mfma(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                   const float* c, float* d, hipStream_t st) {
  hipLaunchKernelGGL(k_debug_mxfp4_mfma, dim3(1), dim3(64), 0, st, a, b, sa, sb, c, d);
  return hipGetLastError();
}

hipError_t launch_attn(const Problem& p, const AttnArgs& a, bool causal, bool fp8, hipStream_t st) {
  return p.head_dim == 64 ? launch_d<64>(p, a, causal, fp8, st) : launch_d<128>(p, a, causal, fp8, st);
}

hipError_t launch_debug_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, int sa, int sb, float* d,
                                 hipStream_t st) {
  hipLaunchKernelGGL(k_debug_fp8_mfma, dim3(1), dim3(64), 0, st, a, b, c, sa, sb, d);
  return hipGetLastError();
}

}  // namespace sage
