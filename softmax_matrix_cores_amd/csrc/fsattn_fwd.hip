// fsattn_fwd.hip -- Fused-Softmax quantized attention forward for gfx950.
//
// The method ("Fused-Softmax shifts an AI attention bottleneck onto faster
// GPU hardware", paragraphs 5-6; "Fused softmax makes quantized attention
// faster on AMD GPUs", section "Move work, keep correction"):
//   * the row-max reference is provisionally frozen; its subtraction and the
//     affine part of Schraudolph's exponential are folded into the Q K^T
//     product: the slope (128 log2 e sigma) sits in Q-hat, the offset
//     C_i = T0 - m_i is the accumulator's initial value of the MFMA;
//   * stage 1: the integer part of the folded score is the BF16 bit pattern
//     of ~2^(score - m); stage 2: BF16 -> MX P with one E8M0 per 32 keys;
//   * O += P V and l += P 1 run on the matrix cores with the same P;
//   * a rollback gate fires when a tile's scores exceed the reference by more
//     than tau: the reference is raised and O, l are rescaled.
//
// Mapping to CDNA4:
//   * v_mfma_scale_f32_16x16x128_f8f6f4 for every product.  D = 128 is one
//     contraction, so the fold C + sum Q K is a single instruction; with FP6
//     and FP4 operands C_i lies on the grid of the scores and the sum is exact.
//   * S^T = K Q^T: the accumulator's rows are keys, its columns queries, so a
//     lane holds 32 scores of ONE query.  The K rows fed to each of the 8
//     MFMAs of a 128-key tile are permuted so that those 32 scores are exactly
//     the keys of the lane's P operand in the PV product: no transpose.
//   * a wave owns NQ blocks of 16 queries; every K and V operand read from LDS
//     feeds NQ MFMAs.  K/V tiles of 128 keys are double-buffered in LDS and
//     fetched with direct global->LDS loads while the previous tile computes.
//   * fast path per score: one float->int convert (stage 1), half a pack and
//     half a max3; the E8M0 of P comes from the block max with integer
//     exponent arithmetic and the whole 32-key block is converted by one
//     v_cvt_scalef32_pk32_fp6_bf16.  A wave ballot on the block maxima sends
//     a tile to the exact rare path when a gate might fire, when a block sits
//     so low that the BF16 subnormal flush could matter, or on tile 0.
//
// Operand lane layouts of the scaled MFMA (measured on gfx950):
//   FP6/FP4 ("contiguous"): lane (r = l%16, g = l/16) holds row r, K elements
//     [32g, 32g+32) and the scale of that 32-block.
//   FP8 ("split"): lane (r, g) holds K elements [16g, 16g+16) in bytes 0-15
//     and [64+16g, 64+16g+16) in bytes 16-31; the scale of 32-block b comes
//     from lane 16b + r.
//   Accumulator: lane (n = l%16, g) holds rows 4g..4g+3 of column n.
#include "internal.h"
#include "mx_device.h"

namespace fsattn {

template <int ELEM> struct Layout { static constexpr bool split = (Fmt<ELEM>::bits == 8); };

// V tile rows in LDS: 4 blocks of 32 keys.  A 24-byte FP6 block is stored as
// two 12-byte halves at offsets 0 and 16 of a 32-byte slot, the placement of a
// 12-byte direct global->LDS load (each lane's data lands on a 16-byte stride).
template <int VELEM> struct VRowLds {
  static constexpr int block = (Fmt<VELEM>::bits == 6) ? 32 : Fmt<VELEM>::bits * 4;
  static constexpr int bytes = 4 * block;
};

constexpr int NW = 4;    // waves per workgroup (one per SIMD)
constexpr int KT = 128;  // keys per tile
#ifndef FSATTN_LDS_DIRECT
#define FSATTN_LDS_DIRECT 1  // K/V codes by direct global->LDS loads (else through registers)
#endif
#ifndef FSATTN_NQ
#define FSATTN_NQ 2  // q-blocks of 16 queries per wave
#endif

template <int ELEM> __device__ __forceinline__ constexpr int block_bytes() { return Fmt<ELEM>::bits * 4; }

// Smallest BF16 pattern of a P block max for which BF16 subnormals of the
// block convert to +0 anyway (x/X at most half the format's smallest
// subnormal): exponent field >= 7 (E2M3), 10 (E3M2), 19 (E4M3).
template <int PELEM> struct PFlush;
template <> struct PFlush<E2M3> { static constexpr float t = 896.0f; };
template <> struct PFlush<E3M2> { static constexpr float t = 1280.0f; };
template <> struct PFlush<E4M3> { static constexpr float t = 2432.0f; };

// a lane's 32 K elements of a row laid out as consecutive 32-element blocks
template <int ELEM, int D>
__device__ __forceinline__ v8i load_row_operand(const uint8_t* row, int g) {
  v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (Layout<ELEM>::split) {
    const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * g);
    a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
    if constexpr (D == 128) {
      const uint4 hi = *reinterpret_cast<const uint4*>(row + 64 + 16 * g);
      a[4] = hi.x; a[5] = hi.y; a[6] = hi.z; a[7] = hi.w;
    }
  } else {
    constexpr int BB = block_bytes<ELEM>();
    if (D == 128 || g < 2) {
      const uint8_t* p = row + BB * g;
      if constexpr (BB == 24) {
        const uint2* p2 = reinterpret_cast<const uint2*>(p);
        uint2 x0 = p2[0], x1 = p2[1], x2 = p2[2];
        a[0] = x0.x; a[1] = x0.y; a[2] = x1.x; a[3] = x1.y; a[4] = x2.x; a[5] = x2.y;
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(p);
        a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
      }
    }
  }
  return a;
}

// a lane's V operand (32 keys of one d row) from the LDS tile row
template <int VELEM>
__device__ __forceinline__ v8i load_v_operand(const uint8_t* row, int g) {
  if constexpr (Fmt<VELEM>::bits == 6) {
    const uint8_t* p = row + 32 * g;
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)hi.x, (int)hi.y, (int)hi.z, 0, 0};
  } else {
    return load_row_operand<VELEM, 128>(row, g);
  }
}

__device__ __forceinline__ float wshfl(float v, int src) { return __shfl(v, src, 64); }
__device__ __forceinline__ int wshfl(int v, int src) { return __shfl(v, src, 64); }

// key (0..127 in the tile) of accumulator j, row r' of lane group g
template <int PELEM>
__device__ __forceinline__ constexpr int key_of(int j, int rr, int g) {
  if constexpr (Layout<PELEM>::split) return (j < 4) ? (16 * g + 4 * j + rr) : (64 + 16 * g + 4 * (j - 4) + rr);
  else return 32 * g + 4 * j + rr;
}
// 64-key gate half of accumulator j for lane group g
template <int PELEM>
__device__ __forceinline__ constexpr int half_of(int j, int g) {
  if constexpr (Layout<PELEM>::split) return j >> 2;
  else return g >> 1;
}

// Stage 1 with the flush and clamp (rare path): BF16 bit pattern of the
// folded score.  v_cvt_u32_f32 truncates toward zero = floor for t >= 0.
__device__ __forceinline__ uint32_t stage1_exact(float t) {
  if (!(t >= 128.0f)) return 0u;
  return min(__float2uint_rz(t), 0x7F7Fu);
}

// E8M0 of a P block from its largest BF16 pattern (integer exponent math)
template <int PELEM>
__device__ __forceinline__ uint32_t p_scale(uint32_t bmax, bool fitmax) {
  constexpr int thr7 = (int)(Fmt<PELEM>::mthr23 >> 16);  // 7-bit mantissa threshold
  const int e = fitmax ? (int)((bmax + (uint32_t)(127 - thr7)) >> 7) : (int)(bmax >> 7);
  if (bmax == 0) return 0u;
  return (uint32_t)min(max(e - Fmt<PELEM>::emax, 0), 254);
}

// S^T for one q-block: 8 MFMAs over the 128-key tile with accumulator init C
template <int QK, int PELEM, int D>
__device__ __forceinline__ void scores_block(v4f (&s)[8], const uint8_t* ldsK, const uint8_t* ldsKs, const v8i& qB,
                                             int qS, float C, int lane) {
  constexpr int RB = D * Fmt<QK>::bits / 8;
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int key = key_of<PELEM>(j, m & 3, m >> 2);
    v8i a = load_row_operand<QK, D>(ldsK + key * RB, g);
    const int sa = (D == 128 || g < 2) ? (int)ldsKs[key * 4 + g] : 127;
    const v4f c = {C, C, C, C};
    s[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qB, c, QK, QK, 0, sa, 0, qS);
  }
}

// rescale O rows (queries 4g + r of this q-block) by rho of their query (held by lane q)
template <int D>
__device__ __forceinline__ void rescale(v4f (&O)[D / 16], v4f& L, float rho, int lane) {
  const int g = lane >> 4;
  float rr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rr[r] = wshfl(rho, 4 * g + r);
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) O[i][r] *= rr[r];
#pragma unroll
  for (int r = 0; r < 4; ++r) L[r] *= rr[r];
}

template <int PELEM>
__device__ __forceinline__ v8i mask_half(const v8i& pA, int g, int keep_half) {
  v8i r = pA;
  if constexpr (Layout<PELEM>::split) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (keep_half != 0) r[i] = 0;
      if (keep_half != 1) r[4 + i] = 0;
    }
  } else {
    if ((g >> 1) != keep_half) r = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }
  return r;
}

// Build the P operand (A of PV) from a lane's 32 folded scores (stage 1 + 2).
// The caller has made every score either a normal input to stage 1 or -inf.
template <int PELEM>
__device__ __forceinline__ void make_p(const v4f (&s)[8], int g, int lane, bool fitmax, v8i& pA, int& pS,
                                       uint32_t (&dsc)[2]) {
  uint32_t w[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b0 = __float2uint_rz(s[j][0]), b1 = __float2uint_rz(s[j][1]);
    const uint32_t b2 = __float2uint_rz(s[j][2]), b3 = __float2uint_rz(s[j][3]);
    w[2 * j] = __builtin_amdgcn_perm(b1, b0, 0x05040100u);
    w[2 * j + 1] = __builtin_amdgcn_perm(b3, b2, 0x05040100u);
  }
  if constexpr (!Layout<PELEM>::split) {
    float tm = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = (j == 0 ? 3 : 0); r < 4; r += 2) tm = fmaxf(fmaxf(tm, s[j][r]), (r + 1 < 4) ? s[j][r + 1] : s[j][r]);
    const uint32_t bmax = (tm >= 128.0f) ? min(__float2uint_rz(tm), 0x7F7Fu) : 0u;
    const uint32_t sc = p_scale<PELEM>(bmax, fitmax);
    v16u wv;
#pragma unroll
    for (int i = 0; i < 16; ++i) wv[i] = w[i];
    const v32bf x = __builtin_bit_cast(v32bf, wv);
    v6i r;
    if constexpr (PELEM == E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(x, e8m0_to_float(sc));
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(x, e8m0_to_float(sc));
    pA = v8i{r[0], r[1], r[2], r[3], r[4], r[5], 0, 0};
    pS = (int)sc;
    dsc[0] = sc;
    dsc[1] = sc;
  } else {
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) { m0 = fmaxf(m0, s[j][r]); m1 = fmaxf(m1, s[4 + j][r]); }
    m0 = fmaxf(m0, wshfl(m0, lane ^ 16));
    m1 = fmaxf(m1, wshfl(m1, lane ^ 16));
    const uint32_t b0 = (m0 >= 128.0f) ? min(__float2uint_rz(m0), 0x7F7Fu) : 0u;
    const uint32_t b1 = (m1 >= 128.0f) ? min(__float2uint_rz(m1), 0x7F7Fu) : 0u;
    const uint32_t s0 = p_scale<PELEM>(b0, fitmax), s1 = p_scale<PELEM>(b1, fitmax);
    const float X0 = e8m0_to_float(s0), X1 = e8m0_to_float(s1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float Xi = (i < 4) ? X0 : X1;
      v2s r = {0, 0};
      const v2bf p0 = __builtin_bit_cast(v2bf, w[2 * i]);
      const v2bf p1 = __builtin_bit_cast(v2bf, w[2 * i + 1]);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, p0, Xi, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, p1, Xi, true);
      pA[i] = (int)((uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16));
    }
    // MFMA scale of 32-block b comes from lane 16b + n:
    // b0 = first half of g=0,1 ; b1 = first half of g=2,3 ; b2 = second half of g=0,1 ; b3 = second half of g=2,3
    const int n = lane & 15;
    const int from_g2 = wshfl((int)s0, n + 32);
    const int from_g1 = wshfl((int)s1, n + 16);
    pS = (g == 0) ? (int)s0 : (g == 1) ? from_g2 : (g == 2) ? from_g1 : (int)s1;
    dsc[0] = s0;
    dsc[1] = s1;
  }
}

template <int PELEM, int VELEM, int D, int NQ>
__device__ __forceinline__ void pv_all(v4f (&O)[NQ][D / 16], v4f (&L)[NQ], const v8i (&pA)[NQ], const int (&pS)[NQ],
                                       const uint8_t* ldsV, const uint8_t* ldsVs, int lane) {
  constexpr int RB = VRowLds<VELEM>::bytes;
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int d = 16 * i + n;
    const v8i b = load_v_operand<VELEM>(ldsV + d * RB, g);
    const int sb = (int)ldsVs[d * 4 + g];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      O[q][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pA[q], b, O[q][i], PELEM, VELEM, 0, pS[q], 0, sb);
  }
  // l += P 1: ones operand (E2M1 code 0x2 = 1.0, scale 2^0)
  const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    L[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pA[q], ones, L[q], PELEM, E2M1, 0, pS[q], 0, 127);
}

// optional P dump (debug): one code byte per key and the E8M0 per 32 keys
template <int PELEM>
__device__ __forceinline__ void dump_p(const FwdArgs& a, int bh, int qq, int k0, int g, const v8i& pA,
                                       const uint32_t (&dsc)[2]) {
  if (bh != a.pd_bh || qq < a.pd_row0 || qq >= a.pd_row1 || qq >= a.Sq) return;
  const int nb32 = a.nb32;
  const size_t S32 = (size_t)nb32 * 32;
  uint8_t* drow = a.pd_codes + (size_t)(qq - a.pd_row0) * S32;
  uint8_t* srow = a.pd_scales + (size_t)(qq - a.pd_row0) * nb32;
  constexpr int bits = Fmt<PELEM>::bits;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int key = k0 + key_of<PELEM>(e >> 2, e & 3, g);
    const int pos = e * bits;
    uint32_t wv = (uint32_t)pA[pos >> 5] >> (pos & 31);
    if ((pos & 31) + bits > 32) wv |= (uint32_t)pA[(pos >> 5) + 1] << (32 - (pos & 31));
    if (key < (int)S32) drow[key] = (uint8_t)(wv & ((1u << bits) - 1));
  }
  if constexpr (Layout<PELEM>::split) {
    const int kb0 = (k0 + 16 * g) / 32, kb1 = (k0 + 64 + 16 * g) / 32;
    if (kb0 < nb32) srow[kb0] = (uint8_t)dsc[0];
    if (kb1 < nb32) srow[kb1] = (uint8_t)dsc[1];
  } else {
    const int kb = (k0 + 32 * g) / 32;
    if (kb < nb32) srow[kb] = (uint8_t)dsc[0];
  }
}

template <int PELEM, int VELEM, int D>
__device__ __forceinline__ void pv_one(v4f (&O)[D / 16], v4f& L, const v8i& pA, int pS, const uint8_t* ldsV,
                                       const uint8_t* ldsVs, int lane) {
  constexpr int RB = VRowLds<VELEM>::bytes;
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int d = 16 * i + n;
    const v8i b = load_v_operand<VELEM>(ldsV + d * RB, g);
    const int sb = (int)ldsVs[d * 4 + g];
    O[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pA, b, O[i], PELEM, VELEM, 0, pS, 0, sb);
  }
  const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
  L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pA, ones, L, PELEM, E2M1, 0, pS, 0, 127);
}

// The exact path for one q-block of a tile: tile-0 reference, rollback gate
// per 64- or 128-key gate tile (the second 64-key half is re-scored with the
// updated accumulator offset), stage-1 flush and clamp, P, and P V with the
// mid-tile rescale when the second half fires.
template <int QK, int VELEM, int PELEM, int D, bool DUMP>
__device__ __forceinline__ void rare_block(v4f (&S)[8], float& C, int& cnt, v4f (&O)[D / 16], v4f& L, const v8i& qB,
                                        int qS, int t, int nk, int k0, float T0, float Tg, const FwdArgs& a,
                                        const uint8_t* ldsK, const uint8_t* ldsKs, const uint8_t* ldsV,
                                        const uint8_t* ldsVs, int bh, int qbase, int lane) {
  const int g = lane >> 4, n = lane & 15;
  float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (half_of<PELEM>(j, g) == 0) m0 = fmaxf(m0, S[j][r]);
      else m1 = fmaxf(m1, S[j][r]);
    }
  m0 = fmaxf(m0, wshfl(m0, lane ^ 16)); m0 = fmaxf(m0, wshfl(m0, lane ^ 32));
  m1 = fmaxf(m1, wshfl(m1, lane ^ 16)); m1 = fmaxf(m1, wshfl(m1, lane ^ 32));
  bool split = false;
  float rho_split = 1.0f;
  if (a.kv128) {
    const float mx = fmaxf(m0, m1);
    if (t == 0) {
      C = T0 - mx;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[j][r] = S[j][r] + C;
    } else {
      float rho = 1.0f;
      if (mx > Tg) {
        const float delta = mx - T0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[j][r] = S[j][r] - delta;
        C -= delta;
        cnt += 1;
        rho = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
      }
      if (__ballot(mx > Tg) != 0) rescale<D>(O, L, rho, lane);
    }
  } else {
    bool recompute = false;
    float rho0 = 1.0f;
    if (t == 0) {
      C = T0 - m0;  // half 0 is the reference tile (scores computed with C = 0)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (half_of<PELEM>(j, g) == 0) S[j][r] = S[j][r] + C;
      recompute = true;
    } else if (m0 > Tg) {
      const float delta = m0 - T0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (half_of<PELEM>(j, g) == 0) S[j][r] = S[j][r] - delta;
      C -= delta;
      cnt += 1;
      rho0 = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
    }
    if (t != 0 && __ballot(m0 > Tg) != 0) {
      recompute = true;
      rescale<D>(O, L, rho0, lane);
    }
    if (recompute) {
      // half 1 is the next gate tile: re-score it with the updated C, one
      // MFMA at a time, keeping the half-0 values of every lane
      constexpr int RB = D * Fmt<QK>::bits / 8;
      const int m = lane & 15;
      const v4f ci = {C, C, C, C};
      m1 = -INFINITY;
#pragma unroll
      for (int j = (Layout<PELEM>::split ? 4 : 0); j < 8; ++j) {
        const int key = key_of<PELEM>(j, m & 3, m >> 2);
        const v8i ka = load_row_operand<QK, D>(ldsK + key * RB, g);
        const int sa = (D == 128 || g < 2) ? (int)ldsKs[key * 4 + g] : 127;
        const v4f s2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qB, ci, QK, QK, 0, sa, 0, qS);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (half_of<PELEM>(j, g) == 1) {
            const float v = (key_of<PELEM>(j, r, g) < nk) ? s2[r] : -INFINITY;
            S[j][r] = v;
            m1 = fmaxf(m1, v);
          }
      }
      m1 = fmaxf(m1, wshfl(m1, lane ^ 16));
      m1 = fmaxf(m1, wshfl(m1, lane ^ 32));
    }
    if (m1 > Tg) {
      const float delta = m1 - T0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (half_of<PELEM>(j, g) == 1) S[j][r] = S[j][r] - delta;
      C -= delta;
      cnt += 1;
      rho_split = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
    }
    split = __ballot(m1 > Tg) != 0;
  }
  // stage-1 flush (patterns with exponent field 0) and clamp, made explicit
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = S[j][r];
      S[j][r] = (v >= 128.0f) ? fminf(v, 32639.5f) : -INFINITY;
    }
  v8i pA;
  int pS;
  uint32_t dsc[2];
  make_p<PELEM>(S, g, lane, a.fitmax != 0, pA, pS, dsc);
  if constexpr (DUMP) dump_p<PELEM>(a, bh, qbase + n, k0, g, pA, dsc);
  if (!split) {
    pv_one<PELEM, VELEM, D>(O, L, pA, pS, ldsV, ldsVs, lane);
  } else {
    pv_one<PELEM, VELEM, D>(O, L, mask_half<PELEM>(pA, g, 0), pS, ldsV, ldsVs, lane);
    rescale<D>(O, L, rho_split, lane);
    pv_one<PELEM, VELEM, D>(O, L, mask_half<PELEM>(pA, g, 1), pS, ldsV, ldsVs, lane);
  }
}

template <int QK, int VELEM, int PELEM, int D, int NQ, bool DUMP>
__global__ void __launch_bounds__(NW * 64, 1) fsattn_fwd_kernel(FwdArgs a) {
  constexpr int QRB = D * Fmt<QK>::bits / 8;      // Q/K row bytes
  constexpr int VBB = Fmt<VELEM>::bits * 4;       // V block bytes
  constexpr int VRB = VRowLds<VELEM>::bytes;      // V LDS row bytes (one d row, 128 keys)
  constexpr int SZ_K = KT * QRB, SZ_KS = KT * 4, SZ_V = D * VRB, SZ_VS = D * 4;
  constexpr int STAGE = SZ_K + SZ_KS + SZ_V + SZ_VS;
  constexpr int QWG = NW * NQ * 16;  // queries per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.y + blockIdx.z * a.H;
  const int Sq = a.Sq, Skv = a.Skv, nb32 = a.nb32;
  const int qw0 = blockIdx.x * QWG + w * NQ * 16;  // first query of this wave

  const uint8_t* kbase = a.kc + (size_t)bh * Skv * QRB;
  const uint8_t* ksbase = a.ks + (size_t)bh * Skv * (D / 32);
  const uint8_t* vbase = a.vc + (size_t)bh * D * nb32 * VBB;
  const uint8_t* vsbase = a.vs + (size_t)bh * D * nb32;

  // ---- per q-block state
  v8i qB[NQ];
  int qS[NQ];
  float C[NQ];
  int cnt[NQ];
  v4f O[NQ][D / 16];
  v4f L[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int qrow = min(qw0 + 16 * q + n, Sq - 1);
    const uint8_t* qp = a.qc + ((size_t)bh * Sq + qrow) * QRB;
    qB[q] = load_row_operand<QK, D>(qp, g);
    qS[q] = (D == 128 || g < 2) ? (int)a.qs[((size_t)bh * Sq + qrow) * (D / 32) + g] : 127;
    C[q] = 0.0f;
    cnt[q] = 0;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) O[q][i] = v4f{0.f, 0.f, 0.f, 0.f};
    L[q] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const float T0 = a.T0, Tg = a.Tg;
  const float TgEff = fminf(Tg, 32639.0f);  // above this the stage-1 clamp could act: take the exact path
  const bool fitmax = a.fitmax != 0;
  const int ntiles = (Skv + KT - 1) / KT;

  // ---- tile loaders: codes by direct global->LDS DMA, scales through registers
  [[maybe_unused]] auto issue_codes = [&](int t, int s) {
    uint8_t* base = smem + s * STAGE;
    const int k0 = t * KT;
    {
      const int64_t lim = (int64_t)Skv * QRB - 16;
#pragma unroll
      for (int i = w; i < SZ_K / 1024; i += NW) {
        int64_t off = (int64_t)k0 * QRB + i * 1024 + lane * 16;
        off = off < lim ? off : lim;
        __builtin_amdgcn_global_load_lds((const void*)(kbase + off), (void*)(base + i * 1024), 16, 0, 0);
      }
    }
    {
      // every lane moves one chunk to LDS offset 16*(64*i + lane) of the V
      // region: 16 bytes of a 16/32-byte block, or one 12-byte half of a
      // 24-byte FP6 block (padded slot)
      constexpr int CPB = VRowLds<VELEM>::block / 16;  // LDS chunks per block
#pragma unroll
      for (int i = w; i < SZ_V / 1024; i += NW) {
        const int ci = i * 64 + lane;
        const int d = ci / (4 * CPB), rem = ci - d * 4 * CPB;
        const int blk = min(4 * t + rem / CPB, nb32 - 1);
        const int part = rem % CPB;
        const uint8_t* gp = vbase + ((size_t)d * nb32 + blk) * VBB + part * (VBB == 24 ? 12 : 16);
        if constexpr (VBB == 24) __builtin_amdgcn_global_load_lds((const void*)gp, (void*)(base + SZ_K + SZ_KS + i * 1024), 12, 0, 0);
        else __builtin_amdgcn_global_load_lds((const void*)gp, (void*)(base + SZ_K + SZ_KS + i * 1024), 16, 0, 0);
      }
    }
  };
  // register-staged copy of the K/V codes of tile t (used when direct loads are off)
  constexpr int NK4 = SZ_K / (NW * 64 * 16), NVW = D * VBB / (NW * 64);  // V words per thread (D*4 blocks)
  uint4 kst[NK4 > 0 ? NK4 : 1];
  uint32_t vst[NVW > 0 ? NVW : 1];
  [[maybe_unused]] auto load_codes_regs = [&](int t) {
    const int k0 = t * KT;
    const int64_t lim = (int64_t)Skv * QRB - 16;
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
      int64_t off = (int64_t)k0 * QRB + (int64_t)(i * NW * 64 + tid) * 16;
      off = off < lim ? off : lim;
      kst[i] = *reinterpret_cast<const uint4*>(kbase + off);
    }
#pragma unroll
    for (int i = 0; i < NVW; ++i) {
      const int wi = i * NW * 64 + tid;  // word index over [d][4 blocks][VBB/4 words]
      const int d = wi / (VBB), rem = wi - d * VBB;
      const int blk = min(4 * t + rem / (VBB / 4), nb32 - 1);
      const int wd = rem % (VBB / 4);
      vst[i] = *reinterpret_cast<const uint32_t*>(vbase + ((size_t)d * nb32 + blk) * VBB + 4 * wd);
    }
  };
  [[maybe_unused]] auto store_codes_regs = [&](int s) {
    uint8_t* base = smem + s * STAGE;
#pragma unroll
    for (int i = 0; i < NK4; ++i) *reinterpret_cast<uint4*>(base + (i * NW * 64 + tid) * 16) = kst[i];
#pragma unroll
    for (int i = 0; i < NVW; ++i) {
      const int wi = i * NW * 64 + tid;
      const int d = wi / (VBB), rem = wi - d * VBB;
      const int blk = rem / (VBB / 4), byte = 4 * (rem % (VBB / 4));
      const int slot = (VBB == 24 && byte >= 12) ? byte + 4 : byte;
      *reinterpret_cast<uint32_t*>(base + SZ_K + SZ_KS + d * VRB + blk * VRowLds<VELEM>::block + slot) = vst[i];
    }
  };
  auto load_scales = [&](int t) -> uint32_t {
    uint32_t r = 0;
    if (tid < KT) {
      const int key = min(t * KT + tid, Skv - 1);
#pragma unroll
      for (int e = 0; e < D / 32; ++e) r |= (uint32_t)ksbase[(size_t)key * (D / 32) + e] << (8 * e);
    } else if (tid < KT + D) {
      const int d = tid - KT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int blk = min(4 * t + e, nb32 - 1);
        r |= (uint32_t)vsbase[(size_t)d * nb32 + blk] << (8 * e);
      }
    }
    return r;
  };
  auto store_scales = [&](uint32_t r, int s) {
    uint8_t* base = smem + s * STAGE;
    if (tid < KT) *reinterpret_cast<uint32_t*>(base + SZ_K + 4 * tid) = r;
    else if (tid < KT + D) *reinterpret_cast<uint32_t*>(base + SZ_K + SZ_KS + SZ_V + 4 * (tid - KT)) = r;
  };

#if FSATTN_LDS_DIRECT
  issue_codes(0, 0);
#else
  load_codes_regs(0);
  store_codes_regs(0);
#endif
  store_scales(load_scales(0), 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < ntiles;
    uint32_t sreg = 0;
    if (more) {
#if FSATTN_LDS_DIRECT
      issue_codes(t + 1, cur ^ 1);
#else
      load_codes_regs(t + 1);
#endif
      sreg = load_scales(t + 1);
    }
    const uint8_t* ldsK = smem + cur * STAGE;
    const uint8_t* ldsKs = ldsK + SZ_K;
    const uint8_t* ldsV = ldsKs + SZ_KS;
    const uint8_t* ldsVs = ldsV + SZ_V;
    const int k0 = t * KT;
    const int nk = min(KT, Skv - k0);

    // ---- folded scores S^T = C + K Q^T for every q-block (K operand shared)
    v4f S[NQ][8];
    {
      constexpr int RB = QRB;
      const int m = lane & 15;
      v4f cinit[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) cinit[q] = v4f{C[q], C[q], C[q], C[q]};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = key_of<PELEM>(j, m & 3, m >> 2);
        const v8i ka = load_row_operand<QK, D>(ldsK + key * RB, g);
        const int sa = (D == 128 || g < 2) ? (int)ldsKs[key * 4 + g] : 127;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          S[q][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qB[q], cinit[q], QK, QK, 0, sa, 0, qS[q]);
      }
    }
    if (nk < KT) {  // keys beyond Skv: -inf (stage 1 -> 0, excluded from maxima)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key_of<PELEM>(j, r, g) >= nk) S[q][j][r] = -INFINITY;
    }

    // ---- fast-path check on the block maxima
    bool rare = (t == 0);
    if (!rare) {
      bool flag = false;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float tm = -INFINITY, lo = INFINITY;
        if constexpr (!Layout<PELEM>::split) {
#pragma unroll
          for (int j = 0; j < 8; ++j) tm = fmaxf(fmaxf(tm, fmaxf(S[q][j][0], S[q][j][1])), fmaxf(S[q][j][2], S[q][j][3]));
          lo = tm;
        } else {
          float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            m0 = fmaxf(fmaxf(m0, fmaxf(S[q][j][0], S[q][j][1])), fmaxf(S[q][j][2], S[q][j][3]));
            m1 = fmaxf(fmaxf(m1, fmaxf(S[q][4 + j][0], S[q][4 + j][1])), fmaxf(S[q][4 + j][2], S[q][4 + j][3]));
          }
          m0 = fmaxf(m0, wshfl(m0, lane ^ 16));
          m1 = fmaxf(m1, wshfl(m1, lane ^ 16));
          tm = fmaxf(m0, m1);
          lo = fminf(m0, m1);
        }
        flag |= (tm > TgEff) || (lo < PFlush<PELEM>::t);
      }
      rare = __ballot(flag) != 0;
    }

    if (rare) {
      // exact per-row gate semantics, BF16 flush and clamp; one q-block at a time
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        rare_block<QK, VELEM, PELEM, D, DUMP>(S[q], C[q], cnt[q], O[q], L[q], qB[q], qS[q], t, nk, k0, T0, Tg, a,
                                              ldsK, ldsKs, ldsV, ldsVs, bh, qw0 + 16 * q, lane);
    } else {
      // ---- stage 1 + 2 -> P operands, then O += P V ; l += P 1 (same P)
      v8i pA[NQ];
      int pS[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        uint32_t dsc[2];
        make_p<PELEM>(S[q], g, lane, fitmax, pA[q], pS[q], dsc);
        if constexpr (DUMP) dump_p<PELEM>(a, bh, qw0 + 16 * q + n, k0, g, pA[q], dsc);
      }
      pv_all<PELEM, VELEM, D, NQ>(O, L, pA, pS, ldsV, ldsVs, lane);
    }

    if (more) {
      store_scales(sreg, cur ^ 1);
#if !FSATTN_LDS_DIRECT
      store_codes_regs(cur ^ 1);
#endif
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16; counts
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qq = qw0 + 16 * q + 4 * g + r;
      if (qq < Sq) {
        const float inv = 1.0f / L[q][r];
        uint16_t* orow = a.out + ((size_t)bh * Sq + qq) * D;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          uint32_t u = __float_as_uint(O[q][i][r] * inv);
          u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // RNE to bf16 (finite values)
          orow[16 * i + n] = (uint16_t)u;
        }
      }
    }
    if (a.counts != nullptr && g == 0 && qw0 + 16 * q + n < Sq) a.counts[(size_t)bh * Sq + qw0 + 16 * q + n] = cnt[q];
  }
}

template <int QK, int VE, int PE, int D>
static hipError_t launch_t(const FwdArgs& a, int B, hipStream_t stream) {
  constexpr int NQ = FSATTN_NQ;
  dim3 grid((unsigned)((a.Sq + NW * NQ * 16 - 1) / (NW * NQ * 16)), (unsigned)a.H, (unsigned)B);
  if (a.pd_codes != nullptr)
    hipLaunchKernelGGL((fsattn_fwd_kernel<QK, VE, PE, D, NQ, true>), grid, dim3(NW * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((fsattn_fwd_kernel<QK, VE, PE, D, NQ, false>), grid, dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <int QK, int VE, int PE>
static hipError_t launch_d(const FwdArgs& a, int B, int D, hipStream_t s) {
  return D == 128 ? launch_t<QK, VE, PE, 128>(a, B, s) : launch_t<QK, VE, PE, 64>(a, B, s);
}

// supported combinations: FP8 P with FP8 V; FP6 (E2M3) P with FP6 or FP4 V
bool fwd_supported(int qk, int ve, int pe) {
  if (pe == E4M3) return ve == E4M3 && (qk == E4M3 || qk == E2M3 || qk == E2M1);
  if (pe == E2M3) return (ve == E2M3 || ve == E2M1) && (qk == E4M3 || qk == E2M3 || qk == E2M1);
  return false;
}

hipError_t launch_fsattn_fwd(const FwdArgs& a, int B, int D, int qk, int ve, int pe, hipStream_t s) {
#define FS_CASE(Q_, V_, P_) \
  if (qk == Q_ && ve == V_ && pe == P_) return launch_d<Q_, V_, P_>(a, B, D, s);
  FS_CASE(E4M3, E4M3, E4M3)
  FS_CASE(E2M3, E4M3, E4M3)
  FS_CASE(E2M1, E4M3, E4M3)
  FS_CASE(E2M3, E2M3, E2M3)
  FS_CASE(E2M1, E2M3, E2M3)
  FS_CASE(E4M3, E2M3, E2M3)
  FS_CASE(E2M1, E2M1, E2M3)
  FS_CASE(E2M3, E2M1, E2M3)
  FS_CASE(E4M3, E2M1, E2M3)
#undef FS_CASE
  return hipErrorInvalidValue;
}

}  // namespace fsattn
