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
//     contraction, so the fold C + sum Q K is a single instruction; with the
//     reference on the integer grid and FP6/FP4 operands the sum is exact.
//   * S^T = K Q^T: the accumulator's rows are keys, its columns queries, so
//     each lane holds 32 scores of ONE query.  The K rows fed to each of the 8
//     MFMAs of a 128-key tile are permuted so that a lane's 32 scores are
//     exactly the keys its P operand of the PV MFMA must hold -- the softmax
//     stage needs no transpose and no cross-lane traffic (FP6/FP4 P).
//   * gate: per-lane max of the scores, one wave ballot; the rollback path is
//     taken only when a lane of the wave exceeds the threshold.
//   * K/V tiles of 128 keys are staged in LDS and shared by 4 waves.
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

constexpr int NW = 4;     // waves per workgroup
constexpr int QW = 16;    // queries per wave
constexpr int KT = 128;   // keys per tile

template <int ELEM> __device__ __forceinline__ constexpr int block_bytes() { return Fmt<ELEM>::bits * 4; }

// load a row operand (32 K-elements of a lane) from a byte row laid out as
// consecutive 32-element blocks.  `row` points at the row start; g = lane/16.
template <int ELEM, int D>
__device__ __forceinline__ v8i load_row_operand(const uint8_t* row, int g) {
  v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (Layout<ELEM>::split) {
    // bytes 0-15: elements [16g,16g+16); bytes 16-31: [64+16g, 64+16g+16)
    const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * g);
    a[0] = lo.x; a[1] = lo.y; a[2] = lo.z; a[3] = lo.w;
    if (D == 128) {
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

__device__ __forceinline__ float wave_shfl(float v, int src) { return __shfl(v, src, 64); }
__device__ __forceinline__ int wave_shfl(int v, int src) { return __shfl(v, src, 64); }

// key index (0..127 within the tile) of accumulator j, row r' for lane group g
template <int PELEM>
__device__ __forceinline__ int key_of(int j, int rr, int g) {
  if constexpr (Layout<PELEM>::split) return (j < 4) ? (16 * g + 4 * j + rr) : (64 + 16 * g + 4 * (j - 4) + rr);
  else return 32 * g + 4 * j + rr;
}
// gate half (64-key semantic tile) of accumulator j for lane group g
template <int PELEM>
__device__ __forceinline__ int half_of(int j, int g) {
  if constexpr (Layout<PELEM>::split) return j >> 2;
  else return g >> 1;
}

template <int QK, int PELEM, int D>
__device__ __forceinline__ void scores(v4f (&acc)[8], const uint8_t* ldsK, const uint8_t* ldsKs, const v8i& qB,
                                       int qS, const float (&cinit)[8], int lane) {
  constexpr int RB = D * Fmt<QK>::bits / 8;  // K row bytes
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // A row m of MFMA j is key key_of(j, m%4, m/4) so that output lane (n, g)
    // receives keys key_of(j, r', g)
    const int key = key_of<PELEM>(j, m & 3, m >> 2);
    v8i a = load_row_operand<QK, D>(ldsK + key * RB, g);
    int sa = (D == 128 || g < 2) ? (int)ldsKs[key * (D / 32) + g] : 127;
    v4f c = {cinit[j], cinit[j], cinit[j], cinit[j]};
    acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qB, c, QK, QK, 0, sa, 0, qS);
  }
}

// Stage 1 for one folded score: BF16 bit pattern of the Schraudolph
// exponential (floor, flush below the smallest normal, clamp to the largest
// finite value).  v_cvt_u32_f32 truncates toward zero, which is floor here.
__device__ __forceinline__ uint32_t stage1(float t) {
  if (!(t >= 128.0f)) return 0u;
  return min(__float2uint_rz(t), 0x7F7Fu);
}

// E8M0 of a P block from its largest BF16 pattern (integer exponent math)
template <int PELEM>
__device__ __forceinline__ uint32_t p_scale(uint32_t bmax, bool fitmax) {
  constexpr int thr7 = (int)(Fmt<PELEM>::mthr23 >> 16);  // 7-bit mantissa threshold
  int e = fitmax ? (int)((bmax + (uint32_t)(127 - thr7)) >> 7) : (int)(bmax >> 7);
  if (bmax == 0) return 0u;
  return (uint32_t)min(max(e - Fmt<PELEM>::emax, 0), 254);
}

// Build the P operand (A of PV) from this lane's 32 folded scores.
// half_mask: bit h set -> keys of gate half h are zeroed (split PV).
template <int PELEM>
__device__ __forceinline__ void make_p(const v4f (&acc)[8], int g, int lane, bool fitmax, v8i& pA, int& pS,
                                       uint32_t (&dump_scale)[2]) {
  uint32_t b[32];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[4 * j + r] = stage1(acc[j][r]);
  if constexpr (!Layout<PELEM>::split) {
    uint32_t bmax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) bmax = max(bmax, b[i]);
    uint32_t sc = p_scale<PELEM>(bmax, fitmax);
    float X = e8m0_to_float(sc);
    v32bf x;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __builtin_bit_cast(__bf16, (uint16_t)b[i]);
    v6i r;
    if constexpr (PELEM == E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(x, X);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(x, X);
    pA = v8i{r[0], r[1], r[2], r[3], r[4], r[5], 0, 0};
    pS = (int)sc;
    dump_scale[0] = sc;
    dump_scale[1] = sc;
  } else {
    // two 16-key halves per lane; a 32-key P block spans lanes g and g^1
    uint32_t m0 = 0, m1 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) { m0 = max(m0, b[i]); m1 = max(m1, b[16 + i]); }
    m0 = max(m0, (uint32_t)wave_shfl((int)m0, lane ^ 16));
    m1 = max(m1, (uint32_t)wave_shfl((int)m1, lane ^ 16));
    uint32_t s0 = p_scale<PELEM>(m0, fitmax), s1 = p_scale<PELEM>(m1, fitmax);
    float X0 = e8m0_to_float(s0), X1 = e8m0_to_float(s1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float Xi = (i < 4) ? X0 : X1;
      v2s r = {0, 0};
      v2bf p0 = {__builtin_bit_cast(__bf16, (uint16_t)b[4 * i + 0]), __builtin_bit_cast(__bf16, (uint16_t)b[4 * i + 1])};
      v2bf p1 = {__builtin_bit_cast(__bf16, (uint16_t)b[4 * i + 2]), __builtin_bit_cast(__bf16, (uint16_t)b[4 * i + 3])};
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, p0, Xi, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, p1, Xi, true);
      pA[i] = (int)((uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16));
    }
    // MFMA scale of 32-block b is read from lane 16b + n:
    // b0 = my first half (g=0), b1 = first half of g=2,3, b2 = second half of g=0,1, b3 = my second half (g=3)
    const int n = lane & 15;
    int from_g2 = wave_shfl((int)s0, n + 32);
    int from_g1 = wave_shfl((int)s1, n + 16);
    pS = (g == 0) ? (int)s0 : (g == 1) ? from_g2 : (g == 2) ? from_g1 : (int)s1;
    dump_scale[0] = s0;
    dump_scale[1] = s1;
  }
}

template <int PELEM>
__device__ __forceinline__ v8i mask_half(const v8i& pA, int g, int keep_half) {
  v8i r = pA;
  if constexpr (Layout<PELEM>::split) {
    // bytes 0-15 = half 0, bytes 16-31 = half 1
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

template <int PELEM, int VELEM, int D>
__device__ __forceinline__ void pv(v4f (&O)[D / 16], v4f& L, const v8i& pA, int pS, const uint8_t* ldsV,
                                   const uint8_t* ldsVs, int lane) {
  constexpr int RB = KT * Fmt<VELEM>::bits / 8;  // V row bytes in LDS (one d row, 128 keys)
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int d = 16 * i + n;
    v8i b = load_row_operand<VELEM, 128>(ldsV + d * RB, g);
    int sb = (int)ldsVs[d * 4 + g];
    O[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pA, b, O[i], PELEM, VELEM, 0, pS, 0, sb);
  }
  // l += P 1: ones operand (E2M1 code 0x2 = 1.0, scale 2^0)
  const v8i ones = {0x22222222, 0x22222222, 0x22222222, 0x22222222, 0, 0, 0, 0};
  L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pA, ones, L, PELEM, E2M1, 0, pS, 0, 127);
}

// rescale O rows (queries 4g + r) by rho of their query (rho lives in lane q)
template <int D>
__device__ __forceinline__ void rescale(v4f (&O)[D / 16], v4f& L, float rho, int lane) {
  const int g = lane >> 4;
  float rr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rr[r] = wave_shfl(rho, 4 * g + r);
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) O[i][r] *= rr[r];
#pragma unroll
  for (int r = 0; r < 4; ++r) L[r] *= rr[r];
}

template <int QK, int VELEM, int PELEM, int D>
__global__ void __launch_bounds__(NW * 64) fsattn_fwd_kernel(FwdArgs a) {
  constexpr int QRB = D * Fmt<QK>::bits / 8;     // Q/K row bytes
  constexpr int VRB = KT * Fmt<VELEM>::bits / 8; // V LDS row bytes
  constexpr int VBB = Fmt<VELEM>::bits * 4;      // V block bytes
  __shared__ __attribute__((aligned(16))) uint8_t ldsK[KT * QRB];
  __shared__ __attribute__((aligned(16))) uint8_t ldsKs[KT * (D / 32)];
  __shared__ __attribute__((aligned(16))) uint8_t ldsV[D * VRB];
  __shared__ __attribute__((aligned(16))) uint8_t ldsVs[D * 4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.y + blockIdx.z * a.H;
  const int q0 = blockIdx.x * (NW * QW) + w * QW;
  const int Sq = a.Sq, Skv = a.Skv;

  // Q operand: lane (n, g) holds query q0+n, D-part g (clamped for ragged tails)
  const int qrow = min(q0 + n, Sq - 1);
  const uint8_t* qrowp = a.qc + ((size_t)bh * Sq + qrow) * QRB;
  const v8i qB = load_row_operand<QK, D>(qrowp, g);
  const int qS = (D == 128 || g < 2) ? (int)a.qs[((size_t)bh * Sq + qrow) * (D / 32) + g] : 127;

  v4f O[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) O[i] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f L = {0.f, 0.f, 0.f, 0.f};
  float C = 0.0f;  // folded accumulator offset of query n (integer-valued)
  int cnt = 0;
  const float T0 = a.T0, Tg = a.Tg;
  const bool fitmax = a.fitmax != 0;

  const int ntiles = (Skv + KT - 1) / KT;
  const uint8_t* kbase = a.kc + (size_t)bh * Skv * QRB;
  const uint8_t* ksbase = a.ks + (size_t)bh * Skv * (D / 32);
  const uint8_t* vbase = a.vc + (size_t)bh * D * a.nb32 * VBB;
  const uint8_t* vsbase = a.vs + (size_t)bh * D * a.nb32;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * KT;
    const int nk = min(KT, Skv - k0);  // valid keys in this tile
    __syncthreads();
    // ---- stage K tile: rows k0..k0+nk-1 (contiguous), zero beyond
    {
      const uint4* src = reinterpret_cast<const uint4*>(kbase + (size_t)k0 * QRB);
      uint4* dst = reinterpret_cast<uint4*>(ldsK);
      const int nvec = KT * QRB / 16, nvalid = nk * QRB / 16;
      for (int i = tid; i < nvec; i += NW * 64) dst[i] = (i < nvalid) ? src[i] : make_uint4(0, 0, 0, 0);
      for (int i = tid; i < KT * (D / 32); i += NW * 64)
        ldsKs[i] = (i < nk * (D / 32)) ? ksbase[(size_t)k0 * (D / 32) + i] : (uint8_t)127;
    }
    // ---- stage V tile: for each d row, key blocks 4t..4t+3 (zero beyond nb32)
    {
      const int blk0 = 4 * t;
      const int nblk = min(4, a.nb32 - blk0);
      constexpr int W8 = VBB / 8;  // 8-byte words per block
      for (int i = tid; i < D * 4 * W8; i += NW * 64) {
        const int d = i / (4 * W8), rem = i - d * 4 * W8, blk = rem / W8, wd = rem - blk * W8;
        uint2 v = make_uint2(0, 0);
        if (blk < nblk)
          v = *reinterpret_cast<const uint2*>(vbase + ((size_t)d * a.nb32 + blk0 + blk) * VBB + 8 * wd);
        *reinterpret_cast<uint2*>(ldsV + d * VRB + blk * VBB + 8 * wd) = v;
      }
      for (int i = tid; i < D * 4; i += NW * 64) {
        const int d = i >> 2, blk = i & 3;
        ldsVs[i] = (blk < nblk) ? vsbase[(size_t)d * a.nb32 + blk0 + blk] : (uint8_t)127;
      }
    }
    __syncthreads();

    // ---- folded scores S^T = C + K Q^T
    v4f acc[8];
    {
      float ci[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ci[j] = C;
      scores<QK, PELEM, D>(acc, ldsK, ldsKs, qB, qS, ci, lane);
    }
    // mask keys beyond Skv
    if (nk < KT) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key_of<PELEM>(j, r, g) >= nk) acc[j][r] = -INFINITY;
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) lmax = fmaxf(lmax, acc[j][r]);

    bool split_pv = false;
    float rho_split = 1.0f;
    const bool slow = (t == 0) || (__ballot(lmax > Tg) != 0);
    if (slow) {
      // exact per-row gate semantics; gate tiles are 64 keys (halves) or 128 keys
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (half_of<PELEM>(j, g) == 0) m0 = fmaxf(m0, acc[j][r]);
          else m1 = fmaxf(m1, acc[j][r]);
        }
      m0 = fmaxf(m0, wave_shfl(m0, lane ^ 16)); m0 = fmaxf(m0, wave_shfl(m0, lane ^ 32));
      m1 = fmaxf(m1, wave_shfl(m1, lane ^ 16)); m1 = fmaxf(m1, wave_shfl(m1, lane ^ 32));
      if (a.kv128) {
        const float mx = fmaxf(m0, m1);
        if (t == 0) {
          C = floorf(T0 - mx);
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] = acc[j][r] + C;
        } else {
          float rho = 1.0f;
          if (mx > Tg) {
            const float delta = ceilf(mx - T0);
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[j][r] = acc[j][r] - delta;
            C -= delta;
            cnt += 1;
            rho = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
          }
          if (__ballot(mx > Tg) != 0) rescale<D>(O, L, rho, lane);  // wave-uniform: shuffles inside
        }
      } else {
        bool recompute = false;
        float rho0 = 1.0f;
        if (t == 0) {
          // half 0 is the reference tile (scores computed with C = 0)
          C = floorf(T0 - m0);
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (half_of<PELEM>(j, g) == 0) acc[j][r] = acc[j][r] + C;
          recompute = true;
        } else if (m0 > Tg) {
          const float delta = ceilf(m0 - T0);
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (half_of<PELEM>(j, g) == 0) acc[j][r] = acc[j][r] - delta;
          C -= delta;
          cnt += 1;
          rho0 = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
        }
        if (t != 0 && __ballot(m0 > Tg) != 0) {
          recompute = true;
          rescale<D>(O, L, rho0, lane);
        }
        if (recompute) {
          // half 1 is the next gate tile: its scores use the updated C
          v4f acc2[8];
          float ci[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) ci[j] = C;
          scores<QK, PELEM, D>(acc2, ldsK, ldsKs, qB, qS, ci, lane);
          m1 = -INFINITY;
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (half_of<PELEM>(j, g) == 1) {
                float v = (key_of<PELEM>(j, r, g) < nk) ? acc2[j][r] : -INFINITY;
                acc[j][r] = v;
                m1 = fmaxf(m1, v);
              }
          m1 = fmaxf(m1, wave_shfl(m1, lane ^ 16));
          m1 = fmaxf(m1, wave_shfl(m1, lane ^ 32));
        }
        if (m1 > Tg) {
          const float delta = ceilf(m1 - T0);
#pragma unroll
          for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (half_of<PELEM>(j, g) == 1) acc[j][r] = acc[j][r] - delta;
          C -= delta;
          cnt += 1;
          rho_split = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
        }
        split_pv = __ballot(m1 > Tg) != 0;
      }
    }

    // ---- stage 1 + stage 2 -> P operand
    v8i pA;
    int pS;
    uint32_t dsc[2];
    make_p<PELEM>(acc, g, lane, fitmax, pA, pS, dsc);

    // optional P dump (debug): codes one byte per key, E8M0 per 32 keys
    if (a.pd_codes != nullptr && bh == a.pd_bh) {
      const int q = q0 + n;
      if (q >= a.pd_row0 && q < a.pd_row1 && q < Sq) {
        const size_t S32 = (size_t)a.nb32 * 32;
        uint8_t* drow = a.pd_codes + (size_t)(q - a.pd_row0) * S32;
        uint8_t* srow = a.pd_scales + (size_t)(q - a.pd_row0) * a.nb32;
        constexpr int bits = Fmt<PELEM>::bits;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int key = k0 + key_of<PELEM>(e >> 2, e & 3, g);
          int pos = e * bits;
          uint32_t wv = (uint32_t)pA[pos >> 5] >> (pos & 31);
          if ((pos & 31) + bits > 32) wv |= (uint32_t)pA[(pos >> 5) + 1] << (32 - (pos & 31));
          if (key < (int)S32) drow[key] = (uint8_t)(wv & ((1u << bits) - 1));
        }
        if constexpr (Layout<PELEM>::split) {
          // this lane computed the scales of the blocks holding keys 16g.. and 64+16g..
          const int kb0 = (k0 + 16 * g) / 32, kb1 = (k0 + 64 + 16 * g) / 32;
          if (kb0 < a.nb32) srow[kb0] = (uint8_t)dsc[0];
          if (kb1 < a.nb32) srow[kb1] = (uint8_t)dsc[1];
        } else {
          const int kb = (k0 + 32 * g) / 32;
          if (kb < a.nb32) srow[kb] = (uint8_t)dsc[0];
        }
      }
    }

    // ---- O += P V ; l += P 1
    if (!split_pv) {
      pv<PELEM, VELEM, D>(O, L, pA, pS, ldsV, ldsVs, lane);
    } else {
      pv<PELEM, VELEM, D>(O, L, mask_half<PELEM>(pA, g, 0), pS, ldsV, ldsVs, lane);
      rescale<D>(O, L, rho_split, lane);
      pv<PELEM, VELEM, D>(O, L, mask_half<PELEM>(pA, g, 1), pS, ldsV, ldsVs, lane);
    }
  }

  // ---- epilogue: O / l -> bf16; counts
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int q = q0 + 4 * g + r;
    if (q < Sq) {
      const float inv = 1.0f / L[r];
      uint16_t* orow = a.out + ((size_t)bh * Sq + q) * D;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        float v = O[i][r] * inv;
        uint32_t u = __float_as_uint(v);
        u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // RNE to bf16 (finite values)
        orow[16 * i + n] = (uint16_t)u;
      }
    }
  }
  if (a.counts != nullptr && g == 0 && q0 + n < Sq) a.counts[(size_t)bh * Sq + q0 + n] = cnt;
}

template <int QK, int VE, int PE, int D>
static hipError_t launch_t(const FwdArgs& a, int B, hipStream_t stream) {
  dim3 grid((unsigned)((a.Sq + NW * QW - 1) / (NW * QW)), (unsigned)a.H, (unsigned)B);
  hipLaunchKernelGGL((fsattn_fwd_kernel<QK, VE, PE, D>), grid, dim3(NW * 64), 0, stream, a);
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
