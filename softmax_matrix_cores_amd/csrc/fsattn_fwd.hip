// fsattn_fwd.hip -- Fused-Softmax quantized attention forward for gfx950.
//
// The method ("Fused-Softmax shifts an AI attention bottleneck onto faster
// GPU hardware", paragraphs 5-6; "Fused softmax makes quantized attention
// faster on AMD GPUs", section "Move work, keep correction"):
//   * the row-max reference is provisionally frozen; its subtraction and the
//     affine part of Schraudolph's exponential are folded into the Q K^T
//     product: the slope (128 log2 e sigma) sits in Q-hat, the offset
//     C_i = T0 - m_i is the accumulator's initial value of the matrix op;
//   * stage 1: the integer part of the folded score is the BF16 bit pattern
//     of ~2^(score - m); stage 2: BF16 -> MX P with one E8M0 per 32 keys;
//   * O += P V and l += P 1 run on the matrix cores with the same P;
//   * a rollback gate fires when a tile's scores exceed the reference by more
//     than tau: the reference is raised and O, l are rescaled.
//
// Mapping to CDNA4:
//   * 8 waves per workgroup (two per SIMD), 32 queries per wave.  Keys advance
//     in steps of 64 with one workgroup barrier per step.  Every wave runs the
//     same schedule: after the barrier it reads the K operands of step u+1,
//     issues the PV products of step u-1 interleaved with the VALU conversion
//     of step u, reads the V operands of step u and issues the score products
//     of step u+1, so that every LDS read has a phase of the step to arrive
//     and the matrix core works while the VALU converts.
//   * every product is v_mfma_scale_f32_32x32x64_f8f6f4: S^T = K Q^T (2 key
//     groups x D/64 feature halves, the fold offset C_i as the accumulator's
//     initial value), O += P V (D/32 feature blocks).  l += P 1 uses one
//     16x16x128 instruction whose ones operand selects, per output column, the
//     lanes of one query (FP6 P), or a 32x32x64 ones operand (FP8 P).
//   * E4M3 Q/K (X8): gfx950's FP8 product does not return the correctly
//     rounded sum (a score can be off by up to about one binary32 step of
//     the accumulator per product), which moves P codes of scores near a
//     stage-1 floor boundary.  So the E4M3 K operands are decoded to BF16
//     (exact: four significant bits times the block scale) on their way from
//     LDS and multiplied with the Q operands decoded once at the start, on
//     v_mfma_f32_32x32x16_bf16 (four per key group and feature half), summed
//     from zero; C_i is added to each score once, in binary32.  The FP8
//     product remains available (fsattn_forward_fp8_products).
//   * the K rows of the score instructions are permuted so that a lane's 32
//     scores are exactly the 32 keys of its P operand in the PV product.
//   * K and V operands sit in an 8-slot LDS ring in operand order, so every
//     operand read is a lane-contiguous ds_read_b128 (plus a ds_read_b64 for
//     the last 8 bytes of an FP6 lane): no bank conflicts.  The ring is filled
//     six steps ahead by buffer_load ... lds DMA.  Every wave issues the same
//     number of loads per step (padding loads read past the end of the buffer
//     into a sink), so each wave waits with one constant s_waitcnt; the step
//     moves the buffer descriptors, so reads past the end of K or V return
//     zeros.
//   * scales: one dword per key holds its K block scales; V scales come in the
//     quantizer's interleaved layout, one dword per lane holding the scales of
//     its PV instructions, picked with op_sel.
//   * fast path per score: one float->int convert (stage 1; the odd score of
//     a pair converts straight into the high half of the packed word) and
//     half a max3.  The E8M0 of P comes from the block max with one fma and
//     a convert (the exact path: integer exponent arithmetic on the block's
//     largest pattern); one v_cvt_scalef32_pk32_fp6_bf16 converts a lane's
//     32 keys.  A wave ballot sends a step to the exact path on the first
//     step, a step holding a masked key (past the batch's key count, or past
//     a row's causal limit), a possible gate fire or stage-1 clamp, or a
//     block low enough that the BF16 subnormal flush could change a code.  A
//     step whose only issue is a gate fire takes a shorter path: the shift,
//     then the fast conversion again.  A fire updates the C splat in place,
//     and FP6 P lives in six registers, so that the fast path carries no
//     register copies between steps.
//   * masks (causal, per-batch query / key counts): a workgroup reads only
//     the keys its valid queries see; causal workgroups start longest first;
//     rows that see no key, and rows past the query count, are stored as 0.
//   * a 128-key gate tile spans two steps: on the even step the scores of the
//     odd step are computed once ahead of time for their maximum only, and
//     computed again (with the gate's new offset) on the odd step.
//
// Operand lane layouts of the 32x32x64 scaled MFMA (measured on gfx950):
//   FP6/FP4: lane (r = l%32, h = l/32) holds row r, K elements [32h, 32h+32)
//     and the scale of that 32-block.
//   FP8: lane (r, h) holds K elements [16h, 16h+16) in bytes 0-15 and
//     [32+16h, 32+16h+16) in bytes 16-31; the scale of block b comes from
//     lane 32b + r.
//   Accumulator: lane (c = l%32, h) register 4i+j holds row 8i+4h+j of
//     column c.
#include <type_traits>

#include "internal.h"
#include "lds_dma.h"
#include "mx_device.h"

namespace fsattn {
namespace {

constexpr int NW = 8;         // waves per workgroup
constexpr int QW = 32;        // queries per wave
constexpr int QWG = NW * QW;  // queries per workgroup
constexpr int KS = 64;        // keys per step
constexpr int NS = 8;         // LDS ring slots
constexpr int PF = NS - 2;    // steps fetched ahead

template <int F> struct Opd {
  static constexpr int bits = Fmt<F>::bits;
  static constexpr bool split = (bits == 8);
  static constexpr int tail = 4 * bits - 16;  // bytes after the first 16 of a lane: 16, 8, 0
  static constexpr int region = 64 * 4 * bits;
};

template <int QK, int VE, int D> struct Geo {
  static constexpr int DH = D / 64;  // feature halves of a score product
  static constexpr int NK = 2 * DH;  // K operands per step
  static constexpr int NV = D / 32;  // V operands per step
  static constexpr int QRB = D * Fmt<QK>::bits / 8;
  static constexpr int VBB = 4 * Fmt<VE>::bits;
  static constexpr int KSB = D / 32;
  // K scales first: their reads then carry no constant offset of their own
  static constexpr int KS_OFF = 0;
  static constexpr int K_OFF = 256;
  static constexpr int V_OFF = K_OFF + NK * Opd<QK>::region;
  static constexpr int VS_OFF = V_OFF + NV * Opd<VE>::region;
  static constexpr int SINK_OFF = VS_OFF + 256;  // 1 KiB per slot for padding loads
  static constexpr int SLOT = SINK_OFF + 1024;
  static constexpr int LDS_BYTES = NS * SLOT;
  // DMA per step: waves 0-3 fetch K, waves 4-7 V.  16-byte loads: operand
  // heads (and FP8 tails); 4-byte loads: FP6 tails (two per operand); one
  // 4-byte load of the scale dwords.  Every wave issues M16 + MT + 1 loads,
  // padded with loads that read past the end of the buffer (zeros) into the
  // slot's sink.
  static constexpr int N16K = NK * (Opd<QK>::tail == 16 ? 2 : 1);
  static constexpr int NTK = Opd<QK>::tail == 8 ? 2 * NK : 0;
  static constexpr int N16V = NV * (Opd<VE>::tail == 16 ? 2 : 1);
  static constexpr int NTV = Opd<VE>::tail == 8 ? 2 * NV : 0;
  static constexpr int M16 = ((N16K > N16V ? N16K : N16V) + 3) / 4;
  static constexpr int MT = ((NTK > NTV ? NTK : NTV) + 3) / 4;
  static constexpr int PER_WAVE = M16 + MT + 1;
};

// key (0..63 in the step) of accumulator register k (0..15) of key group kg, lane half h
template <int PE> __device__ __forceinline__ constexpr int step_key(int kg, int k, int h) {
  return Opd<PE>::split ? 32 * kg + 16 * h + k : 32 * h + 16 * kg + k;
}
// key fed to row rho (0..31) of the K operand of key group kg
template <int PE> __device__ __forceinline__ constexpr int row_key(int kg, int rho) {
  return step_key<PE>(kg, 4 * (rho >> 3) + (rho & 3), (rho >> 2) & 1);
}

// Smallest BF16 pattern of a P block max for which BF16 subnormals of the
// block convert to +0 anyway (x/X at most half the format's smallest
// subnormal): exponent field >= 7 (E2M3), 10 (E3M2), 19 (E4M3).
template <int PELEM> struct PFlush;
template <> struct PFlush<E2M3> { static constexpr float t = 896.0f; };
template <> struct PFlush<E4M3> { static constexpr float t = 2432.0f; };
template <> struct PFlush<E3M2> { static constexpr float t = 1280.0f; };

__device__ __forceinline__ float wshfl(float v, int src) { return __shfl(v, src, 64); }

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
// eight E4M3 codes (two dwords, byte order) times the block scale X, as BF16
// (exact: four significant bits times a power of two, inside BF16's range
// for every scale an operand of finite values gets)
__device__ __forceinline__ v8bf dec8(int w0, int w1, float X) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w0, X, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w0, X, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w1, X, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w1, X, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One lane's MFMA operand from an LDS region in operand order
template <int F> __device__ __forceinline__ v8i lds_operand(const uint8_t* region, int lane) {
  const uint4 x = *reinterpret_cast<const uint4*>(region + 16 * lane);
  if constexpr (Opd<F>::tail == 16) {
    const uint4 y = *reinterpret_cast<const uint4*>(region + 1024 + 16 * lane);
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  } else if constexpr (Opd<F>::tail == 8) {
    const uint2 y = *reinterpret_cast<const uint2*>(region + 1024 + 8 * lane);
    // keep the compiler from pairing this 8-byte read with another operand's
    // into one ds_read2 (the halves would then need moves into the operand)
    asm volatile("" ::: "memory");
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, 0, 0};
  } else {
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  }
}

// byte offsets (from the start of the head's K rows / V^T rows) of the two
// chunks of a lane's K operand and V operand
template <int QK, int D> __device__ __forceinline__ void k_chunks(int key, int dh, int hh, int& a, int& b) {
  constexpr int QRB = D * Fmt<QK>::bits / 8;
  if constexpr (Opd<QK>::split) {
    a = key * QRB + 64 * dh + 16 * hh;
    b = a + 32;
  } else {
    a = key * QRB + (2 * dh + hh) * (4 * Fmt<QK>::bits);
    b = a + 16;
  }
}
template <int VE> __device__ __forceinline__ void v_chunks(int d, int nb32, int hh, int& a, int& b) {
  if constexpr (Opd<VE>::split) {
    a = (d * nb32) * 32 + 16 * hh;
    b = a + 32;
  } else {
    a = (d * nb32 + hh) * (4 * Fmt<VE>::bits);
    b = a + 16;
  }
}

// One DMA load of a step: LDS offset in the slot (padding loads go to the
// slot's sink) and per-lane byte offset.
struct Dma {
  int lds;
  int voff;
};

constexpr int OOB_OFF = 0x40000000;  // past every buffer (per-head sizes are below 2^30)

// 16-byte load `it` of the K (kside) or V side for loader lane `lane`
template <int QK, int VE, int PE, int D>
__device__ Dma dma16(bool kside, int it, int lane, int nb32) {
  using G = Geo<QK, VE, D>;
  const int hh = lane >> 5, rho = lane & 31;
  int a, b;
  if (kside) {
    if (it >= G::N16K) return Dma{G::SINK_OFF, OOB_OFF};
    const int o = it % G::NK, tail = it / G::NK;
    k_chunks<QK, D>(row_key<PE>(o / G::DH, rho), o % G::DH, hh, a, b);
    return Dma{G::K_OFF + o * Opd<QK>::region + 1024 * tail, tail ? b : a};
  }
  if (it >= G::N16V) return Dma{G::SINK_OFF, OOB_OFF};
  const int o = it % G::NV, tail = it / G::NV;
  v_chunks<VE>(32 * o + rho, nb32, hh, a, b);
  return Dma{G::V_OFF + o * Opd<VE>::region + 1024 * tail, tail ? b : a};
}

// 4-byte tail load `it`: dword (lane & 1) of the 8-byte FP6 tail of consumer
// lane L = 32p + (lane >> 1) of operand it/2, p = it & 1
template <int QK, int VE, int PE, int D>
__device__ Dma dma4(bool kside, int it, int lane, int nb32) {
  using G = Geo<QK, VE, D>;
  int a, b;
  if (it >= (kside ? G::NTK : G::NTV)) return Dma{G::SINK_OFF, OOB_OFF};
  const int o = it >> 1, p = it & 1, L = 32 * p + (lane >> 1);
  if (kside) {
    k_chunks<QK, D>(row_key<PE>(o / G::DH, L & 31), o % G::DH, L >> 5, a, b);
    return Dma{G::K_OFF + o * Opd<QK>::region + 1024 + 256 * p, b + 4 * (lane & 1)};
  }
  v_chunks<VE>(32 * o + (L & 31), nb32, L >> 5, a, b);
  return Dma{G::V_OFF + o * Opd<VE>::region + 1024 + 256 * p, b + 4 * (lane & 1)};
}

// scale load of a step: wave 0 of each side, padding for the others.  K: lane
// i = 32 kg + rho loads the scale dword of its key; V: one dword per lane.
template <int QK, int VE, int PE, int D>
__device__ Dma dma_scale(bool kside, int wj, int lane, int ko) {
  using G = Geo<QK, VE, D>;
  if (wj != 0) return Dma{G::SINK_OFF, OOB_OFF};
  if (kside) {
    const int key = row_key<PE>(lane >> 5, lane & 31) + ko;
    return Dma{G::KS_OFF + 4 * lane, (D == 128) ? key * 4 : (key & ~1) * 2};
  }
  return Dma{G::VS_OFF + 4 * lane, 4 * lane};
}

// P operand registers: FP6 P uses 6 (kept as such across the loop and
// widened at each product, so that no copy carries unused registers)
template <int PE> struct POp { typedef v6i T; };
template <> struct POp<E4M3> { typedef v8i T; };
template <> struct POp<E2M1> { typedef v4i T; };
__device__ __forceinline__ v8i widen(const v4i& p) { return v8i{p[0], p[1], p[2], p[3], 0, 0, 0, 0}; }
__device__ __forceinline__ v8i widen(const v6i& p) { return v8i{p[0], p[1], p[2], p[3], p[4], p[5], 0, 0}; }
__device__ __forceinline__ const v8i& widen(const v8i& p) { return p; }

// E8M0 of a P block from its largest BF16 pattern (integer exponent math)
template <int PELEM>
__device__ __forceinline__ uint32_t p_scale(uint32_t bmax) {
  constexpr int thr7 = (int)(Fmt<PELEM>::mthr23 >> 16);  // 7-bit mantissa threshold
  const int e = (int)((bmax + (uint32_t)(127 - thr7)) >> 7);
  if (bmax == 0) return 0u;
  return (uint32_t)min(max(e - Fmt<PELEM>::emax, 0), 254);
}

// Maxima of scores use IEEE 754-2019 maximum (v_maximum3_f32 on gfx950): unlike
// fmaxf it needs no quieting of its inputs in IEEE mode, which cost two extra
// instructions per 16 scores.  On the scores (finite or -inf, never NaN) it
// differs from fmaxf at most in the sign of a zero maximum, which no decision
// here depends on (a zero maximum fails the fast-path range either way).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Stage 1 + pack: BF16 patterns of a lane's 32 scores (element e = 16 kg + k);
// v_cvt_u32_f32 truncates toward zero (= floor for t >= 0) and gives 0 below 0.
// The odd element's convert writes straight into the high half of the word
// (SDWA dst_sel WORD_1, low half preserved): two instructions per pair.  The
// patterns fit 16 bits (the callers clamp at 0x7F7F or prove the bound), so
// the half taken is the whole value.  The compiler does not form SDWA from
// this pattern, hence the inline assembly; it takes the lane maxima d0 / d1
// of S[0] / S[1] as an operand so that it issues after the instructions that
// computed them, which read the same score registers through the compiler and
// so carry whatever wait states a matrix-core result requires.
__device__ __forceinline__ void pack_b(const v16f (&S)[2], uint32_t (&w)[16], float d0, float d1) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kg = i >> 3, k = 2 * (i & 7);
    uint32_t x = __float2uint_rz(S[kg][k]);
    asm("v_cvt_u32_f32_sdwa %0, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
        : "+v"(x)
        : "v"(S[kg][k + 1]), "v"(kg ? d1 : d0));
    w[i] = x;
  }
}


__device__ __forceinline__ float max16(const v16f& s) {
  float m = vmax3(s[0], s[1], s[2]);
#pragma unroll
  for (int k = 3; k < 15; k += 2) m = vmax3(m, s[k], s[k + 1]);
  return vmax(m, s[15]);
}
__device__ __forceinline__ float max32(const v16f (&S)[2]) { return vmax(max16(S[0]), max16(S[1])); }

// P operand from packed patterns and the lane's maxima over key groups 0/1.
// FP6 P: the lane's 32 keys are one block.  FP8 P: elements 0-15 belong to
// block 0 of the step, 16-31 to block 1, each block spanning lanes q and q+32.
template <int PE, bool FAST>
__device__ __forceinline__ void p_from_w(const uint32_t (&w)[16], float m0, float m1, int lane,
                                         typename POp<PE>::T& pA, int& pS,
                                         uint32_t (&dsc)[2]) {
  if constexpr (!Opd<PE>::split) {
    const float tm = __builtin_fmaxf(m0, m1);
    uint32_t sc;
    if constexpr (FAST) {
      // the block max lies in [PFlush, TgEff]: no flush, clamp or zero code
      // ((floor(tm) + 127 - thr7) >> 7) - emax as one fma and a convert: for
      // tm in [PFlush, 32640) tm / 128, the constant and their sum are exact
      // in binary32, and floor((floor(t) + k) / 128) = floor((t + k) / 128)
      constexpr int thr7 = (int)(Fmt<PE>::mthr23 >> 16);
      constexpr float off = (float)(127 - thr7) / 128.0f - (float)Fmt<PE>::emax;
      sc = __float2uint_rz(__builtin_fmaf(tm, 1.0f / 128.0f, off));
    } else {
      const uint32_t bmax = (tm >= 128.0f) ? min(__float2uint_rz(tm), 0x7F7Fu) : 0u;
      sc = p_scale<PE>(bmax);
    }
    v16u wv;
#pragma unroll
    for (int i = 0; i < 16; ++i) wv[i] = w[i];
    const v32bf x = __builtin_bit_cast(v32bf, wv);
    v6i r;
    const float X = FAST ? __uint_as_float(sc << 23) : e8m0_to_float(sc);
    if constexpr (PE == E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(x, X);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(x, X);
    pA = r;
    pS = (int)sc;
    dsc[0] = sc;
    dsc[1] = sc;
  } else {
    const float b0m = vmax(m0, wshfl(m0, lane ^ 32));
    const float b1m = vmax(m1, wshfl(m1, lane ^ 32));
    uint32_t s0, s1;
    float X0, X1;
    if constexpr (FAST) {
      // both block maxima lie in [PFlush, TgEff]: the fma form of the fast
      // path above, no flush, clamp or zero scale
      constexpr int thr7 = (int)(Fmt<PE>::mthr23 >> 16);
      constexpr float off = (float)(127 - thr7) / 128.0f - (float)Fmt<PE>::emax;
      s0 = __float2uint_rz(__builtin_fmaf(b0m, 1.0f / 128.0f, off));
      s1 = __float2uint_rz(__builtin_fmaf(b1m, 1.0f / 128.0f, off));
      X0 = __uint_as_float(s0 << 23);
      X1 = __uint_as_float(s1 << 23);
    } else {
      const uint32_t b0 = (b0m >= 128.0f) ? min(__float2uint_rz(b0m), 0x7F7Fu) : 0u;
      const uint32_t b1 = (b1m >= 128.0f) ? min(__float2uint_rz(b1m), 0x7F7Fu) : 0u;
      s0 = p_scale<PE>(b0);
      s1 = p_scale<PE>(b1);
      X0 = e8m0_to_float(s0);
      X1 = e8m0_to_float(s1);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float Xi = (i < 4) ? X0 : X1;
      // the two converts write both halves of r, so r may start as any
      // value: the patterns word it converts first, which dies there (no
      // register has to be cleared)
      v2s r = __builtin_bit_cast(v2s, w[2 * i]);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, w[2 * i]), Xi, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf, w[2 * i + 1]), Xi, true);
      pA[i] = (int)((uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16));
    }
    pS = (lane >> 5) ? (int)s1 : (int)s0;  // block b's scale comes from lane 32b + q
    dsc[0] = s0;
    dsc[1] = s1;
  }
}

// EFQ-style P ("EFQ-Softmax: Exp-Free Quantization for Softmax", sections
// II.B-C, III.B): E2M1 codes straight from the folded scores, no exponential
// and no BF16 stage.  A lane's 32 scores are one block (element e = 16 kg + k):
//   E    = floor(fl32(max - T0) / 128), clamped to [-1000, 1000]
//   E8M0 = clamp(E + 125, 0, 254)                (E2M1's top binade is 2^2)
//   base = fl32(fl32(T0 + 128 E) + 128 tau)      (exact: integers and a dyadic)
//   code = clamp(floor(fma(t, a, b)), 0, 7)      a = 1 / (128 h), b = -base a,
//                                                both rounded up
// i.e. the count of thresholds tau + j h (j = 1..7) the residual
// (t - T0)/128 - E reaches.  With a and b rounded up, a score exactly on a
// threshold (t = base + 128 j h) lands at or above j.  A score one binary32
// step below one can land there too when that step times a is below b's
// rounding; for the calibrated 128 h = 78 this happens only at t >= 16384,
// for a score exactly one step below a threshold (an exact emulation over
// every binary32 score of the fast path's range finds no other case).
// Masked keys hold -inf: code 0.  FAST: the block max lies in [T0 - 16000,
// TgEff], so E is in [-125, 127], no clamp acts and every product is below
// (1 - tau) / h + 1 <= 4161 (h >= 1/64, tau >= -64): it fits the 16-bit
// halves the codes are packed through.
__device__ __forceinline__ float next_up(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x == 0.0f) return __uint_as_float(1u);
  return __uint_as_float((int32_t)u >= 0 ? u + 1u : u - 1u);
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <bool FAST>
__device__ __forceinline__ void p_efq(const v16f (&S)[2], float m0, float m1, float T0, float ea, float et128,
                                      v4i& pA, int& pS, uint32_t (&dsc)[2]) {
  const float tm = __builtin_fmaxf(m0, m1);
  float ef = __builtin_floorf((tm - T0) * (1.0f / 128.0f));
  if (!FAST) ef = __builtin_fminf(__builtin_fmaxf(ef, -1000.0f), 1000.0f);
  const int E = (int)ef;
  const uint32_t sc = FAST ? (uint32_t)(E + 125) : (uint32_t)min(max(E + 125, 0), 254);
  const float base = (T0 + (float)(128 * E)) + et128;
  // b = -base a rounded up: the product's rounding error decides the step
  const float bn = -base * ea;
  const float b = __builtin_fmaf(-base, ea, -bn) > 0.0f ? next_up(bn) : bn;
  auto ucode = [&](int e) -> float {
    float u = __builtin_fmaf(S[e >> 4][e & 15], ea, b);
    if (!FAST) u = __builtin_fminf(u, 7.0f);
    return u;
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // dword j holds elements 8j .. 8j+7, element 8j+i in bits [4i, 4i+4):
    // halves (8j+i, 8j+i+4) are packed first, clamped to 7 together, then
    // interleaved by nibble.  The float -> u32 converts truncate (floor for
    // u >= 0, 0 below and for -inf); the high half's convert writes straight
    // into the upper 16 bits (SDWA), its input being a product
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t xw = __float2uint_rz(ucode(8 * j + i));
      asm("v_cvt_u32_f32_sdwa %0, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
          : "+v"(xw)
          : "v"(ucode(8 * j + i + 4)));
      u16x2 h2 = __builtin_bit_cast(u16x2, xw);
      h2 = __builtin_elementwise_min(h2, (u16x2){7, 7});
      w[i] = __builtin_bit_cast(uint32_t, h2);
    }
    const uint32_t x = w[0] | (w[1] << 4), y = w[2] | (w[3] << 4);
    pA[j] = (int)(x | (y << 8));
  }
  pS = (int)sc;
  dsc[0] = sc;
  dsc[1] = sc;
}

// optional P dump (debug): one code byte per key and the E8M0 per 32 keys
template <int PE>
__device__ __forceinline__ void dump_p(const FwdArgs& a, int bh, int qq, int q_len, int k0, int hh,
                                       const typename POp<PE>::T& pA,
                                       const uint32_t (&dsc)[2]) {
  if (bh != a.pd_bh || qq < a.pd_row0 || qq >= a.pd_row1 || qq >= q_len) return;
  const int nb32 = a.nb32;
  const size_t S32 = (size_t)nb32 * 32;
  uint8_t* drow = a.pd_codes + (size_t)(qq - a.pd_row0) * S32;
  uint8_t* srow = a.pd_scales + (size_t)(qq - a.pd_row0) * nb32;
  constexpr int bits = Fmt<PE>::bits;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int key = k0 + step_key<PE>(e >> 4, e & 15, hh);
    const int pos = e * bits;
    uint32_t wv = (uint32_t)pA[pos >> 5] >> (pos & 31);
    if ((pos & 31) + bits > 32) wv |= (uint32_t)pA[(pos >> 5) + 1] << (32 - (pos & 31));
    if (key < (int)S32) drow[key] = (uint8_t)(wv & ((1u << bits) - 1));
  }
  const int kb = k0 / 32 + hh;
  if (kb < nb32) srow[kb] = (uint8_t)(Opd<PE>::split ? dsc[hh] : dsc[0]);
}

// O / l of the wave's 32 queries to bf16 (RNE), and the rollback counts.
// Rows past q_len, and rows with l = 0 (no visible key), are stored as 0.
// O lane (c, h) register 4i+j holds query 8i+4h+j, feature 32 o + c.
template <int NV, int D>
__device__ __forceinline__ void store_rows(const FwdArgs& a, int bh, int qw0, int q_len, int n, int hh,
                                           const v16f (&O)[NV], const float (&lq)[16], int cnt) {
  const int Sq = a.Sq;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qq = qw0 + 8 * i + 4 * hh + j;
      if (qq < Sq) {
        const bool live = qq < q_len && lq[4 * i + j] > 0.0f;
        const float inv = live ? 1.0f / lq[4 * i + j] : 0.0f;
        uint16_t* orow = a.out + ((size_t)bh * Sq + qq) * D;
#pragma unroll
        for (int o = 0; o < NV; ++o) {
          uint32_t uo = live ? __float_as_uint(O[o][4 * i + j] * inv) : 0u;
          uo = (uo + 0x7FFFu + ((uo >> 16) & 1u)) >> 16;  // RNE to bf16 (finite values)
          orow[32 * o + n] = (uint16_t)uo;
        }
      }
    }
  if (a.counts != nullptr && hh == 0 && qw0 + n < Sq) a.counts[(size_t)bh * Sq + qw0 + n] = qw0 + n < q_len ? cnt : 0;
}

// l accumulator: FP6 P -> 16x16 layout (v4f), FP8 P -> the layout of O (v16f)
template <int PE> struct LAcc { typedef v4f T; };
template <> struct LAcc<E4M3> { typedef v16f T; };

// value of lane `base/4 + k` for a byte address base; base is made opaque
// first so that the address arithmetic is not hoisted out of the (rare) path
// that uses it, where it would hold registers for the whole loop
__device__ __forceinline__ float lane_bcast(float v, int base, int k) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(base + 4 * k, __float_as_int(v)));
}

// rho of query q is held by lanes q and q+32; O lane (c, h) reg 4i+j holds query 8i+4h+j
template <int PE, int NV>
__device__ __forceinline__ void rescale(v16f (&O)[NV], typename LAcc<PE>::T& L, float rho, int lane) {
  int base = (lane >> 5) << 4;  // byte address of lane 4h
  asm volatile("" : "+v"(base));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float r = lane_bcast(rho, base, 8 * i + j);
#pragma unroll
      for (int o = 0; o < NV; ++o) O[o][4 * i + j] *= r;
      if constexpr (Opd<PE>::split) L[4 * i + j] *= r;
    }
  if constexpr (!Opd<PE>::split) {
    // 16x16 layout: lane (c16, g) reg k holds l of query 4g+k (c16 < 8) or 16+4g+k
    const int c16 = lane & 15, g = (lane >> 4) & 3;
    int lb = 4 * ((c16 < 8 ? 0 : 16) + 4 * g);
    asm volatile("" : "+v"(lb));
#pragma unroll
    for (int k = 0; k < 4; ++k) L[k] *= lane_bcast(rho, lb, k);
  }
}

template <int QK, int VE, int PE, int D, bool KV128, bool DUMP, bool X8>
__global__ void __launch_bounds__(NW * 64, 1) fsattn_fwd_kernel(FwdArgs a) {
  static_assert(!X8 || QK == E4M3, "decoded score products are for E4M3 Q/K");
  using G = Geo<QK, VE, D>;
  using LT = typename LAcc<PE>::T;
  using PT = typename POp<PE>::T;
  constexpr int NV = G::NV;
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int bh = blockIdx.y + blockIdx.z * a.H;
  const int Sq = a.Sq, Skv = a.Skv, nb32 = a.nb32;
  // valid queries and keys of this batch (variable-length attention); with a
  // causal mask query i sees keys k <= i + coff (queries aligned to the end
  // of the keys)
  const int q_len = a.q_lens ? min(max(a.q_lens[blockIdx.z], 0), Sq) : Sq;
  const int kv_len = a.kv_lens ? min(max(a.kv_lens[blockIdx.z], 0), Skv) : Skv;
  const int coff = kv_len - q_len;
  // causal workgroups differ in length: the longest start first
  const int q0 = (a.causal ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x) * QWG;
  const int qw0 = q0 + w * QW;
  // keys the workgroup reads: [0, kend), every key a valid query of it sees
  int kend = q0 < q_len ? kv_len : 0;
  if (a.causal) kend = max(min(kend, min(q0 + QWG, q_len) + coff), 0);
  const int ns = (kend + KS - 1) / KS;
  // keys [0, lim) are visible to this lane's query (lim <= 0: none).  Rows
  // past q_len are computed unmasked and not stored.
  const int lim = (a.causal && qw0 + n < q_len) ? min(kend, qw0 + n + coff + 1) : kend;
  // steps from ums on hold a masked key for some row of the wave (its first
  // row has the smallest limit): they take the exact path, which masks
  const int lim_w = (a.causal && qw0 < q_len) ? min(kend, qw0 + coff + 1) : kend;
  const int ums = max(lim_w, 0) / KS;
  if (ns == 0) {
    // no valid query or no visible key in the workgroup (uniform): zeros
    v16f Oz[G::NV];
    float lz[16];
#pragma unroll
    for (int o = 0; o < G::NV; ++o)
#pragma unroll
      for (int k = 0; k < 16; ++k) Oz[o][k] = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) lz[k] = 0.0f;
    store_rows<G::NV, D>(a, bh, qw0, q_len, n, hh, Oz, lz, 0);
    return;
  }

  // ---- DMA: this wave's loads (the same every step) and its two running
  // buffer descriptors (operand codes and scales of its side)
  const bool kside = w < 4;
  const int wj = w & 3;
  // K scales are read a dword at a time; for D = 64 (two bytes per key) the
  // head may start in the middle of a dword: read from the dword boundary and
  // shift every key by one
  const size_t ks0 = (size_t)bh * Skv * G::KSB;
  const int ko = (D == 64) ? (int)((ks0 >> 1) & 1) : 0;
  int l16[G::M16], v16[G::M16], lt[G::MT > 0 ? G::MT : 1], vt[G::MT > 0 ? G::MT : 1];
#pragma unroll
  for (int k = 0; k < G::M16; ++k) {
    const Dma d = dma16<QK, VE, PE, D>(kside, wj + 4 * k, lane, nb32);
    l16[k] = __builtin_amdgcn_readfirstlane(d.lds);
    v16[k] = d.voff;
  }
#pragma unroll
  for (int k = 0; k < G::MT; ++k) {
    const Dma d = dma4<QK, VE, PE, D>(kside, wj + 4 * k, lane, nb32);
    lt[k] = __builtin_amdgcn_readfirstlane(d.lds);
    vt[k] = d.voff;
  }
  const Dma dsl = dma_scale<QK, VE, PE, D>(kside, wj, lane, ko);
  const int lsc = __builtin_amdgcn_readfirstlane(dsl.lds), vsc_off = dsl.voff;
  uint64_t cbase = kside ? (uint64_t)(uintptr_t)(a.kc + (size_t)bh * Skv * G::QRB)
                         : (uint64_t)(uintptr_t)(a.vc + (size_t)bh * D * nb32 * G::VBB);
  int crem = kside ? kend * G::QRB : D * nb32 * G::VBB;
  const int cstride = kside ? KS * G::QRB : 2 * G::VBB;
  uint64_t sbase = kside ? (uint64_t)(uintptr_t)(a.ks + (ks0 & ~(size_t)3))
                         : (uint64_t)(uintptr_t)(a.vs + (size_t)bh * nb32 * 128);
  int srem = kside ? (((kend + ko) * G::KSB + 3) & ~3) : nb32 * 128;
  const int sstride = kside ? KS * G::KSB : 256;
  int snext = 0;  // next step to fetch
  const uint32_t lds0 = lds_addr(smem);
  // the two descriptors live in SGPRs and move by one step per issue
  v4i rc = rsrc(cbase, crem), rs = rsrc(sbase, srem);
  auto advance = [](v4i& d, int& rem, int stride) {
    uint64_t b = ((uint64_t)(uint32_t)d[1] << 32) | (uint32_t)d[0];
    b += (uint64_t)stride;
    d[0] = (int)(uint32_t)b;
    d[1] = (int)(uint32_t)(b >> 32);
    rem -= stride;
    d[2] = rem > 0 ? rem : 0;
  };

  // loads of step snext into its slot; past the last step they read zeros
  auto issue = [&]() {
    const uint32_t slot = lds0 + (uint32_t)((snext & (NS - 1)) * G::SLOT);
    const uint32_t keep = m0_save();
#pragma unroll
    for (int k = 0; k < G::M16; ++k) dma_x4(rc, slot, (uint32_t)l16[k], v16[k]);
#pragma unroll
    for (int k = 0; k < G::MT; ++k) dma_x1(rc, slot, (uint32_t)lt[k], vt[k]);
    dma_x1(rs, slot, (uint32_t)lsc, vsc_off);
    m0_restore(keep);
    advance(rc, crem, cstride);
    advance(rs, srem, sstride);
    ++snext;
  };

  // ---- Q operands (B of the score product) and their scales
  v8i qB[G::DH];
  int qS[G::DH];
  {
    const int qrow = min(qw0 + n, Sq - 1);
    const uint8_t* qp = a.qc + ((size_t)bh * Sq + qrow) * G::QRB;
    const uint8_t* qsp = a.qs + ((size_t)bh * Sq + qrow) * G::KSB;
#pragma unroll
    for (int dh = 0; dh < G::DH; ++dh) {
      int ca, cb;
      k_chunks<QK, D>(0, dh, hh, ca, cb);
      const uint2 x0 = *reinterpret_cast<const uint2*>(qp + ca);
      const uint2 x1 = *reinterpret_cast<const uint2*>(qp + ca + 8);
      v8i r = {(int)x0.x, (int)x0.y, (int)x1.x, (int)x1.y, 0, 0, 0, 0};
      if constexpr (Opd<QK>::tail == 16) {
        const uint4 y = *reinterpret_cast<const uint4*>(qp + cb);
        r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
      } else if constexpr (Opd<QK>::tail == 8) {
        const uint2 y = *reinterpret_cast<const uint2*>(qp + cb);
        r[4] = y.x; r[5] = y.y;
      }
      qB[dh] = r;
      qS[dh] = (int)qsp[2 * dh + hh];
    }
  }
  // X8: the Q operands decoded to BF16 (exact: 4 significant bits times a
  // power of two), group c of feature half dh = dwords 2c, 2c+1 of qB[dh]
  v8bf qX[X8 ? G::DH : 1][4];
  if constexpr (X8) {
    const int qrow = min(qw0 + n, Sq - 1);
    const uint8_t* qsp = a.qs + ((size_t)bh * Sq + qrow) * G::KSB;
#pragma unroll
    for (int dh = 0; dh < G::DH; ++dh) {
      const float s0 = e8m0_to_float(qsp[2 * dh]), s1 = e8m0_to_float(qsp[2 * dh + 1]);
#pragma unroll
      for (int c = 0; c < 4; ++c) qX[dh][c] = dec8(qB[dh][2 * c], qB[dh][2 * c + 1], c < 2 ? s0 : s1);
    }
  }
  // K scale shift per key group: the dword holds the key's block scales
  // (D = 128) or those of an even/odd key pair (D = 64)
  int ksh[2];
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    const int key = row_key<PE>(kg, n) + ko;
    ksh[kg] = (D == 128 ? 0 : 16 * (key & 1)) + (X8 ? 0 : 8 * hh);
  }
  // ones operand of the l product.  FP6 P (16x16x128, lanes read as rows
  // l%16 and K blocks l/16): column c16 < 8 sums the blocks of query r
  // (K blocks 0 and 2), c16 >= 8 those of query r+16 (blocks 1 and 3).
  v8i ones;
  if constexpr (Opd<PE>::split) {
    ones = v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838};
  } else {
    const int c16 = lane & 15, g = lane >> 4;
    const bool on = ((g & 1) == 0) == (c16 < 8);
    const int v = on ? 0x22222222 : 0;
    ones = v8i{v, v, v, v, 0, 0, 0, 0};
  }

  const float T0 = a.T0, Tg = a.Tg;
  // above TgEff the stage-1 clamp could act: exact path (kept in an SGPR)
  const float TgEff = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(fminf(Tg, 32639.0f))));
  // E2M1 P is the EFQ-style rule (p_efq): its slope and 128 tau
  constexpr bool EFQ = PE == E2M1;
  const float ea = a.efq_a, et128 = a.efq_t128;
  // fast-path lower bound of a block max: the BF16 flush bound, or (EFQ) an
  // E8M0 that needs no clamp (fl32(max - T0) >= -16000, E >= -125)
  // the fast-path range PFlush <= max <= TgEff as one unsigned compare of the
  // float bits: both bounds are positive, so a smaller, negative, infinite or
  // NaN max lands outside [0, RG1) after the subtraction (RG1 = 0: empty)
  const uint32_t RG1 = __builtin_amdgcn_readfirstlane(
      TgEff >= PFlush<EFQ ? E2M3 : PE>::t
          ? __float_as_uint(TgEff) - __float_as_uint(PFlush<EFQ ? E2M3 : PE>::t) + 1u
          : 0u);
  auto low_ok = [&](float mx) -> float {
    if constexpr (EFQ) return (mx - T0) + 16000.0f;
    else return mx - PFlush<PE>::t;
  };

  // X8: the decoded score products start from zero and C is added to each
  // score once, in binary32, after the products (fl32(fl32(sum) + C)); the
  // sum is accumulated at its own magnitude, far below C's.  Otherwise C is
  // the accumulator's initial value (FP6/FP4 products are exact).
  float C = 0.0f;
  v16f Cv;  // C splat: the accumulator's initial value of the score product
#pragma unroll
  for (int k = 0; k < 16; ++k) Cv[k] = 0.0f;
  auto set_C = [&](float c) {
    C = c;
    if constexpr (!X8) {
#pragma unroll
      for (int k = 0; k < 16; ++k) Cv[k] = c;
    }
  };
  int cnt = 0;
  v16f O[NV];
#pragma unroll
  for (int o = 0; o < NV; ++o)
#pragma unroll
    for (int k = 0; k < 16; ++k) O[o][k] = 0.0f;
  LT L;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(LT) / 4); ++k) L[k] = 0.0f;

  // K operands of a step (and the lane's two K block-scale words), read from
  // the LDS ring ahead of the score product that uses them
  struct KOps {
    v8i op[2 * G::DH];
    uint32_t kd[2];
  };
  auto read_k = [&](int s) -> KOps {
    const uint8_t* slot = smem + (s & (NS - 1)) * G::SLOT;
    KOps k;
    k.kd[0] = *reinterpret_cast<const uint32_t*>(slot + G::KS_OFF + 4 * n) >> ksh[0];
    k.kd[1] = *reinterpret_cast<const uint32_t*>(slot + G::KS_OFF + 128 + 4 * n) >> ksh[1];
    // with X8 (ksh without the lane half) byte b of kd holds the key's block b
    // scale (D = 64: of blocks 0 and 1)
#pragma unroll
    for (int i = 0; i < 2 * G::DH; ++i) k.op[i] = lds_operand<QK>(slot + G::K_OFF + i * Opd<QK>::region, lane);
    return k;
  };
  // S^T = K Q^T + C for the 64 keys of a step: both key groups' first
  // feature half (initial value C), then the second
  auto scores_of = [&](v16f (&S)[2], const KOps& k) {
    if constexpr (X8) {
      // decoded K groups against decoded Q groups on the BF16 matrix core:
      // four 32x32x16 products per feature half and key group
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int dh = 0; dh < G::DH; ++dh) {
          const v8i& ka = k.op[kg * G::DH + dh];
          const float s0 = e8m0_to_float((k.kd[kg] >> (16 * dh)) & 0xFFu);
          const float s1 = e8m0_to_float((k.kd[kg] >> (16 * dh + 8)) & 0xFFu);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const v8bf kx = dec8(ka[2 * c], ka[2 * c + 1], c < 2 ? s0 : s1);
            if (dh == 0 && c == 0) S[kg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx, qX[0][0], Cv, 0, 0, 0);
            else S[kg] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx, qX[X8 ? dh : 0][c], S[kg], 0, 0, 0);
          }
        }
      return;
    }
#pragma unroll
    for (int dh = 0; dh < G::DH; ++dh)
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        const int ksc = (int)k.kd[kg];
        const v8i& ka = k.op[kg * G::DH + dh];
        if (dh == 0)
          S[kg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qB[0], Cv, QK, QK, 0, ksc, 0, qS[0]);
        else
          S[kg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qB[G::DH - 1], S[kg], QK, QK, 2, ksc, 0,
                                                                  qS[G::DH - 1]);
      }
    // Cv stays live past the products, so neither of them is selected in the
    // form that accumulates in place over Cv (which costs a copy of Cv)
    asm volatile("" ::"v"(Cv));
  };
  auto scores = [&](v16f (&S)[2], int s) { scores_of(S, read_k(s)); };
  // V operands of a step and the lane's V scale word, read ahead of the PV
  // product that uses them
  struct VOps {
    v8i op[NV];
    int vsc;
  };
  auto read_v = [&](int s) -> VOps {
    const uint8_t* slot = smem + (s & (NS - 1)) * G::SLOT;
    VOps v;
    v.vsc = *reinterpret_cast<const int*>(slot + G::VS_OFF + 4 * lane);
#pragma unroll
    for (int o = 0; o < NV; ++o) v.op[o] = lds_operand<VE>(slot + G::V_OFF + o * Opd<VE>::region, lane);
    return v;
  };
  // O += P V (feature block o) and l += P 1
  auto pv_of = [&](const PT& pa6, int ps, const VOps& v) {
    const v8i pa = widen(pa6);
    O[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, v.op[0], O[0], PE, VE, 0, ps, 0, v.vsc);
    O[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, v.op[1], O[1], PE, VE, 0, ps, 1, v.vsc);
    if constexpr (NV > 2) {
      O[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, v.op[2], O[2], PE, VE, 0, ps, 2, v.vsc);
      O[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, v.op[3], O[3], PE, VE, 0, ps, 3, v.vsc);
    }
    if constexpr (Opd<PE>::split)
      L = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pa, ones, L, PE, E4M3, 0, ps, 0, 127);
    else
      L = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa, ones, L, PE, E2M1, 0, ps, 0, 127);
  };
  auto mask = [&](v16f (&S)[2], int nk) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (step_key<PE>(kg, k, hh) >= nk) S[kg][k] = -INFINITY;
  };
  auto shift = [&](v16f (&S)[2], float d) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int k = 0; k < 16; ++k) S[kg][k] = S[kg][k] + d;
  };
  // 128-key gate tile: the lane's maximum over the odd step s of the tile,
  // with the current offset (its scores are recomputed on step s itself)
  auto ahead_max = [&](int s) -> float {
    v16f Sn[2];
    scores(Sn, s);
    if (s >= ums) mask(Sn, lim - s * KS);
    // X8: max fl32(t + C) = fl32(max t + C), the map being monotonic
    return X8 ? max32(Sn) + C : max32(Sn);
  };

  PT pA = {};
  int pS = 127;

  // fast-path test of step u: the lane's maxima over its two key groups, and
  // whether the step must leave the fast path (a block max below PFlush or
  // the gate-tile max above TgEff)
  // (mnext: the maximum of step u + 1 when u starts a 128-key gate tile)
  struct Check {
    float m0, m1;
    bool bad;  // the step cannot take the fast path (as seen by this lane)
  };
  // the fast-path test on a lane's block max (one P block per lane, 64-key
  // gate tiles); the gate-only path evaluates it again rather than carrying
  // both polarities of the test through the fast path
  auto ok_of = [&](float tm) -> bool {
    if constexpr (!EFQ) return __float_as_uint(tm) - __float_as_uint(PFlush<EFQ ? E2M3 : PE>::t) < RG1;
    else return __builtin_fminf(TgEff - tm, low_ok(tm)) >= 0.0f;
  };
  auto check = [&](const v16f (&S)[2], int u, float mnext) -> Check {
    const float m0 = max16(S[0]), m1 = max16(S[1]);
    float tm, lo;
    if constexpr (Opd<PE>::split) {
      const float b0 = vmax(m0, wshfl(m0, lane ^ 32)), b1 = vmax(m1, wshfl(m1, lane ^ 32));
      lo = __builtin_fminf(b0, b1);
      tm = __builtin_fmaxf(b0, b1);
    } else {
      tm = __builtin_fmaxf(m0, m1);
      lo = tm;
    }
    if constexpr (KV128) {
      if ((u & 1) == 0 && u + 1 < ns) tm = __builtin_fmaxf(tm, mnext);
    }
    if constexpr (!Opd<PE>::split && !KV128 && !EFQ)
      return Check{m0, m1, !(__float_as_uint(tm) - __float_as_uint(PFlush<PE>::t) < RG1)};
    else
      return Check{m0, m1, !(__builtin_fminf(TgEff - tm, low_ok(lo)) >= 0.0f)};
  };

  // exact conversion of step u: masking, reference (FIRST: step 0), gate,
  // flush and clamp; sets pA/pS and the gate outcome (rho, any_fire)
  float rho = 1.0f;
  bool any_fire = false;
  auto exact = [&](v16f (&S)[2], int u, float mnext, uint32_t (&dsc)[2], auto first_t) {
    constexpr bool FIRST = decltype(first_t)::value;
    if (u >= ums) {
      // the limit is formed here, on the rare path (kept from becoming a
      // per-lane counter stepped on every step)
      int uks = u * KS;
      asm volatile("" : "+s"(uks));
      mask(S, lim - uks);
    }
    float m = max32(S);
    if constexpr (KV128) {
      if ((u & 1) == 0 && u + 1 < ns) m = __builtin_fmaxf(m, mnext);
    }
    m = __builtin_fmaxf(m, wshfl(m, lane ^ 32));
    rho = 1.0f;
    any_fire = false;
    if (FIRST) {
      // a row that sees no key keeps P = 0 (its scores stay -inf)
      set_C(m > -INFINITY ? T0 - m : 0.0f);
      shift(S, C);
    } else if (!KV128 || (u & 1) == 0) {
      const bool fire = m > Tg;
      const float delta = fire ? m - T0 : 0.0f;
      if (fire) {
        shift(S, -delta);
        cnt += 1;
        rho = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
      }
      any_fire = __ballot(fire) != 0;
      if (any_fire) {
        // in place: Cv holds C in every register
        C = C - delta;
        if constexpr (!X8) {
#pragma unroll
          for (int k = 0; k < 16; ++k) Cv[k] = Cv[k] - delta;
        }
      }
    }
    if constexpr (EFQ) {
      p_efq<false>(S, max16(S[0]), max16(S[1]), T0, ea, et128, pA, pS, dsc);
    } else {
      float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float v = S[kg][k];
          const float f = (v >= 128.0f) ? __builtin_fminf(v, 32639.5f) : -INFINITY;
          S[kg][k] = f;
          if (kg == 0) mx0 = __builtin_fmaxf(mx0, f);
          else mx1 = __builtin_fmaxf(mx1, f);
        }
      uint32_t wv[16];
      pack_b(S, wv, mx0, mx1);
      p_from_w<PE, false>(wv, mx0, mx1, lane, pA, pS, dsc);
    }
  };

  // gate-only rare step (64-key gate tiles, one P block per lane, no masked
  // key): the fast-path test failed only because a row's maximum passed the
  // gate.  The row maximum, the shift and the shifted lane maxima follow from
  // the test's lane maxima; when every lane's shifted maximum still clears the
  // flush bound the fast conversion is exact on the shifted scores, and the
  // exact path is skipped.  Returns false (nothing changed) otherwise.
  auto gate_fast = [&](v16f (&S)[2], const Check& c, uint32_t (&dsc)[2]) -> bool {
    const float tm = __builtin_fmaxf(c.m0, c.m1);
    const float mrow = __builtin_fmaxf(tm, wshfl(tm, lane ^ 32));
    const bool fire = mrow > Tg;
    const float delta = fire ? mrow - T0 : 0.0f;
    // max(fl32(s - delta)) = fl32(max s - delta): the maps are monotonic
    const float m0 = c.m0 - delta, m1 = c.m1 - delta;
    const bool ok = fire ? low_ok(__builtin_fmaxf(m0, m1)) >= 0.0f : ok_of(tm);
    if (__ballot(!ok) != 0) return false;
    rho = 1.0f;
    if (fire) {
      shift(S, -delta);
      cnt += 1;
      rho = __builtin_amdgcn_exp2f(-delta * (1.0f / 128.0f));
    }
    any_fire = __ballot(fire) != 0;
    if (any_fire) {
      C = C - delta;
      if constexpr (!X8) {
#pragma unroll
        for (int k = 0; k < 16; ++k) Cv[k] = Cv[k] - delta;
      }
    }
    if constexpr (EFQ) {
      p_efq<true>(S, m0, m1, T0, ea, et128, pA, pS, dsc);
    } else {
      uint32_t wv[16];
      pack_b(S, wv, m0, m1);
      p_from_w<PE, true>(wv, m0, m1, lane, pA, pS, dsc);
    }
    return true;
  };

  // one barrier per step: before it each wave waits for its loads of the
  // steps up to u + 1 (u + 2 with 128-key gate tiles, whose odd step is read
  // one step early); after it the loads of step u + PF go into the slot of
  // step u - 2, which every wave finished reading before the barrier
  auto sync = [&]() {
    wait_vm<(KV128 ? PF - 3 : PF - 2) * G::PER_WAVE>();
    barrier();
    issue();
  };
  // scores of step s (and, when s starts a 128-key gate tile, the maximum of
  // step s + 1 with the same offset)
  float mn = 0.0f;
  auto next_scores = [&](v16f (&S)[2], int s) {
    if constexpr (KV128) {
      if ((s & 1) == 0 && s + 1 < ns) mn = ahead_max(s + 1);
    }
    scores(S, s);
  };
  // keep a value computed in a branch inside that branch (the compiler
  // would otherwise sink the producing matrix instructions past the merge)
  auto pin16 = [](v16f& x) { asm volatile("" : "+v"(x)); };

  for (int s = 0; s < PF; ++s) issue();
  v16f S[2];
  sync();
  next_scores(S, 0);
  {
    uint32_t dsc[2];
    exact(S, 0, mn, dsc, std::true_type{});
    if constexpr (DUMP) dump_p<PE>(a, bh, qw0 + n, q_len, 0, hh, pA, dsc);
  }
  // V operands are read a phase ahead except with FP8 P (FP8 V operands
  // are 8 registers each; there the registers are not available)
  constexpr bool PRE_V = !Opd<PE>::split;
  constexpr bool PRE_K = !Opd<QK>::split;  // the same for FP8 K operands
  VOps vop;
  if constexpr (PRE_V) vop = read_v(0);
  next_scores(S, 1);
  // step u: the K operands of step u + 1 are read while the PV products of
  // step u - 1 run on the matrix core and the VALU converts the scores of
  // step u (along the fast path always: on a rare step the exact path
  // overwrites its result); then the V operands of step u are read and the
  // score product of step u + 1 is issued.  Operand reads thus have a whole
  // phase of the step to arrive.
  for (int u = 1; u < ns; ++u) {
    sync();
    KOps kop;
    if constexpr (PRE_K) kop = read_k(u + 1);
    // the PV products and the conversion run at raised wave priority: when
    // both waves of a SIMD can issue, the one feeding the matrix core while
    // converting goes first (the rest of the step runs at the normal level)
    __builtin_amdgcn_s_setprio(3);
    if constexpr (PRE_V) pv_of(pA, pS, vop);
    else pv_of(pA, pS, read_v(u - 1));
    if constexpr (X8) shift(S, C);
    const Check c = check(S, u, mn);
    const bool rare = (u >= ums) | (__ballot(c.bad) != 0);
    uint32_t dsc[2];
    PT pAf;
    int pSf;
    if constexpr (EFQ) {
      p_efq<true>(S, c.m0, c.m1, T0, ea, et128, pAf, pSf, dsc);
    } else {
      uint32_t wv[16];
      pack_b(S, wv, c.m0, c.m1);
      p_from_w<PE, true>(wv, c.m0, c.m1, lane, pAf, pSf, dsc);
    }
    // computed here on every step (not sunk into the fast branch)
    asm volatile("" : "+v"(pAf), "+v"(pSf));
#pragma unroll
    for (int o = 0; o < NV; ++o) pin16(O[o]);
    asm volatile("" : "+v"(L));
    // one PV product per group of VALU work, as measured: 40 with FP8 P (its
    // pair converters make the conversion long), 11 with FP6 operands or
    // EFQ-style P (with FP6 operands the P conversion then lands after the
    // last product, so the new P needs almost no copies), 15 otherwise
    constexpr int VPG = Opd<PE>::split ? 40 : ((EFQ || Opd<QK>::tail == 8) ? 11 : 15);
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * G::DH + 2, 0);
#pragma unroll
    for (int i = 0; i < NV + 1; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPG, 0);
    }
    pA = pAf;
    pS = pSf;
    __builtin_amdgcn_s_setprio(0);
    if (rare) {
      bool done = false;
      if constexpr (!KV128 && !Opd<PE>::split) done = u < ums && gate_fast(S, c, dsc);
      if (!done) exact(S, u, mn, dsc, std::false_type{});
      if (any_fire) rescale<PE, NV>(O, L, rho, lane);
    }
    if constexpr (DUMP) dump_p<PE>(a, bh, qw0 + n, q_len, u * KS, hh, pA, dsc);
    if constexpr (PRE_V) vop = read_v(u);
    if constexpr (KV128) {
      if (((u + 1) & 1) == 0 && u + 2 < ns) mn = ahead_max(u + 2);
    }
    if constexpr (PRE_K) scores_of(S, kop);
    else scores_of(S, read_k(u + 1));
  }
  if constexpr (PRE_V) pv_of(pA, pS, vop);
  else pv_of(pA, pS, read_v(ns - 1));
  wait_vm<0>();  // loads past the end are still in flight

  // ---- epilogue: O / l -> bf16; counts
  float lq[16];
  if constexpr (Opd<PE>::split) {
#pragma unroll
    for (int k = 0; k < 16; ++k) lq[k] = L[k];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int srcl = 16 * (2 * (i & 1) + hh) + 8 * (i >> 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) lq[4 * i + j] = wshfl(L[j], srcl);
    }
  }
  store_rows<NV, D>(a, bh, qw0, q_len, n, hh, O, lq, cnt);
}

template <int QK, int VE, int PE, int D, bool X8>
hipError_t launch_t(const FwdArgs& a, int B, hipStream_t stream) {
  dim3 grid((unsigned)((a.Sq + QWG - 1) / QWG), (unsigned)a.H, (unsigned)B);
  const bool dump = a.pd_codes != nullptr;
  if (a.kv128) {
    if (dump) hipLaunchKernelGGL((fsattn_fwd_kernel<QK, VE, PE, D, true, true, X8>), grid, dim3(NW * 64), 0, stream, a);
    else hipLaunchKernelGGL((fsattn_fwd_kernel<QK, VE, PE, D, true, false, X8>), grid, dim3(NW * 64), 0, stream, a);
  } else {
    if (dump) hipLaunchKernelGGL((fsattn_fwd_kernel<QK, VE, PE, D, false, true, X8>), grid, dim3(NW * 64), 0, stream, a);
    else hipLaunchKernelGGL((fsattn_fwd_kernel<QK, VE, PE, D, false, false, X8>), grid, dim3(NW * 64), 0, stream, a);
  }
  return hipGetLastError();
}

template <int QK, int VE, int PE, bool X8>
hipError_t launch_x(const FwdArgs& a, int B, int D, hipStream_t s) {
  return D == 128 ? launch_t<QK, VE, PE, 128, X8>(a, B, s) : launch_t<QK, VE, PE, 64, X8>(a, B, s);
}
// E4M3 Q/K: decoded BF16 score products unless the FP8 products are asked for
template <int QK, int VE, int PE>
hipError_t launch_d(const FwdArgs& a, int B, int D, hipStream_t s) {
  if constexpr (QK == E4M3) {
    if (!a.fp8_products) return launch_x<QK, VE, PE, true>(a, B, D, s);
  }
  return launch_x<QK, VE, PE, false>(a, B, D, s);
}

}  // namespace

// supported combinations: FP8 P with FP8 V; FP6 (E2M3) P with FP6 or FP4 V;
// FP6 E3M2 P with FP6 (E2M3) or FP4 Q/K/V; EFQ-style FP4 (E2M1) P with FP6
// Q/K/V or FP4 Q/K/V
bool fwd_supported(int qk, int ve, int pe) {
  if (pe == E4M3) return ve == E4M3 && (qk == E4M3 || qk == E2M3 || qk == E2M1);
  if (pe == E2M3) return (ve == E2M3 || ve == E2M1) && (qk == E4M3 || qk == E2M3 || qk == E2M1);
  if (pe == E3M2) return (qk == E2M3 && ve == E2M3) || (qk == E2M1 && ve == E2M1);
  if (pe == E2M1) return (qk == E2M3 && ve == E2M3) || (qk == E2M1 && ve == E2M1);
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
  FS_CASE(E2M3, E2M3, E3M2)
  FS_CASE(E2M1, E2M1, E3M2)
  FS_CASE(E2M3, E2M3, E2M1)
  FS_CASE(E2M1, E2M1, E2M1)
#undef FS_CASE
  return hipErrorInvalidValue;
}

}  // namespace fsattn
