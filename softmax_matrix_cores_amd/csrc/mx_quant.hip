// mx_quant.hip -- MX quantizer for Q, K (blocks along the feature axis) and V
// (blocks along keys, written key-contiguous).
//
// Operand quantization of the method's MXFP8 / MXFP6 / MXFP4 configurations
// ("Fused-Softmax shifts an AI attention bottleneck onto faster GPU
// hardware", paragraphs 7-8).  Q additionally carries the multiplicative part
// of the fold (128*log2(e)*softmax scale, paragraph 6: the Schraudolph map's
// linear transform is folded into the score product).
//
// HBM-bound: each lane owns one 32-element block, reads 64 bytes of bf16,
// takes the block max in registers, derives the E8M0 code with integer
// exponent arithmetic and converts the 32 values with the CDNA4 scaled
// converters, then writes the packed codes and the scale byte.
#include "internal.h"
#include "mx_device.h"

namespace fsattn {

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

// Convert 32 fp32 values into packed element codes of block scale X (the
// hardware converters divide by X).  w receives bits dwords.  bf16_exact:
// every value is an exact bf16 (no prescale applied).
template <int ELEM>
__device__ __forceinline__ void encode32(const float* x, float X, uint32_t* w, bool bf16_exact) {
  if constexpr (ELEM == E4M3 || ELEM == E5M2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v2s r = {0, 0};
      if constexpr (ELEM == E4M3) {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, x[4 * i + 0], x[4 * i + 1], X, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, x[4 * i + 2], x[4 * i + 3], X, true);
      } else {
        r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, x[4 * i + 0], x[4 * i + 1], X, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, x[4 * i + 2], x[4 * i + 3], X, true);
      }
      w[i] = (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
    }
  } else if constexpr (ELEM == E2M3 || ELEM == E3M2) {
    // hardware bf16 -> FP6 converter (RNE of v / X).  Values that are not
    // exact bf16 (a prescale was applied) are first rounded to odd into bf16:
    // truncated, with the OR of the dropped bits kept in the last bit.  bf16
    // keeps at least two more bits than either 6-bit format at every
    // magnitude (subnormals included), so the converter's rounding of the
    // rounded-to-odd value is the correctly rounded result of the fp32 value
    // (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
    // proved algorithms using rounding to odd", IEEE Trans. Computers 2008).
    v32bf v;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t u = __float_as_uint(x[i]);
      const uint32_t b = bf16_exact ? (u >> 16) : ((u >> 16) | min(u & 0xFFFFu, 1u));
      v[i] = __builtin_bit_cast(__bf16, (uint16_t)b);
    }
    v6i r;
    if constexpr (ELEM == E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, X);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(v, X);
#pragma unroll
    for (int i = 0; i < 6; ++i) w[i] = (uint32_t)r[i];
  } else {  // E2M1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t u = 0;
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[8 * i + 0], x[8 * i + 1], X, 0);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[8 * i + 2], x[8 * i + 3], X, 1);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[8 * i + 4], x[8 * i + 5], X, 2);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[8 * i + 6], x[8 * i + 7], X, 3);
      w[i] = u;
    }
  }
}

// Quantize one block held in registers; returns the E8M0 code.
template <int ELEM>
__device__ __forceinline__ uint32_t quant_block(float* x, bool fitmax, uint32_t* w, bool bf16_exact) {
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax_bits = max(amax_bits, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  uint32_t code = e8m0_from_amax_bits<ELEM>(amax_bits, fitmax);
  if (code == 255u) {  // NaN/Inf in the block: outside the contract; scale NaN, codes 0
#pragma unroll
    for (int i = 0; i < Fmt<ELEM>::bits; ++i) w[i] = 0;
    return code;
  }
  float X = e8m0_to_float(code);
  if (!fitmax && (ELEM == E4M3 || ELEM == E5M2)) {
    // OCP floor rule can overflow the FP8 range: saturate explicitly
    float lim = Fmt<ELEM>::maxnorm * X;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = fminf(fmaxf(x[i], -lim), lim);
  }
  encode32<ELEM>(x, X, w, bf16_exact);
  return code;
}

// Non-temporal form for outputs written as whole contiguous runs (axis 0:
// a wave writes 64 consecutive blocks), which no later step of the kernel
// reads: streamed past the caches.  Measured on the video shape: FP6 and FP4
// blocks 2-4 % faster, FP8 blocks 2 % slower; the axis-1 outputs (96-byte
// runs, partial lines) 50 % slower, so they keep ordinary stores.
typedef unsigned v4u_st __attribute__((ext_vector_type(4)));
typedef unsigned v2u_st __attribute__((ext_vector_type(2)));
template <int BYTES>
__device__ __forceinline__ void store_block_nt(uint8_t* dst, const uint32_t* w) {
  if constexpr (BYTES == 24) {
    v2u_st* d = reinterpret_cast<v2u_st*>(dst);
    __builtin_nontemporal_store((v2u_st){w[0], w[1]}, d);
    __builtin_nontemporal_store((v2u_st){w[2], w[3]}, d + 1);
    __builtin_nontemporal_store((v2u_st){w[4], w[5]}, d + 2);
  } else {
    __builtin_nontemporal_store((v4u_st){w[0], w[1], w[2], w[3]}, reinterpret_cast<v4u_st*>(dst));
  }
}

template <int BYTES>
__device__ __forceinline__ void store_block(uint8_t* dst, const uint32_t* w) {
  if constexpr (BYTES == 32) {
    uint4* d = reinterpret_cast<uint4*>(dst);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else if constexpr (BYTES == 24) {
    uint2* d = reinterpret_cast<uint2*>(dst);
    d[0] = make_uint2(w[0], w[1]);
    d[1] = make_uint2(w[2], w[3]);
    d[2] = make_uint2(w[4], w[5]);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// axis 0: one lane per 32-element block of a row; blocks are contiguous in
// both the input row and the packed output.
// EXACT: prescale is 1, so every value is an exact bf16 (no product, and the
// FP6 path needs no rounding to odd); chosen on the host, which keeps the
// other form's arithmetic out of the kernel.
template <int ELEM, bool VEC, bool EXACT>
__global__ void __launch_bounds__(256) mxq_axis0_kernel(const uint16_t* __restrict__ src, int64_t nrows,
                                                        int64_t nb, int64_t ld, float prescale, bool fitmax,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int BB = Fmt<ELEM>::bits * 4;
  int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nrows * nb) return;
  int64_t row = blk / nb, g = blk - row * nb;
  const uint16_t* p = src + row * ld + g * 32;
  float x[32];
  if constexpr (VEC) {
    const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 u = p4[i];
      uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = bf16_to_f32(uu[j] & 0xFFFFu);
        x[8 * i + 2 * j + 1] = bf16_to_f32(uu[j] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = bf16_to_f32(p[i]);
  }
  if constexpr (!EXACT) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] *= prescale;
  }
  uint32_t w[8];
  uint32_t code = quant_block<ELEM>(x, fitmax, w, EXACT);
  // FP6/FP4 blocks leave faster past the caches; 32-byte FP8 blocks do not
  if constexpr (BB < 32) store_block_nt<BB>(codes + blk * BB, w);
  else store_block<BB>(codes + blk * BB, w);
  scales[blk] = (uint8_t)code;
}

// Fused producer step for qk-normed models: RMS-normalise each row (weight w
// per feature), then the prescale and MX quantization along the row.  One
// lane per 32-element block as above; the nb = cols / 32 lanes of a row are
// consecutive lanes of one wave (nb a power of two, at most 64).  Per row:
//   ss = the squares summed in binary64 (each block's in index order, then the
//        block sums in order: every lane adds them in the same order, so the
//        row's lanes agree bit for bit), exact squares of bf16 values;
//   r  = fl32(1 / sqrt(ss / cols + eps)) in binary64 (correctly rounded root
//        and quotient), r = 0 when ss / cols + eps is 0;
//   y  = fl32(fl32(x r) w), then fl32(prescale y) is quantized.
template <int ELEM, bool VEC>
__global__ void __launch_bounds__(256) mxq_rms_kernel(const uint16_t* __restrict__ src, int64_t nrows, int nb,
                                                      int64_t ld, const float* __restrict__ weight, float eps,
                                                      float prescale, bool fitmax, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  constexpr int BB = Fmt<ELEM>::bits * 4;
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = blk < nrows * nb;  // rows never straddle the end: nrows * nb is a multiple of nb
  const int64_t row = blk / nb, g = blk - row * nb;
  float x[32];
  double s = 0.0;
  if (live) {
    const uint16_t* p = src + row * ld + g * 32;
    if constexpr (VEC) {
      const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = p4[i];
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[8 * i + 2 * j] = bf16_to_f32(uu[j] & 0xFFFFu);
          x[8 * i + 2 * j + 1] = bf16_to_f32(uu[j] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = bf16_to_f32(p[i]);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) s += (double)x[i] * (double)x[i];
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.0f;
  }
  // the row total, block sums in block order (every lane of the row alike)
  const int lane = threadIdx.x & 63;
  const int first = lane & ~(nb - 1);
  double ss = 0.0;
  for (int t = 0; t < nb; ++t) ss += __shfl(s, first + t, 64);
  if (!live) return;
  const double a = ss / (double)(32 * nb) + (double)eps;
  const float r = (a == 0.0) ? 0.0f : (float)(1.0 / __builtin_sqrt(a));
  if (weight != nullptr) {
    float wv[32];
    if constexpr (VEC) {
      const float4* w4 = reinterpret_cast<const float4*>(weight + g * 32);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 t = w4[i];
        wv[4 * i] = t.x; wv[4 * i + 1] = t.y; wv[4 * i + 2] = t.z; wv[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) wv[i] = weight[g * 32 + i];
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = ((x[i] * r) * wv[i]) * prescale;
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = (x[i] * r) * prescale;
  }
  uint32_t w[8];
  const uint32_t code = quant_block<ELEM>(x, fitmax, w, false);
  store_block<BB>(codes + blk * BB, w);
  scales[blk] = (uint8_t)code;
}

// axis 1: lane (m, key block kb, column d), d fastest so a wave's loads of one
// key row are contiguous; output row d holds the key blocks of that column.
// Scales are written block-major with the columns interleaved:
// [m][kb][d % 32][d / 32] (cols <= 128), so the four scales a PV lane needs
// for one key block sit in one dword.
template <int ELEM>
__global__ void __launch_bounds__(256) mxq_axis1_kernel(const uint16_t* __restrict__ src, int64_t n_mat,
                                                        int64_t rows, int64_t cols, int64_t ld, int64_t nb,
                                                        float prescale, bool fitmax, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  constexpr int BB = Fmt<ELEM>::bits * 4;
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n_mat * nb * cols) return;
  int64_t d = id % cols;
  int64_t t = id / cols;
  int64_t kb = t % nb;
  int64_t m = t / nb;
  const uint16_t* p = src + (m * rows) * ld + d;
  float x[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    int64_t r = kb * 32 + j;
    x[j] = (r < rows) ? bf16_to_f32(p[r * ld]) * prescale : 0.0f;
  }
  uint32_t w[8];
  uint32_t code = quant_block<ELEM>(x, fitmax, w, prescale == 1.0f);
  int64_t o = (m * cols + d) * nb + kb;
  store_block<BB>(codes + o * BB, w);
  scales[((m * nb + kb) * 32 + (d & 31)) * 4 + (d >> 5)] = (uint8_t)code;
}

// axis 1, direct (cols 64 or 128, rows 16-byte aligned): lane (key block kb,
// column octet co) loads 16 bytes (8 columns) of each of the block's 32 key
// rows and quantizes the eight column blocks from registers.  The COLS / 8
// lanes of one key block read whole rows (a wave covers 64 / (COLS / 8)
// consecutive key blocks, a workgroup KBG = 4 such groups of one matrix), and
// every lane has 32 loads in flight before it converts.  The arithmetic per
// block is the same as mxq_axis1_kernel's (same quant_block, zero padding past
// the last key).
//
// Output: column d's KBG blocks are one contiguous run of the codes
// ([m][d][kb] blocks), and the KBG key blocks' scales one contiguous range
// ([m][kb][32][4]).  A lane's own blocks lie in eight different runs, so the
// workgroup first places its blocks and scales in LDS in output order and
// then writes every run with consecutive lanes on consecutive 8- or 16-byte
// pieces (a few cache lines per store instruction instead of 16-32).  On the
// video V this and the EXACT form together take FP6 from 0.230 to 0.219 ms,
// FP8 from 0.249 to 0.232 and FP4 from 0.176 to 0.169; non-temporal stores of
// the runs are slower for FP6 and FP4 (2 % and 11 %).
constexpr int AX1_TB = 256;  // threads per workgroup
template <int ELEM, int COLS>
struct Ax1Stage {
  // columns per lane: 8 (16-byte loads); 4 columns per lane (more waves per
  // SIMD, half the registers) measured 3 % slower for FP6, 16 % for FP8
  static constexpr int CPL = 8;
  static constexpr int BB = Fmt<ELEM>::bits * 4;  // bytes per block
  static constexpr int LPB = COLS / CPL;           // lanes per key block
  static constexpr int KBW = 64 / LPB;             // key blocks per wave
  static constexpr int KBG = 4 * KBW;              // key blocks per workgroup
  static constexpr int RUN = KBG * BB;             // bytes of one column's run
  static constexpr int CH = (BB % 16 == 0) ? 16 : 8;  // output piece (divides BB; runs are CH-aligned)
  // LDS row pitch: the run plus one piece (the lanes of one key block write
  // rows 8 apart; the pad spreads them over several bank offsets)
  static constexpr int PITCH = RUN + CH;
  static constexpr int SC = KBG * 128;                // scale bytes of the workgroup
  static constexpr int LDS = COLS * PITCH + SC;
};
template <int ELEM, int COLS, bool EXACT>
__global__ void __launch_bounds__(AX1_TB) mxq_axis1_direct_kernel(const uint16_t* __restrict__ src, int64_t n_mat,
                                                                  int64_t rows, int64_t ld, int64_t nb,
                                                                  float prescale, bool fitmax,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
  using G = Ax1Stage<ELEM, COLS>;
  constexpr int BB = G::BB;
  __shared__ __align__(16) uint8_t stage[G::LDS];
  uint8_t* sscale = stage + COLS * G::PITCH;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t wgm = (nb + G::KBG - 1) / G::KBG;  // workgroups per matrix
  const int64_t m = blockIdx.x / wgm;
  const int64_t kb0 = (blockIdx.x - m * wgm) * G::KBG;
  const int kbl = wv * G::KBW + lane / G::LPB;  // the lane's key block within the workgroup
  const int64_t kb = kb0 + kbl;
  // the grid holds whole matrices only (m < n_mat); lanes past the last key
  // block convert nothing but still take part in the barrier
  if (kb < nb) {
    const int co = lane % G::LPB;
    const uint16_t* p = src + (m * rows + kb * 32) * ld + G::CPL * co;
    const int nrow = (int)min((int64_t)32, rows - kb * 32);
    // rows are read once: for the FP6/FP4 outputs, non-temporal loads (past
    // the caches) are faster on the video V (FP6 6 %, FP4 18 %); for FP8 they
    // are 4 % slower, and on the axis-0 kernel 40 % slower
    constexpr bool NT = Fmt<ELEM>::bits < 8;
    typedef unsigned vld __attribute__((ext_vector_type(G::CPL / 2)));
    vld r[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (j < nrow) {
        const vld* a = reinterpret_cast<const vld*>(p + (int64_t)j * ld);
        r[j] = NT ? __builtin_nontemporal_load(a) : *a;
      } else {
        r[j] = (vld)(0u);
      }
    }
#pragma unroll
    for (int e = 0; e < G::CPL; ++e) {
      float x[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t wd = r[j][e >> 1];
        const float f = bf16_to_f32((e & 1) ? (wd >> 16) : (wd & 0xFFFFu));
        x[j] = EXACT ? f : f * prescale;
      }
      uint32_t w[8];
      const uint32_t code = quant_block<ELEM>(x, fitmax, w, EXACT);
      const int d = G::CPL * co + e;
      uint2* q = reinterpret_cast<uint2*>(stage + d * G::PITCH + kbl * BB);
#pragma unroll
      for (int i = 0; i < BB / 8; ++i) q[i] = make_uint2(w[2 * i], w[2 * i + 1]);
      if constexpr (COLS == 128) sscale[kbl * 128 + (d & 31) * 4 + (d >> 5)] = (uint8_t)code;
      else scales[((m * nb + kb) * 32 + (d & 31)) * 4 + (d >> 5)] = (uint8_t)code;
    }
  }
  __syncthreads();
  // the runs: piece pc of column d lies in key block kb0 + (pc * CH) / BB (CH
  // divides BB), and is written when that key block exists
  const int nvalid = (int)min((int64_t)G::KBG, nb - kb0);
  constexpr int PPR = G::RUN / G::CH;  // pieces per run
  for (int c = threadIdx.x; c < COLS * PPR; c += AX1_TB) {
    const int d = c / PPR, pc = c - d * PPR;
    if ((pc * G::CH) / BB >= nvalid) continue;
    uint8_t* dst = codes + ((m * COLS + d) * nb + kb0) * BB + pc * G::CH;
    const uint8_t* sp = stage + d * G::PITCH + pc * G::CH;
    if constexpr (G::CH == 16) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(sp);
    else *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(sp);
  }
  if constexpr (COLS == 128) {
    // 128 scale bytes per key block, contiguous over the workgroup's blocks
    for (int c = threadIdx.x; c < nvalid * 8; c += AX1_TB)
      *reinterpret_cast<uint4*>(scales + (m * nb + kb0) * 128 + 16 * c) =
          *reinterpret_cast<const uint4*>(sscale + 16 * c);
  }
}

template <int ELEM>
static hipError_t launch_elem(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                              int axis, float prescale, bool fitmax, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  const int TB = 256;
  if (axis == 0) {
    int64_t nb = cols / 32, total = n_mat * rows * nb;
    dim3 grid((unsigned)((total + TB - 1) / TB));
    bool vec = (ld % 8 == 0) && ((reinterpret_cast<uintptr_t>(src) & 15) == 0);
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(TB), 0, stream, src, n_mat * rows, nb, ld, prescale, fitmax, codes, scales);
    };
    if (vec) {
      if (prescale == 1.0f) go(mxq_axis0_kernel<ELEM, true, true>);
      else go(mxq_axis0_kernel<ELEM, true, false>);
    } else {
      if (prescale == 1.0f) go(mxq_axis0_kernel<ELEM, false, true>);
      else go(mxq_axis0_kernel<ELEM, false, false>);
    }
  } else {
    int64_t nb = (rows + 31) / 32, total = n_mat * nb * cols;
    const bool direct = (cols == 64 || cols == 128) && (ld % 8 == 0) &&
                        ((reinterpret_cast<uintptr_t>(src) & 15) == 0) &&
                        ((reinterpret_cast<uintptr_t>(scales) & 15) == 0);
    if (direct) {
      const int kbg = 4 * (64 / (int)(cols / 8));  // key blocks per workgroup
      dim3 grid((unsigned)(n_mat * ((nb + kbg - 1) / kbg)));
      auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(AX1_TB), 0, stream, src, n_mat, rows, ld, nb, prescale, fitmax, codes,
                           scales);
      };
      const bool ex = prescale == 1.0f;
      if (cols == 128) {
        if (ex) go(mxq_axis1_direct_kernel<ELEM, 128, true>);
        else go(mxq_axis1_direct_kernel<ELEM, 128, false>);
      } else {
        if (ex) go(mxq_axis1_direct_kernel<ELEM, 64, true>);
        else go(mxq_axis1_direct_kernel<ELEM, 64, false>);
      }
    } else {
      dim3 grid((unsigned)((total + TB - 1) / TB));
      hipLaunchKernelGGL((mxq_axis1_kernel<ELEM>), grid, dim3(TB), 0, stream, src, n_mat, rows, cols, ld, nb,
                         prescale, fitmax, codes, scales);
    }
  }
  return hipGetLastError();
}

template <int ELEM>
static hipError_t launch_rms_elem(const uint16_t* src, int64_t nrows, int64_t cols, int64_t ld, const float* weight,
                                  float eps, float prescale, bool fitmax, uint8_t* codes, uint8_t* scales,
                                  hipStream_t stream) {
  const int TB = 256;
  const int nb = (int)(cols / 32);
  const int64_t total = nrows * nb;
  dim3 grid((unsigned)((total + TB - 1) / TB));
  // 16-byte loads when every row start and the weight are 16-byte aligned
  const bool vec = (ld % 8 == 0) && ((reinterpret_cast<uintptr_t>(src) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(weight) & 15) == 0);
  if (vec)
    hipLaunchKernelGGL((mxq_rms_kernel<ELEM, true>), grid, dim3(TB), 0, stream, src, nrows, nb, ld, weight, eps,
                       prescale, fitmax, codes, scales);
  else
    hipLaunchKernelGGL((mxq_rms_kernel<ELEM, false>), grid, dim3(TB), 0, stream, src, nrows, nb, ld, weight, eps,
                       prescale, fitmax, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mx_rmsnorm(const uint16_t* src, int64_t nrows, int64_t cols, int64_t ld,
                                      const float* weight, float eps, float prescale, int elem, bool fitmax,
                                      uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  switch (elem) {
    case E4M3: return launch_rms_elem<E4M3>(src, nrows, cols, ld, weight, eps, prescale, fitmax, codes, scales, stream);
    case E5M2: return launch_rms_elem<E5M2>(src, nrows, cols, ld, weight, eps, prescale, fitmax, codes, scales, stream);
    case E2M3: return launch_rms_elem<E2M3>(src, nrows, cols, ld, weight, eps, prescale, fitmax, codes, scales, stream);
    case E3M2: return launch_rms_elem<E3M2>(src, nrows, cols, ld, weight, eps, prescale, fitmax, codes, scales, stream);
    case E2M1: return launch_rms_elem<E2M1>(src, nrows, cols, ld, weight, eps, prescale, fitmax, codes, scales, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_mx(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld, int axis,
                              float prescale, int elem, bool fitmax, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream) {
  switch (elem) {
    case E4M3: return launch_elem<E4M3>(src, n_mat, rows, cols, ld, axis, prescale, fitmax, codes, scales, stream);
    case E5M2: return launch_elem<E5M2>(src, n_mat, rows, cols, ld, axis, prescale, fitmax, codes, scales, stream);
    case E2M3: return launch_elem<E2M3>(src, n_mat, rows, cols, ld, axis, prescale, fitmax, codes, scales, stream);
    case E3M2: return launch_elem<E3M2>(src, n_mat, rows, cols, ld, axis, prescale, fitmax, codes, scales, stream);
    case E2M1: return launch_elem<E2M1>(src, n_mat, rows, cols, ld, axis, prescale, fitmax, codes, scales, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fsattn
