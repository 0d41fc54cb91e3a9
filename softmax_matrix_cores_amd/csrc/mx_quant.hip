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

// Round-to-nearest-even of y (already divided by the block scale) into a
// 6-bit format (E2M3 or E3M2), saturating at the largest value, sign kept.
// The quantum of y's binade is a power of two, so y * 2^-quantum is exact and
// v_rndne_f32 performs the one rounding.
template <int ELEM>
__device__ __forceinline__ uint32_t sw_encode6(float y) {
  constexpr int MB = (ELEM == E2M3) ? 3 : 2;          // mantissa bits
  constexpr int BIAS = (ELEM == E2M3) ? 1 : 3;
  constexpr int EMIN = 1 - BIAS;                      // exponent of the smallest normal
  const uint32_t sign = __float_as_uint(y) >> 31;
  float a = fminf(fabsf(y), Fmt<ELEM>::maxnorm);
  int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  e = max(e, EMIN);
  const float scale = __uint_as_float((uint32_t)(MB - e + 127) << 23);  // 2^(MB - e)
  uint32_t n = (uint32_t)__builtin_rintf(a * scale);                    // 0 .. 2^(MB+1)
  uint32_t mag;
  if (e == EMIN && n < (1u << MB)) {
    mag = n;  // subnormal
  } else {
    if (n == (2u << MB)) { e += 1; n = 1u << MB; }
    mag = ((uint32_t)(e + BIAS) << MB) | (n - (1u << MB));
  }
  return (sign << 5) | mag;
}

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
    if (bf16_exact) {
      // the values are exact bf16 (no prescale): hardware bf16 -> FP6 converter
      v32bf v;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(x[i]) >> 16));
      v6i r;
      if constexpr (ELEM == E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, X);
      else r = __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(v, X);
#pragma unroll
      for (int i = 0; i < 6; ++i) w[i] = (uint32_t)r[i];
    } else {
      // fp32 values: exact software round-to-nearest-even into the 6-bit grid
      const float inv = 1.0f / X;  // exact: X is a power of two (2^-127 .. 2^127)
#pragma unroll
      for (int i = 0; i < 6; ++i) w[i] = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        uint32_t c = sw_encode6<ELEM>(x[j] * inv);
        const int pos = 6 * j;
        w[pos >> 5] |= c << (pos & 31);
        if ((pos & 31) > 26) w[(pos >> 5) + 1] |= c >> (32 - (pos & 31));
      }
    }
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
template <int ELEM, bool VEC>
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
        x[8 * i + 2 * j] = bf16_to_f32(uu[j] & 0xFFFFu) * prescale;
        x[8 * i + 2 * j + 1] = bf16_to_f32(uu[j] >> 16) * prescale;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = bf16_to_f32(p[i]) * prescale;
  }
  uint32_t w[8];
  uint32_t code = quant_block<ELEM>(x, fitmax, w, prescale == 1.0f);
  store_block<BB>(codes + blk * BB, w);
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

// axis 1, tiled (cols 64 or 128, 16-byte rows): a workgroup quantizes keys
// [128 t, 128 t + 128) of every column of matrix m.  The bf16 tile (32 KiB at
// most, so four workgroups share a CU's LDS) comes in with 16-byte coalesced
// loads; in LDS each 16-byte chunk of row r sits rotated by 16 ((r / 32) % 4)
// columns (mod cols), so that the column reads below (lanes = 4 key blocks x
// 16 columns) hit 32 distinct banks.  Each thread
// then quantizes (column, 32-key block) units with the key block fastest, so
// neighbouring threads write neighbouring blocks of one column: the packed
// codes leave as contiguous runs.  The arithmetic per block is the same as
// mxq_axis1_kernel's (same quant_block, zero padding past the last key).
constexpr int AX1_KT = 128;  // keys per tile
template <int ELEM, int COLS>
__global__ void __launch_bounds__(256) mxq_axis1_tiled_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                              int64_t ld, int64_t nb, float prescale, bool fitmax,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  constexpr int BB = Fmt<ELEM>::bits * 4;
  constexpr int NBT = AX1_KT / 32;  // key blocks per tile
  constexpr int CPR = COLS / 8;     // 16-byte chunks per row
  constexpr int ROT = 64 / NBT;     // rotation step (columns) per key block
  __shared__ __attribute__((aligned(16))) uint16_t tile[AX1_KT * COLS];
  const int64_t m = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * AX1_KT;
  const int rows_t = (int)min((int64_t)AX1_KT, rows - r0);  // >= 1
  const uint16_t* base = src + (m * rows + r0) * ld;
  for (int c = threadIdx.x; c < AX1_KT * CPR; c += 256) {
    const int r = c / CPR, q = c - r * CPR;
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows_t) u = *reinterpret_cast<const uint4*>(base + (int64_t)r * ld + 8 * q);
    const int col = (8 * q + ROT * ((r >> 5) & (NBT - 1))) & (COLS - 1);
    *reinterpret_cast<uint4*>(tile + r * COLS + col) = u;
  }
  __syncthreads();
  const int nbt = (rows_t + 31) / 32;
  for (int u = threadIdx.x; u < NBT * COLS; u += 256) {
    const int kb = u % NBT, d = u / NBT;
    if (kb >= nbt) continue;
    const int col = (d + ROT * kb) & (COLS - 1);
    float x[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int r = kb * 32 + j;
      x[j] = (r < rows_t) ? bf16_to_f32(tile[r * COLS + col]) * prescale : 0.0f;
    }
    uint32_t w[8];
    const uint32_t code = quant_block<ELEM>(x, fitmax, w, prescale == 1.0f);
    const int64_t kbg = (int64_t)blockIdx.x * NBT + kb;
    const int64_t o = (m * COLS + d) * nb + kbg;
    store_block<BB>(codes + o * BB, w);
    scales[((m * nb + kbg) * 32 + (d & 31)) * 4 + (d >> 5)] = (uint8_t)code;
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
    if (vec)
      hipLaunchKernelGGL((mxq_axis0_kernel<ELEM, true>), grid, dim3(TB), 0, stream, src, n_mat * rows, nb, ld,
                         prescale, fitmax, codes, scales);
    else
      hipLaunchKernelGGL((mxq_axis0_kernel<ELEM, false>), grid, dim3(TB), 0, stream, src, n_mat * rows, nb, ld,
                         prescale, fitmax, codes, scales);
  } else {
    int64_t nb = (rows + 31) / 32, total = n_mat * nb * cols;
    const bool tiled = (cols == 64 || cols == 128) && (ld % 8 == 0) &&
                       ((reinterpret_cast<uintptr_t>(src) & 15) == 0) && n_mat <= 65535;
    if (tiled) {
      dim3 grid((unsigned)((rows + AX1_KT - 1) / AX1_KT), (unsigned)n_mat);
      if (cols == 128)
        hipLaunchKernelGGL((mxq_axis1_tiled_kernel<ELEM, 128>), grid, dim3(TB), 0, stream, src, rows, ld, nb,
                           prescale, fitmax, codes, scales);
      else
        hipLaunchKernelGGL((mxq_axis1_tiled_kernel<ELEM, 64>), grid, dim3(TB), 0, stream, src, rows, ld, nb,
                           prescale, fitmax, codes, scales);
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
