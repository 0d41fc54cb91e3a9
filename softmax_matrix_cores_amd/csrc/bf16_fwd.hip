// bf16_fwd.hip -- conventional BF16 attention forward (the baseline).
//
// The pages compare the quantized kernels against BF16 attention ("Fused-
// Softmax shifts an AI attention bottleneck onto faster GPU hardware",
// paragraph 8) and describe the conventional scheme as repeatedly updating a
// reference maximum and rescaling the accumulated results when it grows
// (paragraph 5).  This kernel is that scheme, FlashAttention style:
//   per 64-key tile: s = q.k (BF16 MFMA, fp32 accumulate), running max m,
//   p = exp2(s*sigma*log2e - m'), O and l rescaled by exp2(m_old - m_new),
//   O += bf16(p) V (BF16 MFMA), l += sum p; finally O / l.
//
// Layout (v_mfma_f32_16x16x32_bf16: lane (r = l%16, g = l/16) holds row r,
// K elements [8g, 8g+8); accumulator lane (n, g) holds rows 4g..4g+3 of
// column n).  Scores are computed transposed, S^T = K Q^T, with the K rows of
// each MFMA permuted so that lane (n, g) receives keys 8g..8g+7 of every
// 32-key chunk for query n -- exactly its A operand of the PV product.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace fsattn {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f_b __attribute__((ext_vector_type(4)));

constexpr int BNW = 4;   // waves
constexpr int BQW = 16;  // queries per wave
constexpr int BKT = 64;  // keys per tile

__device__ __forceinline__ v8bf ld8(const uint16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(v8bf, u);
}

template <int D>
__global__ void __launch_bounds__(BNW * 64) bf16_fwd_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
                                                             int H, int Sq, int Skv, float c_log2) {
  constexpr int KP = D + 8;     // padded K row (elements) in LDS
  constexpr int VP = BKT + 8;   // padded V^T row (elements) in LDS
  __shared__ __attribute__((aligned(16))) uint16_t ldsK[BKT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t ldsVt[D * VP];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.y + blockIdx.z * H;
  const int q0 = blockIdx.x * (BNW * BQW) + w * BQW;
  const uint16_t* kb = k + (size_t)bh * Skv * D;
  const uint16_t* vb = v + (size_t)bh * Skv * D;

  // Q^T operands (B of S^T): lane (n, g), chunk c: Q[q0+n][32c + 8g .. +8]
  const int qrow = min(q0 + n, Sq - 1);
  v8bf qB[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qB[c] = ld8(q + ((size_t)bh * Sq + qrow) * D + 32 * c + 8 * g);

  v4f_b O[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) O[i] = v4f_b{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max (scaled, log2 units) of query n
  float lpart = 0.0f;   // this lane's partial row sum

  const int ntiles = (Skv + BKT - 1) / BKT;
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BKT;
    const int nk = min(BKT, Skv - k0);
    __syncthreads();
    // stage K rows (zero beyond nk) and V transposed
    for (int i = tid; i < BKT * D / 8; i += BNW * 64) {
      const int key = i / (D / 8), c8 = i - key * (D / 8);
      uint4 u = make_uint4(0, 0, 0, 0);
      uint4 uv = make_uint4(0, 0, 0, 0);
      if (key < nk) {
        u = *reinterpret_cast<const uint4*>(kb + (size_t)(k0 + key) * D + 8 * c8);
        uv = *reinterpret_cast<const uint4*>(vb + (size_t)(k0 + key) * D + 8 * c8);
      }
      *reinterpret_cast<uint4*>(ldsK + key * KP + 8 * c8) = u;
      const uint32_t vv[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ldsVt[(8 * c8 + 2 * e) * VP + key] = (uint16_t)(vv[e] & 0xFFFFu);
        ldsVt[(8 * c8 + 2 * e + 1) * VP + key] = (uint16_t)(vv[e] >> 16);
      }
    }
    __syncthreads();

    // S^T blocks j = 0..3 (16 keys each); block j, A row r -> key 32(j/2) + 8(r/4) + 4(j%2) + r%4
    v4f_b s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = lane & 15;
      const int key = 32 * (j >> 1) + 8 * (r >> 2) + 4 * (j & 1) + (r & 3);
      v4f_b acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        v8bf a = ld8(ldsK + key * KP + 32 * c + 8 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[c], acc, 0, 0, 0);
      }
      s[j] = acc;
    }
    // lane (n, g) now holds query n, keys 32(j/2) + 8g + 4(j%2) + r'
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 32 * (j >> 1) + 8 * g + 4 * (j & 1) + r;
        float x = (key < nk) ? s[j][r] * c_log2 : -INFINITY;
        s[j][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(m, tmax);
    const float alpha = exp2f(m - mnew);  // m = -inf on the first tile -> 0
    m = mnew;
    float psum = 0.0f;
    v8bf pA[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(s[2 * cc + h][r] - mnew);
          psum += p;
          pA[cc][4 * h + r] = (__bf16)p;
        }
    lpart = lpart * alpha + psum;
    // rescale O rows (queries 4g + r): alpha of query q lives in lanes with n = q
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) O[i][r] *= ar[r];
    // O += P V: chunk cc, d block i: B lane (n, g) = V^T[16i + n][32cc + 8g .. +8]
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        v8bf b = ld8(ldsVt + (16 * i + n) * VP + 32 * cc + 8 * g);
        O[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pA[cc], b, O[i], 0, 0, 0);
      }
  }
  // l of query n = sum over the 4 lanes of the query
  float l = lpart + __shfl_xor(lpart, 16, 64);
  l += __shfl_xor(l, 32, 64);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qq = q0 + 4 * g + r;
    const float lq = __shfl(l, 4 * g + r, 64);
    if (qq < Sq) {
      const float inv = 1.0f / lq;
      uint16_t* orow = out + ((size_t)bh * Sq + qq) * D;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        __bf16 b = (__bf16)(O[i][r] * inv);
        orow[16 * i + n] = __builtin_bit_cast(uint16_t, b);
      }
    }
  }
}

hipError_t launch_bf16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int B, int H,
                           int Sq, int Skv, int D, float softmax_scale, hipStream_t stream) {
  const float c_log2 = softmax_scale * 1.4426950408889634f;
  dim3 grid((unsigned)((Sq + BNW * BQW - 1) / (BNW * BQW)), (unsigned)H, (unsigned)B);
  if (D == 128)
    hipLaunchKernelGGL(bf16_fwd_kernel<128>, grid, dim3(BNW * 64), 0, stream, q, k, v, out, H, Sq, Skv, c_log2);
  else
    hipLaunchKernelGGL(bf16_fwd_kernel<64>, grid, dim3(BNW * 64), 0, stream, q, k, v, out, H, Sq, Skv, c_log2);
  return hipGetLastError();
}

}  // namespace fsattn
