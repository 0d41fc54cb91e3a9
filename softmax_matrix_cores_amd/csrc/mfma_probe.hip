// mfma_probe.hip -- measurement helper: the matrix-core rate and the shader
// clock of gfx950 under a pure matrix-product load.  The benchmark reports
// the fused kernel's utilisation against the MX peak of the datasheet and
// also against what this kernel reaches on the same box, at the clock it
// observes (the chip lowers its clock under sustained matrix-core load).
//
// Each wave issues `iters` rounds of four independent scaled 32x32x64
// products (four accumulator chains, so no product waits for the previous
// one), or for BF16 four times as many 32x32x16 products (the same work);
// eight waves per workgroup, two per SIMD, like the fused kernel.
// Wave 0 of each workgroup records the shader-clock counter (s_memtime) and
// the constant-rate counter (s_memrealtime) before and after its loop.
#include "fsattn.h"
#include "internal.h"
#include "mx_device.h"

namespace fsattn {
namespace {

constexpr int PROBE_BF16 = 16;
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int F>
__global__ void __launch_bounds__(512, 1) mfma_probe_kernel(int64_t iters, unsigned long long* stamps) {
  const int lane = threadIdx.x & 63;
  v8i a = {lane, lane + 1, lane + 2, lane + 3, lane + 4, lane + 5, lane + 6, lane + 7};
  v8i b = {lane ^ 5, lane ^ 6, lane ^ 7, lane ^ 8, lane ^ 9, lane ^ 10, lane ^ 11, lane ^ 12};
  if constexpr (F == E2M3) {
    a[6] = a[7] = b[6] = b[7] = 0;
  } else if constexpr (F == E2M1) {
    a[4] = a[5] = a[6] = a[7] = b[4] = b[5] = b[6] = b[7] = 0;
  }
  v16f c0, c1, c2, c3;
#pragma unroll
  for (int k = 0; k < 16; ++k) c0[k] = c1[k] = c2[k] = c3[k] = 0.0f;
  __syncthreads();
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int64_t i = 0; i < iters; ++i) {
    if constexpr (F == PROBE_BF16) {
      // 32x32x16 BF16 products (the baseline's instruction), four per chain
      // and round so that a round does the work of one 32x32x64 product
      const v8bf ab = __builtin_bit_cast(v8bf, v4i{a[0], a[1], a[2], a[3]});
      const v8bf bb = __builtin_bit_cast(v8bf, v4i{b[0], b[1], b[2], b[3]});
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, c3, 0, 0, 0);
      }
    } else {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, F, F, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, F, F, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, F, F, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, F, F, 0, 127, 0, 127);
    }
  }
  // the results are consumed so that the products are not removed: a NaN
  // (which these finite codes cannot produce) would zero the first stamp
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    unsigned long long* st = stamps + 4 * (size_t)blockIdx.x;
    st[0] = (s != s) ? 0ull : t0;
    st[1] = t1;
    st[2] = r0;
    st[3] = r1;
  }
}

}  // namespace

hipError_t launch_mfma_probe(int elem, int64_t iters, int wgs, unsigned long long* stamps, hipStream_t stream) {
  const dim3 grid((unsigned)wgs), block(512);
  switch (elem) {
    case E4M3: hipLaunchKernelGGL(mfma_probe_kernel<E4M3>, grid, block, 0, stream, iters, stamps); break;
    case E2M3: hipLaunchKernelGGL(mfma_probe_kernel<E2M3>, grid, block, 0, stream, iters, stamps); break;
    case E2M1: hipLaunchKernelGGL(mfma_probe_kernel<E2M1>, grid, block, 0, stream, iters, stamps); break;
    case PROBE_BF16:
      hipLaunchKernelGGL(mfma_probe_kernel<PROBE_BF16>, grid, block, 0, stream, iters, stamps);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fsattn
