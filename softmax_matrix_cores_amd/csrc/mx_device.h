// mx_device.h -- gfx950 device helpers for the MX formats (GPU side only).
//
// MX = OCP Microscaling v1.0: blocks of 32 element codes sharing one E8M0
// scale 2^(s-127).  The pages name the MXFP8 / MXFP6 / MXFP4 configurations
// ("Fused-Softmax shifts an AI attention bottleneck onto faster GPU
// hardware", paragraphs 7-8).
//
// Element conversion uses the CDNA4 scaled converters
// (v_cvt_scalef32_pk_fp8_*, v_cvt_scalef32_pk32_fp6_bf16,
// v_cvt_scalef32_2xpk16_fp6_f32, v_cvt_scalef32_pk_fp4_*).  With a
// power-of-two scale X they return round-to-nearest-even of x / X, keep the
// sign of zero and the subnormals, and saturate FP6/FP4; FP8 overflow gives
// NaN, so callers clamp where overflow is possible (OCP-floor rule only:
// under the fit-max rule no element exceeds the largest value).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsattn {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v16u __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v32bf __attribute__((ext_vector_type(32)));

enum Elem { E4M3 = 0, E5M2 = 1, E2M3 = 2, E3M2 = 3, E2M1 = 4 };

template <int ELEM> struct Fmt;
// emax: exponent of the largest normal; mthr23: fp32 mantissa field of the
// largest normal's significand (m_max - 1) * 2^23; maxnorm: largest value.
template <> struct Fmt<E4M3> { static constexpr int bits = 8, emax = 8; static constexpr uint32_t mthr23 = 0x600000u; static constexpr float maxnorm = 448.0f; };
template <> struct Fmt<E5M2> { static constexpr int bits = 8, emax = 15; static constexpr uint32_t mthr23 = 0x600000u; static constexpr float maxnorm = 57344.0f; };
template <> struct Fmt<E2M3> { static constexpr int bits = 6, emax = 2; static constexpr uint32_t mthr23 = 0x700000u; static constexpr float maxnorm = 7.5f; };
template <> struct Fmt<E3M2> { static constexpr int bits = 6, emax = 4; static constexpr uint32_t mthr23 = 0x600000u; static constexpr float maxnorm = 28.0f; };
template <> struct Fmt<E2M1> { static constexpr int bits = 4, emax = 2; static constexpr uint32_t mthr23 = 0x400000u; static constexpr float maxnorm = 6.0f; };

// E8M0 code for a block whose largest magnitude has fp32 bit pattern `abits`
// (sign cleared).  Fit-max: ceil(log2(amax / maxnorm)) + 127; OCP floor:
// floor(log2 amax) - emax + 127; clamped to [0, 254]; amax = 0 -> 0;
// NaN/Inf -> 255.  An fp32-subnormal amax always clamps to 0.
template <int ELEM>
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t abits, bool fitmax) {
  uint32_t E = abits >> 23;
  if (E == 255u) return 255u;
  if (E == 0u) return 0u;
  int k = (int)E - Fmt<ELEM>::emax + ((fitmax && (abits & 0x7FFFFFu) > Fmt<ELEM>::mthr23) ? 1 : 0);
  return (uint32_t)min(max(k, 0), 254);
}

// 2^(code-127) as fp32 (code 0 -> the subnormal 2^-127)
__device__ __forceinline__ float e8m0_to_float(uint32_t code) {
  return __uint_as_float(code == 0u ? 0x00400000u : (code << 23));
}

}  // namespace fsattn
