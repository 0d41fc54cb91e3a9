// internal.h -- declarations shared by the library's translation units
// (kernel launchers and their argument block).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsattn {

struct FwdArgs {
  const uint8_t* qc;  // [BH][Sq][D/32][block bytes]
  const uint8_t* qs;  // [BH][Sq][D/32]
  const uint8_t* kc;  // [BH][Skv][D/32][block bytes]
  const uint8_t* ks;  // [BH][Skv][D/32]
  const uint8_t* vc;  // [BH][D][nb32][block bytes]
  const uint8_t* vs;  // [BH][D][nb32]
  uint16_t* out;      // [BH][Sq][D] bf16
  int32_t* counts;    // [BH][Sq] or null
  uint8_t* pd_codes;  // P dump window or null
  uint8_t* pd_scales;
  int H, Sq, Skv, nb32;
  int pd_bh, pd_row0, pd_row1;
  float T0, Tg;  // fl32(128*127 - c), fl32(128*(127+tau) - c)
  int kv128;     // gate tile = 128 keys (else 64)
  int fitmax;
  int causal;              // query i sees keys k <= i + kv_len - q_len
  const int32_t* q_lens;   // [B] valid queries per batch, or null (Sq)
  const int32_t* kv_lens;  // [B] valid keys per batch, or null (Skv)
  float efq_a, efq_t128;   // E2M1 (EFQ-style) P: 1 / (128 h) rounded up, 128 tau
  int fp8_products;        // E4M3 Q/K: score products on the FP8 matrix core (else decoded to BF16)
};

hipError_t launch_quantize_mx(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld, int axis,
                              float prescale, int elem, bool fitmax, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);
hipError_t launch_quantize_mx_rmsnorm(const uint16_t* src, int64_t nrows, int64_t cols, int64_t ld,
                                      const float* weight, float eps, float prescale, int elem, bool fitmax,
                                      uint8_t* codes, uint8_t* scales, hipStream_t stream);
bool fwd_supported(int qk, int ve, int pe);
hipError_t launch_fsattn_fwd(const FwdArgs& a, int B, int D, int qk, int ve, int pe, hipStream_t s);
hipError_t launch_mfma_probe(int elem, int64_t iters, int wgs, unsigned long long* stamps, hipStream_t stream);
hipError_t launch_bf16_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int B, int H,
                           int Sq, int Skv, int D, float softmax_scale, int causal, const int32_t* q_lens,
                           const int32_t* kv_lens, hipStream_t stream);

}  // namespace fsattn
