// fsattn_api.hip -- the extern "C" boundary declared in include/fsattn.h:
// argument validation (before any launch), size helpers, status strings and
// kernel launches on the caller's stream.  No allocation, no global state.
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "fsattn.h"

#include "internal.h"

namespace {

int elem_bits(int e) {
  switch (e) {
    case FSATTN_E4M3:
    case FSATTN_E5M2: return 8;
    case FSATTN_E2M3:
    case FSATTN_E3M2: return 6;
    case FSATTN_E2M1: return 4;
    default: return 0;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t nblocks(int64_t n_mat, int64_t rows, int64_t cols, int axis) {
  if (axis == 0) return n_mat * rows * (cols / 32);
  return n_mat * cols * ((rows + 31) / 32);
}

// fl32(128 * log2(e) * sigma): the multiplicative part of the fold
float fold_prescale(float sigma) { return (float)(128.0 * 1.4426950408889634 * (double)sigma); }

// FP6 formats of P the two-stage conversion produces
bool six_bit(int e) { return e == FSATTN_E2M3 || e == FSATTN_E3M2; }

bool within_ulps(float a, float b, int ulps) {
  int32_t ia, ib;
  __builtin_memcpy(&ia, &a, 4);
  __builtin_memcpy(&ib, &b, 4);
  if ((ia < 0) != (ib < 0)) return a == b;
  int64_t d = (int64_t)ia - (int64_t)ib;
  return d <= ulps && d >= -ulps;
}

}  // namespace

extern "C" {

int fsattn_abi_version(void) { return FSATTN_ABI_VERSION; }

float fsattn_fold_prescale(float softmax_scale) {
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return NAN;
  return fold_prescale(softmax_scale);
}

const char* fsattn_status_str(int s) {
  switch (s) {
    case FSATTN_OK: return "ok";
    case FSATTN_E_INVALID_ARG: return "invalid argument";
    case FSATTN_E_UNSUPPORTED: return "unsupported format combination or size";
    case FSATTN_E_ALIGNMENT: return "pointer not aligned (16 bytes for codes and bf16 tensors)";
    case FSATTN_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int64_t fsattn_mx_codes_bytes(int elem, int64_t n_mat, int64_t rows, int64_t cols, int block_axis) {
  const int bits = elem_bits(elem);
  if (!bits || n_mat < 0 || rows < 0 || cols < 0 || (block_axis != 0 && block_axis != 1)) return -1;
  if (block_axis == 0 && cols % 32) return -1;
  return nblocks(n_mat, rows, cols, block_axis) * bits * 4;
}

int64_t fsattn_mx_scales_bytes(int64_t n_mat, int64_t rows, int64_t cols, int block_axis) {
  if (n_mat < 0 || rows < 0 || cols < 0 || (block_axis != 0 && block_axis != 1)) return -1;
  if (block_axis == 0 && cols % 32) return -1;
  if (block_axis == 1) {
    if (cols > 128) return -1;
    return n_mat * ((rows + 31) / 32) * 128;  // [n_mat][blocks][32][4], see the header
  }
  return (nblocks(n_mat, rows, cols, block_axis) + 3) & ~(int64_t)3;  // padded to whole dwords
}

int fsattn_quantize_mx(const void* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld, int block_axis,
                       float prescale, int elem, int rule, void* codes_out, uint8_t* scales_out, void* stream) {
  if (!elem_bits(elem) || (rule != FSATTN_SCALE_FITMAX && rule != FSATTN_SCALE_OCP_FLOOR)) return FSATTN_E_INVALID_ARG;
  if (block_axis != 0 && block_axis != 1) return FSATTN_E_INVALID_ARG;
  if (n_mat < 0 || rows < 0 || cols < 0 || ld < cols) return FSATTN_E_INVALID_ARG;
  if (block_axis == 0 && cols % 32) return FSATTN_E_INVALID_ARG;
  if (block_axis == 1 && cols > 128) return FSATTN_E_INVALID_ARG;
  if (!isfinite(prescale)) return FSATTN_E_INVALID_ARG;
  if (n_mat == 0 || rows == 0 || cols == 0) return FSATTN_OK;
  if (!src || !codes_out || !scales_out) return FSATTN_E_INVALID_ARG;
  if (!aligned(src, 2) || !aligned(codes_out, 16)) return FSATTN_E_ALIGNMENT;
  if (nblocks(n_mat, rows, cols, block_axis) > ((int64_t)1 << 40)) return FSATTN_E_UNSUPPORTED;
  hipError_t e = fsattn::launch_quantize_mx(static_cast<const uint16_t*>(src), n_mat, rows, cols, ld, block_axis,
                                            prescale, elem, rule == FSATTN_SCALE_FITMAX,
                                            static_cast<uint8_t*>(codes_out), scales_out,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_E_HIP;
}

int fsattn_quantize_mx_rmsnorm(const void* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                               const float* weight, float eps, float prescale, int elem, int rule, void* codes_out,
                               uint8_t* scales_out, void* stream) {
  if (!elem_bits(elem) || (rule != FSATTN_SCALE_FITMAX && rule != FSATTN_SCALE_OCP_FLOOR)) return FSATTN_E_INVALID_ARG;
  if (n_mat < 0 || rows < 0 || cols < 0 || ld < cols) return FSATTN_E_INVALID_ARG;
  if (cols % 32) return FSATTN_E_INVALID_ARG;
  if (!isfinite(prescale) || !(eps >= 0.0f) || !isfinite(eps)) return FSATTN_E_INVALID_ARG;
  // a row's blocks are the consecutive lanes of one wave
  if (cols > 2048 || (cols & (cols - 1)) != 0) return FSATTN_E_UNSUPPORTED;
  if (n_mat == 0 || rows == 0 || cols == 0) return FSATTN_OK;
  if (!src || !codes_out || !scales_out) return FSATTN_E_INVALID_ARG;
  if (!aligned(src, 2) || !aligned(codes_out, 16) || !aligned(weight, 4)) return FSATTN_E_ALIGNMENT;
  if (nblocks(n_mat, rows, cols, 0) > ((int64_t)1 << 40)) return FSATTN_E_UNSUPPORTED;
  hipError_t e = fsattn::launch_quantize_mx_rmsnorm(static_cast<const uint16_t*>(src), n_mat * rows, cols, ld, weight,
                                                    eps, prescale, elem, rule == FSATTN_SCALE_FITMAX,
                                                    static_cast<uint8_t*>(codes_out), scales_out,
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_E_HIP;
}

// the forward of every entry point; efq: E2M1 P by the EFQ-style rule with
// (efq_tau, efq_h), else E2M1 P is refused (the two-stage path has no FP4 P);
// fp8_products: E4M3 Q/K scores on the FP8 matrix core (else from operands
// decoded to BF16)
static int forward_impl(const fsattn_params* p, const fsattn_mask* mask, bool efq, float efq_tau, float efq_h,
                        bool fp8_products, const fsattn_mx_tensor* q, const fsattn_mx_tensor* k,
                        const fsattn_mx_tensor* v, void* out, void* stream) {
  if (!p || !q || !k || !v) return FSATTN_E_INVALID_ARG;
  if (efq) {
    if (p->p_elem != FSATTN_E2M1) return FSATTN_E_INVALID_ARG;
    if (!(efq_h >= 1.0f / 64.0f && efq_h <= 16.0f) || !(efq_tau >= -64.0f && efq_tau <= 64.0f))
      return FSATTN_E_INVALID_ARG;
  } else if (p->p_elem == FSATTN_E2M1) {
    return FSATTN_E_UNSUPPORTED;
  }
  if (mask) {
    if (mask->causal != 0 && mask->causal != 1) return FSATTN_E_INVALID_ARG;
    if (!aligned(mask->q_lens, 4) || !aligned(mask->kv_lens, 4)) return FSATTN_E_ALIGNMENT;
  }
  if (p->B < 0 || p->H < 0 || p->Sq < 0 || p->Skv < 1) return FSATTN_E_INVALID_ARG;
  if (p->D != 64 && p->D != 128) return FSATTN_E_INVALID_ARG;
  if (p->kv_tile < 32 || p->kv_tile % 32) return FSATTN_E_INVALID_ARG;
  if (p->p_scale_rule != FSATTN_SCALE_FITMAX && p->p_scale_rule != FSATTN_SCALE_OCP_FLOOR) return FSATTN_E_INVALID_ARG;
  if (!(p->tau >= 0.0f) || !isfinite(p->tau) || !isfinite(p->schraudolph_c)) return FSATTN_E_INVALID_ARG;
  if (!(p->softmax_scale > 0.0f) || !isfinite(p->softmax_scale)) return FSATTN_E_INVALID_ARG;
  if (!elem_bits(q->elem) || !elem_bits(v->elem) || !elem_bits(p->p_elem)) return FSATTN_E_INVALID_ARG;
  if (q->elem != k->elem) return FSATTN_E_INVALID_ARG;
  if (!within_ulps(q->prescale, fold_prescale(p->softmax_scale), 2)) return FSATTN_E_INVALID_ARG;
  if (k->prescale != 1.0f || v->prescale != 1.0f) return FSATTN_E_INVALID_ARG;
  if (!fsattn::fwd_supported(q->elem, v->elem, p->p_elem)) return FSATTN_E_UNSUPPORTED;
  // the kernels run 64- and 128-key gate tiles and the fit-max rule for P
  if (p->kv_tile != 64 && p->kv_tile != 128) return FSATTN_E_UNSUPPORTED;
  if (p->p_scale_rule != FSATTN_SCALE_FITMAX) return FSATTN_E_UNSUPPORTED;
  if (p->H > 65535 || p->B > 65535) return FSATTN_E_UNSUPPORTED;
  if (p->p_dump_codes) {
    if (!p->p_dump_scales || p->p_b < 0 || p->p_b >= p->B || p->p_h < 0 || p->p_h >= p->H || p->p_row0 < 0 ||
        p->p_row1 <= p->p_row0 || p->p_row1 > p->Sq)
      return FSATTN_E_INVALID_ARG;
  }
  if (p->B == 0 || p->H == 0 || p->Sq == 0) return FSATTN_OK;
  if (!q->codes || !q->scales || !k->codes || !k->scales || !v->codes || !v->scales || !out)
    return FSATTN_E_INVALID_ARG;
  if (!aligned(q->codes, 16) || !aligned(k->codes, 16) || !aligned(v->codes, 16) || !aligned(out, 4))
    return FSATTN_E_ALIGNMENT;
  if (!aligned(k->scales, 4) || !aligned(v->scales, 4)) return FSATTN_E_ALIGNMENT;
  // per-head byte counts of the K and V codes must fit the 32-bit buffer range
  if ((int64_t)p->Skv * p->D > ((int64_t)1 << 30)) return FSATTN_E_UNSUPPORTED;
  fsattn::FwdArgs a;
  a.qc = static_cast<const uint8_t*>(q->codes);
  a.qs = q->scales;
  a.kc = static_cast<const uint8_t*>(k->codes);
  a.ks = k->scales;
  a.vc = static_cast<const uint8_t*>(v->codes);
  a.vs = v->scales;
  a.out = static_cast<uint16_t*>(out);
  a.counts = p->rollback_counts;
  a.pd_codes = p->p_dump_codes;
  a.pd_scales = p->p_dump_scales;
  a.H = p->H;
  a.Sq = p->Sq;
  a.Skv = p->Skv;
  a.nb32 = (p->Skv + 31) / 32;
  a.pd_bh = p->p_b * p->H + p->p_h;
  a.pd_row0 = p->p_row0;
  a.pd_row1 = p->p_row1;
  // T0 = fl32(128*127 - c) maps the reference to 2^0; T_gate = fl32(128*(127+tau) - c)
  a.T0 = (float)(128.0 * 127.0 - (double)p->schraudolph_c);
  a.Tg = (float)(128.0 * (127.0 + (double)p->tau) - (double)p->schraudolph_c);
  a.kv128 = p->kv_tile == 128;
  a.fitmax = 1;
  a.causal = mask ? mask->causal : 0;
  a.q_lens = mask ? mask->q_lens : nullptr;
  a.kv_lens = mask ? mask->kv_lens : nullptr;
  // EFQ-style P: slope a = 1 / (128 h) rounded up to binary32 (so that a
  // score exactly on a threshold gets its code), and 128 tau (exact)
  if (efq) {
    const double A = 1.0 / (128.0 * (double)efq_h);
    float a32 = (float)A;
    if ((double)a32 < A) a32 = nextafterf(a32, INFINITY);
    a.efq_a = a32;
  } else {
    a.efq_a = 0.0f;
  }
  a.efq_t128 = efq ? 128.0f * efq_tau : 0.0f;
  a.fp8_products = fp8_products ? 1 : 0;
  hipError_t e = fsattn::launch_fsattn_fwd(a, p->B, p->D, q->elem, v->elem, p->p_elem,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_E_HIP;
}

int fsattn_forward_masked(const fsattn_params* p, const fsattn_mask* mask, const fsattn_mx_tensor* q,
                          const fsattn_mx_tensor* k, const fsattn_mx_tensor* v, void* out, void* stream) {
  return forward_impl(p, mask, false, 0.0f, 0.0f, false, q, k, v, out, stream);
}

int fsattn_forward_fp8_products(const fsattn_params* p, const fsattn_mask* mask, const fsattn_mx_tensor* q,
                                const fsattn_mx_tensor* k, const fsattn_mx_tensor* v, void* out, void* stream) {
  return forward_impl(p, mask, false, 0.0f, 0.0f, true, q, k, v, out, stream);
}

int fsattn_forward(const fsattn_params* p, const fsattn_mx_tensor* q, const fsattn_mx_tensor* k,
                   const fsattn_mx_tensor* v, void* out, void* stream) {
  return forward_impl(p, nullptr, false, 0.0f, 0.0f, false, q, k, v, out, stream);
}

int fsattn_pattern_gate_tau(float tau, float schraudolph_c, float* tau_out) {
  if (!tau_out || !(tau >= 0.0f) || !isfinite(tau) || !isfinite(schraudolph_c)) return FSATTN_E_INVALID_ARG;
  const double c = (double)schraudolph_c;
  auto gate = [&](float t) { return (float)(128.0 * (127.0 + (double)t) - c); };
  const double f = floor((double)gate(tau));
  if (!(f < 32639.0)) {
    // the clamped stage-1 pattern never exceeds floor(T_gate): never fires
    *tau_out = FLT_MAX;
    return FSATTN_OK;
  }
  // exact threshold: the largest binary32 below floor(T_gate) + 1
  const float X = nextafterf((float)(f + 1.0), -INFINITY);
  float t = (float)(((double)X + c) / 128.0 - 127.0);
  for (int i = 0; i < 8 && gate(t) != X; ++i) t = nextafterf(t, gate(t) < X ? INFINITY : -INFINITY);
  if (gate(t) != X || t < 0.0f) return FSATTN_E_UNSUPPORTED;
  *tau_out = t;
  return FSATTN_OK;
}

int fsattn_forward_efq(const fsattn_params* p, const fsattn_mask* mask, float efq_tau, float efq_h,
                       const fsattn_mx_tensor* q, const fsattn_mx_tensor* k, const fsattn_mx_tensor* v, void* out,
                       void* stream) {
  return forward_impl(p, mask, true, efq_tau, efq_h, false, q, k, v, out, stream);
}

int fsattn_forward_bf16_baseline(const void* q, const void* k, const void* v, int B, int H, int Sq, int Skv, int D,
                                 float softmax_scale, void* out, void* stream) {
  return fsattn_forward_bf16_baseline_masked(q, k, v, B, H, Sq, Skv, D, softmax_scale, nullptr, out, stream);
}

int fsattn_forward_bf16_baseline_masked(const void* q, const void* k, const void* v, int B, int H, int Sq, int Skv,
                                        int D, float softmax_scale, const fsattn_mask* mask, void* out,
                                        void* stream) {
  if (mask) {
    if (mask->causal != 0 && mask->causal != 1) return FSATTN_E_INVALID_ARG;
    if (!aligned(mask->q_lens, 4) || !aligned(mask->kv_lens, 4)) return FSATTN_E_ALIGNMENT;
  }
  if (B < 0 || H < 0 || Sq < 0 || Skv < 1 || (D != 64 && D != 128)) return FSATTN_E_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return FSATTN_E_INVALID_ARG;
  if (H > 65535 || B > 65535) return FSATTN_E_UNSUPPORTED;
  if (B == 0 || H == 0 || Sq == 0) return FSATTN_OK;
  if (!q || !k || !v || !out) return FSATTN_E_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4)) return FSATTN_E_ALIGNMENT;
  hipError_t e = fsattn::launch_bf16_fwd(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), B, H, Sq, Skv,
                                         D, softmax_scale, mask ? mask->causal : 0, mask ? mask->q_lens : nullptr,
                                         mask ? mask->kv_lens : nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_E_HIP;
}

int fsattn_probe_mfma(int fmt, int64_t iters, int workgroups, unsigned long long* stamps, int* wall_clock_khz,
                      void* stream) {
  if (fmt != FSATTN_E4M3 && fmt != FSATTN_E2M3 && fmt != FSATTN_E2M1 && fmt != FSATTN_PROBE_BF16)
    return FSATTN_E_INVALID_ARG;
  if (iters < 1 || iters > ((int64_t)1 << 32) || workgroups < 1 || workgroups > (1 << 20) || !stamps)
    return FSATTN_E_INVALID_ARG;
  if (!aligned(stamps, 8)) return FSATTN_E_ALIGNMENT;
  if (wall_clock_khz) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(wall_clock_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return FSATTN_E_HIP;
  }
  hipError_t e = fsattn::launch_mfma_probe(fmt, iters, workgroups, stamps, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_E_HIP;
}

}  // extern "C"
