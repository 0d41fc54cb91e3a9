/*
 * fsattn.h -- C ABI of the Fused-Softmax quantized-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("Fused-Softmax shifts an AI attention bottleneck onto faster
 * GPU hardware", cybernoise.de article on arXiv 2611.09225, paragraphs 5-6;
 * "Fused softmax makes quantized attention faster on AMD GPUs", chiosa.app,
 * section "What the evidence shows" / "Move work, keep correction"):
 * attention O = softmax(Q K^T) V with Q, K, V MX-quantized; the row-max
 * reference is provisionally frozen and its subtraction, together with the
 * affine part of Schraudolph's exponential, is folded into the Q K^T matrix
 * product; P is produced by a two-stage conversion (a BF16 bit pattern, then
 * MX); the normalisation sum is the product P.1 fed the same quantized P as
 * P V; a rollback gate raises the reference and rescales O and l when a
 * tile's scores exceed the reference by more than tau.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller (allocate
 *    them with the size helpers below).  The library allocates nothing,
 *    keeps no mutable global state and is safe to call from several host
 *    threads.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; the call returns once enqueued.
 *  - Arguments are validated on the host before anything is launched.  On
 *    any error nothing is launched and a negative fsattn_status is returned.
 *    Empty problems (a zero-sized dimension) return FSATTN_OK without a
 *    launch.  A launch failure is reported as FSATTN_E_HIP.
 *  - No C++ exception crosses this boundary.
 */
#ifndef FSATTN_H
#define FSATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSATTN_ABI_VERSION 3

typedef enum {
  FSATTN_OK = 0,
  FSATTN_E_INVALID_ARG = -1, /* null pointer, bad size, bad enum value */
  FSATTN_E_UNSUPPORTED = -2, /* valid request this build does not implement */
  FSATTN_E_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned */
  FSATTN_E_HIP = -4          /* the HIP runtime reported an error */
} fsattn_status;

/* MX element formats (OCP Microscaling v1.0).  The values equal the gfx950
 * matrix-core format selectors. */
typedef enum {
  FSATTN_E4M3 = 0, /* FP8,  max 448   */
  FSATTN_E5M2 = 1, /* FP8,  max 57344 */
  FSATTN_E2M3 = 2, /* FP6,  max 7.5   */
  FSATTN_E3M2 = 3, /* FP6,  max 28    */
  FSATTN_E2M1 = 4  /* FP4,  max 6     */
} fsattn_elem;

/* E8M0 block-scale rule.  FITMAX: the smallest power of two X with
 * max|x|/X <= the format's largest value (no element saturates).
 * OCP_FLOOR: X = 2^(floor(log2 max|x|) - emax), elements above the largest
 * value saturate. */
typedef enum { FSATTN_SCALE_FITMAX = 0, FSATTN_SCALE_OCP_FLOOR = 1 } fsattn_scale_rule;

int fsattn_abi_version(void);
const char* fsattn_status_str(int status);

/*
 * ---- MX byte layout -----------------------------------------------------
 * A block is 32 elements sharing one E8M0 scale byte (value 2^(s-127)).
 * Codes of a block are packed into 32*bits/8 bytes: 8-bit codes one per
 * byte; 6-bit codes as a little-endian bit stream (element j occupies bits
 * [6j, 6j+6) of the 24 bytes); 4-bit codes two per byte, element 2i in the
 * low nibble of byte i.
 *
 * block_axis 0 (Q, K: blocks along the feature dimension):
 *   input  [n_mat][rows][cols] bf16 (row stride ld elements), cols % 32 == 0
 *   codes  [n_mat][rows][cols/32][block bytes]
 *   scales [n_mat][rows][cols/32], followed by up to 3 bytes of padding
 *          (fsattn_mx_scales_bytes rounds up to whole dwords; the forward
 *          reads K scales a dword at a time)
 * block_axis 1 (V: blocks along keys), stored transposed, key-contiguous:
 *   input  [n_mat][rows][cols] bf16, rows = keys, cols = features (cols <= 128)
 *   codes  [n_mat][cols][rows32/32][block bytes], rows32 = rows rounded up to 32;
 *          keys >= rows are zero padding
 *   scales [n_mat][rows32/32][32][4]: the scale of column c, key block b is at
 *          [b][c % 32][c / 32] (bytes of absent columns are left unwritten), so
 *          one dword holds the scales of columns c, c+32, c+64, c+96.
 */
int64_t fsattn_mx_codes_bytes(int elem, int64_t n_mat, int64_t rows, int64_t cols, int block_axis);
int64_t fsattn_mx_scales_bytes(int64_t n_mat, int64_t rows, int64_t cols, int block_axis);

/*
 * fsattn_fold_prescale -- the multiplicative part of the fold: fl32(128 *
 * log2(e) * softmax_scale), the product taken in binary64 and rounded once.
 * Scores of Q-hat . K-hat are then BF16 bit-pattern units of the Schraudolph
 * exponential ("Fused-Softmax shifts an AI attention bottleneck onto faster
 * GPU hardware", paragraph 6: its linear transform is folded into the score
 * product).  Pass the result as fsattn_quantize_mx's prescale for Q; the
 * forward checks it against softmax_scale.  Host-only.  Returns NaN when
 * softmax_scale is not a positive finite number.
 */
float fsattn_fold_prescale(float softmax_scale);

/*
 * fsattn_quantize_mx -- MX-quantize a bf16 tensor (Q, K or V).
 * Quantized operands of the method ("Fused-Softmax shifts an AI attention
 * bottleneck ...", paragraphs 7-8: MXFP8 / MXFP6 / MXFP4 configurations).
 *
 *  src        device bf16, layout above; ld >= cols.
 *  prescale   every value becomes fl32(prescale * x) before quantization.
 *             For Q pass 128 * log2(e) * softmax_scale rounded to fp32: this
 *             is the multiplicative part of the fold (the Schraudolph slope
 *             and the softmax scale).  K and V: 1.0f.
 *  elem, rule element format and E8M0 rule.
 *  codes_out, scales_out  device buffers of fsattn_mx_*_bytes() bytes.
 *  Per block: amax -> E8M0 -> each element x/X rounded to nearest-even in
 *  the element format (sign of zero kept).  Results are bit-exact with the
 *  definition above.  NaN/Inf inputs are outside the contract.
 *  Errors: FSATTN_E_INVALID_ARG (null, negative sizes, cols % 32 != 0 on
 *  axis 0, cols > 128 on axis 1, ld < cols, bad enum), FSATTN_E_ALIGNMENT
 *  (src not 2-byte or codes_out not 16-byte aligned), FSATTN_E_HIP.
 */
int fsattn_quantize_mx(const void* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld, int block_axis,
                       float prescale, int elem, int rule, void* codes_out, uint8_t* scales_out, void* stream);

/*
 * fsattn_quantize_mx_rmsnorm -- the producer step before the path for
 * qk-normed models, fused into one pass: RMS-normalise each row of Q or K,
 * apply a per-feature weight, then the prescale and MX quantization along the
 * row (block_axis 0 output layout, as fsattn_quantize_mx).  The pages' model
 * (a video diffusion transformer, "Fused-Softmax shifts an AI attention
 * bottleneck onto faster GPU hardware", paragraph 9) normalises Q and K before
 * attention; fusing it removes a full read and write of Q and K.
 *
 * Per row x of `cols` bf16 values:
 *   ss = sum of x_j^2 in binary64 (each 32-block's squares in index order,
 *        then the block sums in order);
 *   r  = fl32(1 / sqrt(ss / cols + eps)), quotient, root and reciprocal in
 *        binary64, correctly rounded; r = 0 when ss / cols + eps is 0;
 *   y_j = fl32(fl32(x_j r) w_j), then fl32(prescale y_j) is MX-quantized like
 *        a fsattn_quantize_mx input (the same rule and rounding).
 *  src      device bf16 [n_mat][rows][cols], row stride ld elements.
 *  weight   optional DEVICE float [cols] (NULL: no weight).
 *  eps      >= 0, finite.
 *  Errors: FSATTN_E_INVALID_ARG (null, negative sizes, ld < cols, cols % 32,
 *  bad enum, eps < 0, non-finite eps or prescale), FSATTN_E_UNSUPPORTED
 *  (cols not a power of two in [32, 2048]), FSATTN_E_ALIGNMENT (src not
 *  2-byte, codes_out not 16-byte, weight not 4-byte aligned), FSATTN_E_HIP.
 */
int fsattn_quantize_mx_rmsnorm(const void* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                               const float* weight, float eps, float prescale, int elem, int rule, void* codes_out,
                               uint8_t* scales_out, void* stream);

/* An MX operand as produced by fsattn_quantize_mx. */
typedef struct {
  int elem;              /* fsattn_elem */
  float prescale;        /* the prescale it was quantized with */
  const void* codes;     /* device */
  const uint8_t* scales; /* device */
} fsattn_mx_tensor;

typedef struct {
  int B, H;              /* batch, heads */
  int Sq, Skv;           /* query and key counts (>= 1 for Skv, any length: tails are masked) */
  int D;                 /* head dimension: 64 or 128 */
  float softmax_scale;   /* sigma; must equal q->prescale / (128 log2 e) to within 2 ulp */
  int p_elem;            /* element format of P: E4M3, E2M3 or E3M2 (E2M1: fsattn_forward_efq only) */
  int p_scale_rule;      /* E8M0 rule of P's blocks: FSATTN_SCALE_FITMAX (the kernels implement only
                            this rule; FSATTN_SCALE_OCP_FLOOR returns FSATTN_E_UNSUPPORTED).  The
                            operands may be quantized with either rule: the forward reads their codes
                            and scales as they are */
  float tau;             /* rollback threshold in log2 units of P, >= 0 (default 8); keep it below
                            128 - c/128: above, accepted scores can pass the stage-1 clamp */
  float schraudolph_c;   /* shift c in BF16-pattern units (default 0) */
  int kv_tile;           /* keys per gate tile, a positive multiple of 32; the kernels run 64 and 128
                            (other multiples of 32 return FSATTN_E_UNSUPPORTED) */
  int32_t* rollback_counts; /* optional device [B][H][Sq]: fires per query row; NULL = not written */
  uint8_t* p_dump_codes;    /* optional device [(p_row1-p_row0)][Skv32], one code per key, for rows
                               [p_row0, p_row1) of head (p_b, p_h); NULL = no dump */
  uint8_t* p_dump_scales;   /* optional device [(p_row1-p_row0)][Skv32/32] E8M0 of P */
  int p_b, p_h, p_row0, p_row1;
} fsattn_params;

/*
 * fsattn_forward -- Fused-Softmax attention forward on MX operands.
 *
 * q: [B][H][Sq][D] codes on block_axis 0 quantized with prescale
 *    128*log2(e)*softmax_scale; k: [B][H][Skv][D] block_axis 0; v: block_axis
 *    1 with rows = Skv ([B][H][D][Skv32]).  Q and K share one element format
 *    (E4M3, E2M3 or E2M1); V is E4M3, E2M3 or E2M1.
 * out: device bf16 [B][H][Sq][D].
 *
 * Per query row i and kv tile j (kv_tile keys, ascending):
 *   t = fl32(C_i + sum_d Qhat_id Khat_kd)   (tile 0: C_i = 0, then
 *       C_i = fl32(T0 - max t), t += C_i; T0 = fl32(128*127 - c))
 *   rollback: if max_k t > T_gate = fl32(128*(127+tau) - c) (tiles j >= 1),
 *       delta = fl32(max t - T0); t -= delta; C_i -= delta;
 *       O_i, l_i *= 2^(-delta/128); count_i += 1
 *   stage 1: b = floor(t) as a BF16 bit pattern (0 if t < 128, at most 0x7F7F)
 *   stage 2: P = MX(bf16(b)) per 32 consecutive keys (fit-max E8M0)
 *   O_i += P V, l_i += P 1 (same P); finally O_i / l_i rounded to bf16.
 * FP6/FP4 score products are exact on the matrix core.  E4M3 Q/K are
 * decoded to BF16 (exact for block scales 2^-124 .. 2^119, that is, for
 * every block of finite bf16 inputs whose maximum lies between about 2^-116
 * and 2^127) and summed on the BF16 matrix core from zero, C_i added once in
 * binary32; fsattn_forward_fp8_products keeps the FP8 product.
 * Errors: FSATTN_E_INVALID_ARG (null, sizes, D not 64/128, kv_tile not a
 * positive multiple of 32, tau < 0, bad enum, prescale/softmax_scale
 * mismatch, bad dump window), FSATTN_E_UNSUPPORTED (format combination,
 * kv_tile other than 64 or 128, P scale rule OCP_FLOOR, Skv * D > 2^30),
 * FSATTN_E_ALIGNMENT (codes not 16-byte, K or V scales not 4-byte, out not
 * 4-byte aligned), FSATTN_E_HIP.
 */
int fsattn_forward(const fsattn_params* p, const fsattn_mx_tensor* q, const fsattn_mx_tensor* k,
                   const fsattn_mx_tensor* v, void* out, void* stream);

/*
 * fsattn_forward_masked -- fsattn_forward with causal and variable-length
 * masks.  Masks are applied before the score shift and probability
 * generation ("EFQ-Softmax: Exp-Free Quantization for Softmax", section
 * III.D "Algorithmic Cost and Method Boundary", kernel boundary): a masked
 * key takes no part in any tile maximum (tile-0 reference, rollback gate) and
 * its P is 0.
 * Tiles keep their positions (tile j = keys [j*kv_tile, (j+1)*kv_tile)).
 *
 * mask (may be NULL = no mask, the same as fsattn_forward):
 *   causal   0 or 1.  1: query i of batch b sees key k only if
 *            k <= i + kv_len_b - q_len_b (queries aligned to the end of the
 *            keys, as for a query block appended to a key cache).
 *   q_lens   optional DEVICE int32 [B]: valid queries of each batch (rows
 *            i >= q_len_b are stored as 0 with count 0); NULL = Sq.
 *   kv_lens  optional DEVICE int32 [B]: valid keys of each batch; NULL = Skv.
 *   Lengths are clamped to [0, Sq] / [0, Skv] on the device.  A row that sees
 *   no key is stored as 0 with count 0.  Keys past kv_len_b must still hold
 *   quantizer output (finite codes): they are read and multiplied by P = 0.
 * Everything else (layouts, params, errors) is as for fsattn_forward; in
 * addition FSATTN_E_INVALID_ARG if causal is not 0/1 and FSATTN_E_ALIGNMENT
 * if q_lens or kv_lens is not 4-byte aligned.  The P dump (params) leaves
 * rows past q_len_b untouched.
 */
typedef struct {
  int causal;
  const int32_t* q_lens;
  const int32_t* kv_lens;
} fsattn_mask;

int fsattn_forward_masked(const fsattn_params* p, const fsattn_mask* mask, const fsattn_mx_tensor* q,
                          const fsattn_mx_tensor* k, const fsattn_mx_tensor* v, void* out, void* stream);

/*
 * fsattn_forward_fp8_products -- fsattn_forward_masked (mask may be NULL)
 * with E4M3 Q/K scores taken from the FP8 matrix core (the scaled 32x32x64
 * f8f6f4 product with C_i as its initial value), the pages' kernel design
 * for MXFP8 ("Fused-Softmax shifts an AI attention bottleneck onto faster
 * GPU hardware", paragraphs 7-8).  gfx950's FP8 product does not return the
 * correctly rounded sum: a score can differ from fl32(C_i + sum) by up to
 * about D binary32 steps, and P codes of scores that close to a stage-1
 * floor boundary can differ from the definition above (measured: up to
 * 1.3e-3 of the codes).  fsattn_forward and fsattn_forward_masked instead
 * decode E4M3 Q and K to BF16 (exact) and sum on the BF16 matrix core from
 * zero, adding C_i once in binary32.  For other Q/K formats (exact on the
 * matrix core) the two are the same.  Arguments, errors and layouts as
 * fsattn_forward_masked.
 */
int fsattn_forward_fp8_products(const fsattn_params* p, const fsattn_mask* mask, const fsattn_mx_tensor* q,
                                const fsattn_mx_tensor* k, const fsattn_mx_tensor* v, void* out, void* stream);

/*
 * fsattn_forward_efq -- the forward with P generated directly as MXFP4
 * (E2M1 codes, one E8M0 per 32 keys) by an EFQ-style affine rule in the log
 * domain, in place of stage 1 and stage 2 ("EFQ-Softmax: Exp-Free
 * Quantization for Softmax", paperlayer.ai summary of arXiv 2609.09721,
 * sections II.B-C and III.A-B).  Everything else (the fold, the frozen
 * reference, the rollback gate, masks, O += P V and l += P 1 with the same P)
 * is fsattn_forward_masked's.  For each 32-key block of P and its folded
 * binary32 scores t (after the tile's gate shift; masked keys excluded), with
 * l = (t - T0) / 128 the score in log2 units (the reference maps to T0):
 *   E    = floor(max l) clamped to [-1000, 1000] (the exponent of the block's
 *          largest probability)
 *   E8M0 = clamp(E - 2 + 127, 0, 254)
 *   code = #{ j in 1..7 : l - E >= efq_tau + j efq_h }   (code 7 is E2M1's 6.0)
 * i.e. the residual l - E is compared with uniformly spaced thresholds.  The
 * kernel counts them as clamp(floor(fma(t, a, b)), 0, 7) with
 * a = 1 / (128 efq_h) and b = -(T0 + 128 E + 128 efq_tau) a, both rounded up
 * to binary32: a score exactly on a threshold gets the higher code, and the
 * count is exact except that a score exactly one binary32 step below a
 * threshold may also get it (for the calibrated spacing 128 efq_h = 78 only
 * when t >= 16384).  Masked keys
 * get code 0.  (efq_tau, efq_h) are calibrated offline; -3.875 and
 * 0.609375 minimize the output error on synthetic MXFP4 attention.
 *
 * p->p_elem must be FSATTN_E2M1; Q/K/V are all E2M3 or all E2M1.  A P dump
 * (p_dump_codes) holds the E2M1 codes.  efq_h in [1/64, 16], efq_tau in
 * [-64, 64].  mask may be NULL.
 * Errors: as fsattn_forward_masked; FSATTN_E_INVALID_ARG also for p_elem not
 * E2M1 or (efq_tau, efq_h) out of range; FSATTN_E_UNSUPPORTED for other
 * Q/K/V formats.  (fsattn_forward and fsattn_forward_masked return
 * FSATTN_E_UNSUPPORTED for p_elem E2M1.)
 */
int fsattn_forward_efq(const fsattn_params* p, const fsattn_mask* mask, float efq_tau, float efq_h,
                       const fsattn_mx_tensor* q, const fsattn_mx_tensor* k, const fsattn_mx_tensor* v, void* out,
                       void* stream);

/*
 * fsattn_pattern_gate_tau -- the gate threshold for the rollback-gate
 * shortcut.  The pages report that their fastest 4-bit kernel gates through
 * a shortcut that can miss a recovery trigger in an extreme-score range
 * ("Fused-Softmax shifts an AI attention bottleneck onto faster GPU
 * hardware", cybernoise.de, paragraph 12), without describing it.  Read here
 * as deciding on the stage-1 BF16 patterns: a tile fires when
 * stage1(max t) > floor(T_gate), with T_gate = fl32(128 (127 + tau) - c).
 * For floor(T_gate) < 0x7F7F that is exactly the exact rule (max t > T_gate')
 * at T_gate' = the largest binary32 below floor(T_gate) + 1; at or above
 * 0x7F7F the clamped pattern never exceeds it and the shortcut never fires.
 * This call returns in *tau_out the tau' whose T_gate is T_gate' (FLT_MAX,
 * which never fires, in the second case); fsattn_forward with tau' then runs
 * the shortcut at no extra cost.  It misses tiles whose max lies less than
 * one pattern step above T_gate, and every tile once T_gate >= 0x7F7F.
 * Note that T_gate >= 0x7F7F (tau >= 128 - c/128) lets the exact gate keep
 * scores past the stage-1 clamp too.
 * Host-only, no GPU use.  Errors: FSATTN_E_INVALID_ARG (tau_out NULL, tau < 0
 * or not finite, c not finite), FSATTN_E_UNSUPPORTED (no binary32 tau'
 * reproduces T_gate'; does not happen for c = 0).
 */
int fsattn_pattern_gate_tau(float tau, float schraudolph_c, float* tau_out);

/*
 * fsattn_forward_bf16_baseline -- conventional attention forward in BF16
 * (the baseline the pages compare against, paragraph 8): tiled online
 * softmax with a running max and rescaling ("Conventional implementations
 * repeatedly update a reference maximum and rescale", paragraph 5), BF16
 * matrix products with fp32 accumulation, exp2 in fp32.
 * q [B][H][Sq][D], k, v [B][H][Skv][D], out [B][H][Sq][D]; all bf16, device,
 * contiguous.  D = 64 or 128.
 * Errors: FSATTN_E_INVALID_ARG, FSATTN_E_ALIGNMENT, FSATTN_E_HIP.
 */
int fsattn_forward_bf16_baseline(const void* q, const void* k, const void* v, int B, int H, int Sq, int Skv,
                                 int D, float softmax_scale, void* out, void* stream);

/*
 * fsattn_forward_bf16_baseline_masked -- the BF16 baseline under the masks of
 * fsattn_forward_masked (causal, per-batch device q_lens / kv_lens; mask NULL
 * = fsattn_forward_bf16_baseline): each row's softmax runs over its visible
 * keys; rows that see no key, and rows past q_len, are stored as 0.  The
 * comparison point for masked fused attention (masks precede the softmax,
 * "EFQ-Softmax: Exp-Free Quantization for Softmax", section III.D
 * "Algorithmic Cost and Method Boundary", kernel boundary).  Errors as fsattn_forward_bf16_baseline, plus
 * FSATTN_E_INVALID_ARG if causal is not 0/1 and FSATTN_E_ALIGNMENT if a
 * length array is not 4-byte aligned.
 */
int fsattn_forward_bf16_baseline_masked(const void* q, const void* k, const void* v, int B, int H, int Sq, int Skv,
                                        int D, float softmax_scale, const fsattn_mask* mask, void* out,
                                        void* stream);

/*
 * fsattn_probe_mfma -- measurement helper, not part of the attention path.
 * Runs a kernel that only issues matrix products: `workgroups` workgroups of
 * eight waves (two per SIMD, as the fused forward), each wave `iters` rounds
 * of four independent accumulator chains of one 32x32x64 product per round
 * (fmt FSATTN_E4M3 / E2M3 / E2M1: the scaled MX product with both operands
 * in that format) or four 32x32x16 BF16 products (FSATTN_PROBE_BF16).
 * Per wave, flops = iters * 4 * 2*32*32*64.  Wave 0 of workgroup g writes
 * stamps[4g .. 4g+3] = shader-clock counter (s_memtime) at start and end,
 * constant-rate counter (s_memrealtime, the device's wall-clock rate) at
 * start and end, so the caller can derive the matrix-core rate and the
 * shader clock under that load.  stamps: caller-owned device
 * uint64 [workgroups][4], 8-byte aligned.  wall_clock_khz: optional host
 * int, set to the constant rate of the second counter (kHz) of the current
 * device.
 * Errors: FSATTN_E_INVALID_ARG (fmt, iters outside [1, 2^32], workgroups
 * outside [1, 2^20], stamps NULL), FSATTN_E_ALIGNMENT, FSATTN_E_HIP.
 */
#define FSATTN_PROBE_BF16 16
int fsattn_probe_mfma(int fmt, int64_t iters, int workgroups, unsigned long long* stamps, int* wall_clock_khz,
                      void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FSATTN_H */
