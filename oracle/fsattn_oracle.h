/*
 * fsattn_oracle.h -- CPU oracle for Fused-Softmax quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no source, header, table or helper with the GPU library (which lives under
 * softmax_matrix_cores_amd/csrc and include/), and neither side includes the
 * other.
 *
 * Sources (web pages on the method; cited by title and section/paragraph):
 *  [FS-news]  "Fused-Softmax shifts an AI attention bottleneck onto faster GPU
 *             hardware" (cybernoise.de article on arXiv 2611.09225), body
 *             paragraphs numbered 1..13 from "Making AI calculations ...".
 *  [FS-sum]   "Fused softmax makes quantized attention faster on AMD GPUs"
 *             (chiosa.app summary of arXiv 2611.09225), sections "In plain
 *             words", "The research", "What the evidence shows".
 *  [EFQ]      "EFQ-Softmax: Exp-Free Quantization for Softmax" (paperlayer.ai
 *             summary of arXiv 2609.09721), sections I, II.A-D, III.A-D.
 *
 * Every place where the pages leave a step open is a named reading; the
 * list of readings (R-numbers below) is the oracle's contract.
 *
 * Number formats (OCP Microscaling v1.0 element types + E8M0 scale):
 *   E4M3 (bias 7,  max 448, NaN = S.1111.111, no Inf)
 *   E5M2 (bias 15, max 57344, Inf/NaN at exponent 31)
 *   E2M3 (bias 1,  max 7.5)    E3M2 (bias 3, max 28)    E2M1 (bias 1, max 6)
 *   E8M0 scale: 2^(code-127), code 255 = NaN.
 */
#ifndef FSATTN_ORACLE_H
#define FSATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats (same numbering as the MFMA format selector; values are a
 * public hardware encoding, not shared code) */
enum { FSO_E4M3 = 0, FSO_E5M2 = 1, FSO_E2M3 = 2, FSO_E3M2 = 3, FSO_E2M1 = 4 };

/* E8M0 scale rule.  FITMAX: smallest power of two X with amax/X <= maxnorm,
 * i.e. k = ceil(log2(amax/maxnorm)).  OCP_FLOOR: k = floor(log2 amax) - emax
 * (the OCP v1.0 rule; elements above maxnorm saturate). */
enum { FSO_SCALE_FITMAX = 0, FSO_SCALE_OCP_FLOOR = 1 };

/* switches used by the invariant checks; the method itself is
 * exp=SCHRAUDOLPH, p=MX, fold=FP32 */
enum { FSO_EXP_SCHRAUDOLPH = 0, FSO_EXP_EXACT = 1 };
enum { FSO_P_MX = 0, FSO_P_NONE = 1, FSO_P_EFQ = 2 };
enum { FSO_FOLD_FP32 = 0, FSO_FOLD_EXACT = 1 };
/* rollback gate: the exact rule, or the pattern shortcut of R25 */
enum { FSO_GATE_EXACT = 0, FSO_GATE_PATTERN = 1 };

/* references computed on the same quantized operands */
enum {
  FSO_REF_R1 = 1,   /* exact softmax of the quantized scores, V-hat, P unquantized */
  FSO_REF_R2 = 2,   /* conventional softmax, numerator uses MX-quantized p, denominator sum p */
  FSO_REF_R2P = 3,  /* as R2 but denominator sum of MX-quantized p */
  FSO_REF_R3 = 4    /* FlashAttention online max/rescale per kv tile, MX-quantized p in both sums */
};

#define FSO_OK 0
#define FSO_EINVAL (-1)
#define FSO_ENOMEM (-2)

int fso_version(void);
int fso_default_threads(void);

/* ---- element codec ---- */
int fso_elem_bits(int elem);
double fso_elem_maxnorm(int elem);
double fso_decode(int elem, int code);         /* code -> value */
int fso_encode(int elem, double x);             /* round-to-nearest-even, saturate to +-maxnorm */

/* ---- MX block quantizer ---- */
int fso_scale_code(int elem, int rule, double amax);
/* quantize n<=32 values as one block: codes[n] (one byte each), *scale = E8M0 */
void fso_mxq_block(int elem, int rule, const double* x, int n, uint8_t* codes, uint8_t* scale);

/* bytes of one packed 32-element block */
int fso_block_bytes(int elem);

/*
 * Quantize a bf16 tensor [n_mat][rows][cols] (row stride ld elements) to MX.
 *  block_axis 0: blocks of 32 along cols (cols % 32 == 0).  codes: [n_mat][rows][cols/32][block bytes],
 *                scales [n_mat][rows][cols/32].
 *  block_axis 1: blocks of 32 along rows; output is stored transposed,
 *                codes [n_mat][cols][rows32/32][block bytes], scales [n_mat][cols][rows32/32],
 *                rows32 = rows rounded up to 32, padding rows are zero.
 * prescale: each value becomes fl32(prescale * x) before quantization.
 * Packing inside a block: 8-bit codes one per byte; 6-bit codes form a
 * little-endian bit stream (code j in bits [6j, 6j+6) of 24 bytes); 4-bit
 * codes two per byte, even index in the low nibble.
 */
int fso_quantize_mx(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                    int block_axis, float prescale, int elem, int rule,
                    uint8_t* codes, uint8_t* scales);

/*
 * Fused producer step before the path (RMS-normalised Q/K rows, then the
 * prescale and MX quantization), reading R23: for each row x of `cols`
 * bf16 values (block_axis 0 layout):
 *   ss = sum of x_j^2 in binary64, each 32-block's squares in index order,
 *        then the block sums in order;
 *   r  = fl32(1 / sqrt(ss / cols + eps)), quotient/root/reciprocal in
 *        binary64; r = 0 when ss / cols + eps is 0;
 *   y_j = fl32(fl32(x_j r) w_j) (w = NULL: no weight);
 *   then y is quantized like fso_quantize_mx input: fl32(prescale y), MX.
 * eps >= 0.
 */
int fso_quantize_mx_rmsnorm(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                            const float* weight, float eps, float prescale, int elem, int rule,
                            uint8_t* codes, uint8_t* scales);

/* Schraudolph stage 1: fp32 folded score -> BF16 bit pattern */
uint16_t fso_stage1(float t);

/*
 * R24, EFQ-style direct E2M1 P of one 32-key block ("EFQ-Softmax: Exp-Free
 * Quantization for Softmax", sections II.B-C, III.B): from the block's folded
 * binary32 scores t[0..nvis) (keys nvis..31 absent: code 0; nvis = 0: E8M0 0),
 * in exact arithmetic, with tau and h rounded to binary32 first:
 *   l_k  = (t_k - T0) / 128                  (log2 units, reference at T0)
 *   E    = floor(max l) clamped to [-1000, 1000]  (exponent of the block maximum)
 *   E8M0 = clamp(E - 2 + 127, 0, 254)
 *   code = #{j in 1..7 : l_k - E >= tau + j h}   (E2M1 codes 0..7 = 0 .. 6.0)
 */
void fso_efq_block(const float* t, int nvis, float T0, double tau, double h, uint8_t* codes, uint8_t* scale);

typedef struct {
  int B, H, Sq, Skv, D;
  int qk_elem, v_elem, p_elem, scale_rule;
  double tau;        /* rollback threshold, log2 units */
  double c;          /* Schraudolph shift in BF16-pattern units */
  int kv_tile;       /* keys per gate tile, multiple of 32 */
  int exp_mode, p_mode, fold_mode;
  int nthreads;      /* <= 0: all online CPUs */
  /* p_mode FSO_P_EFQ (R24, needs p_elem E2M1 and the binary32 fold): the
   * threshold shift tau and spacing h, in log2 units; h in [1/64, 16],
   * tau in [-64, 64] */
  double efq_tau, efq_h;
  /* R25: gate_mode FSO_GATE_PATTERN fires a tile (j >= 1) when
   * stage1(max t) > floor(T_gate) instead of max t > T_gate.  gate_misses:
   * optional output [nrows], per row the tiles the exact rule would fire in
   * the same state and the chosen rule does not (0 for the exact rule). */
  int gate_mode;
  int32_t* gate_misses;
} fso_params;

/*
 * Fused-Softmax forward on MX operands in the quantizer's packed layout
 * (Q, K: block_axis 0 with cols = D; V: block_axis 1 with rows = Skv).
 * rows: flattened row ids (b*H + h)*Sq + i, or NULL for all B*H*Sq rows.
 * out_O [nrows][D] (double), out_l [nrows] (may be NULL), counts [nrows] (may be NULL),
 * p_codes [nrows][Skv32] one byte per key and p_scales [nrows][Skv32/32] (both may be NULL).
 */
int fso_forward(const fso_params* p,
                const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                const uint8_t* vc, const uint8_t* vs,
                const int64_t* rows, int64_t nrows,
                double* out_O, double* out_l, int32_t* counts,
                uint8_t* p_codes, uint8_t* p_scales);

/*
 * Masked and variable-length attention (masks go before the score shift and
 * probability generation: "EFQ-Softmax: Exp-Free Quantization for Softmax",
 * section III.D "Algorithmic Cost and Method Boundary", kernel boundary).
 *  causal   query i of batch b sees key k only if k <= i + kv_len_b - q_len_b
 *           (queries aligned to the end of the keys)
 *  q_lens   optional host [B]: valid queries per batch, clamped to [0, Sq]
 *  kv_lens  optional host [B]: valid keys per batch, clamped to [0, Skv]
 * A masked key is absent: it takes no part in a tile's maximum (reference or
 * gate) and its P is 0.  Tiles keep their positions (tile j = keys
 * [j*kv_tile, (j+1)*kv_tile)).  A row with no visible key, and every row
 * i >= q_len_b, has O = 0, l = 0 and count 0.
 */
typedef struct {
  int causal;
  const int32_t* q_lens;
  const int32_t* kv_lens;
} fso_mask;

int fso_forward_masked(const fso_params* p, const fso_mask* m,
                       const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                       const uint8_t* vc, const uint8_t* vs,
                       const int64_t* rows, int64_t nrows,
                       double* out_O, double* out_l, int32_t* counts,
                       uint8_t* p_codes, uint8_t* p_scales);

/*
 * Diagnostics of the forward for rows[0..nrows) (all rows if rows is NULL):
 * t_out [rows][Skv32] the folded binary32 score of each visible key after its
 * tile's gate shift (the value stage 1 floors; other keys untouched), abs_out
 * [rows][Skv32] max_d |Qhat_d Khat_d| in binary64, the magnitude the rounding
 * of a matrix core that does not return the exactly rounded sum scales with.  m may be NULL.  Used to explain P-code differences of such hardware.
 */
int fso_forward_scores(const fso_params* p, const fso_mask* m, const uint8_t* qc, const uint8_t* qs,
                       const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs,
                       const int64_t* rows, int64_t nrows, float* t_out, double* abs_out);


/* References on the same quantized operands (see FSO_REF_*). */
int fso_reference(const fso_params* p, int ref,
                  const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                  const uint8_t* vc, const uint8_t* vs,
                  const int64_t* rows, int64_t nrows, double* out_O);

/* R0: exact softmax attention in double on the bf16 inputs [B][H][S][D], scale sigma. */
int fso_reference_bf16(int B, int H, int Sq, int Skv, int D, double sigma,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int64_t* rows, int64_t nrows, int nthreads, double* out_O);

/* R0 under the mask of fso_forward_masked: row i's softmax runs over its
 * visible keys only; a row that sees no key (or i >= q_len) is 0. */
int fso_reference_bf16_masked(int B, int H, int Sq, int Skv, int D, double sigma, const fso_mask* mask,
                              const uint16_t* q, const uint16_t* k, const uint16_t* v, const int64_t* rows,
                              int64_t nrows, int nthreads, double* out_O);

/* Exact folded score of one (query,key) pair: returns fl32(cinit + sum_d qhat*khat),
 * or the double value when exact_fold != 0.  Exposed for the pins. */
double fso_folded_score(int qk_elem, const uint8_t* qrow_codes, const uint8_t* qrow_scales,
                        const uint8_t* krow_codes, const uint8_t* krow_scales, int D,
                        double cinit, int exact_fold);

#ifdef __cplusplus
}
#endif
#endif
