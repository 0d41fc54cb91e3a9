/*
 * fsattn_oracle.c -- CPU oracle for Fused-Softmax quantized attention.
 *
 * TEST INFRASTRUCTURE ONLY (see fsattn_oracle.h): loaded by the test suite,
 * the smoke check and the benchmark's CPU-baseline leg, never by the library.
 * Plain C11 + pthreads, no SIMD intrinsics, no BLAS.
 *
 * What it computes, step by step, with the passage each step follows:
 *
 *  The method [FS-news, paragraphs 5-6; FS-sum, "What the evidence shows" /
 *  "Move work, keep correction"]:
 *   - scores come from a matrix product of quantized Q and K; the row-max
 *     reference is frozen provisionally and its subtraction is folded into
 *     that product [FS-news 5];
 *   - the exponential is Schraudolph's bit-pattern approximation whose affine
 *     map is folded into the same product [FS-news 6];
 *   - a two-stage conversion builds a BF16 value, then the low-precision P
 *     operand [FS-news 6];
 *   - the normalisation sum is another product that uses the same quantized
 *     P as the output product [FS-news 6; EFQ III.A];
 *   - when later scores exceed a safety threshold the reference is raised and
 *     the accumulated quantities are corrected [FS-news 5, 12].
 *
 *  Readings where the pages are silent (the oracle's contract):
 *   R1  tau is in log2 units of P: tile fires when max score > reference + tau.
 *   R2  initial reference = row max of the first kv tile, not counted:
 *       C_i = fl32(T0 - tmax), so the row max maps to T0 (P = 2^(-c/128)).
 *   R3  on a fire, the new reference is that tile's row max:
 *       delta = fl32(tmax - T0), C_i = fl32(C_i - delta).
 *   R4  gate per row, per kv_tile keys, strict '>', valid keys only.
 *   R5  correction multiplies O and l by exactly 2^(-delta/128).
 *   R6  Schraudolph shift c (default 0) in BF16-pattern units.
 *   R7  stage 1: b = floor(t), t < 128 -> 0 (BF16 subnormals flushed),
 *       upper clamp 0x7F7F (largest finite BF16).
 *   R8  the multiplicative part of the fold, 128*log2(e)*sigma, scales Q
 *       before quantization; the additive part is the accumulator's initial
 *       value C_i = T0 - m_i.
 *   R9  fold rounding: t = fl32(C_i + exact sum), one rounding.
 *   R10 E8M0 rule: fit-max (smallest X with amax/X <= maxnorm).
 *   R11 element rounding RNE, saturating, sign of zero kept.
 *   R12 MX blocks: Q, K along D; V along keys; P along 32 consecutive keys
 *       aligned at multiples of 32.
 *   R13 six-bit P = E2M3.
 *   R14 keys >= Skv are padding: b = 0, excluded from the gate and maxima.
 *   R16 output in fp64 here (the GPU writes bf16).
 *   R19 kv tiles in ascending key order, one pass.
 *   R24 EFQ-style P (p_mode FSO_P_EFQ, see efq_block): E2M1 codes straight
 *       from the folded scores, an exponent-only E8M0 per 32-key block; the
 *       thresholds are compared in exact arithmetic.
 *   R25 gate shortcut (gate_mode FSO_GATE_PATTERN): the tile fires when its
 *       largest stage-1 BF16 pattern exceeds floor(T_gate); a miss is a tile
 *       the exact rule (R1, R4) would fire and the shortcut does not.
 *
 *  fl32(x) below means round-to-nearest-even of the exact x to binary32.
 */
#define _GNU_SOURCE
#include "fsattn_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef __int128 i128;

int fso_version(void) { return 1; }

int fso_default_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/* ------------------------------------------------------------------------ */
/* Element formats (OCP MX v1.0 / OCP FP8)                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
  int ebits, mbits, bias;
  int emax;          /* exponent of the largest normal */
  int max_mfield;    /* mantissa field of the largest normal */
  int nan_top;       /* 1: E4M3-style (only S.1111.111 is NaN); 2: IEEE-style (top exponent reserved) */
} fmt_t;

static const fmt_t FMT[5] = {
    /* E4M3 */ {4, 3, 7, 8, 6, 1},
    /* E5M2 */ {5, 2, 15, 15, 3, 2},
    /* E2M3 */ {2, 3, 1, 2, 7, 0},
    /* E3M2 */ {3, 2, 3, 4, 3, 0},
    /* E2M1 */ {2, 1, 1, 2, 1, 0},
};

static int valid_elem(int e) { return e >= 0 && e <= 4; }

int fso_elem_bits(int elem) { return valid_elem(elem) ? 1 + FMT[elem].ebits + FMT[elem].mbits : 0; }

int fso_block_bytes(int elem) { return fso_elem_bits(elem) * 32 / 8; }

double fso_elem_maxnorm(int elem) {
  const fmt_t* f = &FMT[elem];
  return ldexp(1.0 + (double)f->max_mfield / (1 << f->mbits), f->emax);
}

/* largest mantissa of a normal, as a value in [1,2) */
static double elem_mmax(int elem) {
  const fmt_t* f = &FMT[elem];
  return 1.0 + (double)f->max_mfield / (1 << f->mbits);
}

double fso_decode(int elem, int code) {
  const fmt_t* f = &FMT[elem];
  int nb = f->ebits + f->mbits;
  int sign = (code >> nb) & 1;
  int E = (code >> f->mbits) & ((1 << f->ebits) - 1);
  int M = code & ((1 << f->mbits) - 1);
  double v;
  if (f->nan_top == 1 && E == (1 << f->ebits) - 1 && M == (1 << f->mbits) - 1) return NAN;
  if (f->nan_top == 2 && E == (1 << f->ebits) - 1) v = (M == 0) ? INFINITY : NAN;
  else if (E == 0) v = ldexp((double)M, 1 - f->bias - f->mbits);
  else v = ldexp((double)((1 << f->mbits) + M), E - f->bias - f->mbits);
  return sign ? -v : v;
}

/* value of a code as integer * 2^lsb, lsb = 1 - bias - mbits (exact, finite codes only) */
static int64_t elem_mint(int elem, int code) {
  const fmt_t* f = &FMT[elem];
  int nb = f->ebits + f->mbits;
  int sign = (code >> nb) & 1;
  int E = (code >> f->mbits) & ((1 << f->ebits) - 1);
  int M = code & ((1 << f->mbits) - 1);
  int64_t m = (E == 0) ? (int64_t)M : ((int64_t)((1 << f->mbits) + M) << (E - 1));
  return sign ? -m : m;
}
static int elem_lsb(int elem) { return 1 - FMT[elem].bias - FMT[elem].mbits; }

int fso_encode(int elem, double x) {
  const fmt_t* f = &FMT[elem];
  int nb = f->ebits + f->mbits;
  int sign = signbit(x) ? 1 : 0;
  double a = fabs(x);
  double maxn = fso_elem_maxnorm(elem);
  int mag;
  if (isnan(x)) {
    /* out of contract; a NaN code where the format has one, else max */
    mag = f->nan_top ? ((1 << nb) - 1) : ((1 << nb) - 1);
    return (sign << nb) | mag;
  }
  if (a >= maxn) {
    mag = (f->emax + f->bias) << f->mbits | f->max_mfield;
  } else if (a == 0.0) {
    mag = 0;
  } else {
    int e;
    (void)frexp(a, &e);
    e -= 1; /* a = m * 2^e, m in [1,2) */
    int emin = 1 - f->bias;
    if (e < emin) e = emin;
    double q = ldexp(1.0, e - f->mbits);
    double n = rint(a / q); /* a/q exact (power-of-two division); rint = ties-to-even */
    if (n * q > maxn) {
      mag = (f->emax + f->bias) << f->mbits | f->max_mfield;
    } else {
      int64_t ni = (int64_t)n;
      if (ni < (1 << f->mbits)) {
        mag = (int)ni; /* subnormal, E = 0 (only reachable when e == emin) */
      } else {
        if (ni == (2 << f->mbits)) { e += 1; ni = 1 << f->mbits; }
        mag = ((e + f->bias) << f->mbits) | (int)(ni - (1 << f->mbits));
      }
    }
  }
  return (sign << nb) | mag;
}

/* ------------------------------------------------------------------------ */
/* MX block quantization (R10, R11)                                          */
/* ------------------------------------------------------------------------ */

int fso_scale_code(int elem, int rule, double amax) {
  if (isnan(amax) || isinf(amax)) return 255;
  if (amax == 0.0) return 0;
  int e;
  double m = frexp(amax, &e); /* amax = m * 2^e, m in [0.5,1) */
  m *= 2.0;
  e -= 1; /* m in [1,2) */
  int k = e - FMT[elem].emax;
  if (rule == FSO_SCALE_FITMAX && m > elem_mmax(elem)) k += 1;
  int code = k + 127;
  if (code < 0) code = 0;
  if (code > 254) code = 254;
  return code;
}

void fso_mxq_block(int elem, int rule, const double* x, int n, uint8_t* codes, uint8_t* scale) {
  double amax = 0.0;
  int bad = 0;
  for (int i = 0; i < n; ++i) {
    if (isnan(x[i]) || isinf(x[i])) bad = 1;
    else if (fabs(x[i]) > amax) amax = fabs(x[i]);
  }
  if (bad) {
    *scale = 255;
    for (int i = 0; i < n; ++i) codes[i] = 0;
    return;
  }
  int sc = fso_scale_code(elem, rule, amax);
  *scale = (uint8_t)sc;
  for (int i = 0; i < n; ++i) codes[i] = (uint8_t)fso_encode(elem, ldexp(x[i], 127 - sc));
}

/* pack 32 codes into one block of the documented byte layout */
static void pack_block(int elem, const uint8_t* c, uint8_t* out) {
  int bits = fso_elem_bits(elem);
  int nbytes = bits * 4;
  memset(out, 0, (size_t)nbytes);
  for (int j = 0; j < 32; ++j) {
    for (int b = 0; b < bits; ++b) {
      int pos = j * bits + b;
      if ((c[j] >> b) & 1) out[pos >> 3] |= (uint8_t)(1u << (pos & 7));
    }
  }
}

/* read code j of a packed block */
static int unpack_code(int elem, const uint8_t* blk, int j) {
  int bits = fso_elem_bits(elem);
  int code = 0;
  for (int b = 0; b < bits; ++b) {
    int pos = j * bits + b;
    code |= ((blk[pos >> 3] >> (pos & 7)) & 1) << b;
  }
  return code;
}

static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

typedef struct {
  const uint16_t* src;
  int64_t n_mat, rows, cols, ld;
  int block_axis, elem, rule;
  float prescale;
  uint8_t *codes, *scales;
  int rmsnorm;          /* axis 0 only: RMS-normalise each row first (R23) */
  const float* weight;  /* [cols] per-feature weight, or NULL */
  float eps;
  int64_t nunits; /* axis 0: n_mat*rows rows; axis 1: n_mat*cols columns */
  int64_t next;
  pthread_mutex_t mu;
} quant_job_t;

/* RMS factor of one row (R23): the squares summed in binary64 block by block
 * (each block's 32 squares in index order, then the block sums in order);
 * r = fl32(1 / sqrt(ss / cols + eps)) with the quotient, the root and the
 * reciprocal in binary64; r = 0 when ss / cols + eps is 0 (a zero row stays
 * zero).  The squares of bf16 values are exact in binary64. */
static float rms_factor(const uint16_t* s, int64_t cols, float eps) {
  double ss = 0.0;
  for (int64_t g = 0; g < cols / 32; ++g) {
    double b = 0.0;
    for (int j = 0; j < 32; ++j) {
      double v = bf16_to_double(s[g * 32 + j]);
      b += v * v;
    }
    ss += b;
  }
  double a = ss / (double)cols + (double)eps;
  if (a == 0.0) return 0.0f;
  return (float)(1.0 / sqrt(a));
}

/* quantize every block of one unit (a row on axis 0, a column on axis 1) */
static void quant_unit(const quant_job_t* J, int64_t u) {
  int bb = fso_block_bytes(J->elem);
  double x[32];
  uint8_t c[32];
  if (J->block_axis == 0) {
    int64_t m = u / J->rows, r = u % J->rows, nb = J->cols / 32;
    const uint16_t* s = J->src + m * J->rows * J->ld + r * J->ld;
    const float rf = J->rmsnorm ? rms_factor(s, J->cols, J->eps) : 1.0f;
    for (int64_t g = 0; g < nb; ++g) {
      for (int j = 0; j < 32; ++j) {
        double v = bf16_to_double(s[g * 32 + j]);
        if (J->rmsnorm) {
          /* y = fl32(fl32(x r) w), then the prescale like any operand */
          float y = (float)v * rf;
          if (J->weight) y = y * J->weight[g * 32 + j];
          v = (double)y;
        }
        x[j] = (J->prescale == 1.0f) ? v : (double)(float)((double)J->prescale * v);
      }
      fso_mxq_block(J->elem, J->rule, x, 32, c, J->scales + u * nb + g);
      pack_block(J->elem, c, J->codes + (u * nb + g) * bb);
    }
  } else {
    int64_t m = u / J->cols, col = u % J->cols;
    int64_t nb = (J->rows + 31) / 32;
    const uint16_t* s = J->src + m * J->rows * J->ld;
    for (int64_t g = 0; g < nb; ++g) {
      for (int j = 0; j < 32; ++j) {
        int64_t r = g * 32 + j;
        double v = (r < J->rows) ? bf16_to_double(s[r * J->ld + col]) : 0.0;
        x[j] = (J->prescale == 1.0f) ? v : (double)(float)((double)J->prescale * v);
      }
      fso_mxq_block(J->elem, J->rule, x, 32, c, J->scales + u * nb + g);
      pack_block(J->elem, c, J->codes + (u * nb + g) * bb);
    }
  }
}

static void* quant_worker(void* arg) {
  quant_job_t* J = (quant_job_t*)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t u0 = J->next;
    J->next += 64;
    pthread_mutex_unlock(&J->mu);
    if (u0 >= J->nunits) break;
    int64_t u1 = u0 + 64 < J->nunits ? u0 + 64 : J->nunits;
    for (int64_t u = u0; u < u1; ++u) quant_unit(J, u);
  }
  return NULL;
}

static int quantize_impl(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                         int block_axis, float prescale, int elem, int rule, uint8_t* codes, uint8_t* scales,
                         int rmsnorm, const float* weight, float eps) {
  if (!valid_elem(elem) || (block_axis != 0 && block_axis != 1) || n_mat < 0 || rows < 0 || cols < 0 ||
      ld < cols)
    return FSO_EINVAL;
  if (block_axis == 0 && cols % 32) return FSO_EINVAL;
  if (rmsnorm && (block_axis != 0 || !(eps >= 0.0f))) return FSO_EINVAL;
  quant_job_t J;
  J.rmsnorm = rmsnorm; J.weight = weight; J.eps = eps;
  J.src = src; J.n_mat = n_mat; J.rows = rows; J.cols = cols; J.ld = ld;
  J.block_axis = block_axis; J.elem = elem; J.rule = rule; J.prescale = prescale;
  J.codes = codes; J.scales = scales;
  J.nunits = block_axis == 0 ? n_mat * rows : n_mat * cols;
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  int nt = fso_default_threads();
  if (nt > 64) nt = 64;
  if ((int64_t)nt > J.nunits / 64 + 1) nt = (int)(J.nunits / 64 + 1);
  pthread_t th[64];
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, quant_worker, &J);
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&J.mu);
  return FSO_OK;
}

int fso_quantize_mx(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                    int block_axis, float prescale, int elem, int rule,
                    uint8_t* codes, uint8_t* scales) {
  return quantize_impl(src, n_mat, rows, cols, ld, block_axis, prescale, elem, rule, codes, scales, 0, NULL, 0.0f);
}

int fso_quantize_mx_rmsnorm(const uint16_t* src, int64_t n_mat, int64_t rows, int64_t cols, int64_t ld,
                            const float* weight, float eps, float prescale, int elem, int rule,
                            uint8_t* codes, uint8_t* scales) {
  return quantize_impl(src, n_mat, rows, cols, ld, 0, prescale, elem, rule, codes, scales, 1, weight, eps);
}

/* ------------------------------------------------------------------------ */
/* Exact arithmetic helpers for the folded score (R9)                        */
/* ------------------------------------------------------------------------ */

static int bitlen128(unsigned __int128 v) {
  int n = 0;
  while (v) { ++n; v >>= 1; }
  return n;
}

/* a term of an exact sum: value = m * 2^e */
typedef struct { i128 m; int e; } term_t;

/* Round sum(terms) to binary32 (RNE).  Exact whenever the terms span fewer
 * than ~120 bits, which holds for all MX operand scales a block can carry
 * in practice; beyond that the lowest bits are folded into a sticky bit. */
static void exact_sum(const term_t* t, int n, i128* outm, int* oute) {
  int emin = 1 << 30, top = -(1 << 30);
  for (int i = 0; i < n; ++i) {
    if (t[i].m == 0) continue;
    unsigned __int128 a = t[i].m < 0 ? (unsigned __int128)(-t[i].m) : (unsigned __int128)t[i].m;
    int tp = t[i].e + bitlen128(a);
    if (t[i].e < emin) emin = t[i].e;
    if (tp > top) top = tp;
  }
  if (emin == (1 << 30)) { *outm = 0; *oute = 0; return; }
  int eacc = emin;
  if (top - eacc > 120) eacc = top - 120;
  i128 acc = 0;
  for (int i = 0; i < n; ++i) {
    if (t[i].m == 0) continue;
    int sh = t[i].e - eacc;
    if (sh >= 0) {
      unsigned __int128 a = t[i].m < 0 ? (unsigned __int128)(-t[i].m) : (unsigned __int128)t[i].m;
      a <<= sh;
      acc += t[i].m < 0 ? -(i128)a : (i128)a;
    } else {
      unsigned __int128 a = t[i].m < 0 ? (unsigned __int128)(-t[i].m) : (unsigned __int128)t[i].m;
      unsigned __int128 q = (-sh >= 127) ? 0 : (a >> (-sh));
      int sticky = (-sh >= 127) ? (a != 0) : ((q << (-sh)) != a);
      q = q | (unsigned __int128)sticky;
      acc += t[i].m < 0 ? -(i128)q : (i128)q;
    }
  }
  *outm = acc;
  *oute = eacc;
}

/* value m*2^e rounded to double (RNE) */
static double i128_to_double(i128 m, int e) {
  if (m == 0) return 0.0;
  int neg = m < 0;
  unsigned __int128 a = neg ? (unsigned __int128)(-m) : (unsigned __int128)m;
  int n = bitlen128(a);
  if (n > 53) {
    int sh = n - 53;
    unsigned __int128 q = a >> sh;
    unsigned __int128 rem = a - (q << sh);
    unsigned __int128 half = (unsigned __int128)1 << (sh - 1);
    if (rem > half || (rem == half && (q & 1))) q += 1;
    a = q;
    e += sh;
  }
  double v = ldexp((double)(uint64_t)a, e);
  return neg ? -v : v;
}

/* value m*2^e rounded to binary32 (RNE): round-to-odd at 53 bits, then RNE to 24 */
static float i128_to_float(i128 m, int e) {
  if (m == 0) return 0.0f;
  int neg = m < 0;
  unsigned __int128 a = neg ? (unsigned __int128)(-m) : (unsigned __int128)m;
  int n = bitlen128(a);
  if (n > 53) {
    int sh = n - 53;
    unsigned __int128 q = a >> sh;
    if ((q << sh) != a) q |= 1;
    a = q;
    e += sh;
  }
  double v = ldexp((double)(uint64_t)a, e); /* exact */
  float f = (float)v;                      /* one RNE rounding */
  return neg ? -f : f;
}

/* exact decomposition of a finite double as m * 2^e */
static term_t double_term(double x) {
  term_t t = {0, 0};
  if (x == 0.0) return t;
  int e;
  double m = frexp(x, &e);
  /* m in [0.5,1): scale to a 53-bit integer */
  int64_t mi = (int64_t)ldexp(m, 53);
  t.m = mi;
  t.e = e - 53;
  return t;
}

/* decoded MX row: integer element values and per-block exponent offsets */
typedef struct {
  int D;
  int elem;
  int64_t* mint;  /* [D] */
  int* bexp;      /* [D/32]: scale - 127 + lsb */
  int bad;        /* NaN scale present */
} mxrow_t;

static void decode_row(int elem, const uint8_t* codes, const uint8_t* scales, int D, int64_t* mint, int* bexp,
                       int* bad) {
  int bb = fso_block_bytes(elem);
  *bad = 0;
  for (int g = 0; g < D / 32; ++g) {
    if (scales[g] == 255) *bad = 1;
    bexp[g] = (int)scales[g] - 127 + elem_lsb(elem);
    for (int j = 0; j < 32; ++j) mint[g * 32 + j] = elem_mint(elem, unpack_code(elem, codes + g * bb, j));
  }
}

/* exact Q-hat . K-hat as terms (one per block) */
static int dot_terms(const int64_t* qm, const int* qe, const int64_t* km, const int* ke, int D, term_t* out) {
  int nb = D / 32;
  for (int g = 0; g < nb; ++g) {
    i128 s = 0;
    for (int j = 0; j < 32; ++j) s += (i128)qm[g * 32 + j] * (i128)km[g * 32 + j];
    out[g].m = s;
    out[g].e = qe[g] + ke[g];
  }
  return nb;
}

/* max_d |Qhat_d Khat_d| in binary64 (a diagnostic magnitude, not a score) */
static double max_prod(const int64_t* qm, const int* qe, const int64_t* km, const int* ke, int D) {
  double s = 0.0;
  for (int g = 0; g < D / 32; ++g)
    for (int j = 0; j < 32; ++j) {
      const double x = ldexp(fabs((double)qm[g * 32 + j] * (double)km[g * 32 + j]), qe[g] + ke[g]);
      if (x > s) s = x;
    }
  return s;
}

double fso_folded_score(int qk_elem, const uint8_t* qrow_codes, const uint8_t* qrow_scales,
                        const uint8_t* krow_codes, const uint8_t* krow_scales, int D, double cinit,
                        int exact_fold) {
  int64_t qm[512], km[512];
  int qe[16], ke[16], bq, bk;
  if (D > 512 || D % 32) return NAN;
  decode_row(qk_elem, qrow_codes, qrow_scales, D, qm, qe, &bq);
  decode_row(qk_elem, krow_codes, krow_scales, D, km, ke, &bk);
  if (bq || bk) return NAN;
  term_t t[17];
  int n = dot_terms(qm, qe, km, ke, D, t);
  if (exact_fold) {
    i128 m;
    int e;
    exact_sum(t, n, &m, &e);
    return i128_to_double(m, e) + cinit;
  }
  t[n++] = double_term(cinit);
  i128 m;
  int e;
  exact_sum(t, n, &m, &e);
  return (double)i128_to_float(m, e);
}

/* ------------------------------------------------------------------------ */
/* Schraudolph stage 1 (R7) and stage 2 (R10-R13)                            */
/* ------------------------------------------------------------------------ */

static uint16_t stage1_d(double t) {
  if (!(t >= 128.0)) return 0;
  double f = floor(t);
  if (f > 32639.0) return 0x7F7F;
  return (uint16_t)f;
}

uint16_t fso_stage1(float t) {
  /* Schraudolph's exponential: the integer part of 128*(y+127) - c is the
   * BF16 bit pattern of ~2^y (7-bit mantissa, 8-bit biased exponent)
   * [FS-news 6].  floor, flush exponent-field-0 patterns, clamp to the
   * largest finite BF16. */
  return stage1_d((double)t);
}

/* ------------------------------------------------------------------------ */
/* EFQ-style direct E2M1 P (R24)                                             */
/* ------------------------------------------------------------------------ */

/* One P block of 32 keys from its folded fp32 scores t[0..nvis) (the other
 * keys of the block are absent and get code 0) ["EFQ-Softmax: Exp-Free
 * Quantization for Softmax", sections II.B-C and III.B]:
 *  - the shifted score of key k in log2 units is l_k = (t_k - T0) / 128 (the
 *    fold maps the reference to T0);
 *  - exponent-only block scale from the local maximum: E = floor(l_max),
 *    clamped to [-1000, 1000]; E8M0 = E - 2 + 127 clamped to [0, 254]
 *    (E2M1's top binade is 2^2);
 *  - residual r_k = l_k - E, and codes from uniformly spaced thresholds
 *    tau + j h (j = 1..7): code = #{ j : r_k >= tau + j h }, i.e.
 *    clamp(floor((r_k - tau) / h), 0, 7); code 7 is E2M1's 6.0.
 * tau and h are the binary32 parameters of the call.  Every step is exact in
 * binary64: t_k, T0 are binary32, so t_k - T0, the division by 128, E and
 * r_k are exact, and tau + j h (j <= 7) needs at most 28 significant bits.
 * The values of the block are code value * 2^(E8M0 - 127). */
static void efq_block(const float* t, int nvis, float T0, float tau, float h, uint8_t* codes, uint8_t* scale) {
  for (int i = 0; i < 32; ++i) codes[i] = 0;
  *scale = 0;
  if (nvis <= 0) return;
  float tb = t[0];
  for (int i = 1; i < nvis; ++i)
    if (t[i] > tb) tb = t[i];
  double E = floor(((double)tb - (double)T0) / 128.0);
  if (E < -1000.0) E = -1000.0;
  if (E > 1000.0) E = 1000.0;
  const int s = (int)E - 2 + 127;
  *scale = (uint8_t)(s < 0 ? 0 : (s > 254 ? 254 : s));
  for (int i = 0; i < nvis; ++i) {
    const double r = ((double)t[i] - (double)T0) / 128.0 - E;
    int code = 0;
    for (int j = 1; j <= 7; ++j)
      if (r >= (double)tau + (double)j * (double)h) code = j;
    codes[i] = (uint8_t)code;
  }
}

void fso_efq_block(const float* t, int nvis, float T0, double tau, double h, uint8_t* codes, uint8_t* scale) {
  efq_block(t, nvis, T0, (float)tau, (float)h, codes, scale);
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver                                                       */
/* ------------------------------------------------------------------------ */

typedef struct {
  const fso_params* p;
  const fso_mask* mask; /* NULL: no mask */
  int ref; /* 0 = fused forward, else FSO_REF_* */
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  const int64_t* rows;
  int64_t nrows;
  double* O;
  double* L;
  int32_t* counts;
  int32_t* misses; /* R25: per row, tiles the exact rule fires and the shortcut does not */
  uint8_t* pcodes;
  uint8_t* pscales;
  float* tout;   /* diagnostics: folded scores after the gate shift [rows][S32] */
  double* aout;  /* diagnostics: max_d |Qhat_d Khat_d| [rows][S32] */
  /* per-head decoded K/V, shared read-only */
  int64_t head;  /* (b*H + h) */
  int64_t* kmint; /* [Skv][D] */
  int* kbexp;     /* [Skv][D/32] */
  double* vval;   /* [Skv32][D] (key-major) */
  int kvbad;
  /* row indices (into rows[]) handled for this head */
  int64_t* idx;
  int64_t nidx;
  int64_t next;
  pthread_mutex_t mu;
} job_t;

static int64_t skv32_of(const fso_params* p) { return ((int64_t)p->Skv + 31) / 32 * 32; }

static void decode_head(job_t* J, int64_t head) {
  const fso_params* p = J->p;
  int D = p->D;
  int64_t Skv = p->Skv, S32 = skv32_of(p);
  int qbb = fso_block_bytes(p->qk_elem), vbb = fso_block_bytes(p->v_elem);
  int nbd = D / 32;
  J->kvbad = 0;
  for (int64_t k = 0; k < Skv; ++k) {
    int bad;
    const uint8_t* kc = J->kc + ((head * Skv + k) * nbd) * qbb;
    const uint8_t* ks = J->ks + (head * Skv + k) * nbd;
    decode_row(p->qk_elem, kc, ks, D, J->kmint + k * D, J->kbexp + k * nbd, &bad);
    if (bad) J->kvbad = 1;
  }
  int64_t nbk = S32 / 32;
  for (int d = 0; d < D; ++d)
    for (int64_t g = 0; g < nbk; ++g) {
      int sc = J->vs[((int64_t)head * D + d) * nbk + g];
      const uint8_t* blk = J->vc + (((int64_t)head * D + d) * nbk + g) * vbb;
      for (int j = 0; j < 32; ++j) {
        double v = (sc == 255) ? NAN : ldexp(fso_decode(p->v_elem, unpack_code(p->v_elem, blk, j)), sc - 127);
        J->vval[(g * 32 + j) * D + d] = v;
      }
    }
}

/* value of a BF16 bit pattern */
static double bf16_val(uint16_t b) { return bf16_to_double(b); }

/* scores of one row against all keys: exact sums as terms, reduced per mode */
typedef struct {
  int64_t* qm;
  int qe[16];
  double* tmp;     /* [Skv] */
  double* pv;      /* [S32] probabilities / values before P quantization */
  double* ph;      /* [S32] quantized P values */
  uint8_t* pc;     /* [S32] codes */
  uint8_t* psc;    /* [S32/32] */
} rowbuf_t;

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* last key row `row` may see (-1: none), from the mask (fso_mask) */
static int64_t last_visible_key(int64_t Sq, int64_t Skv, int64_t H, const fso_mask* m, int64_t row) {
  int64_t head = row / Sq, b = head / H, i = row % Sq;
  int64_t qlen = Sq, kvlen = Skv;
  if (m && m->q_lens) qlen = clamp64(m->q_lens[b], 0, Sq);
  if (m && m->kv_lens) kvlen = clamp64(m->kv_lens[b], 0, Skv);
  if (i >= qlen) return -1;
  int64_t lim = kvlen - 1;
  if (m && m->causal && i + kvlen - qlen < lim) lim = i + kvlen - qlen;
  return lim < -1 ? -1 : lim;
}

/* The gate decision of a tile with maximum tmax (tiles j >= 1).  Exact rule
 * (R1, R4): tmax > T_gate.  Shortcut (R25): the fastest 4-bit kernel of the
 * pages gates through a shortcut that can miss a recovery trigger in an
 * extreme-score range ["Fused-Softmax shifts an AI attention bottleneck onto
 * faster GPU hardware", paragraph 12]; the pages do not describe it.  The
 * reading here: the decision is taken on the stage-1 BF16 patterns the
 * two-stage conversion produces anyway, stage1(tmax) > floor(T_gate).  It
 * misses (a) tiles whose max lies in (T_gate, floor(T_gate) + 1), less than
 * one pattern step above the threshold, and (b) every tile once
 * floor(T_gate) >= 0x7F7F, where the clamped pattern cannot exceed it. */
static int gate_fires(const fso_params* p, double tmax, double Tg, int32_t* miss) {
  const int exact_fire = tmax > Tg;
  if (p->gate_mode != FSO_GATE_PATTERN) return exact_fire;
  const int fire = (double)stage1_d(tmax) > floor(Tg);
  if (exact_fire && !fire) ++*miss;
  return fire;
}

static void fused_row(job_t* J, int64_t ri, rowbuf_t* rb) {
  const fso_params* p = J->p;
  int D = p->D, nbd = D / 32;
  int64_t S32 = skv32_of(p);
  int64_t row = J->rows ? J->rows[ri] : ri;
  int64_t head = row / p->Sq;
  /* keys [0, Skv) are visible: a masked row sees a prefix of the keys */
  int64_t Skv = last_visible_key(p->Sq, p->Skv, p->H, J->mask, row) + 1;
  int qbb = fso_block_bytes(p->qk_elem);
  int bad;
  decode_row(p->qk_elem, J->qc + (row * nbd) * qbb, J->qs + row * nbd, D, rb->qm, rb->qe, &bad);
  double* O = J->O + ri * D;
  for (int d = 0; d < D; ++d) O[d] = 0.0;
  double l = 0.0;
  int32_t cnt = 0, miss = 0;
  memset(rb->pc, 0, (size_t)S32);
  memset(rb->psc, 0, (size_t)(S32 / 32));
  if (Skv == 0) {
    /* no visible key: O = 0, l = 0 */
    if (J->L) J->L[ri] = 0.0;
    if (J->counts) J->counts[ri] = 0;
    if (J->misses) J->misses[ri] = 0;
    if (J->pcodes) memset(J->pcodes + ri * S32, 0, (size_t)S32);
    if (J->pscales) memset(J->pscales + ri * (S32 / 32), 0, (size_t)(S32 / 32));
    return;
  }
  const int exact = (p->fold_mode == FSO_FOLD_EXACT);
  /* T0 = 128*127 - c maps the reference to 2^0; T_gate = T0 + 128*tau (R1, R6) */
  double T0 = exact ? (128.0 * 127.0 - p->c) : (double)(float)(128.0 * 127.0 - p->c);
  double Tg = exact ? (128.0 * (127.0 + p->tau) - p->c) : (double)(float)(128.0 * (127.0 + p->tau) - p->c);
  double C = 0.0; /* accumulator initial value (the frozen reference, folded) */
  int bc = p->kv_tile;
  int64_t ntiles = (Skv + bc - 1) / bc;
  term_t tt[17];
  for (int64_t j = 0; j < ntiles; ++j) {
    int64_t k0 = j * bc, k1 = k0 + bc < Skv ? k0 + bc : Skv;
    double tmax = -INFINITY;
    for (int64_t k = k0; k < k1; ++k) {
      int n = dot_terms(rb->qm, rb->qe, J->kmint + k * D, J->kbexp + k * nbd, D, tt);
      double t;
      if (j == 0) {
        /* tile 0: plain scores, reference from their max (R2) */
        i128 m;
        int e;
        exact_sum(tt, n, &m, &e);
        t = exact ? i128_to_double(m, e) : (double)i128_to_float(m, e);
      } else if (exact) {
        i128 m;
        int e;
        exact_sum(tt, n, &m, &e);
        t = C + i128_to_double(m, e);
      } else {
        /* folded product: accumulator starts at C, one fp32 rounding (R8, R9) */
        tt[n++] = double_term(C);
        i128 m;
        int e;
        exact_sum(tt, n, &m, &e);
        t = (double)i128_to_float(m, e);
      }
      rb->tmp[k] = t;
      if (t > tmax) tmax = t;
    }
    if (j == 0) {
      /* frozen reference (R2): the row max maps to T0 */
      C = exact ? (T0 - tmax) : (double)(float)(T0 - tmax);
      for (int64_t k = k0; k < k1; ++k) rb->tmp[k] = exact ? rb->tmp[k] + C : (double)(float)(rb->tmp[k] + C);
    } else if (gate_fires(p, tmax, Tg, &miss)) {
      /* rollback gate (R1, R3, R4, R5) [FS-news 5]: shift that brings this
       * tile's max back to T0 */
      double delta = exact ? (tmax - T0) : (double)(float)(tmax - T0);
      for (int64_t k = k0; k < k1; ++k)
        rb->tmp[k] = exact ? rb->tmp[k] - delta : (double)(float)(rb->tmp[k] - delta);
      C = exact ? C - delta : (double)(float)(C - delta);
      double rho = exp2(-delta / 128.0);
      for (int d = 0; d < D; ++d) O[d] *= rho;
      l *= rho;
      ++cnt;
    }
    if (J->tout) {
      /* diagnostics: the scores stage 1 sees and their largest products */
      for (int64_t k = k0; k < k1; ++k) {
        J->tout[ri * S32 + k] = (float)rb->tmp[k];
        J->aout[ri * S32 + k] = max_prod(rb->qm, rb->qe, J->kmint + k * D, J->kbexp + k * nbd, D);
      }
    }
    /* stage 1: folded score -> BF16 pattern (or the exact exponential); the
     * P blocks of the tile run to its end (to S32 on the last tile of the
     * keys), absent keys giving 0 */
    int64_t kb0 = k0, kb1 = k0 + bc < S32 ? k0 + bc : S32;
    if (p->p_mode == FSO_P_EFQ) {
      /* R24: codes straight from the folded scores, block by block */
      const float etau = (float)p->efq_tau, eh = (float)p->efq_h;
      for (int64_t g = kb0 / 32; g < kb1 / 32; ++g) {
        float tf[32];
        int64_t nv = Skv - g * 32;
        int nvis = nv <= 0 ? 0 : (nv >= 32 ? 32 : (int)nv);
        for (int i = 0; i < nvis; ++i) tf[i] = (float)rb->tmp[g * 32 + i];
        efq_block(tf, nvis, (float)T0, etau, eh, rb->pc + g * 32, rb->psc + g);
        for (int i = 0; i < 32; ++i)
          rb->ph[g * 32 + i] = ldexp(fso_decode(FSO_E2M1, rb->pc[g * 32 + i]), (int)rb->psc[g] - 127);
      }
    }
    for (int64_t k = kb0; k < kb1 && p->p_mode != FSO_P_EFQ; ++k) {
      double v = 0.0;
      if (k < Skv) {
        if (p->exp_mode == FSO_EXP_EXACT) v = exp2((rb->tmp[k] + p->c) / 128.0 - 127.0);
        else v = bf16_val(stage1_d(rb->tmp[k]));
      }
      rb->pv[k] = v;
    }
    /* stage 2: MX quantization of P per 32 consecutive keys (R12, R13) */
    for (int64_t g = kb0 / 32; g < kb1 / 32 && p->p_mode != FSO_P_EFQ; ++g) {
      if (p->p_mode == FSO_P_MX) {
        fso_mxq_block(p->p_elem, p->scale_rule, rb->pv + g * 32, 32, rb->pc + g * 32, rb->psc + g);
        for (int i = 0; i < 32; ++i)
          rb->ph[g * 32 + i] = ldexp(fso_decode(p->p_elem, rb->pc[g * 32 + i]), (int)rb->psc[g] - 127);
      } else {
        for (int i = 0; i < 32; ++i) rb->ph[g * 32 + i] = rb->pv[g * 32 + i];
        rb->psc[g] = 0;
        for (int i = 0; i < 32; ++i) rb->pc[g * 32 + i] = 0;
      }
    }
    /* O += P-hat V-hat ; l += P-hat 1 with the same P-hat [FS-news 6] */
    for (int64_t k = kb0; k < kb1; ++k) {
      double ph = rb->ph[k];
      if (ph == 0.0) continue;
      const double* vr = J->vval + k * D;
      for (int d = 0; d < D; ++d) O[d] += ph * vr[d];
      l += ph;
    }
  }
  for (int d = 0; d < D; ++d) O[d] /= l;
  if (J->L) J->L[ri] = l;
  if (J->counts) J->counts[ri] = cnt;
  if (J->misses) J->misses[ri] = miss;
  if (J->pcodes) memcpy(J->pcodes + ri * S32, rb->pc, (size_t)S32);
  if (J->pscales) memcpy(J->pscales + ri * (S32 / 32), rb->psc, (size_t)(S32 / 32));
  (void)head;
}

/* references on quantized operands: s_k = sum_k / 128 in log2 units */
static void reference_row(job_t* J, int64_t ri, rowbuf_t* rb) {
  const fso_params* p = J->p;
  int D = p->D, nbd = D / 32;
  int64_t Skv = p->Skv, S32 = skv32_of(p);
  int64_t row = J->rows ? J->rows[ri] : ri;
  int qbb = fso_block_bytes(p->qk_elem);
  int bad;
  decode_row(p->qk_elem, J->qc + (row * nbd) * qbb, J->qs + row * nbd, D, rb->qm, rb->qe, &bad);
  term_t tt[17];
  for (int64_t k = 0; k < Skv; ++k) {
    int n = dot_terms(rb->qm, rb->qe, J->kmint + k * D, J->kbexp + k * nbd, D, tt);
    i128 m;
    int e;
    exact_sum(tt, n, &m, &e);
    rb->tmp[k] = i128_to_double(m, e) / 128.0;
  }
  double* O = J->O + ri * D;
  for (int d = 0; d < D; ++d) O[d] = 0.0;
  double l = 0.0;
  if (J->ref == FSO_REF_R3) {
    int bc = p->kv_tile;
    double mrun = -INFINITY;
    for (int64_t k0 = 0; k0 < Skv; k0 += bc) {
      int64_t k1 = k0 + bc < Skv ? k0 + bc : Skv;
      int64_t kb1 = (k1 == Skv) ? S32 : k1;
      double mt = -INFINITY;
      for (int64_t k = k0; k < k1; ++k) if (rb->tmp[k] > mt) mt = rb->tmp[k];
      double mnew = mt > mrun ? mt : mrun;
      if (mrun != -INFINITY && mnew > mrun) {
        double r = exp2(mrun - mnew);
        for (int d = 0; d < D; ++d) O[d] *= r;
        l *= r;
      }
      mrun = mnew;
      for (int64_t k = k0; k < kb1; ++k) rb->pv[k] = (k < Skv) ? exp2(rb->tmp[k] - mrun) : 0.0;
      for (int64_t g = k0 / 32; g < kb1 / 32; ++g) {
        fso_mxq_block(p->p_elem, p->scale_rule, rb->pv + g * 32, 32, rb->pc + g * 32, rb->psc + g);
        for (int i = 0; i < 32; ++i)
          rb->ph[g * 32 + i] = ldexp(fso_decode(p->p_elem, rb->pc[g * 32 + i]), (int)rb->psc[g] - 127);
      }
      for (int64_t k = k0; k < kb1; ++k) {
        double ph = rb->ph[k];
        if (ph == 0.0) continue;
        for (int d = 0; d < D; ++d) O[d] += ph * J->vval[k * D + d];
        l += ph;
      }
    }
  } else {
    double m = -INFINITY;
    for (int64_t k = 0; k < Skv; ++k) if (rb->tmp[k] > m) m = rb->tmp[k];
    for (int64_t k = 0; k < S32; ++k) rb->pv[k] = (k < Skv) ? exp2(rb->tmp[k] - m) : 0.0;
    if (J->ref == FSO_REF_R1) {
      for (int64_t k = 0; k < S32; ++k) rb->ph[k] = rb->pv[k];
    } else {
      for (int64_t g = 0; g < S32 / 32; ++g) {
        fso_mxq_block(p->p_elem, p->scale_rule, rb->pv + g * 32, 32, rb->pc + g * 32, rb->psc + g);
        for (int i = 0; i < 32; ++i)
          rb->ph[g * 32 + i] = ldexp(fso_decode(p->p_elem, rb->pc[g * 32 + i]), (int)rb->psc[g] - 127);
      }
    }
    for (int64_t k = 0; k < S32; ++k) {
      double ph = rb->ph[k];
      if (ph != 0.0)
        for (int d = 0; d < D; ++d) O[d] += ph * J->vval[k * D + d];
      l += (J->ref == FSO_REF_R2) ? rb->pv[k] : ph;
    }
  }
  for (int d = 0; d < D; ++d) O[d] /= l;
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const fso_params* p = J->p;
  int64_t S32 = skv32_of(p);
  rowbuf_t rb;
  rb.qm = (int64_t*)malloc(sizeof(int64_t) * (size_t)p->D);
  rb.tmp = (double*)malloc(sizeof(double) * (size_t)(p->Skv > 0 ? p->Skv : 1));
  rb.pv = (double*)malloc(sizeof(double) * (size_t)S32);
  rb.ph = (double*)malloc(sizeof(double) * (size_t)S32);
  rb.pc = (uint8_t*)malloc((size_t)S32);
  rb.psc = (uint8_t*)malloc((size_t)(S32 / 32 + 1));
  if (!rb.qm || !rb.tmp || !rb.pv || !rb.ph || !rb.pc || !rb.psc) abort();
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t t = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (t >= J->nidx) break;
    int64_t ri = J->idx[t];
    if (J->ref == 0) fused_row(J, ri, &rb);
    else reference_row(J, ri, &rb);
  }
  free(rb.qm); free(rb.tmp); free(rb.pv); free(rb.ph); free(rb.pc); free(rb.psc);
  return NULL;
}

static int check_params(const fso_params* p) {
  if (!p) return 0;
  if (p->B < 0 || p->H < 0 || p->Sq < 0 || p->Skv < 1 || p->D < 32 || p->D % 32 || p->D > 512) return 0;
  if (!valid_elem(p->qk_elem) || !valid_elem(p->v_elem) || !valid_elem(p->p_elem)) return 0;
  if (p->kv_tile < 32 || p->kv_tile % 32) return 0;
  if (!(p->tau >= 0.0)) return 0;
  if (p->p_mode == FSO_P_EFQ) {
    /* R24 takes the binary32 folded scores, with E2M1 P; h in [1/64, 16], |tau| <= 64 */
    if (p->p_elem != FSO_E2M1 || p->fold_mode != FSO_FOLD_FP32) return 0;
    if (!(p->efq_h >= 1.0 / 64.0 && p->efq_h <= 16.0) || !(p->efq_tau >= -64.0 && p->efq_tau <= 64.0)) return 0;
  } else if (p->p_mode != FSO_P_MX && p->p_mode != FSO_P_NONE) {
    return 0;
  }
  if (p->gate_mode != FSO_GATE_EXACT && p->gate_mode != FSO_GATE_PATTERN) return 0;
  return 1;
}

static int run_rows(const fso_params* p, const fso_mask* mask, int ref, const uint8_t* qc, const uint8_t* qs,
                    const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, const int64_t* rows,
                    int64_t nrows, double* out_O, double* out_l, int32_t* counts, uint8_t* pcodes,
                    uint8_t* pscales, float* tout, double* aout) {
  if (!check_params(p)) return FSO_EINVAL;
  int64_t total = (int64_t)p->B * p->H * p->Sq;
  if (!rows) nrows = total;
  for (int64_t i = 0; rows && i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= total) return FSO_EINVAL;
  if (nrows == 0) return FSO_OK;
  int D = p->D;
  int64_t Skv = p->Skv, S32 = skv32_of(p);
  job_t J;
  memset(&J, 0, sizeof J);
  J.p = p; J.mask = mask; J.ref = ref; J.qc = qc; J.qs = qs; J.kc = kc; J.ks = ks; J.vc = vc; J.vs = vs;
  J.rows = rows; J.nrows = nrows; J.O = out_O; J.L = out_l; J.counts = counts; J.pcodes = pcodes; J.pscales = pscales;
  J.tout = tout; J.aout = aout;
  J.misses = p->gate_misses;
  J.kmint = (int64_t*)malloc(sizeof(int64_t) * (size_t)(Skv * D));
  J.kbexp = (int*)malloc(sizeof(int) * (size_t)(Skv * (D / 32)));
  J.vval = (double*)malloc(sizeof(double) * (size_t)(S32 * D));
  J.idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)nrows);
  if (!J.kmint || !J.kbexp || !J.vval || !J.idx) {
    free(J.kmint); free(J.kbexp); free(J.vval); free(J.idx);
    return FSO_ENOMEM;
  }
  pthread_mutex_init(&J.mu, NULL);
  int nth = p->nthreads > 0 ? p->nthreads : fso_default_threads();
  /* process heads one at a time; rows of a head run in parallel */
  int64_t nheads = (int64_t)p->B * p->H;
  char* done = (char*)calloc((size_t)nrows, 1);
  for (int64_t h = 0; h < nheads; ++h) {
    J.nidx = 0;
    for (int64_t i = 0; i < nrows; ++i) {
      int64_t row = rows ? rows[i] : i;
      if (row / p->Sq == h) J.idx[J.nidx++] = i;
    }
    if (!J.nidx) continue;
    decode_head(&J, h);
    J.next = 0;
    int nt = nth < J.nidx ? nth : (int)J.nidx;
    pthread_t th[256];
    if (nt > 256) nt = 256;
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, worker, &J);
    for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  }
  free(done);
  pthread_mutex_destroy(&J.mu);
  free(J.kmint); free(J.kbexp); free(J.vval); free(J.idx);
  return FSO_OK;
}

int fso_forward(const fso_params* p, const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                const uint8_t* vc, const uint8_t* vs, const int64_t* rows, int64_t nrows, double* out_O,
                double* out_l, int32_t* counts, uint8_t* p_codes, uint8_t* p_scales) {
  return run_rows(p, NULL, 0, qc, qs, kc, ks, vc, vs, rows, nrows, out_O, out_l, counts, p_codes, p_scales, NULL,
                  NULL);
}

int fso_forward_masked(const fso_params* p, const fso_mask* m, const uint8_t* qc, const uint8_t* qs,
                       const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs,
                       const int64_t* rows, int64_t nrows, double* out_O, double* out_l, int32_t* counts,
                       uint8_t* p_codes, uint8_t* p_scales) {
  return run_rows(p, m, 0, qc, qs, kc, ks, vc, vs, rows, nrows, out_O, out_l, counts, p_codes, p_scales, NULL,
                  NULL);
}

int fso_forward_scores(const fso_params* p, const fso_mask* m, const uint8_t* qc, const uint8_t* qs,
                       const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vs,
                       const int64_t* rows, int64_t nrows, float* t_out, double* abs_out) {
  if (!t_out || !abs_out) return FSO_EINVAL;
  int64_t n = rows ? nrows : (int64_t)p->B * p->H * p->Sq;
  double* O = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)p->D);
  if (!O) return FSO_ENOMEM;
  int rc = run_rows(p, m, 0, qc, qs, kc, ks, vc, vs, rows, nrows, O, NULL, NULL, NULL, NULL, t_out, abs_out);
  free(O);
  return rc;
}

int fso_reference(const fso_params* p, int ref, const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                  const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, const int64_t* rows, int64_t nrows,
                  double* out_O) {
  if (ref < FSO_REF_R1 || ref > FSO_REF_R3) return FSO_EINVAL;
  return run_rows(p, NULL, ref, qc, qs, kc, ks, vc, vs, rows, nrows, out_O, NULL, NULL, NULL, NULL, NULL, NULL);
}

/* ------------------------------------------------------------------------ */
/* R0: exact softmax attention on the bf16 inputs                            */
/* ------------------------------------------------------------------------ */

typedef struct {
  int B, H, Sq, Skv, D;
  double sigma;
  const uint16_t *q, *k, *v;
  const int64_t* rows;
  int64_t nrows;
  double* O;
  const fso_mask* mask; /* NULL: no mask */
  int64_t next;
  pthread_mutex_t mu;
} r0_t;

static void* r0_worker(void* arg) {
  r0_t* R = (r0_t*)arg;
  int D = R->D;
  double* s = (double*)malloc(sizeof(double) * (size_t)R->Skv);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  if (!s || !qd) abort();
  for (;;) {
    pthread_mutex_lock(&R->mu);
    int64_t ri = R->next++;
    pthread_mutex_unlock(&R->mu);
    if (ri >= R->nrows) break;
    int64_t row = R->rows ? R->rows[ri] : ri;
    int64_t head = row / R->Sq;
    const uint16_t* qr = R->q + row * D;
    for (int d = 0; d < D; ++d) qd[d] = bf16_to_double(qr[d]);
    /* keys [0, nvis) are visible (the mask of fso_forward_masked) */
    const int64_t nvis = last_visible_key(R->Sq, R->Skv, R->H, R->mask, row) + 1;
    double* O = R->O + ri * D;
    for (int d = 0; d < D; ++d) O[d] = 0.0;
    if (nvis == 0) continue;
    double m = -INFINITY;
    for (int64_t k = 0; k < nvis; ++k) {
      const uint16_t* kr = R->k + (head * R->Skv + k) * D;
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += qd[d] * bf16_to_double(kr[d]);
      s[k] = acc * R->sigma;
      if (s[k] > m) m = s[k];
    }
    double l = 0.0;
    for (int64_t k = 0; k < nvis; ++k) {
      double pk = exp(s[k] - m);
      const uint16_t* vr = R->v + (head * R->Skv + k) * D;
      for (int d = 0; d < D; ++d) O[d] += pk * bf16_to_double(vr[d]);
      l += pk;
    }
    for (int d = 0; d < D; ++d) O[d] /= l;
  }
  free(s);
  free(qd);
  return NULL;
}

int fso_reference_bf16(int B, int H, int Sq, int Skv, int D, double sigma, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const int64_t* rows, int64_t nrows, int nthreads, double* out_O) {
  return fso_reference_bf16_masked(B, H, Sq, Skv, D, sigma, NULL, q, k, v, rows, nrows, nthreads, out_O);
}

int fso_reference_bf16_masked(int B, int H, int Sq, int Skv, int D, double sigma, const fso_mask* mask,
                              const uint16_t* q, const uint16_t* k, const uint16_t* v, const int64_t* rows,
                              int64_t nrows, int nthreads, double* out_O) {
  if (B < 0 || H < 0 || Sq < 0 || Skv < 1 || D < 1) return FSO_EINVAL;
  int64_t total = (int64_t)B * H * Sq;
  if (!rows) nrows = total;
  for (int64_t i = 0; rows && i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= total) return FSO_EINVAL;
  r0_t R;
  R.B = B; R.H = H; R.Sq = Sq; R.Skv = Skv; R.D = D; R.sigma = sigma; R.q = q; R.k = k; R.v = v;
  R.rows = rows; R.nrows = nrows; R.O = out_O; R.mask = mask; R.next = 0;
  pthread_mutex_init(&R.mu, NULL);
  int nt = nthreads > 0 ? nthreads : fso_default_threads();
  if (nt > nrows) nt = (int)(nrows > 0 ? nrows : 1);
  if (nt > 256) nt = 256;
  pthread_t th[256];
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, r0_worker, &R);
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&R.mu);
  return FSO_OK;
}
