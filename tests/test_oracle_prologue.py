"""Pins for the oracle's fused producer step (fso_quantize_mx_rmsnorm): RMS-
normalised Q/K rows with a per-feature weight, then the prescale and MX
quantization (reading R23, the ranked next step that fuses the normalisation
before the path into the quantizer).

Pins, each chosen so that a plausible mistake (wrong axis of the mean, a
missing square root, the weight or the prescale dropped or applied twice,
eps ignored, fp32 instead of binary64 accumulation) fails one:
  * independent recomputation in exact rational arithmetic (Fraction sums,
    correctly rounded binary64 root and reciprocal, explicit fl32 products)
    followed by the block quantizer (pinned in test_oracle_codec), on rows
    with a wide magnitude spread;
  * reduction to the plain quantizer: rows of +-1 have r = 1 (eps = 0), so
    the result equals fso_quantize_mx of +-w with the same prescale;
  * scale invariance: x and 2^k x give identical codes and scales (eps = 0);
  * closed forms: a zero row stays zero (codes 0, scale 0) for any eps; a
    constant row of c = 2^j gives y = +-1 exactly.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.test_oracle_codec import _unpack

ELEMS = [0, 2, 4]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32)


def expected_row(xf: np.ndarray, w, eps: float, pre: float) -> np.ndarray:
    """fl32(pre * fl32(fl32(x r) w)) with r from the exact sum of squares."""
    cols = xf.size
    ss = float(sum(Fraction(float(v)) ** 2 for v in xf))  # exact, then one rounding to binary64
    a = ss / cols + float(np.float32(eps))
    r = np.float32(0.0) if a == 0.0 else np.float32(1.0 / math.sqrt(a))
    y = (xf.astype(np.float32) * r).astype(np.float32)
    if w is not None:
        y = (y * w.astype(np.float32)).astype(np.float32)
    return (np.float32(pre) * y).astype(np.float32)


@pytest.mark.parametrize("e", ELEMS)
@pytest.mark.parametrize("cols,use_w", [(64, False), (128, True)])
@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_rmsnorm_matches_exact_recomputation(oracle, e, cols, use_w, eps):
    rng = np.random.default_rng(100 + e + cols)
    n_mat, rows = 2, 23
    x = (rng.standard_normal((n_mat, rows, cols)) * np.exp(rng.uniform(-4, 4, (n_mat, rows, 1)))
         * np.exp(rng.uniform(-2, 2, (n_mat, rows, cols)))).astype(np.float32)
    u = bf16_bits(x)
    xf = bits_to_f32(u)
    w = rng.uniform(0.5, 2.0, cols).astype(np.float32) if use_w else None
    pre = 16.322231
    codes, scales = oracle.quantize_mx_rmsnorm(u, e, prescale=pre, weight=w, eps=eps)
    bb = oracle.block_bytes(e)
    for m in range(n_mat):
        for r in range(rows):
            vals = expected_row(xf[m, r], w, eps, pre)
            for g in range(cols // 32):
                c_exp, s_exp = oracle.mxq_block(e, 0, vals[g * 32:(g + 1) * 32].astype(np.float64))
                assert scales[m, r, g] == s_exp, (m, r, g)
                assert _unpack(codes[m, r, g * bb:(g + 1) * bb], e, 32) == list(c_exp), (m, r, g)


@pytest.mark.parametrize("e", ELEMS)
def test_unit_rows_reduce_to_plain_quantizer(oracle, e):
    """Rows of +-1: ss = cols, r = 1 exactly, so y = +-w."""
    rng = np.random.default_rng(7 + e)
    cols = 128
    signs = rng.choice([-1.0, 1.0], size=(1, 9, cols)).astype(np.float32)
    w = bits_to_f32(bf16_bits(rng.uniform(0.25, 3.0, cols).astype(np.float32)))  # bf16-exact weights
    pre = 5.770780
    a = oracle.quantize_mx_rmsnorm(bf16_bits(signs), e, prescale=pre, weight=w, eps=0.0)
    b = oracle.quantize_mx(bf16_bits(signs * w), 0, e, prescale=pre)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("e", ELEMS)
@pytest.mark.parametrize("k", [-7, 5])
def test_scale_invariance(oracle, e, k):
    rng = np.random.default_rng(31 + e)
    x = rng.standard_normal((2, 11, 64)).astype(np.float32)
    u = bf16_bits(x)
    u2 = bf16_bits(bits_to_f32(u) * np.float32(2.0 ** k))  # exact power-of-two scaling of bf16 values
    w = rng.uniform(0.5, 2.0, 64).astype(np.float32)
    a = oracle.quantize_mx_rmsnorm(u, e, prescale=3.0, weight=w, eps=0.0)
    b = oracle.quantize_mx_rmsnorm(u2, e, prescale=3.0, weight=w, eps=0.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("e", ELEMS)
def test_closed_forms(oracle, e):
    cols = 64
    zero = np.zeros((1, 2, cols), np.uint16)
    for eps in (0.0, 1e-6):
        c, s = oracle.quantize_mx_rmsnorm(zero, e, eps=eps)
        assert not c.any() and not s.any()
    # constant row c = 2^-3: r = 2^3 exactly (eps = 0), y = +-1, block max 1
    x = np.full((1, 1, cols), 0.125, np.float32)
    x[0, 0, ::3] *= -1
    c, s = oracle.quantize_mx_rmsnorm(bf16_bits(x), e, eps=0.0)
    ones = np.sign(x).astype(np.float64).ravel()
    for g in range(cols // 32):
        c_exp, s_exp = oracle.mxq_block(e, 0, ones[g * 32:(g + 1) * 32])
        bb = oracle.block_bytes(e)
        assert s[0, 0, g] == s_exp
        assert _unpack(c[0, 0, g * bb:(g + 1) * bb], e, 32) == list(c_exp)
