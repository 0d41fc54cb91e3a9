"""Pins of the oracle's reference outputs and of its Schraudolph shift c.

"Fused softmax makes quantized attention faster on AMD GPUs", section "The
research", and "Fused-Softmax shifts an AI attention bottleneck onto faster
GPU hardware", paragraph 7: the fused softmax adds at most about 0.3
percentage points of error beyond operand quantization, measured against
conventional softmax on the same quantized operands.  The oracle's readings
of that comparison point (exact softmax of the quantized scores):
  R1   P unquantized;
  R2   numerator with P quantized like the method's P (MX, 32 consecutive keys
       per block), denominator the unquantized sum;
  R2'  numerator and denominator both with the quantized P.
Each is checked against an independent exact-rational evaluation
(tests/spec_numpy.py), and the cases are chosen so that R1, R2 and R2' are
far apart: a denominator taken from the wrong sum fails.

The Schraudolph shift c ("Fused-Softmax shifts ...", paragraph 6) is pinned
by the closed-form band of the shifted stage 1 and by the exact-rational
forward run with c != 0, which fixes the sign and the units of c in the
reference T0 and the gate threshold.
"""
import math
import zlib

import numpy as np
import pytest
import torch

from tests import spec_numpy as spec


def bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def quantize_head(O, q, k, v, sigma, qk, ve):
    Sq, D = q.shape
    Skv = k.shape[0]
    Q = O.quantize_mx(bits(q).reshape(1, Sq, D), 0, qk, prescale=O.softmax_scale_prescale(sigma))
    K = O.quantize_mx(bits(k).reshape(1, Skv, D), 0, qk)
    V = O.quantize_mx(bits(v).reshape(1, Skv, D), 1, ve)
    return Q, K, V


# (name, Sq, Skv, D, qk, v, p, key scale): ragged key counts so that the last
# P block is padded; a key scale of 3 spreads the scores over several binades
REF_CASES = [
    ("fp6", 3, 70, 32, 2, 2, 2, 3.0),
    ("fp8", 3, 45, 32, 0, 0, 0, 3.0),
    ("fp4-p6", 2, 96, 64, 4, 4, 2, 2.0),
    ("fp6-p8", 2, 33, 32, 2, 2, 0, 4.0),
]


@pytest.mark.parametrize("case", REF_CASES, ids=[c[0] for c in REF_CASES])
def test_references_match_exact_spec(oracle, case):
    name, Sq, Skv, D, qk, ve, pe, ks = case
    seed = zlib.crc32(name.encode()) % 1000
    q = rand_bf16((Sq, D), seed)
    k = rand_bf16((Skv, D), seed + 1, ks)
    v = rand_bf16((Skv, D), seed + 2)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_head(oracle, q, k, v, sigma, qk, ve)
    p = oracle.make_params(1, 1, Sq, Skv, D, qk, ve, pe)
    want = spec.references(bits(q), bits(k), bits(v), sigma, qk, ve, pe)
    got = {"R1": oracle.reference(p, oracle.REF_R1, Q, K, V),
           "R2": oracle.reference(p, oracle.REF_R2, Q, K, V),
           "R2'": oracle.reference(p, oracle.REF_R2P, Q, K, V)}
    for r in ("R1", "R2", "R2'"):
        np.testing.assert_allclose(got[r], want[r], rtol=1e-12, atol=1e-13, err_msg=r)
    # the three readings differ by far more than the tolerance on these cases
    def rel(a, b):
        return np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(want["R2"], want["R2'"]) > 1e-4
    assert rel(want["R2"], want["R1"]) > 1e-4


# ---------------------------------------------------------------- Schraudolph shift c

C_RMS = 60801 / 8192  # Schraudolph's RMS-optimal shift, 60801 / 2^20 of an exponent step, in BF16 pattern units


def test_shifted_stage1_band(oracle):
    """With the folded map t = fl32(128 (y + 127) - c), stage 1 gives
    approx(y) / 2^y = 2^(-c/128) (1 + floor(128 f)/128) 2^(-f), f = frac(y - c/128):
    for c = 60801/8192 the band is [0.955417, 1.019657], attained (sup) and
    approached (inf)."""
    hi_b = max(2.0 ** (-C_RMS / 128) * (1 + j / 128) * 2.0 ** (-j / 128) for j in range(128))
    assert abs(hi_b - 1.019657) < 1e-6
    assert abs(2.0 ** (-C_RMS / 128) * 2.0 ** (-1 / 128) - 0.955417) < 1e-6
    rng = np.random.default_rng(3)
    ys = np.concatenate([rng.uniform(-120.0, 20.0, 20000),
                         np.arange(-120, 20) + (57 + C_RMS) / 128.0,
                         np.arange(-120, 20) + (127.999 + C_RMS) / 128.0])
    ratios = []
    for y in ys:
        t = float(np.float32(128.0 * (y + 127.0) - C_RMS))
        b = oracle.stage1(t)
        approx = float(spec.bf16_value(b))
        ratios.append(approx / 2.0 ** ((t + C_RMS) / 128.0 - 127.0))
    ratios = np.array(ratios)
    assert ratios.min() >= 0.955417 * (1 - 1e-6)
    assert ratios.max() <= 1.019657 * (1 + 1e-6)
    assert ratios.max() == pytest.approx(1.019657, abs=2e-6)
    assert ratios.min() == pytest.approx(0.955417, abs=2e-4)


C_CASES = [
    # (name, Sq, Skv, D, qk, v, p, kv_tile, stress rows, tau)
    ("fp6-c", 4, 130, 32, 2, 2, 2, 64, (3, 70, 100, 120), 8.0),
    ("fp8-c", 5, 100, 32, 0, 0, 0, 32, (40, 90), 8.0),
    ("fp4-c-tau1", 4, 96, 32, 4, 4, 2, 32, (50,), 1.0),
]


@pytest.mark.parametrize("case", C_CASES, ids=[c[0] for c in C_CASES])
def test_forward_with_shift_matches_exact_spec(oracle, case):
    name, Sq, Skv, D, qk, ve, pe, bc, stress, tau = case
    seed = zlib.crc32(name.encode()) % 1000
    q = rand_bf16((Sq, D), seed)
    k = rand_bf16((Skv, D), seed + 1).float()
    for r in stress:
        k[r] *= 8.0
    k = k.to(torch.bfloat16)
    v = rand_bf16((Skv, D), seed + 2)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_head(oracle, q, k, v, sigma, qk, ve)
    p = oracle.make_params(1, 1, Sq, Skv, D, qk, ve, pe, tau=tau, c=C_RMS, kv_tile=bc)
    r = oracle.forward(p, Q, K, V, want_p=True)
    O_s, cnt_s, pc_s, ps_s = spec.forward(bits(q), bits(k), bits(v), sigma, qk, ve, pe, tau=tau, kv_tile=bc,
                                          c=C_RMS)
    assert np.array_equal(r["counts"], cnt_s)
    assert np.array_equal(r["p_codes"].astype(np.int64), pc_s)
    assert np.array_equal(r["p_scales"].astype(np.int64), ps_s)
    np.testing.assert_allclose(r["O"], O_s, rtol=1e-12, atol=1e-12)
    assert cnt_s.sum() > 0
    # and c moves the P codes (the shift is not a no-op)
    p0 = oracle.make_params(1, 1, Sq, Skv, D, qk, ve, pe, tau=tau, c=0.0, kv_tile=bc)
    r0 = oracle.forward(p0, Q, K, V, want_p=True)
    assert not np.array_equal(r0["p_codes"], r["p_codes"])


def test_shift_cancels_with_exact_exponential(oracle):
    """c enters the reference T0 and the exponent's offset together: with the
    exact exponential, unquantized P and the exact fold, O does not depend on c."""
    D, Sq, Skv = 64, 12, 150
    q = rand_bf16((Sq, D), 5)
    k = rand_bf16((Skv, D), 6, 3.0)
    v = rand_bf16((Skv, D), 7)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_head(oracle, q, k, v, sigma, 2, 2)
    outs = []
    for c in (0.0, C_RMS, -40.5):
        p = oracle.make_params(1, 1, Sq, Skv, D, 2, 2, 2, tau=2.0, c=c, kv_tile=32, exp_mode=oracle.EXP_EXACT,
                               p_mode=oracle.P_NONE, fold_mode=oracle.FOLD_EXACT)
        outs.append(oracle.forward(p, Q, K, V)["O"])
    np.testing.assert_allclose(outs[1], outs[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(outs[2], outs[0], rtol=1e-12, atol=1e-13)
