"""Pins for the oracle's Fused-Softmax forward pass.

Method: "Fused-Softmax shifts an AI attention bottleneck onto faster GPU
hardware", paragraphs 5-6 (frozen reference folded into the score product,
Schraudolph exponential folded likewise, two-stage BF16 -> MX conversion of P,
P.1 denominator with the same P, rollback when scores exceed the reference by
more than a threshold).

Pins here, each chosen so that a plausible mistake fails one of them:
  * Schraudolph stage 1 against closed-form bounds of 2^y and of exp(x);
  * tiny brute force against an independent exact-rational implementation
    (tests/spec_numpy.py): P codes, scales and rollback counts bit-exact,
    O to 1e-12, across several tiles, ragged tails and planted rollbacks;
  * invariants: exact exponential + unquantized P + exact fold equals exact
    softmax of the quantized scores for any tau (shift invariance); tau = 0
    equals FlashAttention's running-max recurrence; tau huge never fires and
    equals the closed form with the tile-0 reference; V*2^k scales O by 2^k;
    query-row permutation permutes the output; a planted overshoot of
    tau + 1 fires exactly once with the hand-computed shift.
"""
import math
import zlib

import numpy as np
import pytest
import torch

from tests import spec_numpy as spec


def bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def quantize_all(O, q, k, v, sigma, qk, ve):
    """q,k,v bf16 [B,H,S,D] -> oracle MX tensors (Q with the folded prescale)."""
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    alpha = O.softmax_scale_prescale(sigma)
    Q = O.quantize_mx(bits(q).reshape(B * H, Sq, D), 0, qk, prescale=alpha)
    K = O.quantize_mx(bits(k).reshape(B * H, Skv, D), 0, qk)
    V = O.quantize_mx(bits(v).reshape(B * H, Skv, D), 1, ve)
    return Q, K, V


def rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


# ---------------------------------------------------------------- stage 1


def test_stage1_closed_form(oracle):
    # b = floor(t) for t >= 128, flushed below, clamped at the largest finite bf16
    assert oracle.stage1(127.999) == 0
    assert oracle.stage1(-5.0) == 0
    assert oracle.stage1(128.0) == 128
    assert oracle.stage1(16256.75) == 16256
    assert oracle.stage1(40000.0) == 0x7F7F
    # exactness at integer log2: t = 128*(n+127) -> 2^n exactly
    for n in range(-126, 127):
        b = oracle.stage1(128.0 * (n + 127))
        assert float(spec.bf16_value(b)) == 2.0 ** n


def test_schraudolph_bounds_vs_exp2(oracle):
    """approx(y)/2^y lies in [2^(-1/128), max_k (1+k/128) 2^(-k/128)] (c = 0)."""
    inf_b = 2.0 ** (-1 / 128)
    sup_b = max((1 + k / 128) * 2.0 ** (-k / 128) for k in range(128))
    assert abs(sup_b - 1.061474) < 1e-6
    rng = np.random.default_rng(0)
    ts = np.concatenate([rng.uniform(128.0 * 1, 128.0 * 254, 20000),
                         128.0 * np.arange(1, 254) + 57.0, 128.0 * np.arange(1, 254) + 127.999])
    ratios = []
    for t in ts.astype(np.float32):
        b = oracle.stage1(float(t))
        approx = float(spec.bf16_value(b))
        exact = 2.0 ** (float(t) / 128.0 - 127.0)
        ratios.append(approx / exact)
    ratios = np.array(ratios)
    assert ratios.min() >= inf_b * (1 - 1e-12)
    assert ratios.max() <= sup_b * (1 + 1e-12)
    assert ratios.max() == pytest.approx(sup_b, rel=1e-9)  # attained at frac = 57/128
    assert ratios.min() == pytest.approx(inf_b, rel=1e-4)  # approached below an integer


def test_schraudolph_vs_std_exp(oracle):
    """exp(x) through the folded map t = 128 (x log2 e + 127): relative error
    inside the closed-form band [-0.54 %, +6.15 %]."""
    rng = np.random.default_rng(1)
    xs = rng.uniform(-80, 80, 5000)
    for x in xs:
        t = np.float32(128.0 * (x * math.log2(math.e) + 127.0))
        approx = float(spec.bf16_value(oracle.stage1(float(t))))
        rel = approx / math.exp(x) - 1
        assert -0.0055 < rel < 0.0616


# ---------------------------------------------------------------- brute force vs spec

CASES = [
    # (name, Sq, Skv, D, qk, v, p, kv_tile, key_scale_rows)
    ("fp8-2tiles", 6, 128, 32, 0, 0, 0, 64, None),
    ("fp6-tail", 5, 100, 32, 2, 2, 2, 32, None),
    ("fp4-p6", 4, 96, 64, 4, 4, 2, 32, None),
    ("fp8-stress", 5, 160, 32, 0, 0, 0, 32, (70, 101, 130, 150)),
    ("fp6-stress", 4, 130, 32, 2, 2, 2, 64, (3, 70, 100, 120)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_matches_exact_spec(oracle, case):
    name, Sq, Skv, D, qk, ve, pe, bc, stress = case
    seed = zlib.crc32(name.encode()) % 1000
    q = rand_bf16((1, 1, Sq, D), seed)
    k = rand_bf16((1, 1, Skv, D), seed + 1)
    v = rand_bf16((1, 1, Skv, D), seed + 2)
    if stress:
        k = k.float()
        for r in stress:
            k[0, 0, r] *= 8.0
        k = k.to(torch.bfloat16)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_all(oracle, q, k, v, sigma, qk, ve)
    p = oracle.make_params(1, 1, Sq, Skv, D, qk, ve, pe, tau=8.0, kv_tile=bc)
    r = oracle.forward(p, Q, K, V, want_p=True)
    O_s, cnt_s, pc_s, ps_s = spec.forward(bits(q[0, 0]), bits(k[0, 0]), bits(v[0, 0]), sigma, qk, ve, pe,
                                          tau=8.0, kv_tile=bc)
    assert np.array_equal(r["counts"], cnt_s)
    assert np.array_equal(r["p_codes"].astype(np.int64), pc_s)
    assert np.array_equal(r["p_scales"].astype(np.int64), ps_s)
    np.testing.assert_allclose(r["O"], O_s, rtol=1e-12, atol=1e-12)
    if stress:
        assert r["counts"].sum() > 0, "stress case should exercise the rollback path"


# ---------------------------------------------------------------- invariants


def _setup(oracle, Sq=24, Skv=200, D=64, qk=2, ve=2, seed=7, kscale=None):
    q = rand_bf16((1, 2, Sq, D), seed)
    k = rand_bf16((1, 2, Skv, D), seed + 1)
    v = rand_bf16((1, 2, Skv, D), seed + 2)
    if kscale is not None:
        k = (k.float() * kscale).to(torch.bfloat16)
    sigma = 1 / math.sqrt(D)
    return (q, k, v, sigma) + quantize_all(oracle, q, k, v, sigma, qk, ve)


@pytest.mark.parametrize("tau", [0.0, 3.0, 8.0, 1e4])
@pytest.mark.parametrize("bc", [32, 64])
def test_I1_shift_invariance(oracle, tau, bc):
    q, k, v, sigma, Q, K, V = _setup(oracle, kscale=3.0)
    p = oracle.make_params(1, 2, 24, 200, 64, 2, 2, 2, tau=tau, kv_tile=bc, exp_mode=oracle.EXP_EXACT,
                           p_mode=oracle.P_NONE, fold_mode=oracle.FOLD_EXACT)
    r = oracle.forward(p, Q, K, V)
    R1 = oracle.reference(p, oracle.REF_R1, Q, K, V)
    np.testing.assert_allclose(r["O"], R1, rtol=1e-12, atol=1e-12)


def test_I1_fp32_fold_close(oracle):
    """With the binary32 fold left on, agreement is at the fold's rounding level."""
    q, k, v, sigma, Q, K, V = _setup(oracle)
    p = oracle.make_params(1, 2, 24, 200, 64, 2, 2, 2, exp_mode=oracle.EXP_EXACT, p_mode=oracle.P_NONE)
    r = oracle.forward(p, Q, K, V)
    R1 = oracle.reference(p, oracle.REF_R1, Q, K, V)
    np.testing.assert_allclose(r["O"], R1, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("pe", [0, 2])
def test_I2_tau0_is_flash_attention(oracle, pe):
    q, k, v, sigma, Q, K, V = _setup(oracle, kscale=2.0)
    p = oracle.make_params(1, 2, 24, 200, 64, 2, 2, pe, tau=0.0, kv_tile=32, exp_mode=oracle.EXP_EXACT,
                           p_mode=oracle.P_MX, fold_mode=oracle.FOLD_EXACT)
    r = oracle.forward(p, Q, K, V)
    R3 = oracle.reference(p, oracle.REF_R3, Q, K, V)
    np.testing.assert_allclose(r["O"], R3, rtol=1e-12, atol=1e-12)
    assert r["counts"].sum() > 0


def test_I3_tau_huge_never_fires(oracle):
    q, k, v, sigma, Q, K, V = _setup(oracle, kscale=4.0)
    p = oracle.make_params(1, 2, 24, 200, 64, 2, 2, 2, tau=1e4, kv_tile=32)
    r = oracle.forward(p, Q, K, V, want_p=True)
    assert r["counts"].sum() == 0
    # closed form with the tile-0 reference: spec with the same tau
    O_s, cnt_s, pc_s, _ = spec.forward(bits(q[0, 0]), bits(k[0, 0]), bits(v[0, 0]), sigma, 2, 2, 2, tau=1e4,
                                       kv_tile=32)
    np.testing.assert_allclose(r["O"][:24], O_s, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["p_codes"][:24].astype(np.int64), pc_s)


def test_I4_power_of_two_equivariance_and_permutation(oracle):
    q, k, v, sigma, Q, K, V = _setup(oracle, Sq=16, Skv=130, D=32, qk=0, ve=0, seed=3)
    p = oracle.make_params(1, 2, 16, 130, 32, 0, 0, 0, kv_tile=64)
    base = oracle.forward(p, Q, K, V)
    v4 = (v.float() * 4.0).to(torch.bfloat16)
    V4 = oracle.quantize_mx(bits(v4).reshape(2, 130, 32), 1, 0)
    r4 = oracle.forward(p, Q, K, V4)
    assert np.array_equal(r4["O"], base["O"] * 4.0)
    perm = torch.randperm(16, generator=torch.Generator().manual_seed(1))
    qp = q[:, :, perm]
    Qp = oracle.quantize_mx(bits(qp).reshape(2, 16, 32), 0, 0, prescale=oracle.softmax_scale_prescale(sigma))
    rp = oracle.forward(p, Qp, K, V)
    for h in range(2):
        assert np.array_equal(rp["O"][h * 16:(h + 1) * 16], base["O"][h * 16:(h + 1) * 16][perm.numpy()])
        assert np.array_equal(rp["counts"][h * 16:(h + 1) * 16], base["counts"][h * 16:(h + 1) * 16][perm.numpy()])


def test_I5_planted_overshoot(oracle):
    """Two 32-key tiles; one key of tile 1 scores tau+1 log2 units above tile 0's max."""
    D, tau = 32, 8.0
    sigma = 1 / math.sqrt(D)
    q = torch.zeros(1, 1, 1, D)
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros(1, 1, 64, D)
    k[0, 0, :32, 0] = torch.linspace(-1, 1, 32)  # tile-0 max score: 1 * alpha
    # raw score s = alpha * k0 / 128 in log2 units; plant k0 such that s - s0max = tau + 1
    alpha = oracle.softmax_scale_prescale(sigma)
    k[0, 0, 40, 0] = 1.0 + (tau + 1.0) * 128.0 / alpha
    v = torch.randn(1, 1, 64, D, generator=torch.Generator().manual_seed(0))
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    Q, K, V = quantize_all(oracle, q, k, v, sigma, 2, 2)
    p = oracle.make_params(1, 1, 1, 64, D, 2, 2, 2, tau=tau, kv_tile=32)
    r = oracle.forward(p, Q, K, V)
    assert r["counts"][0] == 1
    # hand value of the shift: folded scores are exact here (E2M3 grid), t_max(tile1) - T0
    s = [oracle.folded_score(2, Q[0][0, 0], Q[1][0, 0], K[0][0, kk], K[1][0, kk], D, 0.0, exact=True)
         for kk in range(64)]
    C = 16256.0 - max(s[:32])
    delta = max(s[32:]) + C - 16256.0
    assert delta >= 128 * tau
    # O after the fire equals the spec (which applies the same hand-derivable steps)
    O_s, cnt_s, _, _ = spec.forward(bits(q[0, 0]), bits(k[0, 0]), bits(v[0, 0]), sigma, 2, 2, 2, tau=tau,
                                    kv_tile=32)
    assert cnt_s[0] == 1
    np.testing.assert_allclose(r["O"][0], O_s[0], rtol=1e-12)
    # and a tau just above the overshoot never fires
    p2 = oracle.make_params(1, 1, 1, 64, D, 2, 2, 2, tau=(delta + 1) / 128.0, kv_tile=32)
    assert oracle.forward(p2, Q, K, V)["counts"][0] == 0


def test_reference_bf16_is_softmax(oracle):
    """R0 equals torch's float64 softmax attention on the same bf16 inputs."""
    q = rand_bf16((1, 2, 20, 64), 11)
    k = rand_bf16((1, 2, 50, 64), 12)
    v = rand_bf16((1, 2, 50, 64), 13)
    sigma = 0.125
    O = oracle.reference_bf16(bits(q), bits(k), bits(v), sigma)
    qd, kd, vd = q.double(), k.double(), v.double()
    ref = torch.softmax(qd @ kd.transpose(-1, -2) * sigma, dim=-1) @ vd
    np.testing.assert_allclose(O, ref.reshape(-1, 64).numpy(), rtol=1e-12, atol=1e-13)


def test_rows_subset_equals_full(oracle):
    q, k, v, sigma, Q, K, V = _setup(oracle, kscale=3.0)
    p = oracle.make_params(1, 2, 24, 200, 64, 2, 2, 2, kv_tile=64)
    full = oracle.forward(p, Q, K, V, want_p=True)
    rows = np.array([0, 5, 23, 24, 47])
    sub = oracle.forward(p, Q, K, V, rows=rows, want_p=True)
    assert np.array_equal(sub["O"], full["O"][rows])
    assert np.array_equal(sub["counts"], full["counts"][rows])
    assert np.array_equal(sub["p_codes"], full["p_codes"][rows])
