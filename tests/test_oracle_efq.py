"""Pins of the oracle's EFQ-style E2M1 P rule (reading R24) and its wiring
into the fused forward.

"EFQ-Softmax: Exp-Free Quantization for Softmax", sections II.B-C, III.A-B:
per 32-key block an exponent-only scale from the local maximum, a residual
in the log domain, uniformly spaced thresholds tau + j h mapped to the E2M1
codes 0..7 (code 7 = 6.0), and one P operand for both P V and P 1.

The pins check the oracle against things fixed by that description and by
arithmetic, not against its own formula:
- codes on and just below each threshold, at two block exponents (dyadic
  parameters, so every step is exact);
- an exact-rational evaluation of the rule on random blocks, every key;
- keys exactly on each threshold and one binary32 step below it, with
  spacings h whose reciprocal has no exact binary32 value;
- shift invariance: moving a block by whole binades moves only its E8M0;
- absent keys and empty blocks;
- end to end: identical keys give O = the mean of V-hat (same P in both
  sums); O equals sum(P-hat V-hat) / sum(P-hat) from the dumped P; dumped
  codes equal the rational rule applied to independently recomputed scores.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from softmax_matrix_cores_amd import workloads as W

T0 = 16256.0
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32(x) -> float:
    return float(np.float32(x))


def rational_rule(t, T0_, tau, h):
    """R24 in exact rationals: l = (t - T0)/128, E = floor(max l), code =
    clamp(floor((l - E - tau)/h), 0, 7); also returns each code's distance to
    the nearest threshold in units of h (to skip rounding-sensitive keys)."""
    F = [Fraction(f32(x)) for x in t]
    l = [(x - Fraction(f32(T0_))) / 128 for x in F]
    E = math.floor(max(l))
    tau_f, h_f = Fraction(f32(tau)), Fraction(f32(h))
    codes, dist = [], []
    for x in l:
        z = (x - E - tau_f) / h_f
        codes.append(min(max(math.floor(z), 0), 7))
        dist.append(float(abs(z - round(z))))
    return codes, E, dist


def test_codes_on_and_below_each_threshold(oracle):
    tau, h = -3.5, 0.5
    for E in (0, -3, 2):
        lmax = E + 0.75  # block maximum sets the exponent E
        t = [T0 + 128 * lmax]
        want = [7]  # (0.75 - tau) / h = 8.5: clamped to 7
        for j in range(1, 8):
            on = T0 + 128 * (E + tau + j * h)
            t.append(on)
            want.append(j)
            below = float(np.nextafter(np.float32(on), np.float32(-np.inf)))
            t.append(below)
            want.append(j - 1)
        t.append(T0 + 128 * (E + tau - 1.0))  # far below the first threshold
        want.append(0)
        codes, sc = oracle.efq_block(t, T0, tau, h)
        assert sc == E - 2 + 127
        assert list(codes[: len(want)]) == want, (E, list(codes[: len(want)]))
        assert not codes[len(want):].any()


def test_rule_against_exact_rationals(oracle):
    rng = np.random.default_rng(24)
    checked = 0
    for it in range(300):
        tau, h = [(-3.890625, 0.609375), (-3.7, 0.55), (-2.0, 0.3), (-5.0, 1.1)][it % 4]
        n = 32 if it % 3 else int(rng.integers(1, 33))
        lmax = rng.uniform(-12.0, 3.0)
        l = lmax - rng.exponential(2.5, n)
        l[rng.integers(0, n)] = lmax
        t = [f32(T0 + 128 * x) for x in l]
        codes, sc = oracle.efq_block(t, T0, tau, h, nvis=n)
        want, E, dist = rational_rule(t, T0, tau, h)
        assert sc == min(max(E - 2 + 127, 0), 254)
        for i in range(n):
            assert codes[i] == want[i], (it, i, l[i], codes[i], want[i], dist[i])
            checked += 1
        assert not codes[n:].any()
    assert checked > 8000


@pytest.mark.parametrize("tau,h", [(-3.875, 0.609375), (-3.890625, 0.609375), (-3.25, 0.5625)])
def test_codes_on_thresholds_with_inexact_slope(oracle, tau, h):
    """Keys exactly on a threshold tau + j h (binary32 scores) take code j and
    the next binary32 below takes j - 1, also where 1 / (128 h) has no exact
    binary32 value (h = 39/64, 9/16): the rule is the threshold count itself,
    not a rounded slope."""
    tau32, h32 = np.float32(tau), np.float32(h)
    for E in (0, -4, 1):
        t = [T0 + 128 * (E + 0.8)]
        want = [min(max(math.floor((Fraction(0.8) - Fraction(float(tau32))) / Fraction(float(h32))), 0), 7)]
        for j in range(1, 8):
            thr = Fraction(float(T0)) + 128 * (E + Fraction(float(tau32)) + j * Fraction(float(h32)))
            on = np.float32(float(thr))
            if Fraction(float(on)) != thr:
                continue  # the threshold is not a binary32 score
            t.append(float(on))
            want.append(j)
            t.append(float(np.nextafter(on, np.float32(-np.inf))))
            want.append(j - 1)
        assert len(t) > 9
        codes, sc = oracle.efq_block(t, T0, tau, h)
        assert sc == E - 2 + 127
        assert list(codes[: len(t)]) == want, (tau, h, E, list(codes[: len(t)]), want)


def test_shift_by_whole_binades_moves_only_the_scale(oracle):
    rng = np.random.default_rng(5)
    for tau, h in [(-3.5, 0.5), (-3.890625, 0.609375), (-2.25, 0.375)]:
        l = 0.9 - rng.exponential(2.0, 32)
        base_codes, base_sc = oracle.efq_block([T0 + 128 * x for x in l], T0, tau, h)
        for n in (-40, -7, -1, 1, 5):
            c, sc = oracle.efq_block([T0 + 128 * (x + n) for x in l], T0, tau, h)
            assert sc == base_sc + n
            assert np.array_equal(c, base_codes), (tau, h, n)


def test_absent_keys_and_empty_block(oracle):
    codes, sc = oracle.efq_block([], T0, -3.5, 0.5, nvis=0)
    assert sc == 0 and not codes.any()
    t = [T0] * 32
    codes, sc = oracle.efq_block(t, T0, -3.5, 0.5, nvis=5)
    assert list(codes[:5]) == [7] * 5 and not codes[5:].any()
    assert sc == 125


def bits(x):
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def _efq_params(oracle, B, H, Sq, Skv, D, elem, tau=8.0, efq=(-3.890625, 0.609375), kv_tile=64):
    return oracle.make_params(B, H, Sq, Skv, D, elem, elem, oracle.E2M1, tau=tau, kv_tile=kv_tile,
                              p_mode=oracle.P_EFQ, efq_tau=efq[0], efq_h=efq[1])


def _quant(oracle, q, k, v, elem, sigma):
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    a = oracle.softmax_scale_prescale(sigma)
    Q = oracle.quantize_mx(bits(q).reshape(B * H, Sq, D), 0, elem, prescale=a)
    K = oracle.quantize_mx(bits(k).reshape(B * H, Skv, D), 0, elem)
    V = oracle.quantize_mx(bits(v).reshape(B * H, Skv, D), 1, elem)
    return Q, K, V


def _vhat(oracle, V, elem, Skv, D):
    """Decoded V-hat [Skv, D] of head 0 (codes [D][nb][block], scales [D][nb])."""
    codes, scales = V
    nb = (Skv + 31) // 32
    bpb = {oracle.E2M3: 24, oracle.E2M1: 16}[elem]
    bitsz = {oracle.E2M3: 6, oracle.E2M1: 4}[elem]
    blk = codes.reshape(-1, D, nb, bpb)[0]
    sc = scales.reshape(-1, D, nb)[0].astype(np.int64)
    out = np.zeros((nb * 32, D))
    for d in range(D):
        for g in range(nb):
            stream = int.from_bytes(blk[d, g].tobytes(), "little")
            for j in range(32):
                c = (stream >> (bitsz * j)) & ((1 << bitsz) - 1)
                out[g * 32 + j, d] = oracle.decode(elem, c) * 2.0 ** (sc[d, g] - 127)
    return out[:Skv]


@pytest.mark.parametrize("elem_name", ["e2m3", "e2m1"])
def test_identical_keys_give_mean_of_v(oracle, elem_name):
    elem = oracle.ELEM_NAMES[elem_name]
    D, S = 64, 96
    g = torch.Generator().manual_seed(7)
    q = torch.randn(1, 1, 8, D, generator=g).bfloat16()
    k = torch.randn(1, 1, 1, D, generator=g).bfloat16().expand(1, 1, S, D).contiguous()
    v = torch.randn(1, 1, S, D, generator=g).bfloat16()
    Q, K, V = _quant(oracle, q, k, v, elem, D ** -0.5)
    p = _efq_params(oracle, 1, 1, 8, S, D, elem)
    r = oracle.forward(p, Q, K, V, want_p=True)
    vh = _vhat(oracle, V, elem, S, D)
    # every key has the row maximum: l = 0, E = 0, r = 0, code floor(-tau / h) = 6
    assert (r["p_codes"][:, :S] == math.floor(Fraction(3.890625) / Fraction(0.609375))).all()
    np.testing.assert_allclose(r["O"], np.broadcast_to(vh.mean(0), r["O"].shape), rtol=1e-12, atol=1e-12)


def test_output_is_the_dumped_p_average(oracle):
    """No fires (gate tau 10000): O = sum(P-hat V-hat) / sum(P-hat) with P-hat
    decoded from the dumped codes and scales."""
    elem = oracle.E2M1
    w = W.custom("qknorm-mxfp4", B=1, H=1, Sq=16, Skv=200, D=64)
    q, k, v = W.make_inputs(w)
    Q, K, V = _quant(oracle, q, k, v, elem, w.sigma)
    p = _efq_params(oracle, 1, 1, 16, 200, 64, elem, tau=10000.0)
    r = oracle.forward(p, Q, K, V, want_p=True)
    assert r["counts"].sum() == 0
    vh = _vhat(oracle, V, elem, 200, 64)
    codes, sc = r["p_codes"][:, :200], r["p_scales"]
    ph = np.array(E2M1_VALUES)[codes] * 2.0 ** (np.repeat(sc.astype(np.int64), 32, axis=1)[:, :200] - 127)
    assert (codes[:, 200:] == 0).all() if codes.shape[1] > 200 else True
    want = ph @ vh / ph.sum(1, keepdims=True)
    np.testing.assert_allclose(r["O"], want, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["l"], ph.sum(1), rtol=1e-12)


def test_dumped_codes_follow_the_rule_on_recomputed_scores(oracle):
    """One gate tile (Skv = kv_tile = 64): t = fl32(s + fl32(T0 - max s)) from
    independently recomputed fp32 scores, then the rational rule per block."""
    elem = oracle.E2M1
    tau, h = -3.7, 0.55
    w = W.custom("qknorm-mxfp4", B=1, H=1, Sq=24, Skv=64, D=128)
    q, k, v = W.make_inputs(w)
    Q, K, V = _quant(oracle, q, k, v, elem, w.sigma)
    p = _efq_params(oracle, 1, 1, 24, 64, 128, elem, efq=(tau, h))
    r = oracle.forward(p, Q, K, V, want_p=True)
    qc, qs = Q
    kc, ks = K
    bpr = 128 * 4 // 8
    checked = 0
    for i in range(24):
        s = [f32(oracle.folded_score(elem, qc.reshape(24, bpr)[i], qs.reshape(24, 4)[i], kc.reshape(64, bpr)[j],
                                     ks.reshape(64, 4)[j], 128, 0.0)) for j in range(64)]
        C = f32(T0 - max(s))
        t = [f32(x + C) for x in s]
        for g in range(2):
            want, E, dist = rational_rule(t[32 * g: 32 * g + 32], T0, tau, h)
            assert r["p_scales"][i, g] == min(max(E - 2 + 127, 0), 254)
            for j in range(32):
                if dist[j] > 1e-4:
                    assert r["p_codes"][i, 32 * g + j] == want[j], (i, g, j)
                    checked += 1
    assert checked > 1400


def test_stored_calibration_reproduces(oracle):
    """tests/golden/efq_calibration.json (written by make_efq_calibration.py
    from the oracle) matches what the oracle gives at the stored point."""
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "efq_calibration.json")))
    S, D = 1024, 128
    q, k, v = W.error_study_inputs(0, S=S, D=D)
    elem = oracle.E2M1
    Q, K, V = _quant(oracle, q, k, v, elem, 1 / math.sqrt(D))
    p = _efq_params(oracle, 1, 1, S, S, D, elem, efq=(gold["efq_tau"], gold["efq_h"]))
    O = oracle.forward(p, Q, K, V)["O"]
    R1 = oracle.reference(oracle.make_params(1, 1, S, S, D, elem, elem, oracle.E2M3), oracle.REF_R1, Q, K, V)
    err = np.linalg.norm(O - R1) / np.linalg.norm(R1)
    assert abs(err - gold["error_per_set"]["iid-seed0"]) < 1e-12
