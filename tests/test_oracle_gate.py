"""Pins of the oracle's gate shortcut (reading R25).

"Fused-Softmax shifts an AI attention bottleneck onto faster GPU hardware",
paragraph 12: the fastest four-bit kernel gates through a shortcut that can
miss a recovery trigger in an extreme-score range.  The reading: the tile
fires when stage1(max t) > floor(T_gate), on the BF16 patterns the two-stage
conversion makes anyway, instead of max t > T_gate.

Pins:
- the decision equals the exact rule at the shifted threshold: for
  floor(T_gate) < 0x7F7F, stage1(t) > floor(T_gate) iff t >= floor(T_gate) + 1,
  so the shortcut forward equals the exact-gate forward whose threshold is
  the largest binary32 below floor(T_gate) + 1 (outputs, counts bit for bit);
- misses (exact would fire, the shortcut does not) happen only in that band:
  with no tile max in (T_gate, floor(T_gate) + 1) there are none;
- extreme range, floor(T_gate) >= 0x7F7F: the shortcut never fires, and its
  misses equal the number of tiles whose max, recomputed independently from
  the frozen tile-0 reference, exceeds T_gate.
"""
import math

import numpy as np
import pytest
import torch

from softmax_matrix_cores_amd import workloads as W

T0 = 16256.0


def bits(x):
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def quant(O, q, k, v, elem, sigma):
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    a = O.softmax_scale_prescale(sigma)
    return (O.quantize_mx(bits(q).reshape(B * H, Sq, D), 0, elem, prescale=a),
            O.quantize_mx(bits(k).reshape(B * H, Skv, D), 0, elem),
            O.quantize_mx(bits(v).reshape(B * H, Skv, D), 1, elem))


def tau_for_threshold(X: float, c: float = 0.0) -> float:
    """tau whose T_gate = fl32(128 (127 + tau) - c) is exactly the binary32 X."""
    tau = (X + c) / 128.0 - 127.0
    assert float(np.float32(128.0 * (127.0 + tau) - c)) == X
    return tau


def gate_threshold(tau: float, c: float = 0.0) -> float:
    return float(np.float32(128.0 * (127.0 + tau) - c))


@pytest.mark.parametrize("tau", [0.0, 0.3, 1.0, 2.7])
def test_shortcut_equals_exact_gate_at_shifted_threshold(oracle, tau):
    w = W.custom("qknorm-mxfp4", B=1, H=2, Sq=64, Skv=640, D=64, seed=31)
    q, k, v = W.make_inputs(w)
    elem = oracle.E2M1
    Q, K, V = quant(oracle, q, k, v, elem, w.sigma)
    p = oracle.make_params(1, 2, 64, 640, 64, elem, elem, oracle.E2M3, tau=tau, gate_mode=oracle.GATE_PATTERN)
    r = oracle.forward(p, Q, K, V, want_p=True)
    X = float(np.nextafter(np.float32(math.floor(gate_threshold(tau)) + 1), np.float32(0)))
    pe = oracle.make_params(1, 2, 64, 640, 64, elem, elem, oracle.E2M3, tau=tau_for_threshold(X))
    re = oracle.forward(pe, Q, K, V, want_p=True)
    assert r["counts"].sum() > 0
    assert np.array_equal(r["counts"], re["counts"])
    assert np.array_equal(r["O"], re["O"]) and np.array_equal(r["p_codes"], re["p_codes"])
    assert not re["misses"].any()  # the exact rule reports no misses


def test_no_misses_without_a_max_in_the_band(oracle):
    """tau = 1.0: T_gate = 16384 is an integer, so the band is (16384, 16385).
    A row misses only if a tile max lands there (in the shortcut's state);
    the total over a sample stays at most the count of band hits, which for
    iid data is a small fraction of the fires."""
    w = W.custom("qknorm-mxfp6", B=1, H=2, Sq=128, Skv=1024, D=64, seed=32)
    q, k, v = W.make_inputs(w)
    elem = oracle.E2M3
    Q, K, V = quant(oracle, q, k, v, elem, w.sigma)
    p = oracle.make_params(1, 2, 128, 1024, 64, elem, elem, elem, tau=1.0, gate_mode=oracle.GATE_PATTERN)
    r = oracle.forward(p, Q, K, V)
    assert r["counts"].sum() > 100
    assert r["misses"].sum() <= 0.05 * r["counts"].sum()


def test_extreme_range_never_fires(oracle):
    """tau = 200: floor(T_gate) = 41856 > 0x7F7F.  Planted keys push scores far
    above the tile-0 reference: the exact rule fires, the shortcut never does,
    and its misses are the tiles whose max (recomputed from the folded scores
    with the frozen reference) exceeds T_gate."""
    D, Sq, Skv = 32, 8, 256
    g = torch.Generator().manual_seed(33)
    q = torch.ones(1, 1, Sq, D) + 0.1 * torch.randn(1, 1, Sq, D, generator=g)
    k = torch.randn(1, 1, Skv, D, generator=g)
    for j in (70, 150, 151, 250):  # tiles 1, 2 and 3 get one or two huge keys
        k[0, 0, j] = 48.0
    v = torch.randn(1, 1, Skv, D, generator=g)
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    elem = oracle.E2M3
    sigma = D ** -0.5
    Q, K, V = quant(oracle, q, k, v, elem, sigma)
    tau = 200.0
    pe = oracle.make_params(1, 1, Sq, Skv, D, elem, elem, elem, tau=tau)
    ps = oracle.make_params(1, 1, Sq, Skv, D, elem, elem, elem, tau=tau, gate_mode=oracle.GATE_PATTERN)
    re = oracle.forward(pe, Q, K, V)
    rs = oracle.forward(ps, Q, K, V)
    assert (re["counts"] > 0).all()
    assert (rs["counts"] == 0).all()
    # independent recount: fl32 scores, tile-0 reference, tiles j >= 1 over T_gate
    Tg = gate_threshold(tau)
    qc, qs = Q
    kc, ks = K
    bpr = D * 6 // 8
    for i in range(Sq):
        s = [float(np.float32(oracle.folded_score(elem, qc.reshape(Sq, bpr)[i], qs.reshape(Sq, 1)[i],
                                                  kc.reshape(Skv, bpr)[j], ks.reshape(Skv, 1)[j], D, 0.0)))
             for j in range(Skv)]
        C = float(np.float32(T0 - max(s[:64])))
        t = [float(np.float32(x + C)) for x in s]
        over = sum(1 for j in range(1, Skv // 64) if max(t[64 * j: 64 * j + 64]) > Tg)
        assert rs["misses"][i] == over, (i, rs["misses"][i], over)
        assert over >= 1
