"""The FP8 P-code explanation used by the GPU parity tests (tests/gpu_util.py,
explain_fp8), checked on the CPU with the oracle alone: a floor that lands on
the other side of an integer close to the score is explained; a code changed
anywhere else is not."""
import math

import numpy as np
import torch

from tests import gpu_util as G
from tests import spec_numpy as spec
from tests.test_oracle_forward import quantize_all, rand_bf16


def _case(O):
    q = rand_bf16((1, 1, 6, 64), 31)
    k = rand_bf16((1, 1, 160, 64), 32)
    v = rand_bf16((1, 1, 160, 64), 33)
    Q, K, V = quantize_all(O, q, k, v, 1 / 8, O.E4M3, O.E4M3)
    p = O.make_params(1, 1, 6, 160, 64, O.E4M3, O.E4M3, O.E4M3, kv_tile=64)
    rows = np.arange(6)
    r = O.forward(p, Q, K, V, want_p=True)
    t, _ = O.forward_scores(p, Q, K, V, rows)
    return r["p_codes"], r["p_scales"], t


def test_identical_dump_has_nothing_to_explain(oracle):
    oc, os_, t = _case(oracle)
    assert G.explain_fp8(oracle, oracle.E4M3, oc, os_, oc, os_, t, 64) == (0, 0)


def test_floor_on_the_other_side_is_explained(oracle):
    oc, os_, t = _case(oracle)
    gc = oc.copy()
    flipped = 0
    for r, k in zip(*np.nonzero(t >= 128)):
        n = math.floor(t[r, k])
        if t[r, k] - n > G.fp8_bound(t[r, k], 64):
            continue
        X = 2.0 ** (int(os_[r, k // 32]) - 127)
        c = oracle.encode(oracle.E4M3, G._bf16_val(n - 1) / X)  # a score just below n
        if c != oc[r, k]:
            gc[r, k] = c
            flipped += 1
    assert flipped > 0
    bad, unexplained = G.explain_fp8(oracle, oracle.E4M3, gc, os_, oc, os_, t, 64)
    assert bad == flipped and unexplained == 0


def test_code_changed_away_from_an_integer_is_not_explained(oracle):
    oc, os_, t = _case(oracle)
    frac = np.abs(t - np.rint(t))
    r, k = np.argwhere((frac > 0.3) & (oc > 8) & (t >= 128))[0]
    gc = oc.copy()
    gc[r, k] = oc[r, k] - 1
    assert G.explain_fp8(oracle, oracle.E4M3, gc, os_, oc, os_, t, 64) == (1, 1)
    # a block scale off by one without a close integer is not explained either
    gs = os_.copy()
    g = k // 32
    gs[r, g] += 1
    bT = G._scale_step(oracle, oracle.E4M3, int(gs[r, g]))
    keys = slice(32 * g, 32 * g + 32)
    assert (np.abs(t[r, keys] - bT) > G.fp8_bound(t[r, keys], 64)).all()
    bad, unexplained = G.explain_fp8(oracle, oracle.E4M3, oc, gs, oc, os_, t, 64)
    assert bad == 32 and unexplained == 32


def test_forward_scores_match_exact_spec(oracle):
    """The diagnostic scores are the folded binary32 scores of the exact-rational
    forward (tests/spec_numpy.py) bit for bit, gate shifts included, and the
    largest products are those of the decoded operands."""
    Sq, Skv, D = 4, 200, 64
    q = rand_bf16((1, 1, Sq, D), 41)
    k = rand_bf16((1, 1, Skv, D), 42).float()
    k[0, 0, (90, 150)] *= 8.0  # planted fires in later tiles
    k = k.to(torch.bfloat16)
    v = rand_bf16((1, 1, Skv, D), 43)
    Q, K, V = quantize_all(oracle, q, k, v, 1 / 8, oracle.E4M3, oracle.E4M3)
    p = oracle.make_params(1, 1, Sq, Skv, D, oracle.E4M3, oracle.E4M3, oracle.E4M3, tau=2.0, kv_tile=32)
    t, amax = oracle.forward_scores(p, Q, K, V, np.arange(Sq))
    bits = lambda x: x[0, 0].contiguous().view(torch.int16).numpy().view(np.uint16)
    want = np.zeros((Sq, Skv))
    _, counts, _, _ = spec.forward(bits(q), bits(k), bits(v), 1 / 8, oracle.E4M3, oracle.E4M3, oracle.E4M3,
                                   tau=2.0, kv_tile=32, t_out=want)
    assert counts.sum() > 0
    assert np.array_equal(t[:, :Skv].astype(np.float64), want)
    Qh, Kh, _ = spec.operands(bits(q), bits(k), bits(v), 1 / 8, oracle.E4M3, oracle.E4M3)
    for i in range(Sq):
        for kk in (0, 90, 199):
            assert amax[i, kk] == float(max(abs(a * b) for a, b in zip(Qh[i], Kh[kk])))
