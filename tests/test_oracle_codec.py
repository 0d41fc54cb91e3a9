"""Pins for the oracle's MX codec (element formats, E8M0 rule, block packing,
two-stage BF16 -> MX conversion).

The element formats and the E8M0 scale are the OCP Microscaling v1.0 ones
named by the pages' MXFP8 / MXFP6 / MXFP4 configurations ("Fused-Softmax shifts
an AI attention bottleneck onto faster GPU hardware", paragraphs 7-8).  Pins:
closed forms of the formats (largest values, grids), brute force over every
code, ties-to-even at every midpoint, the E4M3/E5M2 cases that reduce to
PyTorch's float8 casts (a library routine), and an independent grid-search
encoder (tests/spec_numpy.py).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests import spec_numpy as spec

ELEMS = [0, 1, 2, 3, 4]
MAXNORM = {0: 448.0, 1: 57344.0, 2: 7.5, 3: 28.0, 4: 6.0}  # OCP MX v1.0 table values
EMAX = {0: 8, 1: 15, 2: 2, 3: 4, 4: 2}
BITS = {0: 8, 1: 8, 2: 6, 3: 6, 4: 4}


def _finite_codes(O, e):
    out = []
    for c in range(1 << BITS[e]):
        v = O.decode(e, c)
        if np.isfinite(v):
            out.append(c)
    return out


@pytest.mark.parametrize("e", ELEMS)
def test_maxnorm_closed_form(oracle, e):
    assert oracle.maxnorm(e) == MAXNORM[e]
    vals = [oracle.decode(e, c) for c in _finite_codes(oracle, e)]
    assert max(vals) == MAXNORM[e]
    assert min(vals) == -MAXNORM[e]


@pytest.mark.parametrize("e", ELEMS)
def test_round_trip_every_code(oracle, e):
    for c in _finite_codes(oracle, e):
        v = oracle.decode(e, c)
        back = oracle.encode(e, v)
        if v == 0.0:
            # +0 and -0 both round-trip with their sign bit
            assert back == c
        else:
            assert back == c, (e, c, v, back)


@pytest.mark.parametrize("e", ELEMS)
def test_decode_matches_independent_grid(oracle, e):
    for v, c in spec.grid(e):
        assert oracle.decode(e, c) == float(v)


@pytest.mark.parametrize("e", ELEMS)
def test_midpoints_round_to_even_and_monotone(oracle, e):
    g = [float(v) for v, _ in spec.grid(e)]
    codes = [oracle.encode(e, x) for x in g]
    assert codes == sorted(codes), "codes not monotone in value"
    for a, b in zip(g[:-1], g[1:]):
        mid = (a + b) / 2  # exact in double
        c = oracle.encode(e, mid)
        ca, cb = oracle.encode(e, a), oracle.encode(e, b)
        assert c in (ca, cb)
        assert c % 2 == 0, f"midpoint {mid} -> odd code {c}"
        assert oracle.encode(e, np.nextafter(mid, -np.inf)) == ca
        assert oracle.encode(e, np.nextafter(mid, np.inf)) == cb
        assert oracle.encode(e, -mid) == c | (1 << (BITS[e] - 1))


@pytest.mark.parametrize("e", ELEMS)
def test_saturation(oracle, e):
    top = oracle.encode(e, MAXNORM[e])
    assert oracle.encode(e, MAXNORM[e] * 1.5) == top
    assert oracle.encode(e, 1e30) == top
    assert oracle.encode(e, -1e30) == top | (1 << (BITS[e] - 1))


@pytest.mark.parametrize("e", ELEMS)
def test_encode_matches_grid_search_random(oracle, e):
    rng = np.random.default_rng(10 + e)
    xs = rng.standard_normal(400) * MAXNORM[e] / 3
    xs = np.concatenate([xs, rng.standard_normal(100) * MAXNORM[e] / 300])
    for x in xs:
        assert oracle.encode(e, float(x)) == spec.encode(e, Fraction(float(x)))


@pytest.mark.parametrize("e,tdt", [(0, torch.float8_e4m3fn), (1, torch.float8_e5m2)])
def test_fp8_matches_torch_cast(oracle, e, tdt):
    """Library special case: inside +-maxnorm the OCP FP8 encoders are torch's RNE casts."""
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(5000) * MAXNORM[e] / 4,
                         rng.standard_normal(2000) * 2.0 ** -7, np.array([0.0, -0.0])])
    xs = xs[np.abs(xs) <= MAXNORM[e]]
    t = torch.from_numpy(xs).to(tdt).view(torch.uint8).numpy()
    ours = np.array([oracle.encode(e, float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(t, ours)


M_MAX = {0: 1.75, 1: 1.75, 2: 1.875, 3: 1.75, 4: 1.5}


@pytest.mark.parametrize("e", ELEMS)
def test_scale_rule_closed_form(oracle, e):
    for ex in [-140, -20, -3, 0, 1, 7, 30]:
        for m in [1.0, M_MAX[e], np.nextafter(M_MAX[e], 2.0), 1.9999]:
            amax = m * 2.0 ** ex
            k_fit = ex - EMAX[e] + (1 if m > M_MAX[e] else 0)
            k_ocp = ex - EMAX[e]
            assert oracle.scale_code(e, 0, amax) == min(max(k_fit + 127, 0), 254)
            assert oracle.scale_code(e, 1, amax) == min(max(k_ocp + 127, 0), 254)
    assert oracle.scale_code(e, 0, 0.0) == 0


@pytest.mark.parametrize("e", ELEMS)
def test_fitmax_is_tightest(oracle, e):
    rng = np.random.default_rng(5)
    for _ in range(300):
        amax = float(np.exp(rng.uniform(-30, 30)))
        X = 2.0 ** (oracle.scale_code(e, 0, amax) - 127)
        assert amax / X <= MAXNORM[e]
        assert amax / (X / 2) > MAXNORM[e]
        assert spec.scale_code(e, Fraction(amax)) == oracle.scale_code(e, 0, amax)


@pytest.mark.parametrize("e", ELEMS)
def test_block_special_cases(oracle, e):
    codes, sc = oracle.mxq_block(e, 0, np.zeros(32))
    assert sc == 0 and not codes.any()
    x = np.zeros(32)
    x[7] = -3.0
    codes, sc = oracle.mxq_block(e, 0, x)
    X = 2.0 ** (sc - 127)
    assert oracle.decode(e, int(codes[7])) * X == -3.0
    assert all(c == 0 for i, c in enumerate(codes) if i != 7)
    # sign of zero kept
    x = np.zeros(32)
    x[0] = 1.0
    x[1] = -0.0
    codes, _ = oracle.mxq_block(e, 0, x)
    assert codes[1] == 1 << (BITS[e] - 1)


def _unpack(codes_row: np.ndarray, e: int, n: int) -> list[int]:
    """Independent unpacker: little-endian bit stream of `BITS[e]`-bit codes."""
    bits = np.unpackbits(codes_row, bitorder="little")
    w = BITS[e]
    return [int(sum(int(bits[j * w + t]) << t for t in range(w))) for j in range(n)]


@pytest.mark.parametrize("e", ELEMS)
@pytest.mark.parametrize("axis", [0, 1])
def test_quantizer_layout_and_blocks(oracle, e, axis):
    rng = np.random.default_rng(20 + e + 10 * axis)
    x = (rng.standard_normal((2, 45, 64)) * np.exp(rng.uniform(-3, 3, (2, 45, 1)))).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    u = xb.view(torch.int16).numpy().view(np.uint16)
    xf = xb.float().numpy().astype(np.float64)
    pre = 16.322231 if axis == 0 else 1.0
    codes, scales = oracle.quantize_mx(u, axis, e, prescale=pre)
    bb = oracle.block_bytes(e)
    if axis == 0:
        for m in range(2):
            for r in range(45):
                for g in range(2):
                    vals = np.float32(np.float32(pre) * xf[m, r, g * 32:(g + 1) * 32].astype(np.float32))
                    c_exp, s_exp = oracle.mxq_block(e, 0, vals.astype(np.float64))
                    got = _unpack(codes[m, r, g * bb:(g + 1) * bb], e, 32)
                    assert scales[m, r, g] == s_exp
                    assert got == list(c_exp)
    else:
        for m in range(2):
            for col in range(64):
                for g in range(2):
                    blk = np.zeros(32)
                    n = min(32, 45 - g * 32)
                    blk[:n] = xf[m, g * 32:g * 32 + n, col]
                    c_exp, s_exp = oracle.mxq_block(e, 0, blk)
                    got = _unpack(codes[m, col, g * bb:(g + 1) * bb], e, 32)
                    assert scales[m, col, g] == s_exp
                    assert got == list(c_exp)


@pytest.mark.parametrize("p_elem", [0, 2, 3])
def test_two_stage_conversion_exhaustive(oracle, p_elem):
    """Stage 2 of every non-negative BF16 pattern equals RNE of the exact value / X,
    for block maxima in every binade that P can take (P <= 1)."""
    pats = np.arange(128, 0x3F81, dtype=np.uint32)  # normal patterns up to 1.0
    vals = (pats << 16).view(np.float32).astype(np.float64)
    g = spec._GRIDS[p_elem]
    top = float(g[-1][0])
    for bmax in [0x3F80, 0x3F00, 0x3E80, 0x3A00, 0x2000, 0x0100]:
        amax = float(((np.uint32(bmax)) << 16).view(np.float32))
        sc = oracle.scale_code(p_elem, 0, amax)
        X = 2.0 ** (sc - 127)
        sel = vals <= amax
        for x in vals[sel][::7]:
            c = oracle.encode(p_elem, x / X)
            assert c == spec.encode(p_elem, Fraction(x) / Fraction(X))
            assert abs(oracle.decode(p_elem, c) * X) <= top * X
