"""The C-ABI library: it loads, exports every symbol include/fsattn.h declares,
its size helpers follow the documented byte layout, and argument validation
rejects bad calls before anything is launched (no GPU needed for these)."""
import ctypes
import re
import os

import pytest

import softmax_matrix_cores_amd as fs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "fsattn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fsattn_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = fs.lib()
    decl = header_functions()
    assert set(decl) == set(fs.ABI_SYMBOLS), decl
    for name in decl:
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    L = fs.lib()
    assert L.fsattn_abi_version() == 3
    for s in (0, -1, -2, -3, -4):
        assert L.fsattn_status_str(s)
    assert L.fsattn_status_str(-99) == b"unknown status"


@pytest.mark.parametrize("elem,bits", [(0, 8), (1, 8), (2, 6), (3, 6), (4, 4)])
def test_size_helpers(elem, bits):
    # axis 0: [n][rows][cols/32] blocks
    assert fs.mx_sizes(elem, 2, 5, 128, 0) == (2 * 5 * 4 * bits * 4, 2 * 5 * 4)
    # axis 1: [n][cols][ceil(rows/32)] blocks
    assert fs.mx_sizes(elem, 3, 75600, 128, 1) == (3 * 128 * 2363 * bits * 4, 3 * 128 * 2363)
    with pytest.raises(ValueError):
        fs.mx_sizes(elem, 1, 4, 100, 0)  # cols % 32


def _params(**kw):
    base = dict(B=1, H=1, Sq=16, Skv=16, D=128, softmax_scale=128 ** -0.5, p_elem=2, p_scale_rule=0, tau=8.0,
                schraudolph_c=0.0,
                kv_tile=64, rollback_counts=None, p_dump_codes=None, p_dump_scales=None, p_b=0, p_h=0, p_row0=0,
                p_row1=0)
    base.update(kw)
    return fs._Params(**base)


def _mx(elem=2, prescale=None):
    ps = fs.fold_prescale(128 ** -0.5) if prescale is None else prescale
    return fs._MxTensor(elem, ps, 16, 16)  # fake aligned non-null pointers: validation only


def _call(p, q, k, v, out=16):
    return fs.lib().fsattn_forward(ctypes.byref(p), ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), out, None)


def test_forward_validation_rejects_before_launch():
    k1 = _mx(prescale=1.0)
    v1 = _mx(prescale=1.0)
    E = fs.lib()
    assert E.fsattn_forward(None, None, None, None, None, None) == -1
    assert _call(_params(D=96), _mx(), k1, v1) == -1                 # head dim
    assert _call(_params(kv_tile=80), _mx(), k1, v1) == -1           # gate tile: not a multiple of 32
    assert _call(_params(kv_tile=0), _mx(), k1, v1) == -1
    assert _call(_params(kv_tile=96), _mx(), k1, v1) == -2           # a multiple of 32 the kernels do not run
    assert _call(_params(kv_tile=256), _mx(), k1, v1) == -2
    assert _call(_params(p_scale_rule=2), _mx(), k1, v1) == -1       # rule enum
    assert _call(_params(p_scale_rule=1), _mx(), k1, v1) == -2       # OCP-floor P: not implemented
    assert _call(_params(tau=-1.0), _mx(), k1, v1) == -1             # tau
    assert _call(_params(Skv=0), _mx(), k1, v1) == -1                # no keys
    assert _call(_params(), _mx(prescale=3.0), k1, v1) == -1         # fold prescale mismatch
    assert _call(_params(), _mx(elem=2), _mx(elem=4, prescale=1.0), v1) == -1  # Q/K formats differ
    assert _call(_params(p_elem=4), _mx(), k1, v1) == -2             # FP4 P unsupported
    assert _call(_params(p_elem=0), _mx(), k1, v1) == -2             # FP8 P needs FP8 V
    assert _call(_params(p_elem=3, B=0), _mx(), k1, v1) == 0         # E3M2 P with E2M3 operands: accepted
    assert _call(_params(p_elem=3), _mx(elem=0), _mx(elem=0, prescale=1.0), _mx(elem=0, prescale=1.0)) == -2
    assert _call(_params(p_dump_codes=16, p_dump_scales=16, p_row0=4, p_row1=2), _mx(), k1, v1) == -1
    assert _call(_params(), _mx(), k1, v1, out=None) == -1
    bad = fs._MxTensor(2, fs.fold_prescale(128 ** -0.5), 8, 16)      # misaligned codes
    assert _call(_params(), bad, k1, v1) == -3
    assert _call(_params(Sq=0), _mx(), k1, v1) == 0                  # empty: OK, no launch


def test_quantize_validation():
    Q = fs.lib().fsattn_quantize_mx
    assert Q(16, 1, 4, 100, 100, 0, ctypes.c_float(1.0), 2, 0, 16, 16, None) == -1  # cols % 32
    assert Q(16, 1, 4, 128, 64, 0, ctypes.c_float(1.0), 2, 0, 16, 16, None) == -1   # ld < cols
    assert Q(16, 1, 4, 128, 128, 2, ctypes.c_float(1.0), 2, 0, 16, 16, None) == -1  # axis
    assert Q(16, 1, 4, 128, 128, 0, ctypes.c_float(1.0), 7, 0, 16, 16, None) == -1  # elem
    assert Q(16, 1, 4, 128, 128, 0, ctypes.c_float(1.0), 2, 5, 16, 16, None) == -1  # rule
    assert Q(16, 1, 4, 128, 128, 0, ctypes.c_float(1.0), 2, 0, 8, 16, None) == -3   # codes alignment
    assert Q(None, 1, 4, 128, 128, 0, ctypes.c_float(1.0), 2, 0, 16, 16, None) == -1
    assert Q(None, 0, 4, 128, 128, 0, ctypes.c_float(1.0), 2, 0, None, None, None) == 0  # empty


def test_bf16_baseline_validation():
    B = fs.lib().fsattn_forward_bf16_baseline
    assert B(16, 16, 16, 1, 1, 8, 8, 96, ctypes.c_float(0.1), 16, None) == -1
    assert B(16, 16, 16, 1, 1, 8, 0, 128, ctypes.c_float(0.1), 16, None) == -1
    assert B(8, 16, 16, 1, 1, 8, 8, 128, ctypes.c_float(0.1), 16, None) == -3
    assert B(16, 16, 16, 1, 1, 0, 8, 128, ctypes.c_float(0.1), 16, None) == 0


def test_masked_forward_validation_rejects_before_launch():
    k1 = _mx(prescale=1.0)
    v1 = _mx(prescale=1.0)
    M = fs.lib().fsattn_forward_masked

    def call(mask, p=None):
        p = _params() if p is None else p
        q = _mx()
        return M(ctypes.byref(p), ctypes.byref(mask) if mask is not None else None, ctypes.byref(q),
                 ctypes.byref(k1), ctypes.byref(v1), 16, None)

    assert M(None, None, None, None, None, None, None) == -1
    assert call(fs._Mask(2, None, None)) == -1                        # causal must be 0 or 1
    assert call(fs._Mask(1, 2, None)) == -3                           # q_lens alignment
    assert call(fs._Mask(0, None, 6)) == -3                           # kv_lens alignment
    assert call(fs._Mask(1, 16, 16), _params(D=96)) == -1             # the fsattn_forward checks still apply
    assert call(fs._Mask(1, 16, 16), _params(Sq=0)) == 0              # empty: OK, no launch
    assert call(None, _params(B=0)) == 0                              # NULL mask = fsattn_forward


def test_fp8_products_forward_validation_rejects_before_launch():
    """The FP8-product entry point shares the forward's checks (and its NULL mask)."""
    k1 = _mx(prescale=1.0)
    v1 = _mx(prescale=1.0)
    F = fs.lib().fsattn_forward_fp8_products

    def call(mask, p=None, q=None):
        p = _params() if p is None else p
        q = _mx() if q is None else q
        return F(ctypes.byref(p), ctypes.byref(mask) if mask is not None else None, ctypes.byref(q),
                 ctypes.byref(k1), ctypes.byref(v1), 16, None)

    assert F(None, None, None, None, None, None, None) == -1
    assert call(None, _params(D=96)) == -1                            # head dim
    assert call(None, _params(kv_tile=96)) == -2                      # gate tile the kernels do not run
    assert call(fs._Mask(2, None, None)) == -1                        # causal must be 0 or 1
    assert call(None, _params(p_elem=4)) == -2                        # FP4 P: only the EFQ-style entry point
    assert call(None, q=_mx(prescale=3.0)) == -1                      # fold prescale mismatch
    assert call(None, _params(Sq=0)) == 0                             # empty: OK, no launch
    assert call(fs._Mask(1, 16, 16), _params(B=0)) == 0


def test_rmsnorm_quantize_validation():
    R = fs.lib().fsattn_quantize_mx_rmsnorm
    f = ctypes.c_float

    def call(cols=128, ld=128, weight=None, eps=1e-6, pre=1.0, elem=2, rule=0, src=16, codes=16):
        return R(src, 1, 4, cols, ld, weight, f(eps), f(pre), elem, rule, codes, 16, None)

    assert call(cols=100, ld=100) == -1                    # cols % 32
    assert call(ld=64) == -1                               # ld < cols
    assert call(eps=-1.0) == -1                            # eps
    assert call(pre=float("inf")) == -1                    # prescale
    assert call(elem=7) == -1 and call(rule=3) == -1       # enums
    assert call(cols=96, ld=96) == -2                      # not a power of two
    assert call(cols=4096, ld=4096) == -2                  # beyond one wave per row
    assert call(codes=8) == -3 and call(weight=6) == -3    # alignment
    assert call(src=None) == -1
    assert R(None, 0, 4, 128, 128, None, f(1e-6), f(1.0), 2, 0, None, None, None) == 0  # empty


def test_bf16_masked_validation():
    B = fs.lib().fsattn_forward_bf16_baseline_masked
    f = ctypes.c_float(0.1)
    assert B(16, 16, 16, 1, 1, 8, 8, 128, f, ctypes.byref(fs._Mask(2, None, None)), 16, None) == -1
    assert B(16, 16, 16, 1, 1, 8, 8, 128, f, ctypes.byref(fs._Mask(1, 2, None)), 16, None) == -3
    assert B(16, 16, 16, 1, 1, 8, 8, 96, f, ctypes.byref(fs._Mask(1, None, None)), 16, None) == -1
    assert B(16, 16, 16, 1, 1, 0, 8, 128, f, ctypes.byref(fs._Mask(1, 16, 16)), 16, None) == 0
    assert B(16, 16, 16, 1, 1, 0, 8, 128, f, None, 16, None) == 0


def _call_efq(p, q, k, v, tau=-3.875, h=0.609375, out=16, mask=None):
    return fs.lib().fsattn_forward_efq(ctypes.byref(p), mask, ctypes.c_float(tau), ctypes.c_float(h),
                                       ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), out, None)


def test_forward_efq_validation_rejects_before_launch():
    k1, v1 = _mx(prescale=1.0), _mx(prescale=1.0)
    assert _call_efq(_params(p_elem=2), _mx(), k1, v1) == -1            # P must be E2M1
    for h in (1 / 128, 17.0, float("nan"), float("inf")):
        assert _call_efq(_params(p_elem=4), _mx(), k1, v1, h=h) == -1, h
    for tau in (-65.0, 65.0, float("nan")):
        assert _call_efq(_params(p_elem=4), _mx(), k1, v1, tau=tau) == -1, tau
    assert _call_efq(_params(p_elem=4, tau=-1.0), _mx(), k1, v1) == -1  # gate tau
    # Q/K/V must all be E2M3 or all E2M1
    assert _call_efq(_params(p_elem=4), _mx(elem=2), k1, _mx(elem=4, prescale=1.0)) == -2
    assert _call_efq(_params(p_elem=4), _mx(elem=0), _mx(elem=0, prescale=1.0), _mx(elem=0, prescale=1.0)) == -2
    # a valid call with nothing to do returns OK without launching
    assert _call_efq(_params(p_elem=4, B=0), _mx(), k1, v1) == 0
    e4 = _mx(elem=4)
    assert _call_efq(_params(p_elem=4, H=0), e4, _mx(elem=4, prescale=1.0), _mx(elem=4, prescale=1.0)) == 0
    bad = fs._MxTensor(2, fs.fold_prescale(128 ** -0.5), 8, 16)
    assert _call_efq(_params(p_elem=4), bad, k1, v1) == -3               # misaligned codes
    m = fs._Mask(2, None, None)
    assert _call_efq(_params(p_elem=4), _mx(), k1, v1, mask=ctypes.byref(m)) == -1  # causal not 0/1


def test_efq_defaults_are_the_stored_calibration():
    """The binding's default (tau, h) for E2M1 P is the point the offline
    calibration (tests/golden/make_efq_calibration.py, oracle only) stored."""
    import json
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "efq_calibration.json")))
    assert (fs.EFQ_TAU, fs.EFQ_H) == (gold["efq_tau"], gold["efq_h"])


@pytest.mark.parametrize("tau,c", [(0.0, 0.0), (1.0, 0.0), (8.0, 0.0), (2.7, 0.0), (127.0, 0.0), (8.0, 5.5),
                                   (3.25, -20.0)])
def test_pattern_gate_tau_gives_the_shifted_threshold(tau, c):
    """T_gate(tau') is the largest binary32 below floor(T_gate(tau)) + 1."""
    import math
    import numpy as np
    t2 = fs.pattern_gate_tau(tau, c)
    tg = float(np.float32(128.0 * (127.0 + float(np.float32(tau))) - c))
    tg2 = float(np.float32(128.0 * (127.0 + t2) - c))
    assert tg2 == float(np.nextafter(np.float32(math.floor(tg) + 1), np.float32(0)))
    assert tg2 >= tg


def test_pattern_gate_tau_extreme_range_and_errors():
    import numpy as np
    assert fs.pattern_gate_tau(128.0) == float(np.finfo(np.float32).max)
    assert fs.pattern_gate_tau(500.0) == float(np.finfo(np.float32).max)
    out = ctypes.c_float()
    L = fs.lib()
    assert L.fsattn_pattern_gate_tau(ctypes.c_float(-1.0), ctypes.c_float(0.0), ctypes.byref(out)) == -1
    assert L.fsattn_pattern_gate_tau(ctypes.c_float(float("nan")), ctypes.c_float(0.0), ctypes.byref(out)) == -1
    assert L.fsattn_pattern_gate_tau(ctypes.c_float(1.0), ctypes.c_float(0.0), None) == -1


def test_fold_prescale_is_the_rounded_product():
    """fsattn_fold_prescale(sigma) = fl32(128 log2(e) sigma) for the binary32
    sigma it takes: the binary64 product rounded once (numpy's float32
    rounding of the same product)."""
    import math
    import numpy as np
    for sigma in (128 ** -0.5, 0.125, 1.0, 1e-3, 0.3):
        s32 = float(np.float32(sigma))
        want = float(np.float32(128.0 * math.log2(math.e) * s32))
        assert fs.fold_prescale(sigma) == want
    assert abs(fs.fold_prescale(128 ** -0.5) - 16.322231) < 1e-5
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            fs.fold_prescale(bad)
