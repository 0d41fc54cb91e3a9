"""ctypes wrapper around the CPU oracle (``fsattn_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the library under
``softmax_matrix_cores_amd`` never does.  The oracle is the plain, slow CPU
definition of the Fused-Softmax forward pass as the pages describe it
("Fused-Softmax shifts an AI attention bottleneck onto faster GPU hardware",
paragraphs 5-6: frozen reference folded into the score product, Schraudolph
exponential, two-stage BF16 -> MX conversion, P.1 denominator with the same P,
rollback gate).  Its readings of the open points are listed in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "fsattn_oracle.c")

E4M3, E5M2, E2M3, E3M2, E2M1 = 0, 1, 2, 3, 4
ELEM_NAMES = {"e4m3": E4M3, "e5m2": E5M2, "e2m3": E2M3, "e3m2": E3M2, "e2m1": E2M1}
SCALE_FITMAX, SCALE_OCP_FLOOR = 0, 1
EXP_SCHRAUDOLPH, EXP_EXACT = 0, 1
P_MX, P_NONE, P_EFQ = 0, 1, 2
GATE_EXACT, GATE_PATTERN = 0, 1
FOLD_FP32, FOLD_EXACT = 0, 1
REF_R1, REF_R2, REF_R2P, REF_R3 = 1, 2, 3, 4


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-pthread", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("Sq", ctypes.c_int), ("Skv", ctypes.c_int), ("D", ctypes.c_int),
        ("qk_elem", ctypes.c_int), ("v_elem", ctypes.c_int), ("p_elem", ctypes.c_int), ("scale_rule", ctypes.c_int),
        ("tau", ctypes.c_double), ("c", ctypes.c_double), ("kv_tile", ctypes.c_int),
        ("exp_mode", ctypes.c_int), ("p_mode", ctypes.c_int), ("fold_mode", ctypes.c_int),
        ("nthreads", ctypes.c_int), ("efq_tau", ctypes.c_double), ("efq_h", ctypes.c_double),
        ("gate_mode", ctypes.c_int), ("gate_misses", ctypes.c_void_p),
    ]


class Mask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int), ("q_lens", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.fso_decode.restype = ctypes.c_double
        L.fso_decode.argtypes = [ctypes.c_int, ctypes.c_int]
        L.fso_encode.argtypes = [ctypes.c_int, ctypes.c_double]
        L.fso_elem_maxnorm.restype = ctypes.c_double
        L.fso_elem_maxnorm.argtypes = [ctypes.c_int]
        L.fso_scale_code.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double]
        L.fso_mxq_block.argtypes = [ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P, P]
        L.fso_block_bytes.argtypes = [ctypes.c_int]
        L.fso_quantize_mx.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int, P, P]
        L.fso_quantize_mx_rmsnorm.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                              P, ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int, P, P]
        L.fso_stage1.restype = ctypes.c_uint16
        L.fso_stage1.argtypes = [ctypes.c_float]
        L.fso_efq_block.argtypes = [P, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_double, P, P]
        L.fso_forward.argtypes = [ctypes.POINTER(Params), P, P, P, P, P, P, P, ctypes.c_int64, P, P, P, P, P]
        L.fso_forward_scores.argtypes = [ctypes.POINTER(Params), ctypes.c_void_p, P, P, P, P, P, P, P,
                                         ctypes.c_int64, P, P]
        L.fso_forward_masked.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Mask), P, P, P, P, P, P, P,
                                         ctypes.c_int64, P, P, P, P, P]
        L.fso_reference.argtypes = [ctypes.POINTER(Params), ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_int64, P]
        L.fso_reference_bf16.argtypes = [ctypes.c_int] * 5 + [ctypes.c_double, P, P, P, P, ctypes.c_int64,
                                                              ctypes.c_int, P]
        L.fso_reference_bf16_masked.argtypes = [ctypes.c_int] * 5 + [ctypes.c_double, ctypes.POINTER(Mask), P, P, P,
                                                                     P, ctypes.c_int64, ctypes.c_int, P]
        L.fso_folded_score.restype = ctypes.c_double
        L.fso_folded_score.argtypes = [ctypes.c_int, P, P, P, P, ctypes.c_int, ctypes.c_double, ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def elem_bits(elem: int) -> int:
    return {E4M3: 8, E5M2: 8, E2M3: 6, E3M2: 6, E2M1: 4}[elem]


def decode(elem: int, code: int) -> float:
    return lib().fso_decode(elem, int(code))


def encode(elem: int, x: float) -> int:
    return lib().fso_encode(elem, float(x))


def maxnorm(elem: int) -> float:
    return lib().fso_elem_maxnorm(elem)


def scale_code(elem: int, rule: int, amax: float) -> int:
    return lib().fso_scale_code(elem, rule, float(amax))


def mxq_block(elem: int, rule: int, x) -> tuple[np.ndarray, int]:
    x = np.ascontiguousarray(x, dtype=np.float64)
    codes = np.zeros(len(x), np.uint8)
    sc = np.zeros(1, np.uint8)
    lib().fso_mxq_block(elem, rule, _ptr(x), len(x), _ptr(codes), _ptr(sc))
    return codes, int(sc[0])


def stage1(t: float) -> int:
    return int(lib().fso_stage1(float(t)))


def block_bytes(elem: int) -> int:
    return elem_bits(elem) * 4


def quantize_mx(x_bf16: np.ndarray, block_axis: int, elem: int, prescale: float = 1.0,
                rule: int = SCALE_FITMAX) -> tuple[np.ndarray, np.ndarray]:
    """x_bf16: uint16 array [n_mat, rows, cols] of bf16 bit patterns."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.ndim == 3
    n_mat, rows, cols = x.shape
    bb = block_bytes(elem)
    if block_axis == 0:
        codes = np.zeros((n_mat, rows, cols // 32 * bb), np.uint8)
        scales = np.zeros((n_mat, rows, cols // 32), np.uint8)
    else:
        r32 = (rows + 31) // 32 * 32
        codes = np.zeros((n_mat, cols, r32 // 32 * bb), np.uint8)
        scales = np.zeros((n_mat, cols, r32 // 32), np.uint8)
    rc = lib().fso_quantize_mx(_ptr(x), n_mat, rows, cols, cols, block_axis, ctypes.c_float(prescale), elem, rule,
                               _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"fso_quantize_mx failed ({rc})")
    return codes, scales


def quantize_mx_rmsnorm(x_bf16: np.ndarray, elem: int, prescale: float = 1.0, weight=None, eps: float = 1e-6,
                        rule: int = SCALE_FITMAX) -> tuple[np.ndarray, np.ndarray]:
    """RMS-normalised rows, then the prescale and MX quantization (block_axis 0).
    x_bf16: uint16 [n_mat, rows, cols]; weight: float32 [cols] or None."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.ndim == 3
    n_mat, rows, cols = x.shape
    bb = block_bytes(elem)
    codes = np.zeros((n_mat, rows, cols // 32 * bb), np.uint8)
    scales = np.zeros((n_mat, rows, cols // 32), np.uint8)
    w = None if weight is None else np.ascontiguousarray(weight, dtype=np.float32)
    if w is not None and w.shape != (cols,):
        raise ValueError("weight must have cols entries")
    rc = lib().fso_quantize_mx_rmsnorm(_ptr(x), n_mat, rows, cols, cols, _ptr(w), ctypes.c_float(eps),
                                       ctypes.c_float(prescale), elem, rule, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError(f"fso_quantize_mx_rmsnorm failed ({rc})")
    return codes, scales


def make_params(B, H, Sq, Skv, D, qk_elem, v_elem, p_elem, tau=8.0, c=0.0, kv_tile=64, scale_rule=SCALE_FITMAX,
                exp_mode=EXP_SCHRAUDOLPH, p_mode=P_MX, fold_mode=FOLD_FP32, nthreads=0, efq_tau=0.0,
                efq_h=0.5, gate_mode=GATE_EXACT) -> Params:
    return Params(B, H, Sq, Skv, D, qk_elem, v_elem, p_elem, scale_rule, float(tau), float(c), kv_tile,
                  exp_mode, p_mode, fold_mode, nthreads, float(efq_tau), float(efq_h), gate_mode, None)


def efq_block(t, T0: float, tau: float, h: float, nvis: int | None = None):
    """R24 on one block: t = up to 32 folded binary32 scores (keys past nvis
    absent).  Returns (codes uint8[32], E8M0 int)."""
    tf = np.zeros(32, np.float32)
    t = np.asarray(t, np.float32)
    tf[:len(t)] = t
    n = len(t) if nvis is None else nvis
    codes = np.zeros(32, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib().fso_efq_block(_ptr(tf), int(n), ctypes.c_float(T0), ctypes.c_double(tau), ctypes.c_double(h), _ptr(codes),
                        _ptr(sc))
    return codes, int(sc[0])


def forward(p: Params, q, k, v, rows=None, want_p=False, causal=False, q_lens=None, kv_lens=None):
    """q, k, v: (codes, scales) tuples in the quantizer layout.  Returns dict.
    causal / q_lens / kv_lens: the mask of fso_forward_masked (lens: [B] ints).
    With p.gate_mode GATE_PATTERN the dict also holds the per-row "misses"."""
    nrows = p.B * p.H * p.Sq if rows is None else len(rows)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    O = np.zeros((nrows, p.D), np.float64)
    L = np.zeros(nrows, np.float64)
    cnt = np.zeros(nrows, np.int32)
    s32 = (p.Skv + 31) // 32 * 32
    pc = np.zeros((nrows, s32), np.uint8) if want_p else None
    ps = np.zeros((nrows, s32 // 32), np.uint8) if want_p else None
    args = [np.ascontiguousarray(a) for a in (q[0], q[1], k[0], k[1], v[0], v[1])]
    misses = np.zeros(nrows, np.int32)
    p.gate_misses = _ptr(misses)
    if causal or q_lens is not None or kv_lens is not None:
        ql = None if q_lens is None else np.ascontiguousarray(q_lens, dtype=np.int32)
        kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
        for a in (ql, kl):
            if a is not None and a.shape != (p.B,):
                raise ValueError("q_lens / kv_lens must have B entries")
        m = Mask(1 if causal else 0, _ptr(ql), _ptr(kl))
        rc = lib().fso_forward_masked(ctypes.byref(p), ctypes.byref(m), *[_ptr(a) for a in args], _ptr(rows_a),
                                      nrows, _ptr(O), _ptr(L), _ptr(cnt), _ptr(pc), _ptr(ps))
    else:
        rc = lib().fso_forward(ctypes.byref(p), *[_ptr(a) for a in args], _ptr(rows_a), nrows, _ptr(O), _ptr(L),
                               _ptr(cnt), _ptr(pc), _ptr(ps))
    if rc != 0:
        raise ValueError(f"fso_forward failed ({rc})")
    p.gate_misses = None
    out = {"O": O, "l": L, "counts": cnt, "misses": misses}
    if want_p:
        out["p_codes"] = pc
        out["p_scales"] = ps
    return out


def forward_scores(p: Params, q, k, v, rows, causal=False, q_lens=None, kv_lens=None):
    """Diagnostics for the given rows: the folded binary32 scores stage 1 sees
    (after each tile's gate shift; invisible keys left 0) and max_d |Qhat Khat|
    per (row, key), both [rows, Skv32] (fso_forward_scores; masks as forward)."""
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    s32 = (p.Skv + 31) // 32 * 32
    t = np.zeros((len(rows_a), s32), np.float32)
    a = np.zeros((len(rows_a), s32), np.float64)
    args = [np.ascontiguousarray(x) for x in (q[0], q[1], k[0], k[1], v[0], v[1])]
    m = None
    if causal or q_lens is not None or kv_lens is not None:
        ql = None if q_lens is None else np.ascontiguousarray(q_lens, dtype=np.int32)
        kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
        m = Mask(1 if causal else 0, _ptr(ql), _ptr(kl))
    rc = lib().fso_forward_scores(ctypes.byref(p), ctypes.byref(m) if m is not None else None,
                                  *[_ptr(x) for x in args], _ptr(rows_a), len(rows_a), _ptr(t), _ptr(a))
    if rc != 0:
        raise ValueError(f"fso_forward_scores failed ({rc})")
    return t, a


def reference(p: Params, ref: int, q, k, v, rows=None) -> np.ndarray:
    nrows = p.B * p.H * p.Sq if rows is None else len(rows)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    O = np.zeros((nrows, p.D), np.float64)
    args = [np.ascontiguousarray(a) for a in (q[0], q[1], k[0], k[1], v[0], v[1])]
    rc = lib().fso_reference(ctypes.byref(p), ref, *[_ptr(a) for a in args], _ptr(rows_a), nrows, _ptr(O))
    if rc != 0:
        raise ValueError(f"fso_reference failed ({rc})")
    return O


def reference_bf16(q, k, v, sigma: float, rows=None, nthreads: int = 0, causal=False, q_lens=None,
                   kv_lens=None) -> np.ndarray:
    """R0: exact softmax attention on bf16 inputs (uint16 arrays [B,H,S,D]); with
    causal / q_lens / kv_lens, over each row's visible keys (fso_reference_bf16_masked)."""
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    nrows = B * H * Sq if rows is None else len(rows)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    O = np.zeros((nrows, D), np.float64)
    if causal or q_lens is not None or kv_lens is not None:
        ql = None if q_lens is None else np.ascontiguousarray(q_lens, dtype=np.int32)
        kl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
        m = Mask(1 if causal else 0, _ptr(ql), _ptr(kl))
        rc = lib().fso_reference_bf16_masked(B, H, Sq, Skv, D, float(sigma), ctypes.byref(m), _ptr(q), _ptr(k),
                                             _ptr(v), _ptr(rows_a), nrows, nthreads, _ptr(O))
    else:
        rc = lib().fso_reference_bf16(B, H, Sq, Skv, D, float(sigma), _ptr(q), _ptr(k), _ptr(v), _ptr(rows_a),
                                      nrows, nthreads, _ptr(O))
    if rc != 0:
        raise ValueError(f"fso_reference_bf16 failed ({rc})")
    return O


def folded_score(qk_elem, qcodes, qscales, kcodes, kscales, D, cinit, exact=False) -> float:
    a = [np.ascontiguousarray(x, np.uint8) for x in (qcodes, qscales, kcodes, kscales)]
    return lib().fso_folded_score(qk_elem, *[_ptr(x) for x in a], D, float(cinit), int(exact))


def softmax_scale_prescale(sigma: float) -> float:
    """alpha = fl32(128 * log2(e) * sigma): the multiplicative part of the fold."""
    return float(np.float32(128.0 * np.log2(np.e) * sigma))
