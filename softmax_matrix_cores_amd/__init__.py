"""softmax_matrix_cores_amd -- Fused-Softmax quantized attention on AMD MI355X.

Thin ctypes binding over the C ABI in ``include/fsattn.h`` (``libfsattn.so``,
built in-tree by ``softmax_matrix_cores_amd.build``).  This module only
marshals arguments: every step of the attention path runs in the HIP kernels.
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsattn.so")

E4M3, E5M2, E2M3, E3M2, E2M1 = 0, 1, 2, 3, 4
ELEMS = {"e4m3": E4M3, "e5m2": E5M2, "e2m3": E2M3, "e3m2": E3M2, "e2m1": E2M1}
ELEM_BITS = {E4M3: 8, E5M2: 8, E2M3: 6, E3M2: 6, E2M1: 4}
SCALE_FITMAX, SCALE_OCP_FLOOR = 0, 1

# every symbol include/fsattn.h declares
ABI_SYMBOLS = (
    "fsattn_abi_version", "fsattn_status_str", "fsattn_mx_codes_bytes", "fsattn_mx_scales_bytes",
    "fsattn_quantize_mx", "fsattn_quantize_mx_rmsnorm", "fsattn_forward", "fsattn_forward_masked",
    "fsattn_forward_bf16_baseline", "fsattn_forward_bf16_baseline_masked", "fsattn_forward_efq",
    "fsattn_forward_fp8_products",
    "fsattn_pattern_gate_tau", "fsattn_probe_mfma", "fsattn_fold_prescale",
)

# (tau, h) of the EFQ-style E2M1 P rule (fsattn_forward_efq), calibrated offline
# on synthetic MXFP4 attention by minimizing the output error against exact
# softmax on the same quantized operands
EFQ_TAU, EFQ_H = -3.875, 0.609375


class FsattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().fsattn_status_str(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")


class _MxTensor(ctypes.Structure):
    _fields_ = [("elem", ctypes.c_int), ("prescale", ctypes.c_float), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


class _Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("Sq", ctypes.c_int), ("Skv", ctypes.c_int), ("D", ctypes.c_int),
        ("softmax_scale", ctypes.c_float), ("p_elem", ctypes.c_int), ("p_scale_rule", ctypes.c_int),
        ("tau", ctypes.c_float),
        ("schraudolph_c", ctypes.c_float), ("kv_tile", ctypes.c_int),
        ("rollback_counts", ctypes.c_void_p), ("p_dump_codes", ctypes.c_void_p), ("p_dump_scales", ctypes.c_void_p),
        ("p_b", ctypes.c_int), ("p_h", ctypes.c_int), ("p_row0", ctypes.c_int), ("p_row1", ctypes.c_int),
    ]


class _Mask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int), ("q_lens", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfsattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m softmax_matrix_cores_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        V, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.fsattn_abi_version.restype = I
        L.fsattn_fold_prescale.restype = ctypes.c_float
        L.fsattn_fold_prescale.argtypes = [ctypes.c_float]
        L.fsattn_status_str.restype = ctypes.c_char_p
        L.fsattn_status_str.argtypes = [I]
        L.fsattn_mx_codes_bytes.restype = I64
        L.fsattn_mx_codes_bytes.argtypes = [I, I64, I64, I64, I]
        L.fsattn_mx_scales_bytes.restype = I64
        L.fsattn_mx_scales_bytes.argtypes = [I64, I64, I64, I]
        L.fsattn_quantize_mx.restype = I
        L.fsattn_quantize_mx.argtypes = [V, I64, I64, I64, I64, I, ctypes.c_float, I, I, V, V, V]
        L.fsattn_quantize_mx_rmsnorm.restype = I
        L.fsattn_quantize_mx_rmsnorm.argtypes = [V, I64, I64, I64, I64, V, ctypes.c_float, ctypes.c_float, I, I, V,
                                                 V, V]
        L.fsattn_forward.restype = I
        L.fsattn_forward.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(_MxTensor), ctypes.POINTER(_MxTensor),
                                     ctypes.POINTER(_MxTensor), V, V]
        L.fsattn_forward_masked.restype = I
        L.fsattn_forward_masked.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(_Mask),
                                            ctypes.POINTER(_MxTensor), ctypes.POINTER(_MxTensor),
                                            ctypes.POINTER(_MxTensor), V, V]
        L.fsattn_forward_fp8_products.restype = I
        L.fsattn_forward_fp8_products.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(_Mask),
                                                  ctypes.POINTER(_MxTensor), ctypes.POINTER(_MxTensor),
                                                  ctypes.POINTER(_MxTensor), V, V]
        L.fsattn_forward_efq.restype = I
        L.fsattn_forward_efq.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(_Mask), ctypes.c_float,
                                         ctypes.c_float, ctypes.POINTER(_MxTensor), ctypes.POINTER(_MxTensor),
                                         ctypes.POINTER(_MxTensor), V, V]
        L.fsattn_pattern_gate_tau.restype = I
        L.fsattn_pattern_gate_tau.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_float)]
        L.fsattn_probe_mfma.restype = I
        L.fsattn_probe_mfma.argtypes = [I, I64, I, V, ctypes.POINTER(ctypes.c_int), V]
        L.fsattn_forward_bf16_baseline.restype = I
        L.fsattn_forward_bf16_baseline.argtypes = [V, V, V, I, I, I, I, I, ctypes.c_float, V, V]
        L.fsattn_forward_bf16_baseline_masked.restype = I
        L.fsattn_forward_bf16_baseline_masked.argtypes = [V, V, V, I, I, I, I, I, ctypes.c_float,
                                                          ctypes.POINTER(_Mask), V, V]
        _lib = L
    return _lib


def _elem(e) -> int:
    return ELEMS[e] if isinstance(e, str) else int(e)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise FsattnError(fn, status)


def fold_prescale(softmax_scale: float) -> float:
    """fl32(128 * log2(e) * softmax_scale): the multiplicative part of the fold (fsattn_fold_prescale)."""
    v = lib().fsattn_fold_prescale(ctypes.c_float(softmax_scale))
    if v != v:
        raise ValueError(f"softmax_scale must be positive and finite, got {softmax_scale}")
    return float(v)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, numel: int, device: torch.device):
    """Check a buffer before its pointer goes to the library, which has no size
    information: dtype, device, contiguity and at least `numel` elements."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {numel}")


@dataclass
class MXTensor:
    codes: torch.Tensor   # uint8, packed codes
    scales: torch.Tensor  # uint8, E8M0
    elem: int
    prescale: float

    def _c(self) -> _MxTensor:
        return _MxTensor(self.elem, self.prescale, self.codes.data_ptr(), self.scales.data_ptr())


def mx_sizes(elem, n_mat: int, rows: int, cols: int, block_axis: int) -> tuple[int, int]:
    e = _elem(elem)
    cb = lib().fsattn_mx_codes_bytes(e, n_mat, rows, cols, block_axis)
    sb = lib().fsattn_mx_scales_bytes(n_mat, rows, cols, block_axis)
    if cb < 0 or sb < 0:
        raise ValueError("invalid MX tensor shape")
    return cb, sb


def quantize_mx(x: torch.Tensor, block_axis: int, elem, prescale: float = 1.0, rule: int = SCALE_FITMAX,
                stream=None, out: MXTensor | None = None) -> MXTensor:
    """MX-quantize a contiguous bf16 CUDA tensor viewed as [n_mat, rows, cols] (last two dims)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda:
        raise TypeError("quantize_mx expects a bf16 CUDA tensor")
    x = x.contiguous()
    rows, cols = x.shape[-2], x.shape[-1]
    n_mat = x.numel() // max(1, rows * cols) if rows * cols else 0
    e = _elem(elem)
    cb, sb = mx_sizes(e, n_mat, rows, cols, block_axis)
    if out is None:
        codes = torch.empty(cb, dtype=torch.uint8, device=x.device)
        scales = torch.empty(sb, dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out.codes, out.scales
    st = lib().fsattn_quantize_mx(x.data_ptr(), n_mat, rows, cols, cols, block_axis, ctypes.c_float(prescale), e,
                                  rule, codes.data_ptr(), scales.data_ptr(), _stream(stream))
    _check("fsattn_quantize_mx", st)
    return MXTensor(codes, scales, e, float(torch.tensor(prescale, dtype=torch.float32)))


def quantize_mx_rmsnorm(x: torch.Tensor, elem, prescale: float = 1.0, weight: torch.Tensor | None = None,
                        eps: float = 1e-6, rule: int = SCALE_FITMAX, stream=None,
                        out: MXTensor | None = None) -> MXTensor:
    """RMS-normalise the rows of a contiguous bf16 CUDA tensor [..., rows, cols] (optional float32
    weight [cols]), then apply the prescale and MX-quantize along the rows (block_axis 0)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda:
        raise TypeError("quantize_mx_rmsnorm expects a bf16 CUDA tensor")
    x = x.contiguous()
    rows, cols = x.shape[-2], x.shape[-1]
    n_mat = x.numel() // max(1, rows * cols) if rows * cols else 0
    e = _elem(elem)
    if weight is not None and (weight.dtype != torch.float32 or weight.device != x.device or
                               weight.shape != (cols,) or not weight.is_contiguous()):
        raise ValueError("weight must be a contiguous float32 [cols] tensor on the input's device")
    cb, sb = mx_sizes(e, n_mat, rows, cols, 0)
    if out is None:
        codes = torch.empty(cb, dtype=torch.uint8, device=x.device)
        scales = torch.empty(sb, dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out.codes, out.scales
    st = lib().fsattn_quantize_mx_rmsnorm(x.data_ptr(), n_mat, rows, cols, cols,
                                          weight.data_ptr() if weight is not None else None, ctypes.c_float(eps),
                                          ctypes.c_float(prescale), e, rule, codes.data_ptr(), scales.data_ptr(),
                                          _stream(stream))
    _check("fsattn_quantize_mx_rmsnorm", st)
    return MXTensor(codes, scales, e, float(torch.tensor(prescale, dtype=torch.float32)))


def quantize_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, qk_elem, v_elem, softmax_scale: float,
                 stream=None) -> tuple[MXTensor, MXTensor, MXTensor]:
    """Quantize [B,H,S,D] bf16 Q (with the folded prescale), K and V (blocks along keys)."""
    Q = quantize_mx(q, 0, qk_elem, prescale=fold_prescale(softmax_scale), stream=stream)
    K = quantize_mx(k, 0, qk_elem, stream=stream)
    V = quantize_mx(v, 1, v_elem, stream=stream)
    return Q, K, V


def forward(Q: MXTensor, K: MXTensor, V: MXTensor, B: int, H: int, Sq: int, Skv: int, D: int, softmax_scale: float,
            p_elem, tau: float = 8.0, c: float = 0.0, kv_tile: int = 64, counts: torch.Tensor | None = None,
            out: torch.Tensor | None = None, p_dump: tuple | None = None, stream=None, causal: bool = False,
            q_lens: torch.Tensor | None = None, kv_lens: torch.Tensor | None = None, efq_tau: float = EFQ_TAU,
            efq_h: float = EFQ_H, gate: str = "exact", p_scale_rule: int = SCALE_FITMAX,
            fp8_products: bool = False) -> torch.Tensor:
    """Fused-Softmax attention forward.  Returns bf16 [B,H,Sq,D].
    counts: optional int32 [B,H,Sq] written with rollback counts.
    p_dump: optional (b, h, row0, row1, codes uint8 [rows, Skv32], scales uint8 [rows, Skv32/32]).
    causal / q_lens / kv_lens: masks (fsattn_forward_masked); lens are device int32 [B].
    p_elem "e2m1": P straight from the scores by the EFQ-style rule with (efq_tau, efq_h)
    (fsattn_forward_efq).
    gate "pattern": the gate shortcut on stage-1 patterns (fsattn_pattern_gate_tau).
    fp8_products: E4M3 Q/K scores from the FP8 matrix core (fsattn_forward_fp8_products) instead
    of the exact BF16 decode.
    Every buffer is checked (dtype, device, contiguity, size) before the call."""
    dev = Q.codes.device
    if gate == "pattern":
        tau = pattern_gate_tau(tau, c)
    elif gate != "exact":
        raise ValueError(f"unknown gate {gate!r}")
    if min(B, H, Sq) < 0 or Skv < 1 or D not in (64, 128):
        raise ValueError(f"bad shape B={B} H={H} Sq={Sq} Skv={Skv} D={D}")
    # the library sees raw pointers only: every buffer is checked here against
    # the sizes the shapes imply
    for X, name, rows, axis in ((Q, "Q", Sq, 0), (K, "K", Skv, 0), (V, "V", Skv, 1)):
        cb, sb = mx_sizes(X.elem, B * H, rows, D, axis)
        _need(X.codes, name + ".codes", torch.uint8, cb, dev)
        _need(X.scales, name + ".scales", torch.uint8, sb, dev)
    if out is None:
        out = torch.empty(B, H, Sq, D, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, B * H * Sq * D, dev)
    if counts is not None:
        _need(counts, "counts", torch.int32, B * H * Sq, dev)
    p = _Params(B, H, Sq, Skv, D, softmax_scale, _elem(p_elem), p_scale_rule, tau, c, kv_tile,
                counts.data_ptr() if counts is not None else None, None, None, 0, 0, 0, 0)
    if p_dump is not None:
        b, h, r0, r1, pc, ps = p_dump
        if not (0 <= b < B and 0 <= h < H and 0 <= r0 < r1 <= Sq):
            raise ValueError(f"bad P dump window {(b, h, r0, r1)}")
        s32 = (Skv + 31) // 32 * 32
        _need(pc, "p_dump codes", torch.uint8, (r1 - r0) * s32, dev)
        _need(ps, "p_dump scales", torch.uint8, (r1 - r0) * (s32 // 32), dev)
        p.p_dump_codes, p.p_dump_scales = pc.data_ptr(), ps.data_ptr()
        p.p_b, p.p_h, p.p_row0, p.p_row1 = b, h, r0, r1
    q, k, v = Q._c(), K._c(), V._c()
    masked = causal or q_lens is not None or kv_lens is not None
    if masked:
        for t in (q_lens, kv_lens):
            if t is not None and (t.dtype != torch.int32 or t.device != dev or t.shape != (B,) or
                                  not t.is_contiguous()):
                raise ValueError("q_lens / kv_lens must be contiguous int32 [B] on the operands' device")
        m = _Mask(1 if causal else 0, q_lens.data_ptr() if q_lens is not None else None,
                  kv_lens.data_ptr() if kv_lens is not None else None)
    if p.p_elem == ELEMS["e2m1"]:
        st = lib().fsattn_forward_efq(ctypes.byref(p), ctypes.byref(m) if masked else None, ctypes.c_float(efq_tau),
                                      ctypes.c_float(efq_h), ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                      out.data_ptr(), _stream(stream))
        _check("fsattn_forward_efq", st)
        return out
    if fp8_products:
        st = lib().fsattn_forward_fp8_products(ctypes.byref(p), ctypes.byref(m) if masked else None, ctypes.byref(q),
                                               ctypes.byref(k), ctypes.byref(v), out.data_ptr(), _stream(stream))
        _check("fsattn_forward_fp8_products", st)
        return out
    if masked:
        st = lib().fsattn_forward_masked(ctypes.byref(p), ctypes.byref(m), ctypes.byref(q), ctypes.byref(k),
                                         ctypes.byref(v), out.data_ptr(), _stream(stream))
        _check("fsattn_forward_masked", st)
        return out
    st = lib().fsattn_forward(ctypes.byref(p), ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), out.data_ptr(),
                              _stream(stream))
    _check("fsattn_forward", st)
    return out


def pattern_gate_tau(tau: float, c: float = 0.0) -> float:
    """tau' that makes the exact gate the stage-1 pattern shortcut (fsattn_pattern_gate_tau)."""
    out = ctypes.c_float()
    _check("fsattn_pattern_gate_tau", lib().fsattn_pattern_gate_tau(ctypes.c_float(tau), ctypes.c_float(c),
                                                                    ctypes.byref(out)))
    return out.value


def forward_bf16_baseline(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, softmax_scale: float,
                          out: torch.Tensor | None = None, stream=None, causal: bool = False,
                          q_lens: torch.Tensor | None = None, kv_lens: torch.Tensor | None = None) -> torch.Tensor:
    """Conventional BF16 attention forward (online softmax).  q [B,H,Sq,D], k/v [B,H,Skv,D].
    causal / q_lens / kv_lens: the masks of forward() (fsattn_forward_bf16_baseline_masked)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    if k.shape != (B, H, Skv, D) or v.shape != (B, H, Skv, D):
        raise ValueError(f"k and v must be [B, H, Skv, D] matching q {tuple(q.shape)}")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.bfloat16, t.numel(), q.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, q.numel(), q.device)
    if causal or q_lens is not None or kv_lens is not None:
        for t in (q_lens, kv_lens):
            if t is not None and (t.dtype != torch.int32 or t.device != q.device or t.shape != (B,) or
                                  not t.is_contiguous()):
                raise ValueError("q_lens / kv_lens must be contiguous int32 [B] on the inputs' device")
        m = _Mask(1 if causal else 0, q_lens.data_ptr() if q_lens is not None else None,
                  kv_lens.data_ptr() if kv_lens is not None else None)
        st = lib().fsattn_forward_bf16_baseline_masked(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Sq, Skv, D,
                                                       ctypes.c_float(softmax_scale), ctypes.byref(m),
                                                       out.data_ptr(), _stream(stream))
        _check("fsattn_forward_bf16_baseline_masked", st)
        return out
    st = lib().fsattn_forward_bf16_baseline(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, Sq, Skv, D,
                                            ctypes.c_float(softmax_scale), out.data_ptr(), _stream(stream))
    _check("fsattn_forward_bf16_baseline", st)
    return out


PROBE_BF16 = 16


def probe_mfma(fmt, iters: int, workgroups: int, stream=None) -> tuple[torch.Tensor, int]:
    """Run the pure matrix-product kernel (fsattn_probe_mfma); returns the device
    int64 stamps [workgroups, 4] (shader clock start/end, constant-rate counter
    start/end) and that counter's rate in kHz.  fmt: an MX element name / code,
    or "bf16"."""
    f = PROBE_BF16 if fmt == "bf16" else _elem(fmt)
    stamps = torch.zeros(workgroups, 4, dtype=torch.int64, device="cuda")
    khz = ctypes.c_int(0)
    _check("fsattn_probe_mfma", lib().fsattn_probe_mfma(f, int(iters), int(workgroups), stamps.data_ptr(),
                                                        ctypes.byref(khz), _stream(stream)))
    return stamps, int(khz.value)
