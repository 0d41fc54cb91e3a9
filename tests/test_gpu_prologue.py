"""GPU parity of the fused producer step (fsattn_quantize_mx_rmsnorm) against
the oracle's fso_quantize_mx_rmsnorm: codes and scales bit-exact, for FP8 /
FP6 / FP4, D = 64 and 128, with and without a per-feature weight, two eps
values, ragged row counts, zero rows and rows spanning a wide magnitude
range, and the full video Q shape (B=1, H=40, S=75600, D=128) with the
folded prescale."""
import numpy as np
import pytest
import torch

import softmax_matrix_cores_amd as fs
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

NAMES = {"e4m3": 0, "e2m3": 2, "e2m1": 4}


def _inputs(n_mat, rows, cols, seed, dev):
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.randn(n_mat, rows, cols, generator=g, device=dev)
    x = x * torch.exp(torch.empty(n_mat, rows, 1, device=dev).uniform_(-4, 4, generator=g))
    x[:, ::97] = 0.0  # some zero rows
    return x.to(torch.bfloat16)


def _compare(O, x, elem, prescale, weight, eps):
    dev = x.device
    wt = None if weight is None else torch.from_numpy(weight).to(dev)
    T = fs.quantize_mx_rmsnorm(x, elem, prescale=prescale, weight=wt, eps=eps)
    torch.cuda.synchronize()
    u = x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    oc, os_ = O.quantize_mx_rmsnorm(u, NAMES[elem], prescale=prescale, weight=weight, eps=eps)
    gc = T.codes.cpu().numpy().ravel()
    gs = T.scales.cpu().numpy().ravel()
    return np.array_equal(gc, oc.ravel()), np.array_equal(gs[: os_.size], os_.ravel()), int((gc != oc.ravel()).sum())


@pytest.mark.parametrize("elem", ["e4m3", "e2m3", "e2m1"])
@pytest.mark.parametrize("cols,use_w,eps", [(64, False, 1e-6), (128, True, 1e-6), (128, True, 1e-2)])
def test_rmsnorm_quantize_bit_exact(oracle, elem, cols, use_w, eps):
    dev = torch.device("cuda:0")
    x = _inputs(3, 517, cols, 90 + cols + len(elem), dev)
    rng = np.random.default_rng(5)
    weight = rng.uniform(0.5, 2.0, cols).astype(np.float32) if use_w else None
    pre = fs.fold_prescale(cols ** -0.5)
    log(f"[case] rmsnorm {elem} cols={cols} weight={use_w} eps={eps}")
    ok_c, ok_s, nbad = _compare(oracle, x, elem, pre, weight, eps)
    assert ok_c and ok_s, (elem, cols, nbad)


def test_rmsnorm_quantize_video_q(oracle):
    dev = torch.device("cuda:0")
    x = _inputs(40, 75600, 128, 1234, dev)
    weight = np.random.default_rng(6).uniform(0.5, 2.0, 128).astype(np.float32)
    log("[case] rmsnorm video Q 40x75600x128 e2m3")
    ok_c, ok_s, nbad = _compare(oracle, x, "e2m3", fs.fold_prescale(128 ** -0.5), weight, 1e-6)
    assert ok_c and ok_s, nbad


def test_rmsnorm_quantize_unaligned_rows(oracle):
    """Rows at an odd element offset and stride (the scalar-load path)."""
    import ctypes

    dev = torch.device("cuda:0")
    rows, cols = 301, 128
    big = _inputs(1, rows, cols + 1, 77, dev)[0]  # [rows, cols + 1], rows start at odd offsets
    x = big[:, 1:]
    weight = np.random.default_rng(8).uniform(0.5, 2.0, cols).astype(np.float32)
    wt = torch.from_numpy(weight).to(dev)
    e = 2
    cb, sb = fs.mx_sizes(e, 1, rows, cols, 0)
    codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    scales = torch.empty(sb, dtype=torch.uint8, device=dev)
    st = fs.lib().fsattn_quantize_mx_rmsnorm(big.data_ptr() + 2, 1, rows, cols, cols + 1, wt.data_ptr(),
                                             ctypes.c_float(1e-6), ctypes.c_float(2.0), e, 0, codes.data_ptr(),
                                             scales.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    u = x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(1, rows, cols)
    oc, os_ = oracle.quantize_mx_rmsnorm(u, e, prescale=2.0, weight=weight, eps=1e-6)
    assert np.array_equal(codes.cpu().numpy(), oc.ravel())
    assert np.array_equal(scales.cpu().numpy()[: os_.size], os_.ravel())
