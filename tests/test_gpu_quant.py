"""GPU parity of the MX quantizer entry point for the formats and the rule
the forward's workloads do not exercise: E5M2 and E3M2 elements, and the
OCP-floor E8M0 rule (X = 2^(floor(log2 amax) - emax), elements above the
largest value saturate) for every format, both block axes.  Bytes must equal
the oracle's (OCP Microscaling v1.0 block encoding, the MXFP8 / MXFP6 / MXFP4
operands of "Fused-Softmax shifts an AI attention bottleneck onto faster GPU
hardware", paragraphs 7-8)."""
import numpy as np
import pytest
import torch

import softmax_matrix_cores_amd as fs
from tests.gpu_util import bits, log, same_bytes

pytestmark = pytest.mark.gpu

ELEMS = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1"]


def _inputs(n, rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, rows, cols, generator=g)
    # a spread of binades per block, zeros, and a few blocks near the top of
    # bf16's range and in its subnormals
    x = x * torch.exp2(torch.randint(-6, 7, (n, rows, 1), generator=g).float())
    x[:, ::7, :] = 0.0
    x[0, 1, :] *= 2.0 ** 100
    x[0, 2, :] *= 2.0 ** -130
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("rule", [fs.SCALE_FITMAX, fs.SCALE_OCP_FLOOR], ids=["fitmax", "ocp"])
@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("axis", [0, 1])
def test_quantizer_bytes(oracle, elem, rule, axis):
    n, rows, cols = 3, 77, 128
    x = _inputs(n, rows, cols, 100 + ELEMS.index(elem) + 10 * rule + 50 * axis)
    pre = fs.fold_prescale(128 ** -0.5) if axis == 0 else 1.0
    log(f"[quant] {elem} rule={rule} axis={axis}")
    g = fs.quantize_mx(x.cuda(), axis, elem, prescale=pre, rule=rule)
    torch.cuda.synchronize()
    o = oracle.quantize_mx(bits(x), axis, oracle.ELEM_NAMES[elem], prescale=pre, rule=rule)
    assert same_bytes(g, o, axis=axis) == (True, True)


# axis-1 shapes beyond the video case, through the C ABI: D = 64 and a
# prescale (the direct kernel's two paths), column counts 96 and 32 (the
# generic kernel), a key count below one block, and rows ld = cols + 4
# elements apart (unaligned rows: the generic kernel)
AX1_SHAPES = [(77, 64, 1.0, 0), (100, 128, 0.75, 0), (45, 96, 1.0, 0), (20, 32, 1.5, 0), (70, 128, 1.0, 4)]


@pytest.mark.parametrize("shape", AX1_SHAPES, ids=[f"r{r}c{c}p{p}ld{e}" for r, c, p, e in AX1_SHAPES])
@pytest.mark.parametrize("elem", ELEMS)
def test_quantizer_axis1_shapes(oracle, elem, shape):
    import ctypes

    rows, cols, pre, extra = shape
    n, ld = 2, cols + extra
    x = _inputs(n, rows, ld, 300 + ELEMS.index(elem) + rows)
    log(f"[quant] axis1 {elem} rows={rows} cols={cols} prescale={pre} ld={ld}")
    e = fs.ELEMS[elem]
    cb, sb = fs.mx_sizes(e, n, rows, cols, 1)
    codes = torch.zeros(cb, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(sb, dtype=torch.uint8, device="cuda")
    xd = x.cuda()
    st = fs.lib().fsattn_quantize_mx(xd.data_ptr(), n, rows, cols, ld, 1, ctypes.c_float(pre), e, fs.SCALE_FITMAX,
                                     codes.data_ptr(), scales.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, fs.lib().fsattn_status_str(st)
    torch.cuda.synchronize()
    o = oracle.quantize_mx(bits(x[..., :cols]), 1, oracle.ELEM_NAMES[elem], prescale=pre)
    g = fs.MXTensor(codes, scales, e, pre)
    assert same_bytes(g, o, axis=1) == (True, True)


@pytest.mark.parametrize("elem", ["e2m3", "e4m3"])
def test_quantizer_axis1_unaligned_scales(oracle, elem):
    """A scale buffer that is not 16-byte aligned takes the column-per-lane
    axis-1 kernel instead of the staged one: the same bytes as the oracle."""
    import ctypes

    n, rows, cols = 2, 100, 128
    x = _inputs(n, rows, cols, 350 + ELEMS.index(elem))
    e = fs.ELEMS[elem]
    cb, sb = fs.mx_sizes(e, n, rows, cols, 1)
    codes = torch.zeros(cb, dtype=torch.uint8, device="cuda")
    sbuf = torch.zeros(sb + 16, dtype=torch.uint8, device="cuda")
    st = fs.lib().fsattn_quantize_mx(x.cuda().data_ptr(), n, rows, cols, cols, 1, ctypes.c_float(1.0), e,
                                     fs.SCALE_FITMAX, codes.data_ptr(), sbuf.data_ptr() + 1,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 0, fs.lib().fsattn_status_str(st)
    torch.cuda.synchronize()
    o = oracle.quantize_mx(bits(x), 1, oracle.ELEM_NAMES[elem], prescale=1.0)
    g = fs.MXTensor(codes, sbuf[1:sb + 1].clone(), e, 1.0)
    assert same_bytes(g, o, axis=1) == (True, True)
