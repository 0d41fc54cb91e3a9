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
