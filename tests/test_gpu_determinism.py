"""Determinism of the fused forward: every output row has one owner (one
wave computes it, no atomics, a fixed key order), so its bytes cannot depend
on the grid, on which workgroups share the chip, or on timing.  Checked by
(a) two launches of the same call, (b) the same heads computed by separate
calls over subsets of the heads (other grids, other co-resident workgroups),
and (c) a launch that runs while another kernel occupies the chip from a
second stream."""
import pytest
import torch

import softmax_matrix_cores_amd as fs
from softmax_matrix_cores_amd import workloads as W
from tests.gpu_util import log

pytestmark = pytest.mark.gpu


def _run(Q, K, V, w, H, stream=None):
    out = torch.empty(w.B, H, w.Sq, w.D, dtype=torch.bfloat16, device="cuda:0")
    cnt = torch.zeros(w.B, H, w.Sq, dtype=torch.int32, device="cuda:0")
    fs.forward(Q, K, V, w.B, H, w.Sq, w.Skv, w.D, w.sigma, w.p_elem, tau=w.tau, kv_tile=w.kv_tile, counts=cnt,
               out=out, stream=stream)
    return out, cnt


def _head_slice(X: fs.MXTensor, h0, h1, H):
    per = X.codes.numel() // H
    pers = X.scales.numel() // H
    return fs.MXTensor(X.codes[h0 * per:h1 * per], X.scales[h0 * pers:h1 * pers], X.elem, X.prescale)


@pytest.mark.parametrize("elems", [("e2m3", "e2m3", "e2m3"), ("e4m3", "e4m3", "e4m3"), ("e2m1", "e2m1", "e2m3")])
def test_bitwise_deterministic(elems):
    qk, ve, pe = elems
    w = W.custom("stress-mxfp8", name=f"det-{qk}", B=1, H=8, Sq=1000, Skv=1500, D=128, seed=71, qk_elem=qk,
                 v_elem=ve, p_elem=pe)
    log(f"[det] {w.name}")
    q, k, v = W.make_inputs(w, device="cuda:0")
    Q, K, V = fs.quantize_qkv(q, k, v, qk, ve, w.sigma)
    o1, c1 = _run(Q, K, V, w, w.H)
    o2, c2 = _run(Q, K, V, w, w.H)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(c1, c2)
    assert int(c1.sum()) > 0  # the stress keys fire the gate
    # (b) heads [0, 3) and [3, 8) as calls of their own; the scale buffers of
    # Q and K are padded to whole dwords, so the heads are split where a
    # head's scales start on a dword (D = 128: 4 bytes per row)
    parts = []
    for h0, h1 in ((0, 3), (3, 8)):
        Qs, Ks, Vs = (_head_slice(X, h0, h1, w.H) for X in (Q, K, V))
        parts.append(_run(Qs, Ks, Vs, w, h1 - h0))
    torch.cuda.synchronize()
    o3 = torch.cat([p[0] for p in parts], dim=1)
    c3 = torch.cat([p[1] for p in parts], dim=1)
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(c1, c3)
    # (c) concurrent with a large matrix product on another stream
    side = torch.cuda.Stream()
    a = torch.randn(4096, 4096, device="cuda:0")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(4):
            a = a @ a.T * 1e-3
    o4, c4 = _run(Q, K, V, w, w.H, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o4.view(torch.int16)) and torch.equal(c1, c4)
