"""GPU parity of the in-library BF16 attention baseline against the oracle's
exact softmax attention in double (R0) on the same bf16 inputs.  BF16 P and
fp32 accumulation bound the error well inside 1e-2 relative Frobenius."""
import numpy as np
import pytest
import torch

import softmax_matrix_cores_amd as fs
from softmax_matrix_cores_amd import workloads as W
from tests.gpu_util import bits, log, rel_frob

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16-ragged", "qknorm-mxfp6", dict(B=1, H=2, Sq=200, Skv=333, D=128, seed=31)),
    ("bf16-d64", "tiny-mxfp8", dict(B=2, H=1, Sq=77, Skv=150, D=64, seed=32)),
    ("bf16-stress", "stress-mxfp8", dict(B=1, H=2, Sq=128, Skv=700, D=128, seed=33)),
    ("bf16-skv1", "qknorm-mxfp6", dict(B=1, H=1, Sq=5, Skv=1, D=128, seed=34)),
]


@pytest.mark.parametrize("name,base,kw", CASES, ids=[c[0] for c in CASES])
def test_bf16_small(oracle, name, base, kw):
    w = W.custom(base, name=name, **kw)
    log(f"[case] {name}")
    q, k, v = W.make_inputs(w, device="cuda:0")
    out = fs.forward_bf16_baseline(q, k, v, w.sigma)
    torch.cuda.synchronize()
    R0 = oracle.reference_bf16(bits(q), bits(k), bits(v), w.sigma)
    err = rel_frob(out.float().cpu().numpy().reshape(-1, w.D).astype(np.float64), R0)
    log(f"[case] {name}: rel_frob={err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("name", ["stress-mxfp8", "video-mxfp6"])
def test_bf16_full_size_sampled(oracle, name):
    w = W.WORKLOADS[name]
    log(f"[case] bf16 {name}")
    q, k, v = W.make_inputs(w, device="cuda:0")
    out = fs.forward_bf16_baseline(q, k, v, w.sigma)
    torch.cuda.synchronize()
    rows = W.sample_rows(w, 64).numpy()
    R0 = oracle.reference_bf16(bits(q), bits(k), bits(v), w.sigma, rows=rows)
    g = out.float().cpu().numpy().reshape(-1, w.D)[rows]
    err = rel_frob(g.astype(np.float64), R0)
    log(f"[case] bf16 {name}: rel_frob={err:.3e}")
    assert err <= 1e-2


MASKED = [
    # name, base, sizes, causal, q_lens, kv_lens
    ("bf16-causal-square", "qknorm-mxfp6", dict(B=1, H=2, Sq=300, Skv=300, D=128, seed=41), True, None, None),
    ("bf16-causal-q<kv", "tiny-mxfp8", dict(B=1, H=2, Sq=90, Skv=410, D=64, seed=42), True, None, None),
    ("bf16-causal-q>kv", "qknorm-mxfp6", dict(B=1, H=1, Sq=290, Skv=120, D=128, seed=43), True, None, None),
    ("bf16-varlen-causal", "qknorm-mxfp6", dict(B=3, H=1, Sq=260, Skv=300, D=128, seed=44), True, [260, 100, 7],
     [300, 65, 0]),
]


@pytest.mark.parametrize("name,base,kw,causal,q_lens,kv_lens", MASKED, ids=[c[0] for c in MASKED])
def test_bf16_masked(oracle, name, base, kw, causal, q_lens, kv_lens):
    w = W.custom(base, name=name, **kw)
    log(f"[case] {name}")
    q, k, v = W.make_inputs(w, device="cuda:0")
    dev = q.device
    ql = None if q_lens is None else torch.tensor(q_lens, dtype=torch.int32, device=dev)
    kl = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=dev)
    out = fs.forward_bf16_baseline(q, k, v, w.sigma, causal=causal, q_lens=ql, kv_lens=kl)
    torch.cuda.synchronize()
    R0 = oracle.reference_bf16(bits(q), bits(k), bits(v), w.sigma, causal=causal, q_lens=q_lens, kv_lens=kv_lens)
    g = out.float().cpu().numpy().reshape(-1, w.D).astype(np.float64)
    err = rel_frob(g, R0)
    dead = ~R0.any(axis=1)
    log(f"[case] {name}: rel_frob={err:.3e} dead_rows={int(dead.sum())}")
    assert err <= 1e-2
    assert not g[dead].any()
