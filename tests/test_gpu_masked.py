"""GPU parity of the masked forward (fsattn_forward_masked) against the oracle's
fso_forward_masked: causal masks with Sq = Skv, Sq < Skv and Sq > Skv,
per-batch query and key lengths (including an empty batch), both gate tiles,
FP8 / FP6 / FP4 operands, D = 64 and 128, and planted rollbacks.  Criteria as
for the unmasked path (relative Frobenius error <= 1e-2, rollback counts equal
per row, P-code mismatch <= 1e-3); rows that see no key are exactly zero."""
import numpy as np
import pytest

from softmax_matrix_cores_amd import workloads as W
from tests.gpu_util import assert_ok, check_p, run_case

pytestmark = pytest.mark.gpu

CASES = [
    # (name, base, kw, causal, q_lens, kv_lens, dump rows)
    ("causal-square-fp6", "qknorm-mxfp6", dict(B=1, H=2, Sq=333, Skv=333, seed=61, tau=1.0), True, None, None, (0, 96)),
    ("causal-q<kv-fp8", "tiny-mxfp8", dict(B=1, H=2, Sq=100, Skv=421, D=128, seed=62), True, None, None, (0, 100)),
    ("causal-q>kv-fp4", "qknorm-mxfp4", dict(B=1, H=2, Sq=300, Skv=130, seed=63), True, None, None, (150, 300)),
    ("varlen-fp6", "qknorm-mxfp6", dict(B=3, H=2, Sq=260, Skv=300, seed=64), False, [260, 100, 7], [300, 65, 0],
     (0, 64)),
    ("varlen-causal-fp6", "qknorm-mxfp6", dict(B=3, H=2, Sq=260, Skv=300, seed=65, tau=1.0), True, [260, 100, 7],
     [300, 65, 0], (0, 64)),
    ("causal-kv128-fp6", "qknorm-mxfp6", dict(B=1, H=2, Sq=400, Skv=400, kv_tile=128, seed=66, tau=1.0), True, None, None,
     (200, 264)),
    ("causal-d64-fp4", "qknorm-mxfp4", dict(B=2, H=2, Sq=200, Skv=200, D=64, seed=67), True, None, [200, 131],
     (0, 64)),
    ("causal-stress-fp8", "stress-mxfp8", dict(B=1, H=2, Sq=256, Skv=520, seed=68, tau=2.0), True, None, None,
     (0, 128)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_masked_parity(oracle, case):
    name, base, kw, causal, q_lens, kv_lens, drows = case
    w = W.custom(base, name=name, **kw)
    res = run_case(oracle, w, dump_rows=drows, causal=causal, q_lens=q_lens, kv_lens=kv_lens)
    assert_ok(res, defer_p=True)
    if q_lens is not None or (causal and w.Sq > w.Skv) or (kv_lens is not None and 0 in kv_lens):
        assert res["dead_rows"] > 0, res
    if "stress" in name or w.tau < 8.0:
        assert res["total_counts"] > 0, res
    check_p(res)


def test_causal_video_sampled(oracle):
    """Full video size (B=1, H=40, S=75600, D=128, MXFP6) under a causal mask,
    in the launch configuration of the benchmark; oracle rows sampled across
    heads and positions, including the first rows (few visible keys)."""
    w = W.WORKLOADS["video-mxfp6"]
    rng = np.random.default_rng(77)
    heads = rng.integers(0, w.H, 6)
    pos = np.concatenate([[0, 1, 63, 64, 255, 256], rng.integers(0, w.Sq, 10), [w.Sq - 1]])
    rows = np.unique((heads[:, None] * w.Sq + pos[None, :]).ravel())
    res = run_case(oracle, w, rows=rows, causal=True, check_quant=False)
    assert_ok(res)
