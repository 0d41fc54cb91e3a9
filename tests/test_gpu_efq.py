"""GPU parity of the EFQ-style E2M1 P path (fsattn_forward_efq) against the
oracle's reading R24 ("EFQ-Softmax: Exp-Free Quantization for Softmax",
sections II.B-C, III.A-B): P codes straight from the folded scores with an
exponent-only block scale, the same P for P V and P 1.

Cases: FP6 and FP4 Q/K/V, D = 64 and 128, ragged key counts, both gate
tiles, planted rollbacks (gate tau 0 and 1), the calibrated and other
(tau, h) pairs, masks, and the full video shape on sampled rows.  Criteria
as for the two-stage path: relative Frobenius error <= 1e-2, rollback counts
equal per row, P-code mismatch <= 1e-3.  The FP6/FP4 scores are exact on
the matrix core; the oracle compares each score with the thresholds
tau + j h exactly, while the kernel takes one binary32 fused multiply-add per
score whose slope 1 / (128 h) is rounded, so codes may differ for scores
within about 2^-16 of a threshold (a few in 10^5 on these cases)."""
import numpy as np
import pytest

from softmax_matrix_cores_amd import workloads as W
from tests.gpu_util import assert_ok, run_case

pytestmark = pytest.mark.gpu

CASES = [
    # (name, base, kw, run_case kwargs)
    ("efq-fp6-ragged", "qknorm-mxfp6", dict(B=1, H=2, Sq=300, Skv=333, seed=81), dict(dump_rows=(0, 300))),
    ("efq-fp4-d64", "qknorm-mxfp4", dict(B=2, H=2, Sq=257, Skv=190, D=64, seed=82), dict(dump_rows=(0, 257))),
    ("efq-fp6-fires", "qknorm-mxfp6", dict(B=1, H=2, Sq=256, Skv=700, seed=83, tau=0.0), dict(dump_rows=(0, 128))),
    ("efq-fp4-fires", "qknorm-mxfp4", dict(B=1, H=2, Sq=200, Skv=640, seed=84, tau=1.0), dict(dump_rows=(64, 200))),
    ("efq-fp6-kv128", "qknorm-mxfp6", dict(B=1, H=2, Sq=260, Skv=520, seed=85, kv_tile=128, tau=1.0),
     dict(dump_rows=(0, 64))),
    ("efq-fp4-other-params", "qknorm-mxfp4", dict(B=1, H=2, Sq=128, Skv=300, seed=86),
     dict(dump_rows=(0, 128), efq=(-3.7, 0.55))),
    ("efq-fp6-coarse-params", "qknorm-mxfp6", dict(B=1, H=1, Sq=96, Skv=256, seed=87),
     dict(dump_rows=(0, 96), efq=(-8.0, 1.5))),
    ("efq-fp4-causal-varlen", "qknorm-mxfp4", dict(B=3, H=2, Sq=200, Skv=260, seed=88, tau=1.0),
     dict(dump_rows=(0, 64), causal=True, q_lens=[200, 90, 5], kv_lens=[260, 70, 0])),
    ("efq-fp6-iid", "tiny-mxfp8", dict(B=1, H=2, Sq=256, Skv=256, D=128, seed=89, qk_elem="e2m3", v_elem="e2m3"),
     dict(dump_rows=(0, 256))),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_efq_parity(oracle, case):
    name, base, kw, rk = case
    w = W.custom(base, name=name, p_elem="e2m1", **kw)
    res = run_case(oracle, w, **rk)
    assert_ok(res)
    if w.tau < 8.0:
        assert res["total_counts"] > 0, res
    if rk.get("q_lens") is not None:
        assert res["dead_rows"] > 0, res


def test_efq_video_sampled(oracle):
    """Full video size (B=1, H=40, S=75600, D=128) with E2M1 Q/K/V and E2M1 P,
    in the benchmark's launch configuration; 512 oracle rows sampled across
    heads, and P dumps of the first rows, middle rows of a middle head and the
    last rows of the last head."""
    w = W.custom("video-mxfp4", name="video-efq", p_elem="e2m1")
    rows = W.sample_rows(w, 512).numpy()
    res = run_case(oracle, w, rows=rows, dump_head=(0, w.H - 1), dump_rows=(w.Sq - 16, w.Sq), check_quant=False,
                   more_dumps=[(0, 0, 0, 16), (0, w.H // 2, w.Sq // 2, w.Sq // 2 + 16)])
    assert_ok(res)
