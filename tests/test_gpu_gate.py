"""GPU parity of the rollback-gate shortcut (fsattn_pattern_gate_tau: the
exact gate at the shifted threshold) against the oracle's reading R25, which
decides on the stage-1 BF16 patterns ("Fused-Softmax shifts an AI attention
bottleneck onto faster GPU hardware", paragraph 12: the fastest 4-bit
kernel's shortcut can miss a recovery trigger).  In the two FP6 cases the
shortcut does miss triggers the exact rule would take (oracle misses > 0);
rollback counts must equal the oracle's shortcut counts row by row, and the
other criteria are those of the exact path."""
import pytest

from softmax_matrix_cores_amd import workloads as W
from tests.gpu_util import assert_ok, run_case

pytestmark = pytest.mark.gpu

CASES = [
    # (name, base, kw, run_case kwargs)
    ("gate-fp6-tau0", "qknorm-mxfp6", dict(B=1, H=2, Sq=256, Skv=1024, seed=90, tau=0.0), dict(dump_rows=(0, 64))),
    ("gate-fp6-tau1", "qknorm-mxfp6", dict(B=1, H=2, Sq=256, Skv=1024, seed=94, tau=1.0), dict(dump_rows=(0, 64))),
    ("gate-fp4-tau0-kv128", "qknorm-mxfp4", dict(B=1, H=2, Sq=256, Skv=1024, seed=92, tau=0.0, kv_tile=128),
     dict(dump_rows=(0, 64))),
    ("gate-fp4-tau1-efq", "qknorm-mxfp4", dict(B=1, H=2, Sq=256, Skv=1024, seed=93, tau=1.0, p_elem="e2m1"),
     dict(dump_rows=(0, 64))),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pattern_gate_parity(oracle, case):
    name, base, kw, rk = case
    w = W.custom(base, name=name, **kw)
    res = run_case(oracle, w, gate="pattern", **rk)
    assert_ok(res)
    assert res["total_counts"] > 0, res
    if name in ("gate-fp6-tau0", "gate-fp6-tau1"):
        # on these inputs the shortcut does skip triggers the exact rule takes
        assert res["oracle_misses"] > 0, res
