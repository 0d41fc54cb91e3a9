"""GPU parity at the largest key count the library accepts (Skv * D <= 2^30:
Skv = 2^23 - 37 keys at D = 128, a ragged last step), one head, MXFP6, with
every query row checked against the oracle and the quantizer bytes compared
in full.  Collected last: its oracle side needs ~17 GB of host memory and
tens of seconds."""
import pytest

from softmax_matrix_cores_amd import workloads as W
from tests.gpu_util import assert_ok, run_case

pytestmark = pytest.mark.gpu


def test_max_keys(oracle):
    w = W.custom("qknorm-mxfp6", name="max-keys", B=1, H=1, Sq=8, Skv=(1 << 23) - 37, D=128, seed=99)
    res = run_case(oracle, w, dump_rows=(0, 8))
    assert_ok(res)
