"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases span several 128-key tiles, ragged query and key tails, both
head dimensions, every supported format combination, the rollback path
(stress rows, tau = 0) and the no-rollback limit (tau huge); P codes are
compared for a window of rows through the library's P dump.  The benchmark
workloads follow at their full sizes: all rows for the two small ones, 1024
seeded rows (first and last row included) and four P-dump windows for the
large ones, and the quantizer bytes on the full tensors.
"""
import pytest
import torch

from softmax_matrix_cores_amd import workloads as W
from tests.gpu_util import assert_ok, check_p, check_p_fp8_products, run_case

pytestmark = pytest.mark.gpu

SMALL = [
    # name, base recipe, overrides
    ("fp6-ragged", "qknorm-mxfp6", dict(B=1, H=2, Sq=200, Skv=333, D=128, seed=11)),
    ("fp4-ragged", "qknorm-mxfp4", dict(B=2, H=1, Sq=130, Skv=515, D=128, seed=12)),
    ("fp8-ragged", "stress-mxfp8", dict(B=1, H=2, Sq=97, Skv=300, D=128, seed=13)),
    ("fp8-d64", "tiny-mxfp8", dict(B=1, H=2, Sq=70, Skv=190, D=64, seed=14)),
    ("fp6-d64", "qknorm-mxfp6", dict(B=1, H=2, Sq=64, Skv=256, D=64, seed=15)),
    ("fp6-stress", "stress-mxfp8", dict(B=1, H=2, Sq=128, Skv=640, D=128, seed=16, qk_elem="e2m3",
                                        v_elem="e2m3", p_elem="e2m3")),
    ("fp4-stress", "stress-mxfp8", dict(B=1, H=2, Sq=128, Skv=640, D=128, seed=17, qk_elem="e2m1",
                                        v_elem="e2m1", p_elem="e2m3")),
    ("fp6-skv1", "qknorm-mxfp6", dict(B=1, H=1, Sq=33, Skv=1, D=128, seed=18)),
    ("fp8-skv40", "tiny-mxfp8", dict(B=1, H=1, Sq=20, Skv=40, D=128, seed=19)),
    ("fp6-sq1", "qknorm-mxfp6", dict(B=1, H=3, Sq=1, Skv=700, D=128, seed=20)),
]


@pytest.mark.parametrize("name,base,kw", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("kv_tile", [64, 128])
def test_small_cases(oracle, name, base, kw, kv_tile):
    w = W.custom(base, name=name, **kw)
    res = run_case(oracle, w, dump_head=(0, w.H - 1), dump_rows=(0, min(w.Sq, 40)), kv_tile=kv_tile)
    assert_ok(res)


# every Q/K, V, P format combination the library accepts (EFQ-style E2M1 P
# has its own tests), alternating the head dimension
COMBOS = [("e4m3", "e4m3", "e4m3"), ("e2m3", "e4m3", "e4m3"), ("e2m1", "e4m3", "e4m3"),
          ("e2m3", "e2m3", "e2m3"), ("e2m1", "e2m3", "e2m3"), ("e4m3", "e2m3", "e2m3"),
          ("e2m1", "e2m1", "e2m3"), ("e2m3", "e2m1", "e2m3"), ("e4m3", "e2m1", "e2m3"),
          ("e2m3", "e2m3", "e3m2"), ("e2m1", "e2m1", "e3m2")]


@pytest.mark.parametrize("i", range(len(COMBOS)), ids=["-".join(c) for c in COMBOS])
def test_every_format_combination(oracle, i):
    qk, ve, pe = COMBOS[i]
    w = W.custom("stress-mxfp8", name=f"combo-{qk}-{ve}-{pe}", B=1, H=2, Sq=100, Skv=333, D=(64, 128)[i % 2],
                 seed=40 + i, qk_elem=qk, v_elem=ve, p_elem=pe)
    res = run_case(oracle, w, dump_head=(0, 1), dump_rows=(0, 40))
    assert_ok(res, defer_p=True)
    assert res["total_counts"] > 0, res  # the stress keys fire the gate
    check_p(res)


@pytest.mark.parametrize("tau", [0.0, 2.0, 1e4])
@pytest.mark.parametrize("elems", [("e2m3", "e2m3", "e2m3"), ("e4m3", "e4m3", "e4m3"), ("e2m1", "e2m1", "e2m3")])
def test_tau_sweep(oracle, tau, elems):
    qk, ve, pe = elems
    w = W.custom("stress-mxfp8", name=f"tau{tau}-{qk}", B=1, H=2, Sq=96, Skv=520, D=128, seed=21, qk_elem=qk,
                 v_elem=ve, p_elem=pe)
    res = run_case(oracle, w, dump_head=(0, 1), dump_rows=(0, 32), tau=tau)
    assert_ok(res, defer_p=True)
    if tau == 0.0:
        assert res["total_counts"] > 0
    if tau == 1e4:
        assert res["total_counts"] == 0
    check_p(res)


def test_tiny_mxfp8_full(oracle):
    w = W.WORKLOADS["tiny-mxfp8"]
    res = run_case(oracle, w, dump_head=(0, 1), dump_rows=(0, w.Sq))
    assert_ok(res)


def test_stress_mxfp8_full(oracle):
    w = W.WORKLOADS["stress-mxfp8"]
    res = run_case(oracle, w, dump_head=(0, 3), dump_rows=(0, w.Sq))
    assert res["total_counts"] > 0
    assert_ok(res, defer_p=True)
    check_p(res)


# E4M3 Q/K scores from the FP8 matrix core (fsattn_forward_fp8_products): every
# criterion but the P-code one, which that path does not meet; there the
# mismatch stays below the stated limit and every differing code is explained
# by the products' rounding (explain_fp8)
FP8P = [("stress", "stress-mxfp8", None), ("ragged", "stress-mxfp8", dict(B=1, H=2, Sq=97, Skv=300, D=128, seed=13)),
        ("tau0", "stress-mxfp8", dict(B=1, H=2, Sq=96, Skv=520, D=128, seed=21, tau=0.0)),
        ("d64", "tiny-mxfp8", dict(B=1, H=2, Sq=70, Skv=190, D=64, seed=14))]


@pytest.mark.parametrize("name,base,kw", FP8P, ids=[f[0] for f in FP8P])
def test_fp8_products_path(oracle, name, base, kw):
    w = W.WORKLOADS[base] if kw is None else W.custom(base, name=f"fp8p-{name}", **kw)
    res = run_case(oracle, w, dump_head=(0, w.H - 1), dump_rows=(0, w.Sq), fp8_products=True)
    assert_ok(res, defer_p=True)
    check_p_fp8_products(res)


@pytest.mark.parametrize("qk,ve", [("e2m3", "e2m3"), ("e2m1", "e2m1")])
def test_fp8_products_entry_is_the_forward_for_other_formats(qk, ve):
    """FP6/FP4 scores are exact on the matrix core: there the FP8-product entry
    point runs the default forward, bit for bit."""
    import softmax_matrix_cores_amd as fs
    w = W.custom("qknorm-mxfp6", name=f"fp8p-same-{qk}", B=1, H=2, Sq=100, Skv=333, D=128, seed=71,
                 qk_elem=qk, v_elem=ve, p_elem="e2m3")
    q, k, v = W.make_inputs(w, device="cuda:0")
    Q, K, V = fs.quantize_qkv(q, k, v, w.qk_elem, w.v_elem, w.sigma)
    outs = [fs.forward(Q, K, V, w.B, w.H, w.Sq, w.Skv, w.D, w.sigma, w.p_elem, tau=w.tau, fp8_products=f)
            for f in (False, True)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def _block_scaled(q, k, v):
    """Feature block b of Q times 2^(8b), of K times 2^(-8b): every product
    q_d k_d is unchanged, but the four block scales of a row differ by 2^8
    steps, so a block scale applied to the wrong block changes the scores.
    V's key block j (blocks run along keys) times 2^(4 (j mod 4)): its block
    scales differ from one key block to the next as well."""
    D, Skv = q.shape[-1], k.shape[-2]
    f = 2.0 ** (8 * (torch.arange(D) // 32).float())
    g = 2.0 ** (4 * ((torch.arange(Skv) // 32) % 4).float()).view(-1, 1)
    return ((q.float() * f).to(torch.bfloat16), (k.float() / f).to(torch.bfloat16),
            (v.float() * g).to(torch.bfloat16))


def _far_scales(q, k, v):
    """Q times 2^-100 and K times 2^100: products unchanged, block scales near
    2^-104 and 2^96 (inside the range the E4M3 decode is exact for)."""
    return ((q.float() * 2.0 ** -100).to(torch.bfloat16), (k.float() * 2.0 ** 100).to(torch.bfloat16), v)


@pytest.mark.parametrize("qk,ve,pe", [("e4m3", "e4m3", "e4m3"), ("e2m3", "e2m3", "e2m3")])
def test_far_block_scales(oracle, qk, ve, pe):
    w = W.custom("stress-mxfp8", name=f"farscale-{qk}", B=1, H=2, Sq=96, Skv=300, D=128, seed=82, qk_elem=qk,
                 v_elem=ve, p_elem=pe)
    res = run_case(oracle, w, dump_head=(0, 1), dump_rows=(0, 48), transform=_far_scales)
    assert_ok(res, defer_p=True)
    assert res["total_counts"] > 0, res
    check_p(res)


@pytest.mark.parametrize("qk,ve,pe,fp8p", [("e4m3", "e4m3", "e4m3", False), ("e4m3", "e4m3", "e4m3", True),
                                         ("e2m3", "e2m3", "e2m3", False), ("e2m1", "e2m1", "e2m3", False)],
                         ids=["e4m3", "e4m3-fp8-products", "e2m3", "e2m1"])
@pytest.mark.parametrize("D", [64, 128])
def test_block_scales_differ_across_features(oracle, qk, ve, pe, fp8p, D):
    w = W.custom("stress-mxfp8", name=f"bscale-{qk}", B=1, H=2, Sq=96, Skv=300, D=D, seed=81, qk_elem=qk,
                 v_elem=ve, p_elem=pe)
    res = run_case(oracle, w, dump_head=(0, 1), dump_rows=(0, 48), fp8_products=fp8p, transform=_block_scaled)
    assert_ok(res, defer_p=True)
    assert res["total_counts"] > 0, res
    if fp8p:
        check_p_fp8_products(res)
    else:
        check_p(res)


# the Schraudolph shift c != 0 (60801/8192, the RMS-optimal shift in BF16
# pattern units) moves T0, the gate threshold and every stage-1 pattern
@pytest.mark.parametrize("elems", [("e2m3", "e2m3", "e2m3"), ("e2m1", "e2m1", "e2m3"), ("e4m3", "e4m3", "e4m3")])
@pytest.mark.parametrize("kv_tile", [64, 128])
def test_schraudolph_shift(oracle, elems, kv_tile):
    qk, ve, pe = elems
    w = W.custom("stress-mxfp8", name=f"shift-{qk}", B=1, H=2, Sq=160, Skv=450, D=128, seed=61, qk_elem=qk,
                 v_elem=ve, p_elem=pe)
    res = run_case(oracle, w, dump_head=(0, 1), dump_rows=(0, 48), kv_tile=kv_tile, c=60801 / 8192)
    assert_ok(res, defer_p=True)
    assert res["total_counts"] > 0, res
    check_p(res)


@pytest.mark.parametrize("name", ["qknorm-mxfp6", "qknorm-mxfp4", "video-mxfp6", "video-mxfp4", "video-mxfp8"])
def test_large_sampled(oracle, name):
    """1024 seeded query rows (first and last included) against the oracle at
    the full size; P codes of four 16-row windows: the first rows, two heads
    in the middle and the ragged last rows of the last head."""
    w = W.WORKLOADS[name]
    rows = W.sample_rows(w, 1024).numpy()
    mid = w.Sq // 2 - 8
    more = [(0, w.H // 3, mid, mid + 16), (w.B - 1, (2 * w.H) // 3, mid + 4000 % w.Sq // 2, mid + 4000 % w.Sq // 2 + 16),
            (w.B - 1, w.H - 1, w.Sq - 16, w.Sq)]
    res = run_case(oracle, w, rows=rows, dump_head=(0, 0), dump_rows=(0, 16), more_dumps=more)
    assert res["p_rows"] == 64
    assert_ok(res, defer_p=True)
    check_p(res)
