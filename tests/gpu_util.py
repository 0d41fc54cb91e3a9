"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on the
same seeded bf16 inputs and compare by the acceptance criteria
(global relative Frobenius error <= 1e-2, P-code mismatch fraction <= 1e-3,
rollback counts equal per row, quantizer bytes identical)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import softmax_matrix_cores_amd as fs
from softmax_matrix_cores_amd import workloads as W

REL_FROB_TOL = 1e-2
P_MISMATCH_TOL = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(x: torch.Tensor) -> np.ndarray:
    return x.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def oracle_quant(O, q, k, v, w: W.Workload):
    B, H, Sq, D = q.shape
    Skv = k.shape[2]
    qk, ve = O.ELEM_NAMES[w.qk_elem], O.ELEM_NAMES[w.v_elem]
    alpha = O.softmax_scale_prescale(w.sigma)
    Qo = O.quantize_mx(bits(q).reshape(B * H, Sq, D), 0, qk, prescale=alpha)
    Ko = O.quantize_mx(bits(k).reshape(B * H, Skv, D), 0, qk)
    Vo = O.quantize_mx(bits(v).reshape(B * H, Skv, D), 1, ve)
    return Qo, Ko, Vo


def gpu_quant(q, k, v, w: W.Workload):
    dev = torch.device("cuda:0")
    return fs.quantize_qkv(q.to(dev), k.to(dev), v.to(dev), w.qk_elem, w.v_elem, w.sigma)


def interleave_v_scales(s: np.ndarray) -> np.ndarray:
    """Oracle V scales [n, cols, nb] -> the library's block-major layout
    [n, nb, 32, 4] (column c at [c % 32][c // 32]); absent columns compare as 0."""
    n, cols, nb = s.shape
    out = np.zeros((n, nb, 32, 4), np.uint8)
    for c in range(cols):
        out[:, :, c % 32, c // 32] = s[:, c, :]
    return out


def same_bytes(gpu: fs.MXTensor, ora, axis: int = 0) -> tuple[bool, bool]:
    gc = gpu.codes.cpu().numpy().ravel()
    gs = gpu.scales.cpu().numpy().ravel()
    if axis == 0:
        os_ = ora[1].ravel()
        return np.array_equal(gc, ora[0].ravel()), np.array_equal(gs[: os_.size], os_)
    os_ = interleave_v_scales(ora[1])
    n, cols = ora[1].shape[0], ora[1].shape[1]
    gs4 = gs.reshape(os_.shape).copy()
    if cols < 128:
        gs4[:, :, :, (cols + 31) // 32:] = 0
    return np.array_equal(gc, ora[0].ravel()), np.array_equal(gs4, os_)


def oracle_params(O, w: W.Workload, tau=None, kv_tile=None, efq=None, gate="exact", c=0.0):
    """efq = (tau, h): E2M1 P by the EFQ-style rule (p_mode P_EFQ); gate "pattern":
    the stage-1 pattern gate shortcut (gate_mode GATE_PATTERN)."""
    kw = {} if efq is None else dict(p_mode=O.P_EFQ, efq_tau=efq[0], efq_h=efq[1])
    if gate == "pattern":
        kw["gate_mode"] = O.GATE_PATTERN
    return O.make_params(w.B, w.H, w.Sq, w.Skv, w.D, O.ELEM_NAMES[w.qk_elem], O.ELEM_NAMES[w.v_elem],
                         O.ELEM_NAMES[w.p_elem], tau=w.tau if tau is None else tau,
                         kv_tile=w.kv_tile if kv_tile is None else kv_tile, c=c, **kw)


def rel_frob(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def p_mismatch(gc, gs, oc, os_) -> float:
    """Fraction of P elements whose code or block scale differs."""
    gs_e = np.repeat(gs, 32, axis=1)[:, : gc.shape[1]]
    os_e = np.repeat(os_, 32, axis=1)[:, : oc.shape[1]]
    bad = (gc != oc) | (gs_e != os_e)
    return float(bad.mean())


def run_case(O, w: W.Workload, rows=None, dump_head=(0, 0), dump_rows=None, tau=None, kv_tile=None,
             check_quant=True, causal=False, q_lens=None, kv_lens=None, efq=None, gate="exact", c=0.0,
             more_dumps=(), fp8_products=False, transform=None):
    """Full comparison on workload w.  rows: oracle row sample (None = all rows).
    causal / q_lens / kv_lens: masks ([B] lists), sent to both sides.
    efq = (tau, h) for E2M1 P (default: the library's calibrated pair).
    c: the Schraudolph shift (both sides).
    more_dumps: further P-dump windows (b, h, row0, row1), each from a launch
    of its own on the same operands; their P codes join the comparison.
    fp8_products: E4M3 Q/K scores from the FP8 matrix core
    (fsattn_forward_fp8_products); the P-code comparison then also records
    how many differing codes explain_fp8 explains.
    transform: optional (q, k, v) -> (q, k, v) applied to the bf16 inputs of
    both sides.
    Returns a dict of metrics; asserts nothing."""
    masked = causal or q_lens is not None or kv_lens is not None
    if w.p_elem == "e2m1" and efq is None:
        efq = (fs.EFQ_TAU, fs.EFQ_H)
    log(f"[case] {w.name} B={w.B} H={w.H} Sq={w.Sq} Skv={w.Skv} D={w.D} {w.qk_elem}/{w.v_elem}/{w.p_elem} "
        f"tau={w.tau if tau is None else tau} kv_tile={w.kv_tile if kv_tile is None else kv_tile}"
        + (f" causal={causal} q_lens={q_lens} kv_lens={kv_lens}" if masked else "")
        + (f" efq={efq}" if efq is not None else "") + (f" gate={gate}" if gate != "exact" else "")
        + (f" c={c}" if c else ""))
    q, k, v = (x.cpu() for x in W.make_inputs(w, device="cuda:0"))
    if transform is not None:
        q, k, v = transform(q, k, v)
    tau_ = w.tau if tau is None else tau
    kvt = w.kv_tile if kv_tile is None else kv_tile
    res = {"qk_elem": w.qk_elem}
    # GPU path
    Qg, Kg, Vg = gpu_quant(q, k, v, w)
    counts = torch.zeros(w.B, w.H, w.Sq, dtype=torch.int32, device="cuda:0")
    s32 = (w.Skv + 31) // 32 * 32
    pd = None
    if dump_rows is not None:
        r0, r1 = dump_rows
        pc = torch.zeros(r1 - r0, s32, dtype=torch.uint8, device="cuda:0")
        ps = torch.zeros(r1 - r0, s32 // 32, dtype=torch.uint8, device="cuda:0")
        pd = (dump_head[0], dump_head[1], r0, r1, pc, ps)
    mk = {}
    if masked:
        dev = torch.device("cuda:0")
        mk = dict(causal=causal,
                  q_lens=None if q_lens is None else torch.tensor(q_lens, dtype=torch.int32, device=dev),
                  kv_lens=None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=dev))
    if efq is not None:
        mk.update(efq_tau=efq[0], efq_h=efq[1])
    if gate != "exact":
        mk["gate"] = gate
    if fp8_products:
        mk["fp8_products"] = True
    res["fp8_products"] = fp8_products
    out = fs.forward(Qg, Kg, Vg, w.B, w.H, w.Sq, w.Skv, w.D, w.sigma, w.p_elem, tau=tau_, kv_tile=kvt,
                     counts=counts, p_dump=pd, c=c, **mk)
    torch.cuda.synchronize()
    windows = []  # (b, h, r0, r1, gpu codes, gpu scales)
    if pd is not None:
        windows.append((pd[0], pd[1], pd[2], pd[3], pd[4].cpu().numpy(), pd[5].cpu().numpy()))
    for (b, h, r0, r1) in more_dumps:
        pc = torch.zeros(r1 - r0, s32, dtype=torch.uint8, device="cuda:0")
        ps = torch.zeros(r1 - r0, s32 // 32, dtype=torch.uint8, device="cuda:0")
        fs.forward(Qg, Kg, Vg, w.B, w.H, w.Sq, w.Skv, w.D, w.sigma, w.p_elem, tau=tau_, kv_tile=kvt,
                   p_dump=(b, h, r0, r1, pc, ps), c=c, **mk)
        torch.cuda.synchronize()
        windows.append((b, h, r0, r1, pc.cpu().numpy(), ps.cpu().numpy()))
    log(f"[case] {w.name}: GPU done")
    # oracle
    Qo, Ko, Vo = oracle_quant(O, q, k, v, w)
    if check_quant:
        res["quant_q"] = same_bytes(Qg, Qo)
        res["quant_k"] = same_bytes(Kg, Ko)
        res["quant_v"] = same_bytes(Vg, Vo, axis=1)
    p = oracle_params(O, w, tau=tau_, kv_tile=kvt, efq=efq, gate=gate, c=c)
    row_ids = None if rows is None else np.asarray(rows, dtype=np.int64)
    omk = dict(causal=causal, q_lens=q_lens, kv_lens=kv_lens) if masked else {}
    r = O.forward(p, Qo, Ko, Vo, rows=row_ids, **omk)
    gout = out.float().cpu().numpy().reshape(-1, w.D)
    gcnt = counts.cpu().numpy().ravel()
    if row_ids is not None:
        gout = gout[row_ids]
        gcnt = gcnt[row_ids]
    res["rel_frob"] = rel_frob(gout.astype(np.float64), r["O"])
    res["count_mismatch_rows"] = int((gcnt != r["counts"]).sum())
    res["total_counts"] = int(r["counts"].sum())
    res["oracle_misses"] = int(r["misses"].sum())
    res["finite"] = bool(np.isfinite(gout).all())
    if masked:
        # rows the oracle leaves empty (no visible key, or past q_len) must be exactly 0
        dead = r["l"] == 0
        res["dead_rows"] = int(dead.sum())
        res["dead_rows_nonzero"] = int((gout[dead] != 0).any(axis=1).sum()) + int((gcnt[dead] != 0).sum())
    if windows:
        drows = np.concatenate([(b * w.H + h) * w.Sq + np.arange(r0, r1) for b, h, r0, r1, _, _ in windows])
        gc = np.concatenate([x[4] for x in windows])
        gs = np.concatenate([x[5] for x in windows])
        rd = O.forward(p, Qo, Ko, Vo, rows=drows, want_p=True, **omk)
        res["p_rows"] = int(len(drows))
        res["p_mismatch"] = p_mismatch(gc, gs, rd["p_codes"], rd["p_scales"])
        if fp8_products and w.qk_elem == "e4m3" and efq is None:
            t, _ = O.forward_scores(p, Qo, Ko, Vo, drows, **omk)
            steps = []
            res["p_bad"], res["p_unexplained"] = explain_fp8(O, O.ELEM_NAMES[w.p_elem], gc, gs, rd["p_codes"],
                                                             rd["p_scales"], t, w.D, steps)
            if steps:
                res["p_flip_steps_max"] = max(steps)
    log(f"[case] {w.name}: {res}")
    return res


def assert_ok(res: dict, defer_p: bool = False):
    """Every criterion; the P-code check last (or left to `check_p` when a
    test has further assertions of its own)."""
    for key in ("quant_q", "quant_k", "quant_v"):
        if key in res:
            assert res[key] == (True, True), (key, res)
    assert res["finite"], res
    assert res["rel_frob"] <= REL_FROB_TOL, res
    assert res["count_mismatch_rows"] == 0, res
    assert res.get("dead_rows_nonzero", 0) == 0, res
    if not defer_p:
        check_p(res)


# FP8 (E4M3) score products on the FP8 matrix core (the path of
# fsattn_forward_fp8_products; the default forward decodes E4M3 Q/K to BF16
# and meets the criteria like every other format): the matrix core does not
# return the correctly rounded sum on gfx950.  With the accumulator starting
# at the folded offset (about 2^14), the score error measured through the P
# codes of the 4096-key FP8 workload (15 400-15 800 code flips per head) is
# symmetric and reaches 124-136 binary32 steps of t at D = 128, about one
# step per product: fp8_bound allows 2 D steps.  A P code that differs from
# the oracle's is explained when the oracle's folded score t lies within
# that bound of an integer n and the two codes are those of the BF16
# patterns n - 1 and n (a floor on the other side of n); a block scale, when
# one score of its block lies so close to the pattern at which the E8M0
# steps between the two values.  That path's tests require a mismatch below
# FP8_PRODUCTS_LIMIT with every differing element so explained; the 1e-3
# criterion is not met by it.
FP8_PRODUCTS_LIMIT = 1.5e-3


def fp8_bound(t, D: int):
    """2 D binary32 steps of each folded score."""
    return 2 * D * np.spacing(np.abs(np.asarray(t, np.float32))).astype(np.float64)


def _bf16_val(b: int) -> float:
    return 0.0 if b < 128 else float(np.array([b << 16], np.uint32).view(np.float32)[0])


def _scale_step(O, pe: int, hi: int) -> int:
    """Smallest BF16 pattern b whose fit-max E8M0 (as a P block max) is >= hi."""
    lo, up = 128, 0x7F7F
    while lo < up:
        mid = (lo + up) // 2
        if O.scale_code(pe, O.SCALE_FITMAX, _bf16_val(mid)) >= hi:
            up = mid
        else:
            lo = mid + 1
    return lo


def explain_fp8(O, pe: int, gc, gs, oc, os_, t, D: int, steps=None) -> tuple[int, int]:
    """(mismatching elements, unexplained elements) of a P dump against the oracle.
    steps: optional list receiving |t - n| / ulp32(t) of every code flip whose
    two codes are those of the patterns n - 1 and n (the data behind the bound)."""
    S32 = gc.shape[1]
    gse = np.repeat(gs, 32, axis=1)[:, :S32]
    ose = np.repeat(os_, 32, axis=1)[:, :S32]
    bad = (gc != oc) | (gse != ose)
    bound = fp8_bound(t, D)
    unexplained = 0
    for r, g in np.argwhere(gs != os_):
        keys = slice(32 * g, 32 * g + 32)
        ok = abs(int(gs[r, g]) - int(os_[r, g])) == 1
        if ok:
            bT = _scale_step(O, pe, max(int(gs[r, g]), int(os_[r, g])))
            ok = bool((np.abs(t[r, keys].astype(np.float64) - bT) <= bound[r, keys]).any())
        if not ok:
            unexplained += int(bad[r, keys].sum())
    for r, k in np.argwhere((gc != oc) & (gse == ose)):
        n = int(np.rint(t[r, k]))
        X = 2.0 ** (int(ose[r, k]) - 127)
        codes = {O.encode(pe, _bf16_val(b) / X) for b in (n - 1, n)}
        adjacent = codes == {int(gc[r, k]), int(oc[r, k])}
        e = abs(float(t[r, k]) - n)
        if adjacent and steps is not None:
            steps.append(e / float(np.spacing(np.float32(abs(t[r, k])))))
        if not (adjacent and e <= bound[r, k]):
            unexplained += 1
    return int(bad.sum()), unexplained


def check_p(res: dict):
    """P-code mismatch <= 1e-3 (every path of the default forward)."""
    assert res.get("p_mismatch", 0.0) <= P_MISMATCH_TOL, res


def check_p_fp8_products(res: dict):
    """The FP8-product path: mismatch below FP8_PRODUCTS_LIMIT, every differing
    code explained by the products' rounding (explain_fp8)."""
    assert res["fp8_products"] and res["qk_elem"] == "e4m3", res
    assert res["p_mismatch"] <= FP8_PRODUCTS_LIMIT, res
    assert res["p_unexplained"] == 0, res
