"""Misses of the gate shortcut (reading R25) against the exact gate, on
stress inputs with an extreme-score sweep.

"Fused-Softmax shifts an AI attention bottleneck onto faster GPU hardware",
paragraph 12: the fastest four-bit kernel's shortcut can miss a recovery
trigger in an extreme-score range; no such failure was seen in evaluated
calls.  Here: MXFP4 operands (E2M1 Q/K/V, E2M3 P), iid N(0,1) Q/K/V with 1 %
of the key rows scaled by s, s in {1, 8, 64, 512}, gate tau in
{0, 1, 8, 32, 127, 128, 200}.  For each point: exact-gate fires, shortcut
fires, shortcut misses (tiles the exact rule would fire in the shortcut's
state), misses per 10^9 rows, and the relative Frobenius errors of both
outputs against exact softmax on the same quantized operands (R1).

Calls only the oracle and torch's seeded generator.  Writes
tests/golden/gate_shortcut_study.json:
    python tests/golden/make_gate_study.py
"""
import json
import math
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gate_shortcut_study.json")
B, H, Sq, Skv, D = 1, 4, 1024, 2048, 128
SCALES = [1.0, 8.0, 64.0, 512.0]
TAUS = [0.0, 1.0, 8.0, 32.0, 127.0, 128.0, 200.0]


def bits(x):
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def inputs(s: float, seed: int = 2025):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Sq, D, generator=g)
    k = torch.randn(B, H, Skv, D, generator=g)
    v = torch.randn(B, H, Skv, D, generator=g)
    hot = torch.rand(B, H, Skv, generator=g) < 0.01
    k = torch.where(hot[..., None], k * s, k)
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


def main():
    oracle.build(force=False)
    E2M1, E2M3 = oracle.E2M1, oracle.E2M3
    sigma = 1 / math.sqrt(D)
    a = oracle.softmax_scale_prescale(sigma)
    points = []
    for s in SCALES:
        q, k, v = inputs(s)
        n = B * H
        Q = oracle.quantize_mx(bits(q).reshape(n, Sq, D), 0, E2M1, prescale=a)
        K = oracle.quantize_mx(bits(k).reshape(n, Skv, D), 0, E2M1)
        V = oracle.quantize_mx(bits(v).reshape(n, Skv, D), 1, E2M1)
        R1 = oracle.reference(oracle.make_params(B, H, Sq, Skv, D, E2M1, E2M1, E2M3), oracle.REF_R1, Q, K, V)
        nr = np.linalg.norm(R1)
        for tau in TAUS:
            pe = oracle.make_params(B, H, Sq, Skv, D, E2M1, E2M1, E2M3, tau=tau)
            ps = oracle.make_params(B, H, Sq, Skv, D, E2M1, E2M1, E2M3, tau=tau, gate_mode=oracle.GATE_PATTERN)
            re = oracle.forward(pe, Q, K, V)
            rs = oracle.forward(ps, Q, K, V)
            rows = B * H * Sq
            miss = int(rs["misses"].sum())
            pt = {"key_scale": s, "tau": tau, "rows": rows,
                  "exact_fires": int(re["counts"].sum()), "shortcut_fires": int(rs["counts"].sum()),
                  "shortcut_misses": miss, "rows_with_a_miss": int((rs["misses"] > 0).sum()),
                  "misses_per_1e9_rows": miss / rows * 1e9,
                  "err_exact_vs_R1": float(np.linalg.norm(re["O"] - R1) / nr),
                  "err_shortcut_vs_R1": float(np.linalg.norm(rs["O"] - R1) / nr),
                  "shortcut_finite": bool(np.isfinite(rs["O"]).all())}
            points.append(pt)
            print(json.dumps(pt), flush=True)
    # the default gate (tau 8) on 16x more rows, for a rate per 10^9 rows
    HB = 64
    for s in (8.0, 64.0):
        g = torch.Generator().manual_seed(4040)
        q = torch.randn(1, HB, Sq, D, generator=g)
        k = torch.randn(1, HB, Skv, D, generator=g)
        v = torch.randn(1, HB, Skv, D, generator=g)
        hot = torch.rand(1, HB, Skv, generator=g) < 0.01
        k = torch.where(hot[..., None], k * s, k)
        q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
        Q = oracle.quantize_mx(bits(q).reshape(HB, Sq, D), 0, E2M1, prescale=a)
        K = oracle.quantize_mx(bits(k).reshape(HB, Skv, D), 0, E2M1)
        V = oracle.quantize_mx(bits(v).reshape(HB, Skv, D), 1, E2M1)
        ps = oracle.make_params(1, HB, Sq, Skv, D, E2M1, E2M1, E2M3, tau=8.0, gate_mode=oracle.GATE_PATTERN)
        rs = oracle.forward(ps, Q, K, V)
        rows = HB * Sq
        miss = int(rs["misses"].sum())
        pt = {"key_scale": s, "tau": 8.0, "rows": rows, "heads": HB, "seed": 4040,
              "shortcut_fires": int(rs["counts"].sum()), "shortcut_misses": miss,
              "misses_per_1e9_rows": miss / rows * 1e9,
              "upper_95_per_1e9_rows_if_none": (3.0 / rows * 1e9) if miss == 0 else None}
        points.append(pt)
        print(json.dumps(pt), flush=True)
    res = {"source": "Fused-Softmax shifts an AI attention bottleneck onto faster GPU hardware, paragraph 12 "
                     "(a gate shortcut that can miss a recovery trigger at extreme scores); reading R25",
           "script": "tests/golden/make_gate_study.py (oracle only)",
           "shape": {"B": B, "H": H, "Sq": Sq, "Skv": Skv, "D": D, "formats": "E2M1 Q/K/V, E2M3 P",
                     "kv_tile": 64},
           "inputs": "iid N(0,1) bf16 Q/K/V, 1 % of key rows scaled by key_scale, torch seed 2025",
           "points": points}
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
