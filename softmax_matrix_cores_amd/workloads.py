"""Seeded synthetic attention inputs (Q, K, V in bf16) for the five workloads.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic.  The CPU oracle and the GPU library are both fed from it,
so that they see bit-identical bf16 inputs.

Workloads (sizes from the benchmark definition; the pages themselves give no
shapes: their error study uses "synthetic inputs across ten random seeds" and
their speed figures "one long-sequence workload shape", "Fused-Softmax shifts
an AI attention bottleneck onto faster GPU hardware", paragraphs 7-8):

  tiny-mxfp8      B=1 H=2  S=256   D=64   iid N(0,1); E4M3 Q/K/V and P
  stress-mxfp8    B=1 H=16 S=4096  D=128  iid N(0,1), 1% of key rows x8; E4M3
  qknorm-mxfp6    B=2 H=24 S=16384 D=128  RMS-normed Q/K rows x per-head gain
                                          U(0.5,2), V iid; E2M3 Q/K/V and P
  qknorm-mxfp4    B=1 H=40 S=32768 D=128  same recipe; E2M1 Q/K/V, E2M3 P
  video-mxfp6/4   B=1 H=40 S=75600 D=128  21x45x80 latent grid (the token count
                                          of a 720p, 81-frame video DiT, page
                                          paragraph 9), qk-normed Q/K plus a
                                          rank-16 positional term, V iid

Recipe (fixed draw order so any consumer can regenerate it):
  torch.Generator(device).manual_seed(seed); Q, K, V drawn as fp32 randn in
  that order, then the auxiliary draws; every tensor is cast to bf16 (RNE) at
  the end.  softmax scale sigma = 1/sqrt(D); non-causal; Sq = Skv = S.
  Large workloads are drawn on the GPU (milliseconds instead of a minute);
  the oracle then receives a host copy of the very same bf16 tensors.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Skv: int
    D: int
    qk_elem: str  # e4m3 | e2m3 | e2m1 | e3m2 | e5m2
    v_elem: str
    p_elem: str
    recipe: str  # iid | stress | qknorm | video
    seed: int
    tau: float = 8.0
    kv_tile: int = 64

    @property
    def sigma(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> int:
        """Metric flops 4*B*H*Sq*Skv*D (QK^T and PV, non-causal)."""
        return 4 * self.B * self.H * self.Sq * self.Skv * self.D


WORKLOADS = {
    "tiny-mxfp8": Workload("tiny-mxfp8", 1, 2, 256, 256, 64, "e4m3", "e4m3", "e4m3", "iid", 1000),
    "stress-mxfp8": Workload("stress-mxfp8", 1, 16, 4096, 4096, 128, "e4m3", "e4m3", "e4m3", "stress", 2000),
    "qknorm-mxfp6": Workload("qknorm-mxfp6", 2, 24, 16384, 16384, 128, "e2m3", "e2m3", "e2m3", "qknorm", 3000),
    "qknorm-mxfp4": Workload("qknorm-mxfp4", 1, 40, 32768, 32768, 128, "e2m1", "e2m1", "e2m3", "qknorm", 4000),
    "video-mxfp6": Workload("video-mxfp6", 1, 40, 75600, 75600, 128, "e2m3", "e2m3", "e2m3", "video", 5000),
    "video-mxfp4": Workload("video-mxfp4", 1, 40, 75600, 75600, 128, "e2m1", "e2m1", "e2m3", "video", 5000),
}

# latent grid of the video workload: frames x height x width patches
VIDEO_GRID = (21, 45, 80)


def custom(base: str, **kw) -> Workload:
    """A workload with the recipe of `base` and other sizes (for small parity cases)."""
    return replace(WORKLOADS[base], **kw)


def _rms_gain(x: torch.Tensor, gain: torch.Tensor) -> torch.Tensor:
    # qk-norm style rows: x / sqrt(mean(x^2) + 1e-6) * g[h]
    return x / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + 1e-6) * gain.view(1, -1, 1, 1)


def _video_features(n_tokens: int, rank: int, gen: torch.Generator, device) -> torch.Tensor:
    """Seeded low-frequency random Fourier features of the latent grid, [S, rank]."""
    F, Y, X = VIDEO_GRID
    s = torch.arange(n_tokens, dtype=torch.float64, device=device)
    f = torch.div(s, Y * X, rounding_mode="floor")
    y = torch.div(s - f * Y * X, X, rounding_mode="floor")
    x = s - f * Y * X - y * X
    pos = torch.stack([f / F, y / Y, x / X], dim=1)  # [S, 3]
    omega = torch.randint(-4, 5, (rank, 3), generator=gen, device=device).to(torch.float64)
    phi = torch.rand(rank, generator=gen, dtype=torch.float64, device=device) * (2 * math.pi)
    return (math.sqrt(2.0) * torch.cos(2 * math.pi * (pos @ omega.T) + phi)).to(torch.float32)


def make_inputs(w: Workload, device="cpu") -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q [B,H,Sq,D], K [B,H,Skv,D], V [B,H,Skv,D] as contiguous bf16 tensors on `device`.

    The draws use a generator of that device seeded with w.seed, so a given
    (workload, device type) always yields the same tensors; CPU and CUDA
    draws differ from each other.  A comparison feeds both sides from one draw."""
    device = torch.device(device)
    gen = torch.Generator(device).manual_seed(w.seed)
    q = torch.randn(w.B, w.H, w.Sq, w.D, generator=gen, dtype=torch.float32, device=device)
    k = torch.randn(w.B, w.H, w.Skv, w.D, generator=gen, dtype=torch.float32, device=device)
    v = torch.randn(w.B, w.H, w.Skv, w.D, generator=gen, dtype=torch.float32, device=device)
    if w.recipe == "iid":
        pass
    elif w.recipe == "stress":
        # 1% of key rows per (b,h) scaled by 8 (exact in bf16)
        n = max(1, round(0.01 * w.Skv))
        for b in range(w.B):
            for h in range(w.H):
                rows = torch.randperm(w.Skv, generator=gen, device=device)[:n]
                k[b, h, rows] *= 8.0
    elif w.recipe in ("qknorm", "video"):
        gq = torch.rand(w.H, generator=gen, device=device) * 1.5 + 0.5
        gk = torch.rand(w.H, generator=gen, device=device) * 1.5 + 0.5
        q = _rms_gain(q, gq)
        k = _rms_gain(k, gk)
        if w.recipe == "video":
            rank = 16
            if w.Sq != w.Skv:
                raise ValueError("video recipe needs Sq == Skv")
            z = _video_features(w.Sq, rank, gen, device)  # [S, 16]
            rq = torch.randn(w.H, rank, w.D, generator=gen, device=device) * 0.25  # N(0, 1/16)
            rk = torch.randn(w.H, rank, w.D, generator=gen, device=device) * 0.25
            for h in range(w.H):
                q[:, h] += z @ rq[h]
                k[:, h] += z @ rk[h]
    else:
        raise ValueError(f"unknown recipe {w.recipe}")
    return (q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous(),
            v.to(torch.bfloat16).contiguous())


def error_study_inputs(seed: int, S: int = 1024, D: int = 128, H: int = 1) -> tuple[torch.Tensor, ...]:
    """iid N(0,1) Q, K, V [1,H,S,D] bf16 for the ten-seed error study (seeds 0..9)."""
    w = Workload("error-study", 1, H, S, S, D, "e4m3", "e4m3", "e4m3", "iid", seed)
    return make_inputs(w)


def sample_rows(w: Workload, n: int, seed: int = 12345) -> torch.Tensor:
    """Seeded sample of flattened query-row ids (b*H+h)*Sq+i, always including the
    first and the last row (the ragged tail), sorted."""
    total = w.B * w.H * w.Sq
    if n >= total:
        return torch.arange(total, dtype=torch.int64)
    gen = torch.Generator("cpu").manual_seed(seed)
    idx = torch.randperm(total, generator=gen)[: n - 2]
    idx = torch.cat([idx, torch.tensor([0, total - 1])])
    return torch.unique(idx).to(torch.int64)
