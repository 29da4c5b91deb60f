"""Synthetic video-token Q/K/V with controlled attention concentration.

The pages measure SparsePR on four video generation / world models whose
weights, prompts and evaluation suites are not available here.  These inputs
stand in for them: tokens on a frames x height x width latent grid in
frame-major raster order, built from smooth spatio-temporal Fourier features
plus a few planted "object" offsets plus small noise, projected per head.
The per-head logit temperature is set by bisection so that a query needs a
chosen fraction of all keys to hold 90% of its softmax mass (the pages quote
6.2% for one model in the part of the news explainer that contrasts per-query
with pooled support).

Recipe (all draws from numpy PCG64 streams spawned from one seed):
  * p_n = (t/T, y/H, x/W) for token n.
  * F = d/2 frequency vectors w_f ~ N(0, (2*pi*1.5)^2 I_3), phases b_f ~ U[0, 2*pi);
    phi_n = [sin(w.p_n + b), cos(w.p_n + b)] in R^d.
  * 8 anchors a_c ~ U[0,1)^3 and offsets e_c ~ N(0, I_d); token label = nearest
    anchor with the time difference weighted by 0.5.
  * x_n = phi_n + e_{c_n} + eps_n, eps ~ N(0, 0.1^2 I_d).
  * per head W_q, W_k, W_v ~ N(0, 1/d);  Q = tau_h X W_q, K = X W_k, V = X W_v.
  * tau_h: bisection on log(tau) until the mean over 256 evenly spaced queries of
    the 90%-mass key fraction (softmax at scale 1/sqrt(d)) is within 0.05 pp of
    the head's target.
  * cast once to the call dtype (bf16 round-to-nearest-even, or fp32).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention call shape plus the method settings it is run with."""

    name: str
    frames: int
    height: int
    width: int
    heads: int
    d: int
    dtype: str  # "bf16" | "fp32"
    n_kv_groups: int
    n_q_groups: int
    block: int
    density: float
    probe_rows: int
    residual_rank: int
    ridge_lambda: float = 1e-3
    f90_lo: float = 0.06  # 90%-mass key fraction target of head 0
    f90_hi: float = 0.06  # ... of the last head (linear in between)
    seed: int = 20260

    @property
    def n(self) -> int:
        return self.frames * self.height * self.width

    def f90_targets(self) -> np.ndarray:
        if self.heads == 1:
            return np.array([self.f90_lo])
        h = np.arange(self.heads)
        return self.f90_lo + (self.f90_hi - self.f90_lo) * h / (self.heads - 1)


WORKLOADS: Dict[str, Workload] = {
    # tiny single call, fp32
    "c1_tiny_fp32": Workload("c1_tiny_fp32", 4, 16, 16, 1, 64, "fp32",
                             16, 16, 64, 0.25, 64, 16, seed=20260),
    # video-DiT-like call
    "c2_dit_8k": Workload("c2_dit_8k", 8, 32, 32, 12, 64, "bf16",
                          64, 64, 128, 0.25, 64, 32, seed=20261),
    # mid-size video-DiT call, per-head concentration spread 3%..12%
    "c3_dit_32k": Workload("c3_dit_32k", 21, 30, 52, 40, 128, "bf16",
                           256, 256, 128, 0.25, 64, 32,
                           f90_lo=0.03, f90_hi=0.12, seed=20262),
    # long-sequence call, one GPU's full problem
    "c4_long_75k": Workload("c4_long_75k", 21, 45, 80, 40, 128, "bf16",
                            256, 256, 128, 0.22, 64, 32, seed=20263),
    # sweep base (head dim / density / probes / partition varied around it)
    "c5_sweep_32k": Workload("c5_sweep_32k", 21, 30, 52, 40, 128, "bf16",
                             256, 256, 128, 0.25, 64, 32,
                             f90_lo=0.03, f90_hi=0.12, seed=20264),
}


def workload(name: str, **overrides) -> Workload:
    return dataclasses.replace(WORKLOADS[name], **overrides)


def f90_fraction(logits_sorted_desc: torch.Tensor, tau: float, mass: float = 0.9) -> torch.Tensor:
    """Per-row fraction of keys needed to hold `mass` of softmax(tau * logits).

    `logits_sorted_desc` holds each row's logits (already scaled by 1/sqrt(d))
    sorted in descending order, so the smallest prefix is the answer.
    """
    z = (logits_sorted_desc - logits_sorted_desc[:, :1]) * tau
    p = torch.exp(z)
    c = torch.cumsum(p, dim=1)
    total = c[:, -1:]
    need = (c < mass * total).sum(dim=1) + 1
    return need.to(torch.float64) / logits_sorted_desc.shape[1]


def _calibrate_tau(sorted_logits: torch.Tensor, target: float) -> float:
    lo, hi = math.log(1e-3), math.log(1e3)
    tau = 1.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        tau = math.exp(mid)
        f = float(f90_fraction(sorted_logits, tau).mean())
        if abs(f - target) < 5e-4:
            break
        if f > target:  # too diffuse -> sharpen
            lo = mid
        else:
            hi = mid
    return tau


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp32":
        return x.to(torch.float32)
    raise ValueError(dtype)


def make_video_qkv(frames: int, height: int, width: int, heads: int, d: int,
                   dtype: str = "bf16", seed: int = 0,
                   f90_targets: Optional[Sequence[float]] = None,
                   n_calib: int = 256, device: str = "cpu") -> dict:
    """Return {"q","k","v": [1, heads, N, d] tensors on `device`, "tau", "f90_target"}.

    The random draws are made on the host either way; `device` only moves the
    per-head projections and the temperature calibration (values may differ
    from a host run in the last bits, so a test that compares the two sides
    hands both the same generated tensors)."""
    if d % 2:
        raise ValueError("d must be even")
    n = frames * height * width
    if f90_targets is None:
        f90_targets = [0.06] * heads
    f90_targets = list(f90_targets)
    assert len(f90_targets) == heads

    root = np.random.SeedSequence(seed)
    ss_tok, ss_heads = root.spawn(2)
    rng = np.random.default_rng(ss_tok)

    t, y, x = np.meshgrid(np.arange(frames), np.arange(height), np.arange(width), indexing="ij")
    p = np.stack([t.ravel() / frames, y.ravel() / height, x.ravel() / width], axis=1)
    nf = d // 2
    omega = rng.normal(0.0, 2.0 * math.pi * 1.5, size=(nf, 3))
    beta = rng.uniform(0.0, 2.0 * math.pi, size=nf)
    ph = p @ omega.T + beta
    phi = np.concatenate([np.sin(ph), np.cos(ph)], axis=1)
    anchors = rng.uniform(0.0, 1.0, size=(8, 3))
    offsets = rng.normal(0.0, 1.0, size=(8, d))
    wts = np.array([0.5, 1.0, 1.0])
    dist = (((p[:, None, :] - anchors[None, :, :]) * wts) ** 2).sum(-1)
    obj = dist.argmin(axis=1)
    X = phi + offsets[obj] + rng.normal(0.0, 0.1, size=(n, d))
    Xt = torch.from_numpy(X.astype(np.float32)).to(device)

    scale = 1.0 / math.sqrt(d)
    calib_idx = torch.from_numpy(((2 * np.arange(min(n_calib, n)) + 1) * n) // (2 * min(n_calib, n))).to(device)
    qs, ks, vs, taus = [], [], [], []
    for h, ssh in enumerate(ss_heads.spawn(heads)):
        rh = np.random.default_rng(ssh)
        std = math.sqrt(1.0 / d)
        Wq = torch.from_numpy(rh.normal(0.0, std, size=(d, d)).astype(np.float32)).to(device)
        Wk = torch.from_numpy(rh.normal(0.0, std, size=(d, d)).astype(np.float32)).to(device)
        Wv = torch.from_numpy(rh.normal(0.0, std, size=(d, d)).astype(np.float32)).to(device)
        q0 = Xt @ Wq
        kh = Xt @ Wk
        vh = Xt @ Wv
        logits = (q0[calib_idx].double() @ kh.double().T) * scale
        sorted_logits, _ = torch.sort(logits, dim=1, descending=True)
        tau = _calibrate_tau(sorted_logits, f90_targets[h])
        taus.append(tau)
        qs.append(_cast(q0 * tau, dtype))
        ks.append(_cast(kh, dtype))
        vs.append(_cast(vh, dtype))
    return {
        "q": torch.stack(qs)[None].contiguous(),
        "k": torch.stack(ks)[None].contiguous(),
        "v": torch.stack(vs)[None].contiguous(),
        "tau": np.array(taus),
        "f90_target": np.array(f90_targets),
        "calib_idx": calib_idx.cpu().numpy(),
    }


def make_workload_inputs(w: Workload, seed: Optional[int] = None, heads: Optional[int] = None,
                         d: Optional[int] = None, device: str = "cpu") -> dict:
    """Inputs for a named workload (optionally fewer heads or another head dim)."""
    H = w.heads if heads is None else heads
    dd = w.d if d is None else d
    targets = dataclasses.replace(w, heads=w.heads).f90_targets()[:H]
    return make_video_qkv(w.frames, w.height, w.width, H, dd, w.dtype,
                          w.seed if seed is None else seed, targets, device=device)
