"""SparsePR attention as a PyTorch operator (a drop-in for dense SDPA calls).

``torch.ops.sparsepr.attention(q, k, v, ...)`` runs one SparsePR call through
the C ABI on the current stream: partition, router, probes, fit and the
corrected block-sparse attention, all in the library's kernels.  The
operator has a fake (meta) implementation, so it traces under FakeTensor
and torch.compile, and it enqueues without host synchronisation, so it can
be captured in a HIP graph once its workspace exists.

``layout="bhnd"`` takes [B, H, N, d] tensors as SDPA does; ``layout="bnhd"``
takes the [B, N, H, d] activations of a transformer block directly (the
library reads them through their strides, no copy).  The output has the
layout of q.  Every (b, h) is an independent call of the method, so B > 1 is
B*H heads.

Sources: [NE] NE/exec (the pages describe SparsePR as a replacement for the
dense attention call of a video diffusion transformer).
"""

from __future__ import annotations

from typing import Optional

import torch

from . import Workspace, make_config, sparsepr_attention

_workspaces: dict = {}


def _workspace(device) -> Workspace:
    key = (device.type, device.index)
    ws = _workspaces.get(key)
    if ws is None:
        ws = _workspaces[key] = Workspace()
    return ws


def _as_bhnd(t: torch.Tensor, layout: str) -> torch.Tensor:
    if layout == "bhnd":
        return t
    if layout == "bnhd":
        return t.permute(0, 2, 1, 3)
    raise ValueError(f"unknown layout {layout!r} (expected 'bhnd' or 'bnhd')")


@torch.library.custom_op("sparsepr::attention", mutates_args=())
def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, density: float = 0.25,
              n_kv_groups: int = 0, n_q_groups: int = 0, probe_rows: int = 64, residual_rank: int = 32,
              scale: float = 0.0, layout: str = "bhnd", router: int = 0, alpha: float = 0.9) -> torch.Tensor:
    """Corrected SparsePR attention; q, k, v share dtype, shape and layout.

    n_kv_groups / n_q_groups = 0 take the library default clamp(N/128, 1, 256).
    """
    qb, kb, vb = (_as_bhnd(t, layout) for t in (q, k, v))
    B, H, N, d = qb.shape
    kw = dict(density=density, probe_rows=min(probe_rows, N), residual_rank=residual_rank, scale=scale,
              router=router, alpha=alpha)
    if n_kv_groups > 0:
        kw["n_kv_groups"] = n_kv_groups
    if n_q_groups > 0:
        kw["n_q_groups"] = n_q_groups
    cfg = make_config(N, d, **kw)
    out = torch.empty_like(q)
    sparsepr_attention(qb, kb, vb, cfg, out=_as_bhnd(out, layout), workspace=_workspace(q.device))
    return out


@attention.register_fake
def _attention_fake(q, k, v, density=0.25, n_kv_groups=0, n_q_groups=0, probe_rows=64, residual_rank=32,
                    scale=0.0, layout="bhnd", router=0, alpha=0.9):
    torch._check(q.shape == k.shape and q.shape == v.shape, lambda: "q, k, v must share their shape")
    torch._check(q.dim() == 4, lambda: "q, k, v must be 4-D")
    return torch.empty_like(q)


def scaled_dot_product_attention(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                                 scale: Optional[float] = None, density: float = 0.25,
                                 **kw) -> torch.Tensor:
    """SDPA-shaped entry point ([B, H, N, d] inputs, no mask, no dropout)."""
    return torch.ops.sparsepr.attention(query, key, value, density=density,
                                        scale=0.0 if scale is None else float(scale), **kw)
