"""Structural diagnostics of a partition (analysis, not part of the call).

Measures the pages' three structural claims on one call's inputs ([NE]: news
explainer reposted from 科技行者, sections "问题就出在“打包成组”这一步" and
"怎么分组，直接决定了剩下的误差好不好“修补”"; [TS]: "Resumen Técnico: SparsePR ..."
(gist.science) 3, structural analysis, and 4, orthogonal residual energy):

* per-query support: the smallest fraction of keys holding `mass` of a
  query's softmax mass, averaged over the measured queries;
* pooled support: for each query group, the fraction of keys in the union of
  its measured members' supports -- what one shared route must keep for every
  member -- averaged over the measured queries;
* hard-drop error ||O_dense - O_sparse||_F / ||O_dense||_F;
* affine-explainable fraction of the residual R = O_dense - O_sparse: the
  share of ||R||_F^2 that the best affine function of the sparse output
  explains (least squares over all rows), and the unexplained (orthogonal)
  residual energy relative to ||O_dense||_F^2.

The partition, the hard-drop sparse output and the dense output come from the
library's kernels (sparsepr_partition, sparsepr_sparse_attention,
sparsepr_dense_attention).  The measures themselves -- softmax rows of the
measured queries, their sorted cumulative mass, the least-squares projection
-- are computed here with fp64 torch operations on the device; they are
measurements of the kernels' outputs and never feed back into a call.
"""

from __future__ import annotations

import math
from typing import Optional

from . import (_torch, sparsepr_dense_attention, sparsepr_partition, sparsepr_sparse_attention)


def _scale(cfg, d: int) -> float:
    import numpy as np
    s = cfg.scale if cfg.scale > 0 else 1.0 / math.sqrt(d)
    return float(np.float32(s))


def support_counts(p, mass: float = 0.9):
    """Smallest number of keys per row whose probabilities sum to `mass` of the
    row's total, and the row's keys in descending probability (ties by index)."""
    torch = _torch()
    ps, order = torch.sort(p, dim=1, descending=True, stable=True)
    c = torch.cumsum(ps, dim=1)
    thr = mass * c[:, -1:] * (1.0 - 1e-12)
    k = (c < thr).sum(dim=1) + 1
    return torch.clamp(k, max=p.shape[1]), order


def structural_diagnostics(q, k, v, cfg, rows: Optional[list] = None, mass: float = 0.9, workspace=None,
                           row_chunk: int = 256) -> list:
    """Diagnostics per (b, h) slice, in (b, h) order.

    rows: token indices whose support is measured (the same for every slice);
    None measures every row.  The residual measures use every row.
    """
    torch = _torch()
    ql, kl = sparsepr_partition(q, k, v, cfg, workspace=workspace)
    hard = sparsepr_sparse_attention(q, k, v, cfg, ql, kl, workspace=workspace)
    dense = sparsepr_dense_attention(q, k, v, scale=cfg.scale)
    B, H, N, d = q.shape
    s = _scale(cfg, d)
    sel = torch.arange(N, device=q.device) if rows is None else torch.as_tensor(rows, device=q.device)
    res = []
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            od = dense[b, h].double()
            osp = hard[b, h].double()
            r = od - osp
            xa = torch.cat([torch.ones(N, 1, dtype=torch.float64, device=q.device), osp], dim=1)
            qm, _ = torch.linalg.qr(xa)
            left = r - qm @ (qm.T @ r)
            rr = float((r * r).sum())
            ll = float((left * left).sum())
            # supports of the measured rows
            k64 = k[b, h].double()
            labels = ql[bh].long()[sel]
            counts = []
            pooled_sum = 0.0
            unions = {}
            for c0 in range(0, sel.numel(), row_chunk):
                idx = sel[c0:c0 + row_chunk]
                logits = s * (q[b, h, idx].double() @ k64.T)
                p = torch.softmax(logits, dim=1)
                cnt, order = support_counts(p, mass)
                counts.append(cnt)
                lab = labels[c0:c0 + row_chunk]
                for i in range(idx.numel()):
                    g = int(lab[i])
                    m = unions.get(g)
                    if m is None:
                        m = torch.zeros(N, dtype=torch.bool, device=q.device)
                        unions[g] = m
                    m[order[i, :int(cnt[i])]] = True
            counts = torch.cat(counts).double()
            sizes = torch.bincount(labels, minlength=max(unions) + 1 if unions else 1).double()
            for g, m in unions.items():
                pooled_sum += float(m.sum()) / N * float(sizes[g])
            res.append({
                "per_query_support": float(counts.mean()) / N,
                "pooled_support": pooled_sum / float(sel.numel()),
                "hard_drop_error": float(torch.linalg.norm(r) / torch.linalg.norm(od)),
                "affine_explained": 1.0 - ll / rr if rr > 0 else 1.0,
                "orthogonal_energy": ll / float((od * od).sum()),
            })
    return res
