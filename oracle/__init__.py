"""CPU oracle for one SparsePR attention call -- TEST INFRASTRUCTURE ONLY.

This package is a deliberately plain, slow NumPy implementation of what one
SparsePR call computes, written step by step from the pages that describe the
method.  It exists to check the HIP library.  Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it; the product path (``free_block_sparse_amd``) never does, and this
package imports nothing from the product path.

Citation legend used in the docstrings (page title, then section):
  [DG]  "Partition the Support, Reconstruct the Residual: 无训练稀疏注意力用于视频生成与世界模型"
        (ai-feeds.com paper digest); sections 方法/关键模块, 行业影响, 局限.
  [AB]  chatpaper.ai page for the paper; the English abstract.
  [TS]  "Resumen Técnico: SparsePR – Atención Dispersa Libre de Entrenamiento para
        Generación de Vídeo y Modelos de Mundo" (gist.science); sections 2.A, 2.B, 2.C, 4.
  [NE]  news explainer reposted from 科技行者 (huashangw.com); sections named by heading:
        NE/mass    "保留了多少注意力权重，不等于输出的误差有多小"
        NE/method  "SparsePR：先把误差聚拢，再用少量“抽查”去纠正" (incl. Figure 2)
        NE/exec    "稀疏执行怎么落地，误差怎么算才公平"
        NE/pool    "问题就出在"打包成组"这一步" (per-query vs shared-route support)
        NE/repair  "怎么分组，直接决定了剩下的误差好不好"修补"" (affine-explainable residual)

Parity status per function is listed in the header of ``sparsepr_oracle``.
"""

from .sparsepr_oracle import (  # noqa: F401
    OracleConfig,
    budget_pairs,
    dense_attention,
    fit_residual,
    group_by_labels,
    group_means,
    key_coordinates,
    key_metric,
    kmeans,
    query_coordinates,
    route,
    route_alpha,
    sample_queries,
    select_probes,
    sparse_attention,
    sparsepr_call,
    sparsepr_head,
    splitmix64,
    softmax_scale,
    structural_diagnostics,
    support_fraction,
    support_set,
)
