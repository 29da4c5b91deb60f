"""Shared parity cases: seeded inputs, matching oracle and library configs."""

from __future__ import annotations

import dataclasses
import functools

import numpy as np

from oracle import (OracleConfig, dense_attention, group_by_labels, group_means, key_coordinates, kmeans,
                    query_coordinates, softmax_scale, sparsepr_head)
from synth import make_video_qkv, make_workload_inputs, workload


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    frames: int
    height: int
    width: int
    heads: int
    d: int
    dtype: str
    gk: int
    gq: int
    density: float
    probes: int
    rank: int
    f90: float = 0.06
    seed: int = 7
    mode: str = "response_coupled"
    workload: str = ""
    router: str = "budget"
    alpha: float = 0.9
    ridge_mode: str = "relative"
    ridge_lambda: float = 1.0
    rank_cap: float = 1.0
    svd_weighted: bool = False
    centred: bool = False

    @property
    def n(self):
        return self.frames * self.height * self.width

    def oracle_cfg(self) -> OracleConfig:
        return OracleConfig(density=self.density, probe_rows=self.probes, n_kv_groups=self.gk,
                            n_q_groups=self.gq, residual_rank=self.rank, partition_mode=self.mode,
                            router=self.router, alpha=self.alpha, ridge_mode=self.ridge_mode,
                            ridge_lambda=self.ridge_lambda, rank_cap=self.rank_cap,
                            svd_weighted=self.svd_weighted, centred_query_coords=self.centred)

    def lib_cfg_kwargs(self) -> dict:
        return dict(density=self.density, probe_rows=self.probes, n_kv_groups=self.gk, n_q_groups=self.gq,
                    residual_rank=self.rank, partition_mode=0 if self.mode == "response_coupled" else 1,
                    router=0 if self.router == "budget" else 1, alpha=self.alpha, ridge_mode=self.ridge_mode,
                    ridge_lambda=self.ridge_lambda, rank_cap=self.rank_cap, svd_weighted=int(self.svd_weighted),
                    centred_query_coords=int(self.centred))


CASES = {
    # the tiny fp32 call of the workload table (16/16 groups, 64 probes, rank 16)
    "c1_tiny_fp32": Case("c1_tiny_fp32", 4, 16, 16, 1, 64, "fp32", 16, 16, 0.25, 64, 16,
                         workload="c1_tiny_fp32"),
    # bf16, d = 64, ragged groups and a ragged key tail, 2 heads
    "bf16_d64": Case("bf16_d64", 4, 10, 25, 2, 64, "bf16", 12, 10, 0.3, 32, 8, seed=11),
    # bf16, d = 128, few large query groups: several query tiles per group
    "bf16_d128": Case("bf16_d128", 2, 16, 32, 2, 128, "bf16", 16, 4, 0.3, 48, 8, seed=12),
    # comparison partition (independent Q/K k-means)
    "bf16_d64_indep": Case("bf16_d64_indep", 4, 10, 25, 1, 64, "bf16", 12, 10, 0.3, 32, 8, seed=13,
                           mode="independent"),
    # two heads of the 8k video-DiT call
    "c2_two_heads": Case("c2_two_heads", 8, 32, 32, 2, 64, "bf16", 64, 64, 0.25, 64, 32,
                         workload="c2_dit_8k"),
    # many groups: 300 key groups (more than one assignment workgroup's waves
    # hold) and 200 query groups at d = 128
    "many_groups": Case("many_groups", 4, 16, 40, 1, 128, "bf16", 300, 200, 0.3, 32, 8, seed=14),
    # a query group with one granted key group of <= 32 keys and a <= 64-row
    # remainder: one key half of its split tile sees no key at all
    "split_tiny_cell": Case("split_tiny_cell", 4, 10, 25, 2, 64, "bf16", 12, 10, 0.3, 32, 8, seed=21),
    # alpha-coverage router: ragged groups at d = 64, and two heads of the 8k call
    "alpha_bf16_d64": Case("alpha_bf16_d64", 4, 10, 25, 2, 64, "bf16", 12, 10, 0.3, 32, 8, seed=15,
                           router="alpha", alpha=0.8),
    "alpha_c2": Case("alpha_c2", 8, 32, 32, 2, 64, "bf16", 64, 64, 0.25, 64, 32, workload="c2_dit_8k",
                     router="alpha", alpha=0.9),
    # absolute ridge lambda: the tiny fp32 call with the lambda = 1e-3 its
    # workload states, and a bf16 case
    "c1_abs_lambda": Case("c1_abs_lambda", 4, 16, 16, 1, 64, "fp32", 16, 16, 0.25, 64, 16,
                          workload="c1_tiny_fp32", ridge_mode="absolute", ridge_lambda=1e-3),
    "bf16_d128_abs": Case("bf16_d128_abs", 2, 16, 32, 2, 128, "bf16", 16, 4, 0.3, 48, 8, seed=12,
                          ridge_mode="absolute", ridge_lambda=0.05),
    # fit and coordinate variants: the residual subspace from the weighted
    # SVD (a d x d Gram with 200 > d probes, and the dual M x M form), a rank
    # capped at half the probes (16 probes, rank 16 -> 8), centred query
    # coordinates
    "wsvd_d64": Case("wsvd_d64", 4, 10, 25, 2, 64, "bf16", 12, 10, 0.3, 32, 8, seed=16, svd_weighted=True),
    "wsvd_primal": Case("wsvd_primal", 2, 16, 32, 1, 64, "bf16", 16, 8, 0.3, 200, 16, seed=17, svd_weighted=True),
    "cap_m16": Case("cap_m16", 4, 16, 16, 2, 64, "bf16", 16, 16, 0.25, 16, 16, seed=18, rank_cap=0.5),
    "centred_c2": Case("centred_c2", 8, 32, 32, 2, 64, "bf16", 64, 64, 0.25, 64, 32, workload="c2_dit_8k",
                       centred=True),
}


# Degenerate settings and random seeds (tests/test_gpu_edge_cases.py): one
# group on each side, no probes, rank 0, mandatory cells only (over budget),
# fewer tokens than one tile, more than 64 probes, a residual rank above 32,
# and seeds with many small cells and split tiles.
EDGE_CASES = {
    "one_group": Case("one_group", 2, 8, 20, 1, 64, "bf16", 1, 1, 0.3, 16, 4, seed=31),
    "no_probes": Case("no_probes", 2, 8, 20, 1, 64, "bf16", 6, 5, 0.3, 0, 4, seed=32),
    "rank0": Case("rank0", 2, 8, 20, 1, 64, "bf16", 6, 5, 0.3, 16, 0, seed=33),
    "mandatory_only": Case("mandatory_only", 2, 8, 20, 1, 64, "bf16", 8, 8, 0.02, 16, 4, seed=34),
    "tiny_n": Case("tiny_n", 1, 10, 10, 1, 64, "bf16", 4, 4, 0.5, 8, 2, seed=35),
    # more than 64 probes: the dual ridge system of order M = 128 (d = 128),
    # and M = 200 > d = 64 (the primal d x d system)
    "probes128": Case("probes128", 2, 16, 32, 1, 128, "bf16", 16, 4, 0.3, 128, 16, seed=36),
    "probes200_d64": Case("probes200_d64", 2, 16, 32, 1, 64, "bf16", 16, 8, 0.3, 200, 16, seed=37),
    # residual rank 48 > 32: the correction runs over a second, partial block
    # of 32 rank columns (the rest of it zero)
    "rank48": Case("rank48", 2, 16, 32, 1, 128, "bf16", 16, 8, 0.3, 64, 48, seed=38),
    **{f"seed{s}": Case(f"seed{s}", 2, 10, 20, 2, 64 if s % 2 else 128, "bf16", 10, 6, 0.25, 16, 4, seed=40 + s)
       for s in range(6)},
}


def case(name: str) -> Case:
    return CASES[name] if name in CASES else EDGE_CASES[name]


@functools.lru_cache(maxsize=None)
def inputs(name: str):
    c = case(name)
    if c.workload:
        return make_workload_inputs(workload(c.workload), heads=c.heads)
    return make_video_qkv(c.frames, c.height, c.width, c.heads, c.d, c.dtype, c.seed, [c.f90] * c.heads)


@functools.lru_cache(maxsize=None)
def oracle_result(name: str):
    c = case(name)
    x = inputs(name)
    cfg = c.oracle_cfg()
    heads = []
    for h in range(c.heads):
        q = x["q"][0, h].double().numpy()
        k = x["k"][0, h].double().numpy()
        v = x["v"][0, h].double().numpy()
        r = sparsepr_head(q, k, v, cfg, bh=h)
        r["dense"] = dense_attention(q, k, v, r["scale"])
        heads.append(r)
    return heads


def rel_frob(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)).max())


def tolerances(dtype: str):
    """(max-abs, relative Frobenius) bounds for attention outputs.

    bf16: the bounds stated for bf16 outputs against the fp64/fp32 oracle.
    fp32: the kernels accumulate in fp32 over a few thousand terms, so errors
    stay near 1e-6 relative; the bounds leave two orders of margin.
    """
    return (2e-2, 5e-3) if dtype == "bf16" else (1e-4, 1e-5)


def key_labels_from_metric(k64: np.ndarray, m_k, cfg: OracleConfig) -> np.ndarray:
    """The oracle's key k-means run on coordinates built from a given M_K."""
    n, d = k64.shape
    s = softmax_scale(cfg, d)
    r_k = min(cfg.key_coord_rank, d, min(cfg.n_sample_q, n))
    z, _, _ = key_coordinates(k64, np.asarray(m_k, dtype=np.float64), r_k, s)
    labels, _ = kmeans(z, cfg.n_kv_groups, cfg.kmeans_iters)
    return labels


def query_labels_given_keys(q64: np.ndarray, k64: np.ndarray, kv_labels, cfg: OracleConfig) -> np.ndarray:
    """The oracle's query k-means run on the query coordinates that a given
    key partition defines."""
    s = softmax_scale(cfg, q64.shape[1])
    perm_k, nk, off_k = group_by_labels(np.asarray(kv_labels, dtype=np.int64), cfg.n_kv_groups)
    cbar = group_means(k64, perm_k, off_k)
    u = query_coordinates(q64, cbar[nk > 0], s, centred=cfg.centred_query_coords)
    labels, _ = kmeans(u, cfg.n_q_groups, cfg.kmeans_iters)
    return labels


def oracle_key_labels_from_metric(name: str, h: int, m_k) -> np.ndarray:
    """key_labels_from_metric on head h of a named case."""
    return key_labels_from_metric(inputs(name)["k"][0, h].double().numpy(), m_k, case(name).oracle_cfg())


def oracle_out_given_partition(name: str, h: int, q_labels, kv_labels) -> np.ndarray:
    """The oracle's corrected output of head h on a given partition."""
    c = case(name)
    x = inputs(name)
    q, k, v = (x[t][0, h].double().numpy() for t in ("q", "k", "v"))
    r = sparsepr_head(q, k, v, c.oracle_cfg(), bh=h, q_labels=np.asarray(q_labels, dtype=np.int64),
                      kv_labels=np.asarray(kv_labels, dtype=np.int64))
    return r["out"]


def oracle_query_labels_given_keys(name: str, h: int, kv_labels) -> np.ndarray:
    """query_labels_given_keys on head h of a named case."""
    x = inputs(name)
    return query_labels_given_keys(x["q"][0, h].double().numpy(), x["k"][0, h].double().numpy(), kv_labels,
                                   case(name).oracle_cfg())
