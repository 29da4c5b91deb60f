"""Structural diagnostics measured on the library's outputs against the oracle's.

The library's partition, hard-drop output and dense output feed
free_block_sparse_amd.diagnostics; the oracle measures the same partition (the
GPU's labels) with its own fp64 sparse and dense outputs.  Support sizes are
decided in fp64 on both sides from the same bf16 inputs, so they agree
exactly; the residual measures differ by the bf16 rounding of the stored
outputs (relative 2^-9 of |O|, a few percent of the residual at most here).
"""

import numpy as np
import pytest
import torch

import free_block_sparse_amd as sp
from free_block_sparse_amd.diagnostics import structural_diagnostics
from oracle import sparsepr_head, structural_diagnostics as oracle_diagnostics
from parity_cases import case, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["bf16_d64", "bf16_d64_indep"])
def test_diagnostics_match_the_oracle(name):
    c = case(name)
    x = inputs(name)
    print(f"[diag] case={name} N={c.n} H={c.heads} d={c.d}", flush=True)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    cfg = sp.make_config(c.n, c.d, **c.lib_cfg_kwargs())
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(c.n, size=300, replace=False))
    got = structural_diagnostics(q, k, v, cfg, rows=rows.tolist())
    ql, kl = sp.sparsepr_partition(q, k, v, cfg)
    for h in range(c.heads):
        q64, k64, v64 = (x[t][0, h].double().numpy() for t in ("q", "k", "v"))
        qlab = ql[h].cpu().numpy().astype(np.int64)
        klab = kl[h].cpu().numpy().astype(np.int64)
        r = sparsepr_head(q64, k64, v64, c.oracle_cfg(), bh=h, q_labels=qlab, kv_labels=klab)
        want = oracle_diagnostics(q64, k64, v64, qlab, r["hard_drop"], r["scale"], rows=rows)
        g = got[h]
        print(f"  head {h}: " + ", ".join(f"{key} gpu {g[key]:.5f} oracle {want[key]:.5f}" for key in want))
        assert g["per_query_support"] == pytest.approx(want["per_query_support"], abs=1e-12)
        assert g["pooled_support"] == pytest.approx(want["pooled_support"], abs=1e-12)
        assert g["hard_drop_error"] == pytest.approx(want["hard_drop_error"], rel=1e-2)
        assert g["affine_explained"] == pytest.approx(want["affine_explained"], abs=2e-2)
        assert g["orthogonal_energy"] == pytest.approx(want["orthogonal_energy"], rel=5e-2, abs=1e-6)
        # the measures' own invariants
        assert g["pooled_support"] >= g["per_query_support"] > 0.0
        assert 0.0 <= g["affine_explained"] <= 1.0
