"""Degenerate settings and random seeds against the oracle (GPU, C ABI).

Each case is fed the oracle's partition: the routing must match bit for bit,
and the hard-drop and corrected outputs must be finite and within the bf16
bounds.  The cases: one group on each side, no probes, rank 0, only the
mandatory cells (over budget), fewer tokens than one query tile, and six
seeds with many small cells and split tiles (one of those once produced
non-finite rows).
"""

import numpy as np
import pytest
import torch

import free_block_sparse_amd as sp
from parity_cases import EDGE_CASES, case, inputs, max_abs, oracle_result, rel_frob, tolerances

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_edge_case_routing_and_outputs(name):
    c = case(name)
    print(f"[edge] case={name} N={c.n} H={c.heads} d={c.d} G_K={c.gk} G_Q={c.gq} rho={c.density} "
          f"M={c.probes} r={c.rank}", flush=True)
    x = inputs(name)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    cfg = sp.make_config(c.n, c.d, **c.lib_cfg_kwargs())
    heads = oracle_result(name)
    ql = torch.tensor(np.stack([h["q_labels"] for h in heads]), dtype=torch.int32).cuda()
    kl = torch.tensor(np.stack([h["kv_labels"] for h in heads]), dtype=torch.int32).cuda()
    res = sp.sparsepr_route(q, k, v, cfg, ql, kl)
    hard = sp.sparsepr_sparse_attention(q, k, v, cfg, ql, kl)
    out = sp.sparsepr_attention_with_partition(q, k, v, cfg, ql, kl)
    torch.cuda.synchronize()
    stats = sp.stats_to_dicts(res["stats"])
    ma, rf = tolerances(c.dtype)
    for h, r in enumerate(heads):
        rt = r["route"]
        rp = res["csr_rowptr"][h].cpu().numpy()
        assert np.array_equal(rp, rt["csr_rowptr"])
        assert np.array_equal(res["csr_cols"][h, :rp[-1]].cpu().numpy(), rt["csr_cols"])
        assert stats[h]["routed_pairs"] == rt["routed_pairs"]
        assert stats[h]["over_budget"] == int(rt["over_budget"])
        got_h = hard[0, h].double().cpu().numpy()
        got = out[0, h].double().cpu().numpy()
        assert np.isfinite(got_h).all() and np.isfinite(got).all()
        assert max_abs(got_h, r["hard_drop"]) <= ma and rel_frob(got_h, r["hard_drop"]) <= rf
        assert max_abs(got, r["out"]) <= ma and rel_frob(got, r["out"]) <= rf
