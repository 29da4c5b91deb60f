"""The long-sequence call at full size: 40 heads, 75,600 tokens, d = 128, bf16,
density 22%, 256 + 256 groups, 64 probe rows, rank 32 (GPU, C ABI).

The seeded generator runs its per-head projections on the GPU (the host draws
the same random numbers); head 0's bf16 rows are then copied to the host, so
the oracle and the library see identical inputs.  The whole 40-head call runs
once, in the launch configuration of the benchmark's call.  Then:
- every head's output is finite; every head's routed pairs stay within its
  budget (the mandatory cells alone may exceed it) and fall short of it by less
  than one cell, and the reported executed density matches the pair counts;
- head 0's k-means partitions agree with the oracle's on >= 99% of tokens,
  and its corrected error against dense attention (on every eighth row) is
  within 1.1x the oracle's;
- with the oracle's labels injected for head 0, its routing is bit-exact and
  its corrected output is within the bf16 bounds of the oracle's.
"""

import numpy as np
import pytest
import torch

import free_block_sparse_amd as sp
from oracle import OracleConfig, budget_pairs, dense_attention, sparsepr_head
from parity_cases import key_labels_from_metric, max_abs, query_labels_given_keys, rel_frob, tolerances
from synth import make_workload_inputs, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = workload("c4_long_75k")
    print(f"[c4] generating {w.name} on the GPU: H={w.heads} N={w.n} d={w.d}", flush=True)
    x = make_workload_inputs(w, device="cuda")
    q, k, v = x["q"], x["k"], x["v"]
    kw = dict(density=w.density, probe_rows=w.probe_rows, n_kv_groups=w.n_kv_groups, n_q_groups=w.n_q_groups,
              residual_rank=w.residual_rank)
    cfg = sp.make_config(w.n, w.d, **kw)
    ws = sp.Workspace()
    print("[c4] full call", flush=True)
    out = sp.sparsepr_attention(q, k, v, cfg, workspace=ws)
    ql, kl = sp.sparsepr_partition(q, k, v, cfg, workspace=ws)
    _, mk, _, _ = sp.sparsepr_key_metric(q, k, v, cfg, workspace=ws)
    res = sp.sparsepr_route(q, k, v, cfg, ql, kl, workspace=ws)
    torch.cuda.synchronize()
    h64 = {t: x[t][0, 0].double().cpu().numpy() for t in ("q", "k", "v")}
    return dict(w=w, q=q, k=k, v=v, cfg=cfg, ocfg=OracleConfig(**kw), ws=ws, out=out, ql=ql, kl=kl, mk=mk,
                stats=sp.stats_to_dicts(res["stats"]), h64=h64)


def test_c4_all_heads_finite_and_within_budget(c4):
    w = c4["w"]
    assert torch.isfinite(c4["out"].float()).all()
    n2 = float(w.n) * w.n
    for h, st in enumerate(c4["stats"]):
        assert st["budget_pairs"] == budget_pairs(w.density, w.n, w.probe_rows), h
        assert st["routed_pairs"] <= max(st["budget_pairs"], st["mandatory_pairs"]), h
        if st["mandatory_pairs"] <= st["budget_pairs"]:
            # the grant prefix stops at the first cell that does not fit: what
            # is left of the budget is less than that cell, at most the cell of
            # the head's most populous query and key groups
            nq = torch.bincount(c4["ql"][h].long(), minlength=w.n_q_groups).max().item()
            nk = torch.bincount(c4["kl"][h].long(), minlength=w.n_kv_groups).max().item()
            assert st["budget_pairs"] - st["routed_pairs"] < nq * nk, h
        assert abs(st["rho_exec"] - (st["routed_pairs"] + w.probe_rows * w.n) / n2) < 1e-12


@pytest.fixture(scope="module")
def oracle0(c4):
    print("[c4] oracle call on head 0", flush=True)
    h64 = c4["h64"]
    return sparsepr_head(h64["q"], h64["k"], h64["v"], c4["ocfg"], bh=0)


def test_c4_partition_agreement_head0(c4, oracle0):
    h64, ocfg, r = c4["h64"], c4["ocfg"], oracle0
    kl0 = c4["kl"][0].cpu().numpy()
    ql0 = c4["ql"][0].cpu().numpy()
    agree_k = (kl0 == r["kv_labels"]).mean()
    agree_q = (ql0 == r["q_labels"]).mean()
    cond_k = (kl0 == key_labels_from_metric(h64["k"], c4["mk"][0].cpu().numpy(), ocfg)).mean()
    cond_q = (ql0 == query_labels_given_keys(h64["q"], h64["k"], kl0, ocfg)).mean()
    rows = np.arange(0, c4["w"].n, 8)
    dense = dense_attention(h64["q"][rows], h64["k"], h64["v"], r["scale"])
    err_gpu = rel_frob(c4["out"][0, 0].double().cpu().numpy()[rows], dense)
    err_ora = rel_frob(r["out"][rows], dense)
    print(f"  head 0: agreement K {agree_k:.4f} Q {agree_q:.4f} (conditional K {cond_k:.4f} Q {cond_q:.4f}); "
          f"err vs dense on every 8th row gpu {err_gpu:.4f} oracle {err_ora:.4f}", flush=True)
    assert agree_k >= 0.99 and agree_q >= 0.99
    assert err_gpu <= 1.1 * err_ora


def test_c4_oracle_partition_parity_head0(c4, oracle0):
    r = oracle0
    ql_mix, kl_mix = c4["ql"].clone(), c4["kl"].clone()
    ql_mix[0] = torch.from_numpy(r["q_labels"].astype(np.int32))
    kl_mix[0] = torch.from_numpy(r["kv_labels"].astype(np.int32))
    q, k, v, cfg, ws = c4["q"], c4["k"], c4["v"], c4["cfg"], c4["ws"]
    res = sp.sparsepr_route(q, k, v, cfg, ql_mix, kl_mix, workspace=ws)
    corr = sp.sparsepr_attention_with_partition(q, k, v, cfg, ql_mix, kl_mix, workspace=ws)
    torch.cuda.synchronize()
    rt = r["route"]
    rp = res["csr_rowptr"][0].cpu().numpy()
    assert np.array_equal(rp, rt["csr_rowptr"])
    assert np.array_equal(res["csr_cols"][0, :rp[-1]].cpu().numpy(), rt["csr_cols"])
    assert sp.stats_to_dicts(res["stats"])[0]["routed_pairs"] == rt["routed_pairs"]
    got = corr[0, 0].double().cpu().numpy()
    ma, rf = tolerances("bf16")
    print(f"  head 0, oracle partition: corrected max-abs {max_abs(got, r['out']):.3e} "
          f"rel {rel_frob(got, r['out']):.3e}", flush=True)
    assert max_abs(got, r["out"]) <= ma and rel_frob(got, r["out"]) <= rf
