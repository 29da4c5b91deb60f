"""GPU path vs the CPU oracle on the same seeded inputs (small sizes).

Every comparison goes through the C ABI of libsparsepr.  Integer stages
(sample, grouping, permutation, routing) must match bit for bit when the GPU
is fed the oracle's partition; floating outputs must stay inside the stated
tolerances; the partition computed on the GPU must agree with the oracle's on
at least 99% of tokens, with the corrected-output error against dense within
1.1x the oracle's.
"""

import numpy as np
import pytest
import torch

import free_block_sparse_amd as sp
from parity_cases import (CASES, case, inputs, max_abs, oracle_key_labels_from_metric, oracle_out_given_partition,
                          oracle_query_labels_given_keys, oracle_result, rel_frob, tolerances)

pytestmark = pytest.mark.gpu

ALL = list(CASES)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev_inputs(name):
    x = inputs(name)
    return (x["q"].cuda(), x["k"].cuda(), x["v"].cuda())


def lib_cfg(name):
    c = CASES[name]
    return sp.make_config(c.n, c.d, **c.lib_cfg_kwargs())


def oracle_labels(name):
    heads = oracle_result(name)
    ql = torch.tensor(np.stack([h["q_labels"] for h in heads]), dtype=torch.int32).cuda()
    kl = torch.tensor(np.stack([h["kv_labels"] for h in heads]), dtype=torch.int32).cuda()
    return ql, kl


def banner(name, what):
    c = CASES[name]
    print(f"[parity] {what} case={name} N={c.n} H={c.heads} d={c.d} dtype={c.dtype}", flush=True)


@pytest.mark.parametrize("name", ALL)
def test_key_metric_sample_and_spectrum(name):
    c = CASES[name]
    if c.mode != "response_coupled":
        pytest.skip("no key metric in the independent partition")
    banner(name, "key_metric")
    q, k, v = dev_inputs(name)
    smp, mk, ev, km = sp.sparsepr_key_metric(q, k, v, lib_cfg(name))
    torch.cuda.synchronize()
    for h, r in enumerate(oracle_result(name)):
        assert np.array_equal(smp[h].cpu().numpy(), r["sample"])  # integer spec: bit-exact
        mk_gpu = mk[h].cpu().numpy()
        # fp64 sums of exact products: only the order of the additions differs
        assert rel_frob(mk_gpu, r["m_k"]) < 1e-13
        lam_ref = np.sort(np.linalg.eigvalsh(r["m_k"]))[::-1]
        lam = ev[h].cpu().numpy()
        # Weyl: eigenvalues move by at most ||dM||_2 <= ||dM||_F; the fp64
        # reduction and bisection add a backward error of order n eps ||M||_F
        n = mk_gpu.shape[0]
        bound = np.linalg.norm(mk_gpu - r["m_k"]) + 10 * n * 2.3e-16 * np.linalg.norm(r["m_k"])
        assert np.abs(lam - lam_ref).max() <= bound
        check_key_map(km[h].cpu().numpy(), mk_gpu, r["scale"])


def check_key_map(km, mk, s):
    """km km^T must equal s^2 U_r Lambda_r U_r^T for the leading r eigenpairs of
    the metric the library computed (sign- and rotation-free within clusters)."""
    r = km.shape[1]
    lam, vec = np.linalg.eigh(mk)
    lam, vec = lam[::-1], vec[:, ::-1]
    ref = (s * s) * (vec[:, :r] * np.clip(lam[:r], 0, None)) @ vec[:, :r].T
    got = km @ km.T
    gap = lam[r - 1] - lam[r] if r < len(lam) else lam[0]
    # fp64 eigenvectors: subspace error of order n eps ||M|| / gap
    tol = 1000 * 2.3e-16 * (1.0 + lam[0] / max(gap, 1e-30))
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"[parity] key map rel err {err:.2e} (tol {tol:.2e}, boundary gap {gap / lam[0]:.2e} of lambda_1)",
          flush=True)
    assert err <= tol


@pytest.mark.parametrize("kind", ["close_pairs", "repeated_top"])
def test_key_map_with_clustered_spectrum(kind):
    """Metrics whose leading eigenvalues sit in tight clusters (relative gaps
    1e-4 and 1e-3, or exactly repeated): the eigenvectors of the clusters are
    orthogonalised against each other, and exact repeats take the shifted-QR
    path; both must reproduce the leading eigenspaces."""
    n, d, rk = 256, 64, 16
    print(f"[parity] key_map clustered spectrum kind={kind} N={n} d={d} r_K={rk} fp32", flush=True)
    rng = np.random.default_rng(7)
    lam = np.geomspace(1.0, 0.02, d)
    if kind == "close_pairs":
        lam[3] = lam[2] * (1 - 1e-4)
        lam[7] = lam[6] * (1 - 1e-3)
        lam[8] = lam[7] * (1 - 1e-4)
    else:
        lam[1:4] = lam[1]
        lam[9:11] = lam[9]
    u, _ = np.linalg.qr(rng.standard_normal((n, d)))
    v, _ = np.linalg.qr(rng.standard_normal((d, d)))
    q = (np.sqrt(n) * (u * np.sqrt(lam)) @ v.T).astype(np.float32)
    qt = torch.from_numpy(q).reshape(1, 1, n, d).cuda()
    cfg = sp.make_config(n, d, n_sample_q=256, key_coord_rank=rk, n_kv_groups=4, n_q_groups=4,
                         probe_rows=8, residual_rank=4)
    smp, mk, ev, km = sp.sparsepr_key_metric(qt, qt.clone(), qt.clone(), cfg)
    torch.cuda.synchronize()
    assert np.array_equal(np.sort(smp[0].cpu().numpy()), np.arange(n))
    mk64 = mk[0].cpu().numpy()
    lam_ref = np.sort(np.linalg.eigvalsh(mk64))[::-1]
    assert np.abs(ev[0].cpu().numpy() - lam_ref).max() <= 10 * d * 2.3e-16 * np.linalg.norm(mk64)
    check_key_map(km[0].cpu().double().numpy(), mk64, float(np.float32(1.0 / np.sqrt(d))))


@pytest.mark.parametrize("name", ALL)
def test_grouping_and_routing_bit_exact(name):
    banner(name, "route")
    q, k, v = dev_inputs(name)
    ql, kl = oracle_labels(name)
    res = sp.sparsepr_route(q, k, v, lib_cfg(name), ql, kl)
    torch.cuda.synchronize()
    stats = sp.stats_to_dicts(res["stats"])
    for h, r in enumerate(oracle_result(name)):
        assert np.array_equal(res["perm_q"][h].cpu().numpy(), r["perm_q"])
        assert np.array_equal(res["perm_k"][h].cpu().numpy(), r["perm_k"])
        assert np.array_equal(res["off_q"][h].cpu().numpy(), r["off_q"])
        assert np.array_equal(res["off_k"][h].cpu().numpy(), r["off_k"])
        rt = r["route"]
        rp = res["csr_rowptr"][h].cpu().numpy()
        assert np.array_equal(rp, rt["csr_rowptr"])
        assert np.array_equal(res["csr_cols"][h, :rp[-1]].cpu().numpy(), rt["csr_cols"])
        assert stats[h]["routed_pairs"] == rt["routed_pairs"]
        assert stats[h]["rho_exec"] == pytest.approx(rt["rho_exec"], abs=0)


@pytest.mark.parametrize("name", ALL)
def test_sparse_attention_matches_oracle(name):
    banner(name, "sparse_attention")
    c = CASES[name]
    q, k, v = dev_inputs(name)
    ql, kl = oracle_labels(name)
    out = sp.sparsepr_sparse_attention(q, k, v, lib_cfg(name), ql, kl)
    torch.cuda.synchronize()
    ma, rf = tolerances(c.dtype)
    for h, r in enumerate(oracle_result(name)):
        got = out[0, h].double().cpu().numpy()
        assert max_abs(got, r["hard_drop"]) <= ma
        assert rel_frob(got, r["hard_drop"]) <= rf


@pytest.mark.parametrize("name", ALL)
def test_probe_rows_and_fit_match_oracle(name):
    banner(name, "probe_fit")
    c = CASES[name]
    q, k, v = dev_inputs(name)
    ql, kl = oracle_labels(name)
    res = sp.sparsepr_probe_fit(q, k, v, lib_cfg(name), ql, kl)
    torch.cuda.synchronize()
    ma, rf = tolerances(c.dtype)
    for h, r in enumerate(oracle_result(name)):
        assert np.array_equal(res["probe_pos"][h].cpu().numpy(), r["probes"])
        od = res["o_dense"][h].double().cpu().numpy()
        os_ = res["o_sparse"][h].double().cpu().numpy()
        assert max_abs(od, r["o_dense_probe"]) <= ma and rel_frob(od, r["o_dense_probe"]) <= rf
        osp_ref = r["o_sparse_perm"][r["probes"]]
        assert max_abs(os_, osp_ref) <= ma and rel_frob(os_, osp_ref) <= rf
        assert int(res["rank"][h]) == r["fit"]["rank"]


@pytest.mark.parametrize("name", ALL)
def test_fit_matches_oracle_fit_on_the_same_probe_rows(name):
    """The fitted correction itself: B = W V^T and b from the library against
    the oracle's weighted ridge fit run on the library's own probe rows (its
    exact dense and sparse outputs, as fp64) with the oracle's design
    weights for the same probe positions.  Both fits run in fp64 on identical
    inputs; only the eigensolver and the order of additions differ."""
    from oracle import fit_residual

    banner(name, "fit")
    c = CASES[name]
    q, k, v = dev_inputs(name)
    ql, kl = oracle_labels(name)
    res = sp.sparsepr_probe_fit(q, k, v, lib_cfg(name), ql, kl)
    torch.cuda.synchronize()
    oc = c.oracle_cfg()
    for h, r in enumerate(oracle_result(name)):
        od = res["o_dense"][h].double().cpu().numpy()
        os_ = res["o_sparse"][h].double().cpu().numpy()
        f = fit_residual(od - os_, os_, r["probe_weights"], oc.residual_rank, oc.ridge_lambda, oc.rank_cut,
                         relative=oc.ridge_mode == "relative", rank_cap=oc.rank_cap,
                         svd_weighted=oc.svd_weighted)
        rk = int(res["rank"][h])
        assert rk == f["rank"]
        wm = res["W"][h].double().cpu().numpy()[:, :rk]
        vm = res["V"][h].double().cpu().numpy()[:, :rk]
        b_gpu = res["b"][h].double().cpu().numpy()
        bmat = wm @ vm.T
        eb = rel_frob(bmat, f["B"]) if rk else float(np.abs(bmat).max())
        ev = rel_frob(b_gpu, f["b"]) if rk else float(np.abs(b_gpu).max())
        print(f"  head {h}: rank {rk}, B rel err {eb:.2e}, b rel err {ev:.2e}, |B|_2 {np.linalg.norm(f['B'], 2):.3g}")
        # fp32 storage of W, V and b bounds the agreement
        assert eb <= 1e-5 and ev <= 1e-5


@pytest.mark.parametrize("name", ALL)
def test_corrected_output_with_oracle_partition(name):
    banner(name, "attention_with_partition")
    c = CASES[name]
    q, k, v = dev_inputs(name)
    ql, kl = oracle_labels(name)
    out = sp.sparsepr_attention_with_partition(q, k, v, lib_cfg(name), ql, kl)
    torch.cuda.synchronize()
    ma, rf = tolerances(c.dtype)
    for h, r in enumerate(oracle_result(name)):
        got = out[0, h].double().cpu().numpy()
        tok = r["perm_q"][r["probes"]]
        # probe rows carry their exact dense output
        assert max_abs(got[tok], r["dense"][tok]) <= ma
        gain = np.linalg.norm(np.eye(c.d) + r["fit"]["B"], 2)
        print(f"  head {h}: corrected max-abs {max_abs(got, r['out']):.3e} rel {rel_frob(got, r['out']):.3e} "
              f"gain {gain:.1f}")
        ma_h, rf_h = ma, rf
        if c.dtype == "fp32":
            # no stated fp32 bound: fp32 errors of x are amplified by the gain ||I + B||_2
            ma_h, rf_h = ma * gain, rf * gain
        else:
            # the bf16 bound is for outputs on the scale of attention (|o| <= max|v|);
            # a weakly regularised fit can push corrected outputs past it, and the
            # bf16 rounding of the stored output grows with the magnitude
            ma_h = ma * max(1.0, np.abs(r["out"]).max() / np.abs(r["dense"]).max())
        assert max_abs(got, r["out"]) <= ma_h
        assert rel_frob(got, r["out"]) <= rf_h


@pytest.mark.parametrize("name", ALL)
def test_end_to_end_partition_agreement_and_error(name):
    """k-means agreement >= 99% and corrected error <= 1.1x the oracle's.

    Both are unconditional: the GPU's key and query labels against the
    oracle's own partition of the same inputs, and the GPU's corrected error
    against dense attention against the oracle's.  Both sides take every
    k-means decision in fp64 (the GPU re-decides in fp64 each point its fast
    path cannot separate), from an fp64 metric and eigensolve.  The
    conditional figures (each k-means against the oracle's k-means on the
    inputs the GPU's k-means got) are printed beside them.
    """
    banner(name, "attention")
    c = CASES[name]
    q, k, v = dev_inputs(name)
    cfg = lib_cfg(name)
    ql, kl = sp.sparsepr_partition(q, k, v, cfg)
    out, st = sp.sparsepr_attention(q, k, v, cfg, with_stats=True)
    mk = None
    if c.mode == "response_coupled":
        _, mk, _, _ = sp.sparsepr_key_metric(q, k, v, cfg)
    torch.cuda.synchronize()
    stats = sp.stats_to_dicts(st)
    for h, r in enumerate(oracle_result(name)):
        kl_h, ql_h = kl[h].cpu().numpy(), ql[h].cpu().numpy()
        print(f"  head {h}: {stats[h]['kmeans_redecided']} k-means assignments re-decided in fp64 over "
              f"{2 * cfg.kmeans_iters} Lloyd steps of {c.n} points")
        # every case's ridge system is positive definite: no head drops its correction
        assert stats[h]["fit_fallback"] == 0
        if c.mode == "response_coupled":
            ref_k = oracle_key_labels_from_metric(name, h, mk[h].cpu().numpy())
            ref_q = oracle_query_labels_given_keys(name, h, kl_h)
        else:
            ref_k, ref_q = r["kv_labels"], r["q_labels"]
        cond_k = (kl_h == ref_k).mean()
        cond_q = (ql_h == ref_q).mean()
        agree_k = (kl_h == r["kv_labels"]).mean()
        agree_q = (ql_h == r["q_labels"]).mean()
        err_gpu = rel_frob(out[0, h].double().cpu().numpy(), r["dense"])
        err_ora = rel_frob(r["out"], r["dense"])
        err_cond = rel_frob(oracle_out_given_partition(name, h, ql_h, kl_h), r["dense"])
        print(f"  head {h}: agreement K {agree_k:.4f} Q {agree_q:.4f} (conditional K {cond_k:.4f} Q {cond_q:.4f}); "
              f"err vs dense gpu {err_gpu:.4f} oracle {err_ora:.4f} oracle on the GPU partition {err_cond:.4f}")
        assert agree_k >= 0.99 and agree_q >= 0.99
        assert err_gpu <= 1.1 * err_ora
        assert err_gpu <= 1.1 * err_cond


@pytest.mark.parametrize("name", ["c1_tiny_fp32", "bf16_d64", "bf16_d128"])
def test_dense_attention_matches_oracle(name):
    banner(name, "dense_attention")
    c = CASES[name]
    q, k, v = dev_inputs(name)
    out = sp.sparsepr_dense_attention(q, k, v)
    torch.cuda.synchronize()
    ma, rf = tolerances(c.dtype)
    for h, r in enumerate(oracle_result(name)):
        got = out[0, h].double().cpu().numpy()
        assert max_abs(got, r["dense"]) <= ma and rel_frob(got, r["dense"]) <= rf


@pytest.mark.parametrize("name", ["bf16_d64", "c1_tiny_fp32"])
def test_two_runs_are_bitwise_identical(name):
    banner(name, "determinism")
    q, k, v = dev_inputs(name)
    cfg = lib_cfg(name)
    a = sp.sparsepr_attention(q, k, v, cfg)
    b = sp.sparsepr_attention(q, k, v, cfg)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_density_is_dense_attention():
    name = "bf16_d64"
    banner(name, "full density")
    c = CASES[name]
    q, k, v = dev_inputs(name)
    cfg = lib_cfg(name)
    cfg.density = 1.0
    out = sp.sparsepr_attention(q, k, v, cfg)
    dense = sp.sparsepr_dense_attention(q, k, v)
    torch.cuda.synchronize()
    ma, rf = tolerances(c.dtype)
    for h, r in enumerate(oracle_result(name)):
        got = out[0, h].double().cpu().numpy()
        assert max_abs(got, r["dense"]) <= ma and rel_frob(got, r["dense"]) <= rf


def test_main_call_equals_profiled_call():
    """With three heads the main call's output and statistics equal, bit for
    bit, those of the profiling entry point (the same kernels with timing
    events between the stages): every head's query sample is seeded by its
    own head index and its tensors are addressed at its own head offset."""
    from synth.generator import make_video_qkv

    c = case("bf16_d64")
    x = make_video_qkv(c.frames, c.height, c.width, 3, c.d, c.dtype, c.seed, [c.f90] * 3)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    cfg = sp.make_config(c.n, c.d, **c.lib_cfg_kwargs())
    ws = sp.Workspace()
    out_two, st_two = sp.sparsepr_attention(q, k, v, cfg, workspace=ws, with_stats=True)
    out_one, _, st_one = sp.sparsepr_attention_profile(q, k, v, cfg, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_two.view(torch.int16), out_one.view(torch.int16))
    assert torch.equal(st_two, st_one)
