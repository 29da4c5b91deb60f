"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks one oracle function against a published value, a closed form,
an invariant, a brute-force computation written differently, or a special case
that reduces to a library routine, chosen so that a plausible slip (a dropped
term, a wrong sign or index, a transposed operand) fails.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
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
    sparsepr_head,
    splitmix64,
)
from oracle.sparsepr_oracle import strided_seeds
from synth import make_video_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _small_inputs(n_frames=2, hgt=8, wid=8, d=32, seed=3, f90=0.08):
    x = make_video_qkv(n_frames, hgt, wid, 1, d, "fp32", seed, [f90])
    return (x["q"][0, 0].double().numpy(), x["k"][0, 0].double().numpy(),
            x["v"][0, 0].double().numpy())


# --------------------------------------------------------------------------- a1
def test_splitmix64_published_outputs():
    # First three outputs of the published splitmix64 reference generator for state 0.
    g = splitmix64(0)
    assert [next(g) for _ in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                           0x06C45D188009454F]


def test_sample_is_distinct_sorted_and_uniform():
    n, ms = 97, 20
    hits = np.zeros(n)
    for seed in range(400):
        s = sample_queries(n, ms, seed, bh=seed % 5)
        assert len(s) == ms and len(set(s.tolist())) == ms
        assert np.all(np.diff(s) > 0) and s.min() >= 0 and s.max() < n
        hits[s] += 1
    # inclusion probability of every row is ms/n; chi-square with n-1 dof
    exp = 400 * ms / n
    chi2 = ((hits - exp) ** 2 / exp).sum()
    assert chi2 < 160, chi2
    # full-length draw is a permutation
    assert np.array_equal(sample_queries(50, 50, 7, 0), np.arange(50))


def test_key_coordinates_reproduce_response_profile_distance():
    # Closed form: with every eigenvector kept, squared coordinate distance is the
    # mean squared logit difference under the sampled queries.
    q, k, _ = _small_inputs()
    s = 1.0 / math.sqrt(q.shape[1])
    smp = sample_queries(q.shape[0], 40, 11, 0)
    mk = key_metric(q, smp)
    assert np.allclose(mk, mk.T)
    z, lam, vec = key_coordinates(k, mk, q.shape[1], s)
    assert np.all(np.diff(lam) <= 1e-12)
    assert np.allclose(mk @ vec, vec * lam[None, :], atol=1e-10 * np.abs(mk).max())
    rng = np.random.default_rng(0)
    for _ in range(20):
        i, j = rng.integers(0, k.shape[0], 2)
        prof = s * (q[smp] @ (k[i] - k[j]))
        assert np.isclose(((z[i] - z[j]) ** 2).sum(), (prof ** 2).mean(), rtol=1e-9)


def test_key_coordinates_truncation_keeps_leading_directions():
    q, k, _ = _small_inputs()
    s = 0.25
    smp = sample_queries(q.shape[0], 64, 1, 0)
    mk = key_metric(q, smp)
    z_full, lam, _ = key_coordinates(k, mk, q.shape[1], s)
    z8, lam8, _ = key_coordinates(k, mk, 8, s)
    assert np.allclose(lam8, lam[:8])
    # truncated squared norms never exceed full ones and capture the top energy
    assert np.all((z8 ** 2).sum(1) <= (z_full ** 2).sum(1) + 1e-9)
    assert np.allclose(np.abs(z8), np.abs(z_full[:, :8]), rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------------------- a4/a8
def _planted(n_per=40, g=5, dim=6, seed=0, spread=30.0):
    rng = np.random.default_rng(seed)
    centres = rng.normal(0, spread, size=(g, dim))
    lab = np.repeat(np.arange(g), n_per)
    rng.shuffle(lab)
    return centres[lab] + rng.normal(0, 1, size=(len(lab), dim)), lab


def test_kmeans_planted_clusters_are_recovered():
    x, truth = _planted()
    # seeds are strided: make sure every planted cluster owns a seed by sorting
    order = np.argsort(truth, kind="stable")
    x, truth = x[order], truth[order]
    lab, _ = kmeans(x, 5, 10)
    for c in range(5):
        assert len(set(lab[truth == c].tolist())) == 1
    assert len(set(lab.tolist())) == 5


def test_kmeans_lloyd_objective_never_increases_and_labels_are_nearest():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(300, 4)) * np.array([3, 1, 1, 0.5])
    prev = np.inf
    for t in range(1, 8):
        lab, c = kmeans(x, 7, t)
        # brute force: recompute the centres that produced `lab` and the objective
        cprev = x[strided_seeds(300, 7)].copy()
        for _ in range(t - 1):
            l2 = np.array([min(range(7), key=lambda j: float(((xi - cprev[j]) ** 2).sum())) for xi in x])
            for j in range(7):
                if np.any(l2 == j):
                    cprev[j] = x[l2 == j].mean(0)
        brute = np.array([min(range(7), key=lambda j: float(((xi - cprev[j]) ** 2).sum())) for xi in x])
        assert np.array_equal(brute, lab)  # fp64 decisions: exact up to fp64 near-ties (none here)
        obj = sum(float(((x[i] - cprev[lab[i]]) ** 2).sum()) for i in range(300))
        assert obj <= prev + 1e-9
        prev = obj


def test_kmeans_is_rotation_invariant():
    x, _ = _planted(n_per=30, g=4, dim=5, seed=2, spread=10.0)
    rot, _ = np.linalg.qr(np.random.default_rng(3).normal(size=(5, 5)))
    la, _ = kmeans(x, 4, 10)
    lb, _ = kmeans(x @ rot, 4, 10)
    assert np.array_equal(la, lb)


def test_kmeans_empty_cluster_keeps_its_centre():
    # two identical seeds: the second never wins (ties go to the lowest index)
    x = np.array([[0.0], [0.0], [10.0], [10.0]])
    lab, c = kmeans(x, 2, 3)
    assert np.array_equal(lab, [0, 0, 0, 0]) or np.array_equal(lab, [0, 0, 1, 1])
    x = np.array([[5.0], [5.0], [5.0], [5.0]])
    lab, c = kmeans(x, 3, 4)
    assert np.all(lab == 0) and np.allclose(c, 5.0)


# --------------------------------------------------------------------------- a5
def test_grouping_is_a_stable_bijection():
    rng = np.random.default_rng(1)
    lab = rng.integers(0, 9, size=500)
    lab[lab == 4] = 3  # one empty group
    perm, cnt, off = group_by_labels(lab, 9)
    assert np.array_equal(np.sort(perm), np.arange(500))
    assert cnt[4] == 0 and off[-1] == 500
    assert np.array_equal(off[1:] - off[:-1], cnt)
    for g in range(9):
        seg = perm[off[g]:off[g + 1]]
        assert np.all(lab[seg] == g) and np.all(np.diff(seg) > 0)


def test_group_means_match_plain_means():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(200, 3))
    lab = rng.integers(0, 5, size=200)
    perm, cnt, off = group_by_labels(lab, 5)
    gm = group_means(x, perm, off)
    for g in range(5):
        assert np.allclose(gm[g], x[lab == g].mean(0), rtol=1e-13)


# --------------------------------------------------------------------------- a7
def test_query_coordinates_give_the_folded_metric():
    rng = np.random.default_rng(6)
    q = rng.normal(size=(30, 8))
    cbar = rng.normal(size=(5, 8))
    s = 0.3
    u = query_coordinates(q, cbar, s)
    mq = s * s * cbar.T @ cbar
    for i in range(10):
        for j in range(10):
            dq = q[i] - q[j]
            assert np.isclose(((u[i] - u[j]) ** 2).sum(), dq @ mq @ dq, rtol=1e-10, atol=1e-12)
    # coordinate h of query i is the logit it would give a key equal to cbar_h
    assert np.isclose(u[3, 2], s * float(np.dot(q[3], cbar[2])))


# --------------------------------------------------------------------------- a10
def _route_case(seed=0, gq=6, gk=7, d=5, n=None, density=0.3, m=0):
    rng = np.random.default_rng(seed)
    nq = rng.integers(1, 12, size=gq)
    nk = rng.integers(1, 12, size=gk)
    nq[1] = 0
    nk[2] = 0
    n = n or int(max(nq.sum(), nk.sum()))
    # route() takes N for the budget; make both sides sum to N by padding group 0
    nq[0] += n - nq.sum()
    nk[0] += n - nk.sum()
    qbar = rng.normal(size=(gq, d))
    cbar = rng.normal(size=(gk, d))
    return qbar, nq, cbar, nk, n


def test_router_prefix_budget_and_mandatory_cells():
    for seed in range(6):
        qbar, nq, cbar, nk, n = _route_case(seed)
        s = 0.7
        for rho in (0.05, 0.2, 0.35, 0.6, 0.9):
            rt = route(qbar, nq, cbar, nk, s, rho, n, 0)
            g_ = rt["granted"]
            cost = np.outer(nq, nk)
            assert not g_[nq == 0].any() and not g_[:, nk == 0].any()
            # brute-force logits, log-probabilities and best cells written out directly
            for g in np.nonzero(nq > 0)[0]:
                logit = np.array([s * sum(qbar[g, t] * cbar[h, t] for t in range(qbar.shape[1]))
                                  for h in range(len(nk))])
                ok = nk > 0
                best = int(np.nonzero(ok)[0][np.argmax(logit[ok])])
                assert g_[g, best]
                prob = nk[ok] * np.exp(logit[ok] - logit[ok].max())
                prob = prob / prob.sum()
                assert np.allclose(np.exp(rt["key"][g, ok]) * nk[ok], prob, rtol=1e-12)
            # every optional granted cell out-ranks every optional non-granted cell
            mand = np.zeros_like(g_)
            mand[np.arange(len(nq))[nq > 0], rt["mandatory"][nq > 0]] = True
            opt_g = g_ & ~mand
            opt_n = ~g_ & (nq[:, None] > 0) & (nk[None, :] > 0)
            if opt_g.any() and opt_n.any():
                assert rt["key"][opt_g].min() >= rt["key"][opt_n].max()
            total = int(cost[g_].sum())
            if total > rt["budget"]:
                assert not opt_g.any()  # only mandatory cells may exceed the budget
            elif opt_n.any():
                # the best-ranked refused cell would not have fit
                cand = [(-rt["key"][a, b], a, b) for a, b in zip(*np.nonzero(opt_n))]
                _, a, b = min(cand)
                assert total + cost[a, b] > rt["budget"]


def test_alpha_router_is_a_minimum_cover_found_by_brute_force():
    """For every query group, no smaller set of key groups that keeps the
    mandatory best cell retains at least alpha of the estimated mass; the
    granted set retains at least alpha (or takes every key group)."""
    import itertools

    for seed in range(5):
        qbar, nq, cbar, nk, n = _route_case(seed, gq=5, gk=6)
        s = 0.8
        for alpha in (0.3, 0.6, 0.85, 0.97):
            rt = route_alpha(qbar, nq, cbar, nk, s, alpha, n, 0)
            g_ = rt["granted"]
            assert not g_[nq == 0].any() and not g_[:, nk == 0].any()
            ok = np.nonzero(nk > 0)[0]
            for g in np.nonzero(nq > 0)[0]:
                # estimated shares written out from the logits directly
                logit = np.array([s * sum(qbar[g, t] * cbar[h, t] for t in range(qbar.shape[1])) for h in ok])
                w = nk[ok] * np.exp(logit - logit.max())
                share = dict(zip(ok, w / w.sum()))
                best = int(ok[np.argmax(logit)])
                assert g_[g, best]
                got = [int(h) for h in np.nonzero(g_[g])[0]]
                kept = sum(share[h] for h in got)
                a = float(np.float32(alpha))
                assert kept >= a - 1e-12 or len(got) == len(ok)
                others = [int(h) for h in ok if h != best]
                smallest = len(ok)
                for r in range(len(others) + 1):
                    if any(share[best] + sum(share[h] for h in c) >= a + 1e-12 for c in itertools.combinations(others, r)):
                        smallest = r + 1
                        break
                assert len(got) <= smallest


def test_alpha_router_mass_rows_nesting_and_limits():
    qbar, nq, cbar, nk, n = _route_case(4, gq=8, gk=8)
    ok_q, ok_k = nq > 0, nk > 0
    rt = route_alpha(qbar, nq, cbar, nk, 0.6, 0.5, n, 0)
    # the estimated shares of every non-empty query group sum to one
    assert np.allclose(rt["mass"][ok_q].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    prev = None
    for alpha in np.linspace(0.05, 0.99, 20):
        g_ = route_alpha(qbar, nq, cbar, nk, 0.6, alpha, n, 0)["granted"]
        if prev is not None:
            assert (g_ | ~prev).all()  # granted at a smaller alpha stays granted
        prev = g_
    # a vanishing target keeps only the best cells, a full one takes everything
    tiny = route_alpha(qbar, nq, cbar, nk, 0.6, 1e-9, n, 0)
    assert tiny["granted"].sum() == ok_q.sum()
    assert all(tiny["granted"][g, tiny["mandatory"][g]] for g in np.nonzero(ok_q)[0])
    full = route_alpha(qbar, nq, cbar, nk, 0.6, 1.0, n, 0)["granted"]
    assert (full == (ok_q[:, None] & ok_k[None, :])).all()


def test_alpha_router_runs_through_the_full_call():
    """The per-head call with the alpha router: the routed cells cover alpha
    of every query group's estimated mass, and the corrected output is
    closer to dense attention than the uncorrected sparse output."""
    x = make_video_qkv(2, 8, 16, 1, 32, "fp32", 5, [0.08])
    q, k, v = (x[t][0, 0].double().numpy() for t in ("q", "k", "v"))
    cfg = OracleConfig(probe_rows=16, n_kv_groups=8, n_q_groups=8, residual_rank=4, router="alpha", alpha=0.8)
    r = sparsepr_head(q, k, v, cfg, bh=0)
    rt = r["route"]
    kept = (rt["mass"] * rt["granted"]).sum(axis=1)
    assert (kept[rt["mandatory"] >= 0] >= np.float32(0.8) - 1e-12).all()
    dense = dense_attention(q, k, v, r["scale"])
    err = lambda o: np.linalg.norm(o - dense) / np.linalg.norm(dense)
    assert err(r["out"]) < err(r["hard_drop"])


def test_router_is_nested_in_density_and_full_at_one():
    qbar, nq, cbar, nk, n = _route_case(3, gq=8, gk=8)
    prev = None
    for rho in np.linspace(0.02, 0.98, 25):
        g_ = route(qbar, nq, cbar, nk, 0.5, rho, n, 0)["granted"]
        if prev is not None:
            assert np.all(g_ >= prev)
        prev = g_
    full = route(qbar, nq, cbar, nk, 0.5, 1.0, n, 0)
    assert np.array_equal(full["granted"], (nq[:, None] > 0) & (nk[None, :] > 0))
    assert full["rho_route"] == 1.0


def test_budget_counts_probe_rows():
    # executed density = routed cells + exact probe rows (pages' accounting)
    assert budget_pairs(0.25, 1000, 64) == 250000 - 64000
    const = json.load(open(os.path.join(GOLDEN, "pages_constants.json")))
    m = const["probe_rows_per_head"]["value"]
    lo, hi = const["probe_share_percent_range"]["value"]
    # a probe row costs M*N of N^2 pairs: share = M/N; the printed range maps to N
    n_lo, n_hi = math.ceil(m / (hi / 100)), math.floor(m / (lo / 100))
    for n in (n_lo, n_hi):
        qbar, nq, cbar, nk, _ = _route_case(1, n=n)
        rt = route(qbar, nq, cbar, nk, 0.5, 0.25, n, m)
        share = 100 * (rt["rho_exec"] - rt["rho_route"])
        assert lo - 5e-4 <= share <= hi + 5e-4


# --------------------------------------------------------------------------- a11
def test_probe_allocation_hand_example():
    # sizes [5, 0, 3, 1], M = 6: 3 non-empty groups get 2 each, group 3 is capped at 1
    # and its spare probe wraps to group 0; positions floor((t + 1/2) n_g / m_g).
    off = np.array([0, 5, 5, 8, 9])
    pos, w, mg = select_probes(off, 6)
    assert mg.tolist() == [3, 0, 2, 1]
    assert pos.tolist() == [0, 2, 4, 5, 7, 8]
    raw = np.array([5 / 3] * 3 + [3 / 2] * 2 + [1.0])
    assert np.allclose(w, raw * 6 / raw.sum())
    # fewer probes than groups: spread over the group list
    off = np.array([0, 2, 4, 6, 8, 10, 12])
    pos, w, mg = select_probes(off, 2)
    assert mg.tolist() == [0, 1, 0, 0, 1, 0] and pos.tolist() == [3, 9]


def test_probe_weights_are_design_weights():
    rng = np.random.default_rng(2)
    sizes = rng.integers(0, 40, size=30)
    off = np.concatenate([[0], np.cumsum(sizes)])
    for m in (7, 30, 64, 200):
        pos, w, mg = select_probes(off, m)
        assert len(pos) == m == len(set(pos.tolist()))
        assert np.isclose(w.sum(), m)
        g_of = np.searchsorted(off, pos, side="right") - 1
        tot = np.array([w[g_of == g].sum() for g in range(30)])
        probed = mg > 0
        ratio = tot[probed] / sizes[probed]
        assert np.allclose(ratio, ratio[0])


# --------------------------------------------------------------------------- a12/a13
def test_sparse_attention_equals_masked_dense_softmax():
    q, k, v = _small_inputs(d=16, seed=8)
    n = q.shape[0]
    s = 0.25
    rng = np.random.default_rng(9)
    ql = rng.integers(0, 5, size=n)
    kl = rng.integers(0, 6, size=n)
    granted = rng.random((5, 6)) < 0.4
    granted[np.arange(5), rng.integers(0, 6, size=5)] = True
    perm_q, _, off_q = group_by_labels(ql, 5)
    perm_k, _, off_k = group_by_labels(kl, 6)
    osp = sparse_attention(q[perm_q], k[perm_k], v[perm_k], granted, off_q, off_k, s)
    out = np.empty_like(osp)
    out[perm_q] = osp
    # brute force in original token order with an explicit N x N mask
    mask = granted[ql][:, kl]
    logit = np.where(mask, s * q @ k.T, -np.inf)
    p = np.exp(logit - logit.max(1, keepdims=True))
    ref = (p / p.sum(1, keepdims=True)) @ v
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_dense_attention_matches_torch_sdpa_fp64():
    q, k, v = _small_inputs(d=16, seed=10)
    s = 0.25
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=s)[0]
    assert np.allclose(dense_attention(q, k, v, s), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_residual_identity_per_row():
    # R_i = omega_i (O_omit,i - O_sp,i), omega_i = dense mass outside the support
    q, k, v = _small_inputs(d=16, seed=12)
    n = q.shape[0]
    s = 0.3
    rng = np.random.default_rng(13)
    support = rng.random((n, n)) < 0.3
    support[np.arange(n), np.arange(n)] = True
    logit = s * q @ k.T
    p = np.exp(logit - logit.max(1, keepdims=True))
    p = p / p.sum(1, keepdims=True)
    dense = dense_attention(q, k, v, s)
    for i in range(0, n, 7):
        keep = np.nonzero(support[i])[0]
        drop = np.nonzero(~support[i])[0]
        o_sp = dense_attention(q[i:i + 1], k[keep], v[keep], s)[0]
        o_om = dense_attention(q[i:i + 1], k[drop], v[drop], s)[0]
        omega = p[i, drop].sum()
        assert np.allclose(dense[i] - o_sp, omega * (o_om - o_sp), rtol=1e-10, atol=1e-13)


# --------------------------------------------------------------------------- a14
def test_fit_reduces_to_least_squares():
    rng = np.random.default_rng(14)
    m, d = 40, 5
    x = rng.normal(size=(m, d))
    r = rng.normal(size=(m, d))
    f = fit_residual(r, x, np.ones(m), rank=d, lam=1e-13)
    assert f["rank"] == d
    xa = np.hstack([x, np.ones((m, 1))])
    coef, *_ = np.linalg.lstsq(xa, r, rcond=None)
    assert np.allclose(f["B"], coef[:d], atol=1e-9)
    assert np.allclose(f["b"], coef[d], atol=1e-9)


def test_fit_recovers_planted_affine_map_in_subspace():
    rng = np.random.default_rng(15)
    m, d, r = 80, 12, 3
    vstar, _ = np.linalg.qr(rng.normal(size=(d, r)))
    wstar = rng.normal(size=(d, r))
    bstar = rng.normal(size=r) @ vstar.T
    bmat = wstar @ vstar.T
    x = rng.normal(size=(m + 50, d))
    resid = bstar + x @ bmat
    w = rng.uniform(0.5, 2.0, size=m)
    f = fit_residual(resid[:m], x[:m], w, rank=8, lam=1e-12)
    assert f["rank"] == r  # numerical-rank cut removes the empty directions
    assert np.allclose(f["B"], bmat, atol=1e-7) and np.allclose(f["b"], bstar, atol=1e-7)
    pred = f["b"] + x[m:] @ f["B"]
    assert np.allclose(pred, resid[m:], atol=1e-7)


def test_relative_ridge_is_scale_free():
    # scaling the sparse outputs by a leaves the predicted residuals unchanged:
    # the relative penalty grows with a^2 while W shrinks by 1/a
    rng = np.random.default_rng(21)
    m, d = 30, 12
    x = rng.normal(size=(m + 10, d))
    r = rng.normal(size=(m, d))
    w = rng.uniform(0.5, 1.5, size=m)
    f1 = fit_residual(r, x[:m], w, 4, 0.7, relative=True)
    f2 = fit_residual(r, 7.0 * x[:m], w, 4, 0.7, relative=True)
    assert np.allclose(f1["b"] + x[m:] @ f1["B"], f2["b"] + 7.0 * x[m:] @ f2["B"], atol=1e-10)
    # the absolute penalty is not scale free
    g1 = fit_residual(r, x[:m], w, 4, 0.7)
    g2 = fit_residual(r, 7.0 * x[:m], w, 4, 0.7)
    assert not np.allclose(g1["b"] + x[m:] @ g1["B"], g2["b"] + 7.0 * x[m:] @ g2["B"], atol=1e-6)
    # the relative penalty equals lam times the mean eigenvalue of Xc^T D Xc
    xc = x[:m] - (w[:, None] * x[:m]).sum(0) / w.sum()
    lam_eff = 0.7 * np.linalg.eigvalsh(xc.T @ (w[:, None] * xc)).mean()
    g3 = fit_residual(r, x[:m], w, 4, lam_eff)
    assert np.allclose(g3["B"], f1["B"], atol=1e-12) and np.allclose(g3["b"], f1["b"], atol=1e-12)


def test_fit_degenerate_cases():
    rng = np.random.default_rng(16)
    x = rng.normal(size=(20, 6))
    f0 = fit_residual(np.zeros((20, 6)), x, np.ones(20), 4, 1e-3)
    assert f0["rank"] == 0 and not f0["B"].any() and not f0["b"].any()
    r = rng.normal(size=(20, 6))
    w = rng.uniform(0.1, 1, size=20)
    big = fit_residual(r, x, w, 3, 1e12)
    assert np.abs(big["B"]).max() < 1e-9
    v = big["V"]
    assert np.allclose(big["b"], ((w[:, None] * r).sum(0) / w.sum()) @ v @ v.T, atol=1e-9)


# --------------------------------------------------------------------------- end to end
def _cfg(**kw):
    base = dict(density=0.25, probe_rows=16, n_kv_groups=6, n_q_groups=5, residual_rank=4,
                kmeans_iters=5, n_sample_q=64, key_coord_rank=8)
    base.update(kw)
    return OracleConfig(**base)


def test_full_density_is_dense_attention():
    q, k, v = _small_inputs(d=16, seed=17)
    res = sparsepr_head(q, k, v, _cfg(density=1.0))
    dense = dense_attention(q, k, v, res["scale"])
    assert np.allclose(res["out"], dense, rtol=1e-12, atol=1e-12)
    assert res["fit"]["rank"] == 0


def test_call_accounting_and_probe_rows_exact():
    q, k, v = _small_inputs(d=16, seed=18)
    n = q.shape[0]
    for mode in ("response_coupled", "independent"):
        res = sparsepr_head(q, k, v, _cfg(density=0.3, partition_mode=mode))
        rt = res["route"]
        assert rt["rho_exec"] <= 0.3 + 1e-12 or rt["over_budget"]
        assert np.isclose(rt["rho_exec"] - rt["rho_route"], 16 / n)
        dense = dense_attention(q, k, v, res["scale"])
        tok = res["perm_q"][res["probes"]]
        assert np.allclose(res["out"][tok], dense[tok], rtol=1e-12)
        # hard-drop rows equal their masked softmax; corrected rows differ only by b + xB
        hd = res["hard_drop"]
        other = np.setdiff1d(np.arange(n), tok)
        f = res["fit"]
        assert np.allclose(res["out"][other], hd[other] + f["b"] + hd[other] @ f["B"])
