"""Pins of the oracle's fit and coordinate variants (CPU only).

* weighted subspace: the right singular vectors of D^(1/2) R are the leading
  eigenvectors of R^T D R, computed here by a symmetric eigensolver on the
  weighted Gram (a route that shares nothing with the SVD call), and a planted
  heavy-weight direction leads;
* rank cap: the rank is floor(rank_cap * M) when that is the smallest bound,
  and a fit capped below M no longer reproduces the probe residuals exactly;
* centred query coordinates: rows sum to zero, a vector added to every centre
  leaves them unchanged, and their squared distances are the quadratic form of
  the centred centre matrix (the metric the GPU folds into d-space).
"""

import numpy as np

from oracle import fit_residual, query_coordinates


def _align(a, b):
    """Largest principal-angle cosine deficit between two column spans."""
    qa, _ = np.linalg.qr(a)
    qb, _ = np.linalg.qr(b)
    return 1.0 - np.linalg.svd(qa.T @ qb, compute_uv=False).min()


def test_weighted_subspace_is_the_weighted_gram_eigenspace():
    rng = np.random.default_rng(2)
    m, d, r = 40, 24, 6
    res = rng.normal(size=(m, d)) @ np.diag(np.linspace(2.0, 0.2, d))
    x = rng.normal(size=(m, d))
    w = rng.uniform(0.1, 3.0, size=m)
    f = fit_residual(res, x, w, r, 0.1, svd_weighted=True)
    gram = res.T @ (w[:, None] * res)
    evals, evecs = np.linalg.eigh(gram)
    top = evecs[:, ::-1][:, :r]
    assert f["rank"] == r
    assert _align(f["V"], top) < 1e-10
    assert np.allclose(f["sigma"][:r], np.sqrt(evals[::-1][:r]), rtol=1e-10)
    # the unweighted subspace is a different one on these data
    g = fit_residual(res, x, w, r, 0.1, svd_weighted=False)
    assert _align(g["V"], top) > 1e-4


def test_weighted_subspace_follows_heavy_rows_and_uniform_weights_change_nothing():
    rng = np.random.default_rng(3)
    m, d = 30, 16
    res = 0.05 * rng.normal(size=(m, d))
    e = np.zeros(d)
    e[5] = 1.0
    f_dir = np.zeros(d)
    f_dir[9] = 1.0
    res[:3] += 4.0 * e  # three heavy rows along e
    res[3:] += 3.0 * rng.normal(size=(m - 3, 1)) * f_dir  # the bulk along f
    w = np.ones(m)
    w[:3] = 50.0
    f = fit_residual(res, res * 0.1, w, 1, 0.1, svd_weighted=True)
    g = fit_residual(res, res * 0.1, w, 1, 0.1, svd_weighted=False)
    assert abs(f["V"][5, 0]) > 0.99 and abs(g["V"][9, 0]) > 0.99
    u = fit_residual(res, res * 0.1, np.full(m, 2.5), 4, 0.1, svd_weighted=True)
    v = fit_residual(res, res * 0.1, np.full(m, 2.5), 4, 0.1, svd_weighted=False)
    assert _align(u["V"], v["V"]) < 1e-10


def test_rank_cap_bounds_the_rank_and_stops_interpolation():
    rng = np.random.default_rng(4)
    m, d = 16, 64
    res = rng.normal(size=(m, d))
    x = rng.normal(size=(m, d))
    w = np.ones(m)
    full = fit_residual(res, x, w, 32, 1e-9, relative=False)
    capped = fit_residual(res, x, w, 32, 1e-9, relative=False, rank_cap=0.5)
    assert full["rank"] == m and capped["rank"] == m // 2
    assert fit_residual(res, x, w, 5, 1e-9, rank_cap=0.5)["rank"] == 5
    assert fit_residual(res, x, w, 32, 1e-9, rank_cap=0.3)["rank"] == 4  # floor(0.3 * 16)
    # rank M plus an intercept reproduces the M probe residuals (d >= M, tiny lambda)
    pred_full = full["b"] + x @ full["B"]
    assert np.abs(pred_full - res).max() < 1e-5 * np.abs(res).max()
    pred_cap = capped["b"] + x @ capped["B"]
    assert np.abs(pred_cap - res).max() > 1e-2 * np.abs(res).max()


def test_centred_query_coordinates():
    rng = np.random.default_rng(5)
    q = rng.normal(size=(50, 16))
    c = rng.normal(size=(9, 16))
    s = 0.25
    u = query_coordinates(q, c, s, centred=True)
    assert np.abs(u.sum(axis=1)).max() < 1e-12
    t = rng.normal(size=16)
    assert np.allclose(query_coordinates(q, c + t, s, centred=True), u, atol=1e-12)
    assert not np.allclose(query_coordinates(q, c + t, s), query_coordinates(q, c, s))
    ct = c - c.mean(axis=0)
    m_q = s * s * ct.T @ ct
    i, j = 3, 17
    dq = q[i] - q[j]
    assert np.isclose(((u[i] - u[j]) ** 2).sum(), dq @ m_q @ dq, rtol=1e-12)
