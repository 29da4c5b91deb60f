"""Pins of the oracle's weighted ridge fit against formulations written apart
from it (CPU only).

The fit models the probe residuals as an affine function of the sparse
outputs, weighted by the probes' design weights and ridge-regularised, inside
the leading right singular subspace of the residuals (gist.science "Resumen
Técnico", 2.B; ai-feeds digest, method / key modules: weighted affine fit).
Each pin solves the same problem by another route:

* weighted least squares (lambda -> 0, full subspace): rows of [X, 1] and R
  scaled by sqrt(w), solved by ``numpy.linalg.lstsq``;
* weighted ridge with an unpenalised intercept: the augmented system whose
  extra rows sqrt(lambda) I penalise the slope only, again by ``lstsq``, with
  no centring anywhere;
* the subspace: the top-r eigenprojector of R^T R by ``numpy.linalg.eigh``.

Mutants of the fit (an unweighted Gram, weights on X only, sqrt(w) in the
Gram) are built from the oracle's own source and must fail these checks.
"""

import inspect
import textwrap

import numpy as np

import oracle.sparsepr_oracle as O
from oracle import fit_residual


def _problem(seed, m=48, d=7, noise=0.3):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(m, d)) * rng.uniform(0.2, 3.0, size=d)
    bmat = rng.normal(size=(d, d))
    r = 0.5 + x @ bmat + noise * rng.normal(size=(m, d)) * (1 + 3 * (np.arange(m) % 5 == 0))[:, None]
    # strongly non-uniform design weights: every fifth row (the noisiest) is light
    w = np.where(np.arange(m) % 5 == 0, 0.05, 1.0) * rng.uniform(0.5, 4.0, size=m)
    return x, r, w


def _weighted_lstsq(x, r, w):
    m, d = x.shape
    sw = np.sqrt(w)[:, None]
    coef, *_ = np.linalg.lstsq(sw * np.hstack([x, np.ones((m, 1))]), sw * r, rcond=None)
    return coef[:d], coef[d]


def _weighted_ridge_augmented(x, y, w, lam):
    """argmin_{W,a} sum_i w_i |y_i - a - x_i W|^2 + lam |W|_F^2 (a unpenalised)."""
    m, d = x.shape
    sw = np.sqrt(w)[:, None]
    top = sw * np.hstack([x, np.ones((m, 1))])
    pen = np.hstack([np.sqrt(lam) * np.eye(d), np.zeros((d, 1))])
    coef, *_ = np.linalg.lstsq(np.vstack([top, pen]), np.vstack([sw * y, np.zeros((d, y.shape[1]))]), rcond=None)
    return coef[:d], coef[d]


def _top_projector(r, k):
    lam, vec = np.linalg.eigh(r.T @ r)
    v = vec[:, np.argsort(-lam)[:k]]
    return v @ v.T


def _check_least_squares(fit_fn) -> bool:
    x, r, w = _problem(101)
    d = x.shape[1]
    f = fit_fn(r, x, w, d, 1e-13)
    bm, b0 = _weighted_lstsq(x, r, w)
    return f["rank"] == d and np.allclose(f["B"], bm, atol=1e-8) and np.allclose(f["b"], b0, atol=1e-8)


def _check_ridge(fit_fn, relative: bool) -> bool:
    x, r, w = _problem(202)
    m, d = x.shape
    rank, lam = 3, 0.35
    f = fit_fn(r, x, w, rank, lam, relative=relative)
    if f["rank"] != rank:
        return False
    v = f["V"]
    if not np.allclose(v @ v.T, _top_projector(r, rank), atol=1e-10):
        return False
    if relative:
        # trace of the weighted centred Gram over d: sum_i w_i |x_i - xbar_w|^2 / d
        xbar = np.average(x, axis=0, weights=w)
        lam = lam * float(np.sum(w * np.sum((x - xbar) ** 2, axis=1))) / d
    wm, a = _weighted_ridge_augmented(x, r @ v, w, lam)
    return np.allclose(f["B"], wm @ v.T, atol=1e-9) and np.allclose(f["b"], a @ v.T, atol=1e-9)


def test_weighted_fit_equals_weighted_least_squares():
    assert _check_least_squares(fit_residual)


def test_weighted_ridge_equals_augmented_system():
    assert _check_ridge(fit_residual, relative=False)
    assert _check_ridge(fit_residual, relative=True)


def test_weights_matter_in_these_problems():
    # the pins would not see a dropped weighting if uniform weights gave the same fit
    x, r, w = _problem(101)
    bm, _ = _weighted_lstsq(x, r, w)
    bu, _ = _weighted_lstsq(x, r, np.ones_like(w))
    assert not np.allclose(bm, bu, atol=1e-3)


MUTANTS = {
    "unweighted Gram": ("gram = xc.T @ (w[:, None] * xc)", "gram = xc.T @ xc"),
    "weights on X only": ("wmat = np.linalg.solve(a, xc.T @ (w[:, None] * yc))", "wmat = np.linalg.solve(a, xc.T @ yc)"),
    "sqrt(w) in the Gram": ("gram = xc.T @ (w[:, None] * xc)", "gram = xc.T @ (np.sqrt(w)[:, None] * xc)"),
    "unweighted means": ("xbar = (w[:, None] * x).sum(axis=0) / ws", "xbar = x.mean(axis=0)"),
}


def _mutant(old: str, new: str):
    src = textwrap.dedent(inspect.getsource(O.fit_residual))
    assert old in src, f"mutation site not found: {old}"
    ns = dict(vars(O))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["fit_residual"]


def test_planted_slips_fail_the_pins():
    for name, (old, new) in MUTANTS.items():
        fn = _mutant(old, new)
        caught = (not _check_least_squares(fn)) or (not _check_ridge(fn, False)) or (not _check_ridge(fn, True))
        assert caught, f"the pins do not catch the slip: {name}"
