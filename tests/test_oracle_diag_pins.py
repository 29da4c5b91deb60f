"""Pins of the oracle's structural diagnostics (CPU only): brute force over
subsets on tiny distributions, disjoint and identical supports, a planted
affine residual, and the explained fraction against an orthogonal
projection written apart from the least-squares routine."""

import itertools

import numpy as np

from oracle import dense_attention, structural_diagnostics, support_fraction, support_set
from synth import make_video_qkv


def test_support_fraction_is_the_smallest_set_by_brute_force():
    rng = np.random.default_rng(1)
    for _ in range(30):
        n = int(rng.integers(3, 11))
        p = rng.dirichlet(np.full(n, 0.3))
        best = min(len(sub) for r in range(1, n + 1) for sub in itertools.combinations(range(n), r)
                   if p[list(sub)].sum() >= 0.9 * p.sum() * (1 - 1e-12))
        assert support_fraction(p, 0.9) == best / n
        s = support_set(p, 0.9)
        assert len(s) == best and p[s].sum() >= 0.9 - 1e-12


def _qkv(n_frames=2, seed=3):
    x = make_video_qkv(n_frames, 8, 8, 1, 16, "fp32", seed, [0.08])
    return (x[t][0, 0].double().numpy() for t in ("q", "k", "v"))


def test_pooled_support_is_the_union_of_member_supports():
    q, k, v = _qkv()
    n = q.shape[0]
    s = 0.3
    dense = dense_attention(q, k, v, s)
    # identical queries share one support: pooled = per query
    qq = np.repeat(q[:1], n, axis=0)
    d = structural_diagnostics(qq, k, v, np.zeros(n, dtype=np.int64), dense_attention(qq, k, v, s), s)
    assert np.isclose(d["pooled_support"], d["per_query_support"])
    # two groups: pooled support of each is its members' union, by direct count
    labels = (np.arange(n) % 2).astype(np.int64)
    d = structural_diagnostics(q, k, v, labels, dense, s)
    logits = s * q @ k.T
    p = np.exp(logits - logits.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = []
    for g in (0, 1):
        members = np.nonzero(labels == g)[0]
        union = set()
        for i in members:
            union |= set(support_set(p[i]).tolist())
        want += [len(union) / n] * len(members)
    assert np.isclose(d["pooled_support"], np.mean(want))
    assert d["pooled_support"] >= d["per_query_support"]
    assert d["hard_drop_error"] == 0.0 and d["orthogonal_energy"] == 0.0


def test_planted_affine_residual_is_fully_explained():
    q, k, v = _qkv(seed=5)
    n, dv = v.shape
    s = 0.25
    dense = dense_attention(q, k, v, s)
    rng = np.random.default_rng(6)
    a, amat = rng.normal(size=dv) * 0.1, rng.normal(size=(dv, dv)) * 0.1
    # sparse output x with dense - x = a + x A exactly
    x = (dense - a) @ np.linalg.inv(np.eye(dv) + amat)
    d = structural_diagnostics(q, k, v, np.zeros(n, dtype=np.int64), x, s)
    assert d["affine_explained"] > 1 - 1e-10 and d["orthogonal_energy"] < 1e-20


def test_explained_fraction_matches_an_orthogonal_projection():
    q, k, v = _qkv(seed=7)
    n = q.shape[0]
    s = 0.3
    dense = dense_attention(q, k, v, s)
    rng = np.random.default_rng(8)
    x = dense + rng.normal(size=dense.shape) * 0.05 + 0.3 * np.sin(dense)
    d = structural_diagnostics(q, k, v, np.zeros(n, dtype=np.int64), x, s)
    r = dense - x
    qm, _ = np.linalg.qr(np.hstack([np.ones((n, 1)), x]))
    left = r - qm @ (qm.T @ r)
    assert np.isclose(d["affine_explained"], 1 - (left ** 2).sum() / (r ** 2).sum(), rtol=1e-10)
    assert np.isclose(d["orthogonal_energy"], (left ** 2).sum() / (dense ** 2).sum(), rtol=1e-10)
    assert np.isclose(d["hard_drop_error"], np.linalg.norm(r) / np.linalg.norm(dense), rtol=1e-12)
