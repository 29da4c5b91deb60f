"""The k-means assignment's error bound takes one 32x32x16 bf16 MFMA to be
within 18 units of roundoff (u = 2^-24) of the sum of magnitudes of its
inputs,
    |result - (acc + sum_k a_k b_k)| <= 18 u (|acc| + sum_k |a_k b_k|),
the worst case of its 17 terms aligned to the largest with 24-bit truncation
and one final rounding (16 sequential fp32 additions stay within it too).
This checks the bound on the device, through the C ABI, on small products
beside a large accumulator, halfway ties, cancellation, and random patterns
with a wide exponent spread; exact sums are computed with rationals.  The
largest error seen is printed (well under 18 u)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import free_block_sparse_amd as sp

pytestmark = pytest.mark.gpu


def _bf16(x: float) -> float:
    return float(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).float())


def _round_f32(fr: Fraction) -> float:
    """Nearest fp32 to an exact rational (ties to even), with no double rounding."""
    x = np.float32(float(fr))
    cands = {float(x), float(np.nextafter(x, np.float32(np.inf))), float(np.nextafter(x, np.float32(-np.inf)))}
    best = min(cands, key=lambda c: (abs(Fraction(c) - fr), int(np.float32(c).view(np.uint32)) & 1))
    return best


def _sequential(a, b, acc) -> float:
    s = np.float32(acc)
    for x, y in zip(a, b):
        s = np.float32(s + np.float32(x * y))
    return float(s)


def _patterns():
    t, s = 2.0 ** -12, 2.0 ** -13
    pats = [
        ([s] * 16, [t] * 16, 1.0),                                       # 1 + 16 x 2^-25
        ([2.0 ** 12] + [1.0] * 15, [2.0 ** 12] + [1.0] * 15, 0.0),       # 2^24 + 15
        ([1.0] * 15 + [2.0 ** 12], [1.0] * 15 + [2.0 ** 12], 0.0),
        ([2.0 ** 10, 2.0 ** -2] * 8, [2.0 ** 10, 2.0 ** -2, -2.0 ** 10, 2.0 ** -2] * 4, 0.0),
        ([s] * 8 + [0.0] * 8, [2.0 ** -11] * 8 + [0.0] * 8, 1.0),          # halfway ties
        ([2.0 ** -12] + [2.0 ** -15] * 15, [2.0 ** -12] + [2.0 ** -15] * 15, 1.0),
        ([2.0 ** 3] * 16, [4.0] * 16, 2.0 ** 30),
        ([-1.0] * 3 + [2.0 ** -11] * 13, [1.0] * 3 + [2.0 ** -11] * 13, 3.0),
    ]
    rng = np.random.default_rng(2026)
    for _ in range(2000):
        ea, eb = rng.integers(-20, 20, size=16), rng.integers(-20, 20, size=16)
        a = [_bf16(float(m) * 2.0 ** int(e)) for m, e in zip(rng.uniform(-2, 2, 16), ea)]
        b = [_bf16(float(m) * 2.0 ** int(e)) for m, e in zip(rng.uniform(-2, 2, 16), eb)]
        big = max(abs(x * y) for x, y in zip(a, b))
        acc = float(np.float32(rng.uniform(-1, 1) * big * 2.0 ** int(rng.integers(-30, 4))))
        pats.append((a, b, acc))
    return pats


def test_bf16_mfma_error_within_the_assignment_bound():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pats = _patterns()
    print(f"[mfma] {len(pats)} patterns through sparsepr_mfma_rounding_check", flush=True)
    buf = np.zeros((len(pats), 33), np.float32)
    for i, (a, b, c) in enumerate(pats):
        buf[i, :16], buf[i, 16:32], buf[i, 32] = a, b, c
    got = sp.sparsepr_mfma_rounding_check(torch.from_numpy(buf).cuda()).cpu().numpy()
    u = Fraction(1, 2 ** 24)
    worst, n_exact, seq_over = Fraction(0), 0, 0
    for i, (a, b, c) in enumerate(pats):
        exact = Fraction(c) + sum(Fraction(x) * Fraction(y) for x, y in zip(a, b))
        mag = abs(Fraction(c)) + sum(abs(Fraction(x) * Fraction(y)) for x, y in zip(a, b))
        err = abs(Fraction(float(got[i])) - exact)
        n_exact += float(got[i]) == _round_f32(exact)
        seq_over += abs(Fraction(_sequential(a, b, c)) - exact) > u * mag
        if mag > 0:
            worst = max(worst, err / (u * mag))
        assert err <= 18 * u * mag, (i, a, b, c, float(got[i]), float(exact))
    print(f"[mfma] largest error {float(worst):.3g} u (|acc| + sum |products|); correctly rounded on {n_exact} of "
          f"{len(pats)}; 16 sequential fp32 roundings exceed one u on {seq_over}", flush=True)
