"""Pins for the oracle's Randomized Hadamard Transform, norm-based range and
truncation (THC page section 5), CPU only: scipy's Hadamard matrix in
binary64, the transform's orthogonality (H H = d I), norm preservation,
linearity with a shared diagonal, the Rademacher layout against Philox, the
normal quantile t_p, and the truncation fraction."""
import math

import numpy as np
import pytest
import scipy.linalg
import scipy.stats

import oracle


@pytest.mark.parametrize("k", [1, 2, 5, 8, 10])
def test_forward_matches_hadamard_matrix(k):
    d = 1 << k
    rng = np.random.default_rng(k)
    x = (rng.standard_normal(3 * d) * np.exp(rng.uniform(-3, 3, 3 * d))).astype(np.float32)
    seed = 0xABCDEF0123 + k
    y = oracle.rht_forward(x, d, seed)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    D = oracle.rademacher(seed, 0, 3 * d).astype(np.float64)
    for b in range(3):
        xb = x[b * d:(b + 1) * d].astype(np.float64)
        exact = H @ (D[b * d:(b + 1) * d] * xb) / math.sqrt(d)
        bound = (k + 2) * 2.0 ** -24 * np.abs(xb).sum() / math.sqrt(d)
        assert np.all(np.abs(y[b * d:(b + 1) * d] - exact) <= bound + 1e-30)


def test_inverse_and_norm_and_linearity():
    d = 1 << 12
    rng = np.random.default_rng(1)
    xs = [rng.standard_normal(2 * d).astype(np.float32) * 0.01 for _ in range(3)]
    seed = 77
    ys = [oracle.rht_forward(x, d, seed) for x in xs]
    for x, y in zip(xs, ys):
        z = oracle.rht_inverse(y, d, seed)
        assert np.max(np.abs(z - x)) <= 14 * 2.0 ** -24 * np.abs(x).max() * 8
        for b in range(2):
            n0 = np.linalg.norm(x[b * d:(b + 1) * d].astype(np.float64))
            n1 = np.linalg.norm(y[b * d:(b + 1) * d].astype(np.float64))
            assert abs(n1 - n0) <= 1e-5 * n0
    # the transform of the sum is the sum of the transforms (same D)
    tot = oracle.rht_forward((xs[0].astype(np.float64) + xs[1] + xs[2]).astype(np.float32), d, seed)
    assert np.max(np.abs(tot - (ys[0].astype(np.float64) + ys[1] + ys[2]))) <= 1e-6
    # a different seed is a different D
    assert not np.array_equal(oracle.rht_forward(xs[0], d, seed + 1), ys[0])


def test_rademacher_layout_and_balance():
    seed = 0x1122334455667788
    s = oracle.rademacher(seed, 0, 1 << 16)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 5 / math.sqrt(1 << 16)
    for e in (0, 5, 31, 32, 127, 128, 1000, (1 << 35) + 77):
        q = e >> 7
        out = oracle.philox4x32_10([q & 0xFFFFFFFF, q >> 32, 0x52485400, 0],
                                   [seed & 0xFFFFFFFF, seed >> 32])
        bit = (int(out[(e >> 5) & 3]) >> (e & 31)) & 1
        assert oracle.rademacher(seed, e, 1)[0] == (-1.0 if bit else 1.0)


def test_tp_quantile():
    """t_p = Phi^-1(1 - p/2): the two-sided normal quantile (textbook values)."""
    assert abs(scipy.stats.norm.ppf(1 - 0.05 / 2) - 1.959963984540054) < 1e-12
    assert abs(scipy.stats.norm.ppf(1 - 0.01 / 2) - 2.5758293035489004) < 1e-12


def test_range_and_truncation_fraction():
    """M = t_p max_i ||x_i|| / sqrt(d) per block; after the transform about a
    fraction p of coordinates of the largest-norm worker fall outside."""
    d = 1 << 14
    rng = np.random.default_rng(4)
    P, nblk = 3, 2
    xs = [(rng.standard_normal(nblk * d) * (i + 1) * np.exp(rng.uniform(-2, 2, nblk * d)))
          .astype(np.float32) for i in range(P)]
    ss = np.stack([oracle.rht_sumsq(x, d) for x in xs])
    for i in range(P):
        for b in range(nblk):
            ref = np.sum(xs[i][b * d:(b + 1) * d].astype(np.float64) ** 2)
            assert abs(ss[i, b] - ref) <= 1e-12 * ref
    p = 1 / 32
    t_p = float(scipy.stats.norm.ppf(1 - p / 2))
    mM = oracle.rht_range(ss, d, t_p)
    for b in range(nblk):
        want = t_p * math.sqrt(ss[:, b].max()) / math.sqrt(d)
        assert mM[b, 1] == np.float32(want) and mM[b, 0] == -mM[b, 1]
    y = oracle.rht_forward(xs[P - 1], d, 5)      # the largest-norm worker
    frac = np.mean(np.abs(y) > np.repeat(mM[:, 1], d))
    assert abs(frac - p) < 0.25 * p
    yc = oracle.clamp(y, d, mM)
    assert np.all(yc <= np.repeat(mM[:, 1], d)) and np.all(yc >= np.repeat(mM[:, 0], d))
    inside = np.abs(y) <= np.repeat(mM[:, 1], d)
    assert np.array_equal(yc[inside], y[inside])


def test_rht_thc_round_trip_reduces_range_error():
    """End to end on the oracle: transform, truncate, uniform-quantize,
    aggregate, dequantize, inverse transform; the estimate of the average is
    unbiased up to truncation and its NMSE is far below quantizing heavy-tailed
    inputs on their own [min, max] range."""
    d = 1 << 12
    rng = np.random.default_rng(9)
    P, b = 4, 4
    xs = [(rng.laplace(0, 1e-3, 2 * d)).astype(np.float32) for _ in range(P)]
    exact = np.mean(np.stack(xs).astype(np.float64), axis=0)
    t_p = float(scipy.stats.norm.ppf(1 - (1 / 32) / 2))
    ys = [oracle.rht_forward(x, d, 11) for x in xs]
    mM = oracle.rht_range(np.stack([oracle.rht_sumsq(x, d) for x in xs]), d, t_p)
    ys = [oracle.clamp(y, d, mM) for y in ys]
    packed = [oracle.usq_quantize(ys[i], i, d, mM, b, 3) for i in range(P)]
    S = oracle.int_aggregate(packed, 2 * d, b)
    yhat = oracle.dequant(S, P, b, d, mM)
    xhat = oracle.rht_inverse(yhat, d, 11)
    nm_rht = np.sum((xhat - exact) ** 2) / np.sum(exact ** 2)
    mM0 = oracle.minmax(xs, d)
    packed0 = [oracle.usq_quantize(xs[i], i, d, mM0, b, 3) for i in range(P)]
    xhat0 = oracle.dequant(oracle.int_aggregate(packed0, 2 * d, b), P, b, d, mM0)
    nm_plain = np.sum((xhat0 - exact) ** 2) / np.sum(exact ** 2)
    assert nm_rht < 0.5 * nm_plain


def test_ragged_length_is_zero_padded():
    d = 256
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3 * d + 17).astype(np.float32)
    pad = np.concatenate([x, np.zeros(d - 17, dtype=np.float32)])
    assert np.array_equal(oracle.rht_forward(x, d, 3), oracle.rht_forward(pad, d, 3))
    assert np.array_equal(oracle.rht_sumsq(x, d), oracle.rht_sumsq(pad, d))


def test_block_offset_selects_the_same_signs():
    """Transforming blocks q.. on their own (e0 = q d) gives the whole
    vector's blocks q.. (the signs follow global indices)."""
    d, seed = 64, 21
    x = np.random.default_rng(2).standard_normal(5 * d).astype(np.float32)
    y = oracle.rht_forward(x, d, seed)
    assert np.array_equal(oracle.rht_forward(x[2 * d:], d, seed, e0=2 * d), y[2 * d:])
    assert np.array_equal(oracle.rht_inverse(y[3 * d:], d, seed, e0=3 * d),
                          oracle.rht_inverse(y, d, seed)[3 * d:])
    assert not np.array_equal(oracle.rht_forward(x[2 * d:], d, seed), y[2 * d:])
    with pytest.raises(Exception):
        oracle.rht_forward(x, d, seed, e0=5)
