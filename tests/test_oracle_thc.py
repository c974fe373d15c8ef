"""Pins for the oracle's THC path: Philox, the USQ grid and quantizer,
the integer aggregate, dequantization and NMSE (CPU only).

Pins: published known-answer vectors, the THC page's worked examples,
numpy library routines, hand-packed bytes, exact probability arguments
(unbiasedness, Bernoulli variance, exhaustive outcome enumeration).
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                w = [int(v, 16) for v in line.split()]
                rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        assert list(oracle.philox4x32_10(ctr, key)) == out


def test_uniform16_layout_and_uniformity():
    """Element e takes half (e mod 2) of word (e mod 8) / 2 of the Philox
    block g = e / 8 keyed by the seed, counter word 2 = worker."""
    seed, worker = 0x0123456789ABCDEF, 5
    for e in (0, 1, 7, 8, 15, 1 << 33, (1 << 33) + 5, (1 << 40) + 3):
        g = e >> 3
        blk = oracle.philox4x32_10([g & 0xFFFFFFFF, g >> 32, worker, 0],
                                   [seed & 0xFFFFFFFF, seed >> 32])
        j = e & 7
        assert oracle.uniform16(seed, worker, e) == (int(blk[j >> 1]) >> (16 * (j & 1))) & 0xFFFF
    # chi-square over 64 bins of 2^16 draws
    vals = np.array([oracle.uniform16(7, 0, e) for e in range(1 << 16)])
    counts = np.bincount(vals >> 10, minlength=64)
    chi2 = ((counts - 1024.0) ** 2 / 1024.0).sum()
    assert chi2 < 63 + 6 * math.sqrt(2 * 63)


def _grid(m, M, b):
    return np.array([[m, M]], dtype=np.float32)


def test_usq_grid_worked_example():
    """THC page section 4: on [-1, 1] with 2 bits the grid is
    {-1, -1/3, 1/3, 1}; index pairs summing to 3 decode to a value sum 0."""
    mM = _grid(-1.0, 1.0, 2)
    T0 = [-1.0, -1.0 / 3.0, 1.0 / 3.0, 1.0]
    for z, want in enumerate(T0):
        got = oracle.dequant(np.array([z], dtype=np.int32), P=1, b=2, part=0, mM=mM)[0]
        assert abs(float(got) - want) <= 2 * 2.0 ** -24
    for z, z2 in [(0, 3), (1, 2), (2, 1), (3, 0)]:
        avg = oracle.dequant(np.array([z + z2], dtype=np.int32), P=2, b=2, part=0, mM=mM)[0]
        assert float(avg) == 0.0


@pytest.mark.parametrize("b,x,want", [
    (1, [1, 0, 1, 1, 0, 0, 0, 1, 1], [0x8D, 0x01]),
    (2, [1, 2, 3, 0, 3], [0x39, 0x03]),
    (4, [5, 10, 15, 0, 9], [0xA5, 0x0F, 0x09]),
    (8, [7, 255, 0], [7, 255, 0]),
])
def test_pack_layout_by_hand(b, x, want):
    """On the grid m = 0, M = 2^b - 1 every integer input is a grid point
    (f = 0, or the top point where f = 1), so its index is the value itself
    whatever the random draw; bytes are packed least significant bits first."""
    L = (1 << b) - 1
    xs = np.array(x, dtype=np.float32)
    for seed in (1, 2, 3):
        packed = oracle.usq_quantize(xs, 0, 0, _grid(0.0, float(L), b), b, seed)
        assert list(packed) == want
        assert list(oracle.unpack_indices(packed, len(x), b)) == x


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_usq_deterministic_cases(b):
    L = (1 << b) - 1
    rng = np.random.default_rng(b)
    # a = m -> index 0, for any grid
    for m, M in [(-0.3, 0.7), (-1e-3, 2e-3), (5.0, 9.0)]:
        x = np.full(100, m, dtype=np.float32)
        p = oracle.usq_quantize(x, 3, 0, _grid(m, M, b), b, 99)
        assert not oracle.unpack_indices(p, 100, b).any()
    # a = M -> index L where M - m is L times a power of two (s = 2^-k exact)
    for k in (-3, 0, 5):
        M = float(L) * 2.0 ** k
        x = np.full(100, M, dtype=np.float32)
        p = oracle.usq_quantize(x, 1, 0, _grid(0.0, M, b), b, 7)
        assert (oracle.unpack_indices(p, 100, b) == L).all()
    # zero range -> index 0
    x = rng.standard_normal(50).astype(np.float32)
    p = oracle.usq_quantize(x, 0, 0, _grid(0.25, 0.25, b), b, 1)
    assert not p.any()
    out = oracle.dequant(np.zeros(50, dtype=np.int32), P=4, b=b, part=0, mM=_grid(0.25, 0.25, b))
    assert (out == np.float32(0.25)).all()


def test_minmax_equals_numpy():
    rng = np.random.default_rng(0)
    P, N = 5, 1001
    x = rng.standard_normal((P, N)).astype(np.float32)
    for part in (0, 100, 1001, 4096):
        mM = oracle.minmax([x[i] for i in range(P)], part)
        plen = part or N
        for p in range(mM.shape[0]):
            sl = x[:, p * plen:(p + 1) * plen]
            assert mM[p, 0] == sl.min() and mM[p, 1] == sl.max()
    # -0 is canonicalised to +0 at both ends
    z = [np.array([-0.0, -0.0], dtype=np.float32)] * 2
    mM = oracle.minmax(z, 0)
    assert np.signbit(mM).sum() == 0
    # bf16 inputs
    xb = [oracle.f32_to_bf16(x[i]) for i in range(P)]
    mM = oracle.minmax(xb, 0)
    xf = np.stack([oracle.bf16_to_f32(v) for v in xb])
    assert mM[0, 0] == xf.min() and mM[0, 1] == xf.max()


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_usq_unbiased_and_bernoulli_variance(b):
    """THC page section 3: stochastic quantization is unbiased, E[Q(a)] = a;
    its variance is that of a Bernoulli(f) step of size delta, at most
    delta^2 / 4."""
    L = (1 << b) - 1
    rng = np.random.default_rng(100 + b)
    m, M = -0.05, 0.08
    x = rng.uniform(m, M, size=48).astype(np.float32)
    x[0], x[1] = m, M
    mM = _grid(m, M, b)
    K = 4096
    vals = np.empty((K, x.size), dtype=np.float64)
    for k in range(K):
        p = oracle.usq_quantize(x, 0, 0, mM, b, 1000 + k)
        z = oracle.unpack_indices(p, x.size, b)
        vals[k] = oracle.dequant(z, P=1, b=b, part=0, mM=mM)
    delta = (np.float32(M) - np.float32(m)) / L
    mean, var = vals.mean(axis=0), vals.var(axis=0)
    # 5 sigma of the sample mean, the 2^-17 step of the 16-bit draw, and the
    # binary32 rounding of the grid position (a few ulps of L)
    tol = 5 * delta / (2 * math.sqrt(K)) + delta * (2.0 ** -17 + 4 * L * 2.0 ** -24) + 1e-8
    assert np.all(np.abs(mean - x.astype(np.float64)) <= tol)
    f = (x.astype(np.float64) - m) / delta
    f = f - np.minimum(np.floor(f), L - 1)
    assert np.all(var <= delta ** 2 / 4 * 1.15 + 1e-18)
    assert np.allclose(var, f * (1 - f) * delta ** 2, atol=0.08 * delta ** 2 / 4)


def test_exhaustive_outcome_distribution():
    """Brute force on a tiny case: P = 3 workers, N = 2 elements, b = 1 on
    the grid {0, 1}. Every worker rounds up independently with probability
    equal to its value; enumerate all 2^(P N) up/down outcomes to get the
    exact distribution of the aggregate S, and compare with frequencies over
    K seeds (chi-square)."""
    x = np.array([[0.25, 0.5], [0.75, 1.0], [0.0, 0.5]], dtype=np.float32)
    P, N, b = 3, 2, 1
    mM = _grid(0.0, 1.0, b)
    exact = {}
    for ups in itertools.product((0, 1), repeat=P * N):
        pr = 1.0
        for i in range(P):
            for e in range(N):
                pu = float(x[i, e])
                pr *= pu if ups[i * N + e] else 1 - pu
        if pr == 0:
            continue
        S = tuple(sum(ups[i * N + e] for i in range(P)) for e in range(N))
        exact[S] = exact.get(S, 0.0) + pr
    K = 20000
    counts = {}
    for k in range(K):
        packed = [oracle.usq_quantize(x[i], i, 0, mM, b, 5000 + k) for i in range(P)]
        S = tuple(oracle.int_aggregate(packed, N, b))
        counts[S] = counts.get(S, 0) + 1
    assert set(counts) <= set(exact)
    chi2 = sum((counts.get(s, 0) - K * p) ** 2 / (K * p) for s, p in exact.items())
    dof = len(exact) - 1
    assert chi2 < dof + 6 * math.sqrt(2 * dof)


def test_aggregate_is_integer_sum_and_bounded():
    rng = np.random.default_rng(1)
    for P, b in [(1, 8), (4, 4), (32, 8), (64, 8), (8, 2), (7, 1)]:
        N = 777
        L = (1 << b) - 1
        x = rng.standard_normal((P, N)).astype(np.float32)
        mM = oracle.minmax([x[i] for i in range(P)], 100)
        packed = [oracle.usq_quantize(x[i], i, 100, mM, b, 42) for i in range(P)]
        S = oracle.int_aggregate(packed, N, b)
        Z = np.stack([oracle.unpack_indices(p, N, b) for p in packed])
        assert np.array_equal(S, Z.sum(axis=0))
        assert S.min() >= 0 and S.max() <= P * L
        assert P * L < 2 ** 31


def test_homomorphic_decode_of_sum_equals_mean_of_decodes():
    """Decoding the summed indices gives the mean of the per-worker decoded
    values (exact in real arithmetic; binary32 rounding only)."""
    rng = np.random.default_rng(2)
    P, N, b = 6, 500, 4
    x = (rng.standard_normal((P, N)) * 0.01).astype(np.float32)
    mM = oracle.minmax([x[i] for i in range(P)], 0)
    packed = [oracle.usq_quantize(x[i], i, 0, mM, b, 3) for i in range(P)]
    S = oracle.int_aggregate(packed, N, b)
    avg = oracle.dequant(S, P, b, 0, mM).astype(np.float64)
    m, M = float(mM[0, 0]), float(mM[0, 1])
    delta = (M - m) / ((1 << b) - 1)
    per = np.stack([m + oracle.unpack_indices(p, N, b) * delta for p in packed])
    assert np.max(np.abs(avg - per.mean(axis=0))) <= 1e-6 * max(abs(m), abs(M))


def test_nmse_definition_and_expectation():
    """THC page section 2: NMSE = ||x - xhat||^2 / ||x||^2. Its expectation
    for USQ follows from the Bernoulli variance of each worker's rounding:
    E[num] = sum_e sum_i f_ie (1 - f_ie) delta^2 / P^2."""
    rng = np.random.default_rng(4)
    P, N, b = 4, 1 << 14, 4
    L = (1 << b) - 1
    x = (rng.standard_normal((P, N)) * 0.01).astype(np.float32)
    bufs = [x[i].copy() for i in range(P)]
    mM = oracle.minmax(bufs, 0)
    packed = [oracle.usq_quantize(bufs[i], i, 0, mM, b, 11) for i in range(P)]
    S = oracle.int_aggregate(packed, N, b)
    xhat = oracle.dequant(S, P, b, 0, mM)
    oracle.ring_fold(bufs, op=oracle.AVG)
    num, den, nm = oracle.nmse(bufs[0], xhat)
    ref = np.sum((bufs[0].astype(np.float64) - xhat) ** 2) / np.sum(bufs[0].astype(np.float64) ** 2)
    assert abs(nm - ref) <= 1e-12 * ref
    assert num / den == nm
    m, M = float(mM[0, 0]), float(mM[0, 1])
    delta = (M - m) / L
    u = (x.astype(np.float64) - m) / delta
    f = u - np.minimum(np.floor(u), L - 1)
    expect = (f * (1 - f)).sum() * delta ** 2 / P ** 2 / den
    assert abs(nm / expect - 1) < 0.03
    # degenerate denominators
    zero = np.zeros(4, dtype=np.float32)
    assert oracle.nmse(zero, zero)[2] == 0.0
    assert math.isinf(oracle.nmse(zero, np.ones(4, dtype=np.float32))[2])


def test_partitions_use_their_own_grid():
    """Each partition is quantized on its own [m, M] (one grid per 4 MB
    partition, THC page section 2): in every partition the smallest element
    is sent as index 0 and the largest as 2^b - 1 (the deterministic ends of
    stochastic rounding: f = 0 never rounds up, f = 1 always does), which one
    grid over the whole vector does not do for the partitions of small scale;
    and a partition's indices do not move when another partition's grid
    does."""
    rng = np.random.default_rng(8)
    N, part, b = 300, 128, 4
    L = (1 << b) - 1
    x = (rng.standard_normal(N) * np.repeat([1e-3, 1.0, 10.0], 100)).astype(np.float32)
    mM = oracle.minmax([x], part)
    z = oracle.unpack_indices(oracle.usq_quantize(x, 2, part, mM, b, 77), N, b)
    zg = oracle.unpack_indices(oracle.usq_quantize(x, 2, 0, oracle.minmax([x], 0), b, 77), N, b)
    for p in range(mM.shape[0]):
        lo, hi = p * part, min((p + 1) * part, N)
        seg = x[lo:hi]
        assert z[lo + int(np.argmin(seg))] == 0 and z[lo + int(np.argmax(seg))] == L, p
    assert zg[int(np.argmax(x[:part]))] != L      # partition 0 spans a sliver of the whole range
    moved = mM.copy()
    moved[1] = [-100.0, 100.0]
    z2 = oracle.unpack_indices(oracle.usq_quantize(x, 2, part, moved, b, 77), N, b)
    assert np.array_equal(z2[:part], z[:part]) and np.array_equal(z2[2 * part:], z[2 * part:])
    assert not np.array_equal(z2[part:2 * part], z[part:2 * part])


def test_offset_quantize_equals_slice_of_whole():
    """Quantizing one partition on its own with its global index offset gives
    the bytes of that partition in the whole vector's packing."""
    rng = np.random.default_rng(12)
    N, part = 4096 + 40, 1024
    x = rng.standard_normal(N).astype(np.float32)
    mM = oracle.minmax([x], part)
    for b in (1, 2, 4, 8):
        whole = oracle.usq_quantize(x, 3, part, mM, b, 1234)
        for p in range(mM.shape[0]):
            lo, hi = p * part, min((p + 1) * part, N)
            sub = oracle.usq_quantize(x[lo:hi], 3, part, mM[p:p + 1], b, 1234, e_offset=lo)
            assert np.array_equal(sub, whole[lo * b // 8: lo * b // 8 + sub.size])
