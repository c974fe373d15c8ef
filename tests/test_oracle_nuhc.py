"""Pins for the oracle's non-uniform THC (lookup tables; THC page section 4,
Algorithm 2), CPU only."""
import itertools
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv():
    kv = {}
    with open(os.path.join(GOLDEN, "thc_nuhc_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, *v = line.split()
                kv[k] = v
    return kv


def test_page_example_table_values_and_sums():
    kv = _kv()
    T = [int(v) for v in kv["T"]]
    g, b = int(kv["g"][0]), int(kv["b"][0])
    mM = np.array([[float(kv["m"][0]), float(kv["M"][0])]], dtype=np.float32)
    want = [float(v) for v in kv["values"]]
    for z in range(4):
        got = oracle.nuhc_dequant(np.array([T[z]], dtype=np.int32), 1, g, 0, mM)[0]
        assert got == np.float32(want[z])
    for key in ("senders_a", "senders_b"):
        zs = [int(v) for v in kv[key]]
        Y = sum(T[z] for z in zs)
        assert Y == int(kv["table_sum"][0])
        avg = oracle.nuhc_dequant(np.array([Y], dtype=np.int32), len(zs), g, 0, mM)[0]
        assert abs(float(avg) * len(zs) - float(kv["value_sum"][0])) <= 1e-6
    # the table points themselves are reproduced exactly, whatever the draw
    x = np.array([-1.0, -0.5, 0.5, 1.0], dtype=np.float32)
    for seed in (1, 2, 3):
        p = oracle.nuhc_quantize(x, 0, 0, mM, b, g, T, seed)
        assert list(oracle.unpack_indices(p, 4, b)) == [0, 1, 2, 3]
    # and the server sums table values
    packed = [oracle.nuhc_quantize(np.full(1, v, dtype=np.float32), i, 0, mM, b, g, T, 9)
              for i, v in enumerate((-1.0, -1.0, 0.5))]
    assert oracle.nuhc_aggregate(packed, 1, b, g, T)[0] == 3


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_identity_table_is_uniform_thc(b):
    """THC page section 4: with g = 2^b - 1 and the identity table the
    non-uniform scheme is the uniform one."""
    rng = np.random.default_rng(b)
    L = (1 << b) - 1
    T = list(range(L + 1))
    P, N, part = 3, 1000, 256
    x = [(rng.standard_normal(N) * 0.01).astype(np.float32) for _ in range(P)]
    mM = oracle.minmax(x, part)
    for i in range(P):
        u = oracle.usq_quantize(x[i], i, part, mM, b, 77)
        n = oracle.nuhc_quantize(x[i], i, part, mM, b, L, T, 77)
        assert np.array_equal(u, n)
    packed = [oracle.usq_quantize(x[i], i, part, mM, b, 77) for i in range(P)]
    S = oracle.int_aggregate(packed, N, b)
    assert np.array_equal(oracle.nuhc_aggregate(packed, N, b, L, T), S)
    assert np.array_equal(oracle.nuhc_dequant(S, P, L, part, mM), oracle.dequant(S, P, b, part, mM))


def _tables():
    return [(2, 4, [0, 1, 3, 4]), (2, 9, [0, 4, 5, 9]), (4, 36,
            [0, 4, 8, 11, 13, 15, 16, 17, 19, 20, 21, 23, 25, 28, 32, 36]),
            (1, 5, [0, 5])]


@pytest.mark.parametrize("b,g,T", _tables())
def test_unbiased_and_bernoulli_variance(b, g, T):
    rng = np.random.default_rng(g)
    m, M = -0.3, 0.5
    mM = np.array([[m, M]], dtype=np.float32)
    x = rng.uniform(m, M, size=40).astype(np.float32)
    x[0], x[1] = m, M
    K = 4096
    vals = np.empty((K, x.size))
    for k in range(K):
        z = oracle.unpack_indices(oracle.nuhc_quantize(x, 0, 0, mM, b, g, T, 100 + k), x.size, b)
        vals[k] = oracle.nuhc_dequant(np.array([T[v] for v in z], dtype=np.int32), 1, g, 0, mM)
    delta = (np.float32(M) - np.float32(m)) / g
    gaps = np.diff(T)
    tol = 5 * max(gaps) * delta / (2 * math.sqrt(K)) + max(gaps) * delta * (2.0 ** -17 + 1e-5)
    assert np.all(np.abs(vals.mean(axis=0) - x.astype(np.float64)) <= tol)
    # variance of a two-point rounding: at most (gap delta)^2 / 4
    u = np.maximum((x.astype(np.float64) - float(np.float32(m))) / delta, 0.0)
    for j in range(x.size):
        z0 = max(t for t in range(len(T) - 1) if T[t] <= min(math.floor(u[j]), g - 1))
        gap = (T[z0 + 1] - T[z0]) * delta
        assert vals[:, j].var() <= gap ** 2 / 4 * 1.15 + 1e-18


def test_homomorphic_and_bounded():
    rng = np.random.default_rng(5)
    b, g, T = 4, 36, _tables()[2][2]
    P, N = 5, 700
    x = [(rng.standard_normal(N) * 0.02).astype(np.float32) for _ in range(P)]
    mM = oracle.minmax(x, 0)
    packed = [oracle.nuhc_quantize(x[i], i, 0, mM, b, g, T, 3) for i in range(P)]
    Y = oracle.nuhc_aggregate(packed, N, b, g, T)
    Z = np.stack([oracle.unpack_indices(p, N, b) for p in packed])
    assert np.array_equal(Y, np.asarray(T)[Z].sum(axis=0))
    assert Y.min() >= 0 and Y.max() <= P * g
    avg = oracle.nuhc_dequant(Y, P, g, 0, mM).astype(np.float64)
    m, M = float(mM[0, 0]), float(mM[0, 1])
    per = m + np.asarray(T)[Z] * (M - m) / g
    assert np.max(np.abs(avg - per.mean(axis=0))) <= 1e-6 * max(abs(m), abs(M))


def test_exhaustive_outcomes_with_table():
    """P = 2, N = 2 on the page's table: each worker rounds to one of the two
    neighbouring table values with probability proportional to closeness;
    enumerate the four-way outcome distribution of the table sums."""
    b, g, T = 2, 4, [0, 1, 3, 4]
    mM = np.array([[-1.0, 1.0]], dtype=np.float32)
    x = np.array([[0.0, -0.75], [0.75, 0.25]], dtype=np.float32)   # positions u = 2, 0.5, 3.5, 2.5
    delta = 0.5
    probs = []
    for i in range(2):
        row = []
        for e in range(2):
            u = (float(x[i, e]) + 1.0) / delta
            z0 = max(t for t in range(3) if T[t] <= min(math.floor(u), g - 1))
            f = (u - T[z0]) / (T[z0 + 1] - T[z0])
            row.append((z0, f))
        probs.append(row)
    exact = {}
    for ups in itertools.product((0, 1), repeat=4):
        pr, Y = 1.0, [0, 0]
        for i in range(2):
            for e in range(2):
                z0, f = probs[i][e]
                up = ups[2 * i + e]
                pr *= f if up else 1 - f
                Y[e] += T[z0 + up]
        if pr > 0:
            exact[tuple(Y)] = exact.get(tuple(Y), 0) + pr
    K = 20000
    counts = {}
    for k in range(K):
        packed = [oracle.nuhc_quantize(x[i], i, 0, mM, b, g, T, 900 + k) for i in range(2)]
        Y = tuple(oracle.nuhc_aggregate(packed, 2, b, g, T))
        counts[Y] = counts.get(Y, 0) + 1
    assert set(counts) <= set(exact)
    chi2 = sum((counts.get(s, 0) - K * p) ** 2 / (K * p) for s, p in exact.items())
    dof = len(exact) - 1
    assert chi2 < dof + 6 * math.sqrt(2 * dof)


def test_bad_tables_rejected():
    x = np.zeros(4, dtype=np.float32)
    mM = np.array([[0.0, 1.0]], dtype=np.float32)
    for b, g, T in [(2, 4, [1, 2, 3, 4]), (2, 4, [0, 2, 2, 4]), (2, 4, [0, 1, 2, 3]), (2, 2, [0, 1, 2, 2])]:
        with pytest.raises(RuntimeError):
            oracle.nuhc_quantize(x, 0, 0, mM, b, g, T, 1)
