"""Pins of the oracle's bidirectional ring (systemcraft ring all-reduce
lesson, section 11, Exercise 1): a hand-worked example whose binary32
rounding exposes every fold order, the literal two-direction schedule
against the closed-form fold, exact integer sums, and P = 2, where both
directions add the same pair."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dual_ring_example.txt")


def _golden():
    d = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, *v = line.split()
        d[k] = [float(t) for t in v]
    return d


def test_hand_worked_fold_orders():
    g = _golden()
    P, N = int(g["P"][0]), int(g["N"][0])
    for run in (oracle.dual_ring_fold, oracle.dual_ring_stepwise):
        bufs = [np.array(g[f"input_g{i}"], dtype=np.float32) for i in range(P)]
        run(bufs, op=oracle.SUM)
        for b in bufs:
            assert b.tolist() == g["expected_sum"]
    bufs = [np.array(g[f"input_g{i}"], dtype=np.float32) for i in range(P)]
    oracle.ring_fold(bufs, op=oracle.SUM)
    assert bufs[0].tolist() == g["single_ring_sum"]


def _inputs(P, N, dt, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((P, N)) * np.exp(rng.uniform(-8, 8, size=(P, N)))).astype(np.float32)
    if dt == oracle.BF16:
        return [oracle.f32_to_bf16(r) for r in x]
    return [r.copy() for r in x]


@pytest.mark.parametrize("dt", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("op", [oracle.SUM, oracle.AVG])
@pytest.mark.parametrize("P,N,part", [(1, 9, 0), (2, 7, 0), (3, 5, 0), (4, 8, 0), (5, 1000, 0),
                                      (8, 4099, 0), (13, 3001, 700), (6, 11, 4), (7, 0, 0),
                                      (16, 31, 0)])
def test_schedule_equals_closed_form(P, N, part, op, dt):
    a = _inputs(P, N, dt, seed=P * 1000 + N)
    b = [x.copy() for x in a]
    oracle.dual_ring_fold(a, op=op, part=part)
    oracle.dual_ring_stepwise(b, op=op, part=part)
    for i in range(P):
        assert np.array_equal(a[i].view(np.uint8), b[i].view(np.uint8)), i
        assert np.array_equal(a[i].view(np.uint8), a[0].view(np.uint8))


@pytest.mark.parametrize("P,N", [(3, 6), (5, 77), (8, 1024), (9, 100)])
def test_exact_on_small_integers(P, N):
    rng = np.random.default_rng(N)
    x = rng.integers(-1000, 1000, size=(P, N)).astype(np.float32)
    bufs = [r.copy() for r in x]
    oracle.dual_ring_stepwise(bufs, op=oracle.SUM)
    assert np.array_equal(bufs[0], x.sum(axis=0))
    bufs = [r.copy() for r in x]
    oracle.dual_ring_fold(bufs, op=oracle.AVG)
    assert np.array_equal(bufs[0], (x.sum(axis=0) / np.float32(P)).astype(np.float32))


def test_two_workers_match_single_ring():
    a = _inputs(2, 5001, oracle.F32, seed=3)
    b = [x.copy() for x in a]
    oracle.dual_ring_fold(a, op=oracle.AVG)
    oracle.ring_fold(b, op=oracle.AVG)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))


def test_directions_differ_from_single_ring():
    """On wide-range data the two fold orders disagree somewhere for P >= 3."""
    a = _inputs(4, 4000, oracle.F32, seed=9)
    b = [x.copy() for x in a]
    oracle.dual_ring_fold(a, op=oracle.SUM)
    oracle.ring_fold(b, op=oracle.SUM)
    assert not np.array_equal(a[0], b[0])
