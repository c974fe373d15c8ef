"""Pins of the oracle's error feedback and partial aggregation (THC page,
section 5: error feedback; section 8: the server aggregating only the
workers that arrived in time).

Error feedback: on-grid values are sent exactly and leave no error; every
residual is below one grid step; the residual is the worker's own
dequantized value subtracted from what it sent (checked against the
single-worker server average); over many rounds the values sent add up to
the gradients plus the first residual minus the last (telescoping); the
mean residual over seeds is zero (unbiased rounding). Partial aggregation:
on-grid data gives the exact mean of the workers that arrived; over seeds
the estimate is unbiased for that mean, not for all workers'."""
import numpy as np
import pytest

import oracle


def test_on_grid_values_leave_no_error():
    # m = 0, M = 15/8, b = 4: grid step 1/8, u = 8 x exactly, f = 0
    N, b = 4096, 4
    z = np.random.default_rng(1).integers(0, 16, N)
    x = (z / 8.0).astype(np.float32)
    x[0], x[1] = 0.0, 15 / 8                          # pin the extremes
    mM = np.array([[0.0, 15 / 8]], dtype=np.float32)
    pk = oracle.usq_quantize(x, 0, 0, mM, b, seed=7)
    assert np.array_equal(oracle.unpack_indices(pk, N, b), np.rint(x * 8).astype(np.int32))
    assert np.all(oracle.ef_update(x, pk, b, 0, mM) == 0.0)


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_residual_below_one_step_and_equal_to_own_dequant(b):
    N, part = 10007, 1000
    rng = np.random.default_rng(b)
    g = (rng.standard_normal(N) * 0.01).astype(np.float32)
    e = (rng.standard_normal(N) * 0.001).astype(np.float32)
    x = oracle.ef_add(g, e)
    assert np.array_equal(x, (g + e).astype(np.float32))
    mM = oracle.minmax([x], part)
    pk = oracle.usq_quantize(x, 3, part, mM, b, seed=11)
    e2 = oracle.ef_update(x, pk, b, part, mM)
    L = (1 << b) - 1
    step = np.repeat((mM[:, 1] - mM[:, 0]) / L, part)[:N]
    assert np.all(np.abs(e2) <= step * (1 + 1e-6))
    # the worker's own value = what the server's dequant gives for one worker
    own = oracle.dequant(oracle.unpack_indices(pk, N, b), 1, b, part, mM)
    assert np.array_equal(e2, (x - own).astype(np.float32))


def test_bf16_gradient_widened_exactly():
    g32 = np.random.default_rng(2).standard_normal(999).astype(np.float32)
    g = oracle.f32_to_bf16(g32)
    e = np.full(999, 0.5, dtype=np.float32)
    assert np.array_equal(oracle.ef_add(g, e), (oracle.bf16_to_f32(g) + np.float32(0.5)))


def test_table_residual_uses_table_values():
    """THC page section 4 example table T2 = {0, 1, 3, 4}, g = 4."""
    N, b, g, T = 5000, 2, 4, [0, 1, 3, 4]
    x = np.random.default_rng(3).uniform(-1, 1, N).astype(np.float32)
    mM = oracle.minmax([x], 0)
    pk = oracle.nuhc_quantize(x, 0, 0, mM, b, g, T, seed=5)
    e2 = oracle.ef_update(x, pk, b, 0, mM, g=g, T=T)
    m, M = mM[0]
    vals = np.array([m + np.float32(t) * ((M - m) / np.float32(g)) for t in T], dtype=np.float32)
    # the residual is x minus one of the two table values around x
    lo = vals[np.clip(np.searchsorted(vals, x, side="right") - 1, 0, 3)]
    hi = vals[np.clip(np.searchsorted(vals, x, side="left"), 0, 3)]
    assert np.all((e2 == (x - lo)) | (e2 == (x - hi)))
    assert np.any(e2 == (x - lo)) and np.any(e2 != (x - lo))


def test_telescoping_over_rounds():
    """sum_t sent_t + e_T = sum_t grad_t + e_0 (up to binary32 rounding)."""
    N, b, rounds = 4096, 2, 30
    rng = np.random.default_rng(4)
    e = np.zeros(N, dtype=np.float32)
    sent = np.zeros(N)
    grads = np.zeros(N)
    for t in range(rounds):
        g = (rng.standard_normal(N) * 0.01).astype(np.float32)
        x = oracle.ef_add(g, e)
        mM = oracle.minmax([x], 0)
        pk = oracle.usq_quantize(x, 0, 0, mM, b, seed=100 + t)
        e_new = oracle.ef_update(x, pk, b, 0, mM)
        sent += (x - e_new).astype(np.float64)
        grads += g
        e = e_new
    err = np.abs(sent + e - grads)
    assert err.max() < rounds * 4 * np.finfo(np.float32).eps * 0.1


def test_residual_mean_zero_over_seeds():
    N, b = 64, 2
    x = np.random.default_rng(6).uniform(-1, 1, N).astype(np.float32)
    mM = oracle.minmax([x], 0)
    acc = np.zeros(N)
    S = 4000
    for s in range(S):
        acc += oracle.ef_update(x, oracle.usq_quantize(x, 0, 0, mM, b, seed=s), b, 0, mM)
    step = float(mM[0, 1] - mM[0, 0]) / 3
    # each residual is bounded by one step: the mean of S draws is within ~5 sigma
    assert np.all(np.abs(acc / S) < 5 * step / 2 / np.sqrt(S) + 1e-6)


# ---------------------------------------------------------------- partial aggregation

def test_partial_aggregation_exact_on_grid():
    P, N, b = 10, 3000, 4
    rng = np.random.default_rng(8)
    z = rng.integers(0, 16, size=(P, N))
    xs = [(r / 8.0).astype(np.float32) for r in z]
    for x in xs:
        x[0], x[1] = 0.0, 15 / 8
    mM = oracle.minmax(xs, 0)
    packed = [oracle.usq_quantize(xs[i], i, 0, mM, b, seed=1) for i in range(P)]
    arrived = [0, 2, 3, 5, 6, 7, 9]                     # 3 stragglers dropped
    S = oracle.int_aggregate([packed[i] for i in arrived], N, b)
    est = oracle.dequant(S, len(arrived), b, 0, mM)
    want = np.mean(np.stack([xs[i] for i in arrived]).astype(np.float64), axis=0)
    assert np.allclose(est, want, rtol=0, atol=4 * np.finfo(np.float32).eps * 2)


def test_partial_aggregation_unbiased_for_arrived_mean():
    P, N, b = 6, 32, 2
    rng = np.random.default_rng(9)
    xs = [rng.uniform(-1, 1, N).astype(np.float32) for _ in range(P)]
    mM = oracle.minmax(xs, 0)
    arrived = [1, 2, 4, 5]
    acc = np.zeros(N)
    S_ = 3000
    for s in range(S_):
        pk = [oracle.usq_quantize(xs[i], i, 0, mM, b, seed=s) for i in arrived]
        acc += oracle.dequant(oracle.int_aggregate(pk, N, b), len(arrived), b, 0, mM)
    mean_arr = np.mean(np.stack([xs[i] for i in arrived]), axis=0)
    mean_all = np.mean(np.stack(xs), axis=0)
    step = float(mM[0, 1] - mM[0, 0]) / 3
    tol = 5 * step / 2 / np.sqrt(S_ * len(arrived))
    assert np.all(np.abs(acc / S_ - mean_arr) < tol)
    assert np.max(np.abs(mean_arr - mean_all)) > 10 * tol   # a different target
