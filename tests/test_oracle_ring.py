"""Pins for the oracle's ring all-reduce (CPU only).

Each test checks the oracle against something fixed outside it: the
lesson's worked example, exact integer sums, a hand-derived fold order, the
literal step schedule, the recursive-summation error bound, torch's bf16
rounding.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(path):
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            kv[k] = v
    return kv


def test_lesson_demo_values_steps_bytes():
    """Lesson section 7 demo: 4 GPUs x 8 elements -> 100 + 4 i everywhere."""
    kv = _read_kv(os.path.join(GOLDEN, "ring_demo.txt"))
    P, N = int(kv["P"][0]), int(kv["N"][0])
    expect = np.array([float(v) for v in kv["expected_sum"]], dtype=np.float32)
    for stepwise in (False, True):
        bufs = [np.array([float(v) for v in kv[f"input_g{g}"]], dtype=np.float32) for g in range(P)]
        (oracle.ring_stepwise if stepwise else oracle.ring_fold)(bufs, op=oracle.SUM)
        for b in bufs:
            assert np.array_equal(b, expect)
    steps, nbytes = oracle.ring_stats(P, N, 0, int(kv["elem_bytes"][0]))
    assert steps == int(kv["steps"][0])
    assert nbytes == int(kv["bytes_per_gpu"][0])


@pytest.mark.parametrize("P", [2, 3, 4, 5, 7, 8, 16])
@pytest.mark.parametrize("N", [1, 5, 8, 33, 130])
def test_integer_inputs_equal_exact_sum(P, N):
    """Integer-valued fp32 inputs whose partial sums stay below 2^24 make
    every fold order exact: the result must be the integer sum."""
    rng = np.random.default_rng(P * 1000 + N)
    ints = rng.integers(-(1 << 20), 1 << 20, size=(P, N))
    exact = ints.sum(axis=0)
    for fn in (oracle.ring_fold, oracle.ring_stepwise):
        bufs = [ints[i].astype(np.float32) for i in range(P)]
        fn(bufs, op=oracle.SUM)
        for b in bufs:
            assert np.array_equal(b.astype(np.int64), exact)
        bufs = [ints[i].astype(np.float32) for i in range(P)]
        fn(bufs, op=oracle.AVG)
        want = exact.astype(np.float32) / np.float32(P)   # one IEEE division
        for b in bufs:
            assert np.array_equal(b, want)


def _order_probe(P, big_pos):
    """P workers, N = P (one element per chunk). For element e the ring's
    fold starts at worker e (the chunk's index) and continues e+1, e+2, ...
    Worker (e + big_pos) mod P holds 1.0, every other worker 2^-24."""
    N = P
    bufs = [np.full(N, 2.0 ** -24, dtype=np.float32) for _ in range(P)]
    for e in range(N):
        bufs[(e + big_pos) % P][e] = 1.0
    return bufs


@pytest.mark.parametrize("fn", [oracle.ring_fold, oracle.ring_stepwise])
def test_fold_order_is_chunk_owner_first(fn):
    """Hand-derived from the lesson's schedule (section 7): chunk c is sent
    first by worker c, then extended by c+1, ..., c-1. Adding 2^-24 (half an
    ulp of 1) to 1.0 ties and rounds back to 1.0; two such terms added first
    make 2^-23 and survive. So for P = 3:
      big value at fold position 0 or 1 -> 1.0
      big value at fold position 2     -> 1 + 2^-23
    and for P = 4 (three small terms 3 * 2^-24 = 1.5 ulp, tie to even):
      positions 0, 1 -> 1.0; positions 2, 3 -> 1 + 2^-22."""
    cases = {3: [1.0, 1.0, 1.0 + 2.0 ** -23], 4: [1.0, 1.0, 1.0 + 2.0 ** -22, 1.0 + 2.0 ** -22]}
    for P, expect in cases.items():
        for pos, want in enumerate(expect):
            bufs = _order_probe(P, pos)
            fn(bufs, op=oracle.SUM)
            for b in bufs:
                assert np.all(b == np.float32(want)), (P, pos, b)


@pytest.mark.parametrize("P", [2, 3, 4, 5, 8])
def test_owner_after_scatter_reduce(P):
    """After the scatter-reduce phase worker j holds the complete sum of
    chunk (j + 1) mod P (Horovod page 3.4: node j holds chunk
    (j - (N - 1)) mod N)."""
    N = 4 * P + 3   # ragged: C = 5 (P=2..) -> short last chunk
    rng = np.random.default_rng(P)
    ints = rng.integers(-1000, 1000, size=(P, N))
    exact = ints.sum(axis=0)
    bufs = [ints[i].astype(np.float32) for i in range(P)]
    oracle.ring_stepwise(bufs, op=oracle.SUM, rs_only=True)
    C = -(-N // P)
    for j in range(P):
        c = (j + 1) % P
        lo, hi = c * C, min((c + 1) * C, N)
        assert np.array_equal(bufs[j][lo:hi].astype(np.int64), exact[lo:hi])


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 6, 7, 8])
def test_step_schedule_equals_fold_bitwise(P):
    """Brute force: the literal 2(P-1)-step schedule (send copies, add or
    overwrite) gives the same bits as the per-element fold, for random
    magnitudes, ragged N (P not dividing N, N < P) and partitions."""
    rng = np.random.default_rng(7 + P)
    for N in list(range(0, 40)) + [1000, 1001]:
        for part in (0, 7, 64):
            x = (rng.standard_normal((P, N)) * np.exp(rng.uniform(-20, 20, size=(P, N))))
            x = x.astype(np.float32)
            a = [x[i].copy() for i in range(P)]
            b = [x[i].copy() for i in range(P)]
            oracle.ring_fold(a, op=oracle.AVG, part=part)
            oracle.ring_stepwise(b, op=oracle.AVG, part=part)
            for i in range(P):
                assert np.array_equal(a[i].view(np.uint32), b[i].view(np.uint32)), (P, N, part)
                assert np.array_equal(a[i].view(np.uint32), a[0].view(np.uint32))


def test_error_bound_against_exact_sum():
    """|fl(sum) - sum| <= (P-1) u sum|x_i| with u = 2^-24 (recursive
    summation bound), against the correctly rounded exact sum (math.fsum)."""
    rng = np.random.default_rng(3)
    for P in (2, 5, 16, 64):
        N = 257
        x = (rng.standard_normal((P, N)) * 0.01).astype(np.float32)
        bufs = [x[i].copy() for i in range(P)]
        oracle.ring_fold(bufs, op=oracle.SUM)
        for e in range(N):
            col = [float(v) for v in x[:, e]]
            exact = math.fsum(col)
            bound = (P - 1) * 2.0 ** -24 * sum(abs(v) for v in col)
            assert abs(float(bufs[0][e]) - exact) <= bound + 1e-45


def test_avg_power_of_two_is_exact_scaling():
    rng = np.random.default_rng(11)
    for P in (2, 4, 8, 16, 32):
        x = rng.standard_normal((P, 300)).astype(np.float32)
        s = [x[i].copy() for i in range(P)]
        a = [x[i].copy() for i in range(P)]
        oracle.ring_fold(s, op=oracle.SUM)
        oracle.ring_fold(a, op=oracle.AVG)
        assert np.array_equal(a[0], s[0] * np.float32(1.0 / P))


def test_all_buffers_bitwise_equal_and_chunk_rule_when_divisible():
    """Lesson section 7: all GPUs end bitwise synchronized; when P divides N
    the chunk size is exactly N / P, as in the lesson's simulator."""
    rng = np.random.default_rng(5)
    P, N = 4, 64
    x = rng.standard_normal((P, N)).astype(np.float32)
    bufs = [x[i].copy() for i in range(P)]
    oracle.ring_stepwise(bufs, op=oracle.SUM)
    for b in bufs[1:]:
        assert np.array_equal(b.view(np.uint32), bufs[0].view(np.uint32))
    steps, nbytes = oracle.ring_stats(P, N, 0, 4)
    assert steps == 2 * (P - 1) and nbytes == 2 * (P - 1) * (N // P) * 4
    # Horovod page 3.4: data sent per node = 2 (N-1)/N * K
    assert nbytes == 2 * (P - 1) * N * 4 // P


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([
        rng.standard_normal(4096).astype(np.float32) * 1e-3,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.4e38, -3.4e38, 1e-40], dtype=np.float32),
    ])
    # values exactly halfway between two bf16 numbers, both parities
    halves = (np.arange(0, 64, dtype=np.uint32) << 16 | 0x8000) + (0x3F80 << 16)
    x = np.concatenate([x, halves.view(np.float32)])
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("P", [2, 3, 8])
def test_bf16_fp32_accumulation(P):
    """bf16 inputs with integer values: partial sums in fp32 are exact, so the
    result is the exact sum rounded once to bf16 (torch's RNE)."""
    rng = np.random.default_rng(P)
    N = 3 * P + 1
    ints = rng.integers(-256, 256, size=(P, N))
    bufs = [oracle.f32_to_bf16(ints[i].astype(np.float32)) for i in range(P)]
    oracle.ring_fold(bufs, op=oracle.SUM)
    want = torch.from_numpy(ints.sum(axis=0).astype(np.float32)).to(torch.bfloat16)
    want = want.view(torch.int16).numpy().view(np.uint16)
    for b in bufs:
        assert np.array_equal(b, want)
    # the stepwise schedule with fp32 partials agrees with the fold
    x = (rng.standard_normal((P, 1001)) * 1e-3).astype(np.float32)
    a = [oracle.f32_to_bf16(x[i]) for i in range(P)]
    c = [v.copy() for v in a]
    oracle.ring_fold(a, op=oracle.AVG, part=100)
    oracle.ring_stepwise(c, op=oracle.AVG, part=100)
    for i in range(P):
        assert np.array_equal(a[i], c[i])
