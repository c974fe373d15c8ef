"""GPU parity for THC's randomized Hadamard transform step (THC page,
section 5): per-block norms, the norm-based range, the forward transform
with truncation and the inverse, against the oracle -- bit for bit except
the binary64 sums of squares, whose addition order differs (tree against
sequential) and which are held to a relative 1e-12."""
import statistics

import numpy as np
import pytest
import torch

import oracle
from gradient_all_reduce_worker_amd import _native as ga

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 0x0DDB_A11C_0FFE_E123


def _inputs(P, N, dt, seed, scale=0.01):
    rng = np.random.default_rng(seed)
    t = torch.from_numpy((rng.standard_normal((P, N)) * scale).astype(np.float32))
    if dt == ga.BF16:
        t = t.to(torch.bfloat16)
    return [t[i].clone().to(DEV) for i in range(P)]


def _host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


# one tile per block (d <= 4096, several blocks per tile), two passes (d > 4096),
# ragged tails, a single partial block, the largest d
SHAPES = [(2, 2, 7), (3, 8, 1001), (2, 128, 300), (4, 256, 5000), (2, 4096, 3 * 4096 + 5),
          (3, 8192, 2 * 8192 - 3), (2, 1 << 14, (1 << 14) + 77), (2, 1 << 16, 70000),
          (2, 1 << 20, (1 << 21) + 12345), (1, 1 << 22, (1 << 22) + 5), (2, 1 << 12, 100)]


@pytest.mark.parametrize("dt", [ga.F32, ga.BF16])
@pytest.mark.parametrize("P,d,N", SHAPES)
def test_forward_inverse_bit_exact(P, d, N, dt):
    bufs = _inputs(P, N, dt, seed=N + d)
    y = ga.thc_rht_forward(bufs, d, SEED)
    Np = ga.rht_padded(N, d)
    for i in range(P):
        want = oracle.rht_forward(_host(bufs[i]), d, SEED)
        assert want.size == Np
        assert np.array_equal(_bits(y[i].cpu().numpy()[:Np]), _bits(want)), i
    # inverse of an oracle-made vector, written as fp32 and as bf16
    yo = oracle.rht_forward(_host(bufs[0]), d, SEED)
    for out_dt, tdt in ((ga.F32, torch.float32), (ga.BF16, torch.bfloat16)):
        yd = torch.from_numpy(yo.copy()).to(DEV)
        out = ga.thc_rht_inverse(yd, N, d, SEED, out_dtype=tdt)
        want = oracle.rht_inverse(yo, d, SEED, out_dt)[:N]
        assert np.array_equal(_host(out)[:N], want), out_dt


@pytest.mark.parametrize("P,d,N", [(3, 8, 1001), (4, 4096, 3 * 4096 + 5), (2, 1 << 16, 70000),
                                   (2, 1 << 20, (1 << 21) + 12345)])
def test_truncation_and_range(P, d, N):
    bufs = _inputs(P, N, ga.F32, seed=7 * N)
    xs = [_host(b) for b in bufs]
    t_p = statistics.NormalDist().inv_cdf(1 - 1 / 64)
    S = ga.thc_rht_sumsq(bufs, d)
    Sw = np.stack([oracle.rht_sumsq(x, d) for x in xs])
    np.testing.assert_allclose(S.cpu().numpy(), Sw, rtol=1e-12, atol=0)
    # the range from the oracle's sums: bit for bit
    mM = ga.thc_rht_range(torch.from_numpy(Sw).to(DEV), d, t_p)
    mMw = oracle.rht_range(Sw, d, t_p)
    assert np.array_equal(_bits(mM.cpu().numpy()), _bits(mMw))
    y = ga.thc_rht_forward(bufs, d, SEED, mM=mM)
    clipped = 0
    for i in range(P):
        yo = oracle.rht_forward(xs[i], d, SEED)
        yc = oracle.clamp(yo, d, mMw)
        clipped += int(np.count_nonzero(yc != yo))
        assert np.array_equal(_bits(y[i].cpu().numpy()), _bits(yc)), i
    assert clipped > 0                 # the truncation did act on these inputs


def test_sumsq_and_range_edge_cases():
    d = 1 << 10
    # a zero vector gives a zero range; a single non-zero coordinate its magnitude
    z = [torch.zeros(3 * d, device=DEV), torch.zeros(3 * d, device=DEV)]
    z[1][d + 5] = -3.0
    S = ga.thc_rht_sumsq(z, d)
    assert S.cpu().numpy().tolist() == [[0.0, 0.0, 0.0], [0.0, 9.0, 0.0]]
    mM = ga.thc_rht_range(S, d, 2.0).cpu().numpy()
    assert mM[0].tolist() == [0.0, 0.0] and mM[2].tolist() == [0.0, 0.0]
    assert mM[1, 1] == np.float32(2.0 * 3.0 / 32.0) and mM[1, 0] == -mM[1, 1]
    # bf16 input, N not a multiple of d
    bufs = _inputs(2, 2 * d + 3, ga.BF16, seed=4)
    S = ga.thc_rht_sumsq(bufs, d).cpu().numpy()
    Sw = np.stack([oracle.rht_sumsq(_host(b), d) for b in bufs])
    np.testing.assert_allclose(S, Sw, rtol=1e-12, atol=0)


def test_empty_is_noop():
    e = [torch.empty(0, device=DEV)]
    ga.thc_rht_forward(e, 16, SEED, y=[torch.zeros(1, device=DEV)])
    ga.thc_rht_sumsq(e, 16)
    ga.thc_rht_inverse(torch.zeros(16, device=DEV), 0, 16, SEED, out=torch.zeros(1, device=DEV))
    torch.cuda.synchronize()


def test_inverse_undoes_forward():
    """(1/d) H H = I: the round trip returns x within binary32 rounding."""
    d, N = 1 << 16, 3 * (1 << 16) - 11
    x = _inputs(1, N, ga.F32, seed=12)
    y = ga.thc_rht_forward(x, d, SEED)[0]
    back = ga.thc_rht_inverse(y, N, d, SEED)
    err = (back - x[0]).abs().max().item()
    assert err <= 64 * np.finfo(np.float32).eps * x[0].abs().max().item()


@pytest.mark.parametrize("b", [2, 4, 8])
@pytest.mark.parametrize("P,d,N", [(4, 1 << 12, 50001), (3, 1 << 16, 3 * (1 << 16) + 999)])
def test_full_rht_chain_matches_oracle(P, d, N, b):
    """Norms -> range -> forward + truncation -> uniform THC on the
    transformed coordinates (one partition per block) -> integer sum ->
    average -> inverse, against the same chain in the oracle."""
    bufs = _inputs(P, N, ga.F32, seed=N + b)
    xs = [_host(t) for t in bufs]
    t_p = statistics.NormalDist().inv_cdf(1 - 1 / 64)
    qseed = 0xA5A5_0000_1234 + b
    Np = ga.rht_padded(N, d)

    S = ga.thc_rht_sumsq(bufs, d)
    mM = ga.thc_rht_range(S, d, t_p)
    y = ga.thc_rht_forward(bufs, d, SEED, mM=mM)
    packed = ga.thc_usq_quantize(y, mM, b, qseed, part_elems=d)
    Y = ga.thc_int_aggregate(packed, Np, b)
    avg = ga.thc_dequant(Y, Np, P, b, mM, part_elems=d)
    out = ga.thc_rht_inverse(avg, N, d, SEED)

    Sw = np.stack([oracle.rht_sumsq(x, d) for x in xs])
    mMw = oracle.rht_range(Sw, d, t_p)
    # the two sums differ in their last bits at most; the range rounds them
    # to binary32, where these seeded inputs agree
    assert np.array_equal(_bits(mM.cpu().numpy()), _bits(mMw))
    want_packed = []
    for i in range(P):
        yc = oracle.clamp(oracle.rht_forward(xs[i], d, SEED), d, mMw)
        wp = oracle.usq_quantize(yc, i, d, mMw, b, qseed)
        assert np.array_equal(packed[i].cpu().numpy(), wp), i
        want_packed.append(wp)
    Yw = oracle.int_aggregate(want_packed, Np, b)
    assert np.array_equal(Y.cpu().numpy()[:Np], Yw)
    avgw = oracle.dequant(Yw, P, b, d, mMw)
    outw = oracle.rht_inverse(avgw, d, SEED)[:N]
    assert np.array_equal(_bits(out.cpu().numpy()[:N]), _bits(outw))
    # and the estimate is close to the true average (unbiased quantizer;
    # error shrinks with b)
    mean = np.mean(np.stack(xs), axis=0, dtype=np.float64)
    nm = oracle.nmse(mean.astype(np.float32), outw)[2]
    assert nm < {2: 0.6, 4: 0.05, 8: 0.02}[b]


# transform-and-quantize in one call: partial groups of 8 (d < 8, Np not a
# multiple of 8), one tile, a full tile, two passes, several blocks per tile,
# and more blocks (P x Np / d = 90) than one chunk of the pipelined two-pass
# schedule holds (64), so its launches mix both passes
QSHAPES = [(2, 2, 7), (3, 2, 9), (2, 4, 13), (3, 8, 1001), (2, 128, 300), (4, 4096, 3 * 4096 + 5),
           (2, 8192, 2 * 8192 - 3), (2, 1 << 14, (1 << 14) + 77), (2, 1 << 16, 70000),
           (2, 1 << 20, (1 << 20) + 999), (3, 1 << 14, 30 * (1 << 14) - 5),
           (4, 1 << 14, 70 * (1 << 14) - 3)]          # 280 blocks: two pipeline chunks
QMODES = [(1, 0, None), (2, 0, None), (4, 0, None), (8, 0, None),
          (2, 8, (0, 3, 5, 8)), (4, 36, "center"), (8, 1000, "center")]


@pytest.mark.parametrize("dt", [ga.F32, ga.BF16])
@pytest.mark.parametrize("b,g,table", QMODES)
@pytest.mark.parametrize("P,d,N", QSHAPES)
def test_rht_quantize_matches_two_calls_and_oracle(P, d, N, b, g, table, dt):
    """thc_rht_quantize against thc_rht_forward (with truncation) followed by
    the quantizer on the transformed vector, and against the oracle's
    forward -> clamp -> quantize, byte for byte."""
    bufs = _inputs(P, N, dt, seed=3 * N + d + b)
    xs = [_host(t) for t in bufs]
    if table == "center":
        table = ga.center_table(b, g)
    t_p = statistics.NormalDist().inv_cdf(1 - 1 / 32)
    mMw = oracle.rht_range(np.stack([oracle.rht_sumsq(x, d) for x in xs]), d, t_p)
    mM = torch.from_numpy(mMw).to(DEV)
    qseed, w0 = 0x5EED_0000_0000_0077 + b, 5
    Np = ga.rht_padded(N, d)
    nbytes = ga.packed_bytes(Np, b)
    fused = ga.thc_rht_quantize(bufs, d, SEED, mM, b, qseed, worker0=w0, g=g, table=table)
    y = ga.thc_rht_forward(bufs, d, SEED, mM=mM)
    if table is None:
        two = ga.thc_usq_quantize(y, mM, b, qseed, part_elems=d, worker0=w0)
    else:
        two = ga.thc_nuhc_quantize(y, mM, b, g, table, qseed, part_elems=d, worker0=w0)
    for i in range(P):
        got = fused[i].cpu().numpy()[:nbytes]
        assert np.array_equal(got, two[i].cpu().numpy()[:nbytes]), i
        yc = oracle.clamp(oracle.rht_forward(xs[i], d, SEED), d, mMw)
        if table is None:
            want = oracle.usq_quantize(yc, w0 + i, d, mMw, b, qseed)
        else:
            want = oracle.nuhc_quantize(yc, w0 + i, d, mMw, b, g, table, qseed)
        assert np.array_equal(got, want), i


@pytest.mark.parametrize("table", [None, "center"])
@pytest.mark.parametrize("dbits", [15, 17, 18, 19, 21, 22])
def test_rht_quantize_every_column_width(dbits, table):
    """The two-pass call keeps the first pass's output column-blocked for the
    second (column groups of W = 2^(26 - dbits) values, W = 16 .. 2048): every
    block size that takes that path, with a ragged last block, byte for byte
    against the row-major forward transform followed by the quantizer, and
    against the oracle."""
    d = 1 << dbits
    P, N, b = 2, d + 4097, 4
    g = 36 if table else 0
    T = ga.center_table(b, g) if table else None
    bufs = _inputs(P, N, ga.F32, seed=dbits + 7)
    xs = [_host(t) for t in bufs]
    t_p = statistics.NormalDist().inv_cdf(1 - 1 / 32)
    mMw = oracle.rht_range(np.stack([oracle.rht_sumsq(x, d) for x in xs]), d, t_p)
    mM = torch.from_numpy(mMw).to(DEV)
    Np = ga.rht_padded(N, d)
    nbytes = ga.packed_bytes(Np, b)
    print(f"rht_quantize d=2^{dbits} N={N} table={table is not None}", flush=True)
    fused = ga.thc_rht_quantize(bufs, d, SEED, mM, b, 21, g=g, table=T)
    y = ga.thc_rht_forward(bufs, d, SEED, mM=mM)
    two = (ga.thc_usq_quantize(y, mM, b, 21, part_elems=d) if T is None else
           ga.thc_nuhc_quantize(y, mM, b, g, T, 21, part_elems=d))
    for i in range(P):
        got = fused[i].cpu().numpy()[:nbytes]
        assert np.array_equal(got, two[i].cpu().numpy()[:nbytes]), i
    yc = oracle.clamp(oracle.rht_forward(xs[0], d, SEED), d, mMw)
    want = (oracle.usq_quantize(yc, 0, d, mMw, b, 21) if T is None else
            oracle.nuhc_quantize(yc, 0, d, mMw, b, g, T, 21))
    assert np.array_equal(fused[0].cpu().numpy()[:nbytes], want)


def test_rht_quantize_caller_buffers_and_empty():
    """Caller-provided scratch and packed buffers (reused across calls), and
    N = 0 leaves the output untouched."""
    P, d, N, b = 2, 1 << 15, 3 * (1 << 15) - 100, 4
    bufs = _inputs(P, N, ga.F32, seed=99)
    Np = ga.rht_padded(N, d)
    mMw = oracle.rht_range(np.stack([oracle.rht_sumsq(_host(x), d) for x in bufs]), d, 2.0)
    mM = torch.from_numpy(mMw).to(DEV)
    ys = [torch.full((Np,), 7.0, device=DEV) for _ in range(P)]
    pk = [torch.zeros(ga.packed_bytes(Np, b), dtype=torch.uint8, device=DEV) for _ in range(P)]
    first = [t.clone() for t in ga.thc_rht_quantize(bufs, d, SEED, mM, b, 11, y_scratch=ys, packed=pk)]
    again = ga.thc_rht_quantize(bufs, d, SEED, mM, b, 11, y_scratch=ys, packed=pk)
    for i in range(P):
        assert torch.equal(first[i], again[i])
        want = oracle.usq_quantize(oracle.clamp(oracle.rht_forward(_host(bufs[i]), d, SEED), d, mMw),
                                   i, d, mMw, b, 11)
        assert np.array_equal(again[i].cpu().numpy(), want)
    keep = pk[0].clone()
    ga.thc_rht_quantize([torch.empty(0, device=DEV)], d, SEED, mM, b, 11, packed=[pk[0]])
    torch.cuda.synchronize()
    assert torch.equal(pk[0], keep)


@pytest.mark.parametrize("dt", [ga.F32, ga.BF16])
def test_misaligned_inputs_two_pass(dt):
    """Worker vectors that start one element past a 16-byte boundary take
    the element-wise loads of the first pass: same bits."""
    P, d, N = 2, 1 << 14, 3 * (1 << 14) - 7
    big = _inputs(P, N + 1, dt, seed=77)
    bufs = [t[1:] for t in big]
    xs = [_host(t) for t in bufs]
    mMw = oracle.rht_range(np.stack([oracle.rht_sumsq(x, d) for x in xs]), d, 2.0)
    mM = torch.from_numpy(mMw).to(DEV)
    y = ga.thc_rht_forward(bufs, d, SEED, mM=mM)
    pk = ga.thc_rht_quantize(bufs, d, SEED, mM, 4, 5)
    for i in range(P):
        yc = oracle.clamp(oracle.rht_forward(xs[i], d, SEED), d, mMw)
        assert np.array_equal(_bits(y[i].cpu().numpy()), _bits(yc)), i
        assert np.array_equal(pk[i].cpu().numpy(), oracle.usq_quantize(yc, i, d, mMw, 4, 5)), i


@pytest.mark.parametrize("table", [None, "center"])
def test_rht_quantize_max_workers(table):
    """64 workers (the largest P), two passes, two chunks of the pipelined
    schedule; every worker's indices against the oracle."""
    P, d, N, b = 64, 1 << 14, 2 * (1 << 14) - 3, 4
    g = 36 if table else 0
    T = ga.center_table(b, g) if table else None
    bufs = _inputs(P, N, ga.F32, seed=640)
    xs = [_host(t) for t in bufs]
    mMw = oracle.rht_range(np.stack([oracle.rht_sumsq(x, d) for x in xs]), d, 2.0)
    pk = ga.thc_rht_quantize(bufs, d, SEED, torch.from_numpy(mMw).to(DEV), b, 31, g=g, table=T)
    for i in range(P):
        yc = oracle.clamp(oracle.rht_forward(xs[i], d, SEED), d, mMw)
        want = (oracle.nuhc_quantize(yc, i, d, mMw, b, g, T, 31) if table
                else oracle.usq_quantize(yc, i, d, mMw, b, 31))
        assert np.array_equal(pk[i].cpu().numpy(), want), i


NSHAPES = [(2, 8, 1001), (3, 4096, 3 * 4096 + 5), (2, 1 << 14, (1 << 14) + 77),
           (3, 1 << 14, 30 * (1 << 14) - 5), (2, 1 << 20, (1 << 20) + 999), (64, 1 << 14, 3 * (1 << 14) - 9),
           (8, 1 << 14, 40 * (1 << 14) - 9), (33, 1 << 14, 20 * (1 << 14) + 5)]   # 2 and 3 pipeline chunks


@pytest.mark.parametrize("dt", [ga.F32, ga.BF16])
@pytest.mark.parametrize("b,g,table", [(4, 0, None), (4, 36, "center"), (2, 0, None)])
@pytest.mark.parametrize("P,d,N", NSHAPES)
def test_rht_norm_quantize_matches_three_calls(P, d, N, b, g, table, dt):
    """Norms, range and transform-and-quantize in one call against
    thc_rht_sumsq + thc_rht_range + thc_rht_quantize (range and indices bit
    for bit, sums within 1e-12) and against the oracle."""
    bufs = _inputs(P, N, dt, seed=5 * N + d + b)
    xs = [_host(t) for t in bufs]
    if table == "center":
        table = ga.center_table(b, g)
    t_p = statistics.NormalDist().inv_cdf(1 - 1 / 32)
    Np = ga.rht_padded(N, d)
    S1 = ga.thc_rht_sumsq(bufs, d)
    mM1 = ga.thc_rht_range(S1, d, t_p)
    pk1 = ga.thc_rht_quantize(bufs, d, SEED, mM1, b, 17, worker0=3, g=g, table=table)
    S2 = torch.empty_like(S1)
    pk2, mM2, _ = ga.thc_rht_norm_quantize(bufs, d, SEED, t_p, b, 17, worker0=3, g=g, table=table,
                                           sumsq=S2)
    np.testing.assert_allclose(S2.cpu().numpy(), S1.cpu().numpy(), rtol=1e-12, atol=0)
    assert np.array_equal(_bits(mM2.cpu().numpy()), _bits(mM1.cpu().numpy()))
    nbytes = ga.packed_bytes(Np, b)
    Sw = np.stack([oracle.rht_sumsq(x, d) for x in xs])
    mMw = oracle.rht_range(Sw, d, t_p)
    assert np.array_equal(_bits(mM2.cpu().numpy()), _bits(mMw))
    for i in range(P):
        got = pk2[i].cpu().numpy()[:nbytes]
        assert np.array_equal(got, pk1[i].cpu().numpy()[:nbytes]), i
        yc = oracle.clamp(oracle.rht_forward(xs[i], d, SEED), d, mMw)
        want = (oracle.nuhc_quantize(yc, 3 + i, d, mMw, b, g, table, 17) if table is not None
                else oracle.usq_quantize(yc, 3 + i, d, mMw, b, 17))
        assert np.array_equal(got, want), i
