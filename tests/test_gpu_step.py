"""GPU parity for thc_ring_step, the one-read pass that quantizes every
worker's gradient (THC page, section 3), sums the indices and decodes the
average with its NMSE (Algorithm 1; section 2) and leaves the ring's
average in every buffer (Horovod page, section 3.4; ring lesson, sections 4
and 7): every output against the oracle's chain on the same inputs (the
oracle's grid, its indices, its sums, its fold), and against the separate
GPU calls, bit for bit; the NMSE within 1e-6 of the oracle's and 1e-12 of
thc_nmse on the same outputs."""
import numpy as np
import pytest
import torch

import oracle
from gradient_all_reduce_worker_amd import _native as ga

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(P, N, tdt, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((P, N)) * np.exp(rng.uniform(-3, 3, size=(P, 1)))
    t = torch.from_numpy(x.astype(np.float32)).to(tdt)
    return [t[i].clone().to(DEV) for i in range(P)]


def _host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def _to_dev(h, tdt=None):
    t = torch.from_numpy(np.ascontiguousarray(h))
    if tdt == torch.bfloat16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(DEV)


def _u(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


# (P, N, ring_part, q_part): one partition; ragged chunks that straddle
# workgroups (C = ceil(n / P) not a multiple of 2048); chunk boundaries on
# workgroup boundaries; several ring partitions with a short last one;
# quantizer partitions smaller and larger than the ring's; one worker; the
# largest P
SHAPES = [(1, 4096, 0, 0), (2, 8, 0, 0), (3, 2048 * 3 + 40, 0, 0), (4, 1 << 20, 1 << 20, 1 << 20),
          (5, 70000, 1000, 4000), (8, 2048 * 8 * 4, 0, 2048), (8, (1 << 18) + 8 * 333, 1 << 16, 1 << 14),
          (13, 20008, 0, 512), (16, 100000, 8192, 0), (17, 4096 * 5, 0, 4096), (32, 12344, 0, 8),
          (64, 4096 * 3, 2048, 0)]


@pytest.mark.parametrize("tdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("b", [1, 2, 4, 8])
@pytest.mark.parametrize("P,N,rpart,qpart", SHAPES)
def test_step_matches_oracle_chain(P, N, rpart, qpart, b, tdt):
    print(f"thc_ring_step P={P} N={N} ring_part={rpart} q_part={qpart} b={b} {tdt}", flush=True)
    dt = ga.F32 if tdt == torch.float32 else ga.BF16
    bufs = _inputs(P, N, tdt, seed=N + P + 10 * b)
    hosts = [_host(t) for t in bufs]
    seed, w0 = 0x5EED_0000_1234_0000 + b, 3
    # the oracle's chain
    mMh = oracle.minmax(hosts, qpart)
    pk = [oracle.usq_quantize(hosts[i], w0 + i, qpart, mMh, b, seed) for i in range(P)]
    Sw = oracle.int_aggregate(pk, N, b)
    xw = oracle.dequant(Sw, P, b, qpart, mMh, dt)
    avg = [h.copy() for h in hosts]
    oracle.ring_fold(avg, op=oracle.AVG, part=rpart)
    nmw = oracle.nmse(avg[0], xw)
    # the separate GPU calls on copies
    sep = [t.clone() for t in bufs]
    mM = _to_dev(mMh)
    p1 = ga.thc_usq_quantize(sep, mM, b, seed, part_elems=qpart, worker0=w0)
    ga.ga_ring_allreduce_sim(sep, ga.AVG, rpart)
    S1, x1, n1 = ga.thc_aggregate_dequant(p1, N, b, mM, part_elems=qpart, out_dtype=tdt, x_ref=sep[0])
    # the one-read pass
    p2, S2, x2, n2 = ga.thc_ring_step(bufs, mM, b, seed, ring_part=rpart, q_part=qpart, worker0=w0)
    torch.cuda.synchronize()
    nb = ga.packed_bytes(N, b)
    for i in range(P):
        got = p2[i].cpu().numpy()[:nb]
        assert np.array_equal(got, pk[i]), ("packed", i)
        assert np.array_equal(got, p1[i].cpu().numpy()[:nb]), ("packed vs separate", i)
        assert np.array_equal(_u(_host(bufs[i])), _u(avg[i])), ("ring average", i)
        assert torch.equal(bufs[i].view(torch.int16 if dt else torch.int32),
                           sep[i].view(torch.int16 if dt else torch.int32)), ("average vs separate", i)
    assert np.array_equal(S2.cpu().numpy()[:N], Sw)
    assert torch.equal(S2[:N], S1[:N])
    assert np.array_equal(_u(_host(x2)[:N]), _u(xw))
    assert np.array_equal(_u(_host(x2)[:N]), _u(_host(x1)[:N]))
    got = n2.cpu().numpy()
    np.testing.assert_allclose(got, n1.cpu().numpy(), rtol=1e-12, atol=0)
    for k in range(3):
        assert abs(got[k] - nmw[k]) <= 1e-6 * abs(nmw[k]), (k, got, nmw)


@pytest.mark.parametrize("tdt", [torch.float32, torch.bfloat16])
def test_step_two_level_nmse_and_optional_outputs(tdt):
    """More workgroups than one partial group (the NMSE partials are summed
    in two levels); the same outputs when the packed indices, the sums or the
    NMSE are not asked for."""
    P, N, b, part = 2, 8 * 256 * 4100 + 64, 4, 1 << 20
    dt = ga.F32 if tdt == torch.float32 else ga.BF16
    bufs = _inputs(P, N, tdt, seed=7)
    hosts = [_host(t) for t in bufs]
    mMh = oracle.minmax(hosts, part)
    pk = [oracle.usq_quantize(hosts[i], i, part, mMh, b, 9) for i in range(P)]
    Sw = oracle.int_aggregate(pk, N, b)
    xw = oracle.dequant(Sw, P, b, part, mMh, dt)
    avg = [h.copy() for h in hosts]
    oracle.ring_fold(avg, op=oracle.AVG, part=part)
    nmw = oracle.nmse(avg[0], xw)
    mM = _to_dev(mMh)
    again = [t.clone() for t in bufs]
    p2, S2, x2, n2 = ga.thc_ring_step(bufs, mM, b, 9, ring_part=part, q_part=part)
    _, s3, x3, n3 = ga.thc_ring_step(again, mM, b, 9, ring_part=part, q_part=part, keep_packed=False,
                                     keep_sum=False, with_nmse=False)
    torch.cuda.synchronize()
    assert s3 is None and n3 is None
    assert np.array_equal(_u(_host(x2)[:N]), _u(xw)) and torch.equal(x2, x3)
    assert np.array_equal(S2.cpu().numpy()[:N], Sw)
    for i in range(P):
        assert np.array_equal(p2[i].cpu().numpy()[:ga.packed_bytes(N, b)], pk[i]), i
        assert np.array_equal(_u(_host(bufs[i])), _u(avg[i])), i
        assert torch.equal(bufs[i], again[i]), i
    got = n2.cpu().numpy()
    for k in range(3):
        assert abs(got[k] - nmw[k]) <= 1e-6 * abs(nmw[k]), k


def _tie_inputs(P, N):
    """bf16 workers whose average lies exactly halfway between two bf16
    values: every worker holds v and one (element e's worker e mod P) holds v
    plus P/2 units in the last place, so the binary32 fold is exact and the
    average is v + half a unit. Element kinds by e mod 6: near 1 and near -1,
    subnormal (k * 2^-133) positive and negative, -0 in every worker, near
    2^100; v's last bit alternates, so both ties to even (down and up) occur."""
    e = np.arange(N)
    kind, a = e % 6, (e // 6) % (128 - P // 2)
    v = np.select([kind == 0, kind == 1, kind == 2, kind == 3, kind == 4],
                  [0x3F80 + a, 0xBF80 + a, 1 + a, 0x8001 + a, 0x8000], 0x7180 + a).astype(np.uint16)
    bump = np.where(kind == 4, 0, P // 2).astype(np.uint16)
    return [np.where(e % P == w, v + bump, v).astype(np.uint16) for w in range(P)]


@pytest.mark.parametrize("P", [2, 8, 16])
def test_step_bf16_average_rounds_ties_to_even(P):
    """The pass narrows the binary32 average and estimate to bf16 in
    hardware; on exact ties, subnormals and -0 it gives the oracle's
    round-to-nearest-even bits and the separate ring's."""
    N, b, seed = 6 * 2048 * 4, 2, 77
    print(f"thc_ring_step ties P={P} N={N}", flush=True)
    hosts = _tie_inputs(P, N)
    exact = sum(oracle.bf16_to_f32(h).astype(np.float64) for h in hosts) / P
    low = exact.astype(np.float32).view(np.uint32) & 0xFFFF
    kind = np.arange(N) % 6
    assert np.all(low[kind != 4] == 0x8000)                   # every non-zero element is a tie
    mMh = oracle.minmax(hosts, 0)
    pk = [oracle.usq_quantize(hosts[i], i, 0, mMh, b, seed) for i in range(P)]
    Sw = oracle.int_aggregate(pk, N, b)
    xw = oracle.dequant(Sw, P, b, 0, mMh, oracle.BF16)
    avg = [h.copy() for h in hosts]
    oracle.ring_fold(avg, op=oracle.AVG, part=0)
    kept = (exact.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    up = avg[0] != kept
    assert up[kind != 4].any() and (~up[kind != 4]).any()     # ties rounded both ways
    assert np.array_equal(avg[0][kind == 4], np.full((kind == 4).sum(), 0x8000, np.uint16))
    bufs = [_to_dev(h, torch.bfloat16) for h in hosts]
    sep = [t.clone() for t in bufs]
    mM = _to_dev(mMh)
    ga.ga_ring_allreduce_sim(sep, ga.AVG)
    _, S2, x2, _ = ga.thc_ring_step(bufs, mM, b, seed)
    torch.cuda.synchronize()
    for i in range(P):
        assert np.array_equal(_host(bufs[i]), avg[i]), i
        assert np.array_equal(_host(sep[i]), avg[i]), i
    assert np.array_equal(S2.cpu().numpy()[:N], Sw)
    assert np.array_equal(_host(x2)[:N], xw)


def test_step_refuses_what_it_does_not_cover():
    bufs = _inputs(2, 1004, torch.float32, seed=1)           # N not a multiple of 8
    mM = torch.zeros((1, 2), device=DEV)
    with pytest.raises(ga.GAError) as e:
        ga.thc_ring_step(bufs, mM, 4, 1)
    assert e.value.status == -2
    bufs = _inputs(2, 1000, torch.float32, seed=1)
    with pytest.raises(ga.GAError) as e:
        ga.thc_ring_step(bufs, mM, 4, 1, q_part=1004)          # quantizer partition
    assert e.value.status == -2
    big = _inputs(2, 1001, torch.float32, seed=2)
    with pytest.raises(ga.GAError) as e:
        ga.thc_ring_step([t[1:] for t in big], mM, 4, 1)      # not 16-byte aligned
    assert e.value.status == -1
    with pytest.raises(ga.GAError):
        ga.thc_ring_step(bufs, mM, 3, 1)                       # b
    empty = [torch.empty(0, device=DEV), torch.empty(0, device=DEV)]
    ga.thc_ring_step(empty, mM, 4, 1)                          # N = 0: nothing to do
