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
