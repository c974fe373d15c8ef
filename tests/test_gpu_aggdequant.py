"""GPU parity for the fused server-and-worker pass (THC page, Algorithm 1
server sum and decoding, Algorithm 2 with a table, the NMSE of section 2):
thc_aggregate_dequant against the separate thc_int_aggregate /
thc_nuhc_aggregate, thc_dequant / thc_nuhc_dequant and thc_nmse calls (bit
for bit for the sums and the estimate; the NMSE sums within 1e-12) and
against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gradient_all_reduce_worker_amd import _native as ga

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(P, N, tdt, seed):
    rng = np.random.default_rng(seed)
    t = torch.from_numpy((rng.standard_normal((P, N)) * 0.01).astype(np.float32)).to(tdt)
    return [t[i].clone().to(DEV) for i in range(P)]


def _to_dev(h: np.ndarray, tdt=None) -> torch.Tensor:
    """A host array on the device; uint16 arrays are bf16 bit patterns when
    tdt is bfloat16."""
    t = torch.from_numpy(np.ascontiguousarray(h))
    if tdt == torch.bfloat16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(DEV)


def _host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


SHAPES = [(1, 1, 0), (2, 17, 0), (3, 1001, 100), (4, 4096 * 3 + 5, 4096), (8, 70001, 0),
          (5, 20000, 1000), (16, 1 << 18, 1 << 16), (64, 9999, 0), (8, 4096 * 40, 4096 * 8),
          (33, 2048 * 5 + 3, 0), (20, 8192 * 3, 8192)]
MODES = [(1, 0, None), (2, 0, None), (4, 0, None), (8, 0, None), (2, 8, (0, 3, 5, 8)),
         (4, 36, "center"), (8, 1000, "center")]


@pytest.mark.parametrize("tdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("b,g,table", MODES)
@pytest.mark.parametrize("P,N,part", SHAPES)
def test_fused_equals_separate_and_oracle(P, N, part, b, g, table, tdt):
    """Each stage's inputs come from the oracle: the quantizer gets the
    oracle's grid, the server-side calls get the oracle's packed indices and
    the oracle's ring average; every output is compared with the oracle's."""
    bufs = _inputs(P, N, tdt, seed=N + P + b)
    dt = ga.F32 if tdt == torch.float32 else ga.BF16
    if table == "center":
        table = ga.center_table(b, g)
    seed = 0x77 + b
    # the oracle's chain
    hosts = [_host(t) for t in bufs]
    mMh = oracle.minmax(hosts, part)
    if table is None:
        pk = [oracle.usq_quantize(hosts[i], i, part, mMh, b, seed) for i in range(P)]
        Sw = oracle.int_aggregate(pk, N, b)
        xw = oracle.dequant(Sw, P, b, part, mMh, dt)
    else:
        pk = [oracle.nuhc_quantize(hosts[i], i, part, mMh, b, g, table, seed) for i in range(P)]
        Sw = oracle.nuhc_aggregate(pk, N, b, g, table)
        xw = oracle.nuhc_dequant(Sw, P, g, part, mMh, dt)
    avg = [h.copy() for h in hosts]
    oracle.ring_fold(avg, op=oracle.AVG, part=part)
    nmw = oracle.nmse(avg[0], xw)
    # the quantizer on the oracle's grid
    mM = _to_dev(mMh)
    if table is None:
        packed = ga.thc_usq_quantize(bufs, mM, b, seed, part_elems=part)
    else:
        packed = ga.thc_nuhc_quantize(bufs, mM, b, g, table, seed, part_elems=part)
    for i in range(P):
        assert np.array_equal(packed[i].cpu().numpy(), pk[i]), i
    # the server side on the oracle's indices, the NMSE against the oracle's average
    pk_d = [_to_dev(p) for p in pk]
    ref = _to_dev(avg[0], tdt)
    if table is None:
        S1 = ga.thc_int_aggregate(pk_d, N, b)
        x1 = ga.thc_dequant(S1, N, P, b, mM, part_elems=part, out_dtype=tdt)
    else:
        S1 = ga.thc_nuhc_aggregate(pk_d, N, b, g, table)
        x1 = ga.thc_nuhc_dequant(S1, N, P, g, mM, part_elems=part, out_dtype=tdt)
    ws = torch.empty(ga.thc_nmse_ws_bytes(N), dtype=torch.uint8, device=DEV)
    n1 = ga.thc_nmse(ref, x1, torch.empty(3, dtype=torch.float64, device=DEV), ws)
    S2, x2, n2 = ga.thc_aggregate_dequant(pk_d, N, b, mM, part_elems=part, out_dtype=tdt, g=g,
                                          table=table, x_ref=ref)
    assert np.array_equal(S1.cpu().numpy()[:N], Sw)
    assert np.array_equal(S2.cpu().numpy()[:N], Sw)
    assert np.array_equal(_host(x1)[:N], xw)
    assert np.array_equal(_host(x2)[:N], xw)
    a, c = n1.cpu().numpy(), n2.cpu().numpy()
    np.testing.assert_allclose(c, a, rtol=1e-12, atol=0)
    for got in (a, c):
        for k in range(3):
            assert abs(got[k] - nmw[k]) <= 1e-6 * abs(nmw[k]), (k, got, nmw)


def test_without_sum_or_nmse_and_misaligned():
    P, N, b = 4, 50001, 4
    bufs = _inputs(P, N, torch.float32, seed=5)
    mM = ga.thc_minmax(bufs, 0)
    packed = ga.thc_usq_quantize(bufs, mM, b, 3)
    S1 = ga.thc_int_aggregate(packed, N, b)
    x1 = ga.thc_dequant(S1, N, P, b, mM)
    S2, x2, n2 = ga.thc_aggregate_dequant(packed, N, b, mM, keep_sum=False)
    assert S2 is None and n2 is None and torch.equal(x1[:N], x2[:N])
    # output and reference one element past a 16-byte boundary: element paths
    big = torch.zeros(N + 1, device=DEV)
    ref = torch.zeros(N + 1, device=DEV)
    ref[1:] = bufs[0]
    _, x3, n3 = ga.thc_aggregate_dequant(packed, N, b, mM, x_ref=ref[1:], out=big[1:])
    assert torch.equal(x1[:N], x3[:N])
    num = float(((bufs[0].double() - x1[:N].double()) ** 2).sum())
    assert abs(n3[0].item() - num) <= 1e-9 * num


def test_empty_writes_zero_nmse():
    mM = torch.zeros((1, 2), device=DEV)
    packed = [torch.zeros(1, dtype=torch.uint8, device=DEV)]
    ref = torch.zeros(1, device=DEV)
    nm = torch.full((3,), 7.0, dtype=torch.float64, device=DEV)
    ga.thc_aggregate_dequant(packed, 0, 2, mM, x_ref=ref, nmse_out=nm)
    torch.cuda.synchronize()
    assert nm.cpu().numpy().tolist() == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("tdt", [torch.float32, torch.bfloat16])
def test_many_spans_two_level_nmse(tdt):
    """More spans than one partial group (the NMSE partials are summed in
    two levels), on the oracle's indices and average: S and x̂ bit-exact
    against the oracle, NMSE within 1e-6 of the oracle's and within 1e-12 of
    thc_nmse on the same estimate."""
    P, N, b, part = 2, 4096 * 4100 + 5, 4, 1 << 20
    dt = ga.F32 if tdt == torch.float32 else ga.BF16
    bufs = _inputs(P, N, tdt, seed=11)
    hosts = [_host(t) for t in bufs]
    mMh = oracle.minmax(hosts, part)
    pk = [oracle.usq_quantize(hosts[i], i, part, mMh, b, 5) for i in range(P)]
    Sw = oracle.int_aggregate(pk, N, b)
    xw = oracle.dequant(Sw, P, b, part, mMh, dt)
    avg = [h.copy() for h in hosts]
    oracle.ring_fold(avg, op=oracle.AVG, part=part)
    nmw = oracle.nmse(avg[0], xw)
    ref = _to_dev(avg[0], tdt)
    S2, x2, n2 = ga.thc_aggregate_dequant([_to_dev(p) for p in pk], N, b, _to_dev(mMh),
                                          part_elems=part, out_dtype=tdt, x_ref=ref)
    assert np.array_equal(S2.cpu().numpy()[:N], Sw)
    assert np.array_equal(_host(x2)[:N], xw)
    ws = torch.empty(ga.thc_nmse_ws_bytes(N), dtype=torch.uint8, device=DEV)
    n1 = ga.thc_nmse(ref, x2, torch.empty(3, dtype=torch.float64, device=DEV), ws)
    np.testing.assert_allclose(n2.cpu().numpy(), n1.cpu().numpy(), rtol=1e-12, atol=0)
    for k in range(3):
        assert abs(n2[k].item() - nmw[k]) <= 1e-6 * abs(nmw[k]), k
