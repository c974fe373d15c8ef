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
    bufs = _inputs(P, N, tdt, seed=N + P + b)
    dt = ga.F32 if tdt == torch.float32 else ga.BF16
    if table == "center":
        table = ga.center_table(b, g)
    mM = ga.thc_minmax(bufs, part)
    seed = 0x77 + b
    if table is None:
        packed = ga.thc_usq_quantize(bufs, mM, b, seed, part_elems=part)
        S1 = ga.thc_int_aggregate(packed, N, b)
        x1 = ga.thc_dequant(S1, N, P, b, mM, part_elems=part, out_dtype=tdt)
    else:
        packed = ga.thc_nuhc_quantize(bufs, mM, b, g, table, seed, part_elems=part)
        S1 = ga.thc_nuhc_aggregate(packed, N, b, g, table)
        x1 = ga.thc_nuhc_dequant(S1, N, P, g, mM, part_elems=part, out_dtype=tdt)
    ref = [t.clone() for t in bufs]
    ga.ga_ring_allreduce_sim(ref, ga.AVG, part)
    ws = torch.empty(ga.thc_nmse_ws_bytes(N), dtype=torch.uint8, device=DEV)
    n1 = ga.thc_nmse(ref[0], x1, torch.empty(3, dtype=torch.float64, device=DEV), ws)
    S2, x2, n2 = ga.thc_aggregate_dequant(packed, N, b, mM, part_elems=part, out_dtype=tdt, g=g,
                                          table=table, x_ref=ref[0])
    assert torch.equal(S1[:N], S2[:N])
    assert np.array_equal(_host(x1)[:N], _host(x2)[:N])
    a, c = n1.cpu().numpy(), n2.cpu().numpy()
    np.testing.assert_allclose(c, a, rtol=1e-12, atol=0)
    # the oracle on the same packed indices
    pk = [p.cpu().numpy() for p in packed]
    mMh = mM.cpu().numpy()
    if table is None:
        Sw = oracle.int_aggregate(pk, N, b)
        xw = oracle.dequant(Sw, P, b, part, mMh, dt)
    else:
        Sw = oracle.nuhc_aggregate(pk, N, b, g, table)
        xw = oracle.nuhc_dequant(Sw, P, g, part, mMh, dt)
    assert np.array_equal(S2.cpu().numpy()[:N], Sw)
    assert np.array_equal(_host(x2)[:N], xw)


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
    two levels): S and x̂ bit-exact, NMSE within 1e-12 of thc_nmse."""
    P, N, b, part = 2, 4096 * 4100 + 5, 4, 1 << 20
    bufs = _inputs(P, N, tdt, seed=11)
    mM = ga.thc_minmax(bufs, part)
    packed = ga.thc_usq_quantize(bufs, mM, b, 5, part_elems=part)
    S1 = ga.thc_int_aggregate(packed, N, b)
    x1 = ga.thc_dequant(S1, N, P, b, mM, part_elems=part, out_dtype=tdt)
    ref = [t.clone() for t in bufs]
    ga.ga_ring_allreduce_sim(ref, ga.AVG, part)
    ws = torch.empty(ga.thc_nmse_ws_bytes(N), dtype=torch.uint8, device=DEV)
    n1 = ga.thc_nmse(ref[0], x1, torch.empty(3, dtype=torch.float64, device=DEV), ws)
    S2, x2, n2 = ga.thc_aggregate_dequant(packed, N, b, mM, part_elems=part, out_dtype=tdt,
                                          x_ref=ref[0])
    assert torch.equal(S1[:N], S2[:N])
    assert np.array_equal(_host(x1)[:N], _host(x2)[:N])
    np.testing.assert_allclose(n2.cpu().numpy(), n1.cpu().numpy(), rtol=1e-12, atol=0)
