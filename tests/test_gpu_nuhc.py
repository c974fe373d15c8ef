"""GPU parity for non-uniform THC (lookup tables; THC page section 4,
Algorithm 2): quantize, table-sum aggregate and dequant against the oracle,
bit for bit, for several tables including the page's example and identity
tables (which must give the uniform scheme's bytes)."""
import numpy as np
import pytest
import torch

import oracle
from gradient_all_reduce_worker_amd import _native as ga

pytestmark = pytest.mark.gpu
DEV = "cuda"

TABLES = [
    (2, 4, [0, 1, 3, 4]),                       # the page's T2
    (1, 5, [0, 5]),
    (2, 3, [0, 1, 2, 3]),                       # identity: uniform THC
    (4, 36, ga.center_table(4, 36)),
    (4, 15, list(range(16))),                   # identity
    (8, 300, ga.center_table(8, 300)),
    (8, 4095, ga.center_table(8, 4095)),
]


def _inputs(P, N, dt, seed):
    rng = np.random.default_rng(seed)
    t = torch.from_numpy((rng.standard_normal((P, N)) * 0.01).astype(np.float32))
    if dt == ga.BF16:
        t = t.to(torch.bfloat16)
    return [t[i].clone().to(DEV) for i in range(P)]


def _to_dev(h: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(h)).to(DEV)


def _host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


@pytest.mark.parametrize("b,g,T", TABLES)
@pytest.mark.parametrize("dt", [ga.F32, ga.BF16])
# the last shape holds enough coordinates (4 M) that the rare exact-division
# branch of the table rounding (about 1 in 2.6e5) is taken many times
@pytest.mark.parametrize("P,N,part", [(3, 70001, 1000), (4, 8192 * 5 + 100, 8192), (2, 17, 0),
                                      (8, 1 << 18, 1 << 16), (2, 1 << 21, 1 << 20)])
def test_nuhc_quantize_aggregate_dequant(P, N, part, dt, b, g, T):
    bufs = _inputs(P, N, dt, seed=N + b + g)
    seed = 0x1234_5678_9ABC_DEF0 + g
    # every stage starts from the oracle's values: its grid, its indices, its sums
    hosts = [_host(t) for t in bufs]
    mM_h = oracle.minmax(hosts, part)
    mM = _to_dev(mM_h)
    packed = ga.thc_nuhc_quantize(bufs, mM, b, g, T, seed, part_elems=part, worker0=2)
    want = []
    for i in range(P):
        w = oracle.nuhc_quantize(hosts[i], 2 + i, part, mM_h, b, g, T, seed)
        assert np.array_equal(packed[i].cpu().numpy(), w), i
        want.append(w)
    Y = ga.thc_nuhc_aggregate([_to_dev(w) for w in want], N, b, g, T)
    Yw = oracle.nuhc_aggregate(want, N, b, g, T)
    assert np.array_equal(Y.cpu().numpy()[:N], Yw)
    out_dtype = torch.float32 if dt == ga.F32 else torch.bfloat16
    xh = ga.thc_nuhc_dequant(_to_dev(Yw), N, P, g, mM, part_elems=part, out_dtype=out_dtype)
    assert np.array_equal(_host(xh)[:N], oracle.nuhc_dequant(Yw, P, g, part, mM_h, dt))


def test_identity_table_equals_uniform_on_gpu():
    P, N, part, b = 4, 100003, 4096, 4
    bufs = _inputs(P, N, ga.F32, seed=3)
    mM = ga.thc_minmax(bufs, part)
    u = ga.thc_usq_quantize(bufs, mM, b, 99, part_elems=part)
    n = ga.thc_nuhc_quantize(bufs, mM, b, 15, list(range(16)), 99, part_elems=part)
    for a, c in zip(u, n):
        assert torch.equal(a, c)
    S = ga.thc_int_aggregate(u, N, b)
    Y = ga.thc_nuhc_aggregate(u, N, b, 15, list(range(16)))
    assert torch.equal(S, Y)


def test_flat_partition_and_misaligned():
    P, N = 2, 3000
    big = _inputs(P, N + 1, ga.F32, seed=8)
    views = [v[1:] for v in big]
    for v in views:
        v[:1000] = 0.25
    mM_h = oracle.minmax([_host(v) for v in views], 1000)
    assert mM_h[0, 0] == mM_h[0, 1]
    T = [0, 1, 3, 4]
    packed = [torch.zeros(N * 2 // 8 + 1, dtype=torch.uint8, device=DEV)[1:] for _ in views]
    ga.thc_nuhc_quantize(views, _to_dev(mM_h), 2, 4, T, 5, part_elems=1000, packed=packed)
    for i in range(P):
        assert np.array_equal(packed[i].cpu().numpy(),
                              oracle.nuhc_quantize(_host(views[i]), i, 1000, mM_h, 2, 4, T, 5))
