"""Parity at the workloads' full sizes, through the same pipeline (and so the
same launch configuration) that bench.py times.

small, fusion, resnet101: every output element of every worker against the
oracle. vgg16 (32 x 138M fp32) and shard (8 x 2^31 bf16):
  * every partition's grid extremes (and, for vgg16, the error-feedback
    grids and the RHT ranges of every block) against the oracle, streamed
    partition by partition over a thread pool; the whole-vector grid is the
    extreme of the oracle's partition extremes (the THC page's preliminary
    round takes local extremes, then global ones);
  * 16 evenly spaced partitions, first and last included, element by
    element for every stage -- packed indices, ring average, integer sums,
    dequantized values -- with every oracle stage fed the oracle's own
    previous output;
  * the whole-vector NMSE against an fp64 torch evaluation of its definition
    on the same outputs, and all workers' averages bitwise equal.
"""
import gc
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from gradient_all_reduce_worker_amd import _native as ga
from gradient_all_reduce_worker_amd import synth
from gradient_all_reduce_worker_amd.pipeline import Pipeline, t_p

pytestmark = pytest.mark.gpu

# oracle calls release the interpreter lock (ctypes), so threads run them in
# parallel; at most 16 threads, one GPU's share of a host
POOL = max(1, min(16, len(os.sched_getaffinity(0))))
N_SAMPLED = 16


def _u(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _check_partition(w, P, lo, xs, got, mMg, nu_tables=None, arrived=None):
    """Oracle on one partition [lo, lo + n) of a flat workload (first step:
    error-feedback residuals start at zero); mMg is the oracle's grid of the
    whole vector."""
    n = xs[0].size
    xs = [x.copy() for x in xs]
    for b in w.ef_bits:
        k = f"ef{b}"
        xe = [oracle.ef_add(x, np.zeros(n, dtype=np.float32)) for x in xs]
        mMe = oracle.minmax(xe, n)
        assert np.array_equal(got["mM_ef"][k].view(np.uint32), mMe[0].view(np.uint32)), k
        pk = [oracle.usq_quantize(xe[i], i, n, mMe, b, w.quant_seed, e_offset=lo) for i in range(P)]
        for i in range(P):
            assert np.array_equal(got["packed"][k][i], pk[i]), (k, i)
            ew = oracle.ef_update(xe[i], pk[i], b, n, mMe)
            assert np.array_equal(got["err"][k][i].view(np.uint32), ew.view(np.uint32)), (k, i)
        S = oracle.int_aggregate(pk, n, b)
        assert np.array_equal(got["S"][k], S), k
        assert np.array_equal(_u(got["xhat"][k]), _u(oracle.dequant(S, P, b, n, mMe, w.dtype))), k
    mM = oracle.minmax(xs, n)
    assert np.array_equal(got["mM"].view(np.uint32), mM[0].view(np.uint32))
    packed = {}
    for b in w.thc_bits:
        packed[b] = [oracle.usq_quantize(xs[i], i, n, mM, b, w.quant_seed, e_offset=lo)
                     for i in range(P)]
        for i in range(P):
            assert np.array_equal(got["packed"][b][i], packed[b][i]), (b, i)
    for b in w.global_bits:
        k = f"g{b}"
        packed[k] = [oracle.usq_quantize(xs[i], i, 0, mMg, b, w.quant_seed, e_offset=lo)
                     for i in range(P)]
        for i in range(P):
            assert np.array_equal(got["packed"][k][i], packed[k][i]), (k, i)
    for k, (b, g, T) in (nu_tables or {}).items():
        packed[k] = [oracle.nuhc_quantize(xs[i], i, n, mM, b, g, T, w.quant_seed, e_offset=lo)
                     for i in range(P)]
        for i in range(P):
            assert np.array_equal(got["packed"][k][i], packed[k][i]), (k, i)
    oracle.ring_fold(xs, op=oracle.AVG, part=n)
    for i in range(P):
        assert np.array_equal(_u(got["ring"][i]), _u(xs[i])), i
    for b in w.thc_bits:
        S = oracle.int_aggregate(packed[b], n, b)
        assert np.array_equal(got["S"][b], S)
        xh = oracle.dequant(S, P, b, n, mM, w.dtype)
        assert np.array_equal(_u(got["xhat"][b]), _u(xh))
    for b in w.global_bits:
        k = f"g{b}"
        S = oracle.int_aggregate(packed[k], n, b)
        assert np.array_equal(got["S"][k], S), k
        assert np.array_equal(_u(got["xhat"][k]), _u(oracle.dequant(S, P, b, 0, mMg, w.dtype))), k
    if arrived is not None and len(arrived) < P and w.thc_bits:
        b = w.thc_bits[0]
        k = f"part{b}"
        S = oracle.int_aggregate([packed[b][i] for i in arrived], n, b)
        assert np.array_equal(got["S"][k], S), k
        xh = oracle.dequant(S, len(arrived), b, n, mM, w.dtype)
        assert np.array_equal(_u(got["xhat"][k]), _u(xh)), k
    for k, (b, g, T) in (nu_tables or {}).items():
        Y = oracle.nuhc_aggregate(packed[k], n, b, g, T)
        assert np.array_equal(got["S"][k], Y), k
        xh = oracle.nuhc_dequant(Y, P, g, n, mM, w.dtype)
        assert np.array_equal(_u(got["xhat"][k]), _u(xh)), k


def _check_rht_block(pipe, key, p, xs, got):
    """Oracle on block p of an RHT pass: norms, range, transform with
    truncation, table quantizer, table sums, dequant, inverse."""
    b, g, d, T = pipe.rht[key]
    w, P, lo = pipe.w, pipe.P, p * d
    S2 = np.stack([oracle.rht_sumsq(x, d) for x in xs])
    mM = oracle.rht_range(S2, d, t_p(w.rht_p))
    # binary64 sums in another order, rounded to the same binary32 range
    assert np.array_equal(got["mM"].view(np.uint32), mM[0].view(np.uint32)), key
    packed = []
    for i in range(P):
        y = oracle.clamp(oracle.rht_forward(xs[i], d, w.rht_seed, e0=lo), d, mM)
        packed.append(oracle.nuhc_quantize(y, i, d, mM, b, g, T, w.quant_seed, e_offset=lo))
        assert np.array_equal(got["packed"][i], packed[i]), (key, i)
    Y = oracle.nuhc_aggregate(packed, d, b, g, T)
    assert np.array_equal(got["S"], Y), key
    avg = oracle.nuhc_dequant(Y, P, g, d, mM)
    xh = oracle.rht_inverse(avg, d, w.rht_seed, w.dtype, e0=lo)[:xs[0].size]
    assert np.array_equal(_u(got["xhat"]), _u(xh)), key


def _nmse_property(pipe, slab=1 << 26):
    for b in pipe.xhat:
        num = den = 0.0
        for lo in range(0, pipe.N, slab):
            x = pipe.flat[0][lo:lo + slab].double()
            xh = pipe.xhat[b][lo:lo + slab].double()
            num += float(((x - xh) ** 2).sum())
            den += float((x * x).sum())
        got = pipe.nmse[b].cpu().numpy()
        assert abs(got[0] - num) <= 1e-6 * num and abs(got[1] - den) <= 1e-6 * den
        assert abs(got[2] - num / den) <= 1e-6 * (num / den)


def _sampled(n_part: int):
    """N_SAMPLED evenly spaced partitions, the first and the last included."""
    k = min(N_SAMPLED, n_part)
    return sorted({round(j * (n_part - 1) / max(k - 1, 1)) for j in range(k)})


def _oracle_grids(pipe, keep):
    """The oracle over every partition of the pristine gradients: its grid
    per partition, the error-feedback grid (residuals zero) and, per RHT pass,
    the range of every block. Partitions are copied to the host a slab at a
    time and handed to a thread pool; the inputs of the partitions in `keep`
    are returned for the element-by-element checks."""
    w, P, N = pipe.w, pipe.P, pipe.N
    plen = w.part_elems
    n_part = pipe.n_partitions()
    es = w.elem_bytes
    grid = np.empty((n_part, 2), dtype=np.float32)
    ef = {f"ef{b}": np.empty((n_part, 2), dtype=np.float32) for b in w.ef_bits}
    rht = {k: np.empty((n_part, 2), dtype=np.float32) for k in pipe.rht}
    tp = t_p(w.rht_p)
    kept = {}

    def job(p, xs):
        n = xs[0].size
        grid[p] = oracle.minmax(xs, n)[0]
        if ef:
            zero = np.zeros(n, dtype=np.float32)
            g = oracle.minmax([oracle.ef_add(x, zero) for x in xs], n)[0]
            for k in ef:
                ef[k][p] = g
        for k, (_, _, d, _) in pipe.rht.items():
            assert d == plen                 # RHT blocks are the partitions
            S2 = np.stack([oracle.rht_sumsq(x, d) for x in xs])
            rht[k][p] = oracle.rht_range(S2, d, tp)[0]

    per_slab = max(1, (1 << 30) // (P * plen * es))     # about 1 GiB of inputs per slab
    with ThreadPoolExecutor(POOL) as ex:
        for p0 in range(0, n_part, per_slab):
            p1 = min(p0 + per_slab, n_part)
            lo, hi = p0 * plen, min(p1 * plen, N)
            slab = [synth.to_numpy_bits(pipe.flat[i][lo:hi]) for i in range(P)]
            futs = []
            for p in range(p0, p1):
                a, c = p * plen - lo, min((p + 1) * plen, N) - lo
                xs = [np.ascontiguousarray(x[a:c]) for x in slab]
                if p in keep:
                    kept[p] = [x.copy() for x in xs]
                futs.append(ex.submit(job, p, xs))
            for f in futs:
                f.result()
    return grid, ef, rht, kept


@pytest.mark.parametrize("name", ["vgg16", "shard"])
def test_flat_workload_sampled(name):
    pipe = Pipeline(name)
    print(f"workload {name}: P={pipe.P} N={pipe.N}", flush=True)
    pipe.setup()
    n_part = pipe.n_partitions()
    which = _sampled(n_part)
    grid, ef, rht, before = _oracle_grids(pipe, set(which))
    print(f"oracle grids of {n_part} partitions done", flush=True)
    pipe.step()
    torch.cuda.synchronize()
    # every partition's grid, bit for bit
    assert np.array_equal(pipe.mM.cpu().numpy().view(np.uint32), grid.view(np.uint32))
    for k, g in ef.items():
        assert np.array_equal(pipe.mM_ef[k].cpu().numpy().view(np.uint32), g.view(np.uint32)), k
    for k, g in rht.items():
        assert np.array_equal(pipe.rht_mM[k].cpu().numpy().view(np.uint32), g.view(np.uint32)), k
    # the whole vector's grid: global extremes of the oracle's local ones
    mMg = np.array([[grid[:, 0].min(), grid[:, 1].max()]], dtype=np.float32)
    if pipe.w.global_bits:
        assert np.array_equal(pipe.mM_g.cpu().numpy().view(np.uint32), mMg.view(np.uint32))
    after = pipe.sample_outputs(which)
    rht_after = {key: pipe.sample_rht_outputs(key, which) for key in pipe.rht}
    plen = pipe.w.part_elems

    def check(p):
        _check_partition(pipe.w, pipe.P, p * plen, before[p], after[p], mMg, pipe.nu_tables,
                         pipe.arrived)
        for key in pipe.rht:
            _check_rht_block(pipe, key, p, before[p], rht_after[key][p])
        return p

    with ThreadPoolExecutor(POOL) as ex:
        done = list(ex.map(check, which))
    assert done == which
    print(f"{len(which)} partitions checked element by element", flush=True)
    # all workers end with identical averages (every worker of the sampled
    # partitions was compared above; here, whole buffers on device)
    for i in range(1, pipe.P):
        assert torch.equal(pipe.flat[i].view(torch.int16 if pipe.w.dtype else torch.int32),
                           pipe.flat[0].view(torch.int16 if pipe.w.dtype else torch.int32))
    _nmse_property(pipe)
    S_max = max(int(pipe.S[b].max()) for b in pipe.w.thc_bits)
    assert S_max <= pipe.P * ((1 << max(pipe.w.thc_bits)) - 1)


def test_small_workload_full():
    pipe = Pipeline("small")
    pipe.setup()
    xs = pipe.sample_inputs([0])[0]
    pipe.step()
    torch.cuda.synchronize()
    got = pipe.sample_outputs([0])[0]
    _check_partition(pipe.w, pipe.P, 0, xs, got, oracle.minmax(xs, 0))
    ref = [x.copy() for x in xs]
    oracle.ring_fold(ref, op=oracle.AVG, part=0)
    nm = oracle.nmse(ref[0], oracle.dequant(got["S"][4], 4, 4, 0, got["mM"][None, :]))
    assert abs(pipe.nmse[4].cpu().numpy()[2] - nm[2]) <= 1e-6 * nm[2]


@pytest.mark.parametrize("zero_copy", [True, False])
@pytest.mark.parametrize("name", ["fusion", "resnet101"])
def test_fused_workload_full(name, zero_copy):
    pipe = Pipeline(name, zero_copy=zero_copy)
    print(f"workload {name}: P={pipe.P} N={pipe.N}", flush=True)
    pipe.setup()
    w = pipe.w
    host = [[synth.to_numpy_bits(t) for t in pipe.tensors[i]] for i in range(pipe.P)]
    pipe.step()
    torch.cuda.synchronize()
    buf_of, off_of, fill, _ = oracle.fuse_plan(w.sizes, [0] * len(w.sizes), 64 << 20)
    assert (buf_of, off_of, fill) == (pipe.buf_of, pipe.off_of, pipe.fill)
    fused = [oracle.fuse_pack(host[i], buf_of, off_of, fill, np.float32) for i in range(pipe.P)]
    for k in range(len(fill)):
        oracle.ring_fold([fused[i][k] for i in range(pipe.P)], op=oracle.AVG, part=0)
    for i in range(pipe.P):
        out = oracle.fuse_unpack(fused[i], buf_of, off_of, w.sizes)
        for t in range(len(w.sizes)):
            got = synth.to_numpy_bits(pipe.tensors[i][t])
            assert np.array_equal(got.view(np.uint32), out[t].view(np.uint32)), (i, t)


def test_shard_stepwise_staged():
    """The shard's shape (8 x 2^31 bf16, partitions of 2^20) through the
    stepwise schedule with binary32 partials staged between steps: all
    workers bitwise equal, and 16 evenly spaced partitions against the
    oracle's fold element by element."""
    P, N, part = 8, 1 << 31, 1 << 20
    print(f"staged stepwise P={P} N={N} bf16 part={part}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    bufs = [torch.randn(N, generator=g, device="cuda", dtype=torch.bfloat16) * (2.0 ** (i - 4))
            for i in range(P)]
    which = _sampled(N // part)
    before = {p: [x[p * part:(p + 1) * part].cpu().view(torch.int16).numpy().view(np.uint16).copy()
                  for x in bufs] for p in which}
    st = ga.ga_ring_stepwise_staged(bufs, op=ga.AVG, part_elems=part)
    torch.cuda.synchronize()
    assert st["launches"] == 2 * (P - 1)
    for i in range(1, P):
        assert torch.equal(bufs[i].view(torch.int16), bufs[0].view(torch.int16)), i
    for p in which:
        ref = before[p]
        oracle.ring_fold(ref, op=oracle.AVG, part=part)
        got = bufs[0][p * part:(p + 1) * part].cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref[0]), p
