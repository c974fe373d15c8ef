"""The kernels' 64-bit index paths and folded launch grids on the GPU,
against the oracle.

A dispatch holds each grid dimension as a 32-bit count of work-items, so a
kernel whose workgroup count grows with N spreads more than (2^32 - 1) / 256
workgroups over grid x and z. The cases:

* the ring's chunk arithmetic past 2^32 elements (N >= 0xFFFFFF00 takes the
  64-bit branch of the chunk lookup): 2 workers x (2^32 + 2^20 + 27) bf16,
  partitions of 2^20, so one partition starts exactly at element 2^32 and the
  last holds 27 elements (the element kernel);
* the same with a folded grid: 2 workers x (2^34 + 2^20 + 13) binary32;
* the Philox counter's high word: element index e >= 2^35 puts the group
  index g = e / 8 at or above 2^32 (counter word 1 = g >> 32): 1 worker x
  (2^35 + 8,008) elements quantized on a grid given from the host: bf16
  (64 GiB) by thc_usq_quantize's group kernel and by thc_ring_step (folded),
  binary32 (128 GiB) by the lane kernel (folded);
* integer sum and dequant of 2^36 + 40 one-bit indices (folded);
* the block norms of 2^25 + 6 coordinates in blocks of d = 2 (folded), and
  min/max over 2^24 + 3 partitions of 64 elements (folded).

Sampled partitions below and above each boundary are compared with the
oracle element by element (the oracle's quantizer takes the partition's
global index offset); the norms and ranges are compared whole. At most about
140 GB of device memory at a time.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from gradient_all_reduce_worker_amd import _native as ga

pytestmark = pytest.mark.gpu
DEV = "cuda"
PART = 1 << 20


@pytest.fixture(autouse=True)
def _free_memory():
    gc.collect()
    torch.cuda.empty_cache()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _bits(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def _u(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _grid(n_part):
    """Ranges that differ by partition and contain [-4, 4]."""
    p = np.arange(n_part)
    return np.stack([-4.0 - (p % 7), 4.0 + (p % 5)], axis=1).astype(np.float32)


@pytest.mark.parametrize("tdt,N", [(torch.bfloat16, (1 << 32) + PART + 27),
                                   (torch.float32, (1 << 34) + PART + 13)])
def test_ring_beyond_2_32_elements(tdt, N):
    P = 2
    print(f"ring P={P} N={N} {tdt}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    bufs = [torch.randn(N, generator=g, device=DEV, dtype=tdt) for _ in range(P)]
    n_part = -(-N // PART)
    top = (N - 1) // PART                               # the ragged last partition
    edge = top - 1                                      # the partition that starts at 2^32 (2^34)
    assert n_part == top + 1 and edge * PART in (1 << 32, 1 << 34)
    # the first; those below and at 2^31 (2^33), below and at 2^32 (2^34); the last
    which = [0, edge // 2 - 1, edge // 2, edge - 1, edge, top]
    before = {p: [_bits(b[p * PART:min((p + 1) * PART, N)]) for b in bufs] for p in which}
    st = ga.ga_ring_allreduce_sim(bufs, ga.AVG, PART)
    torch.cuda.synchronize()
    assert st["launches"] == 2                          # vectors, then the ragged elements
    for p in which:
        ref = [x.copy() for x in before[p]]
        oracle.ring_fold(ref, op=oracle.AVG, part=PART)
        for i in range(P):
            got = _bits(bufs[i][p * PART:min((p + 1) * PART, N)])
            assert np.array_equal(_u(got), _u(ref[i])), (p, i)


@pytest.mark.parametrize("tdt", [torch.bfloat16, torch.float32])
def test_quantize_and_step_beyond_2_35_elements(tdt):
    """bf16 takes the per-group kernel and then the one-read pass on the same
    vector; binary32 (128 GiB) takes the lane kernel, quantizer only."""
    N, b, seed = (1 << 35) + 8 * 1001, 1, 0x0123_4567_89AB_CDEF
    n_part = -(-N // PART)
    print(f"quantize P=1 N={N} {tdt} b={b}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(12)
    x = torch.randn(N, generator=g, device=DEV, dtype=tdt).clamp_(-4.0, 4.0)
    grid = _grid(n_part)
    mM = torch.from_numpy(grid).to(DEV)
    # 2^34, the last partition below 2^35, the first at 2^35 (groups >= 2^32), the ragged last
    which = [0, 1 << 14, (1 << 15) - 1, 1 << 15, n_part - 1]
    assert (1 << 15) * PART == 1 << 35 and n_part - 1 == 1 << 15
    xs = {p: _bits(x[p * PART:min((p + 1) * PART, N)]) for p in which}
    packed = ga.thc_usq_quantize([x], mM, b, seed, part_elems=PART)[0]
    torch.cuda.synchronize()
    want = {}
    for p in which:
        lo = p * PART
        want[p] = oracle.usq_quantize(xs[p], 0, PART, grid[p:p + 1], b, seed, e_offset=lo)
        got = packed[lo * b // 8: lo * b // 8 + want[p].size].cpu().numpy()
        assert np.array_equal(got, want[p]), p
    if tdt == torch.float32:
        return
    packed.zero_()                                      # the step must write its own indices
    print("quantizer checked; one-read pass", flush=True)
    _, _, xh, _ = ga.thc_ring_step([x], mM, b, seed, ring_part=PART, q_part=PART, packed=[packed],
                                   keep_sum=False, with_nmse=False)
    torch.cuda.synchronize()
    for p in which:
        lo, hi = p * PART, min((p + 1) * PART, N)
        got = packed[lo * b // 8: lo * b // 8 + want[p].size].cpu().numpy()
        assert np.array_equal(got, want[p]), p
        S = oracle.int_aggregate([want[p]], hi - lo, b)
        xw = oracle.dequant(S, 1, b, PART, grid[p:p + 1], oracle.BF16)
        assert np.array_equal(_bits(xh[lo:hi]), xw), p
        assert np.array_equal(_bits(x[lo:hi]), xs[p]), p   # one worker: the average is x


def test_aggregate_dequant_beyond_2_36_indices():
    N, b = (1 << 36) + 40, 1
    n_part = -(-N // PART)
    print(f"aggregate+dequant P=1 N={N} b={b}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(13)
    nbytes = ga.packed_bytes(N, b)
    packed = torch.randint(0, 256, (nbytes,), generator=g, device=DEV, dtype=torch.uint8)
    grid = _grid(n_part)
    mM = torch.from_numpy(grid).to(DEV)
    _, xh, _ = ga.thc_aggregate_dequant([packed], N, b, mM, part_elems=PART, out_dtype=torch.bfloat16,
                                        keep_sum=False)
    torch.cuda.synchronize()
    top = n_part - 1
    assert top == 1 << 16
    for p in [0, 1 << 15, top - 1, top]:
        lo, hi = p * PART, min((p + 1) * PART, N)
        pk = packed[lo * b // 8: (hi * b + 7) // 8].cpu().numpy()
        S = oracle.int_aggregate([pk], hi - lo, b)
        xw = oracle.dequant(S, 1, b, PART, grid[p:p + 1], oracle.BF16)
        assert np.array_equal(_bits(xh[lo:hi]), xw), p


def test_block_norms_of_2_24_blocks():
    P, N, d = 2, (1 << 25) + 6, 2
    print(f"rht_sumsq P={P} N={N} d={d}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(14)
    bufs = [torch.randn(N, generator=g, device=DEV, dtype=torch.bfloat16) for _ in range(P)]
    got = ga.thc_rht_sumsq(bufs, d).cpu().numpy()
    torch.cuda.synchronize()
    assert got.shape == (P, (1 << 24) + 3)
    for i in range(P):
        want = oracle.rht_sumsq(_bits(bufs[i]), d)
        assert np.array_equal(got[i], want), i


def test_minmax_over_2_24_partitions():
    N, part = (1 << 30) + 192, 64
    print(f"minmax P=1 N={N} part={part}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(15)
    x = torch.randn(N, generator=g, device=DEV, dtype=torch.bfloat16)
    got = ga.thc_minmax([x], part).cpu().numpy()
    torch.cuda.synchronize()
    assert got.shape == ((1 << 24) + 3, 2)
    want = oracle.minmax([_bits(x)], part)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
