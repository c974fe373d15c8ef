"""thc_nmse_noalloc (the NMSE of the THC page, section 2, with its partials
in the library's static per-GPU scratch instead of a caller workspace)
against thc_nmse on the same inputs, through the C ABI: two calls in a row,
the second smaller (the scratch keeps the first call's partials), for both
element types. Both run the same kernels in the same order, so the three
doubles must be identical; the oracle's values bound them within 1e-6."""
import numpy as np
import pytest
import torch

import oracle
from gradient_all_reduce_worker_amd import _native as ga

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(N, tdt, seed):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy((rng.standard_normal(N) * 0.01).astype(np.float32))
    xh = x + torch.from_numpy((rng.standard_normal(N) * 0.001).astype(np.float32))
    return x.to(tdt).to(DEV), xh.to(tdt).to(DEV)


def _host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


@pytest.mark.parametrize("tdt", [torch.float32, torch.bfloat16])
def test_noalloc_equals_workspace_call_twice(tdt):
    # first: 2^26 + 12345 elements (about 8,200 partials, two summing levels);
    # second: 70,001 (one level, far fewer partials than the first left behind)
    for N, seed in (((1 << 26) + 12345, 1), (70001, 2)):
        print(f"thc_nmse_noalloc N={N} dtype={tdt}", flush=True)
        x, xh = _pair(N, tdt, seed)
        ref = ga.thc_nmse(x, xh)
        out = torch.full((3,), 7.0, dtype=torch.float64, device=DEV)
        ga.thc_nmse_noalloc(x, xh, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (out, ref)
        num, den, nm = oracle.nmse(_host(x), _host(xh))
        got = out.cpu().numpy()
        assert abs(got[0] - num) <= 1e-6 * num and abs(got[1] - den) <= 1e-6 * den
        assert abs(got[2] - nm) <= 1e-6 * nm


def test_noalloc_empty_and_side_stream():
    out = torch.full((3,), 7.0, dtype=torch.float64, device=DEV)
    e = torch.empty(0, device=DEV)
    ga.thc_nmse_noalloc(e, e, out)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tolist() == [0.0, 0.0, 0.0]
    # on a stream of its own (default priority): same result as thc_nmse
    x, xh = _pair(300001, torch.float32, 3)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ga.thc_nmse_noalloc(x, xh, out, stream=s)
    s.synchronize()
    assert torch.equal(out, ga.thc_nmse(x, xh))
