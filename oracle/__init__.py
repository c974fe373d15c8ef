"""The oracle: a plain CPU implementation of the gradient-aggregation path.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and
the cpu_baseline leg of ``bench.py`` may import, call or link anything under
``oracle/``. The product path (``gradient_all_reduce_worker_amd``) never does,
and the two share no code. Inputs come from the seeded generators; no input
and no expected value ever comes from the HIP path.

The arithmetic lives in ``orc.c`` (ring, THC) and ``fusion.py`` (Tensor
Fusion plan/pack/unpack); this module only marshals numpy arrays.
bf16 arrays are numpy ``uint16`` bit patterns.

Every function here is pinned by CPU tests against facts fixed outside the
oracle (values derived from the pages' worked examples, closed forms,
library routines, brute force on tiny inputs and statistics); see
``tests/test_oracle_*.py``. The one part the pages cannot pin is the choice
of random generator (Philox4x32-10, pinned by its published known-answer
vectors) and the partition length used for the bf16 large-shard workload.
"""
import ctypes as C
import os

import numpy as np

from . import fusion  # noqa: F401  (re-exported)
from .fusion import fuse_pack, fuse_plan, fuse_unpack  # noqa: F401

F32, BF16 = 0, 1
SUM, AVG = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        L = C.CDLL(_LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        L.orc_ring_fold.argtypes = [C.POINTER(vp), i32, i64, i32, i32, i64]
        L.orc_ring_stepwise.argtypes = [C.POINTER(vp), i32, i64, i32, i32, i64, i32]
        L.orc_dual_ring_fold.argtypes = [C.POINTER(vp), i32, i64, i32, i32, i64]
        L.orc_dual_ring_stepwise.argtypes = [C.POINTER(vp), i32, i64, i32, i32, i64]
        L.orc_ring_stats.argtypes = [i32, i64, i64, i32, C.POINTER(i64), C.POINTER(i64)]
        L.orc_ef_add.argtypes = [vp, i32, vp, i64, vp]
        L.orc_ef_add.restype = None
        L.orc_ef_update.argtypes = [vp, vp, i64, i32, i32, vp, i64, vp, vp]
        L.orc_ring_stats.restype = None
        L.orc_minmax.argtypes = [C.POINTER(vp), i32, i64, i32, i64, vp]
        L.orc_philox4x32_10.argtypes = [vp, vp, vp]
        L.orc_philox4x32_10.restype = None
        L.orc_uniform16.argtypes = [C.c_uint64, i32, i64]
        L.orc_uniform16.restype = C.c_uint32
        L.orc_usq_quantize.argtypes = [vp, i64, i32, i32, i64, vp, i32, C.c_uint64, i64, vp]
        L.orc_unpack_indices.argtypes = [vp, i64, i32, vp]
        L.orc_int_aggregate.argtypes = [C.POINTER(vp), i32, i64, i32, vp]
        L.orc_dequant.argtypes = [vp, i64, i32, i32, i64, vp, vp, i32]
        L.orc_nmse.argtypes = [vp, vp, i64, i32, vp]
        L.orc_nuhc_quantize.argtypes = [vp, i64, i32, i32, i64, vp, i32, i32, vp, C.c_uint64, i64, vp]
        L.orc_nuhc_aggregate.argtypes = [C.POINTER(vp), i32, i64, i32, i32, vp, vp]
        L.orc_nuhc_dequant.argtypes = [vp, i64, i32, i32, i64, vp, vp, i32]
        L.orc_rht_forward.argtypes = [vp, i32, i64, i64, C.c_uint64, i64, vp]
        L.orc_rht_inverse.argtypes = [vp, i64, i64, C.c_uint64, i64, vp, i32]
        L.orc_rht_sumsq.argtypes = [vp, i32, i64, i64, vp]
        L.orc_rht_range.argtypes = [vp, i32, i64, i64, C.c_double, vp]
        L.orc_clamp.argtypes = [vp, i64, i64, vp]
        L.orc_clamp.restype = None
        L.orc_rademacher.argtypes = [C.c_uint64, i64, i64, vp]
        L.orc_rademacher.restype = None
        L.orc_f32_to_bf16.argtypes = [vp, i64, vp]
        L.orc_f32_to_bf16.restype = None
        L.orc_bf16_to_f32.argtypes = [vp, i64, vp]
        L.orc_bf16_to_f32.restype = None
        _lib = L
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle buffers are float32 or uint16 (bf16 bits), not {a.dtype}")


def _ptrs(arrs):
    for a in arrs:
        if not a.flags.c_contiguous:
            raise ValueError("oracle buffers must be C-contiguous")
    return (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with {rc}")


def _n_part(N: int, part: int) -> int:
    plen = part if part > 0 else N
    return 0 if N == 0 else (N + plen - 1) // plen


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty(x.shape, dtype=np.float32)
    lib().orc_bf16_to_f32(x.ctypes.data, x.size, out.ctypes.data)
    return out


# ---------------------------------------------------------------- ring
def ring_fold(bufs, op: int = AVG, part: int = 0) -> None:
    """In place: every buffer ends holding the ring's result (see orc.c)."""
    P, N = len(bufs), bufs[0].size
    _check(lib().orc_ring_fold(_ptrs(bufs), P, N, _dt(bufs[0]), op, part), "ring_fold")


def ring_stepwise(bufs, op: int = AVG, part: int = 0, rs_only: bool = False) -> None:
    """In place: the literal 2(P-1)-step schedule with send copies."""
    P, N = len(bufs), bufs[0].size
    _check(lib().orc_ring_stepwise(_ptrs(bufs), P, N, _dt(bufs[0]), op, part, int(rs_only)),
           "ring_stepwise")


def dual_ring_fold(bufs, op: int = AVG, part: int = 0) -> None:
    """In place: the bidirectional ring's result (2P sub-chunks, see orc.c)."""
    P, N = len(bufs), bufs[0].size
    _check(lib().orc_dual_ring_fold(_ptrs(bufs), P, N, _dt(bufs[0]), op, part), "dual_ring_fold")


def dual_ring_stepwise(bufs, op: int = AVG, part: int = 0) -> None:
    """In place: the literal two-direction schedule with send copies."""
    P, N = len(bufs), bufs[0].size
    _check(lib().orc_dual_ring_stepwise(_ptrs(bufs), P, N, _dt(bufs[0]), op, part),
           "dual_ring_stepwise")


def ring_stats(P: int, N: int, part: int, elem_bytes: int):
    steps, nbytes = C.c_int64(), C.c_int64()
    lib().orc_ring_stats(P, N, part, elem_bytes, C.byref(steps), C.byref(nbytes))
    return steps.value, nbytes.value


# ---------------------------------------------------------------- THC
def minmax(bufs, part: int = 0) -> np.ndarray:
    P, N = len(bufs), bufs[0].size
    out = np.zeros((_n_part(N, part), 2), dtype=np.float32)
    if N:
        _check(lib().orc_minmax(_ptrs(bufs), P, N, _dt(bufs[0]), part, out.ctypes.data), "minmax")
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def uniform16(seed: int, worker: int, e: int) -> int:
    return int(lib().orc_uniform16(seed, worker, e))


def usq_quantize(x: np.ndarray, worker: int, part: int, mM: np.ndarray, b: int, seed: int,
                 e_offset: int = 0) -> np.ndarray:
    """e_offset: index of x[0] in the worker's whole vector (keys the generator)."""
    N = x.size
    out = np.zeros((N * b + 7) // 8, dtype=np.uint8)
    mM = np.ascontiguousarray(mM, dtype=np.float32)
    x = np.ascontiguousarray(x)
    _check(lib().orc_usq_quantize(x.ctypes.data, N, _dt(x), worker, part, mM.ctypes.data, b,
                                  seed, e_offset, out.ctypes.data), "usq_quantize")
    return out


def unpack_indices(packed: np.ndarray, N: int, b: int) -> np.ndarray:
    z = np.zeros(N, dtype=np.int32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    _check(lib().orc_unpack_indices(packed.ctypes.data, N, b, z.ctypes.data), "unpack")
    return z


def int_aggregate(packed_list, N: int, b: int) -> np.ndarray:
    S = np.zeros(N, dtype=np.int32)
    packed_list = [np.ascontiguousarray(p, dtype=np.uint8) for p in packed_list]
    _check(lib().orc_int_aggregate(_ptrs(packed_list), len(packed_list), N, b, S.ctypes.data),
           "int_aggregate")
    return S


def dequant(S: np.ndarray, P: int, b: int, part: int, mM: np.ndarray, out_dt: int = F32
            ) -> np.ndarray:
    N = S.size
    S = np.ascontiguousarray(S, dtype=np.int32)
    mM = np.ascontiguousarray(mM, dtype=np.float32)
    out = np.zeros(N, dtype=np.float32 if out_dt == F32 else np.uint16)
    _check(lib().orc_dequant(S.ctypes.data, N, P, b, part, mM.ctypes.data, out.ctypes.data,
                             out_dt), "dequant")
    return out


def nmse(x: np.ndarray, xhat: np.ndarray):
    x = np.ascontiguousarray(x)
    xhat = np.ascontiguousarray(xhat)
    assert x.dtype == xhat.dtype and x.size == xhat.size
    out = np.zeros(3, dtype=np.float64)
    _check(lib().orc_nmse(x.ctypes.data, xhat.ctypes.data, x.size, _dt(x), out.ctypes.data),
           "nmse")
    return float(out[0]), float(out[1]), float(out[2])


# ---------------------------------------------------------------- non-uniform THC
def _table(T):
    return np.ascontiguousarray(T, dtype=np.int32)


def nuhc_quantize(x: np.ndarray, worker: int, part: int, mM: np.ndarray, b: int, g: int, T,
                  seed: int, e_offset: int = 0) -> np.ndarray:
    N = x.size
    out = np.zeros((N * b + 7) // 8, dtype=np.uint8)
    mM = np.ascontiguousarray(mM, dtype=np.float32)
    x = np.ascontiguousarray(x)
    T = _table(T)
    _check(lib().orc_nuhc_quantize(x.ctypes.data, N, _dt(x), worker, part, mM.ctypes.data, b, g,
                                   T.ctypes.data, seed, e_offset, out.ctypes.data), "nuhc_quantize")
    return out


def nuhc_aggregate(packed_list, N: int, b: int, g: int, T) -> np.ndarray:
    Y = np.zeros(N, dtype=np.int32)
    packed_list = [np.ascontiguousarray(p, dtype=np.uint8) for p in packed_list]
    T = _table(T)
    _check(lib().orc_nuhc_aggregate(_ptrs(packed_list), len(packed_list), N, b, g, T.ctypes.data,
                                    Y.ctypes.data), "nuhc_aggregate")
    return Y


def nuhc_dequant(Y: np.ndarray, P: int, g: int, part: int, mM: np.ndarray, out_dt: int = F32
                 ) -> np.ndarray:
    N = Y.size
    Y = np.ascontiguousarray(Y, dtype=np.int32)
    mM = np.ascontiguousarray(mM, dtype=np.float32)
    out = np.zeros(N, dtype=np.float32 if out_dt == F32 else np.uint16)
    _check(lib().orc_nuhc_dequant(Y.ctypes.data, N, P, g, part, mM.ctypes.data, out.ctypes.data,
                                  out_dt), "nuhc_dequant")
    return out


# ---------------------------------------------------------------- RHT pre/post-processing
def rht_forward(x: np.ndarray, d: int, seed: int, e0: int = 0) -> np.ndarray:
    """Zero-pads to a multiple of d; returns ceil(N/d) d binary32 values.
    e0: index of x[0] in the whole vector (a multiple of d; selects the signs)."""
    x = np.ascontiguousarray(x)
    y = np.zeros(-(-x.size // d) * d, dtype=np.float32)
    _check(lib().orc_rht_forward(x.ctypes.data, _dt(x), x.size, d, seed, e0, y.ctypes.data),
           "rht_forward")
    return y


def rht_inverse(y: np.ndarray, d: int, seed: int, out_dt: int = F32, e0: int = 0) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.zeros(y.size, dtype=np.float32 if out_dt == F32 else np.uint16)
    _check(lib().orc_rht_inverse(y.ctypes.data, y.size, d, seed, e0, out.ctypes.data, out_dt),
           "rht_inverse")
    return out


def rademacher(seed: int, e0: int, n: int) -> np.ndarray:
    out = np.zeros(n, dtype=np.float32)
    lib().orc_rademacher(seed, e0, n, out.ctypes.data)
    return out


def rht_sumsq(x: np.ndarray, d: int) -> np.ndarray:
    x = np.ascontiguousarray(x)
    out = np.zeros(-(-x.size // d), dtype=np.float64)
    _check(lib().orc_rht_sumsq(x.ctypes.data, _dt(x), x.size, d, out.ctypes.data), "rht_sumsq")
    return out


def rht_range(sumsq: np.ndarray, d: int, t_p: float) -> np.ndarray:
    """sumsq: [P, nblk] float64 -> mM [nblk, 2] float32."""
    sumsq = np.ascontiguousarray(sumsq, dtype=np.float64)
    P, nblk = sumsq.shape
    mM = np.zeros((nblk, 2), dtype=np.float32)
    _check(lib().orc_rht_range(sumsq.ctypes.data, P, nblk, d, t_p, mM.ctypes.data), "rht_range")
    return mM


def clamp(y: np.ndarray, d: int, mM: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32).copy()
    mM = np.ascontiguousarray(mM, dtype=np.float32)
    lib().orc_clamp(y.ctypes.data, y.size, d, mM.ctypes.data)
    return y


# ---------------------------------------------------------------- error feedback
def ef_add(grad: np.ndarray, e: np.ndarray) -> np.ndarray:
    """x = grad + e in binary32 (grad fp32, or bf16 as uint16 bits)."""
    grad = np.ascontiguousarray(grad)
    e = np.ascontiguousarray(e, dtype=np.float32)
    assert grad.size == e.size
    x = np.zeros(grad.size, dtype=np.float32)
    lib().orc_ef_add(grad.ctypes.data, _dt(grad), e.ctypes.data, grad.size, x.ctypes.data)
    return x


def ef_update(x: np.ndarray, packed: np.ndarray, b: int, part: int, mM: np.ndarray,
              g: int = 0, T=None) -> np.ndarray:
    """e' = x - xhat, xhat = the value of the worker's own indices (table T
    with granularity g, or the uniform grid when T is None)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    mM = np.ascontiguousarray(mM, dtype=np.float32)
    out = np.zeros(x.size, dtype=np.float32)
    Tp = None
    if T is not None:
        Ta = _table(T)
        Tp = Ta.ctypes.data
    _check(lib().orc_ef_update(x.ctypes.data, packed.ctypes.data, x.size, b, g, Tp, part,
                               mM.ctypes.data, out.ctypes.data), "ef_update")
    return out
