"""ctypes binding of libga.so: the C ABI declared in include/ga.h, with the
same names. Argument marshalling only (torch tensors -> device pointers and
the current stream); every step of the path runs in the HIP library.

Functions raise GAError on a non-zero status, carrying ga_last_error().
If libga.so is missing or cannot be loaded, load() raises: there is no
fallback implementation.
"""
import ctypes as C
import os
from typing import List, Optional, Sequence

import numpy as np
import torch

F32, BF16 = 0, 1
SUM, AVG = 0, 1
RING_FUSED, RING_STEPWISE, RING_DUAL = 0, 1, 2
MAX_WORKERS = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libga.so")

EXPORTS = (
    "ga_fuse_plan", "ga_fuse_desc_check", "ga_fuse_pack", "ga_fuse_unpack",
    "ga_ring_allreduce_sim", "thc_minmax", "thc_usq_quantize", "thc_int_aggregate",
    "thc_dequant", "thc_nmse", "thc_nmse_ws_bytes", "thc_nmse_noalloc", "ga_last_error",
    "thc_nuhc_quantize", "thc_nuhc_aggregate", "thc_nuhc_dequant",
    "thc_rht_sumsq", "thc_rht_range", "thc_rht_forward", "thc_rht_inverse",
    "ga_fusion_ring_plan", "ga_fusion_ring_allreduce", "thc_ef_minmax", "thc_ef_quantize",
    "thc_rht_quantize", "thc_aggregate_dequant", "thc_aggregate_dequant_ws_bytes",
    "thc_rht_norm_quantize", "thc_rht_norm_quantize_ws_bytes", "thc_ring_step",
    "thc_ring_step_ws_bytes", "ga_ring_stage_bytes", "ga_ring_stepwise_staged",
    "thc_ring_step_launches", "thc_minmax_combine", "thc_ef_minmax_pair",
)


class GAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class CopyDesc(C.Structure):
    _fields_ = [("src", C.c_void_p), ("dst", C.c_void_p), ("n", C.c_int64), ("start", C.c_int64)]


class RingStats(C.Structure):
    _fields_ = [("steps", C.c_int64), ("bytes_sent_per_worker", C.c_int64),
                ("hbm_bytes", C.c_int64), ("launches", C.c_int64)]


DESC_DTYPE = np.dtype([("src", np.uint64), ("dst", np.uint64), ("n", np.int64), ("start", np.int64)])
# ga_fusion_tensor
FTENSOR_DTYPE = np.dtype([("start", np.int64), ("n", np.int64), ("buf", np.int32),
                          ("reserved", np.int32)])

_lib = None


def load() -> C.CDLL:
    """Load libga.so (built by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = C.CDLL(LIB_PATH)
    vp, i64, i32, u64 = C.c_void_p, C.c_int64, C.c_int32, C.c_uint64
    P64 = C.POINTER(C.c_int64)
    P32 = C.POINTER(C.c_int32)
    L.ga_fuse_plan.argtypes = [P64, P32, i32, i64, P32, P64, P64, P32, P32]
    L.ga_fuse_desc_check.argtypes = [vp, i64, i32, P64]
    L.ga_fuse_pack.argtypes = [vp, i64, i64, i32, vp]
    L.ga_fuse_unpack.argtypes = [vp, i64, i64, i32, vp]
    L.ga_ring_allreduce_sim.argtypes = [C.POINTER(vp), i32, i64, i32, i32, i64, i32,
                                        C.POINTER(RingStats), vp]
    L.ga_ring_stage_bytes.argtypes = [i32, i64]
    L.ga_ring_stage_bytes.restype = C.c_size_t
    L.ga_ring_stepwise_staged.argtypes = [C.POINTER(vp), i32, i64, i32, i32, i64, vp, C.c_size_t,
                                          C.POINTER(RingStats), vp]
    L.thc_minmax.argtypes = [C.POINTER(vp), i32, i64, i32, i64, vp, vp]
    L.thc_minmax_combine.argtypes = [vp, i64, vp, vp]
    L.thc_usq_quantize.argtypes = [C.POINTER(vp), i32, i32, i64, i32, i64, vp, i32, u64,
                                   C.POINTER(vp), vp]
    L.thc_int_aggregate.argtypes = [C.POINTER(vp), i32, i64, i32, vp, vp]
    L.thc_dequant.argtypes = [vp, i64, i32, i32, i64, vp, vp, i32, vp]
    L.thc_nmse.argtypes = [vp, vp, i64, i32, vp, vp, C.c_size_t, vp]
    L.thc_nmse_noalloc.argtypes = [vp, vp, i64, i32, vp, vp]
    L.thc_nmse_ws_bytes.argtypes = [i64]
    L.thc_nmse_ws_bytes.restype = C.c_size_t
    L.thc_nuhc_quantize.argtypes = [C.POINTER(vp), i32, i32, i64, i32, i64, vp, i32, i32,
                                    C.POINTER(i32), u64, C.POINTER(vp), vp]
    L.thc_nuhc_aggregate.argtypes = [C.POINTER(vp), i32, i64, i32, i32, C.POINTER(i32), vp, vp]
    L.thc_nuhc_dequant.argtypes = [vp, i64, i32, i32, i64, vp, vp, i32, vp]
    L.thc_rht_sumsq.argtypes = [C.POINTER(vp), i32, i64, i32, i64, vp, vp]
    L.thc_rht_range.argtypes = [vp, i32, i64, i64, C.c_double, vp, vp]
    L.thc_rht_forward.argtypes = [C.POINTER(vp), i32, i64, i32, i64, u64, vp, C.POINTER(vp), vp]
    L.thc_rht_inverse.argtypes = [vp, i64, i64, u64, vp, i32, vp]
    L.thc_rht_quantize.argtypes = [C.POINTER(vp), i32, i32, i64, i32, i64, u64, vp, i32, i32,
                                   C.POINTER(i32), u64, C.POINTER(vp), C.POINTER(vp), vp]
    L.ga_fusion_ring_plan.argtypes = [vp, vp, i64, i32, i32, P64, i32, i64, i32, vp, i64,
                                      C.POINTER(i64)]
    L.ga_fusion_ring_allreduce.argtypes = [vp, i64, i32, i32, i32, P64, i32, i64, i32,
                                           C.POINTER(RingStats), vp]
    L.thc_ef_minmax.argtypes = [C.POINTER(vp), C.POINTER(vp), i32, i64, i32, i64, vp, vp]
    L.thc_ef_minmax_pair.argtypes = [C.POINTER(vp), C.POINTER(vp), i32, i64, i32, i64, vp, vp, vp]
    L.thc_ef_quantize.argtypes = [C.POINTER(vp), C.POINTER(vp), i32, i32, i64, i32, i64, vp, i32,
                                  i32, C.POINTER(i32), u64, C.POINTER(vp), vp]
    L.thc_aggregate_dequant.argtypes = [C.POINTER(vp), i32, i64, i32, i32, C.POINTER(i32), i64, vp, vp,
                                        vp, i32, vp, vp, vp, C.c_size_t, vp]
    L.thc_aggregate_dequant_ws_bytes.argtypes = [i64]
    L.thc_rht_norm_quantize.argtypes = [C.POINTER(vp), i32, i32, i64, i32, i64, u64, C.c_double, i32,
                                        i32, C.POINTER(i32), u64, vp, vp, C.POINTER(vp), vp, C.c_size_t,
                                        C.POINTER(vp), vp]
    L.thc_ring_step.argtypes = [C.POINTER(vp), i32, i64, i32, i64, vp, i64, i32, u64, i32,
                                C.POINTER(vp), vp, vp, vp, vp, C.c_size_t, vp]
    L.thc_ring_step_ws_bytes.argtypes = [i64]
    L.thc_ring_step_ws_bytes.restype = C.c_size_t
    L.thc_ring_step_launches.argtypes = [i64]
    L.thc_ring_step_launches.restype = i64
    L.thc_rht_norm_quantize_ws_bytes.argtypes = [i32, i64, i64]
    L.thc_rht_norm_quantize_ws_bytes.restype = C.c_size_t
    L.thc_aggregate_dequant_ws_bytes.restype = C.c_size_t
    L.ga_last_error.argtypes = []
    L.ga_last_error.restype = C.c_char_p
    for name in EXPORTS:                 # every other call returns a ga_status
        if not name.endswith(("_bytes", "_launches")) and name != "ga_last_error":
            getattr(L, name).restype = C.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise GAError(status, load().ga_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"gradient buffers are float32 or bfloat16, not {t.dtype}")


def _dev(t: torch.Tensor, what: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def _ptr_array(tensors: Sequence[torch.Tensor], what: str):
    return (C.c_void_p * len(tensors))(*[_dev(t, what) for t in tensors])


# ------------------------------------------------------------------ fusion
def ga_fuse_plan(n_elems: Sequence[int], dtypes: Optional[Sequence[int]], cap_bytes: int):
    """Host-only plan. Returns (buf_of, off_of, fill, buf_dtype) lists."""
    L = load()
    T = len(n_elems)
    n = (C.c_int64 * max(T, 1))(*[int(v) for v in n_elems])
    dts = None if dtypes is None else (C.c_int32 * max(T, 1))(*[int(v) for v in dtypes])
    buf_of = (C.c_int32 * max(T, 1))()
    off_of = (C.c_int64 * max(T, 1))()
    fill = (C.c_int64 * max(T, 1))()
    bdt = (C.c_int32 * max(T, 1))()
    nb = C.c_int32()
    _check(L.ga_fuse_plan(n, dts, T, int(cap_bytes), buf_of, off_of, fill, bdt, C.byref(nb)))
    k = nb.value
    return list(buf_of)[:T], list(off_of)[:T], list(fill)[:k], list(bdt)[:k]


def ga_fuse_desc_check(h_desc: np.ndarray, dt: int) -> int:
    """Validate a host descriptor table (DESC_DTYPE array); return its total."""
    L = load()
    h_desc = np.ascontiguousarray(h_desc, dtype=DESC_DTYPE)
    total = C.c_int64()
    _check(L.ga_fuse_desc_check(h_desc.ctypes.data if h_desc.size else None, h_desc.size, dt,
                                C.byref(total)))
    return total.value


def ga_fuse_pack(d_desc: torch.Tensor, n_desc: int, total: int, dt: int, stream=None) -> None:
    _check(load().ga_fuse_pack(_dev(d_desc, "d_desc"), n_desc, total, dt, _stream(stream)))


def ga_fuse_unpack(d_desc: torch.Tensor, n_desc: int, total: int, dt: int, stream=None) -> None:
    _check(load().ga_fuse_unpack(_dev(d_desc, "d_desc"), n_desc, total, dt, _stream(stream)))


def build_copy_table(srcs: Sequence[int], dsts: Sequence[int], ns: Sequence[int]) -> np.ndarray:
    """Host descriptor table from parallel lists of addresses and counts."""
    t = np.zeros(len(ns), dtype=DESC_DTYPE)
    t["src"] = np.asarray(srcs, dtype=np.uint64)
    t["dst"] = np.asarray(dsts, dtype=np.uint64)
    t["n"] = np.asarray(ns, dtype=np.int64)
    if len(ns):
        t["start"][1:] = np.cumsum(t["n"])[:-1]
    return t


def upload_table(h_desc: np.ndarray, device) -> torch.Tensor:
    """Device copy of a descriptor table, as a uint8 tensor."""
    raw = torch.from_numpy(h_desc.view(np.uint8).copy())
    return raw.to(device)


class FusionTables:
    """Pack and unpack descriptor tables for P workers' tensors and fusion
    buffers, built once on the host from a plan and uploaded once."""

    def __init__(self, worker_tensors: List[List[torch.Tensor]], fusion_bufs: List[List[torch.Tensor]],
                 buf_of: Sequence[int], off_of: Sequence[int]):
        dt = _dt(worker_tensors[0][0])
        self.dt = dt
        es = 4 if dt == F32 else 2
        srcs, dsts, ns = [], [], []
        for w, tensors in enumerate(worker_tensors):
            for t, x in enumerate(tensors):
                if _dt(x) != dt:
                    raise TypeError("one data type per fusion table")
                srcs.append(_dev(x, "tensor"))
                dsts.append(_dev(fusion_bufs[w][buf_of[t]], "fusion buffer") + int(off_of[t]) * es)
                ns.append(x.numel())
        self.h_pack = build_copy_table(srcs, dsts, ns)
        self.h_unpack = build_copy_table(dsts, srcs, ns)
        self.total = ga_fuse_desc_check(self.h_pack, dt)
        ga_fuse_desc_check(self.h_unpack, dt)
        device = worker_tensors[0][0].device
        self.d_pack = upload_table(self.h_pack, device)
        self.d_unpack = upload_table(self.h_unpack, device)
        self.n_desc = len(ns)

    def pack(self, stream=None) -> None:
        ga_fuse_pack(self.d_pack, self.n_desc, self.total, self.dt, stream)

    def unpack(self, stream=None) -> None:
        ga_fuse_unpack(self.d_unpack, self.n_desc, self.total, self.dt, stream)


# ------------------------------------------------------------------ ring
def ga_ring_allreduce_sim(bufs: Sequence[torch.Tensor], op: int = AVG, part_elems: int = 0,
                          mode: int = RING_FUSED, stream=None) -> dict:
    L = load()
    P = len(bufs)
    if P == 0:
        raise ValueError("no buffers")
    N = bufs[0].numel()
    dt = _dt(bufs[0])
    for b in bufs:
        if b.numel() != N or _dt(b) != dt:
            raise ValueError("all worker buffers need the same size and dtype")
    st = RingStats()
    _check(L.ga_ring_allreduce_sim(_ptr_array(bufs, "buffer"), P, N, dt, op, part_elems, mode,
                                   C.byref(st), _stream(stream)))
    return {"steps": st.steps, "bytes_sent_per_worker": st.bytes_sent_per_worker,
            "hbm_bytes": st.hbm_bytes, "launches": st.launches}


def ga_ring_stage_bytes(P: int, N: int) -> int:
    return int(load().ga_ring_stage_bytes(P, N))


def ga_ring_stepwise_staged(bufs: Sequence[torch.Tensor], op: int = AVG, part_elems: int = 0,
                            stage: Optional[torch.Tensor] = None, stream=None) -> dict:
    """The ring schedule one step per launch, partials in a binary32 stage
    (allocated here when not given)."""
    L = load()
    P = len(bufs)
    if P == 0:
        raise ValueError("no buffers")
    N = bufs[0].numel()
    dt = _dt(bufs[0])
    for b in bufs:
        if b.numel() != N or _dt(b) != dt:
            raise ValueError("all worker buffers need the same size and dtype")
    need = ga_ring_stage_bytes(P, N)
    if stage is None and need > 0:
        stage = torch.empty(need // 4, dtype=torch.float32, device=bufs[0].device)
    st = RingStats()
    _check(L.ga_ring_stepwise_staged(_ptr_array(bufs, "buffer"), P, N, dt, op, part_elems,
                                     _dev(stage, "stage") if stage is not None else None,
                                     stage.numel() * stage.element_size() if stage is not None else 0,
                                     C.byref(st), _stream(stream)))
    return {"steps": st.steps, "bytes_sent_per_worker": st.bytes_sent_per_worker,
            "hbm_bytes": st.hbm_bytes, "launches": st.launches}


# ------------------------------------------------------------------ zero-copy fusion ring
FUSION_BLOCK = 256          # GA_FUSION_BLOCK


def fusion_block_bytes(P: int) -> int:
    """GA_FUSION_BLOCK_BYTES(P): a 16-byte header and P pointers."""
    return 16 + 8 * P


def _fills(fill: Sequence[int]):
    return (C.c_int64 * max(len(fill), 1))(*[int(f) for f in fill])


def ga_fusion_ring_plan(h_tensors: np.ndarray, h_ptrs: np.ndarray, P: int, dt: int,
                        fill: Sequence[int], part_elems: int = 0, mode: int = RING_FUSED) -> np.ndarray:
    """Host-only: the planned work blocks (a uint8 array of n_blocks x
    fusion_block_bytes(P)) of a table (FTENSOR_DTYPE rows, buffer by buffer
    in buffer order; h_ptrs uint64 [n_tensors, P]) for the given ring
    geometry."""
    if h_tensors.dtype != FTENSOR_DTYPE or not h_tensors.flags.c_contiguous:
        raise TypeError("h_tensors must be a contiguous FTENSOR_DTYPE array")
    h_ptrs = np.ascontiguousarray(h_ptrs, dtype=np.uint64)
    if h_ptrs.size != h_tensors.size * P:
        raise ValueError("h_ptrs must hold n_tensors x P pointers")
    L = load()
    args = (h_tensors.ctypes.data if h_tensors.size else None,
            h_ptrs.ctypes.data if h_ptrs.size else None, h_tensors.size, P, dt, _fills(fill),
            len(fill), part_elems, mode)
    n = C.c_int64(0)
    _check(L.ga_fusion_ring_plan(*args, None, 0, C.byref(n)))
    work = np.zeros(max(n.value, 1) * fusion_block_bytes(P), dtype=np.uint8)
    _check(L.ga_fusion_ring_plan(*args, work.ctypes.data, n.value, C.byref(n)))
    return work[:n.value * fusion_block_bytes(P)]


class FusionRing:
    """Tensor Fusion without the fusion buffers: the table of a plan's
    tensors (buffer id, offset, size) and the P workers' pointers to them.
    allreduce() folds every buffer of the plan in place in the workers'
    tensors in one launch; allreduce_buffer(k) folds buffer k alone, as a
    caller does when buffers are reduced as they fill. The work blocks of
    each (buffers, mode, part_elems) are planned on the host and uploaded on
    first use."""

    def __init__(self, worker_tensors: List[List[torch.Tensor]], buf_of: Sequence[int],
                 off_of: Sequence[int], fill: Sequence[int]):
        self.P = len(worker_tensors)
        self.dt = _dt(worker_tensors[0][0])
        self.fill = [int(f) for f in fill]
        self.device = worker_tensors[0][0].device
        rows = sorted((int(buf_of[t]), int(off_of[t]), t) for t in range(len(buf_of)))
        self._rows = rows
        self._ptrs = np.zeros((len(rows), self.P), dtype=np.uint64)
        self._sizes = []
        for r, (_, _, t) in enumerate(rows):
            n = worker_tensors[0][t].numel()
            for i in range(self.P):
                x = worker_tensors[i][t]
                if _dt(x) != self.dt or x.numel() != n:
                    raise TypeError("workers' tensors must agree in size and data type")
                self._ptrs[r, i] = _dev(x, "tensor")
            self._sizes.append(n)
        self._work = {}
        self._plan(None, RING_FUSED, 0)        # checks the table now

    def _plan(self, only: Optional[int], mode: int, part_elems: int):
        """The uploaded work of every buffer (only = None) or of buffer
        `only`, renumbered as buffer 0 of a one-buffer table."""
        key = (only, mode, part_elems)
        if key not in self._work:
            rows = [q for q, (b, _, _) in enumerate(self._rows) if only is None or b == only]
            h = np.zeros(len(rows), dtype=FTENSOR_DTYPE)
            for r, q in enumerate(rows):
                k, off, _ = self._rows[q]
                h[r]["buf"] = 0 if only is not None else k
                h[r]["start"] = off
                h[r]["n"] = self._sizes[q]
            fill = [self.fill[only]] if only is not None else self.fill
            work = ga_fusion_ring_plan(h, self._ptrs[rows], self.P, self.dt, fill, part_elems, mode)
            n_blocks = work.size // fusion_block_bytes(self.P)
            d_w = torch.from_numpy(work.copy() if work.size else np.zeros(8, np.uint8)).to(self.device)
            self._work[key] = (d_w, n_blocks, fill)
        return self._work[key]

    def _run(self, only, op, mode, part_elems, stream) -> dict:
        d_w, n_blocks, fill = self._plan(only, mode, part_elems)
        st = RingStats()
        _check(load().ga_fusion_ring_allreduce(d_w.data_ptr(), n_blocks, self.P, self.dt, op,
                                               _fills(fill), len(fill), part_elems, mode,
                                               C.byref(st), _stream(stream)))
        return {"steps": st.steps, "bytes_sent_per_worker": st.bytes_sent_per_worker,
                "hbm_bytes": st.hbm_bytes, "launches": st.launches}

    def allreduce(self, op: int = AVG, mode: int = RING_FUSED, part_elems: int = 0,
                  stream=None) -> dict:
        """Every buffer of the plan, one launch."""
        return self._run(None, op, mode, part_elems, stream)

    def allreduce_buffer(self, k: int, op: int = AVG, mode: int = RING_FUSED, part_elems: int = 0,
                         stream=None) -> dict:
        """Buffer k alone, one launch."""
        return self._run(k, op, mode, part_elems, stream)


# ------------------------------------------------------------------ THC
def n_partitions(N: int, part_elems: int) -> int:
    if N == 0:
        return 0
    plen = part_elems if part_elems > 0 else N
    return (N + plen - 1) // plen


def thc_minmax(bufs: Sequence[torch.Tensor], part_elems: int = 0, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    N = bufs[0].numel()
    if out is None:
        out = torch.empty((max(n_partitions(N, part_elems), 1), 2), dtype=torch.float32,
                          device=bufs[0].device)
    _check(load().thc_minmax(_ptr_array(bufs, "buffer"), len(bufs), N, _dt(bufs[0]), part_elems,
                             _dev(out, "mM"), _stream(stream)))
    return out


def packed_bytes(N: int, b: int) -> int:
    return (N * b + 7) // 8


def thc_minmax_combine(parts: torch.Tensor, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """The whole vector's grid (1 x 2) from thc_minmax's partition grids."""
    if out is None:
        out = torch.empty((1, 2), dtype=torch.float32, device=parts.device)
    _check(load().thc_minmax_combine(_dev(parts, "parts"), parts.numel() // 2, _dev(out, "mM"),
                                     _stream(stream)))
    return out


def thc_usq_quantize(bufs: Sequence[torch.Tensor], mM: torch.Tensor, b: int, seed: int,
                     part_elems: int = 0, worker0: int = 0,
                     packed: Optional[Sequence[torch.Tensor]] = None, stream=None):
    N = bufs[0].numel()
    if packed is None:
        packed = [torch.empty(packed_bytes(N, b), dtype=torch.uint8, device=bufs[0].device)
                  for _ in bufs]
    _check(load().thc_usq_quantize(_ptr_array(bufs, "buffer"), len(bufs), worker0, N, _dt(bufs[0]),
                                   part_elems, _dev(mM, "mM"), b, seed,
                                   _ptr_array(packed, "packed"), _stream(stream)))
    return packed


def thc_int_aggregate(packed: Sequence[torch.Tensor], N: int, b: int,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(max(N, 1), dtype=torch.int32, device=packed[0].device)
    _check(load().thc_int_aggregate(_ptr_array(packed, "packed"), len(packed), N, b,
                                    _dev(out, "sum"), _stream(stream)))
    return out


def thc_dequant(S: torch.Tensor, N: int, P: int, b: int, mM: torch.Tensor, part_elems: int = 0,
                out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(max(N, 1), dtype=out_dtype, device=S.device)
    _check(load().thc_dequant(_dev(S, "sum"), N, P, b, part_elems, _dev(mM, "mM"), _dev(out, "out"),
                              _dt(out), _stream(stream)))
    return out


def thc_nmse_ws_bytes(N: int) -> int:
    return int(load().thc_nmse_ws_bytes(N))


def thc_nmse(x: torch.Tensor, xhat: torch.Tensor, out: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    N = x.numel()
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=x.device)
    if ws is None:
        ws = torch.empty(thc_nmse_ws_bytes(N), dtype=torch.uint8, device=x.device)
    _check(load().thc_nmse(_dev(x, "x"), _dev(xhat, "xhat"), N, _dt(x), _dev(out, "out"),
                           _dev(ws, "ws"), ws.numel(), _stream(stream)))
    return out


def thc_nmse_noalloc(x: torch.Tensor, xhat: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """thc_nmse without a workspace: the library's static per-GPU scratch
    holds the partials; `out` (3 float64 on the device) is the caller's."""
    if x.numel() != xhat.numel() or _dt(x) != _dt(xhat):
        raise ValueError("x and xhat need the same size and dtype")
    if out.dtype != torch.float64 or out.numel() < 3:
        raise ValueError("out must hold 3 float64")
    _check(load().thc_nmse_noalloc(_dev(x, "x"), _dev(xhat, "xhat"), x.numel(), _dt(x),
                                   _dev(out, "out"), _stream(stream)))
    return out


def thc_ring_step_ws_bytes(N: int) -> int:
    return int(load().thc_ring_step_ws_bytes(N))


def thc_ring_step_launches(N: int) -> int:
    return int(load().thc_ring_step_launches(N))


def thc_ring_step(bufs: Sequence[torch.Tensor], mM: torch.Tensor, b: int, seed: int,
                  ring_part: int = 0, q_part: int = 0, worker0: int = 0,
                  packed: Optional[Sequence[torch.Tensor]] = None, keep_packed: bool = True,
                  sum_out: Optional[torch.Tensor] = None, keep_sum: bool = True,
                  xhat: Optional[torch.Tensor] = None, nmse_out: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, with_nmse: bool = True, stream=None):
    """Quantize, ring-average, integer sum, dequant and NMSE in one pass;
    returns (packed or None, sum or None, xhat, nmse or None). The ring
    average is left in every buffer."""
    P = len(bufs)
    N = bufs[0].numel()
    dev = bufs[0].device
    if keep_packed and packed is None:
        packed = [torch.empty(max(packed_bytes(N, b), 8), dtype=torch.uint8, device=dev) for _ in range(P)]
    if not keep_packed:
        packed = None
    if keep_sum and sum_out is None:
        sum_out = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
    if not keep_sum:
        sum_out = None
    if xhat is None:
        xhat = torch.empty(max(N, 1), dtype=bufs[0].dtype, device=dev)
    if with_nmse:
        if nmse_out is None:
            nmse_out = torch.empty(3, dtype=torch.float64, device=dev)
        if ws is None:
            ws = torch.empty(thc_ring_step_ws_bytes(N), dtype=torch.uint8, device=dev)
    else:
        nmse_out = ws = None
    pk = _ptr_array(packed, "packed") if packed is not None else None
    _check(load().thc_ring_step(_ptr_array(bufs, "buffer"), P, N, _dt(bufs[0]), ring_part,
                                _dev(mM, "mM"), q_part, b, seed, worker0, pk,
                                _dev(sum_out, "sum") if sum_out is not None else None,
                                _dev(xhat, "xhat"),
                                _dev(nmse_out, "nmse") if nmse_out is not None else None,
                                _dev(ws, "ws") if ws is not None else None,
                                ws.numel() if ws is not None else 0, _stream(stream)))
    return packed, sum_out, xhat, nmse_out

# ------------------------------------------------------------------ non-uniform THC
def _table_arg(T):
    return (C.c_int32 * len(T))(*[int(v) for v in T])


def thc_nuhc_quantize(bufs: Sequence[torch.Tensor], mM: torch.Tensor, b: int, g: int, table,
                      seed: int, part_elems: int = 0, worker0: int = 0,
                      packed: Optional[Sequence[torch.Tensor]] = None, stream=None):
    N = bufs[0].numel()
    if packed is None:
        packed = [torch.empty(packed_bytes(N, b), dtype=torch.uint8, device=bufs[0].device)
                  for _ in bufs]
    _check(load().thc_nuhc_quantize(_ptr_array(bufs, "buffer"), len(bufs), worker0, N,
                                    _dt(bufs[0]), part_elems, _dev(mM, "mM"), b, g, _table_arg(table),
                                    seed, _ptr_array(packed, "packed"), _stream(stream)))
    return packed


def thc_nuhc_aggregate(packed: Sequence[torch.Tensor], N: int, b: int, g: int, table,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(max(N, 1), dtype=torch.int32, device=packed[0].device)
    _check(load().thc_nuhc_aggregate(_ptr_array(packed, "packed"), len(packed), N, b, g,
                                     _table_arg(table), _dev(out, "sum"), _stream(stream)))
    return out


def thc_nuhc_dequant(S: torch.Tensor, N: int, P: int, g: int, mM: torch.Tensor, part_elems: int = 0,
                     out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(max(N, 1), dtype=out_dtype, device=S.device)
    _check(load().thc_nuhc_dequant(_dev(S, "sum"), N, P, g, part_elems, _dev(mM, "mM"),
                                   _dev(out, "out"), _dt(out), _stream(stream)))
    return out


# ------------------------------------------------------------------ error feedback
def _errs(errs: Sequence[torch.Tensor], N: int):
    if any(e.dtype != torch.float32 or e.numel() != N for e in errs):
        raise ValueError("error buffers must be float32 with N elements")
    return _ptr_array(errs, "error buffer")


def thc_ef_minmax(bufs: Sequence[torch.Tensor], errs: Sequence[torch.Tensor], part_elems: int = 0,
                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    N = bufs[0].numel()
    if out is None:
        out = torch.empty((max(n_partitions(N, part_elems), 1), 2), dtype=torch.float32,
                          device=bufs[0].device)
    _check(load().thc_ef_minmax(_ptr_array(bufs, "buffer"), _errs(errs, N), len(bufs), N,
                                _dt(bufs[0]), part_elems, _dev(out, "mM"), _stream(stream)))
    return out


def thc_ef_minmax_pair(bufs: Sequence[torch.Tensor], errs: Sequence[torch.Tensor], part_elems: int = 0,
                       out_x: Optional[torch.Tensor] = None, out_ef: Optional[torch.Tensor] = None,
                       stream=None):
    """The grids of x and of x + e in one read; returns (grids of x, grids of x + e)."""
    N = bufs[0].numel()
    shape = (max(n_partitions(N, part_elems), 1), 2)
    if out_x is None:
        out_x = torch.empty(shape, dtype=torch.float32, device=bufs[0].device)
    if out_ef is None:
        out_ef = torch.empty(shape, dtype=torch.float32, device=bufs[0].device)
    _check(load().thc_ef_minmax_pair(_ptr_array(bufs, "buffer"), _errs(errs, N), len(bufs), N,
                                     _dt(bufs[0]), part_elems, _dev(out_x, "mM"), _dev(out_ef, "mM"),
                                     _stream(stream)))
    return out_x, out_ef


def thc_ef_quantize(bufs: Sequence[torch.Tensor], errs: Sequence[torch.Tensor], mM: torch.Tensor,
                    b: int, seed: int, part_elems: int = 0, worker0: int = 0, g: int = 0, table=None,
                    packed: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """Quantize grad + e (uniform grid, or table T with granularity g) and
    overwrite e with the new residual."""
    N = bufs[0].numel()
    if packed is None:
        packed = [torch.empty(packed_bytes(N, b), dtype=torch.uint8, device=bufs[0].device)
                  for _ in bufs]
    _check(load().thc_ef_quantize(_ptr_array(bufs, "buffer"), _errs(errs, N), len(bufs), worker0,
                                  N, _dt(bufs[0]), part_elems, _dev(mM, "mM"), b, g,
                                  _table_arg(table) if table is not None else None, seed,
                                  _ptr_array(packed, "packed"), _stream(stream)))
    return packed


def thc_aggregate_dequant_ws_bytes(N: int) -> int:
    return load().thc_aggregate_dequant_ws_bytes(N)


def thc_aggregate_dequant(packed: Sequence[torch.Tensor], N: int, b: int, mM: torch.Tensor,
                          part_elems: int = 0, out_dtype=torch.float32, g: int = 0, table=None,
                          x_ref: Optional[torch.Tensor] = None, keep_sum: bool = True,
                          out: Optional[torch.Tensor] = None, S: Optional[torch.Tensor] = None,
                          nmse_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                          stream=None):
    """Integer sum, dequantized average and (with x_ref) NMSE in one pass;
    returns (S or None, x_hat, nmse or None)."""
    dev = packed[0].device
    if out is None:
        out = torch.empty(max(N, 1), dtype=out_dtype, device=dev)
    if keep_sum and S is None:
        S = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
    if x_ref is not None:
        if nmse_out is None:
            nmse_out = torch.empty(3, dtype=torch.float64, device=dev)
        if ws is None:
            ws = torch.empty(load().thc_aggregate_dequant_ws_bytes(N), dtype=torch.uint8, device=dev)
        if x_ref.dtype != out.dtype or x_ref.numel() < N:
            raise ValueError("x_ref must have the output dtype and N elements")
    _check(load().thc_aggregate_dequant(
        _ptr_array(packed, "packed"), len(packed), N, b, g,
        _table_arg(table) if table is not None else None, part_elems, _dev(mM, "mM"),
        _dev(S, "sum") if keep_sum else None, _dev(out, "out"), _dt(out),
        _dev(x_ref, "x_ref") if x_ref is not None else None,
        _dev(nmse_out, "nmse") if x_ref is not None else None,
        _dev(ws, "ws") if x_ref is not None else None,
        ws.numel() if x_ref is not None else 0, _stream(stream)))
    return (S if keep_sum else None), out, (nmse_out if x_ref is not None else None)


# ------------------------------------------------------------------ randomized Hadamard transform
def rht_padded(N: int, d: int) -> int:
    """Length of a transformed vector: N rounded up to whole blocks of d."""
    return (N + d - 1) // d * d


def thc_rht_sumsq(bufs: Sequence[torch.Tensor], d: int, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    N = bufs[0].numel()
    nblk = (N + d - 1) // d
    if out is None:
        out = torch.empty((len(bufs), max(nblk, 1)), dtype=torch.float64, device=bufs[0].device)
    _check(load().thc_rht_sumsq(_ptr_array(bufs, "buffer"), len(bufs), N, _dt(bufs[0]), d,
                                _dev(out, "sumsq"), _stream(stream)))
    return out


def thc_rht_range(sumsq: torch.Tensor, d: int, t_p: float, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """sumsq: (P, nblk) float64 on the device."""
    P, nblk = sumsq.shape
    if out is None:
        out = torch.empty((max(nblk, 1), 2), dtype=torch.float32, device=sumsq.device)
    _check(load().thc_rht_range(_dev(sumsq, "sumsq"), P, nblk, d, float(t_p), _dev(out, "mM"),
                                _stream(stream)))
    return out


def thc_rht_forward(bufs: Sequence[torch.Tensor], d: int, seed: int,
                    mM: Optional[torch.Tensor] = None,
                    y: Optional[Sequence[torch.Tensor]] = None, stream=None):
    N = bufs[0].numel()
    if y is None:
        y = [torch.empty(max(rht_padded(N, d), 1), dtype=torch.float32, device=bufs[0].device)
             for _ in bufs]
    if any(t.dtype != torch.float32 or t.numel() < rht_padded(N, d) for t in y):
        raise ValueError("y buffers must be float32 with rht_padded(N, d) elements")
    _check(load().thc_rht_forward(_ptr_array(bufs, "buffer"), len(bufs), N, _dt(bufs[0]), d, seed,
                                  _dev(mM, "mM") if mM is not None else None,
                                  _ptr_array(y, "y"), _stream(stream)))
    return y


def thc_rht_quantize(bufs: Sequence[torch.Tensor], d: int, rht_seed: int, mM: torch.Tensor, b: int,
                     q_seed: int, worker0: int = 0, g: int = 0, table=None,
                     y_scratch: Optional[Sequence[torch.Tensor]] = None,
                     packed: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """Truncated forward transform, then uniform (table None) or table
    quantization of the transformed coordinates, one partition per block;
    returns the packed indices of rht_padded(N, d) coordinates. y_scratch
    (float32, rht_padded(N, d) each) is needed when d > 8192."""
    N = bufs[0].numel()
    Np = rht_padded(N, d)
    if packed is None:
        packed = [torch.empty(max(packed_bytes(Np, b), 1), dtype=torch.uint8, device=bufs[0].device)
                  for _ in bufs]
    if any(t.numel() < packed_bytes(Np, b) for t in packed):
        raise ValueError("packed buffers must hold packed_bytes(rht_padded(N, d), b) bytes")
    if y_scratch is None and d > 8192 and N > 0:
        y_scratch = [torch.empty(Np, dtype=torch.float32, device=bufs[0].device) for _ in bufs]
    if y_scratch is not None and any(t.dtype != torch.float32 or t.numel() < Np for t in y_scratch):
        raise ValueError("y_scratch buffers must be float32 with rht_padded(N, d) elements")
    _check(load().thc_rht_quantize(_ptr_array(bufs, "buffer"), len(bufs), worker0, N, _dt(bufs[0]),
                                   d, rht_seed, _dev(mM, "mM"), b, g,
                                   _table_arg(table) if table is not None else None, q_seed,
                                   _ptr_array(y_scratch, "y_scratch") if y_scratch is not None else None,
                                   _ptr_array(packed, "packed"), _stream(stream)))
    return packed


def thc_rht_norm_quantize_ws_bytes(P: int, N: int, d: int) -> int:
    return int(load().thc_rht_norm_quantize_ws_bytes(P, N, d))


def thc_rht_norm_quantize(bufs: Sequence[torch.Tensor], d: int, rht_seed: int, t_p: float, b: int,
                          q_seed: int, worker0: int = 0, g: int = 0, table=None,
                          sumsq: Optional[torch.Tensor] = None, mM: Optional[torch.Tensor] = None,
                          y_scratch: Optional[Sequence[torch.Tensor]] = None,
                          ws: Optional[torch.Tensor] = None,
                          packed: Optional[Sequence[torch.Tensor]] = None, stream=None):
    """Block norms, range and the quantized truncated transform in one call;
    returns (packed, mM, sumsq or None)."""
    N = bufs[0].numel()
    dev = bufs[0].device
    Np = rht_padded(N, d)
    nblk = max(Np // d, 1)
    if mM is None:
        mM = torch.empty((nblk, 2), dtype=torch.float32, device=dev)
    if packed is None:
        packed = [torch.empty(max(packed_bytes(Np, b), 1), dtype=torch.uint8, device=dev) for _ in bufs]
    if y_scratch is None and d > 8192 and N > 0:
        y_scratch = [torch.empty(Np, dtype=torch.float32, device=dev) for _ in bufs]
    if ws is None:
        ws = torch.empty(max(thc_rht_norm_quantize_ws_bytes(len(bufs), N, d), 8),
                         dtype=torch.uint8, device=dev)
    _check(load().thc_rht_norm_quantize(
        _ptr_array(bufs, "buffer"), len(bufs), worker0, N, _dt(bufs[0]), d, rht_seed, float(t_p), b, g,
        _table_arg(table) if table is not None else None, q_seed,
        _dev(sumsq, "sumsq") if sumsq is not None else None, _dev(mM, "mM"),
        _ptr_array(y_scratch, "y_scratch") if y_scratch is not None else None,
        _dev(ws, "ws"), ws.numel(), _ptr_array(packed, "packed"), _stream(stream)))
    return packed, mM, sumsq


def thc_rht_inverse(y: torch.Tensor, N: int, d: int, seed: int, out_dtype=torch.float32,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y (rht_padded(N, d) float32) is overwritten when d > 8192."""
    if out is None:
        out = torch.empty(max(N, 1), dtype=out_dtype, device=y.device)
    if y.dtype != torch.float32 or y.numel() < rht_padded(N, d) or out.numel() < N:
        raise ValueError("y must hold rht_padded(N, d) float32 and out N elements")
    _check(load().thc_rht_inverse(_dev(y, "y"), N, d, seed, _dev(out, "out"), _dt(out),
                                  _stream(stream)))
    return out


def center_table(b: int, g: int, power: float = 2.0):
    """A heuristic non-uniform table: 2^b strictly increasing integers from 0
    to g, denser near the middle of the range (where bell-shaped gradients
    concentrate): T[z] ~ g (1 + sign(t) |t|^power) / 2 with t = 2z/(2^b-1) - 1,
    then forced strictly increasing. The optimal tables of the THC page come
    from an offline integer program that is not reproduced here."""
    n = 1 << b
    if g < n - 1:
        raise ValueError("granularity below 2^b - 1")
    T = []
    for z in range(n):
        t = 2.0 * z / (n - 1) - 1.0
        v = g * (1.0 + (1 if t >= 0 else -1) * abs(t) ** power) / 2.0
        T.append(int(round(v)))
    T[0] = 0
    for z in range(1, n - 1):                   # strictly increasing from the left
        T[z] = max(T[z], T[z - 1] + 1)
    T[-1] = g
    for z in range(n - 2, 0, -1):               # and fitting under g from the right
        T[z] = min(T[z], T[z + 1] - 1)
    return T
