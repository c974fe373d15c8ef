"""One pass of the whole gradient-aggregation path over a workload, on one GPU.

A step runs, in this order, on the current stream:
  fused workloads (Tensor Fusion, Horovod page section 3.4):
      zero_copy (default): ring-average every fusion buffer in place in the
      workers' tensors, all buffers in one launch, no copies;
      else: pack every worker's tensors into its fusion buffers (one
      launch), ring-average each fusion buffer across the P workers, unpack
      the averages back into the tensors (one launch); a tensor larger than
      the fusion buffer is reduced alone, in place;
  flat workloads (one gradient vector per worker):
      THC min/max per partition, USQ quantize for every bit width but the
      first (these read the workers' gradients before the ring overwrites
      them),
      for every THC pass behind the randomized Hadamard transform (THC page
      section 5): per-block norms, the norm-based range, the transform with
      truncation, the table quantizer on the transformed coordinates,
      for every error-feedback pass (THC page section 5): min/max and the
      quantizer on gradient + residual, the residual written back,
      one pass (thc_ring_step) that quantizes the first bit width, leaves
      the ring's exact average in place and sums, dequantizes and measures
      that width's estimate against the average (fused_step; else the
      quantizer, the ring and the tail as three calls),
      then per remaining pass: integer aggregate, dequantize, NMSE of the
      THC estimate against the exact average (for RHT passes: table-sum
      aggregate, dequantize, inverse transform, NMSE); the partial pass
      (THC page section 8) sums only the workers that arrived and divides
      by their count.

Only the binding is called; all arithmetic runs in libga.so. Per-call HIP
events (torch.cuda.Event on the stream the kernels are launched on) time
every stage when a timer is passed.
"""
import statistics
from collections import defaultdict
from typing import Dict, List, Optional

import numpy as np
import torch

from . import _native as ga
from . import synth

# ring_mode value (beside ga.RING_FUSED and ga.RING_DUAL) selecting
# ga_ring_stepwise_staged: the schedule one launch per step, binary32
# partials staged between steps (flat workloads)
RING_STAGED = "staged"


class StageTimer:
    """Events around every library call of a step, per stage name."""

    def __init__(self):
        self.pairs: Dict[str, list] = defaultdict(list)

    def wrap(self, name: str, fn, *a, **k):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn(*a, **k)
        e.record()
        self.pairs[name].append((s, e))
        return out

    def mean_ms(self) -> Dict[str, float]:
        torch.cuda.synchronize()
        return {k: float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in self.pairs.items()}

    def count(self) -> Dict[str, int]:
        return {k: len(v) for k, v in self.pairs.items()}


def _call(timer: Optional[StageTimer], name: str, fn, *a, **k):
    if timer is None:
        return fn(*a, **k)
    return timer.wrap(name, fn, *a, **k)


# Worker buffers whose byte size is a multiple of 64 KiB would start at the
# same offset modulo the HBM channel-interleave period, so the P concurrent
# streams of the ring (same element of every worker) fall on the same
# channels. Such buffers are carved from one allocation with a 12 KiB skew
# between workers (measured on MI355X: 8 x 4 GiB ring 70.6% -> 74.6% of
# peak); other sizes keep one allocation per worker, which measured best.
SKEW_BYTES = 12 << 10


def worker_buffers(P: int, N: int, dtype, device) -> List[torch.Tensor]:
    es = torch.empty((), dtype=dtype).element_size()
    nbytes = N * es
    if P > 1 and nbytes % (64 << 10) == 0:
        stride = (nbytes + SKEW_BYTES) // es
        slab = torch.empty(stride * P, dtype=dtype, device=device)
        return [slab[i * stride: i * stride + N] for i in range(P)]
    return [torch.empty(N, dtype=dtype, device=device) for _ in range(P)]


def t_p(p: float) -> float:
    """Truncation threshold Phi^-1(1 - p/2) of a standard normal."""
    return statistics.NormalDist().inv_cdf(1.0 - p / 2.0)


class Pipeline:
    nu_tables: Dict[str, tuple] = {}
    rht: Dict[str, tuple] = {}

    def __init__(self, name, device="cuda", cap_bytes: int = 64 << 20, zero_copy: bool = True,
                 ring_mode: int = ga.RING_FUSED, fused_tail: bool = True, fused_step: bool = True):
        # a workload by name, or a synth.Workload built by the caller
        self.w = synth.workload(name) if isinstance(name, str) else name
        self.zero_copy = zero_copy
        # the first uniform THC pass, the ring average and that pass's sum,
        # dequant and NMSE in one read (thc_ring_step), where the sizes allow
        # and it measured faster: binary32 at any P (lane pairs; 32 x 138M,
        # b = 4: 7.97 ms against 10.6 ms for the three calls) and bf16 up to
        # 16 workers (8 x 2^31 bf16, b = 2: 13.9 ms against 22.0 ms; 16 x
        # 2^28: 3.5 against 5.8). bf16 holds whole groups per thread, whose
        # loads at 32 workers stay live for the rounding.
        w = self.w
        if ring_mode == RING_STAGED and w.fused:
            raise ValueError("the staged stepwise schedule runs on flat workloads")
        self.fused_step = (fused_step and not w.fused and bool(w.thc_bits) and w.N % 8 == 0
                           and w.part_elems % 8 == 0 and ring_mode == ga.RING_FUSED
                           and (w.dtype == ga.F32 or w.P <= 16))
        # THC's integer sum, dequant and NMSE in one pass (thc_aggregate_dequant)
        # or as the three separate calls
        self.fused_tail = fused_tail
        self.ring_mode = ring_mode
        self.device = torch.device(device)
        self.cap = cap_bytes
        self.tdt = torch.float32 if self.w.dtype == ga.F32 else torch.bfloat16
        self.P = self.w.P
        self.N = self.w.N
        self.nmse: Dict[int, torch.Tensor] = {}

    # ------------------------------------------------------------ setup
    def setup(self) -> None:
        w, dev = self.w, self.device
        if w.fused:
            self.tensors = [synth.worker_tensors(w, i, dev) for i in range(self.P)]
            self.buf_of, self.off_of, self.fill, _ = ga.ga_fuse_plan(w.sizes, None, self.cap)
            if self.zero_copy:
                self.fring = ga.FusionRing(self.tensors, self.buf_of, self.off_of, self.fill)
                torch.cuda.synchronize()
                return
            es = w.elem_bytes
            # a buffer holding one tensor larger than the capacity: reduce that
            # tensor in place instead of copying it
            self.alone = {k for k, f in enumerate(self.fill) if f * es > self.cap}
            self.bufs = [[None if k in self.alone else torch.empty(f, dtype=self.tdt, device=dev)
                          for k, f in enumerate(self.fill)] for _ in range(self.P)]
            for k in self.alone:
                t = self.buf_of.index(k)
                for i in range(self.P):
                    self.bufs[i][k] = self.tensors[i][t]
            keep = [t for t in range(len(w.sizes)) if self.buf_of[t] not in self.alone]
            self.tables = ga.FusionTables([[self.tensors[i][t] for t in keep] for i in range(self.P)],
                                          self.bufs, [self.buf_of[t] for t in keep],
                                          [self.off_of[t] for t in keep]) if keep else None
        else:
            self.flat = worker_buffers(self.P, self.N, self.tdt, dev)
            for i in range(self.P):
                synth.worker_flat(w, i, self.flat[i])
            n_part = ga.n_partitions(self.N, w.part_elems)
            self.mM = torch.empty((n_part, 2), dtype=torch.float32, device=dev)
            self.packed = {b: [torch.empty(ga.packed_bytes(self.N, b), dtype=torch.uint8, device=dev)
                               for _ in range(self.P)] for b in w.thc_bits}
            self.S = {b: torch.empty(self.N, dtype=torch.int32, device=dev) for b in w.thc_bits}
            self.xhat = {b: torch.empty(self.N, dtype=self.tdt, device=dev) for b in w.thc_bits}
            self.nmse = {b: torch.empty(3, dtype=torch.float64, device=dev) for b in w.thc_bits}
            # uniform passes with one grid over the whole vector, keyed "g{b}"
            self.mM_g = torch.empty((1, 2), dtype=torch.float32, device=dev)
            for b in w.global_bits:
                k = f"g{b}"
                self.packed[k] = [torch.empty(ga.packed_bytes(self.N, b), dtype=torch.uint8,
                                              device=dev) for _ in range(self.P)]
                self.S[k] = torch.empty(self.N, dtype=torch.int32, device=dev)
                self.xhat[k] = torch.empty(self.N, dtype=self.tdt, device=dev)
                self.nmse[k] = torch.empty(3, dtype=torch.float64, device=dev)
            # non-uniform THC passes, keyed "nu{b}g{g}", with a centre-dense table
            self.nu_tables = {f"nu{b}g{g}": (b, g, ga.center_table(b, g)) for b, g in w.nuhc}
            for k, (b, g, _) in self.nu_tables.items():
                self.packed[k] = [torch.empty(ga.packed_bytes(self.N, b), dtype=torch.uint8,
                                              device=dev) for _ in range(self.P)]
                self.S[k] = torch.empty(self.N, dtype=torch.int32, device=dev)
                self.xhat[k] = torch.empty(self.N, dtype=self.tdt, device=dev)
                self.nmse[k] = torch.empty(3, dtype=torch.float64, device=dev)
            # RHT passes, keyed "rht{b}g{g}d{log2 d}"; the quantizer's partitions
            # are the transform's blocks
            self.rht = {f"rht{b}g{g}d{k}": (b, g, 1 << k, ga.center_table(b, g))
                        for b, g, k in w.rht}
            self.rht_y, self.rht_sumsq, self.rht_mM, self.rht_avg, self.rht_ws = {}, {}, {}, {}, {}
            for key, (b, g, d, _) in self.rht.items():
                Np = ga.rht_padded(self.N, d)
                # scratch of the transform's first pass (blocks above 8192)
                self.rht_y[key] = worker_buffers(self.P, Np, torch.float32, dev) if d > 8192 else None
                self.rht_sumsq[key] = torch.empty((self.P, Np // d), dtype=torch.float64, device=dev)
                self.rht_ws[key] = torch.empty(
                    max(ga.load().thc_rht_norm_quantize_ws_bytes(self.P, self.N, d), 8),
                    dtype=torch.uint8, device=dev)
                self.rht_mM[key] = torch.empty((Np // d, 2), dtype=torch.float32, device=dev)
                self.packed[key] = [torch.empty(ga.packed_bytes(Np, b), dtype=torch.uint8,
                                                device=dev) for _ in range(self.P)]
                self.S[key] = torch.empty(Np, dtype=torch.int32, device=dev)
                self.rht_avg[key] = torch.empty(Np, dtype=torch.float32, device=dev)
                self.xhat[key] = torch.empty(self.N, dtype=self.tdt, device=dev)
                self.nmse[key] = torch.empty(3, dtype=torch.float64, device=dev)
            # error-feedback passes, keyed "ef{b}", residuals start at zero
            self.err, self.mM_ef = {}, {}
            for b in w.ef_bits:
                k = f"ef{b}"
                self.err[k] = worker_buffers(self.P, self.N, torch.float32, dev)
                for e in self.err[k]:
                    e.zero_()
                self.mM_ef[k] = torch.empty((n_part, 2), dtype=torch.float32, device=dev)
                self.packed[k] = [torch.empty(ga.packed_bytes(self.N, b), dtype=torch.uint8,
                                              device=dev) for _ in range(self.P)]
                self.S[k] = torch.empty(self.N, dtype=torch.int32, device=dev)
                self.xhat[k] = torch.empty(self.N, dtype=self.tdt, device=dev)
                self.nmse[k] = torch.empty(3, dtype=torch.float64, device=dev)
            # partial aggregation of the first uniform pass without the stragglers
            self.dropped = synth.straggler_set(w)
            self.arrived = [i for i in range(self.P) if i not in self.dropped]
            if self.dropped and w.thc_bits:
                k = f"part{w.thc_bits[0]}"
                self.S[k] = torch.empty(self.N, dtype=torch.int32, device=dev)
                self.xhat[k] = torch.empty(self.N, dtype=self.tdt, device=dev)
                self.nmse[k] = torch.empty(3, dtype=torch.float64, device=dev)
            self.ws = torch.empty(ga.thc_nmse_ws_bytes(self.N), dtype=torch.uint8, device=dev)
            self.ws_step = torch.empty(ga.thc_ring_step_ws_bytes(self.N), dtype=torch.uint8, device=dev)
            self.ws_ad = torch.empty(ga.thc_aggregate_dequant_ws_bytes(self.N), dtype=torch.uint8,
                                     device=dev)
            if self.ring_mode == RING_STAGED:
                self.stage = torch.empty(max(ga.ga_ring_stage_bytes(self.P, self.N) // 4, 1),
                                         dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    # ------------------------------------------------------------ step
    def step(self, timer: Optional[StageTimer] = None) -> None:
        w = self.w
        if w.fused and self.zero_copy:
            _call(timer, "fusion_ring", self.fring.allreduce, ga.AVG, self.ring_mode,
                  w.ring_part_elems)
            return
        if w.fused:
            if self.tables is not None:
                _call(timer, "fuse_pack", self.tables.pack)
            for k in range(len(self.fill)):
                _call(timer, "ring_allreduce", ga.ga_ring_allreduce_sim,
                      [self.bufs[i][k] for i in range(self.P)], ga.AVG, w.ring_part_elems,
                      self.ring_mode)
            if self.tables is not None:
                _call(timer, "fuse_unpack", self.tables.unpack)
            return
        part = w.part_elems
        b0 = w.thc_bits[0] if self.fused_step else None
        # with error feedback, the partition grids of x and of the first
        # error-feedback pass's x + e in one read of x and e
        ef0 = f"ef{w.ef_bits[0]}" if w.ef_bits else None
        if ef0:
            _call(timer, f"thc_ef_minmax_pair_{ef0}", ga.thc_ef_minmax_pair, self.flat, self.err[ef0], part,
                  self.mM, self.mM_ef[ef0])
        else:
            _call(timer, "thc_minmax", ga.thc_minmax, self.flat, part, self.mM)
        for b in w.thc_bits:
            if b == b0:
                continue
            _call(timer, f"thc_usq_quantize_b{b}", ga.thc_usq_quantize, self.flat, self.mM, b,
                  w.quant_seed, part, 0, self.packed[b])
        if w.global_bits:
            # the whole vector's grid from the partition grids (no second read)
            _call(timer, "thc_minmax_global", ga.thc_minmax_combine, self.mM, self.mM_g)
        for b in w.global_bits:
            _call(timer, f"thc_usq_quantize_g{b}", ga.thc_usq_quantize, self.flat, self.mM_g, b,
                  w.quant_seed, 0, 0, self.packed[f"g{b}"])
        for k, (b, g, T) in self.nu_tables.items():
            _call(timer, f"thc_nuhc_quantize_{k}", ga.thc_nuhc_quantize, self.flat, self.mM, b, g, T,
                  w.quant_seed, part, 0, self.packed[k])
        tp = t_p(w.rht_p)
        for key, (b, g, d, T) in self.rht.items():
            _call(timer, f"thc_rht_norm_quantize_{key}", ga.thc_rht_norm_quantize, self.flat, d,
                  w.rht_seed, tp, b, w.quant_seed, 0, g, T, self.rht_sumsq[key], self.rht_mM[key],
                  self.rht_y[key], self.rht_ws[key], self.packed[key])
        for b in w.ef_bits:
            k = f"ef{b}"
            if k != ef0:
                _call(timer, f"thc_ef_minmax_{k}", ga.thc_ef_minmax, self.flat, self.err[k], part,
                      self.mM_ef[k])
            _call(timer, f"thc_ef_quantize_{k}", ga.thc_ef_quantize, self.flat, self.err[k],
                  self.mM_ef[k], b, w.quant_seed, part, 0, 0, None, self.packed[k])
        if self.fused_step:
            _call(timer, f"thc_ring_step_b{b0}", ga.thc_ring_step, self.flat, self.mM, b0, w.quant_seed,
                  w.ring_part_elems, part, 0, self.packed[b0], True, self.S[b0], True, self.xhat[b0],
                  self.nmse[b0], self.ws_step)
        elif self.ring_mode == RING_STAGED:
            _call(timer, "ring_staged", ga.ga_ring_stepwise_staged, self.flat, ga.AVG,
                  w.ring_part_elems, self.stage)
        else:
            _call(timer, "ring_allreduce", ga.ga_ring_allreduce_sim, self.flat, ga.AVG,
                  w.ring_part_elems, self.ring_mode)
        for b in w.ef_bits:
            k = f"ef{b}"
            self._tail(timer, k, self.packed[k], b, self.mM_ef[k], part)
        if self.dropped and w.thc_bits:
            b = w.thc_bits[0]
            self._tail(timer, f"part{b}", [self.packed[b][i] for i in self.arrived], b, self.mM, part)
        for key, (b, g, d, T) in self.rht.items():
            Np = self.rht_avg[key].numel()
            self._tail(timer, key, self.packed[key], b, self.rht_mM[key], d, g=g, table=T, n=Np,
                       out=self.rht_avg[key], nmse=False)
            _call(timer, f"thc_rht_inverse_{key}", ga.thc_rht_inverse, self.rht_avg[key], self.N, d,
                  w.rht_seed, self.tdt, self.xhat[key])
            _call(timer, f"thc_nmse_{key}", ga.thc_nmse, self.flat[0], self.xhat[key], self.nmse[key],
                  self.ws)
        for k, (b, g, T) in self.nu_tables.items():
            self._tail(timer, k, self.packed[k], b, self.mM, part, g=g, table=T)
        for b in w.thc_bits:
            if b != b0:
                self._tail(timer, f"b{b}", self.packed[b], b, self.mM, part, sum_key=b)
        for b in w.global_bits:
            k = f"g{b}"
            self._tail(timer, k, self.packed[k], b, self.mM_g, 0)

    def _tail(self, timer, key, packed, b, mM, part, g=0, table=None, n=None, out=None, nmse=True,
              sum_key=None):
        """Server sum, dequantized average and NMSE of one THC pass: one fused
        call, or thc_(nuhc_)aggregate, thc_(nuhc_)dequant and thc_nmse."""
        n = self.N if n is None else n
        sk = key if sum_key is None else sum_key
        out = self.xhat[sk] if out is None else out
        odt = out.dtype
        nP = len(packed)
        if self.fused_tail:
            _call(timer, f"thc_aggregate_dequant_{key}", ga.thc_aggregate_dequant, packed, n, b, mM,
                  part, odt, g, table, self.flat[0] if nmse else None, True, out, self.S[sk],
                  self.nmse[sk] if nmse else None, self.ws_ad if nmse else None)
            return
        if table is None:
            _call(timer, f"thc_int_aggregate_{key}", ga.thc_int_aggregate, packed, n, b, self.S[sk])
            _call(timer, f"thc_dequant_{key}", ga.thc_dequant, self.S[sk], n, nP, b, mM, part, odt, out)
        else:
            _call(timer, f"thc_nuhc_aggregate_{key}", ga.thc_nuhc_aggregate, packed, n, b, g, table,
                  self.S[sk])
            _call(timer, f"thc_nuhc_dequant_{key}", ga.thc_nuhc_dequant, self.S[sk], n, nP, g, mM, part,
                  odt, out)
        if nmse:
            _call(timer, f"thc_nmse_{key}", ga.thc_nmse, self.flat[0], out, self.nmse[sk], self.ws)

    # ------------------------------------------------------------ graphs
    def state_buffers(self) -> List[torch.Tensor]:
        """Every buffer a step reads and then overwrites: the gradients (the
        ring leaves their average in them) and the error-feedback residuals."""
        if self.w.fused:
            return [t for ts in self.tensors for t in ts]
        return list(self.flat) + [e for k in self.err for e in self.err[k]]

    def capture(self, warmup: int = 2) -> torch.cuda.CUDAGraph:
        """One step recorded into a HIP graph: every call of a step only
        enqueues kernels (no allocation, copy or memset), so the graph holds
        the step's kernels with their arguments; replay() runs it again on the
        same buffers. The warm-up steps (on a side stream, as capture wants)
        run first and change the state buffers like any step."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                self.step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step()
        return graph

    # ------------------------------------------------------------ accounting
    def stage_bytes(self) -> Dict[str, float]:
        """Algorithmic HBM bytes of one call of each stage (per launch)."""
        w, P, N, s = self.w, self.P, self.N, self.w.elem_bytes
        out = {}
        if w.fused and self.zero_copy:
            out["fusion_ring"] = 2.0 * P * N * s                     # every buffer, one launch
            return out
        if w.fused:
            moved = sum(int(n) for t, n in enumerate(w.sizes) if self.buf_of[t] not in self.alone)
            out["fuse_pack"] = out["fuse_unpack"] = 2.0 * P * moved * s
            out["ring_allreduce"] = 2.0 * P * N * s / len(self.fill)   # mean over the buffers
            return out
        out["thc_minmax"] = 1.0 * P * N * s
        out["ring_allreduce"] = 2.0 * P * N * s
        # the staged schedule, all 2 (P - 1) launches: step 0 reads two
        # buffers and writes the binary32 stage, the middle steps read the
        # stage and a buffer and write the stage, the last reads the stage
        # and a buffer and writes a buffer; each all-gather step copies N
        rs = (3 * s * N if P == 2 else
              (2 * s + 4) * N + (P - 3) * (8 + s) * N + (4 + 2 * s) * N) if P > 1 else 0
        out["ring_staged"] = float(rs + (P - 1) * 2 * s * N)
        for b in w.thc_bits:
            # gradients read once and the average written back, the indices,
            # the sums and the estimate written
            out[f"thc_ring_step_b{b}"] = 2.0 * P * N * s + P * N * b / 8.0 + 4.0 * N + N * s
        for b in w.thc_bits:
            out[f"thc_usq_quantize_b{b}"] = P * N * (s + b / 8.0)
            out[f"thc_int_aggregate_b{b}"] = P * N * b / 8.0 + 4.0 * N
            out[f"thc_dequant_b{b}"] = 4.0 * N + N * s
            out[f"thc_nmse_b{b}"] = 2.0 * N * s
        if w.global_bits:
            out["thc_minmax_global"] = 8.0 * ga.n_partitions(N, w.part_elems)   # the partition grids
        for b in w.global_bits:
            k = f"g{b}"
            out[f"thc_usq_quantize_{k}"] = P * N * (s + b / 8.0)
            out[f"thc_int_aggregate_{k}"] = P * N * b / 8.0 + 4.0 * N
            out[f"thc_dequant_{k}"] = 4.0 * N + N * s
            out[f"thc_nmse_{k}"] = 2.0 * N * s
        for k, (b, g, _) in self.nu_tables.items():
            out[f"thc_nuhc_quantize_{k}"] = P * N * (s + b / 8.0)
            out[f"thc_nuhc_aggregate_{k}"] = P * N * b / 8.0 + 4.0 * N
            out[f"thc_nuhc_dequant_{k}"] = 4.0 * N + N * s
            out[f"thc_nmse_{k}"] = 2.0 * N * s
        for b in w.ef_bits:
            k = f"ef{b}"
            out[f"thc_ef_minmax_{k}"] = P * N * (s + 4.0)
            out[f"thc_ef_minmax_pair_{k}"] = P * N * (s + 4.0)      # x and e read once, both grids
            out[f"thc_ef_quantize_{k}"] = P * N * (s + 8.0 + b / 8.0)
            out[f"thc_int_aggregate_{k}"] = P * N * b / 8.0 + 4.0 * N
            out[f"thc_dequant_{k}"] = 4.0 * N + N * s
            out[f"thc_nmse_{k}"] = 2.0 * N * s
        if self.dropped and w.thc_bits:
            b = w.thc_bits[0]
            k = f"part{b}"
            out[f"thc_int_aggregate_{k}"] = len(self.arrived) * N * b / 8.0 + 4.0 * N
            out[f"thc_dequant_{k}"] = 4.0 * N + N * s
            out[f"thc_nmse_{k}"] = 2.0 * N * s
        for k, (b, g, d, _) in self.rht.items():
            Np = ga.rht_padded(N, d)
            nblk = Np // d
            out[f"thc_rht_norm_quantize_{k}"] = P * N * s + P * Np * b / 8.0 + 16.0 * P * nblk
            out[f"thc_rht_sumsq_{k}"] = P * N * s + 8.0 * P * nblk
            out[f"thc_rht_range_{k}"] = 8.0 * P * nblk + 8.0 * nblk
            out[f"thc_rht_quantize_{k}"] = P * N * s + P * Np * b / 8.0
            out[f"thc_nuhc_aggregate_{k}"] = P * Np * b / 8.0 + 4.0 * Np
            out[f"thc_nuhc_dequant_{k}"] = 8.0 * Np
            out[f"thc_rht_inverse_{k}"] = 4.0 * Np + N * s
            out[f"thc_nmse_{k}"] = 2.0 * N * s
        # the fused tail: packed indices in, sums and estimate out, the
        # exact average read for the NMSE
        def fused(nP, n, b, s_out, nmse):
            return nP * n * b / 8.0 + 4.0 * n + n * s_out + (n * s if nmse else 0.0)
        for b in w.thc_bits:
            out[f"thc_aggregate_dequant_b{b}"] = fused(P, N, b, s, True)
        for b in w.global_bits:
            out[f"thc_aggregate_dequant_g{b}"] = fused(P, N, b, s, True)
        for k, (b, g, _) in self.nu_tables.items():
            out[f"thc_aggregate_dequant_{k}"] = fused(P, N, b, s, True)
        for b in w.ef_bits:
            out[f"thc_aggregate_dequant_ef{b}"] = fused(P, N, b, s, True)
        if self.dropped and w.thc_bits:
            b = w.thc_bits[0]
            out[f"thc_aggregate_dequant_part{b}"] = fused(len(self.arrived), N, b, s, True)
        for k, (b, g, d, _) in self.rht.items():
            out[f"thc_aggregate_dequant_{k}"] = fused(P, ga.rht_padded(N, d), b, 4.0, False)
        return out

    # ------------------------------------------------------------ sampling
    def partition_ranges(self, which: List[int]):
        plen = self.w.part_elems or self.N
        return [(p, p * plen, min((p + 1) * plen, self.N)) for p in which]

    def n_partitions(self) -> int:
        return ga.n_partitions(self.N, self.w.part_elems)

    def sample_inputs(self, which: List[int]) -> Dict[int, List[np.ndarray]]:
        """Host copies of every worker's elements of the chosen partitions."""
        out = {}
        for p, lo, hi in self.partition_ranges(which):
            out[p] = [synth.to_numpy_bits(self.flat[i][lo:hi]) for i in range(self.P)]
        return out

    def sample_outputs(self, which: List[int]) -> Dict[int, dict]:
        out = {}
        for p, lo, hi in self.partition_ranges(which):
            d = {"ring": [synth.to_numpy_bits(self.flat[i][lo:hi]) for i in range(self.P)],
                 "mM": self.mM[p].cpu().numpy().copy(), "packed": {}, "xhat": {}, "S": {}}
            for b in self.w.thc_bits:
                bl, bh = lo * b // 8, (hi * b + 7) // 8
                d["packed"][b] = [self.packed[b][i][bl:bh].cpu().numpy().copy()
                                  for i in range(self.P)]
                d["xhat"][b] = synth.to_numpy_bits(self.xhat[b][lo:hi])
                d["S"][b] = self.S[b][lo:hi].cpu().numpy().copy()
            d["mM_g"] = self.mM_g[0].cpu().numpy().copy()
            for b in self.w.global_bits:
                k = f"g{b}"
                bl, bh = lo * b // 8, (hi * b + 7) // 8
                d["packed"][k] = [self.packed[k][i][bl:bh].cpu().numpy().copy()
                                  for i in range(self.P)]
                d["xhat"][k] = synth.to_numpy_bits(self.xhat[k][lo:hi])
                d["S"][k] = self.S[k][lo:hi].cpu().numpy().copy()
            for k, (b, g, _) in self.nu_tables.items():
                bl, bh = lo * b // 8, (hi * b + 7) // 8
                d["packed"][k] = [self.packed[k][i][bl:bh].cpu().numpy().copy()
                                  for i in range(self.P)]
                d["xhat"][k] = synth.to_numpy_bits(self.xhat[k][lo:hi])
                d["S"][k] = self.S[k][lo:hi].cpu().numpy().copy()
            d["err"], d["mM_ef"] = {}, {}
            for b in self.w.ef_bits:
                k = f"ef{b}"
                bl, bh = lo * b // 8, (hi * b + 7) // 8
                d["packed"][k] = [self.packed[k][i][bl:bh].cpu().numpy().copy()
                                  for i in range(self.P)]
                d["xhat"][k] = synth.to_numpy_bits(self.xhat[k][lo:hi])
                d["S"][k] = self.S[k][lo:hi].cpu().numpy().copy()
                d["err"][k] = [self.err[k][i][lo:hi].cpu().numpy().copy() for i in range(self.P)]
                d["mM_ef"][k] = self.mM_ef[k][p].cpu().numpy().copy()
            if self.dropped and self.w.thc_bits:
                k = f"part{self.w.thc_bits[0]}"
                d["xhat"][k] = synth.to_numpy_bits(self.xhat[k][lo:hi])
                d["S"][k] = self.S[k][lo:hi].cpu().numpy().copy()
            out[p] = d
        return out

    def sample_rht_outputs(self, key: str, which: List[int]) -> Dict[int, dict]:
        """Block p of an RHT pass: its range, every worker's packed indices
        (whole block, padding included), the table sums and the estimate."""
        b, g, d, _ = self.rht[key]
        out = {}
        for p in which:
            lo, hi = p * d, min((p + 1) * d, self.N)
            bl, bh = lo * b // 8, (lo + d) * b // 8
            out[p] = {"mM": self.rht_mM[key][p].cpu().numpy().copy(),
                      "packed": [self.packed[key][i][bl:bh].cpu().numpy().copy()
                                 for i in range(self.P)],
                      "S": self.S[key][lo:lo + d].cpu().numpy().copy(),
                      "xhat": synth.to_numpy_bits(self.xhat[key][lo:hi])}
        return out
