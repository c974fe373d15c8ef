"""Throughput of the whole gradient-aggregation hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload shard]

One step is one pass of every stage over one batch of synthetic gradients
already resident in HBM (see gradient_all_reduce_worker_amd.pipeline):
for the default workload, 8 simulated workers x 2^31 bf16 gradients each
(Laplace(0, 1e-3)): THC min/max, then one pass that quantizes (USQ b = 2),
ring-averages with fp32 accumulation over 2^20-element partitions, sums the
indices as integers, dequantizes and measures the NMSE (thc_ring_step;
--separate-step runs the quantizer, the ring and the tail as their own
calls). `value` is aggregated gradient bytes (P N elem_bytes) per second of
step time.

Prints ONE JSON line. `roofline` describes the dominant kernel (the
one-read step pass, or the ring where there is none) from HIP events around
its launches inside the timed steps;
`cpu_baseline` times the oracle (plain C) on this host's cores, beside its
one-thread figure: sampled whole partitions of a flat workload, or the
whole pack-ring-unpack step of a fused one; `traffic` comes from the
committed rocprofv3 PMC summary when it was taken on the current ring
source, else null.
"""
import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "aggregated gradient GB/s (P·N·bytes/s) vs HBM peak; THC quantize Gelem/s + NMSE"
HBM_PEAK_GBS = 8000.0
# rocprofv3 PMC summaries of the dominant kernel, per workload: profiles/
# ring_fused_<workload>_pmc.json (flat ring) or fusion_ring_<workload>_pmc.json
# (zero-copy fusion ring), each stamped with the ring source's hash
PMC_FILE = {"ring_fused_vec_kernel": "ring_fused_{}_pmc.json",
            "thc_ring_lane_kernel": "thc_ring_lane_{}_pmc.json",
            "fusion_ring_kernel": "fusion_ring_{}_pmc.json",
            "thc_ring_kernel": "thc_ring_{}_pmc.json"}
CSRC = os.path.join(ROOT, "gradient_all_reduce_worker_amd", "csrc")
KERNEL_SRC = {"ring_fused_vec_kernel": "ring.hip", "fusion_ring_kernel": "ring.hip",
              "thc_ring_lane_kernel": "step.hip",
              "thc_ring_kernel": "step.hip"}

DESCRIPTIONS = {
    "small": "4 workers x 1,048,576 fp32 N(0,0.01^2); ring avg + THC USQ b=4",
    "fusion": "8 workers x 200 fp32 tensors (log-uniform 1K..256K); 64 MiB fusion, ring avg",
    "resnet101": "16 workers x ResNet-101 gradients (314 tensors, 44,549,160 fp32); fusion + ring avg",
    "vgg16": ("32 workers x VGG-16 gradients (138,357,544 fp32); THC USQ b=4,8 (2^20-element "
              "partition grids), USQ b=4 on one grid for the whole vector, table THC "
              "b=4 g=36, RHT (d=2^20, p=1/32) + table THC b=4 g=36 + inverse, USQ b=4 with error "
              "feedback, b=4 partial aggregation without 3 stragglers; ring avg; NMSE"),
    "shard": ("8 workers x 2,147,483,648 bf16 Laplace(0,1e-3); ring avg with fp32 accumulation "
              "in 2^20-element partitions + THC USQ b=2 (uint8-packed), int32 sum, dequant, NMSE"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    with open(os.path.join(CSRC, KERNEL_SRC[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def runtime_copy_rate(nbytes: int = 4 << 30, reps: int = 5) -> dict:
    """The HIP runtime's own device-to-device copy of nbytes (its copy
    kernel: one read and one write stream), timed on this machine after the
    bench's steps. Context for `frac`, not a ceiling: MI355X machines differ
    by several percent for the same streaming kernel, and this shows what a
    vendor streaming kernel reaches on the same machine in the same run."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(reps):
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    t = sorted(ms)[reps // 2]
    gbs = 2 * nbytes / (t * 1e-3) / 1e9
    return {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes": 2 * nbytes}


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from the committed PMC
    summary, if one was measured on this workload and on the kernel's
    current source; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", PMC_FILE[kernel].format(workload))) as f:
            d = json.load(f)
    except (OSError, ValueError, KeyError):
        return None
    if d.get("workload") != workload or d.get("ring_src_sha256_16") != source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


def host_threads() -> int:
    """Host threads for the oracle: the cores this process may run on
    (bounded by OMP_NUM_THREADS when set, and by 16, one GPU's share of the
    host)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(n, 16))


def oracle_partition(pipe, p, inputs) -> int:
    """The oracle over one partition of a flat workload, every stage of the
    step in the step's order; returns the partition's element count."""
    import numpy as np

    import oracle
    from gradient_all_reduce_worker_amd.pipeline import t_p

    w, P = pipe.w, pipe.P
    xs = [a.copy() for a in inputs]
    n = xs[0].size
    lo = p * (w.part_elems or pipe.N)
    mM = oracle.minmax(xs, n)
    packed = {b: [oracle.usq_quantize(xs[i], i, n, mM, b, w.quant_seed, e_offset=lo)
                  for i in range(P)] for b in w.thc_bits}
    if w.global_bits:                               # the partition's extremes stand in for the
        mg = oracle.minmax(xs, 0)                   # whole vector's (same work per element)
    for b in w.global_bits:
        packed[f"g{b}"] = [oracle.usq_quantize(xs[i], i, 0, mg, b, w.quant_seed, e_offset=lo)
                           for i in range(P)]
    for k, (b, g, T) in pipe.nu_tables.items():
        packed[k] = [oracle.nuhc_quantize(xs[i], i, n, mM, b, g, T, w.quant_seed, e_offset=lo)
                     for i in range(P)]
    ef = {}
    for b in w.ef_bits:                             # first step: residuals are zero
        xe = [oracle.ef_add(x, np.zeros(n, dtype=np.float32)) for x in xs]
        me = oracle.minmax(xe, n)
        pk = [oracle.usq_quantize(xe[i], i, n, me, b, w.quant_seed, e_offset=lo) for i in range(P)]
        [oracle.ef_update(xe[i], pk[i], b, n, me) for i in range(P)]
        ef[b] = (me, pk)
    rht = {}
    tp = t_p(w.rht_p)
    for k, (b, g, d, T) in pipe.rht.items():       # blocks of d are the partitions
        rm = oracle.rht_range(np.stack([oracle.rht_sumsq(x, d) for x in xs]), d, tp)
        ys = [oracle.clamp(oracle.rht_forward(x, d, w.rht_seed, e0=lo), d, rm) for x in xs]
        rht[k] = (rm, [oracle.nuhc_quantize(ys[i], i, d, rm, b, g, T, w.quant_seed, e_offset=lo)
                       for i in range(P)])
    oracle.ring_fold(xs, op=oracle.AVG, part=w.ring_part_elems and n)
    for b in w.thc_bits:
        S = oracle.int_aggregate(packed[b], n, b)
        oracle.nmse(xs[0], oracle.dequant(S, P, b, n, mM, w.dtype))
    for b in w.global_bits:
        S = oracle.int_aggregate(packed[f"g{b}"], n, b)
        oracle.nmse(xs[0], oracle.dequant(S, P, b, 0, mg, w.dtype))
    for k, (b, g, T) in pipe.nu_tables.items():
        Y = oracle.nuhc_aggregate(packed[k], n, b, g, T)
        oracle.nmse(xs[0], oracle.nuhc_dequant(Y, P, g, n, mM, w.dtype))
    for b, (me, pk) in ef.items():
        oracle.nmse(xs[0], oracle.dequant(oracle.int_aggregate(pk, n, b), P, b, n, me, w.dtype))
    if len(pipe.arrived) < P and w.thc_bits:
        b = w.thc_bits[0]
        S = oracle.int_aggregate([packed[b][i] for i in pipe.arrived], n, b)
        oracle.nmse(xs[0], oracle.dequant(S, len(pipe.arrived), b, n, mM, w.dtype))
    for k, (b, g, d, T) in pipe.rht.items():
        rm, pk = rht[k]
        avg = oracle.nuhc_dequant(oracle.nuhc_aggregate(pk, d, b, g, T), P, g, d, rm)
        oracle.nmse(xs[0], oracle.rht_inverse(avg, d, w.rht_seed, w.dtype, e0=lo)[:n])
    return n


def cpu_baseline_flat(pipe, samples, budget_s: float, threads: int):
    """The oracle on whole sampled partitions of a flat workload: first on
    one host thread for a quarter of the budget, then partitions in waves of
    one per thread on `threads` host threads for the rest (oracle calls
    release the interpreter lock). Aggregated GB/s of each."""
    from concurrent.futures import ThreadPoolExecutor

    w, P = pipe.w, pipe.P
    order = sorted(samples)
    with ThreadPoolExecutor(threads) as ex:         # untimed: first touch of the host buffers
        list(ex.map(lambda p: oracle_partition(pipe, p, samples[p]), order[:threads]))
    oracle_partition(pipe, order[0], samples[order[0]])    # untimed, on this thread
    t1 = e1 = 0.0
    used1 = 0
    while t1 < budget_s / 4:
        p = order[used1 % len(order)]
        t0 = time.perf_counter()
        e1 += oracle_partition(pipe, p, samples[p])
        t1 += time.perf_counter() - t0
        used1 += 1
    eN = 0
    waves = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        k = 0
        while True:
            ps = [order[(k + j) % len(order)] for j in range(threads)]
            k += threads
            eN += sum(ex.map(lambda p: oracle_partition(pipe, p, samples[p]), ps))
            waves += 1
            if time.perf_counter() - t0 >= budget_s * 3 / 4:
                break
    tN = time.perf_counter() - t0
    one = P * e1 * w.elem_bytes / t1 / 1e9
    many = P * eN * w.elem_bytes / tN / 1e9
    return {"value": round(many, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single_thread_value": round(one, 4),
            "sample": f"{len(order)} of {pipe.n_partitions()} partitions sampled evenly; every stage "
                      f"of the step per partition, after one untimed wave; {threads} host threads, one partition each, "
                      f"{waves} waves ({waves * threads} partitions x {P} workers) in {tN:.1f} s; "
                      f"one thread: {used1} partitions in {t1:.1f} s"}


def cpu_baseline_fused(pipe, host, threads: int):
    """The oracle on the whole step of a fused workload (Tensor Fusion):
    every worker's tensors packed into its fusion buffers, each buffer
    ring-averaged, the buffers unpacked; on one host thread, then on
    `threads` threads (one worker per thread for pack and unpack, one buffer
    per thread for the ring). Aggregated GB/s of each."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    w, P = pipe.w, pipe.P
    buf_of, off_of, fill = pipe.buf_of, pipe.off_of, pipe.fill
    ndt = np.float32 if w.dtype == 0 else np.uint16

    def pack(i):
        return oracle.fuse_pack(host[i], buf_of, off_of, fill, ndt)

    def ring(fused, k):
        oracle.ring_fold([fused[i][k] for i in range(P)], op=oracle.AVG, part=w.ring_part_elems)

    def unpack(fused, i):
        return oracle.fuse_unpack(fused[i], buf_of, off_of, w.sizes)

    def threaded():
        with ThreadPoolExecutor(threads) as ex:
            fused = list(ex.map(pack, range(P)))
            list(ex.map(lambda k: ring(fused, k), range(len(fill))))
            list(ex.map(lambda i: unpack(fused, i), range(P)))

    threaded()                      # untimed: first touch of the host buffers
    t0 = time.perf_counter()
    fused = [pack(i) for i in range(P)]
    for k in range(len(fill)):
        ring(fused, k)
    [unpack(fused, i) for i in range(P)]
    t1 = time.perf_counter() - t0
    del fused
    t0 = time.perf_counter()
    threaded()
    tN = time.perf_counter() - t0
    nbytes = P * pipe.N * w.elem_bytes
    return {"value": round(nbytes / tN / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single_thread_value": round(nbytes / t1 / 1e9, 4),
            "sample": f"the whole step ({P} workers x {len(w.sizes)} tensors, {len(fill)} fusion "
                      f"buffers): pack, ring average, unpack, after one untimed pass; {threads} host threads (pack and unpack "
                      f"one worker per thread, the ring one buffer per thread) in {tN:.2f} s; one "
                      f"thread {t1:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="shard", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-fusion", action="store_true",
                    help="fused workloads: pack -> ring -> unpack instead of the zero-copy ring")
    ap.add_argument("--ring-mode", default="fused", choices=["fused", "dual", "staged"],
                    help="single ring, the bidirectional dual ring fold order, or the single "
                         "ring's schedule one launch per step with binary32 partials staged "
                         "(flat workloads; implies --separate-step)")
    ap.add_argument("--separate-tail", action="store_true",
                    help="THC passes: integer sum, dequant and NMSE as three calls, not one")
    ap.add_argument("--separate-step", action="store_true",
                    help="flat workloads: quantizer, ring and tail as separate calls instead of the "
                         "one-read thc_ring_step")
    ap.add_argument("--graph", action="store_true",
                    help="time the K steps again as replays of one step captured in a HIP graph and "
                         "report those (the stage breakdown and roofline stay the eager steps')")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one 1 GiB torch copy first (PMC calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this build measures one GPU only (P simulated workers in one HBM); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import gradient_all_reduce_worker_amd as ga
    from gradient_all_reduce_worker_amd.pipeline import RING_STAGED, Pipeline, StageTimer

    ga.load()                       # fails loudly without the HIP library
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    pipe = Pipeline(args.workload, zero_copy=not args.copy_fusion, fused_tail=not args.separate_tail,
                    ring_mode={"dual": ga.RING_DUAL, "staged": RING_STAGED}.get(args.ring_mode,
                                                                              ga.RING_FUSED),
                    fused_step=not args.separate_step)
    t0 = time.perf_counter()
    pipe.setup()
    log(f"setup {args.workload}: {time.perf_counter() - t0:.1f} s")

    # host copies for the oracle baseline, taken before the first step
    # overwrites the gradients with their average
    samples = host = None
    threads = host_threads()
    if not args.no_cpu and not pipe.w.fused:
        n_part = pipe.n_partitions()
        want = min(n_part, 4 * threads)
        which = sorted({int(i * n_part / want) for i in range(want)})
        samples = pipe.sample_inputs(which)
    elif not args.no_cpu:
        from gradient_all_reduce_worker_amd import synth
        host = [[synth.to_numpy_bits(t) for t in pipe.tensors[i]] for i in range(pipe.P)]

    if args.copy_probe:
        # a plain device copy of known size (1 GiB read, 1 GiB written), for
        # scaling the PMC byte counters of the kernels against it
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the first pass sees the pristine gradients: its NMSE is the one reported
    # (later passes run the same kernels over the averaged buffers)
    pipe.step()
    torch.cuda.synchronize()
    nmse = {b: pipe.nmse[b].cpu().numpy().tolist() for b in pipe.nmse}
    for _ in range(max(args.warmup - 1, 0)):
        pipe.step()
    torch.cuda.synchronize()

    timer = StageTimer()
    # no garbage collection inside the timed loops: the host runs only a
    # little ahead of the GPU, and a collection of the stage timer's events
    # (vgg16: 34 per step) let the GPU idle 1.5-2 ms in one stage of a run
    # (vgg16 steps 53.1-54.9 ms with it, 52.1-52.8 ms without)
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pipe.step(timer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = timer.mean_ms()
    calls = timer.count()
    log(f"timed {args.steps} steps: {elapsed:.3f} s")
    eager_ms = elapsed / args.steps * 1e3
    if args.graph:
        graph = pipe.capture(warmup=max(args.warmup, 1))
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        log(f"timed {args.steps} graph replays: {elapsed:.3f} s")
    gc.enable()

    P, N, s = pipe.P, pipe.N, pipe.w.elem_bytes
    ms_step = elapsed / args.steps * 1e3
    value = P * N * s / (elapsed / args.steps) / 1e9
    nbytes = pipe.stage_bytes()
    stages = {}
    for k, ms in stage_ms.items():
        gbs = nbytes[k] / (ms * 1e-3) / 1e9
        stages[k] = {"ms": round(ms, 4), "calls_per_step": calls[k] // args.steps,
                     "alg_bytes": nbytes[k], "GB/s": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    quant = {k: round(P * N / (v * 1e-3) / 1e9, 2) for k, v in stage_ms.items()
             if k.startswith(("thc_usq_quantize", "thc_nuhc_quantize"))}

    step_keys = [k for k in stage_ms if k.startswith("thc_ring_step")]
    if step_keys:
        # bf16 buffers hold whole groups per thread, binary32 ones lane pairs
        ring_key = step_keys[0]
        kernel = "thc_ring_lane_kernel" if pipe.w.dtype == ga.F32 else "thc_ring_kernel"
    elif "ring_allreduce" in stage_ms:
        ring_key, kernel = "ring_allreduce", "ring_fused_vec_kernel"
    elif "ring_staged" in stage_ms:
        ring_key, kernel = "ring_staged", "ring_staged_vec_kernel"
    else:
        ring_key, kernel = "fusion_ring", "fusion_ring_kernel"
    ring_ms = stage_ms[ring_key]
    achieved = nbytes[ring_key] / (ring_ms * 1e-3) / 1e9
    # a call of the one-read pass is several equal launches (pieces of 2^26
    # elements), the staged schedule 2 (P - 1): the rate is over the whole
    # call (gaps between launches included), bytes per launch its mean
    launches = (ga.thc_ring_step_launches(N) if ring_key.startswith("thc_ring_step") else
                2 * (P - 1) if ring_key == "ring_staged" else 1)
    per_launch = nbytes[ring_key] / launches
    # the copy path runs one ring launch per fusion buffer: its summary would
    # be per buffer, so only single-launch rings carry traffic
    one_launch = calls[ring_key] // args.steps == 1
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(args.workload, kernel) if one_launch else None,
                "kernel": kernel, "alg_bytes_per_launch": per_launch, "launches_per_call": launches,
                # not in counter runs: their byte scale is the 1 GiB copy above,
                # the largest runtime copy of the run
                "runtime_copy": None if args.copy_probe else runtime_copy_rate()}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # the arithmetic of the path: binary32 folds, grid positions and
        # dequantization on every workload (bf16 gradients are widened
        # exactly; config.elem names the storage type)
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}", "P": P, "N": N,
                   "elem": "bf16" if pipe.w.dtype == ga.BF16 else "fp32",
                   "partition_elems": pipe.w.part_elems, "thc_bits": list(pipe.w.thc_bits),
                   "ring": args.ring_mode,
                   "thc_tail": "separate" if args.separate_tail else "fused",
                   "thc_ring_step": "fused" if pipe.fused_step else "separate",
                   "fusion": (None if not pipe.w.fused else
                              "pack-ring-unpack" if args.copy_fusion else "zero-copy"),
                   "launch": "graph" if args.graph else "eager",
                   "parallelism": "1 GPU, P simulated workers"},
        "roofline": roofline,
        "thc_quantize_gelem_s": quant,
        "nmse": {(f"b{b}" if isinstance(b, int) else b): v[2] for b, v in nmse.items()},
        "stages": stages,
    }
    if args.graph:
        out["eager_ms_per_step"] = round(eager_ms, 4)
    if samples is not None:
        out["cpu_baseline"] = cpu_baseline_flat(pipe, samples, args.cpu_seconds, threads)
    elif host is not None:
        out["cpu_baseline"] = cpu_baseline_fused(pipe, host, threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
