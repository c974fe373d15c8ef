"""Seeded synthetic gradients shaped like the pages' workloads.

This module holds only input generation: layer shapes, value distributions
and seeding. It contains none of the aggregation arithmetic, and it is the
only code that both the HIP path's callers and the oracle's callers share.

Workloads (values are synthetic; no dataset, model or weights are used):

* ``small``  - 4 workers x 1,048,576 fp32 (one 4 MiB partition), N(0, 0.01^2);
  the shape of THC's 4 MB-partition, four-worker microbenchmark
  (THC page, section 2, Figure 2(b)).
* ``fusion`` - 8 workers x 200 fp32 tensors, sizes log-uniform in
  [1024, 262144] elements, N(0, 0.01^2); packed into 64 MiB fusion buffers
  (Horovod page, section 3.4, Tensor Fusion).
* ``resnet101`` - 16 workers x the 314 trainable tensors of ResNet-101
  (44,549,160 fp32), per-tensor scale 1e-3 * U(0.1, 10), Student-t(3) values.
* ``vgg16`` - 32 workers x the 32 trainable tensors of VGG-16
  (138,357,544 fp32, one contiguous vector per worker), per-tensor sigma
  log-uniform in [1e-4, 1e-1], normal values; THC with b = 4 and b = 8 on
  2^20-element partitions, plus non-uniform THC with b = 4 and granularity
  36 (the THC page's scalability setting); the exact average (for the NMSE)
  comes from the ring over the same partitions.
* ``shard`` - 8 workers x 2,147,483,648 bf16, Laplace(0, 1e-3); ring average
  with fp32 accumulation in 2^20-element partitions, THC with b = 2.

Seeding: every random draw comes from a torch.Generator seeded from
``numpy.random.SeedSequence([data_seed, stream, worker, block])``; data_seed
is 1000 + the workload's index, the quantizer seed 2000 + the index.
Values are drawn on the device that will hold them (torch's generators on
CPU and GPU give different streams; each test or bench run feeds the same
drawn values to both the kernels and the oracle).
"""
from dataclasses import dataclass, field
import math
from typing import List, Optional, Tuple

import numpy as np
import torch

F32, BF16 = 0, 1


# ------------------------------------------------------------------ shapes
def resnet101_shapes() -> List[Tuple[str, Tuple[int, ...]]]:
    """Trainable tensors of ResNet-101 in forward order (convs without bias,
    batch-norm weight and bias, fully connected layer with bias)."""
    shapes = [("conv1.w", (64, 3, 7, 7)), ("bn1.w", (64,)), ("bn1.b", (64,))]
    inplanes = 64
    for stage, (planes, blocks) in enumerate(zip((64, 128, 256, 512), (3, 4, 23, 3))):
        for blk in range(blocks):
            pre = f"layer{stage + 1}.{blk}"
            shapes += [
                (pre + ".conv1.w", (planes, inplanes, 1, 1)),
                (pre + ".bn1.w", (planes,)), (pre + ".bn1.b", (planes,)),
                (pre + ".conv2.w", (planes, planes, 3, 3)),
                (pre + ".bn2.w", (planes,)), (pre + ".bn2.b", (planes,)),
                (pre + ".conv3.w", (planes * 4, planes, 1, 1)),
                (pre + ".bn3.w", (planes * 4,)), (pre + ".bn3.b", (planes * 4,)),
            ]
            if blk == 0:
                shapes += [
                    (pre + ".down.w", (planes * 4, inplanes, 1, 1)),
                    (pre + ".down_bn.w", (planes * 4,)), (pre + ".down_bn.b", (planes * 4,)),
                ]
            inplanes = planes * 4
    shapes += [("fc.w", (1000, 2048)), ("fc.b", (1000,))]
    return shapes


def vgg16_shapes() -> List[Tuple[str, Tuple[int, ...]]]:
    """Trainable tensors of VGG-16 in forward order (3x3 convs with bias,
    fc6 4096x25088, fc7 4096x4096, fc8 1000x4096, all with bias)."""
    chans = [64, 64, 128, 128, 256, 256, 256, 512, 512, 512, 512, 512, 512]
    shapes, cin = [], 3
    for i, c in enumerate(chans):
        shapes += [(f"conv{i + 1}.w", (c, cin, 3, 3)), (f"conv{i + 1}.b", (c,))]
        cin = c
    shapes += [("fc6.w", (4096, 25088)), ("fc6.b", (4096,)),
               ("fc7.w", (4096, 4096)), ("fc7.b", (4096,)),
               ("fc8.w", (1000, 4096)), ("fc8.b", (1000,))]
    return shapes


def numel(shape) -> int:
    return int(np.prod(shape, dtype=np.int64)) if len(shape) else 1


# ------------------------------------------------------------------ seeding
def seed_of(*words: int) -> int:
    ss = np.random.SeedSequence([int(w) for w in words])
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


def generator(device, *words: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed_of(*words))
    return g


def host_rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


# ------------------------------------------------------------------ workloads
@dataclass
class Workload:
    name: str
    index: int
    P: int
    dtype: int                      # F32 or BF16
    sizes: List[int]                # per-tensor element counts, ready (reverse) order
    names: List[str] = field(default_factory=list)
    dist: str = "normal"
    fusion_cap_bytes: int = 64 << 20
    part_elems: int = 0             # 0: one partition per fused buffer / vector
    ring_part_elems: int = 0
    thc_bits: Tuple[int, ...] = ()
    global_bits: Tuple[int, ...] = ()   # uniform THC passes with one grid for the whole vector
    nuhc: Tuple[Tuple[int, int], ...] = ()   # (b, g) of non-uniform THC passes
    # (b, g, log2 d) of THC passes behind the randomized Hadamard transform;
    # a fraction rht_p of the transformed coordinates is expected to be cut
    rht: Tuple[Tuple[int, int, int], ...] = ()
    rht_p: float = 1.0 / 32
    ef_bits: Tuple[int, ...] = ()   # uniform THC passes with error feedback
    stragglers: int = 0             # workers the server does not wait for (partial pass)
    fused: bool = True              # run the Tensor Fusion plan over `sizes`

    @property
    def N(self) -> int:
        return int(sum(self.sizes))

    @property
    def data_seed(self) -> int:
        return 1000 + self.index

    @property
    def quant_seed(self) -> int:
        return 2000 + self.index

    @property
    def rht_seed(self) -> int:
        return 3000 + self.index

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2


def _rev(shapes):
    """Gradients become ready from the last layer backwards."""
    shapes = list(reversed(shapes))
    return [n for n, _ in shapes], [numel(s) for _, s in shapes]


def workload(name: str) -> Workload:
    if name == "small":
        return Workload("small", 0, P=4, dtype=F32, sizes=[1 << 20], names=["grad"],
                        dist="normal", part_elems=1 << 20, ring_part_elems=1 << 20, thc_bits=(4,),
                        fused=False)
    if name == "fusion":
        rng = host_rng(1001, 0xF5)
        sizes = [int(round(math.exp(v))) for v in
                 rng.uniform(math.log(1024), math.log(262144), size=200)]
        return Workload("fusion", 1, P=8, dtype=F32, sizes=sizes,
                        names=[f"t{i}" for i in range(200)], dist="normal")
    if name == "resnet101":
        names, sizes = _rev(resnet101_shapes())
        return Workload("resnet101", 2, P=16, dtype=F32, sizes=sizes, names=names,
                        dist="student_t3")
    if name == "vgg16":
        names, sizes = _rev(vgg16_shapes())
        return Workload("vgg16", 3, P=32, dtype=F32, sizes=sizes, names=names,
                        dist="normal_logsigma", part_elems=1 << 20, ring_part_elems=1 << 20,
                        thc_bits=(4, 8), global_bits=(4,), nuhc=((4, 36),), rht=((4, 36, 20),),
                        ef_bits=(4,),
                        stragglers=3, fused=False)
    if name == "shard":
        return Workload("shard", 4, P=8, dtype=BF16, sizes=[1 << 31], names=["shard"],
                        dist="laplace", part_elems=1 << 20, ring_part_elems=1 << 20,
                        thc_bits=(2,), fused=False)
    raise KeyError(name)


WORKLOADS = ("small", "fusion", "resnet101", "vgg16", "shard")


def straggler_set(w: Workload) -> List[int]:
    """The workers the server does not wait for in the partial pass: a
    seeded draw of w.stragglers distinct workers."""
    if w.stragglers <= 0:
        return []
    rng = host_rng(w.data_seed, 0x57A6)
    return sorted(int(i) for i in rng.choice(w.P, size=w.stragglers, replace=False))


def tensor_scales(w: Workload) -> np.ndarray:
    """Per-tensor scale shared by all workers (one draw per tensor)."""
    T = len(w.sizes)
    rng = host_rng(w.data_seed, 0xFFFF)
    if w.dist == "student_t3":
        return 1e-3 * rng.uniform(0.1, 10.0, size=T)
    if w.dist == "normal_logsigma":
        return np.exp(rng.uniform(math.log(1e-4), math.log(1e-1), size=T))
    if w.dist == "laplace":
        return np.full(T, 1e-3)
    return np.full(T, 0.01)


# ------------------------------------------------------------------ values
def _draw(dist: str, n: int, g: torch.Generator, device) -> torch.Tensor:
    """n unit-scale float32 values of the named distribution."""
    if dist in ("normal", "normal_logsigma"):
        return torch.randn(n, generator=g, device=device, dtype=torch.float32)
    if dist == "student_t3":
        z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        chi2 = torch.zeros(n, device=device, dtype=torch.float32)
        for _ in range(3):
            y = torch.randn(n, generator=g, device=device, dtype=torch.float32)
            chi2.addcmul_(y, y)
        t = z / torch.sqrt(chi2 / 3.0)
        return torch.nan_to_num(t, nan=0.0).clamp_(-1e6, 1e6)
    if dist == "laplace":
        e1 = torch.empty(n, device=device, dtype=torch.float32).exponential_(1.0, generator=g)
        e2 = torch.empty(n, device=device, dtype=torch.float32).exponential_(1.0, generator=g)
        return (e1 - e2).clamp_(-1e3, 1e3)
    raise KeyError(dist)


def worker_tensors(w: Workload, worker: int, device="cpu", sizes: Optional[List[int]] = None
                   ) -> List[torch.Tensor]:
    """One worker's gradient tensors (each its own allocation), ready order."""
    sizes = w.sizes if sizes is None else sizes
    scales = tensor_scales(w)
    dt = torch.float32 if w.dtype == F32 else torch.bfloat16
    out = []
    for t, n in enumerate(sizes):
        g = generator(device, w.data_seed, 1, worker, t)
        v = _draw(w.dist, n, g, device).mul_(float(scales[t % len(scales)]))
        out.append(v.to(dt))
    return out


def worker_flat(w: Workload, worker: int, out: torch.Tensor, slab: int = 1 << 27) -> None:
    """Fill `out` (1-D, w.N elements, fp32 or bf16) with one worker's whole
    gradient vector: its tensors concatenated in ready order. Drawn in slabs
    so the temporary stays small."""
    device = out.device
    scales = tensor_scales(w)
    pos = 0
    for t, n in enumerate(w.sizes):
        for s0 in range(0, n, slab):
            m = min(slab, n - s0)
            g = generator(device, w.data_seed, 2, worker, t, s0 // slab)
            v = _draw(w.dist, m, g, device).mul_(float(scales[t]))
            out[pos + s0: pos + s0 + m].copy_(v)
        pos += n


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor: float32 as float32, bf16 as uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)
