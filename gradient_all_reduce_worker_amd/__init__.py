"""MI355X (gfx950) gradient-aggregation hot path for P simulated
data-parallel workers held in one GPU's HBM: Tensor Fusion (pack/unpack or
zero-copy), ring all-reduce (sum | avg; single or bidirectional), and THC
stochastic quantization (uniform and table-based) with homomorphic integer
aggregation, behind an optional randomized Hadamard transform.

The computation lives in libga.so (HIP, built from csrc/ by build.py); the
functions below are its C ABI (include/ga.h) under the same names, with
torch tensors supplying device memory and the current stream. ``synth``
holds the seeded workload generators.
"""
from ._native import (  # noqa: F401
    AVG, BF16, EXPORTS, F32, LIB_PATH, MAX_WORKERS, RING_FUSED, RING_STEPWISE, SUM,
    CopyDesc, FusionTables, GAError, RingStats, build_copy_table, ga_fuse_desc_check,
    ga_fuse_pack, ga_fuse_plan, ga_fuse_unpack, ga_ring_allreduce_sim, load, n_partitions,
    packed_bytes, thc_dequant, thc_int_aggregate, thc_minmax, thc_nmse, thc_nmse_ws_bytes,
    thc_usq_quantize, upload_table, thc_nuhc_quantize, thc_nuhc_aggregate, thc_nuhc_dequant,
    center_table, RING_DUAL, FTENSOR_DTYPE, FusionRing, ga_fusion_ring_plan, rht_padded,
    thc_rht_sumsq, thc_rht_range, thc_rht_forward, thc_rht_inverse, thc_rht_quantize,
    thc_aggregate_dequant, thc_aggregate_dequant_ws_bytes, thc_rht_norm_quantize,
    thc_rht_norm_quantize_ws_bytes, ga_ring_stage_bytes, ga_ring_stepwise_staged,
    fusion_block_bytes, thc_nmse_noalloc, thc_ring_step, thc_ring_step_ws_bytes,
    thc_ring_step_launches, thc_ef_minmax, thc_ef_quantize, thc_minmax_combine,
    thc_ef_minmax_pair,
)
