/*
 * ga.h -- C ABI of libga.so, the MI355X (gfx950) gradient-aggregation hot
 * path: P simulated data-parallel workers whose gradient buffers all sit in
 * one GPU's HBM.
 *
 *   ga_fuse_plan / ga_fuse_pack / ga_fuse_unpack   Tensor Fusion
 *   ga_ring_allreduce_sim                          ring all-reduce (sum | avg;
 *                                                  single or bidirectional)
 *   ga_ring_stepwise_staged                        its schedule step by step,
 *                                                  partials on a binary32 wire
 *   ga_fusion_ring_plan / ga_fusion_ring_allreduce zero-copy fusion ring
 *   thc_minmax / thc_minmax_combine / thc_usq_quantize / thc_int_aggregate /
 *   thc_dequant / thc_nmse
 *   thc_nmse_noalloc (thc_nmse without a workspace, for callers that
 *   cannot allocate)
 *   thc_aggregate_dequant (aggregate + dequant + NMSE in one pass)
 *   thc_ring_step (quantize, ring average, sum, dequant, NMSE: one read)
 *                                                  THC uniform quantization
 *   thc_nuhc_quantize / thc_nuhc_aggregate / thc_nuhc_dequant
 *                                                  THC with lookup tables
 *   thc_ef_minmax / thc_ef_minmax_pair / thc_ef_quantize
 *                                                  error feedback
 *   thc_rht_sumsq / thc_rht_range / thc_rht_forward / thc_rht_inverse /
 *   thc_rht_quantize / thc_rht_norm_quantize
 *                                                  randomized Hadamard
 *                                                  transform, norm-based
 *                                                  range, truncation
 *
 * Pages cited:
 *   [HVD]  "Horovod: Fast and Easy Distributed Deep Learning in TensorFlow"
 *          (paper summary page), section 3.4 (ring-allreduce; Tensor Fusion).
 *   [RING] systemcraft lesson "Collective Communication: Ring All-Reduce",
 *          sections 4, 5 and 7 (schedule, volume, simulator).
 *   [THC]  "THC: Accelerating Distributed Deep Learning Using Tensor
 *          Homomorphic Compression", sections 2-4 (NMSE, uniform THC,
 *          Algorithm 1, aggregation by the server), 4 (Algorithm 2), 5
 *          (randomized Hadamard transform, truncation, norm-based range,
 *          error feedback) and 8 (aggregate width, stragglers).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller allocates and owns every buffer. The library keeps
 *   no state between calls and allocates no device memory.
 * Pointers: "device" pointers are HBM addresses (hipMalloc, or a torch
 *   tensor's data_ptr()); "host" pointers are ordinary process memory.
 *   Arrays of worker pointers (bufs, packed) are host arrays of device
 *   pointers, P <= GA_MAX_WORKERS entries, read during the call only.
 * Alignment: every device pointer must be aligned to its element size.
 *   Buffers whose bases are 16-byte aligned take the 128-bit vector path;
 *   others are handled by a slower per-element path with identical results.
 * Execution: every call that takes `stream` (a hipStream_t; NULL is the
 *   null stream) only enqueues work on it and returns. There is no implicit
 *   device synchronisation; calls on one stream run in order.
 * Errors: a negative status. On GA_EINVAL and GA_ENOTSUP nothing has been
 *   enqueued. GA_EHIP reports a failed launch (hipGetLastError after the
 *   launch). ga_last_error() returns a thread-local message for the last
 *   failure on the calling thread. No C++ exception crosses the ABI.
 * Empty input: N == 0 (or n_desc == 0) is a successful no-op.
 * Values: floating-point inputs must be finite.
 */
#ifndef GA_H
#define GA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int ga_status;
#define GA_OK 0
#define GA_EINVAL (-1)   /* bad argument; nothing enqueued */
#define GA_ENOTSUP (-2)  /* valid but unsupported combination; nothing enqueued */
#define GA_EHIP (-3)     /* the HIP runtime reported an error */

#define GA_MAX_WORKERS 64

typedef enum { GA_F32 = 0, GA_BF16 = 1 } ga_dtype;
typedef enum { GA_SUM = 0, GA_AVG = 1 } ga_op;
typedef enum { GA_RING_FUSED = 0, GA_RING_STEPWISE = 1, GA_RING_DUAL = 2 } ga_ring_mode;

/* ------------------------------------------------------------------ */
/* Tensor Fusion  ([HVD] 3.4, Tensor Fusion steps 1-6)                  */
/* ------------------------------------------------------------------ */

/*
 * ga_fuse_plan -- host only, synchronous.
 * Walks T tensors in the caller's (ready) order and assigns each to a
 * fusion buffer of cap_bytes bytes: a tensor joins the open buffer while it
 * fits in the remaining space and has the buffer's data type (step 1); the
 * buffer is closed at the first tensor that does not, and that tensor opens
 * the next one; an exact fit counts as a fit; a tensor larger than cap_bytes
 * is reduced alone in a buffer of its own. Tensors are placed densely,
 * without padding (step 3: "concatenated into a contiguous memory region").
 *   n_elems[T]   element count of each tensor (>= 0)
 *   dtype_of[T]  ga_dtype of each tensor, or NULL for all GA_F32
 *   cap_bytes    fusion buffer capacity in bytes (> 0; [HVD] default 64 MB)
 * Outputs (host arrays the caller sizes): buf_of[T] buffer id of each
 * tensor; off_of[T] element offset inside that buffer; fill[T] (at most T
 * buffers) element count of each buffer; buf_dtype[T] (nullable) the data
 * type of each buffer; *n_buf the number of buffers.
 */
ga_status ga_fuse_plan(const int64_t* n_elems, const int32_t* dtype_of, int32_t T,
                       int64_t cap_bytes, int32_t* buf_of, int64_t* off_of, int64_t* fill,
                       int32_t* buf_dtype, int32_t* n_buf);

/*
 * One contiguous copy of n elements from src to dst. `start` is the
 * exclusive prefix sum of n over the descriptor table (start[0] = 0,
 * start[k+1] = start[k] + n[k]); the kernel uses it to find the copy that
 * each workgroup's slice of the concatenated index space belongs to.
 */
typedef struct {
    const void* src;   /* device */
    void* dst;         /* device */
    int64_t n;         /* elements */
    int64_t start;     /* elements before this copy in the table */
} ga_copy_desc;

/*
 * ga_fuse_desc_check -- host only. Validates a host copy of a descriptor
 * table (non-null pointers aligned to the element size, n >= 0, consistent
 * start values) and returns the total element count in *total_elems.
 */
ga_status ga_fuse_desc_check(const ga_copy_desc* h_desc, int64_t n_desc, ga_dtype dt,
                             int64_t* total_elems);

/*
 * ga_fuse_pack / ga_fuse_unpack -- one launch performs every copy of the
 * table: pack (step 3) copies each worker's tensors into its fusion buffers,
 * unpack (step 5) copies the reduced buffers back into the tensors. The two
 * differ only in which side of each descriptor is the fusion buffer.
 *   d_desc       device copy of the table (caller uploads it once and may
 *                reuse it across calls); must equal a table that
 *                ga_fuse_desc_check accepts
 *   n_desc       number of descriptors
 *   total_elems  sum of n over the table
 *   dt           element type (GA_F32: 4 bytes, GA_BF16: 2 bytes)
 * Sources and destinations of different descriptors must not overlap.
 * Each copy only touches [src, src + n) and [dst, dst + n).
 */
ga_status ga_fuse_pack(const ga_copy_desc* d_desc, int64_t n_desc, int64_t total_elems,
                       ga_dtype dt, void* stream);
ga_status ga_fuse_unpack(const ga_copy_desc* d_desc, int64_t n_desc, int64_t total_elems,
                         ga_dtype dt, void* stream);

/* ------------------------------------------------------------------ */
/* Ring all-reduce over P simulated workers  ([HVD] 3.4; [RING] 4, 5, 7, 11) */
/* ------------------------------------------------------------------ */

typedef struct {
    int64_t steps;                 /* 2 (P - 1) communication steps per ring */
    int64_t bytes_sent_per_worker; /* sum over partitions of 2 (P-1) C elem_bytes;
                                      dual ring: 2 (P-1) 2 C2 elem_bytes */
    int64_t hbm_bytes;             /* algorithmic HBM bytes of the chosen mode */
    int64_t launches;              /* kernel launches enqueued */
} ga_ring_stats;

/*
 * ga_ring_allreduce_sim -- in place: every one of the P buffers ends holding
 * the element-wise sum (op = GA_SUM) or average (GA_AVG) of all P, exactly
 * as the ring schedule computes it.
 *
 * Each partition [p0, p0 + n) (part_elems elements; 0 means the whole
 * buffer) is cut into P chunks of C = ceil(n / P) elements (trailing chunks
 * shorter or empty). Scatter-reduce runs P - 1 steps: at step s worker i
 * sends chunk (i - s) mod P to worker i + 1, which adds it into its own copy;
 * after it worker j holds the finished sum of chunk (j + 1) mod P. All-gather
 * runs P - 1 steps in which the finished chunk overwrites the other copies.
 * So the sum of chunk c is folded in the order c, c+1, ..., c+P-1 (mod P),
 * in binary32 with round-to-nearest-even and no fused multiply-add; bf16
 * inputs are widened exactly and the partial sums stay binary32 on every
 * hop, with one round-to-nearest-even to bf16 at the end. GA_AVG divides
 * the finished sum by P once (binary32 division).
 *   bufs        host array of P device pointers, each N elements of dt
 *   P           1..GA_MAX_WORKERS
 *   mode        GA_RING_FUSED: one pass that reads every buffer once and
 *               writes every buffer once (2 P N elem_bytes of HBM traffic),
 *               folding each element in the schedule's order.
 *               GA_RING_STEPWISE: one launch per communication step,
 *               2 (P - 1) launches moving the chunks as the schedule does
 *               (5 (P - 1) N elem_bytes); GA_F32 only (bf16 partials need
 *               binary32 storage on the wire) -> GA_ENOTSUP for GA_BF16;
 *               ga_ring_stepwise_staged runs the schedule for either type.
 *               GA_RING_DUAL: the bidirectional ring of [RING] section 11
 *               (Exercise 1), executed like GA_RING_FUSED: each partition
 *               is cut into 2P sub-chunks of C2 = ceil(n / 2P); sub-chunk c
 *               < P goes round clockwise (folded c, c+1, ..., c-1), sub-chunk
 *               P + c counter-clockwise (folded c, c-1, ..., c+1). Same
 *               rounding rules and traffic as GA_RING_FUSED; a different
 *               fold order, so results differ from it in the last bits.
 *   st          optional (nullable) host struct receiving the accounting.
 * GA_RING_FUSED and GA_RING_STEPWISE give bit-identical results.
 */
ga_status ga_ring_allreduce_sim(void* const* bufs, int32_t P, int64_t N, ga_dtype dt, ga_op op,
                                int64_t part_elems, ga_ring_mode mode, ga_ring_stats* st,
                                void* stream);

/*
 * ga_ring_stepwise_staged -- the same schedule one communication step per
 * launch ([RING] sections 4 and 7; [HVD] 3.4), with the partial sums on a
 * binary32 wire: at scatter-reduce step s every element of chunk c has
 * exactly one partial in flight, from worker (c + s) mod P to (c + s + 1)
 * mod P, so one binary32 array of N elements (the stage) holds them all.
 * Step 0 adds the receiver's value to the sender's own, the middle steps
 * add it to the staged partial, the last step (s = P - 2) divides by P
 * (op = GA_AVG) and stores the finished value, rounded once to dt, into the
 * owner's buffer; the P - 1 all-gather steps copy the finished chunk on in
 * dt. Results are bit-identical to ga_ring_allreduce_sim (GA_RING_FUSED),
 * for GA_F32 and GA_BF16: the same fold order and roundings.
 *   bufs, P, N, dt, op, part_elems   as ga_ring_allreduce_sim
 *   d_stage      device, at least ga_ring_stage_bytes(P, N) bytes (4 N when
 *                P > 2, else none: may be null), 16-byte aligned, disjoint
 *                from every buffer; caller-owned, contents on return
 *                unspecified
 *   st           optional accounting: bytes_sent_per_worker counts the
 *                scatter-reduce partials as binary32 and the all-gather
 *                chunks in dt; hbm_bytes the steps' reads and writes
 * Errors (nothing enqueued): GA_EINVAL for a bad dtype, op, size, P,
 * pointer, overlap or a stage that is too small.
 */
size_t ga_ring_stage_bytes(int32_t P, int64_t N);
ga_status ga_ring_stepwise_staged(void* const* bufs, int32_t P, int64_t N, ga_dtype dt, ga_op op,
                                  int64_t part_elems, float* d_stage, size_t stage_bytes,
                                  ga_ring_stats* st, void* stream);

/* ------------------------------------------------------------------ */
/* Zero-copy Tensor Fusion ring  ([HVD] 3.4: Tensor Fusion + ring)      */
/* ------------------------------------------------------------------ */

/*
 * One tensor of a fusion plan: elements [start, start + n) of fusion buffer
 * `buf` (ga_fuse_plan's buffer ids and offsets). A table lists the tensors
 * of one or more buffers, buffer by buffer in increasing id, each buffer's
 * tensors in offset order.
 */
typedef struct {
    int64_t start;    /* offset in its fusion buffer, elements */
    int64_t n;        /* elements */
    int32_t buf;      /* fusion buffer id */
    int32_t reserved; /* 0 */
} ga_fusion_tensor;

/* Work vectors (or elements) per block of the zero-copy fusion ring; one
 * workgroup folds one block. */
#define GA_FUSION_BLOCK 256
/* Bytes of one planned block for P workers: a 16-byte header and P device
 * pointers (the layout is internal to the library). */
#define GA_FUSION_BLOCK_BYTES(P) (16 + 8 * (size_t)(P))

/*
 * ga_fusion_ring_plan -- host only: the work of the zero-copy fusion ring
 * over the buffers a table lists, for ring geometry (part_elems, mode).
 *   h_tensors   n_tensors rows; each row's buf in [0, n_buf), never
 *               decreasing down the table; the rows of a buffer dense in
 *               buffer order (the first starts at 0, start[t + 1] = start[t]
 *               + n[t]) and ending at fill[buf]; a buffer listed in no row
 *               must have fill 0
 *   h_ptrs      n_tensors x P device pointers, tensor-major (h_ptrs[t P + i]
 *               is worker i's copy of tensor t), each non-null and aligned
 *               to the element size; no two of the P n_tensors regions may
 *               overlap
 *   fill        host array of n_buf buffer lengths, elements
 *   part_elems  partition length inside every buffer (0: one partition per
 *               buffer); mode GA_RING_FUSED or GA_RING_DUAL (the chunks and
 *               fold directions of ga_ring_allreduce_sim)
 *   h_work      host array of cap_blocks blocks of GA_FUSION_BLOCK_BYTES(P)
 *               bytes, or null to count only; *n_blocks receives the count
 * Every tensor is cut at its buffer's partition and chunk boundaries; each
 * piece becomes blocks of up to GA_FUSION_BLOCK whole 16-byte vectors (when
 * all P copies are 16-byte aligned) plus blocks of up to GA_FUSION_BLOCK
 * elements for its unaligned ends, each block carrying its fold's first
 * worker and direction and the P copies' addresses of its first vector or
 * element. Enqueues nothing; GA_EINVAL if cap_blocks is too small.
 */
ga_status ga_fusion_ring_plan(const ga_fusion_tensor* h_tensors, void* const* h_ptrs,
                              int64_t n_tensors, int32_t P, ga_dtype dt, const int64_t* fill,
                              int32_t n_buf, int64_t part_elems, ga_ring_mode mode, void* h_work,
                              int64_t cap_blocks, int64_t* n_blocks);

/*
 * ga_fusion_ring_allreduce -- in place in every worker's tensors, for every
 * buffer of the plan, in ONE launch: exactly what ga_fuse_pack,
 * ga_ring_allreduce_sim over each fusion buffer (the plan's part_elems and
 * mode, this op) and ga_fuse_unpack leave in them, bit for bit, without
 * the fusion buffers: each element is folded at its tensor's address in
 * the order its offset in its buffer gives. HBM traffic 2 P (sum of fills)
 * elem_bytes instead of 6 P (sum of fills) elem_bytes.
 *   d_work, n_blocks   device copy of ga_fusion_ring_plan's blocks
 *   P, dt              as planned
 *   fill, n_buf, part_elems, mode
 *                      as planned (the accounting and the launch shape);
 *                      GA_RING_STEPWISE -> GA_ENOTSUP
 *   st                 optional accounting summed over the buffers (steps:
 *                      2 (P - 1) per ring; launches: 1)
 * The device blocks are trusted (ga_fusion_ring_plan made them from checked
 * tables); blocks that do not come from it for these P and dt are undefined.
 */
ga_status ga_fusion_ring_allreduce(const void* d_work, int64_t n_blocks, int32_t P, ga_dtype dt,
                                   ga_op op, const int64_t* fill, int32_t n_buf, int64_t part_elems,
                                   ga_ring_mode mode, ga_ring_stats* st, void* stream);

/* ------------------------------------------------------------------ */
/* THC uniform stochastic quantization  ([THC] 2-4, Algorithm 1)        */
/* ------------------------------------------------------------------ */

/*
 * thc_minmax -- Algorithm 1's preliminary round: per partition p of
 * part_elems elements (0: one partition), m = the smallest and M = the
 * largest element over all P workers' elements of that partition, written
 * as d_mM[2p] = m, d_mM[2p + 1] = M (binary32; a negative zero is returned
 * as +0). d_mM is a device array of 2 * ceil(N / part_elems) floats.
 */
ga_status thc_minmax(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                     int64_t part_elems, float* d_mM, void* stream);

/*
 * thc_minmax_combine -- the extremes of n_part partition grids (thc_minmax's
 * output): d_mM[0] = the smallest m, d_mM[1] = the largest M (+0 for a
 * negative zero). Algorithm 1's preliminary round takes local extremes and
 * then global ones ([THC] section 3); min and max are exact, so this equals
 * thc_minmax over the same elements with one partition, bit for bit, without
 * reading them again.
 *   d_parts   device, 2 n_part floats (8-byte aligned)
 *   d_mM      device, 2 floats (8-byte aligned), disjoint from d_parts
 * n_part = 0: nothing is done. Errors (nothing enqueued): GA_EINVAL for a
 * negative n_part, a null, misaligned or overlapping pointer.
 */
ga_status thc_minmax_combine(const float* d_parts, int64_t n_part, float* d_mM, void* stream);

/*
 * thc_usq_quantize -- every worker quantizes its vector on the shared grid
 * q_k = m + k (M - m) / (2^b - 1), k = 0 .. 2^b - 1, of its partition, by
 * stochastic rounding to one of the two neighbouring grid points (unbiased,
 * [THC] section 3), and emits the b-bit indices packed least significant
 * bits first: element e occupies bits [(e b) mod 8, +b) of byte e b / 8.
 * Arithmetic (binary32, L = 2^b - 1): range = M - m; s = L / range;
 * u = (a - m) s; z0 = min(floor(u), L - 1); f = u - z0; up = (2 r + 1) <
 * f 2^17 with r the element's 16-bit uniform; z = z0 + up; range == 0 gives
 * z = 0. The uniform of element e of worker w is half (e mod 2) of word
 * (e mod 8) / 2 of Philox4x32-10 (Salmon et al., SC'11) on counter
 * (g mod 2^32, g >> 32, w, 0), g = e / 8, key (seed mod 2^32, seed >> 32).
 *   bufs[P]     device vectors of N elements (dt); worker id of bufs[i] is
 *               worker0 + i
 *   d_mM        device grid ends from thc_minmax (same part_elems)
 *   b           1, 2, 4 or 8
 *   packed[P]   host array of device pointers, ceil(N b / 8) bytes each;
 *               bits past element N - 1 in the last byte are written 0
 * Values are expected inside their partition's [m, M] (d_mM from
 * thc_minmax over the same data). Any other value, NaN included, still
 * gives an index in [0, 2^b - 1]: below m it is 0, above M it is 2^b - 1.
 */
ga_status thc_usq_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                           ga_dtype dt, int64_t part_elems, const float* d_mM, int32_t b,
                           uint64_t seed, uint8_t* const* packed, void* stream);

/*
 * thc_int_aggregate -- the server side of Algorithm 1: d_sum[e] = sum over
 * the P workers of their b-bit index of element e, in int32 (exact; at most
 * P (2^b - 1) <= 16320). packed as written by thc_usq_quantize; d_sum is a
 * device array of N int32.
 */
ga_status thc_int_aggregate(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                            int32_t* d_sum, void* stream);

/*
 * thc_dequant -- Algorithm 1's last step: divide the index sum by the
 * number of workers P and map it back onto the grid:
 * delta = range / L; out[e] = m + ((float)S[e] / (float)P) delta (binary32,
 * no fused multiply-add); range == 0 gives m. out_dt GA_BF16 rounds the
 * final value to nearest-even. d_sum: N int32; out: N elements of out_dt.
 */
ga_status thc_dequant(const int32_t* d_sum, int64_t N, int32_t P, int32_t b, int64_t part_elems,
                      const float* d_mM, void* out, ga_dtype out_dt, void* stream);

/*
 * thc_nmse -- [THC] section 2, Figure 2(b): NMSE(x, xhat) =
 * ||x - xhat||^2 / ||x||^2 with binary64 accumulation. Writes
 * d_out[0] = numerator, d_out[1] = denominator, d_out[2] = their ratio
 * (0 if both are 0, +inf if only the denominator is). d_ws is a device
 * workspace of at least thc_nmse_ws_bytes(N) bytes.
 */
ga_status thc_nmse(const void* x, const void* xhat, int64_t N, ga_dtype dt, double* d_out,
                   void* d_ws, size_t ws_bytes, void* stream);
size_t thc_nmse_ws_bytes(int64_t N);

/*
 * thc_nmse_noalloc -- thc_nmse for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): same kernels, same result, bit for bit, but the
 * partials live in a 160 KiB array inside the library, one copy per GPU
 * (held until the process ends), instead of a caller workspace. The call
 * allocates nothing. Every N that thc_nmse_ws_bytes(N) maps to at most
 * 160 KiB is accepted (the piece count is capped near 8,192, so that is
 * every N in practice); a larger need returns GA_EINVAL. The first call on
 * a GPU looks up that GPU's copy (the stream's device). Calls that overlap
 * on one GPU share the array and race: order them on one stream.
 */
ga_status thc_nmse_noalloc(const void* x, const void* xhat, int64_t N, ga_dtype dt, double* d_out,
                           void* stream);

/*
 * thc_ring_step -- one pass over the P workers' buffers that leaves exactly
 * what these calls leave in turn, reading every gradient once:
 *   thc_usq_quantize(bufs, P, worker0, N, dt, q_part, d_mM, b, seed, packed)
 *   ga_ring_allreduce_sim(bufs, P, N, dt, GA_AVG, ring_part, GA_RING_FUSED)
 *   thc_aggregate_dequant(packed, P, N, b, d_mM, q_part, out = xhat in dt,
 *                         sum = d_sum, NMSE against the ring's average)
 * ([THC] sections 2-3, Algorithm 1: quantize, integer sum, decode the
 * average; [HVD] 3.4 and [RING] sections 4, 7: the ring average the
 * estimate is measured against). The indices are made from the gradients
 * before the average overwrites them. packed (host array of P device
 * pointers, each 8-byte aligned, ceil(N b / 8) bytes) and d_sum (N int32,
 * 16-byte aligned) may be null to skip writing them; xhat (N elements of
 * dt, 16-byte aligned) is required; d_nmse (num, den, ratio) may be null,
 * else d_ws holds thc_ring_step_ws_bytes(N) bytes. bufs: 16-byte aligned,
 * disjoint. Packed bytes, sums, x̂ and the averages are bit for bit those
 * of the separate calls; the NMSE sums are in another order (within 1e-12
 * relative). GA_ENOTSUP when N or the quantizer partition is not a multiple
 * of 8 (the separate calls take any size).
 */
ga_status thc_ring_step(void* const* bufs, int32_t P, int64_t N, ga_dtype dt, int64_t ring_part,
                        const float* d_mM, int64_t q_part, int32_t b, uint64_t seed, int32_t worker0,
                        uint8_t* const* packed, int32_t* d_sum, void* xhat, double* d_nmse, void* d_ws,
                        size_t ws_bytes, void* stream);
size_t thc_ring_step_ws_bytes(int64_t N);
/* Kernel launches thc_ring_step enqueues for its pass over N elements (it
 * runs in pieces of 2^26 elements, which measured faster than one launch;
 * the NMSE adds one or two small launches): for timing per launch. */
int64_t thc_ring_step_launches(int64_t N);

/* ------------------------------------------------------------------ */
/* Non-uniform THC: lookup tables  ([THC] section 4, Algorithm 2)       */
/* ------------------------------------------------------------------ */

/*
 * A table T of n = 2^b integers, 0 = T[0] < T[1] < ... < T[n-1] = g, maps
 * the b-bit index a worker sends into the finer integer range {0, ..., g}
 * (granularity g >= 2^b - 1): index z stands for m + T[z] (M - m) / g.
 * With g = 2^b - 1 and T the identity these calls equal the uniform ones.
 * Tables are host arrays (n int32), validated on every call; g above 4095
 * returns GA_ENOTSUP.
 */

/*
 * thc_aggregate_dequant -- THC's last three steps in one pass ([THC]
 * Algorithm 1 server sum and worker decoding; Algorithm 2 with a table;
 * the NMSE of section 2): S = sum_i z_i (h_table NULL) or sum_i T[z_i]
 * (h_table, g), x_hat = the dequantized average (as thc_dequant /
 * thc_nuhc_dequant with the same part_elems and d_mM), and, with x_ref,
 * the NMSE of x_hat against x_ref (as thc_nmse).
 *   packed   P device buffers as written by the quantizer (N indices each)
 *   d_sum    device int32[N], or NULL: S is then not stored
 *   out      device, N elements of out_dt (x_hat)
 *   x_ref    device, N elements of out_dt (the exact average), or NULL: no
 *            NMSE, and d_nmse / d_ws are ignored
 *   d_nmse   device double[3]: sum (x - x_hat)^2, sum x^2, their ratio
 *   d_ws     device workspace of thc_aggregate_dequant_ws_bytes(N) bytes
 * S and x_hat are bit-identical to the separate calls; the NMSE sums may
 * differ from thc_nmse's in their last bits (another summation order).
 * Errors as thc_int_aggregate, thc_dequant and thc_nmse.
 */
ga_status thc_aggregate_dequant(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                                int32_t g, const int32_t* h_table, int64_t part_elems,
                                const float* d_mM, int32_t* d_sum, void* out, ga_dtype out_dt,
                                const void* x_ref, double* d_nmse, void* d_ws, size_t ws_bytes,
                                void* stream);
size_t thc_aggregate_dequant_ws_bytes(int64_t N);

/*
 * thc_nuhc_quantize -- as thc_usq_quantize, but each coordinate is rounded
 * stochastically (unbiased) to one of its two neighbouring table values:
 * binary32 u = (a - m) (g / (M - m)); k = min(floor(u), g - 1); z0 = the
 * largest z with T[z] <= k; lo = T[z0], hi = T[z0 + 1];
 * f = (u - lo) / (hi - lo); z = z0 + [(2 r + 1) < f 2^17], with the same
 * 16-bit uniforms, keying and packing as thc_usq_quantize. A value outside
 * [m, M] takes the first (or last) cell and still an index in [0, 2^b - 1].
 */
ga_status thc_nuhc_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                            ga_dtype dt, int64_t part_elems, const float* d_mM, int32_t b,
                            int32_t g, const int32_t* h_table, uint64_t seed,
                            uint8_t* const* packed, void* stream);

/*
 * thc_nuhc_aggregate -- the server of Algorithm 2: d_sum[e] = sum over the
 * P workers of T[z_i[e]] (int32, at most P g).
 */
ga_status thc_nuhc_aggregate(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                             int32_t g, const int32_t* h_table, int32_t* d_sum, void* stream);

/*
 * thc_nuhc_dequant -- Algorithm 2's last steps: divide by the number of
 * workers and map back: out = m + ((float)S / P) ((M - m) / g), binary32;
 * M == m gives m.
 */
ga_status thc_nuhc_dequant(const int32_t* d_sum, int64_t N, int32_t P, int32_t g,
                           int64_t part_elems, const float* d_mM, void* out, ga_dtype out_dt,
                           void* stream);

/* ------------------------------------------------------------------ */
/* Error feedback and partial aggregation  ([THC] sections 5 and 8)     */
/* ------------------------------------------------------------------ */

/*
 * Error feedback: worker i keeps a binary32 vector e_i of what compression
 * has lost so far; it sends x_i = fl32(grad_i + e_i) and then keeps
 * e_i' = fl32(x_i - xhat_i), where xhat_i is the value its own indices
 * stand for: m + (float)v ((M - m) / levels), or m when M == m, with v = z,
 * levels = 2^b - 1 (uniform) or v = T[z], levels = g (table). That is the
 * server's dequantization of a one-worker sum, so e' needs nothing from
 * the server. errs is a host array of P device pointers to N binary32
 * values each; the fast path needs them 16-byte aligned like the inputs.
 *
 * thc_ef_minmax -- as thc_minmax, over x_i = grad_i + e_i.
 */
ga_status thc_ef_minmax(const void* const* bufs, const float* const* errs, int32_t P, int64_t N,
                        ga_dtype dt, int64_t part_elems, float* d_mM, void* stream);

/*
 * thc_ef_minmax_pair -- thc_minmax and thc_ef_minmax of the same buffers in
 * one read of the gradients and residuals: d_mM_x receives the grids of x
 * alone and d_mM_ef those of x + e, each bit for bit what the single call
 * writes ([THC] section 3, preliminary round; section 5, error feedback).
 *   d_mM_x, d_mM_ef   device, 2 ceil(N / part_elems) floats each (8-byte
 *                     aligned), disjoint
 * Other arguments and errors as thc_ef_minmax.
 */
ga_status thc_ef_minmax_pair(const void* const* bufs, const float* const* errs, int32_t P, int64_t N,
                             ga_dtype dt, int64_t part_elems, float* d_mM_x, float* d_mM_ef,
                             void* stream);

/*
 * thc_ef_quantize -- as thc_usq_quantize (h_table NULL; g ignored) or
 * thc_nuhc_quantize (h_table, g) applied to x_i = grad_i + e_i, with the
 * same indices, packing and keying; then overwrites e_i with x_i - xhat_i.
 * One pass: reads grad and e, writes the packed indices and e.
 *
 * Partial aggregation (stragglers, [THC] section 8): the server may sum
 * only the workers that arrived: pass their packed buffers alone to
 * thc_int_aggregate / thc_nuhc_aggregate and their count as P to
 * thc_dequant / thc_nuhc_dequant; the result estimates the mean of those
 * workers.
 */
ga_status thc_ef_quantize(const void* const* bufs, float* const* errs, int32_t P, int32_t worker0,
                          int64_t N, ga_dtype dt, int64_t part_elems, const float* d_mM, int32_t b,
                          int32_t g, const int32_t* h_table, uint64_t seed, uint8_t* const* packed,
                          void* stream);

/* ------------------------------------------------------------------ */
/* Randomized Hadamard transform  ([THC] section 5)                    */
/* ------------------------------------------------------------------ */

/*
 * A vector of N coordinates is cut into blocks of d = 2^k coordinates
 * (2 <= d <= 2^22); a last, partial block is zero-padded, so a transformed
 * vector holds Np = ceil(N / d) d binary32 values. Block p covers
 * coordinates [p d, (p + 1) d).
 *
 * Forward:  y = (1/sqrt(d)) H D x,  inverse:  x = (1/sqrt(d)) D H y, with H
 * the d x d Walsh-Hadamard matrix (H H = d I) and D a diagonal of random
 * signs shared by every worker (seeded; the same seed must reach both
 * directions). H is applied as the radix-2 butterfly: stage s = 0 .. k-1
 * maps every pair (i, i + 2^s), bit s of i clear, to (a + b, a - b) in
 * binary32; the result is then multiplied by c = fl32(1/sqrt(d)). Results
 * are bit-exact against that loop (the pairing inside a stage does not
 * change any rounding).
 * Signs: Philox4x32-10 keyed by seed (low word first), counter
 * (q mod 2^32, q >> 32, 0x52485400, 0) with q = e / 128; coordinate e is
 * negated when bit e mod 32 of output word (e / 32) mod 4 is set.
 */

/*
 * thc_rht_sumsq -- per-block squared norms of the P worker vectors:
 * d_sumsq[i nblk + p] = sum over the coordinates of block p of x_i[e]^2,
 * binary64 (each square is exact there; the order of the additions is a
 * tree, so results may differ from a sequential sum in the last bits).
 * nblk = ceil(N / d); d_sumsq is a device array of P nblk doubles.
 */
ga_status thc_rht_sumsq(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt, int64_t d,
                        double* d_sumsq, void* stream);

/*
 * thc_rht_range -- the norm-based range of every block, shared by all
 * workers: l_p = sqrt(max over i of d_sumsq[i nblk + p]) (the largest
 * worker norm; the page's "squared norm" is read as the norm, the only
 * reading with the units of a coordinate), M = fl32(t_p l_p / sqrt(d))
 * computed in binary64, m = -M. d_mM receives nblk (m, M) pairs. t_p > 0,
 * normally the standard normal quantile Phi^-1(1 - p/2) of the fraction p
 * of coordinates allowed to fall outside the range.
 */
ga_status thc_rht_range(const double* d_sumsq, int32_t P, int64_t nblk, int64_t d, double t_p,
                        float* d_mM, void* stream);

/*
 * thc_rht_forward -- y_i = RHT(x_i) for P workers (x fp32 or bf16, N
 * coordinates; y_i device buffers of Np binary32, written in full). With
 * d_mM non-NULL each y coordinate of block p is then truncated to
 * [m_p, M_p] (d_mM as from thc_rht_range): the truncation step of THC's
 * RHT variant. y must not overlap x.
 */
ga_status thc_rht_forward(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt, int64_t d,
                          uint64_t seed, const float* d_mM, float* const* y, void* stream);

/*
 * thc_rht_quantize -- the forward transform with truncation followed by
 * THC's quantizer on the transformed coordinates, in one call ([THC]
 * section 5 feeding sections 3 and 4: each block of d coordinates is a
 * partition with its range [m_p, M_p] from d_mM). The packed output is
 * bit-identical to thc_rht_forward(bufs, ..., rht_seed, d_mM, y) followed
 * by thc_usq_quantize (h_table NULL; g ignored) or thc_nuhc_quantize
 * (h_table, g) on y with N' = Np, part_elems = d, worker0 and q_seed; the
 * transformed vector itself is not kept.
 *   bufs       P device vectors of N coordinates (fp32 or bf16)
 *   d_mM       device, Np / d pairs (m_p, M_p) as from thc_rht_range
 *   y_scratch  needed when d > 8192 (else may be NULL): P device buffers
 *              of Np binary32, overwritten; must not overlap bufs
 *   packed     P device buffers of ceil(Np b / 8) bytes, 16-byte aligned
 * Errors as thc_rht_forward and thc_nuhc_quantize; GA_EINVAL when
 * d > 8192 and y_scratch is NULL.
 */
ga_status thc_rht_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                           ga_dtype dt, int64_t d, uint64_t rht_seed, const float* d_mM,
                           int32_t b, int32_t g, const int32_t* h_table, uint64_t q_seed,
                           float* const* y_scratch, uint8_t* const* packed, void* stream);

/*
 * thc_rht_norm_quantize -- the block norms, the norm-based range and the
 * truncated transform quantized, in one call ([THC] section 5 on top of
 * sections 3 and 4): as thc_rht_sumsq, thc_rht_range (t_p) and
 * thc_rht_quantize in sequence, with the same bits for d_mM and the packed
 * indices (the norms are binary64 sums of exact squares, summed in another
 * order: within 1e-12 relative of thc_rht_sumsq's). For d > 8192 the
 * norms come from the first pass of the transform, which reads x anyway.
 *   d_sumsq  device double[P][Np/d] (worker-major) or NULL
 *   d_mM     device, receives Np/d pairs (-M_p, M_p)
 *   y_scratch as thc_rht_quantize (needed when d > 8192)
 *   d_ws     device workspace of thc_rht_norm_quantize_ws_bytes(P, N, d)
 *            bytes (8-byte aligned)
 * Errors as thc_rht_sumsq, thc_rht_range and thc_rht_quantize.
 */
ga_status thc_rht_norm_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                                ga_dtype dt, int64_t d, uint64_t rht_seed, double t_p, int32_t b,
                                int32_t g, const int32_t* h_table, uint64_t q_seed, double* d_sumsq,
                                float* d_mM, float* const* y_scratch, void* d_ws, size_t ws_bytes,
                                uint8_t* const* packed, void* stream);
size_t thc_rht_norm_quantize_ws_bytes(int32_t P, int64_t N, int64_t d);

/*
 * thc_rht_inverse -- out = RHT^-1(y) for one vector: y holds Np binary32
 * (device; used as scratch and overwritten when d > 8192), out receives the
 * first N coordinates as fp32 or bf16 (round to nearest even).
 */
ga_status thc_rht_inverse(float* y, int64_t N, int64_t d, uint64_t seed, void* out,
                          ga_dtype out_dt, void* stream);

/* Thread-local message describing the last failure on this thread. */
const char* ga_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GA_H */
