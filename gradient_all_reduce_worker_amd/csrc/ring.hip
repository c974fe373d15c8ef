// ring.hip -- ring all-reduce over P simulated workers held in one HBM.
//
// Semantics ("Horovod: Fast and Easy Distributed Deep Learning in
// TensorFlow", section 3.4, ring-allreduce; systemcraft lesson "Collective
// Communication: Ring All-Reduce", sections 4 and 7): each partition is cut
// into P chunks of C = ceil(n / P) elements; in scatter-reduce step s worker
// i sends chunk (i - s) mod P to worker i + 1, which adds it into its copy;
// all-gather then overwrites every copy with the finished chunk. The sum of
// chunk c is therefore folded in binary32 in the order c, c+1, ..., c-1.
//
// Two executions of that schedule:
//  * fused: each thread owns 16-byte vectors of the buffer, loads the P
//    workers' vectors in the chunk's rotation order, folds them, averages,
//    and stores the result to all P workers. Every byte of every worker is
//    read once and written once: 2 P N elem_bytes of HBM traffic, the
//    minimum for an in-place all-reduce of P buffers.
//  * stepwise: one launch per communication step, moving chunks as the
//    schedule does (RS step: dst += src; AG step: dst = src). This is one
//    GPU's share of a real multi-GPU ring, run for all P workers at once.
// Both give bit-identical results.
//
// Bidirectional ring (lesson section 11, Exercise 1): each partition is cut
// into 2P sub-chunks of C2 = ceil(n / 2P); sub-chunks 0..P-1 run the
// schedule clockwise (fold c, c+1, ..., c-1), sub-chunks P..2P-1
// counter-clockwise (sub-chunk P + c folds c, c-1, ..., c+1). One GPU
// executes it fused, with the same traffic as the single ring; the two
// directions matter for links, not for HBM.
//
// Rotation is uniform inside a chunk, so a workgroup whose elements all lie
// in one chunk of one partition selects its worker pointers with scalar
// loads; the few workgroups straddling a chunk or partition boundary, the
// ragged tail and unaligned buffers take a per-element path.
#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

#include "common.hpp"

namespace ga {
namespace {

constexpr int kVecPerThread = 1;   // 16-byte vectors per thread (stepwise kernels)

struct Div {                        // average: x / P, or x * (1/P) when exact
    int avg;
    int pow2;
    float pf;
    float recip;
    __device__ __forceinline__ float apply(float x) const { return pow2 ? x * recip : x / pf; }
};

template <ga_dtype DT> struct Elem;

template <> struct Elem<GA_F32> {
    static constexpr int kVec = 4;
    __device__ static __forceinline__ void widen(const uint4& r, float* f) {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
    __device__ static __forceinline__ uint4 narrow(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
    __device__ static __forceinline__ float load1(const void* p, int64_t e) {
        return static_cast<const float*>(p)[e];
    }
    __device__ static __forceinline__ void store1(void* p, int64_t e, float v) {
        static_cast<float*>(p)[e] = v;
    }
};

template <> struct Elem<GA_BF16> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ void widen(const uint4& r, float* f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
    __device__ static __forceinline__ uint4 narrow(const float* f) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
    __device__ static __forceinline__ float load1(const void* p, int64_t e) {
        return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[e] << 16);
    }
    __device__ static __forceinline__ void store1(void* p, int64_t e, float v) {
        static_cast<uint16_t*>(p)[e] = (uint16_t)f32_to_bf16_rne(v);
    }
};

// Partition and chunk of element e.
struct Where {
    int64_t part;
    int chunk;
};

// nch chunks per partition: P for the single ring, 2P for the dual ring.
__device__ __forceinline__ Where locate(int64_t e, int64_t N, int64_t plen, int nch) {
    if (N < 0xFFFFFF00ll) {            // 32-bit index arithmetic is exact here
        const uint32_t ue = (uint32_t)e, un = (uint32_t)N, ul = (uint32_t)plen;
        const uint32_t p = ue / ul, p0 = p * ul;
        const uint32_t n = un - p0 < ul ? un - p0 : ul;
        const uint32_t C = (n + (uint32_t)nch - 1u) / (uint32_t)nch;
        return {(int64_t)p, (int)((ue - p0) / C)};
    }
    int64_t p = e / plen;
    int64_t p0 = p * plen;
    int64_t n = N - p0 < plen ? N - p0 : plen;
    int64_t C = (n + nch - 1) / nch;
    return {p, (int)((e - p0) / C)};
}

// Fold start and direction of a chunk: worker r, then r + dir, r + 2 dir, ...
struct Rot {
    int r;
    int dir;
};

template <bool DUAL>
__device__ __forceinline__ Rot rot_of(int chunk, int P) {
    if (DUAL && chunk >= P) return {chunk - P, -1};
    return {chunk, 1};
}

__device__ __forceinline__ int next_worker(int w, int dir, int P) {
    if (dir > 0) return w + 1 == P ? 0 : w + 1;
    return w == 0 ? P - 1 : w - 1;
}

// ---------------------------------------------------------------- fused fold

// Where the workers' base pointers come from: the kernel-argument table of a
// flat all-reduce, or a row of a device table (one fusion-buffer tensor).
struct ArgPtrs {
    const PtrTable& t;
    __device__ __forceinline__ void* operator[](int w) const { return t.p[w]; }
};
struct RowPtrs {
    void* const* p;
    __device__ __forceinline__ void* operator[](int w) const { return p[w]; }
};

// Element idx of every worker, folded from worker rt.r in direction rt.dir.
template <ga_dtype DT, typename PS>
__device__ __forceinline__ void fold_elem(const PS& bufs, int P, int64_t idx, Rot rt, Div div) {
    using E = Elem<DT>;
    float acc = E::load1(bufs[rt.r], idx);
    int w = rt.r;
    for (int k = 1; k < P; k++) {
        w = next_worker(w, rt.dir, P);
        acc = acc + E::load1(bufs[w], idx);
    }
    if (div.avg) acc = div.apply(acc);
    for (int i = 0; i < P; i++) E::store1(bufs[i], idx, acc);
}

template <ga_dtype DT, bool DUAL>
__device__ __forceinline__ void fold_one(const PtrTable& bufs, int P, int64_t N, int64_t plen,
                                         int64_t e, Div div) {
    fold_elem<DT>(ArgPtrs{bufs}, P, e, rot_of<DUAL>(locate(e, N, plen, DUAL ? 2 * P : P).chunk, P),
                  div);
}

// One 16-byte vector v whose elements all start their fold at worker r
// (lane-varying r: pointers are read per lane).
template <ga_dtype DT, typename PS>
__device__ __forceinline__ void fold_vec(const PS& bufs, int P, int64_t v, Rot rt, Div div) {
    using E = Elem<DT>;
    constexpr int V = E::kVec;
    float acc[V];
    E::widen(load_stream(static_cast<const uint4*>(bufs[rt.r]) + v), acc);
    int w = rt.r;
    for (int k = 1; k < P; k++) {
        w = next_worker(w, rt.dir, P);
        float t[V];
        E::widen(load_stream(static_cast<const uint4*>(bufs[w]) + v), t);
#pragma unroll
        for (int i = 0; i < V; i++) acc[i] = acc[i] + t[i];
    }
    if (div.avg) {
#pragma unroll
        for (int i = 0; i < V; i++) acc[i] = div.apply(acc[i]);
    }
    const uint4 o = E::narrow(acc);
    for (int i = 0; i < P; i++) store_stream(static_cast<uint4*>(bufs[i]) + v, o);
}

// The P workers' 16-byte vectors v[j] (where ok[j]), every element folded
// from worker rt.r in direction rt.dir: BATCH worker loads in flight per
// vector, then the average, stored to all P workers.
template <ga_dtype DT, int VPT, int BATCH, typename PS>
__device__ __forceinline__ void fold_uniform(const PS& bufs, int P, const int64_t* v,
                                             const bool* ok, Rot rt, Div div) {
    using E = Elem<DT>;
    constexpr int V = E::kVec;
    const int r = rt.r;
    float acc[VPT][V];
    {
        const uint4* src = static_cast<const uint4*>(bufs[r]);
#pragma unroll
        for (int j = 0; j < VPT; j++) {
            uint4 raw = ok[j] ? load_stream(src + v[j]) : make_uint4(0, 0, 0, 0);
            E::widen(raw, acc[j]);
        }
    }
    for (int k = 1; k < P; k += BATCH) {
        uint4 raw[BATCH][VPT];
#pragma unroll
        for (int kk = 0; kk < BATCH; kk++) {
            if (k + kk < P) {
                int w = rt.dir < 0 ? r - (k + kk) : r + k + kk;
                if (w >= P) w -= P;
                if (w < 0) w += P;
                const uint4* src = static_cast<const uint4*>(bufs[w]);
#pragma unroll
                for (int j = 0; j < VPT; j++)
                    raw[kk][j] = ok[j] ? load_stream(src + v[j]) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int kk = 0; kk < BATCH; kk++) {
            if (k + kk < P) {
#pragma unroll
                for (int j = 0; j < VPT; j++) {
                    float t[V];
                    E::widen(raw[kk][j], t);
#pragma unroll
                    for (int i = 0; i < V; i++) acc[j][i] = acc[j][i] + t[i];
                }
            }
        }
    }
    uint4 out[VPT];
#pragma unroll
    for (int j = 0; j < VPT; j++) {
        if (div.avg) {
#pragma unroll
            for (int i = 0; i < V; i++) acc[j][i] = div.apply(acc[j][i]);
        }
        out[j] = E::narrow(acc[j]);
    }
    for (int w = 0; w < P; w++) {
        uint4* dst = static_cast<uint4*>(bufs[w]);
#pragma unroll
        for (int j = 0; j < VPT; j++)
            if (ok[j]) store_stream(dst + v[j], out[j]);
    }
}

// VPT 16-byte vectors per thread and BATCH worker loads in flight per
// vector (the host picks them with fold_shape).
template <ga_dtype DT, int VPT, int BATCH, bool DUAL>
__global__ __launch_bounds__(kThreads) void ring_fused_vec_kernel(PtrTable bufs, int P, int64_t N,
                                                                  int64_t plen, int64_t n_vec,
                                                                  Div div) {
    using E = Elem<DT>;
    constexpr int V = E::kVec;
    const int nch = DUAL ? 2 * P : P;
    const int64_t vb0 = flat_block() * (kThreads * VPT);
    if (vb0 >= n_vec) return;                              // past the folded grid's end
    const int64_t vb1 = min(vb0 + (int64_t)(kThreads * VPT), n_vec);
    const Where first = locate(vb0 * V, N, plen, nch);
    const Where last = locate(vb1 * V - 1, N, plen, nch);

    if (first.part != last.part || first.chunk != last.chunk) {
        // straddles a chunk or partition boundary: every thread folds its own
        // vectors with their own rotation; only a vector that itself crosses
        // a boundary goes element by element
        for (int j = 0; j < VPT; j++) {
            const int64_t v = vb0 + threadIdx.x + (int64_t)j * kThreads;
            if (v >= vb1) continue;
            const Where a = locate(v * V, N, plen, nch);
            const Where b = locate(v * V + V - 1, N, plen, nch);
            if (a.part == b.part && a.chunk == b.chunk) {
                fold_vec<DT>(ArgPtrs{bufs}, P, v, rot_of<DUAL>(a.chunk, P), div);
            } else {
                for (int i = 0; i < V; i++) fold_one<DT, DUAL>(bufs, P, N, plen, v * V + i, div);
            }
        }
        return;
    }

    // every element of this workgroup starts its fold at worker r, direction dir
    int64_t v[VPT];
    bool ok[VPT];
#pragma unroll
    for (int j = 0; j < VPT; j++) {
        v[j] = vb0 + threadIdx.x + (int64_t)j * kThreads;
        ok[j] = v[j] < vb1;
    }
    fold_uniform<DT, VPT, BATCH>(ArgPtrs{bufs}, P, v, ok, rot_of<DUAL>(first.chunk, P), div);
}

template <ga_dtype DT, bool DUAL>
__global__ __launch_bounds__(kThreads) void ring_fused_elem_kernel(PtrTable bufs, int P, int64_t N,
                                                                   int64_t plen, int64_t e_begin,
                                                                   int64_t e_end, Div div) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t e = e_begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; e < e_end; e += stride)
        fold_one<DT, DUAL>(bufs, P, N, plen, e, div);
}

// ---------------------------------------------------------------- zero-copy fusion ring

static_assert(GA_FUSION_BLOCK == kThreads, "one fusion-ring block per workgroup");

// Header of a planned block of the zero-copy fusion ring; the P workers'
// pointers (to the block's first vector or element) follow it.
struct FusionBlock {
    int32_t count;   // vectors (kind 0) or elements (kind 1), 1..GA_FUSION_BLOCK
    int32_t start;   // first worker of the fold
    int32_t dir;     // +1 or -1
    int32_t kind;    // 0: 16-byte vectors, 1: single elements
};
static_assert(sizeof(FusionBlock) == 16, "block header is 16 bytes");

// Tensor Fusion without the copies: every fusion buffer of a plan folded at
// its tensors' own memory, all buffers in one launch. The host cut every
// tensor at its buffer's partition and chunk boundaries, so each block lies
// in one chunk of one tensor: one fold start and direction for the whole
// workgroup, the P copies' addresses read once (scalar loads of the block),
// thread i folding vector (or element) i of the block.
template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void fusion_ring_kernel(const uint8_t* __restrict__ work,
                                                               int64_t stride, int64_t n_blocks, int P,
                                                               Div div) {
    const int64_t b = flat_block();
    if (b >= n_blocks) return;                             // past the folded grid's end
    const uint8_t* blk = work + b * stride;
    const FusionBlock h = *reinterpret_cast<const FusionBlock*>(blk);
    const RowPtrs row{reinterpret_cast<void* const*>(blk + sizeof(FusionBlock))};
    const Rot rt{h.start, h.dir};
    const int i = threadIdx.x;
    if (h.kind == 0) {
        int64_t v[1] = {i};
        bool ok[1] = {i < h.count};
        if (P <= 16) fold_uniform<DT, 1, 16>(row, P, v, ok, rt, div);
        else fold_uniform<DT, 1, 8>(row, P, v, ok, rt, div);
    } else if (i < h.count) {
        fold_elem<DT>(row, P, i, rt, div);
    }
}

// ---------------------------------------------------------------- stepwise

// Scatter-reduce step s: the element of chunk c is received by worker
// (c + s + 1) mod P from worker (c + s) mod P and added in. On the last step
// with op = avg the receiver, which now holds the finished sum, divides.
// All-gather step s: worker (c + s) mod P receives chunk c from worker
// (c + s - 1) mod P and overwrites its copy.
struct Step {
    int s;
    int rs;          // 1: scatter-reduce step, 0: all-gather step
    int divide;      // last scatter-reduce step with op = avg
};

__device__ __forceinline__ void step_workers(int c, int P, Step st, int* dst, int* src) {
    int d = st.rs ? c + st.s + 1 : c + st.s;
    d %= P;
    int sr = d - 1 < 0 ? P - 1 : d - 1;
    *dst = d;
    *src = sr;
}

__device__ __forceinline__ void step_one(const PtrTable& bufs, int P, int64_t N, int64_t plen,
                                         int64_t e, Step st, Div div) {
    int d, s;
    step_workers(locate(e, N, plen, P).chunk, P, st, &d, &s);
    float* dst = static_cast<float*>(bufs.p[d]);
    const float* src = static_cast<const float*>(bufs.p[s]);
    float x = src[e];
    if (st.rs) {
        x = dst[e] + x;
        if (st.divide) x = div.apply(x);
    }
    dst[e] = x;
}

__global__ __launch_bounds__(kThreads) void ring_step_vec_kernel(PtrTable bufs, int P, int64_t N,
                                                                 int64_t plen, int64_t n_vec,
                                                                 Step st, Div div) {
    constexpr int V = 4;
    const int64_t vb0 = flat_block() * (kThreads * kVecPerThread);
    if (vb0 >= n_vec) return;                              // past the folded grid's end
    const int64_t vb1 = min(vb0 + (int64_t)(kThreads * kVecPerThread), n_vec);
    const Where first = locate(vb0 * V, N, plen, P);
    const Where last = locate(vb1 * V - 1, N, plen, P);
    if (first.part != last.part || first.chunk != last.chunk) {
        for (int64_t e = vb0 * V + threadIdx.x; e < vb1 * V; e += kThreads)
            step_one(bufs, P, N, plen, e, st, div);
        return;
    }
    int d, s;
    step_workers(first.chunk, P, st, &d, &s);
    float4* dst = static_cast<float4*>(bufs.p[d]);
    const float4* src = static_cast<const float4*>(bufs.p[s]);
    float4 a[kVecPerThread], b[kVecPerThread];
    int64_t v[kVecPerThread];
#pragma unroll
    for (int j = 0; j < kVecPerThread; j++) {
        v[j] = vb0 + threadIdx.x + (int64_t)j * kThreads;
        if (v[j] < vb1) {
            a[j] = src[v[j]];
            if (st.rs) b[j] = dst[v[j]];
        }
    }
#pragma unroll
    for (int j = 0; j < kVecPerThread; j++) {
        if (v[j] >= vb1) continue;
        float4 x = a[j];
        if (st.rs) {
            x.x = b[j].x + x.x; x.y = b[j].y + x.y; x.z = b[j].z + x.z; x.w = b[j].w + x.w;
            if (st.divide) {
                x.x = div.apply(x.x); x.y = div.apply(x.y);
                x.z = div.apply(x.z); x.w = div.apply(x.w);
            }
        }
        dst[v[j]] = x;
    }
}

__global__ __launch_bounds__(kThreads) void ring_step_elem_kernel(PtrTable bufs, int P, int64_t N,
                                                                  int64_t plen, int64_t e_begin,
                                                                  int64_t e_end, Step st, Div div) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t e = e_begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; e < e_end; e += stride)
        step_one(bufs, P, N, plen, e, st, div);
}

// ---------------------------------------------------------------- staged stepwise

// The stepwise schedule with the partials on a binary32 wire: at scatter-
// reduce step s every element e (chunk c) has exactly one partial in flight,
// from worker c + s to worker c + s + 1, so one binary32 array stage[N]
// holds all of them. The receiver adds its own value to the partial (at the
// first step the sender's own value, read from its buffer) and writes the
// stage; at the last step it divides (op = avg) and stores the finished
// value, rounded once, into its own buffer. All-gather steps copy the
// finished chunk between worker buffers in the buffers' own type. The fold
// order and the roundings are those of the fused fold.
struct Staged {
    int s;
    int rs;          // 1: scatter-reduce step, 0: all-gather step
    int first;      // scatter-reduce step 0: the partial comes from the sender's buffer
    int last;       // scatter-reduce step P - 2: the finished value goes to the receiver's buffer
};

template <ga_dtype DT>
__device__ __forceinline__ void staged_one(const PtrTable& bufs, float* stage, int P, int64_t N,
                                           int64_t plen, int64_t e, Staged st, Div div) {
    using E = Elem<DT>;
    int d, s;
    step_workers(locate(e, N, plen, P).chunk, P, Step{st.s, st.rs, 0}, &d, &s);
    if (!st.rs) {                                    // all-gather: the bits as they are
        if (DT == GA_F32) static_cast<uint32_t*>(bufs.p[d])[e] = static_cast<const uint32_t*>(bufs.p[s])[e];
        else static_cast<uint16_t*>(bufs.p[d])[e] = static_cast<const uint16_t*>(bufs.p[s])[e];
        return;
    }
    const float a = st.first ? E::load1(bufs.p[s], e) : stage[e];
    float x = a + E::load1(bufs.p[d], e);
    if (st.last) {
        if (div.avg) x = div.apply(x);
        E::store1(bufs.p[d], e, x);
    } else {
        stage[e] = x;
    }
}

// One 16-byte vector of the buffers' type per thread (4 binary32 or 8 bf16
// elements; the stage holds them in one or two 16-byte vectors); a
// workgroup whose vectors lie in more than one chunk goes element by element.
template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void ring_staged_vec_kernel(PtrTable bufs, float* __restrict__ stage,
                                                                   int P, int64_t N, int64_t plen,
                                                                   int64_t n_vec, Staged st, Div div) {
    using E = Elem<DT>;
    constexpr int V = E::kVec;
    const int64_t vb0 = flat_block() * kThreads;
    if (vb0 >= n_vec) return;                              // past the folded grid's end
    const int64_t vb1 = min(vb0 + (int64_t)kThreads, n_vec);
    const Where first = locate(vb0 * V, N, plen, P);
    const Where last = locate(vb1 * V - 1, N, plen, P);
    if (first.part != last.part || first.chunk != last.chunk) {
        for (int64_t e = vb0 * V + threadIdx.x; e < vb1 * V; e += kThreads)
            staged_one<DT>(bufs, stage, P, N, plen, e, st, div);
        return;
    }
    const int64_t v = vb0 + threadIdx.x;
    if (v >= vb1) return;
    int d, s;
    step_workers(first.chunk, P, Step{st.s, st.rs, 0}, &d, &s);
    uint4* dst = static_cast<uint4*>(bufs.p[d]);
    if (!st.rs) {
        dst[v] = static_cast<const uint4*>(bufs.p[s])[v];
        return;
    }
    constexpr int K = V / 4;                               // stage vectors per buffer vector
    uint4* sv = reinterpret_cast<uint4*>(stage) + K * v;
    float a[V], x[V];
    if (st.first) {
        E::widen(static_cast<const uint4*>(bufs.p[s])[v], a);
    } else {
#pragma unroll
        for (int k = 0; k < K; k++) Elem<GA_F32>::widen(sv[k], a + 4 * k);
    }
    E::widen(dst[v], x);
#pragma unroll
    for (int i = 0; i < V; i++) x[i] = a[i] + x[i];
    if (st.last) {
        if (div.avg) {
#pragma unroll
            for (int i = 0; i < V; i++) x[i] = div.apply(x[i]);
        }
        dst[v] = E::narrow(x);
    } else {
#pragma unroll
        for (int k = 0; k < K; k++) sv[k] = Elem<GA_F32>::narrow(x + 4 * k);
    }
}

template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void ring_staged_elem_kernel(PtrTable bufs, float* __restrict__ stage,
                                                                    int P, int64_t N, int64_t plen,
                                                                    int64_t e_begin, int64_t e_end,
                                                                    Staged st, Div div) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t e = e_begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; e < e_end; e += stride)
        staged_one<DT>(bufs, stage, P, N, plen, e, st, div);
}

int elem_grid(int64_t count) {
    int64_t b = ceil_div(count, kThreads);
    return (int)(b < 65536 ? (b < 1 ? 1 : b) : 65536);
}

bool disjoint(void* const* bufs, int P, int64_t bytes) {
    for (int i = 0; i < P; i++)
        for (int j = i + 1; j < P; j++) {
            uintptr_t a = (uintptr_t)bufs[i], b = (uintptr_t)bufs[j];
            if (a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes) return false;
        }
    return true;
}

// Launch shape of the fused fold, measured on MI355X. Folding P streams and
// writing P back keeps 2P DRAM streams open per workgroup; on large buffers
// fewer resident workgroups per CU keep fewer rows open and stream faster
// (8 x 4 GiB bf16: 0.72 -> 0.79 of 8 TB/s at two workgroups per CU, and
// from 256 MiB moved on: the 200-tensor fusion plan, 8 workers, 553 MB,
// 0.64 -> 0.66 flat and 0.69 -> 0.72 zero-copy; 16 workers of 66 MB:
// 0.68 -> 0.74 at one; 32 workers of 553 MB with four vectors per thread:
// 0.73 -> 0.77 at four). Residency is capped with unused dynamic LDS
// (160 KiB per CU). Small buffers keep full occupancy.
struct FoldShape {
    int vpt;        // 16-byte vectors per thread
    int batch;      // worker loads in flight per vector
    size_t lds;     // dynamic LDS per workgroup (0: no cap)
};

constexpr size_t kLdsPerCu = 160 * 1024;

size_t cap_workgroups_per_cu(int k) { return kLdsPerCu / (size_t)k - 1024; }

FoldShape fold_shape(int P, int64_t total_bytes) {
    const bool big = total_bytes >= (int64_t)1 << 30;
    if (P <= 8) return {1, 16, total_bytes >= ((int64_t)1 << 28) ? cap_workgroups_per_cu(2) : 0};
    if (P <= 16) return {1, 16, big ? cap_workgroups_per_cu(1) : 0};
    return {4, 4, big ? cap_workgroups_per_cu(4) : 0};
}

// The zero-copy fusion ring: a workgroup starts with scalar loads of its
// planned block, as cheaply as the flat fold, so the flat fold's residency
// caps apply (ResNet-101 plan, 16 workers: 0.65 of 8 TB/s at two resident
// workgroups per CU, 0.685 at one; the flat ring over the fusion buffers
// 0.684).
size_t fusion_cap(int P, int64_t total_bytes) { return fold_shape(P, total_bytes).lds; }

// The fused fold over the whole buffer: the vector kernel over 16-byte
// vectors when every buffer is 16-byte aligned, the element kernel for the
// rest. Returns the number of launches, or a negative status.
template <bool DUAL>
int64_t launch_fused(void* const* bufs, int P, int64_t N, ga_dtype dt, int64_t plen, Div div,
                     hipStream_t hs, const char* what) {
    const int64_t n_vec = N / (dt == GA_F32 ? 4 : 8);
    const int64_t vec_elems = n_vec * (dt == GA_F32 ? 4 : 8);
    bool vec_ok = true;
    for (int i = 0; i < P; i++) vec_ok = vec_ok && aligned(bufs[i], 16);
    PtrTable t{};
    for (int i = 0; i < P; i++) t.p[i] = bufs[i];
    int64_t launches = 0;
    ga_status rc;
    if (vec_ok && n_vec > 0) {
        const FoldShape sh = fold_shape(P, 2 * (int64_t)P * N * (int64_t)elem_size(dt));
        const int64_t nb = ceil_div(n_vec, (int64_t)kThreads * sh.vpt);
        if (!flat_fits(nb)) return fail(GA_EINVAL, "%s: N too large", what);
        const dim3 blocks = flat_grid(nb);
        if (dt == GA_F32 && sh.vpt == 4)
            hipLaunchKernelGGL((ring_fused_vec_kernel<GA_F32, 4, 4, DUAL>), dim3(blocks),
                               dim3(kThreads), sh.lds, hs, t, P, N, plen, n_vec, div);
        else if (dt == GA_F32)
            hipLaunchKernelGGL((ring_fused_vec_kernel<GA_F32, 1, 16, DUAL>), dim3(blocks),
                               dim3(kThreads), sh.lds, hs, t, P, N, plen, n_vec, div);
        else if (sh.vpt == 4)
            hipLaunchKernelGGL((ring_fused_vec_kernel<GA_BF16, 4, 4, DUAL>), dim3(blocks),
                               dim3(kThreads), sh.lds, hs, t, P, N, plen, n_vec, div);
        else
            hipLaunchKernelGGL((ring_fused_vec_kernel<GA_BF16, 1, 16, DUAL>), dim3(blocks),
                               dim3(kThreads), sh.lds, hs, t, P, N, plen, n_vec, div);
        launches++;
        if ((rc = check_launch(what))) return rc;
    }
    const int64_t e0 = (vec_ok && n_vec > 0) ? vec_elems : 0;
    if (e0 < N) {
        if (dt == GA_F32)
            hipLaunchKernelGGL((ring_fused_elem_kernel<GA_F32, DUAL>), dim3(elem_grid(N - e0)),
                               dim3(kThreads), 0, hs, t, P, N, plen, e0, N, div);
        else
            hipLaunchKernelGGL((ring_fused_elem_kernel<GA_BF16, DUAL>), dim3(elem_grid(N - e0)),
                               dim3(kThreads), 0, hs, t, P, N, plen, e0, N, div);
        launches++;
        if ((rc = check_launch(what))) return rc;
    }
    return launches;
}

}  // namespace
}  // namespace ga

using namespace ga;

extern "C" ga_status ga_ring_allreduce_sim(void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                           ga_op op, int64_t part_elems, ga_ring_mode mode,
                                           ga_ring_stats* st, void* stream) {
    const char* what = "ga_ring_allreduce_sim";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (op != GA_SUM && op != GA_AVG) return fail(GA_EINVAL, "%s: unknown op %d", what, (int)op);
    if (mode != GA_RING_FUSED && mode != GA_RING_STEPWISE && mode != GA_RING_DUAL)
        return fail(GA_EINVAL, "%s: unknown mode %d", what, (int)mode);
    if (N < 0 || part_elems < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS)
        return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    const size_t es = elem_size(dt);
    if (N == 0) {                       // empty buffers (possibly null): nothing to do
        if (st) *st = ga_ring_stats{0, 0, 0, 0};
        return GA_OK;
    }
    ga_status rc = check_workers(bufs, P, es, what);
    if (rc) return rc;
    if (!disjoint(bufs, P, N * (int64_t)es))
        return fail(GA_EINVAL, "%s: worker buffers overlap", what);
    if (mode == GA_RING_STEPWISE && dt != GA_F32)
        return fail(GA_ENOTSUP, "%s: the stepwise schedule keeps binary32 partials in the worker "
                    "buffers, so it needs GA_F32 buffers", what);

    const int64_t plen = part_elems > 0 ? part_elems : (N > 0 ? N : 1);
    const int64_t n_vec = N / (dt == GA_F32 ? 4 : 8);
    const int64_t vec_elems = n_vec * (dt == GA_F32 ? 4 : 8);
    bool vec_ok = true;
    for (int i = 0; i < P; i++) vec_ok = vec_ok && aligned(bufs[i], 16);

    ga_ring_stats s{};
    {
        // every step sends one chunk per ring; the dual ring sends one
        // sub-chunk of ceil(n / 2P) in each direction
        // whole partitions, then the short last one (closed form, no loop)
        auto part_bytes = [&](int64_t n) {
            return mode == GA_RING_DUAL
                       ? 2 * 2 * (int64_t)(P - 1) * ceil_div(n, 2 * (int64_t)P) * (int64_t)es
                       : 2 * (int64_t)(P - 1) * ceil_div(n, P) * (int64_t)es;
        };
        const int64_t bytes = (N / plen) * part_bytes(plen) + (N % plen ? part_bytes(N % plen) : 0);
        s.steps = N > 0 ? 2 * (int64_t)(P - 1) : 0;
        s.bytes_sent_per_worker = bytes;
        if (mode != GA_RING_STEPWISE)
            s.hbm_bytes = (P > 1) ? 2 * (int64_t)P * N * (int64_t)es : 0;
        else
            s.hbm_bytes = 5 * (int64_t)(P - 1) * N * (int64_t)es;
    }

    hipStream_t hs = static_cast<hipStream_t>(stream);
    Div div{op == GA_AVG, (P & (P - 1)) == 0, (float)P, 1.0f / (float)P};
    int64_t launches = 0;

    if (N > 0 && P > 1) {
        const int64_t vblocks = ceil_div(n_vec, kThreads * kVecPerThread);
        if (!flat_fits(vblocks)) return fail(GA_EINVAL, "%s: N too large", what);
        if (mode == GA_RING_FUSED || mode == GA_RING_DUAL) {
            const int64_t n = mode == GA_RING_DUAL
                                  ? launch_fused<true>(bufs, P, N, dt, plen, div, hs, what)
                                  : launch_fused<false>(bufs, P, N, dt, plen, div, hs, what);
            if (n < 0) return (ga_status)n;
            launches += n;
        } else {
            PtrTable t{};
            for (int i = 0; i < P; i++) t.p[i] = bufs[i];
            const int64_t e0 = (vec_ok && n_vec > 0) ? vec_elems : 0;
            for (int phase = 0; phase < 2; phase++) {
                for (int step = 0; step < P - 1; step++) {
                    Step sp{step, phase == 0, phase == 0 && step == P - 2 && op == GA_AVG};
                    if (vec_ok && n_vec > 0) {
                        hipLaunchKernelGGL(ring_step_vec_kernel, flat_grid(vblocks),
                                           dim3(kThreads), 0, hs, t, P, N, plen, n_vec, sp, div);
                        launches++;
                        if ((rc = check_launch(what))) return rc;
                    }
                    if (e0 < N) {
                        hipLaunchKernelGGL(ring_step_elem_kernel, dim3(elem_grid(N - e0)),
                                           dim3(kThreads), 0, hs, t, P, N, plen, e0, N, sp, div);
                        launches++;
                        if ((rc = check_launch(what))) return rc;
                    }
                }
            }
        }
    }
    s.launches = launches;
    if (st) *st = s;
    return GA_OK;
}

extern "C" size_t ga_ring_stage_bytes(int32_t P, int64_t N) {
    return (P > 2 && N > 0) ? (size_t)N * sizeof(float) : 0;
}

extern "C" ga_status ga_ring_stepwise_staged(void* const* bufs, int32_t P, int64_t N, ga_dtype dt, ga_op op,
                                             int64_t part_elems, float* d_stage, size_t stage_bytes,
                                             ga_ring_stats* st, void* stream) {
    const char* what = "ga_ring_stepwise_staged";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (op != GA_SUM && op != GA_AVG) return fail(GA_EINVAL, "%s: unknown op %d", what, (int)op);
    if (N < 0 || part_elems < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS)
        return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) {
        if (st) *st = ga_ring_stats{0, 0, 0, 0};
        return GA_OK;
    }
    const int64_t es = (int64_t)elem_size(dt);
    ga_status rc = check_workers(bufs, P, (size_t)es, what);
    if (rc) return rc;
    if (!disjoint(bufs, P, N * es)) return fail(GA_EINVAL, "%s: worker buffers overlap", what);
    const size_t need = ga_ring_stage_bytes(P, N);
    if (need > 0) {
        if (!d_stage || !aligned(d_stage, 16))
            return fail(GA_EINVAL, "%s: null or misaligned stage (16 bytes)", what);
        if (stage_bytes < need)
            return fail(GA_EINVAL, "%s: stage of %zu bytes, need %zu", what, stage_bytes, need);
        const uintptr_t a = (uintptr_t)d_stage;
        for (int i = 0; i < P; i++) {
            const uintptr_t b = (uintptr_t)bufs[i];
            if (a < b + (uintptr_t)(N * es) && b < a + need)
                return fail(GA_EINVAL, "%s: stage overlaps worker %d", what, i);
        }
    }
    const int64_t plen = part_elems > 0 ? part_elems : N;
    ga_ring_stats s{};
    {
        // scatter-reduce partials travel in binary32, the all-gather in the
        // buffers' type
        auto part_bytes = [&](int64_t n) { return (int64_t)(P - 1) * ceil_div(n, P) * (4 + es); };
        s.steps = 2 * (int64_t)(P - 1);
        s.bytes_sent_per_worker = (N / plen) * part_bytes(plen) + (N % plen ? part_bytes(N % plen) : 0);
        // step 0 reads two buffers and writes the stage, the middle steps read
        // the stage and a buffer and write the stage, the last reads the
        // stage and a buffer and writes a buffer (P = 2: two buffers in, one
        // out); every all-gather step copies N elements
        const int64_t rs = P == 1 ? 0
                         : P == 2 ? 3 * es * N
                                  : (2 * es + 4) * N + (int64_t)(P - 3) * (8 + es) * N + (4 + 2 * es) * N;
        s.hbm_bytes = rs + (int64_t)(P - 1) * 2 * es * N;
    }
    const int V = dt == GA_F32 ? 4 : 8;
    bool vec_ok = true;
    for (int i = 0; i < P; i++) vec_ok = vec_ok && aligned(bufs[i], 16);
    const int64_t n_vec = vec_ok ? N / V : 0;
    const int64_t vblocks = ceil_div(n_vec, kThreads);
    if (!flat_fits(vblocks)) return fail(GA_EINVAL, "%s: N too large", what);
    const int64_t e0 = n_vec * V;
    PtrTable t{};
    for (int i = 0; i < P; i++) t.p[i] = bufs[i];
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const Div div{op == GA_AVG, (P & (P - 1)) == 0, (float)P, 1.0f / (float)P};
    int64_t launches = 0;
    for (int phase = 0; phase < 2 && P > 1; phase++) {
        for (int step = 0; step < P - 1; step++) {
            const Staged sp{step, phase == 0, phase == 0 && step == 0, phase == 0 && step == P - 2};
            if (n_vec > 0) {
                if (dt == GA_F32)
                    hipLaunchKernelGGL(ring_staged_vec_kernel<GA_F32>, flat_grid(vblocks), dim3(kThreads), 0, hs,
                                       t, d_stage, P, N, plen, n_vec, sp, div);
                else
                    hipLaunchKernelGGL(ring_staged_vec_kernel<GA_BF16>, flat_grid(vblocks), dim3(kThreads), 0, hs,
                                       t, d_stage, P, N, plen, n_vec, sp, div);
                launches++;
                if ((rc = check_launch(what))) return rc;
            }
            if (e0 < N) {
                if (dt == GA_F32)
                    hipLaunchKernelGGL(ring_staged_elem_kernel<GA_F32>, dim3(elem_grid(N - e0)), dim3(kThreads), 0,
                                       hs, t, d_stage, P, N, plen, e0, N, sp, div);
                else
                    hipLaunchKernelGGL(ring_staged_elem_kernel<GA_BF16>, dim3(elem_grid(N - e0)), dim3(kThreads), 0,
                                       hs, t, d_stage, P, N, plen, e0, N, sp, div);
                launches++;
                if ((rc = check_launch(what))) return rc;
            }
        }
    }
    s.launches = launches;
    if (st) *st = s;
    return GA_OK;
}

// ---------------------------------------------------------------- zero-copy fusion ring (host)

namespace {

// Appends the blocks of one piece [a, b) of tensor t (tensor elements, one
// chunk: fold start r, direction dir) to the work array (or only counts).
struct WorkWriter {
    uint8_t* out;
    int64_t cap;
    int64_t n = 0;
    int P;
    int64_t es;
    void* const* ptrs;     // the tensor's P pointers
    void add(int kind, int64_t first, int64_t count, Rot rt) {
        if (out && n < cap) {
            uint8_t* blk = out + n * (int64_t)GA_FUSION_BLOCK_BYTES(P);
            FusionBlock h{(int32_t)count, rt.r, rt.dir, kind};
            memcpy(blk, &h, sizeof h);
            const int64_t unit = kind == 0 ? 16 : es;
            for (int i = 0; i < P; i++) {
                void* q = static_cast<uint8_t*>(ptrs[i]) + first * unit;
                memcpy(blk + sizeof h + 8 * i, &q, 8);
            }
        }
        n++;
    }
    void span(int kind, int64_t lo, int64_t hi, Rot rt) {      // units [lo, hi)
        for (int64_t k = lo; k < hi; k += GA_FUSION_BLOCK)
            add(kind, k, std::min<int64_t>(GA_FUSION_BLOCK, hi - k), rt);
    }
    void piece(int64_t a, int64_t b, bool vec, Rot rt) {
        const int64_t V = 16 / es;
        const int64_t va = ceil_div(a, V), vb = b / V;         // whole vectors inside [a, b)
        if (!vec || va >= vb) {
            span(1, a, b, rt);
            return;
        }
        span(1, a, va * V, rt);
        span(0, va, vb, rt);
        span(1, vb * V, b, rt);
    }
};

}  // namespace

extern "C" ga_status ga_fusion_ring_plan(const ga_fusion_tensor* h_tensors, void* const* h_ptrs,
                                         int64_t n_tensors, int32_t P, ga_dtype dt,
                                         const int64_t* fill, int32_t n_buf, int64_t part_elems,
                                         ga_ring_mode mode, void* h_work, int64_t cap_blocks,
                                         int64_t* n_blocks) {
    const char* what = "ga_fusion_ring_plan";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (P < 1 || P > GA_MAX_WORKERS)
        return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (mode == GA_RING_STEPWISE)
        return fail(GA_ENOTSUP, "%s: the zero-copy ring runs the fused fold only", what);
    if (mode != GA_RING_FUSED && mode != GA_RING_DUAL)
        return fail(GA_EINVAL, "%s: unknown mode %d", what, (int)mode);
    if (n_tensors < 0 || n_buf < 0 || part_elems < 0 || cap_blocks < 0 || !n_blocks)
        return fail(GA_EINVAL, "%s: bad sizes", what);
    if (n_tensors > 0 && (!h_tensors || !h_ptrs)) return fail(GA_EINVAL, "%s: null table", what);
    if (n_buf > 0 && !fill) return fail(GA_EINVAL, "%s: null fills", what);
    for (int32_t k = 0; k < n_buf; k++)
        if (fill[k] < 0) return fail(GA_EINVAL, "%s: buffer %d has fill %lld", what, k, (long long)fill[k]);
    const int64_t es = (int64_t)elem_size(dt);
    const int nch = mode == GA_RING_DUAL ? 2 * P : P;
    int64_t off = 0;
    int32_t cur = 0;             // buffer being walked; buffers below it are complete
    std::vector<std::pair<uintptr_t, uintptr_t>> spans;
    spans.reserve((size_t)(n_tensors * P));
    // the buffer being walked must be complete; buffers before k that no
    // row lists must be empty
    auto skip_to = [&](int32_t k) -> ga_status {
        if (off != fill[cur])
            return fail(GA_EINVAL, "%s: buffer %d's tensors cover %lld elements, its fill is %lld",
                        what, cur, (long long)off, (long long)fill[cur]);
        for (int32_t q = cur + 1; q < k; q++)
            if (fill[q] != 0)
                return fail(GA_EINVAL, "%s: buffer %d has fill %lld but no tensors", what, q,
                            (long long)fill[q]);
        cur = k;
        off = 0;
        return GA_OK;
    };
    // first pass: check the table
    for (int64_t t = 0; t < n_tensors; t++) {
        const ga_fusion_tensor& d = h_tensors[t];
        if (d.buf < 0 || d.buf >= n_buf || d.buf < cur)
            return fail(GA_EINVAL, "%s: tensor %lld has buffer %d (buffers [0, %d), never "
                        "decreasing; the table is at buffer %d)", what, (long long)t, d.buf, n_buf, cur);
        if (d.buf > cur) {
            ga_status rc = skip_to(d.buf);
            if (rc) return rc;
        }
        if (d.n < 0 || d.start != off)
            return fail(GA_EINVAL, "%s: tensor %lld is not dense in buffer order (start %lld, "
                        "expected %lld)", what, (long long)t, (long long)d.start, (long long)off);
        for (int i = 0; i < P; i++) {
            const void* q = h_ptrs[t * P + i];
            if (d.n > 0 && (!q || !aligned(q, (uintptr_t)es)))
                return fail(GA_EINVAL, "%s: tensor %lld, worker %d: null or misaligned pointer",
                            what, (long long)t, i);
            if (d.n > 0) spans.push_back({(uintptr_t)q, (uintptr_t)q + (uintptr_t)(d.n * es)});
        }
        off += d.n;
    }
    if (n_buf > 0) {
        ga_status rc = skip_to(n_buf);
        if (rc) return rc;
    }
    std::sort(spans.begin(), spans.end());
    for (size_t k = 1; k < spans.size(); k++)
        if (spans[k].first < spans[k - 1].second)
            return fail(GA_EINVAL, "%s: two tensor copies overlap", what);
    // second pass: cut every tensor at its buffer's partition and chunk
    // boundaries (the chunk rule of the ring: C = ceil(n_p / nch))
    WorkWriter ww{static_cast<uint8_t*>(h_work), cap_blocks, 0, P, es, nullptr};
    for (int64_t t = 0; t < n_tensors; t++) {
        const ga_fusion_tensor& d = h_tensors[t];
        const int64_t F = fill[d.buf];
        const int64_t plen = part_elems > 0 ? part_elems : F;
        bool vec = true;
        for (int i = 0; i < P; i++) vec = vec && aligned(h_ptrs[t * P + i], 16);
        ww.ptrs = h_ptrs + t * P;
        for (int64_t e = d.start; e < d.start + d.n;) {
            const int64_t p0 = e / plen * plen;
            const int64_t np = std::min(plen, F - p0);
            const int64_t C = ceil_div(np, nch);
            const int c = (int)((e - p0) / C);
            const int64_t end = std::min(p0 + std::min((int64_t)(c + 1) * C, np), d.start + d.n);
            const Rot rt = (mode == GA_RING_DUAL && c >= P) ? Rot{c - P, -1} : Rot{c, 1};
            ww.piece(e - d.start, end - d.start, vec, rt);
            e = end;
        }
    }
    if (h_work && ww.n > cap_blocks)
        return fail(GA_EINVAL, "%s: %lld blocks do not fit in %lld", what, (long long)ww.n,
                    (long long)cap_blocks);
    *n_blocks = ww.n;
    return GA_OK;
}

extern "C" ga_status ga_fusion_ring_allreduce(const void* d_work, int64_t n_blocks, int32_t P,
                                              ga_dtype dt, ga_op op, const int64_t* fill,
                                              int32_t n_buf, int64_t part_elems, ga_ring_mode mode,
                                              ga_ring_stats* st, void* stream) {
    const char* what = "ga_fusion_ring_allreduce";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (op != GA_SUM && op != GA_AVG) return fail(GA_EINVAL, "%s: unknown op %d", what, (int)op);
    if (mode == GA_RING_STEPWISE)
        return fail(GA_ENOTSUP, "%s: the zero-copy ring runs the fused fold only", what);
    if (mode != GA_RING_FUSED && mode != GA_RING_DUAL)
        return fail(GA_EINVAL, "%s: unknown mode %d", what, (int)mode);
    if (P < 1 || P > GA_MAX_WORKERS)
        return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (n_blocks < 0 || n_buf < 0 || part_elems < 0)
        return fail(GA_EINVAL, "%s: negative size", what);
    if (n_buf > 0 && !fill) return fail(GA_EINVAL, "%s: null fills", what);
    int64_t total = 0;
    for (int32_t k = 0; k < n_buf; k++) {
        if (fill[k] < 0) return fail(GA_EINVAL, "%s: negative fill", what);
        total += fill[k];
    }
    if (n_blocks > 0 && total == 0) return fail(GA_EINVAL, "%s: work without tensors", what);
    const int64_t es = (int64_t)elem_size(dt);
    const int nch = mode == GA_RING_DUAL ? 2 * P : P;
    ga_ring_stats s{};
    {
        auto part_bytes = [&](int64_t n) { return 2 * (int64_t)(P - 1) * (nch / P) * ceil_div(n, nch) * es; };
        int64_t bytes = 0;
        for (int32_t k = 0; k < n_buf; k++) {
            if (fill[k] == 0) continue;
            const int64_t plen = part_elems > 0 ? part_elems : fill[k];
            bytes += (fill[k] / plen) * part_bytes(plen) + (fill[k] % plen ? part_bytes(fill[k] % plen) : 0);
        }
        s.steps = total > 0 ? 2 * (int64_t)(P - 1) : 0;
        s.bytes_sent_per_worker = bytes;
        s.hbm_bytes = P > 1 ? 2 * (int64_t)P * total * es : 0;
    }
    if (n_blocks == 0 || P == 1) {
        if (st) *st = s;
        return GA_OK;
    }
    if (!d_work || !aligned(d_work, 8)) return fail(GA_EINVAL, "%s: null or misaligned blocks", what);
    if (!flat_fits(n_blocks)) return fail(GA_EINVAL, "%s: too many blocks", what);
    Div div{op == GA_AVG, (P & (P - 1)) == 0, (float)P, 1.0f / (float)P};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t lds = fusion_cap(P, 2 * (int64_t)P * total * es);
    const int64_t stride = (int64_t)GA_FUSION_BLOCK_BYTES(P);
    const uint8_t* w = static_cast<const uint8_t*>(d_work);
    if (dt == GA_F32)
        hipLaunchKernelGGL((fusion_ring_kernel<GA_F32>), flat_grid(n_blocks), dim3(kThreads), lds, hs, w, stride,
                           n_blocks, P, div);
    else
        hipLaunchKernelGGL((fusion_ring_kernel<GA_BF16>), flat_grid(n_blocks), dim3(kThreads), lds, hs, w, stride,
                           n_blocks, P, div);
    ga_status rc = check_launch(what);
    if (rc) return rc;
    s.launches = 1;
    if (st) *st = s;
    return GA_OK;
}
