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
// Rotation is uniform inside a chunk, so a workgroup whose elements all lie
// in one chunk of one partition selects its worker pointers with scalar
// loads; the few workgroups straddling a chunk or partition boundary, the
// ragged tail and unaligned buffers take a per-element path.
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

__device__ __forceinline__ Where locate(int64_t e, int64_t N, int64_t plen, int P) {
    if (N < 0xFFFFFF00ll) {            // 32-bit index arithmetic is exact here
        const uint32_t ue = (uint32_t)e, un = (uint32_t)N, ul = (uint32_t)plen;
        const uint32_t p = ue / ul, p0 = p * ul;
        const uint32_t n = un - p0 < ul ? un - p0 : ul;
        const uint32_t C = (n + (uint32_t)P - 1u) / (uint32_t)P;
        return {(int64_t)p, (int)((ue - p0) / C)};
    }
    int64_t p = e / plen;
    int64_t p0 = p * plen;
    int64_t n = N - p0 < plen ? N - p0 : plen;
    int64_t C = (n + P - 1) / P;
    return {p, (int)((e - p0) / C)};
}

// ---------------------------------------------------------------- fused fold

template <ga_dtype DT>
__device__ __forceinline__ void fold_one(const PtrTable& bufs, int P, int64_t N, int64_t plen,
                                         int64_t e, Div div) {
    using E = Elem<DT>;
    const int c = locate(e, N, plen, P).chunk;
    float acc = E::load1(bufs.p[c], e);
    int w = c;
    for (int k = 1; k < P; k++) {
        w = (w + 1 == P) ? 0 : w + 1;
        acc = acc + E::load1(bufs.p[w], e);
    }
    if (div.avg) acc = div.apply(acc);
    for (int i = 0; i < P; i++) E::store1(bufs.p[i], e, acc);
}

// One 16-byte vector v whose elements all start their fold at worker r
// (lane-varying r: pointers are read per lane).
template <ga_dtype DT>
__device__ __forceinline__ void fold_vec(const PtrTable& bufs, int P, int64_t v, int r, Div div) {
    using E = Elem<DT>;
    constexpr int V = E::kVec;
    float acc[V];
    E::widen(load_stream(static_cast<const uint4*>(bufs.p[r]) + v), acc);
    int w = r;
    for (int k = 1; k < P; k++) {
        w = (w + 1 == P) ? 0 : w + 1;
        float t[V];
        E::widen(load_stream(static_cast<const uint4*>(bufs.p[w]) + v), t);
#pragma unroll
        for (int i = 0; i < V; i++) acc[i] = acc[i] + t[i];
    }
    if (div.avg) {
#pragma unroll
        for (int i = 0; i < V; i++) acc[i] = div.apply(acc[i]);
    }
    const uint4 o = E::narrow(acc);
    for (int i = 0; i < P; i++) store_stream(static_cast<uint4*>(bufs.p[i]) + v, o);
}

// VPT 16-byte vectors per thread and BATCH worker loads in flight: one vector
// and 16 loads for P <= 8, two vectors and 8 loads for larger P (measured).
template <ga_dtype DT, int VPT, int BATCH>
__global__ __launch_bounds__(kThreads) void ring_fused_vec_kernel(PtrTable bufs, int P, int64_t N,
                                                                  int64_t plen, int64_t n_vec,
                                                                  Div div) {
    using E = Elem<DT>;
    constexpr int V = E::kVec;
    const int64_t vb0 = (int64_t)blockIdx.x * (kThreads * VPT);
    const int64_t vb1 = min(vb0 + (int64_t)(kThreads * VPT), n_vec);
    const Where first = locate(vb0 * V, N, plen, P);
    const Where last = locate(vb1 * V - 1, N, plen, P);

    if (first.part != last.part || first.chunk != last.chunk) {
        // straddles a chunk or partition boundary: every thread folds its own
        // vectors with their own rotation; only a vector that itself crosses
        // a boundary goes element by element
        for (int j = 0; j < VPT; j++) {
            const int64_t v = vb0 + threadIdx.x + (int64_t)j * kThreads;
            if (v >= vb1) continue;
            const Where a = locate(v * V, N, plen, P);
            const Where b = locate(v * V + V - 1, N, plen, P);
            if (a.part == b.part && a.chunk == b.chunk) {
                fold_vec<DT>(bufs, P, v, a.chunk, div);
            } else {
                for (int i = 0; i < V; i++) fold_one<DT>(bufs, P, N, plen, v * V + i, div);
            }
        }
        return;
    }

    const int r = first.chunk;  // every element of this workgroup starts its fold at worker r
    int64_t v[VPT];
    bool ok[VPT];
#pragma unroll
    for (int j = 0; j < VPT; j++) {
        v[j] = vb0 + threadIdx.x + (int64_t)j * kThreads;
        ok[j] = v[j] < vb1;
    }

    float acc[VPT][V];
    {
        const uint4* src = static_cast<const uint4*>(bufs.p[r]);
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
                int w = r + k + kk;
                if (w >= P) w -= P;
                const uint4* src = static_cast<const uint4*>(bufs.p[w]);
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
        uint4* dst = static_cast<uint4*>(bufs.p[w]);
#pragma unroll
        for (int j = 0; j < VPT; j++)
            if (ok[j]) store_stream(dst + v[j], out[j]);
    }
}

template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void ring_fused_elem_kernel(PtrTable bufs, int P, int64_t N,
                                                                   int64_t plen, int64_t e_begin,
                                                                   int64_t e_end, Div div) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t e = e_begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; e < e_end; e += stride)
        fold_one<DT>(bufs, P, N, plen, e, div);
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
    const int64_t vb0 = (int64_t)blockIdx.x * (kThreads * kVecPerThread);
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

}  // namespace
}  // namespace ga

using namespace ga;

extern "C" ga_status ga_ring_allreduce_sim(void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                           ga_op op, int64_t part_elems, ga_ring_mode mode,
                                           ga_ring_stats* st, void* stream) {
    const char* what = "ga_ring_allreduce_sim";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (op != GA_SUM && op != GA_AVG) return fail(GA_EINVAL, "%s: unknown op %d", what, (int)op);
    if (mode != GA_RING_FUSED && mode != GA_RING_STEPWISE)
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
        int64_t bytes = 0;
        for (int64_t p0 = 0; p0 < N; p0 += plen) {
            int64_t n = N - p0 < plen ? N - p0 : plen;
            bytes += 2 * (int64_t)(P - 1) * ceil_div(n, P) * (int64_t)es;
        }
        s.steps = N > 0 ? 2 * (int64_t)(P - 1) : 0;
        s.bytes_sent_per_worker = bytes;
        if (mode == GA_RING_FUSED)
            s.hbm_bytes = (P > 1) ? 2 * (int64_t)P * N * (int64_t)es : 0;
        else
            s.hbm_bytes = 5 * (int64_t)(P - 1) * N * (int64_t)es;
    }

    hipStream_t hs = static_cast<hipStream_t>(stream);
    Div div{op == GA_AVG, (P & (P - 1)) == 0, (float)P, 1.0f / (float)P};
    int64_t launches = 0;

    if (N > 0 && P > 1) {
        const int64_t vblocks = ceil_div(n_vec, kThreads * kVecPerThread);
        if (mode == GA_RING_FUSED) {
            if (vec_ok && n_vec > 0) {
                PtrTable t{};
                for (int i = 0; i < P; i++) t.p[i] = bufs[i];
                const bool wide = P > 8;
                const unsigned blocks = (unsigned)ceil_div(n_vec, (int64_t)kThreads * (wide ? 2 : 1));
                if (dt == GA_F32 && wide)
                    hipLaunchKernelGGL((ring_fused_vec_kernel<GA_F32, 2, 8>), dim3(blocks),
                                       dim3(kThreads), 0, hs, t, P, N, plen, n_vec, div);
                else if (dt == GA_F32)
                    hipLaunchKernelGGL((ring_fused_vec_kernel<GA_F32, 1, 16>), dim3(blocks),
                                       dim3(kThreads), 0, hs, t, P, N, plen, n_vec, div);
                else if (wide)
                    hipLaunchKernelGGL((ring_fused_vec_kernel<GA_BF16, 2, 8>), dim3(blocks),
                                       dim3(kThreads), 0, hs, t, P, N, plen, n_vec, div);
                else
                    hipLaunchKernelGGL((ring_fused_vec_kernel<GA_BF16, 1, 16>), dim3(blocks),
                                       dim3(kThreads), 0, hs, t, P, N, plen, n_vec, div);
                launches++;
                if ((rc = check_launch(what))) return rc;
            }
            const int64_t e0 = (vec_ok && n_vec > 0) ? vec_elems : 0;
            if (e0 < N) {
                PtrTable t{};
                for (int i = 0; i < P; i++) t.p[i] = bufs[i];
                if (dt == GA_F32)
                    hipLaunchKernelGGL(ring_fused_elem_kernel<GA_F32>, dim3(elem_grid(N - e0)),
                                       dim3(kThreads), 0, hs, t, P, N, plen, e0, N, div);
                else
                    hipLaunchKernelGGL(ring_fused_elem_kernel<GA_BF16>, dim3(elem_grid(N - e0)),
                                       dim3(kThreads), 0, hs, t, P, N, plen, e0, N, div);
                launches++;
                if ((rc = check_launch(what))) return rc;
            }
        } else {
            PtrTable t{};
            for (int i = 0; i < P; i++) t.p[i] = bufs[i];
            const int64_t e0 = (vec_ok && n_vec > 0) ? vec_elems : 0;
            for (int phase = 0; phase < 2; phase++) {
                for (int step = 0; step < P - 1; step++) {
                    Step sp{step, phase == 0, phase == 0 && step == P - 2 && op == GA_AVG};
                    if (vec_ok && n_vec > 0) {
                        hipLaunchKernelGGL(ring_step_vec_kernel, dim3((unsigned)vblocks),
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
