// fusion.hip -- Tensor Fusion ("Horovod: Fast and Easy Distributed Deep
// Learning in TensorFlow", section 3.4, Tensor Fusion steps 1-6): the host
// plan that assigns ready tensors to fusion buffers, and one batched copy
// kernel that performs every copy of a pack (step 3) or unpack (step 5).
//
// The copy kernel walks the concatenation of all copies in tiles (8 or
// 16 KiB); a workgroup finds the first copy of its tile by binary search
// over the descriptors' prefix offsets and then copies the pieces of every
// copy that overlaps its tile. Fusion offsets are dense, so a source and its
// destination often differ in alignment modulo 16: the destination side is
// always written with aligned 16-byte stores, and a misaligned source is read
// as two aligned 16-byte loads whose bytes are shifted into place
// (v_alignbyte), so both sides stay on the 128-bit path.
#include "common.hpp"

namespace ga {
namespace {

// Bytes of the concatenation per workgroup: small tiles keep many short
// workgroups in flight, each copying one contiguous piece, which HBM
// streams best; below 8 KiB the binary search per tile dominates. Measured
// (MI355X, pack/unpack of 16 x 178 MB): 32 KiB 0.65 of 8 TB/s, 16 KiB 0.66,
// 8 KiB 0.69-0.70, 4 KiB 0.47; of 8 x 38 MB: 16 KiB best (0.59/0.67).
constexpr int64_t kTileBytesLarge = 8 * 1024;     // copies of 1 GiB or more in all
constexpr int64_t kTileBytesSmall = 16 * 1024;
constexpr int kUnroll = 4;                  // 16-byte vectors in flight per thread

// Bytes of the 8 dwords {a, b} starting at byte offset sh (0..15).
__device__ __forceinline__ uint4 shifted(const uint4& a, const uint4& b, int dw, int by) {
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t r[5];
    // dw (0..3) is uniform over the segment; select the five dwords needed
#pragma unroll
    for (int k = 0; k < 5; k++) {
        uint32_t v = w[k];
        v = dw == 1 ? w[k + 1] : v;
        v = dw == 2 ? w[k + 2] : v;
        v = dw == 3 ? w[k + 3] : v;
        r[k] = v;
    }
    if (by == 0) return make_uint4(r[0], r[1], r[2], r[3]);
    return make_uint4(__builtin_amdgcn_alignbyte(r[1], r[0], by),
                      __builtin_amdgcn_alignbyte(r[2], r[1], by),
                      __builtin_amdgcn_alignbyte(r[3], r[2], by),
                      __builtin_amdgcn_alignbyte(r[4], r[3], by));
}

// Copy bytes [0, nbytes) from s to d with the whole workgroup. nbytes and
// both addresses are multiples of the element size es (2 or 4).
__device__ void copy_segment(const char* __restrict__ s, char* __restrict__ d, int64_t nbytes,
                             int es) {
    // head: elements until the destination is 16-byte aligned
    int64_t head = (16 - ((uintptr_t)d & 15)) & 15;
    if (head > nbytes) head = nbytes;
    for (int64_t o = threadIdx.x * es; o < head; o += kThreads * es) {
        if (es == 4)
            *reinterpret_cast<uint32_t*>(d + o) = *reinterpret_cast<const uint32_t*>(s + o);
        else
            *reinterpret_cast<uint16_t*>(d + o) = *reinterpret_cast<const uint16_t*>(s + o);
    }
    const char* sb = s + head;
    char* db = d + head;
    const int64_t nvec = (nbytes - head) >> 4;
    const int sh = (int)((uintptr_t)sb & 15);
    uint4* dv = reinterpret_cast<uint4*>(db);
    if (sh == 0) {
        const uint4* sv = reinterpret_cast<const uint4*>(sb);
        int64_t v = threadIdx.x;
        for (; v + (kUnroll - 1) * kThreads < nvec; v += kUnroll * kThreads) {
            uint4 t[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; u++) t[u] = sv[v + u * kThreads];
#pragma unroll
            for (int u = 0; u < kUnroll; u++) dv[v + u * kThreads] = t[u];
        }
        for (; v < nvec; v += kThreads) dv[v] = sv[v];
    } else {
        // every 16 needed source bytes lie in two aligned granules, both of
        // which hold at least one byte of the source range
        const uint4* sa = reinterpret_cast<const uint4*>(sb - sh);
        const int dw = sh >> 2, by = sh & 3;
        int64_t v = threadIdx.x;
        for (; v + (kUnroll - 1) * kThreads < nvec; v += kUnroll * kThreads) {
            uint4 lo[kUnroll], hi[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                lo[u] = sa[v + u * kThreads];
                hi[u] = sa[v + u * kThreads + 1];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; u++) dv[v + u * kThreads] = shifted(lo[u], hi[u], dw, by);
        }
        for (; v < nvec; v += kThreads) dv[v] = shifted(sa[v], sa[v + 1], dw, by);
    }
    // tail: the last elements after the final full vector
    const int64_t done = head + (nvec << 4);
    for (int64_t o = done + threadIdx.x * es; o < nbytes; o += kThreads * es) {
        if (es == 4)
            *reinterpret_cast<uint32_t*>(d + o) = *reinterpret_cast<const uint32_t*>(s + o);
        else
            *reinterpret_cast<uint16_t*>(d + o) = *reinterpret_cast<const uint16_t*>(s + o);
    }
}

__global__ __launch_bounds__(kThreads) void fuse_copy_kernel(const ga_copy_desc* __restrict__ desc,
                                                             int64_t n_desc, int64_t total,
                                                             int64_t tile, int es) {
    const int64_t g0 = flat_block() * tile;
    if (g0 >= total) return;                           // past the folded grid's end
    const int64_t g1 = min(g0 + tile, total);
    // last descriptor whose start is <= g0
    int64_t lo = 0, hi = n_desc - 1;
    while (lo < hi) {
        int64_t mid = (lo + hi + 1) >> 1;
        if (desc[mid].start <= g0) lo = mid; else hi = mid - 1;
    }
    for (int64_t k = lo; k < n_desc; k++) {
        const ga_copy_desc dk = desc[k];
        if (dk.start >= g1) break;
        int64_t a = max(g0, dk.start) - dk.start;
        int64_t b = min(g1, dk.start + dk.n) - dk.start;
        if (a >= b) continue;
        copy_segment(static_cast<const char*>(dk.src) + a * es, static_cast<char*>(dk.dst) + a * es,
                     (b - a) * es, es);
    }
}

ga_status launch_copy(const ga_copy_desc* d_desc, int64_t n_desc, int64_t total, ga_dtype dt,
                      void* stream, const char* what) {
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (n_desc < 0 || total < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (n_desc == 0 || total == 0) return GA_OK;
    if (!d_desc || !aligned(d_desc, 8)) return fail(GA_EINVAL, "%s: bad descriptor table", what);
    const int es = (int)elem_size(dt);
    const int64_t tile = (total * es >= ((int64_t)1 << 30) ? kTileBytesLarge : kTileBytesSmall) / es;
    const int64_t blocks = ceil_div(total, tile);
    if (!flat_fits(blocks)) return fail(GA_EINVAL, "%s: too many elements", what);
    hipLaunchKernelGGL(fuse_copy_kernel, flat_grid(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), d_desc, n_desc, total, tile, es);
    return check_launch(what);
}

}  // namespace
}  // namespace ga

using namespace ga;

extern "C" ga_status ga_fuse_plan(const int64_t* n_elems, const int32_t* dtype_of, int32_t T,
                                  int64_t cap_bytes, int32_t* buf_of, int64_t* off_of,
                                  int64_t* fill, int32_t* buf_dtype, int32_t* n_buf) {
    const char* what = "ga_fuse_plan";
    if (T < 0 || cap_bytes <= 0) return fail(GA_EINVAL, "%s: bad T or capacity", what);
    if (!n_buf || (T > 0 && (!n_elems || !buf_of || !off_of || !fill)))
        return fail(GA_EINVAL, "%s: null argument", what);
    int32_t nb = 0;        // buffers opened so far
    int32_t open = -1;     // buffer accepting tensors, -1 if none
    int32_t open_dt = -1;
    int64_t open_bytes = 0;
    for (int32_t t = 0; t < T; t++) {
        const int32_t dt = dtype_of ? dtype_of[t] : GA_F32;
        if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: tensor %d has unknown dtype", what, t);
        if (n_elems[t] < 0) return fail(GA_EINVAL, "%s: tensor %d has negative size", what, t);
        const int64_t bytes = n_elems[t] * (int64_t)elem_size((ga_dtype)dt);
        if (bytes > cap_bytes) {            // larger than the buffer: reduced alone
            fill[nb] = n_elems[t];
            if (buf_dtype) buf_dtype[nb] = dt;
            buf_of[t] = nb;
            off_of[t] = 0;
            nb++;
            open = -1;
            continue;
        }
        if (open < 0 || open_dt != dt || open_bytes + bytes > cap_bytes) {
            open = nb++;
            open_dt = dt;
            open_bytes = 0;
            fill[open] = 0;
            if (buf_dtype) buf_dtype[open] = dt;
        }
        buf_of[t] = open;
        off_of[t] = fill[open];
        fill[open] += n_elems[t];
        open_bytes += bytes;
    }
    *n_buf = nb;
    return GA_OK;
}

extern "C" ga_status ga_fuse_desc_check(const ga_copy_desc* h_desc, int64_t n_desc, ga_dtype dt,
                                        int64_t* total_elems) {
    const char* what = "ga_fuse_desc_check";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (n_desc < 0 || (n_desc > 0 && !h_desc) || !total_elems)
        return fail(GA_EINVAL, "%s: bad table", what);
    const size_t es = elem_size(dt);
    int64_t acc = 0;
    for (int64_t k = 0; k < n_desc; k++) {
        const ga_copy_desc& d = h_desc[k];
        if (d.n < 0) return fail(GA_EINVAL, "%s: copy %lld has negative size", what, (long long)k);
        if (d.start != acc)
            return fail(GA_EINVAL, "%s: copy %lld starts at %lld, expected %lld", what, (long long)k,
                        (long long)d.start, (long long)acc);
        if (d.n > 0 && (!d.src || !d.dst || !aligned(d.src, es) || !aligned(d.dst, es)))
            return fail(GA_EINVAL, "%s: copy %lld has a null or misaligned pointer", what,
                        (long long)k);
        acc += d.n;
    }
    *total_elems = acc;
    return GA_OK;
}

extern "C" ga_status ga_fuse_pack(const ga_copy_desc* d_desc, int64_t n_desc, int64_t total_elems,
                                  ga_dtype dt, void* stream) {
    return launch_copy(d_desc, n_desc, total_elems, dt, stream, "ga_fuse_pack");
}

extern "C" ga_status ga_fuse_unpack(const ga_copy_desc* d_desc, int64_t n_desc,
                                    int64_t total_elems, ga_dtype dt, void* stream) {
    return launch_copy(d_desc, n_desc, total_elems, dt, stream, "ga_fuse_unpack");
}
