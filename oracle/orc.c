/*
 * orc.c -- the oracle: a plain, slow, single-threaded CPU implementation of
 * the data-parallel gradient-aggregation path (ring all-reduce over P
 * simulated workers, THC uniform stochastic quantization, integer
 * aggregation, dequantization, NMSE).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * bench's cpu_baseline leg may load this library. The product path (the HIP
 * library under gradient_all_reduce_worker_amd/csrc) never calls it, and the
 * two share no source: not a header, not a helper, not a constant table.
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * With contraction off and SSE arithmetic (x86-64), every float expression
 * below is evaluated as separate IEEE-754 binary32 operations, rounded to
 * nearest-even, in exactly the order written.
 *
 * Page citations name the page title and the section on it:
 *   [HVD]  "Horovod: Fast and Easy Distributed Deep Learning in TensorFlow"
 *          (paper summary page), section 3.4.
 *   [THC]  "THC: Accelerating Distributed Deep Learning Using Tensor
 *          Homomorphic Compression", sections 2-4 and 8.
 *   [RING] systemcraft lesson "Collective Communication: Ring All-Reduce",
 *          sections 4, 5 and 7.
 * Readings of what the pages leave open are listed where they are used.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_SUM 0
#define ORC_AVG 1

/* ------------------------------------------------------------------ */
/* Element access. bf16 is the top half of a binary32 bit pattern.     */
/* ------------------------------------------------------------------ */

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to bfloat16, round-to-nearest, ties-to-even, by
 * looking at the 16 bits that are dropped: above half -> round up, exactly
 * half -> round up only if the kept part is odd. */
static uint16_t float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

static float load_elem(const void *buf, int dt, int64_t e)
{
    if (dt == ORC_BF16)
        return bf16_to_float(((const uint16_t *)buf)[e]);
    return ((const float *)buf)[e];
}

static void store_elem(void *buf, int dt, int64_t e, float v)
{
    if (dt == ORC_BF16)
        ((uint16_t *)buf)[e] = float_to_bf16(v);
    else
        ((float *)buf)[e] = v;
}

void orc_f32_to_bf16(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = float_to_bf16(x[i]);
}

void orc_bf16_to_f32(const uint16_t *x, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = bf16_to_float(x[i]);
}

/* Partition p covers elements [p*part, min((p+1)*part, N)); part <= 0 means
 * the whole vector is one partition. */
static int64_t part_len(int64_t N, int64_t part)
{
    return part > 0 ? part : N;
}

static int mod_p(int64_t a, int P)
{
    int64_t r = a % P;
    return (int)(r < 0 ? r + P : r);
}

/* ------------------------------------------------------------------ */
/* Ring all-reduce                                                     */
/* ------------------------------------------------------------------ */

/*
 * orc_ring_fold: the value the ring schedule leaves in every buffer, written
 * out element by element.
 *
 * [HVD] 3.4 "The Ring-Allreduce Algorithm" and [RING] section 4: the buffer
 * is cut into P chunks; during scatter-reduce the partial sum of chunk c
 * travels around the ring once, and every worker it passes adds its own copy
 * of the chunk; during all-gather the finished chunk overwrites every other
 * worker's copy. [RING] section 7 fixes the schedule: at step s worker i sends
 * chunk (i - s) mod P and receives chunk (i - s - 1) mod P from worker i - 1.
 * Hence chunk c starts at worker c and is then extended by workers
 * c+1, c+2, ..., c+P-1 (mod P), in that order.
 *
 * Readings: chunk size C = ceil(n / P) with short or empty trailing chunks
 * (the pages assume P divides n); average = one binary32 division of the
 * finished sum by P ([HVD] "dividing element-wise by N"); bf16 inputs are
 * widened exactly, partial sums stay binary32 across all hops and are rounded
 * to bf16 once at the end.
 */
int orc_ring_fold(void *const *bufs, int P, int64_t N, int dt, int op, int64_t part)
{
    if (P < 1 || N < 0)
        return -1;
    int64_t plen = part_len(N, part);
    for (int64_t p0 = 0; p0 < N; p0 += plen) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        int64_t C = (n + P - 1) / P;
        for (int64_t e = p0; e < p0 + n; e++) {
            int c = (int)((e - p0) / C);
            float acc = load_elem(bufs[c], dt, e);
            for (int k = 1; k < P; k++)
                acc = acc + load_elem(bufs[(c + k) % P], dt, e);
            if (op == ORC_AVG)
                acc = acc / (float)P;
            for (int w = 0; w < P; w++)
                store_elem(bufs[w], dt, e, acc);
        }
    }
    return 0;
}

/*
 * One communication step of one ring direction on binary32 working copies,
 * stated from the chunk-owner rule of [RING] sections 4 and 7: at step
 * `shift` worker i holds the running partial (scatter-reduce) or the
 * finished value (all-gather) of ring chunk (i - dir * shift) mod P, and
 * hands it to worker i + dir. Chunk k of the direction is index base + k of
 * the partition's chunks of length C (the last ones short or empty). All P
 * transfers of a step happen at once, so every worker first copies out what
 * it sends; then each receiver adds it in (reduce) or overwrites its copy.
 */
static void ring_step(float **work, float **send, int P, int dir, int base, int64_t C, int64_t n,
                      int shift, int reduce)
{
    for (int i = 0; i < P; i++) {
        int64_t k = base + mod_p(i - (int64_t)dir * shift, P);
        int64_t lo = k * C < n ? k * C : n, hi = (k + 1) * C < n ? (k + 1) * C : n;
        memcpy(send[i], work[i] + lo, (size_t)(hi - lo) * sizeof(float));
    }
    for (int i = 0; i < P; i++) {
        int j = mod_p(i + dir, P);                       /* the receiver */
        int64_t k = base + mod_p(i - (int64_t)dir * shift, P);
        int64_t lo = k * C < n ? k * C : n, hi = (k + 1) * C < n ? (k + 1) * C : n;
        for (int64_t t = lo; t < hi; t++)
            work[j][t] = reduce ? work[j][t] + send[i][t - lo] : send[i][t - lo];
    }
}

/*
 * orc_ring_stepwise: the ring's 2(P-1) communication steps of [RING]
 * section 7 executed one by one on binary32 working copies of every
 * worker's partition: P - 1 scatter-reduce steps (ring_step with shift s,
 * the partial of chunk c growing by one worker per step from worker c on),
 * then P - 1 all-gather steps (shift s - 1: the worker that finished chunk
 * c passes it on, and each receiver overwrites its copy). With op = avg
 * every worker divides its buffer by P at the end ([HVD] 3.4).
 * rs_only != 0 stops after scatter-reduce and stores the binary32 partial
 * state back (fp32 buffers only), so the state after the first phase can be
 * inspected.
 */
int orc_ring_stepwise(void *const *bufs, int P, int64_t N, int dt, int op, int64_t part,
                      int rs_only)
{
    if (P < 1 || N < 0 || (rs_only && dt != ORC_F32))
        return -1;
    int64_t plen = part_len(N, part);
    float **work = (float **)calloc((size_t)P, sizeof(float *));
    float **send = (float **)calloc((size_t)P, sizeof(float *));
    if (!work || !send)
        return -2;
    int rc = 0;
    for (int64_t p0 = 0; p0 < N && rc == 0; p0 += plen) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        int64_t C = (n + P - 1) / P;
        for (int i = 0; i < P; i++) {
            work[i] = (float *)malloc((size_t)n * sizeof(float));
            send[i] = (float *)malloc((size_t)(C > 0 ? C : 1) * sizeof(float));
            if (!work[i] || !send[i])
                rc = -2;
        }
        if (rc == 0) {
            for (int i = 0; i < P; i++)
                for (int64_t t = 0; t < n; t++)
                    work[i][t] = load_elem(bufs[i], dt, p0 + t);
            for (int s = 0; s < P - 1; s++)
                ring_step(work, send, P, +1, 0, C, n, s, 1);
            if (!rs_only) {
                for (int s = 0; s < P - 1; s++)
                    ring_step(work, send, P, +1, 0, C, n, s - 1, 0);
                if (op == ORC_AVG)
                    for (int i = 0; i < P; i++)
                        for (int64_t t = 0; t < n; t++)
                            work[i][t] = work[i][t] / (float)P;
            }
            for (int i = 0; i < P; i++)
                for (int64_t t = 0; t < n; t++)
                    store_elem(bufs[i], dt, p0 + t, work[i][t]);
        }
        for (int i = 0; i < P; i++) {
            free(work[i]);
            free(send[i]);
            work[i] = send[i] = NULL;
        }
    }
    free(work);
    free(send);
    return rc;
}

/*
 * Bidirectional ring ([RING] section 11, Exercise 1 and its worked solution):
 * a partition is cut into 2P sub-chunks; sub-chunks 0 .. P-1 travel a
 * clockwise ring (worker i sends to i + 1) and sub-chunks P .. 2P-1 a
 * counter-clockwise ring (worker i sends to i - 1), both at once. Every
 * ring runs the schedule of section 7 in its own direction: at
 * scatter-reduce step s worker i passes its partial of ring sub-chunk
 * (i - dir s) mod P on, and the neighbour adds its own copy; so a clockwise
 * sub-chunk c is folded x_c, x_{c+1}, ..., x_{c-1} and a counter-clockwise
 * one x_c, x_{c-1}, ..., x_{c+1}.
 *
 * Readings: sub-chunk size C2 = ceil(n / (2P)) with short or empty trailing
 * sub-chunks (the page assumes 2P divides n); average, bf16 and partitions
 * as for the single ring.
 */
int orc_dual_ring_fold(void *const *bufs, int P, int64_t N, int dt, int op, int64_t part)
{
    if (P < 1 || N < 0)
        return -1;
    int64_t plen = part_len(N, part);
    for (int64_t p0 = 0; p0 < N; p0 += plen) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        int64_t C2 = (n + 2 * P - 1) / (2 * P);
        for (int64_t e = p0; e < p0 + n; e++) {
            int k = (int)((e - p0) / C2);
            int dir = k < P ? 1 : -1;
            int c = k < P ? k : k - P;
            float acc = load_elem(bufs[c], dt, e);
            for (int j = 1; j < P; j++)
                acc = acc + load_elem(bufs[mod_p(c + dir * j, P)], dt, e);
            if (op == ORC_AVG)
                acc = acc / (float)P;
            for (int w = 0; w < P; w++)
                store_elem(bufs[w], dt, e, acc);
        }
    }
    return 0;
}

/*
 * orc_dual_ring_stepwise: the steps of the bidirectional ring one by one,
 * P - 1 scatter-reduce steps then P - 1 all-gather steps, both directions
 * in every step (ring_step over sub-chunks of C2; the counter-clockwise
 * ring's chunks are sub-chunks P .. 2P - 1).
 * Scatter-reduce step s moves sub-chunk (i - dir s) of worker i; all-gather
 * step s moves (i - dir (s - 1)), the finished one. avg divides at the end.
 */
int orc_dual_ring_stepwise(void *const *bufs, int P, int64_t N, int dt, int op, int64_t part)
{
    if (P < 1 || N < 0)
        return -1;
    int64_t plen = part_len(N, part);
    float **work = (float **)calloc((size_t)P, sizeof(float *));
    float **send = (float **)calloc((size_t)P, sizeof(float *));
    if (!work || !send)
        return -2;
    int rc = 0;
    for (int64_t p0 = 0; p0 < N && rc == 0; p0 += plen) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        int64_t C2 = (n + 2 * P - 1) / (2 * P);
        for (int i = 0; i < P; i++) {
            work[i] = (float *)malloc((size_t)n * sizeof(float));
            send[i] = (float *)malloc((size_t)(C2 > 0 ? C2 : 1) * sizeof(float));
            if (!work[i] || !send[i])
                rc = -2;
        }
        if (rc == 0) {
            for (int i = 0; i < P; i++)
                for (int64_t t = 0; t < n; t++)
                    work[i][t] = load_elem(bufs[i], dt, p0 + t);
            for (int s = 0; s < P - 1; s++) {
                ring_step(work, send, P, +1, 0, C2, n, s, 1);
                ring_step(work, send, P, -1, P, C2, n, s, 1);
            }
            for (int s = 0; s < P - 1; s++) {
                ring_step(work, send, P, +1, 0, C2, n, s - 1, 0);
                ring_step(work, send, P, -1, P, C2, n, s - 1, 0);
            }
            if (op == ORC_AVG)
                for (int i = 0; i < P; i++)
                    for (int64_t t = 0; t < n; t++)
                        work[i][t] = work[i][t] / (float)P;
            for (int i = 0; i < P; i++)
                for (int64_t t = 0; t < n; t++)
                    store_elem(bufs[i], dt, p0 + t, work[i][t]);
        }
        for (int i = 0; i < P; i++) {
            free(work[i]);
            free(send[i]);
            work[i] = send[i] = NULL;
        }
    }
    free(work);
    free(send);
    return rc;
}

/*
 * Communication accounting as the [RING] section 7 simulator keeps it: each
 * of the 2(P-1) steps sends one chunk of C elements per worker, so a worker
 * sends 2(P-1) * C * elem_bytes per partition ([HVD] 3.4: 2 (N-1)/N * K).
 * Partitions run their rings side by side, so the step count is per ring.
 */
void orc_ring_stats(int P, int64_t N, int64_t part, int elem_bytes, int64_t *steps,
                    int64_t *bytes_per_worker)
{
    int64_t plen = part_len(N, part);
    int64_t bytes = 0;
    for (int64_t p0 = 0; p0 < N; p0 += plen) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        int64_t C = (n + P - 1) / P;
        bytes += 2 * (int64_t)(P - 1) * C * elem_bytes;
    }
    *steps = N > 0 ? 2 * (int64_t)(P - 1) : 0;
    *bytes_per_worker = bytes;
}

/* ------------------------------------------------------------------ */
/* THC preliminary stage: global extremes                              */
/* ------------------------------------------------------------------ */

/*
 * [THC] section 3, Algorithm 1 preliminary round: every worker reports its
 * smallest and largest entry and the parameter server keeps the global
 * extremes. Reading: one [m, M] grid per partition (the 4 MB partitions of
 * [THC] section 2), taken over all P workers' elements of that partition.
 * Both ends are canonicalised with "+ 0.0f" so that -0 becomes +0.
 * Output mM[2*p] = m, mM[2*p+1] = M.
 */
int orc_minmax(const void *const *bufs, int P, int64_t N, int dt, int64_t part, float *mM)
{
    if (P < 1 || N < 0)
        return -1;
    int64_t plen = part_len(N, part);
    int64_t p = 0;
    for (int64_t p0 = 0; p0 < N; p0 += plen, p++) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        float m = load_elem(bufs[0], dt, p0);
        float M = m;
        for (int i = 0; i < P; i++)
            for (int64_t e = p0; e < p0 + n; e++) {
                float v = load_elem(bufs[i], dt, e);
                if (v < m)
                    m = v;
                if (v > M)
                    M = v;
            }
        mM[2 * p] = m + 0.0f;
        mM[2 * p + 1] = M + 0.0f;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 counter-based generator                               */
/* ------------------------------------------------------------------ */

/*
 * Philox4x32 with 10 rounds, from its published definition: J. K. Salmon,
 * M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3", SC'11, section 3.2. One round multiplies words 0 and 2 of the
 * counter by the two Philox multipliers, and builds the next counter from the
 * high product halves XORed with the other two words and the round key, and
 * the low product halves. The round key starts at the user key and is
 * advanced by the two Weyl constants before every round after the first.
 */
static void mul32_hilo(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo)
{
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t MULT_A = 0xD2511F53u, MULT_B = 0xCD9E8D57u;
    const uint32_t WEYL_A = 0x9E3779B9u, WEYL_B = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k0 += WEYL_A;
            k1 += WEYL_B;
        }
        uint32_t hiA, loA, hiB, loB;
        mul32_hilo(MULT_A, x0, &hiA, &loA);
        mul32_hilo(MULT_B, x2, &hiB, &loB);
        uint32_t y0 = hiB ^ x1 ^ k0;
        uint32_t y1 = loB;
        uint32_t y2 = hiA ^ x3 ^ k1;
        uint32_t y3 = loA;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/*
 * The 16-bit uniform for element e of worker w: Philox is called on the
 * counter (g mod 2^32, g >> 32, w, 0) with key (seed mod 2^32, seed >> 32),
 * where g = floor(e / 8); element e takes half (e mod 2) of output word
 * (e mod 8) / 2, low half first. One call thus serves 8 consecutive elements.
 */
static uint32_t uniform16(uint64_t seed, int worker, int64_t e)
{
    uint64_t g = (uint64_t)e >> 3;
    int j = (int)(e & 7);
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)worker, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return (out[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
}

uint32_t orc_uniform16(uint64_t seed, int worker, int64_t e)
{
    return uniform16(seed, worker, e);
}

/* ------------------------------------------------------------------ */
/* THC uniform stochastic quantization                                 */
/* ------------------------------------------------------------------ */

/*
 * orc_usq_quantize: one worker's vector -> b-bit grid indices, packed.
 *
 * [THC] section 3: the 2^b quantization values are spaced uniformly on the
 * global range, q_k = m + k (M - m) / (2^b - 1); stochastic quantization
 * sends the lower neighbour q0 of a with probability (q1 - a)/(q1 - q0) and
 * the upper one q1 otherwise, which makes the result unbiased. The worker
 * sends the index k.
 *
 * Steps, all binary32 (L = 2^b - 1):
 *   range = M - m; if range == 0 every index is 0;
 *   s = L / range;  u = (a - m) * s   (position on the grid, in steps);
 *   z0 = min(floor(u), L - 1);  f = u - z0   (exact: f is the fraction);
 *   go up with probability f: up = (2 r + 1) < f * 2^17 with r the 16-bit
 *   uniform of the element (so P(up) differs from f by at most 2^-17);
 *   z = z0 + up.
 * Packing: element e occupies bits [(e b) mod 8, (e b) mod 8 + b) of byte
 * floor(e b / 8), least significant bits first; unused bits are zero.
 * worker is the worker id keying the generator (counter word 2); e_offset is
 * the index of x[0] in the worker's whole vector (0 for a whole vector; the
 * start of a partition when one partition is quantized on its own), so the
 * generator is keyed by global element indices either way.
 */
int orc_usq_quantize(const void *x, int64_t N, int dt, int worker, int64_t part, const float *mM,
                     int b, uint64_t seed, int64_t e_offset, uint8_t *packed)
{
    if (!(b == 1 || b == 2 || b == 4 || b == 8) || N < 0)
        return -1;
    const int L = (1 << b) - 1;
    int64_t nbytes = (N * b + 7) / 8;
    memset(packed, 0, (size_t)nbytes);
    int64_t plen = part_len(N, part);
    int64_t p = 0;
    for (int64_t p0 = 0; p0 < N; p0 += plen, p++) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        float m = mM[2 * p], M = mM[2 * p + 1];
        float range = M - m;
        float s = (range == 0.0f) ? 0.0f : (float)L / range;
        for (int64_t e = p0; e < p0 + n; e++) {
            uint32_t z = 0;
            if (range != 0.0f) {
                float a = load_elem(x, dt, e);
                float u = (a - m) * s;
                float z0 = floorf(u);
                if (z0 > (float)(L - 1))
                    z0 = (float)(L - 1);
                float f = u - z0;
                uint32_t r = uniform16(seed, worker, e_offset + e);
                int up = (float)(2u * r + 1u) < f * 131072.0f;
                z = (uint32_t)z0 + (uint32_t)up;
            }
            int64_t bit = e * b;
            packed[bit >> 3] |= (uint8_t)(z << (bit & 7));
        }
    }
    return 0;
}

/* Unpacked view of one packed index (used by the aggregate and the tests). */
int orc_unpack_indices(const uint8_t *packed, int64_t N, int b, int32_t *z)
{
    if (!(b == 1 || b == 2 || b == 4 || b == 8))
        return -1;
    const int L = (1 << b) - 1;
    for (int64_t e = 0; e < N; e++) {
        int64_t bit = e * b;
        z[e] = (packed[bit >> 3] >> (bit & 7)) & L;
    }
    return 0;
}

/*
 * [THC] section 3, Algorithm 1 (server side) and section 4: the server only
 * adds the workers' index vectors, coordinate by coordinate: S[e] = sum_i
 * z_i[e], in int32 (exact; at most P (2^b - 1), see [THC] section 8 on the
 * width of the aggregate).
 */
int orc_int_aggregate(const uint8_t *const *packed, int P, int64_t N, int b, int32_t *S)
{
    if (!(b == 1 || b == 2 || b == 4 || b == 8) || P < 1)
        return -1;
    const int L = (1 << b) - 1;
    for (int64_t e = 0; e < N; e++) {
        int64_t bit = e * b;
        int32_t acc = 0;
        for (int i = 0; i < P; i++)
            acc += (packed[i][bit >> 3] >> (bit & 7)) & L;
        S[e] = acc;
    }
    return 0;
}

/*
 * [THC] section 3, Algorithm 1 (last step) and section 4 (divide the sum by
 * the number of workers n, then invert the linear map onto the grid):
 *   delta = range / L;  xhat = m + ((float)S / (float)P) * delta,
 * all binary32; range == 0 gives xhat = m. out_dt = bf16 rounds the final
 * value to nearest-even.
 */
static int dequant_levels(const int32_t *S, int64_t N, int P, int L, int64_t part, const float *mM,
                          void *out, int out_dt)
{
    int64_t plen = part_len(N, part);
    int64_t p = 0;
    for (int64_t p0 = 0; p0 < N; p0 += plen, p++) {
        int64_t n = (N - p0 < plen) ? N - p0 : plen;
        float m = mM[2 * p], M = mM[2 * p + 1];
        float range = M - m;
        float delta = range / (float)L;
        for (int64_t e = p0; e < p0 + n; e++) {
            float v = m;
            if (range != 0.0f) {
                float avg_index = (float)S[e] / (float)P;
                v = m + avg_index * delta;
            }
            store_elem(out, out_dt, e, v);
        }
    }
    return 0;
}

int orc_dequant(const int32_t *S, int64_t N, int P, int b, int64_t part, const float *mM, void *out,
                int out_dt)
{
    if (!(b == 1 || b == 2 || b == 4 || b == 8) || P < 1)
        return -1;
    return dequant_levels(S, N, P, (1 << b) - 1, part, mM, out, out_dt);
}

/* ------------------------------------------------------------------ */
/* Non-uniform THC (lookup table)                                      */
/* ------------------------------------------------------------------ */

/*
 * [THC] section 4, Algorithm 2. A table T maps the 2^b indices a worker may
 * send into the larger integer range <g+1> = {0, ..., g}, with
 * 0 = T[0] < T[1] < ... < T[2^b - 1] = g (granularity g >= 2^b - 1). Index z
 * stands for the value m + T[z] (M - m) / g. Reading: the page's prose
 * writes (M - m)/(g + 1) but its own worked example (T2 = {0, 1, 3, 4},
 * g = 4 on [-1, 1], T2[1] -> -1/2) divides by g; this build divides by g.
 *
 * A worker rounds each coordinate stochastically to one of the two
 * neighbouring table values (unbiased), binary32 throughout:
 *   range = M - m (0: every index 0);  s = g / range;  u = (a - m) s;
 *   k = min(floor(u), g - 1);  z0 = the largest z with T[z] <= k
 *   (at most 2^b - 2, since T[2^b - 1] = g > k);  lo = T[z0], hi = T[z0 + 1];
 *   f = (u - lo) / (hi - lo);  up = (2 r + 1) < f 2^17;  z = z0 + up,
 * with the same 16-bit uniforms and packing as the uniform quantizer. With
 * g = 2^b - 1 and T the identity this is exactly orc_usq_quantize.
 */
static int table_ok(int b, int g, const int32_t *T)
{
    int n = 1 << b;
    if (!(b == 1 || b == 2 || b == 4 || b == 8) || g < n - 1 || T[0] != 0 || T[n - 1] != g)
        return 0;
    for (int z = 1; z < n; z++)
        if (T[z] <= T[z - 1])
            return 0;
    return 1;
}

int orc_nuhc_quantize(const void *x, int64_t N, int dt, int worker, int64_t part, const float *mM,
                      int b, int g, const int32_t *T, uint64_t seed, int64_t e_offset,
                      uint8_t *packed)
{
    if (!table_ok(b, g, T) || N < 0)
        return -1;
    const int n = 1 << b;
    int64_t nbytes = (N * b + 7) / 8;
    memset(packed, 0, (size_t)nbytes);
    int64_t plen = part_len(N, part);
    int64_t p = 0;
    for (int64_t p0 = 0; p0 < N; p0 += plen, p++) {
        int64_t len = (N - p0 < plen) ? N - p0 : plen;
        float m = mM[2 * p], M = mM[2 * p + 1];
        float range = M - m;
        float s = (range == 0.0f) ? 0.0f : (float)g / range;
        for (int64_t e = p0; e < p0 + len; e++) {
            uint32_t z = 0;
            if (range != 0.0f) {
                float a = load_elem(x, dt, e);
                float u = (a - m) * s;
                float k = floorf(u);
                if (k > (float)(g - 1))
                    k = (float)(g - 1);
                int z0 = 0;
                for (int t = 1; t < n; t++)
                    if ((float)T[t] <= k)
                        z0 = t;
                float lo = (float)T[z0], hi = (float)T[z0 + 1];
                float f = (u - lo) / (hi - lo);
                uint32_t r = uniform16(seed, worker, e_offset + e);
                int up = (float)(2u * r + 1u) < f * 131072.0f;
                z = (uint32_t)z0 + (uint32_t)up;
            }
            int64_t bit = e * b;
            packed[bit >> 3] |= (uint8_t)(z << (bit & 7));
        }
    }
    return 0;
}

/* [THC] section 4, Algorithm 2 (server): look every index up in T and add:
 * Y[e] = sum_i T[z_i[e]] (int32, at most P g). */
int orc_nuhc_aggregate(const uint8_t *const *packed, int P, int64_t N, int b, int g,
                       const int32_t *T, int32_t *Y)
{
    if (!table_ok(b, g, T) || P < 1)
        return -1;
    const int L = (1 << b) - 1;
    for (int64_t e = 0; e < N; e++) {
        int64_t bit = e * b;
        int32_t acc = 0;
        for (int i = 0; i < P; i++)
            acc += T[(packed[i][bit >> 3] >> (bit & 7)) & L];
        Y[e] = acc;
    }
    return 0;
}

/* [THC] section 4, Algorithm 2 (worker, last two steps): divide Y by n and
 * map back: xhat = m + ((float)Y / P) (range / g), binary32. */
int orc_nuhc_dequant(const int32_t *Y, int64_t N, int P, int g, int64_t part, const float *mM,
                     void *out, int out_dt)
{
    if (g < 1 || P < 1)
        return -1;
    return dequant_levels(Y, N, P, g, part, mM, out, out_dt);
}

/* ------------------------------------------------------------------ */
/* Randomized Hadamard Transform pre/post-processing                   */
/* ------------------------------------------------------------------ */

/*
 * [THC] section 5: RHT(x) = (1/sqrt(d)) H D x and RHT^-1(y) = (1/sqrt(d)) D H y
 * with H the d x d Hadamard matrix and D a diagonal of independent +-1
 * (Rademacher) signs, applied here to every block of d = 2^k consecutive
 * coordinates (the block is the quantizer's partition).
 *
 * Readings: D is shared by all workers (the transform must be the same
 * linear map for the sum of transformed vectors to invert), drawn from
 * Philox4x32-10 with key (seed mod 2^32, seed >> 32) and counter
 * (q mod 2^32, q >> 32, 0x52485400, 0), q = e / 128: coordinate e takes bit
 * (e mod 32) of output word (e / 32) mod 4, and a set bit means -1. H x is
 * the textbook in-place transform: for s = 0, 1, ..., k-1, every pair
 * (i, i + 2^s) with bit s of i clear becomes (x_i + x_j, x_i - x_j); all in
 * binary32, the scaling by fl32(1/sqrt(d)) after the last stage. The
 * quantizer's integer decisions depend on these values, so the transform
 * runs in the kernels' precision (binary32); its accuracy against the exact
 * transform is pinned separately.
 */
static float rademacher(uint64_t seed, int64_t e)
{
    uint64_t q = (uint64_t)e >> 7;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), 0x52485400u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    uint32_t bit = (out[(e >> 5) & 3] >> (e & 31)) & 1u;
    return bit ? -1.0f : 1.0f;
}

void orc_rademacher(uint64_t seed, int64_t e0, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = rademacher(seed, e0 + i);
}

static void fwht_block(float *v, int64_t d)
{
    for (int64_t h = 1; h < d; h <<= 1)
        for (int64_t i = 0; i < d; i++)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

static int pow2_ok(int64_t d)
{
    return d >= 2 && (d & (d - 1)) == 0;
}

/* y[e] for e in [0, ceil(N/d) d): a vector whose length is not a multiple
 * of d is zero-padded to one; x fp32 or bf16, y fp32. e0 is the index of
 * x[0] in the whole vector (a multiple of d), which selects the signs, so a
 * run of blocks can be transformed on its own. */
int orc_rht_forward(const void *x, int dt, int64_t N, int64_t d, uint64_t seed, int64_t e0,
                    float *y)
{
    if (!pow2_ok(d) || N < 0 || e0 < 0 || e0 % d)
        return -1;
    const float c = (float)(1.0 / sqrt((double)d));
    const int64_t Np = (N + d - 1) / d * d;
    for (int64_t b0 = 0; b0 < Np; b0 += d) {
        for (int64_t i = 0; i < d; i++)
            y[b0 + i] = rademacher(seed, e0 + b0 + i) * (b0 + i < N ? load_elem(x, dt, b0 + i) : 0.0f);
        fwht_block(y + b0, d);
        for (int64_t i = 0; i < d; i++)
            y[b0 + i] = y[b0 + i] * c;
    }
    return 0;
}

/* out[e] = (1/sqrt(d)) D H y, binary32, rounded to bf16 if asked; e0 as
 * for the forward transform. */
int orc_rht_inverse(const float *y, int64_t N, int64_t d, uint64_t seed, int64_t e0, void *out,
                    int out_dt)
{
    if (!pow2_ok(d) || N % d || e0 < 0 || e0 % d)
        return -1;
    const float c = (float)(1.0 / sqrt((double)d));
    float *v = (float *)malloc((size_t)d * sizeof(float));
    if (!v)
        return -2;
    for (int64_t b0 = 0; b0 < N; b0 += d) {
        memcpy(v, y + b0, (size_t)d * sizeof(float));
        fwht_block(v, d);
        for (int64_t i = 0; i < d; i++)
            store_elem(out, out_dt, b0 + i, rademacher(seed, e0 + b0 + i) * (v[i] * c));
    }
    free(v);
    return 0;
}

/*
 * [THC] section 5, norm-based range: every worker computes the norm of each
 * of its blocks; the range of block p is M = (t_p / sqrt(d)) * l_p, m = -M,
 * with l_p the largest norm among the workers. Reading: the page writes
 * "l = max ||x_i||^2"; only the norm itself (not its square) has the units
 * of M, so l is the norm. Sums of squares in binary64 (the squares of
 * binary32 values are exact there), in index order; M rounded once to
 * binary32 from binary64 t_p sqrt(max sum) / sqrt(d).
 */
int orc_rht_sumsq(const void *x, int dt, int64_t N, int64_t d, double *sumsq)
{
    if (!pow2_ok(d) || N < 0)
        return -1;
    for (int64_t b0 = 0, p = 0; b0 < N; b0 += d, p++) {
        double acc = 0.0;
        for (int64_t i = 0; i < d && b0 + i < N; i++) {
            double v = (double)load_elem(x, dt, b0 + i);
            acc += v * v;
        }
        sumsq[p] = acc;
    }
    return 0;
}

int orc_rht_range(const double *sumsq, int P, int64_t nblk, int64_t d, double t_p, float *mM)
{
    if (P < 1 || !pow2_ok(d))
        return -1;
    for (int64_t p = 0; p < nblk; p++) {
        double mx = 0.0;
        for (int i = 0; i < P; i++)
            if (sumsq[(int64_t)i * nblk + p] > mx)
                mx = sumsq[(int64_t)i * nblk + p];
        float M = (float)(t_p * sqrt(mx) / sqrt((double)d));
        mM[2 * p] = -M;
        mM[2 * p + 1] = M;
    }
    return 0;
}

/* [THC] section 5, truncation: coordinates beyond the range are rounded to
 * its ends. */
void orc_clamp(float *y, int64_t N, int64_t d, const float *mM)
{
    for (int64_t e = 0; e < N; e++) {
        int64_t p = e / d;
        if (y[e] < mM[2 * p])
            y[e] = mM[2 * p];
        if (y[e] > mM[2 * p + 1])
            y[e] = mM[2 * p + 1];
    }
}

/*
 * [THC] section 5, error feedback: a worker sends x = grad + e, where e is
 * what its earlier rounds lost to compression, and afterwards keeps the new
 * loss e' = x - xhat, xhat being the value its own indices stand for.
 *
 * Readings: xhat is the worker's own dequantized vector (its indices alone,
 * mapped back as the server's average is with one worker:
 * m + (float)v * ((M - m) / levels), or m when M == m, with v = z and
 * levels = 2^b - 1 for uniform THC, v = T[z] and levels = g for a table),
 * so e' needs no message from the server; e is binary32, the sum x and the
 * difference e' are single binary32 operations; a bf16 gradient is widened
 * exactly first.
 */
void orc_ef_add(const void *grad, int dt, const float *e, int64_t N, float *x)
{
    for (int64_t i = 0; i < N; i++)
        x[i] = load_elem(grad, dt, i) + e[i];
}

int orc_ef_update(const float *x, const uint8_t *packed, int64_t N, int b, int g, const int32_t *T,
                  int64_t part, const float *mM, float *e_out)
{
    if (!(b == 1 || b == 2 || b == 4 || b == 8) || N < 0)
        return -1;
    if (T && !table_ok(b, g, T))
        return -1;
    const int levels = T ? g : (1 << b) - 1;
    int64_t plen = part_len(N, part);
    for (int64_t e = 0; e < N; e++) {
        int64_t p = e / plen;
        float m = mM[2 * p], M = mM[2 * p + 1];
        float range = M - m;
        int64_t bit = e * b;
        uint32_t z = (packed[bit >> 3] >> (bit & 7)) & ((1u << b) - 1u);
        float v = T ? (float)T[z] : (float)z;
        float xh = range != 0.0f ? m + v * (range / (float)levels) : m;
        e_out[e] = x[e] - xh;
    }
    return 0;
}

/*
 * [THC] section 2, Figure 2(b): NMSE(x, xhat) = ||x - xhat||^2 / ||x||^2,
 * accumulated in binary64 in index order. out = {num, den, num/den}; a zero
 * denominator gives 0 when num is 0 and +inf otherwise.
 */
int orc_nmse(const void *x, const void *xhat, int64_t N, int dt, double *out)
{
    double num = 0.0, den = 0.0;
    for (int64_t e = 0; e < N; e++) {
        double a = (double)load_elem(x, dt, e);
        double h = (double)load_elem(xhat, dt, e);
        double d = a - h;
        num += d * d;
        den += a * a;
    }
    out[0] = num;
    out[1] = den;
    out[2] = den != 0.0 ? num / den : (num == 0.0 ? 0.0 : INFINITY);
    return 0;
}
