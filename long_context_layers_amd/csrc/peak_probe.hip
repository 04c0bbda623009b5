// peak_probe.hip — measured ceilings of the GPU the kernels run on (a
// separate library, liblapeak.so, used by the benchmark; not part of the
// lightning_attn C ABI).  The published MI355X figures (8 TB/s HBM3E, 2.5
// PFLOP/s dense bf16 MFMA) are what the roofline fractions are quoted
// against; these probes measure what the same chip sustains:
//
//   la_peak_mfma_bf16   every wave runs independent chains of
//                       v_mfma_f32_32x32x16_bf16 on register operands
//                       (32,768 flop each), 8 waves per CU;
//   la_peak_mfma_bf16_data  the same with operands of random bits that differ
//                       from one MFMA to the next (the switching activity of
//                       products on real data: the energy, not the rate);
//   la_peak_read        a buffer read in 64 KB chunks, one per workgroup, the
//                       whole chunk in flight, folded into a value that is
//                       written only if it takes one particular bit pattern;
//   la_peak_write       the same chunks written;
//   la_peak_copy        chunks read, then written to a second buffer;
//   la_peak_update      chunks read, then written back in place (the access
//                       pattern of a state updated where it lives);
//   la_peak_mix3        chunks of three buffers read and one written (three
//                       bytes read for every byte written: the prefill's mix
//                       of q, k, v in and out back);
//   la_peak_stream_persistent  read, write or the 3:1 mix again, from a
//                       fixed grid of workgroups each streaming its own
//                       contiguous region in 128 KB bursts (higher mixed
//                       rates than one chunk per workgroup on this chip);
//   la_peak_pair_pattern  the prefill's memory pattern without arithmetic:
//                       a pair of workgroups per head slot, each reading the
//                       full q and k rows (the column split), only its half
//                       of every row, or the whole rows of its own tokens;
//   la_peak_l2_read     every workgroup sweeps one small region (a few MB,
//                       held by each XCD's L2) again and again: L2 hits;
//   la_peak_lds_read    every thread reads 16-byte LDS words in a loop, no
//                       bank conflicts;
//   la_peak_valu        four independent chains of integer adds per thread:
//                       every CU busy at a light load (the power of active
//                       CUs with little data movement, for the energy of the
//                       others to be taken relative to).
//
// extern "C", plain pointers and sizes, enqueued on the caller's stream (no
// synchronisation, no allocation).  Return: 0, or the hipError_t of the launch;
// -1 for bad arguments (null pointers; stream sizes that are not a positive
// multiple of 64 KB).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int PT = 256;            // threads per workgroup (4 waves)
constexpr int NACC = 4;            // independent accumulator chains per wave

__global__ __launch_bounds__(PT) void mfma_loop_kernel(int64_t iters, float *sink)
{
    const int lane = threadIdx.x % 64;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 0.001f * (lane + e));
        b[e] = (__bf16)(1.0f - 0.001f * (lane + e));
    }
    f32x16 acc[NACC];
#pragma unroll
    for (int c = 0; c < NACC; ++c) acc[c] = f32x16{};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < NACC; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NACC; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == 12345.678f) sink[blockIdx.x] = s;   // keeps the chains live; never true in practice
}

// each chain has operands of its own, from a hash of (lane, chain, element):
// normal-looking bf16 values in [-2, 2) with random low mantissa bits
__global__ __launch_bounds__(PT) void mfma_data_kernel(int64_t iters, float *sink)
{
    const int lane = threadIdx.x % 64;
    bf16x8 a[NACC], b[NACC];
#pragma unroll
    for (int c = 0; c < NACC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            unsigned h = (unsigned)(lane * 131 + c * 17 + e) * 0x9e3779b9u;
            h ^= h >> 15; h *= 0x85ebca6bu; h ^= h >> 13;
            a[c][e] = (__bf16)((float)(h & 0xffffu) * (4.0f / 65536.0f) - 2.0f);
            b[c][e] = (__bf16)((float)(h >> 16) * (4.0f / 65536.0f) - 2.0f);
        }
    f32x16 acc[NACC];
#pragma unroll
    for (int c = 0; c < NACC; ++c) acc[c] = f32x16{};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < NACC; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NACC; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == 12345.678f) sink[blockIdx.x] = s;   // keeps the chains live; never true in practice
}

// Streams: workgroup g owns the 64 KB chunk g; each thread issues all UNR of
// its 16-byte accesses (elements t + 256 u of the chunk) before using any, so
// a workgroup has the whole chunk in flight (every instruction covers 4 KB of
// consecutive bytes).
constexpr int UNR = 16;
constexpr int64_t CHUNK16 = (int64_t)PT * UNR;      // 16-byte elements per chunk (64 KB)

__global__ __launch_bounds__(PT) void read_kernel(const u32x4 *__restrict__ src,
                                                  float *__restrict__ sink)
{
    const u32x4 *p = src + blockIdx.x * CHUNK16 + threadIdx.x;
    u32x4 x[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) x[u] = __builtin_nontemporal_load(&p[u * PT]);
    u32x4 acc = x[0];
#pragma unroll
    for (int u = 1; u < UNR; ++u) acc ^= x[u];
    const unsigned v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (v == 0x9e3779b9u) sink[blockIdx.x % 4096] = (float)v;   // keeps the loads live
}

__global__ __launch_bounds__(PT) void write_kernel(u32x4 *__restrict__ dst)
{
    u32x4 *p = dst + blockIdx.x * CHUNK16 + threadIdx.x;
    const u32x4 v = {1u, 2u, 3u, 4u};
#pragma unroll
    for (int u = 0; u < UNR; ++u) __builtin_nontemporal_store(v, &p[u * PT]);
}

__global__ __launch_bounds__(PT) void copy_kernel(const u32x4 *__restrict__ src,
                                                  u32x4 *__restrict__ dst)
{
    const u32x4 *p = src + blockIdx.x * CHUNK16 + threadIdx.x;
    u32x4 *q = dst + blockIdx.x * CHUNK16 + threadIdx.x;
    u32x4 x[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) x[u] = __builtin_nontemporal_load(&p[u * PT]);
#pragma unroll
    for (int u = 0; u < UNR; ++u) __builtin_nontemporal_store(x[u], &q[u * PT]);
}

// in-place update: each element read, changed and written back where it lives
// (the access pattern of a state updated in place)
__global__ __launch_bounds__(PT) void update_kernel(u32x4 *__restrict__ buf)
{
    u32x4 *p = buf + blockIdx.x * CHUNK16 + threadIdx.x;
    u32x4 x[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) x[u] = __builtin_nontemporal_load(&p[u * PT]);
#pragma unroll
    for (int u = 0; u < UNR; ++u) __builtin_nontemporal_store(x[u] + 1u, &p[u * PT]);
}

// three reads for every write: chunk g of a, b and c in, their xor out to
// chunk g of d
__global__ __launch_bounds__(PT) void mix3_kernel(const u32x4 *__restrict__ a, const u32x4 *__restrict__ b,
                                                  const u32x4 *__restrict__ c, u32x4 *__restrict__ d)
{
    const int64_t o = blockIdx.x * CHUNK16 + threadIdx.x;
    u32x4 x[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
        x[u] = __builtin_nontemporal_load(&a[o + u * PT]) ^ __builtin_nontemporal_load(&b[o + u * PT]) ^
               __builtin_nontemporal_load(&c[o + u * PT]);
#pragma unroll
    for (int u = 0; u < UNR; ++u) __builtin_nontemporal_store(x[u], &d[o + u * PT]);
}

// Persistent streams: `blocks` workgroups, workgroup g owning the g-th
// contiguous 1/blocks of every buffer and streaming it in bursts of BURST
// 16-byte accesses per thread (128 KB of each buffer per burst): the burst's
// reads of all NR input buffers are issued before any of its writes, so a
// workgroup keeps many reads in flight and writes in runs of 128 KB.  On this
// chip this form sustains a higher mixed read/write rate than one 64 KB chunk
// per workgroup (the form above), so both are measured and the better taken.
constexpr int BURST = 32;
constexpr int64_t BURST16 = (int64_t)PT * BURST;      // 16-byte elements per burst (128 KB)

template <int NR, bool WR>
__global__ __launch_bounds__(PT) void stream_kernel(const u32x4 *__restrict__ a, const u32x4 *__restrict__ b,
                                                    const u32x4 *__restrict__ c, u32x4 *__restrict__ d,
                                                    int64_t region16, float *__restrict__ sink)
{
    const int64_t base = blockIdx.x * region16 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t o = base; o < base + region16 - threadIdx.x; o += BURST16) {
        u32x4 x[BURST];
#pragma unroll
        for (int u = 0; u < BURST; ++u) {
            x[u] = u32x4{(unsigned)u, 1u, 2u, 3u};
            if (NR > 0) x[u] = __builtin_nontemporal_load(&a[o + u * PT]);
            if (NR > 1) x[u] ^= __builtin_nontemporal_load(&b[o + u * PT]);
            if (NR > 2) x[u] ^= __builtin_nontemporal_load(&c[o + u * PT]);
        }
        if (WR) {
#pragma unroll
            for (int u = 0; u < BURST; ++u) __builtin_nontemporal_store(x[u], &d[o + u * PT]);
        } else {
#pragma unroll
            for (int u = 0; u < BURST; ++u) acc ^= x[u];
        }
    }
    const unsigned v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (!WR && v == 0x9e3779b9u) sink[blockIdx.x % 4096] = (float)v;   // keeps the loads live
}

// The prefill's memory pattern without its arithmetic: `heads` head slots of
// T tokens x 256-byte rows in four buffers q, k, v (read) and o (written);
// workgroups w and w + 8 (one XCD) share a slot (slot (w / 16) 8 + w % 8,
// half (w / 8) % 2) and walk its 64-token blocks in order, R blocks loaded
// before their outputs are written.  MODE 0 (the column split): each reads
// the full q and k rows of a block (the partner's copy an L2 hit) and its
// half of every v row, and writes its half of every o row; MODE 1: each
// moves only its half of every row (the same HBM bytes, nothing read twice);
// MODE 2 (a full-width split): each moves the whole rows of its own 32 tokens
// of the block.
template <int MODE, int R>
__global__ __launch_bounds__(PT) void pair_pattern_kernel(const u32x4 *__restrict__ q, const u32x4 *__restrict__ k,
                                                          const u32x4 *__restrict__ v, u32x4 *__restrict__ o,
                                                          int64_t T)
{
    constexpr int ROW16 = 16;                          // 16-byte chunks per row
    const int w = blockIdx.x;
    const int64_t slot = (w / 16) * 8 + w % 8;
    const int half = (w / 8) % 2, t = threadIdx.x;
    // chunk u (0, 1) of this thread within a block: half rows, or whole rows of its tokens
    auto mine = [&](int u) -> int64_t {
        const int c = u * PT + t;
        return MODE == 2 ? half * 32 * ROW16 + c : (c / 8) * ROW16 + half * 8 + c % 8;
    };
    for (int64_t b0 = 0; b0 < T; b0 += 64 * R) {
        u32x4 y[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t blk = (slot * T + b0 + 64 * r) * ROW16;    // first chunk of the block
            u32x4 x = {0u, 0u, 0u, 0u};
            if (MODE == 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u)              // 1024 chunks of q and of k
                    x ^= __builtin_nontemporal_load(&q[blk + u * PT + t]) ^
                         __builtin_nontemporal_load(&k[blk + u * PT + t]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {                // 512 chunks of this workgroup's part
                const int64_t e = blk + mine(u);
                if (MODE != 0) x ^= __builtin_nontemporal_load(&q[e]) ^ __builtin_nontemporal_load(&k[e]);
                y[r][u] = x ^ __builtin_nontemporal_load(&v[e]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                __builtin_nontemporal_store(y[r][u], &o[(slot * T + b0 + 64 * r) * ROW16 + mine(u)]);
    }
}

// L2 hits: each workgroup sweeps the region (region16 16-byte elements, a
// multiple of a chunk) reps times, chunk by chunk, starting at a chunk of its
// own so the workgroups spread over the L2 channels
__global__ __launch_bounds__(PT) void l2_read_kernel(const u32x4 *__restrict__ src, int64_t region16,
                                                     int64_t reps, float *__restrict__ sink)
{
    const int64_t nchunk = region16 / CHUNK16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t r = 0; r < reps; ++r)
        for (int64_t c = 0; c < nchunk; ++c) {
            const u32x4 *p = src + ((c + blockIdx.x) % nchunk) * CHUNK16 + threadIdx.x;
            u32x4 x[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) x[u] = p[u * PT];
#pragma unroll
            for (int u = 0; u < UNR; ++u) acc ^= x[u];
        }
    const unsigned v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (v == 0x9e3779b9u) sink[blockIdx.x % 4096] = (float)v;   // keeps the loads live
}

// LDS reads: 64 KB per workgroup, each thread reading consecutive 16-byte
// words (conflict-free) UNR at a time; the offset is hidden from the compiler
// every iteration so the reads cannot be hoisted out of the loop
constexpr int LDS16 = 4096;                          // 16-byte words (64 KB)
__global__ __launch_bounds__(PT) void lds_read_kernel(int64_t iters, float *__restrict__ sink)
{
    __shared__ u32x4 buf[LDS16];
    for (int i = threadIdx.x; i < LDS16; i += PT) buf[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
    __syncthreads();
    u32x4 acc = {0u, 0u, 0u, 0u};
    int off = threadIdx.x;
    for (int64_t i = 0; i < iters; ++i) {
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= buf[(off + u * PT) & (LDS16 - 1)];
    }
    const unsigned v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (v == 0x9e3779b9u) sink[blockIdx.x % 4096] = (float)v;
}

// active CUs at a light load: four dependent chains of integer adds per thread
__global__ __launch_bounds__(PT) void valu_kernel(int64_t iters, float *__restrict__ sink)
{
    unsigned a = threadIdx.x, b = a ^ 1u, c = a ^ 2u, d = a ^ 3u;
    for (int64_t i = 0; i < iters; ++i) {
        asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
        a += 0x9e3779b9u; b += a; c += b; d += c;
    }
    const unsigned v = a ^ b ^ c ^ d;
    if (v == 0x9e3779b9u) sink[blockIdx.x % 4096] = (float)v;
}

// bytes must be a positive multiple of one chunk (64 KB), grid = chunks
bool chunks_of(int64_t bytes, unsigned *grid) {
    if (bytes <= 0 || bytes % (CHUNK16 * 16) != 0 || bytes / (CHUNK16 * 16) > 0x7fffffff)
        return false;
    *grid = (unsigned)(bytes / (CHUNK16 * 16));
    return true;
}

}  // namespace

extern "C" {

// flop = blocks * 4 waves * iters * NACC * 32768
int la_peak_mfma_bf16(int64_t iters, int64_t blocks, float *sink, void *stream)
{
    if (iters < 1 || blocks < 1 || blocks > 0x7fffffff || !sink) return -1;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(PT), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return (int)hipGetLastError();
}

int la_peak_mfma_chains(void) { return NACC; }

int la_peak_mfma_bf16_data(int64_t iters, int64_t blocks, float *sink, void *stream)
{
    if (iters < 1 || blocks < 1 || blocks > 0x7fffffff || !sink) return -1;
    hipLaunchKernelGGL(mfma_data_kernel, dim3((unsigned)blocks), dim3(PT), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return (int)hipGetLastError();
}

// sink: at least 4096 floats
int la_peak_read(const void *src, int64_t bytes, float *sink, void *stream)
{
    unsigned g;
    if (!src || !sink || !chunks_of(bytes, &g)) return -1;
    hipLaunchKernelGGL(read_kernel, dim3(g), dim3(PT), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), sink);
    return (int)hipGetLastError();
}

int la_peak_write(void *dst, int64_t bytes, void *stream)
{
    unsigned g;
    if (!dst || !chunks_of(bytes, &g)) return -1;
    hipLaunchKernelGGL(write_kernel, dim3(g), dim3(PT), 0, static_cast<hipStream_t>(stream),
                       static_cast<u32x4 *>(dst));
    return (int)hipGetLastError();
}

// bytes read (and as many written)
int la_peak_copy(const void *src, void *dst, int64_t bytes, void *stream)
{
    unsigned g;
    if (!src || !dst || !chunks_of(bytes, &g)) return -1;
    hipLaunchKernelGGL(copy_kernel, dim3(g), dim3(PT), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst));
    return (int)hipGetLastError();
}

int la_peak_update(void *buf, int64_t bytes, void *stream)
{
    unsigned g;
    if (!buf || !chunks_of(bytes, &g)) return -1;
    hipLaunchKernelGGL(update_kernel, dim3(g), dim3(PT), 0, static_cast<hipStream_t>(stream),
                       static_cast<u32x4 *>(buf));
    return (int)hipGetLastError();
}

// bytes: the size of each of the four buffers (3 x bytes read, bytes written)
int la_peak_mix3(const void *a, const void *b, const void *c, void *d, int64_t bytes, void *stream)
{
    unsigned g;
    if (!a || !b || !c || !d || !chunks_of(bytes, &g)) return -1;
    hipLaunchKernelGGL(mix3_kernel, dim3(g), dim3(PT), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(a), static_cast<const u32x4 *>(b),
                       static_cast<const u32x4 *>(c), static_cast<u32x4 *>(d));
    return (int)hipGetLastError();
}

// Persistent forms: `blocks` workgroups (1..65536), bytes a positive multiple
// of blocks * 128 KB.  kind 0: read `a` (sink: at least 4096 floats);
// kind 1: write `d`; kind 2: read a, b, c and write their xor to d (the 3:1
// mix, each buffer `bytes` long).
int la_peak_stream_persistent(int kind, const void *a, const void *b, const void *c, void *d,
                              int64_t bytes, int64_t blocks, float *sink, void *stream)
{
    if (blocks < 1 || blocks > 65536 || bytes <= 0 || bytes % (blocks * BURST16 * 16) != 0) return -1;
    const int64_t region16 = bytes / 16 / blocks;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *pa = static_cast<const u32x4 *>(a), *pb = static_cast<const u32x4 *>(b),
                *pc = static_cast<const u32x4 *>(c);
    u32x4 *pd = static_cast<u32x4 *>(d);
    const dim3 g((unsigned)blocks), t(PT);
    switch (kind) {
    case 0:
        if (!a || !sink) return -1;
        hipLaunchKernelGGL((stream_kernel<1, false>), g, t, 0, s, pa, pa, pa, pd, region16, sink);
        break;
    case 1:
        if (!d) return -1;
        hipLaunchKernelGGL((stream_kernel<0, true>), g, t, 0, s, pa, pa, pa, pd, region16, sink);
        break;
    case 2:
        if (!a || !b || !c || !d) return -1;
        hipLaunchKernelGGL((stream_kernel<3, true>), g, t, 0, s, pa, pb, pc, pd, region16, sink);
        break;
    default:
        return -1;
    }
    return (int)hipGetLastError();
}

// mode 0, 1 or 2 (above); inflight 1 or 4 blocks; heads: a positive multiple
// of 8 (2 * heads workgroups); T: tokens per head, a positive multiple of
// 64 * inflight; each buffer heads * T * 256 bytes
int la_peak_pair_pattern(int mode, int inflight, const void *q, const void *k, const void *v, void *o,
                         int64_t heads, int64_t T, void *stream)
{
    if (!q || !k || !v || !o || mode < 0 || mode > 2 || (inflight != 1 && inflight != 4) ||
        heads < 8 || heads % 8 != 0 || heads > (1 << 20) || T < 64 * inflight || T % (64 * inflight) != 0)
        return -1;
    const dim3 g((unsigned)(2 * heads)), t(PT);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *pq = static_cast<const u32x4 *>(q), *pk = static_cast<const u32x4 *>(k),
                *pv = static_cast<const u32x4 *>(v);
    u32x4 *po = static_cast<u32x4 *>(o);
    const int sel = 3 * (inflight == 4) + mode;
    switch (sel) {
    case 0: hipLaunchKernelGGL((pair_pattern_kernel<0, 1>), g, t, 0, s, pq, pk, pv, po, T); break;
    case 1: hipLaunchKernelGGL((pair_pattern_kernel<1, 1>), g, t, 0, s, pq, pk, pv, po, T); break;
    case 2: hipLaunchKernelGGL((pair_pattern_kernel<2, 1>), g, t, 0, s, pq, pk, pv, po, T); break;
    case 3: hipLaunchKernelGGL((pair_pattern_kernel<0, 4>), g, t, 0, s, pq, pk, pv, po, T); break;
    case 4: hipLaunchKernelGGL((pair_pattern_kernel<1, 4>), g, t, 0, s, pq, pk, pv, po, T); break;
    default: hipLaunchKernelGGL((pair_pattern_kernel<2, 4>), g, t, 0, s, pq, pk, pv, po, T); break;
    }
    return (int)hipGetLastError();
}

// region_bytes: a positive multiple of 64 KB; bytes read = blocks * region_bytes * reps
int la_peak_l2_read(const void *src, int64_t region_bytes, int64_t reps, int64_t blocks, float *sink,
                    void *stream)
{
    unsigned g;
    if (!src || !sink || !chunks_of(region_bytes, &g) || reps < 1 || blocks < 1 ||
        blocks > 0x7fffffff)
        return -1;
    hipLaunchKernelGGL(l2_read_kernel, dim3((unsigned)blocks), dim3(PT), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src),
                       region_bytes / 16, reps, sink);
    return (int)hipGetLastError();
}

// bytes read = blocks * 256 threads * UNR * 16 B * iters
int la_peak_lds_read(int64_t iters, int64_t blocks, float *sink, void *stream)
{
    if (iters < 1 || blocks < 1 || blocks > 0x7fffffff || !sink) return -1;
    hipLaunchKernelGGL(lds_read_kernel, dim3((unsigned)blocks), dim3(PT), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return (int)hipGetLastError();
}

int la_peak_lds_bytes_per_iter(void) { return PT * UNR * 16; }

int la_peak_valu(int64_t iters, int64_t blocks, float *sink, void *stream)
{
    if (iters < 1 || blocks < 1 || blocks > 0x7fffffff || !sink) return -1;
    hipLaunchKernelGGL(valu_kernel, dim3((unsigned)blocks), dim3(PT), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
