// cp.hip — the two steps a sequence-sharded (context-parallel) prefill adds
// once every rank has run the prefill over its own shard from a zero state
// (Ling and Ring 2.6 Technical Report, §4.1.1 and Fig. 10: a local state and
// a local output per rank, an all-gather of the [B,H,D,D] local states, then
// each rank folds the states of the shards before it into its incoming state
// and corrects its local output with it).
//
// cp_fold:    S_in(r) = lambda^L_{r-1} S_in(r-1) + S_loc(r-1),  S_in(0) = S_init,
//   evaluated in this (Horner) order over the shards before r, elementwise over
//   [B,H,d,d] fp32.  Bound by HBM: r + 1 states read and one written, 16-byte
//   accesses, a fixed summation order (deterministic).
// cp_correct: out_a += lambda^(a+1) q_a S_in for the shard's L tokens: the
//   prefill's inter term on its own, a [L,d] x [d,d] product per (b, h) on
//   MFMA with S_in rounded to bf16 (as the prefill's inter term uses it),
//   fp32 accumulation and one bf16 rounding of the corrected output.  Bound
//   by HBM: q read, out read and written, 6d bytes per token-head; at
//   d = 128 that is 42.7 flop per byte against a ridge near 315.
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int FT = 256;            // fold: threads per workgroup
constexpr int FMAX_GRID = 8192;    // fold: grid cap (grid-stride beyond)

struct FoldLens {
    int n[MAX_CP_SHARDS];
};

// init and out may be the same array (each element is read, then written, by
// one thread), so neither is restrict-qualified.
__global__ __launch_bounds__(FT) void cp_fold_kernel(
    const f32x4 *__restrict__ loc, const f32x4 *init, f32x4 *out,
    const float *__restrict__ slopes, FoldLens lens, int nfold, int64_t n4, int64_t slice4,
    int64_t H)
{
    for (int64_t i = blockIdx.x * (int64_t)FT + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * FT) {
        const float s = slopes[(i / slice4) % H];
        f32x4 acc = init ? init[i] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int j = 0; j < nfold; ++j) {
            const float lam = decay_pow(s, lens.n[j]);
            const f32x4 x = __builtin_nontemporal_load(&loc[j * n4 + i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(lam, acc[e], x[e]);
        }
        out[i] = acc;
    }
}

constexpr int CT = 256;            // correct: threads per workgroup (4 waves)
constexpr int TT = 64;             // correct: tokens per tile
constexpr int CTOK = 512;          // correct: tokens per workgroup (8 tiles)
constexpr int CPAD = 8;            // LDS row padding (bf16 elements)
constexpr int RSRC_W3 = 0x00020000;   // buffer descriptor word 3 (raw 32-bit access)

template <int D>
struct CorrSmem {
    uint16_t Q[TT][D + CPAD];
    uint16_t O[TT][D + CPAD];
};

// rows t0 .. t0 + c - 1 of one (b, h) slice (c = 0 past the end): loads past
// the range read zero, stores past it are dropped
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base, int64_t t0,
                                                             int64_t L)
{
    const int64_t c = max((int64_t)0, min((int64_t)TT, L - t0));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(base + t0 * D), (short)0,
                                             (int)(c * D * 2), RSRC_W3);
}

// A workgroup corrects CTOK tokens of one (b, h) in 64-token tiles.  q and
// out tiles move between HBM and LDS as whole rows (thread i takes 16-byte
// chunks i, i + 256, ...: every load or store instruction covers 4 KB of
// consecutive rows), the next tile's loads are issued before the current
// tile's products, and the read-modify-write of out happens in LDS.
// Products: O^T = S^T Q^T with v_mfma_f32_32x32x16_bf16; wave w owns output
// columns 32 (w % NCT) .. +31 for the token halves w / NCT, w / NCT + 4 / NCT,
// ...; A = S^T (row j = lane % 32, k = 8 (lane / 32) + e of each 16-wide k
// step, read once from the fp32 state, rounded to bf16, kept in registers),
// B = Q^T (column = token lane % 32: 16 contiguous bytes of its q row), C
// register r = column 8 (r / 4) + 4 (lane / 32) + r % 4 of token lane % 32.
template <int D>
__global__ __launch_bounds__(CT) void cp_correct_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ slopes,
    const float *__restrict__ s_in, uint16_t *__restrict__ out, int64_t H, int64_t L,
    int64_t chunks)
{
    constexpr int NCT = D / 32;        // 32-column tiles
    constexpr int KS = D / 16;         // 16-wide k steps
    constexpr int NCH = TT * D / 8 / CT;   // 16-byte chunks per thread per tile
    constexpr int CPR = D / 8;         // chunks per row
    __shared__ CorrSmem<D> sm;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int l32 = lane % 32, hf = lane / 32;
    const int ct = wave % NCT;
    const int64_t bh = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
    const float s = slopes[bh % H];

    const float *S = s_in + bh * D * D;
    bf16x8 a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            a[ks][e] = (__bf16)S[(16 * ks + 8 * hf + e) * D + 32 * ct + l32];

    const uint16_t *qb = q + bh * L * D;
    uint16_t *ob = out + bh * L * D;
    const int64_t tbeg = chunk * CTOK;
    const int ntile = (int)((min(L, tbeg + CTOK) - tbeg + TT - 1) / TT);

    uint4 rq[NCH], ro[NCH];
    auto fetch = [&](int64_t t0) {
        const __amdgpu_buffer_rsrc_t rsq = tile_rsrc<D>(qb, t0, L);
        const __amdgpu_buffer_rsrc_t rso = tile_rsrc<D>(ob, t0, L);
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int off = (tid + CT * u) * 16;
            rq[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsq, off, 0, 0));
            ro[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rso, off, 0, 0));
        }
    };
    fetch(tbeg);
    for (int it = 0; it < ntile; ++it) {
        const int64_t t0 = tbeg + (int64_t)it * TT;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int c = tid + CT * u, row = c / CPR, col = (c % CPR) * 8;
            *reinterpret_cast<uint4 *>(&sm.Q[row][col]) = rq[u];
            *reinterpret_cast<uint4 *>(&sm.O[row][col]) = ro[u];
        }
        __syncthreads();
        if (it + 1 < ntile) fetch(t0 + TT);
#pragma unroll
        for (int i = 0; i < (TT / 32) / (4 / NCT); ++i) {
            const int th = wave / NCT + i * (4 / NCT);     // token half of the tile
            const int row = 32 * th + l32;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    a[ks], *reinterpret_cast<const bf16x8 *>(&sm.Q[row][16 * ks + 8 * hf]), acc,
                    0, 0, 0);
            const float sc = decay_pow(s, (int)(t0 + row + 1));
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint2 *p = reinterpret_cast<uint2 *>(&sm.O[row][32 * ct + 8 * g + 4 * hf]);
                uint2 w = *p;
                const float o0 = fmaf(sc, acc[4 * g + 0], bf16_to_f32(w.x & 0xffffu));
                const float o1 = fmaf(sc, acc[4 * g + 1], bf16_to_f32(w.x >> 16));
                const float o2 = fmaf(sc, acc[4 * g + 2], bf16_to_f32(w.y & 0xffffu));
                const float o3 = fmaf(sc, acc[4 * g + 3], bf16_to_f32(w.y >> 16));
                w.x = pack_bf16x2(o0, o1);
                w.y = pack_bf16x2(o2, o3);
                *p = w;
            }
        }
        __syncthreads();
        const __amdgpu_buffer_rsrc_t rst = tile_rsrc<D>(ob, t0, L);
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int c = tid + CT * u, row = c / CPR, col = (c % CPR) * 8;
            const uint4 x = *reinterpret_cast<const uint4 *>(&sm.O[row][col]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), rst, c * 16, 0, 0);
        }
    }
}

}  // namespace

int64_t cp_correct_grid(int64_t B, int64_t H, int64_t L) {
    return B * H * ((L + CTOK - 1) / CTOK);
}

hipError_t launch_cp_fold(const float *loc, const int *lens, int nfold, const float *init,
                          float *out, const float *slopes, int64_t B, int64_t H, int d,
                          hipStream_t stream)
{
    FoldLens fl = {};
    for (int j = 0; j < nfold; ++j) fl.n[j] = lens[j];
    const int64_t slice4 = (int64_t)d * d / 4;
    int64_t n4 = B * H * slice4;
    const int64_t blocks = (n4 + FT - 1) / FT;
    const dim3 grid((unsigned)(blocks < FMAX_GRID ? blocks : FMAX_GRID)), block(FT);
    const f32x4 *l4 = reinterpret_cast<const f32x4 *>(loc);
    const f32x4 *i4 = reinterpret_cast<const f32x4 *>(init);
    f32x4 *o4 = reinterpret_cast<f32x4 *>(out);
    int64_t s4 = slice4, h = H;
    void *args[] = {(void *)&l4, (void *)&i4, (void *)&o4, (void *)&slopes, (void *)&fl,
                    (void *)&nfold, (void *)&n4, (void *)&s4, (void *)&h};
    return hipLaunchKernel((const void *)cp_fold_kernel, grid, block, args, 0, stream);
}

hipError_t launch_cp_correct(const uint16_t *q, const float *slopes, const float *s_in,
                             uint16_t *out, int64_t B, int64_t H, int64_t L, int d,
                             hipStream_t stream)
{
    int64_t chunks = (L + CTOK - 1) / CTOK;
    const dim3 grid((unsigned)cp_correct_grid(B, H, L)), block(CT);
    void *args[] = {(void *)&q, (void *)&slopes, (void *)&s_in, (void *)&out, (void *)&H,
                    (void *)&L, (void *)&chunks};
    const void *fn = d == 64 ? (const void *)cp_correct_kernel<64>
                             : (const void *)cp_correct_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace la
