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
#include "qk_prologue.h"

#include <algorithm>

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
constexpr int CTOK = 128;          // correct: tokens per chunk (2 tiles)
constexpr int CWG = 128;           // correct: workgroups per (segment, b, h) at most
constexpr int CPAD = 8;            // LDS row padding (bf16 elements)
constexpr int RSRC_W3 = 0x00020000;   // buffer descriptor word 3 (raw 32-bit access)

template <int D>
struct CorrSmem {
    uint16_t Q[TT][D + CPAD];
    uint16_t O[TT][D + CPAD];
};

// rows t0 .. t0 + c - 1 of one (b, h) slice, ts elements apart (c = 0 past
// the end): the range ends after the last real row, so loads past it read
// zero and stores past it are dropped
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base, int64_t t0,
                                                             int64_t L, int64_t ts)
{
    const int64_t c = max((int64_t)0, min((int64_t)TT, L - t0));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(base + t0 * ts), (short)0,
                                             c == 0 ? 0 : (int)(((c - 1) * ts + D) * 2), RSRC_W3);
}

// A workgroup corrects the CTOK-token chunks c, c + cstride, ... of one
// (segment, b, h) in 64-token tiles (cstride = min(chunks, CWG) workgroups
// per row, each reading its state once: the corrected tokens of the slowest
// heads spread over many workgroups, at most two tiles apiece in each of
// their chunks; the workgroups of a row whose first tile has underflowed
// return at once).
// q and out tiles move between HBM and LDS as whole rows (thread i takes
// 16-byte chunks i, i + 256, ...: every load or store instruction covers 4 KB
// of consecutive rows), the next tile's loads are issued before the current
// tile's products, and the read-modify-write of out happens in LDS.  A tile
// whose first token's factor lambda^(a+1) has underflowed to exactly 0 in
// fp32 adds nothing, nor does any tile after it (the factor only falls), so
// the workgroup stops there (and at its later chunks, all past that point):
// with decays below 1 the correction is confined
// to the first tokens of the segment, and nothing about the result changes.
// Products: O^T = S^T Q^T with v_mfma_f32_32x32x16_bf16; wave w owns output
// columns 32 (w % NCT) .. +31 for the token halves w / NCT, w / NCT + 4 / NCT,
// ...; A = S^T (row j = lane % 32, k = 8 (lane / 32) + e of each 16-wide k
// step, read once from the fp32 state, rounded to bf16, kept in registers),
// B = Q^T (column = token lane % 32: 16 contiguous bytes of its q row), C
// register r = column 8 (r / 4) + 4 (lane / 32) + r % 4 of token lane % 32.
// Segments: segment g of a (b, h) row covers tokens t_off + g * seg .. (up to
// the row's ntok tokens) and takes the state s_in + (g * BH + bh) * D * D.  A
// shard correction is one segment at t_off = 0.  q and out rows: (b, h) rows
// qhs / ohs elements apart, tokens qts / ots apart (>= D), channels contiguous.
// PROT >= 0: q is the projection's raw q, normalised and rotated (QK Norm +
// RoPE with PROT rotary dims at position pr.pos0 + token) as each tile
// arrives, as the prefill does.
template <int D, int PROT>
__global__ __launch_bounds__(CT) void cp_correct_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ slopes,
    const float *__restrict__ s_in, uint16_t *__restrict__ out, int64_t H, int64_t BH,
    int64_t qhs, int64_t qts, int64_t ohs, int64_t ots, int64_t t_off, int64_t seg, int64_t ntok,
    int64_t chunks, int64_t cstride, QkPrologue pr)
{
    constexpr bool PRO = PROT >= 0;
    static_assert(!PRO || D == pro::PD, "the fused prologue handles 128-channel rows");
    constexpr int NCT = D / 32;        // 32-column tiles
    constexpr int KS = D / 16;         // 16-wide k steps
    constexpr int NCH = TT * D / 8 / CT;   // 16-byte chunks per thread per tile
    constexpr int CPR = D / 8;         // chunks per row
    __shared__ CorrSmem<D> sm;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int l32 = lane % 32, hf = lane / 32;
    const int ct = wave % NCT;
    const int64_t c0 = blockIdx.x % cstride, bh = (blockIdx.x / cstride) % BH;
    const int64_t g = blockIdx.x / cstride / BH;
    const float s = slopes[bh % H];

    const int64_t a0 = t_off + g * seg;                       // the segment's first token
    const int64_t L = max((int64_t)0, min(seg, ntok - a0));   // its tokens
    // tiles of chunk c before the underflow (0: none here or in any later chunk)
    auto tiles = [&](int64_t c) {
        const int64_t tbeg = c * CTOK;
        int n = (int)max((int64_t)0, (min(L, tbeg + CTOK) - tbeg + TT - 1) / TT);
        for (int it = 0; it < n; ++it)
            if (decay_pow(s, (int)(tbeg + (int64_t)it * TT + 1)) == 0.0f) return it;
        return n;
    };
    if (c0 >= chunks || tiles(c0) <= 0) return;

    const float *S = s_in + (g * BH + bh) * D * D;
    bf16x8 a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            a[ks][e] = (__bf16)S[(16 * ks + 8 * hf + e) * D + 32 * ct + l32];

    const uint16_t *qb = q + bh * qhs + a0 * qts;
    uint16_t *ob = out + bh * ohs + a0 * ots;
    // thread chunk u: row (tid + CT u) / CPR, 16 bytes at column 8 ((tid + CT u) % CPR);
    // with PRO q takes the prologue's layout instead: row tid / 4, chunks tid % 4 + 4u
    pro::Lane<PRO ? PROT : 0> pl;
    if constexpr (PRO) {
        static_assert(NCH == pro::NC, "the prologue's row layout");
        QkPrologue qonly = pr;
        qonly.kw = nullptr;
        pl.init(qonly, tid % pro::LPR);
    }
    int qrow[NCH], qcol[NCH], qoff[NCH], ooff[NCH];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int c = tid + CT * u, row = c / CPR, col = (c % CPR) * 8;
        qrow[u] = PRO ? tid / pro::LPR : row;
        qcol[u] = PRO ? (tid % pro::LPR + pro::LPR * u) * 8 : col;
        qoff[u] = (int)((qrow[u] * qts + qcol[u]) * 2);
        ooff[u] = (int)((row * ots + col) * 2);
    }

    uint4 rq[NCH], ro[NCH];
    auto fetch = [&](int64_t t0) {
        const __amdgpu_buffer_rsrc_t rsq = tile_rsrc<D>(qb, t0, L, qts);
        const __amdgpu_buffer_rsrc_t rso = tile_rsrc<D>(ob, t0, L, ots);
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            rq[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsq, qoff[u], 0, 0));
            ro[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rso, ooff[u], 0, 0));
        }
    };
    for (int64_t chunk = c0; chunk < chunks; chunk += cstride) {
    const int64_t tbeg = chunk * CTOK;
    const int ntile = tiles(chunk);
    if (ntile <= 0) break;
    fetch(tbeg);
    for (int it = 0; it < ntile; ++it) {
        const int64_t t0 = tbeg + (int64_t)it * TT;
        if constexpr (PRO) {                 // row tid/4 at position pos0 + a0 + t0 + tid/4
            const pro::RowAngles a = pro::row_angles(pl, pr.pos0 + a0 + t0 + tid / pro::LPR);
            pro::norm_rope<PROT>(rq, pl.wq, a, pr.eps);
        }
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int c = tid + CT * u, row = c / CPR, col = (c % CPR) * 8;
            *reinterpret_cast<uint4 *>(&sm.Q[qrow[u]][qcol[u]]) = rq[u];
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
            for (int gq = 0; gq < 4; ++gq) {
                uint2 *p = reinterpret_cast<uint2 *>(&sm.O[row][32 * ct + 8 * gq + 4 * hf]);
                uint2 w = *p;
                const float o0 = fmaf(sc, acc[4 * gq + 0], bf16_to_f32(w.x & 0xffffu));
                const float o1 = fmaf(sc, acc[4 * gq + 1], bf16_to_f32(w.x >> 16));
                const float o2 = fmaf(sc, acc[4 * gq + 2], bf16_to_f32(w.y & 0xffffu));
                const float o3 = fmaf(sc, acc[4 * gq + 3], bf16_to_f32(w.y >> 16));
                w.x = pack_bf16x2(o0, o1);
                w.y = pack_bf16x2(o2, o3);
                *p = w;
            }
        }
        __syncthreads();
        const __amdgpu_buffer_rsrc_t rst = tile_rsrc<D>(ob, t0, L, ots);
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int c = tid + CT * u, row = c / CPR, col = (c % CPR) * 8;
            const uint4 x = *reinterpret_cast<const uint4 *>(&sm.O[row][col]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), rst, ooff[u], 0, 0);
        }
    }
    }
}

// ---- the sequence split of a prefill whose grid fills at most half the
// device: S segments of each (b = 0, h) row run as one packed launch, the first
// from the caller's state and the others from zero; then the states are
// chained and the later segments' outputs corrected (the same fold and
// correction as the sharded prefill, here on one device).

// slot 0 <- the caller's state, slots 1.. <- 0, cu <- the segment offsets
__global__ __launch_bounds__(FT) void split_prep_kernel(
    const f32x4 *__restrict__ state, f32x4 *__restrict__ slots, int64_t *__restrict__ cu,
    int64_t n4, int nseg, int64_t seg, int64_t ntok)
{
    const int64_t i0 = blockIdx.x * (int64_t)FT + threadIdx.x;
    if (i0 <= nseg) cu[i0] = min(i0 * seg, ntok);
    for (int64_t i = i0; i < n4 * nseg; i += (int64_t)gridDim.x * FT)
        slots[i] = i < n4 ? state[i] : f32x4{0.f, 0.f, 0.f, 0.f};
}

// slot g <- lambda^len(g) slot(g-1) + slot g for g = 1 .. nseg-1 (each slot
// then holds the state at the end of its segment), and the caller's state <-
// the last; one thread per 4 elements, a fixed order (deterministic)
__global__ __launch_bounds__(FT) void split_fold_kernel(
    f32x4 *__restrict__ slots, f32x4 *__restrict__ state, const float *__restrict__ slopes,
    int64_t n4, int64_t slice4, int64_t H, int nseg, int64_t seg, int64_t ntok)
{
    for (int64_t i = blockIdx.x * (int64_t)FT + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * FT) {
        const float s = slopes[(i / slice4) % H];
        f32x4 acc = slots[i];
        for (int g = 1; g < nseg; ++g) {
            const float lam = decay_pow(s, (int)min(seg, ntok - g * seg));
            const f32x4 x = slots[g * n4 + i];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(lam, acc[e], x[e]);
            slots[g * n4 + i] = acc;
        }
        state[i] = acc;
    }
}

}  // namespace

int64_t cp_correct_grid(int64_t B, int64_t H, int64_t L) {
    return B * H * std::min<int64_t>((L + CTOK - 1) / CTOK, CWG);
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

static hipError_t launch_correct(const uint16_t *q, const float *slopes, const float *s_in,
                                 uint16_t *out, int64_t BH, int64_t H, int64_t qhs, int64_t qts,
                                 int64_t ohs, int64_t ots, int64_t t_off, int64_t seg,
                                 int64_t ntok, int64_t nseg, int d, hipStream_t stream,
                                 const QkPrologue *pro = nullptr)
{
    if (pro && d != 128) return hipErrorInvalidValue;
    int64_t chunks = (seg + CTOK - 1) / CTOK;
    int64_t cstride = std::max<int64_t>(1, std::min<int64_t>(chunks, CWG));
    const dim3 grid((unsigned)(nseg * BH * cstride)), block(CT);
    QkPrologue pr = pro ? *pro : QkPrologue{nullptr, nullptr, 0.0, 0, 0.0f, 0};
    void *args[] = {(void *)&q, (void *)&slopes, (void *)&s_in, (void *)&out, (void *)&H,
                    (void *)&BH, (void *)&qhs, (void *)&qts, (void *)&ohs, (void *)&ots,
                    (void *)&t_off, (void *)&seg, (void *)&ntok, (void *)&chunks, (void *)&cstride,
                    (void *)&pr};
    const void *fn = d == 64 ? (const void *)cp_correct_kernel<64, -1>
                               : (const void *)cp_correct_kernel<128, -1>;
    if (pro) {
        switch (pro->rot) {
            case 0: fn = (const void *)cp_correct_kernel<128, 0>; break;
            case 16: fn = (const void *)cp_correct_kernel<128, 16>; break;
            case 32: fn = (const void *)cp_correct_kernel<128, 32>; break;
            case 64: fn = (const void *)cp_correct_kernel<128, 64>; break;
            case 128: fn = (const void *)cp_correct_kernel<128, 128>; break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_cp_correct(const uint16_t *q, const float *slopes, const float *s_in,
                             uint16_t *out, int64_t B, int64_t H, int64_t L, int d,
                             hipStream_t stream)
{
    return launch_correct(q, slopes, s_in, out, B * H, H, L * d, d, L * d, d, 0, L, L, 1, d, stream);
}

int64_t split_workspace_bytes(int64_t H, int nseg, int d)
{
    return nseg < 2 ? 0 : (int64_t)nseg * H * d * d * 4 + ((nseg + 1) * 8 + 255) / 256 * 256;
}

// the segment length of a split into nseg (segments start on 64-token blocks)
int64_t split_segment(int64_t N, int nseg)
{
    const int64_t seg = (N + nseg - 1) / nseg;
    return (seg + 63) / 64 * 64;
}

// workspace: nseg state slots [nseg][H][d][d] fp32, then nseg + 1 offsets;
// slot 0 <- the caller's state, the others <- 0, the offsets <- the segments
hipError_t launch_split_prep(const float *state, float *slots, int64_t **cu, int64_t H, int d,
                              int nseg, int64_t seg, int64_t N, hipStream_t stream)
{
    *cu = reinterpret_cast<int64_t *>(slots + (int64_t)nseg * H * d * d);
    const int64_t n4 = H * ((int64_t)d * d / 4);
    const int64_t blocks = (n4 * nseg + FT - 1) / FT;
    const dim3 grid((unsigned)(blocks < FMAX_GRID ? blocks : FMAX_GRID)), block(FT);
    const f32x4 *in4 = reinterpret_cast<const f32x4 *>(state);
    f32x4 *s4 = reinterpret_cast<f32x4 *>(slots);
    int64_t *c = *cu;
    int64_t nn = n4, sg = seg, nt = N;
    int ns = nseg;
    void *args[] = {(void *)&in4, (void *)&s4, (void *)&c, (void *)&nn, (void *)&ns,
                    (void *)&sg, (void *)&nt};
    return hipLaunchKernel((const void *)split_prep_kernel, grid, block, args, 0, stream);
}

// the slots chained into the state at each segment's end, the last into the caller's state
hipError_t launch_split_fold(float *slots, float *state, const float *slopes, int64_t H, int d,
                              int nseg, int64_t seg, int64_t N, hipStream_t stream)
{
    const int64_t slice4 = (int64_t)d * d / 4, n4 = H * slice4;
    const int64_t blocks = (n4 + FT - 1) / FT;
    const dim3 grid((unsigned)(blocks < FMAX_GRID ? blocks : FMAX_GRID)), block(FT);
    f32x4 *s4 = reinterpret_cast<f32x4 *>(slots);
    f32x4 *st4 = reinterpret_cast<f32x4 *>(state);
    int64_t nn = n4, sl = slice4, hh = H, sg = seg, nt = N;
    int ns = nseg;
    void *args[] = {(void *)&s4, (void *)&st4, (void *)&slopes, (void *)&nn, (void *)&sl,
                    (void *)&hh, (void *)&ns, (void *)&sg, (void *)&nt};
    return hipLaunchKernel((const void *)split_fold_kernel, grid, block, args, 0, stream);
}

hipError_t launch_prefill_bf16_split(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     const float *slopes, uint16_t *out, float *state,
                                     int64_t H, int64_t N, int d, int nseg, int njt,
                                     const Strides &in, const Strides &ost, void *workspace,
                                     hipStream_t stream, const QkPrologue *pro)
{
    float *slots = static_cast<float *>(workspace);
    const int64_t seg = split_segment(N, nseg);
    int64_t *cu = nullptr;
    hipError_t e = launch_split_prep(state, slots, &cu, H, d, nseg, seg, N, stream);
    if (e != hipSuccess) return e;
    const SeqMap map = {cu, H, 0, N, {0, in.sh, in.st}, {0, ost.sh, ost.st}};
    e = launch_prefill_bf16_nowalk(q, k, v, slopes, out, slots, nseg, map, d, stream, njt, pro);
    if (e != hipSuccess) return e;
    e = launch_split_fold(slots, state, slopes, H, d, nseg, seg, N, stream);
    if (e != hipSuccess) return e;
    // segment g >= 1 is corrected with slot g - 1 (the state at its start)
    return launch_correct(q, slopes, slots, out, H, H, in.sh, in.st, ost.sh, ost.st, seg, seg, N,
                          nseg - 1, d, stream, pro);
}

}  // namespace la
