// prefill_bf16.hip — blockwise decayed causal linear attention, bf16
// activations, fp32 accumulation, gfx950 matrix cores.
//
// Method (Ling and Ring 2.6 Technical Report, §4.1.1 and Fig. 10: a local
// output from the tokens of a piece plus a correction from the state carried
// in from everything before it; here the pieces are 64-token blocks handled
// in order inside one workgroup).  For one (b, h), the block of c tokens at
// t0, local indices a, b < c and lambda = exp(-slope_h):
//   P^T[b][a] = lambda^(a-b) (k_b . q_a)  (b <= a), else 0      [intra scores]
//   O^T       = diag-scaled S^T Q^T  (column a times lambda^(a+1))  [inter]
//             + V^T P^T                                         [intra]
//   S         = lambda^c S + K^T diag(lambda^(c-1-b)) V          [state scan]
// Every product is a bf16 x bf16 -> fp32 MFMA (v_mfma_f32_16x16x32_bf16).
// Scores, the bf16 copy of the state and the decay-weighted V are rounded to
// bf16 as MFMA operands; the state itself is accumulated and carried in fp32
// registers for the whole sequence and never rounded.
//
// Work split.  A (b, h) scan is sequential over blocks, and B*H is far below
// the 256 compute units, so each head's 128 state/output columns are split
// over 4 workgroups of 32 columns (the columns of S evolve independently).
// Each workgroup recomputes the block's scores (they need all of d); the
// four workgroups of a head are placed on one XCD so Q and K come from HBM
// once and from that XCD's L2 for the other three.
//
// Wave roles inside a workgroup (4 waves, 16x16 output tiles):
//   scores:  the 10 causal 16x16 tiles of P^T, 2-3 per wave;
//   output:  wave w owns tokens 16w..16w+15 of the block (both 16-col tiles);
//   state:   wave w owns rows (D/4) w .. of the 128 x 32 state slice.
// Operand layouts for v_mfma_f32_16x16x32_bf16 (lane l, l16 = l % 16,
// lg = l / 16): A row l16, k = 8 lg .. 8 lg + 7; B column l16, same k;
// result rows 4 lg + r (r = 0..3), column l16.  A and B are read with the
// same k pattern, so any consistent permutation of k inside an instruction
// leaves the products unchanged.
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int PC = 64;        // tokens per block
constexpr int PJ = 32;        // state / output columns per workgroup
constexpr int PT = 256;       // threads per workgroup (4 waves)
constexpr int PAD = 8;        // bf16 elements of row padding in LDS

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int W>
__device__ __forceinline__ const bf16x8 &frag(const uint16_t (*X)[W], int row, int col) {
    return *reinterpret_cast<const bf16x8 *>(&X[row][col]);
}

// 32-bit word from the low (sel 0) or high (sel 1) halves of two words:
// result = {x.half, y.half} with x in bits 0..15.
__device__ __forceinline__ uint32_t pick_lo(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pick_hi(uint32_t x, uint32_t y) {
    return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

template <int D>
struct alignas(16) Smem {
    uint16_t Q[PC][D + PAD];     // Q block, token-major
    uint16_t K[PC][D + PAD];     // K block, token-major
    uint16_t KT[D][PC + PAD];    // K block, feature-major (for the state update)
    uint16_t VT[PJ][PC + PAD];   // V slice, column-major (intra output)
    uint16_t VW[PJ][PC + PAD];   // V slice times lambda^(c-1-b), column-major
    uint16_t P[PC][PC + PAD];    // decayed causal scores P[a][b]
    uint16_t ST[PJ][D + PAD];    // bf16 copy of the state slice, transposed
};

// global -> register staging of one block (prefetched one block ahead)
template <int D>
struct Stage {
    static constexpr int NQ = PC * D / 8 / PT;            // 16-byte chunks of Q per thread
    static constexpr int NKTASK = (PC / 8) * (D / 4);     // 8x4 tiles of K
    static constexpr int NVTASK = (PC / 4) * (PJ / 4);    // 4x4 tiles of the V slice
    uint4 q[NQ];
    uint2 k[8];
    uint2 v[4];
};

template <int D>
__device__ __forceinline__ void stage_load(Stage<D> &st, const uint16_t *qb, const uint16_t *kb,
                                           const uint16_t *vb, int64_t t0, int64_t N, int j0,
                                           int tid)
{
#pragma unroll
    for (int u = 0; u < Stage<D>::NQ; ++u) {
        const int ch = tid + PT * u;
        const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
        st.q[u] = (t0 + row < N) ? *reinterpret_cast<const uint4 *>(qb + (t0 + row) * D + col)
                                 : make_uint4(0, 0, 0, 0);
    }
    if (tid < Stage<D>::NKTASK) {
        const int rg = tid / (D / 4), cg = tid % (D / 4);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int64_t t = t0 + 8 * rg + r;
            st.k[r] = (t < N) ? *reinterpret_cast<const uint2 *>(kb + t * D + 4 * cg)
                              : make_uint2(0, 0);
        }
    }
    const int vt = PT - 1 - tid;
    if (vt < Stage<D>::NVTASK) {
        const int rg = vt / (PJ / 4), cg = vt % (PJ / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = t0 + 4 * rg + r;
            st.v[r] = (t < N) ? *reinterpret_cast<const uint2 *>(vb + t * D + j0 + 4 * cg)
                              : make_uint2(0, 0);
        }
    }
}

// registers -> LDS, with the K transpose and the decay-weighted V copy.
// wv[r] = lambda^(c-1-b) for this thread's 4 tokens b (0 beyond the block).
template <int D>
__device__ __forceinline__ void stage_store(const Stage<D> &st, Smem<D> &sm, int tid,
                                            const float (&wv)[4])
{
#pragma unroll
    for (int u = 0; u < Stage<D>::NQ; ++u) {
        const int ch = tid + PT * u;
        const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
        *reinterpret_cast<uint4 *>(&sm.Q[row][col]) = st.q[u];
    }
    if (tid < Stage<D>::NKTASK) {
        const int rg = tid / (D / 4), cg = tid % (D / 4);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            *reinterpret_cast<uint2 *>(&sm.K[8 * rg + r][4 * cg]) = st.k[r];
        // column 4cg+e of rows 8rg..8rg+7 -> KT[4cg+e][8rg..8rg+7]
        uint4 c0, c1, c2, c3;
        c0.x = pick_lo(st.k[0].x, st.k[1].x); c0.y = pick_lo(st.k[2].x, st.k[3].x);
        c0.z = pick_lo(st.k[4].x, st.k[5].x); c0.w = pick_lo(st.k[6].x, st.k[7].x);
        c1.x = pick_hi(st.k[0].x, st.k[1].x); c1.y = pick_hi(st.k[2].x, st.k[3].x);
        c1.z = pick_hi(st.k[4].x, st.k[5].x); c1.w = pick_hi(st.k[6].x, st.k[7].x);
        c2.x = pick_lo(st.k[0].y, st.k[1].y); c2.y = pick_lo(st.k[2].y, st.k[3].y);
        c2.z = pick_lo(st.k[4].y, st.k[5].y); c2.w = pick_lo(st.k[6].y, st.k[7].y);
        c3.x = pick_hi(st.k[0].y, st.k[1].y); c3.y = pick_hi(st.k[2].y, st.k[3].y);
        c3.z = pick_hi(st.k[4].y, st.k[5].y); c3.w = pick_hi(st.k[6].y, st.k[7].y);
        *reinterpret_cast<uint4 *>(&sm.KT[4 * cg + 0][8 * rg]) = c0;
        *reinterpret_cast<uint4 *>(&sm.KT[4 * cg + 1][8 * rg]) = c1;
        *reinterpret_cast<uint4 *>(&sm.KT[4 * cg + 2][8 * rg]) = c2;
        *reinterpret_cast<uint4 *>(&sm.KT[4 * cg + 3][8 * rg]) = c3;
    }
    const int vt = PT - 1 - tid;
    if (vt < Stage<D>::NVTASK) {
        const int rg = vt / (PJ / 4), cg = vt % (PJ / 4);
        // V^T: column 4cg+e of rows 4rg..4rg+3
        uint2 t0, t1, t2, t3;
        t0.x = pick_lo(st.v[0].x, st.v[1].x); t0.y = pick_lo(st.v[2].x, st.v[3].x);
        t1.x = pick_hi(st.v[0].x, st.v[1].x); t1.y = pick_hi(st.v[2].x, st.v[3].x);
        t2.x = pick_lo(st.v[0].y, st.v[1].y); t2.y = pick_lo(st.v[2].y, st.v[3].y);
        t3.x = pick_hi(st.v[0].y, st.v[1].y); t3.y = pick_hi(st.v[2].y, st.v[3].y);
        *reinterpret_cast<uint2 *>(&sm.VT[4 * cg + 0][4 * rg]) = t0;
        *reinterpret_cast<uint2 *>(&sm.VT[4 * cg + 1][4 * rg]) = t1;
        *reinterpret_cast<uint2 *>(&sm.VT[4 * cg + 2][4 * rg]) = t2;
        *reinterpret_cast<uint2 *>(&sm.VT[4 * cg + 3][4 * rg]) = t3;
        // decay-weighted copy: element (token r, column e) times wv[r]
        float f[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f[r][0] = bf16_to_f32(st.v[r].x & 0xffffu) * wv[r];
            f[r][1] = bf16_to_f32(st.v[r].x >> 16) * wv[r];
            f[r][2] = bf16_to_f32(st.v[r].y & 0xffffu) * wv[r];
            f[r][3] = bf16_to_f32(st.v[r].y >> 16) * wv[r];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint2 w;
            w.x = pack_bf16x2(f[0][e], f[1][e]);
            w.y = pack_bf16x2(f[2][e], f[3][e]);
            *reinterpret_cast<uint2 *>(&sm.VW[4 * cg + e][4 * rg]) = w;
        }
    }
}

// Score tiles (bt, at) of P^T owned by wave W: the 10 causal 16x16 tiles of
// the 64x64 block, spread so that score + output MFMA counts balance.
template <int W> struct ScoreTiles;
template <> struct ScoreTiles<0> { static constexpr int n = 3; static constexpr int bt[3] = {0, 0, 3}, at[3] = {0, 3, 3}; };
template <> struct ScoreTiles<1> { static constexpr int n = 3; static constexpr int bt[3] = {0, 1, 1}, at[3] = {1, 1, 3}; };
template <> struct ScoreTiles<2> { static constexpr int n = 2; static constexpr int bt[3] = {0, 1, 0}, at[3] = {2, 2, 0}; };
template <> struct ScoreTiles<3> { static constexpr int n = 2; static constexpr int bt[3] = {2, 2, 0}, at[3] = {2, 3, 0}; };

// dec[dl][r]: decay of score element r of a tile whose token-tile offset is
// dl = at - bt, for this lane: lambda^(16 dl + l16 - 4 lg - r), 0 if negative.
template <int D, int W>
__device__ __forceinline__ void score_tiles(Smem<D> &sm, const float (&dec)[4][4], int l16, int lg)
{
    using T = ScoreTiles<W>;
#pragma unroll
    for (int u = 0; u < T::n; ++u) {
        const int bt = T::bt[u], at = T::at[u];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            acc = mfma(frag(sm.K, 16 * bt + l16, 32 * ks + 8 * lg),
                       frag(sm.Q, 16 * at + l16, 32 * ks + 8 * lg), acc);
        const int dl = at - bt;
        uint2 p;
        p.x = pack_bf16x2(acc[0] * dec[dl][0], acc[1] * dec[dl][1]);
        p.y = pack_bf16x2(acc[2] * dec[dl][2], acc[3] * dec[dl][3]);
        *reinterpret_cast<uint2 *>(&sm.P[16 * at + l16][16 * bt + 4 * lg]) = p;
    }
}

template <int D>
__global__ __launch_bounds__(PT) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ slopes,
    uint16_t *__restrict__ out, float *__restrict__ state, int64_t H, int64_t N)
{
    constexpr int NJ = D / PJ;            // workgroups per head
    constexpr int ITW = D / 64;           // 16-row state tiles per wave
    __shared__ Smem<D> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int l = tid % 64, l16 = l % 16, lg = l / 16;

    // XCD-aware placement: workgroup i runs on XCD i % 8; give the NJ
    // workgroups of one head consecutive logical ids on the same XCD.
    const int64_t nwg = gridDim.x;
    int64_t lid = blockIdx.x;
    if (nwg % 8 == 0) lid = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
    const int64_t bh = lid / NJ;
    const int j0 = (int)(lid % NJ) * PJ;
    const float s = slopes[bh % H];

    const uint16_t *qb = q + bh * N * D, *kb = k + bh * N * D, *vb = v + bh * N * D;
    uint16_t *ob = out + bh * N * D;
    float *St = state + bh * D * D;

    // per-lane decay constants
    float dec[4][4];
#pragma unroll
    for (int dl = 0; dl < 4; ++dl)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = 16 * dl + l16 - 4 * lg - r;
            dec[dl][r] = e < 0 ? 0.0f : decay_pow(s, e);
        }
    const float out_scale = decay_pow(s, 16 * w + l16 + 1);     // lambda^(a+1)
    const float full_decay = decay_pow(s, PC);                   // lambda^C
    const int vt = PT - 1 - tid;
    const int vrow = 4 * (vt / (PJ / 4));                          // first token of this thread's V rows
    float wfull[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) wfull[r] = decay_pow(s, PC - 1 - (vrow + r) < 0 ? 0 : PC - 1 - (vrow + r));

    // state slice in registers (fp32) and its bf16 transposed copy in LDS
    f32x4 sacc[ITW][2];
#pragma unroll
    for (int u = 0; u < ITW; ++u)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int it = w * ITW + u;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[u][jt][r] = St[(16 * it + 4 * lg + r) * D + j0 + 16 * jt + l16];
            uint2 p;
            p.x = pack_bf16x2(sacc[u][jt][0], sacc[u][jt][1]);
            p.y = pack_bf16x2(sacc[u][jt][2], sacc[u][jt][3]);
            *reinterpret_cast<uint2 *>(&sm.ST[16 * jt + l16][16 * it + 4 * lg]) = p;
        }
    // scores above the causal diagonal tiles are never written: zero them once
    for (int e = tid; e < PC * (PC + PAD) / 2; e += PT)
        reinterpret_cast<uint32_t *>(&sm.P[0][0])[e] = 0u;

    Stage<D> st;
    stage_load<D>(st, qb, kb, vb, 0, N, j0, tid);

    const int64_t nblk = (N + PC - 1) / PC;
    for (int64_t blk = 0; blk < nblk; ++blk) {
        const int64_t t0 = blk * PC;
        const int c = (int)min((int64_t)PC, N - t0);
        float wv[4];
        if (c == PC) {
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[r] = wfull[r];
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[r] = (vrow + r < c) ? decay_pow(s, c - 1 - (vrow + r)) : 0.0f;
        }
        stage_store<D>(st, sm, tid, wv);
        __syncthreads();                                   // block tiles visible
        if (blk + 1 < nblk) stage_load<D>(st, qb, kb, vb, t0 + PC, N, j0, tid);

        // intra-block scores
        switch (w) {
            case 0: score_tiles<D, 0>(sm, dec, l16, lg); break;
            case 1: score_tiles<D, 1>(sm, dec, l16, lg); break;
            case 2: score_tiles<D, 2>(sm, dec, l16, lg); break;
            default: score_tiles<D, 3>(sm, dec, l16, lg); break;
        }
        // inter-block output from the carried state: O^T = S^T Q^T, column a
        // scaled by lambda^(a+1); tokens 16w..16w+15
        f32x4 oacc[2];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            oacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                oacc[jt] = mfma(frag(sm.ST, 16 * jt + l16, 32 * ks + 8 * lg),
                                frag(sm.Q, 16 * w + l16, 32 * ks + 8 * lg), oacc[jt]);
            oacc[jt] *= out_scale;
        }
        // decayed state scan: S = lambda^c S + K^T (lambda^(c-1-b) V)
        const float sdec = (c == PC) ? full_decay : decay_pow(s, c);
#pragma unroll
        for (int u = 0; u < ITW; ++u)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                const int it = w * ITW + u;
                sacc[u][jt] *= sdec;
#pragma unroll
                for (int ks = 0; ks < PC / 32; ++ks)
                    sacc[u][jt] = mfma(frag(sm.KT, 16 * it + l16, 32 * ks + 8 * lg),
                                       frag(sm.VW, 16 * jt + l16, 32 * ks + 8 * lg), sacc[u][jt]);
            }
        __syncthreads();                                   // scores visible; old ST reads done

        // intra-block output: O^T += V^T P^T over tokens b < 16(w+1)
        const int nks = w / 2 + 1;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
            for (int ks = 0; ks < nks; ++ks)
                oacc[jt] = mfma(frag(sm.VT, 16 * jt + l16, 32 * ks + 8 * lg),
                                frag(sm.P, 16 * w + l16, 32 * ks + 8 * lg), oacc[jt]);
        const int a = 16 * w + l16;
        if (a < c) {
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                uint2 o;
                o.x = pack_bf16x2(oacc[jt][0], oacc[jt][1]);
                o.y = pack_bf16x2(oacc[jt][2], oacc[jt][3]);
                *reinterpret_cast<uint2 *>(ob + (t0 + a) * D + j0 + 16 * jt + 4 * lg) = o;
            }
        }
        // bf16 copy of the new state for the next block's inter term
#pragma unroll
        for (int u = 0; u < ITW; ++u)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                const int it = w * ITW + u;
                uint2 p;
                p.x = pack_bf16x2(sacc[u][jt][0], sacc[u][jt][1]);
                p.y = pack_bf16x2(sacc[u][jt][2], sacc[u][jt][3]);
                *reinterpret_cast<uint2 *>(&sm.ST[16 * jt + l16][16 * it + 4 * lg]) = p;
            }
        __syncthreads();                                   // new ST visible; tiles free
    }

#pragma unroll
    for (int u = 0; u < ITW; ++u)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int it = w * ITW + u;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                St[(16 * it + 4 * lg + r) * D + j0 + 16 * jt + l16] = sacc[u][jt][r];
        }
}

}  // namespace

int64_t prefill_bf16_grid(int64_t B, int64_t H, int d) { return B * H * (d / PJ); }

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *slopes, uint16_t *out, float *state,
                               int64_t B, int64_t H, int64_t N, int d, hipStream_t stream)
{
    const dim3 grid((unsigned)prefill_bf16_grid(B, H, d)), block(PT);
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                    (void *)&out, (void *)&state, (void *)&H, (void *)&N};
    const void *fn = d == 64 ? (const void *)prefill_bf16_kernel<64>
                             : (const void *)prefill_bf16_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace la
