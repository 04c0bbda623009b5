// prefill_f32.hip — blockwise decayed linear attention with fp32 activations.
//
// The block decomposition of the bf16 kernel with every product on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 accumulation; the
// fp32 path keeps full fp32 operands, rounding them to bf16 would cost more
// accuracy than fp32 callers expect).  For one (b, h) and the block of c
// tokens starting at t0 (local a, b < c):
//   P[a][b] = lambda^(a-b) (q_a . k_b)              for b <= a, else 0
//   O[a]    = sum_b P[a][b] v_b + lambda^(a+1) q_a S
//   S       = lambda^c S + sum_b lambda^(c-1-b) k_b^T v_b
// This is the report's split into a local output and a local state per
// sequence piece, joined through the carried [B,H,D,D] state (Ling and Ring
// 2.6 Technical Report, §4.1.1 and Fig. 10), applied block after block.
//
// One workgroup per (sequence, head, 32-column slice of v/S/O) of a dense or
// packed launch, one wave per 32-row tile of the state (D/32 waves), blocks of
// 32 tokens.  Wave t keeps state rows 32t..32t+31 of the slice in registers
// (accumulator layout: lane (column j, half h), register r holds row
// 8 (r/4) + 4h + r%4 of the tile) and per block computes, for its 32
// features, the partial scores S^T = K_t Q_t^T and the partial inter term
// S_t^T Q_t^T (both with Q_t^T as the B operand: the state registers are the
// A operand as they stand), then its state tile's update K_t^T (lambda-
// weighted V).  The partial scores of the D/32 waves are summed through LDS,
// masked and decayed; each wave multiplies V^T by its share of the token rows
// of P^T into its partial output, and the partial outputs are summed through
// LDS (token-major, 16-byte accesses) and stored, 128 bytes per token row.
// The next block's q, k and v are loaded into registers while a block is
// computed; v is double-buffered, q and k single (read only before a block's
// first barrier, the next block's are staged right after it), the partials
// single too (each is read between the barriers that follow its writes and
// written again only after every reader has passed the next block's first
// barrier); the decay factors of a full block are kept in registers.  (Two
// waves per state tile,
// one for the scores and one for the state, measured slower at 64 heads:
// 3.96 against 3.36 ms at 32K tokens.)
#include "la_internal.h"

#include <algorithm>

namespace la {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int FC = 32;      // tokens per block
constexpr int FJ = 32;      // state / output columns per workgroup
constexpr int RP = 4;       // row padding of the LDS tiles (floats)

template <int D>
struct alignas(16) F32Smem {
    float Q[FC][D + RP];                 // (single: read only before a block's first barrier)
    float K[FC][D + RP];
    float V[2][FC][FJ + RP];
    float P[D / 32][FC][FC + RP];        // partial scores of each feature tile, [b][a]
    float O[D / 32][FC][FJ + RP];        // partial outputs of each wave, [a][j]
    float pw[FC + 1];                    // lambda^n, n = 0..FC
};

// contraction index of MFMA step m for lane half h (and the accumulator row of
// register m): 8 (m/4) + 4h + m%4 covers 0..31 once over m = 0..15, h = 0, 1
__device__ __forceinline__ int kk(int m, int h) { return 8 * (m >> 2) + 4 * h + (m & 3); }

__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// (d = 128: registers for two workgroups per CU, which the 80 KB of LDS allow:
// on grids of more than one workgroup per CU, 2.95 -> 2.25 ms for 2 x 16K
// tokens at 64 heads)
template <int D>
__global__ __launch_bounds__(64 * (D / 32), D == 128 ? 2 : 1) void prefill_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ slopes, float *__restrict__ out, float *__restrict__ state,
    SeqMap map)
{
    constexpr int NT = D / 32;                  // feature tiles = waves
    constexpr int NTH = 64 * NT;                // threads
    constexpr int NJ = D / FJ;                  // workgroups per head
    constexpr int NQ = FC * D / 4 / NTH;        // float4 of a q (k) block per thread
    constexpr int NV = FC * FJ / 4 / NTH;       // float4 of a v block slice per thread
    constexpr int BQ = FC / NT;                 // token rows of P^T (and output tokens) per wave
    __shared__ F32Smem<D> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, l32 = lane % 32, h = lane / 32;

    // XCD-aware placement as in the bf16 kernel: the NJ slices of one
    // (sequence, head) run on one XCD at once (q and k from HBM once, then
    // from that XCD's L2), consecutive heads on different XCDs
    const int64_t nbh = gridDim.x / NJ;
    int64_t bh, slice;
    if (nbh % 8 == 0) {
        const int64_t q8 = blockIdx.x / 8;
        bh = (q8 / NJ) * 8 + blockIdx.x % 8;
        slice = q8 % NJ;
    } else {
        bh = blockIdx.x / NJ;
        slice = blockIdx.x % NJ;
    }
    const int j0 = (int)slice * FJ;
    const int64_t hd = bh % map.H;
    const float s = slopes[hd];
    int64_t in0, out0, N;
    seq_slice(map, bh / map.H, hd, &in0, &out0, &N);
    const int64_t ts = map.in.st, ots = map.out.st;   // token strides (elements)
    const float *qb = q + in0, *kb = k + in0, *vb = v + in0;
    float *ob = out + out0;
    if (tid <= FC) sm.pw[tid] = decay_pow(s, tid);

    float *St = state + bh * D * D;
    f32x16 S;                                   // state rows 32 wave + kk(r, h), column j0 + l32
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = St[(32 * wave + kk(r, h)) * D + j0 + l32];

    float4 pq[NQ], pk[NQ], pv[NV];
    auto load = [&](int64_t t0, int c) {        // rows c.. of the block read as zeros
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int e = tid + NTH * u, row = e / (D / 4), c4 = e % (D / 4);
            pq[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            pk[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < c) {
                pq[u] = *reinterpret_cast<const float4 *>(qb + (t0 + row) * ts + 4 * c4);
                pk[u] = *reinterpret_cast<const float4 *>(kb + (t0 + row) * ts + 4 * c4);
            }
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int e = tid + NTH * u, row = e / (FJ / 4), c4 = e % (FJ / 4);
            pv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < c) pv[u] = *reinterpret_cast<const float4 *>(vb + (t0 + row) * ts + j0 + 4 * c4);
        }
    };
    auto stage_qk = [&]() {
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
            const int e = tid + NTH * u, row = e / (D / 4), c4 = e % (D / 4);
            *reinterpret_cast<float4 *>(&sm.Q[row][4 * c4]) = pq[u];
            *reinterpret_cast<float4 *>(&sm.K[row][4 * c4]) = pk[u];
        }
    };
    auto stage_v = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int e = tid + NTH * u, row = e / (FJ / 4), c4 = e % (FJ / 4);
            *reinterpret_cast<float4 *>(&sm.V[buf][row][4 * c4]) = pv[u];
        }
    };

    const int64_t nblk = (N + FC - 1) / FC;
    if (nblk > 0) {
        load(0, (int)min((int64_t)FC, N));
        stage_qk();
        stage_v(0);
    }
    __syncthreads();                            // block 0 and the powers visible
    // per-lane decay factors of a full block: lambda^(a+1) of token a = l32, the
    // weights lambda^(FC-1-b) of the state update's rows b = kk(m, h), the
    // masked lambda^(a-b) of this wave's rows b of P^T, lambda^FC
    const float lam_a1 = sm.pw[l32 + 1], lam_c = sm.pw[FC];
    float vws[16], pmask[BQ / 2];
#pragma unroll
    for (int m = 0; m < 16; ++m) vws[m] = sm.pw[FC - 1 - kk(m, h)];
#pragma unroll
    for (int m = 0; m < BQ / 2; ++m) {
        const int b = BQ * wave + (BQ / 2) * h + m;
        pmask[m] = b <= l32 ? sm.pw[l32 - b] : 0.0f;
    }
    for (int64_t n = 0; n < nblk; ++n) {
        const int buf = (int)(n & 1);
        const int64_t t0 = n * FC;
        const int c = (int)min((int64_t)FC, N - t0);
        // the next block into registers (after the last block: no rows, no
        // accesses).  Unconditional, as is the staging below: with both under
        // a condition the compiler takes the loads as possibly still in flight
        // at the top of the next block and waits there, and since loads and
        // stores share one counter that wait also took the previous block's
        // output stores (3.36 -> 3.06 ms at 64 heads, 32K tokens)
        load(t0 + FC, (int)min((int64_t)FC, N - t0 - FC));

        // partial scores S^T[b][a] and inter term over features 32 wave .. +31:
        // A = K[b][k] (lane b) and S^T[j][k] (the state registers), B = Q^T[k][a] (lane a)
        float qa[16], ka[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 x = *reinterpret_cast<const float4 *>(&sm.Q[l32][32 * wave + 8 * g + 4 * h]);
            const float4 y = *reinterpret_cast<const float4 *>(&sm.K[l32][32 * wave + 8 * g + 4 * h]);
            qa[4 * g] = x.x; qa[4 * g + 1] = x.y; qa[4 * g + 2] = x.z; qa[4 * g + 3] = x.w;
            ka[4 * g] = y.x; ka[4 * g + 1] = y.y; ka[4 * g + 2] = y.z; ka[4 * g + 3] = y.w;
        }
        f32x16 sc = {}, oc = {};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            sc = mfma(ka[m], qa[m], sc);
            oc = mfma(S[m], qa[m], oc);
        }
        oc *= lam_a1;                           // lambda^(a+1) for token a = l32
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.P[wave][kk(r, h)][l32] = sc[r];
        // (all operands read before the chain: its 16 MFMAs depend on each
        // other, so a read per step would put the LDS latency between them)
        float kt[16], vw[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int b = kk(m, h);
            kt[m] = sm.K[b][32 * wave + l32];
            vw[m] = sm.V[buf][b][l32];
        }
        if (c == FC) {
            S *= lam_c;
#pragma unroll
            for (int m = 0; m < 16; ++m) S = mfma(kt[m], vw[m] * vws[m], S);
        } else {                                // the last, partial block (rows b >= c are 0)
            S *= sm.pw[c];
#pragma unroll
            for (int m = 0; m < 16; ++m) S = mfma(kt[m], vw[m] * sm.pw[max(c - 1 - kk(m, h), 0)], S);
        }

        stage_v(buf ^ 1);                       // (after the last block: unused zeros)
        __syncthreads();                        // partial scores visible; q, k of this block read
        stage_qk();                             // the next block's q, k (visible after the next barrier)

        // this wave's token rows b of P^T (summed, masked, decayed) times V^T:
        // A = V^T[j][b] (lane j), B = P^T[b][a] (lane a)
#pragma unroll
        for (int m = 0; m < BQ / 2; ++m) {
            const int b = BQ * wave + (BQ / 2) * h + m;
            float p = 0.0f;
#pragma unroll
            for (int t = 0; t < NT; ++t) p += sm.P[t][b][l32];
            oc = mfma(sm.V[buf][b][l32], p * pmask[m], oc);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4 *>(&sm.O[wave][l32][8 * g + 4 * h]) =
                make_float4(oc[4 * g], oc[4 * g + 1], oc[4 * g + 2], oc[4 * g + 3]);
        __syncthreads();                        // partial outputs visible

        // the outputs of this wave's tokens: 8 lanes per token row, 16 bytes each
#pragma unroll
        for (int pass = 0; pass < BQ / 8; ++pass) {
            const int a = BQ * wave + 8 * pass + lane / 8, j = 4 * (lane % 8);
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float4 x = *reinterpret_cast<const float4 *>(&sm.O[t][a][j]);
                o.x += x.x; o.y += x.y; o.z += x.z; o.w += x.w;
            }
            if (a < c) *reinterpret_cast<float4 *>(ob + (t0 + a) * ots + j0 + j) = o;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) St[(32 * wave + kk(r, h)) * D + j0 + l32] = S[r];
}

}  // namespace

int64_t prefill_f32_grid(int64_t seqs, int64_t H, int d) { return seqs * H * (d / FJ); }

// A dense fp32 prefill over B = 1 can run as S >= 2 segments of the sequence
// at once (the later ones from a zero state, then the fold of the segments'
// states and the correction of the later segments' outputs, as the bf16 split
// does), so that the grid holds the two workgroups per CU the kernel's
// registers and LDS allow (64 heads of 128 channels: 256 workgroups unsplit,
// 512 in two segments; on such grids 2.95 -> 2.25 ms for 32K tokens).  Each
// segment at least F32_SPLIT_MIN_LEN tokens, at most 64 segments.
constexpr int64_t F32_SPLIT_MIN_LEN = 8192;

int prefill_f32_split_plan(int64_t B, int64_t H, int64_t N, int d)
{
    if (B != 1 || H < 1 || N < 2 * F32_SPLIT_MIN_LEN) return 1;
    const int cus = device_cus();
    if (cus <= 0) return 1;
    const int64_t wg = H * (d / FJ);
    int64_t S = std::min<int64_t>(2 * (int64_t)cus / wg, N / F32_SPLIT_MIN_LEN);
    S = std::min<int64_t>(S, 64);
    return S >= 2 ? (int)S : 1;
}

hipError_t launch_prefill_f32(const float *q, const float *k, const float *v,
                              const float *slopes, float *out, float *state,
                              int64_t seqs, const SeqMap &map, int d, hipStream_t stream)
{
    const dim3 grid((unsigned)prefill_f32_grid(seqs, map.H, d)), block(64 * (d / 32));
    SeqMap m = map;
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                    (void *)&out, (void *)&state, (void *)&m};
    const void *fn = d == 64 ? (const void *)prefill_f32_kernel<64>
                             : (const void *)prefill_f32_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

// ---- the sequence split for fp32 q, k, v, out (B = 1, dense [1,H,N,d]): the
// segments on the kernel above, the bf16 split's prep and fold (cp.hip), and
// the correction in fp32 on the fp32 matrix cores.

namespace {

constexpr int FCT = 32;            // fp32 correction: tokens per tile
constexpr int FCW = 64;            // fp32 correction: walkers per (segment, head), at most

// out_a += lambda^(a+1) q_a S for token a of a later segment (S its starting
// state), fp32 operands and accumulation (v_mfma_f32_32x32x2_f32): one
// workgroup per (segment, head, walker), wave w owning output columns
// 32w .. 32w + 31 and holding those columns of S for all D rows as B operands
// (lane = column j, k = lane / 32, row 32t + 8 (m/4) + 4k + m%4 of step (t, m)).
// A 32-token tile is (Q S)[a][j] = sum over the D rows in D/2 MFMAs, the A
// operand Q[a = lane % 32][row] read straight from memory (the waves of a
// workgroup read the same rows, the caches serve the repeats); the result
// (lane = column, register r = token row 8 (r/4) + 4 (lane/32) + r%4) is added
// to out with 128-byte row accesses.  No LDS, no barriers.  A head's tiles are
// those before the first whose first factor lambda^(32 i + 1) is 0 in fp32
// (found by bisection: the factor only falls; nothing after it changes), cut
// into W contiguous runs, one per walker.  The split's layout is dense, token
// rows D floats apart, so a tile's addresses share one base; each 32-row
// slice t of the q operands is loaded right before its 16 products (the
// scheduling barrier keeps the compiler from hoisting all D/2 values' loads),
// which leaves registers for three waves per SIMD.
template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void cp_correct_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ slopes, const float *__restrict__ s_in,
    float *__restrict__ out, int64_t H, int64_t hs, int64_t t_off, int64_t seg, int64_t ntok,
    int64_t W)
{
    constexpr int NT = D / 32;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, l32 = lane % 32, h = lane / 32;
    const int64_t walker = blockIdx.x % W, rest = blockIdx.x / W;
    const int64_t hd = rest % H, g = rest / H;
    const float s = slopes[hd];
    const int64_t a0 = t_off + g * seg;                       // the segment's first token
    const int64_t L = max((int64_t)0, min(seg, ntok - a0));   // its tokens
    int64_t lo = 0, hi = (L + FCT - 1) / FCT;                 // first tile with a zero factor
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (decay_pow(s, (int)(mid * FCT + 1)) == 0.0f) hi = mid; else lo = mid + 1;
    }
    const int64_t per = (lo + W - 1) / W;
    const int64_t i0 = walker * per, i1 = min(lo, i0 + per);
    if (i0 >= i1) return;

    const float *S = s_in + (g * H + hd) * D * D + 32 * wave + l32;
    float sb[NT][16];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int m = 0; m < 16; ++m) sb[t][m] = S[(32 * t + kk(m, h)) * D];
    const float *qb = q + hd * hs + a0 * D + 4 * h;
    float *ob = out + hd * hs + a0 * D + 32 * wave + l32;
    for (int64_t i = i0; i < i1; ++i) {
        const int64_t t0 = i * FCT;
        const int c = (int)min((int64_t)FCT, L - t0);
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            y[r] = 0.f;
            if (kk(r, h) < c) y[r] = ob[(t0 + kk(r, h)) * D];
        }
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float4 qa[4];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                qa[gq] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (l32 < c)
                    qa[gq] = *reinterpret_cast<const float4 *>(qb + (t0 + l32) * D + 32 * t + 8 * gq);
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float4 x = qa[m >> 2];
                const float av = (m & 3) == 0 ? x.x : (m & 3) == 1 ? x.y : (m & 3) == 2 ? x.z : x.w;
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, sb[t][m], acc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int a = kk(r, h);
            if (a < c) ob[(t0 + a) * D] = fmaf(decay_pow(s, (int)(t0 + a + 1)), acc[r], y[r]);
        }
    }
}

}  // namespace

hipError_t launch_prefill_f32_split(const float *q, const float *k, const float *v,
                                    const float *slopes, float *out, float *state, int64_t H,
                                    int64_t N, int d, int nseg, void *workspace,
                                    hipStream_t stream)
{
    float *slots = static_cast<float *>(workspace);
    const int64_t seg = split_segment(N, nseg);
    int64_t *cu = nullptr;
    hipError_t e = launch_split_prep(state, slots, &cu, H, d, nseg, seg, N, stream);
    if (e != hipSuccess) return e;
    const Strides st = {0, N * d, d};
    const SeqMap map = {cu, H, 0, N, st, st};
    e = launch_prefill_f32(q, k, v, slopes, out, slots, nseg, map, d, stream);
    if (e != hipSuccess) return e;
    e = launch_split_fold(slots, state, slopes, H, d, nseg, seg, N, stream);
    if (e != hipSuccess) return e;
    // segment g >= 1 is corrected with slot g - 1 (the state at its start), by
    // about 4096 workgroups in all, at most FCW per segment and head
    const int64_t W = std::max<int64_t>(1, std::min<int64_t>(FCW, 4096 / ((nseg - 1) * H)));
    const dim3 grid((unsigned)((nseg - 1) * H * W)), block(64 * (d / 32));
    int64_t hh = H, hs = N * d, toff = seg, sg = seg, nt = N, w = W;
    void *args[] = {(void *)&q, (void *)&slopes, (void *)&slots, (void *)&out, (void *)&hh,
                    (void *)&hs, (void *)&toff, (void *)&sg, (void *)&nt, (void *)&w};
    const void *fn = d == 64 ? (const void *)cp_correct_f32_kernel<64>
                             : (const void *)cp_correct_f32_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace la
