// prefill_bf16.hip — blockwise decayed causal linear attention, bf16
// activations, fp32 accumulation, gfx950 matrix cores.
//
// Method (Ling and Ring 2.6 Technical Report, §4.1.1 and Fig. 10: a local
// output from the tokens of a piece plus a correction from the state carried
// in from everything before it; here the pieces are 64-token blocks handled
// in order inside one workgroup).  For one (b, h), the block of c tokens at
// t0, local indices a, b < c and lambda = exp(-slope_h):
//   P^T[b][a] = lambda^(a-b) (k_b . q_a)  (b <= a), else 0      [intra scores]
//   O^T       = S^T Q^T with column a scaled by lambda^(a+1)      [inter]
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
// Data movement (wave-specialised).  Waves 4..7 are producers: they only
// load Q, K and the workgroup's 64 x 32 slice of V with 16-byte buffer loads,
// four blocks ahead of use (four register sets), and write them into one of
// two LDS buffers one block ahead (plus a decay-weighted copy of V).  Waves
// 0..3 are consumers: they only read LDS, run the MFMAs and store outputs.
// Keeping global loads and stores in different waves matters on gfx9: one
// counter (vmcnt) tracks both, and a wave with both kinds in flight must
// drain all of them before it can use any loaded register.  Contractions
// over tokens (the state update K^T V and the intra output V^T P^T) need the
// token index contiguous per lane; they read K and V from their token-major
// LDS tiles with ds_read_b64_tr_b16 (gfx950 transposing LDS read) instead of
// keeping transposed copies.  K's 16-byte chunks are XOR-swizzled by row so
// that both its plain reads (8 rows, one chunk) and its transposed reads
// (4 rows, one chunk pair) hit distinct LDS banks.
//
// Consumer wave roles (4 waves, 16x16 output tiles):
//   scores:  the 10 causal 16x16 tiles of P^T, 2-3 per wave;
//   output:  wave w owns tokens 16w..16w+15 of the block (both 16-col tiles);
//   state:   wave w owns rows (D/4) w .. of the D x 32 state slice.
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, l16 = l % 16,
// lg = l / 16): A row l16, k = 8 lg .. 8 lg + 7; B column l16, same k;
// result rows 4 lg + r (r = 0..3), column l16.
// ds_read_b64_tr_b16: within each 16-lane group, lane l16 supplies the
// address of a 4-element chunk; lane l16 receives element l16 % 4 of chunks
// 4e + l16 / 4, e = 0..3.  So if lane l16 points at row r0 + l16/4, column
// c0 + 4 (l16 % 4) of a row-major tile, it receives column c0 + l16 of rows
// r0 .. r0 + 3: a k-contiguous MFMA operand for a contraction over rows.
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int PC = 64;        // tokens per block
constexpr int PJ = 32;        // state / output columns per workgroup
constexpr int PT = 256;       // threads per role (4 consumer + 4 producer waves)
constexpr int NSET = 4;       // producer register sets (blocks in flight)
constexpr int QPAD = 8;       // bf16 padding of Q and state-copy rows
constexpr int VP = 48;        // V row pitch (96 B: transposed reads conflict-free)
constexpr int PP = PC + 8;    // score row pitch

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// two transposing reads -> one 8-element operand (k = 0..3 from p0, 4..7 from p1)
__device__ __forceinline__ bf16x8 ldtr8(const uint16_t *p0, const uint16_t *p1) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
    const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, c);
}

// 16-byte-chunk swizzle of K rows (see the header comment)
__device__ __forceinline__ int kswz(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }

template <int D>
struct alignas(16) Smem {
    uint16_t Q[2][PC][D + QPAD];     // Q blocks, token-major
    uint16_t K[2][PC][D];            // K blocks, token-major, chunk-swizzled
    uint16_t V[2][PC][VP];           // V slices, token-major
    uint16_t VW[2][PC][VP];          // V slices times lambda^(c-1-b)
    uint16_t P[PC][PP];              // decayed causal scores P[a][b]
    uint16_t ST[PJ][D + QPAD];       // bf16 copy of the state slice, transposed
};

// one block's share of this thread, in registers
template <int D>
struct Regs {
    static constexpr int NQ = PC * D / 8 / PT;   // 16-byte chunks of Q (and of K)
    uint4 q[NQ], k[NQ], v;
};

template <int D>
struct Addr {                        // per-thread byte offsets inside a block
    uint32_t qk[Regs<D>::NQ];
    uint32_t v;
};

// Buffer resource over rows [t0, t0 + 64) of a (b, h) slice: 16-byte loads
// at per-thread offsets, rows past N read as zero (hardware range check on
// the descriptor's byte count), stores past N are dropped.
constexpr uint32_t RSRC_WORD3 = 0x00020000u;   // raw buffer, 32-bit data format

// tokens of the block starting at t0 (0 past the end)
__device__ __forceinline__ int block_len(int64_t t0, int64_t N) {
    return (int)max((int64_t)0, min((int64_t)PC, N - t0));
}

template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t *base, int64_t t0,
                                                              int64_t N)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)(base + t0 * D), (short)0,
                                             block_len(t0, N) * D * 2, RSRC_WORD3);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

template <int D>
__device__ __forceinline__ void load_block(Regs<D> &r, const uint16_t *qh, const uint16_t *kh,
                                           const uint16_t *vh, int64_t t0, int64_t N,
                                           const Addr<D> &ad)
{
    const __amdgpu_buffer_rsrc_t rq = block_rsrc<D>(qh, t0, N);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(kh, t0, N);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(vh, t0, N);
#pragma unroll
    for (int u = 0; u < Regs<D>::NQ; ++u) {
        r.q[u] = bload16(rq, ad.qk[u]);
        r.k[u] = bload16(rk, ad.qk[u]);
    }
    r.v = bload16(rv, ad.v);
}

__device__ __forceinline__ uint32_t scale_pair(uint32_t x, float w) {
    return pack_bf16x2(bf16_to_f32(x & 0xffffu) * w, bf16_to_f32(x >> 16) * w);
}

// registers -> LDS buffer BUF; wv = lambda^(c-1-b) for this thread's token b
template <int D, int BUF>
__device__ __forceinline__ void store_block(const Regs<D> &r, Smem<D> &sm, int tid, float wv)
{
#pragma unroll
    for (int u = 0; u < Regs<D>::NQ; ++u) {
        const int ch = tid + PT * u;
        const int row = ch / (D / 8), c8 = ch % (D / 8);
        *reinterpret_cast<uint4 *>(&sm.Q[BUF][row][c8 * 8]) = r.q[u];
        *reinterpret_cast<uint4 *>(&sm.K[BUF][row][(c8 ^ kswz(row)) * 8]) = r.k[u];
    }
    const int vrow = tid / 4, vc = (tid % 4) * 8;
    *reinterpret_cast<uint4 *>(&sm.V[BUF][vrow][vc]) = r.v;
    uint4 w;
    w.x = scale_pair(r.v.x, wv);
    w.y = scale_pair(r.v.y, wv);
    w.z = scale_pair(r.v.z, wv);
    w.w = scale_pair(r.v.w, wv);
    *reinterpret_cast<uint4 *>(&sm.VW[BUF][vrow][vc]) = w;
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
template <int D, int W, int BUF>
__device__ __forceinline__ void score_tiles(Smem<D> &sm, const float (&dec)[4][4], int l16, int lg)
{
    using T = ScoreTiles<W>;
    const int ks0 = kswz(l16);
#pragma unroll
    for (int u = 0; u < T::n; ++u) {
        const int bt = T::bt[u], at = T::at[u];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            acc = mfma(ld8(&sm.K[BUF][16 * bt + l16][((4 * ks + lg) ^ ks0) * 8]),
                       ld8(&sm.Q[BUF][16 * at + l16][32 * ks + 8 * lg]), acc);
        const int dl = at - bt;
        uint2 p;
        p.x = pack_bf16x2(acc[0] * dec[dl][0], acc[1] * dec[dl][1]);
        p.y = pack_bf16x2(acc[2] * dec[dl][2], acc[3] * dec[dl][3]);
        *reinterpret_cast<uint2 *>(&sm.P[16 * at + l16][16 * bt + 4 * lg]) = p;
    }
}

template <int D>
struct Ctx {                          // per-thread constants of one workgroup
    const uint16_t *qh, *kh, *vh;     // this (b, h) slice
    const uint16_t *oh;
    int64_t N, nblk;                  // nblk: blocks processed (a multiple of NSET)
    float s, full_decay, out_scale, wfull;
    float dec[4][4];
    int w, l16, lg, j0;
};

// ---- producer waves (4..7): global -> registers -> LDS --------------------

// stage block blk (register set r) into LDS buffer BUF
template <int D, int BUF>
__device__ __forceinline__ void produce_store(const Ctx<D> &cx, Smem<D> &sm, const Regs<D> &r,
                                              int64_t blk, int p)
{
    const int c = block_len(blk * PC, cx.N);
    const int b = p / 4;
    const float wv = c == PC ? cx.wfull : (b < c ? decay_pow(cx.s, c - 1 - b) : 0.0f);
    store_block<D, BUF>(r, sm, p, wv);
}

// One producer step per block blk: after the block's first barrier, stage
// block blk+1 (register set SET) into the other LDS buffer, then reload SET
// with block blk+1+NSET.  Loads past the end return zeros without touching
// memory, so nothing here is conditional (exact vmcnt waits).
template <int D, int SET>
__device__ __forceinline__ void produce_step(const Ctx<D> &cx, Smem<D> &sm, Regs<D> (&rs)[NSET],
                                             const Addr<D> &ad, int64_t blk, int p)
{
    __syncthreads();                                   // B1 of block blk
    if (SET % 2 == 1) produce_store<D, 1>(cx, sm, rs[SET], blk + 1, p);   // blk even -> buffer 1
    else              produce_store<D, 0>(cx, sm, rs[SET], blk + 1, p);
    load_block<D>(rs[SET], cx.qh, cx.kh, cx.vh, (blk + 1 + NSET) * PC, cx.N, ad);
    __syncthreads();                                   // B2 of block blk
}

template <int D>
__device__ void producer(const Ctx<D> &cx, Smem<D> &sm, int p)
{
    Addr<D> ad;
#pragma unroll
    for (int u = 0; u < Regs<D>::NQ; ++u) {
        const int ch = p + PT * u;
        ad.qk[u] = (uint32_t)(((ch / (D / 8)) * D + (ch % (D / 8)) * 8) * 2);
    }
    ad.v = (uint32_t)(((p / 4) * D + cx.j0 + (p % 4) * 8) * 2);

    Regs<D> rs[NSET];                                   // set i holds block i (mod NSET)
#pragma unroll
    for (int i = 0; i < NSET; ++i) load_block<D>(rs[i], cx.qh, cx.kh, cx.vh, i * PC, cx.N, ad);
    produce_store<D, 0>(cx, sm, rs[0], 0, p);
    load_block<D>(rs[0], cx.qh, cx.kh, cx.vh, NSET * PC, cx.N, ad);

    // block blk stages block blk+1 from set (blk+1) % NSET into buffer (blk+1) % 2
    for (int64_t blk = 0; blk < cx.nblk; blk += NSET) {
        produce_step<D, 1>(cx, sm, rs, ad, blk + 0, p);
        produce_step<D, 2>(cx, sm, rs, ad, blk + 1, p);
        produce_step<D, 3>(cx, sm, rs, ad, blk + 2, p);
        produce_step<D, 0>(cx, sm, rs, ad, blk + 3, p);
    }
}

// ---- consumer waves (0..3): scores, outputs, state scan ---------------------

// one 64-token block held in LDS buffer BUF
template <int D, int BUF>
__device__ __forceinline__ void consume_step(const Ctx<D> &cx, Smem<D> &sm, int64_t blk,
                                             f32x4 (&sacc)[D / 64][2])
{
    constexpr int ITW = D / 64;
    const int w = cx.w, l16 = cx.l16, lg = cx.lg;
    const int64_t t0 = blk * PC;
    const int c = block_len(t0, cx.N);

    __syncthreads();          // B1: buffer BUF staged; previous block fully consumed

    // intra-block scores
    switch (w) {
        case 0: score_tiles<D, 0, BUF>(sm, cx.dec, l16, lg); break;
        case 1: score_tiles<D, 1, BUF>(sm, cx.dec, l16, lg); break;
        case 2: score_tiles<D, 2, BUF>(sm, cx.dec, l16, lg); break;
        default: score_tiles<D, 3, BUF>(sm, cx.dec, l16, lg); break;
    }
    // inter-block output from the carried state: O^T = S^T Q^T, column a
    // scaled by lambda^(a+1); tokens 16w..16w+15
    f32x4 oacc[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
        oacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
            oacc[jt] = mfma(ld8(&sm.ST[16 * jt + l16][32 * ks + 8 * lg]),
                            ld8(&sm.Q[BUF][16 * w + l16][32 * ks + 8 * lg]), oacc[jt]);
        oacc[jt] *= cx.out_scale;
    }
    // decayed state scan: S = lambda^c S + K^T (lambda^(c-1-b) V)
    const float sdec = (c == PC) ? cx.full_decay : decay_pow(cx.s, c);   // 1 for an empty block
    const int trow = l16 >> 2;                 // row within a 4-row transposed read
    const int tcol = 4 * (l16 & 3);            // column offset within a 16-column tile
#pragma unroll
    for (int u = 0; u < ITW; ++u) {
        const int it = w * ITW + u;
        bf16x8 ka[PC / 32];
#pragma unroll
        for (int ks = 0; ks < PC / 32; ++ks) {
            const int r0 = 32 * ks + 8 * lg + trow;
            const int ch = 2 * it + ((l16 & 3) >> 1), sub = 4 * (l16 & 1);
            ka[ks] = ldtr8(&sm.K[BUF][r0][((ch ^ kswz(r0)) * 8) + sub],
                           &sm.K[BUF][r0 + 4][((ch ^ kswz(r0 + 4)) * 8) + sub]);
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            sacc[u][jt] *= sdec;
#pragma unroll
            for (int ks = 0; ks < PC / 32; ++ks) {
                const int r0 = 32 * ks + 8 * lg + trow;
                sacc[u][jt] = mfma(ka[ks],
                                   ldtr8(&sm.VW[BUF][r0][16 * jt + tcol],
                                         &sm.VW[BUF][r0 + 4][16 * jt + tcol]),
                                   sacc[u][jt]);
            }
        }
    }
    __syncthreads();          // B2: scores visible; reads of the old state copy done

    // intra-block output: O^T += V^T P^T over tokens b < 16(w+1)
#pragma unroll
    for (int ks = 0; ks < PC / 32; ++ks) {
        if (ks > w / 2) break;
        const int r0 = 32 * ks + 8 * lg + trow;
        const bf16x8 pb = ld8(&sm.P[16 * w + l16][32 * ks + 8 * lg]);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
            oacc[jt] = mfma(ldtr8(&sm.V[BUF][r0][16 * jt + tcol], &sm.V[BUF][r0 + 4][16 * jt + tcol]),
                            pb, oacc[jt]);
    }
    {   // rows past N are dropped by the descriptor's range check
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const __amdgpu_buffer_rsrc_t ro = block_rsrc<D>(cx.oh, t0, cx.N);
        const int a = 16 * w + l16;
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            u32x2 o;
            o[0] = pack_bf16x2(oacc[jt][0], oacc[jt][1]);
            o[1] = pack_bf16x2(oacc[jt][2], oacc[jt][3]);
            __builtin_amdgcn_raw_buffer_store_b64(o, ro, (a * D + cx.j0 + 16 * jt + 4 * lg) * 2, 0, 0);
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
}

template <int D>
__device__ void consumer(Ctx<D> &cx, Smem<D> &sm, float *St, int tid)
{
    constexpr int ITW = D / 64;
    const int w = cx.w, l16 = cx.l16, lg = cx.lg;
    // per-lane decay constants
#pragma unroll
    for (int dl = 0; dl < 4; ++dl)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = 16 * dl + l16 - 4 * lg - r;
            cx.dec[dl][r] = e < 0 ? 0.0f : decay_pow(cx.s, e);
        }
    cx.out_scale = decay_pow(cx.s, 16 * w + l16 + 1);          // lambda^(a+1)

    // state slice in registers (fp32) and its bf16 transposed copy in LDS
    f32x4 sacc[ITW][2];
#pragma unroll
    for (int u = 0; u < ITW; ++u)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int it = w * ITW + u;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[u][jt][r] = St[(16 * it + 4 * lg + r) * D + cx.j0 + 16 * jt + l16];
            uint2 p;
            p.x = pack_bf16x2(sacc[u][jt][0], sacc[u][jt][1]);
            p.y = pack_bf16x2(sacc[u][jt][2], sacc[u][jt][3]);
            *reinterpret_cast<uint2 *>(&sm.ST[16 * jt + l16][16 * it + 4 * lg]) = p;
        }
    // scores above the causal diagonal tiles are never written: zero them once
    for (int e = tid; e < PC * PP / 2; e += PT) reinterpret_cast<uint32_t *>(&sm.P[0][0])[e] = 0u;

    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        consume_step<D, 0>(cx, sm, blk, sacc);
        consume_step<D, 1>(cx, sm, blk + 1, sacc);
    }

#pragma unroll
    for (int u = 0; u < ITW; ++u)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int it = w * ITW + u;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                St[(16 * it + 4 * lg + r) * D + cx.j0 + 16 * jt + l16] = sacc[u][jt][r];
        }
}

template <int D>
__global__ __launch_bounds__(2 * PT) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ slopes,
    uint16_t *__restrict__ out, float *__restrict__ state, int64_t H, int64_t N)
{
    constexpr int NJ = D / PJ;            // workgroups per head
    __shared__ Smem<D> sm;

    Ctx<D> cx;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    cx.w = wave & 3;
    const int l = tid % 64;
    cx.l16 = l % 16;
    cx.lg = l / 16;

    // XCD-aware placement: workgroup i runs on XCD i % 8; give the NJ
    // workgroups of one head consecutive logical ids on the same XCD.
    const int64_t nwg = gridDim.x;
    int64_t lid = blockIdx.x;
    if (nwg % 8 == 0) lid = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
    const int64_t bh = lid / NJ;
    cx.j0 = (int)(lid % NJ) * PJ;
    cx.s = slopes[bh % H];
    cx.N = N;
    // blocks processed: a multiple of NSET (trailing empty blocks are no-ops)
    cx.nblk = ((N + PC - 1) / PC + NSET - 1) / NSET * NSET;
    cx.qh = q + bh * N * D;
    cx.kh = k + bh * N * D;
    cx.vh = v + bh * N * D;
    cx.oh = out + bh * N * D;
    cx.full_decay = decay_pow(cx.s, PC);                        // lambda^C

    if (wave >= 4) {
        const int p = tid - PT;
        cx.wfull = decay_pow(cx.s, PC - 1 - p / 4);             // lambda^(C-1-b)
        producer<D>(cx, sm, p);
    } else {
        consumer<D>(cx, sm, state + bh * D * D, tid);
    }
}
}  // namespace

int64_t prefill_bf16_grid(int64_t B, int64_t H, int d) { return B * H * (d / PJ); }

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *slopes, uint16_t *out, float *state,
                               int64_t B, int64_t H, int64_t N, int d, hipStream_t stream)
{
    const dim3 grid((unsigned)prefill_bf16_grid(B, H, d)), block(2 * PT);
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                    (void *)&out, (void *)&state, (void *)&H, (void *)&N};
    const void *fn = d == 64 ? (const void *)prefill_bf16_kernel<64>
                             : (const void *)prefill_bf16_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace la
