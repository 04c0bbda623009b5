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
// Every product is a bf16 x bf16 -> fp32 MFMA (v_mfma_f32_32x32x16_bf16).
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
// Roles inside a workgroup (8 waves).  Waves 4..7 are producers: they only
// load Q, K and the workgroup's 64 x 32 slice of V with 16-byte buffer loads,
// four blocks ahead of use (four register sets), and write them into one of
// two LDS buffers one block ahead (plus a decay-weighted copy of V).  Waves
// 0..3 are consumers: they only read LDS, run the MFMAs and store outputs
// (roles below).  Keeping global loads and stores in different waves matters
// on gfx9: one counter (vmcnt) tracks both, and a wave with both kinds in
// flight must drain all of them before it can use any loaded register.
//
// What bounds it: every workgroup of a head pulls the full Q and K blocks
// through its XCD's L2 (the four copies share one HBM read), and LDS carries
// the producers' writes plus every MFMA operand.  Measured at 256K tokens, a
// block takes about 2,000 cycles with LDS about 70% busy, set by the consumer
// waves' reads and their dependent MFMA chains (the HBM stream alone would
// take two thirds of that).  The layout therefore keeps each operand's LDS
// reads few: 32x32x16 MFMAs (half the operand bytes per
// flop of 16x16x32), scores kept in registers and fed straight into V^T P^T,
// Q fragments shared by the score and inter-term products, and one barrier
// per block (double-buffered tiles and state copy).
// Contractions over tokens (the state update K^T V and the intra output
// V^T P^T) need the token index contiguous per lane; they read K and V from
// their token-major LDS tiles with ds_read_b64_tr_b16 (gfx950 transposing LDS
// read).  K's 16-byte chunks are XOR-swizzled by row so that both its plain
// reads (8 rows, one chunk) and its transposed reads (4 rows, one chunk pair)
// hit distinct LDS banks.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (lane l, l32 = l % 32,
// h = l / 32): A row l32, k = 8 h .. 8 h + 7; B column l32, same k; result
// register r (0..15): row 8 (r / 4) + 4 h + r % 4, column l32.
// ds_read_b64_tr_b16: within each 16-lane group, lane l16 supplies the
// address of a 4-element chunk; lane l16 receives element l16 % 4 of chunks
// 4e + l16 / 4, e = 0..3.  So if lane l16 points at row r0 + l16/4, column
// c0 + 4 (l16 % 4) of a row-major tile, it receives column c0 + l16 of rows
// r0 .. r0 + 3: a k-contiguous MFMA operand for a contraction over rows.
#include "la_internal.h"

#include <type_traits>

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int PC = 64;        // tokens per block
constexpr int PJ = 32;        // state / output columns per workgroup
constexpr int NCONS = 4;      // consumer waves
constexpr int PT = 256;       // producer threads (4 waves)
constexpr int NTHREADS = 64 * NCONS + PT;
constexpr int NSET = 4;       // producer register sets (blocks in flight)
constexpr int QPAD = 8;       // bf16 padding of Q and state-copy rows
constexpr int VP = 32;        // V row pitch (64 B, unpadded)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// eight fp32 -> one bf16 operand (round to nearest even)
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16 &x, int base) {
    u32x4 w;
    w[0] = pack_bf16x2(x[base + 0], x[base + 1]);
    w[1] = pack_bf16x2(x[base + 2], x[base + 3]);
    w[2] = pack_bf16x2(x[base + 4], x[base + 5]);
    w[3] = pack_bf16x2(x[base + 6], x[base + 7]);
    return __builtin_bit_cast(bf16x8, w);
}

// 16-byte-chunk swizzle of K rows (see the header comment)
__device__ __forceinline__ int kswz(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }

template <int D>
struct alignas(16) Smem {
    uint16_t Q[2][PC][D + QPAD];     // Q blocks, token-major
    uint16_t K[2][PC][D];            // K blocks, token-major, chunk-swizzled
    uint16_t V[2][PC][VP];           // V slices, token-major
    uint16_t VW[2][PC][VP];          // V slices times lambda^(c-1-b)
    uint16_t ST[2][PJ][D + QPAD];    // bf16 copies of the state slice, transposed
    float OP[2][64][20];             // W3 -> W2 partial outputs (one lane's 16 values)
};

// ---- producer waves: global -> registers -> LDS ----------------------------

template <int D>
struct Regs {                        // one block's share of a producer thread
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

// tokens of the block starting at t0 (0 past the end, and 0 for t0 < 0, so a
// buffer range built from it never reaches before the slice)
__device__ __forceinline__ int block_len(int64_t t0, int64_t N) {
    return t0 < 0 ? 0 : (int)max((int64_t)0, min((int64_t)PC, N - t0));
}

// rows t0 .. t0+63 of a slice whose rows are ts elements apart: the range
// ends right after the last real row, so later rows read as zero and stores
// to them are dropped (ts >= D, and 63*ts + D < 2^31 checked on the host)
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t *base, int64_t t0,
                                                              int64_t N, int ts)
{
    const int c = block_len(t0, N);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(base + t0 * ts), (short)0,
                                             c == 0 ? 0 : ((c - 1) * ts + D) * 2, RSRC_WORD3);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

template <int D>
__device__ __forceinline__ void load_block(Regs<D> &r, const uint16_t *qh, const uint16_t *kh,
                                           const uint16_t *vh, int64_t t0, int64_t N,
                                           int64_t ts, const Addr<D> &ad)
{
    const __amdgpu_buffer_rsrc_t rq = block_rsrc<D>(qh, t0, N, ts);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(kh, t0, N, ts);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(vh, t0, N, ts);
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
__device__ __forceinline__ void store_block(const Regs<D> &r, Smem<D> &sm, int p, float wv)
{
#pragma unroll
    for (int u = 0; u < Regs<D>::NQ; ++u) {
        const int ch = p + PT * u;
        const int row = ch / (D / 8), c8 = ch % (D / 8);
        *reinterpret_cast<uint4 *>(&sm.Q[BUF][row][c8 * 8]) = r.q[u];
        *reinterpret_cast<uint4 *>(&sm.K[BUF][row][(c8 ^ kswz(row)) * 8]) = r.k[u];
    }
    const int vrow = p / 4, vc = (p % 4) * 8;
    *reinterpret_cast<uint4 *>(&sm.V[BUF][vrow][vc]) = r.v;
    uint4 w;
    w.x = scale_pair(r.v.x, wv);
    w.y = scale_pair(r.v.y, wv);
    w.z = scale_pair(r.v.z, wv);
    w.w = scale_pair(r.v.w, wv);
    *reinterpret_cast<uint4 *>(&sm.VW[BUF][vrow][vc]) = w;
}

template <int D>
struct Ctx {                          // per-thread constants of one workgroup
    const uint16_t *qh, *kh, *vh;     // this (b, h) slice
    const uint16_t *oh;
    int64_t N, nblk;                  // nblk: blocks processed (a multiple of NSET)
    int ts, ots;                      // token strides (elements) of q/k/v and of out (<= 2^24)
    float s;
    int j0;
};

template <int D, int BUF>
__device__ __forceinline__ void produce_store(const Ctx<D> &cx, Smem<D> &sm, const Regs<D> &r,
                                              int64_t blk, int p, float wfull)
{
    const int c = block_len(blk * PC, cx.N);
    const int b = p / 4;
    const float wv = c == PC ? wfull : (b < c ? decay_pow(cx.s, c - 1 - b) : 0.0f);
    store_block<D, BUF>(r, sm, p, wv);
}

// One producer step per block blk: after the block's barrier, stage block
// blk+1 (register set SET) into the other LDS buffer, then reload SET with
// block blk+1+NSET.  Loads past the end return zeros without touching
// memory, so nothing here is conditional (exact vmcnt waits).
template <int D, int SET>
__device__ __forceinline__ void produce_step(const Ctx<D> &cx, Smem<D> &sm, Regs<D> (&rs)[NSET],
                                             const Addr<D> &ad, int64_t blk, int p, float wfull)
{
    __syncthreads();                                   // barrier of block blk
    if (SET % 2 == 1) produce_store<D, 1>(cx, sm, rs[SET], blk + 1, p, wfull);
    else              produce_store<D, 0>(cx, sm, rs[SET], blk + 1, p, wfull);
    load_block<D>(rs[SET], cx.qh, cx.kh, cx.vh, (blk + 1 + NSET) * PC, cx.N, cx.ts, ad);
}

template <int D>
__device__ void producer(const Ctx<D> &cx, Smem<D> &sm, int p)
{
    Addr<D> ad;
#pragma unroll
    for (int u = 0; u < Regs<D>::NQ; ++u) {
        const int ch = p + PT * u;
        ad.qk[u] = (uint32_t)(((ch / (D / 8)) * cx.ts + (ch % (D / 8)) * 8) * 2);
    }
    ad.v = (uint32_t)(((p / 4) * cx.ts + cx.j0 + (p % 4) * 8) * 2);
    const float wfull = decay_pow(cx.s, PC - 1 - p / 4);       // lambda^(C-1-b)

    Regs<D> rs[NSET];                                           // set i holds block i (mod NSET)
#pragma unroll
    for (int i = 0; i < NSET; ++i) load_block<D>(rs[i], cx.qh, cx.kh, cx.vh, i * PC, cx.N, cx.ts, ad);
    produce_store<D, 0>(cx, sm, rs[0], 0, p, wfull);
    load_block<D>(rs[0], cx.qh, cx.kh, cx.vh, NSET * PC, cx.N, cx.ts, ad);

    // block blk stages block blk+1 from set (blk+1) % NSET into buffer (blk+1) % 2
    for (int64_t blk = 0; blk < cx.nblk; blk += NSET) {
        produce_step<D, 1>(cx, sm, rs, ad, blk + 0, p, wfull);
        produce_step<D, 2>(cx, sm, rs, ad, blk + 1, p, wfull);
        produce_step<D, 3>(cx, sm, rs, ad, blk + 2, p, wfull);
        produce_step<D, 0>(cx, sm, rs, ad, blk + 3, p, wfull);
    }
    __syncthreads();                                   // final barrier (matches the consumers)
}

// ---- consumer waves: scores, outputs, state scan ---------------------------
//
// Four consumer waves, one per SIMD (each shares its SIMD with one producer):
//   W0  the state scan: S = lambda^c S + K^T (lambda^(c-1-b) V) on all D
//       state rows, and the bf16 copy ST of the new state (double-buffered);
//   W1  tokens 0..31: inter term S^T Q^T + scores P^T(0,0) + V^T P^T, stored;
//   W2  tokens 32..63: inter term + scores P^T(1,1) + their V^T P^T part;
//   W3  tokens 32..63: scores P^T(0,1) + their V^T P^T part, handed to W2
//       through LDS (fp32, double-buffered); W2 adds it one block later and
//       stores that block's tokens 32..63 then.
// The per-wave MFMA counts per block (d = 128) are 16 / 18 / 18 / 10, and the
// sequential part of the method (the state scan) runs on its own wave.

template <int D>
struct Lane {                               // lane coordinates for 32x32 MFMAs
    int l32, h, l16, q2, trow, tcol;
    __device__ explicit Lane(int lane)
        : l32(lane % 32), h(lane / 32), l16(lane % 16), q2((lane / 16) % 2),
          trow((lane % 16) >> 2), tcol(4 * ((lane % 16) & 3)) {}
};

// decay of score accumulator register r for a tile whose a-half is ah and
// b-half bh: lambda^(a-b), 0 above the diagonal
__device__ __forceinline__ void score_decay(float (&dec)[16], float s, int ah, int bh, int l32, int h)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int e = (32 * ah + l32) - (32 * bh + 8 * (r / 4) + 4 * h + r % 4);
        dec[r] = e < 0 ? 0.0f : decay_pow(s, e);
    }
}

// O^T(a-half ah) = scale * S^T Q^T from state copy SB and Q buffer QB
template <int D>
__device__ __forceinline__ f32x16 inter_term(const Smem<D> &sm, int qb, int sb, int ah,
                                              const Lane<D> &ln, float scale, bf16x8 (&qf)[D / 16])
{
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = ld8(&sm.Q[qb][32 * ah + ln.l32][16 * ks + 8 * ln.h]);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        acc = mfma(ld8(&sm.ST[sb][ln.l32][16 * ks + 8 * ln.h]), qf[ks], acc);
    return acc * scale;
}

// score tile P^T(bh, ah) (decayed) from Q fragments qf, then acc += V^T P^T
// over the tile's 32 tokens; the accumulator registers of P^T are the B
// operand directly (registers 8s..8s+7 hold tokens 32bh + 16s + 8e' + 4h + 0..3)
template <int D>
__device__ __forceinline__ void score_pv(const Smem<D> &sm, int buf, int bh,
                                         const bf16x8 (&qf)[D / 16], const float (&dec)[16],
                                         const Lane<D> &ln, f32x16 &acc)
{
    f32x16 pacc = {};
    const int krow = 32 * bh + ln.l32;
    const int ksw = kswz(krow);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        pacc = mfma(ld8(&sm.K[buf][krow][((2 * ks + ln.h) ^ ksw) * 8]), qf[ks], pacc);
#pragma unroll
    for (int r = 0; r < 16; ++r) pacc[r] *= dec[r];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int r0 = 32 * bh + 16 * s2 + 4 * ln.h + ln.trow;
        const bf16x8 va = ldtr8(&sm.V[buf][r0][16 * ln.q2 + ln.tcol],
                                &sm.V[buf][r0 + 8][16 * ln.q2 + ln.tcol]);
        acc = mfma(va, to_bf16x8(pacc, 8 * s2), acc);
    }
}

// store a 32x32 O^T tile (tokens 32ah.., columns j0..j0+31) of block t0.
// Accumulator register group q4 holds columns 8q4 + 4h + 0..3 of token a; a
// lane-half swap (lanes l <-> l+32) of groups (0,1) and (2,3) gives lane h
// columns 8h..8h+7 and 16+8h..16+8h+7, so each row is written as 32-byte runs
// by two 16-byte stores per lane.
template <int D>
__device__ __forceinline__ int out_offset(const Ctx<D> &cx, int ah, const Lane<D> &ln) {
    return ((32 * ah + ln.l32) * cx.ots + cx.j0 + 8 * ln.h) * 2;   // bytes, row 32ah + l32
}

template <int D>
__device__ __forceinline__ void store_out(const Ctx<D> &cx, int64_t t0, int ooff,
                                          const f32x16 &acc)
{
    const __amdgpu_buffer_rsrc_t ro = block_rsrc<D>(cx.oh, t0, cx.N, cx.ots);   // rows past N dropped
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
        const int g0 = 2 * pr, g1 = 2 * pr + 1;
        unsigned x0 = pack_bf16x2(acc[4 * g0 + 0], acc[4 * g0 + 1]);
        unsigned x1 = pack_bf16x2(acc[4 * g0 + 2], acc[4 * g0 + 3]);
        unsigned y0 = pack_bf16x2(acc[4 * g1 + 0], acc[4 * g1 + 1]);
        unsigned y1 = pack_bf16x2(acc[4 * g1 + 2], acc[4 * g1 + 3]);
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        u32x4 o;
        o[0] = s0[0]; o[1] = s1[0]; o[2] = s0[1]; o[3] = s1[1];
        __builtin_amdgcn_raw_buffer_store_b128(o, ro, ooff + 32 * pr, 0, 0);
    }
}

// bf16 copy of state tile it (rows 32it..) into ST[buf][j][i]
template <int D>
__device__ __forceinline__ void write_st(Smem<D> &sm, int buf, int it, const Lane<D> &ln,
                                         const f32x16 &s)
{
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        uint2 p;
        p.x = pack_bf16x2(s[4 * q4 + 0], s[4 * q4 + 1]);
        p.y = pack_bf16x2(s[4 * q4 + 2], s[4 * q4 + 3]);
        *reinterpret_cast<uint2 *>(&sm.ST[buf][ln.l32][32 * it + 8 * q4 + 4 * ln.h]) = p;
    }
}

// W0: the state scan
template <int D>
__device__ void scan_wave(const Ctx<D> &cx, Smem<D> &sm, float *St, int lane)
{
    constexpr int NT = D / 32;                  // 32-row state tiles
    const Lane<D> ln(lane);
    const float full_decay = decay_pow(cx.s, PC);
    const int clast = (int)(cx.N - (cx.N - 1) / PC * PC);          // tokens of the last real block
    const float last_decay = decay_pow(cx.s, clast);

    f32x16 sacc[NT];
#pragma unroll
    for (int it = 0; it < NT; ++it) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sacc[it][r] = St[(32 * it + 8 * (r / 4) + 4 * ln.h + r % 4) * D + cx.j0 + ln.l32];
        write_st<D>(sm, 1, it, ln, sacc[it]);   // read by block 0
    }

    auto step = [&](int64_t blk, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        const int c = block_len(blk * PC, cx.N);
        __syncthreads();
        const float sdec = c == PC ? full_decay : (c == 0 ? 1.0f : last_decay);
        bf16x8 vwf[PC / 16];
#pragma unroll
        for (int ks = 0; ks < PC / 16; ++ks) {
            const int r0 = 16 * ks + 8 * ln.h + ln.trow;
            vwf[ks] = ldtr8(&sm.VW[BUF][r0][16 * ln.q2 + ln.tcol], &sm.VW[BUF][r0 + 4][16 * ln.q2 + ln.tcol]);
        }
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            const int col = 32 * it + 16 * ln.q2 + ln.tcol;        // feature of this lane's chunk
            const int ch = col >> 3, sub = col & 7;
            sacc[it] *= sdec;
#pragma unroll
            for (int ks = 0; ks < PC / 16; ++ks) {
                const int r0 = 16 * ks + 8 * ln.h + ln.trow;
                const bf16x8 ka = ldtr8(&sm.K[BUF][r0][((ch ^ kswz(r0)) * 8) + sub],
                                        &sm.K[BUF][r0 + 4][((ch ^ kswz(r0 + 4)) * 8) + sub]);
                sacc[it] = mfma(ka, vwf[ks], sacc[it]);
            }
            write_st<D>(sm, BUF, it, ln, sacc[it]);
        }
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(blk, std::integral_constant<int, 0>());
        step(blk + 1, std::integral_constant<int, 1>());
    }
    __syncthreads();                            // final barrier (W2's last store)

#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            St[(32 * it + 8 * (r / 4) + 4 * ln.h + r % 4) * D + cx.j0 + ln.l32] = sacc[it][r];
}

// W1: tokens 0..31, complete
template <int D>
__device__ void out0_wave(const Ctx<D> &cx, Smem<D> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 0, 0, ln.l32, ln.h);
    const float scale = decay_pow(cx.s, ln.l32 + 1);               // lambda^(a+1)
    const int ooff = out_offset(cx, 0, ln);
    auto step = [&](int64_t blk, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        __syncthreads();
        bf16x8 qf[D / 16];
        f32x16 acc = inter_term<D>(sm, BUF, BUF ^ 1, 0, ln, scale, qf);
        score_pv<D>(sm, BUF, 0, qf, dec, ln, acc);
        store_out<D>(cx, blk * PC, ooff, acc);
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(blk, std::integral_constant<int, 0>());
        step(blk + 1, std::integral_constant<int, 1>());
    }
    __syncthreads();
}

// W2: tokens 32..63, inter term + diagonal scores; adds W3's part one block later
template <int D>
__device__ void out1_wave(const Ctx<D> &cx, Smem<D> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 1, 1, ln.l32, ln.h);
    const float scale = decay_pow(cx.s, 32 + ln.l32 + 1);
    const int ooff = out_offset(cx, 1, ln);
    f32x16 prev = {};
    auto finish_prev = [&](int64_t pblk, int pbuf) {               // block pblk's tokens 32..63
        const float4 *op = reinterpret_cast<const float4 *>(&sm.OP[pbuf][lane][0]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 x = op[u];
            prev[4 * u + 0] += x.x; prev[4 * u + 1] += x.y;
            prev[4 * u + 2] += x.z; prev[4 * u + 3] += x.w;
        }
        store_out<D>(cx, pblk * PC, ooff, prev);
    };
    auto step = [&](int64_t blk, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        __syncthreads();
        bf16x8 qf[D / 16];
        f32x16 acc = inter_term<D>(sm, BUF, BUF ^ 1, 1, ln, scale, qf);
        score_pv<D>(sm, BUF, 1, qf, dec, ln, acc);
        if (blk > 0) finish_prev(blk - 1, BUF ^ 1);
        prev = acc;
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(blk, std::integral_constant<int, 0>());
        step(blk + 1, std::integral_constant<int, 1>());
    }
    __syncthreads();                            // W3's part of the last block is visible
    if (cx.nblk > 0) finish_prev(cx.nblk - 1, (int)((cx.nblk - 1) & 1));   // (empty sequence: none)
}

// W3: tokens 32..63, off-diagonal scores P^T(0,1) and their V^T P^T part
template <int D>
__device__ void out1x_wave(const Ctx<D> &cx, Smem<D> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 1, 0, ln.l32, ln.h);
    auto step = [&](int64_t blk, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        __syncthreads();
        bf16x8 qf[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = ld8(&sm.Q[BUF][32 + ln.l32][16 * ks + 8 * ln.h]);
        f32x16 acc = {};
        score_pv<D>(sm, BUF, 0, qf, dec, ln, acc);
        float4 *op = reinterpret_cast<float4 *>(&sm.OP[BUF][lane][0]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            op[u] = make_float4(acc[4 * u + 0], acc[4 * u + 1], acc[4 * u + 2], acc[4 * u + 3]);
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(blk, std::integral_constant<int, 0>());
        step(blk + 1, std::integral_constant<int, 1>());
    }
    __syncthreads();
}

// STRIDED = false: rows of q, k, v and out are D elements apart (a
// compile-time token stride; head and sequence offsets still come from the
// map), so the contiguous layouts pay nothing for stride support.
template <int D, bool STRIDED>
__global__ __launch_bounds__(NTHREADS) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ slopes,
    uint16_t *__restrict__ out, float *__restrict__ state, SeqMap map)
{
    constexpr int NJ = D / PJ;            // workgroups per head
    __shared__ Smem<D> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);

    // XCD-aware placement: workgroup i runs on XCD i % 8 and workgroups start
    // in index order.  Workgroups 8q + x (x = 0..7) take slice q % NJ of
    // (sequence, head) slot 8 (q / NJ) + x: the NJ slices of one head run on
    // one XCD at the same time (Q and K come from HBM once, then from that
    // XCD's L2), and consecutive heads of a sequence go to different XCDs, so
    // every XCD gets an equal share of every sequence however long it is.
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
    int64_t in0, out0, N;
    seq_slice(map, bh / map.H, bh % map.H, &in0, &out0, &N);

    Ctx<D> cx;
    cx.j0 = (int)slice * PJ;
    cx.s = slopes[bh % map.H];
    cx.N = N;
    // blocks processed: a multiple of NSET (trailing empty blocks are no-ops;
    // an empty sequence leaves its state unchanged)
    cx.nblk = ((N + PC - 1) / PC + NSET - 1) / NSET * NSET;
    cx.qh = q + in0;
    cx.kh = k + in0;
    cx.vh = v + in0;
    cx.oh = out + out0;
    cx.ts = STRIDED ? (int)map.in.st : D;
    cx.ots = STRIDED ? (int)map.out.st : D;

    const int lane = tid % 64;
    switch (wave) {
        case 0: scan_wave<D>(cx, sm, state + bh * D * D, lane); break;
        case 1: out0_wave<D>(cx, sm, lane); break;
        case 2: out1_wave<D>(cx, sm, lane); break;
        case 3: out1x_wave<D>(cx, sm, lane); break;
        default: producer<D>(cx, sm, tid - 64 * NCONS); break;
    }
}

}  // namespace

int64_t prefill_bf16_grid(int64_t seqs, int64_t H, int d) { return seqs * H * (d / PJ); }

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *slopes, uint16_t *out, float *state,
                               int64_t seqs, const SeqMap &map, int d, hipStream_t stream)
{
    const dim3 grid((unsigned)prefill_bf16_grid(seqs, map.H, d)), block(NTHREADS);
    SeqMap m = map;
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                    (void *)&out, (void *)&state, (void *)&m};
    const bool strided = map.in.st != d || map.out.st != d;
    const void *fn = d == 64 ? (strided ? (const void *)prefill_bf16_kernel<64, true>
                                        : (const void *)prefill_bf16_kernel<64, false>)
                             : (strided ? (const void *)prefill_bf16_kernel<128, true>
                                        : (const void *)prefill_bf16_kernel<128, false>);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace la
