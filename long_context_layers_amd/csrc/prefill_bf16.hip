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
// once and from that XCD's L2 for the other three.  A packed batch of short
// sequences runs one workgroup per (head, column slice) that walks every
// sequence in order (WALK): the pipeline then runs across sequence
// boundaries, the scan hands each final state out and the next initial state
// in (staged in LDS a whole sequence ahead, both moved 16 bytes per lane),
// instead of a workgroup per sequence
// paying its own pipeline fill and drain.
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
// block takes about 2,075 cycles, of which about 1,690 are LDS traffic (some
// 52 KB written, 96 KB read); the consumer waves are each busy 1,600 to 1,800
// cycles of it, mostly waiting on LDS reads, the producers 1,300 to 1,650, and
// relieving any one of them (giving the scan its operands sooner, moving work
// between waves, or even removing Q's LDS traffic) leaves the time per launch
// unchanged.  That time is set by the package power limit: the kernel draws
// the whole 1400 W with the clock held near 2.05 GHz, while its loading half
// and its compute half, each run alone, stay below the limit at 2.4 GHz.  A
// block done in fewer cycles for the same energy only lowers the clock.  The one barrier per block also
// keeps the LDS shared fairly: without it, waves that finish early run ahead
// and starve the busiest one.  The layout therefore keeps each operand's LDS
// reads few: 32x32x16 MFMAs (half the operand bytes per flop of 16x16x32),
// scores kept in registers and fed straight into V^T P^T, Q fragments shared
// by the score and inter-term products, and double-buffered tiles and state
// copy behind that single barrier.
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

#include <atomic>
#include <type_traits>

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
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

// ---- the blocks a workgroup visits, in order --------------------------------

// One block's place: its sequence, its first token within that sequence, the
// sequence's length and the element offsets of the (sequence, head) slice in
// the inputs and the output (j: the sequence's entry in a walk's table).  A
// block never spans two sequences.  Blocks with no tokens (past the end of
// the work) read zeros and their stores are dropped.
struct Pos {
    int64_t seq, t0, n, in0, out0;
    int j;
};

// The non-empty sequences of a walking launch, in order, with their clamped
// offsets (a walking launch has at most WALK_SEQS sequences and fewer than
// 2^31 tokens).  Built once per workgroup, so advancing a position is a
// broadcast LDS read instead of dependent loads of the offsets from memory.
constexpr int WALK_SEQS = 1024;

struct WalkTable {
    int seq[WALK_SEQS], start[WALK_SEQS], len[WALK_SEQS];
    int count;                  // entries
    int nblk;                   // blocks with tokens
};

// one wave fills the table (a barrier must follow before anyone reads it)
__device__ void build_table(WalkTable &tb, const SeqMap &m, int64_t nseq, int lane)
{
    int count = 0, nblk = 0;
    for (int64_t base = 0; base < nseq; base += 64) {
        const int64_t s = base + lane;
        int a = 0, n = 0;
        if (s < nseq) {
            const int64_t a64 = min(max(m.cu[s], (int64_t)0), m.T);
            a = (int)a64;
            n = (int)(min(max(m.cu[s + 1], a64), m.T) - a64);
        }
        const uint64_t mask = __ballot(n > 0);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
        if (n > 0) {
            tb.seq[count + before] = (int)s;
            tb.start[count + before] = a;
            tb.len[count + before] = n;
        }
        count += __popcll(mask);
        int b = (n + PC - 1) / PC;
        for (int off = 32; off > 0; off >>= 1) b += __shfl_xor(b, off);
        nblk += b;
    }
    if (lane == 0) {
        tb.count = count;
        tb.nblk = nblk;
    }
}

// WALK = false: the blocks of one (sequence, head) slice, then blocks past its
// end.  WALK = true (a packed launch with one workgroup per head and column
// slice): the blocks of every non-empty sequence, sequence after sequence, so
// the pipeline below runs across sequence boundaries; then blocks with no
// tokens.  Every value here is uniform across the workgroup.
template <bool WALK>
struct Walk {
    SeqMap map;
    int64_t nseq, h;
    const WalkTable *tb;        // WALK: the table, in LDS
    float *slot;                // WALK: the next sequence's initial state, staged in LDS

    __device__ static int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
    // WALK: the first block of table entry j (no tokens past the table's end)
    __device__ Pos entry(int j) const {
        Pos p = {nseq, 0, 0, 0, 0, j};
        if (j < uni(tb->count)) {
            const int64_t a = uni(tb->start[j]);
            p.seq = uni(tb->seq[j]);
            p.n = uni(tb->len[j]);
            p.in0 = h * map.in.sh + a * map.in.st;
            p.out0 = h * map.out.sh + a * map.out.st;
        }
        return p;
    }
    __device__ Pos first(int64_t seq) const {
        if constexpr (WALK) {
            return entry(0);
        } else {
            Pos p = {seq, 0, 0, 0, 0, 0};
            seq_slice(map, seq, h, &p.in0, &p.out0, &p.n);
            return p;
        }
    }
    __device__ void next(Pos &p) const {
        p.t0 += PC;
        if constexpr (WALK) {
            if (p.t0 >= p.n) p = entry(p.j + 1);
        }
    }
    // the block is the last of its sequence
    __device__ static bool last(const Pos &p) { return p.t0 < p.n && p.t0 + PC >= p.n; }
    // WALK: the sequence of table entry j, or -1 past the table's end
    __device__ int64_t seq_at(int j) const { return j < uni(tb->count) ? uni(tb->seq[j]) : -1; }
    // blocks with tokens
    __device__ int64_t blocks(const Pos &p0) const {
        if constexpr (WALK) return uni(tb->nblk);
        else return (p0.n + PC - 1) / PC;
    }
};

template <int D>
struct Ctx {                          // per-thread constants of one workgroup
    const uint16_t *q, *k, *v;        // the launch's inputs (slices at Pos::in0)
    uint16_t *o;                      // its output (slices at Pos::out0)
    float *state;                     // its states, [sequence][H][D][D]
    int64_t H, h, nblk;               // nblk: blocks processed (a multiple of NSET)
    int ts, ots;                      // token strides (elements) of q/k/v and of out (<= 2^24)
    float s;
    int j0;

    // this workgroup's columns of the state of sequence seq: element (i, j) at i * D + j
    __device__ float *state_of(int64_t seq) const { return state + (seq * H + h) * D * D + j0; }
};

// ---- producer waves: global -> registers -> LDS ----------------------------

template <int D>
struct Regs {                        // one block's share of a producer thread
    static constexpr int NQ = PC * D / 8 / PT;   // 16-byte chunks of Q (and of K)
    uint4 q[NQ], k[NQ], v;
    int c;                           // tokens in the block
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
__device__ __forceinline__ void load_block(Regs<D> &r, const Ctx<D> &cx, const Pos &p,
                                           const Addr<D> &ad)
{
    const __amdgpu_buffer_rsrc_t rq = block_rsrc<D>(cx.q + p.in0, p.t0, p.n, cx.ts);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(cx.k + p.in0, p.t0, p.n, cx.ts);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(cx.v + p.in0, p.t0, p.n, cx.ts);
#pragma unroll
    for (int u = 0; u < Regs<D>::NQ; ++u) {
        r.q[u] = bload16(rq, ad.qk[u]);
        r.k[u] = bload16(rk, ad.qk[u]);
    }
    r.v = bload16(rv, ad.v);
    r.c = block_len(p.t0, p.n);
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

template <int D, int BUF>
__device__ __forceinline__ void produce_store(const Ctx<D> &cx, Smem<D> &sm, const Regs<D> &r,
                                              int p, float wfull)
{
    const int b = p / 4;
    const float wv = r.c == PC ? wfull : (b < r.c ? decay_pow(cx.s, r.c - 1 - b) : 0.0f);
    store_block<D, BUF>(r, sm, p, wv);
}

// One producer step per block blk: after the block's barrier, stage block
// blk+1 (register set SET) into the other LDS buffer, then reload SET with
// block blk+1+NSET (at ld, which then moves on).  Loads past the end return
// zeros without touching memory, so nothing here is conditional (exact vmcnt
// waits).
template <int D, int SET, bool WALK>
__device__ __forceinline__ void produce_step(const Ctx<D> &cx, const Walk<WALK> &wk, Smem<D> &sm,
                                             Regs<D> (&rs)[NSET], const Addr<D> &ad, Pos &ld, int p,
                                             float wfull)
{
    __syncthreads();                                   // barrier of block blk
    if (SET % 2 == 1) produce_store<D, 1>(cx, sm, rs[SET], p, wfull);
    else              produce_store<D, 0>(cx, sm, rs[SET], p, wfull);
    load_block<D>(rs[SET], cx, ld, ad);
    wk.next(ld);
}

template <int D, bool WALK>
__device__ void producer(const Ctx<D> &cx, const Walk<WALK> &wk, Pos ld, Smem<D> &sm, int p)
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
    for (int i = 0; i < NSET; ++i) {
        load_block<D>(rs[i], cx, ld, ad);
        wk.next(ld);
    }
    produce_store<D, 0>(cx, sm, rs[0], p, wfull);
    load_block<D>(rs[0], cx, ld, ad);
    wk.next(ld);

    // block blk stages block blk+1 from set (blk+1) % NSET into buffer (blk+1) % 2
    for (int64_t blk = 0; blk < cx.nblk; blk += NSET) {
        produce_step<D, 1>(cx, wk, sm, rs, ad, ld, p, wfull);
        produce_step<D, 2>(cx, wk, sm, rs, ad, ld, p, wfull);
        produce_step<D, 3>(cx, wk, sm, rs, ad, ld, p, wfull);
        produce_step<D, 0>(cx, wk, sm, rs, ad, ld, p, wfull);
    }
    __syncthreads();                                   // final barrier (matches the consumers)
}

// ---- consumer waves: scores, outputs, state scan ---------------------------
//
// Four consumer waves, one per SIMD (each shares its SIMD with one producer):
//   W0  the state scan: S = lambda^c S + K^T (lambda^(c-1-b) V) on the
//       first D - 32 state rows, and the bf16 copy ST of those rows of the new
//       state (double-buffered); at the last block of a sequence it stores
//       their final state and, when sequences follow (WALK), takes up the next
//       one's initial state, staged in an LDS slot a whole sequence earlier;
//   W1  tokens 0..31: inter term S^T Q^T + scores P^T(0,0) + V^T P^T, stored;
//   W2  tokens 32..63: inter term + scores P^T(1,1) + their V^T P^T part;
//   W3  tokens 32..63: scores P^T(0,1) + their V^T P^T part, handed to W2
//       through LDS (fp32, double-buffered); W2 adds it one block later and
//       stores that block's tokens 32..63 then; and the scan of the last 32
//       state rows, as W0 does for the others.
// The per-wave MFMA counts per block (d = 128) are 12 / 18 / 18 / 14.  Giving
// W3 a quarter of the scan (it was the least busy wave) leaves a dense launch's
// time unchanged but halves the scan's work at every sequence boundary of a
// walk (8% faster with 64-token sequences).

template <int D>
struct Lane {                               // lane coordinates for 32x32 MFMAs
    int l32, h, l16, q2, trow, tcol;
    __device__ explicit Lane(int lane)
        : l32(lane % 32), h(lane / 32), l16(lane % 16), q2((lane / 16) % 2),
          trow((lane % 16) >> 2), tcol(4 * ((lane % 16) & 3)) {}
};

// A state slice in the scan's registers: tile it, register r of lane (l32, h)
// holds row 32 it + 8 (r / 4) + 4 h + r % 4, column l32.  Buffer accesses: the
// lane's part of the offset in one register, each register's part a constant
// (used by the walk, whose scan also holds a second slice; a single-slice scan
// keeps plain pointer accesses, which measured slightly faster there).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_rsrc(const float *st, bool valid = true) {
    // valid = false: a zero range, so loads return zeros and touch no memory
    return __builtin_amdgcn_make_buffer_rsrc((void *)st, (short)0, valid ? ((D - 1) * D + PJ) * 4 : 0,
                                             RSRC_WORD3);
}

template <int D>
__device__ __forceinline__ int state_reg_offset(int it, int r) {   // bytes
    return (32 * it + 8 * (r / 4) + r % 4) * D * 4;
}

// tiles T0 .. T0 + NTL - 1 of the slice at st (x[t] holds tile T0 + t)
template <int D, int T0, int NTL>
__device__ __forceinline__ void load_state(f32x16 (&x)[NTL], const float *st, const Lane<D> &ln)
{
    const __amdgpu_buffer_rsrc_t rs = state_rsrc<D>(st);
    const int lo = (4 * ln.h * D + ln.l32) * 4;
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[t][r] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rs, lo, state_reg_offset<D>(T0 + t, r), 0));
}

template <int D, int T0, int NTL>
__device__ __forceinline__ void store_state(float *st, const f32x16 (&x)[NTL], const Lane<D> &ln)
{
    const __amdgpu_buffer_rsrc_t rs = state_rsrc<D>(st);
    const int lo = (4 * ln.h * D + ln.l32) * 4;
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[t][r]), rs, lo,
                                                  state_reg_offset<D>(T0 + t, r), 0);
}

// WALK: the slot holds state rows in LDS, row-major [D][32] fp32 (row = state
// row, column = this workgroup's column), filled and drained 16 bytes per lane:
// one instruction moves 8 rows (lane l: row 8 i + l / 8, columns 4 (l % 8) ..).

// tiles T0 .. T0 + NTL - 1 of a sequence's initial state into the slot by
// direct global -> LDS loads, so no registers wait for them; valid = false
// stages zeros
template <int D, int T0, int NTL>
__device__ __forceinline__ void stage_state(float *slot, const float *st, int lane, bool valid)
{
    const __amdgpu_buffer_rsrc_t rs = state_rsrc<D>(st, valid);
    const int lo = ((lane >> 3) * D + (lane & 7) * 4) * 4;
#pragma unroll
    for (int i = 0; i < 4 * NTL; ++i) {
        const int row0 = 32 * T0 + 8 * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void *)(slot + row0 * 32), 16, lo, row0 * D * 4, 0, 0);
    }
}

// the staged rows into the scan's registers
template <int D, int T0, int NTL>
__device__ __forceinline__ void read_staged(f32x16 (&x)[NTL], const float *slot, const Lane<D> &ln)
{
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[t][r] = slot[(32 * (T0 + t) + 8 * (r / 4) + 4 * ln.h + r % 4) * 32 + ln.l32];
}

// the final state of these rows out through the slot (its staged contents
// already read): registers -> slot -> 16-byte row pieces -> the state
template <int D, int T0, int NTL>
__device__ __forceinline__ void store_via_slot(float *slot, float *st, const f32x16 (&x)[NTL], const Lane<D> &ln,
                                               int lane)
{
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            slot[(32 * (T0 + t) + 8 * (r / 4) + 4 * ln.h + r % 4) * 32 + ln.l32] = x[t][r];
    const __amdgpu_buffer_rsrc_t rs = state_rsrc<D>(st);
    const int lo = ((lane >> 3) * D + (lane & 7) * 4) * 4;
#pragma unroll
    for (int i = 0; i < 4 * NTL; ++i) {
        const int row0 = 32 * T0 + 8 * i;
        const float4 v = *reinterpret_cast<const float4 *>(&slot[(row0 + (lane >> 3)) * 32 + (lane & 7) * 4]);
        const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, lo, row0 * D * 4, 0);
    }
}

// The block barrier of the waves that stage states (WALK): their own LDS
// writes complete, then the barrier, with no wait for the direct loads still
// in flight (a workgroup fence would wait for those too, their LDS writes
// being counted with vector memory); the clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

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

// store a 32x32 O^T tile (tokens 32ah.., columns j0..j0+31) of the block at p.
// Accumulator register group q4 holds columns 8q4 + 4h + 0..3 of token a; a
// lane-half swap (lanes l <-> l+32) of groups (0,1) and (2,3) gives lane h
// columns 8h..8h+7 and 16+8h..16+8h+7, so each row is written as 32-byte runs
// by two 16-byte stores per lane.
template <int D>
__device__ __forceinline__ int out_offset(const Ctx<D> &cx, int ah, const Lane<D> &ln) {
    return ((32 * ah + ln.l32) * cx.ots + cx.j0 + 8 * ln.h) * 2;   // bytes, row 32ah + l32
}

template <int D>
__device__ __forceinline__ void store_out(const Ctx<D> &cx, const Pos &p, int ooff,
                                          const f32x16 &acc)
{
    const __amdgpu_buffer_rsrc_t ro = block_rsrc<D>(cx.o + p.out0, p.t0, p.n, cx.ots);   // rows past the end dropped
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

// The state scan over tiles T0 .. T0 + NTL - 1 (32 state rows each) of the
// workgroup's column slice: S = lambda^c S + K^T (lambda^(c-1-b) V), fp32 in
// registers for the whole walk, and each block's bf16 copy ST of those rows
// (double-buffered).  At the last block of a sequence it stores the final
// state of its rows and, when sequences follow (WALK), takes up the next one's
// initial state, staged in LDS a whole sequence earlier.  The
// tiles evolve independently, so they can be split over waves: the scan wave
// runs all but the last, the off-diagonal score wave (which had the most
// slack) the last.
template <int D, bool WALK, int T0, int NTL>
struct Scan {
    Lane<D> ln;
    float full_decay;
    f32x16 sacc[NTL];

    __device__ Scan(const Ctx<D> &cx, int lane) : ln(lane), full_decay(decay_pow(cx.s, PC)) {}

    __device__ void init(const Ctx<D> &cx, const Walk<WALK> &wk, const Pos &pos, Smem<D> &sm) {
        if (pos.n > 0) {
            if constexpr (WALK) load_state<D, T0, NTL>(sacc, cx.state_of(pos.seq), ln);
            else {
                const float *St = cx.state_of(pos.seq);
#pragma unroll
                for (int t = 0; t < NTL; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sacc[t][r] = St[(32 * (T0 + t) + 8 * (r / 4) + 4 * ln.h + r % 4) * D + ln.l32];
            }
        } else {
#pragma unroll
            for (int t = 0; t < NTL; ++t) sacc[t] = f32x16{};
        }
        if constexpr (WALK) {
            const int64_t s1 = wk.seq_at(pos.j + 1);
            stage_state<D, T0, NTL>(wk.slot, cx.state_of(s1 >= 0 ? s1 : pos.seq), ln.l32 + 32 * ln.h, s1 >= 0);
        }
#pragma unroll
        for (int t = 0; t < NTL; ++t) write_st<D>(sm, 1, T0 + t, ln, sacc[t]);   // read by block 0
    }

    // block at pos (c tokens; last: it ends its sequence), LDS buffer BUF
    template <int BUF>
    __device__ void step(const Ctx<D> &cx, const Walk<WALK> &wk, const Pos &pos, Smem<D> &sm,
                         int c, bool last) {
        const float sdec = c == PC ? full_decay : (c == 0 ? 1.0f : decay_pow(cx.s, c));
        bf16x8 vwf[PC / 16];
#pragma unroll
        for (int ks = 0; ks < PC / 16; ++ks) {
            const int r0 = 16 * ks + 8 * ln.h + ln.trow;
            vwf[ks] = ldtr8(&sm.VW[BUF][r0][16 * ln.q2 + ln.tcol], &sm.VW[BUF][r0 + 4][16 * ln.q2 + ln.tcol]);
        }
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int col = 32 * (T0 + t) + 16 * ln.q2 + ln.tcol;   // feature of this lane's chunk
            const int ch = col >> 3, sub = col & 7;
            sacc[t] *= sdec;
#pragma unroll
            for (int ks = 0; ks < PC / 16; ++ks) {
                const int r0 = 16 * ks + 8 * ln.h + ln.trow;
                const bf16x8 ka = ldtr8(&sm.K[BUF][r0][((ch ^ kswz(r0)) * 8) + sub],
                                        &sm.K[BUF][r0 + 4][((ch ^ kswz(r0 + 4)) * 8) + sub]);
                sacc[t] = mfma(ka, vwf[ks], sacc[t]);
            }
            write_st<D>(sm, BUF, T0 + t, ln, sacc[t]);
        }
        if constexpr (WALK) {
            if (last) {
                // the next sequence's initial state out of LDS first: the
                // wait for its staging (issued a sequence ago) then covers no
                // store of this block
                const bool more = wk.seq_at(pos.j + 1) >= 0;
                f32x16 nxt[NTL];
                if (more) read_staged<D, T0, NTL>(nxt, wk.slot, ln);
                store_via_slot<D, T0, NTL>(wk.slot, cx.state_of(pos.seq), sacc, ln,   // the final state out
                                           ln.l32 + 32 * ln.h);
                if (more) {
                    // take up the next sequence (its bf16 copy over the one
                    // just written for the next block), then stage the one
                    // after it once the slot has been read
#pragma unroll
                    for (int t = 0; t < NTL; ++t) {
                        sacc[t] = nxt[t];
                        write_st<D>(sm, BUF, T0 + t, ln, sacc[t]);
                    }
                    __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): the slot reads done
                    const int64_t s2 = wk.seq_at(pos.j + 2);
                    stage_state<D, T0, NTL>(wk.slot, cx.state_of(s2 >= 0 ? s2 : pos.seq), ln.l32 + 32 * ln.h,
                                            s2 >= 0);
                }
            }
        }
    }

    // one sequence (no walk): its final state, after the loop (a store inside
    // the step measured slower: it sits on the scan's sequential path)
    __device__ void finish(const Ctx<D> &cx, const Pos &pos) {
        if constexpr (!WALK) {
            if (cx.nblk > 0) {
                float *St = cx.state_of(pos.seq);
#pragma unroll
                for (int t = 0; t < NTL; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        St[(32 * (T0 + t) + 8 * (r / 4) + 4 * ln.h + r % 4) * D + ln.l32] = sacc[t][r];
            }
        }
    }
};

// W0: the state scan on all tiles but the last (pos: block 0)
template <int D, bool WALK>
__device__ void scan_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D> &sm, int lane)
{
    Scan<D, WALK, 0, D / 32 - 1> sc(cx, lane);
    sc.init(cx, wk, pos, sm);
    auto step = [&](auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        const int c = block_len(pos.t0, pos.n);
        const bool last = Walk<WALK>::last(pos);
        if constexpr (WALK) lds_barrier();
        else __syncthreads();
        sc.template step<BUF>(cx, wk, pos, sm, c, last);
        wk.next(pos);
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(std::integral_constant<int, 0>());
        step(std::integral_constant<int, 1>());
    }
    __syncthreads();                            // final barrier (W2's last store)
    sc.finish(cx, pos);
}

// W1: tokens 0..31, complete
template <int D, bool WALK>
__device__ void out0_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 0, 0, ln.l32, ln.h);
    const float scale = decay_pow(cx.s, ln.l32 + 1);               // lambda^(a+1)
    const int ooff = out_offset(cx, 0, ln);
    auto step = [&](auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        __syncthreads();
        bf16x8 qf[D / 16];
        f32x16 acc = inter_term<D>(sm, BUF, BUF ^ 1, 0, ln, scale, qf);
        score_pv<D>(sm, BUF, 0, qf, dec, ln, acc);
        store_out<D>(cx, pos, ooff, acc);
        wk.next(pos);
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(std::integral_constant<int, 0>());
        step(std::integral_constant<int, 1>());
    }
    __syncthreads();
}

// W2: tokens 32..63, inter term + diagonal scores; adds W3's part one block later
template <int D, bool WALK>
__device__ void out1_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 1, 1, ln.l32, ln.h);
    const float scale = decay_pow(cx.s, 32 + ln.l32 + 1);
    const int ooff = out_offset(cx, 1, ln);
    f32x16 prev = {};
    Pos ppos = pos;                                                // block of prev
    auto finish_prev = [&](int pbuf) {                             // that block's tokens 32..63
        const float4 *op = reinterpret_cast<const float4 *>(&sm.OP[pbuf][lane][0]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 x = op[u];
            prev[4 * u + 0] += x.x; prev[4 * u + 1] += x.y;
            prev[4 * u + 2] += x.z; prev[4 * u + 3] += x.w;
        }
        store_out<D>(cx, ppos, ooff, prev);
    };
    auto step = [&](int64_t blk, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        __syncthreads();
        bf16x8 qf[D / 16];
        f32x16 acc = inter_term<D>(sm, BUF, BUF ^ 1, 1, ln, scale, qf);
        score_pv<D>(sm, BUF, 1, qf, dec, ln, acc);
        if (blk > 0) finish_prev(BUF ^ 1);
        prev = acc;
        ppos = pos;
        wk.next(pos);
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(blk, std::integral_constant<int, 0>());
        step(blk + 1, std::integral_constant<int, 1>());
    }
    __syncthreads();                            // W3's part of the last block is visible
    if (cx.nblk > 0) finish_prev((int)((cx.nblk - 1) & 1));   // (no blocks: none)
}

// W3: tokens 32..63, off-diagonal scores P^T(0,1) and their V^T P^T part,
// and the state scan's last tile (pos: block 0)
template <int D, bool WALK>
__device__ void out1x_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 1, 0, ln.l32, ln.h);
    Scan<D, WALK, D / 32 - 1, 1> sc(cx, lane);
    sc.init(cx, wk, pos, sm);
    auto step = [&](auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        const int c = block_len(pos.t0, pos.n);
        const bool last = Walk<WALK>::last(pos);
        if constexpr (WALK) lds_barrier();
        else __syncthreads();
        sc.template step<BUF>(cx, wk, pos, sm, c, last);
        bf16x8 qf[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = ld8(&sm.Q[BUF][32 + ln.l32][16 * ks + 8 * ln.h]);
        f32x16 acc = {};
        score_pv<D>(sm, BUF, 0, qf, dec, ln, acc);
        float4 *op = reinterpret_cast<float4 *>(&sm.OP[BUF][lane][0]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            op[u] = make_float4(acc[4 * u + 0], acc[4 * u + 1], acc[4 * u + 2], acc[4 * u + 3]);
        wk.next(pos);
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(std::integral_constant<int, 0>());
        step(std::integral_constant<int, 1>());
    }
    __syncthreads();
    sc.finish(cx, pos);
}

// STRIDED = false: rows of q, k, v and out are D elements apart (a
// compile-time token stride; head and sequence offsets still come from the
// map), so the contiguous layouts pay nothing for stride support.
// WALK = false: one workgroup per (sequence, head, column slice); WALK = true:
// one per (head, column slice), walking all nseq sequences of a packed map.
template <int D, bool STRIDED, bool WALK>
__global__ __launch_bounds__(NTHREADS) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ slopes,
    uint16_t *__restrict__ out, float *__restrict__ state, SeqMap map, int64_t nseq)
{
    constexpr int NJ = D / PJ;            // workgroups per head
    __shared__ Smem<D> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);

    // XCD-aware placement: workgroup i runs on XCD i % 8 and workgroups start
    // in index order.  Workgroups 8q + x (x = 0..7) take slice q % NJ of
    // (sequence, head) slot 8 (q / NJ) + x (WALK: of head 8 (q / NJ) + x): the
    // NJ slices of one head run on one XCD at the same time (Q and K come from
    // HBM once, then from that XCD's L2), and consecutive heads of a sequence
    // go to different XCDs, so every XCD gets an equal share of every
    // sequence however long it is.
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
    Walk<WALK> wk;
    wk.map = map;
    wk.nseq = nseq;
    wk.h = WALK ? bh : bh % map.H;
    wk.tb = nullptr;
    wk.slot = nullptr;
    const int lane = tid % 64;
    if constexpr (WALK) {
        __shared__ WalkTable tb;
        __shared__ __attribute__((aligned(16))) float slot[D * 32];   // state rows [D][32], staged / drained
        if (wave == 0) build_table(tb, map, nseq, lane);
        __syncthreads();
        wk.tb = &tb;
        wk.slot = slot;
    }
    const Pos p0 = wk.first(WALK ? 0 : bh / map.H);

    Ctx<D> cx;
    cx.q = q;
    cx.k = k;
    cx.v = v;
    cx.o = out;
    cx.state = state;
    cx.H = map.H;
    cx.h = wk.h;
    cx.j0 = (int)slice * PJ;
    cx.s = slopes[wk.h];
    // blocks processed: a multiple of NSET (trailing empty blocks are no-ops;
    // an empty sequence leaves its state unchanged)
    cx.nblk = (wk.blocks(p0) + NSET - 1) / NSET * NSET;
    cx.ts = STRIDED ? (int)map.in.st : D;
    cx.ots = STRIDED ? (int)map.out.st : D;

    switch (wave) {
        case 0: scan_wave<D>(cx, wk, p0, sm, lane); break;
        case 1: out0_wave<D>(cx, wk, p0, sm, lane); break;
        case 2: out1_wave<D>(cx, wk, p0, sm, lane); break;
        case 3: out1x_wave<D>(cx, wk, p0, sm, lane); break;
        default: producer<D>(cx, wk, p0, sm, tid - 64 * NCONS); break;
    }
}

// compute units of the current device (0 if unknown), looked up once per device
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace

int64_t prefill_bf16_grid(int64_t seqs, int64_t H, int d) { return seqs * H * (d / PJ); }

// A packed launch walks its sequences inside one workgroup per (head, column
// slice) when the sequences are short on average (below WALK_MEAN_LEN tokens:
// the walk saves each (sequence, head, slice) its own pipeline fill and drain,
// while a grid of one workgroup per (sequence, head, slice) lets the hardware
// balance long sequences over the compute units as workgroups finish), when
// those workgroups fill whole waves of the device's compute units (every
// workgroup then does the same work: all tokens of its head) and when the
// offsets fit the walk's table (fewer than 2^31 tokens; batches of more than
// WALK_SEQS sequences are walked WALK_SEQS at a time, one launch each).
constexpr int64_t WALK_MEAN_LEN = 8192;

bool prefill_bf16_walks(int64_t seqs, int64_t H, int64_t T, int d, bool packed)
{
    if (!packed || seqs < 2 || T > 0x7fffffff || T / seqs >= WALK_MEAN_LEN) return false;
    const int cus = device_cus();
    return cus > 0 && (H * (d / PJ)) % cus == 0;
}

template <bool WALK>
const void *prefill_fn(int d, bool strided)
{
    if (d == 64)
        return strided ? (const void *)prefill_bf16_kernel<64, true, WALK>
                       : (const void *)prefill_bf16_kernel<64, false, WALK>;
    return strided ? (const void *)prefill_bf16_kernel<128, true, WALK>
                   : (const void *)prefill_bf16_kernel<128, false, WALK>;
}

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *slopes, uint16_t *out, float *state,
                               int64_t seqs, const SeqMap &map, int d, hipStream_t stream)
{
    const bool strided = map.in.st != d || map.out.st != d;
    const dim3 block(NTHREADS);
    if (!prefill_bf16_walks(seqs, map.H, map.T, d, map.cu != nullptr)) {
        SeqMap m = map;
        int64_t nseq = seqs;
        void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                        (void *)&out, (void *)&state, (void *)&m, (void *)&nseq};
        return hipLaunchKernel(prefill_fn<false>(d, strided),
                               dim3((unsigned)prefill_bf16_grid(seqs, map.H, d)), block, args, 0,
                               stream);
    }
    for (int64_t s0 = 0; s0 < seqs; s0 += WALK_SEQS) {
        SeqMap m = map;
        m.cu = map.cu + s0;
        int64_t nseq = seqs - s0 < WALK_SEQS ? seqs - s0 : WALK_SEQS;
        float *st = state + s0 * map.H * d * d;
        void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                        (void *)&out, (void *)&st, (void *)&m, (void *)&nseq};
        const hipError_t e = hipLaunchKernel(prefill_fn<true>(d, strided),
                                             dim3((unsigned)prefill_bf16_grid(1, map.H, d)), block,
                                             args, 0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace la
