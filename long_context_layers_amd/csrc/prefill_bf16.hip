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
// What bounds it: memory traffic, not arithmetic.  A copy of the kernel
// with the consumers' LDS reads and MFMAs removed (the same loads and stores,
// no compute) takes as long as the kernel itself, and one whose package power
// falls below the limit (the redundant score tiles skipped) runs its clock
// 12% higher in the same time.  Two parts of the traffic cost more than their
// HBM bytes: each workgroup of a head pulls the full Q and K blocks through
// its XCD's L2 (three of every four Q/K bytes a compute unit reads are L2
// hits; reading only its own quarter, the same HBM bytes stream 1.4x faster),
// and the output rows are shared between two workgroups per 128-byte line.
// The layout therefore keeps the L2 sharing on one XCD (spreading a head's
// slices over XCDs doubles the time), writes the output as 64-byte row slices
// (below), and keeps each operand's LDS reads few: 32x32x16 MFMAs (half the
// operand bytes per flop of 16x16x32), scores kept in registers and fed
// straight into V^T P^T, Q fragments shared by the score and inter-term
// products, and double-buffered tiles and state copy behind a single barrier
// per block (without it, waves that finish early run ahead and starve the
// busiest one).
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
#include "qk_prologue.h"

#include <algorithm>
#include <atomic>
#include <cmath>
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
constexpr int PJ = 32;        // state / output columns of one column tile
constexpr int NCONS = 4;      // consumer waves
constexpr int PT = 256;       // producer threads (4 waves)
constexpr int NTHREADS = 64 * NCONS + PT;
// producer register sets (blocks in flight; even): 4, or 2 with the fused
// QK prologue (PRO), whose per-lane constants and arithmetic need the registers
template <bool PRO>
constexpr int nset() { return PRO ? 2 : 4; }
static_assert(nset<false>() % 2 == 0 && nset<true>() % 2 == 0, "set i stages into LDS buffer i % 2");
constexpr int QPAD = 8;       // bf16 padding of Q and state-copy rows

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

// NJT: 32-column tiles of the state and output per workgroup (1 or 2)
template <int D, int NJT>
struct alignas(16) Smem {
    static constexpr int W = PJ * NJT;    // columns of the workgroup
    uint16_t Q[2][PC][D + QPAD];     // Q blocks, token-major
    uint16_t K[2][PC][D];            // K blocks, token-major, chunk-swizzled
    uint16_t V[2][PC][W];            // V slices, token-major
    uint16_t VW[2][PC][W];           // V slices times lambda^(c-1-b)
    uint16_t ST[2][W][D + QPAD];     // bf16 copies of the state slice, transposed
    float OP[2][64][16 * NJT + 4];   // W3 -> W2 partial outputs (one lane's 16 values per tile)
    uint16_t OT[2][32][W];           // W1 / W2 output tiles on their way to memory (swizzled)
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
    int64_t tok0;               // the sequence's first token in a packed launch (0: dense)
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
    int empty[WALK_SEQS];       // the empty sequences (their states are zeroed from a zero start)
    int nempty;
};

// The sequences of a walking launch can be walked as `groups` groups side by
// side (more workgroups when one per head and column slice would leave compute
// units idle): a sequence belongs to the group its clamped start offset falls
// in when the launch's token range is cut into `groups` equal parts, so the
// groups carry about equal numbers of tokens, and every sequence, however
// malformed its offsets, belongs to exactly one group.
__device__ __forceinline__ int walk_group(int64_t start, int64_t first, int64_t span, int groups)
{
    if (groups <= 1 || span <= 0) return 0;
    const int64_t g = max(start - first, (int64_t)0) * groups / span;
    return (int)min(g, (int64_t)groups - 1);
}

// one wave fills the table with the sequences of group `group` (a barrier must
// follow before anyone reads it)
__device__ void build_table(WalkTable &tb, const SeqMap &m, int64_t nseq, int lane, int group)
{
    const int groups = m.walk_groups;
    const int64_t first = min(max(m.cu[0], (int64_t)0), m.T);
    const int64_t span = min(max(m.cu[nseq], (int64_t)0), m.T) - first;
    int count = 0, nblk = 0, nempty = 0;
    for (int64_t base = 0; base < nseq; base += 64) {
        const int64_t s = base + lane;
        int a = 0, n = 0;
        bool mine = false;
        if (s < nseq) {
            const int64_t a64 = min(max(m.cu[s], (int64_t)0), m.T);
            a = (int)a64;
            n = (int)(min(max(m.cu[s + 1], a64), m.T) - a64);
            mine = walk_group(a64, first, span, groups) == group;
        }
        if (!mine) n = 0;
        const uint64_t mask = __ballot(n > 0);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
        if (n > 0) {
            tb.seq[count + before] = (int)s;
            tb.start[count + before] = a;
            tb.len[count + before] = n;
        }
        count += __popcll(mask);
        const bool empty = mine && n == 0;
        const uint64_t emask = __ballot(empty);
        const int ebefore = __builtin_amdgcn_mbcnt_hi((uint32_t)(emask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)emask, 0));
        if (empty) tb.empty[nempty + ebefore] = (int)s;
        nempty += __popcll(emask);
        int b = (n + PC - 1) / PC;
        for (int off = 32; off > 0; off >>= 1) b += __shfl_xor(b, off);
        nblk += b;
    }
    if (lane == 0) {
        tb.count = count;
        tb.nblk = nblk;
        tb.nempty = nempty;
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
        Pos p = {nseq, 0, 0, 0, 0, j, 0};
        if (j < uni(tb->count)) {
            const int64_t a = uni(tb->start[j]);
            p.tok0 = a;
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
            Pos p = {seq, 0, 0, 0, 0, 0, 0};
            seq_slice(map, seq, h, &p.in0, &p.out0, &p.n);
            if (map.cu) p.tok0 = min(max(map.cu[seq], (int64_t)0), map.T);
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
    // WALK: the block starts a sequence that starts from a zero state (its
    // inter term is 0: nothing is carried in)
    template <class C>
    __device__ static bool fresh(const C &cx, const Pos &p) { return WALK && cx.zero_init && p.t0 == 0; }
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
    int64_t H, h, nblk;               // nblk: blocks processed (a multiple of the producer's sets)
    int ts, ots;                      // token strides (elements) of q/k/v and of out (<= 2^24)
    float s;
    int j0;
    bool zero_init;                   // states start at zero and are only written
    bool state_out;                   // final states written (false: from zero, outputs only)

    // this workgroup's columns of the state of sequence seq: element (i, j) at i * D + j
    __device__ float *state_of(int64_t seq) const { return state + (seq * H + h) * D * D + j0; }
};

// ---- producer waves: global -> registers -> LDS ----------------------------

template <int D, int NJT>
struct Regs {                        // one block's share of a producer thread
    static constexpr int NQ = PC * D / 8 / PT;   // 16-byte chunks of Q (and of K)
    uint4 q[NQ], k[NQ], v[NJT];      // v[t]: column tile t of the V slice
    int c;                           // tokens in the block
    int64_t pos;                     // its first token's place in the packed token order
};

template <int D, int NJT>
struct Addr {                        // per-thread byte offsets inside a block
    uint32_t qk[Regs<D, NJT>::NQ];
    uint32_t v[NJT];
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

// The loads of one block into a register set: the parts PARTS of it (a mask
// of PART_Q, PART_K, PART_V), and its tokens and position with PART_META.
// (PRO: the quad layout's offsets are ad.qk[0] + 64 u, immediate offsets of
// one register.)
constexpr int PART_Q = 1, PART_K = 2, PART_V = 4, PART_META = 8, PART_ALL = 15;

template <int D, int NJT, bool PRO, int PARTS = PART_ALL>
__device__ __forceinline__ void load_block(Regs<D, NJT> &r, const Ctx<D> &cx, const Pos &p,
                                           const Addr<D, NJT> &ad)
{
    if constexpr ((PARTS & (PART_Q | PART_K)) != 0) {
        const __amdgpu_buffer_rsrc_t rq = block_rsrc<D>(cx.q + p.in0, p.t0, p.n, cx.ts);
        const __amdgpu_buffer_rsrc_t rk = block_rsrc<D>(cx.k + p.in0, p.t0, p.n, cx.ts);
#pragma unroll
        for (int u = 0; u < Regs<D, NJT>::NQ; ++u) {
            const uint32_t off = PRO ? ad.qk[0] + 16 * pro::LPR * u : ad.qk[u];
            if constexpr ((PARTS & PART_Q) != 0) r.q[u] = bload16(rq, off);
            if constexpr ((PARTS & PART_K) != 0) r.k[u] = bload16(rk, off);
        }
    }
    if constexpr ((PARTS & PART_V) != 0) {
        const __amdgpu_buffer_rsrc_t rv = block_rsrc<D>(cx.v + p.in0, p.t0, p.n, cx.ts);
#pragma unroll
        for (int t = 0; t < NJT; ++t) r.v[t] = bload16(rv, ad.v[0] + 2 * PJ * t);
    }
    if constexpr ((PARTS & PART_META) != 0) {
        r.c = block_len(p.t0, p.n);
        r.pos = p.tok0 + p.t0;
    }
}

__device__ __forceinline__ uint32_t scale_pair(uint32_t x, float w) {
    return pack_bf16x2(bf16_to_f32(x & 0xffffu) * w, bf16_to_f32(x >> 16) * w);
}

// Q/K chunk u of producer thread p: its row of the block and 16-byte chunk.
// Without the prologue 16 lanes (D = 128) cover a row, chunk p % (D/8) of
// rows p / (D/8) + u PT / (D/8); with it (PRO) a quad of lanes covers one
// row p / 4, chunks p % 4 + 4u (the prologue's layout: one position per lane).
template <int D, bool PRO>
__device__ __forceinline__ void qk_slot(int p, int u, int &row, int &c8)
{
    if constexpr (PRO) {
        row = p / pro::LPR;
        c8 = p % pro::LPR + pro::LPR * u;
    } else {
        row = (p + PT * u) / (D / 8);
        c8 = p % (D / 8);
    }
}

// registers -> LDS buffer BUF: the parts PARTS of the set; wv = lambda^(c-1-b)
// for this thread's token b (thread p holds 16 bytes of V row p / 4 in each
// column tile)
template <int D, int NJT, int BUF, bool PRO, int PARTS = PART_ALL>
__device__ __forceinline__ void store_block(const Regs<D, NJT> &r, Smem<D, NJT> &sm, int p, float wv)
{
#pragma unroll
    for (int u = 0; u < Regs<D, NJT>::NQ; ++u) {
        int row, c8;
        qk_slot<D, PRO>(p, u, row, c8);
        if constexpr ((PARTS & PART_Q) != 0)
            *reinterpret_cast<uint4 *>(&sm.Q[BUF][row][c8 * 8]) = r.q[u];
        if constexpr ((PARTS & PART_K) != 0)
            *reinterpret_cast<uint4 *>(&sm.K[BUF][row][(c8 ^ kswz(row)) * 8]) = r.k[u];
    }
    if constexpr ((PARTS & PART_V) == 0) return;
    const int vrow = p / 4;
#pragma unroll
    for (int t = 0; t < NJT; ++t) {
        const int vc = PJ * t + (p % 4) * 8;
        *reinterpret_cast<uint4 *>(&sm.V[BUF][vrow][vc]) = r.v[t];
        uint4 w;
        w.x = scale_pair(r.v[t].x, wv);
        w.y = scale_pair(r.v[t].y, wv);
        w.z = scale_pair(r.v[t].z, wv);
        w.w = scale_pair(r.v[t].w, wv);
        *reinterpret_cast<uint4 *>(&sm.VW[BUF][vrow][vc]) = w;
    }
}

// The fused prologue's per-thread state (PROT >= 0: QK Norm + RoPE with PROT
// rotary dims on the Q and K chunks before they go to LDS; -1: none).
template <int PROT>
struct ProState {
    pro::Lane<PROT> ln;
    pro::BlockAngles<PROT> an;       // the angles of the thread's row, block after block
    int64_t pos;                     // position of the thread's row in a block at pos 0
    float eps;
};
template <>
struct ProState<-1> {
};

// lambda^(c-1-b) for this thread's token b of a block of c tokens
template <int D>
__device__ __forceinline__ float v_weight(const Ctx<D> &cx, int c, int p, float wfull)
{
    const int b = p / 4;
    return c == PC ? wfull : (b < c ? decay_pow(cx.s, c - 1 - b) : 0.0f);
}

template <int D, int NJT, int BUF, int PROT>
__device__ __forceinline__ void produce_store(const Ctx<D> &cx, Smem<D, NJT> &sm, Regs<D, NJT> &r,
                                              int p, float wfull, ProState<PROT> &ps)
{
    constexpr bool PRO = PROT >= 0;
    if constexpr (PRO) {                 // row p/4 of the block, at position ps.pos + r.pos
        const pro::RowAngles &a = ps.an.next(ps.ln, ps.pos + r.pos);
        pro::norm_rope<PROT>(r.q, ps.ln.wq, a, ps.eps);
        pro::norm_rope<PROT>(r.k, ps.ln.wk, a, ps.eps);
    }
    store_block<D, NJT, BUF, PRO>(r, sm, p, v_weight(cx, r.c, p, wfull));
}

// One producer step per block blk: after the block's barrier, stage block
// blk+1 (register set SET) into the other LDS buffer, then reload SET with
// block blk+1+NSET (NSET = nset<PRO>(), at ld, which then moves on).  Loads past the end return
// zeros without touching memory, so nothing here is conditional (exact vmcnt
// waits).  With the prologue (PRO) the set is staged and reloaded a part at
// a time, V, then Q, then K, so that the next loads start while the
// prologue's arithmetic runs.
template <int D, int NJT, int SET, bool WALK, int PROT>
__device__ __forceinline__ void produce_step(const Ctx<D> &cx, const Walk<WALK> &wk, Smem<D, NJT> &sm,
                                             Regs<D, NJT> (&rs)[nset<(PROT >= 0)>()], const Addr<D, NJT> &ad,
                                             Pos &ld, int p, float wfull, ProState<PROT> &ps)
{
    constexpr bool PRO = PROT >= 0;
    constexpr int BUF = SET % 2;
    __syncthreads();                                   // barrier of block blk
    Regs<D, NJT> &r = rs[SET];
    if constexpr (PRO) {
        store_block<D, NJT, BUF, PRO, PART_V>(r, sm, p, v_weight(cx, r.c, p, wfull));
        load_block<D, NJT, PRO, PART_V>(r, cx, ld, ad);
        const pro::RowAngles &a = ps.an.next(ps.ln, ps.pos + r.pos);
        pro::norm_rope<PROT>(r.q, ps.ln.wq, a, ps.eps);
        store_block<D, NJT, BUF, PRO, PART_Q>(r, sm, p, 0.0f);
        load_block<D, NJT, PRO, PART_Q>(r, cx, ld, ad);
        pro::norm_rope<PROT>(r.k, ps.ln.wk, a, ps.eps);
        store_block<D, NJT, BUF, PRO, PART_K>(r, sm, p, 0.0f);
        load_block<D, NJT, PRO, PART_K | PART_META>(r, cx, ld, ad);
    } else {
        produce_store<D, NJT, BUF>(cx, sm, r, p, wfull, ps);
        load_block<D, NJT, PRO>(r, cx, ld, ad);
    }
    wk.next(ld);
}

// the NSET producer steps of one round, sets 1 .. NSET-1, then 0
template <int D, int NJT, bool WALK, int PROT, int I>
struct ProduceRound {
    __device__ static __forceinline__ void run(const Ctx<D> &cx, const Walk<WALK> &wk, Smem<D, NJT> &sm,
                                               Regs<D, NJT> (&rs)[nset<(PROT >= 0)>()],
                                               const Addr<D, NJT> &ad, Pos &ld, int p, float wfull,
                                               ProState<PROT> &ps) {
        constexpr int NSET = nset<(PROT >= 0)>();
        produce_step<D, NJT, I % NSET>(cx, wk, sm, rs, ad, ld, p, wfull, ps);
        if constexpr (I < NSET)
            ProduceRound<D, NJT, WALK, PROT, I + 1>::run(cx, wk, sm, rs, ad, ld, p, wfull, ps);
    }
};

template <int D, int NJT, bool WALK, int PROT>
__device__ void producer(const Ctx<D> &cx, const Walk<WALK> &wk, Pos ld, Smem<D, NJT> &sm, int p,
                         const QkPrologue &pr)
{
    constexpr bool PRO = PROT >= 0;
    ProState<PROT> ps;
    if constexpr (PRO) {
        static_assert(D == pro::PD && Regs<D, NJT>::NQ == pro::NC, "the prologue's row layout");
        ps.ln.init(pr, p % pro::LPR);
        ps.an.init(ps.ln);
        ps.pos = pr.pos0 + p / pro::LPR;
        ps.eps = pr.eps;
    }
    Addr<D, NJT> ad;
#pragma unroll
    for (int u = 0; u < Regs<D, NJT>::NQ; ++u) {
        int row, c8;
        qk_slot<D, PRO>(p, u, row, c8);
        ad.qk[u] = (uint32_t)((row * cx.ts + c8 * 8) * 2);
    }
#pragma unroll
    for (int t = 0; t < NJT; ++t)
        ad.v[t] = (uint32_t)(((p / 4) * cx.ts + cx.j0 + PJ * t + (p % 4) * 8) * 2);
    const float wfull = decay_pow(cx.s, PC - 1 - p / 4);       // lambda^(C-1-b)

    constexpr int NSET = nset<PRO>();
    Regs<D, NJT> rs[NSET];                                      // set i holds block i (mod NSET)
#pragma unroll
    for (int i = 0; i < NSET; ++i) {
        load_block<D, NJT, PRO>(rs[i], cx, ld, ad);
        wk.next(ld);
    }
    produce_store<D, NJT, 0>(cx, sm, rs[0], p, wfull, ps);
    load_block<D, NJT, PRO>(rs[0], cx, ld, ad);
    wk.next(ld);

    // block blk stages block blk+1 from set (blk+1) % NSET into buffer (blk+1) % 2
    for (int64_t blk = 0; blk < cx.nblk; blk += NSET)
        ProduceRound<D, NJT, WALK, PROT, 1>::run(cx, wk, sm, rs, ad, ld, p, wfull, ps);
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

// O^T(a-half ah) = scale * S^T Q^T from state copy SB and Q buffer QB, one
// accumulator per column tile (the Q fragments serve every tile)
template <int D, int NJT>
__device__ __forceinline__ void inter_term(const Smem<D, NJT> &sm, int qb, int sb, int ah,
                                           const Lane<D> &ln, float scale, bf16x8 (&qf)[D / 16],
                                           f32x16 (&acc)[NJT], bool zero_state = false)
{
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = ld8(&sm.Q[qb][32 * ah + ln.l32][16 * ks + 8 * ln.h]);
    if (zero_state) {                 // (what the products give on a zero state: +0)
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) acc[jt] = f32x16{};
        return;
    }
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
        f32x16 a = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            a = mfma(ld8(&sm.ST[sb][PJ * jt + ln.l32][16 * ks + 8 * ln.h]), qf[ks], a);
        acc[jt] = a * scale;
    }
}

// score tile P^T(bh, ah) (decayed) from Q fragments qf, then acc += V^T P^T
// over the tile's 32 tokens; the accumulator registers of P^T are the B
// operand directly (registers 8s..8s+7 hold tokens 32bh + 16s + 8e' + 4h + 0..3)
template <int D, int NJT>
__device__ __forceinline__ void score_pv(const Smem<D, NJT> &sm, int buf, int bh,
                                         const bf16x8 (&qf)[D / 16], const float (&dec)[16],
                                         const Lane<D> &ln, f32x16 (&acc)[NJT])
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
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
            const bf16x8 va = ldtr8(&sm.V[buf][r0][PJ * jt + 16 * ln.q2 + ln.tcol],
                                    &sm.V[buf][r0 + 8][PJ * jt + 16 * ln.q2 + ln.tcol]);
            acc[jt] = mfma(va, to_bf16x8(pacc, 8 * s2), acc[jt]);
        }
    }
}

// store a 32x32 O^T tile (tokens 32ah.., columns j0..j0+31) of the block at p.
// Accumulator register group q4 holds columns 8q4 + 4h + 0..3 of token a; a
// lane-half swap (lanes l <-> l+32) of groups (0,1) and (2,3) gives lane h
// columns 8h..8h+7 and 16+8h..16+8h+7 of token l32.  The tile goes through
// the wave's own 2 KB of LDS so that each 16-byte store instruction covers 16
// tokens with four lanes on each token's 64-byte slice, instead of 32 bytes of
// each of 32 tokens: half as many, twice as large pieces of the 128-byte
// lines that two workgroups share, which the memory system absorbs faster
// (the launch is bound by its memory traffic).  Chunk c (8 columns) of tile
// row r sits at chunk c ^ ((r >> 2) & 3): conflict-free for both the row-wise
// writes and the 4-lanes-per-row reads.
// (with two column tiles a row is 128 bytes, eight lanes a row: chunk c of row
// r sits at c ^ (r & 7))
template <int NJT>
__device__ __forceinline__ int ot_chunk(int r, int c) {
    return NJT == 1 ? c ^ ((r >> 2) & 3) : c ^ (r & 7);
}

// per lane, the byte offsets of its 16-byte pieces: store i covers tokens
// 32ah + i * 64/CPR .., CPR = 4 NJT lanes on each token's PJ * NJT columns
template <int D, int NJT>
__device__ __forceinline__ int out_offset(const Ctx<D> &cx, int ah, int i, int lane) {
    constexpr int CPR = 4 * NJT;
    return ((32 * ah + i * (64 / CPR) + lane / CPR) * cx.ots + cx.j0 + 8 * (lane % CPR)) * 2;
}

template <int D, int NJT>
__device__ __forceinline__ void store_out(const Ctx<D> &cx, const Pos &p, const int (&ooff)[2 * NJT],
                                          const f32x16 (&acc)[NJT], uint16_t (*ot)[PJ * NJT],
                                          const Lane<D> &ln, int lane)
{
    constexpr int CPR = 4 * NJT;                  // 16-byte chunks per tile row
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const int g0 = 2 * pr, g1 = 2 * pr + 1;
            unsigned x0 = pack_bf16x2(acc[jt][4 * g0 + 0], acc[jt][4 * g0 + 1]);
            unsigned x1 = pack_bf16x2(acc[jt][4 * g0 + 2], acc[jt][4 * g0 + 3]);
            unsigned y0 = pack_bf16x2(acc[jt][4 * g1 + 0], acc[jt][4 * g1 + 1]);
            unsigned y1 = pack_bf16x2(acc[jt][4 * g1 + 2], acc[jt][4 * g1 + 3]);
            const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
            uint4 o;
            o.x = s0[0]; o.y = s1[0]; o.z = s0[1]; o.w = s1[1];
            *reinterpret_cast<uint4 *>(&ot[ln.l32][8 * ot_chunk<NJT>(ln.l32, 4 * jt + ln.h + 2 * pr)]) = o;
        }
    asm volatile("" : : : "memory");              // the reads below follow the writes
    const __amdgpu_buffer_rsrc_t ro = block_rsrc<D>(cx.o + p.out0, p.t0, p.n, cx.ots);   // rows past the end dropped
#pragma unroll
    for (int i = 0; i < CPR / 2; ++i) {
        const int r = (64 / CPR) * i + lane / CPR;
        const uint4 x = *reinterpret_cast<const uint4 *>(&ot[r][8 * ot_chunk<NJT>(r, lane % CPR)]);
        const u32x4 w = {x.x, x.y, x.z, x.w};
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, ooff[i], 0, 0);
    }
    asm volatile("" : : : "memory");              // the next tile's writes follow these reads
}

// bf16 copy of state tile it (rows 32it..) of column tile jt into ST[buf][j][i]
template <int D, int NJT>
__device__ __forceinline__ void write_st(Smem<D, NJT> &sm, int buf, int it, int jt,
                                         const Lane<D> &ln, const f32x16 &s)
{
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        uint2 p;
        p.x = pack_bf16x2(s[4 * q4 + 0], s[4 * q4 + 1]);
        p.y = pack_bf16x2(s[4 * q4 + 2], s[4 * q4 + 3]);
        *reinterpret_cast<uint2 *>(&sm.ST[buf][PJ * jt + ln.l32][32 * it + 8 * q4 + 4 * ln.h]) = p;
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
// slack) the last.  With NJT column tiles each row tile has NJT accumulators
// (sacc[jt][t]); the walk runs one column tile.
template <int D, int NJT, bool WALK, int T0, int NTL>
struct Scan {
    static_assert(!WALK || NJT == 1, "the walk's state hand-over moves one column tile");
    Lane<D> ln;
    float full_decay;
    f32x16 sacc[NJT][NTL];

    __device__ Scan(const Ctx<D> &cx, int lane) : ln(lane), full_decay(decay_pow(cx.s, PC)) {}

    __device__ void init(const Ctx<D> &cx, const Walk<WALK> &wk, const Pos &pos, Smem<D, NJT> &sm) {
        if (pos.n > 0 && !cx.zero_init) {
            if constexpr (WALK) load_state<D, T0, NTL>(sacc[0], cx.state_of(pos.seq), ln);
            else {
                const float *St = cx.state_of(pos.seq);
#pragma unroll
                for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
                    for (int t = 0; t < NTL; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            sacc[jt][t][r] = St[(32 * (T0 + t) + 8 * (r / 4) + 4 * ln.h + r % 4) * D +
                                                PJ * jt + ln.l32];
            }
        } else {
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
                for (int t = 0; t < NTL; ++t) sacc[jt][t] = f32x16{};
        }
        if constexpr (WALK) {
            const int64_t s1 = wk.seq_at(pos.j + 1);
            if (s1 >= 0 && !cx.zero_init) stage_state<D, T0, NTL>(wk.slot, cx.state_of(s1), ln.l32 + 32 * ln.h, true);
        }
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int t = 0; t < NTL; ++t) write_st<D, NJT>(sm, 1, T0 + t, jt, ln, sacc[jt][t]);   // read by block 0
    }

    // block at pos (c tokens; last: it ends its sequence), LDS buffer BUF
    template <int BUF>
    __device__ void step(const Ctx<D> &cx, const Walk<WALK> &wk, const Pos &pos, Smem<D, NJT> &sm,
                         int c, bool last) {
        // WALK, no state written and the sequence ends here: its state after
        // this block is never used (the next sequence starts from zero and
        // its copy for the next block is written below)
        if (!(WALK && last && !cx.state_out)) update<BUF>(cx, sm, c);
        if constexpr (WALK) {
            if (last) hand_over<BUF>(cx, wk, pos, sm);
        }
    }

    // the block's decayed update of this wave's state tiles, and their bf16
    // copy for the next block's inter term
    template <int BUF>
    __device__ void update(const Ctx<D> &cx, Smem<D, NJT> &sm, int c) {
        const float sdec = c == PC ? full_decay : (c == 0 ? 1.0f : decay_pow(cx.s, c));
        bf16x8 vwf[NJT][PC / 16];
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int ks = 0; ks < PC / 16; ++ks) {
                const int r0 = 16 * ks + 8 * ln.h + ln.trow;
                vwf[jt][ks] = ldtr8(&sm.VW[BUF][r0][PJ * jt + 16 * ln.q2 + ln.tcol],
                                    &sm.VW[BUF][r0 + 4][PJ * jt + 16 * ln.q2 + ln.tcol]);
            }
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int col = 32 * (T0 + t) + 16 * ln.q2 + ln.tcol;   // feature of this lane's chunk
            const int ch = col >> 3, sub = col & 7;
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) sacc[jt][t] *= sdec;
#pragma unroll
            for (int ks = 0; ks < PC / 16; ++ks) {
                const int r0 = 16 * ks + 8 * ln.h + ln.trow;
                const bf16x8 ka = ldtr8(&sm.K[BUF][r0][((ch ^ kswz(r0)) * 8) + sub],
                                        &sm.K[BUF][r0 + 4][((ch ^ kswz(r0 + 4)) * 8) + sub]);
#pragma unroll
                for (int jt = 0; jt < NJT; ++jt) sacc[jt][t] = mfma(ka, vwf[jt][ks], sacc[jt][t]);
            }
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt) write_st<D, NJT>(sm, BUF, T0 + t, jt, ln, sacc[jt][t]);
        }
    }

    // WALK: at the end of a sequence, its final state out and the next one's in
    template <int BUF>
    __device__ void hand_over(const Ctx<D> &cx, const Walk<WALK> &wk, const Pos &pos, Smem<D, NJT> &sm) {
        if constexpr (WALK) {
            {
                // the next sequence's initial state out of LDS first: the
                // wait for its staging (issued a sequence ago) then covers no
                // store of this block
                const bool more = wk.seq_at(pos.j + 1) >= 0;
                f32x16 nxt[NTL];
                if (cx.zero_init) {
                    // from zero nothing is staged: no wait for the slot (which
                    // would also wait for the previous final state's stores)
#pragma unroll
                    for (int t = 0; t < NTL; ++t) nxt[t] = f32x16{};
                } else {
                    // the slot's direct loads (a sequence ago) have landed before
                    // it is read or refilled: they count as vector memory
                    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
                    if (more) read_staged<D, T0, NTL>(nxt, wk.slot, ln);
                }
                if (cx.state_out)
                    store_via_slot<D, T0, NTL>(wk.slot, cx.state_of(pos.seq), sacc[0], ln,   // the final state out
                                               ln.l32 + 32 * ln.h);
                if (more) {
                    // take up the next sequence (its bf16 copy over the one
                    // just written for the next block), then stage the one
                    // after it once the slot has been read
#pragma unroll
                    for (int t = 0; t < NTL; ++t) {
                        sacc[0][t] = nxt[t];
                        write_st<D, NJT>(sm, BUF, T0 + t, 0, ln, sacc[0][t]);
                    }
                    if (!cx.zero_init) {
                        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): the slot reads done
                        const int64_t s2 = wk.seq_at(pos.j + 2);
                        if (s2 >= 0) stage_state<D, T0, NTL>(wk.slot, cx.state_of(s2), ln.l32 + 32 * ln.h,
                                                             true);
                    }
                }
            }
        }
    }

    // one sequence (no walk): its final state, after the loop (a store inside
    // the step measured slower: it sits on the scan's sequential path)
    __device__ void finish(const Ctx<D> &cx, const Pos &pos) {
        if constexpr (!WALK) {
            if (cx.state_out && (cx.nblk > 0 || cx.zero_init)) {   // (an empty sequence from zero: zeros)
                float *St = cx.state_of(pos.seq);
#pragma unroll
                for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
                    for (int t = 0; t < NTL; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            St[(32 * (T0 + t) + 8 * (r / 4) + 4 * ln.h + r % 4) * D + PJ * jt + ln.l32] =
                                sacc[jt][t][r];
            }
        }
    }
};

// W0: the state scan on all tiles but the last (pos: block 0)
template <int D, int NJT, bool WALK>
__device__ void scan_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D, NJT> &sm, int lane)
{
    Scan<D, NJT, WALK, 0, D / 32 - 1> sc(cx, lane);
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

// the per-lane store offsets of a token half ah
template <int D, int NJT>
__device__ __forceinline__ void out_offsets(int (&ooff)[2 * NJT], const Ctx<D> &cx, int ah, int lane) {
#pragma unroll
    for (int i = 0; i < 2 * NJT; ++i) ooff[i] = out_offset<D, NJT>(cx, ah, i, lane);
}

// W1: tokens 0..31, complete
template <int D, int NJT, bool WALK>
__device__ void out0_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D, NJT> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 0, 0, ln.l32, ln.h);
    const float scale = decay_pow(cx.s, ln.l32 + 1);               // lambda^(a+1)
    int ooff[2 * NJT];
    out_offsets<D, NJT>(ooff, cx, 0, lane);
    auto step = [&](auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        __syncthreads();
        bf16x8 qf[D / 16];
        f32x16 acc[NJT];
        inter_term<D, NJT>(sm, BUF, BUF ^ 1, 0, ln, scale, qf, acc, Walk<WALK>::fresh(cx, pos));
        score_pv<D, NJT>(sm, BUF, 0, qf, dec, ln, acc);
        store_out<D, NJT>(cx, pos, ooff, acc, sm.OT[0], ln, lane);
        wk.next(pos);
    };
    for (int64_t blk = 0; blk < cx.nblk; blk += 2) {
        step(std::integral_constant<int, 0>());
        step(std::integral_constant<int, 1>());
    }
    __syncthreads();
}

// W2: tokens 32..63, inter term + diagonal scores; adds W3's part one block later
template <int D, int NJT, bool WALK>
__device__ void out1_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D, NJT> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 1, 1, ln.l32, ln.h);
    const float scale = decay_pow(cx.s, 32 + ln.l32 + 1);
    int ooff[2 * NJT];
    out_offsets<D, NJT>(ooff, cx, 1, lane);
    f32x16 prev[NJT] = {};
    Pos ppos = pos;                                                // block of prev
    auto finish_prev = [&](int pbuf) {                             // that block's tokens 32..63
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
            const float4 *op = reinterpret_cast<const float4 *>(&sm.OP[pbuf][lane][16 * jt]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 x = op[u];
                prev[jt][4 * u + 0] += x.x; prev[jt][4 * u + 1] += x.y;
                prev[jt][4 * u + 2] += x.z; prev[jt][4 * u + 3] += x.w;
            }
        }
        store_out<D, NJT>(cx, ppos, ooff, prev, sm.OT[1], ln, lane);
    };
    auto step = [&](int64_t blk, auto BUFC) {
        constexpr int BUF = decltype(BUFC)::value;
        __syncthreads();
        bf16x8 qf[D / 16];
        f32x16 acc[NJT];
        inter_term<D, NJT>(sm, BUF, BUF ^ 1, 1, ln, scale, qf, acc, Walk<WALK>::fresh(cx, pos));
        score_pv<D, NJT>(sm, BUF, 1, qf, dec, ln, acc);
        if (blk > 0) finish_prev(BUF ^ 1);
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) prev[jt] = acc[jt];
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
template <int D, int NJT, bool WALK>
__device__ void out1x_wave(const Ctx<D> &cx, const Walk<WALK> &wk, Pos pos, Smem<D, NJT> &sm, int lane)
{
    const Lane<D> ln(lane);
    float dec[16];
    score_decay(dec, cx.s, 1, 0, ln.l32, ln.h);
    Scan<D, NJT, WALK, D / 32 - 1, 1> sc(cx, lane);
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
        f32x16 acc[NJT] = {};
        score_pv<D, NJT>(sm, BUF, 0, qf, dec, ln, acc);
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
            float4 *op = reinterpret_cast<float4 *>(&sm.OP[BUF][lane][16 * jt]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                op[u] = make_float4(acc[jt][4 * u + 0], acc[jt][4 * u + 1], acc[jt][4 * u + 2],
                                    acc[jt][4 * u + 3]);
        }
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
// NJT: 32-column tiles per workgroup (2 halves how often each head's Q and K
// are read through L2 and writes whole 128-byte output lines, for half as
// many workgroups per head; the walk takes 1).
template <int D, bool STRIDED, bool WALK, int NJT, int PROT = -1>
__global__ __launch_bounds__(NTHREADS) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ slopes,
    uint16_t *__restrict__ out, float *__restrict__ state, SeqMap map, int64_t nseq,
    QkPrologue pr)
{
    static_assert(!WALK || NJT == 1, "the walk runs one column tile per workgroup");
    constexpr bool PRO = PROT >= 0;
    static_assert(!WALK || !PRO, "the fused prologue runs on dense and split launches");
    constexpr int NJ = D / (PJ * NJT);    // workgroups per head
    __shared__ Smem<D, NJT> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);

    // XCD-aware placement: workgroup i runs on XCD i % 8 and workgroups start
    // in index order.  Workgroups 8q + x (x = 0..7) take slice q % NJ of
    // (sequence, head) slot 8 (q / NJ) + x (WALK: of (group, head) slot
    // 8 (q / NJ) + x, the head being the slot modulo H): the
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
    wk.h = bh % map.H;                   // (WALK: head slot bh = group * H + head)
    wk.tb = nullptr;
    wk.slot = nullptr;
    const int lane = tid % 64;
    if constexpr (WALK) {
        __shared__ WalkTable tb;
        __shared__ __attribute__((aligned(16))) float slot[D * 32];   // state rows [D][32], staged / drained
        if (wave == 0) build_table(tb, map, nseq, lane, (int)(bh / map.H));
        __syncthreads();
        wk.tb = &tb;
        wk.slot = slot;
        if (map.zero_init && state) {    // empty sequences from zero: this slice of their states is 0
            const int64_t j0 = (int64_t)slice * PJ * NJT;
            for (int e = 0; e < tb.nempty; ++e) {
                float *st = state + ((int64_t)tb.empty[e] * map.H + wk.h) * D * D + j0;
                for (int i = tid; i < D * PJ * NJT / 4; i += NTHREADS) {
                    const int row = i / (PJ * NJT / 4), c4 = i % (PJ * NJT / 4);
                    *reinterpret_cast<float4 *>(st + row * D + 4 * c4) = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
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
    cx.j0 = (int)slice * PJ * NJT;
    cx.s = slopes[wk.h];
    cx.zero_init = map.zero_init != 0;
    cx.state_out = state != nullptr;
    // blocks processed: a multiple of the producer's sets (trailing empty blocks are no-ops;
    // an empty sequence leaves its state unchanged)
    constexpr int NSET = nset<PRO>();
    cx.nblk = (wk.blocks(p0) + NSET - 1) / NSET * NSET;
    cx.ts = STRIDED ? (int)map.in.st : D;
    cx.ots = STRIDED ? (int)map.out.st : D;

    switch (wave) {
        case 0: scan_wave<D, NJT>(cx, wk, p0, sm, lane); break;
        case 1: out0_wave<D, NJT>(cx, wk, p0, sm, lane); break;
        case 2: out1_wave<D, NJT>(cx, wk, p0, sm, lane); break;
        case 3: out1x_wave<D, NJT>(cx, wk, p0, sm, lane); break;
        default: producer<D, NJT, WALK, PROT>(cx, wk, p0, sm, tid - 64 * NCONS, pr); break;
    }
}


}  // namespace

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

int64_t prefill_bf16_grid(int64_t seqs, int64_t H, int d, int njt) {
    return seqs * H * (d / (PJ * njt));
}

// Column tiles per workgroup of a grid launch (one workgroup per sequence,
// head and column slice): 64-column workgroups (two tiles, d = 128) whenever
// they still fill the device — they read each head's Q and K through L2 half
// as often and write whole 128-byte output lines, so a block step costs 1.6x
// a 32-column one for twice the columns (measured: 16 sequences of 16K
// tokens at 64 heads 4.25 -> 3.39 ms, 74 mixed ones 4.57 -> 3.58 ms).  The
// dense B = 1 launch, where they would leave half the device idle, runs as
// segments instead (la_prefill_ws).
int prefill_bf16_grid_njt(int64_t seqs, int64_t H, int d)
{
    if (d != 128) return 1;
    const int cus = device_cus();
    return cus > 0 && 2 * H * seqs >= cus ? 2 : 1;
}

// A packed launch walks its sequences inside one workgroup per (head, column
// slice) when that is estimated to be faster than the grid launch above, and
// the sequences are short on average (below WALK_MEAN_LEN tokens: longer ones
// gain from the hardware balancing the grid over the compute units as
// workgroups finish) and the offsets fit the walk's table (fewer than 2^31
// tokens; batches of more than WALK_SEQS sequences are walked WALK_SEQS at a
// time, one launch each).  The estimates, in microseconds, fitted to measured
// launches (H = 32 and 64, 64 .. 16384 tokens per sequence and mixed lengths
// at 256K tokens, d = 128):
//   walk: rounds * (0.98 T/64 + 1.51 nseq) / G * (0.6 + 0.4 occupancy), where
//         G is the number of sequence groups walked side by side (as many as
//         fill the device with H * d/32 workgroups each, at most one per
//         sequence), rounds the number of device-fills the G * H * d/32
//         workgroups take, occupancy the share of those rounds' compute units
//         they use (a block step is that much shorter on a partly idle
//         device), and the per-sequence term the hand-over at a boundary plus
//         the partial last block;
//   grid, 64-column workgroups: 1.57 * (T/64 + 3.2 nseq) * 2H / CUs;
//   grid, 32-column workgroups: 1.05 * (T/64 + 4.25 nseq) * (H * d/32) / CUs,
//         the per-sequence terms being each workgroup's pipeline fill and
//         drain plus its block count rounded up to the producers' four-block
//         unroll.
// So the walk wins for sequences of up to about 256 tokens at 8 to 64 heads
// (measured at 256K tokens, walk / 64-column grid, ms: 64 heads 1024 x 256
// 5.63 / 5.85, 512 x 512 4.76 / 4.50; 32 heads 2.81 / 2.94 and 2.49 / 2.29;
// 8 heads 0.69 / 0.74 and 0.60 / 0.59), the wide grid for longer ones.
constexpr int64_t WALK_MEAN_LEN = 8192;

int prefill_bf16_walk_groups(int64_t nseq, int64_t H, int d)
{
    const int cus = device_cus();
    const int64_t wg = H * (d / PJ);
    if (cus <= 0 || wg >= cus) return 1;
    return (int)std::max<int64_t>(1, std::min<int64_t>(cus / wg, nseq));
}

bool prefill_bf16_walks(int64_t seqs, int64_t H, int64_t T, int d, bool packed)
{
    if (!packed || seqs < 2 || T > 0x7fffffff || T / seqs >= WALK_MEAN_LEN) return false;
    const int cus = device_cus();
    if (cus <= 0) return false;
    const double groups = prefill_bf16_walk_groups(std::min<int64_t>(seqs, WALK_SEQS), H, d);
    const double wg = (double)H * (d / PJ) * groups;
    const double rounds = std::ceil(wg / cus);
    const double occupancy = wg / (rounds * cus);
    const double blocks = (double)T / PC, n = (double)seqs;
    const double walk = rounds * (0.98 * blocks + 1.51 * n) / groups * (0.6 + 0.4 * occupancy);
    const double grid = prefill_bf16_grid_njt(seqs, H, d) == 2
                            ? 1.57 * (blocks + 3.2 * n) * 2.0 * H / cus
                            : 1.05 * (blocks + 4.25 * n) * wg / cus;
    return walk < grid;
}

template <bool WALK>
const void *prefill_fn(int d, bool strided)
{
    if (d == 64)
        return strided ? (const void *)prefill_bf16_kernel<64, true, WALK, 1>
                       : (const void *)prefill_bf16_kernel<64, false, WALK, 1>;
    return strided ? (const void *)prefill_bf16_kernel<128, true, WALK, 1>
                   : (const void *)prefill_bf16_kernel<128, false, WALK, 1>;
}

// A dense launch over B = 1 can run as S >= 2 segments of the sequence at
// once (one packed launch, the later segments from a zero state, then the
// fold of the states and the correction of the later segments' outputs).
// The segments take workgroups of njt 32-column tiles.  Two tiles (64
// columns, d = 128) pass each head's Q and K through L2 twice instead of four
// times and write every output row slice as one whole 128-byte line: a copy
// of the kernel with the compute removed streams the 256K, 64-head workload
// in 3.34 against 4.27 ms.  With njt tiles, S = CUs / (H * d/(32 njt)), each
// segment at least min_len tokens and at most MAX_SPLIT segments; the wide
// tiles are taken unless the narrow ones keep markedly more workgroups busy
// (few heads on a short sequence: the segment length bounds S).  The later
// segments' correction re-reads q and out for up to ~26K tokens of the
// slowest heads, so a split pays on short sequences only when the unsplit
// grid leaves compute units idle (segments from SPLIT_MIN_LEN tokens: at 32
// heads 8K tokens 115 -> 96 us, 16K 237 -> 164 us); when it fills the device
// the gain is the wide tiles' alone and needs segments from SPLIT_MIN_LEN_FULL
// (64 heads: 16K tokens 278 -> 261 us, but 8K 141 -> 148 us).
constexpr int64_t SPLIT_MIN_LEN = 4096;
constexpr int64_t SPLIT_MIN_LEN_FULL = 8192;
constexpr int MAX_SPLIT = 64;

int prefill_split_plan(int64_t B, int64_t H, int64_t N, int d, int *njt)
{
    *njt = 1;
    if (B != 1 || H < 1 || N < 2 * SPLIT_MIN_LEN) return 1;
    const int cus = device_cus();
    if (cus <= 0) return 1;
    const int64_t min_len = H * (d / PJ) >= cus ? SPLIT_MIN_LEN_FULL : SPLIT_MIN_LEN;
    int best_s = 1;
    double best = 0.0;
    for (int t = (d == 128 ? 2 : 1); t >= 1; --t) {
        const int64_t wg = H * (d / (PJ * t));
        int64_t S = std::min<int64_t>(cus / wg, N / min_len);
        S = std::min<int64_t>(S, MAX_SPLIT);
        if (S < 2) continue;
        const double busy = (double)std::min<int64_t>(S * wg, cus) * (t == 2 ? 1.2 : 1.0);
        if (busy > best) { best = busy; best_s = (int)S; *njt = t; }
    }
    return best_s;
}

// the fused-prologue kernels (d = 128, token strides at run time) by column
// tiles and rotary dims (null if unsupported)
template <int NJT>
const void *prologue_fn_njt(int rot)
{
    switch (rot) {
        case 0: return (const void *)prefill_bf16_kernel<128, true, false, NJT, 0>;
        case 16: return (const void *)prefill_bf16_kernel<128, true, false, NJT, 16>;
        case 32: return (const void *)prefill_bf16_kernel<128, true, false, NJT, 32>;
        case 64: return (const void *)prefill_bf16_kernel<128, true, false, NJT, 64>;
        case 128: return (const void *)prefill_bf16_kernel<128, true, false, NJT, 128>;
        default: return nullptr;
    }
}
const void *prologue_fn(int njt, int rot)
{
    return njt == 1 ? prologue_fn_njt<1>(rot) : prologue_fn_njt<2>(rot);
}

// one workgroup per (sequence, head, njt column tiles), never the walk
// (njt = 2: d = 128 only; the fused prologue pro, if given: d = 128 only)
hipError_t launch_prefill_bf16_nowalk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                      const float *slopes, uint16_t *out, float *state,
                                      int64_t seqs, const SeqMap &map, int d, hipStream_t stream,
                                      int njt, const QkPrologue *pro)
{
    const bool strided = map.in.st != d || map.out.st != d;
    if (njt != 1 && (njt != 2 || d != 128)) return hipErrorInvalidValue;
    if (pro && d != 128) return hipErrorInvalidValue;
    SeqMap m = map;
    int64_t nseq = seqs;
    QkPrologue pr = pro ? *pro : QkPrologue{nullptr, nullptr, 0.0, 0, 0.0f, 0};
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                    (void *)&out, (void *)&state, (void *)&m, (void *)&nseq, (void *)&pr};
    if (pro && !prologue_fn(njt, pro->rot)) return hipErrorInvalidValue;
    const void *fn;
    if (pro)
        fn = prologue_fn(njt, pro->rot);
    else
        fn = njt == 1 ? prefill_fn<false>(d, strided)
             : strided ? (const void *)prefill_bf16_kernel<128, true, false, 2>
                       : (const void *)prefill_bf16_kernel<128, false, false, 2>;
    return hipLaunchKernel(fn, dim3((unsigned)prefill_bf16_grid(seqs, map.H, d, njt)),
                           dim3(NTHREADS), args, 0, stream);
}

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *slopes, uint16_t *out, float *state,
                               int64_t seqs, const SeqMap &map, int d, hipStream_t stream)
{
    const bool strided = map.in.st != d || map.out.st != d;
    const dim3 block(NTHREADS);
    if (!prefill_bf16_walks(seqs, map.H, map.T, d, map.cu != nullptr))
        return launch_prefill_bf16_nowalk(q, k, v, slopes, out, state, seqs, map, d, stream,
                                          prefill_bf16_grid_njt(seqs, map.H, d), nullptr);
    for (int64_t s0 = 0; s0 < seqs; s0 += WALK_SEQS) {
        SeqMap m = map;
        m.cu = map.cu + s0;
        int64_t nseq = seqs - s0 < WALK_SEQS ? seqs - s0 : WALK_SEQS;
        m.walk_groups = prefill_bf16_walk_groups(nseq, map.H, d);
        float *st = state ? state + s0 * map.H * d * d : nullptr;
        QkPrologue pr = {nullptr, nullptr, 0.0, 0, 0.0f, 0};
        void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                        (void *)&out, (void *)&st, (void *)&m, (void *)&nseq, (void *)&pr};
        const hipError_t e = hipLaunchKernel(prefill_fn<true>(d, strided),
                                             dim3((unsigned)prefill_bf16_grid(m.walk_groups, map.H, d, 1)),
                                             block, args, 0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace la
