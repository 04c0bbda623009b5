// la_internal.h — declarations shared by the library's own translation units
// (kernel launchers and small device helpers).  Not installed, not part of the
// C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// Element strides of a tensor's rows: element (b or sequence, head h, token
// t, channel i) sits at b*sb + h*sh + t*st + i (channels contiguous).
struct Strides {
    int64_t sb, sh, st;
};

// Where the tokens of one (sequence, head) slice of a prefill launch live.
// Dense launches: slice (b, h) holds N tokens starting at b*sb + h*sh.  Packed
// launches: sequence i is tokens cu[i] .. cu[i+1] of every head, starting at
// h*sh + cu[i]*st (offsets clamped into [0, T], so malformed offsets still
// address only rows of the tensors; sb is unused).  q, k and v share `in`,
// the output has `out`.  The state of slice (seq, h) is state[(seq*H + h)*d*d ..].
struct SeqMap {
    const int64_t *cu;    // null: dense launch
    int64_t H, N, T;      // heads; dense sequence length; packed total length
    Strides in, out;
    int zero_init;        // 1: every sequence starts from a zero state and the states
                          // are only written (empty sequences: zeros), never read;
                          // with a null state pointer nothing is written
    int walk_groups;      // a walking launch: groups of its sequences walked side by side
                          // (0 or 1: one group)
};

// start offsets (elements) of slice (seq, h) in the inputs and the output, and its length
__device__ __forceinline__ void seq_slice(const SeqMap &m, int64_t seq, int64_t h,
                                          int64_t *in0, int64_t *out0, int64_t *len)
{
    if (!m.cu) {
        *in0 = seq * m.in.sb + h * m.in.sh;
        *out0 = seq * m.out.sb + h * m.out.sh;
        *len = m.N;
        return;
    }
    const int64_t a = min(max(m.cu[seq], (int64_t)0), m.T);
    const int64_t b = min(max(m.cu[seq + 1], a), m.T);
    *in0 = h * m.in.sh + a * m.in.st;
    *out0 = h * m.out.sh + a * m.out.st;
    *len = b - a;
}

// length of sequence seq (the same clamping as seq_slice)
__device__ __forceinline__ int64_t seq_len(const SeqMap &m, int64_t seq)
{
    if (!m.cu) return m.N;
    const int64_t a = min(max(m.cu[seq], (int64_t)0), m.T);
    return min(max(m.cu[seq + 1], a), m.T) - a;
}

// QK Norm + RoPE fused into the prefill's loads of q and k (kernel argument;
// the arithmetic is in qk_prologue.h)
struct QkPrologue {
    const float *qw, *kw;     // [128] fp32 RMSNorm weights of q and k
    double theta;             // RoPE base (> 1 when rot > 0)
    int rot;                  // rotary dims: 0, 16, 32, 64 or 128
    float eps;                // RMSNorm epsilon (a normal positive float)
    int64_t pos0;             // position of a sequence's first token
};

// ---- launchers (return the launch status; arguments already validated) ----
// Prefill over `seqs` sequences (B for dense launches, nseq for packed ones).
hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *slopes, uint16_t *out, float *state,
                               int64_t seqs, const SeqMap &map, int d, hipStream_t stream);
hipError_t launch_prefill_f32(const float *q, const float *k, const float *v,
                              const float *slopes, float *out, float *state,
                              int64_t seqs, const SeqMap &map, int d, hipStream_t stream);
// bf16 decode reads q, k, v through element strides (in.st unused by the
// single-token step); out is contiguous
hipError_t launch_decode_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *slopes, float *state, uint16_t *out,
                              int64_t B, int64_t H, int d, const Strides &in, hipStream_t stream);
hipError_t launch_decode_f32(const float *q, const float *k, const float *v,
                             const float *slopes, float *state, float *out,
                             int64_t B, int64_t H, int d, hipStream_t stream);

// T tokens per sequence in one step (1 <= T <= decode_multi_max_tokens())
hipError_t launch_decode_multi_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                    const float *slopes, const int32_t *n_commit, float *state,
                                    uint16_t *out, int64_t B, int64_t H, int T, int d,
                                    const Strides &in, hipStream_t stream);
hipError_t launch_decode_multi_f32(const float *q, const float *k, const float *v,
                                   const float *slopes, const int32_t *n_commit, float *state,
                                   float *out, int64_t B, int64_t H, int T, int d,
                                   hipStream_t stream);
int decode_multi_max_tokens();

// the layer's neighbouring ops (one workgroup per token)
hipError_t launch_qk_norm_rope(const uint16_t *qi, const uint16_t *ki, const uint16_t *vi,
                               int64_t in_stride, const float *qw, const float *kw, double theta,
                               int rot, int64_t pos0, float eps, uint16_t *qo, uint16_t *ko,
                               uint16_t *vo, int inplace, int64_t B, int64_t N, int64_t H, int d,
                               hipStream_t stream);
hipError_t launch_group_norm_gate(const uint16_t *o, const int64_t os[3], const uint16_t *g,
                                  int64_t gate_stride, const float *w, int group, float eps,
                                  uint16_t *y, int64_t B, int64_t N, int64_t H, int d,
                                  hipStream_t stream);

// sequence-sharded prefill: fold of the gathered local states (Horner order
// over the first nfold shards, lens = their token counts) and correction of a
// shard's local output with its incoming state
constexpr int MAX_CP_SHARDS = 64;
hipError_t launch_cp_fold(const float *loc, const int *lens, int nfold, const float *init,
                          float *out, const float *slopes, int64_t B, int64_t H, int d,
                          hipStream_t stream);
hipError_t launch_cp_correct(const uint16_t *q, const float *slopes, const float *s_in,
                             uint16_t *out, int64_t B, int64_t H, int64_t L, int d,
                             hipStream_t stream);
int64_t cp_correct_grid(int64_t B, int64_t H, int64_t L);

// one workgroup per (sequence, head, njt 32-column tiles): never the packed
// walk (njt = 2 only at d = 128)
// (pro: QK Norm + RoPE on q and k as they are loaded, d = 128; positions
// pro->pos0 + t, t counted from a dense sequence's start or, in a packed
// launch, from the first packed token: the segments of one sequence)
hipError_t launch_prefill_bf16_nowalk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                      const float *slopes, uint16_t *out, float *state,
                                      int64_t seqs, const SeqMap &map, int d, hipStream_t stream,
                                      int njt, const QkPrologue *pro = nullptr);

// the sequence split of a dense B = 1 prefill: segments per row (1 = no
// split) on the current device and the column tiles per workgroup (*njt), the
// workspace it needs, and the launches (prep, packed prefill, fold, correct)
int prefill_split_plan(int64_t B, int64_t H, int64_t N, int d, int *njt);
int64_t split_workspace_bytes(int64_t H, int nseg, int d);
// the split's segment length (a multiple of 64), its prep (slot 0 <- the
// caller's state, the others <- 0, *cu <- the segments' offsets after the
// slots) and its fold (each slot <- the state at its segment's end, the last
// into the caller's state)
int64_t split_segment(int64_t N, int nseg);
hipError_t launch_split_prep(const float *state, float *slots, int64_t **cu, int64_t H, int d,
                             int nseg, int64_t seg, int64_t N, hipStream_t stream);
hipError_t launch_split_fold(float *slots, float *state, const float *slopes, int64_t H, int d,
                             int nseg, int64_t seg, int64_t N, hipStream_t stream);
hipError_t launch_prefill_bf16_split(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                     const float *slopes, uint16_t *out, float *state,
                                     int64_t H, int64_t N, int d, int nseg, int njt,
                                     const Strides &in, const Strides &out_strides, void *workspace,
                                     hipStream_t stream, const QkPrologue *pro = nullptr);

// number of workgroups one prefill launch over `seqs` sequences uses, with
// njt 32-column tiles per workgroup
int64_t prefill_bf16_grid(int64_t seqs, int64_t H, int d, int njt = 1);
// whether a packed launch over seqs sequences (T tokens) walks them in one
// workgroup per (head, column slice) on the current device
bool prefill_bf16_walks(int64_t seqs, int64_t H, int64_t T, int d, bool packed);
// column tiles per workgroup of a grid launch (one workgroup per sequence,
// head and slice) over seqs sequences on the current device
int prefill_bf16_grid_njt(int64_t seqs, int64_t H, int d);
int64_t prefill_f32_grid(int64_t seqs, int64_t H, int d);
// compute units of the current device (0 if unknown)
int device_cus();
// segments of a dense fp32 prefill (B = 1) run at once (1: no split)
int prefill_f32_split_plan(int64_t B, int64_t H, int64_t N, int d);
// the fp32 split over nseg >= 2 segments of a dense [1,H,N,d] prefill;
// workspace as for the bf16 split (split_workspace_bytes)
hipError_t launch_prefill_f32_split(const float *q, const float *k, const float *v,
                                    const float *slopes, float *out, float *state, int64_t H,
                                    int64_t N, int d, int nseg, void *workspace,
                                    hipStream_t stream);

// ---- device helpers ----
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// two floats -> packed bf16 pair (round to nearest even; lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// lambda^n for n >= 0 as exp(-s n); n == 0 gives exactly 1 (also for s = +inf)
__device__ __forceinline__ float decay_pow(float s, int n) {
    return n == 0 ? 1.0f : expf(-s * (float)n);
}

}  // namespace la
