/*
 * lightning_attn.h — C ABI of the MI355X (gfx950) decayed causal linear
 * attention library (liblightning_attn.so).
 *
 * The operation.  The Ling and Ring 2.6 Technical Report (Fig. 2, the
 * linear-attention layer) puts a "linear attention kernel" between
 * QK-Norm/RoPE and the grouped RMSNorm; §4.1.1 describes it as linear
 * attention evaluated through an RNN-style recurrence that carries one
 * D x D state per (batch, head), i.e. a [B,H,D,D] tensor.  This library
 * computes that kernel with a per-head exponential decay:
 *
 *     lambda_h = exp(-slopes[h])
 *     o_t = sum_{s<=t} lambda_h^(t-s) (q_t . k_s) v_s + lambda_h^(t+1) q_t S_init
 *     S_t = lambda_h S_{t-1} + k_t^T v_t ,  o_t = q_t S_t ,  S_{-1} = S_init
 *
 * There is no scale factor and no normaliser inside the kernel (the layer
 * normalises afterwards).  Prefill evaluates the sum blockwise (intra-block
 * masked scores times V, plus the inter-block term from the state carried by
 * a decayed scan); decode applies the recurrence to one token.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *    and row-major (the strided calls below say otherwise).  q, k, v, out: [B][H][N][d] for prefill, [B][H][d] for a
 *    decode step.  State: [B][H][d][d] fp32 with i (the k index) slow and j
 *    (the v index) fast, so o = q . S is a row vector times a matrix.
 *    slopes: [H] fp32, shared by every sequence of the batch.
 *  - bf16 means IEEE bfloat16 (1-8-7), stored as 16-bit words.  Results are
 *    rounded to bf16 with round-to-nearest-even; accumulation is fp32 and the
 *    carried state is never rounded below fp32.
 *  - d must be 64 or 128 (LA_ERR_UNSUPPORTED otherwise).  B, H >= 1; N >= 0
 *    (N == 0 is a no-op that leaves the state unchanged; q, k, v and out may
 *    then be NULL, as empty tensors often are).
 *  - Pointers to activations and states must be 16-byte aligned (decode
 *    activations: aligned to their element size); slopes 4-byte aligned.
 *  - out must not overlap q, k, v or the state.
 *  - stream is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *    it and the call returns without synchronising; results are ready when
 *    the stream reaches them.  The library allocates no memory and keeps no
 *    per-call global state; concurrent calls on different streams with
 *    disjoint outputs are safe.  Results are deterministic: the same inputs
 *    on the same GPU give bitwise-equal outputs.
 *  - Argument checks run on the host before any HIP call.  Data values are
 *    not validated: slopes >= 0 (lambda <= 1) is the method's domain; +inf
 *    is accepted and means lambda = 0.
 *  - Return value: LA_OK, or an la_status error code (see la_status_string).
 *    On an error nothing has been enqueued, except LA_ERR_HIP, which reports
 *    a failed launch (the status hipLaunchKernel returned).
 */
#ifndef LIGHTNING_ATTN_H
#define LIGHTNING_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1,  /* null pointer, negative or overflowing size */
    LA_ERR_UNSUPPORTED = 2,  /* d not in {64, 128}, or a grid too large */
    LA_ERR_HIP = 3           /* the kernel launch failed */
} la_status;

/*
 * Prefill, bf16 activations (the hot path).
 *   q, k, v     [B,H,N,d] bf16, read only.
 *   slopes      [H] fp32, read only.
 *   out         [B,H,N,d] bf16, written.
 *   state       [B,H,d,d] fp32, IN/OUT: on entry the initial state S_init
 *               (zero-fill it for a fresh sequence), on exit S_{N-1}.  Passing
 *               the state of one call into the next continues the sequence
 *               (chunked prefill): results equal one call over the
 *               concatenated tokens up to rounding.
 * Source: the report's §4.1.1 (local state and local output per sequence
 * shard, folded through the carried [B,H,D,D] state) and Fig. 2.
 */
int la_prefill(const void *q, const void *k, const void *v, const float *slopes,
               void *out, float *state,
               int64_t B, int64_t H, int64_t N, int64_t d, void *stream);

/*
 * Dense bf16 prefill that cuts each head's sequence into segments run at once
 * when B = 1: with workgroups of 64 output columns (d = 128; 32 at d = 64),
 * which read each head's Q and K through L2 half as often as la_prefill's
 * and write whole 128-byte output lines, S = CUs / (H * d/64) segments (each
 * at least 4096 tokens when la_prefill's grid of H * d/32 workgroups leaves
 * compute units idle, else at least 8192; at most 64 of them; none below 2)
 * run in one launch, the first from the caller's state and the others from zero; the
 * segments' states are then chained into the state at each boundary and the
 * final state, and each later segment's outputs are corrected with the state
 * at its start (o_a += lambda^(a+1) q_a S for its local token index a).  This
 * is the report's context-parallel decomposition (§4.1.1, Fig. 10: local
 * output and local state per piece, joined through the carried state) run on
 * one device.  Same semantics and argument rules as la_prefill; results equal
 * la_prefill's within rounding (the later segments' outputs are rounded to
 * bf16 once more).  Tokens whose factor lambda^(a+1) is exactly 0 in fp32 get
 * no correction work.
 *   la_prefill_workspace_bytes: the workspace bytes la_prefill_ws needs for
 *     these sizes on the calling thread's current device, written to *bytes;
 *     0 means no split (la_prefill_ws then runs exactly as la_prefill and
 *     ignores the workspace).  LA_ERR_INVALID_ARG for a null bytes, B or H
 *     below 1 or N below 0; LA_ERR_UNSUPPORTED for d other than 64 or 128.
 *     Enqueues nothing.
 *   la_prefill_ws: workspace is device memory of at least that many bytes,
 *     256-byte aligned, owned by the caller, not overlapping any argument; its
 *     contents on entry do not matter and are unspecified afterwards.  Calls
 *     that share a workspace must be ordered (one stream).  LA_ERR_INVALID_ARG
 *     also for a workspace that is null, smaller than needed, misaligned or
 *     overlapping, when a split is planned.
 */
int la_prefill_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t *bytes);
int la_prefill_ws(const void *q, const void *k, const void *v, const float *slopes,
                  void *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                  void *workspace, int64_t workspace_bytes, void *stream);

/*
 * la_prefill_ws without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing: when a sequence
 * split is planned it uses a scratch array of 8 MiB + 4 KiB that the library
 * holds on each device it runs on until the process ends (found on the first
 * call on that device; the split needs at most 32 KiB per compute unit plus
 * a few hundred bytes); a split needing more (only on devices with more than
 * 256 compute units) gives LA_ERR_UNSUPPORTED.  Every call on one device shares
 * that array and sets up what it reads itself, so calls that overlap on one
 * device (other streams, other threads) race; order them.  Same semantics,
 * argument rules and results as la_prefill_ws; LA_ERR_HIP also if the
 * scratch cannot be found.
 */
int la_prefill_noalloc(const void *q, const void *k, const void *v, const float *slopes,
                       void *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                       void *stream);

/* Prefill with fp32 activations: same semantics, q, k, v, out are float. */
int la_prefill_f32(const float *q, const float *k, const float *v, const float *slopes,
                   float *out, float *state,
                   int64_t B, int64_t H, int64_t N, int64_t d, void *stream);

/*
 * la_prefill_f32 with a caller's workspace: when B = 1 and the call's grid
 * (H * d/32 workgroups) would not fill the device twice over, each head's
 * sequence runs as S segments at once (each at least 8192 tokens, at most 64;
 * none below 2), the first from the caller's state and the others from zero,
 * then the segments' states are chained and each later segment's outputs are
 * corrected with the state at its start (o_a += lambda^(a+1) q_a S for its
 * local token index a, fp32 throughout) - the decomposition of la_prefill_ws
 * (the report's §4.1.1 and Fig. 10, local output and local state per piece
 * joined through the carried state) for fp32 q, k, v, out.  Same semantics and
 * argument rules as la_prefill_f32; results equal la_prefill_f32's within fp32
 * rounding.  Tokens whose factor lambda^(a+1) is exactly 0 in fp32 get no
 * correction work.
 *   la_prefill_f32_workspace_bytes: the workspace bytes la_prefill_f32_ws
 *     needs for these sizes on the calling thread's current device, written
 *     to *bytes; 0 means no split (la_prefill_f32_ws then runs exactly as
 *     la_prefill_f32 and ignores the workspace).  LA_ERR_INVALID_ARG for a
 *     null bytes, B or H below 1 or N below 0; LA_ERR_UNSUPPORTED for d other
 *     than 64 or 128.  Enqueues nothing.
 *   la_prefill_f32_ws: workspace rules as la_prefill_ws (device memory of at
 *     least that many bytes, 256-byte aligned, owned by the caller, not
 *     overlapping any argument, contents unspecified on entry and exit; calls
 *     sharing a workspace ordered on one stream).
 */
int la_prefill_f32_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t *bytes);
int la_prefill_f32_ws(const float *q, const float *k, const float *v, const float *slopes,
                      float *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                      void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Packed variable-length prefill: nseq independent sequences of different
 * lengths in one launch, each with its own state (the state is reset between
 * sequences, unlike a dense run over the concatenated tokens).
 *   q, k, v     [H,T,d] bf16, read only: the dense layout with B = 1 and
 *               N = T; sequence i occupies rows cu_seqlens[i] ..
 *               cu_seqlens[i+1]-1 of every head.
 *   cu_seqlens  [nseq+1] int64, DEVICE pointer, 8-byte aligned: 0 =
 *               cu[0] <= cu[1] <= ... <= cu[nseq] = T.  Empty sequences are
 *               allowed (their state is left unchanged).  The contents are
 *               not checked on the host; out-of-order or out-of-range offsets
 *               are clamped into [0, T] on the device, so they never address
 *               memory outside the tensors, but the results are then
 *               unspecified.
 *   slopes      [H] fp32, shared by all sequences.
 *   out         [H,T,d] bf16, written (rows outside every sequence untouched).
 *   states      [nseq,H,d,d] fp32, IN/OUT: initial state of each sequence on
 *               entry (zero-fill for fresh sequences), its final state on exit.
 * Results for sequence i equal la_prefill on that sequence alone (B = 1,
 * N = cu[i+1]-cu[i]), bitwise.  T == 0 is a no-op.  Source: the report's
 * §4.1.2 (packed training samples made of many short sub-sequences, each
 * attending only within itself) on top of the §4.1.1 blockwise recurrence.
 */
int la_prefill_varlen(const void *q, const void *k, const void *v, const float *slopes,
                      const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                      int64_t H, int64_t T, int64_t d, void *stream);

/* Packed variable-length prefill with fp32 q, k, v, out: same semantics. */
int la_prefill_varlen_f32(const float *q, const float *k, const float *v, const float *slopes,
                          const int64_t *cu_seqlens, int64_t nseq, float *out, float *states,
                          int64_t H, int64_t T, int64_t d, void *stream);

/*
 * Work split of a packed bf16 prefill (la_prefill_varlen, la_prefill_varlen_strided)
 * with these sizes on the calling thread's current device, written to *walks:
 *   1  one workgroup per (head, 32 output columns) walks the sequences in
 *      order (its pipeline runs across sequence boundaries, and every
 *      workgroup does the same work: all tokens of its head); batches of more
 *      than 1024 sequences are walked 1024 at a time, one kernel launch each;
 *   0  one workgroup per (sequence, head, 32 output columns).
 * The walk is used when nseq >= 2, T < 2^31, the sequences are short on
 * average (T / nseq < 8192: longer ones gain more from the hardware balancing
 * a grid of per-sequence workgroups over the compute units) and a cost
 * estimate from the sizes and the device's compute-unit count favours it: a
 * boundary costs the walk about 1.9 block steps and a per-sequence workgroup
 * about 4.25, while the walk's H*d/32 workgroups may leave compute units idle
 * (on a 256-unit MI355X: always at 64 heads and d = 128, at 32 heads only for
 * sequences of about two blocks or less, never at 16).  Both give the same
 * results, bitwise.  No GPU work is enqueued.  Returns LA_OK; LA_ERR_INVALID_ARG for a
 * null walks, nseq or H below 1 or T below 0; LA_ERR_UNSUPPORTED for d other
 * than 64 or 128.  Source: as la_prefill_varlen (many short sequences packed
 * into one launch, §4.1.2).
 */
int la_prefill_varlen_plan(int64_t nseq, int64_t H, int64_t T, int64_t d, int *walks);

/*
 * Strided prefill: la_prefill / la_prefill_varlen reading q, k, v and writing
 * out through element strides, so the kernel can read straight out of a packed
 * projection buffer ([B,N,(q|k|v|...)*H*d], token-major) and write its output
 * token-major for the next op, with no layout copies in between.  Same
 * arithmetic and results, bitwise, as the contiguous calls.
 *   Row (b, h, t) of q, k, v starts at element
 *     b*in_bstride + h*in_hstride + t*in_tstride        (la_prefill_strided)
 *     h*in_hstride + t*in_tstride, t in [0, T)          (la_prefill_varlen_strided)
 *   from their own base pointers (the three share the strides), and holds d
 *   contiguous bf16 channels; out uses the out_* strides the same way.  The
 *   contiguous calls are the strides (H*N*d, N*d, d) and (T*d, d).
 *   Strides are in elements, >= 0 and multiples of 8 (16-byte rows); token
 *   strides are at least d (a slice's rows never overlap), and above 2^24
 *   give LA_ERR_UNSUPPORTED.  Rows of different heads or sequences of the
 *   inputs may overlap (they are only read); no two output rows may share an
 *   element, and out's span
 *   (base to last element) must not overlap the spans of q, k, v or the state.
 *   State, slopes, cu_seqlens and every other rule: as la_prefill /
 *   la_prefill_varlen.  Source: as la_prefill and la_prefill_varlen (Fig. 2 puts
 *   the kernel between the QKV projection with its QK Norm and RoPE, and the
 *   grouped RMSNorm, which both work in the projection's token-major layout).
 */
int la_prefill_strided(const void *q, const void *k, const void *v, const float *slopes,
                       void *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                       int64_t in_bstride, int64_t in_hstride, int64_t in_tstride,
                       int64_t out_bstride, int64_t out_hstride, int64_t out_tstride,
                       void *stream);

/*
 * la_prefill_strided with the sequence split of la_prefill_ws (same plan,
 * same workspace rules and la_prefill_workspace_bytes; without a split it
 * runs exactly as la_prefill_strided).  Same results as la_prefill_ws on
 * contiguous copies of the same values, bitwise.  Source: as la_prefill_ws
 * and la_prefill_strided.
 */
int la_prefill_strided_ws(const void *q, const void *k, const void *v, const float *slopes,
                          void *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                          int64_t in_bstride, int64_t in_hstride, int64_t in_tstride,
                          int64_t out_bstride, int64_t out_hstride, int64_t out_tstride,
                          void *workspace, int64_t workspace_bytes, void *stream);

/*
 * la_prefill_qk_norm_rope_ws: the layer's attention step straight from the
 * projection's raw q and k.  QK Norm and RoPE (exactly as la_qk_norm_rope
 * defines them: RMSNorm over d with q_norm_weight / k_norm_weight, then
 * rotate-half RoPE on the first rot_dim channels at position pos0 + t) are
 * applied inside the attention kernels as each q and k block is loaded, and
 * the decayed linear attention of la_prefill_strided_ws runs on the result;
 * normalised q and k are never written to memory.  The same as
 * la_qk_norm_rope (in place) followed by la_prefill_strided_ws, up to
 * rounding (here each normalised value is rounded to bf16 once, inside the
 * kernel, where the two-call path stores it as bf16).
 * Source: Ling and Ring 2.6 Technical Report, Fig. 2 (QKV projection -> QK
 * Norm -> RoPE -> linear attention) and §4.3 (QK Norm + RoPE fused into one
 * kernel; here into the attention kernel itself), §2.1.1 (epsilon 1e-6, base
 * 6e6, rotary dims 64 of 128).
 *   q, k, v, slopes, out, state, the strides, workspace: as la_prefill_strided_ws
 *                (the same split plan and la_prefill_workspace_bytes).
 *   q_norm_weight, k_norm_weight  [d] fp32, 16-byte aligned.
 *   theta, rot_dim, pos0: as la_qk_norm_rope; every batch row starts at pos0.
 *   eps        a normal positive float (at least FLT_MIN; zero or subnormal
 *              gives LA_ERR_INVALID_ARG): rows past the end of a block are
 *              loaded as zeros and must normalise to zeros.
 *   d          128 only (other head dims give LA_ERR_UNSUPPORTED);
 *              rot_dim in {0, 16, 32, 64, 128}.
 */
int la_prefill_qk_norm_rope_ws(const void *q, const void *k, const void *v, const float *slopes,
                               const float *q_norm_weight, const float *k_norm_weight,
                               double theta, int64_t rot_dim, int64_t pos0, float eps, void *out,
                               float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                               int64_t in_bstride, int64_t in_hstride, int64_t in_tstride,
                               int64_t out_bstride, int64_t out_hstride, int64_t out_tstride,
                               void *workspace, int64_t workspace_bytes, void *stream);

int la_prefill_varlen_strided(const void *q, const void *k, const void *v, const float *slopes,
                              const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                              int64_t H, int64_t T, int64_t d, int64_t in_hstride,
                              int64_t in_tstride, int64_t out_hstride, int64_t out_tstride,
                              void *stream);

/*
 * la_prefill_varlen_from_zero: la_prefill_varlen_strided for sequences that
 * all start from a zero state (fresh requests), with the states an output
 * only: states [nseq,H,d,d] fp32 is written (the final state of each
 * sequence; zeros for an empty one) and never read, which saves a state read
 * per sequence and head (at 64 tokens per sequence and d = 128 the states are
 * half of the launch's bytes).  The same results as la_prefill_varlen_strided
 * on zero-filled states, bitwise; T = 0 writes zero states.  states may be
 * NULL: no state is written (outputs only, for a forward pass whose final
 * states are not needed, such as a training or scoring pass over packed
 * sequences); the outputs are the same, bitwise.  Every other rule
 * (strides, offsets, sizes, errors): as la_prefill_varlen_strided; the
 * contiguous layout is the strides (T*d, d, T*d, d).  Source: as
 * la_prefill_varlen (Ling and Ring 2.6 Technical Report, §4.1.2: packed
 * variable-length sequences); a zero state is the recurrence's state before
 * any token.
 */
int la_prefill_varlen_from_zero(const void *q, const void *k, const void *v, const float *slopes,
                                const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                                int64_t H, int64_t T, int64_t d, int64_t in_hstride,
                                int64_t in_tstride, int64_t out_hstride, int64_t out_tstride,
                                void *stream);

/*
 * One decode step for B*H sequences (one new token each).
 *   q, k, v     [B,H,d] bf16, read only.
 *   state       [B,H,d,d] fp32, updated in place: S' = lambda S + k^T v.
 *   out         [B,H,d] bf16, written: o = q . S'.
 * The state update happens before the read-out, so the new token attends to
 * itself, exactly as in prefill; N decode steps equal one prefill of N tokens
 * up to rounding.  Source: the report's §4.1.1 recurrence; the serving-side
 * attention step over a carried state (§4.3, Fig. 12).
 */
int la_decode_step(const void *q, const void *k, const void *v, const float *slopes,
                   float *state, void *out,
                   int64_t B, int64_t H, int64_t d, void *stream);

/* Decode step with fp32 q, k, v, out: same semantics. */
int la_decode_step_f32(const float *q, const float *k, const float *v, const float *slopes,
                       float *state, float *out,
                       int64_t B, int64_t H, int64_t d, void *stream);

/*
 * Multi-token decode (draft verification): T tokens per sequence, 1 <= T <= 8,
 * applied in order from the carried state.
 *   q, k, v     [B,H,T,d] bf16, read only (token t of sequence b, head h).
 *   n_commit    [B] int32, DEVICE pointer, or NULL (= T for every sequence):
 *               how many leading tokens of sequence b are folded into the
 *               stored state.  Values outside [0, T] are clamped.
 *   state       [B,H,d,d] fp32, IN/OUT: on exit the state after n_commit[b]
 *               tokens (unchanged for 0).
 *   out         [B,H,T,d] bf16, written for every token:
 *               o_t = q_t S_t,  S_t = lambda S_{t-1} + k_t^T v_t,
 *               S_{-1} = the state on entry (whatever n_commit says).
 * With n_commit = T this equals T calls of la_decode_step (and a prefill of
 * the T tokens) up to rounding.  T > 8 gives LA_ERR_UNSUPPORTED, T < 1
 * LA_ERR_INVALID_ARG.  Source: serving with multi-token prediction (the
 * report's §4.3, Table 7 and Fig. 12) and its Appendix B (four speculative
 * steps, acceptance lengths of about 2.7 to 3.3 in Table 8): several draft
 * tokens are scored against one carried state and only the accepted prefix
 * may advance it.
 */
int la_decode_multi(const void *q, const void *k, const void *v, const float *slopes,
                    const int32_t *n_commit, float *state, void *out,
                    int64_t B, int64_t H, int64_t T, int64_t d, void *stream);

/* Multi-token decode with fp32 q, k, v, out: same semantics. */
int la_decode_multi_f32(const float *q, const float *k, const float *v, const float *slopes,
                        const int32_t *n_commit, float *state, float *out,
                        int64_t B, int64_t H, int64_t T, int64_t d, void *stream);

/*
 * Strided decode (bf16): la_decode_step / la_decode_multi reading q, k, v
 * through element strides, e.g. straight out of a token-major projection
 * buffer of the new token(s), with no layout copy (the serving counterpart of
 * la_prefill_strided).  Row (b, h) of q, k, v starts at element
 * b*in_bstride + h*in_hstride (+ t*in_tstride for token t of la_decode_multi)
 * from each base pointer and holds d contiguous bf16 channels; strides >= 0,
 * inputs 2-byte aligned, their rows may overlap (they are only read).  out
 * stays [B,H,d] / [B,H,T,d] contiguous, 2-byte aligned, and must not overlap
 * the inputs' spans or the state.  Same arithmetic and results, bitwise, as
 * the contiguous calls; every other rule as there.  Source: as la_decode_step
 * and la_decode_multi (the report's §4.3 and Fig. 12 serve the layer of Fig. 2,
 * whose projections are token-major).
 */
int la_decode_step_strided(const void *q, const void *k, const void *v, const float *slopes,
                           float *state, void *out, int64_t B, int64_t H, int64_t d,
                           int64_t in_bstride, int64_t in_hstride, void *stream);

int la_decode_multi_strided(const void *q, const void *k, const void *v, const float *slopes,
                            const int32_t *n_commit, float *state, void *out, int64_t B,
                            int64_t H, int64_t T, int64_t d, int64_t in_bstride,
                            int64_t in_hstride, int64_t in_tstride, void *stream);

/*
 * The layer's neighbouring ops, each one fused kernel (bf16 activations, fp32
 * weights and arithmetic).  Source: the report's Fig. 2 (the linear-attention
 * layer: QKV projection -> QK Norm -> RoPE -> this library's kernel -> grouped
 * RMSNorm, times sigmoid of a gate projection -> output projection), §4.3
 * (QK Norm + RoPE and Group RMSNorm + Sigmoid Gate each fused into one
 * kernel) and §2.1.1 (RMSNorm epsilon 1e-6; RoPE base 6,000,000 with rotary
 * dimension 64, i.e. partial RoPE on part of each head).
 *
 * la_qk_norm_rope: from the projection layout to the kernel layout, or in place.
 *   q_in, k_in, v_in  bf16 rows [B,N,H,d]: element (b,t,h,i) at
 *                     (b*N + t)*in_stride + h*d + i; in_stride >= H*d and a
 *                     multiple of 8 (a packed [q|k|v|...] projection output
 *                     passes three offsets into one buffer).  v_in and
 *                     v_out may both be NULL: v is then not touched.
 *   q_norm_weight, k_norm_weight  [d] fp32, 16-byte aligned.
 *   For q and k: x <- x / sqrt(mean_i x_i^2 + eps) * weight (RMSNorm over the
 *   head dimension), then rotate-half RoPE on the first rot_dim dims at
 *   position p = pos0 + t: for j < rot_dim/2, with a = p * theta^(-2j/rot_dim),
 *     x'_j = x_j cos a - x_{j+rot/2} sin a,   x'_{j+rot/2} = x_{j+rot/2} cos a + x_j sin a;
 *   dims >= rot_dim pass through.  v is only moved.
 *   q_out, k_out, v_out  bf16 [B,H,N,d] (the layout la_prefill reads).  Or
 *                     in place: q_out == q_in and k_out == k_in write q and
 *                     k back over their inputs in the projection layout (for
 *                     la_prefill_strided); q, k and v rows must then share no
 *                     element (one packed buffer with disjoint column ranges
 *                     is fine), and v_out, if given, lies outside all of them.
 *   rot_dim in {0, 16, 32, 64, 128} (<= d), theta > 1 when rot_dim > 0,
 *   pos0 >= 0, eps >= 0.  Other rot_dim values give LA_ERR_UNSUPPORTED.
 *   Out of place, outputs must not overlap the inputs or each other; only
 *   one of q and k in place is LA_ERR_INVALID_ARG.  B*N == 0 is a no-op.
 */
int la_qk_norm_rope(const void *q_in, const void *k_in, const void *v_in, int64_t in_stride,
                    const float *q_norm_weight, const float *k_norm_weight, double theta,
                    int64_t rot_dim, int64_t pos0, float eps, void *q_out, void *k_out,
                    void *v_out, int64_t B, int64_t N, int64_t H, int64_t d, void *stream);

/*
 * la_group_norm_gate: from the kernel's output back to the projection layout.
 *   o            bf16 rows of d channels, row (b, h, t) at element
 *                b*o_bstride + h*o_hstride + t*o_tstride (strides >= 0 and
 *                multiples of 8): (H*N*d, N*d, d) for la_prefill's output,
 *                (N*H*d, d, H*d) for a token-major one (la_prefill_strided).
 *   gate         bf16 rows [B,N,H*d] at token stride gate_stride (>= H*d, a
 *                multiple of 8).
 *   norm_weight  [H*d] fp32, 16-byte aligned.
 *   y[b,t,c] = o_c / sqrt(mean over c's group of o^2 + eps) * norm_weight[c]
 *              * sigmoid(gate[b,t,c]),  c = h*d + i, groups of `group`
 *              consecutive channels inside one head.
 *   y            bf16 [B,N,H*d], contiguous; must not overlap o or gate.
 *   group is a power of two in [8, d] (else LA_ERR_UNSUPPORTED); the pages do
 *   not give the group size (a head, group = d, is the plain reading).
 *   eps >= 0.  B*N == 0 is a no-op.
 */
int la_group_norm_gate(const void *o, int64_t o_bstride, int64_t o_hstride, int64_t o_tstride,
                       const void *gate, int64_t gate_stride, const float *norm_weight,
                       int64_t group, float eps, void *y, int64_t B, int64_t N, int64_t H,
                       int64_t d, void *stream);

/*
 * Sequence-sharded (context-parallel) prefill: the two steps a rank adds after
 * running la_prefill over its own shard of a long sequence from a zero state.
 * Source: the report's §4.1.1 and Fig. 10 - every rank computes a local state
 * and a local output, the [B,H,D,D] local states are all-gathered, each rank
 * folds the states of the shards before it into its incoming state and
 * corrects its local output with it.  The gather itself is the caller's (one
 * all-gather of the local states); these calls do the arithmetic around it.
 *
 * la_cp_fold: the state entering shard `rank`.
 *   local_states  [nshards,B,H,d,d] fp32, read only: shard j's state after its
 *                 own tokens from a zero state (la_prefill's final state), in
 *                 shard order; only the first `rank` are read (may be NULL
 *                 for rank 0).
 *   shard_lens    HOST pointer to nshards int64 token counts (>= 0; only the
 *                 first `rank` are read; may be NULL for rank 0).
 *   nshards       1..64 (more gives LA_ERR_UNSUPPORTED); rank in 0..nshards
 *                 (nshards gives the state after the whole sequence).
 *   state_init    [B,H,d,d] fp32, the state before the sequence, or NULL (zero).
 *   state_in      [B,H,d,d] fp32, written:
 *     S_in(0) = S_init,  S_in(j+1) = lambda^shard_lens[j] S_in(j) + local_states[j],
 *   in that order, fp32.  state_in may be state_init itself (in place); it
 *   must not overlap local_states or partly overlap state_init.
 *
 * la_cp_correct: a shard's output from its local output and incoming state.
 *   q          [B,H,L,d] bf16, read only: the shard's queries.
 *   state_in   [B,H,d,d] fp32 (la_cp_fold's result for this shard).
 *   out        [B,H,L,d] bf16, IN/OUT: the local output (la_prefill from a zero
 *              state) on entry; on exit out_a + lambda^(a+1) q_a . S_in for local
 *              token a, with S_in rounded to bf16 for the product (as the
 *              prefill's inter-block term uses it), fp32 accumulation, one bf16
 *              rounding.  Must not overlap q or state_in.
 *   L == 0 is a no-op; L > 2^31 - 256 gives LA_ERR_UNSUPPORTED.
 * Together: shard r's corrected output and la_cp_fold(rank = nshards) equal one
 * la_prefill over the whole sequence up to rounding.
 */
int la_cp_fold(const float *local_states, const int64_t *shard_lens, int64_t nshards,
               int64_t rank, const float *slopes, const float *state_init, float *state_in,
               int64_t B, int64_t H, int64_t d, void *stream);

int la_cp_correct(const void *q, const float *slopes, const float *state_in, void *out,
                  int64_t B, int64_t H, int64_t L, int64_t d, void *stream);

/* Static, NUL-terminated description of a status code ("unknown status" for
 * values outside la_status).  Never NULL; the caller must not free it. */
const char *la_status_string(int status);

/* ABI version of this header (incremented on incompatible changes). */
int la_abi_version(void);

#define LA_ABI_VERSION 8

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_ATTN_H */
