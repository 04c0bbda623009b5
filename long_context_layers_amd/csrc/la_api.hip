// la_api.hip — the C ABI (include/lightning_attn.h): host-side argument
// checks, then one kernel launch on the caller's stream.  No allocation, no
// synchronisation, no global state.
#include "lightning_attn.h"
#include "la_internal.h"

#include <stdint.h>

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a + na) and [b, b + nb) overlap (byte ranges)
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

// x * y without int64 overflow (both >= 0); false on overflow
bool mul_ok(int64_t x, int64_t y, int64_t *r) {
    if (x < 0 || y < 0) return false;
    if (x != 0 && y > INT64_MAX / x) return false;
    *r = x * y;
    return true;
}

// shared checks for prefill: activations hold `rows` rows of d elements of
// `elem` bytes (B*H*N dense, H*T packed), the state `nstate` d x d fp32 slices
int check_prefill_common(const void *q, const void *k, const void *v, const float *slopes,
                         const void *out, const float *state, int64_t rows, int64_t nstate,
                         int64_t d, int64_t elem)
{
    // with no rows the activations are empty and may be null (nothing is read)
    if (rows > 0 && (!q || !k || !v || !out)) return LA_ERR_INVALID_ARG;
    if (!slopes || !state) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    int64_t act, act_bytes, st, st_bytes;
    if (!mul_ok(rows, d, &act) || !mul_ok(act, elem, &act_bytes) ||
        !mul_ok(nstate, d * d, &st) || !mul_ok(st, 4, &st_bytes))
        return LA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(state, 16) || !aligned(slopes, 4))
        return LA_ERR_INVALID_ARG;
    if (overlap(out, act_bytes, q, act_bytes) || overlap(out, act_bytes, k, act_bytes) ||
        overlap(out, act_bytes, v, act_bytes) || overlap(out, act_bytes, state, st_bytes))
        return LA_ERR_INVALID_ARG;
    return LA_OK;
}

int check_prefill(const void *q, const void *k, const void *v, const float *slopes,
                  const void *out, const float *state, int64_t B, int64_t H, int64_t N,
                  int64_t d, int64_t elem)
{
    if (B < 1 || H < 1 || N < 0) return LA_ERR_INVALID_ARG;
    int64_t bh, rows;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, N, &rows)) return LA_ERR_INVALID_ARG;
    return check_prefill_common(q, k, v, slopes, out, state, rows, bh, d, elem);
}

// packed launches: also cu_seqlens (device, int64, 8-byte aligned, nseq + 1 entries)
int check_varlen(const void *q, const void *k, const void *v, const float *slopes,
                 const int64_t *cu_seqlens, int64_t nseq, const void *out, const float *state,
                 int64_t H, int64_t T, int64_t d, int64_t elem)
{
    if (!cu_seqlens || !aligned(cu_seqlens, 8)) return LA_ERR_INVALID_ARG;
    if (nseq < 1 || H < 1 || T < 0) return LA_ERR_INVALID_ARG;
    int64_t rows, nstate;
    if (!mul_ok(H, T, &rows) || !mul_ok(nseq, H, &nstate)) return LA_ERR_INVALID_ARG;
    return check_prefill_common(q, k, v, slopes, out, state, rows, nstate, d, elem);
}

int check_decode(const void *q, const void *k, const void *v, const float *slopes,
                 const float *state, const void *out, int64_t B, int64_t H, int64_t d,
                 int64_t elem)
{
    if (!q || !k || !v || !slopes || !out || !state) return LA_ERR_INVALID_ARG;
    if (B < 1 || H < 1) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    int64_t bh, act, act_bytes, st, st_bytes;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, d, &act) || !mul_ok(act, elem, &act_bytes) ||
        !mul_ok(bh, d * d, &st) || !mul_ok(st, 4, &st_bytes))
        return LA_ERR_INVALID_ARG;
    if (!aligned(q, elem) || !aligned(k, elem) || !aligned(v, elem) || !aligned(out, elem) ||
        !aligned(state, 16) || !aligned(slopes, 4))
        return LA_ERR_INVALID_ARG;
    if (overlap(out, act_bytes, q, act_bytes) || overlap(out, act_bytes, k, act_bytes) ||
        overlap(out, act_bytes, v, act_bytes) || overlap(out, act_bytes, state, st_bytes))
        return LA_ERR_INVALID_ARG;
    if (bh > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

// multi-token decode: activations [B,H,T,d], optional n_commit [B] int32
int check_decode_multi(const void *q, const void *k, const void *v, const float *slopes,
                       const int32_t *n_commit, const float *state, const void *out,
                       int64_t B, int64_t H, int64_t T, int64_t d, int64_t elem)
{
    if (!q || !k || !v || !slopes || !out || !state) return LA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || T < 1) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    if (T > la::decode_multi_max_tokens()) return LA_ERR_UNSUPPORTED;
    if (n_commit && !aligned(n_commit, 4)) return LA_ERR_INVALID_ARG;
    int64_t bh, act, act_bytes, st, st_bytes;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, T * d, &act) || !mul_ok(act, elem, &act_bytes) ||
        !mul_ok(bh, d * d, &st) || !mul_ok(st, 4, &st_bytes))
        return LA_ERR_INVALID_ARG;
    if (!aligned(q, elem) || !aligned(k, elem) || !aligned(v, elem) || !aligned(out, elem) ||
        !aligned(state, 16) || !aligned(slopes, 4))
        return LA_ERR_INVALID_ARG;
    if (overlap(out, act_bytes, q, act_bytes) || overlap(out, act_bytes, k, act_bytes) ||
        overlap(out, act_bytes, v, act_bytes) || overlap(out, act_bytes, state, st_bytes))
        return LA_ERR_INVALID_ARG;
    if (bh > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

}  // namespace

extern "C" {

int la_prefill(const void *q, const void *k, const void *v, const float *slopes, void *out,
               float *state, int64_t B, int64_t H, int64_t N, int64_t d, void *stream)
{
    const int rc = check_prefill(q, k, v, slopes, out, state, B, H, N, d, 2);
    if (rc != LA_OK) return rc;
    if (la::prefill_bf16_grid(B, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (N == 0) return LA_OK;
    const la::SeqMap map = {nullptr, H, N, 0};
    return hip_status(la::launch_prefill_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), state, B, map,
        (int)d, static_cast<hipStream_t>(stream)));
}

int la_prefill_varlen(const void *q, const void *k, const void *v, const float *slopes,
                      const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                      int64_t H, int64_t T, int64_t d, void *stream)
{
    const int rc = check_varlen(q, k, v, slopes, cu_seqlens, nseq, out, states, H, T, d, 2);
    if (rc != LA_OK) return rc;
    if (la::prefill_bf16_grid(nseq, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (T == 0) return LA_OK;
    const la::SeqMap map = {cu_seqlens, H, 0, T};
    return hip_status(la::launch_prefill_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), states, nseq,
        map, (int)d, static_cast<hipStream_t>(stream)));
}

int la_prefill_f32(const float *q, const float *k, const float *v, const float *slopes,
                   float *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                   void *stream)
{
    const int rc = check_prefill(q, k, v, slopes, out, state, B, H, N, d, 4);
    if (rc != LA_OK) return rc;
    if (la::prefill_f32_grid(B, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (N == 0) return LA_OK;
    const la::SeqMap map = {nullptr, H, N, 0};
    return hip_status(la::launch_prefill_f32(q, k, v, slopes, out, state, B, map, (int)d,
                                             static_cast<hipStream_t>(stream)));
}

int la_prefill_varlen_f32(const float *q, const float *k, const float *v, const float *slopes,
                          const int64_t *cu_seqlens, int64_t nseq, float *out, float *states,
                          int64_t H, int64_t T, int64_t d, void *stream)
{
    const int rc = check_varlen(q, k, v, slopes, cu_seqlens, nseq, out, states, H, T, d, 4);
    if (rc != LA_OK) return rc;
    if (la::prefill_f32_grid(nseq, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (T == 0) return LA_OK;
    const la::SeqMap map = {cu_seqlens, H, 0, T};
    return hip_status(la::launch_prefill_f32(q, k, v, slopes, out, states, nseq, map, (int)d,
                                             static_cast<hipStream_t>(stream)));
}

int la_decode_step(const void *q, const void *k, const void *v, const float *slopes,
                   float *state, void *out, int64_t B, int64_t H, int64_t d, void *stream)
{
    const int rc = check_decode(q, k, v, slopes, state, out, B, H, d, 2);
    if (rc != LA_OK) return rc;
    return hip_status(la::launch_decode_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, state, static_cast<uint16_t *>(out), B, H,
        (int)d, static_cast<hipStream_t>(stream)));
}

int la_decode_step_f32(const float *q, const float *k, const float *v, const float *slopes,
                       float *state, float *out, int64_t B, int64_t H, int64_t d, void *stream)
{
    const int rc = check_decode(q, k, v, slopes, state, out, B, H, d, 4);
    if (rc != LA_OK) return rc;
    return hip_status(la::launch_decode_f32(q, k, v, slopes, state, out, B, H, (int)d,
                                            static_cast<hipStream_t>(stream)));
}

int la_decode_multi(const void *q, const void *k, const void *v, const float *slopes,
                    const int32_t *n_commit, float *state, void *out, int64_t B, int64_t H,
                    int64_t T, int64_t d, void *stream)
{
    const int rc = check_decode_multi(q, k, v, slopes, n_commit, state, out, B, H, T, d, 2);
    if (rc != LA_OK) return rc;
    return hip_status(la::launch_decode_multi_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, n_commit, state, static_cast<uint16_t *>(out),
        B, H, (int)T, (int)d, static_cast<hipStream_t>(stream)));
}

int la_decode_multi_f32(const float *q, const float *k, const float *v, const float *slopes,
                        const int32_t *n_commit, float *state, float *out, int64_t B, int64_t H,
                        int64_t T, int64_t d, void *stream)
{
    const int rc = check_decode_multi(q, k, v, slopes, n_commit, state, out, B, H, T, d, 4);
    if (rc != LA_OK) return rc;
    return hip_status(la::launch_decode_multi_f32(q, k, v, slopes, n_commit, state, out, B, H,
                                                  (int)T, (int)d,
                                                  static_cast<hipStream_t>(stream)));
}

const char *la_status_string(int status)
{
    switch (status) {
        case LA_OK: return "LA_OK: success";
        case LA_ERR_INVALID_ARG:
            return "LA_ERR_INVALID_ARG: null or misaligned pointer, negative or overflowing "
                   "size, or an output overlapping an input";
        case LA_ERR_UNSUPPORTED:
            return "LA_ERR_UNSUPPORTED: head dimension not in {64, 128}, more tokens per "
                   "decode call than supported, or grid too large";
        case LA_ERR_HIP: return "LA_ERR_HIP: the kernel launch failed";
        default: return "unknown status";
    }
}

int la_abi_version(void) { return LA_ABI_VERSION; }

}  // extern "C"
