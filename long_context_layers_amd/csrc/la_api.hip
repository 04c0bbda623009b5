// la_api.hip — the C ABI (include/lightning_attn.h): host-side argument
// checks, then one kernel launch on the caller's stream.  No allocation, no
// synchronisation, no global state.
#include "lightning_attn.h"
#include "la_internal.h"

#include <stdint.h>

#include <cfloat>

#include <atomic>
#include <mutex>

// Scratch of the allocation-free prefill (la_prefill_noalloc): one array per
// device for the life of the process.  In host code `scratch` only stands in
// for the symbol; the device address comes from hipGetSymbolAddress, looked
// up once per device with that device current, and is what every launch gets.
// (the sequence split needs at most 32 KiB of state slots per compute unit
// plus its segment offsets: 8 MiB + 520 bytes on a 256-CU MI355X)
static constexpr int64_t NOALLOC_SCRATCH_BYTES = (int64_t(8) << 20) + 4096;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::atomic<void *> scratch_addr[NOALLOC_MAX_DEVICES];
std::mutex scratch_mu;

// this device's scratch address (LA_OK), or the failure of the lookup
int current_device_scratch(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LA_ERR_HIP;
    }
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return LA_ERR_UNSUPPORTED;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return LA_ERR_HIP;
            }
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return LA_OK;
}

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

bool pow2_in(int64_t x, int64_t lo, int64_t hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

// [rows][width] bf16 rows at `stride` elements apart, width <= stride: the
// byte span they cover (false on overflow)
bool span_ok(int64_t rows, int64_t stride, int64_t width, int64_t *bytes) {
    if (rows == 0) { *bytes = 0; return true; }
    int64_t last;
    if (!mul_ok(rows - 1, stride, &last) || last > INT64_MAX / 2 - width) return false;
    *bytes = (last + width) * 2;
    return true;
}

// A strided view of n[0] x n[1] x n[2] rows of d contiguous elements of
// `elem` bytes, row (i, j, t) at element i*s[0] + j*s[1] + t*s[2]: the byte
// span from the base to one past its last element (false on overflow or a
// negative stride; an empty view spans nothing)
bool view_span(const int64_t n[3], const int64_t s[3], int64_t d, int64_t elem, int64_t *bytes)
{
    for (int i = 0; i < 3; ++i)
        if (n[i] == 0) { *bytes = 0; return true; }
    int64_t last = 0;
    for (int i = 0; i < 3; ++i) {
        int64_t t;
        if (n[i] < 0 || s[i] < 0 || !mul_ok(n[i] - 1, s[i], &t) || last > INT64_MAX - t)
            return false;
        last += t;
    }
    if (last > INT64_MAX / elem - d) return false;
    *bytes = (last + d) * elem;
    return true;
}

// no two elements of the view (spans already checked) share an address: with
// the dimensions of more than one entry sorted by stride, each stride is at
// least the extent of everything below it
bool view_disjoint(const int64_t n[3], const int64_t s[3], int64_t d)
{
    int64_t ss[3], nn[3];
    int m = 0;
    for (int i = 0; i < 3; ++i)
        if (n[i] > 1) { ss[m] = s[i]; nn[m] = n[i]; ++m; }
    for (int i = 1; i < m; ++i)                      // insertion sort by stride
        for (int j = i; j > 0 && ss[j] < ss[j - 1]; --j) {
            const int64_t a = ss[j], b = nn[j];
            ss[j] = ss[j - 1]; nn[j] = nn[j - 1];
            ss[j - 1] = a; nn[j - 1] = b;
        }
    int64_t ext = d;
    for (int i = 0; i < m; ++i) {
        if (ss[i] < ext) return false;
        ext += ss[i] * (nn[i] - 1);
    }
    return true;
}

// strides of the strided prefill: multiples of 8 (16-byte rows), token
// strides small enough for the kernel's 32-bit buffer offsets over a block
constexpr int64_t MAX_TOKEN_STRIDE = int64_t(1) << 24;

bool strides_ok(const int64_t s[3]) {
    for (int i = 0; i < 3; ++i)
        if (s[i] < 0 || s[i] % 8 != 0) return false;
    return true;
}

// strided bf16 prefill: q, k, v share the view (n, si), out has (n, so)
int check_strided(const void *q, const void *k, const void *v, const float *slopes,
                  const void *out, const float *state, const int64_t n[3], const int64_t si[3],
                  const int64_t so[3], int64_t nstate, int64_t d, bool state_optional = false)
{
    int64_t rows;
    if (!mul_ok(n[0], n[1], &rows) || !mul_ok(rows, n[2], &rows)) return LA_ERR_INVALID_ARG;
    if (rows > 0 && (!q || !k || !v || !out)) return LA_ERR_INVALID_ARG;
    if (!slopes || (!state && !state_optional)) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    if (!strides_ok(si) || !strides_ok(so)) return LA_ERR_INVALID_ARG;
    // token rows of one slice never overlap: the kernel's buffer ranges end at
    // a block's last real row, which zero-fills the rows past it only then
    if (si[2] < d || so[2] < d) return LA_ERR_INVALID_ARG;
    int64_t in_bytes, out_bytes, st, st_bytes;
    if (!view_span(n, si, d, 2, &in_bytes) || !view_span(n, so, d, 2, &out_bytes) ||
        !mul_ok(nstate, d * d, &st) || !mul_ok(st, 4, &st_bytes))
        return LA_ERR_INVALID_ARG;
    if (!view_disjoint(n, so, d)) return LA_ERR_INVALID_ARG;
    if (si[2] > MAX_TOKEN_STRIDE || so[2] > MAX_TOKEN_STRIDE) return LA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(state, 16) || !aligned(slopes, 4))
        return LA_ERR_INVALID_ARG;
    if (overlap(out, out_bytes, q, in_bytes) || overlap(out, out_bytes, k, in_bytes) ||
        overlap(out, out_bytes, v, in_bytes) || (state && overlap(out, out_bytes, state, st_bytes)))
        return LA_ERR_INVALID_ARG;
    return LA_OK;
}

// strided bf16 decode: q, k, v rows (b, h, t) at b*s[0] + h*s[1] + t*s[2]
// (n = {B, H, T}), out [B,H,T,d] contiguous; inputs are read element by
// element (2-byte aligned), out and the state as in the contiguous calls
int check_decode_strided(const void *q, const void *k, const void *v, const float *slopes,
                         const float *state, const void *out, const int64_t n[3],
                         const int64_t si[3], int64_t d)
{
    if (!q || !k || !v || !slopes || !out || !state) return LA_ERR_INVALID_ARG;
    if (n[0] < 1 || n[1] < 1) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    int64_t bh, act, out_bytes, st, st_bytes, in_bytes;
    if (!mul_ok(n[0], n[1], &bh) || !mul_ok(bh, n[2] * d, &act) || !mul_ok(act, 2, &out_bytes) ||
        !mul_ok(bh, d * d, &st) || !mul_ok(st, 4, &st_bytes) || !view_span(n, si, d, 2, &in_bytes))
        return LA_ERR_INVALID_ARG;
    if (!aligned(q, 2) || !aligned(k, 2) || !aligned(v, 2) || !aligned(out, 2) ||
        !aligned(state, 16) || !aligned(slopes, 4))
        return LA_ERR_INVALID_ARG;
    if (overlap(out, out_bytes, q, in_bytes) || overlap(out, out_bytes, k, in_bytes) ||
        overlap(out, out_bytes, v, in_bytes) || overlap(out, out_bytes, state, st_bytes))
        return LA_ERR_INVALID_ARG;
    if (bh > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

// dense [seqs, H, N, d] strides, and the packed [H, T, d] ones
la::Strides dense_strides(int64_t H, int64_t N, int64_t d) { return {H * N * d, N * d, d}; }
la::Strides packed_strides(int64_t T, int64_t d) { return {0, T * d, d}; }

// two [rows][width] bf16 arrays whose rows are `stride` elements apart share
// no element: their spans are apart, or b's offset from a, taken modulo the
// stride, leaves a whole row width on both sides
bool rows_disjoint(const void *a, const void *b, int64_t rows, int64_t stride, int64_t width)
{
    int64_t span;
    if (!span_ok(rows, stride, width, &span)) return false;
    if (!overlap(a, span, b, span)) return true;
    const intptr_t delta = reinterpret_cast<intptr_t>(b) - reinterpret_cast<intptr_t>(a);
    if (delta % 2 != 0) return false;
    const int64_t rem = ((int64_t)(delta / 2) % stride + stride) % stride;
    return rem >= width && rem <= stride - width;
}

int check_layer_common(int64_t B, int64_t N, int64_t H, int64_t d)
{
    if (B < 1 || N < 0 || H < 1) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    int64_t bn;
    if (!mul_ok(B, N, &bn)) return LA_ERR_INVALID_ARG;
    if (bn > 0x7fffffff) return LA_ERR_UNSUPPORTED;
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
    const la::Strides s = dense_strides(H, N, d);
    const la::SeqMap map = {nullptr, H, N, 0, s, s};
    return hip_status(la::launch_prefill_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), state, B, map,
        (int)d, static_cast<hipStream_t>(stream)));
}

int la_prefill_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t *bytes)
{
    if (!bytes || B < 1 || H < 1 || N < 0) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    int njt = 1;
    const int nseg = la::prefill_split_plan(B, H, N, (int)d, &njt);
    *bytes = la::split_workspace_bytes(H, nseg, (int)d);
    return LA_OK;
}

int la_prefill_ws(const void *q, const void *k, const void *v, const float *slopes, void *out,
                  float *state, int64_t B, int64_t H, int64_t N, int64_t d, void *workspace,
                  int64_t workspace_bytes, void *stream)
{
    const int rc = check_prefill(q, k, v, slopes, out, state, B, H, N, d, 2);
    if (rc != LA_OK) return rc;
    int njt = 1;
    const int nseg = la::prefill_split_plan(B, H, N, (int)d, &njt);
    if (nseg < 2) return la_prefill(q, k, v, slopes, out, state, B, H, N, d, stream);
    const int64_t need = la::split_workspace_bytes(H, nseg, (int)d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return LA_ERR_INVALID_ARG;
    const uint64_t act = (uint64_t)B * H * N * d * 2, st = (uint64_t)B * H * d * d * 4;
    if (overlap(workspace, need, q, act) || overlap(workspace, need, k, act) ||
        overlap(workspace, need, v, act) || overlap(workspace, need, out, act) ||
        overlap(workspace, need, state, st) || overlap(workspace, need, slopes, H * 4))
        return LA_ERR_INVALID_ARG;
    if (la::prefill_bf16_grid(nseg, H, (int)d, njt) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    const la::Strides s = dense_strides(H, N, d);
    return hip_status(la::launch_prefill_bf16_split(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), state, H, N,
        (int)d, nseg, njt, s, s, workspace, static_cast<hipStream_t>(stream)));
}

int la_prefill_noalloc(const void *q, const void *k, const void *v, const float *slopes,
                       void *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                       void *stream)
{
    const int rc = check_prefill(q, k, v, slopes, out, state, B, H, N, d, 2);
    if (rc != LA_OK) return rc;
    int njt = 1;
    const int nseg = la::prefill_split_plan(B, H, N, (int)d, &njt);
    if (nseg < 2) return la_prefill(q, k, v, slopes, out, state, B, H, N, d, stream);
    if (la::split_workspace_bytes(H, nseg, (int)d) > NOALLOC_SCRATCH_BYTES) return LA_ERR_UNSUPPORTED;
    void *ws = nullptr;
    const int rs = current_device_scratch(&ws);
    if (rs != LA_OK) return rs;
    return la_prefill_ws(q, k, v, slopes, out, state, B, H, N, d, ws, NOALLOC_SCRATCH_BYTES, stream);
}

int la_prefill_varlen(const void *q, const void *k, const void *v, const float *slopes,
                      const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                      int64_t H, int64_t T, int64_t d, void *stream)
{
    const int rc = check_varlen(q, k, v, slopes, cu_seqlens, nseq, out, states, H, T, d, 2);
    if (rc != LA_OK) return rc;
    if (la::prefill_bf16_grid(nseq, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (T == 0) return LA_OK;
    const la::Strides s = packed_strides(T, d);
    const la::SeqMap map = {cu_seqlens, H, 0, T, s, s};
    return hip_status(la::launch_prefill_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), states, nseq,
        map, (int)d, static_cast<hipStream_t>(stream)));
}

int la_prefill_varlen_plan(int64_t nseq, int64_t H, int64_t T, int64_t d, int *walks)
{
    if (!walks || nseq < 1 || H < 1 || T < 0) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    *walks = la::prefill_bf16_walks(nseq, H, T, (int)d, true) ? 1 : 0;
    return LA_OK;
}

int la_prefill_f32(const float *q, const float *k, const float *v, const float *slopes,
                   float *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                   void *stream)
{
    const int rc = check_prefill(q, k, v, slopes, out, state, B, H, N, d, 4);
    if (rc != LA_OK) return rc;
    if (la::prefill_f32_grid(B, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (N == 0) return LA_OK;
    const la::Strides s = dense_strides(H, N, d);
    const la::SeqMap map = {nullptr, H, N, 0, s, s};
    return hip_status(la::launch_prefill_f32(q, k, v, slopes, out, state, B, map, (int)d,
                                             static_cast<hipStream_t>(stream)));
}

int la_prefill_f32_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t *bytes)
{
    if (!bytes || B < 1 || H < 1 || N < 0) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    *bytes = la::split_workspace_bytes(H, la::prefill_f32_split_plan(B, H, N, (int)d), (int)d);
    return LA_OK;
}

int la_prefill_f32_ws(const float *q, const float *k, const float *v, const float *slopes,
                      float *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                      void *workspace, int64_t workspace_bytes, void *stream)
{
    const int rc = check_prefill(q, k, v, slopes, out, state, B, H, N, d, 4);
    if (rc != LA_OK) return rc;
    const int nseg = la::prefill_f32_split_plan(B, H, N, (int)d);
    if (nseg < 2) return la_prefill_f32(q, k, v, slopes, out, state, B, H, N, d, stream);
    const int64_t need = la::split_workspace_bytes(H, nseg, (int)d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return LA_ERR_INVALID_ARG;
    const uint64_t act = (uint64_t)B * H * N * d * 4, st = (uint64_t)B * H * d * d * 4;
    if (overlap(workspace, need, q, act) || overlap(workspace, need, k, act) ||
        overlap(workspace, need, v, act) || overlap(workspace, need, out, act) ||
        overlap(workspace, need, state, st) || overlap(workspace, need, slopes, H * 4))
        return LA_ERR_INVALID_ARG;
    // the segments' grid, and the correction's (at most 64 workgroups per later
    // segment and head)
    if (la::prefill_f32_grid(nseg, H, (int)d) > 0x7fffffff ||
        (int64_t)(nseg - 1) * H * 64 > 0x7fffffff)
        return LA_ERR_UNSUPPORTED;
    return hip_status(la::launch_prefill_f32_split(q, k, v, slopes, out, state, H, N, (int)d, nseg,
                                                   workspace, static_cast<hipStream_t>(stream)));
}

int la_prefill_varlen_f32(const float *q, const float *k, const float *v, const float *slopes,
                          const int64_t *cu_seqlens, int64_t nseq, float *out, float *states,
                          int64_t H, int64_t T, int64_t d, void *stream)
{
    const int rc = check_varlen(q, k, v, slopes, cu_seqlens, nseq, out, states, H, T, d, 4);
    if (rc != LA_OK) return rc;
    if (la::prefill_f32_grid(nseq, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (T == 0) return LA_OK;
    const la::Strides s = packed_strides(T, d);
    const la::SeqMap map = {cu_seqlens, H, 0, T, s, s};
    return hip_status(la::launch_prefill_f32(q, k, v, slopes, out, states, nseq, map, (int)d,
                                             static_cast<hipStream_t>(stream)));
}

int la_prefill_strided(const void *q, const void *k, const void *v, const float *slopes,
                       void *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                       int64_t in_bstride, int64_t in_hstride, int64_t in_tstride,
                       int64_t out_bstride, int64_t out_hstride, int64_t out_tstride,
                       void *stream)
{
    if (B < 1 || H < 1 || N < 0) return LA_ERR_INVALID_ARG;
    int64_t bh;
    if (!mul_ok(B, H, &bh)) return LA_ERR_INVALID_ARG;
    const int64_t n[3] = {B, H, N};
    const int64_t si[3] = {in_bstride, in_hstride, in_tstride};
    const int64_t so[3] = {out_bstride, out_hstride, out_tstride};
    const int rc = check_strided(q, k, v, slopes, out, state, n, si, so, bh, d);
    if (rc != LA_OK) return rc;
    if (la::prefill_bf16_grid(B, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (N == 0) return LA_OK;
    const la::SeqMap map = {nullptr, H, N, 0, {in_bstride, in_hstride, in_tstride},
                            {out_bstride, out_hstride, out_tstride}};
    return hip_status(la::launch_prefill_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), state, B, map,
        (int)d, static_cast<hipStream_t>(stream)));
}

namespace {

// la_prefill_strided_ws, and with pro the same launches with the fused QK Norm + RoPE
int prefill_strided_ws(const void *q, const void *k, const void *v, const float *slopes, void *out,
                       float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                       const int64_t si[3], const int64_t so[3], void *workspace,
                       int64_t workspace_bytes, void *stream, const la::QkPrologue *pro)
{
    if (B < 1 || H < 1 || N < 0) return LA_ERR_INVALID_ARG;
    int64_t bh;
    if (!mul_ok(B, H, &bh)) return LA_ERR_INVALID_ARG;
    const int64_t n[3] = {B, H, N};
    const int rc = check_strided(q, k, v, slopes, out, state, n, si, so, bh, d);
    if (rc != LA_OK) return rc;
    int njt = 1;
    const int nseg = la::prefill_split_plan(B, H, N, (int)d, &njt);
    if (nseg < 2) {
        if (la::prefill_bf16_grid(B, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
        if (N == 0) return LA_OK;
        const la::SeqMap map = {nullptr, H, N, 0, {si[0], si[1], si[2]}, {so[0], so[1], so[2]}};
        const uint16_t *q16 = static_cast<const uint16_t *>(q), *k16 = static_cast<const uint16_t *>(k),
                       *v16 = static_cast<const uint16_t *>(v);
        uint16_t *o16 = static_cast<uint16_t *>(out);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        return hip_status(pro ? la::launch_prefill_bf16_nowalk(q16, k16, v16, slopes, o16, state, B,
                                                               map, (int)d, st,
                                                               la::prefill_bf16_grid_njt(B, H, (int)d), pro)
                              : la::launch_prefill_bf16(q16, k16, v16, slopes, o16, state, B, map,
                                                        (int)d, st));
    }
    const int64_t need = la::split_workspace_bytes(H, nseg, (int)d);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return LA_ERR_INVALID_ARG;
    int64_t in_bytes = 0, out_bytes = 0;
    (void)view_span(n, si, d, 2, &in_bytes);          // checked above
    (void)view_span(n, so, d, 2, &out_bytes);
    const uint64_t st = (uint64_t)bh * d * d * 4;
    if (overlap(workspace, need, q, in_bytes) || overlap(workspace, need, k, in_bytes) ||
        overlap(workspace, need, v, in_bytes) || overlap(workspace, need, out, out_bytes) ||
        overlap(workspace, need, state, st) || overlap(workspace, need, slopes, H * 4))
        return LA_ERR_INVALID_ARG;
    if (pro && (overlap(workspace, need, pro->qw, d * 4) || overlap(workspace, need, pro->kw, d * 4)))
        return LA_ERR_INVALID_ARG;
    if (la::prefill_bf16_grid(nseg, H, (int)d, njt) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    const la::Strides in = {0, si[1], si[2]}, os = {0, so[1], so[2]};
    return hip_status(la::launch_prefill_bf16_split(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), state, H, N,
        (int)d, nseg, njt, in, os, workspace, static_cast<hipStream_t>(stream), pro));
}

}  // namespace

int la_prefill_strided_ws(const void *q, const void *k, const void *v, const float *slopes,
                          void *out, float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                          int64_t in_bstride, int64_t in_hstride, int64_t in_tstride,
                          int64_t out_bstride, int64_t out_hstride, int64_t out_tstride,
                          void *workspace, int64_t workspace_bytes, void *stream)
{
    const int64_t si[3] = {in_bstride, in_hstride, in_tstride};
    const int64_t so[3] = {out_bstride, out_hstride, out_tstride};
    return prefill_strided_ws(q, k, v, slopes, out, state, B, H, N, d, si, so, workspace,
                              workspace_bytes, stream, nullptr);
}

int la_prefill_qk_norm_rope_ws(const void *q, const void *k, const void *v, const float *slopes,
                               const float *q_norm_weight, const float *k_norm_weight,
                               double theta, int64_t rot_dim, int64_t pos0, float eps, void *out,
                               float *state, int64_t B, int64_t H, int64_t N, int64_t d,
                               int64_t in_bstride, int64_t in_hstride, int64_t in_tstride,
                               int64_t out_bstride, int64_t out_hstride, int64_t out_tstride,
                               void *workspace, int64_t workspace_bytes, void *stream)
{
    if (d != 128) return LA_ERR_UNSUPPORTED;
    if (!q_norm_weight || !k_norm_weight || !aligned(q_norm_weight, 16) ||
        !aligned(k_norm_weight, 16))
        return LA_ERR_INVALID_ARG;
    if (rot_dim != 0 && !pow2_in(rot_dim, 16, d)) return LA_ERR_UNSUPPORTED;
    if (rot_dim != 0 && !(theta > 1.0)) return LA_ERR_INVALID_ARG;      // also rejects NaN
    if (N < 0 || pos0 < 0 || pos0 > INT64_MAX - N) return LA_ERR_INVALID_ARG;
    // rows past a block's end load as zeros and must normalise to zeros
    if (!(eps >= FLT_MIN) || !(eps <= FLT_MAX)) return LA_ERR_INVALID_ARG;
    const la::QkPrologue pro = {q_norm_weight, k_norm_weight, theta, (int)rot_dim, eps, pos0};
    const int64_t si[3] = {in_bstride, in_hstride, in_tstride};
    const int64_t so[3] = {out_bstride, out_hstride, out_tstride};
    return prefill_strided_ws(q, k, v, slopes, out, state, B, H, N, d, si, so, workspace,
                              workspace_bytes, stream, &pro);
}

namespace {

// la_prefill_varlen_strided, and with zero_init the same launches from zero
// states that are only written
int prefill_varlen_strided(const void *q, const void *k, const void *v, const float *slopes,
                           const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                           int64_t H, int64_t T, int64_t d, int64_t in_hstride, int64_t in_tstride,
                           int64_t out_hstride, int64_t out_tstride, void *stream, int zero_init)
{
    if (!cu_seqlens || !aligned(cu_seqlens, 8)) return LA_ERR_INVALID_ARG;
    if (nseq < 1 || H < 1 || T < 0) return LA_ERR_INVALID_ARG;
    int64_t nstate;
    if (!mul_ok(nseq, H, &nstate)) return LA_ERR_INVALID_ARG;
    const int64_t n[3] = {1, H, T};
    const int64_t si[3] = {0, in_hstride, in_tstride};
    const int64_t so[3] = {0, out_hstride, out_tstride};
    // from zero the states are an output only, and may be null (nothing written)
    const int rc = check_strided(q, k, v, slopes, out, states, n, si, so, nstate, d, zero_init != 0);
    if (rc != LA_OK) return rc;
    if (la::prefill_bf16_grid(nseq, H, (int)d) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (T == 0 && (!zero_init || !states)) return LA_OK;   // (from zero, empty sequences' states are written)
    la::SeqMap map = {cu_seqlens, H, 0, T, {0, in_hstride, in_tstride}, {0, out_hstride, out_tstride}};
    map.zero_init = zero_init;
    return hip_status(la::launch_prefill_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, static_cast<uint16_t *>(out), states, nseq,
        map, (int)d, static_cast<hipStream_t>(stream)));
}

}  // namespace

int la_prefill_varlen_strided(const void *q, const void *k, const void *v, const float *slopes,
                              const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                              int64_t H, int64_t T, int64_t d, int64_t in_hstride,
                              int64_t in_tstride, int64_t out_hstride, int64_t out_tstride,
                              void *stream)
{
    return prefill_varlen_strided(q, k, v, slopes, cu_seqlens, nseq, out, states, H, T, d,
                                  in_hstride, in_tstride, out_hstride, out_tstride, stream, 0);
}

int la_prefill_varlen_from_zero(const void *q, const void *k, const void *v, const float *slopes,
                                const int64_t *cu_seqlens, int64_t nseq, void *out, float *states,
                                int64_t H, int64_t T, int64_t d, int64_t in_hstride,
                                int64_t in_tstride, int64_t out_hstride, int64_t out_tstride,
                                void *stream)
{
    return prefill_varlen_strided(q, k, v, slopes, cu_seqlens, nseq, out, states, H, T, d,
                                  in_hstride, in_tstride, out_hstride, out_tstride, stream, 1);
}

int la_decode_step(const void *q, const void *k, const void *v, const float *slopes,
                   float *state, void *out, int64_t B, int64_t H, int64_t d, void *stream)
{
    const int rc = check_decode(q, k, v, slopes, state, out, B, H, d, 2);
    if (rc != LA_OK) return rc;
    const la::Strides in = {H * d, d, d};
    return hip_status(la::launch_decode_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, state, static_cast<uint16_t *>(out), B, H,
        (int)d, in, static_cast<hipStream_t>(stream)));
}

int la_decode_step_strided(const void *q, const void *k, const void *v, const float *slopes,
                           float *state, void *out, int64_t B, int64_t H, int64_t d,
                           int64_t in_bstride, int64_t in_hstride, void *stream)
{
    const int64_t n[3] = {B, H, 1};
    const int64_t si[3] = {in_bstride, in_hstride, 0};
    const int rc = check_decode_strided(q, k, v, slopes, state, out, n, si, d);
    if (rc != LA_OK) return rc;
    const la::Strides in = {in_bstride, in_hstride, 0};
    return hip_status(la::launch_decode_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, state, static_cast<uint16_t *>(out), B, H,
        (int)d, in, static_cast<hipStream_t>(stream)));
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
    const la::Strides in = {H * T * d, T * d, d};
    return hip_status(la::launch_decode_multi_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, n_commit, state, static_cast<uint16_t *>(out),
        B, H, (int)T, (int)d, in, static_cast<hipStream_t>(stream)));
}

int la_decode_multi_strided(const void *q, const void *k, const void *v, const float *slopes,
                            const int32_t *n_commit, float *state, void *out, int64_t B,
                            int64_t H, int64_t T, int64_t d, int64_t in_bstride,
                            int64_t in_hstride, int64_t in_tstride, void *stream)
{
    if (T < 1) return LA_ERR_INVALID_ARG;
    if (T > la::decode_multi_max_tokens()) return LA_ERR_UNSUPPORTED;
    if (n_commit && !aligned(n_commit, 4)) return LA_ERR_INVALID_ARG;
    const int64_t n[3] = {B, H, T};
    const int64_t si[3] = {in_bstride, in_hstride, in_tstride};
    const int rc = check_decode_strided(q, k, v, slopes, state, out, n, si, d);
    if (rc != LA_OK) return rc;
    const la::Strides in = {in_bstride, in_hstride, in_tstride};
    return hip_status(la::launch_decode_multi_bf16(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), slopes, n_commit, state, static_cast<uint16_t *>(out),
        B, H, (int)T, (int)d, in, static_cast<hipStream_t>(stream)));
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

int la_qk_norm_rope(const void *q_in, const void *k_in, const void *v_in, int64_t in_stride,
                    const float *q_norm_weight, const float *k_norm_weight, double theta,
                    int64_t rot_dim, int64_t pos0, float eps, void *q_out, void *k_out,
                    void *v_out, int64_t B, int64_t N, int64_t H, int64_t d, void *stream)
{
    int rc = check_layer_common(B, N, H, d);
    if (rc != LA_OK) return rc;
    const int64_t rows = B * N;
    const bool with_v = v_in || v_out;
    if (rows > 0 && (!q_in || !k_in || !q_out || !k_out || (with_v && (!v_in || !v_out))))
        return LA_ERR_INVALID_ARG;
    if (!q_norm_weight || !k_norm_weight || !aligned(q_norm_weight, 16) ||
        !aligned(k_norm_weight, 16))
        return LA_ERR_INVALID_ARG;
    int64_t hd;
    if (!mul_ok(H, d, &hd) || in_stride < hd || in_stride % 8 != 0) return LA_ERR_INVALID_ARG;
    if (rot_dim != 0 && !pow2_in(rot_dim, 16, d)) return LA_ERR_UNSUPPORTED;
    if (rot_dim != 0 && !(theta > 1.0)) return LA_ERR_INVALID_ARG;      // also rejects NaN
    if (pos0 < 0 || pos0 > INT64_MAX - N || !(eps >= 0.0f)) return LA_ERR_INVALID_ARG;
    int64_t rh, in_bytes, out_bytes;
    if (!mul_ok(rows, H, &rh) || !span_ok(rows, in_stride, hd, &in_bytes) ||
        !span_ok(rh, d, d, &out_bytes))
        return LA_ERR_INVALID_ARG;
    // in place: q and k are written back over themselves (projection layout)
    const bool inplace = q_out == q_in && k_out == k_in;
    if (rows > 0 && !inplace && (q_out == q_in || k_out == k_in)) return LA_ERR_INVALID_ARG;
    const int nin = with_v ? 3 : 2;
    const void *ins[3] = {q_in, k_in, v_in};
    const void *outs[3] = {q_out, k_out, v_out};
    for (int i = 0; i < nin; ++i)
        if (!aligned(ins[i], 16) || !aligned(outs[i], 16)) return LA_ERR_INVALID_ARG;
    if (inplace) {
        // q, k and v rows read element-disjoint; the v copy lands outside all of them
        for (int i = 0; i < nin; ++i)
            for (int j = 0; j < i; ++j)
                if (!rows_disjoint(ins[i], ins[j], rows, in_stride, hd)) return LA_ERR_INVALID_ARG;
        if (with_v)
            for (int j = 0; j < 3; ++j)
                if (overlap(v_out, out_bytes, ins[j], in_bytes)) return LA_ERR_INVALID_ARG;
    } else {
        for (int i = 0; i < nin; ++i) {
            for (int j = 0; j < nin; ++j)
                if (overlap(outs[i], out_bytes, ins[j], in_bytes)) return LA_ERR_INVALID_ARG;
            for (int j = 0; j < i; ++j)
                if (overlap(outs[i], out_bytes, outs[j], out_bytes)) return LA_ERR_INVALID_ARG;
        }
    }
    if (rows == 0) return LA_OK;
    return hip_status(la::launch_qk_norm_rope(
        static_cast<const uint16_t *>(q_in), static_cast<const uint16_t *>(k_in),
        static_cast<const uint16_t *>(with_v ? v_in : nullptr), in_stride, q_norm_weight,
        k_norm_weight, theta, (int)rot_dim, pos0, eps, static_cast<uint16_t *>(q_out),
        static_cast<uint16_t *>(k_out), static_cast<uint16_t *>(with_v ? v_out : nullptr),
        inplace ? 1 : 0, B, N, H, (int)d, static_cast<hipStream_t>(stream)));
}

int la_group_norm_gate(const void *o, int64_t o_bstride, int64_t o_hstride, int64_t o_tstride,
                       const void *gate, int64_t gate_stride, const float *norm_weight,
                       int64_t group, float eps, void *y, int64_t B, int64_t N, int64_t H,
                       int64_t d, void *stream)
{
    int rc = check_layer_common(B, N, H, d);
    if (rc != LA_OK) return rc;
    const int64_t rows = B * N;
    if (rows > 0 && (!o || !gate || !y)) return LA_ERR_INVALID_ARG;
    if (!norm_weight || !aligned(norm_weight, 16)) return LA_ERR_INVALID_ARG;
    if (!pow2_in(group, 8, d)) return LA_ERR_UNSUPPORTED;
    int64_t hd;
    if (!mul_ok(H, d, &hd) || gate_stride < hd || gate_stride % 8 != 0) return LA_ERR_INVALID_ARG;
    if (!(eps >= 0.0f)) return LA_ERR_INVALID_ARG;
    const int64_t n[3] = {B, H, N};
    const int64_t os[3] = {o_bstride, o_hstride, o_tstride};
    int64_t o_bytes, g_bytes, y_bytes;
    if (!strides_ok(os) || !view_span(n, os, d, 2, &o_bytes) ||
        !span_ok(rows, gate_stride, hd, &g_bytes) || !span_ok(rows, hd, hd, &y_bytes))
        return LA_ERR_INVALID_ARG;
    if (!aligned(o, 16) || !aligned(gate, 16) || !aligned(y, 16)) return LA_ERR_INVALID_ARG;
    if (overlap(y, y_bytes, o, o_bytes) || overlap(y, y_bytes, gate, g_bytes))
        return LA_ERR_INVALID_ARG;
    if (rows == 0) return LA_OK;
    return hip_status(la::launch_group_norm_gate(
        static_cast<const uint16_t *>(o), os, static_cast<const uint16_t *>(gate), gate_stride,
        norm_weight, (int)group, eps, static_cast<uint16_t *>(y), B, N, H, (int)d,
        static_cast<hipStream_t>(stream)));
}

int la_cp_fold(const float *local_states, const int64_t *shard_lens, int64_t nshards,
               int64_t rank, const float *slopes, const float *state_init, float *state_in,
               int64_t B, int64_t H, int64_t d, void *stream)
{
    if (!slopes || !state_in) return LA_ERR_INVALID_ARG;
    if (B < 1 || H < 1) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    if (nshards < 1 || rank < 0 || rank > nshards) return LA_ERR_INVALID_ARG;
    if (nshards > la::MAX_CP_SHARDS) return LA_ERR_UNSUPPORTED;
    if (rank > 0 && (!local_states || !shard_lens)) return LA_ERR_INVALID_ARG;
    int lens[la::MAX_CP_SHARDS];
    for (int64_t j = 0; j < rank; ++j) {
        if (shard_lens[j] < 0) return LA_ERR_INVALID_ARG;
        if (shard_lens[j] > 0x7fffffff) return LA_ERR_UNSUPPORTED;
        lens[j] = (int)shard_lens[j];
    }
    int64_t bh, st, st_bytes, loc_bytes;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, d * d, &st) || !mul_ok(st, 4, &st_bytes) ||
        !mul_ok(st_bytes, rank, &loc_bytes))
        return LA_ERR_INVALID_ARG;
    if (!aligned(state_in, 16) || !aligned(state_init, 16) || !aligned(local_states, 16) ||
        !aligned(slopes, 4))
        return LA_ERR_INVALID_ARG;
    // state_in may be state_init itself (fold in place), but no other overlap
    if (state_init != state_in && overlap(state_in, st_bytes, state_init, st_bytes))
        return LA_ERR_INVALID_ARG;
    if (rank > 0 && overlap(state_in, st_bytes, local_states, loc_bytes))
        return LA_ERR_INVALID_ARG;
    return hip_status(la::launch_cp_fold(local_states, lens, (int)rank, state_init, state_in,
                                         slopes, B, H, (int)d, static_cast<hipStream_t>(stream)));
}

int la_cp_correct(const void *q, const float *slopes, const float *state_in, void *out,
                  int64_t B, int64_t H, int64_t L, int64_t d, void *stream)
{
    if (!slopes || !state_in) return LA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || L < 0) return LA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    if (L > 0 && (!q || !out)) return LA_ERR_INVALID_ARG;
    int64_t bh, act, act_bytes, st, st_bytes;
    if (!mul_ok(B, H, &bh) || !mul_ok(bh, L, &act) || !mul_ok(act, d * 2, &act_bytes) ||
        !mul_ok(bh, d * d, &st) || !mul_ok(st, 4, &st_bytes))
        return LA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(state_in, 16) || !aligned(slopes, 4))
        return LA_ERR_INVALID_ARG;
    if (overlap(out, act_bytes, q, act_bytes) || overlap(out, act_bytes, state_in, st_bytes))
        return LA_ERR_INVALID_ARG;
    if (L > 0x7fffff00 || la::cp_correct_grid(B, H, L) > 0x7fffffff) return LA_ERR_UNSUPPORTED;
    if (L == 0) return LA_OK;
    return hip_status(la::launch_cp_correct(
        static_cast<const uint16_t *>(q), slopes, state_in, static_cast<uint16_t *>(out), B, H,
        L, (int)d, static_cast<hipStream_t>(stream)));
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
                   "decode call than supported, a rotary dimension or norm group size the "
                   "kernels do not take, a stride, shard count or length above the "
                   "supported limit, a sequence split needing more than the "
                   "8 MiB + 4 KiB scratch of la_prefill_noalloc, or grid too large";
        case LA_ERR_HIP: return "LA_ERR_HIP: the kernel launch failed";
        default: return "unknown status";
    }
}

int la_abi_version(void) { return LA_ABI_VERSION; }

}  // extern "C"
