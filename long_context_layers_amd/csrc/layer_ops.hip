// layer_ops.hip — the linear-attention layer's neighbouring element-wise ops,
// each one fused kernel (Ling and Ring 2.6 Technical Report, Fig. 2: QKV
// projection -> QK Norm -> RoPE -> linear attention kernel -> grouped RMSNorm,
// times sigmoid(gate projection) -> output projection; §4.3 fuses "QK Norm +
// RoPE" and "Group RMSNorm + Sigmoid Gate" into one kernel each; §2.1.1: RMSNorm
// epsilon 1e-6, RoPE base 6,000,000, rotary dimension 64 of the 128 head dims).
//
// qk_norm_rope: q, k rows [B,N,H,d] (projection layout, any token stride) ->
//   RMSNorm over d with a per-tensor weight -> rotate-half RoPE on the first
//   rot dims (pairs j, j + rot/2) at position pos0 + t -> rows [B,H,N,d] (the
//   attention kernel's layout), or back over the inputs in place; v rows are
//   moved to [B,H,N,d] unchanged, or left alone.
// group_norm_gate: o rows (any strides: [B,H,N,d] from the attention kernel,
//   or token-major) -> RMSNorm over groups of G channels with a [H*d] weight
//   -> times sigmoid(gate) -> rows [B,N,H*d].
//
// Both are bound by HBM: every (token, head) row of d bf16 values (256 B at
// d = 128) is read and written once, and a row is contiguous on both sides,
// so the layout change needs no LDS: 16 lanes own one row (16 bytes each),
// a wave moves four rows per instruction, and the row sums of squares are
// reduced across those 16 lanes with cross-lane shuffles.  One workgroup per
// token: the token's rotary angles are computed once per lane (fp64 angle,
// exact reduction to [-pi, pi], then fp32 sin/cos) and reused for all heads.
#include "la_internal.h"

namespace la {
namespace {

constexpr int LT = 256;                 // threads per workgroup (4 waves)

__device__ __forceinline__ void unpack8(const uint4 &x, float (&f)[8]) {
    const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
        f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// sum over the `width` lanes (a power of two <= 16) of an aligned lane group
__device__ __forceinline__ float group_sum(float x, int width) {
    for (int m = width / 2; m >= 1; m /= 2) x += __shfl_xor(x, m, 16);
    return x;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// eight consecutive fp32 weights (16-byte aligned)
__device__ __forceinline__ void ldw8(const float *p, float (&w)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}
__device__ __forceinline__ void st16(uint16_t *p, uint4 x) { *reinterpret_cast<uint4 *>(p) = x; }

// In place (inplace != 0) each q/k row is written back over itself by the 16
// lanes that read it, after they read it, so q, k and their outputs are not
// restrict-qualified.  vi/vo null: v is not touched.
template <int D>
__global__ __launch_bounds__(LT) void qk_norm_rope_kernel(
    const uint16_t *qi, const uint16_t *ki, const uint16_t *__restrict__ vi, int64_t in_stride,
    const float *__restrict__ qw, const float *__restrict__ kw,
    double theta, int rot, int64_t pos0, float eps,
    uint16_t *qo, uint16_t *ko, uint16_t *__restrict__ vo, int inplace,
    int64_t N, int64_t H)
{
    constexpr int CH = D / 8;                         // 16-byte chunks per row
    constexpr int RPP = LT / CH;                      // rows per pass
    const int64_t bt = blockIdx.x;                    // b * N + t
    const int64_t b = bt / N, t = bt % N;
    const int c = threadIdx.x % CH, r0 = threadIdx.x / CH;
    const int half = rot / 2;                         // rotary pairs (j, j + half)
    const bool rotary = 8 * c < rot;
    const int partner_mask = half / 8;                // chunk c <-> c ^ (half / 8)

    // this lane's 8 rotary angles (pair index of element 8c + e), fp64 angle
    // reduced exactly to [-pi, pi] before the fp32 sin/cos
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        cs[e] = 1.0f;
        sn[e] = 0.0f;
        if (rotary) {
            const int j = (8 * c + e) % half;
            const double freq = exp2(-2.0 * j / rot * log2(theta));
            const double a = (double)(pos0 + t) * freq;
            const double red = a - 6.283185307179586 * rint(a / 6.283185307179586);
            sincosf((float)red, &sn[e], &cs[e]);
        }
    }
    // first half of the rotary part: own*cos - partner*sin; second: own*cos + partner*sin
    const float sgn = (8 * c < half) ? -1.0f : 1.0f;
    float wq[8], wk[8];
    ldw8(qw + 8 * c, wq);
    ldw8(kw + 8 * c, wk);

    for (int64_t h = r0; h < H; h += RPP) {
        const int64_t src = bt * in_stride + h * D + 8 * c;
        const int64_t dst = inplace ? src : ((b * H + h) * N + t) * D + 8 * c;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            float x[8];
            unpack8(ld16((which ? ki : qi) + src), x);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
            ss = group_sum(ss, CH);
            const float inv = rsqrtf(ss / (float)D + eps);
            const float *w = which ? wk : wq;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] * inv * w[e];
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __shfl_xor(x[e], partner_mask, 16);   // (no-op pairs when rot == 0)
                y[e] = rotary ? fmaf(x[e], cs[e], sgn * p * sn[e]) : x[e];
            }
            st16((which ? ko : qo) + dst, pack8(y));
        }
        if (vo) st16(vo + ((b * H + h) * N + t) * D + 8 * c, ld16(vi + src));
    }
}

template <int D>
__global__ __launch_bounds__(LT) void group_norm_gate_kernel(
    const uint16_t *__restrict__ o, int64_t osb, int64_t osh, int64_t ost,
    const uint16_t *__restrict__ g, int64_t gate_stride,
    const float *__restrict__ w, int group, float eps, uint16_t *__restrict__ y,
    int64_t N, int64_t H)
{
    constexpr int CH = D / 8;
    constexpr int RPP = LT / CH;
    const int64_t bt = blockIdx.x;
    const int64_t b = bt / N, t = bt % N;
    const int c = threadIdx.x % CH, r0 = threadIdx.x / CH;
    const int lanes = group / 8;                      // lanes per normalisation group

    for (int64_t h = r0; h < H; h += RPP) {
        float x[8], gt[8];
        unpack8(ld16(o + b * osb + h * osh + t * ost + 8 * c), x);
        unpack8(ld16(g + bt * gate_stride + h * D + 8 * c), gt);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        ss = group_sum(ss, lanes);
        const float inv = rsqrtf(ss / (float)group + eps);
        float wv[8], z[8];
        ldw8(w + h * D + 8 * c, wv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sig = 1.0f / (1.0f + expf(-gt[e]));
            z[e] = x[e] * inv * wv[e] * sig;
        }
        st16(y + bt * (H * D) + h * D + 8 * c, pack8(z));
    }
}

}  // namespace

hipError_t launch_qk_norm_rope(const uint16_t *qi, const uint16_t *ki, const uint16_t *vi,
                               int64_t in_stride, const float *qw, const float *kw, double theta,
                               int rot, int64_t pos0, float eps, uint16_t *qo, uint16_t *ko,
                               uint16_t *vo, int inplace, int64_t B, int64_t N, int64_t H, int d,
                               hipStream_t stream)
{
    const dim3 grid((unsigned)(B * N)), block(LT);
    void *args[] = {(void *)&qi, (void *)&ki, (void *)&vi, (void *)&in_stride, (void *)&qw,
                    (void *)&kw, (void *)&theta, (void *)&rot, (void *)&pos0, (void *)&eps,
                    (void *)&qo, (void *)&ko, (void *)&vo, (void *)&inplace, (void *)&N,
                    (void *)&H};
    const void *fn = d == 64 ? (const void *)qk_norm_rope_kernel<64>
                             : (const void *)qk_norm_rope_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_group_norm_gate(const uint16_t *o, const int64_t os[3], const uint16_t *g,
                                  int64_t gate_stride, const float *w, int group, float eps,
                                  uint16_t *y, int64_t B, int64_t N, int64_t H, int d,
                                  hipStream_t stream)
{
    const dim3 grid((unsigned)(B * N)), block(LT);
    int64_t osb = os[0], osh = os[1], ost = os[2];
    void *args[] = {(void *)&o, (void *)&osb, (void *)&osh, (void *)&ost, (void *)&g,
                    (void *)&gate_stride, (void *)&w, (void *)&group, (void *)&eps, (void *)&y,
                    (void *)&N, (void *)&H};
    const void *fn = d == 64 ? (const void *)group_norm_gate_kernel<64>
                             : (const void *)group_norm_gate_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace la
