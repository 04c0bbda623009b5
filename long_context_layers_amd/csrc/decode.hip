// decode.hip — recurrent decode steps per sequence:
//   S' = lambda S + k^T v   (in place, fp32),   o = q S'
// one token per call (decode_kernel) or up to 8 (decode_multi_kernel).
// (Ling and Ring 2.6 Technical Report, §4.1.1: linear attention as an
// RNN-style recurrence over a per-(batch, head) D x D state; serving runs it
// one token per step, §4.3 / Fig. 12.)
//
// The step is bound by HBM: every state is read once and written once
// (2 x 64 KiB per (b, h) at d = 128) while the arithmetic is 4 d^2 flops.
// q, k, v are read through element strides (row (b, h[, t]) at b*sb + h*sh
// [+ t*st], channels contiguous), so they can come straight out of a
// token-major projection buffer; out is [B,H,d] ([B,H,T,d]) contiguous.
// A workgroup streams the D/NS columns js*D/NS .. of one (b, h) state (NS = 1
// for large batches; 2 or 4 when B*H workgroups would not fill the chip: an
// output column only sums over rows, so the column slices are independent):
// thread t owns the 4-column group t % CG of the slice on rows
// t / CG + (256 / CG) m.  All of a thread's rows are loaded up front (dwordx4,
// non-temporal: a state is touched once per step), updated in registers,
// written back, and the partial o = q S' sums over rows are reduced across
// the row groups in LDS (fixed order, no atomics).
#include "la_internal.h"

namespace la {
namespace {

constexpr int DT = 256;   // threads per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ float load_act(const T *p);
template <> __device__ __forceinline__ float load_act<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_act<float>(const float *p) { return *p; }

template <typename T> __device__ __forceinline__ void store_act(T *p, float x);
template <> __device__ __forceinline__ void store_act<uint16_t>(uint16_t *p, float x) {
    *p = __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <> __device__ __forceinline__ void store_act<float>(float *p, float x) { *p = x; }

template <typename T, int D, int NS>
__global__ __launch_bounds__(DT) void decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ slopes, float *__restrict__ state, T *__restrict__ out, int64_t H,
    int64_t sb, int64_t sh)
{
    constexpr int DC = D / NS;        // columns of this workgroup's slice
    constexpr int CG = DC / 4;        // float4 column groups of the slice
    constexpr int RG = DT / CG;       // row groups
    constexpr int RPT = D / RG;       // rows per thread
    __shared__ float red[RG][DC];
    __shared__ float qk[2][D];

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / NS;
    const int j0 = (int)(blockIdx.x % NS) * DC;
    const float lam = decay_pow(slopes[bh % H], 1);
    const int cg = tid % CG, rg = tid / CG;

    f32x4 *S = reinterpret_cast<f32x4 *>(state + bh * D * D + j0);
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = __builtin_nontemporal_load(&S[(rg + RG * m) * (D / 4) + cg]);

    const int64_t in0 = (bh / H) * sb + (bh % H) * sh;
    if (tid < D) {
        qk[0][tid] = load_act<T>(q + in0 + tid);
        qk[1][tid] = load_act<T>(k + in0 + tid);
    }
    const T *vb = v + in0 + j0 + 4 * cg;
    const float v0 = load_act<T>(vb), v1 = load_act<T>(vb + 1), v2 = load_act<T>(vb + 2),
                v3 = load_act<T>(vb + 3);
    __syncthreads();

    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const float ki = qk[1][i], qi = qk[0][i];
        f32x4 x = s[m];
        x.x = fmaf(lam, x.x, ki * v0);
        x.y = fmaf(lam, x.y, ki * v1);
        x.z = fmaf(lam, x.z, ki * v2);
        x.w = fmaf(lam, x.w, ki * v3);
        __builtin_nontemporal_store(x, &S[i * (D / 4) + cg]);
        o0 = fmaf(qi, x.x, o0);
        o1 = fmaf(qi, x.y, o1);
        o2 = fmaf(qi, x.z, o2);
        o3 = fmaf(qi, x.w, o3);
    }
    red[rg][4 * cg + 0] = o0;
    red[rg][4 * cg + 1] = o1;
    red[rg][4 * cg + 2] = o2;
    red[rg][4 * cg + 3] = o3;
    __syncthreads();
    if (tid < DC) {
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) acc += red[g][tid];
        store_act<T>(out + bh * D + j0 + tid, acc);
    }
}

// Several tokens per sequence (multi-token decode / draft verification): for
// t = 0..NT-1, S = lambda S + k_t^T v_t and o_t = q_t S, all in registers; the
// state goes back to HBM right after token ncommit-1 (ncommit = n_commit[b]
// clamped to [0, NT], NT if n_commit is null), so tokens past the committed
// prefix produce outputs but never reach the stored state.  One state read
// and at most one write serve all NT tokens; the NT partial-sum reductions
// share one LDS pass.
constexpr int MAXT = 8;   // tokens per sequence and call

template <typename T, int D, int NS>
__global__ __launch_bounds__(DT) void decode_multi_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ slopes, const int32_t *__restrict__ n_commit,
    float *__restrict__ state, T *__restrict__ out, int64_t H, int NT,
    int64_t sb, int64_t sh, int64_t st)
{
    constexpr int DC = D / NS;        // columns of this workgroup's slice
    constexpr int CG = DC / 4;        // float4 column groups of the slice
    constexpr int RG = DT / CG;       // row groups
    constexpr int RPT = D / RG;       // rows per thread
    __shared__ float red[RG][MAXT][DC];
    __shared__ float qk[MAXT][2][D];

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / NS;
    const int j0 = (int)(blockIdx.x % NS) * DC;
    const float lam = decay_pow(slopes[bh % H], 1);
    const int ncommit = n_commit ? min(max(n_commit[bh / H], 0), NT) : NT;
    const int cg = tid % CG, rg = tid / CG;

    f32x4 *S = reinterpret_cast<f32x4 *>(state + bh * D * D + j0);
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = __builtin_nontemporal_load(&S[(rg + RG * m) * (D / 4) + cg]);

    const int64_t a0 = bh * NT * D;   // first output element of this (b, h)
    const int64_t in0 = (bh / H) * sb + (bh % H) * sh;   // its first input row
    for (int e = tid; e < NT * D; e += DT) {
        qk[e / D][0][e % D] = load_act<T>(q + in0 + (e / D) * st + e % D);
        qk[e / D][1][e % D] = load_act<T>(k + in0 + (e / D) * st + e % D);
    }
    float vv[MAXT][4];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[t][j] = 0.f;
        if (t < NT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) vv[t][j] = load_act<T>(v + in0 + t * st + j0 + 4 * cg + j);
        }
    }
    __syncthreads();

#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        if (t >= NT) break;
        float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float ki = qk[t][1][i], qi = qk[t][0][i];
            f32x4 x = s[m];
            x.x = fmaf(lam, x.x, ki * vv[t][0]);
            x.y = fmaf(lam, x.y, ki * vv[t][1]);
            x.z = fmaf(lam, x.z, ki * vv[t][2]);
            x.w = fmaf(lam, x.w, ki * vv[t][3]);
            s[m] = x;
            o0 = fmaf(qi, x.x, o0);
            o1 = fmaf(qi, x.y, o1);
            o2 = fmaf(qi, x.z, o2);
            o3 = fmaf(qi, x.w, o3);
        }
        if (t == ncommit - 1) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) __builtin_nontemporal_store(s[m], &S[(rg + RG * m) * (D / 4) + cg]);
        }
        red[rg][t][4 * cg + 0] = o0;
        red[rg][t][4 * cg + 1] = o1;
        red[rg][t][4 * cg + 2] = o2;
        red[rg][t][4 * cg + 3] = o3;
    }
    __syncthreads();
    for (int e = tid; e < NT * DC; e += DT) {
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < RG; ++g) acc += red[g][e / DC][e % DC];
        store_act<T>(out + a0 + (e / DC) * D + j0 + e % DC, acc);
    }
}

// column slices per (b, h) state: enough workgroups to fill the chip (the
// single and multi-token kernels use the same split, so their results agree
// bitwise)
int decode_slices(int64_t bh) { return bh <= 256 ? 4 : (bh <= 1024 ? 2 : 1); }

template <typename T, int D>
const void *decode_fn(int ns) {
    return ns == 4 ? (const void *)decode_kernel<T, D, 4>
         : ns == 2 ? (const void *)decode_kernel<T, D, 2> : (const void *)decode_kernel<T, D, 1>;
}

template <typename T, int D>
const void *decode_multi_fn(int ns) {
    return ns == 4 ? (const void *)decode_multi_kernel<T, D, 4>
         : ns == 2 ? (const void *)decode_multi_kernel<T, D, 2>
                   : (const void *)decode_multi_kernel<T, D, 1>;
}

template <typename T>
hipError_t launch_decode_multi(const T *q, const T *k, const T *v, const float *slopes,
                               const int32_t *n_commit, float *state, T *out, int64_t B,
                               int64_t H, int nt, int d, const Strides &in, hipStream_t stream)
{
    const int ns = decode_slices(B * H);
    const dim3 grid((unsigned)(B * H * ns)), block(DT);
    int64_t sb = in.sb, sh = in.sh, st = in.st;
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes, (void *)&n_commit,
                    (void *)&state, (void *)&out, (void *)&H, (void *)&nt, (void *)&sb,
                    (void *)&sh, (void *)&st};
    const void *fn = d == 64 ? decode_multi_fn<T, 64>(ns) : decode_multi_fn<T, 128>(ns);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

template <typename T>
hipError_t launch_decode(const T *q, const T *k, const T *v, const float *slopes, float *state,
                         T *out, int64_t B, int64_t H, int d, const Strides &in,
                         hipStream_t stream)
{
    const int ns = decode_slices(B * H);
    const dim3 grid((unsigned)(B * H * ns)), block(DT);
    int64_t sb = in.sb, sh = in.sh;
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                    (void *)&state, (void *)&out, (void *)&H, (void *)&sb, (void *)&sh};
    const void *fn = d == 64 ? decode_fn<T, 64>(ns) : decode_fn<T, 128>(ns);
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace

hipError_t launch_decode_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *slopes, float *state, uint16_t *out,
                              int64_t B, int64_t H, int d, const Strides &in, hipStream_t stream)
{
    return launch_decode<uint16_t>(q, k, v, slopes, state, out, B, H, d, in, stream);
}

hipError_t launch_decode_f32(const float *q, const float *k, const float *v,
                             const float *slopes, float *state, float *out,
                             int64_t B, int64_t H, int d, hipStream_t stream)
{
    const Strides in = {H * d, d, d};
    return launch_decode<float>(q, k, v, slopes, state, out, B, H, d, in, stream);
}

hipError_t launch_decode_multi_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                    const float *slopes, const int32_t *n_commit, float *state,
                                    uint16_t *out, int64_t B, int64_t H, int nt, int d,
                                    const Strides &in, hipStream_t stream)
{
    return launch_decode_multi<uint16_t>(q, k, v, slopes, n_commit, state, out, B, H, nt, d,
                                         in, stream);
}

hipError_t launch_decode_multi_f32(const float *q, const float *k, const float *v,
                                   const float *slopes, const int32_t *n_commit, float *state,
                                   float *out, int64_t B, int64_t H, int nt, int d,
                                   hipStream_t stream)
{
    const Strides in = {H * nt * d, nt * d, d};
    return launch_decode_multi<float>(q, k, v, slopes, n_commit, state, out, B, H, nt, d, in,
                                      stream);
}

int decode_multi_max_tokens() { return MAXT; }

}  // namespace la
