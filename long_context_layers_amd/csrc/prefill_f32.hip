// prefill_f32.hip — blockwise decayed linear attention with fp32 activations.
//
// The same block decomposition as the bf16 MFMA kernel, evaluated with fp32
// vector FMAs (the fp32 path keeps full fp32 operands; rounding them to bf16
// for the matrix cores would cost more accuracy than fp32 callers expect).
// For one (b, h) and the block of c tokens starting at t0 (local a, b < c):
//   P[a][b] = lambda^(a-b) (q_a . k_b)              for b <= a, else 0
//   O[a]    = sum_b P[a][b] v_b + lambda^(a+1) q_a S
//   S       = lambda^c S + sum_b lambda^(c-1-b) k_b^T v_b
// This is the report's split into a local output and a local state per
// sequence piece, joined through the carried [B,H,D,D] state (Ling and Ring
// 2.6 Technical Report, §4.1.1 and Fig. 10), applied block after block.
//
// One workgroup per (sequence, head, 32-column slice of v/S/O) of a dense or
// packed launch; the slice's state stays in LDS for the whole sequence.  Not a throughput kernel: the fp32 path
// serves small fp32 problems and correctness checks.
#include "la_internal.h"

namespace la {
namespace {

constexpr int FC = 32;      // tokens per block
constexpr int FJ = 32;      // state / output columns per workgroup
constexpr int FT = 256;     // threads per workgroup

template <int D>
__global__ __launch_bounds__(FT) void prefill_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ slopes, float *__restrict__ out, float *__restrict__ state,
    SeqMap map)
{
    constexpr int NJ = D / FJ;
    __shared__ float Qs[FC][D + 1];
    __shared__ float Ks[FC][D + 1];
    __shared__ float Vs[FC][FJ];
    __shared__ float Ps[FC][FC + 1];
    __shared__ float Ss[D][FJ];
    __shared__ float pw[FC + 1];          // lambda^n, n = 0..FC

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / NJ;          // sequence * H + head
    const int j0 = (blockIdx.x % NJ) * FJ;
    const float s = slopes[bh % map.H];
    int64_t in0, out0, N;
    seq_slice(map, bh / map.H, bh % map.H, &in0, &out0, &N);
    const int64_t ts = map.in.st, ots = map.out.st;   // token strides (elements)
    if (tid <= FC) pw[tid] = decay_pow(s, tid);

    float *St = state + bh * D * D;
    for (int e = tid; e < D * FJ; e += FT) Ss[e / FJ][e % FJ] = St[(e / FJ) * D + j0 + e % FJ];

    const float *qb = q + in0, *kb = k + in0, *vb = v + in0;
    float *ob = out + out0;

    for (int64_t t0 = 0; t0 < N; t0 += FC) {
        const int c = (int)min((int64_t)FC, N - t0);
        __syncthreads();   // previous block's readers are done; pw / Ss visible
        for (int e = tid; e < FC * D; e += FT) {
            const int a = e / D, f = e % D;
            const bool ok = a < c;
            Qs[a][f] = ok ? qb[(t0 + a) * ts + f] : 0.0f;
            Ks[a][f] = ok ? kb[(t0 + a) * ts + f] : 0.0f;
        }
        for (int e = tid; e < FC * FJ; e += FT) {
            const int a = e / FJ, j = e % FJ;
            Vs[a][j] = a < c ? vb[(t0 + a) * ts + j0 + j] : 0.0f;
        }
        __syncthreads();
        // decayed causal scores of the block
        for (int e = tid; e < FC * FC; e += FT) {
            const int a = e / FC, b = e % FC;
            float acc = 0.0f;
            if (b <= a) {
                for (int f = 0; f < D; ++f) acc = fmaf(Qs[a][f], Ks[b][f], acc);
                acc *= pw[a - b];
            }
            Ps[a][b] = acc;
        }
        __syncthreads();
        // outputs: intra-block scores times V, plus the carried state's term
        for (int e = tid; e < FC * FJ; e += FT) {
            const int a = e / FJ, j = e % FJ;
            if (a < c) {
                float inter = 0.0f, intra = 0.0f;
                for (int i = 0; i < D; ++i) inter = fmaf(Qs[a][i], Ss[i][j], inter);
                for (int b = 0; b <= a; ++b) intra = fmaf(Ps[a][b], Vs[b][j], intra);
                ob[(t0 + a) * ots + j0 + j] = fmaf(pw[a + 1], inter, intra);
            }
        }
        __syncthreads();
        // decayed state scan: S = lambda^c S + sum_b lambda^(c-1-b) k_b^T v_b
        const float dc = pw[c];
        for (int e = tid; e < D * FJ; e += FT) {
            const int i = e / FJ, j = e % FJ;
            float acc = 0.0f;
            for (int b = 0; b < c; ++b) acc = fmaf(pw[c - 1 - b] * Ks[b][i], Vs[b][j], acc);
            Ss[i][j] = fmaf(dc, Ss[i][j], acc);
        }
    }
    __syncthreads();
    for (int e = tid; e < D * FJ; e += FT) St[(e / FJ) * D + j0 + e % FJ] = Ss[e / FJ][e % FJ];
}

}  // namespace

int64_t prefill_f32_grid(int64_t seqs, int64_t H, int d) { return seqs * H * (d / FJ); }

hipError_t launch_prefill_f32(const float *q, const float *k, const float *v,
                              const float *slopes, float *out, float *state,
                              int64_t seqs, const SeqMap &map, int d, hipStream_t stream)
{
    const dim3 grid((unsigned)prefill_f32_grid(seqs, map.H, d)), block(FT);
    SeqMap m = map;
    void *args[] = {(void *)&q, (void *)&k, (void *)&v, (void *)&slopes,
                    (void *)&out, (void *)&state, (void *)&m};
    const void *fn = d == 64 ? (const void *)prefill_f32_kernel<64>
                             : (const void *)prefill_f32_kernel<128>;
    return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace la
