// qk_prologue.h — QK Norm and RoPE applied to q and k rows as a kernel loads
// them, so that the attention kernels read the projection's raw q and k
// (Ling and Ring 2.6 Technical Report, Fig. 2: QKV projection -> QK Norm ->
// RoPE -> linear attention; §4.3 fuses "QK Norm + RoPE" into one kernel, here
// it moves into the attention kernel's loads instead; §2.1.1: RMSNorm epsilon
// 1e-6, RoPE base 6e6, rotary dimension 64 of the 128 head dims).
//
// For one q or k row x of d = 128 channels at position p:
//   z = x / sqrt(mean_i x_i^2 + eps) * weight                    (RMSNorm)
//   for j < rot/2, a = p * theta^(-2j/rot):
//     z'_j = z_j cos a - z_{j+rot/2} sin a,  z'_{j+rot/2} = z_{j+rot/2} cos a + z_j sin a
//   channels >= rot pass through                                  (rotate-half RoPE)
// The same arithmetic as the stand-alone qk_norm_rope kernel, in fp32, with
// the result rounded once to bf16 (the attention kernels' operand type).
//
// Lane layout: four lanes (one DPP quad) own a row; lane j of the quad loads
// the row's 16-byte chunks j, j+4, j+8 and j+12 (8 channels each; one load
// instruction per chunk covers 64 contiguous bytes of 16 rows).  A rotary
// pair of chunks (c, c + rot/16) then sits in one lane for rot = 64 (chunks
// j and j+4; j+8, j+12 do not rotate) and rot = 128 (j with j+8, j+4 with
// j+12), so the rotation needs no data from other lanes, the non-rotating
// chunks skip it, and a lane's channels share one position: 8 angles per
// row (16 at rot = 128) instead of one per channel.  rot = 16 and 32 pair
// chunks inside the first 64 bytes (lanes j and j ^ rot/16 of the quad; one
// DPP move).  The sum of squares of a row comes from the packed bf16 pairs
// (v_dot2c_f32_bf16) and is reduced over the quad with two DPP adds.
//
// Angles: for each of the lane's pair indices the angle p g (g = the pair's
// frequency in revolutions per position, fp64) is reduced exactly to
// [-1/2, 1/2] revolutions in fp64, and its cosine and sine come from the
// hardware's revolution-based v_cos_f32 / v_sin_f32, for every block (a
// recurrence from block to block measured no faster, and reading weights or
// angle state from LDS on every block measured slower: the consumer waves
// keep the LDS busy).
#pragma once

#include "la_internal.h"

namespace la {
namespace pro {

constexpr int PD = 128;       // head dimension of the prologue
constexpr int LPR = 4;        // lanes per row (one DPP quad)
constexpr int NC = 4;         // 16-byte chunks per lane: j + 4u, u = 0..3

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xf, 0xf, true));
}

// revolutions per position of rotary pair i (frequency theta^(-2i/rot) / 2 pi)
__device__ __forceinline__ double pair_rev(int i, int rot, double log2_theta)
{
    return exp2(-2.0 * i / rot * log2_theta) * 0.15915494309189535;
}

// Per-lane constants, computed once per kernel (ROT: the rotary dims, a
// compile-time constant of the kernel, equal to QkPrologue::rot).
template <int ROT>
struct Lane {
    static_assert(ROT == 0 || ROT == 16 || ROT == 32 || ROT == 64 || ROT == 128, "rotary dims");
    int j;                    // quad index: chunks j + 4u
    float wq[NC][8], wk[NC][8];   // norm weights of the lane's channels (wk: 0 if q only)
    double g[8];              // revolutions per position of the lane's pair indices:
                              //   rot 64: chunk j (and its partner j+4);  rot 128: j (with
                              //   j+8), and j+4 (with j+12) at g * kb;  rot 16, 32: chunk j,
                              //   signed (negative on the first half), 0 off the rotary dims
    double kb;                // rot 128: theta^(-1/2), the frequency ratio of pairs 32 apart

    __device__ void init(const QkPrologue &pr, int quad_lane)
    {
        constexpr int rot = ROT;
        j = quad_lane;
        const double lt = rot > 0 ? log2(pr.theta) : 0.0;
        kb = rot == 128 ? exp2(-0.5 * lt) : 0.0;
#pragma unroll
        for (int u = 0; u < NC; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wq[u][e] = pr.qw[8 * (j + 4 * u) + e];
                wk[u][e] = pr.kw ? pr.kw[8 * (j + 4 * u) + e] : 0.0f;
            }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = 8 * j + e;
            g[e] = 0.0;
            if (rot == 64 || rot == 128) {
                g[e] = pair_rev(ch, rot, lt);
            } else if (rot > 0 && ch < rot) {
                const int half = rot / 2;
                const double f = pair_rev(ch % half, rot, lt);
                g[e] = ch < half ? -f : f;
            }
        }
    }
};

// cos and sin of 2 pi p g k for the lane's 8 pair indices g (k = 1, or kb)
__device__ __forceinline__ void angles(const double (&g)[8], double k, int64_t pos, float (&cs)[8],
                                       float (&sn)[8])
{
    const double p = (double)pos * k;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        double a = p * g[e];
        a -= rint(a);                                   // exact: |a| <= 1/2 revolution
        cs[e] = __builtin_amdgcn_cosf((float)a);
        sn[e] = __builtin_amdgcn_sinf((float)a);
    }
}

// sum of the squares of a chunk's 8 bf16 values plus c, straight from the
// packed pairs (v_dot2c_f32_bf16: exact products, fp32 sums)
__device__ __forceinline__ float sumsq8(uint4 x, float c)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    auto d2 = [](uint32_t a, float acc) {
        const bf16x2_t v = __builtin_bit_cast(bf16x2_t, a);
        return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
    };
    return d2(x.x, d2(x.y, d2(x.z, d2(x.w, c))));
}

// the inverse RMS of the row whose chunks j + 4u this lane holds (the quad's sum)
__device__ __forceinline__ float inv_rms(const uint4 (&x)[NC], float eps)
{
    float s = (sumsq8(x[0], 0.0f) + sumsq8(x[1], 0.0f)) + (sumsq8(x[2], 0.0f) + sumsq8(x[3], 0.0f));
    s += dpp<0xB1>(s);      // quad_perm [1,0,3,2]
    s += dpp<0x4E>(s);      // quad_perm [2,3,0,1]
    return __builtin_amdgcn_rsqf(fmaf(s, 1.0f / PD, eps));
}

// a chunk's 8 values times their weights, in fp32
__device__ __forceinline__ void weigh(uint4 x, const float (&wv)[8], float (&z)[8])
{
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        z[2 * i] = __uint_as_float(xw[i] << 16) * wv[2 * i];
        z[2 * i + 1] = __uint_as_float(xw[i] & 0xffff0000u) * wv[2 * i + 1];
    }
}

__device__ __forceinline__ uint4 pack(const float (&y)[8], float inv)
{
    return make_uint4(pack_bf16x2(y[0] * inv, y[1] * inv), pack_bf16x2(y[2] * inv, y[3] * inv),
                      pack_bf16x2(y[4] * inv, y[5] * inv), pack_bf16x2(y[6] * inv, y[7] * inv));
}

// chunks a (first half of the pairs) and b (second half) of one row, in-lane:
// a' = a cos - b sin, b' = b cos + a sin
__device__ __forceinline__ void rotate_pair(uint4 &xa, uint4 &xb, const float (&wa)[8],
                                            const float (&wb)[8], const float (&cs)[8],
                                            const float (&sn)[8], float inv)
{
    float za[8], zb[8], ya[8], yb[8];
    weigh(xa, wa, za);
    weigh(xb, wb, zb);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        ya[e] = fmaf(za[e], cs[e], -zb[e] * sn[e]);
        yb[e] = fmaf(zb[e], cs[e], za[e] * sn[e]);
    }
    xa = pack(ya, inv);
    xb = pack(yb, inv);
}

__device__ __forceinline__ void scale_only(uint4 &x, const float (&w)[8], float inv)
{
    float z[8];
    weigh(x, w, z);
    x = pack(z, inv);
}

// rot 16 / 32: chunk j rotates with the chunk of quad lane j ^ (rot/16) (one
// DPP move; the first half's sign sits in g, non-rotary lanes have g = 0)
template <int CTRL>
__device__ __forceinline__ void rotate_quad(uint4 &x, const float (&w)[8], const float (&cs)[8],
                                            const float (&sn)[8], float inv)
{
    float z[8], y[8];
    weigh(x, w, z);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fmaf(z[e], cs[e], dpp<CTRL>(z[e]) * sn[e]);
    x = pack(y, inv);
}

// the angles of a lane's row: (ca, sa) of g, and at rot 128 (cb, sb) of g * kb
struct RowAngles {
    float ca[8], sa[8], cb[8], sb[8];
};

// the angles of the lane's row at position pos
template <int ROT>
__device__ __forceinline__ RowAngles row_angles(const Lane<ROT> &L, int64_t pos)
{
    RowAngles a;
    if constexpr (ROT > 0) angles(L.g, 1.0, pos, a.ca, a.sa);
    if constexpr (ROT == 128) angles(L.g, L.kb, pos, a.cb, a.sb);
    return a;
}

// The angles of a lane's row block after block, for a kernel that visits
// one row's blocks in order, 64 positions apart: exact on the first block and
// on every RESYNC-th, in between the previous block's turned by the exact
// angle of 64 positions (a complex multiplication: 4 fp32 operations per
// pair instead of an fp64 reduction, a sine and a cosine), so the rounding
// of the recurrence never exceeds about RESYNC fp32 roundings.  rot = 128
// (two sets of pairs) takes exact angles on every block.
constexpr int RESYNC = 16;

template <int ROT>
struct BlockAngles {
    static constexpr bool TURN = ROT > 0 && ROT < 128;
    RowAngles a;
    float c64[8], s64[8];     // TURN: cos, sin of each pair's angle over 64 positions
    int step;                 // blocks since the last exact angles

    __device__ void init(const Lane<ROT> &L)
    {
        step = 0;
        if constexpr (TURN) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                double r = 64.0 * L.g[e];
                r -= rint(r);
                sincospif(2.0f * (float)r, &s64[e], &c64[e]);
            }
        }
    }
    // the angles of the next block's row, at position pos
    __device__ __forceinline__ const RowAngles &next(const Lane<ROT> &L, int64_t pos)
    {
        if constexpr (TURN) {
            if (step == 0) {
                a = row_angles(L, pos);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float c = a.ca[e], s = a.sa[e];
                    a.ca[e] = fmaf(c, c64[e], -s * s64[e]);
                    a.sa[e] = fmaf(s, c64[e], c * s64[e]);
                }
            }
            step = step + 1 == RESYNC ? 0 : step + 1;
        } else {
            a = row_angles(L, pos);
        }
        return a;
    }
};

// QK Norm + RoPE of one q or k row of the lane (weights w: L.wq or L.wk) in
// place, with the row's angles a.  All four lanes of the quad take part (DPP).
template <int ROT>
__device__ __forceinline__ void norm_rope(uint4 (&x)[NC], const float (&w)[NC][8], const RowAngles &a,
                                          float eps)
{
    const float inv = inv_rms(x, eps);
    if constexpr (ROT == 64) {
        rotate_pair(x[0], x[1], w[0], w[1], a.ca, a.sa, inv);
        scale_only(x[2], w[2], inv);
        scale_only(x[3], w[3], inv);
    } else if constexpr (ROT == 128) {
        rotate_pair(x[0], x[2], w[0], w[2], a.ca, a.sa, inv);
        rotate_pair(x[1], x[3], w[1], w[3], a.cb, a.sb, inv);
    } else {
        if constexpr (ROT == 16) rotate_quad<0xB1>(x[0], w[0], a.ca, a.sa, inv);      // quad_perm [1,0,3,2]
        else if constexpr (ROT == 32) rotate_quad<0x4E>(x[0], w[0], a.ca, a.sa, inv); // quad_perm [2,3,0,1]
        else scale_only(x[0], w[0], inv);
        scale_only(x[1], w[1], inv);
        scale_only(x[2], w[2], inv);
        scale_only(x[3], w[3], inv);
    }
}

}  // namespace pro
}  // namespace la
