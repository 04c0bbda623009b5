// la_internal.h — declarations shared by the library's own translation units
// (kernel launchers and small device helpers).  Not installed, not part of the
// C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// ---- launchers (return the launch status; arguments already validated) ----
hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *slopes, uint16_t *out, float *state,
                               int64_t B, int64_t H, int64_t N, int d, hipStream_t stream);
hipError_t launch_prefill_f32(const float *q, const float *k, const float *v,
                              const float *slopes, float *out, float *state,
                              int64_t B, int64_t H, int64_t N, int d, hipStream_t stream);
hipError_t launch_decode_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *slopes, float *state, uint16_t *out,
                              int64_t B, int64_t H, int d, hipStream_t stream);
hipError_t launch_decode_f32(const float *q, const float *k, const float *v,
                             const float *slopes, float *state, float *out,
                             int64_t B, int64_t H, int d, hipStream_t stream);

// number of workgroups one prefill launch uses (for the host-side grid check)
int64_t prefill_bf16_grid(int64_t B, int64_t H, int d);
int64_t prefill_f32_grid(int64_t B, int64_t H, int d);

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
