// common.hpp -- small device helpers shared by the libgdn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ bf16 <-> fp32
// bf16 is carried as raw uint16 bits.  Widening is exact; narrowing rounds to
// nearest, ties to even, and keeps NaN quiet.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Element access for the two I/O types (float, or bf16 bits in uint16_t).
template <typename T> struct elem;
template <> struct elem<float> {
    static __device__ __forceinline__ float ld(const float *p) { return *p; }
    static __device__ __forceinline__ void st(float *p, float x) { *p = x; }
};
template <> struct elem<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t *p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ void st(uint16_t *p, float x) { *p = f32_to_bf16(x); }
};

// ------------------------------------------------------------------ wave64 reductions
// Sum over the 64 lanes, returned to every lane: an inclusive scan by DPP row shifts
// within each row of 16 lanes, then the row-15 and row-31 broadcasts across rows, leaves
// the total in lane 63, which is read back as a uniform value.  No LDS round trips.
#define GDN_DPP_ADD_(x, ctrl, row_mask) \
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, row_mask, 0xF, true))
__device__ __forceinline__ float wave_sum(float x) {
    GDN_DPP_ADD_(x, 0x111, 0xF);  // row_shr:1
    GDN_DPP_ADD_(x, 0x112, 0xF);  // row_shr:2
    GDN_DPP_ADD_(x, 0x114, 0xF);  // row_shr:4
    GDN_DPP_ADD_(x, 0x118, 0xF);  // row_shr:8
    GDN_DPP_ADD_(x, 0x142, 0xA);  // row_bcast:15 into rows 1 and 3
    GDN_DPP_ADD_(x, 0x143, 0xC);  // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
#undef GDN_DPP_ADD_

// 1 / max(sqrt(ss), eps) with eps = 1e-12: the L2-normalisation factor x / max(|x|, eps).
// Uses the hardware reciprocal square root (about 1 ulp); ss <= eps^2 (zero included)
// gives 1 / eps.
__device__ __forceinline__ float inv_norm(float ss) {
    return ss > 1e-24f ? __builtin_amdgcn_rsqf(ss) : 1e12f;
}

// ------------------------------------------------------------------ gates and activations
// The GatedDeltaNet block's gate maps (handbook page "7. Gated DeltaNet: the token-by-token
// recurrence", parts table): log-decay -exp(A_log) softplus(a + dt_bias), write strength
// sigmoid(b), output gate silu(z).  The per-(token, head) gate maps go through the device
// math library; silu, applied to every element of the streamed block parts, uses the
// hardware exp2 and reciprocal (about 1 ulp each): x / (1 + 2^(-x log2 e)).  Very negative
// x gives 2^(+big) = inf and a reciprocal of 0, so silu -> -0 as it should.
// a token index read from a device cu_seqlens array, clamped into [lo, hi]
__device__ __forceinline__ int64_t clamp_tok(int32_t x, int64_t lo, int64_t hi) {
    const int64_t v = x;
    return v < lo ? lo : (v > hi ? hi : v);
}

__device__ __forceinline__ float softplus_f(float x) { return x > 20.f ? x : log1pf(expf(x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }
__device__ __forceinline__ float silu_f(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.44269504088896341f));
}

// ------------------------------------------------------------------ streaming access
// The state is touched exactly once per decode step: keep it out of the caches.
// (Measured on the 512 MiB decode batch: plain loads and stores instead run 10% slower.)
__device__ __forceinline__ f32x4 ld_stream(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void st_stream(float *p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}

}  // namespace gdn
