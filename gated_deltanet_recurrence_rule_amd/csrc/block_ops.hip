// block_ops.hip -- the parts of the GatedDeltaNet block that sit directly before and after
// the scan (handbook page "7. Gated DeltaNet: the token-by-token recurrence": the block's
// forward listing and the parts table after it).
//
//   conv_silu       the causal depthwise convolution of width 4 over the concatenated
//                   q | k | v channels, then SiLU (parts table, row "in_proj_qkv + conv1d",
//                   and the note under it: position t sees inputs t-3 .. t, every channel
//                   with its own four weights).  Writes q, k, v in the layout the scan reads.
//   gated_rmsnorm   per-head RMS normalisation of the read, times a per-channel weight and
//                   silu(z) (parts table, row "in_proj_z + GatedRMSNorm").
//
// Both are pure streams: every input byte is read about once and every output byte written
// once, so they are HBM-bound and laid out for 16-byte coalesced accesses.  All arithmetic
// is fp32; bf16 outputs are rounded once, to nearest even.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

// 8 consecutive channels of one token: one 16-byte access for bf16, two for fp32.  Every
// access is nontemporal: each byte is touched once, and keeping the streams out of the
// caches measured 5% (convolution) and 8% (norm) faster on the 4 x 16384-token batch.
template <typename T> struct vec8;
template <> struct vec8<uint16_t> {
    typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
    struct raw_t { u4_t a; };
    static __device__ __forceinline__ raw_t ld_raw(const uint16_t *p) {
        return {__builtin_nontemporal_load(reinterpret_cast<const u4_t *>(p))};
    }
    static __device__ __forceinline__ void decode(const raw_t &r, float (&x)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(r.a[i] << 16);
            x[2 * i + 1] = __uint_as_float(r.a[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void ld(const uint16_t *p, float (&x)[8]) { decode(ld_raw(p), x); }
    // round to nearest even through the packed hardware conversion
    static __device__ __forceinline__ void st(uint16_t *p, const float (&x)[8]) {
        typedef float f32x8_t __attribute__((ext_vector_type(8)));
        typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
        const f32x8_t f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
        __builtin_nontemporal_store(__builtin_bit_cast(u4_t, __builtin_convertvector(f, bf16x8_t)),
                                    reinterpret_cast<u4_t *>(p));
    }
};
template <> struct vec8<float> {
    struct raw_t { f32x4 a, b; };
    static __device__ __forceinline__ raw_t ld_raw(const float *p) {
        return {__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p)),
                __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 1)};
    }
    static __device__ __forceinline__ void decode(const raw_t &r, float (&x)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = r.a[i];
            x[4 + i] = r.b[i];
        }
    }
    static __device__ __forceinline__ void ld(const float *p, float (&x)[8]) { decode(ld_raw(p), x); }
    static __device__ __forceinline__ void st(float *p, const float (&x)[8]) {
        const f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4 *>(p));
        __builtin_nontemporal_store(b, reinterpret_cast<f32x4 *>(p) + 1);
    }
};

// ------------------------------------------------------------------ gated RMS norm
// A row is one (token, head) vector of DV values.  LPR = DV / 8 lanes share a row, each
// holding 8 channels; a wave covers 64 / LPR rows per step and the sum of squares is reduced
// over the row's lanes with xor shuffles.
constexpr int kNormThreads = 256;
#ifndef GDN_NORM_STEPS
#define GDN_NORM_STEPS 1
#endif
constexpr int kNormSteps = GDN_NORM_STEPS;  // row groups per wave

template <int DV, typename T>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(
    const T *__restrict__ x, const T *__restrict__ z, const float *__restrict__ w, T *y, int64_t rows,
    float eps) {
    constexpr int LPR = DV / 8;
    constexpr int RPW = 64 / LPR;  // rows per wave per step
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane % LPR;
    const int64_t base = ((int64_t)blockIdx.x * (kNormThreads / 64) + wave) * RPW * kNormSteps;

    float wr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wr[i] = w[8 * sub + i];

    float xv[kNormSteps][8], zv[kNormSteps][8];
#pragma unroll
    for (int s = 0; s < kNormSteps; ++s) {
        const int64_t r = base + (int64_t)s * RPW + lane / LPR;
        if (r < rows) {
            vec8<T>::ld(x + r * DV + 8 * sub, xv[s]);
            vec8<T>::ld(z + r * DV + 8 * sub, zv[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < kNormSteps; ++s) {
        const int64_t r = base + (int64_t)s * RPW + lane / LPR;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += xv[s][i] * xv[s][i];
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
        const float rn = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
        if (r < rows) {
            float out[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = wr[i] * (xv[s][i] * rn) * silu_f(zv[s][i]);
            vec8<T>::st(y + r * DV + 8 * sub, out);
        }
    }
}

template <int DV, typename T>
hipError_t launch_norm(const NormArgs &a, hipStream_t stream) {
    constexpr int rows_per_block = (kNormThreads / 64) * (64 / (DV / 8)) * kNormSteps;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gated_rmsnorm_kernel<DV, T>), dim3((unsigned)blocks), dim3(kNormThreads), 0, stream,
                       static_cast<const T *>(a.x), static_cast<const T *>(a.z), a.w, static_cast<T *>(a.y),
                       a.rows, a.eps);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_norm(const NormArgs &a, hipStream_t stream) {
    switch (a.dv) {
        case 32: return launch_norm<32, T>(a, stream);
        case 64: return launch_norm<64, T>(a, stream);
        case 128: return launch_norm<128, T>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------------------------ causal conv + SiLU
// Thread = 8 consecutive channels x kConvTokens consecutive tokens of the packed batch.  It
// keeps the three previous inputs of its channels in registers and slides them along; the
// window is refilled from the carried state (or zeros) wherever a sequence starts.  A block
// spans 2048 channels of the same tokens, so every load and store instruction of a wave
// covers 1 KiB (bf16) of one token row.
constexpr int kConvThreads = 256;
#ifndef GDN_CONV_TOKENS
#define GDN_CONV_TOKENS 64
#endif
#ifndef GDN_CONV_GROUP
#define GDN_CONV_GROUP 4
#endif
constexpr int kConvTokens = GDN_CONV_TOKENS;  // tokens per thread
constexpr int kConvGroup = GDN_CONV_GROUP;    // token rows loaded before their arithmetic

// sequence holding token t: the largest n with cu[n] <= t (cu non-decreasing, cu[0] = 0)
__device__ __forceinline__ int seq_of(const int32_t *cu, int N, int64_t eq_len, int64_t t) {
    if (!cu) return (int)(t / eq_len);
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_silu_kernel(
    const T *__restrict__ x, const float *__restrict__ w, const int32_t *__restrict__ cu, int64_t eq_len,
    int N, int64_t total_T, const T *__restrict__ state_in, T *__restrict__ q, T *__restrict__ k,
    T *__restrict__ v, int Cq, int Cv) {
    const int Ct = 2 * Cq + Cv;
    const int c = 8 * (blockIdx.y * kConvThreads + threadIdx.x);
    const int64_t tb = (int64_t)blockIdx.x * kConvTokens;
    if (c >= Ct || tb >= total_T) return;
    const int64_t te = tb + kConvTokens < total_T ? tb + kConvTokens : total_T;

    float wt[4][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 w4 = *reinterpret_cast<const float4 *>(w + 4 * (size_t)(c + i));
        wt[0][i] = w4.x; wt[1][i] = w4.y; wt[2][i] = w4.z; wt[3][i] = w4.w;
    }
    // output column: q, k or v (8-channel groups never straddle, Cq and Cv being multiples of 8)
    T *dst;
    int ld, col;
    if (c < Cq) { dst = q; ld = Cq; col = c; }
    else if (c < 2 * Cq) { dst = k; ld = Cq; col = c - Cq; }
    else { dst = v; ld = Cv; col = c - 2 * Cq; }

    // device entries are clamped into [0, total_T] and made non-decreasing, so no cu_seqlens
    // contents can send the kernel outside its buffers
    int n = seq_of(cu, N, eq_len, tb);
    int64_t s0 = cu ? clamp_tok(cu[n], 0, total_T) : (int64_t)n * eq_len;
    int64_t s1 = cu ? clamp_tok(cu[n + 1], s0, total_T) : s0 + eq_len;

    // input at absolute token t of sequence n (t may be up to 3 before its start)
    auto fetch = [&](int64_t t, float (&e)[8]) {
        if (t >= s0) {
            vec8<T>::ld(x + t * Ct + c, e);
        } else if (state_in && s0 - t <= 3) {
            vec8<T>::ld(state_in + ((size_t)n * 3 + (size_t)(3 - (s0 - t))) * Ct + c, e);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = 0.f;
        }
    };
    float e1[8], e2[8], e3[8];  // inputs at t - 3, t - 2, t - 1
    fetch(tb - 3, e1);
    fetch(tb - 2, e2);
    fetch(tb - 1, e3);
    // one token: convolve, SiLU, store, slide the window
    auto step = [&](int64_t t, const float (&cur)[8]) {
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = wt[0][i] * e1[i];
            acc = fmaf(wt[1][i], e2[i], acc);
            acc = fmaf(wt[2][i], e3[i], acc);
            acc = fmaf(wt[3][i], cur[i], acc);
            out[i] = silu_f(acc);
            e1[i] = e2[i];
            e2[i] = e3[i];
            e3[i] = cur[i];
        }
        vec8<T>::st(dst + t * ld + col, out);
    };
    int64_t t = tb;
    while (t < te) {
        if (t >= s1) {
            // the next non-empty sequence starts here (t == s1 for a consistent array):
            // refill the window from its state
            do {
                s0 = s1;
                if (n + 1 < N) {
                    ++n;
                    s1 = cu ? clamp_tok(cu[n + 1], s0, total_T) : s0 + eq_len;
                } else {
                    s1 = total_T;  // only an inconsistent device array gets here
                }
            } while (s1 <= t);
            fetch(t - 3, e1);
            fetch(t - 2, e2);
            fetch(t - 1, e3);
        }
        const int64_t stop = te < s1 ? te : s1;
        // groups of kConvGroup rows; the next group's loads are issued before this group's
        // arithmetic, so a thread keeps a group in flight while it computes
        if (t + kConvGroup <= stop) {
            typename vec8<T>::raw_t rw[kConvGroup];
#pragma unroll
            for (int u = 0; u < kConvGroup; ++u) rw[u] = vec8<T>::ld_raw(x + (t + u) * Ct + c);
            for (; t + kConvGroup <= stop; t += kConvGroup) {
                typename vec8<T>::raw_t nx[kConvGroup];
                const bool more = t + 2 * kConvGroup <= stop;
                if (more) {
#pragma unroll
                    for (int u = 0; u < kConvGroup; ++u) nx[u] = vec8<T>::ld_raw(x + (t + kConvGroup + u) * Ct + c);
                }
#pragma unroll
                for (int u = 0; u < kConvGroup; ++u) {
                    float cur[8];
                    vec8<T>::decode(rw[u], cur);
                    step(t + u, cur);
                }
                if (more) {
#pragma unroll
                    for (int u = 0; u < kConvGroup; ++u) rw[u] = nx[u];
                }
            }
        }
        for (; t < stop; ++t) {
            float cur[8];
            vec8<T>::ld(x + t * Ct + c, cur);
            step(t, cur);
        }
    }
}

// state_out[n] = the last three entries of (state_in[n] ++ inputs of sequence n).  Launched
// after conv_silu_kernel on the same stream, so state_out may be the same buffer as state_in:
// each thread reads its three entries before it writes them.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_state_kernel(
    const T *__restrict__ x, const int32_t *__restrict__ cu, int64_t eq_len, int N, int64_t total_T,
    const T *state_in,
    T *state_out, int Ct) {
    const int c = 8 * (blockIdx.y * kConvThreads + threadIdx.x);
    const int n = blockIdx.x;
    if (c >= Ct || n >= N) return;
    const int64_t s0 = cu ? clamp_tok(cu[n], 0, total_T) : (int64_t)n * eq_len;
    const int64_t len = (cu ? clamp_tok(cu[n + 1], s0, total_T) : s0 + eq_len) - s0;
    float e[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t p = len + j;  // index into (state ++ inputs)
        if (p >= 3) {
            vec8<T>::ld(x + (s0 + p - 3) * Ct + c, e[j]);
        } else if (state_in) {
            vec8<T>::ld(state_in + ((size_t)n * 3 + (size_t)p) * Ct + c, e[j]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) e[j][i] = 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) vec8<T>::st(state_out + ((size_t)n * 3 + j) * Ct + c, e[j]);
}

template <typename T>
hipError_t launch_conv(const ConvArgs &a, hipStream_t stream) {
    const int Ct = 2 * a.Cq + a.Cv;
    const unsigned cblocks = (unsigned)((Ct / 8 + kConvThreads - 1) / kConvThreads);
    if (a.total_T > 0) {
        const int64_t tblocks = (a.total_T + kConvTokens - 1) / kConvTokens;
        if (tblocks > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL((conv_silu_kernel<T>), dim3((unsigned)tblocks, cblocks), dim3(kConvThreads), 0, stream,
                           static_cast<const T *>(a.x), a.w, a.cu_seqlens, a.eq_len, a.N, a.total_T,
                           static_cast<const T *>(a.state_in), static_cast<T *>(a.q), static_cast<T *>(a.k),
                           static_cast<T *>(a.v), a.Cq, a.Cv);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.state_out) {
        hipLaunchKernelGGL((conv_state_kernel<T>), dim3((unsigned)a.N, cblocks), dim3(kConvThreads), 0, stream,
                           static_cast<const T *>(a.x), a.cu_seqlens, a.eq_len, a.N, a.total_T,
                           static_cast<const T *>(a.state_in), static_cast<T *>(a.state_out), Ct);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_conv_silu(const ConvArgs &a, bool bf16, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    return bf16 ? launch_conv<uint16_t>(a, stream) : launch_conv<float>(a, stream);
}

hipError_t launch_gated_rmsnorm(const NormArgs &a, bool bf16, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    return bf16 ? dispatch_norm<uint16_t>(a, stream) : dispatch_norm<float>(a, stream);
}

}  // namespace gdn
