// prefill_recurrent.hip -- token-serial prefill with fp32 arithmetic throughout.
//
// This is the direct form of the handbook's delta_rule (page "7. Gated DeltaNet:
// the token-by-token recurrence", qwen/deltanet.py listing and section "The
// formula"): for each token, decay, look up, write the difference, read.  It is
// the library's path for fp32 inputs (where every product must stay fp32) and
// for shapes the chunked MFMA kernel does not cover.
//
// Mapping: one wave per (sequence, V head, 64-column slice of dv).  Lane j owns
// column j of the table, all DK rows of it in VGPRs, so both reductions over the
// key dimension (S^T k and S^T q) are lane-local; the only cross-lane work per
// token is the L2 norm of q and k, done with wave reductions, and a broadcast of
// the normalised vectors through LDS.  Per token and lane:
//   p = S^T k^,  r = S^T q^  (from the undecayed table)
//   d = b (v - a p),  o = a r + (q^ . k^) d,  S <- a S + k^ d
// (the same identity as the decode step: the new table is a S + k^ d^T).
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

template <int DK, typename T>
__global__ __launch_bounds__(64) void prefill_recurrent_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ order, int64_t span,
    const float *__restrict__ S0, T *__restrict__ o, float *__restrict__ S_T, int HV, int DV, int rep,
    float scale, int delta, GateArgs gate) {
    constexpr int EPL = (DK + 63) / 64;  // q/k elements per lane
    __shared__ float kh_s[DK];
    __shared__ float qh_s[DK];

    // launch rank * HV + h; rank -> sequence through the longest-first order
    const int h = blockIdx.x % HV;
    const int rank = blockIdx.x / HV;
    const int n = order ? order[rank] : rank;
    const int unit = n * HV + h;
    const int hq = h / rep;
    const int HQK = HV / rep;
    const int lane = threadIdx.x;
    const int j = blockIdx.y * 64 + lane;
    const bool active = j < DV;

    int64_t t0, t1;
    if (cu_seqlens) {  // span = total_T: entries clamped into [0, total_T], non-decreasing
        t0 = clamp_tok(cu_seqlens[n], 0, span);
        t1 = clamp_tok(cu_seqlens[n + 1], t0, span);
    } else {
        t0 = (int64_t)n * span;
        t1 = t0 + span;
    }

    float s[DK];
    const size_t tab = (size_t)unit * DK * DV;
#pragma unroll
    for (int i = 0; i < DK; ++i) s[i] = (S0 && active) ? S0[tab + (size_t)i * DV + j] : 0.f;

    // this token's raw q, k, v, g, beta in registers, loaded one token ahead so the global
    // memory latency overlaps the previous token's arithmetic
    float qn[EPL], kn[EPL], vn = 0.f, gn = 0.f, bn = 1.f;
    auto fetch = [&](int64_t t) {
        const T *qp = q + ((size_t)t * HQK + hq) * DK;
        const T *kp = k + ((size_t)t * HQK + hq) * DK;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int i = lane + 64 * e;
            qn[e] = i < DK ? elem<T>::ld(qp + i) : 0.f;
            kn[e] = i < DK ? elem<T>::ld(kp + i) : 0.f;
        }
        const size_t tv = (size_t)t * HV + h;
        vn = active ? elem<T>::ld(v + tv * DV + j) : 0.f;
        gn = g ? g[tv] : 0.f;
        bn = beta ? beta[tv] : 1.f;
    };
    if (t0 < t1) fetch(t0);

    for (int64_t t = t0; t < t1; ++t) {
        float qx[EPL], kx[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            qx[e] = qn[e];
            kx[e] = kn[e];
        }
        const float vj = vn, graw = gn, braw = bn;
        if (t + 1 < t1) fetch(t + 1);
        float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            sq += qx[e] * qx[e];
            sk += kx[e] * kx[e];
            sqk += qx[e] * kx[e];
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        sqk = wave_sum(sqk);
        const float rq = inv_norm(sq) * scale;
        const float rk = inv_norm(sk);
        const float qk = sqk * rq * rk;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int i = lane + 64 * e;
            if (i < DK) {
                qh_s[i] = qx[e] * rq;
                kh_s[i] = kx[e] * rk;
            }
        }
        __syncthreads();

        const size_t tv = (size_t)t * HV + h;
        float a = 1.f, b = 1.f;
        if (g) {
            float x = graw;
            if (gate.alpha_sigmoid) x = -softplus_f(-(x + (gate.dt_bias ? gate.dt_bias[h] : 0.f)));
            else if (gate.A_log) x = -expf(gate.A_log[h]) * softplus_f(x + (gate.dt_bias ? gate.dt_bias[h] : 0.f));
            a = expf(x);
        }
        if (beta) b = gate.beta_logit ? sigmoid_f(braw) : braw;

        // up to DK = 64, four partial sums each, so the two reductions are not one long
        // dependent chain (5% and 11% faster at DK = 32 and 64); at DK = 128 the extra
        // registers cost more than the shorter chain gains
        float p = 0.f, r = 0.f;
        if constexpr (DK <= 64) {
            float pp[4] = {0.f, 0.f, 0.f, 0.f}, rr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < DK; ++i) {
                pp[i & 3] = fmaf(s[i], kh_s[i], pp[i & 3]);
                rr[i & 3] = fmaf(s[i], qh_s[i], rr[i & 3]);
            }
            p = (pp[0] + pp[1]) + (pp[2] + pp[3]);
            r = (rr[0] + rr[1]) + (rr[2] + rr[3]);
        } else {
#pragma unroll
            for (int i = 0; i < DK; ++i) {
                p += s[i] * kh_s[i];
                r += s[i] * qh_s[i];
            }
        }
        const float d = b * (vj - (delta ? a * p : 0.f));
#pragma unroll
        for (int i = 0; i < DK; ++i) s[i] = a * s[i] + kh_s[i] * d;
        if (active) elem<T>::st(o + tv * DV + j, a * r + qk * d);
        __syncthreads();  // kh_s / qh_s are rewritten by the next token
    }

    if (S_T && active) {
#pragma unroll
        for (int i = 0; i < DK; ++i) S_T[tab + (size_t)i * DV + j] = s[i];
    }
}

template <int DK, typename T>
hipError_t launch(const PrefillArgs &a, hipStream_t stream) {
    const int rep = a.HV / a.HQK;
    dim3 grid((unsigned)((int64_t)a.N * a.HV), (unsigned)((a.dv + 63) / 64));
    hipLaunchKernelGGL((prefill_recurrent_kernel<DK, T>), grid, dim3(64), 0, stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), a.g, a.beta, a.cu_seqlens, a.order, a.span(), a.S0,
                       static_cast<T *>(a.o), a.S_T, a.HV, a.dv, rep, a.scale, a.delta, a.gate);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const PrefillArgs &a, hipStream_t stream) {
    switch (a.dk) {
        case 32: return launch<32, T>(a, stream);
        case 64: return launch<64, T>(a, stream);
        case 128: return launch<128, T>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_recurrent(const PrefillArgs &a, bool bf16, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    return bf16 ? dispatch<uint16_t>(a, stream) : dispatch<float>(a, stream);
}

}  // namespace gdn
