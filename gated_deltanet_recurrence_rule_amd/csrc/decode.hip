// decode.hip -- one gated delta-rule token for every (sequence, V head), state in place.
//
// The rule (handbook page "7. Gated DeltaNet: the token-by-token recurrence",
// section "The formula"; the four steps of its figure "one step of the delta
// rule"):  S <- a S;  p = S^T k;  S <- S + k (b (v - p))^T;  o = S^T q.
//
// A workgroup owns one (sequence, V head) table S [DK, DV] fp32 at a time and touches
// it in exactly one read pass and one write pass, which is what makes the step
// HBM-bound at ~8 bytes of state traffic per table element.  The single pass
// rests on two rewrites of the same arithmetic:
//   p = a (S^T k)                          -- look-up on the undecayed table
//   o = a (S^T q) + (q . k) d,  d = b (v - p)
// since the new table is a S + k d^T, so its read is a S^T q + k^T q d.
// Both S^T k and S^T q are therefore reduced from the same registers while
// the table streams in; the write pass needs only d.
//
// Thread layout (NT = DV / 4 * kRowGroups threads, 4 DV at the default 16 row groups; 8
// and 32 measured the same on the 256-sequence batch): thread t owns the column quad
// c = t % (DV/4) (columns 4c..4c+3) and the rows r = t / (DV/4) + kRowGroups m,
// m < DK/kRowGroups.  One wave load instruction therefore covers 64 float4 = whole
// contiguous rows of the table, and each thread keeps DK/kRowGroups float4 of S in
// registers between the read and the write.
//
// Persistent workgroups: the grid is capped (four workgroups per compute unit) and each
// workgroup walks the units blockIdx.x, blockIdx.x + gridDim.x, ...  The next unit's
// table read is issued before the current unit's write pass, so a workgroup's HBM reads
// and writes overlap instead of alternating (on 8192 tables of 128 x 128: 176 us against
// 190 us with one workgroup per unit, bit-identical results).
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

#ifndef GDN_DECODE_ROW_GROUPS
#define GDN_DECODE_ROW_GROUPS 16
#endif
constexpr int kRowGroups = GDN_DECODE_ROW_GROUPS;

template <int DK, int DV, typename T>
__global__ __launch_bounds__((DV / 4) * kRowGroups) void decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ S,
    T *__restrict__ o, int HV, int rep, float scale, int delta, GateArgs gate,
    const T *__restrict__ z, const float *__restrict__ norm_w, float norm_eps, int nunits) {
    constexpr int NQ = DV / 4;          // column quads
    constexpr int NT = NQ * kRowGroups; // threads
    constexpr int RPT = DK / kRowGroups;
    constexpr int NW = NT / 64;         // waves
    constexpr int RG_PER_WAVE = 64 / NQ;

    __shared__ float kh_s[DK];
    __shared__ float qh_s[DK];
    __shared__ float part_s[NW][2][DV];  // per-wave partial S^T k and S^T q
    __shared__ float d_s[DV];
    __shared__ float qk_s;
    __shared__ float ss_s[(DV + 63) / 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cq = tid % NQ;
    const int rg = tid / NQ;
    const size_t toff = (size_t)rg * DV + 4 * cq;  // this thread's first element in a table

    int unit = blockIdx.x;  // n * HV + h
    if (unit >= nunits) return;

    // Issue the whole first table read; everything below overlaps with it.
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = ld_stream(S + (size_t)unit * DK * DV + toff + (size_t)kRowGroups * m * DV);

    for (;;) {
        const int h = unit % HV;
        const int n = unit / HV;
        const int hq = h / rep;
        float *Sp = S + (size_t)unit * DK * DV;

        float a = 1.f, b = 1.f;
        if (g) {
            float x = g[unit];
            if (gate.alpha_sigmoid) x = -softplus_f(-(x + (gate.dt_bias ? gate.dt_bias[h] : 0.f)));
            else if (gate.A_log) x = -expf(gate.A_log[h]) * softplus_f(x + (gate.dt_bias ? gate.dt_bias[h] : 0.f));
            a = expf(x);
        }
        if (beta) b = gate.beta_logit ? sigmoid_f(beta[unit]) : beta[unit];

        // Wave 0: normalise this token's q and k (shared by the `rep` V heads of QK head hq).
        if (wave == 0) {
            const T *qp = q + ((size_t)n * (HV / rep) + hq) * DK;
            const T *kp = k + ((size_t)n * (HV / rep) + hq) * DK;
            constexpr int EPL = (DK + 63) / 64;
            float qx[EPL], kx[EPL];
            float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int i = lane + 64 * e;
                qx[e] = i < DK ? elem<T>::ld(qp + i) : 0.f;
                kx[e] = i < DK ? elem<T>::ld(kp + i) : 0.f;
                sq += qx[e] * qx[e];
                sk += kx[e] * kx[e];
                sqk += qx[e] * kx[e];
            }
            sq = wave_sum(sq);
            sk = wave_sum(sk);
            sqk = wave_sum(sqk);
            const float rq = inv_norm(sq) * scale;
            const float rk = inv_norm(sk);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int i = lane + 64 * e;
                if (i < DK) {
                    qh_s[i] = qx[e] * rq;
                    kh_s[i] = kx[e] * rk;
                }
            }
            if (lane == 0) qk_s = sqk * rq * rk;
        }
        __syncthreads();

        // Partial S^T k and S^T q over this thread's rows.
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int r = rg + kRowGroups * m;
            pk += s[m] * kh_s[r];
            pq += s[m] * qh_s[r];
        }
        // Reduce over the row groups held by this wave, then across waves in LDS.
#pragma unroll
        for (int off = NQ; off < 64; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pk[c] += __shfl_xor(pk[c], off, 64);
                pq[c] += __shfl_xor(pq[c], off, 64);
            }
        }
        if (lane < NQ) {
            *reinterpret_cast<f32x4 *>(&part_s[wave][0][4 * cq]) = pk;
            *reinterpret_cast<f32x4 *>(&part_s[wave][1][4 * cq]) = pq;
        }
        (void)RG_PER_WAVE;
        __syncthreads();

        float oj = 0.f;
        const size_t vo = (size_t)unit * DV + tid;
        if (tid < DV) {
            const int j = tid;
            float ak = 0.f, aq = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                ak += part_s[w][0][j];
                aq += part_s[w][1][j];
            }
            const float d = b * (elem<T>::ld(v + vo) - (delta ? a * ak : 0.f));
            d_s[j] = d;
            oj = a * aq + qk_s * d;
            if (!z) elem<T>::st(o + vo, oj);
        }
        if (z && wave < (DV + 63) / 64) {
            const float ss = wave_sum(tid < DV ? oj * oj : 0.f);
            if (lane == 0) ss_s[wave] = ss;
        }
        __syncthreads();

        // Gated RMS norm of the read (the block's output gate), in fp32 before the one rounding.
        if (z && tid < DV) {
            float ss = 0.f;
#pragma unroll
            for (int w = 0; w < (DV + 63) / 64; ++w) ss += ss_s[w];
            const float r = __builtin_amdgcn_rsqf(ss * (1.f / DV) + norm_eps);
            elem<T>::st(o + vo, norm_w[tid] * (oj * r) * silu_f(elem<T>::ld(z + vo)));
        }

        // The next unit's table read goes out before this unit's write pass.
        const bool more = unit < nunits - (int)gridDim.x;
        const int next = more ? unit + (int)gridDim.x : unit;
        f32x4 sn[RPT];
        if (more) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) sn[m] = ld_stream(S + (size_t)next * DK * DV + toff + (size_t)kRowGroups * m * DV);
        }

        // Write pass: S <- a S + k d^T.
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&d_s[4 * cq]);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int r = rg + kRowGroups * m;
            st_stream(Sp + (size_t)r * DV + 4 * cq, a * s[m] + kh_s[r] * d4);
        }
        if (!more) break;
        __syncthreads();  // every thread is done with this unit's LDS before it is rewritten
        unit = next;
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = sn[m];
    }
}

template <int DK, int DV, typename T>
hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
    const int rep = a.HV / a.HQK;
    const int nunits = a.N * a.HV;  // the caller bounds N * HV by INT32_MAX
    const int cap = a.max_wgs > 0 ? a.max_wgs : nunits;
    dim3 grid((unsigned)(nunits < cap ? nunits : cap));
    static_assert(DK % kRowGroups == 0 && (DV / 4) * kRowGroups >= DV && (DV / 4) * kRowGroups <= 1024,
                  "row groups must divide DK and give DV..1024 threads");
    hipLaunchKernelGGL((decode_kernel<DK, DV, T>), grid, dim3((DV / 4) * kRowGroups), 0, stream,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), a.g, a.beta, a.S, static_cast<T *>(a.o), a.HV,
                       rep, a.scale, a.delta, a.gate, static_cast<const T *>(a.z), a.norm_w, a.norm_eps, nunits);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const DecodeArgs &a, hipStream_t stream) {
#define GDN_DECODE_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch<DK_, DV_, T>(a, stream);
    GDN_DECODE_CASE(32, 32) GDN_DECODE_CASE(32, 64) GDN_DECODE_CASE(32, 128)
    GDN_DECODE_CASE(64, 32) GDN_DECODE_CASE(64, 64) GDN_DECODE_CASE(64, 128)
    GDN_DECODE_CASE(128, 32) GDN_DECODE_CASE(128, 64) GDN_DECODE_CASE(128, 128)
#undef GDN_DECODE_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    return bf16 ? dispatch<uint16_t>(a, stream) : dispatch<float>(a, stream);
}

}  // namespace gdn
