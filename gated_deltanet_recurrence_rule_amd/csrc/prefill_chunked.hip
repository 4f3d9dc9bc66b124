// prefill_chunked.hip -- chunk-parallel prefill on bf16 MFMA with an fp32 table.
//
// The recurrence is the handbook's (page "7. Gated DeltaNet: the token-by-token
// recurrence", section "The formula"):  S_t = a_t S_{t-1} + b_t k_t (v_t - a_t
// S_{t-1}^T k_t)^T,  o_t = S_t^T q_t,  with q, k L2-normalised.  The page says
// only that fast implementations process the sequence in chunks and equal the
// loop exactly; the chunk algebra used here is derived from the formula.
// Inside a chunk of n <= 64 tokens with start table S, G_i = g_1 + ... + g_i,
// gamma_i = exp(G_i), r_k, r_q the per-token norm reciprocals (r_q includes
// `scale`), and raw bf16 rows K, Q, V:
//
//   A_ij  = b_i r_k,i r_k,j (K K^T)_ij exp(G_i - G_j)   j < i   (zero otherwise)
//   P_ij  = r_q,i r_k,j (Q K^T)_ij exp(G_i - G_j)       j <= i
//   Z_i   = b_i (v_i - gamma_i r_k,i (K S)_i)
//   (I + A) Delta = Z                                   (unit lower triangular)
//   O_i   = gamma_i r_q,i (Q S)_i + (P Delta)_i
//   S'    = gamma_n S + K^T diag(r_k,i exp(G_n - G_i)) Delta
//
// Only exp(G_i - G_j) <= 1 and exp(G_n - G_i) <= 1 are formed, never 1/gamma.
// The triangular system is split into two 32-token blocks:
//   Delta_0 = T_0 Z_0,   Delta_1 = T_1 (Z_1 - A_10 Delta_0),   T_b = (I + A_bb)^{-1},
// with T_b built in fp32 from 16x16 forward substitutions and one 16-block merge.
//
// Precision.  MFMA operands are bf16; a value that is not exactly bf16 is either
// rounded once or carried as hi + lo (hi = bf16(x), lo = bf16(x - hi); two or
// three MFMAs).  Raw q, k, v rows are exact bf16.  The table path is carried
// hi + lo: S in K S, T_b, A_10 and Z / Delta in the solve, the scaled Delta in
// K^T D.  The output path rounds once: S in Q S, P and Delta in P Delta.  All
// accumulation is fp32.
//
// Mapping.  One workgroup of 8 waves owns one (sequence, V head, 64-column
// slice of dv) and walks its chunks in order; dv columns of S evolve
// independently, so slices need no communication.
//  * Waves 0-3 ("column waves") each own one 16-column tile of the slice and
//    keep everything of it in MFMA accumulators: the 128 x 16 table slice, and
//    per chunk K S, Q S, Z, Delta, D, O.  A K=32 MFMA whose B operand is two
//    stacked 16-row accumulator tiles takes them as they are, provided the A
//    operand enumerates its 32 k-values in the same order (tile t, row 4*(lane/16)+e);
//    all such products here use that order.
//  * Waves 4-7 ("Gram waves") compute the chunk's Gram tiles and write P, -A_10
//    and T_0, T_1 into LDS already in that MFMA operand order (computing a Gram
//    tile with the two operand roles swapped yields it transposed, which is the
//    operand order directly).
// Three workgroup barriers per chunk: load | Grams + (K S, Q S, Z) | solve + state.
// The next chunk's q, k, v, g, beta are fetched into registers one chunk ahead.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int C = 64;       // chunk length
constexpr int DK = 128;     // key dimension
constexpr int DVS = 64;     // dv columns per workgroup
constexpr int NT = 512;     // threads (8 waves)

constexpr int LK = DK + 8;  // row stride (bf16) of K and Q in LDS
constexpr int LT = C + 8;   // row stride (bf16) of K^T in LDS
constexpr int LW = 36;      // row stride (fp32) of the Gram waves' private 32x32 blocks (16-byte rows)

// LDS layout (bytes)
constexpr int OFF_K = 0;                                   // K  [C][LK] bf16, rows = tokens
constexpr int OFF_Q = OFF_K + C * LK * 2;                  // Q  [C][LK]
constexpr int OFF_KT = OFF_Q + C * LK * 2;                 // K^T [2 chunk parity][DK][LT], swizzled
constexpr int OFF_OPT = OFF_KT + 2 * DK * LT * 2;          // T_b operands [2 b][2 rt][2 hi/lo][64][8]
constexpr int OFF_OPA = OFF_OPT + 2 * 2 * 2 * 64 * 16;     // -A_10 operands [2 rt][2 hi/lo][64][8]
constexpr int OFF_OPP = OFF_OPA + 2 * 2 * 64 * 16;         // P operands [6 (rt, ks)][64][8]
constexpr int OFF_WP = OFF_OPP + 6 * 64 * 16;              // per Gram wave 4,5: Af, Tf [32][LW], Rf [16][17]
constexpr int WP_SZ = (2 * 32 * LW + 16 * 17) * 4;
constexpr int SC_SZ = 6 * C;                               // fp32 per-token scalars of one chunk
constexpr int OFF_SC = OFF_WP + 2 * WP_SZ;                 // scalars [2 chunk parity][SC_SZ]
constexpr int OFF_OST = OFF_SC + 2 * SC_SZ * 4;            // per column wave: one 16x16 bf16 output tile
constexpr int LDS_BYTES = OFF_OST + 4 * 16 * 16 * 2;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 to_bf16(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ f32x8 to_f32(bf16x8 x) { return __builtin_convertvector(x, f32x8); }
__device__ __forceinline__ f32x8 cat(f32x4 a, f32x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void split(f32x8 x, bf16x8 &hi, bf16x8 &lo) {
    hi = to_bf16(x);
    lo = to_bf16(x - to_f32(hi));
}
// hi*hi + hi*lo + lo*hi
__device__ __forceinline__ f32x4 mfma32_x3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mfma32(ah, bh, c);
    c = mfma32(ah, bl, c);
    return mfma32(al, bh, c);
}

// Standard-order operand: row r0 + lane%16, k = k0 + 8*(lane/16) .. +7 of a bf16 row-major matrix.
__device__ __forceinline__ bf16x8 ld_std(const __bf16 *base, int stride, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(base + (r0 + (lane & 15)) * stride + k0 + 8 * (lane >> 4));
}
// Tile order inside every 32-element block: stored position 8g + 4t + e holds element
// 16t + 4g + e.  K and Q rows (over d) and K^T rows (over tokens) are kept in LDS in
// this order, so the 8 tile-order operand values of lane group g = lane/16 are one
// contiguous 16-byte read (ld_std at k0 = 32 * block).  Gram products read both
// operands in the same permuted order, which leaves them unchanged.
__device__ __forceinline__ int tile_pos(int x) {
    const int r = x & 31;
    return (x & ~31) + 8 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3);
}
// K^T bank swizzle: 8-element groups are permuted per 8-row band of K^T so that the
// 16 lanes writing one token hit 16 different banks; groups of 8 stay contiguous.
__device__ __forceinline__ int kt_col(int d, int pos) { return pos ^ (8 * ((d >> 3) & 7)); }

// 2^x on the hardware exponential unit (flushes very negative x to zero).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over each row of 16 lanes, result in every lane of the row (DPP, no LDS traffic).
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
    return x;
}

// A copy of x the compiler cannot see through: lane-dependent addresses derived from
// it are recomputed inside the chunk loop instead of being hoisted out and spilled.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Orders LDS writes before later LDS reads of the same wave (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(NT) void prefill_chunked_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu_seqlens, int64_t eq_len, const float *__restrict__ S0,
    uint16_t *__restrict__ o, float *__restrict__ S_T, int HV, int DV, int rep, float scale) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    __bf16 *sK = reinterpret_cast<__bf16 *>(lds + OFF_K);
    __bf16 *sQ = reinterpret_cast<__bf16 *>(lds + OFF_Q);
    __bf16 *const sKt0 = reinterpret_cast<__bf16 *>(lds + OFF_KT);
    bf16x8 *opT = reinterpret_cast<bf16x8 *>(lds + OFF_OPT);  // [((b*2 + rt)*2 + hl)*64 + lane]
    bf16x8 *opA = reinterpret_cast<bf16x8 *>(lds + OFF_OPA);  // [(rt*2 + hl)*64 + lane]
    bf16x8 *opP = reinterpret_cast<bf16x8 *>(lds + OFF_OPP);  // [idx*64 + lane]
    float *const sc0 = reinterpret_cast<float *>(lds + OFF_SC);
    // Per-token scalars of chunk c live in buffer c % 2 (the next chunk's are written
    // while the current one is still being read):  G (cumulative log-decay times log2 e),
    // gamma = exp(G), r_k = 1/|k|, r_q = scale/|q|, beta, r_k exp(G_n - G).
#define GDN_SCALARS(c)                                         \
    float *sc_ = sc0 + ((c) & 1) * SC_SZ;                      \
    float *sG = sc_, *sGam = sc_ + C, *sRk = sc_ + 2 * C;      \
    float *sRq = sc_ + 3 * C, *sB = sc_ + 4 * C, *sDn = sc_ + 5 * C; \
    __bf16 *sKt = sKt0 + ((c) & 1) * DK * LT;                  \
    (void)sG; (void)sGam; (void)sRk; (void)sRq; (void)sB; (void)sDn; (void)sKt;

    const int unit = blockIdx.x;  // n * HV + h
    const int h = unit % HV;
    const int nseq = unit / HV;
    const int hq = h / rep;
    const int HQK = HV / rep;
    const int col0 = blockIdx.y * DVS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int lr = lane & 15;
    const int lq = lane >> 4;
    const bool colwave = w < 4;

    int64_t t0, t1;
    if (cu_seqlens) {
        t0 = cu_seqlens[nseq];
        t1 = cu_seqlens[nseq + 1];
    } else {
        t0 = (int64_t)nseq * eq_len;
        t1 = t0 + eq_len;
    }

    const int nchunks = (int)((t1 - t0 + C - 1) / C);
    auto chunk_len = [&](int c) { return (int)((t1 - t0 - (int64_t)c * C) < C ? (t1 - t0 - (int64_t)c * C) : C); };

    if (colwave) {
        // ====================== column waves: the table and the per-chunk chain ======
        // Element e of S[dt] is S[16 dt + 4 lq + e][col0 + 16 w + lr].
        f32x4 S[8];
        const size_t tab = (size_t)unit * DK * DV;
        const int mycol = col0 + 16 * w + lr;
        uint16_t *ost = reinterpret_cast<uint16_t *>(lds + OFF_OST) + w * 256;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[dt][e] = S0 ? S0[tab + (size_t)(16 * dt + 4 * lq + e) * DV + mycol] : 0.f;

        // v[16 rt + 4 lq + e][mycol] of the next chunk, fetched one chunk ahead
        uint16_t vreg[4][4];
        const size_t vrs = (size_t)HV * DV;  // token stride of v and o
        const uint16_t *vthr = v + (size_t)h * DV + mycol + (size_t)(4 * lq) * vrs;
        auto prefetch_v = [&](int c) {
            const int nn = chunk_len(c);
            const uint16_t *vc = vthr + (size_t)(t0 + (int64_t)c * C) * vrs;
            if (nn == C) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) vreg[rt][e] = vc[(size_t)(16 * rt + e) * vrs];
            } else {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        vreg[rt][e] = (16 * rt + 4 * lq + e < nn) ? vc[(size_t)(16 * rt + e) * vrs] : (uint16_t)0;
            }
        };
        // output stores: lane writes row lane/4 of a 16-row tile, columns 4 (lane % 4) .. +3
        uint16_t *othr = o + (size_t)h * DV + col0 + 16 * w + 4 * (lane & 3) + (size_t)(lane >> 2) * vrs;
        if (nchunks > 0) {
            prefetch_v(0);
            __syncthreads();  // (0) chunk 0's K, Q, K^T and scalars are in LDS
        }

        for (int c = 0; c < nchunks; ++c) {
            const int ln = opaque(lane);
            const int lrr = ln & 15, lqq = ln >> 4;
            const int64_t c0 = t0 + (int64_t)c * C;
            const int n = chunk_len(c);
            GDN_SCALARS(c)
            float vcur[4][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) vcur[rt][e] = bf16_to_f32(vreg[rt][e]);
            if (c + 1 < nchunks) prefetch_v(c + 1);

            // ---- Y = K S (hi + lo), Oacc = Q S (hi), Z = beta (v - gamma r_k Y)
            f32x4 Z[4], Oacc[4];
            {
                bf16x8 Sh[4], Sl[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) split(cat(S[2 * ks], S[2 * ks + 1]), Sh[ks], Sl[ks]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f}, oa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 kk = ld_std(sK, LK, 16 * rt, 32 * ks, ln);
                        const bf16x8 qq = ld_std(sQ, LK, 16 * rt, 32 * ks, ln);
                        y = mfma32(kk, Sh[ks], y);
                        y = mfma32(kk, Sl[ks], y);
                        oa = mfma32(qq, Sh[ks], oa);
                    }
                    const int i0 = 16 * rt + 4 * lqq;
                    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(sB + i0);
                    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sGam + i0);
                    const f32x4 k4 = *reinterpret_cast<const f32x4 *>(sRk + i0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Z[rt][e] = b4[e] * (vcur[rt][e] - g4[e] * k4[e] * y[e]);
                    Oacc[rt] = oa;
                }
            }
            __syncthreads();  // (A) P, -A_10, T_0, T_1 and r_k exp(G_n - G) of chunk c are in LDS

            // ---- Delta_0 = T_0 Z_0;  Delta_1 = T_1 (Z_1 - A_10 Delta_0)
            f32x4 Dl[4];
            {
                bf16x8 zh, zl;
                split(cat(Z[0], Z[1]), zh, zl);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    Dl[rt] = mfma32_x3(opT[(rt * 2 + 0) * 64 + ln], opT[(rt * 2 + 1) * 64 + ln], zh, zl, zero);
                }
                bf16x8 dh, dl;
                split(cat(Dl[0], Dl[1]), dh, dl);
                f32x4 r1[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    r1[rt] = mfma32_x3(opA[(rt * 2 + 0) * 64 + ln], opA[(rt * 2 + 1) * 64 + ln], dh, dl, Z[2 + rt]);
                bf16x8 rh, rl;
                split(cat(r1[0], r1[1]), rh, rl);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    Dl[2 + rt] = mfma32_x3(opT[((2 + rt) * 2 + 0) * 64 + ln], opT[((2 + rt) * 2 + 1) * 64 + ln],
                                           rh, rl, zero);
                }
            }
            // ---- O = gamma r_q (Q S) + P Delta
            {
                bf16x8 Dsg[2];
                Dsg[0] = to_bf16(cat(Dl[0], Dl[1]));
                Dsg[1] = to_bf16(cat(Dl[2], Dl[3]));
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 pd = {0.f, 0.f, 0.f, 0.f};
                    const int base = rt == 0 ? 0 : (rt == 1 ? 1 : (rt == 2 ? 2 : 4));
#pragma unroll
                    for (int ks = 0; ks <= (rt >> 1); ++ks) pd = mfma32(opP[(base + ks) * 64 + ln], Dsg[ks], pd);
                    const int i0 = 16 * rt + 4 * lqq;
                    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sGam + i0);
                    const f32x4 q4 = *reinterpret_cast<const f32x4 *>(sRq + i0);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ost[(4 * lqq + e) * 16 + lrr] = __builtin_bit_cast(uint16_t, (__bf16)(g4[e] * q4[e] * Oacc[rt][e] + pd[e]));
                    wave_lds_sync();
                    {
                        const int r = ln >> 2, cq = ln & 3;
                        const uint2 val = *reinterpret_cast<const uint2 *>(ost + r * 16 + 4 * cq);
                        if (16 * rt + r < n)
                            *reinterpret_cast<uint2 *>(othr + (size_t)(c0 + 16 * rt) * vrs) = val;
                    }
                    wave_lds_sync();
                }
            }
            // ---- S <- gamma_n S + K^T D,  D = diag(r_k exp(G_n - G)) Delta
            {
                bf16x8 Dh[2], Dlo[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    f32x8 x = cat(Dl[2 * ks], Dl[2 * ks + 1]);
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sDn + 32 * ks + 16 * t + 4 * lqq);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[4 * t + e] *= d4[e];
                    }
                    split(x, Dh[ks], Dlo[ks]);
                }
                const float gam_n = sGam[C - 1];
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    f32x4 acc = S[dt] * gam_n;
                    const int d = 16 * dt + lrr;
                    const __bf16 *rowp = sKt + d * LT;
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const bf16x8 kt = *reinterpret_cast<const bf16x8 *>(rowp + kt_col(d, 32 * ks + 8 * lqq));
                        acc = mfma32(kt, Dh[ks], acc);
                        acc = mfma32(kt, Dlo[ks], acc);
                    }
                    S[dt] = acc;
                }
            }
            __syncthreads();  // (B) chunk c+1's K, Q, K^T and scalars are in LDS
        }
        if (S_T) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) S_T[tab + (size_t)(16 * dt + 4 * lq + e) * DV + mycol] = S[dt][e];
        }
        return;
    }

    // ====================== Gram waves: chunk staging, norms, decay, P, A, T =====
    const int gt = tid - 256;  // 0..255
    const int gw = w - 4;      // 0..3
    // Staging: item gt + 256 p (p = 0, 1) is the token pair (2 pr, 2 pr + 1), pr = gt/16 + 16 p,
    // times the 16-byte segment s = gt % 16 of their q and k rows (d = 8 s .. 8 s + 7).
    const int seg_s = gt & 15;
    uint4 kreg[2][2], qreg[2][2];  // [p][token of the pair]
    float greg = 0.f, breg = 0.f;  // Gram wave 3: token = lane
    const size_t rs = (size_t)HQK * DK;  // token stride of q and k
    const size_t thr_off = (size_t)hq * DK + 8 * seg_s + (size_t)(2 * (gt >> 4)) * rs;
    const uint16_t *kthr = k + thr_off;
    const uint16_t *qthr = q + thr_off;
    auto prefetch_qk = [&](int c) {
        const int nn = chunk_len(c);
        const int64_t cs = t0 + (int64_t)c * C;
        const uint16_t *kc = kthr + (size_t)cs * rs;
        const uint16_t *qc = qthr + (size_t)cs * rs;
        if (nn == C) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    kreg[p][u] = *reinterpret_cast<const uint4 *>(kc + (size_t)(32 * p + u) * rs);
                    qreg[p][u] = *reinterpret_cast<const uint4 *>(qc + (size_t)(32 * p + u) * rs);
                }
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int r = 2 * ((gt >> 4) + 16 * p) + u;
                    kreg[p][u] = make_uint4(0, 0, 0, 0);
                    qreg[p][u] = make_uint4(0, 0, 0, 0);
                    if (r < nn) {
                        kreg[p][u] = *reinterpret_cast<const uint4 *>(kc + (size_t)(32 * p + u) * rs);
                        qreg[p][u] = *reinterpret_cast<const uint4 *>(qc + (size_t)(32 * p + u) * rs);
                    }
                }
        }
        if (gw == 3) {
            const bool ok = lane < nn;
            greg = ok ? g[(size_t)(cs + lane) * HV + h] : 0.f;
            breg = ok ? beta[(size_t)(cs + lane) * HV + h] : 0.f;
        }
    };
    if (nchunks > 0) prefetch_qk(0);

    // chunk c's q, k, g, beta (already in registers) -> LDS, norms, cumulative decay
    auto stage_chunk = [&](int c) {
        GDN_SCALARS(c)
        const int ln = opaque(lane);
        const int gtt = opaque(gt);
        const int sgs = gtt & 15;
        // segment sgs (d = 8 sgs .. +7) sits at two runs of 4 in tile order
        const int p0 = 32 * (sgs >> 2) + 16 * (sgs & 1) + 4 * ((sgs >> 1) & 1);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int pr = (gtt >> 4) + 16 * p;
            float sk[2], sq[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = 2 * pr + u;
                const uint4 kv = kreg[p][u], qv = qreg[p][u];
                *reinterpret_cast<uint2 *>(sK + r * LK + p0) = make_uint2(kv.x, kv.y);
                *reinterpret_cast<uint2 *>(sK + r * LK + p0 + 8) = make_uint2(kv.z, kv.w);
                *reinterpret_cast<uint2 *>(sQ + r * LK + p0) = make_uint2(qv.x, qv.y);
                *reinterpret_cast<uint2 *>(sQ + r * LK + p0 + 8) = make_uint2(qv.z, qv.w);
                const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
                const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                float a = 0.f, bq = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xffff0000u);
                    const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xffff0000u);
                    a += k0 * k0 + k1 * k1;
                    bq += q0 * q0 + q1 * q1;
                }
                sk[u] = a;
                sq[u] = bq;
            }
            // K^T: both tokens of the pair are adjacent in tile order -> one 4-byte write per d
            const int tp = tile_pos(2 * pr);
            const uint32_t k0w[4] = {kreg[p][0].x, kreg[p][0].y, kreg[p][0].z, kreg[p][0].w};
            const uint32_t k1w[4] = {kreg[p][1].x, kreg[p][1].y, kreg[p][1].z, kreg[p][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 8 * sgs + e;
                const uint32_t lo = (e & 1) ? (k0w[e >> 1] >> 16) : (k0w[e >> 1] & 0xffffu);
                const uint32_t hi = (e & 1) ? (k1w[e >> 1] & 0xffff0000u) : (k1w[e >> 1] << 16);
                *reinterpret_cast<uint32_t *>(sKt + d * LT + kt_col(d, tp)) = lo | hi;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                sk[u] = row16_sum(sk[u]);
                sq[u] = row16_sum(sq[u]);
            }
            if (sgs == 0) {
                sRk[2 * pr] = inv_norm(sk[0]);
                sRk[2 * pr + 1] = inv_norm(sk[1]);
                sRq[2 * pr] = inv_norm(sq[0]) * scale;
                sRq[2 * pr + 1] = inv_norm(sq[1]) * scale;
            }
        }
        if (gw == 3) {
            float x = greg * 1.44269504088896341f;  // log2(e)
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (ln >= off) x += y;
            }
            sG[ln] = x;
            sGam[ln] = exp2_hw(x);
            sB[ln] = breg;
        }
    };

    if (nchunks > 0) {
        stage_chunk(0);
        if (nchunks > 1) prefetch_qk(1);
        __syncthreads();  // (0)
    }
    for (int c = 0; c < nchunks; ++c) {
        const int ln = opaque(lane);
        const int lrr = ln & 15, lqq = ln >> 4;
        GDN_SCALARS(c)

        if (gw < 2) {
            // ---- T_b = (I + A_bb)^{-1} for the 32-token block b = gw
            const int b = gw;
            float *Af = reinterpret_cast<float *>(lds + OFF_WP + b * WP_SZ);
            float *Tf = Af + 32 * LW;
            float *Rf = Tf + 32 * LW;
            bf16x8 ka[4], kb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                ka[ks] = ld_std(sK, LK, 32 * b, 32 * ks, ln);
                kb[ks] = ld_std(sK, LK, 32 * b + 16, 32 * ks, ln);
            }
            f32x4 g00 = {0.f, 0.f, 0.f, 0.f}, g10 = g00, g11 = g00;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                g00 = mfma32(ka[ks], ka[ks], g00);
                g10 = mfma32(kb[ks], ka[ks], g10);
                g11 = mfma32(kb[ks], kb[ks], g11);
            }
            // A values of local tile (li, lj): element e at local (16 li + 4 lq + e, 16 lj + lr)
            auto put_a = [&](const f32x4 &acc, int li, int lj) {
                const int j = 32 * b + 16 * lj + lrr;
                const float Gj = sG[j], rkj = sRk[j];
                const int i0 = 32 * b + 16 * li + 4 * lqq;
                const f32x4 G4 = *reinterpret_cast<const f32x4 *>(sG + i0);
                const f32x4 B4 = *reinterpret_cast<const f32x4 *>(sB + i0);
                const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + i0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = (j < i0 + e) ? B4[e] * R4[e] * rkj * acc[e] * exp2_hw(G4[e] - Gj) : 0.f;
                    Af[(16 * li + 4 * lqq + e) * LW + 16 * lj + lrr] = a;
                }
            };
            put_a(g00, 0, 0);
            put_a(g10, 1, 0);
            put_a(g11, 1, 1);
            wave_lds_sync();
            // 16x16 diagonal inverses by forward substitution, one column per lane
            // (lane = (block, column cc)); row i of A is read as four 16-byte broadcasts.
            {
                const int blk = (ln >> 4) & 1, cc = ln & 15;
                const float *Ab = Af + (16 * blk) * LW + 16 * blk;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = (i == cc) ? 1.f : 0.f;
#pragma unroll
                for (int i = 1; i < 16; ++i) {
                    const f32x4 *row = reinterpret_cast<const f32x4 *>(Ab + i * LW);
                    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        if (4 * q4 >= i) break;
                        const f32x4 a4 = row[q4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * q4 + e < i) part[e] += a4[e] * x[4 * q4 + e];
                    }
                    const float sum = (part[0] + part[1]) + (part[2] + part[3]);
                    if (i > cc) x[i] = -sum;
                }
                if (ln < 32) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) Tf[(16 * blk + i) * LW + 16 * blk + cc] = x[i];
                } else {
                    // the upper 16x16 block of T_b is zero
#pragma unroll
                    for (int i = 0; i < 8; ++i) Tf[(8 * ((ln - 32) >> 4) + i) * LW + 16 + (ln & 15)] = 0.f;
                }
            }
            wave_lds_sync();
            // merge: T_10 = -T_11 (A_10 T_00), fp32 MFMA
            {
                f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    r = mfma_f32(Af[(16 + lrr) * LW + 4 * kk + lqq], Tf[(4 * kk + lqq) * LW + lrr], r);
#pragma unroll
                for (int e = 0; e < 4; ++e) Rf[(4 * lqq + e) * 17 + lrr] = r[e];
                wave_lds_sync();
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    t = mfma_f32(Tf[(16 + lrr) * LW + 16 + 4 * kk + lqq], Rf[(4 * kk + lqq) * 17 + lrr], t);
#pragma unroll
                for (int e = 0; e < 4; ++e) Tf[(16 + 4 * lqq + e) * LW + lrr] = -t[e];
            }
            wave_lds_sync();
            // T_b -> tile-order operands (hi, lo) for row tiles rt = 0, 1
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const f32x4 *row = reinterpret_cast<const f32x4 *>(Tf + (16 * rt + lrr) * LW + 4 * lqq);
                const f32x4 x0 = row[0], x1 = row[4];
                bf16x8 hi, lo;
                split(cat(x0, x1), hi, lo);
                opT[((2 * b + rt) * 2 + 0) * 64 + ln] = hi;
                opT[((2 * b + rt) * 2 + 1) * 64 + ln] = lo;
            }
        } else {
            // K blocks as the first (role-swapped) operand of every tile below
            bf16x8 kk[4][4];
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kk[blk][ks] = ld_std(sK, LK, 16 * blk, 32 * ks, ln);
            // P operand idx = (rt, ks), ks <= rt / 2:  0 (0,0) 1 (1,0) 2 (2,0) 3 (2,1) 4 (3,0) 5 (3,1).
            // Tile (rt, kt) from MFMA(K block kt, Q block rt): element e at lane is
            // (Q K^T)[16 rt + lr][16 kt + 4 lq + e], the tile-order operand slot.
            auto p_operand = [&](int idx, const bf16x8 *qq) {
                const int rt = idx == 0 ? 0 : (idx == 1 ? 1 : (idx < 4 ? 2 : 3));
                const int ks = (idx == 3 || idx == 5) ? 1 : 0;
                const int i = 16 * rt + lrr;
                const float ci = sRq[i], Gi = sG[i];
                f32x8 x;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int kt = 2 * ks + t;
                    if (kt > rt) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[4 * t + e] = 0.f;
                        continue;
                    }
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kq = 0; kq < 4; ++kq) acc = mfma32(kk[kt][kq], qq[kq], acc);
                    const int j0 = 16 * kt + 4 * lqq;
                    const f32x4 G4 = *reinterpret_cast<const f32x4 *>(sG + j0);
                    const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + j0);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[4 * t + e] = (j0 + e <= i) ? ci * R4[e] * acc[e] * exp2_hw(Gi - G4[e]) : 0.f;
                }
                opP[idx * 64 + ln] = to_bf16(x);
            };
            bf16x8 qq[4];
            auto load_q = [&](int rt) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) qq[ks] = ld_std(sQ, LK, 16 * rt, 32 * ks, ln);
            };
            if (gw == 2) {
                // -A_10 (rows 32..63, columns 0..31) in tile order, from role-swapped Gram tiles
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int i = 32 + 16 * rt + lrr;
                    const float ci = sB[i] * sRk[i], Gi = sG[i];
                    f32x8 x;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) acc = mfma32(kk[t][ks], kk[2 + rt][ks], acc);
                        const int j0 = 16 * t + 4 * lqq;
                        const f32x4 G4 = *reinterpret_cast<const f32x4 *>(sG + j0);
                        const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + j0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[4 * t + e] = -ci * R4[e] * acc[e] * exp2_hw(Gi - G4[e]);
                    }
                    bf16x8 hi, lo;
                    split(x, hi, lo);
                    opA[(rt * 2 + 0) * 64 + ln] = hi;
                    opA[(rt * 2 + 1) * 64 + ln] = lo;
                }
                sDn[ln] = sRk[ln] * exp2_hw(sG[C - 1] - sG[ln]);
                load_q(0);
                p_operand(0, qq);
                load_q(1);
                p_operand(1, qq);
                load_q(2);
                p_operand(2, qq);
            } else {
                load_q(2);
                p_operand(3, qq);
                load_q(3);
                p_operand(4, qq);
                p_operand(5, qq);
            }
        }
        __syncthreads();  // (A)
        if (c + 1 < nchunks) {
            stage_chunk(c + 1);
            if (c + 2 < nchunks) prefetch_qk(c + 2);
        }
        __syncthreads();  // (B)
    }
}

}  // namespace

bool prefill_chunked_supported(int dk, int dv, bool bf16) { return bf16 && dk == DK && dv % DVS == 0; }

hipError_t launch_prefill_chunked(const PrefillArgs &a, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    const int rep = a.HV / a.HQK;
    dim3 grid((unsigned)((int64_t)a.N * a.HV), (unsigned)(a.dv / DVS));
    hipLaunchKernelGGL(prefill_chunked_kernel, grid, dim3(NT), 0, stream, static_cast<const uint16_t *>(a.q),
                       static_cast<const uint16_t *>(a.k), static_cast<const uint16_t *>(a.v), a.g, a.beta,
                       a.cu_seqlens, a.eq_len, a.S0, static_cast<uint16_t *>(a.o), a.S_T, a.HV, a.dv, rep,
                       a.scale);
    return hipGetLastError();
}

}  // namespace gdn
