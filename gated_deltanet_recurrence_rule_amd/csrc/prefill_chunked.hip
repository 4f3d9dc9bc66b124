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
//   A_ij = b_i r_k,i r_k,j (K K^T)_ij exp(G_i - G_j)   j < i   (zero otherwise)
//   P_ij = r_q,i r_k,j (Q K^T)_ij exp(G_i - G_j)       j <= i
//   T    = (I + A)^{-1}                                 (unit lower triangular)
//   Z_i  = b_i (v_i - gamma_i r_k,i (K S)_i)
//   Delta = T Z
//   O_i  = gamma_i r_q,i (Q S)_i + (P Delta)_i
//   S'   = gamma_n S + K^T diag(r_k,i exp(G_n - G_i)) Delta
//
// Only exp(G_i - G_j) <= 1 and exp(G_n - G_i) <= 1 are formed, never 1/gamma.
//
// Precision.  MFMA operands are bf16; a value that is not exactly bf16 is
// either rounded once or carried as hi + lo (hi = bf16(x), lo = bf16(x - hi),
// two or three MFMAs).  The raw q, k, v rows are exact bf16.  The table path is
// carried hi + lo: S in K S, T and Z in T Z, and the scaled Delta in K^T D.
// The output path rounds once: S in Q S, P and Delta in P Delta.  All
// accumulation is fp32; T is built in fp32.
//
// Mapping.  One workgroup of 4 waves owns one (sequence, V head, 64-column
// slice of dv) and walks its chunks in order, keeping its 128 x 64 slice of S
// in MFMA accumulators (wave w holds table rows 32w..32w+31).  dv columns of S
// evolve independently, so slices need no communication; each slice recomputes
// its chunk's Gram matrices and T.  Everything else of a chunk lives in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int C = 64;       // chunk length
constexpr int DK = 128;     // key dimension
constexpr int DVS = 64;     // dv columns per workgroup
constexpr int NT = 256;     // threads (4 waves)

// LDS row strides (elements), padded so 16 lanes reading 16 rows hit distinct banks.
constexpr int LK = DK + 8;  // rows of K, Q, S^T (bf16)
constexpr int LC = C + 8;   // rows of K^T, P, T, Z^T, D^T, Delta^T, V (bf16)
constexpr int LF = C + 4;   // rows of A and T in fp32

// LDS regions (bytes).  Regions are reused by phases that do not overlap in time.
constexpr int R1 = 0;                              // K [C][LK] | merge scratch | Delta^T [DVS][LC]
constexpr int R1_SZ = C * LK * 2;
constexpr int R2 = R1 + R1_SZ;                     // Q [C][LK] | T fp32 [C][LF] | D^T hi,lo [DVS][LC]
constexpr int R2_SZ = 2 * DVS * LC * 2;
constexpr int R3 = R2 + R2_SZ;                     // K^T [DK][LC]
constexpr int R3_SZ = DK * LC * 2;
constexpr int R4 = R3 + R3_SZ;                     // S^T hi, lo [DVS][LK]
constexpr int R4_SZ = 2 * DVS * LK * 2;
constexpr int R5 = R4 + R4_SZ;                     // P [C][LC]
constexpr int R5_SZ = C * LC * 2;
constexpr int R6 = R5 + R5_SZ;                     // T hi, lo [C][LC]
constexpr int R6_SZ = 2 * C * LC * 2;
constexpr int R7 = R6 + R6_SZ;                     // A fp32 [C][LF] | Z^T hi, lo [DVS][LC]
constexpr int R7_SZ = 2 * DVS * LC * 2;
constexpr int R8 = R7 + R7_SZ;                     // V [C][LC] (DVS columns)
constexpr int R8_SZ = C * LC * 2;
constexpr int R9 = R8 + R8_SZ;                     // per-token scalars, 6 x C floats
constexpr int R9_SZ = 6 * C * 4;
constexpr int LDS_BYTES = R9 + R9_SZ;

static_assert(C * LK * 2 >= 32 * 36 * 4, "merge scratch fits in R1");
static_assert(R2_SZ >= C * LK * 2 && R2_SZ >= C * LF * 4, "R2 holds Q and fp32 T");
static_assert(R7_SZ >= C * LF * 4, "R7 holds fp32 A");
static_assert(R1_SZ >= DVS * LC * 2, "R1 holds Delta^T");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// MFMA 16x16x32 operand: lane l reads row r0 + l%16, elements k0 + 8(l/16) .. +7 of a
// bf16 matrix stored with k contiguous (A row-major, or B stored as B^T row-major).
__device__ __forceinline__ bf16x8 ld_op(const uint16_t *base, int stride, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(base + (r0 + (lane & 15)) * stride + k0 + 8 * (lane >> 4));
}

__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
    hi = f32_to_bf16(x);
    lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// 16x16 fp32 product X * Y (+acc) with X, Y row-major fp32 blocks in LDS.
__device__ __forceinline__ f32x4 mm16_f32(const float *X, int ldx, const float *Y, int ldy, f32x4 acc,
                                          int lane) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = X[(lane & 15) * ldx + 4 * k + (lane >> 4)];
        const float b = Y[(4 * k + (lane >> 4)) * ldy + (lane & 15)];
        acc = mfma_f32(a, b, acc);
    }
    return acc;
}

// Store a 16x16 fp32 accumulator tile (scaled) to a row-major fp32 block.
__device__ __forceinline__ void st_tile_f32(float *Y, int ldy, f32x4 acc, float s, int lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Y[(4 * (lane >> 4) + e) * ldy + (lane & 15)] = s * acc[e];
}

template <typename T>
__global__ __launch_bounds__(NT) void prefill_chunked_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu_seqlens, int64_t eq_len, const float *__restrict__ S0,
    uint16_t *__restrict__ o, float *__restrict__ S_T, int HV, int DV, int rep, float scale) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    uint16_t *sK = reinterpret_cast<uint16_t *>(lds + R1);
    float *sScr = reinterpret_cast<float *>(lds + R1);
    uint16_t *sDelt = reinterpret_cast<uint16_t *>(lds + R1);
    uint16_t *sQ = reinterpret_cast<uint16_t *>(lds + R2);
    float *sTf = reinterpret_cast<float *>(lds + R2);
    uint16_t *sDt_hi = reinterpret_cast<uint16_t *>(lds + R2);
    uint16_t *sDt_lo = sDt_hi + DVS * LC;
    uint16_t *sKt = reinterpret_cast<uint16_t *>(lds + R3);
    uint16_t *sSt_hi = reinterpret_cast<uint16_t *>(lds + R4);
    uint16_t *sSt_lo = sSt_hi + DVS * LK;
    uint16_t *sP = reinterpret_cast<uint16_t *>(lds + R5);
    uint16_t *sT_hi = reinterpret_cast<uint16_t *>(lds + R6);
    uint16_t *sT_lo = sT_hi + C * LC;
    float *sA = reinterpret_cast<float *>(lds + R7);
    uint16_t *sZt_hi = reinterpret_cast<uint16_t *>(lds + R7);
    uint16_t *sZt_lo = sZt_hi + DVS * LC;
    uint16_t *sV = reinterpret_cast<uint16_t *>(lds + R8);
    float *sG = reinterpret_cast<float *>(lds + R9);  // cumulative log-decay
    float *sGam = sG + C;                             // exp(G_i)
    float *sRk = sGam + C;                            // 1 / |k_i|
    float *sRq = sRk + C;                             // scale / |q_i|
    float *sB = sRq + C;                              // beta_i
    float *sDn = sB + C;                              // r_k,i exp(G_n - G_i)

    const int unit = blockIdx.x;  // n * HV + h
    const int h = unit % HV;
    const int nseq = unit / HV;
    const int hq = h / rep;
    const int HQK = HV / rep;
    const int col0 = blockIdx.y * DVS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int lr = lane & 15;   // accumulator column within a tile
    const int lq = lane >> 4;   // accumulator row group within a tile

    int64_t t0, t1;
    if (cu_seqlens) {
        t0 = cu_seqlens[nseq];
        t1 = cu_seqlens[nseq + 1];
    } else {
        t0 = (int64_t)nseq * eq_len;
        t1 = t0 + eq_len;
    }

    // Table slice in accumulators: wave w owns rows 32w..32w+31 as two 16-row tiles
    // (dt = 0, 1) times four 16-column tiles (ct).  Element e of tile (dt, ct) is
    // S[32w + 16dt + 4lq + e][col0 + 16ct + lr].
    f32x4 S[2][4];
    const size_t tab = (size_t)unit * DK * DV;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 32 * w + 16 * dt + 4 * lq + e;
                S[dt][ct][e] = S0 ? S0[tab + (size_t)d * DV + col0 + 16 * ct + lr] : 0.f;
            }

    auto write_St = [&]() {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                uint16_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) split_bf16(S[dt][ct][e], hi[e], lo[e]);
                const int off = (16 * ct + lr) * LK + 32 * w + 16 * dt + 4 * lq;
                *reinterpret_cast<uint2 *>(sSt_hi + off) =
                    make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
                *reinterpret_cast<uint2 *>(sSt_lo + off) =
                    make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
            }
    };
    write_St();

    for (int64_t c0 = t0; c0 < t1; c0 += C) {
        const int n = (int)((t1 - c0) < C ? (t1 - c0) : C);
        __syncthreads();  // the previous chunk is done with every LDS region

        // ---- S1: load the chunk's K, Q (row-major and K^T), V slice, g, beta
#pragma unroll
        for (int p = 0; p < (C * DK / 8) / NT; ++p) {
            const int seg = tid + NT * p;
            const int r = seg / (DK / 8), s = seg % (DK / 8);
            uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
            if (r < n) {
                const size_t off = ((size_t)(c0 + r) * HQK + hq) * DK + 8 * s;
                kv = *reinterpret_cast<const uint4 *>(k + off);
                qv = *reinterpret_cast<const uint4 *>(q + off);
            }
            *reinterpret_cast<uint4 *>(sK + r * LK + 8 * s) = kv;
            *reinterpret_cast<uint4 *>(sQ + r * LK + 8 * s) = qv;
            const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sKt[(8 * s + e) * LC + r] = (uint16_t)(kw[e >> 1] >> (16 * (e & 1)));
        }
#pragma unroll
        for (int p = 0; p < (C * DVS / 8) / NT; ++p) {
            const int seg = tid + NT * p;
            const int r = seg / (DVS / 8), s = seg % (DVS / 8);
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (r < n) vv = *reinterpret_cast<const uint4 *>(v + ((size_t)(c0 + r) * HV + h) * DV + col0 + 8 * s);
            *reinterpret_cast<uint4 *>(sV + r * LC + 8 * s) = vv;
        }
        if (tid < C) {
            const bool ok = tid < n;
            sG[tid] = ok ? g[(size_t)(c0 + tid) * HV + h] : 0.f;
            sB[tid] = ok ? beta[(size_t)(c0 + tid) * HV + h] : 0.f;
        }
        __syncthreads();

        // ---- S2: cumulative log-decay (wave 0) and the norms of q and k (all)
        if (w == 0) {
            float x = sG[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            sG[lane] = x;
            sGam[lane] = expf(x);
        }
        {
            const int r = tid >> 2, part = tid & 3;
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < DK / 4; ++e) {
                const float kx = bf16_to_f32(sK[r * LK + part * (DK / 4) + e]);
                const float qx = bf16_to_f32(sQ[r * LK + part * (DK / 4) + e]);
                sk += kx * kx;
                sq += qx * qx;
            }
            sk += __shfl_xor(sk, 1, 64);
            sk += __shfl_xor(sk, 2, 64);
            sq += __shfl_xor(sq, 1, 64);
            sq += __shfl_xor(sq, 2, 64);
            if (part == 0) {
                sRk[r] = inv_norm(sk);
                sRq[r] = inv_norm(sq) * scale;
            }
        }
        __syncthreads();

        // ---- S3: Gram tiles -> A (fp32), P (bf16); Y = K S (hi+lo); Oacc = Q S (hi)
        // 20 lower-triangular tile jobs: j < 10 are K K^T tiles, j >= 10 are Q K^T tiles.
        for (int job = w; job < 20; job += 4) {
            const bool isA = job < 10;
            int tt = isA ? job : job - 10;
            int ti = 0;
            while (tt > ti) { tt -= ti + 1; ++ti; }
            const int tj = tt;  // ti >= tj
            const uint16_t *X = isA ? sK : sQ;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks)
                acc = mfma_bf16(ld_op(X, LK, 16 * ti, 32 * ks, lane), ld_op(sK, LK, 16 * tj, 32 * ks, lane), acc);
            const int j = 16 * tj + lr;
            const float Gj = sG[j], rkj = sRk[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ti + 4 * lq + e;
                const float dec = expf(sG[i] - Gj);
                if (isA) {
                    sA[i * LF + j] = (j < i) ? sB[i] * sRk[i] * rkj * acc[e] * dec : 0.f;
                } else {
                    sP[i * LC + j] = f32_to_bf16((j <= i) ? sRq[i] * rkj * acc[e] * dec : 0.f);
                }
            }
        }
        // zero the strictly-upper tiles of P (read by the P Delta product's diagonal k-steps)
        for (int idx = tid; idx < 6 * 256; idx += NT) {
            const int tile = idx >> 8, el = idx & 255;
            const int ti = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
            const int tj = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
            sP[(16 * ti + (el >> 4)) * LC + 16 * tj + (el & 15)] = 0;
        }
        f32x4 Y[4], Oacc[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 y = {0.f, 0.f, 0.f, 0.f}, oa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const bf16x8 kk = ld_op(sK, LK, 16 * w, 32 * ks, lane);
                const bf16x8 qq = ld_op(sQ, LK, 16 * w, 32 * ks, lane);
                const bf16x8 shi = ld_op(sSt_hi, LK, 16 * ct, 32 * ks, lane);
                const bf16x8 slo = ld_op(sSt_lo, LK, 16 * ct, 32 * ks, lane);
                y = mfma_bf16(kk, shi, y);
                y = mfma_bf16(kk, slo, y);
                oa = mfma_bf16(qq, shi, oa);
            }
            Y[ct] = y;
            Oacc[ct] = oa;
        }
        __syncthreads();

        // ---- S4: T = (I + A)^{-1} in fp32.  (a) the four 16x16 diagonal blocks by
        // forward substitution, one column per lane of wave 0.
        if (w == 0) {
            const int b = lane >> 4, c = lane & 15;
            const float *Ab = sA + (16 * b) * LF + 16 * b;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) acc += Ab[i * LF + j] * x[j];
                if (i > c) x[i] = -acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sTf[(16 * b + i) * LF + 16 * b + c] = x[i];
        }
        // zero the strictly-upper blocks of T
        for (int idx = tid; idx < 6 * 256; idx += NT) {
            const int tile = idx >> 8, el = idx & 255;
            const int ti = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
            const int tj = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
            sTf[(16 * ti + (el >> 4)) * LF + 16 * tj + (el & 15)] = 0.f;
        }
        __syncthreads();
        // (b) pairs: T_10 = -T_11 A_10 T_00 (wave 0), T_32 = -T_33 A_32 T_22 (wave 1)
        constexpr int LS = 36;  // scratch row stride (fp32)
        if (w < 2) {
            const int b0 = 2 * w;  // blocks (b0+1, b0)
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
            r = mm16_f32(sA + (16 * (b0 + 1)) * LF + 16 * b0, LF, sTf + (16 * b0) * LF + 16 * b0, LF, r, lane);
            st_tile_f32(sScr + 16 * w, LS, r, 1.f, lane);
        }
        __syncthreads();
        if (w < 2) {
            const int b0 = 2 * w;
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
            r = mm16_f32(sTf + (16 * (b0 + 1)) * LF + 16 * (b0 + 1), LF, sScr + 16 * w, LS, r, lane);
            st_tile_f32(sTf + (16 * (b0 + 1)) * LF + 16 * b0, LF, r, -1.f, lane);
        }
        __syncthreads();
        // (c) halves: T[32:64, 0:32] = -T[32:64, 32:64] (A[32:64, 0:32] T[0:32, 0:32]);
        // wave w computes the 16x16 output tile (w / 2, w % 2) of each product.
        {
            const int ri = w >> 1, cj = w & 1;
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                r = mm16_f32(sA + (32 + 16 * ri) * LF + 16 * kb, LF, sTf + (16 * kb) * LF + 16 * cj, LF, r, lane);
            st_tile_f32(sScr + (16 * ri) * LS + 16 * cj, LS, r, 1.f, lane);
        }
        __syncthreads();
        {
            const int ri = w >> 1, cj = w & 1;
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                r = mm16_f32(sTf + (32 + 16 * ri) * LF + 32 + 16 * kb, LF, sScr + (16 * kb) * LS + 16 * cj, LS, r,
                             lane);
            st_tile_f32(sTf + (32 + 16 * ri) * LF + 16 * cj, LF, r, -1.f, lane);
        }
        __syncthreads();
        // (d) T -> hi + lo bf16; Z = beta (V - gamma r_k Y) -> Z^T hi + lo (A is dead now)
        for (int idx = tid; idx < C * C; idx += NT) {
            const int i = idx >> 6, j = idx & 63;
            uint16_t hi, lo;
            split_bf16(sTf[i * LF + j], hi, lo);
            sT_hi[i * LC + j] = hi;
            sT_lo[i * LC + j] = lo;
        }
        __syncthreads();  // sA (aliased by Z^T) and sTf are fully read
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            uint16_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * w + 4 * lq + e;
                const float vv = bf16_to_f32(sV[i * LC + 16 * ct + lr]);
                const float z = sB[i] * (vv - sGam[i] * sRk[i] * Y[ct][e]);
                split_bf16(z, hi[e], lo[e]);
            }
            const int off = (16 * ct + lr) * LC + 16 * w + 4 * lq;
            *reinterpret_cast<uint2 *>(sZt_hi + off) =
                make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
            *reinterpret_cast<uint2 *>(sZt_lo + off) =
                make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
        }
        if (tid < C) sDn[tid] = sRk[tid] * expf(sG[C - 1] - sG[tid]);
        __syncthreads();

        // ---- S6: Delta = T Z (three passes); D = diag(r_k exp(G_n - G)) Delta
        const int nks = (w >> 1) + 1;  // 32-token k-steps needed by row tile w (T is lower triangular)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 dl = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < nks; ++ks) {
                const bf16x8 th = ld_op(sT_hi, LC, 16 * w, 32 * ks, lane);
                const bf16x8 tl = ld_op(sT_lo, LC, 16 * w, 32 * ks, lane);
                const bf16x8 zh = ld_op(sZt_hi, LC, 16 * ct, 32 * ks, lane);
                const bf16x8 zl = ld_op(sZt_lo, LC, 16 * ct, 32 * ks, lane);
                dl = mfma_bf16(th, zh, dl);
                dl = mfma_bf16(th, zl, dl);
                dl = mfma_bf16(tl, zh, dl);
            }
            uint16_t dh[4], dlo[4], dsg[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * w + 4 * lq + e;
                dsg[e] = f32_to_bf16(dl[e]);
                split_bf16(sDn[i] * dl[e], dh[e], dlo[e]);
            }
            const int off = (16 * ct + lr) * LC + 16 * w + 4 * lq;
            *reinterpret_cast<uint2 *>(sDelt + off) =
                make_uint2(dsg[0] | ((uint32_t)dsg[1] << 16), dsg[2] | ((uint32_t)dsg[3] << 16));
            *reinterpret_cast<uint2 *>(sDt_hi + off) =
                make_uint2(dh[0] | ((uint32_t)dh[1] << 16), dh[2] | ((uint32_t)dh[3] << 16));
            *reinterpret_cast<uint2 *>(sDt_lo + off) =
                make_uint2(dlo[0] | ((uint32_t)dlo[1] << 16), dlo[2] | ((uint32_t)dlo[3] << 16));
        }
        __syncthreads();

        // ---- S7: O = gamma r_q (Q S) + P Delta -> global; S <- gamma_n S + K^T D
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 pd = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks < nks; ++ks)
                pd = mfma_bf16(ld_op(sP, LC, 16 * w, 32 * ks, lane), ld_op(sDelt, LC, 16 * ct, 32 * ks, lane), pd);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * w + 4 * lq + e;
                if (i < n) {
                    const float ov = sGam[i] * sRq[i] * Oacc[ct][e] + pd[e];
                    o[((size_t)(c0 + i) * HV + h) * DV + col0 + 16 * ct + lr] = f32_to_bf16(ov);
                }
            }
        }
        const float gam_n = sGam[C - 1];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4 s = S[dt][ct] * gam_n;
#pragma unroll
                for (int ks = 0; ks < C / 32; ++ks) {
                    const bf16x8 kt = ld_op(sKt, LC, 32 * w + 16 * dt, 32 * ks, lane);
                    s = mfma_bf16(kt, ld_op(sDt_hi, LC, 16 * ct, 32 * ks, lane), s);
                    s = mfma_bf16(kt, ld_op(sDt_lo, LC, 16 * ct, 32 * ks, lane), s);
                }
                S[dt][ct] = s;
            }
        __syncthreads();  // every wave is done reading S^T before it is rewritten
        write_St();
    }

    if (S_T) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 32 * w + 16 * dt + 4 * lq + e;
                    S_T[tab + (size_t)d * DV + col0 + 16 * ct + lr] = S[dt][ct][e];
                }
    }
}

}  // namespace

bool prefill_chunked_supported(int dk, int dv, bool bf16) { return bf16 && dk == DK && dv % DVS == 0; }

hipError_t launch_prefill_chunked(const PrefillArgs &a, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    const int rep = a.HV / a.HQK;
    dim3 grid((unsigned)((int64_t)a.N * a.HV), (unsigned)(a.dv / DVS));
    hipLaunchKernelGGL((prefill_chunked_kernel<uint16_t>), grid, dim3(NT), 0, stream,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                       static_cast<const uint16_t *>(a.v), a.g, a.beta, a.cu_seqlens, a.eq_len, a.S0,
                       static_cast<uint16_t *>(a.o), a.S_T, a.HV, a.dv, rep, a.scale);
    return hipGetLastError();
}

}  // namespace gdn
