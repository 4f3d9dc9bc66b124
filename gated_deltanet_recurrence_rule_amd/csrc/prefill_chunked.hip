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
// and inside a 32-token block T_b = [[T_00, 0], [T_10, T_11]] from the inverses T_00, T_11
// of its two diagonal 16-blocks (forward substitution in fp32, one column per lane) and
// the coupling T_10 = -T_11 A_10 T_00, formed on MFMA through W = A_10 T_00.
//
// Precision.  MFMA operands are bf16; a value that is not exactly bf16 is either
// rounded once or carried as hi + lo (hi = bf16(x), lo = bf16(x - hi); two or
// three MFMAs).  Raw q, k, v rows are exact bf16.  The table path is carried
// hi + lo: S in K S, T_b, A_10 and Z / Delta in the solve, the scaled Delta in
// K^T D.  The output path rounds once: S in Q S, P and Delta in P Delta -- except
// for the rules without the look-up, whose growing table is carried hi + lo in Q S
// too.  All accumulation is fp32.
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
//  * Waves 4-7 ("Gram waves") stage the chunks' q, k rows into LDS, form the gates'
//    cumulative decays, and compute the chunk's Gram tiles, writing T_0, T_1 and P into
//    LDS already in that MFMA operand order (computing a Gram tile with the two operand
//    roles swapped yields it transposed, which is the operand order directly); column
//    waves 0 and 2 write the -A_10 tiles.
// One workgroup barrier per chunk: in one period the column waves finish chunk c (the
// solve, the reads, the table update) and start chunk c + 1 (K S, Q S, Z), while the Gram
// waves build the operands of chunk c + 1 and stage chunk c + 2.  K and Q rows and the
// per-token scalars rotate over three buffers, the operands over two.  q, k, g and beta are
// fetched into registers a period before they are staged, v a period before it is used.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int C = 64;       // chunk length
constexpr int DK = 128;     // key dimension
constexpr int DVS = 64;     // dv columns per workgroup
constexpr int NT = 512;     // threads (8 waves)

// Row stride (bf16) of K and Q in LDS.  With rows of 288 bytes the operand reads of 16 rows
// run without bank conflicts, and the transposed reads at twice the conflict-free time;
// 272-byte rows double both (measured on gfx950).
constexpr int LK = DK + 16;

// LDS layout (bytes).  Buffers tagged [3] are selected by chunk index mod 3, [2] by parity.
constexpr int KQ_SZ = 2 * C * LK * 2;                      // K then Q, [C][LK] bf16 each, rows = tokens
constexpr int OFF_KQ = 0;                                  // [3], by chunk index mod 3
constexpr int OPT_SZ = 2 * 2 * 2 * 64 * 16;                // T_b operands [2 b][2 rt][2 hi/lo][64][8]
constexpr int OPA_SZ = 2 * 2 * 64 * 16;                    // -A_10 operands [2 rt][2 hi/lo][64][8]
constexpr int OPP_SZ = 6 * 64 * 16;                        // P operands [6 (rt, ks)][64][8]
constexpr int OP_SZ = OPT_SZ + OPA_SZ + OPP_SZ;
constexpr int OFF_OP = OFF_KQ + 3 * KQ_SZ;                 // [2], by chunk parity
constexpr int SC_SZ = 10 * C;                              // fp32 per-token scalars of one chunk
constexpr int OFF_SC = OFF_OP + 2 * OP_SZ;                 // [3], by chunk index mod 3
constexpr int OFF_FLAG = OFF_SC + 3 * SC_SZ * 4;           // two int hand-over counters (T_00, T_11 of each 32-block)
constexpr int LDS_BYTES = OFF_FLAG + 16;
// The diagonal 16-blocks of A and of their inverses are handed from one Gram wave to
// another through the Q rows of the chunk before the one being built (while chunk c + 1 is
// built, the column waves read only chunk c's K rows): four 16 x 16 fp32 blocks each, rows
// of BR floats, at a stride of DSTR floats.  With rows of 20, the 16 lanes that write or
// read 4 floats of 16 different rows hit 16 different groups of 4 banks.
constexpr int BR = 20;
constexpr int DSTR = 16 * BR + 16;
static_assert(2 * 4 * DSTR * 4 <= KQ_SZ / 2, "hand-over blocks fit in one Q buffer");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 to_bf16(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ f32x8 cat(f32x4 a, f32x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// bf16 pair dot product a.x b.x + a.y b.y + c in one instruction (products are exact in fp32)
__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
// A packed bf16 pair constant held in a scalar register.  (Written as a vector literal,
// (-1, 0) is emitted as the inline constant -1.0, which packed bf16 operands read as (0, -1).)
__device__ __forceinline__ bf16x2 pair_const(uint32_t bits) {
    uint32_t r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(bits));
    return __builtin_bit_cast(bf16x2, r);
}
// hi = bf16(x), lo = bf16(x - hi).  x - hi is exact in fp32; it is formed by a dot product
// of the packed hi pair with (-1, 0) or (0, -1), which also does the widening of hi.
__device__ __forceinline__ void split(f32x8 x, bf16x8 &hi, bf16x8 &lo) {
    hi = to_bf16(x);
    const bf16x2 m0 = pair_const(0x0000bf80u), m1 = pair_const(0xbf800000u);
    const bf16x2 hp[4] = {__builtin_shufflevector(hi, hi, 0, 1), __builtin_shufflevector(hi, hi, 2, 3),
                          __builtin_shufflevector(hi, hi, 4, 5), __builtin_shufflevector(hi, hi, 6, 7)};
    f32x8 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        r[2 * p] = dot2(hp[p], m0, x[2 * p]);
        r[2 * p + 1] = dot2(hp[p], m1, x[2 * p + 1]);
    }
    lo = to_bf16(r);
}
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
    hi = __builtin_convertvector(x, bf16x4);
    const bf16x2 m0 = pair_const(0x0000bf80u), m1 = pair_const(0xbf800000u);
    const bf16x2 hp[2] = {__builtin_shufflevector(hi, hi, 0, 1), __builtin_shufflevector(hi, hi, 2, 3)};
    f32x4 r;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        r[2 * p] = dot2(hp[p], m0, x[2 * p]);
        r[2 * p + 1] = dot2(hp[p], m1, x[2 * p + 1]);
    }
    lo = __builtin_convertvector(r, bf16x4);
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
// 16t + 4g + e.  K and Q rows (over d) are kept in LDS in this order, so the 8 tile-order
// operand values of lane group g = lane/16 are one contiguous 16-byte read (ld_std at
// k0 = 32 * block); K^T operands (over tokens) come from the same K rows by two transposed
// reads (ld_tr), every 4 consecutive d staying contiguous.  Gram products read both
// operands in the same permuted order, which leaves them unchanged.
__device__ __forceinline__ int tile_pos(int x) {
    const int r = x & 31;
    return (x & ~31) + 8 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3);
}
// Transposed LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// loads four 16-bit values A_i[0..3] from its own address, and lane j receives
// A_{j/4}[j%4], A_{4+j/4}[j%4], A_{8+j/4}[j%4], A_{12+j/4}[j%4].  So when lane i points at
// row r0 + i/4 and the four consecutive columns c0 + 4 (i%4) .. + 3 of a row-major bf16
// matrix, lane j receives rows r0 .. r0 + 3 of column c0 + j: a column read from rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 ld_tr(const __bf16 *p) {
    return __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p)));
}

// 2^x on the hardware exponential unit (flushes very negative x to zero).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over each row of 16 lanes, result in every lane of the row (DPP, no LDS traffic).  Every
// source lane of these patterns lies in the row, so no lane takes the bound-control zero.
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
    return x;
}

// Every lambda of the kernel is inlined: an outlined call would save and restore registers
// around it and serialise its latency.
#define GDN_INLINE __attribute__((always_inline))

// A copy of x the compiler cannot see through: lane-dependent addresses derived from
// it are recomputed inside the chunk loop instead of being hoisted out and spilled.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Global traffic goes through raw buffer accesses: a descriptor over a wave-uniform base
// (re-based every chunk, so 32-bit offsets suffice) and a per-lane byte offset in a VGPR.
// The 64-bit address arithmetic then stays out of the vector ALU.  The hardware range check
// covers the vector offset (not a scalar one), so every access puts its row there against a
// descriptor whose range ends at the chunk's last valid row: loads past it read zero without
// a memory access, and stores past it are given an out-of-range offset and dropped.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// acc + a * x in one instruction, with a taken from lane M of this lane's row of 16 (DPP row
// broadcast; the compiler does not fold a broadcast into a multiply-add by itself).  A DPP
// source needs two wait states after a vector write to it, which are not inserted around
// inline asm: a must come straight from a memory load, as it does at every use below.
template <int M>
__device__ __forceinline__ float fma_row_bcast(float a, float x, float acc) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(a), "v"(x), "i"(M));
    return acc;
}
// acc + sum_{m < I} a(lane m) x_m, the newest term x_{I-1} last
template <int I, int M = 0>
__device__ __forceinline__ float row_bcast_dot(float a, const float *x, float acc) {
    if constexpr (M < I) return row_bcast_dot<I, M + 1>(a, x, fma_row_bcast<M>(a, x[M], acc));
    else return acc;
}
// Forward substitution for column fj of (I + A)^{-1}, one column per lane of a row of 16: the lane
// holding column m of -A supplies -A_im by broadcast.  x_i = [i == fj] - sum_{m < i} A_im x_m for
// every i: rows above fj see only zeros and stay 0, row fj gets 1, so no row needs a mask.
template <int I>
__device__ __forceinline__ void solve_rows(float *x, const f32x4 *acol, int fj) {
    if constexpr (I < 16) {
        x[I] = row_bcast_dot<I>(acol[I >> 2][I & 3], x, (I == fj) ? 1.f : 0.f);
        solve_rows<I + 1>(x, acol, fj);
    }
}

// DELTA = false drops the look-up (A = 0, so T = I and Delta = Z = diag(b) V): the decayed
// linear-attention rule of the learn-llm page's update-rule table.
// SPLIT = false compiles the split-sequence passes out (mode 0 only).
template <bool DELTA, bool SPLIT>
__global__ __launch_bounds__(NT) void prefill_chunked_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ order, int64_t span,
    const float *__restrict__ S0, uint16_t *__restrict__ o, float *__restrict__ S_T, int HV, int DV,
    int rep, int NG, int M, int nfirst, float scale, GateArgs gate, SplitArgs sp) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    // Chunk c's K and Q rows and its per-token scalars live in buffers c % 3, the solve /
    // read operands built from them in the buffers of parity c % 2.  Scalars:
    // G (cumulative log-decay times log2 e), gamma = exp(G), r_k = 1/|k|, r_q = scale/|q|,
    // beta, r_k exp(G_n - G), and split decays.  With E_b = G at token 16 b + 15 (the end of
    // 16-token tile b): CF[t] = exp(E_{t/16} - G_t) and RF[b][t] = exp(G_t - E_b) for t past
    // tile b, so a tile with rows i after its columns j (tile b) has exp(G_i - G_j) =
    // RF[b][i] CF[j], both factors <= 1.
#define GDN_CHUNK(c)                                                                        \
    const int par_ = (c) & 1;                                                               \
    __bf16 *sK = reinterpret_cast<__bf16 *>(lds + OFF_KQ + ((c) % 3) * KQ_SZ);              \
    __bf16 *sQ = sK + C * LK;                                                               \
    bf16x8 *opT = reinterpret_cast<bf16x8 *>(lds + OFF_OP + par_ * OP_SZ);                  \
    bf16x8 *opA = opT + OPT_SZ / 16;                                                        \
    bf16x8 *opP = opA + OPA_SZ / 16;                                                        \
    float *sc_ = reinterpret_cast<float *>(lds + OFF_SC) + ((c) % 3) * SC_SZ;               \
    float *sG = sc_, *sGam = sc_ + C, *sRk = sc_ + 2 * C;                                   \
    float *sRq = sc_ + 3 * C, *sB = sc_ + 4 * C, *sDn = sc_ + 5 * C;                        \
    float *sCF = sc_ + 6 * C, *sRF = sc_ + 7 * C;                                           \
    (void)sK; (void)sQ; (void)opT; (void)opA; (void)opP;                                    \
    (void)sG; (void)sGam; (void)sRk; (void)sRq; (void)sB; (void)sDn; (void)sCF; (void)sRF;
    // opT [((b*2 + rt)*2 + hl)*64 + lane], opA [(rt*2 + hl)*64 + lane], opP [idx*64 + lane]

    // Workgroup -> (sequence, V head, column slice).  The M = rep * (DV / 64) workgroups
    // that read the same q and k rows (one sequence, one QK head: group G) get linear ids
    // L = 8 (M (G / 8) + m) + G % 8, i.e. the same L mod 8, so round-robin dispatch over the
    // eight XCDs places them on one XCD and one L2, launched one after another.  Groups are
    // numbered in launch order (sequence rank, segment, then QK head); ids past the last
    // group exit.
    //
    // The grid has up to three parts, each numbered as above, launched in this order.
    //  * Unsplit (mode 0): part 0 holds the nfirst longest sequences on narrow workgroups of 32
    //    columns in which only column waves 0 and 1 hold columns (a chunk then takes ~0.87-0.95
    //    of the time: the column waves' LDS reads of K and Q are halved per CU), so a sequence
    //    that would outlast the rest of the batch finishes sooner on twice the workgroups; part
    //    2 holds the other sequences on 64-column workgroups.
    //  * Split sequences: the first sp.ns launch ranks (every sequence of a small batch, or the
    //    k longest of a packed one) are cut into P = sp.P >= 3 segments of whole chunks; with cps =
    //    ceil(chunks / (P - 1 + w0)), segment 0 is w0 cps chunks long and segment s >= 1 takes
    //    chunks [(w0 + s - 1) cps, (w0 + s) cps).
    //    - map pass (sp.mode 1): part 0 scans segment 0 of the split ranks from S0, writing its
    //      reads; its final table, segment 1's start, goes to sp.starts.  Part 1 runs segments
    //      1 .. P-2 of the split ranks with the table widened to DW = DV + DK columns, started at
    //      [0 | I], the extra columns reading v = 0.  Each column of the table evolves on its own
    //      and affinely in the start state, so the segment's final table is [B | M] with
    //      S_out = M S_in + B.  Reads are not stored; the final table goes to sp.maps,
    //      [P - 2 segments][HV][DK][DW] per split rank.  Part 2 runs the other sequences whole.
    //      Segment 0 goes first: it is the longest stretch of the pass's critical path.
    //    - segment pass (sp.mode 2): part 2 runs segments 1 .. P-1 of the split ranks from
    //      sp.starts, [P - 1][HV][DK][DV] per split rank (the first written by the map pass,
    //      the others chained from the maps), writing their reads; the last writes S_T.
    const int HQK = HV / rep;
    const int mode = SPLIT ? sp.mode : 0;
    const int ns = SPLIT ? sp.ns : 0;
    const int PS = mode == 1 ? sp.P - 2 : (mode == 2 ? sp.P - 1 : 1);  // segments per split rank in a segment part
    const int NG0 = mode == 0 ? nfirst * HQK : (mode == 1 ? ns * HQK : 0);  // groups of part 0
    const int M0 = rep * (DV / (SPLIT ? DVS : DVS / 2));                     // workgroups per group there
    const int NG1 = mode == 1 ? ns * PS * HQK : 0;                           // part 1 (segment maps)
    const int M1 = rep * ((DV + DK) / DVS);
    const int W0 = 8 * M0 * ((NG0 + 7) / 8), W1 = 8 * M1 * ((NG1 + 7) / 8);  // part sizes (multiples of 8)
    const int part = (int)blockIdx.x < W0 ? 0 : ((int)blockIdx.x < W0 + W1 ? 1 : 2);
    const bool narrow = !SPLIT && part == 0;
    const bool mapwg = part == 1;                   // a segment map
    const int DW = mapwg ? DV + DK : DV;            // table width
    const int Lid = (int)blockIdx.x - (part >= 1 ? W0 : 0) - (part == 2 ? W1 : 0);
    const int Mg = part == 0 ? M0 : (part == 1 ? M1 : M);
    const int G = 8 * ((Lid >> 3) / Mg) + (Lid & 7);
    if (G >= (part == 0 ? NG0 : (part == 1 ? NG1 : NG))) return;
    const int mem = (Lid >> 3) % Mg;
    const bool segpart = mapwg || mode == 2;        // groups run segments 1 .. of split ranks
    const int rank = (part == 2 && mode != 2 ? (mode == 0 ? nfirst : ns) : 0) + G / ((segpart ? PS : 1) * HQK);
    const int seg = segpart ? 1 + (G / HQK) % PS : 0;
    const bool splitseq = mode != 0 && rank < ns;    // this sequence is cut into segments
    const int hq = G % HQK;
    const int nseq = order ? order[rank] : rank;
    const int slw = narrow ? DVS / 2 : DVS;         // columns per workgroup
    const int h = hq * rep + mem / (DW / slw);
    const int col0 = (mem % (DW / slw)) * slw;
    const int unit = nseq * HV + h;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int lr = lane & 15;
    const int lq = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, known to be uniform
    const bool colwave = w < 4;

    int64_t t0, t1;
    if (cu_seqlens) {
        // span = total_T here: entries are clamped into [0, total_T] and made non-decreasing,
        // so no device array can send the kernel outside the token buffers
        t0 = clamp_tok(cu_seqlens[nseq], 0, span);
        t1 = clamp_tok(cu_seqlens[nseq + 1], t0, span);
    } else {
        t0 = (int64_t)nseq * span;
        t1 = t0 + span;
    }
    if (splitseq) {
        // segment seg: units [seg == 0 ? 0 : w0 + seg - 1, w0 + seg) of cps chunks each, cps =
        // ceil(chunks / (P - 1 + w0))
        const int64_t len = t1 - t0;
        const int64_t units = sp.P - 1 + sp.w0;
        const int64_t cps = ((len + C - 1) / C + units - 1) / units;
        const int64_t a = (seg == 0 ? 0 : (int64_t)(sp.w0 + seg - 1)) * cps * C;
        const int64_t bnd = (int64_t)(sp.w0 + seg) * cps * C;
        const int64_t s1 = t0 + (bnd < len ? bnd : len);
        t0 += a < len ? a : len;
        t1 = s1;
    }

    const int nchunks = (int)((t1 - t0 + C - 1) / C);
    if (tid == 0) {
        int *fl = reinterpret_cast<int *>(lds + OFF_FLAG);
        fl[0] = 0;
        fl[1] = 0;
    }
    __syncthreads();  // counters cleared before any wave uses them
    auto chunk_len = [&](int c) GDN_INLINE { return (int)((t1 - t0 - (int64_t)c * C) < C ? (t1 - t0 - (int64_t)c * C) : C); };

    // Schedule.  For chunk c the column waves run phase "a" (K S, Q S and Z) and then phase
    // "b" (the solve, the reads, the table update).  One period per chunk, closed by one
    // workgroup barrier: the column waves run phase b of chunk c and phase a of chunk c+1
    // while the Gram waves build T, P (and with column waves 0 and 2, -A_10) of chunk c+1
    // and stage chunk c+2 into LDS.  A prologue stages chunk 0, then builds its operands and
    // stages chunk 1 beside the column waves' phase a of chunk 0.
    // LDS counters: the last chunk whose T_00, T_11 are in LDS, per 32-token block
    int *flag = reinterpret_cast<int *>(lds + OFF_FLAG);
    // The operand tiles of chunk c built from its Gram tiles alone: the read operands P and
    // the coupling -A_10 of the two 32-token blocks.
    //
    // P operand idx = (rt, ks), ks <= rt / 2:  0 (0,0) 1 (1,0) 2 (2,0) 3 (2,1) 4 (3,0) 5 (3,1).
    // Tile (rt, kt) from MFMA(K block kt, Q block rt): element e at lane is
    // (Q K^T)[16 rt + lr][16 kt + 4 lq + e], the tile-order operand slot.
    auto p_operand = [&](int c, int idx) GDN_INLINE {
        const int ln = opaque(lane);
        const int lrr = ln & 15, lqq = ln >> 4;
        GDN_CHUNK(c)
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        auto load_blk = [&](const __bf16 *base, int kb, bf16x8 *dst) GDN_INLINE {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) dst[ks] = ld_std(base, LK, 16 * kb, 32 * ks, ln);
        };
        const int rt = idx == 0 ? 0 : (idx == 1 ? 1 : (idx < 4 ? 2 : 3));
        const int ks = (idx == 3 || idx == 5) ? 1 : 0;
        const int i = 16 * rt + lrr;
        const float ci = sRq[i], Gi = sG[i];
        bf16x8 qq[4];
        load_blk(sQ, rt, qq);
        f32x8 x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kt = 2 * ks + t;
            if (kt > rt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[4 * t + e] = 0.f;
                continue;
            }
            bf16x8 kk[4];
            load_blk(sK, kt, kk);
            f32x4 acc = zero;
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) acc = mfma32(kk[kq], qq[kq], acc);
            const int j0 = 16 * kt + 4 * lqq;
            const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + j0);
            if (kt < rt) {  // every row after every column: split decays, no mask
                const float cr = ci * sRF[kt * C + i];
                const f32x4 CF4 = *reinterpret_cast<const f32x4 *>(sCF + j0);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[4 * t + e] = cr * (R4[e] * CF4[e]) * acc[e];
            } else {
                const f32x4 G4 = *reinterpret_cast<const f32x4 *>(sG + j0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[4 * t + e] = (j0 + e <= i) ? ci * R4[e] * acc[e] * exp2_hw(Gi - G4[e]) : 0.f;
            }
        }
        opP[idx * 64 + ln] = to_bf16(x);
    };
    // -A_10 (rows 32 + 16 rt .., columns 0..31) in tile order, from role-swapped Gram tiles
    auto a_operand = [&](int c, int rt) GDN_INLINE {
        const int ln = opaque(lane);
        const int lrr = ln & 15, lqq = ln >> 4;
        GDN_CHUNK(c)
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        auto load_blk = [&](const __bf16 *base, int kb, bf16x8 *dst) GDN_INLINE {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) dst[ks] = ld_std(base, LK, 16 * kb, 32 * ks, ln);
        };
        const int i = 32 + 16 * rt + lrr;
        const float ci = sB[i] * sRk[i];
        bf16x8 kr[4];
        load_blk(sK, 2 + rt, kr);
        f32x8 x;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x8 kk[4];
            load_blk(sK, t, kk);
            f32x4 acc = zero;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma32(kk[ks], kr[ks], acc);
            const int j0 = 16 * t + 4 * lqq;
            const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + j0);
            const f32x4 CF4 = *reinterpret_cast<const f32x4 *>(sCF + j0);
            const float cr = -ci * sRF[t * C + i];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * t + e] = cr * (R4[e] * CF4[e]) * acc[e];
        }
        bf16x8 hi, lo;
        split(x, hi, lo);
        opA[(rt * 2 + 0) * 64 + ln] = hi;
        opA[(rt * 2 + 1) * 64 + ln] = lo;
    };
    if (colwave && narrow && wu >= 2) {
        // a narrow workgroup's column waves 2 and 3 hold no columns: they take part in the
        // workgroup barriers only (two before the chunk loop, one per chunk)
        if (nchunks > 0)
            for (int i = 0; i < nchunks + 2; ++i) __syncthreads();
        return;
    }
    if (colwave) {
        // ====================== column waves: the table and the per-chunk chain ======
        // Element e of S[dt] is S[16 dt + 4 lq + e][col0 + 16 w + lr].
        f32x4 S[8];
        const int mycol = col0 + 16 * w + lr;
        // start table (row stride DW) and where the final table goes
        const float *Sin = S0 ? S0 + (size_t)unit * DK * DV : nullptr;
        float *Sout = S_T ? S_T + (size_t)unit * DK * DV : nullptr;
        if (mapwg) {
            Sin = nullptr;
            Sout = sp.maps + ((size_t)(rank * (sp.P - 2) + seg - 1) * HV + h) * DK * DW;
        } else if (mode == 1 && splitseq) {
            // segment 0 from S0; its end is segment 1's start
            Sout = sp.starts + ((size_t)rank * (sp.P - 1) * HV + h) * DK * DV;
        } else if (mode == 2) {
            Sin = sp.starts + ((size_t)(rank * (sp.P - 1) + seg - 1) * HV + h) * DK * DV;
            if (seg != sp.P - 1) Sout = nullptr;
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * dt + 4 * lq + e;
                S[dt][e] = Sin ? Sin[(size_t)r * DW + mycol] : ((SPLIT && mycol - DV == r) ? 1.f : 0.f);
            }
        auto store_table = [&]() GDN_INLINE {
            if (Sout) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) Sout[(size_t)(16 * dt + 4 * lq + e) * DW + mycol] = S[dt][e];
            }
        };
        if (nchunks == 0) {
            store_table();
            return;
        }

        // v[16 rt + 4 lq + e][mycol] of the next chunk, fetched one chunk ahead
        uint16_t vreg[4][4];
        const size_t vrs = (size_t)HV * DV;  // token stride of v and o
        const uint32_t rowb = 2u * (uint32_t)vrs;  // bytes per token row of v and o
        const uint16_t *vwave = v + (size_t)h * DV + col0 + 16 * wu;
        // a segment map's identity columns (col0 >= DV) read v = 0, and a map stores no reads:
        // their buffer descriptors cover no bytes, so the hardware returns zeros and drops stores
        const bool vio = !SPLIT || (col0 < DV && !mapwg);
        const bool vin = !SPLIT || col0 < DV;
        const bool reads = !SPLIT || !mapwg;  // segment maps form no reads
        uint16_t *owave = o + (size_t)h * DV + col0 + 16 * wu;
        // Row 16 rt + 4 lq + e of the chunk is read through a descriptor based at row 16 rt whose
        // range ends at the chunk's last valid row, with the lane's byte offset (4 lq + e rows, lr
        // columns) in the vector offset, which is what the hardware range check covers: rows
        // past the chunk, and every row of a chunk past the sequence, read zero without a memory
        // access.  The loads are therefore unconditional, with no zero-filling branch.
        uint32_t voff[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) voff[e] = 2u * (uint32_t)lr + (uint32_t)(4 * lq + e) * rowb;
        auto prefetch_v = [&](int c) GDN_INLINE {
            const int nn = chunk_len(c);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int rem = nn - 16 * rt;
                const uint32_t bytes = (vin && rem > 0) ? (uint32_t)rem * rowb : 0u;
                const rsrc_t vr = make_rsrc(vwave + (size_t)(t0 + (int64_t)c * C + 16 * rt) * vrs, bytes);
#pragma unroll
                for (int e = 0; e < 4; ++e) vreg[rt][e] = __builtin_amdgcn_raw_buffer_load_b16(vr, voff[e], 0, 0);
            }
        };

        // Carried from phase a to phase b of a chunk.  Swapping the operands of a product
        // transposes its accumulator tile: element e of Ot[rt] at this lane is
        // (Q S)[16 rt + lr][16 w + 4 lq + e].  Sg = gamma_n S, the decayed start table that
        // the update adds K^T D to, is formed in phase a before the hi / lo split, so the
        // split may overwrite S's registers (the split's dot product accumulates in place).
        f32x4 Z[4], Ot[4], Sg[8];

        // ---- phase a: Y = K S (hi + lo), Z = beta (v - gamma r_k Y), O^T = S^T Q^T (hi)
        auto phase_a = [&](int c) GDN_INLINE {
            const int ln = opaque(lane);
            const int lqq = ln >> 4;
            GDN_CHUNK(c)
            float vcur[4][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) vcur[rt][e] = bf16_to_f32(vreg[rt][e]);
            // The next chunk's loads go after the conversion, into the registers it frees.  Left to
            // itself the compiler sinks the conversion to its use at the end of the phase, so the
            // loads land in other registers that are copied back at the end of the period, which
            // waits for loads issued only a fraction of a period before.
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(vcur[rt][e]));
            __builtin_amdgcn_sched_barrier(0);
            prefetch_v(c + 1);  // past the last chunk: no bytes in range, the loads read zero
            const float gam_n = sGam[C - 1];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) Sg[dt] = S[dt] * gam_n;
            // contraction block ks outermost: eight independent accumulator chains in flight
            f32x4 y[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                y[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                Ot[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 Sh, Sl;
                split(cat(S[2 * ks], S[2 * ks + 1]), Sh, Sl);
                bf16x8 kk[4], qq[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    kk[rt] = ld_std(sK, LK, 16 * rt, 32 * ks, ln);
                    if (reads) qq[rt] = ld_std(sQ, LK, 16 * rt, 32 * ks, ln);
                }
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if constexpr (DELTA) y[rt] = mfma32(kk[rt], Sh, y[rt]);
                    if (reads) Ot[rt] = mfma32(Sh, qq[rt], Ot[rt]);
                }
                if constexpr (DELTA) {
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) y[rt] = mfma32(kk[rt], Sl, y[rt]);
                } else if (reads) {
                    // without the look-up the table grows with the sequence and so do the
                    // reads: carry the table as hi + lo in Q S as well (no K S to pay for)
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) Ot[rt] = mfma32(Sl, qq[rt], Ot[rt]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int i0 = 16 * rt + 4 * lqq;
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(sB + i0);
                const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sGam + i0);
                const f32x4 k4 = *reinterpret_cast<const f32x4 *>(sRk + i0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Z[rt][e] = DELTA ? b4[e] * (vcur[rt][e] - g4[e] * k4[e] * y[rt][e]) : b4[e] * vcur[rt][e];
            }
        };

        // ---- phase b: solve, reads, table update
        auto phase_b = [&](int c) GDN_INLINE {
            const int ln = opaque(lane);
            const int lrr = ln & 15, lqq = ln >> 4;
            const int64_t c0 = t0 + (int64_t)c * C;
            const int n = chunk_len(c);
            GDN_CHUNK(c)
            // Delta_0 = T_0 Z_0;  Delta_1 = T_1 (Z_1 - A_10 Delta_0);  D = diag(r_k exp(G_n - G)) Delta.
            // D and the bf16 read operands are taken from each Delta half before its hi/lo split,
            // so the split can overwrite it.
            f32x4 Dl[4];
            f32x8 Dx[2];
            bf16x8 Dsg[2];
            if constexpr (!DELTA) {
                // no look-up: Delta = Z
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sDn + 32 * ks + 16 * t + 4 * lqq);
#pragma unroll
                        for (int e = 0; e < 4; ++e) Dx[ks][4 * t + e] = Z[2 * ks + t][e] * d4[e];
                    }
                    Dsg[ks] = to_bf16(cat(Z[2 * ks], Z[2 * ks + 1]));
                }
            } else {
                bf16x8 zh, zl;
                split(cat(Z[0], Z[1]), zh, zl);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                    Dl[rt] = mfma32_x3(opT[(rt * 2 + 0) * 64 + ln], opT[(rt * 2 + 1) * 64 + ln], zh, zl, zero);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sDn + 16 * t + 4 * lqq);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Dx[0][4 * t + e] = Dl[t][e] * d4[e];
                }
                bf16x8 dh, dl;
                split(cat(Dl[0], Dl[1]), dh, dl);
                Dsg[0] = dh;
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
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(sDn + 32 + 16 * t + 4 * lqq);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Dx[1][4 * t + e] = Dl[2 + t][e] * d4[e];
                }
                Dsg[1] = to_bf16(cat(Dl[2], Dl[3]));
            }
            // O^T = gamma r_q (Q S)^T + (P Delta)^T: token 16 rt + lr, 4 adjacent columns per lane
            if (reads) {
                const rsrc_t orr = make_rsrc(owave + (size_t)c0 * vrs, vio ? (uint32_t)n * rowb : 0u);
                const uint32_t ooff = (uint32_t)lrr * rowb + 8u * (uint32_t)lqq;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f32x4 pd = {0.f, 0.f, 0.f, 0.f};
                    const int base = rt == 0 ? 0 : (rt == 1 ? 1 : (rt == 2 ? 2 : 4));
#pragma unroll
                    for (int ks = 0; ks <= (rt >> 1); ++ks) pd = mfma32(Dsg[ks], opP[(base + ks) * 64 + ln], pd);
                    const int i = 16 * rt + lrr;
                    const float gq = sGam[i] * sRq[i];
                    const bf16x4 ob = __builtin_convertvector(gq * Ot[rt] + pd, bf16x4);
                    // rows past the chunk get an offset beyond the descriptor's range, which the
                    // hardware drops (no branch, so the memory counters stay exact)
                    const uint32_t off = (i < n) ? ooff + (uint32_t)(16 * rt) * rowb : 0xFFFFFFF0u;
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ob), orr, off, 0, 0);
                }
            }
            // S <- Sg + K^T D
            {
                bf16x8 Dh[2], Dlo[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) split(Dx[ks], Dh[ks], Dlo[ks]);
                // The A operand K^T (rows d = 16 dt + lr, tokens in tile order) is read from the K
                // rows by two transposed reads: lane i of a group of 16 points at token row
                // 32 ks + 16 t + 4 lq + i/4 and the d-quad 16 dt + 4 (i%4) (stored at tile
                // position 32 (dt/2) + 8 (i%4) + 4 (dt%2)), so lane lr receives tokens
                // 32 ks + 16 t + 4 lq .. + 3 of d = 16 dt + lr.
                const __bf16 *ktp = sK + (4 * lqq + (lrr >> 2)) * LK + 8 * (lrr & 3);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    f32x4 acc = Sg[dt];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const __bf16 *q0 = ktp + 32 * ks * LK + 32 * (dt >> 1) + 4 * (dt & 1);
                        const bf16x8 kt = cat(ld_tr(q0), ld_tr(q0 + 16 * LK));
                        acc = mfma32(kt, Dh[ks], acc);
                        acc = mfma32(kt, Dlo[ks], acc);
                    }
                    S[dt] = acc;
                }
            }
        };

        // Column waves 0 and 2 (0 and 1 in a narrow workgroup) also form the coupling operand
        // -A_10 of the next chunk (one row tile each) where they would otherwise wait for the
        // Gram waves.
        const bool couple = DELTA && (narrow || (wu & 1) == 0);
        const int art = narrow ? wu : wu >> 1;  // its row tile of -A_10
        prefetch_v(0);
        __syncthreads();  // chunk 0 staged
        phase_a(0);
        if (couple) a_operand(0, art);
        __syncthreads();  // operands of chunk 0 built, chunk 1 staged
        for (int c = 0; c + 1 < nchunks; ++c) {
            phase_b(c);
            if (couple) a_operand(c + 1, art);
            phase_a(c + 1);
            __syncthreads();
        }
        phase_b(nchunks - 1);
        __syncthreads();
        store_table();
        return;
    }
    if (nchunks == 0) return;

    // ====================== Gram waves: chunk staging, norms, decay, P, A, T =====
    const int gt = tid - 256;  // 0..255
    const int gw = w - 4;      // 0..3
    // Staging: item gt + 256 p (p = 0, 1) is the token pair (2 pr, 2 pr + 1), pr = gt/16 + 16 p,
    // times the 16-byte segment s = gt % 16 of their q and k rows (d = 8 s .. 8 s + 7).
    uint4 kreg[2][2], qreg[2][2];  // [p][token of the pair]
    float greg = 0.f, breg = 0.f;  // Gram wave 3: token = lane
    // gates from raw projections: the head's exp(A_log) and dt_bias (padding tokens carry raw
    // values that every map sends to 0: -inf for -exp(A_log) softplus and for sigmoid(b), +inf
    // for log sigmoid)
    const float g_ea = gate.A_log ? expf(gate.A_log[h]) : 0.f;
    const float g_dtb = gate.dt_bias ? gate.dt_bias[h] : 0.f;
    const bool g_raw = gate.A_log != nullptr || gate.alpha_sigmoid, b_raw = gate.beta_logit != 0;
    const bool g_sig = gate.alpha_sigmoid != 0;
    const size_t rs = (size_t)HQK * DK;  // token stride of q and k
    // token row of item (p, u) = 8 gw + 32 p + u (uniform) + 2 lq (lane)
    const int gwu = wu - 4;
    const uint32_t qkrow = 2u * (uint32_t)rs;  // bytes per token row of q and k
    // Token row 8 gw + 32 p + u + 2 lq: read through a descriptor based at row 8 gw + 32 p whose
    // range ends at the chunk's last valid row, with the lane's part (2 lq + u rows, 16-byte
    // segment lr) in the vector offset, which the hardware range check covers: rows past the
    // chunk read zero, so the loads need no branch and no zero-filling.
    const uint32_t qoff0 = (uint32_t)(2 * lq) * qkrow + 16u * (uint32_t)lr, qoff1 = qoff0 + qkrow;
    auto prefetch_qk = [&](int c) GDN_INLINE {
        const int nn = chunk_len(c);
        const int64_t cs = t0 + (int64_t)c * C;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r0 = 8 * gwu + 32 * p;
            const uint32_t bytes = nn > r0 ? (uint32_t)(nn - r0) * qkrow : 0u;
            const size_t base = (size_t)(cs + r0) * rs + (size_t)hq * DK;
            const rsrc_t kr = make_rsrc(k + base, bytes), qr = make_rsrc(q + base, bytes);
            kreg[p][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, qoff0, 0, 0));
            kreg[p][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, qoff1, 0, 0));
            qreg[p][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff0, 0, 0));
            qreg[p][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff1, 0, 0));
        }
        if (gwu == 3) {
            const bool ok = lane < nn;
            const uint32_t goff = 4u * (uint32_t)lane * (uint32_t)HV;
            const uint32_t gbytes = nn > 0 ? 4u * (uint32_t)nn * (uint32_t)HV : 0u;
            // no g: a = 1 (G = 0); no beta: b = 1 (padding tokens keep b = 0)
            greg = 0.f;
            breg = ok ? 1.f : 0.f;
            if (g) {
                const rsrc_t gr = make_rsrc(g + (size_t)cs * HV + h, gbytes);
                greg = ok ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gr, goff, 0, 0))
                          : (g_sig ? INFINITY : (gate.A_log ? -INFINITY : 0.f));
            }
            if (beta) {
                const rsrc_t br = make_rsrc(beta + (size_t)cs * HV + h, gbytes);
                breg = ok ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(br, goff, 0, 0))
                          : (gate.beta_logit ? -INFINITY : 0.f);
            }
        }
    };

    // chunk c's q and k (already in registers) -> LDS, and their norms
    auto stage_chunk = [&](int c) GDN_INLINE {
        GDN_CHUNK(c)
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
                    const bf16x2 k2 = __builtin_bit_cast(bf16x2, kw[e]), q2 = __builtin_bit_cast(bf16x2, qw[e]);
                    a = dot2(k2, k2, a);
                    bq = dot2(q2, q2, bq);
                }
                sk[u] = a;
                sq[u] = bq;
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
    };

    // Gram wave 3: chunk c's gates (already in registers, one token per lane) -> the
    // cumulative log-decay G and the decay scalars derived from it, and beta.  Formed right
    // after wave 3's own solve, where it would otherwise wait.
    auto chunk_scalars = [&](int c) GDN_INLINE {
        GDN_CHUNK(c)
        const int ln = opaque(lane);
        // raw gates on the hardware exp2, log2 and reciprocal: softplus(+-t) = max(+-t, 0) +
        // ln(1 + e^-|t|), log sigmoid(t) = -softplus(-t), and sigmoid(b) = 1 / (1 + e^-b) (when
        // 1 + e^-|t| rounds to 1 the term dropped is < 6e-8); then the inclusive prefix sum
        // over the 64 lanes: within rows of 16 by row shifts, then across rows by the row-15
        // and row-31 broadcasts (DPP, no LDS traffic)
        const float tt = greg + g_dtb;
        const float lt = 0.69314718055994531f * __builtin_amdgcn_logf(1.f + exp2_hw(-1.44269504088896341f * fabsf(tt)));
        const float gl = g_raw ? (g_sig ? -(fmaxf(-tt, 0.f) + lt) : -g_ea * (fmaxf(tt, 0.f) + lt)) : greg;
        breg = b_raw ? __builtin_amdgcn_rcpf(1.f + exp2_hw(-1.44269504088896341f * breg)) : breg;
        float x = gl * 1.44269504088896341f;  // log2(e)
#define GDN_DPP_ADD(ctrl, row_mask) \
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, row_mask, 0xF, true))
        GDN_DPP_ADD(0x111, 0xF);  // row_shr:1
        GDN_DPP_ADD(0x112, 0xF);  // row_shr:2
        GDN_DPP_ADD(0x114, 0xF);  // row_shr:4
        GDN_DPP_ADD(0x118, 0xF);  // row_shr:8
        GDN_DPP_ADD(0x142, 0xA);  // row_bcast:15 into rows 1 and 3
        GDN_DPP_ADD(0x143, 0xC);  // row_bcast:31 into rows 2 and 3
#undef GDN_DPP_ADD
        sG[ln] = x;
        sGam[ln] = exp2_hw(x);
        sB[ln] = breg;
        const float E0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
        const float E1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
        const float E2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
        const float E3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
        const int tb = ln >> 4;
        sCF[ln] = exp2_hw((tb == 0 ? E0 : tb == 1 ? E1 : tb == 2 ? E2 : E3) - x);
        sRF[ln] = tb > 0 ? exp2_hw(x - E0) : 0.f;
        sRF[C + ln] = tb > 1 ? exp2_hw(x - E1) : 0.f;
        sRF[2 * C + ln] = tb > 2 ? exp2_hw(x - E2) : 0.f;
    };

    // T_0, T_1, P and r_k exp(G_n - G) of chunk c, from its staged K, Q and scalars (the
    // coupling operand -A_10 comes from column waves 0 and 2).
    //
    // The Gram waves work in pairs, one pair per 32-token block b: waves 1 and 3 solve the two
    // diagonal 16-blocks of T in block b in fp32 and hand them over through LDS; waves 0 and
    // 2 form five tiles of P each meanwhile, then merge the two 16-blocks of their block.
    // Matrices live in MFMA accumulator form: element e at lane (g = lane/16, j = lane%16) is
    // M[4 g + e][j].  With Y and X in that form, Y^T X needs no data movement (lane group g
    // and element e enumerate the contracted index on both sides), so every product below
    // keeps a matrix and its transpose.  The hand-over counter of block b holds the last chunk
    // whose T_00 and T_11 are in LDS.
    f32x4 At;  // waves 0 and 2: A_10^T of their 32-token block, from head to tail
    // part 0 (the head): everything but the 32-block merge; part 1 (the tail): the merge
    auto build_operands = [&](int c, int part) GDN_INLINE {
        const int ln = opaque(lane);
        const int lrr = ln & 15, lqq = ln >> 4;
        GDN_CHUNK(c)
        // the diagonal 16-blocks of A and of T = (I + A)^{-1}, fp32, handed between Gram waves
        float *Adiag = reinterpret_cast<float *>(lds + OFF_KQ + (((c) + 2) % 3) * KQ_SZ + KQ_SZ / 2);  // [4][DSTR]
        float *Tdiag = Adiag + 4 * DSTR;                                             // [4][DSTR]
        const int b = gwu >> 1;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        auto load_blk = [&](const __bf16 *base, int kb, bf16x8 *dst) GDN_INLINE {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) dst[ks] = ld_std(base, LK, 16 * kb, 32 * ks, ln);
        };
        // Products on bf16 MFMA with hi/lo operands.  Y and X in accumulator form split into
        // bf16 (hi, lo); one 16x16x32 MFMA with A = (Yh, Yh) and B = (Xh, Xl) gives
        // Yh^T Xh + Yh^T Xl, a second with A = (Yl, 0) adds Yl^T Xh.
        auto hl = [&](const f32x4 &x, bf16x4 &h, bf16x4 &l) GDN_INLINE { split4(x, h, l); };
        auto prod3 = [&](const bf16x4 &yh, const bf16x4 &yl, const bf16x4 &xh, const bf16x4 &xl, f32x4 acc) GDN_INLINE {
            const bf16x4 z4 = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
            const bf16x8 bx = cat(xh, xl);
            acc = mfma32(cat(yh, yh), bx, acc);
            return mfma32(cat(yl, z4), bx, acc);
        };
        // Row tile rt of T_b as a tile-order (hi, lo) operand: 8 values at lane (g, i) are
        // T_b[16 rt + i][4 g + e] (first 16 columns) and T_b[16 rt + i][16 + 4 g + e].
        auto put_t = [&](int rt, const f32x4 &left_t, const f32x4 &right_t) GDN_INLINE {
            bf16x8 hi, lo;
            split(cat(left_t, right_t), hi, lo);
            opT[((2 * b + rt) * 2 + 0) * 64 + ln] = hi;
            opT[((2 * b + rt) * 2 + 1) * 64 + ln] = lo;
        };

        if constexpr (!DELTA) {
            // no look-up: only P and r_k exp(G_n - G) are needed
            if (part != 0) return;
            if (gwu == 0) {
                p_operand(c, 0);
                p_operand(c, 1);
            } else if (gwu == 1) {
                p_operand(c, 2);
                sDn[ln] = sRk[ln] * exp2_hw(sG[C - 1] - sG[ln]);
            } else if (gwu == 2) {
                p_operand(c, 3);
                p_operand(c, 4);
            } else {
                p_operand(c, 5);
            }
        } else if ((gwu & 1) != 0) {
            if (part != 0) return;
            // waves 1 and 3: the two diagonal 16-blocks T_00, T_11 of the 32-token block b = gwu / 2
            // of T = (I + A)^{-1}, by forward substitution in fp32, for wave gwu - 1 to merge (the
            // coupling operand -A_10 comes from column waves 0 and 2).
            const int blk = 2 * b;
            float *Ad = Adiag + b * 2 * DSTR;  // this block pair of A, then of T
            float *Td = Tdiag + b * 2 * DSTR;
            {
                // Gram tiles of the two diagonal blocks, stored as rows of -A^T: the tile is
                // symmetric, so element e at lane (g, j) is also row i = 4 g + e, column j, and
                // lane (g, j) writes -A[i][j] = -b_i r_k,i r_k,j (K K^T)_ij exp(G_i - G_j) (i > j)
                // to row j, columns 4 g .. 4 g + 3
                bf16x8 kd[4], kn[4];
                load_blk(sK, blk, kd);
                load_blk(sK, blk + 1, kn);
                f32x4 g0 = zero, g1 = zero;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    g0 = mfma32(kd[ks], kd[ks], g0);
                    g1 = mfma32(kn[ks], kn[ks], g1);
                }
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int t0b = 16 * (blk + hb);
                    const f32x4 gd = hb ? g1 : g0;
                    const int tj = t0b + lrr;
                    const float rj = sRk[tj], Gj = sG[tj];
                    const f32x4 B4 = *reinterpret_cast<const f32x4 *>(sB + t0b + 4 * lqq);
                    const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + t0b + 4 * lqq);
                    const f32x4 G4 = *reinterpret_cast<const f32x4 *>(sG + t0b + 4 * lqq);
                    f32x4 a;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a[e] = (lrr < 4 * lqq + e) ? -((B4[e] * R4[e]) * rj * gd[e] * exp2_hw(G4[e] - Gj)) : 0.f;
                    *reinterpret_cast<f32x4 *>(Ad + hb * DSTR + BR * lrr + 4 * lqq) = a;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            {
                // Lane (hb, fj) (lanes 32-63 repeat lanes 0-31) solves (I + A_hb) x = e_fj: x is
                // column fj of T_hb.  It reads column fj of -A_hb (row fj of the stored -A^T) and
                // takes the other columns from the lanes of its row of 16 by broadcast.
                const int hb = (ln >> 4) & 1, fj = ln & 15;
                const float *Ab = Ad + hb * DSTR;
                f32x4 acol[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) acol[q4] = *reinterpret_cast<const f32x4 *>(Ab + BR * fj + 4 * q4);
                float x[16];
                x[0] = (fj == 0) ? 1.f : 0.f;
                solve_rows<1>(x, acol, fj);
                if (ln < 32) {
                    float *Tb = Td + hb * DSTR;
#pragma unroll
                    for (int i = 0; i < 16; ++i) Tb[BR * i + fj] = x[i];
                }
            }
            __hip_atomic_store(flag + b, c + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else {
            // waves 0 and 2: read operands P and, for the 32-token block b = gwu / 2, the coupling
            // T_10 = -T_11 A_10 T_00 on MFMA through W = A_10 T_00, once wave gwu + 1 has solved
            // T_00 and T_11.
            const int blk = 2 * b;
            if (part == 0) {
            // A_10^T from the role-swapped Gram tile of blocks (2 b, 2 b + 1): element e at lane
            // (g, j) is A[16 (blk+1) + j][16 blk + 4 g + e]
            bf16x8 kd[4], kn[4];  // K blocks blk and blk + 1
            {
                load_blk(sK, blk, kd);
                load_blk(sK, blk + 1, kn);
                f32x4 gx = zero;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) gx = mfma32(kd[ks], kn[ks], gx);
                const int i0 = 16 * blk + 4 * lqq;
                const int r = 16 * (blk + 1) + lrr;
                const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + i0);
                const f32x4 CF4 = *reinterpret_cast<const f32x4 *>(sCF + i0);
                const float cr = sB[r] * sRk[r] * sRF[blk * C + r];
#pragma unroll
                for (int e = 0; e < 4; ++e) At[e] = cr * (R4[e] * CF4[e]) * gx[e];
            }
            // P operands idx = (rt, ks) hold tiles (rt, 2 ks) and (rt, 2 ks + 1): wave 0 forms
            // idx 0, 1, 5 and wave 2 idx 2, 3, 4 (five nonzero tiles, 20 MFMAs each), every LDS
            // read before the first store so that the reads are in flight together.  Register
            // arrays are indexed by constants only (a wave-dependent index would move them to
            // scratch memory).
            {
                auto gram = [&](const bf16x8 *x, const bf16x8 *y) GDN_INLINE {
                    f32x4 acc = zero;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) acc = mfma32(x[ks], y[ks], acc);
                    return acc;
                };
                // P[16 rt + j][16 kt + 4 g + e] from (K Q^T) tile (kt, rt)
                auto scale_p = [&](int rt, int kt, const f32x4 &acc) GDN_INLINE {
                    const int i = 16 * rt + lrr;
                    const float ci = sRq[i];
                    const int j0 = 16 * kt + 4 * lqq;
                    const f32x4 R4 = *reinterpret_cast<const f32x4 *>(sRk + j0);
                    f32x4 x;
                    if (kt < rt) {  // every row after every column: split decays, no mask
                        const float cr = ci * sRF[kt * C + i];
                        const f32x4 CF4 = *reinterpret_cast<const f32x4 *>(sCF + j0);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = cr * (R4[e] * CF4[e]) * acc[e];
                    } else {
                        const float Gi = sG[i];
                        const f32x4 G4 = *reinterpret_cast<const f32x4 *>(sG + j0);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            x[e] = (j0 + e <= i) ? ci * R4[e] * acc[e] * exp2_hw(Gi - G4[e]) : 0.f;
                    }
                    return x;
                };
                f32x8 xp[3];
                if (b == 0) {
                    bf16x8 k2[4], k3[4], q0[4], q1[4], q3[4];
                    load_blk(sK, 2, k2);
                    load_blk(sK, 3, k3);
                    load_blk(sQ, 0, q0);
                    load_blk(sQ, 1, q1);
                    load_blk(sQ, 3, q3);
                    xp[0] = cat(scale_p(0, 0, gram(kd, q0)), zero);
                    xp[1] = cat(scale_p(1, 0, gram(kd, q1)), scale_p(1, 1, gram(kn, q1)));
                    xp[2] = cat(scale_p(3, 2, gram(k2, q3)), scale_p(3, 3, gram(k3, q3)));
                } else {
                    bf16x8 k0[4], k1[4], q2[4], q3[4];
                    load_blk(sK, 0, k0);
                    load_blk(sK, 1, k1);
                    load_blk(sQ, 2, q2);
                    load_blk(sQ, 3, q3);
                    xp[0] = cat(scale_p(2, 0, gram(k0, q2)), scale_p(2, 1, gram(k1, q2)));
                    xp[1] = cat(scale_p(2, 2, gram(kd, q2)), zero);
                    xp[2] = cat(scale_p(3, 0, gram(k0, q3)), scale_p(3, 1, gram(k1, q3)));
                }
                const float dn = sRk[ln] * exp2_hw(sG[C - 1] - sG[ln]);
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const int idx = b == 0 ? (u == 2 ? 5 : u) : 2 + u;
                    opP[idx * 64 + ln] = to_bf16(xp[u]);
                }
                if (b == 1) sDn[ln] = dn;
            }
            return;
            }
            // wait for T_00 and T_11 of this chunk (bounded: the solving wave writes them
            // unconditionally; a wait that gave up poisons the block with NaN)
            bool handed = false;
            for (int spin = 0; spin < (1 << 22); ++spin) {
                if (__hip_atomic_load(flag + b, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) > c) {
                    handed = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            // T_00 in accumulator form (element e at lane (g, j) = T[4 g + e][j]) and T_00^T, T_11^T
            // (element e at lane (g, j) = T[j][4 g + e])
            const float *T0 = Tdiag + b * 2 * DSTR, *T1 = T0 + DSTR;
            f32x4 T00, Tt00, Tt11;
#pragma unroll
            for (int e = 0; e < 4; ++e) T00[e] = T0[BR * (4 * lqq + e) + lrr];
            Tt00 = *reinterpret_cast<const f32x4 *>(T0 + BR * lrr + 4 * lqq);
            Tt11 = *reinterpret_cast<const f32x4 *>(T1 + BR * lrr + 4 * lqq);
            if (!handed) {
                const f32x4 nan4 = {NAN, NAN, NAN, NAN};
                T00 = nan4;
                Tt00 = nan4;
                Tt11 = nan4;
            }
            bf16x4 ah, al, th, tl;
            hl(At, ah, al);
            hl(T00, th, tl);
            const f32x4 W = prod3(ah, al, th, tl, zero);  // A_10 T_00
            // T_10^T = -(T_11 W)^T = -W^T T_11^T
            bf16x4 wh, wl;
            hl(W, wh, wl);
            hl(Tt11, th, tl);
            const f32x4 T10t = -prod3(wh, wl, th, tl, zero);
            put_t(0, Tt00, zero);
            put_t(1, T10t, Tt11);
        }
    };

    // One period per chunk, closed by one workgroup barrier: while the column waves finish
    // chunk c and start chunk c + 1, the Gram waves build the operands of chunk c + 1 and
    // stage chunk c + 2 (its rows, norms and gates).  The staging sits between the head and
    // the merge of the build, so the merging waves wait for the solved 16-blocks while doing
    // useful work.  Wave 3 forms the gates of chunk c + 2 before the prefetch of chunk c + 3
    // replaces them in its registers.
    auto period = [&](int x) GDN_INLINE {  // build chunk x, stage chunk x + 1
        build_operands(x, 0);
        if (gwu == 3 && x + 1 < nchunks) chunk_scalars(x + 1);
        if (x + 1 < nchunks) {
            stage_chunk(x + 1);
            if (x + 2 < nchunks) prefetch_qk(x + 2);
        }
        build_operands(x, 1);
    };
    prefetch_qk(0);
    stage_chunk(0);
    if (gwu == 3) chunk_scalars(0);
    if (nchunks > 1) prefetch_qk(1);
    __syncthreads();  // chunk 0 staged
    period(0);
    __syncthreads();  // operands of chunk 0 built, chunk 1 staged
    for (int c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) period(c + 1);
        __syncthreads();
    }
#undef GDN_CHUNK
}

}  // namespace

bool prefill_chunked_supported(int dk, int dv, bool bf16) { return bf16 && dk == DK && dv % DVS == 0; }

hipError_t launch_prefill_chunked(const PrefillArgs &a, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    const int rep = a.HV / a.HQK;
    const int mode = a.split.mode;
    const int ns = mode == 0 ? 0 : a.split.ns;
    if (mode != 0 && (a.split.P < 3 || a.split.w0 < 1 || ns < 1 || ns > a.N)) return hipErrorInvalidValue;
    const int PS = mode == 1 ? a.split.P - 2 : (mode == 2 ? a.split.P - 1 : 1);
    const int nfirst = mode == 0 ? a.narrow : 0;  // narrow sequences (unsplit)
    if (nfirst < 0 || nfirst > a.N) return hipErrorInvalidValue;
    // part 0: the narrow sequences (unsplit) or the split ranks' segment 0 (map pass); part 1:
    // the split ranks' segment maps; part 2, 64-column workgroups: the other sequences, or the
    // split ranks' segments 1 .. P-1 (segment pass)
    const int64_t NG0 = mode == 0 ? (int64_t)nfirst * a.HQK : (mode == 1 ? (int64_t)ns * a.HQK : 0);
    const int64_t M0 = (int64_t)rep * (a.dv / (mode == 0 ? DVS / 2 : DVS));
    const int64_t NG1 = mode == 1 ? (int64_t)ns * PS * a.HQK : 0;
    const int64_t M1 = (int64_t)rep * ((a.dv + DK) / DVS);
    const int64_t NG = mode == 0 ? (int64_t)(a.N - nfirst) * a.HQK
                                 : (mode == 1 ? (int64_t)(a.N - ns) * a.HQK : (int64_t)ns * PS * a.HQK);
    const int64_t M = (int64_t)rep * (a.dv / DVS);
    const int64_t nwg = 8 * M0 * ((NG0 + 7) / 8) + 8 * M1 * ((NG1 + 7) / 8) + 8 * M * ((NG + 7) / 8);
    if (nwg > 0x7fffffffLL || NG > 0x7fffffffLL || NG0 > 0x7fffffffLL || NG1 > 0x7fffffffLL)
        return hipErrorInvalidValue;
    auto kern = a.split.mode != 0 ? (a.delta ? prefill_chunked_kernel<true, true> : prefill_chunked_kernel<false, true>)
                                  : (a.delta ? prefill_chunked_kernel<true, false> : prefill_chunked_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg),
                       dim3(NT), 0, stream,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                       static_cast<const uint16_t *>(a.v), a.g, a.beta, a.cu_seqlens, a.order, a.span(),
                       a.S0, static_cast<uint16_t *>(a.o), a.S_T, a.HV, a.dv, rep, (int)NG, (int)M, nfirst, a.scale, a.gate,
                       a.split);
    return hipGetLastError();
}

}  // namespace gdn
