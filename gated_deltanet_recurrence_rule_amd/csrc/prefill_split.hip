// prefill_split.hip -- chaining the segment maps of split sequences.
//
// A sequence too short of parallel work for the chip (few sequences and heads) is cut into
// P segments of whole chunks.  The recurrence of the handbook page "7. Gated DeltaNet: the
// token-by-token recurrence" (section "The formula") is affine in the table it starts
// from, so a segment that starts from S_in ends at M S_in + B.  The chunked kernel's map
// pass scans segment 0 from S0 (its final table is segment 1's start) and gives the [B | M]
// of segments 1 .. P-2 at once; this kernel chains them, one segment after another, into the
// start tables of segments 2 .. P-1; the segment pass then runs segments 1 .. P-1 at once
// from their tables.
//
// One workgroup per (split sequence, V head, 16 columns of dv): columns of the table evolve
// independently, so a column block chains on its own.  Each step is the product M S_in on
// fp32 MFMA (16 x 16 x 4), B loaded as the accumulators' start value: wave w forms rows
// 32 w .. 32 w + 31.  M comes from memory straight into the A operands, the next two steps'
// already on their way while this one multiplies; S_in sits in LDS transposed (one padded row
// per column), double-buffered, so a step needs one barrier.  The contraction index is
// permuted: in k-step 4 q + e, lane group g (lanes 16 g .. 16 g + 15) carries
// k = 16 q + 4 g + e, so that a lane reads 4 consecutive floats of its M row (and of its
// S_in column) per load, and the four groups together 64 consecutive bytes of the row.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

constexpr int SDK = 128;      // dk of the chunked path
constexpr int SCB = 16;       // columns per workgroup
constexpr int SLT = SDK + 4;  // padded LDS row (one column of S_in)
constexpr int kMaxSplitSegments = 16;  // the planners choose P in 3 .. 16

// NS = P - 2 chain steps, fully unrolled: the maps of steps j + 1 and j + 2 are in flight
// while step j multiplies (three register sets in rotation), with no branch between a
// load and its use.
template <int NS>
__global__ __launch_bounds__(256) void split_chain_kernel(const float *maps, float *starts, int HV, int DV) {
    constexpr int P = NS + 2;
    __shared__ __attribute__((aligned(16))) float St[2][SCB * SLT];
    const int unit = blockIdx.x;  // rank * HV + h
    const int n = unit / HV, h = unit % HV;
    const int c0 = blockIdx.y * SCB;
    const int DW = DV + SDK;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;

    // start table of segment j (1 .. P-1) and map of segment j (1 .. P-2)
    auto sin_at = [&](int j) { return starts + ((size_t)(n * (P - 1) + j - 1) * HV + h) * SDK * DV; };
    auto map_at = [&](int j) { return maps + ((size_t)(n * (P - 2) + j - 1) * HV + h) * SDK * DW; };
    // Operands of one step: A = M rows 32 w + 16 b + r16, k = 16 q + 4 g + e (8 float4 per
    // row block); the accumulators start from B at rows 32 w + 16 b + 4 g + i, column c0 + r16.
    f32x4 m[3][2][8], bv[3][2];
    auto load = [&](int j) {
        const float *map = map_at(j);
        const int slot = j % 3;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float *rp = map + (size_t)(32 * w + 16 * b + r16) * DW + DV + 4 * g;
#pragma unroll
            for (int q = 0; q < 8; ++q) m[slot][b][q] = *reinterpret_cast<const f32x4 *>(rp + 16 * q);
            const float *bp = map + (size_t)(32 * w + 16 * b + 4 * g) * DW + c0 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[slot][b][i] = bp[(size_t)i * DW];
        }
    };
    load(1);
    if (NS >= 2) load(2);
    // segment 1 starts where the map pass's scan of segment 0 ended (all loads issued
    // before the first wait)
    {
        float sv[SDK * SCB / 256];
        const float *s1 = sin_at(1);
#pragma unroll
        for (int i = 0; i < SDK * SCB / 256; ++i) {
            const int idx = tid + 256 * i;
            sv[i] = s1[(size_t)(idx / SCB) * DV + c0 + idx % SCB];
        }
#pragma unroll
        for (int i = 0; i < SDK * SCB / 256; ++i) {
            const int idx = tid + 256 * i;
            St[0][(idx % SCB) * SLT + idx / SCB] = sv[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 1; j <= NS; ++j) {
        if (j + 2 <= NS) load(j + 2);
        __builtin_amdgcn_sched_barrier(0);  // the loads first, ahead of this step's products
        const int slot = j % 3;
        const float *src = St[(j - 1) & 1];
        float *dst = St[j & 1];
        f32x4 sv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) sv[q] = *reinterpret_cast<const f32x4 *>(&src[r16 * SLT + 16 * q + 4 * g]);
        // two accumulators per row block (k-steps 0..15 and 16..31): four independent chains
        f32x4 acc[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            acc[b][0] = bv[slot][b];
            acc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[b][hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(m[slot][b][q + 4 * hh][e],
                                                                         sv[q + 4 * hh][e], acc[b][hh], 0, 0, 0);
        float *out = sin_at(j + 1);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const f32x4 res = acc[b][0] + acc[b][1];
            const int row = 32 * w + 16 * b + 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) out[(size_t)(row + i) * DV + c0 + r16] = res[i];
            *reinterpret_cast<f32x4 *>(&dst[r16 * SLT + row]) = res;
        }
        __syncthreads();  // dst complete for the next step; every read of src done
    }
}

template <int NS>
void launch_chain_steps(const float *maps, float *starts, int32_t ns, int32_t P, int32_t HV, int32_t dv,
                        hipStream_t stream) {
    if constexpr (NS > 1) {
        if (P - 2 < NS) return launch_chain_steps<NS - 1>(maps, starts, ns, P, HV, dv, stream);
    }
    hipLaunchKernelGGL(split_chain_kernel<NS>, dim3((unsigned)(ns * HV), (unsigned)(dv / SCB)), dim3(256), 0, stream,
                       maps, starts, HV, dv);
}

}  // namespace

hipError_t launch_split_chain(const float *maps, float *starts, int32_t ns, int32_t P, int32_t HV, int32_t dv,
                              hipStream_t stream) {
    if (ns == 0 || P < 3) return hipSuccess;
    if (P > kMaxSplitSegments || dv % SCB != 0 || (int64_t)ns * HV > 0x7fffffffLL) return hipErrorInvalidValue;
    launch_chain_steps<kMaxSplitSegments - 2>(maps, starts, ns, P, HV, dv, stream);
    return hipGetLastError();
}

}  // namespace gdn
