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
// One workgroup per (split sequence, V head, 8 columns of dv): columns of the table evolve
// independently, so a column block chains on its own.  Per step it stages M (128 x 128
// fp32, rows padded to 132 floats so that 16 rows read in one wave fall in distinct
// banks) in LDS, the next step's M already on its way in registers; each thread forms
// 4 columns of one row of M S + B with fp32 FMAs.
#include "common.hpp"
#include "kernels.hpp"

namespace gdn {

namespace {

constexpr int SDK = 128;      // dk of the chunked path
constexpr int SLM = SDK + 4;  // padded LDS row of M
constexpr int SCB = 8;        // columns per workgroup

__global__ __launch_bounds__(256) void split_chain_kernel(const float *__restrict__ maps, float *__restrict__ starts,
                                                          int P, int HV, int DV) {
    __shared__ __attribute__((aligned(16))) float Ms[SDK * SLM];
    __shared__ __attribute__((aligned(16))) float Sb[SDK * SCB];
    const int unit = blockIdx.x;  // rank * HV + h
    const int n = unit / HV, h = unit % HV;
    const int c0 = blockIdx.y * SCB;
    const int DW = DV + SDK;
    const int tid = threadIdx.x;
    const int c4 = tid & 1, r = tid >> 1;  // columns c0 + 4 c4 .. + 3 of row r

    // start table of segment j (1 .. P-1) and map of segment j (1 .. P-2)
    auto sin_at = [&](int j) { return starts + ((size_t)(n * (P - 1) + j - 1) * HV + h) * SDK * DV; };
    auto map_at = [&](int j) { return maps + ((size_t)(n * (P - 2) + j - 1) * HV + h) * SDK * DW; };
    // segment 1 starts where the map pass's scan of segment 0 ended
    for (int idx = tid; idx < SDK * SCB; idx += 256) {
        const int row = idx / SCB, col = idx % SCB;
        Sb[idx] = sin_at(1)[(size_t)row * DV + c0 + col];
    }
    // M of the next step is loaded into registers while this step computes (16 float4 per
    // thread), then stored to LDS once every thread is done reading the current one.
    constexpr int NLD = SDK * SDK / 4 / 256;
    f32x4 mreg[NLD];
    auto load_m = [&](int j) {
        const float *map = map_at(j);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int f = tid + 256 * i;
            const int rr = f / (SDK / 4), kq = f % (SDK / 4);
            mreg[i] = *reinterpret_cast<const f32x4 *>(map + (size_t)rr * DW + DV + 4 * kq);
        }
    };
    auto store_m = [&]() {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int f = tid + 256 * i;
            const int rr = f / (SDK / 4), kq = f % (SDK / 4);
            *reinterpret_cast<f32x4 *>(&Ms[rr * SLM + 4 * kq]) = mreg[i];
        }
    };
    if (P > 2) load_m(1);
    for (int j = 1; j + 1 < P; ++j) {
        const float *map = map_at(j);
        __syncthreads();  // Sb holds S_in(j); every read of Ms is done
        store_m();
        __syncthreads();
        if (j + 2 < P) load_m(j + 1);
        f32x4 acc = *reinterpret_cast<const f32x4 *>(map + (size_t)r * DW + c0 + 4 * c4);
        for (int k = 0; k < SDK; k += 4) {
            const f32x4 m0 = *reinterpret_cast<const f32x4 *>(&Ms[r * SLM + k]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const f32x4 sv = *reinterpret_cast<const f32x4 *>(&Sb[(k + kk) * SCB + 4 * c4]);
                acc += m0[kk] * sv;
            }
        }
        __syncthreads();  // every read of Sb done
        *reinterpret_cast<f32x4 *>(&Sb[r * SCB + 4 * c4]) = acc;
        *reinterpret_cast<f32x4 *>(sin_at(j + 1) + (size_t)r * DV + c0 + 4 * c4) = acc;
    }
}

}  // namespace

hipError_t launch_split_chain(const float *maps, float *starts, int32_t ns, int32_t P, int32_t HV, int32_t dv,
                              hipStream_t stream) {
    if (ns == 0 || P < 3) return hipSuccess;
    if (dv % SCB != 0 || (int64_t)ns * HV > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(split_chain_kernel, dim3((unsigned)(ns * HV), (unsigned)(dv / SCB)), dim3(256), 0, stream,
                       maps, starts, P, HV, dv);
    return hipGetLastError();
}

}  // namespace gdn
