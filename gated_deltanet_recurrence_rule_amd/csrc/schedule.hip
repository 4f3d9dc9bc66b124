// schedule.hip -- longest-first order of the sequences of a packed batch.
//
// The prefill kernels give each (sequence, head, column slice) one workgroup and run
// every sequence to its end, so a batch takes as long as its longest sequence plus the
// work queued before it.  Launching the longest sequences first lets the short ones
// fill the machine behind them.  rank(i) = #{j : len_j > len_i} + #{j < i : len_j == len_i}
// is a permutation for any lengths whatsoever; order[rank(i)] = i.  The entries of cu_seqlens
// are read as they are (no clamping): an inconsistent array changes only the order, and the
// scan kernels clamp every entry they use.  Lengths are formed in 64 bits, so no pair of int32
// entries overflows.
#include "kernels.hpp"

namespace gdn {

namespace {

constexpr int RANK_THREADS = 256;
constexpr int RANK_TILE = 1024;

__global__ __launch_bounds__(RANK_THREADS) void rank_kernel(const int32_t *__restrict__ cu, int32_t N,
                                                            int32_t *__restrict__ order) {
    __shared__ int64_t tile[RANK_TILE];
    const int i = blockIdx.x * RANK_THREADS + threadIdx.x;
    const int64_t li = i < N ? (int64_t)cu[i + 1] - cu[i] : 0;
    int32_t rank = 0;
    for (int base = 0; base < N; base += RANK_TILE) {
        const int n = N - base < RANK_TILE ? N - base : RANK_TILE;
        __syncthreads();
        for (int t = threadIdx.x; t < n; t += RANK_THREADS) tile[t] = (int64_t)cu[base + t + 1] - cu[base + t];
        __syncthreads();
        if (i < N)
            for (int t = 0; t < n; ++t) {
                const int64_t lj = tile[t];
                rank += (lj > li) || (lj == li && base + t < i);
            }
    }
    if (i < N) order[rank] = i;
}

}  // namespace

hipError_t launch_longest_first(const int32_t *cu_seqlens, int32_t N, int32_t *order, hipStream_t stream) {
    if (N <= 1) return hipSuccess;
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)((N + RANK_THREADS - 1) / RANK_THREADS)), dim3(RANK_THREADS), 0,
                       stream, cu_seqlens, N, order);
    return hipGetLastError();
}

}  // namespace gdn
