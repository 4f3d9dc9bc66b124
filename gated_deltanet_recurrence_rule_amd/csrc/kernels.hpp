// kernels.hpp -- host-side launchers of the libgdn kernels (internal, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Arguments shared by the launchers, already validated by the C-ABI layer.
// g == nullptr means a = 1 (no decay); beta == nullptr means b = 1; delta == 0 drops the
// look-up (the write is b v instead of b (v - a S^T k)).
struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float *S;
    void *o;
    int32_t N, HQK, HV, dk, dv;
    float scale;
    int32_t delta;
};

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu_seqlens;  // device, or nullptr => equal lengths eq_len
    const int32_t *order;       // device: sequence of each launch rank, or nullptr => identity
    int64_t eq_len;
    int32_t N;
    int64_t total_T;
    const float *S0;
    void *o;
    float *S_T;
    int32_t HQK, HV, dk, dv;
    float scale;
    void *workspace;
    size_t workspace_bytes;
    int32_t delta;
};

// Each returns hipSuccess or the launch error.  `bf16` selects the I/O type.
hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_prefill_recurrent(const PrefillArgs &a, bool bf16, hipStream_t stream);

// Longest-first order of the N sequences of cu_seqlens (device) into order[N] (device).
hipError_t launch_longest_first(const int32_t *cu_seqlens, int32_t N, int32_t *order, hipStream_t stream);
// Sequences whose order costs O(N^2) work at most this large are reordered.
constexpr int32_t kMaxOrderedSequences = 16384;

// Chunked MFMA prefill: bf16 I/O, dk = 128, dv a multiple of 64.
bool prefill_chunked_supported(int dk, int dv, bool bf16);
hipError_t launch_prefill_chunked(const PrefillArgs &a, hipStream_t stream);

}  // namespace gdn
