// kernels.hpp -- host-side launchers of the libgdn kernels (internal, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Gates from raw projections: with A_log set, g holds the raw decay projection a and the
// log-decay is -exp(A_log[h]) softplus(a + dt_bias[h]) (dt_bias may be null = 0); with
// beta_logit set, beta holds the raw projection b and the write strength is sigmoid(b).
// With alpha_sigmoid set instead, g holds the raw a and the log-decay is
// log sigmoid(a + dt_bias[h]).
struct GateArgs {
    const float *A_log = nullptr, *dt_bias = nullptr;
    int32_t beta_logit = 0;
    int32_t alpha_sigmoid = 0;
};

// Split sequences for the chunked prefill (see prefill_chunked.hip): the first ns launch ranks
// are cut into P >= 3 segments, segment 0 w0 times as long as each of the others; mode 0 = no
// split, 1 = map pass (every sequence scanned from S0, a split rank's only through segment 0,
// whose end goes to starts; segments 1 .. P-2 of the split ranks into maps), 2 = segment pass
// (segments 1 .. P-1 of the split ranks from starts).  maps = [ns][P - 2][HV][DK][DV + DK],
// starts = [ns][P - 1][HV][DK][DV] (the start tables of segments 1 .. P-1), both by rank.
struct SplitArgs {
    int32_t P = 1;
    int32_t mode = 0;
    int32_t w0 = 1;
    int32_t ns = 0;
    float *maps = nullptr;
    float *starts = nullptr;
};

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
    GateArgs gate = {};
    // gated RMS norm of the read (z == nullptr: none): o <- w o / sqrt(mean(o^2) + eps) silu(z)
    const void *z = nullptr;
    const float *norm_w = nullptr;
    float norm_eps = 0.f;
    int32_t max_wgs = 0;  // grid cap of the persistent kernel (0: one workgroup per table)
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
    // what the kernels take for the sequence bounds: eq_len without cu_seqlens, else total_T
    // (the range every device entry is clamped into)
    int64_t span() const { return cu_seqlens ? total_T : eq_len; }
    int32_t HQK, HV, dk, dv;
    float scale;
    void *workspace;
    size_t workspace_bytes;
    int32_t delta;
    GateArgs gate = {};
    SplitArgs split = {};
    // chunked prefill without split sequences: the first `narrow` launch ranks (the longest
    // sequences) run on workgroups of 32 columns with two column waves instead of 64 with four
    int32_t narrow = 0;
};

// Gated RMS norm over rows of dv values (rows = tokens x heads; z rows alike; w [dv]):
// y = w x / sqrt(mean(x^2) + eps) silu(z).  y may equal x.
struct NormArgs {
    const void *x, *z;
    const float *w;
    void *y;
    int64_t rows;
    int32_t dv;
    float eps;
};

// Causal depthwise convolution of width 4 + SiLU over the concatenated q | k | v channels
// (Ctot = 2 HQK dk + HV dv), written out as separate q, k, v.  state_in / state_out
// [N, 3, Ctot] hold the three inputs before / at the end of each sequence (null: zeros /
// not written).  cu_seqlens as for prefill.
struct ConvArgs {
    const void *x;
    const float *w;  // [Ctot, 4], w[c][3] weighs the current token
    const int32_t *cu_seqlens;
    int64_t eq_len;
    int32_t N;
    int64_t total_T;
    const void *state_in;
    void *state_out;
    void *q, *k, *v;
    int32_t Cq, Cv;  // HQK dk, HV dv
};

// Each returns hipSuccess or the launch error.  `bf16` selects the I/O type.
hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_gated_rmsnorm(const NormArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_conv_silu(const ConvArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_prefill_recurrent(const PrefillArgs &a, bool bf16, hipStream_t stream);

// Longest-first order of the N sequences of cu_seqlens (device) into order[N] (device).
hipError_t launch_longest_first(const int32_t *cu_seqlens, int32_t N, int32_t *order, hipStream_t stream);
// Sequences whose order costs O(N^2) work at most this large are reordered.
constexpr int32_t kMaxOrderedSequences = 16384;

// Chunked MFMA prefill: bf16 I/O, dk = 128, dv a multiple of 64.
bool prefill_chunked_supported(int dk, int dv, bool bf16);
// Start tables of the ns split ranks: the map pass wrote segment 1's (starts[r][0], the end of
// segment 0); segment j + 1 starts at M_j S_in(j) + B_j with [B_j | M_j] = maps[r][j - 1],
// j = 1 .. P-2 (dk = 128).
hipError_t launch_split_chain(const float *maps, float *starts, int32_t ns, int32_t P, int32_t HV, int32_t dv,
                              hipStream_t stream);
hipError_t launch_prefill_chunked(const PrefillArgs &a, hipStream_t stream);

}  // namespace gdn
