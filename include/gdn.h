/*
 * gdn.h -- C ABI of libgdn, the gated delta-rule scan on MI355X (gfx950).
 *
 * The operation (handbook page "7. Gated DeltaNet: the token-by-token
 * recurrence", section "The formula", and the figure "one step of the delta
 * rule"): each V head keeps a dk x dv fp32 memory table S.  Every token t,
 * with unit-normalised key k_t and query q_t, decay alpha_t = exp(g_t) and
 * write strength beta_t, does
 *
 *     S_t = alpha_t S_{t-1} + beta_t k_t (v_t - alpha_t S_{t-1}^T k_t)^T
 *     o_t = S_t^T (scale * q_t)
 *
 * i.e. decay the table, look k_t up, write beta times the difference into k_t's
 * row, read with q_t.  The learn-llm page 13_linear_attention_viz states the
 * same rule transposed (its update-rule table, Gated DeltaNet row); this
 * library uses the handbook's orientation: S is [dk, dv], dv contiguous.
 *
 * Normalisation is done inside the library: q and k are divided by
 * max(|x|_2, 1e-12) per (token, QK head) before use (the handbook's
 * "Why are q and k normalized to unit length first?").  `scale` multiplies the
 * normalised query; the handbook's listing uses 1/sqrt(dk), its formula uses 1.
 *
 * Head sharing: V head h reads QK head h / (HV / HQK) (the repeat_interleave of
 * the handbook's qwen/deltanet.py listing).  g and beta are per V head.
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers to contiguous row-major arrays (last
 *    index fastest), 16-byte aligned, owned by the caller.  g and beta need
 *    4-byte alignment, cu_seqlens 4-byte alignment.
 *  - q, k, v and o share one element type (gdn_dtype).  g, beta, S, S0 and S_T
 *    are always fp32 (the handbook keeps the table in fp32 because bf16 cannot
 *    hold hundreds of accumulated steps).
 *  - dk and dv must each be 32, 64 or 128.  HV must be a multiple of HQK.
 *  - Calls are asynchronous: work is enqueued on `stream` and the call returns.
 *    Outputs are valid after the stream is synchronised; inputs must not change
 *    before that.  The library allocates no device memory and keeps no state
 *    between calls other than a per-device property cache.
 *  - Every argument is checked before anything is enqueued.  On any error the
 *    call returns a negative gdn_status, enqueues nothing and writes nothing;
 *    gdn_last_error() then gives a message (thread-local).
 *  - Values are not checked: g <= 0 and 0 <= beta <= 1 are the caller's contract
 *    (alpha = exp(g) in (0, 1]); NaN and Inf propagate through the arithmetic.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL                           */
    GDN_ERR_SHAPE = -2,       /* negative size, HV % HQK != 0, mismatched lengths      */
    GDN_ERR_DTYPE = -3,       /* unknown gdn_dtype                                     */
    GDN_ERR_UNSUPPORTED = -4, /* dk or dv not in {32, 64, 128}, an unknown variant, or a
                                 decay gate form with a variant that has no decay      */
    GDN_ERR_ALIGN = -5,       /* a pointer breaks the alignment rule above             */
    GDN_ERR_SEQLENS = -6,     /* cu_seqlens_host malformed, or N does not divide T     */
    GDN_ERR_WORKSPACE = -7,   /* workspace smaller than gdn_prefill_workspace_size()   */
    GDN_ERR_HIP = -8,         /* the HIP runtime reported an error at launch           */
    GDN_ERR_ALIAS = -9,       /* an output overlaps another buffer it must not (below) */
    GDN_ERR_VALUE = -10       /* a scalar argument out of range (e.g. norm_eps < 0)    */
} gdn_status;

typedef enum {
    GDN_BF16 = 0, /* q, k, v, o are bfloat16; o is rounded to nearest even */
    GDN_F32 = 1,  /* q, k, v, o are float32                                */
    /* Range sentinels, never valid arguments: they make every int32 value a value of the
     * type in C++ as well, so an out-of-range argument from C is a defined value that the
     * library rejects with GDN_ERR_DTYPE. */
    GDN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    GDN_DTYPE_RANGE_MAX_ = 2147483647
} gdn_dtype;

/*
 * gdn_variant -- the update rules of the learn-llm page 13_linear_attention_viz
 * (its update-rule table), stated here in the handbook's orientation (S is
 * [dk, dv], o = S^T q).  The library's q, k normalisation and `scale` apply to
 * every variant.
 *
 *   GDN_GATED_DELTA   S <- a S + b k (v - a S^T k)^T   Gated DeltaNet (the default)
 *   GDN_DELTA         S <- S + b k (v - S^T k)^T       DeltaNet: a = 1; g is ignored
 *                                                      and may be NULL
 *   GDN_GATED_LINEAR  S <- a S + b k v^T               Mamba2-style decayed linear
 *                                                      attention: no look-up
 *   GDN_LINEAR        S <- S + b k v^T                 linear attention: a = 1, no look-up
 *
 * The two linear rules of that table carry no write strength: they accept
 * beta == NULL, meaning b = 1.
 */
typedef enum {
    GDN_GATED_DELTA = 0,
    GDN_DELTA = 1,
    GDN_GATED_LINEAR = 2,
    GDN_LINEAR = 3,
    /* range sentinels, never valid arguments (as for gdn_dtype): GDN_ERR_UNSUPPORTED */
    GDN_VARIANT_RANGE_MIN_ = -2147483647 - 1,
    GDN_VARIANT_RANGE_MAX_ = 2147483647
} gdn_variant;

/*
 * gdn_decode_step -- advance every sequence and V head by one token, in place.
 * (The handbook's delta_rule with one token and a kept table; its chapter
 * notes that the table is carried from call to call.)
 *
 *   q, k   [N, HQK, dk]      dtype      this token's query and key (any norm)
 *   v      [N, HV, dv]       dtype      this token's value
 *   g      [N, HV]           fp32       log-decay (alpha = exp(g))
 *   beta   [N, HV]           fp32       write strength
 *   S      [N, HV, dk, dv]   fp32       in: S_{t-1}; out: S_t (updated in place)
 *   o      [N, HV, dv]       dtype      out: S_t^T (scale * q^)
 *
 * N = 0 is a valid no-op.  S and o are outputs: each must be disjoint from the other and
 * from every input (q, k, v, g, beta and the gdn_block_ops arrays of the _ex form), else
 * GDN_ERR_ALIAS.  Inputs may overlap one another (they are only read).
 */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *S, void *o, int32_t N, int32_t HQK,
                           int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                           hipStream_t stream);

/* gdn_decode_step with an update rule other than the default (see gdn_variant);
 * g may be NULL for GDN_DELTA and GDN_LINEAR, beta for GDN_GATED_LINEAR and GDN_LINEAR. */
gdn_status gdn_decode_step_v(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *S, void *o, int32_t N, int32_t HQK,
                             int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                             gdn_variant variant, hipStream_t stream);

/*
 * gdn_prefill_workspace_size -- bytes of device workspace gdn_prefill needs for
 * these sizes on the current device (0 means the workspace pointer may be NULL).
 * Two parts, each rounded to 256 bytes:
 *  - the launch order of the sequences (one int32 each); none for N <= 1 and for
 *    N above 16384 (such batches run in the given order);
 *  - for a batch the chunked kernel runs (bf16, dk = 128, dv a multiple of 64) whose
 *    (sequence, V head, 64-column) workgroups fill at most half the device's compute
 *    units, and where a model of the time in chunk periods says it pays (by 3% or more):
 *    each sequence is cut into P segments, 3 <= P <= 16, the first w0 times as long as
 *    each of the others.  The recurrence is affine in the table a segment starts from,
 *    S_out = M S_in + B (handbook page "7. Gated DeltaNet: the token-by-token recurrence",
 *    section "The formula"): the library scans segment 0 from S0 while it forms the
 *    [B | M] of segments 1 .. P-2, chains them into the start tables of segments 2 .. P-1,
 *    then runs segments 1 .. P-1 at once.  This part holds
 *    N (P-2) HV dk (dv + dk) + N (P-1) HV dk dv floats (22 MiB for one 8192-token sequence
 *    with 16 heads of d = 128 on a 256-compute-unit device, P = 9).
 * The size depends on the current device's compute-unit count: query it with the
 * device current that gdn_prefill will run on.
 */
size_t gdn_prefill_workspace_size(int32_t N, int64_t total_T, int32_t HQK, int32_t HV,
                                  int32_t dk, int32_t dv, gdn_dtype dtype);

/*
 * gdn_prefill_workspace_size_lens -- the workspace for a packed batch whose host lengths are
 * known (cu_seqlens_host, N + 1 int32 entries, read during the call only; NULL gives
 * gdn_prefill_workspace_size).  At least gdn_prefill_workspace_size; more where the batch,
 * unsplit by its sizes, has sequences that would outlast the rest (the 262144-token sequence
 * of a 65-sequence batch, two long prompts among short ones): a model of the time in chunk
 * periods may then cut its k longest sequences (1 <= k <= 8) into P segments as above.  Their
 * first segments are scanned while the other sequences run whole, beside the maps of their
 * middle segments.  The extra part holds k (P-2) HV dk (dv + dk) + k (P-1) HV dk dv floats
 * (20 MiB for that 65-sequence batch with 32 heads of d = 128: k = 1, P = 5).  gdn_prefill, given the host lengths and a workspace of this size, takes
 * that plan; given a smaller one of at least gdn_prefill_workspace_size bytes, it runs the
 * batch unsplit, with the same results to rounding.  Launch order longest first is assumed:
 * batches of more than 16384 sequences qualify only with non-increasing lengths.
 */
size_t gdn_prefill_workspace_size_lens(int32_t N, int64_t total_T, const int32_t *cu_seqlens_host, int32_t HQK,
                                       int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype);

/*
 * gdn_prefill -- run whole sequences of a packed batch (the handbook's
 * delta_rule(q, k, v, g, beta, S) -> (out, S) over a batch of sequences).
 *
 *   q, k        [total_T, HQK, dk]  dtype  tokens of all sequences, packed
 *   v           [total_T, HV, dv]   dtype
 *   g, beta     [total_T, HV]       fp32
 *   cu_seqlens  [N + 1] int32, device: sequence i owns tokens
 *               [cu_seqlens[i], cu_seqlens[i+1]); cu[0] = 0, non-decreasing,
 *               cu[N] = total_T.  Empty sequences are allowed.  NULL means N
 *               equal sequences of total_T / N tokens (N must divide total_T).
 *   cu_seqlens_host  optional host copy of the same array.  When given it is
 *               validated (GDN_ERR_SEQLENS); when NULL the device array is not
 *               validated, but the kernels clamp every entry they read into
 *               [0, total_T] (and each sequence's end to at least its start), so
 *               no contents of it can make them access memory outside the
 *               buffers; the results for an inconsistent array are unspecified.
 *               Sequences are launched longest first: unless the host copy shows
 *               lengths that never increase, a small ranking kernel writes the
 *               order into the workspace ahead of the scan (same stream).  A HIP
 *               error at the scan's launch is then reported as GDN_ERR_HIP after
 *               the ranking kernel (which writes only the workspace) is enqueued.
 *   S0          [N, HV, dk, dv] fp32 start tables, or NULL for empty tables
 *   o           [total_T, HV, dv] dtype, out: per-token reads
 *   S_T         [N, HV, dk, dv] fp32, out: final tables, or NULL to skip.
 *               S_T may be the same pointer as S0 (in-place carry).
 *   workspace   device scratch of at least gdn_prefill_workspace_size() bytes,
 *               16-byte aligned (may be NULL when that size is 0).  With the host
 *               lengths given and workspace_bytes at least
 *               gdn_prefill_workspace_size_lens(), a batch with one sequence that
 *               would outlast the rest may run with that sequence split.
 *
 * Overlaps: o, S_T and the workspace (all workspace_bytes of it) are written, so each
 * must be disjoint from the others and from every input (q, k, v, g, beta, S0,
 * cu_seqlens and the gdn_block_ops arrays of the _ex form) -- except that S_T may be
 * exactly S0.  Any other overlap is GDN_ERR_ALIAS.  Inputs may overlap one another.
 *
 * N = 0 is a valid no-op.
 */
gdn_status gdn_prefill(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const int32_t *cu_seqlens,
                       const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                       const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV, int32_t dk,
                       int32_t dv, gdn_dtype dtype, float scale, void *workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* gdn_prefill with an update rule other than the default (see gdn_variant);
 * g may be NULL for GDN_DELTA and GDN_LINEAR, beta for GDN_GATED_LINEAR and GDN_LINEAR.
 * Without the look-up (the linear rules) the chunked kernel skips the triangular solve. */
gdn_status gdn_prefill_v(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                         const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV, int32_t dk,
                         int32_t dv, gdn_dtype dtype, float scale, gdn_variant variant, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_block_ops -- optional parts of the GatedDeltaNet block run together with the scan
 * by gdn_decode_step_ex / gdn_prefill_ex (handbook page "7. Gated DeltaNet: the
 * token-by-token recurrence": the block's forward listing and the table of its parts).
 * Zero-initialise, then set what is wanted; a NULL gdn_block_ops pointer means none.
 *
 * Gates from the raw projections (parts table, rows "in_proj_b -> sigmoid" and
 * "in_proj_a, dt_bias, A_log"), computed in the scan kernels instead of a separate pass:
 *   A_log       [HV] fp32 or NULL.  Non-NULL: the g array holds the raw decay projection a
 *               and the log-decay used is  g = -exp(A_log[h]) * softplus(a + dt_bias[h])
 *               (always <= 0).  Only for the gated variants (g is read); else
 *               GDN_ERR_UNSUPPORTED.
 *   dt_bias     [HV] fp32, or NULL for zeros: the bias added to a (both decay forms).
 *   alpha_sigmoid  non-zero: the other decay form, that of the learn-llm page
 *               13_linear_attention_viz (its RecurrentMixer computes alpha from an a
 *               projection with a bias): the g array holds the raw a and the decay is
 *               alpha = sigmoid(a + dt_bias[h]), i.e. g = log sigmoid(a + dt_bias[h]).
 *               Gated variants only (GDN_ERR_UNSUPPORTED); excludes A_log (GDN_ERR_VALUE).
 *   beta_logits non-zero: the beta array holds the raw projection b and the write strength
 *               used is sigmoid(b).  Needs a non-NULL beta (GDN_ERR_NULL).
 *
 * Gated RMS norm of the read (parts table, row "in_proj_z + GatedRMSNorm"; its body is not
 * on the page -- the reading taken is y = w * o / sqrt(mean_j o_j^2 + eps) * silu(z) over
 * each (token, V head) vector of dv values):
 *   z           output gate, same shape and element type as o, 16-byte aligned, or NULL
 *               for no norm.  Non-NULL: o receives y instead of the raw read.
 *   norm_w      [dv] fp32 weight, shared by all heads; required with z.
 *   norm_eps    >= 0 (GDN_ERR_VALUE otherwise).
 * Decode normalises the fp32 read before its one rounding.  Prefill runs the scan, then
 * the norm kernel (gdn_gated_rmsnorm) in place on o: for bf16 the read is rounded once
 * before the norm (the chunked kernel spreads a head's dv columns over workgroups, so no
 * workgroup holds a whole vector).
 */
typedef struct gdn_block_ops {
    const float *A_log;
    const float *dt_bias;
    int32_t beta_logits;
    const void *z;
    const float *norm_w;
    float norm_eps;
    int32_t alpha_sigmoid;
} gdn_block_ops;

/* gdn_decode_step_v plus the block parts in `ops` (may be NULL). */
gdn_status gdn_decode_step_ex(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, float *S, void *o, int32_t N, int32_t HQK,
                              int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                              gdn_variant variant, const gdn_block_ops *ops, hipStream_t stream);

/* gdn_prefill_v plus the block parts in `ops` (may be NULL); z is [total_T, HV, dv]. */
gdn_status gdn_prefill_ex(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const int32_t *cu_seqlens,
                          const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                          const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV, int32_t dk,
                          int32_t dv, gdn_dtype dtype, float scale, gdn_variant variant,
                          const gdn_block_ops *ops, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * gdn_prefill_noalloc -- gdn_prefill_ex without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing and calls no allocating
 * routine: the workspace gdn_prefill_ex would take (launch order, and for small batches
 * the split-sequence maps and start tables) lives in a static device array of 24 MiB,
 * one per device, held from the library's load on that device until the process ends.
 * Arguments, checks, results and errors are those of gdn_prefill_ex, bit for bit, plus:
 *  - GDN_ERR_WORKSPACE when gdn_prefill_workspace_size() of these sizes exceeds 24 MiB
 *    (only split batches can: e.g. one 4096-token sequence with 32 V heads of dv = 64
 *    needs 29 MiB on a 256-compute-unit device, one 8192-token sequence with 16 heads of
 *    d = 128 needs 22 MiB);
 *  - GDN_ERR_HIP if the device address of the array cannot be obtained (taken once per
 *    device, at the first call on it, with that device current).
 * Every call on a device shares that device's array, and calls that overlap in time on
 * one device (other streams, other host threads) race on it: serialise them.  The array
 * keeps what the last call wrote; no part of it needs to start at zero.
 */
gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const int32_t *cu_seqlens,
                               const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                               const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV,
                               int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                               gdn_variant variant, const gdn_block_ops *ops, hipStream_t stream);

/*
 * gdn_conv_silu -- the block's causal depthwise short convolution + SiLU, in front of the
 * scan (handbook page "7. Gated DeltaNet: the token-by-token recurrence": the block listing
 * and the parts table, row "in_proj_qkv + conv1d", with the note under the table: the
 * output at position t uses the inputs t-3 .. t only, every channel with its own 4
 * weights).  For every token t of sequence n and channel c:
 *
 *     y[t, c] = silu( w[c, 0] e[t-3, c] + w[c, 1] e[t-2, c] + w[c, 2] e[t-1, c] + w[c, 3] x[t, c] )
 *
 * where e is the sequence's inputs preceded by its carried state (zeros without one).
 *   x          [total_T, Ctot] in dtype, Ctot = 2 HQK dk + HV dv: the concatenated q | k | v
 *              channels of each token (the block's in_proj_qkv output).
 *   w          [Ctot, 4] fp32, 16-byte aligned; w[c][3] weighs the current token.
 *   cu_seqlens, cu_seqlens_host, N, total_T: as for gdn_prefill (NULL cu_seqlens = N equal
 *              lengths; N sequences of one token each is a decode step).
 *   state_in   [N, 3, Ctot] in dtype or NULL (zeros): each sequence's three previous inputs,
 *              oldest first.
 *   state_out  [N, 3, Ctot] or NULL (not written): the last three entries of (state ++ x)
 *              for each sequence; an empty sequence passes its state through.  It may be
 *              the same buffer as state_in.
 *   q, k       [total_T, HQK, dk] and v [total_T, HV, dv] in dtype: y split into the
 *              arrays gdn_prefill and gdn_decode_step read.  fp32 arithmetic; bf16 outputs
 *              rounded once to nearest even.
 * Overlaps: q, k, v and state_out are written: each must be disjoint from the others and
 * from x, w, state_in and cu_seqlens, except that state_out may be exactly state_in
 * (GDN_ERR_ALIAS otherwise).
 * Alignment: every array 16 bytes.  Sizes: dk, dv in {32, 64, 128}, HQK, HV > 0.
 */
gdn_status gdn_conv_silu(const void *x, const float *w, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                         const void *state_in, void *state_out, void *q, void *k, void *v,
                         int32_t HQK, int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype,
                         hipStream_t stream);

/*
 * gdn_gated_rmsnorm -- the block's gated RMS norm on its own (see gdn_block_ops for the
 * formula and the reading):  y[r] = w * x[r] / sqrt(mean_j x[r, j]^2 + eps) * silu(z[r])
 * for every row r of dv values (rows = tokens x V heads).
 *   x, z, y    [rows, dv] in dtype, 16-byte aligned; y may be x (in place), a partial
 *              overlap of y with x or z is GDN_ERR_ALIAS.
 *   w          [dv] fp32.   eps >= 0.   dv in {32, 64, 128}.
 */
gdn_status gdn_gated_rmsnorm(const void *x, const void *z, const float *w, float eps, void *y,
                             int64_t rows, int32_t dv, gdn_dtype dtype, hipStream_t stream);

/*
 * gdn_prefill_kernel_name -- which kernel gdn_prefill runs for these sizes (static text, for
 * profiling and reports), with a workspace of gdn_prefill_workspace_size_lens bytes where
 * cu_seqlens_host (N + 1 int32 entries, read during the call only) is given, else of
 * gdn_prefill_workspace_size bytes:
 *   "prefill_chunked"    bf16, dk = 128, dv a multiple of 64: chunks of 64 tokens
 *                        on bf16 MFMA with an fp32 table;
 *   "prefill_chunked_split"  the same kernel over split sequences (see
 *                        gdn_prefill_workspace_size and gdn_prefill_workspace_size_lens),
 *                        plus the chaining kernel;
 *   "prefill_recurrent"  every other case: token-serial, fp32 arithmetic.
 */
const char *gdn_prefill_kernel_name(int32_t N, int64_t total_T, const int32_t *cu_seqlens_host, int32_t HQK,
                                    int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype);

/*
 * gdn_prefill_narrow_count -- how many sequences gdn_prefill runs on workgroups of 32 value
 * columns instead of 64 (informational, for profiling and tests; it changes only the speed,
 * never the outputs), with a workspace of gdn_prefill_workspace_size_lens bytes where the host
 * lengths are given.  Applies to "prefill_chunked" (not to split sequences):
 *   - every sequence, when the batch's 64-column workgroups (N x HV x dv / 64) would fill at
 *     most half the current device's compute units: twice as many still fit, and each chunk
 *     takes ~0.87 of the time on a workgroup with two column waves;
 *   - else the longest sequences, when gdn_prefill receives the host copy of cu_seqlens
 *     (cu_seqlens_host here, N + 1 int32 entries, read during the call only): a sequence that
 *     would outlast the rest of the batch runs each chunk in ~0.95 of the time on twice the
 *     workgroups while the others share the remaining units.  The rule models the batch's
 *     time in chunk periods and narrows only where that gains 3% or more.
 * total_T is the batch's token count.  Returns 0 for invalid arguments.
 */
int32_t gdn_prefill_narrow_count(int32_t N, int64_t total_T, const int32_t *cu_seqlens_host, int32_t HQK,
                                 int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype);

/* Static text for a status code. */
const char *gdn_status_str(gdn_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char *gdn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
