// api.hip -- the C ABI of libgdn: argument checks, then kernel launches.
//
// Every check runs before anything is enqueued, so a failing call writes
// nothing.  The declarations and their contracts are in include/gdn.h.
#include <stdarg.h>
#include <algorithm>
#include <atomic>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "gdn.h"
#include "kernels.hpp"

// Maximum workspace of gdn_prefill_noalloc (see static_scratch below).
static constexpr size_t kStaticScratchBytes = (size_t)24 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool dim_ok(int32_t d) { return d == 32 || d == 64 || d == 128; }

// `tokens` is the number of tokens the call touches; with none, the token
// arrays may be NULL (an empty tensor has no storage).
// Which inputs a variant reads: the gated ones read g; the look-up ones need beta
// (the linear variants may pass NULL for b = 1).
bool variant_ok(gdn_variant x) { return x == GDN_GATED_DELTA || x == GDN_DELTA || x == GDN_GATED_LINEAR || x == GDN_LINEAR; }
bool variant_gated(gdn_variant x) { return x == GDN_GATED_DELTA || x == GDN_GATED_LINEAR; }
bool variant_delta(gdn_variant x) { return x == GDN_GATED_DELTA || x == GDN_DELTA; }

gdn_status check_common(const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const void *o, int32_t N, int32_t HQK, int32_t HV,
                        int32_t dk, int32_t dv, gdn_dtype dtype, int64_t tokens,
                        gdn_variant variant = GDN_GATED_DELTA) {
    if (!variant_ok(variant)) return fail(GDN_ERR_UNSUPPORTED, "unknown variant %d", (int)variant);
    if (dtype != GDN_BF16 && dtype != GDN_F32) return fail(GDN_ERR_DTYPE, "unknown dtype %d", (int)dtype);
    if (N < 0) return fail(GDN_ERR_SHAPE, "N = %d is negative", N);
    if (HQK <= 0 || HV <= 0) return fail(GDN_ERR_SHAPE, "head counts must be positive (HQK=%d, HV=%d)", HQK, HV);
    if (HV % HQK != 0) return fail(GDN_ERR_SHAPE, "HV (%d) is not a multiple of HQK (%d)", HV, HQK);
    if (!dim_ok(dk) || !dim_ok(dv))
        return fail(GDN_ERR_UNSUPPORTED, "dk=%d, dv=%d: each must be 32, 64 or 128", dk, dv);
    if (tokens == 0) return GDN_OK;
    if (!q || !k || !v || !o) return fail(GDN_ERR_NULL, "q, k, v and o must be non-NULL");
    if (variant_gated(variant) && !g) return fail(GDN_ERR_NULL, "g must be non-NULL for a gated variant");
    if (variant_delta(variant) && !beta) return fail(GDN_ERR_NULL, "beta must be non-NULL for a delta variant");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(GDN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
    if (!aligned(g, 4) || !aligned(beta, 4)) return fail(GDN_ERR_ALIGN, "g and beta must be 4-byte aligned");
    return GDN_OK;
}

// cu_seqlens rules shared by prefill and the convolution; sets eq_len when cu_seqlens is NULL.
gdn_status check_seqlens(const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int32_t N,
                         int64_t total_T, int64_t *eq_len) {
    *eq_len = 0;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(GDN_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
    if (total_T > 0x7fffffffLL) return fail(GDN_ERR_SHAPE, "total_T must fit in int32");
    if (cu_seqlens_host) {
        if (N > 0 && cu_seqlens_host[0] != 0) return fail(GDN_ERR_SEQLENS, "cu_seqlens[0] must be 0");
        for (int32_t i = 0; i < N; ++i)
            if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
                return fail(GDN_ERR_SEQLENS, "cu_seqlens decreases at %d", i);
        if (N > 0 && (int64_t)cu_seqlens_host[N] != total_T)
            return fail(GDN_ERR_SEQLENS, "cu_seqlens[N] = %d but total_T = %lld", cu_seqlens_host[N],
                        (long long)total_T);
    }
    if (!cu_seqlens) {
        if (N == 0) {
            if (total_T != 0) return fail(GDN_ERR_SEQLENS, "N = 0 with total_T = %lld", (long long)total_T);
        } else {
            if (total_T % N != 0)
                return fail(GDN_ERR_SEQLENS, "cu_seqlens is NULL and N (%d) does not divide total_T (%lld)",
                            N, (long long)total_T);
            *eq_len = total_T / N;
        }
    }
    return GDN_OK;
}

// The optional block parts: which gates they transform, and the norm's operands.
gdn_status check_ops(const gdn_block_ops *ops, gdn_variant variant, const float *beta, int64_t tokens) {
    if (!ops) return GDN_OK;
    if ((ops->A_log || ops->alpha_sigmoid) && !variant_gated(variant))
        return fail(GDN_ERR_UNSUPPORTED, "a decay gate form is set but the variant has no decay");
    if (ops->A_log && ops->alpha_sigmoid)
        return fail(GDN_ERR_VALUE, "A_log and alpha_sigmoid are two forms of the decay gate: set one");
    if (ops->z && !(ops->norm_eps >= 0.f)) return fail(GDN_ERR_VALUE, "norm_eps must be >= 0");
    if (tokens == 0) return GDN_OK;
    if (ops->beta_logits && !beta) return fail(GDN_ERR_NULL, "beta_logits needs a non-NULL beta");
    if (ops->z && !ops->norm_w) return fail(GDN_ERR_NULL, "norm_w must be non-NULL with z");
    if (!aligned(ops->A_log, 4) || !aligned(ops->dt_bias, 4) || !aligned(ops->norm_w, 4))
        return fail(GDN_ERR_ALIGN, "A_log, dt_bias and norm_w must be 4-byte aligned");
    if (!aligned(ops->z, 16)) return fail(GDN_ERR_ALIGN, "z must be 16-byte aligned");
    return GDN_OK;
}

// [a, a + na) and [b, b + nb) overlap without being the same start
bool partial_overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || a == b) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// A buffer a call reads or writes: its first byte and length (a NULL or empty one is skipped).
struct Span {
    const void *p;
    size_t n;
    const char *name;
};

bool overlaps(const Span &a, const Span &b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
    return x < y + b.n && y < x + a.n;
}

// Every output must be disjoint from every input and from every other output; the one
// exception allowed is an output that is exactly the input named `same_ok_in` (same first
// byte and length), for the outputs listed as updating that input in place.
gdn_status check_disjoint(const Span *outs, int no, const Span *ins, int ni, const char *same_ok_out = nullptr,
                          const char *same_ok_in = nullptr) {
    for (int i = 0; i < no; ++i) {
        for (int j = 0; j < ni; ++j) {
            if (!overlaps(outs[i], ins[j])) continue;
            const bool exact = outs[i].p == ins[j].p && outs[i].n == ins[j].n;
            if (exact && same_ok_out && same_ok_in && strcmp(outs[i].name, same_ok_out) == 0 &&
                strcmp(ins[j].name, same_ok_in) == 0)
                continue;
            return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[i].name, ins[j].name);
        }
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], outs[j])) return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    return GDN_OK;
}

gdn::GateArgs gate_args(const gdn_block_ops *ops, gdn_variant variant) {
    gdn::GateArgs ga;
    if (ops) {
        ga.A_log = variant_gated(variant) ? ops->A_log : nullptr;
        ga.alpha_sigmoid = (variant_gated(variant) && ops->alpha_sigmoid) ? 1 : 0;
        ga.dt_bias = (ga.A_log || ga.alpha_sigmoid) ? ops->dt_bias : nullptr;
        ga.beta_logit = ops->beta_logits ? 1 : 0;
    }
    return ga;
}

// Compute units of the current device (cached per device, safe to call from several host
// threads; 256, MI355X's count, if the runtime cannot say).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = cache[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cache[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// Split plan for the chunked prefill: the first ns launch ranks are cut into P segments (P = 1:
// no split), segment 0 w0 times as long as each of the others.
struct SplitPlan {
    int32_t P = 1, w0 = 1, ns = 0;
};

// Chain steps in chunk periods: one workgroup per (split sequence, V head, 16 columns), one per
// CU at the register count of the longer chains.  1.2 periods per step and round was measured on
// an earlier, slower chain; the current one takes ~0.8, and the plans hardly change with it.
double chain_step(int64_t ns, int32_t HV, int32_t dv, int64_t cus) {
    const int64_t wgs = ns * HV * (dv / 16);
    return 1.2 * (double)((wgs + cus - 1) / cus);
}

// The plan from the sizes alone: only a batch whose (sequence, V head, 64-column) workgroups, u
// of them, fill at most half the compute units is split, every sequence alike.  The plan
// minimises a model of the time in chunk periods, with c the average chunks per sequence:
//   unsplit, every sequence on 32-column workgroups (see narrow_sequences below): 0.87 c;
//   split: the map pass scans segment 0 on u workgroups while the maps of segments 1 .. P-2
//   (um workgroups each, the table widened by dk columns) take rm = ceil((P-2) um / (CUs - u))
//   rounds of the rest, so segment 0 gets w0 = max(1, rm) units; the segment pass takes
//   rs = ceil((P-1) u / CUs) rounds; with a = ceil(c / (P - 1 + w0)) chunks per unit the time is
//   (w0 + rs) a + 1.2 per chain step and round of its workgroups (P - 2 steps) + 3 for the two
//   extra launches and the second pipeline fill.
// A split is taken only where the model gains at least 3%.
SplitPlan split_plan(int32_t N, int64_t total_T, int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype) {
    SplitPlan best;
    if (N <= 0 || HV <= 0 || total_T <= 0 || !gdn::prefill_chunked_supported(dk, dv, dtype == GDN_BF16))
        return best;
    const int64_t cus = device_cus();
    const int64_t u = (int64_t)N * HV * (dv / 64), um = (int64_t)N * HV * ((dv + dk) / 64);
    if (2 * u > cus) return best;
    const int64_t c = (total_T + 64 * (int64_t)N - 1) / (64 * (int64_t)N);
    const double step = chain_step(N, HV, dv, cus);
    double t_best = 0.97 * 0.87 * (double)c;
    for (int32_t P = 3; P <= 16; ++P) {
        const int64_t rm = ((P - 2) * um + (cus - u) - 1) / (cus - u);
        const int64_t w0 = rm > 1 ? rm : 1;
        const int64_t rs = ((P - 1) * u + cus - 1) / cus;
        const int64_t units = P - 1 + w0;
        const int64_t a = (c + units - 1) / units;
        const double t = (double)((w0 + rs) * a) + (P - 2) * step + 3.0;
        if (t < t_best) {
            t_best = t;
            best.P = P;
            best.w0 = (int32_t)w0;
            best.ns = N;
        }
    }
    return best;
}

// Chunk counts of a packed batch from its host lengths: the largest (longest first; no heap, the
// allocation-free entry shares this) and the 64-column work of the whole batch.
struct LengthStats {
    static constexpr int kTop = 64;
    int64_t top[kTop + 1];
    int ntop = 0;
    double work = 0.0;  // sum of chunks x (HV dv / 64) workgroups
};

LengthStats length_stats(const int32_t *cu_host, int32_t N, int64_t u) {
    LengthStats ls;
    for (int32_t i = 0; i < N; ++i) {
        const int64_t len = (int64_t)cu_host[i + 1] - cu_host[i];
        const int64_t x = len > 0 ? (len + 63) / 64 : 0;
        ls.work += (double)x * (double)u;
        int j;
        if (ls.ntop < LengthStats::kTop + 1) {
            j = ls.ntop++;
        } else {
            if (x <= ls.top[LengthStats::kTop]) continue;  // not among the largest
            j = LengthStats::kTop;
        }
        while (j > 0 && ls.top[j - 1] < x) {
            ls.top[j] = ls.top[j - 1];
            --j;
        }
        ls.top[j] = x;
    }
    return ls;
}

// How many of the longest sequences run on 32-column workgroups (chunked prefill without split
// sequences; host lengths needed), and the modelled time in chunk periods.  Such a workgroup has
// two column waves instead of four and takes ~0.87 of the time per chunk when every compute
// unit runs the kernel, ~0.95 beside the rest of a packed batch (both measured on MI355X; the
// model takes 0.95), so a sequence that would outlast the rest of the batch finishes sooner on
// twice the workgroups while the others share the remaining compute units.  The n longest are
// narrowed for the n that minimises
//   max(0.95 c_0, c_n, rest / (CUs - 2 n u)),  u = HV dv / 64 workgroups per sequence,
// c_i the chunk counts longest first and rest the 64-column work of the others, provided the
// narrow workgroups use at most half the units and the model gains at least 3% over
// max(c_0, work / CUs).
int32_t narrow_sequences(const LengthStats &ls, int32_t N, int64_t u, int64_t cus, double *t_out) {
    const double wide = std::max((double)ls.top[0], ls.work / (double)cus);
    double best = wide, rest = ls.work;
    int32_t n_best = 0;
    for (int32_t n = 1; n <= N && n <= LengthStats::kTop && 4 * n * u <= cus; ++n) {
        rest -= (double)ls.top[n - 1] * (double)u;
        const double longest_wide = n < ls.ntop ? (double)ls.top[n] : 0.0;
        const double t = std::max(std::max(0.95 * (double)ls.top[0], longest_wide), rest / (double)(cus - 2 * n * u));
        if (t < best) {
            best = t;
            n_best = n;
        }
    }
    if (best > 0.97 * wide) {
        best = wide;
        n_best = 0;
    }
    if (t_out) *t_out = best;
    return n_best;
}

// Sequences on 32-column workgroups for an unsplit chunked prefill: all of them when their
// 64-column workgroups would fill at most half the compute units (twice as many still fit),
// else the host rule above, which needs the host lengths and a longest-first launch order.
int32_t narrow_for_batch(int32_t N, int32_t HV, int32_t dv, const int32_t *cu_host, bool longest_first) {
    const int64_t cus = device_cus();
    const int64_t u = (int64_t)HV * (dv / 64);
    if ((int64_t)N * u * 2 <= cus) return N;
    if (!cu_host || !longest_first || N <= 0 || u <= 0) return 0;
    return narrow_sequences(length_stats(cu_host, N, u), N, u, cus, nullptr);
}

// The k longest sequences of a packed batch cut into segments (ns = k, 1 <= k <= 8), for the batch
// the sizes alone leave unsplit, when its host lengths are known and the launch order is longest
// first.  With c_0 >= c_1 >= ... the chunk counts, u (um) a sequence's 64-column workgroups (with
// dk extra columns), a_i = ceil(c_i / (P - 1 + w0)) and rest the unsplit sequences' work, the
// model is
//   map pass:     max(w0 a_0, c_k, (rest + sum_i<k (P-2) um a_i) / (CUs - k u))
//                 (the segments 0 on k u units; the maps and the unsplit sequences on the rest),
//   segment pass: ceil(k (P-1) u / CUs) a_0,
// plus the chain and the fixed 3 as above.  Taken where it gains 3% over the unsplit plan.
SplitPlan split_longest(const LengthStats &ls, int32_t N, int32_t HV, int32_t dk, int32_t dv, int64_t cus,
                        double t_unsplit) {
    SplitPlan best;
    const int64_t u = (int64_t)HV * (dv / 64), um = (int64_t)HV * ((dv + dk) / 64);
    if (u <= 0 || 2 * u > cus) return best;
    double t_best = 0.97 * t_unsplit;
    double rest = ls.work;
    for (int32_t k = 1; k <= 8 && k <= N && k <= ls.ntop && k * u < cus; ++k) {
        rest -= (double)ls.top[k - 1] * (double)u;
        const double ck = k < ls.ntop ? (double)ls.top[k] : 0.0;
        const double step = chain_step(k, HV, dv, cus);
        for (int32_t P = 3; P <= 16; ++P)
            for (int32_t w0 = 1; w0 <= 16; ++w0) {
                const int64_t units = P - 1 + w0;
                int64_t maps = 0;
                for (int32_t i = 0; i < k; ++i) maps += (P - 2) * um * ((ls.top[i] + units - 1) / units);
                const int64_t a0 = (ls.top[0] + units - 1) / units;
                const double pass1 = std::max(std::max((double)(w0 * a0), ck),
                                              (rest + (double)maps) / (double)(cus - k * u));
                const double pass2 = (double)((((int64_t)k * (P - 1) * u + cus - 1) / cus) * a0);
                const double t = pass1 + pass2 + (P - 2) * step + 3.0;
                if (t < t_best) {
                    t_best = t;
                    best.P = P;
                    best.w0 = w0;
                    best.ns = k;
                }
            }
    }
    return best;
}

// The plan for a batch whose host lengths are known and whose launch order is longest first:
// the sizes' plan where it splits, else the longest sequences split where that pays, else the
// narrow rule.
struct LengthPlan {
    SplitPlan split;
    int32_t narrow = 0;
};

LengthPlan plan_for_lengths(int32_t N, int64_t total_T, const int32_t *cu_host, int32_t HV, int32_t dk, int32_t dv,
                            gdn_dtype dtype) {
    LengthPlan lp;
    lp.split = split_plan(N, total_T, HV, dk, dv, dtype);
    if (lp.split.P > 1 || N <= 0 || HV <= 0 || !gdn::prefill_chunked_supported(dk, dv, dtype == GDN_BF16))
        return lp;
    const int64_t cus = device_cus();
    const int64_t u = (int64_t)HV * (dv / 64);
    if ((int64_t)N * u * 2 <= cus) {
        lp.narrow = N;
        return lp;
    }
    const LengthStats ls = length_stats(cu_host, N, u);
    double t_unsplit = 0.0;
    lp.narrow = narrow_sequences(ls, N, u, cus, &t_unsplit);
    const SplitPlan sl = split_longest(ls, N, HV, dk, dv, cus, t_unsplit);
    if (sl.P > 1) {
        lp.split = sl;
        lp.narrow = 0;
    }
    return lp;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace parts: the longest-first order, then (split sequences) the segment maps and
// the segment start tables of the split ranks.
struct WorkspacePlan {
    size_t order = 0, maps = 0, starts = 0;
    SplitPlan split;
    size_t total() const { return order + maps + starts; }
};

WorkspacePlan workspace_for(int32_t N, int32_t HV, int32_t dk, int32_t dv, SplitPlan sp) {
    WorkspacePlan w;
    if (N > 1 && N <= gdn::kMaxOrderedSequences) w.order = round256((size_t)N * 4);
    w.split = sp;
    if (sp.P > 1) {
        w.maps = round256((size_t)sp.ns * (sp.P - 2) * HV * dk * (dv + dk) * 4);
        w.starts = round256((size_t)sp.ns * (sp.P - 1) * HV * dk * dv * 4);
    }
    return w;
}

WorkspacePlan workspace_plan(int32_t N, int64_t total_T, int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype) {
    return workspace_for(N, HV, dk, dv, split_plan(N, total_T, HV, dk, dv, dtype));
}

// Whether the launch order of a batch with these host lengths is longest first: the order
// kernel sorts batches of up to kMaxOrderedSequences; larger ones run in the given order.
bool launches_longest_first(const int32_t *cu_host, int32_t N) {
    if (!cu_host) return false;
    if (N <= gdn::kMaxOrderedSequences) return true;
    for (int32_t i = 1; i < N; ++i)
        if (cu_host[i + 1] - cu_host[i] > cu_host[i] - cu_host[i - 1]) return false;
    return true;
}

gdn_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return GDN_OK;
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Static scratch of the allocation-free prefill (gdn_prefill_noalloc): one array per device,
// loaded with the library's code object and kept until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol; its device address -- different on every
// device -- comes from hipGetSymbolAddress, taken once per device at the entry point's first
// call there, with that device current.  Nothing in the array has to start at zero: every
// part of the workspace (launch order, segment maps, start tables) is written by an earlier
// kernel of the same call before it is read.  Calls that overlap in time on one device share
// the array and race.
std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

gdn_status static_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(GDN_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..63", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

// The prefill behind gdn_prefill_ex (workspace from the caller) and gdn_prefill_noalloc
// (use_scratch: the workspace is the device's static scratch array, and workspace /
// workspace_bytes are ignored).
gdn_status run_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                       const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                       const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV, int32_t dk, int32_t dv,
                       gdn_dtype dtype, float scale, gdn_variant variant, const gdn_block_ops *ops,
                       void *workspace, size_t workspace_bytes, bool use_scratch, hipStream_t stream) {
    g_last_error[0] = 0;
    if (use_scratch) {
        workspace = nullptr;
        workspace_bytes = 0;
    }
    if (total_T < 0) return fail(GDN_ERR_SHAPE, "total_T = %lld is negative", (long long)total_T);
    gdn_status st = check_common(q, k, v, g, beta, o, N, HQK, HV, dk, dv, dtype, total_T, variant);
    if (st != GDN_OK) return st;
    st = check_ops(ops, variant, beta, total_T);
    if (st != GDN_OK) return st;
    if (S0 && !aligned(S0, 16)) return fail(GDN_ERR_ALIGN, "S0 must be 16-byte aligned");
    if (S_T && !aligned(S_T, 16)) return fail(GDN_ERR_ALIGN, "S_T must be 16-byte aligned");
    if ((int64_t)N * HV > 0x7fffffffLL) return fail(GDN_ERR_SHAPE, "N * HV exceeds the grid limit");
    int64_t eq_len = 0;
    st = check_seqlens(cu_seqlens, cu_seqlens_host, N, total_T, &eq_len);
    if (st != GDN_OK) return st;
    if (N > 0) {
        const size_t es = dtype == GDN_BF16 ? 2 : 4;
        const size_t T = (size_t)total_T, nqk = T * HQK * dk * es, nv = T * HV * dv * es, ng = T * HV * 4;
        const size_t ns = (size_t)N * HV * dk * dv * 4;
        const Span outs[] = {{o, nv, "o"}, {S_T, ns, "S_T"}, {workspace, workspace_bytes, "workspace"}};
        const Span ins[] = {{q, nqk, "q"},
                            {k, nqk, "k"},
                            {v, nv, "v"},
                            {variant_gated(variant) ? g : nullptr, ng, "g"},
                            {beta, ng, "beta"},
                            {S0, ns, "S0"},
                            {cu_seqlens, ((size_t)N + 1) * 4, "cu_seqlens"},
                            {ops ? ops->z : nullptr, nv, "z"},
                            {ops ? ops->A_log : nullptr, (size_t)HV * 4, "A_log"},
                            {ops ? ops->dt_bias : nullptr, (size_t)HV * 4, "dt_bias"},
                            {ops && ops->z ? ops->norm_w : nullptr, (size_t)dv * 4, "norm_w"}};
        st = check_disjoint(outs, 3, ins, 11, "S_T", "S0");
        if (st != GDN_OK) return st;
    }
    WorkspacePlan plan = workspace_plan(N, total_T, HV, dk, dv, dtype);
    const size_t need = plan.total();
    if (use_scratch) {
        if (need > kStaticScratchBytes)
            return fail(GDN_ERR_WORKSPACE,
                        "these sizes need %zu bytes of workspace; the static scratch of "
                        "gdn_prefill_noalloc holds %zu (call gdn_prefill_ex with a workspace instead)",
                        need, kStaticScratchBytes);
        if (N == 0) return GDN_OK;
        if (need > 0) {
            st = static_scratch(&workspace);
            if (st != GDN_OK) return st;
            workspace_bytes = kStaticScratchBytes;
        }
    }
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (need > 0 && !workspace) return fail(GDN_ERR_NULL, "workspace must be non-NULL");
    if (workspace && !aligned(workspace, 16)) return fail(GDN_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (N == 0) return GDN_OK;

    // Launch order: longest sequences first.  Equal lengths (cu_seqlens NULL) and host
    // lengths that are already non-increasing keep the given order.
    const int32_t *order = nullptr;
    bool sorted = false;
    if (cu_seqlens && cu_seqlens_host) {
        sorted = true;
        for (int32_t i = 1; i < N && sorted; ++i)
            sorted = cu_seqlens_host[i + 1] - cu_seqlens_host[i] <= cu_seqlens_host[i] - cu_seqlens_host[i - 1];
    }
    if (cu_seqlens && plan.order > 0) {
        if (!sorted) {
            int32_t *ord = static_cast<int32_t *>(workspace);
            gdn_status s2 = hip_status(gdn::launch_longest_first(cu_seqlens, N, ord, stream), "order launch");
            if (s2 != GDN_OK) return s2;
            order = ord;
        }
    }
    gdn::PrefillArgs a{q, k, v, variant_gated(variant) ? g : nullptr, beta, cu_seqlens, order, eq_len, N,
                       total_T, S0, o, S_T, HQK, HV, dk, dv, scale, workspace, workspace_bytes,
                       variant_delta(variant) ? 1 : 0};
    a.gate = gate_args(ops, variant);
    const bool bf16 = dtype == GDN_BF16;
    const bool longest_first = order || sorted;
    if (plan.split.P == 1 && gdn::prefill_chunked_supported(dk, dv, bf16)) {
        // sequences on 32-column workgroups (all of a batch that fills at most half the units;
        // else the longest, when the host lengths are known and the launch order is longest first)
        a.narrow = narrow_for_batch(N, HV, dv, cu_seqlens ? cu_seqlens_host : nullptr, longest_first);
        // or, where that pays, the longest sequence split, if the workspace holds its maps and
        // start tables (gdn_prefill_workspace_size_lens)
        if (cu_seqlens && cu_seqlens_host && longest_first && workspace) {
            const LengthPlan lp = plan_for_lengths(N, total_T, cu_seqlens_host, HV, dk, dv, dtype);
            const WorkspacePlan wl = workspace_for(N, HV, dk, dv, lp.split);
            if (lp.split.P > 1 && wl.total() <= workspace_bytes) {
                plan = wl;
                a.narrow = 0;
            }
        }
    }
    const int32_t P = plan.split.P;
    if (P > 1) {
        // split sequences: segment 0 of the split ranks (and the other sequences whole) beside
        // the maps of their middle segments, the chain, then segments 1 .. P-1 from their start
        // tables
        float *maps = reinterpret_cast<float *>(static_cast<char *>(workspace) + plan.order);
        float *starts = reinterpret_cast<float *>(static_cast<char *>(workspace) + plan.order + plan.maps);
        const int32_t ns = plan.split.ns;
        a.split = gdn::SplitArgs{P, 1, plan.split.w0, ns, maps, starts};
        st = hip_status(gdn::launch_prefill_chunked(a, stream), "chunked prefill (segment maps) launch");
        if (st == GDN_OK)
            st = hip_status(gdn::launch_split_chain(maps, starts, ns, P, HV, dv, stream), "segment chain launch");
        if (st == GDN_OK) {
            a.split = gdn::SplitArgs{P, 2, plan.split.w0, ns, maps, starts};
            st = hip_status(gdn::launch_prefill_chunked(a, stream), "chunked prefill (segments) launch");
        }
    } else if (gdn::prefill_chunked_supported(dk, dv, bf16)) {
        st = hip_status(gdn::launch_prefill_chunked(a, stream), "chunked prefill launch");
    } else {
        st = hip_status(gdn::launch_prefill_recurrent(a, bf16, stream), "prefill launch");
    }
    if (st != GDN_OK || !ops || !ops->z || total_T == 0) return st;
    gdn::NormArgs na{o, ops->z, ops->norm_w, o, total_T * HV, dv, ops->norm_eps};
    return hip_status(gdn::launch_gated_rmsnorm(na, bf16, stream), "gated norm launch");
}

}  // namespace

extern "C" {

const char *gdn_status_str(gdn_status s) {
    switch (s) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "null pointer";
        case GDN_ERR_SHAPE: return "bad shape";
        case GDN_ERR_DTYPE: return "bad dtype";
        case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
        case GDN_ERR_ALIGN: return "misaligned pointer";
        case GDN_ERR_SEQLENS: return "bad sequence lengths";
        case GDN_ERR_WORKSPACE: return "workspace too small";
        case GDN_ERR_HIP: return "HIP runtime error";
        case GDN_ERR_ALIAS: return "overlapping buffers";
        case GDN_ERR_VALUE: return "argument out of range";
    }
    return "unknown status";
}

const char *gdn_last_error(void) { return g_last_error; }

int32_t gdn_version(void) { return 200; /* 0.2.0 */ }

gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *S, void *o, int32_t N, int32_t HQK,
                           int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                           hipStream_t stream) {
    return gdn_decode_step_v(q, k, v, g, beta, S, o, N, HQK, HV, dk, dv, dtype, scale, GDN_GATED_DELTA,
                             stream);
}

gdn_status gdn_decode_step_v(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *S, void *o, int32_t N, int32_t HQK,
                             int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                             gdn_variant variant, hipStream_t stream) {
    return gdn_decode_step_ex(q, k, v, g, beta, S, o, N, HQK, HV, dk, dv, dtype, scale, variant, nullptr,
                              stream);
}

gdn_status gdn_decode_step_ex(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, float *S, void *o, int32_t N, int32_t HQK,
                              int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                              gdn_variant variant, const gdn_block_ops *ops, hipStream_t stream) {
    g_last_error[0] = 0;
    gdn_status st = check_common(q, k, v, g, beta, o, N, HQK, HV, dk, dv, dtype, N, variant);
    if (st != GDN_OK) return st;
    st = check_ops(ops, variant, beta, N);
    if (st != GDN_OK) return st;
    if (N == 0) return GDN_OK;
    if (!S) return fail(GDN_ERR_NULL, "S must be non-NULL");
    if (!aligned(S, 16)) return fail(GDN_ERR_ALIGN, "S must be 16-byte aligned");
    if ((int64_t)N * HV > 0x7fffffffLL) return fail(GDN_ERR_SHAPE, "N * HV exceeds the grid limit");
    {
        const size_t es = dtype == GDN_BF16 ? 2 : 4;
        const size_t nqk = (size_t)N * HQK * dk * es, nv = (size_t)N * HV * dv * es, ng = (size_t)N * HV * 4;
        const Span outs[] = {{S, (size_t)N * HV * dk * dv * 4, "S"}, {o, nv, "o"}};
        const Span ins[] = {{q, nqk, "q"},
                            {k, nqk, "k"},
                            {v, nv, "v"},
                            {variant_gated(variant) ? g : nullptr, ng, "g"},
                            {beta, ng, "beta"},
                            {ops ? ops->z : nullptr, nv, "z"},
                            {ops ? ops->A_log : nullptr, (size_t)HV * 4, "A_log"},
                            {ops ? ops->dt_bias : nullptr, (size_t)HV * 4, "dt_bias"},
                            {ops && ops->z ? ops->norm_w : nullptr, (size_t)dv * 4, "norm_w"}};
        st = check_disjoint(outs, 2, ins, 9);
        if (st != GDN_OK) return st;
    }
    gdn::DecodeArgs a{q, k, v, variant_gated(variant) ? g : nullptr, beta, S, o, N, HQK, HV, dk, dv, scale,
                      variant_delta(variant) ? 1 : 0};
    a.gate = gate_args(ops, variant);
    if (ops && ops->z) {
        a.z = ops->z;
        a.norm_w = ops->norm_w;
        a.norm_eps = ops->norm_eps;
    }
    a.max_wgs = 4 * device_cus();
    return hip_status(gdn::launch_decode(a, dtype == GDN_BF16, stream), "decode launch");
}

size_t gdn_prefill_workspace_size(int32_t N, int64_t total_T, int32_t HQK, int32_t HV,
                                  int32_t dk, int32_t dv, gdn_dtype dtype) {
    (void)HQK;
    if (N < 0 || total_T < 0 || HV <= 0) return 0;
    return workspace_plan(N, total_T, HV, dk, dv, dtype).total();
}

gdn_status gdn_prefill(const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const int32_t *cu_seqlens,
                       const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                       const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV, int32_t dk,
                       int32_t dv, gdn_dtype dtype, float scale, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    return gdn_prefill_v(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, N, total_T, S0, o, S_T, HQK, HV, dk,
                         dv, dtype, scale, GDN_GATED_DELTA, workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_v(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                         const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV, int32_t dk,
                         int32_t dv, gdn_dtype dtype, float scale, gdn_variant variant, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return gdn_prefill_ex(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, N, total_T, S0, o, S_T, HQK, HV, dk, dv,
                          dtype, scale, variant, nullptr, workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_ex(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const int32_t *cu_seqlens,
                          const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                          const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV, int32_t dk,
                          int32_t dv, gdn_dtype dtype, float scale, gdn_variant variant,
                          const gdn_block_ops *ops, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return run_prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, N, total_T, S0, o, S_T, HQK, HV, dk, dv,
                       dtype, scale, variant, ops, workspace, workspace_bytes, false, stream);
}

gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const int32_t *cu_seqlens,
                               const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                               const float *S0, void *o, float *S_T, int32_t HQK, int32_t HV,
                               int32_t dk, int32_t dv, gdn_dtype dtype, float scale,
                               gdn_variant variant, const gdn_block_ops *ops, hipStream_t stream) {
    return run_prefill(q, k, v, g, beta, cu_seqlens, cu_seqlens_host, N, total_T, S0, o, S_T, HQK, HV, dk, dv,
                       dtype, scale, variant, ops, nullptr, 0, true, stream);
}

gdn_status gdn_conv_silu(const void *x, const float *w, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, int32_t N, int64_t total_T,
                         const void *state_in, void *state_out, void *q, void *k, void *v,
                         int32_t HQK, int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype,
                         hipStream_t stream) {
    g_last_error[0] = 0;
    if (dtype != GDN_BF16 && dtype != GDN_F32) return fail(GDN_ERR_DTYPE, "unknown dtype %d", (int)dtype);
    if (N < 0 || total_T < 0) return fail(GDN_ERR_SHAPE, "N and total_T must be >= 0");
    if (HQK <= 0 || HV <= 0) return fail(GDN_ERR_SHAPE, "head counts must be positive (HQK=%d, HV=%d)", HQK, HV);
    if (!dim_ok(dk) || !dim_ok(dv))
        return fail(GDN_ERR_UNSUPPORTED, "dk=%d, dv=%d: each must be 32, 64 or 128", dk, dv);
    const int64_t Ct = 2 * (int64_t)HQK * dk + (int64_t)HV * dv;
    if (Ct > (1LL << 30)) return fail(GDN_ERR_SHAPE, "2 HQK dk + HV dv = %lld channels is too many", (long long)Ct);
    int64_t eq_len = 0;
    gdn_status st = check_seqlens(cu_seqlens, cu_seqlens_host, N, total_T, &eq_len);
    if (st != GDN_OK) return st;
    if (N == 0) return GDN_OK;
    if (total_T > 0 && (!x || !w || !q || !k || !v)) return fail(GDN_ERR_NULL, "x, w, q, k and v must be non-NULL");
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(state_in, 16) || !aligned(state_out, 16))
        return fail(GDN_ERR_ALIGN, "x, w, q, k, v and the states must be 16-byte aligned");
    const size_t es = dtype == GDN_BF16 ? 2 : 4;
    const size_t sbytes = (size_t)N * 3 * (size_t)Ct * es;
    {
        const size_t T = (size_t)total_T, nq = T * HQK * dk * es, nv = T * HV * dv * es;
        const Span outs[] = {{q, nq, "q"}, {k, nq, "k"}, {v, nv, "v"}, {state_out, sbytes, "state_out"}};
        const Span ins[] = {{x, T * (size_t)Ct * es, "x"},
                            {w, (size_t)Ct * 16, "w"},
                            {state_in, sbytes, "state_in"},
                            {cu_seqlens, ((size_t)N + 1) * 4, "cu_seqlens"}};
        st = check_disjoint(outs, 4, ins, 4, "state_out", "state_in");
        if (st != GDN_OK) return st;
    }
    gdn::ConvArgs a{x, w, cu_seqlens, eq_len, N, total_T, state_in, state_out, q, k, v, HQK * dk, HV * dv};
    return hip_status(gdn::launch_conv_silu(a, dtype == GDN_BF16, stream), "conv launch");
}

gdn_status gdn_gated_rmsnorm(const void *x, const void *z, const float *w, float eps, void *y,
                             int64_t rows, int32_t dv, gdn_dtype dtype, hipStream_t stream) {
    g_last_error[0] = 0;
    if (dtype != GDN_BF16 && dtype != GDN_F32) return fail(GDN_ERR_DTYPE, "unknown dtype %d", (int)dtype);
    if (rows < 0) return fail(GDN_ERR_SHAPE, "rows = %lld is negative", (long long)rows);
    if (!dim_ok(dv)) return fail(GDN_ERR_UNSUPPORTED, "dv=%d must be 32, 64 or 128", dv);
    if (!(eps >= 0.f)) return fail(GDN_ERR_VALUE, "eps must be >= 0");
    if (rows == 0) return GDN_OK;
    if (!x || !z || !w || !y) return fail(GDN_ERR_NULL, "x, z, w and y must be non-NULL");
    if (!aligned(x, 16) || !aligned(z, 16) || !aligned(y, 16) || !aligned(w, 4))
        return fail(GDN_ERR_ALIGN, "x, z and y must be 16-byte aligned, w 4-byte");
    const size_t bytes = (size_t)rows * dv * (dtype == GDN_BF16 ? 2 : 4);
    if (partial_overlap(x, bytes, y, bytes) || partial_overlap(z, bytes, y, bytes) || z == y)
        return fail(GDN_ERR_ALIAS, "y may be x, but must not otherwise overlap x or z");
    gdn::NormArgs a{x, z, w, y, rows, dv, eps};
    return hip_status(gdn::launch_gated_rmsnorm(a, dtype == GDN_BF16, stream), "gated norm launch");
}

int32_t gdn_prefill_narrow_count(int32_t N, int64_t total_T, const int32_t *cu_seqlens_host, int32_t HQK,
                                 int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype) {
    (void)HQK;
    if (N <= 0 || HV <= 0 || total_T < 0 || !gdn::prefill_chunked_supported(dk, dv, dtype == GDN_BF16)) return 0;
    if (split_plan(N, total_T, HV, dk, dv, dtype).P > 1) return 0;
    if (cu_seqlens_host && launches_longest_first(cu_seqlens_host, N)) {
        const LengthPlan lp = plan_for_lengths(N, total_T, cu_seqlens_host, HV, dk, dv, dtype);
        return lp.split.P > 1 ? 0 : lp.narrow;
    }
    return narrow_for_batch(N, HV, dv, nullptr, false);
}

size_t gdn_prefill_workspace_size_lens(int32_t N, int64_t total_T, const int32_t *cu_seqlens_host, int32_t HQK,
                                       int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype) {
    const size_t base = gdn_prefill_workspace_size(N, total_T, HQK, HV, dk, dv, dtype);
    if (N <= 0 || total_T < 0 || HV <= 0 || !cu_seqlens_host || !launches_longest_first(cu_seqlens_host, N))
        return base;
    const LengthPlan lp = plan_for_lengths(N, total_T, cu_seqlens_host, HV, dk, dv, dtype);
    const size_t with = workspace_for(N, HV, dk, dv, lp.split).total();
    return with > base ? with : base;
}

const char *gdn_prefill_kernel_name(int32_t N, int64_t total_T, const int32_t *cu_seqlens_host, int32_t HQK,
                                    int32_t HV, int32_t dk, int32_t dv, gdn_dtype dtype) {
    (void)HQK;
    if (!gdn::prefill_chunked_supported(dk, dv, dtype == GDN_BF16)) return "prefill_recurrent";
    if (N <= 0 || HV <= 0 || total_T < 0) return "prefill_chunked";
    bool split = split_plan(N, total_T, HV, dk, dv, dtype).P > 1;
    if (!split && cu_seqlens_host && launches_longest_first(cu_seqlens_host, N))
        split = plan_for_lengths(N, total_T, cu_seqlens_host, HV, dk, dv, dtype).split.P > 1;
    return split ? "prefill_chunked_split" : "prefill_chunked";
}

}  // extern "C"
