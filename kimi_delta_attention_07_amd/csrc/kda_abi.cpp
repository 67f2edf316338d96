// C ABI of libkda.so (declared in include/kda.h): argument validation on the
// host, chunk planning, kernel dispatch and error reporting.  Every check runs
// before the first HIP call, so an invalid call launches nothing, writes
// nothing and touches no device.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kda_internal.h"

namespace {

thread_local std::string g_detail;

kda_status fail(kda_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_detail = buf;
    return s;
}

kda_status ok() {
    g_detail.clear();
    return KDA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2_dim(int d) { return d == 4 || d == 8 || d == 16 || d == 32 || d == 64 || d == 128; }

kda_status check_geom(const kda_geom *g, bool chunk_path) {
    if (!g) return fail(KDA_ERR_NULL, "geom is NULL");
    if (g->H <= 0) return fail(KDA_ERR_SHAPE, "H = %d must be > 0", g->H);
    if (g->d <= 0) return fail(KDA_ERR_SHAPE, "d = %d must be > 0", g->d);
    if (chunk_path) {
        if (g->d != kda::kHeadDim)
            return fail(KDA_ERR_UNSUPPORTED, "the chunk path supports d = 128 only (got %d)", g->d);
    } else if (!is_pow2_dim(g->d)) {
        return fail(KDA_ERR_UNSUPPORTED, "d = %d not in {4, 8, 16, 32, 64, 128}", g->d);
    }
    if (g->conv_k < 1 || g->conv_k > 4)
        return fail(KDA_ERR_UNSUPPORTED, "conv_k = %d not in [1, 4]", g->conv_k);
    if (g->act != KDA_ACT_NONE && g->act != KDA_ACT_SILU)
        return fail(KDA_ERR_UNSUPPORTED, "act = %d is not a kda_act", g->act);
    if (!(g->l2_eps >= 0.0f)) return fail(KDA_ERR_SHAPE, "l2_eps must be >= 0");
    if ((long)g->H * g->d > (1L << 24)) return fail(KDA_ERR_SHAPE, "H * d too large");
    return KDA_OK;
}

// cu_seqlens (host copy): [0] == 0, non-decreasing, last == total_tokens.
kda_status check_seqlens(int32_t n_seqs, int32_t total_tokens, const int32_t *cu_host, long *n_chunks) {
    if (n_seqs <= 0) return fail(KDA_ERR_SHAPE, "n_seqs = %d must be > 0", n_seqs);
    if (total_tokens < 0) return fail(KDA_ERR_SHAPE, "total_tokens = %d must be >= 0", total_tokens);
    if (!cu_host) return fail(KDA_ERR_NULL, "cu_seqlens_host is NULL");
    if (cu_host[0] != 0) return fail(KDA_ERR_SEQLENS, "cu_seqlens[0] = %d, expected 0", cu_host[0]);
    long chunks = 0;
    for (int32_t n = 0; n < n_seqs; ++n) {
        if (cu_host[n + 1] < cu_host[n])
            return fail(KDA_ERR_SEQLENS, "cu_seqlens decreases at %d (%d -> %d)", n, cu_host[n], cu_host[n + 1]);
        chunks += (cu_host[n + 1] - cu_host[n] + kda::kChunk - 1) / kda::kChunk;
    }
    if (cu_host[n_seqs] != total_tokens)
        return fail(KDA_ERR_SHAPE, "total_tokens = %d but cu_seqlens[%d] = %d", total_tokens, n_seqs,
                    cu_host[n_seqs]);
    if (n_chunks) *n_chunks = chunks;
    return KDA_OK;
}

// Most chunks n sequences of T tokens in all can have: sequence i has
// ceil(L_i / 64) = floor((L_i + 63) / 64), and a sum of floors is at most the
// floor of the sum.  Workspace sizes are computed from this bound, so the
// caller needs only the two totals.
long chunk_bound(int32_t n_seqs, int32_t total_tokens) {
    return ((long)total_tokens + (long)(kda::kChunk - 1) * n_seqs) / kda::kChunk;
}

kda_status check_chunk_len(int32_t chunk) {
    if (chunk != kda::kChunk)
        return fail(KDA_ERR_UNSUPPORTED, "chunk = %d: the chunk path uses 64-token chunks only", chunk);
    return KDA_OK;
}

kda_status check_dtype(kda_dtype t) {
    if (t != KDA_F32 && t != KDA_BF16) return fail(KDA_ERR_DTYPE, "dtype %d is not a kda_dtype", (int)t);
    return KDA_OK;
}

struct Ptr {
    const void *p;
    const char *name;
};

kda_status check_required(std::initializer_list<Ptr> ps) {
    for (const Ptr &x : ps)
        if (!x.p) return fail(KDA_ERR_NULL, "%s is NULL", x.name);
    return KDA_OK;
}

kda_status check_aligned(std::initializer_list<Ptr> ps) {
    for (const Ptr &x : ps)
        if (x.p && !aligned16(x.p)) return fail(KDA_ERR_ALIGN, "%s is not 16-byte aligned", x.name);
    return KDA_OK;
}

// gfx950 check of the current device, cached per device ordinal.
std::atomic<int> g_arch_ok[64];

kda_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(KDA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(st, std::memory_order_relaxed);
        if (st == 2) return fail(KDA_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    }
    if (st == 2) return fail(KDA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return KDA_OK;
}

kda_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

#define KDA_TRY(x)                         \
    do {                                   \
        kda_status _s = (x);               \
        if (_s != KDA_OK) return _s;       \
    } while (0)

// Checks shared by the chunk entry points; fills n_chunks.
kda_status check_chunk_common(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                              const int32_t *cu_dev, const int32_t *cu_host, kda_dtype in_dtype,
                              void *workspace, size_t workspace_bytes, long *n_chunks) {
    KDA_TRY(check_geom(geom, true));
    KDA_TRY(check_seqlens(n_seqs, total_tokens, cu_host, n_chunks));
    KDA_TRY(check_dtype(in_dtype));
    if (in_dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "the chunk path takes bf16 inputs only");
    KDA_TRY(check_required({{cu_dev, "cu_seqlens_dev"}, {workspace, "workspace"}}));
    KDA_TRY(check_aligned({{workspace, "workspace"}}));
    const size_t need = kda::chunk_workspace_bytes(geom->H, n_seqs, *n_chunks);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if ((long)n_seqs * geom->H * kda::kTilesV > 0x7fffffffL) return fail(KDA_ERR_SHAPE, "too many sequences x heads");
    return KDA_OK;
}

kda::ChunkParams chunk_params(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens, long n_chunks,
                              const int32_t *cu_dev, const int32_t *cu_host, void *workspace) {
    kda::ChunkParams p{};
    p.T = total_tokens;
    p.H = geom->H;
    p.n_seqs = n_seqs;
    p.n_chunks = (int)n_chunks;
    p.scale = geom->scale;
    p.cu = cu_dev;
    kda::chunk_workspace_carve(workspace, geom->H, n_seqs, n_chunks, p);
    if (n_seqs <= kda::kPlanSeqs) {   // chunk table in the kernel arguments (cu_host is validated)
        p.plan_in_args = 1;
        int32_t off = 0;
        for (int n = 0; n <= n_seqs; ++n) {
            p.plan_cu[n] = cu_host[n];
            p.plan_off[n] = off;
            if (n < n_seqs) off += (cu_host[n + 1] - cu_host[n] + kda::kChunk - 1) / kda::kChunk;
        }
        // the scan takes sequences longest first (ties in index order)
        for (int n = 0; n < n_seqs; ++n) p.plan_order[n] = (uint8_t)n;
        std::stable_sort(p.plan_order, p.plan_order + n_seqs, [&](uint8_t a, uint8_t b) {
            return p.plan_off[a + 1] - p.plan_off[a] > p.plan_off[b + 1] - p.plan_off[b];
        });
    }
    return p;
}

// Scratch of kda_prefill_noalloc: the chunk workspace of callers that cannot
// allocate.  Each GPU the library runs on holds its own copy for the life of
// the process.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is taken once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with it current).
kda_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(KDA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_chunk_backward_workspace_bytes(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens) {
    if (check_geom(geom, true) != KDA_OK) return 0;
    if (n_seqs <= 0 || total_tokens < 0) return 0;
    return kda::bwd_workspace_bytes(geom->H, n_seqs, chunk_bound(n_seqs, total_tokens));
}

kda_status kda_chunk_backward(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                              const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                              const void *q, const void *k, const void *v, const void *log_alpha, const float *beta,
                              const void *gate, const float *initial_state, const void *dy,
                              const float *d_final_state, float *dq, float *dk, float *dv, float *dlog_alpha,
                              float *dbeta, float *dgate, float *d_initial_state, void *workspace,
                              size_t workspace_bytes, void *stream) {
    KDA_TRY(check_geom(geom, true));
    long n_chunks = 0;
    KDA_TRY(check_seqlens(n_seqs, total_tokens, cu_seqlens_host, &n_chunks));
    KDA_TRY(check_dtype(in_dtype));
    if (in_dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "the chunk path takes bf16 inputs only");
    KDA_TRY(check_required({{cu_seqlens_dev, "cu_seqlens_dev"}, {workspace, "workspace"}}));
    if (total_tokens > 0)
        KDA_TRY(check_required({{q, "q"}, {k, "k"}, {v, "v"}, {log_alpha, "log_alpha"}, {beta, "beta"}, {dy, "dy"},
                                {dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {dlog_alpha, "dlog_alpha"}, {dbeta, "dbeta"}}));
    if (gate && total_tokens > 0 && !dgate) return fail(KDA_ERR_NULL, "dgate is NULL while gate is given");
    KDA_TRY(check_aligned({{workspace, "workspace"}, {q, "q"}, {k, "k"}, {v, "v"}, {log_alpha, "log_alpha"},
                           {beta, "beta"}, {gate, "gate"}, {initial_state, "initial_state"}, {dy, "dy"},
                           {d_final_state, "d_final_state"}, {dq, "dq"}, {dk, "dk"}, {dv, "dv"},
                           {dlog_alpha, "dlog_alpha"}, {dbeta, "dbeta"}, {dgate, "dgate"},
                           {d_initial_state, "d_initial_state"}}));
    const size_t need = kda::bwd_workspace_bytes(geom->H, n_seqs, n_chunks);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if ((long)n_seqs * geom->H * kda::kTilesV > 0x7fffffffL || n_chunks * geom->H > 0x7fffffffL)
        return fail(KDA_ERR_SHAPE, "too many sequences or chunks x heads");
    KDA_TRY(check_device());
    kda::BwdParams p{};
    p.c = chunk_params(geom, n_seqs, total_tokens, n_chunks, cu_seqlens_dev, cu_seqlens_host, workspace);
    kda::bwd_workspace_carve(workspace, geom->H, n_seqs, n_chunks, p);
    p.c.records = nullptr;
    p.c.q = static_cast<const uint16_t *>(q);
    p.c.k = static_cast<const uint16_t *>(k);
    p.c.v = static_cast<const uint16_t *>(v);
    p.c.log_alpha = static_cast<const uint16_t *>(log_alpha);
    p.c.beta = beta;
    p.c.gate = static_cast<const uint16_t *>(gate);
    p.c.s0 = initial_state;
    p.dy = static_cast<const uint16_t *>(dy);
    p.ds_final = d_final_state;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dla = dlog_alpha;
    p.dbeta = dbeta;
    p.dgate = gate ? dgate : nullptr;
    p.ds0 = d_initial_state;
    return launched(kda::launch_chunk_backward(p, (hipStream_t)stream), "chunk backward");
}

const char *kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_SEQLENS: return "KDA_ERR_SEQLENS";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char *kda_last_error_detail(void) { return g_detail.c_str(); }

kda_status kda_prologue(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                        const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                        const void *q_raw, const void *k_raw, const void *v_raw, const float *conv_w,
                        const float *conv_cache_in, float *conv_cache_out, const void *beta_logit,
                        const void *gate_logit, void *q_out, void *k_out, void *v_out, float *beta_out,
                        void *gate_out, void *stream) {
    KDA_TRY(check_geom(geom, false));
    KDA_TRY(check_seqlens(n_seqs, total_tokens, cu_seqlens_host, nullptr));
    KDA_TRY(check_dtype(in_dtype));
    KDA_TRY(check_required({{cu_seqlens_dev, "cu_seqlens_dev"}, {conv_w, "conv_w"}}));
    if (total_tokens > 0) {   // per-token arrays: none is touched when every sequence is empty
        KDA_TRY(check_required({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {beta_logit, "beta_logit"},
                                {q_out, "q_out"}, {k_out, "k_out"}, {v_out, "v_out"}, {beta_out, "beta_out"}}));
        if (gate_logit && !gate_out) return fail(KDA_ERR_NULL, "gate_out is NULL while gate_logit is given");
    }
    KDA_TRY(check_aligned({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {conv_w, "conv_w"},
                           {conv_cache_in, "conv_cache_in"}, {conv_cache_out, "conv_cache_out"},
                           {beta_logit, "beta_logit"}, {gate_logit, "gate_logit"}, {q_out, "q_out"},
                           {k_out, "k_out"}, {v_out, "v_out"}, {beta_out, "beta_out"}, {gate_out, "gate_out"}}));
    KDA_TRY(check_device());
    kda::PrologueParams p{};
    p.T = total_tokens;
    p.H = geom->H;
    p.d = geom->d;
    p.K = geom->conv_k;
    p.act = geom->act;
    p.n_seqs = n_seqs;
    p.eps = geom->l2_eps;
    p.cu = cu_seqlens_dev;
    p.q_raw = q_raw;
    p.k_raw = k_raw;
    p.v_raw = v_raw;
    p.beta_logit = beta_logit;
    p.gate_logit = gate_logit;
    p.conv_w = conv_w;
    p.cache_in = geom->conv_k > 1 ? conv_cache_in : nullptr;
    p.cache_out = geom->conv_k > 1 ? conv_cache_out : nullptr;
    p.q_out = q_out;
    p.k_out = k_out;
    p.v_out = v_out;
    p.gate_out = gate_logit ? gate_out : nullptr;
    p.beta_out = beta_out;
    return launched(kda::launch_prologue(p, (int)in_dtype, (hipStream_t)stream), "prologue");
}

size_t kda_prologue_backward_workspace_bytes(const kda_geom *geom, int32_t total_tokens) {
    if (check_geom(geom, false) != KDA_OK || total_tokens < 0) return 0;
    return kda::prologue_bwd_workspace_bytes(geom->H, geom->d, total_tokens);
}

kda_status kda_prologue_backward(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                                 const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                                 const void *q_raw, const void *k_raw, const void *v_raw, const float *conv_w,
                                 const float *conv_cache_in, const void *beta_logit, const void *gate_logit,
                                 const float *dq, const float *dk, const float *dv, const float *dbeta,
                                 const float *dgate, float *dq_raw, float *dk_raw, float *dv_raw, float *dconv_w,
                                 float *dconv_cache_in, float *dbeta_logit, float *dgate_logit, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    KDA_TRY(check_geom(geom, false));
    KDA_TRY(check_seqlens(n_seqs, total_tokens, cu_seqlens_host, nullptr));
    KDA_TRY(check_dtype(in_dtype));
    KDA_TRY(check_required({{cu_seqlens_dev, "cu_seqlens_dev"}, {conv_w, "conv_w"}, {dconv_w, "dconv_w"},
                            {workspace, "workspace"}}));
    if (total_tokens > 0)
        KDA_TRY(check_required({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {beta_logit, "beta_logit"},
                                {dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {dbeta, "dbeta"}, {dq_raw, "dq_raw"},
                                {dk_raw, "dk_raw"}, {dv_raw, "dv_raw"}, {dbeta_logit, "dbeta_logit"}}));
    if (gate_logit && total_tokens > 0 && (!dgate || !dgate_logit))
        return fail(KDA_ERR_NULL, "dgate and dgate_logit are required when gate_logit is given");
    KDA_TRY(check_aligned({{workspace, "workspace"}, {q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"},
                           {conv_w, "conv_w"}, {conv_cache_in, "conv_cache_in"}, {beta_logit, "beta_logit"},
                           {gate_logit, "gate_logit"}, {dq, "dq"}, {dk, "dk"}, {dv, "dv"}, {dbeta, "dbeta"},
                           {dgate, "dgate"}, {dq_raw, "dq_raw"}, {dk_raw, "dk_raw"}, {dv_raw, "dv_raw"},
                           {dconv_w, "dconv_w"}, {dconv_cache_in, "dconv_cache_in"}, {dbeta_logit, "dbeta_logit"},
                           {dgate_logit, "dgate_logit"}}));
    const size_t need = kda::prologue_bwd_workspace_bytes(geom->H, geom->d, total_tokens);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    KDA_TRY(check_device());
    kda::PrologueBwdParams p{};
    p.T = total_tokens;
    p.H = geom->H;
    p.d = geom->d;
    p.K = geom->conv_k;
    p.act = geom->act;
    p.n_seqs = n_seqs;
    p.eps = geom->l2_eps;
    p.cu = cu_seqlens_dev;
    p.q_raw = q_raw;
    p.k_raw = k_raw;
    p.v_raw = v_raw;
    p.conv_w = conv_w;
    p.cache_in = geom->conv_k > 1 ? conv_cache_in : nullptr;
    p.beta_logit = beta_logit;
    p.gate_logit = gate_logit;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dbeta = dbeta;
    p.dgate = gate_logit ? dgate : nullptr;
    p.dq_raw = dq_raw;
    p.dk_raw = dk_raw;
    p.dv_raw = dv_raw;
    p.dconv_w = dconv_w;
    p.dcache_in = geom->conv_k > 1 ? dconv_cache_in : nullptr;
    p.dbeta_logit = dbeta_logit;
    p.dgate_logit = gate_logit ? dgate_logit : nullptr;
    p.workspace = workspace;
    return launched(kda::launch_prologue_backward(p, (int)in_dtype, (hipStream_t)stream), "prologue backward");
}

size_t kda_chunk_workspace_bytes(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens) {
    if (check_geom(geom, true) != KDA_OK) return 0;
    if (n_seqs <= 0 || total_tokens < 0) return 0;
    return kda::chunk_workspace_bytes(geom->H, n_seqs, chunk_bound(n_seqs, total_tokens));
}

kda_status kda_chunk_prepare(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                             const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                             const void *q, const void *k, const void *v, const void *log_alpha,
                             const float *beta, void *workspace, size_t workspace_bytes, void *stream) {
    long n_chunks = 0;
    KDA_TRY(check_chunk_common(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, workspace,
                               workspace_bytes, &n_chunks));
    if (total_tokens > 0)
        KDA_TRY(check_required({{q, "q"}, {k, "k"}, {v, "v"}, {log_alpha, "log_alpha"}, {beta, "beta"}}));
    KDA_TRY(check_aligned({{q, "q"}, {k, "k"}, {v, "v"}, {log_alpha, "log_alpha"}, {beta, "beta"}}));
    KDA_TRY(check_device());
    kda::ChunkParams p = chunk_params(geom, n_seqs, total_tokens, n_chunks, cu_seqlens_dev, cu_seqlens_host, workspace);
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.log_alpha = static_cast<const uint16_t *>(log_alpha);
    p.beta = beta;
    return launched(kda::launch_chunk_prepare(p, (hipStream_t)stream), "chunk prepare");
}

kda_status kda_chunk_scan(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                          const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                          const void *gate, const float *initial_state, float *final_state, void *out,
                          void *workspace, size_t workspace_bytes, void *stream) {
    long n_chunks = 0;
    KDA_TRY(check_chunk_common(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, workspace,
                               workspace_bytes, &n_chunks));
    if (total_tokens > 0) KDA_TRY(check_required({{out, "out"}}));
    KDA_TRY(check_aligned({{gate, "gate"}, {initial_state, "initial_state"}, {final_state, "final_state"},
                           {out, "out"}}));
    KDA_TRY(check_device());
    kda::ChunkParams p = chunk_params(geom, n_seqs, total_tokens, n_chunks, cu_seqlens_dev, cu_seqlens_host, workspace);
    p.gate = static_cast<const uint16_t *>(gate);
    p.s0 = initial_state;
    p.s_final = final_state;
    p.out = static_cast<uint16_t *>(out);
    return launched(kda::launch_chunk_scan(p, (hipStream_t)stream), "chunk scan");
}

kda_status kda_chunk_forward(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                             const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                             int32_t chunk, const void *q, const void *k, const void *v, const void *log_alpha,
                             const float *beta, const void *gate, const float *initial_state, float *final_state,
                             void *out, void *workspace, size_t workspace_bytes, void *stream) {
    // validate everything the two stages need before launching either
    KDA_TRY(check_chunk_len(chunk));
    long n_chunks = 0;
    KDA_TRY(check_chunk_common(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, workspace,
                               workspace_bytes, &n_chunks));
    if (total_tokens > 0)
        KDA_TRY(check_required({{q, "q"}, {k, "k"}, {v, "v"}, {log_alpha, "log_alpha"}, {beta, "beta"}}));
    if (total_tokens > 0) KDA_TRY(check_required({{out, "out"}}));
    KDA_TRY(check_aligned({{q, "q"}, {k, "k"}, {v, "v"}, {log_alpha, "log_alpha"}, {beta, "beta"}, {gate, "gate"},
                           {initial_state, "initial_state"}, {final_state, "final_state"}, {out, "out"}}));
    KDA_TRY(kda_chunk_prepare(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, q, k, v,
                              log_alpha, beta, workspace, workspace_bytes, stream));
    return kda_chunk_scan(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, gate,
                          initial_state, final_state, out, workspace, workspace_bytes, stream);
}

kda_status kda_prefill_prepare(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                               const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                               const void *q_raw, const void *k_raw, const void *v_raw, const float *conv_w,
                               const float *conv_cache_in, float *conv_cache_out, const void *log_alpha,
                               const void *beta_logit, void *workspace, size_t workspace_bytes, void *stream) {
    long n_chunks = 0;
    KDA_TRY(check_chunk_common(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, workspace,
                               workspace_bytes, &n_chunks));
    KDA_TRY(check_required({{conv_w, "conv_w"}}));
    if (total_tokens > 0)
        KDA_TRY(check_required({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {log_alpha, "log_alpha"},
                                {beta_logit, "beta_logit"}}));
    KDA_TRY(check_aligned({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {conv_w, "conv_w"},
                           {conv_cache_in, "conv_cache_in"}, {conv_cache_out, "conv_cache_out"},
                           {log_alpha, "log_alpha"}, {beta_logit, "beta_logit"}}));
    KDA_TRY(check_device());
    kda::ChunkParams p = chunk_params(geom, n_seqs, total_tokens, n_chunks, cu_seqlens_dev, cu_seqlens_host, workspace);
    p.K = geom->conv_k;
    p.act = geom->act;
    p.eps = geom->l2_eps;
    p.q_raw = static_cast<const uint16_t *>(q_raw);
    p.k_raw = static_cast<const uint16_t *>(k_raw);
    p.v_raw = static_cast<const uint16_t *>(v_raw);
    p.log_alpha = static_cast<const uint16_t *>(log_alpha);
    p.beta_logit = static_cast<const uint16_t *>(beta_logit);
    p.conv_w = conv_w;
    p.cache_in = geom->conv_k > 1 ? conv_cache_in : nullptr;
    // The prepare kernel writes the outgoing conv cache itself (from each
    // sequence's last chunk) unless that could race with a read of the
    // incoming one: in place, a sequence of several chunks has its cache read
    // by its first chunk's blocks; out of place, an empty sequence has no
    // chunk to copy its cache through.
    bool fold = false;
    if (conv_cache_out && geom->conv_k > 1) {
        bool any_empty = false, any_multi = false;
        for (int n = 0; n < n_seqs; ++n) {
            const int len = cu_seqlens_host[n + 1] - cu_seqlens_host[n];
            any_empty |= len == 0;
            any_multi |= len > kda::kChunk;
        }
        fold = conv_cache_out == conv_cache_in ? !any_multi : !any_empty;
    }
    p.cache_out = fold ? conv_cache_out : nullptr;
    KDA_TRY(launched(kda::launch_prefill_prepare(p, (hipStream_t)stream), "prefill prepare"));
    if (fold || !conv_cache_out || geom->conv_k <= 1) return KDA_OK;
    // outgoing conv cache, after the prepare kernel has read the incoming one
    kda::PrologueParams c{};
    c.T = total_tokens;
    c.H = geom->H;
    c.d = geom->d;
    c.K = geom->conv_k;
    c.n_seqs = n_seqs;
    c.cu = cu_seqlens_dev;
    c.q_raw = q_raw;
    c.k_raw = k_raw;
    c.v_raw = v_raw;
    c.cache_in = geom->conv_k > 1 ? conv_cache_in : nullptr;
    c.cache_out = geom->conv_k > 1 ? conv_cache_out : nullptr;
    return launched(kda::launch_conv_cache_out(c, (int)in_dtype, (hipStream_t)stream), "conv cache out");
}

kda_status kda_prefill_scan(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                            const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                            const void *gate_logit, const float *initial_state, float *final_state, void *out,
                            void *workspace, size_t workspace_bytes, void *stream) {
    long n_chunks = 0;
    KDA_TRY(check_chunk_common(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, workspace,
                               workspace_bytes, &n_chunks));
    if (total_tokens > 0) KDA_TRY(check_required({{out, "out"}}));
    KDA_TRY(check_aligned({{gate_logit, "gate_logit"}, {initial_state, "initial_state"},
                           {final_state, "final_state"}, {out, "out"}}));
    KDA_TRY(check_device());
    kda::ChunkParams p = chunk_params(geom, n_seqs, total_tokens, n_chunks, cu_seqlens_dev, cu_seqlens_host, workspace);
    p.gate = static_cast<const uint16_t *>(gate_logit);
    p.gate_is_logit = 1;
    p.s0 = initial_state;
    p.s_final = final_state;
    p.out = static_cast<uint16_t *>(out);
    return launched(kda::launch_chunk_scan(p, (hipStream_t)stream), "prefill scan");
}

kda_status kda_prefill(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens, const int32_t *cu_seqlens_dev,
                       const int32_t *cu_seqlens_host, kda_dtype in_dtype, int32_t chunk, const void *q_raw,
                       const void *k_raw, const void *v_raw, const float *conv_w, const float *conv_cache_in,
                       float *conv_cache_out, const void *log_alpha, const void *beta_logit,
                       const void *gate_logit, const float *initial_state, float *final_state, void *out,
                       void *workspace, size_t workspace_bytes, void *stream) {
    // validate what both stages need before launching either
    KDA_TRY(check_chunk_len(chunk));
    long n_chunks = 0;
    KDA_TRY(check_chunk_common(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, workspace,
                               workspace_bytes, &n_chunks));
    KDA_TRY(check_required({{conv_w, "conv_w"}}));
    if (total_tokens > 0)
        KDA_TRY(check_required({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {log_alpha, "log_alpha"},
                                {beta_logit, "beta_logit"}}));
    if (total_tokens > 0) KDA_TRY(check_required({{out, "out"}}));
    KDA_TRY(check_aligned({{gate_logit, "gate_logit"}, {initial_state, "initial_state"},
                           {final_state, "final_state"}, {out, "out"}}));
    KDA_TRY(kda_prefill_prepare(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, q_raw, k_raw,
                                v_raw, conv_w, conv_cache_in, conv_cache_out, log_alpha, beta_logit, workspace,
                                workspace_bytes, stream));
    return kda_prefill_scan(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, gate_logit,
                            initial_state, final_state, out, workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(const kda_geom *geom, int32_t batch, const int32_t *slot_idx_dev, int32_t n_slots,
                           kda_dtype in_dtype, const void *q_raw, const void *k_raw, const void *v_raw,
                           const float *conv_w, float *conv_cache, float *state, const void *log_alpha,
                           const void *beta_logit, const void *gate_logit, kda_dtype out_dtype, void *out,
                           void *stream) {
    KDA_TRY(check_geom(geom, false));
    if (batch <= 0) return fail(KDA_ERR_SHAPE, "batch = %d must be > 0", batch);
    if (n_slots <= 0) return fail(KDA_ERR_SHAPE, "n_slots = %d must be > 0", n_slots);
    if (!slot_idx_dev && batch > n_slots)
        return fail(KDA_ERR_SHAPE, "batch = %d > n_slots = %d with identity slots", batch, n_slots);
    if (batch > 65535 * 256 || geom->H > 65535 || (long)batch * geom->H > 0x7fffffffL)
        return fail(KDA_ERR_SHAPE, "batch or H too large for the grid");
    KDA_TRY(check_dtype(in_dtype));
    KDA_TRY(check_dtype(out_dtype));
    KDA_TRY(check_required({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {conv_w, "conv_w"},
                            {state, "state"}, {log_alpha, "log_alpha"}, {beta_logit, "beta_logit"}, {out, "out"}}));
    if (geom->conv_k > 1 && !conv_cache) return fail(KDA_ERR_NULL, "conv_cache is NULL with conv_k > 1");
    KDA_TRY(check_aligned({{slot_idx_dev, "slot_idx"}, {q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"},
                           {conv_w, "conv_w"}, {conv_cache, "conv_cache"}, {state, "state"},
                           {log_alpha, "log_alpha"}, {beta_logit, "beta_logit"}, {gate_logit, "gate_logit"},
                           {out, "out"}}));
    KDA_TRY(check_device());
    kda::DecodeParams p{};
    p.batch = batch;
    p.H = geom->H;
    p.d = geom->d;
    p.K = geom->conv_k;
    p.act = geom->act;
    p.n_slots = n_slots;
    p.eps = geom->l2_eps;
    p.scale = geom->scale;
    p.slot_idx = slot_idx_dev;
    p.q_raw = q_raw;
    p.k_raw = k_raw;
    p.v_raw = v_raw;
    p.log_alpha = log_alpha;
    p.beta_logit = beta_logit;
    p.gate_logit = gate_logit;
    p.conv_w = conv_w;
    p.conv_cache = conv_cache;
    p.state = state;
    p.out = out;
    return launched(kda::launch_decode(p, (int)in_dtype, (int)out_dtype, (hipStream_t)stream), "decode");
}

// ---------------------------------------------------------------------------
// The mixer's linear maps and the whole mixer prefill
// ---------------------------------------------------------------------------
namespace {

kda_status check_proj_geom(const kda_geom *geom) {
    if (!geom) return fail(KDA_ERR_NULL, "geom is NULL");
    if (geom->H <= 0 || geom->d <= 0) return fail(KDA_ERR_SHAPE, "H = %d and d = %d must be > 0", geom->H, geom->d);
    if ((long)geom->H * geom->d > (1L << 24)) return fail(KDA_ERR_SHAPE, "H * d too large");
    return KDA_OK;
}

// rows x K bf16 operand of the GEMM: K a multiple of 8 (16-byte rows), and
// the whole matrix addressable by one buffer resource (< 4 GiB)
kda_status check_gemm_dims(long rows, long K, const char *what) {
    if (K <= 0 || K % 8 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "%s: inner dimension %ld must be a positive multiple of 8", what, K);
    if (rows * K * 2 >= (1L << 32)) return fail(KDA_ERR_SHAPE, "%s: %ld x %ld bf16 exceeds 4 GiB", what, rows, K);
    return KDA_OK;
}

kda::ProjParams in_proj_params(const kda_geom *geom, int32_t T, int32_t hidden, const void *x, const void *w_in,
                               const float *a_log, const float *dt_bias, void *const outs[6]) {
    kda::ProjParams p{};
    p.M = T;
    p.N = 5 * geom->H * geom->d + geom->H;
    p.K = hidden;
    p.a = static_cast<const uint16_t *>(x);
    p.b = static_cast<const uint16_t *>(w_in);
    p.epi = 1;
    p.H = geom->H;
    p.d = geom->d;
    for (int i = 0; i < 6; ++i) p.seg[i] = static_cast<uint16_t *>(outs[i]);
    p.a_log = a_log;
    p.bias = dt_bias;
    return p;
}

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

kda_status kda_in_projection(const kda_geom *geom, int32_t T, int32_t hidden, const void *x, const void *w_in,
                             const float *a_log, const float *dt_bias, void *q_raw, void *k_raw, void *v_raw,
                             void *gate_logit, void *log_alpha, void *beta_logit, void *stream) {
    KDA_TRY(check_proj_geom(geom));
    if (T < 0) return fail(KDA_ERR_SHAPE, "T = %d must be >= 0", T);
    const long N = 5L * geom->H * geom->d + geom->H;
    KDA_TRY(check_gemm_dims(T, hidden, "x"));
    KDA_TRY(check_gemm_dims(N, hidden, "w_in"));
    KDA_TRY(check_required({{w_in, "w_in"}}));
    if (T > 0)
        KDA_TRY(check_required({{x, "x"}, {q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"},
                                {gate_logit, "gate_logit"}, {log_alpha, "log_alpha"}, {beta_logit, "beta_logit"}}));
    KDA_TRY(check_aligned({{x, "x"}, {w_in, "w_in"}, {a_log, "a_log"}, {dt_bias, "dt_bias"}, {q_raw, "q_raw"},
                           {k_raw, "k_raw"}, {v_raw, "v_raw"}, {gate_logit, "gate_logit"},
                           {log_alpha, "log_alpha"}, {beta_logit, "beta_logit"}}));
    KDA_TRY(check_device());
    void *outs[6] = {q_raw, k_raw, v_raw, gate_logit, log_alpha, beta_logit};
    return launched(kda::launch_gemm(in_proj_params(geom, T, hidden, x, w_in, a_log, dt_bias, outs),
                                     (hipStream_t)stream), "in projection");
}

kda_status kda_out_projection(const kda_geom *geom, int32_t T, int32_t hidden, const void *y, const void *w_out,
                              void *out, void *stream) {
    KDA_TRY(check_proj_geom(geom));
    if (T < 0) return fail(KDA_ERR_SHAPE, "T = %d must be >= 0", T);
    if (hidden <= 0) return fail(KDA_ERR_SHAPE, "hidden = %d must be > 0", hidden);
    const long K = (long)geom->H * geom->d;
    KDA_TRY(check_gemm_dims(T, K, "y"));
    KDA_TRY(check_gemm_dims(hidden, K, "w_out"));
    KDA_TRY(check_required({{w_out, "w_out"}}));
    if (T > 0) KDA_TRY(check_required({{y, "y"}, {out, "out"}}));
    KDA_TRY(check_aligned({{y, "y"}, {w_out, "w_out"}, {out, "out"}}));
    KDA_TRY(check_device());
    kda::ProjParams p{};
    p.M = T;
    p.N = hidden;
    p.K = (int)K;
    p.a = static_cast<const uint16_t *>(y);
    p.b = static_cast<const uint16_t *>(w_out);
    p.out = static_cast<uint16_t *>(out);
    return launched(kda::launch_gemm(p, (hipStream_t)stream), "out projection");
}

size_t kda_mixer_workspace_bytes(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens) {
    if (check_geom(geom, true) != KDA_OK || n_seqs <= 0 || total_tokens < 0) return 0;
    const size_t T = (size_t)total_tokens, C = (size_t)geom->H * geom->d;
    return 5 * al256(T * C * 2) + al256(T * geom->H * 2) + al256(T * C * 2) +
           kda::chunk_workspace_bytes(geom->H, n_seqs, chunk_bound(n_seqs, total_tokens));
}

kda_status kda_mixer_prefill(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                             const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, int32_t hidden,
                             const void *x, const void *w_in, const float *a_log, const float *dt_bias,
                             const float *conv_w, const float *conv_cache_in, float *conv_cache_out,
                             const float *initial_state, float *final_state, const void *w_out, void *out,
                             void *workspace, size_t workspace_bytes, void *stream) {
    // every check of the three stages before the first launch
    KDA_TRY(check_geom(geom, true));
    long n_chunks = 0;
    KDA_TRY(check_seqlens(n_seqs, total_tokens, cu_seqlens_host, &n_chunks));
    const long C = (long)geom->H * geom->d, N = 5 * C + geom->H;
    KDA_TRY(check_gemm_dims(total_tokens, hidden, "x"));
    KDA_TRY(check_gemm_dims(N, hidden, "w_in"));
    KDA_TRY(check_gemm_dims(hidden, C, "w_out"));
    KDA_TRY(check_gemm_dims(total_tokens, C, "the KDA output"));
    KDA_TRY(check_required({{cu_seqlens_dev, "cu_seqlens_dev"}, {w_in, "w_in"}, {w_out, "w_out"},
                            {conv_w, "conv_w"}, {workspace, "workspace"}}));
    if (total_tokens > 0) KDA_TRY(check_required({{x, "x"}, {out, "out"}}));
    KDA_TRY(check_aligned({{x, "x"}, {w_in, "w_in"}, {w_out, "w_out"}, {a_log, "a_log"}, {dt_bias, "dt_bias"},
                           {conv_w, "conv_w"}, {conv_cache_in, "conv_cache_in"},
                           {conv_cache_out, "conv_cache_out"}, {initial_state, "initial_state"},
                           {final_state, "final_state"}, {out, "out"}, {workspace, "workspace"}}));
    const size_t need = kda_mixer_workspace_bytes(geom, n_seqs, total_tokens);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    KDA_TRY(check_device());
    const size_t T = (size_t)total_tokens;
    unsigned char *w = static_cast<unsigned char *>(workspace);
    void *seg[6];
    for (int i = 0; i < 5; ++i) {
        seg[i] = w;
        w += al256(T * C * 2);
    }
    seg[5] = w;
    w += al256(T * geom->H * 2);
    void *y = w;
    w += al256(T * C * 2);
    void *chunk_ws = w;
    const size_t chunk_bytes = workspace_bytes - (size_t)(w - static_cast<unsigned char *>(workspace));
    if (total_tokens > 0)
        KDA_TRY(launched(kda::launch_gemm(in_proj_params(geom, total_tokens, hidden, x, w_in, a_log, dt_bias, seg),
                                          (hipStream_t)stream), "in projection"));
    KDA_TRY(kda_prefill(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, KDA_BF16, kda::kChunk, seg[0],
                        seg[1], seg[2], conv_w, conv_cache_in, conv_cache_out, seg[4], seg[5], seg[3], initial_state,
                        final_state, y, chunk_ws, chunk_bytes, stream));
    if (total_tokens == 0) return ok();
    kda::ProjParams p{};
    p.M = total_tokens;
    p.N = hidden;
    p.K = (int)C;
    p.a = static_cast<const uint16_t *>(y);
    p.b = static_cast<const uint16_t *>(w_out);
    p.out = static_cast<uint16_t *>(out);
    return launched(kda::launch_gemm(p, (hipStream_t)stream), "out projection");
}

kda_status kda_prefill_noalloc(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                               const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                               int32_t chunk, const void *q_raw, const void *k_raw, const void *v_raw,
                               const float *conv_w, const float *conv_cache_in, float *conv_cache_out,
                               const void *log_alpha, const void *beta_logit, const void *gate_logit,
                               const float *initial_state, float *final_state, void *out, void *stream) {
    // Host checks first (nothing here touches a device), then the size limit.
    KDA_TRY(check_chunk_len(chunk));
    KDA_TRY(check_geom(geom, true));
    long n_chunks = 0;
    KDA_TRY(check_seqlens(n_seqs, total_tokens, cu_seqlens_host, &n_chunks));
    const size_t need = kda::chunk_workspace_bytes(geom->H, n_seqs, n_chunks);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES)
        return fail(KDA_ERR_WORKSPACE,
                    "kda_prefill_noalloc: this batch needs %zu bytes of chunk workspace (%ld chunks x %d heads x "
                    "74,240 B + table), more than its fixed scratch of %zu bytes; use kda_prefill with a "
                    "caller-allocated workspace",
                    need, n_chunks, geom->H, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
    // The checks kda_prefill makes of its other arguments, here too, so that
    // every invalid call is answered before a device is touched (the scratch
    // address lookup needs one).
    KDA_TRY(check_dtype(in_dtype));
    if (in_dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "the chunk path takes bf16 inputs only");
    KDA_TRY(check_required({{cu_seqlens_dev, "cu_seqlens_dev"}, {conv_w, "conv_w"}}));
    if (total_tokens > 0)
        KDA_TRY(check_required({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {log_alpha, "log_alpha"},
                                {beta_logit, "beta_logit"}, {out, "out"}}));
    KDA_TRY(check_aligned({{q_raw, "q_raw"}, {k_raw, "k_raw"}, {v_raw, "v_raw"}, {conv_w, "conv_w"},
                           {conv_cache_in, "conv_cache_in"}, {conv_cache_out, "conv_cache_out"},
                           {log_alpha, "log_alpha"}, {beta_logit, "beta_logit"}, {gate_logit, "gate_logit"},
                           {initial_state, "initial_state"}, {final_state, "final_state"}, {out, "out"}}));
    KDA_TRY(check_device());
    void *ws = nullptr;
    KDA_TRY(scratch_address(&ws));
    return kda_prefill(geom, n_seqs, total_tokens, cu_seqlens_dev, cu_seqlens_host, in_dtype, chunk, q_raw, k_raw,
                       v_raw, conv_w, conv_cache_in, conv_cache_out, log_alpha, beta_logit, gate_logit,
                       initial_state, final_state, out, ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}

// ---------------------------------------------------------------------------
// MLA decode token
// ---------------------------------------------------------------------------
namespace {

kda_status check_mla_geom(const kda_mla_geom *g) {
    if (!g) return fail(KDA_ERR_NULL, "geom is NULL");
    if (g->H <= 0 || g->H_kv <= 0 || g->H % g->H_kv != 0)
        return fail(KDA_ERR_SHAPE, "H = %d and H_kv = %d: both must be > 0 and H a multiple of H_kv", g->H, g->H_kv);
    if (g->d_qk <= 0 || g->d_v <= 0) return fail(KDA_ERR_SHAPE, "d_qk = %d and d_v = %d must be > 0", g->d_qk, g->d_v);
    if (g->d_qk > 256 || g->d_v > 256)
        return fail(KDA_ERR_UNSUPPORTED, "d_qk = %d and d_v = %d must be <= 256", g->d_qk, g->d_v);
    if (!std::isfinite(g->scale)) return fail(KDA_ERR_SHAPE, "scale must be finite");
    return KDA_OK;
}

long mla_n_split(int32_t max_len) { return (max_len - 1) / kda::mla_split_tokens() + 1; }

}  // namespace

size_t kda_mla_decode_workspace_bytes(const kda_mla_geom *geom, int32_t batch, int32_t max_len) {
    if (check_mla_geom(geom) != KDA_OK || batch < 0 || max_len <= 0) return 0;
    const size_t n = (size_t)batch * geom->H * mla_n_split(max_len);
    return al256(n * 2 * sizeof(float)) + al256(n * geom->d_v * sizeof(float));
}

kda_status kda_mla_decode_step(const kda_mla_geom *geom, int32_t batch, int32_t max_len,
                               const int32_t *cache_len_dev, const void *q, const void *k_new, const void *v_new,
                               const void *gate_logit, void *k_cache, void *v_cache, void *out, void *workspace,
                               size_t workspace_bytes, void *stream) {
    KDA_TRY(check_mla_geom(geom));
    if (batch < 0 || batch > 65535) return fail(KDA_ERR_SHAPE, "batch = %d must be in [0, 65535]", batch);
    if (geom->H > 65535) return fail(KDA_ERR_SHAPE, "H = %d must be <= 65535", geom->H);
    if (max_len <= 0) return fail(KDA_ERR_SHAPE, "max_len = %d must be > 0", max_len);
    if (mla_n_split(max_len) > 65535)   // the splits are the grid's third dimension
        return fail(KDA_ERR_SHAPE, "max_len = %d must be <= %d", max_len, 65535 * kda::mla_split_tokens());
    // one buffer resource spans a (sequence, kv head) cache block, and one the
    // whole q; each must stay below 4 GiB
    if ((long)max_len * std::max(geom->d_qk, geom->d_v) * 2 >= (1L << 32) ||
        (long)batch * geom->H * std::max(geom->d_qk, geom->d_v) * 2 >= (1L << 32))
        return fail(KDA_ERR_SHAPE, "max_len = %d or batch = %d too large for 32-bit offsets", max_len, batch);
    if (batch == 0) return ok();
    KDA_TRY(check_required({{cache_len_dev, "cache_len_dev"}, {q, "q"}, {k_new, "k_new"}, {v_new, "v_new"},
                            {k_cache, "k_cache"}, {v_cache, "v_cache"}, {out, "out"}, {workspace, "workspace"}}));
    KDA_TRY(check_aligned({{cache_len_dev, "cache_len_dev"}, {q, "q"}, {k_new, "k_new"}, {v_new, "v_new"},
                           {gate_logit, "gate_logit"}, {k_cache, "k_cache"}, {v_cache, "v_cache"}, {out, "out"},
                           {workspace, "workspace"}}));
    const size_t need = kda_mla_decode_workspace_bytes(geom, batch, max_len);
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    KDA_TRY(check_device());
    kda::MlaParams p{};
    p.batch = batch;
    p.H = geom->H;
    p.H_kv = geom->H_kv;
    p.dqk = geom->d_qk;
    p.dv = geom->d_v;
    p.max_len = max_len;
    p.n_split = (int)mla_n_split(max_len);
    p.scale = geom->scale;
    p.cache_len = cache_len_dev;
    p.q = q;
    p.k_new = k_new;
    p.v_new = v_new;
    p.gate = gate_logit;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.out = out;
    const size_t n = (size_t)batch * geom->H * p.n_split;
    p.ws_ml = static_cast<float *>(workspace);
    p.ws_acc = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + al256(n * 2 * sizeof(float)));
    // whole 16-byte chunks when every row is a multiple of 8 channels
    const bool vec = geom->d_qk % 8 == 0 && geom->d_v % 8 == 0;
    return launched(kda::launch_mla_decode(p, vec, (hipStream_t)stream), "mla decode");
}

}  // extern "C"
