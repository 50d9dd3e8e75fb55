// C ABI of libspecverify: argument validation, workspace sizing and kernel
// launch.  Declarations and the meaning of every argument are in
// include/specverify.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/specverify.h"
#include "sv_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return SV_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(sv_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

int check_attn_shape(int B, int K, int Hq, int Hkv, int D, int dtype, const int32_t* kv_len_host,
                     int prefix_len) {
    if (B < 1) return fail(SV_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
    if (B > 65536) return fail(SV_ERR_UNSUPPORTED, "B must be <= 65536 (got %d)", B);
    if (K < 0) return fail(SV_ERR_INVALID_ARG, "K must be >= 0 (got %d)", K);
    if (Hq < 1 || Hkv < 1) return fail(SV_ERR_INVALID_ARG, "head counts must be >= 1");
    if (Hq % Hkv != 0)
        return fail(SV_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
    if (dtype != SV_F32 && dtype != SV_BF16)
        return fail(SV_ERR_INVALID_ARG, "dtype must be SV_F32 or SV_BF16 (got %d)", dtype);
    if (D < 1) return fail(SV_ERR_INVALID_ARG, "head_dim must be >= 1 (got %d)", D);
    if (dtype == SV_BF16) {
        if (D != 64 && D != 128)
            return fail(SV_ERR_UNSUPPORTED, "bf16 attention supports head_dim 64 or 128 (got %d)", D);
        if (B > 2048)
            return fail(SV_ERR_UNSUPPORTED, "bf16 attention supports B <= 2048 sequences per call (got %d)", B);
        if ((Hq / Hkv) * (K + 1) > 64)
            return fail(SV_ERR_UNSUPPORTED,
                        "bf16 attention supports (Hq/Hkv)*(K+1) <= 64 query columns per kv head "
                        "(got %d)", (Hq / Hkv) * (K + 1));
    } else if (D > 256 || D % 4 != 0) {
        return fail(SV_ERR_UNSUPPORTED, "fp32 attention supports head_dim <= 256, multiple of 4 (got %d)", D);
    }
    if (prefix_len < 0) return fail(SV_ERR_INVALID_ARG, "prefix_len must be >= 0");
    if (!kv_len_host) return fail(SV_ERR_INVALID_ARG, "kv_len_host is NULL");
    for (int b = 0; b < B; ++b)
        if (kv_len_host[b] < 0)
            return fail(SV_ERR_INVALID_ARG, "kv_len_host[%d] = %d is negative", b, kv_len_host[b]);
    return SV_OK;
}

// Ragged draft lengths: cu_q_host[0] = 0 and K_b = cu_q_host[b+1] - cu_q_host[b] - 1
// >= 0; *kmax = the largest K_b.
int check_cu_q(int B, const int32_t* cu_q_host, int* kmax) {
    if (!cu_q_host) return fail(SV_ERR_INVALID_ARG, "cu_q_host is NULL");
    if (B < 1) return fail(SV_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
    if (cu_q_host[0] != 0) return fail(SV_ERR_INVALID_ARG, "cu_q_host[0] must be 0 (got %d)", cu_q_host[0]);
    int km = 0;
    for (int b = 0; b < B; ++b) {
        const long long d = static_cast<long long>(cu_q_host[b + 1]) - cu_q_host[b];
        if (d < 1)
            return fail(SV_ERR_INVALID_ARG, "sequence %d has %lld query rows (need K_b + 1 >= 1)", b, d);
        if (d - 1 > km) km = static_cast<int>(d - 1 > 0x7FFFFFFF ? 0x7FFFFFFF : d - 1);
    }
    *kmax = km;
    return SV_OK;
}

int attn_workspace(int B, int K, int Hq, int Hkv, int D, int dtype, const int32_t* kv_len_host,
                   const int32_t* cu_q_host, int prefix_len, size_t* bytes) {
    int rc = check_attn_shape(B, K, Hq, Hkv, D, dtype, kv_len_host, prefix_len);
    if (rc) return rc;
    if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
    const sv::AttnPlan plan =
        sv::attn_plan(B, K, Hq, Hkv, D, dtype == SV_BF16, kv_len_host, cu_q_host, prefix_len);
    if (!plan.ok) return fail(SV_ERR_UNSUPPORTED, "KV length bound too long (bf16: at most 2^25 keys per sequence, 2^30 64-key tiles in all)");
    *bytes = plan.bytes;
    return ok();
}

int attn_run(const void* q, const void* k_cache, const void* v_cache, const int64_t* kv_start,
             const int32_t* kv_len, const int32_t* kv_len_host, const void* k_new,
             const void* v_new, const void* k_prefix, const void* v_prefix, int prefix_len,
             void* out, const int32_t* cu_q, const int32_t* cu_q_host, int rows, int B, int K,
             int Hq, int Hkv, int D, int dtype, float softmax_scale, int32_t* status,
             void* workspace, size_t workspace_bytes, sv_stream_t stream, bool noalloc = false) {
    int rc = check_attn_shape(B, K, Hq, Hkv, D, dtype, kv_len_host, prefix_len);
    if (rc) return rc;
    if (!q || !k_cache || !v_cache || !kv_start || !kv_len || !k_new || !v_new || !out)
        return fail(SV_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if (prefix_len > 0 && (!k_prefix || !v_prefix))
        return fail(SV_ERR_INVALID_ARG, "prefix_len > 0 needs k_prefix and v_prefix");
    const size_t al = dtype == SV_BF16 ? 16 : 4;
    if (!aligned(q, al) || !aligned(k_cache, al) || !aligned(v_cache, al) || !aligned(k_new, al) ||
        !aligned(v_new, al) || !aligned(out, al) || (prefix_len > 0 && (!aligned(k_prefix, al) ||
                                                                       !aligned(v_prefix, al))))
        return fail(SV_ERR_INVALID_ARG, "tensors must be %zu-byte aligned", al);
    if (!isfinite(softmax_scale)) return fail(SV_ERR_INVALID_ARG, "softmax_scale is not finite");
    const sv::AttnPlan plan =
        sv::attn_plan(B, K, Hq, Hkv, D, dtype == SV_BF16, kv_len_host, cu_q_host, prefix_len);
    if (!plan.ok) return fail(SV_ERR_UNSUPPORTED, "KV length bound too long (bf16: at most 2^25 keys per sequence, 2^30 64-key tiles in all)");
    void* counters = nullptr;
    if (noalloc) {
        // the library's fixed scratch: counters in its counter region, the
        // partial results in its data region (sizes checked before any launch)
        size_t cbytes = 0, dbytes = 0;
        sv::noalloc_limits(&cbytes, &dbytes);
        if (plan.counter_bytes > cbytes)
            return fail(SV_ERR_UNSUPPORTED, "B*Hkv = %lld arrival counters exceed the %zu of the "
                        "fixed scratch", static_cast<long long>(B) * Hkv, cbytes / 4);
        if (plan.bytes - plan.counter_bytes > dbytes)
            return fail(SV_ERR_UNSUPPORTED, "%zu bytes of partial results exceed the %zu-byte "
                        "fixed scratch (use spec_verify_attn with a workspace)",
                        plan.bytes - plan.counter_bytes, dbytes);
        hipError_t e = sv::noalloc_scratch(as_stream(stream), &counters, &cbytes, &workspace,
                                           &workspace_bytes);
        if (e != hipSuccess)
            return fail(SV_ERR_HIP, "scratch set-up failed: %s", hipGetErrorString(e));
    } else if (!workspace || workspace_bytes < plan.bytes) {
        return fail(SV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.bytes,
                    workspace ? workspace_bytes : static_cast<size_t>(0));
    }
    sv::AttnArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.kv_start = kv_start;
    a.kv_len = kv_len;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_prefix = prefix_len > 0 ? k_prefix : nullptr;
    a.v_prefix = prefix_len > 0 ? v_prefix : nullptr;
    a.out = out;
    a.status = status;
    a.cu_q = cu_q;
    a.rows = rows;
    a.B = B;
    a.K = K;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.bf16 = dtype == SV_BF16;
    a.prefix_len = prefix_len;
    a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(D));
    a.workspace = workspace;
    a.counters = counters;
    a.ev_start = g_ev_start;
    a.ev_stop = g_ev_stop;
    hipError_t e = sv::attn_launch(a, plan, as_stream(stream));
    if (e != hipSuccess) return fail(SV_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    return ok();
}

int accept_run(const void* target_logits, const void* draft_logits, int logits_dtype,
               const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
               const int32_t* cu_q, long long nt, int B, int K, int V, float temperature,
               float top_p, int top_k, int greedy, int32_t* n_accepted, int32_t* out_tokens,
               int32_t* status, void* workspace, size_t workspace_bytes, sv_stream_t stream,
               const sv::AcceptArgs* fused = nullptr) {
    if (V > sv::accept_max_vocab())
        return fail(SV_ERR_UNSUPPORTED, "vocabulary above %d", sv::accept_max_vocab());
    if (logits_dtype != SV_F32 && logits_dtype != SV_BF16)
        return fail(SV_ERR_INVALID_ARG, "logits_dtype must be SV_F32 or SV_BF16");
    if (!(temperature > 0.0f) || !isfinite(temperature))
        return fail(SV_ERR_INVALID_ARG, "temperature must be finite and > 0");
    if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(SV_ERR_INVALID_ARG, "top_p must be in (0, 1]");
    if (top_k < 0) return fail(SV_ERR_INVALID_ARG, "top_k must be >= 0 (0: off)");
    if (K > sv::accept_max_drafts())
        return fail(SV_ERR_UNSUPPORTED, "K above %d", sv::accept_max_drafts());
    if (2 * nt - B > 0x7FFFFFFF / 64)
        return fail(SV_ERR_UNSUPPORTED, "too many logit rows (%lld)", 2 * nt - B);
    if (B == 0) return ok();
    if (!target_logits || !n_accepted || !out_tokens)
        return fail(SV_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if (K > 0 && !draft_tokens) return fail(SV_ERR_INVALID_ARG, "draft_tokens is NULL");
    if (!greedy) {
        if (!u_sample || (K > 0 && (!u_accept || !draft_logits)))
            return fail(SV_ERR_INVALID_ARG, "draft_logits, u_accept and u_sample are required unless greedy");
    }
    const size_t need = sv::accept_workspace_bytes(B, nt, V);
    if (!workspace || workspace_bytes < need)
        return fail(SV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : static_cast<size_t>(0));
    const size_t al = logits_dtype == SV_BF16 ? 8 : 16;
    if (V % 4 == 0 && (!aligned(target_logits, al) || (draft_logits && !aligned(draft_logits, al))))
        return fail(SV_ERR_INVALID_ARG, "logits must be %zu-byte aligned", al);
    sv::AcceptArgs a{};
    a.target_logits = target_logits;
    a.draft_logits = draft_logits;
    a.draft_tokens = draft_tokens;
    a.u_accept = u_accept;
    a.u_sample = u_sample;
    a.n_accepted = n_accepted;
    a.out_tokens = out_tokens;
    a.status = status;
    a.workspace = workspace;
    a.cu_q = cu_q;
    a.nt = static_cast<int>(nt);
    a.B = B;
    a.K = K;
    a.V = V;
    a.bf16 = logits_dtype == SV_BF16;
    a.greedy = greedy ? 1 : 0;
    a.temperature = temperature;
    a.top_p = top_p;
    a.top_k = top_k;
    if (fused) {
        a.kv_len = fused->kv_len;
        a.kv_start = fused->kv_start;
        a.k_cache = fused->k_cache;
        a.v_cache = fused->v_cache;
        a.k_new = fused->k_new;
        a.v_new = fused->v_new;
        a.tokens_packed = fused->tokens_packed;
        a.cu_tokens = fused->cu_tokens;
        a.row_bytes = fused->row_bytes;
        a.pre_m[0] = fused->pre_m[0];
        a.pre_m[1] = fused->pre_m[1];
        a.pre_s[0] = fused->pre_s[0];
        a.pre_s[1] = fused->pre_s[1];
        a.pre_parts = fused->pre_parts;
    }
    hipError_t e = sv::accept_launch(a, as_stream(stream));
    if (e != hipSuccess) return fail(SV_ERR_HIP, "sampler launch failed: %s", hipGetErrorString(e));
    return ok();
}

int compact_run(const int32_t* n_accepted, const int32_t* out_tokens, int32_t* kv_len,
                const int64_t* kv_start, void* k_cache, void* v_cache, const void* k_new,
                const void* v_new, int32_t* tokens_packed, int32_t* cu_tokens,
                const int32_t* cu_q, int B, int K, int Hkv, int D, int dtype, int32_t* status,
                sv_stream_t stream) {
    if (B < 0 || Hkv < 1 || D < 1)
        return fail(SV_ERR_INVALID_ARG, "need B >= 0, Hkv >= 1, D >= 1");
    if (dtype != SV_F32 && dtype != SV_BF16)
        return fail(SV_ERR_INVALID_ARG, "dtype must be SV_F32 or SV_BF16");
    const int es = dtype == SV_BF16 ? 2 : 4;
    if ((static_cast<size_t>(Hkv) * D * es) % 4 != 0)
        return fail(SV_ERR_UNSUPPORTED, "a KV row must be a multiple of 4 bytes");
    if (B == 0) return ok();
    if (!n_accepted || !out_tokens || !kv_len || !kv_start || !k_cache || !v_cache || !k_new ||
        !v_new || !tokens_packed || !cu_tokens)
        return fail(SV_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    sv::CompactArgs a{};
    a.n_accepted = n_accepted;
    a.out_tokens = out_tokens;
    a.kv_len = kv_len;
    a.kv_start = kv_start;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_new = k_new;
    a.v_new = v_new;
    a.tokens_packed = tokens_packed;
    a.cu_tokens = cu_tokens;
    a.status = status;
    a.cu_q = cu_q;
    a.B = B;
    a.K = K;
    a.Hkv = Hkv;
    a.D = D;
    a.elem_bytes = es;
    hipError_t e = sv::compact_launch(a, as_stream(stream));
    if (e != hipSuccess) return fail(SV_ERR_HIP, "compaction launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* sv_last_error(void) { return g_err; }

int sv_version(void) { return 100; }

int sv_set_kernel_events(void* start, void* stop) {
    if (start && stop) {
        g_ev_start = static_cast<hipEvent_t>(start);
        g_ev_stop = static_cast<hipEvent_t>(stop);
    } else {
        g_ev_start = g_ev_stop = nullptr;
    }
    return ok();
}

int spec_verify_attn_workspace_size(int B, int K, int Hq, int Hkv, int D, int dtype,
                                    const int32_t* kv_len_host, int prefix_len, size_t* bytes) {
    return attn_workspace(B, K, Hq, Hkv, D, dtype, kv_len_host, nullptr, prefix_len, bytes);
}

int spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const int64_t* kv_start, const int32_t* kv_len,
                     const int32_t* kv_len_host, const void* k_new, const void* v_new,
                     const void* k_prefix, const void* v_prefix, int prefix_len,
                     void* out, int B, int K, int Hq, int Hkv, int D, int dtype,
                     float softmax_scale, int32_t* status, void* workspace,
                     size_t workspace_bytes, sv_stream_t stream) {
    const long long rows = static_cast<long long>(B) * (K + 1);
    if (B >= 1 && K >= 0 && rows > 0x7FFFFFFF)
        return fail(SV_ERR_UNSUPPORTED, "B*(K+1) above 2^31 - 1");
    return attn_run(q, k_cache, v_cache, kv_start, kv_len, kv_len_host, k_new, v_new, k_prefix,
                    v_prefix, prefix_len, out, nullptr, nullptr, static_cast<int>(rows), B, K, Hq,
                    Hkv, D, dtype, softmax_scale, status, workspace, workspace_bytes, stream);
}

int spec_verify_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             const int64_t* kv_start, const int32_t* kv_len,
                             const int32_t* kv_len_host, const void* k_new, const void* v_new,
                             const void* k_prefix, const void* v_prefix, int prefix_len,
                             void* out, int B, int K, int Hq, int Hkv, int D, int dtype,
                             float softmax_scale, int32_t* status, sv_stream_t stream) {
    const long long rows = static_cast<long long>(B) * (K + 1);
    if (B >= 1 && K >= 0 && rows > 0x7FFFFFFF)
        return fail(SV_ERR_UNSUPPORTED, "B*(K+1) above 2^31 - 1");
    return attn_run(q, k_cache, v_cache, kv_start, kv_len, kv_len_host, k_new, v_new, k_prefix,
                    v_prefix, prefix_len, out, nullptr, nullptr, static_cast<int>(rows), B, K, Hq,
                    Hkv, D, dtype, softmax_scale, status, nullptr, 0, stream, true);
}

int spec_verify_attn_ragged_workspace_size(int B, int Hq, int Hkv, int D, int dtype,
                                           const int32_t* kv_len_host, const int32_t* cu_q_host,
                                           int prefix_len, size_t* bytes) {
    int kmax = 0;
    int rc = check_cu_q(B, cu_q_host, &kmax);
    if (rc) return rc;
    return attn_workspace(B, kmax, Hq, Hkv, D, dtype, kv_len_host, cu_q_host, prefix_len, bytes);
}

int spec_verify_attn_ragged(const void* q, const void* k_cache, const void* v_cache,
                            const int64_t* kv_start, const int32_t* kv_len,
                            const int32_t* kv_len_host, const void* k_new, const void* v_new,
                            const void* k_prefix, const void* v_prefix, int prefix_len,
                            void* out, const int32_t* cu_q, const int32_t* cu_q_host, int B,
                            int Hq, int Hkv, int D, int dtype, float softmax_scale,
                            int32_t* status, void* workspace, size_t workspace_bytes,
                            sv_stream_t stream) {
    int kmax = 0;
    int rc = check_cu_q(B, cu_q_host, &kmax);
    if (rc) return rc;
    if (!cu_q) return fail(SV_ERR_INVALID_ARG, "cu_q is NULL");
    return attn_run(q, k_cache, v_cache, kv_start, kv_len, kv_len_host, k_new, v_new, k_prefix,
                    v_prefix, prefix_len, out, cu_q, cu_q_host, cu_q_host[B], B, kmax, Hq, Hkv, D,
                    dtype, softmax_scale, status, workspace, workspace_bytes, stream);
}

int spec_accept_workspace_size(int B, int K, int V, size_t* bytes) {
    if (B < 0 || K < 0 || V < 1) return fail(SV_ERR_INVALID_ARG, "need B >= 0, K >= 0, V >= 1");
    if (V > sv::accept_max_vocab())
        return fail(SV_ERR_UNSUPPORTED, "vocabulary above %d", sv::accept_max_vocab());
    if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = sv::accept_workspace_bytes(B, static_cast<long long>(B) * (K + 1), V);
    return ok();
}

int spec_accept(const void* target_logits, const void* draft_logits, int logits_dtype,
                const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                int B, int K, int V, float temperature, float top_p, int greedy,
                int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
                void* workspace, size_t workspace_bytes, sv_stream_t stream) {
    if (B < 0 || K < 0 || V < 1) return fail(SV_ERR_INVALID_ARG, "need B >= 0, K >= 0, V >= 1");
    return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept, u_sample,
                      nullptr, static_cast<long long>(B) * (K + 1), B, K, V, temperature, top_p,
                      0, greedy, n_accepted, out_tokens, status, workspace, workspace_bytes, stream);
}

int spec_accept_ragged_workspace_size(int B, const int32_t* cu_q_host, int V, size_t* bytes) {
    int kmax = 0;
    int rc = check_cu_q(B, cu_q_host, &kmax);
    if (rc) return rc;
    if (V < 1) return fail(SV_ERR_INVALID_ARG, "need V >= 1");
    if (V > sv::accept_max_vocab())
        return fail(SV_ERR_UNSUPPORTED, "vocabulary above %d", sv::accept_max_vocab());
    if (!bytes) return fail(SV_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = sv::accept_workspace_bytes(B, cu_q_host[B], V);
    return ok();
}

int spec_accept_ragged(const void* target_logits, const void* draft_logits, int logits_dtype,
                       const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                       const int32_t* cu_q, const int32_t* cu_q_host, int B, int V,
                       float temperature, float top_p, int greedy, int32_t* n_accepted,
                       int32_t* out_tokens, int32_t* status, void* workspace,
                       size_t workspace_bytes, sv_stream_t stream) {
    int kmax = 0;
    int rc = check_cu_q(B, cu_q_host, &kmax);
    if (rc) return rc;
    if (!cu_q) return fail(SV_ERR_INVALID_ARG, "cu_q is NULL");
    if (V < 1) return fail(SV_ERR_INVALID_ARG, "need V >= 1");
    return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept, u_sample,
                      cu_q, cu_q_host[B], B, kmax, V, temperature, top_p, 0, greedy, n_accepted,
                      out_tokens, status, workspace, workspace_bytes, stream);
}

int spec_accept_ex(const void* target_logits, const void* draft_logits, int logits_dtype,
                   const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                   const int32_t* cu_q, const int32_t* cu_q_host, int B, int K, int V,
                   float temperature, float top_p, int top_k, int greedy, int32_t* n_accepted,
                   int32_t* out_tokens, int32_t* status, void* workspace,
                   size_t workspace_bytes, sv_stream_t stream) {
    if (!cu_q && !cu_q_host) {
        if (B < 0 || K < 0 || V < 1) return fail(SV_ERR_INVALID_ARG, "need B >= 0, K >= 0, V >= 1");
        return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept,
                          u_sample, nullptr, static_cast<long long>(B) * (K + 1), B, K, V,
                          temperature, top_p, top_k, greedy, n_accepted, out_tokens, status,
                          workspace, workspace_bytes, stream);
    }
    int kmax = 0;
    int rc = check_cu_q(B, cu_q_host, &kmax);
    if (rc) return rc;
    if (!cu_q) return fail(SV_ERR_INVALID_ARG, "cu_q is NULL");
    if (V < 1) return fail(SV_ERR_INVALID_ARG, "need V >= 1");
    return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept, u_sample,
                      cu_q, cu_q_host[B], B, kmax, V, temperature, top_p, top_k, greedy,
                      n_accepted, out_tokens, status, workspace, workspace_bytes, stream);
}

int spec_compact_kv(const int32_t* n_accepted, const int32_t* out_tokens, int32_t* kv_len,
                    const int64_t* kv_start, void* k_cache, void* v_cache,
                    const void* k_new, const void* v_new, int32_t* tokens_packed,
                    int32_t* cu_tokens, int B, int K, int Hkv, int D, int dtype,
                    int32_t* status, sv_stream_t stream) {
    if (K < 0) return fail(SV_ERR_INVALID_ARG, "need K >= 0");
    return compact_run(n_accepted, out_tokens, kv_len, kv_start, k_cache, v_cache, k_new, v_new,
                       tokens_packed, cu_tokens, nullptr, B, K, Hkv, D, dtype, status, stream);
}

int spec_accept_compact(const void* target_logits, const void* draft_logits, int logits_dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        const int32_t* cu_q, const int32_t* cu_q_host, int B, int K, int V,
                        float temperature, float top_p, int top_k, int greedy,
                        int32_t* n_accepted, int32_t* out_tokens, int32_t* kv_len,
                        const int64_t* kv_start, void* k_cache, void* v_cache, const void* k_new,
                        const void* v_new, int Hkv, int D, int kv_dtype, int32_t* tokens_packed,
                        int32_t* cu_tokens, int32_t* status, void* workspace,
                        size_t workspace_bytes, sv_stream_t stream) {
    if (Hkv < 1 || D < 1) return fail(SV_ERR_INVALID_ARG, "need Hkv >= 1, D >= 1");
    if (kv_dtype != SV_F32 && kv_dtype != SV_BF16)
        return fail(SV_ERR_INVALID_ARG, "kv_dtype must be SV_F32 or SV_BF16");
    const int es = kv_dtype == SV_BF16 ? 2 : 4;
    if ((static_cast<size_t>(Hkv) * D * es) % 4 != 0)
        return fail(SV_ERR_UNSUPPORTED, "a KV row must be a multiple of 4 bytes");
    if (B > 0 && (!kv_len || !kv_start || !k_cache || !v_cache || !k_new || !v_new ||
                  !tokens_packed || !cu_tokens))
        return fail(SV_ERR_INVALID_ARG, "a required compaction pointer is NULL");
    sv::AcceptArgs f{};
    f.kv_len = kv_len;
    f.kv_start = kv_start;
    f.k_cache = k_cache;
    f.v_cache = v_cache;
    f.k_new = k_new;
    f.v_new = v_new;
    f.tokens_packed = tokens_packed;
    f.cu_tokens = cu_tokens;
    f.row_bytes = static_cast<size_t>(Hkv) * D * es;
    if (!cu_q && !cu_q_host) {
        if (B < 0 || K < 0 || V < 1) return fail(SV_ERR_INVALID_ARG, "need B >= 0, K >= 0, V >= 1");
        return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept,
                          u_sample, nullptr, static_cast<long long>(B) * (K + 1), B, K, V,
                          temperature, top_p, top_k, greedy, n_accepted, out_tokens, status,
                          workspace, workspace_bytes, stream, &f);
    }
    int kmax = 0;
    int rc = check_cu_q(B, cu_q_host, &kmax);
    if (rc) return rc;
    if (!cu_q) return fail(SV_ERR_INVALID_ARG, "cu_q is NULL");
    if (V < 1) return fail(SV_ERR_INVALID_ARG, "need V >= 1");
    return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept, u_sample,
                      cu_q, cu_q_host[B], B, kmax, V, temperature, top_p, top_k, greedy,
                      n_accepted, out_tokens, status, workspace, workspace_bytes, stream, &f);
}

int spec_lm_head_parts(int V) {
    if (V < 1) return fail(SV_ERR_INVALID_ARG, "need V >= 1");
    ok();
    return sv::lm_head_parts(V);
}

int spec_lm_head_stats(const void* hidden, const void* weight, int rows, int H, int V,
                       float temperature, float* logits, float* part_max, double* part_sum,
                       sv_stream_t stream) {
    if (rows < 0 || H < 1 || V < 1) return fail(SV_ERR_INVALID_ARG, "need rows >= 0, H >= 1, V >= 1");
    if (H % 32 != 0) return fail(SV_ERR_UNSUPPORTED, "H must be a multiple of 32");
    if (!(temperature > 0.0f) || !isfinite(temperature))
        return fail(SV_ERR_INVALID_ARG, "temperature must be finite and > 0");
    if (static_cast<long long>(rows) * V > 0x7FFFFFFFLL * 4)
        return fail(SV_ERR_UNSUPPORTED, "rows * V too large");
    if (rows == 0) return ok();
    if (!hidden || !weight || !logits || !part_max || !part_sum)
        return fail(SV_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(logits, 16))
        return fail(SV_ERR_INVALID_ARG, "hidden, weight and logits must be 16-byte aligned");
    sv::LmArgs a{};
    a.hidden = hidden;
    a.weight = weight;
    a.rows = rows;
    a.H = H;
    a.V = V;
    a.temperature = temperature;
    a.logits = logits;
    a.part_max = part_max;
    a.part_sum = part_sum;
    hipError_t e = sv::lm_head_launch(a, as_stream(stream));
    if (e != hipSuccess) return fail(SV_ERR_HIP, "LM head launch failed: %s", hipGetErrorString(e));
    return ok();
}

int spec_accept_prestats(const void* target_logits, const void* draft_logits, int logits_dtype,
                         const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                         const int32_t* cu_q, const int32_t* cu_q_host, int B, int K, int V,
                         float temperature, float top_p, int top_k, int greedy,
                         const float* target_part_max, const double* target_part_sum,
                         const float* draft_part_max, const double* draft_part_sum, int parts,
                         int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
                         void* workspace, size_t workspace_bytes, sv_stream_t stream) {
    if (parts < 1) return fail(SV_ERR_INVALID_ARG, "need parts >= 1");
    if (B > 0 && (!target_part_max || !target_part_sum))
        return fail(SV_ERR_INVALID_ARG, "target row statistics are NULL");
    if (B > 0 && !greedy && (K > 0 || cu_q_host) && (!draft_part_max || !draft_part_sum))
        return fail(SV_ERR_INVALID_ARG, "draft row statistics are NULL");
    sv::AcceptArgs f{};
    f.pre_m[0] = target_part_max;
    f.pre_s[0] = target_part_sum;
    f.pre_m[1] = draft_part_max;
    f.pre_s[1] = draft_part_sum;
    f.pre_parts = parts;
    if (!cu_q && !cu_q_host) {
        if (B < 0 || K < 0 || V < 1) return fail(SV_ERR_INVALID_ARG, "need B >= 0, K >= 0, V >= 1");
        return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept,
                          u_sample, nullptr, static_cast<long long>(B) * (K + 1), B, K, V,
                          temperature, top_p, top_k, greedy, n_accepted, out_tokens, status,
                          workspace, workspace_bytes, stream, &f);
    }
    int kmax = 0;
    int rc = check_cu_q(B, cu_q_host, &kmax);
    if (rc) return rc;
    if (!cu_q) return fail(SV_ERR_INVALID_ARG, "cu_q is NULL");
    if (V < 1) return fail(SV_ERR_INVALID_ARG, "need V >= 1");
    return accept_run(target_logits, draft_logits, logits_dtype, draft_tokens, u_accept, u_sample,
                      cu_q, cu_q_host[B], B, kmax, V, temperature, top_p, top_k, greedy,
                      n_accepted, out_tokens, status, workspace, workspace_bytes, stream, &f);
}

int spec_compact_kv_ragged(const int32_t* n_accepted, const int32_t* out_tokens, int32_t* kv_len,
                           const int64_t* kv_start, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, int32_t* tokens_packed,
                           int32_t* cu_tokens, const int32_t* cu_q, int B, int Hkv, int D,
                           int dtype, int32_t* status, sv_stream_t stream) {
    if (B > 0 && !cu_q) return fail(SV_ERR_INVALID_ARG, "cu_q is NULL");
    return compact_run(n_accepted, out_tokens, kv_len, kv_start, k_cache, v_cache, k_new, v_new,
                       tokens_packed, cu_tokens, cu_q, B, 0, Hkv, D, dtype, status, stream);
}

}  // extern "C"
