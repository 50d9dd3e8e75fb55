/*
 * libspecverify -- the verify step of batched speculative sampling on one
 * AMD Instinct MI355X (gfx950).
 *
 * The step scores K draft tokens per sequence with the target model and keeps
 * the longest prefix that the modified rejection scheme accepts:
 *
 *   spec_verify_attn  target attention for the K+1 verify queries of every
 *                     sequence over its own ragged, unpadded KV cache, with an
 *                     optional shared prompt prefix read once (bifurcated).
 *   spec_accept       softmax with temperature and nucleus on target and draft
 *                     logits, left-to-right accept test min(1, q/p), residual
 *                     resample from (q - p)_+, bonus token when all K pass.
 *   spec_compact_kv   padding-free compaction of the accepted tokens and KV rows.
 *
 * Sources, cited by page title and section:
 *   [SpS] "Accelerating Large Language Model Decoding with Speculative
 *         Sampling" (Chen et al.): "Conditional scoring", "Modified rejection
 *         sampling", Theorem 1.
 *   [BASS] "BASS: Batched Attention-optimized Speculative Sampling": abstract
 *         (batched speculative decoding, each sequence its own accepted length).
 *   [EMS] "EMS-SD: Efficient Multi-sample Speculative Decoding": abstract
 *         (different accepted counts per sample, no padding tokens).
 *   [BIF] bifurcated-attention abstract (Athiwaratkun et al.): attention split
 *         into a GEMM over the shared prefill KV and one over per-sample KV;
 *         same FLOPs, exact result, less memory IO.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory, allocated and owned by the caller,
 *     row-major and contiguous, unless its comment says "host".
 *   - The library never allocates, never synchronizes the device, and enqueues
 *     its kernels only on `stream` (a hipStream_t; NULL = the null stream).
 *   - Return value: SV_OK (0) or a negative sv_status.  On error nothing has
 *     been enqueued and sv_last_error() (thread-local) describes the problem.
 *   - `status`, where present, is a device int32 the caller zeroes; kernels
 *     store the first data error they meet there (SV_DEV_*), never abort.
 *   - `workspace` is caller-owned device memory of at least the size the
 *     matching *_workspace_size call reports.  It must be zero-filled once
 *     before its first use; every call leaves it ready for the next call
 *     with the same B (and, for attention, the same Hkv) -- other lengths,
 *     draft counts and vocabularies may change from call to call if the
 *     workspace is large enough for each.  Zero it again before a call with
 *     another B or Hkv.  One workspace serves one call at a time (calls on
 *     different streams need different workspaces).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sv_stream_t; /* = hipStream_t */

typedef enum {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = -1, /* null pointer, bad size or bad parameter value */
    SV_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim)     */
    SV_ERR_WORKSPACE = -3,   /* workspace smaller than required               */
    SV_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed    */
} sv_status;

/* Element types of tensors. */
enum { SV_F32 = 0, SV_BF16 = 1 };

/* Device-side data errors written to `status` (first one wins). */
enum {
    SV_DEV_OK = 0,
    SV_DEV_BAD_TOKEN = 1,   /* a draft or output token id outside [0, V)          */
    SV_DEV_BAD_UNIFORM = 2, /* a uniform outside [0, 1)                           */
    SV_DEV_BAD_LENGTH = 3,  /* kv_len[b] < 0 or above the host bound kv_len_host  */
    SV_DEV_BAD_COUNT = 4    /* n_accepted[b] outside [0, K]                       */
};

/* Last error message of the calling thread ("" if none). */
const char* sv_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int sv_version(void);

/* ------------------------------------------------------------------------
 * spec_verify_attn -- target attention of the K+1 verify queries.
 *
 * [SpS] "Conditional scoring": one target call scores all K drafted positions
 * plus the next one; attention reads the KV cache of all previous tokens and
 * its cost does not grow with K.  [BASS], [EMS]: sequences keep their own
 * lengths, with no padding.  [BIF]: a prompt prefix shared by all sequences is
 * read once for all of them, with the exact result.
 *
 * For sequence b (0 <= b < B), query j (0 <= j <= K) and query head h, with
 * kv head g = h / (Hq / Hkv) (contiguous grouping; Hq == Hkv is MHA):
 *   keys/values = prefix rows [0, prefix_len)            (if prefix_len > 0)
 *              ++ cache rows kv_start[b] + [0, kv_len[b])
 *              ++ new rows b*(K+1) + [0, j]               (causal among new rows)
 *   out[b*(K+1)+j, h, :] = softmax(scale * K q) V,  scale = softmax_scale, or
 *                          1/sqrt(D) when softmax_scale <= 0.
 * No position term is added: q and k arrive position-encoded.
 *
 * q, out        [B*(K+1), Hq, D]   dtype; row b*(K+1)+j is query j of sequence b
 * k_cache,
 * v_cache       [rows, Hkv, D]     dtype; sequence b owns rows kv_start[b]..
 * kv_start      [B] int64          first cache row of sequence b
 * kv_len        [B] int32          rows cached BEFORE this step (L_b >= 0)
 * kv_len_host   [B] int32, HOST    an upper bound of kv_len (e.g. a copy); it
 *                                  sizes the grid and the workspace only
 * k_new, v_new  [B*(K+1), Hkv, D]  K/V of the K+1 verify tokens
 * k_prefix,
 * v_prefix      [prefix_len, Hkv, D] shared prefix, or NULL with prefix_len 0
 * dtype         SV_BF16 (MFMA path, D in {64, 128}) or SV_F32 (D <= 256)
 * status        device int32 or NULL: SV_DEV_BAD_LENGTH if kv_len > bound
 * Accumulation is fp32; bf16 outputs are rounded to nearest even.
 * ------------------------------------------------------------------------ */
int spec_verify_attn_workspace_size(int B, int K, int Hq, int Hkv, int D, int dtype,
                                    const int32_t* kv_len_host, int prefix_len,
                                    size_t* bytes);

int spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const int64_t* kv_start, const int32_t* kv_len,
                     const int32_t* kv_len_host, const void* k_new, const void* v_new,
                     const void* k_prefix, const void* v_prefix, int prefix_len,
                     void* out, int B, int K, int Hq, int Hkv, int D, int dtype,
                     float softmax_scale, int32_t* status, void* workspace,
                     size_t workspace_bytes, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * spec_verify_attn_noalloc -- spec_verify_attn without a workspace argument
 * and without any device allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * operation, arguments (minus the workspace), kernels and results as
 * spec_verify_attn; its arrival counters and split-K partial results live in
 * a fixed 32 MiB device array of the library, one per GPU, held until the
 * process ends.  The first call on a device looks the array up and enqueues a
 * clear of its counters on `stream`; every completed call leaves them at zero.
 * Limits: B * Hkv <= 65536, and the partial results of the call (the
 * workspace spec_verify_attn_workspace_size reports, less its counter
 * region) within 32 MiB - 256 KiB; larger problems return SV_ERR_UNSUPPORTED
 * before anything is enqueued.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race.
 * ------------------------------------------------------------------------ */
int spec_verify_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             const int64_t* kv_start, const int32_t* kv_len,
                             const int32_t* kv_len_host, const void* k_new, const void* v_new,
                             const void* k_prefix, const void* v_prefix, int prefix_len,
                             void* out, int B, int K, int Hq, int Hkv, int D, int dtype,
                             float softmax_scale, int32_t* status, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * spec_accept -- modified rejection sampling, one verify round per sequence.
 *
 * [SpS] "Modified rejection sampling": with q the target and p the draft
 * distribution, draft x_j is accepted with probability min(1, q(x_j)/p(x_j)),
 * left to right; at the first rejection the position is resampled from
 * (q - p)_+ = max(0, q - p) / sum max(0, q - p); if all K are accepted a bonus
 * token is sampled from the last target row.  Temperature and nucleus modify
 * both distributions first.  Theorem 1: the emitted tokens follow q.
 *
 * Given the uniforms, the result is deterministic:
 *   q'_j, p'_j : softmax((z - max z) / temperature), then, if top_p < 1, the
 *                smallest tie-closed set of top tokens whose mass is >= top_p,
 *                renormalised.
 *   accept x_j iff u_accept[b, j] * p'_j(x_j) < q'_j(x_j)  (p' = 0: iff q' > 0)
 *   draw       : the smallest token id i with u_sample[b] * S < C_i, C the
 *                running sum of the weights in ascending id order, S = C_{V-1};
 *                weights (q'_j - p'_j)_+ after a rejection at j (q'_j if that
 *                has zero mass), q'_K for the bonus.
 *   greedy != 0: accept while x_j == argmax target row j (lowest id on ties);
 *                emit argmax of the stopping row; uniforms are not read.
 * Precision: row normalisers, masses and the draw are computed in fp64.
 *
 * target_logits [B, K+1, V]  logits_dtype (SV_F32 or SV_BF16)
 * draft_logits  [B, K, V]    logits_dtype; may be NULL iff greedy
 * draft_tokens  [B, K] int32 ids in [0, V)
 * u_accept      [B, K] float in [0, 1);  u_sample [B] float in [0, 1)
 * temperature > 0;  0 < top_p <= 1 (1 disables the nucleus)
 * n_accepted    [B] int32 out: n_b in [0, K]
 * out_tokens    [B, K+1] int32 out: drafts 0..n_b-1, the drawn token at n_b,
 *               -1 after it
 * status        device int32 or NULL: SV_DEV_BAD_TOKEN / SV_DEV_BAD_UNIFORM
 * ------------------------------------------------------------------------ */
int spec_accept_workspace_size(int B, int K, int V, size_t* bytes);

int spec_accept(const void* target_logits, const void* draft_logits, int logits_dtype,
                const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                int B, int K, int V, float temperature, float top_p, int greedy,
                int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
                void* workspace, size_t workspace_bytes, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * spec_compact_kv -- padding-free compaction after a verify round.
 *
 * [EMS]: samples accept different numbers of tokens; they are packed without
 * padding tokens.  With e_b = n_accepted[b] + 1:
 *   cu_tokens[0] = 0, cu_tokens[b+1] = cu_tokens[b] + e_b
 *   tokens_packed[cu_tokens[b] + i] = out_tokens[b, i]          (i < e_b)
 *   cache rows kv_start[b] + kv_len[b] + i <- new rows b*(K+1) + i   (K and V)
 *   kv_len[b] += e_b
 * The KV of the inputs 0..n_b of the round becomes valid; the KV of the token
 * drawn at n_b is produced by the next round.  The caller guarantees capacity
 * for kv_len[b] + K + 1 rows at kv_start[b].
 *
 * n_accepted [B] int32, out_tokens [B, K+1] int32 (from spec_accept)
 * kv_len     [B] int32 in/out;  kv_start [B] int64
 * k_cache, v_cache [rows, Hkv, D] dtype, in/out;  k_new, v_new [B*(K+1), Hkv, D]
 * tokens_packed [B*(K+1)] int32 out (first cu_tokens[B] valid; rest untouched)
 * cu_tokens  [B+1] int32 out
 * status     device int32 or NULL: SV_DEV_BAD_COUNT if n_accepted[b] not in [0, K]
 *            (that sequence is then left unchanged)
 * ------------------------------------------------------------------------ */
int spec_compact_kv(const int32_t* n_accepted, const int32_t* out_tokens, int32_t* kv_len,
                    const int64_t* kv_start, void* k_cache, void* v_cache,
                    const void* k_new, const void* v_new, int32_t* tokens_packed,
                    int32_t* cu_tokens, int B, int K, int Hkv, int D, int dtype,
                    int32_t* status, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * Ragged draft lengths -- every sequence with its own K_b.
 *
 * [EMS]: samples may carry different numbers of prediction tokens, handled
 * without padding.  The same three operations, with the K_b + 1 query rows of
 * sequence b packed back to back:
 *   cu_q       [B+1] int32 device: cu_q[0] = 0, sequence b owns query rows
 *              cu_q[b] .. cu_q[b+1]-1, so K_b = cu_q[b+1] - cu_q[b] - 1 >= 0
 *   cu_q_host  [B+1] int32, HOST: the same offsets (they size the grid and the
 *              workspace and bound K_b); the device copy must hold equal values
 * and every "b*(K+1) + j" row of the uniform calls above becomes cu_q[b] + j:
 *   attention  q, out, k_new, v_new [cu_q[B], ...]; query j <= K_b of sequence
 *              b sees its cache and new rows cu_q[b] .. cu_q[b]+j.  The limits
 *              of spec_verify_attn hold with K = max K_b.
 *   sampler    target_logits [cu_q[B], V] (row cu_q[b] + j is target row j of
 *              b), draft_logits [cu_q[B] - B, V], draft_tokens and u_accept
 *              [cu_q[B] - B] (sequence b's K_b entries start at cu_q[b] - b),
 *              u_sample [B], n_accepted [B] (n_b in [0, K_b]), out_tokens
 *              [cu_q[B]] (sequence b's K_b + 1 entries start at cu_q[b]).
 *              K_b <= 64.
 *   compaction new rows cu_q[b] .. cu_q[b] + n_b are appended; out_tokens as
 *              from spec_accept_ragged; tokens_packed [cu_q[B]];
 *              SV_DEV_BAD_COUNT if n_accepted[b] is not in [0, K_b].
 * With cu_q[b] = b*(K+1) every result equals that of the uniform call.
 * ------------------------------------------------------------------------ */
int spec_verify_attn_ragged_workspace_size(int B, int Hq, int Hkv, int D, int dtype,
                                           const int32_t* kv_len_host, const int32_t* cu_q_host,
                                           int prefix_len, size_t* bytes);

int spec_verify_attn_ragged(const void* q, const void* k_cache, const void* v_cache,
                            const int64_t* kv_start, const int32_t* kv_len,
                            const int32_t* kv_len_host, const void* k_new, const void* v_new,
                            const void* k_prefix, const void* v_prefix, int prefix_len,
                            void* out, const int32_t* cu_q, const int32_t* cu_q_host, int B,
                            int Hq, int Hkv, int D, int dtype, float softmax_scale,
                            int32_t* status, void* workspace, size_t workspace_bytes,
                            sv_stream_t stream);

int spec_accept_ragged_workspace_size(int B, const int32_t* cu_q_host, int V, size_t* bytes);

int spec_accept_ragged(const void* target_logits, const void* draft_logits, int logits_dtype,
                       const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                       const int32_t* cu_q, const int32_t* cu_q_host, int B, int V,
                       float temperature, float top_p, int greedy, int32_t* n_accepted,
                       int32_t* out_tokens, int32_t* status, void* workspace,
                       size_t workspace_bytes, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * spec_accept_ex -- spec_accept / spec_accept_ragged with a top-k filter.
 *
 * [SpS] "Modified rejection sampling": standard sampling methods such as
 * top-k and nucleus modify the probabilities before the scheme, for q and p
 * alike.  Order: temperature, then top-k, then nucleus:
 *   top-k (0 < top_k < V): keep the tokens whose logit is >= the top_k-th
 *          largest logit of the row (ties at the boundary are all kept),
 *          renormalised; the nucleus then works on that distribution.
 * top_k = 0 (or >= V) turns it off; greedy ignores it (the argmax is kept).
 * cu_q = cu_q_host = NULL: K drafts in every sequence, the layouts of
 * spec_accept (workspace: spec_accept_workspace_size).  Otherwise the ragged
 * layouts of spec_accept_ragged, K unused (workspace:
 * spec_accept_ragged_workspace_size).  Every other argument as there.
 * ------------------------------------------------------------------------ */
int spec_accept_ex(const void* target_logits, const void* draft_logits, int logits_dtype,
                   const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                   const int32_t* cu_q, const int32_t* cu_q_host, int B, int K, int V,
                   float temperature, float top_p, int top_k, int greedy, int32_t* n_accepted,
                   int32_t* out_tokens, int32_t* status, void* workspace,
                   size_t workspace_bytes, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * spec_accept_compact -- spec_accept_ex and spec_compact_kv in one call.
 *
 * [SpS] "Modified rejection sampling" followed by [EMS]'s padding-free
 * compaction, with the compaction done by the sampler's own kernels: the
 * workgroup that makes a sequence's tokens final appends its accepted KV rows
 * and advances its kv_len, and the last sequence to finish writes cu_tokens
 * and tokens_packed.  No compaction launch, no round trip through n_accepted.
 * Every output equals that of spec_accept_ex followed by spec_compact_kv
 * (uniform: cu_q = cu_q_host = NULL) or spec_compact_kv_ragged (ragged) on the
 * same arguments; the sampler arguments and the workspace are those of
 * spec_accept_ex (its workspace size functions cover this call), the
 * compaction arguments those of spec_compact_kv with kv_dtype its dtype.  The
 * sampler's tokens are always valid counts, so status never takes
 * SV_DEV_BAD_COUNT here.  The workspace's counters are zero on entry (a
 * zero-filled workspace before the first call) and every completed call leaves
 * them at zero.
 * ------------------------------------------------------------------------ */
int spec_accept_compact(const void* target_logits, const void* draft_logits, int logits_dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        const int32_t* cu_q, const int32_t* cu_q_host, int B, int K, int V,
                        float temperature, float top_p, int top_k, int greedy,
                        int32_t* n_accepted, int32_t* out_tokens, int32_t* kv_len,
                        const int64_t* kv_start, void* k_cache, void* v_cache, const void* k_new,
                        const void* v_new, int Hkv, int D, int kv_dtype, int32_t* tokens_packed,
                        int32_t* cu_tokens, int32_t* status, void* workspace,
                        size_t workspace_bytes, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * spec_lm_head_stats -- the target's LM head with the sampler's row
 * statistics in its epilogue.
 *
 * [SpS] "Conditional scoring": one target call scores the K drafts plus one
 * position; its last linear layer turns each row's final hidden state into
 * logits, and the sampler's first need from every row ("Modified rejection
 * sampling": tempered softmax distributions) is its maximum and normaliser.
 *   logits[r][v] = sum_h hidden[r][h] * weight[v][h]   (fp32 accumulation)
 * and, per row r and part i of 64 consecutive ids [64 i, 64 i + 64) of the
 * vocabulary (the last part shorter when V % 64 != 0):
 *   part_max[r][i] = max z,  part_sum[r][i] = sum exp((z - part_max[r][i]) / T)
 * with fp64 sums, so that m_r = max_i part_max and
 * S_r = sum_i part_sum exp((part_max - m_r) / T).
 *
 * hidden   [rows, H] bf16, weight [V, H] bf16 (no bias), both 16-byte aligned
 * logits   [rows, V] fp32 out (16-byte aligned)
 * part_max [rows, parts] fp32 out, part_sum [rows, parts] fp64 out, with
 *          parts = spec_lm_head_parts(V) = ceil(V / 64)
 * H must be a multiple of 32 (SV_ERR_UNSUPPORTED otherwise).  One launch on
 * `stream`; the library allocates nothing.  Errors: negative SV_ERR_* codes
 * before any launch (bad sizes, NULL or misaligned pointers, temperature not
 * finite and > 0).
 * ------------------------------------------------------------------------ */
int spec_lm_head_parts(int V);
int spec_lm_head_stats(const void* hidden, const void* weight, int rows, int H, int V,
                       float temperature, float* logits, float* part_max, double* part_sum,
                       sv_stream_t stream);

/* ------------------------------------------------------------------------
 * spec_accept_prestats -- spec_accept_ex with the rows' statistics from
 * spec_lm_head_stats.
 *
 * For stochastic calls without a filter (top_p = 1, top_k off, not greedy)
 * the sampler takes every row's max and normaliser from the parts instead of
 * its own pass over the logits (one launch and one read of every logit row
 * fewer); with a filter, or greedy, the statistics are not needed and the
 * call is spec_accept_ex.  target_part_* are [nt, parts] for the target
 * rows, draft_part_* [nt - B, parts] for the draft rows (row order of the
 * logits; NULL allowed when there is no draft row), both made at the same
 * temperature as this call.  Every other argument and the workspace as in
 * spec_accept_ex; results agree with it on the same logits up to the fp64
 * rounding of the normalisers (the oracle's decision margins cover it).
 * ------------------------------------------------------------------------ */
int spec_accept_prestats(const void* target_logits, const void* draft_logits, int logits_dtype,
                         const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                         const int32_t* cu_q, const int32_t* cu_q_host, int B, int K, int V,
                         float temperature, float top_p, int top_k, int greedy,
                         const float* target_part_max, const double* target_part_sum,
                         const float* draft_part_max, const double* draft_part_sum, int parts,
                         int32_t* n_accepted, int32_t* out_tokens, int32_t* status,
                         void* workspace, size_t workspace_bytes, sv_stream_t stream);

int spec_compact_kv_ragged(const int32_t* n_accepted, const int32_t* out_tokens, int32_t* kv_len,
                           const int64_t* kv_start, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, int32_t* tokens_packed,
                           int32_t* cu_tokens, const int32_t* cu_q, int B, int Hkv, int D,
                           int dtype, int32_t* status, sv_stream_t stream);

/* ------------------------------------------------------------------------
 * sv_set_kernel_events -- timing instrumentation for the dominant kernel.
 *
 * When `start` and `stop` (hipEvent_t handles created by the caller, with
 * timing enabled) are both non-NULL, every later spec_verify_attn call on the
 * calling thread launches its per-sequence split-K chunk kernel (bf16 KV; the
 * fp32 path's partial kernel) so that the dispatch itself stamps `start` when
 * the kernel begins and `stop` when it ends: hipEventElapsedTime of the pair is
 * that one kernel's duration.  Meant for eager launches; do not leave it on
 * while a stream is captured into a graph.  Passing NULL for either turns it
 * off.  The events stay owned by the caller.  Returns SV_OK.
 * ------------------------------------------------------------------------ */
int sv_set_kernel_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
