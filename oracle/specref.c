/*
 * specref.c -- CPU oracle for the batched speculative-sampling verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 statement of
 * what the verify step computes.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark load it.  It shares no code, header,
 * table or helper with the GPU library, and it never calls it.
 *
 * Sources (cited by page title and section):
 *   [SpS]  "Accelerating Large Language Model Decoding with Speculative
 *          Sampling" (Chen et al.): "Conditional scoring", "Modified rejection
 *          sampling", Theorem 1 and its proof.
 *   [BIF]  The bifurcated-attention abstract (Athiwaratkun et al.): attention
 *          over a shared prefill KV plus per-sample decode KV, exact result.
 *   [EMS]  "EMS-SD: Efficient Multi-sample Speculative Decoding": accepted
 *          lengths differ per sample and are handled without padding tokens.
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes of the repository):
 *   - The K+1 verify queries of sequence b are its last emitted token followed
 *     by the K drafts.  Query j attends to: the shared prefix (if any), the
 *     L_b cached rows of b, and the new rows 0..j of b (causal among the new).
 *   - Scores carry no position term; scale defaults to 1/sqrt(D).
 *   - Grouped heads are contiguous: kv head g = h / (Hq / Hkv).
 *   - Temperature, then nucleus, are applied to both q and p before the scheme.
 *   - Nucleus keeps the smallest tie-closed top set whose mass is >= top_p.
 *   - Top-k (when asked for) comes after temperature and before nucleus and
 *     keeps the k most probable tokens and every tie of the k-th.
 *   - Accept iff u * p < q; if p == 0, accept iff q > 0.
 *   - The draw takes the smallest token id i with u * S < C_i (C = running sum
 *     of the weights in ascending token order, S = C_{V-1}).  If the residual
 *     has zero mass, the draw falls back to q.
 *   - Greedy: argmax (lowest id on ties) replaces every draw.
 *
 * Floating point: every quantity of the method is computed in double.  Inputs
 * (bf16 or f32) convert exactly to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SPECREF_F32 0
#define SPECREF_BF16 1

#define SPECREF_OK 0
#define SPECREF_EINVAL -1
#define SPECREF_ENOMEM -2

/* Ambiguity margins, computed on the oracle's own fp64 values. */
#define ACCEPT_MARGIN 1e-6   /* |u*p - q| < 1e-6 * p               */
#define DRAW_MARGIN 1e-12    /* u*S within 1e-12*S of an interval end */
#define NUCLEUS_MARGIN 1e-12 /* boundary mass within 1e-12 of top_p   */

static double elem(const void *base, int dtype, size_t i) {
    if (dtype == SPECREF_F32) return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Attention for the K+1 verify queries ([SpS] "Conditional scoring": one    */
/* target call scores all drafted positions against the KV cache; [BIF]:     */
/* prefix KV and per-sample KV together give the exact attention).           */
/* ------------------------------------------------------------------------ */

typedef struct {
    const void *q, *k_cache, *v_cache, *k_new, *v_new, *k_prefix, *v_prefix;
    const int64_t *kv_start;
    const int32_t *kv_len;
    int prefix_len, B, K, Hq, Hkv, D, dtype;
    double scale;
} attn_args;

/* Address (element offset) of key/value row t of the key list of query j of
 * sequence b, for kv head g.  The key list is: prefix rows, then the L_b
 * cached rows, then new rows 0..j.  Sets *which to 0 (prefix), 1 (cache),
 * 2 (new). */
static size_t key_offset(const attn_args *a, int b, int t, int g, int *which) {
    size_t hd = (size_t)a->Hkv * a->D;
    if (t < a->prefix_len) {
        *which = 0;
        return (size_t)t * hd + (size_t)g * a->D;
    }
    t -= a->prefix_len;
    if (t < a->kv_len[b]) {
        *which = 1;
        return (size_t)(a->kv_start[b] + t) * hd + (size_t)g * a->D;
    }
    t -= a->kv_len[b];
    *which = 2;
    return (size_t)(b * (a->K + 1) + t) * hd + (size_t)g * a->D;
}

static int attn_one(const attn_args *a, int b, int j, int h, double *o) {
    int G = a->Hq / a->Hkv;
    int g = h / G;
    int n_keys = a->prefix_len + a->kv_len[b] + j + 1;
    size_t qoff = ((size_t)(b * (a->K + 1) + j) * a->Hq + h) * a->D;
    double *s = (double *)malloc(sizeof(double) * (size_t)n_keys);
    if (!s) return SPECREF_ENOMEM;

    /* scores s_t = scale * <q, k_t> */
    double m = -INFINITY;
    for (int t = 0; t < n_keys; ++t) {
        int which;
        size_t off = key_offset(a, b, t, g, &which);
        const void *kb = which == 0 ? a->k_prefix : which == 1 ? a->k_cache : a->k_new;
        double dot = 0.0;
        for (int d = 0; d < a->D; ++d)
            dot += elem(a->q, a->dtype, qoff + d) * elem(kb, a->dtype, off + d);
        s[t] = a->scale * dot;
        if (s[t] > m) m = s[t];
    }
    /* o = sum_t softmax(s)_t v_t */
    double den = 0.0;
    for (int t = 0; t < n_keys; ++t) {
        s[t] = exp(s[t] - m);
        den += s[t];
    }
    for (int d = 0; d < a->D; ++d) o[d] = 0.0;
    for (int t = 0; t < n_keys; ++t) {
        int which;
        size_t off = key_offset(a, b, t, g, &which);
        const void *vb = which == 0 ? a->v_prefix : which == 1 ? a->v_cache : a->v_new;
        for (int d = 0; d < a->D; ++d) o[d] += s[t] * elem(vb, a->dtype, off + d);
    }
    for (int d = 0; d < a->D; ++d) o[d] /= den;
    free(s);
    return SPECREF_OK;
}

/*
 * Output rows: if n_sel < 0, all B*(K+1)*Hq rows are written to out as
 * [B*(K+1), Hq, D]; otherwise only the n_sel (row, head) pairs listed in
 * sel_row/sel_head, written to out as [n_sel, D].  row = b*(K+1) + j.
 */
int specref_verify_attn(const void *q, const void *k_cache, const void *v_cache,
                        const int64_t *kv_start, const int32_t *kv_len,
                        const void *k_new, const void *v_new,
                        const void *k_prefix, const void *v_prefix, int prefix_len,
                        int B, int K, int Hq, int Hkv, int D, int dtype, double scale,
                        const int32_t *sel_row, const int32_t *sel_head, int n_sel,
                        double *out) {
    if (B < 1 || K < 0 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return SPECREF_EINVAL;
    if (dtype != SPECREF_F32 && dtype != SPECREF_BF16) return SPECREF_EINVAL;
    if (prefix_len < 0 || (prefix_len > 0 && (!k_prefix || !v_prefix))) return SPECREF_EINVAL;
    for (int b = 0; b < B; ++b)
        if (kv_len[b] < 0) return SPECREF_EINVAL;
    attn_args a = {q, k_cache, v_cache, k_new, v_new, k_prefix, v_prefix,
                   kv_start, kv_len, prefix_len, B, K, Hq, Hkv, D, dtype,
                   scale > 0.0 ? scale : 1.0 / sqrt((double)D)};
    if (n_sel < 0) {
        for (int r = 0; r < B * (K + 1); ++r)
            for (int h = 0; h < Hq; ++h) {
                int rc = attn_one(&a, r / (K + 1), r % (K + 1), h,
                                  out + ((size_t)r * Hq + h) * D);
                if (rc) return rc;
            }
        return SPECREF_OK;
    }
    for (int i = 0; i < n_sel; ++i) {
        int r = sel_row[i], h = sel_head[i];
        if (r < 0 || r >= B * (K + 1) || h < 0 || h >= Hq) return SPECREF_EINVAL;
        int rc = attn_one(&a, r / (K + 1), r % (K + 1), h, out + (size_t)i * D);
        if (rc) return rc;
    }
    return SPECREF_OK;
}

/* ------------------------------------------------------------------------ */
/* Modified rejection sampling ([SpS] "Modified rejection sampling").        */
/* ------------------------------------------------------------------------ */

/* For qsort: (probability, id) pairs, largest probability first, ties by id. */
typedef struct {
    double pi;
    int id;
} prob_id;

static int by_prob_desc(const void *x, const void *y) {
    const prob_id *a = (const prob_id *)x, *b = (const prob_id *)y;
    if (a->pi > b->pi) return -1;
    if (a->pi < b->pi) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

/*
 * The distribution the scheme uses for one row of logits z[0..V):
 * temperature first, then top-k, then nucleus ([SpS]: standard sampling
 * methods -- it names top-k and nucleus -- modify the probabilities before the
 * rejection scheme is applied).
 *   d_t = z_t - max z ; x_t = d_t / T ; pi_t = exp(x_t) / sum_s exp(x_s)
 *   top-k (0 < top_k < V): keep {t : pi_t >= the top_k-th largest pi} (ties
 *            at the boundary kept), renormalised.
 *   nucleus: tau = the largest value among {pi_t} with sum_{pi_s >= tau} pi_s
 *            >= top_p; keep {t : pi_t >= tau}; pi'_t = pi_t / kept mass.
 * *ambiguous is set when the mass of the kept set, or of the set just above
 * its boundary tie group, is within NUCLEUS_MARGIN of top_p.  (The top-k set
 * is decided by exact comparisons of the logits: never ambiguous.)
 */
static int row_dist(const float *z, int V, double T, int top_k, double top_p, double *pi,
                    int *ambiguous) {
    double m = -INFINITY;
    for (int t = 0; t < V; ++t)
        if ((double)z[t] > m) m = (double)z[t];
    double S = 0.0;
    for (int t = 0; t < V; ++t) {
        pi[t] = exp(((double)z[t] - m) / T);
        S += pi[t];
    }
    for (int t = 0; t < V; ++t) pi[t] /= S;
    *ambiguous = 0;
    const int use_k = top_k > 0 && top_k < V;
    if (!(top_p < 1.0) && !use_k) return SPECREF_OK;

    prob_id *srt = (prob_id *)malloc(sizeof(prob_id) * (size_t)V);
    if (!srt) return SPECREF_ENOMEM;
    for (int t = 0; t < V; ++t) {
        srt[t].pi = pi[t];
        srt[t].id = t;
    }
    qsort(srt, (size_t)V, sizeof(prob_id), by_prob_desc);

    if (use_k) {
        /* keep the top_k largest probabilities and every tie of the last one */
        const double tk = srt[top_k - 1].pi;
        double mass = 0.0;
        for (int t = 0; t < V; ++t)
            if (pi[t] >= tk) mass += pi[t];
        for (int t = 0; t < V; ++t) pi[t] = pi[t] >= tk ? pi[t] / mass : 0.0;
        for (int i = 0; i < V; ++i) srt[i].pi = pi[srt[i].id];
        if (!(top_p < 1.0)) {
            free(srt);
            return SPECREF_OK;
        }
    }

    /* walk tie groups from the top; stop at the first group whose inclusion
     * brings the mass to >= top_p */
    double above = 0.0, tau = srt[V - 1].pi;
    int k = 0;
    while (k < V) {
        int e = k;
        double group = 0.0;
        while (e < V && srt[e].pi == srt[k].pi) group += srt[e++].pi;
        if (above + group >= top_p || e == V) {
            tau = srt[k].pi;
            if (fabs(above + group - top_p) < NUCLEUS_MARGIN ||
                fabs(above - top_p) < NUCLEUS_MARGIN)
                *ambiguous = 1;
            break;
        }
        above += group;
        k = e;
    }
    free(srt);
    double kept = 0.0;
    for (int t = 0; t < V; ++t)
        if (pi[t] >= tau) kept += pi[t];
    for (int t = 0; t < V; ++t) pi[t] = pi[t] >= tau ? pi[t] / kept : 0.0;
    return SPECREF_OK;
}

/*
 * The modified distribution of one row of logits (temperature, then top-k,
 * then nucleus, as row_dist states), exported so that a check can test
 * whether a token has positive probability under q' or (q' - p')_+.
 * pi [V] out; *ambiguous as in row_dist.
 */
int specref_row_dist(const float *z, int V, double temperature, int top_k, double top_p,
                     double *pi, int32_t *ambiguous) {
    if (V < 1 || !(temperature > 0.0) || !(top_p > 0.0) || top_p > 1.0 || top_k < 0)
        return SPECREF_EINVAL;
    int amb = 0;
    int rc = row_dist(z, V, temperature, top_k, top_p, pi, &amb);
    if (ambiguous) *ambiguous = amb;
    return rc;
}

static int argmax_row(const float *z, int V) {
    int best = 0;
    for (int t = 1; t < V; ++t)
        if (z[t] > z[best]) best = t;
    return best;
}

/*
 * Inverse-CDF draw from unnormalised weights w[0..V): the smallest i with
 * u * S < C_i.  *ambiguous when u*S is within DRAW_MARGIN*S of either end of
 * the chosen token's interval [C_{i-1}, C_i).
 */
static int draw(const double *w, int V, double u, int *ambiguous) {
    double S = 0.0;
    for (int t = 0; t < V; ++t) S += w[t];
    double target = u * S, C = 0.0, prev = 0.0;
    int tok = V - 1;
    for (int t = 0; t < V; ++t) {
        prev = C;
        C += w[t];
        if (target < C) {
            tok = t;
            break;
        }
    }
    *ambiguous = (target - prev < DRAW_MARGIN * S) || (C - target < DRAW_MARGIN * S);
    return tok;
}

/*
 * One verify round per sequence b:
 *   for j = 0..K-1 with x = draft_tokens[b, j]:
 *       accept iff u_accept[b, j] * p'_j(x) < q'_j(x)   (p' == 0: iff q' > 0)
 *     stop at the first rejection, n_b = j, and draw from (q'_j - p'_j)_+;
 *   if all K are accepted, n_b = K and draw the bonus token from q'_K.
 *   out_tokens[b] = [x_0 .. x_{n_b - 1}, drawn token, -1 ...]
 *
 * target_logits [B, K+1, V], draft_logits [B, K, V] (unused if greedy).
 * Optional outputs (may be NULL):
 *   q_tok, p_tok [B, K]: q'_j(x_j), p'_j(x_j) for the positions tested (else NaN)
 *   flag_pos [B]: first position whose decision is ambiguous, -1 if none
 *   n_decisions, n_flagged: totals for the ambiguity budget.
 */
int specref_accept(const float *target_logits, const float *draft_logits,
                   const int32_t *draft_tokens, const float *u_accept,
                   const float *u_sample, int B, int K, int V, double temperature,
                   double top_p, int top_k, int greedy, int32_t *n_accepted, int32_t *out_tokens,
                   double *q_tok, double *p_tok, int32_t *flag_pos,
                   int64_t *n_decisions, int64_t *n_flagged) {
    if (B < 0 || K < 0 || V < 1 || !(temperature > 0.0) || !(top_p > 0.0) || top_p > 1.0 ||
        top_k < 0)
        return SPECREF_EINVAL;
    for (int i = 0; i < B * K; ++i)
        if (draft_tokens[i] < 0 || draft_tokens[i] >= V) return SPECREF_EINVAL;
    int64_t decisions = 0, flagged = 0;
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    if (!q || !p || !w) {
        free(q); free(p); free(w);
        return SPECREF_ENOMEM;
    }
    for (int b = 0; b < B; ++b) {
        const float *zt = target_logits + (size_t)b * (K + 1) * V;
        const float *zd = draft_logits ? draft_logits + (size_t)b * K * V : NULL;
        const int32_t *x = draft_tokens + (size_t)b * K;
        int32_t *out = out_tokens + (size_t)b * (K + 1);
        int first_flag = -1, n = K, tok = -1;
        for (int j = 0; j < K; ++j) {
            if (q_tok) q_tok[b * K + j] = NAN;
            if (p_tok) p_tok[b * K + j] = NAN;
        }

        if (greedy) {
            /* Greedy decoding: accept while the draft equals the target argmax. */
            for (int j = 0; j < K; ++j) {
                decisions++;
                int a = argmax_row(zt + (size_t)j * V, V);
                if (x[j] != a) {
                    n = j;
                    tok = a;
                    break;
                }
            }
            if (n == K) tok = argmax_row(zt + (size_t)K * V, V);
            decisions++;
        } else {
            int amb, rc;
            for (int j = 0; j <= K; ++j) {
                rc = row_dist(zt + (size_t)j * V, V, temperature, top_k, top_p, q, &amb);
                if (rc) goto fail;
                if (top_p < 1.0) {
                    decisions++;
                    if (amb) { flagged++; if (first_flag < 0) first_flag = j; }
                }
                if (j == K) {
                    /* all K accepted: bonus token from q'_K */
                    decisions++;
                    tok = draw(q, V, (double)u_sample[b], &amb);
                    if (amb) { flagged++; if (first_flag < 0) first_flag = K; }
                    break;
                }
                rc = row_dist(zd + (size_t)j * V, V, temperature, top_k, top_p, p, &amb);
                if (rc) goto fail;
                if (top_p < 1.0) {
                    decisions++;
                    if (amb) { flagged++; if (first_flag < 0) first_flag = j; }
                }
                double qx = q[x[j]], px = p[x[j]], u = (double)u_accept[b * K + j];
                if (q_tok) q_tok[b * K + j] = qx;
                if (p_tok) p_tok[b * K + j] = px;
                int accept = px > 0.0 ? (u * px < qx) : (qx > 0.0);
                decisions++;
                if (px > 0.0 && fabs(u * px - qx) < ACCEPT_MARGIN * px) {
                    flagged++;
                    if (first_flag < 0) first_flag = j;
                }
                if (accept) continue;
                /* rejected: resample from (q' - p')_+, or from q' if it has no mass */
                n = j;
                double mass = 0.0;
                for (int t = 0; t < V; ++t) {
                    w[t] = q[t] - p[t] > 0.0 ? q[t] - p[t] : 0.0;
                    mass += w[t];
                }
                decisions++;
                tok = draw(mass > 0.0 ? w : q, V, (double)u_sample[b], &amb);
                if (amb) { flagged++; if (first_flag < 0) first_flag = j; }
                break;
            }
        }
        n_accepted[b] = n;
        for (int i = 0; i < n; ++i) out[i] = x[i];
        out[n] = tok;
        for (int i = n + 1; i <= K; ++i) out[i] = -1;
        if (flag_pos) flag_pos[b] = first_flag;
    }
    free(q); free(p); free(w);
    if (n_decisions) *n_decisions = decisions;
    if (n_flagged) *n_flagged = flagged;
    return SPECREF_OK;
fail:
    free(q); free(p); free(w);
    return SPECREF_ENOMEM;
}

/* ------------------------------------------------------------------------ */
/* Padding-free compaction ([EMS]: each sample keeps its own accepted count;  */
/* no padding tokens are inserted).                                           */
/* ------------------------------------------------------------------------ */

/*
 * e_b = n_b + 1 tokens per sequence.  cu = exclusive scan of e (cu[B] = total).
 * packed[cu[b] + i] = out_tokens[b, i] for i < e_b.
 * Cache rows kv_start[b] + kv_len[b] + i  <-  new rows b*(K+1) + i, i < e_b,
 * for K and V; then kv_len[b] += e_b.  elem_bytes is 2 (bf16) or 4 (f32).
 */
int specref_compact_kv(const int32_t *n_accepted, const int32_t *out_tokens,
                       int32_t *kv_len, const int64_t *kv_start, void *k_cache,
                       void *v_cache, const void *k_new, const void *v_new,
                       int32_t *tokens_packed, int32_t *cu_tokens, int B, int K,
                       int Hkv, int D, int elem_bytes) {
    if (B < 0 || K < 0 || Hkv < 1 || D < 1 || (elem_bytes != 2 && elem_bytes != 4))
        return SPECREF_EINVAL;
    size_t row_bytes = (size_t)Hkv * D * elem_bytes;
    cu_tokens[0] = 0;
    for (int b = 0; b < B; ++b) {
        if (n_accepted[b] < 0 || n_accepted[b] > K) return SPECREF_EINVAL;
        cu_tokens[b + 1] = cu_tokens[b] + n_accepted[b] + 1;
    }
    for (int b = 0; b < B; ++b) {
        int e = n_accepted[b] + 1;
        for (int i = 0; i < e; ++i) {
            tokens_packed[cu_tokens[b] + i] = out_tokens[b * (K + 1) + i];
            size_t dst = (size_t)(kv_start[b] + kv_len[b] + i) * row_bytes;
            size_t src = (size_t)(b * (K + 1) + i) * row_bytes;
            memcpy((char *)k_cache + dst, (const char *)k_new + src, row_bytes);
            memcpy((char *)v_cache + dst, (const char *)v_new + src, row_bytes);
        }
        kv_len[b] += e;
    }
    return SPECREF_OK;
}

/* ------------------------------------------------------------------------ */
/* LM head and the softmax statistics of its rows ([SpS] "Conditional       */
/* scoring": the target model scores the K drafts and one more position in   */
/* one call; its last linear layer turns each row's final hidden state into  */
/* logits over the vocabulary, and the sampler's first need from every row   */
/* is its maximum and its normaliser).                                       */
/*   z[r][v] = sum_h hidden[r][h] * W[v][h]   (W stored [V][H], no bias)     */
/*   m = max_v z[v],   S = sum_v exp((z[v] - m) / T)                         */
/* ------------------------------------------------------------------------ */

int specref_lm_head(const void *hidden, const void *weight, int dtype, int rows, int H, int V,
                    double *logits) {
    if (rows < 0 || H < 1 || V < 1 || !hidden || !weight || !logits) return 1;
    for (int r = 0; r < rows; ++r)
        for (int v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += elem(hidden, dtype, (size_t)r * H + h) * elem(weight, dtype, (size_t)v * H + h);
            logits[(size_t)r * V + v] = acc;
        }
    return 0;
}

/* Statistics of one row of (fp32) logits: m = max z, S = sum exp((z - m)/T). */
int specref_row_stats(const float *z, int V, double temperature, double *m, double *S) {
    if (V < 1 || !z || !m || !S || !(temperature > 0.0)) return 1;
    double mx = -INFINITY;
    for (int v = 0; v < V; ++v)
        if ((double)z[v] > mx) mx = (double)z[v];
    double sum = 0.0;
    for (int v = 0; v < V; ++v) sum += exp(((double)z[v] - mx) / temperature);
    *m = mx;
    *S = sum;
    return 0;
}
