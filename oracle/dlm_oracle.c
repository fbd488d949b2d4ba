/*
 * dlm_oracle.c -- plain, slow fp64 CPU oracle of one masked-diffusion
 * denoising step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Every function follows a definition of the pages directly: no blocking,
 * no fusion, no reordering beyond the definition.  Floating point is fp64;
 * bf16 and fp32 inputs are widened exactly.  OpenMP runs independent rows
 * (or columns) in parallel; each output is computed by one thread in a
 * fixed order, so results do not depend on the thread count.
 *
 * Sources (the pages are the gist.science summaries named below):
 *  - "Stopping Computation for Converged Tokens in Masked Diffusion-LM
 *    Decoding" (SureLock), section 2 "core mechanism": active (unlocked)
 *    rows attend to the cached K/V of locked rows; a row locks when the
 *    step-wise KL(p_t || p_{t-1}) falls to eps or below.
 *  - "Multi-Block Diffusion LMs", sections 1, 2.2 and 2.3: block-causal
 *    visibility to a clean prefix, group-aware mask (blocks of one noise
 *    group see each other), block-buffer slot states.
 *  - "Bifocal Diffusion Language Models", section 1: bidirectional versus
 *    causal attention; section 2: prefill once, later steps touch only the
 *    generation block and read the K/V cache.
 *  - "Attention-Based Sampler for Diffusion Language Models", section 2A/2B:
 *    attention-matrix column sums as the decode order; the dynamic attention
 *    threshold for parallel decoding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORA_FULL = 0, ORA_BLOCK_CAUSAL = 1, ORA_GROUP = 2 };
enum { ORA_DUMMY = 0 };
enum { ORA_ROW_SELECT = 1, ORA_ROW_LOCK = 2 };
enum { ORA_SEL_NONE = 0, ORA_SEL_TOPK_CONF = 1, ORA_SEL_THRESH_CONF = 2,
       ORA_SEL_ATTN_DYNAMIC = 3, ORA_SEL_TOPK_SCORE = 4, ORA_SEL_TOPK_MARGIN = 5,
       ORA_SEL_TOPK_LOW_ENTROPY = 6 };

/* Exact bf16 -> fp64 widening: a bf16 value is the top half of an fp32. */
static double wide(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------
 * Effective K/V: the cache with the fresh K/V of the active rows written at
 * their positions (SureLock section 2: locked rows keep their cached K/V,
 * active rows are recomputed).  In place on the caller's copy.
 * ---------------------------------------------------------------------- */
void ora_scatter(uint16_t *cache_k, uint16_t *cache_v, const uint16_t *k,
                 const uint16_t *v, const int32_t *active_idx, int B, int Hkv,
                 int n_cap, int D, int M)
{
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g)
            for (int j = 0; j < M; ++j) {
                int64_t pos = active_idx[(int64_t)b * M + j];
                int64_t dst = (((int64_t)b * Hkv + g) * n_cap + pos) * D;
                int64_t src = (((int64_t)b * Hkv + g) * M + j) * D;
                for (int d = 0; d < D; ++d) {
                    cache_k[dst + d] = k[src + d];
                    cache_v[dst + d] = v[src + d];
                }
            }
}

/* ------------------------------------------------------------------------
 * Visibility of key position n to the query at position i.
 *  FULL:          every key below kv_len (bidirectional attention).
 *  BLOCK_CAUSAL:  the clean prefix, plus generation blocks up to and
 *                 including the query's own block.
 *  GROUP:         the clean prefix, plus every non-dummy slot whose noise
 *                 group is the query's group or an earlier one.
 * Blocks are bs positions wide and start at the prefix length P.
 * ---------------------------------------------------------------------- */
int ora_visible(int kind, int kv_len, int P, int bs, int n_slots,
                const uint8_t *state, const int32_t *group, int i, int n)
{
    if (n < 0 || n >= kv_len)
        return 0;
    if (kind == ORA_FULL)
        return 1;
    if (n < P)
        return 1;
    int slot_n = (n - P) / bs;
    int slot_i = (i - P) / bs;
    if (kind == ORA_BLOCK_CAUSAL)
        return slot_n <= slot_i;
    /* GROUP */
    if (slot_n >= n_slots || slot_i < 0 || slot_i >= n_slots)
        return 0;
    if (state[slot_n] == ORA_DUMMY)
        return 0;
    return group[slot_n] <= group[slot_i];
}

/* ------------------------------------------------------------------------
 * Attention of one active row: scaled dot products with every visible key,
 * log-sum-exp, softmax weights, weighted sum of values.
 * rows: flat indices ((b*Hq + h)*M + j), or NULL for all B*Hq*M rows.
 * out: [n_rows, D] (may be NULL), lse: [n_rows].
 * The query of q-head h reads kv-head h / (Hq/Hkv).
 * A row that sees no key gets out = 0 and lse = -inf.
 * ---------------------------------------------------------------------- */
void ora_attn(const uint16_t *q, const uint16_t *Kc, const uint16_t *Vc,
              const int32_t *active_idx, int B, int Hq, int Hkv, int n_cap,
              int D, int M, int kind, int kv_len, int P, int bs, int n_slots,
              const uint8_t *slot_state, const int32_t *slot_group,
              double scale, int64_t n_rows, const int64_t *rows, double *out,
              double *lse)
{
    const int G = Hq / Hkv;
    if (rows == NULL)
        n_rows = (int64_t)B * Hq * M;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
        char *vis = (char *)malloc((size_t)(kv_len > 0 ? kv_len : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t flat = rows ? rows[r] : r;
            int j = (int)(flat % M);
            int h = (int)((flat / M) % Hq);
            int b = (int)(flat / ((int64_t)M * Hq));
            int g = h / G;
            int i = active_idx[(int64_t)b * M + j];
            const uint8_t *st = slot_state ? slot_state + (int64_t)b * n_slots : NULL;
            const int32_t *gr = slot_group ? slot_group + (int64_t)b * n_slots : NULL;
            const uint16_t *qr = q + flat * D;
            const uint16_t *kb = Kc + ((int64_t)b * Hkv + g) * n_cap * D;
            const uint16_t *vb = Vc + ((int64_t)b * Hkv + g) * n_cap * D;

            double mx = -INFINITY;
            int any = 0;
            for (int n = 0; n < kv_len; ++n) {
                vis[n] = (char)ora_visible(kind, kv_len, P, bs, n_slots, st, gr, i, n);
                if (!vis[n])
                    continue;
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += wide(qr[d]) * wide(kb[(int64_t)n * D + d]);
                s[n] = scale * dot;
                if (s[n] > mx)
                    mx = s[n];
                any = 1;
            }
            if (!any) {
                lse[r] = -INFINITY;
                if (out)
                    for (int d = 0; d < D; ++d)
                        out[r * D + d] = 0.0;
                continue;
            }
            double sum = 0.0;
            for (int n = 0; n < kv_len; ++n)
                if (vis[n])
                    sum += exp(s[n] - mx);
            double L = mx + log(sum);
            lse[r] = L;
            if (out) {
                double *o = out + r * D;
                for (int d = 0; d < D; ++d)
                    o[d] = 0.0;
                for (int n = 0; n < kv_len; ++n) {
                    if (!vis[n])
                        continue;
                    double p = exp(s[n] - L);
                    for (int d = 0; d < D; ++d)
                        o[d] += p * wide(vb[(int64_t)n * D + d]);
                }
            }
        }
        free(s);
        free(vis);
    }
}

/* ------------------------------------------------------------------------
 * Column sums of the attention matrix (Attn-Sampler section 2B: the total
 * attention a key position receives).  For key position n of batch b:
 *     colsum[b, n] = sum over q-heads h, and over active rows j whose
 *                    position lies in [cs_lo, cs_hi), of p_{b,h,j}(n),
 * where p_{b,h,j}(n) = exp(s - lse_{b,h,j}) if n is visible to row j and 0
 * otherwise.  lse_all is [B, Hq, M] from ora_attn over all rows.
 * cols: flat indices (b*kv_len + n), or NULL for all B*kv_len columns.
 * colsum: [n_cols] if per_head == 0, else [n_cols, Hq].
 * Rows whose lse is -inf (no visible key) contribute nothing.
 * ---------------------------------------------------------------------- */
void ora_colsum(const uint16_t *q, const uint16_t *Kc, const int32_t *active_idx,
                int B, int Hq, int Hkv, int n_cap, int D, int M, int kind,
                int kv_len, int P, int bs, int n_slots, const uint8_t *slot_state,
                const int32_t *slot_group, double scale, int cs_lo, int cs_hi,
                int per_head, const double *lse_all, int64_t n_cols,
                const int64_t *cols, double *colsum)
{
    const int G = Hq / Hkv;
    if (cols == NULL)
        n_cols = (int64_t)B * kv_len;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < n_cols; ++c) {
        int64_t flat = cols ? cols[c] : c;
        int n = (int)(flat % kv_len);
        int b = (int)(flat / kv_len);
        const uint8_t *st = slot_state ? slot_state + (int64_t)b * n_slots : NULL;
        const int32_t *gr = slot_group ? slot_group + (int64_t)b * n_slots : NULL;
        double total = 0.0;
        for (int h = 0; h < Hq; ++h) {
            int g = h / G;
            const uint16_t *kr = Kc + (((int64_t)b * Hkv + g) * n_cap + n) * D;
            double head_sum = 0.0;
            for (int j = 0; j < M; ++j) {
                int i = active_idx[(int64_t)b * M + j];
                if (i < cs_lo || i >= cs_hi)
                    continue;
                if (!ora_visible(kind, kv_len, P, bs, n_slots, st, gr, i, n))
                    continue;
                double L = lse_all[((int64_t)b * Hq + h) * M + j];
                if (isinf(L))
                    continue;
                const uint16_t *qr = q + (((int64_t)b * Hq + h) * M + j) * D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += wide(qr[d]) * wide(kr[d]);
                head_sum += exp(scale * dot - L);
            }
            if (per_head)
                colsum[c * Hq + h] = head_sum;
            total += head_sum;
        }
        if (!per_head)
            colsum[c] = total;
    }
}

/* ------------------------------------------------------------------------
 * Posterior of one row (SureLock section 2): p_t = softmax(logits),
 * p_{t-1} = softmax(previous-step logits),
 *     KL = sum_v p_t(v) * (log p_t(v) - log p_{t-1}(v))     (textbook form)
 *     conf = max_v p_t(v),  tok = lowest v attaining the max logit,
 *     lock when KL <= eps.
 * A row that arrives locked is not read: kl = conf = 0, tok = -1, stays
 * locked.
 * rows: row indices or NULL for all R rows; outputs are [n_rows].
 * ---------------------------------------------------------------------- */
void ora_posterior(const float *logits, const float *prev, const uint8_t *locked_in,
                   int64_t R, int64_t V, double eps, int64_t n_rows,
                   const int64_t *rows, double *kl, double *conf, int32_t *tok,
                   uint8_t *locked_out, double *margin, double *entropy,
                   const uint8_t *flags, double conf_gate)
{
    if (rows == NULL)
        n_rows = R;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_rows; ++t) {
        int64_t r = rows ? rows[t] : t;
        if (locked_in[r]) {
            kl[t] = 0.0;
            conf[t] = 0.0;
            tok[t] = -1;
            locked_out[t] = 1;
            margin[t] = 0.0;
            entropy[t] = 0.0;
            continue;
        }
        const float *x = logits + r * V;
        const float *y = prev + r * V;
        /* log-sum-exp of each row, max first for range safety */
        double mx = -INFINITY, my = -INFINITY;
        int64_t arg = 0;
        for (int64_t v = 0; v < V; ++v) {
            if ((double)x[v] > mx) {
                mx = (double)x[v];
                arg = v;
            }
            if ((double)y[v] > my)
                my = (double)y[v];
        }
        double sx = 0.0, sy = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            sx += exp((double)x[v] - mx);
            sy += exp((double)y[v] - my);
        }
        double Lx = mx + log(sx), Ly = my + log(sy);
        double d = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double logp = (double)x[v] - Lx;
            double logq = (double)y[v] - Ly;
            d += exp(logp) * (logp - logq);
        }
        kl[t] = d;
        conf[t] = exp(mx - Lx);
        tok[t] = (int32_t)arg;
        /* The lock test (KL <= eps) applies to rows the caller marks
         * lockable (flags bit 1; every row when flags is NULL).  SureLock
         * section 2: converged, already unmasked tokens are the ones whose
         * computation stops.  The optional confidence gate of that section
         * (a peaked posterior) adds conf >= conf_gate; 0 leaves it off. */
        locked_out[t] = (uint8_t)(d <= eps && (flags == NULL || (flags[r] & ORA_ROW_LOCK)) &&
                                  exp(mx - Lx) >= conf_gate);
        /* Token-level scores of the confidence family (Attn-Sampler page,
         * section 1: confidence, margin, entropy).  margin = p(top-1) -
         * p(top-2), the runner-up being the largest logit at any other
         * index (equal to the top one on a tie; no runner-up when V = 1);
         * entropy = -sum_v p_v ln p_v of p_t. */
        double x2 = -INFINITY;
        for (int64_t v = 0; v < V; ++v)
            if (v != arg && (double)x[v] > x2)
                x2 = (double)x[v];
        margin[t] = exp(mx - Lx) - (x2 == -INFINITY ? 0.0 : exp(x2 - Lx));
        double h = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double logp = (double)x[v] - Lx;
            h -= exp(logp) * logp;
        }
        entropy[t] = h;
    }
}

/* ------------------------------------------------------------------------
 * Unmask selection over consecutive groups of group_rows rows.  Only rows
 * that arrived unlocked, and that the caller marks selectable (flags bit 0;
 * every row when flags is NULL: a still-masked token), are eligible.
 * Order: higher key first, then lower row index.
 *  TOPK_CONF:    the k most confident eligible rows (all if fewer).
 *  THRESH_CONF:  eligible rows with conf > tau; if none, the most
 *                confident eligible row.
 *  ATTN_DYNAMIC: candidates = eligible rows with conf > tau; threshold =
 *                largest score among eligible non-candidates (-inf if
 *                none); select candidates whose score exceeds it; if none,
 *                the eligible row of highest score (Attn-Sampler section 2B).
 *  TOPK_SCORE:   the k eligible rows of highest score.
 *  TOPK_MARGIN:  the k eligible rows of largest margin (margin sampler).
 *  TOPK_LOW_ENTROPY: the k eligible rows of lowest entropy (entropy sampler).
 * sel[r] = tok[r] if selected, else -1.
 * ---------------------------------------------------------------------- */
static const double *g_key;
static int cmp_desc(const void *a, const void *b)
{
    int32_t ra = *(const int32_t *)a, rb = *(const int32_t *)b;
    if (g_key[ra] > g_key[rb])
        return -1;
    if (g_key[ra] < g_key[rb])
        return 1;
    return (ra > rb) - (ra < rb);
}

void ora_select(int mode, int k, int group_rows, double tau, const double *score,
                const double *conf, const int32_t *tok, const uint8_t *locked_in,
                int R, int32_t *sel, const double *margin, const double *entropy,
                const uint8_t *flags)
{
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)(group_rows > 0 ? group_rows : 1));
    /* lowest entropy first: rank by the negated entropy */
    double *neg_entropy = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    for (int r = 0; r < R; ++r)
        neg_entropy[r] = mode == ORA_SEL_TOPK_LOW_ENTROPY ? -entropy[r] : 0.0;
    for (int r = 0; r < R; ++r)
        sel[r] = -1;
    if (mode == ORA_SEL_NONE) {
        free(order);
        free(neg_entropy);
        return;
    }
    for (int g0 = 0; g0 < R; g0 += group_rows) {
        int g1 = g0 + group_rows < R ? g0 + group_rows : R;
        int n = 0;
        for (int r = g0; r < g1; ++r)
            if (!locked_in[r] && (flags == NULL || (flags[r] & ORA_ROW_SELECT)))
                order[n++] = r;
        if (n == 0)
            continue;
        const double *key = (mode == ORA_SEL_TOPK_SCORE || mode == ORA_SEL_ATTN_DYNAMIC) ? score
                            : mode == ORA_SEL_TOPK_MARGIN                         ? margin
                            : mode == ORA_SEL_TOPK_LOW_ENTROPY                    ? neg_entropy
                                                                                  : conf;
        g_key = key;
        qsort(order, (size_t)n, sizeof(int32_t), cmp_desc);
        if (mode == ORA_SEL_TOPK_CONF || mode == ORA_SEL_TOPK_SCORE || mode == ORA_SEL_TOPK_MARGIN ||
            mode == ORA_SEL_TOPK_LOW_ENTROPY) {
            for (int t = 0; t < n && t < k; ++t)
                sel[order[t]] = tok[order[t]];
        } else if (mode == ORA_SEL_THRESH_CONF) {
            int any = 0;
            for (int t = 0; t < n; ++t)
                if (conf[order[t]] > tau) {
                    sel[order[t]] = tok[order[t]];
                    any = 1;
                }
            if (!any)
                sel[order[0]] = tok[order[0]];
        } else if (mode == ORA_SEL_ATTN_DYNAMIC) {
            double thr = -INFINITY;
            for (int t = 0; t < n; ++t)
                if (!(conf[order[t]] > tau) && score[order[t]] > thr)
                    thr = score[order[t]];
            int any = 0;
            for (int t = 0; t < n; ++t)
                if (conf[order[t]] > tau && score[order[t]] > thr) {
                    sel[order[t]] = tok[order[t]];
                    any = 1;
                }
            if (!any)
                sel[order[0]] = tok[order[0]];
        }
    }
    free(order);
    free(neg_entropy);
}

int ora_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
