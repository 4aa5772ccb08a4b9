/*
 * pic_oracle.c -- plain, slow, double-precision CPU oracle for
 * position-independent attention over reused KV spans and query-centric
 * selection + cache fusion.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no source with the HIP path.
 *
 * What it computes, and where the pages define it:
 *
 *  - Keys are kept unrotated in the cache and rotated at the logical position
 *    pi(j) that the key has in the current request, queries at their own
 *    position t; the score is (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d).
 *    [MiniPIC: "Resumen Tecnico: MiniPIC ...", section 2.1, the score equation.]
 *  - The rotation matrix R is RoPE.  Pairing (i, i+d/2), frequencies
 *    theta^(-2i/d), counter-clockwise rotation (y_a = a c - b s,
 *    y_b = a s + b c).  The page only names "the rotation matrix"; this is
 *    the reading used for the Llama family, declared in the design notes.
 *  - Causality is positional: key j is visible to a query at position t iff
 *    0 <= pi(j) <= t; pi(j) = -1 marks an empty or masked slot.  [QCFuse
 *    (de), key contributions: the sparse kernel respects causal constraints;
 *    the positional reading is declared in the design notes.]
 *  - Grouped-query attention: q head h reads kv head floor(h / (Hq/Hkv)).
 *  - Selection mass: the attention of the query over one layer's K decides
 *    which context tokens are recomputed.  [QCFuse (es), methodology B;
 *    QCFuse (de), methodik phase 3.]  Reading: mass_r[j] is the sum over all
 *    of request r's query tokens and all q heads of the softmax probability
 *    that key j receives.
 *  - Selection: per span, the k = min(#candidates, floor(ratio*L + 0.5))
 *    tokens of largest mass, ties to the lower sequence index, listed in
 *    ascending index order.
 *  - Anchors: per span, the tokens with the largest squared key norm (all kv
 *    heads), selected like the mass (see oracle_key_norm).
 *  - Fusion: recomputed rows are mixed back into the cache [QCFuse (es),
 *    "Lo esencial" step 4; QCFuse (de), methodik phase 4] without ever
 *    writing a shared block [MiniPIC section 2.1, benefit paragraph]: fresh
 *    rows go to request-private blocks appended after the sequence, the stale
 *    slot is masked (pi = -1) and the fresh slot takes the stale slot's pi.
 *
 * Storage layouts it reads (documented by the product's public header and by
 * the workload generator):
 *   pool K [num_blocks][Hkv][16][d], pool V [num_blocks][Hkv][d][16] (bf16 bits)
 *   block_table [B][max_blocks], kv_pos [B][max_blocks*16], kv_len [B]
 *   q [total_q][Hq][d] (bf16 bits), q_start [B+1], q_pos [total_q]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 16

typedef struct {
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t batch;
    int32_t num_blocks;
    int32_t max_blocks;
    double rope_theta;
    const uint16_t *pool_k;
    const uint16_t *pool_v;
    const int32_t *block_table;
    const int32_t *kv_len;
    const int32_t *kv_pos;
    const uint16_t *q;
    const int32_t *q_start;
    const int32_t *q_pos;
} oracle_problem;

/* bf16 bit pattern -> exact double. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Rotate x (length d) to logical position pos: for each frequency i < d/2,
 * the pair (x[i], x[i+d/2]) turns by the angle pos * theta^(-2i/d). */
void oracle_rope(int32_t d, double theta, int32_t pos, const double *x, double *y)
{
    int32_t half = d / 2;
    for (int32_t i = 0; i < half; ++i) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)d);
        double ang = (double)pos * inv_freq;
        double c = cos(ang), s = sin(ang);
        double a = x[i], b = x[i + half];
        y[i] = a * c - b * s;
        y[i + half] = a * s + b * c;
    }
}

static int request_of(const oracle_problem *p, int32_t t)
{
    for (int32_t r = 0; r < p->batch; ++r)
        if (t >= p->q_start[r] && t < p->q_start[r + 1])
            return r;
    return -1;
}

static int32_t kv_stride(const oracle_problem *p) { return p->max_blocks * ORACLE_BLOCK; }

/* Physical block of request-sequence slot j of request r, or -1 if unusable. */
static int32_t slot_block(const oracle_problem *p, int32_t r, int32_t j)
{
    int32_t b = p->block_table[(int64_t)r * p->max_blocks + j / ORACLE_BLOCK];
    if (b < 0 || b >= p->num_blocks)
        return -1;
    return b;
}

static void load_key(const oracle_problem *p, int32_t blk, int32_t g, int32_t off, double *out)
{
    int32_t d = p->head_dim;
    const uint16_t *src = p->pool_k + (((int64_t)blk * p->num_kv_heads + g) * ORACLE_BLOCK + off) * d;
    for (int32_t i = 0; i < d; ++i)
        out[i] = bf16_value(src[i]);
}

static double value_elem(const oracle_problem *p, int32_t blk, int32_t g, int32_t off, int32_t i)
{
    int32_t d = p->head_dim;
    const uint16_t *base = p->pool_v + ((int64_t)blk * p->num_kv_heads + g) * (int64_t)d * ORACLE_BLOCK;
    return bf16_value(base[(int64_t)i * ORACLE_BLOCK + off]);
}

/* Keys of (request r, kv head g) rotated at their own pi; rows of masked
 * slots are left zero and flagged in `valid`. */
static void rotate_keys(const oracle_problem *p, int32_t r, int32_t g, double *kr, int32_t *valid)
{
    int32_t d = p->head_dim, n = p->kv_len[r];
    double *tmp = (double *)malloc(sizeof(double) * d);
    for (int32_t j = 0; j < n; ++j) {
        int32_t pi = p->kv_pos[(int64_t)r * kv_stride(p) + j];
        int32_t blk = slot_block(p, r, j);
        valid[j] = (pi >= 0 && blk >= 0);
        if (!valid[j]) {
            memset(kr + (int64_t)j * d, 0, sizeof(double) * d);
            continue;
        }
        load_key(p, blk, g, j % ORACLE_BLOCK, tmp);
        oracle_rope(d, p->rope_theta, pi, tmp, kr + (int64_t)j * d);
    }
    free(tmp);
}

/* Scores of one query row against every slot of its request; visible[j] says
 * whether key j takes part.  Returns the number of visible keys. */
static int32_t row_scores(const oracle_problem *p, int32_t r, int32_t t, int32_t h,
                          const double *kr, const int32_t *valid, double *s, int32_t *visible)
{
    int32_t d = p->head_dim, n = p->kv_len[r];
    double *x = (double *)malloc(sizeof(double) * d);
    double *qr = (double *)malloc(sizeof(double) * d);
    const uint16_t *src = p->q + ((int64_t)t * p->num_q_heads + h) * d;
    for (int32_t i = 0; i < d; ++i)
        x[i] = bf16_value(src[i]);
    int32_t pos = p->q_pos[t];
    oracle_rope(d, p->rope_theta, pos, x, qr);
    double scale = 1.0 / sqrt((double)d);
    int32_t nvis = 0;
    for (int32_t j = 0; j < n; ++j) {
        int32_t pi = p->kv_pos[(int64_t)r * kv_stride(p) + j];
        visible[j] = valid[j] && pi <= pos;
        if (!visible[j]) {
            s[j] = 0.0;
            continue;
        }
        double acc = 0.0;
        for (int32_t i = 0; i < d; ++i)
            acc += qr[i] * kr[(int64_t)j * d + i];
        s[j] = acc * scale;
        ++nvis;
    }
    free(x);
    free(qr);
    return nvis;
}

/* Softmax over the visible keys; returns lse (natural log), -inf if none. */
static double row_softmax(int32_t n, const double *s, const int32_t *visible, double *prob)
{
    double m = -INFINITY;
    for (int32_t j = 0; j < n; ++j)
        if (visible[j] && s[j] > m)
            m = s[j];
    if (m == -INFINITY) {
        for (int32_t j = 0; j < n; ++j)
            prob[j] = 0.0;
        return -INFINITY;
    }
    double z = 0.0;
    for (int32_t j = 0; j < n; ++j)
        z += visible[j] ? exp(s[j] - m) : 0.0;
    for (int32_t j = 0; j < n; ++j)
        prob[j] = visible[j] ? exp(s[j] - m) / z : 0.0;
    return m + log(z);
}

/*
 * Attention output and log-sum-exp for a list of (query token t, q head h)
 * rows, or for every row in (t, h) order when n_rows < 0.
 * out: [rows][d], lse: [rows].  Returns 0, or -1 on a bad row.
 */
int oracle_attention(const oracle_problem *p, int32_t n_rows, const int32_t *row_t,
                     const int32_t *row_h, double *out, double *lse)
{
    int32_t Hq = p->num_q_heads, Hkv = p->num_kv_heads, d = p->head_dim;
    int32_t G = Hq / Hkv;
    int32_t total_q = p->q_start[p->batch];
    int32_t all = n_rows < 0;
    int64_t nr = all ? (int64_t)total_q * Hq : n_rows;
    int32_t max_n = 1;
    for (int32_t r = 0; r < p->batch; ++r)
        if (p->kv_len[r] > max_n)
            max_n = p->kv_len[r];
    double *kr = (double *)malloc(sizeof(double) * (size_t)max_n * d);
    int32_t *valid = (int32_t *)malloc(sizeof(int32_t) * max_n);
    int32_t *visible = (int32_t *)malloc(sizeof(int32_t) * max_n);
    double *s = (double *)malloc(sizeof(double) * max_n);
    double *prob = (double *)malloc(sizeof(double) * max_n);
    int rc = 0;
    /* Rotate a (request, kv head)'s keys once, then serve every listed row
     * that reads them. */
    for (int32_t r = 0; r < p->batch && rc == 0; ++r) {
        for (int32_t g = 0; g < Hkv && rc == 0; ++g) {
            int have = 0;
            for (int64_t k = 0; k < nr; ++k) {
                int32_t t = all ? (int32_t)(k / Hq) : row_t[k];
                int32_t h = all ? (int32_t)(k % Hq) : row_h[k];
                if (t < 0 || t >= total_q || h < 0 || h >= Hq) {
                    rc = -1;
                    break;
                }
                if (request_of(p, t) != r || h / G != g)
                    continue;
                if (!have) {
                    rotate_keys(p, r, g, kr, valid);
                    have = 1;
                }
                int32_t n = p->kv_len[r];
                row_scores(p, r, t, h, kr, valid, s, visible);
                lse[k] = row_softmax(n, s, visible, prob);
                for (int32_t i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int32_t j = 0; j < n; ++j)
                        if (visible[j])
                            acc += prob[j] * value_elem(p, slot_block(p, r, j), g, j % ORACLE_BLOCK, i);
                    out[k * d + i] = acc;
                }
            }
        }
    }
    free(kr);
    free(valid);
    free(visible);
    free(s);
    free(prob);
    return rc;
}

/*
 * Selection mass: mass[r][j] = sum over request r's queries t and all q heads
 * h of the probability key j receives in row (t, h); 0 for keys no row sees.
 * Written for j < kv_len[r] into mass[r * stride + j]; other entries untouched.
 * Rows are added in (t ascending, h ascending) order.
 */
int oracle_mass(const oracle_problem *p, int32_t stride, double *mass)
{
    int32_t Hq = p->num_q_heads, Hkv = p->num_kv_heads, d = p->head_dim;
    int32_t G = Hq / Hkv;
    int32_t max_n = 1;
    for (int32_t r = 0; r < p->batch; ++r)
        if (p->kv_len[r] > max_n)
            max_n = p->kv_len[r];
    double *kr = (double *)malloc(sizeof(double) * (size_t)max_n * d * Hkv);
    int32_t *valid = (int32_t *)malloc(sizeof(int32_t) * max_n);
    int32_t *visible = (int32_t *)malloc(sizeof(int32_t) * max_n);
    double *s = (double *)malloc(sizeof(double) * max_n);
    double *prob = (double *)malloc(sizeof(double) * max_n);
    for (int32_t r = 0; r < p->batch; ++r) {
        int32_t n = p->kv_len[r];
        double *m = mass + (int64_t)r * stride;
        for (int32_t j = 0; j < n; ++j)
            m[j] = 0.0;
        /* valid[] depends only on pi and the block table, so it is the same
         * for every kv head. */
        for (int32_t g = 0; g < Hkv; ++g)
            rotate_keys(p, r, g, kr + (int64_t)g * max_n * d, valid);
        for (int32_t t = p->q_start[r]; t < p->q_start[r + 1]; ++t) {
            for (int32_t h = 0; h < Hq; ++h) {
                int32_t g = h / G;
                row_scores(p, r, t, h, kr + (int64_t)g * max_n * d, valid, s, visible);
                row_softmax(n, s, visible, prob);
                for (int32_t j = 0; j < n; ++j)
                    m[j] += prob[j];
            }
        }
    }
    free(kr);
    free(valid);
    free(visible);
    free(s);
    free(prob);
    return 0;
}

/*
 * Anchor score: the squared norm of each cached token's stored (unrotated)
 * key, summed over every kv head and every dimension; 0 for slots that hold no
 * usable key (pi < 0 or no block).  The pages pick anchor tokens as the small
 * fraction with the highest key norms [QCFuse (es), methodology A, anchor
 * extraction; QCFuse (de), methodik phase 1]; which heads and whether rotated
 * are not stated.  Reading: the whole key vector of the token (all kv heads);
 * RoPE is a rotation, so rotated or not gives the same norm.  Ranking by the
 * squared norm is ranking by the norm.  Written for j < kv_len[r] into
 * norm[r * stride + j]; other entries untouched.
 */
int oracle_key_norm(const oracle_problem *p, int32_t stride, double *norm)
{
    int32_t d = p->head_dim;
    double *x = (double *)malloc(sizeof(double) * d);
    for (int32_t r = 0; r < p->batch; ++r) {
        for (int32_t j = 0; j < p->kv_len[r]; ++j) {
            int32_t pi = p->kv_pos[(int64_t)r * kv_stride(p) + j];
            int32_t blk = slot_block(p, r, j);
            double acc = 0.0;
            if (pi >= 0 && blk >= 0) {
                for (int32_t g = 0; g < p->num_kv_heads; ++g) {
                    load_key(p, blk, g, j % ORACLE_BLOCK, x);
                    for (int32_t i = 0; i < d; ++i)
                        acc += x[i] * x[i];
                }
            }
            norm[(int64_t)r * stride + j] = acc;
        }
    }
    free(x);
    return 0;
}

typedef struct {
    double mass;
    int32_t idx;
} ranked_t;

/* Larger mass first; equal mass -> lower index first. */
static int by_mass_then_index(const void *a, const void *b)
{
    const ranked_t *x = (const ranked_t *)a, *y = (const ranked_t *)b;
    if (x->mass > y->mass)
        return -1;
    if (x->mass < y->mass)
        return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

static int by_index(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/*
 * Per-span top fraction.  For span s (request span_req[s], sequence slots
 * [span_start[s], span_start[s]+span_len[s])), candidates are slots with
 * pi >= 0 and j < kv_len; k = min(#candidates, floor(ratio*L + 0.5)).
 * Writes sel_off[n_spans+1] (CSR) and sel_idx[sel_off[n_spans]] (ascending
 * within a span).  sel_cap bounds sel_idx.  Returns total selected, or -1.
 */
int32_t oracle_select(int32_t n_spans, const int32_t *span_req, const int32_t *span_start,
                      const int32_t *span_len, double ratio, const double *mass, int32_t stride,
                      const int32_t *kv_pos, const int32_t *kv_len, int32_t *sel_off,
                      int32_t *sel_idx, int32_t sel_cap)
{
    int32_t total = 0;
    sel_off[0] = 0;
    for (int32_t s = 0; s < n_spans; ++s) {
        int32_t r = span_req[s], st = span_start[s], L = span_len[s];
        ranked_t *cand = (ranked_t *)malloc(sizeof(ranked_t) * (L > 0 ? L : 1));
        int32_t nc = 0;
        for (int32_t j = st; j < st + L; ++j) {
            if (j >= kv_len[r] || kv_pos[(int64_t)r * stride + j] < 0)
                continue;
            cand[nc].mass = mass[(int64_t)r * stride + j];
            cand[nc].idx = j;
            ++nc;
        }
        int32_t k = (int32_t)floor(ratio * (double)L + 0.5);
        if (k > nc)
            k = nc;
        qsort(cand, (size_t)nc, sizeof(ranked_t), by_mass_then_index);
        if (total + k > sel_cap) {
            free(cand);
            return -1;
        }
        for (int32_t i = 0; i < k; ++i)
            sel_idx[total + i] = cand[i].idx;
        qsort(sel_idx + total, (size_t)k, sizeof(int32_t), by_index);
        total += k;
        sel_off[s + 1] = total;
        free(cand);
    }
    return total;
}

/*
 * Token-level fusion, in place on the given copies.  For request r with
 * selection sel_idx[sel_req_off[r] .. sel_req_off[r+1]) and fresh rows at the
 * same indices of fresh_k/fresh_v ([n][Hkv][d]):
 *   base = 16 * ceil(kv_len[r] / 16); slots kv_len..base-1 get pi = -1;
 *   slot base+i receives fresh row i (K and V, bit for bit) and pi of the
 *   i-th selected slot, which then gets pi = -1 (an entry of -1 leaves the
 *   fresh slot empty);  kv_len[r] = base + count.
 * Returns 0, or -1 if a fresh slot has no usable block.
 */
int oracle_fuse(int32_t batch, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                int32_t max_blocks, const int32_t *block_table, int32_t *kv_len, int32_t *kv_pos,
                uint16_t *pool_k, uint16_t *pool_v, const int32_t *sel_idx,
                const int32_t *sel_req_off, const uint16_t *fresh_k, const uint16_t *fresh_v)
{
    int32_t stride = max_blocks * ORACLE_BLOCK, d = head_dim;
    for (int32_t r = 0; r < batch; ++r) {
        int32_t n0 = kv_len[r];
        int32_t base = ((n0 + ORACLE_BLOCK - 1) / ORACLE_BLOCK) * ORACLE_BLOCK;
        int32_t *pi = kv_pos + (int64_t)r * stride;
        for (int32_t j = n0; j < base; ++j)
            pi[j] = -1;
        int32_t cnt = sel_req_off[r + 1] - sel_req_off[r];
        for (int32_t i = 0; i < cnt; ++i) {
            int32_t row = sel_req_off[r] + i;
            int32_t slot = base + i;
            if (slot >= stride)
                return -1;
            int32_t blk = block_table[(int64_t)r * max_blocks + slot / ORACLE_BLOCK];
            if (blk < 0 || blk >= num_blocks)
                return -1;
            int32_t off = slot % ORACLE_BLOCK;
            for (int32_t g = 0; g < num_kv_heads; ++g) {
                uint16_t *kd = pool_k + (((int64_t)blk * num_kv_heads + g) * ORACLE_BLOCK + off) * d;
                uint16_t *vd = pool_v + ((int64_t)blk * num_kv_heads + g) * (int64_t)d * ORACLE_BLOCK;
                const uint16_t *ks = fresh_k + ((int64_t)row * num_kv_heads + g) * d;
                const uint16_t *vs = fresh_v + ((int64_t)row * num_kv_heads + g) * d;
                for (int32_t e = 0; e < d; ++e) {
                    kd[e] = ks[e];
                    vd[(int64_t)e * ORACLE_BLOCK + off] = vs[e];
                }
            }
            int32_t sel = sel_idx[row];
            if (sel >= 0) {
                pi[slot] = pi[sel];
                pi[sel] = -1;
            } else {
                pi[slot] = -1;
            }
        }
        kv_len[r] = base + cnt;
    }
    return 0;
}
