/*
 * CPU oracle of the decoder-only transformer forward.  TEST INFRASTRUCTURE
 * ONLY: tests, the smoke check and the bench's CPU baseline load it; the
 * product path never does.  It shares no code, header or table with the HIP
 * library.
 *
 * Plain C, built twice from this file: REAL=float (the fp32 oracle) and
 * REAL=double (its float64 shadow).  Every dot product and every reduction is
 * a sequential sum in ascending index order, so results do not depend on the
 * thread count; OpenMP only splits independent output rows.  Matrices are
 * bf16 bit patterns widened exactly (or fp32 for an fp32 model); norm gains
 * and biases are fp32.  The KV cache is REAL.
 *
 * What it computes follows the pages:
 *   - step order: Pantheon "Llama Forward Pass", section "Forward Pass Flow";
 *     sipllm "Transformer forward pass", section "Shared attention";
 *   - RMSNorm: Pantheon, section "RMSNorm";
 *   - RoPE on adjacent pairs (2i, 2i+1), pair i turning theta^(-2i/head_dim)
 *     rad per position: sipllm, "RoPE is adjacent-pair"; rml "The decoder",
 *     "Rotary embeddings"; the halves pairing (i, i + hd/2) and llama3
 *     frequency scaling as described there ("Which dimensions pair", worked
 *     example of the scaling);
 *   - optional bf16 K/V cache (rml, "Attend": the cache stores its dtype);
 *   - GQA head map h -> h*n_kv/n_head: Pantheon, "Grouped Query Attention";
 *   - attention as materialised scores, softmax, weighted sum (rml's AttendRef,
 *     "Attend"); window start max(0, pos-W+1): rml, "Attend";
 *   - circular KV cache (slot pos % max_seq, readable min(pos+1, max_seq)):
 *     Pantheon, "Sliding Window (Mistral)";
 *   - SwiGLU: Pantheon, "SwiGLU FFN";
 *   - MoE: router softmax, top-k by repeated selection with ties to the lower
 *     id, weights p_e / sum of chosen p, weighted sum of expert SwiGLUs:
 *     Pantheon, "Mixture of Experts (Mixtral)"; rml, "Mixture of experts";
 *   - single-pass prefill: positions ascending within each layer, the same
 *     result as one call per token, logits for the last position:
 *     sipllm, "Single-pass prefill";
 *   - batched decode: independent rows with their own cache and position:
 *     Pantheon, "Batched Multi-Sequence Decode";
 *   - checks before any change, nothing mutated on error: rml, "One forward pass".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef REAL
#define REAL float
#endif
typedef REAL real;

#if defined(ORACLE_DOUBLE)
#define R_EXP exp
#define R_SQRT sqrt
#define SYM(name) oracle64_##name
#else
#define R_EXP expf
#define R_SQRT sqrtf
#define SYM(name) oracle32_##name
#endif

#define EXPORT __attribute__((visibility("default")))

enum { O_OK = 0, O_ERR_INVALID = -1, O_ERR_RANGE = -2, O_ERR_NOMEM = -3 };

typedef struct {
    int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
    int32_t n_experts, top_k, qkv_bias, sliding_window, max_seq, n_slots, weight_f32;
    /* 1: keep a linear cache of max_seq positions and mask the window instead of
       using a ring; a second code path that exists only to pin the ring. */
    int32_t window_by_mask;
    double rms_eps, rope_theta;
    /* RoPE variants: pairing 0 = adjacent (2i, 2i+1), 1 = halves (i, i + hd/2);
       scaling 0 = none, 1 = llama3 frequency scaling with factor, low/high
       frequency factors and original context. */
    int32_t rope_pairing, rope_scaling, rope_orig_ctx;
    /* Rounding of K and V when stored in the cache: 0 none (the working
       precision), 1 bf16 (8 significant bits, nearest even), 2 a 24-bit float
       (sign, 8 exponent bits, 15 stored mantissa bits: 16 significant bits,
       nearest even). */
    int32_t kv_round;
    double rope_factor, rope_low_freq_factor, rope_high_freq_factor;
} ocfg;

typedef struct {
    const float *attn_norm;
    const void *wq, *wk, *wv;
    const float *bq, *bk, *bv;
    const void *wo;
    const float *ffn_norm;
    const void *w_gate, *w_up, *w_down, *router;
} olayer;

typedef struct {
    ocfg c;
    const void *embed;
    const float *out_norm;
    const void *lm_head;
    olayer *layers;
    real *kcache, *vcache;  /* [layer][slot][pos][kv_dim] */
    int32_t *len;           /* committed length per slot */
} omodel;

/* ---- weights ---------------------------------------------------------- */

static inline real wget(const void *w, size_t i, int f32) {
    if (f32) return (real)((const float *)w)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)w)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (real)f;
}

/* y[r] = sum_c W[r][c] * a[c] for r in [0, rows); W row-major [rows][cols]. */
static void matvec(const void *W, int f32, int rows, int cols, const real *a, real *y) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++) {
        real s = 0;
        size_t base = (size_t)r * cols;
        for (int c = 0; c < cols; c++) s += wget(W, base + c, f32) * a[c];
        y[r] = s;
    }
}

/* ---- ops (exported for the pins) ------------------------------------- */

/* RMSNorm: out = x / sqrt(mean(x^2) + eps) * g. */
EXPORT void SYM(rmsnorm)(const real *x, const float *g, int d, double eps, real *out) {
    real s = 0;
    for (int i = 0; i < d; i++) s += x[i] * x[i];
    real r = (real)1 / R_SQRT(s / (real)d + (real)eps);
    for (int i = 0; i < d; i++) out[i] = x[i] * r * (real)g[i];
}

/* llama3 frequency scaling of one pair's frequency (rml "The decoder",
   "Rotary embeddings" and its worked example): with wavelength 2*pi/f, pairs
   under orig_ctx/high keep f, pairs over orig_ctx/low turn `factor` times
   slower, and in between smooth = (orig_ctx/wavelength - low) / (high - low)
   blends (1 - smooth) * f/factor + smooth * f. */
EXPORT double SYM(llama3_inv_freq)(double f, double factor, double low, double high, int orig_ctx) {
    const double pi = 3.14159265358979323846;
    double wavelen = 2.0 * pi / f;
    if (wavelen < (double)orig_ctx / high) return f;
    if (wavelen > (double)orig_ctx / low) return f / factor;
    double smooth = ((double)orig_ctx / wavelen - low) / (high - low);
    return (1.0 - smooth) * (f / factor) + smooth * f;
}

/* Rotate the pairs of each of n_heads heads of h[n_heads*hd] in place.  Pair i
   turns pos * theta^(-2i/hd) radians (optionally llama3-scaled), angle formed in
   double; pairing 0 rotates (2i, 2i+1), pairing 1 rotates (i, i + hd/2). */
EXPORT void SYM(rope_ex)(real *h, int n_heads, int hd, int pos, double theta, int pairing, int scaling,
                         double factor, double low, double high, int orig_ctx) {
    for (int i = 0; i < hd / 2; i++) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)hd);
        if (scaling == 1) inv_freq = SYM(llama3_inv_freq)(inv_freq, factor, low, high, orig_ctx);
        double ang = (double)pos * inv_freq;
        real c = (real)cos(ang), s = (real)sin(ang);
        int a = pairing ? i : 2 * i, b = pairing ? i + hd / 2 : 2 * i + 1;
        for (int hh = 0; hh < n_heads; hh++) {
            real *p = h + (size_t)hh * hd;
            real e0 = p[a], e1 = p[b];
            p[a] = e0 * c - e1 * s;
            p[b] = e0 * s + e1 * c;
        }
    }
}

/* Plain RoPE: adjacent pairs, no scaling. */
EXPORT void SYM(rope)(real *h, int n_heads, int hd, int pos, double theta) {
    SYM(rope_ex)(h, n_heads, hd, pos, theta, 0, 0, 1.0, 1.0, 1.0, 1);
}

/* Nearest-even bf16 of a value (through fp32), kept in the oracle's type. */
static real bf16_round(real v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    memcpy(&f, &u, sizeof f);
    return (real)f;
}

/* The value as a float with its low 8 mantissa bits cleared, rounded to
   nearest even first: fp32's layout with 15 stored mantissa bits. */
static real f24_round(real v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u = (u + 0x7Fu + ((u >> 8) & 1u)) & 0xFFFFFF00u;
    memcpy(&f, &u, sizeof f);
    return (real)f;
}

static inline real silu(real z) { return z / ((real)1 + R_EXP(-z)); }

/* Router: softmax over all experts, top-k by repeated selection (ties to the
   lower id), weights renormalised to sum 1 (p_e / sum of chosen p). */
EXPORT void SYM(moe_route)(const real *logits, int n_experts, int k, int32_t *ids, real *w) {
    real p[256];
    real m = logits[0];
    for (int e = 1; e < n_experts; e++) if (logits[e] > m) m = logits[e];
    real z = 0;
    for (int e = 0; e < n_experts; e++) { p[e] = R_EXP(logits[e] - m); z += p[e]; }
    for (int e = 0; e < n_experts; e++) p[e] = p[e] / z;
    char taken[256] = {0};
    real total = 0;
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < n_experts; e++)
            if (!taken[e] && (best < 0 || p[e] > p[best])) best = e;
        taken[best] = 1;
        ids[j] = best;
        w[j] = p[best];
        total += p[best];
    }
    for (int j = 0; j < k; j++) w[j] = w[j] / total;
}

/* Attention of one query head over cached positions [lo, pos] (the AttendRef
   definition): score_j = q.k_j / sqrt(hd), softmax, sum_j prob_j v_j. */
static void attend_head(const real *q, const real *K, const real *V, size_t row_stride,
                        const int *slots, int n, int hd, real *scores, real *out) {
    real scale = R_SQRT((real)hd);
    real m = 0;
    for (int j = 0; j < n; j++) {
        const real *k = K + (size_t)slots[j] * row_stride;
        real s = 0;
        for (int i = 0; i < hd; i++) s += q[i] * k[i];
        s = s / scale;
        scores[j] = s;
        if (j == 0 || s > m) m = s;
    }
    real z = 0;
    for (int j = 0; j < n; j++) { scores[j] = R_EXP(scores[j] - m); z += scores[j]; }
    for (int i = 0; i < hd; i++) out[i] = 0;
    for (int j = 0; j < n; j++) {
        real pj = scores[j] / z;
        const real *v = V + (size_t)slots[j] * row_stride;
        for (int i = 0; i < hd; i++) out[i] += pj * v[i];
    }
}

/* Exported for the pins: causal GQA attention of n positions 0..n-1 with
   q [n][n_heads][hd], k, v [n][n_kv][hd], optional window (0 = none). */
EXPORT void SYM(attention_prefill)(const real *q, const real *k, const real *v, int n,
                                   int n_heads, int n_kv, int hd, int window, real *out) {
    int *slots = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    real *scores = (real *)malloc(sizeof(real) * (size_t)(n > 0 ? n : 1));
    for (int t = 0; t < n; t++) {
        int lo = (window > 0 && t - window + 1 > 0) ? t - window + 1 : 0;
        int cnt = t - lo + 1;
        for (int j = 0; j < cnt; j++) slots[j] = lo + j;
        for (int h = 0; h < n_heads; h++) {
            int g = h * n_kv / n_heads;
            attend_head(q + ((size_t)t * n_heads + h) * hd, k + (size_t)g * hd, v + (size_t)g * hd,
                        (size_t)n_kv * hd, slots, cnt, hd, scores,
                        out + ((size_t)t * n_heads + h) * hd);
        }
    }
    free(slots);
    free(scores);
}

/* ---- model ------------------------------------------------------------ */

/* The cache is a ring of max_seq slots written at pos % max_seq only when the
   window equals max_seq (Pantheon, "Sliding Window (Mistral)": the ring holds
   the window, min(pos+1, max_seq) positions readable).  A window longer than
   max_seq can never bind inside max_seq positions: such a cache is linear and
   full-causal with capacity max_seq (positions past it are a range error). */
static int is_ring(const ocfg *c) {
    return c->sliding_window > 0 && !c->window_by_mask && c->max_seq == c->sliding_window;
}

static int cfg_valid(const ocfg *c) {
    if (c->n_layers <= 0 || c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 ||
        c->head_dim <= 0 || c->ffn_dim <= 0 || c->vocab <= 0 || c->max_seq <= 0 || c->n_slots <= 0)
        return 0;
    if (c->n_heads % c->n_kv_heads) return 0;
    if (c->head_dim % 2) return 0;
    if (!(c->rms_eps > 0) || !(c->rope_theta > 0)) return 0;
    if (c->rope_pairing < 0 || c->rope_pairing > 1 || c->rope_scaling < 0 || c->rope_scaling > 1) return 0;
    if (c->rope_scaling == 1 && (!(c->rope_factor > 0) || !(c->rope_low_freq_factor > 0) ||
                                 !(c->rope_high_freq_factor > c->rope_low_freq_factor) || c->rope_orig_ctx <= 0))
        return 0;
    if (c->n_experts < 0 || c->n_experts > 256) return 0;
    if (c->n_experts > 0 && (c->top_k < 1 || c->top_k > c->n_experts)) return 0;
    if (c->sliding_window < 0) return 0;
    if (c->kv_round < 0 || c->kv_round > 2) return 0;
    if (c->sliding_window > 0 && !c->window_by_mask && c->max_seq > c->sliding_window) return 0;
    return 1;
}

EXPORT void *SYM(create)(const ocfg *c, const void *embed, const float *out_norm,
                         const void *lm_head, const olayer *layers) {
    if (!c || !cfg_valid(c) || !embed || !out_norm || !layers) return NULL;
    omodel *m = (omodel *)calloc(1, sizeof(omodel));
    if (!m) return NULL;
    m->c = *c;
    m->embed = embed;
    m->out_norm = out_norm;
    m->lm_head = lm_head ? lm_head : embed;
    m->layers = (olayer *)malloc(sizeof(olayer) * (size_t)c->n_layers);
    memcpy(m->layers, layers, sizeof(olayer) * (size_t)c->n_layers);
    size_t kv_dim = (size_t)c->n_kv_heads * c->head_dim;
    size_t n = (size_t)c->n_layers * c->n_slots * c->max_seq * kv_dim;
    m->kcache = (real *)calloc(n, sizeof(real));
    m->vcache = (real *)calloc(n, sizeof(real));
    m->len = (int32_t *)calloc((size_t)c->n_slots, sizeof(int32_t));
    if (!m->layers || !m->kcache || !m->vcache || !m->len) {
        free(m->layers); free(m->kcache); free(m->vcache); free(m->len); free(m);
        return NULL;
    }
    return m;
}

EXPORT void SYM(destroy)(void *h) {
    omodel *m = (omodel *)h;
    if (!m) return;
    free(m->layers); free(m->kcache); free(m->vcache); free(m->len); free(m);
}

EXPORT int SYM(reset)(void *h, int slot) {
    omodel *m = (omodel *)h;
    if (slot < -1 || slot >= m->c.n_slots) return O_ERR_INVALID;
    for (int s = 0; s < m->c.n_slots; s++)
        if (slot == -1 || s == slot) m->len[s] = 0;
    return O_OK;
}

EXPORT int SYM(length)(void *h, int slot) { return ((omodel *)h)->len[slot]; }

/* Read access to the cache for the pins: one position's K or V row. */
EXPORT void SYM(kv_row)(void *h, int layer, int slot, int which, int pos, real *out) {
    omodel *m = (omodel *)h;
    const ocfg *c = &m->c;
    size_t kv_dim = (size_t)c->n_kv_heads * c->head_dim;
    int s = is_ring(c) ? pos % c->max_seq : pos;
    size_t off = (((size_t)layer * c->n_slots + slot) * c->max_seq + s) * kv_dim;
    memcpy(out, (which ? m->vcache : m->kcache) + off, kv_dim * sizeof(real));
}

typedef struct {
    real *a, *q, *k, *v, *att, *o, *g, *u, *y, *ye, *rl, *scores;
    int *slots;
} scratch;

static int scratch_alloc(scratch *s, const ocfg *c) {
    size_t d = c->hidden, q = (size_t)c->n_heads * c->head_dim, kv = (size_t)c->n_kv_heads * c->head_dim;
    size_t f = c->ffn_dim;
    s->a = malloc(d * sizeof(real)); s->q = malloc(q * sizeof(real));
    s->k = malloc(kv * sizeof(real)); s->v = malloc(kv * sizeof(real));
    s->att = malloc(q * sizeof(real)); s->o = malloc(d * sizeof(real));
    s->g = malloc(f * sizeof(real)); s->u = malloc(f * sizeof(real));
    s->y = malloc(d * sizeof(real)); s->ye = malloc(d * sizeof(real));
    s->rl = malloc(((size_t)c->n_experts + 1) * sizeof(real));
    s->scores = malloc((size_t)c->max_seq * sizeof(real));
    s->slots = malloc((size_t)c->max_seq * sizeof(int));
    return s->a && s->q && s->k && s->v && s->att && s->o && s->g && s->u && s->y && s->ye &&
           s->rl && s->scores && s->slots;
}

static void scratch_free(scratch *s) {
    free(s->a); free(s->q); free(s->k); free(s->v); free(s->att); free(s->o);
    free(s->g); free(s->u); free(s->y); free(s->ye); free(s->rl); free(s->scores); free(s->slots);
}

/* First half of a block for one position: attention norm, q/k/v (+bias), RoPE,
   K/V stored at the position's slot.  Leaves q in s->q. */
static void block_kv(omodel *m, int l, int slot, int pos, const real *x, scratch *s) {
    const ocfg *c = &m->c;
    const olayer *L = &m->layers[l];
    int f32 = c->weight_f32, d = c->hidden, hd = c->head_dim;
    int qd = c->n_heads * hd, kvd = c->n_kv_heads * hd;
    SYM(rmsnorm)(x, L->attn_norm, d, c->rms_eps, s->a);
    matvec(L->wq, f32, qd, d, s->a, s->q);
    matvec(L->wk, f32, kvd, d, s->a, s->k);
    matvec(L->wv, f32, kvd, d, s->a, s->v);
    if (c->qkv_bias) {
        for (int i = 0; i < qd; i++) s->q[i] += (real)L->bq[i];
        for (int i = 0; i < kvd; i++) s->k[i] += (real)L->bk[i];
        for (int i = 0; i < kvd; i++) s->v[i] += (real)L->bv[i];
    }
    SYM(rope_ex)(s->q, c->n_heads, hd, pos, c->rope_theta, c->rope_pairing, c->rope_scaling, c->rope_factor,
                 c->rope_low_freq_factor, c->rope_high_freq_factor, c->rope_orig_ctx);
    SYM(rope_ex)(s->k, c->n_kv_heads, hd, pos, c->rope_theta, c->rope_pairing, c->rope_scaling, c->rope_factor,
                 c->rope_low_freq_factor, c->rope_high_freq_factor, c->rope_orig_ctx);
    if (c->kv_round == 1) {
        for (int i = 0; i < kvd; i++) s->k[i] = bf16_round(s->k[i]);
        for (int i = 0; i < kvd; i++) s->v[i] = bf16_round(s->v[i]);
    } else if (c->kv_round == 2) {
        for (int i = 0; i < kvd; i++) s->k[i] = f24_round(s->k[i]);
        for (int i = 0; i < kvd; i++) s->v[i] = f24_round(s->v[i]);
    }
    int sl = is_ring(c) ? pos % c->max_seq : pos;
    size_t off = (((size_t)l * c->n_slots + slot) * c->max_seq + sl) * (size_t)kvd;
    memcpy(m->kcache + off, s->k, (size_t)kvd * sizeof(real));
    memcpy(m->vcache + off, s->v, (size_t)kvd * sizeof(real));
}

/* Second half: attention over the readable window, output projection and
   residual, FFN norm, dense SwiGLU or MoE, residual.  Updates x in place. */
static void block_rest(omodel *m, int l, int slot, int pos, real *x, scratch *s,
                       real *router_cap, int32_t *ids_cap) {
    const ocfg *c = &m->c;
    const olayer *L = &m->layers[l];
    int f32 = c->weight_f32, d = c->hidden, hd = c->head_dim, f = c->ffn_dim;
    int qd = c->n_heads * hd, kvd = c->n_kv_heads * hd;
    int ring = is_ring(c);
    int lo = 0;
    if (c->sliding_window > 0 && pos - c->sliding_window + 1 > 0) lo = pos - c->sliding_window + 1;
    int cnt = pos - lo + 1;  /* <= max_seq: a ring holds the window, a linear cache every position */
    for (int j = 0; j < cnt; j++) s->slots[j] = ring ? (lo + j) % c->max_seq : lo + j;
    const real *K = m->kcache + ((size_t)l * c->n_slots + slot) * c->max_seq * (size_t)kvd;
    const real *V = m->vcache + ((size_t)l * c->n_slots + slot) * c->max_seq * (size_t)kvd;
    for (int h = 0; h < c->n_heads; h++) {
        int g = h * c->n_kv_heads / c->n_heads;
        attend_head(s->q + (size_t)h * hd, K + (size_t)g * hd, V + (size_t)g * hd, (size_t)kvd,
                    s->slots, cnt, hd, s->scores, s->att + (size_t)h * hd);
    }
    matvec(L->wo, f32, d, qd, s->att, s->o);
    for (int i = 0; i < d; i++) x[i] += s->o[i];

    SYM(rmsnorm)(x, L->ffn_norm, d, c->rms_eps, s->a);
    if (c->n_experts == 0) {
        matvec(L->w_gate, f32, f, d, s->a, s->g);
        matvec(L->w_up, f32, f, d, s->a, s->u);
        for (int i = 0; i < f; i++) s->g[i] = silu(s->g[i]) * s->u[i];
        matvec(L->w_down, f32, d, f, s->g, s->y);
    } else {
        int E = c->n_experts, k = c->top_k;
        int32_t ids[256];
        real w[256];
        matvec(L->router, f32, E, d, s->a, s->rl);
        if (router_cap) for (int e = 0; e < E; e++) router_cap[e] = s->rl[e];
        SYM(moe_route)(s->rl, E, k, ids, w);
        if (ids_cap) for (int j = 0; j < k; j++) ids_cap[j] = ids[j];
        for (int i = 0; i < d; i++) s->y[i] = 0;
        size_t gsz = (size_t)f * d;  /* one expert's gate/up/down element count */
        for (int j = 0; j < k; j++) {
            size_t eo = (size_t)ids[j] * gsz;
            const void *wg = f32 ? (const void *)((const float *)L->w_gate + eo)
                                 : (const void *)((const uint16_t *)L->w_gate + eo);
            const void *wu = f32 ? (const void *)((const float *)L->w_up + eo)
                                 : (const void *)((const uint16_t *)L->w_up + eo);
            const void *wd = f32 ? (const void *)((const float *)L->w_down + eo)
                                 : (const void *)((const uint16_t *)L->w_down + eo);
            matvec(wg, f32, f, d, s->a, s->g);
            matvec(wu, f32, f, d, s->a, s->u);
            for (int i = 0; i < f; i++) s->g[i] = silu(s->g[i]) * s->u[i];
            matvec(wd, f32, d, f, s->g, s->ye);
            for (int i = 0; i < d; i++) s->y[i] += w[j] * s->ye[i];
        }
    }
    for (int i = 0; i < d; i++) x[i] += s->y[i];
}

static void embed_row(omodel *m, int tok, real *x) {
    const ocfg *c = &m->c;
    for (int i = 0; i < c->hidden; i++) x[i] = wget(m->embed, (size_t)tok * c->hidden + i, c->weight_f32);
}

static void head_row(omodel *m, const real *x, scratch *s, real *logits) {
    const ocfg *c = &m->c;
    SYM(rmsnorm)(x, m->out_norm, c->hidden, c->rms_eps, s->a);
    matvec(m->lm_head, c->weight_f32, c->vocab, c->hidden, s->a, logits);
}

static int capacity_ok(const ocfg *c, int start_pos, int n) {
    if (is_ring(c)) return 1;
    return (long)start_pos + n <= (long)c->max_seq;
}

/*
 * Prefill n tokens of slot `slot` at positions start_pos.. (start_pos must equal
 * the slot's committed length).  Layer by layer, positions ascending.
 * rows/n_rows: ascending row indices (0..n-1) whose final hidden state and
 * logits are wanted; NULL means {n-1}.  With `partial` set, the last layer runs
 * its second half only for those rows (K/V are still stored for every row, so
 * the cache is complete); otherwise every row is computed in every layer.
 * logits: [n_rows][vocab].  Captures (each may be NULL):
 *   hidden_cap [(n_layers+1)][n][hidden]  (after the embedding and each layer;
 *              rows skipped by `partial` in the last layer are left untouched)
 *   router_cap [n_layers][n][n_experts], ids_cap [n_layers][n][top_k].
 */
EXPORT int SYM(prefill)(void *h, int slot, const int32_t *tokens, int n, int start_pos,
                        const int32_t *rows, int n_rows, int partial, real *logits,
                        real *hidden_cap, real *router_cap, int32_t *ids_cap) {
    omodel *m = (omodel *)h;
    const ocfg *c = &m->c;
    if (!m || !tokens || n <= 0 || slot < 0 || slot >= c->n_slots) return O_ERR_INVALID;
    for (int t = 0; t < n; t++) if (tokens[t] < 0 || tokens[t] >= c->vocab) return O_ERR_INVALID;
    if (start_pos != m->len[slot]) return O_ERR_INVALID;
    if (!capacity_ok(c, start_pos, n)) return O_ERR_RANGE;
    int last = n - 1;
    if (!rows) { rows = &last; n_rows = 1; }
    for (int i = 0; i < n_rows; i++)
        if (rows[i] < 0 || rows[i] >= n || (i && rows[i] <= rows[i - 1])) return O_ERR_INVALID;

    int d = c->hidden;
    real *X = (real *)malloc(sizeof(real) * (size_t)n * d);
    char *need = (char *)calloc((size_t)n, 1);
    scratch s;
    if (!X || !need || !scratch_alloc(&s, c)) { free(X); free(need); return O_ERR_NOMEM; }
    for (int i = 0; i < n_rows; i++) need[rows[i]] = 1;

    for (int t = 0; t < n; t++) embed_row(m, tokens[t], X + (size_t)t * d);
    if (hidden_cap) memcpy(hidden_cap, X, sizeof(real) * (size_t)n * d);
    for (int l = 0; l < c->n_layers; l++) {
        int restrict_rows = partial && l == c->n_layers - 1;
        for (int t = 0; t < n; t++) {
            int pos = start_pos + t;
            real *x = X + (size_t)t * d;
            block_kv(m, l, slot, pos, x, &s);
            if (restrict_rows && !need[t]) continue;
            block_rest(m, l, slot, pos, x, &s,
                       router_cap ? router_cap + ((size_t)l * n + t) * c->n_experts : NULL,
                       ids_cap ? ids_cap + ((size_t)l * n + t) * c->top_k : NULL);
            if (hidden_cap) memcpy(hidden_cap + ((size_t)(l + 1) * n + t) * d, x, sizeof(real) * d);
        }
    }
    for (int i = 0; i < n_rows; i++)
        head_row(m, X + (size_t)rows[i] * d, &s, logits + (size_t)i * c->vocab);
    m->len[slot] = start_pos + n;
    scratch_free(&s);
    free(X);
    free(need);
    return O_OK;
}

/*
 * One decode step for B independent rows: row b uses slot b, token tokens[b]
 * at position pos[b] (= slot b's committed length).  logits [B][vocab].
 * Captures as in prefill with n = B.
 */
EXPORT int SYM(decode)(void *h, int B, const int32_t *tokens, const int32_t *pos, real *logits,
                       real *hidden_cap, real *router_cap, int32_t *ids_cap) {
    omodel *m = (omodel *)h;
    const ocfg *c = &m->c;
    if (!m || !tokens || !pos || B <= 0 || B > c->n_slots) return O_ERR_INVALID;
    for (int b = 0; b < B; b++) {
        if (tokens[b] < 0 || tokens[b] >= c->vocab) return O_ERR_INVALID;
        if (pos[b] != m->len[b]) return O_ERR_INVALID;
        if (!capacity_ok(c, pos[b], 1)) return O_ERR_RANGE;
    }
    int d = c->hidden;
    real *X = (real *)malloc(sizeof(real) * (size_t)B * d);
    scratch s;
    if (!X || !scratch_alloc(&s, c)) { free(X); return O_ERR_NOMEM; }
    for (int b = 0; b < B; b++) embed_row(m, tokens[b], X + (size_t)b * d);
    if (hidden_cap) memcpy(hidden_cap, X, sizeof(real) * (size_t)B * d);
    for (int l = 0; l < c->n_layers; l++) {
        for (int b = 0; b < B; b++) {
            real *x = X + (size_t)b * d;
            block_kv(m, l, b, pos[b], x, &s);
            block_rest(m, l, b, pos[b], x, &s,
                       router_cap ? router_cap + ((size_t)l * B + b) * c->n_experts : NULL,
                       ids_cap ? ids_cap + ((size_t)l * B + b) * c->top_k : NULL);
            if (hidden_cap) memcpy(hidden_cap + ((size_t)(l + 1) * B + b) * d, x, sizeof(real) * d);
        }
    }
    for (int b = 0; b < B; b++) head_row(m, X + (size_t)b * d, &s, logits + (size_t)b * c->vocab);
    for (int b = 0; b < B; b++) m->len[b] = pos[b] + 1;
    scratch_free(&s);
    free(X);
    return O_OK;
}

/* Greedy choice: the largest logit, lowest id on ties. */
EXPORT int SYM(argmax)(const real *logits, int vocab) {
    int best = 0;
    for (int i = 1; i < vocab; i++) if (logits[i] > logits[best]) best = i;
    return best;
}
