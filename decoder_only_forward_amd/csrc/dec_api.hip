// Host side of the C ABI: validation, the workspace plan, KV bookkeeping and
// the per-layer launch sequence of prefill and batched decode.
//
// Step order of one layer (Pantheon "Llama Forward Pass", section "Forward Pass
// Flow"; rml "The decoder", section "One forward pass"):
//   norm -> q|k|v projection (+bias) -> RoPE + K/V store -> attention ->
//   output projection + residual (+ FFN norm) -> gate|up -> silu*up -> down
//   (or router -> top-k -> grouped experts) -> residual (+ next norm).
// The residual add and the next RMSNorm share one kernel; split-K partials of
// a projection are summed by the kernel that consumes them.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "dec.h"
#include "kernels.h"
#include "kvcache.h"

static_assert(DEC_KV_F32 == KV_F32 && DEC_KV_BF16 == KV_BF16 && DEC_KV_F24 == KV_F24,
              "the cache formats of the kernels are dec_config.kv_dtype's values");

namespace {

struct EvPair {
    hipEvent_t e1, e2;
};

struct Timing {
    bool on = false;
    double ms = 0;
    int64_t launches = 0;
    double bytes = 0, flops = 0;
    std::vector<EvPair> pending;  // recorded, not yet read
};

// One captured decode step: B rows, attention split count and logits buffer
// fix the launch sequence; tokens/positions enter through the first node
// (set_rows), whose arguments are replaced before each replay.  Per-kernel
// timing and test captures run eagerly instead.
struct GraphEntry {
    int B = 0, S = 0;
    bool greedy = false;    // ends with the greedy choice into amax (device loop)
    float *logits = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipGraphNode_t root = nullptr;
    hipKernelNodeParams kp{};
    unsigned long long used = 0;  // replay clock of the last use (least recently used is evicted)
};

// Captured steps kept per handle.  The attention split count follows the
// context length, so one growing sequence meets a new shape every few hundred
// positions; the oldest-used graph makes room beyond this many.
constexpr size_t MAX_GRAPHS = 16;

struct Plan {  // byte offsets into the workspace
    size_t kv_layer;        // elements of one layer's K (or V) cache
    size_t k, v, ck, cv, kvimg, s_hi, s_lo, x, x2, part2, a_hi, a_lo, a_f32, part, q, attn, rope, tok, pos, slot, amax, ssq;
    size_t moe_ids, moe_w, moe_cnt, moe_off, moe_pairs, moe_inv, g_hi, g_lo, g_f32;
    size_t part_floats, act_elems, total;
    int rows;               // max rows of one pass (max(max_batch, max_prefill))
    // prefill projections on fp16 + fp8 operands: the converted weights of
    // each layer (q|k|v, then for a dense FFN gate|up)
    bool f8;
    size_t f8w, f8_layer;
};

constexpr int MAX_ATTN_SPLITS = 64;

}  // namespace

struct dec_model {
    dec_config c;
    std::vector<dec_layer_weights> L;
    const void *embed;
    const float *out_norm;
    const void *lm_head;
    hipStream_t st;
    char *ws;
    Plan pl;
    char *kc, *vc;          // caches, kv_es bytes per element
    char *ck, *cv;          // chunk K/V of a deferred-commit prefill (ring only)
    void *kvimg;            // prefill attention's K/V tile images (null: not used)
    u16 *s_hi, *s_lo;       // fused SwiGLU output of a prefill (null: not used)
    int kv_es;
    float *x, *x2, *part2, *a_f32, *part, *q, *attn, *moe_w, *g_f32, *ssq;
    u16 *a_hi, *a_lo, *g_hi, *g_lo;
    float2 *rope;
    int32_t *tok, *pos, *slot, *amax, *moe_ids, *moe_cnt, *moe_off, *moe_pairs, *moe_inv;
    std::vector<int> len;
    // converted weights of the prefill projections on fp16 + fp8 operands
    struct F8Layer {
        F8Weights qkv, gu;
    };
    std::vector<F8Layer> f8w;
    float *cap_hidden = nullptr, *cap_router = nullptr;
    int32_t *cap_ids = nullptr;
    Timing tm[DEC_K_COUNT];
    std::vector<hipEvent_t> pool;      // free events for eager timing
    int wf32;
    int ring;
    // decode graphs: captured on `cs`, fenced to the caller's stream by events
    hipStream_t cs = nullptr;
    hipEvent_t fence_in = nullptr, fence_out = nullptr;
    std::vector<GraphEntry> graphs;
    unsigned long long graph_clock = 0;
    std::vector<std::pair<std::vector<long long>, int>> seen;  // shapes met once (captured on the second)
    int static_dev = -1;    // >= 0: the workspace is that device's copy of `scratch`
};

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bytes of one K/V cache element: fp32 4, bf16 2, 24-bit 3
inline size_t kv_elem_bytes(const dec_config &c) {
    return c.kv_dtype == DEC_KV_BF16 ? 2 : (c.kv_dtype == DEC_KV_F24 ? 3 : 4);
}

int proj_splits(const dec_config &c, int N, int K, int B, bool grouped = false) {
    if (c.weight_dtype == DEC_WEIGHT_F32 || B > 64) return 1;
    return grouped ? gemv_grouped_max_splits(K) : gemv_max_splits(N, K);
}

// One decode row of a model whose residual + RMSNorm the next projection's
// blocks form in their prologue (bf16 weights, dense FFN; each block reads the
// row and its k-split partials before its first product, which pays only
// where the projections are short: Qwen2.5-0.5B B = 1 1.232 -> 1.166 ms a
// step, SmolLM2-135M 1.256 -> 1.148, but Mistral-7B, d x F = 58.7 M, 3.600 ->
// 3.690, so the larger FFNs keep the norm kernel).
bool row_norm_fused(const dec_config &c) {
    const long d = c.hidden, F = c.ffn_dim;
    return c.weight_dtype != DEC_WEIGHT_F32 && c.n_experts == 0 && F % 8 == 0 && d % 64 == 0 && d <= 8192 &&
           d * F <= (16l << 20);
}

bool plan(const dec_config &c, Plan &p) {
    const size_t d = c.hidden, hd = c.head_dim, qd = (size_t)c.n_heads * hd, kvd = (size_t)c.n_kv_heads * hd;
    const size_t F = c.ffn_dim, E = c.n_experts, k = c.n_experts ? c.top_k : 0;
    const int rows = std::max(c.max_batch, c.max_prefill);
    const size_t prow = (size_t)rows * std::max<size_t>(k, 1);  // rows incl. MoE pairs
    p.rows = rows;
    p.kv_layer = (size_t)c.max_batch * c.n_kv_heads * c.max_seq * hd;
    const size_t kmax = std::max(std::max(d, qd), F);
    p.act_elems = prow * kmax;
    // fp16 + fp8 prefill operands (bf16 weights: every k is already a multiple of 64)
    p.f8 = c.prefill_operands == DEC_PREFILL_F16_F8 && c.weight_dtype == DEC_WEIGHT_BF16 && c.max_prefill > 64;
    // projection outputs: largest (splits x rows x N) over the projections
    size_t pf = 0;
    auto need = [&](int N, int K, int T) {
        // GEMM rows: room for the k split a 256-CU device takes (a device with
        // another count falls back to one split where the room is short)
        int S = (T <= 64) ? proj_splits(c, N, K, T)
                          : (c.weight_dtype == DEC_WEIGHT_F32 ? 1 : gemm_splits_for(N, K, T, 256));
        if (p.f8 && T > 64) S = std::max(S, gemm_splits_for(N, K, T, 256, 2));
        pf = std::max(pf, (size_t)S * T * N);
    };
    for (int T : {c.max_batch, std::min(c.max_prefill, 64), c.max_prefill}) {
        if (T <= 0) continue;
        need((int)(qd + 2 * kvd), (int)d, T);
        need((int)d, (int)qd, T);
        need(c.vocab, (int)d, std::min(T, 64));  // LM head: decode rows or <= 64 all-logits rows
        if (E) {
            const int TP = T * (int)k;
            need((int)E, (int)d, T);
            const int act = std::min<int>((int)E, TP);
            // grouped projections: splits sized as for act experts' rows (GEMV),
            // or as the grouped GEMM splits k for prefill rows
            const bool f32w_ = c.weight_dtype == DEC_WEIGHT_F32;
            const int Sgu = (T <= 64) ? proj_splits(c, (int)(2 * F) * act, (int)d, T, true) : 1;
            const int Sd = (T <= 64) ? proj_splits(c, (int)d * act, (int)F, T, true)
                                     : (f32w_ ? 1 : gemm_grouped_splits_for((int)d, (int)F, TP, (int)E, 256));
            pf = std::max(pf, (size_t)Sgu * TP * 2 * F);
            pf = std::max(pf, (size_t)Sd * TP * d);
        } else {
            need((int)(2 * F), (int)d, T);
            need((int)d, (int)F, T);
        }
    }
    p.part_floats = pf;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    const size_t es = kv_elem_bytes(c);
    p.k = take(p.kv_layer * c.n_layers * es);
    p.v = take(p.kv_layer * c.n_layers * es);
    // one layer's K/V of a prefill chunk held back from a ring cache until the
    // chunk's attention is done (deferred commit)
    const bool ring = c.sliding_window > 0 && c.max_seq == c.sliding_window;
    p.ck = take(ring ? (size_t)c.max_prefill * kvd * es : 0);
    p.cv = take(ring ? (size_t)c.max_prefill * kvd * es : 0);
    // silu(gate) * up of the dense FFN, written by the fused gate|up GEMM
    // (prefill rows) or GEMV (up to 64 rows)
    const bool fuse_silu = !E && c.weight_dtype != DEC_WEIGHT_F32;
    const size_t s_rows = fuse_silu ? std::max<size_t>(c.max_prefill, std::min(rows, 64)) : 0;
    // the fp16 + fp8 prefill operands reuse the (hi, lo) buffers: fp16 in hi,
    // fp8 rows then [k/32][rows rounded up to 256] scales in lo
    const size_t mpad = ((size_t)c.max_prefill + 255) / 256 * 256;
    auto f8_lo = [&](size_t K) { return p.f8 ? mpad * K + (K / 32) * mpad : 0; };
    p.s_hi = take(s_rows * F * 2);
    p.s_lo = take(s_rows * F * 2);
    // prefill attention's K/V tile images (positions [0, max_seq) of one sequence)
    p.kvimg = take(c.weight_dtype == DEC_WEIGHT_F32 ? 0
                   : attn_tiles_bytes(c.max_seq, c.n_kv_heads, c.head_dim, c.kv_dtype));
    p.x = take((size_t)rows * d * 4);
    // row_norm_fused: the other residual row of one-row decode, and the down
    // projection's k-split partials apart from the partial buffer the next
    // projection writes while its blocks still read them (at most one split
    // per 64 k)
    const bool rnf = row_norm_fused(c);
    p.x2 = take(rnf ? d * 4 : 0);
    p.part2 = take(rnf ? (F + 63) / 64 * d * 4 : 0);
    const bool f32w = c.weight_dtype == DEC_WEIGHT_F32;
    p.a_hi = take(f32w ? 0 : p.act_elems * 2);
    p.a_lo = take(f32w ? 0 : std::max(p.act_elems * 2, f8_lo(d)));
    p.a_f32 = take(f32w ? p.act_elems * 4 : 0);
    p.part = take(pf * 4);
    p.q = take((size_t)rows * qd * 4);
    p.attn = take((size_t)c.max_batch * c.n_heads * MAX_ATTN_SPLITS * (hd + 2) * 4);
    p.rope = take((size_t)rows * (hd / 2) * 8);
    p.tok = take((size_t)rows * 4);
    p.pos = take((size_t)rows * 4);
    p.slot = take((size_t)rows * 4);
    p.amax = take((size_t)c.max_batch * 4);
    p.ssq = take((size_t)rows * ((d + 1023) / 1024) * 4);
    p.moe_ids = take(prow * 4);
    p.moe_w = take(prow * 4);
    p.moe_cnt = take(64 * 4);
    p.moe_off = take(65 * 4);
    p.moe_pairs = take(prow * 4);
    p.moe_inv = take(prow * 4);
    p.g_hi = take(E && !f32w ? prow * d * 2 : 0);
    p.g_lo = take(E && !f32w ? prow * d * 2 : 0);
    p.g_f32 = take(E && f32w ? prow * d * 4 : 0);
    p.f8_layer = p.f8 ? f8_weight_bytes((int)(qd + 2 * kvd), (int)d, false) + (E ? 0 : f8_weight_bytes((int)F, (int)d, true))
                      : 0;
    p.f8w = take(p.f8_layer * c.n_layers);
    p.total = off;
    return true;
}

int validate_cfg(const dec_config *c) {
    if (!c || c->struct_size != sizeof(dec_config)) return DEC_ERR_INVALID;
    if (c->n_layers <= 0 || c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
        c->ffn_dim <= 0 || c->vocab <= 0 || c->max_seq <= 0 || c->max_batch <= 0 || c->max_prefill <= 0)
        return DEC_ERR_INVALID;
    if (c->n_heads % c->n_kv_heads || c->head_dim % 2) return DEC_ERR_INVALID;
    if (!(c->rms_eps > 0) || !(c->rope_theta > 0)) return DEC_ERR_INVALID;
    if (c->n_experts < 0 || (c->n_experts > 0 && (c->top_k < 1 || c->top_k > c->n_experts))) return DEC_ERR_INVALID;
    if (c->sliding_window < 0 || (c->sliding_window > 0 && c->max_seq > c->sliding_window)) return DEC_ERR_INVALID;
    if (c->weight_dtype != DEC_WEIGHT_BF16 && c->weight_dtype != DEC_WEIGHT_F32) return DEC_ERR_INVALID;
    if (c->qkv_bias != 0 && c->qkv_bias != 1) return DEC_ERR_INVALID;
    if (c->rope_pairing != DEC_ROPE_ADJACENT && c->rope_pairing != DEC_ROPE_HALF) return DEC_ERR_INVALID;
    if (c->rope_scaling != DEC_ROPE_PLAIN && c->rope_scaling != DEC_ROPE_LLAMA3) return DEC_ERR_INVALID;
    if (c->rope_scaling == DEC_ROPE_LLAMA3 &&
        (!(c->rope_factor > 0) || !(c->rope_low_freq_factor > 0) ||
         !(c->rope_high_freq_factor > c->rope_low_freq_factor) || c->rope_orig_ctx <= 0))
        return DEC_ERR_INVALID;
    if (c->kv_dtype != DEC_KV_F32 && c->kv_dtype != DEC_KV_BF16 && c->kv_dtype != DEC_KV_F24) return DEC_ERR_INVALID;
    if (c->prefill_operands != DEC_PREFILL_BF16_PAIR && c->prefill_operands != DEC_PREFILL_F16_F8)
        return DEC_ERR_INVALID;
    if (c->prefill_operands == DEC_PREFILL_F16_F8 && c->weight_dtype != DEC_WEIGHT_BF16) return DEC_ERR_INVALID;
    // shapes the kernels are written for
    if (c->max_batch > 64) return DEC_ERR_UNSUPPORTED;
    if (c->head_dim != 16 && c->head_dim != 64 && c->head_dim != 128) return DEC_ERR_UNSUPPORTED;
    if (c->n_heads / c->n_kv_heads > 8) return DEC_ERR_UNSUPPORTED;
    if (c->n_experts > 32 || c->top_k > 8) return DEC_ERR_UNSUPPORTED;
    if (c->hidden % 4 || c->ffn_dim % 4) return DEC_ERR_UNSUPPORTED;
    if (c->weight_dtype == DEC_WEIGHT_BF16 &&
        (c->hidden % 64 || (c->n_heads * c->head_dim) % 64 || c->ffn_dim % 64))
        return DEC_ERR_UNSUPPORTED;
    return DEC_OK;
}

// ---- timing --------------------------------------------------------------------
struct Tick {
    dec_model *m;
    int cls;
    hipEvent_t e1 = nullptr, e2 = nullptr;
    Tick(dec_model *mm, int c) : m(mm), cls(c) {
        if (!m->tm[cls].on) return;
        while (m->pool.size() < 2) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return;
            m->pool.push_back(e);
        }
        e1 = m->pool.back(); m->pool.pop_back();
        e2 = m->pool.back(); m->pool.pop_back();
        hipEventRecord(e1, m->st);
    }
    void done(double bytes, double flops) {
        if (!e1) return;
        hipEventRecord(e2, m->st);
        Timing &t = m->tm[cls];
        t.pending.push_back(EvPair{e1, e2});
        t.launches++;
        t.bytes += bytes;
        t.flops += flops;
    }
    void cancel() {  // nothing was launched: give the events back
        if (!e1) return;
        m->pool.push_back(e1);
        m->pool.push_back(e2);
        e1 = e2 = nullptr;
    }
};

// Read every recorded event pair into the running totals (waits for them).
int harvest(dec_model *m) {
    int rc = DEC_OK;
    for (auto &t : m->tm) {
        for (const EvPair &p : t.pending) {
            float e = 0;
            if (hipEventSynchronize(p.e2) != hipSuccess || hipEventElapsedTime(&e, p.e1, p.e2) != hipSuccess)
                rc = DEC_ERR_DEVICE;
            else
                t.ms += e;
            m->pool.push_back(p.e1);
            m->pool.push_back(p.e2);
        }
        t.pending.clear();
    }
    return rc;
}

double kv_read_bytes(const dec_config &c, int T, const int *hpos) {
    double b = 0;
    const int es = kv_elem_bytes(c);
    for (int i = 0; i < T; i++) b += 2.0 * std::min(hpos[i] + 1, c.max_seq) * c.n_kv_heads * c.head_dim * es;
    return b;
}

int attn_splits_for(const dec_model *m, int T, const int *hpos) {
    const dec_config &c = m->c;
    int maxread = 1;
    for (int b = 0; b < T; b++) maxread = std::max(maxread, std::min(hpos[b] + 1, c.max_seq));
    return std::min(attn_decode_splits(T, c.n_kv_heads, maxread, c.head_dim, c.n_heads / c.n_kv_heads,
                                       c.kv_dtype),
                    MAX_ATTN_SPLITS);
}

// ---- one pass over all layers for T rows ------------------------------------------
struct Pass {
    int T;
    bool decode;        // true: rows are independent sequences (split-KV attention)
    int start_pos;      // prefill: first position; slot = seq
    int seq;
    bool deferred;      // prefill into a ring past its size: K/V held back until attention is done
    const int *hpos;    // host positions of the rows (for byte accounting)
    float *logits;      // destination, or nullptr (no LM head)
    int logit_row0;     // first row that gets logits
    int logit_rows;
    size_t cap_row;     // capture row offset and per-layer row count
    size_t cap_rows;
};

// Projection of T rows.  The result is a set of split partials in `part`; a
// single-split result (GEMM, fp32 weights) goes to `out` instead when given.
Partials proj(dec_model *m, const WSeg *segs, int nseg, int K, int T, const u16 *hi, const u16 *lo,
              const float *f32, int lda, float *out = nullptr, const RowNorm *rn = nullptr,
              const AttnMerge *am = nullptr) {
    int N = 0;
    for (int i = 0; i < nseg; i++) N += segs[i].rows;
    const bool gemv = T <= 64;
    float *dst = out ? out : m->part;
    if (m->wf32) {
        Tick tk(m, gemv ? DEC_K_GEMV : DEC_K_GEMM);
        launch_gemm_f32(m->st, segs, nseg, K, f32, lda, T, dst, N);
        tk.done((double)N * K * 4 + (double)T * K * 4 + (double)T * N * 4, 2.0 * T * N * K);
        return Partials{dst, 1, 0, N};
    }
    if (gemv) {
        const int S = gemv_splits(N, K, T);
        // one split (the LM head): straight into `out`, no reduction pass
        float *g = (out && S == 1) ? out : m->part;
        Tick tk(m, DEC_K_GEMV);
        launch_gemv(m->st, segs, nseg, K, hi, lo, lda, T, g, S, (size_t)T * N, N, rn, am);
        tk.done((double)N * K * 2 + (double)T * K * 4 + (double)T * N * 4, 2.0 * T * N * K);
        return Partials{g, S, (size_t)T * N, N};
    }
    // into the partial buffer, a grid with a half-empty last round, or of fewer
    // tiles than CUs, is split over k (where the buffer holds the splits)
    const size_t tn = (size_t)T * N;
    int S = out ? 1 : gemm_splits(N, K, T);
    if ((size_t)S * tn > m->pl.part_floats) S = 1;
    Tick tk(m, DEC_K_GEMM);
    launch_gemm(m->st, segs, nseg, K, hi, lo, lda, T, dst, N, S, tn);
    tk.done((double)N * K * 2 + (double)T * K * 4 + (double)T * N * 4, 2.0 * T * N * K);
    return Partials{dst, S, S > 1 ? tn : 0, N};
}

// Projection of T > 64 prefill rows on fp16 + fp8 operands (F8Act `a`, the
// converted weights `w`); split partials as proj's.
Partials proj_f8(dec_model *m, const F8Weights &w, int T, const F8Act &a) {
    const size_t tn = (size_t)T * w.N;
    int S = gemm_splits_f8(w.N, w.K, T);
    if ((size_t)S * tn > m->pl.part_floats) S = 1;
    Tick tk(m, DEC_K_GEMM);
    launch_gemm_f8(m->st, w, a.a16, a.a8, a.asc, a.mpad, a.lda, T, m->part, w.N, S, tn);
    tk.done((double)w.N * w.K * 3 + (double)T * w.K * 3 + (double)T * w.N * 4, 2.0 * T * w.N * w.K);
    return Partials{m->part, S, S > 1 ? tn : 0, w.N};
}

// Grouped expert projection over TP = T*k pair rows in expert order.
// row_pairs (decode GEMV only): grouped row r reads token row row_pairs[r] / top_k
// of (hi, lo) instead of row r.
Partials proj_grouped(dec_model *m, const WSeg *segs, int nseg, int K, int T, const u16 *hi, const u16 *lo,
                      const float *f32, int lda, const int32_t *row_pairs = nullptr) {
    const dec_config &c = m->c;
    int N = 0;
    for (int i = 0; i < nseg; i++) N += segs[i].rows;
    const int TP = T * c.top_k, E = c.n_experts;
    const size_t es = (size_t)segs[0].rows * K;
    const int act = std::min(E, TP);
    if (m->wf32) {
        launch_gemm_f32_grouped(m->st, segs, nseg, K, f32, lda, T, E, m->moe_off, es, m->part, N);
        return Partials{m->part, 1, 0, N};
    }
    if (T <= 64) {
        const int S = gemv_grouped_splits(N * act, K, T);
        Tick tk(m, DEC_K_GEMV);
        launch_gemv_grouped(m->st, segs, nseg, K, hi, lo, lda, T, E, m->moe_off, es, m->part, S, (size_t)TP * N, N,
                            row_pairs, c.top_k);
        tk.done((double)N * K * 2 * act + (double)TP * K * 4 + (double)TP * N * 4, 2.0 * TP * N * K);
        return Partials{m->part, S, (size_t)TP * N, N};
    }
    // (the k split only where the partial buffer holds it: the workspace plan
    // sized it for the projections of this shape)
    int S = gemm_grouped_splits(N, K, TP, E);
    if ((size_t)S * TP * N > m->pl.part_floats) S = 1;
    Tick tk(m, DEC_K_GEMM);
    launch_gemm_grouped(m->st, segs, nseg, K, hi, lo, lda, T, E, m->moe_off, es, m->part, N, S, (size_t)TP * N);
    tk.done((double)N * K * 2 * act + (double)TP * K * 4 + (double)TP * N * 4, 2.0 * TP * N * K);
    return Partials{m->part, S, (size_t)TP * N, N};
}

void run_pass(dec_model *m, const Pass &ps) {
    const dec_config &c = m->c;
    const int T = ps.T, d = c.hidden, hd = c.head_dim, nh = c.n_heads, nkv = c.n_kv_heads;
    const int qd = nh * hd, kvd = nkv * hd, F = c.ffn_dim;
    const float eps = (float)c.rms_eps;
    hipStream_t st = m->st;
    const bool f32w = m->wf32;
    u16 *ah = f32w ? nullptr : m->a_hi, *al = f32w ? nullptr : m->a_lo;
    float *af = f32w ? m->a_f32 : nullptr;
    auto caph = [&](int layer) -> float * {
        return m->cap_hidden ? m->cap_hidden + ((size_t)layer * ps.cap_rows + ps.cap_row) * d : nullptr;
    };
    // Prefill rows of a model converted for fp16 + fp8 operands: each producer
    // writes that form where its consumer is such a projection (q|k|v, the
    // fused gate|up), the bf16 pair otherwise (o, down, the LM head, MoE).
    const bool f8 = m->pl.f8 && !ps.decode && T > 64 && gemm_f8_ready();
    const int mpad = (T + 255) / 256 * 256;
    const F8Act fa_d{ah, (uint8_t *)al, (uint8_t *)al + (size_t)mpad * d, d, mpad};
    // the fused gate|up takes these operands where it takes the DMA kernel
    const bool f8_ffn = f8 && c.n_experts == 0 && (long)((F + 127) / 128) * ((T + 255) / 256) >= num_cus();
    // One decode row (row_norm_fused): the residual + RMSNorm before gate|up,
    // before q|k|v (after layer 0) and before the LM head is formed in those
    // projections' own blocks instead of a kernel of its own; the residual row
    // alternates between x and x2.
    const bool rnf = ps.decode && T == 1 && ps.logits && ps.logit_rows == 1 && m->s_hi && row_norm_fused(c);
    float *xc = m->x, *xn = m->x2;
    Partials pend{nullptr, 0, 0, 0};   // the down partials the next projection's prologue adds

    launch_residual_norm(st, RN_EMBED, T, d, m->x, m->tok, m->embed, f32w, Partials{nullptr, 0, 0, 0},
                         Partials{nullptr, 0, 0, 0}, nullptr, nullptr, 0, m->L[0].attn_norm, eps, ah, al, af, caph(0),
                         m->ssq, f8 ? &fa_d : nullptr);
    launch_rope_table(st, m->pos, T, hd, c.rope_theta, c.rope_scaling, c.rope_factor, c.rope_low_freq_factor,
                      c.rope_high_freq_factor, c.rope_orig_ctx, m->rope);

    for (int l = 0; l < c.n_layers; l++) {
        const dec_layer_weights &w = m->L[l];
        char *kc = m->kc + (size_t)l * m->pl.kv_layer * m->kv_es;
        char *vc = m->vc + (size_t)l * m->pl.kv_layer * m->kv_es;
        const int kvk = c.kv_dtype;   // DEC_KV_* values are the kernels' cache formats
        // q | k | v
        WSeg qkv[3] = {{w.wq, qd}, {w.wk, kvd}, {w.wv, kvd}};
        Partials pq;
        if (rnf && pend.p) {
            const RowNorm rn{xc, xn, caph(l), pend, w.attn_norm, eps, d};
            pq = proj(m, qkv, 3, d, T, nullptr, nullptr, nullptr, d, nullptr, &rn);
            std::swap(xc, xn);
        } else {
            pq = f8 ? proj_f8(m, m->f8w[l].qkv, T, fa_d) : proj(m, qkv, 3, d, T, ah, al, af, d);
        }
        // attention -> a (row stride qd)
        // one decode row in 2-32 attention splits: the output projection's
        // blocks merge the splits of their k range (no merge kernel; Mistral-7B
        // B = 1 3.604 -> 3.542 and 3.617 -> 3.595 ms a step on two boxes,
        // Qwen2.5-0.5B 1.166 -> 1.108).  64 splits (the bf16 cache's MFMA
        // attention at 4096 positions) measured 3.510 -> 3.598: the merge
        // kernel stays there.
        bool am_o = false;
        int am_s = 0;
        if (ps.decode) {
            // RoPE and the new K/V rows are formed inside the attention kernel
            const int S = attn_splits_for(m, T, ps.hpos);
            am_o = T == 1 && !f32w && S > 1 && S <= 32;
            const RopeArgs ra{pq, c.qkv_bias ? w.bq : nullptr, c.qkv_bias ? w.bk : nullptr,
                              c.qkv_bias ? w.bv : nullptr, m->rope, c.rope_pairing, m->ring};
            Tick tk(m, DEC_K_ATTN_DECODE);
            launch_attn_decode(st, T, ra, kc, vc, kvk, m->pos, m->slot, nh, nkv, hd, c.max_seq, S, m->attn, ah, al,
                               af, !am_o);
            am_s = S;
            tk.done(kv_read_bytes(c, T, ps.hpos) + 2.0 * T * qd * 4, 0);
        } else {
            // K/V into the layer cache, or held in the chunk buffers (deferred commit)
            launch_rope_kv(st, T, pq, c.qkv_bias ? w.bq : nullptr, c.qkv_bias ? w.bk : nullptr,
                           c.qkv_bias ? w.bv : nullptr, m->rope, m->pos, m->slot, nh, nkv, hd, c.rope_pairing, m->q,
                           ps.deferred ? (void *)m->ck : (void *)kc, ps.deferred ? (void *)m->cv : (void *)vc,
                           c.max_seq, m->ring, kvk, ps.deferred);
            // keys per query: positions [p - window + 1, p] (window 0: [0, p])
            const int W = c.sliding_window;
            double flops = 0, keys = 0;
            for (int t = 0; t < T; t++) {
                const double p = ps.start_pos + t;
                flops += 4.0 * hd * nh * (W ? std::min<double>(p + 1, W) : p + 1);
            }
            keys = W ? std::min<double>(ps.start_pos + T, (double)W + T) : ps.start_pos + T;
            Tick tk(m, DEC_K_ATTN_PREFILL);
            // history is read through ring slots only when the call reaches past
            // max_seq (the deferred case); below that, slot == position
            if (ps.deferred || !m->kvimg ||
                !launch_attn_prefill_tiles(st, T, ps.start_pos, ps.seq, m->q, kc, vc, kvk, nh, nkv, hd, c.max_seq,
                                           m->kvimg, m->part, m->pl.part_floats, ah, al, af))
                launch_attn_prefill(st, T, ps.start_pos, ps.seq, m->q, kc, vc, kvk, nh, nkv, hd, c.max_seq, W,
                                    ps.deferred, ps.deferred ? m->ck : nullptr, ps.deferred ? m->cv : nullptr, ah,
                                    al, af);
            tk.done(keys * kvd * 2 * m->kv_es + 2.0 * T * qd * 4, flops);
            if (ps.deferred)
                launch_commit_chunk(st, m->ck, m->cv, T, ps.start_pos, ps.seq, nkv, hd, m->kv_es, c.max_seq, kc, vc);
        }
        // output projection, residual, FFN norm
        WSeg wo[1] = {{w.wo, d}};
        const AttnMerge am{m->attn, hd, am_s};
        Partials po = proj(m, wo, 1, qd, T, ah, al, af, qd, nullptr, nullptr, am_o ? &am : nullptr);
        // one decode row: the fused gate|up forms this residual + norm itself
        bool rn_gu = false;
        if (rnf) {
            const RowNorm rn{xc, xn, nullptr, po, w.ffn_norm, eps, d};
            Tick tk(m, DEC_K_GEMV);
            rn_gu = launch_gemv_silu(st, w.w_gate, w.w_up, F, d, nullptr, nullptr, d, T, m->s_hi, m->s_lo, F, &rn);
            if (rn_gu) {
                tk.done(2.0 * F * d * 2 + (double)T * d * 4 + (double)T * F * 4, 2.0 * T * 2 * F * d);
                std::swap(xc, xn);
            } else {
                tk.cancel();
            }
        }
        if (!rn_gu)
            launch_residual_norm(st, RN_ADD, T, d, xc, nullptr, nullptr, 0, po, Partials{nullptr, 0, 0, 0}, nullptr,
                                 nullptr, 0, w.ffn_norm, eps, ah, al, af, nullptr, m->ssq, f8_ffn ? &fa_d : nullptr);
        const float *next_gain = (l + 1 < c.n_layers) ? m->L[l + 1].attn_norm : m->out_norm;
        if (c.n_experts == 0) {
            WSeg gu[2] = {{w.w_gate, F}, {w.w_up, F}};
            // a large prefill takes the gate|up GEMM with silu(gate) * up in its epilogue
            bool fused = rn_gu;
            if (fused) {
                // (formed above with the residual + norm)
            } else if (f8_ffn) {
                Tick tk(m, DEC_K_GEMM);
                fused = launch_gemm_f8_silu(st, m->f8w[l].gu, fa_d.a16, fa_d.a8, fa_d.asc, mpad, d, T, m->s_hi,
                                            m->s_lo, F);
                if (fused) tk.done(2.0 * F * d * 3 + (double)T * d * 3 + (double)T * F * 4, 2.0 * T * 2 * F * d);
                else tk.cancel();
            } else if (!f32w && T > 64 && m->s_hi) {
                Tick tk(m, DEC_K_GEMM);
                fused = launch_gemm_silu(st, w.w_gate, w.w_up, F, d, ah, al, d, T, m->s_hi, m->s_lo, F);
                if (fused) tk.done(2.0 * F * d * 2 + (double)T * d * 4 + (double)T * F * 4, 2.0 * T * 2 * F * d);
                else tk.cancel();
            } else if (!f32w && T <= 64 && m->s_hi && (T <= 32 || gemv_splits(2 * F, d, T) == 1)) {
                // decode rows: one k split with silu(gate) * up in the epilogue,
                // its 8-feature tiles spread over the CUs up to 32 rows; above,
                // only where the unfused projection would take one split too
                // (Qwen2.5-0.5B at B = 64 ran 2.55 ms/step fused, 2.42 unfused)
                Tick tk(m, DEC_K_GEMV);
                fused = launch_gemv_silu(st, w.w_gate, w.w_up, F, d, ah, al, d, T, m->s_hi, m->s_lo, F);
                if (fused) tk.done(2.0 * F * d * 2 + (double)T * d * 4 + (double)T * F * 4, 2.0 * T * 2 * F * d);
                else tk.cancel();
            }
            if (!fused) {
                Partials pg = proj(m, gu, 2, d, T, ah, al, af, d);
                launch_silu_mul(st, T, F, pg, ah, al, af);
            }
            WSeg wd[1] = {{w.w_down, d}};
            if (rn_gu) {
                // into the second partial buffer: the next q|k|v (or the LM
                // head) adds these partials in its prologue while it writes
                // its own into the first
                const int S = gemv_splits(d, F, 1);
                Tick tk(m, DEC_K_GEMV);
                launch_gemv(st, wd, 1, F, m->s_hi, m->s_lo, F, 1, m->part2, S, (size_t)d, d);
                tk.done((double)d * F * 2 + (double)F * 4 + (double)d * 4, 2.0 * d * F);
                pend = Partials{m->part2, S, (size_t)d, d};
            } else {
                Partials pd = proj(m, wd, 1, F, T, fused ? m->s_hi : ah, fused ? m->s_lo : al, af, F);
                launch_residual_norm(st, RN_ADD, T, d, xc, nullptr, nullptr, 0, pd, Partials{nullptr, 0, 0, 0},
                                     nullptr, nullptr, 0, next_gain, eps, ah, al, af, caph(l + 1), m->ssq,
                                     f8 && l + 1 < c.n_layers ? &fa_d : nullptr);
                pend = Partials{nullptr, 0, 0, 0};
            }
        } else {
            const int E = c.n_experts, k = c.top_k, TP = T * k;
            // router logits: the GEMV for decode rows and fp32 weights; prefill
            // rows form them inside the top-k kernel
            const bool in_kernel = !f32w && T > 64;
            Partials pr{nullptr, 0, 0, 0};
            if (!in_kernel) {
                WSeg wr[1] = {{w.router, E}};
                pr = proj(m, wr, 1, d, T, ah, al, af, d);
            }
            launch_moe_route(st, T, E, k, pr, in_kernel ? (const u16 *)w.router : nullptr, ah, al, d, d,
                             m->moe_ids, m->moe_w,
                             m->cap_router ? m->cap_router + ((size_t)l * ps.cap_rows + ps.cap_row) * E : nullptr,
                             m->cap_ids ? m->cap_ids + ((size_t)l * ps.cap_rows + ps.cap_row) * k : nullptr,
                             m->moe_cnt, m->moe_off, m->moe_pairs, m->moe_inv);
            // decode rows (bf16 weights): the grouped GEMV reads each grouped row's
            // token row of (ah, al) through the pair map; otherwise the rows are
            // gathered into expert order first
            const bool mapped = !f32w && T <= 64;
            if (!mapped)
                launch_moe_gather(st, T, k, d, m->moe_pairs, ah, al, af, f32w ? nullptr : m->g_hi,
                                  f32w ? nullptr : m->g_lo, f32w ? m->g_f32 : nullptr);
            WSeg gu[2] = {{w.w_gate, F}, {w.w_up, F}};
            // prefill rows: the grouped gate|up GEMM writes silu(gate) * up itself
            bool fused = false;
            if (!f32w && T > 64) {
                Tick tk(m, DEC_K_GEMM);
                const int act = std::min(E, TP);
                fused = launch_gemm_grouped_silu(st, w.w_gate, w.w_up, F, d, m->g_hi, m->g_lo, d, T, E, m->moe_off,
                                                 (size_t)F * d, ah, al, F);
                if (fused) tk.done(2.0 * F * d * 2 * act + (double)TP * d * 4 + (double)TP * F * 4, 2.0 * TP * 2 * F * d);
                else tk.cancel();
            }
            if (!fused) {
                Partials pg = mapped ? proj_grouped(m, gu, 2, d, T, ah, al, nullptr, d, m->moe_pairs)
                                     : proj_grouped(m, gu, 2, d, T, m->g_hi, m->g_lo, m->g_f32, d);
                launch_silu_mul(st, TP, F, pg, ah, al, af);
            }
            WSeg wd[1] = {{w.w_down, d}};
            Partials pd = proj_grouped(m, wd, 1, F, T, ah, al, af, F);
            // the residual reads each token's expert outputs at their grouped rows
            launch_residual_norm(st, RN_ADD, T, d, xc, nullptr, nullptr, 0, Partials{nullptr, 0, 0, 0}, pd,
                                 m->moe_inv, m->moe_w, k, next_gain, eps, ah, al, af, caph(l + 1), m->ssq,
                                 f8 && l + 1 < c.n_layers ? &fa_d : nullptr);
        }
    }
    // LM head on the rows that need logits (a holds the final-norm rows)
    if (ps.logits) {
        const void *head = c.tied_embedding ? m->embed : m->lm_head;
        WSeg hs[1] = {{head, c.vocab}};
        const size_t ro = (size_t)ps.logit_row0 * d;
        Partials pl;
        if (rnf && pend.p) {
            const RowNorm rn{xc, xn, caph(c.n_layers), pend, m->out_norm, eps, d};
            pl = proj(m, hs, 1, d, ps.logit_rows, nullptr, nullptr, nullptr, d, ps.logits, &rn);
        } else {
            pl = proj(m, hs, 1, d, ps.logit_rows, ah ? ah + ro : nullptr, al ? al + ro : nullptr,
                      af ? af + ro : nullptr, d, ps.logits);
        }
        if (pl.p != ps.logits) launch_reduce_splits(st, pl, ps.logit_rows, c.vocab, ps.logits, c.vocab);
    }
}

int check_device(hipError_t e) { return e == hipSuccess ? DEC_OK : DEC_ERR_DEVICE; }

}  // namespace

namespace {

// Lazily made: a non-blocking stream of default priority for decode graphs and
// the two fence events that order it with the caller's stream.
bool graph_stream(dec_model *m) {
    if (m->cs) return true;
    if (hipStreamCreateWithFlags(&m->cs, hipStreamNonBlocking) != hipSuccess) { m->cs = nullptr; return false; }
    if (hipEventCreateWithFlags(&m->fence_in, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&m->fence_out, hipEventDisableTiming) != hipSuccess)
        return false;
    return true;
}

void destroy_graph(GraphEntry &g) {
    if (g.exec) hipGraphExecDestroy(g.exec);
    if (g.graph) hipGraphDestroy(g.graph);
    g.exec = nullptr;
    g.graph = nullptr;
}

unsigned timing_mask(const dec_model *m) {
    unsigned k = 0;
    for (int i = 0; i < DEC_K_COUNT; i++)
        if (m->tm[i].on) k |= 1u << i;
    return k;
}

// Launch a captured step; its first node (the row setup) takes this step's rows,
// token source and history row.
int replay(dec_model *m, GraphEntry &g, const RowArgs &ra, const int32_t *src, int32_t *hist) {
    g.used = ++m->graph_clock;
    int B = g.B;
    int32_t *tok = m->tok, *ps = m->pos, *sl = m->slot;
    void *args[] = {(void *)&ra, (void *)&B, (void *)&src, (void *)&hist, (void *)&tok, (void *)&ps, (void *)&sl};
    hipKernelNodeParams kp = g.kp;
    kp.kernelParams = args;
    kp.extra = nullptr;
    if (hipGraphExecKernelNodeSetParams(g.exec, g.root, &kp) != hipSuccess) return DEC_ERR_DEVICE;
    if (hipEventRecord(m->fence_in, m->st) != hipSuccess || hipStreamWaitEvent(m->cs, m->fence_in, 0) != hipSuccess ||
        hipGraphLaunch(g.exec, m->cs) != hipSuccess || hipEventRecord(m->fence_out, m->cs) != hipSuccess ||
        hipStreamWaitEvent(m->st, m->fence_out, 0) != hipSuccess)
        return DEC_ERR_DEVICE;
    return DEC_OK;
}

// Capture one decode step into a graph (returns null if capture is not possible).
// A greedy step ends with the argmax of its logits into amax.
GraphEntry *capture(dec_model *m, const RowArgs &ra, int B, int S, const int *pos, float *logits, bool greedy) {
    if (!graph_stream(m)) return nullptr;
    GraphEntry g;
    g.B = B;
    g.S = S;
    g.greedy = greedy;
    g.logits = logits;
    hipStream_t user = m->st;
    if (hipEventRecord(m->fence_in, user) != hipSuccess || hipStreamWaitEvent(m->cs, m->fence_in, 0) != hipSuccess)
        return nullptr;
    if (hipStreamBeginCapture(m->cs, hipStreamCaptureModeThreadLocal) != hipSuccess) return nullptr;
    m->st = m->cs;
    launch_set_rows(m->st, ra, B, nullptr, nullptr, m->tok, m->pos, m->slot);
    Pass ps{};
    ps.T = B;
    ps.decode = true;
    ps.hpos = pos;
    ps.logits = logits;
    ps.logit_row0 = 0;
    ps.logit_rows = B;
    ps.cap_row = 0;
    ps.cap_rows = B;
    run_pass(m, ps);
    if (greedy) launch_argmax(m->st, logits, B, m->c.vocab, m->amax);
    m->st = user;
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(m->cs, &graph);
    (void)hipGetLastError();
    if (ec != hipSuccess || !graph) { destroy_graph(g); return nullptr; }
    g.graph = graph;
    size_t n = 0;
    if (hipGraphGetRootNodes(graph, nullptr, &n) != hipSuccess || n != 1) { destroy_graph(g); return nullptr; }
    if (hipGraphGetRootNodes(graph, &g.root, &n) != hipSuccess ||
        hipGraphKernelNodeGetParams(g.root, &g.kp) != hipSuccess ||
        hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0) != hipSuccess) {
        destroy_graph(g);
        return nullptr;
    }
    if (m->graphs.size() >= MAX_GRAPHS) {
        // evict the least recently replayed graph (after the graph stream drains)
        size_t lru = 0;
        for (size_t i = 1; i < m->graphs.size(); i++)
            if (m->graphs[i].used < m->graphs[lru].used) lru = i;
        if (hipStreamSynchronize(m->cs) != hipSuccess) { destroy_graph(g); return nullptr; }
        destroy_graph(m->graphs[lru]);
        m->graphs.erase(m->graphs.begin() + (long)lru);
    }
    m->graphs.push_back(g);
    return &m->graphs.back();
}

}  // namespace

namespace {

// The workspace of handles made by dec_create_noalloc: a file-scope device
// array, one copy per GPU the library runs on, held until the process ends.
// Host code never passes `scratch` itself to a kernel or a copy (in host code
// the name is a stand-in, not a device address): it takes each device's
// address once from hipGetSymbolAddress and uses that.
__device__ __align__(256) unsigned char scratch[DEC_NOALLOC_WORKSPACE_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};   // per device: its copy's address
bool g_scratch_busy[MAX_DEVICES] = {};   // per device: a live handle uses it

}  // namespace

extern "C" {

size_t dec_workspace_bytes(const dec_config *cfg) {
    if (validate_cfg(cfg) != DEC_OK) return 0;
    Plan p;
    plan(*cfg, p);
    return p.total;
}

int dec_create(const dec_config *cfg, const dec_weights *w, void *workspace, size_t ws_bytes, void *hip_stream,
               dec_handle *out) {
    if (!out) return DEC_ERR_INVALID;
    *out = nullptr;
    int rc = validate_cfg(cfg);
    if (rc) return rc;
    if (!w || w->struct_size != sizeof(dec_weights) || !w->embed || !w->out_norm || !w->layers)
        return DEC_ERR_INVALID;
    if (!cfg->tied_embedding && !w->lm_head) return DEC_ERR_INVALID;
    // every weight is read in 16-byte words
    auto misaligned = [](const void *q) { return q && ((uintptr_t)q & 15); };
    if (misaligned(w->embed) || misaligned(w->out_norm) || misaligned(w->lm_head)) return DEC_ERR_INVALID;
    for (int l = 0; l < cfg->n_layers; l++) {
        const dec_layer_weights &L = w->layers[l];
        if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.ffn_norm || !L.w_gate || !L.w_up || !L.w_down)
            return DEC_ERR_INVALID;
        if (cfg->qkv_bias && (!L.bq || !L.bk || !L.bv)) return DEC_ERR_INVALID;
        if (cfg->n_experts && !L.router) return DEC_ERR_INVALID;
        for (const void *q : {(const void *)L.attn_norm, L.wq, L.wk, L.wv, (const void *)L.bq, (const void *)L.bk,
                              (const void *)L.bv, L.wo, (const void *)L.ffn_norm, L.w_gate, L.w_up, L.w_down,
                              L.router})
            if (misaligned(q)) return DEC_ERR_INVALID;
    }
    Plan p;
    plan(*cfg, p);
    if (!workspace || ((uintptr_t)workspace & 255)) return DEC_ERR_INVALID;
    if (ws_bytes < p.total) return DEC_ERR_NOMEM;
    dec_model *m = new (std::nothrow) dec_model();
    if (!m) return DEC_ERR_NOMEM;
    m->c = *cfg;
    m->L.assign(w->layers, w->layers + cfg->n_layers);
    m->embed = w->embed;
    m->out_norm = w->out_norm;
    m->lm_head = cfg->tied_embedding ? w->embed : w->lm_head;
    m->st = (hipStream_t)hip_stream;
    m->ws = (char *)workspace;
    m->pl = p;
    char *b = m->ws;
    m->kc = b + p.k;
    m->vc = b + p.v;
    m->ck = b + p.ck;
    m->cv = b + p.cv;
    m->kvimg = p.kvimg < p.x ? (void *)(b + p.kvimg) : nullptr;
    m->s_hi = p.s_hi < p.s_lo ? (u16 *)(b + p.s_hi) : nullptr;
    m->s_lo = m->s_hi ? (u16 *)(b + p.s_lo) : nullptr;
    m->kv_es = (int)kv_elem_bytes(*cfg);
    m->x = (float *)(b + p.x);
    m->x2 = (float *)(b + p.x2);
    m->part2 = (float *)(b + p.part2);
    m->a_hi = (u16 *)(b + p.a_hi);
    m->a_lo = (u16 *)(b + p.a_lo);
    m->a_f32 = (float *)(b + p.a_f32);
    m->part = (float *)(b + p.part);
    m->q = (float *)(b + p.q);
    m->attn = (float *)(b + p.attn);
    m->rope = (float2 *)(b + p.rope);
    m->tok = (int32_t *)(b + p.tok);
    m->pos = (int32_t *)(b + p.pos);
    m->slot = (int32_t *)(b + p.slot);
    m->amax = (int32_t *)(b + p.amax);
    m->ssq = (float *)(b + p.ssq);
    m->moe_ids = (int32_t *)(b + p.moe_ids);
    m->moe_w = (float *)(b + p.moe_w);
    m->moe_cnt = (int32_t *)(b + p.moe_cnt);
    m->moe_off = (int32_t *)(b + p.moe_off);
    m->moe_pairs = (int32_t *)(b + p.moe_pairs);
    m->moe_inv = (int32_t *)(b + p.moe_inv);
    m->g_hi = (u16 *)(b + p.g_hi);
    m->g_lo = (u16 *)(b + p.g_lo);
    m->g_f32 = (float *)(b + p.g_f32);
    m->len.assign(cfg->max_batch, 0);
    m->wf32 = cfg->weight_dtype == DEC_WEIGHT_F32;
    // a ring of max_seq == window slots; a window longer than max_seq never
    // wraps (positions are capped at max_seq like a full-causal cache)
    m->ring = cfg->sliding_window > 0 && cfg->max_seq == cfg->sliding_window;
    if (p.f8) {
        // the prefill projections' fp16 + fp8 weights, converted on the stream
        const int d = cfg->hidden, qd = cfg->n_heads * cfg->head_dim, kvd = cfg->n_kv_heads * cfg->head_dim;
        const int F = cfg->ffn_dim;
        m->f8w.assign(cfg->n_layers, dec_model::F8Layer{});
        for (int l = 0; l < cfg->n_layers; l++) {
            const dec_layer_weights &L = m->L[l];
            dec_model::F8Layer &f = m->f8w[l];
            char *at = b + p.f8w + (size_t)l * p.f8_layer;
            f.qkv = f8_weights_at(at, qd + 2 * kvd, d, false);
            at += f8_weight_bytes(qd + 2 * kvd, d, false);
            WSeg qkv[3] = {{L.wq, qd}, {L.wk, kvd}, {L.wv, kvd}};
            launch_convert_f8(m->st, qkv, 3, d, false, f.qkv);
            if (!cfg->n_experts) {
                f.gu = f8_weights_at(at, F, d, true);
                WSeg gu[2] = {{L.w_gate, F}, {L.w_up, F}};
                launch_convert_f8(m->st, gu, 2, d, true, f.gu);
            }
        }
        if (hipGetLastError() != hipSuccess) {
            delete m;
            return DEC_ERR_DEVICE;
        }
    }
    *out = m;
    return DEC_OK;
}

int dec_graph_count(dec_handle h) { return h ? (int)h->graphs.size() : DEC_ERR_INVALID; }

void dec_destroy(dec_handle h) {
    if (!h) return;
    if (h->cs) hipStreamSynchronize(h->cs);
    hipStreamSynchronize(h->st);
    harvest(h);
    for (auto &g : h->graphs) destroy_graph(g);
    for (hipEvent_t e : h->pool) hipEventDestroy(e);
    if (h->fence_in) hipEventDestroy(h->fence_in);
    if (h->fence_out) hipEventDestroy(h->fence_out);
    if (h->cs) hipStreamDestroy(h->cs);
    if (h->static_dev >= 0) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        g_scratch_busy[h->static_dev] = false;
    }
    delete h;
}

int dec_create_noalloc(const dec_config *cfg, const dec_weights *w, void *hip_stream, dec_handle *out) {
    if (!out) return DEC_ERR_INVALID;
    *out = nullptr;
    const int vc = validate_cfg(cfg);
    if (vc != DEC_OK) return vc;
    Plan p;
    plan(*cfg, p);
    if (p.total > DEC_NOALLOC_WORKSPACE_BYTES) return DEC_ERR_NOMEM;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return DEC_ERR_DEVICE;
    if (hip_stream) {  // the stream's kernels run on its device: it must be the current one
        int sdev = -1;
        if (hipStreamGetDevice((hipStream_t)hip_stream, &sdev) != hipSuccess) return DEC_ERR_DEVICE;
        if (sdev != dev) return DEC_ERR_INVALID;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DEC_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    if (g_scratch_busy[dev]) return DEC_ERR_INVALID;  // one live handle per device
    const int rc = dec_create(cfg, w, g_scratch_ptr[dev], DEC_NOALLOC_WORKSPACE_BYTES, hip_stream, out);
    if (rc == DEC_OK) {
        g_scratch_busy[dev] = true;
        (*out)->static_dev = dev;
    }
    return rc;
}

int dec_prefill(dec_handle h, int seq, const int32_t *tokens, int n, int start_pos, float *logits) {
    return dec_prefill_ex(h, seq, tokens, n, start_pos, logits, 0);
}

int dec_prefill_ex(dec_handle h, int seq, const int32_t *tokens, int n, int start_pos, float *logits,
                   int all_logits) {
    if (!h || !tokens || !logits || (all_logits != 0 && all_logits != 1)) return DEC_ERR_INVALID;
    const dec_config &c = h->c;
    if (seq < 0 || seq >= c.max_batch || n <= 0) return DEC_ERR_INVALID;
    if (n > c.max_prefill) return DEC_ERR_RANGE;
    for (int i = 0; i < n; i++)
        if (tokens[i] < 0 || tokens[i] >= c.vocab) return DEC_ERR_INVALID;
    if (start_pos != h->len[seq]) return DEC_ERR_INVALID;
    if (!h->ring && (long)start_pos + n > (long)c.max_seq) return DEC_ERR_RANGE;
    if ((long)start_pos + n > 0x7FFFFFFFL) return DEC_ERR_RANGE;
    if (timing_mask(h) && harvest(h) != DEC_OK) return DEC_ERR_DEVICE;

    if (hipMemcpyAsync(h->tok, tokens, sizeof(int32_t) * n, hipMemcpyHostToDevice, h->st) != hipSuccess)
        return DEC_ERR_DEVICE;
    launch_set_seq_rows(h->st, n, start_pos, seq, h->pos, h->slot);
    Pass ps{};
    ps.T = n;
    ps.decode = false;
    ps.start_pos = start_pos;
    ps.seq = seq;
    // positions past the ring's size would overwrite slots the chunk's own
    // earlier queries still read: hold the chunk's K/V back until its
    // attention is done, then commit (zLLM "The Algorithm Layer", section 5:
    // AppendPrefill appends a span after existing history)
    ps.deferred = h->ring && (long)start_pos + n > (long)c.max_seq;
    ps.hpos = nullptr;
    ps.logits = logits;
    ps.logit_row0 = all_logits ? 0 : n - 1;
    ps.logit_rows = all_logits ? n : 1;
    ps.cap_row = 0;
    ps.cap_rows = n;
    run_pass(h, ps);
    if (hipGetLastError() != hipSuccess) return DEC_ERR_DEVICE;
    h->len[seq] = start_pos + n;
    return DEC_OK;
}

int dec_decode(dec_handle h, int B, const int32_t *tokens, const int32_t *pos, float *logits) {
    if (!h || !tokens || !pos || !logits) return DEC_ERR_INVALID;
    const dec_config &c = h->c;
    if (B <= 0 || B > c.max_batch) return DEC_ERR_INVALID;
    for (int b = 0; b < B; b++) {
        if (tokens[b] < 0 || tokens[b] >= c.vocab) return DEC_ERR_INVALID;
        if (pos[b] != h->len[b]) return DEC_ERR_INVALID;
        if (!h->ring && pos[b] + 1 > c.max_seq) return DEC_ERR_RANGE;
        if (pos[b] == 0x7FFFFFFF) return DEC_ERR_RANGE;
    }
    if (timing_mask(h) && harvest(h) != DEC_OK) return DEC_ERR_DEVICE;
    RowArgs ra;
    for (int b = 0; b < B; b++) {
        ra.tok[b] = tokens[b];
        ra.pos[b] = pos[b];
        ra.slot[b] = b;
    }
    if (!h->cap_hidden && !h->cap_ids && !h->cap_router && !timing_mask(h)) {
        // replay (or capture, the second time this shape is seen) one graph per step
        const int S = attn_splits_for(h, B, pos);
        GraphEntry *g = nullptr;
        for (auto &e : h->graphs)
            if (e.B == B && e.S == S && e.logits == logits && !e.greedy) g = &e;
        if (!g) {
            const std::vector<long long> key = {B, S, (long long)(uintptr_t)logits};
            int *count = nullptr;
            for (auto &kv : h->seen)
                if (kv.first == key) count = &kv.second;
            if (!count) {
                h->seen.push_back({key, 1});
            } else if (*count == 1) {
                g = capture(h, ra, B, S, pos, logits, false);
                *count = g ? 2 : 3;  // 3: capture failed, stay eager for this shape
            }
        }
        if (g) {
            if (replay(h, *g, ra, nullptr, nullptr) != DEC_OK) return DEC_ERR_DEVICE;
            for (int b = 0; b < B; b++) h->len[b] = pos[b] + 1;
            return DEC_OK;
        }
    }
    launch_set_rows(h->st, ra, B, nullptr, nullptr, h->tok, h->pos, h->slot);
    Pass ps{};
    ps.T = B;
    ps.decode = true;
    ps.hpos = pos;
    ps.logits = logits;
    ps.logit_row0 = 0;
    ps.logit_rows = B;
    ps.cap_row = 0;
    ps.cap_rows = B;
    run_pass(h, ps);
    if (hipGetLastError() != hipSuccess) return DEC_ERR_DEVICE;
    for (int b = 0; b < B; b++) h->len[b] = pos[b] + 1;
    return DEC_OK;
}

int dec_decode_greedy(dec_handle h, int B, const int32_t *tokens, int steps, int32_t *tokens_out, float *logits) {
    if (!h || !tokens || !tokens_out || !logits) return DEC_ERR_INVALID;
    const dec_config &c = h->c;
    if (B <= 0 || B > c.max_batch || steps <= 0) return DEC_ERR_INVALID;
    for (int b = 0; b < B; b++) {
        if (tokens[b] < 0 || tokens[b] >= c.vocab) return DEC_ERR_INVALID;
        if (!h->ring && (long)h->len[b] + steps > (long)c.max_seq) return DEC_ERR_RANGE;
        if ((long)h->len[b] + steps > 0x7FFFFFFFL) return DEC_ERR_RANGE;
    }
    if (timing_mask(h) && harvest(h) != DEC_OK) return DEC_ERR_DEVICE;
    const bool graphs = !h->cap_hidden && !h->cap_ids && !h->cap_router && !timing_mask(h);
    int hpos[64];
    for (int s = 0; s < steps; s++) {
        RowArgs ra;
        for (int b = 0; b < B; b++) {
            ra.tok[b] = tokens[b];  // read by the first step only
            ra.pos[b] = hpos[b] = h->len[b] + s;
            ra.slot[b] = b;
        }
        // step s > 0 embeds the previous step's choice and appends it to the output
        const int32_t *src = s ? h->amax : nullptr;
        int32_t *hist = s ? tokens_out + (size_t)(s - 1) * B : nullptr;
        GraphEntry *g = nullptr;
        if (graphs) {
            const int S = attn_splits_for(h, B, hpos);
            for (auto &e : h->graphs)
                if (e.B == B && e.S == S && e.logits == logits && e.greedy) g = &e;
            if (!g && steps - s >= 2) {
                // a shape whose capture failed once stays eager (no retry per step)
                const std::vector<long long> key = {B, S, (long long)(uintptr_t)logits, -1};
                bool failed = false;
                for (auto &kv : h->seen)
                    if (kv.first == key) failed = true;
                if (!failed) {
                    g = capture(h, ra, B, S, hpos, logits, true);
                    if (!g) h->seen.push_back({key, 3});
                }
            }
        }
        if (g) {
            if (replay(h, *g, ra, src, hist) != DEC_OK) return DEC_ERR_DEVICE;
            continue;
        }
        launch_set_rows(h->st, ra, B, src, hist, h->tok, h->pos, h->slot);
        Pass ps{};
        ps.T = B;
        ps.decode = true;
        ps.hpos = hpos;
        ps.logits = logits;
        ps.logit_row0 = 0;
        ps.logit_rows = B;
        ps.cap_row = 0;
        ps.cap_rows = B;
        run_pass(h, ps);
        launch_argmax(h->st, logits, B, c.vocab, h->amax);
    }
    launch_copy_ids(h->st, h->amax, B, tokens_out + (size_t)(steps - 1) * B);
    if (hipGetLastError() != hipSuccess) return DEC_ERR_DEVICE;
    for (int b = 0; b < B; b++) h->len[b] += steps;
    return DEC_OK;
}

int dec_kv_reset(dec_handle h, int seq) {
    if (!h || seq < -1 || seq >= h->c.max_batch) return DEC_ERR_INVALID;
    for (int s = 0; s < h->c.max_batch; s++)
        if (seq == -1 || s == seq) h->len[s] = 0;
    return DEC_OK;
}

int dec_kv_length(dec_handle h, int seq) {
    if (!h || seq < 0 || seq >= h->c.max_batch) return DEC_ERR_INVALID;
    return h->len[seq];
}

int dec_greedy(dec_handle h, const float *logits, int B, int32_t *tokens_out) {
    if (!h || !logits || !tokens_out || B <= 0 || B > h->c.max_batch) return DEC_ERR_INVALID;
    launch_argmax(h->st, logits, B, h->c.vocab, h->amax);
    if (hipMemcpyAsync(tokens_out, h->amax, sizeof(int32_t) * B, hipMemcpyDeviceToHost, h->st) != hipSuccess)
        return DEC_ERR_DEVICE;
    return check_device(hipStreamSynchronize(h->st));
}

int dec_sync(dec_handle h) {
    if (!h) return DEC_ERR_INVALID;
    return check_device(hipStreamSynchronize(h->st));
}

int dec_set_capture(dec_handle h, float *hidden, int32_t *expert_ids, float *router) {
    if (!h) return DEC_ERR_INVALID;
    h->cap_hidden = hidden;
    h->cap_ids = expert_ids;
    h->cap_router = router;
    return DEC_OK;
}

int dec_timing_enable(dec_handle h, int kernel_class, int on) {
    if (!h || kernel_class < 0 || kernel_class >= DEC_K_COUNT) return DEC_ERR_INVALID;
    if (hipStreamSynchronize(h->st) != hipSuccess) return DEC_ERR_DEVICE;
    harvest(h);
    Timing &t = h->tm[kernel_class];
    t.on = on != 0;
    t.ms = 0;
    t.launches = 0;
    t.bytes = t.flops = 0;
    return DEC_OK;
}

int dec_timing_read(dec_handle h, int kernel_class, double *total_ms, int64_t *launches, double *bytes,
                    double *flops) {
    if (!h || kernel_class < 0 || kernel_class >= DEC_K_COUNT) return DEC_ERR_INVALID;
    if (hipStreamSynchronize(h->st) != hipSuccess) return DEC_ERR_DEVICE;
    if (harvest(h) != DEC_OK) return DEC_ERR_DEVICE;
    const Timing &t = h->tm[kernel_class];
    if (total_ms) *total_ms = t.ms;
    if (launches) *launches = t.launches;
    if (bytes) *bytes = t.bytes;
    if (flops) *flops = t.flops;
    return DEC_OK;
}

const char *dec_status_str(int s) {
    switch (s) {
        case DEC_OK: return "ok";
        case DEC_ERR_INVALID: return "invalid argument";
        case DEC_ERR_RANGE: return "out of range";
        case DEC_ERR_NOMEM: return "workspace too small";
        case DEC_ERR_DEVICE: return "device error";
        case DEC_ERR_UNSUPPORTED: return "unsupported shape";
    }
    return "unknown status";
}

}  // extern "C"
