// Host-side launch interface of the gfx950 kernels (internal to libdec).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

typedef uint16_t u16;

// A GEMM/GEMV output that may be split along K: the value of (row t, col) is
// the sum over s ascending of p[s*stride + t*ld + col].
struct Partials {
    const float *p;
    int S;
    size_t stride;
    int ld;
};

// One weight matrix [rows][K] of a column-concatenated projection (q|k|v, gate|up).
struct WSeg {
    const void *w;
    int rows;
};

// Prefill activations as fp16 + fp8 split operands: a16 [rows][lda] fp16,
// a8 [rows][lda] fp8 e4m3 and E8M0 scales asc [lda/32][mpad], mpad = rows
// rounded up to 256 (written with f16_split / mx_scale_byte / fp8x4).
struct F8Act {
    u16 *a16;
    uint8_t *a8, *asc;
    int lda, mpad;
};
#define MAX_SEGS 3

// Residual update + RMSNorm of one row per block:
//   mode EMBED:  x = widen(E[tok[t]])
//   otherwise:   x += sum of `add` splits (if any)
//                     + sum_j moe_w[t][j] * (sum of moe splits at grouped row moe_inv[t*k+j]) (if moe_inv)
// then a = x / sqrt(mean(x^2)+eps) * gain written as bf16 (hi, lo) and/or fp32,
// or, with f8 (rows written one block per row), as fp16 + fp8 split operands.
// ssq: scratch of T*ceil(d/1024) floats, used to split the work over columns
// when there are few rows (may be null: one block per row).
enum { RN_EMBED = 0, RN_ADD = 1 };
void launch_residual_norm(hipStream_t st, int mode, int T, int d, float *x, const int32_t *tok,
                          const void *embed, int embed_f32, Partials add, Partials moe, const int32_t *moe_inv,
                          const float *moe_w, int k, const float *gain, float eps, u16 *a_hi,
                          u16 *a_lo, float *a_f32, float *cap, float *ssq, const F8Act *f8 = nullptr);

// cos/sin of pos[t] * f_i for pair i, f_i = theta^(-2i/hd) (llama3-scaled when
// scaling == 1), formed in double: tab[t][i].
void launch_rope_table(hipStream_t st, const int32_t *pos, int T, int hd, double theta, int scaling,
                       double factor, double low, double high, int orig_ctx, float2 *tab);

// q/k/v (+bias) -> RoPE on q and k -> q_out [T][q_dim]; k, v stored in the
// layer's cache [slot][kvh][max_seq][hd] at position pos % max_seq (ring) or pos,
// or, when chunk is set, in rows [T][nkv][hd] of the buffers kc, vc; in the
// cache format kv_kind (KV_F32, KV_BF16 or KV_F24 of kvcache.h).
// pairing 0 rotates elements (2i, 2i+1) of a head, 1 rotates (i, i + hd/2).
void launch_rope_kv(hipStream_t st, int T, Partials qkv, const float *bq, const float *bk,
                    const float *bv, const float2 *tab, const int32_t *pos, const int32_t *slot,
                    int nh, int nkv, int hd, int pairing, float *q_out, void *kc, void *vc, int max_seq,
                    int ring, int kv_kind, int chunk);
// Store a chunk's rows [T][nkv][hd] (es = 4, 2 or 3 bytes per element) at the ring slots of
// positions start.. of sequence slot s: the last min(T, max_seq) rows.
void launch_commit_chunk(hipStream_t st, const void *ck, const void *cv, int T, int start, int s, int nkv, int hd,
                         int es, int max_seq, void *kc, void *vc);

// act[t][j] = silu(g) * u with g = gu(t, j), u = gu(t, F + j); written as bf16
// (hi, lo) and/or fp32 with row stride F.
void launch_silu_mul(hipStream_t st, int T, int F, Partials gu, u16 *hi, u16 *lo, float *f32);

// out[b] = argmax_v logits[b][v], lowest v on ties.
void launch_argmax(hipStream_t st, const float *logits, int B, int V, int32_t *out);

// Decode projection, bf16 weights: out[s][b][n] = sum over split s's K range of
// W[n][k] * (a_hi[b][k] + a_lo[b][k]); 1 <= B <= 64, K a multiple of 64.
// gemv_splits gives the split count to launch with.
int gemv_splits(int N, int K, int B);
int gemv_grouped_splits(int N, int K, int B);   // the split count for launch_gemv_grouped
// upper bounds of gemv_splits and gemv_grouped_splits (host-only, for the workspace plan)
int gemv_max_splits(int N, int K);
int gemv_grouped_max_splits(int K);
int num_cus();
// Residual + RMSNorm of one decode row, formed by a projection's own blocks
// ahead of their products (Pantheon "Llama Forward Pass", section "RMSNorm"):
// x_new = x + the previous projection's split partials (summed in split
// order), a = x_new / sqrt(mean(x_new^2) + eps) * gain; every block reads the
// whole row and keeps the bf16 (hi, lo) pair of its own k range in LDS, and
// block (0, 0) stores x_new (and the capture row, when given).  x and x_new
// are distinct buffers (the other blocks still read x); d <= 8192.
struct RowNorm {
    const float *x;
    float *x_new;
    float *cap;
    Partials add;
    const float *gain;
    float eps;
    int d;
};

// The one decode row's attention output formed inside the output projection's
// blocks (launch_gemv with B = 1): the split-KV partials of the decode
// attention ([head][split][hd + 2]: hd unnormalised outputs, the split's
// maximum, its normaliser) merged per element in split order, as the
// separate merge kernel does (the running maximum and normaliser of rml "The
// decoder", section "Attend", combined over splits).  2 <= splits <= 32.
struct AttnMerge {
    const float *part;
    int hd;
    int splits;
};
void launch_gemv(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi, const u16 *a_lo,
                 int lda, int B, float *out, int ksplit, size_t split_stride, int ldo, const RowNorm *rn = nullptr,
                 const AttnMerge *am = nullptr);

// Prefill projection, bf16 weights, MFMA: out[m][n] = sum_k (a_hi+a_lo)[m][k] W[n][k].
// gemm_splits(N, K, M) gives the k splits to launch with (1 to 16): with S > 1,
// launch_gemm writes S k-split partials, split s at out + s*split_stride (the
// consumer sums them).
// gemm_splits_for takes the CU count (host-only use: the workspace plan).
int gemm_splits(int N, int K, int M);
// kmul: k-tiles of 32 per split a multiple of kmul (2 for the fp16 + fp8 form)
int gemm_splits_for(int N, int K, int M, int cus, int kmul = 1);
int gemm_splits_f8(int N, int K, int M);
void launch_gemm(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi, const u16 *a_lo,
                 int lda, int M, float *out, int ldo, int ksplit = 1, size_t split_stride = 0);

// The gate|up projection of a SwiGLU FFN with silu(gate) * up fused into the
// epilogue, written as bf16 (hi, lo) pairs [M][ldo] (F features).  Taken only
// when the grid has at least one 256 x 256 tile per CU; returns false (nothing
// launched) otherwise.  s_hi/s_lo must not alias a_hi/a_lo.
bool launch_gemm_silu(hipStream_t st, const void *w_gate, const void *w_up, int F, int K, const u16 *a_hi,
                      const u16 *a_lo, int lda, int M, u16 *s_hi, u16 *s_lo, int ldo);
// Decode form of the fused SwiGLU: gate and up of F features (bf16 [F, K]
// each) against B <= 64 activation rows, one k split, silu(gate) * up written
// as bf16 (hi, lo) pairs to s_hi/s_lo [B][ldo].  Returns false (nothing
// launched) for shapes it does not take: K not a multiple of 64 or F not a
// multiple of 8.  With rn (B = 1), the row's residual + RMSNorm is formed in
// the kernel and a_hi/a_lo are not read.
bool launch_gemv_silu(hipStream_t st, const void *w_gate, const void *w_up, int F, int K, const u16 *a_hi,
                      const u16 *a_lo, int lda, int B, u16 *s_hi, u16 *s_lo, int ldo, const RowNorm *rn = nullptr);

// fp32-weight projection (any M): out[m][n] = sum_k a[m][k] W[n][k].
void launch_gemm_f32(hipStream_t st, const WSeg *segs, int nseg, int K, const float *a, int lda,
                     int M, float *out, int ldo);

// The decode rows' q | k | v projection (split partials; fp32 biases when
// given) and the RoPE table of their positions (tab[b][i], see
// launch_rope_table), from which the decode attention forms its queries and
// the K/V row of each row's new position.
struct RopeArgs {
    Partials qkv;
    const float *bq, *bk, *bv;
    const float2 *tab;
    int pairing;   // 0 rotates elements (2i, 2i+1) of a head, 1 rotates (i, i + hd/2)
    int ring;      // the cache is a ring: position p sits at slot p % max_seq
};

// Split-KV decode attention.  Row b (sequence slot slot[b], position pos[b]):
// q and the new K/V row come from ra (RoPE applied as launch_rope_kv does);
// the K/V row is stored at the position's slot of the layer cache (in the
// cache format kv_kind) by the block whose split covers it,
// and the keys/values of the readable slots [0, min(pos+1, max_seq)) are then
// attended.  Writes the attention output as bf16 (hi, lo) and/or fp32 rows
// [B][nh*hd].
int attn_decode_splits(int B, int nkv, int readable, int hd, int G, int kv_kind);
void launch_attn_decode(hipStream_t st, int B, const RopeArgs &ra, void *kc, void *vc, int kv_kind,
                        const int32_t *pos, const int32_t *slot, int nh, int nkv, int hd, int max_seq,
                        int splits, float *part, u16 *o_hi, u16 *o_lo, float *o_f32, bool merge = true);

// Causal prefill attention for T rows of one sequence at positions
// start_pos..start_pos+T-1.  Query p attends to positions [p - window + 1, p]
// (window 0: [0, p]).  Keys/values of positions before start_pos come from the
// layer cache (slot pos % max_seq when ring is set, else pos); the chunk's own
// come from the cache as well (ck == nullptr: already stored there) or from the
// chunk buffers ck, cv [T][nkv][hd] (deferred commit).
void launch_attn_prefill(hipStream_t st, int T, int start_pos, int slot, const float *q,
                         const void *kc, const void *vc, int kv_kind, int nh, int nkv, int hd, int max_seq,
                         int window, int ring, const void *ck, const void *cv, u16 *o_hi, u16 *o_lo,
                         float *o_f32);

// The same attention over pre-split K/V tiles (head_dim 64 or 128, every key
// position at its own slot: start_pos + T <= max_seq).  Each call first writes
// the tiles of positions [0, start_pos + T) of sequence `slot` into `img`
// (attn_tiles_bytes(max_seq, nkv, hd, kv_kind) bytes), then runs the MFMA
// kernel.  A launch of few row blocks splits their key tiles into chunks whose
// partial results go to `part` (part_floats floats of scratch, free during the
// call) and a merge pass; part may be null (no split).  Returns false for an
// unsupported head_dim or group size (nothing launched).
size_t attn_tiles_bytes(int max_pos, int nkv, int hd, int kv_kind);
bool launch_attn_prefill_tiles(hipStream_t st, int T, int start_pos, int slot, const float *q, const void *kc,
                               const void *vc, int kv_kind, int nh, int nkv, int hd, int max_seq, void *img,
                               float *part, size_t part_floats, u16 *o_hi, u16 *o_lo, float *o_f32);

// MoE.  Router logits [T][E] -> softmax, top-k by repeated selection (ties to
// the lower id), renormalised weights; then the (token, slot) pairs are grouped
// by expert (counting sort, stable in (token, slot) order): pairs[r] is the
// pair index t*k+j at grouped row r, and inv[t*k+j] = r.  The logits are the
// split partials `logits`, or, when router_w (bf16 [E][d]) is given, formed
// here from it and the (hi, lo) activation rows a_hi/a_lo [T][lda].
void launch_moe_route(hipStream_t st, int T, int E, int k, Partials logits, const u16 *router_w, const u16 *a_hi,
                      const u16 *a_lo, int d, int lda, int32_t *ids, float *w, float *router_cap, int32_t *ids_cap,
                      int32_t *counts, int32_t *offsets, int32_t *pairs, int32_t *inv);
// Gather the normalised rows of the grouped pairs: dst[i] = src[pairs[i] / k].
void launch_moe_gather(hipStream_t st, int T, int k, int d, const int32_t *pairs, const u16 *src_hi,
                       const u16 *src_lo, const float *src_f32, u16 *dst_hi, u16 *dst_lo, float *dst_f32);
// Grouped expert projections: expert e (grid z) multiplies grouped rows
// [offsets[e], offsets[e+1]) by its slice (segs[i].w + e*expert_stride) of the
// stacked weights [E][rows][K]; out rows follow the grouped order.  Grouped row
// r reads row r of `a`, or, with row_pairs, token row row_pairs[r] / row_k of
// `a` (the activations in token order, no gathered copy).  max_rows bounds any
// expert's row count (a token picks an expert at most once).
void launch_gemv_grouped(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi,
                         const u16 *a_lo, int lda, int max_rows, int E, const int32_t *offsets,
                         size_t expert_stride, float *out, int ksplit, size_t split_stride, int ldo,
                         const int32_t *row_pairs = nullptr, int row_k = 1);
// The MFMA form for prefill rows (bf16 weights): 256-feature x 256-row tiles
// per expert, k split in `ksplit` partials (out + s*split_stride) as
// gemm_grouped_splits(N, K, pairs, E) suggests for `pairs` grouped rows.
int gemm_grouped_splits(int N, int K, int pairs, int E);
int gemm_grouped_splits_for(int N, int K, int pairs, int E, int cus);   // host-only (the workspace plan)
void launch_gemm_grouped(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi,
                         const u16 *a_lo, int lda, int max_rows, int E, const int32_t *offsets,
                         size_t expert_stride, float *out, int ldo, int ksplit = 1, size_t split_stride = 0);
// Grouped gate|up of the experts' SwiGLU with silu(gate) * up in the epilogue,
// written as bf16 (hi, lo) pairs at the grouped rows of s_hi/s_lo [rows][ldo]
// (F features).  Returns false (nothing launched) when K is not a multiple of
// 32.  s_hi/s_lo must not alias a_hi/a_lo.
bool launch_gemm_grouped_silu(hipStream_t st, const void *w_gate, const void *w_up, int F, int K, const u16 *a_hi,
                              const u16 *a_lo, int lda, int max_rows, int E, const int32_t *offsets,
                              size_t expert_stride, u16 *s_hi, u16 *s_lo, int ldo);

// ---- prefill projections on fp16 + fp8 operands (k_gemm.hip) ---------------
// A weight matrix converted once: W16 [npad][K] fp16, rows in the GEMM's tile
// order (SILU: gate and up rows interleaved per tile); the fp8 pass reads each
// weight's upper byte as e5m2.  K a multiple of 64.
struct F8Weights {
    const u16 *w16;
    int N, K, npad;
    bool silu;
};
// the form's kernels can be launched (their LDS attribute is set); decided
// before any producer writes the form
bool gemm_f8_ready();
int f8_npad(int N, bool silu);
size_t f8_weight_bytes(int N, int K, bool silu);      // bytes of one converted matrix (256-aligned parts)
F8Weights f8_weights_at(void *base, int N, int K, bool silu);
// segs: the bf16 row segments (SILU: gate then up, F rows each)
void launch_convert_f8(hipStream_t st, const WSeg *segs, int nseg, int K, bool silu, const F8Weights &w);
// false where the form does not apply (K % 64, a SILU/non-SILU mismatch); the
// k split must leave a multiple of 64 k per split, else one split is taken
bool launch_gemm_f8(hipStream_t st, const F8Weights &w, const u16 *a16, const uint8_t *a8, const uint8_t *asc,
                    int mpad, int lda, int M, float *out, int ldo, int ksplit = 1, size_t split_stride = 0);
bool launch_gemm_f8_silu(hipStream_t st, const F8Weights &w, const u16 *a16, const uint8_t *a8, const uint8_t *asc,
                         int mpad, int lda, int M, u16 *s_hi, u16 *s_lo, int ldo);
void launch_gemm_f32_grouped(hipStream_t st, const WSeg *segs, int nseg, int K, const float *a, int lda,
                             int max_rows, int E, const int32_t *offsets, size_t expert_stride, float *out,
                             int ldo);

// Sum of GEMV split partials into a plain row-major destination.
void launch_reduce_splits(hipStream_t st, Partials src, int T, int N, float *dst, int ldd);

// Up to 64 decode rows passed by value to a setup kernel.
struct RowArgs {
    int32_t tok[64];
    int32_t pos[64];
    int32_t slot[64];
};
// Decode rows (B <= 64): tokens from a.tok, or from device src when given (also
// appended to hist when given); positions and slots from a.
void launch_set_rows(hipStream_t st, const RowArgs &a, int B, const int32_t *src, int32_t *hist, int32_t *tok,
                     int32_t *pos, int32_t *slot);
void launch_copy_ids(hipStream_t st, const int32_t *src, int n, int32_t *dst);
void launch_set_seq_rows(hipStream_t st, int T, int start, int s, int32_t *pos, int32_t *slot);
