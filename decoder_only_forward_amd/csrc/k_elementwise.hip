// Row-wise kernels of the forward: residual add + RMSNorm (with the embedding
// gather as its first-layer form), the RoPE angle table, RoPE fused with the
// K/V cache store, silu(gate)*up, and the greedy argmax.
#include "common.h"
#include "kernels.h"
#include "kvcache.h"

// ---- residual + RMSNorm ----------------------------------------------------
// RMSNorm: a = x / sqrt(mean(x^2) + eps) * g  (Pantheon "Llama Forward Pass",
// section "RMSNorm").  One block of NTH threads per row; each thread keeps its
// float4 chunks of the row in registers between the sum of squares and the
// scaling.
template <int VPT, int NTH>
__global__ void __launch_bounds__(NTH) residual_norm_kernel(
    int mode, int d, float *__restrict__ x, const int32_t *__restrict__ tok,
    const void *__restrict__ embed, int embed_f32, Partials add, Partials moe, const int32_t *__restrict__ moe_inv,
    const float *__restrict__ moe_w, int k, const float *__restrict__ gain, float eps,
    u16 *__restrict__ a_hi, u16 *__restrict__ a_lo, float *__restrict__ a_f32, float *__restrict__ cap, F8Act f8) {
    __shared__ float red[16];
    const int t = blockIdx.x;
    const int nv = d / 4;
    float4 v[VPT];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < VPT; u++) {
        const int i4 = threadIdx.x + u * NTH;
        if (i4 >= nv) break;
        const size_t off = (size_t)t * d + 4 * i4;
        float4 r;
        if (mode == RN_EMBED) {
            const size_t e = (size_t)tok[t] * d + 4 * i4;
            if (embed_f32) {
                r = *reinterpret_cast<const float4 *>((const float *)embed + e);
            } else {
                const uint2 b = *reinterpret_cast<const uint2 *>((const u16 *)embed + e);
                r.x = bf16_bits_to_f32(b.x & 0xFFFFu); r.y = bf16_bits_to_f32(b.x >> 16);
                r.z = bf16_bits_to_f32(b.y & 0xFFFFu); r.w = bf16_bits_to_f32(b.y >> 16);
            }
        } else {
            r = *reinterpret_cast<const float4 *>(x + off);
            if (add.p) {
                const float4 a = sum_splits4(add.p, add.S, add.stride, (size_t)t * add.ld + 4 * i4);
                r.x += a.x; r.y += a.y; r.z += a.z; r.w += a.w;
            }
            if (moe_inv) {
                // the experts' outputs of this token, read at their grouped rows
                float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int j = 0; j < k; j++) {
                    const float w = moe_w[t * k + j];
                    const float4 e = sum_splits4(moe.p, moe.S, moe.stride, (size_t)moe_inv[t * k + j] * moe.ld + 4 * i4);
                    y.x += w * e.x; y.y += w * e.y; y.z += w * e.z; y.w += w * e.w;
                }
                r.x += y.x; r.y += y.y; r.z += y.z; r.w += y.w;
            }
        }
        *reinterpret_cast<float4 *>(x + off) = r;
        if (cap) *reinterpret_cast<float4 *>(cap + off) = r;
        ss += r.x * r.x + r.y * r.y + r.z * r.z + r.w * r.w;
        v[u] = r;
    }
    // the gain is loaded while the block reduces: its latency overlaps the barriers
    float4 g[VPT];
    if (gain) {
#pragma unroll
        for (int u = 0; u < VPT; u++) {
            const int i4 = threadIdx.x + u * NTH;
            if (i4 >= nv) break;
            g[u] = *reinterpret_cast<const float4 *>(gain + 4 * i4);
        }
    }
    const float tot = block_sum(ss, red);
    if (!gain) return;
    const float rs = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int u = 0; u < VPT; u++) {
        const int i4 = threadIdx.x + u * NTH;
        if (i4 >= nv) break;
        const size_t off = (size_t)t * d + 4 * i4;
        float4 a;
        a.x = v[u].x * rs * g[u].x; a.y = v[u].y * rs * g[u].y;
        a.z = v[u].z * rs * g[u].z; a.w = v[u].w * rs * g[u].w;
        if (a_f32) *reinterpret_cast<float4 *>(a_f32 + off) = a;
        if (f8.a16) {
            // fp16 + fp8 operands: the 8 threads of a 32-column block (d a
            // multiple of 32) share its scale, kept by the first of them
            float l0, l1, l2, l3;
            const uint32_t h0 = f16_split(a.x, l0), h1 = f16_split(a.y, l1);
            const uint32_t h2 = f16_split(a.z, l2), h3 = f16_split(a.w, l3);
            float mx = fmaxf(fmaxf(fabsf(l0), fabsf(l1)), fmaxf(fabsf(l2), fabsf(l3)));
            mx = fmaxf(mx, __shfl_xor(mx, 1, WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 2, WAVE));
            mx = fmaxf(mx, __shfl_xor(mx, 4, WAVE));
            const uint32_t sb = mx_scale_byte(mx);
            const size_t fo = (size_t)t * f8.lda + 4 * i4;
            *reinterpret_cast<uint2 *>(f8.a16 + fo) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
            // the fp8 row's 32-k blocks hold k 0-7, 16-23, 8-15, 24-31 (the order
            // the GEMM's lanes take the weights' bytes from their fp16 fragments)
            const int q = i4 & 7, qs = (q == 2 || q == 3) ? q + 2 : ((q == 4 || q == 5) ? q - 2 : q);
            *reinterpret_cast<uint32_t *>(f8.a8 + (size_t)t * f8.lda + 4 * ((i4 & ~7) | qs)) =
                fp8x4(l0, l1, l2, l3, sb);
            if ((threadIdx.x & 7) == 0) f8.asc[(size_t)(i4 >> 3) * f8.mpad + f8_asc_pos(t)] = (uint8_t)sb;
        } else if (a_hi) {
            uint2 h, l;
            split2_bf16(a.x, a.y, h.x, l.x);
            split2_bf16(a.z, a.w, h.y, l.y);
            *reinterpret_cast<uint2 *>(a_hi + off) = h;
            *reinterpret_cast<uint2 *>(a_lo + off) = l;
        }
    }
}

// Few rows (decode) of a row wider than one block covers: the residual update,
// which sums the split-K partials, runs over a (row, 1024-column chunk) grid
// and leaves per-chunk sums of squares; the norm kernel then scales each chunk.
// Chunk sums are added in chunk order, so the result does not depend on
// scheduling.
constexpr int RN_CHUNK = 1024;

__global__ void __launch_bounds__(256) residual_chunk_kernel(
    int d, float *__restrict__ x, Partials add, Partials moe, const int32_t *__restrict__ moe_inv,
    const float *__restrict__ moe_w,
    int k, float *__restrict__ cap, float *__restrict__ ssq) {
    __shared__ float red[16];
    const int t = blockIdx.x, ch = blockIdx.y;
    const int i4 = (ch * RN_CHUNK) / 4 + threadIdx.x;
    float ss = 0.f;
    if (4 * i4 < min(d, (ch + 1) * RN_CHUNK)) {
        const size_t off = (size_t)t * d + 4 * i4;
        float4 r = *reinterpret_cast<const float4 *>(x + off);
        if (add.p) {
            const float4 a = sum_splits4(add.p, add.S, add.stride, (size_t)t * add.ld + 4 * i4);
            r.x += a.x; r.y += a.y; r.z += a.z; r.w += a.w;
        }
        if (moe_inv) {
            float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int j = 0; j < k; j++) {
                const float w = moe_w[t * k + j];
                const float4 e = sum_splits4(moe.p, moe.S, moe.stride, (size_t)moe_inv[t * k + j] * moe.ld + 4 * i4);
                y.x += w * e.x; y.y += w * e.y; y.z += w * e.z; y.w += w * e.w;
            }
            r.x += y.x; r.y += y.y; r.z += y.z; r.w += y.w;
        }
        *reinterpret_cast<float4 *>(x + off) = r;
        if (cap) *reinterpret_cast<float4 *>(cap + off) = r;
        ss = r.x * r.x + r.y * r.y + r.z * r.z + r.w * r.w;
    }
    const float tot = block_sum(ss, red);
    if (threadIdx.x == 0) ssq[t * gridDim.y + ch] = tot;
}

__global__ void __launch_bounds__(256) norm_chunk_kernel(int d, const float *__restrict__ x, const float *__restrict__ ssq,
                                                         int nch, const float *__restrict__ gain, float eps,
                                                         u16 *__restrict__ a_hi, u16 *__restrict__ a_lo,
                                                         float *__restrict__ a_f32) {
    const int t = blockIdx.x, ch = blockIdx.y;
    float tot = 0.f;
    for (int c = 0; c < nch; c++) tot += ssq[t * nch + c];
    const float rs = 1.0f / sqrtf(tot / (float)d + eps);
    const int i4 = (ch * RN_CHUNK) / 4 + threadIdx.x;
    if (4 * i4 >= min(d, (ch + 1) * RN_CHUNK)) return;
    const size_t off = (size_t)t * d + 4 * i4;
    const float4 v = *reinterpret_cast<const float4 *>(x + off);
    const float4 g = *reinterpret_cast<const float4 *>(gain + 4 * i4);
    float4 a;
    a.x = v.x * rs * g.x; a.y = v.y * rs * g.y; a.z = v.z * rs * g.z; a.w = v.w * rs * g.w;
    if (a_f32) *reinterpret_cast<float4 *>(a_f32 + off) = a;
    if (a_hi) {
        uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
        split_bf16(a.x, h0, l0); split_bf16(a.y, h1, l1);
        split_bf16(a.z, h2, l2); split_bf16(a.w, h3, l3);
        *reinterpret_cast<uint2 *>(a_hi + off) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        *reinterpret_cast<uint2 *>(a_lo + off) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
    }
}

void launch_residual_norm(hipStream_t st, int mode, int T, int d, float *x, const int32_t *tok,
                          const void *embed, int embed_f32, Partials add, Partials moe, const int32_t *moe_inv,
                          const float *moe_w, int k, const float *gain, float eps, u16 *a_hi,
                          u16 *a_lo, float *a_f32, float *cap, float *ssq, const F8Act *f8) {
    if (T <= 0) return;
    const int nv = d / 4;
    // fp16 + fp8 operands: prefill rows only (one block per row, d % 32 == 0)
    const F8Act f8a = (f8 && T > 64 && d % 32 == 0) ? *f8 : F8Act{nullptr, nullptr, nullptr, 0, 0};
    if (T <= 64 && nv <= 1024) {
        // few rows: one 1024-thread block per row, one float4 per thread
#define RN1(NT) hipLaunchKernelGGL((residual_norm_kernel<1, NT>), dim3(T), dim3(NT), 0, st, mode, d, x, tok, embed, \
                                   embed_f32, add, moe, moe_inv, moe_w, k, gain, eps, a_hi, a_lo, a_f32, cap, f8a)
        if (nv <= 256) RN1(256);
        else RN1(1024);
#undef RN1
        return;
    }
    if (mode == RN_ADD && T <= 64 && ssq) {
        const int nch = (d + RN_CHUNK - 1) / RN_CHUNK;
        hipLaunchKernelGGL(residual_chunk_kernel, dim3(T, nch), dim3(256), 0, st, d, x, add, moe, moe_inv, moe_w, k, cap, ssq);
        if (gain)
            hipLaunchKernelGGL(norm_chunk_kernel, dim3(T, nch), dim3(256), 0, st, d, x, ssq, nch, gain, eps, a_hi,
                               a_lo, a_f32);
        return;
    }
    const int vpt = (nv + 255) / 256;
#define RN(V) hipLaunchKernelGGL((residual_norm_kernel<V, 256>), dim3(T), dim3(256), 0, st, mode, d, x, tok, \
                                 embed, embed_f32, add, moe, moe_inv, moe_w, k, gain, eps, a_hi, a_lo, a_f32, cap, \
                                 f8a)
    if (vpt <= 1) RN(1);
    else if (vpt <= 2) RN(2);
    else if (vpt <= 4) RN(4);
    else RN(8);
#undef RN
}

// ---- RoPE ------------------------------------------------------------------
// Pair i of a head turns f_i = theta^(-2i/hd) radians per position (rml "The
// decoder", section "Rotary embeddings"); with llama3 scaling (same section and
// its worked example) slow pairs are stretched: a wavelength 2*pi/f_i under
// orig_ctx/high keeps f_i, over orig_ctx/low takes f_i/factor, and in between
// s = (orig_ctx/wavelength - low)/(high - low) mixes (1 - s) f_i/factor + s f_i.
// The angle and its cos/sin are formed in double once per (position, pair) and
// shared by every head.
__global__ void rope_table_kernel(const int32_t *__restrict__ pos, int T, int hd, double theta, int scaling,
                                  double factor, double low, double high, int orig_ctx, float2 *__restrict__ tab) {
    const int half = hd / 2;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * half) return;
    const int t = idx / half, i = idx % half;
    double f = pow(theta, -2.0 * (double)i / (double)hd);
    if (scaling == 1) {
        const double wl = 6.283185307179586476925 / f;
        const double lo_wl = (double)orig_ctx / low, hi_wl = (double)orig_ctx / high;
        if (wl > lo_wl) {
            f = f / factor;
        } else if (wl >= hi_wl) {
            const double sm = ((double)orig_ctx / wl - low) / (high - low);
            f = (1.0 - sm) * (f / factor) + sm * f;
        }
    }
    const double ang = (double)pos[t] * f;
    tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

void launch_rope_table(hipStream_t st, const int32_t *pos, int T, int hd, double theta, int scaling,
                       double factor, double low, double high, int orig_ctx, float2 *tab) {
    const int n = T * (hd / 2);
    if (n <= 0) return;
    hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, pos, T, hd, theta, scaling,
                       factor, low, high, orig_ctx, tab);
}

// Pairs rotate as (e0 c - e1 s, e0 s + e1 c): adjacent elements (2i, 2i+1)
// (sipllm "Transformer forward pass", section "RoPE is adjacent-pair") or
// halves (i, i + hd/2) (rml "Which dimensions pair").  K and V go to the cache
// slot of the position (Pantheon, "Sliding Window (Mistral)": write at
// pos % max_seq when the cache is a ring).  One thread per 4 consecutive pairs
// of a head (hd is 16, 64 or 128), moved as float4 words: elements
// [i, i+4) and [i+hd/2, i+hd/2+4) for halves, [2i, 2i+8) for adjacent pairs
// (and for v, which is not rotated).
// Elements col .. col+3 of cache row `row` (rows of hd elements in the cache
// format kv_kind).
__device__ __forceinline__ void store4(void *cache, size_t row, int col, int hd, int kv_kind, float4 v) {
    char *c = static_cast<char *>(cache);
    if (kv_kind == KV_BF16) kv_store4<KV_BF16, 0>(c + row * kv_row_bytes<KV_BF16>(hd), col, v);
    else if (kv_kind == KV_F24) f24_store4(c + row * kv_row_bytes<KV_F24>(hd), hd, col, v);
    else kv_store4<KV_F32, 0>(c + row * kv_row_bytes<KV_F32>(hd), col, v);
}

__global__ void __launch_bounds__(256) rope_kv_kernel(
    Partials qkv, const float *__restrict__ bq, const float *__restrict__ bk, const float *__restrict__ bv,
    const float2 *__restrict__ tab, const int32_t *__restrict__ pos, const int32_t *__restrict__ slot,
    int nh, int nkv, int hd, int pairing, float *__restrict__ q_out, void *__restrict__ kc,
    void *__restrict__ vc, int max_seq, int ring, int kv_kind, int chunk) {
    const int t = blockIdx.x;
    const int qd = nh * hd, kvd = nkv * hd, half = hd / 2;
    const int npairs = (qd + 2 * kvd) / 2;
    const int pi = 4 * (blockIdx.y * blockDim.x + threadIdx.x);   // first of this thread's 4 pairs
    if (pi >= npairs) return;
    // section, head and pair index within the head (all 4 pairs share them)
    int base, i;
    if (pi < qd / 2) { base = 0; i = pi; }
    else if (pi < (qd + kvd) / 2) { base = qd; i = pi - qd / 2; }
    else { base = qd + kvd; i = pi - (qd + kvd) / 2; }
    const int head = i / half, ip = i % half;
    const bool rotate = base < qd + kvd;
    const bool halves = rotate && pairing;
    // element offsets within the section of the two float4 words
    const int w0 = head * hd + (halves ? ip : 2 * ip);
    const int w1 = halves ? w0 + half : w0 + 4;
    const size_t off = (size_t)t * qkv.ld + base;
    float4 a = sum_splits4(qkv.p, qkv.S, qkv.stride, off + w0);
    float4 c = sum_splits4(qkv.p, qkv.S, qkv.stride, off + w1);
    const float *bias = base == 0 ? bq : (base == qd ? bk : bv);
    if (bias) {
        add4(a, *reinterpret_cast<const float4 *>(bias + w0));
        add4(c, *reinterpret_cast<const float4 *>(bias + w1));
    }
    if (rotate) {
        // pair j: (e0, e1) = (a[j], c[j]) for halves, else elements 2j, 2j+1 of a|c
        float e0[4], e1[4];
        if (halves) {
            e0[0] = a.x; e0[1] = a.y; e0[2] = a.z; e0[3] = a.w;
            e1[0] = c.x; e1[1] = c.y; e1[2] = c.z; e1[3] = c.w;
        } else {
            e0[0] = a.x; e1[0] = a.y; e0[1] = a.z; e1[1] = a.w;
            e0[2] = c.x; e1[2] = c.y; e0[3] = c.z; e1[3] = c.w;
        }
        const float4 cs01 = *reinterpret_cast<const float4 *>(tab + (size_t)t * half + ip);
        const float4 cs23 = *reinterpret_cast<const float4 *>(tab + (size_t)t * half + ip + 2);
        const float cw[4] = {cs01.x, cs01.z, cs23.x, cs23.z}, sw[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float r0 = e0[j] * cw[j] - e1[j] * sw[j], r1 = e0[j] * sw[j] + e1[j] * cw[j];
            e0[j] = r0;
            e1[j] = r1;
        }
        if (halves) {
            a = make_float4(e0[0], e0[1], e0[2], e0[3]);
            c = make_float4(e1[0], e1[1], e1[2], e1[3]);
        } else {
            a = make_float4(e0[0], e1[0], e0[1], e1[1]);
            c = make_float4(e0[2], e1[2], e0[3], e1[3]);
        }
    }
    if (base == 0) {
        *reinterpret_cast<float4 *>(q_out + (size_t)t * qd + w0) = a;
        *reinterpret_cast<float4 *>(q_out + (size_t)t * qd + w1) = c;
    } else {
        const int p = pos[t];
        const int s = ring ? p % max_seq : p;
        void *cache = base == qd ? kc : vc;
        // the layer cache at the position's slot, or row t of a chunk buffer [T][nkv][hd]
        const size_t row = chunk ? (size_t)t * nkv + head : ((size_t)slot[t] * nkv + head) * max_seq + s;
        store4(cache, row, w0 - head * hd, hd, kv_kind, a);
        store4(cache, row, w1 - head * hd, hd, kv_kind, c);
    }
}

void launch_rope_kv(hipStream_t st, int T, Partials qkv, const float *bq, const float *bk,
                    const float *bv, const float2 *tab, const int32_t *pos, const int32_t *slot,
                    int nh, int nkv, int hd, int pairing, float *q_out, void *kc, void *vc, int max_seq,
                    int ring, int kv_kind, int chunk) {
    if (T <= 0) return;
    const int nquads = (nh + 2 * nkv) * hd / 8;
    hipLaunchKernelGGL(rope_kv_kernel, dim3(T, (nquads + 255) / 256), dim3(256), 0, st, qkv, bq, bk, bv, tab, pos,
                       slot, nh, nkv, hd, pairing, q_out, kc, vc, max_seq, ring, kv_kind, chunk);
}

// Commit a chunk's K/V rows [T][nkv][hd] to the ring slots of positions
// start..start+T-1 of sequence slot `s`.  Only the last min(T, max_seq) rows
// are written: an earlier row's slot is taken again by a later one.
__global__ void commit_chunk_kernel(const uint32_t *__restrict__ ck, const uint32_t *__restrict__ cv, int T,
                                    int first, int start, int s, int nkv, int words, int max_seq,
                                    uint32_t *__restrict__ kc, uint32_t *__restrict__ vc) {
    const int t = first + blockIdx.x, h = blockIdx.y;
    if (t >= T) return;
    const size_t src = ((size_t)t * nkv + h) * words;
    const size_t dst = (((size_t)s * nkv + h) * max_seq + (start + t) % max_seq) * words;
    for (int i = threadIdx.x; i < words; i += blockDim.x) {
        kc[dst + i] = ck[src + i];
        vc[dst + i] = cv[src + i];
    }
}

void launch_commit_chunk(hipStream_t st, const void *ck, const void *cv, int T, int start, int s, int nkv, int hd,
                         int es, int max_seq, void *kc, void *vc) {
    const int first = T > max_seq ? T - max_seq : 0;
    const int words = hd * es / 4;   // es = 4, 2 or 3 bytes an element: rows of whole words for hd % 16 == 0
    if (T - first <= 0) return;
    hipLaunchKernelGGL(commit_chunk_kernel, dim3(T - first, nkv), dim3(64), 0, st,
                       static_cast<const uint32_t *>(ck), static_cast<const uint32_t *>(cv), T, first, start, s, nkv,
                       words, max_seq, static_cast<uint32_t *>(kc), static_cast<uint32_t *>(vc));
}

// ---- SwiGLU activation -----------------------------------------------------
// act = silu(gate) * up, silu(z) = z / (1 + e^-z)  (Pantheon, "SwiGLU FFN").
__global__ void __launch_bounds__(256) silu_mul_kernel(int F, Partials gu, u16 *__restrict__ hi,
                                                        u16 *__restrict__ lo, float *__restrict__ f32) {
    const int t = blockIdx.y;
    const int j4 = blockIdx.x * blockDim.x + threadIdx.x;
    if (4 * j4 >= F) return;
    const size_t off = (size_t)t * gu.ld + 4 * j4;
    const float4 g = sum_splits4(gu.p, gu.S, gu.stride, off);
    const float4 u = sum_splits4(gu.p, gu.S, gu.stride, off + F);
    float4 a;
    a.x = g.x / (1.0f + expf(-g.x)) * u.x;
    a.y = g.y / (1.0f + expf(-g.y)) * u.y;
    a.z = g.z / (1.0f + expf(-g.z)) * u.z;
    a.w = g.w / (1.0f + expf(-g.w)) * u.w;
    const size_t o = (size_t)t * F + 4 * j4;
    if (f32) *reinterpret_cast<float4 *>(f32 + o) = a;
    if (hi) {
        uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
        split_bf16(a.x, h0, l0); split_bf16(a.y, h1, l1);
        split_bf16(a.z, h2, l2); split_bf16(a.w, h3, l3);
        *reinterpret_cast<uint2 *>(hi + o) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
        *reinterpret_cast<uint2 *>(lo + o) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
    }
}

void launch_silu_mul(hipStream_t st, int T, int F, Partials gu, u16 *hi, u16 *lo, float *f32) {
    if (T <= 0) return;
    const int n4 = F / 4;
    hipLaunchKernelGGL(silu_mul_kernel, dim3((n4 + 255) / 256, T), dim3(256), 0, st, F, gu, hi, lo, f32);
}

// ---- greedy ------------------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

__global__ void __launch_bounds__(1024) argmax_kernel(const float *__restrict__ logits, int V,
                                                      int32_t *__restrict__ out) {
    __shared__ float sv[16];
    __shared__ int si[16];
    const int b = blockIdx.x;
    const float *row = logits + (size_t)b * V;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    // eight loads per thread in flight, then compared in index order
    constexpr int U = 8;
    for (int i0 = threadIdx.x; i0 < V; i0 += blockDim.x * U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = i0 + u * blockDim.x;
            v[u] = i < V ? row[i] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = i0 + u * blockDim.x;
            if (i < V && better(v[u], i, bv, bi)) { bv = v[u]; bi = i; }
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, WAVE);
        const int oi = __shfl_xor(bi, o, WAVE);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
    if (lane == 0) { sv[w] = bv; si[w] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < (int)(blockDim.x / WAVE); i++)
            if (better(sv[i], si[i], bv, bi)) { bv = sv[i]; bi = si[i]; }
        out[b] = bi == 0x7FFFFFFF ? 0 : bi;
    }
}

void launch_argmax(hipStream_t st, const float *logits, int B, int V, int32_t *out) {
    if (B <= 0) return;
    hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, st, logits, V, out);
}

// ---- small helpers -------------------------------------------------------------
// dst[t][n] = sum over splits of a GEMV output (used where no consumer kernel
// folds the sum in, e.g. the LM head writing the caller's logits).
__global__ void __launch_bounds__(256) reduce_splits_kernel(Partials src, int N, float *__restrict__ dst, int ldd) {
    const int t = blockIdx.y;
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    dst[(size_t)t * ldd + n] = sum_splits(src.p, src.S, src.stride, (size_t)t * src.ld + n);
}

void launch_reduce_splits(hipStream_t st, Partials src, int T, int N, float *dst, int ldd) {
    if (T <= 0) return;
    hipLaunchKernelGGL(reduce_splits_kernel, dim3((N + 255) / 256, T), dim3(256), 0, st, src, N, dst, ldd);
}

// Decode rows travel as a kernel argument (no host buffer has to outlive the
// call): tok/pos of row b, slot b.
// Decode rows: token, position and slot of each row.  The tokens come from the
// arguments, or, when src is given, from device memory (the previous step's
// greedy choice), which is then also appended to hist when that is given.
__global__ void set_rows_kernel(RowArgs a, int B, const int32_t *__restrict__ src, int32_t *__restrict__ hist,
                                int32_t *__restrict__ tok, int32_t *__restrict__ pos, int32_t *__restrict__ slot) {
    const int b = threadIdx.x;
    if (b >= B) return;
    const int32_t t = src ? src[b] : a.tok[b];
    if (hist) hist[b] = t;
    tok[b] = t;
    pos[b] = a.pos[b];
    slot[b] = a.slot[b];
}

void launch_set_rows(hipStream_t st, const RowArgs &a, int B, const int32_t *src, int32_t *hist, int32_t *tok,
                     int32_t *pos, int32_t *slot) {
    hipLaunchKernelGGL(set_rows_kernel, dim3(1), dim3(64), 0, st, a, B, src, hist, tok, pos, slot);
}

// dst[i] = src[i], i < n (n <= 64): the last greedy choice of a device loop.
__global__ void copy_ids_kernel(const int32_t *__restrict__ src, int n, int32_t *__restrict__ dst) {
    const int i = threadIdx.x;
    if (i < n) dst[i] = src[i];
}

void launch_copy_ids(hipStream_t st, const int32_t *src, int n, int32_t *dst) {
    hipLaunchKernelGGL(copy_ids_kernel, dim3(1), dim3(64), 0, st, src, n, dst);
}

// Prefill rows: positions start..start+T-1 of one slot.
__global__ void set_seq_rows_kernel(int T, int start, int s, int32_t *__restrict__ pos, int32_t *__restrict__ slot) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    pos[t] = start + t;
    slot[t] = s;
}

void launch_set_seq_rows(hipStream_t st, int T, int start, int s, int32_t *pos, int32_t *slot) {
    if (T <= 0) return;
    hipLaunchKernelGGL(set_seq_rows_kernel, dim3((T + 255) / 256), dim3(256), 0, st, T, start, s, pos, slot);
}
