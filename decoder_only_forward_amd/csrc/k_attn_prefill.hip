// Causal prefill attention: softmax(q k^T / sqrt(hd) + causal mask) v for the
// positions of one sequence (zLLM "The Algorithm Layer", section 2; Pantheon
// "Llama Forward Pass", "Grouped Query Attention": query head h reads kv head
// h*n_kv/n_head), with the one-pass online softmax of rml "The decoder",
// section "Attend".
#include "common.h"
#include "kernels.h"
#include "kvcache.h"

namespace {

__device__ __forceinline__ void store_out(float v, size_t off, u16 *o_hi, u16 *o_lo, float *o_f32) {
    if (o_f32) o_f32[off] = v;
    if (o_hi) {
        uint32_t h, l;
        split_bf16(v, h, l);
        o_hi[off] = (u16)h;
        o_lo[off] = (u16)l;
    }
}

// Byte address of the K (or V) row of position j for kv head kvh: row t of the
// chunk buffer [T][nkv][HD] for chunk positions when a chunk buffer is given,
// else the layer cache row at slot j % ring_mod (ring) or j.
// GEN = false: every position is in the cache at slot == position.
template <int HD, int KT, bool GEN>
__device__ __forceinline__ const char *kv_row(const void *cache, const void *chunk, size_t head_base, int j,
                                              int start_pos, int ring_mod, int nkv, int kvh) {
    constexpr int RB = kv_row_bytes<KT>(HD);
    if constexpr (!GEN) return static_cast<const char *>(cache) + (head_base + j) * RB;
    if (j >= start_pos)
        return static_cast<const char *>(chunk) + ((size_t)(j - start_pos) * nkv + kvh) * RB;
    const int s = ring_mod ? j % ring_mod : j;
    return static_cast<const char *>(cache) + (head_base + s) * RB;
}

}  // namespace

// ---- prefill ------------------------------------------------------------------
// One thread (or SPLIT adjacent lanes, each HD/SPLIT dims) per (query row,
// head); a block covers BQ query rows x the G heads of one kv head, and K/V
// tiles of BKV positions are staged in LDS once for all of them (the blocked
// prefill of Pantheon "Llama Forward Pass", section "Flash (Blocked) Prefill
// Attention": K/V reads cut from ~P to ~P/BQ).  fp32 arithmetic throughout.
namespace {

constexpr int BQ = 32, BKV = 32, SB = 8;

template <int HD, int G, int SPLIT, int KT, bool GEN>
__global__ void __launch_bounds__(BQ * G * SPLIT) attn_prefill_kernel(
    int T, int start_pos, int slot, const float *__restrict__ q, const void *__restrict__ kc,
    const void *__restrict__ vc, int nh, int nkv, int max_seq, int window, int ring_mod,
    const void *__restrict__ ck, const void *__restrict__ cv, u16 *__restrict__ o_hi, u16 *__restrict__ o_lo,
    float *__restrict__ o_f32) {
    constexpr int D = HD / SPLIT;
    constexpr int NT = BQ * G * SPLIT;
    __shared__ __attribute__((aligned(16))) float sk[BKV][HD];
    __shared__ __attribute__((aligned(16))) float sv[BKV][HD];

    const int kvh = blockIdx.y;
    const int t0 = blockIdx.x * BQ;
    const int tid = threadIdx.x;
    const int part = tid % SPLIT;
    const int g = (tid / SPLIT) % G;
    const int qi = tid / (SPLIT * G);
    const int t = t0 + qi;
    const bool live = t < T;
    const int qpos = start_pos + (live ? t : T - 1);
    const int h = kvh * G + g;

    float qr[D], acc[D];
    const float *qp = q + (size_t)(live ? t : T - 1) * nh * HD + (size_t)h * HD + part * D;
#pragma unroll
    for (int i = 0; i < D; i += 4) {
        const float4 a = *reinterpret_cast<const float4 *>(qp + i);
        qr[i] = a.x; qr[i + 1] = a.y; qr[i + 2] = a.z; qr[i + 3] = a.w;
        acc[i] = acc[i + 1] = acc[i + 2] = acc[i + 3] = 0.f;
    }
    const float scale = 1.0f / sqrtf((float)HD);
    float m = -INFINITY, l = 0.f;

    const size_t head_base = ((size_t)slot * nkv + kvh) * max_seq;
    const int last_pos = start_pos + min(T, t0 + BQ) - 1;  // largest query position of the block
    // GEN: positions may lie before the window (ring past its size)
    const int first_key = GEN && window ? max(0, start_pos + t0 - window + 1) : 0;
    const int lo_q = GEN && window ? qpos - window + 1 : 0;  // this query's oldest key
    for (int kb = first_key; kb <= last_pos; kb += BKV) {
        __syncthreads();
        for (int i = tid; i < BKV * HD / 4; i += NT) {
            const int row = i / (HD / 4), c4 = i % (HD / 4);
            const int j = kb + row;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (j <= last_pos) {
                kv = kv_load4<KT, HD>(kv_row<HD, KT, GEN>(kc, ck, head_base, j, start_pos, ring_mod, nkv, kvh), 4 * c4);
                vv = kv_load4<KT, HD>(kv_row<HD, KT, GEN>(vc, cv, head_base, j, start_pos, ring_mod, nkv, kvh), 4 * c4);
            }
            *reinterpret_cast<float4 *>(&sk[row][4 * c4]) = kv;
            *reinterpret_cast<float4 *>(&sv[row][4 * c4]) = vv;
        }
        __syncthreads();
        const int nkeys = min(BKV, qpos - kb + 1);  // causal: keys kb .. qpos
        for (int j0 = 0; j0 < BKV; j0 += SB) {
            if (j0 >= nkeys) break;
            float s[SB];
#pragma unroll
            for (int jj = 0; jj < SB; jj++) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < D; i += 4) {
                    const float4 kk = *reinterpret_cast<const float4 *>(&sk[j0 + jj][part * D + i]);
                    d += qr[i] * kk.x + qr[i + 1] * kk.y + qr[i + 2] * kk.z + qr[i + 3] * kk.w;
                }
#pragma unroll
                for (int o = SPLIT / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, WAVE);
                s[jj] = (j0 + jj < nkeys && (!GEN || kb + j0 + jj >= lo_q)) ? d * scale : -INFINITY;
            }
            float mx = m;
#pragma unroll
            for (int jj = 0; jj < SB; jj++) mx = fmaxf(mx, s[jj]);
            if (mx == -INFINITY) continue;  // every key of the group is outside the window
            const float corr = expf(m - mx);
            m = mx;
            float pe[SB], ps = 0.f;
#pragma unroll
            for (int jj = 0; jj < SB; jj++) {
                pe[jj] = expf(s[jj] - mx);
                ps += pe[jj];
            }
            l = l * corr + ps;
#pragma unroll
            for (int i = 0; i < D; i++) acc[i] *= corr;
#pragma unroll
            for (int jj = 0; jj < SB; jj++) {
#pragma unroll
                for (int i = 0; i < D; i += 4) {
                    const float4 vv = *reinterpret_cast<const float4 *>(&sv[j0 + jj][part * D + i]);
                    acc[i] += pe[jj] * vv.x; acc[i + 1] += pe[jj] * vv.y;
                    acc[i + 2] += pe[jj] * vv.z; acc[i + 3] += pe[jj] * vv.w;
                }
            }
        }
    }
    if (!live) return;
    const float inv = 1.0f / l;
    const size_t off = (size_t)t * nh * HD + (size_t)h * HD + part * D;
#pragma unroll
    for (int i = 0; i < D; i++) store_out(acc[i] * inv, off + i, o_hi, o_lo, o_f32);
}

template <int HD, int SPLIT, int KT, bool GEN>
bool launch_prefill_hd(hipStream_t st, int G, dim3 grid, int T, int start_pos, int slot, const float *q,
                       const void *kc, const void *vc, int nh, int nkv, int max_seq, int window, int ring_mod,
                       const void *ck, const void *cv, u16 *o_hi, u16 *o_lo, float *o_f32) {
#define AP(GG) hipLaunchKernelGGL((attn_prefill_kernel<HD, GG, SPLIT, KT, GEN>), grid, dim3(BQ * GG * SPLIT), 0, st, T, \
                                  start_pos, slot, q, kc, vc, nh, nkv, max_seq, window, ring_mod, ck, cv, o_hi, \
                                  o_lo, o_f32)
    switch (G) {
        case 1: AP(1); return true;
        case 2: AP(2); return true;
        case 3: AP(3); return true;
        case 4: AP(4); return true;
        case 5: AP(5); return true;
        case 6: AP(6); return true;
        case 7: AP(7); return true;
        case 8: AP(8); return true;
    }
#undef AP
    return false;
}

}  // namespace

// ---- prefill on MFMA ---------------------------------------------------------------
// Flash attention for head_dim 64/128.  A block holds 128 query vectors ((row,
// head) pairs of one kv group) and streams the group's K/V in tiles of 64
// positions through LDS, converted once to bf16 (hi, lo) pairs.  Per wave (32
// query vectors):
//   S^T = K Q^T   (32x32x16 MFMAs; lane q+32h owns 32 scores of query q, so
//                  the row max / sum of the online softmax are in-lane plus one
//                  shuffle)
//   O^T += V^T P^T (P feeds the MFMA straight from the S^T accumulator; the key
//                  order inside the contraction is relabelled to match, and V is
//                  staged transposed so the relabelled reads are 8-byte runs)
// Each product is hi*hi + hi*lo + lo*hi, which keeps the scores and outputs at
// fp32 accuracy (the lo*lo term is below 2^-16 of the total).  A bf16 cache
// holds K and V exactly in bf16, so their lo parts vanish: the tiles are staged
// as stored and each product is hi*hi + hi*lo (Q and P still split).
namespace {

constexpr int NQV = 128, MKV = 64;

__device__ __forceinline__ bf16x8 pack8(const uint32_t *h) {
    u32x4 v;
    v[0] = h[0] | (h[1] << 16); v[1] = h[2] | (h[3] << 16);
    v[2] = h[4] | (h[5] << 16); v[3] = h[6] | (h[7] << 16);
    return __builtin_bit_cast(bf16x8, v);
}

template <int HD, int G, int KT, bool GEN>
__global__ void __launch_bounds__(256, 2) attn_prefill_mfma_kernel(
    int T, int start_pos, int slot, const float *__restrict__ q, const void *__restrict__ kc,
    const void *__restrict__ vc, int nh, int nkv, int max_seq, int window, int ring_mod,
    const void *__restrict__ ck, const void *__restrict__ cv, u16 *__restrict__ o_hi, u16 *__restrict__ o_lo,
    float *__restrict__ o_f32) {
    constexpr int ROWS = NQV / G;
    constexpr int KLD = HD + 8;     // u16 per K row in LDS
    constexpr int VLD = MKV + 4;    // u16 per transposed V row (136 bytes)
    constexpr int KS = HD / 16;     // MFMA k-steps over head_dim
    constexpr int DT = HD / 32;     // output dim tiles
    __shared__ __attribute__((aligned(16))) u16 sKh[MKV * KLD];
    constexpr bool KB = KT == KV_BF16;
    __shared__ __attribute__((aligned(16))) u16 sKl[KB ? 8 : MKV * KLD];
    __shared__ __attribute__((aligned(16))) u16 sVh[HD * VLD];
    __shared__ __attribute__((aligned(16))) u16 sVl[KB ? 8 : HD * VLD];

    // blocks are dispatched in linear order (x fastest): walk the row blocks
    // from the longest (last rows) down, all kv heads of one row block together,
    // so the longest blocks start first on every CU
    const int lin = blockIdx.x + blockIdx.y * gridDim.x;
    const int kvh = lin % gridDim.y;
    const int rb = gridDim.x - 1 - lin / gridDim.y;
    const int t0 = rb * ROWS;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int ql = lane & 31, hh = lane >> 5;
    const int qv = wv * 32 + ql;
    const int row = qv / G, g = qv % G;
    const int t = t0 + row;
    const bool live = row < ROWS && t < T;
    const int qpos = live ? start_pos + t : -1;
    const int h = kvh * G + g;

    // Q^T operand (B of S^T): lane (q + 32hh), k-step s -> dims 16s + 8hh .. +8
    bf16x8 qh[KS], qlo[KS];
    {
        const float *qp = q + (size_t)(live ? t : 0) * nh * HD + (size_t)h * HD + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; s++) {
            uint32_t hb[8], lb[8];
            const float4 a = *reinterpret_cast<const float4 *>(qp + 16 * s);
            const float4 b = *reinterpret_cast<const float4 *>(qp + 16 * s + 4);
            const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; j++) split_bf16(live ? f[j] : 0.f, hb[j], lb[j]);
            qh[s] = pack8(hb);
            qlo[s] = pack8(lb);
        }
    }
    const float zero16v = 0.f;
    floatx16 o[DT];
#pragma unroll
    for (int d = 0; d < DT; d++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[d][e] = zero16v;
    float m = -INFINITY, l = 0.f;
    const float scale = 1.0f / sqrtf((float)HD);

    // largest query position of the wave and of the block
    int wmax = qpos;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wmax = max(wmax, __shfl_xor(wmax, off, WAVE));
    const int last_pos = start_pos + min(T, t0 + ROWS) - 1;
    // GEN: positions may lie before the window (ring past its size)
    const int first_key = GEN && window ? max(0, start_pos + t0 - window + 1) : 0;
    const int lo_q = GEN && window ? qpos - window + 1 : 0;  // this lane's query's oldest key
    const size_t head_base = ((size_t)slot * nkv + kvh) * max_seq;

    for (int kb = first_key; kb <= last_pos; kb += MKV) {
        __syncthreads();
        // K tile -> [key][dim] hi/lo; V tile -> transposed [dim][key] hi/lo
        auto krow = [&](int j) { return kv_row<HD, KT, GEN>(kc, ck, head_base, j, start_pos, ring_mod, nkv, kvh); };
        auto vrow = [&](int j) { return kv_row<HD, KT, GEN>(vc, cv, head_base, j, start_pos, ring_mod, nkv, kvh); };
        if constexpr (KB) {
            for (int i = tid; i < MKV * HD / 8; i += 256) {
                const int key = i / (HD / 8), c8 = i % (HD / 8);
                const int j = kb + key;
                u32x4 kv = {0u, 0u, 0u, 0u};
                if (j <= last_pos) kv = *reinterpret_cast<const u32x4 *>(krow(j) + 16 * c8);
                *reinterpret_cast<u32x4 *>(sKh + key * KLD + 8 * c8) = kv;
            }
            for (int i = tid; i < (MKV / 2) * HD / 8; i += 256) {
                const int kp = i / (HD / 8), c8 = i % (HD / 8);
                const int j = kb + 2 * kp;
                u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = v0;
                if (j <= last_pos) v0 = *reinterpret_cast<const u32x4 *>(vrow(j) + 16 * c8);
                if (j + 1 <= last_pos) v1 = *reinterpret_cast<const u32x4 *>(vrow(j + 1) + 16 * c8);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    // dims 8c8+2e (low halves) and 8c8+2e+1 (high halves)
                    *reinterpret_cast<uint32_t *>(sVh + (8 * c8 + 2 * e) * VLD + 2 * kp) =
                        (v0[e] & 0xFFFFu) | (v1[e] << 16);
                    *reinterpret_cast<uint32_t *>(sVh + (8 * c8 + 2 * e + 1) * VLD + 2 * kp) =
                        (v0[e] >> 16) | (v1[e] & 0xFFFF0000u);
                }
            }
        } else {
            for (int i = tid; i < MKV * HD / 4; i += 256) {
                const int key = i / (HD / 4), c4 = i % (HD / 4);
                const int j = kb + key;
                float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (j <= last_pos) kv = kv_load4<KT, HD>(krow(j), 4 * c4);
                uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
                split_bf16(kv.x, h0, l0); split_bf16(kv.y, h1, l1); split_bf16(kv.z, h2, l2); split_bf16(kv.w, h3, l3);
                *reinterpret_cast<uint2 *>(sKh + key * KLD + 4 * c4) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
                *reinterpret_cast<uint2 *>(sKl + key * KLD + 4 * c4) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
            }
            for (int i = tid; i < (MKV / 2) * HD / 4; i += 256) {
                const int kp = i / (HD / 4), c4 = i % (HD / 4);
                const int j = kb + 2 * kp;
                float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
                if (j <= last_pos) v0 = kv_load4<KT, HD>(vrow(j), 4 * c4);
                if (j + 1 <= last_pos) v1 = kv_load4<KT, HD>(vrow(j + 1), 4 * c4);
                const float a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    uint32_t ha, la, hb, lb;
                    split_bf16(a0[e], ha, la);
                    split_bf16(a1[e], hb, lb);
                    *reinterpret_cast<uint32_t *>(sVh + (4 * c4 + e) * VLD + 2 * kp) = ha | (hb << 16);
                    *reinterpret_cast<uint32_t *>(sVl + (4 * c4 + e) * VLD + 2 * kp) = la | (lb << 16);
                }
            }
        }
        __syncthreads();
        if (kb > wmax) continue;  // every query of this wave is before the tile

        // S^T for the 64 keys: two 32-key sub-tiles
        floatx16 sc[2];
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
#pragma unroll
            for (int e = 0; e < 16; e++) sc[kt][e] = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < KS; s2++) {
                const int off = (kt * 32 + ql) * KLD + 16 * s2 + 8 * hh;
                const bf16x8 kh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sKh + off));
                sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[s2], sc[kt], 0, 0, 0);
                sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qlo[s2], sc[kt], 0, 0, 0);
                if constexpr (!KB) {
                    const bf16x8 klo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sKl + off));
                    sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo, qh[s2], sc[kt], 0, 0, 0);
                }
            }
        }
        // lane holds keys kb + kt*32 + (e/4)*8 + 4hh + e%4 of query qpos
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int key = kb + kt * 32 + (e / 4) * 8 + 4 * hh + (e % 4);
                const float v = (key <= qpos && (!GEN || key >= lo_q)) ? sc[kt][e] * scale : -INFINITY;
                sc[kt][e] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
        const float mnew = fmaxf(m, mx);
        const float corr = (mnew == -INFINITY) ? 1.f : expf(m - mnew);
        float ps = 0.f;
        uint32_t ph[2][16], plo[2][16];
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const float pe = (sc[kt][e] == -INFINITY) ? 0.f : expf(sc[kt][e] - mnew);
                ps += pe;
                split_bf16(pe, ph[kt][e], plo[kt][e]);
            }
        ps += __shfl_xor(ps, 32, WAVE);
        l = l * corr + ps;
        m = mnew;
#pragma unroll
        for (int d = 0; d < DT; d++)
#pragma unroll
            for (int e = 0; e < 16; e++) o[d][e] *= corr;
        // O^T += V^T P^T over 4 k-steps of 16 keys; step ks uses the lane's
        // values e = (ks%2)*8 + j of sub-tile ks/2, i.e. keys 16ks + (j/4)*8 + 4hh + j%4
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const bf16x8 bh = pack8(&ph[ks / 2][(ks % 2) * 8]);
            const bf16x8 bl = pack8(&plo[ks / 2][(ks % 2) * 8]);
#pragma unroll
            for (int d = 0; d < DT; d++) {
                const int vrow = (d * 32 + ql) * VLD + 16 * ks + 4 * hh;
                const uint2 h0 = *reinterpret_cast<const uint2 *>(sVh + vrow);
                const uint2 h1 = *reinterpret_cast<const uint2 *>(sVh + vrow + 8);
                const u32x4 vh4 = {h0.x, h0.y, h1.x, h1.y};
                const bf16x8 ah = __builtin_bit_cast(bf16x8, vh4);
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, o[d], 0, 0, 0);
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, o[d], 0, 0, 0);
                if constexpr (!KB) {
                    const uint2 l0 = *reinterpret_cast<const uint2 *>(sVl + vrow);
                    const uint2 l1 = *reinterpret_cast<const uint2 *>(sVl + vrow + 8);
                    const u32x4 vl4 = {l0.x, l0.y, l1.x, l1.y};
                    const bf16x8 al = __builtin_bit_cast(bf16x8, vl4);
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, o[d], 0, 0, 0);
                }
            }
        }
    }
    if (!live) return;
    const float inv = 1.0f / l;
    const size_t base = (size_t)t * nh * HD + (size_t)h * HD;
#pragma unroll
    for (int d = 0; d < DT; d++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const int dim = d * 32 + gq * 8 + 4 * hh;
#pragma unroll
            for (int e = 0; e < 4; e++) store_out(o[d][4 * gq + e] * inv, base + dim + e, o_hi, o_lo, o_f32);
        }
}

template <int HD, int KT, bool GEN>
bool launch_prefill_mfma_hd(hipStream_t st, int G, int T, int start_pos, int slot, const float *q, const void *kc,
                            const void *vc, int nh, int nkv, int max_seq, int window, int ring_mod, const void *ck,
                            const void *cv, u16 *o_hi, u16 *o_lo, float *o_f32) {
#define APM(GG) hipLaunchKernelGGL((attn_prefill_mfma_kernel<HD, GG, KT, GEN>), dim3((T + NQV / GG - 1) / (NQV / GG), nkv), \
                                   dim3(256), 0, st, T, start_pos, slot, q, kc, vc, nh, nkv, max_seq, window, \
                                   ring_mod, ck, cv, o_hi, o_lo, o_f32)
    switch (G) {
        case 1: APM(1); return true;
        case 2: APM(2); return true;
        case 3: APM(3); return true;
        case 4: APM(4); return true;
        case 5: APM(5); return true;
        case 6: APM(6); return true;
        case 7: APM(7); return true;
        case 8: APM(8); return true;
    }
#undef APM
    return false;
}

}  // namespace

void launch_attn_prefill(hipStream_t st, int T, int start_pos, int slot, const float *q, const void *kc,
                         const void *vc, int kv_kind, int nh, int nkv, int hd, int max_seq, int window, int ring,
                         const void *ck, const void *cv, u16 *o_hi, u16 *o_lo, float *o_f32) {
    if (T <= 0) return;
    const int G = nh / nkv;
    const int ring_mod = ring ? max_seq : 0;
    dim3 grid((T + BQ - 1) / BQ, nkv);
    // the general form (ring slots, chunk buffers, window bound) only for a
    // chunk held back from the cache; otherwise slot == position
#define LM(HD, KT, GEN) launch_prefill_mfma_hd<HD, KT, GEN>(st, G, T, start_pos, slot, q, kc, vc, nh, nkv, max_seq, \
                                                            window, ring_mod, ck, cv, o_hi, o_lo, o_f32)
#define LF(HD, KT, GEN) launch_prefill_hd<HD, 1, KT, GEN>(st, G, grid, T, start_pos, slot, q, kc, vc, nh, nkv, \
                                                          max_seq, window, ring_mod, ck, cv, o_hi, o_lo, o_f32)
#define PICKK(KT, GEN)                  \
    if (hd == 128) LM(128, KT, GEN);        \
    else if (hd == 64) LM(64, KT, GEN);     \
    else LF(16, KT, GEN);
#define PICK(GEN)                                                  \
    if (kv_kind == KV_BF16) { PICKK(KV_BF16, GEN) }                \
    else if (kv_kind == KV_F24) { PICKK(KV_F24, GEN) }             \
    else { PICKK(KV_F32, GEN) }
    if (ck) {
        PICK(true)
    } else {
        PICK(false)
    }
#undef PICK
#undef PICKK
#undef LM
#undef LF
}
