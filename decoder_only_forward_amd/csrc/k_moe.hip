// Mixture-of-experts FFN (Pantheon "Llama Forward Pass", section "Mixture of
// Experts (Mixtral)"; rml "The decoder", section "Mixture of experts"):
// router logits -> softmax over all experts -> top-k by repeated selection,
// ties to the lower id -> weights p_e / (sum of chosen p) -> weighted sum of the
// chosen experts' SwiGLU outputs.
//
// Execution groups (token, slot) pairs by expert (zLLM "The Algorithm Layer",
// section 4: grouped expert execution for multi-token prefill), so each
// selected expert's weights are read once per call and unselected experts are
// never touched.  The grouping is a stable counting sort: deterministic, no
// atomics on data.
#include "common.h"
#include "kernels.h"

namespace {
constexpr int MAXE = 32;
constexpr int MAXK = 8;
constexpr int NT = 256;

// 1. Per token (one wave each): the router logits, from split partials (lg.p)
//    or computed here from the router weights wr [E][d] (bf16) and the token's
//    (hi, lo) activation row; then softmax over the E experts, the top k by
//    repeated selection (ties to the lower id) and the weights p_e / (sum of the
//    chosen p).  Every lane holds every logit; all register indices are
//    compile-time constants.
__device__ __forceinline__ void topk_token(int t, int E, int k, const Partials &lg, const u16 *__restrict__ wr,
                                           const u16 *__restrict__ ah, const u16 *__restrict__ al, int d, int lda,
                                           int32_t *__restrict__ ids, float *__restrict__ w,
                                           float *__restrict__ rcap, int32_t *__restrict__ icap) {
    const int lane = threadIdx.x % WAVE;
    float p[MAXE];
    if (wr) {
        float acc[MAXE];
#pragma unroll
        for (int e = 0; e < MAXE; e++) acc[e] = 0.f;
        const u16 *xh = ah + (size_t)t * lda, *xl = al + (size_t)t * lda;
        for (int k0 = lane * 8; k0 < d; k0 += WAVE * 8) {
            const u32x4 h = *reinterpret_cast<const u32x4 *>(xh + k0);
            const u32x4 l = *reinterpret_cast<const u32x4 *>(xl + k0);
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                x[2 * i] = bf16_bits_to_f32(h[i] & 0xFFFFu) + bf16_bits_to_f32(l[i] & 0xFFFFu);
                x[2 * i + 1] = __uint_as_float(h[i] & 0xFFFF0000u) + __uint_as_float(l[i] & 0xFFFF0000u);
            }
#pragma unroll
            for (int e = 0; e < MAXE; e++) {
                if (e >= E) break;
                const u32x4 wv = *reinterpret_cast<const u32x4 *>(wr + (size_t)e * d + k0);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    acc[e] += bf16_bits_to_f32(wv[i] & 0xFFFFu) * x[2 * i];
                    acc[e] += __uint_as_float(wv[i] & 0xFFFF0000u) * x[2 * i + 1];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < MAXE; e++) p[e] = e < E ? wave_sum(acc[e]) : -INFINITY;
    } else {
        const float v = lane < E ? sum_splits(lg.p, lg.S, lg.stride, (size_t)t * lg.ld + lane) : -INFINITY;
#pragma unroll
        for (int e = 0; e < MAXE; e++) p[e] = __shfl(v, e, WAVE);
    }
    if (rcap) {
        float v = 0.f;
#pragma unroll
        for (int e = 0; e < MAXE; e++)
            if (lane == e) v = p[e];
        if (lane < E) rcap[(size_t)t * E + lane] = v;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < MAXE; e++)
        if (e < E) mx = fmaxf(mx, p[e]);
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < MAXE; e++)
        if (e < E) {
            p[e] = expf(p[e] - mx);
            z += p[e];
        }
#pragma unroll
    for (int e = 0; e < MAXE; e++)
        if (e < E) p[e] = p[e] / z;
    uint32_t taken = 0;
    float total = 0.f;
    int sel[MAXK];
    float selp[MAXK];
#pragma unroll
    for (int j = 0; j < MAXK; j++) {
        sel[j] = 0;
        selp[j] = 0.f;
        if (j >= k) continue;
        int best = -1;
        float bv = 0.f;
#pragma unroll
        for (int e = 0; e < MAXE; e++)
            if (e < E && !(taken >> e & 1u) && (best < 0 || p[e] > bv)) {
                best = e;
                bv = p[e];
            }
        taken |= 1u << best;
        sel[j] = best;
        selp[j] = bv;
        total += bv;
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < MAXK; j++)
            if (j < k) {
                ids[t * k + j] = sel[j];
                w[t * k + j] = selp[j] / total;
                if (icap) icap[t * k + j] = sel[j];
            }
    }
}

__global__ void __launch_bounds__(NT) moe_topk_kernel(int T, int E, int k, Partials lg, const u16 *__restrict__ wr,
                                                      const u16 *__restrict__ ah, const u16 *__restrict__ al,
                                                      int d, int lda, int32_t *__restrict__ ids,
                                                      float *__restrict__ w, float *__restrict__ rcap,
                                                      int32_t *__restrict__ icap) {
    const int t = blockIdx.x * (NT / WAVE) + threadIdx.x / WAVE;
    if (t >= T) return;
    topk_token(t, E, k, lg, wr, ah, al, d, lda, ids, w, rcap, icap);
}

// 2. Stable counting sort of pair index t*k+j by expert (one block): thread
//    i < nthr counts a contiguous run of pairs, the per-expert scan walks the
//    runs in order (only as many runs as there are pairs, for short decode rows).
//    pairs[r] = the pair at grouped row r, inv[pair] = r.
__device__ __forceinline__ void sort_pairs(int n, int E, const int32_t *__restrict__ ids,
                                           int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                           int32_t *__restrict__ pairs, int32_t *__restrict__ inv) {
    __shared__ int cnt[NT][MAXE];
    __shared__ int off[MAXE + 1];
    const int tid = threadIdx.x;
    const int nthr = n < NT ? n : NT;
    const int per = (n + nthr - 1) / nthr;
    const int lo = tid * per, hi = min(n, lo + per);
    for (int e = 0; e < E; e++) cnt[tid][e] = 0;
    for (int i = lo; i < hi; i++) cnt[tid][ids[i]]++;
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int i = 0; i < nthr; i++) {
            const int c = cnt[i][tid];
            cnt[i][tid] = run;
            run += c;
        }
        counts[tid] = run;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; e++) { off[e] = run; run += counts[e]; }
        off[E] = run;
        for (int e = 0; e <= E; e++) offsets[e] = off[e];
    }
    __syncthreads();
    for (int i = lo; i < hi; i++) {
        const int e = ids[i];
        const int r = off[e] + cnt[tid][e]++;
        pairs[r] = i;
        inv[i] = r;
    }
}

__global__ void __launch_bounds__(NT) moe_sort_kernel(int n, int E, const int32_t *__restrict__ ids,
                                                      int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ pairs, int32_t *__restrict__ inv) {
    sort_pairs(n, E, ids, counts, offsets, pairs, inv);
}

// A few decode rows (at most one per wave): both steps in one block, then the
// sort after a block barrier (which makes the block's expert ids visible to
// all its threads).  One launch fewer: Mixtral-8x7B decode at B = 1 1.2 %
// faster; at B = 16 the one block's four passes over the tokens cost more
// than the second launch (3 % slower), so more rows take the two kernels.
__global__ void __launch_bounds__(NT) moe_route_block_kernel(int T, int E, int k, Partials lg,
                                                             int32_t *__restrict__ ids, float *__restrict__ w,
                                                             float *__restrict__ rcap, int32_t *__restrict__ icap,
                                                             int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ pairs, int32_t *__restrict__ inv) {
    for (int t = threadIdx.x / WAVE; t < T; t += NT / WAVE)
        topk_token(t, E, k, lg, nullptr, nullptr, nullptr, 0, 0, ids, w, rcap, icap);
    __syncthreads();
    sort_pairs(T * k, E, ids, counts, offsets, pairs, inv);
}

__global__ void __launch_bounds__(256) moe_gather_kernel(int k, int d, const int32_t *__restrict__ pairs,
                                                         const u16 *__restrict__ sh, const u16 *__restrict__ sl,
                                                         const float *__restrict__ sf, u16 *__restrict__ dh,
                                                         u16 *__restrict__ dl, float *__restrict__ df) {
    const int i = blockIdx.x;
    const int t = pairs[i] / k;
    for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
        if (sf)
            *reinterpret_cast<float4 *>(df + (size_t)i * d + 4 * c) =
                *reinterpret_cast<const float4 *>(sf + (size_t)t * d + 4 * c);
        if (sh) {
            *reinterpret_cast<uint2 *>(dh + (size_t)i * d + 4 * c) =
                *reinterpret_cast<const uint2 *>(sh + (size_t)t * d + 4 * c);
            *reinterpret_cast<uint2 *>(dl + (size_t)i * d + 4 * c) =
                *reinterpret_cast<const uint2 *>(sl + (size_t)t * d + 4 * c);
        }
    }
}

}  // namespace

void launch_moe_route(hipStream_t st, int T, int E, int k, Partials logits, const u16 *router_w, const u16 *a_hi,
                      const u16 *a_lo, int d, int lda, int32_t *ids, float *w, float *router_cap, int32_t *ids_cap,
                      int32_t *counts, int32_t *offsets, int32_t *pairs, int32_t *inv) {
    if (T <= 0) return;
    if (!router_w && T <= NT / WAVE) {
        hipLaunchKernelGGL(moe_route_block_kernel, dim3(1), dim3(NT), 0, st, T, E, k, logits, ids, w, router_cap,
                           ids_cap, counts, offsets, pairs, inv);
        return;
    }
    const int tpb = NT / WAVE;
    hipLaunchKernelGGL(moe_topk_kernel, dim3((T + tpb - 1) / tpb), dim3(NT), 0, st, T, E, k, logits, router_w, a_hi,
                       a_lo, d, lda, ids, w, router_cap, ids_cap);
    hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(NT), 0, st, T * k, E, ids, counts, offsets, pairs, inv);
}

void launch_moe_gather(hipStream_t st, int T, int k, int d, const int32_t *pairs, const u16 *src_hi,
                       const u16 *src_lo, const float *src_f32, u16 *dst_hi, u16 *dst_lo, float *dst_f32) {
    if (T <= 0) return;
    hipLaunchKernelGGL(moe_gather_kernel, dim3(T * k), dim3(256), 0, st, k, d, pairs, src_hi, src_lo, src_f32,
                       dst_hi, dst_lo, dst_f32);
}

