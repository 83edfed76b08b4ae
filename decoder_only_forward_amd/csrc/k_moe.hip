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
constexpr int NT = 256;

__global__ void __launch_bounds__(NT) moe_route_kernel(int T, int E, int k, Partials lg, int32_t *__restrict__ ids,
                                                       float *__restrict__ w, float *__restrict__ rcap,
                                                       int32_t *__restrict__ icap, int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ offsets, int32_t *__restrict__ pairs) {
    __shared__ int cnt[NT][MAXE];
    __shared__ int off[MAXE + 1];
    const int tid = threadIdx.x;
    // 1. per token: EP (E rounded up to a power of two) lanes per token, lane e
    //    < E sums expert e's split partials, then the token's first lane forms
    //    the softmax, the top-k and the renormalised weights
    const int lane = tid % WAVE, wv = tid / WAVE;
    int EP = 1;
    while (EP < E) EP <<= 1;
    const int tpw = WAVE / EP;   // tokens per wave per pass
    for (int base = wv * tpw; base < T; base += (NT / WAVE) * tpw) {
        const int t = base + lane / EP, e0 = lane % EP;
        float v = -INFINITY;
        if (t < T && e0 < E) {
            v = sum_splits(lg.p, lg.S, lg.stride, (size_t)t * lg.ld + e0);
            if (rcap) rcap[(size_t)t * E + e0] = v;
        }
        float p[MAXE];
#pragma unroll
        for (int e = 0; e < MAXE; e++) p[e] = __shfl(v, (lane & ~(EP - 1)) + (e & (EP - 1)), WAVE);
        if (e0 != 0 || t >= T) continue;
        float mx = -INFINITY;
        for (int e = 0; e < E; e++) mx = fmaxf(mx, p[e]);
        float z = 0.f;
        for (int e = 0; e < E; e++) { p[e] = expf(p[e] - mx); z += p[e]; }
        for (int e = 0; e < E; e++) p[e] = p[e] / z;
        uint32_t taken = 0;
        float total = 0.f;
        int sel[MAXE];
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!(taken >> e & 1u) && (best < 0 || p[e] > p[best])) best = e;
            taken |= 1u << best;
            sel[j] = best;
            total += p[best];
        }
        for (int j = 0; j < k; j++) {
            ids[t * k + j] = sel[j];
            w[t * k + j] = p[sel[j]] / total;
            if (icap) icap[t * k + j] = sel[j];
        }
    }
    __syncthreads();
    // 2. stable counting sort of pair index t*k+j by expert: thread i < nthr
    //    counts a contiguous run of pairs, the per-expert scan walks the runs
    //    in order (only as many runs as there are pairs, for short decode rows)
    const int n = T * k;
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
        pairs[off[e] + cnt[tid][e]++] = i;
    }
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

__global__ void __launch_bounds__(256) moe_scatter_kernel(int d, const int32_t *__restrict__ pairs, Partials src,
                                                          float *__restrict__ y) {
    const int i = blockIdx.x;
    const int dst = pairs[i];
    for (int c = threadIdx.x; c < d / 4; c += blockDim.x) {
        const float4 v = sum_splits4(src.p, src.S, src.stride, (size_t)i * src.ld + 4 * c);
        *reinterpret_cast<float4 *>(y + (size_t)dst * d + 4 * c) = v;
    }
}
}  // namespace

void launch_moe_route(hipStream_t st, int T, int E, int k, Partials logits, int32_t *ids, float *w,
                      float *router_cap, int32_t *ids_cap, int32_t *counts, int32_t *offsets, int32_t *pairs) {
    if (T <= 0) return;
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(NT), 0, st, T, E, k, logits, ids, w, router_cap, ids_cap,
                       counts, offsets, pairs);
}

void launch_moe_gather(hipStream_t st, int T, int k, int d, const int32_t *pairs, const u16 *src_hi,
                       const u16 *src_lo, const float *src_f32, u16 *dst_hi, u16 *dst_lo, float *dst_f32) {
    if (T <= 0) return;
    hipLaunchKernelGGL(moe_gather_kernel, dim3(T * k), dim3(256), 0, st, k, d, pairs, src_hi, src_lo, src_f32,
                       dst_hi, dst_lo, dst_f32);
}

void launch_moe_scatter(hipStream_t st, int n_pairs, int d, const int32_t *pairs, Partials src, float *y) {
    if (n_pairs <= 0) return;
    hipLaunchKernelGGL(moe_scatter_kernel, dim3(n_pairs), dim3(256), 0, st, d, pairs, src, y);
}
