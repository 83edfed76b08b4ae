// Decode attention: softmax(q k^T / sqrt(hd)) v over the cached positions of
// each row's sequence (zLLM "The Algorithm Layer", section 2; Pantheon "Llama
// Forward Pass", "Grouped Query Attention": query head h reads kv head
// h*n_kv/n_head), with the one-pass online softmax of rml "The decoder",
// section "Attend": a running maximum and normaliser, the partial output
// rescaled when the maximum grows, no score array.
//
// Split-KV: grid (splits, kv heads, rows).  A block streams one kv head's K/V
// rows of one split once from HBM and applies them to all G query heads of the
// group.  LP lanes share one position (each lane 8 dims, two float4 loads per
// row); every lane group keeps its own softmax state over the positions it
// visits, and the groups are merged at the end (in-wave by shuffles, across
// waves through LDS), then across splits by a merge kernel.
//
// Ring cache: softmax does not depend on key order, and keys are stored already
// rotated, so the readable slots [0, min(pos+1, max_seq)) are read as one
// contiguous range whatever the wrap (Pantheon, "Sliding Window (Mistral)").
#include "common.h"
#include "kernels.h"

namespace {

constexpr int NB = 4;  // positions per lane group per iteration (loads in flight)

// K/V rows are read once per decode step: non-temporal loads stream them past
// the caches.
__device__ __forceinline__ float4 ntload4(const float *p) {
    const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store_out(float v, size_t off, u16 *o_hi, u16 *o_lo, float *o_f32) {
    if (o_f32) o_f32[off] = v;
    if (o_hi) {
        uint32_t h, l;
        split_bf16(v, h, l);
        o_hi[off] = (u16)h;
        o_lo[off] = (u16)l;
    }
}

template <int HD, int G>
__global__ void __launch_bounds__(256) attn_decode_kernel(
    const float *__restrict__ q, const float *__restrict__ kc, const float *__restrict__ vc,
    const int32_t *__restrict__ pos, const int32_t *__restrict__ slot, int nh, int nkv, int max_seq,
    int splits, float *__restrict__ part, u16 *__restrict__ o_hi, u16 *__restrict__ o_lo,
    float *__restrict__ o_f32) {
    constexpr int LP = HD / 8;             // lanes per position
    constexpr int PPW = WAVE / LP;         // positions per wave
    constexpr int NG = 4 * PPW;            // lane groups per block
    __shared__ float sm[4][G], sl[4][G];
    __shared__ float sacc[4][G][HD];

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int u = lane % LP, pg = lane / LP;
    const int gid = wv * PPW + pg;

    const int p = pos[b];
    const int nread = min(p + 1, max_seq);
    const int chunk = (nread + splits - 1) / splits;
    const int beg = split * chunk;
    const int end = min(nread, beg + chunk);

    const size_t head_base = ((size_t)slot[b] * nkv + kvh) * max_seq;
    const float *K = kc + head_base * HD;
    const float *V = vc + head_base * HD;
    const float scale = 1.0f / sqrtf((float)HD);

    float qr[G][8];
#pragma unroll
    for (int g = 0; g < G; g++) {
        const float *qh = q + (size_t)b * nh * HD + (size_t)(kvh * G + g) * HD;
        const float4 a = *reinterpret_cast<const float4 *>(qh + 4 * u);
        const float4 c = *reinterpret_cast<const float4 *>(qh + 4 * LP + 4 * u);
        qr[g][0] = a.x; qr[g][1] = a.y; qr[g][2] = a.z; qr[g][3] = a.w;
        qr[g][4] = c.x; qr[g][5] = c.y; qr[g][6] = c.z; qr[g][7] = c.w;
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; g++) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) acc[g][i] = 0.f;
    }

    for (int base = beg; base < end; base += NG * NB) {
        float4 k0[NB], k1[NB];
        bool valid[NB];
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int j = base + i * NG + gid;
            valid[i] = j < end;
            const int jj = valid[i] ? j : beg;
            k0[i] = ntload4(K + (size_t)jj * HD + 4 * u);
            k1[i] = ntload4(K + (size_t)jj * HD + 4 * LP + 4 * u);
        }
        float4 v0[NB], v1[NB];
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int j = base + i * NG + gid;
            const int jj = valid[i] ? j : beg;
            v0[i] = ntload4(V + (size_t)jj * HD + 4 * u);
            v1[i] = ntload4(V + (size_t)jj * HD + 4 * LP + 4 * u);
        }
        float s[NB][G];
#pragma unroll
        for (int i = 0; i < NB; i++)
#pragma unroll
            for (int g = 0; g < G; g++) {
                float d = qr[g][0] * k0[i].x + qr[g][1] * k0[i].y + qr[g][2] * k0[i].z + qr[g][3] * k0[i].w +
                          qr[g][4] * k1[i].x + qr[g][5] * k1[i].y + qr[g][6] * k1[i].z + qr[g][7] * k1[i].w;
#pragma unroll
                for (int o = LP / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, WAVE);
                s[i][g] = valid[i] ? d * scale : -INFINITY;
            }
#pragma unroll
        for (int g = 0; g < G; g++) {
            float mx = m[g];
#pragma unroll
            for (int i = 0; i < NB; i++) mx = fmaxf(mx, s[i][g]);
            if (mx == -INFINITY) continue;
            const float corr = expf(m[g] - mx);
            m[g] = mx;
            float pe[NB];
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < NB; i++) {
                pe[i] = expf(s[i][g] - mx);
                ps += pe[i];
            }
            l[g] = l[g] * corr + ps;
#pragma unroll
            for (int e = 0; e < 8; e++) acc[g][e] *= corr;
#pragma unroll
            for (int i = 0; i < NB; i++) {
                acc[g][0] += pe[i] * v0[i].x; acc[g][1] += pe[i] * v0[i].y;
                acc[g][2] += pe[i] * v0[i].z; acc[g][3] += pe[i] * v0[i].w;
                acc[g][4] += pe[i] * v1[i].x; acc[g][5] += pe[i] * v1[i].y;
                acc[g][6] += pe[i] * v1[i].z; acc[g][7] += pe[i] * v1[i].w;
            }
        }
    }

    // merge the PPW lane groups of the wave
#pragma unroll
    for (int o = LP; o < WAVE; o <<= 1) {
#pragma unroll
        for (int g = 0; g < G; g++) {
            const float mo = __shfl_xor(m[g], o, WAVE);
            const float lo = __shfl_xor(l[g], o, WAVE);
            const float mx = fmaxf(m[g], mo);
            const float a = mx == -INFINITY ? 0.f : expf(m[g] - mx);
            const float bb = mx == -INFINITY ? 0.f : expf(mo - mx);
            l[g] = l[g] * a + lo * bb;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float ao = __shfl_xor(acc[g][e], o, WAVE);
                acc[g][e] = acc[g][e] * a + ao * bb;
            }
            m[g] = mx;
        }
    }
    if (pg == 0) {
#pragma unroll
        for (int g = 0; g < G; g++) {
            if (u == 0) { sm[wv][g] = m[g]; sl[wv][g] = l[g]; }
#pragma unroll
            for (int e = 0; e < 4; e++) {
                sacc[wv][g][4 * u + e] = acc[g][e];
                sacc[wv][g][4 * LP + 4 * u + e] = acc[g][4 + e];
            }
        }
    }
    __syncthreads();
    // merge the 4 waves: thread (g, i) handles one output element
    for (int idx = threadIdx.x; idx < G * HD; idx += blockDim.x) {
        const int g = idx / HD, i = idx % HD;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; w++) mx = fmaxf(mx, sm[w][g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const float f = mx == -INFINITY ? 0.f : expf(sm[w][g] - mx);
            L += sl[w][g] * f;
            A += sacc[w][g][i] * f;
        }
        const int h = kvh * G + g;
        if (splits == 1) {
            store_out(A / L, (size_t)b * nh * HD + (size_t)h * HD + i, o_hi, o_lo, o_f32);
        } else {
            float *dst = part + (((size_t)b * nh + h) * splits + split) * (HD + 2);
            dst[i] = A;
            if (i == 0) { dst[HD] = mx; dst[HD + 1] = L; }
        }
    }
}

__global__ void attn_merge_kernel(int nh, int hd, int splits, const float *__restrict__ part,
                                  u16 *__restrict__ o_hi, u16 *__restrict__ o_lo, float *__restrict__ o_f32) {
    const int h = blockIdx.x, b = blockIdx.y;
    const float *src = part + ((size_t)b * nh + h) * splits * (hd + 2);
    float mx = -INFINITY;
    for (int s = 0; s < splits; s++) mx = fmaxf(mx, src[s * (hd + 2) + hd]);
    for (int i = threadIdx.x; i < hd; i += blockDim.x) {
        float L = 0.f, A = 0.f;
        for (int s = 0; s < splits; s++) {
            const float ms = src[s * (hd + 2) + hd];
            const float f = ms == -INFINITY ? 0.f : expf(ms - mx);
            L += src[s * (hd + 2) + hd + 1] * f;
            A += src[s * (hd + 2) + i] * f;
        }
        store_out(A / L, (size_t)b * nh * hd + (size_t)h * hd + i, o_hi, o_lo, o_f32);
    }
}

template <int HD>
bool launch_decode_hd(hipStream_t st, int G, dim3 grid, const float *q, const float *kc, const float *vc,
                      const int32_t *pos, const int32_t *slot, int nh, int nkv, int max_seq, int splits,
                      float *part, u16 *o_hi, u16 *o_lo, float *o_f32) {
#define AD(GG) hipLaunchKernelGGL((attn_decode_kernel<HD, GG>), grid, dim3(256), 0, st, q, kc, vc, pos, slot, \
                                  nh, nkv, max_seq, splits, part, o_hi, o_lo, o_f32)
    switch (G) {
        case 1: AD(1); return true;
        case 2: AD(2); return true;
        case 3: AD(3); return true;
        case 4: AD(4); return true;
        case 5: AD(5); return true;
        case 6: AD(6); return true;
        case 7: AD(7); return true;
        case 8: AD(8); return true;
    }
#undef AD
    return false;
}

}  // namespace

int attn_decode_splits(int B, int nkv, int readable, int hd, int G) {
    // fill the resident-block slots once (a second partial round would leave
    // the memory system idle), with at least 128 positions per split
    static int occ_cache[3] = {0, 0, 0};
    const int which = hd == 128 ? 0 : hd == 64 ? 1 : 2;
    if (!occ_cache[which]) {
        int occ = 0;
        const void *fn = hd == 128 ? (const void *)attn_decode_kernel<128, 4>
                       : hd == 64  ? (const void *)attn_decode_kernel<64, 4>
                                   : (const void *)attn_decode_kernel<16, 4>;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 256, 0) != hipSuccess || occ <= 0) occ = 2;
        occ_cache[which] = occ;
    }
    (void)G;
    const int slots = occ_cache[which] * num_cus();
    int s = slots / (B * nkv);
    const int maxs = (readable + 127) / 128;
    if (s > maxs) s = maxs;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    return s;
}

void launch_attn_decode(hipStream_t st, int B, const float *q, const float *kc, const float *vc,
                        const int32_t *pos, const int32_t *slot, int nh, int nkv, int hd, int max_seq,
                        int window, int splits, float *part, u16 *o_hi, u16 *o_lo, float *o_f32) {
    (void)window;
    if (B <= 0) return;
    const int G = nh / nkv;
    dim3 grid(splits, nkv, B);
    if (hd == 128) launch_decode_hd<128>(st, G, grid, q, kc, vc, pos, slot, nh, nkv, max_seq, splits, part, o_hi, o_lo, o_f32);
    else if (hd == 64) launch_decode_hd<64>(st, G, grid, q, kc, vc, pos, slot, nh, nkv, max_seq, splits, part, o_hi, o_lo, o_f32);
    else launch_decode_hd<16>(st, G, grid, q, kc, vc, pos, slot, nh, nkv, max_seq, splits, part, o_hi, o_lo, o_f32);
    if (splits > 1)
        hipLaunchKernelGGL(attn_merge_kernel, dim3(nh, B), dim3(hd < 64 ? 64 : hd), 0, st, nh, hd, splits, part,
                           o_hi, o_lo, o_f32);
}

