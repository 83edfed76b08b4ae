// Causal prefill attention on MFMA over pre-split K/V tiles.
//
// softmax(q k^T / sqrt(hd) + causal mask) v for the positions of one sequence
// (zLLM "The Algorithm Layer", section 2), query head h reading kv head
// h*n_kv/n_head (Pantheon "Llama Forward Pass", "Grouped Query Attention"),
// with the one-pass online softmax of rml "The decoder", section "Attend".
//
// Two kernels per layer:
//  1. kv_tile_kernel writes, once per layer, every 64-position tile of the
//     sequence's K/V as the exact image the attention kernel keeps in LDS:
//     K as bf16 (hi, lo) rows [key][dim] and V transposed, [dim][key], also
//     as (hi, lo); rows are padded so that MFMA operand reads of one lane group
//     fall in distinct banks.  A bf16 cache holds K and V exactly, so its image
//     has no lo halves.  The split and the transpose are then paid once per
//     K/V element instead of once per (element, query block).
//  2. attn_tiles_kernel: a block of 8 waves holds 256 query vectors ((row, head)
//     pairs of one kv group) and walks the key tiles up to its last query.  The
//     next tile's image goes from global memory straight into the other half of
//     a double-buffered LDS area (direct-to-LDS loads) while the current one is
//     multiplied: one barrier per tile.  Per wave (32 query vectors):
//       S^T = K Q^T    (32x32x16 MFMAs; lane q+32h owns 32 scores of query q)
//       O^T += V^T P^T (P straight from the S^T accumulator, keys relabelled
//                       to match the accumulator layout, V^T rows read as
//                       8-byte runs)
//     Each product is hi*hi + hi*lo + lo*hi (hi*hi + hi*lo with a bf16 cache,
//     whose lo part is zero), which keeps scores and outputs at fp32 accuracy.
//     q is scaled by log2(e)/sqrt(hd) before its split, so the softmax runs in
//     base 2 (one exp2 per weight); only tiles that reach past a wave's first
//     query position are masked.
//  A launch of fewer blocks than twice the CUs (few kv heads, a few hundred
//  to a few thousand rows: Qwen2.5-0.5B at 2048 tokens has 57 row blocks x 2
//  kv heads, whose causal lengths run from 1 to 32 tiles) splits the longer
//  row blocks' key tiles into chunks of at most `chunk` tiles, one block each;
//  a split row block's chunks write their unnormalised outputs with the
//  running maximum and normaliser, and attn_chunk_merge_kernel combines them
//  (the split-KV merge of the decode attention, over key chunks).
#include "common.h"
#include "kernels.h"
#include "kvcache.h"

namespace {

constexpr int TK = 64;          // keys per tile
constexpr int NTHR = 512;       // 8 waves
constexpr int NQV = 256;        // query vectors per block
constexpr float LOG2E = 1.4426950408889634f;

template <int HD, bool KB>
struct Img {
    static constexpr int KLD = HD + 8;          // u16 per K row
    static constexpr int VLD = TK + 4;          // u16 per transposed V row
    static constexpr int KH = 0;
    static constexpr int KL = TK * KLD;         // (absent with KB)
    static constexpr int VH = KB ? TK * KLD : 2 * TK * KLD;
    static constexpr int VL = VH + HD * VLD;    // (absent with KB)
    static constexpr int USED = KB ? TK * KLD + HD * VLD : 2 * (TK * KLD + HD * VLD);   // u16
    static constexpr int CHUNKS = (USED * 2 + 16 * NTHR - 1) / (16 * NTHR);            // 16-byte loads per thread
    static constexpr int BYTES = CHUNKS * 16 * NTHR;
};

__device__ __forceinline__ uint32_t bf16_rne(float x) { return f32_to_bf16_bits(x); }

// One tile (64 positions) of one kv head.  Positions >= npos are zero.  A
// 24-bit cache (KT = KV_F24) makes the fp32 cache's image: its rebuilt fp32
// words split exactly into the (hi, lo) pair.
template <int HD, int KT>
__global__ void __launch_bounds__(256) kv_tile_kernel(const void *__restrict__ kc, const void *__restrict__ vc,
                                                      int max_seq, int slot, int nkv, int npos, int ntiles,
                                                      u16 *__restrict__ img) {
    constexpr bool KB = KT == KV_BF16;
    using I = Img<HD, KB>;
    __shared__ float sv[TK][HD + 1];
    const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const size_t hb = ((size_t)slot * nkv + h) * max_seq;
    u16 *out = img + ((size_t)h * ntiles + j) * (I::BYTES / 2);
    const int p0 = j * TK;
    // K rows (and the V tile into LDS)
    for (int i = tid; i < TK * (HD / 4); i += 256) {
        const int r = i / (HD / 4), c4 = i % (HD / 4);
        const int p = p0 + r;
        float kx[4] = {0.f, 0.f, 0.f, 0.f}, vx[4] = {0.f, 0.f, 0.f, 0.f};
        if (p < npos) {
            if constexpr (KB) {
                const uint2 kb2 = *reinterpret_cast<const uint2 *>(static_cast<const u16 *>(kc) + (hb + p) * HD + 4 * c4);
                const uint2 vb2 = *reinterpret_cast<const uint2 *>(static_cast<const u16 *>(vc) + (hb + p) * HD + 4 * c4);
                kx[0] = bf16_bits_to_f32(kb2.x & 0xFFFFu); kx[1] = bf16_bits_to_f32(kb2.x >> 16);
                kx[2] = bf16_bits_to_f32(kb2.y & 0xFFFFu); kx[3] = bf16_bits_to_f32(kb2.y >> 16);
                vx[0] = bf16_bits_to_f32(vb2.x & 0xFFFFu); vx[1] = bf16_bits_to_f32(vb2.x >> 16);
                vx[2] = bf16_bits_to_f32(vb2.y & 0xFFFFu); vx[3] = bf16_bits_to_f32(vb2.y >> 16);
            } else {
                constexpr int RB = kv_row_bytes<KT>(HD);
                const float4 a = kv_load4<KT, HD>(static_cast<const char *>(kc) + (hb + p) * RB, 4 * c4);
                const float4 b = kv_load4<KT, HD>(static_cast<const char *>(vc) + (hb + p) * RB, 4 * c4);
                kx[0] = a.x; kx[1] = a.y; kx[2] = a.z; kx[3] = a.w;
                vx[0] = b.x; vx[1] = b.y; vx[2] = b.z; vx[3] = b.w;
            }
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            split_bf16(kx[e], hi[e], lo[e]);
            sv[r][4 * c4 + e] = vx[e];
        }
        *reinterpret_cast<uint2 *>(out + I::KH + r * I::KLD + 4 * c4) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        if constexpr (!KB)
            *reinterpret_cast<uint2 *>(out + I::KL + r * I::KLD + 4 * c4) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
    }
    // K row padding (never read by the MFMA operands; written for a defined image)
    for (int i = tid; i < TK * 8; i += 256) {
        const int r = i / 8, c = HD + i % 8;
        out[I::KH + r * I::KLD + c] = 0;
        if constexpr (!KB) out[I::KL + r * I::KLD + c] = 0;
    }
    __syncthreads();
    // V transposed: row d holds keys 0..63 (pairs packed in one word), padded to VLD
    for (int i = tid; i < HD * (I::VLD / 2); i += 256) {
        const int d = i / (I::VLD / 2), kp = i % (I::VLD / 2);
        uint32_t wh = 0, wl = 0;
        if (2 * kp < TK) {
            uint32_t h0, l0, h1, l1;
            split_bf16(sv[2 * kp][d], h0, l0);
            split_bf16(sv[2 * kp + 1][d], h1, l1);
            wh = h0 | (h1 << 16);
            wl = l0 | (l1 << 16);
        }
        *reinterpret_cast<uint32_t *>(out + I::VH + d * I::VLD + 2 * kp) = wh;
        if constexpr (!KB) *reinterpret_cast<uint32_t *>(out + I::VL + d * I::VLD + 2 * kp) = wl;
    }
    // tail of the image beyond the used part
    for (int i = I::USED + tid; i < I::BYTES / 2; i += 256) out[i] = 0;
}

__device__ __forceinline__ bf16x8 pack8(const uint32_t *h) {
    u32x4 v;
    v[0] = h[0] | (h[1] << 16); v[1] = h[2] | (h[3] << 16);
    v[2] = h[4] | (h[5] << 16); v[3] = h[6] | (h[7] << 16);
    return __builtin_bit_cast(bf16x8, v);
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

template <int HD, int G, bool KB>
__global__ void __launch_bounds__(NTHR, 1) attn_tiles_kernel(int T, int start_pos, const float *__restrict__ q,
                                                             const u16 *__restrict__ img, int ntiles_all, int nh,
                                                             int chunk, int nch, float *__restrict__ part,
                                                             u16 *__restrict__ o_hi, u16 *__restrict__ o_lo,
                                                             float *__restrict__ o_f32) {
    using I = Img<HD, KB>;
    extern __shared__ __attribute__((aligned(16))) u16 lds[];   // two tile images
    constexpr int ROWS = NQV / G;
    constexpr int KS = HD / 16;     // MFMA k-steps over head_dim
    constexpr int DT = HD / 32;     // output dim tiles
    constexpr int IMGU16 = I::BYTES / 2;

    // blocks are dispatched in linear order (x fastest): walk the row blocks
    // from the longest (last rows) down, the key chunks of a row block and all
    // kv heads together, so the longest blocks start first on every CU
    const int lin = blockIdx.x + blockIdx.y * gridDim.x;
    const int kvh = lin % gridDim.y;
    const int ch = (lin / gridDim.y) % nch;
    const int rb = gridDim.x / nch - 1 - lin / (gridDim.y * nch);
    const int t0 = rb * ROWS;
    const int last_pos = start_pos + min(T, t0 + ROWS) - 1;
    const int ntiles = last_pos / TK + 1;
    const int nchunks = (ntiles + chunk - 1) / chunk;   // of this row block
    const int j0 = ch * chunk, j1 = min(ntiles, j0 + chunk);
    if (j0 >= j1) return;   // a chunk past the row block's keys (block-uniform)
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int ql = lane & 31, hh = lane >> 5;
    const int qv = wv * 32 + ql;
    const int row = qv / G, g = qv % G;
    const int t = t0 + row;
    const bool live = row < ROWS && t < T;
    const int qpos = live ? start_pos + t : -1;
    const int h = kvh * G + g;

    // Q^T operand (B of S^T): lane (q + 32hh), k-step s -> dims 16s + 8hh .. +8, scaled to base 2
    bf16x8 qh[KS], qlo[KS];
    {
        const float qs = LOG2E / sqrtf((float)HD);
        const float *qp = q + (size_t)(live ? t : 0) * nh * HD + (size_t)h * HD + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; s++) {
            uint32_t hb[8], lb[8];
            const float4 a = *reinterpret_cast<const float4 *>(qp + 16 * s);
            const float4 b = *reinterpret_cast<const float4 *>(qp + 16 * s + 4);
            const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; j++) split_bf16(live ? f[j] * qs : 0.f, hb[j], lb[j]);
            qh[s] = pack8(hb);
            qlo[s] = pack8(lb);
        }
    }
    floatx16 o[DT];
#pragma unroll
    for (int d = 0; d < DT; d++)
#pragma unroll
        for (int e = 0; e < 16; e++) o[d][e] = 0.f;
    float m = -INFINITY, l = 0.f;

    // smallest / largest query position of the wave (live lanes)
    int wmax = qpos, wmin = live ? qpos : INT32_MAX;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        wmax = max(wmax, __shfl_xor(wmax, off, WAVE));
        wmin = min(wmin, __shfl_xor(wmin, off, WAVE));
    }
    const u32x4 *src = reinterpret_cast<const u32x4 *>(img + (size_t)kvh * ntiles_all * IMGU16);

    // the next tile's image goes from global memory straight into the other
    // LDS buffer (global_load_lds: lane L of a wave writes 16 bytes at the
    // wave's base + 16 L, so chunk tid + c*NTHR lands at that chunk of the
    // buffer); it is issued at the top of an iteration and waited for at the
    // barrier that ends it
    auto dma = [&](int j, int buf) {
#pragma unroll
        for (int c = 0; c < I::CHUNKS; c++) {
            __attribute__((address_space(3))) u16 *dst =
                (__attribute__((address_space(3))) u16 *)lds + buf * IMGU16 + (size_t)(c * NTHR + wv * WAVE) * 8;
            __builtin_amdgcn_global_load_lds((const void *)(src + (size_t)j * (IMGU16 / 8) + tid + c * NTHR),
                                             (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
        }
    };
    dma(j0, 0);
    __syncthreads();

    for (int j = j0; j < j1; j++) {
        if (j + 1 < j1) dma(j + 1, (j + 1 - j0) & 1);
        const int kb = j * TK;
        if (kb <= wmax) {
            const u16 *sb = lds + ((j - j0) & 1) * IMGU16;
            // S^T for the 64 keys: two 32-key sub-tiles
            floatx16 sc[2];
#pragma unroll
            for (int kt = 0; kt < 2; kt++) {
#pragma unroll
                for (int e = 0; e < 16; e++) sc[kt][e] = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < KS; s2++) {
                    const int off = (kt * 32 + ql) * I::KLD + 16 * s2 + 8 * hh;
                    const bf16x8 kh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sb + I::KH + off));
                    sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qh[s2], sc[kt], 0, 0, 0);
                    sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qlo[s2], sc[kt], 0, 0, 0);
                    if constexpr (!KB) {
                        const bf16x8 kl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sb + I::KL + off));
                        sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qh[s2], sc[kt], 0, 0, 0);
                    }
                }
            }
            // lane holds keys kb + kt*32 + (e/4)*8 + 4hh + e%4 of its query
            if (kb + TK - 1 > wmin) {
#pragma unroll
                for (int kt = 0; kt < 2; kt++)
#pragma unroll
                    for (int e = 0; e < 16; e++) {
                        const int key = kb + kt * 32 + (e / 4) * 8 + 4 * hh + (e % 4);
                        if (key > qpos) sc[kt][e] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int e = 0; e < 16; e++) mx = fmaxf(mx, sc[kt][e]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
            const float mnew = fmaxf(m, mx);
            const float mref = mnew == -INFINITY ? 0.f : mnew;
            const float corr = __builtin_amdgcn_exp2f(m - mref);
            float ps = 0.f;
            uint32_t ph[2][8], plo[2][8];   // (hi, lo) bf16 pairs of weights e, e+1
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(sc[kt][e] - mref);
                    const float p1 = __builtin_amdgcn_exp2f(sc[kt][e + 1] - mref);
                    ps += p0;
                    ps += p1;
                    split2_bf16(p0, p1, ph[kt][e / 2], plo[kt][e / 2]);
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
                const uint32_t *hp = &ph[ks / 2][(ks % 2) * 4], *lp = &plo[ks / 2][(ks % 2) * 4];
                const bf16x8 bh = __builtin_bit_cast(bf16x8, u32x4{hp[0], hp[1], hp[2], hp[3]});
                const bf16x8 bl = __builtin_bit_cast(bf16x8, u32x4{lp[0], lp[1], lp[2], lp[3]});
#pragma unroll
                for (int d = 0; d < DT; d++) {
                    const int vrow = (d * 32 + ql) * I::VLD + 16 * ks + 4 * hh;
                    const uint2 h0 = *reinterpret_cast<const uint2 *>(sb + I::VH + vrow);
                    const uint2 h1 = *reinterpret_cast<const uint2 *>(sb + I::VH + vrow + 8);
                    const bf16x8 ah = __builtin_bit_cast(bf16x8, u32x4{h0.x, h0.y, h1.x, h1.y});
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, o[d], 0, 0, 0);
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, o[d], 0, 0, 0);
                    if constexpr (!KB) {
                        const uint2 l0 = *reinterpret_cast<const uint2 *>(sb + I::VL + vrow);
                        const uint2 l1 = *reinterpret_cast<const uint2 *>(sb + I::VL + vrow + 8);
                        const bf16x8 al = __builtin_bit_cast(bf16x8, u32x4{l0.x, l0.y, l1.x, l1.y});
                        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, o[d], 0, 0, 0);
                    }
                }
            }
        }
        // the other buffer, refilled above, held tile j-1, which every wave
        // finished before the previous barrier; __syncthreads also waits for
        // the direct-to-LDS loads
        __syncthreads();
    }
    if (!live) return;
    if (nchunks > 1) {
        // a chunk of a split row block: unnormalised output, base-2 running
        // maximum and normaliser of (row t, head h) over this chunk's keys
        float *dst = part + (((size_t)ch * T + t) * nh + h) * (HD + 2);
#pragma unroll
        for (int d = 0; d < DT; d++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const int dim = d * 32 + gq * 8 + 4 * hh;
                *reinterpret_cast<float4 *>(dst + dim) =
                    make_float4(o[d][4 * gq], o[d][4 * gq + 1], o[d][4 * gq + 2], o[d][4 * gq + 3]);
            }
        if (hh == 0) { dst[HD] = m; dst[HD + 1] = l; }
        return;
    }
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

// The key chunks of the split row blocks: one wave per (row, head), lane =
// output dim (two dims per lane at head_dim 128).  Lane c first loads chunk c's
// running maximum and normaliser; weights f_c = 2^(m_c - max m), output and
// normaliser summed over ascending c.
template <int HD>
__global__ void __launch_bounds__(256) attn_chunk_merge_kernel(int T, int start_pos, int nh, int rows_per_block,
                                                              int chunk, const float *__restrict__ part,
                                                              u16 *__restrict__ o_hi, u16 *__restrict__ o_lo,
                                                              float *__restrict__ o_f32) {
    const int wid = blockIdx.x * 4 + threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    if (wid >= T * nh) return;
    const int t = wid / nh, h = wid % nh;
    const int rb = t / rows_per_block;
    const int last_pos = start_pos + min(T, (rb + 1) * rows_per_block) - 1;
    const int nchunks = (last_pos / TK + 1 + chunk - 1) / chunk;   // at most 64
    if (nchunks <= 1) return;   // that row block wrote its output directly
    constexpr int DPL = HD / WAVE;
    const size_t cs = (size_t)T * nh * (HD + 2);
    const float *src = part + ((size_t)t * nh + h) * (HD + 2);
    const float mc = lane < nchunks ? src[lane * cs + HD] : -INFINITY;
    const float lc = lane < nchunks ? src[lane * cs + HD + 1] : 0.f;
    const float mx = wave_max(mc);
    const float f = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - mx);
    float L = 0.f, A[DPL];
#pragma unroll
    for (int e = 0; e < DPL; e++) A[e] = 0.f;
#pragma unroll 4
    for (int c = 0; c < nchunks; c++) {
        const float fc = __shfl(f, c, WAVE);
        L += __shfl(lc, c, WAVE) * fc;
#pragma unroll
        for (int e = 0; e < DPL; e++) A[e] += src[c * cs + lane + e * WAVE] * fc;
    }
    const float inv = 1.0f / L;
    const size_t base = (size_t)t * nh * HD + (size_t)h * HD;
#pragma unroll
    for (int e = 0; e < DPL; e++) store_out(A[e] * inv, base + lane + e * WAVE, o_hi, o_lo, o_f32);
}

template <int HD, int G, bool KB>
void set_lds_attr() {
    static bool done = false;
    if (!done) {
        (void)hipFuncSetAttribute((const void *)attn_tiles_kernel<HD, G, KB>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 2 * Img<HD, KB>::BYTES);
        done = true;
    }
}

// Key tiles per chunk for T rows from start_pos (rows_per_block query rows per
// block, nkv kv heads), and the chunk count of the longest row block: a launch
// of at least twice as many (row block, kv head) blocks as CUs is not split
// (the longest-first dispatch order balances it); a smaller one is cut into
// chunks of 2 x (its tiles / CUs) tiles, at least 2, and at most max_chunks per
// row block (the partial buffer's room).  Each chunk costs its block's query
// load, first-tile wait and partial write, and the merge; at Qwen2.5-0.5B's
// 2048 tokens (1974 block-tiles) chunks of 15 tiles (the longest row blocks
// in three) measured 7.45 ms per prefill against 7.81 (8 tiles), 8.27 (4
// tiles) and 8.07 unsplit.
void chunking(int T, int start_pos, int rows_per_block, int nkv, int max_chunks, int &chunk, int &nch) {
    const int rbs = (T + rows_per_block - 1) / rows_per_block;
    const int ntiles_max = (start_pos + T - 1) / TK + 1;
    chunk = ntiles_max;
    nch = 1;
    const int cus = num_cus();
    if ((long)rbs * nkv >= 2L * cus || max_chunks < 2) return;
    long total = 0;
    for (int rb = 0; rb < rbs; rb++) total += (start_pos + std::min(T, (rb + 1) * rows_per_block) - 1) / TK + 1;
    total *= nkv;
    int c = (int)((2 * total + cus - 1) / cus);
    c = std::max(c, 2);
    if ((ntiles_max + c - 1) / c > max_chunks) c = (ntiles_max + max_chunks - 1) / max_chunks;
    chunk = std::min(c, ntiles_max);
    nch = (ntiles_max + chunk - 1) / chunk;
}

template <int HD, int KT>
bool launch_hd(hipStream_t st, int G, int T, int start_pos, int slot, const float *q, const void *kc,
               const void *vc, int nh, int nkv, int max_seq, u16 *img, float *part, size_t part_floats, u16 *o_hi,
               u16 *o_lo, float *o_f32) {
    if (G < 1 || G > 8) return false;
    constexpr bool KB = KT == KV_BF16;
    const int npos = start_pos + T;
    const int ntiles = (npos + TK - 1) / TK;
    constexpr int LDSB = 2 * Img<HD, KB>::BYTES;
    const int rows = NQV / G;
    const size_t per_chunk = (size_t)T * nh * (HD + 2);
    const int max_chunks = part ? (int)std::min<size_t>(part_floats / per_chunk, 64) : 1;
    int chunk, nch;
    chunking(T, start_pos, rows, nkv, max_chunks, chunk, nch);
    const int rbs = (T + rows - 1) / rows;
    hipLaunchKernelGGL((kv_tile_kernel<HD, KT>), dim3(ntiles, nkv), dim3(256), 0, st, kc, vc, max_seq, slot, nkv,
                       npos, ntiles, img);
#define AT(GG)                                                                                                  \
    do {                                                                                                        \
        set_lds_attr<HD, GG, KB>();                                                                             \
        hipLaunchKernelGGL((attn_tiles_kernel<HD, GG, KB>), dim3(rbs * nch, nkv), dim3(NTHR), LDSB, st, T,      \
                           start_pos, q, img, ntiles, nh, chunk, nch, part, o_hi, o_lo, o_f32);                \
    } while (0)
    switch (G) {
        case 1: AT(1); break;
        case 2: AT(2); break;
        case 3: AT(3); break;
        case 4: AT(4); break;
        case 5: AT(5); break;
        case 6: AT(6); break;
        case 7: AT(7); break;
        case 8: AT(8); break;
    }
#undef AT
    if (nch > 1)
        hipLaunchKernelGGL((attn_chunk_merge_kernel<HD>), dim3((T * nh + 3) / 4), dim3(256), 0, st, T, start_pos, nh,
                           rows, chunk, part, o_hi, o_lo, o_f32);
    return true;
}

}  // namespace

size_t attn_tiles_bytes(int max_pos, int nkv, int hd, int kv_kind) {
    const bool kv_bf16 = kv_kind == KV_BF16;
    const size_t ntiles = (size_t)(max_pos + TK - 1) / TK;
    size_t per = 0;
    if (hd == 128) per = kv_bf16 ? Img<128, true>::BYTES : Img<128, false>::BYTES;
    else if (hd == 64) per = kv_bf16 ? Img<64, true>::BYTES : Img<64, false>::BYTES;
    return ntiles * nkv * per;
}

bool launch_attn_prefill_tiles(hipStream_t st, int T, int start_pos, int slot, const float *q, const void *kc,
                               const void *vc, int kv_kind, int nh, int nkv, int hd, int max_seq, void *img,
                               float *part, size_t part_floats, u16 *o_hi, u16 *o_lo, float *o_f32) {
    if (T <= 0) return true;
    const int G = nh / nkv;
    u16 *im = static_cast<u16 *>(img);
#define LH(HD, KT) launch_hd<HD, KT>(st, G, T, start_pos, slot, q, kc, vc, nh, nkv, max_seq, im, part, part_floats, \
                                     o_hi, o_lo, o_f32)
#define LHK(HD) (kv_kind == KV_BF16 ? LH(HD, KV_BF16) : kv_kind == KV_F24 ? LH(HD, KV_F24) : LH(HD, KV_F32))
    if (hd == 128) return LHK(128);
    if (hd == 64) return LHK(64);
#undef LHK
#undef LH
    return false;
}
