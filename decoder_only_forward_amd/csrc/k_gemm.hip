// Prefill projections on MFMA: out[m][n] = sum_k (a_hi + a_lo)[m][k] * W[n][k].
//
// Both operands are k-contiguous ("NT" layout), which is what the bf16 MFMA
// wants.  The weight tile is the A operand (16 output features per MFMA row
// tile), the activation tile the B operand, fed twice (hi then lo) into the
// same accumulator so the fp32 activations keep ~16 significant bits.
//
// Tiles are staged through LDS with 16-byte global loads; rows are padded by 16
// bytes so the MFMA operand reads of one lane group fall in distinct banks.
//
// An optional expert grouping (MoE prefill) runs one grid slice per expert over
// that expert's contiguous rows of `a` and its slice of the weights.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

struct GemmParams {
    const u16 *w[MAX_SEGS];
    int seg_end[MAX_SEGS];
    int nseg;
    int N, K, M;
    const u16 *a_hi, *a_lo;
    int lda;
    float *out;
    int ldo;
    const int32_t *grp_off;
    size_t expert_stride;
    // direct-to-LDS kernel, split over k: block z covers k in
    // [z*kchunk, (z+1)*kchunk) and writes out + z*split_stride (grouped:
    // z = expert * ksplit + split)
    int kchunk;
    size_t split_stride;
    int ksplit;
};

// Block tile: BN = 256 output features (weight rows) x BM = 128 tokens x BK = 64.
// 8 waves as 4 (features) x 2 (tokens), each wave 64 x 64 = 2 x 2 MFMA tiles of
// 32x32x16.  Two LDS stages and two register stages: the global loads of
// k-tile k+2 are in flight while tile k is multiplied, so the HBM/L2 latency is
// hidden behind two tiles of MFMA work.
constexpr int BN = 256, BM = 128, BK = 64;
constexpr int NTHR = 512;
constexpr int LDR = BK + 8;                    // u16 per padded LDS row (144 bytes)
constexpr int STAGE_U16 = (BN + 2 * BM) * LDR; // W, A_hi, A_lo of one k-tile
constexpr int WLOADS = BN * BK / 8 / NTHR;     // 16-byte chunks per thread per tile (4)
constexpr int ALOADS = BM * BK / 8 / NTHR;     // (2) for each of hi and lo

__global__ void __launch_bounds__(NTHR, 1) gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) u16 smem[];
    const int tid = threadIdx.x;
    const int lane = tid % WAVE, wv = tid / WAVE;
    const int wn = wv & 3, wm = wv >> 2;

    int M = p.M, mrow0 = 0;
    size_t wofs = 0;
    if (p.grp_off) {
        const int e = blockIdx.z;
        mrow0 = p.grp_off[e];
        M = p.grp_off[e + 1] - mrow0;
        wofs = (size_t)e * p.expert_stride;
    }
    // tile order: each XCD (blocks are dealt round-robin to 8 of them) walks a
    // contiguous run of tiles, tokens fastest, so a weight tile stays in its L2.
    const int ntn = (p.N + BN - 1) / BN, ntm = gridDim.y;
    int bid = blockIdx.x + blockIdx.y * gridDim.x;
    const int nblk = ntn * ntm;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int tn = bid / ntm, tm = bid % ntm;
    const int m0 = tm * BM;
    if (m0 >= M) return;
    const int n0 = tn * BN;

    // per-thread global offsets (elements) of its 16-byte chunks
    size_t ow[WLOADS], oa[ALOADS];
    const u16 *wbase[WLOADS];
#pragma unroll
    for (int i = 0; i < WLOADS; i++) {
        const int idx = tid + i * NTHR;
        const int row = idx >> 3, ch = idx & 7;
        int n = n0 + row;
        n = n < p.N ? n : p.N - 1;
        const u16 *wp = p.w[0];
        int start = 0;
        if (p.nseg > 1 && n >= p.seg_end[0]) { wp = p.w[1]; start = p.seg_end[0]; }
        if (p.nseg > 2 && n >= p.seg_end[1]) { wp = p.w[2]; start = p.seg_end[1]; }
        wbase[i] = wp;
        ow[i] = wofs + (size_t)(n - start) * p.K + ch * 8;
    }
#pragma unroll
    for (int i = 0; i < ALOADS; i++) {
        const int idx = tid + i * NTHR;
        const int row = idx >> 3, ch = idx & 7;
        int m = m0 + row;
        m = m < M ? m : M - 1;
        oa[i] = (size_t)(mrow0 + m) * p.lda + ch * 8;
    }
    const u16 *__restrict__ ahi = p.a_hi;
    const u16 *__restrict__ alo = p.a_lo;

#define GEMM_GLOAD(W, H, L, kt)                                                                   \
    do {                                                                                          \
        const int k0_ = (kt) * BK;                                                                \
        _Pragma("unroll") for (int i = 0; i < WLOADS; i++)                                        \
            W[i] = *reinterpret_cast<const u32x4 *>(wbase[i] + ow[i] + k0_);                      \
        _Pragma("unroll") for (int i = 0; i < ALOADS; i++) {                                      \
            H[i] = *reinterpret_cast<const u32x4 *>(ahi + oa[i] + k0_);                           \
            L[i] = *reinterpret_cast<const u32x4 *>(alo + oa[i] + k0_);                           \
        }                                                                                         \
    } while (0)
#define GEMM_LSTORE(W, H, L, buf)                                                                 \
    do {                                                                                          \
        u16 *sw_ = smem + (buf) * STAGE_U16;                                                      \
        u16 *sh_ = sw_ + BN * LDR;                                                                \
        u16 *sl_ = sh_ + BM * LDR;                                                                \
        _Pragma("unroll") for (int i = 0; i < WLOADS; i++) {                                      \
            const int idx = tid + i * NTHR;                                                       \
            *reinterpret_cast<u32x4 *>(sw_ + (idx >> 3) * LDR + (idx & 7) * 8) = W[i];            \
        }                                                                                         \
        _Pragma("unroll") for (int i = 0; i < ALOADS; i++) {                                      \
            const int idx = tid + i * NTHR;                                                       \
            *reinterpret_cast<u32x4 *>(sh_ + (idx >> 3) * LDR + (idx & 7) * 8) = H[i];            \
            *reinterpret_cast<u32x4 *>(sl_ + (idx >> 3) * LDR + (idx & 7) * 8) = L[i];            \
        }                                                                                         \
    } while (0)

    const floatx16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    floatx16 acc00 = zero16, acc01 = zero16, acc10 = zero16, acc11 = zero16;

    const int r32 = lane & 31, c2 = lane >> 5;
    const int wrow0 = (wn * 64 + r32) * LDR + c2 * 8;
    const int arow0 = (wm * 64 + r32) * LDR + c2 * 8;
#define GEMM_COMPUTE(buf)                                                                         \
    do {                                                                                          \
        const u16 *sw_ = smem + (buf) * STAGE_U16;                                                \
        const u16 *sh_ = sw_ + BN * LDR;                                                          \
        const u16 *sl_ = sh_ + BM * LDR;                                                          \
        _Pragma("unroll") for (int ks = 0; ks < BK / 16; ks++) {                                  \
            const bf16x8 fw0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sw_ + wrow0 + ks * 16)); \
            const bf16x8 fw1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sw_ + wrow0 + 32 * LDR + ks * 16)); \
            const bf16x8 fh0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sh_ + arow0 + ks * 16)); \
            const bf16x8 fh1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sh_ + arow0 + 32 * LDR + ks * 16)); \
            const bf16x8 fl0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sl_ + arow0 + ks * 16)); \
            const bf16x8 fl1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sl_ + arow0 + 32 * LDR + ks * 16)); \
            acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw0, fh0, acc00, 0, 0, 0);           \
            acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw0, fh1, acc01, 0, 0, 0);           \
            acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw1, fh0, acc10, 0, 0, 0);           \
            acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw1, fh1, acc11, 0, 0, 0);           \
            acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw0, fl0, acc00, 0, 0, 0);           \
            acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw0, fl1, acc01, 0, 0, 0);           \
            acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw1, fl0, acc10, 0, 0, 0);           \
            acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw1, fl1, acc11, 0, 0, 0);           \
        }                                                                                         \
    } while (0)

    const int nk = p.K / BK;
    u32x4 raw[WLOADS], rah[ALOADS], ral[ALOADS];
    u32x4 rbw[WLOADS], rbh[ALOADS], rbl[ALOADS];
    GEMM_GLOAD(raw, rah, ral, 0);
    if (nk > 1) GEMM_GLOAD(rbw, rbh, rbl, 1);
    GEMM_LSTORE(raw, rah, ral, 0);
    if (nk > 2) GEMM_GLOAD(raw, rah, ral, 2);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        // buf 0 holds tile kt; rb* holds tile kt+1; ra* has tile kt+2 in flight
        GEMM_COMPUTE(0);
        if (kt + 1 < nk) {
            GEMM_LSTORE(rbw, rbh, rbl, 1);
            if (kt + 3 < nk) GEMM_GLOAD(rbw, rbh, rbl, kt + 3);
        }
        __syncthreads();
        if (kt + 1 >= nk) break;
        // buf 1 holds tile kt+1; ra* holds tile kt+2; rb* has tile kt+3 in flight
        GEMM_COMPUTE(1);
        if (kt + 2 < nk) {
            GEMM_LSTORE(raw, rah, ral, 0);
            if (kt + 4 < nk) GEMM_GLOAD(raw, rah, ral, kt + 4);
        }
        __syncthreads();
    }
#undef GEMM_GLOAD
#undef GEMM_LSTORE
#undef GEMM_COMPUTE

    // acc<i><j>: features n0 + wn*64 + i*32 + (e/4)*8 + c2*4 + e%4, token m0 + wm*64 + j*32 + r32
    auto store_tile = [&](const floatx16 v, int i, int j) {
        const int m = m0 + wm * 64 + j * 32 + r32;
        if (m >= M) return;
        float *dst = p.out + (size_t)(mrow0 + m) * p.ldo;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int n = n0 + wn * 64 + i * 32 + g * 8 + c2 * 4;
            if (n + 3 < p.N) {
                *reinterpret_cast<float4 *>(dst + n) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
            } else {
                if (n < p.N) dst[n] = v[4 * g];
                if (n + 1 < p.N) dst[n + 1] = v[4 * g + 1];
                if (n + 2 < p.N) dst[n + 2] = v[4 * g + 2];
            }
        }
    };
    store_tile(acc00, 0, 0);
    store_tile(acc01, 0, 1);
    store_tile(acc10, 1, 0);
    store_tile(acc11, 1, 1);
}

constexpr size_t GEMM_LDS = 2 * STAGE_U16 * sizeof(u16);

// The two LDS stages exceed the default dynamic-LDS cap; raise it once.
void gemm_lds_attr() {
    static bool done = false;
    if (!done) {
        (void)hipFuncSetAttribute((const void *)gemm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS);
        done = true;
    }
}

void fill(GemmParams &p, const WSeg *segs, int nseg, int K, const u16 *a_hi, const u16 *a_lo, int lda,
          int M, float *out, int ldo) {
    int end = 0;
    for (int s = 0; s < nseg; s++) {
        p.w[s] = (const u16 *)segs[s].w;
        end += segs[s].rows;
        p.seg_end[s] = end;
    }
    p.nseg = nseg;
    p.N = end;
    p.K = K;
    p.M = M;
    p.a_hi = a_hi;
    p.a_lo = a_lo;
    p.lda = lda;
    p.out = out;
    p.ldo = ldo;
    p.kchunk = K;
    p.split_stride = 0;
    p.ksplit = 1;
}

}  // namespace

// ---- large grids: 256 x 256 tiles fed by direct-to-LDS loads ----------------
// Block tile 256 features x 256 tokens x 32 k; 8 waves as 2 (features) x 4
// (tokens), each 128 x 64 = 4 x 2 MFMA tiles of 32x32x16, so a weight fragment
// read from LDS serves both the hi and the lo pass of two token tiles.  Tiles
// go from global memory straight into a 3-stage LDS ring (global_load_lds, no
// register staging): the loads of k-tile t+2 are in flight while tile t is
// multiplied.  Rows of a stage are 64 bytes with their four 16-byte chunks
// XOR-swizzled by row, so the 16 rows an MFMA operand read touches per lane
// group fall in distinct banks.  The tile order gives each XCD a contiguous
// range of feature tiles, walked four token tiles at a time, so the blocks an
// XCD runs together share few weight and activation panels in its L2.
//
// The grouped (MoE prefill) form runs one grid slice per expert (times the k
// splits): an expert's weights are segs[i].w + e * expert_stride and its rows
// [offsets[e], offsets[e+1]).  The MFMAs of a wave's 32-token sub-tiles past
// the expert's last row are skipped.  An expert's rows of a 512-token prefill
// (about 128-190) fit one 256-token tile, so its weight panel streams from HBM
// once; a 512-feature x 128-token tile, which fills its rows better but reads
// the panel again for a second row tile, measured 17-20 % slower.
namespace {

constexpr int DBN = 256, DBM = 256, DBK = 32;
constexpr int DNTHR = 512;
constexpr int DARR = 256 * DBK;              // u16 per operand array of a stage (16 KB)
constexpr int DSTAGE = 3 * DARR;             // W, A_hi, A_lo
constexpr int DNSTAGE = 3;
constexpr int DGROUP = 4;                    // token tiles an XCD walks together
constexpr size_t DMA_LDS = DNSTAGE * DSTAGE * sizeof(u16);
// grouped form: weights in their own ring of DNWS_G stages, then the DNSTAGE
// stages of the activation pair (160 KB, the whole LDS of a CU)
constexpr int DNWS_G = 4;
constexpr size_t DMA_LDS_G = (DNWS_G * DARR + DNSTAGE * 2 * DARR) * sizeof(u16);
#define LDS_AS __attribute__((address_space(3)))

// 16-byte chunk c (of 4) of row r is stored at chunk c ^ ((r >> 2) & 3) of the row
__device__ __forceinline__ int dswz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// SILU: the SwiGLU form.  p.w[0] is the gate and p.w[1] the up matrix, each
// p.N rows; a block tile covers 128 gate features and the same 128 up
// features (wave wn: 64 of each, its MFMA row tiles 0, 1 gate and 2, 3 up), so
// each lane holds gate and up of the same (feature, token) and the epilogue
// writes silu(gate) * up as bf16 (hi, lo) pairs, row stride p.ldo.
template <bool SILU, bool GROUPED>
__global__ void __launch_bounds__(DNTHR, 1) gemm_dma_kernel(GemmParams p, u16 *__restrict__ s_hi,
                                                            u16 *__restrict__ s_lo) {
    extern __shared__ __attribute__((aligned(16))) u16 smem[];
    const int tid = threadIdx.x;
    const int lane = tid % WAVE, wv = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int wn = wv & 1, wm = wv >> 1;
    int M = p.M, mrow0 = 0, kz = blockIdx.z;
    size_t wofs = 0;
    if constexpr (GROUPED) {
        const int e = blockIdx.z / p.ksplit;
        kz = blockIdx.z - e * p.ksplit;
        mrow0 = p.grp_off[e];
        M = p.grp_off[e + 1] - mrow0;
        wofs = (size_t)e * p.expert_stride;
    }

    constexpr int FPT = SILU ? DBN / 2 : DBN;    // output features per block tile
    const int ntn = (p.N + FPT - 1) / FPT, ntm = gridDim.y;
    const int bid = blockIdx.x + blockIdx.y * gridDim.x;
    int tn, tm;
    if ((ntn & 7) == 0) {
        // blocks are dealt round-robin to 8 XCDs: XCD x owns feature tiles
        // [x*ntn/8, (x+1)*ntn/8) and walks them DGROUP token tiles at a time
        const int x = bid & 7, lt = bid >> 3, nx = ntn >> 3;
        const int G = DGROUP < ntm ? DGROUP : ntm;
        const int tg = lt / (G * nx), rem = lt - tg * G * nx;
        const int gsz = min(G, ntm - tg * G);
        tn = x * nx + rem / gsz;
        tm = tg * G + rem % gsz;
    } else {
        int b = bid;
        const int nblk = ntn * ntm;
        if ((nblk & 7) == 0) b = (b & 7) * (nblk >> 3) + (b >> 3);
        tn = b / ntm;
        tm = b % ntm;
    }
    const int m0 = tm * DBM;
    if (m0 >= M) return;
    const int n0 = tn * FPT;
    const int kz0 = kz * p.kchunk;   // 0 for SILU (one split)

    // load instruction i (0, 1) of an operand array: wave wv fills the 1 KB slot
    // i*8 + wv, lane L the 16-byte chunk slot*64 + L, i.e. row r = chunk / 4 and
    // the logical chunk the swizzle stores there
    const u16 *srcw[2], *srch[2], *srcl[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int P = (i * 8 + wv) * 64 + lane;
        const int r = P >> 2, c = (P & 3) ^ ((r >> 2) & 3);
        if constexpr (SILU) {
            // LDS row r: wave r / 128, MFMA row tile (r % 128) / 32 (0, 1 gate; 2, 3 up)
            const int t = (r & 127) >> 5;
            int f = n0 + (r >> 7) * 64 + (t & 1) * 32 + (r & 31);
            f = f < p.N ? f : p.N - 1;
            srcw[i] = (t < 2 ? p.w[0] : p.w[1]) + wofs + (size_t)f * p.K + kz0 + c * 8;
        } else {
            int n = n0 + r;
            n = n < p.N ? n : p.N - 1;
            const u16 *wp = p.w[0];
            int start = 0;
            if (p.nseg > 1 && n >= p.seg_end[0]) { wp = p.w[1]; start = p.seg_end[0]; }
            if (p.nseg > 2 && n >= p.seg_end[1]) { wp = p.w[2]; start = p.seg_end[1]; }
            srcw[i] = wp + wofs + (size_t)(n - start) * p.K + kz0 + c * 8;
        }
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int P = (i * 8 + wv) * 64 + lane;
        const int r = P >> 2, c = (P & 3) ^ ((r >> 2) & 3);
        int m = m0 + r;
        m = m < M ? m : M - 1;
        srch[i] = p.a_hi + (size_t)(mrow0 + m) * p.lda + kz0 + c * 8;
        srcl[i] = p.a_lo + (size_t)(mrow0 + m) * p.lda + kz0 + c * 8;
    }
    const int nk = min(p.kchunk, p.K - kz0) / DBK;
    // Every iteration issues its loads (the last tile again past the end), so
    // the count of outstanding loads is the same everywhere.  Load instruction
    // i of wave wv covers token rows (i*8 + wv)*16 .. +15 of the tile; a wave
    // issues only the token-row loads of groups holding a row below M (NA of
    // 2: the expert rows of a grouped tile, or the last token tile, often end
    // early).  LDS rows of skipped groups keep stale values, which reach only
    // outputs of tokens >= M, never stored.
    auto load_tile = [&](int kt, int stage, auto na_c) {
        constexpr int NA = decltype(na_c)::value;
        const int k0 = (kt < nk ? kt : nk - 1) * DBK;
        LDS_AS u16 *base = (LDS_AS u16 *)smem + stage * DSTAGE;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int slot = (i * 8 + wv) * 512;
            __builtin_amdgcn_global_load_lds((const void *)(srcw[i] + k0), (LDS_AS void *)(base + slot), 16, 0, 0);
            if (i < NA) {
                __builtin_amdgcn_global_load_lds((const void *)(srch[i] + k0), (LDS_AS void *)(base + DARR + slot),
                                                 16, 0, 0);
                __builtin_amdgcn_global_load_lds((const void *)(srcl[i] + k0),
                                                 (LDS_AS void *)(base + 2 * DARR + slot), 16, 0, 0);
            }
        }
    };

    // grouped form: the weights (streamed from HBM once, no other block reads
    // them) get a ring of DNWS_G stages and are loaded a k-tile further ahead
    // than the activation rows, which other blocks of the expert share in L2
    auto load_w = [&](int kt, int stage) {
        const int k0 = (kt < nk ? kt : nk - 1) * DBK;
        LDS_AS u16 *base = (LDS_AS u16 *)smem + stage * DARR;
#pragma unroll
        for (int i = 0; i < 2; i++)
            __builtin_amdgcn_global_load_lds((const void *)(srcw[i] + k0),
                                             (LDS_AS void *)(base + (i * 8 + wv) * 512), 16, 0, 0);
    };
    auto load_a = [&](int kt, int stage, auto na_c) {
        constexpr int NA = decltype(na_c)::value;
        const int k0 = (kt < nk ? kt : nk - 1) * DBK;
        LDS_AS u16 *base = (LDS_AS u16 *)smem + DNWS_G * DARR + stage * 2 * DARR;
#pragma unroll
        for (int i = 0; i < NA; i++) {
            const int slot = (i * 8 + wv) * 512;
            __builtin_amdgcn_global_load_lds((const void *)(srch[i] + k0), (LDS_AS void *)(base + slot), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(srcl[i] + k0), (LDS_AS void *)(base + DARR + slot), 16,
                                             0, 0);
        }
    };

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

    const int r32 = lane & 31, c2 = lane >> 5;
    // grouped: a wave's 32-token sub-tiles past the expert's last row multiply nothing
    const bool live1 = !GROUPED || m0 + wm * 64 + 32 < M;
    // stage s of the dense ring holds (W, A_hi, A_lo) together; the grouped
    // form reads weight stage ws and activation stage s
    auto compute = [&](int stage, int ws) {
        const u16 *sw = GROUPED ? smem + ws * DARR : smem + stage * DSTAGE;
        const u16 *sh = GROUPED ? smem + DNWS_G * DARR + stage * 2 * DARR : sw + DARR;
        const u16 *sl = sh + DARR;
#pragma unroll
        for (int ks = 0; ks < DBK / 16; ks++) {
            bf16x8 fw[4], fh[2], fl[2];
#pragma unroll
            for (int i = 0; i < 4; i++)
                fw[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                       sw + 8 * dswz(wn * 128 + i * 32 + r32, 2 * ks + c2)));
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int off = 8 * dswz(wm * 64 + j * 32 + r32, 2 * ks + c2);
                fh[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sh + off));
                fl[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sl + off));
            }
            if (!GROUPED || live1) {
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fh[j], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fl[j], acc[i][j], 0, 0, 0);
                    }
            } else if (m0 + wm * 64 < M) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fh[0], acc[i][0], 0, 0, 0);
                    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fl[0], acc[i][0], 0, 0, 0);
                }
            }
        }
    };

    // Barrier between k-tiles: wait until only the newest tile's loads (2 + 2 NA
    // per wave) may be outstanding and every LDS read is done, then s_barrier.
    // (__syncthreads would also wait for the newest tile: its fence covers the
    // LDS writes of every outstanding load.)  s_waitcnt fields: vmcnt, expcnt 7,
    // lgkmcnt 0.  The loop is instantiated per load count, so the waits stay
    // immediates; the waves of a block may take different instances (same
    // barrier count).
    auto ring = [&](auto na_c) {
        constexpr int NA = decltype(na_c)::value;
        if constexpr (!GROUPED) {
            constexpr int WAIT = (2 + 2 * NA) | (7 << 4) | (0 << 8);
            load_tile(0, 0, na_c);
            load_tile(1, 1, na_c);
            __builtin_amdgcn_s_waitcnt(WAIT);
            __builtin_amdgcn_s_barrier();
            for (int kt = 0; kt < nk; kt++) {
                // stage (kt+2)%3 held tile kt-1, which every wave finished reading
                // before the previous barrier; tile kt+1 is complete after this
                // iteration's wait
                load_tile(kt + 2, (kt + 2) % DNSTAGE, na_c);
                compute(kt % DNSTAGE, 0);
                __builtin_amdgcn_s_waitcnt(WAIT);
                __builtin_amdgcn_s_barrier();
            }
        } else {
            // issue order W0 A0 W1 A1 W2, then per k-tile A(kt+2) W(kt+3):
            // once tile kt+1 is complete only W(kt+2), A(kt+2) and W(kt+3)
            // (2 + 2 NA + 2 loads per wave) may still be outstanding.  Weight
            // stage (kt+3)%4 and activation stage (kt+2)%3 held tile kt-1.
            constexpr int WAIT = (4 + 2 * NA) | (7 << 4) | (0 << 8);
            load_w(0, 0);
            load_a(0, 0, na_c);
            load_w(1, 1);
            load_a(1, 1, na_c);
            load_w(2, 2);
            __builtin_amdgcn_s_waitcnt(WAIT);
            __builtin_amdgcn_s_barrier();
            for (int kt = 0; kt < nk; kt++) {
                load_a(kt + 2, (kt + 2) % DNSTAGE, na_c);
                load_w(kt + 3, (kt + 3) % DNWS_G);
                compute(kt % DNSTAGE, kt % DNWS_G);
                __builtin_amdgcn_s_waitcnt(WAIT);
                __builtin_amdgcn_s_barrier();
            }
        }
        // the loads issued past the last tile land in stages nobody reads again;
        // they must finish before the block's LDS is released
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    };
    const int na = (m0 + wv * 16 < M) + (m0 + (8 + wv) * 16 < M);   // wave-uniform
    if (na == 2) ring(std::integral_constant<int, 2>{});
    else if (na == 1) ring(std::integral_constant<int, 1>{});
    else ring(std::integral_constant<int, 0>{});

    if constexpr (SILU) {
        // acc[i][j] (gate, i = 0, 1) and acc[i+2][j] (up): feature
        // n0 + wn*64 + i*32 + (e/4)*8 + c2*4 + e%4, token m0 + wm*64 + j*32 + r32
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int m = m0 + wm * 64 + j * 32 + r32;
                if (m >= M) continue;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int f = n0 + wn * 64 + i * 32 + g * 8 + c2 * 4;
                    uint32_t hb[4], lb[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float gt = acc[i][j][4 * g + e], up = acc[i + 2][j][4 * g + e];
                        split_bf16(gt / (1.0f + expf(-gt)) * up, hb[e], lb[e]);
                    }
                    const size_t off = (size_t)(mrow0 + m) * p.ldo + f;
                    if (f + 3 < p.N) {
                        *reinterpret_cast<uint2 *>(s_hi + off) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                        *reinterpret_cast<uint2 *>(s_lo + off) = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (f + e < p.N) {
                                s_hi[off + e] = (u16)hb[e];
                                s_lo[off + e] = (u16)lb[e];
                            }
                    }
                }
            }
        return;
    }
    // acc[i][j]: features n0 + wn*128 + i*32 + (e/4)*8 + c2*4 + e%4, token m0 + wm*64 + j*32 + r32
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int m = m0 + wm * 64 + j * 32 + r32;
            if (m >= M) continue;
            float *dst = p.out + kz * p.split_stride + (size_t)(mrow0 + m) * p.ldo;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int n = n0 + wn * 128 + i * 32 + g * 8 + c2 * 4;
                const floatx16 &v = acc[i][j];
                if (n + 3 < p.N) {
                    *reinterpret_cast<float4 *>(dst + n) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
                } else {
                    if (n < p.N) dst[n] = v[4 * g];
                    if (n + 1 < p.N) dst[n + 1] = v[4 * g + 1];
                    if (n + 2 < p.N) dst[n + 2] = v[4 * g + 2];
                }
            }
        }
}

bool dma_lds_attr() {
    static int ok = -1;
    if (ok < 0) {
        const void *ks[] = {(const void *)gemm_dma_kernel<false, false>, (const void *)gemm_dma_kernel<true, false>,
                            (const void *)gemm_dma_kernel<false, true>, (const void *)gemm_dma_kernel<true, true>};
        ok = 1;
        for (int i = 0; i < 4; i++)
            if (hipFuncSetAttribute(ks[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)(i < 2 ? DMA_LDS : DMA_LDS_G)) != hipSuccess)
                ok = 0;
    }
    return ok == 1;
}

}  // namespace

int gemm_splits_for(int N, int K, int M, int cus, int kmul) {
    // Grids of at least one 256 x 256 tile per CU take the direct-to-LDS
    // kernel; one whose last round is at most half full (1.5 rounds of q+k+v
    // at 4096 tokens) is split in two over k, which evens the rounds.
    if (K % DBK != 0) return 1;
    const long nb = (long)((N + DBN - 1) / DBN) * ((M + DBM - 1) / DBM);
    const int kt = K / DBK;
    if (nb >= cus) {
        if (kt % (2 * kmul)) return 1;
        const long r1 = (nb + cus - 1) / cus, r2 = (2 * nb + cus - 1) / cus;
        return r2 < 2 * r1 ? 2 : 1;
    }
    // A grid of fewer tiles than CUs (the projections of a small model, or of
    // a few hundred tokens) is split over k where that pays: each split
    // shortens every block's k walk (rounds x k-tiles per split, ~1.6 us per
    // k-tile), and each split past the first writes one more fp32 partial of
    // the output that the consumer reads back (M x N x 8 bytes at ~5 TB/s).
    // Splits keep at least 4 k-tiles.  E.g. Qwen2.5-0.5B at 2048 tokens: q+k+v
    // and o in 4 splits, down (K = 4864) in 8.
    const double tk = 1.6e-6, extra = (double)M * N * 8.0 / 5e12;
    int best = 1;
    double bt = (double)kt * tk;
    for (int s = 2; s <= 16 && kt / s >= 4; s++) {
        if (kt % s || (kt / s) % kmul) continue;
        const double rounds = (double)((nb * s + cus - 1) / cus);
        const double t = rounds * (kt / s) * tk + (s - 1) * extra;
        if (t < bt) { bt = t; best = s; }
    }
    return best;
}

int gemm_splits(int N, int K, int M) { return gemm_splits_for(N, K, M, num_cus()); }
int gemm_splits_f8(int N, int K, int M) { return gemm_splits_for(N, K, M, num_cus(), 2); }

void launch_gemm(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi, const u16 *a_lo,
                 int lda, int M, float *out, int ldo, int ksplit, size_t split_stride) {
    if (M <= 0) return;
    GemmParams p{};
    fill(p, segs, nseg, K, a_hi, a_lo, lda, M, out, ldo);
    // grids of at least one 256 x 256 tile per CU take the direct-to-LDS kernel;
    // smaller ones keep more, smaller blocks
    const long big = (long)((p.N + DBN - 1) / DBN) * ((M + DBM - 1) / DBM);
    if (K % DBK == 0 && (big >= num_cus() || ksplit > 1) && dma_lds_attr()) {
        if (ksplit > 1 && K % (ksplit * DBK) == 0) {
            p.kchunk = K / ksplit;
            p.split_stride = split_stride;
        } else {
            ksplit = 1;
        }
        hipLaunchKernelGGL((gemm_dma_kernel<false, false>),
                           dim3((p.N + DBN - 1) / DBN, (M + DBM - 1) / DBM, ksplit), dim3(DNTHR), DMA_LDS, st, p,
                           nullptr, nullptr);
        return;
    }
    // (one split: the caller asks for more only where gemm_splits gave them)
    dim3 grid((p.N + BN - 1) / BN, (M + BM - 1) / BM, 1);
    gemm_lds_attr();
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(NTHR), GEMM_LDS, st, p);
}

bool launch_gemm_silu(hipStream_t st, const void *w_gate, const void *w_up, int F, int K, const u16 *a_hi,
                      const u16 *a_lo, int lda, int M, u16 *s_hi, u16 *s_lo, int ldo) {
    if (M <= 0) return true;
    const long tiles = (long)((F + DBN / 2 - 1) / (DBN / 2)) * ((M + DBM - 1) / DBM);
    if (K % DBK != 0 || tiles < num_cus() || !dma_lds_attr()) return false;
    GemmParams p{};
    WSeg segs[2] = {{w_gate, F}, {w_up, F}};
    fill(p, segs, 2, K, a_hi, a_lo, lda, M, nullptr, ldo);
    p.N = F;
    hipLaunchKernelGGL((gemm_dma_kernel<true, false>),
                       dim3((F + DBN / 2 - 1) / (DBN / 2), (M + DBM - 1) / DBM, 1), dim3(DNTHR), DMA_LDS, st, p,
                       s_hi, s_lo);
    return true;
}

int gemm_grouped_splits_for(int N, int K, int pairs, int E, int cus) {
    // an expert's row tiles number about pairs/E/256 rounded up: estimate the
    // blocks with rows and split k until the grid fills the CUs one and a half times
    if (K % DBK != 0) return 1;
    const long ntn = (N + DBN - 1) / DBN;
    const long blocks = ntn * ((pairs + DBM - 1) / DBM + E / 2);
    int S = 1;
    while (S < 4 && blocks * S * 2 < 3L * cus && K % (2 * S * DBK) == 0) S *= 2;
    return S;
}

int gemm_grouped_splits(int N, int K, int pairs, int E) { return gemm_grouped_splits_for(N, K, pairs, E, num_cus()); }

void launch_gemm_grouped(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi,
                         const u16 *a_lo, int lda, int max_rows, int E, const int32_t *offsets,
                         size_t expert_stride, float *out, int ldo, int ksplit, size_t split_stride) {
    if (max_rows <= 0) return;
    GemmParams p{};
    fill(p, segs, nseg, K, a_hi, a_lo, lda, max_rows, out, ldo);
    p.grp_off = offsets;
    p.expert_stride = expert_stride;
    if (K % DBK == 0 && dma_lds_attr()) {
        if (ksplit > 1 && K % (ksplit * DBK) == 0) {
            p.kchunk = K / ksplit;
            p.split_stride = split_stride;
            p.ksplit = ksplit;
        }
        hipLaunchKernelGGL((gemm_dma_kernel<false, true>),
                           dim3((p.N + DBN - 1) / DBN, (max_rows + DBM - 1) / DBM, E * p.ksplit), dim3(DNTHR),
                           DMA_LDS_G, st, p, nullptr, nullptr);
        return;
    }
    dim3 grid((p.N + BN - 1) / BN, (max_rows + BM - 1) / BM, E);
    gemm_lds_attr();
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(NTHR), GEMM_LDS, st, p);
}

bool launch_gemm_grouped_silu(hipStream_t st, const void *w_gate, const void *w_up, int F, int K, const u16 *a_hi,
                              const u16 *a_lo, int lda, int max_rows, int E, const int32_t *offsets,
                              size_t expert_stride, u16 *s_hi, u16 *s_lo, int ldo) {
    if (max_rows <= 0) return true;
    if (K % DBK != 0 || !dma_lds_attr()) return false;
    GemmParams p{};
    WSeg segs[2] = {{w_gate, F}, {w_up, F}};
    fill(p, segs, 2, K, a_hi, a_lo, lda, max_rows, nullptr, ldo);
    p.N = F;
    p.grp_off = offsets;
    p.expert_stride = expert_stride;
    hipLaunchKernelGGL((gemm_dma_kernel<true, true>),
                       dim3((F + DBN / 2 - 1) / (DBN / 2), (max_rows + DBM - 1) / DBM, E), dim3(DNTHR), DMA_LDS_G, st,
                       p, s_hi, s_lo);
    return true;
}

// ---- prefill projections on fp16 + fp8 operands -----------------------------
// y = W a with a = a16 + lo (the split of f16_split) and W exact in fp16: the
// hi pass multiplies W16 by a16 on fp16 MFMAs (32x32x16), the lo pass W8 by
// the fp8 lo (e4m3 with an E8M0 scale per 32 k of a row) on the scaled fp8
// MFMA (32x32x64), which runs at twice the bf16 rate.  W8 is no copy: it is
// the upper byte of each fp16 weight, which read as e5m2 is the weight
// truncated to 2 mantissa bits; the lanes take those bytes from the W16
// fragments of the hi pass.  Since |lo| <= 2^-11 |a16|, the truncation and
// e4m3's rounding of lo cost about 2^-14 of a product (a CPU emulation of one
// K = 4096 projection: 2.1e-5 rel L2, against 2.5e-6 for the bf16 pair and
// 2.1e-4 for fp16 alone); the two passes cost 1.5 bf16-MFMA units per
// product against 2 for gemm_dma_kernel's bf16 (hi, lo) pair, and each k-tile
// moves 40 KB into LDS instead of 48.
//
// Operands (bytes): W16 [npad][K] fp16; A16 [M][lda] fp16, A8 [M][lda] e4m3,
// asc [K/32][mpad] (mpad = M rounded up to 256).  Within each 256 rows the
// scales are stored in the order the lanes take them (f8_asc_pos): a lane's 2
// token row tiles (j) give one 16-bit word, byte j being the scale the MFMA's
// selector picks.  An A8 row's 32-k blocks hold k 0-7, 16-23, 8-15, 24-31:
// lane half c2 of a 32x32x16 fp16 fragment holds k 8c2 .. 8c2+7 of each
// 16-k step, so its weight bytes of a k-tile are k {8c2.., 16+8c2..}, which
// the fp8 MFMA pairs with bytes [16 c2, 16 c2 + 16) of the A8 row.  Weight
// rows are stored in the kernel's tile order (the converter writes them so):
// tile tn holds rows [256 tn, 256 tn + 256).  A SILU tile's row r is wave half
// r / 128, MFMA row tile (r % 128) / 32 (0, 1 gate; 2, 3 up), i.e. gate or up
// feature 128 tn + 64 (r / 128) + 32 ((r / 32) & 1) + r % 32.
//
// Stage = one 32-k tile: W16 and A16 as in gemm_dma_kernel (64-byte rows,
// swizzled chunks), A8 (32-byte rows, halves swizzled), the 256 token-row
// scales of the tile's k block.  The fp8 MFMA takes 64 k: lane l (row l % 32,
// half c2 = l / 32) supplies its 16 bytes of its row from the even k-tile and
// the same bytes from the odd one that follows, and the scale of its row's
// even (lanes < 32) or odd (lanes >= 32) k block.  The even tile's fragments
// and scales are kept in registers until the odd tile (the ring refills the
// even tile's stage while the odd one is multiplied).
namespace {

// 16-byte half h of fp8 row r sits at half h ^ f(r) of the row in LDS, so the
// 32 rows an fp8 fragment read touches spread over all banks
__device__ __forceinline__ int f8_half(int r, int h) { return h ^ (((r >> 2) ^ (r >> 3)) & 1); }

struct GemmF8Params {
    const u16 *w16;
    const u16 *a16;
    const uint8_t *a8, *asc;
    int N, K, M, npad, mpad, lda;
    float *out;
    int ldo, kchunk;
    size_t split_stride;
    u16 *s_hi, *s_lo;
};

// stage layout, in u16
constexpr int F8_W16 = 0, F8_A16 = 8192, F8_A8 = 16384, F8_ASC = 20480;
constexpr int F8_STG = 20608;
constexpr size_t F8_LDS = (size_t)DNSTAGE * F8_STG * sizeof(u16);
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <bool SILU>
__global__ void __launch_bounds__(DNTHR, 1) gemm_f8_kernel(GemmF8Params p) {
    extern __shared__ __attribute__((aligned(16))) u16 smem[];
    const int tid = threadIdx.x;
    const int lane = tid % WAVE, wv = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int wn = wv & 1, wm = wv >> 1;
    const int M = p.M, kz = blockIdx.z;
    constexpr int FPT = SILU ? DBN / 2 : DBN;
    const int ntn = (p.N + FPT - 1) / FPT, ntm = gridDim.y;
    const int bid = blockIdx.x + blockIdx.y * gridDim.x;
    int tn, tm;
    if ((ntn & 7) == 0) {
        const int x = bid & 7, lt = bid >> 3, nx = ntn >> 3;
        const int G = DGROUP < ntm ? DGROUP : ntm;
        const int tg = lt / (G * nx), rem = lt - tg * G * nx;
        const int gsz = min(G, ntm - tg * G);
        tn = x * nx + rem / gsz;
        tm = tg * G + rem % gsz;
    } else {
        int b = bid;
        const int nblk = ntn * ntm;
        if ((nblk & 7) == 0) b = (b & 7) * (nblk >> 3) + (b >> 3);
        tn = b / ntm;
        tm = b % ntm;
    }
    const int m0 = tm * DBM;
    if (m0 >= M) return;
    const int n0 = tn * FPT, r0 = tn * DBN;
    const int kz0 = kz * p.kchunk;
    const int nk = min(p.kchunk, p.K - kz0) / DBK;   // even

    // load i (0, 1) of W16 / A16: row (i*8 + wv)*16 + lane/4, logical chunk
    // (lane & 3) ^ ((row >> 2) & 3); A8: row wv*32 + lane/2, logical half
    // f8_half(row, lane & 1); scales: lanes 0-15 of wave 0 the 256 token-row
    // bytes (the other waves load none)
    const u16 *srcw[2], *srca[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int P = (i * 8 + wv) * 64 + lane;
        const int r = P >> 2, c = (P & 3) ^ ((r >> 2) & 3);
        srcw[i] = p.w16 + (size_t)(r0 + r) * p.K + kz0 + c * 8;
        const int m = min(m0 + r, M - 1);
        srca[i] = p.a16 + (size_t)m * p.lda + kz0 + c * 8;
    }
    const int r8 = (wv * 64 + lane) >> 1, c8 = f8_half(r8, lane & 1);
    const uint8_t *srca8 = p.a8 + (size_t)min(m0 + r8, M - 1) * p.lda + kz0 + c8 * 16;
    const uint8_t *srcsc = p.asc + m0 + lane * 16;
    const int kb0 = kz0 / DBK;

    auto load_tile = [&](int kt, int stage, auto na_c, auto sc_c) {
        constexpr int NA = decltype(na_c)::value;
        constexpr int SC = decltype(sc_c)::value;
        const int t = kt < nk ? kt : nk - 1;
        const int k0 = t * DBK;
        LDS_AS u16 *base = (LDS_AS u16 *)smem + stage * F8_STG;
#pragma unroll
        for (int i = 0; i < 2; i++)
            __builtin_amdgcn_global_load_lds((const void *)(srcw[i] + k0),
                                             (LDS_AS void *)(base + F8_W16 + (i * 8 + wv) * 512), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < NA; i++)
            __builtin_amdgcn_global_load_lds((const void *)(srca[i] + k0),
                                             (LDS_AS void *)(base + F8_A16 + (i * 8 + wv) * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(srca8 + k0), (LDS_AS void *)(base + F8_A8 + wv * 512), 16,
                                         0, 0);
        if (SC && lane < 16)
            __builtin_amdgcn_global_load_lds((const void *)(srcsc + (size_t)(kb0 + t) * p.mpad),
                                             (LDS_AS void *)(base + F8_ASC), 16, 0, 0);
    };

    floatx16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

    const int r32 = lane & 31, c2 = lane >> 5;
    // hi pass of one k-tile: fp16 MFMAs as gemm_dma_kernel's bf16 ones
    // w8 gets the upper byte of each W16 fragment element: for the fp8 pass
    // the weight is that byte read as e5m2 (fp16 truncated to 2 mantissa
    // bits), lane half c2 of a tile holding k 8c2 .. 8c2+7 and 16+8c2 ..
    // 16+8c2+7 in its 16 bytes (the A8 rows are stored in that k order)
    auto hi_pass = [&](int s, u32x4 (&w8)[4]) {
        const u16 *sw = smem + s * F8_STG + F8_W16;
        const u16 *sa = smem + s * F8_STG + F8_A16;
#pragma unroll
        for (int ks = 0; ks < DBK / 16; ks++) {
            f16x8 fw[4], fa[2];
#pragma unroll
            for (int i = 0; i < 4; i++)
                fw[i] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                                                      sw + 8 * dswz(wn * 128 + i * 32 + r32, 2 * ks + c2)));
#pragma unroll
            for (int j = 0; j < 2; j++)
                fa[j] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                                                      sa + 8 * dswz(wm * 64 + j * 32 + r32, 2 * ks + c2)));
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const u32x4 b = __builtin_bit_cast(u32x4, fw[i]);
                w8[i][2 * ks] = __builtin_amdgcn_perm(b[1], b[0], 0x07050301u);
                w8[i][2 * ks + 1] = __builtin_amdgcn_perm(b[3], b[2], 0x07050301u);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fw[i], fa[j], acc[i][j], 0, 0, 0);
        }
    };
    // the fp8 fragments of stage s (bytes [16 c2, 16 c2 + 16) of each row) and
    // its scales, packed one byte per row tile (weights: byte i, tokens: byte j)
    auto lo_frags = [&](int s, u32x4 (&a8)[2], uint32_t &as) {
        const uint8_t *sb = reinterpret_cast<const uint8_t *>(smem + s * F8_STG);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int row = wm * 64 + j * 32 + r32;
            a8[j] = *reinterpret_cast<const u32x4 *>(sb + 2 * F8_A8 + row * 32 + f8_half(row, c2) * 16);
        }
        // the scales of the lane's 2 token row tiles
        as = *reinterpret_cast<const uint16_t *>(sb + 2 * F8_ASC + wm * 64 + r32 * 2);
    };

    // per k-tile and wave: 2 W16 + NA A16 + A8 (+ the scales on wave 0) =
    // 3 + NA (+ 1) loads; the wait leaves the newest tile's in flight (see
    // gemm_dma_kernel), and the loop is instantiated per count.  The
    // loop takes k-tiles in pairs (nk is even): the even tile's fp8 fragments
    // and scales stay in registers, since the odd iteration's load refills the
    // even tile's stage.
    auto ring = [&](auto na_c, auto sc_c) {
        constexpr int NA = decltype(na_c)::value;
        constexpr int WAIT = (3 + NA + decltype(sc_c)::value) | (7 << 4) | (0 << 8);
        load_tile(0, 0, na_c, sc_c);
        load_tile(1, 1, na_c, sc_c);
        __builtin_amdgcn_s_waitcnt(WAIT);
        __builtin_amdgcn_s_barrier();
        for (int kt = 0; kt < nk; kt += 2) {
            const int se = kt % DNSTAGE, so = (kt + 1) % DNSTAGE;
            load_tile(kt + 2, (kt + 2) % DNSTAGE, na_c, sc_c);
            u32x4 w8e[4], a8e[2];
            uint32_t ase;
            lo_frags(se, a8e, ase);
            hi_pass(se, w8e);
            __builtin_amdgcn_s_waitcnt(WAIT);
            __builtin_amdgcn_s_barrier();
            load_tile(kt + 3, (kt + 3) % DNSTAGE, na_c, sc_c);
            u32x4 w8o[4], a8o[2];
            uint32_t aso;
            lo_frags(so, a8o, aso);
            // lanes < 32 give the even k block's scales, lanes >= 32 the odd one's;
            // the weights' bytes take scale 2^0
            const int asc = (int)(c2 ? aso : ase);
            hi_pass(so, w8o);
            i32x8 wop[4], aop[2];
#pragma unroll
            for (int i = 0; i < 4; i++)
                wop[i] = i32x8{(int)w8e[i][0], (int)w8e[i][1], (int)w8e[i][2], (int)w8e[i][3],
                               (int)w8o[i][0], (int)w8o[i][1], (int)w8o[i][2], (int)w8o[i][3]};
#pragma unroll
            for (int j = 0; j < 2; j++)
                aop[j] = i32x8{(int)a8e[j][0], (int)a8e[j][1], (int)a8e[j][2], (int)a8e[j][3],
                               (int)a8o[j][0], (int)a8o[j][1], (int)a8o[j][2], (int)a8o[j][3]};
            // (the scale byte selectors are immediates)
#define F8MMA(I, J) \
    acc[I][J] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop[I], aop[J], acc[I][J], 1, 0, 0, 0x7F7F7F7F, J, asc)
            F8MMA(0, 0); F8MMA(0, 1); F8MMA(1, 0); F8MMA(1, 1);
            F8MMA(2, 0); F8MMA(2, 1); F8MMA(3, 0); F8MMA(3, 1);
#undef F8MMA
            __builtin_amdgcn_s_waitcnt(WAIT);
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    };
    const int na = (m0 + wv * 16 < M) + (m0 + (8 + wv) * 16 < M);   // wave-uniform
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (wv == 0) {
        if (na == 2) ring(I2{}, I1{});
        else if (na == 1) ring(I1{}, I1{});
        else ring(I0{}, I1{});
    } else {
        if (na == 2) ring(I2{}, I0{});
        else if (na == 1) ring(I1{}, I0{});
        else ring(I0{}, I0{});
    }

    if constexpr (SILU) {
        // acc[i][j] (gate, i = 0, 1) and acc[i+2][j] (up): feature
        // n0 + wn*64 + i*32 + (e/4)*8 + c2*4 + e%4, token m0 + wm*64 + j*32 + r32
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int m = m0 + wm * 64 + j * 32 + r32;
                if (m >= M) continue;
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int f = n0 + wn * 64 + i * 32 + g * 8 + c2 * 4;
                    uint32_t hb[4], lb[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float gt = acc[i][j][4 * g + e], up = acc[i + 2][j][4 * g + e];
                        split_bf16(gt / (1.0f + expf(-gt)) * up, hb[e], lb[e]);
                    }
                    const size_t off = (size_t)m * p.ldo + f;
                    if (f + 3 < p.N) {
                        *reinterpret_cast<uint2 *>(p.s_hi + off) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                        *reinterpret_cast<uint2 *>(p.s_lo + off) = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (f + e < p.N) {
                                p.s_hi[off + e] = (u16)hb[e];
                                p.s_lo[off + e] = (u16)lb[e];
                            }
                    }
                }
            }
        return;
    }
    // acc[i][j]: features n0 + wn*128 + i*32 + (e/4)*8 + c2*4 + e%4, token m0 + wm*64 + j*32 + r32
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int m = m0 + wm * 64 + j * 32 + r32;
            if (m >= M) continue;
            float *dst = p.out + kz * p.split_stride + (size_t)m * p.ldo;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int n = n0 + wn * 128 + i * 32 + g * 8 + c2 * 4;
                const floatx16 &v = acc[i][j];
                if (n + 3 < p.N) {
                    *reinterpret_cast<float4 *>(dst + n) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
                } else {
                    if (n < p.N) dst[n] = v[4 * g];
                    if (n + 1 < p.N) dst[n + 1] = v[4 * g + 1];
                    if (n + 2 < p.N) dst[n + 2] = v[4 * g + 2];
                }
            }
        }
}

bool f8_lds_attr() {
    static int ok = -1;
    if (ok < 0) {
        ok = hipFuncSetAttribute((const void *)gemm_f8_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)F8_LDS) == hipSuccess &&
             hipFuncSetAttribute((const void *)gemm_f8_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)F8_LDS) == hipSuccess;
    }
    return ok == 1;
}

// Converted weights: row R of the output (kernel tile order), k block kb of
// 32: W16 = fp16(W) (exact for bf16 values in fp16's normal range); rows past
// the matrix are zero.
__global__ void __launch_bounds__(256) convert_f8_kernel(const u16 *__restrict__ s0, const u16 *__restrict__ s1,
                                                          const u16 *__restrict__ s2, int e0, int e1, int N, int K,
                                                          int silu_f, int npad, u16 *__restrict__ w16) {
    const int nb = K / 32;
    const long idx = blockIdx.x * (long)blockDim.x + threadIdx.x;
    if (idx >= (long)npad * nb) return;
    const int R = (int)(idx / nb), kb = (int)(idx % nb);
    const u16 *src = nullptr;
    if (silu_f > 0) {
        const int tn = R >> 8, r = R & 255, t = (r >> 5) & 3;
        const int f = tn * 128 + (r >> 7) * 64 + (t & 1) * 32 + (r & 31);
        if (f < silu_f) src = (t < 2 ? s0 : s1) + (size_t)f * K;
    } else if (R < N) {
        src = R < e0 ? s0 + (size_t)R * K : (R < e1 ? s1 + (size_t)(R - e0) * K : s2 + (size_t)(R - e1) * K);
    }
    u16 *dst16 = w16 + (size_t)R * K + kb * 32;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const u32x4 b = src ? *reinterpret_cast<const u32x4 *>(src + kb * 32 + q * 8) : u32x4{0u, 0u, 0u, 0u};
        u32x4 h;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float lo0, lo1;
            h[e] = f16_split(bf16_bits_to_f32(b[e] & 0xFFFFu), lo0) |
                   (f16_split(__uint_as_float(b[e] & 0xFFFF0000u), lo1) << 16);
        }
        *reinterpret_cast<u32x4 *>(dst16 + q * 8) = h;
    }
}

}  // namespace

bool gemm_f8_ready() { return f8_lds_attr(); }

int f8_npad(int N, bool silu) { return silu ? ((N + 127) / 128) * 256 : ((N + 255) / 256) * 256; }

size_t f8_weight_bytes(int N, int K, bool silu) {
    const size_t np = (size_t)f8_npad(N, silu);
    return (np * K * 2 + 255) & ~(size_t)255;
}

F8Weights f8_weights_at(void *base, int N, int K, bool silu) {
    const size_t np = (size_t)f8_npad(N, silu);
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    char *b = (char *)base;
    F8Weights w;
    w.w16 = (const u16 *)b;
    w.N = N;
    w.K = K;
    w.npad = (int)np;
    w.silu = silu;
    return w;
}

void launch_convert_f8(hipStream_t st, const WSeg *segs, int nseg, int K, bool silu, const F8Weights &w) {
    const u16 *s[3] = {nullptr, nullptr, nullptr};
    int e0 = 0, e1 = 0, end = 0;
    for (int i = 0; i < nseg; i++) {
        s[i] = (const u16 *)segs[i].w;
        end += segs[i].rows;
        if (i == 0) e0 = end;
        if (i == 1) e1 = end;
    }
    if (nseg < 2) e0 = end;
    if (nseg < 3) e1 = end;
    const long n = (long)w.npad * (K / 32);
    hipLaunchKernelGGL(convert_f8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, s[0], s[1], s[2], e0,
                       e1, silu ? 0 : end, K, silu ? w.N : 0, w.npad, (u16 *)w.w16);
}

bool launch_gemm_f8(hipStream_t st, const F8Weights &w, const u16 *a16, const uint8_t *a8, const uint8_t *asc,
                    int mpad, int lda, int M, float *out, int ldo, int ksplit, size_t split_stride) {
    if (M <= 0) return true;
    if (w.silu || w.K % 64 || !f8_lds_attr()) return false;
    if (ksplit < 1 || w.K % (ksplit * 64)) ksplit = 1;
    GemmF8Params p{};
    p.w16 = w.w16;
    p.a16 = a16; p.a8 = a8; p.asc = asc;
    p.N = w.N; p.K = w.K; p.M = M; p.npad = w.npad; p.mpad = mpad; p.lda = lda;
    p.out = out; p.ldo = ldo; p.kchunk = w.K / ksplit; p.split_stride = ksplit > 1 ? split_stride : 0;
    hipLaunchKernelGGL(gemm_f8_kernel<false>, dim3((w.N + DBN - 1) / DBN, (M + DBM - 1) / DBM, ksplit), dim3(DNTHR),
                       F8_LDS, st, p);
    return true;
}

bool launch_gemm_f8_silu(hipStream_t st, const F8Weights &w, const u16 *a16, const uint8_t *a8, const uint8_t *asc,
                         int mpad, int lda, int M, u16 *s_hi, u16 *s_lo, int ldo) {
    if (M <= 0) return true;
    if (!w.silu || w.K % 64 || !f8_lds_attr()) return false;
    GemmF8Params p{};
    p.w16 = w.w16;
    p.a16 = a16; p.a8 = a8; p.asc = asc;
    p.N = w.N; p.K = w.K; p.M = M; p.npad = w.npad; p.mpad = mpad; p.lda = lda;
    p.kchunk = w.K; p.s_hi = s_hi; p.s_lo = s_lo; p.ldo = ldo;
    hipLaunchKernelGGL(gemm_f8_kernel<true>, dim3((w.N + DBN / 2 - 1) / (DBN / 2), (M + DBM - 1) / DBM, 1),
                       dim3(DNTHR), F8_LDS, st, p);
    return true;
}

// ---- fp32 weights (the small fp32 model): one thread per output -----------
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float *__restrict__ w0, const float *__restrict__ w1,
                                                       const float *__restrict__ w2, int e0, int e1, int N, int K,
                                                       const float *__restrict__ a, int lda, float *__restrict__ out,
                                                       int ldo, const int32_t *__restrict__ grp_off,
                                                       size_t expert_stride, int M) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    int m = blockIdx.y, mrow0 = 0;
    size_t wofs = 0;
    if (grp_off) {
        const int e = blockIdx.z;
        mrow0 = grp_off[e];
        if (m >= grp_off[e + 1] - mrow0) return;
        wofs = (size_t)e * expert_stride;
    } else if (m >= M) {
        return;
    }
    if (n >= N) return;
    const float *w = n < e0 ? w0 + (size_t)n * K : (n < e1 ? w1 + (size_t)(n - e0) * K : w2 + (size_t)(n - e1) * K);
    w += wofs;
    const float *x = a + (size_t)(mrow0 + m) * lda;
    float s = 0.f;
    for (int k = 0; k < K; k++) s += w[k] * x[k];
    out[(size_t)(mrow0 + m) * ldo + n] = s;
}

static void launch_f32(hipStream_t st, const WSeg *segs, int nseg, int K, const float *a, int lda, int M,
                       float *out, int ldo, const int32_t *grp, size_t es, int E) {
    const float *w[3] = {nullptr, nullptr, nullptr};
    int e[3] = {0, 0, 0}, end = 0;
    for (int s = 0; s < nseg; s++) {
        w[s] = (const float *)segs[s].w;
        end += segs[s].rows;
        e[s] = end;
    }
    if (nseg < 2) e[0] = end, e[1] = end;
    else if (nseg < 3) e[1] = end;
    dim3 grid((end + 255) / 256, M, E);
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, w[0], w[1], w[2], e[0], e[1], end, K, a, lda,
                       out, ldo, grp, es, M);
}

void launch_gemm_f32(hipStream_t st, const WSeg *segs, int nseg, int K, const float *a, int lda, int M,
                     float *out, int ldo) {
    if (M <= 0) return;
    launch_f32(st, segs, nseg, K, a, lda, M, out, ldo, nullptr, 0, 1);
}

void launch_gemm_f32_grouped(hipStream_t st, const WSeg *segs, int nseg, int K, const float *a, int lda,
                             int max_rows, int E, const int32_t *offsets, size_t expert_stride, float *out,
                             int ldo) {
    if (max_rows <= 0) return;
    launch_f32(st, segs, nseg, K, a, lda, max_rows, out, ldo, offsets, expert_stride, E);
}
