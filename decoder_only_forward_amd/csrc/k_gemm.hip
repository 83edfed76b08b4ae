// Prefill projections on MFMA: out[m][n] = sum_k (a_hi + a_lo)[m][k] * W[n][k].
//
// Both operands are k-contiguous ("NT" layout), which is what the bf16 MFMA
// wants.  The weight tile is the A operand (16 output features per MFMA row
// tile), the activation tile the B operand, fed twice (hi then lo) into the
// same accumulator so the fp32 activations keep ~16 significant bits.
//
// Block tile 128 (features) x 128 (tokens) x 64 (k); 4 waves in 2x2, each wave
// 64 x 64 = 4 x 4 MFMA tiles of 16x16x32.  Tiles are staged through LDS with
// 16-byte global loads; the next k-tile is fetched into registers while the
// current one is multiplied.  Rows are padded by 16 bytes so the MFMA operand
// reads (16 rows x 16 bytes per lane group) fall in distinct banks.
//
// An optional expert grouping (MoE prefill) runs one grid slice per expert over
// that expert's contiguous rows of `a` and its slice of the weights.
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
};

constexpr int BN = 128, BM = 128, BK = 64;
constexpr int LDS_ROW = BK + 8;          // u16 per padded row (144 bytes)
constexpr int TILE_U16 = 128 * LDS_ROW;  // one 128-row tile

__global__ void __launch_bounds__(256, 2) gemm_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) u16 sw[TILE_U16];
    __shared__ __attribute__((aligned(16))) u16 sh[TILE_U16];
    __shared__ __attribute__((aligned(16))) u16 sl[TILE_U16];

    const int tid = threadIdx.x;
    const int lane = tid % WAVE, wv = tid / WAVE;
    const int r = lane & 15, c = lane >> 4;
    const int wn = wv & 1, wm = wv >> 1;  // wave's 64x64 sub-tile: features wn, tokens wm

    int M = p.M, mrow0 = 0;
    size_t wofs = 0;
    if (p.grp_off) {
        const int e = blockIdx.z;
        mrow0 = p.grp_off[e];
        M = p.grp_off[e + 1] - mrow0;
        wofs = (size_t)e * p.expert_stride;
    }
    const int m0 = blockIdx.y * BM;
    if (m0 >= M) return;
    const int n0 = blockIdx.x * BN;

    // global -> LDS assignment: 4 passes of 256 threads over 128 rows x 8 chunks
    const u16 *gw[4];
    const u16 *gh[4];
    const u16 *gl[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int idx = tid + i * 256;
        const int row = idx >> 3, ch = idx & 7;
        int n = n0 + row;
        n = n < p.N ? n : p.N - 1;
        int s = 0, start = 0;
        while (s < p.nseg - 1 && n >= p.seg_end[s]) { start = p.seg_end[s]; s++; }
        gw[i] = p.w[s] + wofs + (size_t)(n - start) * p.K + ch * 8;
        int m = m0 + row;
        m = m < M ? m : M - 1;
        gh[i] = p.a_hi + (size_t)(mrow0 + m) * p.lda + ch * 8;
        gl[i] = p.a_lo + (size_t)(mrow0 + m) * p.lda + ch * 8;
    }
    uint4 rw[4], rh[4], rl[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            rw[i] = *reinterpret_cast<const uint4 *>(gw[i] + k0);
            rh[i] = *reinterpret_cast<const uint4 *>(gh[i] + k0);
            rl[i] = *reinterpret_cast<const uint4 *>(gl[i] + k0);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int idx = tid + i * 256;
            const int row = idx >> 3, ch = idx & 7;
            *reinterpret_cast<uint4 *>(sw + row * LDS_ROW + ch * 8) = rw[i];
            *reinterpret_cast<uint4 *>(sh + row * LDS_ROW + ch * 8) = rh[i];
            *reinterpret_cast<uint4 *>(sl + row * LDS_ROW + ch * 8) = rl[i];
        }
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nk = p.K / BK;
    gload(0);
    for (int kt = 0; kt < nk; kt++) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ks++) {
            bf16x8 fa[4], fh[4], fl[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int wr = wn * 64 + i * 16 + r;
                fa[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(sw + wr * LDS_ROW + ks * 32 + c * 8));
                const int ar = wm * 64 + i * 16 + r;
                fh[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(sh + ar * LDS_ROW + ks * 32 + c * 8));
                fl[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(sl + ar * LDS_ROW + ks * 32 + c * 8));
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fh[j], acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fl[j], acc[i][j], 0, 0, 0);
                }
        }
    }

    // acc[i][j]: features n0 + wn*64 + i*16 + 4c .. +3, token m0 + wm*64 + j*16 + r
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int m = m0 + wm * 64 + j * 16 + r;
        if (m >= M) continue;
        float *dst = p.out + (size_t)(mrow0 + m) * p.ldo;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int n = n0 + wn * 64 + i * 16 + 4 * c;
            const floatx4 v = acc[i][j];
            if (n + 3 < p.N) {
                *reinterpret_cast<float4 *>(dst + n) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                if (n < p.N) dst[n] = v[0];
                if (n + 1 < p.N) dst[n + 1] = v[1];
                if (n + 2 < p.N) dst[n + 2] = v[2];
            }
        }
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
}

}  // namespace

void launch_gemm(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi, const u16 *a_lo,
                 int lda, int M, float *out, int ldo) {
    if (M <= 0) return;
    GemmParams p{};
    fill(p, segs, nseg, K, a_hi, a_lo, lda, M, out, ldo);
    dim3 grid((p.N + BN - 1) / BN, (M + BM - 1) / BM, 1);
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, st, p);
}

void launch_gemm_grouped(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi,
                         const u16 *a_lo, int lda, int max_rows, int E, const int32_t *offsets,
                         size_t expert_stride, float *out, int ldo) {
    if (max_rows <= 0) return;
    GemmParams p{};
    fill(p, segs, nseg, K, a_hi, a_lo, lda, max_rows, out, ldo);
    p.grp_off = offsets;
    p.expert_stride = expert_stride;
    dim3 grid((p.N + BN - 1) / BN, (max_rows + BM - 1) / BM, E);
    hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, st, p);
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
