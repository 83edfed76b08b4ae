// Decode projections: out[b][n] = sum_k W[n][k] * a[b][k] for B <= 64 rows.
//
// The weight matrix is read exactly once per step from HBM and is the A operand
// of bf16 MFMAs (16x16x32).  Activations are fp32 in the forward; they enter
// the MFMA as the pair (hi, lo) of bf16 values whose sum carries ~16 bits, as
// two columns of the B operand, so the product keeps near-fp32 accuracy while
// the weights stay exact.
//
// Block = 4 waves, 128 weight rows (each wave 2 row tiles of 16).  Each 64-k
// stage of the block's weight rows and of the activation columns goes from
// global memory straight into a ring of LDS stages (global_load_lds, no
// register staging), so the weight stream keeps stages in flight while earlier
// ones are multiplied.  Grid = (row tiles, k splits[, experts]) with one block
// per CU and splits = CUs / row tiles, so the matrix is covered in one round;
// split partials are summed by the consumer kernel in a fixed order (no
// atomics).  K must be a multiple of 64 (dec_create admits bf16 weights only
// for such shapes).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

struct GemvParams {
    const u16 *w[MAX_SEGS];
    int seg_end[MAX_SEGS];
    int nseg;
    int N, K;
    const u16 *a_hi, *a_lo;
    int lda, B;
    float *out;
    size_t split_stride;
    int ldo;
    int kps;   // k per split (multiple of 64)
    // Grouped experts: expert e = blockIdx.z owns grouped rows
    // [grp_off[e], grp_off[e+1]) and weight slice e (w + e*expert_stride);
    // grouped row r reads activation row r, or, with row_pairs, the token row
    // row_pairs[r] / row_k (activations in token order).
    const int32_t *grp_off;
    size_t expert_stride;
    const int32_t *row_pairs;
    int row_k;
    int rot;   // start each block's k walk at stage blockIdx.x % stages
    // silu(gate) * up in the epilogue: w[0] gate, w[1] up, N features; the
    // product goes to (s_hi, s_lo) [B][ldo] as bf16 pairs; rt row tiles of 16
    // per block (8 features each)
    u16 *s_hi, *s_lo;
    int rt;
    // residual + RMSNorm of the one batch row formed in the kernel (the RN
    // instances); the (hi, lo) operand of the block's k range then sits in LDS
    RowNorm rn;
    // the one batch row's attention output merged from its split partials in
    // the kernel (the AM instances), into the same LDS operand
    AttnMerge am;
};

constexpr int DKS = 64;            // k per stage
constexpr int DCH = DKS / 8;       // 16-byte chunks per stage row
constexpr int DROWS = 128;         // weight rows per block
constexpr int DNSTAGE = 3;         // LDS ring depth
#define LDS_AS __attribute__((address_space(3)))
constexpr int CPOL_NT = 2;         // cache-policy operand of global_load_lds: the nt bit

template <int NT>
constexpr size_t dma_lds() { return (size_t)DNSTAGE * (DROWS * DKS + 16 * NT * DKS) * 2; }
// one-row instances: the ring, then the (hi, lo) operand of a k range of kps
inline size_t dma_lds_rn(int kps) { return dma_lds<2>() + (size_t)2 * kps * 2; }

// The B operand of one batch row formed by the block itself (PRO): none (the
// ring carries the activation columns), the residual + RMSNorm of the row
// (PRO_RN), or the merge of the row's attention split partials (PRO_AM).
enum { PRO_NONE = 0, PRO_RN = 1, PRO_AM = 2 };

// Stage layout: the weight tile [128 rows][64 k] then the activation tile
// [16*NT columns][64 k] (column t*16 + m: hi of batch row t*8 + m for m < 8,
// lo of batch row t*8 + m - 8 above), bf16; each 128-byte row holds 8 chunks
// of 16 bytes, chunk c of row r stored at c ^ (r & 7), so each group of 8 rows
// an operand read touches covers all banks.
//
// FORM: DENSE, one matrix (up to three row segments); GROUPED, grid z is the
// expert (MoE); SILU_FUSED, row tile t of the block (t < rt <= 8) holds 8
// features of the gate matrix in rows 0-7 and the same 8 of the up matrix in
// rows 8-15, and the epilogue writes silu(gate) * up (single k split only).
// With 8 features per tile the grid can be sized to the CU count (Mistral's
// 14336 features: 7 tiles in each of 256 blocks).
enum { DENSE = 0, SILU_FUSED = 1, GROUPED = 2 };

// s_waitcnt immediate that lets n loads per stage of the newest DNSTAGE-2
// stages stay outstanding: vmcnt (bits 3:0 and 15:14), expcnt 7, lgkmcnt 0
constexpr int ring_wait(int n) {
    return ((n * (DNSTAGE - 2)) & 15) | (7 << 4) | (0 << 8) | (((n * (DNSTAGE - 2)) >> 4) << 14);
}

// PRO_RN / PRO_AM: one batch row whose operand the block forms itself (the
// residual + RMSNorm of p.rn, or the split merge of p.am): the ring carries
// only weights, and the B operand comes from the row's (hi, lo) pair of the
// block's k range, kept in LDS after the ring.
template <int NT, int FORM, int PRO = PRO_NONE>
__global__ void __launch_bounds__(256, 1) gemv_dma_kernel(GemvParams p) {
    constexpr bool SILU = FORM == SILU_FUSED;
    static_assert(NT >= 2, "the activation tile needs one load per wave");
    constexpr bool RN = PRO != PRO_NONE;   // one row, operand in LDS
    static_assert(!RN || (NT == 2 && FORM != GROUPED), "one dense or fused-SwiGLU row");
    static_assert(PRO != PRO_AM || FORM == DENSE, "the merged attention row feeds a dense projection");
    extern __shared__ __attribute__((aligned(16))) u16 smem[];
    __shared__ float rn_red[16];
    constexpr int NSTAGE = DNSTAGE;
    constexpr int WST = DROWS * DKS;           // u16 of the weight tile
    constexpr int STG = WST + 16 * NT * DKS;   // u16 per stage
    constexpr int NW = DROWS * DCH / 256;      // weight loads per thread per stage (4)
    constexpr int NLD = RN ? NW : NW + NT / 2; // 16-byte loads per thread per stage
    // the wave index as a scalar: tests on it branch per wave, not per lane
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, c = lane >> 4;
    int B = p.B, arow0 = 0;
    size_t wofs = 0;
    if constexpr (FORM == GROUPED) {
        // grouped experts: expert e = blockIdx.z owns activation (and output)
        // rows [grp_off[e], grp_off[e+1]) and weight slice e
        const int e = blockIdx.z;
        arow0 = p.grp_off[e];
        B = p.grp_off[e + 1] - arow0;
        if (B <= 0) return;
        wofs = (size_t)e * p.expert_stride;
    }
    const int RT = SILU ? p.rt : DROWS / 16;   // row tiles of 16 in use
    const int n0 = blockIdx.x * (SILU ? 8 * RT : DROWS);
    const int kbeg = blockIdx.y * p.kps;
    const int kend = min(p.K, kbeg + p.kps);
    const int nst = kbeg < kend ? (kend - kbeg) / DKS : 0;
    // Rows whose pitch is a multiple of 8 KB, read at one column offset by
    // every block at once, concentrate on few memory channels; a per-block
    // start stage spreads the column offsets in flight.
    const int rot = p.rot && nst > 0 ? (int)(blockIdx.x % nst) : 0;
    const int KR = kend - kbeg;                      // RN: the operand row's length in LDS
    u16 *act = smem + NSTAGE * STG;                  // RN: hi [KR], then lo [KR]

    // RN prologue: x_new = x + sum of the split partials over the whole row,
    // its sum of squares, then the normed (hi, lo) pair of [kbeg, kend) into
    // LDS; the residual + RMSNorm kernel's operations (split partials summed
    // in order, then added to x; a = x * rs * g), with the sum of squares
    // reduced over this block's 256 threads (its own lane and wave order).
    auto rn_prologue = [&]() {
        const RowNorm &n = p.rn;
        const int nv = n.d / 4;
        constexpr int VPT = 8;
        float4 v[VPT];
        float ss = 0.f;
        const bool first = blockIdx.x == 0 && blockIdx.y == 0;
#pragma unroll
        for (int u = 0; u < VPT; u++) {
            const int i4 = tid + u * 256;
            if (i4 >= nv) break;
            float4 r4 = *reinterpret_cast<const float4 *>(n.x + 4 * i4);
            if (n.add.p) {
                const float4 a = sum_splits4(n.add.p, n.add.S, n.add.stride, (size_t)4 * i4);
                r4.x += a.x; r4.y += a.y; r4.z += a.z; r4.w += a.w;
            }
            v[u] = r4;
            ss += r4.x * r4.x + r4.y * r4.y + r4.z * r4.z + r4.w * r4.w;
            if (first) {
                *reinterpret_cast<float4 *>(n.x_new + 4 * i4) = r4;
                if (n.cap) *reinterpret_cast<float4 *>(n.cap + 4 * i4) = r4;
            }
        }
        const float tot = block_sum(ss, rn_red);
        const float rs = 1.0f / sqrtf(tot / (float)n.d + n.eps);
#pragma unroll
        for (int u = 0; u < VPT; u++) {
            const int i4 = tid + u * 256;
            if (i4 >= nv) break;
            const int k = 4 * i4;
            if (k < kbeg || k >= kend) continue;
            const float4 g = *reinterpret_cast<const float4 *>(n.gain + k);
            float4 a;
            a.x = v[u].x * rs * g.x; a.y = v[u].y * rs * g.y;
            a.z = v[u].z * rs * g.z; a.w = v[u].w * rs * g.w;
            uint2 h, l;
            split2_bf16(a.x, a.y, h.x, l.x);
            split2_bf16(a.z, a.w, h.y, l.y);
            *reinterpret_cast<uint2 *>(act + (k - kbeg)) = h;
            *reinterpret_cast<uint2 *>(act + KR + (k - kbeg)) = l;
        }
    };

    // AM prologue: element k of [kbeg, kend) is dim k % hd of head k / hd;
    // its split partials o_s (unnormalised), maxima m_s and normalisers l_s
    // combine as sum_s f_s o_s / sum_s f_s l_s with f_s = 2^(m_s - max m), the
    // splits taken in ascending order (the split merge kernel's operations and
    // order).  A thread takes two adjacent dims and issues every (m, l) and
    // (o, o') load of its up to 32 splits at once (lanes of one head read the
    // same (m, l)).
    auto am_prologue = [&]() {
        const AttnMerge &a = p.am;
        const int hd = a.hd, S = a.splits, ld = hd + 2;
        for (int k = kbeg + 2 * tid; k < kend; k += 512) {
            const int h = k / hd, i = k % hd;
            const float *src = a.part + (size_t)h * S * ld;
            float2 ml[32], o[32];
#pragma unroll
            for (int u = 0; u < 32; u++) {
                if (u < S) {
                    ml[u] = *reinterpret_cast<const float2 *>(src + u * ld + hd);
                    o[u] = *reinterpret_cast<const float2 *>(src + u * ld + i);
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < 32; u++)
                if (u < S) mx = fmaxf(mx, ml[u].x);
            float A0 = 0.f, A1 = 0.f, L = 0.f;
#pragma unroll
            for (int u = 0; u < 32; u++) {
                if (u < S) {
                    const float f = ml[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[u].x - mx);
                    L += ml[u].y * f;
                    A0 += o[u].x * f;
                    A1 += o[u].y * f;
                }
            }
            uint32_t hi, lo;
            split2_bf16(A0 / L, A1 / L, hi, lo);
            *reinterpret_cast<uint32_t *>(act + (k - kbeg)) = hi;
            *reinterpret_cast<uint32_t *>(act + KR + (k - kbeg)) = lo;
        }
    };

    // load i of this thread fills stage chunk P = (i*4 + wv)*64 + lane (lane
    // L of a wave writes 16 bytes at the wave's base + 16 L): the weight tile
    // for i < NW, the activation tile after; row P / 8, logical chunk
    // (P % 8) ^ (row & 7)
    const u16 *src[NLD];
#pragma unroll
    for (int i = 0; i < NLD; i++) {
        const int P = (i * 4 + wv) * 64 + lane;
        if (i < NW) {
            const int row = P / DCH, lc = (P % DCH) ^ (row & (DCH - 1));
            if constexpr (SILU) {
                int f = n0 + (row >> 4) * 8 + (row & 7);
                f = f < p.N ? f : p.N - 1;
                src[i] = (((row >> 3) & 1) ? p.w[1] : p.w[0]) + (size_t)f * p.K + kbeg + lc * 8;
            } else {
                int n = n0 + row;
                n = n < p.N ? n : p.N - 1;
                const u16 *wp = p.w[0];
                int start = 0;
                if (p.nseg > 1 && n >= p.seg_end[0]) { wp = p.w[1]; start = p.seg_end[0]; }
                if (p.nseg > 2 && n >= p.seg_end[1]) { wp = p.w[2]; start = p.seg_end[1]; }
                src[i] = wp + wofs + (size_t)(n - start) * p.K + kbeg + lc * 8;
            }
        } else {
            const int Q = P - NW * 256;
            const int col = Q / DCH, lc = (Q % DCH) ^ (col & (DCH - 1));
            const int t = col >> 4, m = col & 15;
            int b = t * 8 + (m & 7);
            b = b < B ? b : B - 1;   // columns past B read a valid row; their outputs are not stored
            const int arow = p.row_pairs ? p.row_pairs[arow0 + b] / p.row_k : arow0 + b;
            src[i] = (m < 8 ? p.a_hi : p.a_lo) + (size_t)arow * p.lda + kbeg + lc * 8;
        }
    }
    // Every iteration issues its loads (the last stage again past the end), so
    // the count of outstanding loads is the same everywhere.  A wave issues the
    // first NWL of its weight loads: all NW, or in the SILU form those of rows
    // in the rt tiles (load i of wave wv fills rows 8*(i*4 + wv)..); the loop
    // is instantiated per count, so its vmcnt waits stay immediates.
    auto load_stage = [&](int g, int stage, auto nwl_c) {
        constexpr int NWL = decltype(nwl_c)::value;
        int gg = (g < nst ? g : nst - 1) + rot;
        gg = gg >= nst ? gg - nst : gg;
        const int k0 = gg * DKS;
        // weights are read once: non-temporal (measured 7.1 TB/s for such loads
        // against 6.3 TB/s without the hint); the activation columns, which
        // every block of a split reads, keep the default policy
#pragma unroll
        for (int i = 0; i < NWL; i++) {
            LDS_AS u16 *dst = (LDS_AS u16 *)smem + stage * STG + (i * 4 + wv) * 512;
            __builtin_amdgcn_global_load_lds((const void *)(src[i] + k0), (LDS_AS void *)dst, 16, 0, CPOL_NT);
        }
#pragma unroll
        for (int i = NW; i < NLD; i++) {
            LDS_AS u16 *dst = (LDS_AS u16 *)smem + stage * STG + (i * 4 + wv) * 512;
            __builtin_amdgcn_global_load_lds((const void *)(src[i] + k0), (LDS_AS void *)dst, 16, 0, 0);
        }
    };

    floatx4 acc[2][NT];
#pragma unroll
    for (int rt = 0; rt < 2; rt++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[rt][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // The tiles of a SILU block past rt are multiplied like the others (on
    // stale LDS) but never stored.
    // the ring's first NSTAGE-1 stages
    auto ring_start = [&](auto nwl_c) {
#pragma unroll
        for (int g = 0; g < NSTAGE - 1; g++) load_stage(g, g, nwl_c);
    };
    auto ring_loop = [&](auto nwl_c) {
        constexpr int NWL = decltype(nwl_c)::value;
        // between stages: wait until the loads of the newest NSTAGE-2 stages at
        // most are outstanding and every LDS read is done, then a plain barrier
        // (__syncthreads would also wait for the newest stages)
        constexpr int NA = RN ? 0 : NT / 2;
        static_assert((NWL + NA) * (NSTAGE - 2) < 64, "vmcnt field");
        constexpr int WAIT = ring_wait(NWL + NA);
        __builtin_amdgcn_s_waitcnt(WAIT);
        __builtin_amdgcn_s_barrier();
        for (int g = 0; g < nst; g++) {
            // stage (g-1) % NSTAGE, which this load refills, was finished by every
            // wave before the previous barrier
            load_stage(g + NSTAGE - 1, (g + NSTAGE - 1) % NSTAGE, nwl_c);
            const u16 *sw = smem + (g % NSTAGE) * STG;
            const u16 *sa = sw + WST;
#pragma unroll
            for (int s = 0; s < DKS / 32; s++) {
                const int lc = s * 4 + c;
                bf16x8 wf[2];
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    const int row = wv * 32 + rt * 16 + r;
                    wf[rt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sw + row * DKS + 8 * (lc ^ (row & (DCH - 1)))));
                }
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const int col = t * 16 + r;
                    bf16x8 bf;
                    if constexpr (RN) {
                        // every column reads the one row's hi (col % 16 < 8) or lo
                        int gg = g + rot;
                        gg = gg >= nst ? gg - nst : gg;
                        bf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                            act + ((r & 8) ? KR : 0) + gg * DKS + 8 * lc));
                    } else {
                        bf = __builtin_bit_cast(
                            bf16x8, *reinterpret_cast<const u32x4 *>(sa + col * DKS + 8 * (lc ^ (col & (DCH - 1)))));
                    }
#pragma unroll
                    for (int rt = 0; rt < 2; rt++)
                        acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[rt], bf, acc[rt][t], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_waitcnt(WAIT);
            __builtin_amdgcn_s_barrier();
        }
        // the loads issued past the last stage must land before the block's LDS
        // is released
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    };
    // RN: the row's operand is formed while the ring's first stages are in
    // flight (its LDS writes are complete and visible after the ring's first
    // wait and barrier)
    if (nst > 0) {
        if constexpr (!SILU) {
            ring_start(std::integral_constant<int, NW>{});
            if constexpr (PRO == PRO_RN) rn_prologue();
            if constexpr (PRO == PRO_AM) am_prologue();
            ring_loop(std::integral_constant<int, NW>{});
        } else {
            static_assert(NW == 4, "one instance per weight-load count");
            int nwl = 0;   // wave-uniform
#pragma unroll
            for (int i = 0; i < NW; i++) nwl += i * 4 + wv < 2 * RT;
#define NWL_SWITCH(F)                                          \
            switch (nwl) {                                     \
                case 4: F(std::integral_constant<int, 4>{}); break; \
                case 3: F(std::integral_constant<int, 3>{}); break; \
                case 2: F(std::integral_constant<int, 2>{}); break; \
                case 1: F(std::integral_constant<int, 1>{}); break; \
                default: F(std::integral_constant<int, 0>{}); break; \
            }
            NWL_SWITCH(ring_start)
            if constexpr (PRO == PRO_RN) rn_prologue();
            NWL_SWITCH(ring_loop)
#undef NWL_SWITCH
        }
    }

    // lane (r, c) holds rows 4c..4c+3 of each row tile for column r; column r
    // (hi) and r+8 (lo) of the same batch row are summed.
    if constexpr (SILU) {
        // gate rows 4c.. of a tile sit in lanes c = 0, 1 and the up rows of the
        // same features in lanes c + 2 (32 lanes on); silu(z) = z / (1 + e^-z),
        // as the separate activation kernel forms it
#pragma unroll
        for (int rt = 0; rt < 2; rt++) {
            const int tile = 2 * wv + rt;
            if (tile >= RT) continue;   // wave-uniform
#pragma unroll
            for (int t = 0; t < NT; t++) {
                floatx4 g = acc[rt][t], u;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    g[j] += __shfl_xor(g[j], 8, WAVE);
                    u[j] = __shfl_xor(g[j], 32, WAVE);
                }
                const int b = t * 8 + (r & 7);
                const int f = n0 + 8 * tile + 4 * c;
                if (c < 2 && r < 8 && b < B && f + 3 < p.N) {
                    uint32_t h[4], l[4];
#pragma unroll
                    for (int j = 0; j < 4; j++) split_bf16(g[j] / (1.0f + expf(-g[j])) * u[j], h[j], l[j]);
                    const size_t o = (size_t)b * p.ldo + f;
                    *reinterpret_cast<uint2 *>(p.s_hi + o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
                    *reinterpret_cast<uint2 *>(p.s_lo + o) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
                }
            }
        }
    } else {
        // each tile's hi and lo columns are summed just before its store; a
        // block wholly inside the N rows stores without per-row checks
        float *out = p.out + (size_t)blockIdx.y * p.split_stride;
        auto store = [&](bool tail) {
#pragma unroll
            for (int t = 0; t < NT; t++) {
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    floatx4 v = acc[rt][t];
#pragma unroll
                    for (int j = 0; j < 4; j++) v[j] += __shfl_xor(v[j], 8, WAVE);
                    const int b = t * 8 + (r & 7);
                    if (r < 8 && b < B) {
                        const int nn = n0 + wv * 32 + rt * 16 + 4 * c;
                        float *dst = out + (size_t)(arow0 + b) * p.ldo + nn;
                        if (!tail || nn + 3 < p.N) {
                            *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                        } else {
                            if (nn < p.N) dst[0] = v[0];
                            if (nn + 1 < p.N) dst[1] = v[1];
                            if (nn + 2 < p.N) dst[2] = v[2];
                        }
                    }
                }
            }
        };
        if (n0 + DROWS <= p.N) store(false);
        else store(true);
    }
}

template <int NT, int FORM>
void launch_dma_nt(hipStream_t st, const GemvParams &p, dim3 grid) {
    // rings above 64 KB need the attribute; a failure shows as a launch error
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void *)gemv_dma_kernel<NT, FORM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)dma_lds<NT>());
        attr = true;
    }
    hipLaunchKernelGGL((gemv_dma_kernel<NT, FORM>), grid, dim3(256), dma_lds<NT>(), st, p);
}

// one row with its residual + RMSNorm formed in the kernel
template <int FORM>
void launch_dma_rn(hipStream_t st, const GemvParams &p, dim3 grid) {
    const size_t lds = dma_lds_rn(p.kps);
    static size_t attr = 0;
    if (attr < lds) {
        (void)hipFuncSetAttribute((const void *)gemv_dma_kernel<2, FORM, PRO_RN>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr = lds;
    }
    hipLaunchKernelGGL((gemv_dma_kernel<2, FORM, PRO_RN>), grid, dim3(256), lds, st, p);
}

void launch_dma_am(hipStream_t st, const GemvParams &p, dim3 grid) {
    const size_t lds = dma_lds_rn(p.kps);
    static size_t attr = 0;
    if (attr < lds) {
        (void)hipFuncSetAttribute((const void *)gemv_dma_kernel<2, DENSE, PRO_AM>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr = lds;
    }
    hipLaunchKernelGGL((gemv_dma_kernel<2, DENSE, PRO_AM>), grid, dim3(256), lds, st, p);
}

template <int FORM>
void launch_dma(hipStream_t st, const GemvParams &p, dim3 grid, int rows) {
    const int NT = (rows + 7) / 8;   // up to 16 rows share the two-tile kernel
    if (NT <= 2) launch_dma_nt<2, FORM>(st, p, grid);
    else if (NT <= 4) launch_dma_nt<4, FORM>(st, p, grid);
    else launch_dma_nt<8, FORM>(st, p, grid);
}

}  // namespace

int num_cus() {
    static int n = 0;
    if (!n) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
    }
    return n;
}

int gemv_max_splits(int N, int K) {
    // one block per CU on up to 256 CUs; a matrix of a few rows (the MoE
    // router) gains little from more blocks while its consumer sums S
    // partials per output, so at most 2N splits
    const int tiles = (N + DROWS - 1) / DROWS;
    int s = 256 / tiles;
    if (s > K / DKS) s = K / DKS;
    if (s > 2 * N) s = 2 * N;
    return s < 1 ? 1 : s;
}

int gemv_grouped_max_splits(int K) { return K / 256 > 0 ? K / 256 : 1; }

// MoE grouped projections: which experts have rows is known only on the
// device, so the grid covers all of them; about 1024 blocks over the row
// tiles of the experts that can be active, splits of 256+ k.
int gemv_grouped_splits(int N, int K, int B) {
    (void)B;
    const int tiles = (N + DROWS - 1) / DROWS;
    const int target = 1024;
    int s = (target + tiles - 1) / tiles;
    const int maxs = gemv_grouped_max_splits(K);
    if (s > maxs) s = maxs;
    if (s < 1) s = 1;
    int kps = (K + s - 1) / s;
    kps = (kps + DKS - 1) / DKS * DKS;
    return (K + kps - 1) / kps;
}

int gemv_splits(int N, int K, int B) {
    (void)B;
    // one block per CU, a single round: splits = CUs / row tiles
    const int tiles = (N + DROWS - 1) / DROWS;
    int s = num_cus() / tiles;
    const int maxs = gemv_max_splits(N, K);
    if (s > maxs) s = maxs;
    if (s < 1) s = 1;
    int kps = (K + s - 1) / s;
    kps = (kps + DKS - 1) / DKS * DKS;
    return (K + kps - 1) / kps;
}

void launch_gemv(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi, const u16 *a_lo,
                 int lda, int B, float *out, int ksplit, size_t split_stride, int ldo, const RowNorm *rn,
                 const AttnMerge *am) {
    GemvParams p{};
    int end = 0;
    for (int s = 0; s < nseg; s++) {
        p.w[s] = (const u16 *)segs[s].w;
        end += segs[s].rows;
        p.seg_end[s] = end;
    }
    p.nseg = nseg;
    p.N = end;
    p.K = K;
    p.a_hi = a_hi;
    p.a_lo = a_lo;
    p.lda = lda;
    p.B = B;
    p.out = out;
    p.split_stride = split_stride;
    p.ldo = ldo;
    p.grp_off = nullptr;
    if (B <= 0) return;
    // exactly `ksplit` splits (the consumer sums that many); a trailing split
    // whose range is empty writes zeros
    int kps = (K + ksplit - 1) / ksplit;
    kps = (kps + DKS - 1) / DKS * DKS;
    p.kps = kps;
    // a row pitch that is a multiple of 8 KB with few split offsets: rotate
    p.rot = (K % 4096 == 0 && ksplit < 8) ? 1 : 0;
    if (rn && B == 1) {
        p.rn = *rn;
        launch_dma_rn<DENSE>(st, p, dim3((p.N + DROWS - 1) / DROWS, ksplit, 1));
        return;
    }
    if (am && B == 1) {
        p.am = *am;
        launch_dma_am(st, p, dim3((p.N + DROWS - 1) / DROWS, ksplit, 1));
        return;
    }
    launch_dma<DENSE>(st, p, dim3((p.N + DROWS - 1) / DROWS, ksplit, 1), B);
}

bool launch_gemv_silu(hipStream_t st, const void *w_gate, const void *w_up, int F, int K, const u16 *a_hi,
                      const u16 *a_lo, int lda, int B, u16 *s_hi, u16 *s_lo, int ldo, const RowNorm *rn) {
    if (B <= 0 || B > 64 || K % DKS != 0 || F % 8 != 0) return false;
    if (rn && B != 1) return false;
    // Up to 32 rows the 8-feature tiles are spread over the CUs (rt tiles per
    // block, one block per CU).  With more rows each block's activation tile
    // outweighs its weight rows, and fewer, full blocks (8 tiles) measured
    // faster (Qwen2.5-0.5B at B = 64: 20 us against 22).
    const int units = F / 8, cus = num_cus();
    int rt = B > 32 ? DROWS / 16 : (units + cus - 1) / cus;
    rt = rt < 1 ? 1 : (rt > DROWS / 16 ? DROWS / 16 : rt);
    const int blocks = (units + rt - 1) / rt;
    GemvParams p{};
    p.w[0] = (const u16 *)w_gate;
    p.w[1] = (const u16 *)w_up;
    p.nseg = 2;
    p.N = F;
    p.K = K;
    p.a_hi = a_hi;
    p.a_lo = a_lo;
    p.lda = lda;
    p.B = B;
    p.ldo = ldo;
    p.kps = K;
    p.rot = K % 4096 == 0 ? 1 : 0;
    p.s_hi = s_hi;
    p.s_lo = s_lo;
    p.rt = rt;
    if (rn) {
        p.rn = *rn;
        launch_dma_rn<SILU_FUSED>(st, p, dim3(blocks, 1, 1));
        return true;
    }
    launch_dma<SILU_FUSED>(st, p, dim3(blocks, 1, 1), B);
    return true;
}

// Grouped-expert form used by the MoE decode path (see k_moe.hip).
void launch_gemv_grouped(hipStream_t st, const WSeg *segs, int nseg, int K, const u16 *a_hi,
                         const u16 *a_lo, int lda, int max_rows, int E, const int32_t *offsets,
                         size_t expert_stride, float *out, int ksplit, size_t split_stride, int ldo,
                         const int32_t *row_pairs, int row_k) {
    GemvParams p{};
    int end = 0;
    for (int s = 0; s < nseg; s++) {
        p.w[s] = (const u16 *)segs[s].w;
        end += segs[s].rows;
        p.seg_end[s] = end;
    }
    p.nseg = nseg;
    p.N = end;
    p.K = K;
    p.a_hi = a_hi;
    p.a_lo = a_lo;
    p.lda = lda;
    p.B = max_rows;
    p.out = out;
    p.split_stride = split_stride;
    p.ldo = ldo;
    p.grp_off = offsets;
    p.expert_stride = expert_stride;
    p.row_pairs = row_pairs;
    p.row_k = row_k;
    if (max_rows <= 0) return;
    int kps = (K + ksplit - 1) / ksplit;
    kps = (kps + DKS - 1) / DKS * DKS;
    p.kps = kps;
    p.rot = (K % 4096 == 0 && ksplit < 8) ? 1 : 0;
    launch_dma<GROUPED>(st, p, dim3((p.N + DROWS - 1) / DROWS, ksplit, E), max_rows);
}
