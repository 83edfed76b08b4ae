// Decode attention: softmax(q k^T / sqrt(hd)) v over the cached positions of
// each row's sequence (zLLM "The Algorithm Layer", section 2; Pantheon "Llama
// Forward Pass", "Grouped Query Attention": query head h reads kv head
// h*n_kv/n_head), with the one-pass online softmax of rml "The decoder",
// section "Attend": a running maximum and normaliser, the partial output
// rescaled when the maximum grows, no score array.
//
// Split-KV: grid (splits, kv heads, rows).  A block streams one kv head's K/V
// rows of one split once from HBM and applies them to all G query heads of the
// group.  LP = HD/DPL lanes share one position, each lane holding DPL of its
// dims (DPL = 16 for groups of up to 4 heads, else 8, which bounds the q and
// accumulator registers); a lane reads its dims as 16-byte words interleaved
// with the other lanes of the group, so each load instruction covers a
// contiguous 16*LP-byte run of the row.  Work that every lane of a group
// repeats (score reduction, softmax update) is paid once per LP lanes, so the
// wider lanes halve it per position.  Scores are reduced within a row of 16
// lanes by DPP moves.  The online softmax runs in base 2: q is pre-scaled by
// log2(e)/sqrt(hd), so each weight is one exp2 of a difference.  Each lane
// group keeps its own running state over the positions it visits; the groups
// are merged at the end (in-wave by shuffles, across waves through LDS), then
// across splits by a merge kernel.
//
// Ring cache: softmax does not depend on key order, and keys are stored already
// rotated, so the readable slots [0, min(pos+1, max_seq)) are read as one
// contiguous range whatever the wrap (Pantheon, "Sliding Window (Mistral)").
//
// RoPE and the K/V store are folded into the prologue: every block forms the
// G rotated queries of its group from the projection's split partials (into
// LDS), and the block whose split covers the row's new slot also forms the
// rotated key and the value of the new position and stores them in the cache
// before its first read of it (the same arithmetic, summation order and
// rounding as launch_rope_kv).
#include "common.h"
#include "kernels.h"
#include "kvcache.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// K/V rows are read once per decode step: non-temporal loads stream them past
// the caches.
__device__ __forceinline__ u32x4 ntload16(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v + (v of the lane given by a DPP pattern within its row of 16 lanes)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    const int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false);
    return v + __int_as_float(o);
}

// Sum over each aligned group of LP lanes (LP <= 16); every lane gets its
// group's sum.  quad_perm [1,0,3,2] and [2,3,0,1] pair lanes at distance 1 and
// 2; row_half_mirror then pairs the two quads of 8 lanes, row_mirror the two
// halves of 16.
template <int LP>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (LP >= 2) v = dpp_add<0xB1>(v);
    if constexpr (LP >= 4) v = dpp_add<0x4E>(v);
    if constexpr (LP >= 8) v = dpp_add<0x141>(v);
    if constexpr (LP >= 16) v = dpp_add<0x140>(v);
    return v;
}

// Per-lane view of a cache row: NV 16-byte words of EPW elements each.  Word w
// of lane u sits at element (w*LP + u)*EPW of the row.  A 24-bit row adds, for
// each word of 8 elements, the 8-byte run of their third bytes, two runs to a
// 16-byte register quad after the NV words (with two words a lane, LP = HD/16,
// the two runs are one 16-byte word of the row: one load).
template <int HD, int DPL, int KT>
struct Row {
    static constexpr int EPW = KT == KV_F32 ? 4 : 8;   // elements per 16-byte word
    static constexpr int NV = DPL / EPW;                // words per lane per row
    static constexpr int NW = KT == KV_F24 ? NV + (NV + 1) / 2 : NV;   // register quads per row
    static constexpr int LP = HD / DPL;
    static constexpr int RB = kv_row_bytes<KT>(HD);
    static __device__ __forceinline__ int dim(int u, int e) { return ((e / EPW) * LP + u) * EPW + e % EPW; }
    static __device__ __forceinline__ void load(const char *row, int u, u32x4 (&r)[NW]) {
        constexpr int ES = KT == KV_F32 ? 4 : 2;
#pragma unroll
        for (int w = 0; w < NV; w++) r[w] = ntload16(row + (size_t)((w * LP + u) * EPW) * ES);
        if constexpr (KT == KV_F24) {
            if constexpr (NV == 2 && LP == HD / 16) {
                r[NV] = ntload16(row + f24_lo_off(HD, u * EPW));
            } else {
#pragma unroll
                for (int w = 0; w < NV; w++) {
                    const u32x2 l = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x2 *>(row + f24_lo_off(HD, (w * LP + u) * EPW)));
                    r[NV + w / 2][2 * (w % 2)] = l[0];
                    r[NV + w / 2][2 * (w % 2) + 1] = l[1];
                }
            }
        }
    }
    static __device__ __forceinline__ void unpack(const u32x4 (&r)[NW], float (&f)[DPL]) {
#pragma unroll
        for (int w = 0; w < NV; w++) {
            if constexpr (KT == KV_F24) {
                const u32x2 l = {r[NV + w / 2][2 * (w % 2)], r[NV + w / 2][2 * (w % 2) + 1]};
                float e8[8];
                f24_unpack8(r[w], l, e8);
#pragma unroll
                for (int j = 0; j < 8; j++) f[w * 8 + j] = e8[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    if constexpr (KT == KV_BF16) {
                        f[w * 8 + 2 * j] = __uint_as_float(r[w][j] << 16);
                        f[w * 8 + 2 * j + 1] = __uint_as_float(r[w][j] & 0xFFFF0000u);
                    } else {
                        f[w * 4 + j] = __uint_as_float(r[w][j]);
                    }
                }
            }
        }
    }
};

__device__ __forceinline__ void store_out(float v, size_t off, u16 *o_hi, u16 *o_lo, float *o_f32) {
    if (o_f32) o_f32[off] = v;
    if (o_hi) {
        uint32_t h, l;
        split_bf16(v, h, l);
        o_hi[off] = (u16)h;
        o_lo[off] = (u16)l;
    }
}

template <int G>
constexpr int dims_per_lane() { return G <= 4 ? 16 : 8; }

// Element pair i of a head: (i, i + hd/2) when rotated with pairing 1, else
// (2i, 2i+1).  x0, x1: the pair's q/k/v values (split partials summed in
// order, bias added); rotated by the row's table entry when rot is set.
template <int HD>
__device__ __forceinline__ void rope_pair(const RopeArgs &ra, int b, size_t row, int i, bool rot, const float *bias,
                                          int &e0, int &e1, float &x0, float &x1) {
    e0 = (rot && ra.pairing) ? i : 2 * i;
    e1 = (rot && ra.pairing) ? i + HD / 2 : 2 * i + 1;
    x0 = sum_splits(ra.qkv.p, ra.qkv.S, ra.qkv.stride, row + e0);
    x1 = sum_splits(ra.qkv.p, ra.qkv.S, ra.qkv.stride, row + e1);
    if (bias) { x0 += bias[e0]; x1 += bias[e1]; }
    if (rot) {
        const float2 cs = ra.tab[(size_t)b * (HD / 2) + i];
        const float r0 = x0 * cs.x - x1 * cs.y, r1 = x0 * cs.y + x1 * cs.x;
        x0 = r0;
        x1 = r1;
    }
}

// Prologue of a decode attention block: the G rotated queries of kv head kvh
// into qs[g][HD] (unscaled), and, when the block's position range [beg, end)
// holds the row's new slot, the rotated key and the value of the new position
// stored in the cache.  Ends with a block barrier: the queries are complete in
// LDS and the new K/V row is stored before any wave reads it.
template <int HD, int KT>
__device__ __forceinline__ void decode_prologue(const RopeArgs &ra, void *kc, void *vc, int b, int kvh, int G, int nh,
                                                int nkv, int p, int max_seq, int beg, int end, size_t head_base,
                                                float (*qs)[HD]) {
    constexpr int HALF = HD / 2;
    const int sp = ra.ring ? p % max_seq : p;
    const bool owner = sp >= beg && sp < end;
    const int qd = nh * HD, kvd = nkv * HD;
    const size_t row = (size_t)b * ra.qkv.ld;
    const int nq = G * HALF, ntask = nq + (owner ? 2 * HALF : 0);
    for (int task = threadIdx.x; task < ntask; task += blockDim.x) {
        int e0, e1;
        float x0, x1;
        if (task < nq) {
            const int h = kvh * G + task / HALF;
            rope_pair<HD>(ra, b, row + (size_t)h * HD, task % HALF, true, ra.bq ? ra.bq + h * HD : nullptr, e0, e1,
                          x0, x1);
            qs[task / HALF][e0] = x0;
            qs[task / HALF][e1] = x1;
        } else {
            const bool isk = task < nq + HALF;
            const int i = isk ? task - nq : task - nq - HALF;
            const float *bias = isk ? ra.bk : ra.bv;
            rope_pair<HD>(ra, b, row + (isk ? qd : qd + kvd) + (size_t)kvh * HD, i, isk,
                          bias ? bias + kvh * HD : nullptr, e0, e1, x0, x1);
            const size_t at = (head_base + sp) * HD;
            if constexpr (KT == KV_BF16) {
                u16 *c = static_cast<u16 *>(isk ? kc : vc) + at;
                c[e0] = (u16)f32_to_bf16_bits(x0);
                c[e1] = (u16)f32_to_bf16_bits(x1);
            } else if constexpr (KT == KV_F24) {
                char *c = static_cast<char *>(isk ? kc : vc) + (head_base + sp) * kv_row_bytes<KV_F24>(HD);
                f24_store(c, HD, e0, x0);
                f24_store(c, HD, e1, x1);
            } else {
                float *c = static_cast<float *>(isk ? kc : vc) + at;
                c[e0] = x0;
                c[e1] = x1;
            }
        }
    }
    __syncthreads();
}

// NWV waves a block: 4 (two blocks resident per CU), or 8 where one block per
// CU takes a (row, kv head) pair whole (24-bit cache: its 48 bytes a lane and
// position keep fewer loads in flight than the fp32 cache's 64, so it takes
// twice the waves; Mistral-7B B = 32: 132 us against 135 in 4-wave blocks,
// while the fp32 cache measured 167 against 164).
template <int HD, int G, int KT, int NWV = 4>
__global__ void __launch_bounds__(NWV * 64, 8 / NWV) attn_decode_kernel(
    RopeArgs ra, void *__restrict__ kc, void *__restrict__ vc,
    const int32_t *__restrict__ pos, const int32_t *__restrict__ slot, int nh, int nkv, int max_seq,
    int splits, float *__restrict__ part, u16 *__restrict__ o_hi, u16 *__restrict__ o_lo,
    float *__restrict__ o_f32) {
    constexpr int DPL = dims_per_lane<G>() < HD ? dims_per_lane<G>() : HD;
    constexpr bool KB = KT == KV_BF16;
    using R = Row<HD, DPL, KT>;
    constexpr int LP = R::LP;                 // lanes per position
    constexpr int PPW = WAVE / LP;            // positions per wave
    constexpr int NG = NWV * PPW;             // lane groups per block
    constexpr int NV = R::NV, NW = R::NW;
    // positions per lane group per iteration: 8 (fp32) or 4 (bf16, 24-bit)
    // words of K and of V in flight per lane
    constexpr int NB = (KT == KV_F32 ? 8 : 4) / NV;
    __shared__ float sm[NWV][G], sl[NWV][G];
    __shared__ float sacc[NWV][G][HD];
    __shared__ float qs[G][HD];

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
    const char *K = static_cast<const char *>(kc) + head_base * R::RB;
    const char *V = static_cast<const char *>(vc) + head_base * R::RB;
    const float qscale = LOG2E / sqrtf((float)HD);

    // Prologue: the group's rotated queries into LDS; the block whose range
    // holds the new slot stores the new position's key and value first.
    decode_prologue<HD, KT>(ra, kc, vc, b, kvh, G, nh, nkv, p, max_seq, beg, end, head_base, qs);

    // fp32 and 24-bit caches: q in fp32.  bf16 cache: q as (hi, lo) bf16 pairs matching
    // the packing of the key words, for v_dot2 against the stored keys.
    constexpr int QN = KB ? DPL / 2 : DPL;
    float qr[G][KB ? 1 : DPL];
    uint32_t qph[G][KB ? QN : 1], qpl[G][KB ? QN : 1];
#pragma unroll
    for (int g = 0; g < G; g++) {
        const float *qg = qs[g];
        if constexpr (KB) {
#pragma unroll
            for (int j = 0; j < QN; j++) {
                uint32_t h0, l0, h1, l1;
                split_bf16(qg[R::dim(u, 2 * j)] * qscale, h0, l0);
                split_bf16(qg[R::dim(u, 2 * j + 1)] * qscale, h1, l1);
                qph[g][j] = h0 | (h1 << 16);
                qpl[g][j] = l0 | (l1 << 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < DPL; e++) qr[g][e] = qg[R::dim(u, e)] * qscale;
        }
    }
    float m[G], l[G], acc[G][DPL];
#pragma unroll
    for (int g = 0; g < G; g++) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; i++) acc[g][i] = 0.f;
    }

    // fp32 or 24-bit cache, groups of up to 4 heads: two stages of NS = NB/2 positions
    // per lane group, software-pipelined: the next stage's K/V loads are issued
    // before the current stage's arithmetic, so the stream stays in flight
    // while it runs (the same registers as one batch of NB; measured 1.4 %
    // faster per Mistral decode step at B = 32).  Otherwise (bf16 cache, wider
    // groups, where it measured slower) one batch of NB positions at a time.
    // The running maximum rescales the accumulators only when it grows.
    constexpr bool PIPE = !KB && G <= 4;
    constexpr int NS = PIPE ? NB / 2 : NB;
    static_assert(!PIPE || NB % 2 == 0, "two stages of NB/2 positions");
    const int span = NG * NS;
    const int nstg = beg < end ? (end - beg + span - 1) / span : 0;
    auto load = [&](u32x4 (&kr)[NS][NW], u32x4 (&vr)[NS][NW], int st) {
        const int base = beg + st * span;
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int j = base + i * NG + gid;
            const int jj = j < end ? j : beg;   // rows past the range read the first row, masked below
            R::load(K + (size_t)jj * R::RB, u, kr[i]);
        }
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const int j = base + i * NG + gid;
            const int jj = j < end ? j : beg;
            R::load(V + (size_t)jj * R::RB, u, vr[i]);
        }
    };
    auto step = [&](const u32x4 (&kr)[NS][NW], const u32x4 (&vr)[NS][NW], int st) {
        const int base = beg + st * span;
        float s[NS][G];
#pragma unroll
        for (int i = 0; i < NS; i++) {
            const bool valid = base + i * NG + gid < end;
            if constexpr (KB) {
#pragma unroll
                for (int g = 0; g < G; g++) {
                    float d = 0.f;
#pragma unroll
                    for (int w = 0; w < NV; w++)
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            // copy the element out first: a bit cast of a vector
                            // element reads the vector's first element
                            const uint32_t kw = kr[i][w][j];
                            const bf16x2 kk = __builtin_bit_cast(bf16x2, kw);
                            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qph[g][w * 4 + j]), kk,
                                                                d, false);
                            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qpl[g][w * 4 + j]), kk,
                                                                d, false);
                        }
                    d = group_sum<LP>(d);
                    s[i][g] = valid ? d : -INFINITY;
                }
            } else {
                float kf[DPL];
                R::unpack(kr[i], kf);
#pragma unroll
                for (int g = 0; g < G; g++) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < DPL; e++) d += qr[g][e] * kf[e];
                    d = group_sum<LP>(d);
                    s[i][g] = valid ? d : -INFINITY;
                }
            }
        }
        // online softmax update per head: s becomes the weights of this stage
#pragma unroll
        for (int g = 0; g < G; g++) {
            float mx = m[g];
#pragma unroll
            for (int i = 0; i < NS; i++) mx = fmaxf(mx, s[i][g]);
            if (mx > m[g]) {
                // the maximum grows (from -inf: everything so far is 0)
                const float corr = fast_exp2(m[g] - mx);
                l[g] *= corr;
#pragma unroll
                for (int e = 0; e < DPL; e++) acc[g][e] *= corr;
                m[g] = mx;
            }
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < NS; i++) {
                s[i][g] = s[i][g] == -INFINITY ? 0.f : fast_exp2(s[i][g] - m[g]);
                ps += s[i][g];
            }
            l[g] += ps;
        }
        // weighted V rows, one row live at a time
#pragma unroll
        for (int i = 0; i < NS; i++) {
            float vf[DPL];
            R::unpack(vr[i], vf);
#pragma unroll
            for (int g = 0; g < G; g++)
#pragma unroll
                for (int e = 0; e < DPL; e++) acc[g][e] += s[i][g] * vf[e];
        }
    };
    if constexpr (PIPE) {
        // Pairs of stages; each stage's successor is loaded unconditionally (a
        // stage past the last reads the range's first row and is never used),
        // so every path into a stage has the same loads in flight and its wait
        // covers its own loads only.  (A conditional load, or a path from a
        // mid-pair exit back to the loop head, makes the compiler's waits also
        // cover the stage just issued, which undoes the pipelining.)
        u32x4 kA[NS][NW], vA[NS][NW], kB[NS][NW], vB[NS][NW];
        if (nstg > 0) load(kA, vA, 0);
        const int npair = nstg >> 1;
        for (int it = 0; it < npair; it++) {
            load(kB, vB, 2 * it + 1);
            step(kA, vA, 2 * it);
            load(kA, vA, 2 * it + 2);
            step(kB, vB, 2 * it + 1);
        }
        if (nstg & 1) step(kA, vA, nstg - 1);
    } else {
        for (int st = 0; st < nstg; st++) {
            u32x4 kr[NS][NW], vr[NS][NW];
            load(kr, vr, st);
            step(kr, vr, st);
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
            const float a = mx == -INFINITY ? 0.f : fast_exp2(m[g] - mx);
            const float bb = mx == -INFINITY ? 0.f : fast_exp2(mo - mx);
            l[g] = l[g] * a + lo * bb;
#pragma unroll
            for (int e = 0; e < DPL; e++) {
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
            for (int e = 0; e < DPL; e++) sacc[wv][g][R::dim(u, e)] = acc[g][e];
        }
    }
    __syncthreads();
    // merge the NWV waves: thread (g, i) handles one output element
    for (int idx = threadIdx.x; idx < G * HD; idx += blockDim.x) {
        const int g = idx / HD, i = idx % HD;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWV; w++) mx = fmaxf(mx, sm[w][g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; w++) {
            const float f = mx == -INFINITY ? 0.f : fast_exp2(sm[w][g] - mx);
            L += sl[w][g] * f;
            A += sacc[w][g][i] * f;
        }
        const int h = kvh * G + g;
        if (splits == 1) {
            store_out(A / L, (size_t)b * nh * HD + (size_t)h * HD + i, o_hi, o_lo, o_f32);
        } else {
            // partial: unnormalised output, base-2 running maximum, normaliser
            float *dst = part + (((size_t)b * nh + h) * splits + split) * (HD + 2);
            dst[i] = A;
            if (i == 0) { dst[HD] = mx; dst[HD + 1] = L; }
        }
    }
}

// ---- MFMA form ----------------------------------------------------------------
// The same split-KV online softmax with the products on MFMA, for groups of up
// to 16 query heads, in blocks of NW = 4 or 8 waves.  A wave takes 16
// positions at a time:
//   S^T = K Q^T    one 16x16 tile (positions x heads, heads past G are zero
//                  queries), 16x16x32 bf16 MFMAs over the head dims;
//   O^T += V^T P^T 16x16x16 bf16 MFMAs, one per 16 output dims.
// The score accumulator leaves lane (r, c) the scores of head r at positions
// 4c..4c+3, which are exactly the four keys that lane feeds the P^T operand, so
// the weights never move; every lane's output accumulators are also of head
// r, so the online-softmax state is per lane (the maximum is reduced over the
// four lanes of a head).  Each K/V row is read once for all heads of the
// group.  V goes through a per-wave LDS stage to be read transposed.  fp32
// operands are split into bf16 (hi, lo) pairs, products hi*hi + hi*lo + lo*hi
// (a bf16 cache is exact: hi*hi + hi*lo with the query's pair), which keeps
// fp32 accuracy.  The next chunk's K and V loads are issued before the current
// chunk's arithmetic.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split8(const float (&v)[8], bf16x8 &hi, bf16x8 &lo) {
    u32x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint32_t a, bb;
        split2_bf16(v[2 * j], v[2 * j + 1], a, bb);
        h[j] = a;
        l[j] = bb;
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ void split4(const float (&v)[4], s16x4 &hi, s16x4 &lo) {
    uint32_t h0, l0, h1, l1;
    split2_bf16(v[0], v[1], h0, l0);
    split2_bf16(v[2], v[3], h1, l1);
    hi = __builtin_bit_cast(s16x4, make_uint2(h0, h1));
    lo = __builtin_bit_cast(s16x4, make_uint2(l0, l1));
}

// Order this wave's LDS writes before its other lanes' reads (and the reads
// before the next writes): the waves of a block run different step counts,
// so only the wave itself is synchronised.  A wave's LDS operations complete
// in order, so waiting for them (lgkmcnt 0) and keeping the compiler from
// moving memory accesses across is enough; the next step's global loads stay
// in flight (a workgroup-scope fence would also wait for those).
// s_waitcnt fields: vmcnt 63 (no wait), expcnt 7, lgkmcnt 0.
constexpr int WAIT_LGKM0 = 0xF | (7 << 4) | (0 << 8) | (3 << 14);
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// A 24-bit cache goes the fp32 way from registers on: its rows are rebuilt
// as fp32 words, whose bf16 (hi, lo) split is exact (16 significant bits).
// Its loads take the bf16 cache's dim order (8 consecutive dims a lane: one
// 16-byte word of upper halves and the 8-byte run of their third bytes), and
// its V pieces are 8 elements in two register quads.
template <int HD, int KT>
struct MfmaDec {
    static constexpr bool KB = KT == KV_BF16;
    static constexpr int ES = KB ? 2 : 4;         // bytes of a staged V element
    static constexpr int CH = 16;                 // positions per wave step
    static constexpr int NKS = HD / 32;           // k steps of S^T = K Q^T
    static constexpr int NDT = HD / 16;           // 16-dim tiles of O^T
    static constexpr int KW = KB ? 1 : 2;         // register quads of a lane's 8 key dims
    static constexpr int RB = kv_row_bytes<KT>(HD);   // bytes of a cache row
    static constexpr int EPP = KT == KV_F32 ? 4 : 8;  // elements of a V piece
    static constexpr int VQ = KT == KV_F24 ? 2 : 1;   // register quads of a V piece
    static constexpr int PPR = HD / EPP;          // V pieces per row
    static constexpr int VW = CH * PPR / WAVE;    // V pieces per lane per step
    static constexpr int VLD = KB ? HD + 8 : HD + 4;   // elements per staged V row
    static constexpr int VSTAGE = CH * VLD * ES;  // bytes of one wave's V stage
    static constexpr int SACC = 16 * HD * 4;      // bytes of one wave's output block (the merge)
    static constexpr int WBYTES = VSTAGE > SACC ? VSTAGE : SACC;
};

template <int HD, int KT, int NW>
__global__ void __launch_bounds__(NW * 64, NW <= 4 ? 2 : 1) attn_decode_mfma_kernel(
    RopeArgs ra, void *__restrict__ kc, void *__restrict__ vc, const int32_t *__restrict__ pos,
    const int32_t *__restrict__ slot, int nh, int nkv, int max_seq, int splits, float *__restrict__ part,
    u16 *__restrict__ o_hi, u16 *__restrict__ o_lo, float *__restrict__ o_f32) {
    using C = MfmaDec<HD, KT>;
    constexpr bool KB = C::KB;
    constexpr int CH = C::CH, NKS = C::NKS, NDT = C::NDT, KW = C::KW, VW = C::VW, PPR = C::PPR, ES = C::ES;
    constexpr int VQ = C::VQ, EPP = C::EPP;
    __shared__ float qs[16][HD];
    __shared__ __attribute__((aligned(16))) char wst[NW][C::WBYTES];   // V stage, then the wave's outputs
    __shared__ float sm[NW][16], sl[NW][16];

    const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int r = lane & 15, c = lane >> 4;
    const int G = nh / nkv;

    const int p = pos[b];
    const int nread = min(p + 1, max_seq);
    const int chunk = (nread + splits - 1) / splits;
    const int beg = split * chunk;
    const int end = min(nread, beg + chunk);
    const size_t head_base = ((size_t)slot[b] * nkv + kvh) * max_seq;
    const char *K = static_cast<const char *>(kc) + head_base * C::RB;
    const char *V = static_cast<const char *>(vc) + head_base * C::RB;

    // The 8 dims lane (r, c) takes in k step ks (the same for the query and the
    // keys; any assignment of dims to MFMA k slots gives the same dot product):
    // with 4-byte elements, element e is dim 32ks + 16(e/4) + 4c + e%4, so one
    // load instruction (16 bytes per lane) covers 64 contiguous bytes of each
    // key row; with 2-byte elements (and the 24-bit rows' upper halves) dims
    // 32ks + 8c + e do the same.
    auto kdim = [&](int ks, int e) {
        return KT != KV_F32 ? 32 * ks + 8 * c + e : 32 * ks + 16 * (e >> 2) + 4 * c + (e & 3);
    };
    auto load = [&](int c0, u32x4 (&kr)[NKS][KW], u32x4 (&vr)[VW * VQ]) {
        // A operand of S^T: lane (r, c) reads position c0 + r at dims kdim(ks, .)
        const int j = c0 + r;
        const char *krow = K + (size_t)(j < end ? j : beg) * C::RB;
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) {
            if constexpr (KT == KV_F24) {
                kr[ks][0] = ntload16(krow + kdim(ks, 0) * 2);
                const u32x2 l = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(krow + f24_lo_off(HD, kdim(ks, 0))));
                kr[ks][1][0] = l[0];
                kr[ks][1][1] = l[1];
            } else {
#pragma unroll
                for (int w = 0; w < KW; w++) kr[ks][w] = ntload16(krow + kdim(ks, 4 * w) * ES);
            }
        }
        // V rows c0 .. c0+15 as pieces of EPP elements, piece f = q*64 + lane
#pragma unroll
        for (int q = 0; q < VW; q++) {
            const int f = q * WAVE + lane, rr = f / PPR, cc = f % PPR;
            const int jv = c0 + rr;
            const char *vrow = V + (size_t)(jv < end ? jv : beg) * C::RB;
            if constexpr (KT == KV_F24) {
                vr[2 * q] = ntload16(vrow + 16 * cc);
                const u32x2 l = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(vrow + f24_lo_off(HD, 8 * cc)));
                vr[2 * q + 1][0] = l[0];
                vr[2 * q + 1][1] = l[1];
            } else {
                vr[q] = ntload16(vrow + 16 * cc);
            }
        }
    };

    for (int i = threadIdx.x; i < (16 - G) * HD; i += blockDim.x) qs[G + i / HD][i % HD] = 0.f;
    decode_prologue<HD, KT>(ra, kc, vc, b, kvh, G, nh, nkv, p, max_seq, beg, end, head_base, qs);

    // B operand of S^T: head r's query over kdim's dims, scaled for base-2
    // softmax, as a bf16 (hi, lo) pair
    const float qscale = LOG2E / sqrtf((float)HD);
    bf16x8 qh[NKS], ql[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ks++) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; e++) v[e] = qs[r][kdim(ks, e)] * qscale;
        split8(v, qh[ks], ql[ks]);
    }

    float m = -INFINITY, lsum = 0.f;
    floatx4 o[NDT];
#pragma unroll
    for (int d = 0; d < NDT; d++) o[d] = (floatx4){0.f, 0.f, 0.f, 0.f};
    char *vs = wst[wv];

    auto step = [&](int c0, const u32x4 (&kr)[NKS][KW], const u32x4 (&vr)[VW * VQ]) {
#pragma unroll
        for (int q = 0; q < VW; q++) {
            const int f = q * WAVE + lane, rr = f / PPR, cc = f % PPR;
            if constexpr (KT == KV_F24) {
                // staged as the fp32 words
                float e8[8];
                f24_unpack8(vr[2 * q], (u32x2){vr[2 * q + 1][0], vr[2 * q + 1][1]}, e8);
                float *dst = reinterpret_cast<float *>(vs + rr * C::VLD * ES) + EPP * cc;
                *reinterpret_cast<float4 *>(dst) = make_float4(e8[0], e8[1], e8[2], e8[3]);
                *reinterpret_cast<float4 *>(dst + 4) = make_float4(e8[4], e8[5], e8[6], e8[7]);
            } else {
                *reinterpret_cast<u32x4 *>(vs + rr * C::VLD * ES + 16 * cc) = vr[q];
            }
        }
        floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) {
            if constexpr (KB) {
                const bf16x8 kh = __builtin_bit_cast(bf16x8, kr[ks][0]);
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[ks], st, 0, 0, 0);
            } else {
                bf16x8 kh, kl;
                if constexpr (KT == KV_F24) {
                    // hi: the stored upper halves; lo: the rest of each rebuilt word, exact in bf16
                    float v[8];
                    f24_unpack8(kr[ks][0], (u32x2){kr[ks][1][0], kr[ks][1][1]}, v);
                    u32x4 lw;
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const float l0 = v[2 * j] - __uint_as_float(kr[ks][0][j] << 16);
                        const float l1 = v[2 * j + 1] - __uint_as_float(kr[ks][0][j] & 0xFFFF0000u);
                        lw[j] = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u);
                    }
                    kh = __builtin_bit_cast(bf16x8, kr[ks][0]);
                    kl = __builtin_bit_cast(bf16x8, lw);
                } else {
                    float v[8];
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        v[j] = __uint_as_float(kr[ks][0][j]);
                        v[4 + j] = __uint_as_float(kr[ks][1][j]);
                    }
                    split8(v, kh, kl);
                }
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql[ks], st, 0, 0, 0);
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[ks], st, 0, 0, 0);
            }
        }
        // lane (r, c): head r, positions c0 + 4c + e; online softmax of head r
        float sv[4], tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            sv[e] = c0 + 4 * c + e < end ? st[e] : -INFINITY;
            tmax = fmaxf(tmax, sv[e]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, WAVE));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
        const float mnew = fmaxf(m, tmax);
        const float corr = m == -INFINITY ? 0.f : fast_exp2(m - mnew);
        float pw[4], ps = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            pw[e] = sv[e] == -INFINITY ? 0.f : fast_exp2(sv[e] - mnew);
            ps += pw[e];
        }
        lsum = lsum * corr + ps;
        m = mnew;
        s16x4 ph, pl;
        split4(pw, ph, pl);
        wave_lds_sync();
        // A operand of O^T: lane (r, c) holds dim 16d + r of positions 4c .. 4c+3
#pragma unroll
        for (int d = 0; d < NDT; d++) {
#pragma unroll
            for (int e = 0; e < 4; e++) o[d][e] *= corr;
            if constexpr (KB) {
                const u16 *vrow = reinterpret_cast<const u16 *>(vs) + 16 * d + r;
                uint32_t w0 = (uint32_t)vrow[(4 * c) * C::VLD] | ((uint32_t)vrow[(4 * c + 1) * C::VLD] << 16);
                uint32_t w1 = (uint32_t)vrow[(4 * c + 2) * C::VLD] | ((uint32_t)vrow[(4 * c + 3) * C::VLD] << 16);
                const s16x4 vh = __builtin_bit_cast(s16x4, make_uint2(w0, w1));
                o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vh, ph, o[d], 0, 0, 0);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vh, pl, o[d], 0, 0, 0);
            } else {
                const float *vrow = reinterpret_cast<const float *>(vs) + 16 * d + r;
                float vv[4];
#pragma unroll
                for (int e = 0; e < 4; e++) vv[e] = vrow[(4 * c + e) * C::VLD];
                s16x4 vh, vl;
                split4(vv, vh, vl);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vh, ph, o[d], 0, 0, 0);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vh, pl, o[d], 0, 0, 0);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vl, ph, o[d], 0, 0, 0);
            }
        }
        wave_lds_sync();
    };

    // Steps of this wave: positions c0, c0 + NW*CH, ...  Each step's loads are
    // issued unconditionally one step ahead (a step past the range reads valid
    // rows and is never used), so the count of loads in flight is the same on
    // every path and each step waits only for its own data.
    {
        int c0 = beg + wv * CH;
        const int nsteps = c0 < end ? (end - c0 + NW * CH - 1) / (NW * CH) : 0;
        u32x4 kA[NKS][KW], vA[VW * VQ], kB[NKS][KW], vB[VW * VQ];
        if (nsteps > 0) load(c0, kA, vA);
        for (int it = 0; it < nsteps; it += 2) {
            load(c0 + NW * CH, kB, vB);
            step(c0, kA, vA);
            if (it + 1 >= nsteps) break;
            load(c0 + 2 * NW * CH, kA, vA);
            step(c0 + NW * CH, kB, vB);
            c0 += 2 * NW * CH;
        }
    }
    lsum += __shfl_xor(lsum, 16, WAVE);
    lsum += __shfl_xor(lsum, 32, WAVE);

    // merge the NW waves: each writes its state and its output block (which
    // reuses its V stage) to LDS
    __syncthreads();
    float(*sacc)[HD] = reinterpret_cast<float(*)[HD]>(wst[wv]);
    if (r < G) {
        if (c == 0) { sm[wv][r] = m; sl[wv][r] = lsum; }
#pragma unroll
        for (int d = 0; d < NDT; d++)
#pragma unroll
            for (int e = 0; e < 4; e++) sacc[r][16 * d + 4 * c + e] = o[d][e];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * HD; idx += blockDim.x) {
        const int g = idx / HD, i = idx % HD;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; w++) mx = fmaxf(mx, sm[w][g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) {
            const float f = mx == -INFINITY ? 0.f : fast_exp2(sm[w][g] - mx);
            L += sl[w][g] * f;
            A += reinterpret_cast<const float(*)[HD]>(wst[w])[g][i] * f;
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

// Merge of the splits of one (row, head): weights f_s = 2^(m_s - max m) are
// formed once per split into LDS; every output dim then sums its splits in
// ascending order (the loads of a batch issued together), and so does the
// normaliser.  At most 64 splits (the launcher's bound).
__global__ void __launch_bounds__(128) attn_merge_kernel(int nh, int hd, int splits, const float *__restrict__ part,
                                                         u16 *__restrict__ o_hi, u16 *__restrict__ o_lo,
                                                         float *__restrict__ o_f32) {
    __shared__ float fs[64], ls[64];
    __shared__ float sL;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int ld = hd + 2;
    const float *src = part + ((size_t)b * nh + h) * splits * ld;
    if (tid < WAVE) {
        const float ms = tid < splits ? src[tid * ld + hd] : -INFINITY;
        const float mx = wave_max(ms);
        if (tid < splits) {
            fs[tid] = ms == -INFINITY ? 0.f : fast_exp2(ms - mx);
            ls[tid] = src[tid * ld + hd + 1];
        }
    }
    __syncthreads();
    if (tid == 0) {
        float L = 0.f;
        for (int s = 0; s < splits; s++) L += ls[s] * fs[s];
        sL = L;
    }
    __syncthreads();
    const float L = sL;
    for (int i = tid; i < hd; i += blockDim.x) {
        float A = 0.f;
        int s = 0;
        for (; s + 8 <= splits; s += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) v[u] = src[(s + u) * ld + i];
#pragma unroll
            for (int u = 0; u < 8; u++) A += v[u] * fs[s + u];
        }
        for (; s < splits; s++) A += src[s * ld + i] * fs[s];
        store_out(A / L, (size_t)b * nh * hd + (size_t)h * hd + i, o_hi, o_lo, o_f32);
    }
}

template <int HD, int KT>
bool launch_decode_hd(hipStream_t st, int G, dim3 grid, const RopeArgs &ra, void *kc, void *vc,
                      const int32_t *pos, const int32_t *slot, int nh, int nkv, int max_seq, int splits,
                      float *part, u16 *o_hi, u16 *o_lo, float *o_f32, bool wide) {
    if constexpr (KT == KV_F24 && HD >= 64) {
        // one 8-wave block per (row, kv head) pair
        if (wide && G <= 4) {
#define ADW(GG) hipLaunchKernelGGL((attn_decode_kernel<HD, GG, KT, 8>), grid, dim3(512), 0, st, ra, kc, vc, pos, \
                                   slot, nh, nkv, max_seq, splits, part, o_hi, o_lo, o_f32)
            switch (G) {
                case 1: ADW(1); return true;
                case 2: ADW(2); return true;
                case 3: ADW(3); return true;
                case 4: ADW(4); return true;
            }
#undef ADW
        }
    }
    (void)wide;
#define AD(GG) hipLaunchKernelGGL((attn_decode_kernel<HD, GG, KT>), grid, dim3(256), 0, st, ra, kc, vc, pos, \
                                  slot, nh, nkv, max_seq, splits, part, o_hi, o_lo, o_f32)
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

template <int KT>
const void *decode_probe_fn(int hd) {
    return hd == 128 ? (const void *)attn_decode_kernel<128, 4, KT>
         : hd == 64  ? (const void *)attn_decode_kernel<64, 4, KT>
                     : (const void *)attn_decode_kernel<16, 4, KT>;
}

// Groups of more than 4 heads, and any group with a bf16 cache (head_dim 64 or
// 128), take the MFMA form: the lane-group kernel repeats each position's
// softmax update and V products for every head of the group, which made a
// 7-head group, and the bf16 cache's v_dot2 scores, ALU-limited.  An fp32 or
// 24-bit cache with up to 4 heads stays on the lane-group kernel, which
// streams an fp32 cache at 83 % of HBM (its MFMA form at head_dim 128 spills
// registers).
bool use_mfma(int hd, int G, int kv_kind) {
    return G <= 16 && (hd == 64 || hd == 128) && (G > 4 || kv_kind == KV_BF16);
}

}  // namespace

int attn_decode_splits(int B, int nkv, int readable, int hd, int G, int kv_kind) {
    if (use_mfma(hd, G, kv_kind)) {
        // As many (row, kv head) pairs as CUs: one 8-wave block each, no merge
        // (Mistral-7B, bf16 cache, B = 32: 84 us against 91 us for 4-wave
        // blocks in two splits).  Fewer pairs: 4-wave blocks, two resident per
        // CU, at least one 16-position step per wave (Qwen2.5-0.5B, B = 64:
        // 36 us in four splits against 45 us for one 8-wave block per pair).
        const int pairs = B * nkv;
        if (pairs >= num_cus()) return 1;
        int s = 2 * num_cus() / pairs;
        const int maxs = readable / 64;
        if (s > maxs) s = maxs;
        if (s > 64) s = 64;
        return s < 1 ? 1 : s;
    }
    // One round of blocks.  An fp32 (or 24-bit) cache is streamed at the
    // memory's rate by one block per CU, and each extra split costs the merge
    // pass; with a bf16 cache the lanes' arithmetic is the limit, so every
    // resident-block slot is filled.  At least 128 positions per split.
    const bool kb = kv_kind == KV_BF16;
    static int occ_cache[3] = {0, 0, 0};
    const int which = hd == 128 ? 0 : hd == 64 ? 1 : 2;
    int &occ_c = occ_cache[which];
    if (kb && !occ_c) {
        int occ = 0;
        const void *fn = decode_probe_fn<KV_BF16>(hd);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, 256, 0) != hipSuccess || occ <= 0) occ = 2;
        occ_c = occ;
    }
    (void)G;
    const int slots = (kb ? occ_c : 1) * num_cus();
    int s = slots / (B * nkv);
    const int maxs = readable / 128;
    if (s > maxs) s = maxs;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    return s;
}

void launch_attn_decode(hipStream_t st, int B, const RopeArgs &ra, void *kc, void *vc, int kv_kind,
                        const int32_t *pos, const int32_t *slot, int nh, int nkv, int hd, int max_seq, int splits,
                        float *part, u16 *o_hi, u16 *o_lo, float *o_f32, bool merge) {
    if (B <= 0) return;
    const int G = nh / nkv;
    dim3 grid(splits, nkv, B);
    if (use_mfma(hd, G, kv_kind)) {
        // one 8-wave block per (row, kv head) when the pairs fill the CUs
        // (attn_decode_splits then gives one split), else 4-wave blocks
        const bool wide = splits == 1 && B * nkv >= num_cus();
#define MD(HD, KT, NW) hipLaunchKernelGGL((attn_decode_mfma_kernel<HD, KT, NW>), grid, dim3(NW * 64), 0, st, ra, kc, \
                                          vc, pos, slot, nh, nkv, max_seq, splits, part, o_hi, o_lo, o_f32)
#define MDH(KT)                                                        \
        if (hd == 128) { if (wide) MD(128, KT, 8); else MD(128, KT, 4); } \
        else { if (wide) MD(64, KT, 8); else MD(64, KT, 4); }
        if (kv_kind == KV_BF16) { MDH(KV_BF16) }
        else if (kv_kind == KV_F24) { MDH(KV_F24) }
        else { MDH(KV_F32) }
#undef MDH
#undef MD
        if (splits > 1 && merge)
            hipLaunchKernelGGL(attn_merge_kernel, dim3(nh, B), dim3(hd), 0, st, nh, hd, splits, part, o_hi, o_lo,
                               o_f32);
        return;
    }
    // the lane-group kernel on a 24-bit cache in 8-wave blocks where one split
    // covers the readable range and the pairs fill the CUs
    const bool wide = splits == 1 && B * nkv >= num_cus();
#define LD(HD, KT) launch_decode_hd<HD, KT>(st, G, grid, ra, kc, vc, pos, slot, nh, nkv, max_seq, splits, part, \
                                            o_hi, o_lo, o_f32, wide)
#define LDH(KT)                        \
        if (hd == 128) LD(128, KT);    \
        else if (hd == 64) LD(64, KT); \
        else LD(16, KT);
    if (kv_kind == KV_BF16) { LDH(KV_BF16) }
    else if (kv_kind == KV_F24) { LDH(KV_F24) }
    else { LDH(KV_F32) }
#undef LDH
#undef LD
    if (splits > 1 && merge)
        hipLaunchKernelGGL(attn_merge_kernel, dim3(nh, B), dim3(hd < 64 ? 64 : hd), 0, st, nh, hd, splits, part,
                           o_hi, o_lo, o_f32);
}
