// Device helpers shared by the gfx950 kernels of the decoder forward.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector (a plain ext_vector, unlike uint4, stays in registers
// when held in arrays across loop iterations).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define WAVE 64

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): the pair carries about
// 16 significant bits, so a bf16 MFMA over (hi, lo) against exact bf16 weights
// keeps the product close to fp32 accuracy.
__device__ __forceinline__ void split_bf16(float x, uint32_t &hi, uint32_t &lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// The same split for two values at once, packed as the MFMA operands take
// them (a in the low half, b in the high half): v_cvt_pk_bf16_f32 rounds to
// nearest even, so the bits equal those of split_bf16.
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_cvt){a, b}, bf16x2_cvt));
    const float ah = __uint_as_float(hi << 16), bh = __uint_as_float(hi & 0xFFFF0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_cvt){a - ah, b - bh}, bf16x2_cvt));
}

// ---- fp16 + fp8 split operands of the prefill projections ------------------
// x = hi + lo with hi = fp16(x) (nearest even; |x| above the fp16 maximum is
// first clamped to it) and lo = x - hi, exact in fp32 (|lo| <= 2^-11 |hi| for
// normal hi).  lo is stored as OCP fp8 e4m3 (largest finite 448) with one E8M0
// scale 2^(s - 127) per 32 consecutive k of a row: s - 127 is the smallest
// exponent e with max |lo| <= 448 * 2^e over the 32 values, so the scaled
// values stay finite and the largest keeps e4m3's 3 mantissa bits.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f16_split(float x, float &lo) {
    const _Float16 h = (_Float16)fminf(fmaxf(x, -65504.f), 65504.f);
    lo = x - (float)h;
    return __builtin_bit_cast(uint16_t, h);
}

// E8M0 byte of a block whose largest magnitude is m (0 for an all-zero block).
__device__ __forceinline__ uint32_t mx_scale_byte(float m) {
    if (!(m > 0.f)) return 0u;
    int ex;
    const float f = frexpf(m, &ex);          // m = f * 2^ex, f in [0.5, 1)
    // 448 = 0.875 * 2^9: m <= 448 * 2^(ex - 9) exactly when f <= 0.875
    int e = ex - 9 + (f > 0.875f ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    return (uint32_t)(e + 127);
}

// Four values times 2^(127 - s) as fp8 e4m3 (nearest even), value i in byte i.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, uint32_t s) {
    const int sh = 127 - (int)s;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(a, sh), ldexpf(b, sh), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(c, sh), ldexpf(d, sh), w, true);
    return (uint32_t)w;
}

// Position of row r's scale within its 256-row group, in the order the fp16 +
// fp8 GEMM's lanes read them: wave row group wm = q / 64, row tile
// j = (q / 32) % 2 -> 64 wm + 2 (q % 32) + j.
__host__ __device__ __forceinline__ int f8_asc_pos(int r) {
    const int q = r & 255;
    return (r & ~255) | (q & 192) | ((q & 31) << 1) | ((q >> 5) & 1);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Sum over a block of up to 1024 threads; `red` holds >= 16 floats of LDS.
// Every thread gets the total.  The order is fixed (lane tree, then waves in
// order), so the result is deterministic.
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE, nw = (blockDim.x + WAVE - 1) / WAVE;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; i++) t += red[i];
    return t;
}

// Sum of S split partials of one element: p[s*stride + off], s ascending.
// The loads of a batch are issued together (the partials come from L2 or HBM,
// and one dependent load per split would serialise S memory latencies); the
// additions keep the order s = 0, 1, ..., S-1, so the result is the same.
__device__ __forceinline__ float sum_splits(const float *p, int S, size_t stride, size_t off) {
    float v = p[off];
    int s = 1;
    for (; s + 8 <= S; s += 8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; i++) t[i] = p[(s + i) * stride + off];
#pragma unroll
        for (int i = 0; i < 8; i++) v += t[i];
    }
    if (s + 4 <= S) {
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; i++) t[i] = p[(s + i) * stride + off];
#pragma unroll
        for (int i = 0; i < 4; i++) v += t[i];
        s += 4;
    }
    for (; s < S; s++) v += p[s * stride + off];
    return v;
}

__device__ __forceinline__ void add4(float4 &v, const float4 t) {
    v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
}

__device__ __forceinline__ float4 sum_splits4(const float *p, int S, size_t stride, size_t off) {
    float4 v = *reinterpret_cast<const float4 *>(p + off);
    int s = 1;
    for (; s + 8 <= S; s += 8) {
        float4 t[8];
#pragma unroll
        for (int i = 0; i < 8; i++) t[i] = *reinterpret_cast<const float4 *>(p + (s + i) * stride + off);
#pragma unroll
        for (int i = 0; i < 8; i++) add4(v, t[i]);
    }
    if (s + 4 <= S) {
        float4 t[4];
#pragma unroll
        for (int i = 0; i < 4; i++) t[i] = *reinterpret_cast<const float4 *>(p + (s + i) * stride + off);
#pragma unroll
        for (int i = 0; i < 4; i++) add4(v, t[i]);
        s += 4;
    }
    for (; s < S; s++) add4(v, *reinterpret_cast<const float4 *>(p + s * stride + off));
    return v;
}
