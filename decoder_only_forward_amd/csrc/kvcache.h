// K/V cache element formats (rml "The decoder", section "Attend": the cache
// element type is a choice, and attention widens each row to fp32 as it reads
// it).  The values are dec_config.kv_dtype's.
//
//   KV_F32   fp32, 4 bytes an element.
//   KV_BF16  bf16 rounded to nearest even, 2 bytes.
//   KV_F24   fp32 rounded to nearest even at 15 stored mantissa bits (16
//            significant bits: what a bf16 (hi, lo) pair of an fp32 value
//            carries into the MFMAs), 3 bytes.  A row of HD elements is HD
//            16-bit words (the upper half of each rounded fp32 word) followed
//            by HD bytes (the third bytes); the low byte is zero.  Readers
//            rebuild the fp32 word exactly: (hi << 16) | (lo << 8).  The third
//            bytes go by blocks of 8 elements: block b (elements 8b .. 8b+7,
//            in order) at byte 16 (b % L) + 8 (b / L) of that part, L = HD/16,
//            so blocks b and b + L fill one 16-byte word (the two 8-element
//            words a lane of the decode kernel takes); for HD = 16 the order
//            is plain.
//
// Rows start on 16-byte boundaries for every head_dim that is a multiple of
// 16 (row bytes 4 HD, 2 HD or 3 HD).
#pragma once
#include "common.h"

enum { KV_F32 = 0, KV_BF16 = 1, KV_F24 = 2 };

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int KT>
__host__ __device__ constexpr int kv_row_bytes(int hd) {
    return KT == KV_F32 ? 4 * hd : (KT == KV_BF16 ? 2 * hd : 3 * hd);
}

// Byte offset within a 24-bit row of element e's third byte.
__host__ __device__ constexpr int f24_lo_off(int hd, int e) {
    return 2 * hd + 16 * ((e / 8) % (hd / 16)) + 8 * ((e / 8) / (hd / 16)) + e % 8;
}

// The rounded fp32 word of x (finite x): nearest even at bit 8, low byte 0.
__device__ __forceinline__ uint32_t f24_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7Fu + ((u >> 8) & 1u)) & 0xFFFFFF00u;
}

// Element e of a 24-bit row of hd elements.
__device__ __forceinline__ void f24_store(char *row, int hd, int e, float x) {
    const uint32_t b = f24_bits(x);
    *reinterpret_cast<u16 *>(row + 2 * e) = (u16)(b >> 16);
    *reinterpret_cast<uint8_t *>(row + f24_lo_off(hd, e)) = (uint8_t)(b >> 8);
}

// Elements e .. e+3 (e a multiple of 4: their third bytes are consecutive).
__device__ __forceinline__ void f24_store4(char *row, int hd, int e, float4 v) {
    const uint32_t a = f24_bits(v.x), b = f24_bits(v.y), c = f24_bits(v.z), d = f24_bits(v.w);
    *reinterpret_cast<uint2 *>(row + 2 * e) = make_uint2((a >> 16) | (b & 0xFFFF0000u), (c >> 16) | (d & 0xFFFF0000u));
    *reinterpret_cast<uint32_t *>(row + f24_lo_off(hd, e)) =
        ((a >> 8) & 0xFFu) | (b & 0xFF00u) | ((c << 8) & 0xFF0000u) | ((d << 16) & 0xFF000000u);
}

// fp32 value of element i (0..7) of an 8-element piece: hi holds the upper
// halves (element 2j in the low half of word j), lo the third bytes (element
// e in byte e % 4 of word e / 4).  v_perm_b32 assembles the word: selector
// byte 0x0C gives zero, 0-3 pick bytes of lo's word, 4-7 bytes of hi's word.
template <int I>
__device__ __forceinline__ float f24_elem(const u32x4 &hi, const u32x2 &lo) {
    constexpr uint32_t sel = (I & 1) ? (0x07060000u | ((uint32_t)(I & 3) << 8) | 0x0Cu)
                                     : (0x05040000u | ((uint32_t)(I & 3) << 8) | 0x0Cu);
    return __uint_as_float(__builtin_amdgcn_perm(hi[I / 2], lo[I / 4], sel));
}

__device__ __forceinline__ void f24_unpack8(const u32x4 &hi, const u32x2 &lo, float (&f)[8]) {
    f[0] = f24_elem<0>(hi, lo);
    f[1] = f24_elem<1>(hi, lo);
    f[2] = f24_elem<2>(hi, lo);
    f[3] = f24_elem<3>(hi, lo);
    f[4] = f24_elem<4>(hi, lo);
    f[5] = f24_elem<5>(hi, lo);
    f[6] = f24_elem<6>(hi, lo);
    f[7] = f24_elem<7>(hi, lo);
}

// Four fp32 values of a row in any of the formats, from element e (a multiple of 4).
template <int KT, int HD>
__device__ __forceinline__ float4 kv_load4(const char *row, int e) {
    if constexpr (KT == KV_BF16) {
        const uint2 r = *reinterpret_cast<const uint2 *>(row + (size_t)e * 2);
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
    } else if constexpr (KT == KV_F24) {
        const uint2 h = *reinterpret_cast<const uint2 *>(row + (size_t)e * 2);
        const uint32_t l = *reinterpret_cast<const uint32_t *>(row + f24_lo_off(HD, e));
        return make_float4(__uint_as_float((h.x << 16) | ((l & 0xFFu) << 8)),
                           __uint_as_float((h.x & 0xFFFF0000u) | (l & 0xFF00u)),
                           __uint_as_float((h.y << 16) | ((l >> 8) & 0xFF00u)),
                           __uint_as_float((h.y & 0xFFFF0000u) | ((l >> 16) & 0xFF00u)));
    } else {
        return *reinterpret_cast<const float4 *>(row + (size_t)e * 4);
    }
}

// Store four fp32 values at element e (a multiple of 4) of a row.
template <int KT, int HD>
__device__ __forceinline__ void kv_store4(char *row, int e, float4 v) {
    if constexpr (KT == KV_BF16) {
        *reinterpret_cast<uint2 *>(row + (size_t)e * 2) =
            make_uint2(f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16),
                       f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16));
    } else if constexpr (KT == KV_F24) {
        f24_store4(row, HD, e, v);
    } else {
        *reinterpret_cast<float4 *>(row + (size_t)e * 4) = v;
    }
}
