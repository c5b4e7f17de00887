// Exact q8_0 / q4_0 / binary16 readers shared by every gfx950 kernel of librkv.
//
// Formats: a q8_0 block is 34 bytes, a binary16 scale d followed by 32 int8 codes q,
// element value d*q; a q4_0 block is 18 bytes, a binary16 scale d followed by 16 bytes
// whose byte j carries element j in its low nibble and element j+16 in its high nibble,
// element value d*(n-8).  (Block size 32 as in opencoti-llamafile patch 0070-rolling-kv,
// KV-cache residency hunk; patch 0102 lifts exactly these raw blocks.)
//
// d has 11 significant bits and q (or n-8) at most 8, so d*q is exact in float32; the
// conversion of d keeps binary16 subnormals (v_cvt_f32_f16 honours f16 denormals).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

constexpr int kQ8Block = 34;
constexpr int kQ4Block = 18;
constexpr int kQ8Row = 4 * kQ8Block;  // 128 values
constexpr int kQ4Row = 4 * kQ4Block;

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

// Little-endian 16-bit load from a byte pointer that is at least 2-byte aligned.
__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) {
    return *reinterpret_cast<const uint16_t *>(p);
}

// Element e (0..31) of a q8_0 block.
__device__ __forceinline__ float q8_0_value(const uint8_t *blk, int e) {
    const float d = h2f(ld_u16(blk));
    const int8_t q = static_cast<int8_t>(blk[2 + e]);
    return d * static_cast<float>(q);
}

// Element e (0..31) of a q4_0 block.
__device__ __forceinline__ float q4_0_value(const uint8_t *blk, int e) {
    const float d = h2f(ld_u16(blk));
    const uint32_t byte = blk[2 + (e & 15)];
    const int n = (e < 16) ? (int)(byte & 15u) : (int)(byte >> 4);
    return d * static_cast<float>(n - 8);
}

// Value e (0..127) of a row of 128 values stored as type t.
__device__ __forceinline__ float row_value(const uint8_t *row, int t, int e) {
    if (t == 1) return h2f(ld_u16(row + 2 * e));
    if (t == 8) return q8_0_value(row + (e >> 5) * kQ8Block, e & 31);
    return q4_0_value(row + (e >> 5) * kQ4Block, e & 31);
}

}  // namespace rkv
