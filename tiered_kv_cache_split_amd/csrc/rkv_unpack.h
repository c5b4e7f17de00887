// In-register unpacking of q8_0 / q4_0 blocks into exact matrix-core and vector operands,
// shared by every gfx950 kernel of librkv and by rkv_dequant_rows (which rebuilds each block
// value from these same routines, so a bitwise test of it covers what the kernels execute).
//
// Formats (block size 32, as the KV-cache residency hunk of opencoti-llamafile patch
// 0070-rolling-kv stores the cache; patch 0102 lifts exactly these raw blocks): a q8_0 block is
// 34 bytes, a binary16 scale d then 32 int8 codes q, element value d*q; a q4_0 block is 18
// bytes, a binary16 scale d then 16 bytes whose byte j carries element j in its low nibble and
// element j+16 in its high nibble, element value d*(n-8).
//
// Every form below is exact: codes and nibbles become binary16 integers (1024 + small integer,
// or the small integer itself), and the scale is applied either in fp32 (d has 11 significant
// bits, a code at most 8, so d*q is exact in float32) or split into two binary16 parts whose
// sum is d*q exactly (hi = rn(d*q), lo = d*q - hi: lo has at most 7 significant bits and lies
// on d's own grid, so it is representable; this holds while |d*q| <= 65504).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

constexpr int kQ8Block = 34;  // bytes of a q8_0 block
constexpr int kQ4Block = 18;  // bytes of a q4_0 block
constexpr int kQ8Row = 4 * kQ8Block;  // a row of 128 values
constexpr int kQ4Row = 4 * kQ4Block;

typedef _Float16 uhalf2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uhalf2_t u2h(uint32_t x) { return __builtin_bit_cast(uhalf2_t, x); }
__device__ __forceinline__ uint32_t h2u(uhalf2_t x) { return __builtin_bit_cast(uint32_t, x); }

// binary16 bits -> float32 (exact; binary16 subnormals are kept by v_cvt_f32_f16).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xFFFFu));
}

__device__ __forceinline__ float h2f(uint32_t bits16) { return f16_bits_to_f32(bits16); }

// Little-endian 16-bit load from a byte pointer that is at least 2-byte aligned.
__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

// ---- q8_0 codes

// Offset applied to every q8_0 code by q8_biased: the binary16 value of a code q is 1152 + q.
constexpr float kQ8Bias = 1152.0f;

// Four q8_0 codes (one little-endian word, code i in byte i) -> two binary16 pairs holding
// 1024 + (q + 128) = 1152 + q, exact integers: .x = codes 0, 1, .y = codes 2, 3.  The code byte
// q + 128 (sign bit flipped) becomes the low byte of a binary16 with the exponent byte 0x64.
__device__ __forceinline__ uint2 q8_biased(uint32_t codes4) {
    const uint32_t u = codes4 ^ 0x80808080u;
    return make_uint2(__builtin_amdgcn_perm(0x64646464u, u, 0x05010400u),
                      __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u));
}

// Two biased codes -> the codes themselves as binary16 (exact: small integers).
__device__ __forceinline__ uhalf2_t q8_unbias(uint32_t biased2) {
    const uhalf2_t b = {(_Float16)-kQ8Bias, (_Float16)-kQ8Bias};
    return u2h(biased2) + b;
}

// Two codes (binary16 integers) times the block scale d (binary16 pair), as an exact
// two-part binary16 sum: hi = rn(d*q), lo = d*q - hi.
__device__ __forceinline__ void q8_hi_lo(uhalf2_t q, uhalf2_t dd, uint32_t &hi, uint32_t &lo) {
    const uhalf2_t h = q * dd;
    hi = h2u(h);
    lo = h2u(__builtin_elementwise_fma(q, dd, -h));
}

// Code byte b (0..255 as stored) -> its signed value as float32.
__device__ __forceinline__ float q8_code_f32(uint32_t b) { return (float)(int8_t)(b & 0xFFu); }

// ---- q4_0 nibbles

// Offsets of the in-place forms of q4_nibbles_biased: a low nibble n becomes 1024 + n = 1032 +
// (n - 8); a high nibble n, left in place (bits 4..7), becomes 1024 + 16 n = 1152 + 16 (n - 8).
constexpr float kQ4BiasLo = 1032.0f;
constexpr float kQ4BiasHi = 1152.0f;

// Bytes b0, b1 of a word (selected by sel: 0x0C010C00 takes bytes 0 and 1, 0x0C030C02 bytes 2
// and 3) -> binary16 pairs (1024 + n) for their low nibbles and (1024 + 16 n) for their high
// nibbles, both exact.  `magic` is 0x64006400 (kept in a register by the caller so the
// mask-and-insert is one instruction).
__device__ __forceinline__ void q4_nibbles_biased(uint32_t word, uint32_t sel, uint32_t magic, uint32_t &lo,
                                                  uint32_t &hi) {
    const uint32_t y = __builtin_amdgcn_perm(word, word, sel);  // b0, 0, b1, 0
    lo = (y & 0x000F000Fu) | magic;
    hi = (y & 0x00F000F0u) | magic;
}

// Byte pairs of two words (one byte from each: byte t of `a` and of `b`) -> binary16 pairs
// 1024 + n of their low nibbles (lo) and of their high nibbles (hi).  The nibble fields are
// isolated first (masks of the caller's choice), then byte t of both is moved next to 0x64.
__device__ __forceinline__ uint32_t q4_pair_biased(uint32_t nib_a, uint32_t nib_b, int t) {
    const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + t) << 16) | (uint32_t)t;
    return __builtin_amdgcn_perm(nib_b, nib_a, sel) | 0x64006400u;
}

// The 16 data bytes of a q4_0 block (4 words) -> its 32 values n - 8 as exact binary16 pairs in
// element order: out[i] holds elements 2i, 2i+1 (elements 0..15 from the low nibbles of bytes
// 0..15, elements 16..31 from the high nibbles).
__device__ __forceinline__ void q4_block_centered(const uint32_t (&w)[4], uint32_t (&out)[16]) {
    const uhalf2_t bias = {(_Float16)-kQ4BiasLo, (_Float16)-kQ4BiasLo};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
        out[2 * i] = h2u(u2h(__builtin_amdgcn_perm(0x64646464u, lo, 0x05010400u)) + bias);
        out[2 * i + 1] = h2u(u2h(__builtin_amdgcn_perm(0x64646464u, lo, 0x05030402u)) + bias);
        out[8 + 2 * i] = h2u(u2h(__builtin_amdgcn_perm(0x64646464u, hi, 0x05010400u)) + bias);
        out[8 + 2 * i + 1] = h2u(u2h(__builtin_amdgcn_perm(0x64646464u, hi, 0x05030402u)) + bias);
    }
}

// Element e (0..31) of a q4_0 block given its data bytes: n - 8 as float32.
__device__ __forceinline__ float q4_centered_f32(const uint8_t *data, int e) {
    const uint32_t byte = data[e & 15];
    return (float)((int)(e < 16 ? (byte & 15u) : (byte >> 4)) - 8);
}

}  // namespace rkv
