// Wave64 reductions shared by the gfx950 kernels of librkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

inline constexpr float kLog2e = 1.4426950408889634f;
inline constexpr float kLn2 = 0.6931471805599453f;

// ---- wave64 reductions.  Floats are maxed as order-preserving integer keys so the max is a
// plain integer op on DPP operands; rows of 16 lanes are reduced with DPP, then row pairs and
// wave halves with the gfx950 permlane swaps.
__device__ __forceinline__ int f2key(float x) {
    const int b = __builtin_bit_cast(int, x);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key2f(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF)); }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false); }
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
inline constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;
inline constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i inside each half row

// Max and min of scores, which are never NaN (finite or -inf): plain v_max/v_min, without the
// quieting of NaN operands that fmaxf / fminf add in IEEE mode.
__device__ __forceinline__ float max2_nn(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float max3_nn(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float min3_nn(float a, float b, float c) {
    float r;
    asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Value of lane k summed over the four 16-lane rows, in every row.
__device__ __forceinline__ float fold_rows(float x) {
    const int xi = __builtin_bit_cast(int, x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
    x = __builtin_bit_cast(float, (int)r16[0]) + __builtin_bit_cast(float, (int)r16[1]);
    const int yi = __builtin_bit_cast(int, x);
    const auto r32 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
    return __builtin_bit_cast(float, (int)r32[0]) + __builtin_bit_cast(float, (int)r32[1]);
}

// Max of lane k over the four 16-lane rows, in every row (x never NaN).
__device__ __forceinline__ float fold_rows_max(float x) {
    const int xi = __builtin_bit_cast(int, x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
    x = max2_nn(__builtin_bit_cast(float, (int)r16[0]), __builtin_bit_cast(float, (int)r16[1]));
    const int yi = __builtin_bit_cast(int, x);
    const auto r32 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
    return max2_nn(__builtin_bit_cast(float, (int)r32[0]), __builtin_bit_cast(float, (int)r32[1]));
}

// Soft-capped score in the exp2 domain, l2 * tanh(cs * qk), with tanh(y) = 1 - 2 / (e^{2y} + 1):
// one exp and one reciprocal, exact at both saturations (e^{2y} = inf gives 1, 0 gives -1).
__device__ __forceinline__ float softcap_log2(float qk, float cs, float l2) {
    const float e = __builtin_amdgcn_exp2f((2.0f * kLog2e) * cs * qk);
    return l2 * fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
}

// This wave's LDS writes complete before its later LDS reads (other waves are not ordered).
__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float x) {
    int k = f2key(x);
    k = max(k, dpp_i<kQuadSwap1>(k));
    k = max(k, dpp_i<kQuadSwap2>(k));
    k = max(k, dpp_i<kRowRor4>(k));
    k = max(k, dpp_i<kRowRor8>(k));
    const auto r16 = __builtin_amdgcn_permlane16_swap(k, k, false, false);
    k = max((int)r16[0], (int)r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(k, k, false, false);
    k = max((int)r32[0], (int)r32[1]);
    return key2f(k);
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<kQuadSwap1>(x);
    x += dpp_f<kQuadSwap2>(x);
    x += dpp_f<kRowRor4>(x);
    x += dpp_f<kRowRor8>(x);
    return fold_rows(x);
}

}  // namespace rkv
