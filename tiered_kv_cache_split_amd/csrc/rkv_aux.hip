// Auxiliary gfx950 kernels of librkv: the word-granularity host reader kept as a measured
// contrast to the bulk DMA lift, and the exact row dequantiser behind rkv_dequant_rows.
#include "rkv_internal.h"
#include "rkv_unpack.h"

#include <algorithm>

namespace rkv {

namespace {

// Contrast path: the GPU reads pinned host memory through its device mapping four bytes
// per lane (the word-granularity read patch 0102's commit message measures against the
// bulk DMA).
__global__ void __launch_bounds__(256) uva_read_kernel(const uint32_t *__restrict__ src,
                                                       uint32_t *__restrict__ dst,
                                                       int64_t n_words) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride)
        dst[i] = src[i];
}
__global__ void uva_tail_kernel(const uint8_t *src, uint8_t *dst, int64_t n) {
    const int64_t i = threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// One value of a q8_0 / q4_0 / binary16 row, rebuilt through the unpack routine of one kernel
// family (enum rkv_dequant_form) so that a bitwise comparison covers the routine that family
// runs: the codes or nibbles in the family's binary16 integer form, their offset removed in
// float32 (exact: small integers), times the block scale in float32 (exact); for the prefill
// form the exact two-part binary16 sum.
__device__ __forceinline__ uint32_t word_at(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
__device__ float dequant_value(const uint8_t *row, int type, int form, int e) {
    if (type == T_F16) return f16_bits_to_f32((uint32_t)row[2 * e] | ((uint32_t)row[2 * e + 1] << 8));
    const int i = e & 31;
    if (type == T_Q8_0) {
        const uint8_t *blk = row + kQ8Block * (e >> 5);
        const uint32_t dbits = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
        const uint8_t *codes = blk + 2;
        if (form == 3) return f16_bits_to_f32(dbits) * q8_code_f32(codes[i]);
        const uint2 b = q8_biased(word_at(codes + 4 * (i >> 2)));
        const uint32_t pair = (i & 2) ? b.y : b.x;
        if (form == 1) {
            uint32_t hi, lo;
            q8_hi_lo(q8_unbias(pair), u2h(dbits | (dbits << 16)), hi, lo);
            const int sh = 16 * (i & 1);
            return f16_bits_to_f32(hi >> sh) + f16_bits_to_f32(lo >> sh);
        }
        return (f16_bits_to_f32(pair >> (16 * (i & 1))) - kQ8Bias) * f16_bits_to_f32(dbits);
    }
    // q4_0
    const uint8_t *blk = row + kQ4Block * (e >> 5);
    const uint32_t dbits = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
    const uint8_t *data = blk + 2;
    const float d = f16_bits_to_f32(dbits);
    const int j = i & 15;  // data byte of element i
    if (form == 3) return d * q4_centered_f32(data, i);
    if (form == 1) {
        const uint32_t w[4] = {word_at(data), word_at(data + 4), word_at(data + 8), word_at(data + 12)};
        uint32_t out[16];
        q4_block_centered(w, out);
        return f16_bits_to_f32(out[i >> 1] >> (16 * (i & 1))) * d;
    }
    const uint32_t word = word_at(data + 4 * (j >> 2));
    if (form == 2) {
        // the vector kernels isolate the nibble fields of a word, then pair byte t of two words
        const uint32_t nib = i < 16 ? (word & 0x0F0F0F0Fu) : ((word >> 4) & 0x0F0F0F0Fu);
        return (f16_bits_to_f32(q4_pair_biased(nib, 0u, j & 3)) - kQ4BiasLo) * d;
    }
    uint32_t lo, hi;
    q4_nibbles_biased(word, (j & 2) ? 0x0C030C02u : 0x0C010C00u, 0x64006400u, lo, hi);
    const int sh = 16 * (j & 1);
    if (i < 16) return (f16_bits_to_f32(lo >> sh) - kQ4BiasLo) * d;
    return (f16_bits_to_f32(hi >> sh) - kQ4BiasHi) * 0.0625f * d;
}

__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t *__restrict__ src, int type, int form, int n_values,
                                                      int64_t row_stride, float *__restrict__ dst) {
    const int64_t row = blockIdx.x;
    for (int e = threadIdx.x; e < n_values; e += blockDim.x)
        dst[row * n_values + e] = dequant_value(src + row * row_stride, type, form, e);
}

}  // namespace

// Extent of a padded row list (llama.cpp PR #29510 flash_attn_ext_rows, ggml.h API comment:
// kv_rows with -1 padding), in kRowExtentParts pieces
// per sequence: workgroup (b, part) writes 1 + the last index of its slice holding a pool row
// (0 if none); the extent of sequence b is the maximum over its parts.  Every load of a thread
// is issued before any is used, so the scan costs about one memory latency.
__global__ void __launch_bounds__(256) row_extent_kernel(const int32_t *__restrict__ rows, int64_t rows_s, int64_t n_kv,
                                                         int32_t *__restrict__ extent) {
    __shared__ int s_red[4];
    const int b = blockIdx.x / kRowExtentParts, part = blockIdx.x % kRowExtentParts;
    const int32_t *r = rows + (int64_t)b * rows_s;
    const int64_t len = (n_kv + kRowExtentParts - 1) / kRowExtentParts;
    const int64_t j0 = part * len, j1 = min(n_kv, j0 + len);
    int last = -1;
    for (int64_t base = j0; base < j1; base += 256 * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t j = base + threadIdx.x + 256 * u;
            v[u] = j < j1 ? r[j] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (v[u] >= 0) last = (int)(base + threadIdx.x + 256 * u);
    }
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = last;
    __syncthreads();
    if (threadIdx.x == 0) extent[blockIdx.x] = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3])) + 1;
}

hipError_t launch_row_extent(const int32_t *rows, int64_t rows_s, int64_t n_kv, int n_seq, int32_t *extent, hipStream_t s) {
    if (n_seq <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_extent_kernel, dim3((unsigned)(n_seq * kRowExtentParts)), dim3(256), 0, s, rows, rows_s, n_kv,
                       extent);
    return hipGetLastError();
}

hipError_t launch_uva_read(const void *host_src, void *dst, int64_t nbytes, hipStream_t s) {
    void *dev_view = nullptr;
    hipError_t e = hipHostGetDevicePointer(&dev_view, const_cast<void *>(host_src), 0);
    if (e != hipSuccess) return e;
    const int64_t n_words = nbytes / 4;
    if (n_words > 0) {
        const int64_t blocks = std::min<int64_t>((n_words + 255) / 256, 4096);
        hipLaunchKernelGGL(uva_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const uint32_t *>(dev_view), static_cast<uint32_t *>(dst), n_words);
    }
    const int64_t rem = nbytes - 4 * n_words;
    if (rem > 0)
        hipLaunchKernelGGL(uva_tail_kernel, dim3(1), dim3(4), 0, s,
                           static_cast<const uint8_t *>(dev_view) + 4 * n_words,
                           static_cast<uint8_t *>(dst) + 4 * n_words, rem);
    return hipGetLastError();
}

// Bulk copy of pinned host bytes by a kernel on the copy stream: 8-byte buffer reads of the
// bytes' device view, two in flight per thread, grid-stride over the span.  Unlike a DMA-engine
// copy it needs no hand-off between the copy engine and the compute queue, which is most of the
// cost of small lifts.  It is held to 16 VGPRs so that its waves fit beside two waves of a
// segment kernel that uses up to 248 of a SIMD's 512 registers each, and to 64 workgroups:
// 256 KB of reads in flight keep the link busy, while every CU that hosts a copy workgroup has
// its memory pipeline full of slow host reads, which stalls the compute sharing it (measured:
// 64 workgroups lift at the link's rate and slow an overlapping prefill kernel 8%, 256 by 50%).
__global__ void __launch_bounds__(256) __attribute__((amdgpu_num_vgpr(16)))
lift_copy_kernel(const uint8_t *src_p, uint8_t *dst_p, uint32_t n8) {
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc((void *)src_p, (short)0, (int)(8 * n8), 0x00020000);
    const __amdgpu_buffer_rsrc_t dst = __builtin_amdgcn_make_buffer_rsrc((void *)dst_p, (short)0, (int)(8 * n8), 0x00020000);
    const uint32_t stride = gridDim.x * blockDim.x;
    uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + stride < n8; i += 2 * stride) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b64(src, (int)(8 * i), 0, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b64(src, (int)(8 * (i + stride)), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(a, dst, (int)(8 * i), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(b, dst, (int)(8 * (i + stride)), 0, 0);
    }
    if (i < n8)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_amdgcn_raw_buffer_load_b64(src, (int)(8 * i), 0, 0), dst,
                                              (int)(8 * i), 0, 0);
}

hipError_t launch_lift_copy(const void *host_src, void *dst, int64_t nbytes, hipStream_t s) {
    if (nbytes <= 0) return hipSuccess;
    void *dev_view = nullptr;
    hipError_t e = hipHostGetDevicePointer(&dev_view, const_cast<void *>(host_src), 0);
    if (e != hipSuccess) return e;
    if (((uintptr_t)dev_view | (uintptr_t)dst) % 8 != 0) return hipErrorInvalidValue;
    // pieces of at most 1 GiB keep the byte offsets within 31 bits
    constexpr int64_t kPiece = (int64_t)1 << 30;
    const int64_t n8_all = nbytes / 8;
    for (int64_t p0 = 0; p0 < n8_all; p0 += kPiece / 8) {
        const int64_t n8 = std::min<int64_t>(n8_all - p0, kPiece / 8);
        const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n8 + 511) / 512, 64));
        hipLaunchKernelGGL(lift_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const uint8_t *>(dev_view) + 8 * p0, static_cast<uint8_t *>(dst) + 8 * p0,
                           (uint32_t)n8);
    }
    const int64_t rem = nbytes - 8 * n8_all;
    if (rem > 0)
        hipLaunchKernelGGL(uva_tail_kernel, dim3(1), dim3(8), 0, s,
                           static_cast<const uint8_t *>(dev_view) + 8 * n8_all, static_cast<uint8_t *>(dst) + 8 * n8_all,
                           rem);
    return hipGetLastError();
}

hipError_t launch_dequant_rows(const void *src, int type, int form, int64_t n_rows, int n_values, int64_t row_stride,
                               float *dst, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)n_rows), dim3(256), 0, s, static_cast<const uint8_t *>(src), type,
                       form, n_values, row_stride, dst);
    return hipGetLastError();
}

}  // namespace rkv
