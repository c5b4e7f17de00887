// Auxiliary gfx950 kernels of librkv: the word-granularity host reader kept as a measured
// contrast to the bulk DMA lift, and the exact row dequantiser behind rkv_dequant_rows.
#include "rkv_internal.h"
#include "rkv_quant.h"

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

__global__ void __launch_bounds__(128) dequant_kernel(const uint8_t *__restrict__ src, int type,
                                                      int64_t row_stride,
                                                      float *__restrict__ dst) {
    const int64_t row = blockIdx.x;
    const int e = threadIdx.x;
    dst[row * kHeadDim + e] = row_value(src + row * row_stride, type, e);
}

}  // namespace

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

hipError_t launch_dequant_rows(const void *src, int type, int64_t n_rows, int64_t row_stride,
                               float *dst, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)n_rows), dim3(kHeadDim), 0, s,
                       static_cast<const uint8_t *>(src), type, row_stride, dst);
    return hipGetLastError();
}

}  // namespace rkv
