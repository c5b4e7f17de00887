// Log-sum-exp merge of segment partials on gfx950, and the empty partial written for a
// segment with no keys.
#include "rkv_internal.h"
#include "rkv_wave.h"

#include <math.h>

namespace rkv {

namespace {

// Log-sum-exp merge of partials (patch 0070 streaming_combine_kernel, applied to the
// un-normalised (M, S, VKQ) form).  One workgroup per output row: the segment weights
// e^(M_s - M*) are computed once into LDS, then 32 groups of 32 lanes (four head_dim values
// per lane) accumulate the values of interleaved segments -- many independent loads in
// flight per lane -- and fold through LDS.
constexpr int kMergeThreads = 1024;
constexpr int kMergeGroups = kMergeThreads / 32;
constexpr int kMergeTile = 2048;  // segment weights held in LDS per pass

// Segments [a, b) of a row: all of them, or the row's pair range when one is given.  A segment
// with M = -inf has weight 0 and its values are not used (they need not have been written).
struct RowRange {
    const int2 *pair_range;
    int n_head, heads_per_pair, n_hgrp;
    int64_t rows_per_seq;
    __device__ void of(int64_t row, int n_seg, int &a, int &b) const {
        a = 0;
        b = n_seg;
        if (!pair_range) return;
        const int pair = (int)(row / rows_per_seq) * n_hgrp + (int)(row % n_head) / heads_per_pair;
        const int2 r = pair_range[pair];
        a = max(0, min(r.x, n_seg));
        b = max(a, min(r.y, n_seg));
    }
};

// Up to NS * kMergePartThreads segments over few rows: workgroup (row, part) merges head_dim
// values 16*part .. 16*part+15 of one row (D / 16 parts; partial rows of 2 + D floats) with
// NS segments per thread (thread t: segments t, t + 256, ...), so every load of the merge is
// issued at once by D / 16 times more workgroups than rows and the merge costs one memory
// latency.  M and S are read by every part (8 bytes per segment).
constexpr int kMergePartDim = 16;
constexpr int kMergePartThreads = 256;
constexpr int kMergePartMaxNs = 4;  // segments per thread: up to 1024 segments

template <int D, int NS>
__global__ void __launch_bounds__(kMergePartThreads) merge_parts_kernel(const float *__restrict__ part, int n_seg,
                                                                        int64_t n_rows, float *__restrict__ o,
                                                                        float *__restrict__ lse,
                                                                        float *__restrict__ pout, RowRange rr) {
    constexpr int kW = kMergePartThreads / 64;
    constexpr int kPs = 2 + D;
    __shared__ float s_m[kW];
    __shared__ float s_acc[kW][kMergePartDim + 1];
    const int64_t row = blockIdx.x;
    const int pt = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int sa, sb;
    rr.of(row, n_seg, sa, sb);
    float2 ms[NS];
    float v[NS][kMergePartDim];
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int sg = sa + tid + u * kMergePartThreads;
        const bool has = sg < sb;
        const float *pp = part + ((int64_t)(has ? sg : 0) * n_rows + row) * kPs;
        ms[u] = make_float2(-INFINITY, 0.f);
        if (has) {
            ms[u] = *reinterpret_cast<const float2 *>(pp);
#pragma unroll
            for (int j = 0; j < kMergePartDim / 2; ++j) {
                const float2 x = *reinterpret_cast<const float2 *>(pp + 2 + kMergePartDim * pt + 2 * j);
                v[u][2 * j] = x.x;
                v[u][2 * j + 1] = x.y;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kMergePartDim; ++j) v[u][j] = 0.f;
        }
        mloc = fmaxf(mloc, ms[u].x);
    }
    float M = wave_max(mloc);
    if (lane == 0) s_m[wv] = M;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kW; ++k) M = fmaxf(M, s_m[k]);
    // this thread's weighted S and values (an empty partial, M = -inf, has weight 0 and its
    // values need not have been written), then per-wave sums, then across the waves via LDS
    float sl = 0.f, al[kMergePartDim];
#pragma unroll
    for (int j = 0; j < kMergePartDim; ++j) al[j] = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const float w = (M == -INFINITY || ms[u].x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ms[u].x - M) * kLog2e);
        sl = fmaf(ms[u].y, w, sl);
#pragma unroll
        for (int j = 0; j < kMergePartDim; ++j) al[j] = w > 0.f ? fmaf(v[u][j], w, al[j]) : al[j];
    }
    const float S = wave_sum(sl);
    float acc[kMergePartDim];
#pragma unroll
    for (int j = 0; j < kMergePartDim; ++j) acc[j] = wave_sum(al[j]);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kMergePartDim; ++j) s_acc[wv][j] = acc[j];
        s_acc[wv][kMergePartDim] = S;
    }
    __syncthreads();
    if (tid > kMergePartDim) return;
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < kW; ++k) a += s_acc[k][tid];
    // thread kMergePartDim holds S; the others one head_dim value
    const float Stot = [&] {
        float x = 0.f;
#pragma unroll
        for (int k = 0; k < kW; ++k) x += s_acc[k][kMergePartDim];
        return x;
    }();
    if (pout) {
        float *dst = pout + row * kPs;
        if (tid < kMergePartDim) dst[2 + kMergePartDim * pt + tid] = a;
        else if (pt == 0) {
            dst[0] = M;
            dst[1] = Stot;
        }
        return;
    }
    const bool ok = (M != -INFINITY) && (Stot > 0.f);
    if (tid < kMergePartDim) o[row * D + kMergePartDim * pt + tid] = ok ? a / Stot : 0.f;
    else if (lse && pt == 0) lse[row] = ok ? M + logf(Stot) : -INFINITY;
}

__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const float *__restrict__ part, int n_seg,
                                                              int64_t n_rows, float *__restrict__ o,
                                                              float *__restrict__ lse,
                                                              float *__restrict__ pout, RowRange rr) {
    __shared__ float s_wt[kMergeTile];
    __shared__ float s_red[kMergeThreads / 64];
    __shared__ float s_acc[kMergeGroups][kHeadDim];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, q = tid & 31, grp = tid >> 5;  // lane q holds head_dim q + 32m
    const int64_t step = n_rows * kPartialStride;
    int sa, sb;
    rr.of(row, n_seg, sa, sb);
    const float *base = part + (row + sa * n_rows) * kPartialStride;
    n_seg = sb - sa;

    // M* = max over segments
    float M = -INFINITY;
    for (int s = tid; s < n_seg; s += kMergeThreads) M = fmaxf(M, base[(int64_t)s * step]);
    M = wave_max(M);
    if ((tid & 63) == 0) s_red[tid >> 6] = M;
    __syncthreads();
    M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMergeThreads / 64; ++j) M = fmaxf(M, s_red[j]);
    __syncthreads();

    float S = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int t0 = 0; t0 < n_seg; t0 += kMergeTile) {
            const int nt = min(kMergeTile, n_seg - t0);
            for (int j = tid; j < nt; j += kMergeThreads) {
                const float *pp = base + (int64_t)(t0 + j) * step;
                const float Ms = pp[0];
                const float w = (Ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((Ms - M) * kLog2e);
                s_wt[j] = w;
                S = fmaf(pp[1], w, S);  // each segment's S counted once, by the lane that weighed it
            }
            __syncthreads();
#pragma unroll 4
            for (int j = grp; j < nt; j += kMergeGroups) {
                const float *v = base + (int64_t)(t0 + j) * step + 2 + q;
                const float wj = s_wt[j];
                if (wj > 0.f) {
#pragma unroll
                    for (int m = 0; m < 4; ++m) acc[m] = fmaf(v[32 * m], wj, acc[m]);
                }
            }
            __syncthreads();
        }
    }
    // fold S over the block and acc over the groups
    S = wave_sum(S);
    if ((tid & 63) == 0) s_red[tid >> 6] = S;
#pragma unroll
    for (int m = 0; m < 4; ++m) s_acc[grp][q + 32 * m] = acc[m];
    __syncthreads();
    if (tid >= kHeadDim) return;
    const int d = tid;
    S = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeThreads / 64; ++j) S += s_red[j];
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeGroups; ++j) a += s_acc[j][d];
    if (pout) {
        float *dst = pout + row * kPartialStride;
        if (d == 0) {
            dst[0] = M;
            dst[1] = S;
        }
        dst[2 + d] = a;
        return;
    }
    const bool ok = (M != -INFINITY) && (S > 0.f);
    o[row * kHeadDim + d] = ok ? a / S : 0.f;
    if (lse && d == 0) lse[row] = ok ? M + logf(S) : -INFINITY;
}

// The same merge for many rows over few segments (prefill: thousands of rows, a handful of
// segments): one wave per output row, lane l holding head_dim l and l+64; segment weights
// are computed by the lane of that segment and read back with readlane.
constexpr int kMergeRowsPerBlock = 4;

__global__ void __launch_bounds__(64 * kMergeRowsPerBlock) merge_rows_kernel(const float *__restrict__ part, int n_seg,
                                                                           int64_t n_rows, float *__restrict__ o,
                                                                           float *__restrict__ lse,
                                                                           float *__restrict__ pout, RowRange rr) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kMergeRowsPerBlock + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int64_t step = n_rows * kPartialStride;
    int sa, sb;
    rr.of(row, n_seg, sa, sb);
    const float *base = part + (row + sa * n_rows) * kPartialStride;
    n_seg = sb - sa;
    float M = -INFINITY;
    for (int s = lane; s < n_seg; s += 64) M = fmaxf(M, base[(int64_t)s * step]);
    M = wave_max(M);
    float S = 0.f, a0 = 0.f, a1 = 0.f;
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < n_seg; s0 += 64) {
            const int s = s0 + lane;
            float w = 0.f;
            if (s < n_seg) {
                const float Ms = base[(int64_t)s * step];
                w = (Ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((Ms - M) * kLog2e);
                S = fmaf(base[(int64_t)s * step + 1], w, S);
            }
            const int nt = min(64, n_seg - s0);
            for (int j = 0; j < nt; ++j) {
                const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
                if (wj > 0.f) {
                    const float *v = base + (int64_t)(s0 + j) * step + 2 + lane;
                    a0 = fmaf(v[0], wj, a0);
                    a1 = fmaf(v[64], wj, a1);
                }
            }
        }
    }
    S = wave_sum(S);
    if (pout) {
        float *q = pout + row * kPartialStride;
        if (lane == 0) {
            q[0] = M;
            q[1] = S;
        }
        q[2 + lane] = a0;
        q[66 + lane] = a1;
        return;
    }
    const bool ok = (M != -INFINITY) && (S > 0.f);
    o[row * kHeadDim + lane] = ok ? a0 / S : 0.f;
    o[row * kHeadDim + 64 + lane] = ok ? a1 / S : 0.f;
    if (lse && lane == 0) lse[row] = ok ? M + logf(S) : -INFINITY;
}

// one row per workgroup: (M, S) = (-inf, 0) and dv zeros, for rows of 2 + dv floats
__global__ void __launch_bounds__(128) empty_partials_kernel(float *__restrict__ part, int dv) {
    float *q = part + (int64_t)blockIdx.x * (2 + dv);
    for (int j = threadIdx.x; j < dv; j += blockDim.x) q[2 + j] = 0.f;
    if (threadIdx.x == 0) {
        q[0] = -INFINITY;
        q[1] = 0.f;
    }
}

}  // namespace

hipError_t launch_merge(const float *partials, int n_seg, int64_t n_rows, float *o, float *lse,
                        float *partial_out, hipStream_t s, const MergeRange *range) {
    if (n_rows <= 0) return hipSuccess;
    RowRange rr{};
    if (range) {
        if (range->n_head <= 0 || range->heads_per_pair <= 0 || range->rows_per_seq <= 0) return hipErrorInvalidValue;
        rr = RowRange{range->pair_range, range->n_head, range->heads_per_pair, range->n_hgrp, range->rows_per_seq};
    }
    if (n_rows >= 1024 || n_seg <= 16) {
        // enough rows to fill the chip one wave each (or too few segments to share a row)
        hipLaunchKernelGGL(merge_rows_kernel, dim3((unsigned)((n_rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock)),
                           dim3(64 * kMergeRowsPerBlock), 0, s, partials, n_seg, n_rows, o, lse, partial_out, rr);
    } else if (n_seg <= kMergePartThreads) {
        hipLaunchKernelGGL((merge_parts_kernel<kHeadDim, 1>), dim3((unsigned)n_rows, kHeadDim / kMergePartDim),
                           dim3(kMergePartThreads), 0, s, partials, n_seg, n_rows, o, lse, partial_out, rr);
    } else {
        hipLaunchKernelGGL(merge_kernel, dim3((unsigned)n_rows), dim3(kMergeThreads), 0, s, partials, n_seg, n_rows,
                           o, lse, partial_out, rr);
    }
    return hipGetLastError();
}

template <int D>
void launch_parts_d(const float *partials, int n_seg, int64_t n_rows, float *o, float *lse, float *pout,
                    hipStream_t s) {
    const dim3 grid((unsigned)n_rows, (unsigned)(D / kMergePartDim));
    const RowRange rr{};
    if (n_seg <= kMergePartThreads)
        hipLaunchKernelGGL((merge_parts_kernel<D, 1>), grid, dim3(kMergePartThreads), 0, s, partials, n_seg, n_rows, o,
                           lse, pout, rr);
    else
        hipLaunchKernelGGL((merge_parts_kernel<D, kMergePartMaxNs>), grid, dim3(kMergePartThreads), 0, s, partials,
                           n_seg, n_rows, o, lse, pout, rr);
}

hipError_t launch_merge_parts(const float *partials, int n_seg, int64_t n_rows, int dv, float *o, float *lse,
                              hipStream_t s, float *partial_out) {
    if (n_rows <= 0) return hipSuccess;
    if (n_seg > kMergePartMaxNs * kMergePartThreads || n_rows > ((int64_t)1 << 31) - 1) return hipErrorInvalidValue;
    if (dv == 64)
        launch_parts_d<64>(partials, n_seg, n_rows, o, lse, partial_out, s);
    else if (dv == 128)
        launch_parts_d<128>(partials, n_seg, n_rows, o, lse, partial_out, s);
    else if (dv == 256)
        launch_parts_d<256>(partials, n_seg, n_rows, o, lse, partial_out, s);
    else if (dv == 512)
        launch_parts_d<512>(partials, n_seg, n_rows, o, lse, partial_out, s);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

hipError_t launch_empty_partials(float *partials, int64_t n_rows, hipStream_t s, int dv) {
    if (n_rows <= 0) return hipSuccess;
    if (dv <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_partials_kernel, dim3((unsigned)n_rows), dim3(128), 0, s, partials, dv);
    return hipGetLastError();
}

}  // namespace rkv
