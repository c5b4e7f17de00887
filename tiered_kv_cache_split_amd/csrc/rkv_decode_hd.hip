// Decode segment kernel for head dims other than 128 (64 and 256, dv = dk), and the log-sum-exp
// merge for those value widths.  The streaming op of opencoti-llamafile patch 0070-rolling-kv
// serves several head dims through the same split-and-combine (fattn.cu, the op's supported
// shapes); the partial of a segment is the same (M, S, VKQ) triple as for head dim 128, stored
// with row stride 2 + D.
//
// Workgroup = 4 waves for one (split, KV head, sequence); wave w takes every 4th 64-key chunk
// of the split.  Q.K: a lane owns one key of the chunk and forms the scores of the R query rows
// that read this KV head (Q in LDS, K dequantised value by value from its own row).  Softmax:
// per row, a running max over chunks (wave reductions), weights to LDS.  P.V: a lane owns
// D / 64 consecutive values of head_dim and walks the chunk's visible keys (a wave-wide bit
// mask), so V rows are read with consecutive lanes on consecutive bytes.  The four waves'
// states are combined through LDS at the end.
#include "rkv_internal.h"
#include "rkv_wave.h"

#include <math.h>

namespace rkv {

namespace {

constexpr int kWavesH = 4;
constexpr int kRmax = 8;  // gqa * n_q rows per KV head

template <int T, int D> constexpr int hd_row_bytes() { return T == T_F16 ? 2 * D : (T == T_Q8_0 ? D / 32 * 34 : D / 32 * 18); }

__device__ __forceinline__ float h2f_bits(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

// Value e of a row (exact: binary16 as is, q8_0 d*q, q4_0 d*(n-8) with byte j holding element j
// in its low nibble and element j+16 in its high nibble).
template <int T>
__device__ __forceinline__ float row_value(const uint8_t *row, int e) {
    if constexpr (T == T_F16) {
        return h2f_bits(*reinterpret_cast<const uint16_t *>(row + 2 * e));
    } else if constexpr (T == T_Q8_0) {
        const uint8_t *b = row + 34 * (e >> 5);
        const float d = h2f_bits((uint16_t)(b[0] | (b[1] << 8)));
        return d * (float)(int8_t)b[2 + (e & 31)];
    } else {
        const uint8_t *b = row + 18 * (e >> 5);
        const float d = h2f_bits((uint16_t)(b[0] | (b[1] << 8)));
        const int i = e & 31;
        const int byte = b[2 + (i & 15)];
        const int n = i < 16 ? (byte & 15) : (byte >> 4);
        return d * (float)(n - 8);
    }
}

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int D, int KT, int VT, bool CAP>
__global__ void __launch_bounds__(64 * kWavesH) decode_hd_kernel(const SegParams p) {
    constexpr int EPL = D / 64;  // head_dim values per lane in P.V
    constexpr int PS = 2 + D;    // partial row stride
    __shared__ float s_q[kRmax][D];
    __shared__ float s_p[kWavesH][kRmax][64];
    __shared__ float s_m[kWavesH][kRmax][PS];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int bid = blockIdx.x;
    const int split = bid % p.n_splits;
    bid /= p.n_splits;
    const int g = bid % p.n_head_kv;
    const int b = bid / p.n_head_kv;
    const int R = p.gqa * p.n_q;  // <= kRmax (checked on the host)

    const int64_t c_beg = (int64_t)split * p.cells_per_split;
    const int64_t c_end = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    const uint8_t *kbase = p.k + (int64_t)g * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)g * p.v_s2;

    // Q rows rho = i * gqa + r (query i, head g * gqa + r), scaled, in LDS
    for (int idx = tid; idx < R * D; idx += 64 * kWavesH) {
        const int rho = idx / D, e = idx % D;
        const int r = rho % p.gqa, i = rho / p.gqa;
        s_q[rho][e] = (float)p.q[(int64_t)i * p.q_s1 + (int64_t)(g * p.gqa + r) * p.q_s2 + (int64_t)b * p.q_s3 + e];
    }
    __syncthreads();

    float m[kRmax], l[kRmax], acc[kRmax][EPL];
#pragma unroll
    for (int rho = 0; rho < kRmax; ++rho) {
        m[rho] = -INFINITY;
        l[rho] = 0.f;
#pragma unroll
        for (int k = 0; k < EPL; ++k) acc[rho][k] = 0.f;
    }

    const int64_t n_ch = c_end > c_beg ? (c_end - c_beg + 63) / 64 : 0;
    for (int64_t ch = wave; ch < n_ch; ch += kWavesH) {
        const int64_t c0 = c_beg + 64 * ch;
        const int64_t j = c0 + lane;  // this lane's key (segment-local cell)
        float s[kRmax];
#pragma unroll
        for (int rho = 0; rho < kRmax; ++rho) s[rho] = -INFINITY;
        if (j < c_end) {
            const uint8_t *krow = kbase + j * p.k_s1;
            float dot[kRmax];
#pragma unroll
            for (int rho = 0; rho < kRmax; ++rho) dot[rho] = 0.f;
            for (int e = 0; e < D; ++e) {
                const float kv = row_value<KT>(krow, e);
#pragma unroll
                for (int rho = 0; rho < kRmax; ++rho)
                    if (rho < R) dot[rho] = fmaf(s_q[rho][e], kv, dot[rho]);
            }
#pragma unroll
            for (int rho = 0; rho < kRmax; ++rho) {
                if (rho >= R) continue;
                const int i = rho / p.gqa;
                float x = p.scale_log2 * dot[rho] * 0.6931471805599453f;  // scale * <q, k>
                if (CAP) x = p.cap_l2 * 0.6931471805599453f * tanhf(p.cap_cs * dot[rho]);
                bool vis = p.q_pos0 < 0 || p.pos0 + j <= p.q_pos0 + i;
                if (vis && p.mask) {
                    const float mv = (float)p.mask[p.pos0 + j + (int64_t)i * p.m_s1 + (int64_t)b * p.m_s3];
                    x += mv;
                    vis = mv > -INFINITY;
                }
                s[rho] = vis ? x : -INFINITY;
            }
        }
        // online softmax per row over this chunk (natural-log units)
        uint64_t live = 0;
#pragma unroll
        for (int rho = 0; rho < kRmax; ++rho) {
            if (rho >= R) continue;
            const float cm = wave_max_f(s[rho]);
            float pj = 0.f;
            if (cm > -INFINITY) {
                if (cm > m[rho]) {
                    const float a = m[rho] == -INFINITY ? 0.f : __expf(m[rho] - cm);
                    l[rho] *= a;
#pragma unroll
                    for (int k = 0; k < EPL; ++k) acc[rho][k] *= a;
                    m[rho] = cm;
                }
                pj = s[rho] == -INFINITY ? 0.f : __expf(s[rho] - m[rho]);
            }
            l[rho] += pj;  // per-lane part; summed over the wave at the end
            s_p[wave][rho][lane] = pj;
            live |= __builtin_amdgcn_ballot_w64(pj > 0.f);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        // P.V over the chunk's keys with a nonzero weight
        while (live) {
            const int jj = __builtin_ctzll(live);
            live &= live - 1;
            const uint8_t *vrow = vbase + (c0 + jj) * p.v_s1;
            float vv[EPL];
#pragma unroll
            for (int k = 0; k < EPL; ++k) vv[k] = row_value<VT>(vrow, EPL * lane + k);
#pragma unroll
            for (int rho = 0; rho < kRmax; ++rho) {
                if (rho >= R) continue;
                const float w = s_p[wave][rho][jj];
#pragma unroll
                for (int k = 0; k < EPL; ++k) acc[rho][k] = fmaf(w, vv[k], acc[rho][k]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }

    // the wave's state per row to LDS, then the four waves combined
#pragma unroll
    for (int rho = 0; rho < kRmax; ++rho) {
        if (rho >= R) continue;
        const float lt = wave_sum_f(l[rho]);
        if (lane == 0) {
            s_m[wave][rho][0] = m[rho];
            s_m[wave][rho][1] = lt;
        }
#pragma unroll
        for (int k = 0; k < EPL; ++k) s_m[wave][rho][2 + EPL * lane + k] = acc[rho][k];
    }
    __syncthreads();
    const int slot = p.slot0 + split;
    for (int idx = tid; idx < R * PS; idx += 64 * kWavesH) {
        const int rho = idx / PS, c = idx % PS;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < kWavesH; ++wv) M = fmaxf(M, s_m[wv][rho][0]);
        float v = 0.f;
        if (c == 0) {
            v = M;
        } else if (M > -INFINITY) {
#pragma unroll
            for (int wv = 0; wv < kWavesH; ++wv) {
                const float mw = s_m[wv][rho][0];
                if (mw > -INFINITY) v = fmaf(s_m[wv][rho][c], __expf(mw - M), v);
            }
        }
        const int r = rho % p.gqa, i = rho / p.gqa;
        const int64_t row = (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
        p.partials[((int64_t)slot * p.n_rows + row) * PS + c] = v;
    }
}

// One workgroup of D threads per output row: O = sum_s VKQ_s e^{M_s - M*} / sum_s S_s e^{M_s - M*},
// LSE = M* + ln S*; a row whose segments are all empty gets O = 0 and LSE = -inf.
template <int D>
__global__ void __launch_bounds__(D) merge_hd_kernel(const float *part, int n_seg, int64_t n_rows, float *o,
                                                     float *lse) {
    constexpr int PS = 2 + D;
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    float M = -INFINITY;
    for (int sg = 0; sg < n_seg; ++sg) M = fmaxf(M, part[((int64_t)sg * n_rows + row) * PS]);
    float S = 0.f, a = 0.f;
    if (M > -INFINITY) {
        for (int sg = 0; sg < n_seg; ++sg) {
            const float *q = part + ((int64_t)sg * n_rows + row) * PS;
            if (q[0] == -INFINITY) continue;
            const float w = __expf(q[0] - M);
            S = fmaf(q[1], w, S);
            a = fmaf(q[2 + t], w, a);
        }
    }
    const bool ok = M > -INFINITY && S > 0.f;
    o[row * D + t] = ok ? a / S : 0.f;
    if (t == 0 && lse) lse[row] = ok ? M + logf(S) : -INFINITY;
}

template <int D, int KT, int VT>
hipError_t launch_hd(const SegParams &p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.n_splits * p.n_head_kv * p.n_seq;
    if (blocks <= 0) return hipSuccess;
    if (p.cap_l2 != 0.f)
        launch_seg(decode_hd_kernel<D, KT, VT, true>, dim3((unsigned)blocks), dim3(64 * kWavesH), s, p);
    else
        launch_seg(decode_hd_kernel<D, KT, VT, false>, dim3((unsigned)blocks), dim3(64 * kWavesH), s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_hd_types(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (k_type == T_F16 && v_type == T_F16) return launch_hd<D, T_F16, T_F16>(p, s);
    if (k_type == T_Q8_0 && v_type == T_Q4_0) return launch_hd<D, T_Q8_0, T_Q4_0>(p, s);
    if (k_type == T_Q8_0 && v_type == T_F16) return launch_hd<D, T_Q8_0, T_F16>(p, s);
    if (k_type == T_F16 && v_type == T_Q4_0) return launch_hd<D, T_F16, T_Q4_0>(p, s);
    return hipErrorNotSupported;
}

}  // namespace

bool head_dim_supported(int d) { return d == 64 || d == 128 || d == 256; }

hipError_t launch_decode_hd(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (p.rows || p.gqa * p.n_q > kRmax) return hipErrorNotSupported;
    if (p.d == 64) return launch_hd_types<64>(p, k_type, v_type, s);
    if (p.d == 256) return launch_hd_types<256>(p, k_type, v_type, s);
    return hipErrorNotSupported;
}

hipError_t launch_merge_hd(const float *partials, int n_seg, int64_t n_rows, int dv, float *o, float *lse,
                           hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    if (dv == 64)
        hipLaunchKernelGGL(merge_hd_kernel<64>, dim3((unsigned)n_rows), dim3(64), 0, s, partials, n_seg, n_rows, o, lse);
    else if (dv == 256)
        hipLaunchKernelGGL(merge_hd_kernel<256>, dim3((unsigned)n_rows), dim3(256), 0, s, partials, n_seg, n_rows, o,
                           lse);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

}  // namespace rkv
