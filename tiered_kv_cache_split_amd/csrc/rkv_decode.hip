// Vector (VALU) segment kernel for decode and unified-pool attention on gfx950,
// plus the log-sum-exp merge, the dequantiser used by tests, and the word-granularity
// host reader kept as a measured contrast to the bulk DMA lift.
//
// What a segment computes (opencoti-llamafile patch 0070-rolling-kv, fattn.cu
// streaming_lse_kernel and the tail-partial op): for every output row, over the keys of
// the segment, M = max s_j, S = sum exp(s_j - M), VKQ = sum exp(s_j - M) v_j with
// s_j = scale*<q, k_j> + mask_j; a -inf key contributes nothing.  Rows of one KV head
// (the gqa query heads times the n_q queries) are computed together so every K/V byte
// is read from HBM once.
//
// Launch shape: one 64-lane wave per workgroup; a workgroup owns one (split, KV head,
// sequence) and walks its cells 64 at a time:
//   1. the 64 rows of K and V are fetched with coalesced 8- or 16-byte loads (the raw
//      bytes, f16 or quant blocks) into registers one chunk ahead, then stored to LDS;
//   2. lane c takes cell c: Q.K for all rows with v_dot2_f32_f16 (q8_0 codes become
//      exact binary16 integers through a byte permute and one packed subtract), scale
//      applied per 32-value block;
//   3. online softmax in the exp2 domain, wave-wide max by butterfly;
//   4. P.V with lanes over head_dim: four 16-lane groups take four cells per step, each
//      lane eight values, dequantised exactly in float32;
//   5. after the last chunk the four groups are folded and the partial is written.
#include "rkv_internal.h"
#include "rkv_quant.h"

#include <math.h>

#include <algorithm>

namespace rkv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Chunk fetch geometry of a row format.  A row of `kRow` bytes is read as kMain units
// of kUnit bytes (64/kMain rows per wave instruction, kMain instructions per 64 rows)
// plus, when the row is longer, one tail unit per row (lane l takes row l).  Every lane
// then needs one base offset; the per-instruction step is uniform.
template <int T> struct RowFmt;
template <> struct RowFmt<T_F16> {
    using U = uint4;
    static constexpr int kRow = 256, kUnit = 16, kMain = 16, kTail = 0;
};
template <> struct RowFmt<T_Q8_0> {
    using U = uint2;
    static constexpr int kRow = kQ8Row, kUnit = 8, kMain = 16, kTail = 1;
};
template <> struct RowFmt<T_Q4_0> {
    using U = uint2;
    static constexpr int kRow = kQ4Row, kUnit = 8, kMain = 8, kTail = 1;
};
// LDS row strides: K rows are read one row per lane, so binary16 rows get one spare
// 16-byte unit (272 B) to make the 128-bit reads bank-conflict free; 136-byte q8_0 rows
// already are.  V rows are read by 16-lane groups in full and need no padding.
template <int T> constexpr int k_lds_stride() { return T == T_F16 ? 272 : RowFmt<T>::kRow; }
template <int T> constexpr int v_lds_stride() { return RowFmt<T>::kRow; }

typedef const __attribute__((address_space(4))) uint32_t cu32;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }

// Four bytes starting at byte offset `off` of a register-resident row (off is a
// compile-time constant after unrolling).
template <int N>
__device__ __forceinline__ uint32_t bytes4(const uint32_t (&w)[N], int off) {
    const int i = off >> 2, sh = off & 3;
    if (sh == 0) return w[i];
    return __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
}

// int8 codes (xor 0x80 already applied, so unsigned u = q + 128) -> two binary16 pairs
// (q0,q1), (q2,q3): 0x6400|u is the half 1024+u, minus 1152 gives q exactly.
__device__ __forceinline__ void codes_to_h2(uint32_t u, half2_t &a, half2_t &b) {
    const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x05010400u)) - bias;
    b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x05030402u)) - bias;
}

// Occupancy bound: the per-wave LDS footprint allows about three waves per SIMD for
// quant rows and two for binary16 rows; the register budget is set to match.
template <int KT, int VT, int R> constexpr int waves_per_eu() { return (KT == T_F16 || VT == T_F16 || R >= 4) ? 2 : 3; }

// Fetch 64 rows of one format into registers.  ROWS: gathered pool rows (64-bit
// addresses, -1 reads nothing); otherwise a buffer descriptor over the chunk whose size
// covers exactly the valid rows, so rows past the end read as zero without a branch.
template <int T, bool ROWS>
__device__ __forceinline__ void fetch_rows(typename RowFmt<T>::U (&buf)[RowFmt<T>::kMain + RowFmt<T>::kTail],
                                           const uint8_t *base, int64_t s1, int64_t c0, int64_t nv,
                                           int myrow, int lane) {
    using F = RowFmt<T>;
    using U = typename F::U;
    constexpr int kRpi = 64 / F::kMain;  // rows per instruction
    const int r_in = lane / F::kMain, w = lane % F::kMain;
    if constexpr (ROWS) {
#pragma unroll
        for (int u = 0; u < F::kMain; ++u) {
            const int row = __shfl(myrow, kRpi * u + r_in, 64);
            U x = {};
            if (row >= 0) x = *reinterpret_cast<const U *>(base + (int64_t)row * s1 + w * F::kUnit);
            buf[u] = x;
        }
        if constexpr (F::kTail) {
            U x = {};
            if (myrow >= 0) x = *reinterpret_cast<const U *>(base + (int64_t)myrow * s1 + F::kMain * F::kUnit);
            buf[F::kMain] = x;
        }
    } else {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(base + c0 * s1), (short)0, (int)(nv * s1), 0x00020000);
        const int vo = r_in * (int)s1 + w * F::kUnit;
#pragma unroll
        for (int u = 0; u < F::kMain; ++u) {
            const int o = vo + kRpi * u * (int)s1;
            if constexpr (F::kUnit == 16)
                buf[u] = __builtin_bit_cast(U, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0));
            else
                buf[u] = __builtin_bit_cast(U, __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0));
        }
        if constexpr (F::kTail) {
            const int o = lane * (int)s1 + F::kMain * F::kUnit;
            buf[F::kMain] = __builtin_bit_cast(U, __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0));
        }
    }
}

template <int T>
__device__ __forceinline__ void stash_rows(const typename RowFmt<T>::U (&buf)[RowFmt<T>::kMain + RowFmt<T>::kTail],
                                           uint8_t *lds, int stride, int lane) {
    using F = RowFmt<T>;
    using U = typename F::U;
    constexpr int kRpi = 64 / F::kMain;
    const int r_in = lane / F::kMain, w = lane % F::kMain;
    uint8_t *d = lds + r_in * stride + w * F::kUnit;
#pragma unroll
    for (int u = 0; u < F::kMain; ++u) *reinterpret_cast<U *>(d + kRpi * u * stride) = buf[u];
    if constexpr (F::kTail) *reinterpret_cast<U *>(lds + lane * stride + F::kMain * F::kUnit) = buf[F::kMain];
}

template <int KT, int VT, int R, bool ROWS>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(waves_per_eu<KT, VT, R>())))
decode_seg_kernel(const SegParams p) {
    using KF = RowFmt<KT>;
    using VF = RowFmt<VT>;
    constexpr int kKs = k_lds_stride<KT>(), kVs = v_lds_stride<VT>();
    __shared__ __attribute__((aligned(16))) uint8_t s_k[kChunk * kKs];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kChunk * kVs];
    __shared__ float s_p[R][kChunk];

    const int lane = threadIdx.x;
    int bid = blockIdx.x;
    const int g = bid % p.n_head_kv;
    bid /= p.n_head_kv;
    const int split = bid % p.n_splits;
    const int b = bid / p.n_splits;

    const int64_t c_beg = (int64_t)split * p.cells_per_split;
    const int64_t c_end = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    const uint8_t *kbase = p.k + (int64_t)g * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)g * p.v_s2;
    const int32_t *rows = ROWS ? p.rows + (int64_t)b * p.rows_s : nullptr;

    // rows of this KV head: rho = i*gqa + r  ->  query i, head h = g*gqa + r.  Q words are
    // read through the constant address space so they come in by scalar loads and feed
    // v_dot2 as SGPR operands.
    const uint32_t *qw[R];
    int qi[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const int r = rho % p.gqa, i = rho / p.gqa;
        const int h = g * p.gqa + r;
        qw[rho] = reinterpret_cast<const uint32_t *>(p.q + (int64_t)i * p.q_s1 +
                                                      (int64_t)h * p.q_s2 + (int64_t)b * p.q_s3);
        qi[rho] = i;
    }

    float m[R], l[R], acc[R][8];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        m[rho] = -INFINITY;
        l[rho] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rho][e] = 0.f;
    }

    typename KF::U kb[KF::kMain + KF::kTail];
    typename VF::U vb[VF::kMain + VF::kTail];

    // Row (cell or pool row) of this lane's cell in the chunk starting at c0, -1 if none.
    auto row_of = [&](int64_t c0) -> int {
        const int64_t c = c0 + lane;
        if (c >= c_end) return -1;
        return ROWS ? rows[c] : (int)c;
    };
    auto fetch = [&](int64_t c0, int myrow) {
        const int64_t nv = max((int64_t)0, min((int64_t)kChunk, c_end - c0));
        fetch_rows<KT, ROWS>(kb, kbase, p.k_s1, c0, nv, myrow, lane);
        fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, c0, nv, myrow, lane);
    };

    const int64_t n_chunks = (c_end > c_beg) ? (c_end - c_beg + kChunk - 1) / kChunk : 0;
    int myrow = -1;
    if (n_chunks > 0) {
        myrow = row_of(c_beg);
        fetch(c_beg, myrow);
    }
    const int grp = lane >> 4, kk = lane & 15;

    for (int64_t ch = 0; ch < n_chunks; ++ch) {
        const int64_t c0 = c_beg + ch * kChunk;
        stash_rows<KT>(kb, s_k, kKs, lane);
        stash_rows<VT>(vb, s_v, kVs, lane);
        const int cur_row = myrow;
        __syncthreads();
        // next chunk (past c_end every row is -1 / out of range and nothing is read)
        myrow = row_of(c0 + kChunk);
        fetch(c0 + kChunk, myrow);

        // ---- Q.K, lane = cell
        float s[R];
#pragma unroll
        for (int rho = 0; rho < R; ++rho) s[rho] = 0.f;
        if constexpr (KT == T_Q8_0) {
            const uint8_t *kr = s_k + lane * kKs;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                // block blk: scale at byte 34*blk, codes at 34*blk+2 .. +33 (2 bytes off
                // dword alignment for even blocks)
                uint32_t w[10];
                const int base = 34 * blk, a0 = base & ~3;
#pragma unroll
                for (int j = 0; j < 9; j += 1) w[j] = *reinterpret_cast<const uint32_t *>(kr + a0 + 4 * j);
                const float dk = h2f((base & 3) ? (w[0] >> 16) : w[0]);
                half2_t a[8], c[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int off = (base & 3) + 2 + 4 * t;  // relative to a0
                    const uint32_t x = (off & 3) ? __builtin_amdgcn_alignbyte(w[(off >> 2) + 1], w[off >> 2], off & 3)
                                                 : w[off >> 2];
                    codes_to_h2(x ^ 0x80808080u, a[t], c[t]);
                }
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    // The Q block pointer depends on the previous row's score, so only one
                    // 16-word Q block is held in SGPRs at a time.
                    cu32 *qb = (cu32 *)(qw[rho] + 16 * blk);
                    asm volatile("" : "+s"(qb) : "v"(s[rho > 0 ? rho - 1 : R - 1]));
                    float dot = 0.f;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        dot = __builtin_amdgcn_fdot2(a[t], as_h2(qb[2 * t]), dot, false);
                        dot = __builtin_amdgcn_fdot2(c[t], as_h2(qb[2 * t + 1]), dot, false);
                    }
                    s[rho] = fmaf(dk, dot, s[rho]);
                }
            }
        } else {
            const uint4 *kr = reinterpret_cast<const uint4 *>(s_k + lane * kKs);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint4 x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = kr[4 * q4 + j];
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    cu32 *qb = (cu32 *)(qw[rho] + 16 * q4);
                    asm volatile("" : "+s"(qb) : "v"(s[rho > 0 ? rho - 1 : R - 1]));
                    float dot = s[rho];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        dot = __builtin_amdgcn_fdot2(as_h2(x[j].x), as_h2(qb[4 * j + 0]), dot, false);
                        dot = __builtin_amdgcn_fdot2(as_h2(x[j].y), as_h2(qb[4 * j + 1]), dot, false);
                        dot = __builtin_amdgcn_fdot2(as_h2(x[j].z), as_h2(qb[4 * j + 2]), dot, false);
                        dot = __builtin_amdgcn_fdot2(as_h2(x[j].w), as_h2(qb[4 * j + 3]), dot, false);
                    }
                    s[rho] = dot;
                }
            }
        }

        // ---- scores, online softmax (exp2 domain)
        const int64_t cell = c0 + lane;
        const bool valid = cur_row >= 0;
#pragma unroll
        for (int rho = 0; rho < R; ++rho) {
            float x = s[rho] * p.scale_log2;
            if (valid && p.mask) {
                const _Float16 mv = p.mask[p.pos0 + cell + (int64_t)qi[rho] * p.m_s1 + (int64_t)b * p.m_s3];
                x += (float)mv * kLog2e;
            }
            if (p.q_pos0 >= 0 && p.pos0 + cell > p.q_pos0 + qi[rho]) x = -INFINITY;
            if (!valid) x = -INFINITY;
            const float mn = fmaxf(m[rho], wave_max(x));
            float pr = 0.f;
            if (mn != -INFINITY) {
                const float alpha = __builtin_amdgcn_exp2f(m[rho] - mn);
                pr = __builtin_amdgcn_exp2f(x - mn);
                l[rho] = fmaf(l[rho], alpha, pr);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[rho][e] *= alpha;
                m[rho] = mn;
            }
            s_p[rho][lane] = pr;
        }
        __syncthreads();

        // ---- P.V, lanes over head_dim: group grp takes cell 4*st+grp, lane kk eight values
#pragma unroll 2
        for (int st = 0; st < kChunk / 4; ++st) {
            const int cl = 4 * st + grp;
            float v[8];
            if constexpr (VT == T_Q4_0) {
                const uint8_t *vr = s_v + cl * kVs;
                const int blk = kk >> 2, j4 = kk & 3;
                const float dv = h2f(ld_u16(vr + 18 * blk));
                const int off = 18 * blk + 2 + 4 * j4;
                const uint32_t x = ld_u16(vr + off) | (ld_u16(vr + off + 2) << 16);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v[t] = dv * (float)((int)((x >> (8 * t)) & 15u) - 8);
                    v[4 + t] = dv * (float)((int)((x >> (8 * t + 4)) & 15u) - 8);
                }
            } else {
                const uint4 x = *reinterpret_cast<const uint4 *>(s_v + cl * kVs + 16 * kk);
                const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = h2f(w4[j]);
                    v[2 * j + 1] = h2f(w4[j] >> 16);
                }
            }
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                const float pr = s_p[rho][cl];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[rho][e] = fmaf(pr, v[e], acc[rho][e]);
            }
        }
        __syncthreads();
    }

    // ---- fold the four cell groups, reduce row sums, write the partial
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[rho][e] += __shfl_xor(acc[rho][e], 16, 64);
            acc[rho][e] += __shfl_xor(acc[rho][e], 32, 64);
        }
        l[rho] = wave_sum(l[rho]);
    }
    const int slot = p.slot0 + split;
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const int r = rho % p.gqa, i = rho / p.gqa;
        const int h = g * p.gqa + r;
        const int64_t row = h + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)slot * p.n_rows + row) * kPartialStride;
        if (lane < 16) {
            if constexpr (VT == T_Q4_0) {
                const int blk = kk >> 2, j4 = kk & 3;
                float *o0 = out + 2 + 32 * blk + 4 * j4;
                *reinterpret_cast<float4 *>(o0) = make_float4(acc[rho][0], acc[rho][1], acc[rho][2], acc[rho][3]);
                *reinterpret_cast<float4 *>(o0 + 16) = make_float4(acc[rho][4], acc[rho][5], acc[rho][6], acc[rho][7]);
            } else {
                float *o0 = out + 2 + 8 * kk;
                *reinterpret_cast<float4 *>(o0) = make_float4(acc[rho][0], acc[rho][1], acc[rho][2], acc[rho][3]);
                *reinterpret_cast<float4 *>(o0 + 4) = make_float4(acc[rho][4], acc[rho][5], acc[rho][6], acc[rho][7]);
            }
        }
        if (lane == 0) {
            out[0] = (m[rho] == -INFINITY) ? -INFINITY : m[rho] * kLn2;
            out[1] = l[rho];
        }
    }
}

// Log-sum-exp merge of partials (patch 0070 streaming_combine_kernel, applied to the
// un-normalised (M, S, VKQ) form).  One workgroup per output row: 128 lanes over the
// values times G groups over the segments; groups fold through LDS.
template <int G>
__global__ void __launch_bounds__(128 * G) merge_kernel(const float *__restrict__ part, int n_seg,
                                                        int64_t n_rows, float *__restrict__ o,
                                                        float *__restrict__ lse,
                                                        float *__restrict__ pout) {
    __shared__ float s_acc[G][kHeadDim];
    __shared__ float s_sum[G];
    const int64_t row = blockIdx.x;
    const int d = threadIdx.x & (kHeadDim - 1), grp = threadIdx.x / kHeadDim;
    const int64_t step = n_rows * kPartialStride;
    const float *base = part + row * kPartialStride;
    float M = -INFINITY;
    for (int s = 0; s < n_seg; ++s) M = fmaxf(M, base[s * step]);
    float S = 0.f, acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll 4
        for (int s = grp; s < n_seg; s += G) {
            const float *pp = base + s * step;
            const float Ms = pp[0];
            const float w = (Ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((Ms - M) * kLog2e);
            S = fmaf(pp[1], w, S);
            acc = fmaf(pp[2 + d], w, acc);
        }
    }
    if constexpr (G > 1) {
        s_acc[grp][d] = acc;
        if (d == 0) s_sum[grp] = S;
        __syncthreads();
        if (grp != 0) return;
        acc = 0.f;
        S = 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            acc += s_acc[j][d];
            S += s_sum[j];
        }
    }
    if (pout) {
        float *q = pout + row * kPartialStride;
        if (d == 0) {
            q[0] = M;
            q[1] = S;
        }
        q[2 + d] = acc;
        return;
    }
    const bool ok = (M != -INFINITY) && (S > 0.f);
    o[row * kHeadDim + d] = ok ? acc / S : 0.f;
    if (lse && d == 0) lse[row] = ok ? M + logf(S) : -INFINITY;
}

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

__global__ void __launch_bounds__(128) empty_partials_kernel(float *__restrict__ part) {
    float *q = part + (int64_t)blockIdx.x * kPartialStride;
    q[2 + threadIdx.x] = 0.f;
    if (threadIdx.x == 0) {
        q[0] = -INFINITY;
        q[1] = 0.f;
    }
}

__global__ void __launch_bounds__(128) dequant_kernel(const uint8_t *__restrict__ src, int type,
                                                      int64_t row_stride,
                                                      float *__restrict__ dst) {
    const int64_t row = blockIdx.x;
    const int e = threadIdx.x;
    dst[row * kHeadDim + e] = row_value(src + row * row_stride, type, e);
}

template <int KT, int VT, int R>
hipError_t launch_decode_r(const SegParams &p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.n_splits * p.n_head_kv * p.n_seq;
    if (p.rows)
        hipLaunchKernelGGL((decode_seg_kernel<KT, VT, R, true>), dim3((unsigned)blocks), dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL((decode_seg_kernel<KT, VT, R, false>), dim3((unsigned)blocks), dim3(64), 0, s, p);
    return hipGetLastError();
}

template <int KT, int VT>
hipError_t launch_decode_t(const SegParams &p, int R, hipStream_t s) {
    switch (R) {
        case 1: return launch_decode_r<KT, VT, 1>(p, s);
        case 2: return launch_decode_r<KT, VT, 2>(p, s);
        case 3: return launch_decode_r<KT, VT, 3>(p, s);
        case 4: return launch_decode_r<KT, VT, 4>(p, s);
        case 5: return launch_decode_r<KT, VT, 5>(p, s);
        case 6: return launch_decode_r<KT, VT, 6>(p, s);
        case 7: return launch_decode_r<KT, VT, 7>(p, s);
        case 8: return launch_decode_r<KT, VT, 8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_segment(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    const int R = p.gqa * p.n_q;
    if (k_type == T_Q8_0 && v_type == T_Q4_0) return launch_decode_t<T_Q8_0, T_Q4_0>(p, R, s);
    if (k_type == T_F16 && v_type == T_F16) return launch_decode_t<T_F16, T_F16>(p, R, s);
    if (k_type == T_Q8_0 && v_type == T_F16) return launch_decode_t<T_Q8_0, T_F16>(p, R, s);
    if (k_type == T_F16 && v_type == T_Q4_0) return launch_decode_t<T_F16, T_Q4_0>(p, R, s);
    return hipErrorInvalidValue;
}

hipError_t launch_merge(const float *partials, int n_seg, int64_t n_rows, float *o, float *lse,
                        float *partial_out, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    if (n_seg >= 32)
        hipLaunchKernelGGL(merge_kernel<8>, dim3((unsigned)n_rows), dim3(8 * kHeadDim), 0, s, partials,
                           n_seg, n_rows, o, lse, partial_out);
    else if (n_seg >= 4)
        hipLaunchKernelGGL(merge_kernel<2>, dim3((unsigned)n_rows), dim3(2 * kHeadDim), 0, s, partials,
                           n_seg, n_rows, o, lse, partial_out);
    else
        hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)n_rows), dim3(kHeadDim), 0, s, partials,
                           n_seg, n_rows, o, lse, partial_out);
    return hipGetLastError();
}

hipError_t launch_empty_partials(float *partials, int64_t n_rows, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(empty_partials_kernel, dim3((unsigned)n_rows), dim3(kHeadDim), 0, s, partials);
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

hipError_t launch_dequant_rows(const void *src, int type, int64_t n_rows, int64_t row_stride,
                               float *dst, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)n_rows), dim3(kHeadDim), 0, s,
                       static_cast<const uint8_t *>(src), type, row_stride, dst);
    return hipGetLastError();
}

}  // namespace rkv
