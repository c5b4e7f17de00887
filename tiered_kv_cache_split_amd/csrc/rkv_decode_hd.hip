// Decode segment kernel for head dims other than 128 -- dk = dv in {64, 256, 512} and the
// dk = 576 / dv = 512 pair -- and the log-sum-exp merge for those value widths.  The streaming
// op of opencoti-llamafile patch 0070-rolling-kv serves several head dims through the same
// split-and-combine (fattn.cu, the op's supported shapes, which list 512 and the 576/512 pair
// next to 64 and 256); the partial of a segment is the same (M, S, VKQ) triple as for head dim
// 128, stored with row stride 2 + dv.
//
// Workgroup = 256 threads for one (split, KV head, sequence); it walks the split in chunks of KC
// keys (64 for dk = 64, 16 otherwise) as a pipeline: the next chunk's K and V rows are loaded
// from HBM into registers (4-byte words, consecutive threads on consecutive words of a row)
// while the current chunk is computed from LDS.
//   Q.K  P = 256 / KC threads per key, each over E = dk / P dims (16: half of a q8_0 block;
//        32: one block; at dk = 576, 32 dims of one block plus 4 of the last two blocks, each
//        part times its own block's d), partial dots summed across the P adjacent lanes; the
//        R <= 8 query rows that read this KV head are done together.
//   softmax  wave w owns rows w and w + 4: chunk max, rescale factor and weights, in natural-log
//        units, kept in LDS for the P.V step.
//   P.V  thread t owns output columns t % dv (+ 256 c for dv = 512) of every row over the
//        chunk's keys j with j % KS = t / dv (KS = 256 / dv key subsets for dv < 256, so each V
//        value is dequantised once); the subsets' sums are added through LDS at the end.
// More than 8 rows per KV head (prefill, or decode with a wide query group) are split into row
// groups of 8, one workgroup each, adjacent in the grid so that the groups reading one chunk
// of keys run together.  With a row list (the unified-pool form of llama.cpp PR #29510,
// flash_attn_ext_rows) key j of sequence b is pool cell rows[j + rows_s * b]; a negative
// entry, or one past the pool, reads nothing and is hidden.
#include "rkv_internal.h"
#include "rkv_unpack.h"
#include "rkv_wave.h"

#include <math.h>

namespace rkv {

namespace {

constexpr int kRmax = 8;  // gqa * n_q rows per KV head
constexpr int kThreads = 256;

template <int T, int D> constexpr int hd_row_bytes() { return T == T_F16 ? 2 * D : (T == T_Q8_0 ? D / 32 * 34 : D / 32 * 18); }

__device__ __forceinline__ float h2f_bits(uint32_t x) { return f16_bits_to_f32(x); }

// Sum over each aligned group of P lanes (4, 8 or 16), in every lane of the group: DPP quad
// swaps; for 8 lanes the mirror inside each half row (lane i and 7 - i: the two quads); for 16
// rotations by 4 and 8 inside a 16-lane row.
template <int P>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp_f<kQuadSwap1>(x);
    x += dpp_f<kQuadSwap2>(x);
    if constexpr (P == 8) x += dpp_f<kRowHalfMirror>(x);
    if constexpr (P == 16) {
        x += dpp_f<kRowRor4>(x);
        x += dpp_f<kRowRor8>(x);
    }
    return x;
}

template <int DK, int DV, int KT, int VT>
struct HdGeom {
    static constexpr int KC = DK == 64 ? 64 : (DK == 128 ? 32 : 16);  // keys per chunk
    static constexpr int P = kThreads / KC;                // threads per key in Q.K
    static constexpr int E = DK / P;                       // dims per thread in Q.K (16, 32 or 36)
    // a thread's dims: EM consecutive ones from dim pq * EM (within one quant block), and at
    // dk = 576 also EX = 4 from dim 512 + pq * EX (within one block of the last two)
    static constexpr int EX = DK == 576 ? 4 : 0;
    static constexpr int EM = E - EX;
    static constexpr int KW = hd_row_bytes<KT, DK>() / 4;  // 4-byte words per K row
    static constexpr int VW = hd_row_bytes<VT, DV>() / 4;
    static constexpr int KWP = KW | 1, VWP = VW | 1;       // odd LDS row pitch: no bank conflicts
    static constexpr int NK = (KC * KW + kThreads - 1) / kThreads;  // words per thread per chunk
    static constexpr int NV = (KC * VW + kThreads - 1) / kThreads;
    static constexpr int CPT = DV > kThreads ? DV / kThreads : 1;  // P.V: columns per thread
    static constexpr int KS = DV >= kThreads ? 1 : kThreads / DV;  // P.V: threads per column (key subsets)
    static constexpr int KPS = KC / KS;                    // keys per subset (16)
    static_assert(P == 4 || P == 8 || P == 16, "Q.K groups are DPP quads, half rows or 16-lane rows");
    static_assert(EM == 16 || EM == 32, "a thread's main Q.K dims: half a block or a block");
    static_assert(E % 4 == 0 && DK % 32 == 0 && DV % 32 == 0, "whole quant blocks");
};

// Pool cell of key j: j itself, or rows[j] for a row list (-1: no cell).
__device__ __forceinline__ int64_t key_cell(const int32_t *rows, int64_t n_pool, int64_t j) {
    if (!rows) return j;
    const int32_t c = rows[j];
    return (c >= 0 && c < n_pool) ? (int64_t)c : -1;
}

// Chunk rows [c0, c0 + KC) of one KV head, words of row r in order; keys at or past c_end, and
// keys without a cell, read nothing (0).
template <int NW, int W, int KC>
__device__ __forceinline__ void load_rows(uint32_t (&buf)[NW], const uint8_t *base, int64_t s1, int64_t c0, int64_t c_end,
                                          const int32_t *rows, int64_t n_pool, int tid) {
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        const int f = tid + kThreads * u;
        const int r = f / W, w = f % W;
        buf[u] = 0u;
        if (f < KC * W && c0 + r < c_end) {
            const int64_t cell = key_cell(rows, n_pool, c0 + r);
            if (cell >= 0) buf[u] = *reinterpret_cast<const uint32_t *>(base + cell * s1 + 4 * w);
        }
    }
}
template <int NW, int W, int WP, int KC>
__device__ __forceinline__ void store_rows(const uint32_t (&buf)[NW], uint32_t *lds, int tid) {
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        const int f = tid + kThreads * u;
        if (f < KC * W) lds[(f / W) * WP + f % W] = buf[u];
    }
}

// Value e of a V row in LDS (exact: binary16 as is; q4_0 d*(n-8), byte j of a block holding
// element j in its low nibble and element j+16 in its high nibble).
template <int VT>
__device__ __forceinline__ float v_value(const uint8_t *row, int e) {
    if constexpr (VT == T_F16) {
        return h2f_bits(*reinterpret_cast<const uint16_t *>(row + 2 * e));
    } else {
        const uint8_t *b = row + 18 * (e >> 5);
        return h2f_bits(*reinterpret_cast<const uint16_t *>(b)) * q4_centered_f32(b + 2, e & 31);
    }
}

template <int DK, int DV, int KT, int VT, bool CAP>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DK == 64 ? 4 : (DK <= 256 ? 3 : (DK == 576 && KT == T_F16 ? 1 : 2)))))
decode_hd_kernel(const SegParams p) {
    using G = HdGeom<DK, DV, KT, VT>;
    constexpr int KC = G::KC, P = G::P, E = G::E, PS = 2 + DV;
    // Q row rho, part pq (16 values) at rho * P * QP + pq * QP: a pitch of 20 floats puts the P
    // parts that lanes of one wave read together on distinct LDS banks (a pitch of 16 maps every
    // fourth part to the same banks)
    constexpr int QP = E + 4;
    __shared__ __align__(16) float s_q[kRmax * P * QP];
    __shared__ uint32_t s_k[KC * G::KWP];
    __shared__ uint32_t s_v[KC * G::VWP];
    // scores, then weights; key j of the chunk at (j % KS) * KPS + j / KS so that each key
    // subset's weights are contiguous
    __shared__ __align__(16) float s_s[kRmax][KC];
    __shared__ float s_red[G::KS > 1 ? G::KS * kRmax * DV : 1];  // key-subset sums of P.V
    auto widx = [](int j) { return (j % G::KS) * G::KPS + j / G::KS; };
    __shared__ float s_alpha[kRmax];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // block = ((b * n_head_kv + g) * n_splits + split) * n_rg + rg: the row groups of one
    // (split, KV head, sequence) are adjacent
    const int R_all = p.gqa * p.n_q;
    const int n_rg = (R_all + kRmax - 1) / kRmax;
    int bid = blockIdx.x;
    const int rg = bid % n_rg;
    bid /= n_rg;
    const int split = bid % p.n_splits;
    bid /= p.n_splits;
    const int g = bid % p.n_head_kv;
    const int b = bid / p.n_head_kv;
    const int R0 = kRmax * rg;              // first row (rho = i * gqa + r) of this group
    const int R = min(kRmax, R_all - R0);   // rows of this group; local row rho is row R0 + rho
    const int32_t *rows = p.rows ? p.rows + (int64_t)b * p.rows_s : nullptr;

    const int64_t c_beg = (int64_t)split * p.cells_per_split;
    const int64_t c_end = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    const uint8_t *kbase = p.k + (int64_t)g * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)g * p.v_s2;

    // Q rows rho = i * gqa + r (query i, head g * gqa + r) in LDS; rows past R are zero
    for (int idx = tid; idx < kRmax * DK; idx += kThreads) {
        const int rho = idx / DK, e = idx % DK;
        const int r = (R0 + rho) % p.gqa, i = (R0 + rho) / p.gqa;
        const int part = (G::EX > 0 && e >= 512) ? (e - 512) / G::EX : e / G::EM;
        const int off = (G::EX > 0 && e >= 512) ? G::EM + (e - 512) % G::EX : e % G::EM;
        s_q[rho * P * QP + part * QP + off] = rho < R ? (float)p.q[(int64_t)i * p.q_s1 + (int64_t)(g * p.gqa + r) * p.q_s2 + (int64_t)b * p.q_s3 + e]
                              : 0.f;
    }

    // softmax state of the rows this wave owns (w, w + 4), the same in every lane
    float m_own[2] = {-INFINITY, -INFINITY}, l_own[2] = {0.f, 0.f};
    // P.V accumulators: columns e_pv + 256 c of every row, over key subset ks
    const int e_pv = tid % DV, ks = tid / DV;
    float acc[G::CPT][kRmax];
#pragma unroll
    for (int cp = 0; cp < G::CPT; ++cp)
#pragma unroll
        for (int rho = 0; rho < kRmax; ++rho) acc[cp][rho] = 0.f;

    const int kq = tid / P, pq = tid % P;  // Q.K: key kq of the chunk, dims [pq*E, pq*E + E)

    const int64_t n_ch = c_end > c_beg ? (c_end - c_beg + KC - 1) / KC : 0;
    uint32_t pk[G::NK], pv[G::NV];
    if (n_ch > 0) {
        load_rows<G::NK, G::KW, KC>(pk, kbase, p.k_s1, c_beg, c_end, rows, p.n_pool, tid);
        load_rows<G::NV, G::VW, KC>(pv, vbase, p.v_s1, c_beg, c_end, rows, p.n_pool, tid);
    }
    for (int64_t ch = 0; ch < n_ch; ++ch) {
        const int64_t c0 = c_beg + ch * KC;
        __syncthreads();  // the previous chunk's P.V is done with s_k, s_v and s_s
        store_rows<G::NK, G::KW, G::KWP, KC>(pk, s_k, tid);
        store_rows<G::NV, G::VW, G::VWP, KC>(pv, s_v, tid);
        __syncthreads();
        if (ch + 1 < n_ch) {  // next chunk in flight during this one
            load_rows<G::NK, G::KW, KC>(pk, kbase, p.k_s1, c0 + KC, c_end, rows, p.n_pool, tid);
            load_rows<G::NV, G::VW, KC>(pv, vbase, p.v_s1, c0 + KC, c_end, rows, p.n_pool, tid);
        }

        // ---- Q.K
        {
            const uint8_t *krow = reinterpret_cast<const uint8_t *>(s_k + kq * G::KWP);
            constexpr int EM = G::EM, EX = G::EX;
            const int e0 = pq * EM, e1 = 512 + pq * EX;
            float kv[E];
            float kscale = 1.f;
            if constexpr (KT == T_F16) {
#pragma unroll
                for (int i = 0; i < EM; i += 2) {
                    const uint32_t w = *reinterpret_cast<const uint32_t *>(krow + 2 * (e0 + i));
                    kv[i] = h2f_bits(w & 0xFFFFu);
                    kv[i + 1] = h2f_bits(w >> 16);
                }
#pragma unroll
                for (int i = 0; i < EX; i += 2) {
                    const uint32_t w = *reinterpret_cast<const uint32_t *>(krow + 2 * (e1 + i));
                    kv[EM + i] = h2f_bits(w & 0xFFFFu);
                    kv[EM + i + 1] = h2f_bits(w >> 16);
                }
            } else if constexpr (EX == 0) {
                // the thread's dims lie in one q8_0 block: its scale multiplies the dot
                const uint8_t *blk = krow + 34 * (e0 >> 5);
                kscale = h2f_bits(*reinterpret_cast<const uint16_t *>(blk));
                const uint8_t *codes = blk + 2 + (e0 & 31);
#pragma unroll
                for (int i = 0; i < E; i += 2) {
                    const uint32_t w = *reinterpret_cast<const uint16_t *>(codes + i);
                    kv[i] = q8_code_f32(w);
                    kv[i + 1] = q8_code_f32(w >> 8);
                }
            } else {
                // two blocks: each code times its own block's scale (d * q is exact in fp32)
                const uint8_t *b0 = krow + 34 * (e0 >> 5), *b1 = krow + 34 * (e1 >> 5);
                const float d0 = h2f_bits(*reinterpret_cast<const uint16_t *>(b0));
                const float d1 = h2f_bits(*reinterpret_cast<const uint16_t *>(b1));
#pragma unroll
                for (int i = 0; i < EM; i += 2) {
                    const uint32_t w = *reinterpret_cast<const uint16_t *>(b0 + 2 + (e0 & 31) + i);
                    kv[i] = q8_code_f32(w) * d0;
                    kv[i + 1] = q8_code_f32(w >> 8) * d0;
                }
#pragma unroll
                for (int i = 0; i < EX; i += 2) {
                    const uint32_t w = *reinterpret_cast<const uint16_t *>(b1 + 2 + (e1 & 31) + i);
                    kv[EM + i] = q8_code_f32(w) * d1;
                    kv[EM + i + 1] = q8_code_f32(w >> 8) * d1;
                }
            }
            float dot[kRmax];
#pragma unroll
            for (int rho = 0; rho < kRmax; ++rho) {
                float a = 0.f;
                if (rho < R) {
#pragma unroll
                    for (int i = 0; i < E; i += 4) {
                        const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[rho * P * QP + pq * QP + i]);
                        a = fmaf(q4.x, kv[i], a);
                        a = fmaf(q4.y, kv[i + 1], a);
                        a = fmaf(q4.z, kv[i + 2], a);
                        a = fmaf(q4.w, kv[i + 3], a);
                    }
                }
                dot[rho] = a * kscale;
                // one row's Q slice live at a time (the scheduler would otherwise hoist every
                // row's LDS reads and spill)
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int rho = 0; rho < kRmax; ++rho)
                if (rho < R) dot[rho] = group_sum<P>(dot[rho]);
            // every lane of the key's group holds all row dots: lane pq finishes rows pq, pq + P, ...
            const int64_t j = c0 + kq;  // segment-local cell
            for (int rho = pq; rho < R; rho += P) {
                float dr = dot[0];
#pragma unroll
                for (int k = 1; k < kRmax; ++k) dr = rho == k ? dot[k] : dr;
                const int i = (R0 + rho) / p.gqa;
                float x = CAP ? p.cap_l2 * kLn2 * tanhf(p.cap_cs * dr) : p.scale_log2 * kLn2 * dr;
                bool vis = j < c_end && (p.q_pos0 < 0 || p.pos0 + j <= p.q_pos0 + i) &&
                           (!rows || key_cell(rows, p.n_pool, j) >= 0);
                if (vis && p.mask) {
                    const float mv = (float)p.mask[p.pos0 + j + (int64_t)i * p.m_s1 + (int64_t)b * p.m_s3];
                    x += mv;
                    vis = mv > -INFINITY;
                }
                s_s[rho][widx(kq)] = vis ? x : -INFINITY;
            }
        }
        __syncthreads();

        // ---- online softmax: wave w, rows w and w + 4 (natural-log units)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rho = wave + 4 * h;
            if (rho >= R) continue;
            const float sj = lane < KC ? s_s[rho][widx(lane)] : -INFINITY;
            const float cm = wave_max(sj);
            float alpha = 1.f;
            if (cm > m_own[h]) {
                alpha = m_own[h] == -INFINITY ? 0.f : __expf(m_own[h] - cm);
                m_own[h] = cm;
            }
            const float pj = sj == -INFINITY ? 0.f : __expf(sj - m_own[h]);
            l_own[h] = fmaf(l_own[h], alpha, wave_sum(pj));
            if (lane < KC) s_s[rho][widx(lane)] = pj;
            if (lane == 0) s_alpha[rho] = alpha;
        }
        __syncthreads();

        // ---- P.V over all KC rows of the chunk: rows past the segment's end hold zeros in LDS
        // and have weight 0, as have masked keys
        {
#pragma unroll
            for (int rho = 0; rho < kRmax; ++rho)
                if (rho < R) {
                    const float al = s_alpha[rho];
#pragma unroll
                    for (int cp = 0; cp < G::CPT; ++cp) acc[cp][rho] *= al;
                }
            const uint8_t *vcol = reinterpret_cast<const uint8_t *>(s_v);
#pragma unroll 1
            for (int t = 0; t < G::KPS; t += 4) {
#pragma unroll
                for (int cp = 0; cp < G::CPT; ++cp) {
                    float v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        v[u] = v_value<VT>(vcol + (ks + G::KS * (t + u)) * (4 * G::VWP), e_pv + kThreads * cp);
#pragma unroll
                    for (int rho = 0; rho < kRmax; ++rho) {
                        if (rho < R) {
                            const float4 w = *reinterpret_cast<const float4 *>(&s_s[rho][ks * G::KPS + t]);
                            acc[cp][rho] = fmaf(w.x, v[0], fmaf(w.y, v[1], fmaf(w.z, v[2], fmaf(w.w, v[3], acc[cp][rho]))));
                        }
                    }
                }
            }
        }
    }

    // ---- partials: M and S from the owning waves, VKQ from every thread
    const int slot = p.slot0 + split;
    auto out_row = [&](int rho) {
        const int r = (R0 + rho) % p.gqa, i = (R0 + rho) / p.gqa;
        return ((int64_t)slot * p.n_rows + (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b)) * PS;
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rho = wave + 4 * h;
        if (rho < R && lane == 0) {
            p.partials[out_row(rho)] = m_own[h];
            p.partials[out_row(rho) + 1] = l_own[h];
        }
    }
    if constexpr (G::KS == 1) {
#pragma unroll
        for (int rho = 0; rho < kRmax; ++rho)
            if (rho < R) {
#pragma unroll
                for (int cp = 0; cp < G::CPT; ++cp) p.partials[out_row(rho) + 2 + e_pv + kThreads * cp] = acc[cp][rho];
            }
    } else {
#pragma unroll
        for (int rho = 0; rho < kRmax; ++rho)
            if (rho < R) s_red[(ks * kRmax + rho) * DV + e_pv] = acc[0][rho];
        __syncthreads();
        for (int idx = tid; idx < R * DV; idx += kThreads) {
            const int rho = idx / DV, e = idx % DV;
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < G::KS; ++k) a += s_red[(k * kRmax + rho) * DV + e];
            p.partials[out_row(rho) + 2 + e] = a;
        }
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
#pragma unroll 8
    for (int sg = 0; sg < n_seg; ++sg) M = fmaxf(M, part[((int64_t)sg * n_rows + row) * PS]);
    float S = 0.f, a = 0.f;
    if (M > -INFINITY) {
        // branch-free so that the unrolled loads of several segments are in flight together
#pragma unroll 8
        for (int sg = 0; sg < n_seg; ++sg) {
            const float *q = part + ((int64_t)sg * n_rows + row) * PS;
            const float m = q[0], s = q[1], v = q[2 + t];
            // (an empty partial, M = -inf, need not have written its values)
            const float w = m == -INFINITY ? 0.f : __expf(m - M);
            S = fmaf(s, w, S);
            a = w > 0.f ? fmaf(v, w, a) : a;
        }
    }
    const bool ok = M > -INFINITY && S > 0.f;
    o[row * D + t] = ok ? a / S : 0.f;
    if (t == 0 && lse) lse[row] = ok ? M + logf(S) : -INFINITY;
}

template <int DK, int DV, int KT, int VT>
hipError_t launch_hd(const SegParams &p, hipStream_t s) {
    const int64_t n_rg = ((int64_t)p.gqa * p.n_q + kRmax - 1) / kRmax;
    const int64_t blocks = (int64_t)p.n_splits * p.n_head_kv * p.n_seq * n_rg;
    if (blocks > ((int64_t)1 << 31) - 1) return hipErrorInvalidValue;
    if (blocks <= 0) return hipSuccess;
    if (p.cap_l2 != 0.f)
        launch_seg(decode_hd_kernel<DK, DV, KT, VT, true>, dim3((unsigned)blocks), dim3(kThreads), s, p);
    else
        launch_seg(decode_hd_kernel<DK, DV, KT, VT, false>, dim3((unsigned)blocks), dim3(kThreads), s, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_hd_types(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (k_type == T_F16 && v_type == T_F16) return launch_hd<DK, DV, T_F16, T_F16>(p, s);
    if (k_type == T_Q8_0 && v_type == T_Q4_0) return launch_hd<DK, DV, T_Q8_0, T_Q4_0>(p, s);
    if (k_type == T_Q8_0 && v_type == T_F16) return launch_hd<DK, DV, T_Q8_0, T_F16>(p, s);
    if (k_type == T_F16 && v_type == T_Q4_0) return launch_hd<DK, DV, T_F16, T_Q4_0>(p, s);
    return hipErrorNotSupported;
}

}  // namespace

bool head_dim_supported(int d) { return d == 64 || d == 128 || d == 256 || d == 512 || d == 576; }

bool head_dims_supported(int dk, int dv) {
    return (dk == dv && (dk == 64 || dk == 128 || dk == 256 || dk == 512)) || (dk == 576 && dv == 512);
}

hipError_t launch_decode_hd(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (p.gqa * p.n_q < 1) return hipErrorInvalidValue;
    if (p.d == 64 && p.dv == 64) return launch_hd_types<64, 64>(p, k_type, v_type, s);
    if (p.d == 128 && p.dv == 128) return launch_hd_types<128, 128>(p, k_type, v_type, s);
    if (p.d == 256 && p.dv == 256) return launch_hd_types<256, 256>(p, k_type, v_type, s);
    if (p.d == 512 && p.dv == 512) return launch_hd_types<512, 512>(p, k_type, v_type, s);
    if (p.d == 576 && p.dv == 512) return launch_hd_types<576, 512>(p, k_type, v_type, s);
    return hipErrorNotSupported;
}

hipError_t launch_merge_hd(const float *partials, int n_seg, int64_t n_rows, int dv, float *o, float *lse,
                           hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    // few rows and up to 1024 segments: up to four segments per thread over 16-value parts of
    // each row
    if (n_seg <= 1024 && n_rows < 1024) return launch_merge_parts(partials, n_seg, n_rows, dv, o, lse, s);
    if (dv == 64)
        hipLaunchKernelGGL(merge_hd_kernel<64>, dim3((unsigned)n_rows), dim3(64), 0, s, partials, n_seg, n_rows, o, lse);
    else if (dv == 256)
        hipLaunchKernelGGL(merge_hd_kernel<256>, dim3((unsigned)n_rows), dim3(256), 0, s, partials, n_seg, n_rows, o,
                           lse);
    else if (dv == 512)
        hipLaunchKernelGGL(merge_hd_kernel<512>, dim3((unsigned)n_rows), dim3(512), 0, s, partials, n_seg, n_rows, o,
                           lse);
    else
        return hipErrorNotSupported;
    return hipGetLastError();
}

}  // namespace rkv
