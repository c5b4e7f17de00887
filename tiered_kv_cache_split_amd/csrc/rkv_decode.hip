// Vector (VALU) segment kernel for decode and unified-pool attention on gfx950.
//
// What a segment computes (opencoti-llamafile patch 0070-rolling-kv, fattn.cu
// streaming_lse_kernel and the tail-partial op): for every output row, over the keys of
// the segment, M = max s_j, S = sum exp(s_j - M), VKQ = sum exp(s_j - M) v_j with
// s_j = scale*<q, k_j> + mask_j; a -inf key contributes nothing.  Rows of one KV head
// (the gqa query heads times the n_q queries) are computed together so every K/V byte
// is read from HBM once.
//
// Work is split over cells (split-K); a wave processes 64-cell chunks of one KV head:
//   1. the chunk's raw K and V bytes (f16 or quant blocks) are fetched with coalesced loads
//      into registers one chunk ahead, then stored to LDS;
//   2. lane c takes cell c: Q.K for all rows with v_dot2_f32_f16 (q8_0 codes enter as
//      exact binary16 integers built by a byte permute, their bias removed per block);
//   3. online softmax in the exp2 domain with DPP / permlane wave reductions;
//   4. P.V with lanes over head_dim, two cells per v_dot2 with f16 weights (q4_0 nibbles
//      enter as exact binary16 integers, the block scale folded into the weight);
//   5. after the last chunk the lane groups are folded and the partial is written.
// Two kernels share this per-wave routine: a per-head kernel for any layout and for
// gathered rows, and a cell-major kernel in which a workgroup owns all KV heads of a cell
// range and reads every chunk as one contiguous span (the cache layout of the pages).
#include "rkv.h"
#include "rkv_internal.h"
#include "rkv_unpack.h"
#include "rkv_wave.h"

#include <math.h>

#include <algorithm>

namespace rkv {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Orders this wave's LDS accesses (each wave owns its LDS region; no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }

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
// already are.  q4_0 V rows are read by 16-lane groups and need no padding.
template <int T> constexpr int k_lds_stride() { return T == T_F16 ? 272 : RowFmt<T>::kRow; }

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

// Weight-table slot of cell c.  q4_0 V and LDS-staged binary16 V: P.V pairs cells (c, c+1).
// Binary16 V kept in registers in fetch order: pairs (c, c+4) of each group of 8, stored
// next to each other.
template <bool PAIR_ADJ>
__device__ __forceinline__ int wslot(int c) {
    if constexpr (PAIR_ADJ) return c;
    return 8 * (c >> 3) + 2 * (c & 3) + ((c >> 2) & 1);
}

// q8_0 codes enter v_dot2 as 1152 + q (kQ8Bias); q4_0 nibbles as 1024 + n = kQ4BiasLo + (n - 8)
constexpr float kQ4Bias = kQ4BiasLo;

template <int VT> constexpr int n_wblocks() { return VT == T_Q4_0 ? 4 : 1; }

// Q is read through the constant address space: uniform scalar loads into SGPRs.
typedef const __attribute__((address_space(4))) uint32_t cu32;

// Additive log2-domain term of this lane's cell for every row: the mask, the causal rule and
// cell validity (-inf hides).  Read before the next chunk's loads are issued, so waiting for
// the mask never waits for the prefetch.
template <int R>
__device__ __forceinline__ void score_terms(const SegParams &p, const int (&qi)[R], int b, int64_t cell, bool valid,
                                            float (&xadd)[R]) {
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        float x = valid ? 0.f : -INFINITY;
        if (valid && p.mask) {
            const _Float16 mv = p.mask[p.pos0 + cell + (int64_t)qi[rho] * p.m_s1 + (int64_t)b * p.m_s3];
            x += (float)mv * kLog2e;
        }
        if (p.q_pos0 >= 0 && p.pos0 + cell > p.q_pos0 + qi[rho]) x = -INFINITY;
        xadd[rho] = x;
    }
}

// One chunk of 64 cells for the R rows of one KV head, by one wave:
//   Q.K with lane = cell (the lane's K row `krow` in LDS, Q rows `qw` read by scalar loads,
//   q8_0 codes as exact 1024 + (q + 128) halves with the bias removed through `qsum` [R][4]),
//   online softmax in the exp2 domain with f16 weights written to `wtab` [R][NB][64],
//   then P.V with lanes over head_dim, two cells per v_dot2.  V rows come from LDS
//   (VLDS: row c at vbase + c*vstride) or, for binary16 V, from registers in fetch order.
template <int KT, int VT, int R, bool VLDS>
__device__ __forceinline__ void process_chunk(const uint8_t *krow, const uint8_t *vbase, int vstride,
                                              const typename RowFmt<VT>::U *vreg, const uint32_t *const (&qw)[R],
                                              const float *qsum, _Float16 *wtab, const float (&xadd)[R],
                                              float scale_log2, float cap_cs, float cap_l2, int lane,
                                              float (&m)[R], float (&l)[R],
                                              float (&acc)[R][8], float (&sw)[R][n_wblocks<VT>()]) {
    constexpr bool kVq = (VT == T_Q4_0);
    constexpr int kNB = n_wblocks<VT>();
    constexpr bool kAdj = kVq || VLDS;
    const int grp = lane >> 4, kk = lane & 15;

    // ---- Q.K, lane = cell.  The lane's K row is read from LDS first; then Q comes in half rows
    // (32 words) by scalar loads and feeds v_dot2 as SGPR operands, so no LDS bandwidth is
    // spent broadcasting Q.  Each half-row pointer depends on the previous half's score, so
    // only one half row is held in SGPRs at a time.
    float s[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) s[rho] = 0.f;
    if constexpr (KT == T_Q8_0) {
        uint32_t w[34];
#pragma unroll
        for (int j = 0; j < 17; ++j) {
            const uint2 x = *reinterpret_cast<const uint2 *>(krow + 8 * j);
            w[2 * j] = x.x;
            w[2 * j + 1] = x.y;
        }
        float dep = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            half2_t a[16], c[16];
            float dk[2];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int blk = 2 * hb + bb, base = 34 * blk;
                dk[bb] = h2f((base & 3) ? (w[base >> 2] >> 16) : w[base >> 2]);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int off = base + 2 + 4 * t;  // codes of block blk, bytes off .. off+3
                    const uint32_t x = (off & 3) ? __builtin_amdgcn_alignbyte(w[(off >> 2) + 1], w[off >> 2], off & 3)
                                                 : w[off >> 2];
                    const uint2 bq = q8_biased(x);  // 1152 + q per code, exact
                    a[8 * bb + t] = as_h2(bq.x);
                    c[8 * bb + t] = as_h2(bq.y);
                }
            }
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                cu32 *qb = (cu32 *)(qw[rho] + 32 * hb);
                asm volatile("" : "+s"(qb) : "v"(dep));
                float d0 = 0.f, d1 = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    d0 = __builtin_amdgcn_fdot2(a[t], as_h2(qb[2 * t]), d0, false);
                    d0 = __builtin_amdgcn_fdot2(c[t], as_h2(qb[2 * t + 1]), d0, false);
                    d1 = __builtin_amdgcn_fdot2(a[8 + t], as_h2(qb[16 + 2 * t]), d1, false);
                    d1 = __builtin_amdgcn_fdot2(c[8 + t], as_h2(qb[16 + 2 * t + 1]), d1, false);
                }
                // sum_t (1152 + q_t) Q_t - 1152 sum_t Q_t = sum_t q_t Q_t, per 32-value block
                s[rho] = fmaf(dk[0], fmaf(-kQ8Bias, qsum[rho * 4 + 2 * hb], d0), s[rho]);
                s[rho] = fmaf(dk[1], fmaf(-kQ8Bias, qsum[rho * 4 + 2 * hb + 1], d1), s[rho]);
                dep = s[rho];
            }
        }
    } else {
        const uint4 *kr = reinterpret_cast<const uint4 *>(krow);
        uint4 x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = kr[j];
        float dep = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                cu32 *qb = (cu32 *)(qw[rho] + 32 * hb);
                asm volatile("" : "+s"(qb) : "v"(dep));
                float d0 = s[rho], d1 = 0.f;
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const uint4 x0 = x[8 * hb + j], x1 = x[8 * hb + j + 1];
                    d0 = __builtin_amdgcn_fdot2(as_h2(x0.x), as_h2(qb[4 * j + 0]), d0, false);
                    d0 = __builtin_amdgcn_fdot2(as_h2(x0.y), as_h2(qb[4 * j + 1]), d0, false);
                    d0 = __builtin_amdgcn_fdot2(as_h2(x0.z), as_h2(qb[4 * j + 2]), d0, false);
                    d0 = __builtin_amdgcn_fdot2(as_h2(x0.w), as_h2(qb[4 * j + 3]), d0, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x1.x), as_h2(qb[4 * j + 4]), d1, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x1.y), as_h2(qb[4 * j + 5]), d1, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x1.z), as_h2(qb[4 * j + 6]), d1, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x1.w), as_h2(qb[4 * j + 7]), d1, false);
                }
                s[rho] = d0 + d1;
                dep = s[rho];
            }
        }
    }

    // ---- online softmax (exp2 domain), f16 weights into the chunk table
    float dvs[kNB];
    if constexpr (kVq) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dvs[j] = h2f(ld_u16(vbase + lane * vstride + 18 * j));
    } else {
        dvs[0] = 1.f;
    }
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const float x = cap_l2 != 0.f ? softcap_log2(s[rho], cap_cs, cap_l2) + xadd[rho] : fmaf(s[rho], scale_log2, xadd[rho]);
        const float mn = fmaxf(m[rho], wave_max(x));
        float pr = 0.f;
        if (mn != -INFINITY) {
            if (mn > m[rho]) {  // uniform: rescale what this wave has accumulated so far
                const float alpha = __builtin_amdgcn_exp2f(m[rho] - mn);
                l[rho] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[rho][e] *= alpha;
#pragma unroll
                for (int j = 0; j < kNB; ++j) sw[rho][j] *= alpha;
                m[rho] = mn;
            }
            pr = __builtin_amdgcn_exp2f(x - mn);
            l[rho] += pr;
        }
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const _Float16 wh = (_Float16)(pr * dvs[j]);
            wtab[(rho * kNB + j) * kChunk + wslot<kAdj>(lane)] = wh;
            if constexpr (kVq) sw[rho][j] += (float)wh;
        }
    }
    wave_sync();

    // ---- P.V: lanes over head_dim, eight values per lane; each step pairs two cells in
    // v_dot2 with their f16 weights
#pragma unroll
    for (int st = 0; st < kChunk / 8; ++st) {
        const int pd = 4 * st + grp;  // weight pair (dword) of this step
        if constexpr (kVq) {
            const int blk = kk >> 2, j4 = kk & 3;
            const int c0r = 8 * st + 2 * grp;
            const uint8_t *r0 = vbase + c0r * vstride + 18 * blk + 2 + 4 * j4;
            const uint8_t *r1 = r0 + vstride;
            const uint32_t x0 = ld_u16(r0) | (ld_u16(r0 + 2) << 16);
            const uint32_t x1 = ld_u16(r1) | (ld_u16(r1 + 2) << 16);
            const uint32_t lo0 = x0 & 0x0F0F0F0Fu, lo1 = x1 & 0x0F0F0F0Fu;
            const uint32_t hi0 = (x0 >> 4) & 0x0F0F0F0Fu, hi1 = (x1 >> 4) & 0x0F0F0F0Fu;
            half2_t pl[4], ph[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                pl[t] = as_h2(q4_pair_biased(lo0, lo1, t));  // 1024+n(c0), 1024+n(c1)
                ph[t] = as_h2(q4_pair_biased(hi0, hi1, t));
            }
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                const half2_t wp = as_h2(reinterpret_cast<const uint32_t *>(wtab + (rho * kNB + blk) * kChunk)[pd]);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    acc[rho][t] = __builtin_amdgcn_fdot2(pl[t], wp, acc[rho][t], false);
                    acc[rho][4 + t] = __builtin_amdgcn_fdot2(ph[t], wp, acc[rho][4 + t], false);
                }
            }
        } else {
            uint4 u0, u1;  // binary16 V of the step's two cells, this lane's 16 bytes
            if constexpr (VLDS) {
                const int c0r = 8 * st + 2 * grp;
                u0 = *reinterpret_cast<const uint4 *>(vbase + c0r * vstride + 16 * kk);
                u1 = *reinterpret_cast<const uint4 *>(vbase + (c0r + 1) * vstride + 16 * kk);
            } else {
                u0 = vreg[2 * st];  // cells 8st+grp and 8st+4+grp
                u1 = vreg[2 * st + 1];
            }
            const uint32_t a0[4] = {u0.x, u0.y, u0.z, u0.w}, a1[4] = {u1.x, u1.y, u1.z, u1.w};
            half2_t ev[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ev[2 * j] = as_h2(__builtin_amdgcn_perm(a1[j], a0[j], 0x05040100u));
                ev[2 * j + 1] = as_h2(__builtin_amdgcn_perm(a1[j], a0[j], 0x07060302u));
            }
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                const half2_t wp = as_h2(reinterpret_cast<const uint32_t *>(wtab + rho * kChunk)[pd]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[rho][e] = __builtin_amdgcn_fdot2(ev[e], wp, acc[rho][e], false);
            }
        }
    }
}

// End of a wave's cells: fold the four 16-lane groups, reduce the row sums, remove the q4_0
// offset.  Afterwards lanes 0..15 hold the wave's VKQ values in the lane's element order.
template <int VT, int R>
__device__ __forceinline__ void finish_wave(int lane, float (&l)[R], float (&acc)[R][8],
                                            float (&sw)[R][n_wblocks<VT>()]) {
    const int kk = lane & 15;
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rho][e] = fold_rows(acc[rho][e]);
        l[rho] = wave_sum(l[rho]);
        if constexpr (VT == T_Q4_0) {
            const int blk = kk >> 2;
            float corr = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float t = wave_sum(sw[rho][j]);
                corr = (blk == j) ? t : corr;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[rho][e] = fmaf(-kQ4Bias, corr, acc[rho][e]);
        }
    }
}

// Element index held in acc[.][e] by lane kk (0..15) after finish_wave.
template <int VT>
__device__ __forceinline__ int elem_of(int kk, int e) {
    if constexpr (VT == T_Q4_0) {
        const int blk = kk >> 2, j4 = kk & 3;
        return 32 * blk + 4 * j4 + (e & 3) + ((e >> 2) << 4);
    }
    return 8 * kk + e;
}

// Q rows of KV head g (rho = i*gqa + r: query i, head g*gqa + r) and, for q8_0 K, the sums of
// their 32-value blocks.
template <int R>
__device__ __forceinline__ void q_rows(const SegParams &p, int g, int b, const uint32_t *(&qw)[R], int (&qi)[R]) {
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const int r = rho % p.gqa, i = rho / p.gqa;
        qw[rho] = reinterpret_cast<const uint32_t *>(p.q + (int64_t)i * p.q_s1 + (int64_t)(g * p.gqa + r) * p.q_s2 +
                                                      (int64_t)b * p.q_s3);
        qi[rho] = i;
    }
}
template <int R>
__device__ __forceinline__ void q_block_sums(const SegParams &p, int g, int b, float *qsum, int idx) {
    // idx in [0, 4R): sum of the 32 Q values of block idx&3 of row idx>>2
    const int rho = idx >> 2, blk = idx & 3, r = rho % p.gqa, i = rho / p.gqa;
    const _Float16 *qp = p.q + (int64_t)i * p.q_s1 + (int64_t)(g * p.gqa + r) * p.q_s2 + (int64_t)b * p.q_s3 + 32 * blk;
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 32; ++t) acc += (float)qp[t];
    qsum[idx] = acc;
}

// ============================================================================ per-head kernel
// Any layout and gathered rows.  Workgroup = 4 waves for one (split, KV head, sequence);
// each wave walks every 4th 64-cell chunk with its own LDS region, K (and q4_0 V) rows
// fetched one chunk ahead into registers and stored to LDS; the waves' results are merged
// through LDS at the end.
constexpr int kWaves = 4;

template <int KT, int VT, int R, bool ROWS>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
decode_seg_kernel(const SegParams p) {
    using KF = RowFmt<KT>;
    using VF = RowFmt<VT>;
    constexpr bool kVq = (VT == T_Q4_0);  // q4_0 V goes through LDS; binary16 V is used in registers
    constexpr int kNB = n_wblocks<VT>();
    constexpr int kKs = k_lds_stride<KT>();
    constexpr int kVs = RowFmt<VT>::kRow;
    __shared__ __attribute__((aligned(16))) uint8_t s_k[kWaves][kChunk * kKs];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kWaves][kVq ? kChunk * kVs : 16];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[kWaves][R * kNB * kChunk];
    __shared__ float s_qsum[R * 4];

    // the wave index is uniform per wave: say so, so chunk bases and descriptors stay scalar
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    int bid = blockIdx.x;
    const int split = bid % p.n_splits;
    bid /= p.n_splits;
    const int g = bid % p.n_head_kv;
    const int b = bid / p.n_head_kv;

    const int64_t c_beg = (int64_t)split * p.cells_per_split;
    const int64_t c_end = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    const uint8_t *kbase = p.k + (int64_t)g * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)g * p.v_s2;
    const int32_t *rows = ROWS ? p.rows + (int64_t)b * p.rows_s : nullptr;

    const uint32_t *qw[R];
    int qi[R];
    q_rows<R>(p, g, b, qw, qi);
    if constexpr (KT == T_Q8_0) {
        if (tid < R * 4) q_block_sums<R>(p, g, b, s_qsum, tid);
        __syncthreads();
    }

    float m[R], l[R], acc[R][8], sw[R][kNB];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        m[rho] = -INFINITY;
        l[rho] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rho][e] = 0.f;
#pragma unroll
        for (int j = 0; j < kNB; ++j) sw[rho][j] = 0.f;
    }

    typename KF::U kb[KF::kMain + KF::kTail];
    typename VF::U vb[VF::kMain + VF::kTail];

    // Row (cell or pool row) of this lane's cell in the chunk starting at c0, -1 if none (a
    // list entry outside the pool is none too).
    auto row_of = [&](int64_t c0) -> int {
        const int64_t c = c0 + lane;
        if (c >= c_end) return -1;
        if constexpr (ROWS) {
            const int r = rows[c];
            return (r >= 0 && (int64_t)r < p.n_pool) ? r : -1;
        }
        return (int)c;
    };
    auto nvalid = [&](int64_t c0) { return max((int64_t)0, min((int64_t)kChunk, c_end - c0)); };

    uint8_t *lk = s_k[wave];
    uint8_t *lv = s_v[wave];
    const int64_t n_ch = (c_end > c_beg) ? (c_end - c_beg + kChunk - 1) / kChunk : 0;
    // K rows are fetched one chunk ahead, except when both K and V are binary16: V then sits in
    // registers during Q.K, and holding the next chunk's K as well would spill
    constexpr bool kPrefetchK = kVq || KT != T_F16;
    int myrow = -1;
    if (kPrefetchK && wave < n_ch) {
        const int64_t c0 = c_beg + (int64_t)wave * kChunk;
        myrow = row_of(c0);
        fetch_rows<KT, ROWS>(kb, kbase, p.k_s1, c0, nvalid(c0), myrow, lane);
        if constexpr (kVq) fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, c0, nvalid(c0), myrow, lane);
    }

    for (int64_t ch = wave; ch < n_ch; ch += kWaves) {
        const int64_t c0 = c_beg + ch * kChunk;
        if constexpr (!kPrefetchK) {
            myrow = row_of(c0);
            fetch_rows<KT, ROWS>(kb, kbase, p.k_s1, c0, nvalid(c0), myrow, lane);
        }
        const int cur_row = myrow;
        // a chunk of gathered rows that is all padding contributes nothing (uniform per wave)
        const bool any = !ROWS || __builtin_amdgcn_ballot_w64(cur_row >= 0) != 0;
        // binary16 V without K prefetch: this chunk's rows into registers, in flight during Q.K
        if constexpr (!kVq && !kPrefetchK) {
            if (any) fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, c0, nvalid(c0), cur_row, lane);
        }
        stash_rows<KT>(kb, lk, kKs, lane);
        if constexpr (kVq) stash_rows<VT>(vb, lv, kVs, lane);
        float xadd[R];
        score_terms<R>(p, qi, b, c0 + lane, cur_row >= 0, xadd);
        wave_sync();
        if constexpr (kPrefetchK) {
            // next chunk of this wave (past c_end every row is -1 / out of range: nothing is read)
            const int64_t cn = c0 + kWaves * kChunk;
            myrow = row_of(cn);
            fetch_rows<KT, ROWS>(kb, kbase, p.k_s1, cn, nvalid(cn), myrow, lane);
            if constexpr (kVq) fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, cn, nvalid(cn), myrow, lane);
            // binary16 V: this chunk's rows straight into registers, in flight during Q.K
            if constexpr (!kVq) {
                if (any) fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, c0, nvalid(c0), cur_row, lane);
            }
        }
        if (any)
            process_chunk<KT, VT, R, kVq>(lk + lane * kKs, lv, kVs, vb, qw, s_qsum, s_w[wave], xadd, p.scale_log2,
                                          p.cap_cs, p.cap_l2, lane, m, l, acc, sw);
        wave_sync();
    }
    finish_wave<VT, R>(lane, l, acc, sw);

    // ---- merge the waves of the workgroup through LDS and write the split's partial
    __syncthreads();
    float *mb = reinterpret_cast<float *>(&s_k[0][0]);  // [wave][rho][2 + 128]
    if (lane < 16) {
        const int kk = lane;
#pragma unroll
        for (int rho = 0; rho < R; ++rho) {
            float *d = mb + (wave * R + rho) * kPartialStride + 2;
#pragma unroll
            for (int e = 0; e < 8; ++e) d[elem_of<VT>(kk, e)] = acc[rho][e];
            if (lane == 0) {
                d[-2] = m[rho];
                d[-1] = l[rho];
            }
        }
    }
    __syncthreads();
    const int slot = p.slot0 + split;
    for (int idx = tid; idx < R * kHeadDim; idx += 64 * kWaves) {
        const int rho = idx / kHeadDim, e = idx % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, mb[(wv * R + rho) * kPartialStride]);
        float S = 0.f, V = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) {
                const float *src = mb + (wv * R + rho) * kPartialStride;
                const float wgt = (src[0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(src[0] - M);
                S = fmaf(src[1], wgt, S);
                V = fmaf(src[2 + e], wgt, V);
            }
        }
        const int r = rho % p.gqa, i = rho / p.gqa;
        const int64_t row = (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)slot * p.n_rows + row) * kPartialStride;
        out[2 + e] = V;
        if (e == 0) {
            out[0] = (M == -INFINITY) ? -INFINITY : M * kLn2;
            out[1] = S;
        }
    }
}

// ============================================================================ cell-major kernel
// K/V stored cell-major with the KV heads packed inside each cell (row stride nb[2] equal to
// the row size): the HW heads of a head group in one cell are one contiguous segment.
// Workgroup = HW waves for one (split, head group, sequence); wave w is KV head g0 + w.  Every
// 64-cell chunk is fetched by the whole workgroup as one contiguous span with 16-byte loads
// (one chunk ahead, in registers) and stored to LDS with a small pad per cell so that the
// one-row-per-lane K reads stay bank-conflict free; each wave then runs the Q.K / softmax /
// P.V of its head.
template <int T> constexpr int cell_pad() { return T == T_F16 ? 16 : 8; }

template <int KT, int VT, int R, int HW>
__global__ void __launch_bounds__(64 * HW) __attribute__((amdgpu_waves_per_eu(2)))
decode_cell_kernel(const SegParams p) {
    constexpr int kNB = n_wblocks<VT>();
    constexpr int kRk = RowFmt<KT>::kRow, kRv = RowFmt<VT>::kRow;  // bytes of one head row
    constexpr int kCk = HW * kRk, kCv = HW * kRv;                  // bytes of one cell (head group)
    constexpr int kSk = kCk + cell_pad<KT>(), kSv = kCv + cell_pad<VT>();  // LDS cell strides
    constexpr int kNT = 64 * HW;
    constexpr int kUk = kChunk * kCk / 16, kUv = kChunk * kCv / 16;         // 16-byte units per chunk
    constexpr int kLk = (kUk + kNT - 1) / kNT, kLv = (kUv + kNT - 1) / kNT;  // units per thread
    static_assert(kCk % 16 == 0 && kCv % 16 == 0, "cell segments must be whole 16-byte units");
    __shared__ __attribute__((aligned(16))) uint8_t s_k[kChunk * kSk];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kChunk * kSv];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[HW][R * kNB * kChunk];
    __shared__ float s_qsum[HW][R * 4];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int n_hgrp = p.n_head_kv / HW;
    int bid = blockIdx.x;
    const int split = bid % p.n_splits;
    bid /= p.n_splits;
    const int hgrp = bid % n_hgrp;
    const int b = bid / n_hgrp;
    const int g = hgrp * HW + wave;  // this wave's KV head
    const int64_t c_beg = (int64_t)split * p.cells_per_split;
    const int64_t c_end = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    const uint8_t *kbase = p.k + (int64_t)(hgrp * HW) * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)(hgrp * HW) * p.v_s2;

    const uint32_t *qw[R];
    int qi[R];
    q_rows<R>(p, g, b, qw, qi);
    if constexpr (KT == T_Q8_0) {
        if (lane < R * 4) q_block_sums<R>(p, g, b, s_qsum[wave], lane);
    }
    wave_sync();

    float m[R], l[R], acc[R][8], sw[R][kNB];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        m[rho] = -INFINITY;
        l[rho] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rho][e] = 0.f;
#pragma unroll
        for (int j = 0; j < kNB; ++j) sw[rho][j] = 0.f;
    }

    // per-thread 16-byte units: chunk-relative global offsets (by cell stride) and LDS offsets (padded)
    int gk[kLk], lk[kLk], gv[kLv], lv[kLv];
#pragma unroll
    for (int i = 0; i < kLk; ++i) {
        const int u = tid + kNT * i, cell = u / (kCk / 16), w = u % (kCk / 16);
        gk[i] = (u < kUk) ? cell * (int)p.k_s1 + 16 * w : 0x7FFFFFF0;
        lk[i] = cell * kSk + 16 * w;
    }
#pragma unroll
    for (int i = 0; i < kLv; ++i) {
        const int u = tid + kNT * i, cell = u / (kCv / 16), w = u % (kCv / 16);
        gv[i] = (u < kUv) ? cell * (int)p.v_s1 + 16 * w : 0x7FFFFFF0;
        lv[i] = cell * kSv + 16 * w;
    }
    uint4 kb[kLk], vb[kLv];
    auto fetch = [&](int64_t c0) {
        const int64_t nv = max((int64_t)0, min((int64_t)kChunk, c_end - c0));
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + c0 * p.k_s1), (short)0, (int)(nv * p.k_s1), 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + c0 * p.v_s1), (short)0, (int)(nv * p.v_s1), 0x00020000);
#pragma unroll
        for (int i = 0; i < kLk; ++i) kb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, gk[i], 0, 0));
#pragma unroll
        for (int i = 0; i < kLv; ++i) vb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, gv[i], 0, 0));
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < kLk; ++i) {
            if (kLk * kNT == kUk || tid + kNT * i < kUk) {
                uint2 *d = reinterpret_cast<uint2 *>(s_k + lk[i]);
                d[0] = make_uint2(kb[i].x, kb[i].y);
                d[1] = make_uint2(kb[i].z, kb[i].w);
            }
        }
#pragma unroll
        for (int i = 0; i < kLv; ++i) {
            if (kLv * kNT == kUv || tid + kNT * i < kUv) {
                uint2 *d = reinterpret_cast<uint2 *>(s_v + lv[i]);
                d[0] = make_uint2(vb[i].x, vb[i].y);
                d[1] = make_uint2(vb[i].z, vb[i].w);
            }
        }
    };

    const int64_t n_ch = (c_end > c_beg) ? (c_end - c_beg + kChunk - 1) / kChunk : 0;
    if (n_ch > 0) fetch(c_beg);
    for (int64_t ch = 0; ch < n_ch; ++ch) {
        const int64_t c0 = c_beg + ch * kChunk;
        __syncthreads();  // every wave is done with the previous chunk's LDS
        stash();
        float xadd[R];
        score_terms<R>(p, qi, b, c0 + lane, c0 + lane < c_end, xadd);
        __syncthreads();
        fetch(c0 + kChunk);  // past c_end nothing is read
        process_chunk<KT, VT, R, true>(s_k + lane * kSk + wave * kRk, s_v + wave * kRv, kSv, nullptr, qw,
                                       s_qsum[wave], s_w[wave], xadd, p.scale_log2, p.cap_cs, p.cap_l2, lane, m, l,
                                       acc, sw);
    }
    finish_wave<VT, R>(lane, l, acc, sw);

    // ---- each wave writes the partial of its KV head
    const int slot = p.slot0 + split;
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const int r = rho % p.gqa, i = rho / p.gqa;
        const int64_t row = (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)slot * p.n_rows + row) * kPartialStride;
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) out[2 + elem_of<VT>(lane, e)] = acc[rho][e];
        }
        if (lane == 0) {
            out[0] = (m[rho] == -INFINITY) ? -INFINITY : m[rho] * kLn2;
            out[1] = l[rho];
        }
    }
}

template <int KT, int VT, int R, int HW>
hipError_t launch_cell(const SegParams &p, hipStream_t s, int *occupancy) {
    if (occupancy)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, decode_cell_kernel<KT, VT, R, HW>, 64 * HW, 0);
    launch_seg(decode_cell_kernel<KT, VT, R, HW>, dim3((unsigned)(p.n_splits * (p.n_head_kv / HW) * p.n_seq)),
               dim3(64 * HW), s, p);
    return hipGetLastError();
}

template <int KT, int VT, int R>
hipError_t launch_decode_r(const SegParams &p, hipStream_t s, int *occupancy) {
    if (p.cell_hw > 0) {
        // (q8_0 / q4_0 cell groups go to the matrix-core kernel before the rows are dispatched)
        if constexpr (KT == T_F16 && VT == T_F16) {
            if (decode_mma16_ok(p)) return launch_decode_mma16(p, s, occupancy);
            if (p.cell_hw == 2 && p.d == kHeadDim) return launch_cell<KT, VT, R, 2>(p, s, occupancy);
        }
        return hipErrorInvalidValue;
    }
    if (occupancy) return hipErrorInvalidValue;
    // with q8_0 K and 6 or more rows per KV head the per-head kernel's register arrays spill;
    // the kernel for the other head dims (instantiated at 128, rows in groups of 8) does not
    if constexpr (KT == T_Q8_0 && R >= 6) {
        return launch_decode_hd(p, KT, VT, s);
    } else {
        const int64_t blocks = (int64_t)p.n_splits * p.n_head_kv * p.n_seq;
        if (p.rows)
            launch_seg(decode_seg_kernel<KT, VT, R, true>, dim3((unsigned)blocks), dim3(64 * kWaves), s, p);
        else
            launch_seg(decode_seg_kernel<KT, VT, R, false>, dim3((unsigned)blocks), dim3(64 * kWaves), s, p);
        return hipGetLastError();
    }
}

template <int KT, int VT>
hipError_t launch_decode_t(const SegParams &p, int R, hipStream_t s, int *occupancy) {
    switch (R) {
        case 1: return launch_decode_r<KT, VT, 1>(p, s, occupancy);
        case 2: return launch_decode_r<KT, VT, 2>(p, s, occupancy);
        case 3: return launch_decode_r<KT, VT, 3>(p, s, occupancy);
        case 4: return launch_decode_r<KT, VT, 4>(p, s, occupancy);
        case 5: return launch_decode_r<KT, VT, 5>(p, s, occupancy);
        case 6: return launch_decode_r<KT, VT, 6>(p, s, occupancy);
        case 7: return launch_decode_r<KT, VT, 7>(p, s, occupancy);
        case 8: return launch_decode_r<KT, VT, 8>(p, s, occupancy);
        default: return hipErrorInvalidValue;
    }
}

hipError_t dispatch_decode(const SegParams &p, int k_type, int v_type, hipStream_t s, int *occupancy) {
    const int R = p.gqa * p.n_q;
    // cell groups of q8_0 / q4_0 heads: the matrix-core kernel, any number of rows at head dims
    // other than 128 (row groups of 16)
    if (p.cell_hw > 0 && k_type == T_Q8_0 && v_type == T_Q4_0)
        return decode_mma_ok(p) ? launch_decode_mma(p, s, occupancy) : hipErrorInvalidValue;
    if (k_type == T_Q8_0 && v_type == T_Q4_0) return launch_decode_t<T_Q8_0, T_Q4_0>(p, R, s, occupancy);
    // binary16 cell groups: the matrix-core kernel for any number of rows it takes
    if (p.cell_hw > 0 && k_type == T_F16 && v_type == T_F16 && decode_mma16_ok(p))
        return launch_decode_mma16(p, s, occupancy);
    if (k_type == T_F16 && v_type == T_F16) return launch_decode_t<T_F16, T_F16>(p, R, s, occupancy);
    if (k_type == T_Q8_0 && v_type == T_F16) return launch_decode_t<T_Q8_0, T_F16>(p, R, s, occupancy);
    if (k_type == T_F16 && v_type == T_Q4_0) return launch_decode_t<T_F16, T_Q4_0>(p, R, s, occupancy);
    return hipErrorInvalidValue;
}

}  // namespace

int cell_heads(int dk, int dv, int k_type, int v_type, int n_head_kv, int R, bool rows) {
    if (R < 1) return 0;
    // q8_0 / q4_0: the matrix-core kernel at head dims 64 .. 512 and 576 / 512, over segments
    // and row lists (up to 8 rows per KV head at 128, any number at the other head dims)
    if (k_type == T_Q8_0 && v_type == T_Q4_0)
        return (dk == kHeadDim && R > kMaxRowsVec) ? 0 : decode_mma_heads(dk, dv, n_head_kv, R);
    // binary16 in cell groups (8 KV heads at 64 and 128, 4 at 256, 2 at 512, 1 at 576 / 512):
    // the matrix-core kernel -- persistent up to 8 rows per KV head (also for row lists), in row
    // groups of 16 over segments beyond that (head dims other than 128)
    if (k_type == T_F16 && v_type == T_F16 && (R <= kMaxRowsVec || (!rows && dk != kHeadDim))) {
        const int hw = decode_mma16_heads(dk, dv);
        if (hw > 0 && n_head_kv % hw == 0) return hw;
    }
    if (dk != kHeadDim || dv != kHeadDim || R > kMaxRowsVec) return 0;
    if (rows) return 0;  // other gathered rows: per-head kernel
    if (k_type == T_F16 && v_type == T_F16) return n_head_kv % 2 == 0 ? 2 : 0;
    return 0;
}

int cell_blocks_per_cu(const SegParams &p, int k_type, int v_type) {
    int n = 0;
    if (p.cell_hw <= 0 || dispatch_decode(p, k_type, v_type, nullptr, &n) != hipSuccess || n < 1) return 1;
    return n;
}

bool decode_kernel_persistent(const SegParams &p, int k_type, int v_type) {
    return p.cell_hw > 0 && k_type == T_F16 && v_type == T_F16 && p.gqa * p.n_q <= kMaxRowsVec && decode_mma16_ok(p);
}

int cell_row_groups(const SegParams &p, int k_type, int v_type) {
    if (k_type == T_Q8_0 && v_type == T_Q4_0) return decode_mma_row_groups(p);
    const int R = p.gqa * p.n_q;
    return R > kMaxRowsVec ? (R + 15) / 16 : 1;  // binary16: row groups of 16 beyond 8 rows
}

int decode_kernel_variant(const SegParams &p, int k_type, int v_type) {
    if (p.d != kHeadDim) {
        if (p.cell_hw > 0 && k_type == T_Q8_0 && v_type == T_Q4_0 && decode_mma_ok(p)) return RKV_KERNEL_DECODE_CELL_MFMA;
        if (p.cell_hw > 0 && k_type == T_F16 && v_type == T_F16 && decode_mma16_ok(p))
            return RKV_KERNEL_DECODE_CELL_MFMA16;
        return RKV_KERNEL_DECODE_HD;
    }
    if (p.cell_hw <= 0) return (k_type == T_Q8_0 && p.gqa * p.n_q >= 6) ? RKV_KERNEL_DECODE_HD : RKV_KERNEL_DECODE_HEAD;
    if (k_type == T_Q8_0 && v_type == T_Q4_0 && decode_mma_ok(p)) return RKV_KERNEL_DECODE_CELL_MFMA;
    if (k_type == T_F16 && v_type == T_F16 && decode_mma16_ok(p)) return RKV_KERNEL_DECODE_CELL_MFMA16;
    return RKV_KERNEL_DECODE_CELL;
}

hipError_t launch_decode_segment(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (p.d != kHeadDim && p.cell_hw <= 0) return launch_decode_hd(p, k_type, v_type, s);
    return dispatch_decode(p, k_type, v_type, s, nullptr);
}

}  // namespace rkv
