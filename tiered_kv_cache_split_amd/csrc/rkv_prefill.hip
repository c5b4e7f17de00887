// MFMA segment kernel for prefill on gfx950: many query rows per KV head, so Q.K^T and P.V
// are dense contractions and run on the matrix cores (v_mfma_f32_32x32x16_f16).
//
// What a segment computes is the same partial as the decode kernels (opencoti-llamafile patch
// 0070-rolling-kv, tail-partial op and fattn.cu streaming_lse_kernel): per output row, over
// the keys of the segment, M = max s_j, S = sum exp(s_j - M), VKQ = sum exp(s_j - M) v_j,
// s_j = scale*<q, k_j> + mask_j, keys at positions after the query's own (causal) or with a
// -inf mask contributing nothing.
//
// Workgroup = 8 waves = 256 query rows of one KV head (row rho = i*gqa + r: query i, head
// g*gqa + r) over one split of the segment's keys, 64 keys per tile.  Operands are exact:
//   K  rows [key][d] in LDS as binary16: copied, or for q8_0 the two-part sum hi + lo = d*q
//      (both binary16, exact), so S^T = K.Q^T takes two MFMAs per step for q8_0;
//   V  rows [key][d] in LDS as binary16: copied, or for q4_0 the exact integers n - 8, with the
//      block scales d_V kept apart and folded into the binary16 weights of P.V
//      (W = p * d_V per key and 32-value block: each 32-row output tile of O^T is one block).
// The waves split into two groups of four (one wave of each per SIMD).  Each group alternates
// a matrix phase (P.V of the previous tile, then Q.K of this tile) and a vector phase (online
// softmax of this tile, and its share of the next tile's operand decode: group 0 decodes K,
// group 1 decodes V, each straight from raw bytes it fetched two tiles ahead into registers).
// Group 1 runs one phase behind group 0, so on every SIMD one wave feeds the matrix core while
// the other keeps the vector unit busy; a workgroup barrier ends every phase.
#include "rkv_internal.h"
#include "rkv_unpack.h"
#include "rkv_wave.h"

#include <math.h>

#include <type_traits>

namespace rkv {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f16x_t __attribute__((ext_vector_type(16)));

constexpr int kWavesP = 8;
constexpr int kThreadsP = 64 * kWavesP;
constexpr int kGroupT = kThreadsP / 2;  // threads per wave group
constexpr int kBM = 32 * kWavesP;       // query rows per workgroup
constexpr int kBN = 64;                 // keys per tile
// LDS bytes per K row: D binary16 + 16 (16 rows of a 16-byte read fall on distinct banks)
template <int D> constexpr int k_pitch() { return 2 * D + 16; }
// LDS bytes per V row: D binary16 + 64 (the transposing reads' rows spread over the banks)
template <int D> constexpr int v_pitch() { return 2 * D + 64; }
constexpr int kPD = 4;                  // P.V steps whose operand reads run ahead of the current one
constexpr int kKD = 4;                  // Q.K steps likewise
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;

template <int D, int T> constexpr int row_bytes_of() { return T == T_F16 ? 2 * D : (T == T_Q8_0 ? 34 : 18) * (D / 32); }
// 32-bit words a thread fetches for its part of a row (one block of 32 values, or 64 bytes of
// binary16): a q8_0 block is 34 bytes from an even offset (9 words cover it), a q4_0 block 18
// bytes (5 words)
template <int T> constexpr int raw_words() { return T == T_F16 ? 16 : (T == T_Q8_0 ? 9 : 5); }

// LDS layout (bytes): two K buffers (binary16 hi rows, for q8_0 also the lo rows), then two V
// buffers (binary16 rows, for q4_0 followed by d_V as [block][key slot]).
template <int D, int KT, int VT> struct Lds {
    static constexpr int kKhalf = kBN * k_pitch<D>();
    static constexpr int kKbuf = kKhalf * (KT == T_Q8_0 ? 2 : 1);
    static constexpr int kVdat = kBN * v_pitch<D>();
    static constexpr int kVbuf = kVdat + (VT == T_Q4_0 ? (D / 32) * kBN * 2 : 0);
    static constexpr int kV0 = 2 * kKbuf;
    static constexpr int kSize = 2 * kKbuf + 2 * kVbuf;
};

// Slot of key k (0..63) within its 16-key P.V step: the order in which the binary16 P fragments
// built from the S^T accumulators hold keys (bits 2 and 3 of the in-step index swapped).
__device__ __forceinline__ int pv_slot(int k) { return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ float lane_pair_max(float x) {
    const int xi = __builtin_bit_cast(int, x);
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float lane_pair_sum(float x) {
    const int xi = __builtin_bit_cast(int, x);
    const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

// Buffer resource over the valid rows of a tile (rows past the segment end read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t *base, int64_t s1, int64_t nv, int rb) {
    const int range = nv > 0 ? (int)((nv - 1) * s1 + rb) : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, range, 0x00020000);
}

// Fetch the thread's part (32 values) of a tile key's row: the block's bytes from its
// word-aligned start (q8_0 / q4_0 blocks start 0 or 2 bytes into a word).
template <int T>
__device__ __forceinline__ void fetch_part(uint32_t (&w)[16], __amdgpu_buffer_rsrc_t rs, int off) {
    if constexpr (T == T_F16) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * m, 0, 0));
            w[4 * m] = x.x, w[4 * m + 1] = x.y, w[4 * m + 2] = x.z, w[4 * m + 3] = x.w;
        }
    } else if constexpr (T == T_Q8_0) {
        const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        const uint4 b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
        w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w, w[4] = b.x, w[5] = b.y, w[6] = b.z, w[7] = b.w;
        w[8] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 32, 0, 0);
    } else {
        const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w;
        w[4] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 16, 0, 0);
    }
}

// K row part -> LDS: binary16 copy, or a q8_0 block as exact hi / lo binary16 rows.
// `odd`: the block starts 2 bytes into its first word (its scale is that word's high half).
template <int KT>
__device__ __forceinline__ void decode_k_part(const uint32_t (&w)[16], bool odd, uint8_t *khi, uint8_t *klo) {
    uint4 *dh = reinterpret_cast<uint4 *>(khi);
    if constexpr (KT == T_F16) {
#pragma unroll
        for (int m = 0; m < 4; ++m) dh[m] = make_uint4(w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]);
    } else {
        const uint32_t dbits = odd ? (w[0] >> 16) : (w[0] & 0xFFFFu);
        const uhalf2_t dd = u2h(dbits | (dbits << 16));
        const uint32_t sel = odd ? 0x07060504u : 0x05040302u;  // codes start at byte 4 or 2
        uint32_t hi[16], lo[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint2 b = q8_biased(__builtin_amdgcn_perm(w[i + 1], w[i], sel));
            q8_hi_lo(q8_unbias(b.x), dd, hi[2 * i], lo[2 * i]);
            q8_hi_lo(q8_unbias(b.y), dd, hi[2 * i + 1], lo[2 * i + 1]);
        }
        uint4 *dl = reinterpret_cast<uint4 *>(klo);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            dh[m] = make_uint4(hi[4 * m], hi[4 * m + 1], hi[4 * m + 2], hi[4 * m + 3]);
            dl[m] = make_uint4(lo[4 * m], lo[4 * m + 1], lo[4 * m + 2], lo[4 * m + 3]);
        }
    }
}

// V row part -> LDS: binary16 copy, or a q4_0 block as the exact integers n - 8 (binary16)
// plus its scale at the key's P.V slot of the block's d_V row.
template <int VT>
__device__ __forceinline__ void decode_v_part(const uint32_t (&w)[16], bool odd, uint8_t *vrow, uint16_t *dv_slot) {
    uint4 *dst = reinterpret_cast<uint4 *>(vrow);
    if constexpr (VT == T_F16) {
#pragma unroll
        for (int m = 0; m < 4; ++m) dst[m] = make_uint4(w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]);
    } else {
        const uint32_t dbits = odd ? (w[0] >> 16) : (w[0] & 0xFFFFu);
        const uint32_t sel = odd ? 0x07060504u : 0x05040302u;  // data starts at byte 4 or 2
        const uint32_t dw[4] = {__builtin_amdgcn_perm(w[1], w[0], sel), __builtin_amdgcn_perm(w[2], w[1], sel),
                                __builtin_amdgcn_perm(w[3], w[2], sel), __builtin_amdgcn_perm(w[4], w[3], sel)};
        uint32_t out[16];
        q4_block_centered(dw, out);
#pragma unroll
        for (int m = 0; m < 4; ++m) dst[m] = make_uint4(out[4 * m], out[4 * m + 1], out[4 * m + 2], out[4 * m + 3]);
        *dv_slot = (uint16_t)dbits;
    }
}

// D: head dim of Q, K and V (128 or 64).  CAP: the logit soft-cap is on (a separate
// instantiation, so the plain path carries none of it)
template <int D, int KT, int VT, bool CAP>
__global__ void __launch_bounds__(kThreadsP) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_seg_kernel(const SegParams p, int q_tiles, int n_tasks) {
    using L = Lds<D, KT, VT>;
    constexpr int kKP = k_pitch<D>(), kVP = v_pitch<D>();
    constexpr int NP = D / 32;          // 32-value parts (blocks) of a row; also P.V output tiles
    constexpr int NQK = D / 8;          // Q.K MFMA steps per tile: D/16 k-steps x 2 key halves
    constexpr int NPV = 4 * NP;         // P.V MFMA steps per tile: 4 key steps x NP output tiles
    constexpr int PS = 2 + D;           // partial row stride (M, S, D values)
    constexpr int RW = raw_words<KT>() > raw_words<VT>() ? raw_words<KT>() : raw_words<VT>();
    static_assert(RW <= 16, "raw words");
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::kSize];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool grp0 = wave < 4;  // group 0 decodes K and leads; group 1 decodes V and lags one phase

    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous run of tasks,
    // q tile fastest, so the workgroups sharing one K/V range share an L2.
    const int per = (int)(gridDim.x >> 3);
    const int task = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (task >= n_tasks) return;
    int t = task;
    const int qt = t % q_tiles;
    t /= q_tiles;
    const int g = t % p.n_head_kv;
    t /= p.n_head_kv;
    const int b = t % p.n_seq;
    const int split = t / p.n_seq;

    const int r_tot = p.gqa * p.n_q;
    const int row0 = qt * kBM;
    const int64_t c_begin = (int64_t)split * p.cells_per_split;
    int64_t c_end = c_begin + p.cells_per_split;
    if (c_end > p.n_cells) c_end = p.n_cells;
    if (p.q_pos0 >= 0) {
        // the block's last query sees keys up to its own position
        const int i_last = (min(r_tot, row0 + kBM) - 1) / p.gqa;
        const int64_t lim = p.q_pos0 + i_last - p.pos0 + 1;
        if (lim < c_end) c_end = lim;
    }
    const int n_it = c_end > c_begin ? (int)((c_end - c_begin + kBN - 1) / kBN) : 0;

    const int rl = lane & 31, hh = lane >> 5;
    const int rho = row0 + 32 * wave + rl;
    const bool row_ok = rho < r_tot;
    const int qi = row_ok ? rho / p.gqa : 0;
    const int qr = row_ok ? rho % p.gqa : 0;
    const int wrow0 = min(row0 + 32 * wave, r_tot - 1);
    const int wave_i_first = wrow0 / p.gqa;  // smallest query index of the wave's rows

    // Q^T fragments: lane holds row rho, head_dim 16*ks + 8*hh + 0..7
    half8_t qf[D / 16];
    {
        const uint32_t *qp = reinterpret_cast<const uint32_t *>(
            p.q + (int64_t)qi * p.q_s1 + (int64_t)(g * p.gqa + qr) * p.q_s2 + (int64_t)b * p.q_s3 + 8 * hh);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_ok) v = make_uint4(qp[8 * ks], qp[8 * ks + 1], qp[8 * ks + 2], qp[8 * ks + 3]);
            qf[ks] = __builtin_bit_cast(half8_t, v);
        }
    }
    // Q is complete before any tile load is issued, so no wait inside the loop covers it
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // ---- raw fetch of this thread's row part (group 0: K, group 1: V): key gt / NP, part
    // gt % NP; at D = 64 half of each group's threads have no part
    const int gt = tid & (kGroupT - 1);
    const int fkey = gt / NP, fq = gt % NP;
    const bool fact = kBN * NP == kGroupT || gt < kBN * NP;
    const bool fodd = (fq & 1) != 0;  // q8_0 / q4_0 blocks 1 and 3 start 2 bytes into a word
    const uint8_t *kbase = p.k + (int64_t)g * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)g * p.v_s2;
    const int koff = fkey * (int)p.k_s1 + (((KT == T_F16 ? 64 : 34) * fq) & ~3);
    const int voff = fkey * (int)p.v_s1 + (((VT == T_F16 ? 64 : 18) * fq) & ~3);

    const float c = p.scale_log2;
    float m_used = -INFINITY, l_sum = 0.f;
    f16x_t oacc[NP];
#pragma unroll
    for (int dt = 0; dt < NP; ++dt) oacc[dt] = f16x_t{};
    f16x_t sacc[2];
    half8_t pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) pf[s] = half8_t{};

    // ---- matrix phase: O^T += V^T.W^T for tile it-1 (W = P, times d_V per block for q4_0),
    // then S^T = K.Q^T for tile it.  Operand reads run two MFMAs ahead of their use.
    const int vl = lane & 15, vg = lane >> 4;
    // V^T fragment of step (s, dt): lane (d = 16*(vg&1) + vl of block dt) receives keys
    // 16s + 4*hh + 0..3 (first read) and 16s + 8 + 4*hh + 0..3 (second read): the P slot order
    const int v_lane = (4 * hh + (vl >> 2)) * kVP + (16 * (vg & 1) + 4 * (vl & 3)) * 2;
    const int k_lane = rl * kKP + 16 * hh;
    auto matrix_phase = [&](int it) __attribute__((always_inline)) {
        if (it > 0) {
            const uint8_t *vb = smem + L::kV0 + ((it - 1) & 1) * L::kVbuf;
            const uint8_t *va0 = vb + v_lane;
            const uint8_t *dv0 = vb + L::kVdat + 16 * hh;
            half8_t av[kPD + 1], dv[kPD + 1];
            auto ld = [&](int n) __attribute__((always_inline)) {
                const int s = n / NP, dt = n % NP;
                const uint8_t *va = va0 + 16 * s * kVP + 64 * dt;
                const short4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t *)va);
                const short4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) short4_t *)(va + 8 * kVP));
                av[n % (kPD + 1)] = __builtin_bit_cast(half8_t, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
                if constexpr (VT == T_Q4_0) dv[n % (kPD + 1)] = *reinterpret_cast<const half8_t *>(dv0 + 2 * (dt * kBN + 16 * s));
            };
#pragma unroll
            for (int n = 0; n < kPD; ++n) ld(n);
#pragma unroll
            for (int n = 0; n < NPV; ++n) {
                if (n + kPD < NPV) ld(n + kPD);
                const half8_t wv = (VT == T_Q4_0) ? pf[n / NP] * dv[n % (kPD + 1)] : pf[n / NP];
                oacc[n % NP] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[n % (kPD + 1)], wv, oacc[n % NP], 0, 0, 0);
            }
            constexpr int kRd = VT == T_Q4_0 ? 3 : 2;  // LDS reads per step
            __builtin_amdgcn_sched_group_barrier(0x100, kPD * kRd, 0);
#pragma unroll
            for (int n = 0; n < NPV; ++n) {
                if (n + kPD < NPV) __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
                if constexpr (VT == T_Q4_0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        }
        if (it < n_it) {
            const uint8_t *ka0 = smem + (it & 1) * L::kKbuf + k_lane;
            constexpr int kParts = KT == T_Q8_0 ? 2 : 1;
            half8_t ak[kKD + 1][kParts];
            auto ld = [&](int n) __attribute__((always_inline)) {
                const int ks = n >> 1, kt = n & 1;
                const uint8_t *a = ka0 + 32 * kt * kKP + 32 * ks;
                ak[n % (kKD + 1)][0] = *reinterpret_cast<const half8_t *>(a);
                if constexpr (KT == T_Q8_0) ak[n % (kKD + 1)][1] = *reinterpret_cast<const half8_t *>(a + L::kKhalf);
            };
            sacc[0] = f16x_t{};
            sacc[1] = f16x_t{};
#pragma unroll
            for (int n = 0; n < kKD; ++n) ld(n);
#pragma unroll
            for (int n = 0; n < NQK; ++n) {
                if (n + kKD < NQK) ld(n + kKD);
                const int ks = n >> 1, kt = n & 1;
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak[n % (kKD + 1)][0], qf[ks], sacc[kt], 0, 0, 0);
                if constexpr (KT == T_Q8_0)
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak[n % (kKD + 1)][1], qf[ks], sacc[kt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, kKD * kParts, 0);
#pragma unroll
            for (int n = 0; n < NQK; ++n) {
                if (n + kKD < NQK) __builtin_amdgcn_sched_group_barrier(0x100, kParts, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, kParts, 0);
            }
        }
    };

    // ---- vector phase: online softmax of tile it (exp2 domain, exact running max) into pf
    auto softmax = [&](int it) __attribute__((always_inline)) {
        const int64_t c0 = c_begin + (int64_t)kBN * it;
        // visibility: whole tile visible to every row of the wave, or per element
        const bool full = (c0 + kBN <= p.n_cells) && !p.mask &&
                          (p.q_pos0 < 0 || p.pos0 + c0 + kBN - 1 <= p.q_pos0 + wave_i_first);
        float cc = c;
        if (CAP && full) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kt][i] = softcap_log2(sacc[kt][i], p.cap_cs, p.cap_l2);
            cc = 1.0f;
        } else if (!full) {
            const int64_t nvalid = p.n_cells - c0;
            int64_t lim = p.q_pos0 >= 0 ? p.q_pos0 + qi - p.pos0 - c0 : (int64_t)kBN;
            if (lim > nvalid - 1) lim = nvalid - 1;
            const int lim32 = (int)(lim < -1 ? -1 : (lim > kBN ? kBN : lim));
            // mask values of the lane's 32 keys, all loaded before any is used (indices clamped
            // to the tile's last valid key, so every load is in bounds)
            float mv[2][16];
            if (p.mask) {
                const _Float16 *mrow = p.mask + p.pos0 + c0 + (int64_t)qi * p.m_s1 + (int64_t)b * p.m_s3;
                const int klast = (int)(nvalid < kBN ? nvalid - 1 : kBN - 1);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        mv[kt][i] = (float)mrow[min(32 * kt + 8 * (i >> 2) + 4 * hh + (i & 3), klast)];
            } else {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mv[kt][i] = 0.f;
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = 32 * kt + 8 * (i >> 2) + 4 * hh + (i & 3);
                    float x = CAP ? softcap_log2(sacc[kt][i], p.cap_cs, p.cap_l2) : sacc[kt][i] * c;
                    x = fmaf(mv[kt][i], kLog2eP, x);
                    sacc[kt][i] = kk <= lim32 ? x : -INFINITY;
                }
            }
            cc = 1.0f;
        }
        float mx = -INFINITY;
        if (cc >= 0.f) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
        } else {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, -sacc[kt][i]);
        }
        const float mt = lane_pair_max(mx) * (cc >= 0.f ? cc : -cc);
        const bool need = mt > m_used;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mnew = need ? mt : m_used;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_used - mnew) : 1.0f;
            l_sum *= alpha;
#pragma unroll
            for (int dt = 0; dt < NP; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
            m_used = mnew;
        }
        const float msub = m_used == -INFINITY ? 0.f : m_used;
        const uhalf2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 8 * (s & 1) + 2 * j;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][i], cc, -msub));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][i + 1], cc, -msub));
                const uhalf2_t h = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){p0, p1}, uhalf2_t);
                l_sum = __builtin_amdgcn_fdot2(h, ones, l_sum, false);
                w[j] = h2u(h);
            }
            pf[s] = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
    };

    // ---- the main loop, instantiated once per group so that each group's raw registers are
    // indexed statically (group 0 fetches and decodes K, group 1 V)
    auto body = [&](auto role) __attribute__((always_inline)) {
        constexpr bool G0 = decltype(role)::value;
        constexpr int RT = G0 ? KT : VT;
        uint32_t raw0[16], raw1[16];
        auto fetch = [&](uint32_t (&w)[16], int it) __attribute__((always_inline)) {
            const int64_t c0 = c_begin + (int64_t)kBN * it;
            const int64_t nv = it < n_it ? min((int64_t)kBN, p.n_cells - c0) : 0;
            if (!fact) return;
            if constexpr (G0)
                fetch_part<KT>(w, tile_rsrc(kbase + c0 * p.k_s1, p.k_s1, nv, row_bytes_of<D, KT>()), koff);
            else
                fetch_part<VT>(w, tile_rsrc(vbase + c0 * p.v_s1, p.v_s1, nv, row_bytes_of<D, VT>()), voff);
        };
        auto decode = [&](const uint32_t (&w)[16], int it) __attribute__((always_inline)) {
            if (!fact) return;
            if constexpr (G0) {
                uint8_t *kb = smem + (it & 1) * L::kKbuf;
                decode_k_part<KT>(w, fodd, kb + fkey * kKP + 64 * fq, kb + L::kKhalf + fkey * kKP + 64 * fq);
            } else {
                uint8_t *vb = smem + L::kV0 + (it & 1) * L::kVbuf;
                decode_v_part<VT>(w, fodd, vb + fkey * kVP + 64 * fq,
                                  reinterpret_cast<uint16_t *>(vb + L::kVdat) + fq * kBN + pv_slot(fkey));
            }
        };
        (void)RT;

        // prologue: tiles 0 and 1 fetched, tile 0 decoded, tile 2 fetched
        if (n_it > 0) {
            fetch(raw0, 0);
            fetch(raw1, 1);
            decode(raw0, 0);
            fetch(raw0, 2);
        }
        __syncthreads();
        if constexpr (!G0) __syncthreads();  // group 1 starts one phase later

        // phase pairs: matrix(it) | barrier | vector(it) (softmax, decode of tile it+1, fetch
        // of tile it+3) | barrier.  Unrolled by two so the raw register sets alternate.
        for (int it = 0; it <= n_it; it += 2) {
            __builtin_amdgcn_sched_barrier(0);
            matrix_phase(it);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            if (it < n_it) {
                softmax(it);
                if (it + 1 < n_it) decode(raw1, it + 1);
                fetch(raw1, it + 3);
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
            if (it + 1 > n_it) break;
            matrix_phase(it + 1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            if (it + 1 < n_it) {
                softmax(it + 1);
                if (it + 2 < n_it) decode(raw0, it + 2);
                fetch(raw0, it + 4);
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (G0) __syncthreads();  // group 0 ends one phase earlier
    };
    if (grp0)
        body(std::integral_constant<bool, true>{});
    else
        body(std::integral_constant<bool, false>{});

    // ---- partial of the lane's row: lane holds head dim 32dt + 8(i/4) + 4hh + i%4
    const float l_tot = lane_pair_sum(l_sum);
    if (row_ok) {
        const int64_t r_out = (int64_t)(g * p.gqa + qr) + (int64_t)p.n_head * (qi + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)(p.slot0 + split) * p.n_rows + r_out) * PS;
        if (hh == 0) {
            const float M = m_used == -INFINITY ? -INFINITY : m_used * kLn2P;
            *reinterpret_cast<float2 *>(out) = make_float2(M, l_tot);
        }
#pragma unroll
        for (int dt = 0; dt < NP; ++dt) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float *o = out + 2 + 32 * dt + 8 * a + 4 * hh;
                *reinterpret_cast<float2 *>(o) = make_float2(oacc[dt][4 * a], oacc[dt][4 * a + 1]);
                *reinterpret_cast<float2 *>(o + 2) = make_float2(oacc[dt][4 * a + 2], oacc[dt][4 * a + 3]);
            }
        }
    }
}

template <int D, int KT, int VT>
hipError_t launch_t(const SegParams &p, hipStream_t s) {
    const int q_tiles = (p.gqa * p.n_q + kBM - 1) / kBM;
    const int64_t n_tasks = (int64_t)p.n_splits * q_tiles * p.n_head_kv * p.n_seq;
    if (n_tasks <= 0) return hipSuccess;
    if (n_tasks > ((int64_t)1 << 30)) return hipErrorInvalidValue;
    const int64_t per = (n_tasks + 7) / 8;
    if (p.cap_l2 != 0.f)
        launch_seg(prefill_seg_kernel<D, KT, VT, true>, dim3((unsigned)(8 * per)), dim3(kThreadsP), s, p, q_tiles, (int)n_tasks);
    else
        launch_seg(prefill_seg_kernel<D, KT, VT, false>, dim3((unsigned)(8 * per)), dim3(kThreadsP), s, p, q_tiles, (int)n_tasks);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (k_type == T_Q8_0 && v_type == T_Q4_0) return launch_t<D, T_Q8_0, T_Q4_0>(p, s);
    if (k_type == T_F16 && v_type == T_F16) return launch_t<D, T_F16, T_F16>(p, s);
    if (k_type == T_Q8_0 && v_type == T_F16) return launch_t<D, T_Q8_0, T_F16>(p, s);
    if (k_type == T_F16 && v_type == T_Q4_0) return launch_t<D, T_F16, T_Q4_0>(p, s);
    return hipErrorNotSupported;
}

}  // namespace

int prefill_rows_per_block() { return kBM; }
int prefill_keys_per_iter() { return kBN; }
int prefill_blocks_per_cu() { return 1; }

bool prefill_head_dims_ok(int d, int dv) { return d == dv && (d == kHeadDim || d == 64); }

hipError_t launch_prefill_segment(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (p.rows || !prefill_head_dims_ok(p.d, p.dv)) return hipErrorNotSupported;
    // 64 rows of a tile are addressed with 32-bit offsets from the tile's first row
    if (p.k_s1 * kBN >= ((int64_t)1 << 31) || p.v_s1 * kBN >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    return p.d == 64 ? launch_d<64>(p, k_type, v_type, s) : launch_d<kHeadDim>(p, k_type, v_type, s);
}

}  // namespace rkv
