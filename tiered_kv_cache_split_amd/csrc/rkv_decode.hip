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
constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Value of lane k summed over the four 16-lane rows, in every row.
__device__ __forceinline__ float fold_rows(float x) {
    const int xi = __builtin_bit_cast(int, x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
    x = __builtin_bit_cast(float, (int)r16[0]) + __builtin_bit_cast(float, (int)r16[1]);
    const int yi = __builtin_bit_cast(int, x);
    const auto r32 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
    return __builtin_bit_cast(float, (int)r32[0]) + __builtin_bit_cast(float, (int)r32[1]);
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

typedef const __attribute__((address_space(4))) uint32_t cu32;

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

// Position of cell c's weight in the per-chunk weight table.  q4_0 V: P.V pairs cells
// (c, c+1); binary16 V (read straight from memory in the fetch order): pairs (c, c+4) of
// each group of 8, laid out next to each other.
template <bool VQ>
__device__ __forceinline__ int wslot(int c) {
    if constexpr (VQ) return c;
    return 8 * (c >> 3) + 2 * (c & 3) + ((c >> 2) & 1);
}

constexpr int kWaves = 4;          // waves per workgroup, each with its own chunks and LDS
constexpr float kQ8Bias = 1152.0f;  // q8_0 codes enter v_dot2 as 1024 + (q + 128)
constexpr float kQ4Bias = 1032.0f;  // q4_0 nibbles enter v_dot2 as 1024 + n, value n - 8

template <int KT, int VT, int R, bool ROWS>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
decode_seg_kernel(const SegParams p) {
    using KF = RowFmt<KT>;
    using VF = RowFmt<VT>;
    constexpr bool kVq = (VT == T_Q4_0);  // q4_0 V goes through LDS; binary16 V is used in registers
    constexpr int kNB = kVq ? 4 : 1;      // weights per (row, cell): one per q4_0 block
    constexpr int kKs = k_lds_stride<KT>();
    constexpr int kVs = RowFmt<VT>::kRow;
    __shared__ __attribute__((aligned(16))) uint8_t s_k[kWaves][kChunk * kKs];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kWaves][kVq ? kChunk * kVs : 16];
    __shared__ __attribute__((aligned(16))) _Float16 s_w[kWaves][R][kNB][kChunk];
    __shared__ float s_qsum[R][4];

    // the wave index is uniform per wave: say so, so chunk bases and descriptors stay scalar
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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

    // Rows of this KV head: rho = i*gqa + r  ->  query i, head h = g*gqa + r.  Q words are read
    // through the constant address space: scalar loads, fed to v_dot2 as SGPR operands.
    const uint32_t *qw[R];
    int qi[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const int r = rho % p.gqa, i = rho / p.gqa;
        qw[rho] = reinterpret_cast<const uint32_t *>(p.q + (int64_t)i * p.q_s1 + (int64_t)(g * p.gqa + r) * p.q_s2 +
                                                      (int64_t)b * p.q_s3);
        qi[rho] = i;
    }
    if constexpr (KT == T_Q8_0) {
        // sum of the 32 Q values of each block, for the q8_0 bias fold
        if (tid < R * 4) {
            const int rho = tid >> 2, blk = tid & 3, r = rho % p.gqa, i = rho / p.gqa;
            const _Float16 *qp = p.q + (int64_t)i * p.q_s1 + (int64_t)(g * p.gqa + r) * p.q_s2 + (int64_t)b * p.q_s3 + 32 * blk;
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < 32; ++t) acc += (float)qp[t];
            s_qsum[rho][blk] = acc;
        }
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

    // Row (cell or pool row) of this lane's cell in the chunk starting at c0, -1 if none.
    auto row_of = [&](int64_t c0) -> int {
        const int64_t c = c0 + lane;
        if (c >= c_end) return -1;
        return ROWS ? rows[c] : (int)c;
    };
    auto nvalid = [&](int64_t c0) { return max((int64_t)0, min((int64_t)kChunk, c_end - c0)); };

    uint8_t *lk = s_k[wave];
    uint8_t *lv = s_v[wave];
    const int64_t n_ch = (c_end > c_beg) ? (c_end - c_beg + kChunk - 1) / kChunk : 0;
    int myrow = -1;
    if (wave < n_ch) {
        const int64_t c0 = c_beg + (int64_t)wave * kChunk;
        myrow = row_of(c0);
        fetch_rows<KT, ROWS>(kb, kbase, p.k_s1, c0, nvalid(c0), myrow, lane);
        if constexpr (kVq) fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, c0, nvalid(c0), myrow, lane);
    }
    const int grp = lane >> 4, kk = lane & 15;

    for (int64_t ch = wave; ch < n_ch; ch += kWaves) {
        const int64_t c0 = c_beg + ch * kChunk;
        stash_rows<KT>(kb, lk, kKs, lane);
        if constexpr (kVq) stash_rows<VT>(vb, lv, kVs, lane);
        const int cur_row = myrow;
        wave_sync();
        // next chunk of this wave (past c_end every row is -1 / out of range: nothing is read)
        {
            const int64_t cn = c0 + kWaves * kChunk;
            myrow = row_of(cn);
            fetch_rows<KT, ROWS>(kb, kbase, p.k_s1, cn, nvalid(cn), myrow, lane);
            if constexpr (kVq) fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, cn, nvalid(cn), myrow, lane);
        }
        // binary16 V: this chunk's rows straight into registers, in flight during Q.K
        if constexpr (!kVq) fetch_rows<VT, ROWS>(vb, vbase, p.v_s1, c0, nvalid(c0), cur_row, lane);

        // ---- Q.K, lane = cell
        float s[R];
#pragma unroll
        for (int rho = 0; rho < R; ++rho) s[rho] = 0.f;
        if constexpr (KT == T_Q8_0) {
            const uint8_t *kr = lk + lane * kKs;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                // block blk: scale at byte 34*blk, codes at 34*blk+2 .. +33
                const int base = 34 * blk, a0 = base & ~3;
                uint32_t w[9];
#pragma unroll
                for (int j = 0; j < 9; ++j) w[j] = *reinterpret_cast<const uint32_t *>(kr + a0 + 4 * j);
                const float dk = h2f((base & 3) ? (w[0] >> 16) : w[0]);
                half2_t a[8], c[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int off = (base & 3) + 2 + 4 * t;  // relative to a0
                    const uint32_t x = (off & 3) ? __builtin_amdgcn_alignbyte(w[(off >> 2) + 1], w[off >> 2], off & 3)
                                                 : w[off >> 2];
                    const uint32_t u = x ^ 0x80808080u;  // q + 128 per byte
                    a[t] = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x05010400u));  // 1024+u0, 1024+u1
                    c[t] = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x05030402u));  // 1024+u2, 1024+u3
                }
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    // The Q block pointer depends on the score two rows back, so at most two
                    // 16-word Q blocks are live in SGPRs and the next load overlaps this row.
                    cu32 *qb = (cu32 *)(qw[rho] + 16 * blk);
                    asm volatile("" : "+s"(qb) : "v"(s[(rho + R - 2) % R]));
                    float dot = 0.f;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        dot = __builtin_amdgcn_fdot2(a[t], as_h2(qb[2 * t]), dot, false);
                        dot = __builtin_amdgcn_fdot2(c[t], as_h2(qb[2 * t + 1]), dot, false);
                    }
                    // sum_t (1152 + q_t) Q_t - 1152 sum_t Q_t = sum_t q_t Q_t
                    s[rho] = fmaf(dk, fmaf(-kQ8Bias, s_qsum[rho][blk], dot), s[rho]);
                }
            }
        } else {
            const uint4 *kr = reinterpret_cast<const uint4 *>(lk + lane * kKs);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint4 x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = kr[4 * q4 + j];
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    cu32 *qb = (cu32 *)(qw[rho] + 16 * q4);
                    asm volatile("" : "+s"(qb) : "v"(s[(rho + R - 2) % R]));
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

        // ---- scores, online softmax (exp2 domain), f16 weights into the chunk table
        const int64_t cell = c0 + lane;
        const bool valid = cur_row >= 0;
        float dvs[kNB];
        if constexpr (kVq) {
#pragma unroll
            for (int j = 0; j < 4; ++j) dvs[j] = h2f(ld_u16(lv + lane * kVs + 18 * j));
        } else {
            dvs[0] = 1.f;
        }
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
                s_w[wave][rho][j][wslot<kVq>(lane)] = wh;
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
                const uint8_t *r0 = lv + c0r * kVs + 18 * blk + 2 + 4 * j4;
                const uint8_t *r1 = r0 + kVs;
                const uint32_t x0 = ld_u16(r0) | (ld_u16(r0 + 2) << 16);
                const uint32_t x1 = ld_u16(r1) | (ld_u16(r1 + 2) << 16);
                const uint32_t lo0 = x0 & 0x0F0F0F0Fu, lo1 = x1 & 0x0F0F0F0Fu;
                const uint32_t hi0 = (x0 >> 4) & 0x0F0F0F0Fu, hi1 = (x1 >> 4) & 0x0F0F0F0Fu;
                half2_t pl[4], ph[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + t) << 16) | (uint32_t)t;
                    pl[t] = as_h2(__builtin_amdgcn_perm(lo1, lo0, sel) | 0x64006400u);  // 1024+n(c0), 1024+n(c1)
                    ph[t] = as_h2(__builtin_amdgcn_perm(hi1, hi0, sel) | 0x64006400u);
                }
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    const half2_t wp = as_h2(reinterpret_cast<const uint32_t *>(s_w[wave][rho][blk])[pd]);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        acc[rho][t] = __builtin_amdgcn_fdot2(pl[t], wp, acc[rho][t], false);
                        acc[rho][4 + t] = __builtin_amdgcn_fdot2(ph[t], wp, acc[rho][4 + t], false);
                    }
                }
            } else {
                const uint4 u0 = vb[2 * st], u1 = vb[2 * st + 1];  // cells 8st+grp, 8st+4+grp
                const uint32_t a0[4] = {u0.x, u0.y, u0.z, u0.w}, a1[4] = {u1.x, u1.y, u1.z, u1.w};
                half2_t ev[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ev[2 * j] = as_h2(__builtin_amdgcn_perm(a1[j], a0[j], 0x05040100u));
                    ev[2 * j + 1] = as_h2(__builtin_amdgcn_perm(a1[j], a0[j], 0x07060302u));
                }
#pragma unroll
                for (int rho = 0; rho < R; ++rho) {
                    const half2_t wp = as_h2(reinterpret_cast<const uint32_t *>(s_w[wave][rho][0])[pd]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[rho][e] = __builtin_amdgcn_fdot2(ev[e], wp, acc[rho][e], false);
                }
            }
        }
        wave_sync();
    }

    // ---- per wave: fold the four 16-lane groups, reduce row sums, remove the q4_0 offset
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[rho][e] = fold_rows(acc[rho][e]);
        l[rho] = wave_sum(l[rho]);
        if constexpr (kVq) {
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

    // ---- merge the waves of the workgroup through LDS and write the split's partial
    __syncthreads();
    float *mb = reinterpret_cast<float *>(&s_k[0][0]);  // [wave][rho][2 + 128]
    if (lane < 16) {
#pragma unroll
        for (int rho = 0; rho < R; ++rho) {
            float *d = mb + (wave * R + rho) * kPartialStride + 2;
            if constexpr (kVq) {
                const int blk = kk >> 2, j4 = kk & 3;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    d[32 * blk + 4 * j4 + t] = acc[rho][t];
                    d[32 * blk + 16 + 4 * j4 + t] = acc[rho][4 + t];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    d[8 * kk + 2 * j] = acc[rho][2 * j];
                    d[8 * kk + 2 * j + 1] = acc[rho][2 * j + 1];
                }
            }
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

// Log-sum-exp merge of partials (patch 0070 streaming_combine_kernel, applied to the
// un-normalised (M, S, VKQ) form).  One workgroup per output row: the segment weights
// e^(M_s - M*) are computed once into LDS, then 8 groups of 128 lanes accumulate the
// values of interleaved segments and fold through LDS.
constexpr int kMergeGroups = 8;
constexpr int kMergeThreads = kMergeGroups * kHeadDim;
constexpr int kMergeTile = 2048;  // segment weights held in LDS per pass

__global__ void __launch_bounds__(kMergeThreads) merge_kernel(const float *__restrict__ part, int n_seg,
                                                              int64_t n_rows, float *__restrict__ o,
                                                              float *__restrict__ lse,
                                                              float *__restrict__ pout) {
    __shared__ float s_wt[kMergeTile];
    __shared__ float s_red[kMergeThreads / 64];
    __shared__ float s_acc[kMergeGroups][kHeadDim];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, d = tid & (kHeadDim - 1), grp = tid / kHeadDim;
    const int64_t step = n_rows * kPartialStride;
    const float *base = part + row * kPartialStride;

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

    float S = 0.f, acc = 0.f;
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
            for (int j = grp; j < nt; j += kMergeGroups) acc = fmaf(base[(int64_t)(t0 + j) * step + 2 + d], s_wt[j], acc);
            __syncthreads();
        }
    }
    // fold S over the block and acc over the groups
    S = wave_sum(S);
    if ((tid & 63) == 0) s_red[tid >> 6] = S;
    s_acc[grp][d] = acc;
    __syncthreads();
    if (grp != 0) return;
    S = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeThreads / 64; ++j) S += s_red[j];
    acc = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeGroups; ++j) acc += s_acc[j][d];
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
        hipLaunchKernelGGL((decode_seg_kernel<KT, VT, R, true>), dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, p);
    else
        hipLaunchKernelGGL((decode_seg_kernel<KT, VT, R, false>), dim3((unsigned)blocks), dim3(64 * kWaves), 0, s, p);
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
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)n_rows), dim3(kMergeThreads), 0, s, partials, n_seg, n_rows, o,
                       lse, partial_out);
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
