// MFMA segment kernel for prefill on gfx950: many query rows per KV head, so Q.K^T and P.V
// are dense contractions and run on the matrix cores (v_mfma_f32_32x32x16_f16).
//
// What a segment computes is the same partial as the vector kernel (opencoti-llamafile patch
// 0070-rolling-kv, tail-partial op and fattn.cu streaming_lse_kernel): per output row, over
// the keys of the segment, M = max s_j, S = sum exp(s_j - M), VKQ = sum exp(s_j - M) v_j,
// s_j = scale*<q, k_j> + mask_j, keys at positions after the query's own (causal) or with a
// -inf mask contributing nothing.
//
// Workgroup = 8 waves = 256 query rows of one KV head (row rho = i*gqa + r: query i, head
// g*gqa + r) over one split of the segment's keys, 64 keys per iteration:
//   1. the tile's raw K/V bytes (binary16 or q8_0/q4_0 blocks) are fetched three tiles ahead
//      into registers and staged in LDS (two staging and two operand buffers, one barrier
//      per tile);
//   2. they are decoded once per workgroup, a tile ahead of use, into binary16 MFMA
//      operands in LDS: K as rows [key][d]; q8_0 K exactly, as a rounded binary16 part plus the binary16 residual
//      (d*q has up to 18 significant bits; the two parts carry all of them), so that a large
//      key is not perturbed by rounding; V transposed to [d][key] (q4_0 values d*(n-8)
//      rounded once to binary16, the same rounding P gets);
//   3. each wave forms S^T = K.Q^T for its 32 rows with Q^T held in registers, then an
//      online softmax in the exp2 domain per query column (the running max is raised only
//      when it grows by more than 8, so weights stay <= 256 and most tiles skip rescaling);
//   4. O^T += V^T.P^T with P as binary16 straight from the S^T accumulators (the key order
//      of the accumulator layout is matched by permuting keys when V^T is written);
//   5. the wave writes its rows' partial (M in natural-log units).
#include "rkv_internal.h"
#include "rkv_wave.h"

#include <math.h>

namespace rkv {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));

constexpr int kWavesP = 8;
constexpr int kThreadsP = 64 * kWavesP;
constexpr int kBM = 32 * kWavesP;  // query rows per workgroup
constexpr int kBN = 64;            // keys per iteration
constexpr int kKStride = 272;      // LDS bytes per K row: 128 binary16 + 16 B (conflict-free 128-bit reads)
constexpr int kVtStride = 144;     // LDS bytes per V^T row: 64 binary16 keys + 16 B
constexpr float kLog2eP = 1.4426950408889634f;
constexpr float kLn2P = 0.6931471805599453f;
constexpr float kLazy = 8.0f;      // raise the running max only past this growth (log2 units)

// Bytes of one 128-value row.
template <int T> constexpr int row_bytes_of() { return T == T_F16 ? 256 : (T == T_Q8_0 ? 136 : 72); }
// A tile of 64 rows is fetched as 8-byte units, unit u = row * (row_bytes/8) + column.
template <int T> struct Tile {
    static constexpr int kRow = row_bytes_of<T>();
    static constexpr int kUnits = kRow / 8;
    static constexpr int kTotal = kBN * kUnits;
    static constexpr int kPer = (kTotal + kThreadsP - 1) / kThreadsP;
};

// LDS layout (bytes): two operand sets (binary16 K rows, for q8_0 K also the residual rows,
// and V^T) and two raw staging buffers, so one barrier per tile separates every producer from
// its consumers.
template <int KT, int VT> struct Lds {
    static constexpr int kKlo = kBN * kKStride;                                // q8_0 K only
    static constexpr int kVt = kKlo + (KT == T_Q8_0 ? kBN * kKStride : 0);
    static constexpr int kOp = kVt + kHeadDim * kVtStride;                     // one operand set
    static constexpr int kSv = Tile<KT>::kTotal * 8;                            // raw V after raw K
    static constexpr int kSt = kSv + Tile<VT>::kTotal * 8 + 16;                 // +16: block-window slack
    static constexpr int kSize = 2 * kOp + 2 * kSt;
};

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ uint32_t as_u(half2_t x) { return __builtin_bit_cast(uint32_t, x); }

// Word-aligned view of LDS bytes starting at an even offset o: out[j] = bytes o+4j .. o+4j+3.
template <int NW>
__device__ __forceinline__ void block_words(const uint8_t *lds, int o, uint32_t (&out)[NW]) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(lds + (o & ~3));
    const uint32_t sh = (uint32_t)(o & 3);  // 0 or 2
    uint32_t x[NW + 1];
#pragma unroll
    for (int j = 0; j <= NW; ++j) x[j] = w[j];
#pragma unroll
    for (int j = 0; j < NW; ++j) out[j] = __builtin_amdgcn_alignbyte(x[j + 1], x[j], sh);
}

// Position of key k (0..63) in a V^T row: within each group of 16, bits 2 and 3 of the index
// are swapped, which is the key order of the binary16 P fragments built from S^T.
__device__ __forceinline__ int vt_pos(int k) { return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Fetch the 64-row tile's raw bytes into registers.  `rs` covers exactly the tile's valid rows,
// so units of rows past the end read as zero.
template <int T>
__device__ __forceinline__ void fetch_tile(uint2 (&buf)[Tile<T>::kPer], __amdgpu_buffer_rsrc_t rs,
                                           const int (&off)[Tile<T>::kPer], int tid) {
#pragma unroll
    for (int i = 0; i < Tile<T>::kPer; ++i) {
        if (Tile<T>::kTotal % kThreadsP == 0 || tid + kThreadsP * i < Tile<T>::kTotal)
            buf[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off[i], 0, 0));
    }
}
template <int T>
__device__ __forceinline__ void stash_tile(const uint2 (&buf)[Tile<T>::kPer], uint8_t *stage, int tid) {
#pragma unroll
    for (int i = 0; i < Tile<T>::kPer; ++i) {
        const int u = tid + kThreadsP * i;
        if (Tile<T>::kTotal % kThreadsP == 0 || u < Tile<T>::kTotal) *reinterpret_cast<uint2 *>(stage + 8 * u) = buf[i];
    }
}
template <int T>
__device__ __forceinline__ void tile_offsets(int (&off)[Tile<T>::kPer], int s1, int tid) {
#pragma unroll
    for (int i = 0; i < Tile<T>::kPer; ++i) {
        const int u = tid + kThreadsP * i;
        off[i] = (u / Tile<T>::kUnits) * s1 + (u % Tile<T>::kUnits) * 8;
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t *base, int64_t s1, int64_t nv, int rb) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)((nv - 1) * s1 + rb), 0x00020000);
}

// ---- decode of a staged raw tile into binary16 MFMA operands (once per workgroup)

// K rows: binary16 copy, or q8_0 as hi = rn(d*q) and lo = rn(d*q - hi) (exact).  A thread
// takes 16 values of one key.
template <int KT>
__device__ __forceinline__ void decode_k(const uint8_t *sk, uint8_t *khi, uint8_t *klo, int tid) {
    const int key = tid & 63;
    if constexpr (KT == T_F16) {
        const int part = tid >> 6;  // 32-byte eighth of the row
        const uint4 *src = reinterpret_cast<const uint4 *>(sk + key * 256 + 32 * part);
        uint4 *dst = reinterpret_cast<uint4 *>(khi + key * kKStride + 32 * part);
        dst[0] = src[0];
        dst[1] = src[1];
    } else {
        const int blk = (tid >> 6) & 3, hf = tid >> 8;
        const uint8_t *row = sk + key * 136;
        const int o = 34 * blk;
        const uint32_t dbits = *reinterpret_cast<const uint16_t *>(row + o);
        const half2_t dd = as_h2(dbits | (dbits << 16));
        uint32_t qw[4];
        block_words<4>(row, o + 2 + 16 * hf, qw);
        const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // q + 128 as the low byte of binary16 0x64xx = 1024 + (q + 128): exact integers
            const uint32_t x = qw[j] ^ 0x80808080u;
            const half2_t q01 = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) + bias;
            const half2_t q23 = as_h2(__builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) + bias;
            const half2_t h01 = q01 * dd, h23 = q23 * dd;
            hi[2 * j] = as_u(h01);
            hi[2 * j + 1] = as_u(h23);
            lo[2 * j] = as_u(__builtin_elementwise_fma(q01, dd, -h01));
            lo[2 * j + 1] = as_u(__builtin_elementwise_fma(q23, dd, -h23));
        }
        uint4 *dh = reinterpret_cast<uint4 *>(khi + key * kKStride + 64 * blk + 32 * hf);
        uint4 *dl = reinterpret_cast<uint4 *>(klo + key * kKStride + 64 * blk + 32 * hf);
        dh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        dh[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
        dl[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        dl[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    }
}

// V^T rows [d][key position]: a thread takes two adjacent keys (one 32-bit LDS word per d)
// and 8 values of head_dim.
template <int VT>
__device__ __forceinline__ void decode_v(const uint8_t *sv, uint8_t *vt, int tid) {
    const int kp = tid & 31;
    const int ka = 2 * kp;
    const int col = vt_pos(ka) * 2;  // byte offset of the key pair in a V^T row
    if constexpr (VT == T_F16) {
        const int dq = tid >> 5;  // 8 values of head_dim
        const uint4 a = *reinterpret_cast<const uint4 *>(sv + ka * 256 + 16 * dq);
        const uint4 b = *reinterpret_cast<const uint4 *>(sv + (ka + 1) * 256 + 16 * dq);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
        const uint32_t bw[4] = {b.x, b.y, b.z, b.w};
        uint8_t *dst = vt + 8 * dq * kVtStride + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<uint32_t *>(dst + (2 * j) * kVtStride) = __builtin_amdgcn_perm(bw[j], aw[j], 0x05040100u);
            *reinterpret_cast<uint32_t *>(dst + (2 * j + 1) * kVtStride) = __builtin_amdgcn_perm(bw[j], aw[j], 0x07060302u);
        }
    } else {
        const int blk = (tid >> 5) & 3, half = (tid >> 7) & 1, qq = tid >> 8;
        const int o = 18 * blk;
        const uint8_t *ra = sv + ka * 72, *rb = sv + (ka + 1) * 72;
        const uint32_t da = *reinterpret_cast<const uint16_t *>(ra + o);
        const uint32_t db = *reinterpret_cast<const uint16_t *>(rb + o);
        const half2_t dd = as_h2(da | (db << 16));
        uint32_t wa[2], wb[2];
        block_words<2>(ra, o + 2 + 8 * qq, wa);
        block_words<2>(rb, o + 2 + 8 * qq, wb);
        const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        uint8_t *dst = vt + (32 * blk + 16 * half + 8 * qq) * kVtStride + col;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // nibbles of elements (low nibbles: 0..15 of the block, high nibbles: 16..31)
            const uint32_t na = (wa[j] >> (4 * half)) & 0x0F0F0F0Fu;
            const uint32_t nb = (wb[j] >> (4 * half)) & 0x0F0F0F0Fu;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // halves (1024 + n_a, 1024 + n_b) -> (n - 8) exact -> times (d_a, d_b), rounded once
                const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + e) << 16) | (uint32_t)e;
                const half2_t x = as_h2(__builtin_amdgcn_perm(nb, na, sel) | 0x64006400u) + bias;
                *reinterpret_cast<uint32_t *>(dst + (4 * j + e) * kVtStride) = as_u(x * dd);
            }
        }
    }
}

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

// CAP: the logit soft-cap is on (a separate instantiation, so the plain path carries none of it)
template <int KT, int VT, bool CAP>
__global__ void __launch_bounds__(kThreadsP) __attribute__((amdgpu_waves_per_eu(2)))
prefill_seg_kernel(const SegParams p, int q_tiles, int n_tasks) {
    using L = Lds<KT, VT>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::kSize];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
    half8_t qf[8];
    {
        const uint32_t *qp = reinterpret_cast<const uint32_t *>(
            p.q + (int64_t)qi * p.q_s1 + (int64_t)(g * p.gqa + qr) * p.q_s2 + (int64_t)b * p.q_s3 + 8 * hh);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_ok) v = make_uint4(qp[8 * ks], qp[8 * ks + 1], qp[8 * ks + 2], qp[8 * ks + 3]);
            qf[ks] = __builtin_bit_cast(half8_t, v);
        }
    }
    // Q is complete before any tile load is issued, so no wait inside the loop covers it
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    const uint8_t *kbase = p.k + (int64_t)g * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)g * p.v_s2;
    int koff[Tile<KT>::kPer], voff[Tile<VT>::kPer];
    tile_offsets<KT>(koff, (int)p.k_s1, tid);
    tile_offsets<VT>(voff, (int)p.v_s1, tid);
    uint2 kraw[Tile<KT>::kPer], vraw[Tile<VT>::kPer];
    auto fetch = [&](int it) {
        const int64_t c0 = c_begin + (int64_t)kBN * it;
        const int64_t rem = p.n_cells - c0;
        const int64_t nv = rem < kBN ? rem : (int64_t)kBN;
        fetch_tile<KT>(kraw, tile_rsrc(kbase + c0 * p.k_s1, p.k_s1, nv, row_bytes_of<KT>()), koff, tid);
        fetch_tile<VT>(vraw, tile_rsrc(vbase + c0 * p.v_s1, p.v_s1, nv, row_bytes_of<VT>()), voff, tid);
    };
    auto stash = [&](int s) {
        uint8_t *st = smem + 2 * L::kOp + s * L::kSt;
        stash_tile<KT>(kraw, st, tid);
        stash_tile<VT>(vraw, st + L::kSv, tid);
    };
    auto decode = [&](int s) {
        const uint8_t *st = smem + 2 * L::kOp + s * L::kSt;
        uint8_t *op = smem + s * L::kOp;
        decode_k<KT>(st, op, op + L::kKlo, tid);
        decode_v<VT>(st + L::kSv, op + L::kVt, tid);
    };

    const float c = p.scale_log2;
    float m_used = -INFINITY, l_sum = 0.f;
    f16x_t oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f16x_t{};

    // pipeline: tile it+3 in flight to registers, it+2 staged raw, it+1 being decoded while it
    // is computed; one barrier per tile
    if (n_it > 0) {
        fetch(0);
        stash(0);
    }
    if (n_it > 1) fetch(1);
    __syncthreads();
    if (n_it > 0) decode(0);
    if (n_it > 1) stash(1);
    if (n_it > 2) fetch(2);

    for (int it = 0; it < n_it; ++it) {
        const int cur = it & 1;
        __syncthreads();
        if (it + 1 < n_it) decode(cur ^ 1);
        if (it + 2 < n_it) stash(cur);
        if (it + 3 < n_it) fetch(it + 3);

        const int64_t c0 = c_begin + (int64_t)kBN * it;
        const uint8_t *khi = smem + cur * L::kOp;
        const uint8_t *klo = khi + L::kKlo;
        const uint8_t *vt = khi + L::kVt;

        // ---- S^T = K.Q^T: two 32-key tiles, lane holds key 32kt + 8(i/4) + 4hh + i%4 of row rl
        f16x_t sacc[2] = {f16x_t{}, f16x_t{}};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int off = (32 * kt + rl) * kKStride + (16 * ks + 8 * hh) * 2;
                const half8_t a = *reinterpret_cast<const half8_t *>(khi + off);
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[ks], sacc[kt], 0, 0, 0);
                if constexpr (KT == T_Q8_0) {
                    const half8_t al = *reinterpret_cast<const half8_t *>(klo + off);
                    sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qf[ks], sacc[kt], 0, 0, 0);
                }
            }
        }
        // schedule: three operand reads in flight ahead of the MFMA that consumes them (the
        // default schedule issues each read one MFMA ahead and waits on it)
        constexpr int kNM = KT == T_Q8_0 ? 32 : 16, LA = 3;
        __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
        for (int i = 0; i < kNM - LA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);

        // ---- visibility: whole tile visible to every row of the wave, or per element
        const bool full = (c0 + kBN <= p.n_cells) && !p.mask &&
                          (p.q_pos0 < 0 || p.pos0 + c0 + kBN - 1 <= p.q_pos0 + wave_i_first);
        float cc = c;
        if (CAP && full) {
            // every key visible to every row of the wave: only the soft-cap
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
            const _Float16 *mrow = p.mask ? p.mask + p.pos0 + c0 + (int64_t)qi * p.m_s1 + (int64_t)b * p.m_s3 : nullptr;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = 32 * kt + 8 * (i >> 2) + 4 * hh + (i & 3);
                    float x = CAP ? softcap_log2(sacc[kt][i], p.cap_cs, p.cap_l2) : sacc[kt][i] * c;
                    if (mrow && kk <= lim32) x = fmaf((float)mrow[kk], kLog2eP, x);
                    sacc[kt][i] = kk <= lim32 ? x : -INFINITY;
                }
            }
            cc = 1.0f;
        }

        // ---- online softmax (exp2 domain) for the lane's row; the lane pair (l, l^32) holds it
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
        const bool need = mt > m_used + kLazy;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mnew = need ? mt : m_used;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_used - mnew) : 1.0f;
            l_sum *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
            m_used = mnew;
        }
        const float msub = m_used == -INFINITY ? 0.f : m_used;
        half8_t pf[4];
        const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 8 * (s & 1) + 2 * j;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][i], cc, -msub));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][i + 1], cc, -msub));
                const half2_t h = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){p0, p1}, half2_t);
                l_sum = __builtin_amdgcn_fdot2(h, ones, l_sum, false);
                w[j] = as_u(h);
            }
            pf[s] = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }

        // ---- O^T += V^T.P^T
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const half8_t a = *reinterpret_cast<const half8_t *>(vt + (32 * dt + rl) * kVtStride + (16 * s + 8 * hh) * 2);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[s], oacc[dt], 0, 0, 0);
            }
        }
    }

    // ---- partial of the lane's row: lane holds head_dim 32dt + 8(i/4) + 4hh + i%4
    const float l_tot = lane_pair_sum(l_sum);
    if (row_ok) {
        const int64_t r_out = (int64_t)(g * p.gqa + qr) + (int64_t)p.n_head * (qi + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)(p.slot0 + split) * p.n_rows + r_out) * kPartialStride;
        if (hh == 0) {
            const float M = m_used == -INFINITY ? -INFINITY : m_used * kLn2P;
            *reinterpret_cast<float2 *>(out) = make_float2(M, l_tot);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float *o = out + 2 + 32 * dt + 8 * a + 4 * hh;
                *reinterpret_cast<float2 *>(o) = make_float2(oacc[dt][4 * a], oacc[dt][4 * a + 1]);
                *reinterpret_cast<float2 *>(o + 2) = make_float2(oacc[dt][4 * a + 2], oacc[dt][4 * a + 3]);
            }
        }
    }
}

template <int KT, int VT>
hipError_t launch_t(const SegParams &p, hipStream_t s) {
    const int q_tiles = (p.gqa * p.n_q + kBM - 1) / kBM;
    const int64_t n_tasks = (int64_t)p.n_splits * q_tiles * p.n_head_kv * p.n_seq;
    if (n_tasks <= 0) return hipSuccess;
    if (n_tasks > ((int64_t)1 << 30)) return hipErrorInvalidValue;
    const int64_t per = (n_tasks + 7) / 8;
    if (p.cap_l2 != 0.f)
        launch_seg(prefill_seg_kernel<KT, VT, true>, dim3((unsigned)(8 * per)), dim3(kThreadsP), s, p, q_tiles, (int)n_tasks);
    else
        launch_seg(prefill_seg_kernel<KT, VT, false>, dim3((unsigned)(8 * per)), dim3(kThreadsP), s, p, q_tiles, (int)n_tasks);
    return hipGetLastError();
}

}  // namespace

int prefill_rows_per_block() { return kBM; }
int prefill_keys_per_iter() { return kBN; }
int prefill_blocks_per_cu() { return 1; }

hipError_t launch_prefill_segment(const SegParams &p, int k_type, int v_type, hipStream_t s) {
    if (p.rows) return hipErrorNotSupported;
    // 64 rows of a tile are addressed with 32-bit offsets from the tile's first row
    if (p.k_s1 * kBN >= ((int64_t)1 << 31) || p.v_s1 * kBN >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    if (k_type == T_Q8_0 && v_type == T_Q4_0) return launch_t<T_Q8_0, T_Q4_0>(p, s);
    if (k_type == T_F16 && v_type == T_F16) return launch_t<T_F16, T_F16>(p, s);
    if (k_type == T_Q8_0 && v_type == T_F16) return launch_t<T_Q8_0, T_F16>(p, s);
    if (k_type == T_F16 && v_type == T_Q4_0) return launch_t<T_F16, T_Q4_0>(p, s);
    return hipErrorNotSupported;
}

}  // namespace rkv
