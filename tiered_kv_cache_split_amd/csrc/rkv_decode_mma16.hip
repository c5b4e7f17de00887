// Matrix-core segment kernel for decode over cell-major binary16 K / V caches on gfx950, for a
// resident window, a lifted tail tile, or a unified pool addressed through a row list.
//
// Same partial as the other decode kernels (opencoti-llamafile patch 0070-rolling-kv, fattn.cu
// streaming_lse_kernel and the tail-partial op: M = max s_j, S = sum exp(s_j - M),
// VKQ = sum exp(s_j - M) v_j), and for the row-list form the semantics of patch 0102's
// attention over kv_rows (a negative entry is padding and contributes nothing).  With binary16
// data both contractions go straight to the matrix cores, without any conversion:
//
//   Q.K  D[key][row] = K (A: 16 keys x 32 head_dim, one 16-byte LDS read per lane) times Q^T
//        (B, rows >= R zero): v_mfma_f32_16x16x32_f16.  A lane then holds one query row for
//        four keys, so the softmax needs no LDS round trip and its probabilities are the B
//        operand of P.V as they stand.
//   P.V  O^T[d][row] = V^T (A: 16 head_dim x 16 keys) times P^T: v_mfma_f32_16x16x16_f16, with
//        V^T read by ds_read_b64_tr_b16 (16 lanes fetch four keys x sixteen head_dim values and
//        receive them transposed, one head_dim value of four keys per lane).
//
// Workgroup = 8 waves for one (split, group of 8 KV heads, sequence), wave w = KV head g0 + w.
// A 16-cell chunk of the group (8 x 256 bytes of K and of V per cell) is moved with 16-byte
// buffer loads into registers and from there into one of two LDS stages; two chunks are always
// in flight in registers, together with the chunk's mask values.  Row-list entries are read one
// fetch ahead of the loads that use them; a padding entry's loads are pointed past the buffer
// range (they read nothing) and its key is masked.  The online softmax is exact (the running
// max is raised whenever a chunk exceeds it).
#include "rkv_internal.h"
#include "rkv_wave.h"

#include <math.h>

namespace rkv {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr int kHW = 8;                 // KV heads per workgroup
constexpr int kCh = 16;                // cells per chunk
constexpr int kNT = 64 * kHW;          // threads
constexpr int kRowB = 2 * kHeadDim;    // bytes of one head's K or V row
constexpr int kCell = kHW * kRowB;     // bytes of one cell of the group
constexpr int kS = kCell + 32;         // LDS cell stride: 520 dwords, 8 mod 32 banks
constexpr int kStage = kCh * kS;       // bytes of one LDS stage of one cache
constexpr int kTpc = kNT / kCh;        // threads per cell (32)
constexpr int kM = kCell / 16 / kTpc;  // 16-byte units per thread, cache and chunk (4)
constexpr uint32_t kNowhere = 0x80000000u;  // buffer offset past every range: reads zero
static_assert(kCell % (16 * kTpc) == 0 && kNT % kCh == 0, "thread mapping");

// One chunk in registers: this thread's K and V units, the mask value it stages, whether its
// cell is a key of the segment, and (row lists) the pool row its next fetch will use.
struct Stage16 {
    uint4 k[kM], v[kM];
    uint32_t mk;
    int ok;
    int2 rid;  // row lists: pool rows of the wave's two cells for the next fetch
};

template <int R, bool ROWS>
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2)))
decode_mma16_kernel(const SegParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t s_k[2 * kStage];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[2 * kStage];
    __shared__ __attribute__((aligned(16))) int s_ok[2][kCh];                 // key is visible data
    __shared__ __attribute__((aligned(16))) _Float16 s_mask[2][kHW][kCh];     // mask[row][key]

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int n_hgrp = p.n_head_kv / kHW;
    int bid = blockIdx.x;
    const int b = bid % p.n_seq;  // sequences fastest: long and short row lists interleave
    bid /= p.n_seq;
    const int hgrp = bid % n_hgrp;
    const int split = bid / n_hgrp;
    const int g = hgrp * kHW + wave;  // this wave's KV head
    const int64_t c_beg = (int64_t)split * p.cells_per_split;
    const int64_t c_end = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    const int64_t n_ch = (c_end > c_beg) ? (c_end - c_beg + kCh - 1) / kCh : 0;
    const int qi_row = min(col, R - 1) / p.gqa;  // query position of this lane's row

    if (n_ch == 0) {  // empty split: the neutral partial
        if (col < R) {
            const int r = col % p.gqa, i = col / p.gqa;
            const int64_t row = (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
            float *out = p.partials + ((int64_t)(p.slot0 + split) * p.n_rows + row) * kPartialStride;
            if (grp == 0) {
                out[0] = -INFINITY;
                out[1] = 0.f;
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) out[2 + 16 * dt + 4 * grp + e] = 0.f;
        }
        return;
    }

    const uint8_t *kbase = p.k + (int64_t)(hgrp * kHW) * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)(hgrp * kHW) * p.v_s2;
    const int32_t *__restrict__ rows = ROWS ? p.rows + (int64_t)b * p.rows_s : nullptr;
    const int fcell = tid / kTpc, fsub = tid % kTpc;
    // mask staging: thread t < R * kCh stages mask[row t / kCh][key t % kCh] of a chunk
    const int mrow = tid / kCh, mkey = tid % kCh;
    const bool mthread = p.mask != nullptr && tid < R * kCh;
    const _Float16 *mbase = p.mask ? p.mask + p.pos0 + (int64_t)b * p.m_s3 + (int64_t)(min(mrow, R - 1) / p.gqa) * p.m_s1
                                   : nullptr;
    // row lists: one resource over the whole pool (its size is checked below 2^31 bytes)
    const __amdgpu_buffer_rsrc_t rk_pool = __builtin_amdgcn_make_buffer_rsrc(
        (void *)kbase, (short)0, ROWS ? (int)(p.n_pool * p.k_s1) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv_pool = __builtin_amdgcn_make_buffer_rsrc(
        (void *)vbase, (short)0, ROWS ? (int)(p.n_pool * p.v_s1) : 0, 0x00020000);
    // pool rows of the wave's two cells 2*wave, 2*wave + 1 of the chunk at c0: uniform reads
    // (scalar loads, so waiting for them never waits for the buffer loads in flight); entries
    // past the segment end are padding
    auto rows_of = [&](int64_t c0) __attribute__((always_inline)) {
        const int64_t c = c0 + 2 * wave;
        const int r0 = rows[min(c, c_end - 1)], r1 = rows[min(c + 1, c_end - 1)];
        return make_int2(c < c_end ? r0 : -1, c + 1 < c_end ? r1 : -1);
    };

    auto fetch = [&](Stage16 &st, int64_t c0) __attribute__((always_inline)) {
        const int64_t c = c0 + fcell;
        if constexpr (ROWS) {
            const int r = (fcell & 1) ? st.rid.y : st.rid.x;
            st.ok = r >= 0;
            const uint32_t ok_ = kNowhere;
            const uint32_t ko = r >= 0 ? (uint32_t)r * (uint32_t)p.k_s1 + 16u * fsub : ok_;
            const uint32_t vo = r >= 0 ? (uint32_t)r * (uint32_t)p.v_s1 + 16u * fsub : ok_;
#pragma unroll
            for (int m = 0; m < kM; ++m)
                st.k[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk_pool, ko + 16 * kTpc * m, 0, 0));
#pragma unroll
            for (int m = 0; m < kM; ++m)
                st.v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv_pool, vo + 16 * kTpc * m, 0, 0));
            st.rid = rows_of(c0 + 2 * kCh);  // for this stage's next fetch
        } else {
            st.ok = c < c_end;
            const int64_t nv = max((int64_t)0, min((int64_t)kCh, c_end - c0));
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(kbase + c0 * p.k_s1), (short)0, (int)(nv * p.k_s1), 0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(vbase + c0 * p.v_s1), (short)0, (int)(nv * p.v_s1), 0x00020000);
            const uint32_t ko = (uint32_t)fcell * (uint32_t)p.k_s1 + 16u * fsub;
            const uint32_t vo = (uint32_t)fcell * (uint32_t)p.v_s1 + 16u * fsub;
#pragma unroll
            for (int m = 0; m < kM; ++m)
                st.k[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16 * kTpc * m, 0, 0));
#pragma unroll
            for (int m = 0; m < kM; ++m)
                st.v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * kTpc * m, 0, 0));
        }
        if (mthread) st.mk = __builtin_bit_cast(uint16_t, mbase[min(c0 + mkey, c_end - 1)]);
    };
    auto stash = [&](const Stage16 &st, int buf) __attribute__((always_inline)) {
        uint8_t *dk = s_k + buf * kStage + fcell * kS + 16 * fsub;
        uint8_t *dv = s_v + buf * kStage + fcell * kS + 16 * fsub;
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            *reinterpret_cast<uint4 *>(dk + 16 * kTpc * m) = st.k[m];
            *reinterpret_cast<uint4 *>(dv + 16 * kTpc * m) = st.v[m];
        }
        if (fsub == 0) s_ok[buf][fcell] = st.ok;
        if (mthread) s_mask[buf][mrow][mkey] = __builtin_bit_cast(_Float16, (uint16_t)st.mk);
    };

    float4_t oacc[8];  // O^T[16*dt + 4*grp + e][col]
    float mrun = -INFINITY, lrow = 0.f;  // running max (log2 domain), this lane's part of the sum
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    const float c = p.scale_log2;

    // ---- Q^T as the B operand of Q.K: lane holds row `col`, head_dim 32*blk + 8*grp + 0..7.  Its
    // loads go first so that waiting for them waits for nothing else.
    half8_t qb[4];
    Stage16 sa, sb;  // chunks 2i (sa) and 2i + 1 (sb) of the split
    sa.mk = sb.mk = 0;
    {
        const bool okq = col < R;
        const int r = okq ? col : 0;
        const _Float16 *qrow = p.q + (int64_t)(r / p.gqa) * p.q_s1 + (int64_t)(g * p.gqa + r % p.gqa) * p.q_s2 +
                               (int64_t)b * p.q_s3;
        uint4 qv[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) qv[blk] = *reinterpret_cast<const uint4 *>(qrow + 32 * blk + 8 * grp);
        if constexpr (ROWS) {
            sa.rid = rows_of(c_beg);
            sb.rid = rows_of(c_beg + kCh);
        }
        fetch(sa, c_beg);
        fetch(sb, c_beg + kCh);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) qb[blk] = __builtin_bit_cast(half8_t, okq ? qv[blk] : make_uint4(0, 0, 0, 0));
    }

    // ---- one chunk from LDS stage `buf`
    auto compute = [&](int buf, int64_t c0) __attribute__((always_inline)) {
        const uint8_t *kw = s_k + buf * kStage + wave * kRowB;  // this head's K row of cell j at kw + j*kS
        const uint8_t *vw = s_v + buf * kStage + wave * kRowB;

        // ---- Q.K: D[key 4*grp + ii][row col]
        float4_t dq = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const uint4 a = *reinterpret_cast<const uint4 *>(kw + col * kS + 64 * blk + 16 * grp);
            dq = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), qb[blk], dq, 0, 0, 0);
        }

        // ---- visibility: the key is data (chunk end, padding row), the causal rule, the mask
        const int4 okv = *reinterpret_cast<const int4 *>(&s_ok[buf][4 * grp]);
        const uint2 mv = p.mask ? *reinterpret_cast<const uint2 *>(&s_mask[buf][min(col, R - 1)][4 * grp]) : make_uint2(0, 0);
        const half2_t m01 = __builtin_bit_cast(half2_t, mv.x), m23 = __builtin_bit_cast(half2_t, mv.y);
        const float mvals[4] = {(float)m01[0], (float)m01[1], (float)m23[0], (float)m23[1]};
        const int okk[4] = {okv.x, okv.y, okv.z, okv.w};
        float s[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            bool vis = okk[ii] != 0;
            if (!ROWS && p.q_pos0 >= 0 && p.pos0 + c0 + 4 * grp + ii > p.q_pos0 + qi_row) vis = false;
            float x = dq[ii] * c;
            if (p.mask) x = fmaf(mvals[ii], kLog2e, x);
            s[ii] = vis ? x : -INFINITY;
        }

        // ---- online softmax of row `col` (exact: the max is raised whenever a chunk exceeds it)
        const float mt = fold_rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        if (__builtin_amdgcn_ballot_w64(mt > mrun)) {
            const float mnew = fmaxf(mt, mrun);
            const float a = (mnew > mrun) ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
            mrun = mnew;
            lrow *= a;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[dt] *= a;
        }
        const float msub = mrun == -INFINITY ? 0.f : mrun;
        float pr[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            pr[ii] = __builtin_amdgcn_exp2f(s[ii] - msub);
            lrow += pr[ii];
        }
        const half4_t pb = half4_t{(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};

        // ---- P.V: A = V^T tile (head_dim 16*dt + col, keys 4*grp + 0..3) by a transposing read:
        // lane col of group grp fetches key 4*grp + col / 4, head_dim 16*dt + 4*(col % 4) + 0..3
        const uint8_t *vr = vw + (4 * grp + (col >> 2)) * kS + 8 * (col & 3);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const short4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4_t *)(vr + 32 * dt));
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, t), pb, oacc[dt], 0, 0, 0);
        }
    };

    // ---- pipeline: chunk ch is computed from stage ch % 2 while chunks ch + 2 and ch + 3 are
    // in flight in registers; the barrier before a stash orders it after every wave's reads of
    // that stage (two chunks earlier) and the previous stash before this chunk's reads.  Chunks
    // go in pairs with no exit in between (a chunk past the end has no visible key), so that
    // every path into the loop head has the same loads in flight.
    stash(sa, 0);
    fetch(sa, c_beg + 2 * kCh);
    for (int64_t ch = 0; ch < n_ch; ch += 2) {
        __syncthreads();
        stash(sb, 1);
        fetch(sb, c_beg + (ch + 3) * kCh);
        compute(0, c_beg + ch * kCh);
        __syncthreads();
        stash(sa, 0);
        fetch(sa, c_beg + (ch + 4) * kCh);
        compute(1, c_beg + (ch + 1) * kCh);
    }

    // ---- partial of row `col`: the sum is folded over the four lanes of the row
    const float S = fold_rows(lrow);
    if (col < R) {
        const int r = col % p.gqa, i = col / p.gqa;
        const int64_t row = (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)(p.slot0 + split) * p.n_rows + row) * kPartialStride;
        if (grp == 0) {
            out[0] = (mrun == -INFINITY) ? -INFINITY : mrun * kLn2;
            out[1] = S;
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[2 + 16 * dt + 4 * grp + e] = oacc[dt][e];
    }
}

template <int R, bool ROWS>
hipError_t launch16(const SegParams &p, hipStream_t s, int *occupancy) {
    if (occupancy)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, decode_mma16_kernel<R, ROWS>, kNT, 0);
    launch_seg(decode_mma16_kernel<R, ROWS>, dim3((unsigned)(p.n_splits * (p.n_head_kv / kHW) * p.n_seq)), dim3(kNT),
               s, p);
    return hipGetLastError();
}

template <int R>
hipError_t launch16_r(const SegParams &p, hipStream_t s, int *occupancy) {
    return p.rows ? launch16<R, true>(p, s, occupancy) : launch16<R, false>(p, s, occupancy);
}

}  // namespace

bool decode_mma16_ok(const SegParams &p) {
    const int R = p.gqa * p.n_q;
    if (p.cell_hw != kHW || R < 1 || R > 8 || p.n_head_kv % kHW != 0) return false;
    // row lists address the pool with 32-bit buffer offsets
    if (p.rows && (p.n_pool <= 0 || p.n_pool * p.k_s1 >= ((int64_t)1 << 31) || p.n_pool * p.v_s1 >= ((int64_t)1 << 31)))
        return false;
    return true;
}

hipError_t launch_decode_mma16(const SegParams &p, hipStream_t s, int *occupancy) {
    switch (p.gqa * p.n_q) {
        case 1: return launch16_r<1>(p, s, occupancy);
        case 2: return launch16_r<2>(p, s, occupancy);
        case 3: return launch16_r<3>(p, s, occupancy);
        case 4: return launch16_r<4>(p, s, occupancy);
        case 5: return launch16_r<5>(p, s, occupancy);
        case 6: return launch16_r<6>(p, s, occupancy);
        case 7: return launch16_r<7>(p, s, occupancy);
        case 8: return launch16_r<8>(p, s, occupancy);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rkv
