// Matrix-core segment kernel for decode over cell-major q8_0 K / q4_0 V caches on gfx950.
//
// It computes the same partial as the vector kernel (opencoti-llamafile patch 0070-rolling-kv,
// fattn.cu streaming_lse_kernel and the tail-partial op: M = max s_j, S = sum exp(s_j - M),
// VKQ = sum exp(s_j - M) v_j over the segment's keys), but both contractions of a KV head's
// few query rows (gqa x n_q <= 8) run on v_mfma_f32_16x16x32_f16, which frees the vector
// units for the dequantisation and the softmax:
//
//   Q.K  D[row][key] = Q (A: 16 rows x 32 head_dim, rows >= R zero) times K^T (B: one q8_0
//        block of 16 keys).  The codes q enter B as exact binary16 integers 1024 + (q + 128)
//        built by one byte permute; the accumulator input -1152 * (block sum of Q) removes
//        that offset inside the MFMA, and the block scale d_K is applied per key afterwards.
//   P.V  O^T[d][row] = V^T (A: 16 head_dim x 32 keys) times W^T (B: weights of 32 keys) where
//        W = p * d_V folds the per-key block scale of V into the binary16 weights.  V^T is
//        gathered from the staged raw bytes: a lane takes one byte position of eight keys,
//        whose low and high nibbles are the elements e and e + 16 of the block; they enter
//        as exact 1024 + n, and sum W (kept per V block) removes the offset 1032 (n - 8 for
//        the value, 1024 for the encoding) at the end.
//
// Workgroup = HW (8) waves for one (split, head group, sequence), wave w = KV head g0 + w, as in
// the vector cell-major kernel: every 64-cell chunk is one contiguous span fetched with 16-byte
// buffer loads one chunk ahead and staged in LDS; the online softmax is exact (the running max
// is raised whenever a tile exceeds it) so the binary16 weights stay within range.
#include "rkv_internal.h"
#include "rkv_quant.h"
#include "rkv_wave.h"

#include <math.h>

namespace rkv {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kCh = 64;              // cells per chunk
constexpr float kMagicK = 1152.0f;   // q8_0 code q as binary16 1024 + (q + 128)
constexpr float kMagicV = 1032.0f;   // q4_0 nibble n (value n - 8) as binary16 1024 + n

__device__ __forceinline__ half2_t h2v(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ uint32_t u32v(half2_t x) { return __builtin_bit_cast(uint32_t, x); }

// Max / sum over the 16 lanes of each DPP row (lanes 16g .. 16g + 15), in every lane of the row.
__device__ __forceinline__ float row16_max(float x) {
    int k = f2key(x);
    k = max(k, dpp_i<kQuadSwap1>(k));
    k = max(k, dpp_i<kQuadSwap2>(k));
    k = max(k, dpp_i<kRowRor4>(k));
    k = max(k, dpp_i<kRowRor8>(k));
    return key2f(k);
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<kQuadSwap1>(x);
    x += dpp_f<kQuadSwap2>(x);
    x += dpp_f<kRowRor4>(x);
    x += dpp_f<kRowRor8>(x);
    return x;
}

__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int R, int HW>
__global__ void __launch_bounds__(64 * HW) __attribute__((amdgpu_waves_per_eu(2)))
decode_mma_kernel(const SegParams p) {
    constexpr int kCk = HW * kQ8Row, kCv = HW * kQ4Row;     // bytes of one cell (head group)
    constexpr int kSk = kCk + 8, kSv = kCv + 8;               // LDS cell strides
    constexpr int kNT = 64 * HW;
    static_assert(kCk % 16 == 0 && kCv % 16 == 0, "cell segments must be whole 16-byte units");
    __shared__ __attribute__((aligned(16))) uint8_t s_k[kCh * kSk];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kCh * kSv];
    __shared__ __attribute__((aligned(16))) _Float16 s_p[HW][16 * kCh];  // P[row][key] per wave
    __shared__ __attribute__((aligned(16))) _Float16 s_dv[HW][4 * kCh];  // d_V[block][key] per wave
    __shared__ float s_ml[HW][2][16];                                     // per-row exchange

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
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

    // ---- chunk fetch (registers, one chunk ahead) and staging (LDS, padded cells).  Thread t
    // moves 16-byte units sub, sub + 8, ... of cell t / 8 (sub = t % 8): eight threads cover
    // 128 contiguous bytes of a cell per instruction, and every offset is a per-thread base plus
    // an immediate.
    static_assert(kNT == 8 * kCh || kNT < 8 * kCh, "thread mapping");
    constexpr int kCells = kNT / 8;                       // cells per pass
    constexpr int kPass = kCh / kCells;                   // passes per chunk
    constexpr int kUkc = kCk / 16, kUvc = kCv / 16;       // units per cell
    constexpr int kMk = (kUkc + 7) / 8, kMv = (kUvc + 7) / 8;
    const int fcell = tid >> 3, fsub = tid & 7;
    const int gkb = fcell * (int)p.k_s1 + 16 * fsub, gvb = fcell * (int)p.v_s1 + 16 * fsub;
    const int lkb = fcell * kSk + 16 * fsub, lvb = fcell * kSv + 16 * fsub;
    uint4 kb[kPass][kMk], vb[kPass][kMv];
    auto fetch = [&](int64_t c0) {
        const int64_t nv = max((int64_t)0, min((int64_t)kCh, c_end - c0));
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kbase + c0 * p.k_s1), (short)0, (int)(nv * p.k_s1), 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vbase + c0 * p.v_s1), (short)0, (int)(nv * p.v_s1), 0x00020000);
#pragma unroll
        for (int ps = 0; ps < kPass; ++ps) {
            const int so_k = ps * kCells * (int)p.k_s1, so_v = ps * kCells * (int)p.v_s1;
#pragma unroll
            for (int m = 0; m < kMk; ++m)
                if (8 * m + 8 <= kUkc || fsub + 8 * m < kUkc)
                    kb[ps][m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, gkb + 128 * m, so_k, 0));
#pragma unroll
            for (int m = 0; m < kMv; ++m)
                if (8 * m + 8 <= kUvc || fsub + 8 * m < kUvc)
                    vb[ps][m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, gvb + 128 * m, so_v, 0));
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int ps = 0; ps < kPass; ++ps) {
#pragma unroll
            for (int m = 0; m < kMk; ++m)
                if (8 * m + 8 <= kUkc || fsub + 8 * m < kUkc) {
                    uint2 *d = reinterpret_cast<uint2 *>(s_k + lkb + ps * kCells * kSk + 128 * m);
                    d[0] = make_uint2(kb[ps][m].x, kb[ps][m].y);
                    d[1] = make_uint2(kb[ps][m].z, kb[ps][m].w);
                }
#pragma unroll
            for (int m = 0; m < kMv; ++m)
                if (8 * m + 8 <= kUvc || fsub + 8 * m < kUvc) {
                    uint2 *d = reinterpret_cast<uint2 *>(s_v + lvb + ps * kCells * kSv + 128 * m);
                    d[0] = make_uint2(vb[ps][m].x, vb[ps][m].y);
                    d[1] = make_uint2(vb[ps][m].z, vb[ps][m].w);
                }
        }
    };

    float4_t oacc[8];   // O^T: head_dim 16*dt + 4*grp + i of row `col`
    float swacc[4];     // this lane's part (its 8 keys per step) of the weight sum of V block blk, row `col`
    float mrow[4], lrow[4];  // softmax layout: rows 4*grp + i
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) swacc[blk] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mrow[i] = -INFINITY;
        lrow[i] = 0.f;
    }
    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    // kept in a register so that mask-and-insert compiles to one v_and_or_b32 (two literals
    // cannot share an instruction)
    uint32_t vmagic = 0x64006400u;
    asm volatile("" : "+v"(vmagic));
    const float c = p.scale_log2;
    const uint8_t *kw = s_k + wave * kQ8Row;  // this head's K row of cell j at kw + j*kSk
    const uint8_t *vw = s_v + wave * kQ4Row;
    _Float16 *pw = s_p[wave];
    _Float16 *dvw = s_dv[wave];

    const int64_t n_ch = (c_end > c_beg) ? (c_end - c_beg + kCh - 1) / kCh : 0;
    if (n_ch > 0) fetch(c_beg);  // the first chunk is in flight while Q is prepared

    // ---- Q as the A operand of Q.K: lane holds row `col`, head_dim 32*blk + 8*grp + 0..7
    half8_t qa[4];
    float4_t cneg[4];  // accumulator inputs: -1152 * block sum of Q for the rows 4*grp + i
    {
        const bool ok = col < R;
        const int r = ok ? col : 0;
        const _Float16 *qrow = p.q + (int64_t)(r / p.gqa) * p.q_s1 + (int64_t)(g * p.gqa + r % p.gqa) * p.q_s2 +
                               (int64_t)b * p.q_s3;
        float qs[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(qrow + 32 * blk + 8 * grp);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (ok) v = make_uint4(src[0], src[1], src[2], src[3]);
            qa[blk] = __builtin_bit_cast(half8_t, v);
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += (float)qa[blk][j];
            qs[blk] = fold_rows(sum);  // block sum of row `col`, in every lane of the column
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) cneg[blk][i] = -kMagicK * __shfl(qs[blk], 4 * grp + i, 64);
    }

    for (int64_t ch = 0; ch < n_ch; ++ch) {
        const int64_t c0 = c_beg + ch * kCh;
        __syncthreads();  // every wave is done with the previous chunk's LDS
        stash();
        __syncthreads();
        fetch(c0 + kCh);  // past c_end nothing is read

        // V block scales of the chunk, [block][key], lane = key
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
            dvw[blk * kCh + lane] = __builtin_bit_cast(_Float16, (uint16_t)ld_u16(vw + lane * kSv + kQ4Block * blk));

        // ---- Q.K: s[kt][i] = score of key 16*kt + col for row 4*grp + i
        float s[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const uint8_t *kr = kw + (16 * kt + col) * kSk;
#pragma unroll
            for (int i = 0; i < 4; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int o = kQ8Block * blk + 2 + 8 * grp;  // codes 8*grp .. 8*grp+7 of the block
                uint32_t w0, w1;
                if ((kQ8Block * blk + 2) & 3) {
                    const uint32_t *pw32 = reinterpret_cast<const uint32_t *>(kr + o - 2);
                    const uint32_t x0 = pw32[0], x1 = pw32[1], x2 = pw32[2];
                    w0 = __builtin_amdgcn_alignbyte(x1, x0, 2);
                    w1 = __builtin_amdgcn_alignbyte(x2, x1, 2);
                } else {
                    const uint32_t *pw32 = reinterpret_cast<const uint32_t *>(kr + o);
                    w0 = pw32[0];
                    w1 = pw32[1];
                }
                w0 ^= 0x80808080u;  // q + 128 per byte
                w1 ^= 0x80808080u;
                const uint4 bk = make_uint4(__builtin_amdgcn_perm(0x64646464u, w0, 0x05010400u),
                                            __builtin_amdgcn_perm(0x64646464u, w0, 0x05030402u),
                                            __builtin_amdgcn_perm(0x64646464u, w1, 0x05010400u),
                                            __builtin_amdgcn_perm(0x64646464u, w1, 0x05030402u));
                const float4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[blk], __builtin_bit_cast(half8_t, bk),
                                                                          cneg[blk], 0, 0, 0);
                const float dk = h2f(ld_u16(kr + kQ8Block * blk));
#pragma unroll
                for (int i = 0; i < 4; ++i) s[kt][i] = fmaf(dk, d[i], s[kt][i]);
            }
        }

        // ---- visibility: whole chunk visible, or per element (chunk end, causal rule, mask)
        const bool full = (c0 + kCh <= c_end) && !p.mask && (p.q_pos0 < 0 || p.pos0 + c0 + kCh - 1 <= p.q_pos0);
        float cc = c;
        if (!full) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = min(4 * grp + i, R - 1);
                    const int qi = r / p.gqa;
                    const int64_t key = c0 + 16 * kt + col;
                    bool vis = key < c_end;
                    if (p.q_pos0 >= 0 && p.pos0 + key > p.q_pos0 + qi) vis = false;
                    float x = s[kt][i] * c;
                    if (vis && p.mask)
                        x = fmaf((float)p.mask[p.pos0 + key + (int64_t)qi * p.m_s1 + (int64_t)b * p.m_s3], kLog2e, x);
                    s[kt][i] = vis ? x : -INFINITY;
                }
            }
            cc = 1.0f;
        }

        // ---- online softmax per row (exact: the max is raised whenever a chunk exceeds it)
        float mt[4];
        bool need = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx;
            if (cc >= 0.f)
                mx = fmaxf(fmaxf(s[0][i], s[1][i]), fmaxf(s[2][i], s[3][i]));
            else
                mx = fmaxf(fmaxf(-s[0][i], -s[1][i]), fmaxf(-s[2][i], -s[3][i]));
            mt[i] = row16_max(mx) * (cc >= 0.f ? cc : -cc);
            need = need || (mt[i] > mrow[i]);
        }
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool up = mt[i] > mrow[i];
                const float mnew = up ? mt[i] : mrow[i];
                const float alpha = up ? __builtin_amdgcn_exp2f(mrow[i] - mnew) : 1.0f;
                lrow[i] *= alpha;
                mrow[i] = mnew;
                if (col == 0) s_ml[wave][0][4 * grp + i] = alpha;
            }
            lds_order();
            // the P.V accumulators of this lane belong to row `col`
            const float a = s_ml[wave][0][col];
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[dt] *= a;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) swacc[blk] *= a;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float msub = mrow[i] == -INFINITY ? 0.f : mrow[i];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(s[kt][i], cc, -msub));
                lrow[i] += pv;
                pw[(4 * grp + i) * kCh + 16 * kt + col] = (_Float16)pv;
            }
        }
        lds_order();

        // ---- P.V: per 32-key step and V block, weights W = p * d_V, then the two nibble tiles
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 pf = *reinterpret_cast<const uint4 *>(pw + col * kCh + 32 * ks + 8 * grp);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const uint4 dv = *reinterpret_cast<const uint4 *>(dvw + blk * kCh + 32 * ks + 8 * grp);
                const uint4 wu = make_uint4(u32v(h2v(pf.x) * h2v(dv.x)), u32v(h2v(pf.y) * h2v(dv.y)),
                                            u32v(h2v(pf.z) * h2v(dv.z)), u32v(h2v(pf.w) * h2v(dv.w)));
                const half8_t wf = __builtin_bit_cast(half8_t, wu);
                swacc[blk] = __builtin_amdgcn_fdot2(h2v(wu.x), ones, swacc[blk], false);
                swacc[blk] = __builtin_amdgcn_fdot2(h2v(wu.y), ones, swacc[blk], false);
                swacc[blk] = __builtin_amdgcn_fdot2(h2v(wu.z), ones, swacc[blk], false);
                swacc[blk] = __builtin_amdgcn_fdot2(h2v(wu.w), ones, swacc[blk], false);
                // byte `col` of block blk for keys 32*ks + 8*grp + j: element col (low nibble)
                // and element col + 16 (high nibble)
                const uint8_t *vb0 = vw + (32 * ks + 8 * grp) * kSv + kQ4Block * blk + 2 + col;
                uint32_t bt[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) bt[j] = vb0[j * kSv];
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const uint32_t y = __builtin_amdgcn_perm(bt[2 * jj + 1], bt[2 * jj], 0x0C040C00u);  // b0, 0, b1, 0
                    lo[jj] = (y & 0x000F000Fu) | vmagic;
                    hi[jj] = ((y >> 4) & 0x000F000Fu) | vmagic;
                }
                oacc[2 * blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(half8_t, make_uint4(lo[0], lo[1], lo[2], lo[3])), wf, oacc[2 * blk], 0, 0, 0);
                oacc[2 * blk + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(half8_t, make_uint4(hi[0], hi[1], hi[2], hi[3])), wf, oacc[2 * blk + 1], 0, 0, 0);
            }
        }
    }

    // ---- partial of row `col`: gather its max and sum from the softmax layout; the weight sums
    // are folded over the four lane groups (each holds 8 of every 32 keys)
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) swacc[blk] = fold_rows(swacc[blk]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lrow[i] = row16_sum(lrow[i]);
        if (col == 0) {
            s_ml[wave][0][4 * grp + i] = mrow[i];
            s_ml[wave][1][4 * grp + i] = lrow[i];
        }
    }
    lds_order();
    if (col < R) {
        const float M = s_ml[wave][0][col], S = s_ml[wave][1][col];
        const int r = col % p.gqa, i = col / p.gqa;
        const int64_t row = (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)(p.slot0 + split) * p.n_rows + row) * kPartialStride;
        if (grp == 0) {
            out[0] = (M == -INFINITY) ? -INFINITY : M * kLn2;
            out[1] = S;
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[2 + 16 * dt + 4 * grp + e] = fmaf(-kMagicV, swacc[dt >> 1], oacc[dt][e]);
    }
}

template <int R, int HW>
hipError_t launch_mma(const SegParams &p, hipStream_t s, int *occupancy) {
    if (occupancy)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, decode_mma_kernel<R, HW>, 64 * HW, 0);
    launch_seg(decode_mma_kernel<R, HW>, dim3((unsigned)(p.n_splits * (p.n_head_kv / HW) * p.n_seq)), dim3(64 * HW),
               s, p);
    return hipGetLastError();
}

template <int R>
hipError_t launch_mma_r(const SegParams &p, hipStream_t s, int *occupancy) {
    if (p.cell_hw == 8) return launch_mma<R, 8>(p, s, occupancy);
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_mma_ok(const SegParams &p) { return p.cell_hw == 8 && p.gqa * p.n_q >= 1 && p.gqa * p.n_q <= 8; }

hipError_t launch_decode_mma(const SegParams &p, hipStream_t s, int *occupancy) {
    switch (p.gqa * p.n_q) {
        case 1: return launch_mma_r<1>(p, s, occupancy);
        case 2: return launch_mma_r<2>(p, s, occupancy);
        case 3: return launch_mma_r<3>(p, s, occupancy);
        case 4: return launch_mma_r<4>(p, s, occupancy);
        case 5: return launch_mma_r<5>(p, s, occupancy);
        case 6: return launch_mma_r<6>(p, s, occupancy);
        case 7: return launch_mma_r<7>(p, s, occupancy);
        case 8: return launch_mma_r<8>(p, s, occupancy);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rkv
