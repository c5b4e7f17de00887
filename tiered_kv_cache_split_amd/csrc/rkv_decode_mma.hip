// Matrix-core segment kernel for decode over cell-major q8_0 K / q4_0 V caches on gfx950, at
// head dims 64, 128, 256, 512 and the 576 / 512 pair, over a segment of cells or a row list.
//
// It computes the same partial as the vector kernels (opencoti-llamafile patch 0070-rolling-kv,
// fattn.cu streaming_lse_kernel and the tail-partial op: M = max s_j, S = sum exp(s_j - M),
// VKQ = sum exp(s_j - M) v_j over the segment's keys; for row lists the semantics of
// llama.cpp PR #29510's flash_attn_ext_rows), but both contractions of a KV head's query rows
// (up to 16 per workgroup) run on v_mfma_f32_16x16x32_f16, which frees the vector units for
// the dequantisation and the softmax:
//
//   Q.K  D[key][row] = K (A: 16 keys x 32 head_dim of one q8_0 block) times Q^T (B, rows >= R
//        zero).  The codes q enter A as exact binary16 integers 1024 + (q + 128) built by one
//        byte permute; the accumulator input -1152 * (block sum of Q) removes that offset
//        inside the MFMA, and the block scale d_K is applied per key afterwards.  In this
//        output layout a lane holds one query row for four keys, so the softmax of a row needs
//        no LDS round trip and its probabilities are already the B operand of P.V.
//   P.V  O^T[d][row] = V^T (A: 16 head_dim x 32 keys) times W^T (B: weights of 32 keys) where
//        W = p * d_V folds the per-key block scale of V into the binary16 weights.  V^T comes
//        from one ds_read_b64_tr_b8 per block: a lane receives one byte position of eight
//        keys, whose low and high nibbles are the elements e and e + 16 of the block.  The low
//        nibble enters as exact 1024 + n, the high one in place as 1024 + 16 n; one more MFMA
//        per tile with a constant A of -1032 (or -1152) removes the offset from the same
//        accumulator, so the tiles hold n - 8 (and 16 (n - 8)) times the weights.
//
// Workgroup = one (block of RG row groups, split, group of HW KV heads, sequence): HW * SV * RG
// compute waves (one row group and KV head each, SV waves per head) and loader waves that move
// every 32-cell chunk with buffer loads into registers (two chunks in flight) and from there
// into one of two LDS stages, where each block's scale is split from its data and the data
// lands on 16-byte slots; one barrier per chunk separates the stage being computed from the
// one being filled.  The online softmax is exact (the running max is raised whenever a chunk
// exceeds it), so the binary16 weights stay in range.
#include "rkv_internal.h"
#include "rkv_unpack.h"
#include "rkv_wave.h"

#include <math.h>

namespace rkv {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));

constexpr int kCh = 32;              // cells per chunk
constexpr float kMagicK = kQ8Bias;     // q8_0 code q as binary16 1152 + q (q8_biased)
constexpr float kMagicV = kQ4BiasLo;   // q4_0 low nibble n (value n - 8) as binary16 1032 + (n - 8)
constexpr float kMagicVHi = kQ4BiasHi; // q4_0 high nibble n kept in place: binary16 1152 + 16 (n - 8)

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

// A chunk unit in registers: two q8_0 blocks of one head's K row (68 bytes: bytes 0..35 as nine
// words, the second block's aligned codes 36..67 as two quads), or two q4_0 blocks of its V row
// (36 bytes: bytes 0..19 as five words, the second block's aligned data 20..35 as one quad).
// The aligned quads go to LDS as loaded.
struct KStage {
    uint4 ka0, ka1, kb0, kb1;
    uint32_t kx;
};
struct VStage {
    uint4 va, vb;
    uint32_t vx;
};

// Geometry of a workgroup for head dims DK (Q, K) and DV (V), HW KV heads, SV compute waves
// per head (each of them takes 1 / SV of the V blocks) and RG groups of 16 query rows, each
// with compute waves of its own over the same staged chunks.  A K unit is two blocks of one head's K
// row, a V unit two blocks of its V row; a cell holds kTpcK and kTpcV of them, a chunk kCh cells.
// Loader threads take two V units and NIK K units (the last of them only for the first threads
// when DK > DV) of every chunk; their count kNL is a whole number of waves when HW * DV / 64 is
// a multiple of 4.
template <int DK, int DV, int HW, int SV, int RG>
struct Geo {
    static constexpr int NBK = DK / 32;       // q8_0 blocks per K row
    static constexpr int NBVT = DV / 32;      // q4_0 blocks per V row
    static constexpr int NBV = NBVT / SV;     // V blocks per compute wave
    static constexpr int UK = NBK / 2, UV = NBVT / 2;  // units per head and cell
    static constexpr int kTpcK = HW * UK, kTpcV = HW * UV;  // units per cell
    static constexpr int kNC = 64 * HW * SV * RG;  // compute threads (RG row groups of 16)
    static constexpr int kNL = kCh * kTpcV / 2;  // loader threads
    static constexpr int kKU = kCh * kTpcK;   // K units per chunk
    static constexpr int NIK = (kKU + kNL - 1) / kNL, NIKF = kKU / kNL;  // K units per loader thread (all, full)
    static constexpr int kThreads = kNC + kNL;
    static_assert(DK % 64 == 0 && DV % 64 == 0 && kNL % 64 == 0 && NIK <= 3, "loader threads must fill whole waves");
    // LDS K stage: two planes (code bytes 0..15 and 16..31 of every q8_0 block), each with the
    // block's 16 bytes at a slot of its cell (the first block of each unit in slots 0 .. kTpcK-1,
    // the second in kTpcK .. 2kTpcK-1), then d_K as [head][block][key]
    static constexpr int kKc = 32 * kTpcK + 16;    // K plane cell stride: 2 kTpcK slots + 16 bytes
    static constexpr int kKp = kCh * kKc;          // bytes of one K plane
    static constexpr int kKh = 2 * NBK * kCh + 16; // d_K bytes per head
    static constexpr int kBk = 2 * kKp + HW * kKh; // bytes of one LDS K stage
    // LDS V stage: the 16 data bytes of every q4_0 block at a 16-byte slot of its cell (slots as
    // for K), cells kVc bytes apart plus 64 more from cell 16 on (the transposing reads of 8
    // keys then meet 8 distinct bank quads), followed by d_V as [head][block][P.V slot of the key]
    static constexpr int kVc = 32 * kTpcV + 16;     // V cell stride
    static constexpr int kVd = kCh * kVc + 64;      // data bytes of a V stage
    static constexpr int kVh = 2 * NBVT * kCh + 16; // d_V bytes per head
    static constexpr int kBv = kVd + HW * kVh;      // bytes of one LDS V stage
    // waves of all resident workgroups per SIMD that the register budget allows
    static constexpr int kWavesPerEu = DK >= 256 ? 2 : 3;
    static_assert(NBVT % SV == 0, "V blocks split evenly");
    // wide heads keep the Q.K accumulator inputs (one float4 per block and row) in LDS rather
    // than in registers, and from 512 on the Q^T fragments (16 bytes per lane and block) too;
    // both per head, written by the head's first wave
    static constexpr bool kCinLds = NBK > 4, kQLds = NBK > 8;
    static constexpr int kCin = kCinLds ? RG * HW * NBK * 16 * 16 : 16;  // LDS bytes of the inputs
    static constexpr int kQf = kQLds ? RG * HW * NBK * 64 * 16 : 16;     // LDS bytes of the fragments
};

// Kernel modes: a segment without a mask, a segment with one, a row list (with or without).
enum : int { kModePlain = 0, kModeMask = 1, kModeRows = 2 };

// CAP: the logit soft-cap is on; MODE: the chunk cells are segment cells or row-list entries
// naming pool rows, and with a mask the compute waves fetch each chunk's mask values ahead of
// its Q.K (separate instantiations, so the plain path carries none of it).
// The workgroup's first HW * SV * RG waves compute (wave w: row group w / (HW SV) of the
// workgroup's RG, KV head g0 + (w % (HW SV)) / SV, V blocks of part w % SV); the remaining kNL
// threads only load and stage the chunks (two chunks in flight), so the compute waves never
// wait for memory and hold no staging registers.
template <int DK, int DV, int HW, int SV, int RG, bool CAP, int MODE>
__global__ void __launch_bounds__((Geo<DK, DV, HW, SV, RG>::kThreads))
__attribute__((amdgpu_waves_per_eu((Geo<DK, DV, HW, SV, RG>::kWavesPerEu)))) decode_mma_kernel(const SegParams p) {
    using G = Geo<DK, DV, HW, SV, RG>;
    constexpr int NBK = G::NBK, NBV = G::NBV, UK = G::UK, UV = G::UV, kTpcK = G::kTpcK, kTpcV = G::kTpcV;
    constexpr int kNC = G::kNC, kNL = G::kNL, NIK = G::NIK, NIKF = G::NIKF;
    constexpr int kKc = G::kKc, kKp = G::kKp, kKh = G::kKh, kBk = G::kBk;
    constexpr int kVc = G::kVc, kVd = G::kVd, kVh = G::kVh, kBv = G::kBv;
    constexpr int kPs = 2 + DV;  // partial row: M, S, VKQ[DV]
    constexpr bool ROWS = MODE == kModeRows, MSK = MODE != kModePlain;
    static_assert(kCh == 32, "the key permutation of P.V assumes 32-key chunks");
    __shared__ __attribute__((aligned(16))) uint8_t s_k[2 * kBk];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[2 * kBv];
    __shared__ __attribute__((aligned(16))) uint8_t s_cin[G::kCin];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[G::kQf];
    __shared__ __attribute__((aligned(16))) int s_ok[2][ROWS ? kCh : 4];  // row lists: cell j of the stage is a key

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    // query rows rho = i * gqa + r of a KV head, in groups of 16 (the columns of the MFMA tiles;
    // columns past the group's rows are padding), RG of them per workgroup; the block of row
    // groups is the fastest grid index, so the workgroups reading one chunk run together
    const int R_all = p.gqa * p.n_q, n_rg = (R_all + 15) >> 4, n_rgb = (n_rg + RG - 1) / RG;
    const int n_hgrp = p.n_head_kv / HW;
    int bid = blockIdx.x;
    const int rgb = bid % n_rgb;
    bid /= n_rgb;
    const int split = bid % p.n_splits;
    bid /= p.n_splits;
    const int hgrp = bid % n_hgrp;
    const int b = bid / n_hgrp;
    const bool loader = tid >= kNC;
    const int rgw = loader ? 0 : wave / (HW * SV);  // this compute wave's row group in the workgroup
    const int wh = loader ? 0 : (wave % (HW * SV)) / SV, part = loader ? 0 : wave % SV;  // head, V part
    // this wave's rows R0 .. R0 + R - 1 (none when R <= 0: the last block's spare row groups)
    const int R0 = 16 * (RG * rgb + rgw), R = min(16, R_all - R0);
    const int g = hgrp * HW + wh;  // this compute wave's KV head
    int64_t c_beg = (int64_t)split * p.cells_per_split;
    int64_t c_end = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    if constexpr (ROWS) {
        // a list ends at its extent (1 + its last pool row, from a scan before the launch): the
        // splits share the entries up to it evenly, in whole chunks, and the padding after it
        // is not walked
        if (p.row_extent) {
            int e = 0;
#pragma unroll
            for (int q = 0; q < kRowExtentParts; ++q) e = max(e, p.row_extent[b * kRowExtentParts + q]);
            const int64_t ext = min(p.n_cells, (int64_t)e);
            const int64_t per = ((ext + p.n_splits - 1) / p.n_splits + kCh - 1) / kCh * kCh;
            c_beg = (int64_t)split * per;
            c_end = min(ext, c_beg + per);
        }
    }
    const uint8_t *kbase = p.k + (int64_t)(hgrp * HW) * p.k_s2;
    const uint8_t *vbase = p.v + (int64_t)(hgrp * HW) * p.v_s2;
    // row lists: chunk cells are list entries of sequence b, each naming a pool row (a negative
    // entry, or one outside the pool, is no key)
    const int32_t *rlist = ROWS ? p.rows + (int64_t)b * p.rows_s : nullptr;

    // ---- chunk fetch (registers) and staging (LDS).  K unit t is cell t / kTpcK, sub = t %
    // kTpcK: blocks 2 (sub % UK) and + 1 of head sub / UK, K bytes 68 sub .. 68 sub + 67 of the
    // cell; V unit t likewise with kTpcV, UV and V bytes 36 sub .. 36 sub + 35 (heads are packed
    // in a cell, so consecutive units cover contiguous bytes).  Staging splits the scales from
    // the block data and puts the data on 16-byte slots.  Cells past the segment end lie outside
    // the buffer resource's range and read as zero.
    // A unit's global offset is gb within its chunk (cell-major segment), or sub plus its pool
    // row times the row stride (row list); cell is its cell in the chunk.
    struct KUnit {
        int gb, lb, ls, cell, sub;
    };
    struct VUnit {
        int gb, lb, ls, cell, sub;
    };
    auto k_unit_of = [&](int t) __attribute__((always_inline)) {
        const int fcell = t / kTpcK, fsub = t % kTpcK;
        const int fh = fsub / UK, fb = 2 * (fsub % UK);  // head and first block of the unit
        return KUnit{fcell * (int)p.k_s1 + 68 * fsub, fcell * kKc + 16 * fsub,
                     2 * kKp + fh * kKh + fb * (2 * kCh) + 2 * fcell, fcell, 68 * fsub};
    };
    auto v_unit_of = [&](int t) __attribute__((always_inline)) {
        const int fcell = t / kTpcV, fsub = t % kTpcV;
        const int fh = fsub / UV, fb = 2 * (fsub % UV);
        return VUnit{fcell * (int)p.v_s1 + 36 * fsub, fcell * kVc + 64 * ((fcell >> 4) & 1) + 16 * fsub,
                     kVd + fh * kVh + fb * (2 * kCh) + 2 * (8 * ((fcell >> 2) & 3) + 4 * (fcell >> 4) + (fcell & 3)),
                     fcell, 36 * fsub};
    };
    // buffer resources: the chunk's cells (segment) or the whole pool (row list)
    auto rsrc_k = [&](int64_t c0) __attribute__((always_inline)) {
        const int64_t nv = max((int64_t)0, min((int64_t)kCh, c_end - c0));
        return ROWS ? __builtin_amdgcn_make_buffer_rsrc((void *)kbase, (short)0, (int)(p.n_pool * p.k_s1), 0x00020000)
                     : __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + c0 * p.k_s1), (short)0, (int)(nv * p.k_s1),
                                                         0x00020000);
    };
    auto rsrc_v = [&](int64_t c0) __attribute__((always_inline)) {
        const int64_t nv = max((int64_t)0, min((int64_t)kCh, c_end - c0));
        return ROWS ? __builtin_amdgcn_make_buffer_rsrc((void *)vbase, (short)0, (int)(p.n_pool * p.v_s1), 0x00020000)
                     : __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + c0 * p.v_s1), (short)0, (int)(nv * p.v_s1),
                                                         0x00020000);
    };
    // row lists: the pool row of cell `cell` of the chunk at c0, or -1 (no key: a negative entry,
    // one outside the pool, or a cell past the segment)
    auto pool_row = [&](int64_t c0, int cell) __attribute__((always_inline)) {
        const int64_t c = c0 + cell;
        const int r = c < c_end ? rlist[c] : -1;
        return (r >= 0 && (int64_t)r < p.n_pool) ? r : -1;
    };
    constexpr uint32_t kNowhere = 0x80000000u;  // a buffer offset past every range: reads zero
    auto fetch_k = [&](KStage &st, __amdgpu_buffer_rsrc_t rk, int gkb) __attribute__((always_inline)) {
        st.ka0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, gkb, 0, 0));
        st.ka1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, gkb + 16, 0, 0));
        st.kx = __builtin_amdgcn_raw_buffer_load_b32(rk, gkb + 32, 0, 0);
        st.kb0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, gkb + 36, 0, 0));
        st.kb1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, gkb + 52, 0, 0));
    };
    auto fetch_v = [&](VStage &st, __amdgpu_buffer_rsrc_t rv, int gvb) __attribute__((always_inline)) {
        st.va = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, gvb, 0, 0));
        st.vx = __builtin_amdgcn_raw_buffer_load_b32(rv, gvb + 16, 0, 0);
        st.vb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, gvb + 20, 0, 0));
    };
    auto stash_k = [&](const KStage &st, int buf, const KUnit &u) __attribute__((always_inline)) {
        const int lkb = u.lb, lks = u.ls;
        // words x0 .. x8 (bytes 0..35); the first block's codes start 2 bytes into them (its
        // scale is the low half of x0), the second block's scale is the high half of x8
        const uint32_t x[9] = {st.ka0.x, st.ka0.y, st.ka0.z, st.ka0.w, st.ka1.x, st.ka1.y, st.ka1.z, st.ka1.w, st.kx};
        uint32_t ca[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ca[i] = __builtin_amdgcn_alignbyte(x[i + 1], x[i], 2);
        uint8_t *kd = s_k + buf * kBk;
        *reinterpret_cast<uint4 *>(kd + lkb) = make_uint4(ca[0], ca[1], ca[2], ca[3]);
        *reinterpret_cast<uint4 *>(kd + kKp + lkb) = make_uint4(ca[4], ca[5], ca[6], ca[7]);
        *reinterpret_cast<uint4 *>(kd + lkb + 16 * kTpcK) = st.kb0;
        *reinterpret_cast<uint4 *>(kd + kKp + lkb + 16 * kTpcK) = st.kb1;
        *reinterpret_cast<uint16_t *>(kd + lks) = (uint16_t)x[0];
        *reinterpret_cast<uint16_t *>(kd + lks + 2 * kCh) = (uint16_t)(x[8] >> 16);
    };
    auto stash_v = [&](const VStage &st, int buf, const VUnit &u) __attribute__((always_inline)) {
        const int lvb = u.lb, lvs = u.ls;
        // the first block's data starts 2 bytes into va, vx (its scale is the low half of va.x,
        // the second block's the high half of vx); the second block's data is vb
        uint8_t *vd = s_v + buf * kBv;
        *reinterpret_cast<uint4 *>(vd + lvb) = make_uint4(__builtin_amdgcn_alignbyte(st.va.y, st.va.x, 2),
                                                          __builtin_amdgcn_alignbyte(st.va.z, st.va.y, 2),
                                                          __builtin_amdgcn_alignbyte(st.va.w, st.va.z, 2),
                                                          __builtin_amdgcn_alignbyte(st.vx, st.va.w, 2));
        *reinterpret_cast<uint4 *>(vd + lvb + 16 * kTpcV) = st.vb;
        *reinterpret_cast<uint16_t *>(vd + lvs) = (uint16_t)st.va.x;
        *reinterpret_cast<uint16_t *>(vd + lvs + 2 * kCh) = (uint16_t)(st.vx >> 16);
    };

    // ---- pipeline: chunk ch is computed from stage ch % 2 while the loader threads hold
    // chunks ch + 2 and ch + 3 in registers; the barrier before a stash orders it after every
    // compute wave's reads of that stage (two chunks earlier) and before this chunk's reads.
    // Loads past the segment end read nothing.  The loader threads leave after their last
    // stash; the compute waves meet them at every barrier until then.
    const int64_t n_ch = (c_end > c_beg) ? (c_end - c_beg + kCh - 1) / kCh : 0;
    if (loader) {
        // loader thread lt: K units lt + i kNL (i < NIK; beyond NIKF only while inside the
        // chunk's kKU units) and V units lt, lt + kNL
        const int lt = tid - kNC;
        const bool k_last = lt + NIKF * kNL < G::kKU;  // this thread has a K unit at i = NIKF
        KUnit ku[NIK];
#pragma unroll
        for (int i = 0; i < NIK; ++i) ku[i] = k_unit_of(min(lt + i * kNL, G::kKU - 1));
        const VUnit v0 = v_unit_of(lt), v1 = v_unit_of(lt + kNL);
        KStage ka[NIK], kb[NIK];  // chunks 2i (a) and 2i + 1 (b)
        VStage va0, va1, vb0, vb1;
        // row lists: pool rows of the units' cells for the next fetch of each register set,
        // read one fetch ahead
        int rka[ROWS ? NIK : 1], rkb[ROWS ? NIK : 1], rva[2], rvb[2];
        auto rows_for = [&](int (&rk)[ROWS ? NIK : 1], int (&rv)[2], int64_t c0) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NIK; ++i) rk[i] = pool_row(c0, ku[i].cell);
            rv[0] = pool_row(c0, v0.cell);
            rv[1] = pool_row(c0, v1.cell);
        };
        auto fetch_all = [&](KStage (&ks)[NIK], VStage &x0, VStage &x1, int (&rk)[ROWS ? NIK : 1], int (&rv)[2], int64_t c0)
            __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t rsk = rsrc_k(c0), rsv = rsrc_v(c0);
            if constexpr (ROWS) {
#pragma unroll
                for (int i = 0; i < NIK; ++i)
                    if (i < NIKF || k_last)
                        fetch_k(ks[i], rsk, rk[i] >= 0 ? rk[i] * (int)p.k_s1 + ku[i].sub : (int)kNowhere);
                fetch_v(x0, rsv, rv[0] >= 0 ? rv[0] * (int)p.v_s1 + v0.sub : (int)kNowhere);
                fetch_v(x1, rsv, rv[1] >= 0 ? rv[1] * (int)p.v_s1 + v1.sub : (int)kNowhere);
                rows_for(rk, rv, c0 + 2 * kCh);  // this set's next fetch
            } else {
#pragma unroll
                for (int i = 0; i < NIK; ++i)
                    if (i < NIKF || k_last) fetch_k(ks[i], rsk, ku[i].gb);
                fetch_v(x0, rsv, v0.gb);
                fetch_v(x1, rsv, v1.gb);
            }
        };
        // row lists: whether each cell of the chunk at c0 is a key, for the compute waves (the
        // thread holding the cell's first K unit writes it)
        auto stash_ok = [&](int buf, int64_t c0) __attribute__((always_inline)) {
            if constexpr (ROWS) {
#pragma unroll
                for (int i = 0; i < NIK; ++i) {
                    const int t = lt + i * kNL;
                    if (t < G::kKU && t % kTpcK == 0) s_ok[buf][ku[i].cell] = pool_row(c0, ku[i].cell) >= 0;
                }
            }
        };
        auto stash_all = [&](const KStage (&ks)[NIK], const VStage &x0, const VStage &x1, int buf)
            __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < NIK; ++i)
                if (i < NIKF || k_last) stash_k(ks[i], buf, ku[i]);
            stash_v(x0, buf, v0);
            stash_v(x1, buf, v1);
        };
        if constexpr (ROWS) {
            rows_for(rka, rva, c_beg);
            rows_for(rkb, rvb, c_beg + kCh);
        }
        fetch_all(ka, va0, va1, rka, rva, c_beg);
        fetch_all(kb, vb0, vb1, rkb, rvb, c_beg + kCh);
        stash_all(ka, va0, va1, 0);
        stash_ok(0, c_beg);
        fetch_all(ka, va0, va1, rka, rva, c_beg + 2 * kCh);
        for (int64_t ch = 0; ch < n_ch; ch += 2) {
            __syncthreads();
            stash_all(kb, vb0, vb1, 1);
            stash_ok(1, c_beg + (ch + 1) * kCh);
            fetch_all(kb, vb0, vb1, rkb, rvb, c_beg + (ch + 3) * kCh);
            if (ch + 1 >= n_ch) break;
            __syncthreads();
            stash_all(ka, va0, va1, 0);
            stash_ok(0, c_beg + (ch + 2) * kCh);
            fetch_all(ka, va0, va1, rka, rva, c_beg + (ch + 4) * kCh);
        }
        return;
    }

    // Lane (col, grp) owns query row `col` (rows >= R are padding and never written) and, within
    // a chunk, the keys 16*kt + 4*grp + ii (kt, ii < 2, 4): the Q.K output layout.  Its P.V
    // accumulators hold O^T[d][col] for d = 16*dt + 4*grp + e, so the softmax state of a row lives
    // in the four lanes col, col + 16, col + 32, col + 48 and never crosses LDS.
    float4_t oacc[2 * NBV];
    float mrow = -INFINITY, lrow = 0.f;  // running max (log2 domain) and this lane's part of the sum
#pragma unroll
    for (int dt = 0; dt < 2 * NBV; ++dt) oacc[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    // A operands that remove the nibble offsets inside the P.V MFMAs: every entry -1032 (low
    // nibbles) or -1152 (high nibbles), so each output gains -offset * (sum of its weights)
    const half8_t bias_lo = {(_Float16)-kMagicV, (_Float16)-kMagicV, (_Float16)-kMagicV, (_Float16)-kMagicV,
                             (_Float16)-kMagicV, (_Float16)-kMagicV, (_Float16)-kMagicV, (_Float16)-kMagicV};
    const half8_t bias_hi = {(_Float16)-kMagicVHi, (_Float16)-kMagicVHi, (_Float16)-kMagicVHi, (_Float16)-kMagicVHi,
                             (_Float16)-kMagicVHi, (_Float16)-kMagicVHi, (_Float16)-kMagicVHi, (_Float16)-kMagicVHi};
    // kept in a register so that mask-and-insert compiles to one v_and_or_b32 (two literals
    // cannot share an instruction)
    uint32_t vmagic = 0x64006400u;
    asm volatile("" : "+v"(vmagic));
    const float c = p.scale_log2;
    // transposing V reads: lane col of 16-lane group grp reads 8 bytes (half col % 2) of the key
    // in P.V slot 8 grp + col / 2; it receives byte col of the 8 keys of its slots
    const int vkey = 4 * grp + ((col >> 1) & 3) + 16 * (col >> 3);
    const int vrd = vkey * kVc + 64 * ((vkey >> 4) & 1) + 8 * (col & 1);
    const int qi_row = min(R0 + min(col, max(R, 1) - 1), R_all - 1) / p.gqa;  // query of this lane's row

    // ---- Q^T as the B operand of Q.K: lane holds row `col`, head_dim 32*blk + 8*grp + 0..7
    // accumulator inputs: -1152 * block sum of row `col` of Q, in registers or (wide heads) at
    // s_cin[wh][blk][col]; Q^T fragments in registers or (head dim 512) at s_q[wh][blk][lane].
    // The LDS copies are written before the first barrier and read once per block and chunk.
    float4_t cneg[G::kCinLds ? 1 : NBK];
    half8_t qb[G::kQLds ? 1 : NBK];
    const int cin_off = 16 * (16 * NBK * (wh + HW * rgw) + col);
    const int q_off = 16 * (64 * NBK * (wh + HW * rgw) + lane);
    {
        const bool ok = col < R;
        const int r = min(R0 + (ok ? col : 0), R_all - 1);
        const _Float16 *qrow = p.q + (int64_t)(r / p.gqa) * p.q_s1 + (int64_t)(g * p.gqa + r % p.gqa) * p.q_s2 +
                               (int64_t)b * p.q_s3;
        uint4 qv[NBK];
#pragma unroll
        for (int blk = 0; blk < NBK; ++blk) qv[blk] = *reinterpret_cast<const uint4 *>(qrow + 32 * blk + 8 * grp);
#pragma unroll
        for (int blk = 0; blk < NBK; ++blk) {
            const half8_t qf = __builtin_bit_cast(half8_t, ok ? qv[blk] : make_uint4(0, 0, 0, 0));
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) sum += (float)qf[j];
            const float cb = -kMagicK * fold_rows(sum);  // block sum of row `col`, in every lane of the column
            if constexpr (G::kQLds) {
                if (part == 0) *reinterpret_cast<half8_t *>(s_q + q_off + 1024 * blk) = qf;
            } else {
                qb[blk] = qf;
            }
            if constexpr (G::kCinLds) {
                if (grp == 0 && part == 0)
                    *reinterpret_cast<float4_t *>(s_cin + cin_off + 256 * blk) = float4_t{cb, cb, cb, cb};
            } else {
                cneg[blk] = float4_t{cb, cb, cb, cb};
            }
        }
    }

    // ---- one chunk from LDS stage `buf`
    auto compute = [&](int buf, int64_t c0) __attribute__((always_inline)) {
        const uint8_t *ks = s_k + buf * kBk;
        const uint8_t *vs = s_v + buf * kBv;
        const uint8_t *dkw = ks + 2 * kKp + wh * kKh;  // d_K[block][key] of this head
        // (d_V is staged in P.V slot order: the key of slot 8*gg + jj is 4*gg + jj (jj < 4) or
        // 16 + 4*gg + jj - 4.)

        // the mask values of the lane's keys (keys past the segment end read its last one and
        // are hidden below) are fetched first, pinned here so that their latency overlaps Q.K
        float mpre[2][4];
        if constexpr (MSK) {
            if (p.mask) {
                const _Float16 *mr = p.mask + p.pos0 + (int64_t)b * p.m_s3 + (int64_t)qi_row * p.m_s1;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        mpre[kt][ii] = (float)mr[min(c0 + 16 * kt + 4 * grp + ii, c_end - 1)];
                        asm volatile("" : "+v"(mpre[kt][ii]));
                    }
            }
        }
        // the V^T bytes (one transposing read per block) are read first: their latency then
        // overlaps Q.K and the softmax
        int2_t btr[NBV];
#pragma unroll
        for (int j = 0; j < NBV; ++j) {
            // block blk of head wh is slot UV*wh + blk/2 (+ kTpcV for odd blk) of a cell
            const int blk = NBV * part + j;
            const int vslot = UV * wh + (blk >> 1) + kTpcV * (blk & 1);
            btr[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) int2_t *)(vs + vrd + 16 * vslot));
        }

        // ---- Q.K on the matrix cores: A = K (16 keys x 32 head_dim of one q8_0 block, codes as
        // binary16 1024 + (q + 128)), B = Q^T; d[ii] = score of key 16*kt + 4*grp + ii for row col
        // before the block scale
        // Blocks go in groups of four (all of them at head dim 128; three at 576), with a
        // scheduling fence between groups, so at most eight accumulators of raw scores are live.
        constexpr int kQg = NBK <= 4 ? NBK : (NBK % 4 == 0 ? 4 : 3);
        static_assert(NBK % kQg == 0, "Q.K block groups");
        float s[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) s[kt][ii] = 0.f;
#pragma unroll
        for (int b0 = 0; b0 < NBK; b0 += kQg) {
            float4_t dq[2][kQg], cin[kQg];
            half8_t qin[kQg];
#pragma unroll
            for (int j = 0; j < kQg; ++j) {
                if constexpr (G::kCinLds)
                    cin[j] = *reinterpret_cast<const float4_t *>(s_cin + cin_off + 256 * (b0 + j));
                else
                    cin[j] = cneg[b0 + j];
                if constexpr (G::kQLds)
                    qin[j] = *reinterpret_cast<const half8_t *>(s_q + q_off + 1024 * (b0 + j));
                else
                    qin[j] = qb[b0 + j];
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                // codes 8*grp .. 8*grp+7 of the block: plane grp / 2, half grp % 2 of the slot
                const uint8_t *kr = ks + (grp >> 1) * kKp + (16 * kt + col) * kKc + 8 * (grp & 1);
#pragma unroll
                for (int j = 0; j < kQg; ++j) {
                    const int blk = b0 + j;
                    const int kslot = UK * wh + (blk >> 1) + kTpcK * (blk & 1);
                    const uint2 w = *reinterpret_cast<const uint2 *>(kr + 16 * kslot);
                    const uint2 b0w = q8_biased(w.x), b1w = q8_biased(w.y);  // 1152 + q, exact
                    const uint4 ak = make_uint4(b0w.x, b0w.y, b1w.x, b1w.y);
                    dq[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ak), qin[j],
                                                                       cin[j], 0, 0, 0);
                }
            }
            // scores s[kt][ii] = sum over blocks of d_K * d
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int j = 0; j < kQg; ++j) {
                    const int blk = b0 + j;
                    const uint2 dk2 = *reinterpret_cast<const uint2 *>(dkw + blk * (2 * kCh) + 2 * (16 * kt + 4 * grp));
                    const half2_t d01 = h2v(dk2.x), d23 = h2v(dk2.y);
                    s[kt][0] = fmaf((float)d01[0], dq[kt][j][0], s[kt][0]);
                    s[kt][1] = fmaf((float)d01[1], dq[kt][j][1], s[kt][1]);
                    s[kt][2] = fmaf((float)d23[0], dq[kt][j][2], s[kt][2]);
                    s[kt][3] = fmaf((float)d23[1], dq[kt][j][3], s[kt][3]);
                }
            }
            if constexpr (NBK > kQg) __builtin_amdgcn_sched_barrier(0);
        }

        // the scores are complete here: without this pin the compiler defers the block sums
        // past the visibility branch below and keeps every raw-score accumulator live across it
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) asm volatile("" : "+v"(s[kt][ii]));
        // ---- visibility: whole chunk visible, or per element (chunk end, causal rule, mask)
        const bool full = !ROWS && (c0 + kCh <= c_end) && !p.mask && (p.q_pos0 < 0 || p.pos0 + c0 + kCh - 1 <= p.q_pos0);
        float cc = c;
        if (CAP && full) {
            // every key visible: only the soft-cap
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) s[kt][ii] = softcap_log2(s[kt][ii], p.cap_cs, p.cap_l2);
            cc = 1.0f;
        } else if (!full) {
            // in chunk-relative 32-bit terms: keys below n_in exist, keys up to lim are not after
            // the query (causal rule); mask reads clamp to the segment's last key
            const int n_in = (int)min((int64_t)kCh, c_end - c0);
            const int lim = p.q_pos0 < 0 ? kCh
                                         : (int)max((int64_t)-1, min((int64_t)kCh, p.q_pos0 + qi_row - p.pos0 - c0));
            // row lists: the loaders' flags of the lane's keys
            const int4 ok0 = ROWS ? *reinterpret_cast<const int4 *>(&s_ok[buf][4 * grp]) : make_int4(1, 1, 1, 1);
            const int4 ok1 = ROWS ? *reinterpret_cast<const int4 *>(&s_ok[buf][16 + 4 * grp]) : make_int4(1, 1, 1, 1);
            const int okk[2][4] = {{ok0.x, ok0.y, ok0.z, ok0.w}, {ok1.x, ok1.y, ok1.z, ok1.w}};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int kr = 16 * kt + 4 * grp + ii;
                    const bool vis = kr < n_in && kr <= lim && okk[kt][ii] != 0;
                    float x = CAP ? softcap_log2(s[kt][ii], p.cap_cs, p.cap_l2) : s[kt][ii] * c;
                    if (MSK && p.mask) x = fmaf(mpre[kt][ii], kLog2e, x);
                    s[kt][ii] = vis ? x : -INFINITY;
                }
            }
            cc = 1.0f;
        }

        // ---- online softmax of row `col` (exact: the max is raised whenever a chunk exceeds it)
        float mx;
        if (cc >= 0.f)
            mx = max3_nn(max3_nn(s[0][0], s[0][1], s[0][2]), max3_nn(s[0][3], s[1][0], s[1][1]),
                         max2_nn(s[1][2], s[1][3]));
        else
            mx = -min3_nn(min3_nn(s[0][0], s[0][1], s[0][2]), min3_nn(s[0][3], s[1][0], s[1][1]),
                          -max2_nn(-s[1][2], -s[1][3]));
        const float mt = fold_rows_max(mx) * (cc >= 0.f ? cc : -cc);
        if (__builtin_amdgcn_ballot_w64(mt > mrow)) {
            const float mnew = fmaxf(mt, mrow);
            const float a = (mnew > mrow) ? __builtin_amdgcn_exp2f(mrow - mnew) : 1.0f;
            mrow = mnew;
            lrow *= a;
#pragma unroll
            for (int dt = 0; dt < 2 * NBV; ++dt) oacc[dt] *= a;
        }
        const float msub = mrow == -INFINITY ? 0.f : mrow;
        half2_t pk[4];  // P of P.V slots 8*grp + 2u, 2u + 1 (keys 16*(u/2) + 4*grp + 2*(u%2) + 0, 1)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][2 * (u & 1)], cc, -msub));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][2 * (u & 1) + 1], cc, -msub));
            lrow += p0 + p1;
            pk[u] = half2_t{(_Float16)p0, (_Float16)p1};
        }

        // ---- P.V over the chunk's 32 keys, per V block: B = W^T with W = p * d_V in the slot
        // order above, A = V^T gathered from the staged raw bytes in the same order (byte `col`
        // of the block: element col as the low nibble, element col + 16 as the high one)
#pragma unroll
        for (int j = 0; j < NBV; ++j) {
            const int blk = NBV * part + j;
            const uint4 dv = *reinterpret_cast<const uint4 *>(vs + kVd + wh * kVh + blk * (2 * kCh) + 16 * grp);
            const uint4 wu = make_uint4(u32v(pk[0] * h2v(dv.x)), u32v(pk[1] * h2v(dv.y)),
                                        u32v(pk[2] * h2v(dv.z)), u32v(pk[3] * h2v(dv.w)));
            const half8_t wf = __builtin_bit_cast(half8_t, wu);
            const int2_t bt = btr[j];
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                // 1024 + n (low nibbles) and 1024 + 16 n (high nibbles, in place) of two bytes
                q4_nibbles_biased((uint32_t)bt[jj >> 1], (jj & 1) ? 0x0C030C02u : 0x0C010C00u, vmagic, lo[jj], hi[jj]);
            }
            oacc[2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8_t, make_uint4(lo[0], lo[1], lo[2], lo[3])), wf, oacc[2 * j], 0, 0, 0);
            oacc[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8_t, make_uint4(hi[0], hi[1], hi[2], hi[3])), wf, oacc[2 * j + 1], 0, 0, 0);
            oacc[2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bias_lo, wf, oacc[2 * j], 0, 0, 0);
            oacc[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bias_hi, wf, oacc[2 * j + 1], 0, 0, 0);
        }
    };

    for (int64_t ch = 0; ch < n_ch; ch += 2) {
        __syncthreads();
        compute(0, c_beg + ch * kCh);
        if (ch + 1 >= n_ch) break;
        __syncthreads();
        compute(1, c_beg + (ch + 1) * kCh);
    }

    // ---- partial of row `col`: the sums are folded over the four lanes of the row
    const float S = fold_rows(lrow);
    if (col < R) {
        const int rho = R0 + col, r = rho % p.gqa, i = rho / p.gqa;
        const int64_t row = (g * p.gqa + r) + (int64_t)p.n_head * (i + (int64_t)p.n_q * b);
        float *out = p.partials + ((int64_t)(p.slot0 + split) * p.n_rows + row) * kPs;
        if (grp == 0 && part == 0) {
            out[0] = (mrow == -INFINITY) ? -INFINITY : mrow * kLn2;
            out[1] = S;
        }
        // low nibbles: O = acc; high nibbles (16 (n - 8) after the offset): O = acc / 16
#pragma unroll
        for (int dt = 0; dt < 2 * NBV; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[2 + 16 * (2 * NBV * part + dt) + 4 * grp + e] = (dt & 1) ? oacc[dt][e] * 0.0625f : oacc[dt][e];
    }
}

// compute waves per head: two when dv = 512, where one wave's registers cannot hold the output
// of all sixteen V blocks beside Q; four for the 576 / 512 pair, whose LDS (Q fragments of 18
// blocks) leaves room for one workgroup per CU, so that each SIMD still runs one compute wave
// (every wave computes the whole Q.K: 0.38 of the HBM roofline against 0.29 with two; at
// 512 / 512, two workgroups per CU with two waves per head stay faster, 0.50 against 0.39)
template <int DK, int DV>
constexpr int kSplitV = DK == 576 ? 4 : DV >= 512 ? 2 : 1;

template <int DK, int DV, int HW, int RG, bool CAP, int MODE>
hipError_t launch_mma_c(const SegParams &p, hipStream_t s, int *occupancy) {
    constexpr int SV = kSplitV<DK, DV>;
    constexpr int kThreads = Geo<DK, DV, HW, SV, RG>::kThreads;
    if (occupancy)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy,
                                                            decode_mma_kernel<DK, DV, HW, SV, RG, CAP, MODE>, kThreads, 0);
    const int64_t blocks = (int64_t)p.n_splits * (p.n_head_kv / HW) * p.n_seq * decode_mma_row_groups(p);
    if (blocks > ((int64_t)1 << 31) - 1) return hipErrorInvalidValue;
    launch_seg(decode_mma_kernel<DK, DV, HW, SV, RG, CAP, MODE>, dim3((unsigned)blocks), dim3(kThreads), s, p);
    return hipGetLastError();
}

template <int DK, int DV, int HW, int RG>
hipError_t launch_mma(const SegParams &p, hipStream_t s, int *occupancy) {
    if (p.rows)
        return p.cap_l2 != 0.f ? launch_mma_c<DK, DV, HW, RG, true, kModeRows>(p, s, occupancy)
                               : launch_mma_c<DK, DV, HW, RG, false, kModeRows>(p, s, occupancy);
    if (p.mask)
        return p.cap_l2 != 0.f ? launch_mma_c<DK, DV, HW, RG, true, kModeMask>(p, s, occupancy)
                               : launch_mma_c<DK, DV, HW, RG, false, kModeMask>(p, s, occupancy);
    return p.cap_l2 != 0.f ? launch_mma_c<DK, DV, HW, RG, true, kModePlain>(p, s, occupancy)
                           : launch_mma_c<DK, DV, HW, RG, false, kModePlain>(p, s, occupancy);
}

}  // namespace

// A group of hw KV heads at head dims (dk, dv) has an instantiation when dk = dv, its two LDS
// stages stay near 110 KB (hw * d <= 1024) and its loader threads fill whole waves (hw * d / 64
// a multiple of 4); and for the 576 / 512 pair one head at a time.
static bool mma_group_ok(int dk, int dv, int hw) {
    if (dk == 576) return dv == 512 && hw == 1;
    if (dk != dv) return false;
    if (dk == 512) return hw == 1;  // one head and two workgroups per CU (Q in LDS)
    return (dk == 64 || dk == 128 || dk == 256) && (hw == 8 || hw == 4 || hw == 2 || hw == 1) && hw * dk <= 1024 &&
           (hw * dk / 64) % 4 == 0;
}

// More than 16 rows per KV head: a workgroup of fewer heads takes several row groups over one
// staged chunk, where that fits the register budget (row groups rg of hw heads; 0: none).
static int mma_multi_rows(int dk, int dv, int &hw) {
    if (dk == 64 && dv == 64) return hw = 4, 2;
    if (dk == 256 && dv == 256) return hw = 1, 4;
    if (dk == 512 && dv == 512) return hw = 1, 2;
    return 0;
}

// Row groups per workgroup of the cell-major decode launch for p.
static int mma_rg(const SegParams &p) {
    int hw = 0;
    const int rg = (int64_t)p.gqa * p.n_q > 16 ? mma_multi_rows(p.d, p.dv, hw) : 0;
    return (rg > 0 && hw == p.cell_hw) ? rg : 1;
}

int decode_mma_row_groups(const SegParams &p) {
    const int64_t n_rg = ((int64_t)p.gqa * p.n_q + 15) / 16;
    return (int)((n_rg + mma_rg(p) - 1) / mma_rg(p));
}

int decode_mma_heads(int dk, int dv, int n_head_kv, int R) {
    int hw = 0;
    if (R > 16 && mma_multi_rows(dk, dv, hw) > 0 && n_head_kv % hw == 0) return hw;
    for (int h : {8, 4, 2, 1})
        if (n_head_kv % h == 0 && mma_group_ok(dk, dv, h)) return h;
    return 0;
}

bool decode_mma_ok(const SegParams &p) {
    // rows per KV head: up to 8 at head dim 128 (the decode contract there), any number at the
    // other head dims (row groups of 16)
    const int64_t R = (int64_t)p.gqa * p.n_q;
    return mma_group_ok(p.d, p.dv, p.cell_hw) && R >= 1 && (p.d != kHeadDim || R <= kMaxRowsVec);
}

hipError_t launch_decode_mma(const SegParams &p, hipStream_t s, int *occupancy) {
    if (!decode_mma_ok(p)) return hipErrorInvalidValue;
    if (p.d == 576) return launch_mma<576, 512, 1, 1>(p, s, occupancy);
    const int rg = mma_rg(p);
    switch (p.d * 64 + p.cell_hw * 8 + rg) {
        case 64 * 64 + 8 * 8 + 1: return launch_mma<64, 64, 8, 1>(p, s, occupancy);
        case 64 * 64 + 4 * 8 + 1: return launch_mma<64, 64, 4, 1>(p, s, occupancy);
        case 64 * 64 + 4 * 8 + 2: return launch_mma<64, 64, 4, 2>(p, s, occupancy);
        case 128 * 64 + 8 * 8 + 1: return launch_mma<128, 128, 8, 1>(p, s, occupancy);
        case 128 * 64 + 4 * 8 + 1: return launch_mma<128, 128, 4, 1>(p, s, occupancy);
        case 128 * 64 + 2 * 8 + 1: return launch_mma<128, 128, 2, 1>(p, s, occupancy);
        case 256 * 64 + 4 * 8 + 1: return launch_mma<256, 256, 4, 1>(p, s, occupancy);
        case 256 * 64 + 2 * 8 + 1: return launch_mma<256, 256, 2, 1>(p, s, occupancy);
        case 256 * 64 + 1 * 8 + 1: return launch_mma<256, 256, 1, 1>(p, s, occupancy);
        case 256 * 64 + 1 * 8 + 4: return launch_mma<256, 256, 1, 4>(p, s, occupancy);
        case 512 * 64 + 1 * 8 + 1: return launch_mma<512, 512, 1, 1>(p, s, occupancy);
        case 512 * 64 + 1 * 8 + 2: return launch_mma<512, 512, 1, 2>(p, s, occupancy);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rkv
