// Matrix-core segment kernel for decode over cell-major binary16 K / V caches on gfx950, for a
// resident window, a lifted tail tile, or a unified pool addressed through a row list.
//
// Same partial as the other decode kernels (opencoti-llamafile patch 0070-rolling-kv, fattn.cu
// streaming_lse_kernel and the tail-partial op: M = max s_j, S = sum exp(s_j - M),
// VKQ = sum exp(s_j - M) v_j), and for the row-list form the semantics of llama.cpp PR
// #29510's flash_attn_ext_rows (ggml.h API comment) over kv_rows (a negative entry is padding
// and contributes nothing).  With binary16 data both contractions go straight to the matrix
// cores, without any conversion:
//
//   Q.K  D[key][row] = K (A: 16 keys x 32 head_dim, one 16-byte LDS read per lane) times Q^T
//        (B, rows >= R zero): v_mfma_f32_16x16x32_f16.  A lane then holds one query row for
//        four keys, so the softmax needs no LDS round trip and its probabilities are the B
//        operand of P.V as they stand.
//   P.V  O^T[d][row] = V^T (A: 16 head_dim x 16 keys) times P^T: v_mfma_f32_16x16x16_f16, with
//        V^T read by ds_read_b64_tr_b16 (16 lanes fetch four keys x sixteen head_dim values and
//        receive them transposed, one head_dim value of four keys per lane).
//
// Head dims 64, 128, 256 and 512 (dk = dv): a KV head group of HW heads (8, 8, 4, 2) keeps the
// cell at 1 or 2 KB per cache, and each head gets SV = 8 / HW waves (1, 1, 2, 4), each of which
// computes the head's Q.K (the same scores in every one of them) and 1 / SV of its P.V tiles.
// The 576 / 512 pair takes one KV head per workgroup (8 waves, 1152-byte K and 1024-byte V
// rows, the K stage with its own cell stride; a thread's last K unit slot lies past the cell
// and is left out).
//
// Workgroup = 8 waves, wave w = KV head g0 + w / SV (P.V part w % SV) of the (sequence, group of
// HW KV heads) pair of its current task; the kernel is persistent (work split below).  A chunk
// of 16 cells of the group (32 over a segment at head dim 64; HW x 2d bytes of K and of V per
// cell) is moved with 16-byte buffer loads into registers and from there into one of two LDS
// stages; two chunks are always in flight in registers, together with the chunk's mask values.  Row-list entries are read one
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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNT = 512;               // threads (8 waves)
constexpr int kMaxR = 8;               // query rows per KV head
constexpr uint32_t kNowhere = 0x80000000u;  // buffer offset past every range: reads zero
constexpr int kMaxPairs = 1024;        // (sequence, head group) pairs of one launch

// Geometry at Q / K head dim D (V: the same, or 512 with 576), over a segment of cells or
// (ROWS) a row list.
template <int D, bool ROWS = false>
struct G16 {
    static constexpr int DV = D == 576 ? 512 : D;        // V head dim
    static constexpr int HW = D == 576 ? 1 : D <= 128 ? 8 : 1024 / D;  // KV heads per workgroup
    static constexpr int SV = 8 / HW;                    // waves per KV head
    static constexpr int kRowK = 2 * D, kRowV = 2 * DV;  // bytes of one head's K / V row
    static constexpr int kCellK = HW * kRowK;            // bytes of one cell of the group: K
    static constexpr int kCell = HW * kRowV;             // and V
    // cells per chunk: 16 (one 16-key tile), and 32 over a segment at 64, where a cell is half
    // as large, so that a chunk keeps 64 KB of K and V (0.61 of the HBM roofline against 0.55
    // with 16); row lists keep 16, as a workgroup's run of a list's chunks is short and twice
    // the chunk made its first load and last compute cost more than they saved (41 against 37 us)
    static constexpr int kCh = (kCell >= 2048 || ROWS) ? 16 : 32;
    static constexpr int kTpc = kNT / kCh;               // threads per cell (32 or 16)
    static constexpr int kCpw = 64 / kTpc;               // cells staged by one wave (2 or 4)
    static constexpr int kS = kCell + 32, kSK = kCellK + 32;  // LDS cell strides (V, K): 8 mod 32 banks
    static constexpr int kStage = kCh * kS, kStageK = kCh * kSK;  // bytes of one LDS stage of V / K
    static constexpr int kM = kCell / 16 / kTpc;         // 16-byte units per thread and chunk: V
    static constexpr int kMK = (kCellK / 16 + kTpc - 1) / kTpc;  // and K (the last slot may fall past
    static constexpr bool kKPart = kMK * kTpc * 16 != kCellK;    // the cell, at 576: then unused)
    static constexpr int NB = D / 32;                    // Q.K steps of 32 head_dim values
    static constexpr int NT = DV / 16 / SV;              // P.V tiles of 16 head_dim values per wave
    static constexpr int kPs = 2 + DV;                   // partial row: M, S, VKQ[DV]
    // Q^T of a new pair rides in the stage registers up to 128; wider heads load it when the
    // pair starts (a workgroup meets one or two pairs)
    static constexpr bool kQStage = D <= 128;
    // resident waves per SIMD the registers allow: one workgroup per CU (at 64 with 16-cell
    // chunks two would fit the LDS, but within 128 registers the kernel spilled and ran 9%
    // slower over a segment and 15% slower over row lists)
    static constexpr int kWavesPerEu = 2;
    static_assert(kCell % (16 * kTpc) == 0 && HW * SV == 8 && kS % 128 == 32 && kSK % 128 == 32,
                  "thread and bank mapping");
};

// One chunk (task) in registers: this thread's K and V units, the mask value it stages,
// whether its cell is a key of the segment, the task's pair and first cell, the Q^T operand
// when the task starts a new pair, and (row lists) the pool rows the stage's next fetch uses.
struct Meta {
    int pair;   // (sequence, head group) pair of the task
    int newq;   // the task starts a new pair for this workgroup (q holds its Q^T)
    int64_t c0; // first cell
};
template <int D, bool ROWS>
struct Stage16 {
    uint4 k[G16<D, ROWS>::kMK], v[G16<D, ROWS>::kM];
    half8_t q[G16<D, ROWS>::kQStage ? G16<D, ROWS>::NB : 1];
    uint32_t mk;
    int ok;
    Meta meta;
    int rid[G16<D, ROWS>::kCpw], rin[G16<D, ROWS>::kCpw];  // row lists: raw pool rows of the wave's cells for
                                               // the next fetch, and whether they are keys
};

// Work split: the tasks are the chunks of every (sequence, head group) pair, numbered
// pair-major; workgroup j of G takes the contiguous run of tasks [jT/G, (j+1)T/G) of the T
// tasks, so it meets few pairs (one unless a pair boundary falls in its run).  A row list only
// counts up to its extent (1 + its last pool row, from a scan before the launch), so the
// padding at the end of the shorter lists costs nothing.  A workgroup writes its partial of
// each pair it meets into slot j, and M = -inf, S = 0 (no values) for the other pairs; when
// asked, workgroup 0 also writes each pair's slot range for the merge.
template <int D, int R, bool ROWS>
__global__ void __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(G16<D, ROWS>::kWavesPerEu)))
decode_mma16_kernel(const SegParams p) {
    using GD = G16<D, ROWS>;
    constexpr int kHW = GD::HW, SV = GD::SV, kRowK = GD::kRowK, kRowV = GD::kRowV, kS = GD::kS, kStage = GD::kStage;
    constexpr int kSK = GD::kSK, kStageK = GD::kStageK, kCellK = GD::kCellK, kMK = GD::kMK;
    constexpr int kM = GD::kM, NB = GD::NB, NT = GD::NT, kPs = GD::kPs;
    constexpr int kCh = GD::kCh, kTpc = GD::kTpc, kCpw = GD::kCpw, NU = kCh / 16;  // NU 16-key tiles per chunk
    // R > kMaxR: row groups of 16 (more rows per KV head than the persistent form takes, over a
    // segment): workgroup = (row group, split, head group, sequence), not persistent
    constexpr bool RGM = R > kMaxR;
    static_assert(!(RGM && ROWS), "row groups over segments only");
    __shared__ __attribute__((aligned(16))) uint8_t s_k[2 * kStageK];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[2 * kStage];
    __shared__ __attribute__((aligned(16))) int s_ok[2][kCh];                         // key is visible data
    __shared__ __attribute__((aligned(16))) _Float16 s_mask[2][RGM ? 16 : kMaxR][kCh];  // mask[row][key]
    __shared__ uint32_t s_off[RGM ? 1 : kMaxPairs + 1];  // first task of each pair; s_off[n_pairs] = tasks

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int head = wave / SV, part = wave % SV;  // KV head in the group, P.V part
    const int n_hgrp = p.n_head_kv / kHW;
    const int n_pairs = p.n_seq * n_hgrp;
    // row-group form: this workgroup's rows R0 .. R0 + RR - 1, pair, split and cells
    int R0 = 0, RR = R, rg_pair = 0;
    int64_t c_beg = 0, c_lim = p.n_cells;
    uint32_t G = (uint32_t)p.n_splits, j = blockIdx.x;
    if constexpr (RGM) {
        const int R_all = p.gqa * p.n_q, n_rg = (R_all + 15) >> 4;
        int bid = blockIdx.x;
        const int rg = bid % n_rg;
        bid /= n_rg;
        j = (uint32_t)(bid % p.n_splits);  // the split: partial slot slot0 + j
        bid /= p.n_splits;
        rg_pair = bid;  // (sequence, head group) pair: b * n_hgrp + hgrp
        R0 = 16 * rg;
        RR = min(16, R_all - R0);
        c_beg = (int64_t)j * p.cells_per_split;
        c_lim = min(p.n_cells, c_beg + (int64_t)p.cells_per_split);
    } else {
        if (j >= G) return;  // the grid is exactly G workgroups; slot j must exist
    }
    // ---- task offsets of the pairs: chunks of each pair up to its extent, scanned in LDS (one
    // wave per pair; its lanes read the kRowExtentParts = 64 pieces of the extent at once)
    static_assert(kRowExtentParts == 64, "one extent piece per lane");
    uint32_t n_tasks = 0, t_lo = 0, n_t = 0;  // all tasks, this workgroup's first and count
    if constexpr (RGM) {
        n_t = c_lim > c_beg ? (uint32_t)((c_lim - c_beg + kCh - 1) / kCh) : 0;
    } else {
    for (int pr = wave; pr < n_pairs; pr += kNT / 64) {
        int64_t ext = p.n_cells;
        if (p.row_extent) {
            int e = p.row_extent[(pr / n_hgrp) * kRowExtentParts + lane];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) e = max(e, __shfl_xor(e, o, 64));
            ext = min(ext, (int64_t)e);
        }
        if (lane == 0) s_off[pr + 1] = (uint32_t)((ext + kCh - 1) / kCh);
    }
    if (tid == 0) s_off[0] = 0;
    __syncthreads();
    for (int d = 1; d < n_pairs; d <<= 1) {  // inclusive scan of s_off[1 .. n_pairs]
        uint32_t add[2] = {0, 0};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pr = tid + u * kNT;
            if (pr < n_pairs && pr >= d) add[u] = s_off[pr + 1 - d];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pr = tid + u * kNT;
            if (pr < n_pairs) s_off[pr + 1] += add[u];
        }
        __syncthreads();
    }
    n_tasks = s_off[n_pairs];
    t_lo = (uint32_t)((uint64_t)j * n_tasks / G);
    n_t = (uint32_t)((uint64_t)(j + 1) * n_tasks / G) - t_lo;  // this workgroup's tasks
    if (p.pair_range && j == 0) {
        // workgroup of task t: the largest i with iT/G <= t, i.e. floor(((t + 1) G - 1) / T)
        for (int pr = tid; pr < n_pairs; pr += kNT) {
            const uint32_t lo = s_off[pr], hi = s_off[pr + 1];
            int2 r = make_int2(0, 0);
            if (hi > lo) {
                const int a = (int)(((uint64_t)(lo + 1) * G - 1) / n_tasks);
                const int b = (int)(((uint64_t)hi * G - 1) / n_tasks);
                r = make_int2(p.slot0 + a, p.slot0 + b + 1);
            }
            p.pair_range[pr] = r;
        }
    }
    }  // persistent form
    const int64_t n_cells = c_lim;  // keys end here (segment end, or this split's end)
    const int qi_row = (R0 + min(col, RR - 1)) / p.gqa;  // query position of this lane's row
    const int fcell = tid / kTpc, fsub = tid % kTpc;
    const int mrow = tid / kCh, mkey = tid % kCh;  // mask staging: row tid / kCh, key tid % kCh
    const bool mthread = p.mask != nullptr && tid < RR * kCh;

    // ---- partial of one pair for this lane's row (col < R): slot j.  Buffer stores of four
    // values each keep the store count per partial small and fixed (NT + 1), so that the waits
    // for the loads in flight, which count stores too, stay exact.
    const __amdgpu_buffer_rsrc_t rpart = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.partials + (int64_t)(p.slot0 + j) * p.n_rows * kPs), (short)0,
        (int)(p.n_rows * kPs * sizeof(float)), 0x00020000);
    // (acc null: the empty partial, M and S only -- the merge gives a segment with M = -inf
    // no weight and ignores its values)
    auto write_partial = [&](int pair, float M, float S, const float4_t *acc) __attribute__((always_inline)) {
        if (col >= RR) return;
        const int bb = pair / n_hgrp, g = (pair % n_hgrp) * kHW + head;
        const int r = (R0 + col) % p.gqa, i = (R0 + col) / p.gqa;
        const int row = (g * p.gqa + r) + p.n_head * (i + p.n_q * bb);
        const int base = row * kPs * (int)sizeof(float);
        if (grp == 0 && part == 0)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__builtin_bit_cast(uint32_t, M), __builtin_bit_cast(uint32_t, S)},
                                                  rpart, base, 0, 0);
        if (!acc) return;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[dt]), rpart,
                                                   base + (2 + 16 * (NT * part + dt) + 4 * grp) * (int)sizeof(float), 0, 0);
    };

    // ---- task k of this workgroup: its pair and first cell (k past the end: a phantom task
    // of the last pair with no keys).  Tasks are looked up in increasing order, so a cursor
    // over the pair offsets moves forward a step at a time (one for the fetches, one for the
    // row-list lookahead) instead of searching.
    int cur_f = 0, cur_r = 0, prev_fetch_pair = -1;
    auto task_at = [&](int &cur, uint32_t k, int &pair, int64_t &c0) __attribute__((always_inline)) {
        if constexpr (RGM) {
            pair = rg_pair;
            c0 = c_beg + (int64_t)(n_t > 0 ? min(k, n_t - 1) : 0) * kCh;
        } else {
            const uint32_t t = t_lo + (n_t > 0 ? min(k, n_t - 1) : 0);
            while (cur + 1 < n_pairs && s_off[cur + 1] <= t) ++cur;  // past empty pairs too
            pair = cur;
            c0 = (int64_t)(t - s_off[cur]) * kCh;
        }
    };
    // pool rows of the wave's cells kCpw*wave .. kCpw*wave + kCpw - 1 of task k's chunk, as read
    // (always from inside the list), and whether each is a key: entries past the list end (or
    // of a phantom task) are padding.  The raw value is only combined with the flag when the
    // next fetch uses it, so that waiting for it never waits for the loads issued after it.
    auto rows_of = [&](uint32_t k, int (&raw)[kCpw], int (&inl)[kCpw]) __attribute__((always_inline)) {
        int pair;
        int64_t c0;
        task_at(cur_r, k, pair, c0);
        const int32_t *__restrict__ rl = p.rows + (int64_t)(pair / n_hgrp) * p.rows_s;
        const int64_t c = c0 + kCpw * wave;
        const bool real = k < n_t;
#pragma unroll
        for (int i = 0; i < kCpw; ++i) {
            raw[i] = rl[min(c + i, n_cells - 1)];
            inl[i] = real && c + i < n_cells;
        }
    };

    // Q^T of pair `pair`: lane holds row `col` (rows >= R read row 0 and are never written),
    // head_dim 32*blk + 8*grp + 0..7
    auto load_q = [&](int pair, half8_t *q) __attribute__((always_inline)) {
        const int bb = pair / n_hgrp, hg = pair % n_hgrp;
        const int r = R0 + (col < RR ? col : 0);
        const int g = hg * kHW + head;
        const _Float16 *qrow = p.q + (int64_t)(r / p.gqa) * p.q_s1 + (int64_t)(g * p.gqa + r % p.gqa) * p.q_s2 +
                               (int64_t)bb * p.q_s3;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
            q[blk] = __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4 *>(qrow + 32 * blk + 8 * grp));
    };
    auto fetch = [&](Stage16<D, ROWS> &st, uint32_t k) __attribute__((always_inline)) {
        const bool real = k < n_t;
        int pair;
        int64_t c0;
        task_at(cur_f, k, pair, c0);  // fetches come in task order 0, 1, 2, ...
        st.meta.pair = pair;
        st.meta.c0 = c0;
        st.meta.newq = real && pair != prev_fetch_pair;
        prev_fetch_pair = pair;
        const int bb = pair / n_hgrp, hg = pair % n_hgrp;
        const uint8_t *kbase = p.k + (int64_t)(hg * kHW) * p.k_s2;
        const uint8_t *vbase = p.v + (int64_t)(hg * kHW) * p.v_s2;
        if constexpr (ROWS) {
            int r = -1;
#pragma unroll
            for (int i = 0; i < kCpw; ++i)
                if (fcell % kCpw == i) r = st.rin[i] ? st.rid[i] : -1;
            if (r >= p.n_pool) r = -1;  // outside the pool: read nothing, like padding
            st.ok = r >= 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)kbase, (short)0, (int)(p.n_pool * p.k_s1), 0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)vbase, (short)0, (int)(p.n_pool * p.v_s1), 0x00020000);
            // 24-bit products (pool rows below 2^20 and cell strides below 2^11 here), so the
            // offset is plain 32-bit arithmetic
            const uint32_t ko = r >= 0 ? __umul24((uint32_t)r, (uint32_t)p.k_s1) + 16u * fsub : kNowhere;
            const uint32_t vo = r >= 0 ? __umul24((uint32_t)r, (uint32_t)p.v_s1) + 16u * fsub : kNowhere;
#pragma unroll
            for (int m = 0; m < kMK; ++m)
                if (!GD::kKPart || 16 * (fsub + kTpc * m) < kCellK)
                    st.k[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16 * kTpc * m, 0, 0));
#pragma unroll
            for (int m = 0; m < kM; ++m)
                st.v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * kTpc * m, 0, 0));
            rows_of(k + 2, st.rid, st.rin);  // for this stage's next fetch
        } else {
            st.ok = real && c0 + fcell < n_cells;
            const int64_t nv = real ? max((int64_t)0, min((int64_t)kCh, n_cells - c0)) : 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(kbase + c0 * p.k_s1), (short)0, (int)(nv * p.k_s1), 0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(vbase + c0 * p.v_s1), (short)0, (int)(nv * p.v_s1), 0x00020000);
            const uint32_t ko = (uint32_t)fcell * (uint32_t)p.k_s1 + 16u * fsub;
            const uint32_t vo = (uint32_t)fcell * (uint32_t)p.v_s1 + 16u * fsub;
#pragma unroll
            for (int m = 0; m < kMK; ++m)
                if (!GD::kKPart || 16 * (fsub + kTpc * m) < kCellK)
                    st.k[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16 * kTpc * m, 0, 0));
#pragma unroll
            for (int m = 0; m < kM; ++m)
                st.v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * kTpc * m, 0, 0));
        }
        if (mthread) {
            const _Float16 *mb = p.mask + p.pos0 + (int64_t)bb * p.m_s3 + (int64_t)((R0 + mrow) / p.gqa) * p.m_s1;
            st.mk = __builtin_bit_cast(uint16_t, mb[min(c0 + mkey, n_cells - 1)]);
        }
        if constexpr (GD::kQStage) {
            if (st.meta.newq) load_q(pair, st.q);
        }
    };
    Meta mnext;                                 // the task stashed last: computed next
    half8_t qnext[GD::kQStage ? NB : 1];         // its Q^T when it starts a new pair
    auto stash = [&](const Stage16<D, ROWS> &st, int buf) __attribute__((always_inline)) {
        uint8_t *dk = s_k + buf * kStageK + fcell * kSK + 16 * fsub;
        uint8_t *dv = s_v + buf * kStage + fcell * kS + 16 * fsub;
#pragma unroll
        for (int m = 0; m < kMK; ++m)
            if (!GD::kKPart || 16 * (fsub + kTpc * m) < kCellK) *reinterpret_cast<uint4 *>(dk + 16 * kTpc * m) = st.k[m];
#pragma unroll
        for (int m = 0; m < kM; ++m) *reinterpret_cast<uint4 *>(dv + 16 * kTpc * m) = st.v[m];
        if (fsub == 0) s_ok[buf][fcell] = st.ok;
        if (mthread) s_mask[buf][mrow][mkey] = __builtin_bit_cast(_Float16, (uint16_t)st.mk);
        mnext = st.meta;
        if constexpr (GD::kQStage) {
            if (st.meta.newq) {
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) qnext[blk] = st.q[blk];
            }
        }
    };

    float4_t oacc[NT];  // O^T[16*(NT*part + dt) + 4*grp + e][col]
    float mrun = -INFINITY, lrow = 0.f;  // running max (log2 domain), this lane's part of the sum
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) oacc[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    const float c = p.scale_log2;
    half8_t qb[NB];
    int cur = -1;  // pair being accumulated
    // finish the current pair (a fixed number of stores, so the waits for the loads in flight
    // stay exact)
    auto flush = [&]() __attribute__((always_inline)) {
        if (cur >= 0) {
            const float S = fold_rows(lrow);
            write_partial(cur, mrun == -INFINITY ? -INFINITY : mrun * kLn2, S, oacc);
        }
    };
    // pairs with no task in this workgroup get the empty partial up front (row-group form: an
    // empty split)
    if constexpr (RGM) {
        if (n_t == 0) write_partial(rg_pair, -INFINITY, 0.f, nullptr);
    } else {
        for (int pr = 0; pr < n_pairs; ++pr) {
            const uint32_t lo = s_off[pr], hi = s_off[pr + 1];
            if (!(lo < hi && n_t > 0 && lo < t_lo + n_t && hi > t_lo)) write_partial(pr, -INFINITY, 0.f, nullptr);
        }
    }

    // ---- one task from LDS stage `buf` (its metadata and, for a new pair, its Q^T were taken
    // from the stage registers when the stage was stashed)
    auto compute = [&](int buf, const Meta &mt_) __attribute__((always_inline)) {
        if (mt_.newq) {
            flush();
            cur = mt_.pair;
            if constexpr (GD::kQStage) {
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) qb[blk] = qnext[blk];
            } else {
                load_q(cur, qb);
            }
            mrun = -INFINITY;
            lrow = 0.f;
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) oacc[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
        const uint8_t *kw = s_k + buf * kStageK + head * kRowK;  // this head's K row of cell j at kw + j*kSK
        const uint8_t *vw = s_v + buf * kStage + head * kRowV;

        // ---- Q.K: D[key 16*u + 4*grp + ii][row col] for each 16-key tile u of the chunk
        float4_t dq[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            dq[u] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                const uint4 a = *reinterpret_cast<const uint4 *>(kw + (16 * u + col) * kSK + 64 * blk + 16 * grp);
                dq[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), qb[blk], dq[u], 0, 0, 0);
            }
        }

        // ---- visibility: the key is data (chunk end, padding row), the causal rule, the mask
        float s[NU][4];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int k0 = 16 * u + 4 * grp;  // the lane's first key in the chunk
            const int4 okv = *reinterpret_cast<const int4 *>(&s_ok[buf][k0]);
            const uint2 mv = p.mask ? *reinterpret_cast<const uint2 *>(&s_mask[buf][min(col, RR - 1)][k0]) : make_uint2(0, 0);
            const half2_t m01 = __builtin_bit_cast(half2_t, mv.x), m23 = __builtin_bit_cast(half2_t, mv.y);
            const float mvals[4] = {(float)m01[0], (float)m01[1], (float)m23[0], (float)m23[1]};
            const int okk[4] = {okv.x, okv.y, okv.z, okv.w};
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                bool vis = okk[ii] != 0;
                if (!ROWS && p.q_pos0 >= 0 && p.pos0 + mt_.c0 + k0 + ii > p.q_pos0 + qi_row) vis = false;
                float x = p.cap_l2 != 0.f ? softcap_log2(dq[u][ii], p.cap_cs, p.cap_l2) : dq[u][ii] * c;
                if (p.mask) x = fmaf(mvals[ii], kLog2e, x);
                s[u][ii] = vis ? x : -INFINITY;
                mx = fmaxf(mx, s[u][ii]);
            }
        }

        // ---- online softmax of row `col` (exact: the max is raised whenever a chunk exceeds it)
        const float mt = fold_rows_max(mx);
        if (__builtin_amdgcn_ballot_w64(mt > mrun)) {
            const float mnew = fmaxf(mt, mrun);
            const float a = (mnew > mrun) ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.0f;
            mrun = mnew;
            lrow *= a;
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) oacc[dt] *= a;
        }
        const float msub = mrun == -INFINITY ? 0.f : mrun;
        half4_t pb[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            float pr[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                pr[ii] = __builtin_amdgcn_exp2f(s[u][ii] - msub);
                lrow += pr[ii];
            }
            pb[u] = half4_t{(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
        }

        // ---- P.V: A = V^T tile (head_dim 16*dt + col, keys 16*u + 4*grp + 0..3) by a transposing
        // read: lane col of group grp fetches key 16*u + 4*grp + col / 4, head_dim 16*dt +
        // 4*(col % 4) + 0..3 (this wave's tiles: dt = NT*part .. NT*part + NT - 1)
        const uint8_t *vr = vw + (4 * grp + (col >> 2)) * kS + 8 * (col & 3) + 32 * NT * part;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) {
                const short4_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) short4_t *)(vr + 16 * u * kS + 32 * dt));
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, t), pb[u], oacc[dt], 0, 0, 0);
            }
        }
    };

    // ---- pipeline: task k is computed from stage k % 2 right after a barrier; then the stage
    // of task k + 1 is stashed and task k + 3 fetched into its registers, so two tasks are in
    // flight in registers while one computes.  The barrier orders a stash after every wave's
    // reads of that stage (the task before) and a task's reads after its stash.  Tasks go in
    // pairs with no exit in between (a phantom task has no visible key), so that every path
    // into the loop head has the same loads in flight.
    if (n_t > 0) {
        Stage16<D, ROWS> sa, sb;  // tasks 2i (sa) and 2i + 1 (sb)
        sa.mk = sb.mk = 0;
        if constexpr (ROWS) {
            rows_of(0, sa.rid, sa.rin);
            rows_of(1, sb.rid, sb.rin);
        }
        fetch(sa, 0);
        fetch(sb, 1);
        stash(sa, 0);
        fetch(sa, 2);
        for (uint32_t k = 0; k < n_t; k += 2) {
            __syncthreads();
            compute(0, mnext);
            stash(sb, 1);
            fetch(sb, k + 3);
            __syncthreads();
            compute(1, mnext);
            stash(sa, 0);
            fetch(sa, k + 4);
        }
    }
    flush();
}

template <int D, int R, bool ROWS>
hipError_t launch16(const SegParams &p, hipStream_t s, int *occupancy) {
    if (occupancy)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, decode_mma16_kernel<D, R, ROWS>, kNT, 0);
    // persistent: n_splits workgroups in all, each covering every pair; row groups: one
    // workgroup per (row group, split, head group, sequence)
    int64_t blocks = p.n_splits;
    if (R > kMaxR)
        blocks *= (int64_t)((p.gqa * p.n_q + 15) / 16) * (p.n_head_kv / G16<D, ROWS>::HW) * p.n_seq;
    if (blocks > ((int64_t)1 << 31) - 1) return hipErrorInvalidValue;
    launch_seg(decode_mma16_kernel<D, R, ROWS>, dim3((unsigned)blocks), dim3(kNT), s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch16_d(const SegParams &p, hipStream_t s, int *occupancy) {
    const bool rows = p.rows != nullptr;
    switch (p.gqa * p.n_q) {
        case 1: return rows ? launch16<D, 1, true>(p, s, occupancy) : launch16<D, 1, false>(p, s, occupancy);
        case 2: return rows ? launch16<D, 2, true>(p, s, occupancy) : launch16<D, 2, false>(p, s, occupancy);
        case 3: return rows ? launch16<D, 3, true>(p, s, occupancy) : launch16<D, 3, false>(p, s, occupancy);
        case 4: return rows ? launch16<D, 4, true>(p, s, occupancy) : launch16<D, 4, false>(p, s, occupancy);
        case 5: return rows ? launch16<D, 5, true>(p, s, occupancy) : launch16<D, 5, false>(p, s, occupancy);
        case 6: return rows ? launch16<D, 6, true>(p, s, occupancy) : launch16<D, 6, false>(p, s, occupancy);
        case 7: return rows ? launch16<D, 7, true>(p, s, occupancy) : launch16<D, 7, false>(p, s, occupancy);
        case 8: return rows ? launch16<D, 8, true>(p, s, occupancy) : launch16<D, 8, false>(p, s, occupancy);
        default: return rows ? hipErrorInvalidValue : launch16<D, 16, false>(p, s, occupancy);  // row groups
    }
}

}  // namespace

int decode_mma16_chunk(int d, bool rows) {
    switch (d) {
        case 64: return rows ? G16<64, true>::kCh : G16<64>::kCh;
        case 128: return rows ? G16<128, true>::kCh : G16<128>::kCh;
        case 256: return rows ? G16<256, true>::kCh : G16<256>::kCh;
        case 512: return rows ? G16<512, true>::kCh : G16<512>::kCh;
        case 576: return rows ? G16<576, true>::kCh : G16<576>::kCh;
        default: return 16;
    }
}

int decode_mma16_heads(int d, int dv) {
    if (d == 576) return dv == 512 ? G16<576>::HW : 0;
    if (d != dv) return 0;
    switch (d) {
        case 64: return G16<64>::HW;
        case 128: return G16<128>::HW;
        case 256: return G16<256>::HW;
        case 512: return G16<512>::HW;
        default: return 0;
    }
}

bool decode_mma16_ok(const SegParams &p) {
    const int R = p.gqa * p.n_q;
    const int hw = decode_mma16_heads(p.d, p.dv);
    // more than 8 rows per KV head: row groups of 16 over a segment at the head dims other than
    // 128 (where such calls are prefill, which has a kernel of its own)
    const bool row_groups = R > kMaxR && !p.rows && p.d != kHeadDim;
    if (hw == 0 || p.cell_hw != hw || R < 1 || (R > kMaxR && !row_groups) || p.n_head_kv % hw != 0) return false;
    if (!row_groups && (int64_t)p.n_seq * (p.n_head_kv / hw) > kMaxPairs) return false;
    // row lists address the pool with 32-bit buffer offsets
    if (p.rows && (p.n_pool <= 0 || p.n_pool * p.k_s1 >= ((int64_t)1 << 31) || p.n_pool * p.v_s1 >= ((int64_t)1 << 31) ||
                   p.k_s1 >= (1 << 24) || p.v_s1 >= (1 << 24)))
        return false;
    return true;
}

hipError_t launch_decode_mma16(const SegParams &p, hipStream_t s, int *occupancy) {
    if (!decode_mma16_ok(p)) return hipErrorInvalidValue;
    switch (p.d) {
        case 64: return launch16_d<64>(p, s, occupancy);
        case 128: return launch16_d<128>(p, s, occupancy);
        case 256: return launch16_d<256>(p, s, occupancy);
        case 512: return launch16_d<512>(p, s, occupancy);
        case 576: return launch16_d<576>(p, s, occupancy);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rkv
