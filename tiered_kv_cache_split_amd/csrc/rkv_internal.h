// Internal interface between the host runtime (rkv_runtime.cpp) and the gfx950 kernels
// (rkv_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

constexpr int kHeadDim = 128;          // d == dv for every kernel here
constexpr int kPartialStride = 2 + kHeadDim;
constexpr int kMaxRowsVec = 8;         // vector kernel: n_q * gqa rows per KV head
constexpr int kChunk = 64;             // cells per wave iteration in the vector kernel

enum { T_F32 = 0, T_F16 = 1, T_Q4_0 = 2, T_Q8_0 = 8 };

// One device-resident key segment processed by one kernel launch.
struct SegParams {
    // queries: element strides of query i, head h and sequence b
    const _Float16 *q;
    int64_t q_s1, q_s2, q_s3;
    // keys/values of the segment: byte strides per cell and per KV head
    const uint8_t *k, *v;
    int64_t k_s1, k_s2, v_s1, v_s2;
    // optional row list (unified pool): key j of sequence b is cell rows[j + rows_s*b]
    const int32_t *rows;
    int64_t rows_s;
    int64_t n_pool;    // row lists: cells of the pool the rows index
    // row lists (optional, device): per sequence, kRowExtentParts values whose maximum is 1 +
    // the last list index holding a pool row
    const int32_t *row_extent;
    // optional additive binary16 mask: element strides of query i and sequence b;
    // column = pos0 + j (global key position)
    const _Float16 *mask;
    int64_t m_s1, m_s3;
    int64_t n_cells;   // keys in the segment
    int64_t pos0;      // global position of key 0
    int64_t q_pos0;    // >= 0: causal, query i at q_pos0 + i; -1: none
    int cells_per_split, n_splits;
    int n_head, n_head_kv, n_q, n_seq, gqa;
    float scale_log2;  // scale * log2(e)
    // logit soft-cap: the score becomes cap_l2 * tanh(cap_cs * <q, k>) in the exp2 domain
    // (cap_cs = scale / c, cap_l2 = c * log2(e)); cap_l2 = 0: no cap
    float cap_cs, cap_l2;
    float *partials;   // [slot][n_rows][2 + d]
    int slot0;         // first partial slot used by this segment
    int64_t n_rows;    // n_head * n_q * n_seq
    int cell_hw;       // > 0: cell-major kernel, cell_hw KV heads (packed per cell) per workgroup
    // optional (device, persistent binary16 kernel): receives, per (sequence, head group) pair,
    // the slot range [x, y) holding that pair's partials; slots outside it are not written
    // for the pair beyond M = -inf, S = 0
    int2 *pair_range;
    // optional: events the segment kernel's own dispatch records at its start and end
    hipEvent_t ev_start, ev_stop;
    // head dims of Q/K (d) and V (dv): 128 for every kernel but the decode kernel for other
    // head dims (dk = dv in 64, 256, 512, or dk = 576 with dv = 512)
    int d = kHeadDim;
    int dv = kHeadDim;
};

// Launch a segment kernel; with timing events set, the dispatch itself records them, so the
// interval covers the kernel alone.
template <typename F, typename... Args>
inline void launch_seg(F kernel, dim3 grid, dim3 block, hipStream_t s, const SegParams &p, Args... args) {
    if (p.ev_start)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, p.ev_start, p.ev_stop, 0, p, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, s, p, args...);
}

// KV heads per workgroup of the cell-major kernels for these head dims (dk, dv) and these
// types (0: no instantiation): a workgroup owns that many heads, packed inside each cell, over a
// cell range.
int cell_heads(int dk, int dv, int k_type, int v_type, int n_head_kv, int R, bool rows);
// Resident workgroups per CU of the cell-major kernel selected by p.cell_hw (at least 1).
int cell_blocks_per_cu(const SegParams &p, int k_type, int v_type);

// Launches; every function returns a hipError_t and checks nothing the host has not.
// Which decode kernel launch_decode_segment will run for p (enum rkv_kernel_variant).
int decode_kernel_variant(const SegParams &p, int k_type, int v_type);
hipError_t launch_decode_segment(const SegParams &p, int k_type, int v_type, hipStream_t s);
// Matrix-core decode kernel for cell-major q8_0 K / q4_0 V at head dims 64, 128, 256 and 512
// (dk = dv) and 576 / 512 with p.cell_hw KV heads per workgroup and up to 16 query rows per KV head per
// workgroup (more in row groups; at most 8 in all at head dim 128) (decode_mma_ok); with `occupancy` set it
// reports resident workgroups per CU instead of launching.  decode_mma_heads gives the group
// size it takes for n_head_kv heads at head dims (dk, dv) with R rows per KV head (0: none).
int decode_mma_heads(int dk, int dv, int n_head_kv, int R);
bool decode_mma_ok(const SegParams &p);
// Workgroups per (split, head group, sequence) of the cell-major decode launch: blocks of the
// row groups of 16 query rows per KV head that one workgroup takes together.
int decode_mma_row_groups(const SegParams &p);
hipError_t launch_decode_mma(const SegParams &p, hipStream_t s, int *occupancy);
// The binary16 matrix-core decode kernel (windows, tail tiles and row lists) over groups of
// cell-major KV heads (8 at head dims 64 and 128, 4 at 256, 2 at 512) with gqa * n_q <= 8 rows
// per head; the same occupancy convention.
bool decode_mma16_ok(const SegParams &p);
// KV heads per cell group of the binary16 matrix-core kernel at head dims (d, dv) (0: none),
// and the cells of one of its tasks (chunks) at head dim d over a segment or a row list.
int decode_mma16_heads(int d, int dv);
int decode_mma16_chunk(int d, bool rows);
// Workgroups per (split, head group, sequence) of a non-persistent cell-major launch for p: its
// blocks of row groups.
int cell_row_groups(const SegParams &p, int k_type, int v_type);
// Whether the decode kernel for p is the persistent one: n_splits workgroups then take equal
// contiguous runs of the 16-cell chunks of all (sequence, head group) pairs, numbered
// pair-major, and cells_per_split is unused.
bool decode_kernel_persistent(const SegParams &p, int k_type, int v_type);
hipError_t launch_decode_mma16(const SegParams &p, hipStream_t s, int *occupancy);
// The matrix-core prefill kernel takes dk = dv = 128 or 64.
bool prefill_head_dims_ok(int d, int dv);
hipError_t launch_prefill_segment(const SegParams &p, int k_type, int v_type, hipStream_t s);
// Blocks the prefill kernel uses per (q tile, KV head) along the key axis.
int prefill_rows_per_block();
int prefill_keys_per_iter();
int prefill_blocks_per_cu();  // workgroups of the prefill kernel resident per CU (LDS bound)
// Optional per-row segment ranges for the merge: row r merges slots pair_range[pair(r)] with
// pair(r) = (r / rows_per_seq) * n_hgrp + ((r % n_head) / heads_per_pair), clamped to n_seg.
struct MergeRange {
    const int2 *pair_range;
    int n_head, heads_per_pair, n_hgrp;
    int64_t rows_per_seq;
};
hipError_t launch_merge(const float *partials, int n_seg, int64_t n_rows, float *o, float *lse,
                        float *partial_out, hipStream_t s, const MergeRange *range = nullptr);
// The same merge for partial rows of 2 + dv floats (dv = 64, 128, 256, 512), up to 1024
// segments: up to four segments per thread over 16-value parts of each row.  With
// partial_out the merged (M, S, VKQ) rows go there instead of o / lse.
hipError_t launch_merge_parts(const float *partials, int n_seg, int64_t n_rows, int dv, float *o, float *lse,
                              hipStream_t s, float *partial_out = nullptr);
// Writes (M=-inf, S=0, VKQ=0) for n_rows rows of 2 + dv floats into partial slot 0.
hipError_t launch_empty_partials(float *partials, int64_t n_rows, hipStream_t s, int dv = kHeadDim);
// Row-list extents in kRowExtentParts pieces per sequence: the maximum of
// extent[b * kRowExtentParts + 0 .. kRowExtentParts - 1] is 1 + the last index j < n_kv with
// rows[j + rows_s*b] >= 0, or 0 (n_seq sequences)
constexpr int kRowExtentParts = 64;  // one wave's lanes (the binary16 kernel reads them so)
hipError_t launch_row_extent(const int32_t *rows, int64_t rows_s, int64_t n_kv, int n_seq, int32_t *extent, hipStream_t s);
hipError_t launch_uva_read(const void *host_src, void *dst, int64_t nbytes, hipStream_t s);
// Bulk copy kernel over pinned host memory (source and destination 8-byte aligned).
hipError_t launch_lift_copy(const void *host_src, void *dst, int64_t nbytes, hipStream_t s);
hipError_t launch_dequant_rows(const void *src, int type, int form, int64_t n_rows, int n_values, int64_t row_stride,
                               float *dst, hipStream_t s);

// Head dims other than 128 (rkv_decode_hd.hip): the vector decode kernel (any gqa * n_q, row
// lists) and the merge of partials with row stride 2 + dv.
bool head_dim_supported(int d);              // one tensor's head dim: 64, 128, 256, 512 or 576
bool head_dims_supported(int dk, int dv);   // a (Q/K, V) pair: equal in 64..512, or 576 / 512
hipError_t launch_decode_hd(const SegParams &p, int k_type, int v_type, hipStream_t s);
hipError_t launch_merge_hd(const float *partials, int n_seg, int64_t n_rows, int dv, float *o, float *lse,
                           hipStream_t s);

// Device-side block cache (rkv_bcache.hip): residency map arrays, all device memory.
constexpr int kBcCtl = 16;  // [0] epoch [1] hand [2] pages placed by the last call [3] overflow;
                            // u64 at [4] misses, [6] lookups, [8] calls
struct BcMap {
    int32_t *page_table;  // (n_pages) page -> slot, -1 absent (-2 while a resolve claims it)
    int32_t *slot_page;   // (n_slots) slot -> page, -1 free
    int32_t *slot_stamp;  // (n_slots) epoch of the call that last used the slot
    int32_t *slot_ref;    // (n_slots) clock reference bit
    int32_t *miss_page;   // (n_slots) pages missed by the last call, in claim order
    int32_t *miss_slot;   // (n_slots) their slots
    int32_t *ctl;         // (kBcCtl)
    int64_t n_pages, n_slots;
    int page_size;
};
hipError_t launch_bc_reset(const BcMap &m, hipStream_t s);
// Resolve a selection (int32 cells [n_seq][n_sel], -1 padding), copy the missed pages from the
// host copy's device view into their slots, and (rows != NULL) write each cell's slot-pool row.
hipError_t launch_bc_resolve(const BcMap &m, const int32_t *sel, int64_t n_sel, int n_seq, const uint8_t *host_k,
                             const uint8_t *host_v, uint8_t *pool_k, uint8_t *pool_v, int64_t k_page_bytes,
                             int64_t v_page_bytes, int32_t *rows, hipStream_t s);
hipError_t launch_bc_append(const BcMap &m, const void *k_cell, const void *v_cell, int64_t k_cell_bytes,
                            int64_t v_cell_bytes, int64_t cell, uint8_t *host_k, uint8_t *host_v, uint8_t *pool_k,
                            uint8_t *pool_v, int64_t k_s1, int64_t v_s1, hipStream_t s);

// Tail partial on the host cores (rkv_host_tail.cpp).  Every pointer is host memory.
struct HostTailArgs {
    const uint16_t *q;        // binary16 queries; element strides of query i and head h
    int64_t q_s1, q_s2;
    const uint8_t *k, *v;     // K/V rows of the segment; byte strides per cell and KV head
    int64_t k_s1, k_s2, v_s1, v_s2;
    int k_type, v_type;
    const uint16_t *mask;     // additive binary16, column j = segment cell j; element stride
    int64_t m_s1;             // of query i; NULL: all visible
    int64_t n_cells;          // keys in the segment
    int64_t kv_pos0;          // global position of cell 0 (causal rule)
    int64_t q_pos0;           // >= 0: query i at q_pos0 + i sees positions <= its own
    int n_head, n_head_kv, n_q;
    float scale, softcap;     // softcap 0: none
    float *partial;           // [n_head * n_q][2 + dv], row h + n_head * i
    int d = kHeadDim;         // head dims of Q/K and V: equal in 64..512, or 576 / 512
    int dv = kHeadDim;
};
bool host_tail_supported();          // the CPU has AVX2, FMA and F16C
int host_tail_threads(int requested);  // requested > 0, else the hardware threads (<= 16)
// May throw std::bad_alloc (the chunk partials); thread creation failures are absorbed.
void host_tail_partial(const HostTailArgs &a, int n_threads);

}  // namespace rkv
