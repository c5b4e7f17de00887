// Host runtime of librkv: the C ABI declared in include/rkv.h.
//
// Responsibilities: argument validation (before any device work), the segment planner
// (device window split-K, tail tiles that never straddle wc, global mask offsets), the
// tail lift pipeline (persistent grow-only scratch ring, context-owned copy stream,
// pre-created events, double buffer) and the partials workspace.
//
// Sources: opencoti-llamafile patch 0070-rolling-kv (fattn.cu ggml_cuda_streaming_flash_attn:
// window and tail tiled separately, mask sliced at the global offset, copy stream with
// copy_done/compute_done events created outside graph capture, an entry event that orders
// the copy stream after earlier compute -- bug-255) and patch
// 0102-fattn-bulk-h2d-scratch-ring (bulk raw-byte lift of a host tail into a persistent
// per-slot scratch ring sized for the worst-case tile, never allocated inside capture).
#include "rkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "rkv_internal.h"

using namespace rkv;

namespace {

thread_local std::string g_err;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(RKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define RKV_HIP(call)                                              \
    do {                                                           \
        hipError_t e_ = (call);                                    \
        if (e_ != hipSuccess) return hip_fail(e_, #call);          \
    } while (0)

constexpr int kMaxSlots = 4;
constexpr int kMaxLiftTiming = 64;
constexpr int kMaxKernelTiming = 4096;

int64_t type_block_bytes(int t) {
    switch (t) {
        case RKV_TYPE_F16: return 2;
        case RKV_TYPE_F32: return 4;
        case RKV_TYPE_Q8_0: return 34;
        case RKV_TYPE_Q4_0: return 18;
        default: return 0;
    }
}
// Bytes of one row of d values (d a multiple of 32).
int64_t row_bytes(int t, int64_t d = kHeadDim) {
    switch (t) {
        case RKV_TYPE_F16: return 2 * d;
        case RKV_TYPE_Q8_0: return d / 32 * 34;
        case RKV_TYPE_Q4_0: return d / 32 * 18;
        default: return 0;
    }
}

enum class Mem { Device, PinnedHost, Other };

Mem pointer_kind(const void *p) {
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof a);
    hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of probing an unknown pointer
        return Mem::Other;
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) return Mem::Device;
    if (a.type == hipMemoryTypeHost) return Mem::PinnedHost;
    return Mem::Other;
}

int check_device_ptr(const void *p, const char *name) {
    if (!p) return fail(RKV_ERR_ARG, "%s is NULL", name);
    if (pointer_kind(p) != Mem::Device) return fail(RKV_ERR_ARG, "%s is not device memory", name);
    return RKV_OK;
}

// K/V tensor [128, n_cells, n_head_kv, 1] with contiguous rows (any_d: head dim 64, 128, 256,
// 512 or 576; which pairs of K and V dims go together is checked by the caller).
int check_kv(const rkv_tensor *t, const char *name, bool is_k, bool any_d = false) {
    if (!t) return fail(RKV_ERR_ARG, "%s is NULL", name);
    const bool ok_type = is_k ? (t->type == RKV_TYPE_F16 || t->type == RKV_TYPE_Q8_0)
                              : (t->type == RKV_TYPE_F16 || t->type == RKV_TYPE_Q4_0);
    if (!ok_type) return fail(RKV_ERR_UNSUPPORTED, "%s: type %d not supported", name, t->type);
    if (any_d ? !head_dim_supported((int)std::min<int64_t>(t->ne[0], 1 << 20)) : t->ne[0] != kHeadDim)
        return fail(RKV_ERR_UNSUPPORTED, "%s: head dim %lld not supported here", name, (long long)t->ne[0]);
    if (t->ne[1] < 0 || t->ne[2] <= 0 || t->ne[3] != 1)
        return fail(RKV_ERR_ARG, "%s: bad shape [%lld,%lld,%lld,%lld]", name, (long long)t->ne[0],
                    (long long)t->ne[1], (long long)t->ne[2], (long long)t->ne[3]);
    if (t->ne[1] >= (int64_t)1 << 31) return fail(RKV_ERR_UNSUPPORTED, "%s: more than 2^31 cells", name);
    if (t->nb[0] != type_block_bytes(t->type)) return fail(RKV_ERR_ARG, "%s: rows must be contiguous (nb[0])", name);
    const int64_t rb = row_bytes(t->type, t->ne[0]);
    if (t->ne[1] > 1 && t->nb[1] < rb) return fail(RKV_ERR_ARG, "%s: nb[1] smaller than a row", name);
    if (t->ne[2] > 1 && t->nb[2] < rb) return fail(RKV_ERR_ARG, "%s: nb[2] smaller than a row", name);
    // the head-dim-128 kernels read rows in 8-byte pieces, the kernel for other head dims in
    // 4-byte words (every row size there is a multiple of 4 bytes)
    const int al = t->ne[0] == kHeadDim ? 8 : 4;
    if ((t->nb[1] | t->nb[2]) % al != 0 || ((uintptr_t)t->data) % al != 0)
        return fail(RKV_ERR_UNSUPPORTED, "%s: data and nb[1], nb[2] must be multiples of %d bytes", name, al);
    if (t->nb[1] >= ((int64_t)1 << 25) || t->nb[1] < 0 || t->nb[2] < 0)
        return fail(RKV_ERR_UNSUPPORTED, "%s: cell stride beyond 32 MiB", name);
    if (t->ne[1] > 0 && !t->data) return fail(RKV_ERR_ARG, "%s: data is NULL", name);
    return RKV_OK;
}

int check_q(const rkv_tensor *q, bool allow_seq, bool any_d = false) {
    if (!q || !q->data) return fail(RKV_ERR_ARG, "q is NULL");
    if (q->type != RKV_TYPE_F16) return fail(RKV_ERR_UNSUPPORTED, "q must be F16");
    if (any_d ? !head_dim_supported((int)std::min<int64_t>(q->ne[0], 1 << 20)) : q->ne[0] != kHeadDim)
        return fail(RKV_ERR_UNSUPPORTED, "q head dim %lld not supported here", (long long)q->ne[0]);
    if (q->ne[1] <= 0 || q->ne[2] <= 0 || q->ne[3] <= 0) return fail(RKV_ERR_ARG, "q: bad shape");
    if (!allow_seq && q->ne[3] != 1) return fail(RKV_ERR_ARG, "q: ne[3] must be 1");
    if (q->nb[0] != 2) return fail(RKV_ERR_ARG, "q rows must be contiguous");
    if ((q->nb[1] | q->nb[2] | q->nb[3]) % 4 != 0 || ((uintptr_t)q->data) % 4 != 0)
        return fail(RKV_ERR_UNSUPPORTED, "q data and strides must be multiples of 4 bytes");
    return check_device_ptr(q->data, "q");
}

int check_mask(const rkv_tensor *m, int64_t n_kv, int64_t n_q, int64_t n_seq) {
    if (!m) return RKV_OK;
    if (!m->data) return fail(RKV_ERR_ARG, "mask data is NULL");
    if (m->type != RKV_TYPE_F16) return fail(RKV_ERR_UNSUPPORTED, "mask must be F16");
    if (m->nb[0] != 2) return fail(RKV_ERR_ARG, "mask columns must be contiguous");
    if (m->ne[0] < n_kv || m->ne[1] < n_q)
        return fail(RKV_ERR_ARG, "mask [%lld,%lld] smaller than [n_kv=%lld, n_q=%lld]", (long long)m->ne[0],
                    (long long)m->ne[1], (long long)n_kv, (long long)n_q);
    if (m->ne[3] != 1 && m->ne[3] != n_seq) return fail(RKV_ERR_ARG, "mask ne[3] must be 1 or n_seq");
    if ((m->nb[1] | m->nb[3]) % 2 != 0) return fail(RKV_ERR_ARG, "mask strides must be even");
    return check_device_ptr(m->data, "mask");
}

int same_kv_shape(const rkv_tensor *a, const rkv_tensor *b, const char *what) {
    if (a->type != b->type || a->ne[2] != b->ne[2])
        return fail(RKV_ERR_ARG, "%s: window and tail disagree in type or n_head_kv", what);
    return RKV_OK;
}

}  // namespace

// Decode tails up to this many bytes (K plus V) are read in place under RKV_LIFT_AUTO: below
// it the in-place read beat the copy-kernel lift on the 128-dim decode (1.7 MB q8_0 / q4_0
// tail: 56 against 82 us per call; 4.2 MB binary16: 107 against 121 us), above it the two
// trade places (16.8 MB binary16: 361 against 347 us).
constexpr int64_t kDirectTailMaxDefault = (int64_t)8 << 20;

struct rkv_ctx {
    int device = 0;
    int n_cu = 256;
    hipStream_t copy_stream = nullptr;
    hipEvent_t copy_done[kMaxSlots] = {};
    hipEvent_t compute_done[kMaxSlots] = {};
    hipEvent_t entry = nullptr;
    hipEvent_t lift_t0[kMaxLiftTiming] = {}, lift_t1[kMaxLiftTiming] = {};
    bool lift_timing = false;
    int n_lift_timed = 0;
    // opt-in timing of segment-kernel launches (events on the launching stream)
    std::vector<hipEvent_t> kt0, kt1;
    bool kernel_timing = false;
    int n_kernel_timed = 0;
    void *scr_k[kMaxSlots] = {};
    void *scr_v[kMaxSlots] = {};
    size_t cap_k[kMaxSlots] = {};
    size_t cap_v[kMaxSlots] = {};
    int n_slots = 2;
    float *partials = nullptr;
    size_t partials_cap = 0;  // floats
    int32_t *row_extent = nullptr;  // row lists: per-sequence extents for the persistent kernel
    size_t row_extent_cap = 0;      // bytes
    int2 *pair_range = nullptr;     // row lists: slot range of each pair's partials (up to 1024 pairs)
    size_t pair_range_cap = 0;      // bytes
    int lift_mode = RKV_LIFT_AUTO;
    // RKV_LIFT_AUTO reads a decode tail of at most this many bytes (K plus V) in place
    int64_t direct_tail_max = kDirectTailMaxDefault;
    int splits_override = 0;
    float softcap = 0.f;  // logit soft-cap of later calls (0: none)
    // host tail partial (RKV_TAIL_HOST): pinned staging of Q, the tail's mask columns and the
    // partial; host_in marks Q/mask on the host, host_up the partial's upload
    int tail_mode = RKV_TAIL_LIFT;
    int host_threads = 0;
    void *hq = nullptr, *hmask = nullptr, *hpart = nullptr;
    size_t hq_cap = 0, hmask_cap = 0, hpart_cap = 0;
    hipEvent_t host_in = nullptr, host_up = nullptr;
    bool host_up_pending = false;
    rkv_stats stats = {};
};

struct rkv_bcache {
    int device = 0;
    BcMap m{};
    void *map_mem = nullptr;
    uint8_t *pool_k = nullptr, *pool_v = nullptr;
    uint8_t *view_k = nullptr, *view_v = nullptr;  // device views of the caller's pinned host copy
    int k_type = 0, v_type = 0;
    int64_t d = 0, n_cells = 0, n_head_kv = 0, k_s1 = 0, v_s1 = 0, k_row = 0, v_row = 0;
    int64_t page_size = 0, n_slots = 0;
};

namespace {

bool stream_capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st == hipStreamCaptureStatusActive;
}

// Logit soft-cap constants of a call: s -> c * tanh(scale * qk / c), in the exp2 domain.
void fill_softcap(SegParams &p, const rkv_ctx *ctx, float scale) {
    if (ctx->softcap > 0.f) {
        p.cap_cs = scale / ctx->softcap;
        p.cap_l2 = ctx->softcap * 1.4426950408889634f;
    } else {
        p.cap_cs = p.cap_l2 = 0.f;
    }
}

int ensure_device(rkv_ctx *ctx) {
    int cur = -1;
    RKV_HIP(hipGetDevice(&cur));
    if (cur != ctx->device) RKV_HIP(hipSetDevice(ctx->device));
    return RKV_OK;
}

int grow(void **buf, size_t *cap, size_t need, hipStream_t s) {
    if (*cap >= need) return RKV_OK;
    if (stream_capturing(s))
        return fail(RKV_ERR_CAPTURE, "workspace must grow to %zu bytes while the stream is capturing; call rkv_reserve first", need);
    if (*buf) {
        RKV_HIP(hipDeviceSynchronize());  // earlier work may still read the old buffer
        RKV_HIP(hipFree(*buf));
        *buf = nullptr;
        *cap = 0;
    }
    hipError_t e = hipMalloc(buf, need);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *buf = nullptr;
        return fail(RKV_ERR_NOMEM, "hipMalloc(%zu) failed", need);
    }
    *cap = need;
    return RKV_OK;
}

// Grow-only pinned host buffer (hipHostMalloc); the caller has made sure no copy still
// reads or writes the old one.
int grow_host(void **buf, size_t *cap, size_t need) {
    if (need <= *cap) return RKV_OK;
    if (*buf) (void)hipHostFree(*buf);
    *buf = nullptr;
    *cap = 0;
    hipError_t e = hipHostMalloc(buf, need, hipHostMallocDefault);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *buf = nullptr;
        return fail(RKV_ERR_NOMEM, "pinned host allocation of %zu bytes failed", need);
    }
    *cap = need;
    return RKV_OK;
}

int ensure_partials(rkv_ctx *ctx, int64_t floats, hipStream_t s) {
    void *p = ctx->partials;
    size_t cap = ctx->partials_cap * sizeof(float);
    int st = grow(&p, &cap, (size_t)floats * sizeof(float), s);
    ctx->partials = static_cast<float *>(p);
    ctx->partials_cap = cap / sizeof(float);
    return st;
}

// Split-K factor of a device segment for the vector kernel (4-wave workgroups): about two
// workgroups per CU, i.e. one full round of resident workgroups, with at least 256 cells
// (one chunk per wave) per split.
int vec_splits(const rkv_ctx *ctx, int64_t n_cells, int64_t n_groups, int blocks_per_cu = 2) {
    if (ctx->splits_override > 0)
        return (int)std::max<int64_t>(1, std::min<int64_t>(ctx->splits_override, (n_cells + kChunk - 1) / kChunk));
    if (n_cells <= 0) return 1;
    const int64_t target_blocks = (int64_t)blocks_per_cu * ctx->n_cu;
    int64_t want = (target_blocks + n_groups - 1) / std::max<int64_t>(1, n_groups);
    const int64_t max_by_len = std::max<int64_t>(1, n_cells / 256);
    want = std::max<int64_t>(1, std::min(want, max_by_len));
    return (int)want;
}


void fill_q(SegParams &p, const rkv_tensor *q) {
    p.q = static_cast<const _Float16 *>(q->data);
    p.q_s1 = q->nb[1] / 2;
    p.q_s2 = q->nb[2] / 2;
    p.q_s3 = q->nb[3] / 2;
}

void fill_mask(SegParams &p, const rkv_tensor *m) {
    p.mask = m ? static_cast<const _Float16 *>(m->data) : nullptr;
    p.m_s1 = m ? m->nb[1] / 2 : 0;
    p.m_s3 = (m && m->ne[3] > 1) ? m->nb[3] / 2 : 0;
}

struct Seg {
    const uint8_t *k, *v;
    int64_t k_s1, k_s2, v_s1, v_s2;
    int64_t n_cells, pos0;
};

// KV heads per workgroup of the cell-major kernel for this segment, or 0 when it does not
// apply: every cell must hold the KV heads packed (head stride == row size), cell strides and
// bases must be aligned (4 bytes for the q8_0 / q4_0 kernel, whose loads start on words; 16
// for the others), and the types and head count must have an instantiation.
int use_cell_kernel(const Seg &sg, const SegParams &p, int k_type, int v_type) {
    const int64_t rk = row_bytes(k_type, p.d), rv = row_bytes(v_type, p.dv);
    const int hw = cell_heads(p.d, p.dv, k_type, v_type, p.n_head_kv, p.gqa * p.n_q, p.rows != nullptr);
    if (hw == 0) return 0;
    const int64_t al = (k_type == T_Q8_0 && v_type == T_Q4_0) ? 4 : 16;
    if (p.n_head_kv > 1 && (sg.k_s2 != rk || sg.v_s2 != rv)) return 0;
    if (sg.k_s1 < p.n_head_kv * rk || sg.v_s1 < p.n_head_kv * rv) return 0;
    if ((sg.k_s1 | sg.v_s1) % al != 0) return 0;
    if (((uintptr_t)sg.k | (uintptr_t)sg.v) % al != 0) return 0;
    // row lists: the cell-major kernel addresses the pool with 32-bit offsets
    const int64_t lim = (int64_t)1 << 31;
    if (p.rows && (p.n_pool * sg.k_s1 >= lim || p.n_pool * sg.v_s1 >= lim || sg.k_s1 >= (1 << 24) || sg.v_s1 >= (1 << 24)))
        return 0;
    // binary16 groups the persistent kernel cannot plan (more than 1024 sequence and head-group
    // pairs) go to the vector kernels (the cell kernel of pairs of heads at 128 has no such limit)
    if (k_type == T_F16 && v_type == T_F16 && !(hw == 2 && p.d == kHeadDim)) {
        SegParams pc = p;
        pc.cell_hw = hw;
        if (!decode_mma16_ok(pc)) return 0;
    }
    return hw;
}

// Split-K plan of one device segment: cells per split and number of splits.  The vector
// kernel walks 64-cell chunks; the MFMA kernel walks key tiles of prefill_keys_per_iter().
void seg_plan(const rkv_ctx *ctx, int64_t n_cells, const SegParams &p, bool mfma, int cell_occupancy, bool persistent,
              int row_groups, int64_t &cps, int &n_splits) {
    if (mfma) {
        const int kpi = prefill_keys_per_iter();
        const int64_t q_tiles = ((int64_t)p.gqa * p.n_q + prefill_rows_per_block() - 1) / prefill_rows_per_block();
        // as many splits as keep every launch within one wave of resident workgroups, so all
        // blocks of a segment run concurrently and finish together
        const int64_t groups = q_tiles * p.n_head_kv * p.n_seq;
        const int64_t slots = (int64_t)prefill_blocks_per_cu() * ctx->n_cu;
        int64_t want = ctx->splits_override > 0 ? ctx->splits_override : std::max<int64_t>(1, slots / groups);
        want = std::min<int64_t>(want, std::max<int64_t>(1, (n_cells + kpi - 1) / kpi));
        cps = (n_cells + want - 1) / want;
        cps = std::max<int64_t>(kpi, (cps + kpi - 1) / kpi * kpi);
    } else if (persistent) {
        // binary16 matrix-core kernel: one resident workgroup per slot, each taking a contiguous
        // run of the chunks (16 or 32 cells) of all (sequence, head group) pairs
        const int64_t ch = decode_mma16_chunk(p.d, p.rows != nullptr);
        const int64_t tasks = (int64_t)p.n_seq * (p.n_head_kv / p.cell_hw) * ((n_cells + ch - 1) / ch);
        const int64_t slots = (int64_t)std::max(1, cell_occupancy) * ctx->n_cu;
        const int64_t g = ctx->splits_override > 0 ? ctx->splits_override : slots;
        n_splits = (int)std::max<int64_t>(1, std::min(g, tasks));
        cps = n_cells;
        return;
    } else if (p.cell_hw > 0) {
        // cell-major kernel: one wave of resident workgroups over (split, head group, sequence,
        // row group of 16), at least 256 cells per split
        const int64_t groups = (int64_t)p.n_seq * (p.n_head_kv / p.cell_hw) * row_groups;
        const int64_t slots = (int64_t)std::max(1, cell_occupancy) * ctx->n_cu;
        int64_t want = ctx->splits_override > 0 ? ctx->splits_override : std::max<int64_t>(1, slots / groups);
        want = std::max<int64_t>(1, std::min(want, std::max<int64_t>(1, n_cells / 256)));
        cps = (n_cells + want - 1) / want;
        cps = std::max<int64_t>(kChunk, (cps + kChunk - 1) / kChunk * kChunk);
    } else {
        // the kernel for head dims other than 128 holds four workgroups per CU
        const int splits = vec_splits(ctx, n_cells, (int64_t)p.n_head_kv * p.n_seq, p.d == kHeadDim ? 2 : 4);
        cps = (n_cells + splits - 1) / splits;
        cps = std::max<int64_t>(kChunk, (cps + kChunk - 1) / kChunk * kChunk);
    }
    n_splits = (int)std::max<int64_t>(1, (n_cells + cps - 1) / cps);
}

struct SegPlan {
    int cell_hw;
    int64_t cps;
    int n_splits;
};

SegPlan plan_segment(const rkv_ctx *ctx, const SegParams &base, const Seg &sg, bool mfma, int k_type, int v_type) {
    SegParams p = base;
    p.cell_hw = mfma ? 0 : use_cell_kernel(sg, p, k_type, v_type);
    SegPlan pl{p.cell_hw, 0, 0};
    const int occ = p.cell_hw > 0 ? cell_blocks_per_cu(p, k_type, v_type) : 1;
    seg_plan(ctx, sg.n_cells, p, mfma, occ, p.cell_hw > 0 && decode_kernel_persistent(p, k_type, v_type),
             p.cell_hw > 0 ? cell_row_groups(p, k_type, v_type) : 1, pl.cps, pl.n_splits);
    return pl;
}

// Launch one device segment; `slot` advances by the splits it used.
int run_segment(rkv_ctx *ctx, SegParams base, const Seg &sg, bool mfma, int k_type, int v_type,
                int &slot, hipStream_t s) {
    SegParams p = base;
    p.k = sg.k;
    p.v = sg.v;
    p.k_s1 = sg.k_s1;
    p.k_s2 = sg.k_s2;
    p.v_s1 = sg.v_s1;
    p.v_s2 = sg.v_s2;
    p.n_cells = sg.n_cells;
    p.pos0 = sg.pos0;
    p.slot0 = slot;
    const SegPlan pl = plan_segment(ctx, base, sg, mfma, k_type, v_type);
    p.cell_hw = pl.cell_hw;
    p.n_splits = pl.n_splits;
    p.cells_per_split = (int)pl.cps;
    const bool timed = ctx->kernel_timing && ctx->n_kernel_timed < (int)ctx->kt0.size();
    p.ev_start = timed ? ctx->kt0[ctx->n_kernel_timed] : nullptr;
    p.ev_stop = timed ? ctx->kt1[ctx->n_kernel_timed] : nullptr;
    const hipError_t e = mfma ? launch_prefill_segment(p, k_type, v_type, s) : launch_decode_segment(p, k_type, v_type, s);
    if (e != hipSuccess) return hip_fail(e, mfma ? "prefill segment launch" : "decode segment launch");
    if (timed) ctx->n_kernel_timed++;
    ctx->stats.kernel_variant = mfma ? RKV_KERNEL_PREFILL_MFMA : decode_kernel_variant(p, k_type, v_type);
    slot += p.n_splits;
    ctx->stats.n_segments += 1;
    return RKV_OK;
}

// Geometry of a host tail for tile lifting: each tile of `cells` cells is one contiguous
// span (cell-major: all heads inside a cell) or n_head_kv spans (head-major).
struct TailGeom {
    bool cell_major;
    int64_t nb1, nb2, n_head_kv;
    int64_t tile_bytes(int64_t cells) const { return cell_major ? cells * nb1 : n_head_kv * cells * nb1; }
};

int tail_geom(const rkv_tensor *t, TailGeom &g) {
    const int64_t rb = row_bytes(t->type, t->ne[0]);
    g.nb1 = t->nb[1];
    g.nb2 = t->nb[2];
    g.n_head_kv = t->ne[2];
    if (t->ne[2] == 1 || (t->nb[2] * (t->ne[2] - 1) + rb <= t->nb[1])) {
        g.cell_major = true;
        return RKV_OK;
    }
    if (t->nb[1] == rb && t->nb[2] >= t->ne[1] * rb) {
        g.cell_major = false;
        return RKV_OK;
    }
    return fail(RKV_ERR_UNSUPPORTED, "host tail must be cell-major (heads inside a cell) or head-major contiguous");
}

// Enqueue the lift of cells [loc, loc+cells) of a host tail tensor into ring slot `slot`.
int lift_tile(rkv_ctx *ctx, int mode, const rkv_tensor *t, const TailGeom &g, int64_t loc, int64_t cells,
              int64_t tile_cap_cells, void *dst, hipStream_t cs) {
    const uint8_t *src = static_cast<const uint8_t *>(t->data) + loc * g.nb1;
    // the copy kernel moves 8-byte words: spans that do not start on one (rows of 68 or 36
    // bytes, head dim 64) go through the DMA engine
    if (mode == RKV_LIFT_KERNEL &&
        ((uintptr_t)src | (uintptr_t)dst | (uintptr_t)g.nb1 | (uintptr_t)(g.cell_major ? 0 : g.nb2)) % 8 != 0)
        mode = RKV_LIFT_BULK;
    if (g.cell_major) {
        const int64_t bytes = cells * g.nb1;
        if (mode == RKV_LIFT_UVA) {
            hipError_t e = launch_uva_read(src, dst, bytes, cs);
            if (e != hipSuccess) return hip_fail(e, "uva lift");
        } else if (mode == RKV_LIFT_KERNEL) {
            hipError_t e = launch_lift_copy(src, dst, bytes, cs);
            if (e != hipSuccess) return hip_fail(e, "kernel lift");
        } else {
            RKV_HIP(hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, cs));
        }
        ctx->stats.lift_bytes += bytes;
    } else {
        const int64_t width = cells * g.nb1;
        if (mode == RKV_LIFT_UVA || mode == RKV_LIFT_KERNEL) {
            for (int64_t h = 0; h < g.n_head_kv; ++h) {
                const uint8_t *hs = src + h * g.nb2;
                uint8_t *hd = static_cast<uint8_t *>(dst) + h * tile_cap_cells * g.nb1;
                hipError_t e = mode == RKV_LIFT_UVA ? launch_uva_read(hs, hd, width, cs)
                                                              : launch_lift_copy(hs, hd, width, cs);
                if (e != hipSuccess) return hip_fail(e, "kernel lift");
            }
        } else {
            RKV_HIP(hipMemcpy2DAsync(dst, (size_t)(tile_cap_cells * g.nb1), src, (size_t)g.nb2, (size_t)width,
                                     (size_t)g.n_head_kv, hipMemcpyHostToDevice, cs));
        }
        ctx->stats.lift_bytes += width * g.n_head_kv;
    }
    return RKV_OK;
}

// Common body of decode and prefill.
// ext_partials (optional): a device buffer of ext_cap floats that replaces the context's
// partials workspace; then nothing is allocated, the split-K factor shrinks until the partials
// fit, and the tail must be device-resident.
int attn_window_tail(rkv_ctx *ctx, const rkv_tensor *q, const rkv_tensor *k_win,
                     const rkv_tensor *v_win, const rkv_tensor *k_tail, const rkv_tensor *v_tail,
                     const rkv_tensor *mask, int64_t wc, int64_t tile_kv, float scale,
                     int64_t q_pos0, bool mfma, float *o, float *lse, hipStream_t stream,
                     float *ext_partials = nullptr, int64_t ext_cap = 0, bool prefill = false) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    // dk = dv in 64, 128, 256, 512 and the pair dk = 576 / dv = 512 (prefill at head dims 128
    // and 64 on the matrix-core prefill kernel, everything else on the decode kernels)
    const bool any_d = !mfma || (q && q->ne[0] != kHeadDim);
    int st = check_q(q, false, any_d);
    if (st) return st;
    if (wc < 0) return fail(RKV_ERR_ARG, "wc < 0");
    if (tile_kv <= 0) return fail(RKV_ERR_ARG, "tile_kv must be > 0");
    if (!std::isfinite(scale)) return fail(RKV_ERR_ARG, "scale is not finite");
    if (!o) return fail(RKV_ERR_ARG, "o is NULL");
    if (q_pos0 < -1) return fail(RKV_ERR_ARG, "q_pos0 must be >= -1");
    if ((k_tail == nullptr) != (v_tail == nullptr)) return fail(RKV_ERR_ARG, "k_tail and v_tail must both be given or both NULL");
    if (wc > 0 && (!k_win || !v_win)) return fail(RKV_ERR_ARG, "window tensors missing while wc > 0");
    const rkv_tensor *kref = k_win ? k_win : k_tail;
    const rkv_tensor *vref = v_win ? v_win : v_tail;
    if (!kref) return fail(RKV_ERR_ARG, "no K/V given");
    if (k_win) {
        if ((st = check_kv(k_win, "k_win", true, any_d)) || (st = check_kv(v_win, "v_win", false, any_d))) return st;
        if (k_win->ne[1] < wc || v_win->ne[1] < wc) return fail(RKV_ERR_ARG, "window tensors hold fewer than wc cells");
        if (k_win->ne[2] != v_win->ne[2]) return fail(RKV_ERR_ARG, "k_win and v_win disagree in n_head_kv");
    }
    int64_t n_tail = 0;
    Mem tail_kind = Mem::Device;
    if (k_tail) {
        if ((st = check_kv(k_tail, "k_tail", true, any_d)) || (st = check_kv(v_tail, "v_tail", false, any_d))) return st;
        if (k_tail->ne[1] != v_tail->ne[1] || k_tail->ne[2] != v_tail->ne[2])
            return fail(RKV_ERR_ARG, "k_tail and v_tail disagree in shape");
        if (k_win && ((st = same_kv_shape(k_win, k_tail, "K")) || (st = same_kv_shape(v_win, v_tail, "V")))) return st;
        n_tail = k_tail->ne[1];
        if (n_tail > 0) {
            const Mem a = pointer_kind(k_tail->data), b = pointer_kind(v_tail->data);
            if (a != b) return fail(RKV_ERR_ARG, "k_tail and v_tail live in different memory kinds");
            if (a == Mem::Other && (ctx->tail_mode != RKV_TAIL_HOST || mfma || prefill))
                return fail(RKV_ERR_ARG, "tail is neither device nor pinned host memory (pageable memory cannot be lifted)");
            tail_kind = a;
        }
    }
    const int64_t n_head = q->ne[2], n_q = q->ne[1];
    const int64_t n_head_kv = kref->ne[2];
    if (n_head % n_head_kv != 0) return fail(RKV_ERR_ARG, "n_head %% n_head_kv != 0");
    const int64_t gqa = n_head / n_head_kv;
    const int d = (int)q->ne[0];
    const int dv = (int)vref->ne[0];
    if (kref->ne[0] != d || (k_tail && (k_tail->ne[0] != d || v_tail->ne[0] != dv)) || (v_win && v_win->ne[0] != dv))
        return fail(RKV_ERR_ARG, "K head dims must equal Q's and the V tensors must agree");
    if (!head_dims_supported(d, dv))
        return fail(RKV_ERR_UNSUPPORTED, "head dims dk=%d, dv=%d not supported (dk = dv in 64, 128, 256, 512, or 576/512)",
                    d, dv);
    if (mfma && !prefill_head_dims_ok(d, dv))
        return fail(RKV_ERR_UNSUPPORTED, "the prefill kernel takes dk = dv = 128 or 64 (got %d / %d)", d, dv);
    const int64_t ps = 2 + dv;  // partial row stride
    // the head-dim-128 decode kernels take up to 8 rows per KV head; the kernel for other head
    // dims takes any number in row groups of 8
    if (!mfma && d == kHeadDim && gqa * n_q > kMaxRowsVec)
        return fail(RKV_ERR_UNSUPPORTED, "decode handles n_q*gqa <= %d rows per KV head (got %lld); use rkv_attn_prefill",
                    kMaxRowsVec, (long long)(gqa * n_q));
    const int64_t n_kv = wc + n_tail;
    if ((st = check_mask(mask, n_kv, n_q, 1))) return st;
    if ((st = check_device_ptr(o, "o"))) return st;
    if (lse && (st = check_device_ptr(lse, "lse"))) return st;
    if (k_win && wc > 0 && ((st = check_device_ptr(k_win->data, "k_win")) || (st = check_device_ptr(v_win->data, "v_win")))) return st;
    if ((st = ensure_device(ctx))) return st;

    const int k_type = kref->type, v_type = vref->type;
    SegParams base{};
    fill_q(base, q);
    fill_mask(base, mask);
    base.rows = nullptr;
    base.q_pos0 = q_pos0;
    base.n_head = (int)n_head;
    base.n_head_kv = (int)n_head_kv;
    base.n_q = (int)n_q;
    base.n_seq = 1;
    base.gqa = (int)gqa;
    base.scale_log2 = scale * 1.4426950408889634f;
    fill_softcap(base, ctx, scale);
    base.n_rows = n_head * n_q;
    base.d = d;
    base.dv = dv;

    // ---- plan: window segment, then tail (in place, lifted tiles through the ring, or a
    // partial computed on the host cores)
    // (prefill always computes the tail on the GPU)
    const bool host_tail = n_tail > 0 && tail_kind != Mem::Device && ctx->tail_mode == RKV_TAIL_HOST && !mfma && !prefill;
    // In place: the segment kernels read a pinned tail through its device view, in their own
    // access order, with no lift -- always under RKV_LIFT_DIRECT, and under RKV_LIFT_AUTO for a
    // small decode tail whose cells each kernel reads once (up to 8 rows per KV head), where
    // the lift's extra launch and hand-off between streams cost more than the copy saves
    const int64_t tail_bytes = n_tail * n_head_kv * (row_bytes(kref->type, d) + row_bytes(vref->type, dv));
    const bool auto_direct = ctx->lift_mode == RKV_LIFT_AUTO && !mfma && !prefill && gqa * n_q <= kMaxRowsVec &&
                             tail_bytes <= ctx->direct_tail_max;
    const bool direct = n_tail > 0 && tail_kind == Mem::PinnedHost && !host_tail &&
                        (ctx->lift_mode == RKV_LIFT_DIRECT || auto_direct);
    const bool lifted = n_tail > 0 && tail_kind == Mem::PinnedHost && !host_tail && !direct;
    const int64_t n_tiles = lifted ? (n_tail + tile_kv - 1) / tile_kv : 0;
    TailGeom gk{}, gv{};
    int n_slots = 0;
    const int64_t cap_cells = lifted ? std::min(tile_kv, n_tail) : 0;
    if (lifted) {
        if ((st = tail_geom(k_tail, gk)) || (st = tail_geom(v_tail, gv))) return st;
        n_slots = (int)std::min<int64_t>(ctx->n_slots, n_tiles);
        for (int sl = 0; sl < n_slots; ++sl) {
            if ((st = grow(&ctx->scr_k[sl], &ctx->cap_k[sl], (size_t)gk.tile_bytes(cap_cells), stream))) return st;
            if ((st = grow(&ctx->scr_v[sl], &ctx->cap_v[sl], (size_t)gv.tile_bytes(cap_cells), stream))) return st;
        }
    }
    Seg win{}, dtail{};
    if (wc > 0)
        win = Seg{static_cast<const uint8_t *>(k_win->data), static_cast<const uint8_t *>(v_win->data),
                  k_win->nb[1], k_win->nb[2], v_win->nb[1], v_win->nb[2], wc, 0};
    if (n_tail > 0 && !lifted) {
        const uint8_t *tk = static_cast<const uint8_t *>(k_tail->data), *tv = static_cast<const uint8_t *>(v_tail->data);
        if (direct) {
            void *vk = nullptr, *vv = nullptr;
            if (hipHostGetDevicePointer(&vk, const_cast<void *>(k_tail->data), 0) != hipSuccess ||
                hipHostGetDevicePointer(&vv, const_cast<void *>(v_tail->data), 0) != hipSuccess) {
                (void)hipGetLastError();
                return fail(RKV_ERR_HIP, "no device view of the pinned tail");
            }
            tk = static_cast<const uint8_t *>(vk);
            tv = static_cast<const uint8_t *>(vv);
        }
        dtail = Seg{tk, tv, k_tail->nb[1], k_tail->nb[2], v_tail->nb[1], v_tail->nb[2], n_tail, wc};
    }
    // tile t of the lifted tail, read from ring slot t % n_slots (the ring keeps the tail's
    // cell layout; a head-major tail gets head planes of cap_cells cells)
    auto tile_seg = [&](int64_t t) {
        const int sl = (int)(t % n_slots);
        const int64_t loc = t * tile_kv, cells = std::min(tile_kv, n_tail - loc);
        return Seg{static_cast<const uint8_t *>(ctx->scr_k[sl]), static_cast<const uint8_t *>(ctx->scr_v[sl]),
                   gk.nb1, gk.cell_major ? gk.nb2 : cap_cells * gk.nb1,
                   gv.nb1, gv.cell_major ? gv.nb2 : cap_cells * gv.nb1, cells, wc + loc};
    };
    auto count_slots = [&]() {
        int64_t n = 0;
        if (wc > 0) n += plan_segment(ctx, base, win, mfma, k_type, v_type).n_splits;
        if (n_tail > 0 && !lifted) n += plan_segment(ctx, base, dtail, mfma, k_type, v_type).n_splits;
        for (int64_t t = 0; t < n_tiles; ++t) n += plan_segment(ctx, base, tile_seg(t), mfma, k_type, v_type).n_splits;
        if (host_tail) n += 1;
        return n == 0 ? (int64_t)1 : n;  // n_kv == 0: one empty partial
    };
    int64_t total_slots = count_slots();
    if (ext_partials) {
        if (lifted || host_tail) return fail(RKV_ERR_ARG, "a caller-provided partials buffer needs a device-resident tail");
        const int64_t per_slot = base.n_rows * ps;
        if (per_slot > ext_cap)
            return fail(RKV_ERR_UNSUPPORTED, "one partial of %lld rows needs %lld floats, more than the %lld available",
                        (long long)base.n_rows, (long long)per_slot, (long long)ext_cap);
        // fewer splits until every segment's partials fit (each segment takes at least one slot)
        const int n_seg = (wc > 0 ? 1 : 0) + (n_tail > 0 ? 1 : 0);
        while (total_slots * per_slot > ext_cap) {
            const int64_t cur = ctx->splits_override > 0 ? ctx->splits_override : total_slots;
            const int64_t fit = std::max<int64_t>(1, ext_cap / per_slot / std::max(1, n_seg));
            ctx->splits_override = (int)std::max<int64_t>(1, std::min(cur - 1, fit));
            total_slots = count_slots();
            if (ctx->splits_override == 1 && total_slots * per_slot > ext_cap)
                return fail(RKV_ERR_UNSUPPORTED, "partials of %lld slots exceed the %lld floats available",
                            (long long)total_slots, (long long)ext_cap);
        }
        base.partials = ext_partials;
    } else {
        if ((st = ensure_partials(ctx, total_slots * base.n_rows * ps, stream))) return st;
        base.partials = ctx->partials;
    }
    // every kernel below (segments, empty partial, merge) reads and writes base.partials
    if (!base.partials) return fail(RKV_ERR_HIP, "no partials workspace");

    ctx->stats = rkv_stats{};
    ctx->stats.kernel_variant = mfma ? RKV_KERNEL_PREFILL_MFMA : RKV_KERNEL_DECODE_HEAD;
    // lift mode of this call: the automatic choice reads small decode tails in place (above),
    // lifts the other decode tails with the copy kernel and prefill tails with the DMA engine
    const int lift_mode = direct ? RKV_LIFT_DIRECT
                                 : (ctx->lift_mode == RKV_LIFT_AUTO || ctx->lift_mode == RKV_LIFT_DIRECT)
                                       ? (mfma ? RKV_LIFT_BULK : RKV_LIFT_KERNEL)
                                       : ctx->lift_mode;
    ctx->stats.lift_mode = lift_mode;
    int slot = 0;

    // host tail: Q (and the tail's mask columns) go to pinned host memory ahead of the window
    // kernels, so the host computes the tail partial while the GPU computes the window
    const int64_t q_span = (n_q - 1) * q->nb[1] + (n_head - 1) * q->nb[2] + d * 2;
    if (host_tail) {
        if (stream_capturing(stream)) return fail(RKV_ERR_CAPTURE, "the host tail partial cannot run inside graph capture");
        if (!host_tail_supported()) return fail(RKV_ERR_UNSUPPORTED, "the host tail partial needs a CPU with AVX2, FMA and F16C");
        if (ctx->host_up_pending) {  // the previous call's upload still reads the partial buffer
            RKV_HIP(hipEventSynchronize(ctx->host_up));
            ctx->host_up_pending = false;
        }
        // a previous call that failed between its Q copy and its wait may still be writing the
        // staging buffers: let that copy land before they are reused or regrown
        if (ctx->host_in) RKV_HIP(hipEventSynchronize(ctx->host_in));
        if ((st = grow_host(&ctx->hq, &ctx->hq_cap, (size_t)q_span)) ||
            (mask && (st = grow_host(&ctx->hmask, &ctx->hmask_cap, (size_t)(n_q * n_tail * 2)))) ||
            (st = grow_host(&ctx->hpart, &ctx->hpart_cap, (size_t)(base.n_rows * ps * 4))))
            return st;
        if (!ctx->host_in) RKV_HIP(hipEventCreateWithFlags(&ctx->host_in, hipEventDisableTiming));
        if (!ctx->host_up) RKV_HIP(hipEventCreateWithFlags(&ctx->host_up, hipEventDisableTiming));
        RKV_HIP(hipMemcpyAsync(ctx->hq, q->data, (size_t)q_span, hipMemcpyDeviceToHost, stream));
        if (mask)
            RKV_HIP(hipMemcpy2DAsync(ctx->hmask, (size_t)(n_tail * 2), static_cast<const uint8_t *>(mask->data) + wc * 2,
                                     (size_t)mask->nb[1], (size_t)(n_tail * 2), (size_t)n_q, hipMemcpyDeviceToHost, stream));
        RKV_HIP(hipEventRecord(ctx->host_in, stream));
    }

    if (lifted) {
        // the copy stream starts after all earlier work on the compute stream, so a slot
        // still read by an earlier call is never overwritten
        RKV_HIP(hipEventRecord(ctx->entry, stream));
        RKV_HIP(hipStreamWaitEvent(ctx->copy_stream, ctx->entry, 0));
    }
    auto lift = [&](int64_t t) -> int {
        const int sl = (int)(t % n_slots);
        const int64_t loc = t * tile_kv, cells = std::min(tile_kv, n_tail - loc);
        const bool timed = ctx->lift_timing && ctx->n_lift_timed < kMaxLiftTiming;
        if (timed) RKV_HIP(hipEventRecord(ctx->lift_t0[ctx->n_lift_timed], ctx->copy_stream));
        int r = lift_tile(ctx, lift_mode, k_tail, gk, loc, cells, cap_cells, ctx->scr_k[sl], ctx->copy_stream);
        if (!r) r = lift_tile(ctx, lift_mode, v_tail, gv, loc, cells, cap_cells, ctx->scr_v[sl], ctx->copy_stream);
        if (r) return r;
        if (timed) RKV_HIP(hipEventRecord(ctx->lift_t1[ctx->n_lift_timed++], ctx->copy_stream));
        RKV_HIP(hipEventRecord(ctx->copy_done[sl], ctx->copy_stream));
        ctx->stats.n_tail_tiles += 1;
        return RKV_OK;
    };
    if (lifted) {
        ctx->n_lift_timed = 0;
        if ((st = lift(0))) return st;
    }

    if (wc > 0) {
        const int before = slot;
        if ((st = run_segment(ctx, base, win, mfma, k_type, v_type, slot, stream))) return st;
        ctx->stats.splits_window = slot - before;
    }
    if (n_tail > 0 && !lifted && !host_tail) {
        if ((st = run_segment(ctx, base, dtail, mfma, k_type, v_type, slot, stream))) return st;
    }
    if (host_tail) {
        RKV_HIP(hipEventSynchronize(ctx->host_in));
        HostTailArgs ha{};
        ha.q = static_cast<const uint16_t *>(ctx->hq);
        ha.q_s1 = q->nb[1] / 2;
        ha.q_s2 = q->nb[2] / 2;
        ha.k = static_cast<const uint8_t *>(k_tail->data);
        ha.v = static_cast<const uint8_t *>(v_tail->data);
        ha.k_s1 = k_tail->nb[1];
        ha.k_s2 = k_tail->nb[2];
        ha.v_s1 = v_tail->nb[1];
        ha.v_s2 = v_tail->nb[2];
        ha.k_type = k_type;
        ha.v_type = v_type;
        ha.mask = mask ? static_cast<const uint16_t *>(ctx->hmask) : nullptr;
        ha.m_s1 = n_tail;
        ha.n_cells = n_tail;
        ha.kv_pos0 = wc;
        ha.q_pos0 = q_pos0;
        ha.n_head = (int)n_head;
        ha.n_head_kv = (int)n_head_kv;
        ha.n_q = (int)n_q;
        ha.scale = scale;
        ha.softcap = ctx->softcap;
        ha.partial = static_cast<float *>(ctx->hpart);
        ha.d = d;
        ha.dv = dv;
        const auto t0 = std::chrono::steady_clock::now();
        try {
            host_tail_partial(ha, ctx->host_threads);
        } catch (...) {
            return fail(RKV_ERR_NOMEM, "host memory for the tail partial's chunk partials");
        }
        ctx->stats.host_tail_ms = std::chrono::duration<float, std::milli>(std::chrono::steady_clock::now() - t0).count();
        ctx->stats.tail_host = 1;
        RKV_HIP(hipMemcpyAsync(base.partials + (int64_t)slot * base.n_rows * ps, ctx->hpart,
                               (size_t)(base.n_rows * ps * 4), hipMemcpyHostToDevice, stream));
        RKV_HIP(hipEventRecord(ctx->host_up, stream));
        ctx->host_up_pending = true;
        slot += 1;
    }
    // Tile t+1 goes into slot (t+1) % n_slots once the tile that last used that slot,
    // t+1-n_slots, is computed.  With two or more slots that tile is at most t-1, so the lift
    // is enqueued ahead of tile t's kernel and overlaps it; with a single slot it is tile t
    // itself, so the lift follows tile t's kernel (no prefetch).
    for (int64_t t = 0; t < n_tiles; ++t) {
        const int sl = (int)(t % n_slots);
        const bool next = t + 1 < n_tiles;
        if (next && n_slots > 1) {
            const int ns = (int)((t + 1) % n_slots);
            if (t + 1 >= n_slots) RKV_HIP(hipStreamWaitEvent(ctx->copy_stream, ctx->compute_done[ns], 0));
            if ((st = lift(t + 1))) return st;
        }
        RKV_HIP(hipStreamWaitEvent(stream, ctx->copy_done[sl], 0));
        if ((st = run_segment(ctx, base, tile_seg(t), mfma, k_type, v_type, slot, stream))) return st;
        RKV_HIP(hipEventRecord(ctx->compute_done[sl], stream));
        if (next && n_slots == 1) {
            RKV_HIP(hipStreamWaitEvent(ctx->copy_stream, ctx->compute_done[0], 0));
            if ((st = lift(t + 1))) return st;
        }
    }
    if (d != kHeadDim) {
        // other head dims: the merge of partials with row stride 2 + dv (no partial at all, as
        // for n_kv == 0, gives every row O = 0 and LSE = -inf)
        ctx->stats.n_partials = slot;
        hipError_t e = launch_merge_hd(base.partials, slot, base.n_rows, dv, o, lse, stream);
        if (e != hipSuccess) return hip_fail(e, "merge launch");
        return RKV_OK;
    }
    if (slot == 0) {
        // n_kv == 0: a single empty partial, so every row gets O = 0 and LSE = -inf
        hipError_t e0 = launch_empty_partials(base.partials, base.n_rows, stream);
        if (e0 != hipSuccess) return hip_fail(e0, "empty partial");
        slot = 1;
    }
    ctx->stats.n_partials = slot;
    hipError_t e = launch_merge(base.partials, slot, base.n_rows, o, lse, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return RKV_OK;
}

// ---- allocation-free decode: partials in a file-scope device array.  Each device holds its own
// copy of the array (until the process ends); host code may use the array only through the
// device address hipGetSymbolAddress returns on that device (the name itself is a host-side
// stand-in), looked up once per device and kept here.
constexpr int64_t kNoAllocFloats = (int64_t)2 << 20;  // 8 MiB of partials

}  // namespace

static __device__ __align__(256) float scratch[kNoAllocFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
float *g_noalloc_ptr[kMaxDevices] = {};
int g_noalloc_cu[kMaxDevices] = {};

// The calling thread's current device, its copy of `scratch` and its compute-unit count.
int noalloc_scratch(float **ptr, int *n_cu, int *device) {
    int dev = -1;
    RKV_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(RKV_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(RKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        }
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            return fail(RKV_ERR_HIP, "compute-unit count of device %d", dev);
        }
        g_noalloc_cu[dev] = cus;
        g_noalloc_ptr[dev] = static_cast<float *>(p);
    }
    *ptr = g_noalloc_ptr[dev];
    *n_cu = g_noalloc_cu[dev];
    *device = dev;
    return RKV_OK;
}

}  // namespace

extern "C" {

const char *rkv_version(void) { return "0.1.0"; }

const char *rkv_strerror(int status) {
    switch (status) {
        case RKV_OK: return "ok";
        case RKV_ERR_ARG: return "invalid argument";
        case RKV_ERR_UNSUPPORTED: return "unsupported";
        case RKV_ERR_HIP: return "HIP runtime error";
        case RKV_ERR_NOMEM: return "out of device memory";
        case RKV_ERR_CAPTURE: return "allocation needed during stream capture";
        default: return "unknown status";
    }
}

const char *rkv_last_error(void) { return g_err.c_str(); }

int rkv_create(int device, rkv_ctx **out) {
    if (!out) return fail(RKV_ERR_ARG, "out is NULL");
    *out = nullptr;
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || device < 0 || device >= n) {
        (void)hipGetLastError();
        return fail(RKV_ERR_HIP, "device %d not available (%d devices)", device, n);
    }
    RKV_HIP(hipSetDevice(device));
    rkv_ctx *c = new rkv_ctx();
    c->device = device;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.multiProcessorCount > 0)
        c->n_cu = prop.multiProcessorCount;
    auto bail = [&](hipError_t err, const char *what) {
        rkv_destroy(c);
        return hip_fail(err, what);
    };
    if ((e = hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking)) != hipSuccess) return bail(e, "copy stream");
    for (int i = 0; i < kMaxSlots; ++i) {
        if ((e = hipEventCreateWithFlags(&c->copy_done[i], hipEventDisableTiming)) != hipSuccess) return bail(e, "event");
        if ((e = hipEventCreateWithFlags(&c->compute_done[i], hipEventDisableTiming)) != hipSuccess) return bail(e, "event");
    }
    if ((e = hipEventCreateWithFlags(&c->entry, hipEventDisableTiming)) != hipSuccess) return bail(e, "event");
    for (int i = 0; i < kMaxLiftTiming; ++i) {
        if ((e = hipEventCreate(&c->lift_t0[i])) != hipSuccess) return bail(e, "timing event");
        if ((e = hipEventCreate(&c->lift_t1[i])) != hipSuccess) return bail(e, "timing event");
    }
    *out = c;
    return RKV_OK;
}

void rkv_destroy(rkv_ctx *c) {
    if (!c) return;
    int cur = -1;
    if (hipGetDevice(&cur) == hipSuccess && cur != c->device) (void)hipSetDevice(c->device);
    (void)hipDeviceSynchronize();
    for (int i = 0; i < kMaxSlots; ++i) {
        if (c->scr_k[i]) (void)hipFree(c->scr_k[i]);
        if (c->scr_v[i]) (void)hipFree(c->scr_v[i]);
        if (c->copy_done[i]) (void)hipEventDestroy(c->copy_done[i]);
        if (c->compute_done[i]) (void)hipEventDestroy(c->compute_done[i]);
    }
    for (int i = 0; i < kMaxLiftTiming; ++i) {
        if (c->lift_t0[i]) (void)hipEventDestroy(c->lift_t0[i]);
        if (c->lift_t1[i]) (void)hipEventDestroy(c->lift_t1[i]);
    }
    for (size_t i = 0; i < c->kt0.size(); ++i) {
        (void)hipEventDestroy(c->kt0[i]);
        (void)hipEventDestroy(c->kt1[i]);
    }
    if (c->entry) (void)hipEventDestroy(c->entry);
    if (c->partials) (void)hipFree(c->partials);
    if (c->row_extent) (void)hipFree(c->row_extent);
    if (c->pair_range) (void)hipFree(c->pair_range);
    if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
    if (c->host_in) (void)hipEventDestroy(c->host_in);
    if (c->host_up) (void)hipEventDestroy(c->host_up);
    if (c->hq) (void)hipHostFree(c->hq);
    if (c->hmask) (void)hipHostFree(c->hmask);
    if (c->hpart) (void)hipHostFree(c->hpart);
    (void)hipGetLastError();
    delete c;
}

int rkv_reserve(rkv_ctx *ctx, int64_t max_tile_bytes_k, int64_t max_tile_bytes_v, int n_slots,
                int64_t max_partial_floats) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    if (n_slots < 0 || n_slots > kMaxSlots) return fail(RKV_ERR_ARG, "n_slots must be in [0, %d]", kMaxSlots);
    if (max_tile_bytes_k < 0 || max_tile_bytes_v < 0 || max_partial_floats < 0) return fail(RKV_ERR_ARG, "negative size");
    int st = ensure_device(ctx);
    if (st) return st;
    if (n_slots > 0) ctx->n_slots = n_slots;
    for (int sl = 0; sl < ctx->n_slots; ++sl) {
        if (max_tile_bytes_k > 0 && (st = grow(&ctx->scr_k[sl], &ctx->cap_k[sl], (size_t)max_tile_bytes_k, nullptr))) return st;
        if (max_tile_bytes_v > 0 && (st = grow(&ctx->scr_v[sl], &ctx->cap_v[sl], (size_t)max_tile_bytes_v, nullptr))) return st;
    }
    if (max_partial_floats > 0) {
        if ((st = ensure_partials(ctx, max_partial_floats, nullptr))) return st;
        void *buf = ctx->row_extent;  // row-list extents (up to 1024 sequences)
        st = grow(&buf, &ctx->row_extent_cap, 1024 * kRowExtentParts * sizeof(int32_t), nullptr);
        ctx->row_extent = static_cast<int32_t *>(buf);
        if (st) return st;
        buf = ctx->pair_range;  // slot ranges of up to 1024 pairs
        st = grow(&buf, &ctx->pair_range_cap, 1024 * sizeof(int2), nullptr);
        ctx->pair_range = static_cast<int2 *>(buf);
        if (st) return st;
    }
    return RKV_OK;
}

// Position-window sizing: the steps of the patch 0070 KV-cache sizer (budget, whole-cache
// check, aligned largest fit, at least one unit of window and of tail), with wc <= kv_size.
int rkv_plan_window(rkv_ctx *ctx, int64_t per_cell, int64_t kv_size, int64_t free_bytes, int64_t target_bytes,
                    int64_t reserve_bytes, int64_t align, int64_t *wc) {
    if (!wc) return fail(RKV_ERR_ARG, "wc is NULL");
    if (per_cell <= 0 || kv_size < 0 || align <= 0 || reserve_bytes < 0)
        return fail(RKV_ERR_ARG, "per_cell and align must be > 0, kv_size and reserve_bytes >= 0");
    if (free_bytes < 0) {
        if (!ctx) return fail(RKV_ERR_ARG, "free_bytes < 0 needs a context to query its device");
        int st = ensure_device(ctx);
        if (st) return st;
        size_t fr = 0, tot = 0;
        RKV_HIP(hipMemGetInfo(&fr, &tot));
        free_bytes = (int64_t)fr;
    }
    if (kv_size == 0) {
        *wc = 0;
        return RKV_OK;
    }
    int64_t budget = free_bytes;
    if (target_bytes > 0) budget = std::min(budget, target_bytes);
    budget = budget > reserve_bytes ? budget - reserve_bytes : 0;
    // whole cache fits: per_cell * kv_size <= budget, without overflowing the product
    if (kv_size <= budget / per_cell) {
        *wc = kv_size;
        return RKV_OK;
    }
    int64_t cells = (budget / per_cell) / align * align;
    if (cells < align) cells = align;
    if (kv_size > align && cells > kv_size - align) {
        cells = (kv_size - align) / align * align;
        if (cells < align) cells = align;
    }
    *wc = std::min(cells, kv_size);
    return RKV_OK;
}

int rkv_window_mode(int mode, int64_t wc, int64_t kv_size, int append_only, int v_transposed, int *window) {
    if (!window) return fail(RKV_ERR_ARG, "window is NULL");
    if (mode != RKV_RESIDENCY_AUTO && mode != RKV_RESIDENCY_RESIDENT && mode != RKV_RESIDENCY_WINDOW)
        return fail(RKV_ERR_ARG, "unknown residency mode %d", mode);
    const bool eligible = wc > 0 && wc < kv_size && append_only != 0 && v_transposed == 0;
    *window = (eligible && mode != RKV_RESIDENCY_RESIDENT) ? 1 : 0;
    return RKV_OK;
}

int rkv_choose_tail_mode(int64_t tail_bytes, double h2d_gbps, double host_gbps, int *mode) {
    if (!mode) return fail(RKV_ERR_ARG, "mode is NULL");
    if (tail_bytes < 0) return fail(RKV_ERR_ARG, "tail_bytes < 0");
    if (!(h2d_gbps > 0.0) || !std::isfinite(h2d_gbps) || !(host_gbps > 0.0) || !std::isfinite(host_gbps))
        return fail(RKV_ERR_ARG, "rates must be finite and > 0");
    // equal byte counts: the faster rate gives the shorter tail time
    *mode = (tail_bytes > 0 && host_gbps > h2d_gbps) ? RKV_TAIL_HOST : RKV_TAIL_LIFT;
    return RKV_OK;
}

int rkv_set_tail_mode(rkv_ctx *ctx, int mode, int n_threads) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    if (mode != RKV_TAIL_LIFT && mode != RKV_TAIL_HOST) return fail(RKV_ERR_ARG, "unknown tail mode %d", mode);
    if (n_threads < 0 || n_threads > 256) return fail(RKV_ERR_ARG, "n_threads must be in [0, 256]");
    ctx->tail_mode = mode;
    ctx->host_threads = n_threads;
    return RKV_OK;
}

int rkv_tail_partial_host(const rkv_tensor *q, const rkv_tensor *k, const rkv_tensor *v, const rkv_tensor *mask,
                          int64_t kv_pos0, int64_t q_pos0, float scale, float softcap, float *partial,
                          int n_threads) {
    if (!q || !q->data) return fail(RKV_ERR_ARG, "q is NULL");
    if (q->type != RKV_TYPE_F16) return fail(RKV_ERR_UNSUPPORTED, "q must be F16");
    if (!head_dim_supported((int)std::min<int64_t>(q->ne[0], 1 << 20)))
        return fail(RKV_ERR_UNSUPPORTED, "q head dim %lld not supported", (long long)q->ne[0]);
    if (q->ne[1] <= 0 || q->ne[2] <= 0 || q->ne[3] != 1) return fail(RKV_ERR_ARG, "q: bad shape");
    if (q->nb[0] != 2 || q->nb[1] % 2 != 0 || q->nb[2] % 2 != 0 || q->nb[1] < 0 || q->nb[2] < 0)
        return fail(RKV_ERR_ARG, "q rows must be contiguous and strides even");
    int st;
    if ((st = check_kv(k, "k", true, true)) || (st = check_kv(v, "v", false, true))) return st;
    if (k->ne[1] != v->ne[1] || k->ne[2] != v->ne[2]) return fail(RKV_ERR_ARG, "k and v disagree in shape");
    if (k->ne[0] != q->ne[0]) return fail(RKV_ERR_ARG, "k head dim must equal q's");
    if (!head_dims_supported((int)q->ne[0], (int)v->ne[0]))
        return fail(RKV_ERR_UNSUPPORTED, "head dims dk=%lld, dv=%lld not supported", (long long)q->ne[0], (long long)v->ne[0]);
    const int64_t n_q = q->ne[1], n_head = q->ne[2], n_head_kv = k->ne[2], n_cells = k->ne[1];
    if (n_head % n_head_kv != 0) return fail(RKV_ERR_ARG, "n_head %% n_head_kv != 0");
    if (kv_pos0 < 0) return fail(RKV_ERR_ARG, "kv_pos0 < 0");
    if (q_pos0 < -1) return fail(RKV_ERR_ARG, "q_pos0 must be >= -1");
    if (!std::isfinite(scale)) return fail(RKV_ERR_ARG, "scale is not finite");
    if (!(softcap >= 0.f) || !std::isfinite(softcap)) return fail(RKV_ERR_ARG, "softcap must be finite and >= 0");
    if (!partial) return fail(RKV_ERR_ARG, "partial is NULL");
    if (n_threads < 0 || n_threads > 256) return fail(RKV_ERR_ARG, "n_threads must be in [0, 256]");
    if (mask) {
        if (!mask->data) return fail(RKV_ERR_ARG, "mask data is NULL");
        if (mask->type != RKV_TYPE_F16 || mask->nb[0] != 2) return fail(RKV_ERR_UNSUPPORTED, "mask must be contiguous F16");
        if (mask->ne[0] < kv_pos0 + n_cells || mask->ne[1] < n_q || mask->ne[3] != 1)
            return fail(RKV_ERR_ARG, "mask smaller than [kv_pos0 + n_cells, n_q]");
        if (mask->nb[1] % 2 != 0) return fail(RKV_ERR_ARG, "mask strides must be even");
    }
    if (!host_tail_supported()) return fail(RKV_ERR_UNSUPPORTED, "the host tail partial needs a CPU with AVX2, FMA and F16C");
    HostTailArgs ha{};
    ha.q = static_cast<const uint16_t *>(q->data);
    ha.q_s1 = q->nb[1] / 2;
    ha.q_s2 = q->nb[2] / 2;
    ha.k = static_cast<const uint8_t *>(k->data);
    ha.v = static_cast<const uint8_t *>(v->data);
    ha.k_s1 = k->nb[1];
    ha.k_s2 = k->nb[2];
    ha.v_s1 = v->nb[1];
    ha.v_s2 = v->nb[2];
    ha.k_type = k->type;
    ha.v_type = v->type;
    ha.mask = mask ? static_cast<const uint16_t *>(mask->data) + kv_pos0 : nullptr;
    ha.m_s1 = mask ? mask->nb[1] / 2 : 0;
    ha.n_cells = n_cells;
    ha.kv_pos0 = kv_pos0;
    ha.q_pos0 = q_pos0;
    ha.n_head = (int)n_head;
    ha.n_head_kv = (int)n_head_kv;
    ha.n_q = (int)n_q;
    ha.scale = scale;
    ha.softcap = softcap;
    ha.partial = partial;
    ha.d = (int)q->ne[0];
    ha.dv = (int)v->ne[0];
    try {
        host_tail_partial(ha, n_threads);
    } catch (...) {
        return fail(RKV_ERR_NOMEM, "host memory for the tail partial's chunk partials");
    }
    return RKV_OK;
}

int rkv_set_softcap(rkv_ctx *ctx, float softcap) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    if (!(softcap >= 0.f) || !std::isfinite(softcap)) return fail(RKV_ERR_ARG, "softcap must be finite and >= 0");
    ctx->softcap = softcap;
    return RKV_OK;
}

int rkv_get_stats(const rkv_ctx *ctx, rkv_stats *out) {
    if (!ctx || !out) return fail(RKV_ERR_ARG, "NULL argument");
    *out = ctx->stats;
    return RKV_OK;
}

int rkv_set_lift_mode(rkv_ctx *ctx, int mode) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    if (mode != RKV_LIFT_BULK && mode != RKV_LIFT_UVA && mode != RKV_LIFT_KERNEL && mode != RKV_LIFT_AUTO &&
        mode != RKV_LIFT_DIRECT)
        return fail(RKV_ERR_ARG, "unknown lift mode %d", mode);
    ctx->lift_mode = mode;
    return RKV_OK;
}

int rkv_set_direct_tail_max(rkv_ctx *ctx, int64_t bytes) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    if (bytes < 0) return fail(RKV_ERR_ARG, "bytes < 0");
    ctx->direct_tail_max = bytes;
    return RKV_OK;
}

int rkv_set_splits(rkv_ctx *ctx, int splits) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    if (splits < 0) return fail(RKV_ERR_ARG, "splits < 0");
    ctx->splits_override = splits;
    return RKV_OK;
}

int rkv_set_lift_timing(rkv_ctx *ctx, int on) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    ctx->lift_timing = on != 0;
    ctx->n_lift_timed = 0;
    return RKV_OK;
}

int rkv_set_kernel_timing(rkv_ctx *ctx, int on) {
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    int st = ensure_device(ctx);
    if (st) return st;
    if (on && ctx->kt0.empty()) {
        ctx->kt0.resize(kMaxKernelTiming);
        ctx->kt1.resize(kMaxKernelTiming);
        // no system-scope fence at the events: they time the kernel, not a host-visible flush
        for (int i = 0; i < kMaxKernelTiming; ++i) {
            RKV_HIP(hipEventCreateWithFlags(&ctx->kt0[i], hipEventDisableSystemFence));
            RKV_HIP(hipEventCreateWithFlags(&ctx->kt1[i], hipEventDisableSystemFence));
        }
    }
    ctx->kernel_timing = on != 0;
    ctx->n_kernel_timed = 0;
    return RKV_OK;
}

int rkv_kernel_timing_ms(rkv_ctx *ctx, float *total_ms, int *n_launches) {
    if (!ctx || !total_ms) return fail(RKV_ERR_ARG, "NULL argument");
    float tot = 0.f;
    for (int i = 0; i < ctx->n_kernel_timed; ++i) {
        RKV_HIP(hipEventSynchronize(ctx->kt1[i]));
        float ms = 0.f;
        RKV_HIP(hipEventElapsedTime(&ms, ctx->kt0[i], ctx->kt1[i]));
        tot += ms;
    }
    *total_ms = tot;
    if (n_launches) *n_launches = ctx->n_kernel_timed;
    return RKV_OK;
}

int rkv_lift_timing_ms(rkv_ctx *ctx, float *total_ms, float *span_ms, int *n_lifts) {
    if (!ctx || !total_ms) return fail(RKV_ERR_ARG, "NULL argument");
    float tot = 0.f;
    for (int i = 0; i < ctx->n_lift_timed; ++i) {
        RKV_HIP(hipEventSynchronize(ctx->lift_t1[i]));
        float ms = 0.f;
        RKV_HIP(hipEventElapsedTime(&ms, ctx->lift_t0[i], ctx->lift_t1[i]));
        tot += ms;
    }
    *total_ms = tot;
    if (span_ms) {
        float sp = 0.f;
        if (ctx->n_lift_timed > 0) RKV_HIP(hipEventElapsedTime(&sp, ctx->lift_t0[0], ctx->lift_t1[ctx->n_lift_timed - 1]));
        *span_ms = sp;
    }
    if (n_lifts) *n_lifts = ctx->n_lift_timed;
    return RKV_OK;
}

int rkv_attn_decode_noalloc(const rkv_tensor *q, const rkv_tensor *k, const rkv_tensor *v, const rkv_tensor *mask,
                            float scale, float *o, float *lse, void *stream) {
    if (!k || !v) return fail(RKV_ERR_ARG, "k and v must be given");
    float *scr = nullptr;
    int n_cu = 0, dev = 0;
    int st = noalloc_scratch(&scr, &n_cu, &dev);
    if (st) return st;
    rkv_ctx c;  // planning state only: no stream, event or buffer is created
    c.device = dev;
    c.n_cu = n_cu;
    return attn_window_tail(&c, q, k, v, nullptr, nullptr, mask, k->ne[1], 1, scale, -1, false, o, lse,
                            static_cast<hipStream_t>(stream), scr, kNoAllocFloats);
}

int rkv_attn_decode(rkv_ctx *ctx, const rkv_tensor *q, const rkv_tensor *k_win, const rkv_tensor *v_win,
                    const rkv_tensor *k_tail, const rkv_tensor *v_tail, const rkv_tensor *mask, int64_t wc,
                    int64_t tile_kv, float scale, float *o, float *lse, void *stream) {
    return attn_window_tail(ctx, q, k_win, v_win, k_tail, v_tail, mask, wc, tile_kv, scale, -1, false, o, lse,
                            static_cast<hipStream_t>(stream));
}

int rkv_attn_prefill(rkv_ctx *ctx, const rkv_tensor *q, const rkv_tensor *k_win, const rkv_tensor *v_win,
                     const rkv_tensor *k_tail, const rkv_tensor *v_tail, const rkv_tensor *mask, int64_t wc,
                     int64_t tile_kv, float scale, int64_t q_pos0, float *o, float *lse, void *stream) {
    // head dim 128 runs on the matrix-core prefill kernel, and so does head dim 64 with more
    // than 8 rows per KV head; the rest on the decode kernels (matrix-core where they take the
    // types and head groups, else the vector kernel), which take the causal rule and the mask
    // alike
    bool mfma = !q || q->ne[0] == kHeadDim;
    if (q && q->ne[0] == 64) {
        const rkv_tensor *kr = k_win ? k_win : k_tail;
        const rkv_tensor *vr = v_win ? v_win : v_tail;
        mfma = kr && vr && kr->ne[2] > 0 && q->ne[2] % kr->ne[2] == 0 && vr->ne[0] == 64 &&
               (q->ne[2] / kr->ne[2]) * q->ne[1] > kMaxRowsVec;
    }
    return attn_window_tail(ctx, q, k_win, v_win, k_tail, v_tail, mask, wc, tile_kv, scale, q_pos0, mfma, o, lse,
                            static_cast<hipStream_t>(stream), nullptr, 0, true);
}

int rkv_attn_rows(rkv_ctx *ctx, const rkv_tensor *q, const rkv_tensor *k_pool, const rkv_tensor *v_pool,
                  const int32_t *kv_rows, int64_t n_kv, const rkv_tensor *mask, float scale, float *o, float *lse,
                  void *stream_) {
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    int st = check_q(q, true, true);
    if (st) return st;
    if ((st = check_kv(k_pool, "k_pool", true, true)) || (st = check_kv(v_pool, "v_pool", false, true))) return st;
    if (k_pool->ne[1] != v_pool->ne[1] || k_pool->ne[2] != v_pool->ne[2]) return fail(RKV_ERR_ARG, "k_pool and v_pool disagree in shape");
    const int d = (int)q->ne[0], dv = (int)v_pool->ne[0];
    if (k_pool->ne[0] != d) return fail(RKV_ERR_ARG, "k_pool head dim must equal Q's");
    if (!head_dims_supported(d, dv))
        return fail(RKV_ERR_UNSUPPORTED, "head dims dk=%d, dv=%d not supported (dk = dv in 64, 128, 256, 512, or 576/512)",
                    d, dv);
    const int64_t ps = 2 + dv;  // partial row stride
    if (n_kv < 0 || n_kv >= ((int64_t)1 << 31)) return fail(RKV_ERR_ARG, "bad n_kv");
    if (!std::isfinite(scale)) return fail(RKV_ERR_ARG, "scale is not finite");
    if (!o) return fail(RKV_ERR_ARG, "o is NULL");
    const int64_t n_head = q->ne[2], n_q = q->ne[1], n_seq = q->ne[3];
    const int64_t n_head_kv = k_pool->ne[2];
    if (n_head % n_head_kv != 0) return fail(RKV_ERR_ARG, "n_head %% n_head_kv != 0");
    const int64_t gqa = n_head / n_head_kv;
    if (d == kHeadDim && gqa * n_q > kMaxRowsVec)
        return fail(RKV_ERR_UNSUPPORTED, "rows attention at head dim 128 handles n_q*gqa <= %d", kMaxRowsVec);
    if ((st = check_mask(mask, n_kv, n_q, n_seq))) return st;
    if (n_kv > 0 && (st = check_device_ptr(kv_rows, "kv_rows"))) return st;
    if (k_pool->ne[1] > 0 && ((st = check_device_ptr(k_pool->data, "k_pool")) || (st = check_device_ptr(v_pool->data, "v_pool")))) return st;
    if ((st = check_device_ptr(o, "o"))) return st;
    if (lse && (st = check_device_ptr(lse, "lse"))) return st;
    if ((st = ensure_device(ctx))) return st;

    SegParams p{};
    fill_q(p, q);
    fill_mask(p, mask);
    p.rows = kv_rows;
    p.rows_s = n_kv;
    p.n_pool = k_pool->ne[1];
    p.q_pos0 = -1;
    p.n_head = (int)n_head;
    p.n_head_kv = (int)n_head_kv;
    p.n_q = (int)n_q;
    p.n_seq = (int)n_seq;
    p.gqa = (int)gqa;
    p.scale_log2 = scale * 1.4426950408889634f;
    fill_softcap(p, ctx, scale);
    p.n_rows = n_head * n_q * n_seq;
    p.d = d;
    p.dv = dv;
    const Seg pool{static_cast<const uint8_t *>(k_pool->data), static_cast<const uint8_t *>(v_pool->data),
                   k_pool->nb[1], k_pool->nb[2], v_pool->nb[1], v_pool->nb[2], n_kv, 0};
    const SegPlan plan = plan_segment(ctx, p, pool, false, k_pool->type, v_pool->type);
    const int slots = plan.n_splits;
    if ((st = ensure_partials(ctx, (int64_t)std::max(1, slots) * p.n_rows * ps, stream))) return st;
    p.partials = ctx->partials;
    ctx->stats = rkv_stats{};
    int slot = 0;
    SegParams pk = p;
    pk.cell_hw = plan.cell_hw;
    MergeRange mr{};
    bool ranged = false;
    const bool persistent = n_kv > 0 && decode_kernel_persistent(pk, k_pool->type, v_pool->type);
    if (n_kv > 0 && pk.cell_hw > 0) {
        // the cell-major kernels walk each list up to its last pool row only
        void *buf = ctx->row_extent;
        st = grow(&buf, &ctx->row_extent_cap, std::max<size_t>(1024, (size_t)n_seq) * kRowExtentParts * sizeof(int32_t),
                  stream);
        ctx->row_extent = static_cast<int32_t *>(buf);
        if (st) return st;
        hipError_t e1 = launch_row_extent(kv_rows, n_kv, n_kv, (int)n_seq, ctx->row_extent, stream);
        if (e1 != hipSuccess) return hip_fail(e1, "row extent launch");
        p.row_extent = ctx->row_extent;
    }
    if (persistent) {
        // the persistent kernel reports which slots hold each pair's partials, so that the merge
        // reads only those
        void *buf = ctx->pair_range;
        st = grow(&buf, &ctx->pair_range_cap, 1024 * sizeof(int2), stream);
        ctx->pair_range = static_cast<int2 *>(buf);
        if (st) return st;
        p.pair_range = ctx->pair_range;
        mr = MergeRange{ctx->pair_range, (int)n_head, (int)(gqa * plan.cell_hw), (int)(n_head_kv / plan.cell_hw),
                        n_head * n_q};
        ranged = true;
    }
    if (d != kHeadDim) {
        // other head dims: the vector kernel over the row list, then the merge with row stride
        // 2 + dv (no partial at all gives every row O = 0 and LSE = -inf)
        if (n_kv > 0 && (st = run_segment(ctx, p, pool, false, k_pool->type, v_pool->type, slot, stream))) return st;
        ctx->stats.splits_window = slot;
        ctx->stats.n_partials = slot;
        hipError_t e = launch_merge_hd(ctx->partials, slot, p.n_rows, dv, o, lse, stream);
        if (e != hipSuccess) return hip_fail(e, "merge launch");
        return RKV_OK;
    }
    if (n_kv > 0) {
        if ((st = run_segment(ctx, p, pool, false, k_pool->type, v_pool->type, slot, stream))) return st;
    } else {
        hipError_t e0 = launch_empty_partials(ctx->partials, p.n_rows, stream);
        if (e0 != hipSuccess) return hip_fail(e0, "empty partial");
        slot = 1;
    }
    ctx->stats.splits_window = slot;
    ctx->stats.n_partials = slot;
    hipError_t e = launch_merge(ctx->partials, slot, p.n_rows, o, lse, nullptr, stream, ranged ? &mr : nullptr);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return RKV_OK;
}

int rkv_attn_partial(rkv_ctx *ctx, const rkv_tensor *q, const rkv_tensor *k, const rkv_tensor *v,
                     const rkv_tensor *mask, int64_t kv_pos0, int64_t q_pos0, float scale, float *partial,
                     void *stream_) {
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (!ctx) return fail(RKV_ERR_ARG, "ctx is NULL");
    int st = check_q(q, false, true);
    if (st) return st;
    if ((st = check_kv(k, "k", true, true)) || (st = check_kv(v, "v", false, true))) return st;
    if (k->ne[1] != v->ne[1] || k->ne[2] != v->ne[2]) return fail(RKV_ERR_ARG, "k and v disagree in shape");
    const int d = (int)q->ne[0], dv = (int)v->ne[0];
    if (k->ne[0] != d) return fail(RKV_ERR_ARG, "K head dim must equal Q's");
    if (!head_dims_supported(d, dv))
        return fail(RKV_ERR_UNSUPPORTED, "head dims dk=%d, dv=%d not supported (dk = dv in 64, 128, 256, 512, or 576/512)",
                    d, dv);
    if (kv_pos0 < 0 || q_pos0 < -1) return fail(RKV_ERR_ARG, "bad positions");
    if (!std::isfinite(scale)) return fail(RKV_ERR_ARG, "scale is not finite");
    const int64_t n_head = q->ne[2], n_q = q->ne[1], n_head_kv = k->ne[2];
    if (n_head % n_head_kv != 0) return fail(RKV_ERR_ARG, "n_head %% n_head_kv != 0");
    const int64_t gqa = n_head / n_head_kv;
    // the prefill kernel (head dims 128 and 64) above 8 rows per KV head, else the decode kernels
    const bool mfma = gqa * n_q > kMaxRowsVec && prefill_head_dims_ok(d, dv);
    if ((st = check_mask(mask, kv_pos0 + k->ne[1], n_q, 1))) return st;
    if (k->ne[1] > 0 && ((st = check_device_ptr(k->data, "k")) || (st = check_device_ptr(v->data, "v")))) return st;
    if ((st = check_device_ptr(partial, "partial"))) return st;
    if ((st = ensure_device(ctx))) return st;
    SegParams p{};
    fill_q(p, q);
    fill_mask(p, mask);
    p.q_pos0 = q_pos0;
    p.n_head = (int)n_head;
    p.n_head_kv = (int)n_head_kv;
    p.n_q = (int)n_q;
    p.n_seq = 1;
    p.gqa = (int)gqa;
    p.scale_log2 = scale * 1.4426950408889634f;
    fill_softcap(p, ctx, scale);
    p.n_rows = n_head * n_q;
    p.d = d;
    p.dv = dv;
    const Seg sg{static_cast<const uint8_t *>(k->data), static_cast<const uint8_t *>(v->data), k->nb[1], k->nb[2],
                 v->nb[1], v->nb[2], k->ne[1], kv_pos0};
    const int slots = plan_segment(ctx, p, sg, mfma, k->type, v->type).n_splits;
    if (dv != kHeadDim && slots > 1024)
        return fail(RKV_ERR_UNSUPPORTED, "%d partial slots: the merge into one partial takes up to 1024 at dv %d", slots, dv);
    if ((st = ensure_partials(ctx, (int64_t)slots * p.n_rows * (2 + dv), stream))) return st;
    p.partials = ctx->partials;
    ctx->stats = rkv_stats{};
    ctx->stats.kernel_variant = mfma ? RKV_KERNEL_PREFILL_MFMA : RKV_KERNEL_DECODE_HEAD;
    int slot = 0;
    if (k->ne[1] > 0) {
        if ((st = run_segment(ctx, p, sg, mfma, k->type, v->type, slot, stream))) return st;
    } else {
        hipError_t e0 = launch_empty_partials(ctx->partials, p.n_rows, stream, dv);
        if (e0 != hipSuccess) return hip_fail(e0, "empty partial");
        slot = 1;
    }
    ctx->stats.n_partials = slot;
    hipError_t e = dv == kHeadDim ? launch_merge(ctx->partials, slot, p.n_rows, nullptr, nullptr, partial, stream)
                                  : launch_merge_parts(ctx->partials, slot, p.n_rows, dv, nullptr, nullptr, stream, partial);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return RKV_OK;
}

int rkv_lse_merge(const float *partials, int n_seg, int64_t n_rows, int dv, float *o, float *lse, void *stream) {
    if (!head_dims_supported(dv, dv)) return fail(RKV_ERR_UNSUPPORTED, "dv must be 64, 128, 256 or 512");
    if (n_seg <= 0 || n_rows < 0) return fail(RKV_ERR_ARG, "n_seg must be > 0 and n_rows >= 0");
    if (n_rows == 0) return RKV_OK;
    int st = check_device_ptr(partials, "partials");
    if (st) return st;
    if ((st = check_device_ptr(o, "o"))) return st;
    if (lse && (st = check_device_ptr(lse, "lse"))) return st;
    hipError_t e = dv == kHeadDim
                       ? launch_merge(partials, n_seg, n_rows, o, lse, nullptr, static_cast<hipStream_t>(stream))
                       : launch_merge_hd(partials, n_seg, n_rows, dv, o, lse, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return RKV_OK;
}

int rkv_tail_lift(rkv_ctx *ctx, const void *host_src, int64_t nbytes, int slot, int mode, void **dev_dst,
                  void *copy_stream_) {
    if (!ctx || !host_src || !dev_dst) return fail(RKV_ERR_ARG, "NULL argument");
    if (slot < 0 || slot >= kMaxSlots) return fail(RKV_ERR_ARG, "slot out of range");
    if (nbytes < 0) return fail(RKV_ERR_ARG, "nbytes < 0");
    if (mode != RKV_LIFT_BULK && mode != RKV_LIFT_UVA && mode != RKV_LIFT_KERNEL)
        return fail(RKV_ERR_ARG, "unknown lift mode");
    if (mode == RKV_LIFT_KERNEL && ((uintptr_t)host_src) % 8 != 0)
        return fail(RKV_ERR_UNSUPPORTED, "the kernel lift needs an 8-byte aligned source");
    if (pointer_kind(host_src) != Mem::PinnedHost) return fail(RKV_ERR_ARG, "host_src is not pinned host memory");
    int st = ensure_device(ctx);
    if (st) return st;
    hipStream_t cs = copy_stream_ ? static_cast<hipStream_t>(copy_stream_) : ctx->copy_stream;
    if ((st = grow(&ctx->scr_k[slot], &ctx->cap_k[slot], (size_t)std::max<int64_t>(nbytes, 1), cs))) return st;
    if (mode == RKV_LIFT_UVA) {
        hipError_t e = launch_uva_read(host_src, ctx->scr_k[slot], nbytes, cs);
        if (e != hipSuccess) return hip_fail(e, "uva lift");
    } else if (mode == RKV_LIFT_KERNEL) {
        hipError_t e = launch_lift_copy(host_src, ctx->scr_k[slot], nbytes, cs);
        if (e != hipSuccess) return hip_fail(e, "kernel lift");
    } else if (nbytes > 0) {
        RKV_HIP(hipMemcpyAsync(ctx->scr_k[slot], host_src, (size_t)nbytes, hipMemcpyHostToDevice, cs));
    }
    RKV_HIP(hipEventRecord(ctx->copy_done[slot], cs));
    *dev_dst = ctx->scr_k[slot];
    return RKV_OK;
}

void rkv_bcache_destroy(rkv_bcache *bc) {
    if (!bc) return;
    int cur = -1;
    if (hipGetDevice(&cur) == hipSuccess && cur != bc->device) (void)hipSetDevice(bc->device);
    (void)hipDeviceSynchronize();
    if (bc->map_mem) (void)hipFree(bc->map_mem);
    if (bc->pool_k) (void)hipFree(bc->pool_k);
    if (bc->pool_v) (void)hipFree(bc->pool_v);
    (void)hipGetLastError();
    delete bc;
}

int rkv_bcache_create(const rkv_tensor *k_host, const rkv_tensor *v_host, int64_t page_size, int64_t n_slots,
                      rkv_bcache **out) {
    if (!out) return fail(RKV_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!k_host || !v_host) return fail(RKV_ERR_ARG, "k_host and v_host must be given");
    int st;
    if ((st = check_kv(k_host, "k_host", true, true)) || (st = check_kv(v_host, "v_host", false, true))) return st;
    const int64_t d = k_host->ne[0], n_cells = k_host->ne[1], n_head_kv = k_host->ne[2];
    if (v_host->ne[0] != d || v_host->ne[1] != n_cells || v_host->ne[2] != n_head_kv)
        return fail(RKV_ERR_ARG, "k_host and v_host disagree in shape");
    if (page_size < 1 || n_slots < 1 || n_slots > ((int64_t)1 << 28)) return fail(RKV_ERR_ARG, "bad page_size or n_slots");
    if (n_cells < 1 || n_cells % page_size != 0) return fail(RKV_ERR_ARG, "the host copy must hold whole pages");
    const int64_t n_pages = n_cells / page_size;
    if (n_pages > ((int64_t)1 << 30) || n_slots * page_size > ((int64_t)1 << 31) - 1)
        return fail(RKV_ERR_UNSUPPORTED, "cache too large for 32-bit pages and rows");
    const int64_t k_row = row_bytes(k_host->type, d), v_row = row_bytes(v_host->type, d);
    for (const rkv_tensor *t : {k_host, v_host}) {
        const int64_t rb = t == k_host ? k_row : v_row;
        if (n_head_kv > 1 && t->nb[2] != rb) return fail(RKV_ERR_UNSUPPORTED, "the host copy must be cell-major (heads packed in a cell)");
        if (t->nb[1] < n_head_kv * rb) return fail(RKV_ERR_ARG, "cell stride shorter than a cell");
        if ((page_size * t->nb[1]) % 16 != 0 || ((uintptr_t)t->data) % 16 != 0 || (n_head_kv * rb) % 4 != 0)
            return fail(RKV_ERR_UNSUPPORTED, "pages must be 16-byte multiples on 16-byte aligned host memory");
        if (pointer_kind(t->data) != Mem::PinnedHost) return fail(RKV_ERR_ARG, "the host copy must be pinned host memory");
    }
    int dev = 0;
    RKV_HIP(hipGetDevice(&dev));
    rkv_bcache *bc = new rkv_bcache();
    bc->device = dev;
    bc->k_type = k_host->type;
    bc->v_type = v_host->type;
    bc->d = d;
    bc->n_cells = n_cells;
    bc->n_head_kv = n_head_kv;
    bc->k_s1 = k_host->nb[1];
    bc->v_s1 = v_host->nb[1];
    bc->k_row = k_row;
    bc->v_row = v_row;
    bc->page_size = page_size;
    bc->n_slots = n_slots;
    auto bail = [&](int status, const char *what) {
        rkv_bcache_destroy(bc);
        return fail(status, "%s", what);
    };
    void *vk = nullptr, *vv = nullptr;
    if (hipHostGetDevicePointer(&vk, const_cast<void *>(k_host->data), 0) != hipSuccess ||
        hipHostGetDevicePointer(&vv, const_cast<void *>(v_host->data), 0) != hipSuccess) {
        (void)hipGetLastError();
        return bail(RKV_ERR_HIP, "no device view of the host copy");
    }
    bc->view_k = static_cast<uint8_t *>(vk);
    bc->view_v = static_cast<uint8_t *>(vv);
    const size_t map_ints = (size_t)n_pages + 6 * (size_t)n_slots + kBcCtl + 8;
    if (hipMalloc(&bc->map_mem, map_ints * sizeof(int32_t)) != hipSuccess ||
        hipMalloc(reinterpret_cast<void **>(&bc->pool_k), (size_t)(n_slots * page_size * bc->k_s1)) != hipSuccess ||
        hipMalloc(reinterpret_cast<void **>(&bc->pool_v), (size_t)(n_slots * page_size * bc->v_s1)) != hipSuccess) {
        (void)hipGetLastError();
        return bail(RKV_ERR_NOMEM, "device memory for the block cache");
    }
    int32_t *base = static_cast<int32_t *>(bc->map_mem);
    bc->m.ctl = base;  // first, so its 64-bit counters are 8-byte aligned
    bc->m.page_table = base + kBcCtl;
    bc->m.slot_page = bc->m.page_table + n_pages;
    bc->m.slot_stamp = bc->m.slot_page + n_slots;
    bc->m.slot_ref = bc->m.slot_stamp + n_slots;
    bc->m.miss_page = bc->m.slot_ref + n_slots;
    bc->m.miss_slot = bc->m.miss_page + n_slots;
    bc->m.n_pages = n_pages;
    bc->m.n_slots = n_slots;
    bc->m.page_size = (int)page_size;
    hipError_t e = launch_bc_reset(bc->m, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return bail(RKV_ERR_HIP, "block cache reset");
    }
    *out = bc;
    return RKV_OK;
}

int rkv_bcache_reset(rkv_bcache *bc, void *stream) {
    if (!bc) return fail(RKV_ERR_ARG, "bc is NULL");
    hipError_t e = launch_bc_reset(bc->m, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "block cache reset");
    return RKV_OK;
}

int rkv_bcache_resolve(rkv_bcache *bc, const int32_t *sel, int64_t n_sel, int n_seq, int32_t *rows, void *stream) {
    if (!bc) return fail(RKV_ERR_ARG, "bc is NULL");
    if (n_sel < 0 || n_seq < 1 || n_sel * n_seq > ((int64_t)1 << 31) - 1) return fail(RKV_ERR_ARG, "bad n_sel or n_seq");
    if (n_sel == 0) return RKV_OK;
    int st;
    if ((st = check_device_ptr(sel, "sel"))) return st;
    if (rows && (st = check_device_ptr(rows, "rows"))) return st;
    hipError_t e = launch_bc_resolve(bc->m, sel, n_sel, n_seq, bc->view_k, bc->view_v, bc->pool_k, bc->pool_v,
                                     bc->page_size * bc->k_s1, bc->page_size * bc->v_s1, rows,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "block cache resolve");
    return RKV_OK;
}

int rkv_bcache_pools(const rkv_bcache *bc, rkv_tensor *k_pool, rkv_tensor *v_pool) {
    if (!bc || !k_pool || !v_pool) return fail(RKV_ERR_ARG, "NULL argument");
    const int64_t rows = bc->n_slots * bc->page_size;
    const int64_t kb = bc->k_type == RKV_TYPE_F16 ? 2 : 34, vb = bc->v_type == RKV_TYPE_F16 ? 2 : 18;
    *k_pool = rkv_tensor{bc->pool_k, bc->k_type, {bc->d, rows, bc->n_head_kv, 1}, {kb, bc->k_s1, bc->k_row, rows * bc->k_s1}};
    *v_pool = rkv_tensor{bc->pool_v, bc->v_type, {bc->d, rows, bc->n_head_kv, 1}, {vb, bc->v_s1, bc->v_row, rows * bc->v_s1}};
    return RKV_OK;
}

int rkv_bcache_append(rkv_bcache *bc, const void *k_cell, const void *v_cell, int64_t cell, void *stream) {
    if (!bc || !k_cell || !v_cell) return fail(RKV_ERR_ARG, "NULL argument");
    if (cell < 0 || cell >= bc->n_cells) return fail(RKV_ERR_ARG, "cell %lld outside the cache", (long long)cell);
    if (((uintptr_t)k_cell | (uintptr_t)v_cell) % 4 != 0) return fail(RKV_ERR_ARG, "cell data must be 4-byte aligned");
    int st;
    if ((st = check_device_ptr(k_cell, "k_cell")) || (st = check_device_ptr(v_cell, "v_cell"))) return st;
    hipError_t e = launch_bc_append(bc->m, k_cell, v_cell, bc->n_head_kv * bc->k_row, bc->n_head_kv * bc->v_row, cell,
                                    bc->view_k, bc->view_v, bc->pool_k, bc->pool_v, bc->k_s1, bc->v_s1,
                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "block cache append");
    return RKV_OK;
}

int rkv_bcache_counters(rkv_bcache *bc, rkv_bcache_stats *out) {
    if (!bc || !out) return fail(RKV_ERR_ARG, "NULL argument");
    int32_t c[kBcCtl] = {};
    RKV_HIP(hipDeviceSynchronize());
    RKV_HIP(hipMemcpy(c, bc->m.ctl, sizeof c, hipMemcpyDeviceToHost));
    uint64_t u[3];
    std::memcpy(u, c + 4, sizeof u);
    out->misses = u[0];
    out->lookups = u[1];
    out->calls = u[2];
    out->epoch = c[0];
    out->hand = c[1];
    out->last_misses = c[2];
    out->overflow = c[3];
    return RKV_OK;
}

int rkv_bcache_map(const rkv_bcache *bc, int32_t **page_table, int32_t **slot_page, int64_t *n_pages, int64_t *n_slots) {
    if (!bc || !page_table || !slot_page || !n_pages || !n_slots) return fail(RKV_ERR_ARG, "NULL argument");
    *page_table = bc->m.page_table;
    *slot_page = bc->m.slot_page;
    *n_pages = bc->m.n_pages;
    *n_slots = bc->m.n_slots;
    return RKV_OK;
}

int rkv_dequant_rows(const void *src, int type, int form, int64_t n_rows, int64_t row_values, int64_t row_stride,
                     float *dst, void *stream) {
    if (type != RKV_TYPE_F16 && type != RKV_TYPE_Q8_0 && type != RKV_TYPE_Q4_0)
        return fail(RKV_ERR_UNSUPPORTED, "type %d", type);
    if (form < RKV_DQ_DECODE_MMA || form > RKV_DQ_HEAD_DIM) return fail(RKV_ERR_ARG, "unknown form %d", form);
    if (row_values <= 0 || row_values > 4096 || row_values % 32 != 0) return fail(RKV_ERR_ARG, "row_values must be a multiple of 32 in [32, 4096]");
    if (n_rows < 0 || row_stride < row_bytes(type, row_values)) return fail(RKV_ERR_ARG, "bad n_rows or row_stride");
    if (n_rows == 0) return RKV_OK;
    if (n_rows > ((int64_t)1 << 30)) return fail(RKV_ERR_ARG, "too many rows");
    int st = check_device_ptr(src, "src");
    if (st) return st;
    if ((st = check_device_ptr(dst, "dst"))) return st;
    hipError_t e = launch_dequant_rows(src, type, form, n_rows, (int)row_values, row_stride, dst,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dequant launch");
    return RKV_OK;
}

}  // extern "C"
