/*
 * rkv.h -- C ABI of librkv: flash attention over a KV cache split into position
 * segments, for AMD Instinct MI355X (gfx950).
 *
 * The cache is split in one of two ways:
 *   - a device-resident window of cells [0, wc) plus a tail [wc, n_kv) that may sit in
 *     pinned host memory and is lifted to the GPU tile by tile
 *     (opencoti-llamafile patch 0070-rolling-kv, commit message "position-windowed KV
 *     residency" and fattn.cu ggml_cuda_streaming_flash_attn; patch
 *     0102-fattn-bulk-h2d-scratch-ring, bulk raw-quant lift and persistent scratch ring);
 *   - an arbitrary per-sequence list of rows into a shared cell pool
 *     (llama.cpp PR #29510 "flash_attn_ext_rows", API comment in ggml.h).
 * Every segment yields a partial (M, S, VKQ) per output row and a log-sum-exp merge
 * combines the partials (patch 0070, fattn.cu header comment and streaming_combine_kernel).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are described ggml-style: ne[0] is the fastest dimension, nb[] are byte
 * strides, nb[0] is the element (or quant block) size.  Rows of head_dim values must be
 * contiguous (nb[0] == type size).  Supported head dims (patch 0070, fattn.cu: the streaming
 * op's supported shapes): head_dim == dv in {64, 128, 256, 512}, and head_dim 576 for Q and
 * K with dv 512 for V, on every attention entry point and the host tail partial.  Decode
 * over cell-major caches runs on the matrix-core kernels: q8_0 K / q4_0 V at head_dim == dv in
 * {64, 128, 256, 512} and at 576 / 512 when the KV heads form groups the kernel takes (8 or 4
 * at 64; 8, 4 or 2 at 128; 4, 2 or 1 at 256; 1 at 512 and 576), with n_q * gqa <= 8 at 128 and
 * any number of rows at the other head dims; binary16 K and V at head_dim == dv in {64, 128,
 * 256, 512} in groups of 8, 8, 4 and 2 KV heads, and at 576 / 512 one head at a time, with
 * n_q * gqa <= 8 at 128 and any number of rows at the other head dims (row groups of 16).  Prefill at 128, and
 * at 64 with more than 8 rows per KV head, runs on the matrix-core prefill kernel; everything
 * else on the vector kernels; rkv_lse_merge takes
 * dv 64, 128, 256 or 512; Q in F16;
 * K in F16 or Q8_0; V in F16 or Q4_0.  Q8_0 is a 34-byte block (binary16 scale d, 32
 * int8 codes q; value d*q).  Q4_0 is an 18-byte block (binary16 scale d, 16 bytes; byte
 * j holds element j in its low nibble and element j+16 in its high nibble; value
 * d*(n-8)).  K/V data pointers and their nb[1], nb[2] must be multiples of 8 bytes (of 4
 * bytes for head dims other than 128); Q pointers and strides multiples of 4 bytes.
 *
 *   score s_j = scale * <q, k_j> + mask[j]   (mask additive binary16, -inf hides;
 *                                             column j is the GLOBAL key position)
 *   grouped-query map: query head h reads KV head h / (n_head / n_head_kv).
 *   O = softmax-weighted sum of v_j over visible keys; LSE = ln sum_j exp(s_j).
 *   A row with no visible key gets O = 0 and LSE = -inf.
 *
 * Output layouts: O is float32 [dv, n_head, n_q(, n_seq)] contiguous; LSE is float32
 * [n_head, n_q(, n_seq)] contiguous; output row index r = h + n_head*(i + n_q*b).
 * Partials are float32 [n_seg][n_rows][2 + dv] holding (M, S, VKQ[dv]) with
 * M = max_j s_j (natural-log units), S = sum_j exp(s_j - M), VKQ = sum_j exp(s_j - M) v_j;
 * an empty segment is (-inf, 0, 0...).
 *
 * Every call returns an rkv_status.  Arguments are validated on the host before any
 * device work; nothing aborts across the ABI.  Work is enqueued on the caller's stream
 * (a hipStream_t passed as void*; NULL = the legacy default stream) and the call returns
 * without waiting.  Device faults surface as RKV_ERR_HIP on a later call.
 * rkv_last_error() gives a human-readable reason for the last non-OK status on the
 * calling thread.
 *
 * Ownership: the caller owns every input and output buffer.  An rkv_ctx owns its copy
 * stream, its pre-created events, its persistent grow-only scratch ring and its partials
 * workspace.  One context serves one stream at a time and is not re-entrant.
 */
#ifndef RKV_H
#define RKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rkv_ctx rkv_ctx;

enum rkv_type { RKV_TYPE_F32 = 0, RKV_TYPE_F16 = 1, RKV_TYPE_Q4_0 = 2, RKV_TYPE_Q8_0 = 8 };

enum rkv_status {
    RKV_OK = 0,
    RKV_ERR_ARG = -1,          /* malformed argument (shape, stride, pointer kind)        */
    RKV_ERR_UNSUPPORTED = -2,  /* well-formed but outside what the kernels implement      */
    RKV_ERR_HIP = -3,          /* a HIP runtime call failed                                */
    RKV_ERR_NOMEM = -4,        /* device, pinned or host allocation failed                */
    RKV_ERR_CAPTURE = -5       /* workspace growth needed while the stream is capturing    */
};

enum rkv_lift_mode {
    RKV_LIFT_BULK = 0,  /* hipMemcpyAsync DMA of the raw bytes into the scratch ring         */
    RKV_LIFT_UVA = 1,   /* contrast only: a kernel reads the pinned host bytes word by word  */
    RKV_LIFT_KERNEL = 2,/* a copy kernel on the copy stream (at most 64 workgroups) reads the
                           pinned bytes 8 at a time: no hand-off between a DMA engine and the
                           compute queue, which dominates small lifts                        */
    RKV_LIFT_AUTO = 3,  /* default: decode reads a small tail in place (RKV_LIFT_DIRECT's
                           read; at most rkv_set_direct_tail_max bytes, 8 MiB by default, and
                           up to 8 rows per KV head) and lifts larger ones with the copy
                           kernel; prefill lifts with the DMA engine (the copy kernel's
                           workgroups would slow the MFMA kernel it overlaps)               */
    RKV_LIFT_DIRECT = 4 /* no lift (patch 0102, commit message: the kernel reading the pinned
                           tail at word granularity, there the slow contrast to the bulk
                           lift): the segment kernels read a pinned tail in place through
                           its device view, in their own access order; a device tail and the
                           host tail partial are unaffected                                  */
};

enum rkv_residency_mode {
    RKV_RESIDENCY_AUTO = 0,      /* window + tail when eligible                            */
    RKV_RESIDENCY_RESIDENT = 1,  /* never split the cache by position                      */
    RKV_RESIDENCY_WINDOW = 2     /* window + tail when eligible, resident otherwise        */
};

enum rkv_tail_mode {
    RKV_TAIL_LIFT = 0,  /* host tail lifted tile by tile into the scratch ring (default)     */
    RKV_TAIL_HOST = 1   /* decode: the host cores compute the tail's partial; only the
                           partial crosses PCIe (rkv_set_tail_mode)                           */
};

typedef struct rkv_tensor {
    const void *data;
    int32_t type;   /* enum rkv_type */
    int64_t ne[4];
    int64_t nb[4];
} rkv_tensor;

/* Statistics of the last attention call on a context (host-side planning facts). */
typedef struct rkv_stats {
    int32_t n_segments;       /* device segments launched (window, tail tiles, ...)      */
    int32_t n_partials;       /* partial slots merged                                    */
    int32_t n_tail_tiles;     /* tail tiles lifted                                       */
    int32_t lift_mode;        /* enum rkv_lift_mode used for the tail                    */
    int64_t lift_bytes;       /* raw bytes lifted host -> device                         */
    int32_t splits_window;    /* split-K factor used on the window segment               */
    int32_t kernel_variant;   /* enum rkv_kernel_variant of the last segment launched    */
    int32_t tail_host;        /* 1 if the tail partial was computed on the host cores     */
    float host_tail_ms;       /* wall time of that host computation                      */
} rkv_stats;

/* Segment kernel families (rkv_stats.kernel_variant). */
enum rkv_kernel_variant {
    RKV_KERNEL_DECODE_HEAD = 0,       /* vector decode, one KV head per workgroup (any layout, rows) */
    RKV_KERNEL_PREFILL_MFMA = 1,      /* matrix-core prefill over 256-row query tiles                */
    RKV_KERNEL_DECODE_CELL = 2,       /* vector decode over cell-major groups of KV heads           */
    RKV_KERNEL_DECODE_CELL_MFMA = 3,  /* matrix-core decode over cell-major q8_0/q4_0 head groups   */
    RKV_KERNEL_DECODE_CELL_MFMA16 = 4, /* persistent matrix-core decode over cell groups of binary16
                                          heads: 8 at head dims 64 and 128, 4 at 256, 2 at 512,
                                          1 at 576 / 512
                                          (windows, tail tiles, row lists)                         */
    RKV_KERNEL_DECODE_HD = 5           /* vector decode for head dims other than 128 (window + tail) */
};

/* ---- context ---------------------------------------------------------------------- */

/* Create a context on `device`: a non-blocking copy stream at default priority and a
 * pool of pre-created events (never created during graph capture, as patch 0070's
 * copy/compute double buffer requires).  Returns RKV_ERR_HIP if the device is absent. */
int rkv_create(int device, rkv_ctx **out);

/* Grow (never shrink) the persistent scratch ring and partials workspace so that later
 * calls allocate nothing; call it before capturing a stream into a graph.  Each of the
 * n_slots (1..4) ring slots holds max_tile_bytes_k of K and max_tile_bytes_v of V
 * (patch 0102: worst-case tile capacity, persistent per-slot scratch).  max_partial_floats
 * sizes the partials workspace.  Zero arguments leave that part unchanged. */
int rkv_reserve(rkv_ctx *ctx, int64_t max_tile_bytes_k, int64_t max_tile_bytes_v,
                int n_slots, int64_t max_partial_floats);

/* Free everything the context owns (synchronises its device first). NULL is a no-op. */
void rkv_destroy(rkv_ctx *ctx);

const char *rkv_strerror(int status);
const char *rkv_last_error(void);
int rkv_get_stats(const rkv_ctx *ctx, rkv_stats *out);

/* Choose how tail tiles are lifted by later calls on this context (enum rkv_lift_mode;
 * RKV_LIFT_AUTO until set).  RKV_LIFT_UVA exists only to measure the word-granularity host
 * read of patch 0102's commit message against the bulk copies; it is never the default.
 * rkv_stats.lift_mode reports the mode a call used. */
int rkv_set_lift_mode(rkv_ctx *ctx, int mode);

/* Under RKV_LIFT_AUTO, decode calls read a pinned tail of at most `bytes` bytes (its K plus
 * V bytes) in place instead of lifting it, when there are at most 8 query rows per KV head
 * (each segment kernel then reads every tail byte once).  Default 8 MiB: on the 128-dim
 * decode the in-place read beat the lift below that (one launch and one hand-off between
 * streams fewer) and the two were even above it.  0 lifts every tail; bytes < 0 is
 * RKV_ERR_ARG. */
int rkv_set_direct_tail_max(rkv_ctx *ctx, int64_t bytes);

/* Override the split-K factor of window/pool segments (0 = automatic). */
int rkv_set_splits(rkv_ctx *ctx, int splits);

/* Measurement aid: when on, later calls record timing events around each tail-tile lift on
 * the copy stream (up to 64 per call). */
int rkv_set_lift_timing(rkv_ctx *ctx, int on);

/* Waits for the last call's timed lifts and reports the sum of their durations, the span
 * from the first lift's start to the last lift's end, and how many were timed. */
int rkv_lift_timing_ms(rkv_ctx *ctx, float *total_ms, float *span_ms, int *n_lifts);

/* Measurement aid: when on, every later segment-kernel launch (the per-segment decode, rows
 * or prefill kernel, not the merge) is bracketed by timing events on the stream it is
 * launched on, up to 4096 launches; turning it on resets the record. */
int rkv_set_kernel_timing(rkv_ctx *ctx, int on);

/* Waits for the recorded launches and reports the sum of their durations and their count. */
int rkv_kernel_timing_ms(rkv_ctx *ctx, float *total_ms, int *n_launches);

/* ---- attention -------------------------------------------------------------------- */

/* Decode attention over a window + tail split (patch 0070, ggml_streaming_flash_attn_window:
 * window K/V in one pair of sources, tail K/V in another, a NULL tail meaning one region;
 * tiles never straddle wc; the mask is sliced at the global position).
 * Shown for head_dim 128; head_dim 64, 256 or 512 (Q, K and V alike), or 576 for Q and K
 * with 512 for V (o then [512, n_head, n_q]), takes the same arguments with those leading
 * extents; any other pair of head dims is RKV_ERR_UNSUPPORTED.
 *   q       F16 [128, n_q, n_head, 1], device.  n_q * (n_head/n_head_kv) <= 8 at head dim
 *           128 (any number at the other head dims, in groups of 8 rows).
 *   k_win   [128, >= wc, n_head_kv, 1] device (cells [0, wc) are used); NULL iff wc == 0.
 *   v_win   as k_win with V's type.
 *   k_tail  [128, n_tail, n_head_kv, 1] or NULL.  Pinned host memory (lifted in tiles of
 *           tile_kv cells through the context's scratch ring on its copy stream,
 *           double-buffered against compute) or device memory (read in place).
 *           A pinned host tail must be cell-major-contiguous per tile
 *           (nb[1] >= n_head_kv*row and heads inside a cell) or head-major; pageable host
 *           memory is RKV_ERR_ARG.
 *   mask    F16 [>= n_kv, >= n_q, 1, 1] additive, device, or NULL (all keys visible).
 *   n_kv    = wc + n_tail.  tile_kv > 0.
 *   o       float32 [128, n_head, n_q] device; lse float32 [n_head, n_q] device or NULL.
 * Stream-ordered on `stream`; returns once enqueued. */
int rkv_attn_decode(rkv_ctx *ctx, const rkv_tensor *q,
                    const rkv_tensor *k_win, const rkv_tensor *v_win,
                    const rkv_tensor *k_tail, const rkv_tensor *v_tail,
                    const rkv_tensor *mask, int64_t wc, int64_t tile_kv, float scale,
                    float *o, float *lse, void *stream);

/* Allocation-free decode, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same computation
 * and kernels as rkv_attn_decode over a device-resident cache (k, v hold all n_kv = k->ne[1]
 * keys; no tail), without a context: its split-K partials live in a file-scope device array of
 * 8 MiB (2^21 floats) that each GPU holds from the first call until the process ends.  The
 * first call on a device looks that array's address up (hipGetSymbolAddress); no call
 * allocates.  When the planned partials exceed the array, fewer splits are used (results stay
 * within the decode tolerances, possibly not bit-identical to rkv_attn_decode); a shape whose
 * single partial (n_head * n_q * (2 + dv) floats) exceeds it is RKV_ERR_UNSUPPORTED.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race and give wrong results; serialise them.
 *   q, k, v, mask, scale, o, lse as rkv_attn_decode (k_win = k, v_win = v, wc = n_kv); the
 *   logit soft-cap is off.  Enqueued on `stream` (the calling thread's current device). */
int rkv_attn_decode_noalloc(const rkv_tensor *q, const rkv_tensor *k, const rkv_tensor *v,
                            const rkv_tensor *mask, float scale, float *o, float *lse, void *stream);

/* Prefill attention (patch 0070, fattn.cu ggml_cuda_streaming_flash_attn: the same window +
 * tail streaming op serves a multi-token chunk, with the mask sliced at the global key
 * position, a per-tile flash attention and an LSE per tile for the combine; patch 0102,
 * commit message: 106k-token prefills through lifted tail tiles).  The same arguments as
 * rkv_attn_decode for any n_q, computed at head dim 128 (and at head dim 64 when n_q * gqa
 * > 8) with MFMA f16 tiles: q8_0 K enters the matrix cores as the exact two-part binary16 sum
 * hi + lo = d*q, q4_0 V as the exact binary16 integers n - 8 with the block scales folded
 * into the softmax weights; the other head dims, and 64 with up to 8 rows per KV head, run on
 * the decode kernels (the q8_0 / q4_0 and binary16 matrix-core kernels for any n_q * gqa, in
 * row groups of 16, when the KV heads form their groups; else the vector kernel in groups of
 * 8 rows).  The tail is always computed on the GPU
 * (RKV_TAIL_HOST applies to decode only).  q_pos0 >= 0 makes it
 * causal: query i sits at absolute position q_pos0 + i and sees keys at positions
 * <= q_pos0 + i (in addition to the mask); q_pos0 == -1 uses the mask alone. */
int rkv_attn_prefill(rkv_ctx *ctx, const rkv_tensor *q,
                     const rkv_tensor *k_win, const rkv_tensor *v_win,
                     const rkv_tensor *k_tail, const rkv_tensor *v_tail,
                     const rkv_tensor *mask, int64_t wc, int64_t tile_kv, float scale,
                     int64_t q_pos0, float *o, float *lse, void *stream);

/* Unified-pool attention (llama.cpp PR #29510, ggml_flash_attn_ext_rows): each sequence
 * b attends to its own list of pool rows.
 *   q       F16 [128, n_q, n_head, n_seq] device, n_q * (n_head/n_head_kv) <= 8 at head dim
 *           128 (other head dims as for rkv_attn_decode, any number of rows).
 *   k_pool  [128, n_pool, n_head_kv, 1] device, shared by all sequences; v_pool likewise.
 *   kv_rows int32 [n_kv, n_seq] device, contiguous: key j of sequence b is pool row
 *           kv_rows[j + n_kv*b].  A negative row, or one >= n_pool, is padding: it
 *           contributes nothing and is never dereferenced.  Cell-major q8_0 K / q4_0 V pools
 *           run on the matrix-core decode kernel at every supported head dim, binary16 pools
 *           in groups of 8, 8, 4 or 2 KV heads at head dims 64, 128, 256 or 512 (dk = dv), and
 *           at 576 / 512, on the persistent binary16 kernel, the rest on the vector kernels.
 *   mask    F16 [>= n_kv, >= n_q, 1, n_seq] additive, device, or NULL.
 *   o       float32 [128, n_head, n_q, n_seq]; lse float32 [n_head, n_q, n_seq] or NULL. */
int rkv_attn_rows(rkv_ctx *ctx, const rkv_tensor *q, const rkv_tensor *k_pool,
                  const rkv_tensor *v_pool, const int32_t *kv_rows, int64_t n_kv,
                  const rkv_tensor *mask, float scale, float *o, float *lse, void *stream);

/* One segment's partial over device-resident K/V (the per-segment step of the method):
 * writes (M, S, VKQ) for every output row (row = query * n_head + head) into `partial`
 * float32 [n_rows][2 + dv], at every supported head-dim pair.
 * kv_pos0 is the global position of the segment's first cell (mask column offset and
 * causal position); q_pos0 as in rkv_attn_prefill (-1 = mask only).  Chooses the decode
 * kernels when n_q * gqa <= 8 and at head dims 256, 512 and 576 / 512, the MFMA prefill
 * kernel otherwise (head dims 128 and 64).  An empty segment writes (-inf, 0, 0...). */
int rkv_attn_partial(rkv_ctx *ctx, const rkv_tensor *q, const rkv_tensor *k,
                     const rkv_tensor *v, const rkv_tensor *mask, int64_t kv_pos0,
                     int64_t q_pos0, float scale, float *partial, void *stream);

/* Log-sum-exp merge (patch 0070 streaming_combine_kernel; the tail-partial rule of
 * tail_partial_to_tile_kernel): partials float32 [n_seg][n_rows][2 + dv] on the device
 * -> o float32 [dv, n_rows] and lse float32 [n_rows] (lse may be NULL).  Rows whose
 * segments are all empty get O = 0 and LSE = -inf.  dv is 64, 128, 256 or 512 (otherwise
 * RKV_ERR_UNSUPPORTED).  No context needed. */
int rkv_lse_merge(const float *partials, int n_seg, int64_t n_rows, int dv,
                  float *o, float *lse, void *stream);

/* Lift nbytes raw bytes (binary16 or quant blocks, copied as they are) from pinned host
 * memory into ring slot `slot` of the context (patch 0102: bulk H2D of the raw quant
 * tail into a persistent per-slot scratch ring; K uses the slot's first buffer).
 * *dev_dst receives the slot's device address.  mode RKV_LIFT_BULK issues one
 * hipMemcpyAsync on copy_stream; RKV_LIFT_UVA launches the word-granularity reader
 * kernel instead (contrast measurement); RKV_LIFT_KERNEL the bulk copy kernel (host_src
 * 8-byte aligned).  The slot's copy-done event is recorded on
 * copy_stream.  copy_stream NULL means the context's own copy stream.  The ring grows on
 * demand outside graph capture (RKV_ERR_CAPTURE inside it). */
int rkv_tail_lift(rkv_ctx *ctx, const void *host_src, int64_t nbytes, int slot, int mode,
                  void **dev_dst, void *copy_stream);

/* Tail mode of later rkv_attn_decode calls (patch 0070, the CPU_FA_TAIL tactic: the CPU
 * tail-partial op ggml_flash_attn_ext_tail_partial emits [M, S, VKQ] per output row over the
 * host-resident tail, and the device merges that partial with the window's through the
 * unchanged combine, so only 2 + dv floats per row cross PCIe).
 *   mode      RKV_TAIL_LIFT (default) or RKV_TAIL_HOST.  In RKV_TAIL_HOST a decode call whose
 *             tail is in host memory (pinned or pageable) copies Q and the tail's mask columns
 *             to pinned host buffers of the context, enqueues the window kernels, computes
 *             the tail partial on n_threads host threads while they run, uploads it into the
 *             partials workspace and merges.  The call therefore blocks the calling thread
 *             until Q has reached the host and the tail partial is done; it cannot be
 *             captured (RKV_ERR_CAPTURE).  A tail in device memory, and rkv_attn_prefill,
 *             are computed on the GPU as before.
 *   n_threads host threads (0 = the hardware threads, at most 16).
 * Errors: RKV_ERR_ARG for a NULL context, an unknown mode or n_threads outside [0, 256].
 * The host computation needs a CPU with AVX2, FMA and F16C (RKV_ERR_UNSUPPORTED at the call
 * otherwise). */
int rkv_set_tail_mode(rkv_ctx *ctx, int mode, int n_threads);

/* The tail partial on the host cores alone (the same computation RKV_TAIL_HOST runs):
 * partial float32 [n_head * n_q][2 + dv] in host memory receives (M, S, VKQ) for every row
 * r = h + n_head*i over the keys of k/v (fp32 accumulation; an empty row is (-inf, 0, 0...)).
 *   q        F16 [128, n_q, n_head, 1] in host memory (rows contiguous, even strides).
 *   k, v     [128, n_cells, n_head_kv, 1] in host memory: K F16 or Q8_0, V F16 or Q4_0,
 *            any cell and head strides (cell-major or head-major).
 *   mask     F16 [>= kv_pos0 + n_cells, >= n_q, 1, 1] additive, host memory, or NULL; column
 *            kv_pos0 + j belongs to cell j (global positions, as on the device).
 *   kv_pos0  global position of cell 0; q_pos0 >= 0 makes it causal as in rkv_attn_prefill,
 *            -1 uses the mask alone.  softcap as rkv_set_softcap (0 = none).
 *   n_threads host threads (0 = the hardware threads, at most 16).
 * Synchronous; makes no HIP call, so it runs without a GPU.  Every pointer must be host
 * memory (a device pointer is a contract violation).  Errors: RKV_ERR_ARG / RKV_ERR_UNSUPPORTED
 * as for the device entry points, RKV_ERR_UNSUPPORTED on a CPU without AVX2, FMA and F16C. */
int rkv_tail_partial_host(const rkv_tensor *q, const rkv_tensor *k, const rkv_tensor *v,
                          const rkv_tensor *mask, int64_t kv_pos0, int64_t q_pos0, float scale,
                          float softcap, float *partial, int n_threads);

/* Tail tactic from measured rates (patch 0070: the CPU_FA_TAIL tactic exists for slow links,
 * and an effective host-to-device bandwidth knob, autodetected or set by hand, drives the
 * streaming path).  A lifted tail moves its tail_bytes over the link at h2d_gbps; a host tail
 * partial reads them on the host cores at host_gbps, and only 2 + dv floats per row cross the
 * link.  *mode receives RKV_TAIL_HOST when tail_bytes / host_gbps < tail_bytes / h2d_gbps,
 * RKV_TAIL_LIFT otherwise (the default wins ties and an empty tail).  Pure host arithmetic.
 * Errors: RKV_ERR_ARG for a NULL mode, a negative size or a rate that is not finite and > 0. */
int rkv_choose_tail_mode(int64_t tail_bytes, double h2d_gbps, double host_gbps, int *mode);

/* Logit soft-cap of every later attention call on the context (patch 0070,
 * streaming_lse_kernel soft-cap branch): each scaled score scale*<q,k> becomes
 * softcap * tanh(scale*<q,k> / softcap), before the mask is added.  0 (the default) turns
 * it off.  Errors: RKV_ERR_ARG for a NULL context or a negative or non-finite value. */
int rkv_set_softcap(rkv_ctx *ctx, float softcap);

/* ---- device-side block cache ---------------------------------------------------------- */
/* Strata compare v0.1.2...v0.1.6, "KV streaming for the QSA layers" (kv_stream.hpp header
 * comment, kv_stream.cu): the authoritative K/V stay in pinned host memory; device memory holds
 * n_slots pages of page_size cells and a residency map; before a sparse read, a resolve call
 * makes every page the selection names resident on the device, inside the stream (capturable:
 * nothing is allocated after rkv_bcache_create), and translates the selection into rows of the
 * device slot pools, which rkv_attn_rows then reads like any pool. */
typedef struct rkv_bcache rkv_bcache;

typedef struct rkv_bcache_stats {
    uint64_t misses;      /* pages copied into slots over all resolve calls               */
    uint64_t lookups;     /* selection entries whose predecessor names another page       */
    uint64_t calls;       /* resolve calls                                                */
    int32_t epoch;        /* = calls since the last reset                                 */
    int32_t hand;         /* clock hand (next slot the sweep examines)                    */
    int32_t last_misses;  /* pages placed by the last call                                */
    int32_t overflow;     /* 1 once a call named more pages than it could place           */
} rkv_bcache_stats;

/* Create a block cache over the host copy k_host / v_host: [d, n_cells, n_head_kv, 1] (d in
 * {64, 128, 256}; K F16 or Q8_0, V F16 or Q4_0), cell-major with the heads packed inside a cell,
 * in pinned host memory the caller owns and keeps alive (16-byte aligned; page_size * nb[1] a
 * multiple of 16 bytes; n_cells a multiple of page_size).  Allocates the map (page table,
 * slot arrays, counters) and the two slot pools (n_slots * page_size cells each, cell stride
 * nb[1]) on the current device, every page absent.  Errors: RKV_ERR_ARG / RKV_ERR_UNSUPPORTED
 * for malformed or unsupported shapes and memory kinds, RKV_ERR_NOMEM. */
int rkv_bcache_create(const rkv_tensor *k_host, const rkv_tensor *v_host, int64_t page_size,
                      int64_t n_slots, rkv_bcache **out);
void rkv_bcache_destroy(rkv_bcache *bc);

/* Every page absent, every slot free, counters zero (enqueued on `stream`). */
int rkv_bcache_reset(rkv_bcache *bc, void *stream);

/* Make resident every page named by sel, int32 [n_sel, n_seq] device memory (cell ids, -1 =
 * padding; each list preferably ascending, which makes one lookup per page run): resident pages
 * take this call's epoch and reference bit; each missing page is claimed once and gets a victim
 * slot from a CLOCK (second-chance) sweep that never takes a slot this call uses; the missed
 * pages are copied from the host copy into their slots by a kernel reading host memory directly
 * (zero-copy).  rows (int32 [n_sel, n_seq] device memory, or NULL) receives each entry's row in
 * the slot pools (rkv_bcache_pools), -1 for padding.  The distinct pages of one call must fit
 * in n_slots: pages beyond that stay absent, their rows are -1 and the overflow counter is set.
 * Enqueued on `stream`; calls on one cache must be ordered on one stream. */
int rkv_bcache_resolve(rkv_bcache *bc, const int32_t *sel, int64_t n_sel, int n_seq, int32_t *rows,
                       void *stream);

/* Descriptors of the device slot pools ([d, n_slots*page_size, n_head_kv, 1], the host copy's
 * cell stride), to pass to rkv_attn_rows as k_pool / v_pool with the rows of a resolve call. */
int rkv_bcache_pools(const rkv_bcache *bc, rkv_tensor *k_pool, rkv_tensor *v_pool);

/* Write-through append of cell `cell`: k_cell / v_cell (device memory, n_head_kv rows of K / V
 * in the cache's type, 4-byte aligned) are written to the host copy always and to the cell's
 * slot when its page is resident, so no slot ever holds stale data. */
int rkv_bcache_append(rkv_bcache *bc, const void *k_cell, const void *v_cell, int64_t cell, void *stream);

/* Synchronous read of the counters (waits for the device). */
int rkv_bcache_counters(rkv_bcache *bc, rkv_bcache_stats *out);

/* Testing aid: device addresses of the page table (n_pages int32: slot or -1) and of the slot
 * map (n_slots int32: page or -1). */
int rkv_bcache_map(const rkv_bcache *bc, int32_t **page_table, int32_t **slot_page, int64_t *n_pages,
                   int64_t *n_slots);

/* ---- residency policy (host) ----------------------------------------------------------- */

/* Position-window sizing (patch 0070, KV-cache hunk: the position-axis residency sizer).
 * A cache of kv_size cells whose K and V take per_cell bytes per cell (all layers and
 * streams together) keeps its leading *wc cells resident in device memory; cells
 * [*wc, kv_size) form the pinned-host tail.  Budget = free device bytes (free_bytes when
 * >= 0; otherwise the context device's free memory, which needs ctx), capped at
 * target_bytes when > 0, minus reserve_bytes, never below 0.  The whole cache fits ->
 * *wc = kv_size.  Otherwise *wc = budget / per_cell rounded down to a multiple of align,
 * at least align, and at most kv_size - align rounded down to align (so a tail remains);
 * *wc never exceeds kv_size.  Host arithmetic only (no device work unless free_bytes < 0).
 * Errors: RKV_ERR_ARG for per_cell <= 0, kv_size < 0, align <= 0, reserve_bytes < 0,
 * wc NULL, or free_bytes < 0 without ctx. */
int rkv_plan_window(rkv_ctx *ctx, int64_t per_cell, int64_t kv_size, int64_t free_bytes,
                    int64_t target_bytes, int64_t reserve_bytes, int64_t align, int64_t *wc);

/* Residency mode (patch 0070, KV-cache hunk: the window-mode eligibility rule after the
 * sizer).  mode RKV_RESIDENCY_AUTO: window when eligible; RKV_RESIDENCY_RESIDENT: never;
 * RKV_RESIDENCY_WINDOW: window when eligible, otherwise resident (not an error).
 * Eligible: 0 < wc < kv_size (a real overflow), append_only != 0 (cell index = key
 * position, so the window is the position range [0, wc)) and v_transposed == 0.
 * *window receives 1 or 0.  Errors: RKV_ERR_ARG for an unknown mode or window NULL. */
int rkv_window_mode(int mode, int64_t wc, int64_t kv_size, int append_only, int v_transposed,
                    int *window);

/* ---- testing aid ------------------------------------------------------------------ */

/* Kernel families whose in-register unpacking rkv_dequant_rows reproduces. */
enum rkv_dequant_form {
    RKV_DQ_DECODE_MMA = 0,  /* matrix-core decode: q8_0 codes as binary16 1152 + q, q4_0 low
                               nibbles as 1024 + n and high nibbles in place as 1024 + 16 n    */
    RKV_DQ_PREFILL = 1,     /* prefill: q8_0 d*q as an exact two-part binary16 sum, q4_0 n - 8
                               as binary16 integers                                           */
    RKV_DQ_VECTOR = 2,      /* vector decode: q8_0 as 1152 + q, q4_0 nibble fields paired
                               across words as 1024 + n                                       */
    RKV_DQ_HEAD_DIM = 3     /* vector head-dim kernel: codes and nibbles as float32 integers  */
};

/* Dequantise n_rows rows of row_values values (type F16, Q8_0 or Q4_0; row r at byte offset
 * r*row_stride from src, device memory) into float32 dst [n_rows][row_values], rebuilding every
 * value with the same device unpack routines (rkv_unpack.h) that the kernel family `form`
 * executes: the codes or nibbles in that family's binary16 (or float32) integer form, the
 * family's offset removed and the block scale applied in float32, or for RKV_DQ_PREFILL the
 * exact two-part binary16 sum.  Every form is exact: q8_0 gives d*q and q4_0 d*(n-8) in
 * float32, binary16 subnormal scales kept -- except that RKV_DQ_PREFILL's two parts overflow
 * for q8_0 blocks with |d*q| > 65504 (|d| > 515).  row_values is a multiple of 32, at most
 * 4096.  A testing aid for the exactness of the hot kernels' dequantisation.
 * Errors: RKV_ERR_UNSUPPORTED for another type; RKV_ERR_ARG for an unknown form, a bad
 * row_values, n_rows < 0 or a row_stride shorter than a row. */
int rkv_dequant_rows(const void *src, int type, int form, int64_t n_rows, int64_t row_values,
                     int64_t row_stride, float *dst, void *stream);

/* Library version as "major.minor.patch". */
const char *rkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
