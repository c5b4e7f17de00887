// Device-side block cache over a host-resident KV copy (Strata compare v0.1.2...v0.1.6, "KV
// streaming for the QSA layers": kv_stream.hpp header comment and kv_stream.cu).
//
// The authoritative K/V stay in pinned host memory, cell-major.  Device memory holds n_slots
// pages of page_size cells (all KV heads of a cell, K and V in two pools laid out like the host
// copy), and a residency map: page_table[page] = slot or -1, slot_page[slot] = page or -1,
// slot_stamp (the call that last used the slot), slot_ref (clock reference bit) and ctl
// (epoch, hand, pages placed by the last call, overflow flag, 64-bit counters of misses,
// lookups and calls).  One resolve call makes every page a selection of cells names resident:
//   1. lookups: a resident page takes this call's epoch and its reference bit; a missing page
//      is claimed exactly once (compare-and-swap -1 -> -2) into the miss list;
//   2. a CLOCK sweep (second chance) from the hand takes one victim slot per miss: never a slot
//      this call uses; a free or unreferenced slot is taken; a referenced one passed by the
//      hand loses its bit.  The slots are swept in batches of at most min(1024, n_slots), each
//      slot once per batch; a candidate's rank inside a batch comes from a 64-bit ballot and
//      mbcnt within its wave plus the candidate counts of the waves before it;
//   3. the table is re-pointed (the victim's old page becomes absent).
// A copy kernel then reads the missed pages straight from host memory (zero-copy, 16 bytes per
// lane) into their slots, and a translate kernel turns the selection's cells into slot-pool
// rows for the row-list attention kernel.  Appends write the host copy always and the slot only
// when the page is resident, so slots never hold stale data.
#include "rkv_internal.h"

namespace rkv {

namespace {

constexpr int kBcThreads = 1024;
constexpr int kBcWaves = kBcThreads / 64;

__global__ void __launch_bounds__(256) bc_reset_kernel(BcMap m) {
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, st = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = i0; i < m.n_pages; i += st) m.page_table[i] = -1;
    for (int64_t i = i0; i < m.n_slots; i += st) {
        m.slot_page[i] = -1;
        m.slot_stamp[i] = -1;
        m.slot_ref[i] = 0;
    }
    if (i0 < kBcCtl) m.ctl[i0] = 0;
}

__global__ void __launch_bounds__(kBcThreads) bc_resolve_kernel(BcMap m, const int32_t *__restrict__ sel, int64_t n_sel,
                                                                 int n_seq) {
    __shared__ int s_nmiss, s_lookups, s_cut, s_unplaced;
    __shared__ int s_wsum[kBcWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ps = m.page_size;
    const int n = (int)m.n_slots;
    const int epoch = m.ctl[0] + 1;
    if (tid == 0) {
        s_nmiss = 0;
        s_lookups = 0;
        s_unplaced = 0;
    }
    __syncthreads();

    // 1. lookups and miss claims
    int lookups = 0;
    for (int b = 0; b < n_seq; ++b) {
        const int32_t *sq = sel + (int64_t)b * n_sel;
        for (int64_t i = tid; i < n_sel; i += kBcThreads) {
            const int32_t c = sq[i];
            if (c < 0) continue;
            const int64_t pg = c / ps;
            if (i > 0) {
                const int32_t cp = sq[i - 1];
                if (cp >= 0 && cp / ps == pg) continue;  // one lookup per run of equal pages
            }
            ++lookups;
            if (pg >= m.n_pages) continue;  // outside the cache: the translate kernel gives -1
            const int32_t sl = __hip_atomic_load(&m.page_table[pg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (sl >= 0) {
                m.slot_stamp[sl] = epoch;
                m.slot_ref[sl] = 1;
            } else if (sl == -1 && atomicCAS(&m.page_table[pg], -1, -2) == -1) {
                const int k = atomicAdd(&s_nmiss, 1);
                if (k < n) {
                    m.miss_page[k] = (int32_t)pg;
                } else {
                    m.page_table[pg] = -1;  // more misses than slots: this page stays absent
                    atomicAdd(&s_unplaced, 1);
                }
            }
        }
    }
    atomicAdd(&s_lookups, lookups);
    __syncthreads();

    // 2. one victim per recorded miss: CLOCK sweep from the hand, batch by batch
    const int recorded = min(s_nmiss, n);
    int hand = m.ctl[1], got = 0, scanned = 0;
    const int bmax = min(kBcThreads, n);
    while (got < recorded && scanned < 3 * n) {
        const int width = min(bmax, 3 * n - scanned);
        const int j = tid < width ? (int)(((int64_t)hand + tid) % n) : -1;
        const bool mine = j >= 0 && m.slot_stamp[j] == epoch;
        const bool cand = j >= 0 && !mine && (m.slot_page[j] < 0 || m.slot_ref[j] == 0);
        const uint64_t bal = __ballot(cand);
        const int rank_w =
            (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (lane == 0) s_wsum[wave] = __popcll(bal);
        if (tid == 0) s_cut = width;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kBcWaves; ++w) {
            const int x = s_wsum[w];
            before += w < wave ? x : 0;
            total += x;
        }
        const int rank = before + rank_w;
        const int want = recorded - got;
        if (cand && rank == want - 1) s_cut = tid + 1;  // the hand stops just past the last slot taken
        __syncthreads();
        const int cut = s_cut;
        if (cand && rank < want) {
            m.miss_slot[got + rank] = j;
            m.slot_stamp[j] = epoch;  // taken: a later batch that wraps around skips it
        } else if (j >= 0 && tid < cut && !mine) {
            m.slot_ref[j] = 0;        // second chance used up
        }
        got += min(total, want);
        hand = (int)(((int64_t)hand + cut) % n);
        scanned += cut;
        __syncthreads();
    }

    // 3. re-point the table
    const int placed = got;
    for (int k = tid; k < recorded; k += kBcThreads) {
        const int32_t pg = m.miss_page[k];
        if (k >= placed) {
            m.page_table[pg] = -1;
            continue;
        }
        const int32_t sl = m.miss_slot[k];
        const int32_t old = m.slot_page[sl];
        if (old >= 0) m.page_table[old] = -1;
        m.slot_page[sl] = pg;
        m.slot_stamp[sl] = epoch;
        m.slot_ref[sl] = 1;
        m.page_table[pg] = sl;
    }
    if (tid == 0) {
        m.ctl[0] = epoch;
        m.ctl[1] = hand;
        m.ctl[2] = placed;
        if (placed < recorded || s_unplaced > 0) m.ctl[3] = 1;
        unsigned long long *c = reinterpret_cast<unsigned long long *>(m.ctl + 4);
        c[0] += (unsigned long long)placed;
        c[1] += (unsigned long long)s_lookups;
        c[2] += 1ull;
    }
}

// One workgroup per placed page (grid-stride): the page's K and V spans from the host copy's
// device view into its slot, 16 bytes per lane.
__global__ void __launch_bounds__(256) bc_copy_kernel(BcMap m, const uint4 *__restrict__ hk, const uint4 *__restrict__ hv,
                                                      uint4 *__restrict__ pk, uint4 *__restrict__ pv, int64_t k16, int64_t v16) {
    const int placed = m.ctl[2];
    for (int k = blockIdx.x; k < placed; k += gridDim.x) {
        const int64_t pg = m.miss_page[k], sl = m.miss_slot[k];
        for (int64_t i = threadIdx.x; i < k16; i += blockDim.x) pk[sl * k16 + i] = hk[pg * k16 + i];
        for (int64_t i = threadIdx.x; i < v16; i += blockDim.x) pv[sl * v16 + i] = hv[pg * v16 + i];
    }
}

__global__ void __launch_bounds__(256) bc_rows_kernel(BcMap m, const int32_t *__restrict__ sel, int64_t n,
                                                      int32_t *__restrict__ rows) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int32_t c = sel[i];
    int32_t r = -1;
    if (c >= 0 && c / m.page_size < m.n_pages) {
        const int32_t sl = m.page_table[c / m.page_size];
        if (sl >= 0) r = sl * m.page_size + c % m.page_size;
    }
    rows[i] = r;
}

// Write-through append of one cell: the host copy always, the slot when the page is resident.
__global__ void __launch_bounds__(256) bc_append_kernel(BcMap m, const uint32_t *__restrict__ kc,
                                                        const uint32_t *__restrict__ vc, int64_t kw, int64_t vw,
                                                        int64_t cell, uint8_t *hk, uint8_t *hv, uint8_t *pk,
                                                        uint8_t *pv, int64_t k_s1, int64_t v_s1) {
    const int32_t sl = m.page_table[cell / m.page_size];
    const int64_t row = sl >= 0 ? (int64_t)sl * m.page_size + cell % m.page_size : -1;
    uint32_t *hkr = reinterpret_cast<uint32_t *>(hk + cell * k_s1);
    uint32_t *hvr = reinterpret_cast<uint32_t *>(hv + cell * v_s1);
    for (int64_t i = threadIdx.x; i < kw; i += blockDim.x) {
        const uint32_t x = kc[i];
        hkr[i] = x;
        if (row >= 0) reinterpret_cast<uint32_t *>(pk + row * k_s1)[i] = x;
    }
    for (int64_t i = threadIdx.x; i < vw; i += blockDim.x) {
        const uint32_t x = vc[i];
        hvr[i] = x;
        if (row >= 0) reinterpret_cast<uint32_t *>(pv + row * v_s1)[i] = x;
    }
}

}  // namespace

hipError_t launch_bc_reset(const BcMap &m, hipStream_t s) {
    hipLaunchKernelGGL(bc_reset_kernel, dim3(128), dim3(256), 0, s, m);
    return hipGetLastError();
}

hipError_t launch_bc_resolve(const BcMap &m, const int32_t *sel, int64_t n_sel, int n_seq, const uint8_t *host_k,
                             const uint8_t *host_v, uint8_t *pool_k, uint8_t *pool_v, int64_t k_page_bytes,
                             int64_t v_page_bytes, int32_t *rows, hipStream_t s) {
    hipLaunchKernelGGL(bc_resolve_kernel, dim3(1), dim3(kBcThreads), 0, s, m, sel, n_sel, n_seq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bc_copy_kernel, dim3(128), dim3(256), 0, s, m, reinterpret_cast<const uint4 *>(host_k),
                       reinterpret_cast<const uint4 *>(host_v), reinterpret_cast<uint4 *>(pool_k),
                       reinterpret_cast<uint4 *>(pool_v), k_page_bytes / 16, v_page_bytes / 16);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = n_sel * n_seq;
    if (rows && n > 0)
        hipLaunchKernelGGL(bc_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, m, sel, n, rows);
    return hipGetLastError();
}

hipError_t launch_bc_append(const BcMap &m, const void *k_cell, const void *v_cell, int64_t k_cell_bytes,
                            int64_t v_cell_bytes, int64_t cell, uint8_t *host_k, uint8_t *host_v, uint8_t *pool_k,
                            uint8_t *pool_v, int64_t k_s1, int64_t v_s1, hipStream_t s) {
    hipLaunchKernelGGL(bc_append_kernel, dim3(1), dim3(256), 0, s, m, static_cast<const uint32_t *>(k_cell),
                       static_cast<const uint32_t *>(v_cell), k_cell_bytes / 4, v_cell_bytes / 4, cell, host_k, host_v,
                       pool_k, pool_v, k_s1, v_s1);
    return hipGetLastError();
}

}  // namespace rkv
