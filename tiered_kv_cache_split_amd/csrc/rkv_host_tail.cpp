// Tail partial on the host cores: the segment partial (M, S, VKQ) of every output row over
// keys that live in host memory, so that only (2 + dv) floats per row cross PCIe instead of
// the tail's K/V bytes (opencoti-llamafile patch 0070-rolling-kv: the CPU tail-partial op
// ggml_flash_attn_ext_tail_partial of the CPU_FA_TAIL tactic, whose [M, S, VKQ] rows are
// merged by the unchanged online-softmax combine; fp32 accumulation, threads over rows).
//
// Work split: a unit is (KV head g, query i, group of up to eight of the gqa query heads that
// read head g, key chunk), so each K and V row is dequantised once for all of them.  Keys are
// taken in blocks of 32: the block's scores first, then one running-max update per row and
// block, then the weighted V rows.  Units write their own partials; a final pass merges each
// row's chunks in chunk order, so the result does not depend on which thread ran which unit.
//
// The inner loops use eight-lane vector types compiled for AVX2 + FMA + F16C; the entry points
// refuse to run on a CPU without them.  Head dims: dk = dv in {64, 128, 256, 512}, or dk = 576
// with dv = 512 (the streaming op's shapes, patch 0070 fattn.cu); partial rows are 2 + dv.
#include "rkv_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace rkv {

namespace {

constexpr int kBlk = 32;  // keys per softmax block

#define RKV_HOST_SIMD __attribute__((target("avx2,fma,f16c")))

RKV_HOST_SIMD inline float h2f(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

typedef float f8 __attribute__((ext_vector_type(8)));
typedef float f8u __attribute__((ext_vector_type(8), aligned(4)));  // unaligned access
typedef int i8v __attribute__((ext_vector_type(8)));

RKV_HOST_SIMD inline f8 ld8(const float *p) { return *reinterpret_cast<const f8u *>(p); }
RKV_HOST_SIMD inline void st8(float *p, f8 v) { *reinterpret_cast<f8u *>(p) = v; }
RKV_HOST_SIMD inline float hsum8(f8 v) {
    return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

typedef signed char c8 __attribute__((ext_vector_type(8)));
typedef unsigned char u8v __attribute__((ext_vector_type(8)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

template <class V>
RKV_HOST_SIMD __attribute__((always_inline)) inline V ldv(const void *p) {
    V v;
    std::memcpy(&v, p, sizeof v);
    return v;
}

// One D-value row of K or V in fp32, eight values at a time (q8_0: d*q; q4_0: d*(n-8), byte j
// holding element j in its low nibble and element j+16 in its high nibble; binary16 as is).
template <int D>
RKV_HOST_SIMD __attribute__((always_inline)) inline void dequant_row(const uint8_t *row, int type, float *out) {
    if (type == T_F16) {
        for (int e = 0; e < D; e += 8) st8(out + e, __builtin_convertvector(ldv<h8>(row + 2 * e), f8));
    } else if (type == T_Q8_0) {
        for (int blk = 0; blk < D / 32; ++blk) {
            const uint8_t *b = row + 34 * blk;
            const float d = h2f(ldv<uint16_t>(b));
            for (int e = 0; e < 32; e += 8)
                st8(out + 32 * blk + e, __builtin_convertvector(ldv<c8>(b + 2 + e), f8) * d);
        }
    } else {  // T_Q4_0
        for (int blk = 0; blk < D / 32; ++blk) {
            const uint8_t *b = row + 18 * blk;
            const float d = h2f(ldv<uint16_t>(b));
            for (int j = 0; j < 16; j += 8) {
                const u8v x = ldv<u8v>(b + 2 + j);
                const f8 lo = __builtin_convertvector(x & (unsigned char)15, f8) - 8.0f;
                const f8 hi = __builtin_convertvector(x >> (unsigned char)4, f8) - 8.0f;
                st8(out + 32 * blk + j, lo * d);
                st8(out + 32 * blk + 16 + j, hi * d);
            }
        }
    }
}

// e^x for x <= 0 (eight lanes): x = n ln2 + y with n = round(x log2 e) and |y| <= ln2 / 2, e^y by
// its Taylor series to degree 6 (remainder below 2e-7 relative), 2^n from the exponent bits.
// Arguments below -87 give 0.
RKV_HOST_SIMD inline f8 exp8(f8 x) {
    const f8 t = x * 1.4426950408889634f;
    const f8 n = __builtin_elementwise_floor(t + 0.5f);
    const f8 y = (t - n) * 0.6931471805599453f;
    f8 p = 1.0f / 720.0f;
    p = p * y + 1.0f / 120.0f;
    p = p * y + 1.0f / 24.0f;
    p = p * y + 1.0f / 6.0f;
    p = p * y + 0.5f;
    p = p * y + 1.0f;
    p = p * y + 1.0f;
    const i8v ni = __builtin_convertvector(__builtin_elementwise_max(n, (f8)(-126.0f)), i8v);
    const f8 scale2 = __builtin_bit_cast(f8, (ni + 127) << 23);
    const f8 r = p * scale2;
    return x < -87.0f ? (f8)0.0f : r;
}

// Partial of rows (g*gqa + r0 + r, i), r < R, over keys [c0, c1): out[r][0] = M, [1] = S,
// [2 + e] = VKQ (row stride 2 + DV).  Per block of 32 keys: the visible K rows are dequantised
// once, the R scores of a key are formed together (one pass over its K row), the weights
// exponentiated eight at a time, and V accumulated with the R rows' accumulators of one
// eight-value slice in registers.
template <int R, int DK, int DV>
RKV_HOST_SIMD void run_unit(const HostTailArgs &a, int g, int r0, int i, int64_t c0, int64_t c1, float *out) {
    const int gqa = a.n_head / a.n_head_kv;
    alignas(32) float qv[R][DK];
    alignas(32) float acc[R][DV];
    alignas(32) float kt[kBlk][DK];
    alignas(32) float vt[kBlk][DV];
    alignas(32) float sc[R][kBlk];
    float m[R], l[R];
    for (int r = 0; r < R; ++r) {
        const uint16_t *q = a.q + (int64_t)i * a.q_s1 + (int64_t)(g * gqa + r0 + r) * a.q_s2;
        for (int e = 0; e < DK; ++e) qv[r][e] = a.scale * h2f(q[e]);
        for (int e = 0; e < DV; ++e) acc[r][e] = 0.f;
        m[r] = -INFINITY;
        l[r] = 0.f;
    }
    const uint8_t *kb = a.k + (int64_t)g * a.k_s2, *vb = a.v + (int64_t)g * a.v_s2;
    const uint16_t *mrow = a.mask ? a.mask + (int64_t)i * a.m_s1 : nullptr;
    const bool cap = a.softcap > 0.f;
    bool vis[kBlk];
    float mv[kBlk];
    for (int64_t j0 = c0; j0 < c1; j0 += kBlk) {
        const int nb = (int)std::min<int64_t>(kBlk, c1 - j0);
        bool any = false;
        for (int jj = 0; jj < kBlk; ++jj) {
            const int64_t j = j0 + jj;
            bool v = jj < nb && (a.q_pos0 < 0 || a.kv_pos0 + j <= a.q_pos0 + i);
            float x = 0.f;
            if (v && mrow) {
                x = h2f(mrow[j]);
                v = x > -INFINITY;
            }
            vis[jj] = v;
            mv[jj] = x;
            any = any || v;
        }
        if (!any) continue;
        for (int jj = 0; jj < nb; ++jj)
            if (vis[jj]) dequant_row<DK>(kb + (j0 + jj) * a.k_s1, a.k_type, kt[jj]);
        // scores: one pass over each K row for all R rows
        for (int jj = 0; jj < kBlk; ++jj) {
            if (!vis[jj]) {
                for (int r = 0; r < R; ++r) sc[r][jj] = -INFINITY;
                continue;
            }
            f8 s8[R];
            for (int r = 0; r < R; ++r) s8[r] = 0.f;
            for (int e = 0; e < DK; e += 8) {
                const f8 kv = ld8(&kt[jj][e]);
                for (int r = 0; r < R; ++r) s8[r] = __builtin_elementwise_fma(ld8(&qv[r][e]), kv, s8[r]);
            }
            for (int r = 0; r < R; ++r) {
                float s = hsum8(s8[r]);
                if (cap) s = a.softcap * std::tanh(s / a.softcap);
                sc[r][jj] = s + mv[jj];
            }
        }
        // running max per row and the block's weights
        for (int r = 0; r < R; ++r) {
            float bm = -INFINITY;
            for (int jj = 0; jj < kBlk; ++jj) bm = std::max(bm, sc[r][jj]);
            if (bm == -INFINITY) {
                for (int jj = 0; jj < kBlk; ++jj) sc[r][jj] = 0.f;
                continue;
            }
            if (bm > m[r]) {
                const float alpha = m[r] == -INFINITY ? 0.f : std::exp(m[r] - bm);
                l[r] *= alpha;
                for (int e = 0; e < DV; e += 8) st8(&acc[r][e], ld8(&acc[r][e]) * alpha);
                m[r] = bm;
            }
            f8 lsum = 0.f;
            for (int jj = 0; jj < kBlk; jj += 8) {
                const f8 x = ld8(&sc[r][jj]);
                const f8 p = x == -INFINITY ? (f8)0.f : exp8(x - m[r]);
                st8(&sc[r][jj], p);
                lsum += p;
            }
            l[r] += hsum8(lsum);
        }
        for (int jj = 0; jj < nb; ++jj)
            if (vis[jj]) dequant_row<DV>(vb + (j0 + jj) * a.v_s1, a.v_type, vt[jj]);
        // VKQ: the R accumulators of one 8-value slice stay in registers over the block's keys
        for (int e = 0; e < DV; e += 8) {
            f8 ac[R];
            for (int r = 0; r < R; ++r) ac[r] = ld8(&acc[r][e]);
            for (int jj = 0; jj < nb; ++jj) {
                if (!vis[jj]) continue;
                const f8 vv = ld8(&vt[jj][e]);
                for (int r = 0; r < R; ++r) ac[r] = __builtin_elementwise_fma((f8)sc[r][jj], vv, ac[r]);
            }
            for (int r = 0; r < R; ++r) st8(&acc[r][e], ac[r]);
        }
    }
    for (int r = 0; r < R; ++r) {
        float *o = out + (size_t)r * (2 + DV);
        o[0] = m[r];
        o[1] = l[r];
        std::memcpy(o + 2, acc[r], DV * sizeof(float));
    }
}

// Rows of a unit: the gqa query heads of a KV head, taken eight at a time.
constexpr int kMaxR = 8;

template <int DK, int DV>
void run_rows_d(const HostTailArgs &a, int g, int r0, int R, int i, int64_t c0, int64_t c1, float *out) {
    switch (R) {
        case 1: run_unit<1, DK, DV>(a, g, r0, i, c0, c1, out); break;
        case 2: run_unit<2, DK, DV>(a, g, r0, i, c0, c1, out); break;
        case 3: run_unit<3, DK, DV>(a, g, r0, i, c0, c1, out); break;
        case 4: run_unit<4, DK, DV>(a, g, r0, i, c0, c1, out); break;
        case 5: run_unit<5, DK, DV>(a, g, r0, i, c0, c1, out); break;
        case 6: run_unit<6, DK, DV>(a, g, r0, i, c0, c1, out); break;
        case 7: run_unit<7, DK, DV>(a, g, r0, i, c0, c1, out); break;
        default: run_unit<8, DK, DV>(a, g, r0, i, c0, c1, out); break;
    }
}

void run_rows(const HostTailArgs &a, int g, int r0, int R, int i, int64_t c0, int64_t c1, float *out) {
    if (a.d == 64) run_rows_d<64, 64>(a, g, r0, R, i, c0, c1, out);
    else if (a.d == 256) run_rows_d<256, 256>(a, g, r0, R, i, c0, c1, out);
    else if (a.d == 512) run_rows_d<512, 512>(a, g, r0, R, i, c0, c1, out);
    else if (a.d == 576) run_rows_d<576, 512>(a, g, r0, R, i, c0, c1, out);
    else run_rows_d<kHeadDim, kHeadDim>(a, g, r0, R, i, c0, c1, out);
}

}  // namespace

bool host_tail_supported() {
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") && __builtin_cpu_supports("f16c");
}

int host_tail_threads(int requested) {
    if (requested > 0) return requested;
    const unsigned hc = std::thread::hardware_concurrency();
    return hc ? (int)std::min(hc, 16u) : 1;  // one GPU's share of a multi-GPU host
}

void host_tail_partial(const HostTailArgs &a, int n_threads) {
    const int gqa = a.n_head / a.n_head_kv;
    const int n_rg = (gqa + kMaxR - 1) / kMaxR;  // row groups per (g, i)
    const int threads = host_tail_threads(n_threads);
    // chunks per (g, i, row group): enough units to keep every thread busy, >= 1024 keys each
    const int64_t groups = (int64_t)a.n_head_kv * a.n_q * n_rg;
    int64_t n_chunks = std::max<int64_t>(1, (4 * threads + groups - 1) / groups);
    n_chunks = std::max<int64_t>(1, std::min<int64_t>(n_chunks, (a.n_cells + 1023) / 1024));
    const int64_t chunk = a.n_cells > 0 ? (a.n_cells + n_chunks - 1) / n_chunks : 0;
    const int64_t n_units = groups * n_chunks;
    const int ps = 2 + a.dv;  // partial row stride
    std::vector<float> parts((size_t)n_units * kMaxR * ps);
    auto rows_of = [&](int rg) { return std::min(kMaxR, gqa - rg * kMaxR); };
    std::atomic<int64_t> next{0};
    auto worker = [&]() {
        for (int64_t u = next.fetch_add(1); u < n_units; u = next.fetch_add(1)) {
            const int64_t c = u % n_chunks;
            int64_t t = u / n_chunks;
            const int rg = (int)(t % n_rg);
            t /= n_rg;
            const int g = (int)(t % a.n_head_kv), i = (int)(t / a.n_head_kv);
            const int64_t c0 = std::min(a.n_cells, c * chunk), c1 = std::min(a.n_cells, c0 + chunk);
            run_rows(a, g, rg * kMaxR, rows_of(rg), i, c0, c1, &parts[(size_t)u * kMaxR * ps]);
        }
    };
    const int nt = (int)std::min<int64_t>(threads, n_units);
    std::vector<std::thread> pool;
    pool.reserve(nt);
    try {
        for (int t = 1; t < nt; ++t) pool.emplace_back(worker);
    } catch (...) {
        // no more threads available: the ones started and this one take every unit
    }
    worker();
    for (auto &th : pool) th.join();
    // merge each row's chunks in chunk order
    for (int64_t gr = 0; gr < groups; ++gr) {
        const int rg = (int)(gr % n_rg);
        const int g = (int)((gr / n_rg) % a.n_head_kv), i = (int)(gr / n_rg / a.n_head_kv);
        for (int r = 0; r < rows_of(rg); ++r) {
            auto part = [&](int64_t c) { return &parts[((size_t)(gr * n_chunks + c) * kMaxR + r) * ps]; };
            float M = -INFINITY;
            for (int64_t c = 0; c < n_chunks; ++c) M = std::max(M, part(c)[0]);
            float *o = a.partial + (size_t)((g * gqa + rg * kMaxR + r) + (int64_t)a.n_head * i) * ps;
            float S = 0.f;
            float V[512] = {};
            if (M > -INFINITY) {
                for (int64_t c = 0; c < n_chunks; ++c) {
                    const float *pc = part(c);
                    if (pc[0] == -INFINITY) continue;
                    const float w = std::exp(pc[0] - M);
                    S += pc[1] * w;
                    for (int e = 0; e < a.dv; ++e) V[e] += pc[2 + e] * w;
                }
            }
            o[0] = M;
            o[1] = S;
            std::memcpy(o + 2, V, (size_t)a.dv * sizeof(float));
        }
    }
}

}  // namespace rkv
