// gfx950 (CDNA4) kernels for paged decode attention in a persistent
// work-queue kernel.
//
// What is computed follows the PersistentKV page ("PersistentKV: Page-Aware
// Decode Scheduling for Long-Context LLM Serving on Commodity GPUs",
// Technical Summary, Methodology 1): G query heads share one KV head; K/V are
// read in place through the block table; only tokens below the row's length
// are used; a split range yields a partial online-softmax state that a
// separate merge kernel combines exactly.  The persistent grid pops items
// from the device queue with one atomic per item, as the persistent executor
// on the GPUOS page claims tasks ("GPUOS: A GPU Operating System Primitive
// for Transparent Operation Fusion", section 4.1 "Persistent Kernel
// Executor").
//
// Mapping onto CDNA4.  Decode attention reads 512 bytes of K+V per token and
// KV head for 4*G*D flops (G = 4, D = 128: 4 flop/byte), far below the chip's
// ALU balance, so the kernel is bound by HBM bandwidth and is written as a
// streaming gather, not as matrix-core tiles:
//   * a workgroup is 8 wave64s; it owns one item at a time and its waves take
//     the item's pages round-robin, each wave keeping its own softmax state;
//   * a (page, KV head) slab of K is 16 rows x D bf16 (4 KB at D = 128); a
//     wave reads it with D/32 dwordx4 loads, 8 lanes per token row, each load
//     instruction covering whole 128-byte lines (same for V);
//   * q.K uses v_dot2c_f32_bf16 on the packed bf16 pairs straight from the
//     loads (fp32 accumulate); the 8 lanes of a row reduce with three DPP
//     adds (quad_perm x2, row_half_mirror), no LDS traffic;
//   * each 8-lane group runs its own online softmax over its tokens, with a
//     lazy rescale: the running max is raised only when a score exceeds it by
//     more than 2^8, so the accumulator rescale is rare; results are exact up
//     to rounding because the final normalisation divides by the same sum;
//   * P.V for a bf16 cache is v_dot2 over the lane's two token rows (each
//     dim's two V values and each head's two weights as bf16 pairs, fp32
//     accumulate);
//   * pages are software-pipelined two ahead in registers (three tiles), so
//     each wave keeps up to 16 KB of K/V loads in flight;
//   * at the end of an item the 8 groups of a wave combine by DPP and
//     row-swap permutes and the 8 waves combine through LDS.
// An fp32 cache runs the same kernels on half-page tiles (8 rows of 512 B at
// D = 128), with fp32 FMAs in place of the bf16 dot products and fp32
// weights in P.V.
#include <float.h>
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kTau = 8.0f;               // lazy-rescale threshold, log2 units
constexpr float kNegBig = -FLT_MAX;        // finite "minus infinity" for running maxima
constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 8 consecutive lanes of a half-row.
__device__ __forceinline__ float sum8(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);   // row_half_mirror
    return v;
}

// Reductions over lane bits 3..5 (the eight 8-lane groups of a wave) without
// going through LDS: bit 3 by a DPP rotate of each 16-lane row by 8, bits 4
// and 5 by gfx950's row-swap permutes, which exchange 16-lane rows (bit 4)
// and 32-lane halves (bit 5) between two registers.  Every lane ends with the
// same value, combined in the same order.
__device__ __forceinline__ float swap16_sum(float v) {
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float swap32_sum(float v) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float swap16_max(float v) {
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float swap32_max(float v) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float groups_sum(float v) {
    v += dpp_f<0x128>(v);   // row_ror:8 (lane bit 3)
    return swap32_sum(swap16_sum(v));
}
__device__ __forceinline__ float groups_max(float v) {
    v = fmaxf(v, dpp_f<0x128>(v));
    return swap32_max(swap16_max(v));
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;      // NaN stays NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void report(const Ctrl* c0, uint32_t* host_error, uint32_t code,
                                       uint32_t detail) {
    Ctrl* c = const_cast<Ctrl*>(c0);
    if (atomicCAS(&c->error_code, 0u, code) == 0u) atomicExch(&c->error_detail, detail);
    if (host_error) __hip_atomic_store(host_error, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Element type of the K/V cache.  A tile is the part of one page that a wave
// loads and consumes at a time: the whole page for bf16 (two token rows per
// lane, 8*j + r for j = 0, 1), half a page for fp32 (one token row per lane,
// row 8*h + r of half h); either way 8 KB per wave at D = 128, so both
// element types keep the same registers per tile and the same pipeline.
//
// Lane p of a row's 8 lanes holds 16-byte word w of the row at byte
// 128 w + 16 p, so each load instruction of the 8 lanes covers one whole
// 128-byte line.  Word w holds dims dim(p, w, 0 ..): bf16, 8 dims from
// 64 w + 8 p; fp32, 4 dims from 32 w + 4 p.
struct KvBf16 {
    static constexpr int kBytes = 2;
    static constexpr int kRows = 2;            // token rows per lane in a tile
    static constexpr int kTilesPerPage = 1;
    static constexpr int kDimsPerWord = 8;
};
struct KvF32 {
    static constexpr int kBytes = 4;
    static constexpr int kRows = 1;
    static constexpr int kTilesPerPage = 2;
    static constexpr int kDimsPerWord = 4;
};

// Dim held by lane p in element i of its word w.
template <typename KV>
__device__ __forceinline__ int word_dim(int p, int w, int i) {
    return KV::kDimsPerWord * (8 * w + p) + i;
}

// Per-lane share of one tile of K and V: kRows token rows times NW 16-byte
// words of the row (D / 64 words for bf16, D / 32 for fp32).
template <int D, typename KV>
struct Tile {
    static constexpr int NW = D * KV::kBytes / 128;
    u32x4 k[KV::kRows][NW];
    u32x4 v[KV::kRows][NW];
};

// Byte offsets of the lane's token rows inside a tile (the tile's first row
// is the slab address the loads get).  Rows at or beyond `valid` (counted
// from the tile's first row) are never read: their lanes re-read row 0 of the
// tile (always a valid token) and the consumer masks them.
struct LaneOff {
    uint32_t o0, o1;
};

template <int D, typename KV>
__device__ __forceinline__ LaneOff lane_offsets(int r, int p, int valid) {
    constexpr int RB = D * KV::kBytes;                        // bytes per token row
    const int t0 = r < valid ? r : 0;
    const int t1 = 8 + r < valid ? 8 + r : 0;
    return {(uint32_t)(t0 * RB + p * 16), (uint32_t)(t1 * RB + p * 16)};
}

// Streaming 16-byte load with the non-temporal hint: K/V pages are read
// once per call, so they should not displace anything in L2 or the
// last-level cache (measured on MI355X: random 4 KB K+V slabs stream at
// about 6.7 TB/s with the hint against about 6.0 TB/s without).
__device__ __forceinline__ u32x4 ld_stream(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// The gather of one tile: ks / vs are the wave-uniform addresses of the
// tile's first row, the lane adds its 32-bit row offset; word w sits 128 w
// bytes further on.
template <int D, typename KV>
__device__ __forceinline__ void load_tile(Tile<D, KV>& t, const char* ks, const char* vs, LaneOff o) {
#pragma unroll
    for (int w = 0; w < Tile<D, KV>::NW; ++w) {
        const uint32_t off = 128 * w;
        t.k[0][w] = ld_stream(ks + o.o0 + off);
        if constexpr (KV::kRows == 2) t.k[1][w] = ld_stream(ks + o.o1 + off);
        t.v[0][w] = ld_stream(vs + o.o0 + off);
        if constexpr (KV::kRows == 2) t.v[1][w] = ld_stream(vs + o.o1 + off);
    }
}

template <int D, int G>
struct State {
    float m[G];
    float l[G];
    float acc[G][D / 8];
};

// q.K, online-softmax update and P.V for one tile.  q stays packed bf16 in
// registers; for a bf16 cache K pairs meet it in v_dot2 (fp32 accumulate) and
// P.V runs as v_dot2 over the lane's two token rows with the weights rounded
// to bf16; for an fp32 cache each q pair is widened to fp32 on the fly
// (exact), multiplied with full-precision K, and P.V is fp32 FMA with fp32
// weights.  The accumulator and the softmax sum are fp32 either way.
template <int D, int G, typename KV, bool MASKED>
__device__ __forceinline__ void consume_tile(const Tile<D, KV>& t, const u32x4 (&qv)[G][D / 64],
                                             State<D, G>& st, float c, int r, int valid) {
    constexpr int NPC = D / 64;
    constexpr int R = KV::kRows;
    constexpr int NW = Tile<D, KV>::NW;          // 16-byte words per row and lane
    float s[R][G];
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float a = 0.0f;
#pragma unroll
            for (int k = 0; k < NPC; ++k) {
                if constexpr (KV::kBytes == 2) {
                    a = dot2(t.k[j][k].x, qv[g][k].x, a);
                    a = dot2(t.k[j][k].y, qv[g][k].y, a);
                    a = dot2(t.k[j][k].z, qv[g][k].z, a);
                    a = dot2(t.k[j][k].w, qv[g][k].w, a);
                } else {
                    const u32x4 k0 = t.k[j][2 * k], k1 = t.k[j][2 * k + 1];
                    u32x4 q = qv[g][k];
                    // widen q here, tile by tile: hoisted out of the loop the
                    // widened copy would need D * G / 8 more VGPRs per lane
                    __asm__ volatile("" : "+v"(q));
                    a = fmaf(__uint_as_float(k0.x), bf16_lo(q.x), a);
                    a = fmaf(__uint_as_float(k0.y), bf16_hi(q.x), a);
                    a = fmaf(__uint_as_float(k0.z), bf16_lo(q.y), a);
                    a = fmaf(__uint_as_float(k0.w), bf16_hi(q.y), a);
                    a = fmaf(__uint_as_float(k1.x), bf16_lo(q.z), a);
                    a = fmaf(__uint_as_float(k1.y), bf16_hi(q.z), a);
                    a = fmaf(__uint_as_float(k1.z), bf16_lo(q.w), a);
                    a = fmaf(__uint_as_float(k1.w), bf16_hi(q.w), a);
                }
            }
            s[j][g] = sum8(a) * c;
        }
    }
    u32x4 v[R][NW];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int k = 0; k < NW; ++k) v[j][k] = t.v[j][k];
    if (MASKED) {                                 // the last, partial page of a row
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const bool ok = 8 * j + r < valid;
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (!ok) s[j][g] = -INFINITY;
#pragma unroll
            for (int k = 0; k < NW; ++k)
                if (!ok) v[j][k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float mx[G];
    bool need = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mx[g] = s[0][g];
#pragma unroll
        for (int j = 1; j < R; ++j) mx[g] = fmaxf(mx[g], s[j][g]);
        need |= mx[g] > st.m[g] + kTau;
    }
    if (need) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mn = fmaxf(st.m[g], mx[g]);
            const float a = __builtin_amdgcn_exp2f(st.m[g] - mn);
            st.l[g] *= a;
#pragma unroll
            for (int e = 0; e < D / 8; ++e) st.acc[g][e] *= a;
            st.m[g] = mn;
        }
    }
    // bf16 cache: the lane's two token rows (8 apart) hold the same dims, so
    // P.V runs as v_dot2 over the row pair: each dim's two V values form one
    // bf16 pair (a byte permute, shared by all heads) and each head's two
    // weights another (rounded to nearest even, one conversion), accumulated
    // in fp32.  The softmax sum l keeps the unrounded fp32 weights.
    uint32_t vp[NPC][4][2];
    if constexpr (KV::kBytes == 2) {
#pragma unroll
        for (int k = 0; k < NPC; ++k) {
            const uint32_t a0[4] = {v[0][k].x, v[0][k].y, v[0][k].z, v[0][k].w};
            const uint32_t a1[4] = {v[1][k].x, v[1][k].y, v[1][k].z, v[1][k].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                vp[k][w][0] = __builtin_amdgcn_perm(a1[w], a0[w], 0x05040100u);   // low dims of both rows
                vp[k][w][1] = __builtin_amdgcn_perm(a1[w], a0[w], 0x07060302u);   // high dims of both rows
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if constexpr (KV::kBytes == 2) {
            const float p0 = __builtin_amdgcn_exp2f(s[0][g] - st.m[g]);
            const float p1 = __builtin_amdgcn_exp2f(s[1][g] - st.m[g]);
            st.l[g] += p0 + p1;
            const uint32_t pp = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_t));
#pragma unroll
            for (int k = 0; k < NPC; ++k)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float& lo = st.acc[g][k * 8 + 2 * w];
                    float& hi = st.acc[g][k * 8 + 2 * w + 1];
                    lo = dot2(vp[k][w][0], pp, lo);
                    hi = dot2(vp[k][w][1], pp, hi);
                }
        } else {
            const float p0 = __builtin_amdgcn_exp2f(s[0][g] - st.m[g]);
            st.l[g] += p0;
#pragma unroll
            for (int k = 0; k < NW; ++k) {
                const float x[4] = {__uint_as_float(v[0][k].x), __uint_as_float(v[0][k].y),
                                    __uint_as_float(v[0][k].z), __uint_as_float(v[0][k].w)};
#pragma unroll
                for (int e = 0; e < 4; ++e) st.acc[g][4 * k + e] = fmaf(p0, x[e], st.acc[g][4 * k + e]);
            }
        }
    }
}

// Pages kept in flight ahead of the one being consumed: two when the
// accumulator leaves room for three tiles in 256 VGPRs, else one.
template <int D, int G>
struct PipelineDepth {
    static constexpr int value = (G * D / 8 <= 64) ? 2 : 1;
};

// Wave-uniform description of one item as seen by one wave.
struct WaveItem {
    uint32_t tb, te;       // token range of the item
    int w;                 // wave index in the workgroup
    int hk;                // KV head
};

// One window of up to 64 of this wave's pages: i = wb .. wb + n - 1 of the
// wave's page list (item page w + 8 i), walked tile by tile (a tile is a
// page, or half of one for an fp32 cache).  Loads run ahead of the tile being
// consumed; past the end the look-ahead reads a small workspace region that
// every wave shares (it stays in L2, and its values are never used), so
// that every iteration issues the same loads and the wait counts the
// compiler derives stay exact.  btv holds the window's validated page ids.
template <int D, int G, typename KV>
__device__ __forceinline__ void run_window(const DecodeParams& P, const u32x4 (&qv)[G][D / 64],
                                           State<D, G>& st, int32_t btv, int n, int wb,
                                           const WaveItem& wi, int r, int p) {
    constexpr int TPP = KV::kTilesPerPage;
    constexpr int kTileRows = kPageSize / TPP;
    constexpr uint64_t kSlabBytes = (uint64_t)kPageSize * D * KV::kBytes;
    constexpr uint64_t kTileBytes = kSlabBytes / TPP;
    const char* kbase = reinterpret_cast<const char*>(P.k_pool);
    const char* vbase = reinterpret_cast<const char*>(P.v_pool);
    const uint64_t head_off = (uint64_t)wi.hk * kSlabBytes;
    const uint64_t page_stride = (uint64_t)P.hkv * kSlabBytes;
    // page ii of the window: slab byte offset and number of valid rows (both uniform)
    auto page_of = [&](int ii, int& valid) -> uint64_t {
        const int32_t pg = __builtin_amdgcn_readlane(btv, ii);
        const uint32_t tok0 = wi.tb + (uint32_t)(wi.w + kWaves * (wb + ii)) * kPageSize;
        const uint32_t rem = wi.te - tok0;
        valid = rem < (uint32_t)kPageSize ? (int)rem : kPageSize;
        return (uint64_t)(uint32_t)pg * page_stride + head_off;
    };
    const float c = P.scale_log2;
    // Only the item's last page can be partial; keep it out of the pipelined
    // loop so that the loop issues full-tile loads with loop-invariant lane
    // offsets (no per-tile VGPR temporaries competing with in-flight tiles).
    int vlast;
    const uint64_t slast = page_of(n - 1, vlast);
    const int nf = vlast < kPageSize ? n - 1 : n;               // full pages in the window
    const int nt = nf * TPP;                                    // their tiles
    const LaneOff full = lane_offsets<D, KV>(r, p, kTileRows);
    static_assert(kTileBytes <= (uint64_t)kSinkBytes, "the look-ahead sink must hold a tile");
    auto issue = [&](Tile<D, KV>& T, int ii) {
        int unused;
        const char* ks = P.sink;
        const char* vs = P.sink;
        if (ii < nt) {
            const uint64_t so = page_of(ii / TPP, unused) + (uint64_t)(ii % TPP) * kTileBytes;
            ks = kbase + so;
            vs = vbase + so;
        }
        LaneOff o = full;
        // Keep the lane offset a 32-bit VGPR inside the loop so the loads use
        // the scalar-base + 32-bit-offset form (no 64-bit per-lane address math).
        __asm__ volatile("" : "+v"(o.o0), "+v"(o.o1));
        load_tile<D, KV>(T, ks, vs, o);
    };
    // The loop is rotated so that every iteration first consumes a tile and
    // then refills the registers it just freed: no instruction at the loop
    // head writes a register that a load may still be filling.
    if (nt > 0) {
        if constexpr (PipelineDepth<D, G>::value == 2) {     // three tiles, two ahead
            Tile<D, KV> A, B, C;
            issue(A, 0);
            issue(B, 1);
            issue(C, 2);
            for (int ii = 0;; ii += 3) {
                consume_tile<D, G, KV, false>(A, qv, st, c, r, kTileRows);
                if (ii + 1 >= nt) break;
                issue(A, ii + 3);
                consume_tile<D, G, KV, false>(B, qv, st, c, r, kTileRows);
                if (ii + 2 >= nt) break;
                issue(B, ii + 4);
                consume_tile<D, G, KV, false>(C, qv, st, c, r, kTileRows);
                if (ii + 3 >= nt) break;
                issue(C, ii + 5);
            }
        } else {                                              // two tiles, one ahead
            Tile<D, KV> A, B;
            issue(A, 0);
            issue(B, 1);
            for (int ii = 0;; ii += 2) {
                consume_tile<D, G, KV, false>(A, qv, st, c, r, kTileRows);
                if (ii + 1 >= nt) break;
                issue(A, ii + 2);
                consume_tile<D, G, KV, false>(B, qv, st, c, r, kTileRows);
                if (ii + 2 >= nt) break;
                issue(B, ii + 3);
            }
        }
    }
    // Drain the prefetches issued past the window's end (cache hits) once
    // here, so that no later code, and no later loop entry, inherits loads
    // still in flight into registers it reuses.  s_waitcnt vmcnt(0) with the
    // other counters left at their maxima (GFX9 encoding).
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (nf < n) {                                             // the partial last page
#pragma unroll
        for (int h = 0; h < TPP; ++h) {
            const int vh = vlast - h * kTileRows;               // valid rows of this tile
            if (vh <= 0) break;
            Tile<D, KV> T;
            const uint64_t so = slast + (uint64_t)h * kTileBytes;
            load_tile<D, KV>(T, kbase + so, vbase + so, lane_offsets<D, KV>(r, p, vh));
            consume_tile<D, G, KV, true>(T, qv, st, c, r, vh);
        }
    }
}

// Page-claim schedule for a split (row, KV head): the waves of every item of
// the row claim groups of TPG tiles (PG pages) from a cursor the row's items
// share, so a workgroup on a faster XCD takes more of the row; each wave keeps
// its own online-softmax state over the pages it claimed, and the item's
// partial state covers the pages its waves claimed (disjoint sets, merged
// exactly like ranges).  Claim value 0 is the row's last group when that group
// is short or ends in a partial page (handled first, masked and unpipelined,
// by whichever wave draws it); every other value v names full group
// v - has_tail, whose pages are all full.  The full groups run through the
// three-tile pipeline without a drain between groups: a wave claims the group
// after next at the top of each group and loads the next group's page ids
// there, so both are back before their first use and every wait in the loop
// is for a tile that is consumed next.  When the claims run out the
// look-ahead reads the sink.
template <int D, int G, typename KV>
__device__ __forceinline__ void run_claimed(const DecodeParams& P, const u32x4 (&qv)[G][D / 64],
                                            State<D, G>& st, uint32_t* cursor, const int32_t* bt0,
                                            uint32_t len, int hk, int lane, int r, int p) {
    constexpr int TPP = KV::kTilesPerPage;
    constexpr int TPG = 6;
    constexpr int PG = TPG / TPP;
    constexpr int kTileRows = kPageSize / TPP;
    constexpr uint64_t kSlabBytes = (uint64_t)kPageSize * D * KV::kBytes;
    constexpr uint64_t kTileBytes = kSlabBytes / TPP;
    static_assert(PG * TPP == TPG && PG <= 64 && TPG % 3 == 0 && TPG >= 6, "whole pages per group");
    static_assert(kTileBytes <= (uint64_t)kSinkBytes, "the look-ahead sink must hold a tile");
    const char* kbase = reinterpret_cast<const char*>(P.k_pool);
    const char* vbase = reinterpret_cast<const char*>(P.v_pool);
    const uint64_t head_off = (uint64_t)hk * kSlabBytes;
    const uint64_t page_stride = (uint64_t)P.hkv * kSlabBytes;
    const float c = P.scale_log2;
    const int n_row = (int)((len + kPageSize - 1) / kPageSize);
    const int gf = (int)(len / kPageSize) / PG;           // groups made of full pages only
    const uint32_t has_tail = gf * PG < n_row ? 1u : 0u;  // the rest: short, or a partial last page

    auto claim = [&]() -> uint32_t {
        uint32_t v = 0;
        if (lane == 0) {
            // a lane-private copy of the address keeps this a one-lane atomic
            __attribute__((address_space(1))) uint32_t* cp = (__attribute__((address_space(1))) uint32_t*)cursor;
            __asm__ volatile("" : "+v"(cp));
            v = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return v;
    };
    auto full_group = [&](uint32_t v) -> int {           // -1: the tail, or nothing left
        const uint32_t g = v - has_tail;
        return (has_tail && v == 0u) || g >= (uint32_t)gf ? -1 : (int)g;
    };
    // page ids of cnt pages from row page p0 (lanes 0 .. cnt - 1); entries
    // outside the pool are reported and replaced by page 0
    auto load_ids = [&](int p0, int cnt) -> int32_t {
        int32_t v = 0;
        if (lane < cnt) v = bt0[p0 + lane];
        return v;
    };
    auto check_ids = [&](int32_t v, int cnt) -> int32_t {
        const bool bad = lane < cnt && (uint32_t)v >= (uint32_t)P.num_pages;
        const unsigned long long m = __ballot(bad);
        if (m) {
            if (lane == __ffsll(m) - 1) report(P.ctrl, P.host_error, PKV_DEVERR_PAGE_OOB, (uint32_t)v);
            v = bad ? 0 : v;
        }
        return v;
    };
    const LaneOff full = lane_offsets<D, KV>(r, p, kTileRows);
    auto issue = [&](Tile<D, KV>& T, int32_t ids, int t, bool ok) {
        const char* ks = P.sink;
        const char* vs = P.sink;
        if (ok) {
            const int32_t pg = __builtin_amdgcn_readlane(ids, t / TPP);
            const uint64_t so = (uint64_t)(uint32_t)pg * page_stride + head_off + (uint64_t)(t % TPP) * kTileBytes;
            ks = kbase + so;
            vs = vbase + so;
        }
        LaneOff o = full;
        __asm__ volatile("" : "+v"(o.o0), "+v"(o.o1));
        load_tile<D, KV>(T, ks, vs, o);
    };

    uint32_t v = (uint32_t)__builtin_amdgcn_readfirstlane((int)claim());
    if (has_tail && v == 0u) {
        const int p0 = gf * PG;
        const int cnt = n_row - p0;                       // 1 .. PG pages
        const int32_t ids = check_ids(load_ids(p0, cnt), cnt);
        for (int j = 0; j < cnt; ++j) {
            const int32_t pg = __builtin_amdgcn_readlane(ids, j);
            for (int h = 0; h < TPP; ++h) {
                const int vh = min((int)len - ((p0 + j) * kPageSize + h * kTileRows), kTileRows);
                if (vh <= 0) break;
                Tile<D, KV> T;
                const uint64_t so = (uint64_t)(uint32_t)pg * page_stride + head_off + (uint64_t)h * kTileBytes;
                load_tile<D, KV>(T, kbase + so, vbase + so, lane_offsets<D, KV>(r, p, vh));
                consume_tile<D, G, KV, true>(T, qv, st, c, r, vh);
            }
        }
        v = (uint32_t)__builtin_amdgcn_readfirstlane((int)claim());
    }
    int g = full_group(v);
    if (g < 0) return;
    int32_t ids = check_ids(load_ids(g * PG, PG), PG);
    uint32_t cv = claim();                                // the group after this one
    Tile<D, KV> A, B, C;
    issue(A, ids, 0, true);
    issue(B, ids, 1, true);
    issue(C, ids, 2, true);
    for (;;) {
        const int gn = full_group((uint32_t)__builtin_amdgcn_readfirstlane((int)cv));
        const int32_t ids_raw = load_ids((gn >= 0 ? gn : g) * PG, PG);
        cv = claim();                                     // the group after next
        const bool more = gn >= 0;
        int32_t idn = 0;
        // TPG / 3 rounds of the rotation; tile t + 3 is issued after tile t
        // is consumed, from this group or (the last three) the next one
#pragma unroll
        for (int rnd = 0; rnd < TPG / 3; ++rnd) {
            const int t = 3 * rnd;
            consume_tile<D, G, KV, false>(A, qv, st, c, r, kTileRows);
            if (rnd == TPG / 3 - 1) idn = check_ids(ids_raw, PG);
            if (t + 3 < TPG) issue(A, ids, t + 3, true); else issue(A, idn, t + 3 - TPG, more);
            consume_tile<D, G, KV, false>(B, qv, st, c, r, kTileRows);
            if (t + 4 < TPG) issue(B, ids, t + 4, true); else issue(B, idn, t + 4 - TPG, more);
            consume_tile<D, G, KV, false>(C, qv, st, c, r, kTileRows);
            if (t + 5 < TPG) issue(C, ids, t + 5, true); else issue(C, idn, t + 5 - TPG, more);
        }
        if (!more) break;
        g = gn;
        ids = idn;
    }
    // the look-ahead of the last group (sink reads) and the spare claim
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Steal schedule.  Every item of a split (row, KV head) reads the pages of
// its range past the first pool_share() of them itself, in the fixed
// round-robin order (wave w takes every kWaves-th page); the first
// pool_share() pages of all the row's items form the row's shared pool, which
// the waves of the row's items drain once their own pages are done.  Wave w
// of any item takes only pool pages congruent to w modulo kWaves, claimed
// kPoolClaim at a time from a cursor of its own (one per row, KV head and
// wave index, so no cursor sees more than a few hundred claims), and a wave
// that finishes early claims more, so the row's items end within a few
// microseconds of each other instead of following the speed of the XCD each
// one runs on.  Claimed pages fold into the wave's running state, so an item
// still yields one partial state and the merge is unchanged.
// The pool holds full pages only: the row's partial last page stays in the
// last item's own pages.
constexpr int kPoolEighths = 2;                 // pool share of a full item, in eighths
constexpr int kPoolClaim = 3;                   // pages per claim (whole rotations of three tiles)
constexpr int kPoolStep = kPoolClaim * kWaves;  // pool pages per claim round of the 8 waves

// Pages at the start of an item that belong to the row's pool: cp is the
// queue's range length in pages, n the item's own page count.
__device__ __forceinline__ int pool_share(int cp, int n, bool last) {
    const int k = ((cp * kPoolEighths / 8) / kPoolStep) * kPoolStep;
    if (!last) return n < k ? 0 : k;             // (a full item has n = cp pages)
    const int kl = ((n - 1) / kPoolStep) * kPoolStep;   // keep the last page in the item
    return kl < k ? kl : k;
}

// One claim on a wave's pool cursor (lane 0's atomic; the result is read
// later, with readfirstlane, so its round trip overlaps other work).
__device__ __forceinline__ uint32_t pool_claim(uint32_t* cursor, int lane) {
    uint32_t v = 0;
    if (lane == 0) {
        // a lane-private copy of the address keeps this a one-lane atomic
        __attribute__((address_space(1))) uint32_t* cp = (__attribute__((address_space(1))) uint32_t*)cursor;
        __asm__ volatile("" : "+v"(cp));
        v = __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return v;
}

// first: this wave's first claim, made when the item started.
template <int D, int G, typename KV>
__device__ __forceinline__ void run_pool(const DecodeParams& P, const u32x4 (&qv)[G][D / 64],
                                         State<D, G>& st, uint32_t* cursor, uint32_t first, const int32_t* bt0,
                                         int cp, int nch, uint32_t len, int w, int hk, int lane, int r, int p) {
    constexpr int TPP = KV::kTilesPerPage;
    constexpr int TPG = kPoolClaim * TPP;        // tiles per claim
    constexpr int kTileRows = kPageSize / TPP;
    constexpr uint64_t kSlabBytes = (uint64_t)kPageSize * D * KV::kBytes;
    constexpr uint64_t kTileBytes = kSlabBytes / TPP;
    static_assert(TPG % 3 == 0, "a claim is whole rotations of three tiles");
    const char* kbase = reinterpret_cast<const char*>(P.k_pool);
    const char* vbase = reinterpret_cast<const char*>(P.v_pool);
    const uint64_t head_off = (uint64_t)hk * kSlabBytes;
    const uint64_t page_stride = (uint64_t)P.hkv * kSlabBytes;
    const float c = P.scale_log2;
    const int n_row = (int)((len + kPageSize - 1) / kPageSize);
    // claims: gpi per full item, then those of the last item
    const int gpi = pool_share(cp, cp, false) / kPoolStep;
    const int n_last = n_row - (nch - 1) * cp;
    const uint32_t ng = n_last > 0 ? (uint32_t)((nch - 1) * gpi + pool_share(cp, n_last, true) / kPoolStep) : 0u;

    // Page ids of claim v: wave-uniform scalar loads through the constant
    // address space (the block table does not change during the launch, and
    // a wait for a scalar load does not hold the vector loads in flight).
    typedef const __attribute__((address_space(4))) int32_t cint;
    cint* cbt = (cint*)(uintptr_t)bt0;
    struct Ids { int32_t id[kPoolClaim]; };
    auto claim_ids = [&](uint32_t v) -> Ids {
        Ids o;
        const int ci = (int)(v / (uint32_t)gpi), j = (int)(v % (uint32_t)gpi);
        const int base = ci * cp + j * kPoolStep + w;
#pragma unroll
        for (int i = 0; i < kPoolClaim; ++i) o.id[i] = cbt[base + i * kWaves];
        return o;
    };
    // Pages outside the pool read page 0 instead; the first one is reported
    // after the loop.  Branch-free, so that the wait for the ids sits where
    // they are first used.
    int32_t bad = -1;
    auto check = [&](Ids& o) {
#pragma unroll
        for (int i = 0; i < kPoolClaim; ++i) {
            const bool oob = (uint32_t)o.id[i] >= (uint32_t)P.num_pages;
            bad = (oob && bad < 0) ? o.id[i] : bad;
            o.id[i] = oob ? 0 : o.id[i];
        }
    };
    const LaneOff full = lane_offsets<D, KV>(r, p, kTileRows);
    auto issue = [&](Tile<D, KV>& T, const Ids& o, int t, bool ok) {
        const char* ks = P.sink;
        const char* vs = P.sink;
        if (ok) {
            const uint64_t so = (uint64_t)(uint32_t)o.id[t / TPP] * page_stride + head_off +
                                (uint64_t)(t % TPP) * kTileBytes;
            ks = kbase + so;
            vs = vbase + so;
        }
        LaneOff o_ = full;
        __asm__ volatile("" : "+v"(o_.o0), "+v"(o_.o1));
        load_tile<D, KV>(T, ks, vs, o_);
    };

    const uint32_t v0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)first);
    if (v0 >= ng) return;
    Ids cur = claim_ids(v0);
    uint32_t cv = pool_claim(cursor, lane);               // the claim after this one
    check(cur);
    Tile<D, KV> A, B, C;
    issue(A, cur, 0, true);
    issue(B, cur, 1, true);
    issue(C, cur, 2, true);
    for (;;) {
        // the claim made one claim ago: its round trip overlapped the tiles
        // issued since, so reading it does not wait for them
        const uint32_t vn = (uint32_t)__builtin_amdgcn_readfirstlane((int)cv);
        const bool more = vn < ng;
        Ids nxt = cur;
        if (more) {
            nxt = claim_ids(vn);
            cv = pool_claim(cursor, lane);                // the claim after next
        }
#pragma unroll
        for (int rnd = 0; rnd < TPG / 3; ++rnd) {
            const int t = 3 * rnd;
            consume_tile<D, G, KV, false>(A, qv, st, c, r, kTileRows);
            if (rnd == TPG / 3 - 1) {
                // keep the ids' first use (and the wait for them) after the tile
                __builtin_amdgcn_sched_barrier(0);
                check(nxt);
            }
            if (t + 3 < TPG) issue(A, cur, t + 3, true); else issue(A, nxt, t + 3 - TPG, more);
            consume_tile<D, G, KV, false>(B, qv, st, c, r, kTileRows);
            if (t + 4 < TPG) issue(B, cur, t + 4, true); else issue(B, nxt, t + 4 - TPG, more);
            consume_tile<D, G, KV, false>(C, qv, st, c, r, kTileRows);
            if (t + 5 < TPG) issue(C, cur, t + 5, true); else issue(C, nxt, t + 5 - TPG, more);
        }
        if (!more) break;
        cur = nxt;
    }
    // the look-ahead past the last claim (sink reads) and the spare claim
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (bad >= 0 && lane == 0) report(P.ctrl, P.host_error, PKV_DEVERR_PAGE_OOB, (uint32_t)bad);
}

template <int D, int G>
struct Smem {
    float acc[kWaves][G * D];
    float m[kWaves][G];
    float l[kWaves][G];
    uint32_t next;
    uint32_t last;
};

// Partial states travel between workgroups of one launch in the fused merge;
// there they are stored and loaded as relaxed agent-scope atomics, which the
// hardware keeps coherent across the XCDs' separate L2 caches, so no
// L2-wide write-back or invalidate is needed.
template <bool COHERENT>
__device__ __forceinline__ float ld_partial(const float* p) {
    if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}

template <bool COHERENT>
__device__ __forceinline__ void st_partial(float* p, float v) {
    if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// Final outputs.  Two adjacent bf16 outputs travel as one 32-bit word; in
// the resident loop they are stored system-coherently (relaxed atomic
// stores at system scope) so that the host may read them as soon as the step
// is published, without cache write-backs.
__device__ __forceinline__ void store_out_pair(const DecodeParams& P, int b, size_t h, int d, float o0,
                                               float o1) {
    const uint32_t w = (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(P.out + ((size_t)b * P.hq + h) * P.head_dim + d);
    if (P.coherent_out) __hip_atomic_store(dst, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else *dst = w;
}

__device__ __forceinline__ void store_lse(const DecodeParams& P, int b, size_t h, float v) {
    float* dst = P.lse + (size_t)b * P.hq + h;
    if (P.coherent_out) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else *dst = v;
}

// The page cursors of a (row, KV head): one for the page-claim schedule, one
// per wave index for the steal schedule.
__device__ __forceinline__ void rearm_cursors(const DecodeParams& P, int b, int hk) {
    const int n = P.steal ? kWaves : 1;
    uint32_t* c = P.cursors + ((size_t)b * P.hkv + hk) * n * kCursorStride;
    for (int i = 0; i < n; ++i) atomicExch(c + (size_t)i * kCursorStride, 0u);
}

// Exact merge of partial states (PersistentKV page, Methodology 1, "Sequence
// Splitting"): with M = max_c lse_c and w_c = exp(lse_c - M),
// O = sum_c w_c o_c / sum_c w_c and LSE = M + ln sum_c w_c; no states (or
// only neutral ones) give O = 0, LSE = -inf.  fold_states merges, for head g
// and dims d, d + 1 of KV head hk, the n states at range slots first,
// first + step, ...; they are read 32 at a time, all loads of a block issued
// together, and blocks after the first fold in by rescaling (the same
// identity applied twice).  The result has the form of a range's partial
// state, so merged states can be merged again.
template <int D, int G, bool COHERENT>
__device__ __forceinline__ void fold_states(const DecodeParams& P, int hk, int g, int d, int first, int step, int n,
                                            float& out0, float& out1, float& out_lse) {
    constexpr int CB = 32;
    float M = -INFINITY, L = 0.0f, O0 = 0.0f, O1 = 0.0f;
    for (int c0 = 0; c0 < n; c0 += CB) {
        float lv[CB], o0[CB], o1[CB];
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            lv[j] = -INFINITY;
            o0[j] = 0.0f;
            o1[j] = 0.0f;
            if (c0 + j < n) {
                const size_t s = ((size_t)(first + (c0 + j) * step) * P.hkv + hk) * G + g;
                lv[j] = ld_partial<COHERENT>(P.partial_lse + s);
                // the two dims are adjacent: one 8-byte load
                const uint64_t* po = reinterpret_cast<const uint64_t*>(P.partial_o + s * D + d);
                const uint64_t x = COHERENT ? __hip_atomic_load(po, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *po;
                o0[j] = __uint_as_float((uint32_t)x);
                o1[j] = __uint_as_float((uint32_t)(x >> 32));
            }
        }
        float Mb = -INFINITY;
#pragma unroll
        for (int j = 0; j < CB; ++j) Mb = fmaxf(Mb, lv[j]);
        if (Mb == -INFINITY) continue;
        const float Mn = fmaxf(M, Mb);
        const float a = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
        L *= a;
        O0 *= a;
        O1 *= a;
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const float wgt = lv[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((lv[j] - Mn) * kLog2e);
            L += wgt;
            O0 = fmaf(wgt, o0[j], O0);
            O1 = fmaf(wgt, o1[j], O1);
        }
        M = Mn;
    }
    const bool any = L > 0.0f;
    out0 = any ? O0 / L : 0.0f;
    out1 = any ? O1 / L : 0.0f;
    out_lse = any ? M + logf(L) : -INFINITY;
}

// Rows with more ranges than this merge in two levels: each group of
// kMergeGroup consecutive ranges is folded by the last of its
// workgroups to arrive, into the slot of the group's first range (whose
// state it has just read), and the row's last group folds the group states.
// One workgroup alone would read every range's state of the row through one
// CU (512 KiB for 256 ranges at D = 128, G = 4); in two levels the groups
// are read in parallel and the last step reads one state per group.
constexpr int kMergeGroup = 32;

// The final merge of a (row, KV head): the n states at slots first + k step
// into the outputs.  Each thread merges two adjacent dims of one head.
template <int D, int G, int NT, bool COHERENT>
__device__ void merge_row(const DecodeParams& P, int b, int hk, int first, int step, int n, int tid) {
    for (int t = tid; t < G * D / 2; t += NT) {
        const int g = (2 * t) / D, d = (2 * t) % D;
        const size_t h = (size_t)hk * G + g;
        float o0, o1, lse;
        fold_states<D, G, COHERENT>(P, hk, g, d, first, step, n, o0, o1, lse);
        store_out_pair(P, b, h, d, o0, o1);
        if (d == 0) store_lse(P, b, h, lse);
    }
}

// First level of a two-level merge: fold the n ranges from slot first into
// slot first.  Every state is read before any is overwritten (the barrier),
// and the merged state is stored coherently like a range's.
template <int D, int G, int NT, bool COHERENT>
__device__ void merge_group(const DecodeParams& P, int hk, int first, int n, int tid) {
    static_assert(G * D / 2 <= NT, "one (head, dim pair) per thread");
    const bool has = tid < G * D / 2;
    const int g = (2 * tid) / D, d = (2 * tid) % D;
    float o0 = 0.0f, o1 = 0.0f, lse = -INFINITY;
    if (has) fold_states<D, G, COHERENT>(P, hk, g, d, first, 1, n, o0, o1, lse);
    __syncthreads();
    if (has) {
        const size_t s = ((size_t)first * P.hkv + hk) * G + g;
        st_partial<true>(P.partial_o + s * D + d, o0);
        st_partial<true>(P.partial_o + s * D + d + 1, o1);
        if (d == 0) st_partial<true>(P.partial_lse + s, lse);
    }
}

// Claim the next item for this workgroup.  One-shot launches run a static
// first round (workgroup i runs item i) and pop later items past it; the
// resident loop pops every item (a workgroup claims work only while it runs).
// Under the static schedule the next item is simply idx + grid.
__device__ __forceinline__ uint32_t pop_next(const DecodeParams& P, uint32_t idx) {
    if (P.static_sched) return idx + gridDim.x;
    if (P.static_first && (uint32_t)P.qhdr->n_items <= gridDim.x) return gridDim.x;
    return (P.static_first ? gridDim.x : 0u) + atomicAdd(P.head, 1u);
}

// Whether a workgroup finishing an item must claim another.  Not under the
// static schedule, and not in a one-shot launch whose static first round
// already covers the queue (no more items than workgroups): there every
// claim would come back empty, and the claims of all workgroups would queue
// on the one device-scope counter as their items end.
__device__ __forceinline__ bool claims_needed(const DecodeParams& P) {
    if (P.static_sched) return false;
    return !P.static_first || (uint32_t)P.qhdr->n_items > gridDim.x;
}

// One queue item, decoded and checked (all fields wave-uniform).
struct ItemRef {
    uint32_t idx;
    int b, hk, chunk;
    uint32_t tb, te;
    uint32_t len;          // the row's length in tokens
    int nch, base;
    bool ok;
};

__device__ __forceinline__ ItemRef read_item(const DecodeParams& P, uint32_t idx) {
    ItemRef it;
    it.idx = idx;
    const Item* itp = P.items + idx;
    it.b = __builtin_amdgcn_readfirstlane((int)itp->seq);
    it.hk = __builtin_amdgcn_readfirstlane((int)itp->kv_head);
    it.chunk = __builtin_amdgcn_readfirstlane((int)itp->chunk);
    it.tb = (uint32_t)__builtin_amdgcn_readfirstlane((int)itp->tok_begin);
    it.te = (uint32_t)__builtin_amdgcn_readfirstlane((int)itp->tok_end);
    it.ok = it.b >= 0 && it.b < P.batch && it.hk < P.hkv && it.tb < it.te &&
            it.te <= (uint32_t)P.max_tokens && (it.tb % kPageSize) == 0;
    it.nch = 1;
    it.base = 0;
    it.len = it.te;
    if (it.ok) {
        // the row words in one round trip (part_off has batch + 1 entries)
        const int nch = P.n_chunks[it.b];
        const int base = P.part_off[it.b];
        const int len = P.row_len[it.b];
        it.nch = __builtin_amdgcn_readfirstlane(nch);
        const int base_u = __builtin_amdgcn_readfirstlane(base);
        it.len = (uint32_t)__builtin_amdgcn_readfirstlane(len);
        if (it.nch > 1) {
            it.base = base_u;
            const int slot = (it.base + it.chunk) * P.hkv + it.hk;
            it.ok = it.chunk < it.nch && it.base >= 0 && slot >= 0 && (it.base + it.nch) * P.hkv <= P.max_items &&
                    it.len >= it.te && it.len <= (uint32_t)P.max_tokens;
        } else {
            it.ok = it.nch == 1;
        }
    }
    return it;
}

// ONE_SHOT: compiled for the one-shot decode kernel, which alone takes the
// page-claim and steal schedules (the resident loop claims whole items).
template <int D, int G, typename KV, bool ONE_SHOT>
__device__ void process_item(const DecodeParams& P, Smem<D, G>& sm, const ItemRef& it, uint32_t& nxt) {
    constexpr int NPC = D / 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane >> 3;
    const int p = lane & 7;
    const int b = it.b, hk = it.hk;
    const uint32_t tb = it.tb, te = it.te;
    if (!it.ok) {                                  // uniform over the workgroup
        if (tid == 0) {
            report(P.ctrl, P.host_error, PKV_DEVERR_BAD_ITEM, it.idx);
            nxt = pop_next(P, it.idx);
        }
        return;
    }
    const int n_pages = (int)((te - tb + kPageSize - 1) / kPageSize);
    const int first_page = (int)(tb / kPageSize);

    // q as packed bf16, in the dims this lane's cache words hold: qv[g][k]
    // pairs with word k (bf16) or words 2k, 2k + 1 (fp32, two halves)
    u32x4 qv[G][NPC];
    const uint16_t* qrow = P.q + ((size_t)b * P.hq + (size_t)hk * G) * D;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < NPC; ++k) {
            const uint16_t* lo_src;
            const uint16_t* hi_src;
            if constexpr (KV::kBytes == 2) {
                lo_src = qrow + g * D + word_dim<KV>(p, k, 0);
                hi_src = lo_src + 4;
            } else {
                lo_src = qrow + g * D + word_dim<KV>(p, 2 * k, 0);
                hi_src = qrow + g * D + word_dim<KV>(p, 2 * k + 1, 0);
            }
            const uint64_t* l64 = reinterpret_cast<const uint64_t*>(lo_src);
            const uint64_t* h64 = reinterpret_cast<const uint64_t*>(hi_src);
            uint64_t lo, hi;
            if (P.coherent_in) {            // the host may rewrite q between steps
                lo = __hip_atomic_load(l64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                hi = __hip_atomic_load(h64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            } else if constexpr (KV::kBytes == 2) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(lo_src);
                lo = (uint64_t)x.x | ((uint64_t)x.y << 32);
                hi = (uint64_t)x.z | ((uint64_t)x.w << 32);
            } else {
                lo = *l64;
                hi = *h64;
            }
            qv[g][k] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
        }

    State<D, G> st;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        st.m[g] = kNegBig;
        st.l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < D / 8; ++e) st.acc[g][e] = 0.0f;
    }

    if (ONE_SHOT && P.cursors && it.nch > 1 && !P.steal) {   // page-claim schedule: the row's pages are shared
        run_claimed<D, G, KV>(P, qv, st, P.cursors + ((size_t)b * P.hkv + hk) * kCursorStride,
                              P.block_table + (size_t)b * P.bt_stride, it.len, hk, lane, r, p);
    } else {
        // steal schedule: the item's first pages belong to the row's pool
        const bool pool = ONE_SHOT && P.steal && it.nch > 1;
        int cp = 0, skip = 0;
        if (pool) {
            cp = __builtin_amdgcn_readfirstlane(P.qhdr->chunk_tokens) / kPageSize;
            skip = pool_share(cp, n_pages, it.chunk == it.nch - 1);
        }
        const int nb = n_pages - skip;
        const int nw = nb > w ? (nb - w + kWaves - 1) / kWaves : 0;
        const WaveItem wi{tb + (uint32_t)skip * kPageSize, te, w, hk};
        const int32_t* bt_row = P.block_table + (size_t)b * P.bt_stride + first_page + skip + w;
        uint32_t* cursor = pool ? P.cursors + (((size_t)b * P.hkv + hk) * kWaves + w) * kCursorStride : nullptr;
        // the first pool claim is made now, so its result is back by the time
        // this wave's own pages are done
        const uint32_t first_claim = pool ? pool_claim(cursor, lane) : 0u;
        for (int wb = 0; wb < nw; wb += 64) {
            const int n = nw - wb < 64 ? nw - wb : 64;
            int32_t btv = 0;
            if (lane < n) {
                const int32_t* e = bt_row + (size_t)kWaves * (wb + lane);
                btv = P.coherent_in ? (int32_t)__hip_atomic_load(reinterpret_cast<const uint32_t*>(e), __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_SYSTEM)
                                    : *e;
            }
            const bool badl = lane < n && (uint32_t)btv >= (uint32_t)P.num_pages;
            const unsigned long long badm = __ballot(badl);
            if (badm) {                                   // never read outside the pool
                if (lane == __ffsll(badm) - 1) report(P.ctrl, P.host_error, PKV_DEVERR_PAGE_OOB, (uint32_t)btv);
                btv = badl ? 0 : btv;
            }
            run_window<D, G, KV>(P, qv, st, btv, n, wb, wi, r, p);
        }
        if (pool)
            run_pool<D, G, KV>(P, qv, st, cursor, first_claim, P.block_table + (size_t)b * P.bt_stride, cp, it.nch,
                               it.len, w, hk, lane, r, p);
    }
    // Claim the next item only now, near the end of this one: a claim made
    // earlier would hold an item this workgroup cannot start while another
    // workgroup runs dry.  The claim's result is first used after the
    // barrier below, so its round trip overlaps the reductions and the wait
    // for the other waves.
    uint32_t popped = 0;
    if (tid == 0 && claims_needed(P)) {
        // A lane-private copy of the address keeps the compiler from turning
        // this one-lane atomic into its wave-wide form, which reads the
        // result at once.
        __attribute__((address_space(1))) uint32_t* head =
            (__attribute__((address_space(1))) uint32_t*)P.head;
        __asm__ volatile("" : "+v"(head));
        popped = __hip_atomic_fetch_add(head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // Combine the 8 token groups of this wave (lanes r = 0..7 with equal p):
    // each lane's state is rescaled to the group maximum, then summed over
    // lane bits 3..5 and written to LDS.
    constexpr int DPW = KV::kDimsPerWord;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float M = groups_max(st.m[g]);
        const float a = __builtin_amdgcn_exp2f(st.m[g] - M);
        st.l[g] = groups_sum(st.l[g] * a);
        st.m[g] = M;
#pragma unroll
        for (int e = 0; e < D / 8; ++e) st.acc[g][e] *= a;
    }
    if constexpr (KV::kBytes == 2) {
        // bf16 cache: a reduce-scatter of the V = G * D / 8 accumulator
        // values.  Each row-swap permute exchanges half of two registers, so
        // one permute and one add fold two values over a lane bit; after bits
        // 5, 4 and 3 lane r holds the sums of values r * V / 8 ..
        // (r + 1) * V / 8 - 1, and every lane writes its share.  (About a
        // third of the instructions of summing every value on every lane;
        // under the fp32 cache's register pressure its extra live values
        // cost more than it saves, so that cache keeps the all-reduce below.)
        constexpr int V = G * (D / 8);
        float v1[V / 2];
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {       // bit 5: lanes 0-31 keep the low half
            const int g0 = i / (D / 8), e0 = i % (D / 8);
            const int g1 = (V / 2 + i) / (D / 8), e1 = (V / 2 + i) % (D / 8);
            const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.acc[g0][e0]),
                                                            __float_as_uint(st.acc[g1][e1]), false, false);
            v1[i] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
        }
        float v2[V / 4];
#pragma unroll
        for (int i = 0; i < V / 4; ++i) {       // bit 4: even 16-lane rows keep the low half
            const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v1[i]), __float_as_uint(v1[V / 4 + i]),
                                                            false, false);
            v2[i] = __uint_as_float(t[0]) + __uint_as_float(t[1]);
        }
        const bool b3 = (lane >> 3) & 1;        // bit 3: the partner is 8 lanes away in the row
#pragma unroll
        for (int i = 0; i < V / 8; ++i) {
            const float keep = b3 ? v2[V / 8 + i] : v2[i];
            const float send = b3 ? v2[i] : v2[V / 8 + i];
            const int j = r * (V / 8) + i;
            const int g = j / (D / 8), e = j % (D / 8);
            sm.acc[w][g * D + word_dim<KV>(p, e / DPW, e % DPW)] = keep + dpp_f<0x128>(send);
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < D / 8; ++e) st.acc[g][e] = groups_sum(st.acc[g][e]);
        if (r == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int ww = 0; ww < Tile<D, KV>::NW; ++ww)
#pragma unroll
                    for (int e = 0; e < DPW; ++e)
                        sm.acc[w][g * D + word_dim<KV>(p, ww, e)] = st.acc[g][ww * DPW + e];
        }
    }
    if (r == 0 && p == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) { sm.m[w][g] = st.m[g]; sm.l[w][g] = st.l[g]; }
    }
    __syncthreads();
    if (tid == 0) {
        __asm__ volatile("" : "+v"(popped));     // the claim's first use: after the barrier
        nxt = P.static_sched ? it.idx + gridDim.x : (P.static_first ? gridDim.x : 0u) + popped;
    }

    // Combine the 8 waves; each thread finishes two adjacent dims of one head.
    const bool split = it.nch > 1;
    const int slot = split ? (it.base + it.chunk) * P.hkv + hk : 0;
    for (int t = tid; t < G * D / 2; t += kThreads) {
        const int g = (2 * t) / D, d = (2 * t) % D;
        float M = kNegBig;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][g]);
        float L = 0.0f, O0 = 0.0f, O1 = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float a = __builtin_amdgcn_exp2f(sm.m[ww][g] - M);
            L = fmaf(sm.l[ww][g], a, L);
            O0 = fmaf(sm.acc[ww][g * D + d], a, O0);
            O1 = fmaf(sm.acc[ww][g * D + d + 1], a, O1);
        }
        // a state with no tokens (possible only under the page-claim
        // schedule, for an item whose waves found the row's pages taken) is
        // the neutral partial state
        const bool any = L > 0.0f;
        O0 = any ? O0 / L : 0.0f;
        O1 = any ? O1 / L : 0.0f;
        const float lse = any ? (M + log2f(L)) * kLn2 : -INFINITY;
        if (split) {
            float* po = P.partial_o + ((size_t)slot * G + g) * D + d;
            if (P.fused_merge) {
                st_partial<true>(po, O0);
                st_partial<true>(po + 1, O1);
                if (d == 0) st_partial<true>(P.partial_lse + (size_t)slot * G + g, lse);
            } else {
                po[0] = O0;
                po[1] = O1;
                if (d == 0) P.partial_lse[(size_t)slot * G + g] = lse;
            }
        } else {
            const size_t h = (size_t)hk * G + g;
            store_out_pair(P, b, h, d, O0, O1);
            if (d == 0) store_lse(P, b, h, lse);
        }
    }
    if (split && P.fused_merge) {
        // Last arriver of this (row, KV head) merges all its ranges.  Each
        // thread waits until its coherent partial stores have completed
        // (s_waitcnt vmcnt(0)), the workgroup then counts itself in with one
        // atomic, and the workgroup that completes the count reads every
        // partial with coherent loads issued after it saw the count.  Rows
        // with more than kMergeGroup ranges first count in per group of
        // ranges, and the group's last arriver folds the group and then
        // counts the group in for the row, by the same steps.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        const int ngroups = (it.nch + kMergeGroup - 1) / kMergeGroup;
        const bool two_level = ngroups > 1;
        bool row_step = true;                         // uniform over the workgroup
        if (two_level) {
            const int gfirst = (it.chunk / kMergeGroup) * kMergeGroup;
            const int gn = it.nch - gfirst < kMergeGroup ? it.nch - gfirst : kMergeGroup;
            uint32_t* gcount = P.grp_arrive + (size_t)(it.base + gfirst) * P.hkv + hk;
            if (tid == 0) {
                const uint32_t old = atomicAdd(gcount, 1u);
                sm.last = (old + 1 == (uint32_t)gn) ? 1u : 0u;
            }
            __syncthreads();
            row_step = sm.last != 0;
            if (row_step) {
                if (tid == 0) atomicExch(gcount, 0u);    // every range of the group has arrived
                merge_group<D, G, kThreads, true>(P, hk, it.base + gfirst, gn, tid);
                __builtin_amdgcn_s_waitcnt(0x0F70);
                __syncthreads();
            }
        }
        if (row_step) {
            if (tid == 0) {
                const uint32_t old = atomicAdd(&P.arrive[(size_t)b * P.hkv + hk], 1u);
                sm.last = (old + 1 == (uint32_t)(two_level ? ngroups : it.nch)) ? 1u : 0u;
            }
            __syncthreads();
            if (sm.last) {
                if (two_level)
                    merge_row<D, G, kThreads, true>(P, b, hk, it.base, kMergeGroup, ngroups, tid);
                else
                    merge_row<D, G, kThreads, true>(P, b, hk, it.base, 1, it.nch, tid);
                if (tid == 0) {
                    atomicExch(&P.arrive[(size_t)b * P.hkv + hk], 0u);
                    // every item of the row has arrived, so no wave claims from
                    // its cursors any more: the next launch starts them at zero
                    if (P.cursors) rearm_cursors(P, b, hk);
                }
            }
        }
    }
}

template <int D, int G, typename KV>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams P) {
    __shared__ Smem<D, G> sm;
    const int tid = threadIdx.x;
    Ctrl* ctrl = P.ctrl;
    const uint32_t n_items = (uint32_t)P.qhdr->n_items;
    const uint64_t t_enter = P.trace ? wall_clock64() : 0;
    if (blockIdx.x == 0 && tid == 0) {
        // the next launch's pop counter: idle since the previous launch ended
        if (P.head_next) __hip_atomic_store(P.head_next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomicAdd(&ctrl->decode_calls, 1u);
    }
    if (P.fused_merge) {                 // rows with no tokens take the neutral state
        const int n_rows = P.qhdr->n_merge_rows;
        for (int ri = blockIdx.x; ri < n_rows; ri += gridDim.x) {
            const int b = P.merge_rows[ri];
            if (b < 0 || b >= P.batch || P.n_chunks[b] != 0) continue;
            for (int t = tid; t < P.hq * D / 2; t += kThreads) {
                const int h = (2 * t) / D, d = (2 * t) % D;
                store_out_pair(P, b, h, d, 0.0f, 0.0f);
                if (d == 0) store_lse(P, b, h, -INFINITY);
            }
        }
    }
    uint32_t idx = blockIdx.x;                     // first round: static assignment
    if (P.trace && tid == 0 && n_items + blockIdx.x < (uint32_t)P.trace_cap) {
        // workgroup record after the item records: entry time, start of work
        uint64_t* rec = P.trace + 4ull * (n_items + blockIdx.x);
        rec[0] = (uint64_t)blockIdx.x | (1ull << 63) | ((uint64_t)idx << 32);
        rec[1] = t_enter;
        rec[2] = wall_clock64();
        rec[3] = (uint64_t)__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11)) |
                 ((uint64_t)__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11)) << 32);
    }
    while (idx < n_items) {
        uint32_t nxt = 0;
        uint64_t t_start = 0;
        if (P.trace) t_start = wall_clock64();
        // counted as the item starts, so the add's round trip overlaps the
        // item instead of lengthening the launch's end
        if (tid == 0 && P.done_lines) atomicAdd(P.done_lines + 32 * (blockIdx.x % kDoneLines), 1u);
        process_item<D, G, KV, true>(P, sm, read_item(P, idx), nxt);
        if (P.trace && tid == 0 && idx < (uint32_t)P.trace_cap) {
            const uint64_t t_end = wall_clock64();
            const uint32_t hw = __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));   // HW_ID
            const uint32_t xcc = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11)); // XCC_ID
            uint64_t* rec = P.trace + 4ull * idx;
            rec[0] = (uint64_t)idx | ((uint64_t)blockIdx.x << 32);
            rec[1] = t_start;
            rec[2] = t_end;
            rec[3] = (uint64_t)hw | ((uint64_t)xcc << 32);
        }
        __syncthreads();
        if (tid == 0) sm.next = nxt;
        __syncthreads();
        idx = __builtin_amdgcn_readfirstlane(sm.next);
    }
}

// ---------------------------------------------------------------------------
// Resident session loop.  Launched once; it serves steps that the host
// publishes through an epoch word in host memory, the "publish the input,
// wait for the output" boundary of a persistent kernel (Wave Persistent
// Kernel note, "What a persistent kernel is"; the control record of
// "Runtime and timing boundary").  A step's work is the step's compact queue
// repeated over the layers, in layer-major order: work unit u is item
// u mod n_items of layer u / n_items.  Layer l + 1 of a row starts only after
// every item of layer l of that row has finished, the ordering a layer
// stack imposes.  Waiting cannot deadlock: every grid workgroup is resident
// (one per CU), units are claimed in increasing order, and the unfinished
// unit with the smallest index has all of its predecessors finished.  Every
// wait has a wall-clock limit, so the kernel always exits.

__device__ __forceinline__ uint32_t ld_sys(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t ld_sys64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Wave-uniform copies (scalar registers) of values every lane loaded alike.
__device__ __forceinline__ uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ uint64_t uni64(uint64_t x) {
    return (uint64_t)uni((uint32_t)x) | ((uint64_t)uni((uint32_t)(x >> 32)) << 32);
}
__device__ __forceinline__ uint64_t ld_desc64(const void* p) {
    return uni64(ld_sys64(reinterpret_cast<const uint64_t*>(p)));
}
__device__ __forceinline__ uint32_t ld_desc32(const void* p) {
    return uni(ld_sys(reinterpret_cast<const uint32_t*>(p)));
}

__device__ __forceinline__ uint32_t ld_agt(const void* p) {
    return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agt64(const void* p) {
    return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Item and row metadata come from the device mirror of the step's queue,
// rewritten every other step: agent-coherent loads (no stale L2 lines).
__device__ __forceinline__ ItemRef read_item_mirror(const DecodeParams& P, uint32_t idx) {
    ItemRef it;
    it.idx = idx;
    const uint64_t a = ld_agt64(P.items + idx), b = ld_agt64(reinterpret_cast<const uint64_t*>(P.items + idx) + 1);
    const uint32_t w0 = (uint32_t)a, w1 = (uint32_t)(a >> 32), w2 = (uint32_t)b, w3 = (uint32_t)(b >> 32);
    it.b = __builtin_amdgcn_readfirstlane((int)w0);
    it.hk = __builtin_amdgcn_readfirstlane((int)(w1 & 0xFFFFu));
    it.chunk = __builtin_amdgcn_readfirstlane((int)(w1 >> 16));
    it.tb = (uint32_t)__builtin_amdgcn_readfirstlane((int)w2);
    it.te = (uint32_t)__builtin_amdgcn_readfirstlane((int)w3);
    it.ok = it.b >= 0 && it.b < P.batch && it.hk < P.hkv && it.tb < it.te &&
            it.te <= (uint32_t)P.max_tokens && (it.tb % kPageSize) == 0;
    it.nch = 1;
    it.base = 0;
    it.len = it.te;              // the loop reads each item's own range only
    if (it.ok) {
        const uint32_t nch = ld_agt(P.n_chunks + it.b), base = ld_agt(P.part_off + it.b);
        it.nch = __builtin_amdgcn_readfirstlane((int)nch);
        const int base_u = __builtin_amdgcn_readfirstlane((int)base);
        if (it.nch > 1) {
            it.base = base_u;
            const int slot = (it.base + it.chunk) * P.hkv + it.hk;
            it.ok = it.chunk < it.nch && it.base >= 0 && slot >= 0 && (it.base + it.nch) * P.hkv <= P.max_items;
        } else {
            it.ok = it.nch == 1;
        }
    }
    return it;
}

__device__ __forceinline__ void st_agt(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// KV append (resident loop, append = 1): the item that ends at its row's
// newest token j = te - 1 first writes that token's K and V for its head into
// the cache, so no other workgroup depends on the write (a page lies inside
// one range, ranges being whole pages).  When j opens a page the step's grant
// for the row is the page id, and every head's item writes it into the block
// table (the same value).  Stores are agent-coherent: later steps read the
// row and the entry from other XCDs.  All threads of the workgroup call this.
template <int D, typename KV>
__device__ void append_token(const DecodeParams& Q, const int32_t* grants, const ItemRef& it,
                             const char* new_k, const char* new_v, int tid) {
    const uint32_t j = it.te - 1;
    const int pj = (int)(j / kPageSize), off = (int)(j % kPageSize);
    uint32_t* btw = reinterpret_cast<uint32_t*>(const_cast<int32_t*>(Q.block_table) + (size_t)it.b * Q.bt_stride + pj);
    int32_t page = off == 0 ? (int32_t)ld_agt(reinterpret_cast<const uint32_t*>(grants) + it.b)
                            : (int32_t)ld_sys(btw);
    page = __builtin_amdgcn_readfirstlane(page);
    if ((uint32_t)page >= (uint32_t)Q.num_pages) {             // never write outside the pool
        if (tid == 0) report(Q.ctrl, Q.host_error, PKV_DEVERR_PAGE_OOB, (uint32_t)page);
        return;
    }
    if (off == 0 && tid == 0) st_agt(btw, (uint32_t)page);
    const size_t row = (((size_t)page * Q.hkv + it.hk) * kPageSize + off) * D * KV::kBytes;
    const size_t src = ((size_t)it.b * Q.hkv + it.hk) * D * KV::kBytes;
    uint32_t* dk = reinterpret_cast<uint32_t*>(const_cast<char*>(reinterpret_cast<const char*>(Q.k_pool)) + row);
    uint32_t* dv = reinterpret_cast<uint32_t*>(const_cast<char*>(reinterpret_cast<const char*>(Q.v_pool)) + row);
    const uint32_t* sk = reinterpret_cast<const uint32_t*>(new_k + src);
    const uint32_t* sv = reinterpret_cast<const uint32_t*>(new_v + src);
    for (int t = tid; t < D * KV::kBytes / 4; t += kThreads) {
        st_agt(dk + t, ld_sys(sk + t));
        st_agt(dv + t, ld_sys(sv + t));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);        // the writes are done before any wave reads the page
    __syncthreads();
}

// Spin (thread 0) until *p >= target, the exit flag rises, or the limit.
__device__ __forceinline__ bool wait_at_least(const uint32_t* p, uint32_t target, const LoopParams& L) {
    const uint64_t t0 = wall_clock64();
    while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (__hip_atomic_load(&L.lglobal->dev_exit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
        if (wall_clock64() - t0 > L.timeout_ticks) return false;
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

template <int D, int G, typename KV>
__global__ __launch_bounds__(kThreads) void resident_kernel(LoopParams L) {
    __shared__ Smem<D, G> sm;
    __shared__ uint32_t s_epoch, s_exit;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0) st_sys(&L.lctrl->alive, 1u);
    uint32_t seen = 0;
    for (;;) {
        // 1. wait for the next published step.  Only workgroup 0 polls host
        // memory (one PCIe read per poll); it mirrors what it sees into device
        // memory, which the other workgroups poll.
        if (tid == 0) {
            const uint64_t t0 = wall_clock64();
            uint32_t e = seen, x = 0;
            if (blockIdx.x == 0) {
                for (;;) {
                    // in_epoch and exit_flag share one 64-bit word
                    const uint64_t both = ld_sys64(reinterpret_cast<const uint64_t*>(&L.lctrl->in_epoch));
                    if ((uint32_t)(both >> 32)) { x = 1; break; }
                    e = (uint32_t)both;
                    if (e != seen) break;
                    if (wall_clock64() - t0 > L.timeout_ticks) { x = 2; break; }
                    __builtin_amdgcn_s_sleep(16);
                }
                if (x) {
                    __hip_atomic_store(&L.lglobal->dev_exit, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (x == 2) st_sys(&L.lctrl->exit_reason, 2u);
                }
            } else {
                // steps are taken strictly in order: a workgroup that lags
                // still serves (and checks out of) every step
                for (;;) {
                    x = __hip_atomic_load(&L.lglobal->dev_exit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (x) break;
                    const uint32_t d = __hip_atomic_load(&L.lglobal->dev_epoch, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                    if ((int32_t)(d - seen) >= 1) { e = seen + 1; break; }
                    if (wall_clock64() - t0 > L.timeout_ticks + L.timeout_ticks / 4) { x = 2; break; }
                    __builtin_amdgcn_s_sleep(16);
                }
            }
            s_epoch = e;
            s_exit = x;
        }
        __syncthreads();
        if (s_exit) break;
        const uint32_t e = s_epoch;
        seen = e;
        LoopSlotCtr* ctr = reinterpret_cast<LoopSlotCtr*>(L.counters + (uint64_t)(e & 1u) * L.counter_bytes);
        uint32_t* done = reinterpret_cast<uint32_t*>(ctr + 1);
        if (blockIdx.x == 0 && e > 2u) {
            // the slot last served step e - 2: every workgroup must have
            // checked out of it (and the slot been re-armed) before reuse
            if (tid == 0)
                s_exit = wait_at_least(&ctr->retired, e - 2u, L) ? 0u : 3u;
            __syncthreads();
            if (s_exit) {
                if (tid == 0) st_sys(&L.lctrl->exit_reason, 3u);
                break;
            }
        }
        if (blockIdx.x == 0) {
            // Workgroup 0 copies the step's slot (descriptor, queue header,
            // row tables, items) from host memory into the device mirror with
            // all its threads, then releases the step to the other workgroups.
            const uint64_t* src = reinterpret_cast<const uint64_t*>(L.slots + (uint64_t)(e & 1u) * L.slot_bytes);
            uint64_t* dst = reinterpret_cast<uint64_t*>(L.mirror + (uint64_t)(e & 1u) * L.slot_bytes);
            __shared__ uint32_t s_nitems;
            if (tid == 0) s_nitems = ld_sys(reinterpret_cast<const uint32_t*>(
                                  reinterpret_cast<const unsigned char*>(src) + L.q_hdr_off));
            __syncthreads();
            const uint32_t ni = uni(s_nitems);
            const uint64_t bytes = L.q_items_off + 16ull * (ni < (uint32_t)L.base.max_items ? ni : (uint32_t)L.base.max_items);
            for (uint64_t w = tid; w < bytes / 8; w += kThreads)
                __hip_atomic_store(dst + w, ld_sys64(src + w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (tid == 0) __hip_atomic_store(&L.lglobal->dev_epoch, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // 2. the step's descriptor and queue header, from the device mirror,
        // shared through LDS.
        const unsigned char* slot = L.mirror + (uint64_t)(e & 1u) * L.slot_bytes;
        const LoopDesc* dsc = reinterpret_cast<const LoopDesc*>(slot);
        __shared__ uint64_t s_desc[17];
        if (tid < 17) {                           // 16 descriptor words + n_items | n_merge_rows << 32
            const uint64_t* d64 = tid < 16 ? reinterpret_cast<const uint64_t*>(dsc) + tid
                                           : reinterpret_cast<const uint64_t*>(slot + L.q_hdr_off);
            s_desc[tid] = ld_agt64(d64);
        }
        __syncthreads();
        DecodeParams P = L.base;
        P.q = reinterpret_cast<const uint16_t*>(uni64(s_desc[0]));
        P.k_pool = reinterpret_cast<const uint16_t*>(uni64(s_desc[1]));
        P.v_pool = reinterpret_cast<const uint16_t*>(uni64(s_desc[2]));
        P.block_table = reinterpret_cast<const int32_t*>(uni64(s_desc[3]));
        P.out = reinterpret_cast<uint16_t*>(uni64(s_desc[4]));
        P.lse = reinterpret_cast<float*>(uni64(s_desc[5]));
        const int64_t ls_q = (int64_t)uni64(s_desc[6]);
        const int64_t ls_kv = (int64_t)uni64(s_desc[7]);
        const int64_t ls_bt = (int64_t)uni64(s_desc[8]);
        const int64_t ls_out = (int64_t)uni64(s_desc[9]);
        const int64_t ls_lse = (int64_t)uni64(s_desc[10]);
        P.batch = (int32_t)uni((uint32_t)s_desc[11]);
        P.bt_stride = (int32_t)uni((uint32_t)(s_desc[11] >> 32));
        const int n_layers = (int)uni((uint32_t)s_desc[12]);
        const char* new_k = reinterpret_cast<const char*>(uni64(s_desc[13]));
        const char* new_v = reinterpret_cast<const char*>(uni64(s_desc[14]));
        const int64_t ls_new = (int64_t)uni64(s_desc[15]);
        const int32_t* grants = reinterpret_cast<const int32_t*>(slot + L.grant_off);
        P.qhdr = reinterpret_cast<const QHdr*>(slot + L.q_hdr_off);
        P.n_chunks = reinterpret_cast<const int32_t*>(slot + L.q_nch_off);
        P.part_off = reinterpret_cast<const int32_t*>(slot + L.q_poff_off);
        P.merge_rows = reinterpret_cast<const int32_t*>(slot + L.q_mrows_off);
        P.items = reinterpret_cast<const Item*>(slot + L.q_items_off);
        const uint32_t n_items = uni((uint32_t)s_desc[16]);
        const uint32_t n_mrows = uni((uint32_t)(s_desc[16] >> 32));
        P.head = &ctr->head;
        const uint32_t total = n_items * (uint32_t)n_layers;
        const uint32_t units = total + 1;        // + one unit: rows with no tokens
        bool ok = true;
        if (tid == 0) sm.next = pop_next(P, 0);  // every unit is popped
        __syncthreads();
        uint32_t idx = __builtin_amdgcn_readfirstlane(sm.next);
        while (idx < units) {
            uint32_t nxt = 0;
            int row = -1;
            if (idx < total) {
                const int layer = (int)(idx / n_items);
                const uint32_t i = idx - (uint32_t)layer * n_items;
                DecodeParams Q = P;
                Q.q = P.q + layer * ls_q;
                // the layer stride counts cache elements
                Q.k_pool = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(P.k_pool) +
                                                             layer * ls_kv * KV::kBytes);
                Q.v_pool = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(P.v_pool) +
                                                             layer * ls_kv * KV::kBytes);
                Q.block_table = P.block_table + layer * ls_bt;
                Q.out = P.out + layer * ls_out;
                Q.lse = P.lse + layer * ls_lse;
                Q.partial_o = P.partial_o + (uint64_t)layer * L.partial_o_layer;
                Q.partial_lse = P.partial_lse + (uint64_t)layer * L.partial_lse_layer;
                Q.arrive = P.arrive + (uint64_t)layer * L.arrive_layer;
                Q.grp_arrive = P.grp_arrive + (uint64_t)layer * L.grp_layer;
                // one thread reads the item over PCIe; the workgroup shares it
                __shared__ ItemRef s_it;
                if (tid == 0) s_it = read_item_mirror(Q, i);
                __syncthreads();
                ItemRef it;
                it.idx = uni(s_it.idx);
                it.b = (int)uni((uint32_t)s_it.b);
                it.hk = (int)uni((uint32_t)s_it.hk);
                it.chunk = (int)uni((uint32_t)s_it.chunk);
                it.tb = uni(s_it.tb);
                it.te = uni(s_it.te);
                it.nch = (int)uni((uint32_t)s_it.nch);
                it.base = (int)uni((uint32_t)s_it.base);
                it.len = uni(s_it.len);
                it.ok = uni(s_it.ok ? 1u : 0u) != 0u;
                row = it.ok ? it.b : -1;
                if (layer > 0 && it.ok) {            // the row's previous layer must be complete
                    if (tid == 0) {
                        const uint32_t need = (uint32_t)layer * (uint32_t)it.nch * (uint32_t)P.hkv;
                        s_exit = wait_at_least(done + it.b, need, L) ? 0u : 3u;
                    }
                    __syncthreads();
                    if (s_exit) { ok = false; break; }
                }
                if (L.append && it.ok && it.chunk == it.nch - 1)
                    append_token<D, KV>(Q, grants, it, new_k + layer * ls_new * KV::kBytes,
                                        new_v + layer * ls_new * KV::kBytes, tid);
                process_item<D, G, KV, false>(Q, sm, it, nxt);
            } else {
                // rows with no tokens take the neutral state, in every layer;
                // thread 0 finds them (64 merge rows at a time), all threads write
                __shared__ int32_t s_rows[64];
                __shared__ int32_t s_nrows;
                for (uint32_t r0 = 0; r0 < n_mrows; r0 += 64) {
                    if (tid == 0) {
                        int cnt = 0;
                        for (uint32_t ri = r0; ri < n_mrows && ri < r0 + 64; ++ri) {
                            const int b = (int)ld_agt(P.merge_rows + ri);
                            if (b < 0 || b >= P.batch) continue;
                            if (ld_agt(P.n_chunks + b) == 0) s_rows[cnt++] = b;
                        }
                        s_nrows = cnt;
                    }
                    __syncthreads();
                    const int cnt = (int)uni((uint32_t)s_nrows);
                    for (int j = 0; j < cnt; ++j) {
                        const int b = (int)uni((uint32_t)s_rows[j]);
                        for (int l = 0; l < n_layers; ++l) {
                            DecodeParams Q = P;
                            Q.out = P.out + l * ls_out;
                            Q.lse = P.lse + l * ls_lse;
                            for (int t = tid; t < P.hq * D / 2; t += kThreads) {
                                const int h = (2 * t) / D, d = (2 * t) % D;
                                store_out_pair(Q, b, h, d, 0.0f, 0.0f);
                                if (d == 0) store_lse(Q, b, h, -INFINITY);
                            }
                        }
                    }
                    __syncthreads();
                }
                if (tid == 0) nxt = pop_next(P, idx);
            }
            // publish completion: this unit's outputs are stored, then count it
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            if (tid == 0) {
                if (row >= 0) atomicAdd(done + row, 1u);
                const uint32_t old = atomicAdd(&ctr->step_done, 1u);
                if (old + 1 == units) {              // last unit of the step: publish
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
                    st_sys(&L.lctrl->out_epoch, e);
                }
                sm.next = nxt;
            }
            __syncthreads();
            idx = __builtin_amdgcn_readfirstlane(sm.next);
        }
        if (!ok) {
            if (tid == 0) st_sys(&L.lctrl->exit_reason, 3u);
            break;
        }
        // Check out of the step: this workgroup pops from the slot no more.
        // The last workgroup to check out re-arms the slot's counters, then
        // marks the slot retired for step e.
        if (tid == 0) {
            const uint32_t old = atomicAdd(&ctr->checkout, 1u);
            if (old + 1 == gridDim.x) {
                atomicExch(&ctr->head, 0u);
                atomicExch(&ctr->step_done, 0u);
                for (int b = 0; b < P.batch && b < L.max_batch; ++b) atomicExch(done + b, 0u);
                atomicExch(&ctr->checkout, 0u);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_store(&ctr->retired, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (blockIdx.x == 0 && tid == 0) st_sys(&L.lctrl->heartbeat, e);
    }
    if (blockIdx.x == 0 && tid == 0) st_sys(&L.lctrl->alive, 0u);
}

// The separate merge kernel: one workgroup per (merge row, KV head).
// Merge kernel of the separate-merge mode: one workgroup per (row, KV head),
// with the fused merge's two levels for rows of more than kMergeGroup ranges
// (the groups one after another), so that both modes give the same bits.
template <int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams P) {
    const int n_rows = P.qhdr->n_merge_rows;
    const int ri = blockIdx.x / P.hkv;
    const int hk = blockIdx.x % P.hkv;
    if (ri >= n_rows) return;
    const int b = P.merge_rows[ri];
    if (b < 0 || b >= P.batch) return;
    const int nc = P.n_chunks[b];
    const int base = P.part_off[b];
    if (nc == 1 || nc < 0 || base < 0 || (base + nc) * P.hkv > P.max_items) return;
    if (nc > kMergeGroup) {
        for (int gfirst = 0; gfirst < nc; gfirst += kMergeGroup)
            merge_group<D, G, 256, false>(P, hk, base + gfirst, nc - gfirst < kMergeGroup ? nc - gfirst : kMergeGroup,
                                          threadIdx.x);
        // the group states were stored by this workgroup: wait for them, and
        // read them with coherent loads (not through this CU's L1)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        merge_row<D, G, 256, true>(P, b, hk, base, kMergeGroup, (nc + kMergeGroup - 1) / kMergeGroup, threadIdx.x);
    } else {
        merge_row<D, G, 256, false>(P, b, hk, base, 1, nc, threadIdx.x);
    }
    // the decode kernel has finished: its page cursor starts the next launch at zero
    if (P.cursors && threadIdx.x == 0) rearm_cursors(P, b, hk);
}

// Device queue builder: the same bytes as the host builder, from device
// context lengths, by one workgroup.  Rows are processed in contiguous blocks
// per thread; three block-wide exclusive scans give each row its first item,
// its partial-slot offset and its merge-row position.
constexpr int kBuildThreads = 1024;
constexpr int kBuildMaxRows = 4096;

__device__ int block_exclusive_scan(int v, int* buf) {
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int o = 1; o < kBuildThreads; o <<= 1) {
        const int x = t >= o ? buf[t - o] : 0;
        __syncthreads();
        buf[t] += x;
        __syncthreads();
    }
    const int incl = buf[t];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(kBuildThreads) void build_queue_kernel(BuildParams P) {
    __shared__ int s_buf[kBuildThreads];
    __shared__ int s_item0[kBuildMaxRows + 1];
    __shared__ int s_max, s_bad, s_total[3];
    const int t = threadIdx.x;
    const int B = P.batch;
    if (t == 0) { s_max = 0; s_bad = -1; }
    __syncthreads();
    const int per = (B + kBuildThreads - 1) / kBuildThreads;
    const int r0 = t * per < B ? t * per : B;
    const int r1 = r0 + per < B ? r0 + per : B;
    int lmax = 0;
    for (int b = r0; b < r1; ++b) {
        const int L = P.ctx_lens[b];
        if (L < 0 || L > P.max_tokens) atomicCAS(&s_bad, -1, b);
        lmax = L > lmax ? L : lmax;
    }
    atomicMax(&s_max, lmax);
    __syncthreads();
    // Chunk mode "fit" (chunk 0): the smallest T pages with
    // sum_b ceil(pages_b / T) <= K = max(1, CUs / Hkv), by bisection over T
    // with a block-wide sum per step (clamped at K + 1, which is all the
    // comparison needs); the longest row's pages when no T reaches K; never
    // below the floor P.fit_min_pages.
    int chunk = P.chunk;
    if (chunk == 0) {
        __shared__ unsigned long long s_cnt;
        const unsigned long long budget = (unsigned long long)(P.num_cus / P.hkv > 1 ? P.num_cus / P.hkv : 1);
        const int longest = (s_max + kPageSize - 1) / kPageSize;
        auto ranges = [&](int T) -> unsigned long long {
            unsigned long long local = 0;
            for (int b = r0; b < r1; ++b) {
                const int L = P.ctx_lens[b];
                const int pages = L > 0 ? (L + kPageSize - 1) / kPageSize : 0;
                local += (unsigned long long)((pages + T - 1) / T);
            }
            if (local > budget + 1) local = budget + 1;
            __syncthreads();
            if (t == 0) s_cnt = 0;
            __syncthreads();
            atomicAdd(&s_cnt, local);
            __syncthreads();
            return s_cnt;
        };
        int T = longest > 0 ? longest : 1;
        if (longest > 0 && ranges(longest) <= budget) {
            int lo = 1, hi = longest;
            while (lo < hi) {
                const int mid = lo + (hi - lo) / 2;
                if (ranges(mid) <= budget) hi = mid; else lo = mid + 1;
            }
            T = lo;
        }
        chunk = (T > P.fit_min_pages ? T : P.fit_min_pages) * kPageSize;
    }
    bool split;
    if (P.policy == PKV_POLICY_NO_SPLIT) split = false;
    else if (P.policy == PKV_POLICY_SPLIT) split = true;
    else split = B > 0 && (long long)B * P.hkv < P.num_cus && s_max > chunk;

    auto nchunks = [&](int L) -> int {
        if (L <= 0) return 0;
        return split ? (L + chunk - 1) / chunk : 1;
    };
    int c_items = 0, c_parts = 0, c_merge = 0;
    for (int b = r0; b < r1; ++b) {
        const int nc = nchunks(P.ctx_lens[b]);
        c_items += nc * P.hkv;
        c_parts += nc > 1 ? nc : 0;
        c_merge += nc != 1 ? 1 : 0;
    }
    int o_items = block_exclusive_scan(c_items, s_buf);
    int o_parts = block_exclusive_scan(c_parts, s_buf);
    int o_merge = block_exclusive_scan(c_merge, s_buf);
    if (t == kBuildThreads - 1) {
        s_total[0] = o_items + c_items;
        s_total[1] = o_parts + c_parts;
        s_total[2] = o_merge + c_merge;
    }
    for (int b = r0; b < r1; ++b) {
        const int nc = nchunks(P.ctx_lens[b]);
        P.n_chunks[b] = nc;
        P.row_len[b] = P.ctx_lens[b];
        P.part_off[b] = o_parts;
        s_item0[b] = o_items;
        if (nc != 1) P.merge_rows[o_merge++] = b;
        o_items += nc * P.hkv;
        o_parts += nc > 1 ? nc : 0;
    }
    __syncthreads();
    const int total = s_total[0];
    const bool ok = s_bad < 0 && total <= P.max_items;
    if (t == 0) {
        P.part_off[B] = s_total[1];
        s_item0[B] = total;
        if (s_bad >= 0) report(P.ctrl, P.host_error, PKV_DEVERR_BAD_ITEM, (uint32_t)s_bad);
        else if (total > P.max_items) report(P.ctrl, P.host_error, PKV_DEVERR_BAD_ITEM, (uint32_t)total);
    }
    if (t < 64) {
        int32_t* hw = reinterpret_cast<int32_t*>(P.qhdr);
        int32_t val = 0;
        if (t == 0) val = ok ? total : 0;
        else if (t == 1) val = s_total[2];
        else if (t == 2) val = split ? 1 : 0;
        else if (t == 3) val = chunk;
        else if (t == 4) val = B;
        hw[t] = val;
    }
    __syncthreads();
    if (!ok) return;
    for (int i = t; i < total; i += kBuildThreads) {
        int lo = 0, hi = B - 1;                       // last row with item0 <= i
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_item0[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const int b = lo;
        const int L = P.ctx_lens[b];
        const int nc = nchunks(L);
        const int rel = i - s_item0[b];
        const int h = rel / nc, c = rel % nc;
        Item it;
        it.seq = (uint32_t)b;
        it.kv_head = (uint16_t)h;
        it.chunk = (uint16_t)c;
        it.tok_begin = split ? (uint32_t)(c * chunk) : 0u;
        const long long e = split ? (long long)(c + 1) * chunk : (long long)L;
        it.tok_end = (uint32_t)(e < L ? e : L);
        P.items[i] = it;
    }
}

// Test hook: one wave runs the decode kernel's own gather over every tile of
// one item, in order, and stores the rows it read (k_out / v_out hold the
// item's tokens as [token][D] rows of the cache's element type).
template <int D, typename KV>
__global__ __launch_bounds__(64) void debug_gather_kernel(DecodeParams P, int item_index,
                                                          char* k_out, char* v_out) {
    constexpr int TPP = KV::kTilesPerPage, kTileRows = kPageSize / TPP;
    constexpr size_t kRowBytes = (size_t)D * KV::kBytes;
    const int lane = threadIdx.x;
    const int r = lane >> 3, p = lane & 7;
    if (item_index < 0 || item_index >= P.qhdr->n_items) return;
    const Item it = P.items[item_index];
    if ((int)it.seq >= P.batch || (int)it.kv_head >= P.hkv || it.tok_begin >= it.tok_end) return;
    const int n_pages = (int)((it.tok_end - it.tok_begin + kPageSize - 1) / kPageSize);
    const int first_page = (int)(it.tok_begin / kPageSize);
    for (int j = 0; j < n_pages; ++j) {
        int32_t pg = P.block_table[(size_t)it.seq * P.bt_stride + first_page + j];
        if ((uint32_t)pg >= (uint32_t)P.num_pages) {
            if (lane == 0) report(P.ctrl, P.host_error, PKV_DEVERR_PAGE_OOB, (uint32_t)pg);
            pg = 0;
        }
        const int rem = (int)(it.tok_end - it.tok_begin) - j * kPageSize;
        const int valid = rem < kPageSize ? rem : kPageSize;
        for (int h = 0; h < TPP; ++h) {
            const int vh = valid - h * kTileRows;
            if (vh <= 0) break;
            Tile<D, KV> t;
            const uint64_t slab = ((uint64_t)(uint32_t)pg * P.hkv + it.kv_head) * kPageSize * kRowBytes +
                                  (uint64_t)h * kTileRows * kRowBytes;
            load_tile<D, KV>(t, reinterpret_cast<const char*>(P.k_pool) + slab,
                             reinterpret_cast<const char*>(P.v_pool) + slab, lane_offsets<D, KV>(r, p, vh));
#pragma unroll
            for (int jj = 0; jj < KV::kRows; ++jj) {
                const int tok = 8 * jj + r;
                if (tok >= vh) continue;
                const size_t row = (size_t)(j * kPageSize + h * kTileRows + tok) * kRowBytes;
#pragma unroll
                for (int w = 0; w < Tile<D, KV>::NW; ++w) {
                    const size_t off = row + 128 * w + 16 * p;
                    *reinterpret_cast<u32x4*>(k_out + off) = t.k[jj][w];
                    *reinterpret_cast<u32x4*>(v_out + off) = t.v[jj][w];
                }
            }
        }
    }
}

// Streaming copy used as a bandwidth and traffic-counter reference: each
// thread moves four independent 16-byte vectors per step (grid-stride).
__global__ __launch_bounds__(256) void copy_probe_kernel(u32x4* __restrict__ dst,
                                                         const u32x4* __restrict__ src, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

// Read-only stream: four independent non-temporal 16-byte loads per thread
// per step, folded with xor into one word per thread (kept live by the final
// store).
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n,
                                                         uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const char* s = reinterpret_cast<const char*>(src);
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = ld_stream(s + 16 * i), b = ld_stream(s + 16 * (i + stride));
        const u32x4 c = ld_stream(s + 16 * (i + 2 * stride)), d = ld_stream(s + 16 * (i + 3 * stride));
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n; i += stride) acc ^= ld_stream(s + 16 * i);
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ void init_ctrl_kernel(Ctrl* c, uint32_t* arrive, int n_arrive) {
    uint32_t* w = reinterpret_cast<uint32_t*>(c);          // Ctrl and the items-done counters
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < (int)(kCtrlBytes / 4); i += gridDim.x * blockDim.x)
        w[i] = 0u;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_arrive; i += gridDim.x * blockDim.x)
        arrive[i] = 0u;
}

template <int D, int G>
int launch_decode_t(const DecodeParams& p, int kv_dtype, int grid, hipStream_t s) {
    if (kv_dtype == PKV_KV_F32)
        hipLaunchKernelGGL((decode_kernel<D, G, KvF32>), dim3(grid), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<D, G, KvBf16>), dim3(grid), dim3(kThreads), 0, s, p);
    return (int)hipGetLastError();
}

template <int D, int G>
int launch_merge_t(const DecodeParams& p, int n_rows, hipStream_t s) {
    hipLaunchKernelGGL((merge_kernel<D, G>), dim3(n_rows * p.hkv), dim3(256), 0, s, p);
    return (int)hipGetLastError();
}

}  // namespace

bool supported_shape(int head_dim, int group) {
    if (head_dim == 64) return group == 1 || group == 2 || group == 4 || group == 8;
    if (head_dim == 128) return group == 1 || group == 2 || group == 4;
    return false;
}

#define PKV_DISPATCH(FN, D_, G_, ...)                                           \
    do {                                                                        \
        if (D_ == 128) {                                                        \
            if (G_ == 1) return FN<128, 1>(__VA_ARGS__);                        \
            if (G_ == 2) return FN<128, 2>(__VA_ARGS__);                        \
            if (G_ == 4) return FN<128, 4>(__VA_ARGS__);                        \
        } else if (D_ == 64) {                                                  \
            if (G_ == 1) return FN<64, 1>(__VA_ARGS__);                         \
            if (G_ == 2) return FN<64, 2>(__VA_ARGS__);                         \
            if (G_ == 4) return FN<64, 4>(__VA_ARGS__);                         \
            if (G_ == 8) return FN<64, 8>(__VA_ARGS__);                         \
        }                                                                       \
        return (int)hipErrorInvalidValue;                                       \
    } while (0)

int launch_init_ctrl(Ctrl* ctrl, uint32_t* arrive, int n_arrive, void* stream) {
    hipLaunchKernelGGL(init_ctrl_kernel, dim3(64), dim3(256), 0, (hipStream_t)stream, ctrl, arrive, n_arrive);
    return (int)hipGetLastError();
}

int launch_copy_probe(void* dst, const void* src, size_t bytes, int grid, void* stream) {
    hipLaunchKernelGGL(copy_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), bytes / 16);
    return (int)hipGetLastError();
}

int launch_read_probe(const void* src, size_t bytes, void* sink, int grid, void* stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
    return (int)hipGetLastError();
}

__global__ void zero_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

int launch_zero(void* p, size_t bytes, void* stream) {
    hipLaunchKernelGGL(zero_kernel, dim3(256), dim3(256), 0, (hipStream_t)stream,
                       static_cast<uint32_t*>(p), bytes / 4);
    return (int)hipGetLastError();
}

template <int D, int G>
int launch_resident_t(const LoopParams& lp, int kv_dtype, int grid, hipStream_t s) {
    if (kv_dtype == PKV_KV_F32)
        hipLaunchKernelGGL((resident_kernel<D, G, KvF32>), dim3(grid), dim3(kThreads), 0, s, lp);
    else
        hipLaunchKernelGGL((resident_kernel<D, G, KvBf16>), dim3(grid), dim3(kThreads), 0, s, lp);
    return (int)hipGetLastError();
}

int launch_resident(const LoopParams& lp, int head_dim, int group, int kv_dtype, int grid, void* stream) {
    PKV_DISPATCH(launch_resident_t, head_dim, group, lp, kv_dtype, grid, (hipStream_t)stream);
}

template <int D, int G>
int resident_occupancy_t(int kv_dtype, int* blocks) {
    *blocks = 0;
    hipError_t e = kv_dtype == PKV_KV_F32
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, resident_kernel<D, G, KvF32>, kThreads, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, resident_kernel<D, G, KvBf16>, kThreads, 0);
    return (int)e;
}

int resident_occupancy(int head_dim, int group, int kv_dtype, int* blocks) {
    PKV_DISPATCH(resident_occupancy_t, head_dim, group, kv_dtype, blocks);
}

int launch_decode(const DecodeParams& p, int head_dim, int group, int kv_dtype, int grid, void* stream) {
    PKV_DISPATCH(launch_decode_t, head_dim, group, p, kv_dtype, grid, (hipStream_t)stream);
}

int launch_merge(const DecodeParams& p, int head_dim, int group, int n_rows, void* stream) {
    PKV_DISPATCH(launch_merge_t, head_dim, group, p, n_rows, (hipStream_t)stream);
}

int launch_build_queue(const BuildParams& p, void* stream) {
    if (p.batch > kBuildMaxRows) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(build_queue_kernel, dim3(1), dim3(kBuildThreads), 0, (hipStream_t)stream, p);
    return (int)hipGetLastError();
}

template <int D>
void launch_debug_gather_t(const DecodeParams& p, int kv_dtype, int item_index, char* k_out, char* v_out,
                           hipStream_t s) {
    if (kv_dtype == PKV_KV_F32)
        hipLaunchKernelGGL((debug_gather_kernel<D, KvF32>), dim3(1), dim3(64), 0, s, p, item_index, k_out, v_out);
    else
        hipLaunchKernelGGL((debug_gather_kernel<D, KvBf16>), dim3(1), dim3(64), 0, s, p, item_index, k_out, v_out);
}

int launch_debug_gather(const DecodeParams& p, int head_dim, int kv_dtype, int item_index, void* k_out,
                        void* v_out, void* stream) {
    char* ko = static_cast<char*>(k_out);
    char* vo = static_cast<char*>(v_out);
    if (head_dim == 128)
        launch_debug_gather_t<128>(p, kv_dtype, item_index, ko, vo, (hipStream_t)stream);
    else if (head_dim == 64)
        launch_debug_gather_t<64>(p, kv_dtype, item_index, ko, vo, (hipStream_t)stream);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace pkv
