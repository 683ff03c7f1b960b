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
//   * pages are software-pipelined two ahead in registers (three tiles), so
//     each wave keeps up to 16 KB of K/V loads in flight;
//   * at the end of an item the 8 groups of a wave combine by xor shuffles and
//     the 8 waves combine through LDS.
#include <float.h>
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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

// Per-lane share of one page of K and V: two token rows (8*j + r, j = 0, 1)
// times D/64 pieces of 8 dims (piece 8*k + p of the row).
template <int D>
struct Tile {
    static constexpr int NPC = D / 64;
    u32x4 k[2][NPC];
    u32x4 v[2][NPC];
};

// Byte offsets of the lane's two token rows inside a (page, head) slab.  Rows
// at or beyond `valid` are never read: their lanes re-read row 0 of the same
// page (always a valid token) and the consumer masks them.
struct LaneOff {
    uint32_t o0, o1;
};

template <int D>
__device__ __forceinline__ LaneOff lane_offsets(int r, int p, int valid) {
    const int t0 = r < valid ? r : 0;
    const int t1 = 8 + r < valid ? 8 + r : 0;
    return {(uint32_t)(t0 * D * 2 + p * 16), (uint32_t)(t1 * D * 2 + p * 16)};
}

// Streaming 16-byte load with the non-temporal hint: K/V pages are read
// once per call, so they should not displace anything in L2 or the
// last-level cache (measured on MI355X: random 4 KB K+V slabs stream at
// about 6.7 TB/s with the hint against about 6.0 TB/s without).
__device__ __forceinline__ u32x4 ld_stream(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// The gather of one page: ks / vs are the wave-uniform slab addresses, the
// lane adds its 32-bit row offset; piece k sits 128 bytes further on.
template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& t, const char* ks, const char* vs, LaneOff o) {
#pragma unroll
    for (int k = 0; k < Tile<D>::NPC; ++k) {
        t.k[0][k] = ld_stream(ks + o.o0 + 128 * k);
        t.k[1][k] = ld_stream(ks + o.o1 + 128 * k);
        t.v[0][k] = ld_stream(vs + o.o0 + 128 * k);
        t.v[1][k] = ld_stream(vs + o.o1 + 128 * k);
    }
}

template <int D, int G>
struct State {
    float m[G];
    float l[G];
    float acc[G][D / 8];
};

template <int D, int G, bool MASKED>
__device__ __forceinline__ void consume_tile(const Tile<D>& t, const u32x4 (&qv)[G][D / 64],
                                             State<D, G>& st, float c, int r, int valid) {
    constexpr int NPC = D / 64;
    float s[2][G];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float a = 0.0f;
#pragma unroll
            for (int k = 0; k < NPC; ++k) {
                a = dot2(t.k[j][k].x, qv[g][k].x, a);
                a = dot2(t.k[j][k].y, qv[g][k].y, a);
                a = dot2(t.k[j][k].z, qv[g][k].z, a);
                a = dot2(t.k[j][k].w, qv[g][k].w, a);
            }
            s[j][g] = sum8(a) * c;
        }
    }
    u32x4 v[2][NPC];
#pragma unroll
    for (int k = 0; k < NPC; ++k) { v[0][k] = t.v[0][k]; v[1][k] = t.v[1][k]; }
    if (MASKED) {                                 // the last, partial page of a row
        const bool ok0 = r < valid, ok1 = 8 + r < valid;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (!ok0) s[0][g] = -INFINITY;
            if (!ok1) s[1][g] = -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < NPC; ++k) {
            if (!ok0) v[0][k] = u32x4{0u, 0u, 0u, 0u};
            if (!ok1) v[1][k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float mx[G];
    bool need = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mx[g] = fmaxf(s[0][g], s[1][g]);
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
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float p0 = __builtin_amdgcn_exp2f(s[0][g] - st.m[g]);
        const float p1 = __builtin_amdgcn_exp2f(s[1][g] - st.m[g]);
        st.l[g] += p0 + p1;
#pragma unroll
        for (int k = 0; k < NPC; ++k) {
            const uint32_t a0[4] = {v[0][k].x, v[0][k].y, v[0][k].z, v[0][k].w};
            const uint32_t a1[4] = {v[1][k].x, v[1][k].y, v[1][k].z, v[1][k].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                float& lo = st.acc[g][k * 8 + 2 * w];
                float& hi = st.acc[g][k * 8 + 2 * w + 1];
                lo = fmaf(p1, bf16_lo(a1[w]), fmaf(p0, bf16_lo(a0[w]), lo));
                hi = fmaf(p1, bf16_hi(a1[w]), fmaf(p0, bf16_hi(a0[w]), hi));
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
// wave's page list (item page w + 8 i).  Loads run ahead of the page being
// consumed; past the end the prefetch re-reads the last full page (a cache
// hit) so that every iteration issues the same loads and the wait counts the
// compiler derives stay exact.  btv holds the window's validated page ids.
template <int D, int G>
__device__ __forceinline__ void run_window(const DecodeParams& P, const u32x4 (&qv)[G][D / 64],
                                           State<D, G>& st, int32_t btv, int n, int wb,
                                           const WaveItem& wi, int r, int p) {
    constexpr uint64_t kSlabBytes = (uint64_t)kPageSize * D * 2;
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
    // loop so that the loop issues full-page loads with loop-invariant lane
    // offsets (no per-page VGPR temporaries competing with in-flight tiles).
    int vlast;
    const uint64_t slast = page_of(n - 1, vlast);
    const int nf = vlast < kPageSize ? n - 1 : n;               // full pages in the window
    const LaneOff full = lane_offsets<D>(r, p, kPageSize);
    auto issue = [&](Tile<D>& T, int ii) {
        int unused;
        const uint64_t so = page_of(ii < nf ? ii : nf - 1, unused);
        LaneOff o = full;
        // Keep the lane offset a 32-bit VGPR inside the loop so the loads use
        // the scalar-base + 32-bit-offset form (no 64-bit per-lane address math).
        __asm__ volatile("" : "+v"(o.o0), "+v"(o.o1));
        load_tile<D>(T, kbase + so, vbase + so, o);
    };
    // The loop is rotated so that every iteration first consumes a tile and
    // then refills the registers it just freed: no instruction at the loop
    // head writes a register that a load may still be filling.
    if (nf > 0) {
        if constexpr (PipelineDepth<D, G>::value == 2) {     // three tiles, two pages ahead
            Tile<D> A, B, C;
            issue(A, 0);
            issue(B, 1);
            issue(C, 2);
            for (int ii = 0;; ii += 3) {
                consume_tile<D, G, false>(A, qv, st, c, r, kPageSize);
                if (ii + 1 >= nf) break;
                issue(A, ii + 3);
                consume_tile<D, G, false>(B, qv, st, c, r, kPageSize);
                if (ii + 2 >= nf) break;
                issue(B, ii + 4);
                consume_tile<D, G, false>(C, qv, st, c, r, kPageSize);
                if (ii + 3 >= nf) break;
                issue(C, ii + 5);
            }
        } else {                                              // two tiles, one page ahead
            Tile<D> A, B;
            issue(A, 0);
            issue(B, 1);
            for (int ii = 0;; ii += 2) {
                consume_tile<D, G, false>(A, qv, st, c, r, kPageSize);
                if (ii + 1 >= nf) break;
                issue(A, ii + 2);
                consume_tile<D, G, false>(B, qv, st, c, r, kPageSize);
                if (ii + 2 >= nf) break;
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
        Tile<D> T;
        load_tile<D>(T, kbase + slast, vbase + slast, lane_offsets<D>(r, p, vlast));
        consume_tile<D, G, true>(T, qv, st, c, r, vlast);
    }
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

// Exact merge of the partial states of one split (row, KV head) (PersistentKV
// page, Methodology 1, "Sequence Splitting"): with M = max_c lse_c and
// w_c = exp(lse_c - M), O = sum_c w_c o_c / sum_c w_c and
// LSE = M + ln sum_c w_c.  A row with no ranges gets O = 0, LSE = -inf.
// Ranges are read 32 at a time, all loads of a block issued together; blocks
// after the first fold in by rescaling (the same identity, applied twice).
template <int D, int G, int NT, bool COHERENT>
__device__ void merge_row(const DecodeParams& P, int b, int hk, int nc, int base, int tid) {
    constexpr int CB = 32;
    for (int t = tid; t < G * D; t += NT) {
        const int g = t / D, d = t % D;
        const size_t h = (size_t)hk * G + g;
        float M = -INFINITY, L = 0.0f, O = 0.0f;
        for (int c0 = 0; c0 < nc; c0 += CB) {
            float lv[CB], ov[CB];
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                lv[j] = -INFINITY;
                ov[j] = 0.0f;
                if (c0 + j < nc) {
                    const size_t s = ((size_t)(base + c0 + j) * P.hkv + hk) * G + g;
                    lv[j] = ld_partial<COHERENT>(P.partial_lse + s);
                    ov[j] = ld_partial<COHERENT>(P.partial_o + s * D + d);
                }
            }
            float Mb = -INFINITY;
#pragma unroll
            for (int j = 0; j < CB; ++j) Mb = fmaxf(Mb, lv[j]);
            if (Mb == -INFINITY) continue;
            const float Mn = fmaxf(M, Mb);
            const float a = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
            L *= a;
            O *= a;
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const float wgt = lv[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((lv[j] - Mn) * kLog2e);
                L += wgt;
                O = fmaf(wgt, ov[j], O);
            }
            M = Mn;
        }
        const bool any = L > 0.0f;
        P.out[((size_t)b * P.hq + h) * D + d] = f32_to_bf16_rne(any ? O / L : 0.0f);
        if (d == 0) P.lse[(size_t)b * P.hq + h] = any ? M + logf(L) : -INFINITY;
    }
}

// Claim the next item for this workgroup: the grid's first round is static
// (workgroup i runs item i), later items are popped from the shared head.
__device__ __forceinline__ uint32_t pop_next(const DecodeParams& P) {
    return gridDim.x + atomicAdd(&P.ctrl->head, 1u);
}

template <int D, int G>
__device__ void process_item(const DecodeParams& P, Smem<D, G>& sm, uint32_t idx, uint32_t& nxt) {
    constexpr int NPC = D / 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane >> 3;
    const int p = lane & 7;

    const Item* itp = P.items + idx;
    const int b = __builtin_amdgcn_readfirstlane((int)itp->seq);
    const int hk = __builtin_amdgcn_readfirstlane((int)itp->kv_head);
    const int chunk = __builtin_amdgcn_readfirstlane((int)itp->chunk);
    const uint32_t tb = (uint32_t)__builtin_amdgcn_readfirstlane((int)itp->tok_begin);
    const uint32_t te = (uint32_t)__builtin_amdgcn_readfirstlane((int)itp->tok_end);
    const bool bad = b < 0 || b >= P.batch || hk >= P.hkv || tb >= te ||
                     te > (uint32_t)P.max_tokens || (tb % kPageSize) != 0;
    if (bad) {                                     // uniform over the workgroup
        if (tid == 0) {
            report(P.ctrl, P.host_error, PKV_DEVERR_BAD_ITEM, idx);
            nxt = pop_next(P);
        }
        return;
    }
    const int n_pages = (int)((te - tb + kPageSize - 1) / kPageSize);
    const int first_page = (int)(tb / kPageSize);
    const int nw = n_pages > w ? (n_pages - w + kWaves - 1) / kWaves : 0;

    u32x4 qv[G][NPC];
    const uint16_t* qrow = P.q + ((size_t)b * P.hq + (size_t)hk * G) * D;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < NPC; ++k)
            qv[g][k] = *reinterpret_cast<const u32x4*>(qrow + g * D + (8 * k + p) * 8);

    State<D, G> st;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        st.m[g] = kNegBig;
        st.l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < D / 8; ++e) st.acc[g][e] = 0.0f;
    }

    const WaveItem wi{tb, te, w, hk};
    const int32_t* bt_row = P.block_table + (size_t)b * P.bt_stride + first_page + w;
    for (int wb = 0; wb < nw; wb += 64) {
        const int n = nw - wb < 64 ? nw - wb : 64;
        int32_t btv = lane < n ? bt_row[(size_t)kWaves * (wb + lane)] : 0;
        const bool badl = lane < n && (uint32_t)btv >= (uint32_t)P.num_pages;
        const unsigned long long badm = __ballot(badl);
        if (badm) {                                   // never read outside the pool
            if (lane == __ffsll(badm) - 1) report(P.ctrl, P.host_error, PKV_DEVERR_PAGE_OOB, (uint32_t)btv);
            btv = badl ? 0 : btv;
        }
        run_window<D, G>(P, qv, st, btv, n, wb, wi, r, p);
    }
    // Claim the next item only now, near the end of this one: a claim made
    // earlier would hold an item this workgroup cannot start while another
    // workgroup runs dry.  Its latency hides behind the combine below.
    if (tid == 0) nxt = pop_next(P);

    // Combine the 8 token groups of this wave (lanes r = 0..7 with equal p).
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float M = st.m[g];
        M = fmaxf(M, __shfl_xor(M, 8));
        M = fmaxf(M, __shfl_xor(M, 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float a = __builtin_amdgcn_exp2f(st.m[g] - M);
        float l = st.l[g] * a;
        l += __shfl_xor(l, 8);
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
#pragma unroll
        for (int e = 0; e < D / 8; ++e) {
            float x = st.acc[g][e] * a;
            x += __shfl_xor(x, 8);
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            st.acc[g][e] = x;
        }
        st.m[g] = M;
        st.l[g] = l;
    }
    if (r == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int k = 0; k < NPC; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.acc[w][g * D + (8 * k + p) * 8 + e] = st.acc[g][k * 8 + e];
            if (p == 0) { sm.m[w][g] = st.m[g]; sm.l[w][g] = st.l[g]; }
        }
    }
    __syncthreads();

    const int nch = P.n_chunks[b];
    const bool split = nch > 1;
    const int base = split ? P.part_off[b] : 0;
    const int slot = split ? (base + chunk) * P.hkv + hk : 0;
    if (split && (chunk >= nch || slot < 0 || (base + nch) * P.hkv > P.max_items)) {
        if (tid == 0) report(P.ctrl, P.host_error, PKV_DEVERR_BAD_ITEM, idx);
        return;                                    // uniform over the workgroup (next already claimed)
    }
    for (int t = tid; t < G * D; t += kThreads) {
        const int g = t / D, d = t % D;
        float M = kNegBig;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][g]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float a = __builtin_amdgcn_exp2f(sm.m[ww][g] - M);
            L = fmaf(sm.l[ww][g], a, L);
            O = fmaf(sm.acc[ww][t], a, O);
        }
        O = O / L;
        const float lse = (M + log2f(L)) * kLn2;
        if (split) {
            if (P.fused_merge) {
                st_partial<true>(P.partial_o + ((size_t)slot * G + g) * D + d, O);
                if (d == 0) st_partial<true>(P.partial_lse + (size_t)slot * G + g, lse);
            } else {
                P.partial_o[((size_t)slot * G + g) * D + d] = O;
                if (d == 0) P.partial_lse[(size_t)slot * G + g] = lse;
            }
        } else {
            const size_t h = (size_t)hk * G + g;
            P.out[((size_t)b * P.hq + h) * D + d] = f32_to_bf16_rne(O);
            if (d == 0) P.lse[(size_t)b * P.hq + h] = lse;
        }
    }
    if (split && P.fused_merge) {
        // Last arriver of this (row, KV head) merges all its ranges.  Each
        // thread waits until its coherent partial stores have completed
        // (s_waitcnt vmcnt(0)), the workgroup then counts itself in with one
        // atomic, and the workgroup that completes the count reads every
        // partial with coherent loads issued after it saw the count.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = atomicAdd(&P.arrive[(size_t)b * P.hkv + hk], 1u);
            sm.last = (old + 1 == (uint32_t)nch) ? 1u : 0u;
        }
        __syncthreads();
        if (sm.last) {
            merge_row<D, G, kThreads, true>(P, b, hk, nch, base, tid);
            if (tid == 0) atomicExch(&P.arrive[(size_t)b * P.hkv + hk], 0u);
        }
    }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams P) {
    __shared__ Smem<D, G> sm;
    const int tid = threadIdx.x;
    Ctrl* ctrl = P.ctrl;
    const uint32_t n_items = (uint32_t)P.qhdr->n_items;
    const uint64_t t_enter = P.trace ? wall_clock64() : 0;
    if (P.fused_merge) {                 // rows with no tokens take the neutral state
        const int n_rows = P.qhdr->n_merge_rows;
        for (int ri = blockIdx.x; ri < n_rows; ri += gridDim.x) {
            const int b = P.merge_rows[ri];
            if (b < 0 || b >= P.batch || P.n_chunks[b] != 0) continue;
            for (int t = tid; t < P.hq * D; t += kThreads) {
                P.out[(size_t)b * P.hq * D + t] = 0;
                if (t % D == 0) P.lse[(size_t)b * P.hq + t / D] = -INFINITY;
            }
        }
    }
    uint32_t idx = blockIdx.x;                     // first round: static assignment
    uint32_t done_here = 0;
    if (P.trace && tid == 0 && n_items + blockIdx.x < (uint32_t)P.trace_cap) {
        // workgroup record after the item records: entry time, first pop returned
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
        process_item<D, G>(P, sm, idx, nxt);
        ++done_here;
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
    if (tid == 0) {
        // Thread 0's last pop has returned before this point, so when the
        // done count completes no workgroup can pop again: re-arm the head.
        if (done_here) atomicAdd(&ctrl->items_done, done_here);
        const uint32_t prev = atomicAdd(&ctrl->done, 1u);
        if (prev == gridDim.x - 1) {                        // last workgroup out re-arms
            atomicExch(&ctrl->head, 0u);
            atomicExch(&ctrl->done, 0u);
            atomicAdd(&ctrl->decode_calls, 1u);
        }
    }
}

// The separate merge kernel: one workgroup per (merge row, KV head).
template <int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams P) {
    const int n_rows = P.qhdr->n_merge_rows;
    const int ri = blockIdx.x / P.hkv;
    const int hk = blockIdx.x % P.hkv;
    if (ri >= n_rows) return;
    const int b = P.merge_rows[ri];
    if (b < 0 || b >= P.batch) return;
    const int nc = P.n_chunks[b];
    if (nc == 1 || (P.part_off[b] + nc) * P.hkv > P.max_items) return;
    merge_row<D, G, 256, false>(P, b, hk, nc, P.part_off[b], threadIdx.x);
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
    bool split;
    if (P.policy == PKV_POLICY_NO_SPLIT) split = false;
    else if (P.policy == PKV_POLICY_SPLIT) split = true;
    else split = B > 0 && (long long)B * P.hkv < P.num_cus && s_max > P.chunk;

    auto nchunks = [&](int L) -> int {
        if (L <= 0) return 0;
        return split ? (L + P.chunk - 1) / P.chunk : 1;
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
        else if (t == 3) val = P.chunk;
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
        it.tok_begin = split ? (uint32_t)(c * P.chunk) : 0u;
        const long long e = split ? (long long)(c + 1) * P.chunk : (long long)L;
        it.tok_end = (uint32_t)(e < L ? e : L);
        P.items[i] = it;
    }
}

// Test hook: one wave runs the decode kernel's own gather over every page of
// one item, in order, and stores the rows it read.
template <int D>
__global__ __launch_bounds__(64) void debug_gather_kernel(DecodeParams P, int item_index,
                                                          uint16_t* k_out, uint16_t* v_out) {
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
        Tile<D> t;
        const uint64_t slab = ((uint64_t)(uint32_t)pg * P.hkv + it.kv_head) * kPageSize * D * 2;
        load_tile<D>(t, reinterpret_cast<const char*>(P.k_pool) + slab,
                     reinterpret_cast<const char*>(P.v_pool) + slab, lane_offsets<D>(r, p, valid));
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int tok = 8 * jj + r;
            if (tok >= valid) continue;
            const size_t row = (size_t)(j * kPageSize + tok) * D;
#pragma unroll
            for (int k = 0; k < Tile<D>::NPC; ++k) {
                *reinterpret_cast<u32x4*>(k_out + row + (8 * k + p) * 8) = t.k[jj][k];
                *reinterpret_cast<u32x4*>(v_out + row + (8 * k + p) * 8) = t.v[jj][k];
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
    uint32_t* w = reinterpret_cast<uint32_t*>(c);
    if (blockIdx.x == 0 && threadIdx.x < sizeof(Ctrl) / 4) w[threadIdx.x] = 0u;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_arrive; i += gridDim.x * blockDim.x)
        arrive[i] = 0u;
}

template <int D, int G>
int launch_decode_t(const DecodeParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((decode_kernel<D, G>), dim3(grid), dim3(kThreads), 0, s, p);
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

int launch_decode(const DecodeParams& p, int head_dim, int group, int grid, void* stream) {
    PKV_DISPATCH(launch_decode_t, head_dim, group, p, grid, (hipStream_t)stream);
}

int launch_merge(const DecodeParams& p, int head_dim, int group, int n_rows, void* stream) {
    PKV_DISPATCH(launch_merge_t, head_dim, group, p, n_rows, (hipStream_t)stream);
}

int launch_build_queue(const BuildParams& p, void* stream) {
    if (p.batch > kBuildMaxRows) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(build_queue_kernel, dim3(1), dim3(kBuildThreads), 0, (hipStream_t)stream, p);
    return (int)hipGetLastError();
}

int launch_debug_gather(const DecodeParams& p, int head_dim, int item_index, uint16_t* k_out,
                        uint16_t* v_out, void* stream) {
    if (head_dim == 128)
        hipLaunchKernelGGL((debug_gather_kernel<128>), dim3(1), dim3(64), 0, (hipStream_t)stream, p,
                           item_index, k_out, v_out);
    else if (head_dim == 64)
        hipLaunchKernelGGL((debug_gather_kernel<64>), dim3(1), dim3(64), 0, (hipStream_t)stream, p,
                           item_index, k_out, v_out);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace pkv
