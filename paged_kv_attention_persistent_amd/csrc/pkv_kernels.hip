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
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
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

// Element offset of lane (r, p)'s piece k of token row `tok` in a slab.
template <int D>
__device__ __forceinline__ int piece_off(int tok, int k, int p) {
    return tok * D + (8 * k + p) * 8;
}

// The gather: load the lane's share of page `pg` (slab of KV head hk).  Rows
// at or beyond `valid` are not read: their lanes re-read row 0 of the same
// page (always a valid token) and the caller masks them.
template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& t, const uint16_t* __restrict__ kp,
                                          const uint16_t* __restrict__ vp, size_t slab, int r,
                                          int p, int valid) {
    const uint16_t* ks = kp + slab;
    const uint16_t* vs = vp + slab;
    const int t0 = (r < valid) ? r : 0;
    const int t1 = (8 + r < valid) ? 8 + r : 0;
#pragma unroll
    for (int k = 0; k < Tile<D>::NPC; ++k) {
        t.k[0][k] = *reinterpret_cast<const u32x4*>(ks + piece_off<D>(t0, k, p));
        t.k[1][k] = *reinterpret_cast<const u32x4*>(ks + piece_off<D>(t1, k, p));
        t.v[0][k] = *reinterpret_cast<const u32x4*>(vs + piece_off<D>(t0, k, p));
        t.v[1][k] = *reinterpret_cast<const u32x4*>(vs + piece_off<D>(t1, k, p));
    }
}

template <int D, int G>
struct State {
    float m[G];
    float l[G];
    float acc[G][D / 8];
};

template <int D, int G>
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
    if (valid < kPageSize) {                      // uniform: only the last page of a row
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

// One window of up to 64 of this wave's pages: i = wb .. wb + n - 1 of the
// wave's page list (item page w + 8 i).  Loads run two pages ahead; past the
// end the prefetch re-reads the window's last page (a cache hit) so that every
// iteration issues the same loads and the wait counts stay exact.
template <int D, int G>
__device__ __forceinline__ void run_window(const DecodeParams& P, const u32x4 (&qv)[G][D / 64],
                                           State<D, G>& st, int32_t btv, int n, int wb, int w,
                                           int hk, uint32_t tb, uint32_t te, int r, int p, int lane) {
    const size_t slab_elems = (size_t)kPageSize * D;
    auto page_of = [&](int ii, int& valid) -> size_t {
        int32_t pg = __builtin_amdgcn_readlane(btv, ii);
        if ((uint32_t)pg >= (uint32_t)P.num_pages) {
            if (lane == 0) report(P.ctrl, P.host_error, PKV_DEVERR_PAGE_OOB, (uint32_t)pg);
            pg = 0;
        }
        const int64_t tok0 = (int64_t)tb + (int64_t)(w + 8 * (wb + ii)) * kPageSize;
        const int64_t rem = (int64_t)te - tok0;
        valid = rem < kPageSize ? (int)rem : kPageSize;
        return ((size_t)pg * P.hkv + hk) * slab_elems;
    };
    const float c = P.scale_log2;
    auto clamp = [n](int ii) { return ii < n ? ii : n - 1; };
    if constexpr (PipelineDepth<D, G>::value == 2) {     // three tiles, two pages ahead
        Tile<D> A, B, C;
        int va, vb, vc;
        size_t sa = page_of(0, va);
        load_tile<D>(A, P.k_pool, P.v_pool, sa, r, p, va);
        size_t sb = page_of(clamp(1), vb);
        load_tile<D>(B, P.k_pool, P.v_pool, sb, r, p, vb);
        for (int ii = 0; ii < n; ii += 3) {
            size_t sc = page_of(clamp(ii + 2), vc);
            load_tile<D>(C, P.k_pool, P.v_pool, sc, r, p, vc);
            consume_tile<D, G>(A, qv, st, c, r, va);
            if (ii + 1 >= n) break;
            sa = page_of(clamp(ii + 3), va);
            load_tile<D>(A, P.k_pool, P.v_pool, sa, r, p, va);
            consume_tile<D, G>(B, qv, st, c, r, vb);
            if (ii + 2 >= n) break;
            sb = page_of(clamp(ii + 4), vb);
            load_tile<D>(B, P.k_pool, P.v_pool, sb, r, p, vb);
            consume_tile<D, G>(C, qv, st, c, r, vc);
        }
    } else {                                              // two tiles, one page ahead
        Tile<D> A, B;
        int va, vb;
        size_t sa = page_of(0, va);
        load_tile<D>(A, P.k_pool, P.v_pool, sa, r, p, va);
        for (int ii = 0; ii < n; ii += 2) {
            size_t sb = page_of(clamp(ii + 1), vb);
            load_tile<D>(B, P.k_pool, P.v_pool, sb, r, p, vb);
            consume_tile<D, G>(A, qv, st, c, r, va);
            if (ii + 1 >= n) break;
            sa = page_of(clamp(ii + 2), va);
            load_tile<D>(A, P.k_pool, P.v_pool, sa, r, p, va);
            consume_tile<D, G>(B, qv, st, c, r, vb);
        }
    }
}

template <int D, int G>
struct Smem {
    float acc[kWaves][G * D];
    float m[kWaves][G];
    float l[kWaves][G];
    uint32_t next;
};

template <int D, int G>
__device__ void process_item(const DecodeParams& P, Smem<D, G>& sm, uint32_t idx) {
    constexpr int NPC = D / 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int r = lane >> 3;
    const int p = lane & 7;

    const Item it = P.items[idx];
    const int b = (int)it.seq;
    const int hk = (int)it.kv_head;
    const uint32_t tb = it.tok_begin, te = it.tok_end;
    const bool bad = b >= P.batch || hk >= P.hkv || tb >= te || te > (uint32_t)P.max_tokens ||
                     (tb % kPageSize) != 0;
    if (bad) {                                     // uniform over the workgroup
        if (tid == 0) report(P.ctrl, P.host_error, PKV_DEVERR_BAD_ITEM, idx);
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

    const int32_t* bt_row = P.block_table + (size_t)b * P.bt_stride + first_page + w;
    for (int wb = 0; wb < nw; wb += 64) {
        const int n = nw - wb < 64 ? nw - wb : 64;
        const int32_t btv = lane < n ? bt_row[(size_t)kWaves * (wb + lane)] : 0;
        run_window<D, G>(P, qv, st, btv, n, wb, w, hk, tb, te, r, p, lane);
    }

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
    const int slot = split ? (P.part_off[b] + (int)it.chunk) * P.hkv + hk : 0;
    if (split && ((int)it.chunk >= nch || slot < 0 || slot >= P.max_items)) {
        if (tid == 0) report(P.ctrl, P.host_error, PKV_DEVERR_BAD_ITEM, idx);
        return;                                    // uniform over the workgroup
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
            P.partial_o[((size_t)slot * G + g) * D + d] = O;
            if (d == 0) P.partial_lse[(size_t)slot * G + g] = lse;
        } else {
            const size_t h = (size_t)hk * G + g;
            P.out[((size_t)b * P.hq + h) * D + d] = f32_to_bf16_rne(O);
            if (d == 0) P.lse[(size_t)b * P.hq + h] = lse;
        }
    }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams P) {
    __shared__ Smem<D, G> sm;
    const int tid = threadIdx.x;
    Ctrl* ctrl = P.ctrl;
    const uint32_t n_items = (uint32_t)P.qhdr->n_items;
    if (tid == 0) sm.next = atomicAdd(&ctrl->head, 1u);
    __syncthreads();
    uint32_t idx = sm.next;
    uint32_t done_here = 0;
    while (idx < n_items) {
        uint32_t nxt = 0;
        if (tid == 0) nxt = atomicAdd(&ctrl->head, 1u);   // claim the next item early
        process_item<D, G>(P, sm, idx);
        ++done_here;
        __syncthreads();
        if (tid == 0) sm.next = nxt;
        __syncthreads();
        idx = sm.next;
    }
    if (tid == 0) {
        if (done_here) atomicAdd(&ctrl->items_done, done_here);
        __threadfence();
        const uint32_t prev = atomicAdd(&ctrl->done, 1u);
        if (prev == gridDim.x - 1) {                        // last workgroup out re-arms
            atomicExch(&ctrl->head, 0u);
            atomicExch(&ctrl->done, 0u);
            atomicAdd(&ctrl->decode_calls, 1u);
        }
    }
}

// Exact merge of split partial states (PersistentKV page, Methodology 1,
// "Sequence Splitting"): with M = max_c lse_c and w_c = exp(lse_c - M),
// O = sum_c w_c o_c / sum_c w_c and LSE = M + ln sum_c w_c.  Rows with no
// items (L = 0) receive the neutral state O = 0, LSE = -inf.
template <int D, int G>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams P) {
    const int n_rows = P.qhdr->n_merge_rows;
    const int ri = blockIdx.x / P.hkv;
    const int hk = blockIdx.x % P.hkv;
    if (ri >= n_rows) return;
    const int b = P.merge_rows[ri];
    const int nc = P.n_chunks[b];
    const int base = P.part_off[b];
    for (int t = threadIdx.x; t < G * D; t += 256) {
        const int g = t / D, d = t % D;
        const size_t h = (size_t)hk * G + g;
        float M = -INFINITY;
        for (int c = 0; c < nc; ++c)
            M = fmaxf(M, P.partial_lse[((size_t)(base + c) * P.hkv + hk) * G + g]);
        float O = 0.0f, L = 0.0f, lse = -INFINITY;
        if (M != -INFINITY) {
            for (int c = 0; c < nc; ++c) {
                const size_t s = ((size_t)(base + c) * P.hkv + hk) * G + g;
                const float l = P.partial_lse[s];
                const float wgt = l == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((l - M) * kLog2e);
                L += wgt;
                O = fmaf(wgt, P.partial_o[s * D + d], O);
            }
            O = O / L;
            lse = M + logf(L);
        }
        P.out[((size_t)b * P.hq + h) * D + d] = f32_to_bf16_rne(O);
        if (d == 0) P.lse[(size_t)b * P.hq + h] = lse;
    }
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
        load_tile<D>(t, P.k_pool, P.v_pool, ((size_t)pg * P.hkv + it.kv_head) * kPageSize * D, r, p, valid);
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

__global__ void init_ctrl_kernel(Ctrl* c) {
    uint32_t* w = reinterpret_cast<uint32_t*>(c);
    w[threadIdx.x] = 0u;
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

int launch_init_ctrl(Ctrl* ctrl, void* stream) {
    hipLaunchKernelGGL(init_ctrl_kernel, dim3(1), dim3(sizeof(Ctrl) / 4), 0, (hipStream_t)stream, ctrl);
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
