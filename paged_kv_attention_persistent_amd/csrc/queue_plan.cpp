// Host side of the work queue: configuration defaults, workspace layout, and
// the adaptive split policy plus compact queue builder.
//
// Policy and queue follow the PersistentKV page ("PersistentKV: Page-Aware
// Decode Scheduling for Long-Context LLM Serving on Commodity GPUs",
// Technical Summary): Methodology 1 "Row-Local Bounds" (ranges follow each
// row's true length), "Compact Workqueue" (tasks only for non-empty
// row / KV-head / split intervals) and Methodology 2 "Calibrated Adaptive
// Policy" (split when too few rows exist to fill the GPU, otherwise one task
// per row and head).  The page's third-party route does not exist here and
// becomes the no-split route; the threshold is the occupancy rule
// B * Hkv < CUs with some row longer than one range.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "pkv_internal.h"

namespace pkv {

namespace {

// Environment overrides of a few config fields, for experiments without
// rebuilding the caller: PKV_POLICY (auto | split | nosplit),
// PKV_CHUNK_TOKENS (kv_chunk_tokens), PKV_WG_PER_CU (wg_per_cu) and
// PKV_SCHEDULE (atomic | static | pages | steal).  An empty variable is
// unset; a value that does not parse is refused naming the variable (the
// overridden fields are then checked like any config).
bool env_int(const char* name, int32_t* out, const char** why) {
    const char* v = getenv(name);
    if (!v || !*v) return true;
    char* end = nullptr;
    const long x = strtol(v, &end, 10);
    if (*end || x < INT32_MIN || x > INT32_MAX) { *why = name; return false; }
    *out = (int32_t)x;
    return true;
}

bool env_choice(const char* name, const char* const* names, int n, int32_t* out, const char** why) {
    const char* v = getenv(name);
    if (!v || !*v) return true;
    for (int i = 0; i < n; ++i)
        if (!strcmp(v, names[i])) { *out = i; return true; }
    *why = name;
    return false;
}

pkv_status apply_env(pkv_config* c, const char** why) {
    static const char* const policies[] = {"auto", "nosplit", "split"};      // PKV_POLICY_* order
    static const char* const schedules[] = {"atomic", "static", "pages", "steal"};
    const char* bad = nullptr;
    if (!env_choice("PKV_POLICY", policies, 3, &c->policy, &bad) ||
        !env_int("PKV_CHUNK_TOKENS", &c->kv_chunk_tokens, &bad) ||
        !env_int("PKV_WG_PER_CU", &c->wg_per_cu, &bad) ||
        !env_choice("PKV_SCHEDULE", schedules, 4, &c->schedule, &bad)) {
        *why = !strcmp(bad, "PKV_POLICY") ? "PKV_POLICY must be auto, split or nosplit"
             : !strcmp(bad, "PKV_SCHEDULE") ? "PKV_SCHEDULE must be atomic, static, pages or steal"
             : !strcmp(bad, "PKV_CHUNK_TOKENS") ? "PKV_CHUNK_TOKENS is not an integer"
                                                : "PKV_WG_PER_CU is not an integer";
        return PKV_ERR_INVALID_ARG;
    }
    return PKV_OK;
}

}  // namespace

pkv_status resolve_config(const pkv_config* user_cfg, int device_cus, Resolved* r, const char** why) {
    *why = "";
    if (!user_cfg || !r) { *why = "null config"; return PKV_ERR_INVALID_ARG; }
    if (user_cfg->struct_size != sizeof(pkv_config)) { *why = "pkv_config.struct_size mismatch"; return PKV_ERR_INVALID_ARG; }
    pkv_config env_cfg = *user_cfg;
    if (apply_env(&env_cfg, why) != PKV_OK) return PKV_ERR_INVALID_ARG;
    const pkv_config* cfg = &env_cfg;
    for (int i = 0; i < 2; ++i)
        if (cfg->reserved[i]) { *why = "reserved config fields must be zero"; return PKV_ERR_INVALID_ARG; }
    if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 || cfg->num_q_heads % cfg->num_kv_heads) {
        *why = "num_q_heads must be a positive multiple of num_kv_heads"; return PKV_ERR_INVALID_ARG;
    }
    if (cfg->num_kv_heads > 65535) { *why = "num_kv_heads exceeds 65535"; return PKV_ERR_UNSUPPORTED; }
    r->hq = cfg->num_q_heads;
    r->hkv = cfg->num_kv_heads;
    r->g = r->hq / r->hkv;
    if (!(r->g == 1 || r->g == 2 || r->g == 4 || r->g == 8)) { *why = "group size must be 1, 2, 4 or 8"; return PKV_ERR_UNSUPPORTED; }
    if (!(cfg->head_dim == 64 || cfg->head_dim == 128)) { *why = "head_dim must be 64 or 128"; return PKV_ERR_UNSUPPORTED; }
    r->d = cfg->head_dim;
    if (r->d == 128 && r->g == 8) { *why = "group size 8 is built for head_dim 64 only"; return PKV_ERR_UNSUPPORTED; }
    if (cfg->page_size != kPageSize) { *why = "page_size must be 16"; return PKV_ERR_UNSUPPORTED; }
    r->page = kPageSize;
    if (cfg->num_pages <= 0 || cfg->max_batch <= 0 || cfg->max_pages_per_seq <= 0) {
        *why = "num_pages, max_batch and max_pages_per_seq must be positive"; return PKV_ERR_INVALID_ARG;
    }
    if ((int64_t)cfg->max_pages_per_seq * kPageSize > INT32_MAX) { *why = "max_pages_per_seq too large"; return PKV_ERR_CAPACITY; }
    r->num_pages = cfg->num_pages;
    r->max_batch = cfg->max_batch;
    r->max_pages_per_seq = cfg->max_pages_per_seq;
    if (!isfinite(cfg->scale)) { *why = "scale must be finite"; return PKV_ERR_INVALID_ARG; }
    r->scale = cfg->scale == 0.0f ? 1.0f / sqrtf((float)r->d) : cfg->scale;
    if (cfg->policy < PKV_POLICY_AUTO || cfg->policy > PKV_POLICY_SPLIT) { *why = "unknown policy"; return PKV_ERR_INVALID_ARG; }
    r->policy = cfg->policy;
    if (cfg->order != PKV_ORDER_CANONICAL && cfg->order != PKV_ORDER_LPT) { *why = "unknown order"; return PKV_ERR_INVALID_ARG; }
    r->order = cfg->order;
    r->chunk = cfg->kv_chunk_tokens;                  // 0: chunk mode "fit", chosen per call
    if (r->chunk < 0 || r->chunk % kPageSize) { *why = "kv_chunk_tokens must be 0 or a positive multiple of 16"; return PKV_ERR_INVALID_ARG; }
    r->num_cus = cfg->num_cus > 0 ? cfg->num_cus : device_cus;
    if (r->num_cus <= 0) { *why = "num_cus unknown (set it in the config)"; return PKV_ERR_INVALID_ARG; }
    const int64_t max_tokens = (int64_t)r->max_pages_per_seq * kPageSize;
    r->fit_min_pages = cfg->persistent ? kFitMinPagesLoop : kFitMinPages;
    // Default capacity.  Fixed C-token chunks: Hkv * max_batch * ceil(max_tokens / C).
    // Chunk mode "fit": a queue that does not split holds one item per
    // (row, KV head); a split queue holds at most max(1, CUs / Hkv) ranges per
    // KV head when some range length T reaches that budget (the floor only
    // lengthens ranges), else one range per row.  Hence at most
    // max(Hkv * max_batch, CUs) items, with the CU term taken as
    // max(kFitCuSlots, CUs) so that the layout is the same on every device of
    // up to kFitCuSlots CUs.
    const int64_t max_chunks = r->chunk ? (max_tokens + r->chunk - 1) / r->chunk : 1;
    if (max_chunks > 65535) { *why = "more than 65535 ranges per row"; return PKV_ERR_CAPACITY; }
    if (cfg->max_items < 0) { *why = "max_items must be >= 0"; return PKV_ERR_INVALID_ARG; }
    if (cfg->max_items > 0) {
        r->max_items = cfg->max_items;
    } else {
        int64_t bound = (int64_t)r->hkv * r->max_batch * max_chunks;
        if (!r->chunk) bound = std::max<int64_t>(bound, std::max(kFitCuSlots, r->num_cus));
        if (bound > (int64_t)1 << 28) { *why = "derived max_items too large; set max_items"; return PKV_ERR_CAPACITY; }
        r->max_items = (int)bound;
    }
    r->wg_per_cu = cfg->wg_per_cu == 0 ? 1 : cfg->wg_per_cu;
    if (r->wg_per_cu < 1 || r->wg_per_cu > 8) { *why = "wg_per_cu must be 1..8"; return PKV_ERR_INVALID_ARG; }
    if (cfg->merge_mode != PKV_MERGE_FUSED && cfg->merge_mode != PKV_MERGE_SEPARATE) {
        *why = "unknown merge_mode"; return PKV_ERR_INVALID_ARG;
    }
    r->merge_mode = cfg->merge_mode;
    if (cfg->persistent != 0 && cfg->persistent != 1) { *why = "persistent must be 0 or 1"; return PKV_ERR_INVALID_ARG; }
    r->persistent = cfg->persistent;
    r->num_layers = cfg->num_layers == 0 ? 1 : cfg->num_layers;
    if (r->num_layers < 1 || r->num_layers > 1024) { *why = "num_layers must be 1..1024"; return PKV_ERR_INVALID_ARG; }
    if (!r->persistent && r->num_layers != 1) { *why = "num_layers > 1 needs the resident loop"; return PKV_ERR_INVALID_ARG; }
    r->timeout_ms = cfg->timeout_ms == 0 ? 10000 : cfg->timeout_ms;
    if (r->timeout_ms < 1 || r->timeout_ms > 3600000) { *why = "timeout_ms must be 1..3600000"; return PKV_ERR_INVALID_ARG; }
    if (r->persistent && r->wg_per_cu != 1) { *why = "the resident loop runs one workgroup per CU"; return PKV_ERR_INVALID_ARG; }
    if (cfg->schedule != PKV_SCHEDULE_ATOMIC && cfg->schedule != PKV_SCHEDULE_STATIC &&
        cfg->schedule != PKV_SCHEDULE_PAGES && cfg->schedule != PKV_SCHEDULE_STEAL) {
        *why = "unknown schedule"; return PKV_ERR_INVALID_ARG;
    }
    if (r->persistent && cfg->schedule != PKV_SCHEDULE_ATOMIC) { *why = "the resident loop claims items atomically"; return PKV_ERR_INVALID_ARG; }
    r->schedule = cfg->schedule;
    if (cfg->append != 0 && cfg->append != 1) { *why = "append must be 0 or 1"; return PKV_ERR_INVALID_ARG; }
    if (cfg->append && !r->persistent) { *why = "append needs the resident loop"; return PKV_ERR_INVALID_ARG; }
    r->append = cfg->append;
    if (cfg->kv_dtype != PKV_KV_BF16 && cfg->kv_dtype != PKV_KV_F32) { *why = "unknown kv_dtype"; return PKV_ERR_INVALID_ARG; }
    r->kv_dtype = cfg->kv_dtype;
    if ((int64_t)r->max_items * r->num_layers > ((int64_t)1 << 31) / (4 * r->g * r->d)) {
        *why = "partial-state storage too large"; return PKV_ERR_CAPACITY;
    }
    return PKV_OK;
}

uint64_t loop_grant_bytes(const Resolved& r) { return align256(4ull * r.max_batch); }

uint64_t loop_slot_bytes(const Resolved& r, const pkv_layout& lay) {
    return align256(sizeof(LoopDesc) + loop_grant_bytes(r) + (lay.items_off - lay.queue_off) +
                    16ull * r.max_items);
}

uint64_t arrive_words(const Resolved& r) {
    return ((uint64_t)r.max_batch * r.hkv + (uint64_t)r.max_items) * r.num_layers;
}

uint64_t loop_counter_bytes(const Resolved& r) {
    return align256(sizeof(LoopSlotCtr) + 4ull * r.max_batch);
}

void compute_layout(const Resolved& r, pkv_layout* lay) {
    memset(lay, 0, sizeof(*lay));
    uint64_t off = 0;
    lay->ctrl_off = off;
    off = align256(off + kCtrlBytes);
    lay->queue_off = off;
    off = align256(off + sizeof(QHdr));
    lay->n_chunks_off = off;
    off = align256(off + 4ull * r.max_batch);
    lay->part_off_off = off;
    off = align256(off + 4ull * (r.max_batch + 1));
    lay->row_len_off = off;
    off = align256(off + 4ull * r.max_batch);
    lay->merge_rows_off = off;
    off = align256(off + 4ull * r.max_batch);
    lay->items_off = off;
    off = align256(off + 16ull * r.max_items);
    const uint64_t layers = (uint64_t)r.num_layers;
    lay->partial_o_off = off;
    off = align256(off + 4ull * r.max_items * r.g * r.d * layers);
    lay->partial_lse_off = off;
    off = align256(off + 4ull * r.max_items * r.g * layers);
    lay->arrive_off = off;
    off = align256(off + 4ull * arrive_words(r));
    lay->cursor_off = off;
    // one cursor per (row, KV head), or per (row, KV head, wave) for the steal schedule
    if (r.schedule == PKV_SCHEDULE_PAGES) off = align256(off + 4ull * kCursorStride * r.max_batch * r.hkv);
    if (r.schedule == PKV_SCHEDULE_STEAL) off = align256(off + 4ull * kCursorStride * r.max_batch * r.hkv * kWaves);
    lay->loop_off = off;
    if (r.persistent) off = align256(off + sizeof(LoopGlobal) + 2ull * loop_counter_bytes(r));
    lay->loop_mirror_off = off;
    if (r.persistent) off = align256(off + 2ull * loop_slot_bytes(r, *lay));
    lay->sink_off = off;
    off = align256(off + kSinkBytes);
    lay->total_bytes = off;
    lay->max_items = r.max_items;
}

// Chunk mode "fit": the smallest T pages with sum_b ceil(pages_b / T) <= K,
// K = max(1, CUs / Hkv), so that the split queue still has at most one range
// per workgroup; the longest row's page count when no T reaches K; and never
// below r.fit_min_pages.  The count falls as T grows, so a bisection finds the
// smallest T.
int fit_chunk(const Resolved& r, const int32_t* ctx_lens, int batch, int64_t max_len) {
    const int64_t budget = std::max(1, r.num_cus / r.hkv);
    const int64_t longest = (max_len + r.page - 1) / r.page;
    auto ranges = [&](int64_t T) {
        int64_t n = 0;
        for (int b = 0; b < batch; ++b) {
            const int64_t pages = ((int64_t)ctx_lens[b] + r.page - 1) / r.page;
            n += (pages + T - 1) / T;
        }
        return n;
    };
    int64_t T = std::max<int64_t>(longest, 1);
    if (longest > 0 && ranges(longest) <= budget) {
        int64_t lo = 1, hi = longest;                // ranges(hi) <= budget holds
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (ranges(mid) <= budget) hi = mid; else lo = mid + 1;
        }
        T = lo;
    }
    return (int)(std::max<int64_t>(T, r.fit_min_pages) * r.page);
}

pkv_status plan_queue(const Resolved& r, const int32_t* ctx_lens, int32_t batch, QHdr* qh,
                      int32_t* n_chunks, int32_t* part_off, int32_t* merge_rows, Item* items,
                      int32_t items_cap, pkv_queue_info* info, const char** why, int32_t* row_len) {
    *why = "";
    if (batch < 0 || batch > r.max_batch) { *why = "batch outside [0, max_batch]"; return PKV_ERR_CAPACITY; }
    if (batch > 0 && !ctx_lens) { *why = "null ctx_lens"; return PKV_ERR_INVALID_ARG; }
    const int64_t max_tokens = (int64_t)r.max_pages_per_seq * r.page;
    int64_t max_len = 0, sum_len = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t L = ctx_lens[b];
        if (L < 0) { *why = "negative context length"; return PKV_ERR_INVALID_ARG; }
        if (L > max_tokens) { *why = "context length exceeds max_pages_per_seq * page_size"; return PKV_ERR_CAPACITY; }
        max_len = std::max(max_len, L);
        sum_len += L;
    }
    const int chunk = r.chunk ? r.chunk : fit_chunk(r, ctx_lens, batch, max_len);
    bool split;
    if (r.policy == PKV_POLICY_NO_SPLIT) split = false;
    else if (r.policy == PKV_POLICY_SPLIT) split = true;
    else split = batch > 0 && (int64_t)batch * r.hkv < r.num_cus && max_len > chunk;

    int64_t n_items = 0;
    int n_split_rows = 0, n_merge = 0;
    part_off[0] = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t L = ctx_lens[b];
        const int64_t nc64 = L == 0 ? 0 : (split ? (L + chunk - 1) / chunk : 1);
        if (nc64 > 65535) { *why = "a row needs more than 65535 ranges (16-bit range index)"; return PKV_ERR_CAPACITY; }
        const int32_t nc = (int32_t)nc64;
        n_chunks[b] = nc;
        if (row_len) row_len[b] = (int32_t)L;
        part_off[b + 1] = part_off[b] + (nc > 1 ? nc : 0);
        n_items += (int64_t)nc * r.hkv;
        if (nc > 1) ++n_split_rows;
        if (nc != 1) merge_rows[n_merge++] = b;
    }
    if (n_items > items_cap) { *why = "queue exceeds max_items"; return PKV_ERR_CAPACITY; }

    int64_t k = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t L = ctx_lens[b];
        for (int h = 0; h < r.hkv; ++h) {
            for (int c = 0; c < n_chunks[b]; ++c) {
                Item it;
                it.seq = (uint32_t)b;
                it.kv_head = (uint16_t)h;
                it.chunk = (uint16_t)c;
                it.tok_begin = split ? (uint32_t)((int64_t)c * chunk) : 0u;
                it.tok_end = split ? (uint32_t)std::min<int64_t>(L, (int64_t)(c + 1) * chunk) : (uint32_t)L;
                items[k++] = it;
            }
        }
    }
    if (r.order == PKV_ORDER_LPT) {
        std::stable_sort(items, items + n_items, [](const Item& a, const Item& b) {
            return (a.tok_end - a.tok_begin) > (b.tok_end - b.tok_begin);
        });
    }
    memset(qh, 0, sizeof(*qh));
    qh->n_items = (int32_t)n_items;
    qh->n_merge_rows = n_merge;
    qh->split = split ? 1 : 0;
    qh->chunk_tokens = chunk;
    qh->batch = batch;
    qh->uniform = n_items > 0 ? 1 : 0;
    for (int64_t i = 1; i < n_items && qh->uniform; ++i)
        if (items[i].tok_end - items[i].tok_begin != items[0].tok_end - items[0].tok_begin) qh->uniform = 0;
    if (info) {
        memset(info, 0, sizeof(*info));
        info->n_items = (int32_t)n_items;
        info->split = split ? 1 : 0;
        info->chunk_tokens = chunk;
        info->n_split_rows = n_split_rows;
        info->n_merge_rows = n_merge;
        info->n_partial_slots = part_off[batch] * r.hkv;
        info->launches_per_step = 1 + ((r.merge_mode == PKV_MERGE_SEPARATE && n_merge > 0) ? 1 : 0);
        info->kv_bytes = (uint64_t)sum_len * r.hkv * r.d * (r.kv_dtype == PKV_KV_F32 ? 4ull : 2ull) * 2ull;
        info->partial_bytes = (uint64_t)info->n_partial_slots * r.g * (r.d + 1) * 4ull * 2ull;
    }
    return PKV_OK;
}

}  // namespace pkv
