// Internal definitions shared by the host library (pkv_api.cpp,
// queue_plan.cpp) and the gfx950 kernels (pkv_kernels.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

constexpr int kPageSize = 16;          // tokens per page (the only size built)
constexpr int kThreads = 512;          // 8 waves of 64 lanes per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kDefaultChunk = 4096;

// One queue item: a non-empty token range [tok_begin, tok_end) of one
// (sequence, KV head).  16 bytes, little-endian.
struct Item {
    uint32_t seq;
    uint16_t kv_head;
    uint16_t chunk;
    uint32_t tok_begin;
    uint32_t tok_end;
};
static_assert(sizeof(Item) == 16, "item is 16 bytes");

// Control words at the start of the workspace (device memory).
struct Ctrl {
    uint32_t head;          // next item to pop; reset to 0 by the last workgroup out
    uint32_t done;          // workgroups finished in the current launch
    uint32_t error_code;    // PKV_DEVERR_*
    uint32_t error_detail;
    uint32_t items_done;
    uint32_t decode_calls;
    uint32_t pad[58];
};
static_assert(sizeof(Ctrl) == 256, "ctrl is 256 bytes");

// Queue header, first bytes of the queue region.
struct QHdr {
    int32_t n_items;
    int32_t n_merge_rows;
    int32_t split;
    int32_t chunk_tokens;
    int32_t batch;
    int32_t pad[59];
};
static_assert(sizeof(QHdr) == 256, "queue header is 256 bytes");

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Resolved configuration: defaults filled in, checked.
struct Resolved {
    int hq, hkv, g, d, page, num_pages, max_batch, max_pages_per_seq;
    float scale;
    int policy, order, chunk, num_cus, max_items, wg_per_cu, merge_mode;
};

pkv_status resolve_config(const pkv_config* cfg, int device_cus, Resolved* r, const char** why);
void compute_layout(const Resolved& r, pkv_layout* lay);

// Host queue planner.  Writes the queue header, n_chunks, part_off, merge_rows
// and items into the caller's arrays.  Returns PKV_OK or an error.
pkv_status plan_queue(const Resolved& r, const int32_t* ctx_lens, int32_t batch, QHdr* qh,
                      int32_t* n_chunks, int32_t* part_off, int32_t* merge_rows, Item* items,
                      int32_t items_cap, pkv_queue_info* info, const char** why);

// Kernel parameters (passed by value).
struct DecodeParams {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* block_table;
    uint16_t* out;
    float* lse;
    Ctrl* ctrl;
    const QHdr* qhdr;
    const int32_t* n_chunks;
    const int32_t* part_off;
    const int32_t* merge_rows;
    const Item* items;
    float* partial_o;
    float* partial_lse;
    uint32_t* arrive;           // [max_batch][Hkv] arrival counters (fused merge)
    uint64_t* trace;            // per-item trace records (nullable)
    int32_t trace_cap;
    uint32_t* host_error;       // mapped host word mirrored on device faults (nullable)
    int32_t batch;
    int32_t bt_stride;
    int32_t num_pages;
    int32_t hq;
    int32_t hkv;
    int32_t max_tokens;         // max_pages_per_seq * page size
    int32_t max_items;          // capacity of items and partial slots
    int32_t fused_merge;        // 1: last arriver merges inside the decode kernel
    float scale_log2;           // scale * log2(e)
};

struct BuildParams {
    const int32_t* ctx_lens;
    QHdr* qhdr;
    int32_t* n_chunks;
    int32_t* part_off;
    int32_t* merge_rows;
    Item* items;
    Ctrl* ctrl;
    uint32_t* host_error;
    int32_t batch;
    int32_t hkv;
    int32_t num_cus;
    int32_t chunk;
    int32_t policy;
    int32_t max_items;
    int32_t max_tokens;
};

// Launch wrappers (pkv_kernels.hip).  Return a hipError_t as int.
int launch_init_ctrl(Ctrl* ctrl, uint32_t* arrive, int n_arrive, void* stream);
int launch_decode(const DecodeParams& p, int head_dim, int group, int grid, void* stream);
int launch_merge(const DecodeParams& p, int head_dim, int group, int n_rows, void* stream);
int launch_build_queue(const BuildParams& p, void* stream);
int launch_debug_gather(const DecodeParams& p, int head_dim, int item_index, uint16_t* k_out,
                        uint16_t* v_out, void* stream);
bool supported_shape(int head_dim, int group);
int launch_copy_probe(void* dst, const void* src, size_t bytes, int grid, void* stream);
int launch_read_probe(const void* src, size_t bytes, void* sink, int grid, void* stream);

}  // namespace pkv
