// Internal definitions shared by the host library (pkv_api.cpp,
// queue_plan.cpp) and the gfx950 kernels (pkv_kernels.hip).
#pragma once

#include <stddef.h>
#include <cstddef>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

constexpr int kPageSize = 16;          // tokens per page (the only size built)
constexpr int kThreads = 512;          // 8 waves of 64 lanes per workgroup
constexpr int kWaves = kThreads / 64;
// Chunk mode "fit": shortest range in pages.  One-shot launches take ranges
// down to 16 pages (measured: the shortest ranges that still give one item
// per workgroup are the fastest); the resident loop keeps 64 (measured: its
// layers wait on each other's merges, and 32- or 48-page ranges stepped no
// faster).
constexpr int kFitMinPages = 16;
constexpr int kFitMinPagesLoop = 64;
// CUs that the default queue capacity of chunk mode "fit" covers on any
// device (more when the config names more)
constexpr int kFitCuSlots = 1024;
constexpr int kCursorStride = 32;      // u32 words between page cursors (one 128-byte line each)
constexpr int kSinkBytes = 4096;       // >= the largest tile (16 rows x 128 bf16, 8 rows x 128 fp32)

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

// Control words at the start of the workspace (device memory).  One-shot
// launches alternate between two pop counters: launch k pops from
// head[k & 1] and zeroes head[(k + 1) & 1], which the next launch uses (the
// launches of a handle run one after another), so no launch has to count its
// workgroups out to re-arm its counter.
struct Ctrl {
    uint32_t head[2];       // pop counters of alternate one-shot launches
    uint32_t error_code;    // PKV_DEVERR_*
    uint32_t error_detail;
    uint32_t decode_calls;  // one-shot decode launches
    uint32_t pad[59];
};
static_assert(sizeof(Ctrl) == 256, "ctrl is 256 bytes");
// Items run by one-shot launches, counted as each starts in kDoneLines
// counters one 128-byte line apart (workgroup g adds to counter
// g mod kDoneLines), right after Ctrl, so that the adds of many workgroups
// never queue on one address.  The host sums the counters.
constexpr int kDoneLines = 64;
constexpr uint64_t kCtrlBytes = sizeof(Ctrl) + (uint64_t)kDoneLines * 128;

// Queue header, first bytes of the queue region.
struct QHdr {
    int32_t n_items;
    int32_t n_merge_rows;
    int32_t split;
    int32_t chunk_tokens;
    int32_t batch;
    int32_t uniform;        // 1: every item has the same number of tokens
    int32_t pad[58];
};
static_assert(sizeof(QHdr) == 256, "queue header is 256 bytes");

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Resident-loop control record, in fine-grained (coherent) host memory.
// The host writes in_epoch / exit_flag; the device writes the rest.  The two
// directions sit in different 64-byte lines.
struct LoopCtrl {
    uint32_t in_epoch;          // step the host has published
    uint32_t exit_flag;         // 1: leave the loop
    uint32_t pad0[14];
    uint32_t out_epoch;         // last step the device completed
    uint32_t alive;             // 1 while the resident kernel runs
    uint32_t exit_reason;       // 0 running, 1 exit flag seen, 2 idle timeout, 3 wait timeout
    uint32_t heartbeat;         // steps started
    uint32_t pad1[12];
};
static_assert(sizeof(LoopCtrl) == 128, "loop ctrl is two 64-byte lines");

// Per-step descriptor at the start of each host queue slot.
struct LoopDesc {
    const uint16_t* q;
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    const int32_t* block_table;
    uint16_t* out;
    float* lse;
    int64_t ls_q, ls_kv, ls_bt, ls_out, ls_lse;   // layer strides, elements
    int32_t batch;
    int32_t bt_stride;
    int32_t n_layers;
    uint32_t epoch;
    const uint16_t* new_k;      // append: newest token's K / V, [B][Hkv][D] per layer
    const uint16_t* new_v;
    int64_t ls_new;
    int32_t pad[32];
};
static_assert(sizeof(LoopDesc) == 256, "loop descriptor is 256 bytes");
static_assert(offsetof(LoopDesc, batch) == 88 && offsetof(LoopDesc, bt_stride) == 92 &&
              offsetof(LoopDesc, n_layers) == 96 && offsetof(LoopDesc, new_k) == 104 &&
              offsetof(LoopDesc, ls_new) == 120, "loop descriptor words read as 64-bit pairs");
static_assert(offsetof(QHdr, n_merge_rows) == 4, "queue header words read as one 64-bit pair");

// Device-memory mirror of the host control words, written by workgroup 0
// (the only workgroup that polls host memory) and polled by the others.
struct LoopGlobal {
    uint32_t dev_epoch;         // last step workgroup 0 saw published
    uint32_t dev_exit;          // nonzero: leave the loop (1 exit flag, 2 idle limit)
    uint32_t pad[62];
};

// Device-memory counters of one slot of the resident loop.
// A slot serves steps e, e + 2, ...; it is re-armed only after every
// workgroup has checked out of step e (finished popping from it), and
// workgroup 0 opens it for step e + 2 only after that re-arm.
struct LoopSlotCtr {
    uint32_t head;              // pop counter
    uint32_t pad0[31];
    uint32_t step_done;         // completed work units of the step
    uint32_t pad1[31];
    uint32_t checkout;          // workgroups done with the step
    uint32_t retired;           // last step whose use of the slot has ended
    uint32_t pad2[62];
    // followed by uint32 done[max_batch]: completed items per row
};
static_assert(sizeof(LoopSlotCtr) == 512, "LoopSlotCtr layout");

// Resolved configuration: defaults filled in, checked.
struct Resolved {
    int hq, hkv, g, d, page, num_pages, max_batch, max_pages_per_seq;
    float scale;
    int policy, order, chunk, num_cus, max_items, wg_per_cu, merge_mode;
    int persistent, num_layers, timeout_ms, schedule, append, kv_dtype;
    int fit_min_pages;          // kFitMinPages, or kFitMinPagesLoop for the resident loop
};

pkv_status resolve_config(const pkv_config* cfg, int device_cus, Resolved* r, const char** why);
void compute_layout(const Resolved& r, pkv_layout* lay);
uint64_t loop_counter_bytes(const Resolved& r);
// Words of the arrival region: [layers][max_batch][Hkv] row counters, then
// [layers][max_items] group counters of the two-level merge.
uint64_t arrive_words(const Resolved& r);
uint64_t loop_slot_bytes(const Resolved& r, const pkv_layout& lay);
uint64_t loop_grant_bytes(const Resolved& r);      // append page grants in a slot, after LoopDesc

// Host queue planner.  Writes the queue header, n_chunks, part_off, merge_rows
// and items into the caller's arrays.  Returns PKV_OK or an error.
pkv_status plan_queue(const Resolved& r, const int32_t* ctx_lens, int32_t batch, QHdr* qh,
                      int32_t* n_chunks, int32_t* part_off, int32_t* merge_rows, Item* items,
                      int32_t items_cap, pkv_queue_info* info, const char** why,
                      int32_t* row_len = nullptr);

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
    uint32_t* grp_arrive;       // two-level merge: [max_items] group counters, at the slot of the group's first range
    uint64_t* trace;            // per-item trace records (nullable)
    uint32_t* head;             // pop counter of this queue
    uint32_t* head_next;        // one-shot: the next launch's pop counter, zeroed at the start (nullable)
    uint32_t* done_lines;       // one-shot: items-run counters (kDoneLines, 32 words apart; nullable)
    int32_t trace_cap;
    int32_t head_dim;
    int32_t coherent_out;       // 1: outputs stored system-coherently (resident loop)
    int32_t static_first;       // 1: first round static (one-shot), 0: all pops (resident loop)
    int32_t coherent_in;        // 1: q and block-table entries read with coherent loads
    uint32_t* host_error;       // mapped host word mirrored on device faults (nullable)
    int32_t batch;
    int32_t bt_stride;
    int32_t num_pages;
    int32_t hq;
    int32_t hkv;
    int32_t max_tokens;         // max_pages_per_seq * page size
    int32_t max_items;          // capacity of items and partial slots
    int32_t fused_merge;        // 1: last arriver merges inside the decode kernel
    int32_t static_sched;       // 1: workgroup g runs items g, g + grid, ... (no claims)
    float scale_log2;           // scale * log2(e)
    const char* sink;           // kSinkBytes the look-ahead reads past a window's end
    const int32_t* row_len;     // [batch] tokens per row (the queue's copy of ctx_lens)
    uint32_t* cursors;          // page-claim and steal schedules: [max_batch][Hkv] cursors, kCursorStride apart
                                // (null: split items read their own token range)
    int32_t steal;              // 1: the first pages of every split item go to its row's shared pool
};

// Resident-loop kernel parameters: the per-step constant part of the decode
// parameters plus where the control record, the host queue slots and the
// loop counters live.
struct LoopParams {
    DecodeParams base;          // ctrl, partials, arrive, head_dim, hq, hkv, ...
    LoopCtrl* lctrl;            // device view of the host control record
    unsigned char* slots;       // device view of the two host queue slots
    uint64_t slot_bytes;
    uint64_t q_hdr_off, q_nch_off, q_poff_off, q_mrows_off, q_items_off;  // within a slot
    uint64_t grant_off;         // append: int32 [max_batch] page grants within a slot
    int32_t append;             // 1: write each row's newest token before attention
    LoopGlobal* lglobal;        // device mirror of the control words
    unsigned char* mirror;      // device copies of the two host slots (same layout)
    unsigned char* counters;    // LoopSlotCtr + done[max_batch], two slots
    uint64_t counter_bytes;     // per slot
    uint64_t partial_o_layer;   // elements per layer of partial_o
    uint64_t partial_lse_layer;
    uint64_t arrive_layer;
    uint64_t grp_layer;         // group counters per layer (max_items)
    uint64_t timeout_ticks;     // 100 MHz wall-clock ticks
    int32_t max_batch;
};

struct BuildParams {
    const int32_t* ctx_lens;
    QHdr* qhdr;
    int32_t* n_chunks;
    int32_t* part_off;
    int32_t* row_len;
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
    int32_t fit_min_pages;
};

// Kernel parameters over a workspace laid out by compute_layout (pkv_api.cpp).
// A roctx range around a C-ABI call (seen by rocprofv3 --marker-trace);
// defined in pkv_api.cpp.
struct ApiRange {
    explicit ApiRange(const char* name);
    ~ApiRange();
    ApiRange(const ApiRange&) = delete;
    ApiRange& operator=(const ApiRange&) = delete;
};

DecodeParams decode_params(const Resolved& r, const pkv_layout& lay, unsigned char* ws, const pkv_tensors* t,
                           uint32_t* host_error);
BuildParams build_params(const Resolved& r, const pkv_layout& lay, unsigned char* ws, const int32_t* ctx_lens,
                         int32_t batch, uint32_t* host_error);
// Validation of the caller's tensors against a config; PKV_OK or an error with *why.
pkv_status check_tensor_args(const Resolved& r, const pkv_tensors* t, const char** why);

// Launch wrappers (pkv_kernels.hip).  Return a hipError_t as int.
int launch_init_ctrl(Ctrl* ctrl, uint32_t* arrive, int n_arrive, void* stream);
int launch_zero(void* p, size_t bytes, void* stream);
int launch_decode(const DecodeParams& p, int head_dim, int group, int kv_dtype, int grid, void* stream);
int launch_merge(const DecodeParams& p, int head_dim, int group, int n_rows, void* stream);
int launch_build_queue(const BuildParams& p, void* stream);
int launch_debug_gather(const DecodeParams& p, int head_dim, int kv_dtype, int item_index, void* k_out,
                        void* v_out, void* stream);
bool supported_shape(int head_dim, int group);
int launch_copy_probe(void* dst, const void* src, size_t bytes, int grid, void* stream);
int launch_read_probe(const void* src, size_t bytes, void* sink, int grid, void* stream);
int launch_resident(const LoopParams& lp, int head_dim, int group, int kv_dtype, int grid, void* stream);
// Workgroups of the resident kernel that fit on one CU at once (registers, LDS, waves).
int resident_occupancy(int head_dim, int group, int kv_dtype, int* blocks);

}  // namespace pkv
