/*
 * pkv.h - C ABI of libpkv: decode attention over a block-table paged KV
 * cache, executed by a persistent kernel that drains a device work queue.
 * Target: AMD Instinct MI355X (gfx950, CDNA4), HIP runtime.
 *
 * What is computed (PersistentKV page, "PersistentKV: Page-Aware Decode
 * Scheduling for Long-Context LLM Serving on Commodity GPUs", Technical
 * Summary, Methodology 1 "Native Block-Table Decode Engine"): for every
 * sequence b and query head h, with G = Hq / Hkv and KV head floor(h / G),
 *     s_t   = scale * q[b][h] . K_t          t = 0 .. L_b - 1
 *     out   = sum_t softmax(s)_t V_t          (bf16, rounded to nearest even)
 *     lse   = ln sum_t exp(s_t)               (fp32, natural log)
 * where token t is read in place from page block_table[b][t / P], row
 * t % P (no repacking, "Layout"), only tokens below L_b are read ("Row-Local
 * Bounds"), and a row with L_b = 0 gets out = 0, lse = -inf (the neutral
 * state).  Long rows may be cut into disjoint ranges whose partial states a
 * separate merge kernel combines exactly ("Sequence Splitting"); the work
 * queue holds only non-empty (row, KV head, range) items ("Compact
 * Workqueue"); the split decision is the adaptive policy of Methodology 2
 * "Calibrated Adaptive Policy".  Workgroups pop items with one atomic each,
 * as the persistent executor on the GPUOS page pops tasks ("GPUOS: A GPU
 * Operating System Primitive for Transparent Operation Fusion", section 4.1).
 *
 * Data layout (all row-major, contiguous, 16-byte aligned device memory):
 *   q          bf16  [B][Hq][D]
 *   k_pool     bf16 or fp32 (pkv_config.kv_dtype) [num_pages][Hkv][P][D]
 *   v_pool     the same                    (one (page, head) slab of P*D
 *                                           values is contiguous)
 *   block_table int32 [B][block_table_stride]    entries past ceil(L_b/P)
 *                                                are ignored (may be -1)
 *   ctx_lens   int32 [B]
 *   out        bf16  [B][Hq][D]
 *   lse        fp32  [B][Hq]
 * Supported: page_size 16; head_dim 64 with G in {1, 2, 4, 8}; head_dim 128
 * with G in {1, 2, 4}.
 *
 * Ownership: the caller owns every device buffer, including the workspace
 * (size from pkv_workspace_size) and streams; the library never frees caller
 * memory.  The library itself allocates only host memory: the handle and a
 * small pinned staging area for queue uploads.  A handle is not thread-safe.
 *
 * Errors: every call returns a pkv_status; PKV_OK is 0 and every error is
 * negative.  A call that fails validation enqueues nothing.  A fault detected
 * on the device (a block-table entry outside [0, num_pages), a malformed
 * item) sets an error word in the workspace; the kernel then reads page 0
 * instead (so no access leaves the pool), and the next pkv_decode or
 * pkv_query returns PKV_ERR_DEVICE_FAULT with the word in
 * pkv_runtime_info.  pkv_last_error gives the text of the last failure.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_API __attribute__((visibility("default")))

typedef int32_t pkv_status;
enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misaligned buffer */
    PKV_ERR_UNSUPPORTED = -2,   /* head_dim / page_size / group size not built */
    PKV_ERR_CAPACITY = -3,      /* batch, items or pages exceed the config */
    PKV_ERR_HIP = -4,           /* HIP runtime error (text in pkv_last_error) */
    PKV_ERR_STATE = -5,         /* wrong call order (e.g. decode before build) */
    PKV_ERR_DEVICE_FAULT = -6,  /* device error word set (see pkv_runtime_info) */
    PKV_ERR_TIMEOUT = -7
};

/* Split policy (PersistentKV page, Methodology 2).  AUTO: cut rows into
 * C-token ranges iff B * Hkv < num_cus and some L_b exceeds C; otherwise one
 * item per (row, KV head).  C is kv_chunk_tokens, or with kv_chunk_tokens = 0
 * ("fit", the default) it is chosen per call as P * T with T the smallest
 * page count for which sum_b ceil(ceil(L_b / P) / T) <= max(1, num_cus / Hkv):
 * the shortest ranges that still give at most one item per workgroup (the
 * longest row's page count if the rows alone exceed that bound), and never
 * shorter than 16 pages (64 pages for the resident loop, persistent = 1).
 * Such a queue holds at most max(Hkv * max_batch, num_cus) items, and the
 * default max_items in this mode is max(Hkv * max_batch, num_cus, 1024), so
 * that the layout is the same for every num_cus up to 1024. */
enum { PKV_POLICY_AUTO = 0, PKV_POLICY_NO_SPLIT = 1, PKV_POLICY_SPLIT = 2 };

/* Queue order: CANONICAL = (seq, kv_head, chunk) ascending; LPT = stable sort
 * of the canonical list by item length, longest first. */
enum { PKV_ORDER_CANONICAL = 0, PKV_ORDER_LPT = 1 };

/* Item-to-workgroup assignment in one-shot launches.  ATOMIC (default): the
 * PersistentKV page's work queue -- workgroup g runs item g first, then claims
 * further items with an atomic counter as it finishes (no claims at all when
 * the queue has no more items than workgroups: the first round covers it;
 * and a host-built queue of items of one length in whole rounds of the grid
 * runs round-robin as under STATIC, since claims could not change how much
 * each workgroup runs).
 * Consecutive launches of a handle use two such counters in turn, each
 * launch clearing the other's for the next.  STATIC: the WPK note's
 * compiled schedule -- workgroup g runs items g, g + grid, g + 2 grid, ...
 * with no claims.  Every item is computed the same way in both, so outputs
 * are identical; only the time differs (a scheduling ablation).  PAGES: items
 * are claimed as in ATOMIC, but the workgroups of a split (row, KV head) no
 * longer read fixed token ranges: their waves claim groups of pages (6 tiles,
 * 48 KiB of K+V at D = 128) from a cursor shared by the row's items, so
 * faster workgroups take more of the row; each item still yields one partial
 * state and the merge is the same exact merge (over disjoint page sets).
 * Outputs agree with the other schedules to rounding, not bit for bit.
 * STEAL: items are claimed as in ATOMIC and each item of a split (row, KV
 * head) reads its own range, except the first quarter of every range
 * (rounded down to whole rounds of 8 waves x 3 pages, full pages only): those
 * pages form the row's shared pool, which the waves of the row's items drain
 * 3 pages per claim once their own pages are done (wave w takes the pool
 * pages congruent to w modulo 8, from a cursor per (row, KV head, wave)), so
 * the row's items end close together whichever XCD runs them.  The pages are
 * still read once each and merged exactly; outputs agree with the other
 * schedules to rounding.  The PersistentKV page names work assignment as a
 * deciding variable beside the attention arithmetic (Technical Summary,
 * "Significance and Claims"); these schedules are measured as an ablation.  The resident loop always claims
 * items (ATOMIC). */
enum { PKV_SCHEDULE_ATOMIC = 0, PKV_SCHEDULE_STATIC = 1, PKV_SCHEDULE_PAGES = 2, PKV_SCHEDULE_STEAL = 3 };

/* Element type of the KV cache.  BF16: 2-byte values.  F32: 4-byte values,
 * as in the fp32 attention cache of the text-to-speech model on the WPK note
 * ("Same precision" list); the same kernels read twice the bytes per token,
 * q.K and P.V run in fp32 on the full-precision values (q stays bf16, widened
 * exactly).  q, out and lse keep their types.  One-shot launches and the
 * resident loop (with or without append) take either. */
enum { PKV_KV_BF16 = 0, PKV_KV_F32 = 1 };

/* How split rows are merged (the exact log-sum-exp merge of PersistentKV
 * page, Methodology 1, "Sequence Splitting").  FUSED: inside the decode
 * kernel, the last workgroup to finish a split (row, KV head) merges its
 * partial states (one launch per step); a row of more than 32 ranges merges
 * in two levels, each group of 32 consecutive ranges folded by its last
 * workgroup and the group states by the row's last group.  SEPARATE: a
 * second kernel merges every split row (the two-kernel split + merge
 * scheme), in the same two levels.  Both give the same bits. */
enum { PKV_MERGE_FUSED = 0, PKV_MERGE_SEPARATE = 1 };

/* Device error words (pkv_runtime_info.error_code). */
enum {
    PKV_DEVERR_NONE = 0,
    PKV_DEVERR_PAGE_OOB = 1,    /* block-table entry outside the pool; detail = entry */
    PKV_DEVERR_BAD_ITEM = 2     /* item fields out of range; detail = item index */
};

/* Environment overrides.  Wherever the library resolves a configuration
 * (pkv_workspace_size, pkv_workspace_layout, pkv_create, pkv_plan_queue,
 * pkv_decode_noalloc) these variables, when set and not empty, replace the
 * matching fields before validation, for experiments without rebuilding the
 * caller: PKV_POLICY = auto | split | nosplit (policy), PKV_CHUNK_TOKENS
 * (kv_chunk_tokens), PKV_WG_PER_CU (wg_per_cu), PKV_SCHEDULE = atomic |
 * static | pages | steal (schedule).  A value that does not parse gives
 * PKV_ERR_INVALID_ARG naming the variable; a parsed value is checked like
 * the field itself.  Set them the same for every call of one handle's
 * lifetime: the workspace size depends on them. */
typedef struct pkv_config {
    uint32_t struct_size;       /* sizeof(pkv_config): ABI version check */
    int32_t num_q_heads;        /* Hq */
    int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0 */
    int32_t head_dim;           /* D: 64 or 128 */
    int32_t page_size;          /* P: 16 */
    int32_t num_pages;          /* pages in each of k_pool / v_pool */
    int32_t max_batch;          /* largest B passed to pkv_build_queue */
    int32_t max_pages_per_seq;  /* longest row in pages (bounds L_b and items) */
    float scale;                /* 0 -> 1 / sqrt(D) */
    int32_t policy;             /* PKV_POLICY_* */
    int32_t order;              /* PKV_ORDER_* */
    int32_t kv_chunk_tokens;    /* split range length, a multiple of P; 0 -> fitted per call */
    int32_t num_cus;            /* policy input; 0 -> the device's CU count */
    int32_t max_items;          /* queue capacity; 0 -> bound from the shape */
    int32_t wg_per_cu;          /* persistent grid = CUs * wg_per_cu; 0 -> 1 */
    int32_t merge_mode;         /* PKV_MERGE_* */
    int32_t persistent;         /* 0: one launch per pkv_decode; 1: resident loop (below) */
    int32_t num_layers;         /* resident loop: layers per step (0 -> 1) */
    int32_t timeout_ms;         /* resident loop: wait limit, device and host (0 -> 10000) */
    int32_t schedule;           /* PKV_SCHEDULE_* (one-shot launches) */
    int32_t append;             /* resident loop: 1 -> each step first writes every session's
                                   newest token (K/V from pkv_tensors.new_k / new_v) into the
                                   cache, taking a page from the free list when the token
                                   opens a page (see pkv_loop_set_free_pages) */
    int32_t kv_dtype;           /* PKV_KV_*: element type of k_pool / v_pool */
    int32_t reserved[2];        /* must be zero */
} pkv_config;

typedef struct pkv_tensors {
    const void* q;              /* bf16 [B][Hq][D] */
    const void* k_pool;         /* kv_dtype [num_pages][Hkv][P][D] */
    const void* v_pool;         /* kv_dtype [num_pages][Hkv][P][D] */
    const int32_t* block_table; /* int32 [B][block_table_stride] */
    const int32_t* ctx_lens;    /* int32 [B] (device copy; used by the device
                                   queue builder) */
    void* out;                  /* bf16 [B][Hq][D] */
    float* lse;                 /* fp32 [B][Hq] */
    int32_t batch;              /* B: must equal the batch of the built queue */
    int32_t block_table_stride; /* elements per block-table row; 0 -> max_pages_per_seq */
    /* Resident loop with num_layers > 1: element distance between layer l and
     * l + 1 of q, of each pool, of the block table, of out and of lse (the
     * same queue serves every layer).  Ignored when num_layers is 1. */
    int64_t layer_stride_q, layer_stride_kv, layer_stride_bt, layer_stride_out, layer_stride_lse;
    /* Resident loop with append = 1: the K and V of each session's newest token
     * (token ctx_lens[b] - 1), kv_dtype [B][Hkv][D] per layer, layer l at
     * new_k + l * layer_stride_new elements (likewise new_v).  Null otherwise. */
    const void* new_k;
    const void* new_v;
    int64_t layer_stride_new;
} pkv_tensors;

typedef struct pkv_queue_info {
    int32_t n_items;            /* items in the compact queue */
    int32_t split;              /* policy decision: 1 = ranges of chunk_tokens */
    int32_t chunk_tokens;       /* range length used */
    int32_t n_split_rows;       /* rows with more than one range */
    int32_t n_merge_rows;       /* rows finished by the merge kernel (split or empty) */
    int32_t n_partial_slots;    /* partial states written by the decode kernel */
    int32_t launches_per_step;  /* kernels pkv_decode enqueues (1, or 2 with a separate merge) */
    int32_t reserved;
    uint64_t kv_bytes;          /* K+V bytes of valid tokens (algorithmic read volume) */
    uint64_t partial_bytes;     /* bytes of partial states written and re-read */
} pkv_queue_info;

typedef struct pkv_runtime_info {
    uint32_t error_code;        /* PKV_DEVERR_* */
    uint32_t error_detail;
    uint32_t queue_head;        /* next item index the kernel would pop (0 when idle) */
    uint32_t n_items;           /* items of the current queue */
    uint32_t items_done;        /* items run by one-shot decode launches since create,
                                   counted as each starts (wraps) */
    uint32_t decode_calls;      /* one-shot decode launches since create */
    int32_t grid;               /* persistent workgroups per decode launch */
    int32_t num_cus;            /* CUs of the device */
    uint32_t loop_out_epoch;    /* resident loop: last completed step (0 before the first) */
    uint32_t loop_alive;        /* resident loop: 1 while the kernel runs */
    uint32_t loop_exit_reason;  /* 0 running, 1 exit flag, 2 idle timeout, 3 wait timeout */
    uint32_t loop_steps_started;
} pkv_runtime_info;

/* Workspace regions (byte offsets into the caller's workspace), so that a
 * caller or test can inspect the queue and the partial states in place. */
typedef struct pkv_layout {
    uint64_t ctrl_off;          /* control words (queue head, error word, counters) */
    uint64_t queue_off;         /* queue header: int32 n_items, n_merge_rows, split,
                                   chunk_tokens, batch */
    uint64_t n_chunks_off;      /* int32 [max_batch] */
    uint64_t part_off_off;      /* int32 [max_batch + 1] */
    uint64_t row_len_off;       /* int32 [max_batch]: each row's length in tokens */
    uint64_t merge_rows_off;    /* int32 [max_batch] */
    uint64_t items_off;         /* 16-byte items [max_items]: u32 seq, u16 kv_head,
                                   u16 chunk, u32 tok_begin, u32 tok_end */
    uint64_t partial_o_off;     /* fp32 [layers][max_items][G][D], normalised partial outputs */
    uint64_t partial_lse_off;   /* fp32 [layers][max_items][G], natural-log partial LSE */
    uint64_t arrive_off;        /* uint32 [layers][max_batch][Hkv] arrival counters of the fused merge,
                                   then uint32 [layers][max_items] counters of its two-level form */
    uint64_t cursor_off;        /* PKV_SCHEDULE_PAGES: uint32 page cursors, one 128-byte line per
                                   (row, KV head); PKV_SCHEDULE_STEAL: one per (row, KV head,
                                   wave), 8 waves; empty otherwise */
    uint64_t loop_off;          /* resident loop: control mirror and two slots of step counters */
    uint64_t loop_mirror_off;   /* resident loop: device copies of the two host queue slots */
    uint64_t sink_off;          /* 4 KiB read by the gather's look-ahead past the end of a
                                   page window (the values are never used) */
    uint64_t total_bytes;
    int32_t max_items;
    int32_t reserved;
} pkv_layout;

typedef struct pkv_handle pkv_handle;

/* Bytes of device workspace a handle with this config needs (the caller
 * allocates it: GPUOS page, section 4.3).  PKV_ERR_UNSUPPORTED or
 * PKV_ERR_INVALID_ARG for a config pkv_create would refuse. */
PKV_API pkv_status pkv_workspace_size(const pkv_config* cfg, size_t* bytes);

/* Workspace layout of a config (pure host computation). */
PKV_API pkv_status pkv_workspace_layout(const pkv_config* cfg, pkv_layout* layout);

/* Resident loop (persistent = 1).  pkv_create launches one resident kernel on
 * `stream` (one workgroup per CU, for the handle's lifetime); no kernel is
 * launched per step after that.  Per step the caller runs pkv_build_queue
 * (host planning into a host-memory queue slot; two slots alternate) and
 * pkv_decode, which writes the step descriptor, publishes the step's epoch
 * with a release store to a control record in host memory, and blocks until
 * the kernel publishes the same epoch back (or the timeout: PKV_ERR_TIMEOUT).
 * The kernel drains the step's queue once per layer in layer order; layer
 * l + 1 of a row starts after every item of layer l of that row finished.
 * Outputs are stored system-coherently, so they are readable when pkv_decode
 * returns.  pkv_destroy raises the exit flag and waits for the kernel.  This
 * is the "publish the input, wait for the output" boundary of the Wave
 * Persistent Kernel note ("What a persistent kernel is", "Runtime and timing
 * boundary"); the host cannot run other kernels on the CUs meanwhile. */

/* Create a handle on the current HIP device: the runtime's initialisation
 * call, in the shape of the host API that sets up the persistent executor
 * and its queue on the GPUOS page ("GPUOS: A GPU Operating System Primitive
 * for Transparent Operation Fusion", section 4.3 and Table 1, the init
 * call), with memory that the framework already allocated (section 4.3,
 * "Memory Management and Safety").  workspace: device memory of at least
 * pkv_workspace_size bytes, 256-byte aligned, owned by the caller and kept
 * alive until pkv_destroy.  stream: hipStream_t used for queue uploads
 * (0 = the null stream).  Initialises the workspace's control words
 * (asynchronously on stream).  With persistent = 1 it also launches the
 * resident kernel; PKV_ERR_UNSUPPORTED if its grid (wg_per_cu workgroups
 * per CU) cannot be resident at once on this device.
 *
 * Streams.  One handle runs one piece of device work at a time.  The
 * library orders its own launches across streams with events: a queue
 * upload or device build waits for the previous decode (or gather) that read
 * the queue, and a decode waits for the queue's upload and for the previous
 * decode, whichever streams they ran on.  Calls on the handle's own stream
 * are ordered by the stream alone. */
PKV_API pkv_status pkv_create(const pkv_config* cfg, void* workspace, size_t workspace_bytes,
                              void* stream, pkv_handle** out);

/* Build the compact work queue on the host from host context lengths
 * (int32 [batch]) and enqueue its upload on the handle's stream: the queue
 * of tasks for non-empty (row, KV head, range) intervals of the PersistentKV
 * page ("PersistentKV: Page-Aware Decode Scheduling for Long-Context LLM
 * Serving on Commodity GPUs", Methodology 1 "Compact Workqueue"), with the
 * split decision of Methodology 2 "Calibrated Adaptive Policy" (pkv_config
 * policy above).  Returns after the upload is enqueued; info (nullable)
 * receives the counters.  Errors: PKV_ERR_CAPACITY if batch exceeds
 * max_batch, a length exceeds max_pages_per_seq pages or the items exceed
 * max_items (nothing is uploaded).  In the resident loop the queue goes to
 * a host slot for the next step instead. */
PKV_API pkv_status pkv_build_queue(pkv_handle* h, const int32_t* ctx_lens_host, int32_t batch,
                                   pkv_queue_info* info);

/* Same queue (PersistentKV page, Methodology 1 "Compact Workqueue" and
 * Methodology 2), built on the device from device context lengths (int32
 * [batch]) by one workgroup on stream; bit-identical to pkv_build_queue.
 * Supports PKV_ORDER_CANONICAL only.  The split decision is taken on the
 * device, so the host learns no counters.  A length outside
 * [0, max_pages_per_seq * P] or too many items sets the device error word
 * PKV_DEVERR_BAD_ITEM (detail: the row, or the item count) and leaves an
 * empty queue; the next pkv_decode or pkv_query reports it. */
PKV_API pkv_status pkv_build_queue_device(pkv_handle* h, const int32_t* ctx_lens_device,
                                          int32_t batch, void* stream);

/* Decode attention for the built queue (PersistentKV page, Methodology 1
 * "Native Block-Table Decode Engine": K/V read in place through the block
 * table, "Row-Local Bounds", and "Sequence Splitting" with the exact merge of
 * partial states).  One-shot handles: enqueue on stream (async) the
 * persistent decode kernel, whose workgroups pop queue items with one atomic
 * each (GPUOS page, section 4.1 "Persistent Kernel Executor"), then, with a
 * separate merge and any split or empty row, the merge kernel.  Resident
 * loop: publish one step and block until it completes (below).  Returns
 * PKV_ERR_DEVICE_FAULT (and enqueues nothing) if an earlier call left a
 * device error word set; PKV_ERR_STATE before a queue is built;
 * PKV_ERR_INVALID_ARG for null or misaligned tensors or a batch other than
 * the built queue's. */
PKV_API pkv_status pkv_decode(pkv_handle* h, const pkv_tensors* t, void* stream);

/* Optional timing: hipEvent_t handles (the caller's, created and destroyed by
 * the caller) recorded on the decode stream right before and right after
 * each one-shot decode kernel (not the separate merge; the resident loop
 * records neither).  PKV_ERR_INVALID_ARG when exactly one is null.  Pass
 * nulls to stop recording. */
PKV_API pkv_status pkv_set_decode_events(pkv_handle* h, void* before, void* after);

/* KV append in the resident loop (config append = 1; the next step after
 * the paged attention itself in a decode step, GPUOS page, the key-value cache
 * updates its persistent workers serve).  At every step the session's newest
 * token, index ctx_lens[b] - 1 of the queue built for the step, is written
 * into the cache before attention reads it: row (token mod P) of page
 * block_table[b][token / P] of every layer's pools, from new_k / new_v.  When
 * the token opens a new page (token mod P == 0) the step takes the next page
 * id from the free list and also writes it into block_table[b][token / P] of
 * every layer (a page id indexes every layer's pool alike).  The library owns
 * the free list: pkv_loop_set_free_pages replaces it with a copy of
 * pages[0..n) (ids in [0, num_pages), taken in that order); call it before
 * the first step or between steps.  A step that needs more pages than are
 * left fails with PKV_ERR_CAPACITY before anything is published.
 * PKV_ERR_STATE unless the handle runs the loop with append = 1. */
PKV_API pkv_status pkv_loop_set_free_pages(pkv_handle* h, const int32_t* pages, int32_t n);

/* Pages left on the append free list (into *n). */
PKV_API pkv_status pkv_loop_free_pages(const pkv_handle* h, int32_t* n);

/* Optional per-item trace (diagnostics): when buf (device memory, 32 bytes x
 * capacity) is set, every one-shot decode launch (the resident loop records
 * none) writes four uint64 words per record, at slots below capacity only:
 *   item i, at slot i:             {i | workgroup << 32, start clock,
 *                                   end clock, hardware id | XCC id << 32};
 *   workgroup w, at slot n_items + w: {w | w << 32 | 1 << 63, clock at entry,
 *                                   clock when its first item starts,
 *                                   hardware id | XCC id << 32}.
 * Clocks are the 100 MHz device wall clock.  Slots at or beyond capacity and
 * slots of items that did not run are left as they were.  PKV_ERR_INVALID_ARG
 * for a buffer not 8-byte aligned or a capacity <= 0 with a buffer.  Pass
 * null to stop tracing. */
PKV_API pkv_status pkv_set_trace(pkv_handle* h, void* buf, int32_t capacity);

/* Streaming copy of `bytes` (a multiple of 16) from src to dst on stream,
 * by a grid of `grid` workgroups (0 -> 4 per CU) of 256 threads, with
 * dwordx4 loads and stores: a known-size reference for measured HBM
 * bandwidth and for normalising hardware traffic counters. */
PKV_API pkv_status pkv_copy_probe(void* dst, const void* src, size_t bytes, int32_t grid,
                                  void* stream);

/* Streaming read of `bytes` (a multiple of 16) from src by `grid`
 * workgroups (0 -> 4 per CU) of 256 threads, four independent non-temporal
 * dwordx4 loads per thread per step; each thread stores one xor-folded word to sink
 * (uint32 [grid * 256]).  Measures the HBM read ceiling. */
PKV_API pkv_status pkv_read_probe(const void* src, size_t bytes, void* sink, int32_t grid,
                                  void* stream);

/* Read the control words: the queue head, the items finished, the device
 * error word and, for the resident loop, whether the kernel is alive and
 * which step it completed -- the queue-inspection and liveness calls of the
 * GPUOS page's host API (Table 1, peek_queue and worker_alive).  Synchronises
 * the device for one-shot handles; reads host words only while a resident
 * loop runs.  Returns PKV_ERR_DEVICE_FAULT when the device error word is
 * set (info is filled in either way). */
PKV_API pkv_status pkv_query(pkv_handle* h, pkv_runtime_info* info);

/* Clear the device error word after a reported fault (synchronises the
 * device), so that the handle may be used again (GPUOS page, section 5: a
 * kill switch returns an error code to the host, which decides what next).
 * Also starts the merge's arrival counters and the page cursors at zero
 * again, since a refused item never counted in.  PKV_ERR_STATE while a
 * resident loop runs. */
PKV_API pkv_status pkv_clear_error(pkv_handle* h);

/* Destroy the handle, the shutdown call of the GPUOS page's host API
 * (Table 1): for a resident loop, raise the exit flag and wait until the
 * kernel has left; then free the library's host memory.  Does not free the
 * caller's workspace. */
PKV_API pkv_status pkv_destroy(pkv_handle* h);

PKV_API const char* pkv_status_string(pkv_status s);
PKV_API const char* pkv_last_error(const pkv_handle* h);

/* Host-only planning, no handle and no GPU: the queue pkv_build_queue would
 * upload, written into caller host arrays: items (16-byte entries, capacity
 * items_cap), n_chunks [batch], part_off [batch + 1], merge_rows [batch].
 * num_cus must be set in cfg (no device is queried). */
PKV_API pkv_status pkv_plan_queue(const pkv_config* cfg, const int32_t* ctx_lens, int32_t batch,
                                  void* items, int32_t items_cap, int32_t* n_chunks,
                                  int32_t* part_off, int32_t* merge_rows, pkv_queue_info* info);

/* Test hook: copy the device queue as the decode kernel reads it -- the
 * workspace bytes from pkv_layout.queue_off up to the end of its items
 * (header, n_chunks, part_off, row_len, merge_rows at their layout offsets,
 * then n_items 16-byte items) -- to host memory host_dst of capacity bytes.
 * Waits for the handle's stream first.  *written receives the bytes copied
 * (at most capacity).  One-shot handles only (the resident loop keeps its
 * queue in host memory). */
PKV_API pkv_status pkv_queue_read(pkv_handle* h, void* host_dst, size_t capacity, size_t* written);

/* Test hook: write the K and V rows that the decode kernel's own gather
 * reads for queue item item_index, in token order, to device buffers k_out and
 * v_out ([tok_end - tok_begin][D] of the cache's element type, kv_dtype).
 * Enqueued on stream. */
PKV_API pkv_status pkv_debug_gather(pkv_handle* h, const pkv_tensors* t, int32_t item_index,
                                    void* k_out, void* v_out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * one-shot decode of pkv_build_queue_device + pkv_decode in one call, with
 * no handle and no workspace.  Its scratch (control words, queue, partial
 * states, counters) is a fixed 16 MiB array in the library's device memory,
 * one per device, held until the process ends; configs whose workspace
 * (pkv_workspace_size) exceeds 16 MiB get PKV_ERR_CAPACITY.  Enqueues on
 * stream, in order: a clear of the scratch's control words, the device queue
 * builder over ctx_lens_device (int32 [batch], device memory), the decode
 * kernel and, with a separate merge, the merge kernel.  Allocates nothing
 * (no hipMalloc, no library allocation, no memset).  cfg as for pkv_create
 * (persistent = 0 and the canonical order only, else PKV_ERR_UNSUPPORTED;
 * batch <= 4096); t as for pkv_decode, with t->batch == batch.  error_word
 * (nullable; device or mapped host memory, 4-byte aligned, owned by the
 * caller) receives a PKV_DEVERR_* code when the device finds a block-table
 * entry outside the pool or a bad length; the library never clears it.
 * Every call on a device shares that device's scratch and leaves it in
 * place: calls that overlap on one device (other streams, other threads)
 * race and must be ordered by the caller. */
PKV_API pkv_status pkv_decode_noalloc(const pkv_config* cfg, const int32_t* ctx_lens_device, int32_t batch,
                                      const pkv_tensors* t, uint32_t* error_word, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
