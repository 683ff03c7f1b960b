// C-ABI entry points of libpkv (declared in include/pkv.h).
//
// Ownership follows the GPUOS page's rule that the runtime only receives
// pointers to memory the framework already allocated ("GPUOS: A GPU Operating
// System Primitive for Transparent Operation Fusion", section 4.3 "Memory
// Management and Safety"): every device buffer, the workspace included, is
// the caller's.  Device faults are reported back to the host as an error
// code, in the spirit of that page's kill switches (section 5, "returning an
// error code to the host").
#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>
#include <string.h>

#include <chrono>
#include <string>
#include <thread>
#include <vector>

#include "pkv_internal.h"

using namespace pkv;

namespace pkv {

ApiRange::ApiRange(const char* name) { roctxRangePushA(name); }
ApiRange::~ApiRange() { roctxRangePop(); }

DecodeParams decode_params(const Resolved& r, const pkv_layout& lay, unsigned char* ws, const pkv_tensors* t,
                           uint32_t* host_error) {
    DecodeParams p;
    memset(&p, 0, sizeof(p));
    p.q = static_cast<const uint16_t*>(t ? t->q : nullptr);
    p.k_pool = static_cast<const uint16_t*>(t ? t->k_pool : nullptr);
    p.v_pool = static_cast<const uint16_t*>(t ? t->v_pool : nullptr);
    p.block_table = t ? t->block_table : nullptr;
    p.out = static_cast<uint16_t*>(t ? t->out : nullptr);
    p.lse = t ? t->lse : nullptr;
    p.ctrl = reinterpret_cast<Ctrl*>(ws + lay.ctrl_off);
    p.qhdr = reinterpret_cast<const QHdr*>(ws + lay.queue_off);
    p.n_chunks = reinterpret_cast<const int32_t*>(ws + lay.n_chunks_off);
    p.part_off = reinterpret_cast<const int32_t*>(ws + lay.part_off_off);
    p.merge_rows = reinterpret_cast<const int32_t*>(ws + lay.merge_rows_off);
    p.items = reinterpret_cast<const Item*>(ws + lay.items_off);
    p.partial_o = reinterpret_cast<float*>(ws + lay.partial_o_off);
    p.sink = reinterpret_cast<const char*>(ws + lay.sink_off);
    p.row_len = reinterpret_cast<const int32_t*>(ws + lay.row_len_off);
    p.cursors = (r.schedule == PKV_SCHEDULE_PAGES || r.schedule == PKV_SCHEDULE_STEAL)
                    ? reinterpret_cast<uint32_t*>(ws + lay.cursor_off) : nullptr;
    p.steal = r.schedule == PKV_SCHEDULE_STEAL ? 1 : 0;
    p.partial_lse = reinterpret_cast<float*>(ws + lay.partial_lse_off);
    p.arrive = reinterpret_cast<uint32_t*>(ws + lay.arrive_off);
    p.grp_arrive = p.arrive + (size_t)r.max_batch * r.hkv * r.num_layers;
    p.trace = nullptr;
    p.trace_cap = 0;
    p.head = &reinterpret_cast<Ctrl*>(ws + lay.ctrl_off)->head[0];
    p.head_next = &reinterpret_cast<Ctrl*>(ws + lay.ctrl_off)->head[1];
    p.done_lines = reinterpret_cast<uint32_t*>(ws + lay.ctrl_off + sizeof(Ctrl));
    p.head_dim = r.d;
    p.coherent_out = 0;
    p.static_first = 1;
    p.static_sched = r.schedule == PKV_SCHEDULE_STATIC ? 1 : 0;
    p.coherent_in = 0;
    p.host_error = host_error;
    p.batch = t ? t->batch : 0;
    p.bt_stride = (t && t->block_table_stride) ? t->block_table_stride : r.max_pages_per_seq;
    p.num_pages = r.num_pages;
    p.hq = r.hq;
    p.hkv = r.hkv;
    p.max_tokens = r.max_pages_per_seq * r.page;
    p.max_items = r.max_items;
    p.fused_merge = r.merge_mode == PKV_MERGE_FUSED ? 1 : 0;
    p.scale_log2 = r.scale * 1.44269504088896340736f;
    return p;
}

BuildParams build_params(const Resolved& r, const pkv_layout& lay, unsigned char* ws, const int32_t* ctx_lens,
                         int32_t batch, uint32_t* host_error) {
    BuildParams p;
    memset(&p, 0, sizeof(p));
    p.ctx_lens = ctx_lens;
    p.qhdr = reinterpret_cast<QHdr*>(ws + lay.queue_off);
    p.n_chunks = reinterpret_cast<int32_t*>(ws + lay.n_chunks_off);
    p.part_off = reinterpret_cast<int32_t*>(ws + lay.part_off_off);
    p.row_len = reinterpret_cast<int32_t*>(ws + lay.row_len_off);
    p.merge_rows = reinterpret_cast<int32_t*>(ws + lay.merge_rows_off);
    p.items = reinterpret_cast<Item*>(ws + lay.items_off);
    p.ctrl = reinterpret_cast<Ctrl*>(ws + lay.ctrl_off);
    p.host_error = host_error;
    p.batch = batch;
    p.hkv = r.hkv;
    p.num_cus = r.num_cus;
    p.chunk = r.chunk;
    p.policy = r.policy;
    p.max_items = r.max_items;
    p.max_tokens = r.max_pages_per_seq * r.page;
    p.fit_min_pages = r.fit_min_pages;
    return p;
}

pkv_status check_tensor_args(const Resolved& r, const pkv_tensors* t, const char** why) {
    auto bad = [&](pkv_status s, const char* w) { *why = w; return s; };
    auto aligned = [](const void* p, size_t a) { return ((uintptr_t)p % a) == 0; };
    if (!t) return bad(PKV_ERR_INVALID_ARG, "null tensors");
    if (!t->q || !t->k_pool || !t->v_pool || !t->block_table || !t->out || !t->lse)
        return bad(PKV_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned(t->q, 16) || !aligned(t->k_pool, 16) || !aligned(t->v_pool, 16) || !aligned(t->out, 16))
        return bad(PKV_ERR_INVALID_ARG, "q, k_pool, v_pool and out must be 16-byte aligned");
    if (!aligned(t->block_table, 4) || !aligned(t->lse, 4) || (t->ctx_lens && !aligned(t->ctx_lens, 4)))
        return bad(PKV_ERR_INVALID_ARG, "block_table, ctx_lens and lse must be 4-byte aligned");
    if (t->batch < 0 || t->batch > r.max_batch) return bad(PKV_ERR_CAPACITY, "batch outside [0, max_batch]");
    if (t->block_table_stride < 0 || (t->block_table_stride > 0 && t->block_table_stride < r.max_pages_per_seq))
        return bad(PKV_ERR_INVALID_ARG, "block_table_stride smaller than max_pages_per_seq");
    return PKV_OK;
}

}  // namespace pkv

struct pkv_handle {
    Resolved r;
    pkv_layout lay;
    int device = 0;
    int device_cus = 0;
    int grid = 0;
    unsigned char* ws = nullptr;
    hipStream_t stream = nullptr;
    // pinned staging for queue uploads, double-buffered
    unsigned char* staging[2] = {nullptr, nullptr};
    hipEvent_t staging_evt[2] = {nullptr, nullptr};
    bool staging_pending[2] = {false, false};
    int staging_next = 0;
    size_t staging_bytes = 0;
    hipEvent_t upload_evt = nullptr;    // marks the last write of the device queue (recorded on demand)
    hipStream_t upload_stream = nullptr;
    hipEvent_t consumed_evt = nullptr;  // marks the last kernel that read the queue (recorded on demand)
    hipStream_t consume_stream = nullptr;
    // mapped host word mirrored by the kernels on a device fault
    uint32_t* host_err = nullptr;
    uint32_t* host_err_dev = nullptr;
    bool built = false;
    bool built_on_device = false;
    bool queue_uniform = false;         // host-built queue whose items all have one length
    int batch = 0;
    pkv_queue_info qinfo{};
    hipEvent_t ev_before = nullptr;
    hipEvent_t ev_after = nullptr;
    uint64_t* trace = nullptr;
    int32_t trace_cap = 0;
    uint32_t parity = 0;                // pop counter of the next one-shot launch (Ctrl::head)
    // resident loop
    LoopCtrl* lctrl = nullptr;          // host view (fine-grained, mapped)
    LoopCtrl* lctrl_dev = nullptr;
    unsigned char* slots = nullptr;     // two host queue slots (fine-grained, mapped)
    unsigned char* slots_dev = nullptr;
    uint64_t slot_bytes = 0;
    uint32_t epoch = 0;                 // last published step
    bool loop_running = false;
    // append: the free list (taken in order from free_head) and the lengths of
    // the queue built for the next step
    std::vector<int32_t> free_pages;
    size_t free_head = 0;
    std::vector<int32_t> lens;
    std::string last_error;
};

namespace {

pkv_status fail(pkv_handle* h, pkv_status s, const std::string& why) {
    if (h) h->last_error = why;
    return s;
}

pkv_status hip_fail(pkv_handle* h, hipError_t e, const char* what) {
    return fail(h, PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

DecodeParams make_params(const pkv_handle* h, const pkv_tensors* t) {
    DecodeParams p = decode_params(h->r, h->lay, h->ws, t, h->host_err_dev);
    p.trace = h->trace;
    p.trace_cap = h->trace_cap;
    Ctrl* c = reinterpret_cast<Ctrl*>(h->ws + h->lay.ctrl_off);
    p.head = &c->head[h->parity];
    p.head_next = &c->head[h->parity ^ 1];
    return p;
}

// A host slot: the step descriptor, the append page grants, then the queue.
uint64_t slot_queue_off(const pkv_handle* h) { return sizeof(LoopDesc) + loop_grant_bytes(h->r); }

unsigned char* slot_queue(pkv_handle* h, uint32_t epoch) {
    return h->slots + (uint64_t)(epoch & 1u) * h->slot_bytes + slot_queue_off(h);
}

pkv_status start_loop(pkv_handle* h) {
    h->slot_bytes = loop_slot_bytes(h->r, h->lay);
    hipError_t e;
    if ((e = hipHostMalloc((void**)&h->lctrl, sizeof(LoopCtrl), hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess ||
        (e = hipHostGetDevicePointer((void**)&h->lctrl_dev, h->lctrl, 0)) != hipSuccess ||
        (e = hipHostMalloc((void**)&h->slots, 2 * h->slot_bytes, hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess ||
        (e = hipHostGetDevicePointer((void**)&h->slots_dev, h->slots, 0)) != hipSuccess)
        return hip_fail(h, e, "loop host memory");
    memset(h->lctrl, 0, sizeof(LoopCtrl));
    memset(h->slots, 0, 2 * h->slot_bytes);
    LoopParams lp;
    memset(&lp, 0, sizeof(lp));
    lp.base = make_params(h, nullptr);
    lp.base.coherent_out = 1;
    lp.base.static_first = 0;
    lp.base.fused_merge = 1;           // the loop merges split rows inside the kernel
    lp.base.coherent_in = 1;           // q / block tables may change between steps
    lp.lctrl = h->lctrl_dev;
    lp.slots = h->slots_dev;
    lp.slot_bytes = h->slot_bytes;
    const uint64_t q0 = slot_queue_off(h);
    lp.q_hdr_off = q0;
    lp.q_nch_off = q0 + (h->lay.n_chunks_off - h->lay.queue_off);
    lp.q_poff_off = q0 + (h->lay.part_off_off - h->lay.queue_off);
    lp.q_mrows_off = q0 + (h->lay.merge_rows_off - h->lay.queue_off);
    lp.q_items_off = q0 + (h->lay.items_off - h->lay.queue_off);
    lp.grant_off = sizeof(LoopDesc);
    lp.append = h->r.append;
    lp.lglobal = reinterpret_cast<LoopGlobal*>(h->ws + h->lay.loop_off);
    lp.mirror = h->ws + h->lay.loop_mirror_off;
    lp.counters = h->ws + h->lay.loop_off + sizeof(LoopGlobal);
    lp.counter_bytes = loop_counter_bytes(h->r);
    lp.partial_o_layer = (uint64_t)h->r.max_items * h->r.g * h->r.d;
    lp.partial_lse_layer = (uint64_t)h->r.max_items * h->r.g;
    lp.arrive_layer = (uint64_t)h->r.max_batch * h->r.hkv;
    lp.grp_layer = (uint64_t)h->r.max_items;
    int clock_khz = 0;
    if ((e = hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, h->device)) != hipSuccess ||
        clock_khz <= 0)
        clock_khz = 100000;                                          // 100 MHz, the CDNA wall clock
    lp.timeout_ticks = (uint64_t)h->r.timeout_ms * (uint64_t)clock_khz;
    lp.max_batch = h->r.max_batch;
    int rc = launch_resident(lp, h->r.d, h->r.g, h->r.kv_dtype, h->grid, h->stream);
    if (rc != 0) return hip_fail(h, (hipError_t)rc, "resident launch");
    h->loop_running = true;
    return PKV_OK;
}

void stop_loop(pkv_handle* h) {
    if (h->loop_running) {
        __atomic_store_n(&h->lctrl->exit_flag, 1u, __ATOMIC_RELEASE);
        (void)hipStreamSynchronize(h->stream);
        h->loop_running = false;
    }
    if (h->slots) (void)hipHostFree(h->slots);
    if (h->lctrl) (void)hipHostFree(h->lctrl);
    h->slots = nullptr;
    h->lctrl = nullptr;
}

pkv_status decode_loop(pkv_handle* h, const pkv_tensors* t) {
    if (!h->loop_running) return fail(h, PKV_ERR_STATE, "resident loop not running");
    if (__atomic_load_n(&h->lctrl->alive, __ATOMIC_ACQUIRE) == 0 &&
        __atomic_load_n(&h->lctrl->exit_reason, __ATOMIC_ACQUIRE) != 0)
        return fail(h, PKV_ERR_TIMEOUT, "resident kernel has exited (idle or wait limit)");
    const uint32_t e = h->epoch + 1;
    unsigned char* slot = h->slots + (uint64_t)(e & 1u) * h->slot_bytes;
    LoopDesc* d = reinterpret_cast<LoopDesc*>(slot);
    if (h->r.append) {
        // page grants for the rows whose newest token opens a page, taken
        // from the free list in order; nothing is published if it runs out
        if (!t->new_k || !t->new_v || !aligned(t->new_k, 4) || !aligned(t->new_v, 4))
            return fail(h, PKV_ERR_INVALID_ARG, "append needs new_k and new_v (4-byte aligned)");
        if ((int)h->lens.size() != t->batch) return fail(h, PKV_ERR_STATE, "batch differs from the built queue");
        int32_t* grant = reinterpret_cast<int32_t*>(slot + sizeof(LoopDesc));
        size_t need = 0;
        for (int b = 0; b < t->batch; ++b)
            need += (h->lens[b] >= 1 && (h->lens[b] - 1) % h->r.page == 0) ? 1 : 0;
        if (h->free_head + need > h->free_pages.size())
            return fail(h, PKV_ERR_CAPACITY, "append free list exhausted");
        for (int b = 0; b < t->batch; ++b) {
            const bool opens = h->lens[b] >= 1 && (h->lens[b] - 1) % h->r.page == 0;
            grant[b] = opens ? h->free_pages[h->free_head++] : -1;
        }
        d->new_k = static_cast<const uint16_t*>(t->new_k);
        d->new_v = static_cast<const uint16_t*>(t->new_v);
        d->ls_new = h->r.num_layers > 1 ? t->layer_stride_new : 0;
    } else {
        d->new_k = d->new_v = nullptr;
        d->ls_new = 0;
    }
    d->q = static_cast<const uint16_t*>(t->q);
    d->k_pool = static_cast<const uint16_t*>(t->k_pool);
    d->v_pool = static_cast<const uint16_t*>(t->v_pool);
    d->block_table = t->block_table;
    d->out = static_cast<uint16_t*>(t->out);
    d->lse = t->lse;
    const bool layered = h->r.num_layers > 1;
    d->ls_q = layered ? t->layer_stride_q : 0;
    d->ls_kv = layered ? t->layer_stride_kv : 0;
    d->ls_bt = layered ? t->layer_stride_bt : 0;
    d->ls_out = layered ? t->layer_stride_out : 0;
    d->ls_lse = layered ? t->layer_stride_lse : 0;
    d->batch = t->batch;
    d->bt_stride = t->block_table_stride ? t->block_table_stride : h->r.max_pages_per_seq;
    d->n_layers = h->r.num_layers;
    d->epoch = e;
    __atomic_store_n(&h->lctrl->in_epoch, e, __ATOMIC_RELEASE);     // publish the step
    h->epoch = e;
    const auto t0 = std::chrono::steady_clock::now();
    const auto limit = std::chrono::milliseconds(h->r.timeout_ms);
    uint32_t spins = 0;
    while (__atomic_load_n(&h->lctrl->out_epoch, __ATOMIC_ACQUIRE) != e) {
        if (__atomic_load_n(h->host_err, __ATOMIC_ACQUIRE) != 0)
            return fail(h, PKV_ERR_DEVICE_FAULT, "device error word set (see pkv_query)");
        if ((++spins & 1023u) == 0) {
            if (std::chrono::steady_clock::now() - t0 > limit)
                return fail(h, PKV_ERR_TIMEOUT, "step not completed within timeout_ms");
            if (__atomic_load_n(&h->lctrl->exit_reason, __ATOMIC_ACQUIRE) != 0)
                return fail(h, PKV_ERR_TIMEOUT, "resident kernel left the loop");
        }
    }
    return PKV_OK;
}

// Ordering of the handle's device work across streams.  The device queue (and
// the control words) are written by a queue upload or the device builder and
// read by the decode, merge and gather kernels; a write must not start before
// the last reader on another stream has finished, and a reader must not
// start before the last write.  The handle remembers the stream of the last
// write and of the last reader.  Work on that same stream is ordered by the
// stream; work on another stream first waits for an event recorded on the
// remembered stream at that moment (it marks everything enqueued there so far,
// which includes the write or the reader).  Events are recorded only when a
// call on another stream needs them: an event record after every launch costs
// the back-to-back launches of one stream several microseconds each.
hipError_t after_upload(pkv_handle* h, hipStream_t s) {
    if (s == h->upload_stream) return hipSuccess;
    hipError_t e = hipEventRecord(h->upload_evt, h->upload_stream);
    return e != hipSuccess ? e : hipStreamWaitEvent(s, h->upload_evt, 0);
}
hipError_t after_readers(pkv_handle* h, hipStream_t s) {
    if (s == h->consume_stream) return hipSuccess;
    hipError_t e = hipEventRecord(h->consumed_evt, h->consume_stream);
    return e != hipSuccess ? e : hipStreamWaitEvent(s, h->consumed_evt, 0);
}
void mark_upload(pkv_handle* h, hipStream_t s) { h->upload_stream = s; }
void mark_readers(pkv_handle* h, hipStream_t s) { h->consume_stream = s; }

pkv_status check_tensors(pkv_handle* h, const pkv_tensors* t) {
    const char* why = nullptr;
    const pkv_status s = check_tensor_args(h->r, t, &why);
    return s == PKV_OK ? s : fail(h, s, why);
}

}  // namespace

extern "C" {

PKV_API const char* pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "ok";
        case PKV_ERR_INVALID_ARG: return "invalid argument";
        case PKV_ERR_UNSUPPORTED: return "unsupported shape";
        case PKV_ERR_CAPACITY: return "capacity exceeded";
        case PKV_ERR_HIP: return "HIP runtime error";
        case PKV_ERR_STATE: return "wrong call order";
        case PKV_ERR_DEVICE_FAULT: return "device fault";
        case PKV_ERR_TIMEOUT: return "timeout";
        default: return "unknown status";
    }
}

PKV_API const char* pkv_last_error(const pkv_handle* h) { return h ? h->last_error.c_str() : ""; }

PKV_API pkv_status pkv_workspace_layout(const pkv_config* cfg, pkv_layout* layout) {
    if (!layout) return PKV_ERR_INVALID_ARG;
    Resolved r;
    const char* why;
    // The layout does not depend on the CU count; use 1 when the config leaves it unset.
    pkv_status s = resolve_config(cfg, 1, &r, &why);
    if (s != PKV_OK) return s;
    compute_layout(r, layout);
    return PKV_OK;
}

PKV_API pkv_status pkv_workspace_size(const pkv_config* cfg, size_t* bytes) {
    if (!bytes) return PKV_ERR_INVALID_ARG;
    pkv_layout lay;
    pkv_status s = pkv_workspace_layout(cfg, &lay);
    if (s != PKV_OK) return s;
    *bytes = (size_t)lay.total_bytes;
    return PKV_OK;
}

PKV_API pkv_status pkv_plan_queue(const pkv_config* cfg, const int32_t* ctx_lens, int32_t batch,
                                  void* items, int32_t items_cap, int32_t* n_chunks,
                                  int32_t* part_off, int32_t* merge_rows, pkv_queue_info* info) {
    Resolved r;
    const char* why;
    pkv_status s = resolve_config(cfg, 0, &r, &why);
    if (s != PKV_OK) return s;
    if (!items || !n_chunks || !part_off || !merge_rows || items_cap < 0) return PKV_ERR_INVALID_ARG;
    QHdr qh;
    return plan_queue(r, ctx_lens, batch, &qh, n_chunks, part_off, merge_rows,
                      static_cast<Item*>(items), items_cap, info, &why);
}

PKV_API pkv_status pkv_create(const pkv_config* cfg, void* workspace, size_t workspace_bytes,
                              void* stream, pkv_handle** out) {
    const ApiRange range_("pkv_create");
    if (!out) return PKV_ERR_INVALID_ARG;
    *out = nullptr;
    pkv_handle* h = new (std::nothrow) pkv_handle();
    if (!h) return PKV_ERR_CAPACITY;
    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) { delete h; return PKV_ERR_HIP; }
    e = hipDeviceGetAttribute(&h->device_cus, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess) { delete h; return PKV_ERR_HIP; }
    const char* why;
    pkv_status s = resolve_config(cfg, h->device_cus, &h->r, &why);
    if (s != PKV_OK) { delete h; return s; }
    compute_layout(h->r, &h->lay);
    if (!workspace || workspace_bytes < h->lay.total_bytes || !aligned(workspace, 256)) {
        delete h;
        return PKV_ERR_INVALID_ARG;
    }
    h->ws = static_cast<unsigned char*>(workspace);
    h->stream = static_cast<hipStream_t>(stream);
    h->grid = h->device_cus * h->r.wg_per_cu;
    if (h->r.persistent) {
        // The resident kernel's dependency waits assume that every workgroup
        // of its grid is resident at once; refuse a build whose registers or
        // LDS would not fit wg_per_cu workgroups on a CU.
        int fit = 0;
        if (resident_occupancy(h->r.d, h->r.g, h->r.kv_dtype, &fit) != 0 || fit < h->r.wg_per_cu) {
            h->last_error = "resident kernel does not fit wg_per_cu workgroups per CU";
            delete h;
            return PKV_ERR_UNSUPPORTED;
        }
    }
    h->staging_bytes = h->lay.items_off - h->lay.queue_off + 16ull * h->r.max_items;
    for (int i = 0; i < 2; ++i) {
        if ((e = hipHostMalloc((void**)&h->staging[i], h->staging_bytes, hipHostMallocDefault)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&h->staging_evt[i], hipEventDisableTiming)) != hipSuccess) {
            pkv_destroy(h);
            return PKV_ERR_HIP;
        }
        memset(h->staging[i], 0, h->staging_bytes);
    }
    if ((e = hipEventCreateWithFlags(&h->upload_evt, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&h->consumed_evt, hipEventDisableTiming)) != hipSuccess ||
        (e = hipHostMalloc((void**)&h->host_err, 64, hipHostMallocMapped | hipHostMallocCoherent)) != hipSuccess ||
        (e = hipHostGetDevicePointer((void**)&h->host_err_dev, h->host_err, 0)) != hipSuccess) {
        pkv_destroy(h);
        return PKV_ERR_HIP;
    }
    memset(h->host_err, 0, 64);
    int rc = launch_init_ctrl(reinterpret_cast<Ctrl*>(h->ws + h->lay.ctrl_off),
                              reinterpret_cast<uint32_t*>(h->ws + h->lay.arrive_off),
                              (int)arrive_words(h->r), h->stream);
    if (rc == 0 && h->r.persistent)
        rc = launch_zero(h->ws + h->lay.loop_off, sizeof(LoopGlobal) + 2 * loop_counter_bytes(h->r), h->stream);
    if (rc == 0 && (h->r.schedule == PKV_SCHEDULE_PAGES || h->r.schedule == PKV_SCHEDULE_STEAL))
        // cursors start at zero; the merge re-arms them
        rc = launch_zero(h->ws + h->lay.cursor_off, h->lay.loop_off - h->lay.cursor_off, h->stream);
    if (rc != 0) { pkv_destroy(h); return PKV_ERR_HIP; }
    // an empty queue until the first build
    QHdr* qh = reinterpret_cast<QHdr*>(h->staging[0]);
    memset(qh, 0, sizeof(QHdr));
    e = hipMemcpyAsync(h->ws + h->lay.queue_off, qh, sizeof(QHdr), hipMemcpyHostToDevice, h->stream);
    if (e == hipSuccess) e = hipEventRecord(h->staging_evt[0], h->stream);
    if (e != hipSuccess) { pkv_destroy(h); return PKV_ERR_HIP; }
    mark_upload(h, h->stream);
    mark_readers(h, h->stream);
    h->staging_pending[0] = true;
    h->staging_next = 1;
    if (h->r.persistent) {
        s = start_loop(h);
        if (s != PKV_OK) { pkv_destroy(h); return s; }
    }
    *out = h;
    return PKV_OK;
}

PKV_API pkv_status pkv_build_queue(pkv_handle* h, const int32_t* ctx_lens_host, int32_t batch,
                                   pkv_queue_info* info) {
    const ApiRange range_("pkv_build_queue");
    if (!h) return PKV_ERR_INVALID_ARG;
    if (batch < 0 || batch > h->r.max_batch) return fail(h, PKV_ERR_CAPACITY, "batch outside [0, max_batch]");
    if (batch > 0 && !ctx_lens_host) return fail(h, PKV_ERR_INVALID_ARG, "null ctx_lens");
    if (h->r.persistent) {
        unsigned char* st = slot_queue(h, h->epoch + 1);
        const uint64_t q0 = h->lay.queue_off;
        pkv_queue_info qi;
        const char* why;
        pkv_status s = plan_queue(h->r, ctx_lens_host, batch, reinterpret_cast<QHdr*>(st),
                                  reinterpret_cast<int32_t*>(st + (h->lay.n_chunks_off - q0)),
                                  reinterpret_cast<int32_t*>(st + (h->lay.part_off_off - q0)),
                                  reinterpret_cast<int32_t*>(st + (h->lay.merge_rows_off - q0)),
                                  reinterpret_cast<Item*>(st + (h->lay.items_off - q0)), h->r.max_items, &qi, &why,
                                  reinterpret_cast<int32_t*>(st + (h->lay.row_len_off - q0)));
        if (s != PKV_OK) return fail(h, s, why);
        qi.launches_per_step = 0;             // nothing is launched per step
        h->lens.assign(ctx_lens_host, ctx_lens_host + batch);
        h->built = true;
        h->built_on_device = false;
        h->batch = batch;
        h->qinfo = qi;
        if (info) *info = qi;
        return PKV_OK;
    }
    const int i = h->staging_next;
    hipError_t e;
    if (h->staging_pending[i]) {          // the previous upload from this buffer must have left
        if ((e = hipEventSynchronize(h->staging_evt[i])) != hipSuccess) return hip_fail(h, e, "staging wait");
        h->staging_pending[i] = false;
    }
    unsigned char* st = h->staging[i];
    const uint64_t q0 = h->lay.queue_off;
    QHdr* qh = reinterpret_cast<QHdr*>(st);
    int32_t* n_chunks = reinterpret_cast<int32_t*>(st + (h->lay.n_chunks_off - q0));
    int32_t* part_off = reinterpret_cast<int32_t*>(st + (h->lay.part_off_off - q0));
    int32_t* merge_rows = reinterpret_cast<int32_t*>(st + (h->lay.merge_rows_off - q0));
    Item* items = reinterpret_cast<Item*>(st + (h->lay.items_off - q0));
    pkv_queue_info qi;
    const char* why;
    int32_t* row_len = reinterpret_cast<int32_t*>(st + (h->lay.row_len_off - q0));
    pkv_status s = plan_queue(h->r, ctx_lens_host, batch, qh, n_chunks, part_off, merge_rows, items,
                              h->r.max_items, &qi, &why, row_len);
    if (s != PKV_OK) return fail(h, s, why);
    const size_t bytes = (h->lay.items_off - q0) + 16ull * qi.n_items;
    // the previous queue may still be read by a decode on another stream
    if ((e = after_readers(h, h->stream)) != hipSuccess) return hip_fail(h, e, "stream wait");
    if ((e = after_upload(h, h->stream)) != hipSuccess) return hip_fail(h, e, "stream wait");
    if ((e = hipMemcpyAsync(h->ws + q0, st, bytes, hipMemcpyHostToDevice, h->stream)) != hipSuccess)
        return hip_fail(h, e, "queue upload");
    if ((e = hipEventRecord(h->staging_evt[i], h->stream)) != hipSuccess) return hip_fail(h, e, "event record");
    mark_upload(h, h->stream);
    h->staging_pending[i] = true;
    h->staging_next = 1 - i;
    h->built = true;
    h->built_on_device = false;
    h->queue_uniform = qh->uniform != 0;
    h->batch = batch;
    h->qinfo = qi;
    if (info) *info = qi;
    return PKV_OK;
}

PKV_API pkv_status pkv_build_queue_device(pkv_handle* h, const int32_t* ctx_lens_device, int32_t batch,
                                          void* stream) {
    const ApiRange range_("pkv_build_queue_device");
    if (!h) return PKV_ERR_INVALID_ARG;
    if (batch < 0 || batch > h->r.max_batch) return fail(h, PKV_ERR_CAPACITY, "batch outside [0, max_batch]");
    if (batch > 4096) return fail(h, PKV_ERR_UNSUPPORTED, "device builder supports batch <= 4096");
    if (batch > 0 && (!ctx_lens_device || !aligned(ctx_lens_device, 4)))
        return fail(h, PKV_ERR_INVALID_ARG, "null or misaligned ctx_lens");
    if (h->r.order != PKV_ORDER_CANONICAL) return fail(h, PKV_ERR_UNSUPPORTED, "device builder: canonical order only");
    if (h->r.persistent) return fail(h, PKV_ERR_STATE, "the resident loop takes host-built queues");
    const BuildParams p = build_params(h->r, h->lay, h->ws, ctx_lens_device, batch, h->host_err_dev);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if ((e = after_upload(h, s)) != hipSuccess || (e = after_readers(h, s)) != hipSuccess)
        return hip_fail(h, e, "stream wait");
    int rc = launch_build_queue(p, s);
    if (rc != 0) return hip_fail(h, (hipError_t)rc, "build_queue launch");
    mark_upload(h, s);
    h->built = true;
    h->built_on_device = true;
    h->batch = batch;
    memset(&h->qinfo, 0, sizeof(h->qinfo));
    return PKV_OK;
}

PKV_API pkv_status pkv_decode(pkv_handle* h, const pkv_tensors* t, void* stream) {
    const ApiRange range_("pkv_decode");
    if (!h) return PKV_ERR_INVALID_ARG;
    if (!h->built) return fail(h, PKV_ERR_STATE, "pkv_decode before pkv_build_queue");
    pkv_status s = check_tensors(h, t);
    if (s != PKV_OK) return s;
    if (t->batch != h->batch) return fail(h, PKV_ERR_INVALID_ARG, "batch differs from the built queue");
    if (__atomic_load_n(h->host_err, __ATOMIC_ACQUIRE) != 0)
        return fail(h, PKV_ERR_DEVICE_FAULT, "device error word set (see pkv_query)");
    if (h->r.persistent) {
        if (h->r.num_layers > 1 && (t->layer_stride_q <= 0 || t->layer_stride_kv <= 0 ||
                                    t->layer_stride_bt <= 0 || t->layer_stride_out <= 0 ||
                                    t->layer_stride_lse <= 0))
            return fail(h, PKV_ERR_INVALID_ARG, "layered tensors need positive layer strides");
        return decode_loop(h, t);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    // after the queue's upload, and after the previous decode (the control
    // words and partial states are shared by every launch of the handle)
    if ((e = after_upload(h, st)) != hipSuccess || (e = after_readers(h, st)) != hipSuccess)
        return hip_fail(h, e, "stream wait");
    DecodeParams p = make_params(h, t);
    // A host-built queue of items of one length in whole rounds of the grid:
    // claims could not change how much each workgroup runs and would only
    // queue on the one pop counter as the rounds end, so the launch assigns
    // round-robin (the static schedule: the same item computations, the same
    // outputs).
    if (!h->built_on_device && h->queue_uniform && h->qinfo.n_items > h->grid && h->qinfo.n_items % h->grid == 0)
        p.static_sched = 1;
    if (h->ev_before && (e = hipEventRecord(h->ev_before, st)) != hipSuccess) return hip_fail(h, e, "event record");
    int rc = launch_decode(p, h->r.d, h->r.g, h->r.kv_dtype, h->grid, st);
    if (rc != 0) return hip_fail(h, (hipError_t)rc, "decode launch");
    h->parity ^= 1u;
    if (h->ev_after && (e = hipEventRecord(h->ev_after, st)) != hipSuccess) return hip_fail(h, e, "event record");
    const int merge_rows = h->built_on_device ? h->batch : h->qinfo.n_merge_rows;
    if (h->r.merge_mode == PKV_MERGE_SEPARATE && merge_rows > 0) {
        rc = launch_merge(p, h->r.d, h->r.g, merge_rows, st);
        if (rc != 0) return hip_fail(h, (hipError_t)rc, "merge launch");
    }
    mark_readers(h, st);
    return PKV_OK;
}

PKV_API pkv_status pkv_set_decode_events(pkv_handle* h, void* before, void* after) {
    if (!h) return PKV_ERR_INVALID_ARG;
    if ((before == nullptr) != (after == nullptr)) return fail(h, PKV_ERR_INVALID_ARG, "set both events or neither");
    h->ev_before = static_cast<hipEvent_t>(before);
    h->ev_after = static_cast<hipEvent_t>(after);
    return PKV_OK;
}

PKV_API pkv_status pkv_loop_set_free_pages(pkv_handle* h, const int32_t* pages, int32_t n) {
    if (!h) return PKV_ERR_INVALID_ARG;
    if (!h->r.persistent || !h->r.append) return fail(h, PKV_ERR_STATE, "free pages need a loop with append = 1");
    if (n < 0 || (n > 0 && !pages)) return fail(h, PKV_ERR_INVALID_ARG, "bad free page list");
    for (int32_t i = 0; i < n; ++i)
        if (pages[i] < 0 || pages[i] >= h->r.num_pages) return fail(h, PKV_ERR_INVALID_ARG, "free page outside the pool");
    h->free_pages.assign(pages, pages + n);
    h->free_head = 0;
    return PKV_OK;
}

PKV_API pkv_status pkv_loop_free_pages(const pkv_handle* h, int32_t* n) {
    if (!h || !n) return PKV_ERR_INVALID_ARG;
    *n = (int32_t)(h->free_pages.size() - h->free_head);
    return PKV_OK;
}

PKV_API pkv_status pkv_set_trace(pkv_handle* h, void* buf, int32_t capacity) {
    if (!h) return PKV_ERR_INVALID_ARG;
    if (buf && (capacity <= 0 || !aligned(buf, 8))) return fail(h, PKV_ERR_INVALID_ARG, "bad trace buffer");
    h->trace = static_cast<uint64_t*>(buf);
    h->trace_cap = buf ? capacity : 0;
    return PKV_OK;
}

PKV_API pkv_status pkv_copy_probe(void* dst, const void* src, size_t bytes, int32_t grid, void* stream) {
    if (!dst || !src || bytes == 0 || bytes % 16 || !aligned(dst, 16) || !aligned(src, 16) || grid < 0)
        return PKV_ERR_INVALID_ARG;
    int g = grid;
    if (g == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return PKV_ERR_HIP;
        g = 4 * cus;
    }
    return launch_copy_probe(dst, src, bytes, g, stream) == 0 ? PKV_OK : PKV_ERR_HIP;
}

PKV_API pkv_status pkv_read_probe(const void* src, size_t bytes, void* sink, int32_t grid, void* stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 || !aligned(src, 16) || !aligned(sink, 4) || grid < 0)
        return PKV_ERR_INVALID_ARG;
    int g = grid;
    if (g == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return PKV_ERR_HIP;
        g = 4 * cus;
    }
    return launch_read_probe(src, bytes, sink, g, stream) == 0 ? PKV_OK : PKV_ERR_HIP;
}

PKV_API pkv_status pkv_query(pkv_handle* h, pkv_runtime_info* info) {
    if (!h || !info) return PKV_ERR_INVALID_ARG;
    if (h->loop_running) {               // the resident kernel never idles: read host words only
        memset(info, 0, sizeof(*info));
        info->error_code = __atomic_load_n(h->host_err, __ATOMIC_ACQUIRE);
        info->grid = h->grid;
        info->num_cus = h->device_cus;
        info->n_items = (uint32_t)h->qinfo.n_items;
        info->loop_out_epoch = __atomic_load_n(&h->lctrl->out_epoch, __ATOMIC_ACQUIRE);
        info->loop_alive = __atomic_load_n(&h->lctrl->alive, __ATOMIC_ACQUIRE);
        info->loop_exit_reason = __atomic_load_n(&h->lctrl->exit_reason, __ATOMIC_ACQUIRE);
        info->loop_steps_started = __atomic_load_n(&h->lctrl->heartbeat, __ATOMIC_ACQUIRE);
        if (info->error_code != 0) return fail(h, PKV_ERR_DEVICE_FAULT, "device error word set");
        return PKV_OK;
    }
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(h, e, "device sync");
    Ctrl c;
    uint32_t lines[kDoneLines * 32];
    QHdr q;
    if ((e = hipMemcpy(&c, h->ws + h->lay.ctrl_off, sizeof(c), hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(lines, h->ws + h->lay.ctrl_off + sizeof(Ctrl), sizeof(lines), hipMemcpyDeviceToHost)) !=
            hipSuccess)
        return hip_fail(h, e, "ctrl read");
    if ((e = hipMemcpy(&q, h->ws + h->lay.queue_off, sizeof(q), hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_fail(h, e, "queue header read");
    memset(info, 0, sizeof(*info));
    info->error_code = c.error_code;
    info->error_detail = c.error_detail;
    info->queue_head = c.head[h->parity];
    info->n_items = (uint32_t)q.n_items;
    for (int i = 0; i < kDoneLines; ++i) info->items_done += lines[32 * i];
    info->decode_calls = c.decode_calls;
    info->grid = h->grid;
    info->num_cus = h->device_cus;
    if (c.error_code != 0) return fail(h, PKV_ERR_DEVICE_FAULT, "device error word set");
    return PKV_OK;
}

PKV_API pkv_status pkv_clear_error(pkv_handle* h) {
    if (!h) return PKV_ERR_INVALID_ARG;
    if (h->loop_running) return fail(h, PKV_ERR_STATE, "clear errors after pkv_destroy of a resident loop");
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(h, e, "device sync");
    const uint32_t z[2] = {0u, 0u};
    e = hipMemcpy(h->ws + h->lay.ctrl_off + offsetof(Ctrl, error_code), z, sizeof(z), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(h, e, "clear error");
    // An item the kernel refused never counted in for its row's merge, so the
    // arrival counters (and the page cursors of its row) may be left part-way:
    // start them at zero again.
    int rc = launch_zero(h->ws + h->lay.arrive_off, h->lay.loop_off - h->lay.arrive_off, h->stream);
    if (rc == 0 && (e = hipStreamSynchronize(h->stream)) != hipSuccess) return hip_fail(h, e, "clear counters");
    if (rc != 0) return hip_fail(h, (hipError_t)rc, "clear counters");
    __atomic_store_n(h->host_err, 0u, __ATOMIC_RELEASE);
    return PKV_OK;
}

PKV_API pkv_status pkv_queue_read(pkv_handle* h, void* host_dst, size_t capacity, size_t* written) {
    if (!h || !written) return PKV_ERR_INVALID_ARG;
    *written = 0;
    if (h->r.persistent) return fail(h, PKV_ERR_STATE, "pkv_queue_read needs a one-shot handle");
    if (capacity > 0 && !host_dst) return fail(h, PKV_ERR_INVALID_ARG, "null host_dst");
    // the last write, on whichever stream it was enqueued
    hipError_t e = hipEventRecord(h->upload_evt, h->upload_stream);
    if (e == hipSuccess) e = hipEventSynchronize(h->upload_evt);
    if (e != hipSuccess) return hip_fail(h, e, "event sync");
    QHdr qh;
    e = hipMemcpy(&qh, h->ws + h->lay.queue_off, sizeof(qh), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(h, e, "queue header read");
    if (qh.n_items < 0 || qh.n_items > h->r.max_items) return fail(h, PKV_ERR_DEVICE_FAULT, "queue header out of range");
    const size_t total = (h->lay.items_off - h->lay.queue_off) + 16ull * (size_t)qh.n_items;
    const size_t n = total < capacity ? total : capacity;
    if (n > 0) {
        e = hipMemcpy(host_dst, h->ws + h->lay.queue_off, n, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(h, e, "queue read");
    }
    *written = n;
    return PKV_OK;
}

PKV_API pkv_status pkv_debug_gather(pkv_handle* h, const pkv_tensors* t, int32_t item_index,
                                    void* k_out, void* v_out, void* stream) {
    if (!h) return PKV_ERR_INVALID_ARG;
    if (!h->built) return fail(h, PKV_ERR_STATE, "pkv_debug_gather before pkv_build_queue");
    if (h->r.persistent) return fail(h, PKV_ERR_STATE, "pkv_debug_gather needs a one-shot handle");
    pkv_status s = check_tensors(h, t);
    if (s != PKV_OK) return s;
    if (!k_out || !v_out || !aligned(k_out, 16) || !aligned(v_out, 16))
        return fail(h, PKV_ERR_INVALID_ARG, "k_out and v_out must be 16-byte aligned");
    if (item_index < 0) return fail(h, PKV_ERR_INVALID_ARG, "negative item index");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if ((e = after_upload(h, st)) != hipSuccess || (e = after_readers(h, st)) != hipSuccess)
        return hip_fail(h, e, "stream wait");
    const DecodeParams p = make_params(h, t);
    int rc = launch_debug_gather(p, h->r.d, h->r.kv_dtype, item_index, k_out, v_out, st);
    if (rc != 0) return hip_fail(h, (hipError_t)rc, "gather launch");
    mark_readers(h, st);
    return PKV_OK;
}

PKV_API pkv_status pkv_destroy(pkv_handle* h) {
    const ApiRange range_("pkv_destroy");
    if (!h) return PKV_ERR_INVALID_ARG;
    stop_loop(h);
    if (h->stream || h->staging[0]) (void)hipStreamSynchronize(h->stream);
    for (int i = 0; i < 2; ++i) {
        if (h->staging_evt[i]) (void)hipEventDestroy(h->staging_evt[i]);
        if (h->staging[i]) (void)hipHostFree(h->staging[i]);
    }
    if (h->upload_evt) (void)hipEventDestroy(h->upload_evt);
    if (h->consumed_evt) (void)hipEventDestroy(h->consumed_evt);
    if (h->host_err) (void)hipHostFree(h->host_err);
    delete h;
    return PKV_OK;
}

}  // extern "C"
