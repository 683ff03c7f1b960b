// pkv_decode_noalloc: the one-shot decode (device-built queue + decode +
// merge) for callers that cannot allocate device memory.  Its scratch
// (control words, queue, partial states, counters) is a fixed array in the
// library's own device memory instead of a caller workspace; the library
// resolves its address once per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

namespace pkv {

// The scratch of every pkv_decode_noalloc call on a device: each device holds
// its own copy for as long as the process runs.  In host code the name is a
// stand-in for the device array, never a device address: kernels and copies
// take the address resolved by scratch_on() below.
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
unsigned char* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The device address of this device's scratch, resolved on the first call
// made with the device current.
hipError_t scratch_on(int dev, unsigned char** out) {
    std::call_once(g_once[dev], [dev]() {
        void* p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? static_cast<unsigned char*>(p) : nullptr;
    });
    *out = g_ptr[dev];
    return g_err[dev];
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" PKV_API pkv_status pkv_decode_noalloc(const pkv_config* cfg, const int32_t* ctx_lens_device,
                                                 int32_t batch, const pkv_tensors* t, uint32_t* error_word,
                                                 void* stream) {
    const ApiRange range_("pkv_decode_noalloc");
    if (!cfg || !t) return PKV_ERR_INVALID_ARG;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PKV_ERR_HIP;
    Resolved r;
    const char* why = nullptr;
    pkv_status s = resolve_config(cfg, cus, &r, &why);
    if (s != PKV_OK) return s;
    if (r.persistent || r.order != PKV_ORDER_CANONICAL) return PKV_ERR_UNSUPPORTED;
    if (batch < 0 || batch > r.max_batch || batch > 4096) return PKV_ERR_CAPACITY;
    if (batch > 0 && (!ctx_lens_device || (uintptr_t)ctx_lens_device % 4)) return PKV_ERR_INVALID_ARG;
    if (error_word && (uintptr_t)error_word % 4) return PKV_ERR_INVALID_ARG;
    if ((s = check_tensor_args(r, t, &why)) != PKV_OK) return s;
    if (t->batch != batch) return PKV_ERR_INVALID_ARG;
    pkv_layout lay;
    compute_layout(r, &lay);
    if (lay.total_bytes > kScratchBytes) return PKV_ERR_CAPACITY;
    unsigned char* ws = nullptr;
    if (scratch_on(dev, &ws) != hipSuccess || !ws) return PKV_ERR_HIP;

    // Everything below is enqueued on one stream: clear the control words,
    // arrival counters (and page cursors), build the queue on the device,
    // decode, and merge if asked for separately.  No allocation, no memset
    // node: the clears are small fill kernels.
    const DecodeParams p = decode_params(r, lay, ws, t, error_word);
    const BuildParams bp = build_params(r, lay, ws, ctx_lens_device, batch, error_word);
    int rc = launch_init_ctrl(p.ctrl, p.arrive, (int)arrive_words(r), stream);
    if (rc == 0 && (r.schedule == PKV_SCHEDULE_PAGES || r.schedule == PKV_SCHEDULE_STEAL))
        rc = launch_zero(ws + lay.cursor_off, lay.loop_off - lay.cursor_off, stream);
    if (rc == 0) rc = launch_build_queue(bp, stream);
    if (rc == 0) rc = launch_decode(p, r.d, r.g, r.kv_dtype, cus * r.wg_per_cu, stream);
    if (rc == 0 && r.merge_mode == PKV_MERGE_SEPARATE && batch > 0) rc = launch_merge(p, r.d, r.g, batch, stream);
    return rc == 0 ? PKV_OK : PKV_ERR_HIP;
}
