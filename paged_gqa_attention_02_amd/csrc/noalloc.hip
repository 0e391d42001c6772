// noalloc.hip -- paged_attn_decode_noalloc: the decode call with its scratch
// in a fixed device array of this library instead of a caller's workspace,
// for callers that cannot allocate device memory.
//
// The array is a static __device__ symbol, so every GPU the library runs on
// holds its own copy for the life of the process.  Host code never passes the
// symbol itself (on the host it names a host-side stand-in): the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "paged_attn.h"
#include "pa_internal.h"

namespace {

constexpr uint64_t kScratchBytes = PAGED_ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on device `dev`, looked up on first use.
pa_status scratch_for(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess) return PA_ERR_HIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess) return PA_ERR_HIP;
            const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (cur != dev && hipSetDevice(cur) != hipSuccess) return PA_ERR_HIP;
            if (e != hipSuccess || !ptr) return PA_ERR_HIP;
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return PA_OK;
}

}  // namespace

extern "C" pa_status paged_attn_decode_noalloc(
    const pa_plan* plan, const void* q, int64_t q_stride_b, const void* k_pool,
    const void* v_pool, int64_t kv_stride_page, int64_t kv_stride_tok, int64_t kv_stride_head,
    int64_t num_pages, const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
    int32_t page_size, float scale, float softcap, int32_t window, float k_scale,
    float v_scale, void* out, int64_t out_stride_b, const pa_extras* extras,
    void* hip_stream) {
    if (!plan) return PA_ERR_NULL_POINTER;
    if (plan->workspace_bytes > kScratchBytes) return PA_ERR_WORKSPACE_TOO_SMALL;
    pa::DecodeParams p;
    bool empty = false;
    const pa_status st = pa::decode_prepare(
        PA_MODE_DECODE, plan, q, q_stride_b, k_pool, v_pool, kv_stride_page, kv_stride_tok,
        kv_stride_head, num_pages, block_table, bt_stride, seq_lens, page_size, scale, softcap,
        window, k_scale, v_scale, out, out_stride_b, kScratchBytes, extras, &p, &empty);
    if (st != PA_OK || empty) return st;
    // the kernels run on the stream's device: use that device's copy
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    hipDevice_t dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return PA_ERR_HIP;
    void* ws = nullptr;
    const pa_status sst = scratch_for(dev, &ws);
    if (sst != PA_OK) return sst;
    // the split pass writes every workspace entry the merge reads: nothing in
    // the array needs to start at zero
    return pa::decode_launch(pa::kDecodeBothPasses, *plan, p, ws, stream);
}
