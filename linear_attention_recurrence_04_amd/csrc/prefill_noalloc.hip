// prefill_noalloc.hip -- gdn_chunk_prefill for callers that cannot allocate
// (code under graph capture, tight serving loops): the per-chunk records that
// pass from the prep kernel to the scan kernel live in a fixed device array
// of this library instead of a caller workspace.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy (kNoallocScratchBytes) from module load to process end.
// Host code never uses the array's name as an address; its device address is
// taken once per device with hipGetSymbolAddress and kept here.  Calls on
// one GPU share the array: two calls whose kernels overlap in time (different
// streams without ordering between them) race on it.  Nothing in it has to
// start at zero: the prep kernel writes every record the scan reads.
#include <hip/hip_runtime.h>

#include <atomic>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// device address of `scratch` on each device, taken on the first call there
std::atomic<void*> scratch_ptr[kMaxDevices];

hipError_t scratch_on(int dev, void** out) {
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // the device is current here: hipGetSymbolAddress answers for it
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        scratch_ptr[dev].store(p, std::memory_order_release);   // same value from any thread
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" size_t gdn_chunk_prefill_noalloc_max_workspace(void) { return kNoallocScratchBytes; }

extern "C" gdn_status gdn_chunk_prefill_noalloc(const gdn_problem* p, const void* q,
                                                const void* k, const void* v, const float* log_g,
                                                const float* beta, const float* h0, float* hT,
                                                void* o, void* hip_stream) {
    if (!p) return GDN_ERR_NULL_POINTER;
    // 0 for an invalid problem (reported below) or one that needs no workspace;
    // a call longer than the array holds runs in pieces that fit
    const size_t need = gdn_chunk_prefill_workspace_bytes(p) > 0
                            ? gdn::prefill_mfma_min_workspace_bytes(p->B, p->T, p->Hk, p->Hv)
                            : 0;
    if (need > kNoallocScratchBytes) return GDN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        hipStream_t stream = static_cast<hipStream_t>(hip_stream);
        int cur = 0, dev = 0;
        if (hipGetDevice(&cur) != hipSuccess) return GDN_ERR_HIP;
        if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return GDN_ERR_HIP;
        if (!stream) dev = cur;
        if (dev != cur || dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
        if (scratch_on(dev, &ws) != hipSuccess) return GDN_ERR_HIP;
    }
    return static_cast<gdn_status>(gdn::prefill_checked(p, q, k, v, log_g, beta, h0, hT, o, ws,
                                                        need > 0 ? kNoallocScratchBytes : 0,
                                                        hip_stream));
}
