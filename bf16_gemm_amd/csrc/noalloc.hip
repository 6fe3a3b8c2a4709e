// noalloc.hip -- gemm_run_noalloc: the dense run with its scratch in a
// library-owned device array, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).
//
// The scratch a dense plan needs (the fp32 partial sums of a plan that
// splits K) lives in `scratch`, a file-scope device array of
// kNoallocScratchBytes.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code the array's name is only a
// host-side stand-in, never a device address: its address on each device
// is looked up once per device with hipGetSymbolAddress (the device current)
// and only that pointer is handed to kernels.  Every call on one device
// shares that device's array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace mgemm {

static __device__ __align__(256) unsigned char scratch[MGEMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up on the
// first call made with that device current.
static mgemm_status_t scratch_on_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_error("gemm_run_noalloc: hipGetDevice: %s", hipGetErrorString(e));
        return MGEMM_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("gemm_run_noalloc: device %d beyond the %d devices supported", dev, kMaxDevices);
        return MGEMM_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error("gemm_run_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                      hipGetErrorString(e));
            return MGEMM_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MGEMM_OK;
}

}  // namespace mgemm

using namespace mgemm;

extern "C" mgemm_status_t gemm_run_noalloc(mgemm_plan_t plan, const void *A, const void *B, void *D,
                                           mgemm_stream_t stream)
{
    if (!plan || plan->kind != PLAN_DENSE) {
        set_error("gemm_run_noalloc: null or non-dense plan");
        return MGEMM_ERR_INVALID_ARG;
    }
    const bool split = plan->splits > 1 && plan->tiles > 0 && !plan->noop && !plan->zero_fill;
    if (!split)
        return dense_run(plan, A, B, D, nullptr, nullptr, nullptr, 0, stream);
    if (plan->workspace_bytes > (size_t)MGEMM_NOALLOC_SCRATCH_BYTES) {
        set_error("gemm_run_noalloc: the plan needs %zu bytes of scratch, more than the %u bytes this entry point "
                  "holds per device (use gemm_run with a workspace, or a plan with fewer K ranges)",
                  plan->workspace_bytes, (unsigned)MGEMM_NOALLOC_SCRATCH_BYTES);
        return MGEMM_ERR_WORKSPACE;
    }
    void *ptr = nullptr;
    if (mgemm_status_t st = scratch_on_current_device(&ptr))
        return st;
    return dense_run(plan, A, B, D, nullptr, nullptr, ptr, (size_t)MGEMM_NOALLOC_SCRATCH_BYTES, stream);
}
