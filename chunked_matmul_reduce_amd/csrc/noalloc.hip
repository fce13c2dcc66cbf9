// The fused block for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): mmar_fused_noalloc runs
// the plans of mmar_fused_ex whose workspace (partial-product slots of the sequential
// schedule, the balanced schedule's tail partials, a pre-transposed weight) fits a
// file-scope device array of kScratchBytes, and never allocates.
//
// Each device that loads the library holds its own copy of `scratch` until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the device address is looked up once per device, with that
// device current, by hipGetSymbolAddress, and that address is what the kernels receive.
// Nothing in the workspace has to start at zero (every slot is written before it is read),
// and every call on a device shares that device's array: calls that overlap on one device
// race.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/mmar.h"
#include "mmar_internal.h"

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch`, looked up on the first call on the device.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        mmar::set_error("no current HIP device");
        return MMAR_ENODEV;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        mmar::set_error("device index beyond the static workspace table");
        return MMAR_ENODEV;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            mmar::set_error("hipGetSymbolAddress of the static workspace failed");
            return MMAR_EHIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MMAR_OK;
}

}  // namespace

extern "C" {

size_t mmar_noalloc_workspace_capacity(void) { return kScratchBytes; }

int mmar_fused_noalloc(const uint16_t* X, const uint16_t* W, const uint16_t* bias,
                       const uint16_t* residual, float* out, int64_t M, int64_t N, int64_t K,
                       int32_t P, float p_drop, uint64_t seed, int32_t schedule,
                       int32_t chunk_m, int32_t chunk_n, int32_t ring, int32_t w_mode,
                       int32_t tile, void* stream) {
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    return mmar::fused_fixed_ws(X, W, bias, residual, out, M, N, K, P, p_drop, seed, schedule,
                                chunk_m, chunk_n, ring, w_mode, tile, ws, kScratchBytes, stream);
}

}  // extern "C"
