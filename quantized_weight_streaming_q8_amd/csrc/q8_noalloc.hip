// q8_noalloc.hip -- q8_matmul_narrow_ws with its workspace in a static device
// array, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The split execution of long rows meets through a workspace of one record
// per row block (an arrival counter, then the split partials).  Here that
// workspace is `scratch`, a file-scope device array of kScratchBytes that
// every GPU the library runs on holds until the process ends.  In host code
// the array's name only stands for the symbol; its device address, which
// differs from device to device, comes from hipGetSymbolAddress, taken once
// per device on the first call made with that device current, and only that
// address is ever handed to a kernel.  The first call on a device also
// clears the array with a fill kernel on the caller's stream (no memset
// node, so the call may be captured); from then on every completed call
// leaves the counters at zero for the next, whatever its shape.  All calls
// on one device share the array, so calls that can overlap in time on one
// device race; calls ordered on one stream are fine.

#include "q8narrow.h"
#include "q8_internal.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = Q8_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 16 == 0, "the fill kernel clears 16-byte units");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void* ptr = nullptr;  // device address of `scratch` on this device
    bool cleared = false;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

__global__ void __launch_bounds__(256) clear_scratch_kernel(uint4* p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// This device's scratch address, the array cleared on `st` before first use.
// Returns hipSuccess or the failing call's error.
hipError_t device_scratch(hipStream_t st, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch& d = g_dev[dev];
    if (d.ptr == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        d.ptr = p;
    }
    if (!d.cleared) {
        hipLaunchKernelGGL(clear_scratch_kernel, dim3(512), dim3(256), 0, st,
                           static_cast<uint4*>(d.ptr), (int64_t)(kScratchBytes / 16));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        d.cleared = true;
    }
    *out = d.ptr;
    return hipSuccess;
}

}  // namespace

extern "C" {

q8_status q8_matmul_narrow_noalloc(const void* Wq, const void* Xq,
                                   const int32_t* batch_index, int n_live, int64_t N,
                                   int64_t K, float* Y, hipStream_t stream) {
    if (!q8::matmul_args_ok(Wq, Xq, batch_index, n_live, N, K, Y)) return Q8_ERR_INVALID_ARG;
    const q8::Shape s = q8::make_shape(N, K);
    const q8::Tiling t = q8::choose_tiling(s);
    const size_t need = q8::workspace_bytes(s, t);
    if (need > kScratchBytes) return Q8_ERR_TOO_LARGE;
    if (!q8_device_supported()) return Q8_ERR_UNSUPPORTED;
    void* ws = nullptr;  // shapes that are not split need none
    if (need > 0 && device_scratch(stream, &ws) != hipSuccess) return Q8_ERR_HIP;
    const hipError_t e = q8::launch_matmul(q8::Engine::kMfma, static_cast<const uint8_t*>(Wq),
                                           static_cast<const uint8_t*>(Xq), Q8_MAX_SLOTS,
                                           batch_index, n_live, s, t, Y, ws, stream);
    return e == hipSuccess ? Q8_OK : Q8_ERR_HIP;
}

}  // extern "C"
