// w4a16_linear for callers that cannot allocate device memory (code under
// HIP graph capture, fixed serving loops, harnesses that forbid hipMalloc):
// the same argument checks, kernels and results as w4a16_linear, with the
// workspace in a file-scope device array of fixed size instead of a caller
// buffer.
//
// The array (`scratch`) exists once per GPU the library runs on, for the
// life of the process.  On the host its name is only a stand-in for the
// symbol, never a device address: the address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept per device, and only that pointer is ever handed to a kernel.
//
// Contents: the first kSyncBytes are the zero header of exchange slots
// (every call leaves it zero again); the rest holds FP32 partial sums, which
// need no initialisation.  The array is zero when the code object loads, and
// the first call on a device also clears the header with a kernel on the
// caller's stream.  All calls on one GPU share its array: calls that may run
// at the same time on one GPU (other streams, other threads) race on it.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "w4a16.h"

namespace {

using namespace w4a16;

constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > kSyncBytes && kScratchBytes % 256 == 0, "scratch holds the header and partials");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up
bool g_cleared[kMaxDevices];   // its header cleared by a kernel on that device

__global__ void clear_header_kernel(uint4* p, int64_t n16) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address (looked up on its first use).
w4a16_status_t scratch_address(int* device, void** ptr) {
    if (hipGetDevice(device) != hipSuccess) return W4A16_EHIP;
    if (*device < 0 || *device >= kMaxDevices) return W4A16_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[*device]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4A16_EHIP;
        g_scratch[*device] = p;
    }
    *ptr = g_scratch[*device];
    return W4A16_OK;
}

// Clears the header once per device, on the caller's stream (a kernel, not
// a memset, so it is also safe inside a captured graph).
w4a16_status_t clear_once(int device, void* ptr, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_cleared[device]) return W4A16_OK;
    clear_header_kernel<<<dim3(64), dim3(256), 0, stream>>>(static_cast<uint4*>(ptr), int64_t(kSyncBytes / 16));
    if (hipGetLastError() != hipSuccess) return W4A16_EHIP;
    g_cleared[device] = true;
    return W4A16_OK;
}

}  // namespace

extern "C" {

w4a16_status_t w4a16_linear_noalloc(const void* x, w4a16_dtype_t act_dtype, int64_t m, int64_t k, int64_t ldx,
                                    const void* packed, int64_t n, const void* bias, void* y, int64_t ldy,
                                    void* stream) {
    int device = 0;
    void* ws = nullptr;
    w4a16_status_t st = scratch_address(&device, &ws);
    if (st != W4A16_OK) return st;
    // every argument check (and the workspace limit) before anything is launched
    st = check_linear(x, act_dtype, m, k, ldx, packed, n, bias, y, ldy, ws, kScratchBytes);
    if (st != W4A16_OK || m == 0 || n == 0) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = clear_once(device, ws, s);
    if (st != W4A16_OK) return st;
    return w4a16_linear(x, act_dtype, m, k, ldx, packed, n, bias, y, ldy, ws, kScratchBytes, stream);
}

}  // extern "C"
