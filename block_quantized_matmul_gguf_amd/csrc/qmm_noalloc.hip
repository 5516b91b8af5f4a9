// qmm_noalloc.hip -- qmatmul_run_noalloc: y = x . W^T without a plan and
// without any device allocation, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace that qmatmul_create would allocate (split-K partials,
// prepared or quantized activations, scales) is laid out instead in one
// file-scope device array, `scratch`, of QMM_NOALLOC_SCRATCH_BYTES.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in symbol): on the first call on a device, with that device current,
// hipGetSymbolAddress gives the device address of that device's copy, which is
// kept per device and is what the kernels receive.
//
// Every region of the workspace is written by a call before that call reads
// it, so nothing needs clearing between calls.  All calls on one GPU share the
// array: calls that overlap on one GPU (two streams, or two host threads) race
// on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qmatmul.h"
#include "qmm_internal.h"

static __device__ __align__(256) uint8_t scratch[QMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's address of `scratch`, looked up once per device.
int scratch_address(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return qmm::set_error(QMM_EHIP, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return qmm::set_error(QMM_EUNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return qmm::set_error(QMM_EHIP, e != hipSuccess ? hipGetErrorString(e)
                                                            : "hipGetSymbolAddress returned a null address");
        }
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return QMM_OK;
}

}  // namespace

extern "C" int qmatmul_run_noalloc(int format, int64_t N, int64_t K, int64_t M, int mode, const void* w_blocks,
                                   const float* x, float* y, void* stream)
{
    void* ws = nullptr;
    // validate everything that needs no device first, so errors come without a GPU
    int st = qmm::run_on_scratch(format, N, K, M, mode, w_blocks, x, y, nullptr, QMM_NOALLOC_SCRATCH_BYTES, nullptr,
                                 /*dry_run=*/true);
    if (st != QMM_OK || M == 0) return st;
    st = scratch_address(&ws);
    if (st != QMM_OK) return st;
    return qmm::run_on_scratch(format, N, K, M, mode, w_blocks, x, y, ws, QMM_NOALLOC_SCRATCH_BYTES, stream, false);
}
