// The allocation-free form of mxfp4_linear_fprop, for callers that cannot call hipMalloc (code
// under HIP graph capture, tight serving loops, harnesses that forbid allocation). Its workspace
// (the two quantized operands and any split-K partials) is a file-scope device array that every
// GPU the library runs on holds until the process ends.
#include <atomic>

#include "../../include/mxfp4.h"
#include "internal.h"

namespace {

static_assert(MXFP4_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte lines");

// one copy per device, each at its own device address
static __device__ __align__(256) uint8_t scratch[MXFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up once per device with that
// device current (the host-side name of the array is not a device address). nullptr on failure.
uint8_t *scratch_on_current_device()
{
    static std::atomic<uint8_t *> addr[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    uint8_t *p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    addr[dev].store(static_cast<uint8_t *>(q), std::memory_order_release);
    return static_cast<uint8_t *>(q);
}

}  // namespace

extern "C" mxfp4_status_t mxfp4_linear_fprop_noalloc(const void *x_bf16, const void *w_bf16, int64_t M, int64_t K,
                                                     int64_t N, const mxfp4_linear_cfg_t *cfg, float *y,
                                                     void *stream)
{
    // the size check first: nothing is looked up or launched for a product whose workspace
    // exceeds the array (0 also covers negative or oversized dimensions)
    const size_t need = mxfp4_linear_workspace_bytes(MXFP4_FPROP, M, K, N);
    if (M < 0 || K < 0 || N < 0) return MXFP4_ERR_SHAPE;
    if (need > (size_t)MXFP4_NOALLOC_SCRATCH_BYTES) return MXFP4_ERR_WORKSPACE;
    if (need == 0 && M > 0 && K > 0 && N > 0) return MXFP4_ERR_SHAPE;
    uint8_t *ws = scratch_on_current_device();
    if (!ws) return MXFP4_ERR_DEVICE;
    // the Fprop path writes every byte it later reads (codes and scales of both operands, and each
    // split's partials), so the array's contents from an earlier call need no clearing
    return mxfp4_linear_fprop(x_bf16, w_bf16, M, K, N, cfg, ws, (size_t)MXFP4_NOALLOC_SCRATCH_BYTES, y, stream);
}
