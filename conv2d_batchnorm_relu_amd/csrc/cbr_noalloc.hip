// cbr_noalloc.hip -- the training forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the same kernels as cbr_forward_train, with their scratch in a fixed-size array that
// the library holds on each device for the life of the process instead of a caller
// workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/cbr.h"

namespace {

// The scratch array.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[CBR_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
void *scratch_addr[MAX_DEVICES];   // device address of `scratch` on each device, once looked up
std::mutex scratch_mu;

// Device address of the current device's scratch array (looked up on the first call made
// with that device current).
int device_scratch(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return CBR_E_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CBR_E_HIP;
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return CBR_OK;
}

}  // namespace

extern "C" int cbr_forward_train_noalloc(const cbr_shape *shape, const uint16_t *x, const uint16_t *w,
                                         const float *gamma, const float *beta, const float *run_mean_in,
                                         const float *run_var_in, float eps, float momentum, uint16_t *z,
                                         uint16_t *y, uint32_t *relu_mask, float *saved_mean, float *saved_invstd,
                                         float *run_mean_out, float *run_var_out, void *stream)
{
    const int st = cbr_output_hw(shape, nullptr, nullptr);
    if (st != CBR_OK) return st;
    if (cbr_workspace_bytes(shape, CBR_OP_TRAIN) > (size_t)CBR_NOALLOC_SCRATCH_BYTES) return CBR_E_WORKSPACE;
    void *ws = nullptr;
    const int sst = device_scratch(&ws);
    if (sst != CBR_OK) return sst;
    // Every kernel writes the scratch areas it reads before reading them (statistics
    // rows, including the rows of empty chunks, the finalize's coefficients, the widened
    // first-layer filter), so nothing left by an earlier call is ever read.
    return cbr_forward_train(shape, x, w, gamma, beta, run_mean_in, run_var_in, eps, momentum, z, y, relu_mask,
                             saved_mean, saved_invstd, run_mean_out, run_var_out, ws,
                             (size_t)CBR_NOALLOC_SCRATCH_BYTES, stream);
}
