// hbm_read.hip -- a plain streaming read of a device buffer, timed on the GPU: the
// practical HBM read rate for a given byte count, against which the expert stream kernels
// are compared (include/moe_prof.h, moe_prof_hbm_read).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "common.h"
#include "moe_prof.h"

namespace moe {

// Where a read result would be stored (never in practice).
__device__ uint32_t g_hbm_sink;

// 16 bytes per lane, two independent loads per thread and iteration, grid-stride over the
// buffer; the XOR of everything read is stored only if it equals a constant, so the loads
// cannot be dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void k_hbm_read(const u32x4 *__restrict__ p, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += 2 * stride) {
        const u32x4 a = p[i];
        const u32x4 b = p[min(i + stride, n16 - 1)];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    }
    if (acc == 0x9E3779B9u) g_hbm_sink = acc;
}

}  // namespace moe

extern "C" moe_status moe_prof_hbm_read(const void *buf, size_t bytes, void *stream, double *ms)
{
    if (!buf || !ms || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15)) return MOE_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return MOE_ERR_DEVICE;
    }
    hipExtLaunchKernelGGL(moe::k_hbm_read, dim3(2048), dim3(256), 0, s, e0, e1, 0, (const moe::u32x4 *)buf, bytes / 16);
    hipError_t err = hipGetLastError();
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    float t = 0.f;
    if (err == hipSuccess) err = hipEventElapsedTime(&t, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (err != hipSuccess) return MOE_ERR_DEVICE;
    *ms = t;
    return MOE_OK;
}
