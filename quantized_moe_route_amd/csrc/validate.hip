// validate.hip -- device checks of MOE_F_VALIDATE (include/moe.h).
//
// LazyLoRA README, "Three rules the engine is built around": data that is missing or
// unusable is an error and is never replaced by something else.  With the flag, every
// call first scans what it is about to consume and ORs a bit into a status word in the
// layer's workspace for each kind of out-of-contract value it finds: non-finite
// activations or upstream gradients, E8M0 scale bytes 0xFF (NaN in the format) and 0x00
// (2^-127, below the range whose products the kernels carry exactly), non-finite RVQ3
// codewords.  The kernels that follow still run to completion on whatever they are given;
// the host reports the word as an error at the next call (moe_api.hip).
#include <algorithm>

#include "common.h"
#include "moe.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Every lane of the wave takes part (called after the loops); one atomic per wave.
__device__ __forceinline__ void report(uint32_t *status, uint32_t bits)
{
    bits |= __shfl_xor(bits, 1);
    bits |= __shfl_xor(bits, 2);
    bits |= __shfl_xor(bits, 4);
    bits |= __shfl_xor(bits, 8);
    bits |= __shfl_xor(bits, 16);
    bits |= __shfl_xor(bits, 32);
    if ((threadIdx.x & 63) == 0 && bits) atomicOr(status, bits);
}

__device__ __forceinline__ bool has_zero_byte(uint32_t w) { return ((w - 0x01010101u) & ~w & 0x80808080u) != 0; }

// n16 16-byte chunks of bf16 or fp32 values; all-ones exponent = Inf or NaN.
__global__ __launch_bounds__(256) void k_check_finite(const u32x4 *__restrict__ p, int dt, size_t n16,
                                                      uint32_t *__restrict__ status, uint32_t bit)
{
    uint32_t bad = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = p[i];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t w = v[j];
            const bool hi = (w & 0x7F800000u) == 0x7F800000u;
            const bool lo = dt == DT_BF16 && (w & 0x7F80u) == 0x7F80u;
            if (hi || lo) bad = bit;
        }
    }
    report(status, bad);
}

// Scale bytes (MXFP4) or codebooks (RVQ3) of the experts a call is about to read: unit u of
// blockIdx.y is expert active[u] (u < *n_active), or expert u itself when dense.
struct CheckW {
    const uint8_t *scales[3];  // [E][rows][cols/32] bytes
    size_t scale_bytes[3];     // per expert, a multiple of 16
    const uint16_t *cb[3];     // [E][3][256][8] fp16
    int wfmt;
    const int32_t *active, *n_active;  // null: dense
    uint32_t *status;
};

__global__ __launch_bounds__(256) void k_check_weights(const CheckW a)
{
    const int u = blockIdx.y;
    int e = u;
    if (a.active) {
        if (u >= *a.n_active) return;
        e = a.active[u];
    }
    uint32_t bad = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x, gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int m = 0; m < 3; m++) {
        if (a.wfmt == FMT_MXFP4) {
            const u32x4 *p = (const u32x4 *)(a.scales[m] + (size_t)e * a.scale_bytes[m]);
            const size_t n16 = a.scale_bytes[m] / 16;
            for (size_t i = gid; i < n16; i += stride) {
                const u32x4 v = p[i];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    if (has_zero_byte(~v[j])) bad |= MOE_BAD_SCALE_NAN;
                    if (has_zero_byte(v[j])) bad |= MOE_BAD_SCALE_ZERO;
                }
            }
        } else {
            const u32x4 *p = (const u32x4 *)(a.cb[m] + (size_t)e * 3 * 256 * 8);
            const size_t n16 = (size_t)3 * 256 * 8 * 2 / 16;
            for (size_t i = gid; i < n16; i += stride) {
                const u32x4 v = p[i];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if ((v[j] & 0x7C00u) == 0x7C00u || (v[j] & 0x7C000000u) == 0x7C000000u) bad |= MOE_BAD_CODEWORD;
            }
        }
    }
    report(a.status, bad);
}

__global__ void k_set_u32(uint32_t *p, uint32_t v) { *p = v; }

unsigned blocks16(size_t n16) { return (unsigned)std::max<size_t>(1, std::min<size_t>(2048, (n16 + 255) / 256)); }

}  // namespace

hipError_t launch_check_finite(const void *p, int dt, size_t n, uint32_t *status, uint32_t bit, hipStream_t s)
{
    const size_t n16 = n * (dt == DT_BF16 ? 2 : 4) / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(k_check_finite, dim3(blocks16(n16)), dim3(256), 0, s, (const u32x4 *)p, dt, n16, status, bit);
    return hipGetLastError();
}

hipError_t launch_check_weights(int wfmt, const MatW (&m)[3], const size_t (&scale_bytes)[3], const int32_t *active,
                                const int32_t *n_active, int units, uint32_t *status, hipStream_t s)
{
    if (units <= 0) return hipSuccess;
    CheckW a{};
    size_t per = 0;
    for (int i = 0; i < 3; i++) {
        a.scales[i] = m[i].scales;
        a.scale_bytes[i] = scale_bytes[i];
        a.cb[i] = m[i].cb;
        per = std::max(per, wfmt == FMT_MXFP4 ? scale_bytes[i] / 16 : (size_t)3 * 256 * 8 * 2 / 16);
    }
    a.wfmt = wfmt;
    a.active = active;
    a.n_active = n_active;
    a.status = status;
    const unsigned bx = (unsigned)std::max<size_t>(1, std::min<size_t>(64, (per + 255) / 256));
    hipLaunchKernelGGL(k_check_weights, dim3(bx, units), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_set_u32(uint32_t *p, uint32_t v, hipStream_t s)
{
    hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, s, p, v);
    return hipGetLastError();
}

}  // namespace moe
