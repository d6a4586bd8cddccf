// quant.hip -- MXFP8 quantization of the expert input (activation-quantized prefill).
//
// OCP Microscaling Formats (MX) v1.0: blocks of 32 consecutive elements share an E8M0
// scale 2^s with s = floor(log2 max|v|) - 8 (8 = the largest exponent of the E4M3
// element), clamped to [-127, 127]; each element becomes v / 2^s rounded to the nearest
// E4M3 value (ties to even) and saturated at 448.  The represented value q 2^s has at
// most 4 significant bits, so it is stored exactly as bf16 and every expert kernel
// consumes it as an ordinary bf16 token row.
#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Nearest E4M3 magnitude of a >= 0 (exact fp32 arithmetic: the binade's step is a power of
// two, rintf rounds half to even), saturated at 448.
__device__ __forceinline__ float round_e4m3(float a)
{
    if (a == 0.f) return 0.f;
    int ex;
    frexpf(a, &ex);  // a in [2^(ex-1), 2^ex)
    const int e = max(ex - 1, -6) - 3;
    return fminf(ldexpf(rintf(ldexpf(a, -e)), e), 448.f);
}

template <int XT>
__device__ __forceinline__ float ld_x(const void *x, size_t i)
{
    if constexpr (XT == DT_BF16) return bf16_bits_to_f32(((const uint16_t *)x)[i]);
    return ((const float *)x)[i];
}

// One thread per 32-element block.
template <int XT>
__global__ __launch_bounds__(256) void k_quant_x8(const void *__restrict__ x, size_t nblk, uint16_t *__restrict__ xq)
{
    const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblk) return;
    float v[32], amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        v[i] = ld_x<XT>(x, 32 * b + i);
        amax = fmaxf(amax, fabsf(v[i]));
    }
    int s = -127;
    if (amax > 0.f) {
        int ex;
        frexpf(amax, &ex);
        s = min(max(ex - 1 - 8, -127), 127);
    }
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        const float q0 = copysignf(round_e4m3(fabsf(ldexpf(v[i], -s))), v[i]);
        const float q1 = copysignf(round_e4m3(fabsf(ldexpf(v[i + 1], -s))), v[i + 1]);
        // q 2^s has at most 4 significant bits: its bf16 bits are the top half of the fp32 bits
        o[i / 2] = (__float_as_uint(ldexpf(q0, s)) >> 16) | (__float_as_uint(ldexpf(q1, s)) & 0xFFFF0000u);
    }
    u32x4 *dst = (u32x4 *)(xq + 32 * b);
#pragma unroll
    for (int c = 0; c < 4; c++) dst[c] = u32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
}

}  // namespace

hipError_t launch_quant_x8(const void *x, int xt, size_t n, uint16_t *xq, hipStream_t s)
{
    const size_t nblk = n / 32;
    if (nblk == 0) return hipSuccess;
    const dim3 grid((unsigned)((nblk + 255) / 256));
    if (xt == DT_BF16)
        hipLaunchKernelGGL(k_quant_x8<DT_BF16>, grid, dim3(256), 0, s, x, nblk, xq);
    else
        hipLaunchKernelGGL(k_quant_x8<DT_F32>, grid, dim3(256), 0, s, x, nblk, xq);
    return hipGetLastError();
}

}  // namespace moe
