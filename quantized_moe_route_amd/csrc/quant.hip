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

// One thread per 32-element block (block b = row t, block q of the row).  With mxq, the
// E4M3 codes and the E8M0 scale byte also go to the block-scaled gate/up's operand layout
// (the first of its two terms: row t's bytes of K-step q / 4 at t 2H + 256 (q / 4) +
// 32 (q % 4), the scale as byte 0 of the block's 16-bit pair; the second term is not
// read when x arrives quantized).
template <int XT>
__global__ __launch_bounds__(256) void k_quant_x8(const void *__restrict__ x, size_t nblk, int H, uint16_t *__restrict__ xq,
                                                  uint8_t *__restrict__ mxq, uint8_t *__restrict__ mxs)
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
    if (mxq) {
        const int nb = H / 32;
        const size_t t = b / nb;
        const int qb = (int)(b - t * nb);
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
            // the values q lie on the E4M3 grid: the conversion is exact
            const float q0 = copysignf(round_e4m3(fabsf(ldexpf(v[i], -s))), v[i]);
            const float q1 = copysignf(round_e4m3(fabsf(ldexpf(v[i + 1], -s))), v[i + 1]);
            const float q2 = copysignf(round_e4m3(fabsf(ldexpf(v[i + 2], -s))), v[i + 2]);
            const float q3 = copysignf(round_e4m3(fabsf(ldexpf(v[i + 3], -s))), v[i + 3]);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false) & 0xFFFFu;
            const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, 0, false) & 0xFFFFu;
            w[i / 4] = lo | (hi << 16);
        }
        uint8_t *d = mxq + t * (size_t)(2 * H) + (size_t)(qb >> 2) * 256 + 32 * (qb & 3);
        *(u32x4 *)d = u32x4{w[0], w[1], w[2], w[3]};
        *(u32x4 *)(d + 16) = u32x4{w[4], w[5], w[6], w[7]};
        mxs[2 * b] = (uint8_t)(s + 127);
    }
}

}  // namespace

hipError_t launch_quant_x8(const void *x, int xt, int T, int H, uint16_t *xq, uint8_t *mxq, uint8_t *mxs, hipStream_t s)
{
    const size_t nblk = (size_t)T * (H / 32);
    if (nblk == 0) return hipSuccess;
    const dim3 grid((unsigned)((nblk + 255) / 256));
    if (xt == DT_BF16)
        hipLaunchKernelGGL(k_quant_x8<DT_BF16>, grid, dim3(256), 0, s, x, nblk, H, xq, mxq, mxs);
    else
        hipLaunchKernelGGL(k_quant_x8<DT_F32>, grid, dim3(256), 0, s, x, nblk, H, xq, mxq, mxs);
    return hipGetLastError();
}

}  // namespace moe
