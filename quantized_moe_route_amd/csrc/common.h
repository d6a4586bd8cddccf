// common.h -- device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { FMT_MXFP4 = 0, FMT_RVQ3 = 1 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Split an fp32 value into bf16 hi + lo with hi = rne(f), lo = rne(f - hi).
// |f - (hi + lo)| <= 2^-18 |f|.
__device__ __forceinline__ void split_bf16(float f, uint32_t &hi, uint32_t &lo)
{
    hi = f32_to_bf16_rne(f);
    lo = f32_to_bf16_rne(f - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xFFFFu) | (hi16 << 16); }

// E8M0 scale byte -> fp32 power of two (bytes 1..254 are normal fp32 numbers).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __uint_as_float(b << 23); }

// 32 E2M1 codes (16 bytes, low nibble = even element) times a power-of-two scale,
// converted to 32 bf16 (exact: E2M1 values have at most two significant bits and
// the scales used are normal numbers).  out[d] packs elements 2d (low half) and 2d+1.
__device__ __forceinline__ void decode_fp4x32(u32x4 c, float scale, uint32_t out[16])
{
#pragma unroll
    for (int d = 0; d < 4; d++) {
        bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 0);
        bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 1);
        bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 2);
        bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 3);
        out[4 * d + 0] = __builtin_bit_cast(uint32_t, v0);
        out[4 * d + 1] = __builtin_bit_cast(uint32_t, v1);
        out[4 * d + 2] = __builtin_bit_cast(uint32_t, v2);
        out[4 * d + 3] = __builtin_bit_cast(uint32_t, v3);
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies A row l%16 and
// B column l%16 over the same 8 reduction indices (group l/16); it receives
// D rows 4*(l/16)+0..3 of column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Butterfly reductions over a 64-lane wave; every lane receives a result, and
// lane 0's result is the one callers keep (the association order is fixed).
__device__ __forceinline__ float wave_sum_f32(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_min_f32(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

}  // namespace moe
