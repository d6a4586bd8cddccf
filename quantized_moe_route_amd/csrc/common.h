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

// Split an fp32 value into three bf16 terms hi = rne(f), mid = rne(f - hi), lo = f - hi - mid.
// Each residual is exact in fp32, and for a normal f the last one has at most 8 significant
// bits, so hi + mid + lo == f exactly (bf16 keeps fp32's exponent range).
__device__ __forceinline__ void split_bf16x3(float f, uint32_t &hi, uint32_t &mid, uint32_t &lo)
{
    hi = f32_to_bf16_rne(f);
    const float r1 = f - bf16_bits_to_f32(hi);
    mid = f32_to_bf16_rne(r1);
    lo = f32_to_bf16_rne(r1 - bf16_bits_to_f32(mid));
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

// ---------------------------------------------------------------- wave reductions
//
// Reductions over the 64 lanes of a wave, built from DPP lane permutations within
// each 16-lane row (quad xor 1, quad xor 2, half-row mirror, row mirror) and four
// readlanes across the rows.  Each step combines a lane with its partner by a
// commutative operation, so every lane of a row holds the same value, and the
// cross-row combine runs on wave-uniform values: every lane receives the same
// result, computed in a fixed association order.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, lo | (hi << 32));
}

__device__ __forceinline__ float readlane_f32(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, lo | (hi << 32));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

__device__ __forceinline__ float wave_sum_f32(float v)
{
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

// Sum with a rigorous bound on its rounding error: on entry eb bounds this lane's
// accumulated error (in units of the unit roundoff), on exit it bounds the result's.
// Each add contributes at most u |result| (round to nearest), so the bound follows
// the same tree: eb = eb_a + eb_b + |a + b|.
__device__ __forceinline__ float wave_sum_f32_eb(float v, float &eb)
{
#define MOE_SUM_EB_STEP(C)                    \
    {                                         \
        const float pv = dpp_f32<C>(v);       \
        const float pe = dpp_f32<C>(eb);      \
        v += pv;                              \
        eb = eb + pe + fabsf(v);              \
    }
    MOE_SUM_EB_STEP(kDppXor1)
    MOE_SUM_EB_STEP(kDppXor2)
    MOE_SUM_EB_STEP(kDppHalfMirror)
    MOE_SUM_EB_STEP(kDppMirror)
#undef MOE_SUM_EB_STEP
    const float a = readlane_f32(v, 0), b = readlane_f32(v, 16), c = readlane_f32(v, 32), d = readlane_f32(v, 48);
    const float ea = readlane_f32(eb, 0), eb1 = readlane_f32(eb, 16), ec = readlane_f32(eb, 32), ed = readlane_f32(eb, 48);
    const float ab = a + b, cd = c + d, r = ab + cd;
    eb = ((ea + eb1) + fabsf(ab)) + ((ec + ed) + fabsf(cd)) + fabsf(r);
    return r;
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
    v += dpp_f64<kDppXor1>(v);
    v += dpp_f64<kDppXor2>(v);
    v += dpp_f64<kDppHalfMirror>(v);
    v += dpp_f64<kDppMirror>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ float wave_min_f32(float v)
{
    v = fminf(v, dpp_f32<kDppXor1>(v));
    v = fminf(v, dpp_f32<kDppXor2>(v));
    v = fminf(v, dpp_f32<kDppHalfMirror>(v));
    v = fminf(v, dpp_f32<kDppMirror>(v));
    return fminf(fminf(readlane_f32(v, 0), readlane_f32(v, 16)), fminf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ float wave_max_f32(float v)
{
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// The gated activation of the experts, h = act(g, u) (values match the API's moe_act):
//   SwiGLU: h = g sigmoid(g) u;
//   SiTU (LazyLoRA README, "File map"): h = A(g) B(u), A(g) = 4 tanh(g/4) sigmoid(g),
//   B(u) = 25 tanh(u/25).
enum { ACT_SWIGLU = 0, ACT_SITU = 1 };

__device__ __forceinline__ float act_h(int act, float g, float u)
{
    if (act == ACT_SITU) return 4.f * tanhf(0.25f * g) * sigmoidf_(g) * (25.f * tanhf(u * (1.f / 25.f)));
    return g * sigmoidf_(g) * u;
}

// sech^2(z) = 4 e / (1 + e)^2 with e = exp(-2 |z|): no cancellation where tanh(z) nears 1
// (1 - tanh^2 in fp32 would lose ~eps / sech^2 relative accuracy there).
__device__ __forceinline__ float sech2f_(float z)
{
    const float e = __expf(-2.f * fabsf(z)), d = 1.f + e;
    return 4.f * e / (d * d);
}

// h and its partial derivatives: SwiGLU dh/dg = u s (1 + g (1 - s)), dh/du = g s (s = sigmoid(g));
// SiTU dh/dg = (sech^2(g/4) s + 4 tanh(g/4) s (1 - s)) B(u), dh/du = A(g) sech^2(u/25).
__device__ __forceinline__ void act_grad(int act, float g, float u, float &h, float &dhdg, float &dhdu)
{
    const float s = sigmoidf_(g);
    if (act == ACT_SITU) {
        const float zg = 0.25f * g, zu = u * (1.f / 25.f);
        const float tg = tanhf(zg), tu = tanhf(zu);
        const float A = 4.f * tg * s, B = 25.f * tu;
        h = A * B;
        dhdg = (sech2f_(zg) * s + 4.f * tg * s * (1.f - s)) * B;
        dhdu = A * sech2f_(zu);
        return;
    }
    const float silu = g * s;
    h = silu * u;
    dhdg = u * s * (1.f + g * (1.f - s));
    dhdu = silu;
}

// The adapter's per-token gate/up terms (lgu [T][2I], or null) for I-columns n..n+3 of
// the token of grouped row rr, added to g and u before the activation.
__device__ __forceinline__ void add_lora_gu(const float *lgu, const int32_t *perm, int k, size_t rr, int I, int n, f32x4 &g,
                                            f32x4 &u)
{
    if (!lgu) return;
    const float *p = lgu + (size_t)(perm[rr] / k) * 2 * I + n;
    const float4 dg = *(const float4 *)p, du = *(const float4 *)(p + I);
    g += f32x4{dg.x, dg.y, dg.z, dg.w};
    u += f32x4{du.x, du.y, du.z, du.w};
}

// Exclusive scan of one int per thread over the block (scr: blockDim.x ints of LDS);
// returns the total in *total.  Called by every thread of the block.
__device__ __forceinline__ int block_exclusive_scan(int v, int *scr, int *total)
{
    const int tid = threadIdx.x, n = blockDim.x;
    scr[tid] = v;
    __syncthreads();
    for (int off = 1; off < n; off <<= 1) {
        const int add = tid >= off ? scr[tid - off] : 0;
        __syncthreads();
        scr[tid] += add;
        __syncthreads();
    }
    const int incl = scr[tid];
    *total = scr[n - 1];
    __syncthreads();
    return incl - v;
}

}  // namespace moe
