// expert_frag.h -- MFMA operand fragments for the expert kernels (gfx950).
//
// A wave computes a 16 (weight rows) x 16 (tokens) tile with
// v_mfma_f32_16x16x32_bf16.  Per 256-wide step of the reduction dimension,
// lane l (row l%16, group g = l/16) owns reduction indices [k0 + 64g, k0 + 64g + 64):
// eight MFMA sub-steps s take indices k0 + 64g + 8s + 0..7 from both the
// weight fragment (A) and the token fragment (B), so every sub-step pairs the
// same reduction indices on both sides.  For MXFP4 one lane's 64 indices are
// exactly two 32-element scale blocks = 32 contiguous code bytes.
#pragma once

#include "common.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- weights

template <int WFMT>
struct AFrag;

// MXFP4: exact bf16 dequantization (E2M1 value times a power-of-two scale).
template <>
struct AFrag<FMT_MXFP4> {
    static constexpr bool kTwo = false;
    bf16x8 hi[8];
    bf16x8 lo[1];
    __device__ __forceinline__ void load(const MatW &W, int e, int rows, int cols, int row, int kk,
                                         const uint16_t *)
    {
        const size_t r = (size_t)e * rows + row;
        const uint8_t *c = W.codes + r * (size_t)(cols / 2);
        const uint8_t *sc = W.scales + r * (size_t)(cols / 32);
        u32x4 c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
        float s0 = 1.f, s1 = 1.f;
        if (kk < cols) {
            c0 = *(const u32x4 *)(c + kk / 2);
            s0 = e8m0_to_f32(sc[kk / 32]);
        }
        if (kk + 32 < cols) {
            c1 = *(const u32x4 *)(c + kk / 2 + 16);
            s1 = e8m0_to_f32(sc[kk / 32 + 1]);
        }
        uint32_t d[32];
        decode_fp4x32(c0, s0, d);
        decode_fp4x32(c1, s1, d + 16);
#pragma unroll
        for (int s = 0; s < 8; s++) hi[s] = as_bf16x8(d[4 * s], d[4 * s + 1], d[4 * s + 2], d[4 * s + 3]);
    }
};

// RVQ3: each 8-element vector is the sum of three fp16 codewords read from the
// block's LDS copy of this matrix's codebooks ([3][256][8] fp16).  The fp32 sum
// is split into bf16 hi + lo (|w - hi - lo| <= 2^-18 |w|).
template <>
struct AFrag<FMT_RVQ3> {
    static constexpr bool kTwo = true;
    bf16x8 hi[8];
    bf16x8 lo[8];
    __device__ __forceinline__ void load(const MatW &W, int e, int rows, int cols, int row, int kk,
                                         const uint16_t *cb)
    {
        uint32_t i0[3], i1[3];
#pragma unroll
        for (int st = 0; st < 3; st++) {
            const uint8_t *ip = W.idx + (((size_t)e * 3 + st) * rows + row) * (size_t)(cols / 8) + kk / 8;
            i0[st] = kk < cols ? *(const uint32_t *)ip : 0u;
            i1[st] = kk + 32 < cols ? *(const uint32_t *)(ip + 4) : 0u;
        }
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const bool valid = kk + 32 * (s / 4) < cols;
            float v[8];
#pragma unroll
            for (int d = 0; d < 8; d++) v[d] = 0.f;
#pragma unroll
            for (int st = 0; st < 3; st++) {
                const uint32_t word = s < 4 ? i0[st] : i1[st];
                const uint32_t id = (word >> (8 * (s & 3))) & 0xFFu;
                const u32x4 cw = *(const u32x4 *)(cb + ((size_t)st * 256 + id) * 8);
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    v[2 * d] += (float)__builtin_bit_cast(_Float16, (uint16_t)(cw[d] & 0xFFFFu));
                    v[2 * d + 1] += (float)__builtin_bit_cast(_Float16, (uint16_t)(cw[d] >> 16));
                }
            }
            uint32_t h[8], l[8];
#pragma unroll
            for (int d = 0; d < 8; d++) split_bf16(valid ? v[d] : 0.f, h[d], l[d]);
            hi[s] = as_bf16x8(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
            lo[s] = as_bf16x8(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
        }
    }
};

// Copy one expert's codebooks of matrix W ([3][256][8] fp16 = 12 KB) to LDS.
__device__ __forceinline__ void load_codebooks(const MatW &W, int e, uint16_t *dst)
{
    const u32x4 *src = (const u32x4 *)(W.cb + (size_t)e * 3 * 256 * 8);
    u32x4 *d = (u32x4 *)dst;
    for (int i = threadIdx.x; i < 3 * 256 * 8 / 8; i += blockDim.x) d[i] = src[i];
}

// ---------------------------------------------------------------- tokens

template <int DT>
struct BFrag;

// bf16 rows are exact bf16 operands.
template <>
struct BFrag<DT_BF16> {
    static constexpr bool kTwo = false;
    bf16x8 hi[8];
    bf16x8 lo[1];
    __device__ __forceinline__ void load(const void *src, size_t rowoff, int kk, int K, bool valid)
    {
        const uint16_t *p = (const uint16_t *)src + rowoff + kk;
#pragma unroll
        for (int s = 0; s < 8; s++) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (valid && kk + 32 * (s / 4) < K) v = *(const u32x4 *)(p + 8 * s);
            hi[s] = as_bf16x8(v);
        }
    }
};

// fp32 rows are split into bf16 hi + lo.
template <>
struct BFrag<DT_F32> {
    static constexpr bool kTwo = true;
    bf16x8 hi[8];
    bf16x8 lo[8];
    __device__ __forceinline__ void load(const void *src, size_t rowoff, int kk, int K, bool valid)
    {
        const float *p = (const float *)src + rowoff + kk;
#pragma unroll
        for (int s = 0; s < 8; s++) {
            float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            if (valid && kk + 32 * (s / 4) < K) {
                a = *(const float4 *)(p + 8 * s);
                b = *(const float4 *)(p + 8 * s + 4);
            }
            const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t h[8], l[8];
#pragma unroll
            for (int d = 0; d < 8; d++) split_bf16(f[d], h[d], l[d]);
            hi[s] = as_bf16x8(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
            lo[s] = as_bf16x8(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
        }
    }
};

// acc += A * B over the 8 sub-steps; the lo x lo product (below 2^-36 relative) is dropped.
template <class A, class B>
__device__ __forceinline__ void mma_step(f32x4 &acc, const A &a, const B &b)
{
#pragma unroll
    for (int s = 0; s < 8; s++) {
        acc = mfma16(a.hi[s], b.hi[s], acc);
        if constexpr (A::kTwo) acc = mfma16(a.lo[s], b.hi[s], acc);
        if constexpr (B::kTwo) acc = mfma16(a.hi[s], b.lo[s], acc);
    }
}

}  // namespace moe
