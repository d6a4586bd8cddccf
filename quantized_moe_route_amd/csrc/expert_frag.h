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
//
// Weight fragments are produced in two steps so the kernels can keep several
// K-steps of raw bytes in flight: fetch() issues this lane's global loads for one
// 256-wide K-step into a Raw record, decode() turns a Raw record into MFMA operands.

template <int WFMT>
struct AFrag;

// MXFP4: exact bf16 dequantization (E2M1 value times a power-of-two scale).
//
// fetch() is branch-free: every load is issued unconditionally from an address
// clamped into the row (a K-step past the end re-reads the row's last block, a
// cache hit), and blocks past the end are zeroed when decoded.  Loads under
// divergent branches would make the compiler wait for all outstanding loads at
// the join and defeat the prefetch.
template <>
struct AFrag<FMT_MXFP4> {
    static constexpr bool kTwo = false;
    struct Raw {
        u32x4 c0, c1;
        uint32_t s0, s1;  // scale bytes of the two blocks
        bool v0, v1;      // the blocks exist
    };
    bf16x8 hi[8];
    bf16x8 lo[1];

    __device__ __forceinline__ static void fetch(Raw &r, const MatW &W, int e, int rows, int cols, int row, int kk)
    {
        const size_t rr = (size_t)e * rows + row;
        const uint8_t *c = W.codes + rr * (size_t)(cols / 2);
        const uint8_t *sc = W.scales + rr * (size_t)(cols / 32);
        const int k0 = min(kk, cols - 32), k1 = min(kk + 32, cols - 32);
        r.c0 = *(const u32x4 *)(c + k0 / 2);
        r.c1 = *(const u32x4 *)(c + k1 / 2);
        r.s0 = sc[k0 / 32];
        r.s1 = sc[k1 / 32];
        r.v0 = kk < cols;
        r.v1 = kk + 32 < cols;
    }

    __device__ __forceinline__ void decode(const Raw &r, const uint16_t *)
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
        uint32_t d[32];
        decode_fp4x32(r.v0 ? r.c0 : z, e8m0_to_f32(r.s0), d);
        decode_fp4x32(r.v1 ? r.c1 : z, e8m0_to_f32(r.s1), d + 16);
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
    struct Raw {
        uint32_t i0[3], i1[3];  // stage indices of vectors 0..3 and 4..7
        bool v1;                // the second 32-element block exists
        bool v0;
    };
    bf16x8 hi[8];
    bf16x8 lo[8];

    __device__ __forceinline__ static void fetch(Raw &r, const MatW &W, int e, int rows, int cols, int row, int kk)
    {
        r.v0 = kk < cols;
        r.v1 = kk + 32 < cols;
        const int k0 = min(kk, cols - 32), k1 = min(kk + 32, cols - 32);
#pragma unroll
        for (int st = 0; st < 3; st++) {
            const uint8_t *ip = W.idx + (((size_t)e * 3 + st) * rows + row) * (size_t)(cols / 8);
            r.i0[st] = *(const uint32_t *)(ip + k0 / 8);
            r.i1[st] = *(const uint32_t *)(ip + k1 / 8);
        }
    }

    __device__ __forceinline__ void decode(const Raw &r, const uint16_t *cb)
    {
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const bool valid = s < 4 ? r.v0 : r.v1;
            float v[8];
#pragma unroll
            for (int d = 0; d < 8; d++) v[d] = 0.f;
#pragma unroll
            for (int st = 0; st < 3; st++) {
                const uint32_t word = s < 4 ? r.i0[st] : r.i1[st];
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

// ---------------------------------------------------------------- streaming fetchers
//
// A Fetcher walks one weight row of one matrix in 256-wide K-steps.  init() computes
// the lane's base pointers once; fetch(r, step) issues the loads of K-step `step`
// (a wave-uniform index, so the per-step offset is a scalar); decode() produces the
// MFMA operands.  FULL fetchers require K % 256 == 0: no step is partial, nothing is
// masked, and a prefetch past the last step is clamped to the last step (a cache hit).
// General fetchers handle any K that is a multiple of 32 by clamping and masking.

template <int WFMT, bool FULL>
struct Fetcher;

template <>
struct Fetcher<FMT_MXFP4, true> {
    struct Raw {
        u32x4 c0, c1;
        uint32_t s;  // two scale bytes
    };
    const uint8_t *c;
    const uint8_t *sl;  // this row's scale bytes, staged in LDS by stage_scales()
    // lds_row: the row's scales in LDS (cols/32 bytes)
    __device__ __forceinline__ void init(const MatW &W, int e, int rows, int cols, int row, int g,
                                         const uint8_t *lds_row)
    {
        const size_t rr = (size_t)e * rows + row;
        c = W.codes + rr * (size_t)(cols / 2) + 32 * g;
        sl = lds_row + 2 * g;
    }
    __device__ __forceinline__ void fetch(Raw &r, int step) const
    {
        r.c0 = *(const u32x4 *)(c + 128 * step);
        r.c1 = *(const u32x4 *)(c + 128 * step + 16);
        r.s = *(const uint16_t *)(sl + 8 * step);
    }
    __device__ __forceinline__ static void decode(AFrag<FMT_MXFP4> &a, const Raw &r, const uint16_t *)
    {
        uint32_t d[32];
        decode_fp4x32(r.c0, e8m0_to_f32(r.s & 0xFFu), d);
        decode_fp4x32(r.c1, e8m0_to_f32(r.s >> 8), d + 16);
#pragma unroll
        for (int s = 0; s < 8; s++) a.hi[s] = as_bf16x8(d[4 * s], d[4 * s + 1], d[4 * s + 2], d[4 * s + 3]);
    }
};

// Copy the scale bytes of rows [row0, row0 + n) of matrix W of expert e (n * cols/32
// contiguous bytes) to LDS with 8-byte accesses (cols % 256 == 0 makes every row's
// scale run a multiple of 8 bytes and 8-byte aligned).  Called by the whole block.
__device__ __forceinline__ void stage_scales(uint8_t *dst, const MatW &W, int e, int rows, int cols, int row0, int n)
{
    const int nb = n * (cols / 32) / 8;
    const u32x2 *src = (const u32x2 *)(W.scales + ((size_t)e * rows + row0) * (size_t)(cols / 32));
    for (int i = threadIdx.x; i < nb; i += blockDim.x) ((u32x2 *)dst)[i] = src[i];
}

template <>
struct Fetcher<FMT_MXFP4, false> {
    using Raw = AFrag<FMT_MXFP4>::Raw;
    MatW W;
    int e, rows, cols, row, g;
    __device__ __forceinline__ void init(const MatW &W_, int e_, int rows_, int cols_, int row_, int g_,
                                         const uint8_t *)
    {
        W = W_;
        e = e_;
        rows = rows_;
        cols = cols_;
        row = row_;
        g = g_;
    }
    __device__ __forceinline__ void fetch(Raw &r, int step) const
    {
        AFrag<FMT_MXFP4>::fetch(r, W, e, rows, cols, row, 256 * step + 64 * g);
    }
    __device__ __forceinline__ static void decode(AFrag<FMT_MXFP4> &a, const Raw &r, const uint16_t *cb)
    {
        a.decode(r, cb);
    }
};

template <>
struct Fetcher<FMT_RVQ3, true> {
    struct Raw {
        uint32_t i0[3], i1[3];
    };
    const uint8_t *ip[3];
    __device__ __forceinline__ void init(const MatW &W, int e, int rows, int cols, int row, int g, const uint8_t *)
    {
#pragma unroll
        for (int st = 0; st < 3; st++)
            ip[st] = W.idx + (((size_t)e * 3 + st) * rows + row) * (size_t)(cols / 8) + 8 * g;
    }
    __device__ __forceinline__ void fetch(Raw &r, int step) const
    {
#pragma unroll
        for (int st = 0; st < 3; st++) {
            const u32x2 v = *(const u32x2 *)(ip[st] + 32 * step);
            r.i0[st] = v[0];
            r.i1[st] = v[1];
        }
    }
    __device__ __forceinline__ static void decode(AFrag<FMT_RVQ3> &a, const Raw &r, const uint16_t *cb)
    {
        AFrag<FMT_RVQ3>::Raw q;
#pragma unroll
        for (int st = 0; st < 3; st++) {
            q.i0[st] = r.i0[st];
            q.i1[st] = r.i1[st];
        }
        q.v0 = q.v1 = true;
        a.decode(q, cb);
    }
};

template <>
struct Fetcher<FMT_RVQ3, false> {
    using Raw = AFrag<FMT_RVQ3>::Raw;
    MatW W;
    int e, rows, cols, row, g;
    __device__ __forceinline__ void init(const MatW &W_, int e_, int rows_, int cols_, int row_, int g_,
                                         const uint8_t *)
    {
        W = W_;
        e = e_;
        rows = rows_;
        cols = cols_;
        row = row_;
        g = g_;
    }
    __device__ __forceinline__ void fetch(Raw &r, int step) const
    {
        AFrag<FMT_RVQ3>::fetch(r, W, e, rows, cols, row, 256 * step + 64 * g);
    }
    __device__ __forceinline__ static void decode(AFrag<FMT_RVQ3> &a, const Raw &r, const uint16_t *cb)
    {
        a.decode(r, cb);
    }
};

// Token fragment of one 256-wide K-step from a bf16 row (global or LDS): lane group g
// takes elements 64g + 8s .. +7.  No masking: padded token columns only feed output
// columns that are discarded, and masked weight blocks are zero.
__device__ __forceinline__ void load_row_bf16(bf16x8 (&dst)[8], const uint16_t *p)
{
#pragma unroll
    for (int s = 0; s < 8; s++) dst[s] = as_bf16x8(*(const u32x4 *)(p + 8 * s));
}

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
    static constexpr bool kThree = false;
    bf16x8 hi[8];
    bf16x8 lo[1];
    bf16x8 mid[1];
    __device__ __forceinline__ void load(const void *src, size_t rowoff, int kk, int K, bool valid)
    {
        const uint16_t *p = (const uint16_t *)src + rowoff;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const int k = kk + 8 * s;
            const u32x4 v = *(const u32x4 *)(p + min(k, K - 8));
            hi[s] = as_bf16x8(valid && kk + 32 * (s / 4) < K ? v : z);
        }
    }
};

// fp32 rows (tokens, upstream gradients) are split into three bf16 terms hi + mid + lo,
// which hold all 24 significand bits of a normal fp32 value (split_bf16x3), so the
// products with exact weights stay exact.
template <>
struct BFrag<DT_F32> {
    static constexpr bool kTwo = true;
    static constexpr bool kThree = true;
    bf16x8 hi[8];
    bf16x8 lo[8];
    bf16x8 mid[8];
    __device__ __forceinline__ void load(const void *src, size_t rowoff, int kk, int K, bool valid)
    {
        const float *p = (const float *)src + rowoff;
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const int k = min(kk + 8 * s, K - 8);
            float4 a = *(const float4 *)(p + k);
            float4 b = *(const float4 *)(p + k + 4);
            const bool ok = valid && kk + 32 * (s / 4) < K;
            const float f[8] = {ok ? a.x : 0.f, ok ? a.y : 0.f, ok ? a.z : 0.f, ok ? a.w : 0.f,
                                ok ? b.x : 0.f, ok ? b.y : 0.f, ok ? b.z : 0.f, ok ? b.w : 0.f};
            uint32_t h[8], m[8], l[8];
#pragma unroll
            for (int d = 0; d < 8; d++) split_bf16x3(f[d], h[d], m[d], l[d]);
            hi[s] = as_bf16x8(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
            mid[s] = as_bf16x8(pack2(m[0], m[1]), pack2(m[2], m[3]), pack2(m[4], m[5]), pack2(m[6], m[7]));
            lo[s] = as_bf16x8(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
        }
    }
};

// bf16 row staged in LDS; the caller passes a row that exists (valid = the token is real).
__device__ __forceinline__ void load_bf16x8_lds(bf16x8 (&dst)[8], const uint16_t *row, int kk, int K, bool valid)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 8; s++) {
        const u32x4 v = *(const u32x4 *)(row + min(kk + 8 * s, K - 8));
        dst[s] = as_bf16x8(valid && kk + 32 * (s / 4) < K ? v : z);
    }
}

// Copy n rows of K bf16 values (gathered: row r starts at src + off[r]) to LDS rows of
// stride K + 8 elements, 16 bytes per thread step.  Called by the whole block.
__device__ __forceinline__ void stage_rows_bf16(uint16_t *dst, const uint16_t *src, const size_t *off, int n, int K)
{
    const int per = K / 8;
    for (int c = threadIdx.x; c < n * per; c += blockDim.x) {
        const int r = c / per, q = c - r * per;
        *(u32x4 *)(dst + (size_t)r * (K + 8) + 8 * q) = *(const u32x4 *)(src + off[r] + 8 * q);
    }
}

// fp32 rows stored pre-split as two bf16 planes (hi, lo).
struct BFragPair {
    static constexpr bool kTwo = true;
    static constexpr bool kThree = false;
    bf16x8 hi[8];
    bf16x8 lo[8];
    bf16x8 mid[1];
    __device__ __forceinline__ void load(const uint16_t *phi, const uint16_t *plo, size_t rowoff, int kk, int K,
                                         bool valid)
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const int k = min(kk + 8 * s, K - 8);
            const u32x4 vh = *(const u32x4 *)(phi + rowoff + k);
            const u32x4 vl = *(const u32x4 *)(plo + rowoff + k);
            const bool ok = valid && kk + 32 * (s / 4) < K;
            hi[s] = as_bf16x8(ok ? vh : z);
            lo[s] = as_bf16x8(ok ? vl : z);
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
        if constexpr (B::kThree) acc = mfma16(a.hi[s], b.mid[s], acc);
        if constexpr (A::kTwo && B::kThree) acc = mfma16(a.lo[s], b.mid[s], acc);
        if constexpr (B::kTwo) acc = mfma16(a.hi[s], b.lo[s], acc);
    }
}

}  // namespace moe
