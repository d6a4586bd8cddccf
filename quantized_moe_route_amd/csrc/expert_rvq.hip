// expert_rvq.hip -- few-token expert forward for 3-bit residual-VQ weights (bf16 tokens).
//
// WASTE README, "3 bits per expert weight": each expert matrix is coded as residual VQ,
// 3 stages of 256-entry codebooks over 8-dimensional vectors, so a weight vector (8
// consecutive `in` elements of one row) is C1[i1] + C2[i2] + C3[i3].  The matrix is never
// materialised: since the product is linear, sum_s C_s[i_s] . x = sum_s (C_s[i_s] . x),
// each stage's codeword enters the MFMA directly as an fp16 operand
// (v_mfma_f32_16x16x32_f16 takes 8 consecutive reduction elements per lane, exactly one
// codeword) and there is no decode arithmetic at all:
//  - the expert's codebooks (fp16, 12 KB per matrix) live in LDS; the A operand of a
//    sub-step is one 16-byte LDS read per stage, indexed by the row's index byte;
//  - token rows go to LDS as fp16 times a per-token power of two that puts the row's
//    largest magnitude in [2^13, 2^14): bf16 values are then exact in fp16 (down to 2^-31
//    of the row maximum), and the factor comes off the fp32 result exactly;
//  - for the down product h (fp32) is carried as two fp16 planes hi + lo of the scaled
//    value (|h - hi - lo| <= 2^-22 |h|), packed into MFMA columns 2j and 2j + 1;
//  - index bytes stream through four register stages (three K-steps of prefetch) with
//    the K loop unrolled by four, as in the MXFP4 stream kernels.
// Tokens are processed in passes of up to 4 per expert (the weights are re-read for a
// further pass).
#include <type_traits>

#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kRvqTok = 4;  // tokens per pass

template <int P>
using Stage = std::integral_constant<int, P>;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
}

template <typename F>
__device__ __forceinline__ void k_loop4(int n, F &&step)
{
    int s0 = 0;
    for (; s0 + 4 <= n; s0 += 4) {
        step(Stage<0>(), s0);
        step(Stage<1>(), s0 + 1);
        step(Stage<2>(), s0 + 2);
        step(Stage<3>(), s0 + 3);
    }
    if (s0 < n) step(Stage<0>(), s0);
    if (s0 + 1 < n) step(Stage<1>(), s0 + 1);
    if (s0 + 2 < n) step(Stage<2>(), s0 + 2);
}

__device__ __forceinline__ f32x4 mfma_h(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

// Exponent se with max * 2^-se in [2^13, 2^14) (0 for an all-zero row).
__device__ __forceinline__ int scale_exp(float m)
{
    if (!(m > 0.f)) return 0;
    int e;
    frexpf(m, &e);  // m in [2^(e-1), 2^e)
    return e - 14;
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Copy the expert's codebooks of one matrix ([3][256][8] fp16 = 768 chunks of 16 B) to LDS.
__device__ __forceinline__ void load_cb(u32x4 *dst, const uint16_t *cb, int e)
{
    const u32x4 *src = (const u32x4 *)(cb + (size_t)e * 3 * 256 * 8);
    for (int i = threadIdx.x; i < 3 * 256; i += blockDim.x) dst[i] = src[i];
}

// Block-wide max of |v| per token (nt <= 4 tokens); red: 4 x 4 floats of LDS.
__device__ __forceinline__ void token_max(float (&m)[kRvqTok], float *red, float *out)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < kRvqTok; j++) {
        const float w = wave_max_f32(m[j]);
        if (lane == 0) red[wv * kRvqTok + j] = w;
    }
    __syncthreads();
    if (threadIdx.x < kRvqTok) {
        const int j = threadIdx.x;
        out[j] = fmaxf(fmaxf(red[j], red[kRvqTok + j]), fmaxf(red[2 * kRvqTok + j], red[3 * kRvqTok + j]));
    }
    __syncthreads();
}

}  // namespace

// gate/up + activation.  Block = 4 waves x 16 rows = 64 I-columns of one active expert, gate
// and up tiles per wave.  Dynamic LDS: codebooks (2 x 12 KB), x rows [4][H + 8] fp16.
__global__ __launch_bounds__(256) void k_gateup_rvq(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) u32x4 lds[];
    __shared__ float red[4 * kRvqTok], tmax[kRvqTok];
    __shared__ int sexp[kRvqTok];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, li = lane & 15;
    const int ai = blockIdx.y;
    const int nact = *a.n_active;
    const int e = min(max(a.active[ai], 0), a.E - 1);
    const int H = a.H, I = a.I;
    const int row0 = blockIdx.x * 64 + wv * 16;
    const int nsteps = H / 256, vpr = H / 8;  // index bytes per row and stage
    const uint32_t plane = (uint32_t)I * vpr;  // bytes per stage plane
    const __amdgpu_buffer_rsrc_t ig = buf_rsrc(a.gate.idx + (size_t)e * 3 * plane, 3 * plane);
    const __amdgpu_buffer_rsrc_t iu = buf_rsrc(a.up.idx + (size_t)e * 3 * plane, 3 * plane);
    const uint32_t ioff = (uint32_t)(row0 + li) * vpr + 8 * g;
    u32x2 rg[4][3], ru[4][3];
    auto fetch = [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int s = 0; s < 3; s++) {
            rg[p][s] = ld8(ig, ioff, s * plane + 32 * st);
            ru[p][s] = ld8(iu, ioff, s * plane + 32 * st);
        }
    };
    fetch(Stage<0>(), 0);
    fetch(Stage<1>(), min(1, nsteps - 1));
    fetch(Stage<2>(), min(2, nsteps - 1));
    if (ai >= nact) return;
    u32x4 *cbg = lds, *cbu = lds + 768;
    load_cb(cbg, a.gate.cb, e);
    load_cb(cbu, a.up.cb, e);
    _Float16 *xs = (_Float16 *)(lds + 2 * 768);
    const int xstride = H + 8;
    const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;

    for (int tt0 = 0; tt0 < ntok; tt0 += kRvqTok) {
        const int nt = min(kRvqTok, ntok - tt0);
        if (tt0 > 0) {  // a further pass re-reads the weights from the start
            __syncthreads();
            fetch(Stage<0>(), 0);
            fetch(Stage<1>(), min(1, nsteps - 1));
            fetch(Stage<2>(), min(2, nsteps - 1));
        }
        // per-token scale, then the scaled fp16 rows
        int xrow[kRvqTok];
        float m[kRvqTok];
#pragma unroll
        for (int j = 0; j < kRvqTok; j++) {
            xrow[j] = a.perm[r0 + tt0 + min(j, nt - 1)] / a.k;
            m[j] = 0.f;
            for (int c = tid; c < H / 8; c += 256) {
                const u32x4 v = *(const u32x4 *)((const uint16_t *)a.x + (size_t)xrow[j] * H + 8 * c);
#pragma unroll
                for (int d = 0; d < 4; d++)
                    m[j] = fmaxf(m[j], fmaxf(fabsf(bf16_bits_to_f32(v[d] & 0xFFFFu)), fabsf(bf16_bits_to_f32(v[d] >> 16))));
            }
        }
        token_max(m, red, tmax);
        if (tid < kRvqTok) sexp[tid] = scale_exp(tmax[tid]);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRvqTok; j++) {
            const int se = sexp[j];
            for (int c = tid; c < H / 8; c += 256) {
                const u32x4 v = *(const u32x4 *)((const uint16_t *)a.x + (size_t)xrow[j] * H + 8 * c);
                u32x4 o;
#pragma unroll
                for (int d = 0; d < 4; d++)
                    o[d] = pack_h2(ldexpf(bf16_bits_to_f32(v[d] & 0xFFFFu), -se), ldexpf(bf16_bits_to_f32(v[d] >> 16), -se));
                *(u32x4 *)(xs + (size_t)j * xstride + 8 * c) = o;
            }
        }
        __syncthreads();

        const _Float16 *xl = xs + (size_t)min(li, kRvqTok - 1) * xstride + 64 * g;
        f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
        k_loop4(nsteps, [&](auto P, int st) {
            constexpr int p = decltype(P)::value;
            fetch(Stage<(p + 3) % 4>(), min(st + 3, nsteps - 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 8; s++) {
                const u32x4 B = *(const u32x4 *)(xl + 256 * st + 8 * s);
#pragma unroll
                for (int q = 0; q < 3; q++) {
                    const uint32_t ib = (rg[p][q][s >> 2] >> (8 * (s & 3))) & 0xFFu;
                    const uint32_t iv = (ru[p][q][s >> 2] >> (8 * (s & 3))) & 0xFFu;
                    accg = mfma_h(cbg[256 * q + ib], B, accg);
                    accu = mfma_h(cbu[256 * q + iv], B, accu);
                }
            }
        });

        // lane holds I-columns row0 + 4 g + 0..3 of token tt0 + li
        if (li < nt) {
            const size_t rr = (size_t)(r0 + tt0 + li);
            const int n = row0 + 4 * g, se = sexp[li];
            f32x4 gv, uv;
            uint32_t hh[4], hl[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                gv[r] = ldexpf(accg[r], se);
                uv[r] = ldexpf(accu[r], se);
            }
            add_lora_gu(a.lora_gu, a.perm, a.k, rr, I, n, gv, uv);
#pragma unroll
            for (int r = 0; r < 4; r++) split_bf16(act_h(a.act, gv[r], uv[r]), hh[r], hl[r]);
            *(u32x2 *)(a.h_hi + rr * I + n) = u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
            *(u32x2 *)(a.h_lo + rr * I + n) = u32x2{pack2(hl[0], hl[1]), pack2(hl[2], hl[3])};
            if (a.gu) {
                *(float4 *)(a.gu + (rr * 2 + 0) * I + n) = float4{gv[0], gv[1], gv[2], gv[3]};
                *(float4 *)(a.gu + (rr * 2 + 1) * I + n) = float4{uv[0], uv[1], uv[2], uv[3]};
            }
        }
    }
}

// down + routing weight.  Block = 4 waves x 2 tiles x 16 rows = 128 H-rows of one active
// expert.  MFMA column 2j carries the fp16 hi plane of token j's scaled h, column 2j + 1
// its lo plane.  Dynamic LDS: codebooks (12 KB), h planes [4][2][I + 8] fp16.
__global__ __launch_bounds__(256) void k_down_rvq(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) u32x4 lds[];
    __shared__ float red[4 * kRvqTok], tmax[kRvqTok];
    __shared__ int sexp[kRvqTok];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, li = lane & 15;
    const int ai = blockIdx.y;
    const int nact = *a.n_active;
    const int e = min(max(a.active[ai], 0), a.E - 1);
    const int H = a.H, I = a.I;
    const int m0 = blockIdx.x * 128 + wv * 32;
    const int nsteps = I / 256, vpr = I / 8;
    const uint32_t plane = (uint32_t)H * vpr;
    const __amdgpu_buffer_rsrc_t id = buf_rsrc(a.down.idx + (size_t)e * 3 * plane, 3 * plane);
    const uint32_t ioff0 = (uint32_t)(m0 + li) * vpr + 8 * g, ioff1 = ioff0 + 16 * vpr;
    u32x2 r0_[4][3], r1_[4][3];
    auto fetch = [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int s = 0; s < 3; s++) {
            r0_[p][s] = ld8(id, ioff0, s * plane + 32 * st);
            r1_[p][s] = ld8(id, ioff1, s * plane + 32 * st);
        }
    };
    fetch(Stage<0>(), 0);
    fetch(Stage<1>(), min(1, nsteps - 1));
    fetch(Stage<2>(), min(2, nsteps - 1));
    if (ai >= nact) return;
    u32x4 *cbd = lds;
    load_cb(cbd, a.down.cb, e);
    _Float16 *hs = (_Float16 *)(lds + 768);
    const int hstride = I + 8;
    const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;

    for (int tt0 = 0; tt0 < ntok; tt0 += kRvqTok) {
        const int nt = min(kRvqTok, ntok - tt0);
        if (tt0 > 0) {
            __syncthreads();
            fetch(Stage<0>(), 0);
            fetch(Stage<1>(), min(1, nsteps - 1));
            fetch(Stage<2>(), min(2, nsteps - 1));
        }
        // h = hi + lo (bf16 planes) -> per-token scale -> fp16 hi + lo planes
        float m[kRvqTok];
#pragma unroll
        for (int j = 0; j < kRvqTok; j++) {
            const size_t rr = (size_t)(r0 + tt0 + min(j, nt - 1)) * I;
            m[j] = 0.f;
            for (int c = tid; c < I / 8; c += 256) {
                const u32x4 vh = *(const u32x4 *)(a.h_hi + rr + 8 * c), vl = *(const u32x4 *)(a.h_lo + rr + 8 * c);
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    m[j] = fmaxf(m[j], fabsf(bf16_bits_to_f32(vh[d] & 0xFFFFu) + bf16_bits_to_f32(vl[d] & 0xFFFFu)));
                    m[j] = fmaxf(m[j], fabsf(bf16_bits_to_f32(vh[d] >> 16) + bf16_bits_to_f32(vl[d] >> 16)));
                }
            }
        }
        token_max(m, red, tmax);
        if (tid < kRvqTok) sexp[tid] = scale_exp(tmax[tid]);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRvqTok; j++) {
            const size_t rr = (size_t)(r0 + tt0 + min(j, nt - 1)) * I;
            const int se = sexp[j];
            for (int c = tid; c < I / 8; c += 256) {
                const u32x4 vh = *(const u32x4 *)(a.h_hi + rr + 8 * c), vl = *(const u32x4 *)(a.h_lo + rr + 8 * c);
                u32x4 oh, ol;
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    const float h0 = ldexpf(bf16_bits_to_f32(vh[d] & 0xFFFFu) + bf16_bits_to_f32(vl[d] & 0xFFFFu), -se);
                    const float h1 = ldexpf(bf16_bits_to_f32(vh[d] >> 16) + bf16_bits_to_f32(vl[d] >> 16), -se);
                    const float q0 = (float)(_Float16)h0, q1 = (float)(_Float16)h1;
                    oh[d] = pack_h2(h0, h1);
                    ol[d] = pack_h2(h0 - q0, h1 - q1);
                }
                *(u32x4 *)(hs + (size_t)(2 * j) * hstride + 8 * c) = oh;
                *(u32x4 *)(hs + (size_t)(2 * j + 1) * hstride + 8 * c) = ol;
            }
        }
        __syncthreads();

        // lane column li: plane li & 1 of token li >> 1
        const _Float16 *hl = hs + (size_t)min(li, 2 * kRvqTok - 1) * hstride + 64 * g;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        k_loop4(nsteps, [&](auto P, int st) {
            constexpr int p = decltype(P)::value;
            fetch(Stage<(p + 3) % 4>(), min(st + 3, nsteps - 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 8; s++) {
                const u32x4 B = *(const u32x4 *)(hl + 256 * st + 8 * s);
#pragma unroll
                for (int q = 0; q < 3; q++) {
                    const uint32_t i0 = (r0_[p][q][s >> 2] >> (8 * (s & 3))) & 0xFFu;
                    const uint32_t i1 = (r1_[p][q][s >> 2] >> (8 * (s & 3))) & 0xFFu;
                    acc0 = mfma_h(cbd[256 * q + i0], B, acc0);
                    acc1 = mfma_h(cbd[256 * q + i1], B, acc1);
                }
            }
        });
        // column 2j + 1 (lo plane) onto column 2j
#pragma unroll
        for (int r = 0; r < 4; r++) {
            acc0[r] += dpp_f32<kDppXor1>(acc0[r]);
            acc1[r] += dpp_f32<kDppXor1>(acc1[r]);
        }
        const int j = li >> 1;
        if (j < nt && (li & 1) == 0) {
            const int slot = a.perm[r0 + tt0 + j];
            const float pw = ldexpf(a.w[slot], sexp[j]);
            float *yb = a.ybuf + (size_t)slot * H + m0 + 4 * g;
            *(float4 *)yb = float4{pw * acc0[0], pw * acc0[1], pw * acc0[2], pw * acc0[3]};
            *(float4 *)(yb + 16) = float4{pw * acc1[0], pw * acc1[1], pw * acc1[2], pw * acc1[3]};
        }
    }
}

// bf16 tokens, few tokens per expert, H and I multiples of 256 up to 4096 (LDS), index
// planes addressable with 32-bit offsets.
static size_t lds_gateup(const ExpertFwdArgs &a) { return 2 * 768 * 16 + (size_t)kRvqTok * (a.H + 8) * 2; }
static size_t lds_down(const ExpertFwdArgs &a) { return 768 * 16 + (size_t)2 * kRvqTok * (a.I + 8) * 2; }

bool rvq_dec_supported(const ExpertFwdArgs &a)
{
    return a.wfmt == FMT_RVQ3 && a.xt == DT_BF16 && a.T <= 64 && a.H % 256 == 0 && a.I % 256 == 0 &&
           lds_gateup(a) <= 65536 && lds_down(a) <= 65536 && (size_t)3 * a.H * (a.I / 8) < ((size_t)1 << 32);
}

hipError_t launch_gateup_rvq(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    ProfScope ps(a.prof, PK_GATEUP, s);
    ps.launch(k_gateup_rvq, dim3(a.I / 64, maxU), dim3(256), lds_gateup(a), a);
    return hipGetLastError();
}

hipError_t launch_down_rvq(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    ProfScope ps(a.prof, PK_DOWN, s);
    ps.launch(k_down_rvq, dim3(a.H / 128, maxU), dim3(256), lds_down(a), a);
    return hipGetLastError();
}

}  // namespace moe
