// dense.hip -- the latent projections around the MoE layer (LazyLoRA README, "The engine":
// the latent MoE projections are dense weights beside the router gates; Two Desks, Act II:
// the experts work in a latent space of width 3,584).
//
// One kernel computes out[T][N] = a[T][R] b with bf16 weights w:
//   NT (forward)     b = w^T, w stored [N][R] (R contiguous):  out[t][n] = sum_r a[t][r] w[n][r]
//   NN (transposed)  b = w,   w stored [R][N] (N contiguous):  out[t][n] = sum_r a[t][r] w[r][n]
// a is bf16 (exact MFMA operand) or fp32 (three bf16 terms hi + mid + lo, which hold its 24
// significand bits, so every product is exact); fp32 accumulation, fp32 output.
// Block = 64 tokens x 64 outputs, four waves of 32 x 32 (2 x 2 MFMA 16x16x32 tiles); per
// K-step of 32 the a tile (each term) and the w tile are staged in LDS as [row][32 + 8] bf16
// (the NN tile transposed on its way in), so every MFMA fragment is one 16-byte LDS read.
#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kDT = 64, kDK = 32, kDS = kDK + 8;  // tile rows, K-step, LDS row stride (bf16)

template <int AT, bool NN>
__global__ __launch_bounds__(256) void k_dense(const void *__restrict__ a, const uint16_t *__restrict__ w, int T, int N,
                                               int R, float *__restrict__ out)
{
    constexpr int NTERM = AT == DT_F32 ? 3 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t as[NTERM][kDT * kDS];
    __shared__ __attribute__((aligned(16))) uint16_t bs[kDT * kDS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, li = lane & 15;
    const int wm = wv >> 1, wn = wv & 1;
    const int t0 = blockIdx.y * kDT, n0 = blockIdx.x * kDT;
    // staging coordinates: a and NT w: row tid / 4, 8 consecutive K at 8 (tid % 4)
    const int sr = tid >> 2, sk = 8 * (tid & 3);
    const bool tv = t0 + sr < T;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < R; k0 += kDK) {
        // a tile
        if constexpr (AT == DT_BF16) {
            const u32x4 v = tv ? *(const u32x4 *)((const uint16_t *)a + (size_t)(t0 + sr) * R + k0 + sk) : u32x4{0u, 0u, 0u, 0u};
            *(u32x4 *)(as[0] + sr * kDS + sk) = v;
        } else {
            float f[8];
            if (tv) {
                const float4 p = *(const float4 *)((const float *)a + (size_t)(t0 + sr) * R + k0 + sk);
                const float4 q = *(const float4 *)((const float *)a + (size_t)(t0 + sr) * R + k0 + sk + 4);
                f[0] = p.x; f[1] = p.y; f[2] = p.z; f[3] = p.w; f[4] = q.x; f[5] = q.y; f[6] = q.z; f[7] = q.w;
            } else {
#pragma unroll
                for (int d = 0; d < 8; d++) f[d] = 0.f;
            }
            uint32_t h[8], m[8], l[8];
#pragma unroll
            for (int d = 0; d < 8; d++) split_bf16x3(f[d], h[d], m[d], l[d]);
            *(u32x4 *)(as[0] + sr * kDS + sk) = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
            *(u32x4 *)(as[NTERM - 2] + sr * kDS + sk) = u32x4{pack2(m[0], m[1]), pack2(m[2], m[3]), pack2(m[4], m[5]), pack2(m[6], m[7])};
            *(u32x4 *)(as[NTERM - 1] + sr * kDS + sk) = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
        }
        // w tile as [output][K]
        if constexpr (!NN) {
            *(u32x4 *)(bs + sr * kDS + sk) = *(const u32x4 *)(w + (size_t)(n0 + sr) * R + k0 + sk);
        } else {
            // w rows k0 + tid / 8 (32 of them), 8 consecutive outputs each, stored transposed
            const int kr = tid >> 3, nc = 8 * (tid & 7);
            const u32x4 v = *(const u32x4 *)(w + (size_t)(k0 + kr) * N + n0 + nc);
#pragma unroll
            for (int d = 0; d < 4; d++) {
                bs[(nc + 2 * d) * kDS + kr] = (uint16_t)(v[d] & 0xFFFFu);
                bs[(nc + 2 * d + 1) * kDS + kr] = (uint16_t)(v[d] >> 16);
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const bf16x8 B = as_bf16x8(*(const u32x4 *)(bs + (32 * wn + 16 * j + li) * kDS + 8 * g));
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int q = 0; q < NTERM; q++)
                    acc[i][j] = mfma16(as_bf16x8(*(const u32x4 *)(as[q] + (32 * wm + 16 * i + li) * kDS + 8 * g)), B, acc[i][j]);
        }
        __syncthreads();
    }
    // lane holds tokens t0 + 32 wm + 16 i + 4 g + r, output n0 + 32 wn + 16 j + li
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int t = t0 + 32 * wm + 16 * i + 4 * g + r;
            if (t >= T) continue;
#pragma unroll
            for (int j = 0; j < 2; j++) out[(size_t)t * N + n0 + 32 * wn + 16 * j + li] = acc[i][j][r];
        }
}

}  // namespace

hipError_t launch_dense(const void *a, int at, const uint16_t *w, bool nn, int T, int N, int R, float *out, hipStream_t s)
{
    const dim3 grid((unsigned)(N / kDT), (unsigned)((T + kDT - 1) / kDT));
    if (at == DT_BF16) {
        if (nn)
            hipLaunchKernelGGL((k_dense<DT_BF16, true>), grid, dim3(256), 0, s, a, w, T, N, R, out);
        else
            hipLaunchKernelGGL((k_dense<DT_BF16, false>), grid, dim3(256), 0, s, a, w, T, N, R, out);
    } else {
        if (nn)
            hipLaunchKernelGGL((k_dense<DT_F32, true>), grid, dim3(256), 0, s, a, w, T, N, R, out);
        else
            hipLaunchKernelGGL((k_dense<DT_F32, false>), grid, dim3(256), 0, s, a, w, T, N, R, out);
    }
    return hipGetLastError();
}

}  // namespace moe
