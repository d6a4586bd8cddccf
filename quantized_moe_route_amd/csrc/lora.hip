// lora.hip -- the shared low-rank adapter on the routed experts.
//
// LazyLoRA README, "LoRA": one adapter per MoE layer in the latent space, shared by every
// routed expert, on the gate, up and down projections (rank 16 there); each expert
// product W z becomes (W + s B A) z = W z + s B (A z), with A [r][in], B [out][r] and
// s the adapter scale.  Because the adapter is the same for every expert:
//  - the gate/up terms s B_g (A_g x_t), s B_u (A_u x_t) are per TOKEN ([T][2I]), formed
//    once before the expert kernels and added in their epilogues before the activation;
//  - the down term of a token is s B_d z_t with z_t = sum_j p_tj A_d h_tj = A_d hbar_t,
//    hbar_t = sum_j p_tj h_tj (one gather-sum over the token's slot rows), added to y
//    after the combine;
//  - in the backward, the term s A_d^T (B_d^T dy_t) of W_d^T dy is again per token and is
//    added in the backward down epilogue; the gate/up input gradient gains
//    s A_g^T (B_g^T DG_t) + s A_u^T (B_u^T DU_t) with DG_t, DU_t the sums over the token's
//    slots of dL/dg, dL/du;
//  - the adapter gradients are sums of outer products over tokens (or slots):
//    dB_g = s sum_t DG_t (A_g x_t)^T, dA_g = s sum_t (B_g^T DG_t) x_t^T (up alike),
//    dB_d = s sum_t dy_t z_t^T, dA_d = s sum_s p_s (B_d^T dy_t(s)) h_s^T
//    = s sum_t (B_d^T dy_t) hbar_t^T.
// Everything here is skinny fp32 products (one dimension is the rank) with fp32
// accumulation in a fixed order (row-chunk partial sums reduced in chunk order), shaped
// three ways (tall: a long contiguous reduction per row; row sums: a reduction over token
// rows; wide: a rank-long reduction per output), plus two gather-sums over the grouped
// slot rows.
#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Loads of 4 consecutive elements of a row of fp32 or bf16 values as fp32.
template <int DT>
__device__ __forceinline__ float4 ld4(const void *p, size_t idx)
{
    if constexpr (DT == DT_F32) return *(const float4 *)((const float *)p + idx);
    const u32x2 v = *(const u32x2 *)((const uint16_t *)p + idx);
    return float4{bf16_bits_to_f32(v[0] & 0xFFFFu), bf16_bits_to_f32(v[0] >> 16), bf16_bits_to_f32(v[1] & 0xFFFFu),
                  bf16_bits_to_f32(v[1] >> 16)};
}

// Tall product: C[m][q] = alpha sum_k A[m][k] B(k, q) for q < R <= RM, A row-major with
// K contiguous (fp32 or bf16, row stride lda), B fp32 given as [R][K] (BT) or [K][R].
// A block is 4 waves x 4 rows; the 16 lanes of a row take 4 consecutive k each (256
// contiguous bytes of A per row and step), B comes in chunks of KC columns through LDS,
// and the 16 lanes' partial sums are added with DPP in a fixed order.  K % 4 == 0.
template <int DA, bool BT, int RM>
__global__ __launch_bounds__(256) void k_tall(const void *__restrict__ A, long lda, const float *__restrict__ B, int R, int M,
                                              int K, float *__restrict__ C, long ldc, float alpha)
{
    constexpr int KC = 8192 / RM, NLD = KC / 64;  // K per chunk, A loads per lane per chunk
    __shared__ float Bs[RM][KC + 4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, kl = lane & 15;
    const int row = blockIdx.x * 16 + wv * 4 + (lane >> 4);
    const bool live = row < M;
    float acc[RM];
#pragma unroll
    for (int q = 0; q < RM; q++) acc[q] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KC) {
        float4 a[NLD];
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int k = k0 + 64 * i + 4 * kl;
            a[i] = live && k < K ? ld4<DA>(A, (size_t)row * lda + k) : float4{0.f, 0.f, 0.f, 0.f};
        }
        // the B chunk: every load of the thread first, then the LDS stores
        constexpr int NB = RM * KC / 256;
        float bv[NB];
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int e = tid + 256 * i;
            const int q = BT ? e / KC : e % RM, kk = BT ? e % KC : e / RM, k = k0 + kk;
            bv[i] = q < R && k < K ? (BT ? B[(size_t)q * K + k] : B[(size_t)k * R + q]) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int e = tid + 256 * i;
            Bs[BT ? e / KC : e % RM][BT ? e % KC : e / RM] = bv[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NLD; i++) {
            const int kk = 64 * i + 4 * kl;
#pragma unroll
            for (int q = 0; q < RM; q++) {
                const float4 b = *(const float4 *)&Bs[q][kk];
                acc[q] = fmaf(a[i].x, b.x, fmaf(a[i].y, b.y, fmaf(a[i].z, b.z, fmaf(a[i].w, b.w, acc[q]))));
            }
        }
    }
    // sum over the row's 16 lanes; lane kl stores outputs q = kl, kl + 16, ...
#pragma unroll
    for (int q = 0; q < RM; q++) {
        float v = acc[q];
        v += dpp_f32<kDppXor1>(v);
        v += dpp_f32<kDppXor2>(v);
        v += dpp_f32<kDppHalfMirror>(v);
        v += dpp_f32<kDppMirror>(v);
        if (live && (q & 15) == kl && q < R) C[(size_t)row * ldc + q] = alpha * v;
    }
}

// Row-reduction product, first pass: part[z][q][n] = sum over rows k of chunk z of
// A[k][q] Cm[k][n] for q < R <= RM (A fp32 [K][lda], Cm fp32 or bf16 [K][ldc]).  One wave
// per block covers 256 columns, 4 per lane; the A values of a row are the same for every
// lane.  N % 4 == 0.
template <int DC, int RM>
__global__ __launch_bounds__(64) void k_rowsum(const float *__restrict__ A, long lda, const void *__restrict__ Cm, long ldc, int R,
                                               int N, int K, int kchunk, float *__restrict__ part)
{
    const int n = 4 * (blockIdx.x * 64 + threadIdx.x), z = blockIdx.y;
    const int kb = z * kchunk, ke = min(K, kb + kchunk);
    float acc[RM][4];
#pragma unroll
    for (int q = 0; q < RM; q++) acc[q][0] = acc[q][1] = acc[q][2] = acc[q][3] = 0.f;
    if (n < N) {
        int k = kb;
        for (; k + 4 <= ke; k += 4) {
            float4 c[4];
#pragma unroll
            for (int u = 0; u < 4; u++) c[u] = ld4<DC>(Cm, (size_t)(k + u) * ldc + n);
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int q = 0; q < RM; q++) {
                    const float a = q < R ? A[(size_t)(k + u) * lda + q] : 0.f;
                    acc[q][0] = fmaf(a, c[u].x, acc[q][0]);
                    acc[q][1] = fmaf(a, c[u].y, acc[q][1]);
                    acc[q][2] = fmaf(a, c[u].z, acc[q][2]);
                    acc[q][3] = fmaf(a, c[u].w, acc[q][3]);
                }
        }
        for (; k < ke; k++) {
            const float4 c = ld4<DC>(Cm, (size_t)k * ldc + n);
#pragma unroll
            for (int q = 0; q < RM; q++) {
                const float a = q < R ? A[(size_t)k * lda + q] : 0.f;
                acc[q][0] = fmaf(a, c.x, acc[q][0]);
                acc[q][1] = fmaf(a, c.y, acc[q][1]);
                acc[q][2] = fmaf(a, c.z, acc[q][2]);
                acc[q][3] = fmaf(a, c.w, acc[q][3]);
            }
        }
#pragma unroll
        for (int q = 0; q < RM; q++)
            if (q < R) *(float4 *)(part + ((size_t)z * R + q) * N + n) = float4{acc[q][0], acc[q][1], acc[q][2], acc[q][3]};
    }
}

// Second pass: C(q, n) = alpha sum_z part[z][q][n], chunks in order; C(q, n) at
// C[q scq + n scn].
__global__ __launch_bounds__(256) void k_rowsum_reduce(const float *__restrict__ part, int nz, int R, int N, float *__restrict__ C,
                                                       long scq, long scn, float alpha)
{
    const size_t RN = (size_t)R * N;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < RN; i += (size_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int z = 0; z < nz; z++) s += part[z * RN + i];
        const int q = (int)(i / N), n = (int)(i % N);
        C[(size_t)q * scq + (size_t)n * scn] = alpha * s;
    }
}

// Wide product with a rank-sized reduction: C[m][n] = alpha sum_q a[m][q] b(n, q)
// [+ C[m][n]] for n < N, b given as [N][ldb] (BNQ) or [R][ldb or the range's width],
// q < R <= RM.  Two column
// ranges can be done in one launch: columns n >= N1 take b1, the a values at +a1off and
// write C at +c1off (the gate and up halves of the adapter terms); a block's columns lie
// in one range.  A thread takes 4 columns (their b values stay in registers) of up to
// kWideRows consecutive rows, whose a values the block stages in LDS.  N1, N % 4 == 0.
constexpr int kWideRows = 16;

template <bool BNQ, int RM, bool VEC>
__global__ __launch_bounds__(256) void k_wide(const float *__restrict__ a, long lda, const float *__restrict__ b0,
                                              const float *__restrict__ b1, long ldb, int N1, long c1off, long a1off, int R, int M,
                                              int N, float *__restrict__ C, long ldc, float alpha, int accum)
{
    __shared__ float as[kWideRows][RM];
    const int nb0 = (N1 / 4 + 255) / 256;  // blocks of the first range
    const bool hi = (int)blockIdx.x >= nb0;
    const int Nb = hi ? N - N1 : N1, n = 4 * (((int)blockIdx.x - (hi ? nb0 : 0)) * 256 + (int)threadIdx.x);
    const float *b = hi ? b1 : b0;
    const long aoff = hi ? a1off : 0;
    const int m0 = blockIdx.y * kWideRows, nr = min(kWideRows, M - m0);
    for (int e = threadIdx.x; e < kWideRows * RM; e += blockDim.x) {
        const int i = e / RM, q = e % RM;
        as[i][q] = i < nr && q < R ? a[(size_t)(m0 + i) * lda + aoff + q] : 0.f;
    }
    __syncthreads();
    if (n >= Nb) return;
    float bv[4][RM];
    if constexpr (BNQ) {
        if (VEC) {  // rows of b 16-byte aligned: four values of q per load
#pragma unroll
            for (int c = 0; c < 4; c++)
#pragma unroll
                for (int q = 0; q < RM; q += 4) {
                    const float4 v = q < R ? *(const float4 *)(b + (size_t)(n + c) * ldb + q) : float4{0.f, 0.f, 0.f, 0.f};
                    bv[c][q] = v.x;
                    bv[c][q + 1] = q + 1 < R ? v.y : 0.f;
                    bv[c][q + 2] = q + 2 < R ? v.z : 0.f;
                    bv[c][q + 3] = q + 3 < R ? v.w : 0.f;
                }
        } else {
#pragma unroll
            for (int c = 0; c < 4; c++)
#pragma unroll
                for (int q = 0; q < RM; q++) bv[c][q] = q < R ? b[(size_t)(n + c) * ldb + q] : 0.f;
        }
    } else {  // four consecutive columns per load
#pragma unroll
        for (int q = 0; q < RM; q++) {
            const float4 v = q < R ? *(const float4 *)(b + (size_t)q * (ldb ? ldb : Nb) + n) : float4{0.f, 0.f, 0.f, 0.f};
            bv[0][q] = v.x;
            bv[1][q] = v.y;
            bv[2][q] = v.z;
            bv[3][q] = v.w;
        }
    }
    float *cr = C + (hi ? c1off : 0) + n;
    for (int i = 0; i < nr; i++) {
        float sv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < RM; q++) {
            const float aq = as[i][q];
#pragma unroll
            for (int c = 0; c < 4; c++) sv[c] = fmaf(aq, bv[c][q], sv[c]);
        }
        float *o = cr + (size_t)(m0 + i) * ldc;
        float4 v = float4{alpha * sv[0], alpha * sv[1], alpha * sv[2], alpha * sv[3]};
        if (accum) {
            const float4 c = *(const float4 *)o;
            v = float4{v.x + c.x, v.y + c.y, v.z + c.z, v.w + c.w};
        }
        *(float4 *)o = v;
    }
}

// Few rows: C[m][q] = alpha sum_k A[m][k] B(k, q), one block per (m, q), the block's 256
// threads striding K by 4 and summing in a fixed tree.
template <int DA, bool BT>
__global__ __launch_bounds__(256) void k_dot(const void *__restrict__ A, long lda, const float *__restrict__ B0,
                                             const float *__restrict__ B1, int R, int K, float *__restrict__ C, long ldc, float alpha)
{
    __shared__ float red[4];
    // outputs q >= R take B1 (the second matrix of a pair), column q of C either way
    const int m = blockIdx.y, qq = blockIdx.x, q = qq < R ? qq : qq - R;
    const float *B = qq < R ? B0 : B1;
    float acc = 0.f;
    for (int k = 4 * threadIdx.x; k < K; k += 1024) {
        const float4 av = ld4<DA>(A, (size_t)m * lda + k);
        float4 bv;
        if constexpr (BT)
            bv = *(const float4 *)(B + (size_t)q * K + k);
        else
            bv = float4{B[(size_t)k * R + q], B[(size_t)(k + 1) * R + q], B[(size_t)(k + 2) * R + q], B[(size_t)(k + 3) * R + q]};
        acc = fmaf(av.x, bv.x, fmaf(av.y, bv.y, fmaf(av.z, bv.z, fmaf(av.w, bv.w, acc))));
    }
    const float w = wave_sum_f32(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
    __syncthreads();
    if (threadIdx.x == 0) C[(size_t)m * ldc + qq] = alpha * ((red[0] + red[1]) + (red[2] + red[3]));
}

// Few rows (decode): a block per output; with B1, outputs R..2R-1 of each row use B1.
hipError_t dot2(int da, bool bt, const void *A, long lda, const float *B0, const float *B1, int R, int M, int K, float *C, long ldc,
                float alpha, hipStream_t s)
{
    const dim3 grid(B1 ? 2 * R : R, M);
    if (da == DT_BF16) {
        if (bt)
            hipLaunchKernelGGL((k_dot<DT_BF16, true>), grid, dim3(256), 0, s, A, lda, B0, B1, R, K, C, ldc, alpha);
        else
            hipLaunchKernelGGL((k_dot<DT_BF16, false>), grid, dim3(256), 0, s, A, lda, B0, B1, R, K, C, ldc, alpha);
    } else {
        if (bt)
            hipLaunchKernelGGL((k_dot<DT_F32, true>), grid, dim3(256), 0, s, A, lda, B0, B1, R, K, C, ldc, alpha);
        else
            hipLaunchKernelGGL((k_dot<DT_F32, false>), grid, dim3(256), 0, s, A, lda, B0, B1, R, K, C, ldc, alpha);
    }
    return hipGetLastError();
}

template <int RM>
void launch_tall_rm(int da, bool bt, const void *A, long lda, const float *B, int R, int M, int K, float *C, long ldc, float alpha,
                    hipStream_t s)
{
    const dim3 grid((M + 15) / 16);
    if (da == DT_BF16) {
        if (bt)
            hipLaunchKernelGGL((k_tall<DT_BF16, true, RM>), grid, dim3(256), 0, s, A, lda, B, R, M, K, C, ldc, alpha);
        else
            hipLaunchKernelGGL((k_tall<DT_BF16, false, RM>), grid, dim3(256), 0, s, A, lda, B, R, M, K, C, ldc, alpha);
    } else {
        if (bt)
            hipLaunchKernelGGL((k_tall<DT_F32, true, RM>), grid, dim3(256), 0, s, A, lda, B, R, M, K, C, ldc, alpha);
        else
            hipLaunchKernelGGL((k_tall<DT_F32, false, RM>), grid, dim3(256), 0, s, A, lda, B, R, M, K, C, ldc, alpha);
    }
}

hipError_t tall(int da, bool bt, const void *A, long lda, const float *B, int R, int M, int K, float *C, long ldc, float alpha,
                hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    if (M <= 64) return dot2(da, bt, A, lda, B, nullptr, R, M, K, C, ldc, alpha, s);
    if (R <= 16)
        launch_tall_rm<16>(da, bt, A, lda, B, R, M, K, C, ldc, alpha, s);
    else if (R <= 32)
        launch_tall_rm<32>(da, bt, A, lda, B, R, M, K, C, ldc, alpha, s);
    else
        launch_tall_rm<64>(da, bt, A, lda, B, R, M, K, C, ldc, alpha, s);
    return hipGetLastError();
}

template <int RM>
void launch_rowsum_rm(int dc, const float *A, long lda, const void *Cm, long ldc, int R, int N, int K, int kchunk, int nz,
                      float *part, hipStream_t s)
{
    const dim3 grid((N / 4 + 63) / 64, nz);
    if (dc == DT_BF16)
        hipLaunchKernelGGL((k_rowsum<DT_BF16, RM>), grid, dim3(64), 0, s, A, lda, Cm, ldc, R, N, K, kchunk, part);
    else
        hipLaunchKernelGGL((k_rowsum<DT_F32, RM>), grid, dim3(64), 0, s, A, lda, Cm, ldc, R, N, K, kchunk, part);
}

// C(q, n) = alpha sum_k A[k][q] Cm[k][n] over k < K, written at C[q scq + n scn].
hipError_t rowsum(const float *A, long lda, int dc, const void *Cm, long ldc, int R, int N, int K, float *C, long scq, long scn,
                  float alpha, float *part, size_t cap, hipStream_t s)
{
    if (R <= 0 || N <= 0) return hipSuccess;
    if (R > 32) {  // 32 outputs per lane and column at most (registers): two passes over q
        hipError_t e = rowsum(A, lda, dc, Cm, ldc, 32, N, K, C, scq, scn, alpha, part, cap, s);
        if (e != hipSuccess) return e;
        return rowsum(A + 32, lda, dc, Cm, ldc, R - 32, N, K, C + 32 * scq, scq, scn, alpha, part, cap, s);
    }
    // chunks of rows so that about 1024 waves run, at least 16 rows each
    const int cols = (N / 4 + 63) / 64;
    int nz = std::max(1, std::min((1024 + cols - 1) / cols, (K + 15) / 16));
    while (nz > 1 && (size_t)nz * R * N > cap) nz--;
    const int kchunk = K > 0 ? (K + nz - 1) / nz : 1;
    nz = K > 0 ? (K + kchunk - 1) / kchunk : 1;
    if (R <= 16)
        launch_rowsum_rm<16>(dc, A, lda, Cm, ldc, R, N, K, kchunk, nz, part, s);
    else
        launch_rowsum_rm<32>(dc, A, lda, Cm, ldc, R, N, K, kchunk, nz, part, s);
    const size_t RN = (size_t)R * N;
    hipLaunchKernelGGL(k_rowsum_reduce, dim3((unsigned)std::min<size_t>(2048, (RN + 255) / 256)), dim3(256), 0, s, part, nz, R, N, C,
                       scq, scn, alpha);
    return hipGetLastError();
}

template <int RM>
void launch_wide_rm(bool bnq, const float *a, long lda, long a1off, const float *b0, const float *b1, long ldb, int N1, long c1off,
                    int R, int M, int N, float *C, long ldc, float alpha, bool accum, hipStream_t s)
{
    const dim3 grid((N1 / 4 + 255) / 256 + ((N - N1) / 4 + 255) / 256, (M + kWideRows - 1) / kWideRows);
    // b rows of [N][ldb] are 16-byte aligned when ldb % 4 == 0 (the bases are)
    if (bnq && ldb % 4 == 0)
        hipLaunchKernelGGL((k_wide<true, RM, true>), grid, dim3(256), 0, s, a, lda, b0, b1, ldb, N1, c1off, a1off, R, M, N, C, ldc,
                           alpha, accum ? 1 : 0);
    else if (bnq)
        hipLaunchKernelGGL((k_wide<true, RM, false>), grid, dim3(256), 0, s, a, lda, b0, b1, ldb, N1, c1off, a1off, R, M, N, C, ldc,
                           alpha, accum ? 1 : 0);
    else
        hipLaunchKernelGGL((k_wide<false, RM, true>), grid, dim3(256), 0, s, a, lda, b0, b1, ldb, N1, c1off, a1off, R, M, N, C, ldc,
                           alpha, accum ? 1 : 0);
}

// C[m][n] = alpha sum_q a[m][q] b0(n, q) [+ C] for n < N1, and columns N1 + n' =
// alpha sum_q a[m][a1off + q] b1(n', q) written at C + c1off + n' (b0 == b1, N1 == N: one
// range).  Ranks above 32 run as two passes over q, the second accumulating.
hipError_t wide2(bool bnq, const float *a, long lda, long a1off, const float *b0, const float *b1, int N1, long c1off, int R, int M,
                 int N, float *C, long ldc, float alpha, bool accum, hipStream_t s)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    // row strides of b: [N][R] rows of R; [R][width] rows of the range's width
    if (R <= 16) {
        launch_wide_rm<16>(bnq, a, lda, a1off, b0, b1, bnq ? R : 0, N1, c1off, R, M, N, C, ldc, alpha, accum, s);
    } else {
        const int r1 = std::min(R, 32);
        launch_wide_rm<32>(bnq, a, lda, a1off, b0, b1, bnq ? R : 0, N1, c1off, r1, M, N, C, ldc, alpha, accum, s);
        if (R > 32) {
            // q >= 32: a and b advanced by 32 along q
            const int w0 = N1, w1 = N - N1;
            const float *c0 = bnq ? b0 + 32 : b0 + (size_t)32 * w0, *c1 = bnq ? b1 + 32 : b1 + (size_t)32 * w1;
            if (!bnq && w0 != w1 && b0 != b1) return hipErrorInvalidValue;  // two ranges of different widths: not used
            launch_wide_rm<32>(bnq, a + 32, lda, a1off, c0, c1, bnq ? R : w0, N1, c1off, R - 32, M, N, C, ldc, alpha, true, s);
        }
    }
    return hipGetLastError();
}

hipError_t wide(bool bnq, const float *a, long lda, const float *b, int R, int M, int N, float *C, long ldc, float alpha, bool accum,
                hipStream_t s)
{
    return wide2(bnq, a, lda, 0, b, b, N, 0, R, M, N, C, ldc, alpha, accum, s);
}

// hbar[t][n] = sum_j w[t][j] h(grouped row inv[t k + j], n), j in rank order; h read from
// its bf16 hi + lo planes [S][I] (GU = false) or formed from the pre-activations g, u
// [S][2][I] (GU = true).  Four columns per thread.
template <bool GU>
__global__ __launch_bounds__(256) void k_lora_hbar(const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
                                                   const float *__restrict__ gu, int act, const int32_t *__restrict__ inv,
                                                   const float *__restrict__ w, int k, int I, float *__restrict__ hbar)
{
    const int t = blockIdx.y, n = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (n >= I) return;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
        const size_t row = (size_t)inv[t * k + j];
        const float p = w[t * k + j];
        float h[4];
        if constexpr (GU) {
            const float4 g = *(const float4 *)(gu + (2 * row) * I + n), u = *(const float4 *)(gu + (2 * row + 1) * I + n);
            h[0] = act_h(act, g.x, u.x);
            h[1] = act_h(act, g.y, u.y);
            h[2] = act_h(act, g.z, u.z);
            h[3] = act_h(act, g.w, u.w);
        } else {
            const u32x2 hi = *(const u32x2 *)(h_hi + row * I + n), lo = *(const u32x2 *)(h_lo + row * I + n);
            h[0] = bf16_bits_to_f32(hi[0] & 0xFFFFu) + bf16_bits_to_f32(lo[0] & 0xFFFFu);
            h[1] = bf16_bits_to_f32(hi[0] >> 16) + bf16_bits_to_f32(lo[0] >> 16);
            h[2] = bf16_bits_to_f32(hi[1] & 0xFFFFu) + bf16_bits_to_f32(lo[1] & 0xFFFFu);
            h[3] = bf16_bits_to_f32(hi[1] >> 16) + bf16_bits_to_f32(lo[1] >> 16);
        }
#pragma unroll
        for (int c = 0; c < 4; c++) s[c] += p * h[c];
    }
    *(float4 *)(hbar + (size_t)t * I + n) = float4{s[0], s[1], s[2], s[3]};
}

// dgu[t][c] = sum_j (dL/dg | dL/du)(grouped row inv[t k + j], c) for c < 2I, j in rank
// order; the slot rows are fp32 [S][2I] or bf16 hi + lo planes [S][2I] each.  Four
// columns per thread.
__global__ __launch_bounds__(256) void k_lora_dgu(const void *__restrict__ dgdu, int pair, const int32_t *__restrict__ inv,
                                                  int T, int k, int I, float *__restrict__ dgu)
{
    const int t = blockIdx.y, c = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    const size_t S = (size_t)T * k, row = 2 * (size_t)I;
    if (c >= 2 * I) return;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
        const size_t o = (size_t)inv[t * k + j] * row + c;
        if (pair) {
            const uint16_t *hi = (const uint16_t *)dgdu;
            const u32x2 h = *(const u32x2 *)(hi + o), l = *(const u32x2 *)(hi + S * row + o);
            s[0] += bf16_bits_to_f32(h[0] & 0xFFFFu) + bf16_bits_to_f32(l[0] & 0xFFFFu);
            s[1] += bf16_bits_to_f32(h[0] >> 16) + bf16_bits_to_f32(l[0] >> 16);
            s[2] += bf16_bits_to_f32(h[1] & 0xFFFFu) + bf16_bits_to_f32(l[1] & 0xFFFFu);
            s[3] += bf16_bits_to_f32(h[1] >> 16) + bf16_bits_to_f32(l[1] >> 16);
        } else {
            const float4 v = *(const float4 *)((const float *)dgdu + o);
            s[0] += v.x;
            s[1] += v.y;
            s[2] += v.z;
            s[3] += v.w;
        }
    }
    *(float4 *)(dgu + (size_t)t * row + c) = float4{s[0], s[1], s[2], s[3]};
}

__global__ __launch_bounds__(256) void k_fill_zero(float *__restrict__ p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.f;
}

unsigned blocks_for(size_t n) { return (unsigned)std::max<size_t>(1, std::min<size_t>(4096, (n + 255) / 256)); }

}  // namespace

hipError_t lora_forward_pre(const LoraW &L, const LoraWs &w, const void *x, int xt, int T, int H, int I, hipStream_t s)
{
    const int r = L.r;
    hipError_t e = hipSuccess;
    // vx = [A_g x | A_u x]  [T][2r];  lora_gu = s [vx_g B_g^T | vx_u B_u^T]  [T][2I]
    if (T <= 64)
        e = dot2(xt, true, x, H, L.A[0], L.A[1], r, T, H, w.vx, 2 * r, 1.f, s);
    else
        for (int m = 0; m < 2 && e == hipSuccess; m++) e = tall(xt, true, x, H, L.A[m], r, T, H, w.vx + m * r, 2 * r, 1.f, s);
    // both halves in one launch: columns I.. use B_u, vx_u, and land at +I
    if (e == hipSuccess) e = wide2(true, w.vx, 2 * r, r, L.B[0], L.B[1], I, I, r, T, 2 * I, w.gu, 2 * I, L.scale, false, s);
    return e;
}

hipError_t lora_forward_vx(const LoraW &L, const LoraWs &w, const void *x, int xt, int T, int H, hipStream_t s)
{
    const int r = L.r;
    if (T <= 64) return dot2(xt, true, x, H, L.A[0], L.A[1], r, T, H, w.vx, 2 * r, 1.f, s);
    hipError_t e = hipSuccess;
    for (int m = 0; m < 2 && e == hipSuccess; m++) e = tall(xt, true, x, H, L.A[m], r, T, H, w.vx + m * r, 2 * r, 1.f, s);
    return e;
}

// hbar and z = hbar A_d^T  [T][r]; h from its planes (gu == nullptr) or from g, u.
hipError_t lora_down_z(const LoraW &L, const LoraWs &w, const uint16_t *h_hi, const uint16_t *h_lo, const float *gu, int act,
                       const int32_t *inv, const float *pw, int T, int k, int I, hipStream_t s)
{
    const dim3 grid((I / 4 + 255) / 256, T);
    if (gu)
        hipLaunchKernelGGL(k_lora_hbar<true>, grid, dim3(256), 0, s, h_hi, h_lo, gu, act, inv, pw, k, I, w.hbar);
    else
        hipLaunchKernelGGL(k_lora_hbar<false>, grid, dim3(256), 0, s, h_hi, h_lo, gu, act, inv, pw, k, I, w.hbar);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return tall(DT_F32, true, w.hbar, I, L.A[2], L.r, T, I, w.z, L.r, 1.f, s);
}

hipError_t lora_forward_post(const LoraW &L, const LoraWs &w, const ExpertFwdArgs &a, const int32_t *inv, hipStream_t s)
{
    hipError_t e = lora_down_z(L, w, a.h_hi, a.h_lo, nullptr, a.act, inv, a.w, a.T, a.k, a.I, s);
    if (e != hipSuccess) return e;
    // y += s z B_d^T
    return wide(true, w.z, L.r, L.B[2], L.r, a.T, a.H, a.y, a.H, L.scale, true, s);
}

hipError_t lora_backward_pre(const LoraW &L, const LoraWs &w, const void *dy, int dyt, int T, int H, int I, hipStream_t s)
{
    const int r = L.r;
    // wd = dy B_d  [T][r]; c = s wd A_d  [T][I]
    hipError_t e = tall(dyt, false, dy, H, L.B[2], r, T, H, w.wd, r, 1.f, s);
    if (e != hipSuccess) return e;
    return wide(false, w.wd, r, L.A[2], r, T, I, w.c, I, L.scale, false, s);
}

hipError_t lora_backward_post(const LoraW &L, const LoraWs &w, const ExpertBwdArgs &a, bool pair, hipStream_t s)
{
    const int r = L.r, T = a.T, H = a.H, I = a.I;
    // dgu = per-token sums of dL/dg, dL/du  [T][2I]
    hipLaunchKernelGGL(k_lora_dgu, dim3((I / 2 + 255) / 256, T), dim3(256), 0, s, (const void *)a.dgdu, pair ? 1 : 0, a.inv, T,
                       a.k, I, w.dgu);
    hipError_t e = hipGetLastError();
    // m = [dgu_g B_g | dgu_u B_u]  [T][2r];  dx += s (m_g A_g + m_u A_u)
    for (int m = 0; m < 2 && e == hipSuccess; m++) e = tall(DT_F32, false, w.dgu + (size_t)m * I, 2 * I, L.B[m], r, T, I, w.m + m * r, 2 * r, 1.f, s);
    for (int m = 0; m < 2 && e == hipSuccess; m++) e = wide(false, w.m + m * r, 2 * r, L.A[m], r, T, H, a.dx, H, L.scale, true, s);
    return e;
}

hipError_t lora_grads(const LoraW &L, const LoraWs &w, const ExpertBwdArgs &a, float *const dA[3], float *const dB[3],
                      hipStream_t s)
{
    const int r = L.r, T = a.T, H = a.H, I = a.I;
    hipError_t e = lora_down_z(L, w, a.h_hi, a.h_lo, a.gu, a.act, a.inv, a.w, T, a.k, I, s);
    for (int m = 0; m < 2 && e == hipSuccess; m++) {
        // dB = s dgu^T vx  [I][r];  dA = s m^T x  [r][H]
        e = rowsum(w.vx + m * r, 2 * r, DT_F32, w.dgu + (size_t)m * I, 2 * I, r, I, T, dB[m], 1, r, L.scale, w.part, w.part_cap, s);
        if (e == hipSuccess) e = rowsum(w.m + m * r, 2 * r, a.xt, a.x, H, r, H, T, dA[m], H, 1, L.scale, w.part, w.part_cap, s);
    }
    // dB_d = s dy^T z  [H][r];  dA_d = s wd^T hbar  [r][I]
    if (e == hipSuccess) e = rowsum(w.z, r, a.dyt, a.dy, H, r, H, T, dB[2], 1, r, L.scale, w.part, w.part_cap, s);
    if (e == hipSuccess) e = rowsum(w.wd, r, DT_F32, w.hbar, I, r, I, T, dA[2], I, 1, L.scale, w.part, w.part_cap, s);
    return e;
}

hipError_t fill_zero(float *p, size_t n, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3(blocks_for(n)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace moe
