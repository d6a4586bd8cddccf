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
// Everything here is skinny fp32 GEMMs (one dimension is the rank) with fp32 accumulation
// in a fixed order (split-K partial sums reduced in chunk order), plus three gathers over
// the grouped slot rows.
#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

enum { OD_F32 = 0, OD_BF16 = 1, OD_PAIR = 2 };  // operand storage: fp32, bf16, bf16 hi + lo planes

struct Opnd {
    const void *p, *p2;  // p2: the lo plane of OD_PAIR
    long s0, s1;         // element (i, j) at index i s0 + j s1
};

template <int D>
__device__ __forceinline__ float ld_op(const Opnd &o, long idx)
{
    if constexpr (D == OD_F32) return ((const float *)o.p)[idx];
    if constexpr (D == OD_BF16) return bf16_bits_to_f32(((const uint16_t *)o.p)[idx]);
    return bf16_bits_to_f32(((const uint16_t *)o.p)[idx]) + bf16_bits_to_f32(((const uint16_t *)o.p2)[idx]);
}

// C (M x N) = alpha A (M x K) B (K x N) [+ C]; A element (m, k) = a[m s0 + k s1], B element
// (k, n) = b[k s0 + n s1], C element (m, n) at c[m scm + n scn].  With gridDim.z > 1 each
// z-block sums its chunk of K into part[z][M][N] instead (reduced by k_gemm_reduce).
struct GemmArgs {
    Opnd a, b;
    float *c;
    long scm, scn;
    int M, N, K, kchunk;
    float alpha;
    int accum;
    float *part;
};

constexpr int kBK = 16;

template <int DA, int DB, int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs g)
{
    constexpr int TN = 4, TM = 4, NX = BN / TN;
    static_assert((BM / TM) * (BN / TN) == 256, "256 threads of 4 x 4 outputs");
    __shared__ float As[kBK][BM + 4], Bs[kBK][BN + 4];
    const int tid = threadIdx.x, tx = tid % NX, ty = tid / NX;
    const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;
    const int kb = blockIdx.z * g.kchunk, ke = min(g.K, kb + g.kchunk);
    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = 0.f;
    const bool a_k1 = g.a.s1 == 1, b_n1 = g.b.s1 == 1;
    for (int k0 = kb; k0 < ke; k0 += kBK) {
        for (int e = tid; e < BM * kBK; e += 256) {
            const int mm = a_k1 ? e / kBK : e % BM, kk = a_k1 ? e % kBK : e / BM;
            const int m = m0 + mm, k = k0 + kk;
            As[kk][mm] = (m < g.M && k < ke) ? ld_op<DA>(g.a, (long)m * g.a.s0 + (long)k * g.a.s1) : 0.f;
        }
        for (int e = tid; e < kBK * BN; e += 256) {
            const int nn = b_n1 ? e % BN : e / kBK, kk = b_n1 ? e / BN : e % kBK;
            const int n = n0 + nn, k = k0 + kk;
            Bs[kk][nn] = (n < g.N && k < ke) ? ld_op<DB>(g.b, (long)k * g.b.s0 + (long)n * g.b.s1) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk++) {
            float av[TM], bv[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) av[i] = As[kk][ty * TM + i];
#pragma unroll
            for (int j = 0; j < TN; j++) bv[j] = Bs[kk][tx * TN + j];
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int m = m0 + ty * TM + i;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int n = n0 + tx * TN + j;
            if (n >= g.N) continue;
            if (gridDim.z > 1) {
                g.part[((size_t)blockIdx.z * g.M + m) * g.N + n] = acc[i][j];
            } else {
                float *c = g.c + (long)m * g.scm + (long)n * g.scn;
                *c = g.alpha * acc[i][j] + (g.accum ? *c : 0.f);
            }
        }
    }
}

// C = alpha sum_z part[z] [+ C], the chunks added in order.
__global__ __launch_bounds__(256) void k_gemm_reduce(const GemmArgs g, int nz)
{
    const size_t MN = (size_t)g.M * g.N;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += (size_t)gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int z = 0; z < nz; z++) s += g.part[z * MN + i];
        const int m = (int)(i / g.N), n = (int)(i % g.N);
        float *c = g.c + (long)m * g.scm + (long)n * g.scn;
        *c = g.alpha * s + (g.accum ? *c : 0.f);
    }
}

template <int DA, int DB>
void launch_gemm_t(GemmArgs g, dim3 grid, int bm, int bn, hipStream_t s)
{
    if (bn == 16)
        hipLaunchKernelGGL((k_gemm<DA, DB, 256, 16>), grid, dim3(256), 0, s, g);
    else if (bm == 16)
        hipLaunchKernelGGL((k_gemm<DA, DB, 16, 256>), grid, dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((k_gemm<DA, DB, 64, 64>), grid, dim3(256), 0, s, g);
}

template <int DA>
void launch_gemm_a(int db, GemmArgs g, dim3 grid, int bm, int bn, hipStream_t s)
{
    if (db == OD_F32)
        launch_gemm_t<DA, OD_F32>(g, grid, bm, bn, s);
    else if (db == OD_BF16)
        launch_gemm_t<DA, OD_BF16>(g, grid, bm, bn, s);
    else
        launch_gemm_t<DA, OD_PAIR>(g, grid, bm, bn, s);
}

// Tile shape by the skinny side (rank-sized dimensions are <= 64); K split into chunks
// when the output tiles alone would not fill the chip, partial sums in part (cap floats).
hipError_t gemm(int da, int db, GemmArgs g, float *part, size_t cap, hipStream_t s)
{
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    int bm = 64, bn = 64;
    if (g.N <= 16)
        bm = 256, bn = 16;
    else if (g.M <= 16)
        bm = 16, bn = 256;
    const int tiles = ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
    int nz = 1;
    if (g.K > 0 && tiles < 512) {
        nz = std::min((1024 + tiles - 1) / tiles, (g.K + 255) / 256);
        while (nz > 1 && (size_t)nz * g.M * g.N > cap) nz--;
    }
    g.kchunk = ((g.K + nz - 1) / nz + kBK - 1) / kBK * kBK;
    if (g.K <= 0) g.kchunk = kBK;
    nz = g.K > 0 ? (g.K + g.kchunk - 1) / g.kchunk : 1;
    g.part = part;
    const dim3 grid((g.M + bm - 1) / bm, (g.N + bn - 1) / bn, nz);
    if (da == OD_F32)
        launch_gemm_a<OD_F32>(db, g, grid, bm, bn, s);
    else if (da == OD_BF16)
        launch_gemm_a<OD_BF16>(db, g, grid, bm, bn, s);
    else
        launch_gemm_a<OD_PAIR>(db, g, grid, bm, bn, s);
    if (nz > 1) {
        const size_t MN = (size_t)g.M * g.N;
        hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)std::min<size_t>(1024, (MN + 255) / 256)), dim3(256), 0, s, g, nz);
    }
    return hipGetLastError();
}

GemmArgs gargs(Opnd a, Opnd b, float *c, long scm, long scn, int M, int N, int K, float alpha, bool accum)
{
    GemmArgs g{};
    g.a = a;
    g.b = b;
    g.c = c;
    g.scm = scm;
    g.scn = scn;
    g.M = M;
    g.N = N;
    g.K = K;
    g.alpha = alpha;
    g.accum = accum ? 1 : 0;
    return g;
}

Opnd op(const void *p, long s0, long s1, const void *p2 = nullptr) { return Opnd{p, p2, s0, s1}; }

int od(int dt) { return dt == DT_BF16 ? OD_BF16 : OD_F32; }

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
// order; the slot rows are fp32 [S][2I] or bf16 hi + lo planes [S][2I] each.
__global__ __launch_bounds__(256) void k_lora_dgu(const void *__restrict__ dgdu, int pair, const int32_t *__restrict__ inv,
                                                  int T, int k, int I, float *__restrict__ dgu)
{
    const int t = blockIdx.y;
    const size_t S = (size_t)T * k, row = 2 * (size_t)I;
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < 2 * I; c += gridDim.x * blockDim.x) {
        float s = 0.f;
        for (int j = 0; j < k; j++) {
            const size_t o = (size_t)inv[t * k + j] * row + c;
            if (pair) {
                const uint16_t *hi = (const uint16_t *)dgdu;
                s += bf16_bits_to_f32(hi[o]) + bf16_bits_to_f32(hi[S * row + o]);
            } else {
                s += ((const float *)dgdu)[o];
            }
        }
        dgu[(size_t)t * row + c] = s;
    }
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
    hipError_t e;
    // vx = [A_g x | A_u x]  [T][2r]
    for (int m = 0; m < 2; m++) {
        e = gemm(od(xt), OD_F32, gargs(op(x, H, 1), op(L.A[m], 1, H), w.vx + m * r, 2 * r, 1, T, r, H, 1.f, false),
                 w.part, w.part_cap, s);
        if (e != hipSuccess) return e;
    }
    // lora_gu = s [vx_g B_g^T | vx_u B_u^T]  [T][2I]
    for (int m = 0; m < 2; m++) {
        e = gemm(OD_F32, OD_F32, gargs(op(w.vx + m * r, 2 * r, 1), op(L.B[m], 1, r), w.gu + (size_t)m * I, 2 * I, 1, T, I, r,
                                       L.scale, false),
                 w.part, w.part_cap, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
    return gemm(OD_F32, OD_F32, gargs(op(w.hbar, I, 1), op(L.A[2], 1, I), w.z, L.r, 1, T, L.r, I, 1.f, false), w.part, w.part_cap,
                s);
}

hipError_t lora_forward_post(const LoraW &L, const LoraWs &w, const ExpertFwdArgs &a, const int32_t *inv, hipStream_t s)
{
    hipError_t e = lora_down_z(L, w, a.h_hi, a.h_lo, nullptr, a.act, inv, a.w, a.T, a.k, a.I, s);
    if (e != hipSuccess) return e;
    // y += s z B_d^T
    return gemm(OD_F32, OD_F32, gargs(op(w.z, L.r, 1), op(L.B[2], 1, L.r), a.y, a.H, 1, a.T, a.H, L.r, L.scale, true), w.part,
                w.part_cap, s);
}

hipError_t lora_backward_pre(const LoraW &L, const LoraWs &w, const void *dy, int dyt, int T, int H, int I, hipStream_t s)
{
    const int r = L.r;
    // wd = dy B_d  [T][r]; c = s wd A_d  [T][I]
    hipError_t e = gemm(od(dyt), OD_F32, gargs(op(dy, H, 1), op(L.B[2], r, 1), w.wd, r, 1, T, r, H, 1.f, false), w.part, w.part_cap, s);
    if (e != hipSuccess) return e;
    return gemm(OD_F32, OD_F32, gargs(op(w.wd, r, 1), op(L.A[2], I, 1), w.c, I, 1, T, I, r, L.scale, false), w.part, w.part_cap, s);
}

hipError_t lora_backward_post(const LoraW &L, const LoraWs &w, const ExpertBwdArgs &a, bool pair, hipStream_t s)
{
    const int r = L.r, T = a.T, H = a.H, I = a.I;
    // dgu = per-token sums of dL/dg, dL/du  [T][2I]
    hipLaunchKernelGGL(k_lora_dgu, dim3((2 * I + 255) / 256, T), dim3(256), 0, s, (const void *)a.dgdu, pair ? 1 : 0, a.inv, T,
                       a.k, I, w.dgu);
    hipError_t e = hipGetLastError();
    // m = [dgu_g B_g | dgu_u B_u]  [T][2r]
    for (int m = 0; m < 2 && e == hipSuccess; m++)
        e = gemm(OD_F32, OD_F32, gargs(op(w.dgu + (size_t)m * I, 2 * I, 1), op(L.B[m], r, 1), w.m + m * r, 2 * r, 1, T, r, I, 1.f,
                                       false),
                 w.part, w.part_cap, s);
    // dx += s (m_g A_g + m_u A_u)
    for (int m = 0; m < 2 && e == hipSuccess; m++)
        e = gemm(OD_F32, OD_F32, gargs(op(w.m + m * r, 2 * r, 1), op(L.A[m], H, 1), a.dx, H, 1, T, H, r, L.scale, true), w.part,
                 w.part_cap, s);
    return e;
}

hipError_t lora_grads(const LoraW &L, const LoraWs &w, const ExpertBwdArgs &a, float *const dA[3], float *const dB[3],
                      hipStream_t s)
{
    const int r = L.r, T = a.T, H = a.H, I = a.I;
    hipError_t e = lora_down_z(L, w, a.h_hi, a.h_lo, a.gu, a.act, a.inv, a.w, T, a.k, I, s);
    for (int m = 0; m < 2 && e == hipSuccess; m++) {
        // dB = s dgu^T vx  [I][r];  dA = s m^T x  [r][H]
        e = gemm(OD_F32, OD_F32, gargs(op(w.dgu + (size_t)m * I, 1, 2 * I), op(w.vx + m * r, 2 * r, 1), dB[m], r, 1, I, r, T, L.scale,
                                       false),
                 w.part, w.part_cap, s);
        if (e == hipSuccess)
            e = gemm(OD_F32, od(a.xt), gargs(op(w.m + m * r, 1, 2 * r), op(a.x, H, 1), dA[m], H, 1, r, H, T, L.scale, false), w.part,
                     w.part_cap, s);
    }
    // dB_d = s dy^T z  [H][r]
    if (e == hipSuccess)
        e = gemm(od(a.dyt), OD_F32, gargs(op(a.dy, 1, H), op(w.z, r, 1), dB[2], r, 1, H, r, T, L.scale, false), w.part, w.part_cap, s);
    // dA_d = s wd^T hbar  [r][I]
    if (e == hipSuccess)
        e = gemm(OD_F32, OD_F32, gargs(op(w.wd, 1, r), op(w.hbar, I, 1), dA[2], I, 1, r, I, T, L.scale, false), w.part, w.part_cap,
                 s);
    return e;
}

hipError_t fill_zero(float *p, size_t n, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3(blocks_for(n)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace moe
