// expert_fwd.hip -- routed-expert forward: fused dequant + gate/up + SwiGLU,
// down projection with the routing weight, and a fixed-order combine.
//
// Per routed slot (t, j) with expert e and weight p (LazyLoRA README, "The
// engine" / "Arithmetic": MXFP4 experts consumed packed, fused decode-and-dot,
// fp32 accumulation; "File map": the combine uses the routing weights):
//   g = Wg x_t,  u = Wu x_t,  h = silu(g) * u,  o = Wd h,  y_t = sum_j p_tj o_tj.
// The quantized weights are dequantized in registers straight from HBM (each
// active expert's bytes are read once per token tile) and fed to bf16 MFMA
// with fp32 accumulation.  MXFP4 dequantizes exactly to bf16; bf16 tokens are
// exact; fp32 operands (fp32 tokens, h) are split into bf16 hi + lo.
//
// Block = 4 waves x 16 rows = 64 rows of one active expert (blockIdx.y indexes
// the device-side active list; blocks past *n_active exit), all of that
// expert's tokens in tiles of 16*NTT.
#include "expert_frag.h"

namespace moe {

template <int WFMT, int XT, int NTT>
__global__ __launch_bounds__(256) void k_gateup(const ExpertFwdArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t cbs[WFMT == FMT_RVQ3 ? 2 * 3 * 256 * 8 : 8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int ai = blockIdx.y;
    if (ai >= *a.n_active) return;
    const int e = a.active[ai];
    if constexpr (WFMT == FMT_RVQ3) {
        load_codebooks(a.gate, e, cbs);
        load_codebooks(a.up, e, cbs + 3 * 256 * 8);
        __syncthreads();
    }
    const int H = a.H, I = a.I;
    const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;
    const int n0 = blockIdx.x * 64 + wv * 16;
    if (n0 >= I) return;
    const int row = n0 + li;
    for (int tt0 = 0; tt0 < ntok; tt0 += 16 * NTT) {
        f32x4 accg[NTT], accu[NTT];
        size_t xoff[NTT];
        bool tv[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            accg[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accu[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int j = tt0 + 16 * tt + li;
            tv[tt] = j < ntok;
            xoff[tt] = tv[tt] ? (size_t)(a.perm[r0 + j] / a.k) * H : 0;
        }
        for (int k0 = 0; k0 < H; k0 += 256) {
            const int kk = k0 + 64 * g;
            AFrag<WFMT> ag, au;
            ag.load(a.gate, e, I, H, row, kk, cbs);
            au.load(a.up, e, I, H, row, kk, cbs + 3 * 256 * 8);
#pragma unroll
            for (int tt = 0; tt < NTT; tt++) {
                BFrag<XT> b;
                b.load(a.x, xoff[tt], kk, H, tv[tt]);
                mma_step(accg[tt], ag, b);
                mma_step(accu[tt], au, b);
            }
        }
        // epilogue: lane holds rows n0 + 4g + r for token tt0 + 16tt + li
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            const int j = tt0 + 16 * tt + li;
            if (j >= ntok) continue;
            const size_t rr = (size_t)(r0 + j);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int n = n0 + 4 * g + r;
                const float gv = accg[tt][r], uv = accu[tt][r];
                a.h[rr * I + n] = gv * sigmoidf_(gv) * uv;
                if (a.gu) {
                    a.gu[(rr * 2 + 0) * I + n] = gv;
                    a.gu[(rr * 2 + 1) * I + n] = uv;
                }
            }
        }
    }
}

template <int WFMT, int NTT>
__global__ __launch_bounds__(256) void k_down(const ExpertFwdArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t cbs[WFMT == FMT_RVQ3 ? 3 * 256 * 8 : 8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int ai = blockIdx.y;
    if (ai >= *a.n_active) return;
    const int e = a.active[ai];
    if constexpr (WFMT == FMT_RVQ3) {
        load_codebooks(a.down, e, cbs);
        __syncthreads();
    }
    const int H = a.H, I = a.I;
    const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;
    const int m0 = blockIdx.x * 64 + wv * 16;
    if (m0 >= H) return;
    const int row = m0 + li;
    for (int tt0 = 0; tt0 < ntok; tt0 += 16 * NTT) {
        f32x4 acc[NTT];
        size_t hoff[NTT];
        bool tv[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int j = tt0 + 16 * tt + li;
            tv[tt] = j < ntok;
            hoff[tt] = tv[tt] ? (size_t)(r0 + j) * I : 0;
        }
        for (int k0 = 0; k0 < I; k0 += 256) {
            const int kk = k0 + 64 * g;
            AFrag<WFMT> ad;
            ad.load(a.down, e, H, I, row, kk, cbs);
#pragma unroll
            for (int tt = 0; tt < NTT; tt++) {
                BFrag<DT_F32> b;
                b.load(a.h, hoff[tt], kk, I, tv[tt]);
                mma_step(acc[tt], ad, b);
            }
        }
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            const int j = tt0 + 16 * tt + li;
            if (j >= ntok) continue;
            const int slot = a.perm[r0 + j];
            const float p = a.w[slot];
#pragma unroll
            for (int r = 0; r < 4; r++) a.ybuf[(size_t)slot * H + m0 + 4 * g + r] = p * acc[tt][r];
        }
    }
}

// y[t] = sum over j in rank order of the weighted slot rows (deterministic).
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ ybuf, int T, int H, int k,
                                                 float *__restrict__ y)
{
    const size_t n4 = (size_t)T * H / 4;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        const size_t t = i / (H / 4), m4 = i % (H / 4);
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; j++) {
            const float4 v = *(const float4 *)(ybuf + ((size_t)t * k + j) * H + 4 * m4);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *(float4 *)(y + (size_t)t * H + 4 * m4) = acc;
    }
}

template <int WFMT, int XT, int NTT>
static hipError_t fwd_launch(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    {
        ProfScope ps(a.prof, PK_GATEUP, s);
        hipLaunchKernelGGL((k_gateup<WFMT, XT, NTT>), dim3((a.I + 63) / 64, maxU), dim3(256), 0, s, a);
    }
    {
        ProfScope ps(a.prof, PK_DOWN, s);
        hipLaunchKernelGGL((k_down<WFMT, NTT>), dim3((a.H + 63) / 64, maxU), dim3(256), 0, s, a);
    }
    const size_t n4 = (size_t)a.T * a.H / 4;
    const size_t nb = (n4 + 255) / 256;
    const int blocks = (int)(nb < 4096 ? nb : 4096);
    {
        ProfScope ps(a.prof, PK_COMBINE, s);
        hipLaunchKernelGGL(k_combine, dim3(blocks), dim3(256), 0, s, a.ybuf, a.T, a.H, a.k, a.y);
    }
    return hipGetLastError();
}

template <int WFMT, int XT>
static hipError_t fwd_ntt(const ExpertFwdArgs &a, hipStream_t s)
{
    return a.T <= 64 ? fwd_launch<WFMT, XT, 1>(a, s) : fwd_launch<WFMT, XT, 4>(a, s);
}

template <int WFMT, int XT>
static hipError_t gateup_only(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    ProfScope ps(a.prof, PK_GATEUP, s);
    if (a.T <= 64)
        hipLaunchKernelGGL((k_gateup<WFMT, XT, 1>), dim3((a.I + 63) / 64, maxU), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_gateup<WFMT, XT, 4>), dim3((a.I + 63) / 64, maxU), dim3(256), 0, s, a);
    return hipGetLastError();
}

// gate/up + SwiGLU only (the backward recomputes g and u when they were not saved)
hipError_t launch_gateup_only(const ExpertFwdArgs &a, hipStream_t s)
{
    if (a.wfmt == FMT_MXFP4)
        return a.xt == DT_BF16 ? gateup_only<FMT_MXFP4, DT_BF16>(a, s) : gateup_only<FMT_MXFP4, DT_F32>(a, s);
    return a.xt == DT_BF16 ? gateup_only<FMT_RVQ3, DT_BF16>(a, s) : gateup_only<FMT_RVQ3, DT_F32>(a, s);
}

hipError_t launch_expert_forward(const ExpertFwdArgs &a, hipStream_t s)
{
    if (a.wfmt == FMT_MXFP4)
        return a.xt == DT_BF16 ? fwd_ntt<FMT_MXFP4, DT_BF16>(a, s) : fwd_ntt<FMT_MXFP4, DT_F32>(a, s);
    return a.xt == DT_BF16 ? fwd_ntt<FMT_RVQ3, DT_BF16>(a, s) : fwd_ntt<FMT_RVQ3, DT_F32>(a, s);
}

}  // namespace moe
