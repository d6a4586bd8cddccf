// router.hip -- router logits and top-k + softmax for gfx950.
//
// Router (LazyLoRA README, "File map": top-16 gating with a score-correction
// bias; "The engine": 896 routed experts, top-16): logits l[t][e] = x[t]·Wr[e]
// (+ b[e]), the k largest are selected (equal logits rank the lower expert id
// first) and the combining weights are the softmax over the k selected logits.
//
// Logits are formed in fp32 with fp32 FMA chains.  Alongside each logit the kernels
// store a rigorous bound beta >= |l_fp32 - l_exact| computed a posteriori: with
// round-to-nearest every FMA or add z -> fl(z) errs by at most u |fl(z)| (u = 2^-24,
// Higham, Accuracy and Stability of Numerical Algorithms, sec. 2.2), and in a sum
// the rounding errors add up exactly, so u times the sum of the absolute values of
// all rounded intermediate results of the actual reduction tree bounds the error.
// That sum is accumulated in fp32 beside the logit (its own relative error is far
// below the 1e-3 margin applied).  Tokens whose selection or rank order is not
// decided by the intervals [l - beta, l + beta] have their candidate logits
// recomputed in fp64 (the products of fp32/bf16 inputs are exact in fp64) and are
// re-ranked on those values.
#include "common.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ void load_x4(const void *x, int xt, size_t off, float &a, float &b, float &c, float &d)
{
    if (xt == DT_BF16) {
        u32x2 v = *(const u32x2 *)((const uint16_t *)x + off);
        a = __uint_as_float(v[0] << 16);
        b = __uint_as_float(v[0] & 0xFFFF0000u);
        c = __uint_as_float(v[1] << 16);
        d = __uint_as_float(v[1] & 0xFFFF0000u);
    } else {
        float4 v = *(const float4 *)((const float *)x + off);
        a = v.x; b = v.y; c = v.z; d = v.w;
    }
}

__device__ __forceinline__ float load_x1(const void *x, int xt, size_t off)
{
    return xt == DT_BF16 ? bf16_bits_to_f32(((const uint16_t *)x)[off]) : ((const float *)x)[off];
}

constexpr float kU = 0x1p-24f;

__device__ __forceinline__ float bound_of(float eb, float l)
{
    return 1.001f * kU * eb + kU * fabsf(l) + 1e-30f;
}

// GEMV form for up to 64 tokens and H <= 4096: one block per (pair of experts, group of 8
// tokens).  Thread tid owns the float4 chunks tid + 256 m of both router rows (held in
// registers, all eight loads issued together) and runs one FMA chain per (expert, token)
// over them; the 64 lanes of a wave are summed by the DPP tree and the four wave sums in a
// fixed order.  Grid: (ceil(E / 2), ceil(T / 8)).
constexpr int kGemvMaxT = 64;
constexpr int kGemvMaxH = 4096;
constexpr int kGemvE = 2;  // experts per block

template <int XT>
__global__ __launch_bounds__(256) void k_router_gemv(const void *__restrict__ x, const float *__restrict__ wr,
                                                     const float *__restrict__ bias, int T, int H, int E,
                                                     float *__restrict__ logits, float *__restrict__ beta)
{
    __shared__ float ps[kGemvE][4][8], pe[kGemvE][4][8];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int e0 = blockIdx.x * kGemvE, t0 = blockIdx.y * 8;
    const int n4 = H / 4;
    // A token's x pieces (4 values each, 4 per thread) are loaded as raw bits and widened only
    // when the token is multiplied: widening at the load would wait for it there.  The first
    // token's pieces go out before the Wr rows, each later token's while the one before it is
    // multiplied (unconditionally, which keeps the compiler from moving pending registers at
    // a branch; clamped in bounds, pieces past H count as 0).
    using XRaw = std::conditional_t<XT == DT_BF16, u32x2, u32x4>;
    XRaw xr[4];
    auto load_xr = [&](int t) {
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const size_t off = (size_t)min(t, T - 1) * H + 4 * min(tid + 256 * m, n4 - 1);
            if constexpr (XT == DT_BF16)
                xr[m] = *(const u32x2 *)((const uint16_t *)x + off);
            else
                xr[m] = *(const u32x4 *)((const float *)x + off);
        }
    };
    load_xr(t0);
    float4 w4[kGemvE][4];
#pragma unroll
    for (int j = 0; j < kGemvE; j++) {
        const float *wrow = wr + (size_t)min(e0 + j, E - 1) * H;
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const int c = tid + 256 * m;
            w4[j][m] = c < n4 ? *(const float4 *)(wrow + 4 * c) : float4{0.f, 0.f, 0.f, 0.f};
        }
    }
    float acc[kGemvE][8], eb[kGemvE][8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
#pragma unroll
        for (int j = 0; j < kGemvE; j++) acc[j][u] = eb[j][u] = 0.f;
        const int t = t0 + u;
        if (t >= T) continue;
        float xv[4][4];
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const bool in = tid + 256 * m < n4;
            if constexpr (XT == DT_BF16) {
                xv[m][0] = in ? __uint_as_float(xr[m][0] << 16) : 0.f;
                xv[m][1] = in ? __uint_as_float(xr[m][0] & 0xFFFF0000u) : 0.f;
                xv[m][2] = in ? __uint_as_float(xr[m][1] << 16) : 0.f;
                xv[m][3] = in ? __uint_as_float(xr[m][1] & 0xFFFF0000u) : 0.f;
            } else {
#pragma unroll
                for (int q = 0; q < 4; q++) xv[m][q] = in ? __uint_as_float(xr[m][q]) : 0.f;
            }
        }
        if (u + 1 < 8) load_xr(t + 1);
#pragma unroll
        for (int j = 0; j < kGemvE; j++) {
#pragma unroll
            for (int m = 0; m < 4; m++) {
                if (tid + 256 * m >= n4) break;
                acc[j][u] = fmaf(xv[m][0], w4[j][m].x, acc[j][u]);
                eb[j][u] += fabsf(acc[j][u]);
                acc[j][u] = fmaf(xv[m][1], w4[j][m].y, acc[j][u]);
                eb[j][u] += fabsf(acc[j][u]);
                acc[j][u] = fmaf(xv[m][2], w4[j][m].z, acc[j][u]);
                eb[j][u] += fabsf(acc[j][u]);
                acc[j][u] = fmaf(xv[m][3], w4[j][m].w, acc[j][u]);
                eb[j][u] += fabsf(acc[j][u]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 8; u++) {
        if (t0 + u >= T) break;
#pragma unroll
        for (int j = 0; j < kGemvE; j++) {
            float ebt = eb[j][u];
            const float sv = wave_sum_f32_eb(acc[j][u], ebt);
            if (lane == 0) {
                ps[j][wv][u] = sv;
                pe[j][wv][u] = ebt;
            }
        }
    }
    __syncthreads();
    if (tid < 8 * kGemvE) {
        const int u = tid & 7, j = tid >> 3, t = t0 + u, e = e0 + j;
        if (t < T && e < E) {
            const float s01 = ps[j][0][u] + ps[j][1][u], s23 = ps[j][2][u] + ps[j][3][u], r = s01 + s23;
            const float ebt = ((pe[j][0][u] + pe[j][1][u]) + fabsf(s01)) + ((pe[j][2][u] + pe[j][3][u]) + fabsf(s23)) + fabsf(r);
            const float l = r + (bias ? bias[e] : 0.f);
            logits[(size_t)t * E + e] = l;
            beta[(size_t)t * E + e] = bound_of(ebt, l);
        }
    }
}

// Many tokens: logits on the fp64 matrix cores (v_mfma_f64_16x16x4_f64).  The fp32 (or
// bf16) inputs are exact in fp64 and so are their products; only the fp64 additions
// round, so |l64 - l| <= gamma_H sum_i |x_i w_i| <= gamma_H ||x|| ||w|| (Higham, sec. 3.1,
// any summation order, each add erring by at most u = 2^-53 of its result; Cauchy-Schwarz
// for the sum), taken twice over as a margin for the unit's internal order.  The logit is
// returned in fp32 with beta = that bound + |l64 - l32| + the bias add's rounding, rounded
// upwards, so the top-k certifies on the same intervals as for the fp32 kernels; only
// logits within ~1e-7 of each other call for the fp64 re-ranking.
// Block = 64 tokens x 64 experts, four waves of 32 x 32 (2 x 2 MFMA tiles); K in chunks of
// 32 staged in LDS as fp32 (row stride 36: the 64 single-element fragment reads of an
// MFMA operand hit 64 distinct banks).  Operand layouts: A lane l = (row l % 16, k l / 16),
// B lane l = (k l / 16, column l % 16); result value i of lane l = (row 4 i + l / 16,
// column l % 16).
typedef __attribute__((ext_vector_type(4))) double f64x4;
constexpr int kRfTile = 64, kRfK = 32, kRfStride = 36;

// Split over H (part non-null, gridDim.z slices of whole 32-chunks): slice z writes its
// fp64 partial sums part[z][t][e] and the sums of squares of its x and Wr values,
// part[Z T E + z T + t] and part[Z T E + Z T + z E + e] (identical in every block that stages
// the same row), and k_router_f64_sum forms the logits and bounds.
template <int XT>
__global__ __launch_bounds__(256, 2) void k_router_f64(const void *__restrict__ x, const float *__restrict__ wr,
                                                       const float *__restrict__ bias, int T, int H, int E,
                                                       float *__restrict__ logits, float *__restrict__ beta,
                                                       double *__restrict__ part)
{
    __shared__ __attribute__((aligned(16))) float xs[2][kRfTile * kRfStride];
    __shared__ __attribute__((aligned(16))) float ws[2][kRfTile * kRfStride];
    __shared__ double nx[kRfTile], nw[kRfTile];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int t0 = blockIdx.y * kRfTile, e0 = blockIdx.x * kRfTile;
    // staging: thread tid moves 8 consecutive k of row tid / 4 of both tiles
    const int sr = tid >> 2, sk = 8 * (tid & 3);
    const int st_t = min(t0 + sr, T - 1), st_e = min(e0 + sr, E - 1);
    const bool tok_ok = t0 + sr < T, exp_ok = e0 + sr < E;
    double sx = 0.0, sw = 0.0;  // sums of squares of this thread's staged values
    // The next chunk's raw bits (x: bf16 in xa, or fp32 in xa and xb; Wr in wa, wb) stay in
    // registers, untouched, until the chunk is staged: converting the bf16 x at the load
    // would wait for it right there, one memory round trip per chunk.
    u32x4 xa, xb, wa, wb;
    auto load = [&](int k0) {
        if constexpr (XT == DT_BF16) {
            xa = *(const u32x4 *)((const uint16_t *)x + (size_t)st_t * H + k0 + sk);
        } else {
            xa = *(const u32x4 *)((const float *)x + (size_t)st_t * H + k0 + sk);
            xb = *(const u32x4 *)((const float *)x + (size_t)st_t * H + k0 + sk + 4);
        }
        wa = *(const u32x4 *)(wr + (size_t)st_e * H + k0 + sk);
        wb = *(const u32x4 *)(wr + (size_t)st_e * H + k0 + sk + 4);
    };
    auto store = [&](int buf) {
        float xv[8], wv8[8];
        if constexpr (XT == DT_BF16) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xv[2 * j] = __uint_as_float(xa[j] << 16);
                xv[2 * j + 1] = __uint_as_float(xa[j] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xv[j] = __uint_as_float(xa[j]);
                xv[4 + j] = __uint_as_float(xb[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            wv8[j] = __uint_as_float(wa[j]);
            wv8[4 + j] = __uint_as_float(wb[j]);
        }
        float4 *xd = (float4 *)&xs[buf][sr * kRfStride + sk], *wd = (float4 *)&ws[buf][sr * kRfStride + sk];
        const float m = tok_ok ? 1.f : 0.f, n = exp_ok ? 1.f : 0.f;  // rows past T or E are zero
        xd[0] = float4{m * xv[0], m * xv[1], m * xv[2], m * xv[3]};
        xd[1] = float4{m * xv[4], m * xv[5], m * xv[6], m * xv[7]};
        wd[0] = float4{n * wv8[0], n * wv8[1], n * wv8[2], n * wv8[3]};
        wd[1] = float4{n * wv8[4], n * wv8[5], n * wv8[6], n * wv8[7]};
#pragma unroll
        for (int j = 0; j < 8; j++) {
            sx = fma((double)xv[j], (double)xv[j], sx);
            sw = fma((double)wv8[j], (double)wv8[j], sw);
        }
    };
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    const int mr = 32 * (wv & 1), mc = 32 * (wv >> 1);  // this wave's tokens / experts in the tile
    const int fr = lane & 15, fk = lane >> 4;           // fragment row (or column) and k
    const int Z = gridDim.z, z = blockIdx.z;
    const int nall = H / kRfK, per = nall / Z, cbeg = z * per, nchunks = per;
    load(cbeg * kRfK);
    store(0);
    __syncthreads();
    for (int c = 0; c < nchunks; c++) {
        const int buf = c & 1;
        if (c + 1 < nchunks) load((cbeg + c + 1) * kRfK);
#pragma unroll
        for (int ks = 0; ks < kRfK / 4; ks++) {
            double A[2], B[2];
#pragma unroll
            for (int u = 0; u < 2; u++) {
                A[u] = (double)xs[buf][(mr + 16 * u + fr) * kRfStride + 4 * ks + fk];
                B[u] = (double)ws[buf][(mc + 16 * u + fr) * kRfStride + 4 * ks + fk];
            }
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int b = 0; b < 2; b++) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(A[a], B[b], acc[a][b], 0, 0, 0);
        }
        if (c + 1 < nchunks) store(buf ^ 1);
        __syncthreads();
    }
    // norms: the four threads of a staged row are adjacent lanes
    sx += __shfl_xor(sx, 1, 64);
    sx += __shfl_xor(sx, 2, 64);
    sw += __shfl_xor(sw, 1, 64);
    sw += __shfl_xor(sw, 2, 64);
    if (part) {
        const size_t TE = (size_t)T * E;
        if ((tid & 3) == 0) {
            if (tok_ok) part[(size_t)Z * TE + (size_t)z * T + t0 + sr] = sx;
            if (exp_ok) part[(size_t)Z * TE + (size_t)Z * T + (size_t)z * E + e0 + sr] = sw;
        }
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int b = 0; b < 2; b++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int t = t0 + mr + 16 * a + 4 * i + fk, e = e0 + mc + 16 * b + fr;
                    if (t < T && e < E) part[(size_t)z * TE + (size_t)t * E + e] = acc[a][b][i];
                }
        return;
    }
    if ((tid & 3) == 0) {
        nx[sr] = sqrt(sx);
        nw[sr] = sqrt(sw);
    }
    __syncthreads();
    const double g2 = 2.0 * (double)(H + 1) * 0x1p-53 * (1.0 + 0x1p-20);  // 2 gamma_{H+1}, rounded up
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int tr = mr + 16 * a + 4 * i + fk, ec = mc + 16 * b + fr;
                const int t = t0 + tr, e = e0 + ec;
                if (t >= T || e >= E) continue;
                const double l64 = acc[a][b][i] + (bias ? (double)bias[e] : 0.0);
                const float l32 = (float)l64;
                const double bd = g2 * nx[tr] * nw[ec] + fabs(l64 - (double)l32) + 0x1p-52 * fabs(l64);
                logits[(size_t)t * E + e] = l32;
                beta[(size_t)t * E + e] = (float)(bd * (1.0 + 0x1p-20)) + 1e-30f;
            }
}

// Logits and bounds of the split fp64 router: l64 = the Z slice sums added in slice order
// (+ bias), the norms from the slices' sums of squares, the bound as in k_router_f64 (any
// order of fp64 additions of the H exact products is covered).  One thread per (t, e).
__global__ __launch_bounds__(256) void k_router_f64_sum(const double *__restrict__ part, int Z, const float *__restrict__ bias,
                                                        int T, int H, int E, float *__restrict__ logits,
                                                        float *__restrict__ beta)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x, TE = (size_t)T * E;
    if (i >= TE) return;
    const int t = (int)(i / E), e = (int)(i - (size_t)t * E);
    double pl[16], px[16], pw[16];  // Z <= 16: every load issued before the sums
#pragma unroll
    for (int z = 0; z < 16; z++) {
        const int zz = min(z, Z - 1);
        pl[z] = part[(size_t)zz * TE + i];
        px[z] = part[(size_t)Z * TE + (size_t)zz * T + t];
        pw[z] = part[(size_t)Z * TE + (size_t)Z * T + (size_t)zz * E + e];
    }
    double l64 = 0.0, sx = 0.0, sw = 0.0;
#pragma unroll
    for (int z = 0; z < 16; z++) {
        if (z >= Z) break;
        l64 += pl[z];
        sx += px[z];
        sw += pw[z];
    }
    if (bias) l64 += (double)bias[e];
    const double g2 = 2.0 * (double)(H + 1) * 0x1p-53 * (1.0 + 0x1p-20);  // 2 gamma_{H+1}, rounded up
    const float l32 = (float)l64;
    const double bd = g2 * sqrt(sx) * sqrt(sw) + fabs(l64 - (double)l32) + 0x1p-52 * fabs(l64);
    logits[i] = l32;
    beta[i] = (float)(bd * (1.0 + 0x1p-20)) + 1e-30f;
}

// fp64 logit of expert c for token t: lane l sums its inputs 4l + 256 m in order
// (the fp32 x fp32 or bf16 x fp32 products are exact in fp64), then the fixed wave
// reduction.  The same code path for every expert makes identical router rows give
// identical values.  Called by a whole wave; every lane receives the result.
__device__ double logit_f64(const void *x, int xt, const float *wr, const float *bias, int t, int c, int H, int lane)
{
    double acc = 0.0;
    const float *wrow = wr + (size_t)c * H;
    for (int i0 = lane * 4; i0 < H; i0 += 256 * 8) {
        float4 w4[8];
        float xv[8][4];
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const int i = i0 + 256 * m;
            if (i < H) {
                w4[m] = *(const float4 *)(wrow + i);
                load_x4(x, xt, (size_t)t * H + i, xv[m][0], xv[m][1], xv[m][2], xv[m][3]);
            } else {
                w4[m] = float4{0.f, 0.f, 0.f, 0.f};
                xv[m][0] = xv[m][1] = xv[m][2] = xv[m][3] = 0.f;
            }
        }
#pragma unroll
        for (int m = 0; m < 8; m++) {
            acc = fma((double)xv[m][0], (double)w4[m].x, acc);
            acc = fma((double)xv[m][1], (double)w4[m].y, acc);
            acc = fma((double)xv[m][2], (double)w4[m].z, acc);
            acc = fma((double)xv[m][3], (double)w4[m].w, acc);
        }
    }
    acc = wave_sum_f64(acc);
    if (bias) acc += (double)bias[c];
    return acc;
}

// (value desc, id asc) total order: does (va, ia) rank ahead of (vb, ib)?
template <typename V>
__device__ __forceinline__ bool ahead(V va, int ia, V vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

template <int C>
__device__ __forceinline__ void argbest_step(float &v, int &id)
{
    const float pv = dpp_f32<C>(v);
    const int pi = (int)dpp_u32<C>((uint32_t)id);
    if (ahead(pv, pi, v, id)) { v = pv; id = pi; }
}

template <int C>
__device__ __forceinline__ void argbest_step(double &v, int &id)
{
    const double pv = dpp_f64<C>(v);
    const int pi = (int)dpp_u32<C>((uint32_t)id);
    if (ahead(pv, pi, v, id)) { v = pv; id = pi; }
}

__device__ __forceinline__ float rl(float v, int l) { return readlane_f32(v, l); }
__device__ __forceinline__ double rl(double v, int l) { return readlane_f64(v, l); }

// Wave-wide best (value, id) under the (value desc, id asc) order; every lane gets it.
template <typename V>
__device__ __forceinline__ void wave_argbest(V &v, int &id)
{
    argbest_step<kDppXor1>(v, id);
    argbest_step<kDppXor2>(v, id);
    argbest_step<kDppHalfMirror>(v, id);
    argbest_step<kDppMirror>(v, id);
    V bv = rl(v, 0);
    int bi = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const V ov = rl(v, r);
        const int oi = __builtin_amdgcn_readlane(id, r);
        if (ahead(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    v = bv;
    id = bi;
}

// Sortable key of (logit, expert): under unsigned comparison a larger key ranks
// first in the (value desc, id asc) order.  High word: the float's bits mapped
// monotonically (-0 taken as +0, so equal values compare equal); low word: ~expert.
// Key 0 lies below every real key and marks "no element".
__device__ __forceinline__ uint64_t make_key(float v, int e)
{
    uint32_t u = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
    u ^= (uint32_t)((int32_t)u >> 31) | 0x80000000u;
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ float key_logit(uint64_t k)
{
    const uint32_t u = (uint32_t)(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

__device__ __forceinline__ int key_expert(uint64_t k) { return (int)~(uint32_t)k; }

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l)
{
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return lo | (hi << 32);
}

// Wave-wide maximum of a 64-bit key; every lane gets it.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v)
{
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const uint64_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, s, 64);
        const uint64_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), s, 64);
        const uint64_t p = lo | (hi << 32);
        v = p > v ? p : v;
    }
    return v;
}

// Number of the 64 keys s[0, 64) larger than `mine`.  The LDS reads are wave-uniform
// (broadcasts) and all issued before the first comparison.
__device__ __forceinline__ int count_above64(const uint64_t *s, uint64_t mine)
{
    u32x4 v[32];
#pragma unroll
    for (int i = 0; i < 32; i++) v[i] = ((const u32x4 *)s)[i];
#pragma unroll
    for (int i = 0; i < 32; i++) asm volatile("" : "+v"(v[i]));
    int r = 0;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const uint64_t a = v[i][0] | ((uint64_t)v[i][1] << 32), b = v[i][2] | ((uint64_t)v[i][3] << 32);
        r += (int)(a > mine) + (int)(b > mine);
    }
    return r;
}

template <int N>
__device__ __forceinline__ uint64_t tree_max(const uint64_t *k)
{
    if constexpr (N == 1) {
        return k[0];
    } else {
        const uint64_t a = tree_max<N / 2>(k), b = tree_max<N - N / 2>(k + N / 2);
        return a > b ? a : b;
    }
}

// Per-wave LDS scratch of the top-k.  Entries 64.. of ckey/cb/rkey/rb take the
// writes of lanes that have nothing to store, so that no store needs a branch.
struct TopkScratch {
    uint64_t mkey[64];   // lane maxima
    uint64_t ckey[128];  // candidates
    uint64_t rkey[128];  // candidates in rank order
    float cb[128];       // error bounds of the candidates
    float rb[128];       // ... in rank order
};

// fp64 re-ranking of the candidate set `cand` (bit q: expert lane + 64 q) of token t;
// returns, on lane j < k, the expert ranked j-th (other lanes: rank_id unchanged).
// Called by a whole wave.
template <int PL>
__device__ __noinline__ int rerank_f64(int t, const void *__restrict__ x, int xt, const float *__restrict__ wr,
                                       const float *__restrict__ bias, int H, int k, uint32_t cand, int rank_id)
{
    const int lane = threadIdx.x & 63;
    double dkey[PL];
#pragma unroll
    for (int q = 0; q < PL; q++) {
        dkey[q] = -__builtin_huge_val();
        unsigned long long m = __ballot((cand >> q) & 1u);
        while (m) {
            const int owner = __ffsll((long long)m) - 1;
            m &= m - 1;
            const double v = logit_f64(x, xt, wr, bias, t, owner + 64 * q, H, lane);
            if (lane == owner) dkey[q] = v != v ? -__builtin_huge_val() : v;
        }
    }
    uint32_t taken = 0;
    for (int j = 0; j < k; j++) {
        double bv = -__builtin_huge_val();
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < PL; q++) {
            const int e = lane + 64 * q;
            if (((cand >> q) & 1u) && !((taken >> q) & 1u) && ahead(dkey[q], e, bv, bi)) { bv = dkey[q]; bi = e; }
        }
        wave_argbest(bv, bi);
#pragma unroll
        for (int q = 0; q < PL; q++)
            if (lane + 64 * q == bi) taken |= 1u << q;
        if (lane == j) rank_id = bi;
    }
    return rank_id;
}

// fp64 re-ranking when the candidate set (bit q of cand: expert lane + 64 q) has at most 64
// members.  Candidate i goes to entry i of a compacted list (expert, fp32 logit, bound); only
// the candidates whose interval [l - b, l + b] meets another candidate's get their logit
// recomputed in fp64 (exact products, as in rerank_f64): every other candidate's exact logit
// lies in an interval disjoint from all the others', so its fp32 logit orders it correctly
// against any candidate's exact (or fp64) value.  Ranks are then counted under (value desc,
// id asc).  Returns, on lane j < k, the expert ranked j-th.  Called by a whole wave; uses
// sc's candidate and rank arrays.
template <int PL>
__device__ __noinline__ int rerank_overlap(int t, const void *__restrict__ x, int xt, const float *__restrict__ wr,
                                           const float *__restrict__ bias, const float *__restrict__ logits,
                                           const float *__restrict__ beta, int H, int E, int k, uint32_t cand,
                                           int rank_id, TopkScratch &sc)
{
    const int lane = threadIdx.x & 63;
    float *cl = (float *)sc.ckey, *cb = cl + 64;
    int *cid = (int *)(cl + 128);
    int n = 0;
#pragma unroll
    for (int q = 0; q < PL; q++) {
        const bool c = (cand >> q) & 1u;
        const unsigned long long m = __ballot(c);
        const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (c) {
            const int e = lane + 64 * q;
            const float lv = logits[(size_t)t * E + e];
            cl[pos] = lv != lv ? -__builtin_huge_valf() : lv;
            cb[pos] = beta[(size_t)t * E + e];
            cid[pos] = e;
        }
        n += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const bool mine = lane < n;
    const double li = mine ? (double)cl[lane] : 0.0, bi = mine ? (double)cb[lane] : 0.0;
    bool unc = false;  // differences and sums of two floats are exact in fp64
    for (int j = 0; j < n; j++) unc |= j != lane && fabs(li - (double)cl[j]) <= bi + (double)cb[j];
    unc = unc && mine && li > -__builtin_huge_val();
    double v = mine ? li : -__builtin_huge_val();
    unsigned long long mu = __ballot(unc);
    while (mu) {
        const int owner = __ffsll((long long)mu) - 1;
        mu &= mu - 1;
        const double d = logit_f64(x, xt, wr, bias, t, cid[owner], H, lane);
        if (lane == owner) v = d != d ? -__builtin_huge_val() : d;
    }
    double *cv = (double *)sc.rkey;
    int *rk = (int *)sc.rb;
    if (mine) cv[lane] = v;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const int myid = mine ? cid[lane] : 0x7FFFFFFF;
    int r = 0;
    for (int j = 0; j < n; j++) {
        const double vj = cv[j];
        r += vj > v || (vj == v && cid[j] < myid);
    }
    if (mine && r < k) rk[r] = myid;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    return lane < k ? rk[lane] : rank_id;
}

// Top-k + softmax of token t by one wave.  PL = logits held per lane (E <= 64 PL).
// No block-level barrier inside, so waves of one block may run it for different
// numbers of tokens.
// Selection: every member of the top-k ranks at or above the k-th largest of the 64
// per-lane maxima (those k maxima are k distinct elements), so only elements at or
// above that threshold are candidates.  Ranks are counted, not sorted: each lane
// holds one key and counts the keys above it, reading them from LDS as broadcasts,
// first among the 64 lane maxima (the threshold is the one with k-1 above it), then
// among the candidates when there are at most 64 of them (always, short of massive
// ties); a candidate with r keys above it takes rank r.  Otherwise k rounds of a
// wave-wide maximum decide.
template <int PL>
__device__ __forceinline__ void topk_one(int t, const float *__restrict__ logits, const float *__restrict__ beta,
                                         const void *__restrict__ x, int xt, const float *__restrict__ wr,
                                         const float *__restrict__ bias, int H, int E, int k,
                                         int32_t *__restrict__ ids, float *__restrict__ wts,
                                         int32_t *__restrict__ refined, TopkScratch &sc, int *lds_ids = nullptr,
                                         const float *__restrict__ wbias = nullptr)
{
    const int lane = threadIdx.x & 63;
    const float NEG = -__builtin_huge_valf();
    uint64_t key[PL];
    float l[PL], b[PL];
#pragma unroll
    for (int q = 0; q < PL; q++) {
        const int ec = min(lane + 64 * q, E - 1);  // clamped, so that every load is issued up front
        l[q] = logits[(size_t)t * E + ec];
        b[q] = beta[(size_t)t * E + ec];
    }
#pragma unroll
    for (int q = 0; q < PL; q++) asm volatile("" : "+v"(l[q]), "+v"(b[q]));
#pragma unroll
    for (int q = 0; q < PL; q++) {
        const int e = lane + 64 * q;
        // a NaN logit (non-finite input) ranks last, so every rank still names a valid expert
        key[q] = e < E ? make_key(l[q] != l[q] ? NEG : l[q], e) : 0;
        b[q] = e < E ? b[q] : 0.f;
    }
    // 1. threshold: the k-th largest lane maximum (lanes with an element outnumber k)
    const uint64_t mk = tree_max<PL>(key);
    sc.mkey[lane] = mk;
    // LDS accesses of one wave complete in order; the fence keeps the compiler from
    // moving the reads above the writes
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const int mr = count_above64(sc.mkey, mk);
    const int tl = __ffsll((long long)__ballot(mr == k - 1)) - 1;
    const uint64_t thr = readlane_u64(mk, tl);
    // 2. candidates (key >= thr), compacted into LDS
    int ncand = 0;
#pragma unroll
    for (int q = 0; q < PL; q++) {
        const bool c = key[q] >= thr;
        const unsigned long long m = __ballot(c);
        const int pos = ncand + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        ncand += __popcll(m);
        const int slot = c && pos < 64 ? pos : 64 + lane;
        sc.ckey[slot] = key[q];
        sc.cb[slot] = b[q];
    }
    // lane j < k: key and error bound of the expert ranked j-th
    uint64_t rank_key = 0;
    float rank_b = 0.f;
    if (ncand <= 64) {
        sc.ckey[lane >= ncand ? lane : 64 + lane] = 0;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const uint64_t ck = sc.ckey[lane];
        const float cbl = sc.cb[lane];
        const int cr = count_above64(sc.ckey, ck);
        const int rs = lane < ncand && cr < k ? cr : 64 + lane;
        sc.rkey[rs] = ck;
        sc.rb[rs] = cbl;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        rank_key = lane < k ? sc.rkey[lane] : 0;
        rank_b = lane < k ? sc.rb[lane] : 0.f;
    } else {
        uint32_t taken = 0;  // bit q: key q already ranked
        for (int j = 0; j < k; j++) {
            uint64_t bv = 0;
#pragma unroll
            for (int q = 0; q < PL; q++)
                if (!((taken >> q) & 1u) && key[q] > bv) bv = key[q];
            bv = wave_max_key(bv);
#pragma unroll
            for (int q = 0; q < PL; q++)
                if (key[q] == bv) taken |= 1u << q;
            if (lane == j) rank_key = bv;
        }
        if (lane < k) rank_b = beta[(size_t)t * E + key_expert(rank_key)];
        sc.rkey[lane] = rank_key;
        sc.rb[lane] = rank_b;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    const uint64_t kth = readlane_u64(rank_key, k - 1);
    const float rank_l = key_logit(rank_key);
    // 3. is the ranking certain under the fp32 error intervals?  Every selected logit's
    // interval must lie above every other logit's, and consecutive ranks must not overlap.
    const float lo = wave_min_f32(lane < k ? rank_l - rank_b : __builtin_huge_valf());
    uint32_t cand = 0;  // bit q: selected, or not separable from the selection
    int ncand2 = 0;
#pragma unroll
    for (int q = 0; q < PL; q++) {
        const bool c = key[q] != 0 && (key[q] >= kth || key_logit(key[q]) + b[q] >= lo);
        if (c) cand |= 1u << q;
        ncand2 += __popcll(__ballot(c));
    }
    bool overlap = false;
    if (lane < k - 1) overlap = rank_l - rank_b <= key_logit(sc.rkey[lane + 1]) + sc.rb[lane + 1];
    overlap = __ballot(overlap) != 0;
    int rank_id = key_expert(rank_key);
    bool reranked = false;
    if (ncand2 > k || overlap) {
        // 4. re-rank on fp64 logits (rare: kept out of line): those of the candidates whose
        // intervals overlap (at most 64 candidates), else of every candidate
        rank_id = ncand2 <= 64 ? rerank_overlap<PL>(t, x, xt, wr, bias, logits, beta, H, E, k, cand, rank_id, sc)
                               : rerank_f64<PL>(t, x, xt, wr, bias, H, k, cand, rank_id);
        if (lane == 0 && refined) atomicAdd(refined, 1);
        reranked = true;
    }
    // 5. softmax over the selected fp32 logits, in rank order (rank 0 holds the
    // largest unless the fp64 ranking reordered them)
    const int my_id = lane < k ? rank_id : 0;
    float lj = lane >= k ? NEG : !reranked ? rank_l : logits[(size_t)t * E + my_id];
    // a selection-only bias (wbias) is taken back out of the selected keys: the weights
    // are the softmax of the unbiased logits, whose largest need not rank first
    if (wbias && lane < k) lj -= wbias[my_id];
    const float mx = reranked || wbias ? wave_max_f32(lj) : readlane_f32(lj, 0);
    const float ex = lane < k ? __expf(lj - mx) : 0.f;
    const float den = wave_sum_f32(ex);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        wts[(size_t)t * k + lane] = ex / den;
        if (lds_ids) lds_ids[t * k + lane] = my_id;
    }
}


template <int PL>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, const float *__restrict__ beta,
                                              const void *__restrict__ x, int xt, const float *__restrict__ wr,
                                              const float *__restrict__ bias, int T, int H, int E, int k,
                                              int32_t *__restrict__ ids, float *__restrict__ wts,
                                              int32_t *__restrict__ refined, const float *__restrict__ wbias)
{
    __shared__ TopkScratch scs[4];
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    topk_one<PL>(t, logits, beta, x, xt, wr, bias, H, E, k, ids, wts, refined, scs[wv], nullptr, wbias);
}

// Small batches (T <= 4, T k <= 256): top-k of every token and the grouping of the
// T k slots in one single-block launch (the logits come from k_router_gemv, whose
// kernel boundary makes them visible).  Wave w ranks token w; then the block groups
// the slots, ordered by (expert, slot).
constexpr int kSmallT = 4;  // one wave per token; more tokens run k_topk over several blocks
constexpr int kSmallS = 256;
constexpr int kSmallE = 2048;

template <int PL>
__global__ __launch_bounds__(256) void k_topk_group(const RouteArgs a, const GroupArgs gq)
{
    __shared__ TopkScratch scs[4];
    __shared__ __attribute__((aligned(16))) int cnt[kSmallE];
    __shared__ __attribute__((aligned(16))) int sids[kSmallS];
    __shared__ int scr[256];
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    // slot-list entries past the T k slots read as INT_MAX by the 16-entry counting below
    if (tid < 16 && a.T * a.k + tid < kSmallS) sids[a.T * a.k + tid] = 0x7FFFFFFF;
    if (wv < a.T)  // T <= 4
        topk_one<PL>(wv, a.logits, a.beta, a.x, a.xt, a.wr, a.bias, a.H, a.E, a.k, a.ids, a.w, a.refined, scs[wv],
                     sids, a.wbias);
    __syncthreads();

    const int S = a.T * a.k, E = a.E;
    if (S <= 64) {
        // Up to 64 slots: slot s's grouped row is the number of slots ordered before it
        // (counted by wave 0 against the broadcast slot list); meanwhile every thread counts
        // the offsets and counts of its experts against the same list.
        int *se = cnt;  // sorted experts
        if (wv == 0) {
            const int e = lane < S ? sids[lane] : 0x7FFFFFFF;
            const uint32_t mine = ((uint32_t)e << 10) | (uint32_t)lane;
            int p = 0;
            for (int i = 0; i < S; i++) p += (((uint32_t)sids[i] << 10) | (uint32_t)i) < mine;
            if (lane < S) {
                gq.perm[p] = lane;
                gq.inv[lane] = p;
            }
            se[lane < S ? p : lane] = e;  // slots past S: INT_MAX
            se[64 + lane] = 0x7FFFFFFF;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const bool real = lane < S;
            const int ep = real ? se[lane] : 0;
            const bool first = real && (lane == 0 || se[max(lane - 1, 0)] != ep);
            const unsigned long long m = __ballot(first);
            const int apos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (first) gq.active[apos] = ep;
            if (lane == 0) {
                *gq.n_active = (int)__popcll(m);
                gq.offsets[E] = S;
            }
        }
        // offsets[q] = the slots of experts below q, counts[q] = those of q: counted against
        // the slot list (a count needs no order) read in 16-entry pieces (independent LDS
        // reads; entries past S hold INT_MAX and count for no expert)
        for (int q0 = 0; q0 < E; q0 += 1024) {
            int lo[4] = {0, 0, 0, 0}, hi[4] = {0, 0, 0, 0};
            for (int c0 = 0; c0 < S; c0 += 16) {
                int v[16];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int4 w = *(const int4 *)(sids + c0 + 4 * i);
                    v[4 * i] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
                }
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int q = q0 + tid + 256 * r;
#pragma unroll
                    for (int i = 0; i < 16; i++) {
                        lo[r] += v[i] < q;
                        hi[r] += v[i] <= q;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int q = q0 + tid + 256 * r;
                if (q < E) {
                    gq.offsets[q] = lo[r];
                    gq.counts[q] = hi[r] - lo[r];
                }
            }
        }
        return;
    }

    for (int i = tid; i < E; i += 256) cnt[i] = 0;
    __syncthreads();
    if (tid < S) atomicAdd(&cnt[sids[tid]], 1);
    __syncthreads();
    const int per = (E + 255) / 256;
    const int ea = min(E, tid * per), eb = min(E, ea + per);
    int my = 0, myact = 0;
    for (int q = ea; q < eb; q++) {
        my += cnt[q];
        myact += cnt[q] > 0;
    }
    int total, atot;
    const int base = block_exclusive_scan(my, scr, &total);
    const int abase = block_exclusive_scan(myact, scr, &atot);
    int run = base, arun = abase;
    for (int q = ea; q < eb; q++) {
        const int c = cnt[q];
        gq.counts[q] = c;
        gq.offsets[q] = run;
        if (c > 0) gq.active[arun++] = q;
        cnt[q] = run;  // from here on: first grouped row of expert q
        run += c;
    }
    if (tid == 0) {
        gq.offsets[E] = total;
        *gq.n_active = atot;
    }
    __syncthreads();
    if (tid < S) {
        const int q = sids[tid];
        int rank = 0;
        for (int s2 = 0; s2 < tid; s2++) rank += sids[s2] == q;
        const int pos = cnt[q] + rank;
        gq.perm[pos] = tid;
        gq.inv[tid] = pos;
    }
}

bool route_small_ok(const RouteArgs &a)
{
    return a.T <= kSmallT && a.T * a.k <= kSmallS && a.E <= kSmallE && a.H <= kGemvMaxH;
}

template <int PL>
static hipError_t launch_small_pl(const RouteArgs &a, const GroupArgs &g, hipStream_t s)
{
    {
        ProfScope ps(a.prof, PK_ROUTER_LOGITS, s);
        ps.launch(a.xt == DT_BF16 ? k_router_gemv<DT_BF16> : k_router_gemv<DT_F32>,
                  dim3((a.E + kGemvE - 1) / kGemvE, (a.T + 7) / 8), dim3(256), 0, a.x, a.wr,
                           a.bias, a.T, a.H, a.E, a.logits, a.beta);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ProfScope ps(a.prof, PK_ROUTER_TOPK, s);
    ps.launch(k_topk_group<PL>, dim3(1), dim3(256), 0, a, g);
    return hipGetLastError();
}

hipError_t launch_route_small(const RouteArgs &a, const GroupArgs &g, hipStream_t s)
{
    const int pl = (a.E + 63) / 64;
    if (pl <= 1) return launch_small_pl<1>(a, g, s);
    if (pl <= 2) return launch_small_pl<2>(a, g, s);
    if (pl <= 4) return launch_small_pl<4>(a, g, s);
    if (pl <= 8) return launch_small_pl<8>(a, g, s);
    if (pl <= 14) return launch_small_pl<14>(a, g, s);
    if (pl <= 16) return launch_small_pl<16>(a, g, s);
    return launch_small_pl<32>(a, g, s);
}

template <int PL>
static hipError_t launch_topk_pl(const RouteArgs &a, hipStream_t s)
{
    const dim3 grid((a.T + 3) / 4);
    ProfScope ps(a.prof, PK_ROUTER_TOPK, s);
    ps.launch(k_topk<PL>, grid, dim3(256), 0, a.logits, a.beta, a.x, a.xt, a.wr, a.bias, a.T, a.H, a.E,
                       a.k, a.ids, a.w, a.refined, a.wbias);
    return hipGetLastError();
}

// Slices of H for the fp64 router: up to 16, so that tiles x slices reaches ~256 blocks, each
// slice a whole number of 32-chunks, the partials within the workspace given.
constexpr int kGemvSplitT = 8;  // more tokens than this take the fp64 router (split when its tiles are few)
static int rf64_slices(const RouteArgs &a, int tiles)
{
    if (!a.rpart || a.H % kRfK || tiles >= 256) return 1;
    const int nch = a.H / kRfK;
    int Z = 1;
    for (int c = 2; c <= 16; c++) {
        const size_t need = ((size_t)c * a.T * a.E + (size_t)c * (a.T + a.E)) * 8;
        if (nch % c || need > a.rpart_bytes) continue;
        Z = c;
        if (tiles * c >= 256) break;
    }
    return Z;
}

hipError_t launch_router(const RouteArgs &a, hipStream_t s)
{
    {
    ProfScope ps(a.prof, PK_ROUTER_LOGITS, s);
    const int tiles = ((a.E + kRfTile - 1) / kRfTile) * ((a.T + kRfTile - 1) / kRfTile);
    const int Z = rf64_slices(a, tiles);
    if (a.T <= kGemvMaxT && a.H <= kGemvMaxH && (a.T <= kGemvSplitT || Z == 1)) {
        ps.launch(a.xt == DT_BF16 ? k_router_gemv<DT_BF16> : k_router_gemv<DT_F32>,
                  dim3((a.E + kGemvE - 1) / kGemvE, (a.T + 7) / 8), dim3(256), 0, a.x, a.wr, a.bias,
                           a.T, a.H, a.E, a.logits, a.beta);
    } else if (Z > 1) {
        // few tiles: H split into Z slices so the grid fills the chip, then the slice sums
        const dim3 grid((a.E + kRfTile - 1) / kRfTile, (a.T + kRfTile - 1) / kRfTile, Z);
        if (a.xt == DT_BF16)
            ps.launch(k_router_f64<DT_BF16>, grid, dim3(256), 0, a.x, a.wr, a.bias, a.T, a.H, a.E, a.logits, a.beta, a.rpart);
        else
            ps.launch(k_router_f64<DT_F32>, grid, dim3(256), 0, a.x, a.wr, a.bias, a.T, a.H, a.E, a.logits, a.beta, a.rpart);
        const hipError_t e1 = hipGetLastError();
        if (e1 != hipSuccess) return e1;
        const size_t TE = (size_t)a.T * a.E;
        hipLaunchKernelGGL(k_router_f64_sum, dim3((unsigned)((TE + 255) / 256)), dim3(256), 0, s, (const double *)a.rpart, Z,
                           a.bias, a.T, a.H, a.E, a.logits, a.beta);
    } else {
        const dim3 grid((a.E + kRfTile - 1) / kRfTile, (a.T + kRfTile - 1) / kRfTile);
        if (a.xt == DT_BF16)
            ps.launch(k_router_f64<DT_BF16>, grid, dim3(256), 0, a.x, a.wr, a.bias, a.T, a.H, a.E, a.logits, a.beta,
                      (double *)nullptr);
        else
            ps.launch(k_router_f64<DT_F32>, grid, dim3(256), 0, a.x, a.wr, a.bias, a.T, a.H, a.E, a.logits, a.beta,
                      (double *)nullptr);
    }
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int pl = (a.E + 63) / 64;
    if (pl <= 1) return launch_topk_pl<1>(a, s);
    if (pl <= 2) return launch_topk_pl<2>(a, s);
    if (pl <= 4) return launch_topk_pl<4>(a, s);
    if (pl <= 8) return launch_topk_pl<8>(a, s);
    if (pl <= 14) return launch_topk_pl<14>(a, s);
    if (pl <= 16) return launch_topk_pl<16>(a, s);
    return launch_topk_pl<32>(a, s);
}

}  // namespace moe
