// router.hip -- router logits and top-k + softmax for gfx950.
//
// Router (LazyLoRA README, "File map": top-16 gating with a score-correction
// bias; "The engine": 896 routed experts, top-16): logits l[t][e] = x[t]·Wr[e]
// (+ b[e]), the k largest are selected (equal logits rank the lower expert id
// first) and the combining weights are the softmax over the k selected logits.
//
// Logits are formed in fp32.  Alongside each logit the kernel stores a bound
// beta >= |l_fp32 - l_exact|: each lane's fp32 FMA chain plus the reduction
// tree has depth m, so the error is at most gamma_m * sum|x_i w_i| (Higham,
// Accuracy and Stability of Numerical Algorithms, sec. 3.1); beta uses
// 2 (m+2) 2^-24 (sum|x_i w_i| + |b|), which also covers the rounding of the
// bias add and of the computed absolute sum.  Tokens whose selection or rank
// order is not decided by these intervals have their candidate logits
// recomputed in fp64 (the products of fp32/bf16 inputs are exact in fp64) and
// are re-ranked on those values.
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

// GEMV form for few tokens: grid (ceil(E/16), T), 4 waves per block, each wave
// one (token, expert) pair at a time; lane i-stride 256, 4 consecutive inputs.
__global__ __launch_bounds__(256) void k_router_gemv(const void *__restrict__ x, int xt, const float *__restrict__ wr,
                                                     const float *__restrict__ bias, int H, int E,
                                                     float *__restrict__ logits, float *__restrict__ beta)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.y;
    const float depth = (float)(4 * ((H + 255) / 256) + 6 + 2);
    for (int q = 0; q < 4; q++) {
        const int e = blockIdx.x * 16 + wv * 4 + q;
        if (e >= E) break;
        float acc = 0.f, sab = 0.f;
        for (int i = lane * 4; i < H; i += 256) {
            float4 w4 = *(const float4 *)(wr + (size_t)e * H + i);
            float x0, x1, x2, x3;
            load_x4(x, xt, (size_t)t * H + i, x0, x1, x2, x3);
            acc = fmaf(x0, w4.x, acc);
            acc = fmaf(x1, w4.y, acc);
            acc = fmaf(x2, w4.z, acc);
            acc = fmaf(x3, w4.w, acc);
            sab = fmaf(fabsf(x0), fabsf(w4.x), sab);
            sab = fmaf(fabsf(x1), fabsf(w4.y), sab);
            sab = fmaf(fabsf(x2), fabsf(w4.z), sab);
            sab = fmaf(fabsf(x3), fabsf(w4.w), sab);
        }
        acc = wave_sum_f32(acc);
        sab = wave_sum_f32(sab);
        if (lane == 0) {
            const float b = bias ? bias[e] : 0.f;
            logits[(size_t)t * E + e] = acc + b;
            beta[(size_t)t * E + e] = 2.f * depth * 0x1p-24f * (sab + fabsf(b));
        }
    }
}

// Tiled form for many tokens: block = 32 tokens x 64 experts, K chunks of 32
// staged in LDS; thread (ty, tx) owns tokens 2ty, 2ty+1 and experts tx+16q.
// Each chunk is summed from zero (chain 32) and added to the running total
// (chain ceil(H/32)), so the depth is 32 + ceil(H/32).
__global__ __launch_bounds__(256) void k_router_tiled(const void *__restrict__ x, int xt, const float *__restrict__ wr,
                                                      const float *__restrict__ bias, int T, int H, int E,
                                                      float *__restrict__ logits, float *__restrict__ beta)
{
    __shared__ float xs[32][33];
    __shared__ float ws[64][33];
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int t0 = blockIdx.y * 32, e0 = blockIdx.x * 64;
    float acc[2][4], sab[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int q = 0; q < 4; q++) acc[a][q] = sab[a][q] = 0.f;

    for (int k0 = 0; k0 < H; k0 += 32) {
        // x tile: 32 x 32 values, 4 per thread
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int idx = tid + 256 * r, tt = idx >> 5, kk = idx & 31;
            const int t = t0 + tt, k = k0 + kk;
            xs[tt][kk] = (t < T && k < H) ? load_x1(x, xt, (size_t)t * H + k) : 0.f;
        }
        // Wr tile: 64 x 32 values, 8 per thread
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const int idx = tid + 256 * r, ee = idx >> 5, kk = idx & 31;
            const int e = e0 + ee, k = k0 + kk;
            ws[ee][kk] = (e < E && k < H) ? wr[(size_t)e * H + k] : 0.f;
        }
        __syncthreads();
        float part[2][4], pab[2][4];
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int q = 0; q < 4; q++) part[a][q] = pab[a][q] = 0.f;
#pragma unroll 8
        for (int kk = 0; kk < 32; kk++) {
            const float xa = xs[2 * ty][kk], xb = xs[2 * ty + 1][kk];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float wv = ws[tx + 16 * q][kk];
                part[0][q] = fmaf(xa, wv, part[0][q]);
                part[1][q] = fmaf(xb, wv, part[1][q]);
                pab[0][q] = fmaf(fabsf(xa), fabsf(wv), pab[0][q]);
                pab[1][q] = fmaf(fabsf(xb), fabsf(wv), pab[1][q]);
            }
        }
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                acc[a][q] += part[a][q];
                sab[a][q] += pab[a][q];
            }
        __syncthreads();
    }
    const float depth = (float)(32 + (H + 31) / 32 + 2);
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int t = t0 + 2 * ty + a, e = e0 + tx + 16 * q;
            if (t < T && e < E) {
                const float b = bias ? bias[e] : 0.f;
                logits[(size_t)t * E + e] = acc[a][q] + b;
                beta[(size_t)t * E + e] = 2.f * depth * 0x1p-24f * (sab[a][q] + fabsf(b));
            }
        }
}

// fp64 logit of expert c for token t: each lane sums its inputs i = lane + 64 m
// sequentially (the fp32 x fp32 or bf16 x fp32 products are exact in fp64),
// then a fixed butterfly; lane 0's value is broadcast.  The same code path for
// every expert makes identical router rows give identical values.
__device__ double logit_f64(const void *x, int xt, const float *wr, const float *bias, int t, int c, int H, int lane)
{
    double acc = 0.0;
    for (int i = lane; i < H; i += 64)
        acc = fma((double)load_x1(x, xt, (size_t)t * H + i), (double)wr[(size_t)c * H + i], acc);
    acc = wave_sum_f64(acc);
    acc = __shfl(acc, 0, 64);
    if (bias) acc += (double)bias[c];
    return acc;
}

// (value desc, id asc) total order: does (va, ia) rank ahead of (vb, ib)?
template <typename V>
__device__ __forceinline__ bool ahead(V va, int ia, V vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

template <typename V>
__device__ __forceinline__ void wave_argbest(V &v, int &id)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        V ov = __shfl_xor(v, o, 64);
        int oi = __shfl_xor(id, o, 64);
        if (ahead(ov, oi, v, id)) { v = ov; id = oi; }
    }
}

// One wave per token.  PL = logits held per lane (E <= 64 PL).
template <int PL>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, const float *__restrict__ beta,
                                              const void *__restrict__ x, int xt, const float *__restrict__ wr,
                                              const float *__restrict__ bias, int T, int H, int E, int k,
                                              int32_t *__restrict__ ids, float *__restrict__ wts,
                                              int32_t *__restrict__ refined)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    const float NEG = -__builtin_huge_valf();
    float l[PL], b[PL];
    uint32_t sel = 0, cand = 0;  // bit q: logit q of this lane
    int rank_id = 0;             // lane j < k: expert ranked j-th
#pragma unroll
    for (int q = 0; q < PL; q++) {
        const int e = lane + 64 * q;
        // a NaN logit (non-finite input) ranks last, so every rank still names a valid expert
        const float lv = e < E ? logits[(size_t)t * E + e] : NEG;
        l[q] = lv != lv ? NEG : lv;
        b[q] = e < E ? beta[(size_t)t * E + e] : 0.f;
    }
    // 1. fp32 selection, k rounds of a wave-wide arg-best
    for (int j = 0; j < k; j++) {
        float bv = NEG;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < PL; q++) {
            const int e = lane + 64 * q;
            if (e < E && !((sel >> q) & 1u) && ahead(l[q], e, bv, bi)) { bv = l[q]; bi = e; }
        }
        wave_argbest(bv, bi);
#pragma unroll
        for (int q = 0; q < PL; q++)
            if (lane + 64 * q == bi) sel |= 1u << q;
        if (lane == j) rank_id = bi;
    }
    // 2. is the ranking certain under the fp32 error intervals?
    float lo = __builtin_huge_valf();
#pragma unroll
    for (int q = 0; q < PL; q++)
        if ((sel >> q) & 1u) lo = fminf(lo, l[q] - b[q]);
    lo = wave_min_f32(lo);
    int ncand = 0;
#pragma unroll
    for (int q = 0; q < PL; q++) {
        const int e = lane + 64 * q;
        const bool c = e < E && (((sel >> q) & 1u) || l[q] + b[q] >= lo);
        if (c) cand |= 1u << q;
        ncand += __popcll(__ballot(c));
    }
    bool overlap = false;
    const int next_id = __shfl(rank_id, (lane + 1) & 63, 64);
    if (lane < k - 1) {
        const int ea = rank_id, eb = next_id;
        const float la = logits[(size_t)t * E + ea], lb = logits[(size_t)t * E + eb];
        const float ba = beta[(size_t)t * E + ea], bb = beta[(size_t)t * E + eb];
        overlap = la - ba <= lb + bb;
    }
    overlap = __ballot(overlap) != 0;
    int my_id;
    if (ncand > k || overlap) {
        // 3. re-rank every candidate on fp64 logits
        double key[PL];
#pragma unroll
        for (int q = 0; q < PL; q++) {
            key[q] = -__builtin_huge_val();
            unsigned long long m = __ballot((cand >> q) & 1u);
            while (m) {
                const int owner = __ffsll((long long)m) - 1;
                m &= m - 1;
                const double v = logit_f64(x, xt, wr, bias, t, owner + 64 * q, H, lane);
                if (lane == owner) key[q] = v != v ? -__builtin_huge_val() : v;
            }
        }
        uint32_t taken = 0;
        for (int j = 0; j < k; j++) {
            double bv = -__builtin_huge_val();
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int q = 0; q < PL; q++) {
                const int e = lane + 64 * q;
                if (((cand >> q) & 1u) && !((taken >> q) & 1u) && ahead(key[q], e, bv, bi)) { bv = key[q]; bi = e; }
            }
            wave_argbest(bv, bi);
#pragma unroll
            for (int q = 0; q < PL; q++)
                if (lane + 64 * q == bi) taken |= 1u << q;
            if (lane == j) rank_id = bi;
        }
        if (lane == 0 && refined) atomicAdd(refined, 1);
    }
    // 4. softmax over the selected fp32 logits, in rank order
    my_id = lane < k ? rank_id : 0;
    const float lj = lane < k ? logits[(size_t)t * E + my_id] : NEG;
    const float mx = __shfl(wave_max_f32(lj), 0, 64);
    const float ex = lane < k ? __expf(lj - mx) : 0.f;
    const float den = __shfl(wave_sum_f32(ex), 0, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        wts[(size_t)t * k + lane] = ex / den;
    }
}

template <int PL>
static hipError_t launch_topk_pl(const RouteArgs &a, hipStream_t s)
{
    const dim3 grid((a.T + 3) / 4);
    ProfScope ps(a.prof, PK_ROUTER_TOPK, s);
    hipLaunchKernelGGL(k_topk<PL>, grid, dim3(256), 0, s, a.logits, a.beta, a.x, a.xt, a.wr, a.bias, a.T, a.H, a.E,
                       a.k, a.ids, a.w, a.refined);
    return hipGetLastError();
}

hipError_t launch_router(const RouteArgs &a, hipStream_t s)
{
    {
    ProfScope ps(a.prof, PK_ROUTER_LOGITS, s);
    if (a.T <= 8) {
        hipLaunchKernelGGL(k_router_gemv, dim3((a.E + 15) / 16, a.T), dim3(256), 0, s, a.x, a.xt, a.wr, a.bias, a.H,
                           a.E, a.logits, a.beta);
    } else {
        hipLaunchKernelGGL(k_router_tiled, dim3((a.E + 63) / 64, (a.T + 31) / 32), dim3(256), 0, s, a.x, a.xt, a.wr,
                           a.bias, a.T, a.H, a.E, a.logits, a.beta);
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
