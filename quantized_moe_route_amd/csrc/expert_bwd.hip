// expert_bwd.hip -- input gradient through the frozen routed experts and the router.
//
// The routed experts are one differentiable unit whose backward returns the
// gradient with respect to the latent input (LazyLoRA README, "Routed
// experts": the experts are streamed a second time in the backward and
// dL/dh_latent is computed explicitly; "File map": the native kernel provides
// the transposed product needed for it).  Per slot (t, j, e) with weight p:
//   a  = Wd^T dy_t                  (reduction over the down matrix's rows)
//   dp = <a, h>                     (gradient of the combine w.r.t. p)
//   dh = p a,  dg = dh dact/dg,  du = dh dact/du   (act_grad: SwiGLU or SiTU)
//   dx_tj = Wg^T dg + Wu^T du       (reduction over the gate/up rows)
//   dX_t = sum_j dx_tj + sum_j p_tj (dp_tj - sum_j' p_tj' dp_tj') Wr[e_j]
// The block scales of the stored matrices run along the forward reduction
// dimension, which is not the reduction dimension of these transposed
// products, so each block dequantizes a 64x64 weight tile exactly into LDS in
// transposed order and feeds bf16 MFMA from there.
#include "expert_frag.h"

namespace moe {


constexpr int kTS = 72;  // LDS row stride (bf16) of a transposed 64x64 tile, padded

// Dequantize rows q0..q0+63, columns c0..c0+63 of matrix W (rows x cols) of
// expert e into wt_hi (and wt_lo for RVQ3) as [c][q] bf16.  Rows/columns past
// the matrix are zero.  256 threads: thread -> row q0 + tid/4, 16 columns.
template <int WFMT>
__device__ __forceinline__ void stage_tile_t(const MatW &W, int e, int rows, int cols, int q0, int c0,
                                             uint16_t *wt_hi, uint16_t *wt_lo, const uint16_t *cb)
{
    const int tid = threadIdx.x, ql = tid >> 2, cl = (tid & 3) * 16;
    const int q = q0 + ql, c = c0 + cl;
    float v[16];
    const bool ok = q < rows && c < cols;
    if constexpr (WFMT == FMT_MXFP4) {
        u32x2 raw = {0u, 0u};
        float sc = 0.f;
        if (ok) {
            const size_t r = (size_t)e * rows + q;
            raw = *(const u32x2 *)(W.codes + r * (size_t)(cols / 2) + c / 2);
            sc = e8m0_to_f32(W.scales[r * (size_t)(cols / 32) + c / 32]);
        }
        uint32_t d[16];
        const u32x4 c4 = {raw[0], raw[1], 0u, 0u};
        decode_fp4x32(c4, sc, d);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            wt_hi[(cl + 2 * i) * kTS + ql] = (uint16_t)(d[i] & 0xFFFFu);
            wt_hi[(cl + 2 * i + 1) * kTS + ql] = (uint16_t)(d[i] >> 16);
        }
        (void)v;
        (void)wt_lo;
        (void)cb;
    } else {
#pragma unroll
        for (int d = 0; d < 16; d++) v[d] = 0.f;
        if (ok) {
#pragma unroll
            for (int st = 0; st < 3; st++) {
                const uint8_t *ip = W.idx + (((size_t)e * 3 + st) * rows + q) * (size_t)(cols / 8) + c / 8;
                const uint32_t i2 = ip[0] | ((uint32_t)ip[1] << 8);
#pragma unroll
                for (int vv = 0; vv < 2; vv++) {
                    const uint32_t id = (i2 >> (8 * vv)) & 0xFFu;
                    const u32x4 cw = *(const u32x4 *)(cb + ((size_t)st * 256 + id) * 8);
#pragma unroll
                    for (int d = 0; d < 4; d++) {
                        v[8 * vv + 2 * d] += (float)__builtin_bit_cast(_Float16, (uint16_t)(cw[d] & 0xFFFFu));
                        v[8 * vv + 2 * d + 1] += (float)__builtin_bit_cast(_Float16, (uint16_t)(cw[d] >> 16));
                    }
                }
            }
        }
#pragma unroll
        for (int d = 0; d < 16; d++) {
            uint32_t h, l;
            split_bf16(v[d], h, l);
            wt_hi[(cl + d) * kTS + ql] = (uint16_t)h;
            wt_lo[(cl + d) * kTS + ql] = (uint16_t)l;
        }
    }
}

// A fragment (16 columns x 32 reduction) from a staged transposed tile.
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t *wt, int c, int q)
{
    return as_bf16x8(*(const u32x4 *)(wt + c * kTS + q));
}

// out[c][token] += sum_q W[q][c] * B[token][q] for one staged 64-row chunk.
template <int WFMT, int BT, int NTT>
__device__ __forceinline__ void tile_mma(f32x4 (&acc)[NTT], const uint16_t *wt_hi, const uint16_t *wt_lo, int cw,
                                         const void *bsrc, const size_t (&boff)[NTT], const bool (&tv)[NTT], int q0,
                                         int Q, int g, int li)
{
#pragma unroll
    for (int sub = 0; sub < 2; sub++) {
        const int ql = 32 * sub + 8 * g;
        const bf16x8 ahi = lds_frag(wt_hi, cw + li, ql);
        bf16x8 alo = ahi;
        if constexpr (WFMT == FMT_RVQ3) alo = lds_frag(wt_lo, cw + li, ql);
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            const int q = q0 + ql;
            const bool ok = tv[tt] && q < Q;
            if constexpr (BT == DT_BF16) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (ok) v = *(const u32x4 *)((const uint16_t *)bsrc + boff[tt] + q);
                const bf16x8 b = as_bf16x8(v);
                acc[tt] = mfma16(ahi, b, acc[tt]);
                if constexpr (WFMT == FMT_RVQ3) acc[tt] = mfma16(alo, b, acc[tt]);
            } else {
                float4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
                if (ok) {
                    x0 = *(const float4 *)((const float *)bsrc + boff[tt] + q);
                    x1 = *(const float4 *)((const float *)bsrc + boff[tt] + q + 4);
                }
                const float f[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                uint32_t h[8], l[8];
#pragma unroll
                for (int d = 0; d < 8; d++) split_bf16(f[d], h[d], l[d]);
                const bf16x8 bh = as_bf16x8(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
                const bf16x8 bl = as_bf16x8(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
                acc[tt] = mfma16(ahi, bh, acc[tt]);
                acc[tt] = mfma16(ahi, bl, acc[tt]);
                if constexpr (WFMT == FMT_RVQ3) acc[tt] = mfma16(alo, bh, acc[tt]);
            }
        }
    }
}

// a = Wd^T dy for the block's 64 columns of I, then the activation backward.
template <int WFMT, int DYT, int NTT>
__global__ __launch_bounds__(256) void k_bwd_down(const ExpertBwdArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t wt_hi[64 * kTS];
    __shared__ __attribute__((aligned(16))) uint16_t wt_lo[WFMT == FMT_RVQ3 ? 64 * kTS : 8];
    __shared__ __attribute__((aligned(16))) uint16_t cbs[WFMT == FMT_RVQ3 ? 3 * 256 * 8 : 8];
    __shared__ float red[4][16 * NTT];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int ai = blockIdx.y;
    if (ai >= *a.n_active) return;
    const int e = a.active[ai];
    if constexpr (WFMT == FMT_RVQ3) load_codebooks(a.down, e, cbs);
    const int H = a.H, I = a.I;
    const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;
    const int c0 = blockIdx.x * 64, cw = 16 * wv;
    const int ntiles = dp_tiles(I);
    for (int tt0 = 0; tt0 < ntok; tt0 += 16 * NTT) {
        f32x4 acc[NTT];
        size_t boff[NTT];
        bool tv[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int j = tt0 + 16 * tt + li;
            tv[tt] = j < ntok;
            boff[tt] = tv[tt] ? (size_t)(a.perm[r0 + j] / a.k) * H : 0;
        }
        for (int q0 = 0; q0 < H; q0 += 64) {
            __syncthreads();
            stage_tile_t<WFMT>(a.down, e, H, I, q0, c0, wt_hi, wt_lo, cbs);
            __syncthreads();
            tile_mma<WFMT, DYT, NTT>(acc, wt_hi, wt_lo, cw, a.dy, boff, tv, q0, H, g, li);
        }
        // epilogue
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            const int j = tt0 + 16 * tt + li;
            float dpp = 0.f;
            if (j < ntok) {
                const size_t rr = (size_t)(r0 + j);
                const float p = a.w[a.perm[rr]];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int c = c0 + cw + 4 * g + r;
                    if (c < I) {
                        const float gv = a.gu[(rr * 2) * I + c], uv = a.gu[(rr * 2 + 1) * I + c];
                        float hv, dhdg, dhdu;
                        act_grad(a.act, gv, uv, hv, dhdg, dhdu);
                        // the shared adapter's per-token term of Wd^T dy
                        const float av = acc[tt][r] + (a.lora_c ? a.lora_c[(size_t)(a.perm[rr] / a.k) * I + c] : 0.f);
                        dpp += av * hv;
                        const float dh = p * av;
                        a.dgdu[(rr * 2) * I + c] = dh * dhdg;
                        a.dgdu[(rr * 2 + 1) * I + c] = dh * dhdu;
                    }
                }
            }
            dpp += __shfl_xor(dpp, 16, 64);
            dpp += __shfl_xor(dpp, 32, 64);
            if (g == 0) red[wv][16 * tt + li] = dpp;
        }
        __syncthreads();
        if (threadIdx.x < 16 * NTT) {
            const int j = tt0 + threadIdx.x;
            if (j < ntok) {
                const float s = ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x];
                a.dp_part[(size_t)(r0 + j) * ntiles + blockIdx.x] = s;
            }
        }
    }
}

// dxs[slot] = Wg^T dg + Wu^T du for the block's 64 columns of H.
template <int WFMT, int NTT>
__global__ __launch_bounds__(256) void k_bwd_gateup(const ExpertBwdArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t wt_hi[64 * kTS];
    __shared__ __attribute__((aligned(16))) uint16_t wt_lo[WFMT == FMT_RVQ3 ? 64 * kTS : 8];
    __shared__ __attribute__((aligned(16))) uint16_t cbs[WFMT == FMT_RVQ3 ? 2 * 3 * 256 * 8 : 8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int ai = blockIdx.y;
    if (ai >= *a.n_active) return;
    const int e = a.active[ai];
    if constexpr (WFMT == FMT_RVQ3) {
        load_codebooks(a.gate, e, cbs);
        load_codebooks(a.up, e, cbs + 3 * 256 * 8);
    }
    const int H = a.H, I = a.I;
    const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;
    const int c0 = blockIdx.x * 64, cw = 16 * wv;
    for (int tt0 = 0; tt0 < ntok; tt0 += 16 * NTT) {
        f32x4 acc[NTT];
        bool tv[NTT];
        size_t boff[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mat = 0; mat < 2; mat++) {
            const MatW &W = mat == 0 ? a.gate : a.up;
#pragma unroll
            for (int tt = 0; tt < NTT; tt++) {
                const int j = tt0 + 16 * tt + li;
                tv[tt] = j < ntok;
                boff[tt] = tv[tt] ? ((size_t)(r0 + j) * 2 + mat) * I : 0;
            }
            for (int q0 = 0; q0 < I; q0 += 64) {
                __syncthreads();
                stage_tile_t<WFMT>(W, e, I, H, q0, c0, wt_hi, wt_lo, cbs + mat * 3 * 256 * 8);
                __syncthreads();
                tile_mma<WFMT, DT_F32, NTT>(acc, wt_hi, wt_lo, cw, a.dgdu, boff, tv, q0, I, g, li);
            }
        }
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            const int j = tt0 + 16 * tt + li;
            if (j >= ntok) continue;
            const int slot = a.perm[r0 + j];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int c = c0 + cw + 4 * g + r;
                if (c < H) a.dxs[(size_t)slot * H + c] = acc[tt][r];
            }
        }
    }
}

// dX[t] = sum_j dxs[t*k+j] + sum_j dl_j Wr[e_j] with dl_j = p_j (dp_j - sum_j' p_j' dp_j').
__global__ __launch_bounds__(256) void k_bwd_final(const ExpertBwdArgs a)
{
    __shared__ float dl[64];
    __shared__ int eid[64];
    const int t = blockIdx.x, k = a.k, H = a.H;
    const int ntiles = dp_tiles(a.I);
    if (threadIdx.x < 64) {
        const int j = threadIdx.x;
        float dp = 0.f, p = 0.f;
        int e = 0;
        if (j < k) {
            const size_t slot = (size_t)t * k + j;
            const int rr = a.inv[slot];
            for (int c = 0; c < ntiles; c++) dp += a.dp_part[(size_t)rr * ntiles + c];
            p = a.w[slot];
            e = a.ids[slot];
        }
        float pdp = p * dp;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) pdp += __shfl_xor(pdp, o, 64);
        pdp = __shfl(pdp, 0, 64);
        dl[j] = p * (dp - pdp);
        eid[j] = e;
    }
    __syncthreads();
    for (int i = threadIdx.x * 4; i < H; i += 1024) {
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; j++) {
            const float4 v = *(const float4 *)(a.dxs + ((size_t)t * k + j) * H + i);
            const float4 r = *(const float4 *)(a.wr + (size_t)eid[j] * H + i);
            const float d = dl[j];
            acc.x += v.x + d * r.x;
            acc.y += v.y + d * r.y;
            acc.z += v.z + d * r.z;
            acc.w += v.w + d * r.w;
        }
        for (int j = 0; j < a.k2; j++) {  // the shared experts' rows (no router term)
            const float4 v = *(const float4 *)(a.dxs2 + ((size_t)t * a.k2 + j) * H + i);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *(float4 *)(a.dx + (size_t)t * H + i) = acc;
    }
}

template <int WFMT, int DYT, int NTT>
static hipError_t bwd_launch(const ExpertBwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    {
        ProfScope ps(a.prof, PK_BWD_DOWN, s);
        ps.launch((k_bwd_down<WFMT, DYT, NTT>), dim3((a.I + 63) / 64, maxU), dim3(256), 0, a);
    }
    {
        ProfScope ps(a.prof, PK_BWD_GATEUP, s);
        ps.launch((k_bwd_gateup<WFMT, NTT>), dim3((a.H + 63) / 64, maxU), dim3(256), 0, a);
    }
    if (!a.skip_final) {
        ProfScope ps(a.prof, PK_BWD_FINAL, s);
        ps.launch(k_bwd_final, dim3(a.T), dim3(256), 0, a);
    }
    return hipGetLastError();
}

template <int WFMT, int DYT>
static hipError_t bwd_ntt(const ExpertBwdArgs &a, hipStream_t s)
{
    return a.T <= 64 ? bwd_launch<WFMT, DYT, 1>(a, s) : bwd_launch<WFMT, DYT, 4>(a, s);
}

hipError_t launch_expert_backward(const ExpertBwdArgs &a0, hipStream_t s)
{
    ExpertBwdArgs a = a0;
    if (!a.gu) {
        ExpertFwdArgs f{};
        f.wfmt = a.wfmt;
        f.gate = a.gate;
        f.up = a.up;
        f.down = a.down;
        f.x = a.x;
        f.xt = a.xt;
        f.T = a.T;
        f.H = a.H;
        f.I = a.I;
        f.E = a.E;
        f.k = a.k;
        f.offsets = a.offsets;
        f.perm = a.perm;
        f.active = a.active;
        f.n_active = a.n_active;
        f.w = a.w;
        f.h_hi = a.h_hi;
        f.h_lo = a.h_lo;
        f.gu = a.gu_scratch;
        f.act = a.act;
        f.lora_gu = a.lora_gu;
        f.tok_chunks = a.tok_chunks;
        f.prof = a.prof;
        set_lds_staging(f);
        hipError_t err = launch_gateup_only(f, s);
        if (err != hipSuccess) return err;
        a.gu = a.gu_scratch;
    }
    if (bwd_uses_mm(a)) {
        hipError_t err = launch_bwd_down_mm(a, s);
        if (err == hipSuccess) err = launch_bwd_gateup_mm(a, s);
        if (err != hipSuccess || a.skip_final) return err;
        ProfScope ps(a.prof, PK_BWD_FINAL, s);
        ps.launch(k_bwd_final, dim3(a.T), dim3(256), 0, a);
        return hipGetLastError();
    }
    if (a.wfmt == FMT_MXFP4)
        return a.dyt == DT_BF16 ? bwd_ntt<FMT_MXFP4, DT_BF16>(a, s) : bwd_ntt<FMT_MXFP4, DT_F32>(a, s);
    return a.dyt == DT_BF16 ? bwd_ntt<FMT_RVQ3, DT_BF16>(a, s) : bwd_ntt<FMT_RVQ3, DT_F32>(a, s);
}

}  // namespace moe
