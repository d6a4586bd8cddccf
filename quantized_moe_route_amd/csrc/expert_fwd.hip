// expert_fwd.hip -- routed-expert forward: fused dequant + gate/up + gated activation,
// down projection with the routing weight, and a fixed-order combine.
//
// Per routed slot (t, j) with expert e and weight p (LazyLoRA README, "The
// engine" / "Arithmetic": MXFP4 experts consumed packed, fused decode-and-dot,
// fp32 accumulation; "File map": the combine uses the routing weights):
//   g = Wg x_t,  u = Wu x_t,  h = act(g, u),  o = Wd h,  y_t = sum_j p_tj o_tj,
//   act = SwiGLU silu(g) u, or SiTU (act_h).
// The quantized weights are dequantized in registers straight from HBM (each
// active expert's bytes are read once per token tile) and fed to bf16 MFMA
// with fp32 accumulation.  MXFP4 dequantizes exactly to bf16; bf16 tokens are
// exact; fp32 tokens enter as three bf16 terms (hi + mid + lo, all 24 significand bits),
// h as two (hi + lo).
//
// Block = 4 waves x 16 rows = 64 rows of one active expert (blockIdx.y indexes
// the device-side active list; blocks past *n_active exit), all of that
// expert's tokens in tiles of 16*NTT.
#include "expert_frag.h"

namespace moe {

// Prefetch depth in K-steps of the streaming loops.
constexpr int kPD = 3;
// Largest per-row scale run (bytes) staged in LDS by the full-step MXFP4 kernels (K <= 4096).
constexpr int kMaxScaleRow = 128;

template <int WFMT, int XT, int NTT, bool FULL>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(WFMT == FMT_MXFP4 && XT == DT_BF16 && NTT == 1 && FULL ? 3 : 1)))
void k_gateup(const ExpertFwdArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t cbs[WFMT == FMT_RVQ3 ? 2 * 3 * 256 * 8 : 8];
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_lds[];
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
    const int row = n0 + li;
    // Few-token experts (decode): the block stages its tokens' x rows in LDS once, so the
    // per-step token fragment is an LDS read instead of an L2 round trip.
    const bool staged = XT == DT_BF16 && NTT == 1 && ntok <= a.nl_x;
    if (staged) {
        size_t off[16];
#pragma unroll
        for (int j = 0; j < 16; j++) off[j] = j < ntok ? (size_t)(a.perm[r0 + j] / a.k) * H : 0;
        stage_rows_bf16(xs_lds, (const uint16_t *)a.x, off, ntok, H);
        __syncthreads();
    }
    // MXFP4 full-step path: the block's 64 gate rows and 64 up rows of scale bytes go to
    // LDS once (two contiguous runs), so the K-loop reads scales from LDS.
    constexpr bool kScl = WFMT == FMT_MXFP4 && FULL;
    __shared__ __attribute__((aligned(16))) uint8_t scl[kScl ? 2 * 64 * kMaxScaleRow : 8];
    const int spr = H / 32;  // scale bytes per row
    const int nb0 = blockIdx.x * 64, nbn = min(64, I - nb0);
    if constexpr (kScl) {
        stage_scales(scl, a.gate, e, I, H, nb0, nbn);
        stage_scales(scl + 64 * spr, a.up, e, I, H, nb0, nbn);
        __syncthreads();
    }
    if (n0 >= I) return;
    using AF = AFrag<WFMT>;
    using F = Fetcher<WFMT, FULL>;
    using Raw = typename F::Raw;
    F fg, fu;
    fg.init(a.gate, e, I, H, row, g, scl + (row - nb0) * spr);
    fu.init(a.up, e, I, H, row, g, scl + 64 * spr + (row - nb0) * spr);
    const int nsteps = (H + 255) / 256;
    const uint16_t *xl = xs_lds + (size_t)min(li, ntok - 1) * (H + 8);
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
        // Weights are fetched kPD K-steps ahead of their decode.  Within a step the
        // token fragment is loaded before the next prefetch: loads retire in order,
        // so waiting for the token fragment never waits for the prefetch.
        Raw g0, u0, g1, u1, g2, u2;
        fg.fetch(g0, 0);
        fu.fetch(u0, 0);
        fg.fetch(g1, min(1, nsteps - 1));
        fu.fetch(u1, min(1, nsteps - 1));
        fg.fetch(g2, min(2, nsteps - 1));
        fu.fetch(u2, min(2, nsteps - 1));
        for (int st = 0; st < nsteps; st++) {
            const int kk = 256 * st + 64 * g;
            BFrag<XT> b;
            if constexpr (FULL && XT == DT_BF16) {
                if (staged)
                    load_row_bf16(b.hi, xl + kk);
                else
                    load_row_bf16(b.hi, (const uint16_t *)a.x + xoff[0] + kk);
            } else if constexpr (XT == DT_BF16) {
                if (staged)
                    load_bf16x8_lds(b.hi, xl, kk, H, tv[0]);
                else
                    b.load(a.x, xoff[0], kk, H, tv[0]);
            } else {
                b.load(a.x, xoff[0], kk, H, tv[0]);
            }
            Raw g3, u3;
            fg.fetch(g3, min(st + kPD, nsteps - 1));
            fu.fetch(u3, min(st + kPD, nsteps - 1));
            AF ag, au;
            F::decode(ag, g0, cbs);
            F::decode(au, u0, cbs + 3 * 256 * 8);
#pragma unroll
            for (int tt = 0; tt < NTT; tt++) {
                if (tt > 0) {
                    if constexpr (FULL && XT == DT_BF16)
                        load_row_bf16(b.hi, (const uint16_t *)a.x + xoff[tt] + kk);
                    else
                        b.load(a.x, xoff[tt], kk, H, tv[tt]);
                }
                mma_step(accg[tt], ag, b);
                mma_step(accu[tt], au, b);
            }
            g0 = g1;
            u0 = u1;
            g1 = g2;
            u1 = u2;
            g2 = g3;
            u2 = u3;
        }
        // epilogue: lane holds rows n0 + 4g + r for token tt0 + 16tt + li;
        // h is stored as bf16 hi + lo planes, the operand form of the down product
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            const int j = tt0 + 16 * tt + li;
            if (j >= ntok) continue;
            const size_t rr = (size_t)(r0 + j);
            add_lora_gu(a.lora_gu, a.perm, a.k, rr, I, n0 + 4 * g, accg[tt], accu[tt]);
            uint32_t hh[4], hl[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float gv = accg[tt][r], uv = accu[tt][r];
                split_bf16(act_h(a.act, gv, uv), hh[r], hl[r]);
            }
            const size_t o = rr * I + n0 + 4 * g;
            *(u32x2 *)(a.h_hi + o) = u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
            *(u32x2 *)(a.h_lo + o) = u32x2{pack2(hl[0], hl[1]), pack2(hl[2], hl[3])};
            if (a.gu) {
                *(float4 *)(a.gu + (rr * 2 + 0) * I + n0 + 4 * g) = float4{accg[tt][0], accg[tt][1], accg[tt][2], accg[tt][3]};
                *(float4 *)(a.gu + (rr * 2 + 1) * I + n0 + 4 * g) = float4{accu[tt][0], accu[tt][1], accu[tt][2], accu[tt][3]};
            }
        }
    }
}

// Down projection: each wave owns RT tiles of 16 rows of Wd (rows of H) and shares
// one token fragment across them.
template <int WFMT, int NTT, int RT, bool FULL>
__global__ __launch_bounds__(256) void k_down(const ExpertFwdArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t cbs[WFMT == FMT_RVQ3 ? 3 * 256 * 8 : 8];
    extern __shared__ __attribute__((aligned(16))) uint16_t hs_lds[];
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
    const int m0 = blockIdx.x * (64 * RT) + wv * (16 * RT);
    // Few-token experts stage their h rows (hi and lo planes) in LDS once.
    const bool staged = NTT == 1 && ntok <= a.nl_h;
    const size_t lds_lo = (size_t)a.nl_h * (I + 8);
    if (staged) {
        size_t off[16];
#pragma unroll
        for (int j = 0; j < 16; j++) off[j] = j < ntok ? (size_t)(r0 + j) * I : 0;
        stage_rows_bf16(hs_lds, a.h_hi, off, ntok, I);
        stage_rows_bf16(hs_lds + lds_lo, a.h_lo, off, ntok, I);
        __syncthreads();
    }
    constexpr bool kScl = WFMT == FMT_MXFP4 && FULL;
    __shared__ __attribute__((aligned(16))) uint8_t scl[kScl ? 64 * RT * kMaxScaleRow : 8];
    const int spr = I / 32;
    const int mb0 = blockIdx.x * (64 * RT), mbn = min(64 * RT, H - mb0);
    if constexpr (kScl) {
        stage_scales(scl, a.down, e, H, I, mb0, mbn);
        __syncthreads();
    }
    if (m0 >= H) return;
    bool rv[RT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++) rv[rt] = m0 + 16 * rt < H;
    using AF = AFrag<WFMT>;
    using F = Fetcher<WFMT, FULL>;
    using Raw = typename F::Raw;
    F fd[RT];
#pragma unroll
    for (int rt = 0; rt < RT; rt++) {
        const int r = rv[rt] ? m0 + 16 * rt + li : li;
        fd[rt].init(a.down, e, H, I, r, g, scl + (rv[rt] ? r - mb0 : 0) * spr);
    }
    const int nsteps = (I + 255) / 256;
    const uint16_t *hl = hs_lds + (size_t)min(li, ntok - 1) * (I + 8);
    for (int tt0 = 0; tt0 < ntok; tt0 += 16 * NTT) {
        f32x4 acc[RT][NTT];
        size_t hoff[NTT];
        bool tv[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
#pragma unroll
            for (int rt = 0; rt < RT; rt++) acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int j = tt0 + 16 * tt + li;
            tv[tt] = j < ntok;
            hoff[tt] = tv[tt] ? (size_t)(r0 + j) * I : 0;
        }
        Raw d0[RT], d1[RT], d2[RT];
#pragma unroll
        for (int rt = 0; rt < RT; rt++) {
            fd[rt].fetch(d0[rt], 0);
            fd[rt].fetch(d1[rt], min(1, nsteps - 1));
            fd[rt].fetch(d2[rt], min(2, nsteps - 1));
        }
        for (int st = 0; st < nsteps; st++) {
            const int kk = 256 * st + 64 * g;
            BFragPair b;
            if constexpr (FULL) {
                if (NTT == 1 && staged) {
                    load_row_bf16(b.hi, hl + kk);
                    load_row_bf16(b.lo, hl + lds_lo + kk);
                } else {
                    load_row_bf16(b.hi, a.h_hi + hoff[0] + kk);
                    load_row_bf16(b.lo, a.h_lo + hoff[0] + kk);
                }
            } else {
                if (NTT == 1 && staged) {
                    load_bf16x8_lds(b.hi, hl, kk, I, tv[0]);
                    load_bf16x8_lds(b.lo, hl + lds_lo, kk, I, tv[0]);
                } else {
                    b.load(a.h_hi, a.h_lo, hoff[0], kk, I, tv[0]);
                }
            }
            Raw d3[RT];
#pragma unroll
            for (int rt = 0; rt < RT; rt++) fd[rt].fetch(d3[rt], min(st + kPD, nsteps - 1));
#pragma unroll
            for (int rt = 0; rt < RT; rt++) {
                AF ad;
                F::decode(ad, d0[rt], cbs);
#pragma unroll
                for (int tt = 0; tt < NTT; tt++) {
                    if (tt > 0) {
                        if constexpr (FULL) {
                            load_row_bf16(b.hi, a.h_hi + hoff[tt] + kk);
                            load_row_bf16(b.lo, a.h_lo + hoff[tt] + kk);
                        } else {
                            b.load(a.h_hi, a.h_lo, hoff[tt], kk, I, tv[tt]);
                        }
                    }
                    mma_step(acc[rt][tt], ad, b);
                }
                if (NTT > 1 && rt + 1 < RT) {
                    if constexpr (FULL) {
                        load_row_bf16(b.hi, a.h_hi + hoff[0] + kk);
                        load_row_bf16(b.lo, a.h_lo + hoff[0] + kk);
                    } else {
                        b.load(a.h_hi, a.h_lo, hoff[0], kk, I, tv[0]);
                    }
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; rt++) {
                d0[rt] = d1[rt];
                d1[rt] = d2[rt];
                d2[rt] = d3[rt];
            }
        }
#pragma unroll
        for (int tt = 0; tt < NTT; tt++) {
            const int j = tt0 + 16 * tt + li;
            if (j >= ntok) continue;
            const int slot = a.perm[r0 + j];
            const float p = a.w[slot];
#pragma unroll
            for (int rt = 0; rt < RT; rt++) {
                if (!rv[rt]) continue;
                const f32x4 v = acc[rt][tt];
                *(float4 *)(a.ybuf + (size_t)slot * H + m0 + 16 * rt + 4 * g) = float4{p * v[0], p * v[1], p * v[2], p * v[3]};
            }
        }
    }
}

// y[t] = sum over j in rank order of the weighted slot rows (deterministic).
// The k2 rows of ybuf2 (the shared experts' outputs, null: none) follow the routed slots.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ ybuf, int T, int H, int k,
                                                 const float *__restrict__ ybuf2, int k2, float *__restrict__ y)
{
    const size_t n4 = (size_t)T * H / 4;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        const size_t t = i / (H / 4), m4 = i % (H / 4);
        float4 acc = {0.f, 0.f, 0.f, 0.f};
        // loads of 8 slots are issued together; the sum still runs in rank order
        for (int j0 = 0; j0 < k; j0 += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; u++)
                v[u] = j0 + u < k ? *(const float4 *)(ybuf + ((size_t)t * k + j0 + u) * H + 4 * m4)
                                  : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 8; u++) {
                if (j0 + u >= k) break;
                acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
            }
        }
        for (int j = 0; j < k2; j++) {
            const float4 v = *(const float4 *)(ybuf2 + ((size_t)t * k2 + j) * H + 4 * m4);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *(float4 *)(y + (size_t)t * H + 4 * m4) = acc;
    }
}

static hipError_t launch_combine(const ExpertFwdArgs &a, hipStream_t s)
{
    if (a.skip_combine) return hipSuccess;
    const size_t n4 = (size_t)a.T * a.H / 4;
    const size_t nb = (n4 + 255) / 256;
    const int blocks = (int)(nb < 4096 ? nb : 4096);
    ProfScope ps(a.prof, PK_COMBINE, s);
    ps.launch(k_combine, dim3(blocks), dim3(256), 0, a.ybuf, a.T, a.H, a.k, a.ybuf2, a.ybuf2 ? a.k2 : 0, a.y);
    return hipGetLastError();
}

// Token rows the gate/up kernel stages in LDS (experts with more tokens read theirs from
// the L2 each step): no more than keep three blocks per CU, the kernel's register bound, in
// the CU's 160 KB beside its static LDS (the staged scale bytes or the RVQ3 codebooks).
// With the six rows of 48 KB at the K3 shape only two blocks fit: the 64-token gate/up
// took 1,180 µs with six rows staged, 1,000-1,003 µs with four or five.
template <int WFMT, bool FULL>
static ExpertFwdArgs gateup_staging(const ExpertFwdArgs &a)
{
    ExpertFwdArgs b = a;
    const size_t stat = WFMT == FMT_RVQ3 ? (size_t)2 * 3 * 256 * 8 * 2 : FULL ? (size_t)2 * 64 * kMaxScaleRow : 0;
    const size_t per_block = (size_t)160 * 1024 / 3;
    const int cap = per_block > stat ? (int)((per_block - stat) / ((size_t)(a.H + 8) * 2)) : 0;
    b.nl_x = min(a.nl_x, cap);
    return b;
}

template <int WFMT, int XT, int NTT, bool FULLG, bool FULLD>
static hipError_t fwd_launch(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    {
        ProfScope ps(a.prof, PK_GATEUP, s);
        const ExpertFwdArgs b = gateup_staging<WFMT, FULLG>(a);
        const size_t lds = NTT == 1 && XT == DT_BF16 ? (size_t)b.nl_x * (b.H + 8) * 2 : 0;
        ps.launch((k_gateup<WFMT, XT, NTT, FULLG>), dim3((a.I + 63) / 64, maxU), dim3(256), lds, b);
    }
    {
        ProfScope ps(a.prof, PK_DOWN, s);
        constexpr int RT = NTT == 1 ? 2 : 1;
        const size_t lds = NTT == 1 ? (size_t)a.nl_h * (a.I + 8) * 2 * 2 : 0;
        ps.launch((k_down<WFMT, NTT, RT, FULLD>), dim3((a.H + 64 * RT - 1) / (64 * RT), maxU), dim3(256), lds, a);
    }
    return launch_combine(a, s);
}

template <int WFMT, int XT, int NTT>
static hipError_t fwd_full(const ExpertFwdArgs &a, hipStream_t s)
{
    const bool fg = a.H % 256 == 0 && a.H <= 32 * kMaxScaleRow, fd = a.I % 256 == 0 && a.I <= 32 * kMaxScaleRow;
    if (fg && fd) return fwd_launch<WFMT, XT, NTT, true, true>(a, s);
    if (fg) return fwd_launch<WFMT, XT, NTT, true, false>(a, s);
    if (fd) return fwd_launch<WFMT, XT, NTT, false, true>(a, s);
    return fwd_launch<WFMT, XT, NTT, false, false>(a, s);
}

template <int WFMT, int XT>
static hipError_t fwd_ntt(const ExpertFwdArgs &a, hipStream_t s)
{
    return a.T <= 64 ? fwd_full<WFMT, XT, 1>(a, s) : fwd_full<WFMT, XT, 4>(a, s);
}

template <int WFMT, int XT>
static hipError_t gateup_only(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    ProfScope ps(a.prof, PK_GATEUP, s);
    const dim3 grid((a.I + 63) / 64, maxU);
    const bool f = a.H % 256 == 0 && a.H <= 32 * kMaxScaleRow;
    if (a.T <= 64) {
        const ExpertFwdArgs b = f ? gateup_staging<WFMT, true>(a) : gateup_staging<WFMT, false>(a);
        const size_t lds = XT == DT_BF16 ? (size_t)b.nl_x * (b.H + 8) * 2 : 0;
        if (f)
            ps.launch((k_gateup<WFMT, XT, 1, true>), grid, dim3(256), lds, b);
        else
            ps.launch((k_gateup<WFMT, XT, 1, false>), grid, dim3(256), lds, b);
    } else {
        if (f)
            ps.launch((k_gateup<WFMT, XT, 4, true>), grid, dim3(256), 0, a);
        else
            ps.launch((k_gateup<WFMT, XT, 4, false>), grid, dim3(256), 0, a);
    }
    return hipGetLastError();
}

// gate/up + activation only (the backward recomputes g and u when they were not saved)
hipError_t launch_gateup_only(const ExpertFwdArgs &a, hipStream_t s)
{
    if (use_mm(a)) return launch_gateup_mm(a, s);
    if (dec_supported(a)) return launch_gateup_dec(a, s);
    if (rvq_dec_supported(a)) return launch_gateup_rvq(a, s);
    if (a.wfmt == FMT_MXFP4)
        return a.xt == DT_BF16 ? gateup_only<FMT_MXFP4, DT_BF16>(a, s) : gateup_only<FMT_MXFP4, DT_F32>(a, s);
    return a.xt == DT_BF16 ? gateup_only<FMT_RVQ3, DT_BF16>(a, s) : gateup_only<FMT_RVQ3, DT_F32>(a, s);
}

hipError_t launch_expert_forward(const ExpertFwdArgs &a, hipStream_t s)
{
    if (use_mm(a)) {
        hipError_t err = launch_gateup_mm(a, s);
        if (err == hipSuccess) err = launch_down_mm(a, s);
        if (err == hipSuccess) err = launch_combine(a, s);
        return err;
    }
    if (dec_supported(a)) {
        if (dec_fused_ok(a)) return launch_dec_fused(a, s);
        hipError_t err = launch_gateup_dec(a, s);
        if (err == hipSuccess) err = launch_down_dec(a, s);
        if (err == hipSuccess) err = launch_combine(a, s);
        return err;
    }
    if (a.tok_chunks == 0 && rvq_lut_supported(a)) {
        hipError_t err = launch_rvq_lut(a, s);
        if (err == hipSuccess) err = launch_combine(a, s);
        return err;
    }
    if (rvq_dec_supported(a)) {
        hipError_t err = launch_gateup_rvq(a, s);
        if (err == hipSuccess) err = launch_down_rvq(a, s);
        if (err == hipSuccess) err = launch_combine(a, s);
        return err;
    }
    if (a.wfmt == FMT_MXFP4)
        return a.xt == DT_BF16 ? fwd_ntt<FMT_MXFP4, DT_BF16>(a, s) : fwd_ntt<FMT_MXFP4, DT_F32>(a, s);
    return a.xt == DT_BF16 ? fwd_ntt<FMT_RVQ3, DT_BF16>(a, s) : fwd_ntt<FMT_RVQ3, DT_F32>(a, s);
}

}  // namespace moe
