// expert_dec.hip -- few-token (decode) expert forward for MXFP4 weights and bf16 tokens.
//
// Same arithmetic as the generic kernels of expert_fwd.hip (LazyLoRA README, "The
// engine": MXFP4 experts consumed packed with a fused decode-and-dot and fp32
// accumulation; "Measurement findings": decode is bound by the bytes of the routed
// experts), shaped for the case where every routed expert holds only a few tokens and
// the kernel is a pure stream over the routed experts' bytes:
//  - a wave owns 16 rows of the gate and of the up matrix (or two 16-row tiles of down)
//    and walks K in steps of 256: per step and tile each lane loads 32 contiguous code
//    bytes and the two scale bytes of its 64 reduction indices;
//  - code bytes go through kGuStages / kDnStages register stages (one fewer steps of
//    prefetch); the K loop is unrolled by the stage count so that no stage is ever
//    copied, and the prefetch loads are issued ahead of the step's math;
//  - each wave copies the scale bytes of its 16-row tiles (contiguous) into its own LDS
//    region with two 16-byte loads per lane, issued behind the first code prefetches;
//  - the expert's token rows (x, or the bf16 hi/lo planes of h) are staged in LDS once
//    per block after the first prefetches are in flight; the MFMA B operand is read
//    from there;
//  - buffer loads take a per-lane 32-bit offset and a wave-uniform step offset.
#include <type_traits>

#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

template <int P>
using Stage = std::integral_constant<int, P>;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

template <int I, int N>
struct Unroll {
    template <typename F>
    __device__ __forceinline__ static void run(int s0, F &step)
    {
        step(Stage<I>(), s0 + I);
        Unroll<I + 1, N>::run(s0, step);
    }
    template <typename F>
    __device__ __forceinline__ static void tail(int s0, int n, F &step)
    {
        if (s0 + I < n) step(Stage<I>(), s0 + I);
        Unroll<I + 1, N>::tail(s0, n, step);
    }
};
template <int N>
struct Unroll<N, N> {
    template <typename F>
    __device__ __forceinline__ static void run(int, F &) {}
    template <typename F>
    __device__ __forceinline__ static void tail(int, int, F &) {}
};

// Runs step(Stage<st % NS>, st) for st = 0 .. n-1: the loop body is NS whole steps (so a
// register stage is never copied) with the remainder peeled after it, a single back edge.
template <int NS, typename F>
__device__ __forceinline__ void k_loop(int n, F &&step)
{
    int s0 = 0;
    for (; s0 + NS <= n; s0 += NS) Unroll<0, NS>::run(s0, step);
    Unroll<0, NS - 1>::tail(s0, n, step);
}

constexpr int kGuStages = 4;  // register stages of the weight stream (prefetch distance + 1)
constexpr int kDnStages = 4;

// One tile's raw code bytes for one K-step (32 per lane).
struct Raw {
    u32x4 c0, c1;
};

__device__ __forceinline__ void fetch(Raw &r, __amdgpu_buffer_rsrc_t code, uint32_t coff, int st)
{
    r.c0 = ld16(code, coff, 128 * st);
    r.c1 = ld16(code, coff, 128 * st + 16);
}

// 8 MFMA sub-steps of one K-step for one tile: A from raw bytes and the two scale bytes
// of the lane's blocks, B from LDS.
__device__ __forceinline__ void mma_raw(f32x4 &acc, const Raw &r, uint32_t sc, const bf16x8 (&B)[8])
{
    uint32_t d[32];
    decode_fp4x32(r.c0, e8m0_to_f32(sc & 0xFFu), d);
    decode_fp4x32(r.c1, e8m0_to_f32(sc >> 8), d + 16);
#pragma unroll
    for (int s = 0; s < 8; s++) acc = mfma16(as_bf16x8(d[4 * s], d[4 * s + 1], d[4 * s + 2], d[4 * s + 3]), B[s], acc);
}

// Scale bytes of a wave's 16-row tile (16 * K/32 contiguous bytes, K <= 4096) go to a
// 2 KB LDS region of the wave: two 16-byte loads per lane, issued here, stored by
// put_scales once they have arrived.
struct TileScales {
    u32x4 v0, v1;
};

__device__ __forceinline__ void get_scales(TileScales &t, __amdgpu_buffer_rsrc_t scale, uint32_t tile_off, int lane)
{
    t.v0 = ld16(scale, tile_off + 16 * lane, 0);
    t.v1 = ld16(scale, tile_off + 16 * lane, 1024);
}

__device__ __forceinline__ void put_scales(uint8_t *region, const TileScales &t, int lane)
{
    *(u32x4 *)(region + 16 * lane) = t.v0;
    *(u32x4 *)(region + 1024 + 16 * lane) = t.v1;
}

__device__ __forceinline__ void lds_row8(bf16x8 (&B)[8], const uint16_t *p)
{
#pragma unroll
    for (int s = 0; s < 8; s++) B[s] = as_bf16x8(*(const u32x4 *)(p + 8 * s));
}

// Stage n gathered bf16 rows of K elements (row r at src + off(r)) into LDS rows of
// stride K + 8.  Loads go out four per thread before their stores (indices past the end
// are clamped to the last chunk, whose copy is simply written twice).
template <typename Off>
__device__ __forceinline__ void stage_rows(uint16_t *dst, const uint16_t *src, Off off, int n, int K)
{
    const int per = K / 8, total = n * per;
    for (int c0 = threadIdx.x; c0 < total; c0 += 4 * blockDim.x) {
        u32x4 v[4];
        int r[4], q[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = min(c0 + i * (int)blockDim.x, total - 1);
            r[i] = c / per;
            q[i] = c - r[i] * per;
            v[i] = *(const u32x4 *)(src + off(r[i]) + 8 * q[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) *(u32x4 *)(dst + (size_t)r[i] * (K + 8) + 8 * q[i]) = v[i];
    }
}

}  // namespace

// gate/up + activation.  Block = 4 waves x 16 rows = 64 I-columns of one active expert
// (blockIdx.y indexes the active list); all of the expert's tokens (<= nl_x) in one
// 16-column MFMA tile.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gateup_dec(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    // The weight prefetch needs only e: the active-list entry is read together with the
    // list length (entries past it are stale but name a valid expert) and the first code
    // loads go out before the block learns whether it has work.
    const int ai = blockIdx.y;
    const int nact = *a.n_active;
    const int sh = ai - min(a.E, a.T * a.k);  // >= 0: shared expert sh (every token, weight 1)
    const int e = sh >= 0 ? sh : min(max(a.active[ai], 0), a.E - 1);
    const MatW &Wg = sh >= 0 ? a.sh_gate : a.gate, &Wu = sh >= 0 ? a.sh_up : a.up;
    const int H = a.H, I = a.I;
    const int row0 = blockIdx.x * 64 + wv * 16;
    const int nsteps = H / 256, spr = H / 32;
    const size_t eoc = (size_t)e * I * (H / 2), eos = (size_t)e * I * spr;
    const __amdgpu_buffer_rsrc_t cg = buf_rsrc(Wg.codes + eoc, I * (H / 2));
    const __amdgpu_buffer_rsrc_t cu = buf_rsrc(Wu.codes + eoc, I * (H / 2));
    const uint32_t coff = (uint32_t)(row0 + li) * (H / 2) + 32 * g;

    Raw rg[kGuStages], ru[kGuStages];
#pragma unroll
    for (int s = 0; s < kGuStages - 1; s++) {
        fetch(rg[s], cg, coff, min(s, nsteps - 1));
        fetch(ru[s], cu, coff, min(s, nsteps - 1));
    }
    TileScales tg, tu;
    get_scales(tg, buf_rsrc(Wg.scales + eos, I * spr), (uint32_t)row0 * spr, lane);
    get_scales(tu, buf_rsrc(Wu.scales + eos, I * spr), (uint32_t)row0 * spr, lane);
    if (sh < 0 && ai >= nact) return;
    const int r0 = sh >= 0 ? sh * a.T : a.offsets[e], ntok = sh >= 0 ? a.T : a.offsets[e + 1] - r0;
    // token rows to LDS while the first weight bytes are in flight
    __shared__ uint32_t xrow[16];
    if (threadIdx.x < ntok) xrow[threadIdx.x] = sh >= 0 ? threadIdx.x : (uint32_t)(a.perm[r0 + threadIdx.x] / a.k);
    __syncthreads();
    stage_rows(xs, (const uint16_t *)a.x, [&](int r) { return (size_t)xrow[r] * H; }, ntok, H);
    uint8_t *sreg = (uint8_t *)(xs + (size_t)a.nl_x * (H + 8)) + 4096 * wv;
    put_scales(sreg, tg, lane);
    put_scales(sreg + 2048, tu, lane);
    __syncthreads();

    const uint16_t *xl = xs + (size_t)min(li, ntok - 1) * (H + 8) + 64 * g;
    const uint16_t *slg = (const uint16_t *)(sreg + li * spr + 2 * g);
    const uint16_t *slu = (const uint16_t *)(sreg + 2048 + li * spr + 2 * g);
    f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    k_loop<kGuStages>(nsteps, [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
        const int sn = min(st + kGuStages - 1, nsteps - 1);
        fetch(rg[(p + kGuStages - 1) % kGuStages], cg, coff, sn);
        fetch(ru[(p + kGuStages - 1) % kGuStages], cu, coff, sn);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 B[8];
        lds_row8(B, xl + 256 * st);
        mma_raw(accg, rg[p], slg[4 * st], B);
        mma_raw(accu, ru[p], slu[4 * st], B);
    });

    // lane holds I-columns row0 + 4 g + 0..3 of token li
    if (li < ntok) {
        const size_t rr = (size_t)(r0 + li);
        const int n = row0 + 4 * g;
        if (sh < 0) add_lora_gu(a.lora_gu, a.perm, a.k, rr, I, n, accg, accu);
        uint32_t hh[4], hl[4];
#pragma unroll
        for (int r = 0; r < 4; r++) split_bf16(act_h(a.act, accg[r], accu[r]), hh[r], hl[r]);
        uint16_t *ph = sh >= 0 ? a.sh_h_hi : a.h_hi, *pl = sh >= 0 ? a.sh_h_lo : a.h_lo;
        *(u32x2 *)(ph + rr * I + n) = u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
        *(u32x2 *)(pl + rr * I + n) = u32x2{pack2(hl[0], hl[1]), pack2(hl[2], hl[3])};
        if (a.gu && sh < 0) {
            *(float4 *)(a.gu + (rr * 2 + 0) * I + n) = float4{accg[0], accg[1], accg[2], accg[3]};
            *(float4 *)(a.gu + (rr * 2 + 1) * I + n) = float4{accu[0], accu[1], accu[2], accu[3]};
        }
    }
}

// down + routing weight.  Block = 4 waves x RT tiles x 16 rows = 64 RT H-rows of one
// active expert; h (hi and lo planes) of its tokens (<= nl_h) staged in LDS.
// PACK (at most 8 tokens): MFMA column 2j carries token j's h_hi and column 2j + 1 its
// h_lo, so one MFMA per sub-step covers both planes and the two columns are added in the
// epilogue; otherwise column j is token j and each plane takes its own MFMA.
template <int RT, bool PACK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_down_dec(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t hs[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int ai = blockIdx.y;
    const int nact = *a.n_active;
    const int sh = ai - min(a.E, a.T * a.k);  // as in k_gateup_dec
    const int e = sh >= 0 ? sh : min(max(a.active[ai], 0), a.E - 1);
    const MatW &Wd = sh >= 0 ? a.sh_down : a.down;
    const int H = a.H, I = a.I;
    const int m0 = blockIdx.x * (64 * RT) + wv * (16 * RT);
    const int nsteps = I / 256, spr = I / 32;
    const __amdgpu_buffer_rsrc_t cd = buf_rsrc(Wd.codes + (size_t)e * H * (I / 2), H * (I / 2));
    const __amdgpu_buffer_rsrc_t sd = buf_rsrc(Wd.scales + (size_t)e * H * spr, H * spr);
    uint32_t coff[RT];
#pragma unroll
    for (int t = 0; t < RT; t++) coff[t] = (uint32_t)(m0 + 16 * t + li) * (I / 2) + 32 * g;

    Raw rr[kDnStages][RT];
#pragma unroll
    for (int s = 0; s < kDnStages - 1; s++)
#pragma unroll
        for (int t = 0; t < RT; t++) fetch(rr[s][t], cd, coff[t], min(s, nsteps - 1));
    TileScales ts[RT];
#pragma unroll
    for (int t = 0; t < RT; t++) get_scales(ts[t], sd, (uint32_t)(m0 + 16 * t) * spr, lane);
    if (sh < 0 && ai >= nact) return;
    const int r0 = sh >= 0 ? sh * a.T : a.offsets[e], ntok = sh >= 0 ? a.T : a.offsets[e + 1] - r0;
    const size_t lo = (size_t)a.nl_h * (I + 8);
    stage_rows(hs, sh >= 0 ? a.sh_h_hi : a.h_hi, [&](int r) { return (size_t)(r0 + r) * I; }, ntok, I);
    stage_rows(hs + lo, sh >= 0 ? a.sh_h_lo : a.h_lo, [&](int r) { return (size_t)(r0 + r) * I; }, ntok, I);
    uint8_t *sreg = (uint8_t *)(hs + 2 * lo) + 2048 * RT * wv;
#pragma unroll
    for (int t = 0; t < RT; t++) put_scales(sreg + 2048 * t, ts[t], lane);
    __syncthreads();

    // B row of this lane: PACK -> plane li & 1 of token li >> 1, else token li (hi; lo at + lo)
    const int tok = PACK ? min(li >> 1, ntok - 1) : min(li, ntok - 1);
    const uint16_t *hl = hs + (PACK && (li & 1) ? lo : 0) + (size_t)tok * (I + 8) + 64 * g;
    const uint16_t *sl = (const uint16_t *)(sreg + li * spr + 2 * g);
    f32x4 acc[RT];
#pragma unroll
    for (int t = 0; t < RT; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    k_loop<kDnStages>(nsteps, [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
        const int sn = min(st + kDnStages - 1, nsteps - 1);
#pragma unroll
        for (int t = 0; t < RT; t++) fetch(rr[(p + kDnStages - 1) % kDnStages][t], cd, coff[t], sn);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 B[8], Bl[8];
        lds_row8(B, hl + 256 * st);
        if constexpr (!PACK) lds_row8(Bl, hl + lo + 256 * st);
#pragma unroll
        for (int t = 0; t < RT; t++) {
            const uint32_t sc = sl[1024 * t + 4 * st];
            uint32_t d[32];
            decode_fp4x32(rr[p][t].c0, e8m0_to_f32(sc & 0xFFu), d);
            decode_fp4x32(rr[p][t].c1, e8m0_to_f32(sc >> 8), d + 16);
#pragma unroll
            for (int s = 0; s < 8; s++) {
                const bf16x8 A = as_bf16x8(d[4 * s], d[4 * s + 1], d[4 * s + 2], d[4 * s + 3]);
                acc[t] = mfma16(A, B[s], acc[t]);
                if constexpr (!PACK) acc[t] = mfma16(A, Bl[s], acc[t]);
            }
        }
    });

    if constexpr (PACK) {
        // column 2j + 1 (h_lo part) onto column 2j
#pragma unroll
        for (int t = 0; t < RT; t++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[t][r] += dpp_f32<kDppXor1>(acc[t][r]);
    }
    const int j = PACK ? li >> 1 : li;
    if (j < ntok && (!PACK || (li & 1) == 0)) {
        const int slot = sh >= 0 ? j * a.sh_n + sh : a.perm[r0 + j];
        const float pw = sh >= 0 ? 1.f : a.w[slot];
        float *yb = (sh >= 0 ? a.sh_ybuf : a.ybuf) + (size_t)slot * H + m0 + 4 * g;
#pragma unroll
        for (int t = 0; t < RT; t++)
            *(float4 *)(yb + 16 * t) = float4{pw * acc[t][0], pw * acc[t][1], pw * acc[t][2], pw * acc[t][3]};
    }
}

// All experts hold at most nl_x (nl_h) tokens when T does; H % 256, I % 256 for the
// full K-steps (and the 128-row down blocks); K <= 4096 for the 2 KB scale regions.
bool dec_supported(const ExpertFwdArgs &a)
{
    return a.wfmt == FMT_MXFP4 && a.xt == DT_BF16 && a.T <= a.nl_x && a.T <= a.nl_h && a.T <= 16 &&
           a.H % 256 == 0 && a.I % 256 == 0 && a.H <= 4096 && a.I <= 4096 &&
           (size_t)a.H * a.I < ((size_t)1 << 32);
}

hipError_t launch_gateup_dec(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    ProfScope ps(a.prof, PK_GATEUP, s);
    const size_t lds = (size_t)a.nl_x * (a.H + 8) * 2 + 16384;
    ps.launch(k_gateup_dec, dim3(a.I / 64, maxU + a.sh_n), dim3(256), lds, a);
    return hipGetLastError();
}

hipError_t launch_down_dec(const ExpertFwdArgs &a, hipStream_t s)
{
    constexpr int RT = 1;  // one 16-row tile per wave: 4x as many waves as H / 16 rows per expert
    const int maxU = min(a.E, a.T * a.k);
    ProfScope ps(a.prof, PK_DOWN, s);
    const size_t lds = (size_t)a.nl_h * (a.I + 8) * 2 * 2 + 4 * 2048 * RT;
    const dim3 grid(a.H / (64 * RT), maxU + a.sh_n);
    if (a.T <= 8)
        ps.launch(k_down_dec<RT, true>, grid, dim3(256), lds, a);
    else
        ps.launch(k_down_dec<RT, false>, grid, dim3(256), lds, a);
    return hipGetLastError();
}

}  // namespace moe
