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

// A operand of MFMA sub-step s (reduction indices 8 s .. 8 s + 7 of the lane's 64): the 8
// E2M1 codes of word s % 4 of c0 (s < 4) or c1, times the block scale, as bf16 (exact).
__device__ __forceinline__ bf16x8 decode_sub(const Raw &r, float scale, int s)
{
    const uint32_t w = s < 4 ? r.c0[s & 3] : r.c1[s & 3];
    return as_bf16x8(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3)));
}

// 8 MFMA sub-steps of one K-step for one tile: A decoded from the raw bytes with the two
// scale bytes of the lane's blocks, sub-step by sub-step; B from LDS.
__device__ __forceinline__ void mma_raw(f32x4 &acc, const Raw &r, uint32_t sc, const bf16x8 (&B)[8])
{
    const float s0 = e8m0_to_f32(sc & 0xFFu), s1 = e8m0_to_f32(sc >> 8);
#pragma unroll
    for (int s = 0; s < 8; s++) acc = mfma16(decode_sub(r, s < 4 ? s0 : s1, s), B[s], acc);
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

// Cache policy of the accesses that hand data from one block to another inside the fused
// decode launch (k_dec_fused): sc1 = agent scope.  Such stores are written through to the
// point where every XCD sees them and such loads are served from there, so a block on one
// XCD reads what a block on another XCD wrote (each XCD has its own L2) without a fence over
// the whole cache; a counter incremented after the stores completed (s_waitcnt) publishes
// them.
constexpr int kSc1 = 16;

__device__ __forceinline__ u32x4 ld16_coh(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, kSc1);
}

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// sum_q v[q] b[q] for q < R (v, b 16-byte aligned when R % 4 == 0): four-wide loads, all of a
// group of up to 8 issued before the products.
__device__ __forceinline__ float dot_r(const float *v, const float *b, int R)
{
    float acc = 0.f;
    if (R % 4 == 0) {
        for (int q0 = 0; q0 < R; q0 += 32) {
            float4 va[8], ba[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int q = min(q0 + 4 * i, R - 4);
                va[i] = *(const float4 *)(v + q);
                ba[i] = *(const float4 *)(b + q);
            }
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (q0 + 4 * i < R)
                    acc = fmaf(va[i].w, ba[i].w, fmaf(va[i].z, ba[i].z, fmaf(va[i].y, ba[i].y, fmaf(va[i].x, ba[i].x, acc))));
        }
    } else {
        for (int q = 0; q < R; q++) acc = fmaf(v[q], b[q], acc);
    }
    return acc;
}

// gate/up + activation of one block: 4 waves x 16 rows = 64 I-columns (column block bx) of
// active unit ai; all of the unit's tokens (<= nl_x) in one 16-column MFMA tile.  COH: the h
// planes are stored with the agent-scope policy (read by other blocks of the same launch).
// Returns false (having done nothing else) for an unit past the active list.
template <bool COH, int NS>
__device__ __forceinline__ bool gateup_block(const ExpertFwdArgs &a, int bx, int ai, uint16_t *xs)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    // The weight prefetch needs only e: the active-list entry is read together with the
    // list length (entries past it are stale but name a valid expert) and the first code
    // loads go out before the block learns whether it has work.
    const int nact = *a.n_active;
    const int sh = ai - min(a.E, a.T * a.k);  // >= 0: shared expert sh (every token, weight 1)
    const int e = sh >= 0 ? sh : min(max(a.active[ai], 0), a.E - 1);
    const MatW &Wg = sh >= 0 ? a.sh_gate : a.gate, &Wu = sh >= 0 ? a.sh_up : a.up;
    const int H = a.H, I = a.I;
    const int row0 = bx * 64 + wv * 16;
    const int nsteps = H / 256, spr = H / 32;
    const size_t eoc = (size_t)e * I * (H / 2), eos = (size_t)e * I * spr;
    const __amdgpu_buffer_rsrc_t cg = buf_rsrc(Wg.codes + eoc, I * (H / 2));
    const __amdgpu_buffer_rsrc_t cu = buf_rsrc(Wu.codes + eoc, I * (H / 2));
    const uint32_t coff = (uint32_t)(row0 + li) * (H / 2) + 32 * g;

    Raw rg[NS], ru[NS];
#pragma unroll
    for (int s = 0; s < NS - 1; s++) {
        fetch(rg[s], cg, coff, min(s, nsteps - 1));
        fetch(ru[s], cu, coff, min(s, nsteps - 1));
    }
    TileScales tg, tu;
    get_scales(tg, buf_rsrc(Wg.scales + eos, I * spr), (uint32_t)row0 * spr, lane);
    get_scales(tu, buf_rsrc(Wu.scales + eos, I * spr), (uint32_t)row0 * spr, lane);
    if (sh < 0 && ai >= nact) return false;
    const int r0 = sh >= 0 ? sh * a.T : a.offsets[e], ntok = sh >= 0 ? a.T : a.offsets[e + 1] - r0;
    // token rows to LDS while the first weight bytes are in flight
    __shared__ uint32_t xrow[16];
    if (threadIdx.x < ntok) xrow[threadIdx.x] = sh >= 0 ? threadIdx.x : (uint32_t)(a.perm[r0 + threadIdx.x] / a.k);
    __syncthreads();
    stage_rows(xs, (const uint16_t *)a.x, [&](int r) { return (size_t)xrow[r] * H; }, ntok, H);
    uint8_t *sreg = (uint8_t *)(xs + (size_t)a.nl_x * (H + 8)) + 4096 * wv;
    put_scales(sreg, tg, lane);
    put_scales(sreg + 2048, tu, lane);
    // the fused launch's adapter: lt[t][m][c] = s (B_m vx_m of token t) at the block's column c
    // (m = 0 gate, 1 up), formed while the first weight bytes are in flight
    float *lt = (float *)((uint8_t *)(xs + (size_t)a.nl_x * (H + 8)) + 16384), *hz = lt + a.nl_x * 128;
    const bool lora = a.lora_vx && sh < 0;
    if (lora) {
        const int R = a.lora_r;
        for (int o = threadIdx.x; o < ntok * 128; o += blockDim.x) {
            const int t = o >> 7, m = (o >> 6) & 1, col = o & 63;
            const float *v = a.lora_vx + (size_t)xrow[t] * 2 * R + m * R;
            const float *bm = (m ? a.lora_Bu : a.lora_Bg) + (size_t)(bx * 64 + col) * R;
            lt[o] = a.lora_scale * dot_r(v, bm, R);
        }
    }
    __syncthreads();

    const uint16_t *xl = xs + (size_t)min(li, ntok - 1) * (H + 8) + 64 * g;
    const uint16_t *slg = (const uint16_t *)(sreg + li * spr + 2 * g);
    const uint16_t *slu = (const uint16_t *)(sreg + 2048 + li * spr + 2 * g);
    f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    k_loop<NS>(nsteps, [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
        const int sn = min(st + NS - 1, nsteps - 1);
        fetch(rg[(p + NS - 1) % NS], cg, coff, sn);
        fetch(ru[(p + NS - 1) % NS], cu, coff, sn);
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
        if (lora) {
            const float4 dg = *(const float4 *)(lt + (li * 2) * 64 + wv * 16 + 4 * g);
            const float4 du = *(const float4 *)(lt + (li * 2 + 1) * 64 + wv * 16 + 4 * g);
            accg += f32x4{dg.x, dg.y, dg.z, dg.w};
            accu += f32x4{du.x, du.y, du.z, du.w};
        } else if (sh < 0) {
            add_lora_gu(a.lora_gu, a.perm, a.k, rr, I, n, accg, accu);
        }
        uint32_t hh[4], hl[4];
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            hv[r] = act_h(a.act, accg[r], accu[r]);
            split_bf16(hv[r], hh[r], hl[r]);
        }
        if (lora) *(float4 *)(hz + li * 64 + wv * 16 + 4 * g) = float4{hv[0], hv[1], hv[2], hv[3]};
        uint16_t *ph = sh >= 0 ? a.sh_h_hi : a.h_hi, *pl = sh >= 0 ? a.sh_h_lo : a.h_lo;
        const u32x2 vh = {pack2(hh[0], hh[1]), pack2(hh[2], hh[3])}, vl = {pack2(hl[0], hl[1]), pack2(hl[2], hl[3])};
        if constexpr (COH) {
            // the planes of one unit: rows r0 .. r0 + ntok of I bf16 values each
            const uint32_t nb = (uint32_t)((size_t)(r0 + ntok) * I * 2);
            const uint32_t off = (uint32_t)((rr * I + n) * 2);
            __builtin_amdgcn_raw_buffer_store_b64(vh, buf_rsrc(ph, nb), (int)off, 0, kSc1);
            __builtin_amdgcn_raw_buffer_store_b64(vl, buf_rsrc(pl, nb), (int)off, 0, kSc1);
        } else {
            *(u32x2 *)(ph + rr * I + n) = vh;
            *(u32x2 *)(pl + rr * I + n) = vl;
        }
        if (a.gu && sh < 0) {
            *(float4 *)(a.gu + (rr * 2 + 0) * I + n) = float4{accg[0], accg[1], accg[2], accg[3]};
            *(float4 *)(a.gu + (rr * 2 + 1) * I + n) = float4{accu[0], accu[1], accu[2], accu[3]};
        }
    }
    if (lora) {
        // partials of z = A_d hbar over the block's 64 columns: lora_zp[(slot r + q) I/64 + bx]
        // = p_slot sum_c A_d[q][bx 64 + c] h(slot, c), agent-scope stores (another block sums them)
        __syncthreads();
        const int R = a.lora_r, gx = I / 64;
        const __amdgpu_buffer_rsrc_t zr = buf_rsrc(a.lora_zp, (uint32_t)((size_t)a.T * a.k * R * gx * 4));
        for (int o = threadIdx.x; o < ntok * R; o += blockDim.x) {
            const int t = o / R, q = o - t * R;
            const float *ad = a.lora_Ad + (size_t)q * I + bx * 64;
            const float *hr = hz + t * 64;
            float4 av[16];
#pragma unroll
            for (int c = 0; c < 16; c++) av[c] = *(const float4 *)(ad + 4 * c);
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < 16; c++) {
                const float4 hv4 = *(const float4 *)(hr + 4 * c);
                acc = fmaf(av[c].x, hv4.x, fmaf(av[c].y, hv4.y, fmaf(av[c].z, hv4.z, fmaf(av[c].w, hv4.w, acc))));
            }
            const int slot = a.perm[r0 + t];
            const float v = a.w[slot] * acc;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), zr,
                                                  (int)((((size_t)slot * R + q) * gx + bx) * 4), 0, kSc1);
        }
    }
    return true;
}

}  // namespace

// gate/up + activation.  Block = 4 waves x 16 rows = 64 I-columns of one active expert
// (blockIdx.y indexes the active list); all of the expert's tokens (<= nl_x) in one
// 16-column MFMA tile.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gateup_dec(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
    gateup_block<false, kGuStages>(a, blockIdx.x, blockIdx.y, xs);
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

// ---------------------------------------------------------------------------------------
// Fused decode launch: gate/up, down and combine of every unit in ONE grid.
//
// Blocks [0, ngu) are gate/up blocks as in k_gateup_dec (unit-major, I/64 column blocks per
// unit); blocks [ngu, ngu + ndn) are down blocks (unit-major, H/64 stripes of 64 rows per
// unit).  A down block first issues the loads of ALL its weight bytes (NST K-steps of 32
// bytes per lane, held in registers) and of its scale bytes, and only then waits until the
// I/64 gate/up blocks of its unit have published their h rows (a per-unit counter), so the
// down weights stream while gate/up blocks still run.  It then publishes its p-weighted
// slot rows of the stripe and counts itself into the stripe's counter; the block that
// completes a stripe (n_active + n_shared arrivals) sums the stripe's slot rows of every
// token in rank order, then the shared experts' rows: the order of k_combine, so the result
// is the same bits as the three-launch path.  That block also zeroes the stripe's counter
// and counts the stripe as done; the block that completes the last stripe zeroes the unit
// counters (every down block has passed its wait by then) and the stripe count, so each
// launch finds them at zero (the workspace region is cleared when a layer is first used).
// Each counter has a 128-byte line of its own, and waiting blocks poll it every ~0.2 us.
//
// Progress: on each XCD blocks are dispatched in index order and gate/up blocks (the lower
// indices) never wait, so every block a down block waits for is dispatched and finishes.
// The wait is also bounded (kSpinTicks of the 100 MHz real-time clock): past it the block
// sets kStatusSpinTimeout in the status word and goes on, so the grid always drains.
constexpr uint64_t kSpinTicks = 20000000;  // 200 ms
// 4 waves per SIMD (<= 128 VGPRs): all gate/up blocks and a first quarter of the down blocks
// are resident from the start, and the rest of the down blocks as gate/up blocks finish, so
// every down block has its weight loads in flight by the time the last unit's h is out.
constexpr int kFusedGuStages = 3;  // gate/up register stages
constexpr int kPre = 8;            // down K-steps loaded before the wait

// stage n contiguous bf16 rows (src + r * K) written by other blocks of this launch into LDS
// rows of stride K + 8, with the agent-scope load policy
__device__ __forceinline__ void stage_rows_coh(uint16_t *dst, const uint16_t *src, int n, int K)
{
    const __amdgpu_buffer_rsrc_t r = buf_rsrc(src, (uint32_t)((size_t)n * K * 2));
    const int per = K / 8, total = n * per;
    for (int c0 = threadIdx.x; c0 < total; c0 += 4 * blockDim.x) {
        u32x4 v[4];
        int rw[4], q[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = min(c0 + i * (int)blockDim.x, total - 1);
            rw[i] = c / per;
            q[i] = c - rw[i] * per;
            v[i] = ld16_coh(r, (uint32_t)(c * 16));
        }
#pragma unroll
        for (int i = 0; i < 4; i++) *(u32x4 *)(dst + (size_t)rw[i] * (K + 8) + 8 * q[i]) = v[i];
    }
}

// The adapter's down term for y rows [bx 64, bx 64 + 64) in the fused launch: thread (m, part)
// loads B_d[bx 64 + m][q] for ranks q = part, part + 4, ... before it waits for z (reduced by
// the last routed gate/up block, lora_z_last), then writes pd[part][t][m] = sum over its ranks
// of z[t][q] B_d[bx 64 + m][q] to LDS (scr: T r + 4 T 64 floats).  Returns pd.
__device__ __forceinline__ const float *lora_stripe(const ExpertFwdArgs &a, int bx, float *scr)
{
    const int R = a.lora_r, T = a.T, m = threadIdx.x & 63, part = threadIdx.x >> 6;
    float b[16];
    const float *brow = a.lora_Bd + (size_t)(bx * 64 + m) * R;
#pragma unroll
    for (int i = 0; i < 16; i++) b[i] = part + 4 * i < R ? brow[part + 4 * i] : 0.f;
    if (threadIdx.x == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(a.dec_sync + kSyncLoraZ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
                if (a.status) atomicOr(a.status, kStatusSpinTimeout);
                break;
            }
        }
    }
    __syncthreads();
    float *zs = scr, *pd = scr + ((T * R + 3) & ~3);
    const __amdgpu_buffer_rsrc_t zr = buf_rsrc(a.lora_z, (uint32_t)((size_t)T * R * 4));
    for (int o = threadIdx.x; o < T * R; o += blockDim.x)
        zs[o] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(zr, o * 4, 0, kSc1));
    __syncthreads();
    for (int t = 0; t < T; t++) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i++)
            if (part + 4 * i < R) d = fmaf(zs[t * R + part + 4 * i], b[i], d);
        pd[(part * T + t) * 64 + m] = d;
    }
    __syncthreads();
    return pd;
}

// y rows [bx * 64, bx * 64 + 64) of every token: the slot rows in rank order, then the
// shared experts' rows (agent-scope loads: other blocks wrote them).
__device__ __forceinline__ void combine_stripe(const ExpertFwdArgs &a, int bx, const float *pd = nullptr)
{
    const int H = a.H, k = a.k, k2 = a.sh_n, T = a.T;
    const __amdgpu_buffer_rsrc_t yb = buf_rsrc(a.ybuf, (uint32_t)((size_t)T * k * H * 4));
    const __amdgpu_buffer_rsrc_t ys = buf_rsrc(k2 ? a.sh_ybuf : a.ybuf, (uint32_t)((size_t)T * (k2 ? k2 : k) * H * 4));
    for (int i = threadIdx.x; i < T * 16; i += blockDim.x) {
        const int t = i >> 4, c = bx * 64 + 4 * (i & 15);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += 8) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; u++)
                v[u] = j0 + u < k ? ld16_coh(yb, (uint32_t)((((size_t)t * k + j0 + u) * H + c) * 4)) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < 8; u++) {
                if (j0 + u >= k) break;
                acc += __builtin_bit_cast(f32x4, v[u]);
            }
        }
        for (int j = 0; j < k2; j++) acc += __builtin_bit_cast(f32x4, ld16_coh(ys, (uint32_t)((((size_t)t * k2 + j) * H + c) * 4)));
        if (pd) {
            // the adapter's down term s B_d z: four rank-partial sums per output (lora_stripe)
            const int m = c - bx * 64;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const f32x4 d = *(const f32x4 *)(pd + (i * T + t) * 64 + m);
                acc += a.lora_scale * d;
            }
        }
        *(float4 *)(a.y + (size_t)t * H + c) = float4{acc[0], acc[1], acc[2], acc[3]};
    }
}

// down + routing weight of one block (64 rows of stripe bx, unit ai), its slot rows
// published to the stripe; the stripe's last block also combines it.
template <int NST, bool PACK>
__device__ __forceinline__ void down_block_fused(const ExpertFwdArgs &a, int bx, int ai, uint16_t *hs, int *last)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int nact = *a.n_active;
    const int sh = ai - min(a.E, a.T * a.k);  // as in gateup_block
    const int e = sh >= 0 ? sh : min(max(a.active[ai], 0), a.E - 1);
    const MatW &Wd = sh >= 0 ? a.sh_down : a.down;
    const int H = a.H, I = a.I;
    const int m0 = bx * 64 + wv * 16;
    const int nsteps = I / 256, spr = I / 32;
    const __amdgpu_buffer_rsrc_t cd = buf_rsrc(Wd.codes + (size_t)e * H * (I / 2), H * (I / 2));
    const __amdgpu_buffer_rsrc_t sd = buf_rsrc(Wd.scales + (size_t)e * H * spr, H * spr);
    const uint32_t coff = (uint32_t)(m0 + li) * (I / 2) + 32 * g;
    // the lane's first kPre K-steps of weight bytes in flight before the wait, the rest
    // issued as the first steps' registers free up
    Raw rr[NST];
#pragma unroll
    for (int st = 0; st < (NST < kPre ? NST : kPre); st++)
        if (st < nsteps) fetch(rr[st], cd, coff, st);
    TileScales ts;
    get_scales(ts, sd, (uint32_t)m0 * spr, lane);
    if (sh < 0 && ai >= nact) return;
    if (threadIdx.x == 0) {
        const uint32_t want = (uint32_t)(I / 64);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(a.dec_sync + ai * kSyncPad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
            __builtin_amdgcn_s_sleep(8);
            if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
                if (a.status) atomicOr(a.status, kStatusSpinTimeout);
                break;
            }
        }
    }
    __syncthreads();
    const int r0 = sh >= 0 ? sh * a.T : a.offsets[e], ntok = sh >= 0 ? a.T : a.offsets[e + 1] - r0;
    const size_t lo = (size_t)a.nl_h * (I + 8);
    stage_rows_coh(hs, (sh >= 0 ? a.sh_h_hi : a.h_hi) + (size_t)r0 * I, ntok, I);
    stage_rows_coh(hs + lo, (sh >= 0 ? a.sh_h_lo : a.h_lo) + (size_t)r0 * I, ntok, I);
    uint8_t *sreg = (uint8_t *)(hs + 2 * lo) + 2048 * wv;
    put_scales(sreg, ts, lane);
    __syncthreads();

    const int tok = PACK ? min(li >> 1, ntok - 1) : min(li, ntok - 1);
    const uint16_t *hl = hs + (PACK && (li & 1) ? lo : 0) + (size_t)tok * (I + 8) + 64 * g;
    const uint16_t *sl = (const uint16_t *)(sreg + li * spr + 2 * g);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NST; st++) {
        if (st < nsteps) {
            bf16x8 B[8], Bl[8];
            lds_row8(B, hl + 256 * st);
            if constexpr (!PACK) lds_row8(Bl, hl + lo + 256 * st);
            const uint32_t sc = sl[4 * st];
            const float s0 = e8m0_to_f32(sc & 0xFFu), s1 = e8m0_to_f32(sc >> 8);
#pragma unroll
            for (int s = 0; s < 8; s++) {
                const bf16x8 A = decode_sub(rr[st], s < 4 ? s0 : s1, s);
                acc = mfma16(A, B[s], acc);
                if constexpr (!PACK) acc = mfma16(A, Bl[s], acc);
            }
            if (st + kPre < NST && st + kPre < nsteps) fetch(rr[st + kPre], cd, coff, st + kPre);
        }
    }
    if constexpr (PACK) {
#pragma unroll
        for (int r = 0; r < 4; r++) acc[r] += dpp_f32<kDppXor1>(acc[r]);
    }
    const int j = PACK ? li >> 1 : li;
    if (j < ntok && (!PACK || (li & 1) == 0)) {
        const int slot = sh >= 0 ? j * a.sh_n + sh : a.perm[r0 + j];
        const float pw = sh >= 0 ? 1.f : a.w[slot];
        float *yb = sh >= 0 ? a.sh_ybuf : a.ybuf;
        const size_t rows = (size_t)a.T * (sh >= 0 ? a.sh_n : a.k);
        const f32x4 v = {pw * acc[0], pw * acc[1], pw * acc[2], pw * acc[3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), buf_rsrc(yb, (uint32_t)(rows * H * 4)),
                                               (int)(((size_t)slot * H + m0 + 4 * g) * 4), 0, kSc1);
    }
    wait_stores();
    __syncthreads();
    uint32_t *stripe = a.dec_sync + (kSyncUnits + bx) * kSyncPad;
    if (threadIdx.x == 0) {
        const uint32_t n = __hip_atomic_fetch_add(stripe, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *last = n + 1 == (uint32_t)(nact + a.sh_n);
    }
    __syncthreads();
    if (!*last) return;
    const float *pd = a.lora_vx ? lora_stripe(a, bx, (float *)hs) : nullptr;
    combine_stripe(a, bx, pd);
    if (threadIdx.x == 0) {
        // the stripe is complete: reset its counter; the last complete stripe resets the rest
        __hip_atomic_store(stripe, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t *done = a.dec_sync + (kSyncUnits + kSyncStripes) * kSyncPad;
        const uint32_t n = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n + 1 == (uint32_t)(H / 64)) {
            const int nu = min(a.E, a.T * a.k) + a.sh_n;
            for (int u = 0; u < nu; u++) __hip_atomic_store(a.dec_sync + u * kSyncPad, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.dec_sync + kSyncLoraGu, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.dec_sync + kSyncLoraZ, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The adapter in the fused launch: a routed gate/up block counts itself (its z partials are
// stored); the last of them sums the partials into z[t][q] = sum over the token's slots j in
// rank order and the column blocks c of lora_zp[((t k + j) r + q) I/64 + c] (thread group gi
// of an output takes slots j = gi, gi + ng, ..., each with all its column blocks in one round
// of loads; the groups are then summed in order), stores z [T][r] and raises the flag the
// combining blocks wait for.  scr: 256 + 16 x 64 floats of LDS.
__device__ __forceinline__ void lora_z_last(const ExpertFwdArgs &a, int gx, int *flag, float *scr)
{
    if (threadIdx.x == 0) {
        const uint32_t n = __hip_atomic_fetch_add(a.dec_sync + kSyncLoraGu, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = n + 1 == (uint32_t)(*a.n_active * gx);
    }
    __syncthreads();
    if (!*flag) return;
    float *zs = scr, *zl = scr + 256;
    const int R = a.lora_r, T = a.T, k = a.k;
    const int nout = T * R;  // <= 16 x 64
    const __amdgpu_buffer_rsrc_t zr = buf_rsrc(a.lora_zp, (uint32_t)((size_t)T * k * R * gx * 4));
    for (int o0 = 0; o0 < nout; o0 += 256) {
        const int nb = min(256, nout - o0);  // outputs of this round
        const int ng = min(256 / nb, k);     // thread groups per output
        const int o = o0 + threadIdx.x % nb, gi = threadIdx.x / nb;
        float acc = 0.f;
        if (gi < ng) {
            const int t = o / R, q = o - t * R;
            for (int j = gi; j < k; j += ng) {
                // the gx <= 64 column-block partials of (slot, q): up to 16 loads issued together
                const uint32_t base = (uint32_t)((((size_t)(t * k + j) * R + q) * gx) * 4);
                f32x4 v[16];
#pragma unroll
                for (int i = 0; i < 16; i++)
                    v[i] = 4 * i < gx ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(zr, (int)(base + 16 * i), 0, kSc1))
                                      : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 16; i++) acc += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
            }
        }
        zs[threadIdx.x] = acc;
        __syncthreads();
        if (threadIdx.x < nb) {
            float z = zs[threadIdx.x];
            for (int g2 = 1; g2 < ng; g2++) z += zs[g2 * nb + threadIdx.x];
            zl[o0 + threadIdx.x] = z;
        }
        __syncthreads();
    }
    const __amdgpu_buffer_rsrc_t zo = buf_rsrc(a.lora_z, (uint32_t)((size_t)nout * 4));
    for (int o = threadIdx.x; o < nout; o += blockDim.x)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, zl[o]), zo, (int)(o * 4), 0, kSc1);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(a.dec_sync + kSyncLoraZ, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NST, bool PACK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_dec_fused(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    __shared__ int last;
    const int nu = min(a.E, a.T * a.k) + a.sh_n;
    const int gx = a.I / 64, hx = a.H / 64;
    const int b = blockIdx.x;
    if (b < gx * nu) {
        const int ai = b / gx;
        if (gateup_block<true, kFusedGuStages>(a, b - ai * gx, ai, lds)) {
            wait_stores();
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(a.dec_sync + ai * kSyncPad, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // scratch: the block's scale regions (16 KB past the x rows), free after its K loop
            if (a.lora_vx && ai < min(a.E, a.T * a.k))
                lora_z_last(a, gx, &last, (float *)(lds + (size_t)a.nl_x * (a.H + 8)));
        }
    } else {
        const int d = b - gx * nu;
        down_block_fused<NST, PACK>(a, d % hx, d / hx, lds, &last);
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

bool dec_fused_ok(const ExpertFwdArgs &a)
{
    return a.dec_sync && dec_supported(a) && a.I / 256 <= 12 && a.H / 64 <= kSyncStripes &&
           min(a.E, a.T * a.k) + a.sh_n <= kSyncUnits && !a.skip_combine;
}

template <int NST>
static hipError_t launch_fused_nst(const ExpertFwdArgs &a, hipStream_t s)
{
    const int nu = min(a.E, a.T * a.k) + a.sh_n;
    // gate/up blocks: x rows, 16 KB of scales, and with the adapter its terms and h (768 B a token)
    const size_t lds_g = (size_t)a.nl_x * (a.H + 8) * 2 + 16384 + (a.lora_vx ? (size_t)a.nl_x * 768 : 0),
                 lds_d = (size_t)a.nl_h * (a.I + 8) * 2 * 2 + 4 * 2048;
    const dim3 grid((unsigned)((a.I / 64 + a.H / 64) * nu));
    ProfScope ps(a.prof, PK_GATEUP, s);
    if (a.T <= 8)
        ps.launch(k_dec_fused<NST, true>, grid, dim3(256), lds_g > lds_d ? lds_g : lds_d, a);
    else
        ps.launch(k_dec_fused<NST, false>, grid, dim3(256), lds_g > lds_d ? lds_g : lds_d, a);
    return hipGetLastError();
}

hipError_t launch_dec_fused(const ExpertFwdArgs &a, hipStream_t s)
{
    const int nst = a.I / 256;
    if (nst <= 4) return launch_fused_nst<4>(a, s);
    if (nst <= 8) return launch_fused_nst<8>(a, s);
    return launch_fused_nst<12>(a, s);
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
