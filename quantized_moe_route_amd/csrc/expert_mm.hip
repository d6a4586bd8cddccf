// expert_mm.hip -- grouped-GEMM expert forward for experts holding many tokens (MXFP4).
//
// Same arithmetic as the few-token kernels of expert_fwd.hip (LazyLoRA README, "The
// engine" / "Arithmetic": experts consumed in their packed format, fp32 accumulation;
// "Measurement findings": one sweep over each expert's bytes amortised over all of the
// expert's tokens), organised for experts with tens of tokens (prefill and training
// batches):
//
//  - a block owns one expert, a column block of the output (128 I-columns of gate and
//    up, or 256 rows of H for down) and all of the expert's tokens, up to 96 per pass in
//    at most six tiles of 16 (the tile count is a template parameter chosen per pass, so
//    the inner loop carries no per-tile branches);
//  - the token operand of one K-step (gathered x rows, or the bf16 hi/lo planes of h)
//    is staged in LDS, double-buffered and shared by the block's four waves; each wave
//    applies every token fragment to its four 16-row weight tiles with
//    v_mfma_f32_16x16x32_bf16;
//  - weight codes and scale bytes stream from HBM into registers two K-steps ahead (three
//    register stages, the K loop unrolled by three so that no stage is copied) and are
//    dequantized exactly to bf16 (v_cvt_scalef32_pk_bf16_fp4) right before use;
//  - blocks are spread over the XCDs expert by expert (xcd_split), so that the column
//    blocks of one expert, which all read the same token rows, share one L2.
//
// LDS tile: [96 rows][16 chunks of 16 bytes]; chunk c of row r sits in slot c ^ (r & 15),
// which spreads the 16 rows read by one MFMA operand load over all banks.
#include <type_traits>

#include "common.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMmTT = 6;            // token tiles of 16 per pass
constexpr int kMmTok = 16 * kMmTT;  // tokens per pass

template <int P>
using Stage = std::integral_constant<int, P>;

typedef u32x4 MmTile[kMmTok * 16];

// XCD-aware work split.  The dispatcher hands block b to XCD b % 8; active expert ai
// goes to XCD ai % 8, whose blocks walk their experts in order, nb blocks per expert.
// The grid holds 8 * ceil(maxU / 8) * nb blocks.
__device__ __forceinline__ void xcd_split(int nb, int &ai, int &cb)
{
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int q = j / nb;
    cb = j - q * nb;
    ai = 8 * q + x;
}

static inline int xcd_grid(int maxU, int nb) { return 8 * ((maxU + 7) / 8) * nb; }

static_assert(kMmTok == kTokChunk, "token chunks are one pass");

// The slot rows [r0, r0 + ntok) of work unit ai (an active expert, or with tok_chunks
// one chunk of kTokChunk tokens of expert ai / tok_chunks); false: nothing to do.
__device__ __forceinline__ bool mm_tokens(int tok_chunks, int &ai, const int32_t *n_active, const int32_t *active,
                                          const int32_t *offsets, int &r0, int &ntok)
{
    int c = 0;
    if (tok_chunks > 0) {
        c = ai % tok_chunks;
        ai /= tok_chunks;
    }
    if (ai >= *n_active) return false;
    const int e = active[ai];
    r0 = offsets[e];
    ntok = offsets[e + 1] - r0;
    if (tok_chunks > 0) {
        r0 += c * kTokChunk;
        ntok = min(kTokChunk, ntok - c * kTokChunk);
    }
    return ntok > 0;
}

// Work units of a grouped-GEMM launch: active experts, or expert token chunks.
static inline int mm_units(const ExpertFwdArgs &a)
{
    return a.tok_chunks > 0 ? a.E * a.tok_chunks : min(a.E, a.T * a.k);
}

__device__ __forceinline__ int lds_slot(int row, int chunk) { return row * 16 + (chunk ^ (row & 15)); }

// 8 E2M1 codes (one dword) times a power-of-two scale -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale)
{
    const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return as_bf16x8(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                     __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3));
}

// Buffer resource over [p, p + bytes): raw (untyped) loads through it take a 32-bit lane
// offset plus a wave-uniform offset, so an address costs one VGPR instead of two, and
// offsets past `bytes` read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ u32x2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ uint32_t ld1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// Runs step(Stage<st % 3>, st) for st = 0 .. n-1.  The loop body is three whole steps
// with the remainder peeled after it, so the loop has a single back edge and the wait
// counts the compiler derives at its head stay exact.
template <typename F>
__device__ __forceinline__ void k_loop3(int n, F &&step)
{
    int s0 = 0;
    for (; s0 + 3 <= n; s0 += 3) {
        step(Stage<0>(), s0);
        step(Stage<1>(), s0 + 1);
        step(Stage<2>(), s0 + 2);
    }
    if (s0 < n) step(Stage<0>(), s0);
    if (s0 + 1 < n) step(Stage<1>(), s0 + 1);
}

// Runs step(Stage<st % 6>, st) for st = 0 .. n-1, so that both st % 3 (a register stage)
// and st % 2 (an LDS buffer) are known at compile time in each copy of the body.
template <typename F>
__device__ __forceinline__ void k_loop6(int n, F &&step)
{
    int s0 = 0;
    for (; s0 + 6 <= n; s0 += 6) {
        step(Stage<0>(), s0);
        step(Stage<1>(), s0 + 1);
        step(Stage<2>(), s0 + 2);
        step(Stage<3>(), s0 + 3);
        step(Stage<4>(), s0 + 4);
        step(Stage<5>(), s0 + 5);
    }
    if (s0 < n) step(Stage<0>(), s0);
    if (s0 + 1 < n) step(Stage<1>(), s0 + 1);
    if (s0 + 2 < n) step(Stage<2>(), s0 + 2);
    if (s0 + 3 < n) step(Stage<3>(), s0 + 3);
    if (s0 + 4 < n) step(Stage<4>(), s0 + 4);
}

// Runs step(Stage<st % 2>, st) for st = 0 .. n-1: two register stages.
template <typename F>
__device__ __forceinline__ void k_loop2(int n, F &&step)
{
    int s0 = 0;
    for (; s0 + 2 <= n; s0 += 2) {
        step(Stage<0>(), s0);
        step(Stage<1>(), s0 + 1);
    }
    if (s0 < n) step(Stage<0>(), s0);
}

// ---------------------------------------------------------------- scale bytes in LDS
//
// A block's weight rows take their E8M0 scale bytes from LDS.  Read from global memory a
// few bytes per K-step, each scale line stays live for the block's whole K loop, and with
// two blocks on each of the XCD's CUs those lines and the half-consumed code lines
// outgrow the L2: both are fetched from HBM again and again (1.65x the algorithmic bytes
// measured on the 4096-token gate/up).  Instead the block copies its rows' scale bytes of
// up to kSclRow bytes per row (one K chunk) into LDS with coalesced 16-byte loads before
// the chunk's first step, where every step reads them.  Row pitch kSclRow = 28 dwords, so
// the 16 rows read by one lane group land in 16 distinct banks.

constexpr int kSclRow = 112;  // LDS bytes per weight row and chunk

// Pieces of 16 bytes per thread for NROWS rows of at most kSclRow bytes.
template <int NROWS>
constexpr int scl_pieces() { return (NROWS * (kSclRow / 16) + 255) / 256; }

// Loads the scale bytes [byte0, byte0 + nbytes) of NROWS consecutive rows (row stride
// gstride bytes from boff in resource r; nbytes a multiple of 16, at most kSclRow).  The
// resource is the same for the whole wave, so the loads are plain buffer loads.
template <int NROWS>
__device__ __forceinline__ void scl_load(u32x4 (&v)[scl_pieces<NROWS>()], __amdgpu_buffer_rsrc_t r, uint32_t boff,
                                         int gstride, int byte0, int nbytes)
{
    const int per_row = nbytes >> 4;
#pragma unroll
    for (int k = 0; k < scl_pieces<NROWS>(); k++) {
        const int i = (int)threadIdx.x + 256 * k;
        const int row = i / per_row, j = i - row * per_row;
        v[k] = u32x4{0u, 0u, 0u, 0u};
        if (row < NROWS) v[k] = ld16(r, (uint32_t)row * gstride + 16 * j, boff + byte0);
    }
}

template <int NROWS>
__device__ __forceinline__ void scl_store(const u32x4 (&v)[scl_pieces<NROWS>()], uint8_t *scl, int nbytes)
{
    const int per_row = nbytes >> 4;
#pragma unroll
    for (int k = 0; k < scl_pieces<NROWS>(); k++) {
        const int i = (int)threadIdx.x + 256 * k;
        const int row = i / per_row, j = i - row * per_row;
        if (row < NROWS) *(u32x4 *)(scl + row * kSclRow + 16 * j) = v[k];
    }
}

// The same copy one piece at a time (four registers): for the K chunks after the first,
// inside the K loop, where the weight and token stages hold most registers.  Each piece
// waits for its load; it runs once per 3584 elements of K.
__device__ __forceinline__ void scl_copy_serial(uint8_t *scl, int nrows, __amdgpu_buffer_rsrc_t r, uint32_t boff,
                                                int gstride, int byte0, int nbytes)
{
    const int per_row = nbytes >> 4;
#pragma unroll 1
    for (int i = (int)threadIdx.x; i < nrows * per_row; i += 256) {
        const int row = i / per_row, j = i - row * per_row;
        *(u32x4 *)(scl + row * kSclRow + 16 * j) = ld16(r, (uint32_t)row * gstride + 16 * j, boff + byte0);
    }
}

// ---------------------------------------------------------------- x as two E4M3 terms
//
// For the block-scaled gate/up, each 32-element block of a token row is written as
// x = 2^e1 q1 + 2^e2 q2 (+ a remainder below 2^-20 of the block maximum), q1, q2 E4M3
// (OCP, round to nearest even), e1 = exponent of the block maximum - 7 (so |x| 2^-e1 <
// 256 < 448) and e2 likewise for the remainder x - 2^e1 q1 (exact in fp32).  A bf16 value
// has 8 significant bits and each term carries 4, so only elements more than 2^6 below
// the block maximum can leave a remainder.
// Layout: per token, per K-step of 128 elements, the 128 q1 bytes then the 128 q2 bytes
// (a token row is 2H bytes, like the bf16 row); scales [T][H/32][2] (e1 + 127, e2 + 127).

__device__ __forceinline__ int block_exp(float m)  // exponent of m's leading bit - 7, in E8M0 range
{
    const int e = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127 - 7;
    return e < -127 ? -127 : e;
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }  // -126..127

__global__ __launch_bounds__(256) void k_x_terms(const uint16_t *__restrict__ x, int T, int H, uint8_t *__restrict__ xq,
                                                 uint8_t *__restrict__ xs)
{
    const int nb = H / 32;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)T * nb) return;
    const size_t t = i / nb;
    const int q = (int)(i - t * nb);
    float v[32];
    const u32x4 *src = (const u32x4 *)(x + t * H + 32 * q);
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const u32x4 w = src[c];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            v[8 * c + 2 * j] = __uint_as_float(w[j] << 16);
            v[8 * c + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
    uint8_t *dst = xq + t * (size_t)(2 * H) + (size_t)(q >> 2) * 256 + 32 * (q & 3);
    int eb[2];
#pragma unroll
    for (int p = 0; p < 2; p++) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j++) m = fmaxf(m, fabsf(v[j]));
        const int e = block_exp(m);
        eb[p] = e + 127;
        // 2^-e in two factors, so that e = -127 stays in range
        const float inv_hi = pow2f(-(e >> 1)), inv_lo = pow2f(-(e - (e >> 1)));
        u32x4 out[2];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const float a0 = v[2 * j] * inv_hi * inv_lo, a1 = v[2 * j + 1] * inv_hi * inv_lo;
            const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false) & 0xFFFFu;
            const uint32_t sh = 16 * (j & 1);
            if ((j & 1) == 0) out[j >> 3][(j >> 1) & 3] = pk;
            else out[j >> 3][(j >> 1) & 3] |= pk << sh;
            // remainder for the next term: x - 2^e q (q decoded back from the byte)
            const float d0 = __builtin_amdgcn_cvt_f32_fp8((int)pk, 0), d1 = __builtin_amdgcn_cvt_f32_fp8((int)pk, 1);
            const float sc_hi = pow2f(e >> 1), sc_lo = pow2f(e - (e >> 1));
            v[2 * j] -= d0 * sc_hi * sc_lo;
            v[2 * j + 1] -= d1 * sc_hi * sc_lo;
        }
        *(u32x4 *)(dst + 128 * p) = out[0];
        *(u32x4 *)(dst + 128 * p + 16) = out[1];
    }
    *(uint16_t *)(xs + 2 * i) = (uint16_t)(eb[0] | (eb[1] << 8));
}

// ---------------------------------------------------------------- gate/up + activation
//
// K-step 128: lane group g = lane / 16 owns reduction indices [32g, 32g + 32) of the
// step, one MX scale block = 16 code bytes; sub-step s takes indices 32g + 8s + 0..7
// on both operands.  Wave wv owns I-columns c0 = 128 cb + 32 wv .. +32 of gate
// (tiles 0, 1) and of up (tiles 2, 3).

struct GuBlock {
    __amdgpu_buffer_rsrc_t code[2], scale[2];  // this expert's gate and up matrices
    __amdgpu_buffer_rsrc_t x;                   // the token rows
    uint32_t coff;                              // this lane's code byte offset at K-step 0
    uint32_t sblk;                              // the block's first scale row (byte offset)
    uint32_t sl;                                // this lane's scale byte in LDS (gate rows, K-step 0)
    int c0;                                     // first I-column of this wave
};

constexpr int kGuSclSteps = kSclRow / 4;  // gate/up K-steps per scale chunk (4 scale bytes a step)

// The block's gate (LDS rows 0..127) and up (128..255) scale bytes of the chunk at K-step
// st0: loaded, then stored.
struct GuScl {
    u32x4 g[scl_pieces<128>()], u[scl_pieces<128>()];
};

__device__ __forceinline__ void gu_scl_load(GuScl &v, const GuBlock &b, int H, int st0, int nsteps)
{
    const int nb = 4 * min(kGuSclSteps, nsteps - st0);
    scl_load<128>(v.g, b.scale[0], b.sblk, H / 32, 4 * st0, nb);
    scl_load<128>(v.u, b.scale[1], b.sblk, H / 32, 4 * st0, nb);
}

__device__ __forceinline__ void gu_scl_store(const GuScl &v, uint8_t *scl, int st0, int nsteps)
{
    const int nb = 4 * min(kGuSclSteps, nsteps - st0);
    scl_store<128>(v.g, scl, nb);
    scl_store<128>(v.u, scl + 128 * kSclRow, nb);
}

__device__ __forceinline__ void gu_scl_next(uint8_t *scl, const GuBlock &b, int H, int st0, int nsteps)
{
    const int nb = 4 * min(kGuSclSteps, nsteps - st0);
    __syncthreads();  // every wave is past the previous chunk's last step
    scl_copy_serial(scl, 128, b.scale[0], b.sblk, H / 32, 4 * st0, nb);
    scl_copy_serial(scl + 128 * kSclRow, 128, b.scale[1], b.sblk, H / 32, 4 * st0, nb);
    __syncthreads();
}

// s_waitcnt with only the vector-memory count: vmcnt(n), no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// xs0, xs1: the two x-tile buffers, separate LDS arrays (step st reads buffer st % 2 while
// the next tile streams into the other; as distinct objects the compiler can see that the
// stream does not alias the reads, and need not wait for it before them).
template <int NT>
__device__ __forceinline__ void gateup_pass(const ExpertFwdArgs &a, const GuBlock &b, u32x4 *xs0, u32x4 *xs1,
                                            uint8_t *scl, int r0, int tt0, int nt)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, li = lane & 15;
    const int H = a.H, I = a.I, nsteps = H / 128;
    // The x tile goes straight from memory to LDS (buffer loads with the LDS flag): piece i
    // of wave wv fills the 64 slots 64 (wv + 4 i) .. +63, slot s = 16 row + (chunk ^ (row &
    // 15)), so lane l loads row 16 i + 4 wv + l / 16, chunk (l % 16) ^ (row % 16).  Nothing
    // of it passes through registers.
    uint32_t xoff[NT];  // byte offsets at K-step 0
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int row = 16 * i + 4 * wv + (lane >> 4), chunk = (lane & 15) ^ (row & 15);
        const int tok = a.perm[r0 + tt0 + min(row, nt - 1)] / a.k;
        xoff[i] = ((uint32_t)tok * H + 8 * chunk) * 2;
    }
    auto load_x = [&](u32x4 *dst, int st) {
#pragma unroll
        for (int i = 0; i < NT; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                b.x, (__attribute__((address_space(3))) void *)((char *)dst + 1024 * (wv + 4 * i)), 16, xoff[i],
                256 * st, 0, 0);
    };
    f32x4 acc[4][NT];
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
        for (int tt = 0; tt < NT; tt++) acc[t][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 q[3][4];
    auto load_w = [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int t = 0; t < 4; t++) q[p][t] = ld16(b.code[t >> 1], b.coff, (t & 1) * 8 * H + 64 * st);
    };
    {
        GuScl sv;
        gu_scl_load(sv, b, H, 0, nsteps);
        load_x(xs0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_w(Stage<0>(), 0);
        load_w(Stage<1>(), min(1, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);
        gu_scl_store(sv, scl, 0, nsteps);
        wait_vmcnt<8>();  // the x tile (issued before the eight weight loads)
    }
    __syncthreads();
    // the scale bytes of the step are read from LDS one step ahead
    uint32_t scn[4];
#pragma unroll
    for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + (t >> 1) * 128 * kSclRow + (t & 1) * 16 * kSclRow + 4 * 0];

    k_loop6(nsteps, [&](auto P6, int st) {
        constexpr int p = decltype(P6)::value % 3, parity = decltype(P6)::value & 1;
        u32x4 *const xcur = parity ? xs1 : xs0, *const xnxt = parity ? xs0 : xs1;
        const int sst = st % kGuSclSteps;
        if (sst == 0 && st != 0) {  // the next K chunk (H beyond 3584)
            gu_scl_next(scl, b, H, st, nsteps);
#pragma unroll
            for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + (t >> 1) * 128 * kSclRow + (t & 1) * 16 * kSclRow + 4 * 0];
        }
        // next step's x tile into the other buffer, issued before the weights so that waiting
        // for it leaves the weight prefetch in flight
        load_x(xnxt, min(st + 1, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(Stage<(p + 2) % 3>(), min(st + 2, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the step's MFMAs
        float scale[4];
#pragma unroll
        for (int t = 0; t < 4; t++) scale[t] = e8m0_to_f32(scn[t]);
        if (sst + 1 < kGuSclSteps && st + 1 < nsteps)
#pragma unroll
            for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + (t >> 1) * 128 * kSclRow + (t & 1) * 16 * kSclRow + 4 * (sst + 1)];
#pragma unroll
        for (int s = 0; s < 4; s++) {
            bf16x8 A[4], B[NT];
#pragma unroll
            for (int tt = 0; tt < NT; tt++) B[tt] = as_bf16x8(xcur[lds_slot(16 * tt + li, 4 * g + s)]);
#pragma unroll
            for (int t = 0; t < 4; t++) A[t] = fp4x8_to_bf16(q[p][t][s], scale[t]);
#pragma unroll
            for (int tt = 0; tt < NT; tt++)
#pragma unroll
                for (int t = 0; t < 4; t++) acc[t][tt] = mfma16(A[t], B[tt], acc[t][tt]);
        }
        wait_vmcnt<4>();  // this thread's part of the next x tile (the 4 weight loads came after)
        __syncthreads();
    });

    // the shared adapter's per-token terms for every tile of the lane, loaded together
    f32x4 lgv[NT][2], luv[NT][2];
    if (a.lora_gu) {
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            const int tok = a.perm[r0 + tt0 + min(16 * tt + li, nt - 1)] / a.k;
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const float *p = a.lora_gu + (size_t)tok * 2 * I + b.c0 + 16 * t + 4 * g;
                const float4 dg = *(const float4 *)p, du = *(const float4 *)(p + I);
                lgv[tt][t] = f32x4{dg.x, dg.y, dg.z, dg.w};
                luv[tt][t] = f32x4{du.x, du.y, du.z, du.w};
            }
        }
    }
    // lane (g, li) holds I-columns c0 + 16 (t & 1) + 4 g + 0..3 of token 16 tt + li
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
        const int j = 16 * tt + li;
        if (j >= nt) continue;
        const size_t rr = (size_t)(r0 + tt0 + j);
#pragma unroll
        for (int t = 0; t < 2; t++) {
            f32x4 gv = acc[t][tt], uv = acc[t + 2][tt];
            const int n = b.c0 + 16 * t + 4 * g;
            if (a.lora_gu) {
                gv += lgv[tt][t];
                uv += luv[tt][t];
            }
            uint32_t hh[4], hl[4];
#pragma unroll
            for (int r = 0; r < 4; r++) split_bf16(act_h(a.act, gv[r], uv[r]), hh[r], hl[r]);
            *(u32x2 *)(a.h_hi + rr * I + n) = u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
            *(u32x2 *)(a.h_lo + rr * I + n) = u32x2{pack2(hl[0], hl[1]), pack2(hl[2], hl[3])};
            if (a.gu) {
                *(float4 *)(a.gu + (rr * 2 + 0) * I + n) = float4{gv[0], gv[1], gv[2], gv[3]};
                *(float4 *)(a.gu + (rr * 2 + 1) * I + n) = float4{uv[0], uv[1], uv[2], uv[3]};
            }
        }
    }
}

__global__ __launch_bounds__(256, 2) void k_gateup_mm(const ExpertFwdArgs a)
{
    __shared__ MmTile xs0, xs1;
    __shared__ __attribute__((aligned(16))) uint8_t scl[256 * kSclRow];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int H = a.H, I = a.I;
    int ai, cb, r0, ntok;
    xcd_split(I / 128, ai, cb);
    if (!mm_tokens(a.tok_chunks, ai, a.n_active, a.active, a.offsets, r0, ntok)) return;
    const int e = a.active[ai];
    GuBlock b;
    const size_t eoc = (size_t)e * I * (H / 2), eos = (size_t)e * I * (H / 32);
    b.code[0] = buf_rsrc(a.gate.codes + eoc, I * (H / 2));
    b.code[1] = buf_rsrc(a.up.codes + eoc, I * (H / 2));
    b.scale[0] = buf_rsrc(a.gate.scales + eos, I * (H / 32));
    b.scale[1] = buf_rsrc(a.up.scales + eos, I * (H / 32));
    b.x = buf_rsrc(a.x, (uint32_t)((size_t)a.T * H * 2));
    b.c0 = cb * 128 + wv * 32;
    b.coff = (uint32_t)(b.c0 + li) * (H / 2) + 16 * g;
    b.sblk = (uint32_t)cb * 128 * (H / 32);
    b.sl = (uint32_t)(wv * 32 + li) * kSclRow + g;
    for (int tt0 = 0; tt0 < ntok; tt0 += kMmTok) {
        const int nt = min(kMmTok, ntok - tt0);
        switch ((nt + 15) / 16) {
        case 1: gateup_pass<1>(a, b, xs0, xs1, scl, r0, tt0, nt); break;
        case 2: gateup_pass<2>(a, b, xs0, xs1, scl, r0, tt0, nt); break;
        case 3: gateup_pass<3>(a, b, xs0, xs1, scl, r0, tt0, nt); break;
        case 4: gateup_pass<4>(a, b, xs0, xs1, scl, r0, tt0, nt); break;
        case 5: gateup_pass<5>(a, b, xs0, xs1, scl, r0, tt0, nt); break;
        default: gateup_pass<6>(a, b, xs0, xs1, scl, r0, tt0, nt); break;
        }
    }
}

// ---------------------------------------------------------------- block-scaled gate/up + activation
//
// Same blocking as k_gateup_mm, on v_mfma_scale_f32_16x16x128_f8f6f4: the weight tile
// enters as its FP4 codes with their E8M0 scale (A operand; lane group g holds the
// step's reduction indices 32g .. 32g+31, one MX block, exactly the 16 bytes and the
// scale byte the lane loads), the token tile as the two E4M3 terms of x with their
// block scales (B operand; lane group g holds indices 16g .. 16g+15 and 64+16g ..
// 64+16g+15; the scale of block q of a row or column comes from lane group q).  One
// MFMA per term and 16 x 16 tile covers a K-step of 128, with no dequantization.
// The LDS row of a token holds the step's q1 bytes (chunks 0..7) then q2 (8..15);
// the terms' scales go to a separate 8-byte-per-token array.

template <int PB>
__device__ __forceinline__ f32x4 mfma_mx(u32x4 a, u32x4 b0, u32x4 b1, f32x4 c, uint32_t sa, uint32_t sb)
{
    typedef __attribute__((ext_vector_type(8))) int i32x8;
    typedef __attribute__((ext_vector_type(4))) int i32x4;
    const i32x4 a4 = __builtin_bit_cast(i32x4, a);
    // an FP4 operand occupies the low four registers only; the upper half is left undefined
    const i32x8 A = __builtin_shufflevector(a4, a4, 0, 1, 2, 3, -1, -1, -1, -1);
    const i32x8 B = __builtin_shufflevector(__builtin_bit_cast(i32x4, b0), __builtin_bit_cast(i32x4, b1), 0, 1, 2, 3, 4,
                                            5, 6, 7);
    // A: FP4 (format 4), scale byte 0 of sa; B: E4M3 (format 0), scale byte PB of sb
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 0, 0, (int)sa, PB, (int)sb);
}

typedef u32x2 MmScl[kMmTok];

template <int NT, int NTERM>
__device__ __forceinline__ void gateup_pass_mx(const ExpertFwdArgs &a, const GuBlock &b, MmTile *xs, MmScl *xsc,
                                               uint8_t *scl, int r0, int tt0, int nt)
{
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int H = a.H, I = a.I, nsteps = H / 128;
    const int xr = tid >> 4, xc = tid & 15;  // this thread's x-tile row (+16 i) and chunk
    const __amdgpu_buffer_rsrc_t xsr = buf_rsrc(a.xq_s, (uint32_t)((size_t)a.T * (H / 16)));
    uint32_t xoff[NT];                       // byte offsets at K-step 0
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int tok = a.perm[r0 + tt0 + min(xr + 16 * i, nt - 1)] / a.k;
        xoff[i] = (uint32_t)tok * (2 * H) + 16 * xc;
    }
    // scales: thread tid < 16 NT stages token row tid's 8 bytes per step
    const bool sthr = tid < 16 * NT;
    const uint32_t soffx = (uint32_t)(a.perm[r0 + tt0 + min(tid, nt - 1)] / a.k) * (H / 16);
    f32x4 acc[4][NT];
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
        for (int tt = 0; tt < NT; tt++) acc[t][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 q[2][4];
    auto load_w = [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int t = 0; t < 4; t++) q[p][t] = ld16(b.code[t >> 1], b.coff, (t & 1) * 8 * H + 64 * st);
    };
    {
        GuScl wsv;
        gu_scl_load(wsv, b, H, 0, nsteps);
        u32x4 xv[NT];
#pragma unroll
        for (int i = 0; i < NT; i++) xv[i] = ld16(b.x, xoff[i], 0);
        const u32x2 sv = ld8(xsr, soffx, 0);
        gu_scl_store(wsv, scl, 0, nsteps);
        load_w(Stage<0>(), 0);
#pragma unroll
        for (int i = 0; i < NT; i++) xs[0][lds_slot(xr + 16 * i, xc)] = xv[i];
        if (sthr) xsc[0][tid] = sv;
    }
    __syncthreads();
    uint32_t scn[4];  // the scale bytes of the step, read from LDS one step ahead
#pragma unroll
    for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + (t >> 1) * 128 * kSclRow + (t & 1) * 16 * kSclRow + 4 * 0];

    k_loop2(nsteps, [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
        const int buf = st & 1;
        const int sst = st % kGuSclSteps;
        if (sst == 0 && st != 0) {  // the next K chunk (H beyond 3584)
            gu_scl_next(scl, b, H, st, nsteps);
#pragma unroll
            for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + (t >> 1) * 128 * kSclRow + (t & 1) * 16 * kSclRow + 4 * 0];
        }
        uint32_t sc[4];
#pragma unroll
        for (int t = 0; t < 4; t++) sc[t] = scn[t];
        if (sst + 1 < kGuSclSteps && st + 1 < nsteps)
#pragma unroll
            for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + (t >> 1) * 128 * kSclRow + (t & 1) * 16 * kSclRow + 4 * (sst + 1)];
        u32x4 xv[NT];  // next step's x tile, issued before the weights so waiting for it
        const int stn = min(st + 1, nsteps - 1);  // leaves the weight prefetch in flight
#pragma unroll
        for (int i = 0; i < NT; i++) xv[i] = ld16(b.x, xoff[i], 256 * stn);
        const u32x2 sv = ld8(xsr, soffx, 8 * stn);
        load_w(Stage<p ^ 1>(), stn);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the step's MFMAs
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            const int row = 16 * tt + li;
            const u32x4 b00 = xs[buf][lds_slot(row, g)], b01 = xs[buf][lds_slot(row, 4 + g)];
            const u32x4 b10 = xs[buf][lds_slot(row, 8 + g)], b11 = xs[buf][lds_slot(row, 12 + g)];
            const uint32_t sw = ((const uint16_t *)&xsc[buf][row])[g];
            // term 0 on the four weight tiles, then term 1: dependent MFMAs four apart
#pragma unroll
            for (int t = 0; t < 4; t++) acc[t][tt] = mfma_mx<0>(q[p][t], b00, b01, acc[t][tt], sc[t], sw);
            if constexpr (NTERM == 2) {
#pragma unroll
                for (int t = 0; t < 4; t++) acc[t][tt] = mfma_mx<1>(q[p][t], b10, b11, acc[t][tt], sc[t], sw);
            }
        }
        // the accumulators are pinned here: without it the compiler sinks the step's
        // MFMAs (pure operations) below the later steps and keeps all their operands live
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int tt = 0; tt < NT; tt++) asm volatile("" : "+v"(acc[t][tt]));
#pragma unroll
        for (int i = 0; i < NT; i++) xs[buf ^ 1][lds_slot(xr + 16 * i, xc)] = xv[i];
        if (sthr) xsc[buf ^ 1][tid] = sv;
        __syncthreads();
    });

    // the shared adapter's per-token terms for every tile of the lane, loaded together
    f32x4 lgv[NT][2], luv[NT][2];
    if (a.lora_gu) {
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
            const int tok = a.perm[r0 + tt0 + min(16 * tt + li, nt - 1)] / a.k;
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const float *p = a.lora_gu + (size_t)tok * 2 * I + b.c0 + 16 * t + 4 * g;
                const float4 dg = *(const float4 *)p, du = *(const float4 *)(p + I);
                lgv[tt][t] = f32x4{dg.x, dg.y, dg.z, dg.w};
                luv[tt][t] = f32x4{du.x, du.y, du.z, du.w};
            }
        }
    }
    // lane (g, li) holds I-columns c0 + 16 (t & 1) + 4 g + 0..3 of token 16 tt + li
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
        const int j = 16 * tt + li;
        if (j >= nt) continue;
        const size_t rr = (size_t)(r0 + tt0 + j);
#pragma unroll
        for (int t = 0; t < 2; t++) {
            f32x4 gv = acc[t][tt], uv = acc[t + 2][tt];
            const int n = b.c0 + 16 * t + 4 * g;
            if (a.lora_gu) {
                gv += lgv[tt][t];
                uv += luv[tt][t];
            }
            uint32_t hh[4], hl[4];
#pragma unroll
            for (int r = 0; r < 4; r++) split_bf16(act_h(a.act, gv[r], uv[r]), hh[r], hl[r]);
            *(u32x2 *)(a.h_hi + rr * I + n) = u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
            *(u32x2 *)(a.h_lo + rr * I + n) = u32x2{pack2(hl[0], hl[1]), pack2(hl[2], hl[3])};
            if (a.gu) {
                *(float4 *)(a.gu + (rr * 2 + 0) * I + n) = float4{gv[0], gv[1], gv[2], gv[3]};
                *(float4 *)(a.gu + (rr * 2 + 1) * I + n) = float4{uv[0], uv[1], uv[2], uv[3]};
            }
        }
    }
}

template <int NTERM>
__global__ __launch_bounds__(256, 2) void k_gateup_mx(const ExpertFwdArgs a)
{
    __shared__ MmTile xs[2];
    __shared__ MmScl xsc[2];
    __shared__ __attribute__((aligned(16))) uint8_t scl[256 * kSclRow];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int H = a.H, I = a.I;
    int ai, cb, r0, ntok;
    xcd_split(I / 128, ai, cb);
    if (!mm_tokens(a.tok_chunks, ai, a.n_active, a.active, a.offsets, r0, ntok)) return;
    const int e = a.active[ai];
    GuBlock b;
    const size_t eoc = (size_t)e * I * (H / 2), eos = (size_t)e * I * (H / 32);
    b.code[0] = buf_rsrc(a.gate.codes + eoc, I * (H / 2));
    b.code[1] = buf_rsrc(a.up.codes + eoc, I * (H / 2));
    b.scale[0] = buf_rsrc(a.gate.scales + eos, I * (H / 32));
    b.scale[1] = buf_rsrc(a.up.scales + eos, I * (H / 32));
    b.x = buf_rsrc(a.xq, (uint32_t)((size_t)a.T * H * 2));
    b.c0 = cb * 128 + wv * 32;
    b.coff = (uint32_t)(b.c0 + li) * (H / 2) + 16 * g;
    b.sblk = (uint32_t)cb * 128 * (H / 32);
    b.sl = (uint32_t)(wv * 32 + li) * kSclRow + g;
    for (int tt0 = 0; tt0 < ntok; tt0 += kMmTok) {
        const int nt = min(kMmTok, ntok - tt0);
        switch ((nt + 15) / 16) {
        case 1: gateup_pass_mx<1, NTERM>(a, b, xs, xsc, scl, r0, tt0, nt); break;
        case 2: gateup_pass_mx<2, NTERM>(a, b, xs, xsc, scl, r0, tt0, nt); break;
        case 3: gateup_pass_mx<3, NTERM>(a, b, xs, xsc, scl, r0, tt0, nt); break;
        case 4: gateup_pass_mx<4, NTERM>(a, b, xs, xsc, scl, r0, tt0, nt); break;
        case 5: gateup_pass_mx<5, NTERM>(a, b, xs, xsc, scl, r0, tt0, nt); break;
        default: gateup_pass_mx<6, NTERM>(a, b, xs, xsc, scl, r0, tt0, nt); break;
        }
    }
}

// ---------------------------------------------------------------- down + routing weight
//
// K-step 64 over I: lane group g owns reduction indices [16g, 16g + 16) of the step
// (half an MX scale block, 8 code bytes); sub-step s takes 16g + 8s + 0..7.  The LDS row
// of a token holds the step's 64 bf16 of h_hi (chunks 0..7) then of h_lo (chunks 8..15);
// h = h_hi + h_lo enters as two MFMAs per fragment.  Wave wv owns H-rows
// m0 = 256 rb + 64 wv .. +64 (tiles 0..3).

struct DnBlock {
    __amdgpu_buffer_rsrc_t code, scale;  // this expert's down matrix
    __amdgpu_buffer_rsrc_t h;            // h_hi then h_lo (contiguous planes)
    uint32_t coff;
    uint32_t sblk;  // the block's first scale row (byte offset)
    uint32_t sl;    // this lane's scale byte in LDS (tile 0, K-step 0)
    int m0;
};

constexpr int kDnSclSteps = kSclRow / 2;  // down K-steps per scale chunk (2 scale bytes a step)

__device__ __forceinline__ void dn_scl_next(uint8_t *scl, const DnBlock &b, int I, int st0, int nsteps)
{
    __syncthreads();  // every wave is past the previous chunk's last step
    scl_copy_serial(scl, 256, b.scale, b.sblk, I / 32, 2 * st0, 2 * min(kDnSclSteps, nsteps - st0));
    __syncthreads();
}

// hs0, hs1: the two h-tile buffers (separate LDS arrays, as for the gate/up's x tile).
template <int NT>
__device__ __forceinline__ void down_pass(const ExpertFwdArgs &a, const DnBlock &b, u32x4 *hs0, u32x4 *hs1,
                                          uint8_t *scl, int r0, int tt0, int nt)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, li = lane & 15;
    const int H = a.H, I = a.I, nsteps = I / 64;
    // The h tile goes straight from memory to LDS, as the gate/up's x tile: lane l of wave
    // wv, piece i, loads row 16 i + 4 wv + l / 16, chunk c = (l % 16) ^ (row % 16) (chunks
    // 0..7 from h_hi, 8..15 from h_lo).
    uint32_t hoff[NT];  // byte offsets at K-step 0
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int row = 16 * i + 4 * wv + (lane >> 4), chunk = (lane & 15) ^ (row & 15);
        const uint32_t plane = chunk < 8 ? 0u : (uint32_t)(a.h_lo - a.h_hi) * 2;
        hoff[i] = plane + ((uint32_t)(r0 + tt0 + min(row, nt - 1)) * I + 8 * (chunk & 7)) * 2;
    }
    auto load_h = [&](u32x4 *dst, int st) {
#pragma unroll
        for (int i = 0; i < NT; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                b.h, (__attribute__((address_space(3))) void *)((char *)dst + 1024 * (wv + 4 * i)), 16, hoff[i],
                128 * st, 0, 0);
    };
    f32x4 acc[4][NT];
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
        for (int tt = 0; tt < NT; tt++) acc[t][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x2 q[3][4];
    auto load_w = [&](auto P, int st) {
        constexpr int p = decltype(P)::value;
#pragma unroll
        for (int t = 0; t < 4; t++) q[p][t] = ld8(b.code, b.coff, t * 8 * I + 32 * st);
    };
    {
        u32x4 sv[scl_pieces<256>()];
        scl_load<256>(sv, b.scale, b.sblk, I / 32, 0, 2 * min(kDnSclSteps, nsteps));
        load_h(hs0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_w(Stage<0>(), 0);
        load_w(Stage<1>(), min(1, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);
        scl_store<256>(sv, scl, 2 * min(kDnSclSteps, nsteps));
        wait_vmcnt<8>();  // the h tile (issued before the eight weight loads)
    }
    __syncthreads();
    uint32_t scn[4];  // the scale bytes of the step, read from LDS one step ahead
#pragma unroll
    for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + t * 16 * kSclRow + 2 * 0];

    k_loop6(nsteps, [&](auto P6, int st) {
        constexpr int p = decltype(P6)::value % 3, parity = decltype(P6)::value & 1;
        u32x4 *const hcur = parity ? hs1 : hs0, *const hnxt = parity ? hs0 : hs1;
        const int sst = st % kDnSclSteps;
        if (sst == 0 && st != 0) {  // the next K chunk (I beyond 3584)
            dn_scl_next(scl, b, I, st, nsteps);
#pragma unroll
            for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + t * 16 * kSclRow + 2 * 0];
        }
        load_h(hnxt, min(st + 1, nsteps - 1));  // next step's h tile, before the weights
        __builtin_amdgcn_sched_barrier(0);
        load_w(Stage<(p + 2) % 3>(), min(st + 2, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the step's MFMAs
        float scale[4];
#pragma unroll
        for (int t = 0; t < 4; t++) scale[t] = e8m0_to_f32(scn[t]);
        if (sst + 1 < kDnSclSteps && st + 1 < nsteps)
#pragma unroll
            for (int t = 0; t < 4; t++) scn[t] = scl[b.sl + t * 16 * kSclRow + 2 * (sst + 1)];
#pragma unroll
        for (int s = 0; s < 2; s++) {
            bf16x8 A[4], Bh[NT], Bl[NT];
#pragma unroll
            for (int tt = 0; tt < NT; tt++) {
                Bh[tt] = as_bf16x8(hcur[lds_slot(16 * tt + li, 2 * g + s)]);
                Bl[tt] = as_bf16x8(hcur[lds_slot(16 * tt + li, 8 + 2 * g + s)]);
            }
#pragma unroll
            for (int t = 0; t < 4; t++) A[t] = fp4x8_to_bf16(q[p][t][s], scale[t]);
#pragma unroll
            for (int tt = 0; tt < NT; tt++)
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    acc[t][tt] = mfma16(A[t], Bh[tt], acc[t][tt]);
                    acc[t][tt] = mfma16(A[t], Bl[tt], acc[t][tt]);
                }
        }
        wait_vmcnt<4>();  // this thread's part of the next h tile (the 4 weight loads came after)
        __syncthreads();
    });

    // lane (g, li) holds H-rows m0 + 16 t + 4 g + 0..3 of token 16 tt + li
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
        const int j = 16 * tt + li;
        if (j >= nt) continue;
        const int slot = a.perm[r0 + tt0 + j];
        const float p = a.w[slot];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const f32x4 v = acc[t][tt];
            *(float4 *)(a.ybuf + (size_t)slot * H + b.m0 + 16 * t + 4 * g) =
                float4{p * v[0], p * v[1], p * v[2], p * v[3]};
        }
    }
}

__global__ __launch_bounds__(256, 2) void k_down_mm(const ExpertFwdArgs a)
{
    __shared__ MmTile hs0, hs1;
    __shared__ __attribute__((aligned(16))) uint8_t scl[256 * kSclRow];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int H = a.H, I = a.I;
    int ai, rb, r0, ntok;
    xcd_split(H / 256, ai, rb);
    if (!mm_tokens(a.tok_chunks, ai, a.n_active, a.active, a.offsets, r0, ntok)) return;
    const int e = a.active[ai];
    DnBlock b;
    b.code = buf_rsrc(a.down.codes + (size_t)e * H * (I / 2), H * (I / 2));
    b.scale = buf_rsrc(a.down.scales + (size_t)e * H * (I / 32), H * (I / 32));
    b.h = buf_rsrc(a.h_hi, (uint32_t)((size_t)a.T * a.k * I * 4));
    b.m0 = rb * 256 + wv * 64;
    b.coff = (uint32_t)(b.m0 + li) * (I / 2) + 8 * g;
    b.sblk = (uint32_t)rb * 256 * (I / 32);
    b.sl = (uint32_t)(wv * 64 + li) * kSclRow + (g >> 1);
    for (int tt0 = 0; tt0 < ntok; tt0 += kMmTok) {
        const int nt = min(kMmTok, ntok - tt0);
        switch ((nt + 15) / 16) {
        case 1: down_pass<1>(a, b, hs0, hs1, scl, r0, tt0, nt); break;
        case 2: down_pass<2>(a, b, hs0, hs1, scl, r0, tt0, nt); break;
        case 3: down_pass<3>(a, b, hs0, hs1, scl, r0, tt0, nt); break;
        case 4: down_pass<4>(a, b, hs0, hs1, scl, r0, tt0, nt); break;
        case 5: down_pass<5>(a, b, hs0, hs1, scl, r0, tt0, nt); break;
        default: down_pass<6>(a, b, hs0, hs1, scl, r0, tt0, nt); break;
        }
    }
}

// Buffer offsets are 32-bit: x, the two h planes and one expert matrix must each span
// less than 4 GiB, and h_lo must follow h_hi directly.
bool mm_supported(const ExpertFwdArgs &a)
{
    const size_t S = (size_t)a.T * a.k, lim = (size_t)1 << 32;
    return a.wfmt == FMT_MXFP4 && a.xt == DT_BF16 && a.H % 512 == 0 && a.I % 512 == 0 &&
           (size_t)a.T * a.H * 2 < lim && S * a.I * 4 < lim && (size_t)a.H * a.I < lim &&
           a.h_lo == a.h_hi + S * a.I && (!a.xq || a.xq_s);
}

hipError_t launch_gateup_mm(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = mm_units(a);
    if (!a.xq) {
        ProfScope ps(a.prof, PK_GATEUP, s);
        ps.launch(k_gateup_mm, dim3(xcd_grid(maxU, a.I / 128)), dim3(256), 0, a);
        return hipGetLastError();
    }
    if (a.xq_single) {
        // x arrived MXFP8-quantized: its one E4M3 term is already in place
        ProfScope ps(a.prof, PK_GATEUP, s);
        ps.launch(k_gateup_mx<1>, dim3(xcd_grid(maxU, a.I / 128)), dim3(256), 0, a);
        return hipGetLastError();
    }
    {
        ProfScope ps(a.prof, PK_XTERMS, s);
        const size_t n = (size_t)a.T * (a.H / 32);
        ps.launch(k_x_terms, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (const uint16_t *)a.x, a.T, a.H, a.xq,
                  a.xq_s);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ProfScope ps(a.prof, PK_GATEUP, s);
    ps.launch(k_gateup_mx<2>, dim3(xcd_grid(maxU, a.I / 128)), dim3(256), 0, a);
    return hipGetLastError();
}

hipError_t launch_down_mm(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = mm_units(a);
    ProfScope ps(a.prof, PK_DOWN, s);
    ps.launch(k_down_mm, dim3(xcd_grid(maxU, a.H / 256)), dim3(256), 0, a);
    return hipGetLastError();
}

}  // namespace moe
