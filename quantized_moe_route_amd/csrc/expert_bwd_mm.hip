// expert_bwd_mm.hip -- grouped-GEMM input gradient for experts holding many tokens (MXFP4).
//
// The two transposed products of the expert backward (LazyLoRA README, "Routed experts":
// the experts are streamed again in the backward to form the gradient with respect to
// the latent input; "File map": the native kernel supplies the transposed product):
//   k_bwd_down_mm    a = Wd^T dy per slot, then the activation backward;
//   k_bwd_gateup_mm  dxs = Wg^T dg + Wu^T du per slot.
// Both have the form out[m][token] = sum_k W[k][m] B[token][k] with the stored matrix
// W [K rows][M cols] packed along M, so the MX block scales run along M and the reduction
// runs along the rows.  A block owns one expert, 256 output columns m (64 per wave, four
// 16-wide MFMA tiles) and all of the expert's tokens (passes of up to 96):
//  - per 32-row sub-step, each thread dequantizes one 32-element piece of a W row (one
//    scale) exactly to bf16 and writes it to an LDS tile in natural [k][m] order;
//  - the MFMA A operand (16 m x 32 k) is read from that tile transposed with two
//    ds_read_b64_tr_b16: within a 16-lane group, result lane q gets, as value j, element
//    q % 4 of the 4-element row segment addressed by lane q / 4 + 4 j;
//  - the B operand (token rows, bf16) is staged in LDS per chunk of 128 k, shared by the
//    four waves; for dg/du it arrives as bf16 hi + lo planes (two MFMAs per fragment);
//  - raw weight bytes stream into registers two chunks ahead through buffer loads.
#include <type_traits>

#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kBtTok = 96;     // tokens per pass
constexpr int kWRow = 272;     // bf16 per LDS row of the W sub-step tile (256 + 16 pad)

template <int P>
using Stage = std::integral_constant<int, P>;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ void xcd_split(int nb, int &ai, int &cb)
{
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int q = j / nb;
    cb = j - q * nb;
    ai = 8 * q + x;
}

inline int xcd_grid(int maxU, int nb) { return 8 * ((maxU + 7) / 8) * nb; }

static_assert(kBtTok == kTokChunk, "token chunks are one pass");

// As in the forward grouped GEMM: work unit ai is an active expert, or with tok_chunks one
// chunk of kTokChunk tokens of expert ai / tok_chunks.
__device__ __forceinline__ bool bt_tokens(int tok_chunks, int &ai, const int32_t *n_active, const int32_t *active,
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

inline int bt_units(const ExpertBwdArgs &a) { return a.tok_chunks > 0 ? a.E * a.tok_chunks : min(a.E, a.T * a.k); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ uint32_t ld1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// Element offset of W-tile entry (row, m).  Rows 8..15 and 24..31 are stored with m
// flipped by 64, so the 16 rows one transposed read touches fall into distinct banks; the
// upper half of a row (m >= 128) sits 8 elements further on, so the 16-byte stores of a
// quarter wave (two rows, m = 32 j + 8 v for j = 0..7) fall into 16 distinct bank groups
// instead of pairing j with j + 4.  A transposed read stays within one half.
__device__ __forceinline__ int wt_pos(int row, int m)
{
    const int mm = m ^ (((row >> 3) & 1) << 6);
    return row * kWRow + mm + ((mm >> 7) << 3);
}

// B tile: [96 rows][16 chunks of 16 bytes], chunk c of row r in slot c ^ (r & 15).
__device__ __forceinline__ int bt_slot(int row, int c) { return row * 16 + (c ^ (row & 15)); }

template <typename F>
__device__ __forceinline__ void chunk_loop3(int n, F &&step)
{
    int c0 = 0;
    for (; c0 + 3 <= n; c0 += 3) {
        step(Stage<0>(), c0);
        step(Stage<1>(), c0 + 1);
        step(Stage<2>(), c0 + 2);
    }
    if (c0 < n) step(Stage<0>(), c0);
    if (c0 + 1 < n) step(Stage<1>(), c0 + 1);
}

// Per-block constants.  GU = false: the down matrix (K = H rows of Wd viewed as k, M = I);
// GU = true: gate then up (K = 2I, M = H).
struct BtBlock {
    __amdgpu_buffer_rsrc_t wc[2], ws[2];  // codes / scales of the (one or two) matrices
    __amdgpu_buffer_rsrc_t bsrc;          // B rows: dy (down) or the dg/du hi+lo planes (gate/up)
    uint32_t wvoff, svoff;                // this thread's piece offsets at row 0 of a matrix
    int mb0;                              // first output column of the block
    int M, K, krows;                      // output width, reduction length, rows per matrix
};

// One pass over up to 96 tokens of the block's expert: acc[t][tt] = out[m][token] for
// m = mb0 + 64 wv + 16 t + 4 g + r, token 16 tt + li.
template <int NT, bool GU>
__device__ __forceinline__ void bwdt_mma(const ExpertBwdArgs &a, const BtBlock &b, uint16_t (*wt)[32 * kWRow],
                                         u32x4 *bt, int r0, int tt0, int nt, f32x4 (&acc)[4][NT])
{
    constexpr int SUB = GU ? 2 : 4;  // 32-row sub-steps per chunk; B row = SUB * planes * 64 B = 256 B
    constexpr int CK = 32 * SUB;     // rows per chunk
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, li = lane & 15;
    const int nchunks = b.K / CK;
    const int br = tid >> 4, bc = tid & 15;  // this thread's B-tile row (+16 i) and chunk

    // B source offsets (bytes) of this thread's rows at chunk 0
    uint32_t boff[NT];
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int j = min(br + 16 * i, nt - 1);
        if constexpr (GU) {
            // chunk bc = (sub * 2 + plane) * 4 + g8 -> k = 32 sub + 8 g8 of plane
            const uint32_t plane = (bc >> 2) & 1, sub = bc >> 3, g8 = bc & 3;
            const uint32_t pl_bytes = (uint32_t)((size_t)a.T * a.k * 2 * a.I * 2);
            boff[i] = plane * pl_bytes + ((uint32_t)(r0 + tt0 + j) * (2 * a.I) + 32 * sub + 8 * g8) * 2;
        } else {
            const int tok = a.perm[r0 + tt0 + j] / a.k;
            boff[i] = ((uint32_t)tok * a.H + 8 * bc) * 2;
        }
    }
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
        for (int tt = 0; tt < NT; tt++) acc[t][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 q[3][SUB];
    uint32_t sc[3][SUB];
    // raw pieces of chunk c: row c * CK + 32 s + tid / 8 of matrix (c * CK) / krows
    auto load_w = [&](auto P, int c) {
        constexpr int p = decltype(P)::value;
        const int k0 = c * CK;
        const int mat = GU ? (k0 >= b.krows) : 0;
        const int kr = k0 - mat * b.krows;
#pragma unroll
        for (int s = 0; s < SUB; s++) {
            q[p][s] = ld16(b.wc[mat], b.wvoff, (uint32_t)(kr + 32 * s) * (b.M / 2));
            sc[p][s] = ld1(b.ws[mat], b.svoff, (uint32_t)(kr + 32 * s) * (b.M / 32));
        }
    };
    auto load_b = [&](u32x4 (&v)[NT], int c) {
#pragma unroll
        for (int i = 0; i < NT; i++) v[i] = ld16(b.bsrc, boff[i], (uint32_t)c * (GU ? 128 : 256));
    };
    auto store_b = [&](const u32x4 (&v)[NT]) {
#pragma unroll
        for (int i = 0; i < NT; i++) bt[bt_slot(br + 16 * i, bc)] = v[i];
    };
    // decode raw piece w (one scale) into W-tile buffer wbuf: row tid / 8, m 32 (tid % 8) ..
    auto put_w = [&](uint16_t *wbuf, u32x4 w, uint32_t sbyte) {
        uint32_t d[16];
        decode_fp4x32(w, e8m0_to_f32(sbyte), d);
        const int row = tid >> 3, m = 32 * (tid & 7);
        u32x4 *dst = (u32x4 *)(wbuf + wt_pos(row, m));
#pragma unroll
        for (int v = 0; v < 4; v++) dst[v] = u32x4{d[4 * v], d[4 * v + 1], d[4 * v + 2], d[4 * v + 3]};
    };

    {
        u32x4 yv[NT];
        load_b(yv, 0);
        load_w(Stage<0>(), 0);
        load_w(Stage<1>(), min(1, nchunks - 1));
        store_b(yv);
        put_w(wt[0], q[0][0], sc[0][0]);
    }
    __syncthreads();

    // transposed-read addresses (element offsets within a W tile) of this lane, per A tile
    const int qr = li >> 2, qa = li & 3;
    chunk_loop3(nchunks, [&](auto P, int c) {
        constexpr int p = decltype(P)::value;
        u32x4 yv[NT];
        load_b(yv, min(c + 1, nchunks - 1));
        load_w(Stage<(p + 2) % 3>(), min(c + 2, nchunks - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < SUB; s++) {
            const uint16_t *wb = wt[s & 1];
            bf16x8 A[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int m = 64 * wv + 16 * t + 4 * qa;
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(wb + wt_pos(8 * g + qr, m)));
                const v4i16 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(wb + wt_pos(8 * g + 4 + qr, m)));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                A[t] = as_bf16x8(l2[0], l2[1], h2[0], h2[1]);
            }
#pragma unroll
            for (int tt = 0; tt < NT; tt++) {
                const int row = 16 * tt + li;
                if constexpr (GU) {
                    const bf16x8 Bh = as_bf16x8(bt[bt_slot(row, (2 * s) * 4 + g)]);
                    const bf16x8 Bl = as_bf16x8(bt[bt_slot(row, (2 * s + 1) * 4 + g)]);
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        acc[t][tt] = mfma16(A[t], Bh, acc[t][tt]);
                        acc[t][tt] = mfma16(A[t], Bl, acc[t][tt]);
                    }
                } else {
                    const bf16x8 B = as_bf16x8(bt[bt_slot(row, 4 * s + g)]);
#pragma unroll
                    for (int t = 0; t < 4; t++) acc[t][tt] = mfma16(A[t], B, acc[t][tt]);
                }
            }
            // next sub-step's W tile into the other buffer
            if (s + 1 < SUB)
                put_w(wt[(s + 1) & 1], q[p][s + 1], sc[p][s + 1]);
            else
                put_w(wt[0], q[(p + 1) % 3][0], sc[(p + 1) % 3][0]);
            if (s + 1 == SUB) {
                __syncthreads();  // every wave is done with this chunk's B tile
                store_b(yv);
            }
            __syncthreads();
        }
    });
}

// ---------------------------------------------------------------- kernels

template <int NT>
__device__ __forceinline__ void bwd_down_pass(const ExpertBwdArgs &a, const BtBlock &b, uint16_t (*wt)[32 * kWRow],
                                              u32x4 *bt, int r0, int tt0, int nt)
{
    f32x4 acc[4][NT];
    bwdt_mma<NT, false>(a, b, wt, bt, r0, tt0, nt, acc);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int I = a.I, ntiles = dp_tiles(I);
    const size_t S = (size_t)a.T * a.k;
    uint16_t *dg_hi = (uint16_t *)a.dgdu, *dg_lo = dg_hi + S * 2 * I;
    const int mw = b.mb0 + 64 * wv;
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
        const int j = 16 * tt + li;
        const bool ok = j < nt;
        const size_t rr = (size_t)(r0 + tt0 + min(j, nt - 1));
        const float p = a.w[a.perm[rr]];
        // the shared adapter's per-token term of Wd^T dy (null: none)
        const float *lc = a.lora_c ? a.lora_c + (size_t)(a.perm[rr] / a.k) * I : nullptr;
        float dpp = 0.f;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int m = mw + 16 * t + 4 * g;
            const float4 gv = *(const float4 *)(a.gu + (rr * 2) * I + m);
            const float4 uv = *(const float4 *)(a.gu + (rr * 2 + 1) * I + m);
            const float gg[4] = {gv.x, gv.y, gv.z, gv.w}, uu[4] = {uv.x, uv.y, uv.z, uv.w};
            uint32_t dh_[4], dl_[4], uh_[4], ul_[4];
            const float4 cv = lc ? *(const float4 *)(lc + m) : float4{0.f, 0.f, 0.f, 0.f};
            const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float av = acc[t][tt][r] + cc[r];
                float hv, dhdg, dhdu;
                act_grad(a.act, gg[r], uu[r], hv, dhdg, dhdu);
                dpp += av * hv;
                const float dh = p * av;
                split_bf16(dh * dhdg, dh_[r], dl_[r]);
                split_bf16(dh * dhdu, uh_[r], ul_[r]);
            }
            if (ok) {
                const size_t o = rr * 2 * I + m;
                *(u32x2 *)(dg_hi + o) = u32x2{pack2(dh_[0], dh_[1]), pack2(dh_[2], dh_[3])};
                *(u32x2 *)(dg_lo + o) = u32x2{pack2(dl_[0], dl_[1]), pack2(dl_[2], dl_[3])};
                *(u32x2 *)(dg_hi + o + I) = u32x2{pack2(uh_[0], uh_[1]), pack2(uh_[2], uh_[3])};
                *(u32x2 *)(dg_lo + o + I) = u32x2{pack2(ul_[0], ul_[1]), pack2(ul_[2], ul_[3])};
            }
        }
        dpp += __shfl_xor(dpp, 16, 64);
        dpp += __shfl_xor(dpp, 32, 64);
        if (ok && g == 0) a.dp_part[rr * ntiles + mw / 64] = dpp;
    }
}

template <int NT>
__device__ __forceinline__ void bwd_gateup_pass(const ExpertBwdArgs &a, const BtBlock &b,
                                                uint16_t (*wt)[32 * kWRow], u32x4 *bt, int r0, int tt0, int nt)
{
    f32x4 acc[4][NT];
    bwdt_mma<NT, true>(a, b, wt, bt, r0, tt0, nt, acc);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
    const int mw = b.mb0 + 64 * wv;
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
        const int j = 16 * tt + li;
        if (j >= nt) continue;
        const int slot = a.perm[r0 + tt0 + j];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const f32x4 v = acc[t][tt];
            *(float4 *)(a.dxs + (size_t)slot * a.H + mw + 16 * t + 4 * g) = float4{v[0], v[1], v[2], v[3]};
        }
    }
}

template <bool GU>
__global__ __launch_bounds__(256, 2) void k_bwdt_mm(const ExpertBwdArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t wt[2][32 * kWRow];
    __shared__ u32x4 bt[kBtTok * 16];
    const int tid = threadIdx.x;
    const int H = a.H, I = a.I;
    const int M = GU ? H : I;
    int ai, cb, r0, ntok;
    xcd_split(M / 256, ai, cb);
    if (!bt_tokens(a.tok_chunks, ai, a.n_active, a.active, a.offsets, r0, ntok)) return;
    const int e = a.active[ai];
    BtBlock b;
    b.M = M;
    b.mb0 = cb * 256;
    if constexpr (GU) {
        b.K = 2 * I;
        b.krows = I;
        const size_t oc = (size_t)e * I * (H / 2), os = (size_t)e * I * (H / 32);
        b.wc[0] = buf_rsrc(a.gate.codes + oc, I * (H / 2));
        b.wc[1] = buf_rsrc(a.up.codes + oc, I * (H / 2));
        b.ws[0] = buf_rsrc(a.gate.scales + os, I * (H / 32));
        b.ws[1] = buf_rsrc(a.up.scales + os, I * (H / 32));
        b.bsrc = buf_rsrc(a.dgdu, (uint32_t)((size_t)a.T * a.k * 2 * I * 2 * 2));
    } else {
        b.K = H;
        b.krows = H;
        const size_t oc = (size_t)e * H * (I / 2), os = (size_t)e * H * (I / 32);
        b.wc[0] = b.wc[1] = buf_rsrc(a.down.codes + oc, H * (I / 2));
        b.ws[0] = b.ws[1] = buf_rsrc(a.down.scales + os, H * (I / 32));
        b.bsrc = buf_rsrc(a.dy, (uint32_t)((size_t)a.T * H * 2));
    }
    b.wvoff = (uint32_t)(tid >> 3) * (M / 2) + (b.mb0 + 32 * (tid & 7)) / 2;
    b.svoff = (uint32_t)(tid >> 3) * (M / 32) + (b.mb0 + 32 * (tid & 7)) / 32;
    for (int tt0 = 0; tt0 < ntok; tt0 += kBtTok) {
        const int nt = min(kBtTok, ntok - tt0);
        if constexpr (GU) {
            switch ((nt + 15) / 16) {
            case 1: bwd_gateup_pass<1>(a, b, wt, bt, r0, tt0, nt); break;
            case 2: bwd_gateup_pass<2>(a, b, wt, bt, r0, tt0, nt); break;
            case 3: bwd_gateup_pass<3>(a, b, wt, bt, r0, tt0, nt); break;
            case 4: bwd_gateup_pass<4>(a, b, wt, bt, r0, tt0, nt); break;
            case 5: bwd_gateup_pass<5>(a, b, wt, bt, r0, tt0, nt); break;
            default: bwd_gateup_pass<6>(a, b, wt, bt, r0, tt0, nt); break;
            }
        } else {
            switch ((nt + 15) / 16) {
            case 1: bwd_down_pass<1>(a, b, wt, bt, r0, tt0, nt); break;
            case 2: bwd_down_pass<2>(a, b, wt, bt, r0, tt0, nt); break;
            case 3: bwd_down_pass<3>(a, b, wt, bt, r0, tt0, nt); break;
            case 4: bwd_down_pass<4>(a, b, wt, bt, r0, tt0, nt); break;
            case 5: bwd_down_pass<5>(a, b, wt, bt, r0, tt0, nt); break;
            default: bwd_down_pass<6>(a, b, wt, bt, r0, tt0, nt); break;
            }
        }
        __syncthreads();  // the next pass restages both tiles
    }
}

}  // namespace

// MXFP4, bf16 dy, H and I multiples of 512, 32-bit buffer offsets (see mm_supported).
bool bwd_mm_supported(const ExpertBwdArgs &a)
{
    const size_t S = (size_t)a.T * a.k, lim = (size_t)1 << 32;
    return a.wfmt == FMT_MXFP4 && a.dyt == DT_BF16 && a.H % 512 == 0 && a.I % 512 == 0 &&
           (size_t)a.T * a.H * 2 < lim && S * 2 * a.I * 2 * 2 < lim && (size_t)a.H * a.I < lim;
}

hipError_t launch_bwd_down_mm(const ExpertBwdArgs &a, hipStream_t s)
{
    const int maxU = bt_units(a);
    ProfScope ps(a.prof, PK_BWD_DOWN, s);
    ps.launch(k_bwdt_mm<false>, dim3(xcd_grid(maxU, a.I / 256)), dim3(256), 0, a);
    return hipGetLastError();
}

hipError_t launch_bwd_gateup_mm(const ExpertBwdArgs &a, hipStream_t s)
{
    const int maxU = bt_units(a);
    ProfScope ps(a.prof, PK_BWD_GATEUP, s);
    ps.launch(k_bwdt_mm<true>, dim3(xcd_grid(maxU, a.H / 256)), dim3(256), 0, a);
    return hipGetLastError();
}

}  // namespace moe
