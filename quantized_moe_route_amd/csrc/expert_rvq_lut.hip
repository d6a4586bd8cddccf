// expert_rvq_lut.hip -- few-token RVQ3 expert forward as table lookups.
//
// WASTE README, "3 bits per expert weight": a weight vector (8 consecutive inputs of one
// row) is C1[i1] + C2[i2] + C3[i3], three stages of 256-entry fp16 codebooks.  For a token
// x the product of a row with x is therefore
//     sum over stages s and vectors v of  L_s[v][i_s(row, v)],   L_s[v][c] = C_s[c] . x_v,
// a sum of table entries: every codeword's dot product with every 8-slice of x is formed
// once per token and shared by all rows of the matrix, so per index byte the kernel does one
// 4-byte LDS lookup and one add instead of gathering a 16-byte codeword (the gather kernels
// of expert_rvq.hip are bound by the bank conflicts of those gathers when experts hold one
// token, and read each row's index bytes 32 at a time).
//
// Block = 1024 threads, one matrix of one unit, NS x 128 rows, up to two tokens (gate/up) or
// one token (down) per pass, the index bytes read once per pass.  Rows are
// worked by teams of 8 lanes: for each stage s and group of 128 vectors (one 128-byte line of
// a row's index bytes) the 8 lanes of a team load the line together, 16 bytes each, so one
// wave-wide load covers 8 whole lines (reading a row 64 or 32 bytes at a time, strided by the
// row length, gets markedly less of the HBM rate).  Each team owns NS rows (slots); lane k
// of a team looks up vectors 16k .. 16k + 15 of each of its rows, and the 8 partial sums of
// a row are added across the team at the end.  Per (stage, group):
//  - table L[c][v] (256 codewords x 128 vectors, fp32, 128 KB of LDS: vectors v < 64 and
//    v >= 64 in two 64 KB halves, entry (c, v) at byte (v / 64) * 64 KB + 256 c + 4 (v mod
//    64)), formed by v_mfma_f32_32x32x8_f16: the 32 x 8 block of codewords times the 8 x 32
//    block of token slices is a 32 x 32 tile of the table (fp16 products are exact, sums in
//    fp32).  The token enters as fp16 times a power of two that puts its maximum magnitude
//    in [2^13, 2^14), so bf16 tokens are exact; fp32 h for the down product as two fp16
//    terms hi + lo, both in one v_mfma_f32_32x32x16_f16 (reduction length 16: the codeword
//    against each term);
//  - lookups: lane (team j of its half-wave, k) takes at step i vector 16k + (i xor r) with
//    r = 4j + k / 2, so at every step the 32 lanes of a half-wave read 32 distinct banks.
//    Its 16 index bytes per row have their dwords permuted by r / 4 once; the table address
//    is one v_perm_b32 per lookup: byte 1 is the index byte (picked by a per-lane selector
//    that applies r mod 4), bytes 0 and 2 come from the step's offset.
// Index bytes of the next (stage, group) are loaded while the current one is looked up.
// The launches are persistent, one block per CU: work items (a unit's row block of one
// matrix, all of the unit's tokens) are handed out by an atomic counter, units with the most
// tokens first, so the long items start early and the CUs run out of work together (blocks
// that dispatch in a fixed order to the XCDs left about a sixth of the CU time idle).  A
// one-block launch before them sorts the active units by token count into a shared order
// and zeroes the counters.  The order decides only which block computes an item, not any
// arithmetic, so results do not depend on it.
#include "common.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kLutThreads = 1024;
constexpr int kTeams = kLutThreads / 8;   // teams of 8 lanes, one row per slot
constexpr int kGV = 128;                  // vectors per table group
constexpr int kHalfBytes = 65536;         // table half: 256 codewords x 64 vectors
constexpr int kLutBytes = 2 * kHalfBytes;
constexpr int kCbBytes = 3 * 256 * 16;    // 12 KB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t lrsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

// Exponent se with m * 2^-se in [2^13, 2^14) (0 for an all-zero row).
__device__ __forceinline__ int lut_scale_exp(float m)
{
    if (!(m > 0.f)) return 0;
    int e;
    frexpf(m, &e);
    return e - 14;
}

__device__ __forceinline__ uint32_t pack_h2f(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// v_perm_b32 selectors: all four bytes of the first operand, or of the second
constexpr uint32_t kPermHi = 0x07060504u, kPermLo = 0x03020100u;

// Permute the dwords of w[0..3]: afterwards w[d] is the former w[d xor q] (0 <= q < 4).  Two
// conditional swaps, one v_perm_b32 per dword each.
__device__ __forceinline__ void xor_dwords(uint32_t (&w)[4], int q)
{
    uint32_t t[4];
#pragma unroll
    for (int k = 0; k < 4; k++) t[k] = __builtin_amdgcn_perm(w[k ^ 1], w[k], (q & 1) ? kPermHi : kPermLo);
#pragma unroll
    for (int k = 0; k < 4; k++) w[k] = __builtin_amdgcn_perm(t[k ^ 2], t[k], (q & 2) ? kPermHi : kPermLo);
}

// Block-wide maximum of v (1024 threads; red: 16 floats of LDS).
__device__ __forceinline__ float block_max(float v, float *red)
{
    const float w = wave_max_f32(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kLutThreads / 64; i++) m = fmaxf(m, red[i]);
    __syncthreads();
    return m;
}

// Per-thread geometry of one block.
struct LutGeom {
    int V, s0, ng, nstep;  // index bytes per row and stage; window g covers vectors 128 g - s0
                           // .. 128 g - s0 + 127 (clipped to the row); windows; steps
    uint32_t plane;        // bytes per stage plane
    int k, r;              // lane in team, lookup order (position 16k + (i xor r) at step i)
};

// Rows fall into P = 128 / gcd(V, 128) phases by where they start within a 128-byte line
// (row r starts at byte r V of its plane); a block takes rows of one phase c, r = c mod P,
// and shifts its table windows by s0 = c V mod 128 vectors so that every window of every
// row is whole 128-byte lines (a window that straddled two lines would read each of them
// half, a step apart, and the other half often after the L2 has dropped the line).
__device__ __host__ __forceinline__ int lut_phases(int V)
{
    int p = 128;
    while (p > 1 && V % (128 / p * 2) == 0) p >>= 1;
    return p;
}

// This thread's 16 index bytes of each slot's row for stage-group step st.  The whole offset
// within the unit's index bytes is in the per-lane operand, which is all the buffer range
// check sees: lanes past the group's last vector and slots past the matrix's last row take
// offset 2^31, past the range (index planes are below 2^31 bytes), and read zeros without
// touching memory.
template <int NS>
__device__ __forceinline__ void load_idx(uint32_t (&dst)[NS][4], __amdgpu_buffer_rsrc_t ir, const LutGeom &G, int P,
                                         uint32_t rowoff, uint32_t slot_ok, int st)
{
    const int s = st / G.ng, g = st - s * G.ng;
    const int v0 = kGV * g - G.s0 + 16 * G.k;  // this lane's first vector
    const bool lane_ok = v0 >= 0 && v0 + 16 <= G.V;
    const uint32_t off = (uint32_t)s * G.plane + rowoff + (uint32_t)v0;
    const uint32_t slot_stride = (uint32_t)(kTeams * P) * (uint32_t)G.V;
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const uint32_t o = lane_ok && ((slot_ok >> j) & 1u) ? off + j * slot_stride : 0x80000000u;
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(ir, (int)o, 0, 0);
        dst[j][0] = a[0]; dst[j][1] = a[1]; dst[j][2] = a[2]; dst[j][3] = a[3];
    }
}

// Build the table of stage s for the window starting at vector w0, positions plo .. phi - 1
// (those inside the row), for one token (xs: its NTERM fp16 planes [NTERM][K]): 32 tiles
// of 32 codewords x 32 positions, two per wave; lane supplies codeword / position lane mod
// 32, dimensions 4 (lane / 32) .. + 3, and gets back rows 8 (i / 4) + 4 (lane / 32) + i mod 4
// of the tile's column lane mod 32.
template <int NTERM>
__device__ __forceinline__ void build_table(int s, int w0, int plo, int phi, int K, const _Float16 *xs,
                                            const _Float16 *cbl, char *lut)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll 1
    for (int h = 0; h < 2; h++) {
        const int t = wv + 16 * h, ct = t & 7, vt = t >> 3;
        if (32 * vt < plo || 32 * vt + 32 > phi) continue;
        const int hl = lane >> 5, li = lane & 31;
        f32x16 d = {};
        if constexpr (NTERM == 2) {
            // both terms in one product of reduction length 16: lanes 0..31 pair the codeword
            // with the hi plane, lanes 32..63 with the lo plane (A and B share the lane-to-
            // reduction-index map, so the sum is C . hi + C . lo whatever that map is)
            const h8v A = *(const h8v *)(cbl + (size_t)(256 * s + 32 * ct + li) * 8);
            const h8v B = *(const h8v *)(xs + (size_t)hl * K + 8 * (w0 + 32 * vt + li));
            d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B, d, 0, 0, 0);
        } else {
            const h4v A = *(const h4v *)(cbl + (size_t)(256 * s + 32 * ct + li) * 8 + 4 * hl);
            const h4v B = *(const h4v *)(xs + 8 * (w0 + 32 * vt + li) + 4 * hl);
            d = __builtin_amdgcn_mfma_f32_32x32x8f16(A, B, d, 0, 0, 0);
        }
        const int v = 32 * vt + li;
        char *dst = lut + (v >> 6) * kHalfBytes + 4 * (v & 63) + 256 * (32 * ct + 4 * hl);
#pragma unroll
        for (int i = 0; i < 16; i++) *(float *)(dst + 256 * (8 * (i >> 2) + (i & 3))) = d[i];
    }
}

// Add to acc the table entries picked by the slots' index bytes (already permuted by
// r / 4).  Step i takes vector v = 16k + (i xor r) at byte (v / 64) * 64 KB + 256 c +
// 4 (v mod 64), whose bytes 0 and 2 are those of toff = tb xor 4i (the base and the selectors
// are opaque copies, so that they stay five registers and the per-step offsets are one xor
// each); the lookups of step i + 1 are issued before the adds of step i.
template <int NS>
__device__ __forceinline__ void lookups(const uint32_t (&idx)[NS][4], float (&acc)[NS], const LutGeom &G,
                                        const char *lb)
{
    uint32_t tb = ((uint32_t)(G.k >> 2) << 16) | (64u * (uint32_t)(G.k & 3) + 4u * (uint32_t)G.r);
    uint32_t sel[4];
#pragma unroll
    for (int m = 0; m < 4; m++) sel[m] = 0x0C020000u | ((uint32_t)(4 + (m ^ (G.r & 3))) << 8);
    asm volatile("" : "+v"(tb), "+v"(sel[0]), "+v"(sel[1]), "+v"(sel[2]), "+v"(sel[3]));
    float cur[NS], nxt[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) cur[j] = *(const float *)(lb + __builtin_amdgcn_perm(idx[j][0], tb, sel[0]));
#pragma unroll
    for (int i = 0; i < 16; i++) {
        if (i + 1 < 16) {
            const int n = i + 1;
            const uint32_t toff = tb ^ (4u * n);
#pragma unroll
            for (int j = 0; j < NS; j++) nxt[j] = *(const float *)(lb + __builtin_amdgcn_perm(idx[j][n >> 2], toff, sel[n & 3]));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; j++) acc[j] += cur[j];
#pragma unroll
        for (int j = 0; j < NS; j++) cur[j] = nxt[j];
    }
}

// Stage-group step st for nt <= NT tokens (xs: [NT][NTERM][K]): per token, build the table,
// then add the entries picked by the slots' index bytes (idx, permuted in place once) to
// that token's acc.
template <int NS, int NTERM, int NT>
__device__ __forceinline__ void lut_step(uint32_t (&idx)[NS][4], float (&acc)[NT][NS], const LutGeom &G, int st, int K,
                                         int nt, const _Float16 *xs, const _Float16 *cbl, char *lut)
{
    const int s = st / G.ng, g = st - s * G.ng;
    const int w0 = kGV * g - G.s0;                                     // the window's first vector
    const int plo = max(0, -w0), phi = min(kGV, G.V - w0);             // positions inside the row
    const bool active = 16 * G.k >= plo && 16 * G.k + 16 <= phi;       // (multiples of 32)
#pragma unroll
    for (int t = 0; t < NT; t++) {
        if (t > 0 && t >= nt) break;
        __syncthreads();  // the previous lookups are done
        build_table<NTERM>(s, w0, plo, phi, K, xs + (size_t)t * NTERM * K, cbl, lut);
        __syncthreads();
        if (active) {
            if (t == 0) {
#pragma unroll
                for (int j = 0; j < NS; j++) xor_dwords(idx[j], G.r >> 2);
            }
            lookups<NS>(idx, acc[t], G, lut);
        }
    }
}

// One matrix of one unit for nt <= NT tokens, rows of phase c: slot j of team t is row
// P (rb * NS * 128 + j * 128 + t) + c of NR, K inputs.  On return, out[u] in lane k of each team is the whole sum of its slot
// k's row for token u (scaled by that token's 2^-se).  xs: the tokens as NTERM fp16 planes
// each, [NT][NTERM][K] (LDS); cbl: the matrix's codebooks [3][256][8] fp16 (LDS); lut: 128
// KB of LDS at address 0.
// prep() (which stages the tokens and codebooks in LDS) runs after the first two steps' index
// bytes are requested, so their latency overlaps it.
template <int NS, int NTERM, int NT, typename Prep>
__device__ __forceinline__ void lut_rows(const uint8_t *__restrict__ idx, int NR, int K, int c, int rb, int nt,
                                         const _Float16 *xs, const _Float16 *cbl, char *lut, float (&out)[NT], Prep &&prep)
{
    const int tid = threadIdx.x, lane = tid & 63;
    LutGeom G;
    G.V = K / 8;
    const int P = lut_phases(G.V);
    G.s0 = (c * G.V) & (kGV - 1);
    G.ng = (G.V + G.s0 + kGV - 1) / kGV;
    G.nstep = 3 * G.ng;
    G.plane = (uint32_t)NR * G.V;
    G.k = tid & 7;
    G.r = 4 * ((lane >> 3) & 3) + (G.k >> 1);
    const __amdgpu_buffer_rsrc_t ir = lrsrc(idx, 3 * G.plane);
    const int row0 = P * (rb * NS * kTeams + (tid >> 3)) + c;  // slot 0's row
    const uint32_t rowoff = (uint32_t)row0 * (uint32_t)G.V;
    uint32_t slot_ok = 0;  // bit j: slot j's row is in the matrix
#pragma unroll
    for (int j = 0; j < NS; j++) slot_ok |= (row0 + j * P * kTeams < NR ? 1u : 0u) << j;
    float acc[NT][NS];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int j = 0; j < NS; j++) acc[t][j] = 0.f;
    uint32_t ia[NS][4], ib[NS][4];  // index bytes of two consecutive steps
    // The prefetch is unconditional (the last step re-reads itself): a conditional load makes
    // the wait before the current step's first use cover the prefetch as well.
    load_idx<NS>(ia, ir, G, P, rowoff, slot_ok, 0);
    for (int st = 0; st < G.nstep; st += 2) {
        const int s1 = min(st + 1, G.nstep - 1), s2 = min(st + 2, G.nstep - 1);
        load_idx<NS>(ib, ir, G, P, rowoff, slot_ok, s1);
        if (st == 0) prep();
        lut_step<NS, NTERM, NT>(ia, acc, G, st, K, nt, xs, cbl, lut);
        load_idx<NS>(ia, ir, G, P, rowoff, slot_ok, s2);
        if (st + 1 < G.nstep) lut_step<NS, NTERM, NT>(ib, acc, G, s1, K, nt, xs, cbl, lut);
    }
    // the team's 8 partial sums of each row; lane k keeps slot k's
#pragma unroll
    for (int t = 0; t < NT; t++) {
        out[t] = 0.f;
#pragma unroll
        for (int j = 0; j < NS; j++) {
            float v = acc[t][j];
            v += dpp_f32<kDppXor1>(v);
            v += dpp_f32<kDppXor2>(v);
            v += dpp_f32<kDppHalfMirror>(v);
            if (G.k == j) out[t] = v;
        }
    }
}

// The block's next work item from the launch's counter ctr.
__device__ __forceinline__ int next_item(uint32_t *ctr, int *sh)
{
    __syncthreads();  // every thread has read the previous item
    if (threadIdx.x == 0) *sh = (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return *sh;
}

// Stage the codebooks of one matrix of expert e ([3][256][8] fp16 = 768 x 16 B) in LDS.
__device__ __forceinline__ void stage_cb(_Float16 *dst, const uint16_t *cb, int e)
{
    const u32x4 *src = (const u32x4 *)(cb + (size_t)e * 3 * 256 * 8);
    for (int i = threadIdx.x; i < 3 * 256; i += blockDim.x) ((u32x4 *)dst)[i] = src[i];
}

}  // namespace

// The active units sorted by token count, descending, into ord[0 .. n_active) (one block;
// counts above 64 share the top bin; positions within a bin are taken by atomics, in no fixed
// order, which only moves work between blocks), and the table-lookup counters zeroed.
__global__ __launch_bounds__(1024) void k_lut_order(const ExpertFwdArgs a)
{
    __shared__ int hist[65];
    const int n = *a.n_active;
    for (int i = threadIdx.x; i < 65; i += blockDim.x) hist[i] = 0;
    if (threadIdx.x < 2) a.dec_sync[kSyncLut + threadIdx.x * kSyncPad] = 0u;
    __syncthreads();
    for (int u = threadIdx.x; u < n; u += blockDim.x) {
        const int e = a.active[u];
        atomicAdd(&hist[min(a.offsets[e + 1] - a.offsets[e], 64)], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int c = 64; c >= 0; c--) {
            const int h = hist[c];
            hist[c] = run;
            run += h;
        }
    }
    __syncthreads();
    for (int u = threadIdx.x; u < n; u += blockDim.x) {
        const int e = a.active[u];
        a.lut_ord[atomicAdd(&hist[min(a.offsets[e + 1] - a.offsets[e], 64)], 1)] = u;
    }
}

// gate and up rows: work item (unit u in the heavy-first order, matrix m, row phase c, row
// block rb) is item ((u * 2 + m) * P + c) * nrb + rb; up to two tokens per pass (the index bytes are read once per
// pass): g or u = row . x for every token of the unit, written to gu [S][2][I] (grouped rows).
template <int NS>
__global__ __launch_bounds__(kLutThreads, 1) void k_gu_lut(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) u32x4 lds_u[];
    const int H = a.H, I = a.I;
    char *lut = (char *)lds_u;
    _Float16 *cbl = (_Float16 *)((char *)lds_u + kLutBytes);
    _Float16 *xs = (_Float16 *)((char *)lds_u + kLutBytes + kCbBytes);  // [2][H] fp16
    float *red = (float *)(xs + 2 * H);
    int *sh = (int *)(red + kLutThreads / 64);
    uint32_t *ctr = a.dec_sync + kSyncLut;
    const int P = lut_phases(H / 8), nrb = ((I + P - 1) / P + NS * kTeams - 1) / (NS * kTeams);
    const int nact = *a.n_active, per = 2 * P * nrb;
    float *gu = a.gu ? a.gu : a.gu_ws;
    for (;;) {
        const int item = next_item(ctr, sh);
        if (item >= nact * per) break;
        const int e = a.active[a.lut_ord[item / per]], m = (item % per) / (P * nrb);
        const int c = (item % (P * nrb)) / nrb, rb = item % nrb;
        const MatW &W = m == 0 ? a.gate : a.up;
        const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;
        const uint8_t *idx = W.idx + (size_t)e * 3 * I * (H / 8);
        const int n = P * (rb * NS * kTeams + (threadIdx.x & 7) * kTeams + (threadIdx.x >> 3)) + c;  // slot k's row
        for (int j0 = 0; j0 < ntok; j0 += 2) {
            const int nt = min(2, ntok - j0);
            int se[2] = {0, 0};
            auto prep = [&]() {
                if (j0 == 0) stage_cb(cbl, W.cb, e);
                for (int t = 0; t < nt; t++) {
                    const uint16_t *xr = (const uint16_t *)a.x + (size_t)(a.perm[r0 + j0 + t] / a.k) * H;
                    float mx = 0.f;
                    for (int c = threadIdx.x; c < H; c += kLutThreads) mx = fmaxf(mx, fabsf(bf16_bits_to_f32(xr[c])));
                    se[t] = lut_scale_exp(block_max(mx, red));
                    for (int c = threadIdx.x; c < H / 2; c += kLutThreads) {
                        const uint32_t v = ((const uint32_t *)xr)[c];
                        ((uint32_t *)(xs + (size_t)t * H))[c] =
                            pack_h2f(ldexpf(bf16_bits_to_f32(v & 0xFFFFu), -se[t]), ldexpf(bf16_bits_to_f32(v >> 16), -se[t]));
                    }
                }
            };
            float o[2];
            lut_rows<NS, 1, 2>(idx, I, H, c, rb, nt, xs, cbl, lut, o, prep);
            if ((threadIdx.x & 7) < NS && n < I) {
                for (int t = 0; t < nt; t++) gu[((size_t)(r0 + j0 + t) * 2 + m) * I + n] = ldexpf(o[t], se[t]);
            }
        }
    }
}

// down rows: work item (unit u in the heavy-first order, row phase c, row block rb) is
// (u * P + c) * nrb + rb; per
// token h = act(g, u) (from gu), o = row . h, and the p-weighted slot rows for the combine.
template <int NS>
__global__ __launch_bounds__(kLutThreads, 1) void k_down_lut(const ExpertFwdArgs a)
{
    extern __shared__ __attribute__((aligned(16))) u32x4 lds_u[];
    const int H = a.H, I = a.I;
    char *lut = (char *)lds_u;
    _Float16 *cbl = (_Float16 *)((char *)lds_u + kLutBytes);
    _Float16 *hs = (_Float16 *)((char *)lds_u + kLutBytes + kCbBytes);  // [2][I] fp16: hi, lo
    float *red = (float *)(hs + 2 * I);
    int *sh = (int *)(red + kLutThreads / 64);
    uint32_t *ctr = a.dec_sync + kSyncLut + kSyncPad;
    const int P = lut_phases(I / 8), nrb = ((H + P - 1) / P + NS * kTeams - 1) / (NS * kTeams);
    const int nact = *a.n_active, per = P * nrb;
    const float *gu = a.gu ? a.gu : a.gu_ws;
    for (;;) {
        const int item = next_item(ctr, sh);
        if (item >= nact * per) break;
        const int e = a.active[a.lut_ord[item / per]], c = (item % per) / nrb, rb = item % nrb;
        const int r0 = a.offsets[e], ntok = a.offsets[e + 1] - r0;
        const uint8_t *idx = a.down.idx + (size_t)e * 3 * H * (I / 8);
        const int n = P * (rb * NS * kTeams + (threadIdx.x & 7) * kTeams + (threadIdx.x >> 3)) + c;  // slot k's row
        for (int j = 0; j < ntok; j++) {
            const size_t rr = (size_t)(r0 + j);
            int se = 0;
            auto prep = [&]() {
                if (j == 0) stage_cb(cbl, a.down.cb, e);
                const float *g = gu + rr * 2 * I, *u = g + I;
                float mx = 0.f;
                for (int c = threadIdx.x; c < I; c += kLutThreads) mx = fmaxf(mx, fabsf(act_h(a.act, g[c], u[c])));
                se = lut_scale_exp(block_max(mx, red));
                for (int c = threadIdx.x; c < I; c += kLutThreads) {
                    const float h = ldexpf(act_h(a.act, g[c], u[c]), -se);
                    const _Float16 hi = (_Float16)h;
                    hs[c] = hi;
                    hs[I + c] = (_Float16)(h - (float)hi);
                }
            };
            float o[1];
            lut_rows<NS, 2, 1>(idx, H, I, c, rb, 1, hs, cbl, lut, o, prep);
            const int slot = a.perm[r0 + j];
            if ((threadIdx.x & 7) < NS && n < H) a.ybuf[(size_t)slot * H + n] = ldexpf(a.w[slot], se) * o[0];
        }
    }
}

namespace {

// Dynamic LDS: the table first (at LDS address 0: the kernels have no static LDS, so table
// addresses need no base added), codebooks, token slices, block-maximum scratch, the item
// broadcast word.
size_t lds_sched(const ExpertFwdArgs &) { return 4 * kLutThreads / 64 + 4; }
size_t lds_gu(const ExpertFwdArgs &a) { return (size_t)kLutBytes + kCbBytes + (size_t)4 * a.H + lds_sched(a); }
size_t lds_down(const ExpertFwdArgs &a) { return (size_t)kLutBytes + kCbBytes + (size_t)4 * a.I + lds_sched(a); }

// Compute units of the current device (cached per device).
int device_cus()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 0;
        cached[dev] = v;
    }
    return cached[dev];
}

// Largest dynamic LDS a block of the current device may take (cached per device).
size_t max_lds_per_block()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) return 0;
        cached[dev] = v;
    }
    return (size_t)cached[dev];
}

// Slots per team for NR rows: the fewest padded rows, then the most slots, at most max_ns
// (seven slots would not fit the 128 registers a thread of a 1024-thread block may hold).
int pick_slots(int NR, int max_ns)
{
    int best = max_ns;
    long bw = -1;
    for (int ns = max_ns; ns >= 5; ns--) {
        const long rows = (long)ns * kTeams, w = ((NR + rows - 1) / rows) * rows - NR;
        if (bw < 0 || w < bw) {
            bw = w;
            best = ns;
        }
    }
    return best;
}

template <int NS>
hipError_t launch_gu(const ExpertFwdArgs &a, int maxU, hipStream_t s)
{
    const size_t lds = lds_gu(a);
    hipError_t err = hipFuncSetAttribute((const void *)k_gu_lut<NS>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    const int P = lut_phases(a.H / 8), items = maxU * 2 * P * (((a.I + P - 1) / P + NS * kTeams - 1) / (NS * kTeams));
    ProfScope ps(a.prof, PK_GATEUP, s);
    ps.launch(k_gu_lut<NS>, dim3(min(items, device_cus())), dim3(kLutThreads), lds, a);
    return hipGetLastError();
}

template <int NS>
hipError_t launch_down(const ExpertFwdArgs &a, int maxU, hipStream_t s)
{
    const size_t lds = lds_down(a);
    hipError_t err = hipFuncSetAttribute((const void *)k_down_lut<NS>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    const int P = lut_phases(a.I / 8), items = maxU * P * (((a.H + P - 1) / P + NS * kTeams - 1) / (NS * kTeams));
    ProfScope ps(a.prof, PK_DOWN, s);
    ps.launch(k_down_lut<NS>, dim3(min(items, device_cus())), dim3(kLutThreads), lds, a);
    return hipGetLastError();
}

}  // namespace

// bf16 tokens, no adapter, both widths multiples of 256 (whole 32 x 32 table tiles),
// index planes addressable with 31-bit offsets, the launch counters and unit order present,
// the table, codebooks and token slices within the device's LDS per block.
bool rvq_lut_supported(const ExpertFwdArgs &a)
{
    if (!(a.wfmt == FMT_RVQ3 && a.xt == DT_BF16 && a.T <= 64 && !a.lora_gu && a.gu_ws && a.dec_sync && a.lut_ord &&
          a.H % 256 == 0 && a.I % 256 == 0 && (size_t)3 * a.H * (a.I / 8) < ((size_t)1 << 31) && device_cus() > 0))
        return false;
    const size_t need = lds_gu(a) > lds_down(a) ? lds_gu(a) : lds_down(a);
    return need <= max_lds_per_block();
}

hipError_t launch_rvq_lut(const ExpertFwdArgs &a, hipStream_t s)
{
    const int maxU = min(a.E, a.T * a.k);
    hipError_t err;
    hipLaunchKernelGGL(k_lut_order, dim3(1), dim3(1024), 0, s, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int pg = lut_phases(a.H / 8), pd = lut_phases(a.I / 8);  // rows per phase: ceil(NR / P)
    err = pick_slots((a.I + pg - 1) / pg, 6) == 6 ? launch_gu<6>(a, maxU, s) : launch_gu<5>(a, maxU, s);
    if (err != hipSuccess) return err;
    return pick_slots((a.H + pd - 1) / pd, 6) == 6 ? launch_down<6>(a, maxU, s) : launch_down<5>(a, maxU, s);
}

}  // namespace moe
