// moe_internal.h -- launch interfaces between the C ABI (moe_api.hip) and the
// kernel files.  Host-side only declarations; no torch, no oracle.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace moe {

// Optional per-kernel timing (include/moe_prof.h): two events per launch on the launch stream.
enum { PK_ROUTER_LOGITS = 0, PK_ROUTER_TOPK, PK_GROUP, PK_GATEUP, PK_DOWN, PK_COMBINE, PK_BWD_DOWN, PK_BWD_GATEUP,
       PK_BWD_FINAL, PK_XTERMS, PK_N };

struct Prof {
    uint32_t mask = 0;
    int cap = 0;
    std::vector<hipEvent_t> ev[PK_N];  // 2 * cap events per family
    int n[PK_N] = {};
};

// Launches one kernel; when timing of its family is on, through hipExtLaunchKernelGGL
// with the family's next event pair, which the runtime stamps at the kernel's start and
// end (not at the queue position before and after it).
class ProfScope {
  public:
    ProfScope(Prof *p, int kid, hipStream_t s) : p_(p), kid_(kid), s_(s)
    {
        on_ = p_ && ((p_->mask >> kid_) & 1u) && p_->n[kid_] < p_->cap;
    }
    template <typename K, typename... Args>
    void launch(K kernel, dim3 grid, dim3 block, size_t shmem, Args... args)
    {
        if (on_) {
            const int n = p_->n[kid_]++;
            hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s_, p_->ev[kid_][2 * n],
                                  p_->ev[kid_][2 * n + 1], 0, args...);
            on_ = false;
        } else {
            hipLaunchKernelGGL(kernel, grid, block, shmem, s_, args...);
        }
    }

  private:
    Prof *p_;
    int kid_;
    hipStream_t s_;
    bool on_;
};

struct RouteArgs {
    Prof *prof;
    const void *x;
    int xt;
    const float *wr;
    const float *bias;   // added to the logits (bias modes 1 and 2)
    const float *wbias;  // bias mode 2: taken back out of the selected logits for the weights, else null
    int T, H, E, k;
    double *rpart;       // workspace for the split-K fp64 router (null: no split)
    size_t rpart_bytes;
    float *logits;  // [T][E] workspace
    float *beta;    // [T][E] workspace
    int32_t *ids;
    float *w;
    int32_t *refined;  // device counter of re-ranked tokens (may be null)
};

struct GroupArgs {
    Prof *prof;
    const int32_t *ids;
    int T, k, E;
    int32_t *counts, *offsets, *perm, *inv, *active, *n_active;
};

// Weights of one matrix (gate, up or down) in either format.
struct MatW {
    const uint8_t *codes;     // MXFP4 [E][rows][cols/2]
    const uint8_t *scales;    // MXFP4 [E][rows][cols/32]
    const uint8_t *idx;       // RVQ3  [E][3][rows][cols/8]
    const uint16_t *cb;       // RVQ3  [E][3][256][8] fp16
};

struct ExpertFwdArgs {
    Prof *prof;
    int wfmt;
    MatW gate, up, down;
    const void *x;
    int xt;
    int T, H, I, E, k;
    const int32_t *offsets, *perm, *active, *n_active;
    const float *w;      // routing weights [T][k]
    uint16_t *h_hi;      // [S][I] grouped rows: h = act(g, u) as bf16 hi ...
    uint16_t *h_lo;      // ... + lo (h - hi rounded to bf16)
    float *gu;           // [S][2][I] grouped rows (g, u) or null
    float *ybuf;         // [S][H] slot rows: w * expert output
    float *y;            // [T][H]
    int act;             // ACT_SWIGLU or ACT_SITU
    uint8_t *xq;         // [T][2H] x as two E4M3 terms for the block-scaled gate/up (grouped-GEMM
    uint8_t *xq_s;       // path; null: bf16 path) and [T][H/32][2] their E8M0 block scales
    int nl_x;            // experts with at most this many tokens stage their x rows in LDS
    int nl_h;            // ... and their h rows (down product)
    const float *lora_gu;  // [T][2I] per-token adapter terms added to g | u, or null
    int xq_single;         // xq / xq_s already hold x as one exact E4M3 term (MXFP8 input)
    int tok_chunks;        // > 0: every expert holds the same token count, split into this many
                           // chunks of kTokChunk tokens, one grouped-GEMM block per chunk and column
                           // block (dense experts: the shared experts); 0: one block per expert
    int skip_combine;      // leave the slot rows in ybuf (no k_combine)
    const float *ybuf2;    // [T][k2][H] more slot rows that k_combine adds after the k routed ones
    int k2;
    // Shared experts run as extra units of the few-token stream kernels' launch (sh_n > 0):
    // unit maxU + s is shared expert s with every token (weight 1), its h planes [s T + t]
    // in sh_h_hi / sh_h_lo and its output rows [t sh_n + s] in sh_ybuf.
    int sh_n;
    MatW sh_gate, sh_up, sh_down;
    uint16_t *sh_h_hi, *sh_h_lo;
    float *sh_ybuf;
    // Counters of the fused decode launch and of the RVQ3 table-lookup launches (kSyncWords,
    // zero between launches; null: the three-launch path, no table lookups) and the status
    // word the fused launch's bounded waits report a timeout into.
    uint32_t *dec_sync;
    uint32_t *status;
    float *gu_ws;  // [S][2][I] workspace for g, u when gu is null (the RVQ3 table-lookup path), or null
    int32_t *lut_ord;  // [S] the table-lookup launches' unit order (workspace), or null
    // The shared adapter inside the fused few-token launch (lora_vx non-null; lora_gu is then
    // null): the gate/up blocks add s B_g vx_g, s B_u vx_u to g and u themselves, and write the
    // partials p_j A_d[:, block columns] h_j of z = A_d hbar to lora_zp [S][r][I / 64]; the last
    // gate/up block reduces them into lora_z [T][r] and the combining blocks add s B_d z to y.
    const float *lora_vx;  // [T][2r]: A_g x | A_u x
    const float *lora_Bg, *lora_Bu, *lora_Ad, *lora_Bd;
    int lora_r;
    float lora_scale;
    float *lora_zp, *lora_z;
};

// Counter layout of the fused decode launch: per-unit gate/up completions, per-stripe down
// arrivals, completed stripes; then the RVQ3 table-lookup launches' work counters (gate/up,
// down; zeroed by the launch before them); each counter on its own 128-byte line (kSyncPad
// words).
constexpr int kSyncUnits = 1152;  // >= min(E, 16 k) + n_shared for the few-token path (k <= 64)
constexpr int kSyncStripes = 64;  // >= H / 64
constexpr int kSyncPad = 32;
constexpr int kSyncLut = (kSyncUnits + kSyncStripes + 1) * kSyncPad;  // first table-lookup counter
// the fused launch with the adapter: finished routed gate/up blocks, then the flag that z is out
constexpr int kSyncLoraGu = kSyncLut + 2 * kSyncPad;
constexpr int kSyncLoraZ = kSyncLoraGu + kSyncPad;
constexpr int kSyncWords = kSyncLoraZ + kSyncPad;
constexpr uint32_t kStatusSpinTimeout = 0x80000000u;  // status-word bit: a fused launch gave up waiting

struct ExpertBwdArgs {
    Prof *prof;
    int wfmt;
    MatW gate, up, down;
    const void *x;
    int xt;
    const void *dy;
    int dyt;
    int T, H, I, E, k;
    const int32_t *ids, *offsets, *perm, *inv, *active, *n_active;
    const float *w;
    const float *wr;
    const float *gu;     // [S][2][I] grouped (g, u)
    uint16_t *h_hi;      // scratch for recomputation [S][I] x 2
    uint16_t *h_lo;
    float *gu_scratch;   // [S][2][I] when gu must be recomputed
    float *dgdu;         // [S][2][I] grouped (dg, du)
    float *dp_part;      // [S][ntile] partial <a, h>
    float *dxs;          // [S][H] slot rows
    float *dx;           // [T][H]
    int act;             // ACT_SWIGLU or ACT_SITU
    const float *lora_gu;  // [T][2I] adapter terms of g | u for the recomputation, or null
    const float *lora_c;   // [T][I] adapter term added to a = Wd^T dy per token, or null
    int tok_chunks;        // as in ExpertFwdArgs
    int skip_final;        // leave the slot rows in dxs (no k_bwd_final)
    const float *dxs2;     // [T][k2][H] more slot rows that k_bwd_final adds (no router term)
    int k2;
};

// Token chunk of the grouped-GEMM kernels (one pass of a block).
constexpr int kTokChunk = 96;

// Routing of n_sh experts that every token takes with weight 1 (the shared experts):
// expert s holds tokens 0..T-1 in order (group.hip).
hipError_t launch_dense_routing(int T, int n_sh, int32_t *ids, float *w, int32_t *offsets, int32_t *perm, int32_t *inv,
                                int32_t *active, int32_t *n_active, hipStream_t s);

// Token rows staged in LDS by the few-token (decode) expert kernels: at most 16 rows
// and at most 48 KB of LDS per block.
inline void set_lds_staging(ExpertFwdArgs &a)
{
    const int tmax = a.T < 16 ? a.T : 16;
    const int nx = (int)(48 * 1024 / ((size_t)(a.H + 8) * 2));
    const int nh = (int)(48 * 1024 / ((size_t)(a.I + 8) * 4));
    a.nl_x = tmax < nx ? tmax : nx;
    a.nl_h = tmax < nh ? tmax : nh;
}

hipError_t launch_router(const RouteArgs &a, hipStream_t s);
// Small batches (route_small_ok): router logits, then top-k and grouping in one launch.
bool route_small_ok(const RouteArgs &a);
hipError_t launch_route_small(const RouteArgs &a, const GroupArgs &g, hipStream_t s);
hipError_t launch_group(const GroupArgs &a, hipStream_t s);
hipError_t launch_expert_forward(const ExpertFwdArgs &a, hipStream_t s);
hipError_t launch_gateup_only(const ExpertFwdArgs &a, hipStream_t s);

// Grouped-GEMM forward kernels for experts holding many tokens (expert_mm.hip):
// MXFP4 weights, bf16 tokens, H and I multiples of 512.
bool mm_supported(const ExpertFwdArgs &a);
hipError_t launch_gateup_mm(const ExpertFwdArgs &a, hipStream_t s);
hipError_t launch_down_mm(const ExpertFwdArgs &a, hipStream_t s);
// Few-token MXFP4 kernels (expert_dec.hip) for T <= nl_x, nl_h with bf16 tokens.
bool dec_supported(const ExpertFwdArgs &a);
hipError_t launch_gateup_dec(const ExpertFwdArgs &a, hipStream_t s);
hipError_t launch_down_dec(const ExpertFwdArgs &a, hipStream_t s);
// gate/up, down and combine of the few-token path in one launch (expert_dec.hip)
bool dec_fused_ok(const ExpertFwdArgs &a);
hipError_t launch_dec_fused(const ExpertFwdArgs &a, hipStream_t s);
// Few-token RVQ3 kernels (expert_rvq.hip): codeword gathers as fp16 MFMA operands.
bool rvq_dec_supported(const ExpertFwdArgs &a);
hipError_t launch_gateup_rvq(const ExpertFwdArgs &a, hipStream_t s);
hipError_t launch_down_rvq(const ExpertFwdArgs &a, hipStream_t s);
// Few-token RVQ3 as table lookups (expert_rvq_lut.hip): gate and up into g, u, then down.
bool rvq_lut_supported(const ExpertFwdArgs &a);
hipError_t launch_rvq_lut(const ExpertFwdArgs &a, hipStream_t s);
// taken when the experts average at least 8 tokens each
inline bool use_mm(const ExpertFwdArgs &a) { return (size_t)a.T * a.k >= (size_t)8 * a.E && mm_supported(a); }
hipError_t launch_expert_backward(const ExpertBwdArgs &a, hipStream_t s);

// Grouped-GEMM backward kernels (expert_bwd_mm.hip): MXFP4, bf16 dy, H and I multiples
// of 512.  They keep dg/du as bf16 hi + lo planes [2][S][2I] in the dgdu buffer.
bool bwd_mm_supported(const ExpertBwdArgs &a);
hipError_t launch_bwd_down_mm(const ExpertBwdArgs &a, hipStream_t s);
hipError_t launch_bwd_gateup_mm(const ExpertBwdArgs &a, hipStream_t s);

// The grouped-GEMM backward runs when the experts average at least 8 tokens each; its
// dg/du rows are bf16 hi + lo planes, the generic backward's fp32.
inline bool bwd_uses_mm(const ExpertBwdArgs &a) { return (size_t)a.T * a.k >= (size_t)8 * a.E && bwd_mm_supported(a); }

// MXFP8 quantization of x [T][H] into its represented values as bf16 (quant.hip); with
// mxq / mxs also as the block-scaled gate/up's single-term operand (null: not written).
hipError_t launch_quant_x8(const void *x, int xt, int T, int H, uint16_t *xq, uint8_t *mxq, uint8_t *mxs, hipStream_t s);

// Shared low-rank adapter (lora.hip): weights (borrowed, fp32) and workspace.
struct LoraW {
    int r;
    float scale;
    const float *A[3];  // [r][in]
    const float *B[3];  // [out][r]
};
struct LoraWs {
    float *vx;    // [T][2r]  A_g x | A_u x
    float *gu;    // [T][2I]  s B_g A_g x | s B_u A_u x
    float *hbar;  // [T][I]   sum_j p h over the token's slots
    float *z;     // [T][r]   sum_j p A_d h
    float *wd;    // [T][r]   B_d^T dy
    float *c;     // [T][I]   s A_d^T B_d^T dy
    float *dgu;   // [T][2I]  per-token sums of dL/dg | dL/du
    float *m;     // [T][2r]  B_g^T dgu_g | B_u^T dgu_u
    float *part;  // split-K partial sums
    size_t part_cap;  // floats
};
hipError_t lora_forward_pre(const LoraW &L, const LoraWs &w, const void *x, int xt, int T, int H, int I, hipStream_t s);
// vx = [A_g x | A_u x] only (the fused few-token launch forms the rest itself)
hipError_t lora_forward_vx(const LoraW &L, const LoraWs &w, const void *x, int xt, int T, int H, hipStream_t s);
hipError_t lora_forward_post(const LoraW &L, const LoraWs &w, const ExpertFwdArgs &a, const int32_t *inv, hipStream_t s);
hipError_t lora_backward_pre(const LoraW &L, const LoraWs &w, const void *dy, int dyt, int T, int H, int I, hipStream_t s);
hipError_t lora_backward_post(const LoraW &L, const LoraWs &w, const ExpertBwdArgs &a, bool pair, hipStream_t s);
hipError_t lora_grads(const LoraW &L, const LoraWs &w, const ExpertBwdArgs &a, float *const dA[3], float *const dB[3],
                      hipStream_t s);
hipError_t fill_zero(float *p, size_t n, hipStream_t s);

// MOE_F_VALIDATE (validate.hip): OR `bit` into *status if any of the n bf16/fp32 values at
// p (16-byte aligned, n a multiple of 8) is non-finite; OR the MOE_BAD_* bits of the scale
// bytes (MXFP4) or codewords (RVQ3) of the experts a call reads: active[u] for u <
// *n_active (active non-null), else experts 0..units-1; store v into *p.
hipError_t launch_check_finite(const void *p, int dt, size_t n, uint32_t *status, uint32_t bit, hipStream_t s);
hipError_t launch_check_weights(int wfmt, const MatW (&m)[3], const size_t (&scale_bytes)[3], const int32_t *active,
                                const int32_t *n_active, int units, uint32_t *status, hipStream_t s);
hipError_t launch_set_u32(uint32_t *p, uint32_t v, hipStream_t s);

// Latent projection (dense.hip): out[T][N] = a[T][R] w^T with w [N][R] (nn = false) or
// a[T][R] w with w [R][N] (nn = true); a bf16 or fp32 (at), w bf16; N % 64 == 0, R % 32 == 0.
hipError_t launch_dense(const void *a, int at, const uint16_t *w, bool nn, int T, int N, int R, float *out, hipStream_t s);

// number of I-column tiles whose partial <a, h> sums the backward stores per row
__host__ __device__ inline int dp_tiles(int I) { return (I + 63) / 64; }

}  // namespace moe
