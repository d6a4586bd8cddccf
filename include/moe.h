/*
 * moe.h -- C ABI of the routed-expert MoE layer for AMD Instinct MI355X (gfx950).
 *
 * The layer: a router picks the top-k of E experts per token, the tokens are
 * grouped by expert, each routed expert applies a SwiGLU MLP whose gate, up
 * and down matrices are stored quantized (MXFP4, or 3-bit residual VQ), and
 * the expert outputs are combined with the routing weights.  The input
 * gradient through the frozen experts and the router is also provided.
 *
 * Sources (cited by page and section):
 *  - LazyLoRA README (github heyobi/LazyLora), "The engine": Kimi K3 has 896
 *    routed experts per MoE layer, top-16 routing and MXFP4 expert weights;
 *    the routed experts are one differentiable unit whose backward returns
 *    the gradient with respect to the latent input ("Routed experts");
 *    expert sums accumulate in fp32 ("Arithmetic"); a tensor that is missing
 *    raises instead of being replaced ("Three rules the engine is built
 *    around").  "File map": top-16 gating with a score-correction bias; a
 *    routing record holds the chosen experts and their combining weights.
 *    "LoRA": the expert shape 3584 -> 3072 -> 3584 in the MoE latent space.
 *  - WASTE README (hackernews.jp story 49123386): an embeddable C API whose
 *    open call returns a status and fills an out-handle, a config struct with
 *    an init function for defaults, and a close call; experts stored as
 *    3-bit residual VQ, 3 stages of 256-entry codebooks over 8-dim vectors.
 *  - OCP Microscaling Formats (MX) v1.0: E2M1 elements, E8M0 block scales.
 *
 * Conventions
 *  - Every tensor argument is a DEVICE pointer allocated by the caller
 *    (typically through PyTorch); the library allocates no device memory.
 *  - Every call that takes a stream only enqueues work on it (a hipStream_t
 *    passed as void*; NULL = the null stream) and returns without waiting.
 *    Data-dependent sizes (per-expert token counts, number of active
 *    experts) stay on the device; no call synchronizes with the host.
 *  - Argument checks run on the host, synchronously, before anything is
 *    enqueued; on failure nothing is enqueued and no output is touched.
 *  - No C++ exception crosses this interface.  A failed kernel launch
 *    returns MOE_ERR_DEVICE; faults inside kernels surface at the caller's
 *    next stream synchronization.
 *  - One layer handle may be used from one stream at a time (its workspace
 *    is shared by all calls on it).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* a null pointer, a bad size, a bad dtype, misalignment */
    MOE_ERR_UNSUPPORTED = 2,   /* a valid request the library does not implement */
    MOE_ERR_WORKSPACE = 3,     /* workspace smaller than moe_workspace_size() */
    MOE_ERR_DEVICE = 4,        /* a HIP call failed; text in moe_last_error() */
    MOE_ERR_INTERNAL = 5,
    MOE_ERR_DATA = 6           /* MOE_F_VALIDATE: an earlier call found out-of-contract data on the
                                  device (MOE_BAD_* bits named in moe_last_error()) */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;
typedef enum { MOE_W_MXFP4 = 0, MOE_W_RVQ3 = 1 } moe_wfmt;
typedef enum {
    MOE_ACT_SWIGLU = 0,  /* h = silu(g) * u = g sigmoid(g) u (the configs' activation) */
    MOE_ACT_SITU = 1     /* h = 4 tanh(g/4) sigmoid(g) * 25 tanh(u/25): K3's SiTU (LazyLoRA README,
                            "File map", core/situ_activation.py) */
} moe_act;

/* flags */
enum {
    MOE_F_DETERMINISTIC = 1u, /* combine and gradient reductions in a fixed order (always on: the library has no unordered mode) */
    MOE_F_MX_GATEUP = 2u,     /* grouped-GEMM gate/up (MXFP4, bf16 x, many tokens per expert) on the
                                 gfx950 block-scaled MFMA: weights enter as FP4 codes with their E8M0
                                 scales and x as two E4M3 terms with per-32 scales (each element
                                 carried to about 2^-20 of its block's maximum).  The MFMA's own
                                 summation of the block products is coarser than bf16 MFMA's: y
                                 measured within 2e-6 of max|y| on Gaussian x and within 6e-5 with x
                                 spread over 2^-12..2^6 inside each 32-block.  The g, u it saves
                                 (saved_gu) carry that deviation, and the input gradient from them
                                 up to ~7e-4 on the spread x; with saved_gu = NULL the backward
                                 recomputes g, u on the exact bf16 path (within 1e-4).  More
                                 workspace (3H + H/16 bytes per token).  Off: exact bf16
                                 dequantization and bf16 MFMA. */
    MOE_F_LORA = 4u,          /* workspace for a shared low-rank adapter (moe_set_lora) */
    MOE_F_QUANT_X8 = 8u,      /* moe_forward quantizes x to MXFP8 before the expert products (OCP MX
                                 v1.0: E4M3 elements, one E8M0 scale per 32 consecutive elements,
                                 shared exponent floor(log2 max|x|) - 8, round to nearest even,
                                 saturation at 448): activation-quantized prefill.  The routing
                                 (moe_route) sees x unquantized.  moe_backward_input with saved_gu
                                 = NULL is the exact (unquantized) layer's gradient; with saved_gu
                                 from such a forward it is the quantized layer's, the quantization
                                 passed straight through (its derivative taken as 1).  H must be a
                                 multiple of 32 (always).  More workspace: 2 H bytes per token. */
    MOE_F_VALIDATE = 16u,     /* device checks of the data each call consumes (below) */
    MOE_F_RVQ_GATHER = 32u    /* RVQ3 with few tokens per expert on the codeword-gather kernels
                                 (each stage's codeword an fp16 MFMA operand) instead of the
                                 codeword-table lookups; for comparing the two forms (same
                                 results to the parity bar, different rounding order) */
};

/* MOE_F_VALIDATE (LazyLoRA README, "Three rules the engine is built around": unusable
 * data is an error, never replaced).  Every call on the layer first scans, on the device,
 * what it is about to consume, and ORs these bits into a status word in the workspace:
 *   moe_route           x;
 *   moe_forward         the scale bytes (MXFP4) or codebooks (RVQ3) of the active experts
 *                       and of the shared experts;
 *   moe_backward_input  dy, and the same weights.
 * The call's kernels still run to completion on what they were given (out-of-contract
 * inputs give meaningless outputs, never a fault).  The NEXT call on the layer, or
 * moe_check_status(), synchronizes the stream, reads the word, clears it and returns
 * MOE_ERR_DATA if it was nonzero (without enqueuing anything else).  So with the flag
 * every call costs one host synchronization; without it nothing is checked and values
 * outside the contract give undefined (but finite-time, fault-free) results. */
enum {
    MOE_BAD_X = 1u,           /* a non-finite activation */
    MOE_BAD_DY = 2u,          /* a non-finite upstream gradient */
    MOE_BAD_SCALE_NAN = 4u,   /* an E8M0 scale byte 0xFF (NaN in the format) */
    MOE_BAD_SCALE_ZERO = 8u,  /* an E8M0 scale byte 0x00 (2^-127: the kernels carry products of
                                 normal magnitude only; such a block would be read as zero) */
    MOE_BAD_CODEWORD = 16u    /* a non-finite fp16 RVQ3 codeword */
};

/* Layer description.  moe_desc_init() fills the K3 defaults. */
typedef struct {
    int32_t hidden;      /* H: latent width (K3: 3584); multiple of 32 */
    int32_t inter;       /* I: expert intermediate width (K3: 3072); multiple of 32 */
    int32_t n_experts;   /* E: routed experts (K3: 896); 1..2048 */
    int32_t top_k;       /* k: experts per token (K3: 16); 1..min(E, 64) */
    int32_t max_tokens;  /* largest T any call on this layer will pass; sizes the workspace */
    int32_t wfmt;        /* moe_wfmt */
    int32_t act;         /* moe_act: the gated activation h = act(gate, up) */
    int32_t bias_mode;   /* 0: no router bias; 1: bias added to the logits (selection and weights);
                            2: bias for the selection only (the weights are the softmax of the
                            unbiased logits over the selected experts) */
    uint32_t flags;
    int32_t n_shared;    /* shared experts (K3: 2), 0..top_k: experts every token takes with weight 1
                            beside the routed ones (LazyLoRA README, "The engine": 896 routed and 2
                            shared experts in each MoE layer).  Same shape, format and activation as
                            a routed expert; their outputs are added to y, their input gradient to
                            dx; they get no router term and no adapter.  Default 0. */
    int32_t model_width; /* D: width of the model around the MoE's latent space, 0 = none (default).
                            With D > 0 the layer also holds the latent in/out projections
                            (moe_project_in/out below); D and H multiples of 64. */
} moe_desc;

/* Expert and router weights: BORROWED device pointers.  The caller keeps
 * them alive and unchanged until moe_destroy().  Matrices are stored
 * [out][in] row-major with `in` contiguous: gate and up are [I][H], down is
 * [H][I]; index 0 = gate, 1 = up, 2 = down.
 *
 * MXFP4 (wfmt = MOE_W_MXFP4): codes[m] is [E][out][in/2] bytes, byte j of a
 *   row holding element 2j in its low nibble and 2j+1 in its high nibble
 *   (E2M1: bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa);
 *   scales[m] is [E][out][in/32] E8M0 bytes, one per 32 consecutive `in`
 *   elements, value 2^(byte-127).  Element = E2M1(code) * 2^(scale-127).
 *   codes and scales must be 16-byte aligned.  Scale bytes must lie in 1..254: 0xFF
 *   means NaN in the format, and 0x00 (2^-127) scales every element of its block below the
 *   smallest normal number, which the kernels do not carry; MOE_F_VALIDATE reports both.
 * RVQ3 (wfmt = MOE_W_RVQ3): rvq_idx[m] is [E][3][out][in/8] bytes (stage-
 *   planar); rvq_cb[m] is [E][3][256][8] fp16 codewords.  Elements 8v..8v+7
 *   of a row equal the sum over the three stages s of
 *   rvq_cb[m][e][s][rvq_idx[m][e][s][row][v]].  Both 16-byte aligned.
 * router_w is [E][H] fp32; router_b is [E] fp32 or NULL (required when
 * bias_mode = 1 or 2). */
typedef struct {
    const float *router_w;
    const float *router_b;
    const uint8_t *codes[3];
    const uint8_t *scales[3];
    const uint8_t *rvq_idx[3];
    const uint16_t *rvq_cb[3];
    /* the n_shared shared experts, laid out like the routed ones with n_shared in place of E
       (only those of d->wfmt; NULL when n_shared = 0) */
    const uint8_t *shared_codes[3];
    const uint8_t *shared_scales[3];
    const uint8_t *shared_rvq_idx[3];
    const uint16_t *shared_rvq_cb[3];
    /* latent projections (model_width D > 0; NULL otherwise): bf16 bit patterns, 16-byte
       aligned, proj_in [H][D] (model -> latent), proj_out [D][H] (latent -> model) */
    const uint16_t *proj_in;
    const uint16_t *proj_out;
} moe_weights;

/* Routing record, caller-owned device buffers written by moe_route() and
 * read by moe_forward() / moe_backward_input():
 *   ids      [T][k] int32  chosen experts, ranked by logit (larger first;
 *                          equal logits rank the lower expert id first)
 *   w        [T][k] fp32   combining weights: softmax over the k chosen logits
 *   counts   [E]    int32  slots routed to each expert
 *   offsets  [E+1]  int32  exclusive prefix sum of counts
 *   perm     [T*k]  int32  slot indices t*k+j ordered by (expert, token)
 *   inv      [T*k]  int32  inverse of perm (grouped row of each slot)
 *   active   [E]    int32  experts with a nonzero count, ascending (first
 *                          *n_active entries are meaningful)
 *   n_active [1]    int32  number of active experts */
typedef struct {
    int32_t *ids;
    float *w;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int32_t *inv;
    int32_t *active;
    int32_t *n_active;
} moe_routing;

typedef struct moe_layer moe_layer;

/* Fill *d with the K3 layer: H 3584, I 3072, E 896, k 16, max_tokens 4096,
 * MXFP4, SwiGLU, no bias, deterministic. */
void moe_desc_init(moe_desc *d);

/* Bytes of device workspace the layer needs for d->max_tokens tokens. */
moe_status moe_workspace_size(const moe_desc *d, size_t *bytes);

/* Validate d and w, and create a host-side handle that borrows the weights
 * and the workspace (a device buffer of at least moe_workspace_size() bytes,
 * 256-byte aligned, owned by the caller until moe_destroy()).  Copies *d. */
moe_status moe_layer_create(const moe_desc *d, const moe_weights *w, void *workspace, size_t ws_bytes,
                            moe_layer **out);

/* Router and grouping.  x is [T][H] of dtype xt (fp32 or bf16), 16-byte
 * aligned.  Fills every buffer of *r.  Logits are formed in fp32; tokens whose
 * ranking is not certain under a rigorous fp32 error bound are re-ranked from
 * fp64 logits, so the selection equals the one made on fp64 logits.
 * T = 0 is a no-op.  0 <= T <= max_tokens. */
moe_status moe_route(moe_layer *L, const void *x, int32_t xt, int32_t T, const moe_routing *r, void *stream);

/* Expert forward and combine: y[T][H] fp32 = sum_j w[t][j] * expert_{ids[t][j]}(x[t])
 * + sum_s shared_s(x[t]) (s < n_shared; summed in that order after the routed slots).
 * The shared experts' pre-activations are not saved (moe_backward_input
 * recomputes them).
 * r must come from moe_route() on the same x and T.  If saved_gu is not
 * NULL it receives the gate and up pre-activations [T*k][2][I] fp32 in
 * grouped row order (row = inv[t*k+j]) for moe_backward_input(). */
moe_status moe_forward(moe_layer *L, const void *x, int32_t xt, int32_t T, const moe_routing *r, float *y,
                       float *saved_gu, void *stream);

/* Input gradient through the frozen experts and the router:
 * dx[T][H] fp32 = d/dx of sum_t <dy[t], y[t]> with the routing held fixed
 * (the expert selection is piecewise constant; the gradient flows through
 * the experts and through the softmax weights into the router logits).
 * dy is [T][H] of dtype dyt.  saved_gu from moe_forward() on the same
 * inputs, or NULL to recompute it. */
moe_status moe_backward_input(moe_layer *L, const void *x, int32_t xt, const void *dy, int32_t dyt, int32_t T,
                              const moe_routing *r, const float *saved_gu, float *dx, void *stream);

/* Latent projections (LazyLoRA README, "The engine": the latent MoE projections are dense
 * weights beside the router gates; Two Desks, Act II: the experts run in a latent space of
 * width 3,584).  The layer's input and output live in the model width D; the router, the
 * routed and the shared experts work in the latent width H:
 *   x_latent = x_model proj_in^T   -> moe_route / moe_forward on x_latent -> y_latent
 *   out      = y_latent proj_out^T
 * and the input gradient runs the chain backwards (moe_project_out_backward, then
 * moe_backward_input with dy = its result, then moe_project_in_backward).  Products of the
 * bf16 weights with bf16 or fp32 activations (fp32 carried exactly), fp32 accumulation,
 * fp32 results; all buffers caller-owned device memory, 16-byte aligned.  Errors as for the
 * other calls; MOE_ERR_INVALID_ARG if the layer has no projections (model_width = 0).
 *   moe_project_in           x_model [T][D] (dtype xt) -> x_latent [T][H] fp32
 *   moe_project_out          y_latent [T][H] fp32      -> out [T][D] fp32
 *   moe_project_out_backward dout [T][D] (dtype dt)    -> dy_latent [T][H] fp32 = dout proj_out
 *   moe_project_in_backward  dx_latent [T][H] fp32     -> dx_model [T][D] fp32 = dx_latent proj_in */
moe_status moe_project_in(moe_layer *L, const void *x_model, int32_t xt, int32_t T, float *x_latent, void *stream);
moe_status moe_project_out(moe_layer *L, const float *y_latent, int32_t T, float *out, void *stream);
moe_status moe_project_out_backward(moe_layer *L, const void *dout, int32_t dt, int32_t T, float *dy_latent,
                                    void *stream);
moe_status moe_project_in_backward(moe_layer *L, const float *dx_latent, int32_t T, float *dx_model, void *stream);

/* Shared low-rank adapter on the routed experts (LazyLoRA README, "LoRA": one
 * adapter per MoE layer in the latent space, shared by every routed expert, on
 * the gate, up and down projections; rank 16 there).  While attached, every
 * expert product W z of moe_forward, moe_backward_input and moe_backward_lora
 * becomes (W + scale B A) z = W z + scale B (A z).  BORROWED fp32 device
 * pointers, 16-byte aligned, kept alive and unchanged while attached:
 *   A[0], A[1] [rank][H] and B[0], B[1] [I][rank]  (gate, up)
 *   A[2] [rank][I] and B[2] [H][rank]              (down)
 * scale is typically alpha / rank. */
typedef struct {
    int32_t rank;  /* 1..64 */
    float scale;
    const float *A[3];
    const float *B[3];
} moe_lora;

/* Attach the adapter (lora != NULL) or detach it (NULL).  The layer must have
 * been created with MOE_F_LORA in desc->flags (its workspace holds the
 * adapter's buffers); otherwise, or for a rank outside 1..64, a non-finite
 * scale or a NULL or misaligned pointer: MOE_ERR_INVALID_ARG and nothing
 * changes.  Copies *lora; enqueues nothing. */
moe_status moe_set_lora(moe_layer *L, const moe_lora *lora);

/* moe_backward_input() plus the adapter gradients of sum_t <dy[t], y[t]>
 * (routing held fixed): dA[m] and dB[m] receive fp32 arrays shaped like A[m]
 * and B[m] (overwritten; caller-owned device buffers, 16-byte aligned).  The
 * sums over tokens and slots run in a fixed order, so repeated calls give the
 * same bits.  Requires an attached adapter (else MOE_ERR_INVALID_ARG).  T = 0
 * writes zero gradients. */
moe_status moe_backward_lora(moe_layer *L, const void *x, int32_t xt, const void *dy, int32_t dyt, int32_t T,
                             const moe_routing *r, const float *saved_gu, float *dx, float *const dA[3],
                             float *const dB[3], void *stream);

/* moe_forward() with saved_gu = NULL, for callers that cannot allocate device memory:
 * code under HIP graph capture, serving loops that must not call the allocator, harnesses
 * that forbid it.  Same arguments, semantics and results (the same kernels); the scratch the
 * kernels use (h or, for RVQ3, g and u, the weighted slot rows, counters) is not the layer's
 * workspace but one array of 32 MiB compiled into the library, one copy per GPU, held until
 * the process ends.  The call allocates nothing and calls no allocating routine; it clears
 * that array's counters with a fill kernel on `stream` (no memset).  Limits: T k (4 I + 4 H)
 * bytes (RVQ3: T k (8 I + 4 H)) plus ~157 KB must fit in 32 MiB (K3 shape: T <= 78 at
 * k = 16; RVQ3 at the K3 shape: T <= 53), else MOE_ERR_WORKSPACE and
 * nothing is enqueued; layers with shared experts, an attached adapter, MOE_F_MX_GATEUP,
 * MOE_F_QUANT_X8 or MOE_F_VALIDATE give MOE_ERR_UNSUPPORTED.  Every call on one GPU uses the
 * same array: calls that overlap on one GPU (other streams, other threads, other layers)
 * race and give wrong results; serialize them. */
moe_status moe_forward_static(moe_layer *L, const void *x, int32_t xt, int32_t T, const moe_routing *r, float *y,
                              void *stream);

/* MOE_F_VALIDATE: synchronize stream, return the device status word in *bits (MOE_BAD_*)
 * and clear it.  MOE_ERR_DATA if it was nonzero, MOE_OK if zero; MOE_ERR_INVALID_ARG for
 * a NULL argument or a layer created without MOE_F_VALIDATE. */
moe_status moe_check_status(moe_layer *L, uint32_t *bits, void *stream);

/* Release the handle (NULL is a no-op).  Borrowed memory is not freed. */
void moe_destroy(moe_layer *L);

/* Static text of a status code. */
const char *moe_status_string(moe_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
