/*
 * moe_oracle.h -- declarations of the fp64 CPU oracle (test infrastructure
 * only; the GPU library never includes this header).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

enum { ORACLE_FMT_MXFP4 = 0, ORACLE_FMT_RVQ3 = 1 };
enum { ORACLE_MAT_GATE = 0, ORACLE_MAT_UP = 1, ORACLE_MAT_DOWN = 2 };

/* Low-rank adapter shared by every routed expert of the layer (LazyLoRA
 * README, "LoRA"): each of gate, up and down gets W + scale * B A.
 * A[gate], A[up]: [r][H]; A[down]: [r][I]; B[gate], B[up]: [I][r];
 * B[down]: [H][r]; row-major fp64. */
typedef struct {
    int r;
    double scale;
    const double *A[3];
    const double *B[3];
} oracle_lora;

typedef struct {
    int fmt;
    const uint8_t *codes[3];     /* MXFP4: [E][rows][cols/2]  */
    const uint8_t *scales[3];    /* MXFP4: [E][rows][cols/32] */
    const uint8_t *rvq_idx[3];   /* RVQ3:  [E][3][rows][cols/8] */
    const uint16_t *rvq_cb[3];   /* RVQ3:  [E][3][256][8] fp16 bits */
    int act;                     /* expert activation: ORACLE_ACT_SWIGLU or ORACLE_ACT_SITU */
    const oracle_lora *lora;     /* shared adapter, or NULL */
} oracle_weights;

enum { ORACLE_ACT_SWIGLU = 0, ORACLE_ACT_SITU = 1 };

double oracle_e2m1(unsigned code);
double oracle_e4m3(unsigned code);
void oracle_quantize_mxfp8(int n, const double *x, double *xq, int32_t *exps);
double oracle_e8m0(unsigned b);
double oracle_fp16(uint16_t h);
void oracle_decode_row(const oracle_weights *W, int mat, int e, int H, int I, int row, double *out);
void oracle_decode_matrix(const oracle_weights *W, int mat, int e, int H, int I, double *out);
void oracle_router_logits(int T, int H, int E, const double *x, const double *wr, const double *bias,
                          double *logits, int nthreads);
int oracle_topk_softmax(int T, int E, int k, const double *logits, int32_t *ids, double *w);
void oracle_softmax_at(int T, int E, int k, const double *logits, const int32_t *ids, double *w);
void oracle_group(int T, int k, int E, const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *perm,
                  int32_t *inv, int32_t *active, int32_t *n_active);
void oracle_expert_forward(const oracle_weights *W, int e, int H, int I, const double *x, double *g_out,
                           double *u_out, double *h_out, double *o_out);
void oracle_forward(int T, int H, int I, int k, const double *x, const int32_t *ids, const double *w,
                    const oracle_weights *W, double *y, int nthreads);
void oracle_backward_input(int T, int H, int I, int k, const double *x, const double *dy, const int32_t *ids,
                           const double *w, const double *wr, const oracle_weights *W, double *dx, int nthreads);
/* Gradients of sum_t <dy[t], y[t]> with respect to the adapter's A and B
 * (same layouts as oracle_lora), routing held fixed.  W->lora must be set. */
void oracle_lora_grads(int T, int H, int I, int k, const double *x, const double *dy, const int32_t *ids,
                       const double *w, const oracle_weights *W, double *dA[3], double *dB[3], int nthreads);
/* Latent projection with bf16 weights w [N][K]: out [T][N] = a [T][K] w^T, or with
 * transposed != 0 out [T][K] = a [T][N] w. */
void oracle_dense(int T, int N, int K, const double *a, const uint16_t *w, double *out, int transposed, int nthreads);
#endif
