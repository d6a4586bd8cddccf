/*
 * moe_oracle.c -- plain, slow, fp64 CPU model of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * includes, links or calls anything in this directory, and this file shares
 * no source with it.
 *
 * Every function is the plain definition of one step, evaluated in double
 * precision with plain loops (threads only split independent tokens or
 * token-expert slots; each slot's arithmetic runs sequentially in the order
 * written).  Sources:
 *   - LazyLoRA README (github heyobi/LazyLora), "The engine": K3 has 896
 *     routed experts per MoE layer, top-16 routing, MXFP4 expert weights;
 *     "Routed experts": the routed experts form one unit whose backward
 *     returns the gradient with respect to the latent input; "Arithmetic":
 *     expert sums accumulate in fp32 or wider; "File map": top-16 gating with
 *     a score-correction bias, and a routing record holds the chosen experts
 *     with their combining weights; "LoRA": the expert shape 3584->3072->3584.
 *   - WASTE README (hackernews.jp story 49123386), section on 3 bits per
 *     expert weight: residual VQ with 3 stages of 256-entry codebooks over
 *     8-dimensional vectors.
 *   - OCP Microscaling Formats (MX) v1.0: the E2M1 element and E8M0 scale.
 *   LazyLoRA README, "File map": K3's SiTU expert activation,
 *     4 tanh(g/4) sigmoid(g) x 25 tanh(u/25) (the optional second activation).
 * Readings where the pages are silent (SwiGLU with the gate as the SiLU
 * branch, softmax over the selected logits, ties to the lower expert id,
 * nibble order, block direction, RVQ vector orientation) are the ones listed
 * in the design notes; each is restated beside the code that takes it.
 *
 * Parity pins: every function here is checked by tests against closed forms,
 * brute force, library routines or finite differences; none is "unpinned".
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

/* ------------------------------------------------------------------ */
/* element formats                                                     */
/* ------------------------------------------------------------------ */

/* OCP MX v1.0 FP4 (E2M1): bit 3 sign, bits 2..1 exponent with bias 1,
 * bit 0 mantissa; exponent field 0 is subnormal (0 or 0.5). */
double oracle_e2m1(unsigned code)
{
    unsigned sign = (code >> 3) & 1u, ef = (code >> 1) & 3u, mf = code & 1u;
    double mag = (ef == 0) ? 0.5 * (double)mf : ldexp(1.0 + 0.5 * (double)mf, (int)ef - 1);
    return sign ? -mag : mag;
}

/* OCP MX v1.0 E8M0 scale: 2^(b-127); the byte 0xFF encodes NaN. */
double oracle_e8m0(unsigned b)
{
    return (b == 255u) ? NAN : ldexp(1.0, (int)b - 127);
}

/* IEEE binary16 from its bit fields. */
double oracle_fp16(uint16_t h)
{
    unsigned sign = (h >> 15) & 1u, ef = (h >> 10) & 31u, mf = h & 1023u;
    double v;
    if (ef == 0)
        v = ldexp((double)mf, -24);
    else if (ef == 31)
        v = mf ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + (double)mf, (int)ef - 25);
    return sign ? -v : v;
}

/* OCP MX v1.0 FP8 E4M3: bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0
 * mantissa; exponent field 0 is subnormal (m/8 * 2^-6); exponent 15 with
 * mantissa 7 is NaN, so the largest normal is 1.75 * 2^8 = 448. */
double oracle_e4m3(unsigned code)
{
    unsigned sign = (code >> 7) & 1u, ef = (code >> 3) & 15u, mf = code & 7u;
    double mag;
    if (ef == 15u && mf == 7u)
        mag = NAN;
    else if (ef == 0)
        mag = ldexp((double)mf, -9);
    else
        mag = ldexp(8.0 + (double)mf, (int)ef - 10);
    return sign ? -mag : mag;
}

/* v rounded to the nearest E4M3 value, ties to the even mantissa, magnitudes
 * past 448 saturated to 448 (the MX conversion's clamp).  v is exact here: the
 * grid step of the binade of v is 2^(floor(log2|v|) - 3), 2^-9 below 2^-6. */
static double round_e4m3(double v)
{
    double a = fabs(v);
    if (a == 0.0) return v;
    int ex;
    frexp(a, &ex);                  /* a in [2^(ex-1), 2^ex) */
    int e = ex - 1;                 /* floor(log2 a) */
    double step = ldexp(1.0, (e < -6 ? -6 : e) - 3);
    double q = a / step;            /* exact: step is a power of two */
    double f = floor(q), r = q - f;
    if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0)) f += 1.0;
    double m = f * step;
    if (m > 448.0) m = 448.0;
    return v < 0 ? -m : m;
}

/* OCP MX v1.0 conversion of a row of floats to MXFP8 (E4M3), blocks of 32
 * consecutive elements: the block's shared exponent is floor(log2 max|v|)
 * minus E4M3's largest exponent (8), clamped to E8M0's range [-127, 127] (an
 * all-zero block keeps exponent -127); each element is v / 2^shared rounded to
 * E4M3 and saturated.  xq receives the represented values q * 2^shared (the
 * activations an MXFP8 product consumes), exp the shared exponents. */
void oracle_quantize_mxfp8(int n, const double *x, double *xq, int32_t *exps)
{
    for (int b = 0; b < n / 32; b++) {
        const double *v = x + 32 * b;
        double amax = 0.0;
        for (int i = 0; i < 32; i++)
            if (fabs(v[i]) > amax) amax = fabs(v[i]);
        int se = -127;
        if (amax > 0.0) {
            int ex;
            frexp(amax, &ex);
            se = (ex - 1) - 8;
            if (se < -127) se = -127;
            if (se > 127) se = 127;
        }
        if (exps) exps[b] = se;
        for (int i = 0; i < 32; i++) xq[32 * b + i] = ldexp(round_e4m3(ldexp(v[i], -se)), se);
    }
}

/* ------------------------------------------------------------------ */
/* weight access                                                       */
/* ------------------------------------------------------------------ */

static void mat_shape(int mat, int H, int I, int *rows, int *cols)
{
    /* gate and up map the latent (in = H) to the intermediate (out = I);
     * down maps I back to H.  Stored [out][in], `in` contiguous. */
    if (mat == ORACLE_MAT_DOWN) { *rows = H; *cols = I; }
    else                        { *rows = I; *cols = H; }
}

/* Decode row `row` of matrix `mat` of expert `e` into out[cols] (exact). */
void oracle_decode_row(const oracle_weights *W, int mat, int e, int H, int I, int row, double *out)
{
    int rows, cols;
    mat_shape(mat, H, I, &rows, &cols);
    if (W->fmt == ORACLE_FMT_MXFP4) {
        /* codes [E][rows][cols/2]: byte j holds element 2j in its low nibble
         * and element 2j+1 in its high nibble; scales [E][rows][cols/32]:
         * one E8M0 byte per 32 consecutive elements along `in`. */
        const uint8_t *c = W->codes[mat] + ((size_t)e * rows + row) * (size_t)(cols / 2);
        const uint8_t *s = W->scales[mat] + ((size_t)e * rows + row) * (size_t)(cols / 32);
        for (int i = 0; i < cols; i++) {
            unsigned byte = c[i / 2];
            unsigned code = (i & 1) ? (byte >> 4) : (byte & 15u);
            out[i] = oracle_e2m1(code) * oracle_e8m0(s[i / 32]);
        }
    } else {
        /* RVQ3: idx [E][3][rows][cols/8] (stage-planar), codebooks
         * [E][3][256][8] fp16.  Elements 8v..8v+7 of a row form vector v and
         * equal the sum over the three stages of codebook_s[idx_s[row][v]]. */
        for (int v = 0; v < cols / 8; v++) {
            for (int d = 0; d < 8; d++) out[8 * v + d] = 0.0;
            for (int st = 0; st < 3; st++) {
                const uint8_t *ip = W->rvq_idx[mat] + (((size_t)e * 3 + st) * rows + row) * (size_t)(cols / 8);
                const uint16_t *cb = W->rvq_cb[mat] + (((size_t)e * 3 + st) * 256 + ip[v]) * 8;
                for (int d = 0; d < 8; d++) out[8 * v + d] += oracle_fp16(cb[d]);
            }
        }
    }
}

void oracle_decode_matrix(const oracle_weights *W, int mat, int e, int H, int I, double *out)
{
    int rows, cols;
    mat_shape(mat, H, I, &rows, &cols);
    for (int r = 0; r < rows; r++) oracle_decode_row(W, mat, e, H, I, r, out + (size_t)r * cols);
}

/* ------------------------------------------------------------------ */
/* a minimal thread pool over independent items                        */
/* ------------------------------------------------------------------ */

typedef void (*item_fn)(void *ctx, long item);
typedef struct { item_fn fn; void *ctx; long n; long next; pthread_mutex_t mu; } pool_t;

static void *pool_worker(void *arg)
{
    pool_t *p = (pool_t *)arg;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        long it = p->next++;
        pthread_mutex_unlock(&p->mu);
        if (it >= p->n) break;
        p->fn(p->ctx, it);
    }
    return NULL;
}

static void parallel_for(long n, int nthreads, item_fn fn, void *ctx)
{
    pool_t p = { fn, ctx, n, 0, PTHREAD_MUTEX_INITIALIZER };
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    pthread_t th[256];
    for (int i = 0; i < nthreads; i++) pthread_create(&th[i], NULL, pool_worker, &p);
    for (int i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------------ */
/* router                                                              */
/* ------------------------------------------------------------------ */

/* l[t][e] = sum_i x[t][i] * Wr[e][i], summed sequentially in i, plus b[e]
 * when a bias is given (the score-correction bias added to the logits). */
typedef struct { int H, E; const double *x, *wr, *bias; double *logits; } logit_ctx;

static void logits_token(void *vctx, long t)
{
    logit_ctx *c = (logit_ctx *)vctx;
    for (int e = 0; e < c->E; e++) {
        double acc = 0.0;
        for (int i = 0; i < c->H; i++) acc += c->x[(size_t)t * c->H + i] * c->wr[(size_t)e * c->H + i];
        if (c->bias) acc += c->bias[e];
        c->logits[(size_t)t * c->E + e] = acc;
    }
}

void oracle_router_logits(int T, int H, int E, const double *x, const double *wr, const double *bias,
                          double *logits, int nthreads)
{
    logit_ctx c = { H, E, x, wr, bias, logits };
    parallel_for(T, nthreads, logits_token, &c);
}

/* Expert a ranks ahead of expert b: larger logit first; equal logits (+0 and
 * -0 compare equal) go to the lower expert id. */
static int ranks_before(double la, int a, double lb, int b)
{
    return la > lb || (la == lb && a < b);
}

/* Top-k selection and softmax over the selected logits.
 * ids[t][j] in rank order; w[t][j] = exp(l_j - l_max) / sum_j' exp(l_j' - l_max).
 * Returns 0, or -1 on a non-finite logit or bad arguments. */
int oracle_topk_softmax(int T, int E, int k, const double *logits, int32_t *ids, double *w)
{
    if (k < 1 || k > E) return -1;
    char *taken = (char *)malloc((size_t)E);
    if (!taken) return -1;
    for (int t = 0; t < T; t++) {
        const double *l = logits + (size_t)t * E;
        for (int e = 0; e < E; e++)
            if (!isfinite(l[e])) { free(taken); return -1; }
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || ranks_before(l[e], e, l[best], best))) best = e;
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        double lmax = l[ids[(size_t)t * k]];
        double den = 0.0;
        for (int j = 0; j < k; j++) den += exp(l[ids[(size_t)t * k + j]] - lmax);
        for (int j = 0; j < k; j++) w[(size_t)t * k + j] = exp(l[ids[(size_t)t * k + j]] - lmax) / den;
    }
    free(taken);
    return 0;
}

/* Softmax of each token's logits over given experts (ids[t][0..k), in their
 * order): w[t][j] = exp(l_j - m) / sum_j' exp(l_j' - m), m the largest of
 * them.  With a selection-only router bias the ids come from the biased
 * logits and the weights from the unbiased ones (the bias corrects which
 * experts are chosen, not how they are combined). */
void oracle_softmax_at(int T, int E, int k, const double *logits, const int32_t *ids, double *w)
{
    for (int t = 0; t < T; t++) {
        const double *l = logits + (size_t)t * E;
        const int32_t *id = ids + (size_t)t * k;
        double m = l[id[0]];
        for (int j = 1; j < k; j++)
            if (l[id[j]] > m) m = l[id[j]];
        double den = 0.0;
        for (int j = 0; j < k; j++) den += exp(l[id[j]] - m);
        for (int j = 0; j < k; j++) w[(size_t)t * k + j] = exp(l[id[j]] - m) / den;
    }
}

/* ------------------------------------------------------------------ */
/* grouping                                                            */
/* ------------------------------------------------------------------ */

/* Token-to-expert grouping.  counts[e] = number of slots (t,j) routed to e;
 * offsets = exclusive prefix sum (E+1 entries); perm lists slot indices
 * t*k+j ordered by (expert asc, token asc, j asc); inv is its inverse;
 * active lists the experts with a nonzero count in ascending order and
 * *n_active is their number. */
void oracle_group(int T, int k, int E, const int32_t *ids, int32_t *counts, int32_t *offsets, int32_t *perm,
                  int32_t *inv, int32_t *active, int32_t *n_active)
{
    long S = (long)T * k;
    for (int e = 0; e < E; e++) counts[e] = 0;
    for (long s = 0; s < S; s++) counts[ids[s]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    long r = 0;
    for (int e = 0; e < E; e++)
        for (long s = 0; s < S; s++)
            if (ids[s] == e) { perm[r] = (int32_t)s; inv[s] = (int32_t)r; r++; }
    int u = 0;
    for (int e = 0; e < E; e++)
        if (counts[e] > 0) active[u++] = e;
    *n_active = u;
}

/* ------------------------------------------------------------------ */
/* experts                                                             */
/* ------------------------------------------------------------------ */

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* The gated activation h = act(g, u) and its partial derivatives.
 *   SwiGLU (the reading for the configs): h = g sigmoid(g) u.
 *   SiTU (LazyLoRA README, "File map", the K3 expert activation):
 *     h = A(g) B(u),  A(g) = 4 tanh(g / 4) sigmoid(g),  B(u) = 25 tanh(u / 25);
 *     dA/dg = sech^2(g / 4) sigmoid(g) + 4 tanh(g / 4) sigmoid(g) (1 - sigmoid(g)),
 *     dB/du = sech^2(u / 25). */
static double act_h(int act, double g, double u)
{
    if (act == ORACLE_ACT_SITU) return 4.0 * tanh(g / 4.0) * sigmoid(g) * (25.0 * tanh(u / 25.0));
    return g * sigmoid(g) * u;
}

static void act_grad(int act, double g, double u, double *dhdg, double *dhdu)
{
    double s = sigmoid(g);
    if (act == ORACLE_ACT_SITU) {
        double tg = tanh(g / 4.0), tu = tanh(u / 25.0);
        double cg = cosh(g / 4.0), cu = cosh(u / 25.0);  /* sech^2 = 1 / cosh^2 */
        *dhdg = (s / (cg * cg) + 4.0 * tg * s * (1.0 - s)) * (25.0 * tu);
        *dhdu = 4.0 * tg * s / (cu * cu);
        return;
    }
    *dhdg = u * s * (1.0 + g * (1.0 - s));
    *dhdu = g * s;
}

/* Low-rank adapter (LazyLoRA README, "LoRA": rank 16, alpha 32, one adapter
 * per layer in the latent space shared by all routed experts, on the expert
 * gate, up and down projections).  The adapted matrix is W + scale B A with
 * A [r][in], B [out][r]; the README gives rank and alpha, and the scale is
 * the usual LoRA alpha / r.  Applied to a vector z it adds scale B (A z),
 * which is what these two helpers compute. */

/* v = M z for M [r][n] (v has r entries). */
static void lr_in(int r, int n, const double *M, const double *z, double *v)
{
    for (int q = 0; q < r; q++) {
        double acc = 0.0;
        for (int i = 0; i < n; i++) acc += M[(size_t)q * n + i] * z[i];
        v[q] = acc;
    }
}

/* Row m of scale B v for B [rows][r]. */
static double lr_out(int r, double scale, const double *B, int m, const double *v)
{
    double acc = 0.0;
    for (int q = 0; q < r; q++) acc += B[(size_t)m * r + q] * v[q];
    return scale * acc;
}

/* One expert on one token: g = Wg x, u = Wu x, h = act(g, u) (SwiGLU:
 * silu(g) u with silu(g) = g sigmoid(g)), o = Wd h; with an adapter each
 * product W z becomes (W + scale B A) z = W z + scale B (A z).  Any output
 * pointer may be NULL. */
void oracle_expert_forward(const oracle_weights *W, int e, int H, int I, const double *x, double *g_out,
                           double *u_out, double *h_out, double *o_out)
{
    const oracle_lora *L = W->lora;
    int wmax = H > I ? H : I;
    double *row = (double *)malloc(sizeof(double) * (size_t)wmax);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    double va[64], vu[64], vd[64];
    if (L) {
        lr_in(L->r, H, L->A[ORACLE_MAT_GATE], x, va);
        lr_in(L->r, H, L->A[ORACLE_MAT_UP], x, vu);
    }
    for (int n = 0; n < I; n++) {
        double g = 0.0, u = 0.0;
        oracle_decode_row(W, ORACLE_MAT_GATE, e, H, I, n, row);
        for (int i = 0; i < H; i++) g += row[i] * x[i];
        oracle_decode_row(W, ORACLE_MAT_UP, e, H, I, n, row);
        for (int i = 0; i < H; i++) u += row[i] * x[i];
        if (L) {
            g += lr_out(L->r, L->scale, L->B[ORACLE_MAT_GATE], n, va);
            u += lr_out(L->r, L->scale, L->B[ORACLE_MAT_UP], n, vu);
        }
        h[n] = act_h(W->act, g, u);
        if (g_out) g_out[n] = g;
        if (u_out) u_out[n] = u;
    }
    if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
    if (o_out) {
        if (L) lr_in(L->r, I, L->A[ORACLE_MAT_DOWN], h, vd);
        for (int m = 0; m < H; m++) {
            double o = 0.0;
            oracle_decode_row(W, ORACLE_MAT_DOWN, e, H, I, m, row);
            for (int n = 0; n < I; n++) o += row[n] * h[n];
            if (L) o += lr_out(L->r, L->scale, L->B[ORACLE_MAT_DOWN], m, vd);
            o_out[m] = o;
        }
    }
    free(h);
    free(row);
}

typedef struct {
    const oracle_weights *W;
    int H, I, k;
    const double *x, *dy, *wr, *w;
    const int32_t *ids;
    double *o;      /* [slots][H] forward expert outputs */
    double *dxs;    /* [slots][H] backward per-slot input gradient */
    double *dp;     /* [slots] */
    double *keep;   /* [slots][3][I]: dL/dg, dL/du and h of each slot, or NULL */
} slot_ctx;

static void fwd_slot(void *vctx, long s)
{
    slot_ctx *c = (slot_ctx *)vctx;
    long t = s / c->k;
    oracle_expert_forward(c->W, c->ids[s], c->H, c->I, c->x + (size_t)t * c->H, NULL, NULL, NULL,
                          c->o + (size_t)s * c->H);
}

/* y[t] = sum over j in rank order of w[t][j] * expert_{ids[t][j]}(x[t]). */
void oracle_forward(int T, int H, int I, int k, const double *x, const int32_t *ids, const double *w,
                    const oracle_weights *W, double *y, int nthreads)
{
    long S = (long)T * k;
    double *o = (double *)malloc(sizeof(double) * (size_t)S * H);
    slot_ctx c = { W, H, I, k, x, NULL, NULL, w, ids, o, NULL, NULL, NULL };
    parallel_for(S, nthreads, fwd_slot, &c);
    for (int t = 0; t < T; t++)
        for (int m = 0; m < H; m++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++) acc += w[(size_t)t * k + j] * o[((size_t)t * k + j) * H + m];
            y[(size_t)t * H + m] = acc;
        }
    free(o);
}

/* Backward through one slot (t, j, e) with the upstream gradient dy[t]:
 *   a  = Wd^T dy                (reduces over the down matrix's rows)
 *   dp = <a, h>                 (= <dy, o>, the gradient w.r.t. the weight p)
 *   dh = p a
 *   dg = dh dh/dg,  du = dh dh/du   (SwiGLU: dg = dh u s (1 + g (1 - s)),
 *                                    du = dh g s, s = sigmoid(g); SiTU: act_grad)
 *   dx = Wg^T dg + Wu^T du      (reduces over the gate/up rows).
 * With an adapter every W above is W + scale B A, so Wd^T dy gains
 * scale A_d^T (B_d^T dy) and Wg^T dg gains scale A_g^T (B_g^T dg) (up alike). */
static void bwd_slot(void *vctx, long s)
{
    slot_ctx *c = (slot_ctx *)vctx;
    const oracle_lora *L = c->W->lora;
    int H = c->H, I = c->I, e = c->ids[s];
    long t = s / c->k;
    double p = c->w[s];
    const double *x = c->x + (size_t)t * H, *dy = c->dy + (size_t)t * H;
    int wmax = H > I ? H : I;
    double *g = (double *)malloc(sizeof(double) * (size_t)I);
    double *u = (double *)malloc(sizeof(double) * (size_t)I);
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    double *a = (double *)calloc((size_t)I, sizeof(double));
    double *dgv = (double *)malloc(sizeof(double) * (size_t)I);
    double *duv = (double *)malloc(sizeof(double) * (size_t)I);
    double *row = (double *)malloc(sizeof(double) * (size_t)wmax);
    double *dx = c->dxs + (size_t)s * H;
    oracle_expert_forward(c->W, e, H, I, x, g, u, h, NULL);
    for (int m = 0; m < H; m++) {
        oracle_decode_row(c->W, ORACLE_MAT_DOWN, e, H, I, m, row);
        for (int n = 0; n < I; n++) a[n] += row[n] * dy[m];
    }
    if (L) {
        /* a += scale A_d^T (B_d^T dy) */
        double bd[64];
        const double *Bd = L->B[ORACLE_MAT_DOWN], *Ad = L->A[ORACLE_MAT_DOWN];
        for (int q = 0; q < L->r; q++) {
            double acc = 0.0;
            for (int m = 0; m < H; m++) acc += Bd[(size_t)m * L->r + q] * dy[m];
            bd[q] = acc;
        }
        for (int n = 0; n < I; n++) {
            double acc = 0.0;
            for (int q = 0; q < L->r; q++) acc += Ad[(size_t)q * I + n] * bd[q];
            a[n] += L->scale * acc;
        }
    }
    double dp = 0.0;
    for (int n = 0; n < I; n++) dp += a[n] * h[n];
    c->dp[s] = dp;
    for (int i = 0; i < H; i++) dx[i] = 0.0;
    for (int n = 0; n < I; n++) {
        double dhdg, dhdu;
        act_grad(c->W->act, g[n], u[n], &dhdg, &dhdu);
        double dh = p * a[n];
        double dg = dh * dhdg;
        double du = dh * dhdu;
        dgv[n] = dg;
        duv[n] = du;
        oracle_decode_row(c->W, ORACLE_MAT_GATE, e, H, I, n, row);
        for (int i = 0; i < H; i++) dx[i] += row[i] * dg;
        oracle_decode_row(c->W, ORACLE_MAT_UP, e, H, I, n, row);
        for (int i = 0; i < H; i++) dx[i] += row[i] * du;
    }
    if (L) {
        /* dx += scale A_g^T (B_g^T dg) + scale A_u^T (B_u^T du) */
        for (int mat = ORACLE_MAT_GATE; mat <= ORACLE_MAT_UP; mat++) {
            const double *B = L->B[mat], *A = L->A[mat], *d = mat == ORACLE_MAT_GATE ? dgv : duv;
            for (int q = 0; q < L->r; q++) {
                double m = 0.0;
                for (int n = 0; n < I; n++) m += B[(size_t)n * L->r + q] * d[n];
                for (int i = 0; i < H; i++) dx[i] += L->scale * A[(size_t)q * H + i] * m;
            }
        }
    }
    if (c->keep) {
        double *kp = c->keep + (size_t)s * 3 * I;
        memcpy(kp, dgv, sizeof(double) * (size_t)I);
        memcpy(kp + I, duv, sizeof(double) * (size_t)I);
        memcpy(kp + 2 * (size_t)I, h, sizeof(double) * (size_t)I);
    }
    free(g); free(u); free(h); free(a); free(dgv); free(duv); free(row);
}

/* dX[t] = sum_j dx_tj + sum_j dl_tj * Wr[e_j], with the router term
 * dl_tj = p_tj (dp_tj - sum_j' p_tj' dp_tj') (softmax over the selected
 * logits; the selection itself is piecewise constant and has no gradient;
 * the bias does not depend on x). */
void oracle_backward_input(int T, int H, int I, int k, const double *x, const double *dy, const int32_t *ids,
                           const double *w, const double *wr, const oracle_weights *W, double *dx, int nthreads)
{
    long S = (long)T * k;
    double *dxs = (double *)malloc(sizeof(double) * (size_t)S * H);
    double *dp = (double *)malloc(sizeof(double) * (size_t)S);
    slot_ctx c = { W, H, I, k, x, dy, wr, w, ids, NULL, dxs, dp, NULL };
    parallel_for(S, nthreads, bwd_slot, &c);
    for (int t = 0; t < T; t++) {
        double pdp = 0.0;
        for (int j = 0; j < k; j++) pdp += w[(size_t)t * k + j] * dp[(size_t)t * k + j];
        for (int i = 0; i < H; i++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++) {
                size_t s = (size_t)t * k + j;
                double dl = w[s] * (dp[s] - pdp);
                acc += dxs[s * H + i] + dl * wr[(size_t)ids[s] * H + i];
            }
            dx[(size_t)t * H + i] = acc;
        }
    }
    free(dxs);
    free(dp);
}

/* Adapter gradients of L = sum_t <dy[t], y[t]>, y[t] = sum_j p_tj o_tj, routing
 * held fixed.  Per slot s = (t, j) with dL/dg = dg_s, dL/du = du_s and h_s from
 * the slot backward:
 *   g_s = Wg x_t + scale B_g (A_g x_t)  =>  dB_g += scale dg_s (A_g x_t)^T,
 *                                           dA_g += scale (B_g^T dg_s) x_t^T   (up alike);
 *   o_s = Wd h_s + scale B_d (A_d h_s) and dL/do_s = p_s dy_t
 *                                       =>  dB_d += scale p_s dy_t (A_d h_s)^T,
 *                                           dA_d += scale (B_d^T p_s dy_t) h_s^T.
 * Slots are summed in slot order. */
void oracle_lora_grads(int T, int H, int I, int k, const double *x, const double *dy, const int32_t *ids,
                       const double *w, const oracle_weights *W, double *dA[3], double *dB[3], int nthreads)
{
    const oracle_lora *L = W->lora;
    int r = L->r;
    double sc = L->scale;
    long S = (long)T * k;
    double *dxs = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1) * H);
    double *dp = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double *keep = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1) * 3 * I);
    slot_ctx c = { W, H, I, k, x, dy, NULL, w, ids, NULL, dxs, dp, keep };
    parallel_for(S, nthreads, bwd_slot, &c);
    memset(dA[ORACLE_MAT_GATE], 0, sizeof(double) * (size_t)r * H);
    memset(dA[ORACLE_MAT_UP], 0, sizeof(double) * (size_t)r * H);
    memset(dA[ORACLE_MAT_DOWN], 0, sizeof(double) * (size_t)r * I);
    memset(dB[ORACLE_MAT_GATE], 0, sizeof(double) * (size_t)I * r);
    memset(dB[ORACLE_MAT_UP], 0, sizeof(double) * (size_t)I * r);
    memset(dB[ORACLE_MAT_DOWN], 0, sizeof(double) * (size_t)H * r);
    double v[64], m[64];
    for (long s = 0; s < S; s++) {
        long t = s / k;
        double p = w[s];
        const double *xt = x + (size_t)t * H, *dyt = dy + (size_t)t * H;
        const double *ks = keep + (size_t)s * 3 * I;
        for (int mat = ORACLE_MAT_GATE; mat <= ORACLE_MAT_UP; mat++) {
            const double *d = ks + (mat == ORACLE_MAT_GATE ? 0 : I);
            const double *A = L->A[mat], *B = L->B[mat];
            lr_in(r, H, A, xt, v);                          /* A x_t */
            for (int q = 0; q < r; q++) {                   /* B^T d */
                double acc = 0.0;
                for (int n = 0; n < I; n++) acc += B[(size_t)n * r + q] * d[n];
                m[q] = acc;
            }
            for (int n = 0; n < I; n++)
                for (int q = 0; q < r; q++) dB[mat][(size_t)n * r + q] += sc * d[n] * v[q];
            for (int q = 0; q < r; q++)
                for (int i = 0; i < H; i++) dA[mat][(size_t)q * H + i] += sc * m[q] * xt[i];
        }
        {
            const double *h = ks + 2 * (size_t)I;
            const double *A = L->A[ORACLE_MAT_DOWN], *B = L->B[ORACLE_MAT_DOWN];
            lr_in(r, I, A, h, v);                           /* A_d h_s */
            for (int q = 0; q < r; q++) {                   /* B_d^T (p dy_t) */
                double acc = 0.0;
                for (int mm = 0; mm < H; mm++) acc += B[(size_t)mm * r + q] * p * dyt[mm];
                m[q] = acc;
            }
            for (int mm = 0; mm < H; mm++)
                for (int q = 0; q < r; q++) dB[ORACLE_MAT_DOWN][(size_t)mm * r + q] += sc * p * dyt[mm] * v[q];
            for (int q = 0; q < r; q++)
                for (int n = 0; n < I; n++) dA[ORACLE_MAT_DOWN][(size_t)q * I + n] += sc * m[q] * h[n];
        }
    }
    free(dxs);
    free(dp);
    free(keep);
}

/* ------------------------------------------------------------------ */
/* latent projections (dense bf16 matrices around the MoE)             */
/* ------------------------------------------------------------------ */

/* LazyLoRA README, "The engine": the latent MoE projections sit beside the
 * router gates among the dense (non-expert) weights; Two Desks, Act II: the
 * experts run in a latent space of width 3,584.  A projection is a plain
 * matrix product with bf16 weights w stored [N][K] (K contiguous):
 *   forward     out[t][n] = sum_k a[t][k] w[n][k]      (T x N)
 *   transposed  out[t][k] = sum_n a[t][n] w[n][k]      (T x K)
 * in fp64, each sum taken sequentially in index order. */
typedef struct { int T, N, K, transposed; const double *a; const uint16_t *w; double *out; } dense_ctx;

static double bf16_value(uint16_t b)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)b << 16;
    return (double)v.f;
}

static void dense_row(void *vctx, long t)
{
    const dense_ctx *c = (const dense_ctx *)vctx;
    if (!c->transposed) {
        for (int n = 0; n < c->N; n++) {
            double s = 0.0;
            for (int k = 0; k < c->K; k++) s += c->a[(size_t)t * c->K + k] * bf16_value(c->w[(size_t)n * c->K + k]);
            c->out[(size_t)t * c->N + n] = s;
        }
    } else {
        for (int k = 0; k < c->K; k++) {
            double s = 0.0;
            for (int n = 0; n < c->N; n++) s += c->a[(size_t)t * c->N + n] * bf16_value(c->w[(size_t)n * c->K + k]);
            c->out[(size_t)t * c->K + k] = s;
        }
    }
}

void oracle_dense(int T, int N, int K, const double *a, const uint16_t *w, double *out, int transposed, int nthreads)
{
    dense_ctx c = {T, N, K, transposed, a, w, out};
    parallel_for(T, nthreads, dense_row, &c);
}
