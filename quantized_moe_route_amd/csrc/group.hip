// group.hip -- token-to-expert grouping: histogram -> exclusive scan -> stable permute.
//
// Motivation (LazyLoRA README, "Measurement findings"): with a batch of tokens,
// reading every routed expert once in expert order and serving all of its
// tokens from that one read beats per-token reads; the expert kernels walk
// experts in ascending id and read
// each routed expert's bytes once for all of its tokens; this kernel builds
// that order.  Outputs: counts[e]; offsets = exclusive scan (E+1); perm = slot
// ids t*k+j ordered by (expert, token); inv = its inverse; active = experts
// with count > 0 ascending; *n_active.  Everything stays on the device.
//
// One workgroup of W waves.  Wave w owns a contiguous token range; it builds
// its own histogram in LDS, the per-(wave, expert) bases come from the global
// exclusive scan plus the counts of the earlier waves, and each wave then
// walks its tokens in order handing out positions.  The k slots of one token
// name distinct experts (the router selects without repetition), so the k
// lanes of one token never touch the same counter; tokens are visited one
// after another, which makes the order within each expert ascending in
// token.  Each counter advances in that fixed order, so the result is
// deterministic.
#include "common.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(1024) void k_group(const int32_t *__restrict__ ids, int T, int k, int E,
                                                int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                int32_t *__restrict__ active, int32_t *__restrict__ n_active)
{
    extern __shared__ int lds[];
    const int tid = threadIdx.x, nt = blockDim.x, nw = nt >> 6;
    const int lane = tid & 63, wv = tid >> 6;
    int *hist = lds;              // [nw][E]
    int *scr = lds + nw * E;      // [nt]
    for (int i = tid; i < nw * E; i += nt) hist[i] = 0;
    __syncthreads();

    const int tpw = (T + nw - 1) / nw;
    const int ta = min(T, wv * tpw), tb = min(T, ta + tpw);
    const long sa = (long)ta * k, sb = (long)tb * k;
    for (long s = sa + lane; s < sb; s += 64) atomicAdd(&hist[wv * E + ids[s]], 1);
    __syncthreads();

    // per-expert totals; each thread owns a run of consecutive experts
    const int per = (E + nt - 1) / nt;
    const int ea = min(E, tid * per), eb = min(E, ea + per);
    int my = 0, myact = 0;
    for (int e = ea; e < eb; e++) {
        int c = 0;
        for (int w = 0; w < nw; w++) c += hist[w * E + e];
        my += c;
        myact += c > 0;
    }
    int total;
    const int base = block_exclusive_scan(my, scr, &total);
    int abase_total;
    const int abase = block_exclusive_scan(myact, scr, &abase_total);
    int run = base, arun = abase;
    for (int e = ea; e < eb; e++) {
        int c = 0;
        for (int w = 0; w < nw; w++) {
            const int hw = hist[w * E + e];
            hist[w * E + e] = run + c;  // base of wave w for expert e
            c += hw;
        }
        counts[e] = c;
        offsets[e] = run;
        if (c > 0) active[arun++] = e;
        run += c;
    }
    if (tid == 0) {
        offsets[E] = total;
        *n_active = abase_total;
    }
    __syncthreads();

    // stable placement: the wave visits its tokens in order, B tokens per batch
    const int B = 64 / k;                 // tokens per 64-lane batch (k <= 64)
    const int span = B * k;
    const int my_tok = lane / k;
    for (long s0 = sa; s0 < sb; s0 += span) {
        const long s = s0 + lane;
        const bool valid = lane < span && s < sb;
        const int e = valid ? ids[s] : 0;
        for (int b = 0; b < B; b++) {
            if (valid && my_tok == b) {
                // atomics keep the per-counter order; distinct experts within a token never collide
                const int pos = atomicAdd(&hist[wv * E + e], 1);
                perm[pos] = (int32_t)s;
                inv[s] = pos;
            }
        }
    }
}

hipError_t launch_group(const GroupArgs &a, hipStream_t s)
{
    // 16 waves (fewer when their histograms would exceed 64 KB of LDS): the per-expert
    // sums and scans run over E whatever the slot count, so small batches gain from the
    // waves too
    int nw = 16;
    while (nw > 1 && (size_t)nw * a.E * 4 + (size_t)nw * 64 * 4 > 64 * 1024) nw >>= 1;
    const size_t lds = ((size_t)nw * a.E + (size_t)nw * 64) * sizeof(int);
    ProfScope ps(a.prof, PK_GROUP, s);
    ps.launch(k_group, dim3(1), dim3(nw * 64), lds, a.ids, a.T, a.k, a.E, a.counts, a.offsets, a.perm,
                       a.inv, a.active, a.n_active);
    return hipGetLastError();
}

// Slots t n_sh + j of the dense routing: token t takes expert j with weight 1; grouped by
// expert, expert j's rows are j T + t (token order).
__global__ __launch_bounds__(256) void k_dense_routing(int T, int n_sh, int32_t *__restrict__ ids, float *__restrict__ w,
                                                       int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                       int32_t *__restrict__ inv, int32_t *__restrict__ active,
                                                       int32_t *__restrict__ n_active)
{
    const long n = (long)T * n_sh;
    for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const int t = (int)(i / n_sh), j = (int)(i - (long)t * n_sh);
        const int32_t r = j * T + t;
        ids[i] = j;
        w[i] = 1.f;
        inv[i] = r;
        perm[r] = (int32_t)i;
    }
    if (blockIdx.x == 0 && threadIdx.x <= n_sh) {
        offsets[threadIdx.x] = (int32_t)threadIdx.x * T;
        if (threadIdx.x < n_sh) active[threadIdx.x] = (int32_t)threadIdx.x;
        if (threadIdx.x == 0) *n_active = n_sh;
    }
}

hipError_t launch_dense_routing(int T, int n_sh, int32_t *ids, float *w, int32_t *offsets, int32_t *perm, int32_t *inv,
                                int32_t *active, int32_t *n_active, hipStream_t s)
{
    const long n = (long)T * n_sh;
    const long nb = (n + 255) / 256;
    const int blocks = (int)(nb < 1024 ? nb : 1024);
    hipLaunchKernelGGL(k_dense_routing, dim3(blocks < 1 ? 1 : blocks), dim3(256), 0, s, T, n_sh, ids, w, offsets, perm,
                       inv, active, n_active);
    return hipGetLastError();
}

}  // namespace moe
