// moe_api.hip -- the C ABI declared in include/moe.h: argument validation,
// workspace carving and kernel launches on the caller's stream.
//
// API shape after the WASTE README (hackernews.jp story 49123386): a config
// struct with an init function for defaults, a create call that returns a
// status and fills an out-handle, and a destroy call.  A missing input is an
// error, never replaced (LazyLoRA README, "Three rules the engine is built
// around").
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "moe.h"
#include "moe_internal.h"
#include "moe_prof.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

constexpr int kMaxExperts = 2048;
constexpr int kMaxTopK = 64;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
    size_t logits, beta, h, ybuf, gu, dgdu, dp, xq, xqs;
    size_t l_vx, l_gu, l_hbar, l_z, l_wd, l_c, l_dgu, l_m, l_part;  // adapter (MOE_F_LORA)
    size_t xq8;  // MXFP8-quantized activations as bf16 (MOE_F_QUANT_X8)
    // shared experts: their slot rows (forward outputs, backward input-gradient rows) and
    // their dense routing; the rest of their scratch is the routed slots' (n_shared <= k)
    size_t sh_rows, sh_ids, sh_w, sh_off, sh_perm, sh_inv, sh_act, sh_nact, sh_h;
    size_t status;    // the device status word (MOE_F_VALIDATE findings, internal timeouts)
    size_t dec_sync;  // counters of the fused few-token launch (zero between launches)
    size_t lut_ord;   // the RVQ3 table-lookup launches' unit order [S] int32
    size_t total;
};

constexpr int kMaxLoraRank = 64;
constexpr size_t kLoraPartFloats = (size_t)4 << 20;  // split-K partial sums of the adapter GEMMs

Layout layout_of(const moe_desc &d)
{
    const size_t T = (size_t)d.max_tokens, S = T * (size_t)d.top_k;
    const size_t H = (size_t)d.hidden, I = (size_t)d.inter, E = (size_t)d.n_experts;
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    L.logits = take(T * E * 4);
    L.beta = take(T * E * 4);
    L.h = take(S * I * 4);
    L.ybuf = take(S * H * 4);
    L.gu = take(S * 2 * I * 4);
    L.dgdu = take(S * 2 * I * 4);
    L.dp = take(S * (size_t)moe::dp_tiles((int)I) * 4);
    const bool mx = (d.flags & MOE_F_MX_GATEUP) != 0;
    L.xq = take(mx ? T * H * 2 : 0);
    L.xqs = take(mx ? T * (H / 32) * 2 : 0);
    const bool lo = (d.flags & MOE_F_LORA) != 0;
    const size_t R = lo ? kMaxLoraRank : 0, Tl = lo ? T : 0;
    L.l_vx = take(Tl * 2 * R * 4);
    L.l_gu = take(Tl * 2 * I * 4);
    L.l_hbar = take(Tl * I * 4);
    L.l_z = take(Tl * R * 4);
    L.l_wd = take(Tl * R * 4);
    L.l_c = take(Tl * I * 4);
    L.l_dgu = take(Tl * 2 * I * 4);
    L.l_m = take(Tl * 2 * R * 4);
    L.l_part = take(lo ? kLoraPartFloats * 4 : 0);
    L.xq8 = take((d.flags & MOE_F_QUANT_X8) ? T * H * 2 : 0);
    const size_t NS = (size_t)d.n_shared, Ssh = T * NS;
    L.sh_rows = take(Ssh * H * 4);
    L.sh_ids = take(Ssh * 4);
    L.sh_w = take(Ssh * 4);
    L.sh_off = take(NS ? (NS + 1) * 4 : 0);
    L.sh_perm = take(Ssh * 4);
    L.sh_inv = take(Ssh * 4);
    L.sh_act = take(NS * 4);
    L.sh_nact = take(NS ? 4 : 0);
    L.sh_h = take(std::min<size_t>(T, 16) * NS * I * 4);  // h planes of the shared units of the few-token launch
    L.status = take(4);
    L.dec_sync = take((size_t)moe::kSyncWords * 4);
    L.lut_ord = take(S * 4);
    L.total = off;
    return L;
}

moe_status check_desc(const moe_desc *d)
{
    if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
    if (d->hidden <= 0 || d->hidden % 32) return fail(MOE_ERR_INVALID_ARG, "hidden=%d must be a positive multiple of 32", d->hidden);
    if (d->inter <= 0 || d->inter % 32) return fail(MOE_ERR_INVALID_ARG, "inter=%d must be a positive multiple of 32", d->inter);
    if (d->n_experts < 1 || d->n_experts > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "n_experts=%d must be in 1..%d", d->n_experts, kMaxExperts);
    if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > kMaxTopK)
        return fail(MOE_ERR_INVALID_ARG, "top_k=%d must be in 1..min(n_experts, %d)", d->top_k, kMaxTopK);
    if (d->max_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "max_tokens=%d is negative", d->max_tokens);
    if ((long long)d->max_tokens * d->top_k > (1LL << 30))
        return fail(MOE_ERR_INVALID_ARG, "max_tokens*top_k exceeds 2^30");
    if (d->wfmt != MOE_W_MXFP4 && d->wfmt != MOE_W_RVQ3) return fail(MOE_ERR_INVALID_ARG, "unknown wfmt %d", d->wfmt);
    if (d->act != MOE_ACT_SWIGLU && d->act != MOE_ACT_SITU)
        return fail(MOE_ERR_UNSUPPORTED, "activation %d is not implemented", d->act);
    if (d->bias_mode < 0 || d->bias_mode > 2)
        return fail(MOE_ERR_UNSUPPORTED, "bias_mode %d is not implemented", d->bias_mode);
    if (d->n_shared < 0 || d->n_shared > d->top_k)
        return fail(MOE_ERR_INVALID_ARG, "n_shared=%d must be in 0..top_k=%d", d->n_shared, d->top_k);
    if (d->model_width < 0 || d->model_width % 64 || (d->model_width > 0 && d->hidden % 64))
        return fail(MOE_ERR_INVALID_ARG, "model_width=%d must be 0 or a multiple of 64 (with hidden a multiple of 64)",
                    d->model_width);
    return MOE_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_dtype(int32_t dt, const char *what)
{
    if (dt != MOE_DT_F32 && dt != MOE_DT_BF16) return fail(MOE_ERR_INVALID_ARG, "%s dtype %d is not f32/bf16", what, dt);
    return MOE_OK;
}

moe_status device_status(hipError_t e, const char *where)
{
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

}  // namespace

struct moe_layer {
    moe_desc d;
    moe_weights w;
    char *ws;
    size_t ws_bytes;
    Layout lay;
    moe::Prof prof;
    bool has_lora = false;
    moe::LoraW lora{};
    bool status_armed = false;  // the status word has been cleared once
    bool sync_armed = false;    // the fused launch's counters have been cleared once
};

namespace {

void prof_release(moe::Prof &p)
{
    for (int k = 0; k < moe::PK_N; k++) {
        for (hipEvent_t e : p.ev[k])
            if (e) hipEventDestroy(e);
        p.ev[k].clear();
        p.n[k] = 0;
    }
    p.mask = 0;
    p.cap = 0;
}

}  // namespace

namespace {

moe::LoraWs lora_ws(const moe_layer *L)
{
    moe::LoraWs w{};
    char *b = L->ws;
    w.vx = (float *)(b + L->lay.l_vx);
    w.gu = (float *)(b + L->lay.l_gu);
    w.hbar = (float *)(b + L->lay.l_hbar);
    w.z = (float *)(b + L->lay.l_z);
    w.wd = (float *)(b + L->lay.l_wd);
    w.c = (float *)(b + L->lay.l_c);
    w.dgu = (float *)(b + L->lay.l_dgu);
    w.m = (float *)(b + L->lay.l_m);
    w.part = (float *)(b + L->lay.l_part);
    w.part_cap = kLoraPartFloats;
    return w;
}

moe_status check_layer(const moe_layer *L)
{
    if (!L) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
    return MOE_OK;
}

moe_status check_routing(const moe_routing *r)
{
    if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
    if (!r->ids || !r->w || !r->counts || !r->offsets || !r->perm || !r->inv || !r->active || !r->n_active)
        return fail(MOE_ERR_INVALID_ARG, "a routing buffer is NULL");
    return MOE_OK;
}

moe_status check_tokens(const moe_layer *L, int32_t T)
{
    if (T < 0 || T > L->d.max_tokens)
        return fail(MOE_ERR_INVALID_ARG, "T=%d must be in 0..max_tokens=%d", T, L->d.max_tokens);
    return MOE_OK;
}

moe::MatW matw(const moe_weights &w, int m)
{
    moe::MatW r;
    r.codes = w.codes[m];
    r.scales = w.scales[m];
    r.idx = w.rvq_idx[m];
    r.cb = w.rvq_cb[m];
    return r;
}

moe::MatW shared_matw(const moe_weights &w, int m)
{
    moe::MatW r;
    r.codes = w.shared_codes[m];
    r.scales = w.shared_scales[m];
    r.idx = w.shared_rvq_idx[m];
    r.cb = w.shared_rvq_cb[m];
    return r;
}

// The shared experts' dense routing for T tokens, written into the workspace.
struct DenseRouting {
    int32_t *ids, *off, *perm, *inv, *act, *nact;
    float *w;
};

hipError_t dense_routing(const moe_layer *L, int T, DenseRouting &r, hipStream_t s)
{
    char *b = L->ws;
    r.ids = (int32_t *)(b + L->lay.sh_ids);
    r.w = (float *)(b + L->lay.sh_w);
    r.off = (int32_t *)(b + L->lay.sh_off);
    r.perm = (int32_t *)(b + L->lay.sh_perm);
    r.inv = (int32_t *)(b + L->lay.sh_inv);
    r.act = (int32_t *)(b + L->lay.sh_act);
    r.nact = (int32_t *)(b + L->lay.sh_nact);
    return moe::launch_dense_routing(T, L->d.n_shared, r.ids, r.w, r.off, r.perm, r.inv, r.act, r.nact, s);
}

int tok_chunks(int T) { return (T + moe::kTokChunk - 1) / moe::kTokChunk; }

bool validating(const moe_layer *L) { return (L->d.flags & MOE_F_VALIDATE) != 0; }

uint32_t *status_word(const moe_layer *L) { return (uint32_t *)(L->ws + L->lay.status); }

std::string bad_bits_text(uint32_t b)
{
    static const char *names[] = {"non-finite x", "non-finite dy", "E8M0 scale byte 0xFF (NaN)",
                                  "E8M0 scale byte 0x00 (2^-127)", "non-finite RVQ3 codeword"};
    std::string t;
    for (int i = 0; i < 5; i++)
        if ((b >> i) & 1u) t += (t.empty() ? "" : ", ") + std::string(names[i]);
    if (b & moe::kStatusSpinTimeout) t += (t.empty() ? "" : ", ") + std::string("a fused decode launch gave up waiting (internal)");
    return t;
}

// MOE_F_VALIDATE: reads (host synchronization) and clears the status word left by the
// earlier calls; MOE_ERR_DATA if it was set.  The first call only clears it.
moe_status take_status(moe_layer *L, hipStream_t s, uint32_t *bits_out)
{
    uint32_t bits = 0;
    if (L->status_armed) {
        hipError_t e = hipMemcpyAsync(&bits, status_word(L), 4, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return device_status(e, "reading the validation status");
    }
    if (bits_out) *bits_out = bits;
    if (!L->status_armed || bits) {
        moe_status st = device_status(moe::launch_set_u32(status_word(L), 0u, s), "clearing the validation status");
        if (st != MOE_OK) return st;
        L->status_armed = true;
    }
    if (bits & moe::kStatusSpinTimeout)
        return fail(MOE_ERR_INTERNAL, "an earlier call failed on the device: %s", bad_bits_text(bits).c_str());
    if (bits) return fail(MOE_ERR_DATA, "out-of-contract data found by an earlier call: %s", bad_bits_text(bits).c_str());
    return MOE_OK;
}

size_t mat_scale_bytes(const moe_desc &d, int m)
{
    const size_t rows = m < 2 ? d.inter : d.hidden, cols = m < 2 ? d.hidden : d.inter;
    return rows * (cols / 32);
}

// MOE_F_VALIDATE: scan the weights a forward or backward pass reads (active routed experts
// of r, and the shared experts).
moe_status check_weights(const moe_layer *L, const moe_routing *r, int T, hipStream_t s)
{
    const moe_desc &d = L->d;
    const size_t sb[3] = {mat_scale_bytes(d, 0), mat_scale_bytes(d, 1), mat_scale_bytes(d, 2)};
    const moe::MatW m[3] = {matw(L->w, 0), matw(L->w, 1), matw(L->w, 2)};
    const int units = (int)std::min<long long>(d.n_experts, (long long)T * d.top_k);
    moe_status st = device_status(moe::launch_check_weights(d.wfmt, m, sb, r->active, r->n_active, units,
                                                            status_word(L), s), "validating the expert weights");
    if (st != MOE_OK || d.n_shared == 0) return st;
    const moe::MatW ms[3] = {shared_matw(L->w, 0), shared_matw(L->w, 1), shared_matw(L->w, 2)};
    return device_status(moe::launch_check_weights(d.wfmt, ms, sb, nullptr, nullptr, d.n_shared, status_word(L), s),
                         "validating the shared experts");
}

}  // namespace

extern "C" {

void moe_desc_init(moe_desc *d)
{
    if (!d) return;
    std::memset(d, 0, sizeof *d);
    d->hidden = 3584;
    d->inter = 3072;
    d->n_experts = 896;
    d->top_k = 16;
    d->max_tokens = 4096;
    d->wfmt = MOE_W_MXFP4;
    d->act = MOE_ACT_SWIGLU;
    d->bias_mode = 0;
    d->flags = MOE_F_DETERMINISTIC;
}

moe_status moe_workspace_size(const moe_desc *d, size_t *bytes)
{
    g_last_error.clear();
    moe_status st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = layout_of(*d).total;
    return MOE_OK;
}

moe_status moe_layer_create(const moe_desc *d, const moe_weights *w, void *workspace, size_t ws_bytes,
                            moe_layer **out)
{
    g_last_error.clear();
    moe_status st = check_desc(d);
    if (st != MOE_OK) return st;
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if (!w->router_w) return fail(MOE_ERR_INVALID_ARG, "router_w is NULL");
    if (!aligned(w->router_w, 16)) return fail(MOE_ERR_INVALID_ARG, "router_w must be 16-byte aligned");
    if (d->bias_mode != 0 && !w->router_b) return fail(MOE_ERR_INVALID_ARG, "bias_mode=%d needs router_b", d->bias_mode);
    static const char *names[3] = {"gate", "up", "down"};
    for (int m = 0; m < 3; m++) {
        if (d->wfmt == MOE_W_MXFP4) {
            if (!w->codes[m] || !w->scales[m]) return fail(MOE_ERR_INVALID_ARG, "%s codes/scales missing", names[m]);
            if (!aligned(w->codes[m], 16) || !aligned(w->scales[m], 16))
                return fail(MOE_ERR_INVALID_ARG, "%s codes and scales must be 16-byte aligned", names[m]);
        } else {
            if (!w->rvq_idx[m] || !w->rvq_cb[m]) return fail(MOE_ERR_INVALID_ARG, "%s rvq_idx/rvq_cb missing", names[m]);
            if (!aligned(w->rvq_idx[m], 16) || !aligned(w->rvq_cb[m], 16))
                return fail(MOE_ERR_INVALID_ARG, "%s rvq_idx/rvq_cb must be 16-byte aligned", names[m]);
        }
        if (d->n_shared == 0) continue;
        if (d->wfmt == MOE_W_MXFP4) {
            if (!w->shared_codes[m] || !w->shared_scales[m])
                return fail(MOE_ERR_INVALID_ARG, "shared %s codes/scales missing", names[m]);
            if (!aligned(w->shared_codes[m], 16) || !aligned(w->shared_scales[m], 16))
                return fail(MOE_ERR_INVALID_ARG, "shared %s codes and scales must be 16-byte aligned", names[m]);
        } else {
            if (!w->shared_rvq_idx[m] || !w->shared_rvq_cb[m])
                return fail(MOE_ERR_INVALID_ARG, "shared %s rvq_idx/rvq_cb missing", names[m]);
            if (!aligned(w->shared_rvq_idx[m], 16) || !aligned(w->shared_rvq_cb[m], 16))
                return fail(MOE_ERR_INVALID_ARG, "shared %s rvq_idx/rvq_cb must be 16-byte aligned", names[m]);
        }
    }
    if (d->model_width > 0) {
        if (!w->proj_in || !w->proj_out) return fail(MOE_ERR_INVALID_ARG, "model_width > 0 needs proj_in and proj_out");
        if (!aligned(w->proj_in, 16) || !aligned(w->proj_out, 16))
            return fail(MOE_ERR_INVALID_ARG, "proj_in and proj_out must be 16-byte aligned");
    }
    const Layout lay = layout_of(*d);
    if (!workspace && lay.total > 0) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (ws_bytes < lay.total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, lay.total);
    if (!aligned(workspace, 256)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    moe_layer *L = new (std::nothrow) moe_layer;
    if (!L) return fail(MOE_ERR_INTERNAL, "out of host memory");
    L->d = *d;
    L->w = *w;
    L->ws = (char *)workspace;
    L->ws_bytes = ws_bytes;
    L->lay = lay;
    *out = L;
    return MOE_OK;
}

moe_status moe_route(moe_layer *L, const void *x, int32_t xt, int32_t T, const moe_routing *r, void *stream)
{
    g_last_error.clear();
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK || (st = check_tokens(L, T)) != MOE_OK || (st = check_dtype(xt, "x")) != MOE_OK)
        return st;
    if (T == 0) return MOE_OK;
    if ((st = check_routing(r)) != MOE_OK) return st;
    if (!x) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
    if (!aligned(x, 16)) return fail(MOE_ERR_INVALID_ARG, "x must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    if (validating(L)) {
        if ((st = take_status(L, s, nullptr)) != MOE_OK) return st;
        if ((st = device_status(moe::launch_check_finite(x, xt, (size_t)T * L->d.hidden, status_word(L), MOE_BAD_X, s),
                                "validating x")) != MOE_OK)
            return st;
    }
    moe::RouteArgs a{};
    a.x = x;
    a.xt = xt;
    a.wr = L->w.router_w;
    a.bias = L->d.bias_mode != 0 ? L->w.router_b : nullptr;
    a.wbias = L->d.bias_mode == 2 ? L->w.router_b : nullptr;
    a.T = T;
    a.H = L->d.hidden;
    a.E = L->d.n_experts;
    a.k = L->d.top_k;
    a.logits = (float *)(L->ws + L->lay.logits);
    a.beta = (float *)(L->ws + L->lay.beta);
    // the backward's dg/du region is free while routing: the split-K router's partial sums
    a.rpart = (double *)(L->ws + L->lay.dgdu);
    a.rpart_bytes = (size_t)L->d.max_tokens * L->d.top_k * 2 * L->d.inter * 4;
    a.ids = r->ids;
    a.w = r->w;
    a.refined = nullptr;
    a.prof = &L->prof;
    moe::GroupArgs gq{};
    gq.ids = r->ids;
    gq.T = T;
    gq.k = a.k;
    gq.E = a.E;
    gq.counts = r->counts;
    gq.offsets = r->offsets;
    gq.perm = r->perm;
    gq.inv = r->inv;
    gq.active = r->active;
    gq.n_active = r->n_active;
    gq.prof = &L->prof;
    if (moe::route_small_ok(a)) return device_status(moe::launch_route_small(a, gq, s), "route");
    if ((st = device_status(moe::launch_router(a, s), "router")) != MOE_OK) return st;
    return device_status(moe::launch_group(gq, s), "group");
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Scratch of moe_forward_static: one array per GPU, part of the library's code object, so
// that call allocates nothing.  Every call on a GPU uses that GPU's copy, which keeps the last
// call's contents; calls that overlap on one GPU race on it.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// The device address of the current device's copy of `scratch`, looked up once per device
// with that device current (in host code the array's name is only a stand-in for it).
moe_status static_scratch(char **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d is beyond the %d tracked", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return device_status(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *out = (char *)g_scratch_ptr[dev];
    return MOE_OK;
}

// Carving of `scratch` for T tokens: status word, counters of the fused few-token launch
// and of the table-lookup launches, h as bf16 hi + lo planes [S][I] (RVQ3: the same region,
// twice the size, holds g and u [S][2][I] fp32 for the table-lookup kernels, which take no h
// planes), weighted slot rows [S][H] fp32, the table-lookup unit order [S] (S = T k).
struct StaticLayout {
    size_t status, sync, h, ybuf, ord, total;
};

StaticLayout static_layout(const moe_desc &d, int T)
{
    StaticLayout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    const size_t S = (size_t)T * d.top_k;
    l.status = take(4);
    l.sync = take((size_t)moe::kSyncWords * 4);
    l.h = take(S * d.inter * (d.wfmt == MOE_W_RVQ3 ? 8 : 4));
    l.ybuf = take(S * d.hidden * 4);
    l.ord = take(S * 4);
    l.total = off;
    return l;
}

}  // namespace

namespace {

// Kernel arguments of the routed forward common to every entry point: weights, shapes,
// routing, output, activation; the scratch pointers are the caller's to fill.
moe::ExpertFwdArgs routed_fwd_args(moe_layer *L, const void *x, int32_t xt, int32_t T, const moe_routing *r, float *y)
{
    moe::ExpertFwdArgs a{};
    a.wfmt = L->d.wfmt;
    a.gate = matw(L->w, 0);
    a.up = matw(L->w, 1);
    a.down = matw(L->w, 2);
    a.x = x;
    a.xt = xt;
    a.T = T;
    a.H = L->d.hidden;
    a.I = L->d.inter;
    a.E = L->d.n_experts;
    a.k = L->d.top_k;
    a.offsets = r->offsets;
    a.perm = r->perm;
    a.active = r->active;
    a.n_active = r->n_active;
    a.w = r->w;
    a.y = y;
    a.act = L->d.act;
    a.prof = &L->prof;
    return a;
}

}  // namespace

extern "C" {

moe_status moe_forward(moe_layer *L, const void *x, int32_t xt, int32_t T, const moe_routing *r, float *y,
                       float *saved_gu, void *stream)
{
    g_last_error.clear();
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK || (st = check_tokens(L, T)) != MOE_OK || (st = check_dtype(xt, "x")) != MOE_OK)
        return st;
    if (T == 0) return MOE_OK;
    if ((st = check_routing(r)) != MOE_OK) return st;
    if (!x || !y) return fail(MOE_ERR_INVALID_ARG, "x or y is NULL");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(MOE_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if (saved_gu && !aligned(saved_gu, 16)) return fail(MOE_ERR_INVALID_ARG, "saved_gu must be 16-byte aligned");
    if (validating(L)) {
        if ((st = take_status(L, (hipStream_t)stream, nullptr)) != MOE_OK) return st;
        if ((st = check_weights(L, r, T, (hipStream_t)stream)) != MOE_OK) return st;
    }
    moe::ExpertFwdArgs a = routed_fwd_args(L, x, xt, T, r, y);
    a.h_hi = (uint16_t *)(L->ws + L->lay.h);
    a.h_lo = a.h_hi + (size_t)T * a.k * a.I;
    a.gu = saved_gu;
    a.gu_ws = (float *)(L->ws + L->lay.gu);
    if (!(L->d.flags & MOE_F_RVQ_GATHER)) a.lut_ord = (int32_t *)(L->ws + L->lay.lut_ord);
    a.ybuf = (float *)(L->ws + L->lay.ybuf);
    if (L->d.flags & MOE_F_MX_GATEUP) {
        a.xq = (uint8_t *)(L->ws + L->lay.xq);
        a.xq_s = (uint8_t *)(L->ws + L->lay.xqs);
    }
    const hipStream_t hs = (hipStream_t)stream;
    a.dec_sync = (uint32_t *)(L->ws + L->lay.dec_sync);
    a.status = status_word(L);
    if (!L->sync_armed || !L->status_armed) {
        // the first forward on a layer clears the counters of the fused few-token launch
        // (which keep themselves at zero afterwards) and the status word
        if ((st = device_status(moe::fill_zero((float *)a.dec_sync, moe::kSyncWords, hs), "clearing counters")) != MOE_OK)
            return st;
        if (!L->status_armed &&
            (st = device_status(moe::launch_set_u32(a.status, 0u, hs), "clearing the status word")) != MOE_OK)
            return st;
        L->sync_armed = L->status_armed = true;
    }
    if (L->d.flags & MOE_F_QUANT_X8) {
        // the experts (and the adapter) see x quantized to MXFP8; the routing came from x
        uint16_t *xq = (uint16_t *)(L->ws + L->lay.xq8);
        // with the block-scaled gate/up the same pass writes its operand: one exact E4M3 term
        a.xq_single = a.xq != nullptr;
        if ((st = device_status(moe::launch_quant_x8(x, xt, T, a.H, xq, a.xq, a.xq_s, hs), "quantize x")) != MOE_OK)
            return st;
        a.x = xq;
        a.xt = MOE_DT_BF16;  // the same code as the kernels' bf16 token type
        x = xq;
        xt = MOE_DT_BF16;
    }
    moe::set_lds_staging(a);
    if (L->d.n_shared > 0 && !moe::use_mm(a) && moe::dec_supported(a)) {
        // few tokens: the shared experts are extra units of the routed stream kernels' launch
        a.sh_n = L->d.n_shared;
        a.sh_gate = shared_matw(L->w, 0);
        a.sh_up = shared_matw(L->w, 1);
        a.sh_down = shared_matw(L->w, 2);
        a.sh_h_hi = (uint16_t *)(L->ws + L->lay.sh_h);
        a.sh_h_lo = a.sh_h_hi + (size_t)T * a.sh_n * a.I;
        a.sh_ybuf = (float *)(L->ws + L->lay.sh_rows);
        a.ybuf2 = a.sh_ybuf;
        a.k2 = a.sh_n;
    } else if (L->d.n_shared > 0) {
        // the shared experts first: their slot rows stay in the workspace for the combine
        DenseRouting dr;
        if ((st = device_status(dense_routing(L, T, dr, hs), "shared-expert routing")) != MOE_OK) return st;
        moe::ExpertFwdArgs sa = a;
        sa.gate = shared_matw(L->w, 0);
        sa.up = shared_matw(L->w, 1);
        sa.down = shared_matw(L->w, 2);
        sa.E = sa.k = L->d.n_shared;
        sa.offsets = dr.off;
        sa.perm = dr.perm;
        sa.active = dr.act;
        sa.n_active = dr.nact;
        sa.w = dr.w;
        sa.h_lo = sa.h_hi + (size_t)T * sa.k * sa.I;
        sa.gu = nullptr;
        sa.gu_ws = nullptr;  // sized for the routed slots; the shared units take other kernels
        sa.lut_ord = nullptr;
        sa.ybuf = (float *)(L->ws + L->lay.sh_rows);
        sa.tok_chunks = tok_chunks(T);
        sa.skip_combine = 1;
        moe::set_lds_staging(sa);
        if ((st = device_status(moe::launch_expert_forward(sa, hs), "shared experts")) != MOE_OK) return st;
        a.ybuf2 = sa.ybuf;
        a.k2 = sa.k;
    }
    moe::set_lds_staging(a);
    if (!L->has_lora) return device_status(moe::launch_expert_forward(a, hs), "forward");
    const moe::LoraWs lw = lora_ws(L);
    if (!moe::use_mm(a) && moe::dec_supported(a) && moe::dec_fused_ok(a) &&
        (size_t)T * a.k * L->lora.r * (a.I / 64) <= lw.part_cap) {
        // the fused few-token launch forms the adapter's gate/up and down terms itself from
        // vx = [A_g x | A_u x]; its partials of A_d hbar go to the adapter's split-K region
        if ((st = device_status(moe::lora_forward_vx(L->lora, lw, x, xt, T, a.H, hs), "adapter (A x)")) != MOE_OK)
            return st;
        a.lora_vx = lw.vx;
        a.lora_Bg = L->lora.B[0];
        a.lora_Bu = L->lora.B[1];
        a.lora_Ad = L->lora.A[2];
        a.lora_Bd = L->lora.B[2];
        a.lora_r = L->lora.r;
        a.lora_scale = L->lora.scale;
        a.lora_zp = lw.part;
        a.lora_z = lw.z;
        return device_status(moe::launch_expert_forward(a, hs), "forward");
    }
    if ((st = device_status(moe::lora_forward_pre(L->lora, lw, x, xt, T, a.H, a.I, hs), "adapter (gate/up terms)")) != MOE_OK)
        return st;
    a.lora_gu = lw.gu;
    if ((st = device_status(moe::launch_expert_forward(a, hs), "forward")) != MOE_OK) return st;
    return device_status(moe::lora_forward_post(L->lora, lw, a, r->inv, hs), "adapter (down term)");
}

namespace {

// Input gradient, and the adapter gradients when dA is not NULL.
moe_status backward_impl(moe_layer *L, const void *x, int32_t xt, const void *dy, int32_t dyt, int32_t T,
                         const moe_routing *r, const float *saved_gu, float *dx, float *const *dA, float *const *dB,
                         void *stream)
{
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK || (st = check_tokens(L, T)) != MOE_OK || (st = check_dtype(xt, "x")) != MOE_OK ||
        (st = check_dtype(dyt, "dy")) != MOE_OK)
        return st;
    if (T == 0) return MOE_OK;
    if ((st = check_routing(r)) != MOE_OK) return st;
    if (!x || !dy || !dx) return fail(MOE_ERR_INVALID_ARG, "x, dy or dx is NULL");
    if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16))
        return fail(MOE_ERR_INVALID_ARG, "x, dy and dx must be 16-byte aligned");
    if (saved_gu && !aligned(saved_gu, 16)) return fail(MOE_ERR_INVALID_ARG, "saved_gu must be 16-byte aligned");
    if (validating(L)) {
        const hipStream_t s = (hipStream_t)stream;
        if ((st = take_status(L, s, nullptr)) != MOE_OK) return st;
        if ((st = device_status(moe::launch_check_finite(dy, dyt, (size_t)T * L->d.hidden, status_word(L), MOE_BAD_DY, s),
                                "validating dy")) != MOE_OK)
            return st;
        if ((st = check_weights(L, r, T, s)) != MOE_OK) return st;
    }
    moe::ExpertBwdArgs a{};
    a.wfmt = L->d.wfmt;
    a.gate = matw(L->w, 0);
    a.up = matw(L->w, 1);
    a.down = matw(L->w, 2);
    a.x = x;
    a.xt = xt;
    a.dy = dy;
    a.dyt = dyt;
    a.T = T;
    a.H = L->d.hidden;
    a.I = L->d.inter;
    a.E = L->d.n_experts;
    a.k = L->d.top_k;
    a.ids = r->ids;
    a.offsets = r->offsets;
    a.perm = r->perm;
    a.inv = r->inv;
    a.active = r->active;
    a.n_active = r->n_active;
    a.w = r->w;
    a.wr = L->w.router_w;
    a.gu = saved_gu;
    a.h_hi = (uint16_t *)(L->ws + L->lay.h);
    a.h_lo = a.h_hi + (size_t)T * a.k * a.I;
    a.gu_scratch = (float *)(L->ws + L->lay.gu);
    a.dgdu = (float *)(L->ws + L->lay.dgdu);
    a.dp_part = (float *)(L->ws + L->lay.dp);
    a.dxs = (float *)(L->ws + L->lay.ybuf);
    a.dx = dx;
    a.act = L->d.act;
    // g, u are recomputed (saved_gu = NULL) on the exact bf16 path even with MOE_F_MX_GATEUP
    a.prof = &L->prof;
    const hipStream_t hs = (hipStream_t)stream;
    if (L->d.n_shared > 0) {
        // the shared experts' input-gradient rows first (g, u recomputed; no router term),
        // summed into dx by the routed pass's final kernel
        DenseRouting dr;
        if ((st = device_status(dense_routing(L, T, dr, hs), "shared-expert routing")) != MOE_OK) return st;
        moe::ExpertBwdArgs sb = a;
        sb.gate = shared_matw(L->w, 0);
        sb.up = shared_matw(L->w, 1);
        sb.down = shared_matw(L->w, 2);
        sb.E = sb.k = L->d.n_shared;
        sb.ids = dr.ids;
        sb.offsets = dr.off;
        sb.perm = dr.perm;
        sb.inv = dr.inv;
        sb.active = dr.act;
        sb.n_active = dr.nact;
        sb.w = dr.w;
        sb.gu = nullptr;
        sb.h_lo = sb.h_hi + (size_t)T * sb.k * sb.I;
        sb.dxs = (float *)(L->ws + L->lay.sh_rows);
        sb.tok_chunks = tok_chunks(T);
        sb.skip_final = 1;
        if ((st = device_status(moe::launch_expert_backward(sb, hs), "shared experts (backward)")) != MOE_OK) return st;
        a.dxs2 = sb.dxs;
        a.k2 = sb.k;
    }
    if (!L->has_lora) return device_status(moe::launch_expert_backward(a, hs), "backward_input");
    const moe::LoraWs lw = lora_ws(L);
    const bool grads = dA != nullptr;
    if (!saved_gu || grads) {  // the gate/up terms: for recomputing g, u and for dB_g, dB_u
        if ((st = device_status(moe::lora_forward_pre(L->lora, lw, x, xt, T, a.H, a.I, hs), "adapter (gate/up terms)")) != MOE_OK)
            return st;
        a.lora_gu = lw.gu;
    }
    if ((st = device_status(moe::lora_backward_pre(L->lora, lw, dy, dyt, T, a.H, a.I, hs), "adapter (down term)")) != MOE_OK)
        return st;
    a.lora_c = lw.c;
    if ((st = device_status(moe::launch_expert_backward(a, hs), "backward_input")) != MOE_OK) return st;
    if ((st = device_status(moe::lora_backward_post(L->lora, lw, a, moe::bwd_uses_mm(a), hs), "adapter (input gradient)")) !=
        MOE_OK)
        return st;
    if (!grads) return MOE_OK;
    if (!a.gu) a.gu = a.gu_scratch;  // recomputed by the backward above
    return device_status(moe::lora_grads(L->lora, lw, a, dA, dB, hs), "adapter (gradients)");
}

}  // namespace

moe_status moe_backward_input(moe_layer *L, const void *x, int32_t xt, const void *dy, int32_t dyt, int32_t T,
                              const moe_routing *r, const float *saved_gu, float *dx, void *stream)
{
    g_last_error.clear();
    return backward_impl(L, x, xt, dy, dyt, T, r, saved_gu, dx, nullptr, nullptr, stream);
}

moe_status moe_backward_lora(moe_layer *L, const void *x, int32_t xt, const void *dy, int32_t dyt, int32_t T,
                             const moe_routing *r, const float *saved_gu, float *dx, float *const dA[3], float *const dB[3],
                             void *stream)
{
    g_last_error.clear();
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK) return st;
    if (!L->has_lora) return fail(MOE_ERR_INVALID_ARG, "no adapter is attached (moe_set_lora)");
    if (!dA || !dB) return fail(MOE_ERR_INVALID_ARG, "dA or dB is NULL");
    for (int m = 0; m < 3; m++)
        if (!dA[m] || !dB[m] || !aligned(dA[m], 16) || !aligned(dB[m], 16))
            return fail(MOE_ERR_INVALID_ARG, "dA[%d] and dB[%d] must be non-NULL and 16-byte aligned", m, m);
    if (T == 0) {
        // no tokens: the adapter gradients are zero
        const moe_desc &d = L->d;
        const size_t na[3] = {(size_t)L->lora.r * d.hidden, (size_t)L->lora.r * d.hidden, (size_t)L->lora.r * d.inter};
        const size_t nb[3] = {(size_t)d.inter * L->lora.r, (size_t)d.inter * L->lora.r, (size_t)d.hidden * L->lora.r};
        if ((st = check_tokens(L, T)) != MOE_OK) return st;
        for (int m = 0; m < 3; m++) {
            hipError_t e = moe::fill_zero(dA[m], na[m], (hipStream_t)stream);
            if (e == hipSuccess) e = moe::fill_zero(dB[m], nb[m], (hipStream_t)stream);
            if (e != hipSuccess) return device_status(e, "zero adapter gradients");
        }
        return MOE_OK;
    }
    return backward_impl(L, x, xt, dy, dyt, T, r, saved_gu, dx, dA, dB, stream);
}

moe_status moe_set_lora(moe_layer *L, const moe_lora *lora)
{
    g_last_error.clear();
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK) return st;
    if (!lora) {
        L->has_lora = false;
        L->lora = moe::LoraW{};
        return MOE_OK;
    }
    if (!(L->d.flags & MOE_F_LORA))
        return fail(MOE_ERR_INVALID_ARG, "the layer's workspace was sized without MOE_F_LORA");
    if (lora->rank < 1 || lora->rank > kMaxLoraRank)
        return fail(MOE_ERR_INVALID_ARG, "rank=%d must be in 1..%d", lora->rank, kMaxLoraRank);
    if (!std::isfinite(lora->scale)) return fail(MOE_ERR_INVALID_ARG, "scale is not finite");
    for (int m = 0; m < 3; m++)
        if (!lora->A[m] || !lora->B[m] || !aligned(lora->A[m], 16) || !aligned(lora->B[m], 16))
            return fail(MOE_ERR_INVALID_ARG, "A[%d] and B[%d] must be non-NULL and 16-byte aligned", m, m);
    moe::LoraW w{};
    w.r = lora->rank;
    w.scale = lora->scale;
    for (int m = 0; m < 3; m++) {
        w.A[m] = lora->A[m];
        w.B[m] = lora->B[m];
    }
    L->lora = w;
    L->has_lora = true;
    return MOE_OK;
}



moe_status moe_forward_static(moe_layer *L, const void *x, int32_t xt, int32_t T, const moe_routing *r, float *y,
                              void *stream)
{
    g_last_error.clear();
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK || (st = check_tokens(L, T)) != MOE_OK || (st = check_dtype(xt, "x")) != MOE_OK)
        return st;
    if (L->d.n_shared || L->has_lora || (L->d.flags & (MOE_F_MX_GATEUP | MOE_F_QUANT_X8 | MOE_F_VALIDATE)))
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_forward_static serves the routed layer without shared experts, an attached adapter, "
                    "MOE_F_MX_GATEUP, MOE_F_QUANT_X8 or MOE_F_VALIDATE");
    const StaticLayout sl = static_layout(L->d, T);
    if (sl.total > kStaticScratchBytes)
        return fail(MOE_ERR_WORKSPACE, "T=%d needs %zu bytes of scratch; moe_forward_static has %zu", T, sl.total,
                    kStaticScratchBytes);
    if (T == 0) return MOE_OK;
    if ((st = check_routing(r)) != MOE_OK) return st;
    if (!x || !y) return fail(MOE_ERR_INVALID_ARG, "x or y is NULL");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(MOE_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    char *base = nullptr;
    if ((st = static_scratch(&base)) != MOE_OK) return st;
    const hipStream_t hs = (hipStream_t)stream;
    moe::ExpertFwdArgs a = routed_fwd_args(L, x, xt, T, r, y);
    a.h_hi = (uint16_t *)(base + sl.h);
    a.h_lo = a.h_hi + (size_t)T * a.k * a.I;
    if (L->d.wfmt == MOE_W_RVQ3) {
        a.gu_ws = (float *)(base + sl.h);
        if (!(L->d.flags & MOE_F_RVQ_GATHER)) a.lut_ord = (int32_t *)(base + sl.ord);
    }
    a.ybuf = (float *)(base + sl.ybuf);
    a.status = (uint32_t *)(base + sl.status);
    a.dec_sync = (uint32_t *)(base + sl.sync);
    // the array keeps the previous call's contents: the status word and the counters of the
    // fused launch must start at zero (a fill kernel, no memset node under graph capture)
    if ((st = device_status(moe::fill_zero((float *)(base + sl.status), (sl.h - sl.status) / 4, hs),
                            "clearing the static scratch")) != MOE_OK)
        return st;
    moe::set_lds_staging(a);
    return device_status(moe::launch_expert_forward(a, hs), "forward (static scratch)");
}

}  // extern "C"

namespace {

// One latent projection call: argument checks, then the dense product on the stream.
moe_status project(moe_layer *L, const void *a, int32_t at, int32_t T, float *out, bool in, bool backward, void *stream)
{
    g_last_error.clear();
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK || (st = check_tokens(L, T)) != MOE_OK || (st = check_dtype(at, "input")) != MOE_OK)
        return st;
    if (L->d.model_width <= 0) return fail(MOE_ERR_INVALID_ARG, "the layer has no latent projections (model_width = 0)");
    if (T == 0) return MOE_OK;
    if (!a || !out) return fail(MOE_ERR_INVALID_ARG, "input or output is NULL");
    if (!aligned(a, 16) || !aligned(out, 16)) return fail(MOE_ERR_INVALID_ARG, "input and output must be 16-byte aligned");
    const int D = L->d.model_width, H = L->d.hidden;
    // forward in: [T][D] -> [T][H] with proj_in [H][D]; forward out: [T][H] -> [T][D] with
    // proj_out [D][H]; the backward products take the same matrices untransposed
    const uint16_t *w = in ? L->w.proj_in : L->w.proj_out;
    int N, R;
    if (!backward) {
        N = in ? H : D;
        R = in ? D : H;
    } else {
        N = in ? D : H;
        R = in ? H : D;
    }
    return device_status(moe::launch_dense(a, at, w, backward, T, N, R, out, (hipStream_t)stream), "latent projection");
}

}  // namespace

extern "C" {

moe_status moe_project_in(moe_layer *L, const void *x_model, int32_t xt, int32_t T, float *x_latent, void *stream)
{
    return project(L, x_model, xt, T, x_latent, true, false, stream);
}

moe_status moe_project_out(moe_layer *L, const float *y_latent, int32_t T, float *out, void *stream)
{
    return project(L, y_latent, MOE_DT_F32, T, out, false, false, stream);
}

moe_status moe_project_out_backward(moe_layer *L, const void *dout, int32_t dt, int32_t T, float *dy_latent, void *stream)
{
    return project(L, dout, dt, T, dy_latent, false, true, stream);
}

moe_status moe_project_in_backward(moe_layer *L, const float *dx_latent, int32_t T, float *dx_model, void *stream)
{
    return project(L, dx_latent, MOE_DT_F32, T, dx_model, true, true, stream);
}

moe_status moe_check_status(moe_layer *L, uint32_t *bits, void *stream)
{
    g_last_error.clear();
    moe_status st;
    if ((st = check_layer(L)) != MOE_OK) return st;
    if (!bits) return fail(MOE_ERR_INVALID_ARG, "bits is NULL");
    if (!validating(L)) return fail(MOE_ERR_INVALID_ARG, "the layer was created without MOE_F_VALIDATE");
    *bits = 0;
    return take_status(L, (hipStream_t)stream, bits);
}

void moe_destroy(moe_layer *L)
{
    if (!L) return;
    prof_release(L->prof);
    delete L;
}

moe_status moe_prof_enable(moe_layer *L, uint32_t mask, int32_t max_launches)
{
    g_last_error.clear();
    if (!L) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
    prof_release(L->prof);
    if (mask == 0) return MOE_OK;
    if (max_launches < 1 || max_launches > 65536)
        return fail(MOE_ERR_INVALID_ARG, "max_launches=%d must be in 1..65536", max_launches);
    mask &= (1u << moe::PK_N) - 1u;
    for (int k = 0; k < moe::PK_N; k++) {
        if (!((mask >> k) & 1u)) continue;
        L->prof.ev[k].assign((size_t)2 * max_launches, nullptr);
        for (auto &e : L->prof.ev[k]) {
            hipError_t err = hipEventCreate(&e);
            if (err != hipSuccess) {
                prof_release(L->prof);
                return device_status(err, "hipEventCreate");
            }
        }
    }
    L->prof.cap = max_launches;
    L->prof.mask = mask;
    return MOE_OK;
}

moe_status moe_prof_read(moe_layer *L, int32_t family, double *total_ms, int32_t *launches)
{
    g_last_error.clear();
    if (!L || !total_ms || !launches) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
    if (family < 0 || family >= moe::PK_N) return fail(MOE_ERR_INVALID_ARG, "unknown kernel family %d", family);
    const moe::Prof &p = L->prof;
    double tot = 0.0;
    for (int i = 0; i < p.n[family]; i++) {
        hipError_t err = hipEventSynchronize(p.ev[family][2 * i + 1]);
        if (err != hipSuccess) return device_status(err, "hipEventSynchronize");
        float ms = 0.f;
        err = hipEventElapsedTime(&ms, p.ev[family][2 * i], p.ev[family][2 * i + 1]);
        if (err != hipSuccess) return device_status(err, "hipEventElapsedTime");
        tot += ms;
    }
    *total_ms = tot;
    *launches = p.n[family];
    return MOE_OK;
}

const char *moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_DEVICE: return "device error";
    case MOE_ERR_INTERNAL: return "internal error";
    case MOE_ERR_DATA: return "out-of-contract data";
    }
    return "unknown status";
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
