"""Parity at the K3 shapes (H 3584, I 3072, 896 experts, top-16), in the launch
configuration the benchmark times.  Routing and grouping are compared in full for every
token; y (and dX) for every token of the 64-token and RVQ3 decode batches, and for 64 tokens
of the 4096-token pass chosen from the grouping so that they cover the grouped GEMMs' tile
and pass boundaries (the oracle computes them one by one)."""
import numpy as np
import pytest

import moe_synth as syn
import oracle
from cases import TOL, act_tensor, device_layer, host_case, log, lora_parity, rel_err

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def k3_mxfp4():
    """The K3-shaped MXFP4 layer (15.72 GB of experts) resident on the GPU."""
    w = syn.WORKLOADS["train4096"]
    log("generating the K3 MXFP4 layer on the host")
    c = host_case(w)
    log("uploading")
    L = device_layer(c, max_tokens=4096)
    _sync()
    log("layer ready")
    yield c, L
    L.close()


def _check_full_routing(r, ids, p, E):
    assert np.array_equal(_np(r.ids), ids)
    assert rel_err(_np(r.w), p) <= TOL
    g = oracle.group(ids, E)
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(_np(getattr(r, key)), g[key]), key
    n = int(_np(r.n_active)[0])
    assert n == g["n_active"] and np.array_equal(_np(r.active)[:n], g["active"][:n])
    return g


def tile_tokens(g, k, T, n, seed):
    """At least n tokens chosen from the grouping so that the compared rows cover the grouped
    GEMMs' structure: the first and last rows of 16-token tiles, every expert's partial last
    tile, and the second 96-token pass of the heaviest expert (its rows 96, 111, 112 and last);
    the lightest active expert in full; the rest random."""
    counts, off, perm = g["counts"], g["offsets"], g["perm"]
    active = g["active"][:g["n_active"]]
    rng = np.random.default_rng(seed)

    def tok(e, r):
        return int(perm[off[e] + r]) // k

    picks = []
    heavy = int(active[np.argmax(counts[active])])
    for r in (0, 15, 16, 31, 95, 96, 111, 112, counts[heavy] - 1):
        if r < counts[heavy]:
            picks.append(tok(heavy, r))
    light = int(active[np.argmin(counts[active])])
    picks += [tok(light, r) for r in range(counts[light])]
    for e in rng.choice(active, size=min(len(active), 12), replace=False):
        c = int(counts[e])
        picks += [tok(e, 0), tok(e, c - 1), tok(e, (c - 1) // 16 * 16)]
    picks = sorted(set(picks))
    if len(picks) < n:
        rest = np.setdiff1d(np.arange(T), picks)
        picks = sorted(set(picks) | set(rng.choice(rest, size=n - len(picks), replace=False).tolist()))
    return np.array(picks), heavy


def _run(c, L, name, T, sample, with_bwd):
    """Routing in full; y (and dX with saved and recomputed g, u) on `sample` tokens, or on
    every token when sample >= T, or on the tile-covering set of tile_tokens() when the
    experts average many tokens."""
    w = syn.shrink(c.w, T=T, bias_sd=syn.WORKLOADS[name].bias_sd, x_key=syn.WORKLOADS[name].x_key)
    x_h = syn.activations(w, T)
    bias = syn.router_bias(w)
    x64 = oracle.to_f64(x_h, "bf16")
    log(f"{name}: oracle routing for {T} tokens")
    ids, p, logits = oracle.route(x64, c.wr, bias, w.k)
    gaps = oracle.boundary_gap(logits, ids)
    log(f"{name}: smallest rank gap {gaps.min():.3e}")
    assert gaps.min() > 1e-11, "a seeded rank gap is inside the fp64 residue; pick another seed"
    L2 = L
    if bias is not None:
        import quantized_moe_route_amd as q
        L2 = q.MoELayer(hidden=w.H, inter=w.I, n_experts=w.E, top_k=w.k, max_tokens=T,
                        router_w=L._keep[0], router_b=q.to_device(bias), codes=L._keep[2], scales=L._keep[3])
    x = act_tensor(x_h, "bf16")
    log(f"{name}: GPU route + forward")
    r = L2.route(x)
    gu = L2.new_saved_gu(T) if with_bwd else None
    y = L2.forward(x, r, saved_gu=gu)
    _sync()
    g = _check_full_routing(r, ids, p, w.E)
    log(f"{name}: routing bit-exact; U = {g['n_active']} active experts")
    W = c.oracle_weights()
    if sample >= T:
        toks = np.arange(T)
    elif T * w.k >= 8 * w.E:
        toks, heavy = tile_tokens(g, w.k, T, sample, seed=T)
        log(f"{name}: heaviest expert {heavy} holds {g['counts'][heavy]} tokens")
    else:
        toks = np.sort(np.random.default_rng(T).choice(T, size=sample, replace=False))
    log(f"{name}: oracle forward on {len(toks)} tokens")
    y_ref = oracle.forward(x64[toks], ids[toks], p[toks], W)
    e = rel_err(_np(y)[toks], y_ref)
    log(f"{name}: y rel err {e:.3e}")
    assert e <= TOL
    if with_bwd:
        dy_h = syn.upstream_grad(w, T)
        dy = act_tensor(dy_h, "bf16")
        dx = L2.backward_input(x, dy, r, saved_gu=gu)
        dx2 = L2.backward_input(x, dy, r, saved_gu=None)
        _sync()
        log(f"{name}: oracle backward on the same {len(toks)} tokens")
        dx_ref = oracle.backward_input(x64[toks], oracle.to_f64(dy_h, "bf16")[toks], ids[toks], p[toks], c.wr, W)
        e1, e2 = rel_err(_np(dx)[toks], dx_ref), rel_err(_np(dx2)[toks], dx_ref)
        log(f"{name}: dX rel err {e1:.3e} (saved g/u), {e2:.3e} (recomputed)")
        assert e1 <= TOL and e2 <= TOL
        # every row is finite and the two backward variants agree everywhere
        assert np.isfinite(_np(dx)).all() and rel_err(_np(dx2), _np(dx)) <= 1e-6


def test_decode1_full_size(k3_mxfp4):
    c, L = k3_mxfp4
    _run(c, L, "decode1", 1, 1, with_bwd=False)


def test_decode64_full_size(k3_mxfp4):
    c, L = k3_mxfp4
    _run(c, L, "decode64", 64, 64, with_bwd=False)


def test_train4096_full_size(k3_mxfp4):
    c, L = k3_mxfp4
    _run(c, L, "train4096", 4096, 64, with_bwd=True)


def test_rvq16_full_size():
    w = syn.WORKLOADS["rvq16"]
    log("generating the K3 RVQ3 layer on the host")
    c = host_case(w)
    L = device_layer(c, max_tokens=w.T)
    x64 = c.x64
    ids, p, logits = oracle.route(x64, c.wr, None, w.k)
    assert oracle.boundary_gap(logits, ids).min() > 1e-11
    x = act_tensor(c.x, "bf16")
    r = L.route(x)
    y = L.forward(x, r)
    _sync()
    g = _check_full_routing(r, ids, p, w.E)
    log(f"rvq16: routing bit-exact; U = {g['n_active']}")
    y_ref = oracle.forward(x64, ids, p, c.oracle_weights())  # all 16 tokens
    e = rel_err(_np(y), y_ref)
    log(f"rvq16: y rel err {e:.3e}")
    assert e <= TOL
    L.close()


def test_lora_k3_two_tokens(k3_mxfp4):
    """The K3 layer with a rank-16 shared adapter (LazyLoRA README, "LoRA") on two tokens:
    y, dX and all six adapter gradients in full against the oracle."""
    import quantized_moe_route_amd as q
    from quantized_moe_route_amd import _lib as C
    c, L = k3_mxfp4
    w = syn.shrink(c.w, T=2, x_key=57)
    cc = type(c)(w, syn.activations(w, 2), c.wr, None, syn.upstream_grad(w, 2), codes=c.codes, scales=c.scales)
    router_w, _, codes, scales = L._keep[:4]
    La = q.MoELayer(hidden=w.H, inter=w.I, n_experts=w.E, top_k=w.k, max_tokens=2, router_w=router_w, codes=codes,
                    scales=scales, flags=C.MOE_F_LORA)
    lora_parity(cc, La, "lora-k3-T2", saved=(True,))
    La.close()


def test_shared_experts_k3(k3_mxfp4):
    """The K3 layer with its 2 shared experts (LazyLoRA README, "The engine") beside the 896
    routed ones: one decode token in full, and the 4096-token pass (the shared experts'
    tokens in 43 grouped-GEMM chunks) on sampled tokens, forward and dX."""
    import quantized_moe_route_amd as q
    c, L = k3_mxfp4
    w = c.w
    log("generating 2 shared experts at the K3 shape")
    sh = syn.shared_experts(w, 2)
    Ws = oracle.Weights(w.H, w.I, codes=sh[0], scales=sh[1])
    Ls = q.MoELayer(hidden=w.H, inter=w.I, n_experts=w.E, top_k=w.k, max_tokens=4096, router_w=L._keep[0],
                    codes=L._keep[2], scales=L._keep[3],
                    shared=([q.to_device(a) for a in sh[0]], [q.to_device(a) for a in sh[1]]))
    W = c.oracle_weights()
    for name, T, sample, with_bwd in (("decode1", 1, 1, False), ("train4096", 4096, 16, True)):
        wk = syn.shrink(w, T=T, x_key=syn.WORKLOADS[name].x_key)
        assert syn.WORKLOADS[name].bias_sd in (None, 0.0)
        x_h = syn.activations(wk, T)
        x64 = oracle.to_f64(x_h, "bf16")
        ids, p, _ = oracle.route(x64, c.wr, None, w.k)
        x = act_tensor(x_h, "bf16")
        r = Ls.route(x)
        y = Ls.forward(x, r)
        _sync()
        assert np.array_equal(_np(r.ids), ids)
        # the shared experts' tokens run in 96-token chunks: first and last rows of chunks and of
        # 16-token tiles, the short last chunk, and random ones
        edge = [t for t in (0, 15, 16, 95, 96, 191, 4031, 4032, 4095) if t < T]
        rest = np.setdiff1d(np.arange(T), edge)
        extra = np.random.default_rng(T + 1).choice(rest, size=max(0, sample - len(edge)), replace=False)
        toks = np.sort(np.concatenate([edge, extra]).astype(np.int64))[:max(sample, 1)]
        y_ref = oracle.forward(x64[toks], ids[toks], p[toks], W) + oracle.shared_forward(x64[toks], Ws, 2)
        e = rel_err(_np(y)[toks], y_ref)
        log(f"shared-{name}: y rel err {e:.3e} on tokens {toks.tolist()}")
        assert e <= TOL
        if with_bwd:
            dy_h = syn.upstream_grad(wk, T)
            dx = Ls.backward_input(x, act_tensor(dy_h, "bf16"), r)
            _sync()
            dy64 = oracle.to_f64(dy_h, "bf16")[toks]
            dx_ref = (oracle.backward_input(x64[toks], dy64, ids[toks], p[toks], c.wr, W)
                      + oracle.shared_backward_input(x64[toks], dy64, Ws, 2))
            e = rel_err(_np(dx)[toks], dx_ref)
            log(f"shared-{name}: dX rel err {e:.3e}")
            assert e <= TOL and np.isfinite(_np(dx)).all()
    Ls.close()


def test_latent_projections_k3(k3_mxfp4):
    """The K3 layer (896 routed experts in the 3,584-wide latent space) inside latent
    projections of an assumed model width of 7,168 (the pages do not give it): four tokens,
    forward and input gradient through the whole chain against the oracle."""
    import quantized_moe_route_amd as q
    from test_gpu_latent import chain_parity
    c, L = k3_mxfp4
    D = syn.K3_MODEL_WIDTH_ASSUMED
    w = syn.shrink(c.w, T=4, x_key=71)
    cc = type(c)(w, syn.activations(w, 4), c.wr, None, None, codes=c.codes, scales=c.scales)
    pin, pout = syn.latent_projections(w, D)
    router_w, _, codes, scales = L._keep[:4]
    Lp = q.MoELayer(hidden=w.H, inter=w.I, n_experts=w.E, top_k=w.k, max_tokens=4, router_w=router_w, codes=codes,
                    scales=scales, proj=(q.to_device(pin), q.to_device(pout)))
    chain_parity(cc, D, "latent-k3-T4", L=Lp)
    Lp.close()
