"""The MoE layer inside its latent projections (F4; LazyLoRA README, "The engine": the latent
MoE projections; Two Desks, Act II: the experts run in a latent space of width 3,584) on the
GPU against the oracle: x_latent = x_model proj_in^T, the routed layer on x_latent,
out = y_latent proj_out^T, and the input gradient through the whole chain.

Reading: the projections return fp32, the GPU's latent is the fp32-accumulated product and
the oracle's the fp64 one, so the two routers see inputs that differ by that rounding.  The
GPU's routing is the exact top-k of its own latent, the oracle's of its own, so they agree
whenever every rank gap of the oracle exceeds twice max_e |Wr_e . dx| <= ||dx|| max_e ||Wr_e||
(Cauchy-Schwarz) for that token's latent difference dx; the test checks this condition for its
seeds, then compares the selection bit for bit."""
import numpy as np
import pytest

import moe_synth as syn
import oracle
from cases import TOL, act_tensor, device_layer, host_case, log, rel_err

pytestmark = pytest.mark.gpu

TINY = syn.WORKLOADS["tiny"]


def _np(t):
    return t.detach().cpu().numpy()


def chain_parity(c, D, name, L=None, check_backward=True):
    """Forward and input gradient of the projected layer on c's weights, model width D."""
    import torch

    import quantized_moe_route_amd as q
    w = c.w
    pin, pout = syn.latent_projections(w, D)
    xm_h = syn.model_activations(w, D)
    dout_h = syn.model_upstream_grad(w, D)
    xm64, dout64 = oracle.to_f64(xm_h, w.x_dtype), oracle.to_f64(dout_h, w.x_dtype)
    W = c.oracle_weights()
    # oracle chain
    xl64 = oracle.dense(xm64, pin)
    ids, p, logits = oracle.route(xl64, c.wr, c.bias, w.k)
    y64 = oracle.forward(xl64, ids, p, W)
    out64 = oracle.dense(y64, pout)
    # GPU chain
    if L is None:
        L = device_layer(c, max_tokens=w.T, proj=(q.to_device(pin), q.to_device(pout)))
    xm, dout = act_tensor(xm_h, w.x_dtype), act_tensor(dout_h, w.x_dtype)
    xl = L.project_in(xm)
    r = L.route(xl)
    y = L.forward(xl, r)
    out = L.project_out(y)
    torch.cuda.synchronize()
    gap = oracle.boundary_gap(logits, ids)
    dxl = np.linalg.norm(_np(xl).astype(np.float64) - xl64, axis=1)
    bound = dxl * np.linalg.norm(c.wr.astype(np.float64), axis=1).max()
    ratio = (gap / np.maximum(2 * bound, 1e-300)).min()
    log(f"case {name}: T={w.T} D={D} H={w.H}; min over tokens of rank gap / (2 x logit change bound) {ratio:.3e}")
    assert np.all(gap > 2 * bound), "a seeded rank gap is within the latent rounding's reach; pick another seed"
    assert np.array_equal(_np(r.ids), ids), f"{name}: routing ids"
    e_lat, e_out = rel_err(_np(xl), xl64), rel_err(_np(out), out64)
    log(f"  x_latent rel err {e_lat:.3e}, out rel err {e_out:.3e}")
    assert e_lat <= TOL and e_out <= TOL
    if check_backward:
        dyl64 = oracle.dense(dout64, pout, transposed=True)
        dxl64 = oracle.backward_input(xl64, dyl64, ids, p, c.wr, W)
        dxm64 = oracle.dense(dxl64, pin, transposed=True)
        dyl = L.project_out_backward(dout)
        dxlg = L.backward_input(xl, dyl, r)
        dxm = L.project_in_backward(dxlg)
        torch.cuda.synchronize()
        e_dyl, e_dxm = rel_err(_np(dyl), dyl64), rel_err(_np(dxm), dxm64)
        log(f"  dy_latent rel err {e_dyl:.3e}, dx_model rel err {e_dxm:.3e}")
        assert e_dyl <= TOL and e_dxm <= TOL
    return L


@pytest.mark.parametrize("D", [256, 512, 960])
def test_latent_projections_tiny_fp32(D):
    chain_parity(host_case(TINY), D, f"latent-tiny-D{D}")


def test_latent_projections_bf16_ragged_tokens():
    # bf16 model activations, 37 tokens (a partial 64-token tile), bias and top-3
    w = syn.shrink(TINY, T=37, E=20, k=3, x_dtype="bf16", bias_sd=0.5, x_key=101)
    chain_parity(host_case(w), 1024, "latent-bf16-T37")


def test_latent_projection_errors():
    import quantized_moe_route_amd as q
    c = host_case(TINY)
    L = device_layer(c, max_tokens=8)  # no projections
    with pytest.raises(q.MoeError):
        L.project_in(act_tensor(syn.model_activations(TINY, 256), "f32"))
    L.close()
