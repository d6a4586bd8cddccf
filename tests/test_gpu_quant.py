"""GPU parity of the activation-quantized prefill (MOE_F_QUANT_X8): the expert products
take x quantized to MXFP8 (OCP MX v1.0, E4M3 with an E8M0 scale per 32 elements); the
oracle mirrors the quantization, so the gate stays max|err| / max|ref| <= 1e-4; the
deviation from the unquantized layer is reported, not gated."""
import numpy as np
import pytest

import moe_synth as syn
import oracle
from cases import TOL, act_tensor, device_layer, host_case, log, rel_err

pytestmark = pytest.mark.gpu

TINY = syn.WORKLOADS["tiny"]


def _np(t):
    return t.detach().cpu().numpy()


def run_quant(c, name, flags=0, lora=False):
    import torch

    import quantized_moe_route_amd as q
    from quantized_moe_route_amd import _lib as C
    w = c.w
    log(f"case {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} fmt={w.wfmt} x={w.x_dtype} flags={flags} lora={lora}")
    L = device_layer(c, max_tokens=w.T, flags=flags | C.MOE_F_QUANT_X8 | (C.MOE_F_LORA if lora else 0))
    if lora:
        A, B = syn.lora_adapter(w, 16)
        c.lora = (A, B, 2.0)
        L.set_lora([q.to_device(a) for a in A], [q.to_device(b) for b in B], 2.0)
    x = act_tensor(c.x, w.x_dtype)
    r = L.route(x)
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k)  # the router sees x unquantized
    torch.cuda.synchronize()
    assert np.array_equal(_np(r.ids), ids), f"{name}: routing ids"
    W = c.oracle_weights()
    xq64, _ = oracle.quantize_mxfp8(c.x64)
    y_ref = oracle.forward(xq64, ids, p, W)
    y = L.forward(x, r)
    torch.cuda.synchronize()
    e = rel_err(_np(y), y_ref)
    dev = rel_err(_np(y), oracle.forward(c.x64, ids, p, W))
    log(f"  y rel err {e:.3e} (against the quantized-input oracle); deviation from the unquantized layer {dev:.3e}")
    assert e <= TOL, f"{name}: y {e}"
    assert 0.0 < dev < 0.1, f"{name}: deviation {dev}"
    return L, x, r


def test_quant_tiny_fp32_tokens():
    run_quant(host_case(TINY), "quant-tiny")


def test_quant_single_token_decode_kernels():
    run_quant(host_case(syn.shrink(TINY, T=1, H=1024, I=512, E=16, k=8, x_dtype="bf16", x_key=80)), "quant-dec-T1")


def test_quant_grouped_gemm_and_block_scaled_gateup():
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, T=400, H=512, I=1024, E=8, k=2, x_dtype="bf16", x_key=81)
    run_quant(host_case(w), "quant-mm")
    run_quant(host_case(w), "quant-mx", flags=C.MOE_F_MX_GATEUP)


def test_quant_block_scaled_single_term():
    # x arrives MXFP8-quantized: the quantizer writes the block-scaled gate/up's operand as one
    # exact E4M3 term (fp32 tokens, a ragged last tile per expert, and with the adapter)
    from quantized_moe_route_amd import _lib as C
    run_quant(host_case(syn.shrink(TINY, T=333, H=1024, I=512, E=16, k=3, x_key=84)), "quant-mx-f32",
              flags=C.MOE_F_MX_GATEUP)
    run_quant(host_case(syn.shrink(TINY, T=300, H=1024, I=512, E=16, k=3, x_dtype="bf16", x_key=85)),
              "quant-mx-lora", flags=C.MOE_F_MX_GATEUP, lora=True)


def test_quant_rvq3_and_adapter():
    run_quant(host_case(syn.shrink(syn.WORKLOADS["rvq16"], T=10, H=512, I=768, E=12, k=3, x_key=82)), "quant-rvq3")
    run_quant(host_case(syn.shrink(TINY, T=6, x_dtype="bf16", x_key=83)), "quant-lora", lora=True)


@pytest.mark.parametrize("mx", [False, True])
def test_quant_backward_is_the_exact_layers(mx):
    """moe_backward_input ignores the forward's quantization: recomputing g, u from x it
    returns the same bits as a layer without the flag (with the block-scaled gate/up, the
    recomputation takes x as two exact E4M3 terms again)."""
    import torch

    from quantized_moe_route_amd import _lib as C
    if mx:
        w = syn.shrink(TINY, T=300, H=1024, I=512, E=16, k=3, x_dtype="bf16", with_dy=True, x_key=86)
    else:
        w = syn.shrink(TINY, T=8, x_dtype="bf16", with_dy=True, x_key=84)
    flags = C.MOE_F_MX_GATEUP if mx else 0
    c = host_case(w)
    Lq, x, r = run_quant(c, "quant-bwd" + ("-mx" if mx else ""), flags=flags)
    L0 = device_layer(c, max_tokens=w.T, flags=flags)
    dy = act_tensor(c.dy, w.x_dtype)
    r0 = L0.route(x)
    dq = Lq.backward_input(x, dy, r)
    d0 = L0.backward_input(x, dy, r0)
    torch.cuda.synchronize()
    assert np.array_equal(_np(dq), _np(d0))


@pytest.mark.parametrize("mx", [False, True])
def test_quant_backward_from_saved_preactivations(mx):
    """saved_gu written by a quantized-input forward holds the pre-activations of the quantized
    x; moe_backward_input from them is the input gradient of the quantized layer with the
    quantization passed straight through (d xq / d x taken as 1): the oracle's backward run
    on the quantized x, with the routing (and the router term's Wr) of the unquantized x."""
    import torch

    from quantized_moe_route_amd import _lib as C
    if mx:
        w = syn.shrink(TINY, T=300, H=1024, I=512, E=16, k=3, x_dtype="bf16", with_dy=True, x_key=87)
    else:
        w = syn.shrink(TINY, T=8, x_dtype="bf16", with_dy=True, x_key=88)
    c = host_case(w)
    Lq, x, r = run_quant(c, "quant-saved" + ("-mx" if mx else ""), flags=C.MOE_F_MX_GATEUP if mx else 0)
    gu = Lq.new_saved_gu(w.T)
    Lq.forward(x, r, saved_gu=gu)
    dx = Lq.backward_input(x, act_tensor(c.dy, w.x_dtype), r, saved_gu=gu)
    torch.cuda.synchronize()
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k)
    xq64, _ = oracle.quantize_mxfp8(c.x64)
    dx_ref = oracle.backward_input(xq64, c.dy64, ids, p, c.wr, c.oracle_weights())
    e = rel_err(_np(dx), dx_ref)
    log(f"  dX (saved g/u of the quantized forward) rel err {e:.3e}")
    assert e <= TOL
