"""GPU parity of the shared experts (LazyLoRA README, "The engine": 2 shared experts beside
the 896 routed ones in each MoE layer): every token takes each shared expert with weight 1,
their outputs join the combine after the routed slots and their input gradient joins dX
(no router term).  Against the fp64 oracle on the same seeded inputs (max|err| / max|ref|
<= 1e-4; routing bit-exact), through every kernel family the shared pass can take."""
import numpy as np
import pytest

import moe_synth as syn
import oracle
from cases import TOL, act_tensor, device_layer, host_case, lora_parity, log, rel_err

pytestmark = pytest.mark.gpu

TINY = syn.WORKLOADS["tiny"]


def _np(t):
    return t.detach().cpu().numpy()


def _case(w, n=2, act=0):
    c = host_case(w, with_dy=True)
    c.act = act
    c.shared = syn.shared_experts(w, n)
    return c


def run_shared(c, name, flags=0, saved=(True, False)):
    import torch
    w = c.w
    log(f"case {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} fmt={w.wfmt} x={w.x_dtype} shared={c.n_shared} "
        f"act={c.act} flags={flags}")
    L = device_layer(c, max_tokens=max(w.T, 1), flags=flags)
    x = act_tensor(c.x, w.x_dtype)
    dy = act_tensor(c.dy, w.x_dtype)
    r = L.route(x)
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k, bias_mode=c.bias_mode)
    torch.cuda.synchronize()
    assert np.array_equal(_np(r.ids), ids), f"{name}: routing ids"
    W = c.oracle_weights()
    y_ref = c.ref_forward(c.x64, ids, p, W)
    gu = L.new_saved_gu(w.T)
    y = L.forward(x, r, saved_gu=gu)
    torch.cuda.synchronize()
    e = rel_err(_np(y), y_ref)
    log(f"  y rel err {e:.3e} (shared term alone {np.abs(y_ref - oracle.forward(c.x64, ids, p, W)).max():.3e})")
    assert e <= TOL, f"{name}: y {e}"
    dx_ref = c.ref_backward(c.x64, c.dy64, ids, p, W)
    for sv in saved:
        dx = L.backward_input(x, dy, r, saved_gu=gu if sv else None)
        torch.cuda.synchronize()
        e = rel_err(_np(dx), dx_ref)
        log(f"  dX rel err {e:.3e} (saved routed g/u: {sv})")
        assert e <= TOL, f"{name}: dX {e}"
    # deterministic: the same bits again
    y2 = L.forward(x, r)
    torch.cuda.synchronize()
    assert np.array_equal(_np(y2), _np(y)), f"{name}: repeated forward differs"
    L.close()


def test_shared_tiny_generic_fp32_tokens():
    run_shared(_case(syn.shrink(TINY, with_dy=True)), "shared-tiny")


def test_shared_one_and_k_shared_experts():
    # one shared expert, and as many shared experts as the routed top-k (the largest allowed)
    run_shared(_case(syn.shrink(TINY, x_dtype="bf16", bias_sd=0.5, with_dy=True, x_key=60), n=1, act=1), "shared-1-situ")
    run_shared(_case(syn.shrink(TINY, k=4, x_dtype="bf16", with_dy=True, x_key=61), n=4), "shared-k")


def test_shared_single_token_decode_kernels():
    run_shared(_case(syn.shrink(TINY, T=1, H=1024, I=512, E=16, k=8, x_dtype="bf16", with_dy=True, x_key=62)),
               "shared-dec-T1")


def test_shared_few_tokens_decode_kernels():
    run_shared(_case(syn.shrink(TINY, T=5, H=512, I=768, E=12, k=3, x_dtype="bf16", with_dy=True, x_key=63)),
               "shared-dec-few")


def test_shared_grouped_gemm_token_chunks():
    # 400 tokens: the shared pass takes the grouped GEMMs forward and backward with the
    # tokens of each shared expert split into chunks of 96 (five chunks, the last of 16)
    run_shared(_case(syn.shrink(TINY, T=400, H=512, I=1024, E=8, k=2, x_dtype="bf16", with_dy=True, x_key=64)),
               "shared-mm")


def test_shared_block_scaled_gateup():
    from quantized_moe_route_amd import _lib as C
    run_shared(_case(syn.shrink(TINY, T=300, H=1024, I=512, E=16, k=3, x_dtype="bf16", with_dy=True, x_key=65)),
               "shared-mx", flags=C.MOE_F_MX_GATEUP)


def test_shared_rvq3_paths():
    run_shared(_case(syn.shrink(syn.WORKLOADS["rvq16"], T=10, H=512, I=768, E=12, k=3, with_dy=True, x_key=66)),
               "shared-rvq3-gather")
    run_shared(_case(syn.shrink(syn.WORKLOADS["rvq16"], T=24, H=256, I=128, E=12, k=3, with_dy=True, x_key=67)),
               "shared-rvq3-generic")


def test_shared_with_the_adapter():
    # the adapter is on the routed experts only; the shared experts stay plain
    from quantized_moe_route_amd import _lib as C
    for T, key in ((3, 68), (400, 69)):
        w = syn.shrink(TINY, T=T, H=512, I=1024, E=8, k=2, x_dtype="bf16", with_dy=True, x_key=key)
        c = _case(w)
        L = device_layer(c, max_tokens=T, flags=C.MOE_F_LORA)
        lora_parity(c, L, f"shared-lora-T{T}")
        L.close()


def test_shared_with_quantized_input():
    # MOE_F_QUANT_X8: the shared experts take the MXFP8-quantized x too (they are expert products)
    import torch

    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, T=300, H=1024, I=512, E=16, k=3, x_dtype="bf16", with_dy=True, x_key=70)
    c = _case(w)
    L = device_layer(c, max_tokens=w.T, flags=C.MOE_F_QUANT_X8 | C.MOE_F_MX_GATEUP)
    x = act_tensor(c.x, w.x_dtype)
    r = L.route(x)
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k)
    xq64, _ = oracle.quantize_mxfp8(c.x64)
    y = L.forward(x, r)
    torch.cuda.synchronize()
    e = rel_err(_np(y), c.ref_forward(xq64, ids, p))
    log(f"case shared-quant: y rel err {e:.3e}")
    assert e <= TOL
    L.close()


def test_shared_zero_tokens():
    import torch
    w = syn.shrink(TINY, with_dy=True)
    c = _case(w)
    L = device_layer(c, max_tokens=8)
    x = act_tensor(c.x[:0], w.x_dtype)
    r = L.new_routing(0)
    y = L.forward(x, r)
    dx = L.backward_input(x, x, r)
    torch.cuda.synchronize()
    assert y.shape == (0, w.H) and dx.shape == (0, w.H)
    L.close()


def test_shared_units_of_the_stream_kernels_situ_bias_and_k_shared():
    # few bf16 tokens with H, I multiples of 256: the shared experts are extra units of the
    # routed stream kernels' launch; SiTU with a selection-only bias, and as many shared
    # experts as the top-k
    c = _case(syn.shrink(TINY, T=3, H=512, I=512, E=16, k=4, x_dtype="bf16", bias_sd=0.5, with_dy=True, x_key=71),
              n=4, act=1)
    c.bias_mode = 2
    run_shared(c, "shared-fused-situ-k")


def test_shared_grouped_gemm_beside_generic_routed_kernels():
    # 20 tokens over 64 experts: too few per expert for the routed grouped GEMM (generic
    # kernels) and too many for the stream kernels, while each shared expert holds all 20
    # tokens and takes the grouped GEMM (one chunk)
    run_shared(_case(syn.shrink(TINY, T=20, H=512, I=512, E=64, k=2, x_dtype="bf16", with_dy=True, x_key=72)),
               "shared-mm-beside-generic")
