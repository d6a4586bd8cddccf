"""moe_forward_static, the allocation-free forward (its scratch is an array compiled into the
library, one per GPU): through the C ABI it gives the same bits as moe_forward on the same
inputs, on two calls in a row, the second with fewer tokens (the array keeps the first call's
contents), on the fused single-token launch, the few-token kernels, the generic kernels
(fp32 tokens), RVQ3 and the grouped GEMMs; and it matches the oracle to the parity bar."""
import numpy as np
import pytest

import moe_synth as syn
import oracle
from cases import TOL, act_tensor, device_layer, host_case, log, rel_err

pytestmark = pytest.mark.gpu

TINY = syn.WORKLOADS["tiny"]

CASES = {
    # name: (workload overrides, first T, second T)
    "fused-single-token": (dict(H=1024, I=768, E=16, k=8, x_dtype="bf16"), 4, 1),
    "few-token": (dict(H=512, I=512, E=12, k=3, x_dtype="bf16"), 16, 5),
    "generic-fp32": (dict(H=256, I=128, E=16, k=2), 40, 9),
    "rvq3": (dict(H=512, I=768, E=12, k=3, x_dtype="bf16", wfmt="rvq3"), 10, 3),
    "grouped-gemm": (dict(H=512, I=1024, E=8, k=2, x_dtype="bf16"), 400, 130),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_static_forward_equals_forward(case):
    import torch
    over, T1, T2 = CASES[case]
    base = syn.WORKLOADS["rvq16"] if over.get("wfmt") == "rvq3" else TINY
    w = syn.shrink(base, T=T1, x_key=60, **over)
    c = host_case(w)
    L = device_layer(c, max_tokens=T1)
    W = c.oracle_weights()
    for T in (T1, T2):
        log(f"case {case}: T={T} H={w.H} I={w.I} E={w.E} k={w.k} fmt={w.wfmt} x={w.x_dtype}")
        x = act_tensor(c.x[:T], w.x_dtype)
        r = L.route(x)
        y_ws = L.forward(x, r)
        y_st = L.forward_static(x, r, y=torch.full((T, w.H), float("nan"), dtype=torch.float32, device="cuda"))
        torch.cuda.synchronize()
        assert np.array_equal(y_st.cpu().numpy(), y_ws.cpu().numpy()), f"{case}: T={T} differs from moe_forward"
        ids, p, _ = oracle.route(c.x64[:T], c.wr, c.bias, w.k)
        e = rel_err(y_st.cpu().numpy(), oracle.forward(c.x64[:T], ids, p, W))
        log(f"  y rel err {e:.3e} (bitwise equal to moe_forward)")
        assert e <= TOL
    L.close()


def test_static_forward_rejects_what_it_cannot_hold():
    import quantized_moe_route_amd as q
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, T=8, x_dtype="bf16", x_key=61)
    c = host_case(w)
    L = device_layer(c, max_tokens=8, flags=C.MOE_F_QUANT_X8)
    x = act_tensor(c.x, "bf16")
    r = L.route(x)
    with pytest.raises(q.MoeError) as ei:
        L.forward_static(x, r)
    assert ei.value.status == C.MOE_ERR_UNSUPPORTED
    L.close()
