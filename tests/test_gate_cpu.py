"""The 1e-4 parity gate has teeth: a lossy variant of the method must fail it (CPU only).

The Two Desks write-up (Act II) reports that a GPU expert path with bf16 matmul
arithmetic missed its precision gate (error 5.8e-3) until it moved to fp32 compute; the
LazyLoRA README ("Arithmetic") reports a shift of about 1e-3 in a layer's output from
bf16 accumulation."""
import numpy as np

import moe_synth as syn
import oracle
from cases import TOL, host_case, rel_err

TINY = syn.WORKLOADS["tiny"]


def test_negative_control_bf16_rounding_of_h_fails_the_gate():
    """Rounding the expert intermediate h to bf16 (what a bf16-only path would do) must exceed
    the 1e-4 gate, so the gate can tell the exact path from a lossy one."""
    w = syn.shrink(TINY, T=16, x_key=17)
    c = host_case(w)
    W = c.oracle_weights()
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k)
    y_ref = oracle.forward(c.x64, ids, p, W)
    y_bad = np.zeros_like(y_ref)
    Wd = {}
    for t in range(w.T):
        for j in range(w.k):
            e = int(ids[t, j])
            _, _, h, _ = oracle.expert_forward(W, e, c.x64[t])
            h16 = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(h.astype(np.float32))).astype(np.float64)
            if e not in Wd:
                Wd[e] = oracle.decode_matrix(W, 2, e)
            y_bad[t] += p[t, j] * (Wd[e] @ h16)
    assert rel_err(y_bad, y_ref) > TOL
