"""The C oracle against an independent numpy fp64 implementation of the whole layer
(oracle/cross_numpy.py: its own E2M1/E8M0 and RVQ3 decoding, top-k, grouping and products),
on the tiny workload (8 tokens, H 256, I 128, 16 MXFP4 experts, top-2, fp32 x) and variants:
routing and grouping identical, y and dX within 1e-12 of each other (CPU only)."""
import numpy as np
import pytest

import moe_synth as syn
import oracle
from oracle import cross_numpy as xn
from cases import host_case

TINY = syn.WORKLOADS["tiny"]


def _rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


def _compare(c, bias=None):
    w = c.w
    x64, dy64 = c.x64, oracle.to_f64(syn.upstream_grad(w, w.T), w.x_dtype)
    ids, p, logits = oracle.route(x64, c.wr, bias, w.k)
    if c.codes is not None:
        N = xn.Layer(c.wr, bias, codes=c.codes, scales=c.scales)
    else:
        N = xn.Layer(c.wr, bias, idx=c.idx, cb=c.cb)
    ids2, p2, logits2 = N.route(x64, w.k)
    assert np.array_equal(ids, ids2)
    assert _rel(logits2, logits) < 1e-13 and _rel(p2, p) < 1e-13
    g1, g2 = oracle.group(ids, w.E), xn.group(ids2, w.E)
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(g1[key], g2[key]), key
    assert g1["n_active"] == g2["n_active"]
    assert np.array_equal(g1["active"][:g1["n_active"]], g2["active"])
    W = c.oracle_weights()
    for m in range(3):  # decoded matrices bit for bit
        for e in (0, w.E - 1):
            assert np.array_equal(oracle.decode_matrix(W, m, e), N.mats[m][e])
    y, y2 = oracle.forward(x64, ids, p, W), N.forward(x64, ids2, p2)
    dx, dx2 = oracle.backward_input(x64, dy64, ids, p, c.wr, W), N.backward_input(x64, dy64, ids2, p2)
    assert _rel(y2, y) < 1e-12 and _rel(dx2, dx) < 1e-12, (_rel(y2, y), _rel(dx2, dx))


def test_cross_oracle_tiny_workload():
    _compare(host_case(TINY))


def test_cross_oracle_bias_bf16_and_wider_topk():
    w = syn.shrink(TINY, T=13, E=24, k=5, x_dtype="bf16", bias_sd=0.5, x_key=91)
    c = host_case(w)
    _compare(c, bias=syn.router_bias(w))


@pytest.mark.parametrize("k", [1, 16])
def test_cross_oracle_topk_extremes(k):
    # k = 1 (a single expert per token) and k = E (every expert, the dense softmax)
    _compare(host_case(syn.shrink(TINY, T=5, k=k, x_key=92 + k)))


def test_cross_oracle_rvq3():
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=4, H=256, I=128, E=8, k=3, x_key=95)
    _compare(host_case(w))


def test_cross_oracle_planted_transpose_fails():
    """A slip the cross-check must catch: the numpy side with the down matrix read transposed
    within 16x16 tiles (a plausible layout mistake) disagrees with the C oracle."""
    c = host_case(TINY)
    N = xn.Layer(c.wr, codes=c.codes, scales=c.scales)
    d = N.mats[2]
    E, H, I = d.shape
    t = d.reshape(E, H // 16, 16, I // 16, 16).transpose(0, 1, 4, 3, 2).reshape(E, H, I)
    N.mats[2] = t
    ids, p, _ = oracle.route(c.x64, c.wr, None, TINY.k)
    y = oracle.forward(c.x64, ids, p, c.oracle_weights())
    assert _rel(N.forward(c.x64, ids, p), y) > 1e-3
