"""Shared helpers for the parity tests: build a workload on host and device, run the
oracle on the same host arrays, compare."""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

import moe_synth as syn
import oracle


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@dataclass
class HostCase:
    w: syn.Workload
    x: np.ndarray            # fp32 or bf16 bits
    wr: np.ndarray
    bias: Optional[np.ndarray]
    dy: Optional[np.ndarray]
    codes: Optional[List[np.ndarray]] = None
    scales: Optional[List[np.ndarray]] = None
    idx: Optional[List[np.ndarray]] = None
    cb: Optional[List[np.ndarray]] = None
    act: int = 0  # 0 SwiGLU, 1 SiTU
    bias_mode: int = 1  # with a bias: 1 in the logits, 2 selection only
    lora: Optional[tuple] = None  # (A [3], B [3], scale) fp32 arrays: the shared adapter
    shared: Optional[tuple] = None  # the shared experts: (codes, scales) or (idx, cb), n leading

    @property
    def x64(self):
        return oracle.to_f64(self.x, self.w.x_dtype)

    @property
    def dy64(self):
        return oracle.to_f64(self.dy, self.w.x_dtype)

    def oracle_weights(self):
        if self.codes is not None:
            return oracle.Weights(self.w.H, self.w.I, codes=self.codes, scales=self.scales, act=self.act,
                                  lora=self.lora)
        return oracle.Weights(self.w.H, self.w.I, idx=self.idx, cb=self.cb, act=self.act, lora=self.lora)

    @property
    def n_shared(self) -> int:
        return 0 if self.shared is None else int(self.shared[0][0].shape[0])

    def shared_weights(self):
        a, b = self.shared
        if self.codes is not None:
            return oracle.Weights(self.w.H, self.w.I, codes=a, scales=b, act=self.act)
        return oracle.Weights(self.w.H, self.w.I, idx=a, cb=b, act=self.act)

    def ref_forward(self, x64, ids, p, W=None):
        """The oracle's layer output on x64 for the given routing (routed slots + shared experts)."""
        y = oracle.forward(x64, ids, p, W or self.oracle_weights())
        if self.shared is not None:
            y = y + oracle.shared_forward(x64, self.shared_weights(), self.n_shared)
        return y

    def ref_backward(self, x64, dy64, ids, p, W=None):
        dx = oracle.backward_input(x64, dy64, ids, p, self.wr, W or self.oracle_weights())
        if self.shared is not None:
            dx = dx + oracle.shared_backward_input(x64, dy64, self.shared_weights(), self.n_shared)
        return dx


def host_case(w: syn.Workload, T: Optional[int] = None, with_dy: Optional[bool] = None) -> HostCase:
    T = w.T if T is None else T
    c = HostCase(w, syn.activations(w, T), syn.router_weight(w), syn.router_bias(w),
                 syn.upstream_grad(w, T) if (w.with_dy if with_dy is None else with_dy) else None)
    if w.wfmt == "mxfp4":
        c.codes, c.scales = syn.mxfp4_layer(w)
    else:
        c.idx, c.cb = syn.rvq3_layer(w)
    return c


def act_tensor(a: np.ndarray, dtype: str):
    import quantized_moe_route_amd as q
    return q.bf16_tensor(a) if dtype == "bf16" else q.to_device(np.asarray(a, np.float32))


def device_layer(c: HostCase, max_tokens: int, flags: int = 0, proj=None):
    import quantized_moe_route_amd as q
    w = c.w
    kw = dict(hidden=w.H, inter=w.I, n_experts=w.E, top_k=w.k, max_tokens=max_tokens,
              router_w=q.to_device(c.wr), router_b=None if c.bias is None else q.to_device(c.bias), flags=flags,
              act=c.act, bias_mode=None if c.bias is None else c.bias_mode)
    if c.codes is not None:
        kw["codes"] = [q.to_device(a) for a in c.codes]
        kw["scales"] = [q.to_device(a) for a in c.scales]
    else:
        kw["rvq_idx"] = [q.to_device(a) for a in c.idx]
        kw["rvq_cb"] = [q.to_device(a) for a in c.cb]
    if c.shared is not None:
        kw["shared"] = ([q.to_device(a) for a in c.shared[0]], [q.to_device(a) for a in c.shared[1]])
    if proj is not None:
        kw["proj"] = proj
    return q.MoELayer(**kw)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the parity metric; 0 for an all-zero reference matched exactly)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return float(num / den)


TOL = 1e-4


def fnv1a32(a: np.ndarray) -> int:
    """FNV-1a over the bytes of an array (determinism gate)."""
    h = 0x811C9DC5
    for b in np.ascontiguousarray(a).view(np.uint8).tobytes():
        h = ((h ^ b) * 0x01000193) & 0xFFFFFFFF
    return h


def lora_parity(c: HostCase, L, name: str, rank: int = 16, scale: float = 2.0, saved=(True, False)) -> None:
    """Attach a seeded rank-`rank` adapter to the device layer L (created with MOE_F_LORA
    over c's weights), then compare forward, dX and the adapter gradients with the oracle
    on c's tokens; also: backward_input equals backward_lora's dX bit for bit, repeated
    gradients are bitwise equal, and detaching restores the plain layer."""
    import torch

    import quantized_moe_route_amd as q

    def np_(t):
        return t.detach().cpu().numpy()

    w = c.w
    A, B = syn.lora_adapter(w, rank)
    c.lora = (A, B, scale)
    log(f"case {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} fmt={w.wfmt} x={w.x_dtype} act={c.act} rank={rank}")
    L.set_lora([q.to_device(a) for a in A], [q.to_device(b) for b in B], scale)
    x = act_tensor(c.x, w.x_dtype)
    dy = act_tensor(c.dy, w.x_dtype)
    r = L.route(x)
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k, bias_mode=c.bias_mode)
    torch.cuda.synchronize()
    assert np.array_equal(np_(r.ids), ids), f"{name}: routing ids"
    W = c.oracle_weights()
    y_ref = c.ref_forward(c.x64, ids, p, W)
    dx_ref = c.ref_backward(c.x64, c.dy64, ids, p, W)
    dA_ref, dB_ref = oracle.lora_grads(c.x64, c.dy64, ids, p, W)
    gu = L.new_saved_gu(w.T)
    y = L.forward(x, r, saved_gu=gu)
    torch.cuda.synchronize()
    e = rel_err(np_(y), y_ref)
    log(f"  y rel err {e:.3e}")
    assert e <= TOL, f"{name}: y {e}"
    first = None
    for sv in saved:
        g = gu if sv else None
        dx, dA, dB = L.backward_lora(x, dy, r, saved_gu=g)
        dx_only = L.backward_input(x, dy, r, saved_gu=g)
        torch.cuda.synchronize()
        e = rel_err(np_(dx), dx_ref)
        log(f"  dX rel err {e:.3e} (saved g/u: {sv})")
        assert e <= TOL, f"{name}: dX {e}"
        assert np.array_equal(np_(dx_only), np_(dx)), f"{name}: backward_input and backward_lora disagree on dX"
        for m, nm in enumerate(("gate", "up", "down")):
            ea, eb = rel_err(np_(dA[m]), dA_ref[m]), rel_err(np_(dB[m]), dB_ref[m])
            log(f"  dA[{nm}] {ea:.3e}  dB[{nm}] {eb:.3e}")
            assert ea <= TOL and eb <= TOL, f"{name}: adapter gradient {nm}: dA {ea} dB {eb}"
        if first is None:
            first = (g, dA, dB)
    # the sums run in a fixed order: the same bits again
    _, dA2, dB2 = L.backward_lora(x, dy, r, saved_gu=first[0])
    torch.cuda.synchronize()
    for m in range(3):
        assert np.array_equal(np_(dA2[m]), np_(first[1][m])) and np.array_equal(np_(dB2[m]), np_(first[2][m]))
    # detached: the plain layer again
    L.set_lora()
    y0 = L.forward(x, r)
    torch.cuda.synchronize()
    c.lora = None
    assert rel_err(np_(y0), c.ref_forward(c.x64, ids, p)) <= TOL, f"{name}: detached forward"
