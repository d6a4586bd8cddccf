"""Second, independent fp64 implementation of the whole routed-expert layer in numpy --
TEST INFRASTRUCTURE ONLY (imported by tests/ alone).

It shares no code with ``moe_oracle.c`` or with the GPU library: its own E2M1 / E8M0
decoding (a value table indexed by the 3-bit magnitude, the sign bit applied separately),
its own top-k (a stable sort on (-logit, expert id)), grouping (a stable argsort of the
slots' experts), and the expert products as numpy matrix products.  Two implementations
that agree to ~1e-12 pin each other against slips that a single one could carry unseen
(LazyLoRA README, "How you know this is real": the forward is compared with an
independent implementation of the same model).

Follows the same readings of the pages as the C oracle: OCP MX v1.0 elements (E2M1 codes,
low nibble = even element, one E8M0 scale per 32 consecutive inputs); weights stored
[out][in]; the k largest logits, equal logits ranked by the lower expert id; the combining
weights = the softmax over the selected logits; SwiGLU h = g sigmoid(g) u; y = sum of the
weighted expert outputs in rank order; dX with the routing held fixed, through the experts
and through the softmax weights into the router.
"""
from __future__ import annotations

import numpy as np

# |E2M1| by the 3 magnitude bits (2 exponent bits with bias 1, 1 mantissa bit)
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)


def e2m1_values(codes: np.ndarray) -> np.ndarray:
    """Element values of 4-bit codes (any integer array)."""
    c = np.asarray(codes, np.int64)
    mag = _E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def unpack_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., out, in/2] code bytes and [..., out, in/32] E8M0 bytes -> [..., out, in] float64."""
    codes = np.asarray(codes, np.uint8)
    lo = e2m1_values(codes & 0x0F)
    hi = e2m1_values(codes >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    s = np.ldexp(1.0, np.asarray(scales, np.int64) - 127)
    return vals * np.repeat(s, 32, axis=-1)


def unpack_rvq3(idx: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """[3, out, in/8] stage indices and [3, 256, 8] fp16 bits -> [out, in] float64: every
    8-element run of a row is the sum of its three stage codewords."""
    books = np.asarray(cb, np.uint16).view(np.float16).astype(np.float64)
    idx = np.asarray(idx, np.int64)
    out = books[0][idx[0]] + books[1][idx[1]] + books[2][idx[2]]  # [out, in/8, 8]
    return out.reshape(idx.shape[1], idx.shape[2] * 8)


def topk(logits: np.ndarray, k: int):
    """ids [T][k] by (logit desc, id asc), and the softmax weights over them."""
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))  # last key primary: -logit, then id
        ids[t] = order[:k]
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return ids, z / z.sum(axis=1, keepdims=True)


def group(ids: np.ndarray, E: int) -> dict:
    slots_e = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(slots_e, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(slots_e, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    active = np.nonzero(counts)[0].astype(np.int32)
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv, active=active, n_active=int(active.size))


def _silu_parts(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s, g * s


class Layer:
    """Decoded fp64 weights of a layer: gate/up [E][I][H], down [E][H][I]."""

    def __init__(self, wr, bias=None, codes=None, scales=None, idx=None, cb=None):
        self.wr = np.asarray(wr, np.float64)
        self.bias = None if bias is None else np.asarray(bias, np.float64)
        if codes is not None:
            self.mats = [unpack_mxfp4(codes[m], scales[m]) for m in range(3)]
        else:
            self.mats = [np.stack([unpack_rvq3(idx[m][e], cb[m][e]) for e in range(idx[m].shape[0])]) for m in range(3)]

    def route(self, x64, k):
        logits = x64 @ self.wr.T
        if self.bias is not None:
            logits = logits + self.bias
        ids, p = topk(logits, k)
        return ids, p, logits

    def forward(self, x64, ids, p):
        T, k = ids.shape
        y = np.zeros((T, self.mats[2].shape[1]))
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                g = self.mats[0][e] @ x64[t]
                u = self.mats[1][e] @ x64[t]
                _, silu = _silu_parts(g)
                y[t] += p[t, j] * (self.mats[2][e] @ (silu * u))
        return y

    def backward_input(self, x64, dy64, ids, p):
        T, k = ids.shape
        dx = np.zeros_like(x64)
        for t in range(T):
            dps = np.empty(k)
            parts = []
            for j in range(k):
                e = ids[t, j]
                g = self.mats[0][e] @ x64[t]
                u = self.mats[1][e] @ x64[t]
                s, silu = _silu_parts(g)
                a = self.mats[2][e].T @ dy64[t]
                dps[j] = a @ (silu * u)
                dh = p[t, j] * a
                dg = dh * u * s * (1.0 + g * (1.0 - s))
                du = dh * silu
                parts.append(self.mats[0][e].T @ dg + self.mats[1][e].T @ du)
            dl = p[t] * (dps - p[t] @ dps)
            for j in range(k):
                dx[t] += parts[j] + dl[j] * self.wr[ids[t, j]]
        return dx
