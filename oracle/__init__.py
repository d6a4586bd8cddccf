"""fp64 CPU oracle of the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library does not import it and
shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64, plain loops); this
module only builds it with gcc, loads it with ctypes and converts inputs to
float64 exactly (bf16 / fp32 / fp16 widen exactly to double).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

FMT_MXFP4, FMT_RVQ3 = 0, 1
MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2


def build() -> str:
    """Compile the oracle with gcc (always rebuilds)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-shared", "-fPIC",
                    "-pthread", _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Lora(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int),
                ("scale", ctypes.c_double),
                ("A", ctypes.c_void_p * 3),
                ("B", ctypes.c_void_p * 3)]


class _Weights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int),
                ("codes", ctypes.c_void_p * 3),
                ("scales", ctypes.c_void_p * 3),
                ("rvq_idx", ctypes.c_void_p * 3),
                ("rvq_cb", ctypes.c_void_p * 3),
                ("act", ctypes.c_int),
                ("lora", ctypes.POINTER(_Lora))]

ACT_SWIGLU, ACT_SITU = 0, 1


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        d, i, vp = ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        L.oracle_e2m1.restype = d
        L.oracle_e2m1.argtypes = [ctypes.c_uint]
        L.oracle_e8m0.restype = d
        L.oracle_e8m0.argtypes = [ctypes.c_uint]
        L.oracle_fp16.restype = d
        L.oracle_fp16.argtypes = [ctypes.c_uint16]
        L.oracle_decode_matrix.argtypes = [vp, i, i, i, i, vp]
        L.oracle_router_logits.argtypes = [i, i, i, vp, vp, vp, vp, i]
        L.oracle_topk_softmax.restype = i
        L.oracle_topk_softmax.argtypes = [i, i, i, vp, vp, vp]
        L.oracle_group.argtypes = [i, i, i, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_e4m3.argtypes = [ctypes.c_uint]
        L.oracle_e4m3.restype = ctypes.c_double
        L.oracle_quantize_mxfp8.argtypes = [i, vp, vp, vp]
        L.oracle_quantize_mxfp8.restype = None
        L.oracle_softmax_at.argtypes = [i, i, i, vp, vp, vp]
        L.oracle_softmax_at.restype = None
        L.oracle_expert_forward.argtypes = [vp, i, i, i, vp, vp, vp, vp, vp]
        L.oracle_forward.argtypes = [i, i, i, i, vp, vp, vp, vp, vp, i]
        L.oracle_backward_input.argtypes = [i, i, i, i, vp, vp, vp, vp, vp, vp, vp, i]
        L.oracle_lora_grads.argtypes = [i, i, i, i, vp, vp, vp, vp, vp, vp * 3, vp * 3, i]
        L.oracle_dense.argtypes = [i, i, i, vp, vp, vp, i, i]
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored activations to float64: dtype "bf16" (uint16 bits) or "f32"."""
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


class Weights:
    """Expert weights as stored (numpy arrays, host memory), in the layouts the layer consumes.

    MXFP4: codes[m] [E][rows][cols/2] uint8, scales[m] [E][rows][cols/32] uint8.
    RVQ3:  idx[m] [E][3][rows][cols/8] uint8, cb[m] [E][3][256][8] uint16 (fp16 bits).
    m = 0 gate, 1 up (rows = I, cols = H), 2 down (rows = H, cols = I).
    """

    def __init__(self, H: int, I: int, codes=None, scales=None, idx=None, cb=None, act: int = 0, lora=None):
        self.H, self.I = H, I
        self._keep = []
        s = _Weights()
        s.act = act  # ACT_SWIGLU or ACT_SITU
        self.lora = None
        if lora is not None:
            # lora = (A [gate, up, down], B [gate, up, down], scale); A[m] is [r][in],
            # B[m] is [out][r]; values widened exactly to float64
            A, B, scale = lora
            r = np.asarray(A[0]).shape[0]
            assert 1 <= r <= 64
            shapes_a = [(r, H), (r, H), (r, I)]
            shapes_b = [(I, r), (I, r), (H, r)]
            ls = _Lora()
            ls.r, ls.scale = r, float(scale)
            for m in range(3):
                a64 = np.ascontiguousarray(np.asarray(A[m], np.float64))
                b64 = np.ascontiguousarray(np.asarray(B[m], np.float64))
                assert a64.shape == shapes_a[m] and b64.shape == shapes_b[m], (m, a64.shape, b64.shape)
                self._keep += [a64, b64]
                ls.A[m] = a64.ctypes.data
                ls.B[m] = b64.ctypes.data
            self._lora_struct = ls
            s.lora = ctypes.pointer(ls)
            self.lora = (r, float(scale))
        if codes is not None:
            s.fmt = FMT_MXFP4
            for m in range(3):
                c = np.ascontiguousarray(codes[m], np.uint8)
                sc = np.ascontiguousarray(scales[m], np.uint8)
                self._keep += [c, sc]
                s.codes[m] = c.ctypes.data
                s.scales[m] = sc.ctypes.data
        else:
            s.fmt = FMT_RVQ3
            for m in range(3):
                ia = np.ascontiguousarray(idx[m], np.uint8)
                ca = np.ascontiguousarray(cb[m], np.uint16)
                self._keep += [ia, ca]
                s.rvq_idx[m] = ia.ctypes.data
                s.rvq_cb[m] = ca.ctypes.data
        self.struct = s

    def ref(self):
        return ctypes.byref(self.struct)

    def shape(self, mat: int):
        return (self.I, self.H) if mat in (MAT_GATE, MAT_UP) else (self.H, self.I)


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e8m0(b: int) -> float:
    return lib().oracle_e8m0(b)


def fp16(bits: int) -> float:
    return lib().oracle_fp16(bits)


def decode_matrix(W: Weights, mat: int, e: int) -> np.ndarray:
    rows, cols = W.shape(mat)
    out = np.empty((rows, cols), np.float64)
    lib().oracle_decode_matrix(W.ref(), mat, e, W.H, W.I, _p(out))
    return out


def router_logits(x64: np.ndarray, wr: np.ndarray, bias: Optional[np.ndarray] = None,
                  nthreads: Optional[int] = None) -> np.ndarray:
    x64 = np.ascontiguousarray(x64, np.float64)
    wr64 = np.ascontiguousarray(wr, np.float64)
    b64 = None if bias is None else np.ascontiguousarray(bias, np.float64)
    T, H = x64.shape
    E = wr64.shape[0]
    out = np.empty((T, E), np.float64)
    lib().oracle_router_logits(T, H, E, _p(x64), _p(wr64), _p(b64), _p(out), nthreads or default_threads())
    return out


def topk_softmax(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = lib().oracle_topk_softmax(T, E, k, _p(logits), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle top-k: non-finite logit or bad k")
    return ids, w


def e4m3(code: int) -> float:
    """Value of an OCP MX v1.0 FP8 E4M3 code."""
    return lib().oracle_e4m3(code)


def quantize_mxfp8(x64: np.ndarray):
    """OCP MX v1.0 MXFP8 (E4M3) quantization of each row in blocks of 32 consecutive
    elements: (the represented values q * 2^shared as float64, the shared exponents)."""
    x64 = np.ascontiguousarray(x64, np.float64)
    assert x64.shape[-1] % 32 == 0
    xq = np.empty_like(x64)
    exps = np.empty(x64.size // 32, np.int32)
    lib().oracle_quantize_mxfp8(x64.size, _p(x64), _p(xq), _p(exps))
    return xq, exps.reshape(x64.shape[:-1] + (x64.shape[-1] // 32,))


def softmax_at(logits: np.ndarray, ids: np.ndarray):
    """Softmax of each row of logits over the experts ids[t] (in that order)."""
    logits = np.ascontiguousarray(logits, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    T, E = logits.shape
    k = ids.shape[1]
    w = np.empty((T, k), np.float64)
    lib().oracle_softmax_at(T, E, k, _p(logits), _p(ids), _p(w))
    return w


def route(x64, wr, bias, k, nthreads=None, bias_mode=1):
    """(ids [T][k] int32, w [T][k] float64, logits [T][E] float64).  bias_mode 1: the bias is
    part of the logits (selection and weights); 2: it selects only, the weights are the
    softmax of the unbiased logits over the selected experts.  The returned logits are the
    selection keys."""
    logits = router_logits(x64, wr, bias, nthreads)
    ids, w = topk_softmax(logits, k)
    if bias is not None and bias_mode == 2:
        w = softmax_at(router_logits(x64, wr, None, nthreads), ids)
    return ids, w, logits


def group(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    S = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(S, np.int32)
    inv = np.empty(S, np.int32)
    active = np.zeros(E, np.int32)
    n_active = np.zeros(1, np.int32)
    lib().oracle_group(T, k, E, _p(ids), _p(counts), _p(offsets), _p(perm), _p(inv), _p(active), _p(n_active))
    return dict(counts=counts, offsets=offsets, perm=perm, inv=inv, active=active, n_active=int(n_active[0]))


def expert_forward(W: Weights, e: int, x64: np.ndarray):
    """(g, u, h, o) of one expert on one token."""
    x64 = np.ascontiguousarray(x64, np.float64)
    g = np.empty(W.I)
    u = np.empty(W.I)
    h = np.empty(W.I)
    o = np.empty(W.H)
    lib().oracle_expert_forward(W.ref(), e, W.H, W.I, _p(x64), _p(g), _p(u), _p(h), _p(o))
    return g, u, h, o


def forward(x64: np.ndarray, ids: np.ndarray, w: np.ndarray, W: Weights, nthreads=None) -> np.ndarray:
    x64 = np.ascontiguousarray(x64, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    T, k = ids.shape
    y = np.empty((T, W.H), np.float64)
    lib().oracle_forward(T, W.H, W.I, k, _p(x64), _p(ids), _p(w), W.ref(), _p(y), nthreads or default_threads())
    return y


def backward_input(x64, dy64, ids, w, wr, W: Weights, nthreads=None) -> np.ndarray:
    x64 = np.ascontiguousarray(x64, np.float64)
    dy64 = np.ascontiguousarray(dy64, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    wr64 = np.ascontiguousarray(wr, np.float64)
    T, k = ids.shape
    dx = np.empty((T, W.H), np.float64)
    lib().oracle_backward_input(T, W.H, W.I, k, _p(x64), _p(dy64), _p(ids), _p(w), _p(wr64), W.ref(),
                                _p(dx), nthreads or default_threads())
    return dx


def shared_forward(x64, Ws: Weights, n_shared: int, nthreads=None) -> np.ndarray:
    """Sum over s < n_shared of shared expert s applied to every token with weight 1: the
    shared experts of a K3 MoE layer (LazyLoRA README, "The engine": 2 shared experts beside
    the 896 routed ones), Ws holding them as experts 0..n_shared-1.  The layer output is
    forward(...) of the routed slots plus this."""
    T = x64.shape[0]
    ids = np.tile(np.arange(n_shared, dtype=np.int32), (T, 1))
    return forward(x64, ids, np.ones((T, n_shared)), Ws, nthreads)


def shared_backward_input(x64, dy64, Ws: Weights, n_shared: int, nthreads=None) -> np.ndarray:
    """d/dx of sum_t <dy_t, shared_forward(x)_t>: the shared experts' input gradient.  They
    carry no routing weight to differentiate, so the router term is zero (zero router rows)."""
    T = x64.shape[0]
    ids = np.tile(np.arange(n_shared, dtype=np.int32), (T, 1))
    return backward_input(x64, dy64, ids, np.ones((T, n_shared)), np.zeros((n_shared, Ws.H)), Ws, nthreads)


def lora_grads(x64, dy64, ids, w, W: Weights, nthreads=None):
    """Adapter gradients (dA [gate, up, down], dB [gate, up, down]) of sum_t <dy[t], y[t]>."""
    assert W.lora is not None
    r = W.lora[0]
    x64 = np.ascontiguousarray(x64, np.float64)
    dy64 = np.ascontiguousarray(dy64, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    T, k = ids.shape
    dA = [np.empty((r, W.H)), np.empty((r, W.H)), np.empty((r, W.I))]
    dB = [np.empty((W.I, r)), np.empty((W.I, r)), np.empty((W.H, r))]
    vp3 = ctypes.c_void_p * 3
    lib().oracle_lora_grads(T, W.H, W.I, k, _p(x64), _p(dy64), _p(ids), _p(w), W.ref(),
                            vp3(*[a.ctypes.data for a in dA]), vp3(*[b.ctypes.data for b in dB]),
                            nthreads or default_threads())
    return dA, dB


def dense(a64: np.ndarray, w_bits: np.ndarray, transposed: bool = False, nthreads=None) -> np.ndarray:
    """Latent projection with bf16 weights w [N][K] (uint16 bits): a [T][K] -> a w^T [T][N], or
    with transposed a [T][N] -> a w [T][K]."""
    a64 = np.ascontiguousarray(a64, np.float64)
    w_bits = np.ascontiguousarray(w_bits, np.uint16)
    N, K = w_bits.shape
    T = a64.shape[0]
    out = np.zeros((T, K if transposed else N))
    lib().oracle_dense(T, N, K, _p(a64), _p(w_bits), _p(out), int(transposed), nthreads or default_threads())
    return out


def layer_forward(x64, wr, bias, k, W: Weights, nthreads=None, bias_mode=1):
    """Route then run the experts: (y, ids, w)."""
    ids, w, _ = route(x64, wr, bias, k, nthreads, bias_mode)
    return forward(x64, ids, w, W, nthreads), ids, w


def boundary_gap(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Per token: the smallest gap between consecutive logits in rank order over the first
    k+1 ranks (0 means an exact tie decided by expert id)."""
    T, k = ids.shape
    out = np.empty(T)
    for t in range(T):
        l = logits[t]
        sel = l[ids[t]]
        rest = np.delete(l, ids[t])
        nxt = rest.max() if rest.size else -np.inf
        seq = np.concatenate([sel, [nxt]])
        out[t] = np.min(seq[:-1] - seq[1:]) if seq.size > 1 else np.inf
    return out


__all__ = [n for n in dir() if not n.startswith("_")]
