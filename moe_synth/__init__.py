"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only draws random numbers and packs them into the storage formats
the layer consumes (bf16 / fp16 bit patterns, packed 4-bit codes, 8-bit
scale bytes, RVQ index bytes).  It holds none of the layer's arithmetic: no
dequantization, no routing, no matmul.  Both the fp64 oracle and the GPU
library read the arrays produced here; neither imports the other.

Every tensor is drawn from its own PCG64 stream keyed by
``SeedSequence(entropy=20260909, spawn_key=(family, tensor_id, index))`` so
any single expert can be regenerated alone.

Workload shapes follow the Kimi-K3 description on the LazyLoRA README
("The engine": 896 routed experts, top-16, latent 3,584, MXFP4 experts;
"LoRA": the 3584 -> 3072 -> 3584 expert shape) and the WASTE README
(3-bit residual VQ, 3 stages of 256-entry codebooks over 8-dim vectors).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

ENTROPY = 20260909

# tensor ids inside a family
_T_X, _T_WR, _T_BIAS, _T_DY = 1, 2, 3, 4
_T_CODES, _T_SCALES = 10, 20          # + matrix index (0 gate, 1 up, 2 down)
_T_RVQ_IDX, _T_RVQ_CB = 30, 40        # + matrix index
_T_LORA_A, _T_LORA_B = 50, 60         # + matrix index
_T_PROJ_IN, _T_PROJ_OUT, _T_XM, _T_DOUT = 70, 71, 72, 73  # latent projections, model-width x and dout

# family ids: the K3-shaped MXFP4 layer is shared by the three MXFP4 K3 workloads
FAMILY_TINY, FAMILY_K3_MXFP4, FAMILY_K3_RVQ = 1, 2, 4

MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2


def _rng(family: int, tensor: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=ENTROPY, spawn_key=(family, tensor, index)))


def _raw_bytes(family: int, tensor: int, index: int, n: int) -> np.ndarray:
    """n uniform bytes: little-endian bytes of raw 64-bit PCG64 outputs."""
    bg = np.random.PCG64(np.random.SeedSequence(entropy=ENTROPY, spawn_key=(family, tensor, index)))
    words = (n + 7) // 8
    return bg.random_raw(words).view(np.uint8)[:n]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    x_dtype: str          # "f32" or "bf16"
    wfmt: str             # "mxfp4" or "rvq3"
    family: int
    bias_sd: float = 0.0  # 0 => no router bias
    with_dy: bool = False
    x_key: int = 0        # distinguishes the activations of workloads sharing a family


WORKLOADS: Dict[str, Workload] = {
    # 8 tokens, hidden 256, intermediate 128, 16 experts, top-2, fp32 activations
    "tiny": Workload("tiny", 8, 256, 128, 16, 2, "f32", "mxfp4", FAMILY_TINY, with_dy=True),
    # K3 shape, single-token decode, all 896 experts resident
    "decode1": Workload("decode1", 1, 3584, 3072, 896, 16, "bf16", "mxfp4", FAMILY_K3_MXFP4, x_key=2),
    # K3 shape, 64-token decode, router bias N(0, 0.5)
    "decode64": Workload("decode64", 64, 3584, 3072, 896, 16, "bf16", "mxfp4", FAMILY_K3_MXFP4,
                         bias_sd=0.5, x_key=3),
    # K3 shape, 16-token decode with 3-bit residual-VQ experts
    "rvq16": Workload("rvq16", 16, 3584, 3072, 896, 16, "bf16", "rvq3", FAMILY_K3_RVQ, x_key=4),
    # K3 shape, 4096-token forward + input gradient, upstream grad bf16 N(0, 0.01^2)
    "train4096": Workload("train4096", 4096, 3584, 3072, 896, 16, "bf16", "mxfp4", FAMILY_K3_MXFP4,
                          with_dy=True, x_key=5),
}


def matrix_shape(mat: int, H: int, I: int):
    """(rows, cols) of the stored [out][in] matrix: gate/up are I x H, down is H x I."""
    return (I, H) if mat in (MAT_GATE, MAT_UP) else (H, I)


def activations(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """x[T][H]: N(0,1) as fp32, or rounded to bf16 bit patterns (uint16)."""
    T = w.T if T is None else T
    x = _rng(w.family, _T_X, w.x_key).standard_normal((T, w.H), dtype=np.float32)
    return x if w.x_dtype == "f32" else f32_to_bf16_bits(x)


def router_weight(w: Workload) -> np.ndarray:
    """Wr[E][H] fp32 N(0, 0.02^2)."""
    return (_rng(w.family, _T_WR).standard_normal((w.E, w.H), dtype=np.float32) * np.float32(0.02))


def router_bias(w: Workload) -> Optional[np.ndarray]:
    if w.bias_sd == 0.0:
        return None
    return _rng(w.family, _T_BIAS, w.x_key).standard_normal(w.E, dtype=np.float32) * np.float32(w.bias_sd)


def upstream_grad(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """dY[T][H]: N(0, 0.01^2) rounded to bf16 bits (fp32 for the fp32-activation workload)."""
    T = w.T if T is None else T
    d = _rng(w.family, _T_DY, w.x_key).standard_normal((T, w.H), dtype=np.float32) * np.float32(0.01)
    return d if w.x_dtype == "f32" else f32_to_bf16_bits(d)


def mxfp4_expert(w: Workload, mat: int, e: int):
    """One expert's packed matrix: codes [rows][cols/2] (uniform bytes = two uniform
    4-bit codes), scales [rows][cols/32] uniform in {119..123} (2^-8 .. 2^-4)."""
    rows, cols = matrix_shape(mat, w.H, w.I)
    codes = _raw_bytes(w.family, _T_CODES + mat, e, rows * cols // 2).reshape(rows, cols // 2)
    scales = _rng(w.family, _T_SCALES + mat, e).integers(119, 124, size=(rows, cols // 32), dtype=np.uint8)
    return codes, scales


def mxfp4_layer(w: Workload, experts=None):
    """All (or the listed) experts of the layer: codes[3] [E][rows][cols/2], scales[3] [E][rows][cols/32]."""
    ids = range(w.E) if experts is None else experts
    codes, scales = [], []
    for mat in range(3):
        rows, cols = matrix_shape(mat, w.H, w.I)
        c = np.empty((len(ids), rows, cols // 2), np.uint8)
        s = np.empty((len(ids), rows, cols // 32), np.uint8)
        for i, e in enumerate(ids):
            c[i], s[i] = mxfp4_expert(w, mat, e)
        codes.append(c)
        scales.append(s)
    return codes, scales


def rvq3_expert(w: Workload, mat: int, e: int):
    """One expert's 3-bit RVQ matrix: idx [3][rows][cols/8] uniform bytes, codebooks
    [3][256][8] fp16 bit patterns, stage s (1-based) drawn from N(0, (0.02/s)^2)."""
    rows, cols = matrix_shape(mat, w.H, w.I)
    idx = _raw_bytes(w.family, _T_RVQ_IDX + mat, e, 3 * rows * cols // 8).reshape(3, rows, cols // 8)
    g = _rng(w.family, _T_RVQ_CB + mat, e).standard_normal((3, 256, 8), dtype=np.float32)
    sd = np.array([0.02 / 1, 0.02 / 2, 0.02 / 3], np.float32).reshape(3, 1, 1)
    cb = (g * sd).astype(np.float16).view(np.uint16)
    return idx, cb


def rvq3_layer(w: Workload, experts=None):
    ids = range(w.E) if experts is None else experts
    idxs, cbs = [], []
    for mat in range(3):
        rows, cols = matrix_shape(mat, w.H, w.I)
        ia = np.empty((len(ids), 3, rows, cols // 8), np.uint8)
        ca = np.empty((len(ids), 3, 256, 8), np.uint16)
        for i, e in enumerate(ids):
            ia[i], ca[i] = rvq3_expert(w, mat, e)
        idxs.append(ia)
        cbs.append(ca)
    return idxs, cbs


def lora_adapter(w: Workload, r: int = 16, b_sd: float = 0.05):
    """The layer's shared low-rank adapter as fp32 arrays: A[m] [r][in] ~ N(0, 1/in) (the
    scale of a freshly initialised A, so A z has unit-order entries for unit-order z) and
    B[m] [out][r] ~ N(0, b_sd^2) (nonzero, as after some training steps; a fresh B is 0),
    for m = gate, up, down (in = H, H, I; out = I, I, H).  Rank 16 is the LazyLoRA
    README's ("LoRA")."""
    A, B = [], []
    for mat in range(3):
        rows, cols = matrix_shape(mat, w.H, w.I)
        A.append((_rng(w.family, _T_LORA_A + mat, r).standard_normal((r, cols), dtype=np.float32)
                  * np.float32(1.0 / np.sqrt(cols))).astype(np.float32))
        B.append((_rng(w.family, _T_LORA_B + mat, r).standard_normal((rows, r), dtype=np.float32)
                  * np.float32(b_sd)).astype(np.float32))
    return A, B


def shared_experts(w: Workload, n: int = 2):
    """The layer's n shared experts in its weight format (K3: 2, LazyLoRA README, "The
    engine"), drawn like routed experts E .. E+n-1: MXFP4 (codes, scales) or RVQ3 (idx, cb),
    each a list over gate, up, down with a leading dimension n."""
    ids = range(w.E, w.E + n)
    return mxfp4_layer(w, ids) if w.wfmt == "mxfp4" else rvq3_layer(w, ids)


def shrink(w: Workload, **kw) -> Workload:
    """A workload with some fields replaced (used by tests for reduced sizes)."""
    return dataclasses.replace(w, **kw)


# K3's model width around the 3,584-wide latent space is not on the pages; this stands in for it
# (twice the latent width) where a K3-shaped test needs one.
K3_MODEL_WIDTH_ASSUMED = 7168


def latent_projections(w: Workload, D: int):
    """proj_in [H][D] and proj_out [D][H] as bf16 bit patterns: N(0, 1/in_width), so the
    projected activations keep unit scale."""
    pin = _rng(w.family, _T_PROJ_IN, D).standard_normal((w.H, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    pout = _rng(w.family, _T_PROJ_OUT, D).standard_normal((D, w.H), dtype=np.float32) * np.float32(1.0 / np.sqrt(w.H))
    return f32_to_bf16_bits(pin), f32_to_bf16_bits(pout)


def model_activations(w: Workload, D: int, T: Optional[int] = None) -> np.ndarray:
    """x_model [T][D]: N(0,1) rounded to bf16 bits (fp32 for the fp32-activation workload)."""
    T = w.T if T is None else T
    x = _rng(w.family, _T_XM, w.x_key).standard_normal((T, D), dtype=np.float32)
    return x if w.x_dtype == "f32" else f32_to_bf16_bits(x)


def model_upstream_grad(w: Workload, D: int, T: Optional[int] = None) -> np.ndarray:
    """dout [T][D]: N(0, 0.01^2) rounded to bf16 bits (fp32 for the fp32-activation workload)."""
    T = w.T if T is None else T
    d = _rng(w.family, _T_DOUT, w.x_key).standard_normal((T, D), dtype=np.float32) * np.float32(0.01)
    return d if w.x_dtype == "f32" else f32_to_bf16_bits(d)
