"""Routed-expert MoE layer for AMD Instinct MI355X (gfx950): Python binding.

Every step of the layer runs in the HIP kernels of libmoe_mi355x.so behind
the C ABI of include/moe.h.  This module only allocates device buffers with
PyTorch, passes their addresses and the current stream, and checks status
codes.  If the library is missing it raises; there is no other path.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import _lib as C
from ._lib import MoeError  # noqa: F401

__all__ = ["MoELayer", "Routing", "MoeError", "to_device", "bf16_tensor", "lib_path"]


def lib_path() -> str:
    from .build import LIB_PATH
    return LIB_PATH


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return C.MOE_DT_BF16
    if t.dtype == torch.float32:
        return C.MOE_DT_F32
    raise TypeError(f"unsupported activation dtype {t.dtype} (bf16 or fp32)")


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def to_device(a: np.ndarray, device="cuda"):
    """Upload a numpy array unchanged (uint16 arrays keep their bits)."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bf16_tensor(bits: np.ndarray, device="cuda"):
    """bf16 device tensor from uint16 bit patterns."""
    return to_device(np.ascontiguousarray(bits, np.uint16), device).view(_torch().bfloat16)


@dataclass
class Routing:
    """Routing record written by MoELayer.route (device tensors); see include/moe.h."""
    T: int
    ids: object
    w: object
    counts: object
    offsets: object
    perm: object
    inv: object
    active: object
    n_active: object

    def c_struct(self) -> C.MoeRouting:
        r = C.MoeRouting()
        for n in ("ids", "w", "counts", "offsets", "perm", "inv", "active", "n_active"):
            setattr(r, n, getattr(self, n).data_ptr())
        return r


class MoELayer:
    """One routed-expert layer over borrowed device weights.

    MXFP4: pass codes=[gate, up, down] ([E][out][in/2] uint8) and scales ([E][out][in/32] uint8).
    RVQ3:  pass rvq_idx=[...] ([E][3][out][in/8] uint8) and rvq_cb=[...] ([E][3][256][8] fp16 bits).
    router_w: [E][H] fp32; router_b: [E] fp32 or None.  bias_mode: 1 (default with a bias) adds
    the bias to the logits, 2 uses it for the selection only.  Shared experts (taken by every
    token with weight 1): shared=[gate, up, down] in the routed experts' format with n_shared in
    place of E (MXFP4: a pair (codes, scales) of such lists; RVQ3: (rvq_idx, rvq_cb)).  Latent
    projections: proj=(proj_in [H][D], proj_out [D][H]) bf16 (uint16 bits or torch.bfloat16), D the
    model width.  All tensors on the same GPU and kept alive by this object.
    """

    def __init__(self, *, hidden: int, inter: int, n_experts: int, top_k: int, max_tokens: int, router_w,
                 router_b=None, codes: Optional[Sequence] = None, scales: Optional[Sequence] = None,
                 rvq_idx: Optional[Sequence] = None, rvq_cb: Optional[Sequence] = None, flags: int = 0,
                 act: int = 0, bias_mode: Optional[int] = None, shared=None, proj=None):
        torch = _torch()
        L = C.lib()
        d = C.MoeDesc()
        L.moe_desc_init(ctypes.byref(d))
        d.hidden, d.inter, d.n_experts, d.top_k, d.max_tokens = hidden, inter, n_experts, top_k, max_tokens
        d.wfmt = C.MOE_W_MXFP4 if codes is not None else C.MOE_W_RVQ3
        d.bias_mode = (1 if router_b is not None else 0) if bias_mode is None else bias_mode
        d.flags |= flags
        d.act = act
        d.n_shared = 0 if shared is None else int(shared[0][0].shape[0])
        d.model_width = 0 if proj is None else int(proj[0].shape[1])
        self.D = d.model_width
        self.desc = d
        self.H, self.I, self.E, self.k, self.max_tokens = hidden, inter, n_experts, top_k, max_tokens
        self.device = router_w.device
        self._keep = [router_w, router_b, codes, scales, rvq_idx, rvq_cb, shared, proj]
        self._lora = None
        w = C.MoeWeights()
        w.router_w = router_w.data_ptr()
        w.router_b = _ptr(router_b)
        for m in range(3):
            if codes is not None:
                w.codes[m] = codes[m].data_ptr()
                w.scales[m] = scales[m].data_ptr()
            else:
                w.rvq_idx[m] = rvq_idx[m].data_ptr()
                w.rvq_cb[m] = rvq_cb[m].data_ptr()
            if shared is not None and codes is not None:
                w.shared_codes[m] = shared[0][m].data_ptr()
                w.shared_scales[m] = shared[1][m].data_ptr()
            elif shared is not None:
                w.shared_rvq_idx[m] = shared[0][m].data_ptr()
                w.shared_rvq_cb[m] = shared[1][m].data_ptr()
        if proj is not None:
            w.proj_in, w.proj_out = proj[0].data_ptr(), proj[1].data_ptr()
        self.weights = w
        nbytes = ctypes.c_size_t()
        C.check(L.moe_workspace_size(ctypes.byref(d), ctypes.byref(nbytes)), "moe_workspace_size")
        self.workspace_bytes = nbytes.value
        self.workspace = torch.empty(max(256, nbytes.value), dtype=torch.uint8, device=self.device)
        h = ctypes.c_void_p()
        C.check(L.moe_layer_create(ctypes.byref(d), ctypes.byref(w), self.workspace.data_ptr(),
                                   self.workspace.numel(), ctypes.byref(h)), "moe_layer_create")
        self._h = h

    # ------------------------------------------------------------------
    def new_routing(self, T: int) -> Routing:
        torch = _torch()
        i32 = dict(dtype=torch.int32, device=self.device)
        S = max(1, T * self.k)
        return Routing(T, torch.empty((T, self.k), **i32), torch.empty((T, self.k), dtype=torch.float32,
                                                                    device=self.device),
                       torch.empty(self.E, **i32), torch.empty(self.E + 1, **i32), torch.empty(S, **i32),
                       torch.empty(S, **i32), torch.empty(self.E, **i32), torch.empty(1, **i32))

    def route(self, x, routing: Optional[Routing] = None) -> Routing:
        T = x.shape[0]
        r = routing or self.new_routing(T)
        rs = r.c_struct()
        C.check(C.lib().moe_route(self._h, x.data_ptr(), _dtype_code(x), T, ctypes.byref(rs), _stream()),
                "moe_route")
        return r

    def forward(self, x, routing: Routing, y=None, saved_gu=None):
        torch = _torch()
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        rs = routing.c_struct()
        C.check(C.lib().moe_forward(self._h, x.data_ptr(), _dtype_code(x), T, ctypes.byref(rs), y.data_ptr(),
                                    _ptr(saved_gu), _stream()), "moe_forward")
        return y

    def forward_static(self, x, routing: Routing, y=None):
        """moe_forward_static: the forward with the library's own per-GPU scratch (no
        workspace, no allocation by the library; y must be preallocated for an
        allocation-free call)."""
        torch = _torch()
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        rs = routing.c_struct()
        C.check(C.lib().moe_forward_static(self._h, x.data_ptr(), _dtype_code(x), T, ctypes.byref(rs), y.data_ptr(),
                                           _stream()), "moe_forward_static")
        return y

    def backward_input(self, x, dy, routing: Routing, saved_gu=None, dx=None):
        torch = _torch()
        T = x.shape[0]
        if dx is None:
            dx = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        rs = routing.c_struct()
        C.check(C.lib().moe_backward_input(self._h, x.data_ptr(), _dtype_code(x), dy.data_ptr(), _dtype_code(dy),
                                           T, ctypes.byref(rs), _ptr(saved_gu), dx.data_ptr(), _stream()),
                "moe_backward_input")
        return dx

    def set_lora(self, A=None, B=None, scale: float = 1.0):
        """Attach the shared low-rank adapter (A = [gate, up, down] fp32 [r][in] device tensors,
        B = [gate, up, down] fp32 [out][r]), or detach it with no arguments.  The layer must
        have been created with flags including MOE_F_LORA."""
        L = C.lib()
        if A is None:
            C.check(L.moe_set_lora(self._h, None), "moe_set_lora")
            self._lora = None
            return
        s = C.MoeLora()
        s.rank, s.scale = int(A[0].shape[0]), float(scale)
        for m in range(3):
            s.A[m], s.B[m] = A[m].data_ptr(), B[m].data_ptr()
        C.check(L.moe_set_lora(self._h, ctypes.byref(s)), "moe_set_lora")
        self._lora = (list(A), list(B), s.rank)

    def backward_lora(self, x, dy, routing: Routing, saved_gu=None, dx=None):
        """Input gradient and the adapter gradients: (dx, dA [3], dB [3])."""
        torch = _torch()
        A, B, r = self._lora
        T = x.shape[0]
        if dx is None:
            dx = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        dA = [torch.empty_like(a) for a in A]
        dB = [torch.empty_like(b) for b in B]
        rs = routing.c_struct()
        vp3 = ctypes.c_void_p * 3
        C.check(C.lib().moe_backward_lora(self._h, x.data_ptr(), _dtype_code(x), dy.data_ptr(), _dtype_code(dy), T,
                                          ctypes.byref(rs), _ptr(saved_gu), dx.data_ptr(),
                                          vp3(*[a.data_ptr() for a in dA]), vp3(*[b.data_ptr() for b in dB]),
                                          _stream()), "moe_backward_lora")
        return dx, dA, dB

    def _project(self, fn, a, T, width, dtype=None):
        torch = _torch()
        out = torch.empty((T, width), dtype=torch.float32, device=self.device)
        L = C.lib()
        if dtype is None:
            C.check(getattr(L, fn)(self._h, a.data_ptr(), T, out.data_ptr(), _stream()), fn)
        else:
            C.check(getattr(L, fn)(self._h, a.data_ptr(), dtype, T, out.data_ptr(), _stream()), fn)
        return out

    def project_in(self, x_model):
        """Latent input x_model proj_in^T [T][H] fp32 (x_model [T][D] bf16 or fp32)."""
        return self._project("moe_project_in", x_model, x_model.shape[0], self.H, _dtype_code(x_model))

    def project_out(self, y_latent):
        """Model-width output y_latent proj_out^T [T][D] fp32 (y_latent [T][H] fp32)."""
        return self._project("moe_project_out", y_latent, y_latent.shape[0], self.D)

    def project_out_backward(self, dout):
        """dy_latent = dout proj_out [T][H] fp32 (dout [T][D] bf16 or fp32)."""
        return self._project("moe_project_out_backward", dout, dout.shape[0], self.H, _dtype_code(dout))

    def project_in_backward(self, dx_latent):
        """dx_model = dx_latent proj_in [T][D] fp32 (dx_latent [T][H] fp32)."""
        return self._project("moe_project_in_backward", dx_latent, dx_latent.shape[0], self.D)

    def check_status(self) -> int:
        """MOE_F_VALIDATE: synchronize, return and clear the device status word (MOE_BAD_* bits);
        raises MoeError(MOE_ERR_DATA) if it was nonzero."""
        bits = ctypes.c_uint32()
        C.check(C.lib().moe_check_status(self._h, ctypes.byref(bits), _stream()), "moe_check_status")
        return bits.value

    def new_saved_gu(self, T: int):
        torch = _torch()
        return torch.empty((max(1, T * self.k), 2, self.I), dtype=torch.float32, device=self.device)

    def prof_enable(self, families, max_launches: int = 4096):
        """Bracket each launch of the given kernel families (ids from _lib.PROF_*) with HIP events."""
        mask = 0
        for f in families:
            mask |= 1 << f
        C.check(C.lib().moe_prof_enable(self._h, mask, max_launches), "moe_prof_enable")

    def prof_read(self, family: int):
        """(total milliseconds, launches) recorded for one kernel family (synchronizes)."""
        ms, n = ctypes.c_double(), ctypes.c_int32()
        C.check(C.lib().moe_prof_read(self._h, family, ctypes.byref(ms), ctypes.byref(n)), "moe_prof_read")
        return ms.value, n.value

    def close(self):
        if getattr(self, "_h", None):
            C.lib().moe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
