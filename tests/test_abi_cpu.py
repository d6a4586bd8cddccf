"""Host-side checks of the C ABI: the library loads, exports every declared entry point, and
rejects bad arguments synchronously without touching the device (no compute calls here)."""
import ctypes
import glob
import os
import re

import pytest

import quantized_moe_route_amd as q
from quantized_moe_route_amd import _lib as C

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def _declared():
    names = set()
    for h in glob.glob(os.path.join(INCLUDE, "*.h")):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    assert _declared() == sorted(C.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = C.lib()
    for name in _declared():
        assert hasattr(L, name), name


def _desc(**kw):
    d = C.MoeDesc()
    C.lib().moe_desc_init(ctypes.byref(d))
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_desc_defaults_are_the_k3_layer():
    d = _desc()
    assert (d.hidden, d.inter, d.n_experts, d.top_k, d.max_tokens) == (3584, 3072, 896, 16, 4096)
    assert d.wfmt == C.MOE_W_MXFP4 and d.act == C.MOE_ACT_SWIGLU and d.bias_mode == 0


def test_workspace_size_and_desc_validation():
    L = C.lib()
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=1)), ctypes.byref(n)) == C.MOE_OK
    small = n.value
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=64)), ctypes.byref(n)) == C.MOE_OK
    assert n.value > small
    bad = [dict(hidden=100), dict(inter=0), dict(n_experts=0), dict(n_experts=5000), dict(top_k=0),
           dict(top_k=65), dict(n_experts=8, top_k=9), dict(max_tokens=-1), dict(wfmt=7), dict(bias_mode=3),
           dict(act=2), dict(act=-1)]
    for act in (C.MOE_ACT_SWIGLU, C.MOE_ACT_SITU):
        assert L.moe_workspace_size(ctypes.byref(_desc(act=act)), ctypes.byref(n)) == C.MOE_OK
    for kw in bad:
        st = L.moe_workspace_size(ctypes.byref(_desc(**kw)), ctypes.byref(n))
        assert st in (C.MOE_ERR_INVALID_ARG, C.MOE_ERR_UNSUPPORTED), kw
        assert L.moe_last_error()
    assert L.moe_workspace_size(None, ctypes.byref(n)) == C.MOE_ERR_INVALID_ARG


def _fake_weights(wfmt=C.MOE_W_MXFP4, align=256):
    # host-side validation only reads the pointer values; nothing dereferences them here
    w = C.MoeWeights()
    w.router_w = 0x10000
    for m in range(3):
        if wfmt == C.MOE_W_MXFP4:
            w.codes[m] = 0x20000 + m * align
            w.scales[m] = 0x30000 + m * 256
        else:
            w.rvq_idx[m] = 0x20000 + m * align
            w.rvq_cb[m] = 0x30000 + m * 256
    return w


def _create(d, w, ws=0x100000, ws_bytes=None):
    L = C.lib()
    if ws_bytes is None:
        n = ctypes.c_size_t()
        L.moe_workspace_size(ctypes.byref(d), ctypes.byref(n))
        ws_bytes = n.value
    h = ctypes.c_void_p()
    st = L.moe_layer_create(ctypes.byref(d), ctypes.byref(w), ws, ws_bytes, ctypes.byref(h))
    return st, h


def test_create_validation_and_destroy():
    L = C.lib()
    d = _desc(max_tokens=8)
    st, h = _create(d, _fake_weights())
    assert st == C.MOE_OK and h.value
    L.moe_destroy(h)
    L.moe_destroy(None)
    w = _fake_weights()
    w.codes[1] = None
    assert _create(d, w)[0] == C.MOE_ERR_INVALID_ARG and b"up" in L.moe_last_error()
    assert _create(d, _fake_weights(align=8))[0] == C.MOE_ERR_INVALID_ARG  # codes not 16-byte aligned
    w = _fake_weights()
    w.router_w = None
    assert _create(d, w)[0] == C.MOE_ERR_INVALID_ARG
    assert _create(_desc(max_tokens=8, bias_mode=1), _fake_weights())[0] == C.MOE_ERR_INVALID_ARG
    assert _create(_desc(max_tokens=8, bias_mode=2), _fake_weights())[0] == C.MOE_ERR_INVALID_ARG
    assert _create(d, _fake_weights(), ws_bytes=16)[0] == C.MOE_ERR_WORKSPACE
    assert _create(d, _fake_weights(), ws=0x100010)[0] == C.MOE_ERR_WORKSPACE
    assert _create(_desc(max_tokens=8, wfmt=C.MOE_W_RVQ3), _fake_weights())[0] == C.MOE_ERR_INVALID_ARG
    st, h = _create(_desc(max_tokens=8, wfmt=C.MOE_W_RVQ3), _fake_weights(C.MOE_W_RVQ3))
    assert st == C.MOE_OK
    L.moe_destroy(h)


def test_calls_reject_bad_arguments_before_enqueueing():
    L = C.lib()
    d = _desc(max_tokens=8)
    st, h = _create(d, _fake_weights())
    assert st == C.MOE_OK
    r = C.MoeRouting()
    for i, n in enumerate(("ids", "w", "counts", "offsets", "perm", "inv", "active", "n_active")):
        setattr(r, n, 0x40000 + 256 * i)
    x, y = 0x50000, 0x60000
    # T beyond max_tokens, negative T, bad dtype, null routing, null/misaligned x
    assert L.moe_route(h, x, C.MOE_DT_BF16, 9, ctypes.byref(r), None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_route(h, x, C.MOE_DT_BF16, -1, ctypes.byref(r), None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_route(h, x, 5, 1, ctypes.byref(r), None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_route(h, x, C.MOE_DT_BF16, 1, None, None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_route(h, None, C.MOE_DT_BF16, 1, ctypes.byref(r), None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_route(h, x + 2, C.MOE_DT_BF16, 1, ctypes.byref(r), None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, x, C.MOE_DT_BF16, 1, ctypes.byref(r), None) == C.MOE_ERR_INVALID_ARG
    r2 = C.MoeRouting()
    ctypes.memmove(ctypes.byref(r2), ctypes.byref(r), ctypes.sizeof(r))
    r2.perm = None
    assert L.moe_route(h, x, C.MOE_DT_BF16, 1, ctypes.byref(r2), None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_forward(h, x, C.MOE_DT_BF16, 1, ctypes.byref(r), None, None, None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_forward(h, x, C.MOE_DT_BF16, 1, ctypes.byref(r), y + 4, None, None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_backward_input(h, x, C.MOE_DT_BF16, None, C.MOE_DT_BF16, 1, ctypes.byref(r), None, y,
                                None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_backward_input(h, x, C.MOE_DT_BF16, x, 9, 1, ctypes.byref(r), None, y, None) == C.MOE_ERR_INVALID_ARG
    # T = 0 is a valid no-op that touches nothing
    assert L.moe_route(h, None, C.MOE_DT_BF16, 0, ctypes.byref(r), None) == C.MOE_OK
    assert L.moe_forward(h, None, C.MOE_DT_BF16, 0, ctypes.byref(r), None, None, None) == C.MOE_OK
    assert L.moe_backward_input(h, None, C.MOE_DT_BF16, None, C.MOE_DT_BF16, 0, ctypes.byref(r), None, None,
                                None) == C.MOE_OK
    assert L.moe_route(h, None, C.MOE_DT_BF16, 0, None, None) == C.MOE_OK  # empty buffers may be NULL
    assert L.moe_status_string(C.MOE_ERR_DEVICE) == b"device error"
    L.moe_destroy(h)


def test_prof_argument_checks():
    L = C.lib()
    st, h = _create(_desc(max_tokens=8), _fake_weights())
    assert L.moe_prof_enable(None, 1, 4) == C.MOE_ERR_INVALID_ARG
    assert L.moe_prof_enable(h, 1, 0) == C.MOE_ERR_INVALID_ARG
    assert L.moe_prof_enable(h, 0, 0) == C.MOE_OK  # disable needs no events
    ms, n = ctypes.c_double(), ctypes.c_int32()
    assert L.moe_prof_read(h, 99, ctypes.byref(ms), ctypes.byref(n)) == C.MOE_ERR_INVALID_ARG
    assert L.moe_prof_read(h, 3, ctypes.byref(ms), ctypes.byref(n)) == C.MOE_OK and n.value == 0
    L.moe_destroy(h)
    # the reference stream checks its buffer before launching anything
    assert L.moe_prof_hbm_read(None, 1024, None, ctypes.byref(ms)) == C.MOE_ERR_INVALID_ARG
    assert L.moe_prof_hbm_read(0x1000, 1000, None, ctypes.byref(ms)) == C.MOE_ERR_INVALID_ARG  # not 16-byte sized
    assert L.moe_prof_hbm_read(0x1008, 1024, None, ctypes.byref(ms)) == C.MOE_ERR_INVALID_ARG  # misaligned
    assert L.moe_prof_hbm_read(0x1000, 1024, None, None) == C.MOE_ERR_INVALID_ARG


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(C, "_lib", None)
    monkeypatch.setattr(C, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        C.lib()


def _fake_lora(rank=16, scale=2.0, align=256):
    s = C.MoeLora()
    s.rank, s.scale = rank, scale
    for m in range(3):
        s.A[m] = 0x40000 + m * align
        s.B[m] = 0x50000 + m * align
    return s


def test_lora_argument_checks():
    L = C.lib()
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=8)), ctypes.byref(n0)) == C.MOE_OK
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=8, flags=C.MOE_F_LORA)), ctypes.byref(n1)) == C.MOE_OK
    assert n1.value > n0.value  # the adapter's buffers
    # a layer sized without MOE_F_LORA refuses an adapter
    st, h = _create(_desc(max_tokens=8), _fake_weights())
    assert st == C.MOE_OK
    assert L.moe_set_lora(h, ctypes.byref(_fake_lora())) == C.MOE_ERR_INVALID_ARG
    assert L.moe_set_lora(h, None) == C.MOE_OK  # detaching is always allowed
    # moe_backward_lora needs an attached adapter (checked before anything else is touched)
    vp3 = ctypes.c_void_p * 3
    r = C.MoeRouting()
    dA, dB = vp3(0x1000, 0x2000, 0x3000), vp3(0x4000, 0x5000, 0x6000)
    assert L.moe_backward_lora(h, 0x1000, C.MOE_DT_BF16, 0x1000, C.MOE_DT_BF16, 1, ctypes.byref(r), None, 0x1000, dA, dB,
                               None) == C.MOE_ERR_INVALID_ARG
    L.moe_destroy(h)
    st, h = _create(_desc(max_tokens=8, flags=C.MOE_F_LORA), _fake_weights())
    assert st == C.MOE_OK
    assert L.moe_set_lora(None, ctypes.byref(_fake_lora())) == C.MOE_ERR_INVALID_ARG
    for bad in (_fake_lora(rank=0), _fake_lora(rank=65), _fake_lora(scale=float("inf")), _fake_lora(scale=float("nan")),
                _fake_lora(align=8)):
        assert L.moe_set_lora(h, ctypes.byref(bad)) == C.MOE_ERR_INVALID_ARG
    nul = _fake_lora()
    nul.B[2] = None
    assert L.moe_set_lora(h, ctypes.byref(nul)) == C.MOE_ERR_INVALID_ARG
    assert L.moe_set_lora(h, ctypes.byref(_fake_lora())) == C.MOE_OK
    assert L.moe_set_lora(h, ctypes.byref(_fake_lora(rank=64))) == C.MOE_OK
    # with an adapter: NULL or misaligned gradient buffers are refused
    assert L.moe_backward_lora(h, 0x1000, C.MOE_DT_BF16, 0x1000, C.MOE_DT_BF16, 1, ctypes.byref(r), None, 0x1000, None, dB,
                               None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_backward_lora(h, 0x1000, C.MOE_DT_BF16, 0x1000, C.MOE_DT_BF16, 1, ctypes.byref(r), None, 0x1000,
                               vp3(0x1000, 0x2008, 0x3000), dB, None) == C.MOE_ERR_INVALID_ARG
    L.moe_destroy(h)


def test_shared_expert_argument_checks():
    L = C.lib()
    assert _desc().n_shared == 0
    n0, n2 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=8)), ctypes.byref(n0)) == C.MOE_OK
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=8, n_shared=2)), ctypes.byref(n2)) == C.MOE_OK
    assert n2.value > n0.value  # the shared experts' slot rows and routing
    for bad in (dict(n_shared=-1), dict(n_shared=17), dict(n_experts=8, top_k=2, n_shared=3)):
        assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=8, **bad)), ctypes.byref(n0)) == C.MOE_ERR_INVALID_ARG
    d = _desc(max_tokens=8, n_shared=2)
    assert _create(d, _fake_weights())[0] == C.MOE_ERR_INVALID_ARG  # shared weights missing
    w = _fake_weights()
    for m in range(3):
        w.shared_codes[m] = 0x40000 + m * 256
        w.shared_scales[m] = 0x50000 + m * 256
    st, h = _create(d, w)
    assert st == C.MOE_OK
    L.moe_destroy(h)
    w.shared_scales[1] = 0x50008
    assert _create(d, w)[0] == C.MOE_ERR_INVALID_ARG  # misaligned
    # RVQ3 layers take the RVQ3 arrays of the shared experts
    d3 = _desc(max_tokens=8, n_shared=1, wfmt=C.MOE_W_RVQ3)
    w3 = _fake_weights(C.MOE_W_RVQ3)
    assert _create(d3, w3)[0] == C.MOE_ERR_INVALID_ARG
    for m in range(3):
        w3.shared_rvq_idx[m] = 0x40000 + m * 256
        w3.shared_rvq_cb[m] = 0x50000 + m * 256
    st, h = _create(d3, w3)
    assert st == C.MOE_OK
    L.moe_destroy(h)


def test_validate_argument_checks():
    """MOE_F_VALIDATE: the status call exists and needs a validating layer (no device work here)."""
    L = C.lib()
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=8)), ctypes.byref(n0)) == C.MOE_OK
    assert L.moe_workspace_size(ctypes.byref(_desc(max_tokens=8, flags=C.MOE_F_VALIDATE)), ctypes.byref(n1)) == C.MOE_OK
    assert n1.value == n0.value  # the status word is always part of the workspace
    bits = ctypes.c_uint32(7)
    assert L.moe_check_status(None, ctypes.byref(bits), None) == C.MOE_ERR_INVALID_ARG
    st, h = _create(_desc(max_tokens=8), _fake_weights())
    assert st == C.MOE_OK
    assert L.moe_check_status(h, ctypes.byref(bits), None) == C.MOE_ERR_INVALID_ARG
    assert b"MOE_F_VALIDATE" in L.moe_last_error()
    L.moe_destroy(h)
    st, h = _create(_desc(max_tokens=8, flags=C.MOE_F_VALIDATE), _fake_weights(), ws_bytes=n1.value)
    assert st == C.MOE_OK
    assert L.moe_check_status(h, None, None) == C.MOE_ERR_INVALID_ARG
    # arguments are still checked before the status word is read
    r = C.MoeRouting()
    assert L.moe_route(h, 0x50000, C.MOE_DT_BF16, 9, ctypes.byref(r), None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_status_string(C.MOE_ERR_DATA) == b"out-of-contract data"
    L.moe_destroy(h)


def test_static_forward_argument_checks():
    """moe_forward_static refuses, before touching the device, token counts whose scratch
    exceeds its 32 MiB array and layers it does not serve."""
    L = C.lib()
    st, h = _create(_desc(max_tokens=4096), _fake_weights())
    assert st == C.MOE_OK
    r = C.MoeRouting()
    for i, n in enumerate(("ids", "w", "counts", "offsets", "perm", "inv", "active", "n_active")):
        setattr(r, n, 0x40000 + 256 * i)
    x, y = 0x50000, 0x60000
    # K3 shape: 26,624 bytes per slot, 16 slots per token: 79 tokens no longer fit
    assert L.moe_forward_static(h, x, C.MOE_DT_BF16, 79, ctypes.byref(r), y, None) == C.MOE_ERR_WORKSPACE
    assert b"32" in L.moe_last_error() or b"33554432" in L.moe_last_error()
    assert L.moe_forward_static(h, x, C.MOE_DT_BF16, 1, None, y, None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_forward_static(h, x, C.MOE_DT_BF16, 1, ctypes.byref(r), y + 4, None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_forward_static(h, None, C.MOE_DT_BF16, 0, ctypes.byref(r), None, None) == C.MOE_OK
    L.moe_destroy(h)
    st, h = _create(_desc(max_tokens=8, flags=C.MOE_F_QUANT_X8), _fake_weights())
    assert L.moe_forward_static(h, x, C.MOE_DT_BF16, 1, ctypes.byref(r), y, None) == C.MOE_ERR_UNSUPPORTED
    L.moe_destroy(h)
    # RVQ3 holds g and u (8 I bytes per slot) where the other formats hold h (4 I): at the K3
    # shape 38,912 bytes per slot, so 53 tokens fit and 54 do not (53 passes the size check
    # and stops at the missing routing)
    st, h = _create(_desc(max_tokens=4096, wfmt=C.MOE_W_RVQ3), _fake_weights(C.MOE_W_RVQ3))
    assert st == C.MOE_OK
    assert L.moe_forward_static(h, x, C.MOE_DT_BF16, 54, ctypes.byref(r), y, None) == C.MOE_ERR_WORKSPACE
    assert L.moe_forward_static(h, x, C.MOE_DT_BF16, 53, None, y, None) == C.MOE_ERR_INVALID_ARG
    L.moe_destroy(h)


def test_latent_projection_argument_checks():
    """model_width: 0 or a multiple of 64 (with H a multiple of 64); a layer with it needs both
    projection matrices, 16-byte aligned; projection calls on a layer without them fail."""
    L = C.lib()
    n = ctypes.c_size_t()
    for mw in (-64, 100, 32):
        assert L.moe_workspace_size(ctypes.byref(_desc(model_width=mw)), ctypes.byref(n)) == C.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_size(ctypes.byref(_desc(model_width=512, hidden=3552)), ctypes.byref(n)) == C.MOE_ERR_INVALID_ARG
    d = _desc(max_tokens=8, model_width=7168)
    assert _create(d, _fake_weights())[0] == C.MOE_ERR_INVALID_ARG  # no projections given
    w = _fake_weights()
    w.proj_in, w.proj_out = 0x70000, 0x80008  # proj_out misaligned
    assert _create(d, w)[0] == C.MOE_ERR_INVALID_ARG
    w.proj_out = 0x80000
    st, h = _create(d, w)
    assert st == C.MOE_OK
    assert L.moe_project_in(h, None, C.MOE_DT_BF16, 1, 0x90000, None) == C.MOE_ERR_INVALID_ARG
    assert L.moe_project_out(h, 0x90000, 9, 0xA0000, None) == C.MOE_ERR_INVALID_ARG  # T > max_tokens
    assert L.moe_project_out(h, None, 0, None, None) == C.MOE_OK  # T = 0
    L.moe_destroy(h)
    st, h = _create(_desc(max_tokens=8), _fake_weights())
    assert L.moe_project_in(h, 0x90000, C.MOE_DT_BF16, 1, 0xA0000, None) == C.MOE_ERR_INVALID_ARG
    assert b"model_width" in L.moe_last_error()
    L.moe_destroy(h)
