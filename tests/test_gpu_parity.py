"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded
inputs.  Routing ids, grouping and permutations must be bit-exact; y, dX and the routing
weights within max|err| / max|ref| <= 1e-4."""
import numpy as np
import pytest

import moe_synth as syn
import oracle
from cases import TOL, act_tensor, device_layer, fnv1a32, host_case, log, rel_err

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _np(t):
    return t.detach().cpu().numpy()


def check_routing(r, ids, p, E, name):
    _sync()
    gids = _np(r.ids)
    assert np.array_equal(gids, ids), f"{name}: routing ids differ at {np.argwhere(gids != ids)[:5]}"
    assert rel_err(_np(r.w), p) <= TOL, f"{name}: routing weights"
    g = oracle.group(ids, E)
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(_np(getattr(r, key))[: g[key].size], g[key]), f"{name}: {key}"
    n = int(_np(r.n_active)[0])
    assert n == g["n_active"] and np.array_equal(_np(r.active)[:n], g["active"][:n]), f"{name}: active"


def run_small(c, T=None, saved=True, name="", flags=0):
    """Full comparison of route, forward and (when dY is present) backward."""
    w = c.w
    T = w.T if T is None else T
    log(f"case {name}: T={T} H={w.H} I={w.I} E={w.E} k={w.k} fmt={w.wfmt} x={w.x_dtype} flags={flags}")
    L = device_layer(c, max_tokens=max(T, 1), flags=flags)
    x = act_tensor(c.x, w.x_dtype)
    r = L.route(x)
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k, bias_mode=c.bias_mode)
    check_routing(r, ids, p, w.E, name)
    W = c.oracle_weights()
    y_ref = oracle.forward(c.x64, ids, p, W)
    gu = L.new_saved_gu(T) if saved else None
    y = L.forward(x, r, saved_gu=gu)
    _sync()
    e = rel_err(_np(y), y_ref)
    log(f"  y rel err {e:.3e}")
    assert e <= TOL, f"{name}: y rel err {e}"
    if c.dy is not None:
        dy = act_tensor(c.dy, w.x_dtype)
        dx_ref = oracle.backward_input(c.x64, c.dy64, ids, p, c.wr, W)
        for g in ([gu, None] if saved else [None]):
            dx = L.backward_input(x, dy, r, saved_gu=g)
            _sync()
            e = rel_err(_np(dx), dx_ref)
            log(f"  dX rel err {e:.3e} (saved_gu={'yes' if g is not None else 'no'})")
            # g, u saved by the block-scaled gate/up carry its summation deviation: the bound
            # include/moe.h states for MOE_F_MX_GATEUP; recomputed ones are exact
            bound = MX_SAVED_BOUND if g is not None and flags & 2 else TOL
            assert e <= bound, f"{name}: dX rel err {e}"
    return L, x, r, y


TINY = syn.WORKLOADS["tiny"]
MX_SAVED_BOUND = 7e-4  # dX from the g, u a MOE_F_MX_GATEUP forward saved (include/moe.h)


def test_tiny_config_full():
    run_small(host_case(TINY), name="tiny")


def test_tiny_bf16_activations_and_bias():
    w = syn.shrink(TINY, x_dtype="bf16", bias_sd=0.5, x_key=7)
    run_small(host_case(w), name="tiny-bf16-bias")


@pytest.mark.parametrize("T,k,E", [(1, 8, 64), (4, 16, 128), (8, 2, 16), (100, 4, 40)])
def test_selection_only_router_bias(T, k, E):
    """bias_mode 2: the bias (sd 1, large against the logits) decides the selection, the
    unbiased logits the weights; the fused small-batch routing (T <= 4), the per-token
    top-k kernel, the generic and few-token expert paths, and the router term of dX."""
    w = syn.shrink(TINY, T=T, k=k, E=E, x_dtype="bf16", bias_sd=1.0, with_dy=True, x_key=70 + T)
    c = host_case(w)
    c.bias_mode = 2
    run_small(c, name=f"bias-select-T{T}")


def test_ragged_shapes_span_tiles():
    # H, I multiples of 32 but not of 64 or 256; T, E, k odd-sized
    w = syn.shrink(TINY, T=37, H=160, I=96, E=20, k=3, x_key=8)
    run_small(host_case(w), name="ragged")


def test_many_tokens_per_expert_uses_multi_tile_path():
    # T > 64 selects the 4-tile token path; 8 experts with k=4 give ~50 tokens per expert
    w = syn.shrink(TINY, T=100, E=8, k=4, x_dtype="bf16", x_key=9)
    run_small(host_case(w), name="multi-tile")


def test_grouped_gemm_path_multi_pass():
    # T * k >= 8 E with MXFP4, bf16 x and H, I multiples of 512 selects the grouped-GEMM
    # kernels; ~100 tokens per expert puts some experts over one 96-token pass
    w = syn.shrink(TINY, T=400, H=512, I=1024, E=8, k=2, x_dtype="bf16", x_key=15)
    run_small(host_case(w), name="mm-multi-pass")


def test_grouped_gemm_path_skew_and_idle_experts():
    # one expert takes every token (four passes, the last a single partial tile); with
    # E = 24 and k = 3 most experts see one or two tiles and some none
    w = syn.shrink(TINY, T=300, H=1024, I=512, E=24, k=3, x_dtype="bf16", bias_sd=0.0, x_key=16)
    c = host_case(w)
    c.bias = np.zeros(w.E, np.float32)
    c.bias[5] = 100.0
    run_small(c, name="mm-skew")


@pytest.mark.parametrize("mx", [False, True])
def test_grouped_gemm_scale_chunks(mx):
    # H = I = 4096: the blocks stage their weight rows' scale bytes in LDS 3584 elements of K
    # at a time, so the gate/up (32 K-steps) and the down (64 K-steps) each cross one chunk
    # boundary, the second chunk a short one
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, T=16, H=4096, I=4096, E=4, k=2, x_dtype="bf16", with_dy=not mx, x_key=27)
    run_small(host_case(w), name="mm-scale-chunks" + ("-mx" if mx else ""), flags=C.MOE_F_MX_GATEUP if mx else 0)


def test_block_scaled_gateup_multi_pass_and_recompute():
    # MOE_F_MX_GATEUP: the grouped-GEMM gate/up on block-scaled MFMA (FP4 weights, x as two
    # E4M3 terms); ~100 tokens per expert spans every token-tile count and a second pass;
    # the backward without saved g/u recomputes them on the same kernel
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, T=400, H=512, I=1024, E=8, k=2, x_dtype="bf16", with_dy=True, x_key=25)
    run_small(host_case(w), saved=False, name="mx-multi-pass", flags=C.MOE_F_MX_GATEUP)


def test_block_scaled_gateup_skew():
    # one expert takes every token (four passes, the last a single partial tile)
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, T=300, H=1024, I=512, E=24, k=3, x_dtype="bf16", bias_sd=0.0, with_dy=True, x_key=26)
    c = host_case(w)
    c.bias = np.zeros(w.E, np.float32)
    c.bias[5] = 100.0
    run_small(c, name="mx-skew", flags=C.MOE_F_MX_GATEUP)


def test_block_scaled_gateup_wide_x_range_deviation():
    """x elements spread over 2^-12 .. 2^6 inside each 32-block.  The two E4M3 terms still
    carry the small elements to ~2^-21 of the block maximum, but the block-scaled MFMA's own
    summation then loses precision on the small products.  y stays within the 1e-4 gate
    (measured ~6e-5), and so does dX recomputed on the exact path (saved_gu = NULL); dX from
    the g, u saved by the block-scaled forward is the gradient at those pre-activations and is
    checked against the bound the header states (measured ~6e-4)."""
    import quantized_moe_route_amd as q
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(TINY, T=300, H=1024, I=512, E=24, k=3, x_dtype="bf16", with_dy=True, x_key=27)
    c = host_case(w)
    rng = np.random.default_rng(27)
    f = (c.x.astype(np.uint32) << 16).view(np.float32) * np.exp2(rng.integers(-12, 7, size=c.x.shape)).astype(np.float32)
    c.x = (f.view(np.uint32) >> 16).astype(np.uint16)  # power-of-two scaling: still exact bf16
    ids, p, _ = oracle.route(c.x64, c.wr, c.bias, w.k)
    W = c.oracle_weights()
    y_ref = oracle.forward(c.x64, ids, p, W)
    dx_ref = oracle.backward_input(c.x64, c.dy64, ids, p, c.wr, W)
    errs = {}
    for name, flags in (("bf16", 0), ("mx", C.MOE_F_MX_GATEUP)):
        L = device_layer(c, max_tokens=w.T, flags=flags)
        x, dy = act_tensor(c.x, "bf16"), act_tensor(c.dy, "bf16")
        r = L.route(x)
        gu = L.new_saved_gu(w.T)
        y = L.forward(x, r, saved_gu=gu)
        dx_saved = L.backward_input(x, dy, r, saved_gu=gu)
        dx = L.backward_input(x, dy, r, saved_gu=None)
        _sync()
        errs[name] = (rel_err(_np(y), y_ref), rel_err(_np(dx), dx_ref), rel_err(_np(dx_saved), dx_ref))
        log(f"  wide-range x, {name} gate/up: y rel err {errs[name][0]:.3e}, dX rel err {errs[name][1]:.3e} "
            f"(recomputed), {errs[name][2]:.3e} (from the saved g, u)")
    assert max(errs["bf16"]) <= TOL
    assert errs["mx"][0] <= TOL and errs["mx"][1] <= TOL
    assert errs["mx"][2] <= MX_SAVED_BOUND


def _scale_x(c, e):
    """Multiply every activation by 2^e (exact for bf16 bits and fp32)."""
    if c.w.x_dtype == "bf16":
        f = (c.x.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0**e)
        c.x = (f.view(np.uint32) >> 16).astype(np.uint16)
    else:
        c.x = (c.x * np.float32(2.0**e)).astype(np.float32)


SITU_CASES = {
    # name: (workload overrides, x scale exponent, flags): the generic kernels (fp32 x), the
    # single-token and few-token stream kernels, the grouped GEMMs with their backward, the
    # block-scaled gate/up, the RVQ3 gather kernels; x scaled so that g/4 and u/25 reach the
    # bent parts of both tanh branches.  The SiTU derivatives sech^2(g/4) and s (1 - s) change
    # by a relative amount of the order of the ABSOLUTE error of g, so dX's relative error
    # grows like max|g| times the precision x enters the products with: exact for bf16 x on
    # the bf16 paths and for fp32 x (three bf16 terms hold all 24 significand bits).  The
    # block-scaled gate/up's forward (two E4M3 terms) is checked on y only; its backward
    # recomputes g, u on the exact path.
    "generic": (dict(T=37, with_dy=True), 5, 0),
    "dec-T1": (dict(T=1, H=1024, I=256, E=16, k=8, x_dtype="bf16"), 5, 0),
    "dec-few": (dict(T=6, H=512, I=768, E=12, k=3, x_dtype="bf16", with_dy=True), 5, 0),
    "mm": (dict(T=400, H=512, I=1024, E=8, k=2, x_dtype="bf16", with_dy=True), 5, 0),
    "mm-mx": (dict(T=400, H=512, I=1024, E=8, k=2, x_dtype="bf16"), 5, 2),
}


@pytest.mark.parametrize("case", sorted(SITU_CASES))
def test_situ_activation_paths(case):
    """SiTU experts (MOE_ACT_SITU) through every forward and backward kernel family."""
    over, e, flags = SITU_CASES[case]
    w = syn.shrink(TINY, x_key=30, **over)
    c = host_case(w)
    c.act = 1
    _scale_x(c, e)
    run_small(c, name=f"situ-{case}", flags=flags)


def test_situ_activation_rvq3():
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=24, H=256, I=128, E=12, k=3, with_dy=True, x_key=31)
    c = host_case(w)
    c.act = 1
    _scale_x(c, 6)
    run_small(c, name="situ-rvq3")


def test_decode_path_few_tokens():
    # MXFP4, bf16 x, T <= 16 with every token row fitting the LDS stage selects the
    # few-token stream kernels; I = 768 is not a multiple of the 4-step unroll
    w = syn.shrink(TINY, T=6, H=512, I=768, E=12, k=3, x_dtype="bf16", x_key=17)
    run_small(host_case(w), name="dec-few")


def test_decode_path_single_token_full_tile():
    w = syn.shrink(TINY, T=1, H=1024, I=256, E=16, k=8, x_dtype="bf16", x_key=18)
    run_small(host_case(w), name="dec-T1")


def test_decode_path_unpacked_planes():
    # 9..16 tokens: the few-token down kernel gives each plane of h its own MFMA
    w = syn.shrink(TINY, T=12, H=512, I=512, E=8, k=2, x_dtype="bf16", x_key=20)
    run_small(host_case(w), name="dec-unpacked")


def test_decode_path_single_token_ten_steps():
    # one token, 16 of 24 experts, ten K-steps per row (not a multiple of the four-step
    # unroll); with dY the backward recomputes g and u on the few-token kernel
    w = syn.shrink(TINY, T=1, H=2560, I=2560, E=24, k=16, x_dtype="bf16", with_dy=True, x_key=40)
    run_small(host_case(w), name="dec-T1-10steps")


@pytest.mark.parametrize("T,k,E,bias_sd", [(2, 16, 40, 1.0), (3, 8, 24, 0.0), (4, 8, 32, 0.5)])
def test_decode_few_tokens_shared_experts(T, k, E, bias_sd):
    # 2..4 tokens sharing experts (each expert holds 1..T of them), I = 4096: the few-token
    # kernels while the h rows fit their LDS stage (T = 2), the generic kernels beyond
    w = syn.shrink(TINY, T=T, H=1024, I=4096, E=E, k=k, x_dtype="bf16", bias_sd=bias_sd, with_dy=True,
                   x_key=41 + T)
    run_small(host_case(w), name=f"dec-T{T}-shared")


def test_rvq3_small():
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=24, H=256, I=128, E=12, k=3, with_dy=True)
    run_small(host_case(w), name="rvq3-small")


def test_rvq3_table_lookup_path():
    # bf16 x, H and I multiples of 256, T <= 64, no adapter: the table-lookup kernels (one row
    # block per matrix, a half table group for H = 512 and a three-quarter one for I = 768)
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=10, H=512, I=768, E=12, k=3, with_dy=True, x_key=21)
    run_small(host_case(w), name="rvq3-lut")


def test_rvq3_codeword_gather_flag():
    # MOE_F_RVQ_GATHER: the layer of test_rvq3_table_lookup_path on the codeword-gather kernels
    from quantized_moe_route_amd import _lib as C
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=10, H=512, I=768, E=12, k=3, with_dy=True, x_key=21)
    run_small(host_case(w), name="rvq3-gather-flag", flags=C.MOE_F_RVQ_GATHER)


def test_rvq3_table_lookup_many_tokens_per_unit():
    # ~13 tokens per expert: one pass per token, the index bytes re-read per pass
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=40, H=256, I=512, E=6, k=2, with_dy=True, x_key=22)
    run_small(host_case(w), name="rvq3-lut-passes")


def test_rvq3_table_lookup_row_blocks():
    # two row blocks per matrix (gate/up: 7 slots x 128 rows = 896, I = 1792; down: 5 slots,
    # 640 rows, H = 1280), groups of 128 + 32 and 128 + 96 vectors
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=6, H=1280, I=1792, E=10, k=4, with_dy=True, x_key=23)
    run_small(host_case(w), name="rvq3-lut-blocks")


def test_rvq3_table_lookup_blocks_take_several_items():
    # 128 active experts x 2 matrices x 2 row blocks = 512 gate/up work items and 256 down
    # items for a launch of one block per CU: blocks draw several items each
    w = syn.shrink(syn.WORKLOADS["rvq16"], T=48, H=1024, I=1024, E=128, k=8, with_dy=True, x_key=24)
    run_small(host_case(w), name="rvq3-lut-persistent")


def test_single_token_and_k1():
    w = syn.shrink(TINY, T=1, k=1, x_key=10)
    run_small(host_case(w), name="T1-k1")


def test_all_tokens_to_one_expert_max_skew():
    w = syn.shrink(TINY, T=64, x_dtype="bf16", x_key=11)
    c = host_case(w)
    c.bias = np.zeros(w.E, np.float32)
    c.bias[5] = 100.0  # every token ranks expert 5 first
    run_small(c, name="skew")


def test_exact_ties_from_duplicate_router_rows():
    w = syn.shrink(TINY, T=32, x_key=12)
    c = host_case(w)
    c.wr[9] = c.wr[2]
    c.wr[12] = c.wr[2]
    c.wr[7] = c.wr[4]
    run_small(c, name="ties")


def test_near_ties_one_ulp_apart():
    """Router rows differing by one fp32 ulp in a single element: the fp32 logits cannot
    separate them, the fp64 re-ranking must."""
    w = syn.shrink(TINY, T=48, E=16, k=4, x_key=13)
    c = host_case(w)
    for a, b in ((1, 5), (3, 11), (0, 14)):
        c.wr[b] = c.wr[a]
        c.wr[b, 17] = np.nextafter(c.wr[a, 17], np.float32(np.inf))
    run_small(c, name="near-ties")


def test_many_token_router_ties_and_near_ties():
    """T > 64 takes the fp64 matrix-core logits: exact duplicate router rows must tie (lower
    id first) and one-ulp near-ties must be ordered by the fp64 re-ranking."""
    w = syn.shrink(TINY, T=150, E=16, k=4, x_key=28)
    c = host_case(w)
    c.wr[9] = c.wr[2]
    c.wr[12] = c.wr[2]
    for a, b in ((1, 5), (3, 11)):
        c.wr[b] = c.wr[a]
        c.wr[b, 17] = np.nextafter(c.wr[a, 17], np.float32(np.inf))
    run_small(c, name="f64-router-ties")


def test_small_batch_fused_routing_ties():
    """T <= 4 routes through the combined top-k + grouping kernel; exact duplicate router
    rows and one-ulp near-ties must resolve there as they do in the separate kernels."""
    w = syn.shrink(TINY, T=4, E=16, k=4, x_key=19)
    c = host_case(w)
    c.wr[9] = c.wr[2]
    c.wr[12] = c.wr[2]
    c.wr[3] = c.wr[6]
    c.wr[11] = c.wr[6]
    c.wr[11, 40] = np.nextafter(c.wr[6, 40], np.float32(np.inf))
    run_small(c, name="fused-ties")


def test_massive_ties_beyond_64_candidates():
    """Logits equal to the bias and tied across each lane's experts (e, e + 64, ...): more
    than 64 experts pass the lane-maximum threshold, so the top-k takes k rounds of
    wave-wide maxima, and the equal values send every token through the fp64 re-ranking.
    T = 4 runs the single-block top-k + grouping, T = 8 the multi-block top-k."""
    for T in (4, 8):
        w = syn.shrink(TINY, T=T, E=896, k=16, x_key=20 + T)
        c = host_case(w)
        c.wr[:] = 0.0
        e = np.arange(w.E)
        c.bias = np.where(e % 64 < 16, 10.0 - 0.001 * (e % 64), 0.0).astype(np.float32)
        run_small(c, name=f"massive-ties-T{T}")


def test_zero_input_and_signed_zero_logits():
    w = syn.shrink(TINY, T=4, x_key=14)
    c = host_case(w)
    c.x[:] = 0.0
    c.x[1, 0] = -0.0
    run_small(c, name="zeros")


def test_T0_is_a_noop():
    import torch
    c = host_case(syn.shrink(TINY, T=1))
    L = device_layer(c, max_tokens=4)
    r = L.new_routing(0)
    x = torch.empty((0, TINY.H), dtype=torch.float32, device="cuda")
    L.route(x, r)
    y = L.forward(x, r)
    assert y.shape == (0, TINY.H)
    dx = L.backward_input(x, x, r)
    assert dx.shape == (0, TINY.H)


def test_selection_experts_closed_form_on_gpu():
    """Selection-matrix experts give y = 2^c silu(2^a x) 2^b x on the selected inputs; checks the
    GPU dequantizer's nibble order and scale handling against the closed form directly."""
    from test_oracle_pins import _selection_closed_form, _selection_mxfp4
    H, I, E, k, T = 256, 128, 6, 3, 16
    shifts, exps = (5, 77, 200), (1, -2, [0, 1, -1, 2, -3, 3])
    codes, scales = _selection_mxfp4(H, I, E, shifts, exps)
    w = syn.shrink(TINY, T=T, H=H, I=I, E=E, k=k, x_key=15)
    c = host_case(w)
    c.codes, c.scales = codes, scales
    L, x, r, y = run_small(c, name="selection")
    ids, p = _np(r.ids), _np(r.w).astype(np.float64)
    errs = []
    for t in range(T):
        want = sum(p[t, j] * _selection_closed_form(c.x64[t], H, I, shifts, exps, exps[2][ids[t, j]])
                   for j in range(k))
        errs.append(rel_err(_np(y)[t], want))
    log(f"  selection experts: max per-token rel err {max(errs):.3e}")
    # fp32 x enters the products exactly (three bf16 terms); what remains is the fp32 sigmoid,
    # h carried as bf16 hi + lo (2^-18) and fp32 accumulation
    assert max(errs) <= 1e-5


def test_repeat_calls_are_bitwise_deterministic():
    w = syn.shrink(TINY, T=40, E=12, k=3, x_dtype="bf16", with_dy=True, x_key=16)
    c = host_case(w)
    L, x, r, y = run_small(c, name="determinism")
    dy = act_tensor(c.dy, "bf16")
    hashes_y, hashes_dx = set(), set()
    for _ in range(5):
        r2 = L.route(x)
        hashes_y.add(fnv1a32(_np(L.forward(x, r2))))
        hashes_dx.add(fnv1a32(_np(L.backward_input(x, dy, r2))))
    assert len(hashes_y) == 1 and len(hashes_dx) == 1
