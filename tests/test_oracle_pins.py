"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: the OCP MX
value table, sizes printed on the pages, library routines (numpy, scipy,
math.fsum), brute force on tiny inputs, closed forms of constructed experts,
and central finite differences for the input gradient.
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import moe_synth as syn
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ---------------------------------------------------------------- formats

def test_e2m1_matches_ocp_table():
    for row in _golden_rows("e2m1_ocp_mx_v1.txt"):
        code, val = row.split()
        got = oracle.e2m1(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e8m0_all_bytes():
    for b in range(255):
        assert oracle.e8m0(b) == 2.0 ** (b - 127)
    assert math.isnan(oracle.e8m0(255))


def test_fp16_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _table():
    return np.array([float(r.split()[1]) for r in _golden_rows("e2m1_ocp_mx_v1.txt")])


def test_mxfp4_nibble_order_and_block_direction():
    """Low nibble = even element, high nibble = odd element; one scale per 32
    consecutive elements along the input dimension (the MX block)."""
    H, I, E = 64, 32, 2
    rng = np.random.default_rng(7)
    codes = [rng.integers(0, 256, (E, r, c // 2), dtype=np.uint8) for r, c in ((I, H), (I, H), (H, I))]
    scales = [rng.integers(100, 140, (E, r, c // 32), dtype=np.uint8) for r, c in ((I, H), (I, H), (H, I))]
    W = oracle.Weights(H, I, codes=codes, scales=scales)
    tab = _table()
    for mat in range(3):
        for e in range(E):
            D = oracle.decode_matrix(W, mat, e)
            rows, cols = D.shape
            for r in (0, rows - 1):
                for i in sorted({0, 1, 30, 31, 32, 33, cols - 1} & set(range(cols))):
                    byte = int(codes[mat][e, r, i // 2])
                    nib = byte & 15 if i % 2 == 0 else byte >> 4
                    assert D[r, i] == tab[nib] * 2.0 ** (int(scales[mat][e, r, i // 32]) - 127)


def test_expert_reads_only_its_own_bytes():
    """Expert e's decode depends on exactly its own span of (cols/2 + cols/32) bytes per row
    (4.25 bits per weight): poisoning every other expert with NaN scales changes nothing."""
    H, I, E = 64, 32, 3
    rng = np.random.default_rng(3)
    shapes = ((I, H), (I, H), (H, I))
    codes = [rng.integers(0, 256, (E, r, c // 2), dtype=np.uint8) for r, c in shapes]
    scales = [rng.integers(119, 124, (E, r, c // 32), dtype=np.uint8) for r, c in shapes]
    clean = oracle.Weights(H, I, codes=codes, scales=scales)
    for e in range(E):
        poisoned_s = [s.copy() for s in scales]
        poisoned_c = [c.copy() for c in codes]
        for m in range(3):
            for o in range(E):
                if o != e:
                    poisoned_s[m][o] = 255
                    poisoned_c[m][o] = 0x77
        Wp = oracle.Weights(H, I, codes=poisoned_c, scales=poisoned_s)
        for m in range(3):
            assert np.array_equal(oracle.decode_matrix(Wp, m, e), oracle.decode_matrix(clean, m, e))


def _mxfp4_bytes_per_expert(H, I):
    w = syn.shrink(syn.WORKLOADS["decode1"], H=H, I=I)
    return sum(sum(a.nbytes for a in syn.mxfp4_expert(w, m, 0)) for m in range(3))


def _rvq3_bytes_per_expert(H, I):
    w = syn.shrink(syn.WORKLOADS["rvq16"], H=H, I=I)
    return sum(sum(a.nbytes for a in syn.rvq3_expert(w, m, 0)) for m in range(3))


def test_printed_sizes_pin_the_formats():
    """The storage formats reproduce the sizes the pages print (K3 shape: H 3584, I 3072,
    896 experts per MoE layer, 92 MoE layers, top-16)."""
    H, I, E, L, k = 3584, 3072, 896, 92, 16
    mx = _mxfp4_bytes_per_expert(H, I)
    rvq = _rvq3_bytes_per_expert(H, I)
    assert mx == 17_547_264 and rvq == 12_423_168
    derived = {
        "mxfp4_bytes_per_expert": mx / 1e6,
        "mxfp4_bytes_per_expert_short": mx / 1e6,
        "mxfp4_bytes_per_layer": E * mx / 1e9,
        "routed_experts_total": L * E,
        "latent_vector_fp32": H * 4 / 1e3,
        "expert_share_of_checkpoint": L * E * mx / 2**30 / 1453.74,
        "rvq3_expert_bytes_per_token": L * k * rvq / 2**30,
        "lora_params_per_expert": 2 * (H * 16 + 16 * I) + (I * 16 + 16 * H),
    }
    for row in _golden_rows("page_sizes.txt"):
        name, printed, unit, tol, _src = [p.strip() for p in row.split("|")]
        got, want = derived[name], float(printed)
        assert abs(got - want) <= float(tol) * want, (name, got, want)


# ---------------------------------------------------------------- router

def _tiny_router(seed=0, T=8, H=256, E=16):
    rng = np.random.default_rng(seed)
    x = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    return x.astype(np.float64), wr


def test_e4m3_table_against_ocp_mx_landmarks():
    for row in _golden_rows("e4m3_ocp_mx_v1.txt"):
        code, val = int(row.split()[0], 16), row.split()[1]
        got = oracle.e4m3(code)
        if val == "nan":
            assert math.isnan(got), hex(code)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (hex(code), got)


def _e4m3_finite():
    vals = [oracle.e4m3(c) for c in range(256)]
    return np.array(sorted({v for v in vals if not math.isnan(v) and v >= 0}))


def test_mxfp8_quantizer_grid_ties_and_saturation():
    """With a block whose largest magnitude lies in [256, 512) the shared exponent is 0, so
    the quantizer rounds elements straight onto the E4M3 grid: every finite E4M3 value is a
    fixed point, midpoints go to the even mantissa, other points to the nearest value, and
    magnitudes past 448 saturate to 448 (the MX conversion's clamp)."""
    grid = _e4m3_finite()
    assert grid.size == 127 and grid[-1] == 448.0
    mids = (grid[:-1] + grid[1:]) / 2
    inner = grid[:-1] + (grid[1:] - grid[:-1]) * 0.3
    for vals in (grid, mids, inner, -grid, -mids):
        n = (len(vals) + 30) // 31 * 31
        v = np.resize(vals, n).reshape(-1, 31)
        blocks = np.concatenate([np.full((v.shape[0], 1), 300.0), v], axis=1)  # amax in [256, 512)
        xq, ex = oracle.quantize_mxfp8(blocks)
        assert np.all(ex == 0)
        got, src = xq[:, 1:].ravel()[: len(vals)], v.ravel()[: len(vals)]
        a = np.abs(src)
        # reference: nearest grid value, ties to the even code (the even mantissa)
        idx = np.searchsorted(grid, a)
        lo, hi = grid[np.maximum(idx - 1, 0)], grid[np.minimum(idx, grid.size - 1)]
        want = np.where(a - lo < hi - a, lo, hi)
        tie = (a - lo) == (hi - a)
        codes = {oracle.e4m3(c): c for c in range(128) if not math.isnan(oracle.e4m3(c))}
        even_lo = np.array([codes[x] % 2 == 0 for x in lo])
        want = np.where(tie, np.where(even_lo, lo, hi), want)
        want = np.where(np.isin(a, grid), a, want)
        assert np.array_equal(np.abs(got), want), np.argwhere(np.abs(got) != want)[:5]
        assert np.array_equal(np.signbit(got), np.signbit(src))  # the sign is kept, also for -0
    # saturation, the shared exponent of powers of two, an all-zero block
    xq, ex = oracle.quantize_mxfp8(np.array([[460.0, 500.0, -511.0] + [1.0] * 29]))
    assert ex[0, 0] == 0 and list(xq[0, :3]) == [448.0, 448.0, -448.0]
    for k in (-20, -3, 0, 5, 40):
        xq, ex = oracle.quantize_mxfp8(np.array([[2.0 ** k] + [0.0] * 31]))
        assert ex[0, 0] == k - 8 and xq[0, 0] == 2.0 ** k
    xq, ex = oracle.quantize_mxfp8(np.zeros((1, 32)))
    assert ex[0, 0] == -127 and not xq.any()


def test_mxfp8_quantizer_against_torch_float8():
    """Inside the E4M3 range PyTorch's float8_e4m3fn cast rounds to nearest even, the same
    decision the quantizer takes: compare on random blocks scaled by their shared exponent."""
    import torch
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 32)) * np.exp2(rng.integers(-10, 10, (64, 1)))).astype(np.float32).astype(np.float64)
    xq, ex = oracle.quantize_mxfp8(x)
    scaled = x / np.exp2(ex)
    assert np.abs(scaled).max() < 512
    inside = np.minimum(np.abs(scaled), 448.0) * np.sign(scaled)
    ref = torch.tensor(inside, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy() * np.exp2(ex)
    assert np.array_equal(xq, ref)


def test_selection_only_bias():
    """bias_mode 2: the bias picks the experts, the unbiased logits weight them.  A large
    bias on each token's lowest-logit expert forces it into the top 2; its weight is then
    the sigmoid of the UNBIASED logit gap (k = 2 closed form), and the selection equals the
    one of bias_mode 1; a zero bias gives mode 1's weights bit for bit."""
    x, wr = _tiny_router(5)
    T, E = x.shape[0], wr.shape[0]
    raw = oracle.router_logits(x, wr)
    low = np.argmin(raw, axis=1)
    for t in range(T):
        bias = np.zeros(E, np.float32)
        bias[low[t]] = 100.0
        ids2, p2, keys = oracle.route(x[t:t + 1], wr, bias, 2, bias_mode=2)
        ids1, p1, _ = oracle.route(x[t:t + 1], wr, bias, 2, bias_mode=1)
        assert np.array_equal(ids1, ids2) and ids2[0, 0] == low[t]
        l1, l2 = raw[t, ids2[0, 0]], raw[t, ids2[0, 1]]
        assert abs(p2[0, 0] - 1.0 / (1.0 + math.exp(l2 - l1))) <= 1e-15
        assert abs(p2.sum() - 1.0) <= 1e-15
        assert p2[0, 0] < 0.5 < p1[0, 0]  # forced in by the bias, yet the smaller weight
    z = np.zeros(E, np.float32)
    a = oracle.route(x, wr, z, 4, bias_mode=2)
    b = oracle.route(x, wr, z, 4, bias_mode=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_router_logits_against_numpy_and_fsum():
    x, wr = _tiny_router(1)
    b = np.linspace(-1, 1, wr.shape[0]).astype(np.float32)
    got = oracle.router_logits(x, wr, b)
    ref = x @ wr.astype(np.float64).T + b.astype(np.float64)
    scale = np.abs(x) @ np.abs(wr.astype(np.float64)).T + np.abs(b)
    assert np.all(np.abs(got - ref) <= 1e-13 * scale)
    for t in range(x.shape[0]):
        for e in range(wr.shape[0]):
            exact = math.fsum(list(x[t] * wr[e].astype(np.float64)) + [float(b[e])])
            assert abs(got[t, e] - exact) <= x.shape[1] * 2.0**-52 * scale[t, e]


def _brute_topk(l, k):
    E = l.shape[0]
    rank = np.array([sum(1 for f in range(E) if l[f] > l[e] or (l[f] == l[e] and f < e)) for e in range(E)])
    order = np.argsort(rank)
    return order[:k]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    T, E = 5, 12
    # a coarse grid forces many exact ties; signed zeros included
    logits = rng.integers(-3, 4, (T, E)).astype(np.float64) * 0.5
    logits[0, 3] = -0.0
    logits[0, 5] = 0.0
    for k in (1, 2, 5, E):
        ids, _ = oracle.topk_softmax(logits, k)
        for t in range(T):
            assert list(ids[t]) == list(_brute_topk(logits[t], k)), (t, k)


def test_topk_duplicate_router_rows_tie_to_lower_id():
    x, wr = _tiny_router(2, T=6, E=16)
    wr[9] = wr[2]
    wr[12] = wr[2]
    wr[7] = wr[4]
    logits = oracle.router_logits(x, wr, None)
    assert np.array_equal(logits[:, 9], logits[:, 2]) and np.array_equal(logits[:, 12], logits[:, 2])
    ids, _ = oracle.topk_softmax(logits, 16)
    for t in range(6):
        pos = {e: j for j, e in enumerate(ids[t])}
        assert pos[2] < pos[9] < pos[12] and pos[4] < pos[7]


def test_topk_one_ulp_apart():
    x, wr = _tiny_router(4, T=4, E=8)
    wr[5] = wr[1]
    i = int(np.argmax(np.abs(x[0])))
    wr[5, i] = np.nextafter(wr[1, i], np.float32(np.inf if x[0, i] > 0 else -np.inf))
    logits = oracle.router_logits(x, wr, None)
    assert logits[0, 5] > logits[0, 1]
    ids, _ = oracle.topk_softmax(logits, 8)
    pos = {e: j for j, e in enumerate(ids[0])}
    assert pos[5] < pos[1]


def test_softmax_closed_forms():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((20, 10)) * 3
    for k in (1, 2, 4, 10):
        ids, w = oracle.topk_softmax(logits, k)
        assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-15 * k)
        assert np.all(np.diff(w, axis=1) <= 0)
        if k == 1:
            assert np.all(w == 1.0)
        if k == 2:
            l0 = np.take_along_axis(logits, ids[:, :1], 1)[:, 0]
            l1 = np.take_along_axis(logits, ids[:, 1:2], 1)[:, 0]
            assert np.allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-15, atol=0)
        if k == 10:
            dense = scipy.special.softmax(logits, axis=1)
            assert np.allclose(w, np.take_along_axis(dense, ids, 1), rtol=1e-14, atol=0)


# ---------------------------------------------------------------- grouping

@pytest.mark.parametrize("T,E,k", [(1, 896, 16), (37, 16, 2), (64, 40, 7), (0, 8, 2), (9, 4, 4)])
def test_group_invariants_and_unpermute(T, E, k):
    rng = np.random.default_rng(T * 131 + E)
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    g = oracle.group(ids, E)
    S = T * k
    assert g["counts"].sum() == S
    assert np.array_equal(g["counts"], np.bincount(ids.ravel(), minlength=E))
    assert g["offsets"][0] == 0 and np.all(np.diff(g["offsets"]) == g["counts"])
    perm, inv = g["perm"], g["inv"]
    assert np.array_equal(np.sort(perm), np.arange(S))
    assert np.array_equal(inv[perm], np.arange(S)) and np.array_equal(perm[inv], np.arange(S))
    key = [(int(ids.ravel()[s]), s // k if k else 0) for s in perm]
    assert all(key[i] < key[i + 1] for i in range(len(key) - 1))
    act = g["active"][: g["n_active"]]
    assert np.array_equal(act, np.nonzero(g["counts"])[0])
    # unpermute(permute(X)) == X bitwise on the replicated [T][k][H] tensor
    X = rng.standard_normal((T, 1, 5)).repeat(k, 1).reshape(S, 5)
    grouped = X[perm]
    back = grouped[inv]
    assert np.array_equal(back, X)


# ---------------------------------------------------------------- experts

def _selection_mxfp4(H, I, E, shifts, exps):
    """Experts whose matrices are scaled permutation-like selections:
    gate[n][(n+sg)%H] = 2^a, up[n][(n+su)%H] = 2^b, down[(n+sd)%H][n] = 2^c_e.
    Code 2 encodes 1.0 in E2M1; the scale byte 127+s encodes 2^s."""
    sg, su, sd = shifts
    shapes = ((I, H), (I, H), (H, I))
    codes = [np.zeros((E, r, c // 2), np.uint8) for r, c in shapes]
    scales = [np.full((E, r, c // 32), 127, np.uint8) for r, c in shapes]
    a, b, cs = exps
    for e in range(E):
        for n in range(I):
            for mat, (row, col, ex) in enumerate(((n, (n + sg) % H, a), (n, (n + su) % H, b),
                                                  ((n + sd) % H, n, cs[e]))):
                codes[mat][e, row, col // 2] |= np.uint8(2 << (4 * (col % 2)))
                scales[mat][e, row, col // 32] = 127 + ex
    return codes, scales


def _selection_closed_form(x, H, I, shifts, exps, ce):
    sg, su, sd = shifts
    a, b, _ = exps
    o = np.zeros(H)
    for n in range(I):
        gv = 2.0**a * x[(n + sg) % H]
        uv = 2.0**b * x[(n + su) % H]
        o[(n + sd) % H] += 2.0**ce * gv / (1.0 + math.exp(-gv)) * uv
    return o


def test_selection_experts_closed_form_and_combine():
    H, I, E, k, T = 256, 128, 6, 3, 4
    shifts, exps = (5, 77, 200), (1, -2, [0, 1, -1, 2, -3, 3])
    codes, scales = _selection_mxfp4(H, I, E, shifts, exps)
    W = oracle.Weights(H, I, codes=codes, scales=scales)
    x, wr = _tiny_router(9, T=T, H=H, E=E)
    y, ids, w = oracle.layer_forward(x, wr, None, k, W)
    for t in range(T):
        want = sum(w[t, j] * _selection_closed_form(x[t], H, I, shifts, exps, exps[2][ids[t, j]])
                   for j in range(k))
        assert np.allclose(y[t], want, rtol=1e-14, atol=1e-300)


def _selection_rvq3(H, I, E, shifts):
    """RVQ3 experts decoding to 0/1 selections; the 1.0 is split over the stages as
    0.5 + 0.25 + 0.25 so all three codebooks and index planes take part.  Codebook
    entry 1+d of every stage is c_s * unit_vector(d); entry 0 is zero."""
    sg, su, sd = shifts
    shapes = ((I, H), (I, H), (H, I))
    idx = [np.zeros((E, 3, r, c // 8), np.uint8) for r, c in shapes]
    cb = [np.zeros((E, 3, 256, 8), np.float16) for _ in shapes]
    for mat in range(3):
        for st, cst in enumerate((0.5, 0.25, 0.25)):
            for d in range(8):
                cb[mat][:, st, 1 + d, d] = cst
    for n in range(I):
        for mat, (row, col) in enumerate(((n, (n + sg) % H), (n, (n + su) % H), ((n + sd) % H, n))):
            idx[mat][:, :, row, col // 8] = 1 + col % 8
    return idx, [c.view(np.uint16) for c in cb]


def test_rvq3_selection_experts_closed_form():
    H, I, E, k, T = 256, 128, 4, 2, 3
    shifts = (3, 100, 17)
    idx, cb = _selection_rvq3(H, I, E, shifts)
    W = oracle.Weights(H, I, idx=idx, cb=cb)
    x, wr = _tiny_router(11, T=T, H=H, E=E)
    y, ids, w = oracle.layer_forward(x, wr, None, k, W)
    for t in range(T):
        want = _selection_closed_form(x[t], H, I, shifts, (0, 0, None), 0)
        assert np.allclose(y[t], want, rtol=1e-14, atol=1e-300)


def test_rvq3_residual_sum_of_random_codebooks():
    """Decoded vector = sum of the three indexed stage codewords (fp16 widened exactly)."""
    w = syn.shrink(syn.WORKLOADS["rvq16"], H=64, I=32, E=2)
    idx, cb = syn.rvq3_layer(w)
    W = oracle.Weights(64, 32, idx=idx, cb=cb)
    cbf = [c.view(np.float16).astype(np.float64) for c in cb]
    for mat in range(3):
        D = oracle.decode_matrix(W, mat, 1)
        rows, cols = D.shape
        for r in (0, rows // 2, rows - 1):
            for v in (0, cols // 8 - 1):
                want = sum(cbf[mat][1, s, idx[mat][1, s, r, v]] for s in range(3))
                assert np.array_equal(D[r, 8 * v: 8 * v + 8], want)


def _tiny_layer(E=16, identical=False, seed_family=syn.FAMILY_TINY, act=oracle.ACT_SWIGLU, lora=None):
    w = syn.WORKLOADS["tiny"]
    w = syn.shrink(w, E=E)
    if identical:
        one_c, one_s = syn.mxfp4_layer(w, experts=[0])
        codes = [np.repeat(c, E, 0) for c in one_c]
        scales = [np.repeat(s, E, 0) for s in one_s]
    else:
        codes, scales = syn.mxfp4_layer(w)
    return w, oracle.Weights(w.H, w.I, codes=codes, scales=scales, act=act, lora=lora)


def _tiny_lora(w, r=16, scale=2.0):
    A, B = syn.lora_adapter(w, r)
    return (A, B, scale)


def _act_probe(act):
    """h = act(g, u) of the oracle's expert at chosen (g, u): a one-expert selection layer
    with g_n = x_n and u_n = x_{n+128} (shifts 0 and 128, unit scales), read back as h."""
    H, I = 256, 128
    codes, scales = _selection_mxfp4(H, I, 1, (0, 128, 0), (0, 0, [0]))
    W = oracle.Weights(H, I, codes=codes, scales=scales, act=act)

    def h_of(pairs):
        x = np.zeros(H)
        for n, (gv, uv) in enumerate(pairs):
            x[n], x[n + 128] = gv, uv
        g, u, h, _ = oracle.expert_forward(W, 0, x)
        assert np.array_equal(g[: len(pairs)], [p[0] for p in pairs])  # the probe reaches g, u exactly
        assert np.array_equal(u[: len(pairs)], [p[1] for p in pairs])
        return h[: len(pairs)]
    return h_of


def test_situ_activation_limits():
    """SiTU (LazyLoRA README, "File map"): h = A(g) B(u), A(g) = 4 tanh(g/4) sigmoid(g),
    B(u) = 25 tanh(u/25).  Pinned by limits the definition fixes, not by its formula: zeros;
    saturation at A = 4 and B = 25 (the outer factors); slopes A(g)/g -> 1/2 and B(u)/u -> 1
    at 0 (with the saturations they fix the inner scales 1/4 and 1/25); A(g) / (-4 e^g) -> 1
    as g -> -inf (the sigmoid factor); B odd."""
    h = _act_probe(oracle.ACT_SITU)
    v = h([(0.0, 3.0), (2.0, 0.0), (400.0, 4000.0), (1e-6, 4000.0), (400.0, 1e-6), (-40.0, 4000.0),
           (1.5, 2.5), (1.5, -2.5)])
    assert v[0] == 0.0 and v[1] == 0.0
    assert v[2] == 100.0
    assert abs(v[3] / (25 * 1e-6) - 0.5) < 1e-6
    assert abs(v[4] / (4 * 1e-6) - 1.0) < 1e-9
    assert abs(v[5] / (25 * -4 * math.exp(-40.0)) - 1.0) < 1e-8
    assert v[6] == -v[7] and v[6] > 0
    # SwiGLU through the same probe: g sigmoid(g) u at a point, and its slope 1/2 at g = 0
    s = _act_probe(oracle.ACT_SWIGLU)([(1e-6, 1.0), (400.0, 2.0)])
    assert abs(s[0] / 1e-6 - 0.5) < 1e-6 and s[1] == 800.0


def test_k1_single_expert_is_textbook_swiglu_mlp():
    w, W = _tiny_layer(E=16)
    x = oracle.to_f64(syn.activations(w), "f32")
    Wg, Wu, Wd = (oracle.decode_matrix(W, m, 5) for m in range(3))
    ids = np.full((w.T, 1), 5, np.int32)
    y = oracle.forward(x, ids, np.ones((w.T, 1)), W)
    g, u = x @ Wg.T, x @ Wu.T
    ref = (scipy.special.expit(g) * g * u) @ Wd.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max())


def test_identical_experts_make_routing_irrelevant_and_router_grad_zero():
    w, W = _tiny_layer(E=16, identical=True)
    x = oracle.to_f64(syn.activations(w), "f32")
    wr = syn.router_weight(w)
    dy = oracle.to_f64(syn.upstream_grad(w), "f32")
    y, ids, p = oracle.layer_forward(x, wr, None, w.k, W)
    one = np.zeros((w.T, 1), np.int32)
    y1 = oracle.forward(x, one, np.ones((w.T, 1)), W)
    assert np.allclose(y, y1, rtol=1e-13, atol=1e-15 * np.abs(y1).max())
    dx = oracle.backward_input(x, dy, ids, p, wr, W)
    dx1 = oracle.backward_input(x, dy, one, np.ones((w.T, 1)), wr, W)
    assert np.allclose(dx, dx1, rtol=1e-12, atol=1e-13 * np.abs(dx1).max())


def test_backward_is_linear_in_dy():
    w, W = _tiny_layer()
    x = oracle.to_f64(syn.activations(w), "f32")
    wr = syn.router_weight(w)
    ids, p, _ = oracle.route(x, wr, None, w.k)
    rng = np.random.default_rng(12)
    d1, d2 = rng.standard_normal((2, w.T, w.H))
    a = oracle.backward_input(x, 2 * d1 + 3 * d2, ids, p, wr, W)
    b = 2 * oracle.backward_input(x, d1, ids, p, wr, W) + 3 * oracle.backward_input(x, d2, ids, p, wr, W)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14 * np.abs(b).max())


def _loss(x, dy, wr, bias, k, W, bias_mode=1):
    y, ids, _ = oracle.layer_forward(x, wr, bias, k, W, nthreads=1, bias_mode=bias_mode)
    return float(np.sum(dy * y)), ids


@pytest.mark.parametrize("with_bias,act,lora,bias_mode", [(False, 0, False, 1), (True, 0, False, 1), (False, 1, False, 1),
                                                          (False, 0, True, 1), (True, 1, True, 1), (True, 0, False, 2),
                                                          (True, 1, True, 2)])
def test_backward_matches_central_finite_differences(with_bias, act, lora, bias_mode):
    """Directional derivatives of L(x) = sum_t <dY_t, y_t(x)> by central differences in fp64,
    with a step relative to the tensor norm and routing-flip detection (a direction whose
    perturbation changes any token's expert set is retried with half the step); SwiGLU and
    SiTU experts, with and without the shared adapter, with the router bias in the logits or
    in the selection only."""
    w0 = syn.WORKLOADS["tiny"]
    w, W = _tiny_layer(act=act, lora=_tiny_lora(w0) if lora else None)
    x = oracle.to_f64(syn.activations(w), "f32")
    wr = syn.router_weight(w)
    bias = np.linspace(-0.3, 0.3, w.E).astype(np.float32) if with_bias else None
    dy = oracle.to_f64(syn.upstream_grad(w), "f32") * 100.0
    ids, p, _ = oracle.route(x, wr, bias, w.k, bias_mode=bias_mode)
    dx = oracle.backward_input(x, dy, ids, p, wr, W)
    rng = np.random.default_rng(99)
    dirs = [rng.standard_normal(x.shape) for _ in range(6)]
    for t, i in ((0, 0), (3, 17), (7, 255)):
        v = np.zeros_like(x)
        v[t, i] = 1.0
        dirs.append(v)
    checked = 0
    for v in dirs:
        eps = 1e-6 * np.linalg.norm(x) / np.linalg.norm(v)
        for _ in range(8):
            lp, ip = _loss(x + eps * v, dy, wr, bias, w.k, W, bias_mode)
            lm, im = _loss(x - eps * v, dy, wr, bias, w.k, W, bias_mode)
            if np.array_equal(ip, ids) and np.array_equal(im, ids):
                break
            eps /= 2
        else:
            continue
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(dx * v))
        assert abs(fd - an) <= 1e-7 * max(abs(an), 1e-3 * np.linalg.norm(dx) * np.linalg.norm(v)), (fd, an)
        checked += 1
    assert checked >= 7


def test_backward_router_term_by_finite_differences_on_router_logits():
    """With the experts fixed, only the router term depends on Wr; perturbing x along a
    direction orthogonal to every gate/up row isolates it (selection experts read only
    the first I inputs, so directions on the remaining inputs see only the router)."""
    H, I, E, k, T = 256, 128, 6, 3, 2
    shifts, exps = (0, 0, 0), (0, 0, [0, 1, -1, 2, 0, 1])
    codes, scales = _selection_mxfp4(H, I, E, shifts, exps)
    W = oracle.Weights(H, I, codes=codes, scales=scales)
    x, wr = _tiny_router(21, T=T, H=H, E=E)
    dy = np.random.default_rng(8).standard_normal((T, H))
    ids, p, _ = oracle.route(x, wr, None, k)
    dx = oracle.backward_input(x, dy, ids, p, wr, W)
    for t in range(T):
        v = np.zeros_like(x)
        v[t, I:] = np.random.default_rng(t).standard_normal(H - I)
        eps = 1e-6 * np.linalg.norm(x) / np.linalg.norm(v)
        lp, ip = _loss(x + eps * v, dy, wr, None, k, W)
        lm, im = _loss(x - eps * v, dy, wr, None, k, W)
        assert np.array_equal(ip, ids) and np.array_equal(im, ids)
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(dx * v))
        assert abs(an) > 1e-6 and abs(fd - an) <= 1e-7 * abs(an)


# ---------------------------------------------------------------- shared low-rank adapter


def _merged_forward(x, ids, p, W, lora, act):
    """y from dense merged matrices W_e + scale B A (the identity a LoRA adapter merges by),
    one numpy matmul chain per slot -- a different association from the oracle's
    W z + scale B (A z)."""
    A, B, sc = lora
    T, k = ids.shape
    y = np.zeros((T, W.H))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            Wg, Wu, Wd = (oracle.decode_matrix(W, m, e) + sc * (B[m].astype(np.float64) @ A[m].astype(np.float64))
                          for m in range(3))
            g, u = Wg @ x[t], Wu @ x[t]
            if act == oracle.ACT_SITU:
                h = 4 * np.tanh(g / 4) * scipy.special.expit(g) * 25 * np.tanh(u / 25)
            else:
                h = g * scipy.special.expit(g) * u
            y[t] += p[t, j] * (Wd @ h)
    return y


@pytest.mark.parametrize("act", [oracle.ACT_SWIGLU, oracle.ACT_SITU])
def test_lora_forward_equals_merged_weights(act):
    w0 = syn.WORKLOADS["tiny"]
    lora = _tiny_lora(w0)
    w, W = _tiny_layer(act=act, lora=lora)
    x = oracle.to_f64(syn.activations(w), "f32")
    wr = syn.router_weight(w)
    ids, p, _ = oracle.route(x, wr, None, w.k)
    y = oracle.forward(x, ids, p, W)
    ref = _merged_forward(x, ids, p, W, lora, act)
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())
    # the adapter moves the output by much more than the tolerance
    _, W0 = _tiny_layer(act=act)
    assert np.abs(oracle.forward(x, ids, p, W0) - y).max() > 1e-2 * np.abs(y).max()


def test_lora_with_zero_B_is_the_plain_layer():
    w0 = syn.WORKLOADS["tiny"]
    A, B, sc = _tiny_lora(w0)
    w, W = _tiny_layer(lora=(A, [np.zeros_like(b) for b in B], sc))
    _, W0 = _tiny_layer()
    x = oracle.to_f64(syn.activations(w), "f32")
    dy = oracle.to_f64(syn.upstream_grad(w), "f32")
    wr = syn.router_weight(w)
    ids, p, _ = oracle.route(x, wr, None, w.k)
    assert np.array_equal(oracle.forward(x, ids, p, W), oracle.forward(x, ids, p, W0))
    assert np.array_equal(oracle.backward_input(x, dy, ids, p, wr, W), oracle.backward_input(x, dy, ids, p, wr, W0))
    # with B = 0 only dB can be nonzero; dA vanishes identically
    dA, dB = oracle.lora_grads(x, dy, ids, p, W)
    assert all(np.all(a == 0) for a in dA) and all(np.abs(b).max() > 0 for b in dB)


@pytest.mark.parametrize("act", [oracle.ACT_SWIGLU, oracle.ACT_SITU])
def test_lora_grads_match_central_finite_differences(act):
    """Directional derivatives of L = sum_t <dY_t, y_t> with respect to each of the six adapter
    matrices, routing held fixed (it does not depend on the adapter), by central differences
    in fp64 on the forward; random directions and single entries."""
    w0 = syn.shrink(syn.WORKLOADS["tiny"], T=12)
    A, B, sc = _tiny_lora(w0, r=4)
    A = [a.astype(np.float64) for a in A]
    B = [b.astype(np.float64) for b in B]
    w, W = _tiny_layer(act=act, lora=(A, B, sc))
    w = syn.shrink(w, T=12)
    x = oracle.to_f64(syn.activations(w), "f32")
    dy = oracle.to_f64(syn.upstream_grad(w), "f32") * 100.0
    wr = syn.router_weight(w)
    ids, p, _ = oracle.route(x, wr, None, w.k)
    dA, dB = oracle.lora_grads(x, dy, ids, p, W)
    codes, scales = syn.mxfp4_layer(w)

    def loss(A_, B_):
        Wl = oracle.Weights(w.H, w.I, codes=codes, scales=scales, act=act, lora=(A_, B_, sc))
        return float(np.sum(dy * oracle.forward(x, ids, p, Wl, nthreads=1)))

    rng = np.random.default_rng(5)
    for which in ("A", "B"):
        for m in range(3):
            P = A if which == "A" else B
            G = (dA if which == "A" else dB)[m]
            dirs = [rng.standard_normal(P[m].shape) for _ in range(2)]
            v = np.zeros(P[m].shape)
            v[-1, 1] = 1.0
            dirs.append(v)
            for v in dirs:
                eps = 1e-5 * np.linalg.norm(P[m]) / np.linalg.norm(v)
                Pp = [q.copy() for q in P]
                Pm = [q.copy() for q in P]
                Pp[m] = P[m] + eps * v
                Pm[m] = P[m] - eps * v
                lp = loss(Pp, B) if which == "A" else loss(A, Pp)
                lm = loss(Pm, B) if which == "A" else loss(A, Pm)
                fd = (lp - lm) / (2 * eps)
                an = float(np.sum(G * v))
                assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3 * np.linalg.norm(G) * np.linalg.norm(v)), \
                    (which, m, fd, an)


# ---------------------------------------------------------------- shared experts


def _tiny_shared(w, act=oracle.ACT_SWIGLU, n=2):
    sc, ss = syn.shared_experts(w, n)
    return oracle.Weights(w.H, w.I, codes=sc, scales=ss, act=act)


@pytest.mark.parametrize("act", [oracle.ACT_SWIGLU, oracle.ACT_SITU])
def test_shared_experts_are_dense_mlps_added_with_weight_one(act):
    """The shared-expert term equals the textbook gated MLPs on the decoded matrices (numpy
    products), summed over the shared experts with weight 1; one shared expert alone equals
    the routed layer run on that expert with k = 1."""
    w, _ = _tiny_layer(E=16)
    Ws = _tiny_shared(w, act)
    x = oracle.to_f64(syn.activations(w), "f32")
    ref = np.zeros((w.T, w.H))
    for s in range(2):
        Wg, Wu, Wd = (oracle.decode_matrix(Ws, m, s) for m in range(3))
        g, u = x @ Wg.T, x @ Wu.T
        if act == oracle.ACT_SWIGLU:
            h = scipy.special.expit(g) * g * u
        else:
            h = 4 * np.tanh(g / 4) * scipy.special.expit(g) * 25 * np.tanh(u / 25)
        ref += h @ Wd.T
    got = oracle.shared_forward(x, Ws, 2)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max())
    one = oracle.shared_forward(x, Ws, 1)
    k1 = oracle.forward(x, np.zeros((w.T, 1), np.int32), np.ones((w.T, 1)), Ws)
    assert np.array_equal(one, k1)


def test_shared_backward_matches_central_finite_differences():
    """dX of the layer with two shared experts (routed term with its router part, plus the
    shared experts' input gradient) against central differences of L(x) = sum <dY, y(x)>,
    with routing-flip detection as in the routed-layer pin."""
    w, W = _tiny_layer()
    Ws = _tiny_shared(w)
    x = oracle.to_f64(syn.activations(w), "f32")
    wr = syn.router_weight(w)
    dy = oracle.to_f64(syn.upstream_grad(w), "f32") * 100.0
    ids, p, _ = oracle.route(x, wr, None, w.k)
    dx = oracle.backward_input(x, dy, ids, p, wr, W) + oracle.shared_backward_input(x, dy, Ws, 2)

    def loss(xx):
        y, ii, _ = oracle.layer_forward(xx, wr, None, w.k, W, nthreads=1)
        return float(np.sum(dy * (y + oracle.shared_forward(xx, Ws, 2, nthreads=1)))), ii

    rng = np.random.default_rng(7)
    checked = 0
    for v in [rng.standard_normal(x.shape) for _ in range(6)]:
        eps = 1e-6 * np.linalg.norm(x) / np.linalg.norm(v)
        for _ in range(8):
            lp, ip = loss(x + eps * v)
            lm, im = loss(x - eps * v)
            if np.array_equal(ip, ids) and np.array_equal(im, ids):
                break
            eps /= 2
        else:
            continue
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(dx * v))
        assert abs(fd - an) <= 1e-7 * max(abs(an), 1e-3 * np.linalg.norm(dx) * np.linalg.norm(v)), (fd, an)
        checked += 1
    assert checked >= 5
    # the shared part alone is linear in dY and has no router term: zero dY, zero gradient
    assert not np.any(oracle.shared_backward_input(x, np.zeros_like(dy), Ws, 2))


# ---------------------------------------------------------------- latent projections


def _bf16_f64(bits):
    return oracle.to_f64(bits, "bf16")


def test_dense_projection_against_numpy_both_orientations():
    """oracle.dense against numpy float64 products of the decoded bf16 matrix, in both
    orientations, with a non-square matrix so that a transposed operand cannot pass."""
    rng = np.random.default_rng(31)
    w = syn.f32_to_bf16_bits(rng.standard_normal((96, 160), dtype=np.float32))  # [N][K]
    a = rng.standard_normal((5, 160))
    wf = _bf16_f64(w)
    assert np.abs(oracle.dense(a, w) - a @ wf.T).max() <= 1e-12 * np.abs(a @ wf.T).max()
    b = rng.standard_normal((5, 96))
    got = oracle.dense(b, w, transposed=True)
    assert got.shape == (5, 160)
    assert np.abs(got - b @ wf).max() <= 1e-12 * np.abs(b @ wf).max()


def test_dense_projection_identity_and_permutation():
    """Closed forms: the identity matrix returns the input exactly; a permutation matrix
    permutes it, forward (w^T applied) and transposed (w applied, the inverse permutation)."""
    n = 64
    perm = np.random.default_rng(5).permutation(n)
    eye = syn.f32_to_bf16_bits(np.eye(n, dtype=np.float32))
    P = np.zeros((n, n), np.float32)
    P[np.arange(n), perm] = 1.0  # row i picks input perm[i]
    Pb = syn.f32_to_bf16_bits(P)
    a = np.random.default_rng(6).standard_normal((3, n))
    assert np.array_equal(oracle.dense(a, eye), a)
    assert np.array_equal(oracle.dense(a, Pb), a[:, perm])
    back = np.empty_like(a)
    back[:, perm] = a
    assert np.array_equal(oracle.dense(a, Pb, transposed=True), back)


def test_latent_chain_gradient_by_finite_differences():
    """The layer inside its latent projections: out = proj_out(moe(proj_in(x_model))).  dX_model
    composed as proj_in-backward(backward_input(proj_out-backward(dout))) matches central
    differences of L(x_model) = sum <dout, out(x_model)>, with routing-flip detection."""
    w0 = syn.WORKLOADS["tiny"]
    w, W = _tiny_layer()
    D = 192
    pin, pout = syn.latent_projections(w, D)
    xm = oracle.to_f64(syn.model_activations(w, D), "f32")
    wr = syn.router_weight(w)
    dout = oracle.to_f64(syn.model_upstream_grad(w, D), "f32") * 100.0

    def out_of(xx):
        xl = oracle.dense(xx, pin)
        y, ii, _ = oracle.layer_forward(xl, wr, None, w.k, W, nthreads=1)
        return oracle.dense(y, pout), ii, xl

    _, ids, xl = out_of(xm)
    ids_, p, _ = oracle.route(xl, wr, None, w.k)
    assert np.array_equal(ids, ids_)
    dyl = oracle.dense(dout, pout, transposed=True)
    dxl = oracle.backward_input(xl, dyl, ids, p, wr, W)
    dxm = oracle.dense(dxl, pin, transposed=True)
    assert dxm.shape == xm.shape
    rng = np.random.default_rng(17)
    checked = 0
    for v in [rng.standard_normal(xm.shape) for _ in range(6)]:
        eps = 1e-6 * np.linalg.norm(xm) / np.linalg.norm(v)
        for _ in range(8):
            op, ip, _ = out_of(xm + eps * v)
            om, im, _ = out_of(xm - eps * v)
            if np.array_equal(ip, ids) and np.array_equal(im, ids):
                break
            eps /= 2
        else:
            continue
        fd = float(np.sum(dout * op) - np.sum(dout * om)) / (2 * eps)
        an = float(np.sum(dxm * v))
        assert abs(fd - an) <= 1e-7 * max(abs(an), 1e-3 * np.linalg.norm(dxm) * np.linalg.norm(v)), (fd, an)
        checked += 1
    assert checked >= 5
    assert w0.H == w.H
