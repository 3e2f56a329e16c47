"""Pins of the oracle to facts outside itself (no GPU).

Each test ties one oracle function to something it does not compute itself:
hand-derived worked examples (tests/golden/hand_examples.json), library
routines (numpy's float16 conversion, numpy/scipy linear algebra and the
logistic function), brute force over all candidates, and the special cases of
the compensated layer that reduce to a plain product (SPEAR summary, section
2.1 A: effective weight W~ + alpha*B*diag(gamma(Ax))*A; alpha = 0 is plain W4,
gamma == 1 is the static low-rank correction W~ + alpha*B*A of the prior
static compensators named in section 1 and 3.1).
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def hx(s):
    return int(s, 16)


# ------------------------------------------------------------------ formats
def test_half_decode_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_decode_matches_float32_top_half():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    ok = np.isfinite(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_double_to_half_matches_numpy_rounding():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.uniform(-9, 4.6, 4000),
        # exact ties between neighbouring halves, normal and subnormal
        (np.arange(1, 200) + 0.5) * 2.0 ** -24,
        (1024 + np.arange(0, 300) + 0.5) * 2.0 ** -20,
        [0.0, -0.0, 65504.0, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8],
    ])
    for v in vals:
        ref = np.float64(v).astype(np.float16)
        if not np.isfinite(ref):
            continue
        assert oracle.double_to_half(v) == int(np.array(ref).view(np.uint16)), v


def test_double_to_half_saturates_instead_of_overflowing():
    # reading for scales: finite overflow clamps to the largest half
    assert oracle.double_to_half(65519.0) == 0x7BFF
    assert oracle.double_to_half(65520.0) == 0x7BFF
    assert oracle.double_to_half(1e9) == 0x7BFF
    assert oracle.double_to_half(-1e9) == 0xFBFF


def _bf16_brute(v):
    """Nearest bf16 by exhaustive comparison with the two neighbours."""
    f = np.float32(v)
    u = int(np.array(f).view(np.uint32))
    cands = set()
    for base in (u & 0xFFFF0000, (u & 0xFFFF0000) + 0x10000, (u & 0xFFFF0000) - 0x10000):
        cands.add((base >> 16) & 0xFFFF)
    best = None
    for c in cands:
        cv = float(np.array([c << 16], np.uint32).view(np.float32)[0])
        d = abs(cv - v)
        key = (d, c & 1)  # ties: even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_double_to_bf16_matches_brute_force_and_generator():
    rng = np.random.default_rng(2)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.uniform(-6, 6, 3000),
        (256 + np.arange(0, 100) + 0.5) * 2.0 ** -8,   # exact ties
        (256 + np.arange(0, 100) + 0.5 + 2.0 ** -30) * 2.0 ** -8,  # just above ties
    ])
    got = np.array([oracle.double_to_bf16(v) for v in vals], np.uint16)
    brute = np.array([_bf16_brute(v) for v in vals], np.uint16)
    assert np.array_equal(got, brute)
    # the input generator rounds independently; both must agree
    assert np.array_equal(synth.bf16_bits_from_f64(vals), got)


def test_double_to_bf16_is_single_rounding():
    # 1 + 2^-8 + 2^-30: via float32 it would first become 1 + 2^-8 (a tie) and
    # then round to even = 1.0; the correct single rounding goes up.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.double_to_bf16(v) == 0x3F81


def test_sigmoid_matches_scipy_and_never_overflows():
    z = np.concatenate([np.linspace(-50, 50, 1001), [-800.0, -745.0, 700.0, 800.0]])
    got = np.array([oracle.sigmoid(v) for v in z])
    ref = expit(z)
    assert np.all(np.isfinite(got))
    assert np.allclose(got, ref, rtol=1e-15, atol=1e-300)
    assert oracle.sigmoid(40.0) == 1.0          # used for the gamma == 1 special case


# ---------------------------------------------------------------- quantizer
@pytest.mark.parametrize("case", ["quant_sym", "quant_asym", "quant_asym_positive"])
def test_quantizer_hand_examples(golden, case):
    ex = golden[case]
    W = np.array([ex["W"]], np.float32)
    asym = case.startswith("quant_asym")
    wq, sc, zs = oracle.quantize_rtn(W, ex["group_size"], asym)
    assert int(wq[0, 0]) == hx(ex["word"])
    assert int(sc[0, 0]) == hx(ex["scale_bits"])
    assert list(oracle.codes(wq, 8)[0]) == ex["codes"]
    if asym:
        assert int(zs[0, 0]) == hx(ex["zero_word"])
    assert list(oracle.dequant(wq, sc, zs, 8, 8)[0]) == ex["dequant"]


def test_quantizer_hand_example_two_groups(golden):
    ex = golden["quant_asym_two_groups"]
    W = np.array([ex["W"]], np.float32)
    wq, sc, zs = oracle.quantize_rtn(W, ex["group_size"], True)
    assert [int(w) for w in wq[0]] == [hx(w) for w in ex["words"]]
    assert [int(s) for s in sc[0]] == [hx(s) for s in ex["scale_bits"]]
    assert int(zs[0, 0]) == hx(ex["zero_word"])
    assert list(oracle.zero_points(zs, 1, 2)[0]) == [2, 0]


def _brute_force_check(W, wq, sc, zs, g, asym):
    """Each code must be the nearest of the 16 candidates to W (ties: even c-z),
    or the end of the code range when W lies outside it."""
    N, K = W.shape
    G = K // g
    C = oracle.codes(wq, K)
    Z = oracle.zero_points(zs, N, G) if asym else np.full((N, G), 8)
    for n in range(N):
        for j in range(G):
            s = float(np.array(sc[n, j]).view(np.float16))
            z = Z[n, j]
            cand = (np.arange(16) - z) * s          # exact
            for k in range(j * g, (j + 1) * g):
                w = float(W[n, k])
                d = np.abs(w - cand)                 # exact: both on a fine grid
                best = np.flatnonzero(d == d.min())
                if len(best) > 1:                    # tie: even (c - z)
                    best = [c for c in best if (c - z) % 2 == 0]
                assert C[n, k] == best[0], (n, k, w, s, z, C[n, k], best)


@pytest.mark.parametrize("asym,g", [(False, 64), (True, 32), (True, 64)])
def test_quantizer_codes_are_nearest_by_brute_force(asym, g):
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    W[0, 5] = 0.0
    W[1, : g] = 0.0                      # all-zero group: scale becomes 1
    W[2, 7] = W[2, 6] = np.float32(1.5 * 2.0 ** -8)  # candidates for ties
    wq, sc, zs = oracle.quantize_rtn(W, g, asym)
    _brute_force_check(W, wq, sc, zs, g, asym)


def test_quantizer_scales_follow_numpy_half_rounding():
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    for asym, g in [(False, 256), (True, 128), (False, 64)]:
        wq, sc, zs = oracle.quantize_rtn(W, g, asym)
        for n in range(8):
            for j in range(256 // g):
                blk = W[n, j * g:(j + 1) * g].astype(np.float64)
                if asym:
                    lo, hi = min(0.0, blk.min()), max(0.0, blk.max())
                    want = np.float16((hi - lo) / 15.0)
                else:
                    want = np.float16(np.abs(blk).max() / 7.0)
                assert int(sc[n, j]) == int(np.array(want).view(np.uint16))
                if asym:
                    s = float(want)
                    z = int(np.clip(np.rint(-lo / s), 0, 15))
                    assert oracle.zero_points(zs, 8, 256 // g)[n, j] == z


def test_quantizer_symmetric_extremes_and_error_bound():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((5, 512)) * 0.02).astype(np.float32)
    wq, sc, _ = oracle.quantize_rtn(W, 512, False)
    C = oracle.codes(wq, 512)
    Wt = oracle.dequant(wq, sc, None, 512, 512)
    for n in range(5):
        s = float(np.array(sc[n, 0]).view(np.float16))
        a = int(np.argmax(np.abs(W[n])))
        assert C[n, a] in (1, 15)                       # absmax maps to +-7
        assert C[n].min() >= 1 and C[n].max() <= 15     # -8 never needed
        assert np.max(np.abs(W[n] - Wt[n])) <= s / 2   # no clipping


def test_quantizer_symmetric_is_idempotent():
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    for g in (256, 64):
        wq, sc, _ = oracle.quantize_rtn(W, g, False)
        Wt = oracle.dequant(wq, sc, None, 256, g).astype(np.float32)
        wq2, sc2, _ = oracle.quantize_rtn(Wt, g, False)
        assert np.array_equal(wq, wq2) and np.array_equal(sc, sc2)


def test_quantizer_asymmetric_full_range_is_idempotent():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    wq, sc, zs = oracle.quantize_rtn(W, 128, True)
    C = oracle.codes(wq, 128)
    Wt = oracle.dequant(wq, sc, zs, 128, 128).astype(np.float32)
    wq2, sc2, zs2 = oracle.quantize_rtn(Wt, 128, True)
    for n in range(4):
        if C[n].min() == 0 and C[n].max() == 15:   # range spans all codes
            assert np.array_equal(wq[n], wq2[n]) and sc[n, 0] == sc2[n, 0]


# --------------------------------------------- per-tensor scales (Quasar)
# Quasar summary, "Targeted quantization": one symmetric scaling factor per
# tensor for the verify pass.
def test_per_tensor_hand_example(golden):
    e = golden["quant_per_tensor"]
    W = np.array(e["W"], np.float32)
    wq, sc, zs = oracle.quantize_rtn_per_tensor(W)
    assert zs is None
    assert [hex(int(w)) for w in wq[:, 0]] == [w.lower() for w in e["words"]]
    assert np.all(sc == hx(e["scale_bits"]))
    assert oracle.codes(wq, 8).tolist() == e["codes"]
    assert oracle.dequant(wq, sc, None, 8, 8).tolist() == e["dequant"]


def test_per_tensor_single_row_is_per_channel():
    rng = np.random.default_rng(11)
    for K in (8, 256, 1024):
        W = (rng.standard_normal((1, K)) * 0.02).astype(np.float32)
        a = oracle.quantize_rtn_per_tensor(W)
        b = oracle.quantize_rtn(W, K, False)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_per_tensor_scale_is_numpy_half_of_the_global_max_and_codes_are_nearest():
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((24, 512)) * 0.02).astype(np.float32)
    W[5] *= 4.0                                     # one row holds the tensor's max
    wq, sc, _ = oracle.quantize_rtn_per_tensor(W)
    want = np.array(np.float16(np.abs(W.astype(np.float64)).max() / 7.0)).view(np.uint16)
    assert np.all(sc == want)
    s = float(np.array(want).view(np.float16))
    C = oracle.codes(wq, 512)
    assert C.min() >= 1 and C.max() <= 15            # -8 is never needed
    Wt = oracle.dequant(wq, sc, None, 512, 512)
    assert np.max(np.abs(W - Wt)) <= s / 2           # nearest code, no clipping
    # the rows without the max keep that common scale (not their own)
    own = oracle.quantize_rtn(W[:1], 512, False)[1]
    assert int(own[0, 0]) != int(want)


def test_per_tensor_zero_tensor_gets_unit_scale():
    wq, sc, _ = oracle.quantize_rtn_per_tensor(np.zeros((3, 16), np.float32))
    assert np.all(sc == 0x3C00) and np.all(oracle.codes(wq, 16) == 8)


def test_quantizer_zero_group_gets_unit_scale():
    W = np.zeros((2, 16), np.float32)
    for asym in (False, True):
        wq, sc, zs = oracle.quantize_rtn(W, 8, asym)
        assert np.all(sc == 0x3C00)
        assert np.all(oracle.dequant(wq, sc, zs, 16, 8) == 0.0)


# ------------------------------------------------------------------- layer
def _layer(K, N, r, T, g, asym, seed, b_scale=0.5):
    spec = synth.small_spec(K, N, r, g, asym, seed_base=seed)
    W = synth.weights(spec)
    x = synth.activations(spec, T)
    A, B, gv, bv = synth.compensator(spec)
    bv = (np.random.default_rng(seed).standard_normal(r) * b_scale).astype(np.float32)
    wq, sc, zs = oracle.quantize_rtn(W, g, asym)
    return dict(x=x, wq=wq, sc=sc, zs=zs, A=A, B=B, g=gv, b=bv, K=K, N=N, r=r, T=T, gs=g)


def _fwd(L, alpha=1.0, **over):
    d = dict(L)
    d.update(over)
    return oracle.forward(d["x"], d["wq"], d["sc"], d["zs"], d["A"], d["B"], d["g"], d["b"],
                          alpha, d["gs"])


def _xf(L):
    return synth.bf16_bits_to_f32(L["x"]).astype(np.float64)


def _bf(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64)


def test_layer_hand_example(golden):
    ex = golden["layer_tiny"]
    codes = np.array(ex["codes"])
    wq = np.zeros((2, 1), np.uint32)
    for n in range(2):
        for k in range(8):
            wq[n, 0] |= np.uint32(codes[n, k] << (4 * k))
    sc = np.full((2, 1), np.array(np.float16(ex["scale"])).view(np.uint16), np.uint16)
    x = synth.bf16_bits_from_f64(np.array([ex["x"]], np.float64))
    A = synth.bf16_bits_from_f64(np.array(ex["A"], np.float64))
    B = synth.bf16_bits_from_f64(np.array(ex["B"], np.float64))
    g = np.array(ex["g"], np.float32)
    b = np.array(ex["b"], np.float32)
    y, u, v = oracle.forward(x, wq, sc, None, A, B, g, b, ex["alpha"], 8, return_uv=True)
    assert np.allclose(y[0], ex["y"], rtol=0, atol=1e-15)
    assert np.allclose(u[0], ex["u"], rtol=0, atol=0)
    assert np.allclose(v[0], ex["v"], rtol=0, atol=1e-16)


@pytest.mark.parametrize("asym,g", [(False, 64), (True, 16)])
def test_alpha_zero_is_the_plain_w4_product(asym, g):
    L = _layer(64, 40, 6, 3, g, asym, 11)
    y = _fwd(L, alpha=0.0)
    ref = _xf(L) @ oracle.dequant(L["wq"], L["sc"], L["zs"], 64, g).T
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("asym,g", [(False, 64), (True, 16)])
def test_unit_gate_is_the_static_low_rank_correction(asym, g):
    L = _layer(64, 40, 6, 3, g, asym, 12)
    ones = np.zeros(6, np.float32)
    forty = np.full(6, 40.0, np.float32)
    y = _fwd(L, alpha=0.75, g=ones, b=forty)
    Wt = oracle.dequant(L["wq"], L["sc"], L["zs"], 64, g)
    Weff = Wt + 0.75 * _bf(L["B"]) @ _bf(L["A"])     # static W~ + alpha B A
    assert np.allclose(y, _xf(L) @ Weff.T, rtol=1e-13, atol=1e-13)


# ------------------------------------------------ bottleneck-MLP gate
# SPEAR summary, section 2.1 A: the gate is a bottleneck MLP; the oracle's
# form is sigmoid(W2 relu(W1 u + b1) + b2).  Pinned through cases that reduce
# it to the (pinned) elementwise gate.
def _mlp(r, h, seed):
    return synth.mlp_gate(synth.small_spec(64, 40, r, 64, False, seed_base=seed), r, h)


def test_mlp_gate_with_zero_w2_is_the_constant_elementwise_gate():
    L = _layer(64, 40, 6, 3, 64, False, 21)
    m = _mlp(6, 3, 21)
    m["w2"][:] = 0.0
    y = oracle.forward(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], None, None, 0.8, 64,
                       mlp=m)
    ref = _fwd(L, alpha=0.8, g=np.zeros(6, np.float32), b=m["b2"])
    assert np.allclose(y, ref, rtol=1e-15, atol=1e-15)


def test_mlp_gate_with_identity_bottleneck_is_the_elementwise_gate():
    # W1 = I, b1 = c large (relu is the identity there), W2 = diag(g),
    # b2 = b - g c:  W2 relu(u + c) + b2 = g u + b.
    L = _layer(64, 40, 6, 3, 64, True, 22)
    c = 50.0
    m = {"w1": np.eye(6, dtype=np.float32), "b1": np.full(6, c, np.float32),
         "w2": np.diag(L["g"]).astype(np.float32),
         "b2": (L["b"].astype(np.float64) - L["g"].astype(np.float64) * c).astype(np.float32)}
    y = oracle.forward(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], None, None, 0.9, 64,
                       mlp=m)
    # b2 = b - g c is rounded to fp32, so the two gates differ by that rounding
    assert np.allclose(y, _fwd(L, alpha=0.9), rtol=1e-6, atol=1e-6)


def test_mlp_gate_relu_clips_negative_bottleneck_inputs():
    # b1 far below any W1 u: every hidden unit is clipped to 0 and the gate is
    # sigmoid(b2) whatever W2 is (an identity activation would not give this).
    L = _layer(64, 40, 6, 3, 64, False, 23)
    m = _mlp(6, 4, 23)
    m["b1"][:] = -1.0e6
    y = oracle.forward(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], None, None, 1.0, 64,
                       mlp=m)
    ref = _fwd(L, alpha=1.0, g=np.zeros(6, np.float32), b=m["b2"])
    assert np.allclose(y, ref, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("h", [1, 3, 6])
def test_mlp_gate_factored_path_equals_explicit_effective_weight(h):
    L = _layer(48, 16, 6, 2, 16, True, 24 + h)
    m = _mlp(6, h, 24 + h)
    args = (L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], None, None, 0.7, 16)
    y = oracle.forward(*args, mlp=m)
    ye = oracle.forward_effective_weight(*args, mlp=m)
    assert np.allclose(y, ye, rtol=1e-12, atol=1e-14)
    # and the gate really depends on the token (not the constant sigmoid(b2))
    yc = _fwd(L, alpha=0.7, g=np.zeros(6, np.float32), b=m["b2"])
    assert not np.allclose(y, yc, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("r,h", [(6, 3), (5, 9), (8, 1)])
def test_mlp_gate_matches_an_independent_numpy_evaluation(r, h):
    # gamma(u) = sigmoid(W2 relu(W1 u + b1) + b2) evaluated by numpy matrix
    # products and scipy's logistic function over the header's layouts
    # (w1 [h][r], w2 [r][h]) with h != r and non-symmetric random weights, so
    # a transposed W1 or W2 (or a swapped bias) gives other numbers.  u comes
    # from the oracle and is itself pinned to x A^T by numpy.
    L = _layer(64, 24, r, 4, 16, True, 40 + r + h)
    rng = np.random.default_rng(900 + 10 * r + h)
    m = {"w1": rng.standard_normal((h, r)).astype(np.float32),
         "b1": (0.3 * rng.standard_normal(h)).astype(np.float32),
         "w2": rng.standard_normal((r, h)).astype(np.float32),
         "b2": (0.5 * rng.standard_normal(r)).astype(np.float32)}
    y, u, v = oracle.forward(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], None, None, 0.8,
                             16, return_uv=True, mlp=m)
    uref = _xf(L) @ _bf(L["A"]).T
    assert np.allclose(u, uref, rtol=1e-14, atol=1e-14)
    w1, b1 = m["w1"].astype(np.float64), m["b1"].astype(np.float64)
    w2, b2 = m["w2"].astype(np.float64), m["b2"].astype(np.float64)
    hid = np.maximum(uref @ w1.T + b1, 0.0)                  # [T][h]
    gam = expit(hid @ w2.T + b2)                              # [T][r]
    assert np.any((hid > 0) & (hid < 1e3)) and np.any(hid == 0.0)   # relu active both ways
    assert np.allclose(v, gam * uref, rtol=1e-12, atol=1e-14)
    Wt = oracle.dequant(L["wq"], L["sc"], L["zs"], 64, 16)
    a32 = float(np.float32(0.8))                              # alpha crosses the ABI as fp32
    yref = _xf(L) @ Wt.T + a32 * (gam * uref) @ _bf(L["B"]).T
    assert np.allclose(y, yref, rtol=1e-12, atol=1e-13)
    # the sampled form uses the same gate
    ti, ni = np.array([0, 3, 1, 2]), np.array([23, 0, 7, 11])
    ys = oracle.forward_sampled(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], None, None,
                                0.8, 16, ti, ni, mlp=m)
    assert np.array_equal(ys, y[ti, ni])


def test_correction_vanishes_when_projection_is_zero():
    L = _layer(64, 40, 6, 4, 64, False, 13)
    A = _bf(L["A"]).copy()
    A[:, 32:] = 0.0                                   # A supported on channels 0..31
    x = _xf(L).copy()
    x[:, :32] = 0.0                                   # x zero there -> A x == 0
    Ab = synth.bf16_bits_from_f64(A)
    xb = synth.bf16_bits_from_f64(x)
    y1 = _fwd(L, x=xb, A=Ab)
    y0 = _fwd(L, x=xb, A=Ab, alpha=0.0)
    assert np.array_equal(y1, y0)


def test_compensator_only_path_matches_library_products():
    # all codes equal the zero-point -> W~ == 0 -> y = alpha * B (gamma(Ax) . Ax)
    L = _layer(64, 40, 6, 3, 16, True, 14)
    wq = np.full_like(L["wq"], 0x88888888)
    zs = np.full_like(L["zs"], 0x88888888)
    y = _fwd(L, wq=wq, zs=zs, alpha=1.25)
    u = _xf(L) @ _bf(L["A"]).T
    v = expit(L["g"].astype(np.float64) * u + L["b"].astype(np.float64)) * u
    assert np.allclose(y, 1.25 * v @ _bf(L["B"]).T, rtol=1e-13, atol=1e-15)


def test_projection_and_gate_outputs_match_library_products():
    L = _layer(96, 24, 5, 4, 32, True, 15)
    y, u, v = oracle.forward(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], L["g"], L["b"],
                             1.0, 32, return_uv=True)
    uref = _xf(L) @ _bf(L["A"]).T
    assert np.allclose(u, uref, rtol=1e-14, atol=1e-14)
    gam = expit(L["g"].astype(np.float64) * uref + L["b"].astype(np.float64))
    assert np.allclose(v, gam * uref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("K,N,r,T,g,asym", [(8, 8, 1, 1, 8, False), (24, 16, 3, 3, 8, True),
                                            (64, 40, 8, 2, 64, False), (32, 12, 5, 3, 16, True)])
def test_factored_path_equals_explicit_effective_weight(K, N, r, T, g, asym):
    L = _layer(K, N, r, T, g, asym, 16 + K)
    y = _fwd(L, alpha=0.9)
    ye = oracle.forward_effective_weight(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"],
                                         L["g"], L["b"], 0.9, g)
    scale = max(1.0, np.abs(ye).max())
    assert np.max(np.abs(y - ye)) <= 1e-12 * scale


def test_rank_zero_is_plain_w4():
    L = _layer(64, 16, 4, 2, 64, False, 17)
    y0 = oracle.forward(L["x"], L["wq"], L["sc"], None, None, None, None, None, 1.0, 64)
    ya = _fwd(L, alpha=0.0)
    assert np.array_equal(y0, ya)


def test_sampled_forward_matches_full_forward():
    L = _layer(128, 48, 8, 5, 32, True, 18)
    y = _fwd(L)
    rng = np.random.default_rng(0)
    ti = rng.integers(0, 5, 40)
    ni = rng.integers(0, 48, 40)
    ys = oracle.forward_sampled(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], L["g"],
                                L["b"], 1.0, 32, ti, ni)
    assert np.array_equal(ys, y[ti, ni])


@pytest.mark.parametrize("alpha", [0.0, 0.7, -1.3])
def test_sampled_forward_matches_full_forward_at_any_alpha(alpha):
    # forward_sampled is the reference of the full-size GPU checks; at
    # alpha != 1 it must scale the correction exactly as the full forward
    # does, and at alpha = 0 give the plain W4 product of numpy.
    L = _layer(128, 40, 8, 4, 32, True, 60)
    y = _fwd(L, alpha=alpha)
    rng = np.random.default_rng(61)
    ti = rng.integers(0, 4, 30)
    ni = rng.integers(0, 40, 30)
    ys = oracle.forward_sampled(L["x"], L["wq"], L["sc"], L["zs"], L["A"], L["B"], L["g"],
                                L["b"], alpha, 32, ti, ni)
    assert np.array_equal(ys, y[ti, ni])
    Wt = oracle.dequant(L["wq"], L["sc"], L["zs"], 128, 32)
    u = _xf(L) @ _bf(L["A"]).T
    v = expit(L["g"].astype(np.float64) * u + L["b"].astype(np.float64)) * u
    yref = _xf(L) @ Wt.T + float(np.float32(alpha)) * v @ _bf(L["B"]).T   # alpha is fp32
    assert np.allclose(ys, yref[ti, ni], rtol=1e-12, atol=1e-13)


def test_outputs_do_not_depend_on_batch_composition():
    L = _layer(64, 24, 4, 6, 16, True, 19)
    y = _fwd(L)
    for t in range(6):
        yt = _fwd(L, x=L["x"][t:t + 1])
        assert np.array_equal(yt[0], y[t])


# SERQ single-matrix reconstruction (SERQ summary, section 2): y = W~ x + R x[S]
# with S = [s0, s0 + k).

def _serq_case(K, N, k, T, g, asym, seed):
    L = _layer(K, N, k, T, g, asym, seed)
    rng = np.random.default_rng(seed + 7000)
    R = synth.bf16_bits_from_f64(rng.standard_normal((N, k)) * 0.05)
    return L, R


@pytest.mark.parametrize("s0", [0, 8, 40])
def test_serq_is_spear_with_a_selector_and_a_unit_gate(s0):
    # A = the 0/1 selector of channels s0 .. s0 + k, g = 0 and b = 1e30 (sigmoid
    # exactly 1 in double), alpha = 1, B = R: the SPEAR forward then sums the
    # same products in the same order, so the two agree bit for bit.
    L, R = _serq_case(64, 40, 6, 3, 64, True, 31)
    k, K = 6, 64
    A = np.zeros((k, K), np.float64)
    A[np.arange(k), s0 + np.arange(k)] = 1.0
    y_serq = oracle.forward_serq(L["x"], L["wq"], L["sc"], L["zs"], s0, R, 64)
    y_spear = oracle.forward(L["x"], L["wq"], L["sc"], L["zs"], synth.bf16_bits_from_f64(A), R,
                             np.zeros(k, np.float32), np.full(k, 1e30, np.float32), 1.0, 64)
    assert np.array_equal(y_serq, y_spear)


def test_serq_with_zero_matrix_is_the_plain_w4_product():
    L, R = _serq_case(64, 40, 6, 3, 64, False, 32)
    y = oracle.forward_serq(L["x"], L["wq"], L["sc"], L["zs"], 16, np.zeros_like(R), 64)
    assert np.array_equal(y, _fwd(L, alpha=0.0))


@pytest.mark.parametrize("asym,g", [(False, 48), (True, 16)])
def test_serq_matches_a_dense_matmul_with_the_scattered_matrix(asym, g):
    # (W~ + R P) x with P the k x K selector, as one numpy matmul over the
    # dequantized weights: a different summation path from the oracle's loops.
    K, N, k, T, s0 = 48, 24, 5, 4, 16
    L, R = _serq_case(K, N, k, T, g, asym, 33 + g)
    Wt = oracle.dequant(L["wq"], L["sc"], L["zs"], K, g)
    Rd = _bf(R)
    Wfull = Wt.copy()
    Wfull[:, s0:s0 + k] += Rd
    y_ref = _xf(L) @ Wfull.T
    y = oracle.forward_serq(L["x"], L["wq"], L["sc"], L["zs"], s0, R, g)
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    ys = oracle.forward_serq_sampled(L["x"], L["wq"], L["sc"], L["zs"], s0, R, g,
                                     [0, 3, 2], [0, 23, 7])
    assert np.array_equal(ys, y[[0, 3, 2], [0, 23, 7]])
