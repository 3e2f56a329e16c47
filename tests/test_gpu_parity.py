"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every case prints its name, shape and seed before touching the GPU.  Inputs
come from the seeded generators in `synth`; each side quantizes the fp32
weights itself (or both receive the same randomly drawn packed bytes), so no
value crosses from the HIP path into the oracle.

Bars: quantized bytes and fp32 dequantized weights bit-exact; one-hot
activations through the production kernels bit-exact; layer outputs within
half a bf16 ulp + 2e-3 * max|y_ref| (tests/helpers.py).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantization_error_compensation_amd as q
import synth
from helpers import (check_bf16_output, from_dev_u16, from_dev_u32, to_dev_bf16, to_dev_f32,
                     to_dev_u16, to_dev_u32)

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a GPU"
    q.load_library()
    return _t


# ------------------------------------------------------------ GPU plumbing
def gpu_quantize(torch, W, group_size, asym):
    N, K = W.shape
    d = q.make_desc(K, N, 0, group_size, asym)
    wq, sc, zs = q.alloc_packed(d)
    q.spear_ec_quantize_rtn(d, to_dev_f32(W), wq, sc, zs)
    torch.cuda.synchronize()
    return wq, sc, zs


class Layer:
    """One layer's inputs, on both sides."""

    def __init__(self, torch, spec, T, rank=None, salt=0, g=None, b=None, x=None):
        self.spec = spec
        self.K, self.N, self.g = spec.d_in, spec.d_out, spec.group_size
        self.r = spec.rank if rank is None else rank
        self.asym = spec.asym
        self.W = synth.weights(spec, salt)
        self.x = synth.activations(spec, T, salt) if x is None else x
        A, B, gv, bv = synth.compensator(spec, self.r, salt)
        self.A, self.B = A, B
        self.gv = gv if g is None else g
        self.bv = bv if b is None else b
        self.alpha = spec.alpha
        # oracle side
        self.o_wq, self.o_sc, self.o_zs = oracle.quantize_rtn(self.W, self.g, self.asym)
        # GPU side (its own quantizer)
        self.d_wq, self.d_sc, self.d_zs = gpu_quantize(torch, self.W, self.g, self.asym)
        self.desc = q.make_desc(self.K, self.N, self.r, self.g, self.asym)
        self.upload_compensator(torch)

    def upload_compensator(self, torch):
        if self.r:
            self.d_A, self.d_B = to_dev_bf16(self.A), to_dev_bf16(self.B)
            self.d_g, self.d_b = to_dev_f32(self.gv), to_dev_f32(self.bv)
        else:
            self.d_A = self.d_B = self.d_g = self.d_b = None

    def run(self, torch, x_bits, path="auto", alpha=None, ws=None):
        T = x_bits.shape[0]
        y = torch.empty((T, self.N), dtype=torch.bfloat16, device="cuda")
        if ws is None:
            ws = q.alloc_workspace(self.desc, max(T, 1))
        fn = {"auto": q.spear_ec_linear, "decode": q.spear_ec_linear_decode,
              "prefill": q.spear_ec_linear_prefill}[path]
        fn(self.desc, to_dev_bf16(x_bits), self.d_wq, self.d_sc, self.d_zs, self.d_A, self.d_B,
           self.d_g, self.d_b, self.alpha if alpha is None else alpha, y, ws)
        torch.cuda.synchronize()
        return from_dev_u16(y)

    def reference(self, x_bits, alpha=None):
        return oracle.forward(x_bits, self.o_wq, self.o_sc, self.o_zs,
                              self.A if self.r else None, self.B, self.gv, self.bv,
                              self.alpha if alpha is None else alpha, self.g)


# ------------------------------------------------------- quantize / dequant
QUANT_CASES = [
    (96, 512, 512, False), (80, 1024, 128, True), (64, 384, 128, False), (32, 256, 256, True),
    (48, 2048, 128, True), (16, 128, 128, True),
]


@pytest.mark.parametrize("N,K,g,asym", QUANT_CASES)
def test_quantizer_bytes_match_oracle(torch, N, K, g, asym):
    note(f"quantize N={N} K={K} g={g} asym={asym}")
    spec = synth.small_spec(K, N, 0, g, asym, seed_base=7000 + K)
    W = synth.weights(spec)
    W[0, :] = 0.0                                       # zero row -> scale 1
    W[1, : min(g, K)] = np.float32(2.0 ** -30)          # scale underflows fp16 -> 1
    W[2, 5] = W[2, 6] = np.float32(0.02)                # repeated values
    wq, sc, zs = gpu_quantize(torch, W, g, asym)
    o_wq, o_sc, o_zs = oracle.quantize_rtn(W, g, asym)
    assert np.array_equal(from_dev_u32(wq), o_wq)
    assert np.array_equal(from_dev_u16(sc), o_sc)
    if asym:
        assert np.array_equal(from_dev_u32(zs), o_zs)


def test_quantizer_hand_examples_on_gpu(torch, golden):
    for case in ("quant_sym", "quant_asym", "quant_asym_positive"):
        ex = golden[case]
        note(f"quantize hand example {case}")
        W = np.zeros((16, 128), np.float32)              # one 16 x 128 block, example in row 0
        W[0, :8] = ex["W"]
        # per-channel over 8 columns is not a supported group; use 8 identical
        # copies so the 128-column group has the same range as the example
        W[0, :] = np.tile(np.array(ex["W"], np.float32), 16)
        asym = case.startswith("quant_asym")
        wq, sc, zs = gpu_quantize(torch, W, 128, asym)
        assert int(from_dev_u32(wq)[0, 0]) == int(ex["word"], 16)
        assert int(from_dev_u16(sc)[0, 0]) == int(ex["scale_bits"], 16)


@pytest.mark.parametrize("N,K,g,asym", [(64, 1024, 128, True), (32, 512, 512, False),
                                        (16, 256, 128, False), (48, 1536, 1536, True)])
def test_dequant_bit_exact_on_random_packed_bytes(torch, N, K, g, asym):
    note(f"dequant N={N} K={K} g={g} asym={asym}")
    rng = np.random.default_rng(100 + K)
    G = K // g
    wq = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = np.array(rng.uniform(1e-4, 4.0, (N, G)), np.float16).view(np.uint16)
    zs = rng.integers(0, 2 ** 32, (N, (G + 7) // 8), dtype=np.uint64).astype(np.uint32) if asym else None
    d = q.make_desc(K, N, 0, g, asym)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    q.spear_ec_dequant_f32(d, to_dev_u32(wq), to_dev_u16(sc),
                           to_dev_u32(zs) if asym else None, out)
    torch.cuda.synchronize()
    ref = oracle.dequant(wq, sc, zs, K, g).astype(np.float32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------ layer parity
LAYER_CASES = [
    # K, N, r, g, asym, T
    (512, 512, 16, 512, False, 4),      # c0-shaped
    (1024, 400, 32, 128, True, 1),
    (1024, 400, 32, 128, True, 5),
    (1024, 400, 32, 128, True, 16),
    (1024, 400, 32, 128, True, 17),
    (1024, 400, 32, 128, True, 32),
    (1024, 400, 32, 128, True, 33),
    (1024, 400, 32, 128, True, 200),
    (768, 272, 64, 768, False, 1),
    (768, 272, 64, 768, False, 24),
    (768, 272, 64, 768, False, 130),
    (128, 16, 16, 128, False, 3),       # single block, single row tile
    (2048, 96, 128, 128, False, 7),     # max rank, symmetric group-wise
    (2048, 96, 128, 128, False, 77),
    (640, 160, 0, 640, True, 9),        # rank 0: plain W4, asymmetric per-channel
    (640, 160, 0, 640, True, 150),
    # odd block counts per row (9, 3): decode runs that start on an odd block
    # move one unit on, runs cross band edges, r = 48 repeats a rank tile
    (1152, 400, 48, 128, True, 7),
    (1152, 400, 48, 128, True, 24),
    (1152, 400, 48, 128, True, 40),
    (384, 208, 16, 384, False, 3),
    (384, 208, 16, 384, False, 31),
]


@pytest.mark.parametrize("K,N,r,g,asym,T", LAYER_CASES)
def test_layer_matches_oracle(torch, K, N, r, g, asym, T):
    note(f"layer K={K} N={N} r={r} g={g} asym={asym} T={T}")
    spec = synth.small_spec(K, N, r, g, asym, seed_base=8000 + K + T)
    bv = (np.random.default_rng(T).standard_normal(r) * 0.5).astype(np.float32)
    L = Layer(torch, spec, T, b=bv)
    assert np.array_equal(from_dev_u32(L.d_wq), L.o_wq)  # both quantizers agree
    yref = L.reference(L.x)
    paths = ["auto", "prefill"] + (["decode"] if T <= 32 else [])
    for path in paths:
        note(f"  path={path}")
        y = L.run(torch, L.x, path)
        ok, st = check_bf16_output(y, yref)
        assert ok, (path, st)


# ------------------------------------ per-tensor verify pass (Quasar)
# Quasar summary, "Targeted quantization": the verify forward runs on int4
# weights with one symmetric per-tensor scale; no compensator; a verify batch
# is the drafted tokens plus one.
@pytest.mark.parametrize("N,K", [(64, 512), (208, 1024), (16, 128)])
def test_per_tensor_quantizer_bytes_match_oracle(torch, N, K):
    note(f"per-tensor quantize N={N} K={K}")
    rng = np.random.default_rng(N + K)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[N // 3] = 0.0                                  # a zero row keeps the common scale
    W[N // 2] *= 3.0                                 # the row holding the tensor's max
    d = q.make_desc(K, N, 0, K, False, True)
    wq, sc, zs = q.alloc_packed(d)
    assert zs is None
    q.spear_ec_quantize_rtn(d, to_dev_f32(W), wq, sc, zs)
    torch.cuda.synchronize()
    o_wq, o_sc, _ = oracle.quantize_rtn_per_tensor(W)
    assert np.array_equal(from_dev_u32(wq), o_wq)
    assert np.array_equal(sc.view(torch.int16).cpu().numpy().view(np.uint16), o_sc)


@pytest.mark.parametrize("K,N,T", [(1024, 400, 2), (1024, 400, 5), (1024, 400, 9), (4096, 256, 9)])
def test_per_tensor_verify_pass_matches_oracle(torch, K, N, T):
    note(f"verify pass K={K} N={N} T={T}")
    spec = synth.small_spec(K, N, 0, K, False, seed_base=9000 + K + T)
    W = synth.weights(spec)
    x = synth.activations(spec, T)
    d = q.make_desc(K, N, 0, K, False, True)
    wq, sc, zs = q.alloc_packed(d)
    q.spear_ec_quantize_rtn(d, to_dev_f32(W), wq, sc, zs)
    o_wq, o_sc, _ = oracle.quantize_rtn_per_tensor(W)
    yref = oracle.forward(x, o_wq, o_sc, None, None, None, None, None, 1.0, K)
    ws = q.alloc_workspace(d, T)
    for fn in (q.spear_ec_linear, q.spear_ec_linear_decode):
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        fn(d, to_dev_bf16(x), wq, sc, zs, None, None, None, None, 1.0, y, ws)
        torch.cuda.synchronize()
        ok, st = check_bf16_output(from_dev_u16(y), yref)
        assert ok, (fn.__name__, st)


# ------------------------------------------------- bottleneck-MLP gate
# SPEAR summary, section 2.1 A: the gate is a bottleneck MLP,
# sigmoid(W2 relu(W1 u + b1) + b2) here.  Decode (rank bands, the MLP pass of
# the last rank band, correction) and prefill (one finishing workgroup per
# token) against the oracle; r = 128 has two rank bands.
MLP_CASES = [
    # K, N, r, h, g, asym, T
    (1024, 400, 32, 8, 128, True, 1),
    (1024, 400, 32, 8, 128, True, 16),
    (1024, 400, 32, 8, 128, True, 33),
    (1024, 400, 32, 1, 128, True, 7),
    (768, 272, 64, 16, 768, False, 24),
    (768, 272, 64, 16, 768, False, 130),
    (2048, 96, 128, 32, 128, False, 5),
    (2048, 96, 128, 128, 128, False, 40),
]


@pytest.mark.parametrize("K,N,r,h,g,asym,T", MLP_CASES)
def test_mlp_gate_layer_matches_oracle(torch, K, N, r, h, g, asym, T):
    note(f"MLP gate K={K} N={N} r={r} h={h} g={g} asym={asym} T={T}")
    spec = synth.small_spec(K, N, r, g, asym, seed_base=11000 + K + T + h)
    L = Layer(torch, spec, T)
    m = synth.mlp_gate(spec, r, h)
    dm = {k: to_dev_f32(v) for k, v in m.items()}
    yref = oracle.forward(L.x, L.o_wq, L.o_sc, L.o_zs, L.A, L.B, None, None, L.alpha, L.g, mlp=m)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    ws = q.alloc_workspace(L.desc, T)
    for rep in range(2):   # the second call checks the gate counters were reset
        q.spear_ec_linear_mlp_gate(L.desc, to_dev_bf16(L.x), L.d_wq, L.d_sc, L.d_zs, L.d_A, L.d_B,
                                   dm["w1"], dm["b1"], dm["w2"], dm["b2"], L.alpha, y, ws)
        torch.cuda.synchronize()
        assert int(ws[:16].view(torch.int32)[3].item()) == 0
        ok, st = check_bf16_output(from_dev_u16(y), yref)
        assert ok, (rep, st)


SERQ_CASES = [
    # K, N, k (salient channels), s0, g, asym, T
    (1024, 400, 32, 0, 128, True, 1),
    (1024, 400, 32, 64, 128, True, 16),
    (1024, 400, 32, 984, 128, True, 33),     # last channels of x
    (768, 272, 64, 8, 768, False, 24),
    (768, 272, 64, 8, 768, False, 130),
    (2048, 96, 128, 256, 128, False, 5),
    (2048, 96, 128, 256, 128, False, 40),
    (512, 48, 16, 496, 512, True, 32),
]


@pytest.mark.parametrize("K,N,k,s0,g,asym,T", SERQ_CASES)
def test_serq_layer_matches_oracle(torch, K, N, k, s0, g, asym, T):
    note(f"SERQ K={K} N={N} k={k} s0={s0} g={g} asym={asym} T={T}")
    spec = synth.small_spec(K, N, k, g, asym, seed_base=12000 + K + T + s0)
    L = Layer(torch, spec, T, x=synth.serq_activations(spec, T))
    R = synth.serq_matrix(spec, k)
    yref = oracle.forward_serq(L.x, L.o_wq, L.o_sc, L.o_zs, s0, R, L.g)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    ws = q.alloc_workspace(L.desc, T)
    for rep in range(2):   # the second call reuses the workspace
        q.spear_ec_linear_serq(L.desc, to_dev_bf16(L.x), L.d_wq, L.d_sc, L.d_zs, s0,
                               to_dev_bf16(R), y, ws)
        torch.cuda.synchronize()
        assert int(ws[:16].view(torch.int32)[3].item()) == 0
        ok, st = check_bf16_output(from_dev_u16(y), yref)
        assert ok, (rep, st)


@pytest.mark.parametrize("K,N,r,g,asym", [(1024, 400, 32, 128, True), (512, 256, 16, 512, False)])
def test_random_packed_bytes_through_both_paths(torch, K, N, r, g, asym):
    """Externally quantized weights (uniform random codes, scales and zero-points)."""
    note(f"random packed K={K} N={N} g={g} asym={asym}")
    rng = np.random.default_rng(5)
    G = K // g
    wq = rng.integers(0, 2 ** 32, (N, K // 8), dtype=np.uint64).astype(np.uint32)
    sc = np.array(rng.uniform(1e-4, 2e-3, (N, G)), np.float16).view(np.uint16)
    zs = rng.integers(0, 2 ** 32, (N, (G + 7) // 8), dtype=np.uint64).astype(np.uint32) if asym else None
    spec = synth.small_spec(K, N, r, g, asym, seed_base=8100)
    x = synth.activations(spec, 40)
    A, B, gv, bv = synth.compensator(spec)
    desc = q.make_desc(K, N, r, g, asym)
    for T, path in [(3, "decode"), (20, "decode"), (40, "prefill"), (3, "prefill")]:
        note(f"  T={T} path={path}")
        xs = x[:T]
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        ws = q.alloc_workspace(desc, T)
        fn = q.spear_ec_linear_decode if path == "decode" else q.spear_ec_linear_prefill
        fn(desc, to_dev_bf16(xs), to_dev_u32(wq), to_dev_u16(sc), to_dev_u32(zs) if asym else None,
           to_dev_bf16(A), to_dev_bf16(B), to_dev_f32(gv), to_dev_f32(bv), 1.0, y, ws)
        torch.cuda.synchronize()
        yref = oracle.forward(xs, wq, sc, zs, A, B, gv, bv, 1.0, g)
        ok, st = check_bf16_output(from_dev_u16(y), yref)
        assert ok, (T, path, st)


# ------------------------------------------------------ exact special cases
@pytest.mark.parametrize("K,N,g,asym", [(1024, 128, 128, True), (512, 64, 512, False)])
def test_one_hot_activation_returns_dequantized_column(torch, K, N, g, asym):
    """x = e_k, alpha = 0: y[:, n] is W~[n, k] rounded to bf16, exactly."""
    note(f"one-hot K={K} N={N} g={g} asym={asym}")
    spec = synth.small_spec(K, N, 16, g, asym, seed_base=8200)
    ks = [0, 1, 7, 8, 127, 128, 300, K - 1]
    x = np.zeros((len(ks), K), np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80                                  # bf16 1.0
    L = Layer(torch, spec, 1, x=x)
    Wt = oracle.dequant(L.o_wq, L.o_sc, L.o_zs, K, g)
    want = oracle.double_to_bf16_array(Wt[:, ks].T)
    for path in ("decode", "prefill"):
        for alpha in (0.0,):
            y = L.run(torch, x, path, alpha=alpha)
            assert np.array_equal(y, want), path


def test_alpha_zero_equals_rank_zero_bitwise(torch):
    spec = synth.small_spec(1024, 256, 32, 128, True, seed_base=8300)
    for T in (4, 48):
        note(f"alpha=0 vs r=0 T={T}")
        L = Layer(torch, spec, T)
        L0 = Layer(torch, synth.small_spec(1024, 256, 0, 128, True, seed_base=8300), T, rank=0)
        for path in ("prefill",) + (("decode",) if T <= 32 else ()):
            ya = L.run(torch, L.x, path, alpha=0.0)
            y0 = L0.run(torch, L.x, path)
            assert np.array_equal(ya, y0), path


def test_correction_vanishes_when_projection_is_zero(torch):
    spec = synth.small_spec(1024, 192, 32, 128, True, seed_base=8400)
    T = 12
    note("Ax = 0")
    L = Layer(torch, spec, T)
    A = L.A.copy()
    A[:, 512:] = 0                                        # A supported on columns < 512
    x = L.x.copy()
    x[:, :512] = 0                                        # x zero there
    L.A = A
    L.upload_compensator(torch)
    for path in ("decode", "prefill"):
        y1 = L.run(torch, x, path)
        y0 = L.run(torch, x, path, alpha=0.0)
        assert np.array_equal(y1, y0), path


def test_unit_gate_matches_static_low_rank_reference(torch):
    spec = synth.small_spec(1024, 192, 32, 128, True, seed_base=8500)
    note("gamma == 1")
    L = Layer(torch, spec, 20, g=np.zeros(32, np.float32), b=np.full(32, 40.0, np.float32))
    yref = L.reference(L.x)
    for path in ("decode", "prefill"):
        ok, st = check_bf16_output(L.run(torch, L.x, path), yref)
        assert ok, (path, st)


def test_tokens_are_independent_and_paths_agree(torch):
    spec = synth.small_spec(2048, 320, 32, 128, True, seed_base=8600)
    L = Layer(torch, spec, 32)
    note("token independence")
    y32 = L.run(torch, L.x, "decode")
    for t in (0, 13, 31):
        y1 = L.run(torch, L.x[t:t + 1], "decode")
        assert np.array_equal(y1[0], y32[t])
    for T in (16, 32):
        yd = L.run(torch, L.x[:T], "decode")
        yp = L.run(torch, L.x[:T], "prefill")
        ok, st = check_bf16_output(yd, L.reference(L.x[:T]))
        assert ok, st
        ok, st = check_bf16_output(yp, L.reference(L.x[:T]))
        assert ok, st


def test_workspace_is_reusable_across_calls(torch):
    spec = synth.small_spec(1024, 256, 32, 128, True, seed_base=8700)
    L = Layer(torch, spec, 64)
    ws = q.alloc_workspace(L.desc, 64)
    note("workspace reuse")
    for T in (64, 5, 32, 1, 40, 5):
        for rep in range(2):
            y = L.run(torch, L.x[:T], "auto", ws=ws)
            ok, st = check_bf16_output(y, L.reference(L.x[:T]))
            assert ok, (T, rep, st)
    assert int((ws[: 4096 * 4].view(torch.int32) != 0).sum()) == 0   # counters and error word at zero


def test_zero_tokens_is_a_no_op(torch):
    spec = synth.small_spec(512, 64, 16, 512, False, seed_base=8800)
    L = Layer(torch, spec, 1)
    y = torch.full((1, 64), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = q.alloc_workspace(L.desc, 1)
    x = to_dev_bf16(L.x)[:0]
    q.spear_ec_linear(L.desc, x, L.d_wq, L.d_sc, L.d_zs, L.d_A, L.d_B, L.d_g, L.d_b, 1.0, y, ws)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
