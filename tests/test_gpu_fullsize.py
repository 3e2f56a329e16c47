"""GPU parity at the full layer sizes of the benchmark workloads (needs an MI355X).

Each workload's layer is built at its real shape, quantized by both sides
(bytes compared whole), and run through the dispatcher entry point exactly as
bench.py calls it (one workspace sized for the call's token count).  The fp64
oracle is too slow for every output of these layers, so it computes a sample
of outputs one by one: the first and last token, the first and last rows,
rows on both sides of the 128-row band edges (decode bands; every other one
is a 256-row prefill tile edge) that the sample draws, and
random (token, row) pairs.  The sampled outputs meet the same elementwise bar
as the small cases; every output must be finite.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantization_error_compensation_amd as q
import synth
from helpers import (REL_TOL, bf16_bits_to_f64, from_dev_u16, from_dev_u32, half_ulp_bf16,
                     to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a GPU"
    q.load_library()
    return _t


def sample_points(T, N, n_random, seed):
    rng = np.random.default_rng(seed)
    ts = [0, T - 1] + list(rng.integers(0, T, n_random))
    ns = [0, N - 1] + list(rng.integers(0, N, n_random))
    edges = rng.integers(1, max(2, N // 128), 4) * 128        # band edges: rows 128k - 1, 128k
    for e in edges:
        if e < N:
            ts += [int(rng.integers(0, T)), int(rng.integers(0, T))]
            ns += [int(e) - 1, int(e)]
    ts += [T - 1, 0]
    ns += [0, N - 1]
    return np.array(ts, np.int32), np.array(ns, np.int32)


def check_sampled(y_bits, t_idx, n_idx, yref):
    y = bf16_bits_to_f64(y_bits[t_idx, n_idx])
    m = float(np.abs(yref).max())
    err = np.abs(y - yref)
    bound = half_ulp_bf16(yref) + REL_TOL * m
    worst = int(np.argmax(err - bound))
    return bool(np.all(err <= bound)), {"max_abs_err": float(err.max()), "ref_max": m,
                                        "worst": (int(t_idx[worst]), int(n_idx[worst]))}


class FullLayer:
    def __init__(self, torch, name):
        self.spec = spec = synth.CONFIGS[name]
        self.K, self.N, self.g, self.asym = spec.d_in, spec.d_out, spec.group_size, spec.asym
        note(f"{name}: weights {self.N}x{self.K}, g={self.g}, asym={self.asym}")
        W = synth.weights(spec)
        if spec.per_tensor:
            self.o_wq, self.o_sc, self.o_zs = oracle.quantize_rtn_per_tensor(W)
        else:
            self.o_wq, self.o_sc, self.o_zs = oracle.quantize_rtn(W, self.g, self.asym)
        d = q.make_desc(self.K, self.N, 0, self.g, self.asym, spec.per_tensor)
        self.d_wq, self.d_sc, self.d_zs = q.alloc_packed(d)
        note(f"{name}: GPU quantize")
        q.spear_ec_quantize_rtn(d, to_dev_f32(W), self.d_wq, self.d_sc, self.d_zs)
        torch.cuda.synchronize()
        del W

    def bytes_match(self):
        ok = np.array_equal(from_dev_u32(self.d_wq), self.o_wq)
        ok &= np.array_equal(self.d_sc.view(__import__("torch").int16).cpu().numpy().view(np.uint16),
                             self.o_sc)
        if self.asym:
            ok &= np.array_equal(from_dev_u32(self.d_zs), self.o_zs)
        return bool(ok)

    def run_and_check(self, torch, T, r, seed):
        spec = self.spec
        x = synth.activations(spec, T)
        A, B, gv, bv = synth.compensator(spec, r)
        desc = q.make_desc(self.K, self.N, r, self.g, self.asym, spec.per_tensor)
        y = torch.empty((T, self.N), dtype=torch.bfloat16, device="cuda")
        ws = q.alloc_workspace(desc, T)
        dev = (to_dev_bf16(A), to_dev_bf16(B), to_dev_f32(gv), to_dev_f32(bv)) if r else (None,) * 4
        note(f"  T={T} r={r}: spear_ec_linear")
        q.spear_ec_linear(desc, to_dev_bf16(x), self.d_wq, self.d_sc, self.d_zs, *dev, spec.alpha,
                          y, ws)
        torch.cuda.synchronize()
        err_word = int(ws[:16].view(torch.int32)[3].item())
        yb = from_dev_u16(y)
        ti, ni = sample_points(T, self.N, 200, seed)
        yref = oracle.forward_sampled(x, self.o_wq, self.o_sc, self.o_zs, A if r else None, B, gv,
                                      bv, spec.alpha, self.g, ti, ni)
        ok, st = check_sampled(yb, ti, ni, yref)
        finite = bool(np.all(np.isfinite(bf16_bits_to_f64(yb))))
        return ok and finite and err_word == 0, dict(st, finite=finite, err_word=err_word)


def test_full_size_mlp_gate_c3(torch):
    """The 70B down-projection with the bottleneck-MLP gate (h = 16): decode
    (T = 16, 1) and prefill (T = 512), sampled against the oracle."""
    L = FullLayer(torch, "c3")
    spec = L.spec
    m = synth.mlp_gate(spec, spec.rank, 16)
    dm = {k: to_dev_f32(v) for k, v in m.items()}
    for i, T in enumerate((16, 1, 512)):
        x = synth.activations(spec, T)
        A, B, _, _ = synth.compensator(spec)
        desc = q.make_desc(L.K, L.N, spec.rank, L.g, L.asym)
        y = torch.empty((T, L.N), dtype=torch.bfloat16, device="cuda")
        ws = q.alloc_workspace(desc, T)
        note(f"  MLP gate T={T}")
        q.spear_ec_linear_mlp_gate(desc, to_dev_bf16(x), L.d_wq, L.d_sc, L.d_zs, to_dev_bf16(A),
                                   to_dev_bf16(B), dm["w1"], dm["b1"], dm["w2"], dm["b2"],
                                   spec.alpha, y, ws)
        torch.cuda.synchronize()
        assert int(ws[:16].view(torch.int32)[3].item()) == 0
        ti, ni = sample_points(T, L.N, 200, 700 + i)
        yref = oracle.forward_sampled(x, L.o_wq, L.o_sc, L.o_zs, A, B, None, None, spec.alpha,
                                      L.g, ti, ni, mlp=m)
        ok, st = check_sampled(from_dev_u16(y), ti, ni, yref)
        assert ok, (T, st)


def test_full_size_serq_c3(torch):
    """The 70B down-projection with SERQ's single-matrix reconstruction of 64
    salient channels (at the front after the offline permutation, and at an
    inner offset): decode (T = 16, 1, 32) and prefill (T = 512), sampled
    against the oracle."""
    L = FullLayer(torch, "c3")
    spec = L.spec
    k = 64
    R = synth.serq_matrix(spec, k)
    dR = to_dev_bf16(R)
    desc = q.make_desc(L.K, L.N, k, L.g, L.asym)
    for i, (T, s0) in enumerate(((16, 0), (1, 0), (32, 4096), (512, 0))):
        x = synth.serq_activations(spec, T)
        y = torch.empty((T, L.N), dtype=torch.bfloat16, device="cuda")
        ws = q.alloc_workspace(desc, T)
        note(f"  SERQ T={T} s0={s0}")
        q.spear_ec_linear_serq(desc, to_dev_bf16(x), L.d_wq, L.d_sc, L.d_zs, s0, dR, y, ws)
        torch.cuda.synchronize()
        assert int(ws[:16].view(torch.int32)[3].item()) == 0
        ti, ni = sample_points(T, L.N, 200, 800 + i)
        yref = oracle.forward_serq_sampled(x, L.o_wq, L.o_sc, L.o_zs, s0, R, L.g, ti, ni)
        ok, st = check_sampled(from_dev_u16(y), ti, ni, yref)
        assert ok, (T, s0, st)


@pytest.mark.parametrize("name,runs", [
    ("c1", [(1, 32), (8, 32), (32, 32)]),
    ("c2", [(2048, 64), (1, 64)]),
    ("c3", [(16, 64), (512, 64), (1, 64), (32, 64)]),
    ("c4", [(1, 0), (1, 16), (1, 64), (1, 128), (16, 0), (16, 128), (256, 64), (4096, 128)]),
    ("v1", [(9, 0), (2, 0), (5, 0)]),
])
def test_full_size_layer(torch, name, runs):
    L = FullLayer(torch, name)
    assert L.bytes_match(), f"{name}: quantized bytes differ"
    for i, (T, r) in enumerate(runs):
        ok, st = L.run_and_check(torch, T, r, seed=100 * i + T)
        assert ok, (name, T, r, st)
