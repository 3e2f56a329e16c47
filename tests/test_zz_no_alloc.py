"""spear_ec_linear_static, the entry point that allocates nothing (needs an
MI355X): it runs the same kernels as spear_ec_linear on the library's own
static scratch, so its outputs must equal spear_ec_linear's bit for bit (and
meet the oracle's bar).  Two calls in a row on the shared scratch, the second
smaller (prefill, then decode), on two layers; and a call too large for the
scratch is refused before anything is launched."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantization_error_compensation_amd as q
import synth
from helpers import check_bf16_output, from_dev_u16, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a GPU"
    q.load_library()
    return _t


@pytest.mark.parametrize("K,N,r,g,asym,Ts", [(2048, 1024, 32, 128, True, (200, 8)),
                                             (4096, 768, 64, 4096, False, (40, 1)),
                                             (28672, 8192, 64, 128, True, (512, 16))])
def test_static_scratch_equals_workspace_call(torch, K, N, r, g, asym, Ts):
    note(f"static scratch K={K} N={N} r={r} g={g} asym={asym} T={Ts}")
    spec = synth.small_spec(K, N, r, g, asym, seed_base=77000 + K + r)
    W = synth.weights(spec)
    A, B, gv, bv = synth.compensator(spec, r)
    d = q.make_desc(K, N, r, g, asym)
    wq, sc, zs = q.alloc_packed(d)
    q.spear_ec_quantize_rtn(d, to_dev_f32(W), wq, sc, zs)
    o_wq, o_sc, o_zs = oracle.quantize_rtn(W, g, asym)
    del W
    dev = (to_dev_bf16(A), to_dev_bf16(B), to_dev_f32(gv), to_dev_f32(bv))
    for i, T in enumerate(Ts):                       # the second call is smaller
        x = synth.activations(spec, T, salt=i)
        dx = to_dev_bf16(x)
        y_ws = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        y_st = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = q.alloc_workspace(d, T)
        q.spear_ec_linear(d, dx, wq, sc, zs, *dev, spec.alpha, y_ws, ws)
        q.spear_ec_linear_static(d, dx, wq, sc, zs, *dev, spec.alpha, y_st)
        torch.cuda.synchronize()
        assert torch.equal(y_st, y_ws), f"call {i} (T={T}) differs from spear_ec_linear"
        ts = np.array(sorted({0, T // 2, T - 1}))
        y_ref = oracle.forward(x[ts], o_wq, o_sc, o_zs, A, B, gv, bv, spec.alpha, g)
        ok, st = check_bf16_output(from_dev_u16(y_st)[ts], y_ref)
        assert ok, (T, st)


def test_static_scratch_refuses_a_call_too_large(torch):
    d = q.make_desc(8192, 8192, 128, 8192, False)     # 4096 tokens need about 72 MiB
    x = torch.zeros((4096, 8192), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((4096, 8192), dtype=torch.bfloat16, device="cuda")
    wq, sc, zs = q.alloc_packed(d)
    A = torch.zeros((128, 8192), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8192, 128), dtype=torch.bfloat16, device="cuda")
    gv = torch.zeros(128, dtype=torch.float32, device="cuda")
    with pytest.raises(q.SpearEcError) as e:
        q.spear_ec_linear_static(d, x, wq, sc, zs, A, B, gv, gv, 1.0, y)
    assert e.value.status == 4
