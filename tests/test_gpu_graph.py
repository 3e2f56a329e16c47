"""The layer's calls replayed from a HIP graph (needs an MI355X).

A serving loop with static shapes captures its calls once and replays them;
the SPEAR summary (section 2.2 A) places the decode-phase compensator in a
static graph.  Every call leaves its workspace as it found it (counters back
at zero), so a replay must reproduce the eager result exactly.  Each case
captures a decode call and a prefill call on one stream, replays the graph
three times with eager work and synchronizations in between, and compares
every replay's outputs with the eager outputs bit for bit; the eager outputs
themselves are checked against the oracle.
"""
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


GRAPH_CASES = [  # K, N, rank, group, asym, decode tokens, prefill tokens
    (2048, 1024, 32, 128, True, 16, 96),
    (1536, 768, 64, 1536, False, 5, 160),
    (1024, 512, 0, 128, True, 32, 40),
]


@pytest.mark.parametrize("K,N,r,g,asym,Td,Tp", GRAPH_CASES)
def test_graph_replay_matches_eager(torch, K, N, r, g, asym, Td, Tp):
    note(f"graph replay K={K} N={N} r={r} g={g} asym={asym} Td={Td} Tp={Tp}")
    spec = synth.small_spec(K, N, r, g, asym, seed_base=8100 + K + r)
    W = synth.weights(spec)
    xd_bits, xp_bits = synth.activations(spec, Td), synth.activations(spec, Tp, salt=1)
    A, B, gv, bv = synth.compensator(spec, r)
    d = q.make_desc(K, N, r, g, asym)
    wq, sc, zs = q.alloc_packed(d)
    q.spear_ec_quantize_rtn(d, to_dev_f32(W), wq, sc, zs)
    dA, dB = (to_dev_bf16(A), to_dev_bf16(B)) if r else (None, None)
    dg, db = (to_dev_f32(gv), to_dev_f32(bv)) if r else (None, None)
    xd, xp = to_dev_bf16(xd_bits), to_dev_bf16(xp_bits)
    yd = torch.empty((Td, N), dtype=torch.bfloat16, device="cuda")
    yp = torch.empty((Tp, N), dtype=torch.bfloat16, device="cuda")
    ws = q.alloc_workspace(d, max(Td, Tp))

    def calls(st):
        q.spear_ec_linear(d, xd, wq, sc, zs, dA, dB, dg, db, spec.alpha, yd, ws, st)
        q.spear_ec_linear(d, xp, wq, sc, zs, dA, dB, dg, db, spec.alpha, yp, ws, st)

    calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref_d, ref_p = from_dev_u16(yd), from_dev_u16(yp)

    o_wq, o_sc, o_zs = oracle.quantize_rtn(W, g, asym)
    for bits, out in ((xd_bits, ref_d), (xp_bits, ref_p)):
        y_ref = oracle.forward(bits, o_wq, o_sc, o_zs, A if r else None, B, gv, bv, spec.alpha, g)
        ok, st = check_bf16_output(out, y_ref)
        assert ok, st

    cap = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        calls(cap)
    torch.cuda.synchronize()

    # eager work between replays: another call of the same layer on other
    # tokens, through the same workspace, and a fill of the outputs
    x_other = to_dev_bf16(synth.activations(spec, Td, salt=2))
    y_other = torch.empty((Td, N), dtype=torch.bfloat16, device="cuda")
    for rep in range(3):
        note(f"  replay {rep}")
        q.spear_ec_linear(d, x_other, wq, sc, zs, dA, dB, dg, db, spec.alpha, y_other, ws)
        yd.fill_(float("nan"))
        yp.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_u16(yd), ref_d), f"decode output differs on replay {rep}"
        assert np.array_equal(from_dev_u16(yp), ref_p), f"prefill output differs on replay {rep}"
