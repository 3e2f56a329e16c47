"""C-ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects bad arguments with the documented
status codes before any HIP call (so no kernel is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

import quantization_error_compensation_amd as q
from quantization_error_compensation_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from quantization_error_compensation_amd import build
        build.build()
    return q.load_library()


def header_functions():
    text = open(os.path.join(ROOT, "include", "spear_ec.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spear_ec_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert header_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(spear_ec_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_status_strings(lib):
    assert q.spear_ec_version() == 1
    for code in range(6):
        assert q.spear_ec_status_string(code)
    assert q.spear_ec_status_string(99) == "unknown status"


def _call(lib, name, desc, tokens, ptrs=None, ws_bytes=0, alpha=1.0):
    p = ptrs or {}
    get = lambda k: p.get(k)  # noqa: E731
    return getattr(lib, name)(ctypes.byref(desc) if desc is not None else None, tokens,
                              get("x"), get("wq"), get("sc"), get("z"), get("A"), get("B"),
                              get("g"), get("b"), alpha, get("y"), get("ws"), ws_bytes, None)


FAKE = {k: 0x10000 * (i + 1) for i, k in enumerate(["x", "wq", "sc", "z", "A", "B", "g", "b", "y", "ws"])}


@pytest.mark.parametrize("name", ["spear_ec_linear", "spear_ec_linear_decode", "spear_ec_linear_prefill"])
def test_validation_codes(lib, name):
    good = q.make_desc(512, 512, 16, 512, False)
    assert _call(lib, name, None, 4, FAKE) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call(lib, name, good, -1, FAKE) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call(lib, name, good, 0) == binding.SPEAR_EC_OK           # no-op, nothing touched
    for bad in [q.make_desc(500, 512, 16, 500, False), q.make_desc(512, 520, 16, 512, False),
                q.make_desc(512, 512, 20, 512, False), q.make_desc(512, 512, 144, 512, False),
                q.make_desc(512, 512, 16, 64, False), q.make_desc(262144, 512, 16, 128, False)]:
        assert _call(lib, name, bad, 4, FAKE) == binding.SPEAR_EC_ERR_UNSUPPORTED
    assert _call(lib, name, q.make_desc(512, 512, 16, 512, False), 4,
                 {**FAKE, "x": None}) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call(lib, name, q.make_desc(512, 512, 16, 128, True), 4,
                 {**FAKE, "z": None}) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call(lib, name, good, 4, {**FAKE, "A": None}) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call(lib, name, good, 4, {**FAKE, "x": FAKE["x"] + 2}) == binding.SPEAR_EC_ERR_MISALIGNED
    assert _call(lib, name, good, 4, {**FAKE, "ws": None}) == binding.SPEAR_EC_ERR_WORKSPACE
    # per-tensor scales: symmetric and per-channel layout only
    for bad in [q.make_desc(512, 512, 16, 512, True, True), q.make_desc(512, 512, 16, 128, False, True)]:
        assert _call(lib, name, bad, 4, FAKE) == binding.SPEAR_EC_ERR_UNSUPPORTED
    assert _call(lib, name, q.make_desc(512, 512, 16, 512, False, True), 0) == binding.SPEAR_EC_OK
    assert _call(lib, name, good, 4, FAKE, ws_bytes=64) == binding.SPEAR_EC_ERR_WORKSPACE
    assert q.spear_ec_last_error()
    # rank 0: compensator pointers may be NULL (still stopped by the small workspace)
    r0 = q.make_desc(512, 512, 0, 512, False)
    assert _call(lib, name, r0, 4, {**FAKE, "A": None, "B": None, "g": None, "b": None},
                 ws_bytes=64) == binding.SPEAR_EC_ERR_WORKSPACE


def _call_mlp(lib, desc, tokens, ptrs, hidden, ws_bytes=1 << 30):
    get = lambda k: ptrs.get(k)
    return lib.spear_ec_linear_mlp_gate(ctypes.byref(desc) if desc is not None else None, tokens,
                                        get("x"), get("wq"), get("sc"), get("z"), get("A"),
                                        get("B"), hidden, get("w1"), get("b1"), get("w2"),
                                        get("b2"), 1.0, get("y"), get("ws"), ws_bytes, None)


def test_mlp_gate_validation_codes(lib):
    fake = {**FAKE, **{k: 0x10000 * (20 + i) for i, k in enumerate(["w1", "b1", "w2", "b2"])}}
    good = q.make_desc(512, 512, 16, 512, False)
    assert _call_mlp(lib, good, 0, fake, 8) == binding.SPEAR_EC_OK
    for hidden in (0, 129, -1):
        assert _call_mlp(lib, good, 4, fake, hidden) == binding.SPEAR_EC_ERR_UNSUPPORTED
    for k in ("w1", "b1", "w2", "b2", "A"):
        assert _call_mlp(lib, good, 4, {**fake, k: None}, 8) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call_mlp(lib, good, 4, {**fake, "w2": fake["w2"] + 4}, 8) == binding.SPEAR_EC_ERR_MISALIGNED
    # rank 0: the gate is not used and may be absent
    r0 = q.make_desc(512, 512, 0, 512, False)
    assert _call_mlp(lib, r0, 0, {}, 0) == binding.SPEAR_EC_OK


def _call_serq(lib, desc, tokens, ptrs, s0, ws_bytes=1 << 30):
    get = lambda k: ptrs.get(k)
    return lib.spear_ec_linear_serq(ctypes.byref(desc) if desc is not None else None, tokens,
                                    get("x"), get("wq"), get("sc"), get("z"), s0, get("B"),
                                    get("y"), get("ws"), ws_bytes, None)


def test_serq_validation_codes(lib):
    good = q.make_desc(512, 512, 16, 512, False)
    assert _call_serq(lib, good, 0, FAKE, 8) == binding.SPEAR_EC_OK
    r0 = q.make_desc(512, 512, 0, 512, False)
    assert _call_serq(lib, r0, 4, FAKE, 0) == binding.SPEAR_EC_ERR_UNSUPPORTED
    for s0 in (-8, 4, 512 - 8, 512):  # negative, not a multiple of 8, past d_in
        assert _call_serq(lib, good, 4, FAKE, s0) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    for k in ("B", "x", "y", "wq"):
        assert _call_serq(lib, good, 4, {**FAKE, k: None}, 8) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call_serq(lib, good, 4, {**FAKE, "B": FAKE["B"] + 4}, 8) == binding.SPEAR_EC_ERR_MISALIGNED
    assert _call_serq(lib, good, 4, FAKE, 8, ws_bytes=64) == binding.SPEAR_EC_ERR_WORKSPACE
    assert _call_serq(lib, good, -1, FAKE, 8) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT


def test_decode_rejects_more_than_32_tokens(lib):
    d = q.make_desc(512, 512, 16, 512, False)
    assert _call(lib, "spear_ec_linear_decode", d, 33, FAKE, ws_bytes=1 << 40) == \
        binding.SPEAR_EC_ERR_UNSUPPORTED


def test_workspace_bytes(lib):
    d = q.make_desc(4096, 4096, 32, 128, True)
    sizes = [q.spear_ec_workspace_bytes(d, t) for t in (1, 8, 32, 33, 512, 4096)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert q.spear_ec_workspace_bytes(d, -1) == 0
    assert q.spear_ec_workspace_bytes(q.make_desc(100, 16, 0, 100, False), 8) == 0


def test_quantize_and_dequant_validation(lib):
    d = q.make_desc(256, 64, 0, 128, True)
    assert lib.spear_ec_quantize_rtn(ctypes.byref(d), 0x10000, 0x20000, 0x30000, None, None) == \
        binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert lib.spear_ec_quantize_rtn(ctypes.byref(d), 0x10004, 0x20000, 0x30000, 0x40000, None) == \
        binding.SPEAR_EC_ERR_MISALIGNED
    assert lib.spear_ec_dequant_f32(ctypes.byref(q.make_desc(256, 64, 0, 64, False)), 0x10000,
                                    0x20000, None, 0x30000, None) == binding.SPEAR_EC_ERR_UNSUPPORTED


def test_workspace_status_validation(lib):
    bits = ctypes.c_int32(-7)
    assert lib.spear_ec_workspace_status(None, 1 << 20, None, ctypes.byref(bits)) == \
        binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert lib.spear_ec_workspace_status(0x10000, 1 << 20, None, None) == \
        binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert lib.spear_ec_workspace_status(0x10000, 8, None, ctypes.byref(bits)) == \
        binding.SPEAR_EC_ERR_WORKSPACE
    assert bits.value == -7          # nothing written on a validation error


@pytest.mark.parametrize("name", ["spear_ec_linear", "spear_ec_linear_decode", "spear_ec_linear_prefill"])
def test_output_flag_is_accepted_and_unknown_flags_are_not(lib, name):
    f32 = q.make_desc(512, 512, 16, 512, False, out_f32=True)
    assert f32.flags == binding.SPEAR_EC_OUT_F32
    assert _call(lib, name, f32, 0) == binding.SPEAR_EC_OK
    assert _call(lib, name, f32, 4, FAKE, ws_bytes=64) == binding.SPEAR_EC_ERR_WORKSPACE
    bad = q.make_desc(512, 512, 16, 512, False)
    bad.flags = 8
    assert _call(lib, name, bad, 4, FAKE) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT


def _call_static(lib, desc, tokens, ptrs, alpha=1.0):
    get = lambda k: ptrs.get(k)  # noqa: E731
    return lib.spear_ec_linear_static(ctypes.byref(desc) if desc is not None else None, tokens,
                                      get("x"), get("wq"), get("sc"), get("z"), get("A"), get("B"),
                                      get("g"), get("b"), alpha, get("y"), None)


def test_static_scratch_entry_validation(lib):
    good = q.make_desc(512, 512, 16, 512, False)
    assert _call_static(lib, None, 4, FAKE) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call_static(lib, good, -1, FAKE) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call_static(lib, good, 0, {}) == binding.SPEAR_EC_OK          # no-op
    assert _call_static(lib, good, 4, {**FAKE, "y": None}) == binding.SPEAR_EC_ERR_INVALID_ARGUMENT
    assert _call_static(lib, good, 4, {**FAKE, "A": FAKE["A"] + 2}) == binding.SPEAR_EC_ERR_MISALIGNED
    assert _call_static(lib, q.make_desc(512, 520, 16, 512, False), 4, FAKE) == \
        binding.SPEAR_EC_ERR_UNSUPPORTED
    # more scratch than the library holds: rejected before any HIP call
    big = q.make_desc(131072, 131072, 128, 128, True)
    assert _call_static(lib, big, 65536, FAKE) == binding.SPEAR_EC_ERR_WORKSPACE
    assert "static scratch" in q.spear_ec_last_error()
