"""Python binding of libspear_ec (ctypes; argument marshalling only).

Every function here has the name of the C entry point it calls and does
nothing but turn torch tensors into device pointers, pick the current HIP
stream, and raise on a non-zero status.  All computation happens in the HIP
kernels of libspear_ec.so.  There is no fallback: if the library is missing,
importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SPEAR_EC_LIB names another build of the library to load (for example a
# host-only build with sanitizers, used by the CPU tests).
LIB_PATH = os.environ.get("SPEAR_EC_LIB") or os.path.join(HERE, "libspear_ec.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "spear_ec.h")

SPEAR_EC_OK = 0
SPEAR_EC_ERR_INVALID_ARGUMENT = 1
SPEAR_EC_ERR_UNSUPPORTED = 2
SPEAR_EC_ERR_MISALIGNED = 3
SPEAR_EC_ERR_WORKSPACE = 4
SPEAR_EC_ERR_HIP = 5
SPEAR_EC_ZEROS = 1
SPEAR_EC_PER_TENSOR = 2
SPEAR_EC_OUT_F32 = 4
SPEAR_EC_WS_WAIT_TIMEOUT = 1
SPEAR_EC_DECODE_MAX_TOKENS = 32

EXPORTED = (
    "spear_ec_workspace_bytes", "spear_ec_workspace_status", "spear_ec_linear", "spear_ec_linear_decode",
    "spear_ec_linear_prefill", "spear_ec_linear_static", "spear_ec_linear_mlp_gate",
    "spear_ec_linear_serq",
    "spear_ec_step_latency_us", "spear_ec_pick_chunk", "spear_ec_lut_measure",
    "spear_ec_quantize_rtn",
    "spear_ec_dequant_f32", "spear_ec_status_string", "spear_ec_last_error", "spear_ec_version",
)


class spear_ec_desc(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("flags", ctypes.c_int32)]


class spear_ec_lut_kind(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("tokens", ctypes.POINTER(ctypes.c_int32)),
                ("us", ctypes.POINTER(ctypes.c_float)), ("count", ctypes.c_int32)]


class SpearEcError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"libspear_ec status {status}: {text}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspear_ec.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m quantization_error_compensation_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    DP = ctypes.POINTER(spear_ec_desc)
    lib.spear_ec_workspace_bytes.argtypes = [DP, i32]
    lib.spear_ec_workspace_bytes.restype = sz
    lib.spear_ec_workspace_status.argtypes = [P, sz, P, ctypes.POINTER(i32)]
    lib.spear_ec_workspace_status.restype = ctypes.c_int
    lin = [DP, i32, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, sz, P]
    for name in ("spear_ec_linear", "spear_ec_linear_decode", "spear_ec_linear_prefill"):
        getattr(lib, name).argtypes = lin
        getattr(lib, name).restype = ctypes.c_int
    lib.spear_ec_linear_static.argtypes = [DP, i32, P, P, P, P, P, P, P, P, ctypes.c_float, P, P]
    lib.spear_ec_linear_static.restype = ctypes.c_int
    lib.spear_ec_linear_mlp_gate.argtypes = [DP, i32, P, P, P, P, P, P, i32, P, P, P, P,
                                             ctypes.c_float, P, P, sz, P]
    lib.spear_ec_linear_mlp_gate.restype = ctypes.c_int
    lib.spear_ec_linear_serq.argtypes = [DP, i32, P, P, P, P, i32, P, P, P, sz, P]
    lib.spear_ec_linear_serq.restype = ctypes.c_int
    KP = ctypes.POINTER(spear_ec_lut_kind)
    f32 = ctypes.c_float
    lib.spear_ec_step_latency_us.argtypes = [KP, i32, i32, i32, f32]
    lib.spear_ec_step_latency_us.restype = f32
    lib.spear_ec_pick_chunk.argtypes = [KP, i32, i32, f32, f32, i32, i32]
    lib.spear_ec_pick_chunk.restype = i32
    lib.spear_ec_lut_measure.argtypes = [DP, ctypes.POINTER(i32), i32, i32, P, P, P, P, P, P, P, P,
                                         f32, P, P, sz, P, ctypes.POINTER(f32)]
    lib.spear_ec_lut_measure.restype = ctypes.c_int
    lib.spear_ec_quantize_rtn.argtypes = [DP, P, P, P, P, P]
    lib.spear_ec_quantize_rtn.restype = ctypes.c_int
    lib.spear_ec_dequant_f32.argtypes = [DP, P, P, P, P, P]
    lib.spear_ec_dequant_f32.restype = ctypes.c_int
    lib.spear_ec_status_string.argtypes = [ctypes.c_int]
    lib.spear_ec_status_string.restype = ctypes.c_char_p
    lib.spear_ec_last_error.argtypes = []
    lib.spear_ec_last_error.restype = ctypes.c_char_p
    lib.spear_ec_version.argtypes = []
    lib.spear_ec_version.restype = ctypes.c_int
    _lib = lib
    return lib


def make_desc(d_in: int, d_out: int, rank: int, group_size: int, zeros: bool,
              per_tensor: bool = False, out_f32: bool = False) -> spear_ec_desc:
    flags = ((SPEAR_EC_ZEROS if zeros else 0) | (SPEAR_EC_PER_TENSOR if per_tensor else 0) |
             (SPEAR_EC_OUT_F32 if out_f32 else 0))
    return spear_ec_desc(d_in, d_out, rank, group_size, flags)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int):
    if status != SPEAR_EC_OK:
        lib = load_library()
        raise SpearEcError(status, (lib.spear_ec_last_error() or b"").decode() or
                           lib.spear_ec_status_string(status).decode())


def spear_ec_version() -> int:
    return load_library().spear_ec_version()


def spear_ec_status_string(status: int) -> str:
    return load_library().spear_ec_status_string(status).decode()


def spear_ec_last_error() -> str:
    return load_library().spear_ec_last_error().decode()


def spear_ec_workspace_bytes(desc: spear_ec_desc, max_tokens: int) -> int:
    return int(load_library().spear_ec_workspace_bytes(ctypes.byref(desc), int(max_tokens)))


def spear_ec_workspace_status(workspace, stream=None) -> int:
    """Synchronize the stream, return the workspace's error bits
    (SPEAR_EC_WS_*, 0 = none) and clear them."""
    bits = ctypes.c_int32(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().spear_ec_workspace_status(_ptr(workspace), ws_bytes, _stream(stream),
                                                    ctypes.byref(bits)))
    return int(bits.value)


def _linear(name, desc, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace, stream):
    tokens = int(x.shape[0])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = getattr(load_library(), name)
    _check(fn(ctypes.byref(desc), tokens, _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(A),
              _ptr(B), _ptr(g), _ptr(b), float(alpha), _ptr(y), _ptr(workspace), ws_bytes,
              _stream(stream)))


def spear_ec_linear(desc, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace, stream=None):
    """Phase-aware dispatch: decode for <= 32 tokens, prefill above."""
    _linear("spear_ec_linear", desc, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace, stream)


def spear_ec_linear_decode(desc, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace,
                           stream=None):
    _linear("spear_ec_linear_decode", desc, x, wq, scales, zeros, A, B, g, b, alpha, y,
            workspace, stream)


def spear_ec_linear_prefill(desc, x, wq, scales, zeros, A, B, g, b, alpha, y, workspace,
                            stream=None):
    _linear("spear_ec_linear_prefill", desc, x, wq, scales, zeros, A, B, g, b, alpha, y,
            workspace, stream)


def spear_ec_linear_static(desc, x, wq, scales, zeros, A, B, g, b, alpha, y, stream=None):
    """spear_ec_linear on the library's own scratch (no workspace argument)."""
    _check(load_library().spear_ec_linear_static(
        ctypes.byref(desc), int(x.shape[0]), _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(A),
        _ptr(B), _ptr(g), _ptr(b), float(alpha), _ptr(y), _stream(stream)))


def spear_ec_linear_mlp_gate(desc, x, wq, scales, zeros, A, B, w1, b1, w2, b2, alpha, y,
                             workspace, stream=None):
    """Same layer with the bottleneck-MLP gate (w1 [h][r], b1 [h], w2 [r][h],
    b2 [r], fp32 device tensors; h from w1's first dimension)."""
    tokens = int(x.shape[0])
    hidden = int(w1.shape[0]) if w1 is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().spear_ec_linear_mlp_gate(
        ctypes.byref(desc), tokens, _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(A),
        _ptr(B), hidden, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), float(alpha), _ptr(y),
        _ptr(workspace), ws_bytes, _stream(stream)))


def spear_ec_linear_serq(desc, x, wq, scales, zeros, salient_begin, R, y, workspace,
                         stream=None):
    """SERQ single-matrix reconstruction: y = W~ x + R x[:, s0 : s0 + k]
    (k = desc.rank, R bf16 [d_out][k])."""
    tokens = int(x.shape[0])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().spear_ec_linear_serq(
        ctypes.byref(desc), tokens, _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros),
        int(salient_begin), _ptr(R), _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)))


def _kinds(kinds):
    """[{tokens, us, count}] -> a ctypes array of spear_ec_lut_kind (and the
    arrays it points to, kept alive with it)."""
    keep = []
    arr = (spear_ec_lut_kind * max(1, len(kinds)))()
    for i, k in enumerate(kinds):
        t = (ctypes.c_int32 * len(k["tokens"]))(*[int(v) for v in k["tokens"]])
        u = (ctypes.c_float * len(k["us"]))(*[float(v) for v in k["us"]])
        keep += [t, u]
        arr[i] = spear_ec_lut_kind(len(k["tokens"]), t, u, int(k["count"]))
    return arr, keep


def spear_ec_step_latency_us(kinds, decode_tokens, chunk_tokens, overhead_us=0.0) -> float:
    arr, _keep = _kinds(kinds)
    return float(load_library().spear_ec_step_latency_us(arr, len(kinds), int(decode_tokens),
                                                         int(chunk_tokens), float(overhead_us)))


def spear_ec_pick_chunk(kinds, decode_tokens, itl_us, overhead_us=0.0, max_chunk=8192,
                        granule=32) -> int:
    arr, _keep = _kinds(kinds)
    return int(load_library().spear_ec_pick_chunk(arr, len(kinds), int(decode_tokens),
                                                  float(itl_us), float(overhead_us),
                                                  int(max_chunk), int(granule)))


def spear_ec_lut_measure(desc, tokens, reps, x, wq, scales, zeros, A, B, g, b, alpha, y,
                         workspace, stream=None):
    """Latency (us) of one spear_ec_linear call at each token count."""
    n = len(tokens)
    t = (ctypes.c_int32 * n)(*[int(v) for v in tokens])
    out = (ctypes.c_float * n)()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().spear_ec_lut_measure(
        ctypes.byref(desc), t, n, int(reps), _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(A),
        _ptr(B), _ptr(g), _ptr(b), float(alpha), _ptr(y), _ptr(workspace), ws_bytes,
        _stream(stream), out))
    return [float(v) for v in out]


def spear_ec_quantize_rtn(desc, w, wq, scales, zeros, stream=None):
    _check(load_library().spear_ec_quantize_rtn(ctypes.byref(desc), _ptr(w), _ptr(wq),
                                                _ptr(scales), _ptr(zeros), _stream(stream)))


def spear_ec_dequant_f32(desc, wq, scales, zeros, w_out, stream=None):
    _check(load_library().spear_ec_dequant_f32(ctypes.byref(desc), _ptr(wq), _ptr(scales),
                                               _ptr(zeros), _ptr(w_out), _stream(stream)))
