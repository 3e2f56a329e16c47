"""Plain fp64 CPU oracle for the error-compensated W4 linear layer.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may use this package; the product path never does.  The
arithmetic lives in ``spear_oracle.cpp`` (single-threaded C++, double
precision); this module only loads that library and marshals numpy arrays.

What each function follows is stated in the C++ file: the RTN quantizer
(SPEAR summary, section 3.1, RTN per-channel setting), the dequantization, the
compensated product with the effective weight
W~ + alpha * B * diag(gamma(A x)) * A (SPEAR summary, section 2.1 A), and
SERQ's single-matrix reconstruction W~ x + R x[S] (SERQ summary, section 2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spear_oracle.cpp")
_LIB = os.path.join(_HERE, "libspear_oracle.so")
_lib = None

# IEEE double semantics: no contraction into fused multiply-adds, no fast-math.
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = False) -> str:
    """Compile the oracle with the host compiler (g++)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", *CXXFLAGS, _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # SPEAR_ORACLE_LIB: another build of this same source (the sanitizer
        # test loads one built with AddressSanitizer and UBSan)
        lib = ctypes.CDLL(os.environ.get("SPEAR_ORACLE_LIB") or build())
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_half_to_double.restype = ctypes.c_double
        lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_double.restype = ctypes.c_double
        lib.orc_double_to_half.argtypes = [ctypes.c_double]
        lib.orc_double_to_half.restype = ctypes.c_uint16
        lib.orc_double_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_double_to_bf16.restype = ctypes.c_uint16
        lib.orc_sigmoid.argtypes = [ctypes.c_double]
        lib.orc_sigmoid.restype = ctypes.c_double
        lib.orc_quantize_rtn.argtypes = [P, i32, i32, i32, i32, P, P, P]
        lib.orc_quantize_rtn.restype = i32
        lib.orc_quantize_rtn_per_tensor.argtypes = [P, i32, i32, P, P]
        lib.orc_quantize_rtn_per_tensor.restype = i32
        lib.orc_code.argtypes = [P, i32, i32, i32]
        lib.orc_code.restype = i32
        lib.orc_zero.argtypes = [P, i32, i32, i32]
        lib.orc_zero.restype = i32
        lib.orc_dequant.argtypes = [P, P, P, i32, i32, i32, P]
        lib.orc_dequant.restype = None
        fwd = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, ctypes.c_float]
        lib.orc_forward.argtypes = fwd + [P, P, P]
        lib.orc_forward.restype = None
        lib.orc_forward_sampled.argtypes = fwd + [i32, P, P, P]
        lib.orc_forward_sampled.restype = None
        lib.orc_forward_effective_weight.argtypes = fwd + [P]
        lib.orc_forward_effective_weight.restype = None
        serq = [i32, i32, i32, i32, i32, P, P, P, P, i32, P]
        lib.orc_forward_serq.argtypes = serq + [P]
        lib.orc_forward_serq.restype = None
        lib.orc_forward_serq_sampled.argtypes = serq + [i32, P, P, P]
        lib.orc_forward_serq_sampled.restype = None
        lib.orc_set_mlp_gate.argtypes = [i32, P, P, P, P]
        lib.orc_set_mlp_gate.restype = None
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- formats
def half_to_double(bits: int) -> float:
    return _load().orc_half_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return _load().orc_bf16_to_double(int(bits))


def double_to_half(v: float) -> int:
    return int(_load().orc_double_to_half(float(v)))


def double_to_bf16(v: float) -> int:
    return int(_load().orc_double_to_bf16(float(v)))


def double_to_bf16_array(a: np.ndarray) -> np.ndarray:
    f = _load().orc_double_to_bf16
    flat = np.asarray(a, dtype=np.float64).ravel()
    return np.fromiter((f(float(v)) for v in flat), dtype=np.uint16, count=flat.size).reshape(np.shape(a))


def sigmoid(z: float) -> float:
    return _load().orc_sigmoid(float(z))


# ------------------------------------------------------------ quantization
def quantize_rtn(W: np.ndarray, group_size: int, asym: bool):
    """RTN int4 quantization + packing. Returns (wq uint32 [N][K/8],
    scales uint16 (fp16 bits) [N][G], zeros uint32 [N][ceil(G/8)] or None)."""
    W = _c(W, np.float32)
    N, K = W.shape
    G = K // group_size
    wq = np.zeros((N, K // 8), np.uint32)
    sc = np.zeros((N, G), np.uint16)
    zs = np.zeros((N, (G + 7) // 8), np.uint32) if asym else None
    rc = _load().orc_quantize_rtn(_p(W), N, K, group_size, int(bool(asym)), _p(wq), _p(sc), _p(zs))
    if rc != 0:
        raise ValueError("oracle quantizer rejected the shape")
    return wq, sc, zs


def quantize_rtn_per_tensor(W: np.ndarray):
    """Symmetric per-tensor RTN int4 quantization + packing (Quasar summary,
    "Targeted quantization"). Returns (wq uint32 [N][K/8], scales uint16 [N][1],
    all equal, None)."""
    W = _c(W, np.float32)
    N, K = W.shape
    wq = np.zeros((N, K // 8), np.uint32)
    sc = np.zeros((N, 1), np.uint16)
    if _load().orc_quantize_rtn_per_tensor(_p(W), N, K, _p(wq), _p(sc)) != 0:
        raise ValueError("oracle quantizer rejected the shape")
    return wq, sc, None


def codes(wq: np.ndarray, K: int) -> np.ndarray:
    """Unpacked codes (int [N][K]) read one by one through the oracle."""
    wq = _c(wq, np.uint32)
    lib = _load()
    N = wq.shape[0]
    out = np.empty((N, K), np.int32)
    for n in range(N):
        for k in range(K):
            out[n, k] = lib.orc_code(_p(wq), K, n, k)
    return out


def zero_points(zeros, N: int, G: int) -> np.ndarray:
    lib = _load()
    z = _c(zeros, np.uint32)
    return np.array([[lib.orc_zero(_p(z), G, n, j) for j in range(G)] for n in range(N)], np.int32)


def dequant(wq, scales, zeros, K: int, group_size: int) -> np.ndarray:
    wq = _c(wq, np.uint32)
    sc = _c(scales, np.uint16)
    zs = _c(zeros, np.uint32)
    N = wq.shape[0]
    out = np.empty((N, K), np.float64)
    _load().orc_dequant(_p(wq), _p(sc), _p(zs), N, K, group_size, _p(out))
    return out


# ------------------------------------------------------------- the layer
def _fwd_args(x, wq, scales, zeros, A, B, g, b):
    x = _c(x, np.uint16)
    wq = _c(wq, np.uint32)
    sc = _c(scales, np.uint16)
    zs = _c(zeros, np.uint32)
    T, K = x.shape
    N = wq.shape[0]
    r = 0 if A is None else int(np.shape(A)[0])
    A = _c(A, np.uint16) if r else None
    B = _c(B, np.uint16) if r else None
    g = _c(g, np.float32) if r else None
    b = _c(b, np.float32) if r else None
    return x, wq, sc, zs, A, B, g, b, T, K, N, r


class _MlpGate:
    """Context: the oracle's gate is the bottleneck MLP (w1 [h][r], b1 [h],
    w2 [r][h], b2 [r], fp32) inside, the elementwise sigmoid after."""

    def __init__(self, mlp):
        self.arrays = None
        if mlp is not None:
            w1, b1, w2, b2 = (_c(mlp[k], np.float32) for k in ("w1", "b1", "w2", "b2"))
            self.arrays = (w1, b1, w2, b2)

    def __enter__(self):
        if self.arrays is not None:
            w1, b1, w2, b2 = self.arrays
            _load().orc_set_mlp_gate(int(w1.shape[0]), _p(w1), _p(b1), _p(w2), _p(b2))

    def __exit__(self, *exc):
        if self.arrays is not None:
            _load().orc_set_mlp_gate(0, None, None, None, None)


def forward(x, wq, scales, zeros, A, B, g, b, alpha, group_size, return_uv=False, mlp=None):
    """y (double [T][N]) of the compensated layer; x, A, B are bf16 bit arrays.
    mlp: None (elementwise gate from g, b) or dict(w1, b1, w2, b2) (bottleneck
    MLP gate; g and b are then unused)."""
    x, wq, sc, zs, A, B, g, b, T, K, N, r = _fwd_args(x, wq, scales, zeros, A, B, g, b)
    y = np.empty((T, N), np.float64)
    u = np.empty((T, max(r, 1)), np.float64)
    v = np.empty((T, max(r, 1)), np.float64)
    with _MlpGate(mlp):
        _load().orc_forward(T, K, N, r, group_size, _p(x), _p(wq), _p(sc), _p(zs), _p(A), _p(B),
                            _p(g), _p(b), float(alpha), _p(y), _p(u), _p(v))
    if return_uv:
        return y, u[:, :r], v[:, :r]
    return y


def forward_sampled(x, wq, scales, zeros, A, B, g, b, alpha, group_size, t_idx, n_idx, mlp=None):
    x, wq, sc, zs, A, B, g, b, T, K, N, r = _fwd_args(x, wq, scales, zeros, A, B, g, b)
    ti = _c(t_idx, np.int32)
    ni = _c(n_idx, np.int32)
    y = np.empty(ti.size, np.float64)
    with _MlpGate(mlp):
        _load().orc_forward_sampled(T, K, N, r, group_size, _p(x), _p(wq), _p(sc), _p(zs), _p(A),
                                    _p(B), _p(g), _p(b), float(alpha), int(ti.size), _p(ti),
                                    _p(ni), _p(y))
    return y


def forward_effective_weight(x, wq, scales, zeros, A, B, g, b, alpha, group_size, mlp=None):
    x, wq, sc, zs, A, B, g, b, T, K, N, r = _fwd_args(x, wq, scales, zeros, A, B, g, b)
    y = np.empty((T, N), np.float64)
    with _MlpGate(mlp):
        _load().orc_forward_effective_weight(T, K, N, r, group_size, _p(x), _p(wq), _p(sc),
                                             _p(zs), _p(A), _p(B), _p(g), _p(b), float(alpha),
                                             _p(y))
    return y


def _serq_args(x, wq, scales, zeros, s0, R):
    x = _c(x, np.uint16)
    wq = _c(wq, np.uint32)
    sc = _c(scales, np.uint16)
    zs = None if zeros is None else _c(zeros, np.uint32)
    R = _c(R, np.uint16)
    T, K = x.shape
    N, k = R.shape
    if not (0 <= s0 and s0 + k <= K):
        raise ValueError("salient channels out of range")
    return x, wq, sc, zs, R, T, K, N, k


def forward_serq(x, wq, scales, zeros, s0, R, group_size):
    """y (double [T][N]) of SERQ's single-matrix reconstruction:
    W~ x + R x[:, s0 : s0 + k]; x, R (d_out x k) are bf16 bit arrays."""
    x, wq, sc, zs, R, T, K, N, k = _serq_args(x, wq, scales, zeros, s0, R)
    y = np.empty((T, N), np.float64)
    _load().orc_forward_serq(T, K, N, k, group_size, _p(x), _p(wq), _p(sc), _p(zs), int(s0),
                             _p(R), _p(y))
    return y


def forward_serq_sampled(x, wq, scales, zeros, s0, R, group_size, t_idx, n_idx):
    x, wq, sc, zs, R, T, K, N, k = _serq_args(x, wq, scales, zeros, s0, R)
    ti = _c(t_idx, np.int32)
    ni = _c(n_idx, np.int32)
    y = np.empty(ti.size, np.float64)
    _load().orc_forward_serq_sampled(T, K, N, k, group_size, _p(x), _p(wq), _p(sc), _p(zs),
                                     int(s0), _p(R), int(ti.size), _p(ti), _p(ni), _p(y))
    return y
