"""Seeded synthetic inputs for the compensated W4 linear layer.

This module is shared by the tests and the benchmark and holds none of the
layer's arithmetic: it only draws Gaussian tensors with numpy's PCG64
generator and stores them in the input dtypes (fp32 weights, bf16 activations
and compensator factors, fp32 gate vectors).  Quantization, unpacking and the
compensated product live elsewhere (the oracle on the CPU, the HIP library on
the GPU), each written independently.

Workloads (shapes and value distributions of the five layer configurations the
layer is evaluated on):
  c0  d_in=d_out=512, 4 tokens, symmetric per-channel, rank 16
  c1  d_in=d_out=4096 (7B attention projection), 1/8/32 decode tokens,
      group 128 asymmetric with int4 zero-points, rank 32
  c2  d_in=4096 -> d_out=11008 (7B MLP up-projection), 2048 prefill tokens,
      symmetric per-channel, rank 64, 0.5% outlier channels x30
  c3  d_in=28672 -> d_out=8192 (70B MLP down-projection), one step of 512
      prefill + 16 decode tokens, group 128 asymmetric, rank 64, W std 0.01
  c4  d_in=d_out=8192 sweep, rank {0,16,64,128} x tokens {1,16,256,4096},
      symmetric per-channel

Distributions: W ~ N(0, 0.02) (c3: 0.01) drawn in fp64 and rounded to fp32;
x ~ N(0, 1) with a fixed set of round_half_up(frac * d_in) outlier channels
(frac 1%, factor 20; c2: 0.5%, 30) multiplied in fp64 and rounded once,
directly, to bf16; A ~ N(0, variance 1/d_in); B ~ N(0, 0.01); g ~ N(1, 0.1)
(fp32); b = 0; alpha = 1.  Seeds: 1000 * config + tensor id
(W 1, x 2, outlier set 3, A 4, B 5, g 6, b 7, MLP gate 8-11, SERQ's R 12).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TENSOR_W, TENSOR_X, TENSOR_OUTLIERS, TENSOR_A, TENSOR_B, TENSOR_G, TENSOR_BIAS = 1, 2, 3, 4, 5, 6, 7
TENSOR_W1, TENSOR_B1, TENSOR_W2, TENSOR_B2 = 8, 9, 10, 11   # bottleneck-MLP gate
TENSOR_R = 12                                                # SERQ reconstruction matrix


@dataclass(frozen=True)
class LayerSpec:
    d_in: int
    d_out: int
    rank: int
    group_size: int            # == d_in for per-channel
    asym: bool                 # asymmetric with zero-points
    w_std: float = 0.02
    outlier_frac: float = 0.01
    outlier_scale: float = 20.0
    alpha: float = 1.0
    seed_base: int = 0         # 1000 * config index
    tokens: tuple = field(default=(4,))
    per_tensor: bool = False   # one symmetric scale for the whole tensor


CONFIGS = {
    "c0": LayerSpec(512, 512, 16, 512, False, seed_base=0, tokens=(4,)),
    "c1": LayerSpec(4096, 4096, 32, 128, True, seed_base=1000, tokens=(1, 8, 32)),
    "c2": LayerSpec(4096, 11008, 64, 4096, False, outlier_frac=0.005, outlier_scale=30.0,
                    seed_base=2000, tokens=(2048,)),
    "c3": LayerSpec(28672, 8192, 64, 128, True, w_std=0.01, seed_base=3000, tokens=(512, 16)),
    "c4": LayerSpec(8192, 8192, 128, 8192, False, seed_base=4000, tokens=(1, 16, 256, 4096)),
    # Quasar-shaped verify pass (Quasar summary, "Targeted quantization"):
    # symmetric per-tensor int4, no compensator, draft length + 1 tokens; the
    # layer shape and value distributions are those of c4.
    "v1": LayerSpec(8192, 8192, 0, 8192, False, seed_base=5000, tokens=(2, 5, 9),
                    per_tensor=True),
}
C4_RANKS = (0, 16, 64, 128)


def bf16_bits_from_f64(a) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even) in one step and
    return the 16-bit patterns.  Finite inputs below bf16 overflow only."""
    a = np.asarray(a, np.float64)
    mag = np.abs(a)
    _, e = np.frexp(mag)                                   # mag = m * 2^e, m in [0.5, 1)
    quantum = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)   # 8 significant bits
    r = np.rint(mag / quantum) * quantum
    f32 = np.copysign(r, a).astype(np.float32)             # exact: <= 8 significant bits
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(spec: LayerSpec, tensor: int, salt: int = 0) -> np.random.Generator:
    return np.random.default_rng(spec.seed_base + tensor + 100000 * salt)


def weights(spec: LayerSpec, salt: int = 0, rows: int | None = None) -> np.ndarray:
    """fp32 [d_out][d_in] (or its first `rows` rows: the same stream prefix)."""
    n = spec.d_out if rows is None else rows
    w = _rng(spec, TENSOR_W, salt).standard_normal((n, spec.d_in))
    return (w * spec.w_std).astype(np.float32)


def outlier_channels(spec: LayerSpec, salt: int = 0) -> np.ndarray:
    count = int(np.floor(spec.outlier_frac * spec.d_in + 0.5))
    return np.sort(_rng(spec, TENSOR_OUTLIERS, salt).choice(spec.d_in, size=count, replace=False))


def activations(spec: LayerSpec, tokens: int, salt: int = 0) -> np.ndarray:
    """bf16 bits [tokens][d_in]: N(0,1) with scaled outlier channels."""
    x = _rng(spec, TENSOR_X, salt).standard_normal((tokens, spec.d_in))
    ch = outlier_channels(spec, salt)
    x[:, ch] *= spec.outlier_scale
    return bf16_bits_from_f64(x)


def compensator(spec: LayerSpec, rank: int | None = None, salt: int = 0):
    """(A bf16 bits [r][d_in], B bf16 bits [d_out][r], g fp32 [r], b fp32 [r]).

    Smaller ranks are the leading slices of the full-rank draw (nested
    compensators, so a rank sweep shares everything but the rank)."""
    R = spec.rank
    r = R if rank is None else rank
    A = _rng(spec, TENSOR_A, salt).standard_normal((R, spec.d_in)) / np.sqrt(spec.d_in)
    B = _rng(spec, TENSOR_B, salt).standard_normal((spec.d_out, R)) * 0.01
    g = (1.0 + 0.1 * _rng(spec, TENSOR_G, salt).standard_normal(R)).astype(np.float32)
    b = np.zeros(R, np.float32)
    return (bf16_bits_from_f64(A[:r]), np.ascontiguousarray(bf16_bits_from_f64(B[:, :r])),
            g[:r].copy(), b[:r].copy())


def mlp_gate(spec: LayerSpec, rank: int, hidden: int, salt: int = 0):
    """Bottleneck-MLP gate parameters (fp32): w1 [h][r] ~ N(0, 1/r), b1 [h] ~
    N(0, 0.1), w2 [r][h] ~ N(0, 1/h), b2 [r] ~ N(1, 0.5), so that the gate
    varies between tokens around sigmoid(1)."""
    w1 = _rng(spec, TENSOR_W1, salt).standard_normal((hidden, rank)) / np.sqrt(rank)
    b1 = 0.1 * _rng(spec, TENSOR_B1, salt).standard_normal(hidden)
    w2 = _rng(spec, TENSOR_W2, salt).standard_normal((rank, hidden)) / np.sqrt(hidden)
    b2 = 1.0 + 0.5 * _rng(spec, TENSOR_B2, salt).standard_normal(rank)
    return {k: np.ascontiguousarray(v, dtype=np.float32)
            for k, v in (("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2))}


def serq_activations(spec: LayerSpec, tokens: int, salt: int = 0) -> np.ndarray:
    """bf16 bits [tokens][d_in] for SERQ: the same draw as activations() with
    the outlier channels at the front, [0, count) (SERQ's offline permutation
    makes the salient channels contiguous), so salient_begin = 0."""
    x = _rng(spec, TENSOR_X, salt).standard_normal((tokens, spec.d_in))
    count = int(np.floor(spec.outlier_frac * spec.d_in + 0.5))
    x[:, :count] *= spec.outlier_scale
    return bf16_bits_from_f64(x)


def serq_matrix(spec: LayerSpec, k: int, salt: int = 0) -> np.ndarray:
    """SERQ's reconstruction matrix R, bf16 bits [d_out][k] ~ N(0, 0.01) (B's
    distribution)."""
    R = _rng(spec, TENSOR_R, salt).standard_normal((spec.d_out, k)) * 0.01
    return np.ascontiguousarray(bf16_bits_from_f64(R))


def small_spec(d_in: int, d_out: int, rank: int, group_size: int, asym: bool,
               seed_base: int = 900000, **kw) -> LayerSpec:
    """A test-sized layer with the c0 distributions."""
    return LayerSpec(d_in, d_out, rank, group_size, asym, seed_base=seed_base, **kw)
