"""libspear_ec: error-compensated 4-bit linear layer for MI355X (gfx950).

y = dequant(Wq) x + alpha * B diag(gamma(A x)) A x with gamma(u) =
sigmoid(g * u + b) (SPEAR summary, section 2.1 A), computed by hand-written
HIP kernels behind the C ABI declared in include/spear_ec.h.  This package
holds the kernels (csrc/), their build script (build.py) and a ctypes binding
(binding.py) with the same names as the C entry points.  PyTorch is used only
to hold device memory and to supply the current stream.
"""
from .binding import (  # noqa: F401
    EXPORTED, SPEAR_EC_DECODE_MAX_TOKENS, SPEAR_EC_OUT_F32, SPEAR_EC_PER_TENSOR,
    SPEAR_EC_WS_WAIT_TIMEOUT, SPEAR_EC_ZEROS, SpearEcError,
    load_library, make_desc,
    spear_ec_dequant_f32, spear_ec_desc, spear_ec_last_error, spear_ec_linear,
    spear_ec_linear_decode, spear_ec_linear_mlp_gate, spear_ec_linear_prefill,
    spear_ec_linear_static,
    spear_ec_linear_serq, spear_ec_lut_kind, spear_ec_lut_measure, spear_ec_pick_chunk,
    spear_ec_step_latency_us,
    spear_ec_quantize_rtn,
    spear_ec_status_string, spear_ec_version, spear_ec_workspace_bytes,
    spear_ec_workspace_status,
)


def packed_shapes(desc):
    """Shapes of the packed weight tensors for a desc: (wq, scales, zeros or None)."""
    G = desc.d_in // desc.group_size
    zs = (desc.d_out, (G + 7) // 8) if desc.flags & SPEAR_EC_ZEROS else None
    return (desc.d_out, desc.d_in // 8), (desc.d_out, G), zs


def alloc_packed(desc, device="cuda"):
    """Empty device tensors for the packed weights: wq (int32 bits), scales
    (int16 bits of fp16), zeros (int32 bits) or None."""
    import torch
    wq_s, sc_s, zs_s = packed_shapes(desc)
    wq = torch.empty(wq_s, dtype=torch.int32, device=device)
    sc = torch.empty(sc_s, dtype=torch.int16, device=device)
    zs = torch.empty(zs_s, dtype=torch.int32, device=device) if zs_s else None
    return wq, sc, zs


def alloc_workspace(desc, max_tokens, device="cuda"):
    """Zero-filled workspace for calls of up to max_tokens tokens."""
    import torch
    n = spear_ec_workspace_bytes(desc, max_tokens)
    if n == 0:
        raise ValueError("invalid desc or token count")
    return torch.zeros(n, dtype=torch.uint8, device=device)
