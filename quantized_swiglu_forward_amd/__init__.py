"""Fused quantized SwiGLU expansion for AMD Instinct MI355X (gfx950).

``hidden = silu(x Wg^T) * (x Wu^T)`` with affine group-quantized Wg/Wu, computed
by the hand-written HIP kernels of ``libswiglu_q.so``.  This module only
marshals arguments into the library's C ABI (``include/swiglu_q.h``): every
step of the computation runs in the HIP kernels, and nothing here falls back
to another implementation.  PyTorch supplies device memory and streams.

Functions with the C names take raw device pointers (ints) or tensors and
return the integer status; ``forward`` / ``debug_gemm_tensors`` are tensor
conveniences that allocate outputs with torch and raise ``SwigluQError``.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libswiglu_q.so")

(SWQ_OK, SWQ_ERR_NULL, SWQ_ERR_SHAPE, SWQ_ERR_UNSUPPORTED, SWQ_ERR_ALIGN, SWQ_ERR_HIP, SWQ_ERR_WORKSPACE,
 SWQ_ERR_TOO_LARGE) = range(8)
SWQ_MATCH, SWQ_F32, SWQ_F32_BF16OUT = 0, 1, 2
SWQ_PATH_GEMV, SWQ_PATH_MFMA, SWQ_PATH_AUTO = 0, 1, -1
SWQ_LINEAR_BF16, SWQ_LINEAR_F32 = 0, 1

_lib = None


class SwigluQError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: status {status} ({strerror(status)})" if what else
                         f"status {status} ({strerror(status)})")


def lib():
    """Load ``libswiglu_q.so``; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m quantized_swiglu_forward_amd.build`")
    _lib = load_library(LIB_PATH)
    return _lib


def load_library(path):
    """A ctypes handle on a build of the library at ``path`` (the product, or
    its LDS-poison debug twin ``libswiglu_q_ldspoison.so``) with every entry
    point's signature declared."""
    L = ctypes.CDLL(path)
    vp, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
    L.swiglu_q_forward.argtypes = [vp] * 7 + [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp]
    L.swiglu_q_forward.restype = i32
    L.swiglu_q_forward_f16.argtypes = [vp] * 7 + [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp]
    L.swiglu_q_forward_f16.restype = i32
    L.swiglu_q_forward_noalloc.argtypes = [vp] * 7 + [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp]
    L.swiglu_q_forward_noalloc.restype = i32
    L.swiglu_q_linear.argtypes = [vp] * 4 + [i64, i64, i64, i32, i32, i32, vp, vp]
    L.swiglu_q_linear.restype = i32
    L.swiglu_q_mlp.argtypes = [vp] * 11 + [i64, i64, i64, i64, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    L.swiglu_q_mlp.restype = i32
    L.swiglu_q_debug_gemm.argtypes = [vp] * 7 + [i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp]
    L.swiglu_q_debug_gemm.restype = i32
    L.swiglu_q_supported.argtypes = [i64, i32, i32, i32, i32, i32]
    L.swiglu_q_supported.restype = i32
    L.swiglu_q_set_m_threshold.argtypes = [i32]
    L.swiglu_q_set_m_threshold.restype = None
    L.swiglu_q_path_for.argtypes = [i64, i64, i64]
    L.swiglu_q_path_for.restype = i32
    L.swiglu_q_get_m_threshold.argtypes = []
    L.swiglu_q_get_m_threshold.restype = i32
    L.swiglu_q_call_count.argtypes = [i32]
    L.swiglu_q_call_count.restype = u64
    L.swiglu_q_reset_counts.argtypes = []
    L.swiglu_q_reset_counts.restype = None
    L.swiglu_q_staging_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32]
    L.swiglu_q_staging_bytes.restype = i64
    L.swiglu_q_set_max_calls.argtypes = [i64]
    L.swiglu_q_set_max_calls.restype = None
    L.swiglu_q_under_cap.argtypes = []
    L.swiglu_q_under_cap.restype = i32
    L.swiglu_q_strerror.argtypes = [i32]
    L.swiglu_q_strerror.restype = ctypes.c_char_p
    L.swiglu_q_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32]
    L.swiglu_q_workspace_bytes.restype = i64
    L.swiglu_q_release_workspace.argtypes = []
    L.swiglu_q_release_workspace.restype = i32
    L.swiglu_q_version.argtypes = []
    L.swiglu_q_version.restype = ctypes.c_char_p
    return L


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- the C entry points, same names ---------------------------------------

def swiglu_q_forward(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u,
                     precision_mode, out, stream=None) -> int:
    return lib().swiglu_q_forward(_ptr(x), _ptr(Wg), _ptr(sg), _ptr(bg), _ptr(Wu), _ptr(su), _ptr(bu),
                                  M, H, I, bits_g, gs_g, bits_u, gs_u, precision_mode, _ptr(out),
                                  _stream(stream))


def swiglu_q_forward_f16(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u,
                         precision_mode, out, stream=None) -> int:
    return lib().swiglu_q_forward_f16(_ptr(x), _ptr(Wg), _ptr(sg), _ptr(bg), _ptr(Wu), _ptr(su), _ptr(bu),
                                      M, H, I, bits_g, gs_g, bits_u, gs_u, precision_mode, _ptr(out),
                                      _stream(stream))


def swiglu_q_forward_noalloc(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u,
                             precision_mode, out, stream=None) -> int:
    return lib().swiglu_q_forward_noalloc(_ptr(x), _ptr(Wg), _ptr(sg), _ptr(bg), _ptr(Wu), _ptr(su), _ptr(bu),
                                          M, H, I, bits_g, gs_g, bits_u, gs_u, precision_mode, _ptr(out),
                                          _stream(stream))


def swiglu_q_linear(x, W, s, b, M, K, N, bits, gs, out_mode, out, stream=None) -> int:
    return lib().swiglu_q_linear(_ptr(x), _ptr(W), _ptr(s), _ptr(b), M, K, N, bits, gs, out_mode, _ptr(out),
                                 _stream(stream))


def swiglu_q_mlp(x, Wg, sg, bg, Wu, su, bu, Wd, sd, bd, residual, M, H, I, Ho, bits_g, gs_g, bits_u, gs_u,
                 bits_d, gs_d, out_mode, out, stream=None) -> int:
    return lib().swiglu_q_mlp(_ptr(x), _ptr(Wg), _ptr(sg), _ptr(bg), _ptr(Wu), _ptr(su), _ptr(bu), _ptr(Wd),
                              _ptr(sd), _ptr(bd), _ptr(residual), M, H, I, Ho, bits_g, gs_g, bits_u, gs_u, bits_d,
                              gs_d, out_mode, _ptr(out), _stream(stream))


def swiglu_q_path_for(M, H, I) -> int:
    return lib().swiglu_q_path_for(M, H, I)


def swiglu_q_debug_gemm(x, Wg, sg, bg, Wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u, path,
                        gate_out, up_out, stream=None) -> int:
    return lib().swiglu_q_debug_gemm(_ptr(x), _ptr(Wg), _ptr(sg), _ptr(bg), _ptr(Wu), _ptr(su), _ptr(bu),
                                     M, H, I, bits_g, gs_g, bits_u, gs_u, path, _ptr(gate_out),
                                     _ptr(up_out), _stream(stream))


def swiglu_q_supported(H, bits_g, gs_g, bits_u, gs_u, precision_mode) -> int:
    return lib().swiglu_q_supported(H, bits_g, gs_g, bits_u, gs_u, precision_mode)


def swiglu_q_set_m_threshold(T: int) -> None:
    lib().swiglu_q_set_m_threshold(T)


def swiglu_q_get_m_threshold() -> int:
    return lib().swiglu_q_get_m_threshold()


def swiglu_q_call_count(path: int) -> int:
    return lib().swiglu_q_call_count(path)


def swiglu_q_reset_counts() -> None:
    lib().swiglu_q_reset_counts()


def swiglu_q_set_max_calls(n: int) -> None:
    lib().swiglu_q_set_max_calls(n)


def swiglu_q_under_cap() -> int:
    return lib().swiglu_q_under_cap()


def swiglu_q_strerror(status: int) -> str:
    return lib().swiglu_q_strerror(status).decode()


def swiglu_q_workspace_bytes(M, H, I, bits_g, gs_g, bits_u, gs_u) -> int:
    return lib().swiglu_q_workspace_bytes(M, H, I, bits_g, gs_g, bits_u, gs_u)


def swiglu_q_staging_bytes(M, H, I, bits_g, gs_g, bits_u, gs_u, path=SWQ_PATH_AUTO) -> int:
    return lib().swiglu_q_staging_bytes(M, H, I, bits_g, gs_g, bits_u, gs_u, path)


def swiglu_q_release_workspace() -> int:
    return lib().swiglu_q_release_workspace()


def swiglu_q_version() -> str:
    return lib().swiglu_q_version().decode()


strerror = swiglu_q_strerror


# ---- tensor conveniences ----------------------------------------------------
#
# Like the pages' host entry, these take activations of any leading shape
# [..., H]: the leading dimensions are collapsed into M rows (which must then be
# one contiguous [M, H] block) and restored on the output ("mlx-bun 0.0.7 ->
# 0.0.9" diff, page 42, fused-swiglu-kernel.ts, host entry).

_BITS16 = ("torch.bfloat16", "torch.int16", "torch.uint16")


def _rows(x, what, f16=False):
    """(x as [M, H], leading shape) for bf16 activations (or their int16/uint16
    bit patterns; with f16, float16 activations); raises for any other dtype
    or a non-contiguous tensor."""
    ok = _BITS16 + (("torch.float16",) if f16 else ())
    if str(x.dtype) not in ok:
        raise TypeError(f"{what}: x must be bfloat16{' or float16' if f16 else ''} "
                        f"(or its 16-bit patterns), not {x.dtype}")
    if x.dim() < 1:
        raise ValueError(f"{what}: x needs at least one dimension")
    if not x.is_contiguous():
        raise ValueError(f"{what}: x must be contiguous (rows are read without strides)")
    lead = tuple(x.shape[:-1])
    return x.reshape(-1, x.shape[-1]), lead


def forward(x, wg, sg, bg, wu, su, bu, bits_g, gs_g, bits_u=None, gs_u=None,
            mode=SWQ_MATCH, out=None, stream=None):
    """``hidden`` for device tensors: x [..., H] (bf16 or int16/uint16 bit
    patterns), packed codes int32/uint32 [I, H*bits/32], scales/biases bf16
    [I, H/gs].  float16 x (with float16 scales and biases) runs
    swiglu_q_forward_f16.  Returns ``out`` ([..., I]: float32 in SWQ_F32,
    else x's 16-bit type)."""
    import torch
    bits_u = bits_g if bits_u is None else bits_u
    gs_u = gs_g if gs_u is None else gs_u
    x2, lead = _rows(x, "forward", f16=True)
    f16 = x.dtype == torch.float16
    if any((t.dtype == torch.float16) != f16 for t in (sg, bg, su, bu)):
        raise TypeError("forward: scales and biases must have x's type (float16 with float16 x, bf16 otherwise)")
    M, H = int(x2.shape[0]), int(x2.shape[1])
    I = int(wg.shape[0])
    if out is None:
        dt = torch.float32 if mode == SWQ_F32 else (torch.float16 if f16 else torch.bfloat16)
        out = torch.empty(lead + (I,), dtype=dt, device=x.device)
    entry = swiglu_q_forward_f16 if f16 else swiglu_q_forward
    rc = entry(x2, wg, sg, bg, wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u, mode, out, stream)
    if rc != SWQ_OK:
        raise SwigluQError(rc, entry.__name__)
    return out


def linear(x, w, s, b, bits, gs, out_mode=SWQ_LINEAR_BF16, out=None, stream=None):
    """``x W^T`` for device tensors: x [..., K] bf16, packed codes [N, K*bits/32],
    scales/biases bf16 [N, K/gs].  Returns ``out`` ([..., N], bf16 or float32)."""
    import torch
    x2, lead = _rows(x, "linear")
    M, K = int(x2.shape[0]), int(x2.shape[1])
    N = int(w.shape[0])
    if out is None:
        dt = torch.float32 if out_mode == SWQ_LINEAR_F32 else torch.bfloat16
        out = torch.empty(lead + (N,), dtype=dt, device=x.device)
    rc = swiglu_q_linear(x2, w, s, b, M, K, N, bits, gs, out_mode, out, stream)
    if rc != SWQ_OK:
        raise SwigluQError(rc, "swiglu_q_linear")
    return out


def mlp(x, wg, sg, bg, wu, su, bu, wd, sd, bd, spec_g, spec_u, spec_d, residual=None,
        out_mode=SWQ_LINEAR_BF16, out=None, stream=None):
    """``residual + (silu(x Wg^T) * (x Wu^T)) Wd^T`` for device tensors; each
    spec is (bits, group size); Wd is [Ho, I*bits_d/32]; x is [..., H] and the
    residual, when given, bf16 [..., Ho].  Returns ``out`` ([..., Ho], bf16 or
    float32 by out_mode)."""
    import torch
    x2, lead = _rows(x, "mlp")
    M, H = int(x2.shape[0]), int(x2.shape[1])
    I, Ho = int(wg.shape[0]), int(wd.shape[0])
    if residual is not None:
        residual, rlead = _rows(residual, "mlp residual")
        if rlead != lead or int(residual.shape[1]) != Ho:
            raise ValueError(f"mlp: residual must be [..., {Ho}] with x's leading shape {lead}")
    if out is None:
        dt = torch.float32 if out_mode == SWQ_LINEAR_F32 else torch.bfloat16
        out = torch.empty(lead + (Ho,), dtype=dt, device=x.device)
    rc = swiglu_q_mlp(x2, wg, sg, bg, wu, su, bu, wd, sd, bd, residual, M, H, I, Ho, spec_g[0], spec_g[1],
                      spec_u[0], spec_u[1], spec_d[0], spec_d[1], out_mode, out, stream)
    if rc != SWQ_OK:
        raise SwigluQError(rc, "swiglu_q_mlp")
    return out


def debug_gemm_tensors(x, wg, sg, bg, wu, su, bu, bits_g, gs_g, bits_u=None, gs_u=None,
                       path=SWQ_PATH_AUTO, stream=None):
    """Pre-epilogue float32 (gate, up) from the kernel of ``path``."""
    import torch
    bits_u = bits_g if bits_u is None else bits_u
    gs_u = gs_g if gs_u is None else gs_u
    x, _ = _rows(x, "debug_gemm")
    M, H = int(x.shape[0]), int(x.shape[1])
    I = int(wg.shape[0])
    g = torch.empty((M, I), dtype=torch.float32, device=x.device)
    u = torch.empty((M, I), dtype=torch.float32, device=x.device)
    rc = swiglu_q_debug_gemm(x, wg, sg, bg, wu, su, bu, M, H, I, bits_g, gs_g, bits_u, gs_u, path, g, u, stream)
    if rc != SWQ_OK:
        raise SwigluQError(rc, "swiglu_q_debug_gemm")
    return g, u


def to_device(prob, device="cuda"):
    """Copy a host problem (numpy bit patterns) to device tensors; returns the
    tuple (x, wg, sg, bg, wu, su, bu), x and the scales and biases as bf16, or
    float16 for a problem drawn with binary16 activations."""
    import numpy as np
    import torch
    dt16 = torch.float16 if getattr(prob, "act", "bf16") == "f16" else torch.bfloat16

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(dt16)

    def t32(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)

    return (t16(prob.x), t32(prob.wg), t16(prob.sg), t16(prob.bg),
            t32(prob.wu), t16(prob.su), t16(prob.bu))
