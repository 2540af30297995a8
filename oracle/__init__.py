"""CPU oracle for the fused quantized SwiGLU expansion (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``quantized_swiglu_forward_amd``) and never imports it.

* ``swiglu_pairs`` / ``swiglu_full`` -- the float64 reference of
  ``hidden = silu(x Wg^T) * (x Wu^T)`` with affine group-quantized weights,
  in plain C (``swiglu_oracle.c``), one output element at a time.
* ``qmm`` -- one plain quantized projection (the unfused building block), and
  ``qmm_pairs`` -- the same sums element by element with their scales (the
  reference of the quantized linear ``y = x W^T``).
* ``mlp_pairs`` -- the whole MLP: the MATCH forward's hidden tensor in bf16,
  its down projection and the residual.
* ``exact`` -- an exact rational brute force for tiny shapes.
* ``compare`` -- the per-element error metric used by the parity tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swiglu_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

MATCH, F32, F32_BF16OUT = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-Wall", "-shared",
                        "-fPIC", "-o", tmp, _SRC, "-lm", "-lpthread"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """Load the oracle library, building it only if nothing is built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    L = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    L.oracle_swiglu_pairs.argtypes = [vp] * 7 + [i64, i64, i64, i32, i32, i32, i32, i32,
                                                 i64, vp, vp, vp, vp, vp, vp, vp, i32]
    L.oracle_swiglu_pairs.restype = i32
    L.oracle_swiglu_pairs_act.argtypes = [vp] * 7 + [i64, i64, i64, i32, i32, i32, i32, i32,
                                                     i64, vp, vp, vp, vp, vp, vp, vp, i32, i32]
    L.oracle_swiglu_pairs_act.restype = i32
    L.oracle_f16_rne_array.argtypes = [vp, i64, vp]
    L.oracle_f16_rne_array.restype = None
    L.oracle_f16_value_array.argtypes = [vp, i64, vp]
    L.oracle_f16_value_array.restype = None
    L.oracle_f16_rne.argtypes = [ctypes.c_double]
    L.oracle_f16_rne.restype = ctypes.c_uint16
    L.oracle_qmm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
    L.oracle_qmm.restype = i32
    L.oracle_unpack.argtypes = [vp, i64, i64, i32, vp]
    L.oracle_unpack.restype = i32
    L.oracle_bf16_rne_array.argtypes = [vp, i64, vp]
    L.oracle_bf16_rne_array.restype = None
    L.oracle_silu_array.argtypes = [vp, i64, vp]
    L.oracle_silu_array.restype = None
    L.oracle_bf16_rne.argtypes = [ctypes.c_double]
    L.oracle_bf16_rne.restype = ctypes.c_uint16
    L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_value.restype = ctypes.c_double
    _lib = L
    return L


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def swiglu_pairs(prob, mode, ms=None, ns=None, nthreads=0, want=("g", "u", "nu_g", "nu_u", "h")):
    """Evaluate selected output elements of a ``synth.Problem``.

    ``ms``/``ns`` are equal-length index arrays; ``None`` means every element
    in row-major order.  A problem drawn with binary16 activations
    (``prob.act == "f16"``) is read and, in MATCH, rounded as binary16.
    Returns a dict of float64 arrays named g, u, nu_g, nu_u, h (h is the
    unrounded float64 hidden value), and ``act``."""
    L = lib()
    x = _c(prob.x, np.uint16)
    wg, sg, bg = _c(prob.wg, np.uint32), _c(prob.sg, np.uint16), _c(prob.bg, np.uint16)
    wu, su, bu = _c(prob.wu, np.uint32), _c(prob.su, np.uint16), _c(prob.bu, np.uint16)
    if ms is None:
        n = prob.M * prob.I
        msa = nsa = None
    else:
        msa, nsa = _c(ms, np.int64), _c(ns, np.int64)
        if msa.shape != nsa.shape:
            raise ValueError("ms and ns differ in length")
        n = msa.size
    out = {k: np.empty(n, dtype=np.float64) for k in want}
    act = act_code(prob)
    rc = L.oracle_swiglu_pairs_act(_p(x), _p(wg), _p(sg), _p(bg), _p(wu), _p(su), _p(bu),
                                   prob.M, prob.H, prob.I, prob.bits_g, prob.gs_g,
                                   prob.bits_u, prob.gs_u, int(mode), n, _p(msa), _p(nsa),
                                   _p(out.get("g")), _p(out.get("u")), _p(out.get("nu_g")),
                                   _p(out.get("nu_u")), _p(out.get("h")), act, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out["act"] = act
    return out


def act_code(prob):
    """0 for bf16 activations (the default), 1 for binary16."""
    a = getattr(prob, "act", "bf16")
    if a not in ("bf16", "f16"):
        raise ValueError(f"unknown activation type {a!r}")
    return 1 if a == "f16" else 0


def swiglu_full(prob, mode, nthreads=0):
    """Every output element, each array reshaped to ``[M, I]``."""
    r = swiglu_pairs(prob, mode, nthreads=nthreads)
    return {k: (v.reshape(prob.M, prob.I) if k != "act" else v) for k, v in r.items()}


def qmm(x_bits, W, S, B, M, H, N, bits, gs):
    """Plain quantized projection ``y = x W^T`` in float64, ``[M, N]``."""
    L = lib()
    y = np.empty((M, N), dtype=np.float64)
    x, W, S, B = _c(x_bits, np.uint16), _c(W, np.uint32), _c(S, np.uint16), _c(B, np.uint16)
    if L.oracle_qmm(_p(x), _p(W), _p(S), _p(B), M, H, N, bits, gs, _p(y)) != 0:
        raise ValueError("oracle rejected its arguments")
    return y


def qmm_pairs(x_bits, W, S, B, M, H, N, bits, gs, ms=None, ns=None, nthreads=0):
    """``y = x W^T`` and its scale ``nu = sqrt(sum_k (x_k w_k)^2)`` in float64 at
    the elements (ms[p], ns[p]) (every element, row-major, when None): the
    oracle's gate dot product with W in both slots.  Returns (y, nu)."""
    L = lib()
    x, W, S, B = _c(x_bits, np.uint16), _c(W, np.uint32), _c(S, np.uint16), _c(B, np.uint16)
    if ms is None:
        n = M * N
        msa = nsa = None
    else:
        msa, nsa = _c(ms, np.int64), _c(ns, np.int64)
        if msa.shape != nsa.shape:
            raise ValueError("ms and ns differ in length")
        n = msa.size
    y = np.empty(n, dtype=np.float64)
    nu = np.empty(n, dtype=np.float64)
    rc = L.oracle_swiglu_pairs(_p(x), _p(W), _p(S), _p(B), _p(W), _p(S), _p(B), M, H, N, bits, gs, bits, gs, 1,
                               n, _p(msa), _p(nsa), _p(y), None, _p(nu), None, None, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return y, nu


def mlp_pairs(prob, Wd, Sd, Bd, bits_d, gs_d, Ho, residual=None, ms=None, ns=None, nthreads=0):
    """The whole MLP ``y = residual + hidden Wd^T`` at the elements (ms[p],
    ns[p]) of ``[M, Ho]`` (every element, row-major, when None), as the pages'
    fused MLP defines it ("mlx-bun 0.0.7 -> 0.0.9" diff, page 42,
    fused-mlp-kernel.ts: SwiGLU of the tile, then its down projection; the
    residual of minicpm5.ts's LlamaMLP.forward, page 41, added to the result).
    ``hidden`` is the forward in MATCH rounded to bf16 (the activation type),
    computed for every row that is asked for; the down projection is the
    float64 sum over the exactly dequantized ``Wd`` [Ho, I].  Returns
    (y, nu, rows, hidden_bits): nu = sqrt(sum_i (hidden_i wd_i)^2), rows the
    distinct rows evaluated and hidden_bits their bf16 hidden rows."""
    M, I = prob.M, prob.I
    if ms is None:
        ms = np.repeat(np.arange(M, dtype=np.int64), Ho)
        ns = np.tile(np.arange(Ho, dtype=np.int64), M)
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    rows = np.unique(ms)
    hm = np.repeat(rows, I)
    hn = np.tile(np.arange(I, dtype=np.int64), rows.size)
    h = swiglu_pairs(prob, MATCH, hm, hn, nthreads=nthreads, want=("h",))["h"]
    hidden_bits = bf16_rne(h).reshape(rows.size, I)
    local = np.searchsorted(rows, ms)
    y, nu = qmm_pairs(hidden_bits, Wd, Sd, Bd, rows.size, I, Ho, bits_d, gs_d, local, ns, nthreads=nthreads)
    if residual is not None:
        y = y + bf16_value(np.asarray(residual, dtype=np.uint16)[ms, ns])
    return y, nu, rows, hidden_bits


def unpack(W, rows, H, bits):
    """All codes of a packed ``[rows, H]`` matrix as uint8."""
    L = lib()
    W = _c(W, np.uint32)
    out = np.empty((rows, H), dtype=np.uint8)
    if L.oracle_unpack(_p(W), rows, H, bits, _p(out)) != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def bf16_rne(v):
    """float64 array -> bf16 bit patterns (uint16), rounded from the double."""
    L = lib()
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    L.oracle_bf16_rne_array(_p(v), v.size, _p(out))
    return out


def bf16_value(bits):
    """bf16 bit patterns -> float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_rne(v):
    """float64 array -> IEEE binary16 bit patterns (uint16), rounded from the double."""
    L = lib()
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    L.oracle_f16_rne_array(_p(v), v.size, _p(out))
    return out


def f16_value(bits):
    """IEEE binary16 bit patterns -> float64 (the C oracle's decoder)."""
    L = lib()
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    L.oracle_f16_value_array(_p(b), b.size, _p(out))
    return out


def silu(v):
    L = lib()
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    L.oracle_silu_array(_p(v), v.size, _p(out))
    return out
