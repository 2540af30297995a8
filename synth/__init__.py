"""Seeded synthetic inputs for the fused quantized SwiGLU expansion.

This module feeds both the CPU oracle and the HIP path, and holds none of the
method's arithmetic. It only

* draws random numbers with ``numpy.random.default_rng(seed)`` (PCG64),
* rounds float32 draws to bfloat16 with torch's CPU cast (round to nearest,
  ties to even), and
* packs integer codes into uint32 words in the storage layout of MLX-style
  affine quantization: codes run along K (the hidden dimension H), ``32/bits``
  codes per word, code ``j`` of a word in bits ``[bits*j, bits*j + bits)``
  (least significant first).  The packed row of output feature ``n`` is
  ``H*bits/32`` words; scales and biases are ``[I, H/gs]``.
  (Layout: "mlx-bun 0.0.8 -> 0.0.10" diff, page 41, fused-swiglu-kernel.ts,
  docstring of the host entry, and the packed-row byte count in the kernel
  source.  The in-word bit order is not printed on the pages; least
  significant first is the reading taken.)

bf16 values travel as ``uint16`` bit patterns, packed codes as ``uint32``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Config", "CONFIGS", "Problem", "make_problem", "make_custom",
    "to_bf16_bits", "bf16_bits_to_f32", "to_f16_bits", "f16_bits_to_f32", "pack_codes", "decode_xs",
]


def to_bf16_bits(a) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), torch's RNE CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(a) -> np.ndarray:
    """float32 array -> IEEE binary16 bit patterns (uint16), numpy's RNE cast."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def f16_bits_to_f32(b) -> np.ndarray:
    """binary16 bit patterns -> float32 (exact widening)."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes ``[rows, H]`` into uint32 words ``[rows, H*bits/32]``,
    codes running along K, least significant bits first within a word."""
    codes = np.asarray(codes)
    rows, H = codes.shape
    pf = 32 // bits
    if H % pf:
        raise ValueError(f"H={H} is not a multiple of {pf} codes per word")
    c = codes.astype(np.uint32).reshape(rows, H // pf, pf)
    shifts = np.arange(pf, dtype=np.uint32) * np.uint32(bits)
    return np.bitwise_or.reduce(c << shifts, axis=2).astype(np.uint32)


@dataclass(frozen=True)
class Config:
    """One synthetic workload: shapes, quantization specs and distributions."""
    name: str
    M: int
    H: int
    I: int
    bits_g: int
    gs_g: int
    bits_u: int
    gs_u: int
    seed: int
    x_sigma: float = 1.0
    s_lo: float = 0.005
    s_hi: float = 0.02
    # "factor": bias = -8 * scale * U[0.9, 1.1];  "half": bias = -2^(bits-1) * scale
    bias_mode: str = "factor"
    calls: int = 1            # decode workload: number of fresh-x calls
    describe: str = ""
    act: str = "bf16"         # activation type: "bf16" or "f16" (binary16 x, scales and biases)


CONFIGS = {
    0: Config("tiny_prefill", 6, 256, 768, 4, 64, 4, 64, seed=0,
              describe="tiny prefill M=6 H=256 I=768, 4-bit gs64 gate/up"),
    1: Config("decode_gemv", 1, 2048, 5632, 4, 64, 4, 64, seed=1, calls=1000,
              describe="decode GEMV M=1 H=2048 I=5632, 4-bit gs64, 1000 calls"),
    2: Config("mid_prefill", 512, 2048, 8192, 4, 64, 4, 64, seed=2,
              describe="mid prefill M=512 H=2048 I=8192, 4-bit gs64"),
    3: Config("large_prefill", 2048, 4096, 14336, 4, 64, 4, 64, seed=3,
              x_sigma=0.5, s_lo=0.002, s_hi=0.01,
              describe="large prefill M=2048 H=4096 I=14336, 4-bit gs64"),
    4: Config("mixed_long_prefill", 8192, 2560, 10240, 8, 32, 4, 64, seed=4,
              bias_mode="half",
              describe="mixed-quant prefill M=8192 H=2560 I=10240, "
                       "gate 8-bit gs32, up 4-bit gs64"),
}


@dataclass
class Problem:
    """Host copies of every input of one call (bf16 as uint16 bits)."""
    M: int
    H: int
    I: int
    bits_g: int
    gs_g: int
    bits_u: int
    gs_u: int
    x: np.ndarray            # uint16 [M, H]
    wg: np.ndarray           # uint32 [I, H*bits_g/32]
    sg: np.ndarray           # uint16 [I, H/gs_g]
    bg: np.ndarray           # uint16 [I, H/gs_g]
    wu: np.ndarray           # uint32 [I, H*bits_u/32]
    su: np.ndarray           # uint16 [I, H/gs_u]
    bu: np.ndarray           # uint16 [I, H/gs_u]
    codes_g: np.ndarray | None = None   # uint8 [I, H] (kept only on request)
    codes_u: np.ndarray | None = None
    xs: np.ndarray | None = None         # uint16 [calls, H] fresh decode inputs
    extra: dict = field(default_factory=dict)
    act: str = "bf16"                    # type of x, scales and biases: "bf16" or "f16" (binary16)

    def args(self):
        """Positional tuple in the order of the forward entry point."""
        return (self.x, self.wg, self.sg, self.bg, self.wu, self.su, self.bu)


_TO16 = {"bf16": (to_bf16_bits, bf16_bits_to_f32), "f16": (to_f16_bits, f16_bits_to_f32)}


def _draw_matrix(rng, I, H, bits, gs, s_lo, s_hi, bias_mode, act="bf16"):
    to16, from16 = _TO16[act]
    codes = rng.integers(0, 1 << bits, size=(I, H), dtype=np.uint8)
    s_bits = to16(rng.uniform(s_lo, s_hi, size=(I, H // gs)).astype(np.float32))
    s = from16(s_bits)
    if bias_mode == "factor":
        f = rng.uniform(0.9, 1.1, size=(I, H // gs)).astype(np.float32)
        b_bits = to16((np.float32(-8.0) * s * f).astype(np.float32))
    elif bias_mode == "half":
        b_bits = to16((np.float32(-(1 << (bits - 1))) * s).astype(np.float32))
    else:
        raise ValueError(bias_mode)
    return codes, pack_codes(codes, bits), s_bits, b_bits


def make_custom(M, H, I, bits_g=4, gs_g=64, bits_u=None, gs_u=None, seed=0,
                x_sigma=1.0, s_lo=0.005, s_hi=0.02, bias_mode="factor",
                calls=0, keep_codes=False, act="bf16") -> Problem:
    """Draw one problem. Order of draws: x, gate codes, gate scales, gate bias
    factors, up codes, up scales, up bias factors, then (if ``calls``) the
    ``[calls, H]`` fresh decode inputs.  ``act`` = "f16" rounds x, the scales
    and the biases to binary16 instead of bf16 (the same draws)."""
    bits_u = bits_g if bits_u is None else bits_u
    gs_u = gs_g if gs_u is None else gs_u
    to16 = _TO16[act][0]
    rng = np.random.default_rng(seed)
    x = to16((rng.standard_normal((M, H), dtype=np.float32) * np.float32(x_sigma)).astype(np.float32))
    cg, wg, sg, bg = _draw_matrix(rng, I, H, bits_g, gs_g, s_lo, s_hi, bias_mode, act)
    cu, wu, su, bu = _draw_matrix(rng, I, H, bits_u, gs_u, s_lo, s_hi, bias_mode, act)
    xs = None
    if calls:
        xs = to16((rng.standard_normal((calls, H), dtype=np.float32) * np.float32(x_sigma)).astype(np.float32))
    return Problem(M, H, I, bits_g, gs_g, bits_u, gs_u, x, wg, sg, bg, wu, su, bu,
                   codes_g=cg if keep_codes else None,
                   codes_u=cu if keep_codes else None, xs=xs, act=act)


def make_down(Ho, I, bits=4, gs=64, seed=0, s_lo=0.005, s_hi=0.02, bias_mode="factor"):
    """The down projection of a whole MLP: packed codes [Ho, I*bits/32], bf16
    scales and biases [Ho, I/gs] (bit patterns), drawn as the gate and up."""
    rng = np.random.default_rng(seed)
    _, w, s, b = _draw_matrix(rng, Ho, I, bits, gs, s_lo, s_hi, bias_mode)
    return w, s, b


def make_residual(M, Ho, seed=0, sigma=1.0) -> np.ndarray:
    """A bf16 residual stream [M, Ho] (bit patterns), N(0, sigma^2)."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits((rng.standard_normal((M, Ho), dtype=np.float32) * np.float32(sigma)).astype(np.float32))


def make_problem(cfg: int | Config, keep_codes=False, with_calls=True) -> Problem:
    """The synthetic problem of a named configuration (seed = its index)."""
    c = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    return make_custom(c.M, c.H, c.I, c.bits_g, c.gs_g, c.bits_u, c.gs_u,
                       seed=c.seed, x_sigma=c.x_sigma, s_lo=c.s_lo, s_hi=c.s_hi,
                       bias_mode=c.bias_mode,
                       calls=(c.calls if (with_calls and c.calls > 1) else 0),
                       keep_codes=keep_codes, act=c.act)


def decode_xs(cfg: int | Config) -> np.ndarray:
    """The fresh ``[calls, H]`` decode inputs of a configuration."""
    p = make_problem(cfg, with_calls=True)
    if p.xs is None:
        raise ValueError("configuration has no repeated decode calls")
    return p.xs
