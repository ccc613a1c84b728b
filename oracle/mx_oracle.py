"""Plain CPU oracle for MXFP8 K/V storage.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path; it
imports nothing from the product path.

The pages (page "SGLang and Miles Add Day-0 Support for Inkling", section
"Relative Logits Optimization", paragraph "MXFP8 Support") store K and V in
MXFP8: Q.K^T runs as an MXFP8 product, P.V stays in bf16 with V dequantised
on the fly, and the quantisation is fused into the attention prologue.  They
name the format and give no detail; MXFP8 is the OCP Microscaling (MX)
format, and this module writes out its published definition:

* element format E4M3 (the OCP 8-bit floating point "E4M3"): sign, 4
  exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
  subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so the largest
  magnitude is 1.75 * 2^8 = 448;
* blocks of 32 consecutive elements share one scale, an E8M0 byte e holding
  2^(e - 127) (255 is NaN);
* conversion of a block: shared exponent = floor(log2(max |x|)) - 8 (8 being
  the largest exponent of an E4M3 normal), clamped to [-127, 127]; each
  element is x / 2^shared rounded to E4M3 to nearest, ties to even, and
  clamped to +-448.

Readings (listed in the design notes): a block whose elements are all zero
gets the scale byte 127 (2^0); blocks run along the head dimension D (four
per 128-wide row); Q is quantised the same way (per (token, head) row) for
the MXFP8 product, and the dequantised values are exact in bf16 / fp32.

Parity status: ``e4m3_decode`` is pinned to torch's float8_e4m3fn (the same
OCP format, a library routine) over all 256 codes; ``e4m3_round`` to torch's
cast over a dense sweep of finite inputs in range; ``mx_quantize`` to closed
forms (blocks that are exact on the grid come back unchanged, the scale
puts the block maximum in [256, 512)) and to the element error bound.
"""

from __future__ import annotations

import math
from typing import Tuple

import torch

__all__ = ["E4M3_MAX", "MX_BLOCK", "e4m3_decode", "e4m3_round", "e4m3_encode", "mx_quantize", "mx_dequantize",
           "e8m0_value", "mx_round"]

E4M3_MAX = 448.0
MX_BLOCK = 32
_EMAX_ELEM = 8  # exponent of the largest E4M3 normal (1.75 * 2^8)


def e4m3_decode(code: int) -> float:
    """Value of one E4M3 byte (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_encode(v: float) -> int:
    """Nearest E4M3 byte to the finite value v (ties to even), magnitudes
    beyond 448 clamped to 448."""
    sign = 0x80 if (v < 0 or (v == 0 and math.copysign(1.0, v) < 0)) else 0
    a = abs(v)
    if a >= 2.0 ** -6:
        e = math.frexp(a)[1] - 1          # a = (1 + f) * 2^e
        q = round(a / 2.0 ** (e - 3))     # 8 .. 16, exact division, round() ties to even
        if q == 16:
            e, q = e + 1, 8
        if e > _EMAX_ELEM or (e == _EMAX_ELEM and q > 14):
            return sign | 0x7E
        return sign | ((e + 7) << 3) | (q - 8)
    m = round(a * 2.0 ** 9)               # subnormal quantum 2^-9; m == 8 is the smallest normal
    return sign | m


def e4m3_round(v: float) -> float:
    return e4m3_decode(e4m3_encode(v))


def e8m0_value(byte: int) -> float:
    return float("nan") if byte == 255 else 2.0 ** (byte - 127)


def mx_quantize(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP8 of x [..., D] (D a multiple of 32) along the last axis.

    Returns (codes uint8 [..., D], scales uint8 [..., D / 32]).  The
    arithmetic is exact: x is taken as float64 (every bf16 / fp32 value is
    exact there) and scaled by powers of two.
    """
    D = x.shape[-1]
    assert D % MX_BLOCK == 0
    flat = x.to(torch.float64).reshape(-1, D // MX_BLOCK, MX_BLOCK).tolist()
    codes, scales = [], []
    for row in flat:
        crow, srow = [], []
        for blk in row:
            amax = max(abs(t) for t in blk)
            if amax == 0.0:
                shared = 0
            else:
                shared = min(max(math.frexp(amax)[1] - 1 - _EMAX_ELEM, -127), 127)
            srow.append(shared + 127)
            crow.extend(e4m3_encode(t / 2.0 ** shared) for t in blk)
        codes.append(crow)
        scales.append(srow)
    shape = tuple(x.shape)
    return (torch.tensor(codes, dtype=torch.uint8).reshape(shape),
            torch.tensor(scales, dtype=torch.uint8).reshape(shape[:-1] + (D // MX_BLOCK,)))


_DECODE_TABLE = torch.tensor([e4m3_decode(c) for c in range(256)], dtype=torch.float64)


def mx_dequantize(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """float64 values of MXFP8 codes [..., D] with scales [..., D / 32]."""
    vals = _DECODE_TABLE[codes.to(torch.int64)]
    sc = torch.tensor([e8m0_value(b) for b in range(256)], dtype=torch.float64)[scales.to(torch.int64)]
    return vals * sc.repeat_interleave(MX_BLOCK, dim=-1)


def mx_round(x: torch.Tensor) -> torch.Tensor:
    """x [..., D] through MXFP8 and back (float64): the values an MXFP8 K, V
    or Q row stands for.  Attention over an MXFP8 cache is the oracle's
    attention on these values (the MXFP8 product of Q and K is exact in its
    fp32 accumulation up to rounding order; V is dequantised exactly)."""
    codes, scales = mx_quantize(x)
    return mx_dequantize(codes, scales)
