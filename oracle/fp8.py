"""FP8 E4M3FN decoding and 128x128 block dequantisation (oracle side).

TEST INFRASTRUCTURE ONLY (see :mod:`oracle`).

[EcoSpec, Fig. 1(c)]: the DeepSeek-V3.1 experts are stored in FP8, one routed
expert being 7168 x 2048 x 3 bytes.  The pages do not name the FP8 encoding;
the reading here is the OCP 8-bit floating point E4M3 format ("FN": finite,
no infinities), the FP8 format of the gfx950 matrix cores, with one fp32 scale
per 128 x 128 block of each [out, in] weight matrix:  w = decode(q) * s.

E4M3FN, from the OCP FP8 specification: 1 sign bit, 4 exponent bits (bias 7),
3 mantissa bits.  Exponent field 0 encodes subnormals m * 2^-9; all other
fields encode (1 + m/8) * 2^(e-7), except S.1111.111 which is NaN.  There are
no infinities; the largest finite magnitude is 448.
"""

from __future__ import annotations

import math

import numpy as np


def decode_e4m3fn(code: int) -> float:
    """Value of one E4M3FN byte, straight from the format definition."""
    code = int(code) & 0xFF
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def decode_table() -> np.ndarray:
    """fp64 values of all 256 codes."""
    return np.array([decode_e4m3fn(c) for c in range(256)], dtype=np.float64)


_TABLE = None


def dequant_blocks(codes, scales, block: int = 128) -> np.ndarray:
    """w[o, i] = decode(codes[o, i]) * scales[o // block, i // block] in fp64."""
    global _TABLE
    if _TABLE is None:
        _TABLE = decode_table()
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float64)
    vals = _TABLE[codes]
    s = np.repeat(np.repeat(scales, block, axis=0), block, axis=1)
    return vals * s[: codes.shape[0], : codes.shape[1]]


def fp8_expert_fn(q13, s13, q2, s2, block: int = 128):
    """Expert accessor for fp8 weights q13[E,2,I,H] (+ s13[E,2,I/b,H/b]) and
    q2[E,H,I] (+ s2[E,H/b,I/b]); returns exact fp64 (Wg, Wu, Wd)."""
    def fn(e):
        return (dequant_blocks(q13[e][0], s13[e][0], block),
                dequant_blocks(q13[e][1], s13[e][1], block),
                dequant_blocks(q2[e], s2[e], block))
    return fn
