"""Storage-format emulation: bfloat16 and OCP fp8 e4m3, written from the formats.

The published K/V pages hold bf16 (the pages' "BF16" backend, thelatestinai.com
listing, Table 1 and Table 5). The quantised path stores Q and K as fp8 with
scales (the pages name an FP8 K/V payload "and scale", Table 8, and a
SageAttention backend, Tables 1, 5 and 6). The e4m3 format used here is the OCP
8-bit float: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities,
largest finite 448, smallest normal 2^-6, subnormal step 2^-9, and all-ones
exponent+mantissa is NaN. Encoding rounds to nearest, ties to even, and
saturates at +-448.
"""
from __future__ import annotations

import numpy as np

FP8_E4M3_MAX = 448.0
BF16_MAX = float.fromhex("0x1.fep127")


def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value of fp64 input, ties to even (returned as fp64)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, E = np.frexp(a)                           # a = f * 2^E, 0.5 <= f < 1
    E = np.maximum(E, -125)                      # below 2^-126 the spacing is fixed
    ulp = np.ldexp(1.0, (E - 8).astype(np.int64))  # 8 significant bits
    r = np.rint(a / ulp) * ulp                   # rint: half to even
    r = np.where(r > BF16_MAX, np.inf, r)
    r = np.where(a == 0, 0.0, r)
    return np.copysign(r, x)


def fp8_e4m3_decode(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 0xF
    m = code & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7)))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


_MAGS = fp8_e4m3_decode(np.arange(0x7F))        # the 127 finite non-negative values, ascending


def fp8_e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of fp64 input, ties to the even code, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP8_E4M3_MAX)
    hi = np.clip(np.searchsorted(_MAGS, a, side="left"), 1, 0x7E)
    lo = hi - 1
    dlo = a - _MAGS[lo]
    dhi = _MAGS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == 0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def fp8_block_quantize(x: np.ndarray, block: int = 64):
    """Quantise x[N, d] (one chunk, one head) in blocks of `block` tokens.

    Each block gets the fp32 scale absmax/448 (1 for an all-zero block); codes
    are the e4m3 encoding of x / scale. Returns (codes uint8 [N, d],
    scales float32 [ceil(N/block)]).
    """
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[0]
    nb = (N + block - 1) // block
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.ones(nb, dtype=np.float32)
    for b in range(nb):
        blk = x[b * block:(b + 1) * block]
        amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
        s = np.float32(amax) / np.float32(FP8_E4M3_MAX) if amax > 0 else np.float32(1.0)
        scales[b] = s
        codes[b * block:(b + 1) * block] = fp8_e4m3_encode(blk / np.float64(s))
    return codes, scales
