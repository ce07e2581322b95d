"""FP8 E4M3 KV-cache codec (oracle; test infrastructure only).

[PA] = page "KV Cache 与 PagedAttention：显存复用与长上下文推理" (plumephp.com/ai-kv-cache-paged-attention),
       block "量化原理": FP16 -> FP8 (E4M3) halves KV memory; scaling is per channel or per token.

The page names only "E4M3".  Reading taken: the OCP 8-bit floating point
format E4M3FN (bias 7, no infinities, S.1111.111 is NaN, largest finite 448),
the one whose range matches a per-token scale of absmax/448.

Encoding is written as a table search, not bit manipulation: a value maps
to the nearest finite E4M3FN value; of two equally near values the one with an even
code (mantissa LSB 0) wins; anything beyond 448 in magnitude maps to 448
(saturation -- no NaN is produced from a finite input).
"""

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def _code_value(code: int) -> float:
    """Value of one E4M3FN code, from the format definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:                       # subnormal: 0.mmm x 2^(1-7)
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def decode_table() -> np.ndarray:
    """float64[256]: the value of every byte code (NaN for 0x7F and 0xFF)."""
    return np.array([_code_value(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
_POS_VALUES = _TABLE[:0x7F]


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """Round float values to E4M3FN codes: nearest finite value, ties to even code, saturate.

    For each magnitude the two neighbouring finite values (below and above in
    the sorted table of the 127 non-negative finite values) are compared; the
    nearer one wins, an exact tie goes to the even code.  Magnitudes beyond
    448 (and infinity) become 448.  NaN maps to 0x7F.  The sign bit of the
    input is kept (-0.0 -> 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)                   # saturation: beyond 448 is 448
    mag = np.where(np.isnan(mag), 0.0, mag)
    hi = np.clip(np.searchsorted(_POS_VALUES, mag, side="left"), 0, 0x7E)   # first value >= mag
    lo = np.clip(hi - 1, 0, 0x7E)                                          # last value < mag
    d_hi = np.abs(_POS_VALUES[hi] - mag)
    d_lo = np.abs(mag - _POS_VALUES[lo])
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    code = pick.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(NAN_CODE), code).astype(np.uint8)


def quantize_per_token(x: np.ndarray):
    """Quantise the last axis of x (one token of one KV head per row) with one fp32 scale per row.

    scale = float32(absmax) / float32(448), an IEEE single-precision division;
    each element is divided by that scale in single precision and encoded.
    A row whose scale is zero (absmax 0, or a scale that underflows) stores
    scale 0 and all-zero codes.  Input values must be finite.
    Returns (codes uint8 same shape as x, scales float32 shape x.shape[:-1]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x32), axis=-1)
    scale = (absmax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    q = (x32 / safe[..., None]).astype(np.float32)
    codes = encode(q)
    codes = np.where((scale == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, scale


def dequantize_per_token(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [..., D] uint8 and scales [...] float32 -> float64 values (exact products)."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def quantize_per_channel(x: np.ndarray, channel_scale: np.ndarray) -> np.ndarray:
    """Codes of x [..., Hkv, D] with static scales [Hkv, D]: encode(float32(x / scale)), the quotient
    an IEEE single-precision division (values beyond the code range saturate to +-448)."""
    q = (np.asarray(x, dtype=np.float32) / np.asarray(channel_scale, dtype=np.float32)).astype(np.float32)
    return encode(q)
