"""INT8 KV-cache codec (oracle; test infrastructure only).

[PA] = page "KV Cache 与 PagedAttention：显存复用与长上下文推理" (plumephp.com/ai-kv-cache-paged-attention),
       block "量化原理": FP16 -> INT8 halves KV memory (2 bytes -> 1 byte) and is the
       common choice; scaling is per channel or per token; "收益评估": 32K tokens
       x 80 layers go from about 10 GiB in FP16 to about 5 GiB in INT8.

Readings taken where the page gives only the names:
  * symmetric per-token scaling, one scale per (token, KV head) for K and one
    for V, as for FP8: scale = float32(absmax) / float32(127) (IEEE single
    precision division);
  * code = round(x / scale) with the quotient formed in single precision,
    rounded to the nearest integer with ties to even, saturated to [-127, 127]
    (the code -128 is never produced, so the range is symmetric);
  * a row whose scale is zero stores scale 0 and all-zero codes;
  * codes are stored as two's-complement int8.
"""

import numpy as np

INT8_MAX = 127.0


def decode(codes: np.ndarray) -> np.ndarray:
    """Exact float64 value of int8 codes (without their scale)."""
    return np.asarray(codes).astype(np.int8).astype(np.float64)


def encode(q: np.ndarray) -> np.ndarray:
    """float32 quotients -> int8 codes: nearest integer, ties to even, saturated to +-127."""
    r = np.rint(np.asarray(q, dtype=np.float64))          # numpy rint rounds half to even
    return np.clip(r, -INT8_MAX, INT8_MAX).astype(np.int8)


def quantize_per_token(x: np.ndarray):
    """Quantise the last axis of x with one fp32 scale per row.

    Returns (codes int8 same shape as x, scales float32 shape x.shape[:-1]).
    Input values must be finite.
    """
    x32 = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x32), axis=-1)
    scale = (absmax / np.float32(INT8_MAX)).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    q = (x32 / safe[..., None]).astype(np.float32)
    codes = encode(q)
    codes = np.where((scale == 0)[..., None], np.int8(0), codes).astype(np.int8)
    return codes, scale


def dequantize_per_token(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [..., D] int8 and scales [...] float32 -> float64 values (exact products)."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def quantize_per_channel(x: np.ndarray, channel_scale: np.ndarray) -> np.ndarray:
    """Codes of x [..., Hkv, D] with static scales [Hkv, D]: encode(float32(x / scale)), the quotient
    an IEEE single-precision division (values beyond the code range saturate to +-127)."""
    q = (np.asarray(x, dtype=np.float32) / np.asarray(channel_scale, dtype=np.float32)).astype(np.float32)
    return encode(q)
