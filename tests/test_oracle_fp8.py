"""Oracle pins: E4M3FN codec against the OCP format definition and torch's float8 cast."""
import numpy as np
import pytest
import torch

from oracle import fp8


def test_decode_table_spec_values():
    t = fp8.decode_table()
    assert t[0x7E] == 448.0
    assert t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x07] == 7 / 8 * 2.0 ** -6  # largest subnormal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x38] == 1.0
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254


def test_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(ref[~both_nan], ours[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(ours))


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(codes)), codes)


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_below_saturation():
    rng = np.random.default_rng(7)
    vals = fp8.decode_table()
    fin = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    mids = (fin[1:] + fin[:-1]) / 2                       # exact ties -> must go to even code
    nudged = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                             np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    x = np.concatenate([
        rng.standard_normal(20000) * 50,
        rng.standard_normal(5000) * 1e-3,                 # subnormal region
        mids, -mids, nudged, -nudged, fin, -fin,
        [2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11, 460.0, -463.9],
    ]).astype(np.float32)
    x = x[np.abs(x) < 464]
    assert np.array_equal(fp8.encode(x), _torch_codes(x))


def test_saturation_not_nan():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -464.0, -np.inf], dtype=np.float32)
    assert fp8.encode(x).tolist() == [0x7E] * 6 + [0xFE] * 2
    assert fp8.encode(np.array([np.nan])).tolist() == [0x7F]


def test_quantize_per_token_scale_rule():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 8, 128)) * rng.uniform(0.01, 100, (64, 8, 1))).astype(np.float32)
    x[3, 2] = 0.0
    codes, scale = fp8.quantize_per_token(x)
    absmax = np.abs(x).max(-1)
    assert scale.dtype == np.float32
    assert np.array_equal(scale, (absmax / np.float32(448)).astype(np.float32))
    assert scale[3, 2] == 0 and not codes[3, 2].any()
    # the largest element of every nonzero row lands on +-448
    am = np.abs(x).argmax(-1)
    top = np.take_along_axis(codes, am[..., None], -1)[..., 0]
    nz = absmax > 0
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # dequantised error: half a step of the 3-bit mantissa, or half the subnormal step
    deq = fp8.dequantize_per_token(codes, scale)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale[..., None].astype(np.float64) * 2.0 ** -10) * (1 + 1e-5)
    assert np.all(np.abs(deq - x) <= bound)
