"""Pins of the INT8 KV codec (oracle/int8.py): crafted rows with an exact scale of 1, the rounding
and saturation rules, the error bound, symmetry, and zero rows (page PA, block 量化原理)."""
import numpy as np
import torch

from oracle import int8, paging


def test_scale_one_rows_are_round_half_even():
    # absmax 127 -> scale = 127 / 127 = 1 exactly, so codes are the rounded values themselves
    vals = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, -126.5, 3.4999998, 3.5000002, 0.0, -0.0, -127.0],
                    dtype=np.float32)
    codes, scale = int8.quantize_per_token(vals[None])
    assert scale[0] == np.float32(1.0)
    assert codes[0].tolist() == [127, 0, 2, 2, 0, -2, 126, -126, 3, 4, 0, 0, -127]


def test_matches_torch_round_and_clamp():
    """torch.round is round-half-to-even on the same float32 quotient."""
    rng = np.random.default_rng(127)
    x = (rng.standard_normal((500, 128)) * rng.uniform(0.01, 50, (500, 1))).astype(np.float32)
    x[3] = 0.0
    x[7, :5] = [1e-30, -1e-30, 0, 0, 0]
    codes, scale = int8.quantize_per_token(x)
    t = torch.from_numpy(x)
    s = (t.abs().amax(dim=-1) / 127.0).to(torch.float32)
    safe = torch.where(s == 0, torch.ones_like(s), s)
    ref = torch.clamp(torch.round(t / safe[:, None]), -127, 127).to(torch.int8)
    ref[s == 0] = 0
    assert np.array_equal(scale, s.numpy())
    assert np.array_equal(codes, ref.numpy())


def test_error_bound_symmetry_and_range():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((300, 64)).astype(np.float32)
    codes, scale = int8.quantize_per_token(x)
    deq = int8.dequantize_per_token(codes, scale)
    # |x - code * scale| <= scale / 2, up to the single-precision rounding of the quotient
    assert np.all(np.abs(deq - x) <= scale[:, None].astype(np.float64) * (0.5 + 1e-6))
    assert codes.min() >= -127 and codes.max() <= 127
    assert np.all(np.abs(codes).max(axis=1) == 127)                     # the absmax element hits 127
    neg, nscale = int8.quantize_per_token(-x)
    assert np.array_equal(neg, -codes) and np.array_equal(nscale, scale)
    assert np.array_equal(int8.decode(np.arange(-128, 128, dtype=np.int8)), np.arange(-128, 128).astype(float))


def test_zero_row_and_paged_storage():
    codes, scale = int8.quantize_per_token(np.zeros((2, 16), np.float32))
    assert np.all(codes == 0) and np.all(scale == 0)
    pools = paging.new_pools(2, 1, 64, "int8")
    assert pools[0].dtype == np.int8 and pools[2].shape == (2, 1, 16)
    row = np.zeros((1, 1, 64), np.float32)
    row[0, 0, 9] = -127.0                                                    # scale exactly 1
    paging.write_tokens(pools, "int8", row, row, "f32", [[1]], [0], [6])
    assert np.argwhere(pools[0] == -127).tolist() == [[1, 0, 0, 6, 9]]          # K chunk 0, row 6, lane 9
    assert np.argwhere(pools[1] == -127).tolist() == [[1, 0, 0, 9, 1, 0, 2]]    # V chunk (0, 9, 1), (u 0, e 2)
    K, V = paging.gather_logical(pools, "int8", [1], [6])
    assert K[0, 0, 9] == -127.0 and V[0, 0, 9] == -127.0 and np.count_nonzero(K) == 1
