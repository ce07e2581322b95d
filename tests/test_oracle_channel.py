"""Pins of the per-channel KV codecs (fp8_ch, int8_ch): codes scaled by one static scale per
(KV head, channel) instead of one per token (page PA, block 量化原理, which names per-channel
and per-token scaling as the common choices).  Power-of-two scales make every division exact, so
representable values survive the paged round trip bit for bit at every (head, channel): a scale
applied to the wrong head or channel, or a transposed scale array, fails these."""
import numpy as np
import pytest

from oracle import attention, fp8, int8, paging, policies

HKV, D = 2, 64


def _pow2_scales(seed):
    """Distinct power-of-two scales per (head, channel), 2^-6 .. 2^5."""
    rng = np.random.default_rng(seed)
    return (2.0 ** rng.integers(-6, 6, (HKV, D))).astype(np.float32)


def _representable(kv_dtype, rng, shape):
    """Values exactly representable in the code set (E4M3 finite values or integers in [-127, 127])."""
    if kv_dtype == "fp8_ch":
        table = fp8.decode_table()
        finite = table[np.isfinite(table)]
        return rng.choice(finite, shape)
    return rng.integers(-127, 128, shape).astype(np.float64)


@pytest.mark.parametrize("kv_dtype", ["fp8_ch", "int8_ch"])
def test_representable_values_roundtrip_exactly(kv_dtype):
    rng = np.random.default_rng(11)
    ks, vs = _pow2_scales(1), _pow2_scales(2)
    nb, L = 6, 40
    table = [4, 1, 3]
    pools = paging.new_pools(nb, HKV, D, kv_dtype, k_channel=ks, v_channel=vs)
    ck, cv = _representable(kv_dtype, rng, (L, HKV, D)), _representable(kv_dtype, rng, (L, HKV, D))
    k = (ck * ks).astype(np.float32)          # exact: a power-of-two multiple of a short mantissa
    v = (cv * vs).astype(np.float32)
    paging.write_tokens(pools, kv_dtype, k, v, "f32", [table], [0] * L, list(range(L)))
    K, V = paging.gather_logical(pools, kv_dtype, table, np.arange(L))
    assert np.array_equal(K, k.astype(np.float64)) and np.array_equal(V, v.astype(np.float64))
    # the stored codes are the code-set values themselves, K at chunk d // 16, row o, lane d % 16
    codec = fp8 if kv_dtype == "fp8_ch" else int8
    p, h, d = 21, 1, 37
    assert codec.decode(pools[0][table[p // 16], h, d // 16, p % 16, d % 16]) == ck[p, h, d]
    assert pools[2] is not None and np.array_equal(pools[2], ks) and np.array_equal(pools[3], vs)


def test_fp8_channel_error_bound_and_saturation():
    rng = np.random.default_rng(12)
    s = _pow2_scales(3)
    x = (rng.standard_normal((300, HKV, D)) * s * 40).astype(np.float32)
    x[0, 0, 0] = 1000.0 * s[0, 0]                       # beyond 448 * s: saturates
    x[0, 1, 5] = -449.0 * s[1, 5]
    codes = fp8.quantize_per_channel(x, s)
    deq = fp8.decode(codes) * s
    assert deq[0, 0, 0] == 448.0 * s[0, 0] and deq[0, 1, 5] == -448.0 * s[1, 5]
    inside = np.abs(x / s) <= 448
    # E4M3 has 3 mantissa bits: relative error <= 2^-4 for normal quotients (>= 2^-6),
    # absolute error <= 2^-10 (half the subnormal step) times the scale below that
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10)
    assert np.all(err[inside] <= bound[inside])
    assert not np.any(np.isnan(deq))


def test_int8_channel_error_bound_and_saturation():
    rng = np.random.default_rng(13)
    s = _pow2_scales(4)
    x = (rng.standard_normal((300, HKV, D)) * s * 50).astype(np.float32)
    x[1, 0, 3] = 300.0 * s[0, 3]
    x[2, 1, 63] = -127.5 * s[1, 63]
    codes = int8.quantize_per_channel(x, s)
    assert codes[1, 0, 3] == 127 and codes[2, 1, 63] == -127
    assert codes.min() >= -127 and codes.max() <= 127
    deq = codes.astype(np.float64) * s
    inside = np.abs(x / s) <= 127
    assert np.all(np.abs(deq - x)[inside] <= (s * 0.5)[None].repeat(300, 0)[inside])
    # ties go to even: quotients k + 0.5 are exact with power-of-two scales
    half = (np.array([0.5, 1.5, 2.5, -0.5, -3.5], np.float32)[:, None, None] * s[None]).astype(np.float32)
    got = int8.quantize_per_channel(half, s)
    assert got[:, 0, 0].tolist() == [0, 2, 2, 0, -4]


def test_uniform_channel_scale_equals_per_token_codes():
    """A row quantised per token with scale absmax/448 gets the same codes as per-channel storage
    whose every channel scale equals that row's scale."""
    rng = np.random.default_rng(14)
    row = rng.standard_normal((1, 1, D)).astype(np.float32)
    codes, scale = fp8.quantize_per_token(row)
    s = np.full((1, D), scale[0, 0], np.float32)
    assert np.array_equal(fp8.quantize_per_channel(row, s), codes)


@pytest.mark.parametrize("kv_dtype", ["fp8_ch", "int8_ch"])
def test_copy_and_compact_move_codes_only(kv_dtype):
    """Block copy and eviction compaction move codes; the static channel scales stay as they are and
    attention over the compacted cache equals attention over the kept positions of the original."""
    rng = np.random.default_rng(15)
    nb, L = 24, 150
    ks, vs = _pow2_scales(5), _pow2_scales(6)
    perm = rng.permutation(nb)
    src_table = list(perm[:10])
    pools = paging.new_pools(nb, HKV, D, kv_dtype, k_channel=ks, v_channel=vs)
    k = (rng.standard_normal((L, HKV, D)) * ks * 30).astype(np.float32)
    v = (rng.standard_normal((L, HKV, D)) * vs * 30).astype(np.float32)
    paging.write_tokens(pools, kv_dtype, k, v, "f32", [src_table], [0] * L, list(range(L)))
    paging.copy_blocks(pools, [(src_table[2], perm[20])])
    assert np.array_equal(pools[0][perm[20]], pools[0][src_table[2]])
    assert np.array_equal(pools[2], ks) and np.array_equal(pools[3], vs)
    keep = policies.keep_select(rng.random(L), L, 4, 16, 20, "all")
    n = len(keep)
    dst_table = list(perm[10:10 + -(-n // 16)])
    K0, V0 = paging.gather_logical(pools, kv_dtype, src_table, keep)
    paging.compact(pools, kv_dtype, src_table, keep, dst_table)
    K1, V1 = paging.gather_logical(pools, kv_dtype, dst_table, np.arange(n))
    assert np.array_equal(K0, K1) and np.array_equal(V0, V1)
    assert np.array_equal(pools[2], ks) and np.array_equal(pools[3], vs)
    q = rng.standard_normal((4, D))
    out, _ = attention.paged_decode(pools, kv_dtype, q, dst_table, n, 0.125)
    ref, _ = attention.decode_attention(q, K0, V0, 0.125)
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_channel_pools_need_scales():
    with pytest.raises(ValueError):
        paging.new_pools(2, HKV, D, "int8_ch")
