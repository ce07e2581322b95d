"""Oracle pins: block mapping, pool layout, token write and block copy.

The pages fix the mapping position -> physical block (worked examples in
tests/golden/page_numbers.json); the intra-block layout is a convention, pinned
here by bijectivity and by write-then-read round trips.
"""
import json
import os

import numpy as np
import pytest

from oracle import fp8, paging

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_pa_layout_example_slots():
    reqs = GOLD["pa_layout_example"]["requests"]
    first_last = {}
    for name, r in reqs.items():
        table = r["blocks"]
        n = r["tokens"]
        for p in range(n):
            assert paging.physical_block(table, p, 16) == table[p // 16]
        first_last[name] = (paging.slot(table, 0, 16), paging.slot(table, n - 1, 16))
    assert first_last == {"A": (112, 50), "B": (80, 89), "C": (128, 149)}


def test_lc_block_table_example():
    g = GOLD["lc_block_table_example"]
    for tok, blk in g["block_of_token"].items():
        assert paging.physical_block(g["table"], int(tok), 32) == blk


def test_unmapped_entry_raises():
    with pytest.raises(IndexError):
        paging.physical_block([3, -1], 20, 8)
    with pytest.raises(IndexError):
        paging.physical_block([3, 8], 20, 8)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "f16"])
def test_layout_is_a_bijection(kv_dtype):
    """Filling every slot of a pool with distinct raw values writes every pool element exactly once,
    at the index the documented layout formula gives."""
    nb, hkv, d = 2, 1, 64
    st = paging.storage_dtype(kv_dtype)
    pools = paging.new_pools(nb, hkv, d, kv_dtype)
    n = nb * 16
    vals = np.arange(1, n * hkv * d + 1).astype(st).reshape(n, hkv, d)     # <= 2048: exact in f16
    assert len(np.unique(vals)) == vals.size
    table = [1, 0]
    paging.write_tokens(pools, kv_dtype, vals, vals[::-1].copy(), kv_dtype, [table], [0] * n, list(range(n)))
    k, v = pools[0], pools[1]
    assert sorted(k.ravel().tolist()) == sorted(vals.ravel().tolist())
    assert sorted(v.ravel().tolist()) == sorted(vals.ravel().tolist())
    x, y = 16 // np.dtype(st).itemsize, 4 // np.dtype(st).itemsize
    assert k.shape == (nb, hkv, d // x, 16, x) and v.shape == (nb, hkv, d // (16 * y), 16, 4, y, 4)
    for p, h, i in [(0, 0, 0), (17, 0, 5), (31, 0, 63), (9, 0, 40), (22, 0, 17)]:
        b, o, t = table[p // 16], p % 16, i // 16
        assert k[b, h, i // x, o, i % x] == vals[p, h, i]                      # K: chunk i // X, row o
        assert v[b, h, t // y, i % 16, o // 4, t % y, o % 4] == vals[n - 1 - p, h, i]   # V chunk


def test_fp8_v_layout_single_element():
    """One non-zero V element per row quantises to the code of 448 (0x7E), found at the layout's index."""
    nb, hkv, d = 1, 2, 128
    for p, h, i in [(0, 0, 0), (5, 1, 77), (15, 0, 127), (10, 1, 33)]:
        pools = paging.new_pools(nb, hkv, d, "fp8")
        row = np.zeros((1, hkv, d), np.float32)
        row[0, h, i] = 3.0
        paging.write_tokens(pools, "fp8", row, row, "f32", [[0]], [0], [p])
        v = pools[1]
        hits = np.argwhere(v == 0x7E)
        t = i // 16
        assert hits.tolist() == [[0, h, t // 4, i % 16, p // 4, t % 4, p % 4]]
        assert np.argwhere(pools[0] == 0x7E).tolist() == [[0, h, i // 16, p, i % 16]]


def _src(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(dtype)


@pytest.mark.parametrize("kv_dtype,src_dtype", [("f32", "f32"), ("bf16", "bf16"), ("f16", "f16"),
                                                ("fp8", "bf16"), ("fp8", "f32"), ("fp8", "f16")])
def test_write_then_gather_roundtrip(kv_dtype, src_dtype):
    rng = np.random.default_rng(3)
    nb, hkv, d = 12, 2, 64
    lens = [35, 70]
    perm = rng.permutation(nb)
    tables = [list(perm[0:3]), list(perm[3:8])]
    pools = paging.new_pools(nb, hkv, d, kv_dtype)
    for s, L in enumerate(lens):
        k = _src(rng, (L, hkv, d), src_dtype)
        v = _src(rng, (L, hkv, d), src_dtype)
        paging.write_tokens(pools, kv_dtype, k, v, src_dtype, tables, [s] * L, list(range(L)))
        K, V = paging.gather_logical(pools, kv_dtype, tables[s], np.arange(L))
        kf, vf = paging.to_f64(k, src_dtype), paging.to_f64(v, src_dtype)
        if kv_dtype == "fp8":
            ck, sk = fp8.quantize_per_token(kf.astype(np.float32))
            cv, sv = fp8.quantize_per_token(vf.astype(np.float32))
            assert np.array_equal(K, fp8.dequantize_per_token(ck, sk))
            assert np.array_equal(V, fp8.dequantize_per_token(cv, sv))
            assert np.max(np.abs(K - kf)) < 0.1 * np.max(np.abs(kf))
        else:
            assert np.array_equal(K, kf) and np.array_equal(V, vf)


def test_bf16_storage_decode():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = paging.to_f64(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 0.0 and np.signbit(vals[3])
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127
    assert vals[5] == 2.0 ** -133


def test_copy_blocks_is_copy_on_write_data_half():
    rng = np.random.default_rng(5)
    pools = paging.new_pools(6, 2, 64, "fp8")
    for a in pools:
        a[...] = rng.integers(0, 120, a.shape).astype(a.dtype)
    before = [a.copy() for a in pools]
    paging.copy_blocks(pools, [(1, 4)])
    for a, b in zip(pools, before):
        assert np.array_equal(a[4], b[1])                       # copied bytes
        keep = [i for i in range(6) if i != 4]
        assert np.array_equal(a[keep], b[keep])                 # nothing else touched
    # a later write into the copy leaves the shared original alone
    k = np.ones((1, 2, 64), np.float32)
    paging.write_tokens(pools, "fp8", k, k, "f32", [[4]], [0], [3])
    assert np.array_equal(pools[0][1], before[0][1])
    assert not np.array_equal(pools[0][4], before[0][1])


@pytest.mark.parametrize("kv_dtype,src_dtype", [("f32", "f32"), ("bf16", "bf16"), ("fp8", "bf16")])
def test_compact_moves_kept_tokens_to_a_dense_prefix(kv_dtype, src_dtype):
    """After compaction, logical position i of the new table holds exactly what keep[i] held,
    no block outside the destination changes, and attention over the compacted cache equals
    attention over the original cache restricted to the kept positions."""
    from oracle import attention, policies
    rng = np.random.default_rng(7)
    nb, hkv, d, L = 24, 2, 64, 150
    perm = rng.permutation(nb)
    src_table = list(perm[:10])                       # 150 tokens in 10 blocks
    pools = paging.new_pools(nb, hkv, d, kv_dtype)
    for a in pools:
        if a is not None:
            a.view(np.uint8)[...] = rng.integers(0, 256, a.view(np.uint8).shape, dtype=np.uint8)
    k, v = _src(rng, (L, hkv, d), src_dtype), _src(rng, (L, hkv, d), src_dtype)
    paging.write_tokens(pools, kv_dtype, k, v, src_dtype, [src_table], [0] * L, list(range(L)))
    keep = policies.keep_select(rng.random(L), L, 4, 16, 20, "all")
    n = len(keep)
    dst_table = list(perm[10:10 + -(-n // 16)])
    before = [None if a is None else a.copy() for a in pools]
    K0, V0 = paging.gather_logical(pools, kv_dtype, src_table, keep)
    paging.compact(pools, kv_dtype, src_table, keep, dst_table)
    K1, V1 = paging.gather_logical(pools, kv_dtype, dst_table, np.arange(n))
    assert np.array_equal(K0, K1) and np.array_equal(V0, V1)
    others = [b for b in range(nb) if b not in dst_table]
    for a, b0 in zip(pools, before):
        if a is not None:
            assert np.array_equal(a[others].view(np.uint8), b0[others].view(np.uint8))   # bytes: NaN patterns too
    q = rng.standard_normal((4, d))
    out_c, _ = attention.paged_decode(pools, kv_dtype, q, dst_table, n, 0.125)
    Kf, Vf = paging.gather_logical(before, kv_dtype, src_table, np.arange(L))
    mask = np.zeros(L, bool)
    mask[keep] = True
    out_r, _ = attention.decode_attention(q, Kf, Vf, 0.125, keep=mask)
    assert np.array_equal(out_c, out_r)
