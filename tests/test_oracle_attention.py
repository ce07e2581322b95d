"""Oracle pins: fp64 decode attention and the H2O mass.

Pinned against a scalar math.fsum evaluation, torch's scaled_dot_product_attention
in float64 (GQA via enable_gqa, which maps query head h to KV head h // G),
closed forms of softmax attention, and invariance under a shuffle of physical blocks.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention, paging, policies


def _scalar_attention(q, K, V, scale, keep):
    """Independent scalar evaluation with exactly summed dot products."""
    hq, d = q.shape
    L, hkv, _ = K.shape
    g = hq // hkv
    out = np.zeros((hq, d))
    for h in range(hq):
        kv = h // g
        z = [scale * math.fsum(q[h, i] * K[p, kv, i] for i in range(d)) if keep[p] else None for p in range(L)]
        m = max(x for x in z if x is not None)
        w = [math.exp(x - m) if x is not None else 0.0 for x in z]
        lam = math.fsum(w)
        for i in range(d):
            out[h, i] = math.fsum(w[p] * V[p, kv, i] for p in range(L)) / lam
    return out


def _tiny_paged(rng, lens=(35, 70), hq=8, hkv=2, d=64, nb=16, tables=None):
    pools = paging.new_pools(nb, hkv, d, "f32", fill=np.nan)
    if tables is None:
        perm = rng.permutation(nb)
        tables, at = [], 0
        for L in lens:
            n = -(-L // 16)
            tables.append(list(perm[at:at + n]))
            at += n
    srcs = []
    for s, L in enumerate(lens):
        k = rng.standard_normal((L, hkv, d)).astype(np.float32)
        v = rng.standard_normal((L, hkv, d)).astype(np.float32)
        paging.write_tokens(pools, "f32", k, v, "f32", tables, [s] * L, list(range(L)))
        srcs.append((k.astype(np.float64), v.astype(np.float64)))
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32).astype(np.float64)
    return pools, tables, srcs, q


@pytest.mark.parametrize("layout", ["seeded", "page"])
def test_paged_matches_scalar_fsum(layout):
    rng = np.random.default_rng(2831)
    tables = [[7, 12, 3], [8, 1, 2, 0, 9]] if layout == "page" else None
    pools, tables, srcs, q = _tiny_paged(rng, tables=tables)
    for s, L in enumerate((35, 70)):
        out, probs = attention.paged_decode(pools, "f32", q[s], tables[s], L, 1 / 8)
        ref = _scalar_attention(q[s], *srcs[s], 1 / 8, np.ones(L, bool))
        assert np.max(np.abs(out - ref)) <= 1e-13


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (32, 8), (8, 1)])
def test_matches_torch_sdpa_fp64(hq, hkv):
    rng = np.random.default_rng(hq * 100 + hkv)
    L, d = 300, 128
    q = rng.standard_normal((hq, d))
    K = rng.standard_normal((L, hkv, d))
    V = rng.standard_normal((L, hkv, d))
    out, _ = attention.decode_attention(q, K, V, 1 / math.sqrt(d))
    tq = torch.from_numpy(q)[None, :, None, :]                    # [1, Hq, 1, D]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()  # [1, Hkv, L, D]
    tv = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    ref = F.scaled_dot_product_attention(tq, tk, tv, scale=1 / math.sqrt(d), enable_gqa=hq != hkv)
    assert np.max(np.abs(out - ref[0, :, 0, :].numpy())) <= 1e-12


def test_streaming_subset_matches_sdpa_with_mask():
    rng = np.random.default_rng(4)
    L, hq, hkv, d = 200, 8, 2, 64
    q = rng.standard_normal((hq, d))
    K = rng.standard_normal((L, hkv, d))
    V = rng.standard_normal((L, hkv, d))
    keep = policies.streaming_keep(L, 4, 37)
    out, probs = attention.decode_attention(q, K, V, 0.125, keep)
    tq = torch.from_numpy(q)[None, :, None, :]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None].contiguous()
    tv = torch.from_numpy(V).permute(1, 0, 2)[None].contiguous()
    mask = torch.from_numpy(keep)[None, None, None, :]
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.125, enable_gqa=True)
    assert np.max(np.abs(out - ref[0, :, 0, :].numpy())) <= 1e-12
    assert np.all(probs[:, ~keep] == 0)


def test_closed_forms():
    rng = np.random.default_rng(9)
    hq, hkv, d = 8, 2, 16
    q = rng.standard_normal((hq, d))
    V = rng.standard_normal((5, hkv, d))
    # a single key: the output is that key's value vector, for every head of its group
    out, probs = attention.decode_attention(q, rng.standard_normal((1, hkv, d)), V[:1], 0.3)
    for h in range(hq):
        assert np.array_equal(out[h], V[0, h // 4])
    assert np.all(probs == 1.0)
    # identical keys: uniform weights, output = mean of the values
    K = np.repeat(rng.standard_normal((1, hkv, d)), 5, axis=0)
    out, probs = attention.decode_attention(q, K, V, 0.3)
    for h in range(hq):
        assert np.allclose(out[h], V[:, h // 4].mean(0), rtol=0, atol=1e-15)
    # a convex combination stays inside the per-dimension range of the values
    K = rng.standard_normal((5, hkv, d)) * 3
    out, _ = attention.decode_attention(q, K, V, 1.0)
    for h in range(hq):
        assert np.all(out[h] <= V[:, h // 4].max(0) + 1e-15) and np.all(out[h] >= V[:, h // 4].min(0) - 1e-15)


def test_group_mapping_is_contiguous():
    """Query head h reads KV head h // G: give each KV head a distinct constant value."""
    hq, hkv, d, L = 8, 2, 4, 3
    V = np.zeros((L, hkv, d))
    V[:, 1, :] = 1.0
    out, _ = attention.decode_attention(np.ones((hq, d)), np.zeros((L, hkv, d)), V, 1.0)
    assert np.array_equal(out[:, 0], [0, 0, 0, 0, 1, 1, 1, 1])


def test_block_permutation_invariance():
    rng = np.random.default_rng(12)
    pools, tables, srcs, q = _tiny_paged(rng)
    perm = rng.permutation(16)                      # physical block b moves to perm[b]
    moved = tuple(None if a is None else np.empty_like(a) for a in pools)
    for a, m in zip(pools, moved):
        if a is not None:
            m[perm] = a
    mtables = [[int(perm[b]) for b in t] for t in tables]
    for s, L in enumerate((35, 70)):
        a, pa = attention.paged_decode(pools, "f32", q[s], tables[s], L, 0.125)
        b, pb = attention.paged_decode(moved, "f32", q[s], mtables[s], L, 0.125)
        assert np.array_equal(a, b) and np.array_equal(pa, pb)


def test_mass_is_a_distribution_and_matches_torch_softmax():
    rng = np.random.default_rng(21)
    hq, hkv, d, L = 32, 8, 128, 500
    q = rng.standard_normal((hq, d))
    K = rng.standard_normal((L, hkv, d))
    V = rng.standard_normal((L, hkv, d))
    _, probs = attention.decode_attention(q, K, V, 1 / math.sqrt(d))
    mass = attention.head_mean_mass(probs)
    assert np.all(mass >= 0) and abs(mass.sum() - 1) <= 1e-12
    tk = torch.from_numpy(K).repeat_interleave(hq // hkv, dim=1)  # [L, Hq, D]
    logits = torch.einsum("hd,lhd->hl", torch.from_numpy(q), tk) / math.sqrt(d)
    ref = torch.softmax(logits, dim=-1).mean(0).numpy()
    assert np.max(np.abs(mass - ref)) <= 1e-15 * L


def test_unmapped_read_raises_but_dropped_blocks_are_not_read():
    rng = np.random.default_rng(1)
    pools = paging.new_pools(8, 1, 16, "f32", fill=np.nan)
    L, S, W = 100, 4, 20
    table = [-1] * 7
    table[0], table[5], table[6] = 3, 4, 5                    # blocks {0} and {5, 6} hold the keep-set
    keep_pos = np.nonzero(policies.streaming_keep(L, S, W))[0]
    k = rng.standard_normal((len(keep_pos), 1, 16)).astype(np.float32)
    paging.write_tokens(pools, "f32", k, k, "f32", [table], [0] * len(keep_pos), keep_pos.tolist())
    out, probs = attention.paged_decode(pools, "f32", rng.standard_normal((2, 16)), table, L, 0.3, S, W)
    assert np.all(np.isfinite(out)) and np.all(probs[:, ~policies.streaming_keep(L, S, W)] == 0)
    with pytest.raises(IndexError):
        attention.paged_decode(pools, "f32", rng.standard_normal((2, 16)), table, L, 0.3)


# ---------------------------------------------------------------------------- multi-query (chunked prefill)

def test_prefill_single_query_is_decode():
    rng = np.random.default_rng(11)
    K, V = rng.standard_normal((40, 2, 16)), rng.standard_normal((40, 2, 16))
    q = rng.standard_normal((1, 8, 16))
    out = attention.prefill_attention(q, K, V, 0.25)
    ref, _ = attention.decode_attention(q[0], K, V, 0.25)
    assert np.array_equal(out[0], ref)


@pytest.mark.parametrize("prefix,n_q,hq,hkv", [(0, 37, 8, 2), (50, 20, 4, 4), (100, 1, 8, 1), (3, 64, 16, 2)])
def test_prefill_matches_torch_sdpa_with_bottom_right_causal_mask(prefix, n_q, hq, hkv):
    """torch SDPA in float64 with the causal mask aligned to the end of the context (query i at
    position prefix + i sees keys 0..prefix + i); prefix 0 is SDPA's own is_causal."""
    rng = np.random.default_rng(prefix + n_q)
    L, d = prefix + n_q, 32
    K, V = rng.standard_normal((L, hkv, d)), rng.standard_normal((L, hkv, d))
    q = rng.standard_normal((n_q, hq, d))
    out = attention.prefill_attention(q, K, V, 1 / math.sqrt(d))
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]            # [1, Hq, n_q, D]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None]
    tv = torch.from_numpy(V).permute(1, 0, 2)[None]
    mask = torch.arange(L)[None, :] <= (prefix + torch.arange(n_q))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=True)
    assert np.max(np.abs(out - ref[0].permute(1, 0, 2).numpy())) <= 1e-12
    if prefix == 0:
        ref2 = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
        assert np.max(np.abs(out - ref2[0].permute(1, 0, 2).numpy())) <= 1e-12


def test_prefill_scalar_fsum_and_paging():
    """Tiny case by scalar math.fsum, and the paged version through a shuffled table is identical."""
    rng = np.random.default_rng(12)
    L, n_q, hq, hkv, d = 21, 5, 4, 2, 16
    K, V = rng.standard_normal((L, hkv, d)), rng.standard_normal((L, hkv, d))
    q = rng.standard_normal((n_q, hq, d))
    out = attention.prefill_attention(q, K, V, 0.3)
    for i in range(n_q):
        keep = np.arange(L) <= L - n_q + i
        ref = _scalar_attention(q[i], K, V, 0.3, keep)
        assert np.max(np.abs(out[i] - ref)) <= 1e-13
    pools = paging.new_pools(6, hkv, d, "f32", fill=np.nan)
    table = [4, 1]
    paging.write_tokens(pools, "f32", K.astype(np.float32), V.astype(np.float32), "f32", [table], [0] * L,
                        list(range(L)))
    got = attention.paged_prefill(pools, "f32", q, table, L, 0.3)
    exp = attention.prefill_attention(q, K.astype(np.float32).astype(np.float64),
                                      V.astype(np.float32).astype(np.float64), 0.3)
    assert np.array_equal(got, exp)
    with pytest.raises(ValueError):
        attention.prefill_attention(q, K[:3], V[:3], 0.3)
