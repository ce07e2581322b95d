"""GPU parity of every entry point against the CPU oracle, at sizes the oracle finishes in seconds.

Bars: slots, pool bytes, FP8 codes and H2O keep-sets bit-exact; attention
output within 2e-3 max-abs (f32/bf16/f16 KV) or 1e-2 (FP8 KV, oracle applying
the same dequantisation); H2O mass within 1e-4 relative.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention, fp8, paging, policies
from paged_kv_cache_283_amd import ops

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import _harness as H

TOL = {"f32": 2e-3, "bf16": 2e-3, "f16": 2e-3, "fp8": 1e-2, "int8": 1e-2, "fp8_ch": 1e-2, "int8_ch": 1e-2}
CODE8 = ("fp8", "int8", "fp8_ch", "int8_ch")


def _case_workload(kv, q, d, hq, hkv, seed, lens=(35, 70), **kw):
    src = "bf16" if kv in CODE8 else kv
    return dataclasses.replace(W.WORKLOADS["tiny"], name=f"t-{kv}-{q}-{d}", kv_dtype=kv, src_dtype=src, q_dtype=q,
                               head_dim=d, num_q_heads=hq, num_kv_heads=hkv, seed=seed, pool_blocks=None,
                               extra_blocks=3, lens=tuple(lens), num_seqs=len(lens), **kw)


def _max_err(case, out, **kw):
    err = 0.0
    for s in range(case.lay.lens.shape[0]):
        ref, _ = case.oracle(s, **kw)
        err = max(err, H.max_err(H.to_f64(out[s]), ref))
    return err


# ---------------------------------------------------------------------------- slots

def test_decode_and_token_slots_match_oracle():
    w = dataclasses.replace(W.WORKLOADS["llama3"], num_seqs=20, len_range=(1, 300))
    lay = W.make_layout(w)
    tables = torch.from_numpy(lay.tables).cuda()
    lens = torch.from_numpy(lay.lens).cuda()
    got = ops.paged_decode_slots(tables, lens, lay.num_blocks).cpu().numpy()
    ref = [paging.slot(lay.tables[s], int(lay.lens[s]) - 1, lay.num_blocks) for s in range(20)]
    assert got.tolist() == ref
    seq, pos, _ = lay.fill_tokens()
    got = ops.paged_token_slots(tables, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                                lay.num_blocks).cpu().numpy()
    ref = [paging.slot(lay.tables[s], int(p), lay.num_blocks) for s, p in zip(seq, pos)]
    assert got.tolist() == ref
    # unusable lengths, positions and table entries give -1
    bad_t = tables.clone()
    bad_t[0, 0] = -1
    bad_t[1, 0] = lay.num_blocks
    bad_l = lens.clone()
    bad_l[0] = 1
    bad_l[1] = 1
    bad_l[2] = 0
    bad_l[3] = lay.tables.shape[1] * 16 + 1
    got = ops.paged_decode_slots(bad_t, bad_l, lay.num_blocks).cpu().numpy()
    assert got[:4].tolist() == [-1, -1, -1, -1]
    got = ops.paged_token_slots(tables, torch.tensor([0, 25, -1, 0], dtype=torch.int32).cuda(),
                                torch.tensor([-1, 0, 0, 1 << 20], dtype=torch.int32).cuda(), lay.num_blocks)
    assert got.cpu().tolist() == [-1, -1, -1, -1]


# ---------------------------------------------------------------------------- write

@pytest.mark.parametrize("kv,src,d", [("f32", "f32", 64), ("bf16", "bf16", 128), ("f16", "f16", 128),
                                      ("fp8", "bf16", 128), ("fp8", "f32", 64), ("fp8", "f16", 128),
                                      ("int8", "bf16", 128), ("int8", "f32", 64), ("int8", "f16", 128),
                                      ("fp8_ch", "bf16", 128), ("fp8_ch", "f32", 64), ("int8_ch", "bf16", 128),
                                      ("int8_ch", "f16", 64), ("fp8", "bf16", 64), ("int8", "f16", 64)])
def test_write_pool_bytes_bit_exact(kv, src, d):
    w = dataclasses.replace(_case_workload(kv, "bf16", d, 8, 2, 91, lens=(35, 70, 16, 1)), src_dtype=src)
    case = H.Case(w)
    lay = case.lay
    # oracle pools: all bytes 0xFF, then the same tokens written by the oracle's own slot arithmetic
    kc, vc = H.channel_pair(w)
    ref = list(paging.new_pools(lay.num_blocks, 2, d, kv, k_channel=kc, v_channel=vc))
    for a in ref:
        if a is not None and a.ndim > 2:          # static channel scales keep their values
            a.view(np.uint8)[...] = 0xFF
    seq, pos, rows = lay.fill_tokens()
    ks = case.ksrc.cpu()[torch.from_numpy(rows)]
    vs = case.vsrc.cpu()[torch.from_numpy(rows)]
    conv = {"f32": lambda t: t.numpy(), "f16": lambda t: t.numpy(),
            "bf16": lambda t: t.view(torch.int16).numpy().view(np.uint16)}
    paging.write_tokens(ref, kv, conv[src](ks), conv[src](vs), src, lay.tables, seq, pos)
    for got, exp in zip(case.pools, ref):
        if exp is None:
            assert got is None
            continue
        g = got.cpu().contiguous().view(torch.uint8).numpy().reshape(-1)
        assert np.array_equal(g, exp.view(np.uint8).reshape(-1))



@pytest.mark.parametrize("kv,src", [("bf16", "bf16"), ("fp8", "bf16"), ("int8", "f16"), ("f32", "f32")])
def test_write_scattered_slots_bit_exact(kv, src):
    """An explicit slot list made of runs of consecutive slots in shuffled order (runs that start off a
    multiple of 4, quads split between workgroups, lone tokens), with skipped (-1) and out-of-range
    slots, stores exactly the bytes the oracle's write stores; every other byte stays untouched."""
    nb, hkv, d, t = 12, 2, 128, 160
    rng = np.random.default_rng(283)
    total = nb * 16
    runs = np.split(np.arange(total), np.sort(rng.choice(np.arange(1, total), 40, replace=False)))
    slots = np.concatenate([runs[i] for i in rng.permutation(len(runs))])[:t].astype(np.int64)
    skip = rng.choice(t, 10, replace=False)
    slots[skip[:5]] = -1
    slots[skip[5:]] = total + 3
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[src]
    ks = torch.from_numpy(rng.standard_normal((t, hkv, d)).astype(np.float32) * 3).to(tdt)
    vs = torch.from_numpy(rng.standard_normal((t, hkv, d)).astype(np.float32) * 3).to(tdt)
    got = ops.allocate_pools(nb, hkv, d, W.storage_dtype(kv), "cuda", fill_byte=0xFF)
    ops.paged_kv_write(ks.cuda(), vs.cuda(), got[0], got[1], torch.from_numpy(slots).cuda(), got[2], got[3])
    ref = list(paging.new_pools(nb, hkv, d, kv))
    for a in ref:
        if a is not None:
            a.view(np.uint8)[...] = 0xFF
    ok = (slots >= 0) & (slots < total)
    conv = {"f32": lambda x: x.numpy(), "f16": lambda x: x.numpy(),
            "bf16": lambda x: x.view(torch.int16).numpy().view(np.uint16)}
    table = np.arange(nb, dtype=np.int32)[None, :]
    paging.write_tokens(ref, kv, conv[src](ks[torch.from_numpy(ok)]), conv[src](vs[torch.from_numpy(ok)]), src,
                        table, np.zeros(int(ok.sum()), np.int32), slots[ok])
    for g, e in zip(got, ref):
        if e is None:
            assert g is None
            continue
        assert np.array_equal(g.cpu().contiguous().view(torch.uint8).numpy().reshape(-1), e.view(np.uint8).reshape(-1))

def test_fp8_encoder_on_crafted_values():
    """Rows whose absmax is 448 have scale exactly 1, so codes are the encoder applied to the values."""
    table = fp8.decode_table()
    fin = np.sort(table[np.isfinite(table) & (table >= 0)])
    mids = (fin[1:] + fin[:-1]) / 2
    vals = np.concatenate([fin, mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(500)),
                           [2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -12, 1e-30, -0.0, 447.99, 440.0, 2.0 ** -6 - 2.0 ** -12]])
    vals = vals.astype(np.float32)
    d = 128
    n = -(-vals.size // (d - 1))
    rows = np.zeros((n, d), np.float32)
    flat = np.zeros(n * (d - 1), np.float32)
    flat[: vals.size] = vals
    rows[:, 1:] = flat.reshape(n, d - 1)
    rows[:, 0] = 448.0
    k = torch.from_numpy(rows.reshape(n, 1, d)).cuda()
    nb = -(-n // 16)
    kp, vp, ks, vs = ops.allocate_pools(nb, 1, d, torch.uint8, "cuda", fill_byte=0xFF)
    ops.paged_kv_write(k, k, kp, vp, torch.arange(n, dtype=torch.int64).cuda(), ks, vs)
    assert torch.all(ks.view(-1)[:n] == 1.0)
    codes = H.k_token_rows(kp).view(nb * 16, d)[:n].cpu().numpy()
    assert np.array_equal(codes, fp8.encode(rows))
    vcodes = H.v_token_rows(vp).view(nb * 16, d)[:n].cpu().numpy()
    assert np.array_equal(vcodes, codes)


def test_fp8_zero_rows_and_skipped_slots():
    k = torch.zeros((3, 2, 64), dtype=torch.bfloat16, device="cuda")
    k[1, 1, 5] = -3.0
    kp, vp, ks, vs = ops.allocate_pools(2, 2, 64, torch.uint8, "cuda", fill_byte=0xFF)
    ops.paged_kv_write(k, k, kp, vp, torch.tensor([3, -1, 40], dtype=torch.int64).cuda(), ks, vs)
    # token 0 -> slot 3 (all zero: scale 0, codes 0); token 1 skipped (-1); token 2 out of the pool, skipped
    krows, vrows = H.k_token_rows(kp), H.v_token_rows(vp)           # [32 slots][2][64]
    assert torch.all(krows[3] == 0) and torch.all(vrows[3] == 0)
    assert torch.all(ks[0, :, 3] == 0) and torch.all(vs[0, :, 3] == 0)
    for rows in (krows, vrows):
        left = rows.clone()
        left[3] = 0xFF
        assert torch.all(left == 0xFF)
    for t in (ks.view(torch.uint8), vs.view(torch.uint8)):
        left = t.clone()
        left.view(2, 2, 16, 4)[0, :, 3] = 0xFF
        assert torch.all(left == 0xFF)


# ---------------------------------------------------------------------------- attention

GRID = [
    # kv, q, d, hq, hkv
    ("f32", "f32", 64, 8, 2),
    ("f32", "bf16", 128, 4, 4),
    ("bf16", "bf16", 128, 32, 8),
    ("bf16", "f32", 128, 8, 1),
    ("bf16", "bf16", 64, 16, 1),
    ("bf16", "f16", 128, 6, 3),
    ("f16", "f16", 128, 8, 4),
    ("f16", "f32", 64, 16, 8),
    ("fp8", "bf16", 128, 32, 8),
    ("fp8", "f32", 64, 8, 8),
    ("fp8", "f16", 128, 16, 2),
    ("int8", "bf16", 128, 32, 8),
    ("int8", "f32", 64, 8, 2),
    ("fp8_ch", "bf16", 128, 32, 8),
    ("fp8_ch", "f32", 64, 8, 2),
    ("int8_ch", "bf16", 128, 16, 2),
    ("int8_ch", "f16", 64, 8, 8),
]
LENS = (1, 15, 16, 17, 35, 70, 511, 512, 513, 1100, 2049)


@pytest.mark.parametrize("kv,q,d,hq,hkv", GRID)
def test_attention_matches_oracle(kv, q, d, hq, hkv):
    w = _case_workload(kv, q, d, hq, hkv, seed=hq * 131 + d + hkv, lens=LENS)
    case = H.Case(w)
    out = case.attend()
    err = _max_err(case, out)
    print(f"{kv}/{q} D={d} G={hq // hkv}: max abs err {err:.3e}")
    assert err <= TOL[kv]


@pytest.mark.parametrize("kv,qd", [("int8", "f32"), ("int8_ch", "f32"), ("int8", "bf16")])
@pytest.mark.parametrize("factor", [2e4, 1e-6])
def test_int8_queries_far_outside_f16_range(kv, qd, factor):
    """INT8 K enters QK as f16, so q is rescaled by a power of two into f16's range first: queries
    whose magnitudes would overflow f16 (2e4 x N(0, 1) reaches 9e4) or fall into its subnormals
    (1e-6) must still match the oracle (near one-hot and near uniform softmax respectively).  bf16
    queries take the path with one QK MFMA per step (no low half)."""
    w = _case_workload(kv, qd, 128, 32, 8, 61, lens=(700, 33, 1500))
    case = H.Case(w)
    q = (case.q.float() * factor).to(case.q.dtype).contiguous()
    out = case.attend(q=q)
    err = max(H.max_err(H.to_f64(out[s]), case.oracle(s, q=q)[0]) for s in range(3))
    print(f"{kv} q x {factor}: max abs err {err:.3e}")
    assert err <= TOL[kv]


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_low_precision_output(out_dtype):
    w = _case_workload("bf16", "bf16", 128, 32, 8, 5, lens=(700, 33))
    case = H.Case(w)
    o32 = case.attend(torch.float32)
    o16 = case.attend(out_dtype)
    assert torch.equal(o32.to(out_dtype), o16)        # same fp32 result, rounded once on store


@pytest.mark.parametrize("layout", ["seeded", "page"])
def test_tiny_workload(layout):
    w = W.WORKLOADS["tiny"]
    page = [[7, 12, 3], [8, 1, 2, 0, 9]] if layout == "page" else None
    case = H.Case(w, page_tables=page)
    err = _max_err(case, case.attend())
    assert err <= 2e-3
    # StreamingLLM sub-case: 4 sinks + window 8
    out = case.attend(num_sinks=4, window=8)
    assert _max_err(case, out, num_sinks=4, window=8) <= 2e-3


def test_scale_argument_is_used():
    w = _case_workload("bf16", "bf16", 128, 8, 2, 77, lens=(300, 40))
    case = H.Case(w)
    for sc in (0.02, 0.3):
        assert _max_err(case, case.attend(scale=sc), scale=sc) <= 2e-3


def test_physical_block_permutation_is_bit_identical():
    w = _case_workload("bf16", "bf16", 128, 32, 8, 12, lens=(1500, 37, 800))
    case = H.Case(w)
    out = case.attend()
    nb = case.lay.num_blocks
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(3)).cuda()
    moved = []
    for p in case.pools:
        if p is None:
            moved.append(None)
            continue
        m = torch.empty_like(p)
        m[perm] = p
        moved.append(m)
    tables = case.tables.clone()
    valid = tables >= 0
    tables[valid] = perm[tables[valid].long()].int()
    out2 = torch.empty_like(out)
    ops.paged_decode_attn(out2, case.q, moved[0], moved[1], tables, case.lens, case.lay.max_len)
    assert torch.equal(out, out2)


def test_streaming_unmapped_blocks_and_poison_never_read():
    """Table entries of dropped blocks are -1 and unkept slots of kept blocks are NaN."""
    L, S, Wn = 3000, 4, 700
    w = dataclasses.replace(_case_workload("bf16", "bf16", 128, 32, 8, 44, lens=(L, L - 5, 30)),
                            num_sinks=S, window=Wn)
    lay = W.make_layout(w)
    tables = lay.tables.copy()
    for s in range(3):
        keep = policies.streaming_keep(int(lay.lens[s]), S, Wn)
        used = np.unique(np.nonzero(keep)[0] // 16)
        drop = np.setdiff1d(np.arange(tables.shape[1]), used)
        tables[s, drop] = -1
    case = H.Case(w)
    case.tables = torch.from_numpy(tables).cuda()
    # rewrite: poison everything, then write only kept positions
    case.pools = H.make_pools(w, lay.num_blocks)
    for s in range(3):
        L_s = int(lay.lens[s])
        kept = np.nonzero(policies.streaming_keep(L_s, S, Wn))[0]
        rows = torch.from_numpy(H.logical_rows(lay, s, kept)).cuda()
        slots = ops.paged_token_slots(case.tables, torch.full((kept.size,), s, dtype=torch.int32).cuda(),
                                      torch.from_numpy(kept.astype(np.int32)).cuda(), lay.num_blocks)
        ops.paged_kv_write(case.ksrc[rows].contiguous(), case.vsrc[rows].contiguous(), case.pools[0],
                           case.pools[1], slots)
    out = case.attend()
    assert torch.isfinite(out).all()
    assert _max_err(case, out) <= 2e-3


def test_invalid_device_values_poison_only_their_sequence():
    w = _case_workload("bf16", "bf16", 128, 32, 8, 8, lens=(600, 600, 600, 600))
    case = H.Case(w)
    good = case.attend()
    tables = case.tables.clone()
    tables[1, 3] = -1                                  # a kept block unmapped
    tables[2, 0] = case.lay.num_blocks + 5             # a kept block outside the pool
    lens = case.lens.clone()
    lens[3] = case.lay.max_len + 1                     # longer than max_context_len
    out = torch.empty_like(good)
    k, v, _, _ = case.pools
    ops.paged_decode_attn(out, case.q, k, v, tables, lens, case.lay.max_len)
    assert torch.equal(out[0], good[0])
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all() and torch.isnan(out[3]).all()
    lens[3] = 0
    ops.paged_decode_attn(out, case.q, k, v, case.tables, lens, case.lay.max_len)
    assert torch.isnan(out[3]).all() and torch.equal(out[:3], good[:3])


# ---------------------------------------------------------------------------- copy-on-write

@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8", "int8_ch"])
def test_copy_on_write(kv):
    """Four sequences share four blocks; seq 3 gets a private copy of its last block (a COW)."""
    w = dataclasses.replace(_case_workload(kv, "bf16", 128, 32, 8, 21, lens=(64,) * 4), shared_prefix=(4, 4),
                            extra_blocks=2)
    case = H.Case(w)
    before = case.attend()
    src = int(case.lay.tables[3, 3])
    dst = int(case.lay.unused_blocks[0])
    assert (case.lay.tables[:, 3] == src).all()
    k, v, ks, vs = case.pools
    ch_before = [None if t is None else t.clone() for t in (ks, vs)]
    ops.kv_block_copy(k, v, torch.tensor([[src, dst]], dtype=torch.int32).cuda(), ks, vs)
    for p in case.pools:
        if p is not None and p.dim() > 2:
            assert torch.equal(p[dst].view(torch.uint8), p[src].view(torch.uint8))
    if kv.endswith("_ch"):                           # static channel scales are not per block: untouched
        assert torch.equal(ks, ch_before[0]) and torch.equal(vs, ch_before[1])
    tables = case.tables.clone()
    tables[3, 3] = dst
    after = torch.empty_like(before)
    ops.paged_decode_attn(after, case.q, k, v, tables, case.lens, 64, k_scale=ks, v_scale=vs)
    assert torch.equal(before, after)
    # a divergent write into seq 3's private block leaves the sharers alone
    new_k = torch.randn((1, 8, 128), device="cuda").to(torch.bfloat16)
    ops.paged_kv_write(new_k, new_k, k, v, torch.tensor([dst * 16 + 15], dtype=torch.int64).cuda(), ks, vs)
    ops.paged_decode_attn(after, case.q, k, v, tables, case.lens, 64, k_scale=ks, v_scale=vs)
    assert torch.equal(before[:3], after[:3]) and not torch.equal(before[3], after[3])


def test_block_copy_skips_invalid_pairs():
    kp = torch.arange(4 * 2 * 16 * 64, dtype=torch.float32, device="cuda").view(4, 2, 16, 16, 4)
    vp = kp.clone().view(4, 2, 64, 16)
    ref_k, ref_v = kp.clone(), vp.clone()
    pairs = torch.tensor([[0, 0], [-1, 2], [1, 9], [2, 3]], dtype=torch.int32).cuda()
    ops.kv_block_copy(kp, vp, pairs)
    ref_k[3] = ref_k[2]
    ref_v[3] = ref_v[2]
    assert torch.equal(kp, ref_k) and torch.equal(vp, ref_v)


# ---------------------------------------------------------------------------- H2O

def test_h2o_mass_and_accumulation():
    w = _case_workload("bf16", "bf16", 128, 32, 8, 31, lens=(2049, 700, 35, 5000))
    case = H.Case(w)
    maxl = case.lay.max_len
    scores = torch.zeros((4, maxl + 3), dtype=torch.float32, device="cuda")
    acc = np.zeros((4, maxl + 3))
    for step in range(3):
        q = W.queries(w, step=step, device="cuda")
        out = case.attend(q=q, attn_mass=scores)
        for s in range(4):
            ref, probs = case.oracle(s, q=q)
            assert np.max(np.abs(H.to_f64(out[s]) - ref)) <= 2e-3
            acc[s, : probs.shape[1]] += probs.mean(axis=0)
    got = scores.cpu().numpy().astype(np.float64)
    assert np.all(got[:, maxl:] == 0)
    rel = np.max(np.abs(got - acc) / np.maximum(acc, 1e-30))
    print(f"mass max rel err {rel:.3e}")
    assert rel <= 1e-4


def test_h2o_mass_with_streaming_keep_set():
    w = dataclasses.replace(_case_workload("bf16", "bf16", 128, 32, 8, 32, lens=(3000, 100)), num_sinks=4,
                            window=600)
    case = H.Case(w)
    scores = torch.zeros((2, 3000), dtype=torch.float32, device="cuda")
    case.attend(attn_mass=scores)
    for s in range(2):
        _, probs = case.oracle(s)
        exp = probs.mean(axis=0)
        got = scores[s, : exp.size].cpu().numpy()
        keep = exp > 0
        assert np.all(got[~keep] == 0)
        assert np.max(np.abs(got[keep] - exp[keep]) / exp[keep]) <= 1e-4


@pytest.mark.parametrize("kv,d,hq,hkv", [("bf16", 64, 512, 64), ("fp8", 128, 288, 36)])
def test_h2o_mass_more_than_256_query_heads(kv, d, hq, hkv):
    """The mass stages the heads' (max, exp-sum) in LDS 256 heads at a time: 512 heads take two full
    chunks, 288 a full and a ragged one.  The 5000-token sequence is cut into several segments, so
    the mass workgroups merge its heads' segment pairs themselves."""
    w = _case_workload(kv, "bf16", d, hq, hkv, 43, lens=(5000, 300, 17))
    case = H.Case(w)
    maxl = case.lay.max_len
    scores = torch.zeros((3, maxl + 5), dtype=torch.float32, device="cuda")
    out = case.attend(attn_mass=scores)
    got = scores.cpu().numpy().astype(np.float64)
    for s in range(3):
        ref, probs = case.oracle(s)
        assert np.max(np.abs(H.to_f64(out[s]) - ref)) <= TOL[kv]
        exp = probs.mean(axis=0)
        assert np.max(np.abs(got[s, : exp.size] - exp) / exp) <= 1e-4
        assert np.all(got[s, exp.size:] == 0)


def test_tiny_h2o_sub_case_budget_24_recent_8():
    """The tiny workload's H2O sub-case: four decode steps accumulate the mass on the GPU, then the
    GPU keep-set (budget 24, recent 8) equals the oracle's selection on the oracle's own mass, taken
    in fp32 like the kernel's.  Where two candidates are closer than the mass tolerance the order
    may legitimately differ; the test asserts there is no such near-tie at the cut here."""
    w = W.WORKLOADS["tiny"]
    case = H.Case(w)
    maxl = case.lay.max_len
    scores = torch.zeros((2, maxl), dtype=torch.float32, device="cuda")
    acc = np.zeros((2, maxl))
    for step in range(4):
        q = W.queries(w, step=step, device="cuda")
        case.attend(q=q, attn_mass=scores)
        for s in range(2):
            _, probs = case.oracle(s, q=q)
            acc[s, : probs.shape[1]] += attention.head_mean_mass(probs)
    idx, cnt = ops.h2o_select(scores, case.lens, maxl, 24, 8)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for s in range(2):
        L = int(case.lay.lens[s])
        ref = policies.h2o_select(acc[s].astype(np.float32), L, 24, 8)
        assert cnt[s] == ref.size and idx[s, : ref.size].tolist() == ref.tolist(), s
        if L > 24:                                    # the cut among candidates is not a near-tie
            cand = np.sort(acc[s, : L - 8])[::-1]
            assert cand[15] - cand[16] > 1e-4 * cand[15]
    assert cnt.tolist() == [24, 24]


def test_h2o_select_bit_exact():
    rng = np.random.default_rng(5)
    B, maxl = 24, 3000
    scores = rng.integers(0, 50, size=(B, maxl)).astype(np.float32) / 7       # many ties
    scores[3, :100] = np.nan
    scores[4, :] = -0.0
    scores[4, ::3] = 0.0
    scores[5] = rng.random(maxl).astype(np.float32)
    scores[6, 10] = np.inf
    lens = rng.integers(1, maxl + 1, size=B).astype(np.int32)
    lens[0], lens[1], lens[2] = 1, 600, 601
    budget, recent = 600, 150
    for bud, rec in ((budget, recent), (600, 600), (600, 0), (1, 1), (1, 0)):
        idx, cnt = ops.h2o_select(torch.from_numpy(scores).cuda(), torch.from_numpy(lens).cuda(), maxl, bud, rec)
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        for s in range(B):
            ref = policies.h2o_select(scores[s], int(lens[s]), bud, rec)
            assert cnt[s] == ref.size
            assert idx[s, : ref.size].tolist() == ref.tolist(), (bud, rec, s)
            assert np.all(idx[s, ref.size:] == -1)
    bad = torch.from_numpy(lens).cuda()
    bad[7] = 0
    bad[8] = maxl + 1
    idx, cnt = ops.h2o_select(torch.from_numpy(scores).cuda(), bad, maxl, budget, recent)
    assert cnt[7].item() == -1 and cnt[8].item() == -1 and torch.all(idx[7:9] == -1)


# ---------------------------------------------------------------------------- eviction: keep-set + compaction

KEEP_RULES = [(4, 256, 252, "all"),      # should_cache (PA 组合)
              (0, 150, 450, "rest"),     # H2OEviction.select, budget 600
              (4, 64, 100, "rest"),      # sinks + window + heavy hitters of the middle
              (0, 0, 600, "all"),        # evict_tokens, budget 600
              (2, 0, 0, "rest"), (0, 600, 0, "rest"), (1, 1, 1, "all")]


def test_keep_select_bit_exact():
    rng = np.random.default_rng(55)
    B, maxl = 24, 3000
    scores = rng.integers(0, 50, size=(B, maxl)).astype(np.float32) / 7       # many ties
    scores[3, :100] = np.nan
    scores[4, :] = -0.0
    scores[4, ::3] = 0.0
    scores[5] = rng.random(maxl).astype(np.float32)
    scores[6, 10] = np.inf
    scores[9, 2000:] = -np.inf
    lens = rng.integers(1, maxl + 1, size=B).astype(np.int32)
    lens[0], lens[1], lens[2], lens[10] = 1, 600, 601, 3
    sc, ln = torch.from_numpy(scores).cuda(), torch.from_numpy(lens).cuda()
    for sinks, recent, heavy, mode in KEEP_RULES:
        idx, cnt = ops.keep_select(sc, ln, maxl, sinks, recent, heavy, mode)
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        for s in range(B):
            ref = policies.keep_select(scores[s], int(lens[s]), sinks, recent, heavy, mode)
            assert cnt[s] == ref.size, (sinks, recent, heavy, mode, s)
            assert idx[s, : ref.size].tolist() == ref.tolist(), (sinks, recent, heavy, mode, s)
            assert np.all(idx[s, ref.size:] == -1)
    bad = ln.clone()
    bad[7], bad[8] = 0, maxl + 1
    idx, cnt = ops.keep_select(sc, bad, maxl, 4, 256, 252, "all")
    assert cnt[7].item() == -1 and cnt[8].item() == -1 and torch.all(idx[7:9] == -1)


_NP = {torch.float32: np.float32, torch.bfloat16: np.uint16, torch.float16: np.float16, torch.uint8: np.uint8,
       torch.int8: np.int8}


def _host_pools(pools, kv):
    """Host copies of device pools as the oracle's storage arrays (same shapes, same bytes)."""
    return [None if t is None else t.detach().cpu().contiguous().view(torch.uint8).numpy().view(
        _NP[t.dtype]).reshape(t.shape) for t in pools]


@pytest.mark.parametrize("kv,d", [("f32", 64), ("bf16", 128), ("f16", 64), ("fp8", 128), ("fp8", 64), ("int8", 128),
                                  ("fp8_ch", 128), ("int8_ch", 64)])
def test_compact_pool_bytes_bit_exact(kv, d):
    """kv_compact moves kept tokens exactly as the oracle's compact does; no other byte changes."""
    lens = (35, 70, 300, 1, 129)
    w = dataclasses.replace(_case_workload(kv, "bf16", d, 8, 2, 77, lens=lens), extra_blocks=40)
    case = H.Case(w)
    lay = case.lay
    rng = np.random.default_rng(8)
    keeps = [policies.keep_select(rng.random(L), L, 4, 16, 20, "all") for L in lens]
    keeps[1] = np.arange(70)                          # keep all (a full copy)
    keeps[3] = np.array([], dtype=np.int64)           # evict everything
    stride = max(1, max(k.size for k in keeps))
    keep_idx = np.full((len(lens), stride), -1, np.int32)
    for s, k in enumerate(keeps):
        keep_idx[s, : k.size] = k
    counts = np.array([k.size for k in keeps], np.int32)
    free = list(lay.unused_blocks)
    dst_w = max(1, -(-stride // 16))
    dst = np.full((len(lens), dst_w), -1, np.int32)
    for s, k in enumerate(keeps):
        for j in range(-(-k.size // 16)):
            dst[s, j] = free.pop()
    ref = _host_pools(case.pools, kv)
    for s in range(len(lens)):
        paging.compact(ref, kv, lay.tables[s], keeps[s], dst[s], lay.num_blocks)
    k, v, ks, vs = case.pools
    ops.kv_compact(k, v, case.tables, torch.from_numpy(dst).cuda(), torch.from_numpy(keep_idx).cuda(),
                   torch.from_numpy(counts).cuda(), ks, vs)
    for got, exp in zip(case.pools, ref):
        if exp is None:
            continue
        assert np.array_equal(got.cpu().contiguous().view(torch.uint8).numpy().reshape(-1),
                              exp.view(np.uint8).reshape(-1))


def test_compact_skips_and_poisons_invalid_entries():
    w = dataclasses.replace(_case_workload("bf16", "bf16", 64, 8, 2, 78, lens=(40, 40)), extra_blocks=8)
    case = H.Case(w)
    lay = case.lay
    free = list(lay.unused_blocks)
    keep_idx = torch.tensor([[0, 1, 5000, 3], [0, 1, 2, 3]], dtype=torch.int32).cuda()   # 5000: outside the table
    dst = torch.tensor([[free[0]], [lay.num_blocks + 5]], dtype=torch.int32).cuda()     # seq 1: bad destination
    counts = torch.tensor([4, 4], dtype=torch.int32).cuda()
    before = [t.clone() for t in case.pools if t is not None]
    k, v, _, _ = case.pools
    ops.kv_compact(k, v, case.tables, dst, keep_idx, counts)
    krows, vrows = H.k_token_rows(k), H.v_token_rows(v)
    b0 = int(free[0])
    assert torch.all(krows[b0 * 16 + 2].view(torch.int16) == -1) and torch.all(vrows[b0 * 16 + 2].view(torch.int16) == -1)
    for o, p in ((0, 0), (1, 1), (3, 3)):
        src = int(lay.tables[0, p // 16]) * 16 + p % 16
        assert torch.equal(krows[b0 * 16 + o], H.k_token_rows(before[0])[src])
        assert torch.equal(vrows[b0 * 16 + o], H.v_token_rows(before[1])[src])
    # only block b0's first four slots changed
    changed = (krows.view(torch.int16) != H.k_token_rows(before[0]).view(torch.int16)).any(-1).any(-1)
    assert set(torch.nonzero(changed).flatten().tolist()) <= {b0 * 16 + i for i in range(4)}
    # a count above the stride skips the sequence entirely
    ops.kv_compact(k, v, case.tables, dst, keep_idx, torch.tensor([9, 0], dtype=torch.int32).cuda())
    assert torch.equal(H.k_token_rows(k).view(torch.int16), krows.view(torch.int16))   # bits (NaN included)


def test_eviction_end_to_end_mass_select_compact_attend():
    """Decode with H2O mass -> should_cache keep-set on the GPU -> compaction into fresh blocks ->
    decode over the compacted cache equals the oracle's attention over its own keep-set."""
    lens = (600, 1200, 90, 2000)
    w = dataclasses.replace(_case_workload("bf16", "bf16", 128, 32, 8, 79, lens=lens), extra_blocks=140)
    case = H.Case(w)
    lay = case.lay
    L = lay.max_len
    scores = torch.zeros((len(lens), L), dtype=torch.float32, device="cuda")
    case.attend(attn_mass=scores)
    idx, cnt = ops.keep_select(scores, case.lens, L, 4, 256, 252, "all")
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    free = list(lay.unused_blocks)
    dst = np.full((len(lens), 32), -1, np.int32)
    ref_keeps = []
    for s, Ls in enumerate(lens):
        _, probs = case.oracle(s)
        ref_keep = policies.keep_select(probs.mean(axis=0), Ls, 4, 256, 252, "all")
        assert idx_h[s, : cnt_h[s]].tolist() == ref_keep.tolist(), s
        ref_keeps.append(ref_keep)
        for j in range(-(-int(cnt_h[s]) // 16)):
            dst[s, j] = free.pop()
    k, v, ks, vs = case.pools
    dst_t = torch.from_numpy(dst).cuda()
    ops.kv_compact(k, v, case.tables, dst_t, idx, cnt, ks, vs)
    q = W.queries(w, step=1, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ops.paged_decode_attn(out, q, k, v, dst_t, cnt, 512, k_scale=ks, v_scale=vs)
    worst = 0.0
    for s in range(len(lens)):
        rows = torch.from_numpy(H.logical_rows(lay, s, ref_keeps[s])).to(case.ksrc.device)
        kr, vr = H.to_f64(case.ksrc.index_select(0, rows)), H.to_f64(case.vsrc.index_select(0, rows))
        ref, _ = attention.decode_attention(H.to_f64(q[s]), kr, vr, 1 / math.sqrt(w.head_dim))
        worst = max(worst, H.max_err(H.to_f64(out[s]), ref))
    print(f"eviction end to end: kept {cnt_h.tolist()}, max abs err {worst:.3e}")
    assert worst <= 2e-3


def test_block_manager_drives_the_compacting_decode_step():
    """The host flow of an eviction folded into a decode step: BlockManager.append_tokens gives the
    step's token its place, compact() hands out fresh blocks for the kept count + 1 (the source blocks
    stay referenced), paged_decode_attn_compact attends the kept tokens and the new one while moving
    them, release_compacted() frees the sources.  The step's output and a later decode over the
    manager's tables match the oracle on the kept rows."""
    from paged_kv_cache_283_amd.block_manager import BlockManager

    hq, hkv, d, nb = 16, 4, 128, 260
    lens0 = [200, 57, 1000, 16]
    seqs = list(range(len(lens0)))
    g = torch.Generator().manual_seed(11)
    rng = np.random.default_rng(11)
    rows = torch.randn((sum(lens0) + len(lens0), hkv, d), generator=g).to(torch.bfloat16)   # token source rows
    row_of = {}                                          # (seq, position) -> source row
    k = torch.full(ops.k_pool_shape(nb, hkv, d, torch.bfloat16), float("nan"), dtype=torch.bfloat16).cuda()
    v = torch.full(ops.v_pool_shape(nb, hkv, d, torch.bfloat16), float("nan"), dtype=torch.bfloat16).cuda()
    bm = BlockManager(nb)
    r = 0
    for s, L in zip(seqs, lens0):
        bm.add_sequence(s, L)
        slots = torch.from_numpy(bm.slot_mapping(s, np.arange(L)).astype(np.int64)).cuda()
        ops.paged_kv_write(rows[r:r + L].cuda(), rows[r:r + L].flip(1).contiguous().cuda(), k, v, slots)
        for p in range(L):
            row_of[(s, p)] = r + p
        r += L
    # the step: one new token per sequence, then the eviction applied while attending
    new_rows = []
    for s, L in zip(seqs, lens0):
        bm.append_tokens(s, 1)
        row_of[(s, L)] = r
        new_rows.append(r)
        r += 1
    src_tables = bm.block_tables(seqs)
    lens = bm.context_lens(seqs)
    keeps = [np.sort(rng.choice(L, size=max(0, L // 3), replace=False)) for L in lens0]
    keeps[3] = np.arange(0)                             # keep nothing old: only the new token stays
    dst_lists = [bm.compact(s, kk.size + 1)[1] for s, kk in zip(seqs, keeps)]
    width = max(len(t) for t in dst_lists)
    dst = np.full((len(seqs), width), -1, np.int32)
    for i, t in enumerate(dst_lists):
        dst[i, : len(t)] = t
    stride = max(1, max(kk.size for kk in keeps))
    keep_idx = np.full((len(seqs), stride), -1, np.int32)
    for i, kk in enumerate(keeps):
        keep_idx[i, : kk.size] = kk
    q = torch.randn((len(seqs), hq, d), generator=g).to(torch.bfloat16).cuda()
    k_new = rows[new_rows].cuda()
    v_new = rows[new_rows].flip(1).contiguous().cuda()
    out = torch.empty((len(seqs), hq, d), dtype=torch.float32, device="cuda")
    max_len = int(lens.max())
    ops.paged_decode_attn_compact(out, q, k, v, torch.from_numpy(src_tables).cuda(), torch.from_numpy(lens).cuda(),
                                  max_len, torch.from_numpy(keep_idx).cuda(),
                                  torch.tensor([kk.size for kk in keeps], dtype=torch.int32).cuda(),
                                  torch.from_numpy(dst).cuda(), k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    assert bm.release_compacted() > 0
    assert [bm.lens[s] for s in seqs] == [kk.size + 1 for kk in keeps]
    q2 = torch.randn((len(seqs), hq, d), generator=g).to(torch.bfloat16).cuda()
    out2 = torch.empty_like(out)
    lens2 = bm.context_lens(seqs)
    max_len2 = int(lens2.max())
    ops.paged_decode_attn(out2, q2, k, v, torch.from_numpy(bm.block_tables(seqs, -(-max_len2 // 16))).cuda(),
                          torch.from_numpy(lens2).cuda(), max_len2)
    scale = 1 / math.sqrt(d)
    worst = 0.0
    for i, (s, L) in enumerate(zip(seqs, lens0)):
        idx = [row_of[(s, int(p))] for p in keeps[i]] + [row_of[(s, L)]]
        kr = H.to_f64(rows[idx])
        vr = H.to_f64(rows[idx].flip(1).contiguous())
        for qq, o in ((q, out), (q2, out2)):
            ref, _ = attention.decode_attention(H.to_f64(qq[i]), kr, vr, scale)
            worst = max(worst, H.max_err(H.to_f64(o[i]), ref))
    print(f"block manager + compacting step: kept {[kk.size for kk in keeps]}, max abs err {worst:.3e}")
    assert worst <= TOL["bf16"]


COMPACT_LENS = (35, 70, 300, 1000, 17, 1, 129, 2000, 640, 48)


def _compact_keeps(lens, append, seed):
    """Keep lists (ascending positions of the old tokens) of many shapes: sparse and dense random
    subsets, keep-all, keep-none, a policy keep-set (sinks + recent window + heavy hitters), one half."""
    rng = np.random.default_rng(seed)
    keeps = []
    for s, L in enumerate(lens):
        old = L - 1 if append else L
        kind = s % 6
        if kind == 0:
            k = np.flatnonzero(rng.random(old) < 0.25)
        elif kind == 1:
            k = np.arange(old)
        elif kind == 2:
            k = np.flatnonzero(rng.random(old) < 0.08)
        elif kind == 3:
            k = policies.keep_select(rng.random(old), old, 4, 16, max(1, old // 5), "all") if old else np.arange(0)
        elif kind == 4:
            k = np.arange(0)
        else:
            k = np.arange(old // 2)
        keeps.append(np.asarray(k, dtype=np.int64))
    return keeps


COMPACT_GRID = [
    # kv, q, d, hq, hkv, append
    ("bf16", "bf16", 128, 32, 8, True),
    ("bf16", "bf16", 128, 32, 8, False),
    ("f16", "f16", 64, 16, 2, True),
    ("bf16", "bf16", 64, 8, 8, True),      # G = 1
    ("f16", "f16", 128, 16, 1, False),     # G = 16
    ("fp8", "bf16", 128, 32, 8, True),     # 8-bit pools: codes and per-token scales move
    ("int8", "bf16", 64, 16, 2, True),
    ("int8", "f16", 128, 32, 8, False),
    ("fp8_ch", "bf16", 128, 32, 8, True),  # static per-channel scales stay
    ("int8_ch", "bf16", 64, 8, 1, False),
]


def _stored_rows(w, case, s, positions):
    """float64 values the pool holds for sequence s's given positions (the oracle's codec)."""
    rows = torch.from_numpy(H.logical_rows(case.lay, s, positions)).to(case.ksrc.device)
    kc, vc = H.channel_pair(w)
    return (H.stored_values(w.kv_dtype, H.to_f64(case.ksrc.index_select(0, rows)), kc),
            H.stored_values(w.kv_dtype, H.to_f64(case.vsrc.index_select(0, rows)), vc))


@pytest.mark.parametrize("kv,q,d,hq,hkv,append", COMPACT_GRID)
def test_decode_attn_compact_matches_oracle(kv, q, d, hq, hkv, append):
    """paged_decode_attn_compact: the output equals the oracle's attention over the kept tokens (and
    the new one), and the pools end up exactly as the oracle's append (new token at L - 1) followed by
    its compaction of the kept positions (and L - 1) into the destination blocks; a decode over the
    destination tables afterwards matches the oracle too.  Ten sequences (more than 8: the long ones are
    cut at range boundaries, so several waves fill one sequence's destination blocks), with one
    length-1 sequence and keep-none lists; keep-none without a new token attends nothing (NaN)."""
    lens = COMPACT_LENS
    w = dataclasses.replace(_case_workload(kv, q, d, hq, hkv, seed=4100 + d + hq, lens=lens), extra_blocks=400,
                            src_dtype=q if kv in CODE8 else kv)
    case = H.Case(w, hold_last=append)
    lay = case.lay
    n_seq = len(lens)
    keeps = _compact_keeps(lens, append, seed=d + hq)
    stride = max(1, max(k.size for k in keeps))
    keep_idx = np.full((n_seq, stride), -1, np.int32)
    for s, k in enumerate(keeps):
        keep_idx[s, : k.size] = k
    counts = np.array([k.size for k in keeps], np.int32)
    free = list(lay.unused_blocks)
    dst_w = -(-(stride + 1) // 16)
    dst = np.full((n_seq, dst_w), -1, np.int32)
    for s, k in enumerate(keeps):
        for jb in range(-(-(k.size + int(append)) // 16)):
            dst[s, jb] = free.pop()
    k_new, v_new = case.newest_rows() if append else (None, None)

    # the oracle: append (new token at L - 1), then compaction of the kept positions (+ L - 1)
    ref = _host_pools(case.pools, kv)
    if append:
        paging.write_tokens(ref, kv, H.to_host(k_new), H.to_host(v_new), w.src_dtype, lay.tables,
                            list(range(n_seq)), [L - 1 for L in lens])
    moved = [np.concatenate([k, [L - 1]]) if append else k for k, L in zip(keeps, lens)]
    for s in range(n_seq):
        paging.compact(ref, kv, lay.tables[s], moved[s], dst[s], lay.num_blocks)

    k, v, ks, vs = case.pools
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    dst_t = torch.from_numpy(dst).cuda()
    ops.paged_decode_attn_compact(out, case.q, k, v, case.tables, case.lens, lay.max_len,
                                  torch.from_numpy(keep_idx).cuda(), torch.from_numpy(counts).cuda(), dst_t,
                                  k_new=k_new, v_new=v_new, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    for got, exp in zip(case.pools, ref):
        if exp is not None:
            assert np.array_equal(got.cpu().contiguous().view(torch.uint8).numpy().reshape(-1),
                                  exp.view(np.uint8).reshape(-1))
    scale = 1 / math.sqrt(d)
    worst = 0.0
    for s in range(n_seq):
        if moved[s].size == 0:
            assert torch.isnan(out[s]).all(), s
            continue
        kr, vr = _stored_rows(w, case, s, moved[s])
        ref_out, _ = attention.decode_attention(H.to_f64(case.q[s]), kr, vr, scale)
        worst = max(worst, H.max_err(H.to_f64(out[s]), ref_out))
        if s == 7:
            keep_rows, keep_v = kr, vr
    # the next step over the destination tables
    new_lens = torch.tensor([m.size for m in moved], dtype=torch.int32).cuda()
    q2 = W.queries(w, step=1, device="cuda")
    out2 = torch.empty(q2.shape, dtype=torch.float32, device="cuda")
    ops.paged_decode_attn(out2, q2, k, v, dst_t, new_lens, 16 * dst_w, k_scale=ks, v_scale=vs)
    ref2, _ = attention.decode_attention(H.to_f64(q2[7]), keep_rows, keep_v, scale)
    err2 = H.max_err(H.to_f64(out2[7]), ref2)
    print(f"compacting decode {kv}/{q} D={d} G={hq // hkv} append={append}: kept {counts.tolist()}, "
          f"max abs err {worst:.3e}, next step {err2:.3e}")
    assert worst <= TOL[kv] and err2 <= TOL[kv]


@pytest.mark.parametrize("kv,q,d,hq,hkv,append", [("bf16", "bf16", 128, 32, 8, True), ("f16", "f16", 64, 16, 2, False),
                                                  ("fp8", "bf16", 128, 32, 8, True)])
def test_decode_attn_compact_with_h2o_mass(kv, q, d, hq, hkv, append):
    """The compacting step with the H2O mass: entry i of the compacted score row is the moved token's
    source score plus this step's mass of it (the oracle's head-mean probabilities over the kept tokens
    and the new one, 1e-4 relative, plus the fp32 rounding of the sum); entries past the moved tokens
    keep their values; output and pools as without the mass."""
    lens = COMPACT_LENS
    w = dataclasses.replace(_case_workload(kv, q, d, hq, hkv, seed=4300 + d, lens=lens), extra_blocks=400,
                            src_dtype=q if kv in CODE8 else kv)
    case = H.Case(w, hold_last=append)
    lay = case.lay
    n_seq, L = len(lens), lay.max_len
    keeps = _compact_keeps(lens, append, seed=7 + d)
    stride = max(1, max(k.size for k in keeps))
    keep_idx = np.full((n_seq, stride), -1, np.int32)
    for s_, k_ in enumerate(keeps):
        keep_idx[s_, : k_.size] = k_
    counts = np.array([k_.size for k_ in keeps], np.int32)
    free = list(lay.unused_blocks)
    dst_w = -(-(stride + 1) // 16)
    dst = np.full((n_seq, dst_w), -1, np.int32)
    for s_, k_ in enumerate(keeps):
        for jb in range(-(-(k_.size + int(append)) // 16)):
            dst[s_, jb] = free.pop()
    rng = np.random.default_rng(99)
    src_scores = rng.random((n_seq, L)).astype(np.float32)
    src_t = torch.from_numpy(src_scores).cuda()
    dst_t = torch.full((n_seq, L), -7.0, dtype=torch.float32, device="cuda")
    k_new, v_new = case.newest_rows() if append else (None, None)
    k, v, ks, vs = case.pools
    out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    ops.paged_decode_attn_compact(out, case.q, k, v, case.tables, case.lens, L, torch.from_numpy(keep_idx).cuda(),
                                  torch.from_numpy(counts).cuda(), torch.from_numpy(dst).cuda(), k_new=k_new,
                                  v_new=v_new, k_scale=ks, v_scale=vs, attn_mass_src=src_t, attn_mass=dst_t)
    torch.cuda.synchronize()
    got = dst_t.cpu().numpy().astype(np.float64)
    assert torch.equal(src_t.cpu(), torch.from_numpy(src_scores))      # the source rows are only read
    scale = 1 / math.sqrt(d)
    worst_out, worst_mass = 0.0, 0.0
    for s_, Ls in enumerate(lens):
        moved = np.concatenate([keeps[s_], [Ls - 1]]) if append else keeps[s_]
        if moved.size == 0:
            assert np.all(got[s_] == -7.0)
            continue
        kr, vr = _stored_rows(w, case, s_, moved)
        ref, probs = attention.decode_attention(H.to_f64(case.q[s_]), kr, vr, scale)
        worst_out = max(worst_out, H.max_err(H.to_f64(out[s_]), ref))
        mass = attention.head_mean_mass(probs)
        exp = src_scores[s_, moved].astype(np.float64) + mass
        err = np.abs(got[s_, : moved.size] - exp)
        bound = 1e-4 * mass + 2.0 ** -22 * np.abs(exp)
        worst_mass = max(worst_mass, float(np.max(err / bound)))
        assert np.all(got[s_, moved.size:] == -7.0), s_
    print(f"compacting step with mass {kv}/{q} D={d}: out err {worst_out:.3e}, mass err / bound {worst_mass:.3f}")
    assert worst_out <= TOL[kv] and worst_mass <= 1.0


def test_decode_attn_compact_poisons_bad_counts_and_skips_bad_destinations():
    """A count past the list or past the old tokens poisons its sequence (NaN output, nothing copied;
    the new token is still stored at L - 1); a destination entry outside the pool skips just the
    tokens that fall in it."""
    lens = (200, 300, 150, 90)
    w = dataclasses.replace(_case_workload("bf16", "bf16", 128, 16, 4, seed=4242, lens=lens), extra_blocks=80)
    case = H.Case(w, hold_last=True)
    lay = case.lay
    keeps = [np.arange(0, 199, 3), np.arange(0, 299, 2), np.arange(0, 149, 7), np.arange(0, 89, 5)]
    stride = max(kk.size for kk in keeps)
    keep_idx = np.full((4, stride), -1, np.int32)
    for s, kk in enumerate(keeps):
        keep_idx[s, : kk.size] = kk
    counts = np.array([kk.size for kk in keeps], np.int32)
    counts[1] = stride + 1            # past the list
    counts[2] = 150                   # past the 149 old tokens
    free = list(lay.unused_blocks)
    dst = np.full((4, 12), -1, np.int32)
    for s, kk in enumerate(keeps):
        for jb in range(-(-(kk.size + 1) // 16)):
            dst[s, jb] = free.pop()
    dst[3, 1] = lay.num_blocks + 7    # sequence 3 (19 tokens): tokens 16..18 fall in an entry outside the pool
    k_new, v_new = case.newest_rows()
    ref = _host_pools(case.pools, "bf16")
    paging.write_tokens(ref, "bf16", H.to_host(k_new), H.to_host(v_new), "bf16", lay.tables, [0, 1, 2, 3],
                        [L - 1 for L in lens])
    paging.compact(ref, "bf16", lay.tables[0], np.concatenate([keeps[0], [lens[0] - 1]]), dst[0], lay.num_blocks)
    paging.compact(ref, "bf16", lay.tables[3], keeps[3][:16], dst[3, :1], lay.num_blocks)
    k, v, _, _ = case.pools
    out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    ops.paged_decode_attn_compact(out, case.q, k, v, case.tables, case.lens, lay.max_len,
                                  torch.from_numpy(keep_idx).cuda(), torch.from_numpy(counts).cuda(),
                                  torch.from_numpy(dst).cuda(), k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()
    assert torch.isfinite(out[[0, 3]]).all()
    for got, exp in zip(case.pools, ref):
        if exp is not None:
            assert np.array_equal(got.cpu().contiguous().view(torch.uint8).numpy().reshape(-1),
                                  exp.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32", "int8", "fp8_ch"])
def test_append_equals_slots_then_write(kv):
    """paged_kv_append stores exactly what paged_decode_slots + paged_kv_write store, and skips the
    sequences whose decode slot is -1."""
    d = 64 if kv == "f32" else 128
    w = dataclasses.replace(_case_workload(kv, "f32" if kv == "f32" else "bf16", d, 8, 2, 93,
                                           lens=(35, 70, 16, 1, 200)), extra_blocks=4)
    a, b = H.Case(w, hold_last=True), H.Case(w, hold_last=True)
    lens = a.lens.clone()
    lens[3] = 0                                    # invalid length: skipped by both
    tables = a.tables.clone()
    tables[4, (int(lens[4]) - 1) // 16] = a.lay.num_blocks + 7   # table entry outside the pool: skipped
    k_new, v_new = a.newest_rows()
    ka, va, ksa, vsa = a.pools
    kb, vb, ksb, vsb = b.pools
    ops.paged_kv_append(k_new, v_new, ka, va, tables, lens, ksa, vsa)
    slots = ops.paged_decode_slots(tables, lens, b.lay.num_blocks)
    assert slots[3].item() == -1 and slots[4].item() == -1
    ops.paged_kv_write(k_new, v_new, kb, vb, slots, ksb, vsb)
    for x, y in zip(a.pools, b.pools):
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    out = a.attend()                                # and the appended tokens are attended correctly
    for s in (0, 1, 2):
        ref, _ = a.oracle(s)
        assert np.max(np.abs(H.to_f64(out[s]) - ref)) <= TOL[kv]


APPEND_ATTN_GRID = [
    # kv, src, q, d, hq, hkv, num_sinks, window, mass   (8-bit pools: fused when src == q, else two launches)
    ("bf16", "bf16", "bf16", 128, 32, 8, 0, 0, False),
    ("bf16", "bf16", "f32", 64, 16, 2, 0, 0, True),
    ("bf16", "bf16", "bf16", 128, 16, 1, 0, 0, False),
    ("f16", "f16", "f16", 128, 16, 16, 4, 40, False),
    ("f16", "f16", "bf16", 64, 8, 4, 0, 0, True),
    ("f32", "f32", "f32", 64, 8, 2, 0, 0, False),
    ("f32", "f32", "f32", 128, 16, 1, 2, 100, True),
    ("fp8", "bf16", "bf16", 128, 32, 8, 0, 0, False),
    ("fp8", "f32", "f32", 64, 8, 2, 4, 40, True),
    ("fp8", "bf16", "f16", 128, 16, 2, 0, 0, False),
    ("int8", "bf16", "bf16", 128, 32, 8, 4, 64, True),
    ("int8", "f16", "f16", 64, 16, 16, 0, 0, False),
    ("int8", "bf16", "f32", 128, 8, 8, 0, 0, False),
    ("fp8_ch", "bf16", "bf16", 64, 8, 2, 0, 0, False),
    ("fp8_ch", "bf16", "bf16", 128, 32, 8, 0, 0, True),
    ("int8_ch", "bf16", "bf16", 128, 16, 2, 0, 0, False),
    ("int8_ch", "f32", "f32", 64, 8, 4, 0, 0, False),
]
APPEND_LENS = (1, 15, 16, 17, 35, 70, 511, 512, 513, 1100, 2049, 300, 64)


@pytest.mark.parametrize("kv,src,q,d,hq,hkv,sinks,window,mass", APPEND_ATTN_GRID)
def test_append_attn_equals_append_then_attend(kv, src, q, d, hq, hkv, sinks, window, mass):
    """paged_decode_append_attn (the new token -- quantised in the kernel for 8-bit pools -- enters the
    attention kernel's operands, and the kernel stores it) leaves the output, the pools and the H2O
    mass bit-identical to paged_kv_append followed by paged_decode_attn, and matches the oracle.  Both calls get
    max_context_len = 2048, so sequence 10 (2049 tokens) is unusable for attention (NaN) while its
    token is still appended; sequence 11 has an unusable length and sequence 12 a last table entry
    outside the pool (NaN outputs, nothing stored)."""
    w = dataclasses.replace(_case_workload(kv, q, d, hq, hkv, seed=hq * 7 + d + hkv + window, lens=APPEND_LENS),
                            src_dtype=src, num_sinks=sinks, window=window, extra_blocks=4)
    a, b = H.Case(w, hold_last=True), H.Case(w, hold_last=True)
    assert int(a.lay.lens[10]) == 2049 and a.lay.max_len == 2049
    for c in (a, b):
        c.lens[11] = 0
        c.tables[12, (int(c.lay.lens[12]) - 1) // 16] = c.lay.num_blocks + 5
    k_new, v_new = a.newest_rows()
    ka, va, ksa, vsa = a.pools
    kb, vb, ksb, vsb = b.pools
    L = 2048
    n = len(APPEND_LENS)
    mass_a = torch.zeros((n, L), dtype=torch.float32, device="cuda") if mass else None
    mass_b = mass_a.clone() if mass else None
    out_a = torch.empty((n, hq, d), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    ops.paged_kv_append(k_new, v_new, ka, va, a.tables, a.lens, ksa, vsa)
    ops.paged_decode_attn(out_a, a.q, ka, va, a.tables, a.lens, L, k_scale=ksa, v_scale=vsa, num_sinks=sinks,
                          window=window, attn_mass=mass_a)
    ops.paged_decode_append_attn(out_b, b.q, k_new, v_new, kb, vb, b.tables, b.lens, L, k_scale=ksb, v_scale=vsb,
                                 num_sinks=sinks, window=window, attn_mass=mass_b)
    torch.cuda.synchronize()
    for x, y in zip(a.pools, b.pools):
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    valid = [s for s in range(n) if s not in (10, 11, 12)]
    assert torch.equal(out_a[valid], out_b[valid])
    for s in (10, 11, 12):
        assert torch.isnan(out_b[s]).all()
    if mass:
        assert torch.equal(mass_a[valid], mass_b[valid])
        assert torch.equal(mass_b[10:12], torch.zeros_like(mass_b[10:12]))
    err = max(H.max_err(H.to_f64(out_b[s]), b.oracle(s)[0]) for s in valid)
    print(f"append+attend {kv}<-{src}/{q} D={d} G={hq // hkv} sinks={sinks} window={window}: max abs err {err:.3e}")
    assert err <= TOL[kv]
    if kv not in CODE8:   # sequence 10's token was stored, not skipped by both paths
        slot = int(a.lay.tables[10][2048 // 16]) * 16 + 2048 % 16
        assert torch.equal(H.k_token_rows(kb)[slot].contiguous().view(torch.uint8), k_new[10].view(torch.uint8))
        assert torch.equal(H.v_token_rows(vb)[slot].contiguous().view(torch.uint8), v_new[10].view(torch.uint8))


@pytest.mark.parametrize("kv,d,hq,hkv", [("bf16", 128, 32, 8), ("fp8", 128, 32, 8), ("f32", 64, 16, 1)])
def test_append_attn_repeated_step_is_idempotent(kv, d, hq, hkv):
    """bench.py repeats the decode step on the same pools: the second call finds the token already in
    its slot (stored after the first call's waves finished) and must give the same output, pools and
    H2O mass; the mass window cuts the longer sequences into several chunks."""
    w = _case_workload(kv, "bf16" if kv != "f32" else "f32", d, hq, hkv, seed=77, lens=APPEND_LENS[:11])
    c = H.Case(w, hold_last=True)
    L = c.lay.max_len
    mass1 = torch.zeros((11, L), dtype=torch.float32, device="cuda")
    mass2 = torch.zeros_like(mass1)
    out1 = c.decode_step(attn_mass=mass1)
    torch.cuda.synchronize()
    pools1 = [x.clone() if x is not None else None for x in c.pools]
    out2 = c.decode_step(attn_mass=mass2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    assert torch.equal(mass1, mass2)
    for x, y in zip(pools1, c.pools):
        if x is not None:
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    err = max(H.max_err(H.to_f64(out2[s]), c.oracle(s)[0]) for s in range(11))
    assert err <= TOL[kv]


@pytest.mark.parametrize("lens", [(35, 70, 300, 1000, 17, 129, 64, 2000, 900, 33, 4096, 250),   # one wave per head merge
                                  (700, 1500, 3000)])                                          # four-wave merge
def test_decode_graph_replays_equal_eager(lens):
    """Both decode entry points captured in a HIP graph replay to the eager result bit for bit, with
    eager calls on other queries (same workspace) and synchronisations between the replays: nothing
    a call leaves in the workspace changes a later call, and no captured node depends on a value the
    host computed at capture time from device state."""
    w = _case_workload("bf16", "bf16", 128, 32, 8, seed=9100, lens=lens)
    case = H.Case(w)
    k, v, ks, vs = case.pools
    b, hq, d = case.q.shape
    L = case.lay.max_len
    ws = ops.alloc_workspace(b, hq, d, L, 0, 0, False, case.q.device)
    q2 = case.q.flip(0).contiguous()

    def call(out, q, noalloc):
        if noalloc:
            ops.paged_decode_attn_noalloc(out, q, k, v, case.tables, case.lens, L, k_scale=ks, v_scale=vs)
        else:
            ops.paged_decode_attn(out, q, k, v, case.tables, case.lens, L, k_scale=ks, v_scale=vs, workspace=ws)

    for noalloc in (False, True):
        ref, ref2 = torch.empty_like(case.q, dtype=torch.float32), torch.empty_like(case.q, dtype=torch.float32)
        call(ref, case.q, noalloc)
        call(ref2, q2, noalloc)
        torch.cuda.synchronize()
        out = torch.empty_like(ref)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(out, case.q, noalloc)
        for _ in range(3):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), noalloc
            o2 = torch.full_like(ref, float("nan"))
            call(o2, q2, noalloc)
            torch.cuda.synchronize()
            assert torch.equal(o2, ref2), noalloc
    err = max(H.max_err(H.to_f64(ref[s]), case.oracle(s)[0]) for s in range(b))
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------------------- multi-query (chunked prefill)

def _prefill_case(kv, q, d, hq, hkv, seed, lens, n_qs):
    w = _case_workload(kv, q, d, hq, hkv, seed, lens=lens)
    case = H.Case(w)
    g = torch.Generator().manual_seed(seed)
    T = int(sum(n_qs))
    qt = torch.randn((T, hq, d), generator=g).to(W.storage_dtype(q) if q != "f32" else torch.float32).cuda()
    qs = torch.tensor(np.concatenate([[0], np.cumsum(n_qs)]).astype(np.int32)).cuda()
    return w, case, qt, qs


def _prefill_oracle(w, case, qt, qs, s, scale=None):
    L = int(case.lay.lens[s])
    kr, vr = H.kept_source(w, case.lay, s, case.ksrc, case.vsrc)
    kc, vc = H.channel_pair(w)
    kr, vr = H.stored_values(w.kv_dtype, kr, kc), H.stored_values(w.kv_dtype, vr, vc)
    a, b = int(qs[s]), int(qs[s + 1])
    scale = 1 / math.sqrt(w.head_dim) if scale is None else scale
    return attention.prefill_attention(H.to_f64(qt[a:b]), kr, vr, scale)


PREFILL_GRID = [
    # kv, q, d, hq, hkv
    ("bf16", "bf16", 128, 32, 8),     # G = 4: 4 query tokens per wave
    ("fp8", "bf16", 128, 32, 8),
    ("int8", "bf16", 128, 32, 8),
    ("fp8_ch", "bf16", 128, 32, 8),
    ("int8_ch", "f16", 64, 16, 2),
    ("f32", "f32", 64, 8, 2),
    ("f16", "f16", 128, 16, 16),      # G = 1: 16 query tokens per wave
    ("bf16", "f32", 64, 16, 2),       # G = 8, split query operand
    ("bf16", "bf16", 128, 16, 1),     # G = 16: one token per wave
]


@pytest.mark.parametrize("kv,q,d,hq,hkv", PREFILL_GRID)
def test_prefill_matches_oracle(kv, q, d, hq, hkv):
    # whole prompt, chunk after a prefix, single token, ragged tails, and a chunk after a longer
    # prefix (many block pairs every column sees whole, then pairs across the causal limits)
    lens = (70, 300, 17, 129, 1, 1000)
    n_qs = (70, 37, 1, 64, 1, 150)
    w, case, qt, qs = _prefill_case(kv, q, d, hq, hkv, 101, lens, n_qs)
    out = torch.full(qt.shape, float("nan"), dtype=torch.float32, device="cuda")
    k, v, ks, vs = case.pools
    ops.paged_prefill_attn(out, qt, k, v, case.tables, case.lens, qs, case.lay.max_len, max(n_qs),
                           k_scale=ks, v_scale=vs)
    worst = 0.0
    for s in range(len(lens)):
        ref = _prefill_oracle(w, case, qt, qs, s)
        a, b = int(qs[s]), int(qs[s + 1])
        worst = max(worst, H.max_err(H.to_f64(out[a:b]), ref))
    print(f"prefill {kv}/{q} d{d} {hq}/{hkv}: max abs err {worst:.3e}")
    assert worst <= TOL[kv]


@pytest.mark.parametrize("kv,q,d,hq,hkv", [("bf16", "bf16", 128, 32, 8), ("fp8", "bf16", 128, 32, 8),
                                           ("int8_ch", "f16", 64, 16, 2), ("f32", "f32", 64, 8, 2)])
def test_prefill_scale_sign_and_zero(kv, q, d, hq, hkv):
    """The logit factor's sign is folded into the query operands (the largest logit is then the
    largest raw product): negative and zero scales give the oracle's result."""
    lens, n_qs = (300, 90, 1000), (37, 90, 100)
    w, case, qt, qs = _prefill_case(kv, q, d, hq, hkv, 104, lens, n_qs)
    k, v, ks, vs = case.pools
    for sc in (-0.07, 0.0, 0.2):
        out = torch.full(qt.shape, float("nan"), dtype=torch.float32, device="cuda")
        ops.paged_prefill_attn(out, qt, k, v, case.tables, case.lens, qs, case.lay.max_len, max(n_qs),
                               scale=sc, k_scale=ks, v_scale=vs)
        worst = 0.0
        for s in range(len(lens)):
            ref = _prefill_oracle(w, case, qt, qs, s, scale=sc)
            a, b = int(qs[s]), int(qs[s + 1])
            worst = max(worst, H.max_err(H.to_f64(out[a:b]), ref))
        assert worst <= TOL[kv], (sc, worst)


def test_prefill_last_row_equals_decode():
    """The last query row of a chunk attends to the whole context: it is the decode step's attention."""
    lens = (200, 1000)
    n_qs = (50, 9)
    w, case, qt, qs = _prefill_case("bf16", "bf16", 128, 32, 8, 102, lens, n_qs)
    out = torch.empty(qt.shape, dtype=torch.float32, device="cuda")
    k, v, _, _ = case.pools
    ops.paged_prefill_attn(out, qt, k, v, case.tables, case.lens, qs, case.lay.max_len, 50)
    last = qt[qs[1:].long() - 1].contiguous()
    dec = torch.empty(last.shape, dtype=torch.float32, device="cuda")
    ops.paged_decode_attn(dec, last, k, v, case.tables, case.lens, case.lay.max_len)
    # The decode kernel feeds PV with ~16-bit probabilities (bf16 high + low parts), the prefill
    # kernel with f16 ones (11 significant bits, relative rounding error <= 2^-11): the two rows
    # differ by at most 2^-11 of the largest |V| (plus accumulation order).
    vmax = float(case.vsrc.abs().max())
    assert torch.max(torch.abs(dec - out[qs[1:].long() - 1])).item() <= 2.0 ** -11 * vmax + 1e-5


def test_prefill_v_beyond_f16_range():
    """bf16 V values past f16's largest finite value (65504) become inf in the f16 PV pass; the
    workgroups that saw one compute again with the high/low probability split.  Every output is
    finite and within the split path's accuracy of the oracle (probabilities to 2^-15, fp32 sums);
    the untouched sequence keeps the 2e-3 bar."""
    lens, n_qs = (300, 1000, 70), (37, 150, 70)
    w, case, qt, qs = _prefill_case("bf16", "bf16", 128, 32, 8, 105, lens, n_qs)
    vs = case.vsrc
    r1 = torch.from_numpy(H.logical_rows(case.lay, 1, np.array([5, 900]))).to(vs.device).long()
    r2 = torch.from_numpy(H.logical_rows(case.lay, 2, np.array([0]))).to(vs.device).long()
    vs[r1[0], 3, 17] = 7.0e4         # one element early in the context: every row of the chunk sees it
    vs[r1[1], :, 5] = -2.5e5         # one dim of every head inside the chunk: rows after it see it
    vs[r2[0], 0, :] = 1.0e6          # a whole row of KV head 0 at the first position of a prompt
    H.fill(w, case.lay, case.pools, case.ksrc, vs, case.tables)
    out = torch.full(qt.shape, float("nan"), dtype=torch.float32, device="cuda")
    k, v, _, _ = case.pools
    ops.paged_prefill_attn(out, qt, k, v, case.tables, case.lens, qs, case.lay.max_len, max(n_qs))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    for s in range(len(lens)):
        ref = _prefill_oracle(w, case, qt, qs, s)
        a, b = int(qs[s]), int(qs[s + 1])
        _, vr = H.kept_source(w, case.lay, s, case.ksrc, vs)
        tol = TOL["bf16"] + 2.0 ** -13 * float(np.abs(vr).max())
        err = H.max_err(H.to_f64(out[a:b]), ref)
        print(f"prefill with large V, sequence {s}: max abs err {err:.3e} (bound {tol:.3e})")
        assert err <= tol, (s, err, tol)


@pytest.mark.parametrize("kv,jump", [("bf16", 0.6), ("bf16", 30.0), ("f16", 30.0)])
def test_prefill_late_logit_jump(kv, jump):
    """A key past a chunk's first block pair whose logit exceeds every earlier one: by about 10
    (base 2, jump 0.6), the f16 path keeps the first pair's max and the probabilities reach ~2^10;
    by several hundred (jump 30) they pass f16's range, and the workgroup computes again with the
    split path.  Both match the oracle."""
    lens, n_qs = (300, 1000), (37, 120)
    w, case, qt, qs = _prefill_case(kv, kv, 128, 32, 8, 106, lens, n_qs)
    g = torch.Generator().manual_seed(7)
    u = torch.randn(128, generator=g)
    qt[:] = u.to(qt.dtype).to(qt.device)                        # every query row and head: u
    ks = case.ksrc
    r = torch.from_numpy(H.logical_rows(case.lay, 0, np.array([200]))).to(ks.device).long()
    r1 = torch.from_numpy(H.logical_rows(case.lay, 1, np.array([700, 950]))).to(ks.device).long()
    ks[r] = (jump * u).to(ks.dtype).to(ks.device)               # all KV heads
    ks[r1] = (jump * u).to(ks.dtype).to(ks.device)
    H.fill(w, case.lay, case.pools, ks, case.vsrc, case.tables)
    out = torch.full(qt.shape, float("nan"), dtype=torch.float32, device="cuda")
    k, v, _, _ = case.pools
    ops.paged_prefill_attn(out, qt, k, v, case.tables, case.lens, qs, case.lay.max_len, max(n_qs))
    worst = 0.0
    for s in range(len(lens)):
        ref = _prefill_oracle(w, case, qt, qs, s)
        a, b = int(qs[s]), int(qs[s + 1])
        worst = max(worst, H.max_err(H.to_f64(out[a:b]), ref))
    print(f"prefill {kv} with a late logit jump x{jump}: max abs err {worst:.3e}")
    assert worst <= TOL[kv]


@pytest.mark.parametrize("kv", ["bf16", "f16"])
def test_prefill_context_beyond_one_table_chunk(kv):
    """A context of 20000 tokens is 1250 blocks: the kernel stages its block table 1024 entries at
    a time, so the ring restarts (prologue, V rewrite of the first pair, running-max check) inside
    the sequence.  A 64-row chunk at the end and a 40-row chunk after 16384 + 8 tokens, against the
    oracle."""
    lens, n_qs = (20000, 16432), (64, 40)
    w, case, qt, qs = _prefill_case(kv, kv, 128, 8, 2, 107, lens, n_qs)
    out = torch.full(qt.shape, float("nan"), dtype=torch.float32, device="cuda")
    k, v, _, _ = case.pools
    ops.paged_prefill_attn(out, qt, k, v, case.tables, case.lens, qs, case.lay.max_len, max(n_qs))
    worst = 0.0
    for s in range(len(lens)):
        ref = _prefill_oracle(w, case, qt, qs, s)
        a, b = int(qs[s]), int(qs[s + 1])
        worst = max(worst, H.max_err(H.to_f64(out[a:b]), ref))
    print(f"prefill {kv} over 20000 / 16432 tokens: max abs err {worst:.3e}")
    assert worst <= TOL[kv]


def test_prefill_16bit_outputs_are_the_rounded_f32_output():
    """bf16 and f16 outputs (written four dims per store) are the f32 output of the same call rounded
    to nearest even, element for element."""
    lens, n_qs = (300, 1000), (37, 150)
    w, case, qt, qs = _prefill_case("bf16", "bf16", 128, 32, 8, 108, lens, n_qs)
    k, v, _, _ = case.pools
    outs = {}
    for dt in (torch.float32, torch.bfloat16, torch.float16):
        outs[dt] = torch.empty(qt.shape, dtype=dt, device="cuda")
        ops.paged_prefill_attn(outs[dt], qt, k, v, case.tables, case.lens, qs, case.lay.max_len, max(n_qs))
    ref = outs[torch.float32]
    for dt in (torch.bfloat16, torch.float16):
        assert torch.equal(outs[dt], ref.to(dt)), dt


def test_prefill_invalid_sequences():
    lens = (40, 40, 40)
    n_qs = (8, 8, 8)
    w, case, qt, qs = _prefill_case("bf16", "bf16", 64, 8, 2, 103, lens, n_qs)
    lens_bad = case.lens.clone()
    lens_bad[1] = 5                                   # shorter than its chunk: NaN rows
    tables = case.tables.clone()
    tables[2, 0] = case.lay.num_blocks + 3            # a block outside the pool: NaN rows
    out = torch.zeros(qt.shape, dtype=torch.float32, device="cuda")
    k, v, _, _ = case.pools
    ops.paged_prefill_attn(out, qt, k, v, tables, lens_bad, qs, case.lay.max_len, 8)
    assert torch.all(torch.isfinite(out[0:8])) and torch.all(torch.isnan(out[8:24]))
    # rows outside [0, num_tokens): the sequence is skipped, nothing written
    qs_bad = qs.clone()
    qs_bad[3] = 30
    out2 = torch.zeros(qt.shape, dtype=torch.float32, device="cuda")
    ops.paged_prefill_attn(out2, qt, k, v, case.tables, case.lens, qs_bad, case.lay.max_len, 8)
    assert torch.all(out2[16:24] == 0) and torch.all(torch.isfinite(out2[:16]))


# ---------------------------------------------------------------------------- prefix caching

def test_prefix_cache_hit_prefills_only_the_suffix():
    """Request b shares request a's 2048-token prompt through the prefix cache: only b's 300 new
    tokens are written, and the causal attention of b's chunk over the shared blocks equals the
    oracle over b's whole context; a's own decode is unaffected."""
    from paged_kv_cache_283_amd.block_manager import PrefixCachingBlockManager
    hq, hkv, d = 32, 8, 128
    g = torch.Generator().manual_seed(4242)
    rng = np.random.default_rng(4242)
    prompt = rng.integers(0, 32000, 2048).tolist()
    suf_a, suf_b = rng.integers(0, 32000, 100).tolist(), rng.integers(0, 32000, 300).tolist()
    rows = {name: (torch.randn((n, hkv, d), generator=g).to(torch.bfloat16),
                   torch.randn((n, hkv, d), generator=g).to(torch.bfloat16))
            for name, n in (("p", 2048), ("a", 100), ("b", 300))}
    bm = PrefixCachingBlockManager(320)
    k, v, ks, vs = ops.allocate_pools(320, hkv, d, torch.bfloat16, "cuda", fill_byte=0xFF)

    def write(seq, positions, kr, vr):
        slots = torch.from_numpy(bm.slot_mapping(seq, positions)).cuda()
        ops.paged_kv_write(kr.cuda(), vr.cuda(), k, v, slots)

    _, cached_a = bm.add_cached_sequence("a", prompt + suf_a)
    assert cached_a == 0
    write("a", np.arange(2148), torch.cat([rows["p"][0], rows["a"][0]]), torch.cat([rows["p"][1], rows["a"][1]]))
    bm.commit("a")
    tab_b, cached_b = bm.add_cached_sequence("b", prompt + suf_b)
    assert cached_b == 2048 and tab_b[:128] == bm.tables["a"][:128]
    write("b", np.arange(2048, 2348), rows["b"][0], rows["b"][1])          # the only prefill work of b
    tables = torch.from_numpy(bm.block_tables(["a", "b"])).cuda()
    lens = torch.from_numpy(bm.context_lens(["a", "b"])).cuda()
    q = torch.randn((1 + 300, hq, d), generator=g).to(torch.bfloat16).cuda()
    qs = torch.tensor([0, 1, 301], dtype=torch.int32).cuda()               # a: its last token; b: its chunk
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ops.paged_prefill_attn(out, q, k, v, tables, lens, qs, 2348, 300)
    f64 = lambda t: t.to(torch.float64).numpy()
    ka, va = f64(torch.cat([rows["p"][0], rows["a"][0]])), f64(torch.cat([rows["p"][1], rows["a"][1]]))
    kb, vb = f64(torch.cat([rows["p"][0], rows["b"][0]])), f64(torch.cat([rows["p"][1], rows["b"][1]]))
    ref_a = attention.prefill_attention(H.to_f64(q[0:1]), ka, va, 1 / math.sqrt(d))
    ref_b = attention.prefill_attention(H.to_f64(q[1:301]), kb, vb, 1 / math.sqrt(d))
    err = max(H.max_err(H.to_f64(out[0:1]), ref_a), H.max_err(H.to_f64(out[1:301]), ref_b))
    print(f"prefix cache: b reused {cached_b} tokens, max abs err {err:.3e}")
    assert err <= 2e-3


# ---------------------------------------------------------------------------- swap to host

@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8", "fp8_ch"])
def test_swap_out_and_back_into_other_blocks(kv):
    """A sequence's blocks go to pinned host slots byte for byte, its pool blocks are overwritten,
    and after swapping back into different blocks its attention is bit-identical."""
    w = dataclasses.replace(_case_workload(kv, "bf16", 128, 32, 8, 131, lens=(100, 300, 50)), extra_blocks=24)
    case = H.Case(w)
    lay = case.lay
    before = case.attend()
    pools = case.pools
    arena = ops.allocate_host_arena(32, 8, 128, pools[0].dtype, per_token_scales=not kv.endswith("_ch"))
    nblk = -(-300 // 16)
    src = lay.tables[1, :nblk].astype(np.int32)
    slots = np.arange(5, 5 + nblk, dtype=np.int32)[::-1].copy()
    ops.kv_swap(pools, arena, torch.from_numpy(np.stack([src, slots], 1)).cuda(), to_host=True)
    torch.cuda.synchronize()
    for p, a in zip(pools, arena):
        if a is not None:
            assert torch.equal(a[torch.from_numpy(slots).long()].view(torch.uint8),
                               p[torch.from_numpy(src).long()].cpu().view(torch.uint8))
    for p in pools:                                   # the pool blocks are reused by someone else
        if p is not None and p.dim() > 2:
            p.view(torch.uint8)[torch.from_numpy(src).long()] = 0xFF
    dst = np.asarray(lay.unused_blocks[:nblk], dtype=np.int32)
    ops.kv_swap(pools, arena, torch.from_numpy(np.stack([dst, slots], 1)).cuda(), to_host=False)
    tables = case.tables.clone()
    tables[1, :nblk] = torch.from_numpy(dst).cuda()
    after = torch.empty_like(before)
    k, v, ks, vs = pools
    ops.paged_decode_attn(after, case.q, k, v, tables, case.lens, lay.max_len, k_scale=ks, v_scale=vs)
    assert torch.equal(before, after)
    # out-of-range pairs are skipped
    ops.kv_swap(pools, arena, torch.tensor([[-1, 0], [0, 99], [lay.num_blocks, 1]], dtype=torch.int32).cuda(),
                to_host=True)
    torch.cuda.synchronize()
