"""paged_decode_attn_noalloc (the library's fixed per-device workspace, for callers that cannot
allocate) against paged_decode_attn with a caller workspace, through the C ABI.

The two run the same kernels on the same inputs, so their outputs (and H2O mass) must be
bit-identical; the first call is also checked against the fp64 oracle at the usual bars
(2e-3 max-abs for bf16 KV, mass 1e-4 relative).  Two calls in a row, the second smaller, show
that what the first left in the shared array does not leak into the second.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from paged_kv_cache_283_amd import _lib, ops

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import _harness as H


def _both(case, attn_mass_rows=None, **kw):
    """(out_noalloc, out_workspace, mass_noalloc, mass_workspace) for one case."""
    w = case.w
    k, v, ks, vs = case.pools
    outs, masses = [], []
    for fn in (ops.paged_decode_attn_noalloc, ops.paged_decode_attn):
        out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
        mass = None
        if attn_mass_rows is not None:
            mass = torch.zeros((w.num_seqs, attn_mass_rows), dtype=torch.float32, device="cuda")
        fn(out, case.q, k, v, case.tables, case.lens, case.lay.max_len, k_scale=ks, v_scale=vs,
           num_sinks=w.num_sinks, window=w.window, attn_mass=mass, **kw)
        outs.append(out)
        masses.append(mass)
    torch.cuda.synchronize()
    return outs[0], outs[1], masses[0], masses[1]


def test_noalloc_equals_workspace_call_two_calls_second_smaller():
    # call 1: the Llama-3-8B layer decode workload (64 sequences, lengths 512..8192)
    big = H.Case(W.WORKLOADS["llama3"])
    a, b, _, _ = _both(big)
    assert torch.equal(a, b)
    worst = 0.0
    for s in (0, 21, 42, 63):
        ref, _ = big.oracle(s)
        worst = max(worst, H.max_err(H.to_f64(a[s]), ref))
    assert worst <= 2e-3
    # call 2: fewer, shorter sequences, with the H2O mass (a different layout of the array)
    small = dataclasses.replace(W.WORKLOADS["llama3"], name="noalloc-small", num_seqs=5, len_range=(20, 3000),
                                seed=2851)
    case = H.Case(small)
    maxl = case.lay.max_len
    a2, b2, ma, mb = _both(case, attn_mass_rows=maxl + 3)
    assert torch.equal(a2, b2) and torch.equal(ma, mb)
    got = ma.cpu().numpy().astype(np.float64)
    for s in range(small.num_seqs):
        ref, probs = case.oracle(s)
        assert np.max(np.abs(H.to_f64(a2[s]) - ref)) <= 2e-3
        exp = probs.mean(axis=0)
        assert np.max(np.abs(got[s, : exp.size] - exp) / exp) <= 1e-4
    print(f"noalloc: llama3 max abs err {worst:.3e}; second call bit-identical to the workspace call")


def test_noalloc_streaming_then_tiny():
    """The StreamingLLM keep-set (sinks + window over 131072-token logical contexts), then the tiny
    fp32 workload: each bit-identical to the workspace call."""
    w = dataclasses.replace(W.WORKLOADS["streaming"], num_seqs=8, lens=(131072,) * 8)
    case = H.Case(w)
    a, b, _, _ = _both(case)
    assert torch.equal(a, b)
    ref, _ = case.oracle(3)
    assert np.max(np.abs(H.to_f64(a[3]) - ref)) <= 2e-3
    tiny = H.Case(W.WORKLOADS["tiny"])
    a2, b2, _, _ = _both(tiny)
    assert torch.equal(a2, b2)


def test_noalloc_rejects_calls_beyond_its_fixed_workspace():
    w = W.WORKLOADS["llama3"]
    case = H.Case(dataclasses.replace(w, num_seqs=2, len_range=(100, 200)))
    k, v, _, _ = case.pools
    out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    # 2 sequences of up to 2^21 tokens with the mass: far beyond 64 MiB of workspace
    tables = torch.full((2, (1 << 21) // 16), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.PagedKVError) as e:
        ops.paged_decode_attn_noalloc(out, case.q, k, v, tables, case.lens, 1 << 21,
                                      attn_mass=torch.zeros((2, 1 << 21), device="cuda"))
    assert e.value.status == _lib.EWORKSPACE
