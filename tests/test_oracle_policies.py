"""Oracle pins: StreamingLLM keep-set and H2O selection.

The keep predicate is checked against a literal simulation of the page's
append-then-trim list; the H2O selection against a rank-counting brute force
and against torch.topk run the way the page's select runs it.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import policies

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


class _ListStreamingCache:
    """The page's StreamingKVCache behaviour on token ids: append, then trim the middle once over capacity."""

    def __init__(self, num_sinks, window):
        self.s, self.w, self.ids = num_sinks, window, []

    def append(self, t):
        self.ids.append(t)
        if len(self.ids) > self.s + self.w:
            self.ids = self.ids[: self.s] + self.ids[-self.w:]


@pytest.mark.parametrize("sinks", [0, 1, 4])
@pytest.mark.parametrize("window", [1, 8, 16, 33])
def test_keep_predicate_equals_list_simulation(sinks, window):
    c = _ListStreamingCache(sinks, window)
    for L in range(1, 81):
        c.append(L - 1)
        pred = np.nonzero(policies.streaming_keep(L, sinks, window))[0].tolist()
        assert pred == c.ids, (L, sinks, window)


def test_streaming_workload_keep_set():
    d = GOLD["streaming_defaults"]
    keep = np.nonzero(policies.streaming_keep(131072, d["num_sinks"], d["window"]))[0]
    assert keep.size == 4100
    assert keep[:4].tolist() == [0, 1, 2, 3] and keep[4] == 126976 and keep[-1] == 131071


def test_window_off_keeps_everything():
    assert policies.streaming_keep(50, 4, 0).all() and policies.streaming_keep(50, 0, -3).all()


def _brute_select(scores, L, budget, recent):
    """Position p < L - recent is a heavy hitter iff fewer than budget - recent candidates outrank it."""
    if L <= budget:
        return list(range(L))
    cand, k = L - recent, budget - recent
    s = [(-np.inf if np.isnan(x) else x) for x in scores[:cand]]
    sel = []
    for p in range(cand):
        better = sum(1 for q in range(cand) if s[q] > s[p] or (s[q] == s[p] and q < p))
        if better < k:
            sel.append(p)
    return sel + list(range(cand, L))


def test_select_matches_rank_brute_force_with_ties():
    rng = np.random.default_rng(99)
    for trial in range(300):
        L = int(rng.integers(1, 40))
        budget = int(rng.integers(0, 30))
        recent = int(rng.integers(0, budget + 1))
        scores = rng.integers(0, 4, size=48).astype(np.float64)          # many ties
        if trial % 7 == 0:
            scores[rng.integers(0, 48, 3)] = np.nan
        got = policies.h2o_select(scores, L, budget, recent).tolist()
        assert got == _brute_select(scores, L, budget, recent)
        assert len(got) == min(budget, L) or (L <= budget and len(got) == L)
        assert got == sorted(got)


def test_select_matches_page_topk_without_ties():
    """With distinct scores the page's select (topk of the candidates + recent, sorted) gives the same set."""
    rng = np.random.default_rng(5)
    d = GOLD["h2o_defaults"]
    budget, recent = d["budget"], d["recent"]
    for L in (2049, 4096, 8192):
        scores = torch.from_numpy(rng.random(8192))
        head = scores[: L - recent].topk(budget - recent).indices.tolist()
        page = sorted(set(head + list(range(L - recent, L))))
        assert policies.h2o_select(scores.numpy(), L, budget, recent).tolist() == page


def test_accumulate_growing_context():
    scores = np.zeros(10)
    scores = policies.h2o_accumulate(scores, np.array([0.5, 0.5]))
    scores = policies.h2o_accumulate(scores, np.array([0.25, 0.25, 0.5]))
    scores = policies.h2o_accumulate(scores, np.array([0.1, 0.2, 0.3, 0.4]))
    assert np.allclose(scores, [0.85, 0.95, 0.8, 0.4, 0, 0, 0, 0, 0, 0], atol=0, rtol=1e-15)
    with pytest.raises(ValueError):
        policies.h2o_accumulate(np.zeros(2), np.ones(3))


def test_select_rejects_bad_budget():
    with pytest.raises(ValueError):
        policies.h2o_select(np.zeros(5), 5, 2, 3)


# ---------------------------------------------------------------------------- keep_select

def _brute_keep(scores, L, sinks, recent, heavy, candidates):
    """Rank counting: p is a heavy hitter iff fewer than `heavy` candidates outrank it."""
    s = [(-np.inf if np.isnan(x) else x) for x in scores[:L]]
    forced = [p < sinks or p >= L - recent for p in range(L)]
    cand = [p for p in range(L) if candidates == "all" or not forced[p]]
    keep = []
    for p in range(L):
        if forced[p]:
            keep.append(p)
            continue
        if p in cand or candidates == "all":
            better = sum(1 for q in cand if s[q] > s[p] or (s[q] == s[p] and q < p))
            if better < heavy:
                keep.append(p)
    return keep


def test_keep_select_matches_rank_brute_force_with_ties():
    rng = np.random.default_rng(283)
    for trial in range(400):
        L = int(rng.integers(1, 50))
        sinks, recent, heavy = (int(x) for x in rng.integers(0, 20, 3))
        mode = policies.CANDIDATES[trial % 2]
        scores = rng.integers(0, 4, size=64).astype(np.float64)
        if trial % 5 == 0:
            scores[rng.integers(0, 64, 4)] = np.nan
        if trial % 9 == 0:
            scores[rng.integers(0, 64, 4)] = -0.0
        got = policies.keep_select(scores, L, sinks, recent, heavy, mode).tolist()
        assert got == _brute_keep(scores, L, sinks, recent, heavy, mode), (L, sinks, recent, heavy, mode)
        assert got == sorted(set(got))


def test_keep_select_rest_without_sinks_is_h2o_select():
    rng = np.random.default_rng(17)
    for _ in range(200):
        L = int(rng.integers(1, 60))
        budget = int(rng.integers(0, 40))
        recent = int(rng.integers(0, budget + 1))
        scores = rng.integers(0, 5, size=64).astype(np.float64)
        assert (policies.keep_select(scores, L, 0, recent, budget - recent, "rest").tolist()
                == policies.h2o_select(scores, L, budget, recent).tolist())


def test_keep_select_is_the_page_should_cache_predicate():
    """PA 组合: cached iff p < sink_size, or recent, or p in scores.argsort()[-h2o_size:] (distinct scores)."""
    c = GOLD["combined_policy"]
    sink_size, window_size = c["sinks"], c["window"]
    h2o_size = c["total"] - sink_size - window_size
    assert h2o_size == c["heavy"]
    rng = np.random.default_rng(512)
    for L in (1, 5, 200, 300, 511, 512, 513, 1000, 4096):
        scores = rng.permutation(L).astype(np.float64) / L           # distinct: argsort is unambiguous
        top = set(np.argsort(scores)[-h2o_size:].tolist()) if h2o_size else set()

        def should_cache(pos, is_recent):
            if pos < sink_size or is_recent:
                return True
            return pos in top

        page = [p for p in range(L) if should_cache(p, p >= L - window_size)]
        got = policies.keep_select(scores, L, sink_size, window_size, h2o_size, "all").tolist()
        assert got == page, L
        assert len(got) <= c["total"]


def test_keep_select_is_the_page_evict_tokens():
    """SO 4.2 evict_tokens: the `budget` highest accumulated scores (torch.topk), nothing forced."""
    rng = np.random.default_rng(42)
    for L, budget in ((100, 10), (8192, 2048), (300, 300), (50, 80)):
        scores = torch.from_numpy(rng.random(L))
        top = scores.topk(min(budget, L)).indices.tolist()
        got = policies.keep_select(scores.numpy(), L, 0, 0, budget, "all").tolist()
        assert got == sorted(top)


def test_keep_select_rejects_bad_arguments():
    with pytest.raises(ValueError):
        policies.keep_select(np.zeros(4), 4, -1, 0, 1, "all")
    with pytest.raises(ValueError):
        policies.keep_select(np.zeros(4), 4, 0, 0, 1, "middle")
