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
