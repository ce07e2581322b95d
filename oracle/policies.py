"""KV keep-set policies: StreamingLLM sinks + window, H2O heavy hitters (oracle; test infrastructure only).

[LC] = page "长上下文优化：注意力稀疏化与 KV Cache 管理" (plumephp.com/llm-long-context-optimization):
       StreamingKVCache snippet (defaults 4 sinks, window 4096) and H2OEviction
       snippet (defaults budget 2048, recent 512; update_scores, select).
[SO] = page "系统优化", section 4.1 "StreamingLLM 详解": keep the first few tokens
       (usually 4) plus the most recent W; section 4.2 "KV Cache 淘汰", the H2O
       pseudocode evict_tokens: keep the `budget` highest accumulated scores.
[PA] = page "KV Cache 与 PagedAttention：显存复用与长上下文推理", the 组合 snippet
       should_cache: a position is cached if it is one of the first sink_size,
       if it is recent, or if it is among the h2o_size highest scores.

Readings where the pages are silent or inconsistent:
  * window counts the most recent W positions including the token being
    decoded; window <= 0 switches the policy off (attend to everything);
  * scores live in a buffer of the maximum context length, positions the
    buffer has not seen yet start at 0 (the page's slice-add breaks once the
    new weights are longer than the old scores);
  * heavy-hitter ties go to the lower position; a NaN score ranks below every
    number; if the context is no longer than the budget everything is kept;
  * heavy hitters are drawn only from positions before the recent window and
    the result is returned in ascending position order.
  * keep_select covers the three rules with one shape: forced positions (the
    first num_sinks and the last `recent`) united with the `heavy` highest
    scores of a candidate set -- the positions that are not forced
    (H2OEviction.select, with num_sinks = 0) or every position (should_cache
    ranks all scores; evict_tokens has nothing forced).  should_cache's
    heavy set may overlap the forced ones, so it keeps at most
    sink + window + h2o positions.  Kept tokens are listed in ascending position
    order for every rule (evict_tokens' gather in score order is a detail of
    the gather; decode attention does not depend on the order of its keys).
"""

import numpy as np


def streaming_keep(context_len: int, num_sinks: int, window: int) -> np.ndarray:
    """bool [context_len]: position p is attended iff p < num_sinks or p >= context_len - window."""
    p = np.arange(context_len)
    if window <= 0:
        return np.ones(context_len, dtype=bool)
    return (p < num_sinks) | (p >= context_len - window)


def h2o_accumulate(scores: np.ndarray, mass: np.ndarray) -> np.ndarray:
    """scores[:len(mass)] += mass, in a buffer at least as long as mass (new positions start at 0)."""
    if mass.shape[0] > scores.shape[0]:
        raise ValueError("score buffer shorter than the context")
    out = np.array(scores, dtype=np.float64, copy=True)
    out[: mass.shape[0]] += mass
    return out


def h2o_select(scores, kv_len: int, budget: int, recent: int) -> np.ndarray:
    """Positions kept by H2O: the last `recent` positions plus the (budget - recent)
    highest-scoring earlier positions, in ascending order (int64)."""
    if recent < 0 or budget < recent:
        raise ValueError("need 0 <= recent <= budget")
    if kv_len <= budget:
        return np.arange(kv_len, dtype=np.int64)
    cand = kv_len - recent
    s = np.asarray(scores[:cand], dtype=np.float64)
    s = np.where(np.isnan(s), -np.inf, s)
    order = np.lexsort((np.arange(cand), -s))   # score high -> low, then position low -> high
    heavy = np.sort(order[: budget - recent])
    return np.concatenate([heavy, np.arange(cand, kv_len)]).astype(np.int64)


CANDIDATES = ("rest", "all")


def keep_select(scores, kv_len: int, num_sinks: int, recent: int, heavy: int, candidates: str) -> np.ndarray:
    """Positions kept by an eviction rule, ascending (int64).

    forced  = {p < num_sinks} | {p >= kv_len - recent}
    C       = positions not forced ("rest") or all of [0, kv_len) ("all")
    heavy_s = the `heavy` highest scores in C (all of C if it is smaller),
              higher score first, then lower position; NaN ranks like -inf
    keep    = forced | heavy_s
    """
    if min(num_sinks, recent, heavy) < 0 or candidates not in CANDIDATES:
        raise ValueError("need num_sinks, recent, heavy >= 0 and candidates in ('rest', 'all')")
    p = np.arange(kv_len)
    forced = (p < num_sinks) | (p >= kv_len - recent)
    cand = p[~forced] if candidates == "rest" else p
    s = np.asarray(scores[:kv_len], dtype=np.float64)[cand]
    s = np.where(np.isnan(s), -np.inf, s)
    order = np.lexsort((cand, -s))               # score high -> low, then position low -> high
    keep = forced.copy()
    keep[cand[order[:heavy]]] = True
    return p[keep].astype(np.int64)
