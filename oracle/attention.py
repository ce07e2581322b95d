"""Single-token decode attention in float64 (oracle; test infrastructure only).

[LC] = page "长上下文优化：注意力稀疏化与 KV Cache 管理" (plumephp.com/llm-long-context-optimization):
       the MHA/GQA/MQA table (n_kv_heads between 1 and n_heads), the H2OEviction
       snippet's update_scores (attention weights summed over query positions,
       averaged over heads, accumulated per position), and the Flash sketch
       (tiling + online softmax only change how the same result is reached).
[PA] = page "KV Cache 与 PagedAttention：显存复用与长上下文推理": decode reads KV block by block
       through the block table ("三大运行时组件"), so paging does not change the result.

[SO] = page "系统优化", 4.5 "Chunked Prefill" and "分页 KV Cache + 前缀缓存": a long prompt
       is processed in chunks interleaved with decode steps, over a paged
       cache whose prefix may be shared; [PA] "共享场景的价值": a prefix-cache hit
       skips the prefill of the shared part.

Readings where the pages are silent:
  * query head h uses KV head h // G, G = n_heads / n_kv_heads (contiguous groups);
  * softmax scale is an argument (1/sqrt(head_dim) in every workload here);
  * the decoded token is already in the cache and attends to itself;
  * a prefill chunk of n_q tokens is the last n_q positions of the sequence,
    already written to the cache; its token i (position p = L - n_q + i)
    attends causally to positions 0..p, i.e. everything before the chunk
    (the cached or shared prefix) and the chunk up to itself.
"""

import numpy as np

from . import paging, policies


def decode_attention(q, K, V, scale: float, keep=None):
    """Plain softmax attention of one query token over logical keys/values.

    q [Hq][D], K and V [L][Hkv][D] (float64).  keep: bool [L] or None (all).
    Returns (out [Hq][D], probs [Hq][L]) with probs 0 at positions not kept.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hq, d = q.shape
    L, hkv, _ = K.shape
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    idx = np.arange(L) if keep is None else np.nonzero(np.asarray(keep, dtype=bool))[0]
    if idx.size == 0:
        raise ValueError("no key position to attend to")
    out = np.zeros((hq, d))
    probs = np.zeros((hq, L))
    for g in range(hkv):
        heads = slice(g * group, (g + 1) * group)          # the query heads reading KV head g
        z = scale * (K[idx, g, :] @ q[heads].T)           # [n_kept, G] logits
        w = np.exp(z - z.max(axis=0))
        pi = w / w.sum(axis=0)
        out[heads] = pi.T @ V[idx, g, :]
        probs[heads, idx] = pi.T
    return out, probs


def head_mean_mass(probs):
    """H2O per-position mass of one decode step: mean over query heads of the probabilities.

    With one query position, the page's sum over query positions is the
    identity, so this is probs.mean over the head axis.
    """
    return np.asarray(probs, dtype=np.float64).mean(axis=0)


def paged_decode(pools, kv_dtype: str, q, table_row, context_len: int, scale: float,
                 num_sinks: int = 0, window: int = 0, num_blocks=None):
    """Decode attention of one sequence read through its block table.

    Positions outside the StreamingLLM keep-set (policies.streaming_keep) are
    neither read nor attended.  Returns (out [Hq][D], probs [Hq][context_len]).
    """
    if context_len < 1:
        raise ValueError("context_len must be >= 1")
    keep = policies.streaming_keep(context_len, num_sinks, window)
    pos = np.nonzero(keep)[0]
    Kk, Vk = paging.gather_logical(pools, kv_dtype, table_row, pos, num_blocks)
    hkv, d = Kk.shape[1], Kk.shape[2]
    K = np.zeros((context_len, hkv, d))
    V = np.zeros((context_len, hkv, d))
    K[pos], V[pos] = Kk, Vk
    return decode_attention(q, K, V, scale, keep)


def prefill_attention(q, K, V, scale: float):
    """Causal attention of the last n_q positions of a sequence over its whole context.

    q [n_q][Hq][D]; K, V [L][Hkv][D] with L >= n_q.  Query i sits at position
    L - n_q + i and attends to positions 0..L - n_q + i: each row is the decode
    attention of that token over the context cut after it.  Returns out
    [n_q][Hq][D].
    """
    q = np.asarray(q, dtype=np.float64)
    n_q, L = q.shape[0], np.asarray(K).shape[0]
    if n_q < 1 or n_q > L:
        raise ValueError("need 1 <= n_q <= L")
    out = np.empty(q.shape)
    for i in range(n_q):
        p = L - n_q + i
        out[i], _ = decode_attention(q[i], K[: p + 1], V[: p + 1], scale)
    return out


def paged_prefill(pools, kv_dtype: str, q, table_row, context_len: int, scale: float, num_blocks=None):
    """prefill_attention of one sequence whose context is read through its block table."""
    K, V = paging.gather_logical(pools, kv_dtype, table_row, np.arange(context_len), num_blocks)
    return prefill_attention(q, K, V, scale)
