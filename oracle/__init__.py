"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE, not product code.

A plain, slow, obviously correct numpy (float64) statement of what the paged
decode path computes, written from the pages themselves:

  [LC] "长上下文优化：注意力稀疏化与 KV Cache 管理"
       https://www.plumephp.com/llm-long-context-optimization/
       (headings stripped; cited by snippet: kv_cache_gb, StreamingKVCache,
       H2OEviction, the block-table sketch, the MHA/GQA/MQA table)
  [PA] "KV Cache 与 PagedAttention：显存复用与长上下文推理"
       https://www.plumephp.com/ai-kv-cache-paged-attention/
       (cited by its bullet-block headers, e.g. "PagedAttention 的设计")
  [SO] "系统优化"
       https://www.threethreeliu.top/projects/knowledge-inference-optimization-memory-9b32e2e927
       (cited by its numbered sections, e.g. 4.2)

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It imports nothing but the Python
standard library and numpy, and shares no code, table or constant generator
with the HIP library under ``paged_kv_cache_283_amd/``.

Modules
-------
sizes      KV-cache byte formulas                      [LC] kv_cache_gb, [PA] 显存公式
fp8        OCP FP8 E4M3FN codec + per-token scaling    [PA] 量化原理
paging     block mapping, pool layout, write, COW       [PA] PagedAttention 的设计 / 三大运行时组件
attention  fp64 softmax decode attention, H2O mass      [LC] MHA/GQA table, H2OEviction.update_scores
policies   StreamingLLM keep-set, H2O top-k selection   [LC] StreamingKVCache, H2OEviction.select

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against page-printed values, closed forms, a library routine or brute force
(see ``tests/test_oracle_*.py``); none is "parity unpinned".
"""

from . import sizes, fp8, paging, attention, policies  # noqa: F401
