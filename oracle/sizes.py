"""KV-cache size formulas (oracle; test infrastructure only).

[LC] = page "长上下文优化：注意力稀疏化与 KV Cache 管理" (plumephp.com/llm-long-context-optimization)
[PA] = page "KV Cache 与 PagedAttention：显存复用与长上下文推理" (plumephp.com/ai-kv-cache-paged-attention)

Both pages state the same product: one K and one V vector per layer, per KV
head, per token, each head_dim elements of dtype_bytes bytes ([LC] opening
formula and kv_cache_gb snippet; [PA] block "显存公式").
"""

GIB = 1024 ** 3


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> int:
    """Bytes of K+V held per token across all layers ([LC] opening formula)."""
    return 2 * n_layers * n_kv_heads * head_dim * dtype_bytes


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, bytes_per: int = 2) -> int:
    """Total K+V bytes of one sequence ([PA] block "显存公式", kv_cache_size snippet)."""
    return kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per) * seq_len


def kv_cache_gib(n_layers: int, n_kv_heads: int, head_dim: int, max_len: int,
                 batch: int = 1, dtype_bytes: int = 2) -> float:
    """K+V of a batch in GiB, 1024**3-byte units ([LC] kv_cache_gb snippet).

    The page prints 2.0 / 32.0 / 16.0 next to its three example calls; the
    arithmetic of the function itself gives half of each (1.0 / 16.0 / 8.0),
    which also agrees with the page's own 128k-token estimate and with the
    per-request sizes of [SO] section 5.  This function follows the formula.
    """
    return kv_bytes_per_token(n_layers, n_kv_heads, head_dim, dtype_bytes) * max_len * batch / GIB


def blocks_needed(num_tokens: int, block_size: int = 16) -> int:
    """Physical blocks a sequence of num_tokens occupies ([PA] "PagedAttention 的设计":
    fixed-size blocks, only the last one partly filled)."""
    if num_tokens < 0:
        raise ValueError("num_tokens must be >= 0")
    return -(-num_tokens // block_size)


def last_block_fill(num_tokens: int, block_size: int = 16) -> int:
    """Tokens held by the last block of a sequence (1..block_size; 0 for an empty one)."""
    if num_tokens <= 0:
        return 0
    r = num_tokens % block_size
    return block_size if r == 0 else r
