"""Paged KV storage: block mapping, pool layout, token write, block copy (oracle; test infrastructure only).

[LC] = page "长上下文优化：注意力稀疏化与 KV Cache 管理" (plumephp.com/llm-long-context-optimization),
       the block-table sketch (logical tokens 0-15 / 16-31 / 32.. in physical blocks 7 / 2 / 19).
[PA] = page "KV Cache 与 PagedAttention：显存复用与长上下文推理" (plumephp.com/ai-kv-cache-paged-attention),
       blocks "PagedAttention 的设计", "物理布局示意", "三大运行时组件", and the copy_on_write snippet.

What the pages fix: a sequence's tokens are cut into fixed 16-token blocks;
logical block j of a sequence lives in the physical block its block table
names at index j; physical blocks come from one shared pool.  What they leave
open and is taken here as the storage convention (the same one the HIP
library documents):

  K pool  [num_blocks][num_kv_heads][head_dim/X][16][X]          X = 16 bytes of elements:
                                                                8 for bf16/f16, 16 for fp8/int8, 4 for f32
  V pool  [num_blocks][num_kv_heads][head_dim/(16Y)][16][4][Y][4] Y = 4 / bytes per element:
                                                                2 for bf16/f16, 4 for fp8/int8, 1 for f32
  scales  [num_blocks][num_kv_heads][16] float32                 fp8 and int8 only, K and V separately
  channel scales [num_kv_heads][head_dim] float32                fp8_ch and int8_ch: static, given by the
                                                                caller, one per (KV head, channel)

(K element (token o, dim d) of a block tile sits at chunk d // X, row o, lane
d % X.  V element (token o, dim d), with t = d // 16, sits at index
[t // Y][d % 16][o // 4][t % Y][o % 4]: each 16-byte chunk holds 4 consecutive
tokens of Y dims 16 apart.)

Storage dtypes are held here as raw numpy arrays: "f32" float32, "bf16" uint16
bit patterns, "f16" float16, "fp8" uint8 E4M3FN codes, "int8" int8 codes; "fp8_ch" and
"int8_ch" hold the same codes scaled per channel instead of per token.
"""

import numpy as np

from . import fp8, int8

BLOCK_SIZE = 16
DTYPES = ("f32", "bf16", "f16", "fp8", "int8", "fp8_ch", "int8_ch")
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.float16, "fp8": np.uint8, "int8": np.int8,
            "fp8_ch": np.uint8, "int8_ch": np.int8}
_CODECS = {"fp8": fp8, "int8": int8}       # quantised storage: codes + one scale per (token, KV head)
_CHANNEL = {"fp8_ch": fp8, "int8_ch": int8}  # codes + one static scale per (KV head, channel)


def quantised(kv_dtype: str) -> bool:
    """Codes with one scale per (token, KV head), stored beside them in the pool."""
    return kv_dtype in _CODECS


def channel_scaled(kv_dtype: str) -> bool:
    """Codes with static per-(KV head, channel) scales given by the caller."""
    return kv_dtype in _CHANNEL


def storage_dtype(kv_dtype: str):
    return _STORAGE[kv_dtype]


def k_chunk(kv_dtype: str) -> int:
    """Elements per 16-byte K chunk."""
    return 16 // np.dtype(_STORAGE[kv_dtype]).itemsize


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (fp8 codes decode without their scale)."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = a.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("fp8", "fp8_ch"):
        return fp8.decode(a)
    if dtype in ("int8", "int8_ch"):
        return int8.decode(a)
    raise ValueError(dtype)


def physical_block(table_row, pos: int, num_blocks: int, block_size: int = BLOCK_SIZE) -> int:
    """Physical block of logical position pos ([PA] 物理布局示意): the table entry of block pos // 16.

    Raises if the entry is not a valid pool index (e.g. -1 for an unmapped block).
    """
    b = int(table_row[pos // block_size])
    if not 0 <= b < num_blocks:
        raise IndexError(f"position {pos}: table entry {b} is not a block of a {num_blocks}-block pool")
    return b


def slot(table_row, pos: int, num_blocks: int, block_size: int = BLOCK_SIZE) -> int:
    """Flat token slot in the pool: physical block * 16 + offset inside the block."""
    return physical_block(table_row, pos, num_blocks, block_size) * block_size + pos % block_size


def v_chunk_dims(kv_dtype: str) -> int:
    """Dims (16 apart) per 16-byte V chunk of 4 tokens."""
    return 4 // np.dtype(_STORAGE[kv_dtype]).itemsize


def _v_groups(head_dim: int, kv_dtype: str) -> int:
    y = v_chunk_dims(kv_dtype)
    if head_dim % (16 * y):
        raise ValueError(f"head_dim {head_dim} is not a multiple of {16 * y} ({kv_dtype} V chunks)")
    return head_dim // (16 * y)


def _v_put(v_tile_o, row, kv_dtype):
    """Store row[Hkv][D] into the V chunks of one token offset: view [Hkv][G][16][Y]."""
    hkv, g, c, y = v_tile_o.shape
    v_tile_o[...] = np.asarray(row).reshape(hkv, g, y, c).transpose(0, 1, 3, 2)


def _v_get(v_tile_o):
    """Inverse of _v_put: [Hkv][G][16][Y] chunk view -> [Hkv][D]."""
    hkv, g, c, y = v_tile_o.shape
    return v_tile_o.transpose(0, 1, 3, 2).reshape(hkv, g * y * c)


def new_pools(num_blocks: int, num_kv_heads: int, head_dim: int, kv_dtype: str, fill=0, k_channel=None,
              v_channel=None):
    """Allocate (k_pool, v_pool, k_scale, v_scale) in the documented layout.  The scales are per-token
    arrays for fp8/int8, the given per-channel arrays [Hkv][D] for fp8_ch/int8_ch, else None."""
    st = storage_dtype(kv_dtype)
    x = k_chunk(kv_dtype)
    y = v_chunk_dims(kv_dtype)
    k = np.full((num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x), fill, dtype=st)
    v = np.full((num_blocks, num_kv_heads, _v_groups(head_dim, kv_dtype), 16, 4, y, 4), fill, dtype=st)
    if quantised(kv_dtype):
        ks = np.zeros((num_blocks, num_kv_heads, BLOCK_SIZE), dtype=np.float32)
        vs = np.zeros((num_blocks, num_kv_heads, BLOCK_SIZE), dtype=np.float32)
    elif channel_scaled(kv_dtype):
        if k_channel is None or v_channel is None:
            raise ValueError("fp8_ch/int8_ch pools need k_channel and v_channel [Hkv][D]")
        ks = np.asarray(k_channel, dtype=np.float32).reshape(num_kv_heads, head_dim)
        vs = np.asarray(v_channel, dtype=np.float32).reshape(num_kv_heads, head_dim)
    else:
        ks = vs = None
    return k, v, ks, vs


def write_tokens(pools, kv_dtype: str, k_src, v_src, src_dtype: str, table_rows, seq_ids, positions):
    """Store new tokens' K and V (all KV heads) at the slots their block tables give.

    k_src, v_src: [T][Hkv][D] raw source arrays in src_dtype.  Token t belongs
    to sequence seq_ids[t] at logical position positions[t].  For f32/bf16/f16
    pools the source dtype must equal the pool dtype and the bytes are stored
    unchanged; for fp8/int8 pools each (token, KV head) row is quantised with its
    own scale (quantize_per_token); for fp8_ch/int8_ch pools each element is
    divided by its channel's static scale and encoded (quantize_per_channel).
    Mutates pools in place.
    """
    k_pool, v_pool, k_scale, v_scale = pools
    nb, hkv, nc, _, x = k_pool.shape
    if quantised(kv_dtype) or channel_scaled(kv_dtype):
        if quantised(src_dtype) or channel_scaled(src_dtype):
            raise ValueError("fp8/int8 pools take f32/bf16/f16 sources")
    if quantised(kv_dtype):
        codec = _CODECS[kv_dtype]
        kq, ks = codec.quantize_per_token(to_f64(k_src, src_dtype).astype(np.float32))
        vq, vs = codec.quantize_per_token(to_f64(v_src, src_dtype).astype(np.float32))
    elif channel_scaled(kv_dtype):
        codec = _CHANNEL[kv_dtype]
        kq = codec.quantize_per_channel(to_f64(k_src, src_dtype).astype(np.float32), k_scale)
        vq = codec.quantize_per_channel(to_f64(v_src, src_dtype).astype(np.float32), v_scale)
    elif src_dtype != kv_dtype:
        raise ValueError("a non-fp8 pool stores source bytes of its own dtype")
    for t, (s, p) in enumerate(zip(seq_ids, positions)):
        b = physical_block(table_rows[s], p, nb)
        o = p % BLOCK_SIZE
        if quantised(kv_dtype) or channel_scaled(kv_dtype):
            k_pool[b, :, :, o, :] = kq[t].reshape(hkv, nc, x)
            _v_put(v_pool[b, :, :, :, o // 4, :, o % 4], vq[t], kv_dtype)
            if quantised(kv_dtype):
                k_scale[b, :, o] = ks[t]
                v_scale[b, :, o] = vs[t]
        else:
            k_pool[b, :, :, o, :] = np.asarray(k_src[t]).reshape(hkv, nc, x)
            _v_put(v_pool[b, :, :, :, o // 4, :, o % 4], v_src[t], kv_dtype)


def gather_logical(pools, kv_dtype: str, table_row, positions, num_blocks=None):
    """Logical K, V [len(positions)][Hkv][D] as float64, dequantised for fp8.

    Each position is looked up through the block table ([LC] block-table sketch);
    reading an unmapped (-1) or out-of-pool entry raises.
    """
    k_pool, v_pool, k_scale, v_scale = pools
    nb = k_pool.shape[0] if num_blocks is None else num_blocks
    hkv, d = k_pool.shape[1], k_pool.shape[2] * k_pool.shape[4]
    K = np.empty((len(positions), hkv, d))
    V = np.empty((len(positions), hkv, d))
    for i, p in enumerate(positions):
        b = physical_block(table_row, int(p), nb)
        o = int(p) % BLOCK_SIZE
        k = to_f64(k_pool[b, :, :, o, :].reshape(hkv, d), kv_dtype)
        v = to_f64(_v_get(v_pool[b, :, :, :, o // 4, :, o % 4]), kv_dtype)
        if quantised(kv_dtype):
            k = k * k_scale[b, :, o].astype(np.float64)[:, None]
            v = v * v_scale[b, :, o].astype(np.float64)[:, None]
        elif channel_scaled(kv_dtype):
            k = k * k_scale.astype(np.float64)
            v = v * v_scale.astype(np.float64)
        K[i], V[i] = k, v
    return K, V


def copy_blocks(pools, pairs):
    """Copy whole physical blocks src -> dst (K, V and, for fp8, both scales).

    This is the data half of copy-on-write ([PA] 三大运行时组件 and the
    copy_on_write snippet): before a write into a block that other sequences
    still reference, its contents go to a fresh private block.  Pairs apply in
    order.
    """
    nb = pools[0].shape[0]
    for arr in pools:
        if arr is None or arr.ndim == 2:      # absent, or static per-channel scales (not per block)
            continue
        assert arr.shape[0] == nb
        for src, dst in pairs:
            arr[dst] = arr[src]


def compact(pools, kv_dtype: str, src_table_row, keep_positions, dst_table_row, num_blocks=None):
    """Apply an eviction keep-set: the token at logical position keep_positions[i]
    of the source table moves to logical position i of the destination table
    (stored bytes of K, V and, for fp8, both scales, all KV heads).

    This is the storage half of evicting tokens ([SO] 4.2 evict_tokens returns
    the cache restricted to the kept indices; [LC] StreamingKVCache keeps
    sinks + window the same way): the kept tokens become a dense prefix of
    fresh blocks, so the cache shrinks to ceil(n / 16) blocks.  Every source is
    read before any destination is written.  Mutates pools in place.
    """
    k_pool, v_pool, k_scale, v_scale = pools
    nb = k_pool.shape[0] if num_blocks is None else num_blocks
    src = [(physical_block(src_table_row, int(p), nb), int(p) % BLOCK_SIZE) for p in keep_positions]
    rows = []
    for b, o in src:
        per_token = k_scale is not None and k_scale.ndim == 3
        rows.append((k_pool[b, :, :, o, :].copy(), v_pool[b, :, :, :, o // 4, :, o % 4].copy(),
                     k_scale[b, :, o].copy() if per_token else None,
                     v_scale[b, :, o].copy() if per_token else None))
    for i, (k, v, ks, vs) in enumerate(rows):
        b, o = physical_block(dst_table_row, i, nb), i % BLOCK_SIZE
        k_pool[b, :, :, o, :] = k
        v_pool[b, :, :, :, o // 4, :, o % 4] = v
        if ks is not None:
            k_scale[b, :, o] = ks
            v_scale[b, :, o] = vs
