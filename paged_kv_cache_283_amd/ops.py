"""Python binding of the C ABI: torch tensors in, device pointers and the current HIP stream out.

Argument marshalling only -- every step of the decode path runs in the gfx950
kernels of libpagedkv.so.  Function names and argument meanings are those of
include/pagedkv.h; shapes are read off the tensors.

Storage dtypes: torch.float32 / bfloat16 / float16 pools hold those values;
torch.uint8 or torch.float8_e4m3fn pools hold OCP E4M3FN codes and torch.int8
pools hold INT8 codes.  8-bit pools come with float32 scale tensors: per-token
scales [num_blocks][num_kv_heads][16] (written by the library), or static
per-channel scales [num_kv_heads][head_dim] (given by the caller) -- the scale
tensors' rank tells the two apart.  Pool shapes:
K [num_blocks][num_kv_heads][head_dim/X][16][X] (X = 16 bytes of elements),
V [num_blocks][num_kv_heads][head_dim/(16Y)][16][4][Y][4] (Y = 4 / element bytes);
allocate_pools builds both.
"""
import ctypes
import math

import torch

from . import _lib

BLOCK_SIZE = 16

_FLOAT_CODES = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16, torch.float16: _lib.F16}


def _fp8_dtypes():
    out = {torch.uint8}
    if hasattr(torch, "float8_e4m3fn"):
        out.add(torch.float8_e4m3fn)
    return out


def float_code(dtype: torch.dtype) -> int:
    try:
        return _FLOAT_CODES[dtype]
    except KeyError:
        raise TypeError(f"expected float32, bfloat16 or float16, got {dtype}") from None


def kv_code(dtype: torch.dtype) -> int:
    """Storage code of a pool dtype: float32/bfloat16/float16 values, uint8 (or float8_e4m3fn) E4M3FN
    codes, int8 codes."""
    if dtype in _fp8_dtypes():
        return _lib.FP8_E4M3
    if dtype == torch.int8:
        return _lib.INT8
    return float_code(dtype)


def quantised(dtype: torch.dtype) -> bool:
    """Pools of 8-bit codes (which carry float32 scales)."""
    return kv_code(dtype) in (_lib.FP8_E4M3, _lib.INT8)


_CHANNEL_CODES = {_lib.FP8_E4M3: _lib.FP8_E4M3_CHANNEL, _lib.INT8: _lib.INT8_CHANNEL}


def pool_code(k_pool, k_scale=None, v_scale=None):
    """Storage code of a pool with its scale tensors: an 8-bit pool whose scales are
    [num_kv_heads][head_dim] uses the per-channel format, one with [num_blocks][num_kv_heads][16]
    (or no scales, for calls that take none) the per-token one.  Shapes are checked here since the
    library cannot see array sizes."""
    code = kv_code(k_pool.dtype)
    if code not in _CHANNEL_CODES or k_scale is None:
        return code
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    d = k_pool.shape[2] * k_pool.shape[4]
    if v_scale is None or v_scale.shape != k_scale.shape:
        raise ValueError("k_scale and v_scale must have the same shape")
    _need(k_scale, torch.float32, "k_scale")
    _need(v_scale, torch.float32, "v_scale")
    if tuple(k_scale.shape) == (hkv, d):
        return _CHANNEL_CODES[code]
    if tuple(k_scale.shape) == (nb, hkv, BLOCK_SIZE):
        return code
    raise ValueError(f"scales must be [{nb}][{hkv}][{BLOCK_SIZE}] (per token) or [{hkv}][{d}] (per channel), "
                     f"got {tuple(k_scale.shape)}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must be on a GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Prepared:
    """A library call with every argument already marshalled: calling it re-issues the same
    launch on the same stream (for benchmark and serving loops that repeat a step).  It holds a
    reference to every buffer the binding allocated for the call (a workspace, a slot mapping), so
    their memory stays with this launch for as long as the object lives."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name, args, keep=()):
        self.name = name
        self.fn = getattr(_lib.load(), name)
        self.args = tuple(args)
        self.keep = tuple(keep)

    def __call__(self):
        status = self.fn(*self.args)
        if status != _lib.OK:
            _lib.check(self.name, status)


def _issue(name, args, prepare, stream=None, scratch=()):
    """Run (or prepare) a call.  scratch: tensors this binding allocated for the call; a prepared
    call keeps them, and on a stream other than the current one they are recorded on it, so the
    caching allocator does not hand their memory out again before the call has run."""
    if prepare:
        return Prepared(name, args, scratch)
    _lib.call(name, *args)
    if stream is not None and scratch and stream != torch.cuda.current_stream(stream.device):
        for t in scratch:
            t.record_stream(stream)
    return None


def k_chunk(dtype: torch.dtype) -> int:
    """Elements per 16-byte chunk of the K pool layout [NB][Hkv][D/X][16][X]."""
    return 16 // torch.empty((), dtype=dtype).element_size()


def k_pool_shape(num_blocks, num_kv_heads, head_dim, dtype):
    x = k_chunk(dtype)
    return (num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x)


def v_chunk_dims(dtype: torch.dtype) -> int:
    """Dims (16 apart) per 16-byte chunk of the V pool layout [NB][Hkv][D/(16Y)][16][4][Y][4]."""
    return 4 // torch.empty((), dtype=dtype).element_size()


def v_pool_shape(num_blocks, num_kv_heads, head_dim, dtype):
    y = v_chunk_dims(dtype)
    if head_dim % (16 * y):
        raise ValueError(f"head_dim {head_dim} is not a multiple of {16 * y}")
    return (num_blocks, num_kv_heads, head_dim // (16 * y), BLOCK_SIZE, 4, y, 4)


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def paged_decode_slots(block_tables, context_lens, num_blocks, slot_mapping=None, stream=None, prepare=False):
    """int64 slot of every sequence's newest token (position context_lens - 1); -1 where unusable."""
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    b = context_lens.shape[0]
    made = ()
    if slot_mapping is None:
        slot_mapping = torch.empty(b, dtype=torch.int64, device=context_lens.device)
        made = (slot_mapping,)
    p = _issue("paged_decode_slots", (_ptr(block_tables), block_tables.shape[1], _ptr(context_lens), b,
                                      int(num_blocks), BLOCK_SIZE, _ptr(slot_mapping), _stream(stream)), prepare,
               scratch=made)
    return p if prepare else slot_mapping


def paged_token_slots(block_tables, seq_ids, positions, num_blocks, slot_mapping=None, stream=None):
    """int64 slots of (seq_ids[t], positions[t]) tokens; -1 where unusable."""
    _need(block_tables, torch.int32, "block_tables")
    _need(seq_ids, torch.int32, "seq_ids")
    _need(positions, torch.int32, "positions")
    t = seq_ids.shape[0]
    if positions.shape[0] != t:
        raise ValueError("seq_ids and positions must have the same length")
    if slot_mapping is None:
        slot_mapping = torch.empty(t, dtype=torch.int64, device=seq_ids.device)
    _lib.call("paged_token_slots", _ptr(block_tables), block_tables.shape[1], block_tables.shape[0],
              _ptr(seq_ids), _ptr(positions), t, int(num_blocks), BLOCK_SIZE, _ptr(slot_mapping), _stream(stream))
    return slot_mapping


def paged_kv_write(k_new, v_new, k_pool, v_pool, slot_mapping, k_scale=None, v_scale=None, stream=None,
                   prepare=False):
    """Store [T][Hkv][D] new K/V rows at their slots (8-bit pools quantise per row, or per channel
    with the given static scales)."""
    _need(slot_mapping, torch.int64, "slot_mapping")
    t, hkv, d = k_new.shape
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must match")
    nb = k_pool.shape[0]
    if (tuple(k_pool.shape) != k_pool_shape(nb, hkv, d, k_pool.dtype)
            or tuple(v_pool.shape) != v_pool_shape(nb, hkv, d, v_pool.dtype)):
        raise ValueError(f"pools must be {k_pool_shape(nb, hkv, d, k_pool.dtype)} (K) and "
                         f"{v_pool_shape(nb, hkv, d, v_pool.dtype)} (V)")
    if slot_mapping.shape[0] != t:
        raise ValueError("slot_mapping must have one entry per token")
    return _issue("paged_kv_write", (_ptr(k_new), _ptr(v_new), float_code(k_new.dtype), _ptr(k_pool),
                                     _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale),
                                     _ptr(slot_mapping), t, nb, hkv, d, BLOCK_SIZE, _stream(stream)), prepare)


def paged_kv_append(k_new, v_new, k_pool, v_pool, block_tables, context_lens, k_scale=None, v_scale=None,
                    stream=None, prepare=False):
    """Decode-step write: token s of k_new/v_new [B][Hkv][D] to position context_lens[s] - 1 of sequence s."""
    b, hkv, d = k_new.shape
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must match")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    nb = k_pool.shape[0]
    if (tuple(k_pool.shape) != k_pool_shape(nb, hkv, d, k_pool.dtype)
            or tuple(v_pool.shape) != v_pool_shape(nb, hkv, d, v_pool.dtype)):
        raise ValueError("pool shapes do not match k_new")
    if context_lens.shape[0] != b or block_tables.shape[0] != b:
        raise ValueError("one table row and one length per sequence")
    return _issue("paged_kv_append", (_ptr(k_new), _ptr(v_new), float_code(k_new.dtype), _ptr(k_pool), _ptr(v_pool),
                                      _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale), _ptr(block_tables),
                                      block_tables.shape[1], _ptr(context_lens), b, nb, hkv, d, BLOCK_SIZE,
                                      _stream(stream)), prepare)


def allocate_pools(num_blocks, num_kv_heads, head_dim, kv_dtype=torch.bfloat16, device="cuda", fill_byte=None,
                   channel_scales=None):
    """(k_pool, v_pool, k_scale, v_scale) in the library's layout.  Scales are None for float pools;
    for 8-bit pools (torch.uint8 / float8_e4m3fn / int8) they are per-token scale tensors, or, when
    channel_scales = (k_channel, v_channel) is given, those [num_kv_heads][head_dim] float32 tensors
    (copied to the device).  fill_byte sets every pool and per-token scale byte (0xFF = NaN everywhere)."""
    k = torch.empty(k_pool_shape(num_blocks, num_kv_heads, head_dim, kv_dtype), dtype=kv_dtype, device=device)
    v = torch.empty(v_pool_shape(num_blocks, num_kv_heads, head_dim, kv_dtype), dtype=kv_dtype, device=device)
    ks = vs = None
    if channel_scales is not None:
        if not quantised(kv_dtype):
            raise ValueError("per-channel scales need an 8-bit pool dtype")
        ks, vs = (torch.as_tensor(c, dtype=torch.float32).to(device).contiguous() for c in channel_scales)
        if tuple(ks.shape) != (num_kv_heads, head_dim) or tuple(vs.shape) != (num_kv_heads, head_dim):
            raise ValueError(f"channel scales must be [{num_kv_heads}][{head_dim}]")
    elif quantised(kv_dtype):
        ks = torch.empty((num_blocks, num_kv_heads, BLOCK_SIZE), dtype=torch.float32, device=device)
        vs = torch.empty((num_blocks, num_kv_heads, BLOCK_SIZE), dtype=torch.float32, device=device)
    if fill_byte is not None:
        for t in (k, v) if channel_scales is not None else (k, v, ks, vs):
            if t is not None:
                t.view(torch.uint8).fill_(fill_byte)
    return k, v, ks, vs


def write_positions(block_tables, seq_ids, positions, k_rows, v_rows, k_pool, v_pool, k_scale=None, v_scale=None,
                    stream=None):
    """Prefill-style write: token t = (seq_ids[t], positions[t]) with rows k_rows[t], v_rows[t]
    (slots looked up on the GPU, then one cache write)."""
    slots = paged_token_slots(block_tables, seq_ids, positions, k_pool.shape[0], stream=stream)
    paged_kv_write(k_rows, v_rows, k_pool, v_pool, slots, k_scale, v_scale, stream=stream)
    return slots


def workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, num_sinks=0, window=0, want_mass=False):
    return int(_lib.load().paged_decode_attn_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                                             num_sinks, window, int(bool(want_mass))))


def alloc_workspace(num_seqs, num_q_heads, head_dim, max_context_len, num_sinks=0, window=0,
                    want_mass=False, device="cuda"):
    n = workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, num_sinks, window, want_mass)
    # torch's caching allocator returns 256-byte aligned blocks.
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def paged_decode_attn(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale=None,
                      k_scale=None, v_scale=None, num_sinks=0, window=0, attn_mass=None, workspace=None,
                      stream=None, prepare=False):
    """Decode attention of q [B][Hq][D] over the paged pools into out [B][Hq][D].

    attn_mass (float32 [B][>= max_context_len]) receives += the H2O mass of the kept positions.
    """
    b, hq, d = q.shape
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    if tuple(out.shape) != (b, hq, d):
        raise ValueError("out must have q's shape")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mass_stride = 0
    if attn_mass is not None:
        _need(attn_mass, torch.float32, "attn_mass")
        mass_stride = attn_mass.shape[1]
    made = ()
    if workspace is None:
        workspace = alloc_workspace(b, hq, d, max_context_len, num_sinks, window, attn_mass is not None, q.device)
        made = (workspace,)
    args = (_ptr(out), float_code(out.dtype), _ptr(q), float_code(q.dtype), _ptr(k_pool), _ptr(v_pool),
            _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), int(max_context_len), b, nb, hq, hkv, d, BLOCK_SIZE, float(scale), int(num_sinks),
            int(window), _ptr(attn_mass), mass_stride, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    p = _issue("paged_decode_attn", args, prepare, stream, made)
    return p if prepare else out


def paged_decode_attn_noalloc(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale=None,
                              k_scale=None, v_scale=None, num_sinks=0, window=0, attn_mass=None, stream=None,
                              prepare=False):
    """paged_decode_attn with the library's fixed per-device workspace: this call allocates nothing
    (for graph capture and loops that must not allocate).  Calls that overlap on one GPU race."""
    b, hq, d = q.shape
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    if tuple(out.shape) != (b, hq, d):
        raise ValueError("out must have q's shape")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mass_stride = 0
    if attn_mass is not None:
        _need(attn_mass, torch.float32, "attn_mass")
        mass_stride = attn_mass.shape[1]
    args = (_ptr(out), float_code(out.dtype), _ptr(q), float_code(q.dtype), _ptr(k_pool), _ptr(v_pool),
            _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), int(max_context_len), b, nb, hq, hkv, d, BLOCK_SIZE, float(scale), int(num_sinks),
            int(window), _ptr(attn_mass), mass_stride, _stream(stream))
    p = _issue("paged_decode_attn_noalloc", args, prepare)
    return p if prepare else out


def paged_decode_append_attn(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, max_context_len,
                             scale=None, k_scale=None, v_scale=None, num_sinks=0, window=0, attn_mass=None,
                             workspace=None, stream=None, prepare=False):
    """One decode step: the new token k_new/v_new [B][Hkv][D] goes to position context_lens[s] - 1 of
    sequence s, then q [B][Hq][D] attends over the paged pools into out (paged_kv_append followed by
    paged_decode_attn, in one attention launch for 16-bit and f32 pools)."""
    b, hq, d = q.shape
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    if tuple(out.shape) != (b, hq, d):
        raise ValueError("out must have q's shape")
    if tuple(k_new.shape) != (b, hkv, d) or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim] of one dtype")
    if (tuple(k_pool.shape) != k_pool_shape(nb, hkv, d, k_pool.dtype)
            or tuple(v_pool.shape) != v_pool_shape(nb, hkv, d, v_pool.dtype)):
        raise ValueError("pool shapes do not match k_new")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if context_lens.shape[0] != b or block_tables.shape[0] != b:
        raise ValueError("one table row and one length per sequence")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mass_stride = 0
    if attn_mass is not None:
        _need(attn_mass, torch.float32, "attn_mass")
        mass_stride = attn_mass.shape[1]
    made = ()
    if workspace is None:
        workspace = alloc_workspace(b, hq, d, max_context_len, num_sinks, window, attn_mass is not None, q.device)
        made = (workspace,)
    args = (_ptr(out), float_code(out.dtype), _ptr(q), float_code(q.dtype), _ptr(k_new), _ptr(v_new),
            float_code(k_new.dtype), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
            pool_code(k_pool, k_scale, v_scale), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
            int(max_context_len), b, nb, hq, hkv, d, BLOCK_SIZE, float(scale), int(num_sinks), int(window),
            _ptr(attn_mass), mass_stride, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    p = _issue("paged_decode_append_attn", args, prepare, stream, made)
    return p if prepare else out


def compact_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, want_mass=False):
    return int(_lib.load().paged_decode_attn_compact_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                                                     int(bool(want_mass))))


def paged_decode_attn_compact(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len, keep_idx,
                              keep_count, dst_tables, k_new=None, v_new=None, scale=None, k_scale=None, v_scale=None,
                              attn_mass_src=None, attn_mass=None, workspace=None, stream=None, prepare=False):
    """A decode step that applies an eviction keep-set in the same pass: q [B][Hq][D] attends the kept
    positions keep_idx[s][:keep_count[s]] of each sequence (plus, with k_new/v_new [B][Hkv][D], the new
    token stored at position context_lens[s] - 1), and those tokens move, in order, to logical positions
    0.. of dst_tables[s] (16-bit pools with q of the pool's dtype, or 8-bit pools with their scales and
    bf16/f16 q; k_new/v_new in q's dtype).  With attn_mass (float32 [B][>= max_len],
    the compacted H2O score rows) and attn_mass_src (the rows before the step): entry i gets the moved
    token's source score plus this step's mass."""
    b, hq, d = q.shape
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    if tuple(out.shape) != (b, hq, d):
        raise ValueError("out must have q's shape")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        if tuple(k_new.shape) != (b, hkv, d) or v_new.shape != k_new.shape or k_new.dtype != q.dtype \
                or v_new.dtype != q.dtype:
            raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim] of q's dtype")
    for t, name in ((block_tables, "block_tables"), (context_lens, "context_lens"), (keep_idx, "keep_idx"),
                    (keep_count, "keep_count"), (dst_tables, "dst_tables")):
        _need(t, torch.int32, name)
    if not (context_lens.shape[0] == block_tables.shape[0] == keep_idx.shape[0] == keep_count.shape[0]
            == dst_tables.shape[0] == b):
        raise ValueError("one table row, length, keep list and destination row per sequence")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if (attn_mass is None) != (attn_mass_src is None):
        raise ValueError("give both attn_mass and attn_mass_src, or neither")
    src_stride = dst_stride = 0
    if attn_mass is not None:
        _need(attn_mass, torch.float32, "attn_mass")
        _need(attn_mass_src, torch.float32, "attn_mass_src")
        src_stride, dst_stride = attn_mass_src.shape[1], attn_mass.shape[1]
    made = ()
    if workspace is None:
        n = compact_workspace_size(b, hq, d, max_context_len, attn_mass is not None)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
        made = (workspace,)
    args = (_ptr(out), float_code(out.dtype), _ptr(q), float_code(q.dtype), _ptr(k_new), _ptr(v_new),
            _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale),
            _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), int(max_context_len), _ptr(keep_idx), keep_idx.shape[1], _ptr(keep_count),
            _ptr(dst_tables), dst_tables.shape[1], b, nb, hq, hkv, d, BLOCK_SIZE, float(scale),
            _ptr(attn_mass_src), src_stride, _ptr(attn_mass), dst_stride, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    p = _issue("paged_decode_attn_compact", args, prepare, stream, made)
    return p if prepare else out


def paged_prefill_attn(out, q, k_pool, v_pool, block_tables, context_lens, query_start, max_context_len,
                       max_query_len, scale=None, k_scale=None, v_scale=None, stream=None, prepare=False):
    """Causal multi-query attention: q/out [T][Hq][D]; sequence s owns rows
    [query_start[s], query_start[s+1]), its last positions of a context of context_lens[s] tokens."""
    t, hq, d = q.shape
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    if tuple(out.shape) != (t, hq, d):
        raise ValueError("out must have q's shape")
    for x, n in ((block_tables, "block_tables"), (context_lens, "context_lens"), (query_start, "query_start")):
        _need(x, torch.int32, n)
    b = context_lens.shape[0]
    if query_start.shape[0] != b + 1 or block_tables.shape[0] != b:
        raise ValueError("query_start needs num_seqs + 1 entries and block_tables one row per sequence")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    args = (_ptr(out), float_code(out.dtype), _ptr(q), float_code(q.dtype), _ptr(k_pool), _ptr(v_pool),
            _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), _ptr(query_start), t, int(max_context_len), int(max_query_len), b, nb, hq, hkv, d,
            BLOCK_SIZE, float(scale), _stream(stream))
    return _issue("paged_prefill_attn", args, prepare)


def _host_ptr(t):
    if t is None:
        return None
    if t.is_cuda or not t.is_pinned():
        raise ValueError("host arenas must be pinned CPU tensors (pin_memory=True)")
    return ctypes.c_void_p(t.data_ptr())


def allocate_host_arena(num_slots, num_kv_heads, head_dim, kv_dtype=torch.bfloat16, per_token_scales=True):
    """Pinned host (k, v, k_scale, v_scale) mirroring the pool layout with num_slots blocks (scale rows
    only for 8-bit pools with per-token scales; per-channel scales stay on the device)."""
    k = torch.empty(k_pool_shape(num_slots, num_kv_heads, head_dim, kv_dtype), dtype=kv_dtype, pin_memory=True)
    v = torch.empty(v_pool_shape(num_slots, num_kv_heads, head_dim, kv_dtype), dtype=kv_dtype, pin_memory=True)
    ks = vs = None
    if quantised(kv_dtype) and per_token_scales:
        ks = torch.empty((num_slots, num_kv_heads, BLOCK_SIZE), dtype=torch.float32, pin_memory=True)
        vs = torch.empty((num_slots, num_kv_heads, BLOCK_SIZE), dtype=torch.float32, pin_memory=True)
    return k, v, ks, vs


def kv_swap(pools, arena, block_slot_pairs, to_host, stream=None, prepare=False):
    """Copy pool blocks to host slots (to_host=True) or back, for int32 pairs [n][2] {block, slot}."""
    k, v, ks, vs = pools
    hk, hv, hks, hvs = arena
    _need(block_slot_pairs, torch.int32, "block_slot_pairs")
    if hk.dtype != k.dtype or tuple(hk.shape[1:]) != tuple(k.shape[1:]) or tuple(hv.shape[1:]) != tuple(v.shape[1:]):
        raise ValueError("the host arena must mirror the pool layout")
    nb, hkv = k.shape[0], k.shape[1]
    d = k.shape[2] * k.shape[4]
    args = (_ptr(k), _ptr(v), _ptr(ks), _ptr(vs), pool_code(k, ks, vs), _host_ptr(hk), _host_ptr(hv), _host_ptr(hks),
            _host_ptr(hvs), _ptr(block_slot_pairs), block_slot_pairs.shape[0], nb, hk.shape[0], hkv, d, BLOCK_SIZE,
            1 if to_host else 0, _stream(stream))
    return _issue("kv_swap", args, prepare)


def kv_block_copy(k_pool, v_pool, block_pairs, k_scale=None, v_scale=None, stream=None):
    """Copy whole blocks per int32 [n][2] {src, dst} pair (the data half of copy-on-write)."""
    _need(block_pairs, torch.int32, "block_pairs")
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    d = k_pool.shape[2] * k_pool.shape[4]
    _lib.call("kv_block_copy", _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale),
              _ptr(block_pairs), block_pairs.shape[0], nb, hkv, d, BLOCK_SIZE, _stream(stream))


def h2o_select(scores, kv_lens, max_kv_len, budget, recent, keep_idx=None, keep_count=None, stream=None):
    """H2O keep-set per sequence: (keep_idx int32 [B][budget] ascending, -1 padded; keep_count int32 [B])."""
    _need(scores, torch.float32, "scores")
    _need(kv_lens, torch.int32, "kv_lens")
    b = kv_lens.shape[0]
    if keep_idx is None:
        keep_idx = torch.empty((b, budget), dtype=torch.int32, device=scores.device)
    if keep_count is None:
        keep_count = torch.empty(b, dtype=torch.int32, device=scores.device)
    _lib.call("h2o_select", _ptr(scores), scores.shape[1], _ptr(kv_lens), b, int(max_kv_len), int(budget),
              int(recent), _ptr(keep_idx), _ptr(keep_count), _stream(stream))
    return keep_idx, keep_count


_CANDIDATES = {"rest": _lib.CAND_REST, "all": _lib.CAND_ALL}


def keep_select(scores, kv_lens, max_kv_len, num_sinks, recent, heavy, candidates="rest", keep_idx=None,
                keep_count=None, stream=None):
    """Eviction keep-set per sequence (kv_keep_select): forced sinks + recent window united with the
    `heavy` top scores of the non-forced ("rest") or of all ("all") positions.
    Returns (keep_idx int32 [B][stride] ascending, -1 padded; keep_count int32 [B])."""
    _need(scores, torch.float32, "scores")
    _need(kv_lens, torch.int32, "kv_lens")
    b = kv_lens.shape[0]
    if keep_idx is None:
        width = max(1, min(int(num_sinks) + int(recent) + int(heavy), int(max_kv_len)))
        keep_idx = torch.empty((b, width), dtype=torch.int32, device=scores.device)
    if keep_count is None:
        keep_count = torch.empty(b, dtype=torch.int32, device=scores.device)
    _lib.call("kv_keep_select", _ptr(scores), scores.shape[1], _ptr(kv_lens), b, int(max_kv_len), int(num_sinks),
              int(recent), int(heavy), _CANDIDATES[candidates], _ptr(keep_idx), keep_idx.shape[1], _ptr(keep_count),
              _stream(stream))
    return keep_idx, keep_count


def kv_compact(k_pool, v_pool, src_tables, dst_tables, keep_idx, keep_count, k_scale=None, v_scale=None,
               stream=None):
    """Move each sequence's kept tokens (keep_idx, keep_count) from their slots under src_tables to
    positions 0..n-1 under dst_tables (fresh blocks)."""
    for t, n in ((src_tables, "src_tables"), (dst_tables, "dst_tables"), (keep_idx, "keep_idx"),
                 (keep_count, "keep_count")):
        _need(t, torch.int32, n)
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    d = k_pool.shape[2] * k_pool.shape[4]
    b = keep_count.shape[0]
    if src_tables.shape[0] != b or dst_tables.shape[0] != b or keep_idx.shape[0] != b:
        raise ValueError("tables, keep_idx and keep_count must have one row per sequence")
    _lib.call("kv_compact", _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), pool_code(k_pool, k_scale, v_scale),
              _ptr(src_tables), src_tables.shape[1], _ptr(dst_tables), dst_tables.shape[1], _ptr(keep_idx),
              keep_idx.shape[1], _ptr(keep_count), b, nb, hkv, d, BLOCK_SIZE, _stream(stream))


def timing_begin(capacity):
    _lib.call("pkv_timing_begin", int(capacity))


def timing_end(capacity):
    buf = (ctypes.c_float * capacity)()
    n = _lib.load().pkv_timing_end(buf, capacity)
    if n < 0:
        _lib.check("pkv_timing_end", _lib.EDEVICE)
    return [buf[i] for i in range(n)]


def probe_read(src, sink, stream=None):
    _lib.call("pkv_probe_read", _ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream))


def probe_copy(dst, src, stream=None):
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _lib.call("pkv_probe_copy", _ptr(dst), _ptr(src), n, _stream(stream))
