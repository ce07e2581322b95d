"""Seeded synthetic inputs for the paged decode workloads (shared by tests, bench and smoke).

This module holds input recipes only -- sequence lengths, block-table layouts,
random K/V/q values -- and none of the method's arithmetic: no slot
computation, no quantisation, no attention.  Both the HIP path and the CPU
oracle consume what it produces.

Workloads (shapes from the model families the pages use; all data N(0, 1)):
  tiny       2 seqs of 35 and 70 tokens, 8 q / 2 KV heads, head_dim 64, fp32,
             16-block pool, seeded permutation tables (or the page's own tables)
  llama3     Llama-3-8B layer decode: 64 seqs, lengths U{512..8192},
             32 q / 8 KV heads, head_dim 128, bf16, shuffled blocks
  fp8long    16 seqs x 32768 tokens, FP8 KV from a bf16 source, seqs 0-3 share
             the 128 blocks of a 2048-token prefix
  streaming  32 seqs, logical length 131072, 4 sinks + 4096 window; only the
             blocks holding kept positions are mapped
  h2o        32 seqs x 8192 tokens, full attention + mass, budget 2048 / recent 512
  llama2     Llama-2-70B stack: 80 layers, 8 seqs x 32768, 64 q / 8 KV heads, bf16
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

BLOCK = 16


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str                  # "f32" | "bf16" | "f16" | "fp8" | "int8" | "fp8_ch" | "int8_ch"
    src_dtype: str                 # dtype of the new K/V rows written into the cache
    q_dtype: str
    seed: int
    lens: Optional[Tuple[int, ...]] = None     # explicit lengths, else len_range
    len_range: Tuple[int, int] = (1, 1)         # inclusive uniform range
    num_sinks: int = 0
    window: int = 0
    budget: int = 0
    recent: int = 0
    mass: bool = False
    num_layers: int = 1
    table_width: Optional[int] = None
    mapped_ranges: Optional[Tuple[Tuple[int, int], ...]] = None  # logical block ranges holding data
    shared_prefix: Tuple[int, int] = (0, 0)     # (sequences, leading blocks) shared by seqs 0..n-1
    extra_blocks: int = 1                       # unreferenced (poisoned) blocks in the pool
    pool_blocks: Optional[int] = None           # fixed pool size (else just enough + extra)
    chunk: int = 0                              # multi-query: query tokens per sequence (its last positions)


WORKLOADS = {
    "tiny": Workload("tiny", 2, 8, 2, 64, "f32", "f32", "f32", 2831, lens=(35, 70), pool_blocks=16),
    "llama3": Workload("llama3", 64, 32, 8, 128, "bf16", "bf16", "bf16", 2832, len_range=(512, 8192)),
    "prefill": Workload("prefill", 4, 32, 8, 128, "bf16", "bf16", "bf16", 2836, lens=(8192,) * 4, chunk=2048),
    "fp8long": Workload("fp8long", 16, 32, 8, 128, "fp8", "bf16", "bf16", 2833, lens=(32768,) * 16,
                        shared_prefix=(4, 128)),
    "int8long": Workload("int8long", 16, 32, 8, 128, "int8", "bf16", "bf16", 2837, lens=(32768,) * 16),
    "fp8chlong": Workload("fp8chlong", 16, 32, 8, 128, "fp8_ch", "bf16", "bf16", 2838, lens=(32768,) * 16),
    "streaming": Workload("streaming", 32, 32, 8, 128, "bf16", "bf16", "bf16", 2834, lens=(131072,) * 32,
                          num_sinks=4, window=4096, table_width=8192,
                          mapped_ranges=((0, 1), (7936, 8192)), extra_blocks=0),
    "h2o": Workload("h2o", 32, 32, 8, 128, "bf16", "bf16", "bf16", 2834, lens=(8192,) * 32, mass=True,
                    budget=2048, recent=512, extra_blocks=0),
    "llama2": Workload("llama2", 8, 64, 8, 128, "bf16", "bf16", "bf16", 2835, lens=(32768,) * 8,
                       num_layers=80, extra_blocks=0),
}


@dataclass
class Layout:
    """Block tables and which logical positions of each sequence carry data."""
    lens: np.ndarray                     # int32 [B]
    tables: np.ndarray                   # int32 [B][W], -1 = unmapped
    num_blocks: int
    data_pos: List[np.ndarray] = field(default_factory=list)   # per seq: positions with data (sorted)
    data_row: List[np.ndarray] = field(default_factory=list)   # per seq: source row of each such position
    write_mask: List[np.ndarray] = field(default_factory=list) # per seq: this seq writes the position
    n_rows: int = 0                      # rows of the K/V source arrays
    unused_blocks: np.ndarray = None     # physical blocks no table references

    @property
    def max_len(self) -> int:
        return int(self.lens.max()) if self.lens.size else 1

    def fill_tokens(self):
        """(seq_ids int32, positions int32, rows int64) of every position some sequence writes."""
        s, p, r = [], [], []
        for i, (pos, row, m) in enumerate(zip(self.data_pos, self.data_row, self.write_mask)):
            s.append(np.full(int(m.sum()), i, dtype=np.int32))
            p.append(pos[m].astype(np.int32))
            r.append(row[m])
        return np.concatenate(s), np.concatenate(p), np.concatenate(r)


def lengths(w: Workload, rng=None) -> np.ndarray:
    if w.lens is not None:
        return np.asarray(w.lens, dtype=np.int32)
    rng = rng or np.random.default_rng(w.seed)
    lo, hi = w.len_range
    return rng.integers(lo, hi + 1, size=w.num_seqs).astype(np.int32)


def make_layout(w: Workload, lens=None, page_tables=None, shuffle=True) -> Layout:
    """Seeded block tables: physical ids drawn from one permutation of the pool
    (shuffle=False hands them out in order, a contiguous placement for comparison)."""
    rng = np.random.default_rng(w.seed)
    lens = lengths(w, rng) if lens is None else np.asarray(lens, dtype=np.int32)
    b = lens.shape[0]
    if b != w.num_seqs:
        raise ValueError(f"{b} lengths for a workload of {w.num_seqs} sequences")
    nblk = [-(-int(n) // BLOCK) for n in lens]
    width = w.table_width or max(nblk)
    mapped = []
    for n in nblk:
        if w.mapped_ranges is None:
            mapped.append(np.arange(n))
        else:
            mapped.append(np.concatenate([np.arange(a, min(e, n)) for a, e in w.mapped_ranges]))
    n_share, share_blocks = w.shared_prefix
    need = sum(len(m) for m in mapped) - max(n_share - 1, 0) * share_blocks
    nb = w.pool_blocks or (need + w.extra_blocks)
    if nb < need:
        raise ValueError("pool too small for the layout")
    perm = rng.permutation(nb).astype(np.int32) if shuffle else np.arange(nb, dtype=np.int32)
    tables = np.full((b, width), -1, dtype=np.int32)
    at = 0
    for s in range(b):
        if page_tables is not None:
            tables[s, : len(page_tables[s])] = page_tables[s]
            continue
        for lb in mapped[s]:
            if s < n_share and s > 0 and lb < share_blocks:
                tables[s, lb] = tables[0, lb]
            else:
                tables[s, lb] = perm[at]
                at += 1
    used = np.unique(tables[tables >= 0])
    unused = np.setdiff1d(np.arange(nb, dtype=np.int32), used)

    lay = Layout(lens=lens, tables=tables, num_blocks=nb, unused_blocks=unused)
    row = 0
    owner_rows = None
    for s in range(b):
        pos = np.concatenate([np.arange(lb * BLOCK, min((lb + 1) * BLOCK, int(lens[s]))) for lb in mapped[s]])
        rows = np.arange(row, row + pos.size, dtype=np.int64)
        mask = np.ones(pos.size, dtype=bool)
        if 0 < s < n_share:
            shared = pos < share_blocks * BLOCK
            rows[shared] = owner_rows[: int(shared.sum())]
            mask[shared] = False
            rows[~shared] = np.arange(row, row + int((~shared).sum()), dtype=np.int64)
            row += int((~shared).sum())
        else:
            row += pos.size
        if s == 0:
            owner_rows = rows
        lay.data_pos.append(pos)
        lay.data_row.append(rows)
        lay.write_mask.append(mask)
    lay.n_rows = row
    return lay


# ---- random values ---------------------------------------------------------------

def _torch():
    import torch
    return torch


def torch_dtype(name: str):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def randn(shape, dtype: str, seed: int, device="cpu"):
    """N(0, 1) values of a storage dtype, from torch's seeded generator on `device`."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch_dtype(dtype))


def kv_source(w: Workload, lay: Layout, layer: int = 0, device="cpu"):
    """(k, v): [n_rows][Hkv][D] source rows of one layer."""
    shape = (lay.n_rows, w.num_kv_heads, w.head_dim)
    base = w.seed * 100 + layer
    return randn(shape, w.src_dtype, 2 * base, device), randn(shape, w.src_dtype, 2 * base + 1, device)


def queries(w: Workload, layer: int = 0, step: int = 0, device="cpu"):
    return randn((w.num_seqs, w.num_q_heads, w.head_dim), w.q_dtype, w.seed * 1000 + 7 * layer + step + 17, device)


def chunk_queries(w: Workload, device="cpu"):
    """Multi-query rows [num_seqs * chunk][Hq][D] (sequence-major) and query_start int32 [num_seqs + 1]."""
    import numpy as np
    q = randn((w.num_seqs * w.chunk, w.num_q_heads, w.head_dim), w.q_dtype, w.seed * 1000 + 29, device)
    start = np.arange(w.num_seqs + 1, dtype=np.int32) * w.chunk
    return q, start


def storage_dtype(kv_dtype: str):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.uint8,
            "int8": torch.int8, "fp8_ch": torch.uint8, "int8_ch": torch.int8}[kv_dtype]


CHANNEL_CODE_MAX = {"fp8_ch": 448.0, "int8_ch": 127.0}


def channel_scales(w: Workload, layer: int = 0):
    """Static per-channel scales (k, v), float32 numpy [Hkv][D], for the per-channel storage formats:
    each channel is given a calibrated range of 4 * 2^u, u ~ U(-1, 1) (the unit-variance source rows
    reach beyond it now and then, and saturate), and scale = range / largest code."""
    import numpy as np
    cmax = CHANNEL_CODE_MAX[w.kv_dtype]
    rng = np.random.default_rng(w.seed * 100 + layer + 51)
    shape = (w.num_kv_heads, w.head_dim)
    k = (4.0 * 2.0 ** rng.uniform(-1, 1, shape) / cmax).astype(np.float32)
    v = (4.0 * 2.0 ** rng.uniform(-1, 1, shape) / cmax).astype(np.float32)
    return k, v
