"""Host-side block allocator with reference counts and copy-on-write.

Page "KV Cache 与 PagedAttention：显存复用与长上下文推理" (plumephp.com/ai-kv-cache-paged-attention):
  "PagedAttention 的设计"  -- fixed 16-token blocks; one block table per request
                             mapping logical to physical blocks; free blocks in
                             one global pool; only a sequence's last block is
                             partly filled.
  "三大运行时组件"          -- the block allocator, the per-request table, and
                             reference counts with copy-on-write: a block shared
                             by several requests has its count raised, and a
                             write into a shared block first copies it.
  "共享场景的价值"          -- parallel samples of one prompt share its prefix;
                             beam search shares until the fork.
  copy_on_write snippet    -- new blocks start with refcount 1; the old block's
                             count drops by one; the table entry is swapped.

The tables here hold block ids; the GPU-side data copy of a COW is the
kv_block_copy entry point, run by the caller with the (src, dst) pairs these
methods return, before writing into the new block.
"""
import hashlib
from collections import OrderedDict, deque

import numpy as np

BLOCK_SIZE = 16


class OutOfBlocks(RuntimeError):
    """The shared pool has no free block left."""


class HostBlockStore:
    """Slots of a pinned host arena that hold swapped-out blocks (one slot per block)."""

    def __init__(self, num_slots: int):
        if num_slots < 1:
            raise ValueError("num_slots must be >= 1")
        self.num_slots = num_slots
        self._free = deque(range(num_slots))

    @property
    def num_free(self) -> int:
        return len(self._free)

    def alloc(self, n: int):
        if n > len(self._free):
            raise OutOfBlocks(f"host arena: {n} slots needed, {len(self._free)} free")
        return [self._free.popleft() for _ in range(n)]

    def release(self, slots) -> None:
        self._free.extend(slots)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        if block_size != BLOCK_SIZE:
            raise ValueError("block_size must be 16")
        if num_blocks < 1:
            raise ValueError("num_blocks must be >= 1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.refcount = np.zeros(num_blocks, dtype=np.int32)
        self._free = deque(range(num_blocks))
        self.tables = {}          # seq id -> list of physical block ids
        self.lens = {}            # seq id -> tokens held
        self.swapped = {}         # seq id -> (host slots, tokens held) while swapped out
        self.cow_copies = 0
        self._pending = []        # source blocks of compactions not yet released

    # ---- pool ---------------------------------------------------------------
    def _alloc(self) -> int:
        if not self._free:
            raise OutOfBlocks(f"all {self.num_blocks} blocks are in use")
        b = self._free.popleft()
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise RuntimeError(f"block {b} released more often than referenced")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self._free.append(b)

    @property
    def num_free(self) -> int:
        return len(self._free)

    # ---- sequences ------------------------------------------------------------
    def add_sequence(self, seq, num_tokens: int = 0):
        """Register a sequence holding num_tokens tokens; returns its block table."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        need = -(-num_tokens // self.block_size)
        if need > self.num_free:
            raise OutOfBlocks(f"sequence of {num_tokens} tokens needs {need} blocks, {self.num_free} free")
        self.tables[seq] = [self._alloc() for _ in range(need)]
        self.lens[seq] = num_tokens
        return list(self.tables[seq])

    def fork(self, parent, child):
        """child shares every block of parent (refcounts + 1), as parallel samples of one prompt do."""
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        for b in self.tables[parent]:
            self.refcount[b] += 1
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        return list(self.tables[child])

    def copy_on_write(self, seq, logical_idx: int):
        """Give seq a private copy of its logical block if the block is shared.

        Returns (src, dst) for the device copy, or None if the block is not shared.
        """
        old = self.tables[seq][logical_idx]
        if self.refcount[old] <= 1:
            return None
        new = self._alloc()
        self.refcount[old] -= 1
        self.tables[seq][logical_idx] = new
        self.cow_copies += 1
        return (old, new)

    def append_tokens(self, seq, n: int = 1):
        """Reserve slots for n new tokens of seq.

        Returns (slots int64 [n], copies): copies are (src, dst) block pairs that
        must be copied on the device before the new tokens are written, because
        the block receiving them was shared.
        """
        slots = np.empty(n, dtype=np.int64)
        copies = []
        table = self.tables[seq]
        for i in range(n):
            pos = self.lens[seq]
            lb = pos // self.block_size
            if lb == len(table):
                table.append(self._alloc())
            else:
                pair = self.copy_on_write(seq, lb)
                if pair is not None:
                    copies.append(pair)
            slots[i] = table[lb] * self.block_size + pos % self.block_size
            self.lens[seq] = pos + 1
        return slots, copies

    def compact(self, seq, num_kept: int):
        """Give seq fresh blocks for a dense prefix of num_kept tokens (eviction).

        Returns (old_table, new_table): the caller enqueues kv_compact from
        old_table to new_table with the keep-set, or lets the next decode step
        move the tokens (paged_decode_attn_compact over old_table: append the
        step's token first, then compact to the kept count + 1; the kept tokens
        and the new one land in new_table).  The old blocks are not
        released yet: they stay referenced until release_compacted(), so the
        fresh blocks of another sequence compacted before that call are never
        one of them, and one batched kv_compact over every sequence compacted
        so far has no destination slot that is also a source slot.  Call
        release_compacted() once those kv_compact calls are enqueued; device
        work that writes the released blocks must come after them on the same
        stream.
        """
        if num_kept < 0 or num_kept > self.lens[seq]:
            raise ValueError(f"num_kept {num_kept} outside [0, {self.lens[seq]}]")
        need = -(-num_kept // self.block_size)
        if need > self.num_free:
            raise OutOfBlocks(f"compaction to {num_kept} tokens needs {need} blocks, {self.num_free} free")
        old = self.tables[seq]
        new = [self._alloc() for _ in range(need)]
        self._pending.extend(old)
        self.tables[seq] = new
        self.lens[seq] = num_kept
        return list(old), list(new)

    def release_compacted(self) -> int:
        """Release the source blocks of every compact() since the last call (shared ones only lose
        that sequence's reference); returns how many references were dropped."""
        n = len(self._pending)
        for b in self._pending:
            self._release(b)
        self._pending = []
        return n

    def swap_out(self, seq, store: HostBlockStore):
        """Move seq out of the pool ([PA] 三大运行时组件: blocks can be swapped out to CPU RAM).

        Returns pairs (block, host slot) for kv_swap(..., to_host=True).  The
        pool blocks are released here (a shared block only loses this
        reference); device work that writes them must be enqueued after the
        swap on the same stream.
        """
        table = self.tables[seq]
        slots = store.alloc(len(table))
        pairs = list(zip(table, slots))
        for b in table:
            self._release(b)
        del self.tables[seq]
        self.swapped[seq] = (slots, self.lens.pop(seq))
        return pairs

    def swap_in(self, seq, store: HostBlockStore):
        """Bring a swapped-out seq back into fresh blocks.

        Returns pairs (block, host slot) for kv_swap(..., to_host=False); the
        host slots return to the store (later swaps that reuse them are
        ordered after this one on the same stream).
        """
        slots, n_tok = self.swapped[seq]
        if len(slots) > self.num_free:
            raise OutOfBlocks(f"swap-in of {len(slots)} blocks, {self.num_free} free")
        del self.swapped[seq]
        table = [self._alloc() for _ in slots]
        self.tables[seq] = table
        self.lens[seq] = n_tok
        store.release(slots)
        return list(zip(table, slots))

    def free(self, seq) -> None:
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lens[seq]

    # ---- views for the kernels --------------------------------------------------
    def slot_mapping(self, seq, positions) -> np.ndarray:
        """int64 slots of the given logical positions of seq."""
        table = self.tables[seq]
        pos = np.asarray(positions, dtype=np.int64)
        if pos.size and (pos.min() < 0 or pos.max() >= self.lens[seq]):
            raise IndexError("position outside the sequence")
        blocks = np.asarray(table, dtype=np.int64)[pos // self.block_size]
        return blocks * self.block_size + pos % self.block_size

    def block_tables(self, seqs, width=None) -> np.ndarray:
        """int32 [len(seqs)][width] tables, -1 beyond each sequence's blocks."""
        width = width if width is not None else max((len(self.tables[s]) for s in seqs), default=0)
        out = np.full((len(seqs), max(width, 1)), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.tables[s]
            if len(t) > width:
                raise ValueError(f"sequence {s} has {len(t)} blocks > width {width}")
            out[i, : len(t)] = t
        return out

    def context_lens(self, seqs) -> np.ndarray:
        return np.array([self.lens[s] for s in seqs], dtype=np.int32)

    def stats(self) -> dict:
        used = self.num_blocks - self.num_free
        return {"free_blocks": self.num_free, "used_blocks": used,
                "shared_blocks": int((self.refcount > 1).sum()), "cow_copies": self.cow_copies,
                "internal_fragmentation_tokens": int(sum(len(t) * self.block_size - self.lens[s]
                                                         for s, t in self.tables.items()))}


class PrefixCachingBlockManager(BlockManager):
    """BlockManager whose full blocks are also found by the token prefix they complete.

    Page "KV Cache 与 PagedAttention：显存复用与长上下文推理", section "共享场景的价值": requests
    that share a system prompt, a RAG document or a conversation history can
    share its KV; with vLLM-style prefix caching a new request is compared,
    block by block, with the prefixes already cached, and the part that
    matches needs no prefill; cached blocks are shared physically, with
    reference counts and copy-on-write.  Since matching goes by prefix, the
    page recommends placing reused text at the start of the prompt.

    Design: each full block is keyed by a chained digest, hash(parent key,
    its 16 token ids), so a key names the whole prefix up to the end of that
    block.  Blocks are registered once their KV is written (`commit`).  A
    cached block whose last user frees it keeps its contents and its key and
    waits in an LRU list; allocation takes never-cached free blocks first and
    then evicts the least recently freed cached block.  Only full blocks are
    shared, and writes only ever go to a sequence's partial last block, so a
    shared block is never written.

    A sequence's blocks are keyed only while the token id of every position
    it holds is known.  One that loses that (added with tokens but no ids,
    extended without ids, or compacted by eviction, after which its
    positions are no longer a prefix of any prompt) becomes uncacheable:
    commit() registers nothing more for it, and its blocks registered before
    keep their (correct) keys.
    """

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        super().__init__(num_blocks, block_size)
        self._by_key = {}               # prefix key -> block
        self._key_of = {}               # block -> prefix key
        self._evictable = OrderedDict()  # cached blocks with refcount 0, least recently freed first
        self.tokens = {}                # seq -> token ids held, None once unknown (uncacheable)
        self.hits = 0                   # blocks reused from the cache
        self.evictions = 0

    @staticmethod
    def block_key(parent, tokens) -> bytes:
        """Chained key of a full block: digest of the parent key and the block's token ids."""
        h = hashlib.blake2b(digest_size=16)
        h.update(parent if parent is not None else b"\x00")
        h.update(np.asarray(tokens, dtype=np.int64).tobytes())
        return h.digest()

    def _keys(self, tokens):
        keys, parent = [], None
        for i in range(len(tokens) // self.block_size):
            parent = self.block_key(parent, tokens[i * self.block_size:(i + 1) * self.block_size])
            keys.append(parent)
        return keys

    # ---- pool: free blocks first, then the least recently freed cached block
    def _alloc(self) -> int:
        if not self._free and self._evictable:
            b, _ = self._evictable.popitem(last=False)
            del self._by_key[self._key_of.pop(b)]
            self._free.append(b)
            self.evictions += 1
        return super()._alloc()

    def _release(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise RuntimeError(f"block {b} released more often than referenced")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            if b in self._key_of:
                self._evictable[b] = None       # keep contents and key; reusable until evicted
            else:
                self._free.append(b)

    @property
    def num_free(self) -> int:
        return len(self._free) + len(self._evictable)

    @property
    def num_cached(self) -> int:
        return len(self._key_of)

    # ---- sequences ------------------------------------------------------------
    def match_prefix(self, tokens):
        """Cached blocks holding the longest block-aligned prefix of tokens."""
        out = []
        for k in self._keys(tokens):
            b = self._by_key.get(k)
            if b is None:
                break
            out.append(b)
        return out

    def add_cached_sequence(self, seq, tokens):
        """Register seq with its prompt tokens, reusing cached blocks for the longest cached prefix.

        Returns (table, num_cached_tokens): the KV of positions < num_cached_tokens
        is already in the pool; the caller prefills only the rest.  At least the
        last prompt token is always left to compute (its query is needed).
        """
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        tokens = list(tokens)
        hits = self.match_prefix(tokens)
        if hits and len(hits) * self.block_size >= len(tokens):
            hits = hits[:-1]
        need = -(-len(tokens) // self.block_size) - len(hits)
        for b in hits:                       # take the hits first so allocation cannot evict them
            if self.refcount[b] == 0:
                del self._evictable[b]
            self.refcount[b] += 1
        if need > self.num_free:
            for b in hits:
                self._release(b)
            raise OutOfBlocks(f"sequence of {len(tokens)} tokens needs {need} new blocks, {self.num_free} free")
        self.tables[seq] = hits + [self._alloc() for _ in range(need)]
        self.lens[seq] = len(tokens)
        self.tokens[seq] = tokens
        self.hits += len(hits)
        return list(self.tables[seq]), len(hits) * self.block_size

    def add_sequence(self, seq, num_tokens: int = 0):
        table = super().add_sequence(seq, num_tokens)
        self.tokens[seq] = [] if num_tokens == 0 else None    # ids of a non-empty start are unknown
        return table

    def commit(self, seq):
        """Make seq's full blocks findable (call once their KV has been written).  Does nothing for a
        sequence whose token ids are not all known."""
        table = self.tables[seq]
        tokens = self.tokens.get(seq)
        if tokens is None or len(tokens) != self.lens[seq]:
            return
        for i, k in enumerate(self._keys(tokens)):
            b = table[i]
            if k in self._by_key or b in self._key_of:
                continue                     # already cached (shared) or registered under its key
            self._by_key[k] = b
            self._key_of[b] = k

    def append_tokens(self, seq, n: int = 1, token_ids=None):
        if token_ids is not None and len(token_ids) != n:
            raise ValueError("one token id per appended token")
        out = super().append_tokens(seq, n)
        known = self.tokens.get(seq)
        if known is not None:
            # without ids the positions from here on are unknown: the sequence stops being cacheable
            self.tokens[seq] = known + [int(t) for t in token_ids] if token_ids is not None else None
        return out

    def fork(self, parent, child):
        table = super().fork(parent, child)
        known = self.tokens.get(parent)
        self.tokens[child] = None if known is None else list(known)
        return table

    def compact(self, seq, num_kept: int):
        # kept tokens are no longer the prefix of a prompt: the sequence becomes uncacheable
        out = super().compact(seq, num_kept)
        self.tokens[seq] = None
        return out

    def free(self, seq) -> None:
        super().free(seq)
        self.tokens.pop(seq, None)

    def stats(self) -> dict:
        out = super().stats()
        out.update(cached_blocks=self.num_cached, evictable_blocks=len(self._evictable),
                   prefix_hits=self.hits, evictions=self.evictions)
        return out
