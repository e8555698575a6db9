"""Pure-Python model of the paged-KV block manager.  (Test infrastructure.)

Sources:
* "vLLM的'内存分页'到底多神奇" (xxqk.cn), §2 "PagedAttention核心思想": memory is
  cut into fixed-size pages; each sequence keeps a page table of the
  physical pages it uses, which need not be contiguous; a scheduler hands out
  pages from a free-page list and takes them back when a request ends;
  sequences with the same prompt prefix can point at the same physical pages.
* same page, §3 phase 1: a sequence's pages are taken on demand, one more
  each time the current page fills (with 8-token pages, token 9 opens page 2).
* same page, §3 phase 3: a finished sequence's pages go back to the free
  list; pages shared through prefix caching carry a reference count and are
  returned only when the last sharer ends; the sharing works like
  copy-on-write (a writer gets its own copy of a shared page).
* same page, §4: admission control refuses (or queues) a request when not
  enough free pages exist, instead of risking an out-of-memory failure;
  aborting a request frees all of its pages.

Policy choices the pages leave open:
* the free list is a LIFO stack; it starts as ``free_order`` (or ascending
  ids) with ``free_order[0]`` on top; a block whose refcount drops to zero is
  pushed back on top, and a sequence's blocks are pushed in table order;
* ``append`` is all-or-nothing: if the free list cannot cover the new blocks
  it fails with NO_BLOCKS and changes nothing;
* ``fork`` shares every block, a partly filled last block included;
* appending into a partly filled last block that is shared first takes a
  fresh block for it (before any new tail block, counted in the
  all-or-nothing admission), drops one reference of the shared block and
  records a pending copy (shared, fresh); pending copies are kept in order
  until the device performs them, frees included;
* block ids are int32; tables export padded with -1.

Prefix caching ("vLLM 生产级落地深剖" (musen-ai.com), §2: sequences with the
same prompt prefix reuse the same physical blocks; §5: blocks are found by
hashing) — the readings:
* only appends that carry token ids (``append_tokens``) take part; a
  sequence whose ids are not all known (created or grown by ``append``) is
  never keyed, and ``append_tokens`` on it is ``append``;
* a block that token-aware appends fill completely is registered under the
  tuple of all token ids from position 0 to its end (this model keys on the
  ids themselves; the library hashes them), unless that key is already
  registered;
* when such an append reaches a block boundary, the following full blocks
  of new tokens are looked up in order until the first miss; a found block
  is shared (refcount + 1; taken off the free list, wherever it sits, when
  its refcount was 0) and its tokens get slot -1; the rest are fresh blocks;
* physical order within one call: found blocks taken, then the
  copy-on-write block, then fresh blocks in logical order;
* a block keeps its key while in use and after it is freed, until it is
  popped from the free list for new contents.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence

OK, ERR_INVALID, ERR_NO_BLOCKS, ERR_UNSUPPORTED, ERR_HIP, ERR_UNKNOWN_SEQ = 0, -1, -2, -3, -4, -5


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        # Python list used as a stack: the top is the last element.
        self.free: List[int] = list(reversed(order))
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.pending: List[tuple] = []   # copy-on-write block copies (src, dst), in order
        self.toks: Dict[int, Optional[List[int]]] = {}   # token ids of keyed sequences (None: not keyed)
        self.cache: Dict[tuple, int] = {}                # prefix ids -> registered block
        self.block_key: Dict[int, tuple] = {}
        self.lookups = 0
        self.hits = 0

    def _pop(self) -> int:
        blk = self.free.pop()
        key = self.block_key.pop(blk, None)
        if key is not None:
            del self.cache[key]
        return blk

    # ---------------------------------------------------------------- ops
    def append(self, seq: int, n: int):
        """Grow ``seq`` by n tokens. Returns (status, slots)."""
        if n < 0:
            return ERR_INVALID, []
        table = self.tables.get(seq, [])
        L = self.lens.get(seq, 0)
        bs = self.block_size
        have = len(table)
        cow = n > 0 and have > 0 and L % bs != 0 and self.ref[table[-1]] > 1
        tail = -(-(L + n) // bs) - have
        if tail + cow > len(self.free):
            return ERR_NO_BLOCKS, []
        table = list(table)
        if cow:
            old, blk = table[-1], self._pop()
            self.ref[blk] += 1
            self.ref[old] -= 1
            table[-1] = blk
            self.pending.append((old, blk))
        for _ in range(tail):
            blk = self._pop()
            self.ref[blk] += 1
            table.append(blk)
        if n > 0 or seq not in self.tables:
            self.toks[seq] = None
        self.tables[seq] = table
        self.lens[seq] = L + n
        slots = [table[p // bs] * bs + p % bs for p in range(L, L + n)]
        return OK, slots

    def append_batch(self, seqs: Sequence[int], n: int):
        """Grow every sequence in ``seqs`` by n tokens as one admission
        decision: either all of them get their pages or nothing changes
        (same page, §4). Returns (status, [slots of seqs[0], ...])."""
        seqs = [int(s) for s in seqs]
        if n < 0 or len(set(seqs)) != len(seqs):
            return ERR_INVALID, []
        bs = self.block_size
        need = 0
        dropped: Dict[int, int] = {}
        for s in seqs:
            L, t = self.lens.get(s, 0), self.tables.get(s, [])
            need += -(-(L + n) // bs) - len(t)
            if n > 0 and t and L % bs != 0 and self.ref[t[-1]] - dropped.get(t[-1], 0) > 1:
                need += 1
                dropped[t[-1]] = dropped.get(t[-1], 0) + 1
        if need > len(self.free):
            return ERR_NO_BLOCKS, []
        out = []
        for s in seqs:
            st, slots = self.append(s, n)
            assert st == OK
            out.append(slots)
        return OK, out

    def fork(self, src: int, dst: int) -> int:
        if src not in self.tables:
            return ERR_UNKNOWN_SEQ
        if dst in self.tables or dst == src:
            return ERR_INVALID
        self.tables[dst] = list(self.tables[src])
        self.lens[dst] = self.lens[src]
        t = self.toks.get(src)
        self.toks[dst] = None if t is None else list(t)
        for blk in self.tables[dst]:
            self.ref[blk] += 1
        return OK

    def free_seq(self, seq: int) -> int:
        if seq not in self.tables:
            return ERR_UNKNOWN_SEQ
        for blk in self.tables.pop(seq):
            self.ref[blk] -= 1
            if self.ref[blk] == 0:
                self.free.append(blk)
        del self.lens[seq]
        self.toks.pop(seq, None)
        return OK

    def append_tokens(self, seq: int, ids: Sequence[int]):
        """Token-aware append with prefix caching. Returns (status, slots,
        n_cached); slots are -1 for tokens found in cached blocks."""
        ids = [int(x) for x in ids]
        n = len(ids)
        if seq in self.tables and self.toks.get(seq) is None:
            st, slots = self.append(seq, n)
            return st, slots, 0
        bs = self.block_size
        table = list(self.tables.get(seq, []))
        L = self.lens.get(seq, 0)
        have = len(table)
        r = L % bs
        fill = min(n, bs - r) if r else 0
        cow = fill > 0 and self.ref[table[-1]] > 1
        all_ids = (self.toks.get(seq) or []) + ids
        tail_key = tuple(all_ids[:(L // bs + 1) * bs]) if r and r + fill == bs else None
        plan = []              # (key, found block or None) per new full block
        searching = True
        pos, lb = fill, have
        lookups = 0
        while n - pos >= bs:
            key = tuple(all_ids[:(lb + 1) * bs])
            hit = None
            if searching:
                lookups += 1
                hit = self.cache.get(key)
                if hit is None:
                    searching = False
            plan.append((key, hit))
            pos += bs
            lb += 1
        rem = n - pos
        hits = [h for _, h in plan if h is not None]
        fresh = len(plan) - len(hits) + (1 if rem > 0 else 0)
        need = sum(1 for h in hits if self.ref[h] == 0) + cow + fresh
        if need > len(self.free):
            return ERR_NO_BLOCKS, [], 0
        for h in hits:                          # (1) cached blocks taken
            if self.ref[h] == 0:
                self.free.remove(h)
            self.ref[h] += 1
        if cow:                                 # (2) the copy-on-write block
            old, blk = table[-1], self._pop()
            self.ref[blk] += 1
            self.ref[old] -= 1
            table[-1] = blk
            self.pending.append((old, blk))
        for key, h in plan:                     # (3) fresh blocks in logical order
            if h is None:
                h = self._pop()
                self.ref[h] += 1
            table.append(h)
        if rem > 0:
            blk = self._pop()
            self.ref[blk] += 1
            table.append(blk)
        if tail_key is not None and tail_key not in self.cache:
            self.cache[tail_key] = table[have - 1]
            self.block_key[table[have - 1]] = tail_key
        for i, (key, h) in enumerate(plan):
            if h is None and key not in self.cache:
                self.cache[key] = table[have + i]
                self.block_key[table[have + i]] = key
        slots = []
        for p in range(L, L + n):
            i = p // bs - have
            if p - L >= fill and 0 <= i < len(plan) and plan[i][1] is not None:
                slots.append(-1)
            else:
                slots.append(table[p // bs] * bs + p % bs)
        self.tables[seq] = table
        self.lens[seq] = L + n
        self.toks[seq] = all_ids
        self.lookups += lookups
        self.hits += len(hits)
        return OK, slots, sum(1 for x in slots if x < 0)

    def prefix_stats(self):
        return {"cached_blocks": len(self.cache), "lookups": self.lookups, "hits": self.hits}

    def block_tables(self, seqs: Iterable[int], max_blocks: int):
        """(status, tables [n][max_blocks] padded -1, lens [n])."""
        tables, lens = [], []
        for s in seqs:
            if s not in self.tables:
                return ERR_UNKNOWN_SEQ, None, None
            t = self.tables[s]
            if len(t) > max_blocks:
                return ERR_INVALID, None, None
            tables.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return OK, tables, lens

    def stats(self) -> dict:
        bs = self.block_size
        fill = [0] * self.num_blocks
        for s, t in self.tables.items():
            L = self.lens[s]
            for i, blk in enumerate(t):
                fill[blk] = max(fill[blk], min(bs, L - i * bs))
        used = sum(1 for r in self.ref if r > 0)
        return {
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": sum(1 for r in self.ref if r > 1),
            "filled_slots": sum(fill),
            "allocated_slots": used * bs,
            "pending_copies": len(self.pending),
        }

    # -------------------------------------------------------------- checks
    def check_invariants(self) -> None:
        """Conservation, refcount = table occurrences, and no duplicate frees."""
        assert len(set(self.free)) == len(self.free), "block on the free list twice"
        count = [0] * self.num_blocks
        for t in self.tables.values():
            for blk in t:
                count[blk] += 1
        assert count == self.ref, "refcount != number of table occurrences"
        used = {b for b in range(self.num_blocks) if self.ref[b] > 0}
        assert used.isdisjoint(self.free), "a used block is on the free list"
        assert len(used) + len(self.free) == self.num_blocks, "blocks lost or duplicated"
        for s, t in self.tables.items():
            assert len(t) == -(-self.lens[s] // self.block_size), "table length != ceil(L/bs)"
        # prefix keys: cache and block_key are inverse maps, and a keyed block
        # at logical index i of a keyed sequence holds that sequence's ids 0..(i+1)*bs
        assert {b: k for k, b in self.cache.items()} == self.block_key, "cache / block_key disagree"
        bs = self.block_size
        for s, t in self.tables.items():
            ids = self.toks.get(s)
            if ids is None:
                continue
            assert len(ids) == self.lens[s], "token ids != length"
            for i, blk in enumerate(t):
                k = self.block_key.get(blk)
                if k is not None:
                    assert k == tuple(ids[:(i + 1) * bs]), "a keyed block's key is not its prefix"


def blocks_needed(n_tokens: int, block_size: int) -> int:
    """Pages a sequence of n tokens occupies: ceil(n / block_size)."""
    return -(-n_tokens // block_size)


def kv_block_bytes(block_size: int, heads: int, head_dim: int, elem_bytes: int) -> int:
    """K+V bytes of one block: block_size * 2 * heads * head_dim * elem_bytes
    ("LLM推理优化：技术原理解析总览", §3.3, the per-page size formula)."""
    return block_size * 2 * heads * head_dim * elem_bytes
