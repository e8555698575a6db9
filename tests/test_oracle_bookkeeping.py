"""Pins for the block-manager model and the scatter oracle (CPU only).

* worked counts printed on the pages (tests/golden/page_counts.json);
* a hand-derived LIFO example;
* invariants after every operation of seeded random op streams:
  conservation of blocks, refcount = table occurrences, atomic failure,
  no leaks once everything is freed, tail waste in closed form;
* scatter: bit-exact against an element-by-element copy, a scatter→gather
  round trip, untouched slots keep their sentinel, negative slots skipped;
* mutation checks on the model.
"""
import copy
import json
import os

import numpy as np
import pytest

import oracle.attention as OA
from oracle.block_manager import (BlockManagerModel, blocks_needed, kv_block_bytes, OK,
                                  ERR_INVALID, ERR_NO_BLOCKS, ERR_UNSUPPORTED, ERR_UNKNOWN_SEQ)
from oracle.scatter import write_kv

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_counts.json")))


# ------------------------------------------------------------- page counts
@pytest.mark.parametrize("case", GOLD["pages_for_tokens"], ids=lambda c: f"{c['tokens']}@{c['block_size']}")
def test_pages_for_tokens(case):
    assert blocks_needed(case["tokens"], case["block_size"]) == case["pages"]
    bm = BlockManagerModel(case["pages"] + 1, case["block_size"])
    st, slots = bm.append(1, case["tokens"])
    assert st == OK and len(bm.tables[1]) == case["pages"]


def test_ninth_token_opens_a_new_page():
    # 8-token pages: tokens 1..8 share page 1, token 9 goes to offset 0 of a new page.
    bm = BlockManagerModel(4, 8)
    st, s8 = bm.append(0, 8)
    st, s9 = bm.append(0, 1)
    assert len({s // 8 for s in s8}) == 1
    assert s9[0] % 8 == 0 and s9[0] // 8 != s8[0] // 8
    assert len(bm.tables[0]) == 2


@pytest.mark.parametrize("case", GOLD["table_bytes"], ids=lambda c: f"{c['requests']}x{c['tokens']}")
def test_table_bytes(case):
    entries = case["requests"] * blocks_needed(case["tokens"], case["block_size"])
    assert entries * case["entry_bytes"] == case["bytes"]


@pytest.mark.parametrize("case", GOLD["kv_block_bytes"], ids=lambda c: f"bs{c['block_size']}")
def test_kv_block_bytes(case):
    assert kv_block_bytes(case["block_size"], case["heads"], case["head_dim"], case["elem_bytes"]) == case["bytes"]


def test_preallocation_bytes():
    c = GOLD["preallocation"][0]
    assert blocks_needed(c["batched_tokens"], c["block_size"]) == c["pages"]
    assert c["pages"] * kv_block_bytes(16, 32, 128, 2) == c["bytes"]


def test_tiny_workload_needs_nine_blocks():
    assert sum(blocks_needed(L, 16) for L in (7, 16, 33, 50)) == 9


# ------------------------------------------------------------ LIFO example
def test_lifo_worked_example():
    """Hand-derived: pool of 6 blocks, free_order = [4, 1, 5, 0, 3, 2], bs 4."""
    bm = BlockManagerModel(6, 4, [4, 1, 5, 0, 3, 2])
    st, s = bm.append(10, 6)            # needs 2 blocks: pops 4, then 1
    assert st == OK and bm.tables[10] == [4, 1]
    assert s == [16, 17, 18, 19, 4, 5]  # 4*4+0..3, then 1*4+0..1
    st, s = bm.append(11, 3)            # pops 5
    assert bm.tables[11] == [5] and s == [20, 21, 22]
    st, s = bm.append(10, 3)            # len 6 -> 9: one more block, pops 0
    assert bm.tables[10] == [4, 1, 0] and s == [6, 7, 0]
    assert bm.append(12, 9) == (ERR_NO_BLOCKS, [])   # needs 3 blocks, only 3 and 2 are free
    assert bm.free_seq(10) == OK        # pushes 4, 1, 0 in table order: top is 0
    st, s = bm.append(12, 5)            # pops 0, then 1
    assert bm.tables[12] == [0, 1]
    # Free stack now, top first: 4, 3, 2.
    assert bm.fork(12, 13) == OK        # 5 tokens: the partly filled block 1 is shared too
    assert bm.ref[0] == 2 and bm.ref[1] == 2
    st, s = bm.append(13, 2)            # child writes into shared block 1: copy-on-write pops 4
    assert st == OK and bm.tables[13] == [0, 4] and s == [17, 18]
    assert bm.pending == [(1, 4)] and bm.ref[1] == 1 and bm.ref[4] == 1
    st, s = bm.append(12, 3)            # parent now owns block 1 alone: no copy, fills it
    assert bm.tables[12] == [0, 1] and s == [5, 6, 7] and bm.pending == [(1, 4)]
    assert bm.free_seq(13) == OK        # block 4 is free again; its copy stays recorded
    assert bm.pending == [(1, 4)] and bm.free == [2, 3, 4]
    bm.pending = []                     # the device performed the copy
    assert bm.fork(12, 14) == OK        # len 8, aligned
    st, s = bm.append(14, 1)            # opens its own block: pops 4
    assert bm.tables[14] == [0, 1, 4] and s == [16]
    assert bm.fork(14, 15) == OK        # len 9: shares 0, 1 and the partly filled 4
    # 15 grows 9 -> 17: one copy block plus two tail blocks, only 3 and 2 free.
    assert bm.append(15, 8) == (ERR_NO_BLOCKS, [])
    assert bm.tables[15] == [0, 1, 4] and bm.pending == [] and bm.free == [2, 3]
    st, s = bm.append(15, 7)            # 9 -> 16: copy pops 3, tail pops 2
    assert st == OK and bm.tables[15] == [0, 1, 3, 2]
    assert s == [13, 14, 15, 8, 9, 10, 11] and bm.pending == [(4, 3)]
    assert bm.ref[4] == 1 and bm.ref[0] == 3
    for q in (12, 14, 15):
        assert bm.free_seq(q) == OK
    assert bm.free_seq(11) == OK
    assert sorted(bm.free) == list(range(6))


# -------------------------------------------------------- random op streams
def random_ops(rng, n_ops, max_seqs=12, max_tokens=70):
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        s = int(rng.integers(0, max_seqs))
        if r < 0.55:
            ops.append(("append", s, int(rng.integers(0, max_tokens))))
        elif r < 0.75:
            ops.append(("fork", s, int(rng.integers(0, max_seqs))))
        else:
            ops.append(("free", s))
    return ops


def apply(bm, op):
    if op[0] == "append":
        return bm.append(op[1], op[2])[0]
    if op[0] == "fork":
        return bm.fork(op[1], op[2])
    return bm.free_seq(op[1])


@pytest.mark.parametrize("seed", range(8))
def test_random_streams_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    bs = [8, 16, 32][seed % 3]
    bm = BlockManagerModel(40, bs, rng.permutation(40))
    for op in random_ops(rng, 400):
        before = copy.deepcopy((bm.free, bm.ref, bm.tables, bm.lens))
        st = apply(bm, op)
        if st != OK:
            assert copy.deepcopy((bm.free, bm.ref, bm.tables, bm.lens)) == before, f"{op} failed but changed state"
        bm.check_invariants()
        stats = bm.stats()
        assert stats["free_blocks"] + stats["used_blocks"] == 40
        # tail waste closed form when nothing is shared: Σ (ceil(L/bs)·bs − L)
        if stats["shared_blocks"] == 0:
            waste = sum(-(-L // bs) * bs - L for L in bm.lens.values())
            assert stats["allocated_slots"] - stats["filled_slots"] == waste
    for s in list(bm.tables):
        assert bm.free_seq(s) == OK
    assert sorted(bm.free) == list(range(40)) and not any(bm.ref)


def test_error_codes():
    bm = BlockManagerModel(4, 16)
    assert bm.append(0, -1)[0] == ERR_INVALID
    assert bm.free_seq(99) == ERR_UNKNOWN_SEQ
    assert bm.fork(99, 1) == ERR_UNKNOWN_SEQ
    bm.append(0, 16)
    assert bm.fork(0, 0) == ERR_INVALID
    bm.append(1, 1)
    assert bm.fork(0, 1) == ERR_INVALID       # destination exists
    assert bm.block_tables([0, 1], 0)[0] == ERR_INVALID
    assert bm.block_tables([0, 7], 4)[0] == ERR_UNKNOWN_SEQ
    st, t, l = bm.block_tables([1, 0], 3)
    assert st == OK and t == [[bm.tables[1][0], -1, -1], [bm.tables[0][0], -1, -1]] and l == [1, 16]


def test_prefix_share_refcount_128():
    bm = BlockManagerModel(200, 16)
    bm.append(0, 2048)
    for b in range(1, 128):
        assert bm.fork(0, b) == OK
    assert all(bm.ref[blk] == 128 for blk in bm.tables[0])
    assert bm.stats()["shared_blocks"] == 128


# ----------------------------------------------------------------- scatter
@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_scatter_bit_exact_and_sentinel(dtype):
    rng = np.random.default_rng(1)
    nb, bs, H, D, T = 9, 8, 2, 4, 30
    sentinel = np.array(0x7FC1 if dtype == np.uint16 else np.nan, dtype=dtype)
    kc = np.full((nb, bs, H, D), sentinel, dtype=dtype)
    vc = kc.copy()
    key = rng.integers(0, 2 ** 15, (T, H, D)).astype(dtype)
    val = rng.integers(0, 2 ** 15, (T, H, D)).astype(dtype)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    slots[[3, 11]] = -1
    write_kv(kc, vc, key, val, slots)
    flat_k = kc.reshape(nb * bs, H, D)
    written = set()
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(flat_k[s].view(np.uint8), key[t].view(np.uint8))
            assert np.array_equal(vc.reshape(nb * bs, H, D)[s].view(np.uint8), val[t].view(np.uint8))
            written.add(int(s))
    for s in set(range(nb * bs)) - written:
        assert np.array_equal(flat_k[s].view(np.uint8), np.full((H, D), sentinel, dtype).view(np.uint8))


def test_scatter_then_gather_round_trip():
    rng = np.random.default_rng(2)
    bs, H, D = 16, 2, 8
    bm = BlockManagerModel(20, bs, rng.permutation(20))
    lens = [5, 16, 40]
    kc = np.zeros((20, bs, H, D), np.float32)
    vc = np.zeros_like(kc)
    data = {}
    for s, L in enumerate(lens):
        k, v = rng.standard_normal((L, H, D)).astype(np.float32), rng.standard_normal((L, H, D)).astype(np.float32)
        half = L // 2
        for a, n in ((0, half), (half, L - half)):       # two appends per sequence
            st, slots = bm.append(s, n)
            write_kv(kc, vc, k[a:a + n], v[a:a + n], np.array(slots))
        data[s] = (k, v)
    st, tables, tl = bm.block_tables(range(3), 3)
    for s, L in enumerate(lens):
        assert np.array_equal(OA.gather_sequence(kc, tables[s], L, bs), data[s][0])
        assert np.array_equal(OA.gather_sequence(vc, tables[s], L, bs), data[s][1])


def test_scatter_mutant_off_by_one_is_caught():
    """A scatter that writes slot+1 breaks the round trip."""
    kc = np.zeros((2, 4, 1, 1), np.float32)
    vc = np.zeros_like(kc)
    key = np.arange(1, 4, dtype=np.float32).reshape(3, 1, 1)
    flat = kc.reshape(8, 1, 1)
    for t, s in enumerate([0, 1, 2]):
        flat[s + 1] = key[t]
    assert not np.array_equal(OA.gather_sequence(kc, [0], 3, 4), key)


# ------------------------------------------------- copy-on-write round trip
def _round_trip_mismatches(wl):
    from oracle.cache import OracleCache
    c = OracleCache(wl)
    bad = []
    for s in range(wl.B):
        L = int(c.seq_lens[s])
        k, v = wl.seq_kv(s)
        gk = OA.gather_sequence(c.k_cache, c.block_tables[s], L, wl.block_size)
        gv = OA.gather_sequence(c.v_cache, c.block_tables[s], L, wl.block_size)
        if not (np.array_equal(gk.view(np.uint8), k.view(np.uint8)) and
                np.array_equal(gv.view(np.uint8), v.view(np.uint8))):
            bad.append(s)
    return c, bad


def test_cache_round_trip_with_copy_on_write():
    """A 1000-token prefix (last block half full) forked 32 ways: every
    sequence reads back exactly its logical rows through its table, and the
    partial block was copied once per writer that still found it shared."""
    import workloads as W
    wl = W.config("prefix_cow")
    c, bad = _round_trip_mismatches(wl)
    assert bad == []
    part = [int(c.block_tables[s][62]) for s in range(wl.B)]
    writers = [s for s in range(wl.B) if wl.seq_lens[s] > 1000]
    # all writers but the last get private copies; non-writers and the last writer keep the original
    original = part[writers[-1]]
    assert all(part[s] == original for s in range(wl.B) if s not in writers[:-1])
    assert len({part[s] for s in writers[:-1]} | {original}) == len(writers)


def test_round_trip_catches_a_dropped_copy(monkeypatch):
    """Mutation: an append that forgets its copy-on-write copy must fail the round trip."""
    import workloads as W
    real = BlockManagerModel.append

    def forgetful(self, seq, n):
        r = real(self, seq, n)
        self.pending = []
        return r

    monkeypatch.setattr(BlockManagerModel, "append", forgetful)
    _, bad = _round_trip_mismatches(W.config("prefix_cow"))
    assert bad


# ------------------------------------------------------------ prefix caching
def test_prefix_cache_worked_example():
    """Hand-derived: 8 blocks of 4 tokens, ascending free order (0 handed out first)."""
    bm = BlockManagerModel(8, 4)
    st, s, c = bm.append_tokens(0, [1, 2, 3, 4, 5, 6, 7, 8, 9])     # lookup of the first block misses
    assert (st, c) == (OK, 0) and bm.tables[0] == [0, 1, 2] and s == list(range(9))
    st, s, c = bm.append_tokens(1, [1, 2, 3, 4, 5, 6, 7, 8, 10, 11])  # two full blocks found
    assert c == 8 and bm.tables[1] == [0, 1, 3] and s == [-1] * 8 + [12, 13]
    st, s, c = bm.append_tokens(2, [1, 2, 3, 4, 9, 9, 9, 9])         # first found, second new
    assert c == 4 and bm.tables[2] == [0, 4] and s == [-1] * 4 + [16, 17, 18, 19]
    assert bm.free_seq(0) == OK and bm.free_seq(1) == OK
    assert bm.free == [7, 6, 5, 2, 1, 3]                              # block 1 free but still keyed
    st, s, c = bm.append_tokens(3, [1, 2, 3, 4, 5, 6, 7, 8])          # block 1 taken back off the free list
    assert c == 8 and bm.tables[3] == [0, 1] and bm.free == [7, 6, 5, 2, 3] and bm.ref[1] == 1
    assert bm.free_seq(2) == OK and bm.free == [7, 6, 5, 2, 3, 4]
    st, s = bm.append(4, 5)                                          # plain append pops 4: its key is dropped
    assert bm.tables[4] == [4, 3] and s == [16, 17, 18, 19, 12]
    assert bm.prefix_stats()["cached_blocks"] == 2
    st, s, c = bm.append_tokens(5, [1, 2, 3, 4, 9, 9, 9, 9])         # the evicted block misses now
    assert c == 4 and bm.tables[5] == [0, 2] and s == [-1] * 4 + [8, 9, 10, 11]
    assert bm.prefix_stats() == {"cached_blocks": 3, "lookups": 9, "hits": 6}
    st, s, c = bm.append_tokens(6, [1, 2, 3, 4, 5, 6])
    assert c == 4 and bm.tables[6] == [0, 5] and s == [-1] * 4 + [20, 21]   # positions 4, 5 of block 5
    st, s, c = bm.append_tokens(6, [7, 8])                           # completes a block equal to block 1:
    assert c == 0 and s == [22, 23]                                  # positions 6, 7 of block 5
    assert bm.prefix_stats()["cached_blocks"] == 3                   # the key stays with block 1
    assert bm.cache[(1, 2, 3, 4, 5, 6, 7, 8)] == 1 and 5 not in bm.block_key
    bm.check_invariants()


@pytest.mark.parametrize("seed", range(4))
def test_prefix_cache_invariants_on_streams(seed):
    rng = np.random.default_rng(50 + seed)
    bs = [4, 8, 16, 32][seed]
    bm = BlockManagerModel(64, bs, rng.permutation(64))
    tmpl = [list(rng.integers(0, 20, 5 * bs)) for _ in range(3)]
    live, nxt = [], 0
    for _ in range(300):
        r = rng.random()
        if r < 0.5 or not live:
            ids = tmpl[int(rng.integers(0, 3))][:int(rng.integers(1, 5 * bs + 1))] + \
                list(rng.integers(0, 20, int(rng.integers(0, bs))))
            before = copy.deepcopy((bm.free, bm.ref, bm.tables, bm.lens, bm.cache, bm.block_key))
            st, slots, c = bm.append_tokens(nxt, ids)
            if st != OK:
                assert copy.deepcopy((bm.free, bm.ref, bm.tables, bm.lens, bm.cache, bm.block_key)) == before
            else:
                live.append(nxt)
                assert c == sum(1 for x in slots if x < 0) and c % bs == 0
            nxt += 1
        elif r < 0.75:
            assert bm.free_seq(live.pop(int(rng.integers(0, len(live))))) == OK
        else:
            s = live[int(rng.integers(0, len(live)))]
            bm.append_tokens(s, list(rng.integers(0, 20, int(rng.integers(0, 2 * bs)))))
        bm.check_invariants()
    assert bm.prefix_stats()["hits"] > 0


def test_cache_round_trip_with_prefix_caching():
    """48 requests share a 1000-token prompt, each appended with its token ids:
    the 62 full prompt blocks are found by lookup (refcount 48), and every
    sequence still reads back exactly its logical rows."""
    import workloads as W
    wl = W.config("prompt_cache")
    c, bad = _round_trip_mismatches(wl)
    assert bad == []
    assert c.bm.prefix_stats()["hits"] == (wl.B - 1) * (1000 // 16)
    shared = {int(b) for b in c.block_tables[0][:62]}
    assert all(c.bm.ref[b] == wl.B for b in shared)
    assert all(int(c.block_tables[s][62]) not in shared for s in range(wl.B))
