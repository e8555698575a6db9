"""Host-side checks of the C-ABI library (no GPU needed).

* libpa.so loads and exports every function include/pa.h declares;
* the C++ block manager, driven through the C ABI, matches the Python model
  bit for bit (statuses, slots, tables, lengths, stats) on seeded op streams;
* the same C++ block manager built on its own with g++ under AddressSanitizer
  and UBSan replays the same streams with identical output;
* argument validation of the device entry points fails before any launch.
"""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")
CSRC = os.path.join(ROOT, "paged_kv_cache_indirect_amd", "csrc")

pa = pytest.importorskip("paged_kv_cache_indirect_amd")
from oracle.block_manager import BlockManagerModel  # noqa: E402

FAKE_K, FAKE_V = 0x10000, 0x20000   # aligned, never dereferenced by host-only calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(pa.lib, n), f"libpa.so does not export {n}"


def make_pool(nb, bs, order=None, hkv=2, d=64, dtype=pa.PA_BF16):
    layout = pa._Layout(nb, bs, hkv, d, dtype)
    h = ctypes.c_void_p()
    arr = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
    st = pa.lib.pa_alloc_pool(ctypes.byref(layout), FAKE_K, FAKE_V,
                              None if arr is None else arr.ctypes.data, ctypes.byref(h))
    return st, h.value


def random_ops(rng, n_ops, max_seqs=10, max_tokens=80):
    # shared prompts: token-aware appends often start with one of these
    templates = [rng.integers(0, 40, 120) for _ in range(3)]
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        s = int(rng.integers(0, max_seqs))
        if r < 0.15:
            t = templates[int(rng.integers(0, 3))]
            ids = list(t[:int(rng.integers(0, 121))]) + list(rng.integers(0, 40, int(rng.integers(0, 20))))
            ops.append(("tokens", s, [int(x) for x in ids]))
        elif r < 0.4:
            ops.append(("append", s, int(rng.integers(0, max_tokens))))
        elif r < 0.5:
            # a batch of distinct sequences (sometimes a repeated id: rejected)
            k = int(rng.integers(0, 5))
            ids = [int(x) for x in rng.choice(max_seqs + 2, size=k, replace=False)]
            if k and rng.random() < 0.1:
                ids.append(ids[0])
            ops.append(("batch", int(rng.integers(0, max_tokens // 3)), ids))
        elif r < 0.7:
            ops.append(("fork", s, int(rng.integers(0, max_seqs))))
        elif r < 0.9:
            ops.append(("free", s))
        else:
            ops.append(("tables", int(rng.integers(0, 12)), [int(x) for x in rng.integers(0, max_seqs, 3)]))
    return ops


def run_model(nb, bs, order, ops):
    m = BlockManagerModel(nb, bs, order)
    out = []
    for op in ops:
        if op[0] == "append":
            st, slots = m.append(op[1], op[2])
            out.append((st, list(slots)))
        elif op[0] == "batch":
            st, slots = m.append_batch(op[2], op[1])
            out.append((st, [x for row in slots for x in row]))
        elif op[0] == "tokens":
            st, slots, cached = m.append_tokens(op[1], op[2])
            out.append((st, list(slots) if st == 0 else [], cached if st == 0 else 0))
        elif op[0] == "fork":
            out.append((m.fork(op[1], op[2]),))
        elif op[0] == "free":
            out.append((m.free_seq(op[1]),))
        else:
            st, t, l = m.block_tables(op[2], op[1])
            out.append((st, l, t))
        s = m.stats()
        ps = m.prefix_stats()
        out.append(tuple(s[k] for k in ("free_blocks", "used_blocks", "shared_blocks", "filled_slots",
                                        "allocated_slots")) +
                   tuple(ps[k] for k in ("cached_blocks", "lookups", "hits")) +
                   tuple(x for c in m.pending for x in c))
    return out


def run_abi(pool, ops):
    out = []
    for op in ops:
        if op[0] == "append":
            slots = np.empty(max(op[2], 1), dtype=np.int64)
            st = pa.lib.pa_seq_append(pool, op[1], op[2], slots.ctypes.data)
            out.append((st, slots[:op[2]].tolist() if st == 0 else []))
        elif op[0] == "batch":
            ids = np.array(op[2], dtype=np.int64)
            slots = np.empty(max(len(ids) * op[1], 1), dtype=np.int64)
            st = pa.lib.pa_seq_append_batch(pool, ids.ctypes.data, len(ids), op[1], slots.ctypes.data)
            out.append((st, slots[:len(ids) * op[1]].tolist() if st == 0 else []))
        elif op[0] == "tokens":
            ids = np.array(op[2], dtype=np.int32)
            slots = np.empty(max(len(ids), 1), dtype=np.int64)
            cached = ctypes.c_int32()
            st = pa.lib.pa_seq_append_tokens(pool, op[1], ids.ctypes.data, len(ids), slots.ctypes.data,
                                             ctypes.byref(cached))
            out.append((st, slots[:len(ids)].tolist() if st == 0 else [], cached.value if st == 0 else 0))
        elif op[0] == "fork":
            out.append((pa.lib.pa_seq_fork(pool, op[1], op[2]),))
        elif op[0] == "free":
            out.append((pa.lib.pa_seq_free(pool, op[1]),))
        else:
            mb, ids = op[1], np.array(op[2], dtype=np.int64)
            t = np.zeros((len(ids), max(mb, 1)), np.int32)
            l = np.zeros(len(ids), np.int32)
            st = pa.lib.pa_block_tables(pool, ids.ctypes.data, len(ids), mb, t.ctypes.data, l.ctypes.data)
            out.append((st, l.tolist(), t[:, :mb].tolist()) if st == 0 else (st, None, None))
        s = pa.pa_pool_stats(pool)
        ps = pa.pa_pool_prefix_stats(pool)
        out.append(tuple(s[k] for k in ("free_blocks", "used_blocks", "shared_blocks", "filled_slots",
                                        "allocated_slots")) +
                   tuple(ps[k] for k in ("cached_blocks", "lookups", "hits")) +
                   tuple(x for c in pa.pa_pool_pending_copies(pool) for x in c))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_cpp_block_manager_matches_model(seed):
    rng = np.random.default_rng(100 + seed)
    nb, bs = 48, [8, 16, 32][seed % 3]
    order = rng.permutation(nb) if seed % 2 else None
    ops = random_ops(rng, 500)
    st, pool = make_pool(nb, bs, order)
    assert st == 0
    try:
        assert run_abi(pool, ops) == run_model(nb, bs, order, ops)
    finally:
        pa.pa_free_pool(pool)


def test_workload_op_streams_match_model():
    """The tables the named workloads build (tiny, prefix sharing) agree."""
    import workloads as W
    for wl in (W.config("tiny"), W.make_prefix_share("p", 16, 64, [0, 5, 16, 40] * 4, 8, 2, 64, 16,
                                                        "bf16", 7)):
        st, pool = make_pool(wl.num_blocks, wl.block_size, wl.free_order, wl.Hkv, wl.D)
        m = BlockManagerModel(wl.num_blocks, wl.block_size, wl.free_order)
        for op in wl.ops:
            if op[0] == "append":
                a = pa.pa_seq_append(pool, op[1], op[2])
                stm, b = m.append(op[1], op[2])
                assert stm == 0 and a.tolist() == b
            else:
                pa.pa_seq_fork(pool, op[1], op[2])
                assert m.fork(op[1], op[2]) == 0
        t, l = pa.pa_block_tables(pool, list(range(wl.B)), wl.max_blocks)
        stm, tm, lm = m.block_tables(range(wl.B), wl.max_blocks)
        assert t.tolist() == tm and l.tolist() == lm
        pa.pa_free_pool(pool)


def test_exhaustion_is_atomic_and_no_leaks():
    st, pool = make_pool(10, 16)
    pa.pa_seq_append(pool, 1, 100)                         # 7 blocks
    before = pa.pa_pool_stats(pool)
    with pytest.raises(pa.PaError) as e:
        pa.pa_seq_append(pool, 2, 64)                      # needs 4, 3 free
    assert e.value.status == pa.PA_ERR_NO_BLOCKS
    assert "not enough free blocks" in pa.pa_last_error()
    assert pa.pa_pool_stats(pool) == before
    with pytest.raises(pa.PaError):
        pa.pa_block_tables(pool, [2], 8)                   # sequence 2 was not created
    pa.pa_seq_append(pool, 1, 12)                          # 112 = 7 blocks exactly
    pa.pa_seq_fork(pool, 1, 3)
    pa.pa_seq_free(pool, 1)
    t, l = pa.pa_block_tables(pool, [3], 8)
    assert l.tolist() == [112] and (t[0, :7] >= 0).all()
    pa.pa_seq_free(pool, 3)
    assert pa.pa_pool_stats(pool)["free_blocks"] == 10
    with pytest.raises(pa.PaError) as e:
        pa.pa_seq_free(pool, 3)
    assert e.value.status == pa.PA_ERR_UNKNOWN_SEQ
    pa.pa_free_pool(pool)


def test_append_batch_is_all_or_nothing():
    st, pool = make_pool(10, 16)
    pa.pa_seq_append(pool, 1, 16)                          # 1 block, full
    before = pa.pa_pool_stats(pool)
    with pytest.raises(pa.PaError) as e:                   # needs 1 + 5 + 5 = 11 > 9
        pa.pa_seq_append_batch(pool, [1, 2, 3], 80)
    assert e.value.status == pa.PA_ERR_NO_BLOCKS
    assert pa.pa_pool_stats(pool) == before
    with pytest.raises(pa.PaError):
        pa.pa_block_tables(pool, [2], 8)                   # not created
    with pytest.raises(pa.PaError) as e:
        pa.pa_seq_append_batch(pool, [1, 1], 1)
    assert e.value.status == pa.PA_ERR_INVALID
    slots = pa.pa_seq_append_batch(pool, [1, 2, 3], 1)     # 3 new blocks: 1 crosses, 2/3 are new
    assert slots.shape == (3, 1)
    t, l = pa.pa_block_tables(pool, [1, 2, 3], 4)
    assert l.tolist() == [17, 1, 1]
    assert slots[:, 0].tolist() == [t[0, 1] * 16, t[1, 0] * 16, t[2, 0] * 16]
    pa.pa_free_pool(pool)


def test_alloc_pool_rejects_bad_geometry():
    assert make_pool(10, 12)[0] == pa.PA_ERR_UNSUPPORTED       # block_size 12
    assert make_pool(10, 16, d=96)[0] == pa.PA_ERR_UNSUPPORTED  # head_dim 96
    assert make_pool(0, 16)[0] == pa.PA_ERR_INVALID
    assert make_pool(4, 16, order=[0, 1, 1, 2])[0] == pa.PA_ERR_INVALID
    assert make_pool(4, 16, dtype=7)[0] == pa.PA_ERR_UNSUPPORTED


def _expected_items(B, L, pt):
    """Work items the short-context rule expects at partition pt: two kv
    heads per group (8 kv heads -> 4 groups), lengths uniform in [0, L]."""
    return max(B, 1) * 4 * (max(L, 1) / (2 * pt) + 0.5)


def test_decode_partition_policy():
    """The library's partition for partition_tokens = 0. Work items are
    (sequence, group of two kv heads, partition). Contexts of 8192 tokens and
    more: the fewest partitions giving 256 items at max_seq_len. Shorter ones:
    the smallest partition whose expected item count (lengths uniform in
    [0, max_seq_len]) is at most 480 (448 for an FP8 pool). Kept within
    [640, 8192] tokens and rounded up to a multiple of 64."""
    pools = {bs: make_pool(64, bs, hkv=8, d=128)[1] for bs in (8, 16, 32)}
    fp8_pool = make_pool(64, 16, hkv=8, d=128, dtype=pa.PA_FP8_E4M3)[1]
    f = pa.pa_decode_partition_tokens
    p16 = pools[16]
    assert f(p16, 64, 4087) == 1536       # 8B-shaped batch: 256 head-group pairs
    assert f(p16, 64, 4142) == 1536
    assert f(fp8_pool, 64, 4142) == 1664  # FP8: more margin below two items per CU
    assert f(p16, 56, 4100) == 1280
    assert f(p16, 64, 32768) == 8192      # long context, capped
    assert f(p16, 8, 32768) == 4096       # long contexts: 8 partitions -> 256 items
    assert f(p16, 128, 3068) == 3520      # 512 pairs fill the GPU: one partition
    assert f(p16, 48, 1591) == 640        # floor
    assert f(p16, 1, 32768) == 640
    assert f(p16, 4, 50) == 640 and f(p16, 0, 0) == 640
    assert f(pools[8], 64, 20000) == 8192 and f(pools[32], 64, 2000) == 768   # block size plays no part
    assert f(None, 4, 100) == 0 and f(p16, -1, 100) == 0
    rng = np.random.default_rng(3)
    for _ in range(300):
        B = int(rng.integers(0, 300))
        L = int(rng.integers(0, 70000))
        pt = f(p16, B, L)
        assert pt % 64 == 0 and 640 <= pt <= 8192, (B, L, pt)
        if pt in (640, 8192):
            continue
        if L >= 8192:
            parts = -(-256 // (max(B, 1) * 4))   # partitions for 256 items
            assert pt == -(-(-(-L // parts)) // 64) * 64, (B, L, pt)
        elif pt < L:
            # smallest multiple of 64 within the expected-item target
            assert _expected_items(B, L, pt) <= 480 + 1e-9 < _expected_items(B, L, pt - 64), (B, L, pt)
        # the 512-token workspace bounds the default's
        assert pa.lib.pa_decode_workspace_bytes(B, 32, 128, L, pt) <= pa.lib.pa_decode_workspace_bytes(B, 32, 128, L, 0)
    for p in list(pools.values()) + [fp8_pool]:
        pa.pa_free_pool(p)


def test_decode_partition_for_host_lengths():
    """pa_append_decode_args's partition for partition_tokens = 0, from the
    lengths: all sequences >= 8192 tokens -> the shape rule; otherwise the
    smallest multiple of 64 (>= 512) with at most 480 items (4 head groups
    of two kv heads x sum_b max(1, ceil(L_b / pt))), else one partition per
    sequence."""
    st, p16 = make_pool(64, 16, hkv=8, d=128)
    f = pa.pa_decode_partition_tokens_for_lengths
    import workloads as W
    assert f(p16, W.config("gqa8b").seq_lens, 4142) == 1536
    assert f(p16, [512] * 63 + [32768], 32768) == 576            # the long one split finely
    assert f(p16, [32768] * 8, 32768) == pa.pa_decode_partition_tokens(p16, 8, 32768) == 4096
    assert f(p16, [3000] * 128, 3072) == 3008                      # 512 items at least: one partition each
    assert f(None, [1, 2], 10) == 0 and f(p16, [1, 2], -1) == 0

    def items(L, pt):
        return 4 * sum(max(1, -(-x // pt)) for x in L)

    rng = np.random.default_rng(5)
    for _ in range(200):
        B = int(rng.integers(1, 130))
        hi = int(rng.integers(1, 9000))
        L = rng.integers(0, hi + 1, B).tolist()
        msl = max(L) + int(rng.integers(0, 50))
        pt = f(p16, L, msl)
        top = max(512, -(-max(max(L), 1) // 64) * 64)
        if min(L) >= 8192:
            continue
        assert pt % 64 == 0 and 512 <= pt <= top, (L, pt)
        if items(L, top) > 480:
            assert pt == top
        else:
            assert items(L, pt) <= 480 and (pt == 512 or items(L, pt - 64) > 480), (pt, items(L, pt))
    pa.pa_free_pool(p16)


def test_device_entry_points_validate_before_launch():
    st, pool = make_pool(64, 16, hkv=8, d=128)
    assert st == 0
    dummy = 0x40000
    ws = pa.lib.pa_decode_workspace_bytes(64, 32, 128, 4097, 512)   # 9 partitions
    assert ws == 64 * 32 * 9 * 130 * 4 + 16   # partial states + the recorded partition
    assert pa.lib.pa_decode_workspace_bytes(64, 32, 128, 512, 512) == 0   # one partition covers it
    # G = 3 is outside the supported set
    assert pa.lib.pa_decode(pool, dummy, dummy, dummy, 256, dummy, 4, 24, 0.1, 4096, 0, dummy, ws, None) \
        == pa.PA_ERR_UNSUPPORTED
    # Hq not a multiple of Hkv
    assert pa.lib.pa_decode(pool, dummy, dummy, dummy, 256, dummy, 4, 12, 0.1, 4096, 0, dummy, ws, None) \
        == pa.PA_ERR_INVALID
    # max_seq_len beyond the table width
    assert pa.lib.pa_decode(pool, dummy, dummy, dummy, 16, dummy, 4, 32, 0.1, 4096, 0, dummy, ws, None) \
        == pa.PA_ERR_INVALID
    # workspace missing / too small / misaligned
    assert pa.lib.pa_decode(pool, dummy, dummy, dummy, 257, dummy, 4, 32, 0.1, 4097, 0, None, 0, None) \
        == pa.PA_ERR_INVALID
    assert "workspace too small" in pa.pa_last_error()
    # partition size rules
    assert pa.lib.pa_decode(pool, dummy, dummy, dummy, 256, dummy, 4, 32, 0.1, 4096, 100, dummy, 1 << 30, None) \
        == pa.PA_ERR_UNSUPPORTED
    big = (1 << 24) + 64   # past the largest partition accepted
    assert pa.lib.pa_decode(pool, dummy, dummy, dummy, 256, dummy, 4, 32, 0.1, 4096, big, dummy, 1 << 30, None) \
        == pa.PA_ERR_UNSUPPORTED
    assert "at most 16777216" in pa.pa_last_error()
    # misaligned q
    assert pa.lib.pa_decode(pool, dummy, dummy + 2, dummy, 256, dummy, 4, 32, 0.1, 4096, 0, dummy, ws, None) \
        == pa.PA_ERR_INVALID
    # B == 0 is a no-op
    assert pa.lib.pa_decode(pool, None, None, None, 0, None, 0, 32, 0.1, 0, 0, None, 0, None) == pa.PA_OK
    assert pa.lib.pa_write_kv(pool, None, None, None, 0, None) == pa.PA_OK
    assert pa.lib.pa_write_kv(pool, dummy, dummy, None, 5, None) == pa.PA_ERR_INVALID
    assert pa.lib.pa_write_kv(pool, dummy, dummy, dummy, -1, None) == pa.PA_ERR_INVALID
    # fused append + decode: pa_decode's checks, then its new rows
    ad = pa.lib.pa_append_decode
    assert ad(pool, dummy, dummy, dummy, dummy, dummy, dummy, 256, dummy, 4, 24, 0.1, 4096, 0, dummy, ws, None) \
        == pa.PA_ERR_UNSUPPORTED                                  # G = 3
    assert ad(pool, dummy, dummy, None, dummy, dummy, dummy, 256, dummy, 4, 32, 0.1, 4096, 0, dummy, ws, None) \
        == pa.PA_ERR_INVALID                                      # null key
    assert ad(pool, dummy, dummy, dummy + 4, dummy, dummy, dummy, 256, dummy, 4, 32, 0.1, 4096, 0, dummy, ws,
              None) == pa.PA_ERR_INVALID                          # misaligned key
    assert ad(pool, dummy, dummy, dummy, dummy, None, dummy, 256, dummy, 4, 32, 0.1, 4096, 0, dummy, ws, None) \
        == pa.PA_ERR_INVALID                                      # null slots
    assert ad(pool, None, None, None, None, None, None, 0, None, 0, 32, 0.1, 0, 0, None, 0, None) == pa.PA_OK
    pa.pa_free_pool(pool)
    st, f8 = make_pool(16, 16, hkv=2, d=128, dtype=pa.PA_FP8_E4M3)
    assert ad(f8, dummy, dummy, dummy, dummy, dummy, dummy, 16, dummy, 2, 8, 0.1, 256, 0, dummy, 1 << 20, None) \
        == pa.PA_ERR_UNSUPPORTED
    aa = pa.lib.pa_append_decode_args
    slots_h = np.zeros(200, dtype=np.int64)
    lens_h = np.ones(200, dtype=np.int32)
    assert aa(f8, dummy, dummy, dummy, dummy, slots_h.ctypes.data, dummy, 16, lens_h.ctypes.data, 2, 8, 0.1, 256, 0,
              dummy, 1 << 20, None) == pa.PA_ERR_UNSUPPORTED
    pa.pa_free_pool(f8)
    st, pool = make_pool(64, 16, hkv=8, d=128)
    # launch-argument variant: at most 128 sequences; the host arrays are required
    assert aa(pool, dummy, dummy, dummy, dummy, slots_h.ctypes.data, dummy, 256, lens_h.ctypes.data, 129, 32, 0.1,
              4096, 0, dummy, 1 << 30, None) == pa.PA_ERR_UNSUPPORTED
    assert "at most 128" in pa.pa_last_error()
    assert aa(pool, dummy, dummy, dummy, dummy, None, dummy, 256, lens_h.ctypes.data, 4, 32, 0.1, 4096, 0, dummy,
              1 << 30, None) == pa.PA_ERR_INVALID
    assert aa(pool, dummy, dummy, dummy, dummy, slots_h.ctypes.data, dummy, 256, None, 4, 32, 0.1, 4096, 0, dummy,
              1 << 30, None) == pa.PA_ERR_INVALID
    assert aa(pool, None, None, None, None, None, None, 0, None, 0, 32, 0.1, 0, 0, None, 0, None) == pa.PA_OK
    pa.pa_free_pool(pool)
    st, fpool = make_pool(16, 16, hkv=2, d=64, dtype=pa.PA_F32)
    assert pa.lib.pa_prefill(fpool, dummy, dummy, dummy, dummy, 4, dummy, 2, 4, 16, 0.1, None) \
        == pa.PA_ERR_UNSUPPORTED
    pa.pa_free_pool(fpool)


# ----------------------------------------------------------- sanitizers
def _driver_input(nb, bs, order, ops):
    lines = [f"{nb} {bs} {0 if order is None else nb} " + ("" if order is None else " ".join(map(str, order)))]
    for op in ops:
        if op[0] == "append":
            lines.append(f"a {op[1]} {op[2]}")
        elif op[0] == "batch":
            lines.append(f"b {op[1]} {len(op[2])} " + " ".join(map(str, op[2])))
        elif op[0] == "tokens":
            lines.append(f"k {op[1]} {len(op[2])} " + " ".join(map(str, op[2])))
        elif op[0] == "fork":
            lines.append(f"f {op[1]} {op[2]}")
        elif op[0] == "free":
            lines.append(f"x {op[1]}")
        else:
            lines.append(f"t {op[1]} {len(op[2])} " + " ".join(map(str, op[2])))
        lines.append("s")
    return "\n".join(lines) + "\n"


def _model_lines(nb, bs, order, ops):
    res = run_model(nb, bs, order, ops)
    lines = []
    for op, r, s in zip(ops, res[0::2], res[1::2]):
        if op[0] in ("append", "batch"):
            lines.append(" ".join([str(r[0])] + [str(x) for x in r[1]]))
        elif op[0] == "tokens":
            lines.append(" ".join([str(r[0])] + ([str(r[2])] + [str(x) for x in r[1]] if r[0] == 0 else [])))
        elif op[0] in ("fork", "free"):
            lines.append(str(r[0]))
        else:
            if r[0] == 0:
                lines.append(" ".join([str(r[0])] + [str(x) for x in r[1]] +
                                      [str(x) for row in r[2] for x in row]))
            else:
                lines.append(str(r[0]))
        lines.append(" ".join(map(str, s)))
    return lines


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_block_manager_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "bm_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-I", CSRC, os.path.join(CSRC, "block_manager.cpp"),
           os.path.join(os.path.dirname(__file__), "bm_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    for seed in range(6):
        rng = np.random.default_rng(200 + seed)
        nb, bs = 40, [8, 16, 32][seed % 3]
        order = rng.permutation(nb).tolist() if seed % 2 else None
        ops = random_ops(rng, 400) if seed < 4 else prefix_ops(rng, 300, bs)
        p = subprocess.run([exe], input=_driver_input(nb, bs, order, ops), capture_output=True, text=True,
                           env=env, timeout=120)
        assert p.returncode == 0, p.stderr[-3000:]
        assert p.stdout.strip().splitlines() == _model_lines(nb, bs, order, ops)


def test_fp8_pool_rules():
    assert make_pool(16, 16, hkv=2, d=64, dtype=pa.PA_FP8_E4M3)[0] == pa.PA_ERR_UNSUPPORTED   # needs D 128
    st, pool = make_pool(16, 16, hkv=2, d=128, dtype=pa.PA_FP8_E4M3)
    assert st == 0
    assert pa.lib.pa_pool_set_kv_scales(pool, 0.5, 0.25) == pa.PA_OK
    for bad in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (float("inf"), 1.0)):
        assert pa.lib.pa_pool_set_kv_scales(pool, *bad) == pa.PA_ERR_INVALID, bad
    dummy = 0x40000
    # prefill is bf16-only; an FP8 pool is refused before any launch
    assert pa.lib.pa_prefill(pool, dummy, dummy, dummy, dummy, 4, dummy, 2, 4, 16, 0.1, None) \
        == pa.PA_ERR_UNSUPPORTED
    pa.pa_free_pool(pool)
    st, bpool = make_pool(16, 16, hkv=2, d=128, dtype=pa.PA_BF16)
    assert pa.lib.pa_pool_set_kv_scales(bpool, 0.5, 0.5) == pa.PA_ERR_UNSUPPORTED
    pa.pa_free_pool(bpool)


def test_step_entry_points_validate_before_launch():
    st, pool = make_pool(64, 16, hkv=2, d=128)
    assert st == 0
    dummy = 0x40000
    d = pa._StepDesc()
    d.num_q_heads, d.scale, d.max_blocks = 8, 0.1, 16
    assert pa.lib.pa_step(pool, ctypes.byref(d), None) == pa.PA_OK          # every part empty: no-op
    d.num_new_tokens = 4                                                       # rows without pointers
    assert pa.lib.pa_step(pool, ctypes.byref(d), None) == pa.PA_ERR_INVALID
    d.key = d.value = d.slot_mapping = dummy
    d.dec_batch, d.dec_out, d.dec_q, d.dec_block_tables, d.dec_seq_lens = 2, dummy, dummy, dummy, dummy
    d.dec_max_seq_len = 16 * 16 + 1                                          # beyond max_blocks * bs
    assert pa.lib.pa_step(pool, ctypes.byref(d), None) == pa.PA_ERR_INVALID
    d.dec_max_seq_len = 256
    d.pre_batch, d.pre_out, d.pre_q, d.pre_cu_q_lens = 1, dummy, dummy + 2, dummy       # misaligned q
    d.pre_block_tables, d.pre_seq_lens, d.pre_max_q_len = dummy, dummy, 16
    assert pa.lib.pa_step(pool, ctypes.byref(d), None) == pa.PA_ERR_INVALID
    g = ctypes.c_void_p()
    assert pa.lib.pa_step_graph_create(pool, ctypes.byref(d), ctypes.byref(g)) == pa.PA_ERR_INVALID
    assert pa.lib.pa_step_graph_launch(None, None) == pa.PA_ERR_INVALID
    pa.lib.pa_step_graph_destroy(None)
    # pending copy-on-write copies must be run before a capture
    pa.pa_seq_append(pool, 0, 5)
    pa.pa_seq_fork(pool, 0, 1)
    pa.pa_seq_append(pool, 1, 1)
    assert pa.pa_pool_stats(pool)["pending_copies"] == 1
    e = pa._StepDesc()
    e.num_q_heads, e.scale, e.max_blocks = 8, 0.1, 16
    assert pa.lib.pa_step_graph_create(pool, ctypes.byref(e), ctypes.byref(g)) == pa.PA_ERR_INVALID
    assert "pending" in pa.pa_last_error()
    pa.pa_free_pool(pool)


def prefix_ops(rng, n_ops, bs):
    """Token-aware appends of sequences that share prompts, with frees (so
    cached blocks are found on the free list and evicted by later pops),
    continuations, forks and a few plain appends."""
    templates = [rng.integers(0, 30, 6 * bs) for _ in range(4)]
    ops, live, nxt = [], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.45 or not live:
            t = templates[int(rng.integers(0, 4))]
            ids = list(t[:int(rng.integers(bs, 6 * bs + 1))]) + list(rng.integers(0, 30, int(rng.integers(0, bs))))
            ops.append(("tokens", nxt, [int(x) for x in ids]))
            live.append(nxt)
            nxt += 1
        elif r < 0.6:
            s = live[int(rng.integers(0, len(live)))]
            ops.append(("tokens", s, [int(x) for x in rng.integers(0, 30, int(rng.integers(0, 2 * bs)))]))
        elif r < 0.8:
            s = live.pop(int(rng.integers(0, len(live))))
            ops.append(("free", s))
        elif r < 0.9:
            s = live[int(rng.integers(0, len(live)))]
            ops.append(("fork", s, nxt))
            live.append(nxt)
            nxt += 1
        else:
            s = live[int(rng.integers(0, len(live)))]
            ops.append(("append", s, int(rng.integers(0, bs))))
    return ops


@pytest.mark.parametrize("seed", range(6))
def test_prefix_cache_streams_match_model(seed):
    rng = np.random.default_rng(300 + seed)
    nb, bs = 96, [8, 16, 32][seed % 3]
    order = rng.permutation(nb) if seed % 2 else None
    ops = prefix_ops(rng, 400, bs)
    st, pool = make_pool(nb, bs, order)
    assert st == 0
    try:
        got, want = run_abi(pool, ops), run_model(nb, bs, order, ops)
        assert got == want
        cached = sum(r[2] for op, r in zip(ops, want[0::2]) if op[0] == "tokens")
        assert cached >= 5 * bs, f"stream exercised too few cached tokens ({cached})"
        print(f"seed {seed} bs {bs}: {cached} cached tokens, {pa.pa_pool_prefix_stats(pool)}")
    finally:
        pa.pa_free_pool(pool)


def test_tier_block_size_follows_the_page_tiers():
    """Tiers printed in the inference overview page, §3.3: bs 32 below 1024
    tokens, 16 from 1024 to below 8192, 8 from 8192 on."""
    for L, bs in [(0, 32), (1, 32), (1023, 32), (1024, 16), (4096, 16), (8191, 16), (8192, 8), (32768, 8),
                  (1 << 40, 8)]:
        assert pa.pa_tier_block_size(L) == bs, L
