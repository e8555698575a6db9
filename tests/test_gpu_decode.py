"""GPU parity: KV scatter and paged decode (HIP, through the C ABI) vs the CPU oracle.

Same seeded inputs on both sides. The GPU side builds its pool with the C++
block manager + the HIP scatter; the oracle side with the Python model + the
scatter oracle. Checks:
* block tables and lengths: bit-exact;
* the scattered pools: bit-exact, including never-written slots, which both
  sides poison with NaN (so a kernel reading a tail slot or a padded table
  entry shows up as NaN in its output);
* decode outputs: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 max-abs
  <= 1e-5 — over the tiny, 8B-GQA, long-context and prefix-sharing
  workloads in full, and small ragged shapes
  spanning several partitions and a ragged tail, G in {1,2,4,8}, D in
  {64,128}, block_size in {8,16,32}, empty and one-token sequences;
* invariance of the output under the KV partition size.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle.attention as OA  # noqa: E402
import workloads as W  # noqa: E402
from oracle.cache import OracleCache  # noqa: E402


def _harness():
    from tests import harness
    return harness


TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}


def assert_close(got, ref, dtype, what=""):
    err = np.abs(got.astype(np.float64) - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = TOL[dtype]
    print(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
          f"rel_rms={err.max() / max(np.sqrt((ref ** 2).mean()), 1e-30):.3e}", flush=True)
    assert err.max() <= mx, f"{what}: max abs err {err.max()}"
    assert err.mean() <= mean, f"{what}: mean abs err {err.mean()}"


def widen_out(t, dtype):
    h = _harness().to_host(t, dtype)
    return OA.widen(h, dtype)


def build_both(wl, only=None):
    print(f"[build] {wl.name} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} bs={wl.block_size} "
          f"{wl.dtype} max_len={wl.max_seq_len} nb={wl.num_blocks}", flush=True)
    gpu = _harness().GpuCache(wl)
    ora = OracleCache(wl, only=only)
    assert np.array_equal(gpu.tables_host, ora.block_tables), "block tables differ"
    assert np.array_equal(gpu.lens_host, ora.seq_lens), "seq_lens differ"
    return gpu, ora


def oracle_out(wl, ora, seqs=None):
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    q = wl.queries()[seqs]
    out, _ = OA.paged_decode(q, ora.k_cache, ora.v_cache, ora.block_tables[seqs], ora.seq_lens[seqs],
                             wl.scale, wl.dtype)
    return out


def small(lens, Hq=8, Hkv=2, D=128, bs=16, dtype="bf16", seed=5, **kw):
    return W.make_decode(f"small{len(lens)}", lens, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, dtype=dtype,
                         seed=seed, **kw)


# ------------------------------------------------------------------ scatter
@pytest.mark.parametrize("name", ["tiny", "gqa8b", "prefix", "prefix_cow", "prompt_cache"])
def test_write_kv_bit_exact(name):
    wl = W.config(name)
    gpu, ora = build_both(wl)
    hk = _harness().to_host(gpu.k_cache, wl.dtype)
    hv = _harness().to_host(gpu.v_cache, wl.dtype)
    assert np.array_equal(hk.view(np.uint8), ora.k_cache.view(np.uint8)), "k_cache differs"
    assert np.array_equal(hv.view(np.uint8), ora.v_cache.view(np.uint8)), "v_cache differs"
    gpu.close()


def test_write_kv_skips_negative_and_out_of_range_slots():
    h = _harness()
    wl = small([20, 9], Hq=2, Hkv=2, D=64, bs=8, dtype="f32")
    gpu = h.GpuCache(wl)
    before = h.to_host(gpu.k_cache, "f32").copy()
    rng = np.random.default_rng(0)
    k = rng.standard_normal((4, 2, 64)).astype(np.float32)
    nslots = wl.num_blocks * wl.block_size
    gpu.write(k, k, np.array([-1, nslots, nslots + 100, -7]))
    torch.cuda.synchronize()
    assert np.array_equal(h.to_host(gpu.k_cache, "f32").view(np.uint8), before.view(np.uint8))
    gpu.close()


# ------------------------------------------------------------------- decode
def test_decode_tiny_fp32():
    wl = W.config("tiny")
    gpu, ora = build_both(wl)
    got = widen_out(gpu.decode(), wl.dtype)
    assert_close(got, oracle_out(wl, ora), wl.dtype, "tiny")
    gpu.close()


SMALL_CASES = [
    # lens, Hq, Hkv, D, bs, dtype, partition_tokens
    ([1, 7, 16, 17, 63, 64, 65, 500, 1025], 8, 2, 128, 16, "bf16", 128),
    ([0, 1, 300, 2049], 8, 2, 128, 16, "bf16", 512),
    ([33, 1000, 5], 4, 4, 128, 8, "bf16", 64),
    ([777, 64, 31], 16, 2, 128, 32, "bf16", 256),
    ([900, 2, 129], 2, 1, 64, 16, "bf16", 128),
    ([450, 3, 1], 16, 2, 64, 32, "bf16", 512),
    ([7, 16, 33, 50, 600], 2, 2, 64, 16, "f32", 64),
    ([300, 1, 129], 8, 2, 128, 8, "f32", 128),
    ([1300, 70], 8, 1, 64, 16, "f32", 256),
]


@pytest.mark.parametrize("lens,Hq,Hkv,D,bs,dtype,pt", SMALL_CASES)
def test_decode_small_shapes(lens, Hq, Hkv, D, bs, dtype, pt):
    wl = small(lens, Hq, Hkv, D, bs, dtype)
    gpu, ora = build_both(wl)
    ws = gpu.workspace_for(pt)
    got = widen_out(gpu.decode(pt, ws), dtype)
    assert_close(got, oracle_out(wl, ora), dtype, f"small {lens} G={Hq // Hkv} D={D} bs={bs} pt={pt}")
    gpu.close()


def test_decode_gqa8b_full():
    wl = W.config("gqa8b")
    gpu, ora = build_both(wl)
    ref = oracle_out(wl, ora)
    for pt in (512, 256, 1024, 2048, 4096, 0):   # 0: the library's choice (1536 tokens here)
        ws = gpu.workspace_for(pt)
        got = widen_out(gpu.decode(pt, ws), wl.dtype)
        assert_close(got, ref, wl.dtype, f"gqa8b pt={pt}")
    gpu.close()


def test_decode_long_context_full():
    """All 8 sequences of 32768 tokens, every q head, at the configured
    512-token partitions (64 per sequence), at 4096 and at the library's
    choice."""
    wl = W.config("long")
    gpu, ora = build_both(wl)
    ref = oracle_out(wl, ora)
    for pt in (512, 4096, 0):   # 0: the library's choice (8 partitions of 4096)
        got = widen_out(gpu.decode(pt, gpu.workspace_for(pt)), wl.dtype)
        assert_close(got, ref, wl.dtype, f"long pt={pt} (all {wl.B} sequences)")
    gpu.close()


def test_decode_prefix_sharing_full():
    wl = W.config("prefix")
    gpu, ora = build_both(wl)
    from paged_kv_cache_indirect_amd import pa_pool_stats
    st = pa_pool_stats(gpu.pool)
    assert st["shared_blocks"] == wl.prefix_len // wl.block_size
    got = widen_out(gpu.decode(512, gpu.workspace_for(512)), wl.dtype)
    assert_close(got, oracle_out(wl, ora), wl.dtype, "prefix")
    gpu.close()


def test_decode_copy_on_write_prefix_full():
    """32 sequences forked from a prefix whose last block is half full: the
    appends copy that block (HIP block copy before the scatter) and decode
    reads each sequence's own copy."""
    wl = W.config("prefix_cow")
    gpu, ora = build_both(wl)
    from paged_kv_cache_indirect_amd import pa_pool_stats
    st = pa_pool_stats(gpu.pool)
    model = ora.bm.stats()
    for key in ("free_blocks", "used_blocks", "shared_blocks", "filled_slots", "allocated_slots"):
        assert st[key] == model[key], key
    assert st["pending_copies"] == 0
    got = widen_out(gpu.decode(512, gpu.workspace_for(512)), wl.dtype)
    assert_close(got, oracle_out(wl, ora), wl.dtype, "prefix_cow")
    gpu.close()


def test_decode_prompt_cache_full():
    """48 requests appended with their token ids share a 1000-token prompt
    found by prefix-cache lookup (no fork): the C++ manager agrees with the
    model on tables, counters and cache keys; decode matches the oracle."""
    wl = W.config("prompt_cache")
    gpu, ora = build_both(wl)
    from paged_kv_cache_indirect_amd import pa_pool_prefix_stats, pa_pool_stats
    assert pa_pool_prefix_stats(gpu.pool) == ora.bm.prefix_stats()
    assert pa_pool_stats(gpu.pool)["shared_blocks"] == 1000 // wl.block_size
    got = widen_out(gpu.decode(512, gpu.workspace_for(512)), wl.dtype)
    assert_close(got, oracle_out(wl, ora), wl.dtype, "prompt_cache")
    gpu.close()


def test_write_kv_with_no_rows_runs_pending_copies():
    """T == 0 performs the pending copy-on-write copies and nothing else."""
    import paged_kv_cache_indirect_amd as pa
    h = _harness()
    nb, bs, hkv, d = 6, 8, 2, 64
    kc = torch.zeros((nb, bs, hkv, d), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    pool = pa.pa_alloc_pool(kc, vc, np.arange(nb, dtype=np.int32))
    try:
        slots = pa.pa_seq_append(pool, 0, 5)
        rows = torch.arange(5 * hkv * d, dtype=torch.float32, device="cuda").reshape(5, hkv, d) + 1
        pa.pa_write_kv(pool, rows, -rows, torch.from_numpy(np.asarray(slots, np.int64)).cuda())
        pa.pa_seq_fork(pool, 0, 1)
        pa.pa_seq_append(pool, 1, 2)
        (src, dst), = pa.pa_pool_pending_copies(pool)
        e = torch.empty((0, hkv, d), dtype=torch.float32, device="cuda")
        pa.pa_write_kv(pool, e, e, torch.empty(0, dtype=torch.int64, device="cuda"))
        torch.cuda.synchronize()
        assert pa.pa_pool_pending_copies(pool) == []
        k = h.to_host(kc, "f32")
        v = h.to_host(vc, "f32")
        assert np.array_equal(k[dst], k[src]) and np.array_equal(v[dst], v[src])
        assert np.array_equal(k[src][:5], rows.cpu().numpy())
        untouched = [b for b in range(nb) if b not in (src, dst)]
        assert not k[untouched].any() and not v[untouched].any()
        # A chain in one flush: 3 copies 0's block into b, 4 (a fork of 3)
        # copies b into c. b -> c must run after src -> b (separate launches).
        pa.pa_seq_fork(pool, 0, 3)
        pa.pa_seq_append(pool, 3, 1)
        pa.pa_seq_fork(pool, 3, 4)
        pa.pa_seq_append(pool, 4, 1)
        (s1, b), (s2, c) = pa.pa_pool_pending_copies(pool)
        assert s1 == src and s2 == b
        kc[b].fill_(7.0)
        kc[c].fill_(9.0)
        pa.pa_write_kv(pool, e, e, torch.empty(0, dtype=torch.int64, device="cuda"))
        torch.cuda.synchronize()
        k = h.to_host(kc, "f32")
        assert np.array_equal(k[b], k[src]) and np.array_equal(k[c], k[src])
    finally:
        pa.pa_free_pool(pool)


@pytest.mark.parametrize("bs,pt", [(8, 2048), (8, 8192), (16, 4096), (16, 16384), (32, 8000), (32, 16000)])
def test_decode_long_partitions(bs, pt):
    """Long partitions: each wave streams a quarter of its partition and holds
    the block ids of its range 64 at a time, so quarters of more than 64
    blocks take several windows (bs 8 / pt 8192: 4 windows per wave; bs 32 /
    pt 16000: quarters start mid-block). Lengths around one and two
    partitions, plus the library's default."""
    lens = [pt, pt - 1, pt + 1, 2 * pt, 17, 1, 0]
    wl = small(lens, Hq=8, Hkv=2, D=128, bs=bs, dtype="bf16", seed=21)
    gpu, ora = build_both(wl)
    ref = oracle_out(wl, ora)
    for p in (pt, 0):
        got = widen_out(gpu.decode(p, gpu.workspace_for(p)), "bf16")
        assert_close(got, ref, "bf16", f"bs={bs} pt={p} lens={lens}")
    gpu.close()


@pytest.mark.parametrize("B,pt", [(300, 64), (300, 0), (1100, 128), (1100, 0)])
def test_decode_large_batches(B, pt):
    """Batches past the sizes where the work list is compact (up to 1024
    sequences) and where one-partition batches are ordered: 300 sequences
    (compact list, several partitions each at pt 64) and 1100 (the plain
    (kv head, sequence, partition) mapping). Ragged short lengths, empty ones
    included."""
    rng = np.random.default_rng(B + pt)
    lens = rng.integers(0, 300, B).tolist()
    lens[0], lens[-1] = 0, 299
    wl = small(lens, Hq=8, Hkv=2, D=64, bs=16, dtype="bf16", seed=31)
    gpu, ora = build_both(wl)
    got = widen_out(gpu.decode(pt, gpu.workspace_for(pt)), "bf16")
    assert_close(got, oracle_out(wl, ora), "bf16", f"B={B} pt={pt}")
    gpu.close()


@pytest.mark.parametrize("lens,Hq,Hkv,D,bs,dtype,pt", [
    # 3 kv heads (one per workgroup, four waves each): 203 partitions x 3 = 609 items
    ([33000, 20500, 17000, 9000, 5000, 700, 1, 64, 511, 513, 1025, 12345], 6, 3, 128, 16, "bf16", 512),
    # 8 kv heads (pairs): odd partition counts, 135 partitions x 4 = 540 items
    ([33000, 20000, 513, 1, 9000, 4097], 32, 8, 128, 16, "bf16", 512),
    # fp32, head_dim 64, block size 8: 530 partitions x 1 = 530 items
    ([40000, 35000, 30000, 20000, 9000, 3, 257], 4, 2, 64, 8, "f32", 256),
])
def test_decode_many_items_one_partition_per_wave(lens, Hq, Hkv, D, bs, dtype, pt):
    """Plain decodes whose (sequence, kv-head group, partition) items exceed
    two per CU (512 on MI355X): each wave of a head then streams a whole
    partition and writes its own partial state. Sequences whose partition
    count is not a multiple of the waves per head leave waves of their last
    item empty; one-partition sequences write their output directly."""
    wl = small(lens, Hq, Hkv, D, bs, dtype, seed=71)
    gpu, ora = build_both(wl)
    got = widen_out(gpu.decode(pt, gpu.workspace_for(pt)), dtype)
    assert_close(got, oracle_out(wl, ora), dtype, f"many items G={Hq // Hkv} Hkv={Hkv} D={D} pt={pt}")
    gpu.close()


def test_decode_partition_invariance_and_max_seq_len_slack():
    from paged_kv_cache_indirect_amd import pa_decode
    wl = small([1, 40, 511, 512, 513, 1500], Hq=8, Hkv=2, D=128, bs=16, dtype="bf16", seed=9)
    gpu, ora = build_both(wl)
    ref = oracle_out(wl, ora)
    # A table wider than needed (padded with -1) lets the grid be sized for a
    # longer max_seq_len than any sequence has.
    wide = torch.full((wl.B, wl.max_blocks + 50), -1, dtype=torch.int32, device="cuda")
    wide[:, :wl.max_blocks] = gpu.block_tables
    outs = []
    for pt in (64, 128, 512, 2048):
        for slack in (0, 700):
            msl = wl.max_seq_len + slack
            out = torch.empty_like(gpu.q)
            pa_decode(gpu.pool, out, gpu.q, wide, gpu.seq_lens, wl.scale, msl, pt,
                      gpu.workspace_for(pt, msl))
            outs.append(widen_out(out, "bf16"))
            assert_close(outs[-1], ref, "bf16", f"pt={pt} slack={slack}")
    spread = max(np.abs(o - outs[0]).max() for o in outs)
    assert spread <= 2e-2
    gpu.close()


@pytest.mark.parametrize("lens,Hq,Hkv", [
    ([300] * 15 + [9000], 32, 8),          # one long context among short ones
    ([9000, 8500, 12000, 64, 1], 8, 2),    # long contexts plus two tiny ones
    ([8192, 9000, 10000], 8, 2),           # every sequence long: the shape rule stays
])
def test_decode_default_partition_from_device_lengths(lens, Hq, Hkv):
    """pa_decode with partition_tokens = 0 and max_seq_len >= 8192 picks its
    partition on the device from the lengths: bit-identical to pa_decode at
    the partition the host rule gives for the same lengths
    (pa_decode_partition_tokens_for_lengths), and within the bf16 bar of
    the oracle."""
    from paged_kv_cache_indirect_amd import pa_decode_partition_tokens_for_lengths, pa_decode_partition_tokens
    wl = small(lens, Hq=Hq, Hkv=Hkv, D=128, bs=16, seed=41)
    gpu, ora = build_both(wl)
    msl = wl.max_seq_len
    host_pt = pa_decode_partition_tokens_for_lengths(gpu.pool, wl.seq_lens, msl)
    if min(lens) >= 8192:
        assert host_pt == pa_decode_partition_tokens(gpu.pool, wl.B, msl)
    print(f"[auto partition] lens={lens} host rule {host_pt}", flush=True)
    auto = gpu.decode(0, gpu.workspace_for(0)).clone()
    fixed = gpu.decode(host_pt, gpu.workspace_for(host_pt)).clone()
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int16), fixed.view(torch.int16)), "device choice differs from the host rule"
    assert_close(widen_out(auto, wl.dtype), oracle_out(wl, ora), wl.dtype, f"auto partition {lens}")
    gpu.close()
