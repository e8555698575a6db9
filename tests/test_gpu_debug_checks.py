"""GPU: the library's debug checks reject duplicate slots and block ids outside
the pool before anything is launched, and let valid calls through unchanged.

Every rejected call here is refused on the host (the checks copy the integer
inputs to the host first), so no kernel ever sees the bad input.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import workloads as W  # noqa: E402


@pytest.fixture
def debug_on():
    import paged_kv_cache_indirect_amd as pa
    was = pa.pa_set_debug_checks(True)
    yield pa
    pa.pa_set_debug_checks(was)


def _small():
    from tests import harness
    wl = W.make_decode("dbg", [20, 37, 5], Hq=8, Hkv=2, D=128, block_size=16, dtype="bf16", seed=12)
    return wl, harness.GpuCache(wl)


def test_duplicate_slots_are_rejected(debug_on):
    pa = debug_on
    print("[debug checks] duplicate slots", flush=True)
    wl, cache = _small()
    try:
        before = cache.k_cache.clone()
        rows = torch.ones((3, wl.Hkv, wl.D), dtype=torch.bfloat16, device="cuda")
        dup = torch.tensor([5, 9, 5], dtype=torch.int64, device="cuda")
        with pytest.raises(pa.PaError) as e:
            pa.pa_write_kv(cache.pool, rows, rows, dup)
        assert e.value.status == pa.PA_ERR_INVALID and "twice" in str(e.value)
        torch.cuda.synchronize()
        assert torch.equal(cache.k_cache.view(torch.int16), before.view(torch.int16))   # nothing launched
        # Negative (skipped) slots may repeat; distinct slots pass.
        ok = torch.tensor([-1, 9, -1], dtype=torch.int64, device="cuda")
        pa.pa_write_kv(cache.pool, rows, rows, ok)
        torch.cuda.synchronize()
    finally:
        cache.close()


def test_bad_table_ids_are_rejected(debug_on):
    pa = debug_on
    print("[debug checks] table ids", flush=True)
    wl, cache = _small()
    try:
        cache.decode(0, cache.workspace_for(0))          # valid tables pass
        torch.cuda.synchronize()
        for bad in (wl.num_blocks, -1, 1 << 30):
            tab = cache.block_tables.clone()
            tab[1, 2] = bad                             # sequence 1 (37 tokens) reads blocks 0..2
            with pytest.raises(pa.PaError) as e:
                pa.pa_decode(cache.pool, cache.out, cache.q, tab, cache.seq_lens, wl.scale, wl.max_seq_len)
            assert e.value.status == pa.PA_ERR_INVALID and "block_tables[1][2]" in str(e.value)
        # Entries past ceil(L / bs) are never read: anything goes there.
        wide = torch.full((wl.B, wl.max_blocks + 3), 1 << 30, dtype=torch.int32, device="cuda")
        for b, L in enumerate(wl.seq_lens.tolist()):
            n = -(-L // wl.block_size)
            wide[b, :n] = cache.block_tables[b, :n]
        pa.pa_decode(cache.pool, cache.out, cache.q, wide, cache.seq_lens, wl.scale, wl.max_seq_len)
        torch.cuda.synchronize()
    finally:
        cache.close()


def test_fused_append_may_leave_its_own_entry_unset(debug_on):
    pa = debug_on
    print("[debug checks] fused append", flush=True)
    wl, cache = _small()
    try:
        ids = np.arange(wl.B, dtype=np.int64)
        slots = pa.pa_seq_append_batch(cache.pool, ids, 1)[:, 0].copy()
        mb = wl.max_blocks + 1
        tables, lens = pa.pa_block_tables(cache.pool, ids, mb)
        # sequence 0 grows from 20 to 21 tokens (its block 1 is already in the
        # table); sequence 2 from 5 to 6. Blank the entries of every new token's
        # block: the call fills them in itself.
        for b, L in enumerate(lens.tolist()):
            tables[b, (L - 1) // wl.block_size] = -1
        tab = torch.from_numpy(tables).cuda()
        k, v, q = wl.decode_step_inputs(0)
        from tests import harness
        kd, vd, qd = (harness.to_device(x, "bf16", "cuda") for x in (k, v, q))
        out = torch.empty_like(qd)
        pa.pa_append_decode_args(cache.pool, out, qd, kd, vd, slots, tab, lens, wl.scale, int(lens.max()))
        torch.cuda.synchronize()
        # A duplicated slot in the step is refused.
        dup = slots.copy()
        dup[1] = dup[0]
        with pytest.raises(pa.PaError) as e:
            pa.pa_append_decode_args(cache.pool, out, qd, kd, vd, dup, tab, lens, wl.scale, int(lens.max()))
        assert e.value.status == pa.PA_ERR_INVALID
    finally:
        cache.close()


def test_prefill_tables_are_checked(debug_on):
    pa = debug_on
    print("[debug checks] prefill tables", flush=True)
    from tests import harness
    wl = W.make_prefill("dbg_pf", [40, 0], [30, 20], Hq=8, Hkv=2, D=128, block_size=32, dtype="bf16", seed=13)
    cache = harness.GpuCache(wl)
    try:
        cache.prefill()
        torch.cuda.synchronize()
        tab = cache.block_tables.clone()
        tab[0, 1] = wl.num_blocks + 7
        with pytest.raises(pa.PaError) as e:
            pa.pa_prefill(cache.pool, cache.out, cache.q, cache.cu_q_lens, tab, cache.seq_lens, wl.scale, 30)
        assert e.value.status == pa.PA_ERR_INVALID
    finally:
        cache.close()
