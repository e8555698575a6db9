"""GPU: pa_decode_static (no allocation, partial states in the library's static
device scratch) against pa_decode (caller's workspace) through the C ABI.

Two calls in a row on one pool's GPU, the second with a smaller batch and
shorter sequences, each split into several KV partitions so that the scratch
is used: outputs equal pa_decode's bit for bit (same kernels, same partition)
and the oracle's to the bf16 bar. A shape whose partial states exceed the
scratch is refused before anything is launched.
"""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle.attention as OA  # noqa: E402
import workloads as W  # noqa: E402
from oracle.cache import OracleCache  # noqa: E402

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def _lib():
    import paged_kv_cache_indirect_amd as pa
    return pa


def _decode_both(pa, cache, wl, pt):
    """pa_decode with a torch workspace, then pa_decode_static, both through
    the raw C ABI on torch's current stream; returns both outputs."""
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    B, Hq, D = wl.B, wl.Hq, wl.D
    mb = int(cache.block_tables.shape[1])
    need = pa.pa_decode_workspace_bytes(B, Hq, D, wl.max_seq_len, pt)
    assert 0 < need <= pa.PA_DECODE_STATIC_SCRATCH_BYTES, need
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref_out = torch.full_like(cache.q, float("nan"))
    st = pa.lib.pa_decode(cache.pool, ref_out.data_ptr(), cache.q.data_ptr(), cache.block_tables.data_ptr(), mb,
                          cache.seq_lens.data_ptr(), B, Hq, ctypes.c_float(wl.scale), wl.max_seq_len, pt,
                          ws.data_ptr(), need, stream)
    assert st == pa.PA_OK, pa.pa_last_error()
    out = torch.full_like(cache.q, float("nan"))
    st = pa.lib.pa_decode_static(cache.pool, out.data_ptr(), cache.q.data_ptr(), cache.block_tables.data_ptr(), mb,
                                 cache.seq_lens.data_ptr(), B, Hq, ctypes.c_float(wl.scale), wl.max_seq_len, pt,
                                 stream)
    assert st == pa.PA_OK, pa.pa_last_error()
    torch.cuda.synchronize()
    return ref_out, out


def _check_against_oracle(wl, cache, out):
    ora = OracleCache(wl)
    assert np.array_equal(cache.tables_host, ora.block_tables)
    ref, _ = OA.paged_decode(wl.queries(), ora.k_cache, ora.v_cache, ora.block_tables, ora.seq_lens, wl.scale,
                             wl.dtype)
    from tests import harness
    got = OA.widen(harness.to_host(out, wl.dtype), wl.dtype)
    err = np.abs(got - ref)
    print(f"  vs oracle: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert np.isfinite(got).all() and err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_decode_static_matches_decode_twice_second_smaller():
    pa = _lib()
    from tests import harness
    cases = [
        # a larger batch first, then a smaller one (fewer sequences, shorter, other partition)
        (W.make_decode("static_a", [3000, 1717, 4096, 900, 2500, 64, 3333, 1200], Hq=32, Hkv=8, D=128,
                       block_size=16, dtype="bf16", seed=31), 512),
        (W.make_decode("static_b", [700, 129, 1500], Hq=32, Hkv=8, D=128, block_size=16, dtype="bf16",
                       seed=32), 256),
    ]
    for wl, pt in cases:
        print(f"[no-alloc] {wl.name} B={wl.B} max_len={wl.max_seq_len} pt={pt}", flush=True)
        cache = harness.GpuCache(wl)
        try:
            ref_out, out = _decode_both(pa, cache, wl, pt)
            assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "differs from pa_decode"
            _check_against_oracle(wl, cache, out)
        finally:
            cache.close()


def test_decode_static_binding_and_default_partition():
    pa = _lib()
    from tests import harness
    wl = W.make_decode("static_c", [5, 40, 1000, 2049], Hq=8, Hkv=2, D=128, block_size=16, dtype="f32", seed=33)
    print(f"[no-alloc] {wl.name} fp32 default partition", flush=True)
    cache = harness.GpuCache(wl)
    try:
        out = torch.empty_like(cache.q)
        pa.pa_decode_static(cache.pool, out, cache.q, cache.block_tables, cache.seq_lens, wl.scale, wl.max_seq_len,
                            64)
        ref_out = torch.empty_like(cache.q)
        pa.pa_decode(cache.pool, ref_out, cache.q, cache.block_tables, cache.seq_lens, wl.scale, wl.max_seq_len, 64)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        ora = OracleCache(wl)
        ref, _ = OA.paged_decode(wl.queries(), ora.k_cache, ora.v_cache, ora.block_tables, ora.seq_lens, wl.scale,
                                 "f32")
        assert np.abs(out.cpu().numpy().astype(np.float64) - ref).max() <= 1e-5
    finally:
        cache.close()


def test_decode_static_refuses_shapes_beyond_its_scratch():
    pa = _lib()
    from tests import harness
    wl = W.make_decode("static_big", [100, 200], Hq=32, Hkv=8, D=128, block_size=16, dtype="bf16", seed=34)
    cache = harness.GpuCache(wl)
    try:
        out = torch.zeros_like(cache.q)
        # 2 sequences x 32 heads x (2^20 / 64 partitions) x 130 floats > 32 MiB
        msl = 1 << 20
        tab = torch.full((wl.B, msl // wl.block_size), -1, dtype=torch.int32, device="cuda")
        tab[:, :cache.block_tables.shape[1]] = cache.block_tables
        with pytest.raises(pa.PaError) as e:
            pa.pa_decode_static(cache.pool, out, cache.q, tab, cache.seq_lens, wl.scale, msl, 64)
        assert e.value.status == pa.PA_ERR_UNSUPPORTED and "scratch" in str(e.value)
        torch.cuda.synchronize()
        assert not out.view(torch.int16).any()     # nothing ran
    finally:
        cache.close()
