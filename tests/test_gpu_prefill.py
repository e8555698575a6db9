"""GPU parity: chunked causal prefill (HIP bf16 MFMA, through the C ABI) vs the CPU oracle.

Same seeded inputs on both sides; the GPU cache is built by the C++ block
manager + HIP scatter, the oracle cache by the Python model + scatter oracle,
with never-written slots poisoned with NaN on both sides. Checks, to the bf16
bar (max-abs <= 2e-2, mean-abs <= 2e-3):
* small ragged shapes: chunk lengths that are not multiples of the query tile,
  contexts of 0 and past several KV tiles, block_size 8/16/32, G in {1,2,4,8},
  D in {64,128}, an empty chunk;
* the full 16 x 512-row workload over U[0,7680] cached tokens, every row and
  head;
* rows before the cache start (chunk longer than the cache) are zero;
* the last row of each chunk equals GPU decode at the same cache length.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle.attention as OA  # noqa: E402
import workloads as W  # noqa: E402
from oracle.cache import OracleCache  # noqa: E402

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def _h():
    from tests import harness
    return harness


def assert_close(got, ref, what):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    print(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= MAX_ABS, f"{what}: max abs err {err.max()}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean abs err {err.mean()}"


def build(wl, only=None):
    print(f"[build] {wl.name} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} bs={wl.block_size} "
          f"q_lens={wl.q_lens.tolist()[:8]} lens={wl.seq_lens.tolist()[:8]}", flush=True)
    gpu = _h().GpuCache(wl)
    ora = OracleCache(wl, only=only)
    assert np.array_equal(gpu.tables_host, ora.block_tables)
    return gpu, ora


SMALL = [
    # ctx, q_lens, Hq, Hkv, D, bs
    ([0, 0, 0], [1, 33, 130], 8, 2, 128, 32),
    ([5, 64, 100, 1000], [17, 64, 40, 129], 32, 8, 128, 32),
    ([37, 0, 300], [200, 7, 64], 8, 8, 128, 16),
    ([130, 3], [31, 90], 4, 2, 128, 8),
    ([70, 0, 500], [45, 128, 33], 16, 2, 128, 16),
    ([12, 250], [65, 100], 8, 1, 64, 32),
    ([0, 77], [129, 20], 4, 2, 64, 16),
    ([40, 0, 9], [0, 50, 300], 8, 2, 128, 32),     # an empty chunk
    # 72 short chunks at 4 q heads per kv head: 576 work items, 72 per XCD,
    # so each persistent workgroup takes items from three bands (the second
    # one in reverse order, the third one partial)
    (np.random.default_rng(61).integers(0, 200, 72).tolist(),
     np.random.default_rng(62).integers(1, 64, 72).tolist(), 32, 8, 64, 16),
]


@pytest.mark.parametrize("ctx,qlens,Hq,Hkv,D,bs", SMALL)
def test_prefill_small_shapes(ctx, qlens, Hq, Hkv, D, bs):
    wl = W.make_prefill("pf_small", ctx, qlens, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, dtype="bf16", seed=21)
    gpu, ora = build(wl)
    got = OA.widen(_h().to_host(gpu.prefill(), "bf16"), "bf16")
    torch.cuda.synchronize()
    ref, _ = OA.paged_prefill(wl.queries(), wl.cu_q_lens(), ora.k_cache, ora.v_cache, ora.block_tables,
                              ora.seq_lens, wl.scale, "bf16")
    assert_close(got, ref, f"prefill ctx={ctx} q={qlens} G={Hq // Hkv} D={D} bs={bs}")
    gpu.close()


def test_prefill_full_workload_all_rows():
    """Every row and head of the 16 x 512-row chunk workload over U[0,7680]
    cached tokens, against the oracle's matrix form of the same causal
    attention; a sample of rows also against its row-by-row form."""
    wl = W.config("prefill")
    gpu, ora = build(wl)
    got = OA.widen(_h().to_host(gpu.prefill(), "bf16"), "bf16")
    ref, _ = OA.paged_prefill_masked(wl.queries(), wl.cu_q_lens(), ora.k_cache, ora.v_cache, ora.block_tables,
                                     ora.seq_lens, wl.scale, "bf16")
    assert_close(got, ref, f"prefill full workload, all {got.shape[0]} rows x {got.shape[1]} heads")
    rows = [(b, i) for b in (0, wl.B - 1) for i in (0, 63, 64, int(wl.q_lens[b]) - 1)]
    ref_rows, _ = OA.paged_prefill(wl.queries(), wl.cu_q_lens(), ora.k_cache, ora.v_cache, ora.block_tables,
                                   ora.seq_lens, wl.scale, "bf16", rows=rows)
    cu = wl.cu_q_lens()
    idx = [cu[b] + i for b, i in rows]
    np.testing.assert_allclose(ref[idx], ref_rows[idx], rtol=0, atol=1e-12)
    gpu.close()


def test_prefill_rows_before_cache_start_are_zero():
    from paged_kv_cache_indirect_amd import pa_prefill
    # Cache of 20 tokens; a 30-row query chunk claims all of them: rows 0..9
    # sit before the cache start.
    wl = W.make_prefill("pf_neg", [0], [20], Hq=8, Hkv=2, D=128, block_size=16, dtype="bf16", seed=4)
    gpu, ora = build(wl)
    q30 = W.draw_values(np.random.default_rng(5), (30, 8, 128), "bf16")
    qd = _h().to_device(q30, "bf16", "cuda")
    out = torch.empty_like(qd)
    cu = torch.tensor([0, 30], dtype=torch.int32, device="cuda")
    pa_prefill(gpu.pool, out, qd, cu, gpu.block_tables, gpu.seq_lens, wl.scale, 30)
    got = OA.widen(_h().to_host(out, "bf16"), "bf16")
    ref, _ = OA.paged_prefill(q30, np.array([0, 30]), ora.k_cache, ora.v_cache, ora.block_tables,
                              ora.seq_lens, wl.scale, "bf16")
    assert np.array_equal(got[:10], np.zeros_like(got[:10]))
    assert_close(got, ref, "prefill with rows before the cache start")
    gpu.close()


def test_prefill_last_row_matches_gpu_decode():
    from paged_kv_cache_indirect_amd import pa_decode
    wl = W.make_prefill("pf_dec", [300, 0, 1500], [100, 64, 77], Hq=32, Hkv=8, D=128, block_size=32,
                        dtype="bf16", seed=6)
    gpu, _ = build(wl)
    pre = gpu.prefill().clone()
    cu = wl.cu_q_lens()
    last = torch.stack([gpu.q[int(cu[b + 1]) - 1] for b in range(wl.B)]).contiguous()
    dout = torch.empty_like(last)
    pa_decode(gpu.pool, dout, last, gpu.block_tables, gpu.seq_lens, wl.scale, int(wl.seq_lens.max()), 512,
              gpu.workspace_for(512))
    a = OA.widen(_h().to_host(pre, "bf16"), "bf16")[[int(cu[b + 1]) - 1 for b in range(wl.B)]]
    d = OA.widen(_h().to_host(dout, "bf16"), "bf16")
    err = np.abs(a - d).max()
    print(f"prefill last row vs decode: max_abs={err:.3e}", flush=True)
    assert err <= MAX_ABS
    gpu.close()
