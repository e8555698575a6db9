"""GPU parity: the fused decode step (pa_append_decode: scatter of one new row
per sequence, fill-in of the new token's table entry, paged decode) against
the CPU oracle replaying the same steps, and against the separate
pa_write_kv + pa_block_tables + pa_decode path.

Each case builds the same workload three times: a fused-path pool, an
unfused-path pool (both through the C ABI) and the oracle's pool (Python
block-manager model + scatter oracle). Then every step:
* all three block managers hand out the same slots (bit-exact);
* the fused path keeps one device table, uploaded once before the first step
  and afterwards changed only by pa_append_decode itself;
* the fused output is within the bf16 (max-abs 2e-2, mean-abs 2e-3) or fp32
  (1e-5) bounds of the oracle's fp64 decode over its own pool and tables, and
  of the unfused output (the fused kernel adds the new token after the rest
  of its range, with an exact rescale, so the two round differently);
After the last step the fused pool equals the unfused pool and the oracle's
pool bit for bit (never-written slots poisoned with NaN on all sides), and the
fused path's device table equals the exported tables.
Both entry points are covered: slots and lengths in device memory
(pa_append_decode) and from host arrays in the launch arguments
(pa_append_decode_args). Cases cover steps that open new blocks (block sizes 8, 16, 32), copy-on-write
of a shared partly filled block (the new token's block is a fresh copy), rows
with slot -1 (no new token), several partitions per sequence, G in {1, 4, 8},
D in {64, 128}, and the 8B-shaped batch at full size.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle.attention as OA  # noqa: E402
import workloads as W  # noqa: E402
from oracle.cache import OracleCache  # noqa: E402

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def run_case(wl, steps, pt, skip=(), host_args=False):
    from tests import harness
    from paged_kv_cache_indirect_amd import (pa_append_decode, pa_append_decode_args, pa_block_tables,
                                             pa_decode, pa_seq_append_batch, pa_write_kv)
    print(f"[case] {wl.name} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} bs={wl.block_size} {wl.dtype} "
          f"steps={steps} pt={pt} skip={list(skip)} host_args={host_args}", flush=True)
    dev = "cuda"
    fused = harness.GpuCache(wl, device=dev)
    plain = harness.GpuCache(wl, device=dev)
    ora = OracleCache(wl)
    B, bs = wl.B, wl.block_size
    ids = np.arange(B, dtype=np.int64)
    msl = wl.max_seq_len + steps
    max_blocks = -(-msl // bs)
    t0, _ = pa_block_tables(fused.pool, ids, max_blocks)
    tab_fused = torch.from_numpy(t0).to(dev)      # changed only by pa_append_decode from here on
    ws = fused.workspace_for(pt, msl)
    ws_plain = plain.workspace_for(pt, msl)
    mx, mean = TOL[wl.dtype]
    for s in range(steps):
        k, v, q = wl.decode_step_inputs(s)
        sf = pa_seq_append_batch(fused.pool, ids, 1)[:, 0].copy()
        sp = pa_seq_append_batch(plain.pool, ids, 1)[:, 0].copy()
        st, so = ora.bm.append_batch(range(B), 1)
        assert st == 0
        so = np.asarray([x[0] for x in so], dtype=np.int64)
        assert np.array_equal(sf, sp) and np.array_equal(sf, so), "slots differ"
        for b in skip:          # no new token for b: its newest slot keeps what it holds
            sf[b] = sp[b] = so[b] = -1
        # oracle: pending copy-on-write copies, then the scatter
        for src, dst in ora.bm.pending:
            ora.k_cache[dst] = ora.k_cache[src]
            ora.v_cache[dst] = ora.v_cache[src]
        ora.bm.pending = []
        keep = so >= 0
        ora._scatter(k[keep], v[keep], so[keep])
        st, tables, lens = ora.bm.block_tables(range(B), max_blocks)
        tables = np.asarray(tables, dtype=np.int32)
        lens = np.asarray(lens, dtype=np.int32)
        ref, _ = OA.paged_decode(q, ora.k_cache, ora.v_cache, tables, lens, wl.scale, wl.dtype)

        kd = harness.to_device(k, wl.dtype, dev)
        vd = harness.to_device(v, wl.dtype, dev)
        qd = harness.to_device(q, wl.dtype, dev)
        lens_d = torch.from_numpy(lens).to(dev)
        # unfused: scatter, exported tables, decode
        pa_write_kv(plain.pool, kd, vd, torch.from_numpy(sp).to(dev))
        tp, lp = pa_block_tables(plain.pool, ids, max_blocks)
        assert np.array_equal(tp, tables) and np.array_equal(lp, lens), "tables differ from the model"
        out_plain = torch.empty_like(qd)
        pa_decode(plain.pool, out_plain, qd, torch.from_numpy(tp).to(dev), lens_d, wl.scale, msl, pt, ws_plain)
        # fused
        out_fused = torch.empty_like(qd)
        if host_args:     # slots and lengths from host arrays, in the launch arguments
            pa_append_decode_args(fused.pool, out_fused, qd, kd, vd, sf, tab_fused, lens, wl.scale, msl, pt, ws)
        else:
            pa_append_decode(fused.pool, out_fused, qd, kd, vd, torch.from_numpy(sf).to(dev), tab_fused, lens_d,
                             wl.scale, msl, pt, ws)
        torch.cuda.synchronize()
        got = OA.widen(harness.to_host(out_fused, wl.dtype), wl.dtype).astype(np.float64)
        unf = OA.widen(harness.to_host(out_plain, wl.dtype), wl.dtype).astype(np.float64)
        live = [b for b in range(B) if b not in skip]   # skipped rows read a poisoned slot
        err = np.abs(got[live] - ref[live])
        d = np.abs(got[live] - unf[live])
        print(f"  step {s}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} vs unfused {d.max():.3e}", flush=True)
        assert np.isfinite(got[live]).all()
        assert err.max() <= mx and err.mean() <= mean, f"step {s}: {err.max()} {err.mean()}"
        assert d.max() <= mx and d.mean() <= mean, f"step {s}: fused vs unfused {d.max()} {d.mean()}"
        if skip:   # rows without a new token decode exactly as pa_decode does
            assert torch.equal(_bits(out_fused[list(skip)]), _bits(out_plain[list(skip)]))
    for name in ("k_cache", "v_cache"):
        a = harness.to_host(getattr(fused, name), wl.dtype)
        bb = harness.to_host(getattr(plain, name), wl.dtype)
        oc = getattr(ora, name)
        assert np.array_equal(a.view(np.uint8), bb.view(np.uint8)), f"{name}: fused pool differs from unfused"
        assert np.array_equal(a.view(np.uint8), oc.view(np.uint8)), f"{name}: fused pool differs from the oracle"
    tp, _ = pa_block_tables(plain.pool, ids, max_blocks)
    assert np.array_equal(tab_fused.cpu().numpy(), tp), "device table differs from the exported tables"
    fused.close()
    plain.close()


SMALL = [
    # lens, Hq, Hkv, D, bs, dtype, pt, steps, skip
    ([15, 16, 31, 1, 47, 64, 100, 7, 0, 33], 8, 2, 128, 16, "bf16", 64, 3, ()),
    ([15, 16, 31, 1, 47, 64, 100, 7, 0, 33], 8, 2, 128, 16, "bf16", 0, 2, (3, 6)),  # their steps open no block
    ([7, 8, 9, 23, 24, 300, 511], 8, 1, 128, 8, "bf16", 128, 3, ()),
    ([31, 32, 33, 95, 200, 1000], 32, 4, 128, 32, "bf16", 0, 2, ()),
    ([5, 16, 17, 70, 129], 4, 4, 64, 16, "f32", 64, 3, ()),
    ([3, 40, 64, 65, 250], 16, 2, 64, 8, "bf16", 0, 2, ()),
]


@pytest.mark.parametrize("host_args", [False, True])
@pytest.mark.parametrize("lens,Hq,Hkv,D,bs,dtype,pt,steps,skip", SMALL)
def test_append_decode_small(lens, Hq, Hkv, D, bs, dtype, pt, steps, skip, host_args):
    need = sum(-(-(L + steps) // bs) for L in lens)
    wl = W.make_decode("append_small", lens, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, dtype=dtype, seed=11,
                       num_blocks=need + 8)
    run_case(wl, steps, pt, skip, host_args)


def test_append_decode_copy_on_write():
    """Six sequences forked from a 1000-token prefix whose last block is half
    full; four still share that block when the steps start, so the first
    step's appends take fresh copies of it (run by the fused call before its
    launch), whose ids the fused step writes into the device table."""
    wl = W.make_prefix_share("cow_step", 6, 1000, [0, 0, 0, 5, 0, 17], Hq=8, Hkv=2, D=128, block_size=16,
                             dtype="bf16", seed=21)
    run_case(wl, 2, 0)
    run_case(wl, 2, 256, host_args=True)


@pytest.mark.parametrize("host_args", [False, True])
def test_append_decode_gqa8b_full(host_args):
    run_case(W.config("gqa8b"), 2, 0, host_args=host_args)


def test_append_decode_rejects_fp8_pool():
    import paged_kv_cache_indirect_amd as pa
    from tests import harness
    wl = W.make_decode("fp8_small", [20, 40], Hq=8, Hkv=2, D=128, block_size=16, dtype="bf16", seed=3,
                       kv_dtype="fp8", k_scale=0.02, v_scale=0.02)
    cache = harness.GpuCache(wl)
    kd = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    slots = torch.full((2,), -1, dtype=torch.int64, device="cuda")
    with pytest.raises(pa.PaError) as e:
        pa.pa_append_decode(cache.pool, cache.out, cache.q, kd, kd, slots, cache.block_tables, cache.seq_lens,
                            wl.scale, wl.max_seq_len)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED
    cache.close()
