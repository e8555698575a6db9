"""GPU parity of the decode's placement of work items on the CUs by length rank.

When a launch's (sequence, kv-head group, partition) items number more than
one but at most two per CU, the decode ranks the sequences by partition
length (on the host when the lengths come in the launch arguments, in the
kernel for device lengths of up to 256 sequences) and gives every workgroup
its item by rank. A wrong permutation would leave outputs unwritten or
written twice; these cases check every output against the oracle at the
boundaries of that path: ties in length everywhere, empty sequences, exactly
2 x CU items, one item past the CU count, 256 sequences (the largest the
kernel ranks) and 257 (not ranked). Tolerances as for the other decode tests
(bf16: max 2e-2, mean 2e-3).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle.attention as OA  # noqa: E402
import workloads as W  # noqa: E402
from oracle.cache import OracleCache  # noqa: E402

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


CASES = {"ties_2x": 1, "one_past": 2, "rank_256": 3, "unranked_257": 4}   # label -> length seed


def _build(label):
    """(lens, Hq, Hkv, pt), sized against the CU count of the device."""
    C = _cus()
    rng = np.random.default_rng(CASES[label])
    pt = 512
    if label == "ties_2x":          # NG = 4; every sequence 2 partitions of equal length: 2C items
        B = C // 4
        return [pt + pt // 2] * B, 32, 8, pt
    if label == "one_past":         # NG = 4; one partition each (zeros among them), one sequence with two
        B = C // 4 + 1
        lens = rng.integers(0, pt + 1, B).tolist()
        lens[0], lens[1], lens[-1] = 0, 0, 2 * pt - 7
        return lens, 32, 8, pt
    if label == "rank_256":         # NG = 1 (two kv heads, one workgroup); 256 sequences, 1-2 partitions
        lens = rng.integers(0, 2 * pt, 256).tolist()
        lens[5] = 0
        return lens, 8, 2, pt
    if label == "unranked_257":     # one sequence more than the kernel ranks
        lens = rng.integers(0, 2 * pt, 257).tolist()
        return lens, 8, 2, pt
    raise KeyError(label)


def _items(lens, Hkv, pt):
    groups = Hkv // 2 if Hkv % 2 == 0 else Hkv
    return groups * sum(max(1, -(-L // pt)) for L in lens)


@pytest.mark.parametrize("label", list(CASES))
def test_decode_placement_by_rank(label):
    from tests import harness
    from paged_kv_cache_indirect_amd import pa_append_decode_args
    lens, Hq, Hkv, pt = _build(label)
    C = _cus()
    n = _items(lens, Hkv, pt)
    print(f"[case] {label}: B={len(lens)} Hq={Hq} Hkv={Hkv} pt={pt} items={n} CUs={C}", flush=True)
    if label != "unranked_257":
        assert C < n <= 2 * C, (n, C)
    wl = W.make_decode(f"place_{label}", lens, Hq=Hq, Hkv=Hkv, D=128, block_size=16, dtype="bf16", seed=41)
    gpu = harness.GpuCache(wl)
    ora = OracleCache(wl)
    assert np.array_equal(gpu.tables_host, ora.block_tables)
    ref, _ = OA.paged_decode(wl.queries(), ora.k_cache, ora.v_cache, ora.block_tables, ora.seq_lens,
                             wl.scale, wl.dtype)
    ws = gpu.workspace_for(pt)
    outs = {"device lengths": OA.widen(harness.to_host(gpu.decode(pt, ws), "bf16"), "bf16")}
    if wl.B <= 128:   # lengths in the launch arguments, no new tokens
        out = torch.empty_like(gpu.q)
        rows = torch.zeros((wl.B, wl.Hkv, wl.D), dtype=torch.bfloat16, device="cuda")
        pa_append_decode_args(gpu.pool, out, gpu.q, rows, rows, np.full(wl.B, -1, np.int64), gpu.block_tables,
                              np.asarray(wl.seq_lens, np.int32), wl.scale, wl.max_seq_len, pt, ws)
        torch.cuda.synchronize()
        outs["launch-argument lengths"] = OA.widen(harness.to_host(out, "bf16"), "bf16")
    for what, got in outs.items():
        err = np.abs(got.astype(np.float64) - ref)
        print(f"  {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
        assert np.isfinite(got).all(), what
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (what, err.max(), err.mean())
    gpu.close()
