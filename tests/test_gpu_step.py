"""GPU: one mixed serving step (scatter + decode + chunked prefill) through
pa_step and through a captured HIP graph (pa_step_graph_*).

* The captured graph, replayed over several steps with the host refreshing
  its fixed input buffers (and unrelated eager GPU work plus synchronisations
  between replays), gives outputs bit-identical to the eager pa_step path on
  an identical second pool, every replay.
* The eager step matches the fp64 oracle (decode and prefill rows) at the
  last step, within the bf16 tolerances (max-abs <= 2e-2, mean-abs <= 2e-3),
  and both pools' tables match the oracle's block manager.

Three batches: a small decode, beside which the prefill keeps every CU, and
two decodes of 140-160 sequences (one item for every second CU or more),
beside which the prefill serves its items with fewer workgroups and leaves
the other CUs to the decode: head_dim 128 with 4 q heads per kv head and
100-row chunks, and head_dim 64 with 8 per kv head, block size 32 and 70-row
chunks; both chunk lengths end in a partial query tile.
"""
import dataclasses

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


def widen(t):
    return OA.widen(_harness().to_host(t, "bf16"), "bf16")


def small_mixed():
    return W.make_mixed("mixed_small", [100, 7, 530, 1, 64], [0, 45, 300], 40, 3, Hq=8, Hkv=2, D=128,
                        block_size=16, dtype="bf16", seed=31)


def wide_mixed():
    rng = np.random.default_rng(47)
    dec = rng.integers(1, 300, 160).tolist()
    pre = [0, 45, 700, 2500, 3000] + rng.integers(0, 3000, 19).tolist()
    return W.make_mixed("mixed_wide", dec, pre, 100, 2, Hq=8, Hkv=2, D=128, block_size=16, dtype="bf16", seed=47)


def wide_mixed_d64_g8():
    rng = np.random.default_rng(53)
    dec = rng.integers(1, 200, 140).tolist()
    pre = [0, 31, 900, 2000] + rng.integers(0, 2000, 12).tolist()
    return W.make_mixed("mixed_wide_d64", dec, pre, 70, 2, Hq=16, Hkv=2, D=64, block_size=32, dtype="bf16",
                        seed=53)


@pytest.mark.parametrize("make", [small_mixed, wide_mixed, wide_mixed_d64_g8],
                         ids=["small_decode", "prefill_beside_decode", "prefill_beside_decode_d64_g8"])
def test_graph_replays_match_eager_and_oracle(make):
    wl = make()
    h = _harness()
    eager = h.MixedRunner(wl, use_graph=False)
    graph = h.MixedRunner(wl, use_graph=True)
    try:
        for s in range(wl.plan["steps"]):
            print(f"[step {s}] eager + graph", flush=True)
            eager.prepare(s)
            graph.prepare(s)
            assert np.array_equal(eager.host_tables, graph.host_tables)
            eager.launch()
            graph.launch()
            torch.cuda.synchronize()
            junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
            torch.cuda.synchronize()
            assert torch.isfinite(junk)
            assert torch.equal(eager.dec_out, graph.dec_out), f"step {s}: decode outputs differ"
            assert torch.equal(eager.pre_out, graph.pre_out), f"step {s}: prefill outputs differ"
        # replay the last step once more: same inputs, same outputs
        graph.launch()
        torch.cuda.synchronize()
        assert torch.equal(eager.dec_out, graph.dec_out) and torch.equal(eager.pre_out, graph.pre_out)

        last = wl.plan["steps"] - 1
        ora = OracleCache(dataclasses.replace(wl, ops=W.ops_through(wl, last)))
        Bd = wl.plan["Bd"]
        assert np.array_equal(eager.host_tables, ora.block_tables)
        qd, qp = W.mixed_step_queries(wl, last)
        ref_d, _ = OA.paged_decode(qd, ora.k_cache, ora.v_cache, ora.block_tables[:Bd], ora.seq_lens[:Bd],
                                   wl.scale, wl.dtype)
        cu = np.arange(wl.plan["Bp"] + 1, dtype=np.int32) * wl.plan["chunk"]
        ref_p, _ = OA.paged_prefill(qp, cu, ora.k_cache, ora.v_cache, ora.block_tables[Bd:], ora.seq_lens[Bd:],
                                    wl.scale, wl.dtype)
        for got, ref, what in ((widen(eager.dec_out), ref_d, "decode"), (widen(eager.pre_out), ref_p, "prefill")):
            err = np.abs(got - ref)
            print(f"mixed step {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
            assert err.max() <= 2e-2 and err.mean() <= 2e-3, what
    finally:
        eager.close()
        graph.close()
