"""Build a workload's paged cache on the CPU with the oracle's own pieces.  (Test infrastructure.)

Replays the workload's op stream through the Python block-manager model,
scatters each appended row with the scatter oracle (FP8 caches store the
rows' E4M3 codes, quantised by ``oracle.fp8``), and exports the tables.
Shares nothing with the HIP path: only the seeded workload description comes
from the common generator module.
"""
from __future__ import annotations

import numpy as np

from .attention import widen
from .block_manager import BlockManagerModel
from .fp8 import NAN_CODE, quantize_e4m3
from .scatter import write_kv

SENTINEL_BF16 = 0x7FC1          # NaN patterns for never-written slots
SENTINEL_F32 = np.uint32(0x7FC00001).view(np.float32)


class OracleCache:
    """``only``: if given, K/V rows are scattered only for these sequences (the
    bookkeeping still covers all of them) — enough to compute sampled outputs
    of a large workload. A shared prefix is written with sequence 0."""

    def __init__(self, wl, poison: bool = True, only=None):
        self.wl = wl
        only = None if only is None else set(int(s) for s in only) | ({0} if wl.prefix_len else set())
        shape = (wl.num_blocks, wl.block_size, wl.Hkv, wl.D)
        if wl.cache_dtype == "fp8":
            self.k_cache = np.full(shape, NAN_CODE if poison else 0, dtype=np.uint8)
        elif wl.dtype == "bf16":
            self.k_cache = np.full(shape, SENTINEL_BF16 if poison else 0, dtype=np.uint16)
        else:
            self.k_cache = np.full(shape, SENTINEL_F32 if poison else 0, dtype=np.float32)
        self.v_cache = self.k_cache.copy()
        self.bm = BlockManagerModel(wl.num_blocks, wl.block_size, wl.free_order)
        for op in wl.ops:
            if op[0] == "append":
                seq, n = op[1], op[2]
                start = self.bm.lens.get(seq, 0)
                st, slots = self.bm.append(seq, n)
                if st != 0:
                    raise RuntimeError(f"oracle block manager refused {op}: status {st}")
                # Copy-on-write copies recorded by the append run before its rows land.
                for src, dst in self.bm.pending:
                    self.k_cache[dst] = self.k_cache[src]
                    self.v_cache[dst] = self.v_cache[src]
                self.bm.pending = []
                if only is None or seq in only:
                    k, v = wl.kv_rows(seq, start, n)
                    self._scatter(k, v, np.asarray(slots, dtype=np.int64))
            elif op[0] == "tokens":
                seq, ids = op[1], op[2]
                start = self.bm.lens.get(seq, 0)
                st, slots, _ = self.bm.append_tokens(seq, ids)
                if st != 0:
                    raise RuntimeError(f"oracle block manager refused a token append: status {st}")
                for src, dst in self.bm.pending:
                    self.k_cache[dst] = self.k_cache[src]
                    self.v_cache[dst] = self.v_cache[src]
                self.bm.pending = []
                if only is None or seq in only:
                    k, v = wl.kv_rows(seq, start, len(ids))
                    self._scatter(k, v, np.asarray(slots, dtype=np.int64))   # -1 slots (cached) skipped
            elif op[0] == "fork":
                assert self.bm.fork(op[1], op[2]) == 0
            elif op[0] == "free":
                assert self.bm.free_seq(op[1]) == 0
        wl.drop_cached()
        st, tables, lens = self.bm.block_tables(range(wl.B), wl.max_blocks)
        self.block_tables = np.asarray(tables, dtype=np.int32)
        self.seq_lens = np.asarray(lens, dtype=np.int32)

    def _scatter(self, k, v, slots):
        if self.wl.cache_dtype == "fp8":
            k = quantize_e4m3(widen(k, self.wl.dtype).astype(np.float32), self.wl.k_scale)
            v = quantize_e4m3(widen(v, self.wl.dtype).astype(np.float32), self.wl.v_scale)
        if len(slots) <= 4096:
            write_kv(self.k_cache, self.v_cache, k, v, slots)
            return
        # Large appends: same row-by-row definition, in bounded pieces.
        for a in range(0, len(slots), 4096):
            write_kv(self.k_cache, self.v_cache, k[a:a + 4096], v[a:a + 4096], slots[a:a + 4096])
