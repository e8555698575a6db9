"""Populate a device pool from a seeded workload through the C ABI.

Used by the GPU tests, the smoke check and the benchmark. Every step runs
through libpa: the host block manager hands out slots (pa_seq_append /
pa_seq_fork), the HIP scatter writes K/V (pa_write_kv), tables come from
pa_block_tables. Torch only allocates device memory and supplies the stream.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from paged_kv_cache_indirect_amd import (pa_alloc_pool, pa_block_tables, pa_decode, pa_decode_workspace_bytes, pa_free_pool,
               pa_pool_set_kv_scales, pa_prefill, pa_seq_append, pa_seq_append_tokens, pa_seq_fork, pa_seq_free,
               pa_write_kv)

# NaN bit patterns used to poison never-written cache slots.
SENTINEL_BF16 = 0x7FC1
SENTINEL_F32 = 0x7FC00001
SENTINEL_FP8 = 0x7F


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host values (float32, or uint16 bf16 bits) -> device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> host float32 array, uint16 bf16 bits, or uint8 E4M3 codes."""
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if dtype == "fp8":
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


class GpuCache:
    """A device pool filled with a workload's K/V, plus its tables and queries."""

    def __init__(self, wl, device="cuda", poison: bool = True, chunk_tokens: int = 1 << 16):
        self.wl = wl
        self.device = device
        tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn}[wl.cache_dtype]
        shape = (wl.num_blocks, wl.block_size, wl.Hkv, wl.D)
        self.k_cache = torch.empty(shape, dtype=tdt, device=device)
        self.v_cache = torch.empty(shape, dtype=tdt, device=device)
        if poison:
            if wl.cache_dtype == "fp8":
                self.k_cache.view(torch.uint8).fill_(SENTINEL_FP8)
                self.v_cache.view(torch.uint8).fill_(SENTINEL_FP8)
            elif wl.dtype == "bf16":
                self.k_cache.view(torch.int16).fill_(SENTINEL_BF16)
                self.v_cache.view(torch.int16).fill_(SENTINEL_BF16)
            else:
                self.k_cache.view(torch.int32).fill_(SENTINEL_F32)
                self.v_cache.view(torch.int32).fill_(SENTINEL_F32)
        self.pool = pa_alloc_pool(self.k_cache, self.v_cache, wl.free_order)
        if wl.cache_dtype == "fp8":
            pa_pool_set_kv_scales(self.pool, wl.k_scale, wl.v_scale)
        self.slots = {}
        for op in wl.ops:
            if op[0] == "append":
                seq, n = op[1], op[2]
                start = self.slots_len(seq)
                slots = pa_seq_append(self.pool, seq, n)
                self.slots.setdefault(seq, []).append(slots)
                for a in range(0, n, chunk_tokens):       # bounded host→device staging
                    m = min(chunk_tokens, n - a)
                    k, v = wl.kv_rows(seq, start + a, m)
                    self.write(k, v, slots[a:a + m])
            elif op[0] == "tokens":
                seq, ids = op[1], op[2]
                start = self.slots_len(seq)
                slots, _ = pa_seq_append_tokens(self.pool, seq, ids)
                self.slots.setdefault(seq, []).append(slots)
                for a in range(0, len(ids), chunk_tokens):   # -1 slots (cached blocks) are skipped
                    m = min(chunk_tokens, len(ids) - a)
                    k, v = wl.kv_rows(seq, start + a, m)
                    self.write(k, v, slots[a:a + m])
            elif op[0] == "fork":
                pa_seq_fork(self.pool, op[1], op[2])
                self.slots[op[2]] = list(self.slots.get(op[1], []))
            elif op[0] == "free":
                pa_seq_free(self.pool, op[1])
                self.slots.pop(op[1], None)
        wl.drop_cached()
        tables, lens = pa_block_tables(self.pool, list(range(wl.B)), wl.max_blocks)
        self.tables_host, self.lens_host = tables, lens
        self.block_tables = torch.from_numpy(tables).to(device)
        self.seq_lens = torch.from_numpy(lens).to(device)
        self.q = to_device(wl.queries(), wl.dtype, device)
        self.out = torch.empty_like(self.q)
        self.cu_q_lens = None
        if wl.kind == "prefill":
            self.cu_q_lens = torch.from_numpy(wl.cu_q_lens()).to(device)
        torch.cuda.synchronize()

    def slots_len(self, seq: int) -> int:
        return sum(len(s) for s in self.slots.get(seq, []))

    def write(self, k: np.ndarray, v: np.ndarray, slots: np.ndarray) -> None:
        kd = to_device(k, self.wl.dtype, self.device)
        vd = to_device(v, self.wl.dtype, self.device)
        sd = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).to(self.device)
        pa_write_kv(self.pool, kd, vd, sd)

    # ---------------------------------------------------------- hot path
    def workspace_for(self, partition_tokens: int = 0, max_seq_len: Optional[int] = None):
        msl = self.wl.max_seq_len if max_seq_len is None else max_seq_len
        need = pa_decode_workspace_bytes(self.wl.B, self.wl.Hq, self.wl.D, msl, partition_tokens)
        return torch.empty(need, dtype=torch.uint8, device=self.device) if need else None

    def decode(self, partition_tokens: int = 0, workspace=None, out=None, max_seq_len=None, stream=None):
        out = self.out if out is None else out
        msl = self.wl.max_seq_len if max_seq_len is None else max_seq_len
        pa_decode(self.pool, out, self.q, self.block_tables, self.seq_lens, self.wl.scale, msl,
                  partition_tokens, workspace, stream)
        return out

    def prefill(self, out=None, stream=None):
        out = self.out if out is None else out
        pa_prefill(self.pool, out, self.q, self.cu_q_lens, self.block_tables, self.seq_lens,
                   self.wl.scale, int(self.wl.q_lens.max()), stream)
        return out

    def close(self) -> None:
        if self.pool:
            pa_free_pool(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MixedRunner:
    """Mixed decode + chunked-prefill serving steps of a ``make_mixed``
    workload on one pool, through pa_step (eager) or a captured step graph.

    The pool starts from the workload's initial appends. Every step's device
    inputs live in fixed buffers allocated once (new K/V rows, slots, both
    sets of tables and lengths, cu_q_lens, queries, outputs, workspace), so a
    graph captured on the first step replays later steps after the host
    refreshes those buffers: append on the host block manager, export tables,
    one host-to-device copy per buffer.
    """

    def __init__(self, wl, device="cuda", use_graph: bool = False, partition_tokens: int = 0):
        from paged_kv_cache_indirect_amd import StepDesc
        p = wl.plan
        self.wl, self.device, self.use_graph = wl, device, use_graph
        self.Bd, self.Bp, self.chunk = p["Bd"], p["Bp"], p["chunk"]
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        shape = (wl.num_blocks, wl.block_size, wl.Hkv, wl.D)
        self.k_cache = torch.zeros(shape, dtype=tdt, device=device)
        self.v_cache = torch.zeros(shape, dtype=tdt, device=device)
        self.pool = pa_alloc_pool(self.k_cache, self.v_cache, wl.free_order)
        self.lens = {}
        for op in wl.ops[:p["n_init"]]:
            seq, n = op[1], op[2]
            slots = pa_seq_append(self.pool, seq, n)
            k, v = wl.kv_rows(seq, 0, n)
            if n:
                pa_write_kv(self.pool, to_device(k, wl.dtype, device), to_device(v, wl.dtype, device),
                            torch.from_numpy(slots).to(device))
            self.lens[seq] = n
        self.max_blocks = wl.max_blocks
        self.max_seq_len = wl.max_seq_len
        T = self.Bd + self.Bp * self.chunk
        self.T = T
        mk = lambda *s, dt=tdt: torch.zeros(s, dtype=dt, device=device)  # noqa: E731
        self.key, self.value = mk(T, wl.Hkv, wl.D), mk(T, wl.Hkv, wl.D)
        self.slots = mk(T, dt=torch.int64)
        self.dec_q, self.dec_out = mk(self.Bd, wl.Hq, wl.D), mk(self.Bd, wl.Hq, wl.D)
        self.dec_tables = mk(self.Bd, self.max_blocks, dt=torch.int32)
        self.dec_lens = mk(self.Bd, dt=torch.int32)
        self.pre_q, self.pre_out = mk(self.Bp * self.chunk, wl.Hq, wl.D), mk(self.Bp * self.chunk, wl.Hq, wl.D)
        self.pre_tables = mk(self.Bp, self.max_blocks, dt=torch.int32)
        self.pre_lens = mk(self.Bp, dt=torch.int32)
        self.cu = torch.from_numpy(np.arange(self.Bp + 1, dtype=np.int32) * self.chunk).to(device)
        need = pa_decode_workspace_bytes(self.Bd, wl.Hq, wl.D, self.max_seq_len, partition_tokens)
        self.workspace = mk(max(need, 16), dt=torch.uint8)
        self.desc = StepDesc(num_q_heads=wl.Hq, scale=wl.scale, max_blocks=self.max_blocks, key=self.key,
                             value=self.value, slot_mapping=self.slots, dec_out=self.dec_out, dec_q=self.dec_q,
                             dec_block_tables=self.dec_tables, dec_seq_lens=self.dec_lens,
                             dec_max_seq_len=self.max_seq_len, partition_tokens=partition_tokens,
                             workspace=self.workspace, pre_out=self.pre_out, pre_q=self.pre_q,
                             pre_cu_q_lens=self.cu, pre_block_tables=self.pre_tables, pre_seq_lens=self.pre_lens,
                             pre_max_q_len=self.chunk)
        self.graph = None
        self.host_tables = None
        self.staged = None
        torch.cuda.synchronize()

    def stage_inputs(self) -> None:
        """Generate every step's new K/V rows and queries up front and keep them
        in HBM, so that prepare() only moves them into the step buffers."""
        import workloads as W
        wl, p = self.wl, self.wl.plan
        lens = dict(self.lens)
        keys, vals, qds, qps = [], [], [], []
        for step in range(p["steps"]):
            ks, vs = [], []
            for seq in range(self.Bd + self.Bp):
                n = 1 if seq < self.Bd else self.chunk
                k, v = wl.kv_rows(seq, lens[seq], n)
                ks.append(k)
                vs.append(v)
                lens[seq] += n
            keys.append(np.concatenate(ks))
            vals.append(np.concatenate(vs))
            qd, qp = W.mixed_step_queries(wl, step)
            qds.append(qd)
            qps.append(qp)
        dev = self.device
        self.staged = [to_device(np.stack(x), wl.dtype, dev) for x in (keys, vals, qds, qps)]
        torch.cuda.synchronize()

    def prepare(self, step: int) -> None:
        """Host side of step ``step``: appends on the block manager and the
        table export, then the step's inputs into the fixed buffers (device
        copies from the staged inputs; one upload each for slots, tables,
        lengths)."""
        if getattr(self, "staged", None) is None:
            self.stage_inputs()
        slots = []
        order = list(range(self.Bd + self.Bp))
        for seq in order:
            n = 1 if seq < self.Bd else self.chunk
            slots.append(pa_seq_append(self.pool, seq, n))
            self.lens[seq] += n
        tables, lens = pa_block_tables(self.pool, order, self.max_blocks)
        self.host_tables, self.host_lens = tables, lens
        k, v, qd, qp = (x[step] for x in self.staged)
        self.key.copy_(k)
        self.value.copy_(v)
        self.dec_q.copy_(qd)
        self.pre_q.copy_(qp)
        self.slots.copy_(torch.from_numpy(np.concatenate(slots)))
        self.dec_tables.copy_(torch.from_numpy(tables[:self.Bd]))
        self.dec_lens.copy_(torch.from_numpy(lens[:self.Bd]))
        self.pre_tables.copy_(torch.from_numpy(tables[self.Bd:]))
        self.pre_lens.copy_(torch.from_numpy(lens[self.Bd:]))

    def launch(self, stream=None) -> None:
        """The device side of a prepared step: pa_step, or the captured graph."""
        from paged_kv_cache_indirect_amd import pa_step, pa_step_graph_create, pa_step_graph_launch
        if not self.use_graph:
            pa_step(self.pool, self.desc, stream)
            return
        if self.graph is None:
            torch.cuda.synchronize()     # the buffer uploads above ran on torch's stream
            self.graph = pa_step_graph_create(self.pool, self.desc)
        pa_step_graph_launch(self.graph, stream)

    def close(self) -> None:
        from paged_kv_cache_indirect_amd import pa_step_graph_destroy
        torch.cuda.synchronize()
        if self.graph is not None:
            pa_step_graph_destroy(self.graph)
            self.graph = None
        if self.pool:
            pa_free_pool(self.pool)
            self.pool = None
