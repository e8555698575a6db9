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

from . import (pa_alloc_pool, pa_block_tables, pa_decode, pa_decode_workspace_bytes, pa_free_pool,
               pa_pool_set_kv_scales, pa_prefill, pa_seq_append, pa_seq_fork, pa_seq_free, pa_write_kv)

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
