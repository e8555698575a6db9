"""KV append scatter (slot_mapping write).  (Test infrastructure.)

Source: "LLM推理优化：技术原理解析总览" (dpshk.com), §2.2 "域三": with paging,
a new token costs one page allocation and one page-table update instead of a
realloc-and-copy of the whole cache; "vLLM的'内存分页'到底多神奇" (xxqk.cn),
§3 phase 1: a token lands in the current page until it is full, and the next
token takes a fresh page.

A slot is a flat index into the pool viewed as [num_blocks * block_size,
Hkv, D]; slot s lives in physical block s // block_size at offset
s % block_size. Negative slots are padding and are skipped; so are slots past
the end of the pool.
"""
from __future__ import annotations

import numpy as np

__all__ = ["write_kv"]


def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray, value: np.ndarray,
             slot_mapping: np.ndarray) -> None:
    """In place: cache[slot // bs, slot % bs] = row, for every slot >= 0 (bit copy)."""
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    for t in range(len(slot_mapping)):
        s = int(slot_mapping[t])
        if s < 0 or s >= nb * bs:
            continue
        k_cache[s // bs, s % bs] = key[t]
        v_cache[s // bs, s % bs] = value[t]
