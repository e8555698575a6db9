"""Paged attention, written out from its definition, in fp64.  (Test infrastructure.)

Source: "vLLM的'内存分页'到底多神奇 — 用PagedAttention原理图解告别长文本推理OOM"
(xxqk.cn), §3 "从原理到实践", phase 2: the kernel walks a sequence's page
table, fetches each physical page's K and V, joins the pages along the token
axis into one logical K/V tensor, then runs ordinary attention
(scores = q·Kᵀ, softmax over tokens, weights·V). The pool layout
[num_blocks, block_size, num_heads, head_dim] is from "LLM推理优化：技术原理
解析总览" (dpshk.com), §3.3.

Readings where the pages are silent:
* scores carry a caller-supplied ``scale`` (the pages' sketch has none);
* grouped-query heads: q head h reads kv head h // (Hq/Hkv);
* ``seq_lens[b]`` counts the valid cache entries at call time (the new
  token included); slots past it in the last block are ignored, and table
  entries past ceil(L/bs) are never read;
* K and V are two pools with the same layout, indexed by the same block id;
* softmax is the exact two-pass form (max, then sum) in fp64;
* chunked prefill: query row i of a chunk of length n over a cache of length
  L sits at absolute position L - n + i and attends to tokens 0..L-n+i
  (none when that position is negative, i.e. the chunk is longer than the
  cache: zero output);
* an empty sequence (L = 0) yields a zero output and log-sum-exp -inf;
* an FP8 cache holds E4M3 codes; a K code c is read as value(c)·k_scale and
  a V code as value(c)·v_scale (``oracle.fp8``), exactly, before attention.
"""
from __future__ import annotations

import numpy as np

from .fp8 import decode_e4m3

__all__ = [
    "widen", "widen_kv", "gather_sequence", "attend", "paged_decode", "paged_prefill",
    "paged_prefill_masked", "partial_state", "merge_partials",
]


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> fp64. bf16 arrives as uint16 bit patterns: shifting
    them into the high half of an fp32 word gives the exact value."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def widen_kv(a: np.ndarray, kv_dtype: str, scale: float = 1.0) -> np.ndarray:
    """Stored cache elements -> fp64 values: fp32 / bf16 as ``widen``; FP8
    codes decoded from the E4M3 definition and multiplied by the pool scale
    (exact in fp64: a 4-bit by 24-bit significand product)."""
    if kv_dtype == "fp8":
        return decode_e4m3(a) * np.float64(np.float32(scale))
    return widen(a, kv_dtype)


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, L: int, block_size: int) -> np.ndarray:
    """Logical rows 0..L-1 of one sequence: [L, Hkv, D] (cache dtype kept).

    Walk the logical blocks in order, fetch each mapped physical block
    (shape [block_size, Hkv, D]), concatenate along tokens, cut to L.
    """
    nblk = -(-L // block_size)
    pages = [cache[int(table_row[i])] for i in range(nblk)]
    if not pages:
        return cache[:0].reshape((0,) + cache.shape[2:])
    return np.concatenate(pages, axis=0)[:L]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Exact softmax attention of one query vector over [L, D] keys/values.

    Returns (out [D], lse). Two passes: max of the scores, then the
    exponentials shifted by it; out = Σ w·V / Σ w, lse = m + log Σ w.
    """
    L = K.shape[0]
    if L == 0:
        return np.zeros(q.shape[-1], dtype=np.float64), -np.inf
    s = scale * (K @ q)
    m = s.max()
    w = np.exp(s - m)
    denom = w.sum()
    return (w @ V) / denom, m + np.log(denom)


def _gqa_group(Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return Hq // Hkv


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, seq_lens: np.ndarray, scale: float, dtype: str,
                 kv_dtype: str = "", k_scale: float = 1.0, v_scale: float = 1.0):
    """Decode attention for every (sequence, q head).

    q [B, Hq, D]; k_cache/v_cache [num_blocks, block_size, Hkv, D];
    block_tables int [B, max_blocks]; seq_lens int [B]. ``kv_dtype`` is the
    cache element type ("" = ``dtype``); FP8 caches use the pool scales.
    Returns (out [B, Hq, D] fp64, lse [B, Hq] fp64).
    """
    kvd = kv_dtype or dtype
    B, Hq, D = q.shape
    block_size, Hkv = k_cache.shape[1], k_cache.shape[2]
    G = _gqa_group(Hq, Hkv)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        K = widen_kv(gather_sequence(k_cache, block_tables[b], L, block_size), kvd, k_scale)
        V = widen_kv(gather_sequence(v_cache, block_tables[b], L, block_size), kvd, v_scale)
        qb = widen(q[b], dtype)
        for h in range(Hq):
            g = h // G
            out[b, h], lse[b, h] = attend(qb[h], K[:, g, :], V[:, g, :], scale)
    return out, lse


def paged_prefill(q: np.ndarray, cu_q_lens: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  block_tables: np.ndarray, seq_lens: np.ndarray, scale: float, dtype: str,
                  rows=None):
    """Causal chunked-prefill attention.

    q [T, Hq, D] holds the chunks of all sequences back to back;
    cu_q_lens [B+1] their offsets. Sequence b's chunk has n_b rows and its
    cache (chunk included) has L_b tokens. Row i attends to tokens
    0..L_b - n_b + i. ``rows`` optionally restricts the work to a list of
    (b, i) pairs (others stay zero). Returns (out [T, Hq, D], lse [T, Hq]).
    """
    T, Hq, D = q.shape
    block_size, Hkv = k_cache.shape[1], k_cache.shape[2]
    G = _gqa_group(Hq, Hkv)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    B = len(seq_lens)
    want = None if rows is None else {}
    if rows is not None:
        for b, i in rows:
            want.setdefault(int(b), []).append(int(i))
    for b in range(B):
        if want is not None and b not in want:
            continue
        L = int(seq_lens[b])
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        n = r1 - r0
        K = widen(gather_sequence(k_cache, block_tables[b], L, block_size), dtype)
        V = widen(gather_sequence(v_cache, block_tables[b], L, block_size), dtype)
        for i in (range(n) if want is None else want[b]):
            pos = L - n + i
            qi = widen(q[r0 + i], dtype)
            for h in range(Hq):
                g = h // G
                kv = max(pos + 1, 0)   # a row before the cache start sees no keys
                out[r0 + i, h], lse[r0 + i, h] = attend(qi[h], K[:kv, g, :], V[:kv, g, :], scale)
    return out, lse


def paged_prefill_masked(q: np.ndarray, cu_q_lens: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                         block_tables: np.ndarray, seq_lens: np.ndarray, scale: float, dtype: str):
    """The same causal chunked prefill as ``paged_prefill``, one matrix per
    (sequence, q head) instead of one vector per row, so that a whole
    512-row chunk over thousands of cached tokens is checked in seconds.

    For sequence b with n rows over L cached tokens: gather K_b, V_b through
    the table (as in decode), S = scale · Q_bh K_gᵀ ([n, L]), set S[i, t] to
    -inf where t > L - n + i (the causal mask over absolute positions), take
    the exact two-pass softmax of each row (row max, then exp and sum), and
    return weights · V_g. A row whose position is negative has every key
    masked: zero output, lse -inf. Returns (out [T, Hq, D], lse [T, Hq]).
    """
    T, Hq, D = q.shape
    block_size, Hkv = k_cache.shape[1], k_cache.shape[2]
    G = _gqa_group(Hq, Hkv)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        r0, r1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        K = widen(gather_sequence(k_cache, block_tables[b], L, block_size), dtype)
        V = widen(gather_sequence(v_cache, block_tables[b], L, block_size), dtype)
        Q = widen(q[r0:r1], dtype)                                   # [n, Hq, D]
        pos = (L - n) + np.arange(n)                                 # absolute position of each row
        allowed = np.arange(L)[None, :] <= pos[:, None]              # [n, L]
        seen = allowed.any(axis=1)                                   # rows with at least one key
        for h in range(Hq):
            g = h // G
            S = scale * (Q[:, h, :] @ K[:, g, :].T)                  # [n, L]
            S = np.where(allowed, S, -np.inf)
            m = np.where(seen, S.max(axis=1, initial=-np.inf), 0.0)
            W = np.exp(S - m[:, None])                               # masked entries give 0
            den = W.sum(axis=1)
            num = W @ V[:, g, :]
            ok = seen & (den > 0)
            out[r0:r1, h] = np.where(ok[:, None], num / np.where(ok, den, 1.0)[:, None], 0.0)
            lse[r0:r1, h] = np.where(ok, m + np.log(np.where(ok, den, 1.0)), -np.inf)
    return out, lse


def partial_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Unnormalised softmax state of one token range: (m, l, acc).

    m = max score, l = Σ exp(s - m), acc = Σ exp(s - m)·V. An empty range
    gives (-inf, 0, 0). Split-KV decode computes one such state per
    partition.
    """
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(V.shape[-1], dtype=np.float64)
    s = scale * (K @ q)
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ V


def merge_partials(states):
    """Log-sum-exp merge of partial states into (out, lse).

    M = max m_p; out = Σ e^(m_p - M) acc_p / Σ e^(m_p - M) l_p;
    lse = M + log Σ e^(m_p - M) l_p. Empty states (m = -inf) contribute 0.
    """
    ms = np.array([m for m, _, _ in states], dtype=np.float64)
    M = ms.max()
    if not np.isfinite(M):
        return np.zeros_like(states[0][2]), -np.inf
    num = np.zeros_like(states[0][2])
    den = 0.0
    for m, l, acc in states:
        if not np.isfinite(m):
            continue
        f = np.exp(m - M)
        num = num + f * acc
        den += f * l
    return num / den, M + np.log(den)
