"""Seeded synthetic inputs for paged KV-cache attention.

This module is shared by the CPU oracle tests and the HIP path's tests and
benchmark. It draws random numbers and describes *what* a workload contains
(sequence lengths, the physical-block order of the pool, the logical K/V rows
of every sequence, the queries, and the stream of block-manager operations
that builds the cache). It performs none of the method's arithmetic: no
block-table lookup, slot computation, scatter, gather or attention happens
here. Each side (oracle, HIP path) does those itself.

Every random draw comes from NumPy's PCG64 seeded by a SeedSequence built
from ``[seed, tag, index]``, so any one sequence's K/V can be regenerated on
its own (the oracle can recompute sampled outputs of a full-size workload
without materialising the whole cache). Values are N(0, 1) drawn in fp32; for
bf16 workloads they are rounded to bf16 with round-to-nearest-even and kept
as their raw uint16 bit patterns.

Workload shapes follow the five configurations the paged-attention pages
motivate (vLLM PagedAttention explainer, xxqk.cn, "从原理到实践" §3; LLM
inference overview, dpshk.com, §3.3 for the [num_blocks, block_size,
num_heads, head_dim] pool layout and block_size 16):

* ``tiny``   - 4 seqs, lengths {7,16,33,50}, 2 q = 2 kv heads, D 64, bs 16, fp32,
               32-block pool in a seeded random order.
* ``gqa8b``  - 64 seqs, lengths U[512,4096], 32 q / 8 kv heads, D 128, bf16,
               bs 16, shuffled pool of ceil(1.1 x need) blocks.
* ``long``   - 8 seqs of 32768 tokens, 32/8 heads, D 128, bf16, bs 16,
               split-KV partitions of 512 tokens.
* ``prefix`` - 128 seqs sharing one 2048-token prefix (same physical blocks,
               refcount 128) plus unique suffixes U[0,1024], 32/8, D 128,
               bf16, bs 16.
* ``prefill``- 16 seqs, each a 512-token causal query chunk over existing
               paged context of length U[0,7680], 32/8, D 128, bf16, bs 32.

One more case exercises copy-on-write of a partly filled shared block (it is
a parity case, not a benchmark configuration):

* ``prefix_cow`` - 32 seqs forked from one 1000-token prefix (1000 = 62·16
               + 8: the last prefix block is half full) plus suffixes
               U[0,300], 32/8, D 128, bf16, bs 16.
* ``mixed`` - serving steps mixing decode and chunked prefill: 56 decode
               sequences U[512,4096] plus 8 prefill sequences with cached
               context U[0,4096] taking 256-token chunks, 8 steps, 32/8, D 128,
               bf16, bs 16 (seed 1007).
* ``prompt_cache`` - 48 requests sharing a 1000-token prompt (62 full
               blocks + 8 tokens) plus own tokens U[1,600], each appended with
               its token ids so that prefix caching finds the shared blocks;
               32/8, D 128, bf16, bs 16 (seed 1008).
* ``gqa8b_fp8`` - the ``gqa8b`` shape (seed 1006) with an FP8 (E4M3) cache:
               bf16 rows quantised with per-tensor scales k 0.0137, v 0.0129
               (N(0,1) values up to about 6 map inside ±448).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload", "make_decode", "make_prefix_share", "make_prefill", "make_mixed", "make_prompt_cache",
    "CONFIGS", "config", "round_to_bf16_bits", "draw_values", "mixed_step_queries", "ops_through",
]

# Tags that separate the independent random streams of one workload.
_TAG_LENS, _TAG_PERM, _TAG_KV, _TAG_Q, _TAG_PREFIX, _TAG_STEP, _TAG_TOKENS = 0, 1, 2, 3, 4, 5, 6


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Input generation only: used to produce bf16 test data from fp32 draws.
    Inputs are finite N(0,1) draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) values: float32 array for 'f32', uint16 bf16 bits for 'bf16'."""
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return v
    if dtype == "bf16":
        return round_to_bf16_bits(v)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass
class Workload:
    """A seeded synthetic paged-attention workload.

    ``ops`` is the block-manager operation stream that builds the cache:
    ``("append", seq, n)``, ``("tokens", seq, ids)`` (a token-aware append of
    len(ids) tokens), ``("fork", src, dst)``, ``("free", seq)``.
    After every ``append``, the ``n`` new logical rows
    ``kv_rows(seq, start, n)`` (positions start..start+n-1 of ``seq``) are to be
    written into the slots that append returned.
    """
    name: str
    kind: str                      # "decode" | "prefill"
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    dtype: str                     # "f32" | "bf16": q, out and the K/V rows handed to the scatter
    seed: int
    seq_lens: np.ndarray           # int32 [B], cache length at call time
    num_blocks: int
    free_order: np.ndarray         # int32 [num_blocks] permutation, popped first at index 0
    ops: List[tuple]
    scale: float
    q_lens: Optional[np.ndarray] = None     # prefill: int32 [B] query-chunk length
    partition_tokens: int = 512
    prefix_len: int = 0            # shared-prefix workloads
    kv_dtype: str = ""             # cache element type: "" = dtype, or "fp8" (E4M3 codes, bf16 rows in)
    k_scale: float = 1.0           # FP8 caches: per-tensor scales (code value * scale)
    v_scale: float = 1.0
    plan: Optional[dict] = None    # mixed decode + prefill steps (make_mixed)
    _cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict, repr=False)
    _prefix: Optional[Tuple[np.ndarray, np.ndarray]] = field(default=None, repr=False)

    # ---------------------------------------------------------------- sizes
    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.cache_dtype == "fp8" else self.elem_bytes

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.B else 0

    @property
    def max_blocks(self) -> int:
        """Block-table row width: enough logical blocks for the longest sequence."""
        return max(1, -(-self.max_seq_len // self.block_size))

    # ------------------------------------------------------------ K/V rows
    def _own_kv(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """The K/V rows a sequence owns (its full contents, or its suffix)."""
        if seq not in self._cache:
            n = int(self.seq_lens[seq]) - self.prefix_len
            rng = _rng(self.seed, _TAG_KV, seq)
            k = draw_values(rng, (n, self.Hkv, self.D), self.dtype)
            v = draw_values(rng, (n, self.Hkv, self.D), self.dtype)
            self._cache[seq] = (k, v)
        return self._cache[seq]

    def prefix_kv(self) -> Tuple[np.ndarray, np.ndarray]:
        if self._prefix is None:
            rng = _rng(self.seed, _TAG_PREFIX, 0)
            shape = (self.prefix_len, self.Hkv, self.D)
            self._prefix = (draw_values(rng, shape, self.dtype), draw_values(rng, shape, self.dtype))
        return self._prefix

    def kv_rows(self, seq: int, start: int, n: int) -> Tuple[np.ndarray, np.ndarray]:
        """Logical K/V rows [start, start+n) of ``seq``: arrays [n, Hkv, D]."""
        P = self.prefix_len
        if n == 0:
            e = np.empty((0, self.Hkv, self.D), dtype=np.float32 if self.dtype == "f32" else np.uint16)
            return e, e.copy()
        parts_k, parts_v = [], []
        if start < P:
            pk, pv = self.prefix_kv()
            e = min(P, start + n)
            parts_k.append(pk[start:e]); parts_v.append(pv[start:e])
        if start + n > P:
            ok, ov = self._own_kv(seq)
            s = max(start, P) - P
            e = start + n - P
            parts_k.append(ok[s:e]); parts_v.append(ov[s:e])
        if len(parts_k) == 1:
            return parts_k[0], parts_v[0]
        return np.concatenate(parts_k), np.concatenate(parts_v)

    def seq_kv(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """All logical K/V rows of ``seq`` (contiguous, [L, Hkv, D])."""
        return self.kv_rows(seq, 0, int(self.seq_lens[seq]))

    def drop_cached(self) -> None:
        self._cache.clear()
        self._prefix = None

    # --------------------------------------------------------------- queries
    @property
    def num_q_rows(self) -> int:
        return self.B if self.kind == "decode" else int(self.q_lens.sum())

    def queries(self) -> np.ndarray:
        """Decode: [B, Hq, D]; prefill: [sum(q_lens), Hq, D] (sequence-major)."""
        return draw_values(_rng(self.seed, _TAG_Q, 0), (self.num_q_rows, self.Hq, self.D), self.dtype)

    def decode_step_inputs(self, step: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Inputs of decode step ``step`` after the cache is built: the new
        token's K and V rows of every sequence ([B, Hkv, D] each) and the
        step's queries ([B, Hq, D])."""
        rng = _rng(self.seed, _TAG_STEP, step)
        k = draw_values(rng, (self.B, self.Hkv, self.D), self.dtype)
        v = draw_values(rng, (self.B, self.Hkv, self.D), self.dtype)
        q = draw_values(rng, (self.B, self.Hq, self.D), self.dtype)
        return k, v, q

    def cu_q_lens(self) -> np.ndarray:
        assert self.q_lens is not None
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    # ---------------------------------------------------------- byte counts
    def kv_bytes(self) -> int:
        """Logical K+V bytes one call reads: sum_b L_b * Hkv * D * 2 * elem."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * self.kv_elem_bytes

    def unique_kv_bytes(self) -> int:
        if not self.prefix_len:
            return self.kv_bytes()
        tok = int(self.seq_lens.astype(np.int64).sum()) - (self.B - 1) * self.prefix_len
        return tok * self.Hkv * self.D * 2 * self.kv_elem_bytes


def _pool(seed: int, need: int, factor: float, fixed: Optional[int]) -> Tuple[int, np.ndarray]:
    nb = fixed if fixed is not None else max(need, int(math.ceil(factor * need)))
    perm = _rng(seed, _TAG_PERM, 0).permutation(nb).astype(np.int32)
    return nb, perm


def make_decode(name: str, lens: Sequence[int], Hq: int, Hkv: int, D: int, block_size: int,
                dtype: str, seed: int, pool_factor: float = 1.1, num_blocks: Optional[int] = None,
                partition_tokens: int = 512, scale: Optional[float] = None, kv_dtype: str = "",
                k_scale: float = 1.0, v_scale: float = 1.0) -> Workload:
    """Decode workload: one query token per sequence over a paged cache of ``lens``.
    ``kv_dtype="fp8"`` stores the bf16 rows as E4M3 codes with the given scales."""
    lens = np.asarray(lens, dtype=np.int32)
    need = int(sum(-(-int(L) // block_size) for L in lens))
    nb, perm = _pool(seed, need, pool_factor, num_blocks)
    ops = [("append", b, int(L)) for b, L in enumerate(lens)]
    return Workload(name=name, kind="decode", B=len(lens), Hq=Hq, Hkv=Hkv, D=D,
                    block_size=block_size, dtype=dtype, seed=seed, seq_lens=lens,
                    num_blocks=nb, free_order=perm, ops=ops,
                    scale=scale if scale is not None else 1.0 / math.sqrt(D),
                    partition_tokens=partition_tokens, kv_dtype=kv_dtype, k_scale=k_scale,
                    v_scale=v_scale)


def make_prefix_share(name: str, B: int, prefix_len: int, suffix_lens: Sequence[int], Hq: int,
                      Hkv: int, D: int, block_size: int, dtype: str, seed: int,
                      pool_factor: float = 1.1, partition_tokens: int = 512) -> Workload:
    """B sequences whose first ``prefix_len`` tokens live in the same physical blocks.

    Sequence 0 appends the prefix; sequences 1..B-1 fork it (every prefix
    block ends with refcount B); then every sequence appends its own suffix,
    in order 0..B-1. When ``prefix_len`` is not a multiple of ``block_size``
    the last prefix block is only partly filled, so each suffix append that
    still finds it shared takes a private copy of it first (copy-on-write).
    """
    suffix_lens = np.asarray(suffix_lens, dtype=np.int32)
    lens = (suffix_lens + prefix_len).astype(np.int32)
    # Upper bound on blocks: the prefix, plus for each non-empty suffix every
    # block past the prefix's full blocks (its copy of a partial block included).
    full = prefix_len // block_size
    need = -(-prefix_len // block_size) + int(sum(-(-(prefix_len + int(s)) // block_size) - full
                                                  for s in suffix_lens if s > 0))
    nb, perm = _pool(seed, need, pool_factor, None)
    ops: List[tuple] = [("append", 0, prefix_len)]
    ops += [("fork", 0, b) for b in range(1, B)]
    ops += [("append", b, int(s)) for b, s in enumerate(suffix_lens)]
    return Workload(name=name, kind="decode", B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                    dtype=dtype, seed=seed, seq_lens=lens, num_blocks=nb, free_order=perm,
                    ops=ops, scale=1.0 / math.sqrt(D), prefix_len=prefix_len,
                    partition_tokens=partition_tokens)


def make_prompt_cache(name: str, B: int, prompt_len: int, suffix_lens: Sequence[int], Hq: int, Hkv: int,
                      D: int, block_size: int, dtype: str, seed: int, vocab: int = 32000,
                      pool_factor: float = 1.1) -> Workload:
    """B requests that start with the same ``prompt_len``-token prompt, each
    appended in one token-aware call (op ``("tokens", seq, ids)``) so that the
    block manager finds the prompt's full blocks by their token ids instead of
    being told to fork. The K/V rows of prompt positions are the shared
    prefix rows (equal ids at equal positions give equal K/V)."""
    suffix_lens = np.asarray(suffix_lens, dtype=np.int32)
    lens = (suffix_lens + prompt_len).astype(np.int32)
    rng = _rng(seed, _TAG_TOKENS, 0)
    prompt = rng.integers(0, vocab, prompt_len).astype(np.int32)
    ops = []
    for b in range(B):
        own = _rng(seed, _TAG_TOKENS, b + 1).integers(0, vocab, int(suffix_lens[b])).astype(np.int32)
        ops.append(("tokens", b, np.concatenate([prompt, own])))
    full = prompt_len // block_size
    need = full + int(sum(-(-int(L) // block_size) - full for L in lens))
    nb, perm = _pool(seed, need, pool_factor, None)
    return Workload(name=name, kind="decode", B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                    dtype=dtype, seed=seed, seq_lens=lens, num_blocks=nb, free_order=perm, ops=ops,
                    scale=1.0 / math.sqrt(D), prefix_len=prompt_len)


def make_prefill(name: str, ctx_lens: Sequence[int], q_lens: Sequence[int], Hq: int, Hkv: int,
                 D: int, block_size: int, dtype: str, seed: int, pool_factor: float = 1.1) -> Workload:
    """Chunked prefill: each sequence has ``ctx`` cached tokens, then a ``q_len`` chunk.

    The chunk's own K/V rows are appended to the cache before attention, so
    the cache length at call time is ``ctx + q_len``.
    """
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    ql = np.asarray(q_lens, dtype=np.int32)
    lens = (ctx + ql).astype(np.int32)
    need = int(sum(-(-int(L) // block_size) for L in lens))
    nb, perm = _pool(seed, need, pool_factor, None)
    ops = [("append", b, int(L)) for b, L in enumerate(lens)]
    return Workload(name=name, kind="prefill", B=len(lens), Hq=Hq, Hkv=Hkv, D=D,
                    block_size=block_size, dtype=dtype, seed=seed, seq_lens=lens,
                    num_blocks=nb, free_order=perm, ops=ops, scale=1.0 / math.sqrt(D),
                    q_lens=ql)


def make_mixed(name: str, dec_lens: Sequence[int], pre_ctx: Sequence[int], chunk: int, steps: int, Hq: int,
               Hkv: int, D: int, block_size: int, dtype: str, seed: int, pool_factor: float = 1.1) -> Workload:
    """Serving steps that mix decode and chunked prefill in one batch.

    Sequences 0..Bd-1 decode: they start with ``dec_lens`` cached tokens and
    gain one token per step. Sequences Bd..Bd+Bp-1 prefill: they start with
    ``pre_ctx`` cached tokens and gain a ``chunk``-token chunk per step. Step
    s appends (decode sequences first, in order, then prefill sequences), then
    attends: each decode sequence with one query, each chunk with its rows.
    ``ops`` holds the initial appends followed by every step's appends;
    ``seq_lens`` are the lengths after the last step. ``plan`` records the
    split; ``ops_through(s)`` gives the ops that build the cache of step s.
    """
    dec = np.asarray(dec_lens, dtype=np.int32)
    pre = np.asarray(pre_ctx, dtype=np.int32)
    Bd, Bp = len(dec), len(pre)
    final = np.concatenate([dec + steps, pre + steps * chunk]).astype(np.int32)
    need = int(sum(-(-int(L) // block_size) for L in final))
    nb, perm = _pool(seed, need, pool_factor, None)
    init = [("append", b, int(L)) for b, L in enumerate(np.concatenate([dec, pre]))]
    per_step = [("append", b, 1) for b in range(Bd)] + [("append", Bd + i, chunk) for i in range(Bp)]
    ops = init + per_step * steps
    plan = {"Bd": Bd, "Bp": Bp, "chunk": chunk, "steps": steps, "n_init": len(init), "n_step": len(per_step)}
    return Workload(name=name, kind="mixed", B=Bd + Bp, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                    dtype=dtype, seed=seed, seq_lens=final, num_blocks=nb, free_order=perm, ops=ops,
                    scale=1.0 / math.sqrt(D), q_lens=np.full(Bp, chunk, dtype=np.int32), plan=plan)


def mixed_step_queries(wl: Workload, step: int) -> Tuple[np.ndarray, np.ndarray]:
    """Queries of mixed step ``step``: decode [Bd, Hq, D] and the chunks' rows
    [Bp * chunk, Hq, D] (sequence by sequence)."""
    p = wl.plan
    rng = _rng(wl.seed, _TAG_STEP, step)
    qd = draw_values(rng, (p["Bd"], wl.Hq, wl.D), wl.dtype)
    qp = draw_values(rng, (p["Bp"] * p["chunk"], wl.Hq, wl.D), wl.dtype)
    return qd, qp


def ops_through(wl: Workload, step: int) -> List[tuple]:
    """The ops of a mixed workload up to and including step ``step``'s appends."""
    p = wl.plan
    return wl.ops[:p["n_init"] + (step + 1) * p["n_step"]]


def _uniform_ints(seed: int, lo: int, hi: int, n: int) -> np.ndarray:
    """n integers uniform on [lo, hi] inclusive."""
    return _rng(seed, _TAG_LENS, 0).integers(lo, hi + 1, size=n).astype(np.int32)


def config(name: str) -> Workload:
    """The five named workloads at full size."""
    if name == "tiny":
        return make_decode("tiny", [7, 16, 33, 50], Hq=2, Hkv=2, D=64, block_size=16,
                           dtype="f32", seed=1000, num_blocks=32)
    if name == "gqa8b":
        s = 1001
        return make_decode("gqa8b", _uniform_ints(s, 512, 4096, 64), Hq=32, Hkv=8, D=128,
                           block_size=16, dtype="bf16", seed=s)
    if name == "long":
        return make_decode("long", [32768] * 8, Hq=32, Hkv=8, D=128, block_size=16,
                           dtype="bf16", seed=1002)
    if name == "prefix":
        s = 1003
        return make_prefix_share("prefix", 128, 2048, _uniform_ints(s, 0, 1024, 128), Hq=32,
                                 Hkv=8, D=128, block_size=16, dtype="bf16", seed=s)
    if name == "gqa8b_fp8":
        s = 1006
        return make_decode("gqa8b_fp8", _uniform_ints(s, 512, 4096, 64), Hq=32, Hkv=8, D=128,
                           block_size=16, dtype="bf16", seed=s, kv_dtype="fp8", k_scale=0.0137,
                           v_scale=0.0129)
    if name == "mixed":
        s = 1007
        return make_mixed("mixed", _uniform_ints(s, 512, 4096, 56), _rng(s, _TAG_LENS, 1).integers(
                          0, 4097, 8).astype(np.int32), 256, 8, Hq=32, Hkv=8, D=128, block_size=16,
                          dtype="bf16", seed=s)
    if name == "prompt_cache":
        s = 1008
        return make_prompt_cache("prompt_cache", 48, 1000, _uniform_ints(s, 1, 600, 48), Hq=32, Hkv=8, D=128,
                                 block_size=16, dtype="bf16", seed=s)
    if name == "prefix_cow":
        s = 1005
        return make_prefix_share("prefix_cow", 32, 1000, _uniform_ints(s, 0, 300, 32), Hq=32,
                                 Hkv=8, D=128, block_size=16, dtype="bf16", seed=s)
    if name == "prefill":
        s = 1004
        return make_prefill("prefill", _uniform_ints(s, 0, 7680, 16), [512] * 16, Hq=32, Hkv=8,
                            D=128, block_size=32, dtype="bf16", seed=s)
    raise KeyError(name)


CONFIGS = ("tiny", "gqa8b", "long", "prefix", "prefill")
