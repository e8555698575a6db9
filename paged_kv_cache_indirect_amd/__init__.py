"""paged_kv_cache_indirect_amd — paged KV-cache attention on AMD MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (the C ABI declared in
``include/pa.h``). Each ``pa_*`` function here has the same name as the C
entry point and only marshals arguments: torch tensors become device
pointers, numpy arrays become host pointers, the current torch stream becomes
the hipStream_t. Every step of the computation runs in the library's HIP
kernels and host block manager. If the library is not built, importing this
package raises: there is no fallback path.

Build it with ``python paged_kv_cache_indirect_amd/build.py`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import itertools
import os
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "PaError", "PA_OK", "PA_ERR_INVALID", "PA_ERR_NO_BLOCKS", "PA_ERR_UNSUPPORTED", "PA_ERR_HIP",
    "PA_ERR_UNKNOWN_SEQ", "PA_F32", "PA_BF16", "PA_FP8_E4M3", "LIB_PATH", "lib",
    "pa_alloc_pool", "pa_free_pool", "pa_seq_append", "pa_seq_append_batch", "pa_seq_fork", "pa_seq_free",
    "pa_block_tables", "pa_pool_stats", "pa_pool_pending_copies", "pa_pool_set_kv_scales", "pa_write_kv",
    "pa_decode_workspace_bytes", "pa_decode", "pa_prefill", "pa_last_error", "StepDesc", "pa_step",
    "pa_step_graph_create", "pa_step_graph_launch", "pa_step_graph_destroy", "pa_seq_append_tokens",
    "pa_pool_prefix_stats", "pa_tier_block_size", "pa_decode_partition_tokens", "pa_append_decode",
    "pa_append_decode_args", "pa_decode_partition_tokens_for_lengths", "pa_pool_layout", "pa_set_debug_checks",
    "pa_decode_static", "PA_DECODE_STATIC_SCRATCH_BYTES",
]

PA_OK, PA_ERR_INVALID, PA_ERR_NO_BLOCKS, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_UNKNOWN_SEQ = 0, -1, -2, -3, -4, -5
PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_DECODE_STATIC_SCRATCH_BYTES = 32 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_cache_indirect_amd/build.py`")

# One HIP runtime per process: torch ships its own libamdhip64 (soname
# libamdhip64.so.7, the same as the system one). Loading torch first makes the
# library's libamdhip64.so.7 dependency bind to that already-loaded runtime, so
# torch's device pointers and streams are valid in the library.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)


class _Layout(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class _Stats(ctypes.Structure):
    _fields_ = [("free_blocks", ctypes.c_int32), ("used_blocks", ctypes.c_int32),
                ("shared_blocks", ctypes.c_int32), ("pending_copies", ctypes.c_int32),
                ("filled_slots", ctypes.c_int64), ("allocated_slots", ctypes.c_int64)]


class _StepDesc(ctypes.Structure):
    _fields_ = [("key", ctypes.c_void_p), ("value", ctypes.c_void_p), ("slot_mapping", ctypes.c_void_p),
                ("num_new_tokens", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("scale", ctypes.c_float),
                ("max_blocks", ctypes.c_int32),
                ("dec_out", ctypes.c_void_p), ("dec_q", ctypes.c_void_p), ("dec_block_tables", ctypes.c_void_p),
                ("dec_seq_lens", ctypes.c_void_p), ("dec_batch", ctypes.c_int32),
                ("dec_max_seq_len", ctypes.c_int32), ("partition_tokens", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("pre_out", ctypes.c_void_p), ("pre_q", ctypes.c_void_p), ("pre_cu_q_lens", ctypes.c_void_p),
                ("pre_block_tables", ctypes.c_void_p), ("pre_seq_lens", ctypes.c_void_p),
                ("pre_batch", ctypes.c_int32), ("pre_max_q_len", ctypes.c_int32)]


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "pa_alloc_pool": (_i32, [ctypes.POINTER(_Layout), _vp, _vp, _vp, ctypes.POINTER(_vp)]),
    "pa_free_pool": (None, [_vp]),
    "pa_seq_append_tokens": (_i32, [_vp, _i64, _vp, _i32, _vp, _vp]),
    "pa_pool_prefix_stats": (_i32, [_vp, _vp]),
    "pa_tier_block_size": (_i32, [_i64]),
    "pa_step": (_i32, [_vp, ctypes.POINTER(_StepDesc), _vp]),
    "pa_step_graph_create": (_i32, [_vp, ctypes.POINTER(_StepDesc), ctypes.POINTER(_vp)]),
    "pa_step_graph_launch": (_i32, [_vp, _vp]),
    "pa_step_graph_destroy": (None, [_vp]),
    "pa_pool_set_kv_scales": (_i32, [_vp, ctypes.c_float, ctypes.c_float]),
    "pa_seq_append": (_i32, [_vp, _i64, _i32, _vp]),
    "pa_seq_append_batch": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "pa_seq_fork": (_i32, [_vp, _i64, _i64]),
    "pa_seq_free": (_i32, [_vp, _i64]),
    "pa_block_tables": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "pa_pool_stats": (_i32, [_vp, ctypes.POINTER(_Stats)]),
    "pa_pool_layout": (_i32, [_vp, ctypes.POINTER(_Layout)]),
    "pa_pool_pending_copies": (_i32, [_vp, _vp, _vp, _i32, _vp]),
    "pa_write_kv": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_partition_tokens": (_i32, [_vp, _i32, _i32]),
    "pa_decode_partition_tokens_for_lengths": (_i32, [_vp, _vp, _i32, _i32]),
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _vp]),
    "pa_append_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _i32, _vp,
                                _sz, _vp]),
    "pa_append_decode_args": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _i32,
                                     _vp, _sz, _vp]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_set_debug_checks": (_i32, [_i32]),
    "pa_decode_static": (_i32, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _f32, _i32, _i32, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.pa_last_error().decode(errors="replace")
        super().__init__(f"{where} failed with status {status}: {msg}")


def _check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PaError(status, where)


def _dptr(t) -> int:
    """Device pointer of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return PA_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------- argument checks
# The library sizes every device access from the pool's layout, so a tensor
# whose shape or element type disagrees with it would be read or written out
# of bounds on the device. Each device call checks its tensors here first
# (shape and dtype, then that they live on a GPU) and raises ValueError.

def pa_pool_layout(pool: int) -> dict:
    """The pool's geometry: num_blocks, block_size, num_kv_heads, head_dim, dtype."""
    lay = _Layout()
    _check(lib.pa_pool_layout(pool, ctypes.byref(lay)), "pa_pool_layout")
    return {"num_blocks": lay.num_blocks, "block_size": lay.block_size, "num_kv_heads": lay.num_kv_heads,
            "head_dim": lay.head_dim, "dtype": lay.dtype}


def _compute_dtype(layout: dict):
    """Element type of q, out and K/V rows for a pool: the pool's own, bf16
    for an FP8 pool."""
    import torch
    return {PA_F32: torch.float32, PA_BF16: torch.bfloat16, PA_FP8_E4M3: torch.bfloat16}[layout["dtype"]]


def _want(t, name: str, shape, dtype) -> None:
    """``t`` must be a contiguous tensor of ``dtype`` on a GPU whose shape is
    ``shape`` (entries None are free)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != len(shape) or any(w is not None and int(g) != w for g, w in zip(t.shape, shape)):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple('*' if w is None else w for w in shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _want_gpu(**named) -> None:
    """Every given tensor (None skipped) lives on a GPU. Called after the
    shape and dtype checks of a call."""
    for name, t in named.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _want_rows(layout: dict, name: str, t, rows=None) -> None:
    """q / out ([rows, Hq, D]) against the pool: head_dim, element type and
    a q-head count that is a multiple of the kv heads."""
    if t is None:
        raise ValueError(f"{name} is required")
    _want(t, name, (rows, None, layout["head_dim"]), _compute_dtype(layout))
    if int(t.shape[1]) % layout["num_kv_heads"]:
        raise ValueError(f"{name}: {int(t.shape[1])} q heads is not a multiple of {layout['num_kv_heads']} kv heads")


def _want_kv_rows(layout: dict, name: str, t, rows=None) -> None:
    """New K/V rows [rows, Hkv, D] for a scatter into the pool."""
    _want(t, name, (rows, layout["num_kv_heads"], layout["head_dim"]), _compute_dtype(layout))


def _want_workspace(t, name: str = "workspace") -> None:
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _want_host(a, name: str, n: int, dtype) -> np.ndarray:
    """A host array of at least n entries, converted to ``dtype``."""
    import torch
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError(f"{name} must be a host array")
        a = a.numpy()
    arr = np.ascontiguousarray(a, dtype=dtype).reshape(-1)
    if arr.size < n:
        raise ValueError(f"{name} needs {n} entries, got {arr.size}")
    return arr


# ------------------------------------------------------------------- pools
# Pools this binding created, by handle: a generation number that changes
# whenever a handle is reused for a new pool, so a step description checked
# against one pool is checked again against the next pool at that handle.
_pool_gen = {}
_pool_gen_next = itertools.count(1)


def pa_alloc_pool(k_cache, v_cache, free_order: Optional[Sequence[int]] = None) -> int:
    """Create a pool over k_cache/v_cache (torch device tensors [nb, bs, Hkv, D]).
    Returns the opaque handle (an int)."""
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.dim() != 4 or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must be matching [num_blocks, block_size, Hkv, D] tensors")
    if not (k_cache.is_cuda and v_cache.is_cuda and k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("k_cache and v_cache must be contiguous GPU tensors")
    nb, bs, hkv, d = (int(x) for x in k_cache.shape)
    layout = _Layout(nb, bs, hkv, d, _dtype_code(k_cache))
    order = None
    if free_order is not None:
        order = np.ascontiguousarray(free_order, dtype=np.int32)
        if order.shape != (nb,):
            raise ValueError("free_order must have num_blocks entries")
    handle = _vp()
    _check(lib.pa_alloc_pool(ctypes.byref(layout), _dptr(k_cache), _dptr(v_cache),
                             None if order is None else order.ctypes.data, ctypes.byref(handle)),
           "pa_alloc_pool")
    _pool_gen[handle.value] = next(_pool_gen_next)
    return handle.value


def pa_free_pool(pool: int) -> None:
    _pool_gen.pop(pool, None)
    lib.pa_free_pool(pool)


def pa_seq_append(pool: int, seq_id: int, n_tokens: int) -> np.ndarray:
    """Returns the new tokens' flat slots (host int64 array)."""
    slots = np.empty(max(n_tokens, 0), dtype=np.int64)
    _check(lib.pa_seq_append(pool, seq_id, n_tokens, slots.ctypes.data if n_tokens > 0 else None),
           "pa_seq_append")
    return slots


def pa_seq_append_batch(pool: int, seq_ids, n_tokens: int, slots_out: Optional[np.ndarray] = None) -> np.ndarray:
    """Grow every sequence in ``seq_ids`` by ``n_tokens`` (all-or-nothing).
    Returns host int64 slots [n, n_tokens]; ``slots_out`` (a C-contiguous
    int64 array of that shape) is filled and returned when given."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    n = len(ids)
    if slots_out is None:
        slots_out = np.empty((n, max(n_tokens, 0)), dtype=np.int64)
    elif slots_out.dtype != np.int64 or not slots_out.flags.c_contiguous or slots_out.size < n * max(n_tokens, 0):
        raise ValueError("slots_out must be a C-contiguous int64 array of n * n_tokens entries")
    _check(lib.pa_seq_append_batch(pool, ids.ctypes.data, n, n_tokens,
                                   slots_out.ctypes.data if n_tokens > 0 else None),
           "pa_seq_append_batch")
    return slots_out


def pa_seq_fork(pool: int, src_seq_id: int, dst_seq_id: int) -> None:
    _check(lib.pa_seq_fork(pool, src_seq_id, dst_seq_id), "pa_seq_fork")


def pa_seq_free(pool: int, seq_id: int) -> None:
    _check(lib.pa_seq_free(pool, seq_id), "pa_seq_free")


def pa_block_tables(pool: int, seq_ids: Sequence[int], max_blocks: int, tables_out: Optional[np.ndarray] = None,
                    lens_out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Returns (tables int32 [n, max_blocks] padded -1, seq_lens int32 [n]) on the host.
    ``tables_out`` / ``lens_out`` (C-contiguous int32 of those sizes) are
    filled in place when given."""
    ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
    n = len(ids)
    tables = np.empty((n, max_blocks), dtype=np.int32) if tables_out is None else tables_out
    lens = np.empty(n, dtype=np.int32) if lens_out is None else lens_out
    for a, size in ((tables, n * max_blocks), (lens, n)):
        if a.dtype != np.int32 or not a.flags.c_contiguous or a.size < size:
            raise ValueError("tables_out / lens_out must be C-contiguous int32 arrays large enough")
    _check(lib.pa_block_tables(pool, ids.ctypes.data, n, max_blocks, tables.ctypes.data, lens.ctypes.data),
           "pa_block_tables")
    return tables, lens


def pa_pool_stats(pool: int) -> dict:
    s = _Stats()
    _check(lib.pa_pool_stats(pool, ctypes.byref(s)), "pa_pool_stats")
    return {"free_blocks": s.free_blocks, "used_blocks": s.used_blocks,
            "shared_blocks": s.shared_blocks, "filled_slots": s.filled_slots,
            "allocated_slots": s.allocated_slots, "pending_copies": s.pending_copies}


def pa_pool_pending_copies(pool: int) -> list:
    """Pending copy-on-write block copies [(src, dst), ...] in run order."""
    n = ctypes.c_int32()
    cap = pa_pool_stats(pool)["pending_copies"]
    src = np.empty(max(cap, 1), dtype=np.int32)
    dst = np.empty(max(cap, 1), dtype=np.int32)
    _check(lib.pa_pool_pending_copies(pool, src.ctypes.data, dst.ctypes.data, cap, ctypes.byref(n)),
           "pa_pool_pending_copies")
    return list(zip(src[:n.value].tolist(), dst[:n.value].tolist()))


def pa_last_error() -> str:
    return lib.pa_last_error().decode(errors="replace")


def pa_set_debug_checks(enable: bool) -> bool:
    """Turn the library's host-side checks of slots and block tables on or
    off (process-wide); returns the previous setting."""
    return bool(lib.pa_set_debug_checks(1 if enable else 0))


# ------------------------------------------------------------ device ops
def pa_pool_set_kv_scales(pool: int, k_scale: float, v_scale: float) -> None:
    """Per-tensor scales of an FP8 pool (a code c stands for value(c) * scale)."""
    _check(lib.pa_pool_set_kv_scales(pool, float(k_scale), float(v_scale)), "pa_pool_set_kv_scales")


def pa_write_kv(pool: int, key, value, slot_mapping, stream=None) -> None:
    """key/value: device [T, Hkv, D]; slot_mapping: device int64 [T]."""
    import torch
    lay = pa_pool_layout(pool)
    _want(slot_mapping, "slot_mapping", (None,), torch.int64)
    T = int(slot_mapping.shape[0])
    _want_kv_rows(lay, "key", key, T)
    _want_kv_rows(lay, "value", value, T)
    _want_gpu(key=key, value=value, slot_mapping=slot_mapping)
    _check(lib.pa_write_kv(pool, _dptr(key), _dptr(value), _dptr(slot_mapping), T, _stream(stream)),
           "pa_write_kv")


def pa_decode_workspace_bytes(B: int, num_q_heads: int, head_dim: int, max_seq_len: int,
                              partition_tokens: int = 0) -> int:
    return int(lib.pa_decode_workspace_bytes(B, num_q_heads, head_dim, max_seq_len, partition_tokens))


def pa_decode_partition_tokens(pool: int, B: int, max_seq_len: int) -> int:
    """The KV partition pa_decode uses for partition_tokens=0 on this pool."""
    return int(lib.pa_decode_partition_tokens(pool, B, max_seq_len))


def pa_decode_partition_tokens_for_lengths(pool: int, seq_lens, max_seq_len: int) -> int:
    """The partition pa_append_decode_args picks for partition_tokens = 0
    from the host lengths ``seq_lens`` (int32 [B])."""
    ln = np.ascontiguousarray(seq_lens, dtype=np.int32).reshape(-1)
    return int(lib.pa_decode_partition_tokens_for_lengths(pool, ln.ctypes.data if ln.size else None, int(ln.size),
                                                          int(max_seq_len)))


def _check_decode_args(pool, out, q, block_tables, seq_lens=None, workspace=None) -> dict:
    """q/out [B, Hq, D] of the pool's compute type, block_tables int32
    [B, max_blocks], seq_lens int32 [B] (None: lengths on the host)."""
    import torch
    lay = pa_pool_layout(pool)
    _want_rows(lay, "q", q)
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _want(out, "out", (B, Hq, lay["head_dim"]), q.dtype)
    _want(block_tables, "block_tables", (B, None), torch.int32)
    if seq_lens is not None:
        _want(seq_lens, "seq_lens", (B,), torch.int32)
    _want_workspace(workspace)
    _want_gpu(out=out, q=q, block_tables=block_tables, seq_lens=seq_lens, workspace=workspace)
    return lay


def pa_decode(pool: int, out, q, block_tables, seq_lens, scale: float, max_seq_len: int,
              partition_tokens: int = 0, workspace=None, stream=None) -> None:
    """out/q: device [B, Hq, D]; block_tables: device int32 [B, max_blocks];
    seq_lens: device int32 [B]. ``workspace`` (device uint8 tensor) is
    allocated here with torch when not given and needed."""
    _check_decode_args(pool, out, q, block_tables, seq_lens, workspace)
    B, Hq, D = (int(x) for x in q.shape)
    need = pa_decode_workspace_bytes(B, Hq, D, max_seq_len, partition_tokens)
    if need and workspace is None:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pa_decode(pool, _dptr(out), _dptr(q), _dptr(block_tables), int(block_tables.shape[1]),
                         _dptr(seq_lens), B, Hq, float(scale), int(max_seq_len), int(partition_tokens),
                         _dptr(workspace), ws_bytes, _stream(stream)),
           "pa_decode")


def pa_decode_static(pool: int, out, q, block_tables, seq_lens, scale: float, max_seq_len: int,
                     partition_tokens: int = 0, stream=None) -> None:
    """pa_decode with the partial states in the library's static device
    scratch: no workspace argument, and nothing is allocated (here or in the
    library). Calls that overlap on one GPU share that scratch and race."""
    _check_decode_args(pool, out, q, block_tables, seq_lens)
    B, Hq, _ = (int(x) for x in q.shape)
    _check(lib.pa_decode_static(pool, _dptr(out), _dptr(q), _dptr(block_tables), int(block_tables.shape[1]),
                                _dptr(seq_lens), B, Hq, float(scale), int(max_seq_len), int(partition_tokens),
                                _stream(stream)),
           "pa_decode_static")


def pa_append_decode(pool: int, out, q, key, value, slot_mapping, block_tables, seq_lens, scale: float,
                     max_seq_len: int, partition_tokens: int = 0, workspace=None, stream=None) -> None:
    """pa_write_kv of one new row per sequence, then pa_decode, in one launch.
    key/value: device [B, Hkv, D]; slot_mapping: device int64 [B] (slot of
    sequence b's newest token, or < 0); block_tables: device int32
    [B, max_blocks], whose entry for each new token's block is filled in."""
    import torch
    lay = _check_decode_args(pool, out, q, block_tables, seq_lens, workspace)
    B, Hq, D = (int(x) for x in q.shape)
    _want_kv_rows(lay, "key", key, B)
    _want_kv_rows(lay, "value", value, B)
    _want(slot_mapping, "slot_mapping", (B,), torch.int64)
    _want_gpu(key=key, value=value, slot_mapping=slot_mapping)
    need = pa_decode_workspace_bytes(B, Hq, D, max_seq_len, partition_tokens)
    if need and workspace is None:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pa_append_decode(pool, _dptr(out), _dptr(q), _dptr(key), _dptr(value), _dptr(slot_mapping),
                                _dptr(block_tables), int(block_tables.shape[1]), _dptr(seq_lens), B, Hq,
                                float(scale), int(max_seq_len), int(partition_tokens), _dptr(workspace), ws_bytes,
                                _stream(stream)),
           "pa_append_decode")


def pa_append_decode_args(pool: int, out, q, key, value, slots: np.ndarray, block_tables, seq_lens: np.ndarray,
                          scale: float, max_seq_len: int, partition_tokens: int = 0, workspace=None,
                          stream=None) -> None:
    """pa_append_decode with the slots (int64 [B]) and lengths (int32 [B])
    given as host arrays, passed in the launch arguments (B <= 128)."""
    lay = _check_decode_args(pool, out, q, block_tables, None, workspace)
    B, Hq, D = (int(x) for x in q.shape)
    _want_kv_rows(lay, "key", key, B)
    _want_kv_rows(lay, "value", value, B)
    sl = _want_host(slots, "slots", B, np.int64)
    ln = _want_host(seq_lens, "seq_lens", B, np.int32)
    _want_gpu(key=key, value=value)
    need = pa_decode_workspace_bytes(B, Hq, D, max_seq_len, partition_tokens)
    if need and workspace is None:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.pa_append_decode_args(pool, _dptr(out), _dptr(q), _dptr(key), _dptr(value), sl.ctypes.data,
                                     _dptr(block_tables), int(block_tables.shape[1]), ln.ctypes.data, B, Hq,
                                     float(scale), int(max_seq_len), int(partition_tokens), _dptr(workspace),
                                     ws_bytes, _stream(stream)),
           "pa_append_decode_args")


def pa_prefill(pool: int, out, q, cu_q_lens, block_tables, seq_lens, scale: float, max_q_len: int,
               stream=None) -> None:
    """out/q: device [T, Hq, D] bf16; cu_q_lens: device int32 [B+1];
    block_tables: device int32 [B, max_blocks]; seq_lens: device int32 [B].
    The rows cu_q_lens names (its last entry) must fit in q and out: that
    value lives on the device and is not checked here."""
    import torch
    lay = pa_pool_layout(pool)
    _want_rows(lay, "q", q)
    T, Hq = int(q.shape[0]), int(q.shape[1])
    _want(out, "out", (T, Hq, lay["head_dim"]), q.dtype)
    _want(seq_lens, "seq_lens", (None,), torch.int32)
    B = int(seq_lens.shape[0])
    _want(cu_q_lens, "cu_q_lens", (B + 1,), torch.int32)
    _want(block_tables, "block_tables", (B, None), torch.int32)
    _want_gpu(out=out, q=q, cu_q_lens=cu_q_lens, block_tables=block_tables, seq_lens=seq_lens)
    _check(lib.pa_prefill(pool, _dptr(out), _dptr(q), _dptr(cu_q_lens), _dptr(block_tables),
                          int(block_tables.shape[1]), _dptr(seq_lens), B, Hq, int(max_q_len),
                          float(scale), _stream(stream)),
           "pa_prefill")


class StepDesc:
    """One mixed step's buffers (torch device tensors, or None for a part
    that is skipped), marshalled into the C struct ``pa_step_desc``.

    key/value [T, Hkv, D] and slot_mapping int64 [T] feed the scatter;
    dec_out/dec_q [Bd, Hq, D], dec_block_tables int32 [Bd, max_blocks] and
    dec_seq_lens int32 [Bd] the decode; pre_out/pre_q [Tp, Hq, D],
    pre_cu_q_lens int32 [Bp + 1], pre_block_tables int32 [Bp, max_blocks] and
    pre_seq_lens int32 [Bp] the prefill. The tensors are kept referenced
    here, so a graph captured from this description keeps valid pointers
    while the object lives."""

    def __init__(self, *, num_q_heads: int, scale: float, max_blocks: int, key=None, value=None,
                 slot_mapping=None, dec_out=None, dec_q=None, dec_block_tables=None, dec_seq_lens=None,
                 dec_max_seq_len: int = 0, partition_tokens: int = 0, workspace=None, pre_out=None, pre_q=None,
                 pre_cu_q_lens=None, pre_block_tables=None, pre_seq_lens=None, pre_max_q_len: int = 0):
        self.tensors = [key, value, slot_mapping, dec_out, dec_q, dec_block_tables, dec_seq_lens, workspace,
                        pre_out, pre_q, pre_cu_q_lens, pre_block_tables, pre_seq_lens]
        self.named = dict(key=key, value=value, slot_mapping=slot_mapping, dec_out=dec_out, dec_q=dec_q,
                          dec_block_tables=dec_block_tables, dec_seq_lens=dec_seq_lens, workspace=workspace,
                          pre_out=pre_out, pre_q=pre_q, pre_cu_q_lens=pre_cu_q_lens,
                          pre_block_tables=pre_block_tables, pre_seq_lens=pre_seq_lens)
        self.num_q_heads = int(num_q_heads)
        self.max_blocks = int(max_blocks)
        d = _StepDesc()
        d.key, d.value, d.slot_mapping = _dptr(key), _dptr(value), _dptr(slot_mapping)
        d.num_new_tokens = 0 if slot_mapping is None else int(slot_mapping.shape[0])
        d.num_q_heads, d.scale, d.max_blocks = int(num_q_heads), float(scale), int(max_blocks)
        d.dec_out, d.dec_q = _dptr(dec_out), _dptr(dec_q)
        d.dec_block_tables, d.dec_seq_lens = _dptr(dec_block_tables), _dptr(dec_seq_lens)
        d.dec_batch = 0 if dec_seq_lens is None else int(dec_seq_lens.shape[0])
        d.dec_max_seq_len, d.partition_tokens = int(dec_max_seq_len), int(partition_tokens)
        d.workspace = _dptr(workspace)
        d.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        d.pre_out, d.pre_q, d.pre_cu_q_lens = _dptr(pre_out), _dptr(pre_q), _dptr(pre_cu_q_lens)
        d.pre_block_tables, d.pre_seq_lens = _dptr(pre_block_tables), _dptr(pre_seq_lens)
        d.pre_batch = 0 if pre_seq_lens is None else int(pre_seq_lens.shape[0])
        d.pre_max_q_len = int(pre_max_q_len)
        self.c = d
        self._checked = None  # (pool handle, generation) the tensors were last checked against


def _check_step(pool: int, desc: StepDesc) -> None:
    """Each part of the step that runs (a non-zero count) against the pool's
    layout, as pa_write_kv, pa_decode and pa_prefill check theirs. The
    description's pointers and counts are fixed when it is built, and a
    pool's layout never changes, so the check runs once per pool this binding
    created (every call for a pool made elsewhere)."""
    import torch
    gen = _pool_gen.get(pool)
    key = None if gen is None else (pool, gen)
    if key is not None and desc._checked == key:
        return
    lay = pa_pool_layout(pool)
    t = desc.named
    Hq, mb = desc.num_q_heads, desc.max_blocks
    if t["slot_mapping"] is not None and int(t["slot_mapping"].shape[0]) > 0:
        _want(t["slot_mapping"], "slot_mapping", (None,), torch.int64)
        T = int(t["slot_mapping"].shape[0])
        _want_kv_rows(lay, "key", t["key"], T)
        _want_kv_rows(lay, "value", t["value"], T)
    if t["dec_seq_lens"] is not None and int(t["dec_seq_lens"].shape[0]) > 0:
        _want(t["dec_seq_lens"], "dec_seq_lens", (None,), torch.int32)
        B = int(t["dec_seq_lens"].shape[0])
        _want(t["dec_q"], "dec_q", (B, Hq, lay["head_dim"]), _compute_dtype(lay))
        _want(t["dec_out"], "dec_out", (B, Hq, lay["head_dim"]), _compute_dtype(lay))
        _want(t["dec_block_tables"], "dec_block_tables", (B, mb), torch.int32)
        _want_workspace(t["workspace"])
    if t["pre_seq_lens"] is not None and int(t["pre_seq_lens"].shape[0]) > 0:
        _want(t["pre_seq_lens"], "pre_seq_lens", (None,), torch.int32)
        B = int(t["pre_seq_lens"].shape[0])
        _want(t["pre_q"], "pre_q", (None, Hq, lay["head_dim"]), _compute_dtype(lay))
        _want(t["pre_out"], "pre_out", tuple(int(x) for x in t["pre_q"].shape), _compute_dtype(lay))
        _want(t["pre_cu_q_lens"], "pre_cu_q_lens", (B + 1,), torch.int32)
        _want(t["pre_block_tables"], "pre_block_tables", (B, mb), torch.int32)
    _want_gpu(**t)
    desc._checked = key


def pa_step(pool: int, desc: StepDesc, stream=None) -> None:
    _check_step(pool, desc)
    _check(lib.pa_step(pool, ctypes.byref(desc.c), _stream(stream)), "pa_step")


def pa_step_graph_create(pool: int, desc: StepDesc) -> int:
    _check_step(pool, desc)
    g = _vp()
    _check(lib.pa_step_graph_create(pool, ctypes.byref(desc.c), ctypes.byref(g)), "pa_step_graph_create")
    return g.value


def pa_step_graph_launch(graph: int, stream=None) -> None:
    _check(lib.pa_step_graph_launch(graph, _stream(stream)), "pa_step_graph_launch")


def pa_step_graph_destroy(graph: int) -> None:
    lib.pa_step_graph_destroy(graph)


class _PrefixStats(ctypes.Structure):
    _fields_ = [("cached_blocks", ctypes.c_int32), ("lookups", ctypes.c_int64), ("hits", ctypes.c_int64)]


def pa_seq_append_tokens(pool: int, seq_id: int, token_ids) -> tuple:
    """Token-aware append with prefix caching. Returns (slots int64 array with
    -1 where the K/V is already cached, number of cached tokens)."""
    ids = np.ascontiguousarray(token_ids, dtype=np.int32)
    n = len(ids)
    slots = np.empty(max(n, 1), dtype=np.int64)
    cached = ctypes.c_int32()
    _check(lib.pa_seq_append_tokens(pool, seq_id, ids.ctypes.data if n else None, n,
                                    slots.ctypes.data if n else None, ctypes.byref(cached)),
           "pa_seq_append_tokens")
    return slots[:n], cached.value


def pa_pool_prefix_stats(pool: int) -> dict:
    st = _PrefixStats()
    _check(lib.pa_pool_prefix_stats(pool, ctypes.byref(st)), "pa_pool_prefix_stats")
    return {"cached_blocks": st.cached_blocks, "lookups": st.lookups, "hits": st.hits}


def pa_tier_block_size(expected_len: int) -> int:
    return int(lib.pa_tier_block_size(int(expected_len)))
