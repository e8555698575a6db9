"""The Python binding rejects tensors that disagree with the pool's layout.

The kernels size every device access from the pool's geometry, so a q with a
smaller head_dim, a narrower dtype or index tensors of the wrong width would
be read or written out of bounds on the device. The binding checks each call's
tensors against ``pa_pool_layout`` first and raises ValueError. Runs on the
CPU: the pool is created through the C ABI over placeholder addresses (pool
creation and the layout getter never touch device memory), and the checks
fire before any library call that would.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pa = pytest.importorskip("paged_kv_cache_indirect_amd")

NB, BS, HKV, D = 64, 16, 2, 128


@pytest.fixture
def pool():
    def make(dtype):
        lay = pa._Layout(NB, BS, HKV, D, dtype)
        h = ctypes.c_void_p()
        assert pa.lib.pa_alloc_pool(ctypes.byref(lay), ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), None,
                                    ctypes.byref(h)) == pa.PA_OK
        made.append(h.value)
        return h.value
    made = []
    yield make
    for h in made:
        pa.pa_free_pool(h)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_layout_getter(pool):
    p = pool(pa.PA_BF16)
    assert pa.pa_pool_layout(p) == {"num_blocks": NB, "block_size": BS, "num_kv_heads": HKV, "head_dim": D,
                                    "dtype": pa.PA_BF16}
    with pytest.raises(pa.PaError):
        pa.pa_pool_layout(None)


def test_decode_checks(pool):
    p = pool(pa.PA_BF16)
    B, Hq = 3, 8
    good = dict(out=t(B, Hq, D), q=t(B, Hq, D), block_tables=t(B, 4, dtype=torch.int32),
                seq_lens=t(B, dtype=torch.int32))

    def call(**kw):
        a = dict(good, **kw)
        pa.pa_decode(p, a["out"], a["q"], a["block_tables"], a["seq_lens"], 0.1, 64)

    bad = [
        dict(q=t(B, Hq, 64), out=t(B, Hq, 64)),                 # head_dim of another pool
        dict(q=t(B, Hq, D, dtype=torch.float32)),                # dtype of another pool
        dict(q=t(B, 7, D), out=t(B, 7, D)),                      # q heads not a multiple of kv heads
        dict(out=t(B, Hq, 64)),                                  # out smaller than q
        dict(out=t(B + 1, Hq, D)),
        dict(block_tables=t(B, 4, dtype=torch.int64)),           # index widths
        dict(seq_lens=t(B, dtype=torch.int64)),
        dict(seq_lens=t(B - 1, dtype=torch.int32)),
        dict(block_tables=t(B - 1, 4, dtype=torch.int32)),
        dict(q=t(B, Hq, 2 * D)[:, :, ::2]),                      # not contiguous
        {},                                                      # matching, but host tensors
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            call(**kw)


def test_append_decode_checks(pool):
    p = pool(pa.PA_BF16)
    B, Hq = 3, 8
    good = dict(out=t(B, Hq, D), q=t(B, Hq, D), key=t(B, HKV, D), value=t(B, HKV, D),
                slots=t(B, dtype=torch.int64), block_tables=t(B, 4, dtype=torch.int32),
                seq_lens=t(B, dtype=torch.int32))

    def call(**kw):
        a = dict(good, **kw)
        pa.pa_append_decode(p, a["out"], a["q"], a["key"], a["value"], a["slots"], a["block_tables"],
                            a["seq_lens"], 0.1, 64)

    for kw in [dict(key=t(B, HKV, 64)), dict(value=t(B, 4, D)), dict(key=t(B, HKV, D, dtype=torch.float32)),
               dict(slots=t(B, dtype=torch.int32)), dict(slots=t(B + 2, dtype=torch.int64)), {}]:
        with pytest.raises(ValueError):
            call(**kw)

    def call_args(slots=np.zeros(B, np.int64), lens=np.ones(B, np.int32), **kw):
        a = dict(good, **kw)
        pa.pa_append_decode_args(p, a["out"], a["q"], a["key"], a["value"], slots, a["block_tables"], lens, 0.1, 64)

    for kw in [dict(slots=np.zeros(B - 1, np.int64)), dict(lens=np.ones(1, np.int32)), dict(key=t(B, 1, D)), {}]:
        with pytest.raises(ValueError):
            call_args(**kw)


def test_write_kv_checks(pool):
    p = pool(pa.PA_BF16)
    T = 5
    for key, value, slots in [
        (t(T, HKV, 64), t(T, HKV, 64), t(T, dtype=torch.int64)),        # head_dim
        (t(T, 1, D), t(T, 1, D), t(T, dtype=torch.int64)),              # kv heads
        (t(T, HKV, D, dtype=torch.float32), t(T, HKV, D, dtype=torch.float32), t(T, dtype=torch.int64)),
        (t(T, HKV, D), t(T, HKV, D), t(T, dtype=torch.int32)),          # slot width
        (t(T + 1, HKV, D), t(T + 1, HKV, D), t(T, dtype=torch.int64)),  # more rows than slots... checked
        (t(T, HKV, D), t(T, HKV, D), t(T, dtype=torch.int64)),          # matching, but host tensors
    ]:
        with pytest.raises(ValueError):
            pa.pa_write_kv(p, key, value, slots)


def test_fp8_pool_takes_bf16_rows(pool):
    p = pool(pa.PA_FP8_E4M3)
    with pytest.raises(ValueError, match="bfloat16"):
        pa.pa_write_kv(p, t(2, HKV, D, dtype=torch.float8_e4m3fn), t(2, HKV, D, dtype=torch.float8_e4m3fn),
                       t(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU"):           # right types, host memory
        pa.pa_write_kv(p, t(2, HKV, D), t(2, HKV, D), t(2, dtype=torch.int64))


def test_prefill_checks(pool):
    p = pool(pa.PA_BF16)
    T, Hq, B = 40, 8, 2
    good = dict(out=t(T, Hq, D), q=t(T, Hq, D), cu=t(B + 1, dtype=torch.int32),
                block_tables=t(B, 4, dtype=torch.int32), seq_lens=t(B, dtype=torch.int32))

    def call(**kw):
        a = dict(good, **kw)
        pa.pa_prefill(p, a["out"], a["q"], a["cu"], a["block_tables"], a["seq_lens"], 0.1, 32)

    for kw in [dict(q=t(T, Hq, 64), out=t(T, Hq, 64)), dict(out=t(T - 1, Hq, D)), dict(cu=t(B, dtype=torch.int32)),
               dict(cu=t(B + 1, dtype=torch.int64)), dict(block_tables=t(B + 1, 4, dtype=torch.int32)), {}]:
        with pytest.raises(ValueError):
            call(**kw)


def test_step_checks(pool):
    p = pool(pa.PA_BF16)
    Bd, Hq, mb = 2, 8, 4
    base = dict(num_q_heads=Hq, scale=0.1, max_blocks=mb, dec_out=t(Bd, Hq, D), dec_q=t(Bd, Hq, D),
                dec_block_tables=t(Bd, mb, dtype=torch.int32), dec_seq_lens=t(Bd, dtype=torch.int32),
                dec_max_seq_len=64)
    for kw in [dict(dec_q=t(Bd, Hq, 64)), dict(dec_block_tables=t(Bd, mb + 1, dtype=torch.int32)),
               dict(key=t(3, HKV, D), value=t(3, HKV, D), slot_mapping=t(3, dtype=torch.int32)), {}]:
        desc = pa.StepDesc(**dict(base, **kw))
        with pytest.raises(ValueError):
            pa.pa_step(p, desc)
        with pytest.raises(ValueError):
            pa.pa_step_graph_create(p, desc)


def test_debug_switch_round_trip():
    was = pa.pa_set_debug_checks(True)
    try:
        assert pa.pa_set_debug_checks(False) is True
        assert pa.pa_set_debug_checks(False) is False
    finally:
        pa.pa_set_debug_checks(was)
