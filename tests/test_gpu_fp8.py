"""GPU parity of the FP8 (E4M3) KV cache: quantising scatter and decode (HIP, through the C ABI).

* quantisation bit-exact against the oracle codec: every finite bf16 value
  (and ±inf, ±0) at scale 1, and random values at the non-power-of-two
  scales of the FP8 workload, with values beyond ±448 saturating;
* the whole FP8 pool of the 8B-shaped GQA batch bit-exact against the
  oracle's, never-written slots included (both poison them with the NaN code);
* decode over an FP8 pool within the bf16 tolerances (max-abs <= 2e-2,
  mean-abs <= 2e-3) against the fp64 oracle on the dequantised values, for
  the 8B-shaped batch and ragged small shapes (G in {1, 2, 4, 8}, block sizes
  8/16/32, several partitions, empty and one-token sequences);
* output invariance under the partition size.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle.attention as OA  # noqa: E402
import oracle.fp8 as F8  # noqa: E402
import workloads as W  # noqa: E402
from oracle.cache import OracleCache  # noqa: E402

TOL = (2e-2, 2e-3)


def _pa():
    import paged_kv_cache_indirect_amd as pa
    return pa


def _harness():
    from tests import harness
    return harness


def assert_close(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    print(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert err.max() <= TOL[0], f"{what}: max abs err {err.max()}"
    assert err.mean() <= TOL[1], f"{what}: mean abs err {err.mean()}"


def quantize_on_gpu(values_f32, k_scale, v_scale):
    """Scatter rows of bf16 values (Hkv 2, D 128) into a fresh FP8 pool; return
    the K and V codes of the written slots in row order."""
    pa = _pa()
    h = _harness()
    hkv, d, bs = 2, 128, 16
    per_row = hkv * d
    n = len(values_f32)
    T = -(-n // per_row)
    flat = np.zeros(T * per_row, np.float32)
    flat[:n] = values_f32
    bits = (flat.view(np.uint32) >> 16).astype(np.uint16)          # exact: inputs are bf16 values
    rows = bits.reshape(T, hkv, d)
    nb = -(-T // bs) + 1
    kc = torch.zeros((nb, bs, hkv, d), dtype=torch.float8_e4m3fn, device="cuda")
    vc = torch.zeros_like(kc)
    pool = pa.pa_alloc_pool(kc, vc, np.arange(nb, dtype=np.int32))
    try:
        pa.pa_pool_set_kv_scales(pool, k_scale, v_scale)
        slots = pa.pa_seq_append(pool, 0, T)
        key = h.to_device(rows, "bf16", "cuda")
        pa.pa_write_kv(pool, key, key, torch.from_numpy(slots).cuda())
        torch.cuda.synchronize()
        kf = h.to_host(kc, "fp8").reshape(-1, hkv, d)[slots].reshape(-1)[:n]
        vf = h.to_host(vc, "fp8").reshape(-1, hkv, d)[slots].reshape(-1)[:n]
    finally:
        pa.pa_free_pool(pool)
    return kf, vf, (bits[:n].astype(np.uint32) << 16).view(np.float32)


def test_quantize_every_bf16_value_scale_one():
    u = np.arange(65536, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    # every bf16 value except fp32 subnormals; NaNs of both signs included
    keep = np.isnan(f) | (np.abs(f) >= np.float32(1.2e-38)) | (f == 0)
    x = f[keep]
    assert np.isnan(x).sum() == 254
    print(f"[fp8 quantize] {len(x)} bf16 values (NaNs included), scale 1", flush=True)
    kq, vq, xin = quantize_on_gpu(x, 1.0, 1.0)
    ref = F8.quantize_e4m3(xin, 1.0)
    bad = np.nonzero(kq != ref)[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. x={xin[bad[:5]]} gpu={kq[bad[:5]]} oracle={ref[bad[:5]]}"
    assert np.array_equal(vq, ref)


@pytest.mark.parametrize("k_scale,v_scale", [(0.0137, 0.0129), (3.0, 0.25)])
def test_quantize_random_values_scaled(k_scale, v_scale):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200_000) * rng.choice([0.003, 1.0, 8.0], 200_000)).astype(np.float32)
    kq, vq, xin = quantize_on_gpu(x, k_scale, v_scale)
    assert np.array_equal(kq, F8.quantize_e4m3(xin, k_scale))
    assert np.array_equal(vq, F8.quantize_e4m3(xin, v_scale))


def build_both(wl, only=None):
    print(f"[build] {wl.name} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} bs={wl.block_size} fp8 "
          f"k_scale={wl.k_scale} v_scale={wl.v_scale} max_len={wl.max_seq_len}", flush=True)
    gpu = _harness().GpuCache(wl)
    ora = OracleCache(wl, only=only)
    assert np.array_equal(gpu.tables_host, ora.block_tables)
    assert np.array_equal(gpu.lens_host, ora.seq_lens)
    return gpu, ora


def oracle_out(wl, ora, seqs=None):
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    out, _ = OA.paged_decode(wl.queries()[seqs], ora.k_cache, ora.v_cache, ora.block_tables[seqs],
                             ora.seq_lens[seqs], wl.scale, wl.dtype, wl.cache_dtype, wl.k_scale, wl.v_scale)
    return out


def widen_out(t):
    return OA.widen(_harness().to_host(t, "bf16"), "bf16")


def test_fp8_gqa8b_pool_bit_exact_and_decode():
    wl = W.config("gqa8b_fp8")
    gpu, ora = build_both(wl)
    hk = _harness().to_host(gpu.k_cache, "fp8")
    hv = _harness().to_host(gpu.v_cache, "fp8")
    assert np.array_equal(hk, ora.k_cache), "k_cache codes differ"
    assert np.array_equal(hv, ora.v_cache), "v_cache codes differ"
    ref = oracle_out(wl, ora)
    for pt in (512, 1024):
        got = widen_out(gpu.decode(pt, gpu.workspace_for(pt)))
        assert_close(got, ref, f"gqa8b_fp8 pt={pt}")
    gpu.close()


SMALL = [
    # lens, Hq, Hkv, bs, partition_tokens
    ([1, 7, 16, 17, 63, 64, 65, 500, 1025], 8, 2, 16, 128),
    ([0, 1, 300, 2049], 8, 2, 16, 512),
    ([33, 1000, 5], 4, 4, 8, 64),
    ([777, 64, 31], 16, 2, 32, 256),
    ([900, 2, 129], 2, 1, 16, 128),
]


@pytest.mark.parametrize("lens,Hq,Hkv,bs,pt", SMALL)
def test_fp8_decode_small_shapes(lens, Hq, Hkv, bs, pt):
    wl = W.make_decode(f"fp8small{len(lens)}", lens, Hq=Hq, Hkv=Hkv, D=128, block_size=bs, dtype="bf16",
                       seed=9, kv_dtype="fp8", k_scale=0.021, v_scale=0.017)
    gpu, ora = build_both(wl)
    got = widen_out(gpu.decode(pt, gpu.workspace_for(pt)))
    assert_close(got, oracle_out(wl, ora), f"fp8 small {lens} G={Hq // Hkv} bs={bs} pt={pt}")
    gpu.close()
