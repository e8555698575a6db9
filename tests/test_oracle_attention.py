"""Pins for the attention oracle (CPU only).

The oracle is checked against things other than itself:
* a library routine: torch's fp64 CPU scaled_dot_product_attention (with its
  own grouped-query mapping) on the unpaged, contiguous K/V;
* brute force: pure-Python loops with math.exp that address each token
  through the block table one by one;
* invariances the definition implies: relabelling physical blocks, and
  sharing prefix blocks vs private copies, leave the output bit-identical;
* closed forms: L = 1, scale = 0, identical keys, a dominant key;
* the log-sum-exp merge identity over random cut points;
* mutation checks: a plausible mistake planted in a copy of the oracle makes
  at least one of these pins fail.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as OA
import workloads as W

TOL = 1e-12


# ----------------------------------------------------------------- helpers
def page_out(seqs, bs, num_blocks, perm):
    """Place contiguous per-sequence rows [L, H, D] into a pool block by block.

    Logical block i of sequence b goes to physical block perm[next]; tail
    slots and unused blocks are filled with NaN so that reading them shows.
    Returns (pool [num_blocks, bs, H, D], tables [B, max_blocks] padded -1).
    """
    H, D = seqs[0].shape[1], seqs[0].shape[2]
    pool = np.full((num_blocks, bs, H, D), np.nan)
    nblk = [-(-s.shape[0] // bs) for s in seqs]
    mb = max(1, max(nblk))
    tables = np.full((len(seqs), mb), -1, dtype=np.int64)
    it = iter(perm)
    for b, s in enumerate(seqs):
        for i in range(nblk[b]):
            p = int(next(it))
            rows = s[i * bs:(i + 1) * bs]
            pool[p, :rows.shape[0]] = rows
            tables[b, i] = p
    return pool, tables


def sdpa_decode(q, K, V, scale):
    """torch fp64 SDPA for one sequence: q [Hq, D], K/V [L, Hkv, D] -> [Hq, D]."""
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


def random_case(rng, lens, Hq, Hkv, D, bs, extra_blocks=3):
    Ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    Vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    q = rng.standard_normal((len(lens), Hq, D))
    need = sum(-(-L // bs) for L in lens)
    nb = need + extra_blocks
    perm = rng.permutation(nb)
    return Ks, Vs, q, nb, perm


CASES = [
    # lens, Hq, Hkv, D, bs
    ([7, 16, 33, 50], 2, 2, 64, 16),
    ([1, 15, 16, 17, 64, 100], 8, 2, 32, 16),
    ([3, 9, 31, 32, 33], 4, 1, 16, 8),
    ([40, 5, 70], 6, 3, 8, 32),
]


# ------------------------------------------------------------ library pin
@pytest.mark.parametrize("lens,Hq,Hkv,D,bs", CASES)
def test_decode_matches_unpaged_sdpa(lens, Hq, Hkv, D, bs):
    rng = np.random.default_rng(7)
    Ks, Vs, q, nb, perm = random_case(rng, lens, Hq, Hkv, D, bs)
    kpool, tables = page_out(Ks, bs, nb, perm)
    vpool, _ = page_out(Vs, bs, nb, perm)
    scale = 1.0 / math.sqrt(D)
    # fp64 pools: paged_decode's widen('f32') would round them to fp32, so this
    # pin drives the fp64 gather + attend core directly.
    out = np.zeros_like(q)
    for b, L in enumerate(lens):
        for h in range(Hq):
            K = OA.gather_sequence(kpool, tables[b], L, bs)[:, h // (Hq // Hkv)]
            V = OA.gather_sequence(vpool, tables[b], L, bs)[:, h // (Hq // Hkv)]
            out[b, h], _ = OA.attend(q[b, h], K, V, scale)
        ref = sdpa_decode(q[b], Ks[b], Vs[b], scale)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=TOL)


@pytest.mark.parametrize("lens,Hq,Hkv,D,bs", CASES)
def test_paged_decode_api_matches_sdpa_on_f32_data(lens, Hq, Hkv, D, bs):
    """Same pin through the public paged_decode entry, on fp32-representable data."""
    rng = np.random.default_rng(11)
    Ks, Vs, q, nb, perm = random_case(rng, lens, Hq, Hkv, D, bs)
    Ks = [k.astype(np.float32).astype(np.float64) for k in Ks]
    Vs = [v.astype(np.float32).astype(np.float64) for v in Vs]
    q = q.astype(np.float32)
    kpool, tables = page_out(Ks, bs, nb, perm)
    vpool, _ = page_out(Vs, bs, nb, perm)
    scale = 1.0 / math.sqrt(D)
    out, lse = OA.paged_decode(q, kpool.astype(np.float32), vpool.astype(np.float32), tables,
                               np.array(lens), scale, "f32")
    for b in range(len(lens)):
        ref = sdpa_decode(q[b].astype(np.float64), Ks[b], Vs[b], scale)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=TOL)
        # lse: log Σ exp(scale q·k) computed independently with torch.logsumexp
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = torch.from_numpy(Ks[b][:, g] @ q[b, h].astype(np.float64) * scale)
            assert abs(lse[b, h] - torch.logsumexp(s, 0).item()) < 1e-10


def test_bf16_widening_is_exact():
    # bf16 bit patterns with known values: 1.0 = 0x3F80, -2.0 = 0xC000, 0.15625 = 0x3E20
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x0000, 0x8000], dtype=np.uint16)
    np.testing.assert_array_equal(OA.widen(bits, "bf16"), [1.0, -2.0, 0.15625, 0.0, -0.0])
    # generator's rounding: RNE on a tie and a non-tie
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    np.testing.assert_array_equal(OA.widen(W.round_to_bf16_bits(x), "bf16"),
                                  [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7])


# ----------------------------------------------------------- brute force
def brute_force_decode(q, kpool, vpool, tables, lens, scale, Hkv):
    """Pure-Python loops: each token fetched through its table entry on its own."""
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    G = Hq // Hkv
    bs = len(kpool[0])
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            scores = []
            for t in range(lens[b]):
                blk, off = tables[b][t // bs], t % bs
                scores.append(scale * math.fsum(q[b][h][d] * kpool[blk][off][g][d] for d in range(D)))
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            tot = math.fsum(w)
            for d in range(D):
                out[b][h][d] = math.fsum(w[t] * vpool[tables[b][t // bs]][t % bs][g][d]
                                         for t in range(lens[b])) / tot
    return np.array(out)


def test_decode_brute_force_tiny_workload():
    """The tiny workload (4 seqs, lengths 7/16/33/50, 32-block permuted pool)."""
    from oracle.block_manager import BlockManagerModel
    from oracle.scatter import write_kv
    wl = W.config("tiny")
    bm = BlockManagerModel(wl.num_blocks, wl.block_size, wl.free_order)
    kc = np.zeros((wl.num_blocks, wl.block_size, wl.Hkv, wl.D), np.float32)
    vc = np.zeros_like(kc)
    for op in wl.ops:
        st, slots = bm.append(op[1], op[2])
        assert st == 0
        k, v = wl.kv_rows(op[1], 0, op[2])
        write_kv(kc, vc, k, v, np.array(slots))
    st, tables, lens = bm.block_tables(range(wl.B), wl.max_blocks)
    tables = np.array(tables)
    q = wl.queries()
    out, _ = OA.paged_decode(q, kc, vc, tables, np.array(lens), wl.scale, "f32")
    ref = brute_force_decode(q.astype(np.float64).tolist(), kc.astype(np.float64).tolist(),
                             vc.astype(np.float64).tolist(), tables.tolist(), lens, wl.scale, wl.Hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=TOL)


# ------------------------------------------------------------ invariances
@pytest.mark.parametrize("lens,Hq,Hkv,D,bs", CASES)
def test_permutation_invariance_bit_exact(lens, Hq, Hkv, D, bs):
    rng = np.random.default_rng(3)
    Ks, Vs, q, nb, perm = random_case(rng, lens, Hq, Hkv, D, bs, extra_blocks=10)
    outs = []
    for p in (perm, rng.permutation(nb), np.arange(nb)):
        kpool, tables = page_out([k.astype(np.float32) for k in Ks], bs, nb, p)
        vpool, _ = page_out([v.astype(np.float32) for v in Vs], bs, nb, p)
        outs.append(OA.paged_decode(q.astype(np.float32), kpool.astype(np.float32),
                                    vpool.astype(np.float32), tables, np.array(lens),
                                    0.125, "f32")[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_prefix_sharing_invariance_bit_exact():
    """Shared physical prefix blocks vs private copies give identical outputs."""
    rng = np.random.default_rng(5)
    bs, Hkv, Hq, D, P = 16, 2, 4, 32, 48
    pk, pv = rng.standard_normal((P, Hkv, D)), rng.standard_normal((P, Hkv, D))
    suffix = [0, 5, 16, 21]
    sk = [rng.standard_normal((s, Hkv, D)) for s in suffix]
    sv = [rng.standard_normal((s, Hkv, D)) for s in suffix]
    q = rng.standard_normal((len(suffix), Hq, D)).astype(np.float32)
    full_k = [np.concatenate([pk, k]).astype(np.float32) for k in sk]
    full_v = [np.concatenate([pv, v]).astype(np.float32) for v in sv]
    lens = np.array([P + s for s in suffix])
    # private copies: every sequence holds its own copy of the prefix blocks
    nb = sum(-(-L // bs) for L in lens)
    perm = rng.permutation(nb)
    kpool, tables = page_out(full_k, bs, nb, perm)
    vpool, _ = page_out(full_v, bs, nb, perm)
    out_private = OA.paged_decode(q, kpool.astype(np.float32), vpool.astype(np.float32), tables,
                                  lens, 0.2, "f32")[0]
    # shared: prefix blocks 0..2 once, each sequence's suffix blocks after them
    npre = P // bs
    nb2 = npre + sum(-(-s // bs) for s in suffix)
    k2 = np.full((nb2, bs, Hkv, D), np.nan, np.float32)
    v2 = np.full_like(k2, np.nan)
    k2[:npre] = pk.astype(np.float32).reshape(npre, bs, Hkv, D)
    v2[:npre] = pv.astype(np.float32).reshape(npre, bs, Hkv, D)
    t2 = np.full((len(suffix), tables.shape[1]), -1)
    nxt = npre
    for b, s in enumerate(suffix):
        t2[b, :npre] = np.arange(npre)
        for i in range(-(-s // bs)):
            rows = sk[b][i * bs:(i + 1) * bs]
            k2[nxt, :len(rows)] = rows
            v2[nxt, :len(rows)] = sv[b][i * bs:(i + 1) * bs]
            t2[b, npre + i] = nxt
            nxt += 1
    out_shared = OA.paged_decode(q, k2, v2, t2, lens, 0.2, "f32")[0]
    assert np.array_equal(out_private, out_shared)


# ----------------------------------------------------------- closed forms
def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    V = rng.standard_normal((1, 8))
    out, lse = OA.attend(rng.standard_normal(8), rng.standard_normal((1, 8)), V, 0.3)
    assert np.array_equal(out, V[0])


def test_zero_scale_gives_mean_of_values():
    rng = np.random.default_rng(2)
    K, V = rng.standard_normal((37, 16)), rng.standard_normal((37, 16))
    out, lse = OA.attend(rng.standard_normal(16), K, V, 0.0)
    np.testing.assert_allclose(out, V.mean(0), rtol=0, atol=TOL)
    assert abs(lse - math.log(37)) < TOL


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    k = rng.standard_normal(16)
    K, V = np.tile(k, (21, 1)), rng.standard_normal((21, 16))
    out, _ = OA.attend(rng.standard_normal(16), K, V, 0.7)
    np.testing.assert_allclose(out, V.mean(0), rtol=0, atol=TOL)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((50, 32))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((50, 32))
    for t in (0, 17, 49):
        out, _ = OA.attend(2000.0 * K[t], K, V, 1.0)
        np.testing.assert_allclose(out, V[t], rtol=0, atol=1e-9)


def test_empty_sequence():
    out, lse = OA.attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.array_equal(out, np.zeros(4)) and lse == -np.inf


# ------------------------------------------------------------- prefill
def sdpa_masked(q, K, V, scale, mask):
    """q [n, Hq, D], K/V [L, Hkv, D], mask [n, L] bool (True = attend)."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale,
                                       enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


def prefill_case(rng, ctx, qlens, Hq, Hkv, D, bs):
    lens = [c + n for c, n in zip(ctx, qlens)]
    Ks, Vs, _, nb, perm = random_case(rng, lens, Hq, Hkv, D, bs)
    Ks = [k.astype(np.float32) for k in Ks]
    Vs = [v.astype(np.float32) for v in Vs]
    q = rng.standard_normal((sum(qlens), Hq, D)).astype(np.float32)
    kpool, tables = page_out(Ks, bs, nb, perm)
    vpool, _ = page_out(Vs, bs, nb, perm)
    cu = np.concatenate([[0], np.cumsum(qlens)])
    return Ks, Vs, q, kpool.astype(np.float32), vpool.astype(np.float32), tables, np.array(lens), cu


@pytest.mark.parametrize("ctx,qlens,Hq,Hkv,D,bs", [
    ([0, 0, 0], [5, 16, 33], 4, 2, 16, 16),
    ([0, 3, 40, 17], [7, 1, 20, 32], 4, 1, 16, 8),
    ([64, 0], [12, 40], 6, 3, 8, 32),
])
def test_prefill_matches_masked_sdpa(ctx, qlens, Hq, Hkv, D, bs):
    rng = np.random.default_rng(8)
    Ks, Vs, q, kp, vp, tables, lens, cu = prefill_case(rng, ctx, qlens, Hq, Hkv, D, bs)
    out, _ = OA.paged_prefill(q, cu, kp, vp, tables, lens, 0.25, "f32")
    for b, (c, n) in enumerate(zip(ctx, qlens)):
        L = c + n
        mask = np.arange(L)[None, :] <= (c + np.arange(n))[:, None]
        ref = sdpa_masked(q[cu[b]:cu[b + 1]].astype(np.float64), Ks[b].astype(np.float64),
                          Vs[b].astype(np.float64), 0.25, mask)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=0, atol=TOL)
        if c == 0:   # library causal mask (top-left aligned) coincides when there is no context
            qt = torch.from_numpy(np.ascontiguousarray(q[cu[b]:cu[b + 1]].astype(np.float64).transpose(1, 0, 2)))[None]
            kt = torch.from_numpy(np.ascontiguousarray(Ks[b].astype(np.float64).transpose(1, 0, 2)))[None]
            vt = torch.from_numpy(np.ascontiguousarray(Vs[b].astype(np.float64).transpose(1, 0, 2)))[None]
            ref2 = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.25,
                                                  enable_gqa=True)[0].numpy().transpose(1, 0, 2)
            np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref2, rtol=0, atol=TOL)


@pytest.mark.parametrize("ctx,qlens,Hq,Hkv,D,bs", [
    ([0, 0, 0], [5, 16, 33], 4, 2, 16, 16),
    ([0, 3, 40, 17], [7, 1, 20, 32], 4, 1, 16, 8),
    ([64, 0, 9], [12, 40, 0], 6, 3, 8, 32),       # an empty chunk
])
def test_prefill_masked_matches_masked_sdpa(ctx, qlens, Hq, Hkv, D, bs):
    """The matrix form of the causal prefill against the library's masked
    attention (fp64 SDPA with an explicit boolean mask)."""
    rng = np.random.default_rng(18)
    Ks, Vs, q, kp, vp, tables, lens, cu = prefill_case(rng, ctx, qlens, Hq, Hkv, D, bs)
    out, lse = OA.paged_prefill_masked(q, cu, kp, vp, tables, lens, 0.25, "f32")
    for b, (c, n) in enumerate(zip(ctx, qlens)):
        if n == 0:
            continue
        L = c + n
        mask = np.arange(L)[None, :] <= (c + np.arange(n))[:, None]
        ref = sdpa_masked(q[cu[b]:cu[b + 1]].astype(np.float64), Ks[b].astype(np.float64),
                          Vs[b].astype(np.float64), 0.25, mask)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref, rtol=0, atol=TOL)
    assert np.all(np.isfinite(lse))


def test_prefill_masked_rows_before_cache_start():
    """A 6-row chunk over a 4-token cache: rows at negative positions see no
    keys (zero output, lse -inf), the row at position 0 returns V[0], the last
    row attends to every token (library SDPA, no mask)."""
    rng = np.random.default_rng(11)
    Ks, Vs, q, kp, vp, tables, lens, cu = prefill_case(rng, [0], [4], 2, 1, 8, 8)   # L = 4
    q6 = rng.standard_normal((6, 2, 8)).astype(np.float32)
    out, lse = OA.paged_prefill_masked(q6, np.array([0, 6]), kp, vp, tables, lens, 0.5, "f32")
    assert np.array_equal(out[:2], np.zeros((2, 2, 8))) and np.all(lse[:2] == -np.inf)
    np.testing.assert_array_equal(out[2, :, :], np.repeat(Vs[0][0:1, 0, :].astype(np.float64), 2, 0))
    ref = sdpa_masked(q6[5:6].astype(np.float64), Ks[0].astype(np.float64), Vs[0].astype(np.float64),
                      0.5, np.ones((1, 4), bool))
    np.testing.assert_allclose(out[5], ref[0], rtol=0, atol=TOL)


def test_prefill_masked_brute_force():
    """Pure-Python loops with math.exp over a paged bf16 cache (tables walked
    by hand, one score at a time) against the matrix form."""
    rng = np.random.default_rng(19)
    ctx, qlens, Hq, Hkv, D, bs = [3, 0], [4, 5], 4, 2, 8, 4
    lens = [c + n for c, n in zip(ctx, qlens)]
    nb = sum(-(-L // bs) for L in lens) + 2
    kp = W.draw_values(rng, (nb, bs, Hkv, D), "bf16")
    vp = W.draw_values(rng, (nb, bs, Hkv, D), "bf16")
    q = W.draw_values(rng, (sum(qlens), Hq, D), "bf16")
    perm = rng.permutation(nb)
    tables = np.full((2, 3), -1, dtype=np.int32)
    k = 0
    for b, L in enumerate(lens):
        for i in range(-(-L // bs)):
            tables[b, i] = perm[k]
            k += 1
    cu = np.concatenate([[0], np.cumsum(qlens)])
    out, _ = OA.paged_prefill_masked(q, cu, kp, vp, tables, np.array(lens), 0.3, "bf16")

    def val(bits):
        return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])

    for b, (c, n) in enumerate(zip(ctx, qlens)):
        L = c + n
        for i in range(n):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                scores = []
                for t in range(L - n + i + 1):
                    blk, off = int(tables[b, t // bs]), t % bs
                    scores.append(0.3 * sum(val(q[cu[b] + i, h, d]) * val(kp[blk, off, g, d]) for d in range(D)))
                m = max(scores)
                w = [math.exp(x - m) for x in scores]
                for d in range(D):
                    acc = 0.0
                    for t, wt in enumerate(w):
                        blk, off = int(tables[b, t // bs]), t % bs
                        acc += wt * val(vp[blk, off, g, d])
                    assert abs(acc / sum(w) - out[cu[b] + i, h, d]) < 1e-12


def test_prefill_last_row_equals_decode():
    rng = np.random.default_rng(9)
    Ks, Vs, q, kp, vp, tables, lens, cu = prefill_case(rng, [10, 0, 33], [6, 9, 16], 4, 2, 16, 16)
    out, lse = OA.paged_prefill(q, cu, kp, vp, tables, lens, 0.3, "f32")
    last = np.stack([q[cu[b + 1] - 1] for b in range(3)])
    dout, dlse = OA.paged_decode(last, kp, vp, tables, lens, 0.3, "f32")
    for b in range(3):
        np.testing.assert_allclose(out[cu[b + 1] - 1], dout[b], rtol=0, atol=TOL)


def test_prefill_rows_before_cache_start_are_empty():
    # A chunk of 6 rows over a cache of 4 tokens: rows 0 and 1 sit at
    # positions -2 and -1 and see no keys; row 2 sees token 0 only, so its
    # output is V[0] exactly; the last row sees all 4 tokens.
    rng = np.random.default_rng(11)
    Ks, Vs, q, kp, vp, tables, lens, cu = prefill_case(rng, [0], [4], 2, 1, 8, 8)   # L = 4
    q6 = rng.standard_normal((6, 2, 8)).astype(np.float32)
    out, lse = OA.paged_prefill(q6, np.array([0, 6]), kp, vp, tables, lens, 0.5, "f32")
    assert np.array_equal(out[:2], np.zeros((2, 2, 8))) and np.all(lse[:2] == -np.inf)
    np.testing.assert_array_equal(out[2, :, :], np.repeat(Vs[0][0:1, 0, :].astype(np.float64), 2, 0))
    ref = sdpa_masked(q6[5:6].astype(np.float64), Ks[0].astype(np.float64), Vs[0].astype(np.float64),
                      0.5, np.ones((1, 4), bool))
    np.testing.assert_allclose(out[5], ref[0], rtol=0, atol=TOL)


def test_prefill_rows_subset_matches_full():
    rng = np.random.default_rng(10)
    Ks, Vs, q, kp, vp, tables, lens, cu = prefill_case(rng, [10, 4], [6, 9], 4, 2, 16, 16)
    full, _ = OA.paged_prefill(q, cu, kp, vp, tables, lens, 0.3, "f32")
    part, _ = OA.paged_prefill(q, cu, kp, vp, tables, lens, 0.3, "f32", rows=[(0, 5), (1, 0), (1, 8)])
    for b, i in [(0, 5), (1, 0), (1, 8)]:
        assert np.array_equal(part[cu[b] + i], full[cu[b] + i])


# -------------------------------------------------------------- LSE merge
@pytest.mark.parametrize("seed", range(5))
def test_lse_merge_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    L, D = int(rng.integers(1, 300)), 24
    q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)) * 2, rng.standard_normal((L, D))
    cuts = np.sort(rng.integers(0, L + 1, size=int(rng.integers(0, 6))))
    bounds = [0, *cuts.tolist(), L]
    states = [OA.partial_state(q, K[a:b], V[a:b], 0.4) for a, b in zip(bounds[:-1], bounds[1:])]
    out, lse = OA.merge_partials(states)
    ref, ref_lse = OA.attend(q, K, V, 0.4)
    np.testing.assert_allclose(out, ref, rtol=0, atol=TOL)
    assert abs(lse - ref_lse) < 1e-10


# ------------------------------------------------------------- mutations
def _pins_pass(mod):
    """Run a subset of the pins against (possibly mutated) oracle functions."""
    try:
        test_decode_matches_unpaged_sdpa(*CASES[1])
        test_paged_decode_api_matches_sdpa_on_f32_data(*CASES[3])
        test_prefill_matches_masked_sdpa([0, 3, 40, 17], [7, 1, 20, 32], 4, 1, 16, 8)
        test_prefill_masked_matches_masked_sdpa([0, 3, 40, 17], [7, 1, 20, 32], 4, 1, 16, 8)
        test_prefill_masked_matches_masked_sdpa([64, 0, 9], [12, 40, 0], 6, 3, 8, 32)
        test_prefill_masked_rows_before_cache_start()
        for s in range(3):
            test_lse_merge_equals_unsplit(s)
        test_decode_brute_force_tiny_workload()
    except AssertionError:
        return False
    return True


def test_pins_pass_on_real_oracle():
    assert _pins_pass(OA)


MUTANTS = {}


def _mut(name):
    def deco(fn):
        MUTANTS[name] = fn
        return fn
    return deco


@_mut("table ignored (logical block used as physical)")
def _m1(monkeypatch):
    orig = OA.gather_sequence
    monkeypatch.setattr(OA, "gather_sequence",
                        lambda c, row, L, bs: orig(c, np.arange(len(row)), L, bs))


@_mut("GQA mapping h % Hkv")
def _m2(monkeypatch):
    def paged_decode(q, kc, vc, bt, sl, scale, dtype):
        B, Hq, D = q.shape
        bs, Hkv = kc.shape[1], kc.shape[2]
        out = np.zeros((B, Hq, D)); lse = np.zeros((B, Hq))
        for b in range(B):
            K = OA.widen(OA.gather_sequence(kc, bt[b], int(sl[b]), bs), dtype)
            V = OA.widen(OA.gather_sequence(vc, bt[b], int(sl[b]), bs), dtype)
            for h in range(Hq):
                out[b, h], lse[b, h] = OA.attend(OA.widen(q[b, h], dtype), K[:, h % Hkv], V[:, h % Hkv], scale)
        return out, lse
    monkeypatch.setattr(OA, "paged_decode", paged_decode)


@_mut("scale dropped")
def _m3(monkeypatch):
    orig = OA.attend
    monkeypatch.setattr(OA, "attend", lambda q, K, V, s: orig(q, K, V, 1.0))


@_mut("tail of last block read (L rounded up to whole blocks)")
def _m4(monkeypatch):
    orig = OA.gather_sequence
    monkeypatch.setattr(OA, "gather_sequence",
                        lambda c, row, L, bs: np.nan_to_num(orig(c, row, -(-L // bs) * bs, bs)))


@_mut("causal bound off by one")
def _m5(monkeypatch):
    orig = OA.attend
    def paged_prefill(q, cu, kc, vc, bt, sl, scale, dtype, rows=None):
        T, Hq, D = q.shape
        bs, Hkv = kc.shape[1], kc.shape[2]
        G = Hq // Hkv
        out = np.zeros((T, Hq, D)); lse = np.zeros((T, Hq))
        for b in range(len(sl)):
            L = int(sl[b]); r0, r1 = int(cu[b]), int(cu[b + 1]); n = r1 - r0
            K = OA.widen(OA.gather_sequence(kc, bt[b], L, bs), dtype)
            V = OA.widen(OA.gather_sequence(vc, bt[b], L, bs), dtype)
            for i in range(n):
                pos = L - n + i
                for h in range(Hq):
                    out[r0 + i, h], lse[r0 + i, h] = orig(OA.widen(q[r0 + i, h], dtype),
                                                          K[:pos, h // G], V[:pos, h // G], scale)
        return out, lse
    monkeypatch.setattr(OA, "paged_prefill", paged_prefill)


def _masked_mutant(monkeypatch, allowed_fn, kv_head_fn):
    """A matrix-form prefill with one planted change: the key mask or the
    kv head a q head reads."""
    def paged_prefill_masked(q, cu, kc, vc, bt, sl, scale, dtype):
        T, Hq, D = q.shape
        bs, Hkv = kc.shape[1], kc.shape[2]
        out = np.zeros((T, Hq, D)); lse = np.full((T, Hq), -np.inf)
        for b in range(len(sl)):
            L = int(sl[b]); r0, r1 = int(cu[b]), int(cu[b + 1]); n = r1 - r0
            if n == 0:
                continue
            K = OA.widen(OA.gather_sequence(kc, bt[b], L, bs), dtype)
            V = OA.widen(OA.gather_sequence(vc, bt[b], L, bs), dtype)
            Q = OA.widen(q[r0:r1], dtype)
            pos = (L - n) + np.arange(n)
            allowed = allowed_fn(np.arange(L)[None, :], pos[:, None])
            for h in range(Hq):
                g = kv_head_fn(h, Hq, Hkv)
                S = np.where(allowed, scale * (Q[:, h] @ K[:, g].T), -np.inf)
                m = S.max(axis=1, initial=-np.inf)
                m = np.where(np.isfinite(m), m, 0.0)
                Wt = np.exp(S - m[:, None])
                den = Wt.sum(axis=1)
                out[r0:r1, h] = np.where(den[:, None] > 0, (Wt @ V[:, g]) / np.where(den > 0, den, 1)[:, None], 0)
                lse[r0:r1, h] = np.where(den > 0, m + np.log(np.where(den > 0, den, 1)), -np.inf)
        return out, lse
    monkeypatch.setattr(OA, "paged_prefill_masked", paged_prefill_masked)


@_mut("matrix-form prefill: causal mask t < pos")
def _m8(monkeypatch):
    _masked_mutant(monkeypatch, lambda t, p: t < p, lambda h, Hq, Hkv: h // (Hq // Hkv))


@_mut("matrix-form prefill: kv head h % Hkv")
def _m9(monkeypatch):
    _masked_mutant(monkeypatch, lambda t, p: t <= p, lambda h, Hq, Hkv: h % Hkv)


@_mut("merge without rescaling by exp(m_p - M)")
def _m6(monkeypatch):
    def merge(states):
        num = sum(acc for _, _, acc in states)
        den = sum(l for _, l, _ in states)
        return num / den, 0.0
    monkeypatch.setattr(OA, "merge_partials", merge)


@_mut("softmax max not subtracted consistently (sum uses raw exp)")
def _m7(monkeypatch):
    def attend(q, K, V, scale):
        if K.shape[0] == 0:
            return np.zeros(q.shape[-1]), -np.inf
        s = scale * (K @ q)
        m = s.max()
        return (np.exp(s - m) @ V) / np.exp(s).sum(), m
    monkeypatch.setattr(OA, "attend", attend)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert not _pins_pass(OA), f"no pin caught the planted mistake: {name}"
