"""Pins for the oracle's INT8 key/value cache mode (TileMix abstract: INT8
key/value caches), checked against things other than itself:

- a numpy brute force that dequantises the cache (K^ = s_k * k8,
  V^ = s_v * v8) and runs softmax(scale * Q K^T + mask) V^, with the INT8
  routed cells taken from the cached codes;
- bit-exact equality with the fp16 path when the cache represents fp16
  tensors exactly (power-of-two scales, a +-127 code in every row, so the
  fp16 path's own quantiser reproduces the cached codes);
- the cache encoder against the numpy restatement of the quantiser.
"""
import numpy as np
import pytest

import workloads
from test_oracle_pins import np_bits, np_quantize, rand16


def np_attention_one_kv8(q, k8, sk, v8, sv, scale, causal, route=None, tpb=1, tile_q=64, tile_k=64):
    """q [Lq,d] fp16, k8/v8 [Lk,d] int8, sk/sv [Lk] fp32 -> fp64 [Lq,d]."""
    Lq, Lk = q.shape[0], k8.shape[0]
    kd = sk.astype(np.float64)[:, None] * k8.astype(np.float64)
    vd = sv.astype(np.float64)[:, None] * v8.astype(np.float64)
    sc = float(np.float32(scale))
    S = sc * (q.astype(np.float64) @ kd.T)
    if route is not None:
        q8, sq = np_quantize(q)
        dot = q8.astype(np.int64) @ k8.astype(np.int64).T
        S8 = sc * sq.astype(np.float64)[:, None] * sk.astype(np.float64)[None, :] * dot.astype(np.float64)
        n_qt = -(-Lq // tile_q)
        n_g = -(-(-(-Lk // tile_k)) // tpb)
        bits = np_bits(route, n_qt, n_g)
        qt = np.arange(Lq) // tile_q
        g = (np.arange(Lk) // tile_k) // tpb
        S = np.where(bits[qt[:, None], g[None, :]], S8, S)
    if causal:
        S = np.where(np.tril(np.ones((Lq, Lk), dtype=bool), k=Lk - Lq), S, -np.inf)
    e = np.exp(S - S.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ vd


def np_attention_kv8(q, k8, sk, v8, sv, scale, causal, cu=None, route=None, tpb=1, tile_q=64, tile_k=64):
    out = np.zeros(q.shape, dtype=np.float64)
    if cu is not None:
        G = q.shape[0] // k8.shape[0]
        r0 = 0
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            n_qt = -(-(b - a) // tile_q)
            rows = None if route is None else route[r0:r0 + n_qt]
            r0 += n_qt
            for h in range(q.shape[0]):
                if b > a:
                    hk = h // G
                    out[h, a:b] = np_attention_one_kv8(q[h, a:b], k8[hk, a:b], sk[hk, a:b], v8[hk, a:b],
                                                       sv[hk, a:b], scale, causal, rows, tpb, tile_q, tile_k)
        return out
    G = q.shape[1] // k8.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            hk = h // G
            out[b, h] = np_attention_one_kv8(q[b, h], k8[b, hk], sk[b, hk], v8[b, hk], sv[b, hk], scale, causal,
                                             route, tpb, tile_q, tile_k)
    return out


def rand_cache(rng, shape):
    """Random codes in [-127, 127] and positive fp32 scales of a non-trivial spread."""
    k8 = rng.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)
    sk = (rng.uniform(0.5, 2.0, size=shape[:-1]) / 127).astype(np.float32)
    return k8, sk


@pytest.mark.parametrize("heads", [(1, 1), (4, 2), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_kv8_vs_bruteforce(orc, heads, causal, d):
    rng = np.random.default_rng(900 + d + 10 * heads[0] + heads[1] + causal)
    for (qsl, ksl) in [(1, 1), (5, 17), (65, 65), (17, 130)]:
        if causal and qsl > ksl:
            continue
        q = rand16(rng, (2, heads[0], qsl, d))
        k8, sk = rand_cache(rng, (2, heads[1], ksl, d))
        v8, sv = rand_cache(rng, (2, heads[1], ksl, d))
        got = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.1, causal=causal)
        ref = np_attention_kv8(q, k8, sk, v8, sv, 0.1, causal)
        assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("tile", [(2, 2), (4, 2), (64, 64)])
@pytest.mark.parametrize("tpb", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_kv8_routed_vs_bruteforce(orc, tile, tpb, causal):
    rng = np.random.default_rng(950 + tile[0] + 7 * tile[1] + tpb + causal)
    qsl, ksl, d = 19, 23, 64
    q = rand16(rng, (1, 4, qsl, d))
    k8, sk = rand_cache(rng, (1, 2, ksl, d))
    v8, sv = rand_cache(rng, (1, 2, ksl, d))
    n_qt = -(-qsl // tile[0])
    n_g = workloads.n_route_groups(ksl, tpb, tile[1])
    route = workloads.pack_bits(rng.random((n_qt, n_g)) < 0.5)
    got = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.2, causal=causal, route=route, tiles_per_bit=tpb,
                           tile_q=tile[0], tile_k=tile[1])
    ref = np_attention_kv8(q, k8, sk, v8, sv, 0.2, causal, route=route, tpb=tpb, tile_q=tile[0], tile_k=tile[1])
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_kv8_varlen_vs_bruteforce(orc, routed, causal):
    rng = np.random.default_rng(970 + routed + 2 * causal)
    lens = [1, 5, 0, 17, 9]
    cu = workloads.cu_seqlens_of(lens)
    T, d = int(cu[-1]), 64
    q = rand16(rng, (4, T, d))
    k8, sk = rand_cache(rng, (2, T, d))
    v8, sv = rand_cache(rng, (2, T, d))
    route = None
    if routed:
        n_rows = sum(-(-L // 4) for L in lens)
        route = workloads.pack_bits(rng.random((n_rows, workloads.n_route_groups(T, 1, 4))) < 0.5)
    got = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.15, causal=causal, cu_seqlens=cu, route=route,
                           tiles_per_bit=1, tile_q=4, tile_k=4)
    ref = np_attention_kv8(q, k8, sk, v8, sv, 0.15, causal, cu=cu, route=route, tpb=1, tile_q=4, tile_k=4)
    assert np.max(np.abs(got - ref)) <= 1e-12


def exact_cache(rng, shape, e):
    """Codes with a +-127 in every row and scale 2^-e: s * code is an exact fp16
    value and the quantiser maps that fp16 row back to the same codes and scale."""
    c = rng.integers(-127, 128, size=shape, dtype=np.int64)
    idx = rng.integers(0, shape[-1], size=shape[:-1])
    np.put_along_axis(c, idx[..., None], np.where(rng.random(shape[:-1]) < 0.5, 127, -127)[..., None], axis=-1)
    s = np.full(shape[:-1], 2.0 ** -e, dtype=np.float32)
    x = (c.astype(np.float64) * 2.0 ** -e).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), c * 2.0 ** -e)
    return c.astype(np.int8), s, x


@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_kv8_exact_cache_equals_fp16_path_bitexact(orc, routed, causal):
    rng = np.random.default_rng(990 + routed + 2 * causal)
    qsl, ksl, d = 70, 150, 128
    q = rand16(rng, (1, 4, qsl, d))
    k8, sk, k = exact_cache(rng, (1, 2, ksl, d), 5)
    v8, sv, v = exact_cache(rng, (1, 2, ksl, d), 6)
    qk8, qsk = orc.quantize_rows(k)
    assert np.array_equal(qk8, k8) and np.array_equal(qsk, sk)
    route = None
    if routed:
        route = workloads.pack_bits(rng.random((2, workloads.n_route_groups(ksl, 1))) < 0.5)
    a = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.09, causal=causal, route=route, tiles_per_bit=1)
    b = orc.attn_fwd(q, k, v, scale=0.09, causal=causal, route=route, tiles_per_bit=1)
    assert np.array_equal(a, b)


def test_kv8_rows_entry_matches_full(orc):
    rng = np.random.default_rng(995)
    q = rand16(rng, (2, 4, 40, 64))
    k8, sk = rand_cache(rng, (2, 2, 50, 64))
    v8, sv = rand_cache(rng, (2, 2, 50, 64))
    route = workloads.pack_bits(rng.random((1, 1)) < 2)
    full = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.1, causal=True, route=route, tiles_per_bit=4)
    rows = [(0, 0, 0), (1, 3, 39), (0, 2, 17), (1, 1, 5)]
    got = orc.attn_rows_kv8(q, k8, sk, v8, sv, rows, scale=0.1, causal=True, route=route, tiles_per_bit=4)
    for n, (s, h, i) in enumerate(rows):
        assert np.array_equal(got[n], full[s, h, i])


def test_cache_encoder_vs_numpy(orc):
    rng = np.random.default_rng(996)
    x = rand16(rng, (3, 5, 33, 64), sd=3.0)
    x[0, 0, 0] = 0                      # zero row: scale 0, codes 0
    x[0, 0, 1] = np.float16(0.5)        # constant row: every code 127
    x[1, 2, 3, :8] = np.float16(65504)  # the fp16 maximum
    q8, s = orc.quantize_rows(x)
    rq, rs = np_quantize(x)
    assert np.array_equal(q8, rq) and np.array_equal(s, rs)
    assert s[0, 0, 0] == 0 and not q8[0, 0, 0].any()
    assert np.all(q8[0, 0, 1] == 127)


def test_kv8_rejects_undefined_problems(orc):
    rng = np.random.default_rng(997)
    q = rand16(rng, (1, 4, 64))
    k8, sk = rand_cache(rng, (1, 4, 64))
    with pytest.raises(ValueError):      # cu_seqlens does not end at T
        orc.attn_fwd_kv8(q, k8, sk, k8, sk, scale=0.1, causal=True, cu_seqlens=[0, 3])
    q4 = rand16(rng, (1, 1, 5, 64))
    k4, s4 = rand_cache(rng, (1, 1, 4, 64))
    with pytest.raises(ValueError):      # causal with qsl > ksl
        orc.attn_fwd_kv8(q4, k4, s4, k4, s4, scale=0.1, causal=True)
