"""Pins for the CPU oracle: it is checked against things other than itself.

- an independent numpy brute force of softmax(scale*QK^T + mask) V, with
  np.repeat for grouped-query heads, np.tril for the bottom-right causal mask,
  np.unpackbits for the routing bitmask and its own numpy INT8 quantiser;
- torch's CPU float64 scaled_dot_product_attention (a library routine) on
  the dense special case;
- closed forms and invariants (rows sum to one, causal row 0 is V[0], equal
  scores give the mean of V, the two-key logistic, GQA as MHA with repeated
  heads, bottom-right as the tail of a full causal run, packed = per-sequence,
  power-of-two scale equivariance, routing special cases);
- hand-worked quantiser examples from tests/golden and an exhaustive fp16
  sweep against the numpy quantiser;
- the page's throughput table for the FLOP convention.

Sources: "Nax Refactor" (ml-explore/mlx pull request 3271) timing tables;
TileMix abstract (Lattice paper summary).
"""
import math
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# --------------------------------------------------------------------------
# Independent numpy brute force
# --------------------------------------------------------------------------


def np_quantize(x16):
    """Per-row symmetric INT8 codes and fp32 scales, numpy only."""
    x32 = np.asarray(x16, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = (amax / np.float32(127)).astype(np.float32)
        inv = (np.float32(127) / amax).astype(np.float32)
    zero = amax == 0
    inv = np.where(zero, np.float32(0), inv)
    prod = x32.astype(np.float64) * inv.astype(np.float64)[..., None]
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    s = np.where(zero, np.float32(0), s).astype(np.float32)
    return q, s


def np_bits(words, n_rows, n_g):
    w = np.ascontiguousarray(words, dtype=np.uint32)
    b = np.unpackbits(w.view(np.uint8), bitorder="little").reshape(n_rows, -1)
    return b[:, :n_g].astype(bool)


def np_attention_one(q, k, v, scale, causal, route=None, tpb=1, tile_q=64, tile_k=64):
    """q [Lq,d], k/v [Lk,d] fp16 -> fp64 [Lq,d]."""
    Lq, Lk = q.shape[0], k.shape[0]
    qf, kf, vf = (a.astype(np.float64) for a in (q, k, v))
    S = float(np.float32(scale)) * (qf @ kf.T)
    if route is not None:
        q8, sq = np_quantize(q)
        k8, sk = np_quantize(k)
        dot = q8.astype(np.int64) @ k8.astype(np.int64).T
        S8 = float(np.float32(scale)) * sq.astype(np.float64)[:, None] * \
            sk.astype(np.float64)[None, :] * dot.astype(np.float64)
        n_qt = -(-Lq // tile_q)
        n_g = -(-(-(-Lk // tile_k)) // tpb)
        bits = np_bits(route, n_qt, n_g)
        qt = np.arange(Lq) // tile_q
        g = (np.arange(Lk) // tile_k) // tpb
        cell = bits[qt[:, None], g[None, :]]
        S = np.where(cell, S8, S)
    if causal:
        vis = np.tril(np.ones((Lq, Lk), dtype=bool), k=Lk - Lq)
        S = np.where(vis, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    P = e / e.sum(axis=1, keepdims=True)
    return P @ vf


def np_attention(q, k, v, scale, causal, cu=None, route=None, tpb=1, tile_q=64, tile_k=64):
    if cu is not None:
        out = np.zeros(q.shape, dtype=np.float64)
        G = q.shape[0] // k.shape[0]
        r0 = 0
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            n_qt = -(-(b - a) // tile_q)
            rows = None if route is None else route[r0:r0 + n_qt]
            r0 += n_qt
            for h in range(q.shape[0]):
                if b > a:
                    out[h, a:b] = np_attention_one(q[h, a:b], k[h // G, a:b], v[h // G, a:b], scale, causal,
                                                   rows, tpb, tile_q, tile_k)
        return out
    B, Hq = q.shape[:2]
    G = Hq // k.shape[1]
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    out = np.zeros(q.shape, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            out[b, h] = np_attention_one(q[b, h], kr[b, h], vr[b, h], scale, causal, route, tpb, tile_q, tile_k)
    return out


def rand16(rng, shape, sd=1.0):
    return (rng.standard_normal(shape) * sd).astype(np.float16)


# --------------------------------------------------------------------------
# Dense / GQA / mask / varlen vs brute force
# --------------------------------------------------------------------------

LENS = [1, 2, 3, 5, 17, 64, 65, 130]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(1, 1), (4, 2), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_vs_bruteforce(orc, d, heads, causal):
    rng = np.random.default_rng(1000 + d + 10 * heads[0] + heads[1] + int(causal))
    for qsl in LENS:
        for ksl in LENS:
            if causal and qsl > ksl:
                continue
            if (qsl * ksl) > 2000 and rng.random() < 0.7:
                continue  # keep the CPU suite short; the rest still spans the grid
            B = 2 if qsl < 20 else 1
            q = rand16(rng, (B, heads[0], qsl, d))
            k = rand16(rng, (B, heads[1], ksl, d))
            v = rand16(rng, (B, heads[1], ksl, d))
            scale = 1 / math.sqrt(d)
            got = orc.attn_fwd(q, k, v, scale=scale, causal=causal)
            ref = np_attention(q, k, v, scale, causal)
            assert np.max(np.abs(got - ref)) <= 1e-12, (qsl, ksl)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_vs_bruteforce(orc, causal):
    rng = np.random.default_rng(77 + causal)
    lens = [5, 0, 64, 1, 70]
    cu = workloads.cu_seqlens_of(lens)
    T = int(cu[-1])
    q = rand16(rng, (4, T, 64))
    k = rand16(rng, (2, T, 64))
    v = rand16(rng, (2, T, 64))
    got = orc.attn_fwd(q, k, v, scale=0.125, causal=causal, cu_seqlens=cu)
    ref = np_attention(q, k, v, 0.125, causal, cu=cu)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_dense_vs_torch_sdpa_float64(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    B, Hq, Hk, qsl, ksl, d = 2, 4, 2, 37, 70, 64
    q, k, v = rand16(rng, (B, Hq, qsl, d)), rand16(rng, (B, Hk, ksl, d)), rand16(rng, (B, Hk, ksl, d))
    for causal in (False, True):
        got = orc.attn_fwd(q, k, v, scale=0.125, causal=causal)
        tq = torch.from_numpy(q.astype(np.float64))
        tk = torch.from_numpy(k.astype(np.float64)).repeat_interleave(Hq // Hk, dim=1)
        tv = torch.from_numpy(v.astype(np.float64)).repeat_interleave(Hq // Hk, dim=1)
        mask = None
        if causal:
            mask = torch.ones(qsl, ksl, dtype=torch.bool).tril(diagonal=ksl - qsl)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.125)
        assert np.max(np.abs(got - ref.numpy())) <= 1e-12


# --------------------------------------------------------------------------
# Routed (TileMix) cells vs brute force with small tiles
# --------------------------------------------------------------------------


@pytest.mark.parametrize("tile", [(2, 2), (4, 2), (2, 4), (64, 64)])
@pytest.mark.parametrize("tpb", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_routed_vs_bruteforce(orc, tile, tpb, causal):
    tq, tk = tile
    rng = np.random.default_rng(900 + tq * 7 + tk + tpb * 31 + causal)
    for (qsl, ksl) in [(5, 17), (17, 17), (13, 40), (65, 130), (1, 9)]:
        if causal and qsl > ksl:
            continue
        d = 64
        q = rand16(rng, (1, 4, qsl, d))
        k = rand16(rng, (1, 2, ksl, d))
        v = rand16(rng, (1, 2, ksl, d))
        n_qt = -(-qsl // tq)
        n_g = -(-(-(-ksl // tk)) // tpb)
        bits = rng.random((n_qt, n_g)) < 0.5
        route = workloads.pack_bits(bits)
        got = orc.attn_fwd(q, k, v, scale=0.125, causal=causal, route=route, tiles_per_bit=tpb,
                           tile_q=tq, tile_k=tk)
        ref = np_attention(q, k, v, 0.125, causal, route=route, tpb=tpb, tile_q=tq, tile_k=tk)
        assert np.max(np.abs(got - ref)) <= 1e-12, (qsl, ksl)


@pytest.mark.parametrize("tile", [(2, 2), (4, 4), (64, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_routed_varlen_vs_bruteforce(orc, tile, causal):
    """Packed batch with a bitmask: each sequence reads its own stacked rows."""
    tq, tk = tile
    rng = np.random.default_rng(950 + tq + causal)
    lens = [5, 0, 17, 1, 40]
    cu = workloads.cu_seqlens_of(lens)
    T = int(cu[-1])
    tpb = 2
    q, k, v = rand16(rng, (4, T, 64)), rand16(rng, (2, T, 64)), rand16(rng, (2, T, 64))
    n_rows = sum(-(-L // tq) for L in lens)
    n_g_T = -(-(-(-T // tk)) // tpb)
    route = workloads.pack_bits(rng.random((n_rows, n_g_T)) < 0.5)
    got = orc.attn_fwd(q, k, v, scale=0.125, causal=causal, cu_seqlens=cu, route=route, tiles_per_bit=tpb,
                       tile_q=tq, tile_k=tk)
    ref = np_attention(q, k, v, 0.125, causal, cu=cu, route=route, tpb=tpb, tile_q=tq, tile_k=tk)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_routed_varlen_is_per_sequence(orc):
    rng = np.random.default_rng(960)
    lens = [70, 1, 150]
    cu = workloads.cu_seqlens_of(lens)
    T = int(cu[-1])
    q, k, v = rand16(rng, (4, T, 64)), rand16(rng, (2, T, 64)), rand16(rng, (2, T, 64))
    n_qts = [-(-L // 64) for L in lens]
    n_g_T = -(-(-(-T // 64)) // 1)
    bits = rng.random((sum(n_qts), n_g_T)) < 0.5
    route = workloads.pack_bits(bits)
    packed = orc.attn_fwd(q, k, v, scale=0.125, causal=True, cu_seqlens=cu, route=route, tiles_per_bit=1)
    r0 = 0
    for s, L in enumerate(lens):
        a, b = cu[s], cu[s + 1]
        own = workloads.pack_bits(bits[r0:r0 + n_qts[s], :-(-L // 64)])
        r0 += n_qts[s]
        one = orc.attn_fwd(np.ascontiguousarray(q[None, :, a:b]), np.ascontiguousarray(k[None, :, a:b]),
                           np.ascontiguousarray(v[None, :, a:b]), scale=0.125, causal=True, route=own,
                           tiles_per_bit=1)
        assert np.array_equal(packed[:, a:b], one[0])


def test_all_ones_is_uniform_int8(orc):
    rng = np.random.default_rng(11)
    q, k, v = rand16(rng, (1, 2, 70, 128)), rand16(rng, (1, 1, 150, 128)), rand16(rng, (1, 1, 150, 128))
    n_qt, n_g = 2, 3
    ones = workloads.pack_bits(np.ones((n_qt, n_g), dtype=bool))
    got = orc.attn_fwd(q, k, v, scale=0.088388346, causal=True, route=ones, tiles_per_bit=1)
    # uniform INT8 = brute force with every cell INT8
    ref = np.zeros_like(got)
    q8, sq = np_quantize(q[0])
    k8, sk = np_quantize(k[0])
    for h in range(2):
        S = float(np.float32(0.088388346)) * sq[h].astype(np.float64)[:, None] * sk[0].astype(np.float64)[None, :] * \
            (q8[h].astype(np.int64) @ k8[0].astype(np.int64).T)
        S = np.where(np.tril(np.ones((70, 150), bool), k=80), S, -np.inf)
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        ref[0, h] = P @ v[0, 0].astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_all_zero_mask_is_dense_bitexact(orc):
    rng = np.random.default_rng(12)
    q, k, v = rand16(rng, (1, 4, 100, 64)), rand16(rng, (1, 2, 200, 64)), rand16(rng, (1, 2, 200, 64))
    zeros = workloads.pack_bits(np.zeros((2, 1), dtype=bool))
    for causal in (False, True):
        a = orc.attn_fwd(q, k, v, scale=0.125, causal=causal, route=zeros, tiles_per_bit=4)
        b = orc.attn_fwd(q, k, v, scale=0.125, causal=causal)
        assert np.array_equal(a, b)


def test_single_bit_flip_changes_only_its_qtile(orc):
    rng = np.random.default_rng(13)
    qsl = ksl = 256
    q, k, v = rand16(rng, (1, 2, qsl, 64)), rand16(rng, (1, 1, ksl, 64)), rand16(rng, (1, 1, ksl, 64))
    base_bits = np.zeros((4, 4), dtype=bool)
    base = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=workloads.pack_bits(base_bits), tiles_per_bit=1)
    for (qt, g) in [(0, 0), (2, 1), (3, 3)]:
        bits = base_bits.copy()
        bits[qt, g] = True
        out = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=workloads.pack_bits(bits), tiles_per_bit=1)
        diff = np.any(out != base, axis=(0, 1, 3))
        rows = np.nonzero(diff)[0]
        assert rows.size > 0 and rows.min() >= 64 * qt and rows.max() < 64 * (qt + 1)


def test_illegal_group_bits_are_ignored(orc):
    rng = np.random.default_rng(14)
    q, k, v = rand16(rng, (1, 1, 256, 64)), rand16(rng, (1, 1, 256, 64)), rand16(rng, (1, 1, 256, 64))
    legal = np.tril(np.ones((4, 4), dtype=bool))          # qt >= g when tiles_per_bit = 1
    bits = rng.random((4, 4)) < 0.5
    a = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=workloads.pack_bits(bits & legal), tiles_per_bit=1)
    b = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=workloads.pack_bits(bits | ~legal), tiles_per_bit=1)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------


@pytest.mark.parametrize("routed", [False, True])
def test_rows_sum_to_one(orc, routed):
    rng = np.random.default_rng(21)
    q, k, v = rand16(rng, (1, 2, 90, 64)), rand16(rng, (1, 2, 130, 64)), rand16(rng, (1, 2, 130, 64))
    v[..., 0] = 1.0
    route = workloads.pack_bits(rng.random((2, 3)) < 0.5) if routed else None
    for causal in (False, True):
        o = orc.attn_fwd(q, k, v, scale=0.125, causal=causal, route=route, tiles_per_bit=1)
        assert np.max(np.abs(o[..., 0] - 1.0)) <= 1e-12


@pytest.mark.parametrize("routed", [False, True])
def test_causal_row0_is_v0(orc, routed):
    rng = np.random.default_rng(22)
    q, k, v = rand16(rng, (1, 4, 70, 128)), rand16(rng, (1, 2, 70, 128)), rand16(rng, (1, 2, 70, 128))
    route = workloads.pack_bits(np.ones((2, 1), dtype=bool)) if routed else None
    o = orc.attn_fwd(q, k, v, scale=0.088388346, causal=True, route=route, tiles_per_bit=2)
    for h in range(4):
        assert np.array_equal(o[0, h, 0], v[0, h // 2, 0].astype(np.float64))
        assert np.array_equal(orc.round_f16(o[0, h, 0]), v[0, h // 2, 0])


@pytest.mark.parametrize("routed", [False, True])
def test_equal_scores_give_mean(orc, routed):
    rng = np.random.default_rng(23)
    qsl, ksl = 40, 100
    q = np.zeros((1, 1, qsl, 64), dtype=np.float16)
    k, v = rand16(rng, (1, 1, ksl, 64)), rand16(rng, (1, 1, ksl, 64))
    route = workloads.pack_bits(np.ones((1, 2), dtype=bool)) if routed else None
    vf = v[0, 0].astype(np.float64)
    o = orc.attn_fwd(q, k, v, scale=0.125, causal=False, route=route, tiles_per_bit=1)
    assert np.max(np.abs(o[0, 0] - vf.mean(axis=0))) <= 1e-12
    o = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=route, tiles_per_bit=1)
    for i in range(qsl):
        n = i + (ksl - qsl) + 1
        assert np.max(np.abs(o[0, 0, i] - vf[:n].mean(axis=0))) <= 1e-12


def test_two_keys_logistic(orc):
    rng = np.random.default_rng(24)
    q, k, v = rand16(rng, (1, 1, 3, 64)), rand16(rng, (1, 1, 2, 64)), rand16(rng, (1, 1, 2, 64))
    o = orc.attn_fwd(q, k, v, scale=0.125, causal=False)
    for i in range(3):
        s = [0.125 * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, i], k[0, 0, j])) for j in range(2)]
        p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        exp = p0 * v[0, 0, 0].astype(np.float64) + (1 - p0) * v[0, 0, 1].astype(np.float64)
        assert np.max(np.abs(o[0, 0, i] - exp)) <= 1e-13


@pytest.mark.parametrize("routed", [False, True])
def test_gqa_is_mha_with_repeated_heads(orc, routed):
    rng = np.random.default_rng(25)
    q, k, v = rand16(rng, (2, 6, 50, 64)), rand16(rng, (2, 2, 80, 64)), rand16(rng, (2, 2, 80, 64))
    route = workloads.pack_bits(rng.random((1, 2)) < 0.5) if routed else None
    a = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=route, tiles_per_bit=1)
    b = orc.attn_fwd(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), scale=0.125, causal=True,
                     route=route, tiles_per_bit=1)
    assert np.array_equal(a, b)


def test_bottom_right_is_tail_of_full_causal(orc):
    rng = np.random.default_rng(26)
    ksl = 150
    q, k, v = rand16(rng, (1, 2, ksl, 64)), rand16(rng, (1, 1, ksl, 64)), rand16(rng, (1, 1, ksl, 64))
    full = orc.attn_fwd(q, k, v, scale=0.125, causal=True)
    for qsl in (1, 37, 64, 149):
        tail = orc.attn_fwd(np.ascontiguousarray(q[:, :, ksl - qsl:]), k, v, scale=0.125, causal=True)
        assert np.array_equal(tail, full[:, :, ksl - qsl:])


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_is_per_sequence(orc, causal):
    rng = np.random.default_rng(27)
    lens = [33, 1, 0, 90]
    cu = workloads.cu_seqlens_of(lens)
    T = int(cu[-1])
    q, k, v = rand16(rng, (4, T, 64)), rand16(rng, (1, T, 64)), rand16(rng, (1, T, 64))
    packed = orc.attn_fwd(q, k, v, scale=0.125, causal=causal, cu_seqlens=cu)
    for s, L in enumerate(lens):
        if L == 0:
            continue
        a, b = cu[s], cu[s + 1]
        one = orc.attn_fwd(np.ascontiguousarray(q[None, :, a:b]), np.ascontiguousarray(k[None, :, a:b]),
                           np.ascontiguousarray(v[None, :, a:b]), scale=0.125, causal=causal)
        assert np.array_equal(packed[:, a:b], one[0])


@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("kexp", [-2, 1])
def test_power_of_two_scale_equivariance(orc, routed, kexp):
    rng = np.random.default_rng(28)
    q, k, v = rand16(rng, (1, 2, 70, 64)), rand16(rng, (1, 1, 130, 64)), rand16(rng, (1, 1, 130, 64))
    route = workloads.pack_bits(rng.random((2, 3)) < 0.5) if routed else None
    a = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=route, tiles_per_bit=1)
    q2 = (q.astype(np.float64) * 2.0 ** kexp).astype(np.float16)
    assert np.array_equal(q2.astype(np.float64), q.astype(np.float64) * 2.0 ** kexp)
    b = orc.attn_fwd(q2, k, v, scale=0.125 * 2.0 ** -kexp, causal=True, route=route, tiles_per_bit=1)
    assert np.array_equal(a, b)


def test_rows_entry_matches_full(orc):
    rng = np.random.default_rng(29)
    q, k, v = rand16(rng, (2, 4, 100, 64)), rand16(rng, (2, 2, 180, 64)), rand16(rng, (2, 2, 180, 64))
    route = workloads.pack_bits(rng.random((2, 1)) < 0.5)
    full = orc.attn_fwd(q, k, v, scale=0.125, causal=True, route=route, tiles_per_bit=4)
    rows = [(0, 0, 0), (1, 3, 99), (0, 2, 64), (1, 1, 63), (0, 3, 17)]
    got = orc.attn_rows(q, k, v, rows, scale=0.125, causal=True, route=route, tiles_per_bit=4)
    for r, (s, h, i) in enumerate(rows):
        assert np.array_equal(got[r], full[s, h, i])
    cu = workloads.cu_seqlens_of([30, 70])
    qp, kp, vp = rand16(rng, (4, 100, 64)), rand16(rng, (2, 100, 64)), rand16(rng, (2, 100, 64))
    fullp = orc.attn_fwd(qp, kp, vp, scale=0.125, causal=True, cu_seqlens=cu)
    gotp = orc.attn_rows(qp, kp, vp, [(1, 3, 69), (0, 0, 0), (1, 0, 5)], scale=0.125, causal=True, cu_seqlens=cu)
    assert np.array_equal(gotp[0], fullp[3, 30 + 69])
    assert np.array_equal(gotp[1], fullp[0, 0])
    assert np.array_equal(gotp[2], fullp[0, 35])


def test_rejects_undefined_problems(orc):
    z = np.zeros((1, 1, 4, 64), dtype=np.float16)
    with pytest.raises(ValueError):
        orc.attn_fwd(z, z[:, :, :2], z[:, :, :2], scale=1.0, causal=True)   # qsl > ksl causal


# --------------------------------------------------------------------------
# fp16 codec
# --------------------------------------------------------------------------


def test_f16_decoder_all_patterns(orc):
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits[::7]])
    r = ref[::7]
    fin = np.isfinite(r)
    assert np.array_equal(got[fin], r[fin])
    assert np.array_equal(np.isnan(got), np.isnan(r))


def test_f16_encoder_rne(orc):
    rng = np.random.default_rng(30)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-8, 4.9, 3000),
                        np.arange(-2048, 2049) + 0.5, [65519.9, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, 0.0]])
    got = orc.round_f16(x)
    ref = x.astype(np.float16)          # numpy's double -> half is correctly rounded
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


# --------------------------------------------------------------------------
# Quantiser
# --------------------------------------------------------------------------


def _golden_quant():
    cases = []
    with open(os.path.join(GOLDEN, "quantizer_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            amax, s, xs, qs = [p.strip() for p in line.split("|")]
            cases.append((float(amax), float.fromhex(s), [float(t) for t in xs.split()],
                          [int(t) for t in qs.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_quant())
def test_quantizer_worked_examples(orc, case):
    amax, s, xs, qs = case
    x = np.array(xs, dtype=np.float16)
    assert np.array_equal(x.astype(np.float64), np.array(xs))    # every value is exact in fp16
    q8, sc = orc.quantize_row(x)
    assert q8.tolist() == qs
    assert float(sc) == s


def test_quantizer_exhaustive_fp16_sweep(orc):
    """Every finite fp16 x with |x| <= amax, for a set of amax values."""
    rng = np.random.default_rng(31)
    allx = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    allx = allx[np.isfinite(allx)]
    amaxes = [127.0, 254.0, 63.5, 1.0, 2.0 ** -10, 0.5, 65504.0, 3.0, 6.103515625e-05] + \
        [float(a) for a in np.abs(rng.standard_normal(40) * 4).astype(np.float16) if a > 0]
    for amax in amaxes:
        xs = allx[np.abs(allx.astype(np.float64)) <= amax]
        d = 255
        n = -(-xs.size // d)
        rows = np.zeros((n, d + 1), dtype=np.float16)
        rows[:, 0] = np.float16(amax)
        flat = np.zeros(n * d, dtype=np.float16)
        flat[:xs.size] = xs
        rows[:, 1:] = flat.reshape(n, d)
        ref_q, ref_s = np_quantize(rows)
        for r in range(0, n, max(1, n // 60)):
            q8, s = orc.quantize_row(rows[r])
            assert np.array_equal(q8, ref_q[r]), (amax, r)
            assert s == ref_s[r]


def test_int_dot_bound():
    # |dot| <= 127^2 * d < 2^24 for d <= 128, so an int32 accumulator and its fp32 value are exact
    assert 127 * 127 * 128 < 2 ** 24


# --------------------------------------------------------------------------
# Routing bitmask decode
# --------------------------------------------------------------------------


def test_route_bit_decode_vs_unpackbits(orc):
    rng = np.random.default_rng(32)
    for n_g in (1, 31, 32, 33, 64, 65, 100):
        n_rows = 7
        bits = rng.random((n_rows, n_g)) < 0.5
        words = workloads.pack_bits(bits)
        wpr = words.shape[1]
        assert wpr == -(-n_g // 32)
        ref = np_bits(words, n_rows, n_g)
        assert np.array_equal(ref, bits)
        for qt in range(n_rows):
            for g in range(n_g):
                assert orc.route_bit(words, wpr, qt, g) == int(ref[qt, g])


def test_words_per_row(orc):
    assert orc.words_per_row(16384, 64, 4) == 2
    assert orc.words_per_row(64, 64, 4) == 1
    assert orc.words_per_row(64 * 4 * 32 + 1, 64, 4) == 2
    assert workloads.n_route_groups(16384, 4) == 64


# --------------------------------------------------------------------------
# Throughput convention vs the page's table
# --------------------------------------------------------------------------


def test_metric_flop_matches_published_table():
    """FLOP convention: printed tflops == FLOP * 64 / t_fus within t_fus rounding."""
    with open(os.path.join(GOLDEN, "mlx_pr3271_fused_after.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 18
    for r in rows:
        B, qsl, ksl, hd, nq, nk = map(int, r[:6])
        causal = int(r[8])
        t_fus, tflops = float(r[10]), float(r[11])
        flop = workloads.metric_flop(B, nq, qsl, ksl, hd, causal)
        lo = flop * 64 / (t_fus + 0.0005) / 1e12
        hi = flop * 64 / (t_fus - 0.0005) / 1e12
        assert lo <= tflops <= hi, r
        # the un-halved count would miss the causal rows
        if causal:
            assert not (lo * 2 <= tflops <= hi * 2)
