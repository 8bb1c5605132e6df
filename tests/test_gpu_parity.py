"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Tolerance on fp16 outputs for N(0,1) inputs: max abs error <= 4e-3 and mean
abs error <= 5e-4.  Integer work (INT8 codes, routing decode) is compared
bit-exactly.  Small cases span several tiles with ragged tails; the
full-size workloads are run in the launch configuration bench.py times and
checked on sampled rows the oracle computes one by one.
"""
import sys

import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_ERR = 4e-3
MEAN_ERR = 5e-4


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_prefill_amd as A
    A.load()
    return A


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def words_tensor(route):
    return None if route is None else dev(np.ascontiguousarray(route, dtype=np.uint32).view(np.int32))


def gpu_attn(A, q, k, v, scale, causal, cu=None, route=None, tpb=4):
    out = A.attn_fwd(dev(q), dev(k), dev(v), scale=scale, causal=causal,
                     cu_seqlens=None if cu is None else dev(np.asarray(cu, dtype=np.int32)),
                     route_bitmask=words_tensor(route), tiles_per_bit=tpb)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(got, ref, label=""):
    g = got.astype(np.float64)
    assert np.all(np.isfinite(g)), label
    err = np.abs(g - ref)
    assert err.max() <= MAX_ERR and err.mean() <= MEAN_ERR, \
        "%s max %.3g mean %.3g" % (label, err.max(), err.mean())
    return err.max(), err.mean()


def rand16(rng, shape):
    return rng.standard_normal(shape).astype(np.float16)


# --------------------------------------------------------------------------
# small and ragged shapes vs the full oracle
# --------------------------------------------------------------------------

SHAPES = [(1, 1), (5, 70), (64, 64), (65, 65), (130, 130), (200, 333), (333, 200), (300, 1000)]


@pytest.fixture(params=["kg1", "kg2", "nw8", "nw2"])
def key_groups(request, monkeypatch):
    """The workgroup shapes of non-routed calls: four query wavefronts with one
    key group, or with two key groups that take alternate key tiles and merge
    in LDS (what small grids get by default), eight query wavefronts (what
    large grids get), or two query wavefronts with two key groups (what small
    causal hdim-64 grids get; larger head groups are split in pairs)."""
    if request.param in ("nw8", "nw2"):
        monkeypatch.setenv("ATTN_QUERY_WAVES", request.param[2])
        return int(request.param[2]) * 10
    monkeypatch.setenv("ATTN_QUERY_WAVES", "4")
    monkeypatch.setenv("ATTN_KEY_GROUPS", request.param[2])
    return int(request.param[2])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(3, 3), (4, 2), (8, 2), (8, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_dense_ragged(A, orc, d, heads, causal, key_groups):
    rng = np.random.default_rng(d * 100 + heads[0] * 10 + heads[1] + causal)
    for (qsl, ksl) in SHAPES:
        if causal and qsl > ksl:
            continue
        B = 2 if qsl <= 70 else 1
        say("dense d=%d heads=%s causal=%d B=%d qsl=%d ksl=%d shape=%d" % (d, heads, causal, B, qsl, ksl, key_groups))
        q, k, v = rand16(rng, (B, heads[0], qsl, d)), rand16(rng, (B, heads[1], ksl, d)), \
            rand16(rng, (B, heads[1], ksl, d))
        scale = float(np.float32(1 / np.sqrt(d)))
        got = gpu_attn(A, q, k, v, scale, causal)
        ref = orc.attn_fwd(q, k, v, scale=scale, causal=causal)
        check(got, ref, (qsl, ksl))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(2, 2), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ragged(A, orc, d, heads, causal, key_groups):
    rng = np.random.default_rng(7 + d + heads[1] + causal)
    lens = [1, 63, 64, 65, 200, 0, 130, 7]
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    say("varlen d=%d heads=%s causal=%d lens=%s shape=%d" % (d, heads, causal, lens, key_groups))
    q, k, v = rand16(rng, (heads[0], T, d)), rand16(rng, (heads[1], T, d)), rand16(rng, (heads[1], T, d))
    got = gpu_attn(A, q, k, v, 0.1, causal, cu=cu)
    ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, cu_seqlens=cu)
    check(got, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(2, 2), (4, 2), (8, 2), (12, 3)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tpb", [1, 3, 4])
def test_routed_ragged(A, orc, d, heads, causal, tpb, waves8):
    rng = np.random.default_rng(3 * d + heads[0] + 5 * heads[1] + causal + 11 * tpb)
    for (qsl, ksl) in [(64, 64), (130, 130), (200, 700), (333, 200)]:
        if causal and qsl > ksl:
            continue
        say("routed d=%d heads=%s causal=%d tpb=%d qsl=%d ksl=%d shape=%s" % (d, heads, causal, tpb, qsl, ksl,
                                                                           waves8))
        q, k, v = rand16(rng, (1, heads[0], qsl, d)), rand16(rng, (1, heads[1], ksl, d)), \
            rand16(rng, (1, heads[1], ksl, d))
        route = W.draw_route(qsl, ksl, tpb, 0.5, seed=int(rng.integers(1 << 30)))
        scale = float(np.float32(1 / np.sqrt(d)))
        got = gpu_attn(A, q, k, v, scale, causal, route=route, tpb=tpb)
        ref = orc.attn_fwd(q, k, v, scale=scale, causal=causal, route=route, tiles_per_bit=tpb)
        check(got, ref, (qsl, ksl))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(2, 2), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tpb", [1, 3, 4])
def test_routed_varlen_ragged(A, orc, d, heads, causal, tpb, waves8):
    """Packed batch with a bitmask: every sequence reads its own stacked rows."""
    rng = np.random.default_rng(500 + d + 7 * heads[1] + causal + 13 * tpb)
    lens = [1, 63, 64, 65, 200, 0, 130, 7]
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    n_rows = sum(-(-L // 64) for L in lens)
    n_g = W.n_route_groups(T, tpb)
    route = W.pack_bits(rng.random((n_rows, n_g)) < 0.5)
    say("routed varlen d=%d heads=%s causal=%d tpb=%d shape=%s" % (d, heads, causal, tpb, waves8))
    q, k, v = rand16(rng, (heads[0], T, d)), rand16(rng, (heads[1], T, d)), rand16(rng, (heads[1], T, d))
    got = gpu_attn(A, q, k, v, 0.1, causal, cu=cu, route=route, tpb=tpb)
    ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, cu_seqlens=cu, route=route, tiles_per_bit=tpb)
    check(got, ref)


@pytest.mark.parametrize("shape", ["nw2", "kg2", "nw8"])
@pytest.mark.parametrize("qsl", [64, 200, 448, 1000])
def test_gpu_causal_paired_block_order(A, orc, monkeypatch, shape, qsl):
    """Causal row blocks with the second half of the grid run light-first
    (what a fully resident grid of two-wavefront workgroups gets): every row
    is computed once, for even and odd block counts and every shape."""
    rng = np.random.default_rng(4700 + qsl + 7 * ["nw2", "kg2", "nw8"].index(shape))
    q, k, v = rand16(rng, (1, 8, qsl, 64)), rand16(rng, (1, 4, qsl + 37, 64)), rand16(rng, (1, 4, qsl + 37, 64))
    if shape == "kg2":
        monkeypatch.setenv("ATTN_QUERY_WAVES", "4")
        monkeypatch.setenv("ATTN_KEY_GROUPS", "2")
    else:
        monkeypatch.setenv("ATTN_QUERY_WAVES", shape[2])
    monkeypatch.setenv("ATTN_KSPLIT", "1")
    monkeypatch.setenv("ATTN_PAIR_BLOCKS", "1")
    say("paired blocks shape=%s qsl=%d" % (shape, qsl))
    got = gpu_attn(A, q, k, v, 0.125, True)
    ref = orc.attn_fwd(q, k, v, scale=0.125, causal=True)
    check(got, ref, (shape, qsl))


@pytest.mark.parametrize("shape", ["nw2", "kg2", "nw8"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ks", ["2", "3"])
def test_gpu_dense_split_keys_all_shapes(A, orc, monkeypatch, shape, causal, ks):
    """Key range split over workgroups (fp32 partials and the merge kernel)
    under every non-routed workgroup shape, at hdim 64 with a head group of 2."""
    rng = np.random.default_rng(4500 + 3 * int(ks) + causal + 10 * ["nw2", "kg2", "nw8"].index(shape))
    q, k, v = rand16(rng, (1, 4, 200, 64)), rand16(rng, (1, 2, 2100, 64)), rand16(rng, (1, 2, 2100, 64))
    if shape == "kg2":
        monkeypatch.setenv("ATTN_QUERY_WAVES", "4")
        monkeypatch.setenv("ATTN_KEY_GROUPS", "2")
    else:
        monkeypatch.setenv("ATTN_QUERY_WAVES", shape[2])
    monkeypatch.setenv("ATTN_KSPLIT", ks)
    say("dense split shape=%s causal=%d splits=%s" % (shape, causal, ks))
    got = gpu_attn(A, q, k, v, 0.125, causal)
    ref = orc.attn_fwd(q, k, v, scale=0.125, causal=causal)
    check(got, ref, (shape, ks))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tpb", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lowp", ["int8", "fp8"])
@pytest.mark.parametrize("ks", ["2", "3", "5"])
def test_gpu_routed_split_keys(A, orc, monkeypatch, d, tpb, causal, lowp, ks, waves8):
    """Key range split over workgroups on routed calls: every split walks its
    own tiles of each route (FP16 pass, then low-precision pass) from a start
    that may fall inside a routing group and inside a bitmask word (40 tiles,
    up to 40 groups, two words per row)."""
    rng = np.random.default_rng(4000 + d + 7 * tpb + causal + 3 * int(ks) + (lowp == "fp8"))
    qsl, ksl = 100, 2500
    q, k, v = rand16(rng, (1, 8, qsl, d)), rand16(rng, (1, 2, ksl, d)), rand16(rng, (1, 2, ksl, d))
    route = W.pack_bits(rng.random((-(-qsl // 64), W.n_route_groups(ksl, tpb))) < 0.5)
    monkeypatch.setenv("ATTN_KSPLIT", ks)
    say("routed split d=%d tpb=%d causal=%d lowp=%s splits=%s shape=%s" % (d, tpb, causal, lowp, ks, waves8))
    got = A.attn_fwd(dev(q), dev(k), dev(v), scale=0.1, causal=causal, route_bitmask=words_tensor(route),
                     tiles_per_bit=tpb, lowp=lowp)
    torch.cuda.synchronize()
    ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, route=route, tiles_per_bit=tpb, lowp=lowp)
    check(got.cpu().numpy(), ref, (lowp, ks))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("ks", ["2", "3", "8"])
def test_gpu_split_merge_repeatable(A, orc, monkeypatch, d, ks):
    """Key splits and their merge (summed in split order) give bit-identical
    outputs on repeated calls, with another split call of a different grid
    between them, dense and packed, and agree with the oracle."""
    rng = np.random.default_rng(4700 + d + int(ks))
    monkeypatch.setenv("ATTN_KSPLIT", ks)
    q, k, v = rand16(rng, (2, 4, 150, d)), rand16(rng, (2, 2, 1500, d)), rand16(rng, (2, 2, 1500, d))
    cu = [0, 700, 1150, 1900]
    pq, pk, pv = rand16(rng, (4, 1900, d)), rand16(rng, (2, 1900, d)), rand16(rng, (2, 1900, d))
    say("split merge repeat d=%d splits=%s" % (d, ks))
    dense = [gpu_attn(A, q, k, v, 0.09, True) for _ in range(2)]
    packed = gpu_attn(A, pq, pk, pv, 0.09, True, cu=cu)
    dense.append(gpu_attn(A, q, k, v, 0.09, True))
    packed2 = gpu_attn(A, pq, pk, pv, 0.09, True, cu=cu)
    for o in dense[1:]:
        assert np.array_equal(o.view(np.uint16), dense[0].view(np.uint16))
    assert np.array_equal(packed.view(np.uint16), packed2.view(np.uint16))
    check(dense[0], orc.attn_fwd(q, k, v, scale=0.09, causal=True), ("dense", ks))
    check(packed, orc.attn_fwd(pq, pk, pv, scale=0.09, causal=True, cu_seqlens=cu), ("packed", ks))


@pytest.mark.parametrize("waves", ["4", "8"])
def test_gpu_routed_varlen_zero_mask_is_dense(A, monkeypatch, waves):
    """Routed calls run one key group; both calls are pinned to the same
    number of query wavefronts."""
    monkeypatch.setenv("ATTN_KEY_GROUPS", "1")
    monkeypatch.setenv("ATTN_QUERY_WAVES", waves)
    rng = np.random.default_rng(510)
    lens = [100, 1, 250, 64]
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    q, k, v = rand16(rng, (8, T, 128)), rand16(rng, (2, T, 128)), rand16(rng, (2, T, 128))
    zeros = W.pack_bits(np.zeros((sum(-(-L // 64) for L in lens), W.n_route_groups(T, 4)), dtype=bool))
    for causal in (False, True):
        a = gpu_attn(A, q, k, v, 0.1, causal, cu=cu, route=zeros, tpb=4)
        b = gpu_attn(A, q, k, v, 0.1, causal, cu=cu)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("d", [64, 128])
def test_routed_all_int8(A, orc, d):
    rng = np.random.default_rng(40 + d)
    qsl = ksl = 300
    q, k, v = rand16(rng, (1, 4, qsl, d)), rand16(rng, (1, 1, ksl, d)), rand16(rng, (1, 1, ksl, d))
    route = W.pack_bits(np.ones((5, 5), dtype=bool))
    say("all-int8 d=%d" % d)
    for causal in (False, True):
        got = gpu_attn(A, q, k, v, 0.1, causal, route=route, tpb=1)
        ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, route=route, tiles_per_bit=1)
        check(got, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lowp", ["int8", "fp8"])
def test_negative_scale(A, orc, d, lowp, waves8):
    """A negative scale (the queries are negated in the prologue, before any
    low-precision codes are made), dense and routed, both workgroup shapes."""
    rng = np.random.default_rng(50 + d + (lowp == "fp8"))
    q, k, v = rand16(rng, (1, 8, 100, d)), rand16(rng, (1, 2, 150, d)), rand16(rng, (1, 2, 150, d))
    route = W.pack_bits(rng.random((2, 3)) < 0.5)
    say("negative scale d=%d lowp=%s shape=%s" % (d, lowp, waves8))
    for r in (None, route):
        got = A.attn_fwd(dev(q), dev(k), dev(v), scale=-0.125, causal=True, route_bitmask=words_tensor(r),
                         tiles_per_bit=1, lowp=lowp)
        torch.cuda.synchronize()
        ref = orc.attn_fwd(q, k, v, scale=-0.125, causal=True, route=r, tiles_per_bit=1, lowp=lowp)
        check(got.cpu().numpy(), ref)


# --------------------------------------------------------------------------
# invariants on the GPU
# --------------------------------------------------------------------------


@pytest.mark.parametrize("routed", [False, True])
def test_gpu_causal_row0_is_v0(A, routed):
    rng = np.random.default_rng(60)
    q, k, v = rand16(rng, (1, 8, 200, 128)), rand16(rng, (1, 2, 200, 128)), rand16(rng, (1, 2, 200, 128))
    route = W.pack_bits(np.ones((4, 1), dtype=bool)) if routed else None
    got = gpu_attn(A, q, k, v, 0.088388346, True, route=route, tpb=4)
    for h in range(8):
        assert np.array_equal(got[0, h, 0], v[0, h // 4, 0])


@pytest.mark.parametrize("routed", [False, True])
def test_gpu_equal_scores_give_mean(A, routed):
    rng = np.random.default_rng(61)
    q = np.zeros((1, 4, 70, 64), dtype=np.float16)
    k, v = rand16(rng, (1, 4, 250, 64)), rand16(rng, (1, 4, 250, 64))
    route = W.pack_bits(np.ones((2, 4), dtype=bool)) if routed else None
    got = gpu_attn(A, q, k, v, 0.125, False, route=route, tpb=1)
    mean = v.astype(np.float64).mean(axis=2)
    assert np.max(np.abs(got.astype(np.float64) - mean[:, :, None, :])) <= 1e-3


@pytest.mark.parametrize("routed", [False, True])
def test_gpu_rows_sum_to_one(A, routed):
    rng = np.random.default_rng(62)
    q, k, v = rand16(rng, (1, 4, 190, 128)), rand16(rng, (1, 1, 400, 128)), rand16(rng, (1, 1, 400, 128))
    v[..., 0] = 1.0
    route = W.pack_bits(rng.random((3, 7)) < 0.5) if routed else None
    for causal in (False, True):
        got = gpu_attn(A, q, k, v, 0.09, causal, route=route, tpb=1)
        assert np.max(np.abs(got[..., 0].astype(np.float64) - 1.0)) <= 2e-3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("waves", ["4", "8"])
def test_gpu_all_zero_mask_is_dense_bitexact(A, d, monkeypatch, waves):
    """Routed calls run one key group; the dense call is pinned to the same
    shape (four or eight query wavefronts)."""
    monkeypatch.setenv("ATTN_KEY_GROUPS", "1")
    monkeypatch.setenv("ATTN_QUERY_WAVES", waves)
    rng = np.random.default_rng(63)
    q, k, v = rand16(rng, (1, 8, 300, d)), rand16(rng, (1, 2, 300, d)), rand16(rng, (1, 2, 300, d))
    zeros = W.pack_bits(np.zeros((5, 2), dtype=bool))
    for causal in (False, True):
        a = gpu_attn(A, q, k, v, 0.1, causal, route=zeros, tpb=4)
        b = gpu_attn(A, q, k, v, 0.1, causal)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("kg", ["1", "2", "nw8", "nw2"])
def test_gpu_varlen_equals_separate_calls(A, monkeypatch, kg):
    """Same tiling (fixed workgroup shape, no split over workgroups):
    bit-identical; default launch plans: within fp16 rounding."""
    rng = np.random.default_rng(64)
    lens = [70, 1, 129, 300]
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    q, k, v = rand16(rng, (8, T, 128)), rand16(rng, (2, T, 128)), rand16(rng, (2, T, 128))
    packed = gpu_attn(A, q, k, v, 0.1, True, cu=cu)
    monkeypatch.setenv("ATTN_KSPLIT", "1")
    if kg in ("nw8", "nw2"):
        monkeypatch.setenv("ATTN_QUERY_WAVES", kg[2])
    else:
        monkeypatch.setenv("ATTN_QUERY_WAVES", "4")
        monkeypatch.setenv("ATTN_KEY_GROUPS", kg)
    packed1 = gpu_attn(A, q, k, v, 0.1, True, cu=cu)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        one1 = gpu_attn(A, q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], 0.1, True)
        assert np.array_equal(packed1[:, a:b].view(np.uint16), one1[0].view(np.uint16))
        err = np.abs(packed[:, a:b].astype(np.float64) - one1[0].astype(np.float64))
        assert err.max() <= 2e-3


def test_gpu_bottom_right_is_tail_of_full(A):
    rng = np.random.default_rng(65)
    ksl = 600
    q, k, v = rand16(rng, (1, 4, ksl, 128)), rand16(rng, (1, 1, ksl, 128)), rand16(rng, (1, 1, ksl, 128))
    full = gpu_attn(A, q, k, v, 0.1, True)
    for qsl in (1, 100, 128, 333):
        tail = gpu_attn(A, q[:, :, ksl - qsl:], k, v, 0.1, True)
        err = np.abs(tail.astype(np.float64) - full[:, :, ksl - qsl:].astype(np.float64))
        assert err.max() <= 2e-3


@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("kexp", [-1, 2])
def test_gpu_power_of_two_scale_equivariance(A, routed, kexp):
    rng = np.random.default_rng(66)
    q, k, v = rand16(rng, (1, 4, 150, 64)), rand16(rng, (1, 2, 230, 64)), rand16(rng, (1, 2, 230, 64))
    route = W.pack_bits(rng.random((3, 4)) < 0.5) if routed else None
    a = gpu_attn(A, q, k, v, 0.125, True, route=route, tpb=1)
    q2 = (q.astype(np.float64) * 2.0 ** kexp).astype(np.float16)
    b = gpu_attn(A, q2, k, v, 0.125 * 2.0 ** -kexp, True, route=route, tpb=1)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


# --------------------------------------------------------------------------
# INT8 codes and routing decode, bit-exact
# --------------------------------------------------------------------------


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("path", [0, 1])
def test_gpu_quantizer_bitexact(A, orc, d, path):
    rng = np.random.default_rng(70 + d + path)
    rows = np.concatenate([
        rand16(rng, (200, d)),
        (rng.standard_normal((50, d)) * 1e-3).astype(np.float16),
        (rng.standard_normal((50, d)) * 3e3).astype(np.float16),
        np.zeros((3, d), dtype=np.float16),
    ])
    # rows whose codes sit on exact ties: amax 127 (inv 1) with half-integers
    tie = np.zeros((4, d), dtype=np.float16)
    tie[:, 0] = 127
    tie[:, 1:] = (np.arange(1, d) % 40 - 20 + 0.5).astype(np.float16)
    rows = np.ascontiguousarray(np.concatenate([rows, tie]))
    say("quantizer d=%d path=%d rows=%d" % (d, path, rows.shape[0]))
    q8, s = A.attn_debug_quantize_rows(dev(rows), path=path)
    q8, s = q8.cpu().numpy(), s.cpu().numpy()
    for r in range(rows.shape[0]):
        rq, rs = orc.quantize_row(rows[r])
        assert np.array_equal(q8[r], rq), r
        assert s[r] == rs, r


@pytest.mark.parametrize("causal", [False, True])
def test_gpu_route_dump_bitexact(A, orc, causal):
    rng = np.random.default_rng(80 + causal)
    for (qsl, ksl, tpb) in [(16384, 16384, 4), (512, 4096, 4), (100, 4000, 3), (64, 64, 1), (2100, 2100, 2)]:
        if causal and qsl > ksl:
            continue
        n_qt, n_kt = -(-qsl // 64), -(-ksl // 64)
        n_g = -(-n_kt // tpb)
        bits = rng.random((n_qt, n_g)) < 0.5
        words = W.pack_bits(bits)
        got = A.attn_debug_route_dump(words_tensor(words), qsl, ksl, causal, tpb).cpu().numpy()
        wpr = words.shape[1]
        off = ksl - qsl
        exp = np.zeros((n_qt, n_kt), dtype=np.uint8)
        for qt in range(n_qt):
            last = min(qt * 64 + 64, qsl) - 1
            for kt in range(n_kt):
                if causal and kt * 64 > last + off:
                    exp[qt, kt] = 2
                else:
                    exp[qt, kt] = orc.route_bit(words, wpr, qt, kt // tpb)
        assert np.array_equal(got, exp), (qsl, ksl, tpb)


def test_gpu_single_bit_flip_changes_only_its_qtile(A, orc):
    """Adversarial K (one large entry per row) makes INT8 scores differ from FP16
    by far more than the tolerance, so every routed bit is visible."""
    rng = np.random.default_rng(90)
    qsl = ksl = 256
    q = rand16(rng, (1, 4, qsl, 64))
    k = (rng.standard_normal((1, 1, ksl, 64)) * 0.05).astype(np.float16)
    k[..., 0] = 60.0
    v = rand16(rng, (1, 1, ksl, 64))
    base_bits = np.zeros((4, 4), dtype=bool)
    base = gpu_attn(A, q, k, v, 0.125, False, route=W.pack_bits(base_bits), tpb=1)
    for (qt, g) in [(0, 0), (1, 3), (3, 2)]:
        bits = base_bits.copy()
        bits[qt, g] = True
        got = gpu_attn(A, q, k, v, 0.125, False, route=W.pack_bits(bits), tpb=1)
        changed = np.nonzero(np.any(got != base, axis=(0, 1, 3)))[0]
        assert changed.size > 0 and changed.min() >= 64 * qt and changed.max() < 64 * (qt + 1)
        ref = orc.attn_fwd(q, k, v, scale=0.125, causal=False, route=W.pack_bits(bits), tiles_per_bit=1)
        check(got, ref)


# --------------------------------------------------------------------------
# the measured workloads at full size
# --------------------------------------------------------------------------


def sample_rows(rng, w, n_per_head):
    rows = []
    if w.varlen:
        for h in range(w.n_qh):
            for s, L in enumerate(w.seqlens):
                pick = {0, L - 1} | set(rng.integers(0, L, n_per_head).tolist())
                rows += [(s, h, int(i)) for i in sorted(pick)]
    else:
        for b in range(w.B):
            for h in range(w.n_qh):
                pick = {0, w.qsl - 1} | set(rng.integers(0, w.qsl, n_per_head).tolist())
                rows += [(b, h, int(i)) for i in sorted(pick)]
    return rows


def block_rows(rng, w):
    """One row (at a random position) in every 64-row query block of every
    head and sequence, plus each sequence's first and last row: every
    workgroup of the launch (a workgroup owns whole 64-row blocks of one
    head group, and every key split contributes to every row) writes at
    least one checked row."""
    rows = []
    seqs = list(enumerate(w.seqlens)) if w.varlen else [(b, w.qsl) for b in range(w.B)]
    for s, L in seqs:
        for h in range(w.n_qh):
            pick = {0, L - 1}
            for m0 in range(0, L, 64):
                pick.add(int(rng.integers(m0, min(m0 + 64, L))))
            rows += [(s, h, i) for i in sorted(pick)]
    return rows


def gather(out, rows, varlen, cu):
    if varlen:
        return np.stack([out[h, cu[s] + i] for (s, h, i) in rows])
    return np.stack([out[b, h, i] for (b, h, i) in rows])


# full oracle up to this many (query head, query, key) triples: the 256-token
# case, the 1024-token pair and the 512 x 4096 bottom-right case
FULL_ORACLE_PAIRS = 7.0e7


@pytest.mark.parametrize("name", [n for n, w in W.WORKLOADS.items() if not w.kv8 and w.lowp == "int8"])
def test_workload_full_size(A, orc, name):
    """The measured workloads at full size in the launch plan bench.py times:
    element by element against the whole oracle where it finishes in
    seconds, else on one row of every 64-row query block of every head."""
    w = W.WORKLOADS[name]
    say("workload", name)
    q, k, v = W.draw_qkv(w)
    route = W.route_for(w)
    cu = W.cu_seqlens_of(w.seqlens) if w.varlen else None
    got = gpu_attn(A, q, k, v, w.scale, w.causal, cu=cu, route=route, tpb=w.tiles_per_bit or 4)
    assert np.all(np.isfinite(got.astype(np.float32)))
    rng = np.random.default_rng(1234)
    if not w.varlen and w.B * w.n_qh * w.qsl * w.ksl <= FULL_ORACLE_PAIRS:
        ref = orc.attn_fwd(q, k, v, scale=w.scale, causal=w.causal, cu_seqlens=cu, route=route,
                           tiles_per_bit=w.tiles_per_bit or 4)
        mx, mn = check(got, ref, name)
        say("  all %d rows max %.3g mean %.3g" % (w.B * w.n_qh * w.qsl, mx, mn))
        return
    rows = block_rows(rng, w)
    ref = orc.attn_rows(q, k, v, rows, scale=w.scale, causal=w.causal, cu_seqlens=cu, route=route,
                        tiles_per_bit=w.tiles_per_bit or 4)
    mx, mn = check(gather(got, rows, w.varlen, cu), ref, name)
    say("  rows %d max %.3g mean %.3g" % (len(rows), mx, mn))
