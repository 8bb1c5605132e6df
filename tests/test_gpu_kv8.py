"""GPU parity of the INT8 key/value cache path (attn_fwd_kv8) and its encoder
(attn_quantize_rows) against the CPU fp64 oracle, through the C ABI.

Caches are encoded on the CPU by the oracle's encoder (no input comes from
the HIP path).  Tolerance as for the fp16 path: max abs error <= 4e-3 and
mean abs error <= 5e-4 on fp16 outputs; the encoder is compared bit-exactly.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import MAX_ERR, MEAN_ERR, block_rows, check, dev, gather, rand16, say, words_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_prefill_amd as A
    A.load()
    return A


def gpu_kv8(A, q, k8, sk, v8, sv, scale, causal, cu=None, route=None, tpb=4):
    out = A.attn_fwd_kv8(dev(q), dev(k8), dev(sk), dev(v8), dev(sv), scale=scale, causal=causal,
                         cu_seqlens=None if cu is None else dev(np.asarray(cu, dtype=np.int32)),
                         route_bitmask=words_tensor(route), tiles_per_bit=tpb)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def encode(orc, k, v):
    k8, sk = orc.quantize_rows(k)
    v8, sv = orc.quantize_rows(v)
    return k8, sk, v8, sv


@pytest.mark.parametrize("d", [64, 128])
def test_gpu_cache_encoder_bitexact(A, orc, d):
    rng = np.random.default_rng(1100 + d)
    x = rand16(rng, (3, 7, 45, d))
    x = (x.astype(np.float32) * rng.uniform(0.01, 30.0, size=(3, 7, 45, 1))).astype(np.float16)
    x[0, 0, 0] = 0
    x[0, 0, 1] = np.float16(-2.0)
    x[2, 6, 44, :5] = np.float16(65504)
    q8, s = A.attn_quantize_rows(dev(x))
    torch.cuda.synchronize()
    r8, rs = orc.quantize_rows(x)
    assert np.array_equal(q8.cpu().numpy(), r8)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


SHAPES = [(1, 1), (5, 70), (64, 64), (65, 65), (130, 130), (200, 333), (333, 200), (300, 1000)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(3, 3), (8, 2), (8, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_gpu_kv8_dense_ragged(A, orc, d, heads, causal, waves8):
    rng = np.random.default_rng(1200 + d + 10 * heads[0] + heads[1] + causal)
    for (qsl, ksl) in SHAPES:
        if causal and qsl > ksl:
            continue
        B = 2 if qsl <= 70 else 1
        say("kv8 dense d=%d heads=%s causal=%d B=%d qsl=%d ksl=%d" % (d, heads, causal, B, qsl, ksl))
        q = rand16(rng, (B, heads[0], qsl, d))
        k8, sk, v8, sv = encode(orc, rand16(rng, (B, heads[1], ksl, d)), rand16(rng, (B, heads[1], ksl, d)))
        scale = float(np.float32(1 / np.sqrt(d)))
        got = gpu_kv8(A, q, k8, sk, v8, sv, scale, causal)
        ref = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=scale, causal=causal)
        check(got, ref, (qsl, ksl))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(4, 2), (12, 3)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tpb", [1, 3])
def test_gpu_kv8_routed_ragged(A, orc, d, heads, causal, tpb, waves8):
    rng = np.random.default_rng(1300 + d + 7 * heads[1] + causal + 13 * tpb)
    for (qsl, ksl) in [(64, 64), (130, 130), (200, 333), (300, 1000)]:
        if causal and qsl > ksl:
            continue
        say("kv8 routed d=%d heads=%s causal=%d tpb=%d qsl=%d ksl=%d" % (d, heads, causal, tpb, qsl, ksl))
        q = rand16(rng, (1, heads[0], qsl, d))
        k8, sk, v8, sv = encode(orc, rand16(rng, (1, heads[1], ksl, d)), rand16(rng, (1, heads[1], ksl, d)))
        route = W.pack_bits(rng.random((-(-qsl // 64), W.n_route_groups(ksl, tpb))) < 0.5)
        got = gpu_kv8(A, q, k8, sk, v8, sv, 0.1, causal, route=route, tpb=tpb)
        ref = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.1, causal=causal, route=route, tiles_per_bit=tpb)
        check(got, ref, (qsl, ksl))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_gpu_kv8_varlen_ragged(A, orc, d, routed, causal, waves8):
    rng = np.random.default_rng(1400 + d + routed + 2 * causal)
    lens = [1, 63, 64, 65, 200, 0, 130, 7]
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    q = rand16(rng, (8, T, d))
    k8, sk, v8, sv = encode(orc, rand16(rng, (2, T, d)), rand16(rng, (2, T, d)))
    route = None
    if routed:
        n_rows = sum(-(-L // 64) for L in lens)
        route = W.pack_bits(rng.random((n_rows, W.n_route_groups(T, 1))) < 0.5)
    say("kv8 varlen d=%d routed=%d causal=%d" % (d, routed, causal))
    got = gpu_kv8(A, q, k8, sk, v8, sv, 0.1, causal, cu=cu, route=route, tpb=1)
    ref = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.1, causal=causal, cu_seqlens=cu, route=route,
                           tiles_per_bit=1)
    check(got, ref)


def test_gpu_kv8_all_int8_and_zero_rows(A, orc):
    """Every group INT8, with zero K and V rows (scale 0) in the cache."""
    rng = np.random.default_rng(1500)
    q = rand16(rng, (1, 4, 300, 128))
    k = rand16(rng, (1, 1, 300, 128))
    v = rand16(rng, (1, 1, 300, 128))
    k[0, 0, 17] = 0
    v[0, 0, 5] = 0
    v[0, 0, 250] = 0
    k8, sk, v8, sv = encode(orc, k, v)
    route = W.pack_bits(np.ones((5, 5), dtype=bool))
    for causal in (False, True):
        got = gpu_kv8(A, q, k8, sk, v8, sv, 0.09, causal, route=route, tpb=1)
        ref = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.09, causal=causal, route=route, tiles_per_bit=1)
        check(got, ref)


@pytest.mark.parametrize("routed", [False, True])
def test_gpu_kv8_split_keys(A, orc, monkeypatch, routed):
    """Key range split over workgroups (partials and merge) on the cache path,
    with and without a bitmask (routed splits walk each route's tiles from
    their own start)."""
    rng = np.random.default_rng(1600 + routed)
    q = rand16(rng, (1, 8, 100, 128))
    k8, sk, v8, sv = encode(orc, rand16(rng, (1, 2, 2000, 128)), rand16(rng, (1, 2, 2000, 128)))
    route = W.pack_bits(rng.random((2, W.n_route_groups(2000, 1))) < 0.5) if routed else None
    ref = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.1, causal=True, route=route, tiles_per_bit=1)
    for ks in ("1", "3", "4"):
        monkeypatch.setenv("ATTN_KSPLIT", ks)
        check(gpu_kv8(A, q, k8, sk, v8, sv, 0.1, True, route=route, tpb=1), ref, ks)


@pytest.mark.parametrize("name", [n for n, w in W.WORKLOADS.items() if w.kv8])
def test_kv8_workload_full_size(A, orc, name):
    w = W.WORKLOADS[name]
    say("workload", name)
    q, k, v = W.draw_qkv(w)
    k8, sk, v8, sv = encode(orc, k, v)
    del k, v
    route = W.route_for(w)
    cu = W.cu_seqlens_of(w.seqlens) if w.varlen else None
    got = gpu_kv8(A, q, k8, sk, v8, sv, w.scale, w.causal, cu=cu, route=route, tpb=w.tiles_per_bit or 4)
    rows = block_rows(np.random.default_rng(1234), w)
    ref = orc.attn_rows_kv8(q, k8, sk, v8, sv, rows, scale=w.scale, causal=w.causal, cu_seqlens=cu, route=route,
                            tiles_per_bit=w.tiles_per_bit or 4)
    mx, mn = check(gather(got, rows, w.varlen, cu), ref, name)
    say("  rows %d max %.3g mean %.3g (bar %.0e / %.0e)" % (len(rows), mx, mn, MAX_ERR, MEAN_ERR))
    assert np.all(np.isfinite(got.astype(np.float32)))


@pytest.mark.parametrize("vmul", [1e-3, 1e4])
@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_gpu_kv8_value_magnitudes(A, orc, vmul, routed, d, waves8):
    """Value caches far from unit scale: values of order 1e-3 (their fp16
    probabilities times v_scale would be fp16 subnormals if the scales were
    applied as they are) and of order 1e4 with some rows at amax 6e4 (where
    p * v_scale would overflow fp16 while p reaches 2^8 between rescales).
    Checked relative to the value magnitude: |gpu - oracle| / vmul within the
    usual bar."""
    rng = np.random.default_rng(1700 + d + routed + int(np.log10(vmul)))
    qsl, ksl = 150, 700
    q = rand16(rng, (1, 8, qsl, d))
    k = rand16(rng, (1, 2, ksl, d))
    v = np.clip(rng.standard_normal((1, 2, ksl, d)) * vmul, -6.0e4, 6.0e4)
    if vmul > 1:
        v[0, :, ::37, 3] = 6.0e4          # rows at the top of the fp16 range
    v = v.astype(np.float16)
    k8, sk, v8, sv = encode(orc, k, v)
    route = W.pack_bits(rng.random((3, W.n_route_groups(ksl, 2))) < 0.5) if routed else None
    for causal in (False, True):
        say("kv8 magnitude vmul=%g d=%d routed=%d causal=%d" % (vmul, d, routed, causal))
        got = gpu_kv8(A, q, k8, sk, v8, sv, 0.1, causal, route=route, tpb=2)
        assert np.all(np.isfinite(got.astype(np.float32)))
        ref = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.1, causal=causal, route=route, tiles_per_bit=2)
        check(got.astype(np.float64) / vmul, ref / vmul, (vmul, causal))
