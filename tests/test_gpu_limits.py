"""GPU parity at the limits of the path, against the CPU fp64 oracle through
the C ABI: very long context, tensors above 2 GiB (64-bit offsets), and many
short packed sequences.  Large inputs are drawn on the device by torch's
seeded generator (plumbing; not the path under test) and the oracle sees the
slices of the sampled heads.  Tolerance as everywhere: max abs error <= 4e-3,
mean <= 5e-4."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import check, dev, rand16, say, words_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_prefill_amd as A
    A.load()
    return A


def device_normal(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.float16)


def sampled_check(orc, q, k, v, out, heads, rows, scale, causal, route=None, tpb=4, label=""):
    """Oracle rows (b=0, h, i) for each sampled head, on that head's slices."""
    G = q.shape[1] // k.shape[1]
    for h in heads:
        hk = h // G
        qh = q[:, h:h + 1].cpu().numpy()
        kh = k[:, hk:hk + 1].cpu().numpy()
        vh = v[:, hk:hk + 1].cpu().numpy()
        ref = orc.attn_rows(qh, kh, vh, [(0, 0, i) for i in rows], scale=scale, causal=causal, route=route,
                            tiles_per_bit=tpb)
        got = out[0, h, rows].cpu().numpy()
        mx, mn = check(got, ref, "%s head %d" % (label, h))
        say("  %s head %d rows %d max %.3g mean %.3g" % (label, h, len(rows), mx, mn))


def test_gpu_long_context_routed(A, orc):
    """131072 tokens, causal, GQA 4:1, TileMix bitmask (2048 query tiles x 512 groups)."""
    L, d = 131072, 128
    say("long context %d" % L)
    q, k, v = device_normal((1, 4, L, d), 11), device_normal((1, 1, L, d), 12), device_normal((1, 1, L, d), 13)
    route = W.draw_route(L, L, 4, 0.5, seed=14)
    out = A.attn_fwd(q, k, v, scale=0.088, causal=True, route_bitmask=words_tensor(route), tiles_per_bit=4)
    torch.cuda.synchronize()
    rng = np.random.default_rng(15)
    rows = sorted({0, 1, 63, 64, L - 1} | set(rng.integers(0, L, 7).tolist()))
    sampled_check(orc, q, k, v, out, [0, 3], rows, 0.088, True, route=route, label="long")
    assert torch.isfinite(out.float()).all()


def test_gpu_over_2gib_tensors(A, orc):
    """q and out of 2.28 GB each (64 heads x 139301 x 128 fp16, a ragged length): row
    offsets past 2^31 bytes."""
    L, d = 139301, 128
    say("over 2 GiB: q [1, 64, %d, %d]" % (L, d))
    q = device_normal((1, 64, L, d), 21)
    k, v = device_normal((1, 8, L, d), 22), device_normal((1, 8, L, d), 23)
    assert q.numel() * 2 > 2 ** 31
    out = A.attn_fwd(q, k, v, scale=0.088, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(24)
    rows = sorted({0, L - 1} | set(rng.integers(0, L, 4).tolist()))
    sampled_check(orc, q, k, v, out, [0, 37, 63], rows, 0.088, True, label="2GiB")
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("routed", [False, True])
def test_gpu_many_short_sequences(A, orc, routed):
    """600 packed sequences of 1..300 tokens, causal, d64, GQA 4:1, full oracle."""
    rng = np.random.default_rng(31 + routed)
    lens = rng.integers(1, 301, 600).tolist()
    lens[5] = 0
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    say("many sequences: %d, T=%d routed=%d" % (len(lens), T, routed))
    q, k, v = rand16(rng, (4, T, 64)), rand16(rng, (1, T, 64)), rand16(rng, (1, T, 64))
    route = None
    if routed:
        n_rows = sum(-(-L // 64) for L in lens)
        route = W.pack_bits(rng.random((n_rows, W.n_route_groups(T, 1))) < 0.5)
    got = A.attn_fwd(dev(q), dev(k), dev(v), scale=0.125, causal=True, cu_seqlens=dev(np.asarray(cu, np.int32)),
                     route_bitmask=words_tensor(route), tiles_per_bit=1)
    torch.cuda.synchronize()
    ref = orc.attn_fwd(q, k, v, scale=0.125, causal=True, cu_seqlens=cu, route=route, tiles_per_bit=1)
    check(got.cpu().numpy(), ref, "many")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("qsl", [1, 7])
@pytest.mark.parametrize("routed", [False, True])
def test_gpu_few_queries_long_keys(A, orc, d, qsl, routed):
    """A few query rows against 70000 keys (bottom-right causal: every row
    sees nearly all of them): the key range is split over the most
    workgroups and merged; full oracle."""
    rng = np.random.default_rng(5000 + d + qsl + 3 * routed)
    L = 70000
    say("few queries: qsl=%d ksl=%d d=%d routed=%d" % (qsl, L, d, routed))
    q, k, v = rand16(rng, (1, 8, qsl, d)), rand16(rng, (1, 2, L, d)), rand16(rng, (1, 2, L, d))
    route = W.pack_bits(rng.random((1, W.n_route_groups(L, 2))) < 0.5) if routed else None
    got = A.attn_fwd(dev(q), dev(k), dev(v), scale=0.1, causal=True, route_bitmask=words_tensor(route),
                     tiles_per_bit=2)
    torch.cuda.synchronize()
    ref = orc.attn_fwd(q, k, v, scale=0.1, causal=True, route=route, tiles_per_bit=2)
    check(got.cpu().numpy(), ref, (qsl, d, routed))
