"""GPU parity of the FP8 route (attn_fwd_lowp_stream with ATTN_LOWP_FP8_E4M3:
rowwise-scaled e4m3 scores on the groups whose routing bit is set) and of its
two quantisers against the CPU fp64 oracle, through the C ABI.  The e4m3
codes and scales are compared bit-exactly; outputs to max abs error <= 4e-3,
mean <= 5e-4."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import block_rows, check, dev, gather, rand16, say, words_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_prefill_amd as A
    A.load()
    return A


def gpu_fp8(A, q, k, v, scale, causal, cu=None, route=None, tpb=4):
    out = A.attn_fwd(dev(q), dev(k), dev(v), scale=scale, causal=causal,
                     cu_seqlens=None if cu is None else dev(np.asarray(cu, dtype=np.int32)),
                     route_bitmask=words_tensor(route), tiles_per_bit=tpb, lowp="fp8")
    torch.cuda.synchronize()
    return out.cpu().numpy()


def e4m3_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("path", [2, 3])
def test_gpu_fp8_quantizer_bitexact(A, orc, d, path):
    rng = np.random.default_rng(1800 + d + path)
    rows = 96
    x = rand16(rng, (rows, d))
    x = (x.astype(np.float32) * rng.choice([1e-5, 1e-3, 0.05, 1.0, 9.0, 700.0], size=(rows, 1))).astype(np.float16)
    x[0] = 0
    x[1] = np.float16(0.25)
    # rows of exact e4m3 values (with a +-448): every code lands on a table entry
    tab = e4m3_table()
    fin = tab[np.isfinite(tab)]
    for r in range(2, 10):
        vals = rng.choice(fin, size=d)
        vals[rng.integers(d)] = 448.0
        x[r] = (vals * 2.0 ** -(r + 2)).astype(np.float16)
    q8, s = A.attn_debug_quantize_rows(dev(x), path=path)
    torch.cuda.synchronize()
    got_c = q8.cpu().numpy().view(np.uint8)
    got_s = s.cpu().numpy()
    for r in range(rows):
        rc, rs = orc.quantize_row_fp8(x[r])
        assert np.array_equal(got_c[r], rc), (r, got_c[r][:8], rc[:8])
        assert got_s[r].view(np.uint32) == np.float32(rs).view(np.uint32), r


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(3, 3), (8, 2), (12, 3)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tpb", [1, 3])
def test_gpu_fp8_routed_ragged(A, orc, d, heads, causal, tpb, waves8):
    rng = np.random.default_rng(1900 + d + 7 * heads[0] + heads[1] + causal + 13 * tpb)
    for (qsl, ksl) in [(1, 1), (64, 64), (130, 130), (200, 333), (300, 1000)]:
        if causal and qsl > ksl:
            continue
        say("fp8 routed d=%d heads=%s causal=%d tpb=%d qsl=%d ksl=%d" % (d, heads, causal, tpb, qsl, ksl))
        q, k, v = rand16(rng, (1, heads[0], qsl, d)), rand16(rng, (1, heads[1], ksl, d)), \
            rand16(rng, (1, heads[1], ksl, d))
        route = W.pack_bits(rng.random((-(-qsl // 64), W.n_route_groups(ksl, tpb))) < 0.5)
        got = gpu_fp8(A, q, k, v, 0.1, causal, route=route, tpb=tpb)
        ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, route=route, tiles_per_bit=tpb, lowp="fp8")
        check(got, ref, (qsl, ksl))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gpu_fp8_varlen_and_all_fp8(A, orc, d, causal, waves8):
    rng = np.random.default_rng(1950 + d + causal)
    lens = [1, 63, 64, 65, 200, 0, 130, 7]
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    q, k, v = rand16(rng, (8, T, d)), rand16(rng, (2, T, d)), rand16(rng, (2, T, d))
    n_rows = sum(-(-L // 64) for L in lens)
    for p in (0.5, 1.0):
        route = W.pack_bits(rng.random((n_rows, W.n_route_groups(T, 1))) < p)
        say("fp8 varlen d=%d causal=%d p=%.1f" % (d, causal, p))
        got = gpu_fp8(A, q, k, v, 0.1, causal, cu=cu, route=route, tpb=1)
        ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, cu_seqlens=cu, route=route, tiles_per_bit=1,
                           lowp="fp8")
        check(got, ref)


@pytest.mark.parametrize("waves", ["4", "8"])
def test_gpu_fp8_zero_mask_is_dense_bitexact(A, monkeypatch, waves):
    monkeypatch.setenv("ATTN_KEY_GROUPS", "1")
    monkeypatch.setenv("ATTN_QUERY_WAVES", waves)
    rng = np.random.default_rng(1990)
    q, k, v = rand16(rng, (1, 8, 300, 128)), rand16(rng, (1, 2, 300, 128)), rand16(rng, (1, 2, 300, 128))
    zeros = W.pack_bits(np.zeros((5, 2), dtype=bool))
    a = gpu_fp8(A, q, k, v, 0.1, True, route=zeros, tpb=4)
    b = A.attn_fwd(dev(q), dev(k), dev(v), scale=0.1, causal=True).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("name", [n for n, w in W.WORKLOADS.items() if w.lowp == "fp8"])
def test_fp8_workload_full_size(A, orc, name):
    w = W.WORKLOADS[name]
    say("workload", name)
    q, k, v = W.draw_qkv(w)
    route = W.route_for(w)
    got = gpu_fp8(A, q, k, v, w.scale, w.causal, route=route, tpb=w.tiles_per_bit)
    rows = block_rows(np.random.default_rng(1234), w)
    ref = orc.attn_rows(q, k, v, rows, scale=w.scale, causal=w.causal, route=route, tiles_per_bit=w.tiles_per_bit,
                        lowp="fp8")
    mx, mn = check(gather(got, rows, False, None), ref, name)
    say("  rows %d max %.3g mean %.3g" % (len(rows), mx, mn))
