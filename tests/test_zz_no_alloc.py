"""The allocation-free entry point (attn_fwd_noalloc_stream) through the C
ABI against attn_fwd_lowp_stream on the same inputs: two calls in a row on
the shared static scratch, the second smaller than the first, for calls that
use that scratch (routed calls keep their quantised K rows there, split-key
calls their fp32 partials).  The two entry points run the same kernels in
the same launch plan, so the outputs are compared bit for bit, and each is
also checked against the oracle at the usual bar."""
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


def both(A, q, k, v, scale, causal, route, tpb, lowp, cu=None):
    """(noalloc output, lowp_stream output) as numpy fp16, same inputs."""
    dq, dk, dv = dev(q), dev(k), dev(v)
    rt = words_tensor(route)
    dcu = None if cu is None else dev(np.asarray(cu, dtype=np.int32))
    if cu is None:
        B, n_qh, qsl, d = q.shape
        n_kvh, ksl = k.shape[1], k.shape[2]
    else:
        n_qh, qsl, d = q.shape
        n_kvh, ksl = k.shape[0], k.shape[1]
        B = len(cu) - 1
    a = torch.full_like(dq, float("nan"))
    b = torch.full_like(dq, float("nan"))
    lp = {"int8": 0, "fp8": 1}[lowp]
    A.attn_fwd_noalloc_stream(dq, dk, dv, a, B, qsl, ksl, d, n_qh, n_kvh, scale, causal, dcu, rt, tpb, lp)
    A.attn_fwd_lowp_stream(dq, dk, dv, b, B, qsl, ksl, d, n_qh, n_kvh, scale, causal, dcu, rt, tpb, lp)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


CASES = [
    # (label, heads, qsl, ksl, d, causal, tpb or 0, lowp, ATTN_KSPLIT)
    ("routed int8, split 3", (8, 2), 300, 3000, 128, True, 4, "int8", "3"),
    ("routed fp8, split 2", (4, 1), 130, 1500, 64, False, 3, "fp8", "2"),
    ("dense, split 4", (8, 2), 200, 2100, 64, True, 0, "int8", "4"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gpu_noalloc_matches_allocating_entry_point(A, orc, monkeypatch, case):
    label, heads, qsl, ksl, d, causal, tpb, lowp, ks = case
    monkeypatch.setenv("ATTN_KSPLIT", ks)
    rng = np.random.default_rng(9900 + qsl + ksl)
    # the second call is smaller in every dimension
    for (nq, nk, B) in ((qsl, ksl, 2), (qsl // 2 + 1, ksl // 2 + 3, 1)):
        q = rand16(rng, (B, heads[0], nq, d))
        k, v = rand16(rng, (B, heads[1], nk, d)), rand16(rng, (B, heads[1], nk, d))
        route = W.pack_bits(rng.random((-(-nq // 64), W.n_route_groups(nk, tpb))) < 0.5) if tpb else None
        say("noalloc %s B=%d qsl=%d ksl=%d" % (label, B, nq, nk))
        a, b = both(A, q, k, v, 0.1, causal, route, tpb or 4, lowp)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), label
        ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, route=route, tiles_per_bit=tpb or 4, lowp=lowp)
        check(a, ref, label)


def test_gpu_noalloc_packed_then_smaller(A, orc, monkeypatch):
    """Packed routed batch, then a smaller packed batch, split keys."""
    monkeypatch.setenv("ATTN_KSPLIT", "2")
    rng = np.random.default_rng(9950)
    for lens in ([700, 1, 1300], [130, 64]):
        cu = W.cu_seqlens_of(lens)
        T = int(cu[-1])
        q, k, v = rand16(rng, (8, T, 128)), rand16(rng, (2, T, 128)), rand16(rng, (2, T, 128))
        rows = sum(-(-L // 64) for L in lens)
        route = W.pack_bits(rng.random((rows, W.n_route_groups(T, 2))) < 0.5)
        say("noalloc packed lens=%s" % (lens,))
        a, b = both(A, q, k, v, 0.1, True, route, 2, "int8", cu=cu)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
        ref = orc.attn_fwd(q, k, v, scale=0.1, causal=True, cu_seqlens=cu, route=route, tiles_per_bit=2)
        check(a, ref)
