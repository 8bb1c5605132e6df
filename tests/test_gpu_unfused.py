"""GPU parity of the unfused baseline (attn_fwd_unfused_stream: score GEMM,
masked softmax, P.V GEMM) against the CPU fp64 oracle, through the C ABI.
Same tolerance as the fused path: max abs error <= 4e-3, mean <= 5e-4."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import check, dev, gather, rand16, sample_rows, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_prefill_amd as A
    A.load()
    return A


def unfused(A, q, k, v, scale, causal):
    out = A.attn_fwd_unfused(dev(q), dev(k), dev(v), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return out.cpu().numpy()


SHAPES = [(1, 1), (5, 70), (64, 64), (65, 65), (130, 130), (200, 333), (333, 200), (300, 1000)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(3, 3), (8, 2), (8, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_gpu_unfused_ragged(A, orc, d, heads, causal):
    rng = np.random.default_rng(1700 + d + 10 * heads[0] + heads[1] + causal)
    for (qsl, ksl) in SHAPES:
        if causal and qsl > ksl:
            continue
        B = 2 if qsl <= 70 else 1
        say("unfused d=%d heads=%s causal=%d B=%d qsl=%d ksl=%d" % (d, heads, causal, B, qsl, ksl))
        q, k, v = rand16(rng, (B, heads[0], qsl, d)), rand16(rng, (B, heads[1], ksl, d)), \
            rand16(rng, (B, heads[1], ksl, d))
        scale = float(np.float32(1 / np.sqrt(d)))
        got = unfused(A, q, k, v, scale, causal)
        ref = orc.attn_fwd(q, k, v, scale=scale, causal=causal)
        check(got, ref, (qsl, ksl))


def test_gpu_unfused_negative_scale_and_fused_agreement(A, orc):
    rng = np.random.default_rng(1750)
    q, k, v = rand16(rng, (1, 4, 200, 64)), rand16(rng, (1, 2, 300, 64)), rand16(rng, (1, 2, 300, 64))
    for scale, causal in ((-0.125, False), (0.2, True)):
        got = unfused(A, q, k, v, scale, causal)
        check(got, orc.attn_fwd(q, k, v, scale=scale, causal=causal))
        fused = A.attn_fwd(dev(q), dev(k), dev(v), scale=scale, causal=causal).cpu().numpy()
        assert np.max(np.abs(fused.astype(np.float64) - got.astype(np.float64))) <= 4e-3


@pytest.mark.parametrize("name", ["dense_1024_d64", "dense_1024_d64_causal", "bottomright_512x4096_d128"])
def test_gpu_unfused_workload(A, orc, name):
    w = W.WORKLOADS[name]
    say("unfused workload", name)
    q, k, v = W.draw_qkv(w)
    got = unfused(A, q, k, v, w.scale, w.causal)
    rows = sample_rows(np.random.default_rng(1234), w, 6)
    ref = orc.attn_rows(q, k, v, rows, scale=w.scale, causal=w.causal)
    check(gather(got, rows, False, None), ref, name)
