"""The routing bitmask on the GPU, bit-exactly, through the forward kernel's
own routed loop, and tile loads that must not read past a tensor's end.

TileMix abstract: routing decisions are packed into compact bitmasks and
each tile group is dispatched through the FP16 or the INT8 score path.

* Visit trace (attn_debug_route_trace): the forward kernel counts, at every
  key tile each workgroup visits, one FP16 or one low-precision visit.  The
  expected counts come from the bitmask alone, decoded here with
  np.unpackbits (little bit order) and the causal legality rule: every
  visible tile is visited exactly once per workgroup column, on the route of
  its group's bit, and no other tile is visited.  Run at the geometry of the
  16384-token TileMix workload (4 tiles per bit, rows of two words, eight
  query wavefronts with four LDS stages), with key splits starting inside a
  group and inside a word, every routed workgroup shape, bottom-right
  causal masks and packed batches with stacked rows.
* Adversarial inputs: keys whose INT8 (or FP8) codes drop the component that
  the FP16 score sees, so the two routes give different scores (the INT8
  scores are exactly 0, the FP16 ones spread over several units) and values
  that are constant per key tile with a sign pattern, so a group taken on the
  wrong route moves the output far past the tolerance.  Compared element by
  element with the oracle at the same geometries.
* Tails: K and V (and cache scales) as views at the end of a larger buffer
  whose remainder is NaN; ragged key lengths.  Reads past the last key must
  return zeros, so the output stays finite and matches the oracle.
"""
import numpy as np
import pytest

import workloads as W
from route_inputs import ADV_SCALE, adversarial
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


def unpack_rows(words, n_g):
    """bits [rows, n_g] of uint32 rows, least significant bit first."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    b = np.unpackbits(w.view(np.uint8).reshape(w.shape[0], -1), axis=1, bitorder="little")
    return b[:, :n_g].astype(bool)


def expected_trace(words, tpb, causal, qsl, ksl, columns, bm, lens=None):
    """uint32 counts [rows, ceil(ksl/64)] that the trace must read: every
    workgroup (bm query rows of one 64-row query tile, one per workgroup
    column) visits each key tile that some of its rows can see, on the route
    of that tile's group bit."""
    n_kt_all = -(-ksl // 64)
    n_g_all = -(-n_kt_all // tpb)
    bits = unpack_rows(words, n_g_all)
    if lens is None:
        probs = [(0, qsl, ksl)]
    else:
        probs, r0 = [], 0
        for L in lens:
            if L > 0:
                probs.append((r0, L, L))
                r0 += -(-L // 64)
    assert 64 % bm == 0
    exp = np.zeros((bits.shape[0], n_kt_all), dtype=np.int64)
    for (r0, Lq, Lk) in probs:
        n_kt = -(-Lk // 64)
        for m0 in range(0, Lq, bm):
            qt = m0 // 64
            last = min(m0 + bm, Lq) - 1
            n_vis = min(n_kt, (last + Lk - Lq) // 64 + 1) if causal else n_kt
            for kt in range(n_vis):
                exp[r0 + qt, kt] += columns * (0x10000 if bits[r0 + qt, kt // tpb] else 1)
    return exp


SHAPES = {  # name: (heads, ATTN_QUERY_WAVES or None)
    "nw8": ((8, 2), "8"),     # four-head groups, eight query wavefronts, four LDS stages
    "nw4": ((8, 2), "4"),     # four-head groups, four query wavefronts
    "nw4g2": ((4, 2), None),  # two-head groups
    "nw2": ((3, 3), None),    # one-head groups: two query wavefronts
}


def plan_columns(A, B, qsl, ksl, d, heads, causal, tpb, packed, lowp):
    return A.attn_debug_plan(B, qsl, ksl, d, heads[0], heads[1], causal, tpb, packed=packed, routed=True,
                             fp8=(lowp == "fp8"))


def run_trace(A, monkeypatch, shape, ks, d, qsl, ksl, causal, tpb, lowp, seed, lens=None):
    heads, nw = SHAPES[shape]
    if nw:
        monkeypatch.setenv("ATTN_QUERY_WAVES", nw)
    else:
        monkeypatch.delenv("ATTN_QUERY_WAVES", raising=False)
    monkeypatch.setenv("ATTN_KSPLIT", str(ks))
    rng = np.random.default_rng(seed)
    if lens is None:
        B = 1
        q, k, v = rand16(rng, (1, heads[0], qsl, d)), rand16(rng, (1, heads[1], ksl, d)), \
            rand16(rng, (1, heads[1], ksl, d))
        rows = -(-qsl // 64)
        cu = None
    else:
        B = len(lens)
        cu = W.cu_seqlens_of(lens)
        T = int(cu[-1])
        qsl = ksl = T
        q, k, v = rand16(rng, (heads[0], T, d)), rand16(rng, (heads[1], T, d)), rand16(rng, (heads[1], T, d))
        rows = sum(-(-L // 64) for L in lens)
    words = W.pack_bits(rng.random((rows, W.n_route_groups(ksl, tpb))) < 0.5)
    pl = plan_columns(A, B, qsl, ksl, d, heads, causal, tpb, lens is not None, lowp)
    if nw:
        assert pl["query_waves"] == int(nw), pl
    assert pl["key_splits"] == ks, pl
    say("trace shape=%s splits=%d d=%d qsl=%d ksl=%d causal=%d tpb=%d lowp=%s lens=%s plan=%s"
        % (shape, ks, d, qsl, ksl, causal, tpb, lowp, lens, pl))
    out, trace = A.attn_debug_route_trace(
        dev(q), dev(k), dev(v), words_tensor(words), scale=0.1, causal=causal,
        cu_seqlens=None if cu is None else dev(np.asarray(cu, dtype=np.int32)), tiles_per_bit=tpb, lowp=lowp)
    torch.cuda.synchronize()
    got = trace.cpu().numpy()
    exp = expected_trace(words, tpb, causal, qsl, ksl, pl["columns"], pl["rows_per_wg"], lens)
    assert np.array_equal(got[:exp.shape[0]], exp), \
        "first mismatch at %s" % (np.argwhere(got[:exp.shape[0]] != exp)[:5].tolist(),)
    assert not got[exp.shape[0]:].any()
    return q, k, v, words, cu, out


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("ks", [1, 2, 3, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_gpu_route_trace_tilemix_geometry(A, monkeypatch, shape, ks, causal):
    """Rows of two words (33 groups of 4 tiles), a ragged last tile and a
    partial last group, 200 query rows against 8300 keys (bottom-right when
    causal); splits of 130 tiles into 2, 3 and 5 start inside groups and, at
    5 (splits of 26 tiles), inside the second word's range."""
    run_trace(A, monkeypatch, shape, ks, 128, 200, 8300, causal, 4, "int8", 9000 + ks + 7 * causal)


@pytest.mark.parametrize("lowp", ["int8", "fp8"])
@pytest.mark.parametrize("tpb", [1, 3, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_gpu_route_trace_square_causal(A, monkeypatch, lowp, tpb, d):
    """A 2112-token causal prefill (33 query tiles, diagonal groups cut by the
    mask), eight query wavefronts, two key splits."""
    run_trace(A, monkeypatch, "nw8", 2, d, 2112, 2112, True, tpb, lowp, 9100 + tpb + d)


@pytest.mark.parametrize("shape", ["nw8", "nw2"])
@pytest.mark.parametrize("causal", [False, True])
def test_gpu_route_trace_packed(A, monkeypatch, shape, causal):
    """Packed batch over 8192 tokens (rows of two words): each sequence reads
    its own stacked rows, including an empty sequence and a one-token one."""
    run_trace(A, monkeypatch, shape, 1, 128, 0, 0, causal, 4, "int8", 9200 + causal,
              lens=[4200, 0, 1, 64, 3999])


def test_gpu_route_trace_full_tilemix_workload(A, monkeypatch):
    """The 16384-token TileMix workload itself, in the launch plan bench.py
    times (no overrides): every visible tile of every query tile on its
    bit's route, once per workgroup column."""
    monkeypatch.delenv("ATTN_QUERY_WAVES", raising=False)
    monkeypatch.delenv("ATTN_KSPLIT", raising=False)
    w = W.WORKLOADS["tilemix_16384_d128_causal"]
    q, k, v = W.draw_qkv(w)
    words = W.route_for(w)
    pl = A.attn_debug_plan(1, w.qsl, w.ksl, w.hdim, w.n_qh, w.n_kvh, True, w.tiles_per_bit, routed=True)
    say("trace tilemix workload plan=%s" % (pl,))
    _, trace = A.attn_debug_route_trace(dev(q), dev(k), dev(v), words_tensor(words), scale=w.scale, causal=True,
                                        tiles_per_bit=w.tiles_per_bit)
    torch.cuda.synchronize()
    exp = expected_trace(words, w.tiles_per_bit, True, w.qsl, w.ksl, pl["columns"], pl["rows_per_wg"])
    assert np.array_equal(trace.cpu().numpy(), exp)


# --------------------------------------------------------------------------
# adversarial inputs: a misrouted group moves the output past the tolerance
# --------------------------------------------------------------------------


@pytest.mark.parametrize("shape", ["nw8", "nw4", "nw2"])
@pytest.mark.parametrize("ks", [1, 2, 3])
@pytest.mark.parametrize("lowp", ["int8", "fp8"])
def test_gpu_adversarial_tilemix_geometry(A, orc, monkeypatch, shape, ks, lowp):
    """200 query rows, 8300 keys, 4 tiles per bit (two-word rows), causal
    bottom-right, element by element against the oracle."""
    heads, nw = SHAPES[shape]
    if nw:
        monkeypatch.setenv("ATTN_QUERY_WAVES", nw)
    monkeypatch.setenv("ATTN_KSPLIT", str(ks))
    rng = np.random.default_rng(9400 + ks + 5 * (lowp == "fp8") + 11 * list(SHAPES).index(shape))
    d, qsl, ksl, tpb = 128, 200, 8300, 4
    q, k, v = adversarial(rng, heads, qsl, ksl, d, lowp)
    words = W.pack_bits(rng.random((-(-qsl // 64), W.n_route_groups(ksl, tpb))) < 0.5)
    say("adversarial shape=%s splits=%d lowp=%s" % (shape, ks, lowp))
    scale = ADV_SCALE[lowp]
    got = A.attn_fwd(dev(q), dev(k), dev(v), scale=scale, causal=True, route_bitmask=words_tensor(words),
                     tiles_per_bit=tpb, lowp=lowp)
    torch.cuda.synchronize()
    ref = orc.attn_fwd(q, k, v, scale=scale, causal=True, route=words, tiles_per_bit=tpb, lowp=lowp)
    check(got.cpu().numpy(), ref, (shape, ks, lowp))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tpb", [1, 3])
def test_gpu_adversarial_square_causal(A, orc, monkeypatch, d, tpb):
    """1100-token causal prefill, eight query wavefronts, two splits."""
    monkeypatch.setenv("ATTN_QUERY_WAVES", "8")
    monkeypatch.setenv("ATTN_KSPLIT", "2")
    rng = np.random.default_rng(9500 + d + tpb)
    q, k, v = adversarial(rng, (4, 1), 1100, 1100, d, "int8")
    words = W.pack_bits(rng.random((-(-1100 // 64), W.n_route_groups(1100, tpb))) < 0.5)
    got = A.attn_fwd(dev(q), dev(k), dev(v), scale=0.1, causal=True, route_bitmask=words_tensor(words),
                     tiles_per_bit=tpb)
    torch.cuda.synchronize()
    ref = orc.attn_fwd(q, k, v, scale=0.1, causal=True, route=words, tiles_per_bit=tpb)
    check(got.cpu().numpy(), ref, (d, tpb))


@pytest.mark.parametrize("shape", ["nw8", "nw2"])
@pytest.mark.parametrize("causal", [False, True])
def test_gpu_adversarial_packed(A, orc, monkeypatch, shape, causal):
    """Packed batch over 8300 tokens (two-word rows, stacked per sequence)."""
    heads, nw = {"nw8": ((4, 1), "8"), "nw2": ((2, 2), None)}[shape]
    if nw:
        monkeypatch.setenv("ATTN_QUERY_WAVES", nw)
    rng = np.random.default_rng(9600 + causal + 3 * (shape == "nw2"))
    lens = [4100, 1, 130, 4069]
    cu = W.cu_seqlens_of(lens)
    T = int(cu[-1])
    q, k, v = adversarial(rng, heads, 0, 0, 128, "int8", lens=lens)
    rows = sum(-(-L // 64) for L in lens)
    words = W.pack_bits(rng.random((rows, W.n_route_groups(T, 4))) < 0.5)
    say("adversarial packed shape=%s causal=%d" % (shape, causal))
    got = A.attn_fwd(dev(q), dev(k), dev(v), scale=0.0884, causal=causal,
                     cu_seqlens=dev(np.asarray(cu, dtype=np.int32)), route_bitmask=words_tensor(words),
                     tiles_per_bit=4)
    torch.cuda.synchronize()
    ref = orc.attn_fwd(q, k, v, scale=0.0884, causal=causal, cu_seqlens=cu, route=words, tiles_per_bit=4)
    check(got.cpu().numpy(), ref, (shape, causal))


# --------------------------------------------------------------------------
# reads past the end of K and V
# --------------------------------------------------------------------------


def nan_tailed(a, extra):
    """a copied into the front of a device buffer whose next `extra` elements
    are NaN (fp16) or the largest value (int8); returns the view."""
    flat = torch.from_numpy(np.ascontiguousarray(a)).reshape(-1)
    buf = torch.empty(flat.numel() + extra, dtype=flat.dtype, device="cuda")
    if flat.dtype in (torch.float16, torch.float32):
        buf.fill_(float("nan"))
    else:
        buf.fill_(127)
    buf[:flat.numel()].copy_(flat.cuda())
    return buf[:flat.numel()].view(a.shape)


SHAPE_ENV = {"kg1": {"ATTN_QUERY_WAVES": "4", "ATTN_KEY_GROUPS": "1"},
             "kg2": {"ATTN_QUERY_WAVES": "4", "ATTN_KEY_GROUPS": "2"},
             "nw8": {"ATTN_QUERY_WAVES": "8"}, "nw2": {"ATTN_QUERY_WAVES": "2"}}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("ksl", [200, 1500])
@pytest.mark.parametrize("shape", list(SHAPE_ENV))
@pytest.mark.parametrize("routed", [False, True])
def test_gpu_tail_reads_return_zero(A, orc, monkeypatch, d, ksl, shape, routed):
    """K and V end three tiles before a NaN region; every launch shape, ragged
    key lengths, causal (bottom-right) and not."""
    for kk, vv in SHAPE_ENV[shape].items():
        monkeypatch.setenv(kk, vv)
    rng = np.random.default_rng(9700 + d + ksl + 3 * routed + 7 * list(SHAPE_ENV).index(shape))
    heads = (8, 2)
    qsl = 100
    q, k, v = rand16(rng, (1, heads[0], qsl, d)), rand16(rng, (1, heads[1], ksl, d)), \
        rand16(rng, (1, heads[1], ksl, d))
    words = W.pack_bits(rng.random((2, W.n_route_groups(ksl, 3))) < 0.5) if routed else None
    dk, dv = nan_tailed(k, 3 * 64 * d), nan_tailed(v, 3 * 64 * d)
    for causal in (False, True):
        say("tail d=%d ksl=%d shape=%s routed=%d causal=%d" % (d, ksl, shape, routed, causal))
        got = A.attn_fwd(dev(q), dk, dv, scale=0.1, causal=causal, route_bitmask=words_tensor(words),
                         tiles_per_bit=3)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        assert np.all(np.isfinite(got.astype(np.float32)))
        ref = orc.attn_fwd(q, k, v, scale=0.1, causal=causal, route=words, tiles_per_bit=3)
        check(got, ref, (d, ksl, shape, routed, causal))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("routed", [False, True])
def test_gpu_tail_reads_return_zero_kv8(A, orc, monkeypatch, d, routed):
    """INT8 key/value cache whose codes end before a region of 127s and whose
    scales end before a NaN region; ragged keys, eight query wavefronts."""
    monkeypatch.setenv("ATTN_QUERY_WAVES", "8")
    rng = np.random.default_rng(9800 + d + routed)
    ksl = 1500
    q = rand16(rng, (1, 8, 100, d))
    k8, sk = orc.quantize_rows(rand16(rng, (1, 2, ksl, d)))
    v8, sv = orc.quantize_rows(rand16(rng, (1, 2, ksl, d)))
    words = W.pack_bits(rng.random((2, W.n_route_groups(ksl, 3))) < 0.5) if routed else None
    tail = 3 * 64 * d
    got = A.attn_fwd_kv8(dev(q), nan_tailed(k8, tail), nan_tailed(sk, 3 * 64), nan_tailed(v8, tail),
                         nan_tailed(sv, 3 * 64), scale=0.1, causal=False, route_bitmask=words_tensor(words),
                         tiles_per_bit=3)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.all(np.isfinite(got.astype(np.float32)))
    ref = orc.attn_fwd_kv8(q, k8, sk, v8, sv, scale=0.1, causal=False, route=words, tiles_per_bit=3)
    check(got, ref, (d, routed))
