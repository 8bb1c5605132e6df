"""Pins for the oracle's FP8 route (rowwise-scaled e4m3 score cells), checked
against things other than itself:

- torch's float8_e4m3fn type (a library): every bit pattern's value, and the
  rounding of fp32 values (one correctly rounded conversion) on a sweep that
  includes every e4m3 midpoint and the subnormal range;
- a numpy restatement of the rowwise quantiser and a numpy brute force of the
  attention with FP8 cells;
- bit-exact equality with the FP16 path on inputs that rowwise FP8 codes
  represent exactly.

Sources: "Add rowwise scaling to Float8Inference module" (pytorch-labs
float8_experimental issue 305): rowwise ("AxisWise") dynamic scaling; TileMix
abstract: per-tile-group score precision chosen by a routing bitmask.
"""
import numpy as np
import pytest

import workloads
from test_oracle_pins import np_bits, rand16

torch = pytest.importorskip("torch")


def torch_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_all_codes_vs_torch(orc):
    ref = torch_e4m3_values()
    for c in range(256):
        got = orc.e4m3_decode(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
    assert orc.e4m3_decode(0x7e) == 448.0 and orc.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_roundtrip(orc):
    for c in range(256):
        v = orc.e4m3_decode(c)
        if np.isnan(v):
            continue
        assert orc.e4m3_encode(v) == (0 if v == 0 else c), c


def test_e4m3_round_vs_torch_sweep(orc):
    vals = torch_e4m3_values()
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = (fin[:-1] + fin[1:]) / 2                        # every tie between neighbours
    rng = np.random.default_rng(2000)
    rand = np.concatenate([rng.uniform(-460, 460, 4000), rng.uniform(-0.02, 0.02, 2000),
                           rng.standard_normal(2000) * 30])
    sweep = np.concatenate([fin, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                            rand, [447.9, 448.0, 455.9, 463.9, 2.0 ** -10, 2.0 ** -10 * 3]])
    sweep = sweep.astype(np.float32)                       # fp32 inputs: torch rounds once
    ref = torch.from_numpy(sweep).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    for x, r in zip(sweep, ref):
        assert orc.e4m3_round(float(x)) == r, (float(x), r)


def np_e4m3_round(y):
    """Nearest e4m3 values of float64 y, ties to even (numpy restatement)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, E = np.frexp(a)
    e = np.maximum(E - 1, -6)
    q = np.ldexp(1.0, e - 3)
    r = np.minimum(np.rint(a / q) * q, 448.0)
    return np.where(a == 0, 0.0, np.sign(y) * r)


def np_quantize_fp8(x16):
    """Rowwise FP8 values (as float64) and fp32 scales, numpy only."""
    x32 = np.asarray(x16, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = (amax / np.float32(448)).astype(np.float32)
        inv = (np.float32(448) / amax).astype(np.float32)
    zero = amax == 0
    inv = np.where(zero, np.float32(0), inv)
    vals = np_e4m3_round(x32.astype(np.float64) * inv.astype(np.float64)[..., None])
    return vals, np.where(zero, np.float32(0), s).astype(np.float32)


def test_fp8_quantizer_vs_numpy(orc):
    rng = np.random.default_rng(2001)
    rows = [rand16(rng, (128,), sd=sd) for sd in (1e-3, 0.1, 1.0, 7.0, 300.0)]
    rows += [np.zeros(64, np.float16), np.full(64, np.float16(-3.0)),
             np.array([65504] + [1] * 63, dtype=np.float16), rand16(rng, (64,), sd=1e-6)]
    for x in rows:
        codes, s = orc.quantize_row_fp8(x)
        vals, rs = np_quantize_fp8(x[None])
        assert s == rs[0]
        got = np.array([orc.e4m3_decode(c) for c in codes])
        assert np.array_equal(got, vals[0])


def np_attention_one_fp8(q, k, v, scale, causal, route, tpb, tile_q, tile_k):
    Lq, Lk = q.shape[0], k.shape[0]
    sc = float(np.float32(scale))
    S = sc * (q.astype(np.float64) @ k.astype(np.float64).T)
    qv, sq = np_quantize_fp8(q)
    kv, sk = np_quantize_fp8(k)
    S8 = sc * sq.astype(np.float64)[:, None] * sk.astype(np.float64)[None, :] * (qv @ kv.T)
    n_qt = -(-Lq // tile_q)
    n_g = -(-(-(-Lk // tile_k)) // tpb)
    bits = np_bits(route, n_qt, n_g)
    cell = bits[(np.arange(Lq) // tile_q)[:, None], ((np.arange(Lk) // tile_k) // tpb)[None, :]]
    S = np.where(cell, S8, S)
    if causal:
        S = np.where(np.tril(np.ones((Lq, Lk), dtype=bool), k=Lk - Lq), S, -np.inf)
    e = np.exp(S - S.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)) @ v.astype(np.float64)


@pytest.mark.parametrize("tile", [(2, 2), (4, 2), (64, 64)])
@pytest.mark.parametrize("tpb", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_route_vs_bruteforce(orc, tile, tpb, causal):
    rng = np.random.default_rng(2100 + tile[0] + 7 * tile[1] + tpb + causal)
    qsl, ksl, d, G = 19, 23, 64, 2
    q, k, v = rand16(rng, (1, 4, qsl, d)), rand16(rng, (1, 2, ksl, d)), rand16(rng, (1, 2, ksl, d))
    route = workloads.pack_bits(rng.random((-(-qsl // tile[0]), workloads.n_route_groups(ksl, tpb, tile[1]))) < 0.5)
    got = orc.attn_fwd(q, k, v, scale=0.2, causal=causal, route=route, tiles_per_bit=tpb, tile_q=tile[0],
                       tile_k=tile[1], lowp="fp8")
    for h in range(4):
        ref = np_attention_one_fp8(q[0, h], k[0, h // G], v[0, h // G], 0.2, causal, route, tpb, tile[0], tile[1])
        assert np.max(np.abs(got[0, h] - ref)) <= 1e-12


def exact_fp8_rows(rng, shape):
    """fp16 rows that rowwise FP8 represents exactly: e4m3 values times 2^-6
    with a +-448 in every row (so the row's scale is exactly 2^-6)."""
    vals = torch_e4m3_values()
    fin = vals[np.isfinite(vals)]
    x = rng.choice(fin, size=shape)
    idx = rng.integers(0, shape[-1], size=shape[:-1])
    np.put_along_axis(x, idx[..., None], np.where(rng.random(shape[:-1]) < 0.5, 448.0, -448.0)[..., None], axis=-1)
    out = (x * 2.0 ** -6).astype(np.float16)
    assert np.array_equal(out.astype(np.float64), x * 2.0 ** -6)
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_exact_inputs_equal_fp16_path_bitexact(orc, causal):
    rng = np.random.default_rng(2200 + causal)
    q = exact_fp8_rows(rng, (1, 4, 70, 128))
    k = exact_fp8_rows(rng, (1, 2, 150, 128))
    v = rand16(rng, (1, 2, 150, 128))
    route = workloads.pack_bits(rng.random((2, workloads.n_route_groups(150, 1))) < 0.5)
    a = orc.attn_fwd(q, k, v, scale=0.01, causal=causal, route=route, tiles_per_bit=1, lowp="fp8")
    b = orc.attn_fwd(q, k, v, scale=0.01, causal=causal)
    assert np.array_equal(a, b)
    c = orc.attn_fwd(q, k, v, scale=0.01, causal=causal, route=route, tiles_per_bit=1, lowp="int8")
    assert not np.array_equal(c, b)          # the INT8 codes of the same rows are not exact


def test_fp8_zero_mask_is_dense_and_rows_entry(orc):
    rng = np.random.default_rng(2300)
    q, k, v = rand16(rng, (1, 4, 90, 64)), rand16(rng, (1, 2, 90, 64)), rand16(rng, (1, 2, 90, 64))
    zeros = workloads.pack_bits(np.zeros((2, 1), dtype=bool))
    a = orc.attn_fwd(q, k, v, scale=0.1, causal=True, route=zeros, lowp="fp8")
    assert np.array_equal(a, orc.attn_fwd(q, k, v, scale=0.1, causal=True))
    ones = workloads.pack_bits(np.ones((2, 1), dtype=bool))
    full = orc.attn_fwd(q, k, v, scale=0.1, causal=True, route=ones, lowp="fp8")
    rows = [(0, 0, 0), (0, 3, 89), (0, 1, 64)]
    got = orc.attn_rows(q, k, v, rows, scale=0.1, causal=True, route=ones, lowp="fp8")
    for n, (s, h, i) in enumerate(rows):
        assert np.array_equal(got[n], full[s, h, i])
    vone = np.ones_like(v)
    assert np.allclose(orc.attn_fwd(q, k, vone, scale=0.1, causal=True, route=ones, lowp="fp8"), 1.0, atol=1e-14)
