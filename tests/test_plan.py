"""Host logic of the launch planner, on the CPU (no device needed): the
workgroup shape, grid and key splits that the forward entry points choose,
read through the attn_debug_plan test hook.

Invariants checked on every plan of a sweep of shapes and call kinds:
- the shape is one that the kernel dispatch instantiates (wavefronts 2, 4
  or 8; key groups 1 or 2; the kinds of call each shape serves);
- heads per workgroup divide the head group and the wavefronts; rows per
  workgroup = 32 x wavefronts / heads;
- a routed workgroup stays inside one 64-row query tile (the bitmask has one
  row per query tile);
- the row blocks cover every query row and the grid is columns x splits x
  blocks;
- a key split keeps at least 8 key tiles per split;
- the light-first pairing appears only where it is meant to.
With no device visible the planner takes 256 CUs, MI355X's count.
"""
import itertools
import math

import pytest

HEADS = [(1, 1), (4, 4), (32, 32), (8, 2), (32, 8), (12, 3), (6, 2), (32, 1), (3, 3)]
LENS = [(1, 1), (63, 63), (64, 64), (65, 200), (256, 256), (1000, 1000), (512, 4096), (4096, 4096),
        (16384, 16384), (1, 70000)]
KINDS = [dict(), dict(packed=True), dict(routed=True), dict(routed=True, packed=True), dict(kv8=True),
         dict(kv8=True, routed=True), dict(routed=True, fp8=True), dict(routed=True, fp8=True, packed=True)]


@pytest.fixture(scope="module")
def A():
    import attention_prefill_amd as A
    A.load()
    return A


def valid_shape(nw, ks, routed, kv8, fp8, hd):
    """The (wavefronts, key groups) shapes the dispatch instantiates for this kind of call."""
    if fp8 and (not routed or kv8):
        return False
    if ks == 2:
        return not routed and not kv8 and nw in (2, 4)
    if nw == 2:
        return routed
    return nw in (4, 8)


def check_plan(pl, B, qsl, ksl, hd, nqh, nkvh, causal, packed=False, routed=False, kv8=False, fp8=False):
    G = nqh // nkvh
    nw, ks, hpw, bm = pl["query_waves"], pl["key_groups"], pl["heads_per_wg"], pl["rows_per_wg"]
    assert valid_shape(nw, ks, routed, kv8, fp8, hd), pl
    assert hpw in (1, 2, 4) and G % hpw == 0 and nw % hpw == 0, pl
    assert bm == (nw // hpw) * 32, pl
    if routed:
        assert ks == 1 and 64 % bm == 0, pl
    assert pl["columns"] == (1 if packed else B) * nkvh * (G // hpw), pl
    if packed:
        lens = [qsl // B] * B          # the planner only sees the total; any split into B lengths fits
        lens[-1] += qsl - sum(lens)
        assert pl["row_blocks"] >= sum(math.ceil(L / bm) for L in lens), pl
    else:
        assert pl["row_blocks"] * bm >= qsl and (pl["row_blocks"] - 1) * bm < qsl, pl
    assert 1 <= pl["key_splits"] <= 8, pl
    n_kt = math.ceil(ksl / 64)
    assert pl["key_splits"] == 1 or n_kt >= 8 * pl["key_splits"], pl
    assert pl["grid"] == pl["columns"] * pl["key_splits"] * pl["row_blocks"], pl
    assert 0 < pl["grid"] < 2 ** 31, pl
    if pl["pair_blocks"]:
        assert causal and not packed and nw == 2 and ks == 2 and pl["key_splits"] == 1, pl
        assert pl["grid"] == 2 * 256 and pl["row_blocks"] % 2 == 0, pl
    if (routed and not kv8) or pl["key_splits"] > 1:
        assert pl["scratch_bytes"] > 0, pl


def test_plan_invariants_sweep(A):
    n = 0
    for (nqh, nkvh), (qsl, ksl), hd, causal, kind in itertools.product(HEADS, LENS, (64, 128), (False, True), KINDS):
        if causal and qsl > ksl:
            continue
        if kind.get("packed") and qsl != ksl:
            continue
        for B in ((1, 3) if kind.get("packed") else (1, 2)):
            if kind.get("packed") and qsl < B:
                continue
            pl = A.attn_debug_plan(B, qsl, ksl, hd, nqh, nkvh, causal, 2, **kind)
            check_plan(pl, B, qsl, ksl, hd, nqh, nkvh, causal, **kind)
            n += 1
    assert n > 1000


@pytest.mark.parametrize("env", [{"ATTN_QUERY_WAVES": "2"}, {"ATTN_QUERY_WAVES": "4"}, {"ATTN_QUERY_WAVES": "8"},
                                 {"ATTN_KEY_GROUPS": "1"}, {"ATTN_KEY_GROUPS": "2"}, {"ATTN_KSPLIT": "3"},
                                 {"ATTN_PAIR_BLOCKS": "1"}, {"ATTN_QUERY_WAVES": "9"}, {"ATTN_KSPLIT": "12"}])
def test_plan_overrides_stay_valid(A, monkeypatch, env):
    """The launch-shape overrides (test and tuning hooks) never produce a
    shape the dispatch lacks; values out of range are ignored."""
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    for (nqh, nkvh), (qsl, ksl), hd, causal, kind in itertools.product(
            [(4, 4), (8, 2), (12, 3), (32, 1)], [(64, 64), (300, 1000), (4096, 4096)], (64, 128), (False, True),
            KINDS[:7]):
        if kind.get("packed") and qsl != ksl:
            continue
        pl = A.attn_debug_plan(1, qsl, ksl, hd, nqh, nkvh, causal, 1, **kind)
        G = nqh // nkvh
        nw, ks = pl["query_waves"], pl["key_groups"]
        assert valid_shape(nw, ks, kind.get("routed", False), kind.get("kv8", False), kind.get("fp8", False), hd), \
            (env, kind, pl)
        assert G % pl["heads_per_wg"] == 0 and nw % pl["heads_per_wg"] == 0
        if kind.get("routed"):
            assert 64 % pl["rows_per_wg"] == 0
        if env.get("ATTN_KSPLIT") == "3":
            assert pl["key_splits"] == 3
        if env.get("ATTN_KSPLIT") == "12":
            assert pl["key_splits"] <= 8
        if env.get("ATTN_QUERY_WAVES") == "8" and not kind.get("routed"):
            assert nw == 8
        if env.get("ATTN_QUERY_WAVES") == "2" and not kind.get("routed") and not kind.get("kv8"):
            assert nw == 2 and ks == 2
        if env.get("ATTN_QUERY_WAVES") == "9":
            assert nw in (2, 4, 8)


@pytest.mark.parametrize("args,kind,expect", [
    # the default workload's two calls: two key groups; the causal call in
    # 64-row workgroups, two per CU, paired light-first
    ((1, 1024, 1024, 64, 32, 32, False), {}, dict(query_waves=4, key_groups=2, key_splits=1, grid=256)),
    ((1, 1024, 1024, 64, 32, 32, True), {}, dict(query_waves=2, key_groups=2, pair_blocks=1, grid=512)),
    # 256^2 with 4 heads: fewer workgroups than CUs
    ((1, 256, 256, 64, 4, 4, False), {}, dict(query_waves=2, key_groups=2)),
    # large grids: eight query wavefronts, four heads of 64 rows per workgroup
    ((1, 4096, 4096, 128, 32, 8, True), {}, dict(query_waves=8, key_groups=1, heads_per_wg=4, rows_per_wg=64)),
    ((1, 16384, 16384, 128, 32, 8, True), dict(routed=True), dict(query_waves=8, heads_per_wg=4, rows_per_wg=64)),
    ((1, 16384, 16384, 128, 32, 8, True), dict(routed=True, fp8=True), dict(query_waves=8, rows_per_wg=64)),
    ((1, 4096, 4096, 128, 32, 8, True), dict(kv8=True), dict(query_waves=8)),
    # short queries against long keys: key groups and a key split
    ((1, 512, 4096, 128, 32, 8, True), {}, dict(query_waves=4, key_groups=2, key_splits=2)),
    # routed calls: an odd head group takes two wavefronts, a group of two four
    ((1, 4096, 4096, 64, 32, 32, True), dict(routed=True), dict(query_waves=2, heads_per_wg=1, rows_per_wg=64)),
    ((1, 4096, 4096, 64, 16, 8, True), dict(routed=True), dict(query_waves=4, heads_per_wg=2, rows_per_wg=64)),
    # hdim 128 never takes the two-wavefront, two-group shape on its own
    ((1, 1024, 1024, 128, 32, 32, True), {}, dict(query_waves=4, key_groups=2)),
])
def test_plan_choices(A, args, kind, expect):
    """The shapes chosen for the workloads whose timings decided the rules."""
    pl = A.attn_debug_plan(*args, 4, **kind)
    for k, v in expect.items():
        assert pl[k] == v, (k, pl)


def test_plan_rejects_bad_sizes_and_flags(A):
    with pytest.raises(A.AttnError):
        A.attn_debug_plan(1, 10, 5, 64, 4, 4, True)          # causal with qsl > ksl
    with pytest.raises(A.AttnError):
        A.attn_debug_plan(1, 64, 64, 96, 4, 4, False)        # hdim
    with pytest.raises(A.AttnError):
        A.attn_debug_plan(1, 64, 64, 64, 4, 4, False, 4, kv8=True, routed=True, fp8=True)   # FP8 on a cache
    lib = A.load()
    import ctypes
    out = (ctypes.c_int64 * 10)()
    assert lib.attn_debug_plan(1, 64, 64, 64, 4, 4, 0, 4, 16, out) != 0                     # unknown flag bit
    assert lib.attn_debug_plan(1, 64, 64, 64, 4, 4, 0, 4, 0, None) != 0                     # null output


def test_route_group_index_rule():
    """The route cursor finds a tile's routing group without a division:
    q = high 32 bits of t * floor((2^32 - 1) / d), plus one if (q + 1) * d <= t.
    The rule must equal t // d for every tile index 0 <= t < 2^31 and every
    tiles-per-bit d >= 1 (uint32 arithmetic, no overflow in (q + 1) * d)."""
    import random
    rng = random.Random(7)
    for d in list(range(1, 260)) + [1000, 4096, 65535, 65536, 1 << 20, (1 << 31) - 1]:
        rcp = 0xFFFFFFFF // d
        ts = list(range(0, 3000)) + [rng.randrange(0, 1 << 31) for _ in range(3000)] + \
            [(1 << 31) - 1, (1 << 31) - 2, d - 1, d, d + 1, 32 * d - 1, 32 * d]
        for t in (t for t in ts if t < (1 << 31)):
            q = (t * rcp) >> 32
            assert (q + 1) * d < (1 << 32)
            if (q + 1) * d <= t:
                q += 1
            assert q == t // d, (t, d)
