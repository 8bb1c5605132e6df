"""ctypes wrapper around liboracle.so, the CPU fp64 attention oracle.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module; the product path
(attention_prefill_amd) never does, and the two share no code.

All arrays are host numpy arrays; fp16 tensors are numpy float16.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB_PATH selects another build of oracle.c (the sanitizer
        # build of the CPU test run)
        path = os.environ.get("ORACLE_LIB_PATH")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build_oracle(force=False)
        lib = ctypes.CDLL(path)
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_f16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_quantize_row.argtypes = [_P, _I, _P, _P]
        lib.oracle_quantize_row.restype = None
        lib.oracle_quantize_rows.argtypes = [_P, ctypes.c_longlong, _I, _P, _P]
        lib.oracle_quantize_rows.restype = None
        lib.oracle_route_words_per_row.argtypes = [_I, _I, _I]
        lib.oracle_route_words_per_row.restype = _I
        lib.oracle_route_bit.argtypes = [_P, _I, _I, _I]
        lib.oracle_route_bit.restype = _I
        common = [_P, _P, _P]
        shape = [_I] * 6 + [ctypes.c_float, _I, _P, _P, _I, _I, _I]
        lib.oracle_attn_fwd.argtypes = common + [_P] + shape + [_I]
        lib.oracle_attn_fwd.restype = _I
        lib.oracle_attn_rows.argtypes = common + shape + [_P, _I, _P, _I]
        lib.oracle_attn_rows.restype = _I
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_round.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_round.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_quantize_row_fp8.argtypes = [_P, _I, _P, _P]
        lib.oracle_quantize_row_fp8.restype = None
        lib.oracle_attn_fwd_lowp.argtypes = common + [_P] + shape + [_I, _I]
        lib.oracle_attn_fwd_lowp.restype = _I
        lib.oracle_attn_rows_lowp.argtypes = common + shape + [_I, _P, _I, _P, _I]
        lib.oracle_attn_rows_lowp.restype = _I
        cache = [_P, _P, _P, _P, _P]
        lib.oracle_attn_fwd_kv8.argtypes = cache + [_P] + shape + [_I]
        lib.oracle_attn_fwd_kv8.restype = _I
        lib.oracle_attn_rows_kv8.argtypes = cache + shape + [_P, _I, _P, _I]
        lib.oracle_attn_rows_kv8.restype = _I
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _bits(a):
    a = np.ascontiguousarray(a, dtype=np.float16)
    return a.view(np.uint16)


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(int(bits))


def f64_to_f16_bits(x: float) -> int:
    return int(_load().oracle_f64_to_f16_rne(float(x)))


def round_f16(a: np.ndarray) -> np.ndarray:
    """fp16 round-to-nearest-even of a float64 array, by the oracle's encoder."""
    lib = _load()
    flat = np.asarray(a, dtype=np.float64).ravel()
    out = np.fromiter((lib.oracle_f64_to_f16_rne(float(x)) for x in flat), dtype=np.uint16,
                      count=flat.size)
    return out.view(np.float16).reshape(np.shape(a))


def quantize_row(x: np.ndarray):
    """(q8 int8[d], s float32) of one fp16 row."""
    xb = _bits(x)
    q8 = np.zeros(xb.shape[0], dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    _load().oracle_quantize_row(_ptr(xb), xb.shape[0], _ptr(q8), _ptr(s))
    return q8, np.float32(s[0])


def words_per_row(ksl: int, tile_k: int = 64, tiles_per_bit: int = 4) -> int:
    return _load().oracle_route_words_per_row(ksl, tile_k, tiles_per_bit)


def route_bit(words: np.ndarray, wpr: int, qt: int, g: int) -> int:
    w = np.ascontiguousarray(words, dtype=np.uint32)
    return _load().oracle_route_bit(_ptr(w), wpr, qt, g)


def _shape_args(q, k, cu_seqlens):
    if cu_seqlens is None:
        B, n_qh, qsl, d = q.shape
        Bk, n_kvh, ksl, dk = k.shape
        assert Bk == B and dk == d
    else:
        n_qh, T, d = q.shape
        n_kvh, Tk, dk = k.shape
        assert Tk == T and dk == d
        B = len(cu_seqlens) - 1
        qsl = ksl = T
    return B, qsl, ksl, d, n_qh, n_kvh


def _common(q, k, v, cu_seqlens, route):
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    assert kb.shape == vb.shape
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    rt = None if route is None else np.ascontiguousarray(route, dtype=np.uint32)
    return qb, kb, vb, cu, rt


_LOWP = {"int8": 0, "fp8": 1}


def attn_fwd(q, k, v, *, scale, causal=False, cu_seqlens=None, route=None,
             tiles_per_bit=4, tile_q=64, tile_k=64, lowp="int8", nthreads=0) -> np.ndarray:
    """The exact fp64 attention output, same shape as q.  lowp: the format a
    set routing bit selects ("int8", or "fp8" for e4m3 with rowwise scales)."""
    qb, kb, vb, cu, rt = _common(q, k, v, cu_seqlens, route)
    B, qsl, ksl, d, n_qh, n_kvh = _shape_args(qb, kb, cu)
    out = np.zeros(qb.shape, dtype=np.float64)
    rc = _load().oracle_attn_fwd_lowp(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(out), B, qsl, ksl, d, n_qh,
                                      n_kvh, float(np.float32(scale)), int(bool(causal)), _ptr(cu),
                                      _ptr(rt), int(tiles_per_bit), int(tile_q), int(tile_k),
                                      _LOWP[lowp], int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_fwd rejected its arguments (code %d)" % rc)
    return out


def attn_rows(q, k, v, rows, *, scale, causal=False, cu_seqlens=None, route=None,
              tiles_per_bit=4, tile_q=64, tile_k=64, lowp="int8", nthreads=0) -> np.ndarray:
    """Output rows for the (s, h, i) triples in rows, as float64 [len(rows), d]."""
    qb, kb, vb, cu, rt = _common(q, k, v, cu_seqlens, route)
    B, qsl, ksl, d, n_qh, n_kvh = _shape_args(qb, kb, cu)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    out = np.zeros((r.shape[0], d), dtype=np.float64)
    rc = _load().oracle_attn_rows_lowp(_ptr(qb), _ptr(kb), _ptr(vb), B, qsl, ksl, d, n_qh, n_kvh,
                                       float(np.float32(scale)), int(bool(causal)), _ptr(cu), _ptr(rt),
                                       int(tiles_per_bit), int(tile_q), int(tile_k), _LOWP[lowp], _ptr(r),
                                       r.shape[0], _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments (code %d)" % rc)
    return out


def quantize_rows(x: np.ndarray):
    """(codes int8, scales float32) of every last-axis row of an fp16 array:
    the INT8 key/value cache encoding (same rule as quantize_row)."""
    xb = _bits(x)
    d = xb.shape[-1]
    rows = xb.size // d
    q8 = np.zeros(xb.shape, dtype=np.int8)
    s = np.zeros(xb.shape[:-1], dtype=np.float32)
    _load().oracle_quantize_rows(_ptr(xb), rows, d, _ptr(q8), _ptr(s))
    return q8, s


def _cache(q, k8, k_scale, v8, v_scale, cu_seqlens, route):
    qb = _bits(q)
    k8 = np.ascontiguousarray(k8, dtype=np.int8)
    v8 = np.ascontiguousarray(v8, dtype=np.int8)
    ks = np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    assert k8.shape == v8.shape and ks.shape == vs.shape == k8.shape[:-1]
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    rt = None if route is None else np.ascontiguousarray(route, dtype=np.uint32)
    return qb, k8, ks, v8, vs, cu, rt


def attn_fwd_kv8(q, k8, k_scale, v8, v_scale, *, scale, causal=False, cu_seqlens=None, route=None,
                 tiles_per_bit=4, tile_q=64, tile_k=64, nthreads=0) -> np.ndarray:
    """Exact fp64 output with INT8 key/value cache inputs (K^ = k_scale * k8,
    V^ = v_scale * v8), same shape as q."""
    qb, k8, ks, v8, vs, cu, rt = _cache(q, k8, k_scale, v8, v_scale, cu_seqlens, route)
    B, qsl, ksl, d, n_qh, n_kvh = _shape_args(qb, k8, cu)
    out = np.zeros(qb.shape, dtype=np.float64)
    rc = _load().oracle_attn_fwd_kv8(_ptr(qb), _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs), _ptr(out),
                                     B, qsl, ksl, d, n_qh, n_kvh, float(np.float32(scale)),
                                     int(bool(causal)), _ptr(cu), _ptr(rt), int(tiles_per_bit),
                                     int(tile_q), int(tile_k), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_fwd_kv8 rejected its arguments (code %d)" % rc)
    return out


def attn_rows_kv8(q, k8, k_scale, v8, v_scale, rows, *, scale, causal=False, cu_seqlens=None,
                  route=None, tiles_per_bit=4, tile_q=64, tile_k=64, nthreads=0) -> np.ndarray:
    """attn_fwd_kv8 output rows for the (s, h, i) triples in rows, float64 [len(rows), d]."""
    qb, k8, ks, v8, vs, cu, rt = _cache(q, k8, k_scale, v8, v_scale, cu_seqlens, route)
    B, qsl, ksl, d, n_qh, n_kvh = _shape_args(qb, k8, cu)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    out = np.zeros((r.shape[0], d), dtype=np.float64)
    rc = _load().oracle_attn_rows_kv8(_ptr(qb), _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs), B, qsl, ksl,
                                      d, n_qh, n_kvh, float(np.float32(scale)), int(bool(causal)),
                                      _ptr(cu), _ptr(rt), int(tiles_per_bit), int(tile_q),
                                      int(tile_k), _ptr(r), r.shape[0], _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_rows_kv8 rejected its arguments (code %d)" % rc)
    return out


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_round(y: float) -> float:
    """The e4m3 value nearest to y (ties to even, zero results +0)."""
    return _load().oracle_e4m3_round(float(y))


def e4m3_encode(r: float) -> int:
    return int(_load().oracle_e4m3_encode(float(r)))


def quantize_row_fp8(x: np.ndarray):
    """(codes uint8[d] e4m3 bit patterns, s float32) of one fp16 row."""
    xb = _bits(x)
    c = np.zeros(xb.shape[0], dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    _load().oracle_quantize_row_fp8(_ptr(xb), xb.shape[0], _ptr(c), _ptr(s))
    return c, np.float32(s[0])
