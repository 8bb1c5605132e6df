"""ctypes binding of libattn_mi355x.so (include/attn.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  Tensors are torch CUDA (HIP) tensors; torch supplies device memory
and the current stream.  There is no fallback: if the library is not built,
or a call fails, an exception says so.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIB_PATH selects another build of the same library (for instance one
# compiled with a build-time alternative, for A/B timing)
LIB_PATH = os.environ.get("ATTN_LIB_PATH") or os.path.join(PKG, "libattn_mi355x.so")

ATTN_OK = 0
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
                4: "ATTN_ERR_ARG", 5: "ATTN_ERR_HIP"}

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


def load():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libattn_mi355x.so is not built (run __graft_entry__.build() or "
                               "python attention_prefill_amd/build.py)")
        lib = ctypes.CDLL(LIB_PATH)
        fwd_args = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I]
        lib.attn_fwd.argtypes = fwd_args
        lib.attn_fwd.restype = _I
        lib.attn_fwd_stream.argtypes = fwd_args + [_P]
        lib.attn_fwd_stream.restype = _I
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_abi_version.argtypes = []
        lib.attn_abi_version.restype = _I
        lib.attn_debug_quantize_rows.argtypes = [_P, _I, _I, _P, _P, _I, _P]
        lib.attn_debug_quantize_rows.restype = _I
        lib.attn_debug_route_dump.argtypes = [_P, _I, _I, _I, _I, _P, _P]
        lib.attn_debug_route_dump.restype = _I
        kv8_args = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I]
        lib.attn_fwd_kv8.argtypes = kv8_args
        lib.attn_fwd_kv8.restype = _I
        lib.attn_fwd_kv8_stream.argtypes = kv8_args + [_P]
        lib.attn_fwd_kv8_stream.restype = _I
        lib.attn_quantize_rows.argtypes = [_P, ctypes.c_int64, _I, _P, _P, _P]
        lib.attn_quantize_rows.restype = _I
        lib.attn_fwd_lowp_stream.argtypes = fwd_args + [_I, _P]
        lib.attn_fwd_lowp_stream.restype = _I
        lib.attn_fwd_unfused_stream.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]
        lib.attn_fwd_unfused_stream.restype = _I
        lib.attn_debug_plan.argtypes = [_I] * 9 + [ctypes.POINTER(ctypes.c_int64)]
        lib.attn_debug_plan.restype = _I
        lib.attn_debug_route_trace.argtypes = fwd_args + [_I, _P, ctypes.c_int64, _P]
        lib.attn_debug_route_trace.restype = _I
        lib.attn_debug_check_cu_seqlens.argtypes = [_P, _I, _I]
        lib.attn_debug_check_cu_seqlens.restype = _I
        lib.attn_fwd_noalloc_stream.argtypes = fwd_args + [_I, _P]
        lib.attn_fwd_noalloc_stream.restype = _I
        _lib = lib
    return _lib


def attn_last_error() -> str:
    return load().attn_last_error().decode()


def attn_abi_version() -> int:
    return load().attn_abi_version()


def _check(status):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def attn_fwd_stream(q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal,
                    cu_seqlens=None, route_bitmask=None, tiles_per_bit=4, stream=None):
    """Direct mirror of the C entry point (sizes passed explicitly)."""
    _check(load().attn_fwd_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, qsl, ksl, hdim, n_qh,
                                  n_kvh, float(scale), int(bool(causal)), _ptr(cu_seqlens),
                                  _ptr(route_bitmask), int(tiles_per_bit), _stream(stream)))


def _shapes(q, k, cu_seqlens):
    import torch
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("dense q/k/v must be 4-D [B, H, S, d]")
        B, n_qh, qsl, d = q.shape
        Bk, n_kvh, ksl, dk = k.shape
        if Bk != B:
            raise ValueError("q and k batch sizes differ")
    else:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("packed q/k/v must be 3-D [H, T, d]")
        n_qh, qsl, d = q.shape
        n_kvh, ksl, dk = k.shape
        B = cu_seqlens.numel() - 1
    if dk != d:
        raise ValueError("q and k head dims differ")
    return B, qsl, ksl, d, n_qh, n_kvh


def route_words_per_row(ksl, tiles_per_bit):
    """uint32 words per bitmask row: ceil(ceil(ceil(ksl / 64) / tiles_per_bit) / 32)."""
    n_g = -(-(-(-ksl // 64)) // tiles_per_bit)
    return -(-n_g // 32)


def _check_route_size(route_bitmask, qsl, ksl, tiles_per_bit, cu_seqlens):
    """The words the kernel reads (include/attn.h): ceil(qsl/64) rows dense;
    packed, one row per 64-row query tile of each sequence, at least
    ceil(T/64) rows (the exact count, from the lengths, under
    ATTN_DEBUG_VALIDATE=1, which reads cu_seqlens back from the device)."""
    if route_bitmask is None:
        return
    if int(tiles_per_bit) < 1:
        return      # the library reports ATTN_ERR_ARG
    wpr = route_words_per_row(ksl, int(tiles_per_bit))
    rows = -(-qsl // 64)
    if cu_seqlens is not None and os.environ.get("ATTN_DEBUG_VALIDATE") == "1":
        cu = cu_seqlens.cpu().tolist()
        rows = sum(-(-(b - a) // 64) for a, b in zip(cu[:-1], cu[1:]) if b > a)
    if route_bitmask.numel() < rows * wpr:
        raise ValueError("route_bitmask holds %d words; the kernel reads %d (%d rows of %d words)"
                         % (route_bitmask.numel(), rows * wpr, rows, wpr))


def _out_route(q, out, route_bitmask):
    import torch
    if route_bitmask is not None:
        if route_bitmask.dtype not in (torch.int32, torch.uint32):
            raise TypeError("route_bitmask must hold 32-bit words")
        _need(route_bitmask, "route_bitmask", route_bitmask.dtype)
    if out is None:
        return torch.empty_like(q)
    _need(out, "out", torch.float16)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return out


LOWP = {"int8": 0, "fp8": 1}


def attn_fwd(q, k, v, out=None, *, scale=None, causal=False, cu_seqlens=None,
             route_bitmask=None, tiles_per_bit=4, lowp="int8", stream=None):
    """Fused attention forward; sizes are read from the tensor shapes.

    dense:  q [B, n_qh, qsl, d], k/v [B, n_kvh, ksl, d]
    packed: q [n_qh, T, d], k/v [n_kvh, T, d], cu_seqlens int32 [B + 1]
    route_bitmask: int32 / uint32-valued tensor of packed routing words.
    lowp: what a set routing bit selects, "int8" or "fp8" (e4m3, rowwise scales).
    Returns out (allocated when None).  Enqueued on torch's current stream.
    """
    import torch
    _need(q, "q", torch.float16)
    _need(k, "k", torch.float16)
    _need(v, "v", torch.float16)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, qsl, ksl, d, n_qh, n_kvh = _shapes(q, k, cu_seqlens)
    out = _out_route(q, out, route_bitmask)
    _check_route_size(route_bitmask, qsl, ksl, tiles_per_bit, cu_seqlens)
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    if lowp == "int8":
        attn_fwd_stream(q, k, v, out, B, qsl, ksl, d, n_qh, n_kvh, scale, causal, cu_seqlens,
                        route_bitmask, tiles_per_bit, stream)
    else:
        attn_fwd_lowp_stream(q, k, v, out, B, qsl, ksl, d, n_qh, n_kvh, scale, causal, cu_seqlens,
                             route_bitmask, tiles_per_bit, LOWP[lowp], stream)
    return out


def attn_fwd_lowp_stream(q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal,
                         cu_seqlens=None, route_bitmask=None, tiles_per_bit=4, lowp_format=0, stream=None):
    """Direct mirror of the C entry point (sizes passed explicitly)."""
    _check(load().attn_fwd_lowp_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, qsl, ksl, hdim, n_qh,
                                       n_kvh, float(scale), int(bool(causal)), _ptr(cu_seqlens),
                                       _ptr(route_bitmask), int(tiles_per_bit), int(lowp_format),
                                       _stream(stream)))


def attn_fwd_noalloc_stream(q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal,
                            cu_seqlens=None, route_bitmask=None, tiles_per_bit=4, lowp_format=0, stream=None):
    """Direct mirror of the allocation-free C entry point (static device
    scratch, sizes passed explicitly)."""
    _check(load().attn_fwd_noalloc_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, qsl, ksl, hdim, n_qh,
                                          n_kvh, float(scale), int(bool(causal)), _ptr(cu_seqlens),
                                          _ptr(route_bitmask), int(tiles_per_bit), int(lowp_format),
                                          _stream(stream)))


def attn_debug_quantize_rows(x, path=0, stream=None):
    """(q8 int8 [rows, d], s float32 [rows]) from the device quantiser."""
    import torch
    _need(x, "x", torch.float16)
    rows, d = x.shape
    q8 = torch.empty((rows, d), dtype=torch.int8, device=x.device)
    s = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _check(load().attn_debug_quantize_rows(_ptr(x), rows, d, _ptr(q8), _ptr(s), int(path), _stream(stream)))
    return q8, s


def attn_debug_route_dump(route_bitmask, qsl, ksl, causal, tiles_per_bit, device="cuda", stream=None):
    """uint8 [ceil(qsl/64), ceil(ksl/64)]: 0 FP16, 1 INT8, 2 not visited."""
    import torch
    n_qt, n_kt = -(-qsl // 64), -(-ksl // 64)
    out = torch.empty((n_qt, n_kt), dtype=torch.uint8, device=device)
    _check(load().attn_debug_route_dump(_ptr(route_bitmask), qsl, ksl, int(bool(causal)),
                                        int(tiles_per_bit), _ptr(out), _stream(stream)))
    return out


def attn_debug_route_trace(q, k, v, route_bitmask, *, scale=None, causal=False, cu_seqlens=None,
                           tiles_per_bit=4, lowp="int8", stream=None):
    """(out, trace): a routed forward call that also records the tiles its
    workgroups visit.  trace is int64 [rows, ceil(ksl/64)] (rows = bitmask
    rows, packed: the bound ceil(T/64) + B): per tile, the number of FP16
    visits plus 0x10000 times the number of low-precision visits."""
    import torch
    _need(q, "q", torch.float16)
    _need(k, "k", torch.float16)
    _need(v, "v", torch.float16)
    B, qsl, ksl, d, n_qh, n_kvh = _shapes(q, k, cu_seqlens)
    out = _out_route(q, None, route_bitmask)
    _check_route_size(route_bitmask, qsl, ksl, tiles_per_bit, cu_seqlens)
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    n_kt = -(-ksl // 64)
    rows = -(-qsl // 64) + (B if cu_seqlens is not None else 0)
    trace = torch.empty((rows, n_kt), dtype=torch.int32, device=q.device)
    _check(load().attn_debug_route_trace(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, qsl, ksl, d, n_qh, n_kvh,
                                         float(scale), int(bool(causal)), _ptr(cu_seqlens), _ptr(route_bitmask),
                                         int(tiles_per_bit), LOWP[lowp], _ptr(trace), trace.numel(),
                                         _stream(stream)))
    return out, trace.to(torch.int64) & 0xffffffff


def attn_debug_check_cu_seqlens(cu_seqlens, T):
    """The ATTN_DEBUG_VALIDATE rule on a host int32 array (numpy); raises
    AttnError when it fails.  No device needed."""
    import numpy as np
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    _check(load().attn_debug_check_cu_seqlens(cu.ctypes.data_as(ctypes.c_void_p), int(cu.size - 1), int(T)))


def attn_fwd_kv8_stream(q, k8, k_scale, v8, v_scale, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal,
                        cu_seqlens=None, route_bitmask=None, tiles_per_bit=4, stream=None):
    """Direct mirror of the C entry point (sizes passed explicitly)."""
    _check(load().attn_fwd_kv8_stream(_ptr(q), _ptr(k8), _ptr(k_scale), _ptr(v8), _ptr(v_scale), _ptr(out),
                                      B, qsl, ksl, hdim, n_qh, n_kvh, float(scale), int(bool(causal)),
                                      _ptr(cu_seqlens), _ptr(route_bitmask), int(tiles_per_bit),
                                      _stream(stream)))


def attn_fwd_kv8(q, k8, k_scale, v8, v_scale, out=None, *, scale=None, causal=False, cu_seqlens=None,
                 route_bitmask=None, tiles_per_bit=4, stream=None):
    """Fused attention forward on an INT8 key/value cache.

    k8/v8: int8 codes in the layout of k/v; k_scale/v_scale: float32 per row
    ([B, n_kvh, ksl] dense, [n_kvh, T] packed); the keys and values are
    k_scale * k8 and v_scale * v8 (attn_quantize_rows makes such a cache).
    """
    import torch
    _need(q, "q", torch.float16)
    _need(k8, "k8", torch.int8)
    _need(v8, "v8", torch.int8)
    _need(k_scale, "k_scale", torch.float32)
    _need(v_scale, "v_scale", torch.float32)
    if k8.shape != v8.shape or k_scale.shape != v_scale.shape or tuple(k_scale.shape) != tuple(k8.shape[:-1]):
        raise ValueError("k8/v8 must share a shape and k_scale/v_scale must be its leading dims")
    B, qsl, ksl, d, n_qh, n_kvh = _shapes(q, k8, cu_seqlens)
    out = _out_route(q, out, route_bitmask)
    _check_route_size(route_bitmask, qsl, ksl, tiles_per_bit, cu_seqlens)
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    attn_fwd_kv8_stream(q, k8, k_scale, v8, v_scale, out, B, qsl, ksl, d, n_qh, n_kvh, scale, causal,
                        cu_seqlens, route_bitmask, tiles_per_bit, stream)
    return out


def attn_quantize_rows(x, stream=None):
    """(codes int8, scales float32 [leading dims]) of every last-axis row of an
    fp16 tensor: the INT8 key/value cache encoding, on the device."""
    import torch
    _need(x, "x", torch.float16)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    q8 = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    s = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(load().attn_quantize_rows(_ptr(x), rows, d, _ptr(q8), _ptr(s), _stream(stream)))
    return q8, s


def attn_fwd_unfused(q, k, v, out=None, *, scale=None, causal=False, stream=None):
    """The unfused baseline (score GEMM, masked softmax, P.V GEMM) on dense
    fp16 q [B, n_qh, qsl, d], k/v [B, n_kvh, ksl, d]; same result as attn_fwd."""
    import torch
    _need(q, "q", torch.float16)
    _need(k, "k", torch.float16)
    _need(v, "v", torch.float16)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, qsl, ksl, d, n_qh, n_kvh = _shapes(q, k, None)
    out = _out_route(q, out, None)
    if scale is None:
        scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    _check(load().attn_fwd_unfused_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, qsl, ksl, d, n_qh, n_kvh,
                                          float(scale), int(bool(causal)), _stream(stream)))
    return out


PLAN_FIELDS = ("query_waves", "key_groups", "heads_per_wg", "rows_per_wg", "columns", "row_blocks",
               "key_splits", "pair_blocks", "grid", "scratch_bytes")


def attn_debug_plan(B, qsl, ksl, hdim, n_qh, n_kvh, causal, tiles_per_bit=4, *, packed=False, routed=False,
                    kv8=False, fp8=False):
    """The launch plan the forward entry points would use for these sizes
    (test hook; no device needed): a dict of PLAN_FIELDS."""
    out = (ctypes.c_int64 * 10)()
    flags = int(bool(packed)) | (int(bool(routed)) << 1) | (int(bool(kv8)) << 2) | (int(bool(fp8)) << 3)
    _check(load().attn_debug_plan(B, qsl, ksl, hdim, n_qh, n_kvh, int(bool(causal)), int(tiles_per_bit), flags, out))
    return dict(zip(PLAN_FIELDS, (int(x) for x in out)))
