"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/attn.h declares, and rejects bad arguments with the documented codes
before touching the device (every pointer below is a fake, never read)."""
import ctypes
import os
import re

import pytest

import attention_prefill_amd as A
from attention_prefill_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, UNSUP, ARG = 0, 1, 2, 3, 4
FAKE = 0x10000          # 16-byte aligned, never dereferenced on error paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ["attn_fwd", "attn_fwd_stream", "attn_last_error", "attn_abi_version",
              "attn_debug_quantize_rows", "attn_debug_route_dump", "attn_fwd_kv8", "attn_fwd_kv8_stream",
              "attn_quantize_rows", "attn_fwd_unfused_stream", "attn_fwd_lowp_stream", "attn_debug_plan",
              "attn_debug_route_trace", "attn_debug_check_cu_seqlens"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_abi_version():
    assert A.attn_abi_version() == 1


def call(q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=1, qsl=64, ksl=64, hdim=64, n_qh=4, n_kvh=2,
         scale=0.125, causal=0, cu=None, route=None, tpb=4):
    lib = A.load()
    return lib.attn_fwd(q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal, cu, route, tpb)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(out=None), NULL),
    (dict(B=0), SHAPE), (dict(qsl=0), SHAPE), (dict(ksl=-1), SHAPE), (dict(n_qh=0), SHAPE),
    (dict(n_kvh=0), SHAPE), (dict(n_qh=6, n_kvh=4), SHAPE),
    (dict(causal=1, qsl=65, ksl=64), SHAPE),
    (dict(cu=FAKE, qsl=64, ksl=63), SHAPE),
    (dict(hdim=96), UNSUP), (dict(hdim=256), UNSUP),
    (dict(scale=float("nan")), ARG), (dict(scale=float("inf")), ARG), (dict(scale=0.0), ARG),
    (dict(route=FAKE, tpb=0), ARG),
    (dict(q=FAKE + 8), ARG), (dict(out=FAKE + 2), ARG), (dict(route=FAKE + 2), ARG),
])
def test_validation_codes(kw, code):
    assert call(**kw) == code
    assert A.attn_last_error() != ""


def call_kv8(q=FAKE, k8=FAKE, ks=FAKE, v8=FAKE, vs=FAKE, out=FAKE, B=1, qsl=64, ksl=64, hdim=64, n_qh=4,
             n_kvh=2, scale=0.125, causal=0, cu=None, route=None, tpb=4):
    lib = A.load()
    return lib.attn_fwd_kv8(q, k8, ks, v8, vs, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal, cu, route, tpb)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k8=None), NULL), (dict(ks=None), NULL), (dict(v8=None), NULL),
    (dict(vs=None), NULL), (dict(out=None), NULL),
    (dict(qsl=0), SHAPE), (dict(n_qh=6, n_kvh=4), SHAPE), (dict(causal=1, qsl=65, ksl=64), SHAPE),
    (dict(ksl=20000000, hdim=128), SHAPE),
    (dict(hdim=96), UNSUP), (dict(scale=0.0), ARG), (dict(route=FAKE, tpb=0), ARG),
    (dict(k8=FAKE + 8), ARG), (dict(v8=FAKE + 4), ARG), (dict(ks=FAKE + 2), ARG), (dict(vs=FAKE + 1), ARG),
])
def test_kv8_validation_codes(kw, code):
    assert call_kv8(**kw) == code
    assert A.attn_last_error() != ""


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4, 2, 0.1, 0), NULL),
    ((FAKE, FAKE, FAKE, FAKE, 1, 65, 64, 64, 4, 2, 0.1, 1), SHAPE),
    ((FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 96, 4, 2, 0.1, 0), UNSUP),
    ((FAKE, FAKE, FAKE, FAKE, 64, 16384, 16384, 128, 32, 8, 0.1, 0), SHAPE),   # 3.3 TB of scores
    ((FAKE + 2, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4, 2, 0.1, 0), ARG),
])
def test_unfused_validation_codes(args, code):
    assert A.load().attn_fwd_unfused_stream(*args, None) == code
    assert A.attn_last_error() != ""


def test_lowp_format_validation():
    lib = A.load()
    args = (FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4, 2, 0.125, 0, None, FAKE, 4)
    assert lib.attn_fwd_lowp_stream(*args, 2, None) == ARG
    assert lib.attn_fwd_lowp_stream(*args, -1, None) == ARG
    assert "lowp" in A.attn_last_error()
    assert lib.attn_fwd_lowp_stream(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 96, 4, 2, 0.125, 0, None, FAKE, 4,
                                    1, None) == UNSUP
    assert lib.attn_debug_quantize_rows(FAKE, 4, 64, FAKE, FAKE, 4, None) == ARG


def test_cache_encoder_validates():
    lib = A.load()
    assert lib.attn_quantize_rows(None, 4, 64, FAKE, FAKE, None) == NULL
    assert lib.attn_quantize_rows(FAKE, -1, 64, FAKE, FAKE, None) == SHAPE
    assert lib.attn_quantize_rows(FAKE, 1 << 31, 64, FAKE, FAKE, None) == SHAPE
    assert lib.attn_quantize_rows(FAKE, 4, 80, FAKE, FAKE, None) == UNSUP
    assert lib.attn_quantize_rows(FAKE + 4, 4, 64, FAKE, FAKE, None) == ARG


def test_error_message_names_the_problem():
    assert call(hdim=80) == UNSUP
    assert "hdim" in A.attn_last_error()
    assert call(n_qh=5, n_kvh=2) == SHAPE
    assert "multiple" in A.attn_last_error()


def test_debug_hooks_validate():
    lib = A.load()
    assert lib.attn_debug_quantize_rows(None, 4, 64, FAKE, FAKE, 0, None) == NULL
    assert lib.attn_debug_quantize_rows(FAKE, 4, 96, FAKE, FAKE, 0, None) == UNSUP
    assert lib.attn_debug_quantize_rows(FAKE, 4, 64, FAKE, FAKE, 7, None) == ARG
    assert lib.attn_debug_route_dump(FAKE, 64, 64, 0, 4, None, None) == NULL
    assert lib.attn_debug_route_dump(FAKE, 65, 64, 1, 4, FAKE, None) == SHAPE
    assert lib.attn_debug_route_dump(FAKE, 64, 64, 0, 0, FAKE, None) == ARG


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        A.attn_fwd(q, q, q)


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "attention_prefill_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_route_trace_hook_validates():
    lib = A.load()
    base = (FAKE, FAKE, FAKE, FAKE, 1, 128, 640, 64, 4, 2, 0.1, 0, None)
    # no bitmask, no trace buffer, misaligned trace buffer, too few words
    assert lib.attn_debug_route_trace(*base, None, 4, 0, FAKE, 40, None) == NULL
    assert lib.attn_debug_route_trace(*base, FAKE, 4, 0, None, 40, None) == NULL
    assert lib.attn_debug_route_trace(*base, FAKE, 4, 0, FAKE + 2, 40, None) == ARG
    assert lib.attn_debug_route_trace(*base, FAKE, 4, 0, FAKE, 19, None) == SHAPE
    assert "20 words" in A.attn_last_error()
    # the forward rules still apply
    assert lib.attn_debug_route_trace(*base, FAKE, 0, 0, FAKE, 40, None) == ARG
    assert lib.attn_debug_route_trace(*base, FAKE, 4, 5, FAKE, 40, None) == ARG


@pytest.mark.parametrize("cu,T,ok", [
    ([0, 5, 5, 12], 12, True), ([0], 0, None), ([0, 0], 0, True), ([0, 64, 200], 200, True),
    ([1, 5, 12], 12, False), ([0, 7, 5, 12], 12, False), ([0, 5, 11], 12, False), ([0, 5, 13], 12, False),
    ([0, -1, 12], 12, False),
])
def test_cu_seqlens_rule_on_host_arrays(cu, T, ok):
    """The rule ATTN_DEBUG_VALIDATE applies before a packed launch:
    cu[0] = 0, non-decreasing, cu[B] = T (B = 0 is a shape error)."""
    if ok is None:
        with pytest.raises(A.AttnError) as e:
            A.attn_debug_check_cu_seqlens(cu, T)
        assert e.value.status == SHAPE
        return
    if ok:
        A.attn_debug_check_cu_seqlens(cu, T)
    else:
        with pytest.raises(A.AttnError) as e:
            A.attn_debug_check_cu_seqlens(cu, T)
        assert e.value.status == ARG and "cu_seqlens" in str(e.value)


def test_binding_checks_bitmask_length(orc):
    """The binding rejects a bitmask shorter than the words the kernel reads
    (ceil(qsl/64) rows of ceil(ceil(ceil(ksl/64)/tpb)/32) words); the row
    width agrees with the oracle's bitmask layout."""
    torch = pytest.importorskip("torch")
    for ksl in (1, 64, 65, 2048, 2049, 8192, 8193, 16384, 70000):
        for tpb in (1, 3, 4):
            assert _lib.route_words_per_row(ksl, tpb) == orc.words_per_row(ksl, 64, tpb)
    wpr = _lib.route_words_per_row(8300, 4)
    assert wpr == 2
    ok = torch.zeros(4 * wpr, dtype=torch.int32)
    _lib._check_route_size(ok, 200, 8300, 4, None)
    with pytest.raises(ValueError, match="kernel reads 8"):
        _lib._check_route_size(ok[:-1], 200, 8300, 4, None)
    # packed: at least ceil(T/64) rows
    _lib._check_route_size(torch.zeros(130 * 2, dtype=torch.int32), 8300, 8300, 4,
                           torch.tensor([0, 8300], dtype=torch.int32))
    with pytest.raises(ValueError):
        _lib._check_route_size(torch.zeros(129 * 2, dtype=torch.int32), 8300, 8300, 4,
                               torch.tensor([0, 8300], dtype=torch.int32))


def test_noalloc_rejects_oversized_scratch():
    """The allocation-free entry point: a routed call whose quantised K rows
    alone exceed its 64 MiB static scratch returns ATTN_ERR_SHAPE before any
    device work (fake pointers, never read)."""
    lib = A.load()
    # 8 kv heads x 65536 keys x (128 + 4) bytes = 69 MB of K codes and scales
    st = lib.attn_fwd_noalloc_stream(FAKE, FAKE, FAKE, FAKE, 1, 64, 65536, 128, 8, 8, 0.1, 0, None, FAKE, 4, 0, None)
    assert st == SHAPE and "scratch" in A.attn_last_error()
    # the forward argument rules apply first
    assert lib.attn_fwd_noalloc_stream(FAKE, FAKE, FAKE, None, 1, 64, 64, 64, 4, 2, 0.1, 0, None, None, 4, 0,
                                       None) == NULL
    assert lib.attn_fwd_noalloc_stream(FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 64, 4, 2, 0.1, 0, None, FAKE, 4, 7,
                                       None) == ARG
