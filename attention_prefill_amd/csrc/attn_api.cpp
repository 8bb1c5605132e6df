// attn_api.cpp -- the C ABI declared in include/attn.h: argument validation
// (on the host, before any device work), stream-ordered scratch, dispatch
// to the kernel launchers, and error reporting.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "attn_internal.h"

namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

attn_status hip_fail(hipError_t e, const char* what) {
    return fail(ATTN_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Checks every argument rule of include/attn.h; touches no device memory.
attn_status validate(const attn::Problem& p) {
    const bool kv8 = p.k8 != nullptr || p.v8 != nullptr || p.k_scale != nullptr || p.v_scale != nullptr;
    if (kv8) {
        if (!p.q || !p.k8 || !p.k_scale || !p.v8 || !p.v_scale || !p.out)
            return fail(ATTN_ERR_NULL, "q, k8, k_scale, v8, v_scale and out must be non-null device pointers");
    } else if (!p.q || !p.k || !p.v || !p.out) {
        return fail(ATTN_ERR_NULL, "q, k, v and out must be non-null device pointers");
    }
    if (p.B <= 0 || p.qsl <= 0 || p.ksl <= 0 || p.n_qh <= 0 || p.n_kvh <= 0)
        return fail(ATTN_ERR_SHAPE, "B, qsl, ksl, n_qh, n_kvh must be positive (got %d, %d, %d, %d, %d)",
                    p.B, p.qsl, p.ksl, p.n_qh, p.n_kvh);
    if (p.n_qh % p.n_kvh != 0)
        return fail(ATTN_ERR_SHAPE, "n_qh (%d) must be a multiple of n_kvh (%d)", p.n_qh, p.n_kvh);
    if (p.causal && p.qsl > p.ksl)
        return fail(ATTN_ERR_SHAPE, "causal attention needs qsl <= ksl (got %d > %d): rows would see no key",
                    p.qsl, p.ksl);
    if (p.cu_seqlens && p.qsl != p.ksl)
        return fail(ATTN_ERR_SHAPE, "packed input needs qsl == ksl == total tokens (got %d, %d)", p.qsl, p.ksl);
    if (p.hdim != 64 && p.hdim != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "hdim must be 64 or 128 (got %d)", p.hdim);
    if (!std::isfinite(p.scale) || p.scale == 0.0f)
        return fail(ATTN_ERR_ARG, "scale must be finite and non-zero");
    if (p.route && p.tiles_per_bit < 1)
        return fail(ATTN_ERR_ARG, "tiles_per_bit must be >= 1 with a bitmask (got %d)", p.tiles_per_bit);
    if (p.lowp != ATTN_LOWP_INT8 && p.lowp != ATTN_LOWP_FP8_E4M3)
        return fail(ATTN_ERR_ARG, "lowp_format must be ATTN_LOWP_INT8 or ATTN_LOWP_FP8_E4M3 (got %d)", p.lowp);
    if (p.lowp == ATTN_LOWP_FP8_E4M3 && kv8)
        return fail(ATTN_ERR_UNSUPPORTED, "an INT8 key/value cache has no FP8 codes");
    if (kv8) {
        if (!aligned16(p.q) || !aligned16(p.k8) || !aligned16(p.v8) || !aligned16(p.out))
            return fail(ATTN_ERR_ARG, "q, k8, v8 and out must be 16-byte aligned");
        if (!aligned4(p.k_scale) || !aligned4(p.v_scale))
            return fail(ATTN_ERR_ARG, "k_scale and v_scale must be 4-byte aligned");
    } else if (!aligned16(p.q) || !aligned16(p.k) || !aligned16(p.v) || !aligned16(p.out)) {
        return fail(ATTN_ERR_ARG, "q, k, v and out must be 16-byte aligned");
    }
    if ((p.cu_seqlens && !aligned4(p.cu_seqlens)) || (p.route && !aligned4(p.route)))
        return fail(ATTN_ERR_ARG, "cu_seqlens and route_bitmask must be 4-byte aligned");
    const double elems_q = (double)p.B * p.n_qh * p.qsl * p.hdim;
    const double elems_k = (double)p.B * p.n_kvh * p.ksl * p.hdim;
    // the tile loads address one (sequence, kv head) slab of K or V through a
    // 32-bit buffer range
    if (elems_q > 9.0e15 || elems_k > 9.0e15 || (double)p.B * p.n_kvh * p.ksl > 2.0e9 ||
        (double)p.ksl * p.hdim * 2 > 2.0e9)
        return fail(ATTN_ERR_SHAPE, "problem too large");
    return ATTN_OK;
}

bool env_on(const char* name) {
    const char* v = getenv(name);
    return v && v[0] == '1' && v[1] == 0;
}

// Scratch comes from a stream-ordered memory pool that the library creates
// for each device on first use and owns (the device's default pool and its
// settings are left alone).  Its release threshold is the maximum, so freed
// blocks stay cached in the pool for the next call instead of going back to
// the system at every synchronise.
attn_status scratch_pool(hipMemPool_t* out) {
    static std::mutex mu;
    static std::vector<hipMemPool_t> pools;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    if ((int)pools.size() <= dev) pools.resize(dev + 1, nullptr);
    if (!pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return hip_fail(e, "hipMemPoolCreate of the scratch pool");
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return hip_fail(e, "hipMemPoolSetAttribute of the scratch pool");
        }
        pools[dev] = pool;
    }
    *out = pools[dev];
    return ATTN_OK;
}

attn_status scratch_alloc(void** ptr, size_t bytes, hipStream_t st) {
    hipMemPool_t pool = nullptr;
    attn_status ps = scratch_pool(&pool);
    if (ps != ATTN_OK) return ps;
    hipError_t e = hipMallocFromPoolAsync(ptr, bytes, pool, st);
    if (e != hipSuccess) return hip_fail(e, "hipMallocFromPoolAsync of scratch");
    return ATTN_OK;
}

// The cu_seqlens rule of include/attn.h on a host copy: [0] = 0,
// non-decreasing, [B] = T.
attn_status check_cu_seqlens(const int32_t* cu, int B, int T) {
    if (cu[0] != 0) return fail(ATTN_ERR_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
    for (int i = 0; i < B; ++i)
        if (cu[i + 1] < cu[i])
            return fail(ATTN_ERR_ARG, "cu_seqlens must be non-decreasing (cu_seqlens[%d] = %d > cu_seqlens[%d] = %d)",
                        i, cu[i], i + 1, cu[i + 1]);
    if (cu[B] != T) return fail(ATTN_ERR_ARG, "cu_seqlens[%d] must equal the total tokens %d (got %d)", B, T, cu[B]);
    return ATTN_OK;
}

// Debug switches (environment, read at every call):
//   ATTN_DEBUG_VALIDATE=1  copy cu_seqlens to the host (synchronising the
//                          stream) and check its contents before launching;
//   ATTN_DEBUG_SYNC=1      synchronise the stream after the launch and report
//                          a failed kernel as ATTN_ERR_HIP from this call.
attn_status debug_validate(const attn::Problem& p, hipStream_t st) {
    if (!p.cu_seqlens || !env_on("ATTN_DEBUG_VALIDATE")) return ATTN_OK;
    std::vector<int32_t> host((size_t)p.B + 1);
    hipError_t e = hipMemcpyAsync(host.data(), p.cu_seqlens, host.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "ATTN_DEBUG_VALIDATE: reading cu_seqlens");
    return check_cu_seqlens(host.data(), p.B, p.qsl);
}

attn_status debug_sync(hipStream_t st, const char* what) {
    if (!env_on("ATTN_DEBUG_SYNC")) return ATTN_OK;
    hipError_t e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, what);
    return ATTN_OK;
}

attn_status run_forward(const attn::Problem& p, hipStream_t st) {
    attn_status vs = validate(p);
    if (vs != ATTN_OK) return vs;
    vs = debug_validate(p, st);
    if (vs != ATTN_OK) return vs;
    void* scratch = nullptr;
    const size_t sbytes = attn::forward_scratch_bytes(p);
    if (sbytes) {
        vs = scratch_alloc(&scratch, sbytes, st);
        if (vs != ATTN_OK) return vs;
    }
    hipError_t e = attn::launch_forward(p, scratch, st);
    if (scratch) {
        hipError_t e2 = hipFreeAsync(scratch, st);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(e, "attention forward launch");
    vs = debug_sync(st, "attention forward (ATTN_DEBUG_SYNC)");
    if (vs != ATTN_OK) return vs;
    g_last_error.clear();
    return ATTN_OK;
}

// The unfused baseline: same validation, dense only, and a cap on the score
// scratch (6 bytes per query-key pair).
attn_status run_unfused(const attn::Problem& p, hipStream_t st) {
    attn_status vs = validate(p);
    if (vs != ATTN_OK) return vs;
    const size_t bytes = attn::unfused_scratch_bytes(p);
    if ((double)p.B * p.n_qh * p.qsl * p.ksl * 6.0 > 64.0e9)
        return fail(ATTN_ERR_SHAPE, "unfused scores need %.1f GB of scratch (limit 64 GB)",
                    (double)p.B * p.n_qh * p.qsl * p.ksl * 6.0 / 1e9);
    void* scratch = nullptr;
    vs = scratch_alloc(&scratch, bytes, st);
    if (vs != ATTN_OK) return vs;
    hipError_t e = attn::launch_unfused(p, scratch, st);
    hipError_t e2 = hipFreeAsync(scratch, st);
    if (e == hipSuccess) e = e2;
    if (e != hipSuccess) return hip_fail(e, "unfused attention");
    vs = debug_sync(st, "unfused attention (ATTN_DEBUG_SYNC)");
    if (vs != ATTN_OK) return vs;
    g_last_error.clear();
    return ATTN_OK;
}

attn_status quantize_rows(const void* x, long long rows, int32_t hdim, int8_t* q8, float* scale_out,
                          int32_t path, hipStream_t st) {
    if (!x || !q8 || !scale_out) return fail(ATTN_ERR_NULL, "null pointer");
    if (rows < 0 || rows > 0x7fffffffLL) return fail(ATTN_ERR_SHAPE, "rows must be in [0, 2^31)");
    if (hdim != 64 && hdim != 128) return fail(ATTN_ERR_UNSUPPORTED, "hdim must be 64 or 128");
    if (!aligned16(x) || !aligned16(q8) || !aligned4(scale_out))
        return fail(ATTN_ERR_ARG, "x and q8 must be 16-byte aligned, scale_out 4-byte aligned");
    hipError_t e = attn::launch_quantize_rows(x, rows, hdim, q8, scale_out, path, st);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    g_last_error.clear();
    return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_fwd_stream(const void* q, const void* k, const void* v, void* out, int32_t B,
                            int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                            float scale, int32_t causal, const int32_t* cu_seqlens,
                            const uint32_t* route_bitmask, int32_t tiles_per_bit, void* hip_stream) {
    attn::Problem p{q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal != 0,
                    cu_seqlens, route_bitmask, tiles_per_bit};
    return run_forward(p, (hipStream_t)hip_stream);
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* out, int32_t B,
                     int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                     float scale, int32_t causal, const int32_t* cu_seqlens,
                     const uint32_t* route_bitmask, int32_t tiles_per_bit) {
    return attn_fwd_stream(q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal, cu_seqlens,
                           route_bitmask, tiles_per_bit, nullptr);
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

attn_status attn_fwd_lowp_stream(const void* q, const void* k, const void* v, void* out, int32_t B,
                                 int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                                 float scale, int32_t causal, const int32_t* cu_seqlens,
                                 const uint32_t* route_bitmask, int32_t tiles_per_bit, int32_t lowp_format,
                                 void* hip_stream) {
    attn::Problem p{q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal != 0,
                    cu_seqlens, route_bitmask, tiles_per_bit};
    p.lowp = lowp_format;
    return run_forward(p, (hipStream_t)hip_stream);
}

attn_status attn_fwd_kv8_stream(const void* q, const int8_t* k8, const float* k_scale, const int8_t* v8,
                                const float* v_scale, void* out, int32_t B, int32_t qsl, int32_t ksl,
                                int32_t hdim, int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                                const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                                int32_t tiles_per_bit, void* hip_stream) {
    attn::Problem p{q, nullptr, nullptr, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal != 0,
                    cu_seqlens, route_bitmask, tiles_per_bit};
    p.k8 = k8;
    p.k_scale = k_scale;
    p.v8 = v8;
    p.v_scale = v_scale;
    if (!k8 || !k_scale || !v8 || !v_scale || !q || !out)
        return fail(ATTN_ERR_NULL, "q, k8, k_scale, v8, v_scale and out must be non-null device pointers");
    return run_forward(p, (hipStream_t)hip_stream);
}

attn_status attn_fwd_kv8(const void* q, const int8_t* k8, const float* k_scale, const int8_t* v8,
                         const float* v_scale, void* out, int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                         int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                         const int32_t* cu_seqlens, const uint32_t* route_bitmask, int32_t tiles_per_bit) {
    return attn_fwd_kv8_stream(q, k8, k_scale, v8, v_scale, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal,
                               cu_seqlens, route_bitmask, tiles_per_bit, nullptr);
}

attn_status attn_fwd_unfused_stream(const void* q, const void* k, const void* v, void* out, int32_t B,
                                    int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                                    float scale, int32_t causal, void* hip_stream) {
    attn::Problem p{q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal != 0, nullptr, nullptr, 1};
    return run_unfused(p, (hipStream_t)hip_stream);
}

attn_status attn_quantize_rows(const void* x_f16, int64_t rows, int32_t hdim, int8_t* q8, float* scale_out,
                               void* hip_stream) {
    return quantize_rows(x_f16, (long long)rows, hdim, q8, scale_out, 0, (hipStream_t)hip_stream);
}

attn_status attn_debug_quantize_rows(const void* x_f16, int32_t rows, int32_t hdim, int8_t* q8,
                                     float* scale_out, int32_t path, void* hip_stream) {
    if (path < 0 || path > 3) return fail(ATTN_ERR_ARG, "path must be 0, 1, 2 or 3");
    return quantize_rows(x_f16, (long long)rows, hdim, q8, scale_out, path, (hipStream_t)hip_stream);
}

attn_status attn_debug_plan(int32_t B, int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                            int32_t causal, int32_t tiles_per_bit, int32_t flags, int64_t* plan_out) {
    if (!plan_out) return fail(ATTN_ERR_NULL, "plan_out must be a non-null host pointer");
    if (flags & ~15) return fail(ATTN_ERR_ARG, "flags has unknown bits (0x%x)", (unsigned)flags);
    // stand-in device addresses: validated for alignment, never read
    char* const fake = reinterpret_cast<char*>(uintptr_t(1) << 20);
    attn::Problem p{fake, fake, fake, fake, B, qsl, ksl, hdim, n_qh, n_kvh, 1.0f, causal != 0,
                    (flags & 1) ? reinterpret_cast<const int32_t*>(fake) : nullptr,
                    (flags & 2) ? reinterpret_cast<const uint32_t*>(fake) : nullptr, tiles_per_bit};
    if (flags & 4) {
        p.k8 = reinterpret_cast<const int8_t*>(fake);
        p.v8 = reinterpret_cast<const int8_t*>(fake);
        p.k_scale = reinterpret_cast<const float*>(fake);
        p.v_scale = reinterpret_cast<const float*>(fake);
    }
    if (flags & 8) p.lowp = ATTN_LOWP_FP8_E4M3;
    attn_status vs = validate(p);
    if (vs != ATTN_OK) return vs;
    long long out[10];
    attn::forward_plan(p, out);
    for (int i = 0; i < 10; ++i) plan_out[i] = out[i];
    g_last_error.clear();
    return ATTN_OK;
}

attn_status attn_fwd_noalloc_stream(const void* q, const void* k, const void* v, void* out, int32_t B,
                                    int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                                    float scale, int32_t causal, const int32_t* cu_seqlens,
                                    const uint32_t* route_bitmask, int32_t tiles_per_bit, int32_t lowp_format,
                                    void* hip_stream) {
    attn::Problem p{q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal != 0,
                    cu_seqlens, route_bitmask, tiles_per_bit};
    p.lowp = lowp_format;
    attn_status vs = validate(p);
    if (vs != ATTN_OK) return vs;
    const size_t sbytes = attn::forward_scratch_bytes(p);
    if (sbytes > attn::NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_SHAPE, "this call needs %zu bytes of scratch; the allocation-free entry point has %zu",
                    sbytes, attn::NOALLOC_SCRATCH_BYTES);
    void* scratch = nullptr;
    hipError_t e = attn::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "looking up the static scratch");
    hipStream_t st = (hipStream_t)hip_stream;
    e = attn::launch_forward(p, scratch, st);
    if (e != hipSuccess) return hip_fail(e, "attention forward launch");
    vs = debug_sync(st, "attention forward (ATTN_DEBUG_SYNC)");
    if (vs != ATTN_OK) return vs;
    g_last_error.clear();
    return ATTN_OK;
}

attn_status attn_debug_route_trace(const void* q, const void* k, const void* v, void* out, int32_t B,
                                   int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                                   float scale, int32_t causal, const int32_t* cu_seqlens,
                                   const uint32_t* route_bitmask, int32_t tiles_per_bit, int32_t lowp_format,
                                   uint32_t* trace_out, int64_t trace_words, void* hip_stream) {
    if (!route_bitmask) return fail(ATTN_ERR_NULL, "the route trace needs a routing bitmask");
    if (!trace_out) return fail(ATTN_ERR_NULL, "trace_out must be a non-null device pointer");
    if (!aligned4(trace_out)) return fail(ATTN_ERR_ARG, "trace_out must be 4-byte aligned");
    attn::Problem p{q, k, v, out, B, qsl, ksl, hdim, n_qh, n_kvh, scale, causal != 0,
                    cu_seqlens, route_bitmask, tiles_per_bit};
    p.lowp = lowp_format;
    attn_status vs = validate(p);
    if (vs != ATTN_OK) return vs;
    const long long n_kt = (ksl + 63) / 64;
    const long long rows = cu_seqlens ? (qsl + 63) / 64 + B : (qsl + 63) / 64;
    if (trace_words < rows * n_kt)
        return fail(ATTN_ERR_SHAPE, "trace_out needs %lld words (got %lld)", rows * n_kt, (long long)trace_words);
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e = hipMemsetAsync(trace_out, 0, (size_t)trace_words * sizeof(uint32_t), st);
    if (e != hipSuccess) return hip_fail(e, "clearing trace_out");
    p.trace = trace_out;
    return run_forward(p, st);
}

attn_status attn_debug_check_cu_seqlens(const int32_t* cu_seqlens_host, int32_t B, int32_t T) {
    if (!cu_seqlens_host) return fail(ATTN_ERR_NULL, "cu_seqlens_host is null");
    if (B <= 0) return fail(ATTN_ERR_SHAPE, "B must be positive (got %d)", B);
    attn_status vs = check_cu_seqlens(cu_seqlens_host, B, T);
    if (vs == ATTN_OK) g_last_error.clear();
    return vs;
}

attn_status attn_debug_route_dump(const uint32_t* route_bitmask, int32_t qsl, int32_t ksl,
                                  int32_t causal, int32_t tiles_per_bit, uint8_t* route_out,
                                  void* hip_stream) {
    if (!route_out) return fail(ATTN_ERR_NULL, "route_out is null");
    if (qsl <= 0 || ksl <= 0) return fail(ATTN_ERR_SHAPE, "qsl and ksl must be positive");
    if (causal && qsl > ksl) return fail(ATTN_ERR_SHAPE, "causal needs qsl <= ksl");
    if (tiles_per_bit < 1) return fail(ATTN_ERR_ARG, "tiles_per_bit must be >= 1");
    if (route_bitmask && !aligned4(route_bitmask)) return fail(ATTN_ERR_ARG, "route_bitmask must be 4-byte aligned");
    hipError_t e = attn::launch_route_dump(route_bitmask, qsl, ksl, causal != 0, tiles_per_bit, route_out,
                                           (hipStream_t)hip_stream);
    if (e != hipSuccess) return hip_fail(e, "route dump launch");
    g_last_error.clear();
    return ATTN_OK;
}

}  // extern "C"
