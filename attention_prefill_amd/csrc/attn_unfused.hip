// attn_unfused.hip -- the unfused attention forward on MI355X: the composed
// path that the "Nax Refactor" page (ml-explore/mlx pull request 3271) times
// against its fused kernel (the t_unfs and speed_up columns of its timing
// tables).  It materialises the scores:
//   S = Q K^T           one strided-batched rocBLAS GEMM per call, fp16 in,
//                       fp32 out, per (batch element, kv head) so that the G
//                       query heads of a kv head are one [G*qsl, d] operand
//   P = softmax(c * S)  a masked row softmax in base 2 (c = scale*log2(e)),
//                       fp32 arithmetic, fp16 P (hand-written, below)
//   O = P V             a second strided-batched GEMM, fp16 in and out,
//                       fp32 accumulation
// The scores and P live in stream-ordered scratch: 6 bytes per (query, key)
// pair.  This is a baseline for the fused kernel, not a fast path: it moves
// the whole score matrix through HBM three times.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <stdint.h>

#include <mutex>

#include "attn_internal.h"

namespace attn {
namespace {

constexpr int SM_THREADS = 256;
constexpr float LOG2E_U = 1.4426950408889634f;

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
    for (int o = 32; o > 0; o >>= 1) {
        const float w = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, w) : v + w;
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();                     // red may still be read by a previous reduction
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < SM_THREADS / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

// One workgroup per score row.  Row r of the [rows, ksl] score matrix is
// query i = r % qsl of its head; under a causal mask key j is visible iff
// j <= i + ksl - qsl (bottom-right aligned).  Masked entries of P are 0.
__global__ __launch_bounds__(SM_THREADS) void masked_softmax_kernel(const float* __restrict__ S,
                                                                    _Float16* __restrict__ P, int qsl,
                                                                    int ksl, int causal, float c) {
    __shared__ float red[SM_THREADS / 64];
    const long long r = blockIdx.x;
    const int i = (int)(r % qsl);
    const int lim = causal ? min(ksl - 1, i + ksl - qsl) : ksl - 1;   // last visible key
    const float* s = S + r * (long long)ksl;
    _Float16* p = P + r * (long long)ksl;

    float m = -INFINITY;
    for (int j = threadIdx.x; j <= lim; j += SM_THREADS) m = fmaxf(m, s[j] * c);
    m = block_reduce(m, true, red);
    float l = 0.0f;
    for (int j = threadIdx.x; j <= lim; j += SM_THREADS) l += __builtin_amdgcn_exp2f(s[j] * c - m);
    l = block_reduce(l, false, red);
    const float inv = 1.0f / l;
    for (int j = threadIdx.x; j < ksl; j += SM_THREADS)
        p[j] = (_Float16)(j <= lim ? __builtin_amdgcn_exp2f(s[j] * c - m) * inv : 0.0f);
}

// One rocBLAS handle per device, created on first use; calls on one device
// take its lock (a handle carries a stream and is not shared concurrently).
struct Blas {
    std::mutex mu;
    rocblas_handle h = nullptr;
};
Blas g_blas[64];

hipError_t blas_error(rocblas_status s) {
    return s == rocblas_status_success ? hipSuccess
           : s == rocblas_status_memory_error ? hipErrorOutOfMemory
                                               : hipErrorLaunchFailure;
}

}  // namespace

size_t unfused_scratch_bytes(const Problem& p) {
    const size_t pairs = (size_t)p.B * p.n_qh * p.qsl * p.ksl;
    const size_t s_bytes = (pairs * sizeof(float) + 255) / 256 * 256;
    return s_bytes + pairs * sizeof(_Float16);
}

hipError_t launch_unfused(const Problem& p, void* scratch, hipStream_t st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    Blas& b = g_blas[dev];
    std::lock_guard<std::mutex> lock(b.mu);
    if (!b.h) {
        rocblas_status s = rocblas_create_handle(&b.h);
        if (s != rocblas_status_success) {
            b.h = nullptr;
            return blas_error(s);
        }
    }
    rocblas_status s = rocblas_set_stream(b.h, st);
    if (s != rocblas_status_success) return blas_error(s);

    const size_t pairs = (size_t)p.B * p.n_qh * p.qsl * p.ksl;
    float* S = (float*)scratch;
    _Float16* P = (_Float16*)((char*)scratch + (pairs * sizeof(float) + 255) / 256 * 256);
    const int G = p.n_qh / p.n_kvh;
    const int M = G * p.qsl;                  // query rows of one kv head
    const int batch = p.B * p.n_kvh;
    const float one = 1.0f, zero = 0.0f;

    // S^T (column-major ksl x M) = K (d x ksl, transposed) * Q^T (d x M)
    s = rocblas_gemm_strided_batched_ex(
        b.h, rocblas_operation_transpose, rocblas_operation_none, p.ksl, M, p.hdim, &one,
        p.k, rocblas_datatype_f16_r, p.hdim, (rocblas_stride)p.ksl * p.hdim,
        p.q, rocblas_datatype_f16_r, p.hdim, (rocblas_stride)M * p.hdim, &zero,
        S, rocblas_datatype_f32_r, p.ksl, (rocblas_stride)M * p.ksl,
        S, rocblas_datatype_f32_r, p.ksl, (rocblas_stride)M * p.ksl,
        batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    if (s != rocblas_status_success) return blas_error(s);

    const long long rows = (long long)p.B * p.n_qh * p.qsl;
    hipLaunchKernelGGL(masked_softmax_kernel, dim3((unsigned)rows), dim3(SM_THREADS), 0, st, S, P, p.qsl,
                       p.ksl, p.causal ? 1 : 0, p.scale * LOG2E_U);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // O^T (column-major d x M) = V^T (d x ksl) * P^T (ksl x M)
    const float one_h = 1.0f, zero_h = 0.0f;
    s = rocblas_gemm_strided_batched_ex(
        b.h, rocblas_operation_none, rocblas_operation_none, p.hdim, M, p.ksl, &one_h,
        p.v, rocblas_datatype_f16_r, p.hdim, (rocblas_stride)p.ksl * p.hdim,
        P, rocblas_datatype_f16_r, p.ksl, (rocblas_stride)M * p.ksl, &zero_h,
        p.out, rocblas_datatype_f16_r, p.hdim, (rocblas_stride)M * p.hdim,
        p.out, rocblas_datatype_f16_r, p.hdim, (rocblas_stride)M * p.hdim,
        batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    return blas_error(s);
}

}  // namespace attn
