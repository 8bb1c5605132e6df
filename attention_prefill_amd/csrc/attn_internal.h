// attn_internal.h -- host-side interface between the C ABI (attn_api.cpp)
// and the kernel launchers (attn_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// A validated forward problem (see include/attn.h for the meaning of each field).
struct Problem {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int B, qsl, ksl, hdim, n_qh, n_kvh;
    float scale;
    bool causal;
    const int32_t* cu_seqlens;      // device, or nullptr
    const uint32_t* route;          // device, or nullptr
    int tiles_per_bit;
    // INT8 key/value cache (k and v unused when k8 is set): codes and per-row scales
    const int8_t* k8 = nullptr;
    const float* k_scale = nullptr;
    const int8_t* v8 = nullptr;
    const float* v_scale = nullptr;
    // what a set routing bit selects: 0 INT8, 1 FP8 e4m3 (rowwise scales)
    int lowp = 0;
    // test hook (routed calls): device uint32 [bitmask rows, ceil(ksl / 64)],
    // zeroed by the caller; every workgroup adds 1 (FP16) or 0x10000 (low
    // precision) at each key tile it visits
    uint32_t* trace = nullptr;
};

// Device scratch a forward call needs (bytes): quantised K rows for routed
// calls and split-key partials when the key range is split.  0 if none.
size_t forward_scratch_bytes(const Problem& p);

// The allocation-free entry point's device scratch: a static device array of
// this many bytes per device; noalloc_scratch gives its address on the
// current device (looked up once per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);
// The launch plan of a forward call (no device access): query wavefronts per
// workgroup, key groups, heads per workgroup, rows per workgroup, workgroup
// columns, row blocks per column, key splits, light-first pairing, grid size,
// scratch bytes.
void forward_plan(const Problem& p, long long out[10]);

// Enqueue the whole forward pass on stream.  scratch must hold
// forward_scratch_bytes(p) bytes (may be null when that is 0).
hipError_t launch_forward(const Problem& p, void* scratch, hipStream_t stream);

// The unfused baseline: scores, a masked softmax and P.V as separate passes
// (attn_unfused.hip).  Dense problems only; scratch holds the fp32 scores
// and the fp16 probabilities.
size_t unfused_scratch_bytes(const Problem& p);
hipError_t launch_unfused(const Problem& p, void* scratch, hipStream_t stream);

// Quantisers (include/attn.h): path 0 K-row pass INT8, 1 query prologue
// INT8, 2 K-row pass FP8, 3 query prologue FP8.
hipError_t launch_quantize_rows(const void* x, long long rows, int hdim, int8_t* q8, float* s,
                                int path, hipStream_t stream);
hipError_t launch_route_dump(const uint32_t* route, int qsl, int ksl, bool causal,
                             int tiles_per_bit, uint8_t* out, hipStream_t stream);

}  // namespace attn
