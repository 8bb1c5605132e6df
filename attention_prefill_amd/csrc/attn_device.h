// attn_device.h -- device-side pieces of the forward kernel
// (attn_kernels.hip): vector types, the buffer
// resource of a tile, the INT8 / FP8 quantisation rules, half-wave
// reductions, the routing-bitmask cursor and the kernel argument block.
// Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace attn {

// Arguments of the forward kernels (one block, passed by value).
struct FwdArgs {
    const _Float16* q;
    const _Float16* k;
    const _Float16* v;
    _Float16* out;
    const int8_t* k8;       // INT8 K rows (routed: quantised per call; cache: the caller's)
    const float* sk;        // their scales
    const int8_t* v8;       // INT8 V rows of a key/value cache, or null
    const float* sv;        // their scales
    const int32_t* cu;      // packed sequence offsets, or null
    const uint32_t* route;  // routing bitmask, or null
    int B, qsl, ksl, n_qh, n_kvh, G, HPW;
    int combos;             // workgroup columns: (batch x) kv heads x head groups
    int n_mblk;             // query blocks per column (packed: upper bound)
    int tiles_per_bit, wpr;
    float c;                // |scale| * log2(e)
    int neg;                // scale < 0: queries are negated
    int pair_blocks;        // causal, whole grid resident: the second half of the
                            // row blocks runs light-first (see make_plan)
    int ksplit;             // key-range splits per query block (1: write out directly)
    float* part_o;          // split partials: [ksplit, rows, HD] O / l (fp32)
    float* part_l;          // and [ksplit, rows] log2 of the softmax denominator, base-2 units
    long long part_rows;    // output rows (B * n_qh * qsl, or n_qh * T)
    uint32_t* trace;        // test hook (routed calls), or null: visit counts per
                            // (bitmask row, key tile), +1 FP16, +0x10000 low precision
    int trace_nkt;          // key tiles per trace row
};

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int TK = 64;          // keys per routing tile
constexpr int TQ = 64;          // query rows per routing tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RNE_MAGIC = 12582912.0f;   // 1.5 * 2^23
// dword 3 of a raw buffer descriptor (32-bit data format, no swizzle, no
// index stride): reads beyond num_records return zero.
constexpr int BUF_DWORD3 = 0x00020000;

// The buffer resource of tile kt of a slab of `bytes` bytes cut into tiles
// of `tile` bytes: based at the tile's first byte and holding only the bytes
// left in the slab (none for a tile past its end).  Tile loads keep their
// per-lane offset in the VGPR offset and pass no scalar offset, so the
// descriptor's range check covers every byte they read: reads past the end
// of the slab return zero and never touch the memory that follows it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes, int tile, int kt) {
    const int o = __builtin_amdgcn_readfirstlane(kt * tile);
    const int n = bytes > o ? bytes - o : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + o), (short)0, n, BUF_DWORD3);
}

// ---------------------------------------------------------------------------
// INT8 quantisation rule shared by the K pass, the query prologue and the
// test hook.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void quant_scale(float amax, float& s, float& inv) {
    if (amax == 0.0f) {
        s = 0.0f;
        inv = 0.0f;
    } else {
        s = amax / 127.0f;       // IEEE division (no fast-math in this build)
        inv = 127.0f / amax;
    }
}

// round-half-even(x * inv) with the product exact: |x * inv| <= 127 + eps, so
// x*inv + 1.5*2^23 lies in [2^23, 2^24) where the fp32 spacing is 1 and the
// single rounding of the fused multiply-add is the integer rounding; the
// even offset keeps ties at even.
__device__ __forceinline__ int quant_code(float x, float inv) {
    float r = __builtin_fmaf(x, inv, RNE_MAGIC) - RNE_MAGIC;
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// FP8 route: e4m3 codes with rowwise scales, s = fl32(amax/448) and
// code = the e4m3 value nearest to x * fl32(448/amax) (product exact, ties to
// even).  Near |y| the e4m3 spacing is 2^(e-3), e = max(floor(log2|y|), -6);
// adding C = 1.5 * 2^(e+20), whose fp32 spacing is that same 2^(e-3), in one
// fused multiply-add rounds the exact product once to that spacing, and
// subtracting C leaves the e4m3 value (|y| <= 448 keeps e <= 8).  A product
// that rounds up across a power of two in fl32(x * inv) picks the larger
// spacing, which yields the same power of two.  Zero results are +0.
__device__ __forceinline__ float fp8_round(float x, float inv) {
    const float hi = x * inv;
    int e = (int)((__builtin_bit_cast(unsigned, hi) >> 23) & 0xffu) - 127;
    e = e < -6 ? -6 : e;
    const float C = __builtin_bit_cast(float, ((unsigned)(e + 147) << 23) | 0x400000u);
    return __builtin_fmaf(x, inv, C) - C;
}

// Four e4m3 codes (exact values, so the conversion does not round), byte b = v[b].
__device__ __forceinline__ unsigned fp8_pack4(float v0, float v1, float v2, float v3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
    return (unsigned)w;
}

__device__ __forceinline__ void fp8_scale(float amax, float& s, float& inv) {
    if (amax == 0.0f) {
        s = 0.0f;
        inv = 0.0f;
    } else {
        s = amax / 448.0f;
        inv = 448.0f / amax;
    }
}

__device__ __forceinline__ float f_from_u(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned u_from_f(float f) { return __builtin_bit_cast(unsigned, f); }

// max of a value over lanes l and l^32
__device__ __forceinline__ float halfwave_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(u_from_f(v), u_from_f(v), false, false);
    return fmaxf(f_from_u(r[0]), f_from_u(r[1]));
}

__device__ __forceinline__ float halfwave_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(u_from_f(v), u_from_f(v), false, false);
    return f_from_u(r[0]) + f_from_u(r[1]);
}

// Query rows held in the score B-operand layout: lane l (g = l/32) holds
// Q[row l%32][32*kb + 16*g + 8*e + j] in qf[2*kb + e][j].  The INT8 operand
// for k-step ks holds the 16 codes of d = 32*ks + 16*g + j, j = 0..15.
// FP8 codes use the same byte positions; an FP8 MFMA operand (64 values)
// is the pair of INT8 operands ks = 2k, 2k+1.
template <int HD, bool FP8 = false>
__device__ __forceinline__ void quantize_q_regs(const f16x8 (&qf)[HD / 16], i32x4 (&q8)[HD / 32],
                                                float& s_out) {
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < HD / 16; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)qf[t][j]));
    amax = halfwave_max(amax);
    float s, inv;
    if constexpr (FP8) fp8_scale(amax, s, inv);
    else quant_scale(amax, s, inv);
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if constexpr (FP8) {
                float r[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int j = 4 * w + b;
                    r[b] = fp8_round((float)qf[2 * ks + j / 8][j % 8], inv);
                }
                q8[ks][w] = (int)fp8_pack4(r[0], r[1], r[2], r[3]);
            } else {
                unsigned word = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    int j = 4 * w + b;
                    int c = quant_code((float)qf[2 * ks + j / 8][j % 8], inv);
                    word |= ((unsigned)c & 0xffu) << (8 * b);
                }
                q8[ks][w] = (int)word;
            }
        }
    }
    s_out = s;
}

// Exact int8 -> fp16 of the four signed bytes of w: with u = b + 128 in the low
// byte and 0x64 above it, a 16-bit lane holds the fp16 value 1024 + u, and
// subtracting 1152 leaves b.  Lanes hold bytes 0,1 (first word), 2,3 (second).
// A pointer into LDS (address space 3), for the builtins that take one.
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Transposed 8-byte LDS reads (ds_read_b64_tr_b16): within each group of 16
// lanes, lane 4a + b receives as element j the element b of the four
// 16-bit values that lane 4j + a addresses.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)LDS_PTR(const char, p);
}

// Four 8-key operand fragments from transposed reads: fragment i takes the
// two reads at LDS byte address a_i and a_i + H (its keys 0-3 and 4-7 of a
// row-major [key][d] tile whose rows are H / 4 bytes).  The reads and the wait for
// them are one asm block: written with the builtin, every such read would be
// made to wait for all direct tile loads in flight, which the compiler
// cannot tell apart from it; the barrier protocol of the callers already
// orders these reads after the loads of their stage.
template <int H>
__device__ __forceinline__ void lds_read_tr16_x4(unsigned a0, unsigned a1, unsigned a2, unsigned a3,
                                                 f16x8 (&f)[4]) {
    f16x4 r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "i"(H)
        : "memory");
    f[0] = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
    f[1] = __builtin_shufflevector(r2, r3, 0, 1, 2, 3, 4, 5, 6, 7);
    f[2] = __builtin_shufflevector(r4, r5, 0, 1, 2, 3, 4, 5, 6, 7);
    f[3] = __builtin_shufflevector(r6, r7, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ u32x2 widen_i8x4(unsigned w) {
    const unsigned u = w ^ 0x80808080u;
    const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
    const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// ---------------------------------------------------------------------------
// Routing decode.  One bitmask row belongs to one 64-row query tile; bit g of
// the row (word g / 32, bit g % 32, least significant first) routes the group
// of key tiles [g * tiles_per_bit, (g + 1) * tiles_per_bit): 1 = the
// low-precision score path, 0 = FP16.  The cursor walks a key-tile range
// [t, end) of one route: next(t, c) is the first tile >= t whose group's bit
// is c, or end.  It scans the cached word with a count of trailing zeros
// (of ~word for route 0) and reads a new word every 32 groups; a start
// inside a group or a word is allowed.  Each decode also records the run of
// consecutive groups of that route (within the cached word) around the tile
// it returns, so that the calls that follow inside the run, one per tile,
// return at once.  Every value is uniform over the wavefront.  The forward kernel's routed passes and the route-dump test
// hook both walk their tiles with this cursor.
// ---------------------------------------------------------------------------
struct RouteCursor {
    const uint32_t* row;
    int tpb;      // key tiles per bit
    int end;      // one past the last tile of the range
    int wi;       // index of the cached word, -1 for none
    uint32_t w;   // the cached word
    uint32_t rcp; // floor((2^32 - 1) / tpb), for the group index of a tile
    int run_lo;   // tiles [run_lo, run_hi) are known to take route run_c
    int run_hi;
    bool run_c;

    __device__ __forceinline__ RouteCursor(const uint32_t* r, int tiles_per_bit, int e)
        : row(r), tpb(tiles_per_bit), end(e), wi(-1), w(0),
          rcp(__builtin_amdgcn_readfirstlane(0xffffffffu / (uint32_t)tiles_per_bit)),
          run_lo(0), run_hi(0), run_c(false) {}

    // t / tpb for 0 <= t < 2^31 without a division: the high product
    // underestimates the quotient by at most one, and one step corrects it
    __device__ __forceinline__ int group_of(int t) const {
        uint32_t q = __umulhi((uint32_t)t, rcp);
        if ((q + 1) * (uint32_t)tpb <= (uint32_t)t) ++q;
        return (int)q;
    }

    __device__ __forceinline__ int next(int t, bool c) {
        if (c == run_c && t >= run_lo && t < run_hi) return t;
        while (t < end) {
            const int gi = __builtin_amdgcn_readfirstlane(group_of(t));
            if ((gi >> 5) != wi) {
                wi = gi >> 5;
                w = __builtin_amdgcn_readfirstlane(row[wi]);
            }
            const uint32_t wv = (c ? w : ~w) >> (gi & 31);
            if (wv) {
                // first group of route c at or after gi, and the length of
                // the run of route-c groups it starts (to the word's end at
                // most: the bits shifted in above it are zeros)
                const int k0 = (int)__builtin_ctz(wv);
                const uint32_t rest = ~(wv >> k0);
                const int n1 = rest ? (int)__builtin_ctz(rest) : 32;
                const int gf = gi + k0;
                const int r = min(end, max(t, gf * tpb));
                run_c = c;
                run_lo = r;
                run_hi = min(end, (gf + n1) * tpb);
                return r;
            }
            t = (wi + 1) * 32 * tpb;
        }
        return end;
    }
};



// Running max starts finite so that no exp2 argument is ever (-inf) - (-inf).
constexpr float M_INIT = -1.0e30f;
// The reference max of a row moves only when a new score exceeds it by more
// than TAU (log2 units); until then exp2(x - m) <= 2^TAU, which fp16 P and
// the fp32 sums hold exactly as well as values <= 1.  The result O / l does
// not depend on the reference chosen.
constexpr float TAU = 8.0f;

}  // namespace
}  // namespace attn
