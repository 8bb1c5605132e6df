// attn_kernels.hip -- fused attention forward (prefill) for gfx950 (MI355X).
//
// The operation is the fused scaled-dot-product attention timed in the
// "Nax Refactor" page (ml-explore/mlx pull request 3271, fused vs unfused
// timing tables), with the TileMix option (TileMix abstract): a bitmask
// routes each (64-row query tile, group of 64-key tiles) through an FP16 or
// an INT8 QK^T score computation, and both routes update one online-softmax
// state (running max m, running sum l, fp32 output accumulator).
//
// Kernel structure (one workgroup = KS key groups of NW wavefronts of 64 lanes):
//   * work decomposition: a workgroup owns HPW query heads of one kv head
//     and BM = 32*NW/HPW query rows; every wavefront owns 32 rows of one
//     head.  With KS = 2 a second group of NW wavefronts owns the same rows
//     and takes every other key tile; the two online-softmax states merge
//     through LDS at the end (small grids get two wavefronts per SIMD this
//     way without a second pass; small causal grids use NW = 2, two
//     workgroups per CU, so heavy and light query blocks share CUs).
//     Grid order is heavy-first for causal
//     masks and keeps the workgroups of one kv head on one XCD (index mod 8)
//     when the number of head groups is a multiple of 8.
//   * tile loader: 64-key K and V tiles (and INT8/FP8 codes with their
//     scales) are read through buffer descriptors that end at the sequence's
//     last byte (reads past it return zeros).  The fp16 and routed kernels
//     load them straight into LDS (buffer loads with LDS as the
//     destination) in an XOR-swizzled row-major layout, four stages with
//     the tile two ahead and a barrier every other tile for eight
//     wavefronts, two stages and a barrier per tile otherwise.  The INT8
//     key/value-cache kernels go global -> registers -> LDS, widening the
//     codes to fp16 on the way.
//   * score MFMA: the transposed score tile S^T = K Q^T is computed with
//     v_mfma_f32_32x32x16_f16 (FP16 route), v_mfma_i32_32x32x32_i8 (INT8
//     route) or v_mfma_f32_32x32x64_f8f6f4 on e4m3 codes (FP8 route).  In the 32x32 accumulator layout a lane then owns one query
//     (column) and 16 keys, so row max / row sum are in-register plus one
//     v_permlane32_swap between the two half-waves.  K rows are read with
//     bits 2 and 3 of the row index swapped; this makes the score layout
//     coincide with the B-operand layout of the P.V MFMA, so P never leaves
//     registers.
//   * P.V MFMA: O^T += V^T P^T with v_mfma_f32_32x32x16_f16.  Directly
//     loaded V stays [key][d] in LDS and each V^T fragment (8 keys of one d)
//     is two transposed 8-byte reads (ds_read_b64_tr_b16); the register
//     path stores V transposed, [d][key], for one 16-byte read.
//   * online softmax in base 2 with the scale folded into one FMA per
//     score; O is rescaled only when some row max of the wavefront moved by
//     more than a threshold.
//   * INT8 route: K rows are quantised once per call by a separate pass
//     (quantize_rows_kernel); the query rows of a wavefront are quantised in
//     its prologue.  Per-token symmetric codes: s = fl32(amax/127),
//     q = RNE(x * fl32(127/amax)) with the product exact (one FMA against
//     1.5*2^23), int32 dot products, dequantised as dot * (s_k*c) * s_q.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <math.h>

#include <mutex>
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

// Device scratch of the allocation-free entry point (attn_fwd_noalloc_stream):
// quantised K rows and split-key partials live here instead of in memory
// allocated per call.  One copy per device, held from module load until the
// process ends; every call on a device shares it.
static __device__ __align__(256) char scratch[attn::NOALLOC_SCRATCH_BYTES];

namespace attn {
namespace {

#ifndef ATTN_KEY_TILE
#define ATTN_KEY_TILE 64
#endif
constexpr int BN = ATTN_KEY_TILE;   // keys per kernel tile (64 or 32)
static_assert(BN == 64 || BN == 32, "key tile must be 64 or 32");
constexpr int NKB = BN / 32;        // 32-key score blocks per tile
#ifndef ATTN_STAGES4
#define ATTN_STAGES4 1
#endif
// Where routed calls quantise their K rows: 0 = once per call in a pass of
// their own (quantize_rows_kernel) whose codes the low-precision tiles load;
// 1 = in the tile loader of every workgroup, from the fp16 K tile, as it is
// staged into LDS (the same device rounding, so the same codes).  Both are
// built and timed; 0 is the default (measured faster).
#ifndef ATTN_FUSED_KQUANT
#define ATTN_FUSED_KQUANT 0
#endif
// Tile loads of the hdim-128 four-stage kernels (fp16 K and V, INT8 or FP8
// K codes and their scales): 1 = buffer loads that write LDS directly (no
// staging registers, no LDS store instructions, no transpose work on the
// VALU); 0 = loads into registers and LDS stores, as the other kernels.
#ifndef ATTN_DMA
#define ATTN_DMA 1
#endif
// ---------------------------------------------------------------------------
// LDS layout of one stage on the register path (INT8 key/value caches; the
// directly loaded layout is LdsDma below): the K tile (fp16 [key][d], or
// INT8 codes [key][d]), the V tile stored transposed, [d][key], so that the
// P.V operand (8 consecutive keys of one d) is a single 16-byte read, and
// the tile's per-key scales (K scales times |scale|*log2(e), then V scales).
// Row pitches are padded so that the row-parallel operand reads and the
// staging writes spread over the banks.
// ---------------------------------------------------------------------------
// LDS stages of a kernel shape: the eight-wavefront kernels keep four
// (tiles are stored two ahead, so one barrier covers two tiles); the others
// two.
__host__ __device__ constexpr int n_stages(int nw, int ks, bool routed) {
    return (ATTN_STAGES4 && nw == 8 && ks == 1) ? 4 : 2;
}
// Kernel shapes whose tiles travel from global memory to LDS directly.
__host__ __device__ constexpr bool use_dma(int hd, int nw, int ks, bool routed, bool kv8) {
    return ATTN_DMA && !ATTN_FUSED_KQUANT && BN == 64 && (hd == 128 || hd == 64) && !kv8 && nw >= 2;
}

// Directly loaded stages are unpadded and row-major, with the 16-byte
// chunks of each row permuted by an XOR of the row index, so that the
// operand reads of 16 lanes (16-byte reads) or 32 lanes (8-byte transposed
// reads), all at one column of different rows, fall on distinct banks:
// - fp16 K: chunk c of row r at c ^ (r & 15) (hdim 128, 16 chunks per
//   256-byte row) or c ^ ((r >> 1) & 7) (hdim 64, 8 chunks per 128-byte
//   row, two rows per bank sweep);
// - INT8 / FP8 K codes: c ^ ((r >> 1) & 7) (hdim 128, 128-byte rows) or
//   c ^ ((r >> 2) & 3) (hdim 64, 64-byte rows);
// - V, [key][d], read four keys by 4 x 4 d at a time: chunk c of key r at
//   c ^ (4 * (r & 3)) (hdim 128) or c ^ (4 * ((r >> 1) & 1)) (hdim 64).
// The per-key scales of a tile follow the V tile (raw s_k, then s_v).
template <int HD>
struct LdsDma {
    static constexpr int KBYTES = BN * HD * 2;
    static constexpr int KREG = KBYTES;
    static constexpr int VBYTES = BN * HD * 2;
    static constexpr int SCL = 2 * BN * 4;
    static constexpr int STAGE = KREG + VBYTES + SCL;
    static constexpr int TOTAL = 2 * STAGE;
    static constexpr int CPR = HD * 2 / 16;       // 16-byte chunks per fp16 row
    static constexpr int KRPB = 1024 / (HD * 2);  // fp16 rows per 1 KB load block
    static constexpr int KBLK = BN / KRPB;        // load blocks per fp16 tile
    static constexpr int C8PR = HD / 16;          // 16-byte chunks per code row
    static constexpr int K8RPB = 1024 / HD;       // code rows per load block
    static constexpr int K8BLK = BN / K8RPB;      // load blocks per code tile
    // chunk permutations: rows that share a 256-byte bank sweep (1, 2 or 4
    // of them) keep their natural order and the next rows are XORed apart
    __device__ static int kswz(int r) { return (r / (256 / (HD * 2))) & (CPR - 1); }
    __device__ static int k8swz(int r) { return (r / (256 / HD)) & (C8PR - 1); }
    __device__ static int vswz(int r) { return HD == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

template <int HD>
struct Lds {
    static constexpr int KP = HD + 8;            // fp16 elements per K row
    static constexpr int VTP = BN + 8;           // fp16 elements per V^T row
    static constexpr int K8P = HD + 16;          // bytes per INT8 K row
    static constexpr int KBYTES = BN * KP * 2;
    static constexpr int K8BYTES = BN * K8P;
    static constexpr int KREG = KBYTES > K8BYTES ? KBYTES : K8BYTES;
    static constexpr int VBYTES = HD * VTP * 2;
    static constexpr int SCL = 2 * BN * 4;
    static constexpr int STAGE = KREG + VBYTES + SCL;
    static constexpr int TOTAL = 2 * STAGE;
};


// ---------------------------------------------------------------------------
// Fused forward kernel.
// ---------------------------------------------------------------------------
template <int HD, int NW, int KS, bool CAUSAL, bool VARLEN, bool ROUTED, bool KV8, bool FP8>
__global__ __launch_bounds__(NW * KS * 64, (NW == 2 && KS == 2) ? 2 : (NW != 4 || KS > 1) ? 1 : (BN == 32 ? 3 : 2))
void attn_fwd_kernel(FwdArgs a) {
    using L = Lds<HD>;
    constexpr int NT = NW * 64;                        // threads of one key group
    constexpr int KTOT = BN * HD / 8;                  // 16-byte fp16 K chunks per tile
    constexpr int K8TOT = BN * HD / 16;                // 16-byte INT8 K chunks per tile
    constexpr int KCH = (KTOT + NT - 1) / NT;          // ... per thread
    constexpr int K8CH = (K8TOT + NT - 1) / NT;
    constexpr int VBLK = (BN / 4) * (HD / 8);          // 4-key x 8-d V blocks per tile
    constexpr int VB = (VBLK + NT - 1) / NT;           // V blocks per thread
    constexpr int NDB = HD / 32;                       // 32-row blocks of d in O^T
    // four LDS stages and tiles stored two ahead: a barrier every other tile
    constexpr int NST = n_stages(NW, KS, ROUTED);
    // tiles loaded straight into LDS (layout: LdsDma)
    constexpr bool DMA = use_dma(HD, NW, KS, ROUTED, KV8);
    static_assert(!DMA || (NW >= 2 && (HD == 128 || HD == 64) && BN == 64), "direct-load shape");
    // Tiles in flight ahead of the one computed, on the register path.  Two
    // need a second staging set, which only the hdim-64 FP16 kernel has
    // registers for.
    constexpr int PF = (HD == 64 && !ROUTED && !KV8 && NW == 4 && BN == 64 && !DMA) ? 2 : 1;
    using DG = LdsDma<HD>;
    constexpr int STG = DMA ? LdsDma<HD>::STAGE : L::STAGE;     // bytes of one stage
    constexpr int KRG = DMA ? LdsDma<HD>::KREG : L::KREG;       // V tile offset in a stage
    constexpr int VBY = DMA ? LdsDma<HD>::VBYTES : L::VBYTES;   // scales follow the V tile
    // Request all of a tile's K and V fragments before its first MFMA (the
    // hdim-64 kernel has the registers for them).
    constexpr bool EARLY = (HD == 64);

    extern __shared__ __attribute__((aligned(16))) char smem[];

    // KS key groups of NW wavefronts: every group owns the same query rows and
    // takes every KS-th key tile; their softmax states merge at the end.
    // (wave-uniform values go through readfirstlane so that the compiler keeps
    // them, and the buffer offsets derived from them, in scalar registers)
    const int kgp = __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT);
    const int tid = (int)threadIdx.x % NT;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int g = l >> 5;
    const int lq = l & 31;
    const int HPW = a.HPW;
    const int BM = (NW / HPW) * 32;

    // ---- work decomposition -------------------------------------------------
    const int combo = blockIdx.x % a.combos;
    const int split = (blockIdx.x / a.combos) % a.ksplit;
    const int rank = blockIdx.x / (a.combos * a.ksplit);
    const int hpc = a.G / HPW;
    const int hsub = combo % hpc;
    const int hk = (combo / hpc) % a.n_kvh;
    const int h = hk * a.G + hsub * HPW + (w % HPW);

    int mb, Lq, Lk;
    int rrow0 = 0;                  // first routing-bitmask row of this sequence
    size_t qrow0, krow0;            // row index of row 0 of (sequence, head) in q / k
    if constexpr (VARLEN) {
        int t = rank, s = -1;
        mb = 0;
        for (int ss = a.B - 1; ss >= 0; --ss) {
            int Ls = a.cu[ss + 1] - a.cu[ss];
            int nb = (Ls + BM - 1) / BM;
            if (t < nb) { s = ss; mb = nb - 1 - t; break; }
            t -= nb;
        }
        if (s < 0) return;          // uniform for the workgroup, before any barrier
        const int start = a.cu[s];
        const int T = a.cu[a.B];
        Lq = Lk = a.cu[s + 1] - start;
        qrow0 = (size_t)h * T + start;
        krow0 = (size_t)hk * T + start;
        if constexpr (ROUTED) {
            // sequences stack their own query-tile rows in order
            for (int ss = 0; ss < s; ++ss) rrow0 += (a.cu[ss + 1] - a.cu[ss] + TQ - 1) / TQ;
        }
    } else {
        const int b = combo / (hpc * a.n_kvh);
        const int half = a.n_mblk / 2;
        mb = !CAUSAL ? rank : (a.pair_blocks && rank >= half) ? rank - half : a.n_mblk - 1 - rank;
        Lq = a.qsl;
        Lk = a.ksl;
        qrow0 = ((size_t)b * a.n_qh + h) * Lq;
        krow0 = ((size_t)b * a.n_kvh + hk) * Lk;
    }
    const _Float16* qb = a.q + qrow0 * HD;
    _Float16* ob = a.out + qrow0 * HD;
    const _Float16* kb = a.k + krow0 * HD;
    const _Float16* vb = a.v + krow0 * HD;
    const int8_t* k8b = (ROUTED || KV8) ? a.k8 + krow0 * HD : nullptr;
    const float* skb = (ROUTED || KV8) ? a.sk + krow0 : nullptr;
    const int8_t* v8b = KV8 ? a.v8 + krow0 * HD : nullptr;
    const float* svb = KV8 ? a.sv + krow0 : nullptr;

    const int off = CAUSAL ? (Lk - Lq) : 0;     // bottom-right alignment
    const int m0 = mb * BM;
    const int r0 = m0 + (w / HPW) * 32;          // first row of this wavefront
    const int n_kt = (Lk + BN - 1) / BN;
    const int wg_last = min(m0 + BM, Lq) - 1;
    const int nkt = CAUSAL ? min(n_kt, (wg_last + off) / BN + 1) : n_kt;
    const bool wave_active = r0 < Lq;
    const int w_nkt = !wave_active ? 0
                    : CAUSAL ? min(n_kt, (min(r0 + 31, Lq - 1) + off) / BN + 1) : n_kt;

    // this workgroup's row of the routing bitmask (one 64-row query tile)
    const uint32_t* rrow = ROUTED ? a.route + (size_t)(rrow0 + m0 / TQ) * a.wpr : nullptr;

    // ---- query rows into the score B-operand layout ---------------------------
    const int qi = r0 + lq;
    f16x8 qf[HD / 16];
    {
        // rows past the end read the last row (finite values, never stored)
        const _Float16* qp = qb + (size_t)min(qi, Lq - 1) * HD + 16 * g;
#pragma unroll
        for (int kb2 = 0; kb2 < HD / 32; ++kb2) {
            qf[2 * kb2] = *(const f16x8*)(qp + 32 * kb2);
            qf[2 * kb2 + 1] = *(const f16x8*)(qp + 32 * kb2 + 8);
        }
    }

    i32x4 q8[ROUTED ? HD / 32 : 1];     // INT8 query codes (routed), set after the prologue wait
    float sq_mul = 1.0f;
    // INT8 value cache: the value scales enter the staged V relative to a
    // power of two (vfac = 2^-e, with 2^e near the largest scale of the
    // workgroup's key range), which the epilogue multiplies back (vfac_inv,
    // exact)
    float vfac = 1.0f, vfac_inv = 1.0f;
    // INT8 key cache, FP16 tiles: the key scales enter the staged K likewise
    // (kfac), and the scores are multiplied back by kfac_inv (exact)
    float kfac = 1.0f, kfac_inv = 1.0f;

    // ---- tile loader ------------------------------------------------------------
    // Register path (gload / lstore; the direct loads are `dma` below).
    // K: 16-byte chunks of rows.  V: per thread a block of 4 keys x 8 d, read as
    // four 16-byte row pieces and written transposed as eight 8-byte pieces.
    // Loads go through buffer resources covering one tile and the rest of this
    // sequence's rows (tile_rsrc): reads past the last key return zeros
    // (those keys are masked to -inf, so P is exactly 0 there), and the
    // per-lane offsets are loop invariant, so nothing in the loop waits on
    // the loads of the next tile before its LDS store.
    const int slab = Lk * HD * 2;
    constexpr int TB16 = BN * HD * 2;     // bytes of an fp16 K or V tile
    constexpr int TB8 = BN * HD;          // bytes of an INT8 K or V tile
    constexpr int TBS = BN * 4;           // bytes of a tile's per-key scales
    // Staging registers of one tile between its global loads and its LDS
    // store.  With PF = 2 two sets alternate, so the loads of tile t+2 are
    // issued while tile t is computed and have two tiles' time to land.
    struct Staging {
        u32x4 kreg[KCH];
        u32x4 vreg[VB][4];
        u32x2 v8reg[VB][4];     // INT8 V cache: 8 codes of each of 4 keys
        u32x4 svk[VB];          // ... and the scales of those 4 keys
        float skrow[K8CH];      // INT8 K cache, FP16 tiles: the scale of each chunk's key
        u32x4 skreg;
    };
    // The two-set pipeline waits for the older set with a load count, so every
    // lane issues the same number of loads: the first half of the waves loads
    // the V tile (one 4-key x 8-d block per thread), the second half the K tile
    // (four 16-byte chunks per thread), four loads each, unconditionally
    // (loads past the sequence end return zeros and are never used).
    struct Staging2 {
        u32x4 r[4];
    };
    using Set = typename std::conditional<PF == 2, Staging2, Staging>::type;
    Set set0, set1;
    const bool v_half = w < NW / 2;
    const int th = tid % (NT / 2);

    // Branch-free loads (descriptor picked per wave, offsets per lane) so the
    // wait-count analysis sees one straight path.
    static_assert(PF == 1 || ((BN / 4) * (HD / 8) == NT / 2 && BN * HD / 8 == 4 * (NT / 2)),
                  "balanced loader shape");
    const _Float16* base2 = v_half ? vb : kb;
    int voff2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        voff2[i] = v_half ? ((4 * (th % (BN / 4)) + i) * HD + 8 * (th / (BN / 4))) * 2
                          : (th + i * (NT / 2)) * 16;
    auto gload2 = [&](Staging2& sg, int kt) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs2 = tile_rsrc(base2, slab, TB16, kt);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sg.r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs2, voff2[i], 0, 0));
    };
    auto lstore2 = [&](const Staging2& sg, int stage) __attribute__((always_inline)) {
        char* kbuf = smem + (stage * KS + kgp) * STG;
        if (v_half) {
            _Float16* vt = (_Float16*)(kbuf + L::KREG);
            const int kg = th % (BN / 4), dc = th / (BN / 4);
            _Float16* dst = vt + (8 * dc) * L::VTP + 4 * kg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                *(u32x2*)(dst + (2 * j) * L::VTP) =
                    u32x2{__builtin_amdgcn_perm(sg.r[1][j], sg.r[0][j], 0x05040100u),
                          __builtin_amdgcn_perm(sg.r[3][j], sg.r[2][j], 0x05040100u)};
                *(u32x2*)(dst + (2 * j + 1) * L::VTP) =
                    u32x2{__builtin_amdgcn_perm(sg.r[1][j], sg.r[0][j], 0x07060302u),
                          __builtin_amdgcn_perm(sg.r[3][j], sg.r[2][j], 0x07060302u)};
            }
        } else {
            _Float16* k16 = (_Float16*)kbuf;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int c = th + n * (NT / 2);
                *(u32x4*)(k16 + (c / (HD / 8)) * L::KP + (c % (HD / 8)) * 8) = sg.r[n];
            }
        }
    };

    auto gload = [&](Staging& sg, int kt, bool i8) __attribute__((always_inline)) {
        u32x4(&kreg)[KCH] = sg.kreg;
        u32x4(&vreg)[VB][4] = sg.vreg;
        u32x4& skreg = sg.skreg;
        if (KV8 || (ROUTED && i8 && !ATTN_FUSED_KQUANT)) {
            const __amdgpu_buffer_rsrc_t k8rs = tile_rsrc(k8b, Lk * HD, TB8, kt);
#pragma unroll
            for (int n = 0; n < K8CH; ++n) {
                const int c = tid + n * NT;     // row c / (HD/16), 16-byte column c % (HD/16)
                if (K8TOT % NT == 0 || c < K8TOT)
                    kreg[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(k8rs, c * 16, 0, 0));
            }
            const __amdgpu_buffer_rsrc_t skrs = tile_rsrc(skb, Lk * 4, TBS, kt);
            if (KV8 && !i8) {
                // FP16 tiles of a key cache: the scale of each chunk's key (the
                // staged tile holds code * s_k * kfac)
#pragma unroll
                for (int n = 0; n < K8CH; ++n) {
                    const int c = tid + n * NT;
                    if (K8TOT % NT == 0 || c < K8TOT)
                        sg.skrow[n] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                            skrs, (c / (HD / 16)) * 4, 0, 0));
                }
            } else if (tid < BN / 4) {
                skreg = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(skrs, tid * 16, 0, 0));
            }
        } else {
            const __amdgpu_buffer_rsrc_t krs = tile_rsrc(kb, slab, TB16, kt);
#pragma unroll
            for (int n = 0; n < KCH; ++n) {
                const int c = tid + n * NT;     // row c / (HD/8), 16-byte column c % (HD/8)
                if (KTOT % NT == 0 || c < KTOT)
                    kreg[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, c * 16, 0, 0));
            }
        }
        if constexpr (KV8) {
            const __amdgpu_buffer_rsrc_t v8rs = tile_rsrc(v8b, Lk * HD, TB8, kt);
            const __amdgpu_buffer_rsrc_t svrs = tile_rsrc(svb, Lk * 4, TBS, kt);
#pragma unroll
            for (int n = 0; n < VB; ++n) {
                const int bi = tid + n * NT;
                if (VBLK % NT == 0 || bi < VBLK) {
                    const int kg = bi % (BN / 4);
                    const int dc = bi / (BN / 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sg.v8reg[n][i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                            v8rs, (4 * kg + i) * HD + 8 * dc, 0, 0));
                    sg.svk[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(svrs, kg * 16, 0, 0));
                }
            }
        } else {
            const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(vb, slab, TB16, kt);
#pragma unroll
            for (int n = 0; n < VB; ++n) {
                const int bi = tid + n * NT;
                if (VBLK % NT == 0 || bi < VBLK) {
                    const int kg = bi % (BN / 4);
                    const int dc = bi / (BN / 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vreg[n][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                            vrs, ((4 * kg + i) * HD + 8 * dc) * 2, 0, 0));
                }
            }
        }
    };

    auto lstore = [&](const Staging& sg, int stage, bool i8) __attribute__((always_inline)) {
        const u32x4(&kreg)[KCH] = sg.kreg;
        const u32x4(&vreg)[VB][4] = sg.vreg;
        const u32x4& skreg = sg.skreg;
        char* kbuf = smem + (stage * KS + kgp) * STG;
        _Float16* vt = (_Float16*)(kbuf + L::KREG);
        float* scl = (float*)(kbuf + L::KREG + L::VBYTES);
        if (((KV8 && i8) || (ROUTED && i8 && !ATTN_FUSED_KQUANT)) && tid < BN / 4)
            *(f32x4*)(scl + 4 * tid) = __builtin_bit_cast(f32x4, skreg) * a.c;
        if (ROUTED && i8 && !KV8 && ATTN_FUSED_KQUANT) {
            // the fp16 K tile quantised here: the HD/8 consecutive lanes that
            // hold one row share its absolute maximum, then each codes its 8
            // values with the rule of the per-call pass (same functions)
#pragma unroll
            for (int n = 0; n < KCH; ++n) {
                const int c = tid + n * NT;
                const int row = c / (HD / 8);
                const int part = c % (HD / 8);
                const f16x8 xv = __builtin_bit_cast(f16x8, kreg[n]);
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)xv[j]));
#pragma unroll
                for (int o = 1; o < HD / 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
                float sc, inv;
                unsigned w0 = 0, w1 = 0;
                if constexpr (FP8) {
                    fp8_scale(amax, sc, inv);
                    w0 = fp8_pack4(fp8_round((float)xv[0], inv), fp8_round((float)xv[1], inv),
                                   fp8_round((float)xv[2], inv), fp8_round((float)xv[3], inv));
                    w1 = fp8_pack4(fp8_round((float)xv[4], inv), fp8_round((float)xv[5], inv),
                                   fp8_round((float)xv[6], inv), fp8_round((float)xv[7], inv));
                } else {
                    quant_scale(amax, sc, inv);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w0 |= ((unsigned)quant_code((float)xv[j], inv) & 0xffu) << (8 * j);
                        w1 |= ((unsigned)quant_code((float)xv[4 + j], inv) & 0xffu) << (8 * j);
                    }
                }
                if (KTOT % NT == 0 || c < KTOT) {
                    *(u32x2*)(kbuf + row * L::K8P + part * 8) = u32x2{w0, w1};
                    if (part == 0) scl[row] = sc * a.c;
                }
            }
        } else if (ROUTED && i8) {
#pragma unroll
            for (int n = 0; n < K8CH; ++n) {
                const int c = tid + n * NT;
                const int row = c / (HD / 16);
                const int col = (c % (HD / 16)) * 16;
                if (K8TOT % NT == 0 || c < K8TOT) *(u32x4*)(kbuf + row * L::K8P + col) = kreg[n];
            }
        } else if (KV8) {
            // FP16 route on an INT8 key cache: the codes widened to fp16 (exact)
            // and scaled per key (below)
            _Float16* k16 = (_Float16*)kbuf;
#pragma unroll
            for (int n = 0; n < K8CH; ++n) {
                const int c = tid + n * NT;
                const int row = c / (HD / 16);
                const int col = (c % (HD / 16)) * 16;
                if (K8TOT % NT == 0 || c < K8TOT) {
                    // widened codes times the key's scale times kfac, in fp16
                    // (the products stay below 2^8)
                    const float ks = sg.skrow[n] * kfac;
                    const f16x2 h = {(_Float16)ks, (_Float16)ks};
                    // (one product per widened word: a u32x2 built from two f16x2
                    // products in one expression came out as the first product twice)
                    auto mul = [&](unsigned w) { return __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, w) * h); };
                    auto wide = [&](unsigned w) __attribute__((always_inline)) {
                        const u32x2 p2 = widen_i8x4(w);
                        return u32x2{mul(p2[0]), mul(p2[1])};
                    };
                    const u32x2 w0 = wide(kreg[n][0]), w1 = wide(kreg[n][1]);
                    const u32x2 w2 = wide(kreg[n][2]), w3 = wide(kreg[n][3]);
                    *(u32x4*)(k16 + row * L::KP + col) = u32x4{w0[0], w0[1], w1[0], w1[1]};
                    *(u32x4*)(k16 + row * L::KP + col + 8) = u32x4{w2[0], w2[1], w3[0], w3[1]};
                }
            }
        } else {
            _Float16* k16 = (_Float16*)kbuf;
#pragma unroll
            for (int n = 0; n < KCH; ++n) {
                const int c = tid + n * NT;
                const int row = c / (HD / 8);
                const int col = (c % (HD / 8)) * 8;
                if (KTOT % NT == 0 || c < KTOT) *(u32x4*)(k16 + row * L::KP + col) = kreg[n];
            }
        }
#pragma unroll
        for (int n = 0; n < VB; ++n) {
            const int bi = tid + n * NT;
            if (VBLK % NT == 0 || bi < VBLK) {
                const int kg = bi % (BN / 4);
                const int dc = bi / (BN / 4);
                u32x4 r0w = vreg[n][0], r1w = vreg[n][1], r2w = vreg[n][2], r3w = vreg[n][3];
                if constexpr (KV8) {
                    // INT8 value cache: each key's row of 8 codes widened to
                    // fp16 (exact) and multiplied by the key's scale times
                    // vfac, rounded to fp16 (the products stay below 2^8)
                    const f32x4 sv4 = __builtin_bit_cast(f32x4, sg.svk[n]) * vfac;
                    auto row8 = [](u32x2 c, float sv) __attribute__((always_inline)) {
                        const u32x2 a0 = widen_i8x4(c[0]), a1 = widen_i8x4(c[1]);
                        const f16x2 h = {(_Float16)sv, (_Float16)sv};
                        auto mul = [&](unsigned w) { return __builtin_bit_cast(unsigned, __builtin_bit_cast(f16x2, w) * h); };
                        return u32x4{mul(a0[0]), mul(a0[1]), mul(a1[0]), mul(a1[1])};
                    };
                    r0w = row8(sg.v8reg[n][0], sv4[0]);
                    r1w = row8(sg.v8reg[n][1], sv4[1]);
                    r2w = row8(sg.v8reg[n][2], sv4[2]);
                    r3w = row8(sg.v8reg[n][3], sv4[3]);
                }
                _Float16* dst = vt + (8 * dc) * L::VTP + 4 * kg;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // d = 8*dc + 2j takes the low halves, d + 1 the high halves
                    *(u32x2*)(dst + (2 * j) * L::VTP) =
                        u32x2{__builtin_amdgcn_perm(r1w[j], r0w[j], 0x05040100u),
                              __builtin_amdgcn_perm(r3w[j], r2w[j], 0x05040100u)};
                    *(u32x2*)(dst + (2 * j + 1) * L::VTP) =
                        u32x2{__builtin_amdgcn_perm(r1w[j], r0w[j], 0x07060302u),
                              __builtin_amdgcn_perm(r3w[j], r2w[j], 0x07060302u)};
                }
            }
        }
    };

    // Direct tile loads (DMA kernels): each wavefront of the key group writes
    // whole 1 KB LDS blocks, 64 lanes x 16 bytes in lane order; each lane
    // fetches the global chunk that the swizzled layout puts at its slot.
    // fp16 K and V: 16 blocks of 4 rows each; INT8/FP8 codes: 8 blocks of 8
    // rows; block b goes to wavefront b % NW.  The 64 key scales (4 bytes a
    // lane) come with wavefront 0.  Reads past the sequence end return zeros, as above.
    auto dma = [&](int kt, int stage, bool i8) __attribute__((always_inline)) {
        if constexpr (DMA) {
            char* base = smem + (stage * KS + kgp) * STG;
            if (ROUTED && i8) {
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(k8b, Lk * HD, TB8, kt);
#pragma unroll
                for (int i = 0; i < (DG::K8BLK + NW - 1) / NW; ++i) {
                    const int blk = w + NW * i;
                    const int row = DG::K8RPB * blk + l / DG::C8PR;
                    const int c = (l % DG::C8PR) ^ DG::k8swz(row);
                    if (DG::K8BLK % NW == 0 || blk < DG::K8BLK)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, base + blk * 1024), 16,
                                                                 row * HD + c * 16, 0, 0, 0);
                }
                if (w == 0) {
                    const __amdgpu_buffer_rsrc_t ss = tile_rsrc(skb, Lk * 4, TBS, kt);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ss, LDS_PTR(void, base + KRG + VBY), 4, l * 4, 0, 0, 0);
                }
            } else {
                const __amdgpu_buffer_rsrc_t rs = tile_rsrc(kb, slab, TB16, kt);
#pragma unroll
                for (int i = 0; i < (DG::KBLK + NW - 1) / NW; ++i) {
                    const int blk = w + NW * i;
                    const int row = DG::KRPB * blk + l / DG::CPR;
                    const int c = (l % DG::CPR) ^ DG::kswz(row);
                    if (DG::KBLK % NW == 0 || blk < DG::KBLK)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, base + blk * 1024), 16,
                                                                 row * (HD * 2) + c * 16, 0, 0, 0);
                }
            }
            const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(vb, slab, TB16, kt);
#pragma unroll
            for (int i = 0; i < (DG::KBLK + NW - 1) / NW; ++i) {
                const int blk = w + NW * i;
                const int row = DG::KRPB * blk + l / DG::CPR;
                const int c = (l % DG::CPR) ^ DG::vswz(row);
                if (DG::KBLK % NW == 0 || blk < DG::KBLK)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, LDS_PTR(void, base + KRG + blk * 1024), 16,
                                                             row * (HD * 2) + c * 16, 0, 0, 0);
            }
        }
    };
    // every wave's direct loads complete, then the barrier
    auto dsync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    // ---- state --------------------------------------------------------------------
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float m_run = M_INIT;
    float l_run = 0.0f;

    // K row read by this lane for the score A operand: bits 2 and 3 swapped
    const int krow = (lq & ~12) | ((lq & 4) << 1) | ((lq & 8) >> 1);
    // Operand read offsets in a directly loaded stage (swizzles of LdsDma):
    // koff[t]: the fp16 K fragment of d-step t (chunk 2g + 4(t/2) + t%2) of
    // row krow; k8off[j]: the 16-byte code chunk g + 2j of row krow; voff[db]:
    // this lane's 8-byte source of the transposed V reads of d block db,
    // key 8*(l/32) + (l%16)/4 (+4 for the second read), d 32db + 16*((l/16)%2)
    // + 4*(l%4): within 16 lanes, transposed lane 4a + b takes element b of
    // source lane 4j + a as its element j, so lane l ends up with d = l % 32
    // and the 4 consecutive keys of each read.
    int koff[DMA ? HD / 16 : 1], k8off[DMA ? HD / 32 : 1], voff[DMA ? NDB : 1];
    if constexpr (DMA) {
        // rows 32*kb32 + krow share the swizzle of krow (32 is a multiple of
        // every swizzle period)
#pragma unroll
        for (int t = 0; t < HD / 16; ++t)
            koff[t] = krow * (HD * 2) + (((2 * g + 4 * (t / 2) + (t % 2)) ^ DG::kswz(krow)) << 4);
#pragma unroll
        for (int j = 0; j < HD / 32; ++j) k8off[j] = krow * HD + (((g + 2 * j) ^ DG::k8swz(krow)) << 4);
        const int q4 = (l >> 2) & 3;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            voff[db] = (8 * (l >> 5) + q4) * (HD * 2) +
                       (((4 * db + 2 * ((l >> 4) & 1) + ((l & 3) >> 1)) ^ DG::vswz(q4)) << 4) + 8 * (l & 1);
    }

    // One key tile: scores, optional mask, online softmax, P.V.
    auto tile = [&](auto mask_tag, int stage, int kt, bool i8) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const char* kbuf = smem + (stage * KS + kgp) * STG;
        const _Float16* vt = (const _Float16*)(kbuf + KRG);
        float x[NKB][16];
        float amul;
        f16x8 vfr[EARLY ? 2 * NKB : 1][EARLY ? NDB : 1];   // V fragments requested with K
        // per-key scales of the tile (INT8 tiles, key/value caches)
        const float* skc = (const float*)(kbuf + KRG + VBY);
        // x[kb32][i] *= the scale of its key: this lane's keys are
        // 32*kb32 + 8*g + (i%8) + 16*(i/8)
        auto key_scale = [&](int kb32) __attribute__((always_inline)) {
            const float* sp = skc + 32 * kb32 + 8 * g;
            const f32x4 s0 = *(const f32x4*)(sp);
            const f32x4 s1 = *(const f32x4*)(sp + 4);
            const f32x4 s2 = *(const f32x4*)(sp + 16);
            const f32x4 s3 = *(const f32x4*)(sp + 20);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[kb32][i] *= s0[i];
                x[kb32][4 + i] *= s1[i];
                x[kb32][8 + i] *= s2[i];
                x[kb32][12 + i] *= s3[i];
            }
        };
        if (ROUTED && i8 && FP8) {
            // v_mfma_f32_32x32x64_f8f6f4 with both formats e4m3 and no block
            // scales; operand k = 64 values = the INT8 operands 2k and 2k+1
#pragma unroll
            for (int kb32 = 0; kb32 < NKB; ++kb32) {
                f32x16 acc = f32x16{};
                const int8_t* kr = (const int8_t*)kbuf + (32 * kb32 + krow) * L::K8P + 16 * g;
                const char* kd = kbuf + 32 * kb32 * HD;
#pragma unroll
                for (int k2 = 0; k2 < HD / 64; ++k2) {
                    const i32x4 a0 = DMA ? *(const i32x4*)(kd + k8off[DMA ? 2 * k2 : 0]) : *(const i32x4*)(kr + 64 * k2);
                    const i32x4 a1 = DMA ? *(const i32x4*)(kd + k8off[DMA ? 2 * k2 + 1 : 0])
                                         : *(const i32x4*)(kr + 64 * k2 + 32);
                    const i32x8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    const i32x4 b0 = q8[2 * k2], b1 = q8[2 * k2 + 1];
                    const i32x8 bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) x[kb32][i] = acc[i];
                key_scale(kb32);
            }
            // direct loads keep the raw key scales: |scale|*log2(e) joins sq here
            amul = DMA ? sq_mul * a.c : sq_mul;
        } else if (ROUTED && i8) {
#pragma unroll
            for (int kb32 = 0; kb32 < NKB; ++kb32) {
                i32x16 acc = i32x16{};
                const int8_t* kr = (const int8_t*)kbuf + (32 * kb32 + krow) * L::K8P + 16 * g;
                const char* kd = kbuf + 32 * kb32 * HD;
#pragma unroll
                for (int ks = 0; ks < HD / 32; ++ks) {
                    i32x4 av = DMA ? *(const i32x4*)(kd + k8off[DMA ? ks : 0]) : *(const i32x4*)(kr + 32 * ks);
                    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, q8[ks], acc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) x[kb32][i] = (float)acc[i];
                key_scale(kb32);
            }
            // direct loads keep the raw key scales: |scale|*log2(e) joins sq here
            amul = DMA ? sq_mul * a.c : sq_mul;
        } else {
            const _Float16* k16 = (const _Float16*)kbuf;
            if constexpr (EARLY) {
                // every K and V fragment of the tile is requested up front: the
                // K reads land back to back for the score MFMAs and the V reads
                // land under the softmax instead of in front of each MFMA
                f16x8 kfr[NKB][HD / 16];
#pragma unroll
                for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
                    for (int t = 0; t < HD / 16; ++t)
                        kfr[kb32][t] = DMA ? *(const f16x8*)(kbuf + 32 * kb32 * (HD * 2) + koff[DMA ? t : 0])
                                           : *(const f16x8*)(k16 + (32 * kb32 + krow) * L::KP + 16 * g +
                                                             32 * (t / 2) + 8 * (t % 2));
                if constexpr (DMA) {
                    static_assert(NDB == 2, "up-front transposed reads: two d blocks");
                    // two 16-key steps per asm block: fragments (kk, 0), (kk, 1),
                    // (kk + 1, 0), (kk + 1, 1)
#pragma unroll
                    for (int kk = 0; kk < 2 * NKB; kk += 2) {
                        const unsigned va = lds_addr(vt) + kk * 16 * (HD * 2);
                        const unsigned vb2 = va + 16 * (HD * 2);
                        f16x8 fr[4];
                        lds_read_tr16_x4<4 * (HD * 2)>(va + voff[0], va + voff[DMA ? 1 : 0], vb2 + voff[0],
                                                       vb2 + voff[DMA ? 1 : 0], fr);
                        vfr[kk][0] = fr[0];
                        vfr[kk][DMA ? 1 : 0] = fr[1];
                        vfr[kk + 1][0] = fr[2];
                        vfr[kk + 1][DMA ? 1 : 0] = fr[3];
                    }
                } else {
                    const _Float16* vrow = vt + lq * L::VTP + 8 * g;
#pragma unroll
                    for (int kk = 0; kk < 2 * NKB; ++kk)
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            vfr[kk][db] = *(const f16x8*)(vrow + (32 * db) * L::VTP + 16 * kk);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb32 = 0; kb32 < NKB; ++kb32) {
                    f32x16 acc = f32x16{};
#pragma unroll
                    for (int t = 0; t < HD / 16; ++t)
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfr[kb32][t], qf[t], acc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i) x[kb32][i] = acc[i];
                }
            } else {
#pragma unroll
                for (int kb32 = 0; kb32 < NKB; ++kb32) {
                    f32x16 acc = f32x16{};
                    const _Float16* kr = k16 + (32 * kb32 + krow) * L::KP + 16 * g;
                    const char* kd = kbuf + 32 * kb32 * (HD * 2);
#pragma unroll
                    for (int t = 0; t < HD / 16; ++t) {
                        const f16x8 av = DMA ? *(const f16x8*)(kd + koff[DMA ? t : 0])
                                             : *(const f16x8*)(kr + 32 * (t / 2) + 8 * (t % 2));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qf[t], acc, 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) x[kb32][i] = acc[i];
                }
            }
            // on a key cache the staged keys are code * s_k * kfac (kfac a power of two)
            amul = KV8 ? a.c * kfac_inv : a.c;

        }

        if constexpr (MASK) {
            // keys past the end and the bottom-right causal boundary
            const int lim = CAUSAL ? min(Lk - 1, qi + off) : Lk - 1;
            const int kl = kt * BN + 8 * g;
#pragma unroll
            for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kl + 32 * kb32 + (i % 8) + 16 * (i / 8) > lim) x[kb32][i] = -INFINITY;
        }

        // O^T += V^T P^T over the two 16-key steps of one 32-key block
        const _Float16* vrow = vt + lq * L::VTP + 8 * g;
        auto pv = [&](int kb32, const f16x8(&pkb)[2]) __attribute__((always_inline)) {
            if constexpr (DMA && NDB == 2) {
                // keys 16kk + 8(l/32) + 0..7 of d = 32db + l%32 for both 16-key
                // steps of the block (already read when up front)
                f16x8 fr[4];
                if (EARLY && !(ROUTED && i8)) {
                    fr[0] = vfr[2 * kb32][0];
                    fr[1] = vfr[2 * kb32][EARLY ? 1 : 0];
                    fr[2] = vfr[EARLY ? 2 * kb32 + 1 : 0][0];
                    fr[3] = vfr[EARLY ? 2 * kb32 + 1 : 0][EARLY ? 1 : 0];
                } else {
                    const unsigned va = lds_addr(vt) + 2 * kb32 * 16 * (HD * 2);
                    const unsigned vb2 = va + 16 * (HD * 2);
                    lds_read_tr16_x4<4 * (HD * 2)>(va + voff[0], va + voff[DMA ? 1 : 0], vb2 + voff[0],
                                                   vb2 + voff[DMA ? 1 : 0], fr);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int db = 0; db < 2; ++db)
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[2 * t + db], pkb[t], o[db], 0, 0, 0);
                return;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int kk = 2 * kb32 + t;
                if constexpr (DMA) {
                    // keys 16kk + 8(l/32) + 0..7 of d = 32db + l%32, every db
                    const unsigned va = lds_addr(vt) + kk * 16 * (HD * 2);
                    f16x8 fr[4];
                    lds_read_tr16_x4<4 * (HD * 2)>(va + voff[0], va + voff[DMA && NDB == 4 ? 1 : 0],
                                                   va + voff[DMA && NDB == 4 ? 2 : 0],
                                                   va + voff[DMA && NDB == 4 ? 3 : 0], fr);
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[db], pkb[t], o[db], 0, 0, 0);
                } else {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const f16x8 av = (EARLY && !(ROUTED && i8)) ? vfr[kk][db]
                                                                     : *(const f16x8*)(vrow + (32 * db) * L::VTP + 16 * kk);
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pkb[t], o[db], 0, 0, 0);
                    }
                }
            }
        };

        // online softmax in base 2 with a lazily moved reference max
        float mt = -INFINITY;
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
            for (int i = 0; i < 16; ++i) mt = fmaxf(mt, x[kb32][i]);
        mt = halfwave_max(mt) * amul;
        if (__any(mt > m_run + TAU)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        }
        const float nm = -m_run;
        f16x8 pk[NKB][2];
        float rs = 0.0f;
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb32][8 * t + j], amul, nm));
                    rs += p;
                    pk[kb32][t][j] = (_Float16)p;
                }
            }
        l_run += rs;
#pragma unroll
        for (int kb32 = 0; kb32 < NKB; ++kb32) pv(kb32, pk[kb32]);
    };

    // Tiles [0, nfull) are fully visible to every row of the workgroup; the
    // rest (the causal diagonal and a partial last tile) go through the
    // masked variant.  Two loops keep the two variants' live ranges apart.
    const int nfull = min(nkt, min(Lk / BN, CAUSAL ? (m0 + off + 1) / BN : nkt));
    // this workgroup's share of the key tiles when the key range is split
    const int chunk = (nkt + a.ksplit - 1) / a.ksplit;
    const int kt0 = min(nkt, split * chunk);
    const int kt1 = min(nkt, kt0 + chunk);

    // Iteration it covers tiles kt0 + KS*it .. + KS-1, one per key group; the
    // first it_full iterations have every tile below nfull.  Tile it of this
    // group lives in LDS stage it % NST (and, on the register path, in
    // staging set it % PF).
    const int n_it = (kt1 - kt0 + KS - 1) / KS;
    const int it_full = max(0, (min(nfull, kt1) - kt0) / KS);
    const int kt_first = kt0 + kgp;
    auto has = [&](int it) __attribute__((always_inline)) { return it < n_it && kt_first + KS * it < kt1; };

    const int kt_end = min(w_nkt, kt1);

    if constexpr (KV8) {
        // The value-cache scales multiply the widened codes as the V tile is
        // staged (one fp16 product per value, once per workgroup), first
        // brought to [1, 2) at their largest by an exact power of two:
        // code * s_v * vfac stays below 2^8 (no overflow for any scale), and
        // keys whose scale is near the largest keep full fp16 precision
        // whatever the value magnitude (no subnormal values).  The key-cache
        // scales of FP16 tiles are normalised the same way.
        float mx = 0.0f, mk = 0.0f;
        const int j1 = min(kt1 * BN, Lk);
        for (int j = kt0 * BN + (int)threadIdx.x; j < j1; j += NW * KS * 64) {
            mx = fmaxf(mx, fabsf(svb[j]));
            mk = fmaxf(mk, fabsf(skb[j]));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, o));
            mk = fmaxf(mk, __shfl_xor(mk, o));
        }
        float* red = (float*)smem;
        if ((threadIdx.x & 63) == 0) {
            red[2 * (threadIdx.x >> 6)] = mx;
            red[2 * (threadIdx.x >> 6) + 1] = mk;
        }
        __syncthreads();
        mx = 0.0f;
        mk = 0.0f;
#pragma unroll
        for (int i = 0; i < NW * KS; ++i) {
            mx = fmaxf(mx, red[2 * i]);
            mk = fmaxf(mk, red[2 * i + 1]);
        }
        __syncthreads();
        // a power of two f and its inverse with m * f in [1, 2) (1 and 1 for
        // a zero or non-finite m)
        auto pow2_norm = [](float m, float& f, float& f_inv) __attribute__((always_inline)) {
            const int e = (int)((u_from_f(m) >> 23) & 0xffu);    // biased exponent
            if (e != 0 && e != 255) {
                const int sh = max(-126, min(126, 127 - e));       // m * 2^sh in [1, 2)
                f = f_from_u((unsigned)(127 + sh) << 23);
                f_inv = f_from_u((unsigned)(127 - sh) << 23);
            }
        };
        pow2_norm(mx, vfac, vfac_inv);
        pow2_norm(mk, kfac, kfac_inv);

    }
    auto query_prologue = [&]() __attribute__((always_inline)) {
        if (a.neg) {
#pragma unroll
            for (int t = 0; t < HD / 16; ++t) qf[t] = -qf[t];
        }
    };
    if constexpr (ROUTED) {
        // Routed calls take their tiles in two passes, first every FP16 tile
        // and then every low-precision tile, each in key order, so that each
        // pass runs a loop body specialised for its route (the online-softmax
        // state does not depend on the order of the tiles).  The bitmask word
        // in use is cached; a new word is read every 32 groups.
        static_assert(KS == 1 && PF == 1 && BN == TK, "routed calls: one key group of 64-key tiles");
        RouteCursor cur(rrow, a.tiles_per_bit, kt1);
        // first tile >= t of this workgroup's range whose route is c, else kt1
        auto next_of = [&](int t, bool c) __attribute__((always_inline)) { return cur.next(t, c); };
        // test hook: count every tile the workgroup visits, by route
        uint32_t* const trace = a.trace ? a.trace + (size_t)(rrow0 + m0 / TQ) * a.trace_nkt : nullptr;
        if constexpr (DMA) {
        // Direct loads: each pass starts in stage 0 with its first tile
        // resident (and, with four stages, its second in flight), and loads
        // the tile two (one) ahead of the one it computes into the stage
        // freed two steps (one step) before.  The
        // steps of fully visible tiles are unrolled by four so that every
        // stage offset is a constant: the compiler then sees that the loads
        // in flight write other stages than the one read and waits for them
        // only at the barriers.  The last (masked) tiles of a pass use a
        // computed stage.
        auto dpass = [&](auto cls_tag, int kt) __attribute__((always_inline)) {
            constexpr bool C = decltype(cls_tag)::value;
            int kn = next_of(kt + 1, C);
            int kn2 = kn < kt1 ? next_of(kn + 1, C) : kt1;
            auto step = [&](auto mask_tag, int S) __attribute__((always_inline)) {
                constexpr bool MASK = decltype(mask_tag)::value;
                if (trace && tid == 0) atomicAdd(trace + kt, C ? 0x10000u : 1u);
                if constexpr (NST == 4) {
                    if (kn2 < kt1) dma(kn2, (S + 2) & 3, C);
                } else {
                    if (kn < kt1) dma(kn, S ^ 1, C);
                }
                if (MASK ? kt < kt_end : wave_active) tile(mask_tag, S, kt, C);
                if (NST == 2 || (S & 1)) dsync();
                kt = kn;
                kn = kn2;
                if (kn2 < kt1) kn2 = next_of(kn2 + 1, C);
            };
            const int full_end = min(nfull, kt1);
            int si = 0;
            while (true) {
                if (kt >= full_end) break;
                step(std::false_type{}, 0);
                si = 1 & (NST - 1);
                if (kt >= full_end) break;
                step(std::false_type{}, 1 & (NST - 1));
                si = 2 & (NST - 1);
                if (kt >= full_end) break;
                step(std::false_type{}, 2 & (NST - 1));
                si = 3 & (NST - 1);
                if (kt >= full_end) break;
                step(std::false_type{}, 3 & (NST - 1));
                si = 0;
            }
            while (kt < kt1) {
                step(std::true_type{}, si);
                si = (si + 1) & (NST - 1);
            }
            dsync();
        };
        int kt = next_of(kt0, false);
        int kt2 = kt < kt1 ? next_of(kt + 1, false) : kt1;
        if (kt < kt1) dma(kt, 0, false);
        if (NST == 4 && kt2 < kt1) dma(kt2, 1, false);
        query_prologue();
        dsync();
        dpass(std::false_type{}, kt);
        kt = next_of(kt0, true);
        kt2 = kt < kt1 ? next_of(kt + 1, true) : kt1;
        if (kt < kt1) {
            dma(kt, 0, true);
            if (NST == 4 && kt2 < kt1) dma(kt2, 1, true);
            float sq;
            quantize_q_regs<HD, FP8>(qf, q8, sq);
            sq_mul = sq > 0.0f ? sq : 1.0f;
            dsync();
            dpass(std::true_type{}, kt);
        }
        } else {
        int st = 0;
        // tiles [kt, kt1) of route C: the first (kt) already in LDS stage st
        // and, with four stages, the second in stage st+1; with four stages
        // tiles are stored two ahead and a barrier follows every other step
        // (and the end of the pass, after which the next pass may store into
        // any stage)
        auto pass = [&](auto cls_tag, int kt) __attribute__((always_inline)) {
            constexpr bool C = decltype(cls_tag)::value;
            int kn = next_of(kt + 1, C);
            int kn2 = (NST == 4 && kn < kt1) ? next_of(kn + 1, C) : kt1;
            int si = 0;
            auto step = [&](auto mask_tag) __attribute__((always_inline)) {
                constexpr bool MASK = decltype(mask_tag)::value;
                if (trace && tid == 0) atomicAdd(trace + kt, C ? 0x10000u : 1u);
                if constexpr (NST == 4) {
                    if (kn2 < kt1) gload(set0, kn2, C);
                    if (MASK ? kt < kt_end : wave_active) tile(mask_tag, st, kt, C);
                    if (kn2 < kt1) lstore(set0, (st + 2) & 3, C);
                    if (si & 1) __syncthreads();
                    ++si;
                    st = (st + 1) & 3;
                    kt = kn;
                    kn = kn2;
                    if (kn2 < kt1) kn2 = next_of(kn2 + 1, C);
                } else {
                    if (kn < kt1) gload(set0, kn, C);
                    if (MASK ? kt < kt_end : wave_active) tile(mask_tag, st, kt, C);
                    if (kn < kt1) lstore(set0, st ^ 1, C);
                    __syncthreads();
                    st ^= 1;
                    kt = kn;
                    if (kn < kt1) kn = next_of(kn + 1, C);
                }
            };
            const int full_end = min(nfull, kt1);
            while (kt < full_end) step(std::false_type{});
            while (kt < kt1) step(std::true_type{});
            if constexpr (NST == 4) __syncthreads();
        };
        // first two tiles of route c from kt0 (the second is kt1 with two stages)
        auto first2 = [&](bool c, int& t0, int& t1) __attribute__((always_inline)) {
            t0 = next_of(kt0, c);
            t1 = (NST == 4 && t0 < kt1) ? next_of(t0 + 1, c) : kt1;
        };
        int kt, kt2;
        first2(false, kt, kt2);
        if (kt < kt1) gload(set0, kt, false);
        if constexpr (NST == 4) {
            if (kt2 < kt1) gload(set1, kt2, false);
        }
        __builtin_amdgcn_s_waitcnt(0);
        query_prologue();
        if (kt < kt1) lstore(set0, st, false);
        if constexpr (NST == 4) {
            if (kt2 < kt1) lstore(set1, (st + 1) & 3, false);
        }
        __syncthreads();
        pass(std::false_type{}, kt);
        first2(true, kt, kt2);
        if (kt < kt1) {
            gload(set0, kt, true);
            if constexpr (NST == 4) {
                if (kt2 < kt1) gload(set1, kt2, true);
            }
            // the query codes are made here, so that they are not live
            // through the FP16 pass
            float sq;
            quantize_q_regs<HD, FP8>(qf, q8, sq);
            sq_mul = sq > 0.0f ? sq : 1.0f;   // a zero row has all-zero INT8 scores
            lstore(set0, st, true);
            if constexpr (NST == 4) {
                if (kt2 < kt1) lstore(set1, (st + 1) & 3, true);
            }
            __syncthreads();
            pass(std::true_type{}, kt);
        }
        }
    } else if constexpr (DMA) {
    // Direct loads, four stages (one key group): tiles 0 and 1 in stages 0
    // and 1; step it loads tile it + 2 into the stage step it - 2 read,
    // computes tile it and, after odd steps, waits for its loads and meets
    // the barrier.  Two stages (per key group): step it loads tile it + 1 into
    // the stage step it - 1 read and every step ends with the wait and the
    // barrier.  Fully
    // visible tiles run unrolled by four with constant stage offsets (see the
    // routed passes), the masked tail with a computed stage.
    if (has(0)) dma(kt_first, 0, false);
    if (NST == 4 && has(1)) dma(kt_first + KS, 1, false);
    query_prologue();
    dsync();
    auto dstep = [&](auto mask_tag, int S, int it) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int kt = kt_first + KS * it;
        if constexpr (NST == 4) {
            if (has(it + 2)) dma(kt + 2 * KS, (S + 2) & 3, false);
        } else {
            if (has(it + 1)) dma(kt + KS, S ^ 1, false);
        }
        if (MASK ? kt < kt_end : wave_active) tile(mask_tag, S, kt, false);
        if (NST == 2 || (S & 1)) dsync();
    };
    int it = 0;
    while (true) {
        if (it >= it_full) break;
        dstep(std::false_type{}, 0, it++);
        if (it >= it_full) break;
        dstep(std::false_type{}, 1 & (NST - 1), it++);
        if (it >= it_full) break;
        dstep(std::false_type{}, 2 & (NST - 1), it++);
        if (it >= it_full) break;
        dstep(std::false_type{}, 3 & (NST - 1), it++);
    }
    for (; it < n_it; ++it) dstep(std::true_type{}, it & (NST - 1), it);
    } else {
    // Prologue: the first PF tiles' loads go out behind the query loads, and
    // one wait covers them all.
    if constexpr (PF == 2) {
        gload2(set0, kt_first);
        gload2(set1, kt_first + KS);
    } else {
        if (has(0)) gload(set0, kt_first, false);
        if constexpr (NST == 4) {
            if (has(1)) gload(set1, kt_first + KS, false);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    query_prologue();
    if constexpr (PF == 2) lstore2(set0, 0);
    else if (has(0)) lstore(set0, 0, false);
    if constexpr (NST == 4) {
        if (has(1)) lstore(set1, 1, false);
    }
    __syncthreads();

    // One iteration; P is the parity of it (selects the staging sets).
    auto iter = [&](auto mask_tag, auto par_tag, int it) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr int P = decltype(par_tag)::value;
        const int kt = kt_first + KS * it;
        if constexpr (PF == 2) {
            // tile it+1 is already in flight (set (it+1)%2); issue tile it+2
            // into set it%2, which tile it left at its LDS store.  Loads and
            // stores of tiles past the end are harmless (zeros, into a stage
            // nobody reads), and keeping them unconditional keeps the load
            // count that the store of set (it+1)%2 waits for exact.
            gload2(P == 0 ? set0 : set1, kt + 2 * KS);
            if (MASK ? kt < kt_end : wave_active) tile(mask_tag, it & 1, kt, false);
            lstore2(P == 0 ? set1 : set0, (it + 1) & 1);
        } else if constexpr (NST == 4) {
            // tile it+2 goes to stage (it+2)%4, last read in iteration it-2;
            // a barrier after every odd iteration separates each store from
            // its reads and each read from the next store into its stage
            if (has(it + 2)) gload(set0, kt + 2 * KS, false);
            if (MASK ? kt < kt_end : wave_active) tile(mask_tag, it & 3, kt, false);
            if (has(it + 2)) lstore(set0, (it + 2) & 3, false);
            if (it & 1) __syncthreads();
            return;
        } else {
            if (has(it + 1)) gload(set0, kt + KS, false);
            if (MASK ? kt < kt_end : wave_active) tile(mask_tag, it & 1, kt, false);
            if (has(it + 1)) lstore(set0, (it + 1) & 1, false);
        }
        __syncthreads();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int it = 0;
    // iterations [it, it_end); with two staging sets the body is unrolled by
    // two so that each set is a fixed register range
    auto run = [&](auto mask_tag, int it_end) __attribute__((always_inline)) {
        if constexpr (PF == 2) {
            if ((it & 1) && it < it_end) iter(mask_tag, P1{}, it++);
            for (; it + 1 < it_end; it += 2) {
                iter(mask_tag, P0{}, it);
                iter(mask_tag, P1{}, it + 1);
            }
            if (it < it_end) iter(mask_tag, P0{}, it++);
        } else {
            for (; it < it_end; ++it) iter(mask_tag, P0{}, it);
        }
    };
    run(std::false_type{}, it_full);
    run(std::true_type{}, n_it);
    }

    if constexpr (KS > 1) {
        // Merge the key groups' states into group 0 through LDS (every stage
        // is free after the loop's last barrier).  Lane layouts agree across
        // groups, so the merge is lane by lane: O = sum_g 2^(m_g - m) O_g,
        // l likewise, m = max_g m_g.
        constexpr int NE4 = NDB * 4 + 1;       // f32x4 slots per lane: O, then (m, l)
        static_assert((KS - 1) * NW * NE4 * 64 * 16 <= STG * NST * KS, "merge buffer exceeds LDS");
        f32x4* xb = (f32x4*)smem;
        if (kgp > 0) {
            f32x4* dst = xb + (size_t)((kgp - 1) * NW + w) * NE4 * 64 + l;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(db * 4 + r) * 64] = f32x4{o[db][4 * r], o[db][4 * r + 1], o[db][4 * r + 2], o[db][4 * r + 3]};
            dst[NDB * 4 * 64] = f32x4{m_run, l_run, 0.0f, 0.0f};
        }
        __syncthreads();
        if (kgp > 0) return;
#pragma unroll
        for (int j = 1; j < KS; ++j) {
            const f32x4* src = xb + (size_t)((j - 1) * NW + w) * NE4 * 64 + l;
            const f32x4 ml = src[NDB * 4 * 64];
            const float m_new = fmaxf(m_run, ml[0]);
            const float a0 = __builtin_amdgcn_exp2f(m_run - m_new);
            const float a1 = __builtin_amdgcn_exp2f(ml[0] - m_new);
            l_run = l_run * a0 + ml[1] * a1;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const f32x4 ov = src[(db * 4 + r) * 64];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[db][4 * r + e] = o[db][4 * r + e] * a0 + ov[e] * a1;
                }
        }
    }

    // ---- epilogue: O / l -> fp16, or a split partial --------------------------------
    const float l_tot = halfwave_sum(l_run);
    if (a.ksplit > 1) {
        if (wave_active && qi < Lq) {
            // keys of this split: O / l and m + log2(l); a split with no visible key
            // for the row contributes nothing (-inf)
            const bool any = l_tot > 0.0f;
            const float inv_l = any ? vfac_inv / l_tot : 0.0f;
            const size_t prow = (size_t)split * a.part_rows + qrow0 + qi;
            float* po = a.part_o + prow * HD + 4 * g;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    f32x4 fv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) fv[e] = o[db][4 * r + e] * inv_l;
                    *(f32x4*)(po + 32 * db + 8 * r) = fv;
                }
            if (g == 0) a.part_l[prow] = any ? m_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;
        }
        return;
    }
    if (wave_active && qi < Lq) {
        const float inv_l = vfac_inv / l_tot;
        _Float16* op = ob + (size_t)qi * HD + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                f16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(o[db][4 * r + e] * inv_l);
                *(f16x4*)(op + 32 * db + 8 * r) = hv;
            }
    }
}

// ---------------------------------------------------------------------------
// K-row quantisation pass (and test hook path 0): rows of HD fp16 values,
// HD/8 lanes per row, 8 values per lane.
// ---------------------------------------------------------------------------
template <int HD, bool FP8 = false>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const _Float16* __restrict__ x,
                                                            int8_t* __restrict__ q8,
                                                            float* __restrict__ s, long long rows) {
    constexpr int LPR = HD / 8;
    const long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long row = gt / LPR;
    const int part = (int)(gt % LPR);
    const bool ok = row < rows;
    f16x8 v = ok ? *(const f16x8*)(x + row * HD + part * 8) : f16x8{};
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)v[j]));
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    float sc, inv;
    unsigned w0 = 0, w1 = 0;
    if constexpr (FP8) {
        fp8_scale(amax, sc, inv);
        w0 = fp8_pack4(fp8_round((float)v[0], inv), fp8_round((float)v[1], inv), fp8_round((float)v[2], inv),
                       fp8_round((float)v[3], inv));
        w1 = fp8_pack4(fp8_round((float)v[4], inv), fp8_round((float)v[5], inv), fp8_round((float)v[6], inv),
                       fp8_round((float)v[7], inv));
    } else {
        quant_scale(amax, sc, inv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w0 |= ((unsigned)quant_code((float)v[j], inv) & 0xffu) << (8 * j);
            w1 |= ((unsigned)quant_code((float)v[4 + j], inv) & 0xffu) << (8 * j);
        }
    }
    if (ok) {
        *(uint2*)(q8 + row * HD + part * 8) = uint2{w0, w1};
        if (part == 0) s[row] = sc;
    }
}

// ---------------------------------------------------------------------------
// Merge of split-key partials: out = sum_s w_s O_s / sum_s w_s with
// w_s = 2^(L_s - max L), the same rescale the online softmax applies.
// HD/8 lanes per row, 8 values per lane.
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256) void merge_splits_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_l,
                                                           _Float16* __restrict__ out,
                                                           long long rows, int ks) {
    constexpr int LPR = HD / 8;
    const long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long row = gt / LPR;
    const int part = (int)(gt % LPR);
    if (row >= rows) return;
    float mx = -INFINITY;
    for (int sp = 0; sp < ks; ++sp) mx = fmaxf(mx, part_l[sp * rows + row]);
    f32x4 a0 = f32x4{}, a1 = f32x4{};
    float wsum = 0.0f;
    for (int sp = 0; sp < ks; ++sp) {
        const float lv = part_l[sp * rows + row];
        if (lv == -INFINITY) continue;
        const float wv = __builtin_amdgcn_exp2f(lv - mx);
        const float* src = part_o + ((size_t)sp * rows + row) * HD + part * 8;
        a0 += wv * *(const f32x4*)src;
        a1 += wv * *(const f32x4*)(src + 4);
        wsum += wv;
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    f16x8 hv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hv[e] = (_Float16)(a0[e] * inv);
        hv[4 + e] = (_Float16)(a1[e] * inv);
    }
    *(f16x8*)(out + row * HD + part * 8) = hv;
}

// Test hook path 1: the query prologue quantiser on 32-row blocks.
template <int HD, bool FP8 = false>
__global__ __launch_bounds__(64) void quantize_qrows_kernel(const _Float16* __restrict__ x,
                                                            int8_t* __restrict__ q8,
                                                            float* __restrict__ s, int rows) {
    const int l = threadIdx.x, g = l >> 5, lq = l & 31;
    const int row = blockIdx.x * 32 + lq;
    f16x8 qf[HD / 16];
    const _Float16* qp = x + (size_t)row * HD + 16 * g;
#pragma unroll
    for (int kb2 = 0; kb2 < HD / 32; ++kb2) {
        qf[2 * kb2] = row < rows ? *(const f16x8*)(qp + 32 * kb2) : f16x8{};
        qf[2 * kb2 + 1] = row < rows ? *(const f16x8*)(qp + 32 * kb2 + 8) : f16x8{};
    }
    i32x4 q8r[HD / 32];
    float sc;
    quantize_q_regs<HD, FP8>(qf, q8r, sc);
    if (row < rows) {
#pragma unroll
        for (int ks = 0; ks < HD / 32; ++ks)
            *(i32x4*)(q8 + (size_t)row * HD + 32 * ks + 16 * g) = q8r[ks];
        if (g == 0) s[row] = sc;
    }
}

// Test hook: the route each (query tile, key tile) takes, walked with the
// forward kernel's cursor and legality rule.  One wavefront per query tile
// (every lane walks the same, uniform, cursor; lane 0 writes): the tiles of
// the causally visible range [0, n_vis) take route 0 or 1, the rest 2.
__global__ __launch_bounds__(64) void route_dump_kernel(const uint32_t* route, int qsl, int ksl, int causal,
                                                        int tiles_per_bit, int wpr, uint8_t* out) {
    const int n_kt = (ksl + TK - 1) / TK;
    const int qt = blockIdx.x;
    const int last_row = min(qt * TQ + TQ, qsl) - 1;
    const int n_vis = causal ? min(n_kt, (last_row + (ksl - qsl)) / TK + 1) : n_kt;
    uint8_t* o = out + (size_t)qt * n_kt;
    for (int kt = threadIdx.x; kt < n_kt; kt += 64) o[kt] = 2;
    __syncthreads();
    if (route == nullptr) {
        for (int kt = threadIdx.x; kt < n_vis; kt += 64) o[kt] = 0;
        return;
    }
    RouteCursor cur(route + (size_t)qt * wpr, tiles_per_bit, n_vis);
    for (int c = 0; c < 2; ++c)
        for (int kt = cur.next(0, c != 0); kt < n_vis; kt = cur.next(kt + 1, c != 0))
            if (threadIdx.x == 0) o[kt] = (uint8_t)c;
}

template <typename K>
hipError_t set_lds(K kernel, int bytes) {
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int HD, int NW, int KS, bool CAUSAL, bool VARLEN, bool ROUTED, bool KV8, bool FP8>
hipError_t launch_fwd_t(const FwdArgs& a, int grid, hipStream_t st) {
    auto kern = attn_fwd_kernel<HD, NW, KS, CAUSAL, VARLEN, ROUTED, KV8, FP8>;
    constexpr int stage = use_dma(HD, NW, KS, ROUTED, KV8) ? LdsDma<HD>::STAGE : Lds<HD>::STAGE;
    constexpr int lds = stage * n_stages(NW, KS, ROUTED) * KS;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * KS * 64), lds, st, a);
    return hipGetLastError();
}

template <int HD, int NW, int KS, bool ROUTED, bool KV8, bool FP8 = false>
hipError_t dispatch_mask(const FwdArgs& a, int grid, bool causal, bool varlen, hipStream_t st) {
    if (varlen)
        return causal ? launch_fwd_t<HD, NW, KS, true, true, ROUTED, KV8, FP8>(a, grid, st)
                      : launch_fwd_t<HD, NW, KS, false, true, ROUTED, KV8, FP8>(a, grid, st);
    return causal ? launch_fwd_t<HD, NW, KS, true, false, ROUTED, KV8, FP8>(a, grid, st)
                  : launch_fwd_t<HD, NW, KS, false, false, ROUTED, KV8, FP8>(a, grid, st);
}

// Instantiated shapes: two query wavefronts with one key group for routed
// calls with an odd head group, and with two key groups for small non-routed
// fp16 grids; two key groups for non-routed fp16 calls only; eight query
// wavefronts for every kind of call; FP8 routes on fp16 inputs only.
template <int HD>
hipError_t dispatch(const FwdArgs& a, int grid, int NW, int KS, bool causal, bool varlen, bool routed,
                    bool kv8, bool fp8, hipStream_t st) {
    if (fp8 && (!routed || kv8 || KS != 1)) return hipErrorInvalidConfiguration;
    if (NW == 2 && KS == 2) {
        if (routed || kv8) return hipErrorInvalidConfiguration;
        return dispatch_mask<HD, 2, 2, false, false>(a, grid, causal, varlen, st);
    }
    if (NW == 2) {
        if (!routed || KS != 1) return hipErrorInvalidConfiguration;
        if (fp8) return dispatch_mask<HD, 2, 1, true, false, true>(a, grid, causal, varlen, st);
        return kv8 ? dispatch_mask<HD, 2, 1, true, true>(a, grid, causal, varlen, st)
                   : dispatch_mask<HD, 2, 1, true, false>(a, grid, causal, varlen, st);
    }
    if (KS == 2) {
        if (routed || kv8) return hipErrorInvalidConfiguration;
        return dispatch_mask<HD, 4, 2, false, false>(a, grid, causal, varlen, st);
    }
    if (NW == 8) {
        if (KS != 1) return hipErrorInvalidConfiguration;
        if (routed)
            return fp8 ? dispatch_mask<HD, 8, 1, true, false, true>(a, grid, causal, varlen, st)
                       : kv8 ? dispatch_mask<HD, 8, 1, true, true>(a, grid, causal, varlen, st)
                             : dispatch_mask<HD, 8, 1, true, false>(a, grid, causal, varlen, st);
        return kv8 ? dispatch_mask<HD, 8, 1, false, true>(a, grid, causal, varlen, st)
                   : dispatch_mask<HD, 8, 1, false, false>(a, grid, causal, varlen, st);
    }
    if (routed) {
        if (fp8) return dispatch_mask<HD, 4, 1, true, false, true>(a, grid, causal, varlen, st);
        return kv8 ? dispatch_mask<HD, 4, 1, true, true>(a, grid, causal, varlen, st)
                   : dispatch_mask<HD, 4, 1, true, false>(a, grid, causal, varlen, st);
    }
    return kv8 ? dispatch_mask<HD, 4, 1, false, true>(a, grid, causal, varlen, st)
               : dispatch_mask<HD, 4, 1, false, false>(a, grid, causal, varlen, st);
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, long long rows, int hdim, int8_t* q8, float* s,
                                int path, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
    const _Float16* xh = (const _Float16*)x;
    if (path == 0 || path == 2) {
        // K-row pass: INT8 (0) or FP8 (2)
        const long long threads = (long long)rows * (hdim / 8);
        const int grid = (int)((threads + 255) / 256);
        auto k = hdim == 64 ? (path == 0 ? quantize_rows_kernel<64, false> : quantize_rows_kernel<64, true>)
                            : (path == 0 ? quantize_rows_kernel<128, false> : quantize_rows_kernel<128, true>);
        hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, st, xh, q8, s, rows);
    } else {
        // query-prologue quantiser: INT8 (1) or FP8 (3)
        const int grid = (int)((rows + 31) / 32);
        auto k = hdim == 64 ? (path == 1 ? quantize_qrows_kernel<64, false> : quantize_qrows_kernel<64, true>)
                            : (path == 1 ? quantize_qrows_kernel<128, false> : quantize_qrows_kernel<128, true>);
        hipLaunchKernelGGL(k, dim3(grid), dim3(64), 0, st, xh, q8, s, (int)rows);
    }
    return hipGetLastError();
}

hipError_t launch_route_dump(const uint32_t* route, int qsl, int ksl, bool causal,
                             int tiles_per_bit, uint8_t* out, hipStream_t st) {
    const int n_kt = (ksl + TK - 1) / TK;
    const int n_qt = (qsl + TQ - 1) / TQ;
    const int n_g = (n_kt + tiles_per_bit - 1) / tiles_per_bit;
    const int wpr = (n_g + 31) / 32;
    (void)n_kt;
    hipLaunchKernelGGL(route_dump_kernel, dim3(n_qt), dim3(64), 0, st, route, qsl, ksl,
                       causal ? 1 : 0, tiles_per_bit, wpr, out);
    return hipGetLastError();
}

// Compute units of the current device (cached per device).
static int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

static int largest_div(int G, int cap) {
    for (int d = cap; d > 1; d >>= 1)
        if (G % d == 0) return d;
    return 1;
}

// Launch plan of one forward call: workgroup shape, key splits, scratch layout.
struct Plan {
    int NW, KS, HPW, BM, combos, n_mblk, ksplit;
    int pair_blocks;
    long long grid;
    size_t k8_off, sk_off, po_off, pl_off, bytes;   // scratch layout (bytes)
    long long out_rows;
};

static size_t round_up(size_t x) { return (x + 255) / 256 * 256; }

static Plan make_plan(const Problem& p) {
    Plan pl{};
    const bool varlen = p.cu_seqlens != nullptr;
    const bool routed = p.route != nullptr;
    const bool kv8 = p.k8 != nullptr;
    const int G = p.n_qh / p.n_kvh;
    const long long simds = 4LL * cu_count();
    const int n_kt = (p.ksl + BN - 1) / BN;
    pl.HPW = largest_div(G, 4);
    auto blocks_of = [&](int nw) {        // query-row blocks per workgroup column
        const int bm = (nw / pl.HPW) * 32;
        return varlen ? (p.qsl + bm - 1) / bm + p.B : (p.qsl + bm - 1) / bm;
    };
    // key-range splits that bring w wavefronts to two per SIMD, keeping at
    // least sixteen tiles per split (the fp32 partials and their merge cost
    // more than they return otherwise)
    auto splits_for = [&](long long w) {
        int ks = 1;
        while (ks < 8 && w * ks < 2 * simds && n_kt >= 16 * ks) ks *= 2;
        return ks;
    };
    pl.combos = (varlen ? 1 : p.B) * p.n_kvh * (G / pl.HPW);
    // Workgroup shape.  A routed workgroup stays inside one 64-row query tile
    // (two wavefronts when the head group is odd).  Calls whose grid gives
    // two wavefronts per SIMD even so take eight query wavefronts (routed ones
    // only when the head group holds four heads, so that the eight stay inside
    // one 64-row query tile): each K/V tile then serves twice the rows,
    // halving the tile loads and LDS stores per FLOP.  (With fewer, four
    // wavefronts and two key groups hide latency better than eight and a
    // split key range.)
    pl.NW = 4;
    if (routed && pl.HPW == 1) pl.NW = 2;
    const bool nw8_ok = !routed || pl.HPW == 4;
    if (nw8_ok && (long long)pl.combos * blocks_of(8) * 8 >= 2 * simds) pl.NW = 8;
    // Small fp16 grids (under two wavefronts per SIMD) run one workgroup per
    // CU.  Under a causal mask whose diagonal spans most of the keys, the
    // workgroups of the last query rows visit every key tile and those of the
    // first rows almost none, so the launch lasts as long as its heaviest
    // workgroup; a grid with fewer workgroups than CUs leaves CUs idle.  Both
    // take 64-row workgroups of two query wavefronts and two key groups, two
    // per CU, so a heavy block shares its CU with a light one.  (Only where
    // the head group already fits two wavefronts: splitting a larger group
    // halves the rows each K/V tile serves, and at hdim 128 two such
    // workgroups exceed the CU's LDS.)
    const bool fp16_small = !routed && !kv8 && p.hdim == 64 && pl.HPW <= 2 && n_kt >= 2 &&
                            (long long)pl.combos * blocks_of(4) * 4 < 2 * simds;
    const bool diag = p.causal && p.ksl - p.qsl < p.qsl;
    if (pl.NW == 4 && fp16_small && (diag || (long long)pl.combos * blocks_of(4) < simds / 4)) pl.NW = 2;
    const char* force_nw = getenv("ATTN_QUERY_WAVES");
    if (force_nw && force_nw[0] && force_nw[1] == 0) {
        const int f = force_nw[0] - '0';
        if (!routed && (f == 4 || f == 8 || (f == 2 && !kv8))) pl.NW = f;
        if (routed && ((f == 4 && pl.HPW > 1) || (f == 8 && nw8_ok))) pl.NW = f;
    }
    if (pl.NW == 2 && !routed && pl.HPW > 2) {
        pl.HPW = largest_div(G, 2);
        pl.combos = (varlen ? 1 : p.B) * p.n_kvh * (G / pl.HPW);
    }
    pl.BM = (pl.NW / pl.HPW) * 32;
    pl.n_mblk = blocks_of(pl.NW);
    // Small grids leave SIMDs with one wavefront or none, so nothing hides
    // the latency of one wavefront's loads, softmax and MFMA chains.  First
    // give each workgroup a second key group (same rows, alternate key tiles,
    // merged in LDS); then, if SIMDs are still idle, split the key range over
    // workgroups: up to two wavefronts per SIMD.
    const long long waves = (long long)pl.combos * pl.n_mblk * pl.NW;
    const bool kg2_ok = !routed && !kv8 && pl.NW == 4;
    pl.KS = (kg2_ok && waves < 2 * simds && n_kt >= 2) ? 2 : 1;
    const char* force_kg = getenv("ATTN_KEY_GROUPS");
    if (kg2_ok && force_kg && (force_kg[0] == '1' || force_kg[0] == '2') && force_kg[1] == 0)
        pl.KS = force_kg[0] - '0';
    if (pl.NW == 2 && !routed) pl.KS = 2;     // the only non-routed two-wavefront shape
    int ks = splits_for(waves * pl.KS);
    const char* force = getenv("ATTN_KSPLIT");
    if (force && force[0] >= '1' && force[0] <= '8' && force[1] == 0) ks = force[0] - '0';
    pl.ksplit = ks;
    pl.grid = (long long)pl.combos * pl.ksplit * pl.n_mblk;
    // Causal row blocks run heavy-first.  When every workgroup of the grid is
    // resident at once, two to a CU (two-wavefront workgroups), workgroups i
    // and i + grid/2 share a CU; the second half then runs light-first, so
    // the heaviest block shares its CU with the lightest one and every CU
    // gets about the same number of key tiles.
    pl.pair_blocks = (p.causal && !varlen && pl.NW == 2 && pl.KS == 2 && !routed && pl.ksplit == 1 &&
                      pl.grid == 2LL * cu_count() && pl.n_mblk % 2 == 0) ? 1 : 0;
    const char* force_pair = getenv("ATTN_PAIR_BLOCKS");
    if (force_pair && (force_pair[0] == '0' || force_pair[0] == '1') && force_pair[1] == 0)
        pl.pair_blocks = (force_pair[0] == '1' && p.causal && !varlen) ? 1 : 0;
    pl.out_rows = varlen ? (long long)p.n_qh * p.qsl : (long long)p.B * p.n_qh * p.qsl;
    size_t off = 0;
    if (routed && !kv8 && !ATTN_FUSED_KQUANT) {
        const size_t krows = varlen ? (size_t)p.n_kvh * p.ksl : (size_t)p.B * p.n_kvh * p.ksl;
        pl.k8_off = off;
        off += round_up(krows * p.hdim);
        pl.sk_off = off;
        off += round_up(krows * sizeof(float));
    }
    if (pl.ksplit > 1) {
        pl.po_off = off;
        off += round_up((size_t)pl.ksplit * pl.out_rows * p.hdim * sizeof(float));
        pl.pl_off = off;
        off += round_up((size_t)pl.ksplit * pl.out_rows * sizeof(float));
    }
    pl.bytes = off;
    return pl;
}

size_t forward_scratch_bytes(const Problem& p) { return make_plan(p).bytes; }

// The device address of `scratch` on the current device, looked up once per
// device with that device current (host code never passes the array's own
// name, a host-side stand-in, to the device).
hipError_t noalloc_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

void forward_plan(const Problem& p, long long out[10]) {
    const Plan pl = make_plan(p);
    out[0] = pl.NW;
    out[1] = pl.KS;
    out[2] = pl.HPW;
    out[3] = pl.BM;
    out[4] = pl.combos;
    out[5] = pl.n_mblk;
    out[6] = pl.ksplit;
    out[7] = pl.pair_blocks;
    out[8] = pl.grid;
    out[9] = (long long)pl.bytes;
}

hipError_t launch_forward(const Problem& p, void* scratch, hipStream_t st) {
    const Plan pl = make_plan(p);
    FwdArgs a;
    a.q = (const _Float16*)p.q;
    a.k = (const _Float16*)p.k;
    a.v = (const _Float16*)p.v;
    a.out = (_Float16*)p.out;
    a.cu = p.cu_seqlens;
    a.route = p.route;
    a.B = p.B;
    a.qsl = p.qsl;
    a.ksl = p.ksl;
    a.n_qh = p.n_qh;
    a.n_kvh = p.n_kvh;
    a.G = p.n_qh / p.n_kvh;
    a.c = fabsf(p.scale) * LOG2E;
    a.neg = p.scale < 0.0f ? 1 : 0;
    a.tiles_per_bit = p.route ? p.tiles_per_bit : 1;
    a.k8 = p.k8;            // INT8 key/value cache, or null
    a.sk = p.k_scale;
    a.v8 = p.v8;
    a.sv = p.v_scale;
    a.HPW = pl.HPW;
    a.combos = pl.combos;
    a.n_mblk = pl.n_mblk;
    a.pair_blocks = pl.pair_blocks;
    a.ksplit = pl.ksplit;
    a.part_rows = pl.out_rows;
    a.part_o = pl.ksplit > 1 ? (float*)((char*)scratch + pl.po_off) : nullptr;
    a.part_l = pl.ksplit > 1 ? (float*)((char*)scratch + pl.pl_off) : nullptr;
    a.trace = p.route ? p.trace : nullptr;
    a.trace_nkt = (p.ksl + TK - 1) / TK;
    const bool varlen = p.cu_seqlens != nullptr;
    const bool routed = p.route != nullptr;

    const bool kv8 = p.k8 != nullptr;
    if (routed) {
        const int n_kt = (p.ksl + TK - 1) / TK;
        const int n_g = (n_kt + p.tiles_per_bit - 1) / p.tiles_per_bit;
        a.wpr = (n_g + 31) / 32;
        if (!kv8 && !ATTN_FUSED_KQUANT) {
            // INT8 codes of every K row, once per call (a cache brings its own)
            const size_t krows = varlen ? (size_t)p.n_kvh * p.ksl : (size_t)p.B * p.n_kvh * p.ksl;
            a.k8 = (const int8_t*)((char*)scratch + pl.k8_off);
            a.sk = (const float*)((char*)scratch + pl.sk_off);
            hipError_t e = launch_quantize_rows(p.k, (long long)krows, p.hdim, (int8_t*)a.k8, (float*)a.sk,
                                                p.lowp == 1 ? 2 : 0, st);
            if (e != hipSuccess) return e;
        }
    } else {
        a.wpr = 0;
    }

    if (pl.grid <= 0) return hipSuccess;
    if (pl.grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int grid = (int)pl.grid;
    hipError_t e;
    const bool fp8 = routed && p.lowp == 1;
    if (p.hdim == 64)
        e = dispatch<64>(a, grid, pl.NW, pl.KS, p.causal, varlen, routed, kv8, fp8, st);
    else
        e = dispatch<128>(a, grid, pl.NW, pl.KS, p.causal, varlen, routed, kv8, fp8, st);
    if (e != hipSuccess || pl.ksplit == 1) return e;
    const long long threads = pl.out_rows * (p.hdim / 8);
    const int mgrid = (int)((threads + 255) / 256);
    if (p.hdim == 64)
        hipLaunchKernelGGL(merge_splits_kernel<64>, dim3(mgrid), dim3(256), 0, st, a.part_o, a.part_l,
                           a.out, pl.out_rows, pl.ksplit);
    else
        hipLaunchKernelGGL(merge_splits_kernel<128>, dim3(mgrid), dim3(256), 0, st, a.part_o, a.part_l,
                           a.out, pl.out_rows, pl.ksplit);
    return hipGetLastError();
}

}  // namespace attn
