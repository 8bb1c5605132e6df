/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention-forward (prefill)
 * library, libattn_mi355x.so.
 *
 * The operation (attn_fwd) is fused scaled-dot-product attention forward,
 * as timed in the "Nax Refactor" page (ml-explore/mlx pull request 3271,
 * fused-vs-unfused timing tables over B, qsl, ksl, hdim, n_qh, n_kvh, causal
 * in float16), with the TileMix option (TileMix abstract, Lattice paper
 * summary): a compact bitmask routes each (query tile, key-tile group)
 * through an FP16 or an INT8 QK^T score computation, and both routes update
 * one online-softmax state.
 *
 * For every batch element (or packed sequence) s, query head h, row i:
 *   out[s,h,i,:] = sum_j softmax_j(S[i,j]) * v[s,hk,j,:],  hk = h / (n_qh/n_kvh)
 *   S[i,j] = scale * <q[s,h,i,:], k[s,hk,j,:]>                 (FP16 route)
 *   S[i,j] = scale * s_q[i] * s_k[j] * <q8[s,h,i,:], k8[s,hk,j,:]>  (INT8 route)
 * over the visible keys j: all j < ksl, or, when causal, j <= i + (ksl - qsl)
 * (bottom-right aligned).  INT8 codes are per token: amax = max_d |x_d|,
 * s = fl32(amax / 127), q8_d = round-half-even(x_d * fl32(127 / amax)) with
 * the product exact; a zero row has s = 0 and q8 = 0.  V stays fp16.
 *
 * Memory: every tensor pointer is DEVICE memory owned by the caller,
 * contiguous, 16-byte aligned.  fp16 is IEEE binary16.
 *   dense  (cu_seqlens == NULL): q, out [B, n_qh, qsl, hdim]; k, v [B, n_kvh, ksl, hdim]
 *   packed (cu_seqlens != NULL): q, out [n_qh, T, hdim];    k, v [n_kvh, T, hdim]
 *     with T = qsl = ksl and cu_seqlens int32 [B + 1] on the device,
 *     cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = T.  Each sequence is
 *     its own attention problem (causal per sequence when causal != 0).
 * route_bitmask (device, uint32, may be NULL = every tile FP16): one bit per
 *   (64-row query tile qt, group g of tiles_per_bit adjacent 64-key tiles),
 *   shared by all heads and batch elements.  Rows of wpr = ceil(n_g / 32)
 *   words, n_g = ceil(ceil(ksl / 64) / tiles_per_bit); bit g of row qt is
 *   (route_bitmask[qt * wpr + g / 32] >> (g % 32)) & 1; 1 = INT8, 0 = FP16.
 *   Tile indices count from row 0 of q and row 0 of k.  Bits of groups that
 *   the causal mask leaves empty for a query tile are ignored.
 *   Packed input: each sequence s has its own rows, one per 64-row query tile
 *   of that sequence (counted from its start), stacked in sequence order, so
 *   the row of (s, qt) is qt + sum over s' < s of ceil(L_s'/64); wpr is
 *   computed with ksl = T, and bits of groups past the sequence's own key
 *   tiles are ignored.
 *   Size: the bitmask must hold ceil(qsl / 64) * wpr words (dense), or
 *   (sum over s of ceil(L_s / 64)) * wpr words (packed); the library cannot
 *   see its length, and a shorter array is read past its end.
 * out is fully overwritten.  Nothing the caller passes is retained.
 *
 * Calls are asynchronous: they validate the arguments on the host, enqueue
 * work on the given stream and return.  Routed calls (quantised K rows) and
 * calls whose grid is split along the keys (fp32 partial results) use
 * stream-ordered device scratch (allocated and freed on the same stream) from
 * a memory pool that the library creates per device on first use and keeps
 * until the process ends; freed blocks stay cached in that pool for the next
 * call.  The device's default pool is not touched.  Errors are reported by
 * the return code; a thread-local message is available from
 * attn_last_error().  Argument errors are detected before any device work is
 * enqueued.
 *
 * The contents of cu_seqlens are the caller's responsibility: the kernels
 * trust them.  Two environment switches help debugging (read at every call):
 *   ATTN_DEBUG_VALIDATE=1  the forward entry points copy cu_seqlens to the
 *     host (synchronising the stream) and return ATTN_ERR_ARG unless
 *     cu_seqlens[0] = 0, it is non-decreasing and cu_seqlens[B] = T;
 *   ATTN_DEBUG_SYNC=1  every entry point synchronises its stream after the
 *     launch and returns ATTN_ERR_HIP if a kernel failed.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* q, k, v or out is NULL */
    ATTN_ERR_SHAPE = 2,        /* a size <= 0, n_qh % n_kvh != 0, causal with
                                  qsl > ksl, packed with qsl != ksl, or a
                                  K / V slab of 2^31 bytes or more */
    ATTN_ERR_UNSUPPORTED = 3,  /* hdim not 64 or 128 */
    ATTN_ERR_ARG = 4,          /* scale not finite or zero; tiles_per_bit < 1
                                  with a bitmask; pointer not 16-byte aligned */
    ATTN_ERR_HIP = 5           /* the HIP runtime reported an error */
} attn_status;

#define ATTN_ABI_VERSION 1

/* The format a set routing bit selects (attn_fwd_lowp_stream). */
typedef enum {
    ATTN_LOWP_INT8 = 0,      /* per-token INT8, the rule above (attn_fwd's route) */
    ATTN_LOWP_FP8_E4M3 = 1   /* per-token FP8 e4m3, rowwise dynamic scaling */
} attn_lowp;

/* Fused attention forward on the null (default) stream.  scale may be
 * negative; tiles_per_bit is read only when route_bitmask != NULL. */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* out,
                     int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                     int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                     const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                     int32_t tiles_per_bit);

/* Same, enqueued on hip_stream (a hipStream_t; NULL = null stream). */
attn_status attn_fwd_stream(const void* q, const void* k, const void* v, void* out,
                            int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                            int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                            const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                            int32_t tiles_per_bit, void* hip_stream);

/* Fused attention forward on an INT8 key/value cache (TileMix abstract:
 * INT8 key/value caches are supported).  The keys and values are
 *   K^[s,hk,j,:] = k_scale[s,hk,j] * k8[s,hk,j,:],
 *   V^[s,hk,j,:] = v_scale[s,hk,j] * v8[s,hk,j,:],
 * and out is the attention of q over them:
 *   FP16 route: S[i,j] = scale * <q[s,h,i,:], K^[s,hk,j,:]>
 *   INT8 route: S[i,j] = scale * s_q[i] * k_scale[j] * <q8[s,h,i,:], k8[s,hk,j,:]>
 * with q8, s_q the per-token codes of the query row (the rule above); the
 * cached codes are the INT8 keys, not requantised.  Every other argument,
 * the masks, the packed layout and the bitmask are those of attn_fwd.
 *   k8, v8: device int8 in the layout of k and v; 16-byte aligned.
 *   k_scale, v_scale: device fp32, one per K / V row ([B, n_kvh, ksl] dense,
 *   [n_kvh, T] packed); 4-byte aligned.
 * attn_quantize_rows builds such a cache from fp16 rows.  The value codes
 * (and, for FP16 cells, the key codes) are multiplied by their row's scale
 * in fp16 as the kernel stages them, after division of the scales by a
 * power of two near the largest |v_scale| (|k_scale|) of the keys a
 * workgroup visits (multiplied back, exactly, in fp32), so any finite scale
 * works without overflow, and the precision of the staged values depends
 * only on the ratio of a row's scale to that largest scale, not on the
 * values' magnitude.  INT8 cells use the codes and k_scale as they are.
 * Errors as attn_fwd (ATTN_ERR_NULL names the cache pointers). */
attn_status attn_fwd_kv8(const void* q, const int8_t* k8, const float* k_scale,
                         const int8_t* v8, const float* v_scale, void* out,
                         int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                         int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                         const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                         int32_t tiles_per_bit);

/* Same, enqueued on hip_stream (a hipStream_t; NULL = null stream). */
attn_status attn_fwd_kv8_stream(const void* q, const int8_t* k8, const float* k_scale,
                                const int8_t* v8, const float* v_scale, void* out,
                                int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                                int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                                const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                                int32_t tiles_per_bit, void* hip_stream);

/* The unfused baseline the "Nax Refactor" page times against its fused
 * kernel (the t_unfs / speed_up columns of its timing tables): the same
 * attention as attn_fwd for dense fp16 inputs (no packed batches, no
 * bitmask), computed as separate passes over a materialised score matrix --
 * S = Q K^T (rocBLAS strided-batched GEMM, fp32 scores), a masked row
 * softmax (fp16 P), O = P V (GEMM, fp32 accumulation).  Arguments as
 * attn_fwd.  Uses 6 bytes of stream-ordered scratch per (query, key) pair
 * of the whole call; more than 64 GB is ATTN_ERR_SHAPE.  One rocBLAS handle
 * per device is created on first use and kept; calls on one device
 * serialise on it.  For comparison runs, not a production path. */
attn_status attn_fwd_unfused_stream(const void* q, const void* k, const void* v, void* out,
                                    int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                                    int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                                    void* hip_stream);

/* The INT8 cache encoder: per-token codes and scales (the rule above) of
 * rows fp16 rows of hdim values.  x_f16: device [rows, hdim] fp16, 16-byte
 * aligned; q8: device int8 [rows, hdim], 16-byte aligned; scale_out: device
 * fp32 [rows], 4-byte aligned.  0 <= rows < 2^31.  Asynchronous on
 * hip_stream. */
attn_status attn_quantize_rows(const void* x_f16, int64_t rows, int32_t hdim, int8_t* q8,
                               float* scale_out, void* hip_stream);

/* The TileMix route with a choice of low-precision format for the groups
 * whose bit is set.  lowp_format ATTN_LOWP_INT8 is attn_fwd_stream.
 * ATTN_LOWP_FP8_E4M3 takes the rowwise dynamic scaling of the "Add rowwise
 * scaling to Float8Inference module" page (one scale per row from its
 * absolute maximum) with e4m3 codes (sign, 4 exponent bits biased by 7, 3
 * mantissa bits, largest finite 448; the FP8 MFMA of gfx950 runs at the
 * INT8 rate):
 *   s = fl32(amax / 448), code = the e4m3 value nearest to x * fl32(448 / amax)
 *   (product exact, ties to the even mantissa; a zero row has s = 0, codes 0),
 *   S[i,j] = scale * s_q[i] * s_k[j] * sum_d e4m3(q)[i,d] * e4m3(k)[j,d].
 * Other arguments and errors as attn_fwd_stream; any other lowp_format is
 * ATTN_ERR_ARG. */
attn_status attn_fwd_lowp_stream(const void* q, const void* k, const void* v, void* out,
                                 int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                                 int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                                 const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                                 int32_t tiles_per_bit, int32_t lowp_format, void* hip_stream);

/* attn_fwd_lowp_stream for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, kernels and result, but the scratch that
 * routed calls (quantised K rows) and split-key calls (fp32 partials) need
 * comes from a static device array of 64 MiB per device, held from library
 * load until the process ends, instead of from the stream-ordered pool.  The
 * call allocates nothing (no hipMalloc, hipFree or pool call).  A call whose
 * scratch would exceed 64 MiB returns ATTN_ERR_SHAPE before any device work
 * (for example routed calls over more than about 60 M key rows x hdim bytes).
 * Every call on one device shares that array and nothing in it needs to
 * start at zero: calls that overlap in time on one device (on different
 * streams, or from different threads) race on it and must be serialised by
 * the caller.  ATTN_DEBUG_VALIDATE is not applied here (it would allocate a
 * host copy); ATTN_DEBUG_SYNC is. */
attn_status attn_fwd_noalloc_stream(const void* q, const void* k, const void* v, void* out,
                                    int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                                    int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                                    const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                                    int32_t tiles_per_bit, int32_t lowp_format, void* hip_stream);

/* Message for the last non-OK status returned on this thread ("" if none).
 * The string is owned by the library and valid until the next call. */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the loaded library. */
int32_t attn_abi_version(void);

/* Test hooks for bit-exact checks of the quantisers (rules above).
 * x_f16: device [rows, hdim] fp16; q8: device int8 [rows, hdim] (FP8 paths:
 * e4m3 bit patterns); scale_out: device fp32 [rows].  path 0 runs the INT8
 * K-row quantiser used before routed calls, path 1 the INT8 query-row
 * quantiser of the attention prologue, paths 2 and 3 the same two for FP8.
 * Asynchronous on hip_stream. */
attn_status attn_debug_quantize_rows(const void* x_f16, int32_t rows, int32_t hdim,
                                     int8_t* q8, float* scale_out, int32_t path,
                                     void* hip_stream);

/* Test hook for the routing decode (TileMix abstract: routing decisions
 * packed into compact bitmasks): writes, for every (query tile qt, key tile
 * kt) of a qsl x ksl problem, the route that the bitmask gives, decoded by
 * the same device cursor the forward kernel's routed passes walk, over the
 * same causally visible tile range: 0 = FP16, 1 = INT8 (or the
 * low-precision route), 2 = not visited (the causal mask leaves that tile
 * empty for every row of qt).  route_out: device uint8 [ceil(qsl/64),
 * ceil(ksl/64)].  Asynchronous on hip_stream.  attn_debug_route_trace
 * records what the forward kernel itself visits. */
attn_status attn_debug_route_dump(const uint32_t* route_bitmask, int32_t qsl, int32_t ksl,
                                  int32_t causal, int32_t tiles_per_bit, uint8_t* route_out,
                                  void* hip_stream);

/* Test hook: a routed forward call (the arguments and result of
 * attn_fwd_lowp_stream; route_bitmask must be set) that also records the
 * tiles its workgroups visit.  trace_out: device uint32 [rows, ceil(ksl/64)]
 * with rows = ceil(qsl/64) (dense) or the packed bitmask's row count, row r
 * holding the tiles of bitmask row r; trace_words is its length, which must
 * be at least rows * ceil(ksl/64) (packed: (ceil(T/64) + B) * ceil(T/64)).
 * The call clears it, then every workgroup adds 1 at each key tile it visits
 * on the FP16 route and 0x10000 at each one it visits on the low-precision
 * route, in the kernel's own routed loop.  A routed workgroup holds 32 or 64
 * rows of one query tile (attn_debug_plan's rows per workgroup) for one
 * workgroup column (batch element, kv head, query-head group), so a tile
 * that every workgroup of its query tile visits reads n or n << 16, with n
 * the number of such workgroups.  Asynchronous on hip_stream.  Not for
 * production: the counts use device atomics. */
attn_status attn_debug_route_trace(const void* q, const void* k, const void* v, void* out,
                                   int32_t B, int32_t qsl, int32_t ksl, int32_t hdim,
                                   int32_t n_qh, int32_t n_kvh, float scale, int32_t causal,
                                   const int32_t* cu_seqlens, const uint32_t* route_bitmask,
                                   int32_t tiles_per_bit, int32_t lowp_format,
                                   uint32_t* trace_out, int64_t trace_words, void* hip_stream);

/* Test hook for the cu_seqlens rule that ATTN_DEBUG_VALIDATE applies, on a
 * HOST array of B + 1 entries: ATTN_OK if cu_seqlens_host[0] = 0, it is
 * non-decreasing and cu_seqlens_host[B] = T, else ATTN_ERR_ARG with a message
 * naming the entry.  No device access. */
attn_status attn_debug_check_cu_seqlens(const int32_t* cu_seqlens_host, int32_t B, int32_t T);

/* Test hook for the launch planner: the workgroup shape and grid that the
 * forward entry points would launch for these sizes.  Nothing is launched and
 * no device memory is touched.  flags: bit 0 packed batch (cu_seqlens set,
 * qsl == ksl == total tokens, B sequences), bit 1 routed (route_bitmask set),
 * bit 2 INT8 key/value cache, bit 3 FP8 route; other bits are ATTN_ERR_ARG.
 * The sizes are validated as for attn_fwd (scale taken as 1).  plan_out: host
 * int64[10], filled on ATTN_OK with: query wavefronts per workgroup, key
 * groups per workgroup, query heads per workgroup, query rows per workgroup,
 * workgroup columns, row blocks per column, key splits, 1 if the second half
 * of the causal row blocks runs light-first, grid size, scratch bytes.  The
 * plan uses the current device's CU count, or 256 when no device is
 * visible. */
attn_status attn_debug_plan(int32_t B, int32_t qsl, int32_t ksl, int32_t hdim, int32_t n_qh, int32_t n_kvh,
                            int32_t causal, int32_t tiles_per_bit, int32_t flags, int64_t* plan_out);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_MI355X_H */
