/*
 * oracle.h -- CPU fp64 attention oracle (test infrastructure only; see
 * oracle.c for what it computes and the pages it follows).
 *
 * All pointers are host memory.  fp16 tensors are passed as their IEEE
 * binary16 bit patterns (uint16_t).  Dense layout: q/out [B, n_qh, qsl, d],
 * k/v [B, n_kvh, ksl, d].  Packed layout (cu_seqlens != NULL): q/out
 * [n_qh, T, d], k/v [n_kvh, T, d], T = cu_seqlens[B] = qsl = ksl.
 * tile_q / tile_k set the routing tile sizes (<= 0 selects 64).
 */
#ifndef ATTN_ORACLE_H
#define ATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_OK = 0, ORACLE_ERR_ARG = 1, ORACLE_ERR_NOMEM = 2 };

double   oracle_f16_to_f64(uint16_t h);
uint16_t oracle_f64_to_f16_rne(double x);

/* q8[0..d) and the fp32 scale s of one row x[0..d) of fp16 bits. */
void oracle_quantize_row(const uint16_t* x, int d, int8_t* q8, float* s_out);

/* FP8 e4m3 (sign, 4 exponent bits with bias 7, 3 mantissa bits, max 448):
 * decode a bit pattern; round a value to the nearest e4m3 value (ties to
 * even, zero results +0); encode an exact e4m3 value. */
double  oracle_e4m3_decode(uint8_t c);
double  oracle_e4m3_round(double y);
uint8_t oracle_e4m3_encode(double r);

/* Rowwise dynamic FP8 codes of one fp16 row: s = fl32(amax/448), codes the
 * e4m3 values nearest to x * fl32(448/amax). */
void oracle_quantize_row_fp8(const uint16_t* x, int d, uint8_t* codes, float* s_out);

/* Every row of an [rows, d] fp16 array (the INT8 key/value cache encoder). */
void oracle_quantize_rows(const uint16_t* x, long long rows, int d, int8_t* q8, float* s_out);

int oracle_route_words_per_row(int ksl, int tile_k, int tiles_per_bit);
int oracle_route_bit(const uint32_t* words, int wpr, int qt, int g);

/* Full output, fp64, same layout as q.  Returns ORACLE_OK or an error. */
int oracle_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* out,
                    int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                    float scale, int causal, const int32_t* cu_seqlens,
                    const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                    int nthreads);

/* Selected output rows only: rows holds nrows triples (s, h, i) with s the
 * batch element (or packed sequence), h the query head, i the row within
 * that sequence; out is [nrows, d] fp64. */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                     float scale, int causal, const int32_t* cu_seqlens,
                     const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                     const int32_t* rows, int nrows, double* out, int nthreads);

/* INT8 key/value cache inputs: k8, v8 int8 in the layout of k, v; k_scale,
 * v_scale fp32 per row ([B, n_kvh, ksl] or [n_kvh, T]).  The keys and
 * values are K^ = k_scale * k8 and V^ = v_scale * v8; INT8 routed cells use
 * k8 and k_scale as the key codes. */
int oracle_attn_fwd_kv8(const uint16_t* q, const int8_t* k8, const float* k_scale,
                        const int8_t* v8, const float* v_scale, double* out,
                        int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                        float scale, int causal, const int32_t* cu_seqlens,
                        const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                        int nthreads);

int oracle_attn_rows_kv8(const uint16_t* q, const int8_t* k8, const float* k_scale,
                         const int8_t* v8, const float* v_scale,
                         int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                         float scale, int causal, const int32_t* cu_seqlens,
                         const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                         const int32_t* rows, int nrows, double* out, int nthreads);

/* lowp selects what a set routing bit means: 0 INT8 (as oracle_attn_fwd),
 * 1 FP8 e4m3 with rowwise scales. */
int oracle_attn_fwd_lowp(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* out,
                         int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                         float scale, int causal, const int32_t* cu_seqlens,
                         const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                         int lowp, int nthreads);

int oracle_attn_rows_lowp(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                          float scale, int causal, const int32_t* cu_seqlens,
                          const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                          int lowp, const int32_t* rows, int nrows, double* out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
