/*
 * oracle.c -- plain, slow, CPU fp64 reference for fused attention forward
 * (prefill) with optional TileMix FP16/INT8 score routing.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the HIP path is
 * measured against.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load it.  It shares no code, header,
 * table or helper with attention_prefill_amd/ and never calls into it.
 *
 * What it computes (the plain definition, not the fused method):
 *
 *   For every batch element (or packed sequence) s, query head h, query row i
 *     O[s,h,i,:] = sum_j P[i,j] * V[s,hk,j,:],   P[i,.] = softmax_j(S[i,j])
 *   over the visible keys j, with hk = h / (n_qh / n_kvh) and
 *     S[i,j] = scale * <Q[s,h,i,:], K[s,hk,j,:]>              (FP16 cell)
 *     S[i,j] = scale * s_q[i] * s_k[j] * sum_d q8[i,d]*k8[j,d]  (INT8 cell)
 *
 * Sources (the pages this follows):
 *  - "Nax Refactor" (ml-explore/mlx pull request 3271), the before/after
 *    attention timing tables: the operation is fused scaled-dot-product
 *    attention over (B, qsl, ksl, hdim, n_qh, n_kvh, causal) in float16;
 *    n_kvh < n_qh rows are grouped-query attention; the qsl=512, ksl=4096
 *    causal rows take about as long as the non-causal ones, which only a
 *    bottom-right aligned mask allows.
 *  - TileMix (Lattice paper summary), abstract: score tiles, compact routing
 *    bitmasks, each tile group computed through FP16 or INT8 scores, one
 *    shared online-softmax state, one routing bit per group of adjacent key
 *    tiles, all legal tile groups routed, grouped-query attention and
 *    variable-length batches supported.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - GQA head map is blocked: hk = h / G.
 *  - Causal masks are bottom-right aligned: key j is visible to row i iff
 *    j <= i + (ksl - qsl).  causal with qsl > ksl is rejected.
 *  - Packed variable-length input is head-major [H, T, d] with cu_seqlens
 *    (B+1 int32, cu[0] = 0, non-decreasing); qsl = ksl = T; each sequence
 *    is causal or not as the flag says.
 *  - INT8 quantisation is per token (row of Q per query head, row of K per
 *    kv head), symmetric: amax = max|x|; if amax == 0 then s = 0 and q8 = 0;
 *    else s = fl32(amax/127), inv = fl32(127/amax) (both IEEE fp32 divides),
 *    q8 = RNE(x * inv) with the product taken exactly.  V is never quantised.
 *  - The bitmask holds one bit per (q-tile, key-tile group), shared by all
 *    heads and batch elements; rows of wpr = ceil(n_groups/32) uint32 words,
 *    bit g of row qt is (w[qt*wpr + g/32] >> (g%32)) & 1; 1 = INT8.
 *    Tile indices count from row 0 of Q and row 0 of K.
 *  - Packed batches with a bitmask: every sequence s has its own rows, one
 *    per query tile of that sequence (tiles counted from its start), stacked
 *    in sequence order; row r0(s) = sum over s' < s of ceil(L_s'/tile_q).
 *    All rows have wpr words for the packed length T; bits of groups past a
 *    sequence's own key tiles are never read.
 *  - INT8 key/value caches (oracle_attn_fwd_kv8): K and V arrive as INT8
 *    codes with one fp32 scale per row, made by the same quantiser; the
 *    keys and values they stand for are K^ = s_k * k8 and V^ = s_v * v8.
 *    FP16 cells take the fp16 query against K^; INT8 cells take the
 *    quantised query against the cached codes (no second quantisation of
 *    K^); the output weights V^.
 *  - FP8 route (oracle_attn_fwd_lowp with lowp = 1): a set routing bit
 *    selects FP8 instead of INT8 for the whole call.  The format is e4m3
 *    (bias 7, largest finite 448, no infinities) with rowwise dynamic
 *    scaling read from "Add rowwise scaling to Float8Inference module":
 *    s = fl32(amax/448), codes = e4m3 nearest to x * fl32(448/amax) (product
 *    exact, ties to even, zero results +0); cells take
 *    scale * s_q * s_k * sum_d e4m3(q) * e4m3(k), exact in fp64.
 *  - Output is the exact fp64 result; a fp16 round-to-nearest-even encoder
 *    is provided for exact special cases.
 *
 * Parallelism: OpenMP over query rows inside one (s, h).  Heads run one
 * after another so only one score matrix is alive at a time.
 */
#include "oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* IEEE binary16 <-> double, written out from the format definition.       */
/* ---------------------------------------------------------------------- */

double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)m, -24);               /* subnormal or zero */
    else if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + m), e - 25);   /* 1.m * 2^(e-15) */
    return sign ? -mag : mag;
}

uint16_t oracle_f64_to_f16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    if (a >= 65520.0)                               /* rounds to infinity */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {                      /* subnormal binade */
        double m = nearbyint(ldexp(a, 24));         /* exact scale, one rounding */
        return sign | (uint16_t)m;                  /* m == 1024 is the smallest normal */
    }
    int E;
    frexp(a, &E);                                   /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                                  /* a in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(a, 10 - e));         /* in [1024, 2048] */
    if (m == 2048.0) { m = 1024.0; e += 1; }
    if (e > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* ---------------------------------------------------------------------- */
/* Per-token symmetric INT8 quantisation (TileMix abstract: INT8 score     */
/* computation; scale rule and rounding are the stated reading).           */
/* ---------------------------------------------------------------------- */

void oracle_quantize_row(const uint16_t* x, int d, int8_t* q8, float* s_out)
{
    float amax = 0.0f;
    for (int t = 0; t < d; ++t) {
        float a = (float)fabs(oracle_f16_to_f64(x[t]));   /* exact in fp32 */
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int t = 0; t < d; ++t) q8[t] = 0;
        *s_out = 0.0f;
        return;
    }
    volatile float num = 127.0f;     /* keep both divides as single fp32 ops */
    float s = amax / num;
    float inv = num / amax;
    for (int t = 0; t < d; ++t) {
        double prod = oracle_f16_to_f64(x[t]) * (double)inv;  /* exact: 11 x 24 bits */
        double r = nearbyint(prod);                           /* ties to even */
        if (r > 127.0) r = 127.0;
        if (r < -127.0) r = -127.0;
        q8[t] = (int8_t)r;
    }
    *s_out = s;
}

/* ---------------------------------------------------------------------- */
/* Routing bitmask (TileMix abstract: compact bitmasks, one bit per group  */
/* of adjacent key tiles).                                                 */
/* ---------------------------------------------------------------------- */

/* ---------------------------------------------------------------------- */
/* FP8 e4m3 ("e4m3fn": sign, 4 exponent bits with bias 7, 3 mantissa bits; */
/* no infinities; 0x7f and 0xff are NaN; largest finite value 448)         */
/* ---------------------------------------------------------------------- */

double oracle_e4m3_decode(uint8_t c)
{
    int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (c & 0x80) ? -v : v;
}

/* The e4m3 value nearest to y, ties to the even mantissa, limited to +-448;
 * a result of zero is +0.  The spacing of e4m3 values near |y| is
 * 2^(e-3) with e = max(floor(log2|y|), -6) (the subnormal spacing is 2^-9). */
double oracle_e4m3_round(double y)
{
    if (y == 0.0) return 0.0;
    double a = fabs(y);
    int E;
    frexp(a, &E);                    /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;
    if (e < -6) e = -6;
    double q = ldexp(1.0, e - 3);
    double r = nearbyint(a / q) * q; /* a / q is exact; nearbyint rounds ties to even */
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return 0.0;
    return y < 0 ? -r : r;
}

/* Bit pattern of an exact e4m3 value (zero encodes as 0x00). */
uint8_t oracle_e4m3_encode(double r)
{
    if (r == 0.0) return 0;
    double a = fabs(r);
    int E;
    frexp(a, &E);
    int e = E - 1;
    uint8_t code;
    if (e < -6) {
        code = (uint8_t)(a / ldexp(1.0, -9));                    /* subnormal: m * 2^-9 */
    } else {
        int m = (int)((a / ldexp(1.0, e) - 1.0) * 8.0);          /* (1 + m/8) * 2^e */
        code = (uint8_t)(((e + 7) << 3) | m);
    }
    return (uint8_t)(code | (r < 0 ? 0x80 : 0));
}

/* Rowwise dynamic FP8 codes of one fp16 row ("Add rowwise scaling to
 * Float8Inference module", rowwise / axiswise dynamic scaling, read with
 * e4m3 and its largest finite value 448): amax = max |x|, s = fl32(amax/448),
 * inv = fl32(448/amax), code = e4m3 nearest to x * inv (product exact); a
 * zero row has s = 0 and codes 0. */
void oracle_quantize_row_fp8(const uint16_t* x, int d, uint8_t* codes, float* s_out)
{
    float amax = 0.0f;
    for (int t = 0; t < d; ++t) {
        float a = (float)fabs(oracle_f16_to_f64(x[t]));
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        for (int t = 0; t < d; ++t) codes[t] = 0;
        *s_out = 0.0f;
        return;
    }
    volatile float num = 448.0f;     /* keep both divides as single fp32 ops */
    float s = amax / num;
    float inv = num / amax;
    for (int t = 0; t < d; ++t)
        codes[t] = oracle_e4m3_encode(oracle_e4m3_round(oracle_f16_to_f64(x[t]) * (double)inv));
    *s_out = s;
}

/* Every row of an [rows, d] fp16 array, by oracle_quantize_row. */
void oracle_quantize_rows(const uint16_t* x, long long rows, int d, int8_t* q8, float* s_out)
{
    for (long long r = 0; r < rows; ++r)
        oracle_quantize_row(x + (size_t)r * d, d, q8 + (size_t)r * d, s_out + r);
}

int oracle_route_words_per_row(int ksl, int tile_k, int tiles_per_bit)
{
    int n_kt = (ksl + tile_k - 1) / tile_k;
    int n_g = (n_kt + tiles_per_bit - 1) / tiles_per_bit;
    return (n_g + 31) / 32;
}

int oracle_route_bit(const uint32_t* words, int wpr, int qt, int g)
{
    return (int)((words[(size_t)qt * wpr + (size_t)(g / 32)] >> (g % 32)) & 1u);
}

/* ---------------------------------------------------------------------- */
/* Attention                                                               */
/* ---------------------------------------------------------------------- */

typedef struct {
    const uint16_t *q, *k, *v;
    /* INT8 key/value cache mode (k and v unused): codes and per-row scales */
    const int8_t *k8, *v8;
    const float *sk, *sv;
    int B, qsl, ksl, d, n_qh, n_kvh, causal;
    double scale;
    const int32_t* cu;
    const uint32_t* route;
    int tiles_per_bit, tile_q, tile_k, wpr;
    int lowp;                 /* what a set routing bit selects: 0 INT8, 1 FP8 e4m3 */
} problem;

/* Offsets of sequence s, head h in the dense [B,H,S,d] or packed [H,T,d]
 * layouts, and the lengths (Lq, Lk) of that sequence. */
static size_t q_base(const problem* p, int s, int h, int* Lq)
{
    if (p->cu) {
        int T = p->cu[p->B];
        *Lq = p->cu[s + 1] - p->cu[s];
        return ((size_t)h * T + (size_t)p->cu[s]) * p->d;
    }
    *Lq = p->qsl;
    return (((size_t)s * p->n_qh + h) * p->qsl) * p->d;
}

static size_t kv_base(const problem* p, int s, int hk, int* Lk)
{
    if (p->cu) {
        int T = p->cu[p->B];
        *Lk = p->cu[s + 1] - p->cu[s];
        return ((size_t)hk * T + (size_t)p->cu[s]) * p->d;
    }
    *Lk = p->ksl;
    return (((size_t)s * p->n_kvh + hk) * p->ksl) * p->d;
}

/* First bitmask row of sequence s: 0 for dense input (rows are shared by the
 * batch), else the query tiles of the sequences before it. */
static int route_row0(const problem* p, int s)
{
    if (!p->cu) return 0;
    int r = 0;
    for (int t = 0; t < s; ++t) {
        int L = p->cu[t + 1] - p->cu[t];
        r += (L + p->tile_q - 1) / p->tile_q;
    }
    return r;
}

static int visible(const problem* p, int i, int j, int Lq, int Lk)
{
    return !p->causal || j <= i + (Lk - Lq);
}

/* Value t of key / value row j of the slab starting at element kb: the fp16
 * tensor's value, or in cache mode the dequantised s * code (exact in fp64). */
static double key_val(const problem* p, size_t kb, int j, int t)
{
    if (p->k8) return (double)p->sk[kb / p->d + j] * (double)p->k8[kb + (size_t)j * p->d + t];
    return oracle_f16_to_f64(p->k[kb + (size_t)j * p->d + t]);
}

static double val_val(const problem* p, size_t kb, int j, int t)
{
    if (p->v8) return (double)p->sv[kb / p->d + j] * (double)p->v8[kb + (size_t)j * p->d + t];
    return oracle_f16_to_f64(p->v[kb + (size_t)j * p->d + t]);
}

/* Codes of one row in the routed low-precision format (FP8 codes are kept as
 * their bit patterns in the int8 array). */
static void quantize_one(const problem* p, const uint16_t* x, int8_t* codes, float* s)
{
    if (p->lowp == 1) oracle_quantize_row_fp8(x, p->d, (uint8_t*)codes, s);
    else oracle_quantize_row(x, p->d, codes, s);
}

/* Quantised rows for one (s, head) slab of L rows, or NULL when unrouted. */
typedef struct { int8_t* q8; float* s; } qrows;

static qrows quantize_slab(const problem* p, const uint16_t* base, int L)
{
    qrows r = { NULL, NULL };
    if (!p->route || L == 0) return r;
    r.q8 = (int8_t*)malloc((size_t)L * p->d);
    r.s = (float*)malloc((size_t)L * sizeof(float));
    for (int i = 0; i < L; ++i)
        quantize_one(p, base + (size_t)i * p->d, r.q8 + (size_t)i * p->d, r.s + i);
    return r;
}

static void free_qrows(qrows r) { free(r.q8); free(r.s); }

/* INT8 K rows of the slab starting at element kb: quantised from the fp16
 * keys, or in cache mode the cached codes and scales themselves. */
static qrows key_codes(const problem* p, size_t kb, int L)
{
    if (p->k8) {
        qrows r = { NULL, NULL };
        if (!p->route || L == 0) return r;
        r.q8 = (int8_t*)malloc((size_t)L * p->d);
        r.s = (float*)malloc((size_t)L * sizeof(float));
        memcpy(r.q8, p->k8 + kb, (size_t)L * p->d);
        memcpy(r.s, p->sk + kb / p->d, (size_t)L * sizeof(float));
        return r;
    }
    return quantize_slab(p, p->k + kb, L);
}

/* Scores of query row i against all Lk keys; masked cells get -inf. */
static void score_row(const problem* p, const uint16_t* qrow, size_t kb,
                      const qrows* qq, const qrows* kq, int i, int Lq, int Lk, int rrow0,
                      double* S)
{
    int qt = rrow0 + i / p->tile_q;
    for (int j = 0; j < Lk; ++j) {
        if (!visible(p, i, j, Lq, Lk)) { S[j] = -INFINITY; continue; }
        int int8_cell = 0;
        if (p->route) {
            int g = (j / p->tile_k) / p->tiles_per_bit;
            int8_cell = oracle_route_bit(p->route, p->wpr, qt, g);
        }
        if (int8_cell) {
            const int8_t* a = qq->q8 + (size_t)i * p->d;
            const int8_t* b = kq->q8 + (size_t)j * p->d;
            double dot;
            if (p->lowp == 1) {
                /* products of two e4m3 values have at most 8 significant bits
                 * between 2^-18 and 2^18, so the fp64 sum is exact */
                dot = 0.0;
                for (int t = 0; t < p->d; ++t)
                    dot += oracle_e4m3_decode((uint8_t)a[t]) * oracle_e4m3_decode((uint8_t)b[t]);
            } else {
                int64_t idot = 0;
                for (int t = 0; t < p->d; ++t) idot += (int64_t)a[t] * (int64_t)b[t];
                dot = (double)idot;
            }
            S[j] = p->scale * (double)qq->s[i] * (double)kq->s[j] * dot;
        } else {
            /* fp16 x fp16 and fp16 x (fp32 * int8) products are exact in fp64 */
            double acc = 0.0;
            for (int t = 0; t < p->d; ++t)
                acc += oracle_f16_to_f64(qrow[t]) * key_val(p, kb, j, t);
            S[j] = p->scale * acc;
        }
    }
}

/* In-place row softmax over Lk cells (base e), then out = P . V. */
static void softmax_pv_row(const problem* p, double* S, int Lk, size_t kb, double* out)
{
    double m = -INFINITY;
    for (int j = 0; j < Lk; ++j) if (S[j] > m) m = S[j];
    double l = 0.0;
    for (int j = 0; j < Lk; ++j) {
        S[j] = (S[j] == -INFINITY) ? 0.0 : exp(S[j] - m);
        l += S[j];
    }
    for (int t = 0; t < p->d; ++t) out[t] = 0.0;
    for (int j = 0; j < Lk; ++j) {
        if (S[j] == 0.0) continue;
        double pj = S[j] / l;
        for (int t = 0; t < p->d; ++t) out[t] += pj * val_val(p, kb, j, t);
    }
}

static int check_problem(const problem* p)
{
    if (!p->q) return ORACLE_ERR_ARG;
    if (p->k8 ? (!p->v8 || !p->sk || !p->sv) : (!p->k || !p->v)) return ORACLE_ERR_ARG;
    if (p->B <= 0 || p->qsl <= 0 || p->ksl <= 0 || p->d <= 0 || p->n_qh <= 0 || p->n_kvh <= 0)
        return ORACLE_ERR_ARG;
    if (p->n_qh % p->n_kvh) return ORACLE_ERR_ARG;
    if (p->causal && p->qsl > p->ksl) return ORACLE_ERR_ARG;
    if (p->cu) {
        if (p->qsl != p->ksl || p->cu[0] != 0 || p->cu[p->B] != p->qsl) return ORACLE_ERR_ARG;
        for (int s = 0; s < p->B; ++s) if (p->cu[s + 1] < p->cu[s]) return ORACLE_ERR_ARG;
    }
    if (p->route && (p->tiles_per_bit < 1 || p->tile_q < 1 || p->tile_k < 1)) return ORACLE_ERR_ARG;
    if (p->lowp != 0 && p->lowp != 1) return ORACLE_ERR_ARG;
    if (p->lowp == 1 && p->k8) return ORACLE_ERR_ARG;   /* an INT8 cache has no FP8 codes */
    return 0;
}

static problem make_problem(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                            float scale, int causal, const int32_t* cu,
                            const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k)
{
    problem p;
    p.q = q; p.k = k; p.v = v;
    p.k8 = NULL; p.v8 = NULL; p.sk = NULL; p.sv = NULL;
    p.B = B; p.qsl = qsl; p.ksl = ksl; p.d = d; p.n_qh = n_qh; p.n_kvh = n_kvh;
    p.causal = causal ? 1 : 0;
    p.scale = (double)scale;                 /* caller's fp32 scale, widened */
    p.cu = cu; p.route = route;
    p.tiles_per_bit = tiles_per_bit;
    p.tile_q = tile_q > 0 ? tile_q : 64;
    p.tile_k = tile_k > 0 ? tile_k : 64;
    p.wpr = route ? oracle_route_words_per_row(ksl, p.tile_k, tiles_per_bit > 0 ? tiles_per_bit : 1) : 0;
    p.lowp = 0;
    return p;
}

static int run_fwd(problem p, double* out, int nthreads)
{
    const uint16_t* q = p.q;
    const int B = p.B, d = p.d, n_qh = p.n_qh, n_kvh = p.n_kvh;
    int rc = check_problem(&p);
    if (rc) return rc;
    if (!out) return ORACLE_ERR_ARG;
    int fe = fegetround();
    fesetround(FE_TONEAREST);
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
    int G = n_qh / n_kvh;
    for (int s = 0; s < B; ++s) {
        const int rrow0 = route_row0(&p, s);
        for (int hk = 0; hk < n_kvh; ++hk) {
            int Lk;
            size_t kb = kv_base(&p, s, hk, &Lk);
            qrows kq = key_codes(&p, kb, Lk);
            for (int h = hk * G; h < (hk + 1) * G; ++h) {
                int Lq;
                size_t qb = q_base(&p, s, h, &Lq);
                if (Lq == 0) continue;
                qrows qq = quantize_slab(&p, q + qb, Lq);
                /* the whole Lq x Lk score matrix of this (s, h) */
                double* S = (double*)malloc((size_t)Lq * (size_t)(Lk > 0 ? Lk : 1) * sizeof(double));
                if (!S) { free_qrows(qq); free_qrows(kq); fesetround(fe); return ORACLE_ERR_NOMEM; }
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
#endif
                for (int i = 0; i < Lq; ++i)
                    score_row(&p, q + qb + (size_t)i * d, kb, &qq, &kq, i, Lq, Lk, rrow0,
                              S + (size_t)i * Lk);
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
#endif
                for (int i = 0; i < Lq; ++i)
                    softmax_pv_row(&p, S + (size_t)i * Lk, Lk, kb, out + qb + (size_t)i * d);
                free(S);
                free_qrows(qq);
            }
            free_qrows(kq);
        }
    }
    fesetround(fe);
    return 0;
}

static int run_rows(problem p, const int32_t* rows, int nrows, double* out, int nthreads)
{
    const uint16_t* q = p.q;
    const int B = p.B, d = p.d, n_qh = p.n_qh, n_kvh = p.n_kvh;
    int rc = check_problem(&p);
    if (rc) return rc;
    if (!out || !rows || nrows < 0) return ORACLE_ERR_ARG;
    for (int r = 0; r < nrows; ++r) {
        int s = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        int Lq;
        if (s < 0 || s >= B || h < 0 || h >= n_qh || i < 0) return ORACLE_ERR_ARG;
        q_base(&p, s, h, &Lq);
        if (i >= Lq) return ORACLE_ERR_ARG;
    }
    int fe = fegetround();
    fesetround(FE_TONEAREST);
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
#endif
    int G = n_qh / n_kvh;
    int err = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (int r = 0; r < nrows; ++r) {
        int s = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        int hk = h / G, Lq, Lk;
        size_t qb = q_base(&p, s, h, &Lq);
        size_t kb = kv_base(&p, s, hk, &Lk);
        qrows qq = { NULL, NULL }, kq = { NULL, NULL };
        if (p.route) {
            /* the row needs its own quantised Q row and every quantised K row */
            qq.q8 = (int8_t*)malloc((size_t)(i + 1) * d);
            qq.s = (float*)malloc((size_t)(i + 1) * sizeof(float));
            quantize_one(&p, q + qb + (size_t)i * d, qq.q8 + (size_t)i * d, qq.s + i);
            kq = key_codes(&p, kb, Lk);
        }
        double* S = (double*)malloc((size_t)(Lk > 0 ? Lk : 1) * sizeof(double));
        if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = ORACLE_ERR_NOMEM;
        } else {
            score_row(&p, q + qb + (size_t)i * d, kb, &qq, &kq, i, Lq, Lk, route_row0(&p, s), S);
            softmax_pv_row(&p, S, Lk, kb, out + (size_t)r * d);
            free(S);
        }
        free_qrows(qq);
        free_qrows(kq);
    }
    fesetround(fe);
    return err;
}

int oracle_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* out,
                    int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                    float scale, int causal, const int32_t* cu_seqlens,
                    const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                    int nthreads)
{
    return run_fwd(make_problem(q, k, v, B, qsl, ksl, d, n_qh, n_kvh, scale, causal,
                                cu_seqlens, route, tiles_per_bit, tile_q, tile_k),
                   out, nthreads);
}

int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                     float scale, int causal, const int32_t* cu_seqlens,
                     const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                     const int32_t* rows, int nrows, double* out, int nthreads)
{
    return run_rows(make_problem(q, k, v, B, qsl, ksl, d, n_qh, n_kvh, scale, causal,
                                 cu_seqlens, route, tiles_per_bit, tile_q, tile_k),
                    rows, nrows, out, nthreads);
}

/* INT8 key/value cache ("INT8 key/value caches", TileMix abstract): K and V
 * arrive as per-token INT8 codes with fp32 scales, K^ = s_k * k8 and
 * V^ = s_v * v8.  FP16 cells score the fp16 query against K^, INT8 cells use
 * the cached codes as the key side of the integer dot product, and the
 * output weights V^. */
static problem make_problem_kv8(const uint16_t* q, const int8_t* k8, const float* sk,
                                const int8_t* v8, const float* sv,
                                int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                                float scale, int causal, const int32_t* cu,
                                const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k)
{
    problem p = make_problem(q, NULL, NULL, B, qsl, ksl, d, n_qh, n_kvh, scale, causal,
                             cu, route, tiles_per_bit, tile_q, tile_k);
    p.k8 = k8; p.sk = sk; p.v8 = v8; p.sv = sv;
    return p;
}

int oracle_attn_fwd_kv8(const uint16_t* q, const int8_t* k8, const float* k_scale,
                        const int8_t* v8, const float* v_scale, double* out,
                        int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                        float scale, int causal, const int32_t* cu_seqlens,
                        const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                        int nthreads)
{
    return run_fwd(make_problem_kv8(q, k8, k_scale, v8, v_scale, B, qsl, ksl, d, n_qh, n_kvh,
                                    scale, causal, cu_seqlens, route, tiles_per_bit, tile_q, tile_k),
                   out, nthreads);
}

int oracle_attn_rows_kv8(const uint16_t* q, const int8_t* k8, const float* k_scale,
                         const int8_t* v8, const float* v_scale,
                         int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                         float scale, int causal, const int32_t* cu_seqlens,
                         const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                         const int32_t* rows, int nrows, double* out, int nthreads)
{
    return run_rows(make_problem_kv8(q, k8, k_scale, v8, v_scale, B, qsl, ksl, d, n_qh, n_kvh,
                                     scale, causal, cu_seqlens, route, tiles_per_bit, tile_q, tile_k),
                    rows, nrows, out, nthreads);
}

/* The TileMix route with FP8 e4m3 as the low-precision format: cells whose
 * bit is set take scale * s_q * s_k * sum_d e4m3(q8) * e4m3(k8) with the
 * rowwise FP8 codes above (lowp = 1); lowp = 0 is oracle_attn_fwd. */
int oracle_attn_fwd_lowp(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* out,
                         int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                         float scale, int causal, const int32_t* cu_seqlens,
                         const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                         int lowp, int nthreads)
{
    problem p = make_problem(q, k, v, B, qsl, ksl, d, n_qh, n_kvh, scale, causal,
                             cu_seqlens, route, tiles_per_bit, tile_q, tile_k);
    p.lowp = lowp;
    return run_fwd(p, out, nthreads);
}

int oracle_attn_rows_lowp(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          int B, int qsl, int ksl, int d, int n_qh, int n_kvh,
                          float scale, int causal, const int32_t* cu_seqlens,
                          const uint32_t* route, int tiles_per_bit, int tile_q, int tile_k,
                          int lowp, const int32_t* rows, int nrows, double* out, int nthreads)
{
    problem p = make_problem(q, k, v, B, qsl, ksl, d, n_qh, n_kvh, scale, causal,
                             cu_seqlens, route, tiles_per_bit, tile_q, tile_k);
    p.lowp = lowp;
    return run_rows(p, rows, nrows, out, nthreads);
}
