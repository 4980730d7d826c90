/*
 * CPU oracle for the 8-bit (SageAttention-form) attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP path under bit_quantized_exact_amd/.
 *
 * It is deliberately plain and slow: fp64 loops, two-pass softmax, no tiling,
 * no online rescaling, no blocking beyond what the definitions state.  The one
 * exception is O5, the 8-bit P.V model: there the rounding of each weight is
 * defined relative to the online softmax's running maximum, so O5 follows the
 * online algorithm over key tiles, step by step as the pages describe it.
 *
 * Sources (web pages; cited by title and section):
 *   [MHA-GQA]  "注意力即一切：从 MHA 到 GQA" (bojinhu.xyz):
 *              §2.2 (the four steps of attention), §2.3 (causal mask),
 *              §4.1 (MQA), §5.1 (GQA grouping).
 *   [SA]       "又快又准，即插即用！清华8比特量化Attention，两倍加速于
 *              FlashAttention2…" (SageAttention, 17aitech reprint of a
 *              jiqizhixin article), section 技术方案 ("technical approach"):
 *              K smoothing, per-block INT8 Q/K, INT8 QK^T with INT32
 *              accumulation, FP16 P and V.
 *   [FA-guide] "FlashAttention" guide (aiunderstanding.org): FAQ on exactness.
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes of the repository):
 *   - mean(K) is the per-channel mean over all tokens of one (batch, kv-head),
 *     the only reading under which [SA]'s claimed invariance
 *     softmax(QK^T) = softmax(Q(K-mean K)^T) holds.
 *   - The channel sum is exact; it is rounded once to fp64, divided by S in
 *     fp64 and rounded to fp32.
 *   - Block quantisation is symmetric absmax: a = max|x|, r = 127/a (fp32,
 *     round-to-nearest-even), q = clamp(rint(x*r), -127, 127), delta = a/127.
 *     An all-zero block gives q = 0, delta = 0.
 *   - Q is not smoothed.  1/sqrt(D) is applied at dequantisation, not folded
 *     into Q before quantisation.
 *   - Causal means key j is visible to query i iff j <= i (one sequence length).
 *     With a KV cache (Sq queries, Sk cached keys) the queries are the last Sq
 *     positions: query i sees keys j <= Sk - Sq + i (bottom-right alignment).
 *   - A row with no visible key (cannot happen for square causal) gives O = 0
 *     and lse = -inf.
 *   - FP8 means OCP E4M3 (bias 7, max 448, no infinities).  FP8 Q/K blocks use
 *     the INT8 rule with 448 in place of 127 and E4M3 rounding (nearest, ties
 *     to even) in place of rint + clamp.  8-bit P is E4M3(448 p) / 448 with p
 *     <= 1 taken against the running maximum; 8-bit V has one E4M3 scale per
 *     (batch, kv-head, channel) over all tokens.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ------------------------------------------------------------------------ */
/* IEEE binary16 decoding (from the format definition: 1 sign bit, 5       */
/* exponent bits with bias 15, 10 fraction bits; exponent 0 = subnormal,    */
/* exponent 31 = inf/nan).                                                  */
/* ------------------------------------------------------------------------ */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);                 /* frac * 2^-10 * 2^-14 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);  /* 1.frac * 2^(e-15)   */
    }
    return sign ? -v : v;
}

void oracle_half_array_to_double(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_half_to_double(h[i]);
}

/* Round a finite double to the nearest binary16 value (ties to even),
 * returned as a double.  Values beyond the fp16 range saturate to +-inf. */
double oracle_round_to_half(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                 /* ax = m * 2^e, m in [0.5, 1) */
    int ulp_exp = (e - 1) - 10;    /* 11 significant bits in the normal range */
    if (ulp_exp < -24) ulp_exp = -24;  /* subnormal spacing */
    double r = ldexp(rint(ldexp(ax, -ulp_exp)), ulp_exp);
    if (r > 65504.0) r = INFINITY;
    return x < 0 ? -r : r;
}

static double* decode_all(const uint16_t* h, int64_t n)
{
    double* d = (double*)malloc((size_t)n * sizeof(double));
    if (!d) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) d[i] = oracle_half_to_double(h[i]);
    return d;
}

static int check_map(int Hq, int Hkv, const int32_t* kv_map)
{
    for (int h = 0; h < Hq; ++h)
        if (kv_map[h] < 0 || kv_map[h] >= Hkv) return -4;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O1: exact attention in fp64 ([MHA-GQA] §2.2, §2.3, §5.1).                */
/*   s_ij = sm_scale * sum_c Q[b,h,i,c] K[b,map[h],j,c]  (visible j only)   */
/*   p_ij = exp(s_ij - max_j s_ij), l_i = sum_j p_ij                        */
/*   O[b,h,i,:] = sum_j p_ij V[b,map[h],j,:] / l_i ; lse_i = m_i + ln l_i   */
/* rows: query rows to evaluate for every (b,h) (NULL = all S rows).        */
/* out: [B, Hq, nrows, D] fp64; lse: [B, Hq, nrows] or NULL.                */
/* ------------------------------------------------------------------------ */
int oracle_attention(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                     const uint16_t* q_f16, const uint16_t* k_f16, const uint16_t* v_f16,
                     const int32_t* kv_map, int32_t causal, double sm_scale,
                     const int32_t* rows, int32_t nrows,
                     double* out, double* lse, int32_t nthreads)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0) return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (!rows) nrows = S;
    if (nthreads > 0) omp_set_num_threads(nthreads);

    int64_t nkv = (int64_t)B * Hkv * S * D;
    double* K = decode_all(k_f16, nkv);
    double* V = decode_all(v_f16, nkv);
    if (!K || !V) { free(K); free(V); return -5; }

    int64_t total = (int64_t)B * Hq * nrows;
    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)S * sizeof(double));
        double* qrow = (double*)malloc((size_t)D * sizeof(double));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !qrow || !acc) {
#pragma omp atomic write
            status = -5;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < total; ++t) {
                int64_t bh = t / nrows;
                int32_t r = (int32_t)(t % nrows);
                int32_t i = rows ? rows[r] : r;
                int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
                int32_t kh = kv_map[h];
                const uint16_t* qp = q_f16 + (((int64_t)b * Hq + h) * S + i) * D;
                const double* Kh = K + ((int64_t)b * Hkv + kh) * S * D;
                const double* Vh = V + ((int64_t)b * Hkv + kh) * S * D;
                double* o = out + t * D;
                for (int c = 0; c < D; ++c) qrow[c] = oracle_half_to_double(qp[c]);

                int32_t nvis = causal ? (i + 1 < S ? i + 1 : S) : S;
                if (nvis <= 0) {
                    for (int c = 0; c < D; ++c) o[c] = 0.0;
                    if (lse) lse[t] = -INFINITY;
                    continue;
                }
                /* pass 1: scores and their maximum */
                double m = -INFINITY;
                for (int32_t j = 0; j < nvis; ++j) {
                    double dot = 0.0;
                    for (int c = 0; c < D; ++c) dot += qrow[c] * Kh[(int64_t)j * D + c];
                    s[j] = dot * sm_scale;
                    if (s[j] > m) m = s[j];
                }
                /* pass 2: weights, their sum and the weighted sum of V */
                double l = 0.0;
                for (int c = 0; c < D; ++c) acc[c] = 0.0;
                for (int32_t j = 0; j < nvis; ++j) {
                    double p = exp(s[j] - m);
                    l += p;
                    for (int c = 0; c < D; ++c) acc[c] += p * Vh[(int64_t)j * D + c];
                }
                for (int c = 0; c < D; ++c) o[c] = acc[c] / l;
                if (lse) lse[t] = m + log(l);
            }
        }
        free(s); free(qrow); free(acc);
    }
    free(K); free(V);
    return status;
}

/* ------------------------------------------------------------------------ */
/* O2: K channel mean over tokens ([SA] 技术方案, K smoothing).             */
/*   sum_c = sum over all S tokens of K[b,k,:,c], accumulated in fp64.      */
/*   Every fp16 value is an integer multiple of 2^-24, so the fp64 sum is   */
/*   exact while every partial sum stays below 2^29 in magnitude; the       */
/*   function checks sum_j |K| < 2^29 per channel and returns -4 if not.    */
/*   mu_c = (float)(sum_c / S) : one fp64 division, then RNE to fp32.       */
/* ------------------------------------------------------------------------ */
int oracle_k_mean(int32_t B, int32_t Hkv, int32_t S, int32_t D,
                  const uint16_t* k_f16, float* mu)
{
    if (B <= 0 || Hkv <= 0 || S <= 0 || D <= 0) return -1;
    int status = 0;
    for (int64_t bk = 0; bk < (int64_t)B * Hkv; ++bk) {
        const uint16_t* Kh = k_f16 + bk * S * D;
        for (int c = 0; c < D; ++c) {
            double sum = 0.0, sabs = 0.0;
            for (int32_t j = 0; j < S; ++j) {
                double x = oracle_half_to_double(Kh[(int64_t)j * D + c]);
                sum += x;
                sabs += fabs(x);
            }
            if (!(sabs < 536870912.0)) status = -4;   /* 2^29 */
            mu[bk * D + c] = (float)(sum / (double)S);
        }
    }
    return status;
}

/* Smoothed K in fp32: ks = (float)K - mu  (one fp32 subtraction).          */
void oracle_smooth_k(int32_t B, int32_t Hkv, int32_t S, int32_t D,
                     const uint16_t* k_f16, const float* mu, float* ks)
{
    for (int64_t bk = 0; bk < (int64_t)B * Hkv; ++bk)
        for (int32_t j = 0; j < S; ++j)
            for (int c = 0; c < D; ++c) {
                int64_t idx = (bk * S + j) * D + c;
                float x = (float)oracle_half_to_double(k_f16[idx]);
                ks[idx] = x - mu[bk * D + c];
            }
}

/* fp16 -> fp32 widening of a whole array (exact).                          */
void oracle_half_array_to_float(const uint16_t* h, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (float)oracle_half_to_double(h[i]);
}

/* ------------------------------------------------------------------------ */
/* O3: per-block symmetric INT8 quantisation ([SA] 技术方案: Q and K are    */
/* quantised to INT8 with one scale per FlashAttention-sized block).        */
/* x: [nmat, S, D] fp32.  Block b covers rows [b*block, min(S,(b+1)*block)) */
/* of one matrix (the last block may be partial).                           */
/* q: [nmat, S, D] int8;  scale: [nmat, ceil(S/block)] fp32.                */
/* ------------------------------------------------------------------------ */
void oracle_quant_blocks(int64_t nmat, int32_t S, int32_t D, int32_t block,
                         const float* x, int8_t* q, float* scale)
{
    int32_t nblk = (S + block - 1) / block;
    for (int64_t mtx = 0; mtx < nmat; ++mtx) {
        for (int32_t bi = 0; bi < nblk; ++bi) {
            int32_t r0 = bi * block, r1 = r0 + block < S ? r0 + block : S;
            const float* xb = x + (mtx * S + r0) * D;
            int8_t* qb = q + (mtx * S + r0) * D;
            int64_t n = (int64_t)(r1 - r0) * D;
            float a = 0.0f;
            for (int64_t e = 0; e < n; ++e) {
                float v = fabsf(xb[e]);
                if (v > a) a = v;
            }
            if (a == 0.0f) {
                for (int64_t e = 0; e < n; ++e) qb[e] = 0;
                scale[mtx * nblk + bi] = 0.0f;
                continue;
            }
            float r = 127.0f / a;
            for (int64_t e = 0; e < n; ++e) {
                float t = rintf(xb[e] * r);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
                qb[e] = (int8_t)t;
            }
            scale[mtx * nblk + bi] = a / 127.0f;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Integer scores ([SA] 技术方案: INT8 QK^T with an INT32 accumulator).     */
/*   S32[b,h,i,j] = sum_c q[b,h,i,c] * k[b,map[h],j,c], exact in int64,     */
/*   then checked to fit in int32.  Entries with j > i under the causal     */
/*   mask are set to `fill`.  s_out: [B, Hq, nrows, S].                     */
/* ------------------------------------------------------------------------ */
int oracle_scores_i32(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                      const int8_t* q_i8, const int8_t* k_i8, const int32_t* kv_map,
                      int32_t causal, const int32_t* rows, int32_t nrows,
                      int32_t* s_out, int32_t fill)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0) return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (!rows) nrows = S;
    int status = 0;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < (int64_t)B * Hq * nrows; ++t) {
        int64_t bh = t / nrows;
        int32_t r = (int32_t)(t % nrows);
        int32_t i = rows ? rows[r] : r;
        int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
        const int8_t* qp = q_i8 + (((int64_t)b * Hq + h) * S + i) * D;
        const int8_t* kp = k_i8 + ((int64_t)b * Hkv + kv_map[h]) * S * D;
        for (int32_t j = 0; j < S; ++j) {
            if (causal && j > i) { s_out[t * S + j] = fill; continue; }
            int64_t dot = 0;
            for (int c = 0; c < D; ++c) dot += (int64_t)qp[c] * (int64_t)kp[(int64_t)j * D + c];
            if (dot > INT32_MAX || dot < INT32_MIN) {
#pragma omp atomic write
                status = -4;
            }
            s_out[t * S + j] = (int32_t)dot;
        }
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* O4: the quantised-attention model (diagnostic).  Exact softmax attention */
/* whose scores are the dequantised integer scores                          */
/*   s_ij = S32_ij * dQ[i/BQ] * dK[j/BK] * sm_scale          (fp64)         */
/* and whose weights enter the P.V product rounded to fp16 ([SA] 技术方案:  */
/* P and V stay FP16).  The row sum l uses the unrounded weights when       */
/* l_from_rounded == 0 and the fp16-rounded ones otherwise.                 */
/* ------------------------------------------------------------------------ */
int oracle_quant_attention(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                           const int8_t* q_i8, const float* q_scale, int32_t bq,
                           const int8_t* k_i8, const float* k_scale, int32_t bk,
                           const uint16_t* v_f16, const int32_t* kv_map,
                           int32_t causal, double sm_scale, int32_t l_from_rounded,
                           const int32_t* rows, int32_t nrows,
                           double* out, double* lse, int32_t nthreads)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || bq <= 0 || bk <= 0) return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (!rows) nrows = S;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int32_t nbq = (S + bq - 1) / bq, nbk = (S + bk - 1) / bk;

    int64_t nkv = (int64_t)B * Hkv * S * D;
    double* V = decode_all(v_f16, nkv);
    if (!V) return -5;
    int64_t total = (int64_t)B * Hq * nrows;
    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)S * sizeof(double));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !acc) {
#pragma omp atomic write
            status = -5;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < total; ++t) {
                int64_t bh = t / nrows;
                int32_t r = (int32_t)(t % nrows);
                int32_t i = rows ? rows[r] : r;
                int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
                int32_t kh = kv_map[h];
                const int8_t* qp = q_i8 + (((int64_t)b * Hq + h) * S + i) * D;
                const int8_t* Kh = k_i8 + ((int64_t)b * Hkv + kh) * S * D;
                const double* Vh = V + ((int64_t)b * Hkv + kh) * S * D;
                double dq = (double)q_scale[((int64_t)b * Hq + h) * nbq + i / bq];
                const float* dk = k_scale + ((int64_t)b * Hkv + kh) * nbk;
                double* o = out + t * D;
                int32_t nvis = causal ? (i + 1 < S ? i + 1 : S) : S;
                if (nvis <= 0) {
                    for (int c = 0; c < D; ++c) o[c] = 0.0;
                    if (lse) lse[t] = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (int32_t j = 0; j < nvis; ++j) {
                    int64_t dot = 0;
                    for (int c = 0; c < D; ++c) dot += (int64_t)qp[c] * (int64_t)Kh[(int64_t)j * D + c];
                    s[j] = (double)dot * dq * (double)dk[j / bk] * sm_scale;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int c = 0; c < D; ++c) acc[c] = 0.0;
                for (int32_t j = 0; j < nvis; ++j) {
                    double p = exp(s[j] - m);
                    double pr = oracle_round_to_half(p);
                    l += l_from_rounded ? pr : p;
                    for (int c = 0; c < D; ++c) acc[c] += pr * Vh[(int64_t)j * D + c];
                }
                for (int c = 0; c < D; ++c) o[c] = acc[c] / l;
                if (lse) lse[t] = m + log(l);
            }
        }
        free(s); free(acc);
    }
    free(V);
    return status;
}

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (the OCP "e4m3fn" format) from its definition: 1 sign bit, 4    */
/* exponent bits with bias 7, 3 fraction bits; exponent 0 is subnormal      */
/* (f * 2^-9); there is no infinity and S.1111.111 is NaN, so the largest   */
/* finite magnitude is 1.75 * 2^8 = 448.  Used for the FP8 alternative that */
/* the SageAttention article compares INT8 with ([SA] 技术方案: INT8 Q/K is */
/* more accurate than FP8; 8-bit P and V lose accuracy in some layers).     */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int expo = (c >> 3) & 0xf;
    int frac = c & 7;
    double v;
    if (expo == 15 && frac == 7) return NAN;
    if (expo == 0) v = ldexp((double)frac, -9);
    else v = ldexp((double)(8 + frac), expo - 10);      /* 1.fff * 2^(e-7) */
    return sign ? -v : v;
}

/* Nearest E4M3 value of x (ties to even); magnitudes that round beyond 448
 * saturate to 448.  The sign of x is kept (a negative x that rounds to zero
 * gives -0). */
double oracle_e4m3_round(double x)
{
    if (x == 0.0 || isnan(x)) return x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                  /* ax = m * 2^e, m in [0.5, 1) */
    int ulp_exp = (e - 1) - 3;      /* 4 significant bits in the normal range */
    if (ulp_exp < -9) ulp_exp = -9; /* subnormal spacing 2^-9 */
    double r = ldexp(rint(ldexp(ax, -ulp_exp)), ulp_exp);
    if (r > 448.0) r = 448.0;
    return signbit(x) ? -r : r;
}

/* Code of an E4M3 value (x must lie on the grid, |x| <= 448). */
uint8_t oracle_e4m3_encode(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double ax = fabs(x);
    if (ax == 0.0) return sign;
    if (ax < ldexp(1.0, -6)) return sign | (uint8_t)(ax * 512.0);   /* subnormal: f * 2^-9 */
    int e;
    double m = frexp(ax, &e);       /* ax = m * 2^e, m in [0.5, 1) -> 1.fff * 2^(e-1) */
    int expo = e - 1 + 7;
    int frac = (int)((m * 2.0 - 1.0) * 8.0);
    return sign | (uint8_t)(expo << 3) | (uint8_t)frac;
}

void oracle_e4m3_round_array(const double* x, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_round(x[i]);
}

void oracle_e4m3_decode_array(const uint8_t* c, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* O3 with an E4M3 grid instead of the INT8 one (the FP8 alternative): per */
/* block a = max|x|, r = 448/a (fp32, RNE), t = clamp(x*r, -448, 448) in    */
/* fp32, code = E4M3(t) (nearest, ties to even), delta = a/448.  a == 0     */
/* gives r = 0, codes of +-0 and delta = 0.                                 */
void oracle_quant_blocks_e4m3(int64_t nmat, int32_t S, int32_t D, int32_t block,
                              const float* x, uint8_t* q, float* scale)
{
    int32_t nblk = (S + block - 1) / block;
    for (int64_t mtx = 0; mtx < nmat; ++mtx) {
        for (int32_t bi = 0; bi < nblk; ++bi) {
            int32_t r0 = bi * block, r1 = r0 + block < S ? r0 + block : S;
            const float* xb = x + (mtx * S + r0) * D;
            uint8_t* qb = q + (mtx * S + r0) * D;
            int64_t n = (int64_t)(r1 - r0) * D;
            float a = 0.0f;
            for (int64_t e = 0; e < n; ++e) {
                float v = fabsf(xb[e]);
                if (v > a) a = v;
            }
            float r = a == 0.0f ? 0.0f : 448.0f / a;
            for (int64_t e = 0; e < n; ++e) {
                float t = xb[e] * r;
                if (t > 448.0f) t = 448.0f;
                if (t < -448.0f) t = -448.0f;
                qb[e] = oracle_e4m3_encode(oracle_e4m3_round((double)t));
            }
            scale[mtx * nblk + bi] = a == 0.0f ? 0.0f : a / 448.0f;
        }
    }
}

/* 8-bit V of the P.V ablation: one E4M3 scale per (batch, kv-head, channel) */
/* over all tokens, a_c = max_j |V[j,c]|, r = 448/a_c, code = E4M3(clamp(   */
/* v*r)), delta_c = a_c/448.  codes: [B,Hkv,S,D]; scale: [B,Hkv,D].          */
void oracle_quant_v_e4m3(int32_t B, int32_t Hkv, int32_t S, int32_t D,
                         const uint16_t* v_f16, uint8_t* codes, float* scale)
{
    for (int64_t bk = 0; bk < (int64_t)B * Hkv; ++bk) {
        const uint16_t* Vh = v_f16 + bk * S * D;
        for (int c = 0; c < D; ++c) {
            float a = 0.0f;
            for (int32_t j = 0; j < S; ++j) {
                float v = fabsf((float)oracle_half_to_double(Vh[(int64_t)j * D + c]));
                if (v > a) a = v;
            }
            float r = a == 0.0f ? 0.0f : 448.0f / a;
            for (int32_t j = 0; j < S; ++j) {
                float t = (float)oracle_half_to_double(Vh[(int64_t)j * D + c]) * r;
                if (t > 448.0f) t = 448.0f;
                if (t < -448.0f) t = -448.0f;
                codes[(bk * S + j) * D + c] = oracle_e4m3_encode(oracle_e4m3_round((double)t));
            }
            scale[bk * D + c] = a == 0.0f ? 0.0f : a / 448.0f;
        }
    }
}

/* O4 on E4M3 codes: the same quantised-attention model as                 */
/* oracle_quant_attention, with scores sum_c dec(q) dec(k) (exact in fp64:  */
/* every product of two E4M3 values has at most 8 significant bits).       */
int oracle_quant_attention_e4m3(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                                const uint8_t* q_f8, const float* q_scale, int32_t bq,
                                const uint8_t* k_f8, const float* k_scale, int32_t bk,
                                const uint16_t* v_f16, const int32_t* kv_map,
                                int32_t causal, double sm_scale, int32_t l_from_rounded,
                                const int32_t* rows, int32_t nrows,
                                double* out, double* lse, int32_t nthreads)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || bq <= 0 || bk <= 0) return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (!rows) nrows = S;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int32_t nbq = (S + bq - 1) / bq, nbk = (S + bk - 1) / bk;
    int64_t nkv = (int64_t)B * Hkv * S * D;
    double* V = decode_all(v_f16, nkv);
    double* Kd = (double*)malloc((size_t)nkv * sizeof(double));
    if (!V || !Kd) { free(V); free(Kd); return -5; }
    oracle_e4m3_decode_array(k_f8, Kd, nkv);
    int64_t total = (int64_t)B * Hq * nrows;
    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)S * sizeof(double));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        double* qrow = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !acc || !qrow) {
#pragma omp atomic write
            status = -5;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < total; ++t) {
                int64_t bh = t / nrows;
                int32_t r = (int32_t)(t % nrows);
                int32_t i = rows ? rows[r] : r;
                int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
                int32_t kh = kv_map[h];
                const uint8_t* qp = q_f8 + (((int64_t)b * Hq + h) * S + i) * D;
                const double* Kh = Kd + ((int64_t)b * Hkv + kh) * S * D;
                const double* Vh = V + ((int64_t)b * Hkv + kh) * S * D;
                double dq = (double)q_scale[((int64_t)b * Hq + h) * nbq + i / bq];
                const float* dk = k_scale + ((int64_t)b * Hkv + kh) * nbk;
                double* o = out + t * D;
                for (int c = 0; c < D; ++c) qrow[c] = oracle_e4m3_decode(qp[c]);
                int32_t nvis = causal ? (i + 1 < S ? i + 1 : S) : S;
                double m = -INFINITY;
                for (int32_t j = 0; j < nvis; ++j) {
                    double dot = 0.0;
                    for (int c = 0; c < D; ++c) dot += qrow[c] * Kh[(int64_t)j * D + c];
                    s[j] = dot * dq * (double)dk[j / bk] * sm_scale;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int c = 0; c < D; ++c) acc[c] = 0.0;
                for (int32_t j = 0; j < nvis; ++j) {
                    double p = exp(s[j] - m);
                    double pr = oracle_round_to_half(p);
                    l += l_from_rounded ? pr : p;
                    for (int c = 0; c < D; ++c) acc[c] += pr * Vh[(int64_t)j * D + c];
                }
                for (int c = 0; c < D; ++c) o[c] = acc[c] / l;
                if (lse) lse[t] = m + log(l);
            }
        }
        free(s); free(acc); free(qrow);
    }
    free(V); free(Kd);
    return status;
}

/* ------------------------------------------------------------------------ */
/* O5: the 8-bit P.V ablation ([SA] 技术方案 reports that 8-bit P and V     */
/* fail in some layers).  Scores as O4 (INT8 Q/K).  The weights are        */
/* quantised inside the online softmax ("FlashAttention" guide, FAQ;       */
/* [MHA-GQA] §8.2): keys arrive in tiles of `tile` keys; for each tile     */
/*   m_t = max(m_{t-1}, max_j s_j),  alpha = exp(m_{t-1} - m_t),            */
/*   p_j = exp(s_j - m_t),  l_t = alpha l_{t-1} + sum_j p_j,                */
/*   acc_t = alpha acc_{t-1} + sum_j (E4M3(448 p_j) / 448) V'_j,            */
/* where V'_j = dec(v_code[j,c]) * delta_c, and O = acc / l.  The weight of */
/* a key is therefore rounded relative to the running maximum at its tile. */
/* p_quant = 0 keeps p unrounded (then O equals exact attention on the     */
/* same scores and V').  v_codes: [B,Hkv,S,D]; v_scale: [B,Hkv,D].         */
/*                                                                          */
/* tie_slack (nullable, one value per output row): a bound on how far the  */
/* row's O may move when a weight whose 448 p lies within a relative        */
/* distance tie_rel of a half-way point between two E4M3 values is rounded */
/* to the other neighbour (as a computation of p with a relative error     */
/* below tie_rel may do): the sum over those weights of one E4M3 step of   */
/* the weight, carried to the final maximum like acc, times max_c |V'_jc|, */
/* divided by l.  It is 0 for a row with no such weight.                   */
/* ------------------------------------------------------------------------ */
/* Spacing of the E4M3 grid around x (0 <= x <= 448): 2^(e-3) in the binade */
/* [2^e, 2^(e+1)) of the normal numbers (e >= -6), 2^-9 among the          */
/* subnormals below 2^-6.  Distance from x to the nearest half-way point   */
/* between two neighbouring grid values of that binade.                    */
static double e4m3_spacing(double x)
{
    if (x < 0.015625) return 0.001953125;
    int e = 0;
    frexp(x, &e);                 /* x = f 2^e, f in [0.5, 1): binade 2^(e-1) */
    return ldexp(1.0, e - 1 - 3);
}
static double e4m3_tie_distance(double x)
{
    double sp = e4m3_spacing(x);
    double base = 0.0;
    if (x >= 0.015625) {
        int e = 0;
        frexp(x, &e);
        base = ldexp(1.0, e - 1);
    }
    double u = (x - base) / sp;   /* position in grid steps within the binade */
    return fabs((u - floor(u)) - 0.5) * sp;
}

int oracle_pv8_attention(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                         const int8_t* q_i8, const float* q_scale, int32_t bq,
                         const int8_t* k_i8, const float* k_scale, int32_t bk,
                         const uint8_t* v_codes, const float* v_scale, const int32_t* kv_map,
                         int32_t causal, double sm_scale, int32_t tile, int32_t p_quant,
                         const int32_t* rows, int32_t nrows,
                         double* out, double* lse, double tie_rel, double* tie_slack, int32_t nthreads)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || bq <= 0 || bk <= 0 || tile <= 0 || tie_rel < 0.0)
        return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (!rows) nrows = S;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int32_t nbq = (S + bq - 1) / bq, nbk = (S + bk - 1) / bk;
    int64_t total = (int64_t)B * Hq * nrows;
    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)S * sizeof(double));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !acc) {
#pragma omp atomic write
            status = -5;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < total; ++t) {
                int64_t bh = t / nrows;
                int32_t r = (int32_t)(t % nrows);
                int32_t i = rows ? rows[r] : r;
                int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
                int32_t kh = kv_map[h];
                const int8_t* qp = q_i8 + (((int64_t)b * Hq + h) * S + i) * D;
                const int8_t* Kh = k_i8 + ((int64_t)b * Hkv + kh) * S * D;
                const uint8_t* Vc = v_codes + ((int64_t)b * Hkv + kh) * S * D;
                const float* dv = v_scale + ((int64_t)b * Hkv + kh) * D;
                double dq = (double)q_scale[((int64_t)b * Hq + h) * nbq + i / bq];
                const float* dk = k_scale + ((int64_t)b * Hkv + kh) * nbk;
                double* o = out + t * D;
                int32_t nvis = causal ? (i + 1 < S ? i + 1 : S) : S;
                for (int32_t j = 0; j < nvis; ++j) {
                    int64_t dot = 0;
                    for (int c = 0; c < D; ++c) dot += (int64_t)qp[c] * (int64_t)Kh[(int64_t)j * D + c];
                    s[j] = (double)dot * dq * (double)dk[j / bk] * sm_scale;
                }
                double m = -INFINITY, l = 0.0, slack = 0.0;
                for (int c = 0; c < D; ++c) acc[c] = 0.0;
                for (int32_t j0 = 0; j0 < nvis; j0 += tile) {
                    int32_t j1 = j0 + tile < nvis ? j0 + tile : nvis;
                    double mt = m;
                    for (int32_t j = j0; j < j1; ++j)
                        if (s[j] > mt) mt = s[j];
                    double alpha = exp(m - mt);     /* exp(-inf) = 0 on the first tile */
                    l *= alpha;
                    slack *= alpha;
                    for (int c = 0; c < D; ++c) acc[c] *= alpha;
                    for (int32_t j = j0; j < j1; ++j) {
                        double p = exp(s[j] - mt);
                        l += p;
                        double pq = p_quant ? oracle_e4m3_round(p * 448.0) / 448.0 : p;
                        double vmax = 0.0;
                        for (int c = 0; c < D; ++c) {
                            double vv = oracle_e4m3_decode(Vc[(int64_t)j * D + c]) * (double)dv[c];
                            acc[c] += pq * vv;
                            if (fabs(vv) > vmax) vmax = fabs(vv);
                        }
                        double x = p * 448.0;
                        if (p_quant && e4m3_tie_distance(x) <= tie_rel * x)
                            slack += e4m3_spacing(x) / 448.0 * vmax;
                    }
                    m = mt;
                }
                for (int c = 0; c < D; ++c) o[c] = acc[c] / l;
                if (lse) lse[t] = m + log(l);
                if (tie_slack) tie_slack[t] = slack / l;
            }
        }
        free(s); free(acc);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* O1 and O4 with a query length different from the key length: the       */
/* KV-cache case ([MHA-GQA] §3.4: the keys and values of all earlier       */
/* tokens are kept, and the queries of the current token(s) attend over    */
/* them).  Sq queries, Sk >= Sq cached keys; the queries are the LAST Sq    */
/* positions of the sequence, so under the causal mask query i sees keys   */
/* j <= (Sk - Sq) + i.  q: [B,Hq,Sq,D]; k, v: [B,Hkv,Sk,D].                */
/* Written separately from the square functions above (no shared code).    */
/* ------------------------------------------------------------------------ */
int oracle_attention_kv(int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Sk, int32_t D,
                        const uint16_t* q_f16, const uint16_t* k_f16, const uint16_t* v_f16,
                        const int32_t* kv_map, int32_t causal, double sm_scale,
                        double* out, double* lse, int32_t nthreads)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk < Sq || D <= 0) return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int64_t total = (int64_t)B * Hq * Sq;
    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)Sk * sizeof(double));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !acc) {
#pragma omp atomic write
            status = -5;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < total; ++t) {
                int32_t i = (int32_t)(t % Sq);
                int64_t bh = t / Sq;
                int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
                int64_t kvbase = ((int64_t)b * Hkv + kv_map[h]) * Sk * D;
                const uint16_t* qp = q_f16 + t * D;
                int32_t last = causal ? (Sk - Sq) + i : Sk - 1;   /* last visible key */
                double m = -INFINITY;
                for (int32_t j = 0; j <= last; ++j) {
                    double dot = 0.0;
                    for (int c = 0; c < D; ++c)
                        dot += oracle_half_to_double(qp[c]) * oracle_half_to_double(k_f16[kvbase + (int64_t)j * D + c]);
                    s[j] = dot * sm_scale;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int c = 0; c < D; ++c) acc[c] = 0.0;
                for (int32_t j = 0; j <= last; ++j) {
                    double p = exp(s[j] - m);
                    l += p;
                    for (int c = 0; c < D; ++c) acc[c] += p * oracle_half_to_double(v_f16[kvbase + (int64_t)j * D + c]);
                }
                for (int c = 0; c < D; ++c) out[t * D + c] = acc[c] / l;
                if (lse) lse[t] = m + log(l);
            }
        }
        free(s); free(acc);
    }
    return status;
}

/* O4 for the KV-cache case: INT8 scores S32 * dQ[i/bq] * dK[j/bk] * sm_scale */
/* with the weights rounded to fp16 for the P.V product (l from unrounded    */
/* weights).  q_i8 [B,Hq,Sq,D], q_scale [B,Hq,ceil(Sq/bq)]; k_i8 [B,Hkv,Sk,D],*/
/* k_scale [B,Hkv,ceil(Sk/bk)] (K smoothed with its mean over the Sk cached   */
/* tokens).                                                                  */
int oracle_quant_attention_kv(int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Sk, int32_t D,
                              const int8_t* q_i8, const float* q_scale, int32_t bq,
                              const int8_t* k_i8, const float* k_scale, int32_t bk,
                              const uint16_t* v_f16, const int32_t* kv_map, int32_t causal,
                              double sm_scale, double* out, double* lse, int32_t nthreads)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk < Sq || D <= 0 || bq <= 0 || bk <= 0) return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int32_t nbq = (Sq + bq - 1) / bq, nbk = (Sk + bk - 1) / bk;
    int64_t total = (int64_t)B * Hq * Sq;
    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)Sk * sizeof(double));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !acc) {
#pragma omp atomic write
            status = -5;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < total; ++t) {
                int32_t i = (int32_t)(t % Sq);
                int64_t bh = t / Sq;
                int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
                int64_t bk_idx = (int64_t)b * Hkv + kv_map[h];
                const int8_t* qp = q_i8 + t * D;
                const int8_t* Kh = k_i8 + bk_idx * Sk * D;
                const uint16_t* Vh = v_f16 + bk_idx * Sk * D;
                double dq = (double)q_scale[bh * nbq + i / bq];
                int32_t last = causal ? (Sk - Sq) + i : Sk - 1;
                double m = -INFINITY;
                for (int32_t j = 0; j <= last; ++j) {
                    int64_t dot = 0;
                    for (int c = 0; c < D; ++c) dot += (int64_t)qp[c] * (int64_t)Kh[(int64_t)j * D + c];
                    s[j] = (double)dot * dq * (double)k_scale[bk_idx * nbk + j / bk] * sm_scale;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int c = 0; c < D; ++c) acc[c] = 0.0;
                for (int32_t j = 0; j <= last; ++j) {
                    double p = exp(s[j] - m);
                    l += p;
                    double pr = oracle_round_to_half(p);
                    for (int c = 0; c < D; ++c) acc[c] += pr * oracle_half_to_double(Vh[(int64_t)j * D + c]);
                }
                for (int c = 0; c < D; ++c) out[t * D + c] = acc[c] / l;
                if (lse) lse[t] = m + log(l);
            }
        }
        free(s); free(acc);
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* Attention under a tile-level mask (the APB page: a FlashAttention       */
/* kernel whose attention mask has a changed shape, built from an anchor   */
/* block, passing blocks and the local context).  mask[qt * nkt + kt] for */
/* query tile qt = i / tq and key tile kt = j / tk:                        */
/*   0: key j invisible to query i;  1: visible;  2: visible iff j <= i.   */
/* Exact fp64 (quant == NULL) or the O4 quantised model (quant != NULL:    */
/* INT8 scores with block scales, weights rounded to fp16 for P.V, l from  */
/* the unrounded weights).  A row with no visible key gives O = 0 and      */
/* lse = -inf.  q, k, v share the sequence length S.                       */
/* ------------------------------------------------------------------------ */
typedef struct {
    const int8_t* q_i8; const float* q_scale; int32_t bq;
    const int8_t* k_i8; const float* k_scale; int32_t bk;
} oracle_quant_in;

static int masked_impl(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                       const uint16_t* q_f16, const uint16_t* k_f16, const uint16_t* v_f16,
                       const oracle_quant_in* quant, const int32_t* kv_map,
                       const uint8_t* mask, int32_t tq, int32_t tk, double sm_scale,
                       double* out, double* lse, int32_t nthreads)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || tq <= 0 || tk <= 0) return -1;
    if (check_map(Hq, Hkv, kv_map)) return -4;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int32_t nkt = (S + tk - 1) / tk;
    int64_t total = (int64_t)B * Hq * S;
    int status = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)S * sizeof(double));
        int32_t* vis = (int32_t*)malloc((size_t)S * sizeof(int32_t));
        double* acc = (double*)malloc((size_t)D * sizeof(double));
        if (!s || !vis || !acc) {
#pragma omp atomic write
            status = -5;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < total; ++t) {
                int32_t i = (int32_t)(t % S);
                int64_t bh = t / S;
                int32_t b = (int32_t)(bh / Hq), h = (int32_t)(bh % Hq);
                int64_t kvb = ((int64_t)b * Hkv + kv_map[h]) * S * D;
                int32_t nv = 0;
                for (int32_t j = 0; j < S; ++j) {
                    uint8_t m = mask[(int64_t)(i / tq) * nkt + j / tk];
                    if (m == 1 || (m == 2 && j <= i)) vis[nv++] = j;
                }
                double* o = out + t * D;
                if (nv == 0) {
                    for (int c = 0; c < D; ++c) o[c] = 0.0;
                    if (lse) lse[t] = -INFINITY;
                    continue;
                }
                double mx = -INFINITY;
                for (int32_t a = 0; a < nv; ++a) {
                    int32_t j = vis[a];
                    if (quant) {
                        const int8_t* qp = quant->q_i8 + t * D;
                        const int8_t* kp = quant->k_i8 + kvb + (int64_t)j * D;
                        int64_t dot = 0;
                        for (int c = 0; c < D; ++c) dot += (int64_t)qp[c] * (int64_t)kp[c];
                        int32_t nbq = (S + quant->bq - 1) / quant->bq, nbk = (S + quant->bk - 1) / quant->bk;
                        s[a] = (double)dot * (double)quant->q_scale[bh * nbq + i / quant->bq] *
                               (double)quant->k_scale[((int64_t)b * Hkv + kv_map[h]) * nbk + j / quant->bk] * sm_scale;
                    } else {
                        double dot = 0.0;
                        for (int c = 0; c < D; ++c)
                            dot += oracle_half_to_double(q_f16[t * D + c]) *
                                   oracle_half_to_double(k_f16[kvb + (int64_t)j * D + c]);
                        s[a] = dot * sm_scale;
                    }
                    if (s[a] > mx) mx = s[a];
                }
                double l = 0.0;
                for (int c = 0; c < D; ++c) acc[c] = 0.0;
                for (int32_t a = 0; a < nv; ++a) {
                    double p = exp(s[a] - mx);
                    l += p;
                    double pw = quant ? oracle_round_to_half(p) : p;
                    for (int c = 0; c < D; ++c)
                        acc[c] += pw * oracle_half_to_double(v_f16[kvb + (int64_t)vis[a] * D + c]);
                }
                for (int c = 0; c < D; ++c) o[c] = acc[c] / l;
                if (lse) lse[t] = mx + log(l);
            }
        }
        free(s); free(vis); free(acc);
    }
    return status;
}

int oracle_attention_masked(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                            const uint16_t* q_f16, const uint16_t* k_f16, const uint16_t* v_f16,
                            const int32_t* kv_map, const uint8_t* mask, int32_t tq, int32_t tk,
                            double sm_scale, double* out, double* lse, int32_t nthreads)
{
    return masked_impl(B, Hq, Hkv, S, D, q_f16, k_f16, v_f16, NULL, kv_map, mask, tq, tk, sm_scale,
                       out, lse, nthreads);
}

int oracle_quant_attention_masked(int32_t B, int32_t Hq, int32_t Hkv, int32_t S, int32_t D,
                                  const int8_t* q_i8, const float* q_scale, int32_t bq,
                                  const int8_t* k_i8, const float* k_scale, int32_t bk,
                                  const uint16_t* v_f16, const int32_t* kv_map, const uint8_t* mask,
                                  int32_t tq, int32_t tk, double sm_scale, double* out, double* lse,
                                  int32_t nthreads)
{
    oracle_quant_in qi = {q_i8, q_scale, bq, k_i8, k_scale, bk};
    if (bq <= 0 || bk <= 0) return -1;
    return masked_impl(B, Hq, Hkv, S, D, NULL, NULL, v_f16, &qi, kv_map, mask, tq, tk, sm_scale,
                       out, lse, nthreads);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
