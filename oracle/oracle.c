/*
 * Plain fp64 CPU oracle for softmax attention — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * this library.  It shares no code, header, table or helper with the GPU
 * path: every routine here is written from the definition of the operation,
 * in double precision, as plainly as possible.  Nothing here is blocked,
 * fused or reordered beyond what the definition states.
 *
 * Sources (the web pages this build follows):
 *  - "flashattention-kernels" page (cyk1337 paper-daily), §0 lineage and §1
 *    four-layer breakdown: exact softmax attention is the semantics every
 *    FlashAttention-style kernel keeps; tiling + online softmax only change
 *    how it is evaluated.  §3 (inference side): Flash-Decoding splits the KV
 *    sequence into chunks, computes partial attention per chunk, then reduces.
 *  - "cuda-kernel-pretrain" page (cyk1337 paper-daily), §2 (attention): the
 *    IO-aware kernel keeps exactness; numerics must be regression-checked
 *    against an unfused reference.  §3: GQA/MQA share one K/V head per group.
 *  - "GPU kernel overview" page (zhaifeiyue.github.io/overview/kernel.html),
 *    SageAttention chain and the "INT for QK, FP for PV" insight: Smooth-K,
 *    per-block INT8 Q/K for QK^T, FP8 (E4M3) for P and V.
 *
 * Conventions (readings of what the pages leave open):
 *  - inputs are bf16 bit patterns (uint16), decoded exactly to double;
 *  - causal masking is top-left aligned: key j is visible to query i iff j <= i;
 *  - kv head of query head h is h / (H / Hkv) (consecutive groups);
 *  - lse is the natural-log log-sum-exp of the scaled, masked scores;
 *  - a row with no visible key gets O = 0 and lse = -inf.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, S.1111.111 is NaN, largest finite magnitude 448.
 * Decoding is the closed form of the format definition.
 */
double oracle_e4m3_decode(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 7;
    double mag;
    if (e == 0xF && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6); /* subnormal */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/*
 * Encode to E4M3 with round-to-nearest, ties to the even code, saturating at
 * +-448 (infinities also saturate; NaN maps to the NaN code).  The positive
 * finite codes 0x00..0x7E are strictly increasing in value, so the nearest
 * code is found by a binary search over that ordered table followed by a
 * comparison with the neighbour above.
 */
uint8_t oracle_e4m3_encode(double x)
{
    uint8_t sign = 0;
    double a = x;
    if (isnan(x))
        return 0x7F;
    if (a < 0) {
        sign = 0x80;
        a = -a;
    }
    if (a >= 448.0)
        return sign | 0x7E;
    /* largest code c in [0, 0x7E] with value(c) <= a */
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    if (c < 0x7E) {
        double below = oracle_e4m3_decode((uint8_t)c);
        double above = oracle_e4m3_decode((uint8_t)(c + 1));
        double db = a - below, da = above - a;
        if (da < db || (da == db && ((c + 1) & 1) == 0))
            c = c + 1;
    }
    return sign | (uint8_t)c;
}

double oracle_e4m3_round(double x) { return oracle_e4m3_decode(oracle_e4m3_encode(x)); }

/* Symmetric INT8 quantisation: round half to even, clamp to [-127, 127]. */
static int quant_i8(double x, double delta)
{
    double r = nearbyint(x / delta); /* default FP environment: ties to even */
    if (r > 127.0)
        r = 127.0;
    if (r < -127.0)
        r = -127.0;
    return (int)r;
}

int oracle_quant_i8(double x, double delta) { return quant_i8(x, delta); }

/* ------------------------------------------------------------------------ */
/* Exact attention, one query row at a time                                  */
/* ------------------------------------------------------------------------ */

/*
 * Row (b, h, i) of softmax(Q K^T * scale + mask) V over the keys j in
 * [k_lo, k_hi) that the mask leaves visible.  The score row and the
 * probability row are materialised explicitly.
 *
 * Layouts: q [B,H,Nq,d]; k, v [B,Hkv,Nk,d]; all bf16 bits, contiguous.
 * kv_len (may be NULL): per-batch number of valid keys (decode caches);
 * keys at or beyond kv_len[b] are never read.
 * Returns |1 - sum_j P_ij| (0 for an empty row).
 */
static double attn_row(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                       const int32_t *kv_len, int64_t k_lo, int64_t k_hi,
                       double scale, int64_t row, double *o_row, double *lse_out,
                       double *S, double *P)
{
    int64_t i = row % Nq;
    int64_t bh = row / Nq;
    int64_t h = bh % H;
    int64_t b = bh / H;
    int64_t g = h / (H / Hkv);
    const uint16_t *qi = q + ((b * H + h) * (int64_t)Nq + i) * d;
    const uint16_t *kb = k + (b * Hkv + g) * (int64_t)Nk * d;
    const uint16_t *vb = v + (b * Hkv + g) * (int64_t)Nk * d;
    (void)B;

    int64_t hi = k_hi;
    if (hi > Nk)
        hi = Nk;
    if (kv_len && hi > kv_len[b])
        hi = kv_len[b];
    if (causal && hi > i + 1)
        hi = i + 1;
    int64_t lo = k_lo < 0 ? 0 : k_lo;

    for (int c = 0; c < d; ++c)
        o_row[c] = 0.0;
    if (hi <= lo) {
        *lse_out = -INFINITY;
        return 0.0;
    }
    int64_t n = hi - lo;

    /* scores */
    for (int64_t j = 0; j < n; ++j) {
        const uint16_t *kj = kb + (lo + j) * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += bf16_to_f64(qi[c]) * bf16_to_f64(kj[c]);
        S[j] = dot * scale;
    }
    /* explicit softmax */
    double m = S[0];
    for (int64_t j = 1; j < n; ++j)
        if (S[j] > m)
            m = S[j];
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        P[j] = exp(S[j] - m);
        sum += P[j];
    }
    double psum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        P[j] /= sum;
        psum += P[j];
    }
    /* O = P V */
    for (int64_t j = 0; j < n; ++j) {
        const uint16_t *vj = vb + (lo + j) * d;
        for (int c = 0; c < d; ++c)
            o_row[c] += P[j] * bf16_to_f64(vj[c]);
    }
    *lse_out = m + log(sum);
    return fabs(1.0 - psum);
}

/*
 * Exact attention for the listed rows (flattened (b*H + h)*Nq + i), or for
 * every row when rows == NULL.  Outputs o [nrows, d] and lse [nrows] in fp64.
 * Keys are restricted to [k_lo, k_hi) (pass 0 and Nk for the whole sequence).
 * Returns the largest |1 - sum_j P_ij| seen (a self-check of the softmax),
 * or -1 on invalid arguments.
 */
double oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                        const int32_t *kv_len, int64_t k_lo, int64_t k_hi,
                        double scale, const int64_t *rows, int64_t nrows,
                        double *o, double *lse, int nthreads)
{
    if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || Nq <= 0 || Nk <= 0 || d <= 0)
        return -1.0;
    if (!rows)
        nrows = (int64_t)B * H * Nq;
    double worst = 0.0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(max : worst)
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)Nk);
        double *P = (double *)malloc(sizeof(double) * (size_t)Nk);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = rows ? rows[r] : r;
            double e = attn_row(q, k, v, B, H, Hkv, Nq, Nk, d, causal, kv_len, k_lo, k_hi,
                                scale, row, o + r * d, lse + r, S, P);
            if (e > worst)
                worst = e;
        }
        free(S);
        free(P);
    }
    return worst;
}

/*
 * Gradients of O = softmax(Q K^T * scale + mask) V with respect to Q, K and V
 * for an upstream gradient dO (the backward pass of the attention forward;
 * "GPU kernel overview" page, SageBwd / training gaps; "flashattention-
 * kernels" page §0, FA2/FA3 as training kernels).  The pages print no
 * formula; these are the chain rule through the definition, row by row:
 *     P_i   = softmax over the visible keys of S_i,  S_ij = scale * Q_i . K_j
 *     dP_ij = dO_i . V_j
 *     D_i   = sum_j P_ij dP_ij
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale * sum_j dS_ij K_j
 *     dK_j += scale * dS_ij Q_i,   dV_j += P_ij dO_i
 * A kv head's dK and dV sum over the query heads of its group.
 * q, dout [B,H,N,d]; k, v [B,Hkv,N,d] (bf16 bits).  dq [B,H,N,d] and
 * dk, dv [B,Hkv,N,d] are written in fp64.  Returns 0, or -1 on invalid
 * arguments.
 */
int oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const uint16_t *dout, int B, int H, int Hkv, int N, int d, int causal,
                    double scale, double *dq, double *dk, double *dv, int nthreads)
{
    if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || N <= 0 || d <= 0)
        return -1;
    const int G = H / Hkv;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    memset(dk, 0, sizeof(double) * (size_t)B * Hkv * N * d);
    memset(dv, 0, sizeof(double) * (size_t)B * Hkv * N * d);
    /* one (batch, kv head) per iteration: its dK and dV have one writer */
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)N);
        double *P = (double *)malloc(sizeof(double) * (size_t)N);
        double *dP = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t bg = 0; bg < (int64_t)B * Hkv; ++bg) {
            const int64_t b = bg / Hkv, g = bg % Hkv;
            const uint16_t *kb = k + bg * (int64_t)N * d;
            const uint16_t *vb = v + bg * (int64_t)N * d;
            double *dkb = dk + bg * (int64_t)N * d;
            double *dvb = dv + bg * (int64_t)N * d;
            for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                const int64_t bh = b * H + h;
                for (int64_t i = 0; i < N; ++i) {
                    const uint16_t *qi = q + (bh * N + i) * d;
                    const uint16_t *doi = dout + (bh * N + i) * d;
                    double *dqi = dq + (bh * N + i) * d;
                    const int64_t n = causal ? i + 1 : N;
                    for (int64_t j = 0; j < n; ++j) {
                        double dot = 0.0, dd = 0.0;
                        for (int c = 0; c < d; ++c) {
                            dot += bf16_to_f64(qi[c]) * bf16_to_f64(kb[j * d + c]);
                            dd += bf16_to_f64(doi[c]) * bf16_to_f64(vb[j * d + c]);
                        }
                        S[j] = dot * scale;
                        dP[j] = dd;
                    }
                    double m = S[0];
                    for (int64_t j = 1; j < n; ++j)
                        if (S[j] > m)
                            m = S[j];
                    double sum = 0.0;
                    for (int64_t j = 0; j < n; ++j) {
                        P[j] = exp(S[j] - m);
                        sum += P[j];
                    }
                    double D = 0.0;
                    for (int64_t j = 0; j < n; ++j) {
                        P[j] /= sum;
                        D += P[j] * dP[j];
                    }
                    for (int c = 0; c < d; ++c)
                        dqi[c] = 0.0;
                    for (int64_t j = 0; j < n; ++j) {
                        const double ds = P[j] * (dP[j] - D);
                        for (int c = 0; c < d; ++c) {
                            dqi[c] += scale * ds * bf16_to_f64(kb[j * d + c]);
                            dkb[j * d + c] += scale * ds * bf16_to_f64(qi[c]);
                            dvb[j * d + c] += P[j] * bf16_to_f64(doi[c]);
                        }
                    }
                }
            }
        }
        free(S);
        free(P);
        free(dP);
    }
    return 0;
}

/*
 * Merge of partial results over disjoint key sets (the reduction step of
 * split-KV decoding): with M = max_s lse_s and w_s = exp(lse_s - M),
 * O = sum_s w_s O_s / sum_s w_s and lse = M + ln sum_s w_s.
 * o_parts [nparts, nrows, d], lse_parts [nparts, nrows]; parts whose lse is
 * -inf (no visible key) carry no weight.
 */
void oracle_lse_merge(const double *o_parts, const double *lse_parts, int nparts,
                      int64_t nrows, int d, double *o, double *lse)
{
    for (int64_t r = 0; r < nrows; ++r) {
        double M = -INFINITY;
        for (int s = 0; s < nparts; ++s)
            if (lse_parts[s * nrows + r] > M)
                M = lse_parts[s * nrows + r];
        for (int c = 0; c < d; ++c)
            o[r * d + c] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int s = 0; s < nparts; ++s) {
            double w = exp(lse_parts[s * nrows + r] - M);
            wsum += w;
            for (int c = 0; c < d; ++c)
                o[r * d + c] += w * o_parts[((int64_t)s * nrows + r) * d + c];
        }
        for (int c = 0; c < d; ++c)
            o[r * d + c] /= wsum;
        lse[r] = M + log(wsum);
    }
}

/* ------------------------------------------------------------------------ */
/* SageAttention-style quantised attention, emulated step by step            */
/* ------------------------------------------------------------------------ */

/*
 * Quantisation state computed once per call from the bf16 inputs:
 *  kmean[b,g,c]     Smooth-K channel mean of K over all Nk tokens
 *  qhat, qdelta     per (b, h, 64-token block) INT8 codes of Q and their scale
 *  khat, kdelta     the same for K - kmean
 *  vhat, vdelta     per (b, g, channel) E4M3 values of V / vdelta (decoded)
 */
typedef struct {
    double *kmean;
    int8_t *qhat, *khat;
    double *qdelta, *kdelta;
    double *vq;     /* decoded E4M3 value of V / vdelta */
    double *vdelta;
} sage_state;

static void sage_prepare(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         int B, int H, int Hkv, int N, int d, int blk, int smooth_k,
                         sage_state *st)
{
    /*
     * The quantisation decisions (INT8 codes, E4M3 codes) are taken in fp32,
     * the precision the GPU kernel takes them in: the pages fix no precision
     * for them, and taking an integer decision in a different precision than
     * the kernel would flip codes at rounding ties.  Each step is otherwise
     * the plain formula: K' = K - kmean; delta = max|x| / 127; code =
     * rint(x * (127 / max|x|)); V code = E4M3(V * (448 / max|V|)).  The mean
     * itself is taken in fp64 and rounded to fp32.
     */
    int64_t nqb = (N + blk - 1) / blk;
    st->kmean = (double *)calloc((size_t)B * Hkv * d, sizeof(double));
    st->qhat = (int8_t *)malloc((size_t)B * H * N * d);
    st->khat = (int8_t *)malloc((size_t)B * Hkv * N * d);
    st->qdelta = (double *)malloc(sizeof(double) * (size_t)B * H * nqb);
    st->kdelta = (double *)malloc(sizeof(double) * (size_t)B * Hkv * nqb);
    st->vq = (double *)malloc(sizeof(double) * (size_t)B * Hkv * N * d);
    st->vdelta = (double *)malloc(sizeof(double) * (size_t)B * Hkv * d);

#pragma omp parallel for
    for (int64_t bg = 0; bg < (int64_t)B * Hkv; ++bg) {
        const uint16_t *kb = k + bg * (int64_t)N * d;
        if (smooth_k) {
            for (int c = 0; c < d; ++c) {
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    s += bf16_to_f64(kb[n * d + c]);
                st->kmean[bg * d + c] = (double)(float)(s / N);
            }
        }
        /* INT8 per 64-token block of K - kmean */
        for (int64_t t = 0; t < nqb; ++t) {
            int64_t n0 = t * blk, n1 = n0 + blk < N ? n0 + blk : N;
            float amax = 0.0f;
            for (int64_t n = n0; n < n1; ++n)
                for (int c = 0; c < d; ++c) {
                    float x = (float)bf16_to_f64(kb[n * d + c]) - (float)st->kmean[bg * d + c];
                    if (fabsf(x) > amax)
                        amax = fabsf(x);
                }
            float inv = amax > 0.0f ? 127.0f / amax : 1.0f;
            st->kdelta[bg * nqb + t] = amax > 0.0f ? (double)(amax / 127.0f) : 1.0;
            for (int64_t n = n0; n < n1; ++n)
                for (int c = 0; c < d; ++c) {
                    float x = (float)bf16_to_f64(kb[n * d + c]) - (float)st->kmean[bg * d + c];
                    st->khat[(bg * N + n) * d + c] = (int8_t)quant_i8((double)(x * inv), 1.0);
                }
        }
        /* V: per-channel scale over all tokens, E4M3 values */
        const uint16_t *vb = v + bg * (int64_t)N * d;
        for (int c = 0; c < d; ++c) {
            float amax = 0.0f;
            for (int64_t n = 0; n < N; ++n)
                if (fabsf((float)bf16_to_f64(vb[n * d + c])) > amax)
                    amax = fabsf((float)bf16_to_f64(vb[n * d + c]));
            float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
            st->vdelta[bg * d + c] = amax > 0.0f ? (double)(amax / 448.0f) : 1.0;
            for (int64_t n = 0; n < N; ++n)
                st->vq[(bg * N + n) * d + c] =
                    oracle_e4m3_round((double)((float)bf16_to_f64(vb[n * d + c]) * inv));
        }
    }
    /* INT8 per 64-token block of Q */
#pragma omp parallel for
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const uint16_t *qb = q + bh * (int64_t)N * d;
        for (int64_t t = 0; t < nqb; ++t) {
            int64_t n0 = t * blk, n1 = n0 + blk < N ? n0 + blk : N;
            float amax = 0.0f;
            for (int64_t n = n0; n < n1; ++n)
                for (int c = 0; c < d; ++c)
                    if (fabsf((float)bf16_to_f64(qb[n * d + c])) > amax)
                        amax = fabsf((float)bf16_to_f64(qb[n * d + c]));
            float inv = amax > 0.0f ? 127.0f / amax : 1.0f;
            st->qdelta[bh * nqb + t] = amax > 0.0f ? (double)(amax / 127.0f) : 1.0;
            for (int64_t n = n0; n < n1; ++n)
                for (int c = 0; c < d; ++c)
                    st->qhat[(bh * N + n) * d + c] =
                        (int8_t)quant_i8((double)((float)bf16_to_f64(qb[n * d + c]) * inv), 1.0);
        }
    }
}

static void sage_free(sage_state *st)
{
    free(st->kmean);
    free(st->qhat);
    free(st->khat);
    free(st->qdelta);
    free(st->kdelta);
    free(st->vq);
    free(st->vdelta);
}

/*
 * Quantised attention for the listed rows, following the recipe's steps in
 * order:
 *   1. Smooth-K: K' = K - mean_n K (per channel, all tokens of the kv head);
 *   2. INT8 Q and K' per 64-token block, delta = max|x| / 127;
 *   3. V per channel: delta_V = max_n |V| / 448, V^ = E4M3(V / delta_V);
 *   4. S_ij = scale * dQ(i) * dK(j) * (q^_i . k^_j)   (exact integer dot);
 *   5. keys in tiles of `tile_n` from key 0 upward, with a running max m:
 *        m' = max(m, max of the tile's visible scores),
 *        p_j = exp(S_ij - m'),  l = l * exp(m - m') + sum_j p_j,
 *        P^_j = E4M3(448 * p_j),
 *        acc = acc * exp(m - m') + sum_j P^_j V^_j;
 *   6. O = acc * delta_V / (448 * l);
 *      lse = m + ln l + scale * (q_i . kmean)  (the true LSE: Smooth-K shifts
 *      every score of row i by the constant -scale * q_i . kmean).
 * The static factor 448 puts P in E4M3's full range (P lies in [0, 1]); its
 * inverse is folded into the final division.  The result depends on tile_n
 * because P is quantised against the running max.
 * p_scale: factor applied to p before the E4M3 cast (448 for the recipe);
 * quant_p = 0 skips P quantisation, quant_v = 0 skips V quantisation (used for
 * error attributions); quant_qk = 0 uses the unquantised (smoothed) Q and K;
 * l_quant = 1 makes l the sum of the quantised P^_j / 448 instead of the
 * unrounded p_j (an alternative reading, for the same attributions).
 */
double oracle_sage_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int B, int H, int Hkv, int N, int d, int causal, double scale,
                        int blk, int tile_n, int smooth_k, int quant_qk, int quant_p,
                        int quant_v, double p_scale, int l_quant,
                        const int64_t *rows, int64_t nrows, double *o, double *lse,
                        int nthreads)
{
    if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || N <= 0 || d <= 0 || blk <= 0 || tile_n <= 0)
        return -1.0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    if (!rows)
        nrows = (int64_t)B * H * N;
    sage_state st;
    sage_prepare(q, k, v, B, H, Hkv, N, d, blk, smooth_k, &st);
    int64_t nqb = (N + blk - 1) / blk;

#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)tile_n);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = rows ? rows[r] : r;
            int64_t i = row % N, bh = row / N, h = bh % H, b = bh / H;
            int64_t g = h / (H / Hkv), bg = b * Hkv + g;
            const int8_t *qh = st.qhat + (bh * N + i) * d;
            const uint16_t *qraw = q + (bh * N + i) * d;
            double dq = st.qdelta[bh * nqb + i / blk];
            int64_t nvis = causal ? i + 1 : N;
            double m = -INFINITY, l = 0.0;
            for (int c = 0; c < d; ++c)
                acc[c] = 0.0;
            for (int64_t j0 = 0; j0 < nvis; j0 += tile_n) {
                int64_t j1 = j0 + tile_n < nvis ? j0 + tile_n : nvis;
                double tmax = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    double sc;
                    if (quant_qk) {
                        const int8_t *kh = st.khat + (bg * N + j) * d;
                        int64_t dot = 0;
                        for (int c = 0; c < d; ++c)
                            dot += (int64_t)qh[c] * kh[c];
                        sc = scale * dq * st.kdelta[bg * nqb + j / blk] * (double)dot;
                    } else {
                        const uint16_t *kr = k + (bg * N + j) * d;
                        double dot = 0.0;
                        for (int c = 0; c < d; ++c)
                            dot += bf16_to_f64(qraw[c]) * (bf16_to_f64(kr[c]) - st.kmean[bg * d + c]);
                        sc = scale * dot;
                    }
                    S[j - j0] = sc;
                    if (sc > tmax)
                        tmax = sc;
                }
                double mnew = tmax > m ? tmax : m;
                double alpha = exp(m - mnew); /* exp(-inf) = 0 on the first tile */
                l *= alpha;
                for (int c = 0; c < d; ++c)
                    acc[c] *= alpha;
                for (int64_t j = j0; j < j1; ++j) {
                    double p = exp(S[j - j0] - mnew);
                    double ph = quant_p ? oracle_e4m3_round(p_scale * p) : p_scale * p;
                    /* l sums the unrounded p (the recipe); l_quant instead sums
                     * the quantised values ph / p_scale, an alternative reading
                     * kept for comparison */
                    l += l_quant ? ph / p_scale : p;
                    const double *vj = st.vq + (bg * N + j) * d;
                    const uint16_t *vr = v + (bg * N + j) * d;
                    for (int c = 0; c < d; ++c) {
                        double vv = quant_v ? vj[c] : bf16_to_f64(vr[c]) / st.vdelta[bg * d + c];
                        acc[c] += ph * vv;
                    }
                }
                m = mnew;
            }
            double qk = 0.0;
            for (int c = 0; c < d; ++c)
                qk += bf16_to_f64(qraw[c]) * st.kmean[bg * d + c];
            for (int c = 0; c < d; ++c)
                o[r * d + c] = acc[c] * st.vdelta[bg * d + c] / (p_scale * l);
            lse[r] = m + log(l) + scale * qk;
        }
        free(S);
        free(acc);
    }
    sage_free(&st);
    return 0.0;
}

/*
 * Expose the quantisation state for tests of the individual steps:
 * kmean [B,Hkv,d], qhat [B,H,N,d], qdelta [B,H,nblk], khat [B,Hkv,N,d],
 * kdelta [B,Hkv,nblk], vq [B,Hkv,N,d] (decoded E4M3 of V/delta_V),
 * vdelta [B,Hkv,d].  Any output pointer may be NULL.
 */
int oracle_sage_quantise(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         int B, int H, int Hkv, int N, int d, int blk, int smooth_k,
                         double *kmean, int8_t *qhat, double *qdelta, int8_t *khat,
                         double *kdelta, double *vq, double *vdelta)
{
    if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || N <= 0 || d <= 0 || blk <= 0)
        return -1;
    sage_state st;
    sage_prepare(q, k, v, B, H, Hkv, N, d, blk, smooth_k, &st);
    int64_t nqb = (N + blk - 1) / blk;
    if (kmean)
        memcpy(kmean, st.kmean, sizeof(double) * (size_t)B * Hkv * d);
    if (qhat)
        memcpy(qhat, st.qhat, (size_t)B * H * N * d);
    if (qdelta)
        memcpy(qdelta, st.qdelta, sizeof(double) * (size_t)B * H * nqb);
    if (khat)
        memcpy(khat, st.khat, (size_t)B * Hkv * N * d);
    if (kdelta)
        memcpy(kdelta, st.kdelta, sizeof(double) * (size_t)B * Hkv * nqb);
    if (vq)
        memcpy(vq, st.vq, sizeof(double) * (size_t)B * Hkv * N * d);
    if (vdelta)
        memcpy(vdelta, st.vdelta, sizeof(double) * (size_t)B * Hkv * d);
    sage_free(&st);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 quantised attention (SageAttention3-style, MX block formats)        */
/* ------------------------------------------------------------------------ */

/*
 * OCP MX FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no
 * infinities or NaN.  Exponent field 0 is subnormal (0 or 0.5); otherwise
 * 2^(E-1) * (1 + M/2).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
double oracle_e2m1_decode(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* Nearest E2M1 code, ties to the even code, saturating at +-6 (the positive
 * codes 0..7 are increasing in value). */
uint8_t oracle_e2m1_encode(double x)
{
    uint8_t sign = x < 0 ? 8 : 0;
    double a = fabs(x);
    if (a >= 6.0)
        return sign | 7;
    int c = 0;
    while (c < 7 && oracle_e2m1_decode((uint8_t)(c + 1)) <= a)
        ++c;
    if (c < 7) {
        double db = a - oracle_e2m1_decode((uint8_t)c);
        double da = oracle_e2m1_decode((uint8_t)(c + 1)) - a;
        if (da < db || (da == db && ((c + 1) & 1) == 0))
            c = c + 1;
    }
    return sign | (uint8_t)c;
}

/*
 * Exponent e of the shared E8M0 scale 2^e of one MX block: the smallest
 * power of two with amax <= 6 * 2^e, so that the block's largest element
 * lands on E2M1's largest magnitude or below it and nothing saturates (the
 * block's maximum maps into [0, 6 * 2^e], as SageAttention3 maps each block
 * onto the FP4 range).  Clamped to E8M0's range [-127, 127]; an all-zero
 * block gets e = 0.
 */
int oracle_mx_scale_exp(double amax)
{
    if (!(amax > 0.0))
        return 0;
    int e = -127;
    while (e < 127 && amax > ldexp(6.0, e))
        ++e;
    return e;
}

/*
 * OCP MX FP6 E2M3: 1 sign bit, 2 exponent bits (bias 1), 3 mantissa bits, no
 * infinities or NaN.  Exponent field 0 is subnormal (M/8); otherwise
 * 2^(E-1) * (1 + M/8).  The positive magnitudes are the multiples of 1/8 in
 * [0, 2), of 1/4 in [2, 4) and of 1/2 in [4, 7.5].
 */
double oracle_e2m3_decode(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 3) & 3, m = code & 7;
    double mag = e == 0 ? m / 8.0 : ldexp(1.0 + m / 8.0, e - 1);
    return s ? -mag : mag;
}

/* Nearest E2M3 code, ties to the even code, saturating at +-7.5 (the
 * positive codes 0..31 are increasing in value). */
uint8_t oracle_e2m3_encode(double x)
{
    uint8_t sign = x < 0 ? 32 : 0;
    double a = fabs(x);
    if (a >= 7.5)
        return sign | 31;
    int c = 0;
    while (c < 31 && oracle_e2m3_decode((uint8_t)(c + 1)) <= a)
        ++c;
    if (c < 31) {
        double db = a - oracle_e2m3_decode((uint8_t)c);
        double da = oracle_e2m3_decode((uint8_t)(c + 1)) - a;
        if (da < db || (da == db && ((c + 1) & 1) == 0))
            c = c + 1;
    }
    return sign | (uint8_t)c;
}

/* The element formats of the MX blocks: E2M1 (FP4) and E2M3 (FP6). */
enum { MX_E2M1 = 0, MX_E2M3 = 1 };

static double mx_elem_max(int elem) { return elem == MX_E2M3 ? 7.5 : 6.0; }

static double mx_elem_round(int elem, double y)
{
    return elem == MX_E2M3 ? oracle_e2m3_decode(oracle_e2m3_encode(y))
                           : oracle_e2m1_decode(oracle_e2m1_encode(y));
}

/*
 * Exponent e of the shared scale 2^e of an MX block whose elements have the
 * largest magnitude `emax`: the smallest e with amax <= emax * 2^e, clamped
 * to E8M0's range [-127, 127]; an all-zero block gets e = 0.
 */
int oracle_mx_scale_exp_max(double amax, double emax)
{
    if (!(amax > 0.0))
        return 0;
    int e = -127;
    while (e < 127 && amax > ldexp(emax, e))
        ++e;
    return e;
}

typedef struct {
    double *kmean; /* [B*Hkv][d] (fp32 values) */
    double *qd;    /* [B*H][N][d]   dequantised MX Q */
    double *kd;    /* [B*Hkv][N][d] dequantised MX K - kmean */
    double *vd;    /* [B*Hkv][N][d] dequantised MX V */
    int elem;      /* MX_E2M1 or MX_E2M3 */
} mx_state;

/* Dequantised value of x in an MX block of the state's element format with
 * shared exponent e. */
static double mx_round(const mx_state *st, double x, int e)
{
    return ldexp(mx_elem_round(st->elem, ldexp(x, -e)), e);
}

/* The block exponent in the state's element format. */
static int mx_block_exp(const mx_state *st, double amax)
{
    return oracle_mx_scale_exp_max(amax, mx_elem_max(st->elem));
}

static void mx_prepare(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H,
                       int Hkv, int N, int d, int smooth_k, int quant_qk, int quant_v,
                       mx_state *st)
{
    /*
     * Q and K - kmean: blocks of 32 consecutive channels of one token (the
     * contraction dimension of Q K^T); V: blocks of 32 consecutive tokens of
     * one channel (the contraction dimension of P V).  K - kmean is formed
     * in fp32 (as the kernel does); every other value is exact.
     */
    st->kmean = (double *)calloc((size_t)B * Hkv * d, sizeof(double));
    st->qd = (double *)malloc(sizeof(double) * (size_t)B * H * N * d);
    st->kd = (double *)malloc(sizeof(double) * (size_t)B * Hkv * N * d);
    st->vd = (double *)malloc(sizeof(double) * (size_t)B * Hkv * N * d);
#pragma omp parallel for
    for (int64_t bg = 0; bg < (int64_t)B * Hkv; ++bg) {
        const uint16_t *kb = k + bg * (int64_t)N * d, *vb = v + bg * (int64_t)N * d;
        if (smooth_k) {
            for (int c = 0; c < d; ++c) {
                double s = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    s += bf16_to_f64(kb[n * d + c]);
                st->kmean[bg * d + c] = (double)(float)(s / N);
            }
        }
        for (int64_t n = 0; n < N; ++n)
            for (int c0 = 0; c0 < d; c0 += 32) {
                double x[32], amax = 0.0;
                for (int c = 0; c < 32; ++c) {
                    x[c] = (double)((float)bf16_to_f64(kb[n * d + c0 + c]) -
                                    (float)st->kmean[bg * d + c0 + c]);
                    if (fabs(x[c]) > amax)
                        amax = fabs(x[c]);
                }
                int e = mx_block_exp(st, amax);
                /* without quantisation K - kmean is taken exactly */
                for (int c = 0; c < 32; ++c)
                    st->kd[(bg * N + n) * d + c0 + c] =
                        quant_qk ? mx_round(st, x[c], e)
                                 : bf16_to_f64(kb[n * d + c0 + c]) - st->kmean[bg * d + c0 + c];
            }
        for (int c = 0; c < d; ++c)
            for (int64_t n0 = 0; n0 < N; n0 += 32) {
                int64_t n1 = n0 + 32 < N ? n0 + 32 : N;
                double amax = 0.0;
                for (int64_t n = n0; n < n1; ++n)
                    if (fabs(bf16_to_f64(vb[n * d + c])) > amax)
                        amax = fabs(bf16_to_f64(vb[n * d + c]));
                int e = mx_block_exp(st, amax);
                for (int64_t n = n0; n < n1; ++n) {
                    double x = bf16_to_f64(vb[n * d + c]);
                    st->vd[(bg * N + n) * d + c] = quant_v ? mx_round(st, x, e) : x;
                }
            }
    }
#pragma omp parallel for
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const uint16_t *qb = q + bh * (int64_t)N * d;
        for (int64_t n = 0; n < N; ++n)
            for (int c0 = 0; c0 < d; c0 += 32) {
                double amax = 0.0;
                for (int c = 0; c < 32; ++c)
                    if (fabs(bf16_to_f64(qb[n * d + c0 + c])) > amax)
                        amax = fabs(bf16_to_f64(qb[n * d + c0 + c]));
                int e = mx_block_exp(st, amax);
                for (int c = 0; c < 32; ++c) {
                    double x = bf16_to_f64(qb[n * d + c0 + c]);
                    st->qd[(bh * N + n) * d + c0 + c] = quant_qk ? mx_round(st, x, e) : x;
                }
            }
    }
}

/*
 * MX quantised attention for the listed rows, elements E2M1 (elem 0, MXFP4)
 * or E2M3 (elem 1, MXFP6), the steps in order:
 *   1. Smooth-K: K' = K - mean_n K (per channel, all tokens of the kv head);
 *   2. Q and K' to MX blocks of 32 channels, V in blocks of 32 tokens (the
 *      element format's codes, shared power-of-two scale 2^e with e the
 *      smallest exponent that keeps the block's max within the format's
 *      largest magnitude, oracle_mx_scale_exp_max);
 *   3. S_ij = scale * (q^_i . k^_j);
 *   4. keys in tiles of tile_n (a multiple of 32) from key 0 upward, with the
 *      exact running max m: m' = max(m, the tile's max visible score),
 *      p_j = exp(S_ij - m') in (0, 1] (the per-row normalisation), l =
 *      l * exp(m - m') + sum_j p_j, and P^ = MX(p) in blocks of 32
 *      consecutive keys (the block's max sets its scale), acc = acc *
 *      exp(m - m') + sum_j P^_j V^_j;
 *   5. O = acc / l;  lse = m + ln l + scale * (q_i . kmean).
 * quant_qk / quant_p / quant_v = 0 skip a quantisation step.
 */
double oracle_mx_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H,
                      int Hkv, int N, int d, int causal, double scale, int tile_n, int elem,
                      int smooth_k, int quant_qk, int quant_p, int quant_v,
                      const int64_t *rows, int64_t nrows, double *o, double *lse, int nthreads)
{
    if (B <= 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || N <= 0 || d <= 0 || d % 32 != 0 ||
        tile_n <= 0 || tile_n % 32 != 0 || (elem != MX_E2M1 && elem != MX_E2M3))
        return -1.0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    if (!rows)
        nrows = (int64_t)B * H * N;
    mx_state st;
    st.elem = elem;
    mx_prepare(q, k, v, B, H, Hkv, N, d, smooth_k, quant_qk, quant_v, &st);
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)tile_n);
        double *P = (double *)malloc(sizeof(double) * (size_t)tile_n);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t row = rows ? rows[r] : r;
            int64_t i = row % N, bh = row / N, h = bh % H, b = bh / H;
            int64_t g = h / (H / Hkv), bg = b * Hkv + g;
            const double *qr = st.qd + (bh * N + i) * d;
            const uint16_t *qraw = q + (bh * N + i) * d;
            int64_t nvis = causal ? i + 1 : N;
            double m = -INFINITY, l = 0.0;
            for (int c = 0; c < d; ++c)
                acc[c] = 0.0;
            for (int64_t j0 = 0; j0 < nvis; j0 += tile_n) {
                int64_t j1 = j0 + tile_n < nvis ? j0 + tile_n : nvis;
                double tmax = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    const double *kr = st.kd + (bg * N + j) * d;
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c)
                        dot += qr[c] * kr[c];
                    S[j - j0] = scale * dot;
                    if (S[j - j0] > tmax)
                        tmax = S[j - j0];
                }
                double mnew = tmax > m ? tmax : m;
                double alpha = exp(m - mnew);
                l *= alpha;
                for (int c = 0; c < d; ++c)
                    acc[c] *= alpha;
                for (int64_t j = j0; j < j1; ++j) {
                    P[j - j0] = exp(S[j - j0] - mnew);
                    l += P[j - j0];
                }
                /* P^ per block of 32 consecutive keys (masked keys are 0) */
                for (int64_t u0 = j0; u0 < j1; u0 += 32) {
                    int64_t u1 = u0 + 32 < j1 ? u0 + 32 : j1;
                    double pmax = 0.0;
                    for (int64_t j = u0; j < u1; ++j)
                        if (P[j - j0] > pmax)
                            pmax = P[j - j0];
                    int e = mx_block_exp(&st, pmax);
                    for (int64_t j = u0; j < u1; ++j) {
                        double ph = quant_p ? mx_round(&st, P[j - j0], e) : P[j - j0];
                        const double *vr = st.vd + (bg * N + j) * d;
                        for (int c = 0; c < d; ++c)
                            acc[c] += ph * vr[c];
                    }
                }
                m = mnew;
            }
            double qk = 0.0;
            for (int c = 0; c < d; ++c)
                qk += bf16_to_f64(qraw[c]) * st.kmean[bg * d + c];
            for (int c = 0; c < d; ++c)
                o[r * d + c] = acc[c] / l;
            lse[r] = m + log(l) + scale * qk;
        }
        free(S);
        free(P);
        free(acc);
    }
    free(st.kmean);
    free(st.qd);
    free(st.kd);
    free(st.vd);
    return 0.0;
}

/* The MXFP4 recipe: oracle_mx_rows with E2M1 elements. */
double oracle_mxfp4_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H,
                         int Hkv, int N, int d, int causal, double scale, int tile_n,
                         int smooth_k, int quant_qk, int quant_p, int quant_v,
                         const int64_t *rows, int64_t nrows, double *o, double *lse,
                         int nthreads)
{
    return oracle_mx_rows(q, k, v, B, H, Hkv, N, d, causal, scale, tile_n, MX_E2M1, smooth_k,
                          quant_qk, quant_p, quant_v, rows, nrows, o, lse, nthreads);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
