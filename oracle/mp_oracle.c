/*
 * CPU oracle for SimHash-sampled decode attention (MagicPIG,
 * "MagicPIG: LSH Sampling for Efficient LLM Generation", arXiv 2410.16179v2).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the HIP implementation.
 *
 * It is the plain, slow statement of what the method computes, in fp64,
 * one function per step and in the pages' order:
 *
 *   key mean          Section 4.3 "Data pre-processing" (k_avg of Section 3.1)
 *   SimHash codes     Section 2.2 "Locality sensitive hashing"; Section 4.3
 *                     "Hash function selection"
 *   sampled set       Section 4.3, Equation 10 (at least two of L tables)
 *   sampling prob.    Section 4.3, Equations 10 and 11
 *   estimator         Section 4.3, Equations 9 and 11; Algorithm 1
 *
 * Readings taken where the pages leave a step open:
 *   - encoder inputs are rounded to bf16 (the GPU GEMM precision):
 *     x = bf16(fp32(k) - mu), w = bf16(W[:, j]), y = bf16(q); queries are not
 *     centred; the projection z = x.w is evaluated exactly (fp64);
 *   - bit = (z > 0); column j = l*K + b is bit b (LSB first) of table l;
 *   - the angle in Equation 10 is taken between q and the centred key k - mu
 *     (the vector that was hashed), both unrounded;
 *   - the logit q.k/sqrt(d) uses the raw key (Equation 11 as written);
 *   - the sampling probability is the binomial tail "at least 2 of L",
 *     which is what Equation 10's closed form equals;
 *   - forced ("static") keys take probability 1 (authors' reply on sink
 *     tokens, page 3);
 *   - an empty sampled set gives out = 0 and lse = -inf;
 *   - the optional lift of Section 4.2, Equation 8 (not used by the authors,
 *     Section 5.1) is applied to the vector that is hashed, the centred key
 *     x = bf16(k - mu): with r the largest |x| of the build keys (fp64 sums,
 *     rounded once to fp32 and frozen with mu), the lifted key is
 *     [x, bf16(fp32(sqrt(max(0, r^2 - |x|^2))))] and the lifted query
 *     [bf16(q), 0]; the sampling angle is that between [q, 0] and the lifted
 *     key, whose norm is r, so cos = q.(k - mu) / (|q| r).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* ---------------------------------------------------------------------------
 * bf16 rounding: keep the upper 16 bits of the fp32 pattern, rounding the
 * discarded lower 16 bits to nearest with ties to even.  NaN stays NaN.
 * ------------------------------------------------------------------------- */
float orc_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
        u = (u | 0x00400000u) & 0xffff0000u; /* quiet NaN */
    } else {
        uint32_t kept = u & 0xffff0000u;
        uint32_t rest = u & 0x0000ffffu;
        uint32_t kept_lsb = (u >> 16) & 1u;
        if (rest > 0x8000u || (rest == 0x8000u && kept_lsb))
            kept += 0x00010000u; /* carries into the exponent when needed */
        u = kept;
    }
    memcpy(&x, &u, sizeof u);
    return x;
}

/* ---------------------------------------------------------------------------
 * Key mean (Section 4.3 "Data pre-processing"): mu = (1/n) sum_i k_i, summed
 * in fp64 in index order and rounded once to fp32.  n = 0 gives mu = 0.
 * keys: n rows of d floats, row stride `stride` floats.
 * ------------------------------------------------------------------------- */
void orc_key_mean(const float *keys, int64_t n, int d, int64_t stride, float *mu)
{
    for (int t = 0; t < d; ++t) {
        double s = 0.0;
        for (int64_t i = 0; i < n; ++i)
            s += (double)keys[i * stride + t];
        mu[t] = n > 0 ? (float)(s / (double)n) : 0.0f;
    }
}

/* ---------------------------------------------------------------------------
 * SimHash codes (Section 2.2; Section 4.3 "Hash function selection").
 * For each row r: x = bf16(fp32(row - mu_r)) with mu_r = mu + r * mu_stride
 * (mu may be NULL: no centring; mu_stride 0: one mean for every row),
 * z_j = sum_t x_t * bf16(W[t][j]) in fp64, bit_j = (z_j > 0), and
 * code_l = sum_{b<K} bit_{l*K+b} << b.
 *
 * W is d x (K*L), row-major (Algorithm 1's W in R^{d x (K x L)}).
 * codes[r * code_row_stride + l * code_table_stride] receives code_l.
 * margin (nullable, [nrows][K*L]) receives, per projection column j, the
 * relative size |z_j| / (|x| |w_j|) of the projection that decides bit j:
 * a bit whose margin is tiny depends on the rounding order of the sum.
 * When |x| |w_j| = 0 the projection is exactly 0 and the bit exactly 0,
 * whatever the order, so the margin is +inf.
 * ------------------------------------------------------------------------- */
void orc_encode(const float *rows, int64_t nrows, int d, int64_t row_stride, const float *mu,
                int64_t mu_stride, const float *W, int K, int L, uint16_t *codes, int64_t code_row_stride,
                int64_t code_table_stride, float *margin)
{
    const int ncol = K * L;
    double *wb = (double *)malloc(sizeof(double) * (size_t)d * (size_t)(ncol > 0 ? ncol : 1));
    double *wnorm = (double *)malloc(sizeof(double) * (size_t)(ncol > 0 ? ncol : 1));
    for (int j = 0; j < ncol; ++j) {
        double s = 0.0;
        for (int t = 0; t < d; ++t) {
            double w = (double)orc_bf16(W[(int64_t)t * ncol + j]);
            wb[(int64_t)j * d + t] = w;
            s += w * w;
        }
        wnorm[j] = sqrt(s);
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        double *x = (double *)malloc(sizeof(double) * (size_t)d);
        double xn = 0.0;
        for (int t = 0; t < d; ++t) {
            float k = rows[r * row_stride + t];
            float c = mu ? k - mu[r * mu_stride + t] : k; /* fp32 subtraction */
            x[t] = (double)orc_bf16(c);
            xn += x[t] * x[t];
        }
        xn = sqrt(xn);
        for (int l = 0; l < L; ++l) {
            unsigned code = 0;
            for (int b = 0; b < K; ++b) {
                const int j = l * K + b;
                double z = 0.0;
                for (int t = 0; t < d; ++t)
                    z += x[t] * wb[(int64_t)j * d + t];
                if (z > 0.0)
                    code |= 1u << b;
                if (margin) {
                    const double den = xn * wnorm[j];
                    margin[r * ncol + j] = den > 0.0 ? (float)(fabs(z) / den) : INFINITY;
                }
            }
            codes[r * code_row_stride + (int64_t)l * code_table_stride] = (uint16_t)code;
        }
        free(x);
    }
    free(wb);
    free(wnorm);
}

/* ---------------------------------------------------------------------------
 * Lift radius of Section 4.2, Equation 8 (r = max_i |k_i|), taken over the
 * vectors that are hashed, x_i = bf16(fp32(k_i) - mu): |x_i|^2 summed in
 * fp64, the largest of them, its square root rounded once to fp32.
 * ------------------------------------------------------------------------- */
float orc_lift_radius(const float *rows, int64_t n, int d, int64_t row_stride, const float *mu)
{
    double best = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int t = 0; t < d; ++t) {
            const double x = (double)orc_bf16(rows[i * row_stride + t] - mu[t]);
            s += x * x;
        }
        if (s > best) best = s;
    }
    return (float)sqrt(best);
}

/* ---------------------------------------------------------------------------
 * SimHash codes of lifted keys (Section 4.2, Equation 8, then Section 2.2):
 * row r becomes x = bf16(fp32(row - mu_r)) (mu_r = mu + r * mu_stride, or no
 * centring when mu is NULL) extended by the coordinate
 * e = bf16(fp32(sqrt(max(0, R^2 - |x|^2)))) (fp64 inside the root; R the
 * lift radius), so that every lifted key has norm R up to rounding.  A row
 * with lift = 0 is a lifted query: its extra coordinate is 0.  W is
 * (d + 1) x (K*L); z_j = sum_t x_t bf16(W[t][j]) + e bf16(W[d][j]) exactly
 * (fp64); bit_j = (z_j > 0).  margin as in orc_encode, over the d + 1
 * coordinates.
 * ------------------------------------------------------------------------- */
void orc_encode_lifted(const float *rows, int64_t nrows, int d, int64_t row_stride, const float *mu,
                       int64_t mu_stride, int lift, float R, const float *W, int K, int L, uint16_t *codes,
                       int64_t code_row_stride, int64_t code_table_stride, float *margin)
{
    const int ncol = K * L, d1 = d + 1;
    double *wb = (double *)malloc(sizeof(double) * (size_t)d1 * (size_t)(ncol > 0 ? ncol : 1));
    double *wnorm = (double *)malloc(sizeof(double) * (size_t)(ncol > 0 ? ncol : 1));
    for (int j = 0; j < ncol; ++j) {
        double s = 0.0;
        for (int t = 0; t < d1; ++t) {
            double w = (double)orc_bf16(W[(int64_t)t * ncol + j]);
            wb[(int64_t)j * d1 + t] = w;
            s += w * w;
        }
        wnorm[j] = sqrt(s);
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        double *x = (double *)malloc(sizeof(double) * (size_t)d1);
        double xx = 0.0;
        for (int t = 0; t < d; ++t) {
            float k = rows[r * row_stride + t];
            float c = mu ? k - mu[r * mu_stride + t] : k; /* fp32 subtraction */
            x[t] = (double)orc_bf16(c);
            xx += x[t] * x[t];
        }
        double e = 0.0;
        if (lift) {
            double rem = (double)R * (double)R - xx;
            e = (double)orc_bf16((float)sqrt(rem > 0.0 ? rem : 0.0));
        }
        x[d] = e;
        const double xn = sqrt(xx + e * e);
        for (int l = 0; l < L; ++l) {
            unsigned code = 0;
            for (int b = 0; b < K; ++b) {
                const int j = l * K + b;
                double z = 0.0;
                for (int t = 0; t < d1; ++t)
                    z += x[t] * wb[(int64_t)j * d1 + t];
                if (z > 0.0)
                    code |= 1u << b;
                if (margin) {
                    const double den = xn * wnorm[j];
                    margin[r * ncol + j] = den > 0.0 ? (float)(fabs(z) / den) : INFINITY;
                }
            }
            codes[r * code_row_stride + (int64_t)l * code_table_stride] = (uint16_t)code;
        }
        free(x);
    }
    free(wb);
    free(wnorm);
}

/* ---------------------------------------------------------------------------
 * Per-table collision probability of SimHash (Section 2.2): one random
 * hyperplane separates two vectors at angle theta with probability
 * theta/pi, so K independent ones all agree with probability
 * (1 - theta/pi)^K.  The cosine is clamped to [-1, 1].
 * ------------------------------------------------------------------------- */
double orc_table_collision_prob(double cos_qk, int K)
{
    if (cos_qk > 1.0) cos_qk = 1.0;
    if (cos_qk < -1.0) cos_qk = -1.0;
    double u = 1.0 - acos(cos_qk) / M_PI;
    return pow(u, (double)K);
}

/* ---------------------------------------------------------------------------
 * Sampling probability (Section 4.3, Equation 10): a key is sampled when it
 * shares its code with the query in at least T of the L independent tables,
 * each matching with probability p.  Written as the binomial tail
 * P = sum_{j=T}^{L} C(L,j) p^j (1-p)^(L-j); for the pages' threshold T = 2
 * this is the quantity Equation 10 states in closed form.  The tail sum has
 * no cancellation.
 * ------------------------------------------------------------------------- */
double orc_sampling_prob_pt(double p, int L, int T)
{
    double P = 0.0, c = 1.0; /* c = C(L, j) */
    for (int j = 0; j <= L; ++j) {
        if (j > 0) c = c * (double)(L - j + 1) / (double)j;
        if (j >= T)
            P += c * pow(p, (double)j) * pow(1.0 - p, (double)(L - j));
    }
    return P;
}

double orc_sampling_prob_p(double p, int L) { return orc_sampling_prob_pt(p, L, 2); }

double orc_sampling_prob_t(double cos_qk, int K, int L, int T)
{
    return orc_sampling_prob_pt(orc_table_collision_prob(cos_qk, K), L, T);
}

double orc_sampling_prob(double cos_qk, int K, int L) { return orc_sampling_prob_t(cos_qk, K, L, 2); }

/* ---------------------------------------------------------------------------
 * Sampled set of one query head (Section 4.3 "Hash function selection",
 * Algorithm 1 "Query hash tables"): key i is sampled when its code equals
 * the query's code in at least T of the L tables (the pages use T = 2).  Keys i < n_static_head
 * and i >= n - n_static_tail are always included and flagged as forced
 * (Algorithm 1's static cache K_T, V_T; the authors' reply on sink tokens).
 * codes: table l of key i at codes[l * table_stride + i].
 * Writes the ascending index list (nullable) and forced flags (nullable);
 * returns its length.
 * ------------------------------------------------------------------------- */
int64_t orc_scan_t(const uint16_t *codes, int64_t table_stride, int64_t n, int L, int T, const uint16_t *qcode,
                   int64_t n_static_head, int64_t n_static_tail, int32_t *idx, uint8_t *forced)
{
    int64_t cnt = 0;
    for (int64_t i = 0; i < n; ++i) {
        int is_forced = (i < n_static_head) || (i >= n - n_static_tail);
        int matches = 0;
        for (int l = 0; l < L; ++l)
            matches += codes[(int64_t)l * table_stride + i] == qcode[l];
        if (is_forced || matches >= T) {
            if (idx) idx[cnt] = (int32_t)i;
            if (forced) forced[cnt] = (uint8_t)is_forced;
            ++cnt;
        }
    }
    return cnt;
}

int64_t orc_scan(const uint16_t *codes, int64_t table_stride, int64_t n, int L, const uint16_t *qcode,
                 int64_t n_static_head, int64_t n_static_tail, int32_t *idx, uint8_t *forced)
{
    return orc_scan_t(codes, table_stride, n, L, 2, qcode, n_static_head, n_static_tail, idx, forced);
}

/* ---------------------------------------------------------------------------
 * Estimator of one query head over its sampled set (Equations 9 and 11,
 * Algorithm 1 "Compute attention output estimation"):
 *   s_i   = q.k_i / sqrt(d)                      (raw key)
 *   cos_i = q.(k_i - mu) / (|q| |k_i - mu|)      (0 if a norm is 0)
 *   lnP_i = ln P(cos_i), tail from T             (0 for forced keys)
 *   out   = sum_i softmax(s - lnP)_i v_i,  lse = logsumexp(s - lnP)
 * An empty set gives out = 0, lse = -inf.  mu may be NULL (no centring).
 * logw (nullable, [cnt]) receives s_i - lnP_i.
 * ------------------------------------------------------------------------- */
void orc_attend_lt(const float *q, const float *keys, const float *vals, int64_t row_stride, int d,
                   const float *mu, float rlift, int K, int L, int T, const int32_t *idx, const uint8_t *forced,
                   int64_t cnt, double *out, double *lse, double *logw);

void orc_attend_t(const float *q, const float *keys, const float *vals, int64_t row_stride, int d,
                  const float *mu, int K, int L, int T, const int32_t *idx, const uint8_t *forced, int64_t cnt,
                  double *out, double *lse, double *logw)
{
    orc_attend_lt(q, keys, vals, row_stride, d, mu, 0.0f, K, L, T, idx, forced, cnt, out, lse, logw);
}

/* As orc_attend_t; with rlift > 0 the keys were hashed lifted (Equation 8)
 * with radius rlift, and the sampling angle is that between [q, 0] and the
 * lifted key (norm rlift): cos = q.(k - mu) / (|q| rlift). */
void orc_attend_lt(const float *q, const float *keys, const float *vals, int64_t row_stride, int d,
                   const float *mu, float rlift, int K, int L, int T, const int32_t *idx, const uint8_t *forced,
                   int64_t cnt, double *out, double *lse, double *logw)
{
    for (int t = 0; t < d; ++t)
        out[t] = 0.0;
    if (cnt == 0) {
        *lse = -INFINITY;
        return;
    }
    double *lw = (double *)malloc(sizeof(double) * (size_t)cnt);
    double qn = 0.0;
    for (int t = 0; t < d; ++t)
        qn += (double)q[t] * (double)q[t];
    qn = sqrt(qn);
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double M = -INFINITY;
    for (int64_t s = 0; s < cnt; ++s) {
        const float *k = keys + (int64_t)idx[s] * row_stride;
        double qk = 0.0, qc = 0.0, cn = 0.0;
        for (int t = 0; t < d; ++t) {
            double kt = (double)k[t];
            double ct = kt - (mu ? (double)mu[t] : 0.0);
            qk += (double)q[t] * kt;
            qc += (double)q[t] * ct;
            cn += ct * ct;
        }
        cn = rlift > 0.0f ? (double)rlift : sqrt(cn);
        double lnP = 0.0;
        if (!(forced && forced[s])) {
            double cosv = (qn > 0.0 && cn > 0.0) ? qc / (qn * cn) : 0.0;
            lnP = log(orc_sampling_prob_t(cosv, K, L, T));
        }
        lw[s] = qk * inv_sqrt_d - lnP;
        if (lw[s] > M) M = lw[s];
    }
    double Z = 0.0;
    for (int64_t s = 0; s < cnt; ++s) {
        double e = exp(lw[s] - M);
        Z += e;
        const float *v = vals + (int64_t)idx[s] * row_stride;
        for (int t = 0; t < d; ++t)
            out[t] += e * (double)v[t];
    }
    for (int t = 0; t < d; ++t)
        out[t] /= Z;
    *lse = M + log(Z);
    if (logw)
        memcpy(logw, lw, sizeof(double) * (size_t)cnt);
    free(lw);
}

void orc_attend(const float *q, const float *keys, const float *vals, int64_t row_stride, int d,
                const float *mu, int K, int L, const int32_t *idx, const uint8_t *forced, int64_t cnt,
                double *out, double *lse, double *logw)
{
    orc_attend_t(q, keys, vals, row_stride, d, mu, K, L, 2, idx, forced, cnt, out, lse, logw);
}

/* ---------------------------------------------------------------------------
 * Code-store build of one layer: per unit u (batch x KV head) the key mean
 * over its n keys, then the centred codes of every key.
 *   keys  [U][cap][d] fp32       kmean [U][d]       codes [U][L][cap]
 * ------------------------------------------------------------------------- */
void orc_build(const float *keys, int64_t U, int64_t n, int64_t cap, int d, const float *W, int K, int L,
               float *kmean, uint16_t *codes, float *margin /* nullable [U][n][K*L] */)
{
    for (int64_t u = 0; u < U; ++u) {
        const float *ku = keys + u * cap * d;
        orc_key_mean(ku, n, d, d, kmean + u * d);
        orc_encode(ku, n, d, d, kmean + u * d, 0, W, K, L, codes + u * (int64_t)L * cap, 1, cap,
                   margin ? margin + u * n * (int64_t)K * L : NULL);
    }
}

/* ---------------------------------------------------------------------------
 * Decode of one layer (Algorithm 1 for every query head, threshold T).
 * Query head h reads KV head h / (Hq / Hkv).
 *   q [B][Hq][d]; keys, vals [B][Hkv][cap][d]; codes [B][Hkv][L][cap];
 *   kmean [B][Hkv][d]; qcodes [B][Hq][L] (NULL: encode q here, uncentred);
 *   out [B][Hq][d]; lse [B][Hq]; idx [B][Hq][cap] (nullable); count [B][Hq].
 * ------------------------------------------------------------------------- */
void orc_decode_lt(const float *q, const float *keys, const float *vals, const uint16_t *codes,
                   const float *kmean, const float *rlift, const float *W, const uint16_t *qcodes_in, int B, int Hq,
                   int Hkv, int64_t n, int64_t cap, int d, int K, int L, int T, int64_t n_static_head,
                   int64_t n_static_tail, uint16_t *qcodes_out, float *out, float *lse, int32_t *idx,
                   int32_t *count);

void orc_decode_t(const float *q, const float *keys, const float *vals, const uint16_t *codes,
                  const float *kmean, const float *W, const uint16_t *qcodes_in, int B, int Hq, int Hkv,
                  int64_t n, int64_t cap, int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail,
                  uint16_t *qcodes_out, float *out, float *lse, int32_t *idx, int32_t *count)
{
    orc_decode_lt(q, keys, vals, codes, kmean, NULL, W, qcodes_in, B, Hq, Hkv, n, cap, d, K, L, T, n_static_head,
                  n_static_tail, qcodes_out, out, lse, idx, count);
}

/* As orc_decode_t; rlift (nullable, [B][Hkv]) gives each unit's lift radius
 * when its keys were hashed lifted (Equation 8).  Queries are encoded (when
 * qcodes_in is NULL) with the first d rows of W: their extra coordinate is 0. */
void orc_decode_lt(const float *q, const float *keys, const float *vals, const uint16_t *codes,
                   const float *kmean, const float *rlift, const float *W, const uint16_t *qcodes_in, int B, int Hq,
                   int Hkv, int64_t n, int64_t cap, int d, int K, int L, int T, int64_t n_static_head,
                   int64_t n_static_tail, uint16_t *qcodes_out, float *out, float *lse, int32_t *idx,
                   int32_t *count)
{
    const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
        const int64_t b = bh / Hq, h = bh % Hq, u = b * Hkv + h / G;
        const float *qh = q + bh * d;
        uint16_t *qc = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)L);
        if (qcodes_in)
            memcpy(qc, qcodes_in + bh * L, sizeof(uint16_t) * (size_t)L);
        else
            orc_encode(qh, 1, d, d, NULL, 0, W, K, L, qc, 0, 1, NULL);
        if (qcodes_out)
            memcpy(qcodes_out + bh * L, qc, sizeof(uint16_t) * (size_t)L);
        int32_t *list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
        uint8_t *forced = (uint8_t *)malloc((size_t)(n > 0 ? n : 1));
        int64_t cnt = orc_scan_t(codes + u * (int64_t)L * cap, cap, n, L, T, qc, n_static_head, n_static_tail,
                                 list, forced);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        double l;
        orc_attend_lt(qh, keys + u * cap * d, vals + u * cap * d, d, d, kmean + u * d, rlift ? rlift[u] : 0.0f, K,
                      L, T, list, forced, cnt, o, &l, NULL);
        for (int t = 0; t < d; ++t)
            out[bh * d + t] = (float)o[t];
        if (lse) lse[bh] = (float)l;
        if (count) count[bh] = (int32_t)cnt;
        if (idx)
            memcpy(idx + bh * cap, list, sizeof(int32_t) * (size_t)cnt);
        free(o);
        free(forced);
        free(list);
        free(qc);
    }
}

void orc_decode(const float *q, const float *keys, const float *vals, const uint16_t *codes,
                const float *kmean, const float *W, const uint16_t *qcodes_in, int B, int Hq, int Hkv,
                int64_t n, int64_t cap, int d, int K, int L, int64_t n_static_head, int64_t n_static_tail,
                uint16_t *qcodes_out, float *out, float *lse, int32_t *idx, int32_t *count)
{
    orc_decode_t(q, keys, vals, codes, kmean, W, qcodes_in, B, Hq, Hkv, n, cap, d, K, L, 2, n_static_head,
                 n_static_tail, qcodes_out, out, lse, idx, count);
}

/* Threads the oracle's parallel loops use from now on (timing only; the
 * results do not depend on it). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
