/*
 * kv4_oracle.c -- plain, slow, fp64 CPU oracle for the KV4 decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header or table with the HIP
 * kernels.
 *
 * What it computes, and where the method is stated (KV4-RL: "Unlocking Faster
 * Asynchronous Rollouts for RLVR with INT4 KV Cache Quantization",
 * arXiv 2610.14448):
 *   - the b-bit affine quantizer x^ = Delta*c + m with c in {0..2^b-1}, Delta > 0
 *     (Section 3, eq. 3.3), used with b = 4 and FP16 Delta and m per group of
 *     channels of one token-head vector (Section 5.1; Appendix A.3, "Encoding
 *     and allocation"; Appendix D.4, Fig. A4b for groups finer than a head);
 *   - symmetric per-(token, head) INT8 side copies computed from the source
 *     vector, not from its INT4 rounding (Appendix A.3);
 *   - the protected set: the first s positions and the w most recent positions
 *     (Section 5.2, "Bounded selective protection"), read from the INT8 copy,
 *     all other positions read from INT4, disjointly (Section 5.3);
 *   - exact softmax attention over the dequantized cache.  The paper's
 *     regional merge (eq. A1) and context splits reach this same result; the
 *     oracle therefore does not implement them.
 *
 * Readings of steps the pages leave open (the pages fix only "affine INT4 with
 * FP16 scale and offset" and "symmetric INT8"):
 *   Q-1  m = fp16_rne(min x); r = fp32(max x - m); Delta = fp16_rne(fp32(r/15));
 *        Delta = 0 when r <= 0 or when it rounds to zero; stored zeros are +0.
 *   Q-2  c = integer in [0,15] nearest to the exact real (x - m)/Delta, ties to
 *        even; c = 0 when Delta = 0.
 *   Q-4  s = fp16_rne(fp32(amax/127)); c = integer nearest to the exact x/s,
 *        ties to even, clamped to [-127,127]; c = 0 when s = 0.
 *   Q-5  protected = [0, min(S,n)) U [max(S, n-R), n); INT4 = the rest.
 *   Q-6  q head j reads kv head j / (Hq/Hkv); the new token attends to itself.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * fp32 steps are ordinary C float arithmetic (SSE, FLT_EVAL_METHOD == 0),
 * each correctly rounded to nearest-even.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float expressions evaluated in float (FLT_EVAL_METHOD 0)"
#endif

/* ------------------------------------------------------------------------ */
/* IEEE binary16 conversion, written from the format's definition.           */
/* ------------------------------------------------------------------------ */

/* Round a binary32 value to the nearest binary16 value, ties to even.
 * Values whose magnitude rounds to 65520 or more become infinity; NaN stays
 * a quiet NaN.  Returns the binary16 bit pattern (sign kept, -0 stays -0). */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)f);               /* exact */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                            /* a = mant * 2^e2, mant in [0.5,1) */
    int E = e2 - 1;                           /* floor(log2 a) */
    if (E < -14) E = -14;                     /* subnormal range shares one quantum */
    double quantum = ldexp(1.0, E - 10);      /* spacing of binary16 values near a */
    double N = nearbyint(a / quantum);        /* exact scaling, then round half even */
    uint32_t Ni = (uint32_t)N;                /* 0 .. 2048 */
    if (E == -14 && Ni < 1024u) return (uint16_t)(sign | Ni);   /* subnormal or zero */
    if (Ni == 2048u) { Ni = 1024u; E += 1; }  /* mantissa carry into the exponent */
    if (E > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(((uint32_t)(E + 15) << 10) | (Ni - 1024u)));
}

/* Exact value of a binary16 bit pattern. */
double orc_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int E = (h >> 10) & 31;
    int M = h & 1023;
    double v;
    if (E == 0) v = ldexp((double)M, -24);
    else if (E == 31) v = M ? NAN : INFINITY;
    else v = ldexp((double)(1024 + M), E - 25);
    return s ? -v : v;
}

/* Convert many values at once (used by the conversion pin tests). */
void orc_f32_to_f16_array(const float* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f64_array(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(h[i]);
}

static uint16_t plus_zero(uint16_t h) { return h == 0x8000u ? (uint16_t)0 : h; }

/* ------------------------------------------------------------------------ */
/* Q-1 / Q-2: asymmetric INT4 with FP16 scale and offset per group.          */
/* ------------------------------------------------------------------------ */

/* One token-head vector x[d] (bf16 values carried exactly in float).
 * codes[d] get values 0..15; delta[d/G], offs[d/G] get binary16 patterns. */
void orc_quant_int4_vec(const float* x, int d, int G, uint8_t* codes,
                        uint16_t* delta, uint16_t* offs)
{
    for (int g = 0; g < d / G; ++g) {
        const float* xg = x + (size_t)g * G;
        float lo = xg[0], hi = xg[0];
        for (int i = 1; i < G; ++i) {
            if (xg[i] < lo) lo = xg[i];
            if (xg[i] > hi) hi = xg[i];
        }
        uint16_t mb = plus_zero(orc_f32_to_f16(lo));
        float mf = (float)orc_f16_to_f64(mb);     /* exact: binary16 fits binary32 */
        float r = hi - mf;                        /* one binary32 rounding */
        uint16_t db = 0;
        if (r > 0.0f) {
            float qq = r / 15.0f;                 /* correctly rounded binary32 division */
            db = plus_zero(orc_f32_to_f16(qq));
        }
        delta[g] = db;
        offs[g] = mb;
        double D = orc_f16_to_f64(db), M = orc_f16_to_f64(mb);
        for (int i = 0; i < G; ++i) {
            int c = 0;
            if (db != 0) {
                /* nearest grid point M + c*D; the midpoint between codes k and
                 * k+1 is M + (k+1/2)*D, exact in binary64 because M and D are
                 * binary16 values. At a midpoint, the even code wins. */
                double xv = (double)xg[i];
                for (int k = 0; k < 15; ++k) {
                    double mid = M + ((double)k + 0.5) * D;
                    if (xv > mid || (xv == mid && ((k + 1) % 2) == 0)) ++c;
                }
            }
            codes[(size_t)g * G + i] = (uint8_t)c;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q-4: symmetric INT8 with an FP16 scale per token-head vector.             */
/* ------------------------------------------------------------------------ */

void orc_quant_int8_vec(const float* x, int d, int8_t* codes, uint16_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < d; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float qq = amax / 127.0f;                     /* correctly rounded binary32 division */
    uint16_t sb = plus_zero(orc_f32_to_f16(qq));
    *scale = sb;
    double S = orc_f16_to_f64(sb);
    for (int i = 0; i < d; ++i) {
        int c = 0;
        if (sb != 0) {
            double a = fabs((double)x[i]);
            /* nearest multiple c*S of the magnitude, c <= 127; midpoints
             * (k+1/2)*S are exact in binary64; ties go to the even c. */
            for (int k = 0; k < 127; ++k) {
                double mid = ((double)k + 0.5) * S;
                if (a > mid || (a == mid && ((k + 1) % 2) == 0)) ++c;
            }
            if (x[i] < 0.0f) c = -c;
        }
        codes[i] = (int8_t)c;
    }
}

/* Batched forms over nvec consecutive vectors of d channels. */
void orc_quant_int4(const float* x, int64_t nvec, int d, int G, uint8_t* codes,
                    uint16_t* delta, uint16_t* offs)
{
    int ng = d / G;
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nvec; ++v)
        orc_quant_int4_vec(x + v * d, d, G, codes + v * d, delta + v * ng, offs + v * ng);
}

void orc_quant_int8(const float* x, int64_t nvec, int d, int8_t* codes, uint16_t* scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nvec; ++v)
        orc_quant_int8_vec(x + v * d, d, codes + v * d, scale + v);
}

/* ------------------------------------------------------------------------ */
/* R-10: the fixed normalized Hadamard transform of keys (after RoPE, before */
/* quantization) and of queries (before attention), KV4-RL Section 5.1 and   */
/* Appendix A.3 "Encoding and allocation"; scores are kept because HH^T = I  */
/* (eq. 3.4).                                                                */
/* ------------------------------------------------------------------------ */

/* y = x H / sqrt(d) for the Sylvester Hadamard matrix H of order d (a power
 * of two, H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), in binary32 and in one
 * fixed order (the pages fix no order; bit-exact stored codes need one):
 * stages of span h = 1, 2, 4, ..., d/2, each replacing every pair
 * (z[c], z[c+h]) with c & h == 0 by (z[c] + z[c+h], z[c] - z[c+h]), each sum one
 * binary32 rounding; then every element times the binary32 value nearest
 * 1/sqrt(d), one more rounding. */
void orc_wht_f32(const float* x, int64_t nvec, int d, float* y)
{
    const float s = (float)(1.0 / sqrt((double)d));
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nvec; ++v) {
        float z[1024];
        for (int c = 0; c < d && c < 1024; ++c) z[c] = x[v * d + c];
        for (int h = 1; h < d && d <= 1024; h <<= 1)
            for (int c = 0; c < d; ++c)
                if ((c & h) == 0) {
                    const float a = z[c], b = z[c + h];
                    z[c] = a + b;
                    z[c + h] = a - b;
                }
        for (int c = 0; c < d && c < 1024; ++c) y[v * d + c] = z[c] * s;
    }
}

float orc_wht_scale(int d) { return (float)(1.0 / sqrt((double)d)); }

/* ------------------------------------------------------------------------ */
/* Q-5: which copy a position is read from.                                  */
/* ------------------------------------------------------------------------ */

/* 1 if position p of an n-token context reads the INT8 side copy. */
int orc_is_protected(int64_t p, int64_t n, int S, int R)
{
    int64_t sink_end = n < S ? n : S;
    int64_t rec_start = n - R > S ? n - R : S;
    return p < sink_end || (p >= rec_start && p < n);
}

/* ------------------------------------------------------------------------ */
/* Q-6: softmax attention over the dequantized cache, in binary64.           */
/* ------------------------------------------------------------------------ */

/*
 * Mixed cache.  Positions of all B sequences are stored back to back; sequence
 * b owns rows [pos_off[b], pos_off[b] + seq_lens[b]).  Per row r and kv head h:
 *   k4[(r*Hkv+h)*d + c]      INT4 code of channel c (0..15)
 *   k4d/k4m[(r*Hkv+h)*ng+g]  binary16 Delta / m of group g (ng = d/G)
 *   k8[(r*Hkv+h)*d + c]      INT8 code, k8s[r*Hkv+h] binary16 scale
 * and the same for V.  q is [B][Hq][d] (bf16 values in float); out [B][Hq][d].
 */
void orc_attend_mixed(int B, const int32_t* seq_lens, const int64_t* pos_off,
                      int Hq, int Hkv, int d, int G, int S, int R, double sm_scale,
                      const float* q,
                      const uint8_t* k4, const uint16_t* k4d, const uint16_t* k4m,
                      const uint8_t* v4, const uint16_t* v4d, const uint16_t* v4m,
                      const int8_t* k8, const uint16_t* k8s,
                      const int8_t* v8, const uint16_t* v8s,
                      double* out)
{
    int ng = d / G;
    int gqa = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bj = 0; bj < (int64_t)B * Hq; ++bj) {
        int b = (int)(bj / Hq), j = (int)(bj % Hq);
        int h = j / gqa;
        int64_t n = seq_lens[b];
        const float* qj = q + ((int64_t)b * Hq + j) * d;
        double* o = out + ((int64_t)b * Hq + j) * d;
        double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double* vh = (double*)malloc(sizeof(double) * (size_t)d);
        double smax = -INFINITY;
        for (int64_t p = 0; p < n; ++p) {
            int64_t row = (pos_off[b] + p) * Hkv + h;
            int prot = orc_is_protected(p, n, S, R);
            double dot = 0.0;
            for (int c = 0; c < d; ++c) {
                double kh;
                if (prot) kh = orc_f16_to_f64(k8s[row]) * (double)k8[row * d + c];
                else kh = orc_f16_to_f64(k4d[row * ng + c / G]) * (double)k4[row * d + c]
                          + orc_f16_to_f64(k4m[row * ng + c / G]);
                dot += (double)qj[c] * kh;
            }
            s[p] = sm_scale * dot;
            if (s[p] > smax) smax = s[p];
        }
        double den = 0.0;
        for (int64_t p = 0; p < n; ++p) { s[p] = exp(s[p] - smax); den += s[p]; }
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t p = 0; p < n; ++p) {
            int64_t row = (pos_off[b] + p) * Hkv + h;
            int prot = orc_is_protected(p, n, S, R);
            for (int c = 0; c < d; ++c) {
                if (prot) vh[c] = orc_f16_to_f64(v8s[row]) * (double)v8[row * d + c];
                else vh[c] = orc_f16_to_f64(v4d[row * ng + c / G]) * (double)v4[row * d + c]
                             + orc_f16_to_f64(v4m[row * ng + c / G]);
            }
            double w = s[p] / den;
            for (int c = 0; c < d; ++c) o[c] += w * vh[c];
        }
        free(vh);
        free(s);
    }
}

/* BF16 cache (the comparator): keys and values are the source values. */
void orc_attend_dense(int B, const int32_t* seq_lens, const int64_t* pos_off,
                      int Hq, int Hkv, int d, double sm_scale,
                      const float* q, const float* k, const float* v, double* out)
{
    int gqa = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bj = 0; bj < (int64_t)B * Hq; ++bj) {
        int b = (int)(bj / Hq), j = (int)(bj % Hq);
        int h = j / gqa;
        int64_t n = seq_lens[b];
        const float* qj = q + ((int64_t)b * Hq + j) * d;
        double* o = out + ((int64_t)b * Hq + j) * d;
        double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double smax = -INFINITY;
        for (int64_t p = 0; p < n; ++p) {
            const float* kp = k + ((pos_off[b] + p) * Hkv + h) * d;
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += (double)qj[c] * (double)kp[c];
            s[p] = sm_scale * dot;
            if (s[p] > smax) smax = s[p];
        }
        double den = 0.0;
        for (int64_t p = 0; p < n; ++p) { s[p] = exp(s[p] - smax); den += s[p]; }
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t p = 0; p < n; ++p) {
            const float* vp = v + ((pos_off[b] + p) * Hkv + h) * d;
            double w = s[p] / den;
            for (int c = 0; c < d; ++c) o[c] += w * (double)vp[c];
        }
        free(s);
    }
}

/* ------------------------------------------------------------------------ */
/* The integer decode path (KV4-RL Appendix A.3, "Integer decode path" and   */
/* "Protected path and reconstruction"; Section 5.3), in binary64.           */
/* ------------------------------------------------------------------------ */

/*
 * The pages state the steps (INT8 query; integer QK on widened INT4 codes with
 * the scales and offsets applied to the integer sums; FP32 softmax; an 8-bit
 * probability operand carrying the value scales for an integer PV with an
 * affine correction; integer QK and higher-precision PV for the protected
 * positions) but not the operand scales.  Readings:
 *   I-1 q (already in the keys' basis when keys are rotated) is quantized per
 *       (sequence, q head) with Q-4: scale s_q, codes qi.
 *   I-2 INT4 position t: score = sm_scale * s_q * sum_g (Delta_g I_g + m_g Q_g),
 *       I_g = sum_{c in g} qi_c k4_c and Q_g = sum_{c in g} qi_c (integers).
 *   I-3 protected position t: score = sm_scale * s_q * s_k * sum_c qi_c k8_c.
 *   I-4 p_t = exp(score_t - max) over the whole context; the normalizer is
 *       sum_t p_t of the unquantized probabilities.
 *   I-5 8-bit probability operand: INT4 positions are cut into blocks
 *       [8k, 8k + 8) (a half page, the unit of the stored V codes); per block
 *       B, value group g and q head, w_t = p_t Delta^v_{t,g},
 *       sigma = max_{t in B} w_t / 255 and u_t = the integer nearest to
 *       w_t / sigma (ties to even; 0 when sigma = 0).
 *   I-6 numerator of channel c: over INT4 positions
 *       sum_B sigma_B sum_t u_t v4_{t,c} + sum_t p_t m^v_{t,g(c)}; over protected
 *       positions sum_t p_t s_v v8_{t,c} (no probability quantization).
 * The pages merge the two regions' outputs by their log-normalizers (eq. A1);
 * the codes u do not depend on the reference maximum, so that merge reaches
 * this single-softmax result in exact arithmetic.
 *
 * bound[c] is the change of out[c] if every code u whose w/sigma lies within
 * eps of a half-integer moved by one: sum of sigma_B v4_{t,c} over those codes,
 * divided by the normalizer.  (An implementation computing p in lower
 * precision may round exactly those codes the other way.)
 */
void orc_attend_int(int B, const int32_t* seq_lens, const int64_t* pos_off,
                    int Hq, int Hkv, int d, int G, int S, int R, double sm_scale,
                    const float* q,
                    const uint8_t* k4, const uint16_t* k4d, const uint16_t* k4m,
                    const uint8_t* v4, const uint16_t* v4d, const uint16_t* v4m,
                    const int8_t* k8, const uint16_t* k8s,
                    const int8_t* v8, const uint16_t* v8s,
                    double eps, double* out, double* bound)
{
    int ng = d / G;
    int gqa = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bj = 0; bj < (int64_t)B * Hq; ++bj) {
        int b = (int)(bj / Hq), j = (int)(bj % Hq);
        int h = j / gqa;
        int64_t n = seq_lens[b];
        const float* qj = q + ((int64_t)b * Hq + j) * d;
        double* o = out + ((int64_t)b * Hq + j) * d;
        double* bd = bound + ((int64_t)b * Hq + j) * d;
        int8_t* qi = (int8_t*)malloc((size_t)d);
        uint16_t sqb;
        orc_quant_int8_vec(qj, d, qi, &sqb);                       /* I-1 */
        double sq = orc_f16_to_f64(sqb);
        double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double smax = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            int64_t row = (pos_off[b] + t) * Hkv + h;
            double acc = 0.0;
            if (orc_is_protected(t, n, S, R)) {                    /* I-3 */
                int64_t I = 0;
                for (int c = 0; c < d; ++c) I += (int64_t)qi[c] * (int64_t)k8[row * d + c];
                acc = orc_f16_to_f64(k8s[row]) * (double)I;
            } else {                                               /* I-2 */
                for (int g = 0; g < ng; ++g) {
                    int64_t I = 0, Q = 0;
                    for (int c = g * G; c < (g + 1) * G; ++c) {
                        I += (int64_t)qi[c] * (int64_t)k4[row * d + c];
                        Q += qi[c];
                    }
                    acc += orc_f16_to_f64(k4d[row * ng + g]) * (double)I +
                           orc_f16_to_f64(k4m[row * ng + g]) * (double)Q;
                }
            }
            p[t] = sm_scale * sq * acc;
            if (p[t] > smax) smax = p[t];
        }
        double den = 0.0;                                          /* I-4 */
        for (int64_t t = 0; t < n; ++t) { p[t] = exp(p[t] - smax); den += p[t]; }
        for (int c = 0; c < d; ++c) { o[c] = 0.0; bd[c] = 0.0; }
        for (int64_t t = 0; t < n; ++t) {                          /* I-6, protected */
            if (!orc_is_protected(t, n, S, R)) continue;
            int64_t row = (pos_off[b] + t) * Hkv + h;
            double sv = orc_f16_to_f64(v8s[row]);
            for (int c = 0; c < d; ++c) o[c] += p[t] * (sv * (double)v8[row * d + c]);
        }
        for (int64_t t0 = 0; t0 < n; t0 += 8) {                    /* I-5, I-6, INT4 blocks */
            int64_t t1 = t0 + 8 < n ? t0 + 8 : n;
            for (int g = 0; g < ng; ++g) {
                double wmax = 0.0;
                for (int64_t t = t0; t < t1; ++t) {
                    if (orc_is_protected(t, n, S, R)) continue;
                    int64_t row = (pos_off[b] + t) * Hkv + h;
                    double w = p[t] * orc_f16_to_f64(v4d[row * ng + g]);
                    if (w > wmax) wmax = w;
                }
                double sigma = wmax / 255.0;
                for (int64_t t = t0; t < t1; ++t) {
                    if (orc_is_protected(t, n, S, R)) continue;
                    int64_t row = (pos_off[b] + t) * Hkv + h;
                    double u = 0.0;
                    int near = 0;
                    if (sigma > 0.0) {
                        double x = p[t] * orc_f16_to_f64(v4d[row * ng + g]) / sigma;
                        u = rint(x);
                        near = fabs(x - floor(x) - 0.5) < eps;
                    }
                    double mv = orc_f16_to_f64(v4m[row * ng + g]);
                    for (int c = g * G; c < (g + 1) * G; ++c) {
                        o[c] += sigma * u * (double)v4[row * d + c] + p[t] * mv;
                        if (near) bd[c] += sigma * (double)v4[row * d + c];
                    }
                }
            }
        }
        for (int c = 0; c < d; ++c) { o[c] /= den; bd[c] /= den; }
        free(p);
        free(qi);
    }
}

/* ------------------------------------------------------------------------ */
/* Prefill attention (KV4-RL Appendix A.3, "Protected path and              */
/* reconstruction": prefill and carried-prefix reconstruction run BF16      */
/* attention over the newly computed K/V), in binary64.                     */
/* ------------------------------------------------------------------------ */

/*
 * Reading P-1: causal softmax attention of every position i of a sequence over
 * the positions [0, i] of the same sequence, on the bf16 source values (no
 * quantization).  Sequences are packed: sequence b owns rows [cu[b], cu[b+1])
 * of q [T][Hq][d] and of k, v [T][Hkv][d]; q head j reads kv head j/(Hq/Hkv);
 * out is [T][Hq][d].
 */
void orc_prefill_attn(int B, const int32_t* cu, int Hq, int Hkv, int d, double sm_scale,
                      const float* q, const float* k, const float* v, double* out)
{
    int gqa = Hq / Hkv;
    int64_t T = cu[B];
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t tj = 0; tj < T * Hq; ++tj) {
        int64_t t = tj / Hq;
        int j = (int)(tj % Hq), h = j / gqa;
        int b = 0;
        while (cu[b + 1] <= t) ++b;
        int64_t t0 = cu[b];
        const float* qt = q + (t * Hq + j) * d;
        double* o = out + (t * Hq + j) * d;
        int64_t m = t - t0 + 1;                       /* positions [t0, t] */
        double* s = (double*)malloc(sizeof(double) * (size_t)m);
        double smax = -INFINITY;
        for (int64_t p = 0; p < m; ++p) {
            const float* kp = k + ((t0 + p) * Hkv + h) * d;
            double dot = 0.0;
            for (int c = 0; c < d; ++c) dot += (double)qt[c] * (double)kp[c];
            s[p] = sm_scale * dot;
            if (s[p] > smax) smax = s[p];
        }
        double den = 0.0;
        for (int64_t p = 0; p < m; ++p) { s[p] = exp(s[p] - smax); den += s[p]; }
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t p = 0; p < m; ++p) {
            const float* vp = v + ((t0 + p) * Hkv + h) * d;
            double w = s[p] / den;
            for (int c = 0; c < d; ++c) o[c] += w * (double)vp[c];
        }
        free(s);
    }
}

/* Number of OpenMP threads a parallel region will use (for reporting). */
int orc_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp master
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
