/*
 * oracle.c -- plain CPU definition of the softcapped-routing fused FP8 MoE forward.
 * TEST INFRASTRUCTURE ONLY (see oracle.h for the page keys [FMF8], [H200], [WEAVE] and the
 * list of results whose parity is unpinned).  Single-threaded, no blocking, no fusion.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define QBLK 128 /* [FMF8] problem table: 128-wide FP8 quantisation blocks */

/* ------------------------------------------------------------------------------------ */
/* Number formats                                                                       */
/* ------------------------------------------------------------------------------------ */

/* E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field 0 holds the
 * subnormals m * 2^-9; 0x7F and 0xFF are NaN, so the largest finite magnitude is
 * 1.75 * 2^8 = 448. */
double orc_e4m3_value(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return s ? -mag : mag;
}

uint8_t orc_e4m3_encode(float y) {
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a >= 448.0) return sign | 0x7E;              /* saturate, never NaN */
    if (a < ldexp(1.0, -6)) {                        /* subnormal spacing 2^-9 */
        double q = nearbyint(a * 512.0);             /* exact scaling; ties to even */
        return sign | (uint8_t)q;                    /* q == 8 is code 0x08 = 2^-6 */
    }
    int ex;
    frexp(a, &ex);                                   /* a in [2^(ex-1), 2^ex) */
    int E = ex - 1;                                  /* unbiased exponent, -6..8 */
    double q = nearbyint(ldexp(a, 3 - E));           /* significand * 8, in [8, 16] */
    if (q == 16.0) { q = 8.0; E += 1; }
    return sign | (uint8_t)(((E + 7) << 3) | (int)(q - 8.0));
}

uint8_t orc_e4m3_encode_bruteforce(float y) {
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3_value((uint8_t)c) - a);
        /* strictly closer wins; on an exact tie prefer the code with an even mantissa */
        if (d < bestd || (d == bestd && (c & 1) == 0)) { bestd = d; best = c; }
    }
    return sign | (uint8_t)best;
}

/* bfloat16 keeps 8 significant bits and fp32's exponent range (subnormal spacing 2^-133). */
uint16_t orc_bf16_from_double(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int qexp = (ex - 1) - 7;                         /* spacing of 8-bit significands */
    if (qexp < -133) qexp = -133;
    double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
    float f = (float)r;                              /* exact, or +inf on overflow */
    if (r > 0x1.FEp127) f = INFINITY;
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return sign | (uint16_t)(bits >> 16);
}

double orc_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------------------ */
/* [FMF8] Baseline kernel 1: softmax with softcapping (tanh), then top-k                */
/* ------------------------------------------------------------------------------------ */

int orc_route(const float* logits, int M, int E, int k, float cap, int32_t* ids,
              float* weights) {
    if (!logits || !ids || !weights || M < 0 || E < 1 || k < 1 || k > E) return -1;
    char* taken = (char*)malloc((size_t)E);
    double* c = (double*)malloc(sizeof(double) * (size_t)k);
    if (!taken || !c) { free(taken); free(c); return -1; }
    for (int t = 0; t < M; ++t) {
        const float* row = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        /* Selection by the raw logit: softcap and softmax are strictly increasing maps, so
         * the top-k of the probabilities is the top-k of the logits.  Repeated argmax with
         * a strict comparison keeps the lowest index among equal values (and -0 == +0).
         * The pages say nothing of non-finite logits; a NaN is taken to rank below every
         * number, so it is chosen only when fewer than k numbers remain, lowest index first. */
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || (!isnan(row[e]) && (isnan(row[best]) || row[e] > row[best])))
                    best = e;
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        for (int j = 0; j < k; ++j) {
            double l = (double)row[ids[(size_t)t * k + j]];
            c[j] = (cap > 0.0f) ? (double)cap * tanh(l / (double)cap) : l;
        }
        /* softmax over all E experts restricted to the selected k and renormalised is the
         * softmax over the k selected capped logits. */
        double s = 0.0;
        for (int j = 0; j < k; ++j) s += exp(c[j] - c[0]);
        for (int j = 0; j < k; ++j) weights[(size_t)t * k + j] = (float)(exp(c[j] - c[0]) / s);
    }
    free(taken);
    free(c);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* [FMF8] Baseline kernels 2-3: per-expert counts and exclusive prefix sum              */
/* ------------------------------------------------------------------------------------ */

int orc_layout(const int32_t* ids, int M, int k, int E, int32_t* counts, int32_t* offsets) {
    if (!ids || !counts || !offsets || M < 0 || k < 1 || E < 1) return -1;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long r = 0; r < (long)M * k; ++r) {
        int e = ids[r];
        if (e < 0 || e >= E) return -1;
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    return 0;
}

int orc_tasks(const int32_t* counts, const int32_t* offsets, int E, int n_blocks,
              int chunk_rows, int32_t* tasks, int max_tasks) {
    if (!counts || !offsets || !tasks || E < 1 || n_blocks < 1 || chunk_rows < 1) return -1;
    int n = 0;
    for (int e = 0; e < E; ++e) {
        for (int rb = 0; rb < counts[e]; rb += chunk_rows) {
            int cnt = counts[e] - rb < chunk_rows ? counts[e] - rb : chunk_rows;
            for (int nb = 0; nb < n_blocks; ++nb) {
                if (n >= max_tasks) return -1;
                tasks[4 * n + 0] = e;
                tasks[4 * n + 1] = offsets[e] + rb;
                tasks[4 * n + 2] = cnt;
                tasks[4 * n + 3] = nb;
                ++n;
            }
        }
    }
    return n;
}

/* ------------------------------------------------------------------------------------ */
/* [FMF8] Baseline kernel 4 / Fusion 2 (QSG): scale = amax/448, value * (1/scale)       */
/* ------------------------------------------------------------------------------------ */

/* One quantisation block of `count` values (128 for activations, 128*128 for weights).
 * Written with explicit fp32 operations: the scale is the fp32 quotient amax/448, the multiplier its
 * fp32 reciprocal, and each value is multiplied in fp32 before encoding. */
static void quant_block(const float* vals, int count, uint8_t* codes, float* scale_out) {
    float amax = 0.0f;
    for (int i = 0; i < count; ++i) {
        float a = fabsf(vals[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {                              /* all zeros: keep only the signs */
        *scale_out = 0.0f;
        for (int i = 0; i < count; ++i) codes[i] = signbit(vals[i]) ? 0x80 : 0x00;
        return;
    }
    float scale = amax / 448.0f;                     /* fp32 quotient, correctly rounded */
    float inv = 1.0f / scale;                        /* fp32 reciprocal, correctly rounded */
    *scale_out = scale;
    for (int i = 0; i < count; ++i) {
        float y = vals[i] * inv;                     /* fp32 product */
        codes[i] = orc_e4m3_encode(y);
    }
}

int orc_quant_act(const uint16_t* x, int M, int K, uint8_t* q, float* scales) {
    if (!x || !q || !scales || M < 0 || K < QBLK || K % QBLK) return -1;
    int Kb = K / QBLK;
    float vals[QBLK];
    uint8_t codes[QBLK];
    for (int t = 0; t < M; ++t) {
        for (int b = 0; b < Kb; ++b) {
            for (int i = 0; i < QBLK; ++i)
                vals[i] = (float)orc_bf16_value(x[(size_t)t * K + b * QBLK + i]);
            quant_block(vals, QBLK, codes, &scales[(size_t)t * Kb + b]);
            memcpy(q + (size_t)t * K + b * QBLK, codes, QBLK);
        }
    }
    return 0;
}

int orc_quant_weights(const float* w, int E, int N, int K, uint8_t* q, float* scales) {
    if (!w || !q || !scales || E < 1 || N % QBLK || K % QBLK || N < QBLK || K < QBLK) return -1;
    int Nb = N / QBLK, Kb = K / QBLK;
    float* vals = (float*)malloc(sizeof(float) * QBLK * QBLK);
    uint8_t* codes = (uint8_t*)malloc(QBLK * QBLK);
    if (!vals || !codes) { free(vals); free(codes); return -1; }
    for (int e = 0; e < E; ++e)
        for (int nb = 0; nb < Nb; ++nb)
            for (int b = 0; b < Kb; ++b) {
                for (int i = 0; i < QBLK; ++i)
                    for (int j = 0; j < QBLK; ++j)
                        vals[i * QBLK + j] =
                            w[((size_t)e * N + nb * QBLK + i) * K + b * QBLK + j];
                quant_block(vals, QBLK * QBLK, codes,
                            &scales[((size_t)e * Nb + nb) * Kb + b]);
                for (int i = 0; i < QBLK; ++i)
                    memcpy(q + ((size_t)e * N + nb * QBLK + i) * K + b * QBLK,
                           codes + i * QBLK, QBLK);
            }
    free(vals);
    free(codes);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* [FMF8] Baseline kernel 5: sort & gather into expert-contiguous rows                  */
/* ------------------------------------------------------------------------------------ */

int orc_sort_gather(const int32_t* ids, int M, int k, int E, const int32_t* offsets,
                    const uint8_t* q, const float* scales, int K, int32_t* sorted_route_ids,
                    uint8_t* a_q, float* a_scales) {
    if (!ids || !offsets || !q || !scales || !sorted_route_ids || !a_q || !a_scales ||
        M < 0 || k < 1 || E < 1 || K % QBLK)
        return -1;
    int Kb = K / QBLK;
    long R = (long)M * k;
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!cursor) return -1;
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (long r = 0; r < R; ++r) {
        int e = ids[r];
        long slot = cursor[e]++;
        long t = r / k;
        sorted_route_ids[slot] = (int32_t)r;
        memcpy(a_q + slot * K, q + t * K, (size_t)K);
        for (int b = 0; b < Kb; ++b) a_scales[b * R + slot] = scales[t * Kb + b];
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* [FMF8] Baseline kernel 6: grouped GEMM with per-K-block scaling                      */
/* ------------------------------------------------------------------------------------ */

int orc_gemm_fp8(const uint8_t* a_q, const float* a_scales, int rows, const uint8_t* w_q,
                 const float* w_scales, const int32_t* offsets, int E, int N, int K,
                 double* C) {
    if (!a_q || !a_scales || !w_q || !w_scales || !offsets || !C || rows < 0 || E < 1 ||
        N % QBLK || K % QBLK)
        return -1;
    int Nb = N / QBLK, Kb = K / QBLK;
    double dq[256];
    for (int c = 0; c < 256; ++c) dq[c] = orc_e4m3_value((uint8_t)c);
    for (int e = 0; e < E; ++e) {
        for (long r = offsets[e]; r < offsets[e + 1]; ++r) {
            const uint8_t* a = a_q + r * K;
            for (int n = 0; n < N; ++n) {
                const uint8_t* w = w_q + ((size_t)e * N + n) * K;
                double acc = 0.0;
                for (int b = 0; b < Kb; ++b) {
                    /* products of two E4M3 values have at most 8 significant bits and lie in
                     * [2^-18, 2^18); 128 of them add up exactly in double. */
                    double bs = 0.0;
                    for (int i = b * QBLK; i < (b + 1) * QBLK; ++i) bs += dq[a[i]] * dq[w[i]];
                    double sa = a_scales[(size_t)b * rows + r];
                    double sb = w_scales[((size_t)e * Nb + n / QBLK) * Kb + b];
                    acc += bs * sa * sb;
                }
                C[r * N + n] = acc;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* [FMF8] Baseline kernel 7: routing-weighted scatter-add                               */
/* ------------------------------------------------------------------------------------ */

int orc_scatter(const double* C, const int32_t* sorted_route_ids, int rows,
                const float* weights, int M, int k, int N, double* y64, uint16_t* y) {
    if (!C || !sorted_route_ids || !weights || !y || M < 0 || k < 1 || N < 1) return -1;
    double* acc = (double*)calloc((size_t)M * N, sizeof(double));
    if (!acc) return -1;
    for (long s = 0; s < rows; ++s) {
        long r = sorted_route_ids[s];
        long t = r / k;
        double w = weights[r];
        for (int n = 0; n < N; ++n) acc[t * N + n] += w * C[s * N + n];
    }
    for (long i = 0; i < (long)M * N; ++i) {
        y[i] = orc_bf16_from_double(acc[i]);
        if (y64) y64[i] = acc[i];
    }
    free(acc);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Whole forward, in the pages' stage order                                             */
/* ------------------------------------------------------------------------------------ */

int orc_forward(const float* logits, const uint16_t* x, const uint8_t* w_q,
                const float* w_scales, int M, int E, int k, int K, int N, float cap,
                uint16_t* y, double* y64, int32_t* ids_out, float* weights_out,
                int32_t* counts_out, int32_t* offsets_out, int32_t* sorted_out,
                uint8_t* a_q_out, float* a_scales_out, double* C_out) {
    if (!logits || !x || !w_q || !w_scales || !y || M < 1 || E < 1 || k < 1 || k > E ||
        K % QBLK || N % QBLK || K < QBLK || N < QBLK)
        return -1;
    long R = (long)M * k;
    int Kb = K / QBLK;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * R);
    float* wts = (float*)malloc(sizeof(float) * R);
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (E + 1));
    uint8_t* q = (uint8_t*)malloc((size_t)M * K);
    float* qs = (float*)malloc(sizeof(float) * (size_t)M * Kb);
    int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * R);
    uint8_t* a_q = (uint8_t*)malloc((size_t)R * K);
    float* a_s = (float*)malloc(sizeof(float) * (size_t)R * Kb);
    double* C = (double*)malloc(sizeof(double) * (size_t)R * N);
    int rc = -1;
    if (!ids || !wts || !counts || !offsets || !q || !qs || !sorted || !a_q || !a_s || !C)
        goto done;
    if (orc_route(logits, M, E, k, cap, ids, wts)) goto done;
    if (orc_layout(ids, M, k, E, counts, offsets)) goto done;
    if (orc_quant_act(x, M, K, q, qs)) goto done;
    if (orc_sort_gather(ids, M, k, E, offsets, q, qs, K, sorted, a_q, a_s)) goto done;
    if (orc_gemm_fp8(a_q, a_s, (int)R, w_q, w_scales, offsets, E, N, K, C)) goto done;
    if (orc_scatter(C, sorted, (int)R, wts, M, k, N, y64, y)) goto done;
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * R);
    if (weights_out) memcpy(weights_out, wts, sizeof(float) * R);
    if (counts_out) memcpy(counts_out, counts, sizeof(int32_t) * E);
    if (offsets_out) memcpy(offsets_out, offsets, sizeof(int32_t) * (E + 1));
    if (sorted_out) memcpy(sorted_out, sorted, sizeof(int32_t) * R);
    if (a_q_out) memcpy(a_q_out, a_q, (size_t)R * K);
    if (a_scales_out) memcpy(a_scales_out, a_s, sizeof(float) * (size_t)R * Kb);
    if (C_out) memcpy(C_out, C, sizeof(double) * (size_t)R * N);
    rc = 0;
done:
    free(ids); free(wts); free(counts); free(offsets); free(q); free(qs);
    free(sorted); free(a_q); free(a_s); free(C);
    return rc;
}

int orc_forward_tokens(const float* logits, const uint16_t* x, const uint8_t* w_q,
                       const float* w_scales, int M, int E, int k, int K, int N, float cap,
                       const int32_t* tokens, int ntok, uint16_t* y, double* y64) {
    if (!logits || !x || !w_q || !w_scales || !tokens || !y || M < 1 || E < 1 || k < 1 ||
        k > E || K % QBLK || N % QBLK || ntok < 0)
        return -1;
    int Kb = K / QBLK, Nb = N / QBLK;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * k);
    float* wts = (float*)malloc(sizeof(float) * k);
    uint8_t* q = (uint8_t*)malloc((size_t)K);
    float* qs = (float*)malloc(sizeof(float) * Kb);
    double* acc = (double*)malloc(sizeof(double) * N);
    double dq[256];
    int rc = -1;
    if (!ids || !wts || !q || !qs || !acc) goto done;
    for (int c = 0; c < 256; ++c) dq[c] = orc_e4m3_value((uint8_t)c);
    for (int i = 0; i < ntok; ++i) {
        int t = tokens[i];
        if (t < 0 || t >= M) goto done;
        if (orc_route(logits + (size_t)t * E, 1, E, k, cap, ids, wts)) goto done;
        if (orc_quant_act(x + (size_t)t * K, 1, K, q, qs)) goto done;
        for (int n = 0; n < N; ++n) acc[n] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[j];
            for (int n = 0; n < N; ++n) {
                const uint8_t* w = w_q + ((size_t)e * N + n) * K;
                double c = 0.0;
                for (int b = 0; b < Kb; ++b) {
                    double bs = 0.0;
                    for (int kk = b * QBLK; kk < (b + 1) * QBLK; ++kk) bs += dq[q[kk]] * dq[w[kk]];
                    c += bs * (double)qs[b] * (double)w_scales[((size_t)e * Nb + n / QBLK) * Kb + b];
                }
                acc[n] += (double)wts[j] * c;
            }
        }
        for (int n = 0; n < N; ++n) {
            y[(size_t)i * N + n] = orc_bf16_from_double(acc[n]);
            if (y64) y64[(size_t)i * N + n] = acc[n];
        }
    }
    rc = 0;
done:
    free(ids); free(wts); free(q); free(qs); free(acc);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* [H200] BF16 grouped GEMM on compact expert rows                                      */
/* ------------------------------------------------------------------------------------ */

int orc_gemm_bf16(const uint16_t* A, int rows, int K, const uint16_t* W, int N,
                  const int32_t* offsets, int E, const int32_t* rows_list, int nlist,
                  uint16_t* out, double* out64) {
    if (!A || !W || !offsets || !out || rows < 0 || K < 1 || N < 1 || E < 1) return -1;
    int n_out = rows_list ? nlist : rows;
    for (int i = 0; i < n_out; ++i) {
        long r = rows_list ? rows_list[i] : i;
        if (r < 0 || r >= rows) return -1;
        int e = -1;
        for (int g = 0; g < E; ++g)
            if (r >= offsets[g] && r < offsets[g + 1]) { e = g; break; }
        if (e < 0) return -1;
        const uint16_t* a = A + r * K;
        for (int n = 0; n < N; ++n) {
            const uint16_t* w = W + ((size_t)e * N + n) * K;
            double acc = 0.0;
            for (int kk = 0; kk < K; ++kk) acc += orc_bf16_value(a[kk]) * orc_bf16_value(w[kk]);
            out[(size_t)i * N + n] = orc_bf16_from_double(acc);
            if (out64) out64[(size_t)i * N + n] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* [WEAVE] section 3.1: the gate (router projection) counted in the layer's forward      */
/* ------------------------------------------------------------------------------------ */

/* logits[t][e] = fp32( sum_h x[t][h] * w_gate[e][h] ): bf16 operands, every product and the
 * sum in double, one rounding to fp32 (logits64, optional, keeps the double sums). */
int orc_router_logits(const uint16_t* x, int M, int H, const uint16_t* w_gate, int E,
                      float* logits, double* logits64) {
    if (!x || !w_gate || !logits || M < 0 || H < 1 || E < 1) return -1;
    for (long t = 0; t < M; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += orc_bf16_value(x[t * H + h]) * orc_bf16_value(w_gate[(size_t)e * H + h]);
            logits[t * E + e] = (float)acc;
            if (logits64) logits64[t * E + e] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* [WEAVE] Mixtral-like layer: route, per-route expert FFN with SiLU gating, combine    */
/* ------------------------------------------------------------------------------------ */

int orc_ffn_tokens(const float* logits, const uint16_t* x, const uint16_t* w_up,
                   const uint16_t* w_down, int M, int E, int k, int H, int F, float cap,
                   const int32_t* tokens, int ntok, uint16_t* y, double* y64) {
    if (!logits || !x || !w_up || !w_down || !y || M < 1 || E < 1 || k < 1 || k > E ||
        H < 1 || F < 1)
        return -1;
    int n_out = tokens ? ntok : M;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * k);
    float* wts = (float*)malloc(sizeof(float) * k);
    double* h = (double*)malloc(sizeof(double) * 2 * (size_t)F);
    double* act = (double*)malloc(sizeof(double) * (size_t)F);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    int rc = -1;
    if (!ids || !wts || !h || !act || !acc) goto done;
    for (int i = 0; i < n_out; ++i) {
        int t = tokens ? tokens[i] : i;
        if (t < 0 || t >= M) goto done;
        if (orc_route(logits + (size_t)t * E, 1, E, k, cap, ids, wts)) goto done;
        const uint16_t* xt = x + (size_t)t * H;
        for (int n = 0; n < H; ++n) acc[n] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[j];
            for (int f = 0; f < 2 * F; ++f) {
                const uint16_t* w = w_up + ((size_t)e * 2 * F + f) * H;
                double s = 0.0;
                for (int kk = 0; kk < H; ++kk) s += orc_bf16_value(xt[kk]) * orc_bf16_value(w[kk]);
                h[f] = s;
            }
            for (int f = 0; f < F; ++f) {
                double g = h[f], u = h[F + f];
                double silu = g / (1.0 + exp(-g));
                act[f] = orc_bf16_value(orc_bf16_from_double(silu * u));
            }
            for (int n = 0; n < H; ++n) {
                const uint16_t* w = w_down + ((size_t)e * H + n) * F;
                double s = 0.0;
                for (int f = 0; f < F; ++f) s += act[f] * orc_bf16_value(w[f]);
                acc[n] += (double)wts[j] * s;
            }
        }
        for (int n = 0; n < H; ++n) {
            y[(size_t)i * H + n] = orc_bf16_from_double(acc[n]);
            if (y64) y64[(size_t)i * H + n] = acc[n];
        }
    }
    rc = 0;
done:
    free(ids); free(wts); free(h); free(act); free(acc);
    return rc;
}

/* ------------------------------------------------------------------------------------ */
/* [FMF8] comparison section, "vLLM full MLP" reference: gate+up, SiLU, down in FP8     */
/* ------------------------------------------------------------------------------------ */

int orc_swiglu_f32(const double* h, int rows, int I, float* act) {
    if (!h || !act || rows < 0 || I < 1) return -1;
    for (long r = 0; r < rows; ++r)
        for (int f = 0; f < I; ++f) {
            double g = h[r * 2 * I + f], u = h[r * 2 * I + I + f];
            act[r * I + f] = (float)(g / (1.0 + exp(-g)) * u);
        }
    return 0;
}

int orc_quant_rows_f32(const float* v, int rows, int K, uint8_t* q, float* scales) {
    if (!v || !q || !scales || rows < 0 || K < QBLK || K % QBLK) return -1;
    int Kb = K / QBLK;
    for (long r = 0; r < rows; ++r)
        for (int b = 0; b < Kb; ++b)
            quant_block(v + r * K + b * QBLK, QBLK, q + r * K + b * QBLK, &scales[r * Kb + b]);
    return 0;
}

/* one row of the block-scaled FP8 GEMM: out[n] = sum_b sa[b] * sw[e][n/128][b] *
 * sum_{i in block b} e4m3(a[i]) * e4m3(w[e][n][i]) */
static void gemm_fp8_row(const double* dq, const uint8_t* a, const float* sa,
                         const uint8_t* w, const float* sw, int e, int N, int K, double* out) {
    int Nb = N / QBLK, Kb = K / QBLK;
    for (int n = 0; n < N; ++n) {
        const uint8_t* wr = w + ((size_t)e * N + n) * K;
        double c = 0.0;
        for (int b = 0; b < Kb; ++b) {
            double bs = 0.0;
            for (int i = b * QBLK; i < (b + 1) * QBLK; ++i) bs += dq[a[i]] * dq[wr[i]];
            c += bs * (double)sa[b] * (double)sw[((size_t)e * Nb + n / QBLK) * Kb + b];
        }
        out[n] = c;
    }
}

int orc_mlp_tokens(const float* logits, const uint16_t* x, const uint8_t* w1_q,
                   const float* w1_scales, const uint8_t* w2_q, const float* w2_scales,
                   int M, int E, int k, int H, int I, float cap, const int32_t* tokens,
                   int ntok, uint16_t* y, double* y64) {
    if (!logits || !x || !w1_q || !w1_scales || !w2_q || !w2_scales || !y || M < 1 || E < 1 ||
        k < 1 || k > E || H < QBLK || H % QBLK || I < QBLK || I % QBLK || ntok < 0)
        return -1;
    int n_out = tokens ? ntok : M;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * k);
    float* wts = (float*)malloc(sizeof(float) * k);
    uint8_t* xq = (uint8_t*)malloc((size_t)H);
    float* xs = (float*)malloc(sizeof(float) * (H / QBLK));
    double* h1 = (double*)malloc(sizeof(double) * 2 * (size_t)I);
    float* act = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* aq = (uint8_t*)malloc((size_t)I);
    float* as = (float*)malloc(sizeof(float) * (I / QBLK));
    double* h2 = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    double dq[256];
    int rc = -1;
    if (!ids || !wts || !xq || !xs || !h1 || !act || !aq || !as || !h2 || !acc) goto done;
    for (int c = 0; c < 256; ++c) dq[c] = orc_e4m3_value((uint8_t)c);
    for (int i = 0; i < n_out; ++i) {
        int t = tokens ? tokens[i] : i;
        if (t < 0 || t >= M) goto done;
        if (orc_route(logits + (size_t)t * E, 1, E, k, cap, ids, wts)) goto done;
        if (orc_quant_act(x + (size_t)t * H, 1, H, xq, xs)) goto done;
        for (int n = 0; n < H; ++n) acc[n] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = ids[j];
            gemm_fp8_row(dq, xq, xs, w1_q, w1_scales, e, 2 * I, H, h1);
            if (orc_swiglu_f32(h1, 1, I, act)) goto done;
            if (orc_quant_rows_f32(act, 1, I, aq, as)) goto done;
            gemm_fp8_row(dq, aq, as, w2_q, w2_scales, e, H, I, h2);
            for (int n = 0; n < H; ++n) acc[n] += (double)wts[j] * h2[n];
        }
        for (int n = 0; n < H; ++n) {
            y[(size_t)i * H + n] = orc_bf16_from_double(acc[n]);
            if (y64) y64[(size_t)i * H + n] = acc[n];
        }
    }
    rc = 0;
done:
    free(ids); free(wts); free(xq); free(xs); free(h1); free(act); free(aq); free(as);
    free(h2); free(acc);
    return rc;
}
