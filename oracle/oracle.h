/*
 * oracle.h -- plain, slow, single-threaded CPU definition of the softcapped-routing
 * fused FP8 MoE forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls this
 * code: only the test suite, the package's smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or constant with the HIP library.
 *
 * Pages cited (by title; sections named as printed on the page):
 *   [FMF8]  "Fused MoE FP8: 8.09 -> 13.18 TFLOPS (1.63x)" (Croqtile tutorial)
 *   [H200]  "H200 MoE Grouped GEMM: routed-row accounting, online replay and SM90 tuning"
 *   [WEAVE] repost blog on the "Weave" paper (fine-grained dynamic SM scheduling for MoE)
 *
 * Arithmetic: every floating-point result is formed in IEEE double and rounded only where
 * the path stores a narrower type (fp32 routing weights and scales, E4M3 codes, BF16
 * outputs).  The FP8 quantiser follows the stated fp32 steps exactly (amax/448 and the
 * reciprocal are fp32 operations) because its codes are compared bit for bit.
 *
 * Parity unpinned (covered by tolerance or canonicalisation, not by exact pins):
 *   - the last-ulp fp32 values of the routing weights (tanh/exp implementations differ);
 *   - the summation order of fp32 accumulations on the device;
 *   - the order of rows inside one expert segment (slots come from atomics).
 *
 * All functions return 0 on success and -1 on invalid arguments.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ---------------------------------------------------------------- */
/* OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF are NaN, max finite 448). */
double  orc_e4m3_value(uint8_t code);
/* Round-to-nearest-even encoding; |y| >= 448 saturates to 0x7E|sign; underflow keeps the
 * sign (so -0.0 and tiny negatives give 0x80); NaN gives 0x7F (outside the domain). */
uint8_t orc_e4m3_encode(float y);
/* Same value by exhaustive nearest search over all 127 non-negative finite codes (ties
 * to the even code).  Used only by the oracle's own self-checks. */
uint8_t orc_e4m3_encode_bruteforce(float y);
/* Round an IEEE double to bfloat16 (round to nearest, ties to even). */
uint16_t orc_bf16_from_double(double v);
double   orc_bf16_value(uint16_t bits);

/* ---- [FMF8] Baseline kernel 1 (Route): softcapped softmax + top-k ------------------ */
/* ids[t*k+j]: the k experts with the largest raw logit, ties to the lower index, in
 * descending order.  weights[t*k+j] = softmax over the selected capped logits
 * c = cap*tanh(l/cap) (cap <= 0: c = l), i.e. renormalised to sum 1. */
int orc_route(const float* logits, int M, int E, int k, float cap,
              int32_t* ids, float* weights);

/* ---- [FMF8] Baseline kernels 2-3 (Count Experts, Build Layout) --------------------- */
/* counts[e] = #routes to e; offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e]
 * (offsets has E+1 entries, so offsets[E] = M*k). */
int orc_layout(const int32_t* ids, int M, int k, int E, int32_t* counts, int32_t* offsets);

/* ---- [WEAVE] task list: per expert, chunks of chunk_rows rows, crossed with n blocks */
/* tasks[i*4 + {0,1,2,3}] = {expert, row_begin, row_count, n_block}, in expert order.
 * Returns the number of tasks, or -1 if it would exceed max_tasks. */
int orc_tasks(const int32_t* counts, const int32_t* offsets, int E, int n_blocks,
              int chunk_rows, int32_t* tasks, int max_tasks);

/* ---- [FMF8] Baseline kernel 4 (Quantize Input): 1x128 blockwise E4M3 --------------- */
/* x: bf16 bits [M][K]; q: codes [M][K]; scales: fp32 [M][K/128]. */
int orc_quant_act(const uint16_t* x, int M, int K, uint8_t* q, float* scales);
/* 128x128 blockwise: w fp32 [E][N][K] -> codes [E][N][K], scales [E][N/128][K/128]. */
int orc_quant_weights(const float* w, int E, int N, int K, uint8_t* q, float* scales);

/* ---- [FMF8] Baseline kernel 5 (Sort & Gather) -------------------------------------- */
/* Expert e's segment [offsets[e], offsets[e+1]) lists its routes r = t*k+j in ascending
 * r.  a_q[slot] = q[t], a_scales[b*(M*k) + slot] = scales[t][b] (transposed scales). */
int orc_sort_gather(const int32_t* ids, int M, int k, int E, const int32_t* offsets,
                    const uint8_t* q, const float* scales, int K,
                    int32_t* sorted_route_ids, uint8_t* a_q, float* a_scales);

/* ---- [FMF8] Baseline kernel 6 (Grouped GEMM), block-scaled ------------------------- */
/* C[r][n] = sum_b a_scales[b][r] * w_scales[e][n/128][b] * sum_{k in block b}
 *           dq(a_q[r][k]) * dq(w_q[e][n][k])   for r in expert e's segment. */
int orc_gemm_fp8(const uint8_t* a_q, const float* a_scales, int rows,
                 const uint8_t* w_q, const float* w_scales, const int32_t* offsets,
                 int E, int N, int K, double* C);

/* ---- [FMF8] Baseline kernel 7 (Scatter to Output) ---------------------------------- */
/* y[t][n] = sum over slots s with sorted_route_ids[s]/k == t of weights[r]*C[s][n];
 * y64 (optional) keeps the double sums, y gets them rounded to bf16 once. */
int orc_scatter(const double* C, const int32_t* sorted_route_ids, int rows,
                const float* weights, int M, int k, int N, double* y64, uint16_t* y);

/* ---- whole forward: route -> layout -> quantise -> sort/gather -> GEMM -> scatter -- */
/* Optional intermediates may be NULL. */
int orc_forward(const float* logits, const uint16_t* x, const uint8_t* w_q,
                const float* w_scales, int M, int E, int k, int K, int N, float cap,
                uint16_t* y, double* y64, int32_t* ids, float* weights, int32_t* counts,
                int32_t* offsets, int32_t* sorted_route_ids, uint8_t* a_q, float* a_scales,
                double* C);

/* The same output for a list of tokens only (each token's output depends on its own
 * routes alone, so the sort/gather is a relabelling that does not change any value). */
int orc_forward_tokens(const float* logits, const uint16_t* x, const uint8_t* w_q,
                       const float* w_scales, int M, int E, int k, int K, int N, float cap,
                       const int32_t* tokens, int ntok, uint16_t* y, double* y64);

/* ---- [H200] BF16 grouped GEMM (pure GEMM on compact expert rows) ------------------- */
/* Router projection ([WEAVE] section 3.1 counts the gate in the layer): x bf16 [M][H],
 * w_gate bf16 [E][H] -> logits f32 [M][E] = fp32(sum_h x*w in double); logits64 optional. */
int orc_router_logits(const uint16_t* x, int M, int H, const uint16_t* w_gate, int E,
                      float* logits, double* logits64);

/* out[i][n] = bf16( sum_k A[r][k] * W[e(r)][n][k] ) for r = rows_list[i] (all rows when
 * rows_list is NULL); e(r) is the expert whose segment [offsets[e], offsets[e+1]) holds r. */
int orc_gemm_bf16(const uint16_t* A, int rows, int K, const uint16_t* W, int N,
                  const int32_t* offsets, int E, const int32_t* rows_list, int nlist,
                  uint16_t* out, double* out64);

/* ---- [WEAVE] Mixtral-like expert FFN layer (route, gated-up, SiLU*up, down, combine) */
/* w_up [E][2F][H] (rows 0..F-1 gate, F..2F-1 up), w_down [E][H][F].
 * act = bf16(silu(g) * u), d = act . w_down^T, y[t] = bf16(sum_j w_j d_j), for the listed
 * tokens (all when tokens is NULL). */
int orc_ffn_tokens(const float* logits, const uint16_t* x, const uint16_t* w_up,
                   const uint16_t* w_down, int M, int E, int k, int H, int F, float cap,
                   const int32_t* tokens, int ntok, uint16_t* y, double* y64);

/* ---- [FMF8] comparison section, "vLLM full MLP" reference: the expert MLP around the
 * grouped GEMM (gate+up projection, SiLU gating, down projection), here in FP8 ---------- */
/* act[r][f] = fp32(silu(g) * u) with g = h[r][f], u = h[r][I + f] and
 * silu(g) = g / (1 + e^-g), formed in double and rounded once to fp32. */
int orc_swiglu_f32(const double* h, int rows, int I, float* act);
/* The QSG quantiser on fp32 rows: per row and 128-column block, scale = fp32(amax/448),
 * code = e4m3(fp32(v * fp32(1/scale))); codes [rows][K], scales [rows][K/128]. */
int orc_quant_rows_f32(const float* v, int rows, int K, uint8_t* q, float* scales);
/* The layer for the listed tokens (all when tokens is NULL), in stage order: route; x
 * quantised per 128 (orc_quant_act); per route j of token t with expert e,
 *   h1 = the block-scaled FP8 GEMM of x_q against w1[e] [2I][H] (rows 0..I-1 gate, I..2I-1
 *        up; scales w1_scales [E][2I/128][H/128]),
 *   act = orc_swiglu_f32(h1), requantised per 128 (orc_quant_rows_f32),
 *   h2 = the block-scaled FP8 GEMM of act_q against w2[e] [H][I] (scales [E][H/128][I/128]);
 * y[t] = bf16(sum_j w_j h2_j), all sums in double. */
int orc_mlp_tokens(const float* logits, const uint16_t* x, const uint8_t* w1_q,
                   const float* w1_scales, const uint8_t* w2_q, const float* w2_scales,
                   int M, int E, int k, int H, int I, float cap, const int32_t* tokens,
                   int ntok, uint16_t* y, double* y64);

#ifdef __cplusplus
}
#endif
#endif
