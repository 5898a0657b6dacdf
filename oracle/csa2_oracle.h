/*
 * csa2_oracle.h -- plain CPU oracle for the CSA2 compressed-sparse-attention
 * decode path with FP4 (E2M1) global KV.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant with the GPU library.
 *
 * Everything is computed in double precision from the plain definitions.
 * Pages cited (by address and section):
 *   [P1] helmcode.com/deepseek-v41-flash
 *   [P4] louisbouchard.ai/deepseek-v41-flash-kv-cache-writing-benchmark
 *   [P5] 0x0moeen.in/writes/deepseek-v4-1-flash-kv-cache
 */
#ifndef CSA2_ORACLE_H
#define CSA2_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Real value of a 4-bit E2M1 code (sign, 2 exponent bits with bias 1,
 * 1 mantissa bit).  [P1 §04 FP4]: global KV elements are E2M1. */
double csa2o_e2m1_value(int code);

/* Real value of an E4M3 byte in the "FN" variant (bias 7, no infinities,
 * 0x7F/0xFF are NaN).  [P1 §04 FP4]: one E4M3 scale per 16 channels. */
double csa2o_e4m3_value(int byte);

/* Scale byte for a 16-channel block whose largest magnitude is amax:
 * the E4M3 value nearest to the real number amax/6, ties to the even
 * mantissa, saturating at 448.  Found by exhaustive search over the 127
 * non-negative finite E4M3 values. */
int csa2o_scale_byte(double amax);

/* 4-bit code for element x under block scale s (s >= 0): the E2M1 grid
 * value g*s nearest to |x| (ties to even code), sign bit = sign bit of x.
 * s == 0 gives magnitude 0.  Found by exhaustive search over the 8 grid
 * magnitudes. */
int csa2o_e2m1_code(double x, double s);

/* Quantize `rows` rows of `dim` fp32 values (dim % 16 == 0, even channel
 * in the low nibble).  codes: [rows][dim/2], scales: [rows][dim/16]. */
void csa2o_quantize_rows(const float* x, int64_t rows, int32_t dim,
                         uint8_t* codes, uint8_t* scales);

/* Dequantize rows: out[r][c] = e2m1(code) * e4m3(scale of block c/16). */
void csa2o_dequant_rows(const uint8_t* codes, const uint8_t* scales,
                        int64_t rows, int32_t dim, double* out);

/* Indexer score of the listed cache rows (one query):
 *   score = sum_h w[h] * max(0, q[h] . k_row)
 * q: [H][dim] (values of the bf16 query, as fp32), w: [H].
 * rows: [n] row numbers into codes/scales (one sequence's cache). */
void csa2o_index_score(const uint8_t* codes, const uint8_t* scales,
                       int32_t dim, const float* q, const float* w,
                       int32_t H, const int64_t* rows, int64_t n,
                       double* out);

/* Top-k of score[0..n_valid): order by score descending, then slot
 * ascending; keep the first min(k, n_valid); map each slot through
 * slot_pos (if not NULL); write them ascending to out[0..k) and pad the
 * rest with -1.  Returns the number of valid entries written. */
int32_t csa2o_topk(const double* score, int64_t n_valid, int32_t k,
                   const int32_t* slot_pos, int32_t* out);

/* Sparse attention of one query token.
 *   q: [H][D] (bf16 values as fp32); the main cache rows idx[0..K)
 *   (entries < 0 skipped) are dequantized FP4 rows; swa: [S][D] E4M3
 *   bytes times swa_scale are the window rows (all S are visible).
 *   One softmax over the union: logit = sm_scale * q_h . k, value = the
 *   first dv channels of the same row.
 *   out: [H][dv], lse: [H] (natural log).  No entries: out = 0, lse = -inf. */
void csa2o_sparse_attn(const float* q, int32_t H, int32_t D, int32_t dv,
                       const uint8_t* codes, const uint8_t* scales,
                       const int32_t* idx, int32_t K,
                       const uint8_t* swa, double swa_scale, int32_t S,
                       double sm_scale, double* out, double* lse);

/* Number of OpenMP threads the oracle uses (1 when built without OpenMP). */
int32_t csa2o_num_threads(void);
/* Threads for the oracle's later parallel loops (n >= 1). */
void csa2o_set_num_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
