/*
 * csa2.h -- C ABI of libcsa2.so: the CSA2 compressed-sparse-attention step
 * with an FP4 (E2M1) global KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The step has five parts, each an entry point below:
 *   quantize-on-write of KV rows into FP4, indexer scoring of cached
 *   positions, per-query Top-K selection (optionally through a candidate
 *   pool), sparse attention over the Top-K rows plus an FP8 sliding window,
 *   and the per-layer Full / Reindex / Reuse modes that chain them.
 *
 * Pages cited (address and section):
 *   [P1] helmcode.com/deepseek-v41-flash
 *   [P4] louisbouchard.ai/deepseek-v41-flash-kv-cache-writing-benchmark
 *   [P5] 0x0moeen.in/writes/deepseek-v4-1-flash-kv-cache
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state between calls.  Scratch memory is
 *    a caller-owned device workspace sized by the matching *_workspace_bytes
 *    query.  A workspace must be zero-filled once before its first use
 *    (csa2_workspace_init); every successful call leaves its control words
 *    zero again, so it can be reused by the next call without clearing.  One
 *    workspace must not be used by two calls that may run concurrently.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous; results are valid once the stream has been synchronised.
 *  - Every argument is checked on the host before anything is launched; an
 *    invalid argument returns an error status and launches nothing.  A HIP
 *    launch failure returns CSA2_ERR_HIP; outputs are then undefined and
 *    the workspace must be re-initialised.  csa2_last_error() gives a
 *    per-thread message for the last failure.  No C++ exception crosses
 *    this interface.
 *  - Non-finite inputs are unsupported (results unspecified).
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *
 * FP4 cache layout ([P1 §04 "FP4"]: E2M1 elements, one E4M3 scale per 16
 * channels, no extra global scale).  For a row of `dim` channels:
 *    codes  : dim/2 bytes, channel 2i in the low nibble of byte i,
 *             nibble = sign | 2 exponent bits (bias 1) | 1 mantissa bit;
 *    scales : dim/16 bytes, E4M3 ("FN": bias 7, 0x7F/0xFF NaN, max 448),
 *             scale of channels [16j, 16j+16).
 * A cache holds `cap` rows per sequence, sequences back to back:
 *    codes[B][cap][dim/2], scales[B][cap][dim/16]  (two planes).
 * Row value = e2m1(code) * e4m3(scale) (exact in fp16 and bf16).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,        /* a required pointer is NULL */
  CSA2_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  CSA2_ERR_DTYPE = 3,       /* unknown dtype code */
  CSA2_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  CSA2_ERR_UNSUPPORTED = 5, /* valid request outside what the kernels cover */
  CSA2_ERR_HIP = 6,         /* a HIP runtime call or launch failed */
  CSA2_ERR_INCOMPLETE = 7   /* a bounded wait of a one-wait launch ran out (csa2_workspace_check) */
} csa2_status;

/* Static per-layer mode ([P1 §03 "CSA2"]; [P5 "Then every layer stops asking
 * the same question"]: the mode is fixed per layer, not chosen at run time). */
typedef enum {
  CSA2_MODE_FULL = 0,    /* writes its KV, scores every visible position, selects */
  CSA2_MODE_REINDEX = 1, /* reuses another layer's KV, rescores with its own query */
  CSA2_MODE_REUSE = 2    /* reuses another layer's KV and Top-K selection */
} csa2_mode;

typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1 } csa2_dtype;

/* An FP4 cache: two device planes, see the layout above. */
typedef struct {
  uint8_t* codes;  /* [B][cap][dim/2] */
  uint8_t* scales; /* [B][cap][dim/16] */
  int32_t dim;     /* channels per row, a multiple of 16 */
  int64_t cap;     /* rows per sequence */
} csa2_fp4_cache;

/* Main cache in the FP8 variant (E4M3 rows with one fp32 scale per row; the
 * earlier format the pages describe for V4 Flash's global KV, [P1 §04]). */
typedef struct {
  uint8_t* codes;  /* [B][cap][dim] E4M3 bytes */
  float* scales;   /* [B][cap] */
  int32_t dim;     /* channels per row */
  int64_t cap;     /* rows per sequence */
} csa2_fp8_cache;

/* Limits the kernels accept. */
#define CSA2_MAX_K 16384        /* Top-K and pool size */
#define CSA2_MAX_W 16384        /* sliding-window length */
#define CSA2_HEADS 16           /* query heads of the attention kernel */
#define CSA2_MAX_INDEX_HEADS 16 /* indexer heads */

/* ------------------------------------------------------------------ */
/* Quantize-on-write ([P1 §04 "FP4"]: E2M1 codes with an E4M3 scale per 16
 * channels, applied after RoPE, so the rows passed here are post-RoPE).
 *
 * For every 16-channel block: amax = max |x|; scale = the E4M3 value nearest
 * to amax/6 (ties to the even mantissa, saturating at 448); each element's
 * code = the E2M1 value nearest to x/scale (ties to the even code, clamped
 * at +-6, sign bit = sign bit of x; a zero scale gives magnitude 0).
 *
 *   x           : device, `rows` rows of `dim` elements (dtype), row i at
 *                 x + i * x_row_stride elements.
 *   dst_rows    : device int64 [rows] destination row of each input row in
 *                 the planes (row index counted over all sequences, i.e.
 *                 b * cap + position), or NULL for rows 0..rows-1.
 *   codes/scales: device planes receiving dim/2 and dim/16 bytes per row.
 * Errors: NULL pointers, rows < 0, dim % 16 != 0 or dim > 4096, stride < dim,
 * unknown dtype.  rows == 0 launches nothing. */
csa2_status csa2_quantize_kv(const void* x, csa2_dtype dtype, int64_t rows, int32_t dim,
                             int64_t x_row_stride, const int64_t* dst_rows, uint8_t* codes,
                             uint8_t* scales, void* stream);

/* FP8 quantize-on-write of main-cache rows (the FP8 variant; the pages give
 * no scale layout for it, read here as one fp32 scale per row): scale =
 * amax/448 over the row (1 for an all-zero row), byte = E4M3 of
 * clamp(x/scale, -448, 448) rounded to nearest even (IEEE fp32 divisions).
 *   codes  : device [rows][dim] bytes;  scales : device f32 [rows] (both at
 *            the destination rows);  other arguments as csa2_quantize_kv.
 * Errors: as csa2_quantize_kv. */
csa2_status csa2_quantize_kv_fp8(const void* x, csa2_dtype dtype, int64_t rows, int32_t dim,
                                 int64_t x_row_stride, const int64_t* dst_rows, uint8_t* codes,
                                 float* scales, void* stream);

/* Rotary embedding fused with the quantize-on-write ([P1 §04 "FP4"]: the
 * quantisation is applied after RoPE; the pages give no rotary parameters, so
 * the angles come from the caller).  The last rope_dim channels of each row
 * hold rotary pairs (channels dim-rope_dim+2i, +2i+1); pair i of row r is
 * rotated by the caller's (c, s) = cos_sin[r][i]:
 *   y0 = x0*c - x1*s,  y1 = x0*s + x1*c,
 * each product and each sum rounded to fp32 separately (no fused
 * multiply-add), then every 16-channel block is quantized exactly as by
 * csa2_quantize_kv.
 *
 *   rope_dim : a multiple of 16 in [0, dim] (0: plain quantize-on-write).
 *   cos_sin  : device fp32 [rows][rope_dim/2][2] (cos, sin); may be NULL
 *              when rope_dim == 0.
 *   other arguments as csa2_quantize_kv.
 * Errors: those of csa2_quantize_kv, a rope_dim out of range, cos_sin NULL
 * with rope_dim > 0. */
csa2_status csa2_rope_quantize_kv(const void* x, csa2_dtype dtype, int64_t rows, int32_t dim,
                                  int64_t x_row_stride, int32_t rope_dim, const float* cos_sin,
                                  const int64_t* dst_rows, uint8_t* codes, uint8_t* scales,
                                  void* stream);

/* ------------------------------------------------------------------ */
/* Indexer scoring ([P1 §03 "CSA2"]: a Reindex layer scores positions again
 * with its own query; [P4 "Share the cache and the search work"]: the first
 * global indexing layer scans the visible context; [P5]: layers share the
 * indexer keys, stored in FP4).  For query row r (sequence b = r / T):
 *
 *   score[r][s] = sum_h w[r][h] * max(0, q_idx[r][h] . key_b(pos(s)))
 *
 * where pos(s) = s (flat) or pool[r][s] (pool given), for s < n_valid[r].
 * Entries s >= n_valid[r] of the score row are left unspecified.
 *
 *   icache   : FP4 index-key cache (dim = D_I, a multiple of 128, <= 512).
 *   q_idx    : device bf16 [B*T][H_I][D_I];  w : device f32 [B*T][H_I].
 *   n_valid  : device int32 [B*T]; flat: positions [0, n_valid) are
 *              visible (must be <= cap); pool: the number of valid slots.
 *   pool     : device int32 [B*T][P] ascending positions (< cap) or NULL.
 *   scores   : device f32 [B*T][n_out]; n_out >= every n_valid.
 * Precision: products of the bf16 query and the exactly dequantized keys are
 * accumulated in fp32 (each head's query is scaled by a power of two into
 * fp16 range for the matrix cores; the scaling is undone exactly).
 * Errors: NULL pointers, H_I outside [1,16], D_I not a multiple of 128 or
 * > 512, B/T < 1, n_out < 1, P < 1 with a pool. */
csa2_status csa2_index_score(const csa2_fp4_cache* icache, int32_t B, int32_t T,
                             const uint16_t* q_idx, const float* w, int32_t H_I,
                             const int32_t* n_valid, const int32_t* pool, int32_t P,
                             int64_t n_out, float* scores, void* stream);

/* ------------------------------------------------------------------ */
/* Top-K selection ([P4 "Share the cache and the search work"]: sparse
 * attention selects a fixed number of global entries from the indexer
 * scores; a candidate pool is selected the same way).  For each row r:
 * order slots s < n_valid[r] by score descending, equal scores (-0 == +0)
 * by slot ascending; keep the first min(k, n_valid[r]); write their
 * positions (slot_pos[r][s] when slot_pos is given, else s) ascending into
 * idx_out[r][0..), padding with -1 up to k.  count_out[r] (optional)
 * receives min(k, n_valid[r]).  slot_pos, when given, must be strictly
 * increasing over the valid slots of each row.
 *
 *   scores : device f32 [rows][n];  n_valid : device int32 [rows] (<= n).
 *   ws     : workspace of csa2_topk_workspace_bytes(rows, n, k) bytes.
 * Errors: NULL pointers, rows < 1, n < 1, k < 1 or k > CSA2_MAX_K,
 * n > 2^25, workspace too small. */
size_t csa2_topk_workspace_bytes(int32_t rows, int64_t n, int32_t k);
csa2_status csa2_topk(const float* scores, int32_t rows, int64_t n, const int32_t* n_valid,
                      const int32_t* slot_pos, int32_t k, int32_t* idx_out, int32_t* count_out,
                      void* ws, size_t ws_bytes, void* stream);

/* How a pass selects (chosen from its shape; csa2_set_topk_variant can force
 * one for tests).  The one-wait variant runs when all of the pass's select
 * blocks fit on the device at once by the occupancy query: each block then
 * waits, with a bounded poll, for a record that the row's last block sends
 * it.  If another process or stream keeps some of those blocks from being
 * resident, the poll runs out: that block writes nothing of its part of
 * idx_out and sets a flag in the workspace's control words.  The call still
 * returns CSA2_OK (the failure happens on the device, after the return);
 * csa2_workspace_check reports it as CSA2_ERR_INCOMPLETE and clears the
 * flag.  Records carry the launch's generation, so a record left behind by
 * such a launch is never taken by a later one, and later calls on the same
 * workspace are correct.
 *
 * Prefill passes of csa2_layer_step over long contexts (32 or more tokens
 * per sequence, 128-channel index keys, 1 to 4 indexer heads, K <= 2048,
 * 2^15 to 2^18 cache slots, no pool) select without a score matrix
 * (CSA2_TOPK_SAMPLED): every 32nd position is scored first and each row's
 * threshold is set from those samples so that about 2K positions pass it;
 * the full scan keeps only the positions at or above it, and the exact
 * Top-K is taken among them.  A row whose kept positions come short of K
 * or overflow their room is scored in full and selected by the ROW kernel,
 * so the result is the same index set, in the same order, as the other
 * variants give.  CSA2_TOPK_ROW or any score-matrix variant forced for such
 * a pass runs it the older way.
 *
 * Rows of at most 2^14 slots (a candidate pool's rows, short contexts)
 * select with one block per row and the row's keys in registers
 * (CSA2_TOPK_BAND): a 1024-key sample brackets the K-th largest key between
 * two keys with a wide margin, one pass counts the keys above the bracket
 * and lists those inside it, and the exact K-th is found among the listed
 * keys.  When the bracket misses (or too many keys share it, as with many
 * equal scores) the block runs the exact selection of the ROW kernel
 * instead: the index set and its order never depend on the sample. */
typedef enum {
  CSA2_TOPK_AUTO = 0,             /* chosen from the shape */
  CSA2_TOPK_ROW = 1,              /* one block per row, in LDS (rows of <= 2^18 slots) */
  CSA2_TOPK_ONE_WAIT = 2,         /* resident blocks; the row's last block sends records */
  CSA2_TOPK_SELECT = 3,           /* 4096-score blocks; the row's last block finishes */
  CSA2_TOPK_SELECT_CUT = 4,       /* ... after a kernel that finds each row's cut bin */
  CSA2_TOPK_SELECT_LARGE = 5,     /* 16384-score blocks; the row's last block finishes */
  CSA2_TOPK_SELECT_LARGE_CUT = 6, /* ... after the cut kernel */
  CSA2_TOPK_SAMPLED = 7,          /* prefill passes: sampled threshold, candidates only */
  CSA2_TOPK_SAMPLED_FALLBACK = 8, /* ... with every row sent to the exact path */
  CSA2_TOPK_BAND = 9,             /* one block per row of <= 2^14 slots: a sampled key band */
  CSA2_TOPK_BAND_EXACT = 10       /* ... with every row sent to the block's exact selection */
} csa2_topk_variant;
/* Flag in csa2_topk_last_variant(): the finishing block merged two sorted
 * lists (rows over 2^19 slots) instead of reading back a bitmap. */
#define CSA2_TOPK_LIST_FINISH 16

/* ------------------------------------------------------------------ */
/* Sparse attention ([P4 "Share the cache and the search work"]: attention
 * over the selected global entries alongside a local 128-token window;
 * [P1 §04 "FP4"]: the window KV stays in FP8).  For query row r (sequence
 * b = r / T, position p = q_pos[r]) and head h, one softmax over the union
 * of
 *   - the main-cache rows idx[r][j] (entries < 0 skipped), dequantized, and
 *   - the window rows holding positions [p-W+1, p] that are present in the
 *     window array (row i of sequence b holds position swa_pos0[b] + i),
 *     valued e4m3(byte) * swa_scale[b];
 * with logit = sm_scale * q[r][h] . k and value = the first dv channels of
 * the same row:
 *   out[r][h] = sum_j softmax_j(logit) * v_j,  lse[r][h] = log sum_j exp(logit_j).
 * The same position in both sets counts twice.  No entries: out = 0,
 * lse = -inf.
 *
 *   q        : device bf16 [B*T][H][D], H == CSA2_HEADS, D = kv->dim.
 *   kv       : FP4 main cache (dim a multiple of 64, <= 1024).
 *   idx      : device int32 [B*T][K], entries < kv->cap or negative.
 *   swa      : device uint8 [B][S][D] E4M3;  swa_scale : device f32 [B];
 *   swa_pos0 : device int32 [B];  0 <= W <= CSA2_MAX_W window length; S >= 0 rows.
 *   q_pos    : device int32 [B*T].
 *   out      : device f32 [B*T][H][dv] (dv a multiple of 64, <= D);
 *   lse      : device f32 [B*T][H] or NULL.
 *   ws       : workspace of csa2_sparse_attn_workspace_bytes(B*T, K, W, dv).
 * Precision: logits accumulate in fp32 from exact fp16 key values and the
 * bf16 query scaled per head by a power of two; probabilities are rounded
 * to fp16 for the value product, accumulated in fp32.
 * Errors: NULL pointers, H != CSA2_HEADS, bad D/dv, K < 0 (K == 0 allowed),
 * W < 0 or W > CSA2_MAX_W, S < 0, workspace too small. */
size_t csa2_sparse_attn_workspace_bytes(int32_t rows, int32_t K, int32_t W, int32_t dv);
csa2_status csa2_sparse_attn(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                             const csa2_fp4_cache* kv, const int32_t* idx, int32_t K,
                             const uint8_t* swa, const float* swa_scale, const int32_t* swa_pos0,
                             int32_t S, int32_t W, const int32_t* q_pos, float sm_scale,
                             int32_t dv, float* out, float* lse, void* ws, size_t ws_bytes,
                             void* stream);

/* The same attention in one launch (a Reuse layer's whole decode step):
 * each block computes its split, publishes the partial with device-coherent
 * stores and waits until all splits of its query row have arrived, then
 * merges a slice of the row's output.  Used when every block of the grid
 * fits on the device at once (rows x splits within the occupancy limit, one
 * round of 64 entries per split); otherwise the split and merge kernels of
 * csa2_sparse_attn run.  Arguments, workspace and results are those of
 * csa2_sparse_attn, bit for bit.  The wait is bounded: if it runs out (the
 * grid did not become resident, e.g. with other work occupying the device),
 * a control word stays set and the output is not written; csa2_workspace_check
 * reports it as CSA2_ERR_INCOMPLETE.  Callers that run other kernels
 * concurrently on the device should use csa2_sparse_attn. */
csa2_status csa2_sparse_attn_one_launch(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                                        const csa2_fp4_cache* kv, const int32_t* idx, int32_t K,
                                        const uint8_t* swa, const float* swa_scale,
                                        const int32_t* swa_pos0, int32_t S, int32_t W,
                                        const int32_t* q_pos, float sm_scale, int32_t dv,
                                        float* out, float* lse, void* ws, size_t ws_bytes,
                                        void* stream);

/* The same attention over an FP8 main cache (csa2_fp8_cache; the V4-Flash
 * style global KV of [P1 §04], E4M3 with one fp32 scale per row): a selected
 * row's key and value are e4m3(byte) * scale[row].  The window and every
 * other argument are as for csa2_sparse_attn (the same workspace size).
 * Inside a split, each row's scale multiplies its logit, and the value
 * product uses p_j * scale_j / max_scale (rounded to fp16) with the split's
 * largest row scale applied to its partial output. */
csa2_status csa2_sparse_attn_fp8(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                                 const csa2_fp8_cache* kv, const int32_t* idx, int32_t K,
                                 const uint8_t* swa, const float* swa_scale,
                                 const int32_t* swa_pos0, int32_t S, int32_t W,
                                 const int32_t* q_pos, float sm_scale, int32_t dv, float* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ */
/* One CSA2 layer for B sequences of T query tokens each ([P1 §03 "CSA2"]:
 * Full builds its KV and searches, Reindex reuses an earlier Full layer's
 * KV and rescores with its own query, Reuse reuses both KV and selection,
 * each layer keeping its own query and window; [P4]: the first indexing
 * layer keeps a candidate pool that later indexing layers search).
 *
 *   FULL    : quantize new_kv / new_ikey into kv / icache at rows q_pos;
 *             score positions [0, q_pos] of icache with q_idx, w_idx;
 *             if P > 0: pool_out = Top-P (ascending), pool_count_out =
 *             its size, idx_out = Top-K inside the pool (== flat Top-K);
 *             else idx_out = Top-K; attend over idx_out and the window.
 *   REINDEX : no write; score icache with its own q_idx, w_idx over
 *             [0, q_pos] (pool_in == NULL) or over pool_in's
 *             pool_count_in valid slots; Top-K -> idx_out; attend.
 *   REUSE   : attend over idx_in.
 * kv / icache are the layer's own caches for FULL and the referenced
 * layer's caches otherwise.  Its Top-K passes select as csa2_topk does
 * (including the one-wait variant and its csa2_workspace_check report). */
typedef struct {
  int32_t B, T;          /* sequences, query tokens per sequence */
  int32_t H, D, dv;      /* 16 query heads, row channels, value channels */
  int32_t H_I, D_I;      /* indexer heads and channels */
  int32_t K;             /* Top-K (<= CSA2_MAX_K) */
  int32_t P;             /* FULL: pool size to keep (0 = none) */
  int32_t S, W;          /* window array rows per sequence, window length */
  float sm_scale;
  csa2_fp4_cache kv;     /* main cache, dim D */
  csa2_fp4_cache icache; /* index-key cache, dim D_I (unused by REUSE) */
  const int32_t* q_pos;  /* [B*T] position of each query token */
  const void* new_kv;    /* FULL: [B*T][D] rows to write */
  const void* new_ikey;  /* FULL: [B*T][D_I] rows to write */
  csa2_dtype new_dtype;  /* dtype of new_kv / new_ikey */
  const uint16_t* q;     /* bf16 [B*T][H][D] */
  const uint16_t* q_idx; /* bf16 [B*T][H_I][D_I] (FULL, REINDEX) */
  const float* w_idx;    /* [B*T][H_I] (FULL, REINDEX) */
  const uint8_t* swa;    /* [B][S][D] E4M3 */
  const float* swa_scale;   /* [B] */
  const int32_t* swa_pos0;  /* [B] */
  const int32_t* idx_in;    /* REUSE: [B*T][K] */
  int32_t* idx_out;         /* FULL, REINDEX: [B*T][K] */
  const int32_t* pool_in;   /* REINDEX (optional): [B*T][P_in] */
  const int32_t* pool_count_in; /* REINDEX with pool_in: [B*T] */
  int32_t P_in;             /* row length of pool_in */
  int32_t* pool_out;        /* FULL with P > 0: [B*T][P] */
  int32_t* pool_count_out;  /* FULL with P > 0: [B*T] */
  float* out;               /* [B*T][H][dv] */
  float* lse;               /* [B*T][H] or NULL */
} csa2_layer_args;

size_t csa2_workspace_bytes(csa2_mode mode, const csa2_layer_args* a);
csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, void* ws,
                            size_t ws_bytes, void* stream);

/* The layer step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It runs exactly the launches of csa2_layer_step, with the workspace taken
 * from a static device array inside the library instead of an argument:
 * CSA2_STATIC_SCRATCH_BYTES on every GPU the library runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller still passes every input and
 * output in `a`.  On the first call on a device the array's address is
 * looked up and the array is zero-filled by a kernel on `stream` (again
 * after a call that returned CSA2_ERR_HIP).  Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents: calls that may overlap
 * on one GPU (other host threads or streams) race and must be serialised by
 * the caller.  Errors: those of csa2_layer_step, and CSA2_ERR_WORKSPACE when
 * the step needs more than CSA2_STATIC_SCRATCH_BYTES (csa2_workspace_bytes
 * gives the need; prefill chunks of thousands of tokens exceed it). */
#define CSA2_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
csa2_status csa2_layer_step_static(csa2_mode mode, const csa2_layer_args* a, void* stream);

/* ------------------------------------------------------------------ */
/* Helpers. */
/* Stored bytes per token of an FP4 row: dim/2 + dim/16 (324 for 576). */
int64_t csa2_fp4_bytes_per_token(int32_t dim);
/* Zero-fill a workspace on `stream` with a kernel (safe inside graph capture). */
csa2_status csa2_workspace_init(void* ws, size_t ws_bytes, void* stream);
/* Calls work through their query rows in passes of at most CSA2_PASS_ROWS
 * rows, and a prefill layer step that selects without a score matrix
 * (CSA2_TOPK_SAMPLED) in passes of at most CSA2_PREFILL_PASS_ROWS (a
 * 4096-token chunk: two passes); the workspace holds one pass's buffers. */
#define CSA2_PASS_ROWS 256
#define CSA2_PREFILL_PASS_ROWS 2048
/* Bytes at the start of a workspace that hold control words for
 * min(rows, CSA2_PASS_ROWS) query rows: they must be zero when a call
 * starts, and every successful call leaves them zero. */
size_t csa2_workspace_control_bytes(int32_t rows);
const char* csa2_status_string(csa2_status s);
/* Message of the last failing call on this host thread ("" if none). */
const char* csa2_last_error(void);
/* Library version string. */
const char* csa2_version(void);
/* Optional launch timing for measurement.  After csa2_profile_begin(), every
 * launch of the kernels below is bracketed by a pair of HIP events recorded
 * on the launch stream; csa2_profile_end() waits for them, writes the number
 * of launches and their summed duration (ms) per kernel, and stops
 * recording.  Kernel ids: 0 quantize-on-write, 1 indexer scoring, 2 Top-K
 * select, 3 sparse attention, 4 pool gather.  Not thread-safe; not for use
 * under graph capture.  `counts` and `total_ms` hold 5 entries. */
#define CSA2_PROFILE_KERNELS 5
csa2_status csa2_profile_begin(void);
csa2_status csa2_profile_end(int32_t* counts, double* total_ms);
/* sizeof(csa2_layer_args) and sizeof(csa2_fp4_cache) as compiled into the
 * library, so bindings can check their struct layout. */
size_t csa2_layer_args_size(void);
size_t csa2_fp4_cache_size(void);

/* Measurement reference: a plain streaming read of `bytes` (a multiple of
 * 16) at `src` by `blocks` blocks of 256 threads (16-byte non-temporal
 * loads), each block writing one folded word to sink[block] so that no load
 * can be dropped.  Its rate is the achievable HBM read bandwidth the hot
 * path's streaming kernels are compared with.  Errors: NULL pointers, bytes
 * not a positive multiple of 16, blocks outside [1, 2^20]. */
csa2_status csa2_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                             void* stream);

/* Reports whether a one-wait launch on this workspace gave up waiting
 * (see the Top-K variants above and csa2_sparse_attn_one_launch).  Waits
 * for `stream`, reads the wait-failure flags of the control words of
 * min(rows, CSA2_PASS_ROWS) query rows (rows = the largest B*T used with
 * the workspace), and returns CSA2_ERR_INCOMPLETE if any is set, after zeroing
 * the whole control block (every call on the workspace has finished, so
 * nothing is still writing to it).  The outputs of the calls since the last
 * check are then incomplete.  Returns CSA2_OK when no flag is set.
 * Errors: NULL workspace, ws_bytes below csa2_workspace_control_bytes(rows),
 * a HIP failure while reading. */
csa2_status csa2_workspace_check(void* ws, size_t ws_bytes, int32_t rows, void* stream);

/* Diagnostics for tests (process-wide, not for use while other threads
 * launch).  csa2_set_topk_variant forces a Top-K variant on every later pass
 * that it can serve (a pass it cannot serve -- rows too long for ROW, a grid
 * too large for ONE_WAIT -- keeps its own choice) and returns the previous
 * setting; CSA2_TOPK_AUTO restores the default.  csa2_topk_last_variant
 * gives the variant the calling thread's last Top-K pass ran (with
 * CSA2_TOPK_LIST_FINISH or-ed in when it applies), -1 before any.
 * csa2_set_wait_limit sets the polls a one-wait block makes before it gives
 * up (default 2^20, about 10 ms or more; 0 gives up at once, which forces
 * the failure path) and returns the previous limit. */
int32_t csa2_set_topk_variant(int32_t variant);
int32_t csa2_topk_last_variant(void);
uint32_t csa2_set_wait_limit(uint32_t polls);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
