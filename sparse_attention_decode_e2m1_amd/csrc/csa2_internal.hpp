// csa2_internal.hpp -- launchers and workspace layout shared by the HIP
// translation units of libcsa2.so.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

constexpr int32_t kScoreChunk = 2048;  // positions per scoring block (fewer when the scan is small)
constexpr int64_t kScanMinBlocks = 512; // ... so that a scan has at least this many blocks
constexpr int kScoreGroup = 4;         // consecutive 16-position tiles per wave load
constexpr int32_t kTopkChunk = 4096;        // scores per select block (4 per thread)
constexpr int32_t kTopkChunkLarge = 16384;  // ... when a pass has many rows (16 per thread)
constexpr int32_t kAttnSplit = 64;      // entries per attention split (one tile per wave)
constexpr int32_t kMaxSplits = 512;     // (CSA2_MAX_K + CSA2_MAX_W) / kAttnSplit
constexpr int64_t kMaxTopkN = int64_t(1) << 25;  // longest score row Top-K accepts

// Every call keeps the control words of query row r -- the Top-K histogram
// copies and counters -- in one fixed-size block at the start of the
// workspace.  They are zero between calls, so any workspace left by a
// previous call (of any kind or shape) is ready for the next.
constexpr int kMaxHistCopies = 8;
constexpr int64_t kHistWords = int64_t(kMaxHistCopies) * 4096;  // copies x 4096 bins
// + the Top-K arrival counter (word 0) and the Top-K cut bin (word 1)
constexpr int64_t kCtlWordsPerRow = kHistWords + 64;

struct TopkWs {
  uint32_t* hist;        // row r at hist + r * hist_stride (kHistCopies x 4096 bins)
  int64_t hist_stride;   // in words
  // Per select block b of row r, regions of `chunk` entries at offset
  // r * stride + b * chunk (chunk = kTopkChunk or kTopkChunkLarge): the positions kept outright and the
  // candidates' 64-bit rank values, each in position order.
  uint32_t* above;
  int64_t above_stride;
  uint64_t* cand;
  int64_t cand_stride;
  uint32_t* counts;      // row r at counts + r * counts_stride: (kept, candidates) per block
  int64_t counts_stride;
  uint32_t* ctr;         // row r at ctr + r * ctr_stride: select blocks arrived (zero between calls)
  int64_t ctr_stride;
  uint32_t* cut;         // row r at cut + r * ctr_stride: the cut bin, when precomputed
  int32_t hist_copies;   // histogram copies in use (1 .. kHistCopies)
};

struct AttnWs {
  float* part;        // [rows][nsplit][16*dv + 32]
};

struct AttnSplit {
  int32_t nsg, nsw, nsplit;  // splits of global entries, of window entries, total
};
inline AttnSplit attn_split(int32_t K, int32_t W, int32_t rounds = 1) {
  AttnSplit s;
  const int32_t span = kAttnSplit * rounds;  // entries per split
  s.nsg = (K + span - 1) / span;
  if (s.nsg < 1) s.nsg = 1;  // one split still writes the empty result
  s.nsw = (W + span - 1) / span;
  s.nsplit = s.nsg + s.nsw;
  return s;
}
// Rounds (of 64 entries) per attention split for a pass of `rows` rows: one,
// unless the grid would exceed kAttnGridBlocks blocks (the split kernel's
// blocks an MI355X holds at once, two per compute unit: a grid just past it
// would run a second wave of blocks); then doubled, up to 8, keeping
// at least 2 splits per row (FP4 main cache only: the FP8 variant takes one
// round).  A function of the shape alone, so the workspace query sizes the
// partials of every pass exactly.
constexpr int64_t kAttnGridBlocks = 512;
inline int32_t attn_rounds(int64_t rows, int32_t K, int32_t W, bool kv8) {
  int32_t rounds = 1;
  AttnSplit sp = attn_split(K, W, rounds);
  while (!kv8 && (int64_t)sp.nsplit * rows > kAttnGridBlocks && sp.nsplit > 2 && rounds < 8) {
    rounds *= 2;
    sp = attn_split(K, W, rounds);
  }
  return rounds;
}

// Process-wide diagnostic controls (set through csa2_set_topk_variant and
// csa2_set_wait_limit) and what the last Top-K launch of this thread ran.
enum TopkVariant : int32_t {
  kTopkAuto = 0,         // chosen from the pass's shape
  kTopkRow = 1,          // one block per row, selection in LDS (rows <= kRowTopkMaxN slots)
  kTopkOneWait = 2,      // every block resident; the row's last block sends records
  kTopkSelect = 3,       // 4096-score blocks; the row's last block finishes
  kTopkSelectCut = 4,    // ... after a per-row cut kernel
  kTopkSelectLarge = 5,  // 16384-score blocks; the row's last block finishes
  kTopkSelectLargeCut = 6,
  kTopkSampled = 7,          // prefill: a sampled threshold, then the candidates above it only
  kTopkSampledFallback = 8,  // ... with every row sent to the exact path (a test of that path)
  kTopkBand = 9,             // one block per row, a sampled key band (rows <= kRowTopkSmallN slots)
  kTopkBandExact = 10,       // ... with every row sent to its exact LDS selection (a test of that path)
  kTopkVariants = 11,
};
constexpr int32_t kTopkListFinish = 16;  // flag: the finishing block merged sorted lists
int32_t topk_variant_forced();
void set_topk_last(int32_t v);
uint32_t wait_limit();
uint32_t next_generation();  // per one-wait launch (records carry it)

// Launch timing: while the library profiles a call, its launchers attach
// the call's start and stop events to the first and last kernel they launch
// (the events then carry the kernels' own start and end times).
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
  bool started = false, stopped = false;
};
LaunchTiming& launch_timing();
#define CSA2_KERNEL(FIRST, LAST, kernel, grid, block, lds, st, ...)                           \
  do {                                                                                      \
    LaunchTiming& _lt = launch_timing();                                                    \
    if (_lt.start) {                                                                        \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, st, (FIRST) ? _lt.start : nullptr,    \
                            (LAST) ? _lt.stop : nullptr, 0, __VA_ARGS__);                   \
      _lt.started |= (FIRST);                                                               \
      _lt.stopped |= (LAST);                                                                \
    } else {                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, lds, st, __VA_ARGS__);                        \
    }                                                                                       \
  } while (0)

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int32_t dim, int64_t stride,
                           const int64_t* dst_rows, uint8_t* codes, uint8_t* scales,
                           hipStream_t st);
// FP8 main-cache rows: per row, scale = amax/448 (1 for an all-zero row) and
// byte = E4M3(clamp(x / scale, +-448)), round to nearest even.
hipError_t launch_quantize_fp8(const void* x, bool bf16, int64_t rows, int32_t dim, int64_t stride,
                               const int64_t* dst_rows, uint8_t* codes, float* scales,
                               hipStream_t st);
hipError_t launch_rope_quantize(const void* x, bool bf16, int64_t rows, int32_t dim,
                                int64_t stride, int32_t rope_dim, const float* cos_sin,
                                const int64_t* dst_rows, uint8_t* codes, uint8_t* scales,
                                hipStream_t st);
// A Full layer's new rows in a decode step (one query token per sequence):
// row r of kv / ikey goes to cache row (r / T) * cap + q_pos[r] of the main
// and index caches.  The decode scan writes them itself (one extra block per
// query row, which also scores the new position), so the step needs no
// separate quantize-on-write launch.
struct NewRows {
  const void* kv = nullptr;    // [rows][kv_dim]
  const void* ikey = nullptr;  // [rows][DI]
  bool bf16 = false;
  const int32_t* q_pos = nullptr;
  uint8_t* kv_codes = nullptr;
  uint8_t* kv_scales = nullptr;
  int64_t kv_cap = 0;
  int32_t kv_dim = 0;
};
// Shapes whose new rows the decode scan writes itself (otherwise a separate
// quantize-on-write launch comes first).
bool fresh_rows_supported(bool pool, int32_t T, int32_t HI, int32_t DI, int32_t kv_dim);
hipError_t launch_index_score(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                              int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                              const float* w, int32_t HI, const int32_t* n_valid,
                              int32_t nv_add, const int32_t* pool, int32_t P, int64_t n_max,
                              float* scores, int64_t n_out, uint32_t* hist, int64_t hist_stride,
                              int32_t hist_copies, hipStream_t st, int32_t row0 = 0,
                              const NewRows* fresh = nullptr);
// Prefill passes (32 or more tokens per sequence in whole waves of one
// sequence, 128-channel keys, at most 4 indexer heads, no pool) score with
// the tokens x positions kernel, which writes every visible score.
bool index_tokens_pass(bool pool, int32_t T, int32_t HI, int32_t DI, int32_t row0);
hipError_t launch_index_tokens(const uint8_t* codes, const uint8_t* scales, int64_t cap,
                               int32_t rows, int32_t T, const uint16_t* q_idx, const float* w,
                               int32_t HI, const int32_t* n_valid, int32_t nv_add, int64_t n_max,
                               float* scores, int64_t n_out, hipStream_t st, int32_t row0,
                               bool last);
hipError_t launch_topk_hist(const float* scores, int32_t rows, int64_t n, const int32_t* n_valid,
                            int32_t nv_add, int64_t n_max, uint32_t* hist, int64_t hist_stride,
                            int32_t hist_copies, hipStream_t st, bool first = true);
// Passes of at least kRowTopkMinRows rows of at most kRowTopkMaxN slots, and
// passes of any number of rows of at most kRowTopkSmallN slots, select with
// one block per row (topk_row_pass); that path reads no score histogram, so
// a caller that takes it (row_ok = true) builds none.
constexpr int32_t kRowTopkMinRows = 64;
constexpr int64_t kRowTopkMaxN = 262144;
constexpr int64_t kRowTopkSmallN = 16384;
bool topk_row_pass(int32_t rows, int64_t n_max);

// Prefill selection without a score matrix.  Every kSampleStride-th
// position is scored first; each row's threshold is read off those samples
// low enough that, in expectation, twice the row's K positions pass it; the
// full scan then keeps only the positions at or above it (about 2K per row
// instead of every score), and the exact Top-K is taken among them.  A row
// whose candidates come short of K, or overflow the room for them, is
// scored in full again and selected by the one-block-per-row kernel, so the
// result never depends on the sample.  With a stride of 32 the threshold
// sits 6.7 standard deviations (of the sample's rank noise) above K for
// K = 2048 on independent scores (16: 8.7); 2.310 -> 2.274 ms per 4096-token
// chunk against 16.
constexpr int kSampleStride = 32;
constexpr int kCandCap = 8192;    // candidates kept per row
constexpr int kCandStage = 128;   // list room per token of a scoring block (1 in 8 positions)
struct SampledSel {
  float* samp;        // row r: sample m (position kSampleStride * m) at samp + r * ns_stride + m
  int64_t ns_stride;
  uint32_t* thr;      // per row: the candidates' key threshold
  uint32_t* count;    // per row: candidates written
  uint32_t* fail;     // per row: nonzero sends the row to the exact path
  uint2* cand;        // row r: kCandCap (score key, slot) pairs at cand + r * kCandCap
};
// The prefill passes whose shapes allow it (flat scan, tokens x positions
// kernel, K <= 2048, at least 32 K positions, at most kRowTopkMaxN), and
// those that take it (the shapes, and a forced Top-K variant that allows it).
bool sampled_select_shapes(int32_t rows, int32_t T, int32_t HI, int32_t DI, int32_t row0,
                           int32_t K, int64_t n_max);
bool sampled_select_pass(int32_t rows, int32_t T, int32_t HI, int32_t DI, int32_t row0,
                         int32_t K, int64_t n_max);
hipError_t launch_index_sample(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                               int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                               const float* w, int32_t HI, const int32_t* n_valid,
                               int32_t nv_add, int64_t n_max, const SampledSel& sel,
                               hipStream_t st, int32_t row0);
hipError_t launch_index_candidates(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                                   int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                                   const float* w, int32_t HI, const int32_t* n_valid,
                                   int32_t nv_add, int64_t n_max, const SampledSel& sel,
                                   hipStream_t st, int32_t row0);
// The full score rows of the rows whose fail word is set (others untouched).
hipError_t launch_index_score_failed(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                                     int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                                     const float* w, int32_t HI, const int32_t* n_valid,
                                     int32_t nv_add, int64_t n_max, float* scores, int64_t n_out,
                                     const uint32_t* fail, hipStream_t st, int32_t row0);
hipError_t launch_sample_threshold(int32_t rows, const int32_t* n_valid, int32_t nv_add,
                                   int64_t n_max, int32_t k, const SampledSel& sel,
                                   bool force_fail, hipStream_t st);
hipError_t launch_sampled_final(int32_t rows, const int32_t* n_valid, int32_t nv_add,
                                int64_t n_max, int32_t k, int32_t* idx_out,
                                const SampledSel& sel, hipStream_t st);
// topk_row_kernel over the rows whose fail word is set.
hipError_t launch_topk_row_failed(const float* scores, int32_t rows, int64_t n,
                                  const int32_t* n_valid, int32_t nv_add, int32_t k,
                                  int32_t* idx_out, const uint32_t* fail, hipStream_t st);
hipError_t launch_topk_select(const float* scores, int32_t rows, int64_t n,
                              const int32_t* n_valid, int32_t nv_add, int64_t n_max,
                              const int32_t* slot_pos, int32_t k, int32_t* idx_out,
                              int32_t* count_out, const TopkWs& w, hipStream_t st,
                              bool row_ok = false, float* gather_out = nullptr,
                              bool* gathered = nullptr);
hipError_t launch_sparse_attn(const uint16_t* q, int32_t rows, int32_t T, int32_t D, int32_t dv,
                              const uint8_t* codes, const uint8_t* scales, int64_t cap,
                              const int32_t* idx, int32_t K, const uint8_t* swa,
                              const float* swa_scale, const int32_t* swa_pos0, int32_t S,
                              int32_t W, const int32_t* q_pos, float sm_scale, float* out,
                              float* lse, const AttnWs& w, hipStream_t st, int32_t row0 = 0,
                              const float* row_scale = nullptr,
                              uint32_t* one_launch_ctl = nullptr);
// Control words of the one-launch attention within a row's control block
// (arrivals, departures, the failed-wait flag).
constexpr int64_t kAttnCtlWord = kHistWords + 8;
size_t attn_lds_bytes(int32_t dv);
// out[r][s] = scores[r][pool[r][s]] for s < count[r], and the histogram of
// those scores into hist (row stride hist_stride).
hipError_t launch_gather_scores(const float* scores, int64_t n, const int32_t* pool, int32_t P,
                                const int32_t* count, int32_t rows, float* out,
                                uint32_t* hist, int64_t hist_stride, int32_t hist_copies,
                                hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// Blocks of `kernel` (with `threads` threads and `lds` bytes of dynamic LDS)
// that the current device holds at once, from the occupancy query; cached
// per (kernel, threads, LDS, device) and safe to call from several threads.
// 0 if the query fails.
int64_t device_resident_blocks(const void* kernel, int threads, size_t lds);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                              hipStream_t st);
// Quantize-on-write of one decode/prefill step: rows r of x1 (dim1) and x2
// (dim2) go to cache row (r / T) * cap + q_pos[r] of their planes.
hipError_t launch_quantize_step(const void* x1, const void* x2, bool bf16, int32_t rows,
                                int32_t T, const int32_t* q_pos, int32_t dim1, int64_t cap1,
                                uint8_t* codes1, uint8_t* scales1, int32_t dim2, int64_t cap2,
                                uint8_t* codes2, uint8_t* scales2, hipStream_t st);

}  // namespace csa2
