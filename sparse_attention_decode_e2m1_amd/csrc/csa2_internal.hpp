// csa2_internal.hpp -- launchers and workspace layout shared by the HIP
// translation units of libcsa2.so.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

constexpr int32_t kScoreChunk = 2048;  // positions per scoring block
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
hipError_t launch_index_score(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                              int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                              const float* w, int32_t HI, const int32_t* n_valid,
                              int32_t nv_add, const int32_t* pool, int32_t P, int64_t n_max,
                              float* scores, int64_t n_out, uint32_t* hist, int64_t hist_stride,
                              int32_t hist_copies, hipStream_t st, int32_t row0 = 0);
hipError_t launch_topk_hist(const float* scores, int32_t rows, int64_t n, const int32_t* n_valid,
                            int32_t nv_add, int64_t n_max, uint32_t* hist, int64_t hist_stride,
                            int32_t hist_copies, hipStream_t st, bool first = true);
// Passes of at least kRowTopkMinRows rows of at most kRowTopkMaxN slots can
// select with one block per row (topk_row_pass); that path reads no score
// histogram, so a caller that takes it (row_ok = true) builds none.
constexpr int32_t kRowTopkMinRows = 64;
constexpr int64_t kRowTopkMaxN = 262144;
bool topk_row_pass(int32_t rows, int64_t n_max);
hipError_t launch_topk_select(const float* scores, int32_t rows, int64_t n,
                              const int32_t* n_valid, int32_t nv_add, int64_t n_max,
                              const int32_t* slot_pos, int32_t k, int32_t* idx_out,
                              int32_t* count_out, const TopkWs& w, hipStream_t st,
                              bool row_ok = false);
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
// Quantize-on-write of one decode/prefill step: rows r of x1 (dim1) and x2
// (dim2) go to cache row (r / T) * cap + q_pos[r] of their planes.
hipError_t launch_quantize_step(const void* x1, const void* x2, bool bf16, int32_t rows,
                                int32_t T, const int32_t* q_pos, int32_t dim1, int64_t cap1,
                                uint8_t* codes1, uint8_t* scales1, int32_t dim2, int64_t cap2,
                                uint8_t* codes2, uint8_t* scales2, hipStream_t st);

}  // namespace csa2
