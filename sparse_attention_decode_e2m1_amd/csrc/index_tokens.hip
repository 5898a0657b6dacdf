// index_tokens.hip -- indexer scoring of a prefill chunk.
//
// Every query token of the chunk scores every visible cached position,
//     score = sum_h w_h * max(0, q_h . k_s),
// over the same FP4 index keys as the decode scan (helmcode.com/deepseek-
// v41-flash, section "03 · CSA2"; louisbouchard.ai/deepseek-v41-flash-kv-
// cache-writing-benchmark, "Share the cache and the search work": the first
// indexing layer scans the whole visible context).  With many tokens per
// sequence this is a genuine tokens x positions contraction, so it runs on
// MFMA with each key tile dequantized once for 16 tokens per wave.  The
// prefill selection without a score matrix (a sampled threshold, the
// candidates at or above it, the exact path for rows that need it) is built
// from three modes of the same kernel.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

// Row groups of 4 tokens per wave, and positions per block (4 groups: at
// most 256 registers, two waves per SIMD; 8 groups need 448 and leave one).
constexpr int kPrefillGroups = 4;
constexpr int32_t kPrefillChunk = 1024;
// A listed candidate's second word: its slot in the block (kEntTokShift
// bits), its token in the block (6 bits), then its rank among the token's
// entries of the block.
constexpr int kEntTokShift = 12, kEntRankShift = kEntTokShift + 6;
static_assert(kPrefillChunk <= (1 << kEntTokShift), "a candidate's slot in its block fits");
static_assert(kCandStage * 8 == kPrefillChunk, "list room: one in eight positions per token");

// Many query tokens of one sequence score the same positions, so the scan
// becomes a tokens x positions contraction: MFMA rows = 4 tokens x 4 heads,
// columns = 16 positions, k = channels.  A wave holds the query fragments of
// 4 NG tokens (NG row groups) in registers and dequantizes each key tile once
// for all of them: 4 NG MFMAs per 16-position tile.  Lane (i, g) of row group
// j then holds the four heads of token 4j + g at position i, so the score
// needs no cross-lane sum.  Token t sees positions below n_valid[t] + nv_add.
// The fragments take 16 NG registers, so NG trades the dequantisation's share
// against waves per SIMD.
//
// MODE selects what becomes of the scores:
//   kTokAll      every score stored in the score row (only the rows whose
//                fail word is set when `fail` is given);
//   kTokSample   the scan runs over samples m (position kSampleStride * m)
//                and stores each in the row's sample list;
//   kTokCand     only scores whose key reaches the row's threshold are kept:
//                listed per wave in LDS, then appended to each token's row
//                list with one claim per token and block.
enum { kTokAll = 0, kTokSample = 1, kTokCand = 2 };

// Compare predicates of the lane-mask compare builtins (LLVM's numbering).
constexpr int kCmpOge = 3, kCmpUlt = 36, kCmpSlt = 40;

// a if this lane's bit of `mask` is set, else b (one v_cndmask on the mask)
__device__ __forceinline__ uint32_t lane_select(uint64_t mask, uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(mask));
  return r;
}

template <int NCH, int NG, int MODE>
__global__ __launch_bounds__(256) void index_score_tokens_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t cap,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int32_t HI, int32_t T,
    const int32_t* __restrict__ n_valid, int32_t nv_add, int32_t rows, float* __restrict__ scores,
    int64_t n_out, int32_t chunk, int32_t row0, const uint32_t* __restrict__ fail,
    SampledSel sel) {
  constexpr int DI = 128 * NCH;
  constexpr int ROWB = DI / 2;
  constexpr int ROWS = DI / 16;
  constexpr int TPW = 4 * NG;  // tokens per wave
  constexpr int TPB = 4 * TPW; // tokens per block
  constexpr int PSTEP = (MODE == kTokSample) ? kSampleStride : 1;  // positions per scanned slot
  static_assert(TPW <= 32, "the visible-length reduction covers 32 lanes");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int rbase = blockIdx.y * TPB + wave * TPW;  // first token row of this wave
  // The candidate mode has block-wide barriers: a wave without work skips
  // the scan instead of returning.  Each wave lists its kept scores as
  // (score bits, slot in the block | token in the block << kEntTokShift |
  // rank among the token's entries << kEntRankShift); lanes that keep
  // nothing write a sink entry
  // of their own past the list, so the scan has no branch.
  constexpr int WCAP = TPW * kCandStage;  // list entries per wave
  static_assert(MODE != kTokCand || (TPB <= 64 && WCAP <= (1 << (32 - kEntRankShift))),
                "list entry fields");
  __shared__ uint2 wbuf[MODE == kTokCand ? 4 : 1][MODE == kTokCand ? WCAP + 64 : 1];
  __shared__ uint32_t wtot[MODE == kTokCand ? 4 : 1];
  __shared__ uint32_t lcnt[MODE == kTokCand ? TPB : 1];
  __shared__ uint32_t lbase[MODE == kTokCand ? TPB : 1];
  bool live_wave = rbase < rows;
  if constexpr (MODE != kTokCand) {
    if (!live_wave) return;  // no block-wide barrier below
    if (fail) {              // only the waves holding a failed row
      const bool f = fail[min(rbase + (lane & (TPW - 1)), rows - 1)] != 0u;
      if (__ballot(f) == 0ull) return;
    }
  }
  const int rb = min(rbase, rows - 1);
  const int b = (row0 + rb) / T;  // the wave's tokens share the sequence
  // the wave's longest visible length (in scanned slots)
  int64_t nvmax;
  {
    const int tr = min(rb + (lane & (TPW - 1)), rows - 1);
    int64_t m = min(min((int64_t)n_valid[tr] + nv_add, n_out), cap);
#pragma unroll
    for (int d = 1; d < TPW; d <<= 1) m = max(m, (int64_t)__shfl_xor(m, d, kWave));
    nvmax = (m + PSTEP - 1) / PSTEP;
  }
  const int64_t start = (int64_t)blockIdx.x * chunk;
  if (start >= nvmax) {
    if constexpr (MODE != kTokCand) return;
    live_wave = false;
  }
  const int64_t end = min(nvmax, start + chunk);

  // query fragments: row i of group j = token 4j + i/4, head i%4
  f16x8 qv[NG][NCH][4];
  float wq[NG][4];
  // candidate mode, token 4j + g: the smallest score whose key reaches the
  // row's threshold and the end of its range relative to the block's first
  // slot (within the block's slots); the wave's list length
  float thrf[NG];
  int lim[NG];
  uint32_t wcnt = 0u;
  {
    const int h = i & 3;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int t = min(rb + 4 * j + (i >> 2), rows - 1);
      const bool live = h < HI;
      const uint16_t* qr = q_idx + ((int64_t)t * HI + (live ? h : 0)) * DI;
      float vals[NCH][4][8];
      float amax = 0.0f;
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint4 raw = *reinterpret_cast<const uint4*>(qr + 128 * c2 + 32 * g + 8 * kk);
          const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            vals[c2][kk][2 * x] = bf16_to_f32(wd[x] & 0xFFFFu);
            vals[c2][kk][2 * x + 1] = bf16_to_f32(wd[x] >> 16);
          }
#pragma unroll
          for (int x = 0; x < 8; ++x) amax = fmaxf(amax, fabsf(vals[c2][kk][x]));
        }
      amax = fmaxf(amax, shfl_xor(amax, 16));
      amax = fmaxf(amax, shfl_xor(amax, 32));
      const int qexp = fp16_exponent_for(amax);
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int x = 0; x < 8; ++x)
            qv[j][c2][kk][x] = live ? (_Float16)ldexpf(vals[c2][kk][x], qexp) : (_Float16)0.0f;
      // epilogue weights of token 4j + g, heads rr (exponent from lane 4g + rr)
      const int te = min(rb + 4 * j + g, rows - 1);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = __shfl(qexp, 4 * g + rr, kWave);
        const float wv = w[(int64_t)te * HI + min(rr, HI - 1)];  // unconditional load
        wq[j][rr] = (rr < HI) ? ldexpf(wv, -e) : 0.0f;
      }
      if constexpr (MODE == kTokCand) {
        // a token past the last row keeps nothing
        const uint32_t tk = sel.thr[te];
        // the score whose key is tk (keys below that of -inf: every score)
        thrf[j] = (tk <= 0x007FFFFFu) ? -INFINITY
                                      : __uint_as_float((tk & 0x80000000u) ? (tk & 0x7FFFFFFFu) : ~tk);
        const int64_t nvt = (rb + 4 * j + g < rows)
                                ? min(min((int64_t)n_valid[te] + nv_add, n_out), cap) : (int64_t)0;
        lim[j] = (int)max(min(nvt, end) - start, (int64_t)0);
      }
    }
  }

  const uint8_t* cbase = codes + (int64_t)b * cap * ROWB;
  const uint8_t* sbase = scales + (int64_t)b * cap * ROWS;
  const int sshift = 16 * (g & 1);
  const int ntiles = live_wave ? (int)((end - start + 15) >> 4) : 0;
  auto load_tile = [&](int tile, u32x4 (&cw)[NCH], uint32_t (&sw)[NCH]) {
    int64_t s = start + (int64_t)tile * 16 + i;
    if (s >= end) s = end - 1;
    const int64_t pr = s * PSTEP;  // cache row of the slot
    // ordinary loads: the block's four waves and the other row groups'
    // blocks read the same rows, so they should stay in the caches
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
      cw[c2] = *reinterpret_cast<const u32x4*>(cbase + pr * ROWB + 64 * c2 + 16 * g);
      sw[c2] = *reinterpret_cast<const uint32_t*>(sbase + pr * ROWS + 8 * c2 + 4 * (g >> 1));
    }
  };
  // a ring of PF tiles in flight ahead of the one being computed
  constexpr int PF = 4;
  u32x4 cw[PF][NCH];
  uint32_t sw[PF][NCH];
  if (ntiles > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) load_tile(min(p, ntiles - 1), cw[p], sw[p]);
  }
  for (int t0 = 0; t0 < ntiles; t0 += PF) {
    // Tiles past the end recompute the clamped last position and store the
    // same value there, so the body is straight-line code (no early exit)
    // and the waits for each ring slot count only its own loads.
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int tile = t0 + p;
      f16x8 kb[NCH][4];
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) {
        const uint32_t s2b = sw[p][c2] >> sshift;
        const f16x2 s_lo = scale_pair(s2b & 0xFFu);
        const f16x2 s_hi = scale_pair((s2b >> 8) & 0xFFu);
        kb[c2][0] = fp4x8_to_f16(cw[p][c2].x, s_lo);
        kb[c2][1] = fp4x8_to_f16(cw[p][c2].y, s_lo);
        kb[c2][2] = fp4x8_to_f16(cw[p][c2].z, s_hi);
        kb[c2][3] = fp4x8_to_f16(cw[p][c2].w, s_hi);
      }
      // refill this ring slot with the tile PF ahead (clamped in range)
      load_tile(min(tile + PF, ntiles - 1), cw[p], sw[p]);
      const int rel = tile * 16 + i;
      const int64_t s = start + rel;
      // the NG row groups' products interleaved (independent accumulators)
      f32x4 acc[NG];
#pragma unroll
      for (int j = 0; j < NG; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int j = 0; j < NG; ++j) acc[j] = mfma16x16x32(qv[j][c2][kk], kb[c2][kk], acc[j]);
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        float part = 0.0f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) part += wq[j][rr] * relu(acc[j][rr]);
        const int64_t tr = min(rbase + 4 * j + g, rows - 1);
        if constexpr (MODE == kTokAll) {
          // Unconditional (clamped) store, as in index_score_kernel: tokens
          // past the last row computed that row's score (clamped query and
          // weights), and slots past a token's visible range are never read
          // for it.
          scores[tr * n_out + min(s, end - 1)] = part;
        } else if constexpr (MODE == kTokSample) {
          sel.samp[tr * sel.ns_stride + min(s, end - 1)] = part;
        } else {
          // Slots past the end (a padded tile, or past the token's visible
          // range) keep nothing, so no position is listed twice.  A kept
          // score takes the next place of the wave's list (lanes in order);
          // past the list's end it is dropped and counted, which sends the
          // wave's tokens to the exact path.  (-0 passes a threshold of +0,
          // as its key equals that of +0.)
          // The lane masks come straight from the compares (signed rel <
          // lim, ordered part >= threshold, unsigned p < WCAP) and select
          // each lane's entry, so no condition is turned into a value and
          // back.
          const uint64_t m = __builtin_amdgcn_sicmp(rel, lim[j], kCmpSlt) &
                             __builtin_amdgcn_fcmpf(part, thrf[j], kCmpOge);
          const uint32_t p = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)m, wcnt));
          const uint64_t put = m & __builtin_amdgcn_uicmp(p, (uint32_t)WCAP, kCmpUlt);
          const uint32_t tokb = (uint32_t)(wave * TPW + 4 * j + g);
          wbuf[wave][lane_select(put, p, (uint32_t)(WCAP + lane))] =
              make_uint2(__float_as_uint(part), (uint32_t)rel | (tokb << kEntTokShift));
          wcnt += (uint32_t)__popcll(m);
        }
      }
    }
  }
  if constexpr (MODE == kTokCand) {
    if (lane == 0) wtot[wave] = wcnt;
    if (tid < TPB) lcnt[tid] = 0u;
    __syncthreads();
    // each listed entry's rank among its token's entries
    for (int x = tid; x < 4 * WCAP; x += 256) {
      const int wv = x / WCAP, e = x - wv * WCAP;
      if ((uint32_t)e < min(wtot[wv], (uint32_t)WCAP)) {
        const uint32_t y = wbuf[wv][e].y;
        const uint32_t rank = atomicAdd(&lcnt[(y >> kEntTokShift) & 63u], 1u);
        wbuf[wv][e].y = y | (rank << kEntRankShift);
      }
    }
    __syncthreads();
    // one claim per token on its row's list; a token whose wave's list
    // overflowed, or whose row's list ran out, sends its row to the exact path
    const int trow0 = blockIdx.y * TPB;
    if (tid < TPB) {
      const int t = trow0 + tid;
      const uint32_t n = lcnt[tid];
      uint32_t base = 0u;
      if (t < rows) {
        if (n > 0u) base = atomicAdd(sel.count + t, n);
        if (wtot[tid / TPW] > (uint32_t)WCAP || base + n > (uint32_t)kCandCap) sel.fail[t] = 1u;
      }
      lbase[tid] = base;
    }
    __syncthreads();
    for (int x = tid; x < 4 * WCAP; x += 256) {
      const int wv = x / WCAP, e = x - wv * WCAP;
      if ((uint32_t)e < min(wtot[wv], (uint32_t)WCAP)) {
        const uint2 v = wbuf[wv][e];
        const uint32_t tk = (v.y >> kEntTokShift) & 63u;
        const uint32_t pos = lbase[tk] + (v.y >> kEntRankShift);
        if (trow0 + (int)tk < rows && pos < (uint32_t)kCandCap)
          sel.cand[(int64_t)(trow0 + (int)tk) * kCandCap + pos] =
              make_uint2(score_key(__uint_as_float(v.x)),
                         (uint32_t)(start + (v.y & ((1u << kEntTokShift) - 1u))));
      }
    }
  }
}

bool index_tokens_pass(bool pool, int32_t T, int32_t HI, int32_t DI, int32_t row0) {
  return !pool && HI <= 4 && T >= 32 && T % 32 == 0 && row0 % 32 == 0 && DI == 128;
}

hipError_t launch_index_tokens(const uint8_t* codes, const uint8_t* scales, int64_t cap,
                               int32_t rows, int32_t T, const uint16_t* q_idx, const float* w,
                               int32_t HI, const int32_t* n_valid, int32_t nv_add, int64_t n_max,
                               float* scores, int64_t n_out, hipStream_t st, int32_t row0,
                               bool last) {
  constexpr int NG = kPrefillGroups;
  const int32_t pchunk = kPrefillChunk;
  const dim3 g2((unsigned)((n_max + pchunk - 1) / pchunk), (unsigned)((rows + 16 * NG - 1) / (16 * NG)));
  CSA2_KERNEL(true, last, (index_score_tokens_kernel<1, NG, kTokAll>), g2, dim3(256), 0, st,
              codes, scales, cap, q_idx, w, HI, T, n_valid, nv_add, rows, scores, n_out, pchunk,
              row0, nullptr, SampledSel{});
  return hipGetLastError();
}

// ------------------------------------------------ sampled prefill selection
bool sampled_select_shapes(int32_t rows, int32_t T, int32_t HI, int32_t DI, int32_t row0,
                           int32_t K, int64_t n_max) {
  return HI <= 4 && T >= 32 && T % 32 == 0 && row0 % 32 == 0 && DI == 128 && K >= 1 &&
         K <= 2048 && n_max >= 32768 && n_max <= kRowTopkMaxN && rows >= 1;
}

bool sampled_select_pass(int32_t rows, int32_t T, int32_t HI, int32_t DI, int32_t row0,
                         int32_t K, int64_t n_max) {
  const int32_t f = topk_variant_forced();
  if (f != kTopkAuto && f != kTopkSampled && f != kTopkSampledFallback) return false;
  return sampled_select_shapes(rows, T, HI, DI, row0, K, n_max);
}

static hipError_t launch_tokens_mode(int mode, const uint8_t* codes, const uint8_t* scales,
                                     int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                                     const float* w, int32_t HI, const int32_t* n_valid,
                                     int32_t nv_add, int64_t slots, float* scores, int64_t n_out,
                                     const uint32_t* fail, const SampledSel& sel, hipStream_t st,
                                     int32_t row0) {
  constexpr int NG = kPrefillGroups;
  // the sample scan has 1/kSampleStride of the slots: smaller chunks keep
  // its grid as wide as the full scan's
  const int32_t pchunk = mode == kTokSample ? kPrefillChunk / 4 : kPrefillChunk;
  if (slots <= 0 || rows <= 0) return hipSuccess;
  const dim3 g2((unsigned)((slots + pchunk - 1) / pchunk), (unsigned)((rows + 16 * NG - 1) / (16 * NG)));
  if (mode == kTokAll)
    CSA2_KERNEL(true, true, (index_score_tokens_kernel<1, NG, kTokAll>), g2, dim3(256), 0, st,
                codes, scales, cap, q_idx, w, HI, T, n_valid, nv_add, rows, scores, n_out, pchunk,
                row0, fail, sel);
  else if (mode == kTokSample)
    CSA2_KERNEL(true, true, (index_score_tokens_kernel<1, NG, kTokSample>), g2, dim3(256), 0, st,
                codes, scales, cap, q_idx, w, HI, T, n_valid, nv_add, rows, scores, n_out, pchunk,
                row0, fail, sel);
  else
    CSA2_KERNEL(true, true, (index_score_tokens_kernel<1, NG, kTokCand>), g2, dim3(256), 0, st,
                codes, scales, cap, q_idx, w, HI, T, n_valid, nv_add, rows, scores, n_out, pchunk,
                row0, fail, sel);
  return hipGetLastError();
}

hipError_t launch_index_sample(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                               int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                               const float* w, int32_t HI, const int32_t* n_valid,
                               int32_t nv_add, int64_t n_max, const SampledSel& sel,
                               hipStream_t st, int32_t row0) {
  if (DI != 128 || HI > 4) return hipErrorInvalidValue;
  const int64_t ns = (n_max + kSampleStride - 1) / kSampleStride;
  // the kernel clamps each token's range to n_out (here: the cache's slots)
  return launch_tokens_mode(kTokSample, codes, scales, cap, rows, T, q_idx, w, HI, n_valid, nv_add,
                            ns, nullptr, n_max, nullptr, sel, st, row0);
}

hipError_t launch_index_candidates(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                                   int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                                   const float* w, int32_t HI, const int32_t* n_valid,
                                   int32_t nv_add, int64_t n_max, const SampledSel& sel,
                                   hipStream_t st, int32_t row0) {
  if (DI != 128 || HI > 4) return hipErrorInvalidValue;
  return launch_tokens_mode(kTokCand, codes, scales, cap, rows, T, q_idx, w, HI, n_valid, nv_add,
                            n_max, nullptr, n_max, nullptr, sel, st, row0);
}

hipError_t launch_index_score_failed(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                                     int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                                     const float* w, int32_t HI, const int32_t* n_valid,
                                     int32_t nv_add, int64_t n_max, float* scores, int64_t n_out,
                                     const uint32_t* fail, hipStream_t st, int32_t row0) {
  if (DI != 128 || HI > 4) return hipErrorInvalidValue;
  return launch_tokens_mode(kTokAll, codes, scales, cap, rows, T, q_idx, w, HI, n_valid, nv_add,
                            n_max, scores, n_out, fail, SampledSel{}, st, row0);
}

}  // namespace csa2
