// index_score.hip -- indexer scoring of cached positions (decode).
//
// For a query row r and every listed position s:
//     score = sum_h w_h * max(0, q_h . k_s)
// over FP4 index keys (helmcode.com/deepseek-v41-flash, section "03 · CSA2":
// a Reindex layer scores the positions again with its own query;
// louisbouchard.ai/deepseek-v41-flash-kv-cache-writing-benchmark, "Share the
// cache and the search work": the first indexing layer scans the whole
// visible context, later ones only a candidate pool).
//
// The scan streams 72 bytes per position (64 code bytes + 8 scale bytes for
// 128 channels) and is HBM-bound.  MFMA 16x16x32 (fp16 in, fp32 out) takes
// rows = indexer heads, columns = 16 positions (a tile), k = channels.  With
// at most 16/TPA heads, TPA tiles share one accumulator: tile slot j's heads
// sit in rows [j*16/TPA, (j+1)*16/TPA) of the A operand (zero elsewhere), so
// after the slots' MFMAs lane (i, g) holds rows 4g..4g+3 of position i and,
// with four heads, every lane finishes one score by itself.
//
// Lane (i, g) of a tile loads the 16 code bytes [16g, 16g+16) of position i
// -- the 64 lanes together read 1 KiB of contiguous codes -- plus the aligned
// scale word holding its two scale bytes, and dequantizes them exactly to
// fp16.  Channel 32g + 8kk + j of a 128-channel chunk feeds k-slot 8g + j of
// MFMA kk, and the query fragments use the same mapping.  The query is
// scaled per head by a power of two into fp16 range; that factor is folded
// into the head weight (exact unless that weight underflows).
//
// The block also builds a histogram of the top 12 bits of each score's
// ordered key and adds it to one of the row's global histogram copies, which
// the Top-K select pass then uses to find the bin holding the K-th score.
#include <type_traits>

#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

// Two scale bytes (low half of `word`) as fp16 (exact: E4M3 lies inside
// fp16's normal range).
__device__ __forceinline__ f16x2 scale_pair2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
}

template <int NCH, int TPA, int GT, bool POOL>  // 128-channel chunks, tiles per accumulator,
                                                // tiles per group, positions from a pool list
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t cap,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int32_t HI, int32_t T,
    const int32_t* __restrict__ n_valid, const int32_t* __restrict__ pool, int32_t P,
    int32_t nv_add, float* __restrict__ scores, int64_t n_out, uint32_t* __restrict__ hist,
    int64_t hist_stride, int32_t hist_copies, int32_t chunk, int32_t row0) {
  constexpr int DI = 128 * NCH;
  constexpr int ROWB = DI / 2;    // code bytes per row
  constexpr int ROWS = DI / 16;   // scale bytes per row
  constexpr int HG = 16 / TPA;    // MFMA rows per tile slot
  constexpr int GPS = HG / 4;     // lane groups g covering one slot
  constexpr int NACC = GT / TPA;  // accumulators per group
  static_assert(GT % TPA == 0 && HG >= 4, "tile packing");
  __shared__ uint32_t lhist[kHistBins];

  const int r = blockIdx.y;
  const int b = (row0 + r) / T;
  // visible entries, clamped to what the score row and the key list hold
  const int64_t nv = min(min((int64_t)n_valid[r] + nv_add, n_out), POOL ? (int64_t)P : cap);
  const int64_t start = (int64_t)blockIdx.x * chunk;
  if (start >= nv) return;  // uniform for the whole block
  const int64_t end = min(nv, start + chunk);

  // the wave index is uniform: kept in a scalar register, the whole-group
  // test below is a scalar branch
  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;

  if (hist) {
    for (int k = tid; k < kHistBins; k += 256) lhist[k] = 0u;
  }

  const uint8_t* cbase = codes + (int64_t)b * cap * ROWB;
  const uint8_t* sbase = scales + (int64_t)b * cap * ROWS;
  const int32_t* prow = POOL ? pool + (int64_t)r * P : nullptr;
  float* srow = scores + (int64_t)r * n_out;

  // Each wave takes groups of GT consecutive tiles (GT KiB of contiguous
  // codes for 128 channels in flat mode); the four waves of a round cover
  // 4*GT consecutive tiles.  The next group's loads are issued before the
  // current group is computed, into the other of two register buffers.
  // The scale bytes of lane (i, g) are bytes 2g, 2g+1 of each chunk's
  // scales; they are fetched as the aligned 32-bit word holding them.
  const int ntiles = (int)((end - start + 15) >> 4);
  const int nrounds = (ntiles + 4 * GT - 1) / (4 * GT);
  // Whole chunks of a flat scan read every group at fixed offsets from one
  // address; the last chunk of a row (and pool lists) compute each tile's
  // rows, clamped to the range (lanes past the end reload the last position;
  // their scores are masked).  Each variant is straight-line code.
  auto load_group = [&](auto per_tile, int rnd, u32x4 (&cw)[GT][NCH], uint32_t (&sw)[GT][NCH]) {
    const int tile0 = (rnd * 4 + wave) * GT;
    if constexpr (!decltype(per_tile)::value) {
      const int64_t p0 = start + (int64_t)tile0 * 16;
      const uint8_t* cp = cbase + (p0 + i) * ROWB + 16 * g;
      const uint8_t* sp = sbase + (p0 + i) * ROWS + 4 * (g >> 1);
#pragma unroll
      for (int t = 0; t < GT; ++t)
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          cw[t][c2] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(cp + t * 16 * ROWB + 64 * c2));
          sw[t][c2] = *reinterpret_cast<const uint32_t*>(sp + t * 16 * ROWS + 8 * c2);
        }
    } else {
      int64_t rows[GT];
#pragma unroll
      for (int t = 0; t < GT; ++t) {
        const int64_t s = min(start + (int64_t)(tile0 + t) * 16 + i, end - 1);
        rows[t] = POOL ? (int64_t)prow[s] : s;
      }
#pragma unroll
      for (int t = 0; t < GT; ++t)
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          cw[t][c2] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(cbase + rows[t] * ROWB + 64 * c2 + 16 * g));
          sw[t][c2] =
              *reinterpret_cast<const uint32_t*>(sbase + rows[t] * ROWS + 8 * c2 + 4 * (g >> 1));
        }
    }
  };
  const int sshift = 16 * (g & 1);

  const bool whole = !POOL && chunk == kScoreChunk && end - start == chunk;  // block-uniform
  u32x4 cwA[GT][NCH], cwB[GT][NCH];
  uint32_t swA[GT][NCH], swB[GT][NCH];
  // the first group is requested before the query is prepared, so the
  // scan's first HBM round trip overlaps the query's
  if (nrounds > 0) {
    if (whole) load_group(std::false_type{}, 0, cwA, swA);
    else load_group(std::true_type{}, 0, cwA, swA);
  }

  // ---- query fragments: MFMA row i holds head i % HG of tile slot i / HG
  const int hrow = i % HG, srow_slot = i / HG;
  f16x8 qv[TPA][NCH][4];
  int qexp;
  {
    float vals[NCH][4][8];
    float amax = 0.0f;
    const bool live = hrow < HI;
    const uint16_t* qr = q_idx + ((int64_t)r * HI + (live ? hrow : 0)) * DI;
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 raw = *reinterpret_cast<const uint4*>(qr + 128 * c2 + 32 * g + 8 * kk);
        const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vals[c2][kk][2 * j] = bf16_to_f32(wd[j] & 0xFFFFu);
          vals[c2][kk][2 * j + 1] = bf16_to_f32(wd[j] >> 16);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(vals[c2][kk][j]));
      }
    amax = fmaxf(amax, shfl_xor(amax, 16));
    amax = fmaxf(amax, shfl_xor(amax, 32));
    qexp = fp16_exponent_for(amax);
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f16x8 a;
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = live ? (_Float16)ldexpf(vals[c2][kk][j], qexp) : (_Float16)0.0f;
#pragma unroll
        for (int sl = 0; sl < TPA; ++sl) qv[sl][c2][kk] = (sl == srow_slot) ? a : f16x8{};
      }
  }
  // Accumulator rows of lane (i, g): 4g + rr = slot g / GPS, head 4(g % GPS) + rr.
  // Head weights carry the factor that undoes the query scaling.
  float wq[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int h = 4 * (g % GPS) + rr;
    const int e = __shfl(qexp, h, kWave);  // lane h holds head h of slot 0
    wq[rr] = (h < HI) ? ldexpf(w[(int64_t)r * HI + h], -e) : 0.0f;
  }
  const int my_slot = g / GPS;
  const bool owner = (g % GPS) == 0;
  if (hist) __syncthreads();

  auto compute_group = [&](int rnd, const u32x4 (&cw)[GT][NCH], const uint32_t (&sw)[GT][NCH]) {
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sl = 0; sl < TPA; ++sl) {
        const int t = a * TPA + sl;
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          const f16x2 sp = scale_pair2(sw[t][c2] >> sshift);
          const f16x2 s_lo = {sp[0], sp[0]}, s_hi = {sp[1], sp[1]};
          acc = mfma16x16x32(qv[sl][c2][0], fp4x8_to_f16(cw[t][c2].x, s_lo), acc);
          acc = mfma16x16x32(qv[sl][c2][1], fp4x8_to_f16(cw[t][c2].y, s_lo), acc);
          acc = mfma16x16x32(qv[sl][c2][2], fp4x8_to_f16(cw[t][c2].z, s_hi), acc);
          acc = mfma16x16x32(qv[sl][c2][3], fp4x8_to_f16(cw[t][c2].w, s_hi), acc);
        }
      }
      float part = 0.0f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part += wq[rr] * fmaxf(acc[rr], 0.0f);
      if constexpr (GPS >= 2) part += shfl_xor(part, 16);
      if constexpr (GPS >= 4) part += shfl_xor(part, 32);
      const int64_t s = start + (int64_t)((rnd * 4 + wave) * GT + a * TPA + my_slot) * 16 + i;
      // Lanes past the end scored the clamped last position, so storing at the
      // clamped slot writes the same value; an unconditional store keeps the
      // count of outstanding memory operations fixed, so waiting for the next
      // group's loads does not also wait for these stores.
      if (owner) srow[min(s, end - 1)] = part;
      if (owner && s < end && hist) atomicAdd(&lhist[score_key(part) >> kHistShift], 1u);
    }
  };
  // Rounds in pairs, alternating the two buffers.  A whole chunk has a fixed
  // number of rounds and is unrolled completely, so every load and wait is
  // placed at compile time.
  if (whole) {
    constexpr int NR = kScoreChunk / (64 * GT);
    static_assert(NR % 2 == 0 && NR * 64 * GT == kScoreChunk, "whole chunks");
#pragma unroll
    for (int rnd = 0; rnd < NR; rnd += 2) {
      load_group(std::false_type{}, rnd + 1, cwB, swB);
      compute_group(rnd, cwA, swA);
      if (rnd + 2 < NR) load_group(std::false_type{}, rnd + 2, cwA, swA);
      compute_group(rnd + 1, cwB, swB);
    }
  } else {
    for (int rnd = 0; rnd < nrounds; rnd += 2) {
      if (rnd + 1 < nrounds) load_group(std::true_type{}, rnd + 1, cwB, swB);
      compute_group(rnd, cwA, swA);
      if (rnd + 1 >= nrounds) break;
      if (rnd + 2 < nrounds) load_group(std::true_type{}, rnd + 2, cwA, swA);
      compute_group(rnd + 1, cwB, swB);
    }
  }
  if (hist) {
    __syncthreads();
    uint32_t* gh = hist + (int64_t)r * hist_stride + (blockIdx.x % hist_copies) * kHistBins;
    // every bin of this thread is read before any is added, so the LDS reads
    // overlap; bin tid + 256 j keeps each atomic instruction on 256
    // contiguous bytes
    uint32_t cv[kHistBins / 256];
#pragma unroll
    for (int j = 0; j < kHistBins / 256; ++j) cv[j] = lhist[tid + 256 * j];
#pragma unroll
    for (int j = 0; j < kHistBins / 256; ++j)
      if (cv[j]) atomicAdd(gh + tid + 256 * j, cv[j]);
  }
}


// ---------------------------------------------------------------- prefill
// Row groups of 4 tokens per wave, and positions per block, of the prefill
// scoring kernel (4 groups: 178 registers, two waves per SIMD; 8 groups need
// 448 and leave one).
constexpr int kPrefillGroups = 4;
constexpr int32_t kPrefillChunk = 512;

// Many query tokens of one sequence score the same positions, so the scan
// becomes a tokens x positions contraction: MFMA rows = 4 tokens x 4 heads,
// columns = 16 positions, k = channels.  A wave holds the query fragments of
// 4 NG tokens (NG row groups) in registers and dequantizes each key tile once
// for all of them: 4 NG MFMAs per 16-position tile.  Lane (i, g) of row group
// j then holds the four heads of token 4j + g at position i, so the score
// needs no cross-lane sum.  Token t sees positions below n_valid[t] + nv_add.
// The fragments take 16 NG registers, so NG trades the dequantisation's share
// against waves per SIMD.
template <int NCH, int NG>
__global__ __launch_bounds__(256) void index_score_tokens_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t cap,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int32_t HI, int32_t T,
    const int32_t* __restrict__ n_valid, int32_t nv_add, int32_t rows, float* __restrict__ scores,
    int64_t n_out, int32_t chunk, int32_t row0) {
  constexpr int DI = 128 * NCH;
  constexpr int ROWB = DI / 2;
  constexpr int ROWS = DI / 16;
  constexpr int TPW = 4 * NG;  // tokens per wave
  static_assert(TPW <= 32, "the visible-length reduction covers 32 lanes");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int rbase = blockIdx.y * 4 * TPW + wave * TPW;  // first token row of this wave
  if (rbase >= rows) return;                             // no block-wide barrier below
  const int b = (row0 + rbase) / T;                      // the wave's tokens share the sequence
  // the wave's longest visible length
  int64_t nvmax;
  {
    const int tr = min(rbase + (lane & (TPW - 1)), rows - 1);
    int64_t m = min(min((int64_t)n_valid[tr] + nv_add, n_out), cap);
#pragma unroll
    for (int d = 1; d < TPW; d <<= 1) m = max(m, (int64_t)__shfl_xor(m, d, kWave));
    nvmax = m;
  }
  const int64_t start = (int64_t)blockIdx.x * chunk;
  if (start >= nvmax) return;
  const int64_t end = min(nvmax, start + chunk);

  // query fragments: row i of group j = token 4j + i/4, head i%4
  f16x8 qv[NG][NCH][4];
  float wq[NG][4];
  {
    const int h = i & 3;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int t = min(rbase + 4 * j + (i >> 2), rows - 1);
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
      const int te = min(rbase + 4 * j + g, rows - 1);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int e = __shfl(qexp, 4 * g + rr, kWave);
        const float wv = w[(int64_t)te * HI + min(rr, HI - 1)];  // unconditional load
        wq[j][rr] = (rr < HI) ? ldexpf(wv, -e) : 0.0f;
      }
    }
  }

  const uint8_t* cbase = codes + (int64_t)b * cap * ROWB;
  const uint8_t* sbase = scales + (int64_t)b * cap * ROWS;
  const int sshift = 16 * (g & 1);
  const int ntiles = (int)((end - start + 15) >> 4);
  auto load_tile = [&](int tile, u32x4 (&cw)[NCH], uint32_t (&sw)[NCH]) {
    int64_t s = start + (int64_t)tile * 16 + i;
    if (s >= end) s = end - 1;
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
      cw[c2] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(cbase + s * ROWB + 64 * c2 + 16 * g));
      sw[c2] = *reinterpret_cast<const uint32_t*>(sbase + s * ROWS + 8 * c2 + 4 * (g >> 1));
    }
  };
  // a ring of PF tiles in flight ahead of the one being computed
  constexpr int PF = 4;
  u32x4 cw[PF][NCH];
  uint32_t sw[PF][NCH];
#pragma unroll
  for (int p = 0; p < PF; ++p) load_tile(min(p, max(ntiles - 1, 0)), cw[p], sw[p]);
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
      const int64_t s = start + (int64_t)tile * 16 + i;
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) acc = mfma16x16x32(qv[j][c2][kk], kb[c2][kk], acc);
        float part = 0.0f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) part += wq[j][rr] * fmaxf(acc[rr], 0.0f);
        // Unconditional (clamped) store, as in index_score_kernel: tokens past
      // the last row computed that row's score (clamped query and weights),
      // and slots past a token's visible range are never read for it.
      scores[(int64_t)min(rbase + 4 * j + g, rows - 1) * n_out + min(s, end - 1)] = part;
      }
    }
  }
}

hipError_t launch_index_score(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                              int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                              const float* w, int32_t HI, const int32_t* n_valid,
                              int32_t nv_add, const int32_t* pool, int32_t P, int64_t n_max,
                              float* scores, int64_t n_out, uint32_t* hist, int64_t hist_stride,
                              int32_t hist_copies, hipStream_t st, int32_t row0) {
  if (n_max <= 0 || rows == 0) return hipSuccess;
  // Prefill chunks (32 or more tokens per sequence, whole waves of one
  // sequence, 128-channel keys) take the tokens x positions kernel; the Top-K histogram is then
  // built from the written scores.
  if (!pool && HI <= 4 && T >= 32 && T % 32 == 0 && row0 % 32 == 0 && DI == 128) {
    constexpr int NG = kPrefillGroups;
    const int32_t pchunk = kPrefillChunk;
    const dim3 g2((unsigned)((n_max + pchunk - 1) / pchunk), (unsigned)((rows + 16 * NG - 1) / (16 * NG)));
    CSA2_KERNEL(true, !hist, (index_score_tokens_kernel<1, NG>), g2, dim3(256), 0, st, codes,
                scales, cap, q_idx, w, HI, T, n_valid, nv_add, rows, scores, n_out, pchunk, row0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !hist) return e;
    return launch_topk_hist(scores, rows, n_out, n_valid, nv_add, n_max, hist, hist_stride,
                            hist_copies, st, false);
  }
  const int32_t chunk = kScoreChunk;
  const int64_t nchunks = (n_max + chunk - 1) / chunk;
  const dim3 grid((unsigned)nchunks, (unsigned)rows), block(256);
#define CSA2_IS_LAUNCH(NCH, TPA, GT)                                                           \
  do {                                                                                         \
    if (pool)                                                                                  \
      CSA2_KERNEL(true, true, (index_score_kernel<NCH, TPA, GT, true>), grid, block, 0, st,    \
                  codes, scales, cap, q_idx, w, HI, T, n_valid, pool, P, nv_add, scores, n_out, \
                  hist, hist_stride, hist_copies, chunk, row0);                                \
    else                                                                                       \
      CSA2_KERNEL(true, true, (index_score_kernel<NCH, TPA, GT, false>), grid, block, 0, st,   \
                  codes, scales, cap, q_idx, w, HI, T, n_valid, pool, P, nv_add, scores, n_out, \
                  hist, hist_stride, hist_copies, chunk, row0);                                \
  } while (0)
  switch (DI / 128) {
    case 1:
      if (HI <= 4) CSA2_IS_LAUNCH(1, 4, 8);
      else if (HI <= 8) CSA2_IS_LAUNCH(1, 2, 8);
      else CSA2_IS_LAUNCH(1, 1, 4);
      break;
    case 2:
      if (HI <= 8) CSA2_IS_LAUNCH(2, 2, 4);
      else CSA2_IS_LAUNCH(2, 1, 4);
      break;
    case 3:
      CSA2_IS_LAUNCH(3, 1, 2);
      break;
    case 4:
      CSA2_IS_LAUNCH(4, 1, 2);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef CSA2_IS_LAUNCH
  return hipGetLastError();
}

}  // namespace csa2
