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
// 128 channels) and is HBM-bound.  One wave scores 16 positions per step with
// 4 fp16 MFMA 16x16x32 (rows = indexer heads, columns = positions, k =
// channels): lane (i, g) loads the 16 code bytes [16g, 16g+16) of position i
// -- the 64 lanes together read 1 KiB of contiguous codes -- plus the two
// scale bytes of its 32 channels, and dequantizes them exactly to fp16.
// Channel 32g + 8kk + j of the row feeds k-slot 8g + j of MFMA kk, and the
// query fragments use the same mapping.
//
// The block also builds a histogram of the top 12 bits of each score's
// ordered key and adds it to a per-row global histogram, which the Top-K
// select pass then uses to find the bin holding the K-th score.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

template <int NCH>  // index-key channels / 128
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t cap,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int32_t HI, int32_t T,
    const int32_t* __restrict__ n_valid, const int32_t* __restrict__ pool, int32_t P,
    int32_t nv_add, float* __restrict__ scores, int64_t n_out, uint32_t* __restrict__ hist,
    int64_t hist_stride, int32_t chunk, int32_t row0) {
  constexpr int DI = 128 * NCH;
  constexpr int ROWB = DI / 2;    // code bytes per row
  constexpr int ROWS = DI / 16;   // scale bytes per row
  __shared__ uint32_t lhist[kHistBins];

  const int r = blockIdx.y;
  const int b = (row0 + r) / T;
  // visible entries, clamped to what the score row and the key list hold
  const int64_t nv = min(min((int64_t)n_valid[r] + nv_add, n_out), pool ? (int64_t)P : cap);
  const int64_t start = (int64_t)blockIdx.x * chunk;
  if (start >= nv) return;  // uniform for the whole block
  const int64_t end = min(nv, start + chunk);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;

  if (hist) {
    for (int k = tid; k < kHistBins; k += 256) lhist[k] = 0u;
  }

  // ---- query fragments: head i (zero rows for i >= HI), scaled into fp16.
  f16x8 qa[NCH][4];
  int qexp;
  {
    float vals[NCH][4][8];
    float amax = 0.0f;
    const uint16_t* qr = q_idx + ((int64_t)r * HI + (i < HI ? i : 0)) * DI;
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
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          qa[c2][kk][j] = (i < HI) ? (_Float16)ldexpf(vals[c2][kk][j], qexp) : (_Float16)0.0f;
  }
  // Accumulator rows held by this lane: heads 4g + rr.  Fetch their weights
  // and the exponent that undoes the query scaling.
  float wr[4];
  int er[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int h = 4 * g + rr;
    er[rr] = __shfl(qexp, h & 15, kWave);
    wr[rr] = (h < HI) ? w[(int64_t)r * HI + h] : 0.0f;
  }
  if (hist) __syncthreads();

  const uint8_t* cbase = codes + (int64_t)b * cap * ROWB;
  const uint8_t* sbase = scales + (int64_t)b * cap * ROWS;
  const int32_t* prow = pool ? pool + (int64_t)r * P : nullptr;
  float* srow = scores + (int64_t)r * n_out;

  // Each wave takes groups of G consecutive tiles (G KiB of contiguous codes
  // in flat mode); the four waves of a round cover 4G consecutive tiles.
  // The next group's loads are issued before the current group is computed,
  // so about 2G tiles per wave are in flight.
  constexpr int G = kScoreGroup;
  const int ntiles = (int)((end - start + 15) >> 4);
  const int nrounds = (ntiles + 4 * G - 1) / (4 * G);
  auto row_of = [&](int tile) -> int64_t {
    int64_t s = start + (int64_t)tile * 16 + i;
    if (s >= end) s = end - 1;  // clamp: keep the load in bounds, masked later
    return prow ? (int64_t)prow[s] : s;
  };
  // The scale bytes of lane (i, g) are bytes 2g, 2g+1 of the row's scales;
  // they are fetched as the aligned 32-bit word holding them, so nothing has
  // to wait for the loads until the group is computed.
  auto load_group = [&](int rnd, u32x4 (&cw)[G][NCH], uint32_t (&sw)[G][NCH]) {
    int64_t rows[G];
#pragma unroll
    for (int j = 0; j < G; ++j) rows[j] = row_of((rnd * 4 + wave) * G + j);
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) {
        cw[j][c2] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(cbase + rows[j] * ROWB + 64 * c2 + 16 * g));
        sw[j][c2] =
            *reinterpret_cast<const uint32_t*>(sbase + rows[j] * ROWS + 8 * c2 + 4 * (g >> 1));
      }
    }
  };
  const int sshift = 16 * (g & 1);

  u32x4 cw[G][NCH], ncw[G][NCH];
  uint32_t sw[G][NCH], nsw[G][NCH];
  if (nrounds > 0) load_group(0, cw, sw);
  for (int rnd = 0; rnd < nrounds; ++rnd) {
    if (rnd + 1 < nrounds) load_group(rnd + 1, ncw, nsw);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c2 = 0; c2 < NCH; ++c2) {
        const uint32_t s2b = sw[j][c2] >> sshift;
        const f16x2 s_lo = scale_pair(s2b & 0xFFu);
        const f16x2 s_hi = scale_pair((s2b >> 8) & 0xFFu);
        acc = mfma16x16x32(qa[c2][0], fp4x8_to_f16(cw[j][c2].x, s_lo), acc);
        acc = mfma16x16x32(qa[c2][1], fp4x8_to_f16(cw[j][c2].y, s_lo), acc);
        acc = mfma16x16x32(qa[c2][2], fp4x8_to_f16(cw[j][c2].z, s_hi), acc);
        acc = mfma16x16x32(qa[c2][3], fp4x8_to_f16(cw[j][c2].w, s_hi), acc);
      }
      float part = 0.0f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part += wr[rr] * fmaxf(ldexpf(acc[rr], -er[rr]), 0.0f);
      part += shfl_xor(part, 16);
      part += shfl_xor(part, 32);
      const int64_t s = start + (int64_t)((rnd * 4 + wave) * G + j) * 16 + i;
      if (g == 0 && s < end) {
        srow[s] = part;
        if (hist) atomicAdd(&lhist[score_key(part) >> kHistShift], 1u);
      }
    }
    if (rnd + 1 < nrounds) {
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          cw[j][c2] = ncw[j][c2];
          sw[j][c2] = nsw[j][c2];
        }
    }
  }
  if (hist) {
    __syncthreads();
    uint32_t* gh = hist + (int64_t)r * hist_stride + (blockIdx.x % kHistCopies) * kHistBins;
    for (int k = tid; k < kHistBins; k += 256) {
      const uint32_t c = lhist[k];
      if (c) atomicAdd(gh + k, c);
    }
  }
}

hipError_t launch_index_score(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                              int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                              const float* w, int32_t HI, const int32_t* n_valid,
                              int32_t nv_add, const int32_t* pool, int32_t P, int64_t n_max,
                              float* scores, int64_t n_out, uint32_t* hist, int64_t hist_stride,
                              hipStream_t st, int32_t row0) {
  const int32_t chunk = kScoreChunk;
  const int64_t nchunks = (n_max + chunk - 1) / chunk;
  if (nchunks == 0 || rows == 0) return hipSuccess;
  const dim3 grid((unsigned)nchunks, (unsigned)rows), block(256);
  switch (DI / 128) {
    case 1:
      hipLaunchKernelGGL(index_score_kernel<1>, grid, block, 0, st, codes, scales, cap, q_idx, w,
                         HI, T, n_valid, pool, P, nv_add, scores, n_out, hist, hist_stride, chunk, row0);
      break;
    case 2:
      hipLaunchKernelGGL(index_score_kernel<2>, grid, block, 0, st, codes, scales, cap, q_idx, w,
                         HI, T, n_valid, pool, P, nv_add, scores, n_out, hist, hist_stride, chunk, row0);
      break;
    case 3:
      hipLaunchKernelGGL(index_score_kernel<3>, grid, block, 0, st, codes, scales, cap, q_idx, w,
                         HI, T, n_valid, pool, P, nv_add, scores, n_out, hist, hist_stride, chunk, row0);
      break;
    case 4:
      hipLaunchKernelGGL(index_score_kernel<4>, grid, block, 0, st, codes, scales, cap, q_idx, w,
                         HI, T, n_valid, pool, P, nv_add, scores, n_out, hist, hist_stride, chunk, row0);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa2
