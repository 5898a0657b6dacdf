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
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

template <int NCH, int TPA, int GT>  // 128-channel chunks, tiles per accumulator, tiles per group
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t cap,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int32_t HI, int32_t T,
    const int32_t* __restrict__ n_valid, const int32_t* __restrict__ pool, int32_t P,
    int32_t nv_add, float* __restrict__ scores, int64_t n_out, uint32_t* __restrict__ hist,
    int64_t hist_stride, int32_t chunk, int32_t row0) {
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
  const int64_t nv = min(min((int64_t)n_valid[r] + nv_add, n_out), pool ? (int64_t)P : cap);
  const int64_t start = (int64_t)blockIdx.x * chunk;
  if (start >= nv) return;  // uniform for the whole block
  const int64_t end = min(nv, start + chunk);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;

  if (hist) {
    for (int k = tid; k < kHistBins; k += 256) lhist[k] = 0u;
  }

  const uint8_t* cbase = codes + (int64_t)b * cap * ROWB;
  const uint8_t* sbase = scales + (int64_t)b * cap * ROWS;
  const int32_t* prow = pool ? pool + (int64_t)r * P : nullptr;
  float* srow = scores + (int64_t)r * n_out;

  // Each wave takes groups of GT consecutive tiles (GT KiB of contiguous
  // codes for 128 channels in flat mode); the four waves of a round cover
  // 4*GT consecutive tiles.  The next group's loads are issued before the
  // current group is computed.
  const int ntiles = (int)((end - start + 15) >> 4);
  const int nrounds = (ntiles + 4 * GT - 1) / (4 * GT);
  auto row_of = [&](int tile) -> int64_t {
    int64_t s = start + (int64_t)tile * 16 + i;
    if (s >= end) s = end - 1;  // clamp: keep the load in bounds, masked later
    return prow ? (int64_t)prow[s] : s;
  };
  // The scale bytes of lane (i, g) are bytes 2g, 2g+1 of each chunk's
  // scales; they are fetched as the aligned 32-bit word holding them, so
  // nothing has to wait for the loads until the group is computed.
  auto load_group = [&](int rnd, u32x4 (&cw)[GT][NCH], uint32_t (&sw)[GT][NCH]) {
    int64_t rows[GT];
#pragma unroll
    for (int t = 0; t < GT; ++t) rows[t] = row_of((rnd * 4 + wave) * GT + t);
#pragma unroll
    for (int t = 0; t < GT; ++t) {
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

  u32x4 cw[GT][NCH], ncw[GT][NCH];
  uint32_t sw[GT][NCH], nsw[GT][NCH];
  // the first group is requested before the query is prepared, so the
  // scan's first HBM round trip overlaps the query's
  if (nrounds > 0) load_group(0, cw, sw);

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

  for (int rnd = 0; rnd < nrounds; ++rnd) {
    if (rnd + 1 < nrounds) load_group(rnd + 1, ncw, nsw);
#pragma unroll
    for (int a = 0; a < NACC; ++a) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sl = 0; sl < TPA; ++sl) {
        const int t = a * TPA + sl;
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          const uint32_t s2b = sw[t][c2] >> sshift;
          const f16x2 s_lo = scale_pair(s2b & 0xFFu);
          const f16x2 s_hi = scale_pair((s2b >> 8) & 0xFFu);
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
      if (owner && s < end) {
        srow[s] = part;
        if (hist) atomicAdd(&lhist[score_key(part) >> kHistShift], 1u);
      }
    }
    if (rnd + 1 < nrounds) {
#pragma unroll
      for (int t = 0; t < GT; ++t)
#pragma unroll
        for (int c2 = 0; c2 < NCH; ++c2) {
          cw[t][c2] = ncw[t][c2];
          sw[t][c2] = nsw[t][c2];
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
#define CSA2_IS_LAUNCH(NCH, TPA, GT)                                                           \
  CSA2_KERNEL(true, true, (index_score_kernel<NCH, TPA, GT>), grid, block, 0, st, codes, scales, cap, \
                     q_idx, w, HI, T, n_valid, pool, P, nv_add, scores, n_out, hist,             \
                     hist_stride, chunk, row0)
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
