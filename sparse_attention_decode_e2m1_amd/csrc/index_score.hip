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
#include "csa2_quant.hpp"

namespace csa2 {

// Two scale bytes (low half of `word`) as fp16 (exact: E4M3 lies inside
// fp16's normal range).
__device__ __forceinline__ f16x2 scale_pair2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
}

// A Full layer's decode step writes its new rows inside the scan launch
// (128-channel index keys, 1, 2 or 4 indexer heads): the last wave of some
// of the query row's blocks quantizes them, one element per lane (exactly
// as the quantize-on-write kernels do).  The first block's wave takes the
// index key (two passes of 64 channels) and scores the new position p =
// q_pos[r] from the key it has just quantized; pass j of the main-KV row
// (64 channels) goes to block (1 + j) mod (the row's blocks).  No block of
// the launch reads a cache row while it is being written: every block of
// the row scans positions [0, p).  A wave issues these loads first, ahead
// of its scan loads, computes once its query is in, stores after its scan
// (stores share the load counter and would hold up its later waits), and
// never waits on the rest of its block.  The score is
// sum_h w_h * max(0, q_h . k) with the bf16 query and the exact dequantized
// key, summed in fp32; it joins the row's histogram.
constexpr int kFreshWave = 3;
constexpr int kFreshMaxKvPasses = 2;  // main-KV passes a block's wave keeps in registers

struct FreshRegs {
  uint32_t xk[2];                  // index key channels lane, 64 + lane (raw f32 / bf16 bits)
  uint32_t q[4];                   // head h's channel pair (2 lane, 2 lane + 1), bf16
  float wq;                        // lane h < H_I: weight of head h
  uint32_t xv[kFreshMaxKvPasses];  // main-KV channel 64 j + lane of this block's passes j
};
struct FreshOut {
  uint32_t kw[2], ks[2];           // index key: code words and scale bytes of the two passes
  uint32_t vw[kFreshMaxKvPasses], vs[kFreshMaxKvPasses];  // main KV, per pass
  float sc;                        // score (lane 0)
};

template <typename In>
__device__ __forceinline__ uint32_t raw_elem(const void* base, int64_t i) {
  if constexpr (sizeof(In) == 4) return static_cast<const uint32_t*>(base)[i];
  else return (uint32_t) static_cast<const uint16_t*>(base)[i];
}
template <typename In>
__device__ __forceinline__ float raw_value(uint32_t v) {
  if constexpr (sizeof(In) == 4) return __uint_as_float(v);
  else return bf16_to_f32(v);
}

// pass j of the main-KV row belongs to block (1 + j) % nblk; the k-th of
// this block's passes (k < kFreshMaxKvPasses) is j = blk - 1 + k * nblk
__device__ __forceinline__ int fresh_kv_pass(int blk, int nblk, int k) {
  return (blk == 0 ? nblk - 1 : blk - 1) + k * nblk;
}

// Loads only (every branch is wave-uniform; lanes read in-range addresses).
template <typename In>
__device__ __forceinline__ void fresh_load(const NewRows& nw, int r, int32_t HI,
                                           const uint16_t* __restrict__ q_idx,
                                           const float* __restrict__ w, bool index_part,
                                           FreshRegs& f) {
  const int lane = threadIdx.x & 63;
  if (index_part) {
    const void* ik = static_cast<const In*>(nw.ikey) + (int64_t)r * 128;
    f.xk[0] = raw_elem<In>(ik, lane);
    f.xk[1] = raw_elem<In>(ik, 64 + lane);
    const uint32_t* qrow = reinterpret_cast<const uint32_t*>(q_idx + (int64_t)r * HI * 128);
#pragma unroll
    for (int h = 0; h < 4; ++h) f.q[h] = qrow[min(h, HI - 1) * 64 + lane];
    f.wq = w[(int64_t)r * HI + min(lane, HI - 1)];
  }
  const void* kv = static_cast<const In*>(nw.kv) + (int64_t)r * nw.kv_dim;
  const int npass = nw.kv_dim >> 6;
#pragma unroll
  for (int k = 0; k < kFreshMaxKvPasses; ++k) {
    const int j = fresh_kv_pass(blockIdx.x, gridDim.x, k);
    f.xv[k] = raw_elem<In>(kv, min(64 * j, 64 * (npass - 1)) + lane);
  }
}

template <typename In>
__device__ FreshOut fresh_compute(const NewRows& nw, int32_t HI, bool index_part,
                                  const FreshRegs& f) {
  __shared__ float kdeq[128];  // the new index key's exact values (this wave's only)
  const int lane = threadIdx.x & 63;
  FreshOut o{};
#pragma unroll
  for (int k = 0; k < kFreshMaxKvPasses; ++k) {
    float d;
    quantize_lane(raw_value<In>(f.xv[k]), &d, &o.vw[k], &o.vs[k]);
  }
  if (!index_part) return o;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float d;
    quantize_lane(raw_value<In>(f.xk[p]), &d, &o.kw[p], &o.ks[p]);
    kdeq[64 * p + lane] = d;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the key's values are in LDS
  const float k0 = kdeq[2 * lane], k1 = kdeq[2 * lane + 1];
  float sc = 0.0f;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if (h >= HI) break;
    float acc = bf16_to_f32(f.q[h] & 0xFFFFu) * k0 + bf16_to_f32(f.q[h] >> 16) * k1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
    sc += __shfl(f.wq, h, kWave) * relu(acc);
  }
  o.sc = sc;
  return o;
}

__device__ __forceinline__ void fresh_store(const NewRows& nw, int64_t p, int b,
                                            uint8_t* __restrict__ icodes,
                                            uint8_t* __restrict__ iscales, int64_t cap,
                                            int64_t nv, float* __restrict__ srow,
                                            uint32_t* __restrict__ hist, bool index_part,
                                            const FreshOut& o) {
  const int lane = threadIdx.x & 63, e = lane & 15;
  const int npass = nw.kv_dim >> 6;
  // lane e == 0 / 8 of each 16-lane row holds a code word, e == 0 the scale
  if (p >= 0 && p < nw.kv_cap) {
    const int64_t dr = (int64_t)b * nw.kv_cap + p;
#pragma unroll
    for (int k = 0; k < kFreshMaxKvPasses; ++k) {
      const int j = fresh_kv_pass(blockIdx.x, gridDim.x, k);
      if (j < npass) {
        const int c = 64 * j + lane;  // this lane's channel
        if ((e & 7) == 0)
          *reinterpret_cast<uint32_t*>(nw.kv_codes + dr * (nw.kv_dim >> 1) + (c >> 1)) = o.vw[k];
        if (e == 0) nw.kv_scales[dr * (nw.kv_dim >> 4) + (c >> 4)] = (uint8_t)o.vs[k];
      }
    }
  }
  if (!index_part || p < 0 || p >= cap) return;
  const int64_t dr = (int64_t)b * cap + p;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = 64 * q + lane;
    if ((e & 7) == 0) *reinterpret_cast<uint32_t*>(icodes + dr * 64 + (c >> 1)) = o.kw[q];
    if (e == 0) iscales[dr * 8 + (c >> 4)] = (uint8_t)o.ks[q];
  }
  if (lane == 0 && p < nv) {  // the position is visible to this row
    srow[p] = o.sc;
    if (hist) atomicAdd(hist + (score_key(o.sc) >> kHistShift), 1u);
  }
}

template <int NCH, int TPA, int GT, bool POOL>  // 128-channel chunks, tiles per accumulator,
                                                // tiles per group, positions from a pool list
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t cap,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int32_t HI, int32_t T,
    const int32_t* __restrict__ n_valid, const int32_t* __restrict__ pool, int32_t P,
    int32_t nv_add, float* __restrict__ scores, int64_t n_out, uint32_t* __restrict__ hist,
    int64_t hist_stride, int32_t hist_copies, int32_t chunk, int32_t row0, NewRows fresh) {
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
  const int64_t start = (int64_t)blockIdx.x * chunk;
  // the wave index is uniform: kept in a scalar register, the whole-group
  // test below is a scalar branch
  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const uint8_t* cbase = codes + (int64_t)b * cap * ROWB;
  const uint8_t* sbase = scales + (int64_t)b * cap * ROWS;
  const int32_t* prow = POOL ? pool + (int64_t)r * P : nullptr;
  float* srow = scores + (int64_t)r * n_out;
  int64_t end = 0;  // set below, once the row's visible length is known

  // Each wave takes groups of GT consecutive tiles (GT KiB of contiguous
  // codes for 128 channels in flat mode); the four waves of a round cover
  // 4*GT consecutive tiles.  The next group's loads are issued before the
  // current group is computed, into the other of two register buffers.
  // The scale bytes of lane (i, g) are bytes 2g, 2g+1 of each chunk's
  // scales; they are fetched as the aligned 32-bit word holding them.
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
  u32x4 cwA[GT][NCH], cwB[GT][NCH];
  uint32_t swA[GT][NCH], swB[GT][NCH];
  // The new rows' loads go first, ahead of this wave's scan loads (one wave
  // of some of the row's blocks, known from the block and wave alone).
  const bool fresh_on = !POOL && fresh.ikey;
  const bool fresh_wave = fresh_on && wave == kFreshWave &&
                          (blockIdx.x == 0 || (int)blockIdx.x <= (fresh.kv_dim >> 6));  // wave-uniform
  // A flat scan's chunk that lies inside the cache requests its first group
  // of a whole chunk before the row's visible length arrives (every such
  // row is allocated, so the loads are in bounds); it is used if the chunk
  // turns out whole, and requested again per tile otherwise.
  const bool guess_whole = !POOL && !fresh_wave && chunk == kScoreChunk && start + chunk <= cap;
  if (guess_whole) load_group(std::false_type{}, 0, cwA, swA);

  // visible entries, clamped to what the score row and the key list hold
  int64_t nv = min(min((int64_t)n_valid[r] + nv_add, n_out), POOL ? (int64_t)P : cap);
  const int64_t nv_all = nv;  // the new position counts as visible to the fresh score
  // the new position (loaded once: later loads queue behind the scan's)
  const int64_t p_new = fresh_on ? (int64_t)fresh.q_pos[r] : -1;
  if (fresh_on) nv = min(nv, max(p_new, (int64_t)0));  // scanned: [0, q_pos)
  // blocks past the scanned range still take their part of the new rows
  if (start >= nv && !(fresh_on && (int)blockIdx.x <= (fresh.kv_dim >> 6)))
    return;  // uniform for the whole block
  end = min(nv, start + chunk);

  if (hist) {
    for (int k = tid; k < kHistBins; k += 256) lhist[k] = 0u;
  }

  const int ntiles = (int)((end - start + 15) >> 4);
  const int nrounds = (ntiles + 4 * GT - 1) / (4 * GT);
  const int sshift = 16 * (g & 1);

  const bool whole = !POOL && chunk == kScoreChunk && end - start == chunk;  // block-uniform
  const bool idx_part = fresh_on && blockIdx.x == 0;
  FreshRegs fr;
  if (fresh_wave) {
    if (fresh.bf16) fresh_load<uint16_t>(fresh, r, HI, q_idx, w, idx_part, fr);
    else fresh_load<float>(fresh, r, HI, q_idx, w, idx_part, fr);
  }
  // the first group is requested before the query is prepared, so the
  // scan's first HBM round trip overlaps the query's
  if (nrounds > 0 && !(whole && guess_whole)) {
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
  // the new rows (one wave of the row's first block), once the wave's loads
  // and its query are in; stored after its scan
  FreshOut fo{};
  if (fresh_wave) {
    if (fresh.bf16) fo = fresh_compute<uint16_t>(fresh, HI, idx_part, fr);
    else fo = fresh_compute<float>(fresh, HI, idx_part, fr);
  }
  auto fresh_done = [&]() {
    if (fresh_wave)
      fresh_store(fresh, p_new, b, const_cast<uint8_t*>(codes), const_cast<uint8_t*>(scales), cap,
                  nv_all, srow, hist ? hist + (int64_t)r * hist_stride : nullptr, idx_part, fo);
  };
  if (fresh_on && start >= nv) {
    fresh_done();
    return;
  }
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
      for (int rr = 0; rr < 4; ++rr) part += wq[rr] * relu(acc[rr]);
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
  fresh_done();
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


bool fresh_rows_supported(bool pool, int32_t T, int32_t HI, int32_t DI, int32_t kv_dim) {
  return !pool && T == 1 && (HI == 1 || HI == 2 || HI == 4) && DI == 128 && kv_dim > 0 &&
         kv_dim % 64 == 0;
}

hipError_t launch_index_score(const uint8_t* codes, const uint8_t* scales, int32_t DI,
                              int64_t cap, int32_t rows, int32_t T, const uint16_t* q_idx,
                              const float* w, int32_t HI, const int32_t* n_valid,
                              int32_t nv_add, const int32_t* pool, int32_t P, int64_t n_max,
                              float* scores, int64_t n_out, uint32_t* hist, int64_t hist_stride,
                              int32_t hist_copies, hipStream_t st, int32_t row0,
                              const NewRows* fresh) {
  if (n_max <= 0 || rows == 0) return hipSuccess;
  const NewRows nw = fresh ? *fresh : NewRows{};
  if (nw.ikey && !fresh_rows_supported(pool != nullptr, T, HI, DI, nw.kv_dim))
    return hipErrorInvalidValue;
  // Prefill chunks take the tokens x positions kernel; the Top-K histogram
  // is then built from the written scores.
  if (index_tokens_pass(pool != nullptr, T, HI, DI, row0)) {
    hipError_t e = launch_index_tokens(codes, scales, cap, rows, T, q_idx, w, HI, n_valid, nv_add,
                                       n_max, scores, n_out, st, row0, !hist);
    if (e != hipSuccess || !hist) return e;
    return launch_topk_hist(scores, rows, n_out, n_valid, nv_add, n_max, hist, hist_stride,
                            hist_copies, st, false);
  }
  // 2048 positions per block, halved (down to 64) until the launch has at
  // least two blocks per compute unit: a 16K-slot pool or a 4K context would
  // otherwise scan with a handful of blocks
  int32_t chunk = kScoreChunk;
  while (chunk > 64 && ((n_max + chunk - 1) / chunk) * rows < kScanMinBlocks) chunk >>= 1;
  int64_t nchunks = (n_max + chunk - 1) / chunk;
  // every 64-channel pass of a new main-KV row needs a block of its row
  if (nw.ikey)
    nchunks = std::max<int64_t>(nchunks, ((nw.kv_dim >> 6) + kFreshMaxKvPasses - 1) / kFreshMaxKvPasses);
  const dim3 grid((unsigned)nchunks, (unsigned)rows), block(256);
#define CSA2_IS_LAUNCH(NCH, TPA, GT)                                                           \
  do {                                                                                         \
    if (pool)                                                                                  \
      CSA2_KERNEL(true, true, (index_score_kernel<NCH, TPA, GT, true>), grid, block, 0, st,    \
                  codes, scales, cap, q_idx, w, HI, T, n_valid, pool, P, nv_add, scores, n_out, \
                  hist, hist_stride, hist_copies, chunk, row0, nw);                            \
    else                                                                                       \
      CSA2_KERNEL(true, true, (index_score_kernel<NCH, TPA, GT, false>), grid, block, 0, st,   \
                  codes, scales, cap, q_idx, w, HI, T, n_valid, pool, P, nv_add, scores, n_out, \
                  hist, hist_stride, hist_copies, chunk, row0, nw);                            \
  } while (0)
  switch (DI / 128) {
    case 1:
      if (HI <= 4) CSA2_IS_LAUNCH(1, 4, 4);
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
