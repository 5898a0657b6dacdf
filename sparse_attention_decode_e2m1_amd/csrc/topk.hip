// topk.hip -- per-row Top-K selection over fp32 scores.
//
// louisbouchard.ai/deepseek-v41-flash-kv-cache-writing-benchmark, "Share the
// cache and the search work": sparse attention keeps a fixed number of
// global entries chosen from the indexer scores, and the first indexing
// layer keeps a larger candidate pool the same way.  Order: score
// descending, equal scores (-0 == +0) by slot ascending; the output lists the
// kept positions ascending and pads with -1.
//
// Scores map to order-preserving 32-bit keys; each candidate is ranked by the
// 64-bit value (key << 32 | ~slot), which is unique, so the K best form a
// strict prefix and there are no ties left to break.
//
//  1. A histogram of the top 12 key bits per row, kept as kHistCopies copies
//     (a block adds into copy blockIdx % kHistCopies: device-scope atomics on
//     one address serialise).  Built by the scoring kernel, or here by
//     topk_hist_kernel.
//  2. topk_select_kernel, one 1024-thread block per 4096 scores of a row
//     (16384 when a pass has many rows): the block sums the histogram copies and finds the bin b1 holding
//     the K-th key.  Its scores above b1 are kept outright; those in b1 are
//     candidates.  Wave w takes a contiguous run of slots, so a count pass
//     and a prefix over the 16 wave totals place both lists in position
//     order in the block's own regions.  The regions and the block's counts
//     are written with device-coherent stores; then the block counts itself
//     in the row's arrival counter.
//  3. The row's last block to arrive finishes it: it turns the counts into
//     offsets, gathers the lists into LDS, resolves the remaining entries
//     among the candidates by radix selection over the 64-bit rank values,
//     and writes the kept slots in slot order -- read back from an LDS
//     bitmap for rows up to 2^19 slots, else merged from the two sorted
//     lists by binary search.  It then clears the histogram copies and the
//     counter for the next call.
// Every pass over memory issues all of a thread's loads before using them.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__global__ __launch_bounds__(256) void topk_hist_kernel(const float* __restrict__ scores,
                                                        int64_t n,
                                                        const int32_t* __restrict__ n_valid,
                                                        int32_t nv_add,
                                                        uint32_t* __restrict__ hist,
                                                        int64_t hist_stride,
                                                        int32_t hist_copies) {
  constexpr int PT = kTopkChunk / 256;
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  const int64_t start = (int64_t)blockIdx.x * kTopkChunk;
  if (start >= nv) return;
  for (int k = threadIdx.x; k < kHistBins; k += 256) lhist[k] = 0u;
  const float* srow = scores + (int64_t)r * n;
  float v[PT];
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int64_t s = start + j * 256 + threadIdx.x;
    v[j] = (s < nv) ? srow[s] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PT; ++j)
    if (start + j * 256 + threadIdx.x < nv) atomicAdd(&lhist[score_key(v[j]) >> kHistShift], 1u);
  __syncthreads();
  uint32_t* gh = hist + (int64_t)r * hist_stride + (blockIdx.x % hist_copies) * kHistBins;
  for (int k = threadIdx.x; k < kHistBins; k += 256)
    if (lhist[k]) atomicAdd(gh + k, lhist[k]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<0x111, 0xF>(x);  // row_shr:1
  x += dpp_u32<0x112, 0xF>(x);  // row_shr:2
  x += dpp_u32<0x114, 0xF>(x);  // row_shr:4
  x += dpp_u32<0x118, 0xF>(x);  // row_shr:8
  x += dpp_u32<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_u32<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Exclusive prefix sum over the block (NT threads); `tmp` holds NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = tmp[w];
    off += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

// The bin holding the k-th largest key: count(bins > b1) < k <= count(bins
// >= b1), from the row's 12-bit key histogram summed over its `copies`
// copies (thread t of NT takes bins [t*BPT, (t+1)*BPT)).  Written to *b1 by
// the thread that finds it (left unchanged when the histogram holds fewer
// than k keys); every thread calls it.
template <int NT>
__device__ __forceinline__ void find_cut(const uint32_t* rh, int copies, int32_t k, uint32_t* tmp,
                                         int* b1) {
  constexpr int BPT = kHistBins / NT, NV = BPT / 4;
  static_assert(BPT % 4 == 0, "whole uint4 per thread");
  uint4 hc[kHistCopies][NV];
#pragma unroll
  for (int c = 0; c < kHistCopies; ++c)
#pragma unroll
    for (int v = 0; v < NV; ++v)
      hc[c][v] = (c < copies)
                     ? *reinterpret_cast<const uint4*>(rh + c * kHistBins + BPT * threadIdx.x + 4 * v)
                     : make_uint4(0, 0, 0, 0);
  uint32_t h[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) h[j] = 0u;
#pragma unroll
  for (int c = 0; c < kHistCopies; ++c)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      h[4 * v] += hc[c][v].x;
      h[4 * v + 1] += hc[c][v].y;
      h[4 * v + 2] += hc[c][v].z;
      h[4 * v + 3] += hc[c][v].w;
    }
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) sum += h[j];
  uint32_t total;
  const uint32_t excl = block_scan<NT>(sum, tmp, &total);
  const uint32_t above = total - excl - sum;  // keys in bins of higher threads
  if (above < (uint32_t)k && above + sum >= (uint32_t)k) {
    uint32_t acc = above;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (acc < (uint32_t)k && acc + h[j] >= (uint32_t)k) *b1 = BPT * threadIdx.x + j;
      acc += h[j];
    }
  }
  __syncthreads();
}

// Rows with many select blocks find their cut once: one block per row.
__global__ __launch_bounds__(kSelThreads) void topk_cut_kernel(const int32_t* __restrict__ n_valid,
                                                               int32_t nv_add, int64_t n, int32_t k,
                                                               TopkWs w) {
  __shared__ uint32_t tmp[kSelWaves];
  __shared__ int s_b1;
  const int r = blockIdx.x;
  if (threadIdx.x == 0) s_b1 = 0x7FFFFFFF;
  __syncthreads();
  if (min((int64_t)n_valid[r] + nv_add, n) > k)
    find_cut<kSelThreads>(w.hist + (int64_t)r * w.hist_stride, w.hist_copies, k, tmp, &s_b1);
  if (threadIdx.x == 0) w.cut[(int64_t)r * w.ctr_stride] = (uint32_t)s_b1;
}

// Radix selection of the need-th largest rank value among C candidates
// (all sharing the top 12 key bits): 11-bit digits at shifts 41, 30, 19, 8,
// then 8 bits at 0; stops once a whole bucket is taken.  for_each(f) calls f
// on every candidate (each once, spread over the block's threads).  With
// GIVEN0, the first digit's histogram is already at hand (thread t holds
// bins [t*BPT, (t+1)*BPT) in g0) and that pass skips the candidates.
// Returns the threshold: the candidates >= it (low 52 bits compared) are the
// need largest.  All NT threads call it.
template <int N>
struct Bins {  // a thread's share of a histogram, passed by value (kept in registers)
  uint32_t v[N];
};
template <int NT, bool GIVEN0, typename ForEach>
__device__ uint64_t radix_threshold(uint32_t need, uint32_t* rhist, uint32_t* tmp,
                                    ForEach&& for_each, Bins<2048 / NT> g0) {
  constexpr int BPT = 2048 / NT;
  __shared__ int s_dig;
  __shared__ uint32_t s_dig_above, s_dig_count;
  const int tid = threadIdx.x;
  if (need == 0) return ~0ull;
  uint64_t prefix = 0;
  uint32_t rem = need;
  for (int p = 0; p < 5; ++p) {
    const int sh = p < 4 ? 41 - 11 * p : 0, wd = p < 4 ? 11 : 8;
    const int nb = 1 << wd;
    const bool given = GIVEN0 && p == 0;
    if (!given)
      for (int j = tid; j < 2048; j += NT) rhist[j] = 0u;
    if (tid == 0) {
      s_dig = 0;
      s_dig_above = 0;
      s_dig_count = 0;
    }
    __syncthreads();
    if (!given) {
      const uint64_t hi_mask = (~0ull << (sh + wd)) & ((1ull << 52) - 1);
      for_each([&](uint64_t x) {
        if ((x & hi_mask) == prefix) atomicAdd(&rhist[(uint32_t)(x >> sh) & (uint32_t)(nb - 1)], 1u);
      });
      __syncthreads();
    }
    // digit d with count(> d) < rem <= count(>= d); BPT bins per thread
    // (bins past nb were cleared, so they count zero)
    const int b0 = BPT * tid;
    uint32_t cv[BPT], sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      cv[j] = given ? g0.v[j] : rhist[b0 + j];
      sum += cv[j];
    }
    uint32_t tot;
    const uint32_t ex = block_scan<NT>(sum, tmp, &tot);
    uint32_t acc = tot - ex - sum;  // keys in the bins of higher threads
    if (acc < rem && acc + sum >= rem) {
#pragma unroll
      for (int j = BPT - 1; j >= 0; --j) {
        if (acc < rem && acc + cv[j] >= rem) {
          s_dig = b0 + j;
          s_dig_above = acc;
          s_dig_count = cv[j];
        }
        acc += cv[j];
      }
    }
    __syncthreads();
    const uint32_t d = (uint32_t)s_dig;
    rem -= s_dig_above;
    prefix |= (uint64_t)d << sh;
    const bool whole_bucket = s_dig_count == rem;
    __syncthreads();
    if (whole_bucket) break;
  }
  return prefix;
}
template <int NT, typename ForEach>
__device__ uint64_t radix_threshold(uint32_t need, uint32_t* rhist, uint32_t* tmp,
                                    ForEach&& for_each) {
  return radix_threshold<NT, false>(need, rhist, tmp, for_each, Bins<2048 / NT>{});
}

// Completion of row r by its last block (all select blocks of the row have
// written their regions and counts), for rows too long for the bitmap: the
// kept slots are listed (kept outright, then chosen, each in slot order) and
// merged.
__device__ void finish_row(int r, int64_t nv, int64_t n, const int32_t* __restrict__ slot_pos,
                           int32_t k, int nblk, int32_t* __restrict__ idx_out,
                           int32_t* __restrict__ count_out, const TopkWs& w, int32_t lds_cand,
                           int32_t chunk, uint32_t* smem, uint32_t* tmp) {
  constexpr int NT = kSelThreads;
  uint32_t* rhist = smem;                      // 2048 radix bins
  uint32_t* offA = rhist + 2048;               // nblk + 1
  uint32_t* offE = offA + (nblk + 1);          // nblk + 1
  uint32_t* list = offE + (nblk + 1);          // k kept slots
  uint64_t* cl = reinterpret_cast<uint64_t*>(list + ((k + 1) & ~1));  // lds_cand candidates
  const int tid = threadIdx.x;
  int32_t* orow = idx_out + (int64_t)r * k;
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)r * n : nullptr;

  if (nv <= k) {
    for (int j = tid; j < k; j += NT) orow[j] = (j < nv) ? (sp ? sp[j] : j) : -1;
    if (count_out && tid == 0) count_out[r] = (int32_t)nv;
    return;
  }
  // ---- per-block counts -> offsets
  const uint32_t* crow = w.counts + (int64_t)r * w.counts_stride;
  constexpr int kMaxPer = (int)(kMaxTopkN / kTopkChunk / NT);  // blocks per thread
  static_assert(kMaxPer >= 1 && kMaxPer <= 8, "counts held in registers");
  const int per = (nblk + NT - 1) / NT;
  uint32_t ca[kMaxPer], ce[kMaxPer];
  uint32_t a_loc = 0, e_loc = 0;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int b = tid * per + j;
    const bool in = j < per && b < nblk;
    ca[j] = in ? ld_coh(crow + 2 * b) : 0u;
    ce[j] = in ? ld_coh(crow + 2 * b + 1) : 0u;
  }
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    a_loc += ca[j];
    e_loc += ce[j];
  }
  uint32_t A, C;
  uint32_t ra = block_scan<NT>(a_loc, tmp, &A);
  uint32_t rc = block_scan<NT>(e_loc, tmp, &C);
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    const int b = tid * per + j;
    if (j < per && b < nblk) {
      offA[b] = ra;
      offE[b] = rc;
      ra += ca[j];
      rc += ce[j];
    }
  }
  if (tid == 0) {
    offA[nblk] = A;
    offE[nblk] = C;
  }
  __syncthreads();
  const uint32_t need = (uint32_t)k - min(A, (uint32_t)k);
  // element c of a family of per-block regions: block = last b with off[b] <= c
  auto block_of = [&](const uint32_t* off, uint32_t c) -> int {
    int lo = 0, hi = nblk - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  const uint32_t* abase = w.above + (int64_t)r * w.above_stride;
  const uint64_t* cbase = w.cand + (int64_t)r * w.cand_stride;
  auto cand_at = [&](uint32_t c) -> uint64_t {
    const int b = block_of(offE, c);
    return ld_coh(cbase + (int64_t)b * chunk + (c - offE[b]));
  };
  // ---- gather the kept ("above") positions and the candidates
  const uint32_t Ak = min(A, (uint32_t)k);
  const bool in_lds = C <= (uint32_t)lds_cand;
  {
    // TPB threads per select block (a power of two), each copying every
    // TPB-th entry of the block's two regions; indices are clamped rather
    // than branched on, so a thread's loads are in flight together.
    const uint32_t nC = in_lds ? C : 0u;
    int tpb = 1;
    while (tpb * 2 * nblk <= NT) tpb *= 2;
    const int bpp = NT / tpb;
    for (int b0 = 0; b0 < nblk; b0 += bpp) {
      const int b = b0 + tid / tpb, j = tid % tpb;
      const bool live = b < nblk;
      const int bb = live ? b : 0;
      const uint32_t a_lo = min(offA[bb], Ak), a_hi = live ? min(offA[bb + 1], Ak) : a_lo;
      const uint32_t e_lo = min(offE[bb], nC), e_hi = live ? min(offE[bb + 1], nC) : e_lo;
      const uint32_t* ar = abase + (int64_t)bb * chunk;
      const uint64_t* cr = cbase + (int64_t)bb * chunk;
      const uint32_t na = a_hi - a_lo, ne = e_hi - e_lo;
      for (uint32_t i0 = j; i0 < max(na, ne); i0 += 8 * tpb) {
        uint32_t ta[8];
        uint64_t tc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t i = i0 + u * tpb;
          ta[u] = ld_coh(ar + min(i, max(na, 1u) - 1u));
          tc[u] = ld_coh(cr + min(i, max(ne, 1u) - 1u));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t i = i0 + u * tpb;
          if (i < na) {
            list[a_lo + i] = ta[u];
          }
          if (i < ne) cl[e_lo + i] = tc[u];
        }
      }
    }
  }
  __syncthreads();
  auto for_each = [&](auto&& f) {
    if (in_lds) {
      for (uint32_t c = tid; c < C; c += NT) f(cl[c]);
    } else {
      for (uint32_t c0 = 0; c0 < C; c0 += NT * 4) {
        uint64_t t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t c = c0 + u * NT + tid;
          if (c < C) t[u] = cand_at(c);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c0 + u * NT + tid < C) f(t[u]);
      }
    }
  };
  const uint64_t thr = radix_threshold<NT>(need, rhist, tmp, for_each);
  const uint64_t low52 = (1ull << 52) - 1;
  // ---- chosen candidates (rank value within b1 >= thr), kept in slot
  // order: the concatenated candidate regions are slot-ordered.
  uint32_t kept;  // k unless the histogram disagreed with the scores
  {
    const uint32_t per_c = (C + NT - 1) / NT;
    const uint32_t lo = min(tid * per_c, C), hi = min(lo + per_c, C);
    uint32_t cnt = 0;
    for (uint32_t c = lo; c < hi; ++c) {
      const uint64_t x = in_lds ? cl[c] : cand_at(c);
      cnt += (need > 0 && (x & low52) >= thr) ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t o = Ak + block_scan<NT>(cnt, tmp, &tot);
    kept = Ak + min(tot, need);
    for (uint32_t c = lo; c < hi; ++c) {
      const uint64_t x = in_lds ? cl[c] : cand_at(c);
      if (need > 0 && (x & low52) >= thr && o < kept) list[o++] = rank_slot(x);
    }
  }
  __syncthreads();
  // ---- merge list[0, Ak) and list[Ak, kept) (both ascending) into orow:
  // an element's output slot is its index in its own list plus the number
  // of smaller elements in the other (four searches in flight per thread)
  {
    const uint32_t nch = kept - Ak;
    int topA = 1, topC = 1;
    while (topA * 2 <= (int)Ak) topA *= 2;
    while (topC * 2 <= (int)nch) topC *= 2;
    const int topM = max(topA, topC);
    for (uint32_t i0 = 0; i0 < (uint32_t)k; i0 += NT * 4) {
      uint32_t x[4], cnt[4], lo[4], len[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = i0 + u * NT + tid;
        const bool live = i < kept;
        x[u] = live ? list[i] : 0u;
        lo[u] = (i < Ak) ? Ak : 0u;        // the other list
        len[u] = live ? ((i < Ak) ? nch : Ak) : 0u;
        cnt[u] = 0;
      }
      for (int step = topM; step > 0; step >>= 1) {
        uint32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = list[lo[u] + min(cnt[u] + (uint32_t)step, max(len[u], 1u)) - 1];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t nx = cnt[u] + (uint32_t)step;
          cnt[u] = (nx <= len[u] && v[u] < x[u]) ? nx : cnt[u];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = i0 + u * NT + tid;
        if (i >= (uint32_t)k) continue;
        if (i >= kept) {
          orow[i] = -1;
          continue;
        }
        const uint32_t pos = (i < Ak) ? i + cnt[u] : (i - Ak) + cnt[u];
        orow[pos] = sp ? sp[x[u]] : (int32_t)x[u];
      }
    }
  }
  if (count_out && tid == 0) count_out[r] = (int32_t)kept;
}

// Rows of up to kBitmapSlots slots: the select blocks publish their kept
// slots as a bitmap (one bit per slot, in the row's `above` region), so the
// row's last block fetches, in one round trip, the per-block counts, the
// bitmap and the first `spec` candidates of every block (as many as kCP
// loads per thread allow, a power of two).  The chosen
// candidates are marked in the same (LDS) bitmap, which is then read back in
// slot order: wave w takes a contiguous run of words, 64 at a time, and
// lane offsets come from wave prefix sums.  The output is staged in LDS and
// written with whole-row coalesced stores.
constexpr int64_t kBitmapSlots = int64_t(1) << 19;
constexpr int kCP = 8;  // early candidate loads per thread

__device__ void finish_row_bm(int r, int64_t nv, int64_t n, const int32_t* __restrict__ slot_pos,
                              int32_t k, int nblk, int32_t* __restrict__ idx_out,
                              int32_t* __restrict__ count_out, const TopkWs& w, int32_t lds_cand,
                              int32_t bm_words, int32_t chunk, uint32_t* smem, uint32_t* tmp) {
  constexpr int NT = kSelThreads, NW = kSelWaves;
  constexpr int kBW = (int)(kBitmapSlots / 64 / NT);                 // bitmap u64 words per thread
  static_assert(kBitmapSlots / kTopkChunk <= NT, "one block's counts per thread");
  uint32_t* rhist = smem;                          // 2048 radix bins
  uint32_t* offE = rhist + 2048;                   // nblk + 1
  uint32_t* bm = offE + 2 * (nblk + 1);            // bm_words (8-byte aligned)
  uint64_t* cl = reinterpret_cast<uint64_t*>(bm + bm_words);  // lds_cand candidates
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* orow = idx_out + (int64_t)r * k;
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)r * n : nullptr;

  if (nv <= k) {
    for (int j = tid; j < k; j += NT) orow[j] = (j < nv) ? (sp ? sp[j] : j) : -1;
    if (count_out && tid == 0) count_out[r] = (int32_t)nv;
    return;
  }
  // ---- one round trip: counts, bitmap, early candidates (each thread
  // issues all of its loads before using any; out-of-range ones are skipped
  // rather than clamped, since many loads of one address serialise)
  const uint32_t* crow = w.counts + (int64_t)r * w.counts_stride;
  const uint64_t* gbm = reinterpret_cast<const uint64_t*>(w.above + (int64_t)r * w.above_stride);
  const uint64_t* cbase = w.cand + (int64_t)r * w.cand_stride;
  const int nw64 = bm_words / 2;
  const int vw64 = (int)((nv + 63) >> 6);  // words holding valid slots
  uint32_t ca = 0u, ce = 0u;
  if (tid < nblk) {
    ca = ld_coh(crow + 2 * tid);
    ce = ld_coh(crow + 2 * tid + 1);
  }
  uint64_t bw[kBW];
#pragma unroll
  for (int m = 0; m < kBW; ++m) bw[m] = (tid + m * NT < vw64) ? ld_coh(gbm + tid + m * NT) : 0ull;
  int lspec = 0;  // log2 of candidates fetched early per block
  while ((2 << lspec) * nblk <= NT * kCP && (2 << lspec) <= chunk) ++lspec;
  const int spec = 1 << lspec;
  uint64_t cv[kCP];
#pragma unroll
  for (int m = 0; m < kCP; ++m) {
    const int f = tid + m * NT;
    cv[m] = (f < nblk * spec) ? ld_coh(cbase + (int64_t)(f >> lspec) * chunk + (f & (spec - 1))) : 0ull;
  }
  uint64_t* bm64 = reinterpret_cast<uint64_t*>(bm);
#pragma unroll
  for (int m = 0; m < kBW; ++m) {
    const int j = tid + m * NT;
    if (j < nw64) bm64[j] = (j < vw64) ? bw[m] : 0ull;
  }
  // counts -> candidate offsets: thread b holds block b's counts, so the
  // waves' own prefix sums and one exchange of wave totals suffice (the
  // radix bins serve as scratch)
  const uint32_t ie = wave_incl_scan(ce), ia = wave_incl_scan(ca);
  if (lane == 63) {
    rhist[wave] = ie;
    rhist[NW + wave] = ia;
  }
  __syncthreads();
  uint32_t A = 0, C = 0, eb0 = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    const uint32_t te = rhist[x];
    eb0 += (x < wave) ? te : 0u;
    C += te;
    A += rhist[NW + x];
  }
  if (tid < nblk) offE[tid] = eb0 + ie - ce;
  if (tid == 0) offE[nblk] = C;
  __syncthreads();
  const uint32_t need = (uint32_t)k - min(A, (uint32_t)k);
  const bool in_lds = C <= (uint32_t)lds_cand;
  if (in_lds) {
#pragma unroll
    for (int m = 0; m < kCP; ++m) {
      const int f = tid + m * NT, b = f >> lspec, i = f & (spec - 1);
      if (b < nblk && (uint32_t)i < offE[b + 1] - offE[b]) cl[offE[b] + i] = cv[m];
    }
    // blocks with more than spec candidates: the rest, TPB threads per
    // block, each with up to 8 loads in flight
    constexpr int TPB = NT / (int)(kBitmapSlots / kTopkChunk);
    for (int b0 = 0; b0 < nblk; b0 += NT / TPB) {
      const int b = b0 + tid / TPB, j = tid % TPB;
      const uint32_t eb = (b < nblk) ? offE[b + 1] - offE[b] : 0u;
      for (uint32_t i0 = spec + j; i0 < eb; i0 += 8 * TPB) {
        uint64_t t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t i = i0 + u * TPB;
          t[u] = (i < eb) ? ld_coh(cbase + (int64_t)b * chunk + i) : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * TPB < eb) cl[offE[b] + i0 + u * TPB] = t[u];
      }
    }
  }
  __syncthreads();
  auto cand_at = [&](uint32_t c) -> uint64_t {
    int lo = 0, hi = nblk - 1;  // block = last b with offE[b] <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offE[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return ld_coh(cbase + (int64_t)lo * chunk + (c - offE[lo]));
  };
  auto for_each = [&](auto&& f) {
    if (in_lds) {
      for (uint32_t c = tid; c < C; c += NT) f(cl[c]);
    } else {
      for (uint32_t c = tid; c < C; c += NT) f(cand_at(c));
    }
  };
  const uint64_t thr = radix_threshold<NT>(need, rhist, tmp, for_each);
  const uint64_t low52 = (1ull << 52) - 1;
  if (need > 0) for_each([&](uint64_t x) {
    if ((x & low52) >= thr) {
      const uint32_t sl = rank_slot(x);
      atomicOr(&bm[sl >> 5], 1u << (sl & 31));
    }
  });
  __syncthreads();
  // ---- marked slots in slot order, over 64-bit words
  const int WPW = ((nw64 + NW - 1) / NW + 63) & ~63;
  const int wb = min(wave * WPW, nw64), we = min(wb + WPW, nw64);
  uint32_t cnt = 0;
  for (int j = wb + lane; j < we; j += 64) cnt += (uint32_t)__popcll(bm64[j]);
  const uint32_t wtotal = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt), 63);
  if (lane == 0) tmp[wave] = wtotal;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    const uint32_t t = tmp[x];
    base += (x < wave) ? t : 0u;
    tot += t;
  }
  const uint32_t kept = min(tot, (uint32_t)k);
  // staged in the candidate area (no longer read) when it holds k slots
  uint32_t* ob = (2 * (int64_t)lds_cand >= k) ? reinterpret_cast<uint32_t*>(cl) : nullptr;
  uint32_t o = base;
  for (int j0 = wb; j0 < we; j0 += 64) {
    const int j = j0 + lane;
    uint64_t word = (j < we) ? bm64[j] : 0ull;
    const uint32_t c = (uint32_t)__popcll(word);
    const uint32_t incl = wave_incl_scan(c);
    uint32_t pos = o + incl - c;
    o += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    while (word) {
      const uint32_t sl = 64u * (uint32_t)j + (uint32_t)(__ffsll((unsigned long long)word) - 1);
      word &= word - 1ull;
      if (pos < kept) {
        if (ob) ob[pos] = sl;
        else orow[pos] = sp ? sp[sl] : (int32_t)sl;
      }
      ++pos;
    }
  }
  if (ob) {
    __syncthreads();
    for (int j = tid; j < k; j += NT) orow[j] = (j < (int)kept) ? (sp ? sp[ob[j]] : (int32_t)ob[j]) : -1;
  } else {
    for (uint32_t i = kept + tid; i < (uint32_t)k; i += NT) orow[i] = -1;
  }
  if (count_out && tid == 0) count_out[r] = (int32_t)kept;
}

template <int PL>  // scores per lane: a block takes 1024 * PL consecutive slots
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void topk_select_kernel(
    const float* __restrict__ scores, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t nv_add, const int32_t* __restrict__ slot_pos, int32_t k, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, TopkWs w, int32_t lds_cand, int32_t bm_words, bool use_cut) {
  extern __shared__ uint64_t smem64[];
  uint32_t* smem = reinterpret_cast<uint32_t*>(smem64);
  __shared__ uint32_t tmp[kSelWaves];
  __shared__ uint32_t wtot[2][kSelWaves];  // kept / candidates per wave
  __shared__ int s_b1, s_last;

  const int r = blockIdx.y, nblk = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  constexpr int32_t kChunk = kSelThreads * PL;
  const int64_t start = (int64_t)blockIdx.x * kChunk;
  const int64_t wstart = start + (int64_t)wave * 64 * PL;
  uint32_t* rh = w.hist + (int64_t)r * w.hist_stride;

  if (nv > k) {
    uint32_t* crow = w.counts + (int64_t)r * w.counts_stride + 2 * blockIdx.x;
    if (start >= nv) {
      if (tid == 0) {
        st_coh(crow, 0u);
        st_coh(crow + 1, 0u);
      }
    } else {
      // this wave's scores: slots wstart + 64j + lane
      const float* srow = scores + (int64_t)r * n;
      float v[PL];
#pragma unroll
      for (int j = 0; j < PL; ++j) v[j] = srow[min(wstart + 64 * j + lane, nv - 1)];
      // the row's histogram summed over its copies: bins [4t, 4t+4)
      if (tid == 0) s_b1 = 0x7FFFFFFF;  // replaced below; keeps an inconsistent histogram harmless
      if (use_cut) {
        if (tid == 0) s_b1 = (int)w.cut[(int64_t)r * w.ctr_stride];
        __syncthreads();
      } else {
        find_cut<kSelThreads>(rh, w.hist_copies, k, tmp, &s_b1);
      }
      const uint32_t b1 = (uint32_t)s_b1;
      // count pass: this wave's kept and candidate totals
      uint32_t na = 0, ne = 0;
      uint32_t keys[PL];
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        const int64_t s = wstart + 64 * j + lane;
        keys[j] = score_key(v[j]);
        const uint32_t bin = keys[j] >> kHistShift;
        na += (uint32_t)__popcll(__ballot(s < nv && bin > b1));
        ne += (uint32_t)__popcll(__ballot(s < nv && bin == b1));
      }
      if (lane == 0) {
        wtot[0][wave] = na;
        wtot[1][wave] = ne;
      }
      __syncthreads();
      uint32_t oa = 0, oe = 0, ta = 0, te = 0;
#pragma unroll
      for (int x = 0; x < kSelWaves; ++x) {
        const uint32_t a = wtot[0][x], c = wtot[1][x];
        oa += (x < wave) ? a : 0u;
        oe += (x < wave) ? c : 0u;
        ta += a;
        te += c;
      }
      // write pass, in slot order: candidates listed; kept slots listed, or
      // (bitmap rows) published as this wave's bitmap words
      uint32_t* ra = w.above + (int64_t)r * w.above_stride + (int64_t)blockIdx.x * kChunk;
      uint64_t* gbm = reinterpret_cast<uint64_t*>(w.above + (int64_t)r * w.above_stride);
      uint64_t* rc = w.cand + (int64_t)r * w.cand_stride + (int64_t)blockIdx.x * kChunk;
      const uint64_t lt = lanemask_lt();
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        const int64_t s = wstart + 64 * j + lane;
        const uint32_t bin = keys[j] >> kHistShift;
        const bool ab = s < nv && bin > b1;
        const bool eq = s < nv && bin == b1;
        const uint64_t ma = __ballot(ab), me = __ballot(eq);
        if (bm_words > 0) {
          if (lane == 0) st_coh(gbm + ((wstart + 64 * j) >> 6), ma);
        } else if (ab) {
          st_coh(ra + oa + (uint32_t)__popcll(ma & lt), (uint32_t)s);
        }
        if (eq) st_coh(rc + oe + (uint32_t)__popcll(me & lt), rank_value(keys[j], (uint32_t)s));
        oa += (uint32_t)__popcll(ma);
        oe += (uint32_t)__popcll(me);
      }
      if (tid == 0) {
        st_coh(crow, ta);
        st_coh(crow + 1, te);
      }
    }
  }
  // ---- arrival; the row's last block completes it
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (tid == 0) {
    uint32_t* ctr = w.ctr + (int64_t)r * w.ctr_stride;
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (uint32_t)nblk - 1u;
    if (s_last) {
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w.cut[(int64_t)r * w.ctr_stride] = 0u;  // every block of the row has read it
    }
  }
  __syncthreads();
  if (!s_last) return;
  if (bm_words > 0)
    finish_row_bm(r, nv, n, slot_pos, k, nblk, idx_out, count_out, w, lds_cand, bm_words, kChunk,
                  smem, tmp);
  else
    finish_row(r, nv, n, slot_pos, k, nblk, idx_out, count_out, w, lds_cand, kChunk, smem, tmp);
  // ---- leave the histogram copies zero for the next call (every block of
  // the row has read them)
  uint4* h4p = reinterpret_cast<uint4*>(rh);
  for (int j = tid; j < w.hist_copies * kHistBins / 4; j += kSelThreads) h4p[j] = make_uint4(0, 0, 0, 0);
}

// ------------------------------------------------------- one-wait variant
// When every select block of a pass can be resident at once, the row's last
// block to arrive only finds the threshold among the candidates and sends
// each block of the row a record: where the block's part of the output
// starts and which of its candidates are chosen.  Each block waits for its
// record (its only wait on another block, bounded by the wait limit's polls) and
// writes its own kept slots from the scores it still holds.  512 threads and
// 8 scores per thread, so two blocks fit on a compute unit.
constexpr int kCoopThreads = 512;
constexpr int kCoopWaves = kCoopThreads / 64;
constexpr int kCoopPL = kTopkChunk / kCoopThreads;  // scores per thread
constexpr int kCoopCP = 8;                          // early candidate loads per thread
constexpr size_t kCoopLds = 17 * 1024;               // dynamic LDS of a block
// Records live in histogram copies 4..7 of the row's control block (the
// passes that use this variant keep at most 4 copies); word 2 after the
// histogram words flags a record that never came.
constexpr int64_t kRecWordOffset = 4 * int64_t(kHistBins);
// Then the candidates' first radix digit histogram (2048 bins), added to by
// the select blocks and cleared by the completing block.
constexpr int64_t kL2WordOffset = kRecWordOffset + 2 * kCoopThreads;
static_assert(kTopkChunk == 4096, "12-bit block-relative slots in packed candidates");
static_assert(kL2WordOffset + 2048 <= kHistWords, "records and digit bins fit the control block");

// Record of block b, written by the completing block and cleared by b: bit
// 63 set; bit 62: no candidate chosen; bits 61..42: kt; bits 41..29: rel;
// bits 28..15: the launch's generation; bits 14..0: the output offset of the
// block's first kept slot (< 2^15 since k <= 16384).  A candidate of block b
// (its key's top 12 bits are the cut bin) with low 20 key bits lo at
// block-relative slot l is chosen iff lo > kt, or lo == kt and l < rel.  A
// block takes only a record of its own launch's generation, so a record left
// by a launch whose wait gave up is never mistaken for the current one.
constexpr uint32_t kGenMask = 0x3FFFu;
__device__ __forceinline__ uint64_t coop_record(bool none, uint32_t kt, uint32_t rel,
                                                uint32_t gen, uint32_t off) {
  return (1ull << 63) | ((uint64_t)none << 62) | ((uint64_t)(kt & 0xFFFFFu) << 42) |
         ((uint64_t)(rel & 0x1FFFu) << 29) | ((uint64_t)(gen & kGenMask) << 15) |
         (uint64_t)(off & 0x7FFFu);
}
__device__ __forceinline__ bool record_is(uint64_t rec, uint32_t gen) {
  return (rec >> 63) && (((uint32_t)(rec >> 15) & kGenMask) == (gen & kGenMask));
}

constexpr int kBucketMax = kCoopThreads;  // candidates of the cut digit ranked directly

// The completing block of row r (every block of the row has published its
// counts, candidates and first-digit bins): the threshold among the
// candidates, each block's count of chosen candidates, the blocks' output
// offsets, and one record per block holding visible slots (its own goes to
// *own).  The candidates come straight from the first round trip (the first
// `spec` of each block, in registers; the rest of a block, if any, from
// memory).  The first radix digit's histogram is complete, so the cut digit
// d0 is known at once; candidates above it are chosen, and the few sharing
// it are ranked against each other (a full radix selection only when more
// than kBucketMax share it).
__device__ void coop_complete(int r, int64_t nv, int32_t k, int nblk, int32_t* __restrict__ orow,
                              int32_t* __restrict__ count_out, const TopkWs& w, uint32_t* smem,
                              uint32_t* tmp, uint32_t* rh, uint64_t* recs, uint64_t* own,
                              uint32_t gen) {
  constexpr int NT = kCoopThreads, NW = kCoopWaves, CH = kTopkChunk, BPT = 2048 / NT;
  uint32_t* cntE = smem;                    // candidates per block
  uint32_t* chosen = cntE + NT;             // chosen candidates per block (register pass)
  uint32_t* rhist = chosen + NT;            // 2048 radix bins (many ties only)
  uint64_t* bucket = reinterpret_cast<uint64_t*>(rhist + 2048);  // kBucketMax
  uint32_t* pcs = reinterpret_cast<uint32_t*>(bucket + kBucketMax);  // kCoopCP x NW counts
  __shared__ uint32_t chosen2[kCoopThreads];  // chosen candidates per block (the other passes)
  __shared__ uint32_t s_tot[3][NW];           // per wave: kept, candidates, first-digit bins
  __shared__ uint32_t s_pick0[3];             // the first cut digit, the count above it, its count
  __shared__ uint32_t s_nb, s_rest;
  __shared__ uint64_t s_thr;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* crow = w.counts + (int64_t)r * w.counts_stride;
  // candidates are packed 32-bit words (see the select pass); expand() gives
  // the 64-bit rank value of block b's word (key bits 19..0, ~row slot)
  const uint32_t* cbase = reinterpret_cast<const uint32_t*>(w.cand + (int64_t)r * w.cand_stride);
  auto expand = [&](uint32_t p, int b) -> uint64_t {
    const uint32_t slot = (uint32_t)b * CH + (uint32_t)(CH - 1) - (p & (uint32_t)(CH - 1));
    return ((uint64_t)(p >> 12) << 32) | (uint64_t)(0xFFFFFFFFu - slot);
  };
  uint32_t* l2 = rh + kL2WordOffset;
  // ---- one round trip: counts, the first spec candidates of each block, the
  // first-digit bins
  uint32_t ca = 0u, ce = 0u;
  if (tid < nblk) {
    ca = ld_coh(crow + 2 * tid);
    ce = ld_coh(crow + 2 * tid + 1);
  }
  int lspec = 0;
  while ((2 << lspec) * nblk <= NT * kCoopCP && (2 << lspec) <= CH) ++lspec;
  const int spec = 1 << lspec;
  uint32_t cv[kCoopCP];
#pragma unroll
  for (int m = 0; m < kCoopCP; ++m) {
    const int f = tid + m * NT;
    cv[m] = (f < nblk * spec) ? ld_coh(cbase + (int64_t)(f >> lspec) * CH + (f & (spec - 1))) : 0u;
  }
  Bins<BPT> g0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) g0.v[j] = ld_coh(l2 + BPT * tid + j);
  // ---- totals (kept, candidates, first-digit bins by wave); per-block
  // candidate counts to LDS
  uint32_t gsum = 0u;
#pragma unroll
  for (int j = 0; j < BPT; ++j) gsum += g0.v[j];
  const uint32_t gincl = wave_incl_scan(gsum);  // bins of this wave's threads up to this one
  {
    const uint32_t sa = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(ca), 63);
    const uint32_t se = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(ce), 63);
    const uint32_t sg = (uint32_t)__builtin_amdgcn_readlane((int)gincl, 63);
    if (lane == 0) {
      s_tot[0][wave] = sa;
      s_tot[1][wave] = se;
      s_tot[2][wave] = sg;
    }
  }
  if (tid < nblk) {
    cntE[tid] = ce;
    chosen[tid] = 0u;
    chosen2[tid] = 0u;
  }
  if (tid == 0) {
    s_nb = 0u;
    s_thr = ~0ull;
    s_rest = 0u;
    s_pick0[0] = s_pick0[1] = s_pick0[2] = 0u;
  }
  __syncthreads();
  if (ce > (uint32_t)spec) s_rest = 1u;  // some block has candidates beyond the first round trip
  uint32_t A = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) A += s_tot[0][x];
  // every select block has added its bins: clear them (a store that depends
  // on the loaded value cannot overtake the load)
#pragma unroll
  for (int j = 0; j < BPT; ++j)
    if (g0.v[j] != 0u) l2[BPT * tid + j] = 0u;
  const uint32_t need = (uint32_t)k - min(A, (uint32_t)k);

  // every candidate once: f(x) on the lanes holding one (x = 0 elsewhere is
  // never passed); the counts of the register-held blocks are read first
  // (f(x, uni): uni when the wave's lanes calling f hold candidates of one block)
  auto for_all_u = [&](auto&& f) {
    bool has[kCoopCP];
#pragma unroll
    for (int m = 0; m < kCoopCP; ++m) {
      const int fi = tid + m * NT, b = fi >> lspec;
      has[m] = b < nblk && (uint32_t)(fi & (spec - 1)) < cntE[min(b, nblk - 1)];
    }
#pragma unroll
    for (int m = 0; m < kCoopCP; ++m)
      if (has[m]) f(expand(cv[m], (tid + m * NT) >> lspec), lspec >= 6);
    constexpr int TPB = 8;
    for (int b0 = 0; b0 < nblk; b0 += NT / TPB) {
      const int b = b0 + tid / TPB;
      const uint32_t eb = (b < nblk) ? cntE[b] : 0u;
      for (uint32_t i = spec + tid % TPB; i < eb; i += TPB)
        f(expand(ld_coh(cbase + (int64_t)b * CH + i), b), false);
    }
  };
  auto for_all = [&](auto&& f) { for_all_u([&](uint64_t x, bool) { f(x); }); };
  // chosen2[b] += lanes with ch set whose candidate is in block b (one LDS
  // add per distinct block of the wave)
  auto add_chosen = [&](bool ch, uint32_t b, bool uni) {
    uint64_t pend = __ballot(ch);
    if (uni) {
      if (pend && lane == __ffsll((unsigned long long)pend) - 1) atomicAdd(&chosen2[b], (uint32_t)__popcll(pend));
      return;
    }
    while (pend) {
      const int l = __ffsll((unsigned long long)pend) - 1;
      const uint32_t bl = (uint32_t)__builtin_amdgcn_readlane((int)b, l);
      const uint64_t mm = __ballot(ch && b == bl);
      if (lane == l) atomicAdd(&chosen2[bl], (uint32_t)__popcll(mm));
      pend &= ~mm;
    }
  };
  uint64_t thr = ~0ull;  // rank values (low 52 bits) >= thr are chosen; ~0: none
  if (need > 0) {
    // the first digit d0 with count(> d0) < need <= count(>= d0): thread t
    // holds bins [t BPT, (t+1) BPT); the bins above its own are the total
    // less the bins up to it
    {
      uint32_t gbel = gincl, gtot = 0u;
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        const uint32_t c = s_tot[2][x];
        gbel += (x < wave) ? c : 0u;
        gtot += c;
      }
      uint32_t acc = gtot - gbel;  // bins of higher threads
      if (acc < need && acc + gsum >= need) {
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
          if (acc < need && acc + g0.v[j] >= need) {
            s_pick0[0] = BPT * tid + j;
            s_pick0[1] = acc;
            s_pick0[2] = g0.v[j];
          }
          acc += g0.v[j];
        }
      }
    }
    __syncthreads();
    const uint32_t d0 = s_pick0[0], above0 = s_pick0[1], cnt0 = s_pick0[2];
    const uint32_t rem = need - min(above0, need);
    const bool whole = cnt0 == rem;
    // one pass: digits above d0 chosen (d0 too when its bucket is taken
    // whole); otherwise d0's candidates gathered for ranking
    if (lspec >= 6 && s_rest == 0u) {
      // every candidate is in registers, and the lanes of a wave holding
      // register m all hold candidates of block (tid + m*NT) >> lspec: the
      // chosen count of each (register, wave) is one ballot, kept in lane m
      // and stored once per wave; branch-free, so the registers interleave
      uint32_t cnt[kCoopCP];
#pragma unroll
      for (int m = 0; m < kCoopCP; ++m) cnt[m] = cntE[min((tid + m * NT) >> lspec, nblk - 1)];
      const uint32_t dlo = whole ? d0 : d0 + 1;  // chosen outright: digit >= dlo
      uint32_t pcv = 0u;
      uint64_t anyb = 0ull;
#pragma unroll
      for (int m = 0; m < kCoopCP; ++m) {
        const int fi = tid + m * NT;
        const bool has = ((fi >> lspec) < nblk) & ((uint32_t)(fi & (spec - 1)) < cnt[m]);
        const uint32_t dg = cv[m] >> 21;  // key bits 19..9
        const uint32_t c = (uint32_t)__popcll(__ballot(has & (dg >= dlo)));
        pcv = (lane == m) ? c : pcv;
        anyb |= __ballot(has & !whole & (dg == d0));
      }
      if (lane < kCoopCP) pcs[lane * NW + wave] = pcv;
      if (anyb) {  // the cut digit's candidates, for ranking
#pragma unroll
        for (int m = 0; m < kCoopCP; ++m) {
          const int fi = tid + m * NT;
          const bool has = ((fi >> lspec) < nblk) & ((uint32_t)(fi & (spec - 1)) < cnt[m]);
          const uint64_t mb = __ballot(has & ((cv[m] >> 21) == d0));
          if (mb) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_nb, (uint32_t)__popcll(mb));
            base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
            const uint32_t p = base + (uint32_t)__popcll(mb & lanemask_lt());
            if (((mb >> lane) & 1ull) && p < (uint32_t)kBucketMax) bucket[p] = expand(cv[m], fi >> lspec);
          }
        }
      }
      __syncthreads();
      // block b's candidates are registers' lanes [b*spec, (b+1)*spec): spec/64 waves' counts
      // (chosen[] is written here only, by its own thread; the other passes add to chosen2[])
      if (tid < nblk) {
        uint32_t c = 0;
        for (int f0 = tid * spec; f0 < (tid + 1) * spec; f0 += 64) c += pcs[(f0 / NT) * NW + (f0 % NT) / 64];
        chosen[tid] = c;
      }
    } else {
      for_all_u([&](uint64_t x, bool uni) {
        const uint32_t dg = (uint32_t)(x >> 41) & 2047u;
        const bool ch = dg > d0 || (whole && dg == d0);
        add_chosen(ch, rank_slot(x) / CH, uni);
        if (!whole && dg == d0) {
          const uint32_t p = atomicAdd(&s_nb, 1u);
          if (p < (uint32_t)kBucketMax) bucket[p] = x;
        }
      });
      __syncthreads();  // (the register pass ended with one)
    }
    const uint64_t low52 = (1ull << 52) - 1;
    if (whole) {
      thr = (uint64_t)d0 << 41;
    } else if (s_nb <= (uint32_t)kBucketMax) {
      // rank of each bucket member among the bucket (rank values are unique)
      const uint32_t nb = s_nb;
      bool ch = false;
      uint64_t x = 0;
      if ((uint32_t)tid < nb) {
        x = bucket[tid];
        uint32_t rk = 0;
        for (uint32_t i = 0; i < nb; ++i) rk += (bucket[i] > x) ? 1u : 0u;
        ch = rk < rem;
        if (rk + 1 == rem) s_thr = x & low52;
      }
      add_chosen(ch, rank_slot(x) / CH, false);
      __syncthreads();
      thr = s_thr;
    } else {
      // many equal leading bits (ties): radix selection over all candidates
      thr = radix_threshold<NT, true>(need, rhist, tmp, for_all, g0);
      for_all([&](uint64_t x) {
        add_chosen(((uint32_t)(x >> 41) & 2047u) == d0 && (x & low52) >= thr, rank_slot(x) / CH, false);
      });
    }
  }
  __syncthreads();
  // ---- output offsets: kept and chosen slots of the blocks before (by the
  // first wave alone when the row has at most 64 blocks)
  const bool one_wave = nblk <= 64;
  if (one_wave && wave != 0) return;
  const uint32_t vb = (tid < nblk) ? ca + chosen[tid] + chosen2[tid] : 0u;
  uint32_t tot, off;
  if (one_wave) {
    const uint32_t inc = wave_incl_scan(vb);
    off = inc - vb;
    tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  } else {
    off = block_scan<NT>(vb, tmp, &tot);
  }
  // the chosen candidates are those with (lo, ~slot) >= thr: with lo == kt,
  // the slots up to slot_t
  const bool none = thr == ~0ull;
  const uint32_t kt = (uint32_t)(thr >> 32) & 0xFFFFFu;
  const int64_t slot_t = (int64_t)(0xFFFFFFFFu - (uint32_t)(thr & 0xFFFFFFFFull));
  if (tid < nblk && (int64_t)tid * CH < nv) {
    const int64_t rel = min(max(slot_t - (int64_t)tid * CH + 1, (int64_t)0), (int64_t)CH);
    const uint64_t rec = coop_record(none, kt, (uint32_t)rel, gen, off);
    if (tid == (int)blockIdx.x) *own = rec;
    else st_coh(recs + tid, rec);
  }
  const uint32_t kept = min(tot, (uint32_t)k);  // k unless the histogram disagreed with the scores
  for (uint32_t i = kept + tid; i < (uint32_t)k; i += one_wave ? 64u : (uint32_t)NT) orow[i] = -1;
  if (count_out && tid == 0) count_out[r] = (int32_t)kept;
}

__global__ __launch_bounds__(kCoopThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void topk_coop_kernel(
    const float* __restrict__ scores, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t nv_add, const int32_t* __restrict__ slot_pos, int32_t k, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, TopkWs w, uint32_t gen, uint32_t wait_limit,
    float* __restrict__ gout) {
  // gout (optional, row stride k): each kept slot's score at its output
  // place (a candidate pool's scores, gathered for the selection inside it)
  constexpr int NT = kCoopThreads, NW = kCoopWaves, PL = kCoopPL;
  extern __shared__ uint64_t smem64[];
  uint32_t* smem = reinterpret_cast<uint32_t*>(smem64);
  __shared__ uint32_t tmp[NW];
  __shared__ uint32_t wtot[2][NW];  // kept / candidates per wave
  __shared__ int s_b1, s_last;
  __shared__ uint64_t s_rec;
  __shared__ uint32_t s_keys[kTopkChunk];  // the block's score keys, kept across the wait

  const int r = blockIdx.y, nblk = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  const int64_t start = (int64_t)blockIdx.x * kTopkChunk;
  uint32_t* rh = w.hist + (int64_t)r * w.hist_stride;
  int32_t* orow = idx_out + (int64_t)r * k;
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)r * n : nullptr;

  if (nv <= k) {
    // every visible slot is kept, in place; block 0 pads and clears the
    // histogram (no block reads it)
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int64_t s = start + j * NT + tid;
      if (s < nv) {
        orow[s] = sp ? sp[s] : (int32_t)s;
        if (gout) gout[(int64_t)r * k + s] = scores[(int64_t)r * n + s];
      }
    }
    if (blockIdx.x == 0) {
      for (int64_t j = nv + tid; j < k; j += NT) orow[j] = -1;
      if (count_out && tid == 0) count_out[r] = (int32_t)nv;
      uint4* h4p = reinterpret_cast<uint4*>(rh);
      for (int j = tid; j < w.hist_copies * kHistBins / 4; j += NT) h4p[j] = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  const bool active = start < nv;
  uint32_t* l2 = rh + kL2WordOffset;
  int32_t pos[PL];
  uint32_t* crow = w.counts + (int64_t)r * w.counts_stride + 2 * blockIdx.x;
  if (!active) {
    if (tid == 0) {
      st_coh(crow, 0u);
      st_coh(crow + 1, 0u);
    }
  } else {
    const float* srow = scores + (int64_t)r * n;
    // block-relative slots: thread slot wrel + 64 j is visible iff below nvb
    const int nvb = (int)min(nv - start, (int64_t)kTopkChunk);
    const int wrel = wave * 64 * PL + lane;
    float v[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) v[j] = srow[start + min(wrel + 64 * j, nvb - 1)];
#pragma unroll
    for (int j = 0; j < PL; ++j) pos[j] = sp ? sp[start + min(wrel + 64 * j, nvb - 1)] : 0;
    if (tid == 0) s_b1 = 0x7FFFFFFF;  // replaced below; keeps an inconsistent histogram harmless
    find_cut<NT>(rh, w.hist_copies, k, tmp, &s_b1);
    const uint32_t b1 = (uint32_t)s_b1;
    // keys of slots past the visible ones are 0: below every score's key
    // and below the cut bin's (b1 is the bin of a visible key)
    const uint32_t klo = b1 << kHistShift, khi = klo | ((1u << kHistShift) - 1u);
    uint32_t na = 0, ne = 0;
    uint32_t keys[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      keys[j] = (wrel + 64 * j < nvb) ? score_key(v[j]) : 0u;
      s_keys[wrel + 64 * j] = keys[j];
      na += (uint32_t)__popcll(__ballot(keys[j] > khi));
      ne += (uint32_t)__popcll(__ballot(keys[j] >= klo && keys[j] <= khi));
    }
    if (lane == 0) {
      wtot[0][wave] = na;
      wtot[1][wave] = ne;
    }
    __syncthreads();
    uint32_t oe = 0, ta = 0, te = 0;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const uint32_t c = wtot[1][x];
      oe += (x < wave) ? c : 0u;
      ta += wtot[0][x];
      te += c;
    }
    // the candidates' rank values, listed in slot order in the block's region
    // each as one word: key bits 19..0 above the block-relative slot's
    // complement (12 bits), so larger words rank first within the block
    uint32_t* rc = reinterpret_cast<uint32_t*>(w.cand + (int64_t)r * w.cand_stride) +
                   (int64_t)blockIdx.x * kTopkChunk;
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const bool eq = keys[j] >= klo && keys[j] <= khi;
      const uint64_t me = __ballot(eq);
      if (eq) {
        st_coh(rc + oe + (uint32_t)__popcll(me & lt),
               ((keys[j] & 0xFFFFFu) << 12) | (uint32_t)(kTopkChunk - 1 - (wrel + 64 * j)));
        atomicAdd(l2 + ((keys[j] >> 9) & 2047u), 1u);  // first radix digit: key bits 19..9
      }
      oe += (uint32_t)__popcll(me);
    }
    if (tid == 0) {
      st_coh(crow, ta);
      st_coh(crow + 1, te);
    }
  }
  // ---- arrival; the row's last block completes it
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  uint32_t* ctr = w.ctr + (int64_t)r * w.ctr_stride;
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == (uint32_t)nblk - 1u;
    if (s_last) {
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      w.cut[(int64_t)r * w.ctr_stride] = 0u;
    }
  }
  __syncthreads();
  uint64_t* recs = reinterpret_cast<uint64_t*>(rh + kRecWordOffset);
  if (s_last) {
    coop_complete(r, nv, k, nblk, orow, count_out, w, smem, tmp, rh, recs, &s_rec, gen);
    // every block of the row has read the histogram copies: leave them zero
    uint4* h4p = reinterpret_cast<uint4*>(rh);
    for (int j = tid; j < w.hist_copies * kHistBins / 4; j += NT) h4p[j] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }
  if (!active) return;
  // ---- this block's record
  if (tid == 0) {
    uint64_t rec = 0ull;
    if (s_last) {
      rec = s_rec;
    } else {
      // A wait limit of 0 gives up at once (the host forces the failure path).
      uint64_t* mine = recs + blockIdx.x;
      uint32_t it = 0;
      bool got = false;
      if (wait_limit > 0) {
        while (!(got = record_is(rec = ld_coh(mine), gen)) && ++it < wait_limit)
          __builtin_amdgcn_s_sleep(2);
      }
      if (got) st_coh(mine, (uint64_t)0);
      else {
        rec = 0ull;
        st_coh(ctr + 2, 1u);  // no record: the pass failed (csa2_workspace_check reports it)
      }
    }
    s_rec = rec;
  }
  __syncthreads();
  const uint64_t rec = s_rec;
  if ((rec >> 63) == 0ull) return;
  const bool none = (rec >> 62) & 1ull;
  const uint32_t kt = (uint32_t)(rec >> 42) & 0xFFFFFu;
  const int rel = (int)((rec >> 29) & 0x1FFFu);
  const uint32_t off = (uint32_t)rec & 0x7FFFu;
  // the block's kept slots: key above KT, or equal to KT at a block-relative
  // slot below rel (no candidate chosen: every key of the cut bin is at or
  // below KT and rel is 0); slots past the visible ones hold key 0 < KT
  const uint32_t b1 = (uint32_t)s_b1;
  const uint32_t KT = (b1 << kHistShift) | (none ? 0xFFFFFu : kt);
  const int relv = none ? 0 : rel;
  const int wrel = wave * 64 * PL + lane;
  // ---- kept slots of this block, in slot order, from offset `off`
  uint64_t msel[PL];
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const uint32_t key = s_keys[wrel + 64 * j];
    const bool sel = key > KT || (key == KT && wrel + 64 * j < relv);
    msel[j] = __ballot(sel);
    cnt += (uint32_t)__popcll(msel[j]);
  }
  if (lane == 0) wtot[0][wave] = cnt;
  __syncthreads();
  uint32_t o = off;
#pragma unroll
  for (int x = 0; x < NW; ++x) o += (x < wave) ? wtot[0][x] : 0u;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const uint32_t p = __builtin_amdgcn_mbcnt_hi((uint32_t)(msel[j] >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)msel[j], o));
    if (((msel[j] >> lane) & 1ull) && p < (uint32_t)k) {
      orow[p] = sp ? pos[j] : (int32_t)(start + wrel + 64 * j);
      if (gout) {  // the score back from its key (-0 comes back as +0, the same key)
        const uint32_t key = s_keys[wrel + 64 * j];
        gout[(int64_t)r * k + p] = __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
      }
    }
    o += (uint32_t)__popcll(msel[j]);
  }
}

// ------------------------------------------------------- one block per row
// Passes of many rows (at least kRowTopkMinRows) of up to kRowTopkMaxN
// slots: one block of kRowThreads per row does the whole selection in LDS,
// so no block waits on another and no histogram is built beforehand.
//   1. a 12-bit key histogram of the row and the bin b1 of the k-th largest;
//   2. a pass marking the slots above b1 in a bitmap and listing b1's
//      candidates (key, slot) -- or, if b1 holds more than kRowCand, further
//      passes over the row for the next digits;
//   3. the exact threshold key T from 11- and 9-bit histograms; keys above T
//      are kept, keys equal to T go to a tie bitmap whose lowest `need` slots
//      are kept (the lower slot wins a tie);
//   4. the kept slots written in slot order from the bitmaps.
constexpr int kRowThreads = 1024;
constexpr int kRowCand = 4096;

// The bin (of nbins, counted from the top) where the running count from the
// top reaches `need` (1 <= need <= total); *bin, *above (count in the bins
// above it) and, if given, *count (the bin's own count) are written by the
// thread that finds it.
template <int NT>
__device__ __forceinline__ void find_bin_desc(const uint32_t* h, int nbins, uint32_t need,
                                              uint32_t* tmp, uint32_t* bin, uint32_t* above,
                                              uint32_t* count = nullptr) {
  const int tid = threadIdx.x;
  constexpr int BPT = kHistBins / NT;  // at most 4 bins per thread
  const int bpt = nbins >= NT ? nbins / NT : 1;
  uint32_t c[BPT];
  uint32_t sum = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int d = tid * bpt + q;  // d-th bin from the top
    c[q] = (q < bpt && d < nbins) ? h[nbins - 1 - d] : 0u;
    sum += c[q];
  }
  uint32_t tot;
  uint32_t acc = block_scan<NT>(sum, tmp, &tot);
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    if (q < bpt && acc < need && acc + c[q] >= need) {
      *bin = (uint32_t)(nbins - 1 - (tid * bpt + q));
      *above = acc;
      if (count) *count = c[q];
    }
    acc += c[q];
  }
  __syncthreads();
}

// SMALL: rows of at most kRowTopkSmallN slots, whose keys the block loads
// once into registers (16 per thread) and every pass reads from there.
// The selection of row r by one block of NT threads (every thread calls
// it); `lds` is the block's dynamic LDS (kHistBins + 2 nwp + 2 kRowCand words).
template <bool SMALL, int NT = kRowThreads>
__device__ __forceinline__ void row_select(int r, const float* __restrict__ scores, int64_t n,
                                           const int32_t* __restrict__ n_valid, int32_t nv_add,
                                           const int32_t* __restrict__ slot_pos, int32_t k,
                                           int32_t* __restrict__ idx_out,
                                           int32_t* __restrict__ count_out, int32_t nwp,
                                           uint32_t* lds) {
  constexpr int NW = NT / 64, UN = 8;
  static_assert(!SMALL || NT == kRowThreads, "register batches of the row kernel");
  uint32_t* hist = lds;               // kHistBins
  uint32_t* keep = hist + kHistBins;  // nwp words: slots kept
  uint32_t* tie = keep + nwp;         // nwp words: slots whose key equals the threshold
  uint32_t* ckey = tie + nwp;         // kRowCand candidate keys
  uint32_t* cslot = ckey + kRowCand;  // and their slots
  __shared__ uint32_t tmp[NW];
  __shared__ uint32_t s_bin, s_above, s_ncand;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t nv = max(min((int64_t)n_valid[r] + nv_add, n), (int64_t)0);
  const float* srow = scores + (int64_t)r * n;
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)r * n : nullptr;
  int32_t* orow = idx_out + (int64_t)r * k;
  if (nv <= k) {  // every visible slot is kept, in place
    for (int64_t s = tid; s < k; s += NT) orow[s] = (s < nv) ? (sp ? sp[s] : (int32_t)s) : -1;
    if (count_out && tid == 0) count_out[r] = (int32_t)nv;
    return;
  }
  // the keys of batch `base` (UN-deep, coalesced): from registers for SMALL
  // rows (all loaded at once here), else loaded
  constexpr int NB = SMALL ? (int)(kRowTopkSmallN / (NT * UN)) : 1;
  static_assert(!SMALL || NB * NT * UN == kRowTopkSmallN, "register batches");
  uint32_t kr[SMALL ? NB * UN : 1];
  if constexpr (SMALL) {
#pragma unroll
    for (int x = 0; x < NB * UN; ++x) kr[x] = score_key(srow[min((int64_t)x * NT + tid, nv - 1)]);
  }
  auto batch_keys = [&](int64_t base, int bi, uint32_t (&key)[UN]) {
    if constexpr (SMALL) {
#pragma unroll
      for (int u = 0; u < UN; ++u) key[u] = kr[bi * UN + u];
    } else {
      float v[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) v[u] = srow[min(base + (int64_t)u * NT + tid, nv - 1)];
#pragma unroll
      for (int u = 0; u < UN; ++u) key[u] = score_key(v[u]);
    }
  };
  // body(base, bi) for every UN-deep batch of the row: SMALL rows run all NB
  // register batches (straight-line; slots past nv are not ok), others loop
  auto batches = [&](auto&& body) {
    if constexpr (SMALL) {
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) body((int64_t)bi * NT * UN, bi);
    } else {
      for (int64_t base = 0; base < nv; base += (int64_t)NT * UN) body(base, 0);
    }
  };
  // every slot of the row; fn runs on every lane (slots past nv have ok ==
  // false), so it may use ballots
  auto for_slots = [&](auto&& fn) {
    batches([&](int64_t base, int bi) {
      uint32_t key[UN];
      batch_keys(base, bi, key);
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int64_t s = base + (int64_t)u * NT + tid;
        fn(s, s < nv, key[u]);
      }
    });
  };
  // a wave's 64 consecutive slots start at an even word it alone writes
  auto mark_wave = [&](uint32_t* bm, int64_t s, uint64_t m) {
    if (lane == 0 && m) {
      const int64_t w0 = (s - lane) >> 5;
      bm[w0] |= (uint32_t)m;
      if (m >> 32) bm[w0 + 1] |= (uint32_t)(m >> 32);
    }
  };

  // ---- 1. 12-bit histogram, cut bin b1
  for (int j = tid; j < kHistBins + 2 * nwp; j += NT) lds[j] = 0u;
  __syncthreads();
  for_slots([&](int64_t, bool ok, uint32_t key) {
    if (ok) atomicAdd(&hist[key >> kHistShift], 1u);
  });
  __syncthreads();
  find_bin_desc<NT>(hist, kHistBins, (uint32_t)k, tmp, &s_bin, &s_above);
  const uint32_t b1 = s_bin, need1 = (uint32_t)k - s_above, cnt1 = hist[b1];
  __syncthreads();  // hist is reused below
  for (int j = tid; j < kHistBins; j += NT) hist[j] = 0u;
  if (tid == 0) s_ncand = 0u;
  __syncthreads();

  // ---- 2. slots above b1; the next digit (key bits 19..9) of b1's keys.
  // The bitmap words are still zero and each belongs to one wave, so they
  // are stored, not or-ed; a wave reserves room for a whole batch's
  // candidates with one counter update.
  const bool in_lds = cnt1 <= (uint32_t)kRowCand;
  batches([&](int64_t base, int bi) {
    uint32_t kb[UN];
    batch_keys(base, bi, kb);
    uint64_t mc[UN];
    uint32_t nc = 0;
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int64_t s = base + (int64_t)u * NT + tid;
      const bool ok = s < nv;
      const uint32_t key = kb[u], bin = key >> kHistShift;
      const uint64_t mk = __ballot(ok && bin > b1);
      if (lane == 0 && s - lane < nv) {
        const int64_t w0 = (s - lane) >> 5;
        keep[w0] = (uint32_t)mk;
        if (mk >> 32) keep[w0 + 1] = (uint32_t)(mk >> 32);
      }
      const bool isc = ok && bin == b1;
      if (isc) atomicAdd(&hist[(key >> 9) & 2047u], 1u);
      mc[u] = __ballot(isc);
      nc += (uint32_t)__popcll(mc[u]);
    }
    if (in_lds && nc) {  // wave-uniform
      uint32_t cb = 0;
      if (lane == 0) cb = atomicAdd(&s_ncand, nc);
      cb = __builtin_amdgcn_readfirstlane(cb);
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        if ((mc[u] >> lane) & 1ull) {
          const uint32_t p = cb + (uint32_t)__popcll(mc[u] & lanemask_lt());
          ckey[p] = kb[u];
          cslot[p] = (uint32_t)(base + (int64_t)u * NT + tid);
        }
        cb += (uint32_t)__popcll(mc[u]);
      }
    }
  });
  __syncthreads();
  find_bin_desc<NT>(hist, 2048, need1, tmp, &s_bin, &s_above);
  const uint32_t b2 = s_bin, need2 = need1 - s_above;
  const uint32_t p23 = (b1 << 11) | b2;  // key bits 31..9 of the threshold
  __syncthreads();
  for (int j = tid; j < 512; j += NT) hist[j] = 0u;
  __syncthreads();

  // ---- 3. the last digit (key bits 8..0), the threshold key, the marks
  if (in_lds) {
    for (uint32_t c = tid; c < cnt1; c += NT)
      if ((ckey[c] >> 9) == p23) atomicAdd(&hist[ckey[c] & 511u], 1u);
  } else {
    for_slots([&](int64_t, bool ok, uint32_t key) {
      if (ok && (key >> 9) == p23) atomicAdd(&hist[key & 511u], 1u);
    });
  }
  __syncthreads();
  find_bin_desc<NT>(hist, 512, need2, tmp, &s_bin, &s_above);
  const uint32_t T = (p23 << 9) | s_bin, need3 = need2 - s_above;
  if (in_lds) {
    for (uint32_t c = tid; c < cnt1; c += NT) {
      const uint32_t key = ckey[c], s = cslot[c];
      if (key > T) atomicOr(&keep[s >> 5], 1u << (s & 31));
      else if (key == T) atomicOr(&tie[s >> 5], 1u << (s & 31));
    }
  } else {
    for_slots([&](int64_t s, bool ok, uint32_t key) {
      const bool inb = ok && (key >> kHistShift) == b1;
      mark_wave(keep, s, __ballot(inb && key > T));
      mark_wave(tie, s, __ballot(inb && key == T));
    });
  }
  __syncthreads();

  // ---- 4. the lowest need3 tie slots join the kept ones; output in slot order
  const int nw = (int)((nv + 31) >> 5);
  const int wpt = (nw + NT - 1) / NT;  // words per thread, contiguous
  const int w_lo = min(tid * wpt, nw), w_hi = min(w_lo + wpt, nw);
  uint32_t tcount = 0;
  for (int w = w_lo; w < w_hi; ++w) tcount += (uint32_t)__popc(tie[w]);
  uint32_t tot;
  uint32_t tb = block_scan<NT>(tcount, tmp, &tot);  // tie slots before this thread's words
  uint32_t kcount = 0;
  for (int w = w_lo; w < w_hi; ++w) {
    uint32_t tw = tie[w], take = 0;
    const uint32_t c = (uint32_t)__popc(tw);
    if (tb + c <= need3) {
      take = tw;
    } else {
      for (uint32_t i = tb; i < need3; ++i) {  // the lowest need3 - tb bits
        take |= tw & (0u - tw);
        tw &= tw - 1u;
      }
    }
    tb += c;
    const uint32_t sel = keep[w] | take;
    keep[w] = sel;
    kcount += (uint32_t)__popc(sel);
  }
  uint32_t o = block_scan<NT>(kcount, tmp, &tot);  // tot == k
  for (int w = w_lo; w < w_hi; ++w) {
    uint32_t m = keep[w];
    while (m) {
      const int64_t s = (int64_t)w * 32 + (__ffs(m) - 1);
      orow[o++] = sp ? sp[s] : (int32_t)s;
      m &= m - 1u;
    }
  }
  if (count_out && tid == 0) count_out[r] = k;
}

template <bool SMALL>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(
    const float* __restrict__ scores, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t nv_add, const int32_t* __restrict__ slot_pos, int32_t k, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, int32_t nwp, const uint32_t* __restrict__ only) {
  if (only && only[blockIdx.x] == 0u) return;  // a row the sampled selection has finished
  extern __shared__ uint32_t lds[];
  row_select<SMALL>(blockIdx.x, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp,
                    lds);
}

// ------------------------------------------- one block per row: key band
// Rows of up to 2^14 slots (a candidate pool's rows, short contexts), one
// block of kBandThreads per row with the row's keys in registers (key 0,
// below every score's key, past the visible slots).  The per-key steps are
// ballots and lane counts, no per-key LDS atomic:
//   1. a sample of 4096 keys (4 per thread, spread over the row) is histogrammed
//      in 4096 bins over its own key range; the bins where the sample's
//      count from the top reaches e -+ (4 sqrt(e) + 8), e = k * samples /
//      slots the expected sample count above the k-th key, give two keys
//      1 <= L <= H;
//   2. one pass counts the keys at or above H and lists the keys in [L, H)
//      with their slots in LDS (ballots and lane counts);
//   3. if A = count(>= H) < k <= A + listed, the k-th largest of the row is
//      the (k - A)-th largest of the list: a 12-bit histogram of the listed
//      keys relative to L gives its bin, and that bin's members are ranked
//      directly (key, then the lower slot);
//   4. the kept slots (key above the threshold's, or equal with a slot not
//      after its) are written in slot order from one ballot per register.
// The sample only sets the bracket: when it misses (or the list or the cut
// bin overflows) the block runs the exact LDS selection of the row kernel
// instead, so the result is the same index set and order either way.
constexpr int kBandThreads = kRowThreads;  // 16 waves hide the latency of each step
constexpr int kBandCand = 4096;  // listed keys of the bracket
constexpr int kBandRank = 1024;  // members of the cut bin ranked directly

// Maximum over the wave (every lane gets it): DPP row shifts and row
// broadcasts, then lane 63's value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0x111, 0xF>(x));  // row_shr:1 (lanes without a source see 0)
  x = max(x, dpp_u32<0x112, 0xF>(x));  // row_shr:2
  x = max(x, dpp_u32<0x114, 0xF>(x));  // row_shr:4
  x = max(x, dpp_u32<0x118, 0xF>(x));  // row_shr:8
  x = max(x, dpp_u32<0x142, 0xA>(x));  // row_bcast:15 into rows 1 and 3
  x = max(x, dpp_u32<0x143, 0xC>(x));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Popcount of m's bits below this lane, plus c.
__device__ __forceinline__ uint32_t lane_rank(uint64_t m, uint32_t c) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, c));
}

// The bins (of kHistBins, counted from the top) where the running count
// from the top reaches need_a and need_b (each 0 to skip, else 1 <= need <=
// total): written to bin[0], bin[1] (and the count above bin[0] and its own
// count to *above_a, *count_a) by the threads that find them.  One scan.
template <int NT>
__device__ __forceinline__ void find_two_desc(const uint32_t* h, uint32_t need_a, uint32_t need_b,
                                              uint32_t* tmp, uint32_t* bin, uint32_t* above_a,
                                              uint32_t* count_a) {
  constexpr int BPT = kHistBins / NT;
  static_assert(BPT % 4 == 0, "16-byte reads");
  const int tid = threadIdx.x;
  // thread t takes bins BPT (NT - 1 - t) .. + BPT - 1, read as 16-byte words
  const uint4* hp = reinterpret_cast<const uint4*>(h) + (NT - 1 - tid) * (BPT / 4);
  uint32_t c[BPT];  // from the top
  uint32_t sum = 0u;
#pragma unroll
  for (int j = 0; j < BPT / 4; ++j) {
    const uint4 hv = hp[BPT / 4 - 1 - j];
    c[4 * j] = hv.w;
    c[4 * j + 1] = hv.z;
    c[4 * j + 2] = hv.y;
    c[4 * j + 3] = hv.x;
    sum += hv.x + hv.y + hv.z + hv.w;
  }
  // exclusive prefix over the block (the wave totals' slots are written
  // again only after the barrier that ends this call)
  constexpr int NW = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t inc = wave_incl_scan(sum);
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  uint32_t acc = inc - sum;
#pragma unroll
  for (int x = 0; x < NW; ++x) acc += (x < wave) ? tmp[x] : 0u;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const uint32_t b = (uint32_t)(kHistBins - 1 - (tid * BPT + q));
    if (acc < need_a && acc + c[q] >= need_a) {
      bin[0] = b;
      *above_a = acc;
      *count_a = c[q];
    }
    if (acc < need_b && acc + c[q] >= need_b) bin[1] = b;
    acc += c[q];
  }
  __syncthreads();
}

template <int G>  // 4G keys per thread: rows of up to 4G * kBandThreads slots
__global__ __launch_bounds__(kBandThreads) void topk_band_kernel(
    const float* __restrict__ scores, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t nv_add, const int32_t* __restrict__ slot_pos, int32_t k, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, int32_t nwp, uint32_t force_exact) {
  constexpr int NT = kBandThreads, NW = NT / 64, PER = 4 * G;
  static_assert(G >= 1 && G * NW <= 64, "segment counts in one wave");
  extern __shared__ uint32_t lds[];
  uint32_t* hist = lds;                // kHistBins bins (later the cut bin's members)
  uint32_t* ckey = hist + kHistBins;   // kBandCand listed keys
  uint32_t* cslot = ckey + kBandCand;  // and their slots
  __shared__ uint32_t tmp[NW];
  __shared__ uint32_t s_red[3][NW];
  __shared__ uint32_t s_cnt[G * NW];
  __shared__ uint32_t s_bin[2], s_above, s_count, s_ncand, s_nrank, s_ties;
  __shared__ uint64_t s_thr;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nv = max(min((int64_t)n_valid[r] + nv_add, n), (int64_t)0);
  const float* srow = scores + (int64_t)r * n;
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)r * n : nullptr;
  int32_t* orow = idx_out + (int64_t)r * k;
  if (nv <= k) {  // every visible slot is kept, in place
    for (int64_t s = tid; s < k; s += NT) orow[s] = (s < nv) ? (sp ? sp[s] : (int32_t)s) : -1;
    if (count_out && tid == 0) count_out[r] = (int32_t)nv;
    return;
  }
  if (nv > (int64_t)PER * NT) {  // not a shape of this kernel: the exact selection
    row_select<false, NT>(r, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, lds);
    return;
  }
  const int nvi = (int)nv;
  // Register group g of thread t holds slots 4 (g NT + t) + c, c = 0..3
  // (16-byte loads; the host launches this kernel only for rows of a
  // multiple of 4 slots, so a group is within the row whenever its first
  // slot is).  The sample is group (t / 4) mod G of thread t, loaded first.
  int ss[4];
  uint32_t ks[4];
  {
    const int s0 = 4 * (((tid >> 2) % G) * NT + tid);
    const float4 sv4 = (s0 < nvi) ? *reinterpret_cast<const float4*>(srow + s0)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    const float sf[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ss[j] = s0 + j;
      ks[j] = (ss[j] < nvi) ? score_key(sf[j]) : 0u;
    }
  }
  float4 v[G];
  int4 pos[G];  // the slot map's positions (read only with a slot map)
#pragma unroll
  for (int g = 0; g < G; ++g) pos[g] = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int s0 = 4 * (g * NT + tid);
    v[g] = (s0 < nvi) ? *reinterpret_cast<const float4*>(srow + s0) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (sp) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int s0 = 4 * (g * NT + tid);
      pos[g] = (s0 < nvi) ? *reinterpret_cast<const int4*>(sp + s0) : make_int4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < kHistBins / (4 * NT); ++j)
    reinterpret_cast<uint4*>(hist)[tid + j * NT] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) {
    s_ncand = 0u;
    s_nrank = 0u;
    s_ties = 0u;
  }

  // ---- 1. the sample: its count, key range and histogram
  {
    uint32_t nmn = 0u, mx = 0u, c = 0u;  // per thread: ~min, max, count
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool sv = ss[j] < nvi;
      nmn = max(nmn, sv ? ~ks[j] : 0u);
      mx = max(mx, sv ? ks[j] : 0u);
      c += (uint32_t)__popcll(__ballot(sv));
    }
    const uint32_t mn = ~wave_max_u32(nmn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
      s_red[0][wave] = mn;
      s_red[1][wave] = mx;
      s_red[2][wave] = c;
    }
  }
  __syncthreads();
  uint32_t bmin = 0xFFFFFFFFu, bmax = 0u, ns = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    bmin = min(bmin, s_red[0][w]);
    bmax = max(bmax, s_red[1][w]);
    ns += s_red[2][w];
  }
  // ns >= 1: slot 0 (thread 0, j = 0) is sampled and visible
  const uint32_t span = bmax - bmin;
  const int sh = span >= (uint32_t)kHistBins ? 32 - __clz((int)span) - 12 : 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (ss[j] < nvi) atomicAdd(&hist[(ks[j] - bmin) >> sh], 1u);
  __syncthreads();
  const float e = (float)k * (float)ns / (float)nvi;
  const float m = 4.0f * sqrtf(e) + 8.0f;
  const int r_hi = (int)floorf(e - m), r_lo = (int)ceilf(e + m);
  // r_hi < e < ns (k < visible slots); r_lo past ns: no lower bracket
  find_two_desc<NT>(hist, r_hi >= 1 ? (uint32_t)r_hi : 0u, r_lo <= (int)ns ? (uint32_t)r_lo : 0u,
                    tmp, s_bin, &s_above, &s_count);
  uint32_t H = 0xFFFFFFFFu, L = 1u;  // no finite score's key reaches 0xFFFFFFFF
  bool hnone = true;
  if (r_hi >= 1) {
    const uint64_t h64 = (uint64_t)bmin + ((uint64_t)(s_bin[0] + 1u) << sh);
    hnone = h64 >= 0xFFFFFFFFull;
    H = hnone ? 0xFFFFFFFFu : (uint32_t)h64;
  }
  if (r_lo <= (int)ns) L = max(bmin + (s_bin[1] << sh), 1u);
  // the bins are read (the find ends with a barrier): clear them for step 3
#pragma unroll
  for (int j = 0; j < kHistBins / (4 * NT); ++j)
    reinterpret_cast<uint4*>(hist)[tid + j * NT] = make_uint4(0u, 0u, 0u, 0u);

  // ---- 2. count at or above H, list [L, H)
  uint32_t key[PER];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int s0 = 4 * (g * NT + tid);
    key[4 * g] = (s0 < nvi) ? score_key(v[g].x) : 0u;
    key[4 * g + 1] = (s0 + 1 < nvi) ? score_key(v[g].y) : 0u;
    key[4 * g + 2] = (s0 + 2 < nvi) ? score_key(v[g].z) : 0u;
    key[4 * g + 3] = (s0 + 3 < nvi) ? score_key(v[g].w) : 0u;
  }
  {
    uint32_t na = 0u, nc = 0u;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const uint64_t mab = __ballot(key[x] >= H);
      const uint64_t mge = __ballot(key[x] >= L);
      na += (uint32_t)__popcll(mab);
      nc += (uint32_t)__popcll(mge & ~mab);
    }
    uint32_t cb = 0u;
    if (lane == 0) {
      s_red[0][wave] = na;
      if (nc) cb = atomicAdd(&s_ncand, nc);
    }
    cb = (uint32_t)__builtin_amdgcn_readfirstlane((int)cb);
    if (cb + nc <= (uint32_t)kBandCand) {  // else the list overflows: the exact path below
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const bool bd = key[x] >= L && key[x] < H;
        const uint64_t mb = __ballot(bd);
        if (bd) {
          const uint32_t p = lane_rank(mb, cb);
          ckey[p] = key[x];
          cslot[p] = (uint32_t)(4 * ((x >> 2) * NT + tid) + (x & 3));
        }
        cb += (uint32_t)__popcll(mb);
      }
    }
  }
  __syncthreads();
  uint32_t A = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) A += s_red[0][w];
  const uint32_t ncand = s_ncand;
  if (force_exact || A >= (uint32_t)k || A + ncand < (uint32_t)k || ncand > (uint32_t)kBandCand) {
    __syncthreads();  // every thread has read s_red and s_ncand
    row_select<false, NT>(r, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, lds);
    return;
  }

  // ---- 3. the (k - A)-th largest listed key: its bin relative to L, then
  // the bin's members ranked directly
  const uint32_t need = (uint32_t)k - A;
  const uint32_t top = hnone ? bmax : H - 1u;  // the listed keys are below H
  const uint32_t span2 = top > L ? top - L : 0u;
  const int sh2 = span2 >= (uint32_t)kHistBins ? 32 - __clz((int)span2) - 12 : 0;
  auto digit = [&](uint32_t kk) { return min((kk - L) >> sh2, (uint32_t)(kHistBins - 1)); };
  for (uint32_t c = tid; c < ncand; c += NT) atomicAdd(&hist[digit(ckey[c])], 1u);
  __syncthreads();
  find_two_desc<NT>(hist, need, 0u, tmp, s_bin, &s_above, &s_count);
  const uint32_t dc = s_bin[0], rem = need - s_above, cnt_c = s_count;
  if (cnt_c > (uint32_t)kBandRank) {  // thousands of keys in one bin (ties): the exact selection
    __syncthreads();
    row_select<false, NT>(r, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, lds);
    return;
  }
  uint64_t* mem = reinterpret_cast<uint64_t*>(hist);  // the bins are read: members go here
  for (uint32_t c = tid; c < ncand; c += NT) {
    const uint32_t kk = ckey[c];
    if (digit(kk) == dc) mem[atomicAdd(&s_nrank, 1u)] = rank_value(kk, cslot[c]);
  }
  __syncthreads();
  for (uint32_t i = tid; i < cnt_c; i += NT) {
    const uint64_t x = mem[i];
    uint32_t rk = 0u, eq = 0u;  // members ranked above; members of the same key (itself too)
    for (uint32_t j = 0; j < cnt_c; ++j) {
      const uint64_t y = mem[j];
      rk += (y > x) ? 1u : 0u;
      eq += ((y >> 32) == (x >> 32)) ? 1u : 0u;
    }
    if (rk + 1u == rem) {
      s_thr = x;
      s_ties = eq > 1u ? 1u : 0u;  // another key equals the threshold's
    }
  }
  __syncthreads();
  const uint64_t thr = s_thr;
  const uint32_t TK = (uint32_t)(thr >> 32), TS = rank_slot(thr);
  const bool ties = s_ties != 0u;

  // ---- 4. kept slots in slot order.  Segment (g, wave) is the 256
  // consecutive slots 4 (g NT + 64 wave) .. + 255, lane-major; a lane's kept
  // slots of the group take consecutive places after those of the lanes
  // below it.
  uint32_t sel[G], lex[G];
  uint32_t pcv = 0u;  // lane g: the count of segment (g, wave)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t bits = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t kk = key[4 * g + c];
      const uint32_t s = (uint32_t)(4 * (g * NT + tid) + c);
      const bool kept = ties ? (kk > TK || (kk == TK && s <= TS)) : kk >= TK;
      bits |= kept ? (1u << c) : 0u;
    }
    sel[g] = bits;
    const uint32_t cnt = (uint32_t)__popc(bits);
    const uint32_t inc = wave_incl_scan(cnt);
    lex[g] = inc - cnt;
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    pcv = (lane == g) ? tot : pcv;
  }
  if (lane < G) s_cnt[lane * NW + wave] = pcv;
  __syncthreads();
  // exclusive prefix of the segment counts in (g, wave) order: lane l holds
  // entry l = g NW + wave
  const uint32_t cl = lane < G * NW ? s_cnt[lane] : 0u;
  const uint32_t pre = wave_incl_scan(cl) - cl;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t p = (uint32_t)__builtin_amdgcn_readlane((int)pre, g * NW + wv) + lex[g];
    const uint32_t bits = sel[g];
    const int s0 = 4 * (g * NT + tid);
    const int q[4] = {pos[g].x, pos[g].y, pos[g].z, pos[g].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((bits >> c) & 1u) {
        if (p < (uint32_t)k) orow[p] = sp ? q[c] : s0 + c;
        ++p;
      }
    }
  }
  if (count_out && tid == 0) count_out[r] = k;
}

// The forced variant as the score-matrix selection sees it (the sampled
// prefill variants leave these passes their own choice).
static int32_t forced_select_variant() {
  const int32_t f = topk_variant_forced();
  return (f == kTopkSampled || f == kTopkSampledFallback) ? (int32_t)kTopkAuto : f;
}

bool topk_row_pass(int32_t rows, int64_t n_max) {
  const int32_t f = forced_select_variant();
  if (f == kTopkRow) return n_max <= kRowTopkMaxN;
  if (f == kTopkBand || f == kTopkBandExact) return n_max <= kRowTopkSmallN;
  if (f != kTopkAuto) return false;
  return (rows >= kRowTopkMinRows && n_max <= kRowTopkMaxN) || n_max <= kRowTopkSmallN;
}

static int32_t topk_blocks(int64_t n_max, int32_t chunk) {
  const int64_t b = (n_max + chunk - 1) / chunk;
  return (int32_t)(b < 1 ? 1 : b);
}

// Blocks of topk_coop_kernel the current device holds at once (0 if the
// query fails, which disables that variant).
static int64_t coop_capacity() {
  return device_resident_blocks((const void*)topk_coop_kernel, kCoopThreads, kCoopLds);
}

hipError_t launch_topk_hist(const float* scores, int32_t rows, int64_t n, const int32_t* n_valid,
                            int32_t nv_add, int64_t n_max, uint32_t* hist, int64_t hist_stride,
                            int32_t hist_copies, hipStream_t st, bool first) {
  const int64_t nchunks = (n_max + kTopkChunk - 1) / kTopkChunk;
  if (nchunks == 0) return hipSuccess;
  CSA2_KERNEL(first, true, topk_hist_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(256), 0, st,
                     scores, n, n_valid, nv_add, hist, hist_stride, hist_copies);
  return hipGetLastError();
}

// ------------------------------------------------ sampled prefill selection
// Threshold of row r from its samples (one block of kThrThreads per row,
// the samples held in registers): the key at which the count of visible
// samples from the top reaches M = 2 need / kSampleStride + 16 (need =
// min(k, visible slots)), to 20 bits (the 12-bit bin, then 12 more bits
// inside it); every sample at or above the M-th largest is at or above it.
// A row with at most M visible samples takes every visible slot (threshold
// 0).  force_fail sets an unreachable threshold, so every row with something
// to select takes the exact path.  Also clears the row's candidate count
// and fail word.
constexpr int kThrThreads = 512;
constexpr int kThrPer = 16;  // samples per thread: rows of up to 2^18 slots
static_assert(kThrThreads * kThrPer * kSampleStride >= kRowTopkMaxN, "samples fit the block");
__global__ __launch_bounds__(kThrThreads) void sample_threshold_kernel(
    const int32_t* __restrict__ n_valid, int32_t nv_add, int64_t n_max, int32_t k,
    SampledSel sel, uint32_t force_fail) {
  constexpr int NT = kThrThreads;
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t tmp[NT / 64];
  __shared__ uint32_t s_bin, s_above;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = max(min((int64_t)n_valid[r] + nv_add, n_max), (int64_t)0);
  const int nsv = (int)((nv + kSampleStride - 1) / kSampleStride);  // visible samples
  const int64_t need = min((int64_t)k, nv);
  const int M = (int)min((int64_t)nsv, 2 * need / kSampleStride + 16);
  const float* sr = sel.samp + (int64_t)r * sel.ns_stride;
  uint32_t thr = 0u;
  if (force_fail) {
    thr = 0xFFFFFFFFu;
  } else if (nsv > M) {
    // every load issued before any is used
    uint32_t key[kThrPer];
#pragma unroll
    for (int q = 0; q < kThrPer; ++q) {
      const int m = tid + q * NT;
      key[q] = (m < nsv) ? score_key(sr[m]) : 0u;
    }
    for (int j = tid; j < kHistBins; j += NT) hist[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kThrPer; ++q)
      if (tid + q * NT < nsv) atomicAdd(&hist[key[q] >> kHistShift], 1u);
    __syncthreads();
    find_bin_desc<NT>(hist, kHistBins, (uint32_t)M, tmp, &s_bin, &s_above);
    const uint32_t b1 = s_bin, rem = (uint32_t)M - s_above;
    for (int j = tid; j < kHistBins; j += NT) hist[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kThrPer; ++q)
      if (tid + q * NT < nsv && (key[q] >> kHistShift) == b1)
        atomicAdd(&hist[(key[q] >> 8) & (kHistBins - 1)], 1u);
    __syncthreads();
    find_bin_desc<NT>(hist, kHistBins, rem, tmp, &s_bin, &s_above);
    thr = (b1 << kHistShift) | (s_bin << 8);
  }
  if (tid == 0) {
    sel.thr[r] = thr;
    sel.count[r] = 0u;
    sel.fail[r] = 0u;
  }
}

// Exact Top-K of row r among its candidates (one block of 1024 per row, the
// candidates in registers): the key T of the need-th largest from 12-, 12-
// and 8-bit histograms; keys above T are kept, keys equal to T go to a tie
// bitmap whose lowest slots fill the rest (the lower slot wins a tie), and
// the kept slots are written in slot order, -1 after them.  A row whose
// list is short, overflowed, or was flagged is left to the exact path (its
// fail word set).
constexpr int kFinThreads = 1024;
constexpr int kFinPer = kCandCap / kFinThreads;
__global__ __launch_bounds__(kFinThreads) void sampled_final_kernel(
    const int32_t* __restrict__ n_valid, int32_t nv_add, int64_t n_max, int32_t k,
    int32_t* __restrict__ idx_out, SampledSel sel) {
  constexpr int NT = kFinThreads;
  extern __shared__ uint32_t fin_lds[];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t tmp[NT / 64];
  __shared__ uint32_t s_bin, s_above, s_cnt;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int64_t nv = max(min((int64_t)n_valid[r] + nv_add, n_max), (int64_t)0);
  const uint32_t need = (uint32_t)min((int64_t)k, nv);
  const uint32_t c = sel.count[r];
  if (sel.fail[r] != 0u || c > (uint32_t)kCandCap || c < need) {
    if (tid == 0) sel.fail[r] = 1u;
    return;
  }
  int32_t* orow = idx_out + (int64_t)r * k;
  const int nwords = (int)((nv + 31) >> 5);
  uint32_t* keep = fin_lds;        // nwords
  uint32_t* tie = keep + nwords;   // nwords
  const uint2* cr = sel.cand + (int64_t)r * kCandCap;
  uint32_t ck[kFinPer], cs[kFinPer];
#pragma unroll
  for (int q = 0; q < kFinPer; ++q) {
    const uint32_t x = tid + q * NT;
    const uint2 e = (x < c) ? cr[x] : make_uint2(0u, 0u);
    ck[q] = e.x;
    cs[q] = e.y;
  }
  for (int x = tid; x < nwords; x += NT) keep[x] = tie[x] = 0u;
  uint32_t T = 0u, above = 0u;
  if (need > 0u) {
    // three levels: bits 31..20, 19..8, 7..0 of the need-th largest key
    uint32_t pre = 0u;  // the key bits fixed so far
    for (int lvl = 0; lvl < 3; ++lvl) {
      const int shift = lvl == 0 ? 20 : (lvl == 1 ? 8 : 0);
      const int nb = lvl == 2 ? 256 : kHistBins;
      const int hi = lvl == 0 ? 32 : (lvl == 1 ? 20 : 8);  // bits above `hi` are fixed
      for (int j = tid; j < kHistBins; j += NT) hist[j] = 0u;
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kFinPer; ++q)
        if (tid + q * NT < c && (hi == 32 || (ck[q] >> hi) == pre))
          atomicAdd(&hist[(ck[q] >> shift) & (uint32_t)(nb - 1)], 1u);
      __syncthreads();
      find_bin_desc<NT>(hist, nb, need - above, tmp, &s_bin, &s_above, &s_cnt);
      above += s_above;
      pre = (hi == 32 ? 0u : (pre << (hi - shift))) | s_bin;
      // the bin holds exactly the keys still needed: every key with this
      // prefix is kept, so the threshold is the key just below the prefix
      // (no tie left to resolve) and the finer digits are not needed
      if (lvl < 2 && s_cnt == need - above && (pre << shift) != 0u) {
        above += s_cnt;
        pre = (pre << shift) - 1u;
        break;
      }
    }
    T = pre;
  }
  // keys above T kept; keys equal to T listed as ties
#pragma unroll
  for (int q = 0; q < kFinPer; ++q) {
    if (tid + q * NT < c && need > 0u) {
      if (ck[q] > T) atomicOr(&keep[cs[q] >> 5], 1u << (cs[q] & 31));
      else if (ck[q] == T) atomicOr(&tie[cs[q] >> 5], 1u << (cs[q] & 31));
    }
  }
  __syncthreads();
  // thread t takes words [t*wpt, (t+1)*wpt): the lowest need - above ties
  // join the kept slots, then every kept slot is written in slot order
  const int wpt = (nwords + NT - 1) / NT;
  const uint32_t tneed = need - above;
  uint32_t tc = 0;
  for (int q = 0; q < wpt; ++q) {
    const int wi = tid * wpt + q;
    if (wi < nwords) tc += (uint32_t)__popc(tie[wi]);
  }
  uint32_t tot;
  uint32_t tb = block_scan<NT>(tc, tmp, &tot);
  uint32_t kc = 0;
  for (int q = 0; q < wpt; ++q) {
    const int wi = tid * wpt + q;
    if (wi >= nwords) break;
    uint32_t m = tie[wi], kw = keep[wi];
    while (m && tb < tneed) {
      kw |= m & (~m + 1u);  // lowest tie of the word
      m &= m - 1u;
      ++tb;
    }
    keep[wi] = kw;  // this thread's own words
    kc += (uint32_t)__popc(kw);
  }
  uint32_t o = block_scan<NT>(kc, tmp, &tot);
  for (int q = 0; q < wpt; ++q) {
    const int wi = tid * wpt + q;
    if (wi >= nwords) break;
    uint32_t m = keep[wi];
    while (m) {
      const int bit = __builtin_ctz(m);
      if (o < (uint32_t)k) orow[o] = wi * 32 + bit;
      ++o;
      m &= m - 1u;
    }
  }
  for (uint32_t x = need + tid; x < (uint32_t)k; x += NT) orow[x] = -1;
}

hipError_t launch_sample_threshold(int32_t rows, const int32_t* n_valid, int32_t nv_add,
                                   int64_t n_max, int32_t k, const SampledSel& sel,
                                   bool force_fail, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  CSA2_KERNEL(true, true, sample_threshold_kernel, dim3((unsigned)rows), dim3(kThrThreads), 0, st,
              n_valid, nv_add, n_max, k, sel, force_fail ? 1u : 0u);
  return hipGetLastError();
}

hipError_t launch_sampled_final(int32_t rows, const int32_t* n_valid, int32_t nv_add,
                                int64_t n_max, int32_t k, int32_t* idx_out,
                                const SampledSel& sel, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (n_max > kRowTopkMaxN) return hipErrorInvalidValue;
  const size_t lds = (size_t)2 * ((n_max + 31) / 32) * 4;  // kept and tie bitmaps
  static const hipError_t raised = hipFuncSetAttribute(
      (const void*)sampled_final_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(2 * (kRowTopkMaxN / 32) * 4));
  if (raised != hipSuccess) return raised;
  CSA2_KERNEL(true, true, sampled_final_kernel, dim3((unsigned)rows), dim3(kFinThreads), lds, st,
              n_valid, nv_add, n_max, k, idx_out, sel);
  return hipGetLastError();
}

// Raised once per process (thread-safe static initialisation).
static hipError_t raise_row_lds() {
  static const hipError_t raised = []() {
    const int bytes = (int)((kHistBins + 2 * ((kRowTopkMaxN / 32 + 3) & ~3) + 2 * kRowCand) *
                            sizeof(uint32_t));
    const void* fns[] = {(const void*)topk_row_kernel<false>, (const void*)topk_row_kernel<true>,
                         (const void*)topk_band_kernel<1>, (const void*)topk_band_kernel<2>,
                         (const void*)topk_band_kernel<4>};
    hipError_t e = hipSuccess;
    for (const void* f : fns)
      if (e == hipSuccess) e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return e;
  }();
  return raised;
}

hipError_t launch_topk_row_failed(const float* scores, int32_t rows, int64_t n,
                                  const int32_t* n_valid, int32_t nv_add, int32_t k,
                                  int32_t* idx_out, const uint32_t* fail, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (n > kRowTopkMaxN) return hipErrorInvalidValue;
  const int32_t nwp = (int32_t)(((n + 31) / 32 + 3) & ~3);
  const size_t lds = (size_t)(kHistBins + 2 * nwp + 2 * kRowCand) * sizeof(uint32_t);
  hipError_t e = raise_row_lds();
  if (e != hipSuccess) return e;
  CSA2_KERNEL(true, true, topk_row_kernel<false>, dim3((unsigned)rows), dim3(kRowThreads), lds,
              st, scores, n, n_valid, nv_add, nullptr, k, idx_out, nullptr, nwp, fail);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int32_t rows, int64_t n,
                              const int32_t* n_valid, int32_t nv_add, int64_t n_max,
                              const int32_t* slot_pos, int32_t k, int32_t* idx_out,
                              int32_t* count_out, const TopkWs& w, hipStream_t st,
                              bool row_ok, float* gather_out, bool* gathered) {
  if (gathered) *gathered = false;
  // Many rows, no histogram built: one block per row.
  if (row_ok && topk_row_pass(rows, n_max)) {
    const int32_t nwp = (int32_t)(((n + 31) / 32 + 3) & ~3);
    const size_t lds = (size_t)(kHistBins + 2 * nwp + 2 * kRowCand) * sizeof(uint32_t);
    hipError_t e = raise_row_lds();
    if (e != hipSuccess) return e;
    // rows of up to 2^14 slots: the key band (unless the row kernel is forced)
    const int32_t fv = forced_select_variant();
    // (16-byte loads: row strides of a multiple of 4 slots, aligned bases)
    const bool aligned = n % 4 == 0 && ((uintptr_t)scores & 15u) == 0 &&
                         ((uintptr_t)slot_pos & 15u) == 0;
    if (fv != kTopkRow && n_max <= kRowTopkSmallN && aligned) {
      const uint32_t exact = fv == kTopkBandExact ? 1u : 0u;
      if (n_max <= 4 * kBandThreads)
        CSA2_KERNEL(true, true, topk_band_kernel<1>, dim3((unsigned)rows), dim3(kBandThreads), lds,
                    st, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, exact);
      else if (n_max <= 8 * kBandThreads)
        CSA2_KERNEL(true, true, topk_band_kernel<2>, dim3((unsigned)rows), dim3(kBandThreads), lds,
                    st, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, exact);
      else
        CSA2_KERNEL(true, true, topk_band_kernel<4>, dim3((unsigned)rows), dim3(kBandThreads), lds,
                    st, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, exact);
      set_topk_last(exact ? kTopkBandExact : kTopkBand);
      return hipGetLastError();
    }
    // rows of more than one batch and at most kRowTopkSmallN slots keep
    // their keys in registers (a 16K pool row: 1.8 us less per step of
    // three; a 4K row loads one batch either way and is faster without)
    if (n > (int64_t)kRowThreads * 8 && n <= kRowTopkSmallN)
      CSA2_KERNEL(true, true, topk_row_kernel<true>, dim3((unsigned)rows), dim3(kRowThreads), lds,
                  st, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, nullptr);
    else
      CSA2_KERNEL(true, true, topk_row_kernel<false>, dim3((unsigned)rows), dim3(kRowThreads), lds,
                  st, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, nwp, nullptr);
    set_topk_last(kTopkRow);
    return hipGetLastError();
  }
  // A variant forced by csa2_set_topk_variant runs when the pass allows it;
  // otherwise the choice falls back to the shape's own.
  int32_t forced = forced_select_variant();
  if (forced == kTopkBand || forced == kTopkBandExact) forced = kTopkAuto;  // rows too long for it
  // Passes whose blocks can all be resident at once take the one-wait variant.
  if (forced == kTopkAuto || forced == kTopkOneWait) {
    const int32_t nblk = topk_blocks(n_max, kTopkChunk);
    if (w.hist_copies <= 4 && nblk <= kCoopThreads &&
        (int64_t)rows * nblk <= coop_capacity()) {
      CSA2_KERNEL(true, true, topk_coop_kernel, dim3((unsigned)nblk, (unsigned)rows),
                  dim3(kCoopThreads), kCoopLds, st, scores, n, n_valid, nv_add, slot_pos, k,
                  idx_out, count_out, w, next_generation(), wait_limit(), gather_out);
      if (gathered) *gathered = gather_out != nullptr;
      set_topk_last(kTopkOneWait);
      return hipGetLastError();
    }
  }
  // many rows: bigger blocks (fewer, each with more scores)
  bool large = (int64_t)rows * topk_blocks(n_max, kTopkChunk) > 1024;
  if (forced >= kTopkSelect && forced <= kTopkSelectLargeCut) large = forced >= kTopkSelectLarge;
  const int32_t chunk = large ? kTopkChunkLarge : kTopkChunk;
  const int32_t nblk = topk_blocks(n_max, chunk);
  // LDS of the completing block: radix bins, 2 offset arrays, the kept-slot
  // bitmap (rows up to kBitmapSlots) or list, then as many candidates as fit.
  constexpr size_t kBudget = 150 * 1024;
  const int32_t bm_words = (n <= kBitmapSlots) ? (int32_t)(((n + 31) / 32 + 3) & ~3) : 0;
  const int32_t xwords = bm_words > 0 ? bm_words : k;
  const size_t fixed = (size_t)(2048 + 2 * (nblk + 1) + ((xwords + 1) & ~1)) * 4;
  int32_t lds_cand = fixed < kBudget ? (int32_t)((kBudget - fixed) / 8) : 0;
  if (lds_cand > 16384) lds_cand = 16384;
  const size_t lds = fixed + (size_t)lds_cand * 8;
  static const hipError_t raised = []() {
    hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel<4>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)topk_select_kernel<16>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    return e;
  }();
  if (raised != hipSuccess) return raised;
  // many blocks per row: find each row's cut once instead of in every block
  bool use_cut = (int64_t)rows * nblk > 1024;
  if (forced >= kTopkSelect && forced <= kTopkSelectLargeCut)
    use_cut = forced == kTopkSelectCut || forced == kTopkSelectLargeCut;
  set_topk_last((large ? (use_cut ? kTopkSelectLargeCut : kTopkSelectLarge)
                       : (use_cut ? kTopkSelectCut : kTopkSelect)) |
                (bm_words == 0 ? kTopkListFinish : 0));
  if (use_cut)
    CSA2_KERNEL(true, false, topk_cut_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, st,
                n_valid, nv_add, n, k, w);
  if (large)
    CSA2_KERNEL(!use_cut, true, topk_select_kernel<16>, dim3((unsigned)nblk, (unsigned)rows),
                dim3(kSelThreads), lds, st, scores, n, n_valid, nv_add, slot_pos, k, idx_out,
                count_out, w, lds_cand, bm_words, use_cut);
  else
    CSA2_KERNEL(!use_cut, true, topk_select_kernel<4>, dim3((unsigned)nblk, (unsigned)rows),
                dim3(kSelThreads), lds, st, scores, n, n_valid, nv_add, slot_pos, k, idx_out,
                count_out, w, lds_cand, bm_words, use_cut);
  return hipGetLastError();
}

}  // namespace csa2
