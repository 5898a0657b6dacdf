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
//  2. topk_select_kernel, many blocks per row: each block sums the copies and
//     finds the bin b1 holding the K-th key.  Its elements above b1 are kept;
//     those in b1 are candidates.  Both go to the block's own regions as
//     position-ordered lists (block-wide prefix sums, no atomics), with their
//     counts.
//  3. topk_final_kernel, one block per row: gathers the lists into LDS,
//     resolves the remaining entries among the candidates by radix selection
//     over the 64-bit rank values, keeps the chosen ones in position order,
//     merges the two sorted lists by binary search and writes the output.
//     It then clears the histogram copies for the next call.
// Every pass over memory issues all of a thread's loads before using them.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kPerThread = kTopkChunk / 256;  // scores per thread per select block
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(256) void topk_hist_kernel(const float* __restrict__ scores,
                                                        int64_t n,
                                                        const int32_t* __restrict__ n_valid,
                                                        int32_t nv_add,
                                                        uint32_t* __restrict__ hist,
                                                        int64_t hist_stride) {
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  const int64_t start = (int64_t)blockIdx.x * kTopkChunk;
  if (start >= nv) return;
  for (int k = threadIdx.x; k < kHistBins; k += 256) lhist[k] = 0u;
  const float* srow = scores + (int64_t)r * n;
  float v[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t s = start + j * 256 + threadIdx.x;
    v[j] = (s < nv) ? srow[s] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (start + j * 256 + threadIdx.x < nv) atomicAdd(&lhist[score_key(v[j]) >> kHistShift], 1u);
  __syncthreads();
  uint32_t* gh = hist + (int64_t)r * hist_stride + (blockIdx.x % kHistCopies) * kHistBins;
  for (int k = threadIdx.x; k < kHistBins; k += 256)
    if (lhist[k]) atomicAdd(gh + k, lhist[k]);
}

// Exclusive prefix sum over a block of NT threads; `tmp` holds NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
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
  return off + x - v;
}

__global__ __launch_bounds__(256) void topk_select_kernel(
    const float* __restrict__ scores, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t nv_add, int32_t k, const uint32_t* __restrict__ hist, int64_t hist_stride,
    TopkWs w) {
  __shared__ uint32_t tmp[8];
  __shared__ uint32_t cnt[kPerThread * 4];  // packed (above << 16 | cand) per (j, wave)
  __shared__ int s_b1;

  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  if (nv <= k) return;  // the final kernel takes every valid slot
  const int64_t start = (int64_t)blockIdx.x * kTopkChunk;
  uint32_t* crow = w.counts + (int64_t)r * w.counts_stride + 2 * blockIdx.x;
  if (start >= nv) {
    if (tid == 0) crow[0] = crow[1] = 0u;
    return;
  }
  const float* srow = scores + (int64_t)r * n;
  // scores of this thread: for each j the 4 waves cover 256 consecutive slots
  float v[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t s = start + 256 * j + 64 * wave + lane;
    v[j] = (s < nv) ? srow[s] : 0.0f;
  }
  // histogram of the row summed over its copies; this thread's bins [16t, 16t+16)
  uint32_t h16[16];
  {
    const uint32_t* rh = hist + (int64_t)r * hist_stride;
#pragma unroll
    for (int j = 0; j < 16; ++j) h16[j] = 0u;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) {
      const uint4* p = reinterpret_cast<const uint4*>(rh + c * kHistBins + 16 * tid);
      const uint4 a = p[0], b = p[1], d = p[2], e = p[3];
      h16[0] += a.x; h16[1] += a.y; h16[2] += a.z; h16[3] += a.w;
      h16[4] += b.x; h16[5] += b.y; h16[6] += b.z; h16[7] += b.w;
      h16[8] += d.x; h16[9] += d.y; h16[10] += d.z; h16[11] += d.w;
      h16[12] += e.x; h16[13] += e.y; h16[14] += e.z; h16[15] += e.w;
    }
  }
  if (tid == 0) s_b1 = 0x7FFFFFFF;  // replaced below; keeps an inconsistent histogram harmless
  {
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += h16[j];
    uint32_t total;
    const uint32_t excl = block_exclusive_scan256(sum, tmp, &total);
    const uint32_t above = total - excl - sum;  // elements in bins of higher threads
    if (above < (uint32_t)k && above + sum >= (uint32_t)k) {
      uint32_t acc = above;
      bool found = false;
#pragma unroll
      for (int j = 15; j >= 0; --j) {
        if (!found && acc + h16[j] >= (uint32_t)k) {
          s_b1 = 16 * tid + j;
          found = true;
        }
        acc += h16[j];
      }
    }
    __syncthreads();
  }
  const uint32_t b1 = (uint32_t)s_b1;
  // counts per (j, wave), packed above << 16 | candidates
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t s = start + 256 * j + 64 * wave + lane;
    const uint32_t bin = (s < nv) ? (score_key(v[j]) >> kHistShift) : 0u;
    const uint32_t na = (uint32_t)__popcll(__ballot(s < nv && bin > b1));
    const uint32_t ne = (uint32_t)__popcll(__ballot(s < nv && bin == b1));
    if (lane == 0) cnt[4 * j + wave] = (na << 16) | ne;
  }
  __syncthreads();
  // exclusive offsets in (j, wave) order = slot order
  static_assert(kPerThread * 4 <= 256, "one count per thread");
  uint32_t total;
  const uint32_t mine = (tid < kPerThread * 4) ? cnt[tid] : 0u;
  const uint32_t excl = block_exclusive_scan256(mine, tmp, &total);
  if (tid < kPerThread * 4) cnt[tid] = excl;
  __syncthreads();
  uint32_t* ra = w.above + (int64_t)r * w.above_stride + (int64_t)blockIdx.x * kTopkChunk;
  uint64_t* rc = w.cand + (int64_t)r * w.cand_stride + (int64_t)blockIdx.x * kTopkChunk;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t s = start + 256 * j + 64 * wave + lane;
    const uint32_t key = (s < nv) ? score_key(v[j]) : 0u;
    const uint32_t bin = key >> kHistShift;
    const bool ab = s < nv && bin > b1;
    const bool eq = s < nv && bin == b1;
    const uint64_t ma = __ballot(ab), me = __ballot(eq);
    const uint32_t base = cnt[4 * j + wave];
    if (ab) ra[(base >> 16) + (uint32_t)__popcll(ma & lanemask_lt())] = (uint32_t)s;
    if (eq) rc[(base & 0xFFFFu) + (uint32_t)__popcll(me & lanemask_lt())] = rank_value(key, (uint32_t)s);
  }
  if (tid == 0) {
    crow[0] = total >> 16;
    crow[1] = total & 0xFFFFu;
  }
}

__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(
    int64_t n, const int32_t* __restrict__ n_valid, int32_t nv_add,
    const int32_t* __restrict__ slot_pos, int32_t k, int32_t nblk, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, uint32_t* __restrict__ hist, int64_t hist_stride,
    TopkWs w, int32_t lds_cand) {
  extern __shared__ uint32_t smem[];
  uint32_t* rhist = smem;                      // 2048 radix bins
  uint32_t* offA = rhist + 2048;               // nblk + 1
  uint32_t* offE = offA + (nblk + 1);          // nblk + 1
  uint32_t* list = offE + (nblk + 1);          // k: kept positions (above, then chosen)
  uint64_t* cl = reinterpret_cast<uint64_t*>(list + ((k + 1) & ~1));  // lds_cand candidates
  __shared__ uint32_t tmp[16];
  __shared__ int s_dig;
  __shared__ uint32_t s_dig_above;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  int32_t* orow = idx_out + (int64_t)r * k;
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)r * n : nullptr;
  uint32_t* rh = hist + (int64_t)r * hist_stride;

  if (nv <= k) {
    for (int j = tid; j < k; j += kFinalThreads) orow[j] = (j < nv) ? (sp ? sp[j] : j) : -1;
    if (count_out && tid == 0) count_out[r] = (int32_t)nv;
  } else {
    // ---- per-block counts -> offsets
    const uint32_t* crow = w.counts + (int64_t)r * w.counts_stride;
    const int per = (nblk + kFinalThreads - 1) / kFinalThreads;
    uint32_t a_loc = 0, e_loc = 0;
    for (int j = 0; j < per; ++j) {
      const int b = tid * per + j;
      if (b < nblk) {
        a_loc += crow[2 * b];
        e_loc += crow[2 * b + 1];
      }
    }
    uint32_t A, C;
    uint32_t ra = block_scan<kFinalThreads>(a_loc, tmp, &A);
    uint32_t rc = block_scan<kFinalThreads>(e_loc, tmp, &C);
    for (int j = 0; j < per; ++j) {
      const int b = tid * per + j;
      if (b < nblk) {
        offA[b] = ra;
        offE[b] = rc;
        ra += crow[2 * b];
        rc += crow[2 * b + 1];
      }
    }
    if (tid == 0) {
      offA[nblk] = A;
      offE[nblk] = C;
    }
    __syncthreads();
    const uint32_t need = (uint32_t)k - min(A, (uint32_t)k);
    // list element c of a family of per-block regions: block = last b with off[b] <= c
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
      return cbase[(int64_t)b * kTopkChunk + (c - offE[b])];
    };
    // ---- gather the kept ("above") positions and the candidates
    const uint32_t Ak = min(A, (uint32_t)k);
    for (uint32_t c0 = 0; c0 < Ak; c0 += kFinalThreads * 4) {
      uint32_t t[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t c = c0 + u * kFinalThreads + tid;
        if (c < Ak) {
          const int b = block_of(offA, c);
          t[u] = abase[(int64_t)b * kTopkChunk + (c - offA[b])];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t c = c0 + u * kFinalThreads + tid;
        if (c < Ak) list[c] = t[u];
      }
    }
    const bool in_lds = C <= (uint32_t)lds_cand;
    if (in_lds) {
      for (uint32_t c0 = 0; c0 < C; c0 += kFinalThreads * 4) {
        uint64_t t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t c = c0 + u * kFinalThreads + tid;
          if (c < C) t[u] = cand_at(c);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t c = c0 + u * kFinalThreads + tid;
          if (c < C) cl[c] = t[u];
        }
      }
    }
    __syncthreads();
    auto for_each = [&](auto&& f) {
      if (in_lds) {
        for (uint32_t c = tid; c < C; c += kFinalThreads) f(cl[c]);
      } else {
        for (uint32_t c0 = 0; c0 < C; c0 += kFinalThreads * 4) {
          uint64_t t[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t c = c0 + u * kFinalThreads + tid;
            if (c < C) t[u] = cand_at(c);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c0 + u * kFinalThreads + tid < C) f(t[u]);
        }
      }
    };
    // ---- radix selection of the need-th largest rank value among the
    // candidates (all share the 12 top bits b1): 11-bit digits at shifts 41,
    // 30, 19, 8, then 8 bits at 0; stop once a whole bucket is taken.
    uint64_t thr = ~0ull;
    if (need > 0) {
      uint64_t prefix = 0;
      uint32_t rem = need;
      const int shifts[5] = {41, 30, 19, 8, 0};
      const int widths[5] = {11, 11, 11, 11, 8};
      for (int p = 0; p < 5; ++p) {
        const int sh = shifts[p], wd = widths[p];
        const int nb = 1 << wd;
        for (int j = tid; j < 2048; j += kFinalThreads) rhist[j] = 0u;
        if (tid == 0) {
          s_dig = 0;
          s_dig_above = 0;
        }
        __syncthreads();
        const uint64_t hi_mask = (~0ull << (sh + wd)) & ((1ull << 52) - 1);
        for_each([&](uint64_t x) {
          if ((x & hi_mask) == prefix) atomicAdd(&rhist[(uint32_t)(x >> sh) & (uint32_t)(nb - 1)], 1u);
        });
        __syncthreads();
        // digit d with count(> d) < rem <= count(>= d); 2 bins per thread
        const int b0 = 2 * tid;
        const uint32_t c0v = (b0 < nb) ? rhist[b0] : 0u, c1v = (b0 + 1 < nb) ? rhist[b0 + 1] : 0u;
        uint32_t tot;
        const uint32_t ex = block_scan<kFinalThreads>(c0v + c1v, tmp, &tot);
        const uint32_t above = tot - ex - c0v - c1v;
        if (above < rem && above + c1v >= rem) {
          s_dig = b0 + 1;
          s_dig_above = above;
        } else if (above + c1v < rem && above + c1v + c0v >= rem) {
          s_dig = b0;
          s_dig_above = above + c1v;
        }
        __syncthreads();
        const uint32_t d = (uint32_t)s_dig;
        rem -= s_dig_above;
        prefix |= (uint64_t)d << sh;
        const bool whole_bucket = rhist[d] == rem;
        __syncthreads();
        if (whole_bucket) break;
      }
      thr = prefix;
    }
    // ---- chosen candidates (rank value within b1 >= thr), kept in slot
    // order: the concatenated candidate regions are slot-ordered.
    const uint64_t low52 = (1ull << 52) - 1;
    uint32_t kept;  // k unless the histogram disagreed with the scores
    {
      const uint32_t per_c = (C + kFinalThreads - 1) / kFinalThreads;
      const uint32_t lo = min(tid * per_c, C), hi = min(lo + per_c, C);
      uint32_t cnt = 0;
      for (uint32_t c = lo; c < hi; ++c) {
        const uint64_t x = in_lds ? cl[c] : cand_at(c);
        cnt += (need > 0 && (x & low52) >= thr) ? 1u : 0u;
      }
      uint32_t tot;
      uint32_t o = Ak + block_scan<kFinalThreads>(cnt, tmp, &tot);
      kept = Ak + min(tot, need);
      for (uint32_t c = lo; c < hi; ++c) {
        const uint64_t x = in_lds ? cl[c] : cand_at(c);
        if (need > 0 && (x & low52) >= thr && o < kept) list[o++] = rank_slot(x);
      }
    }
    __syncthreads();
    // ---- merge list[0, Ak) and list[Ak, kept) (both ascending) into orow
    for (uint32_t i = tid; i < (uint32_t)k; i += kFinalThreads) {
      if (i >= kept) {
        orow[i] = -1;
        continue;
      }
      const uint32_t x = list[i];
      uint32_t lo, hi;  // lower bound of x in the other list
      if (i < Ak) { lo = Ak; hi = kept; } else { lo = 0; hi = Ak; }
      const uint32_t base = lo;
      while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (list[mid] < x) lo = mid + 1; else hi = mid;
      }
      const uint32_t pos = (i < Ak) ? i + (lo - base) : (i - Ak) + lo;
      orow[pos] = sp ? sp[x] : (int32_t)x;
    }
    if (count_out && tid == 0) count_out[r] = (int32_t)kept;
  }
  // ---- leave the histogram copies zero for the next call
  uint4* h4 = reinterpret_cast<uint4*>(rh);
  for (int j = tid; j < kHistCopies * kHistBins / 4; j += kFinalThreads) h4[j] = make_uint4(0, 0, 0, 0);
}

static int32_t topk_blocks(int64_t n_max) {
  const int64_t b = (n_max + kTopkChunk - 1) / kTopkChunk;
  return (int32_t)(b < 1 ? 1 : b);
}

hipError_t launch_topk_hist(const float* scores, int32_t rows, int64_t n, const int32_t* n_valid,
                            int32_t nv_add, int64_t n_max, uint32_t* hist, int64_t hist_stride,
                            hipStream_t st) {
  const int64_t nchunks = (n_max + kTopkChunk - 1) / kTopkChunk;
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(256), 0, st,
                     scores, n, n_valid, nv_add, hist, hist_stride);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int32_t rows, int64_t n,
                              const int32_t* n_valid, int32_t nv_add, int64_t n_max,
                              const int32_t* slot_pos, int32_t k, int32_t* idx_out,
                              int32_t* count_out, const TopkWs& w, hipStream_t st) {
  const int32_t nblk = topk_blocks(n_max);
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)nblk, (unsigned)rows), dim3(256), 0, st,
                     scores, n, n_valid, nv_add, k, w.hist, w.hist_stride, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // final kernel: LDS = radix bins + 2 offset arrays + k list + candidates
  const size_t fixed = (size_t)(2048 + 2 * (nblk + 1) + ((k + 1) & ~1)) * 4;
  const size_t budget = 150 * 1024;
  int32_t lds_cand = (int32_t)((budget - fixed) / 8);
  if (lds_cand > 16384) lds_cand = 16384;
  if (lds_cand < 0) lds_cand = 0;
  const size_t lds = fixed + (size_t)lds_cand * 8;
  static bool lds_raised = false;
  if (!lds_raised) {
    e = hipFuncSetAttribute((const void*)topk_final_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)budget);
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)rows), dim3(kFinalThreads), lds, st, n,
                     n_valid, nv_add, slot_pos, k, nblk, idx_out, count_out, w.hist, w.hist_stride,
                     w, lds_cand);
  return hipGetLastError();
}

}  // namespace csa2
