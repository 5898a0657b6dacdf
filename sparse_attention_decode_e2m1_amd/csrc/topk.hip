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
//  1. A 4096-bin histogram of the top 12 key bits per row (built by the
//     scoring kernel, or by topk_hist_kernel).
//  2. topk_select_kernel, many blocks per row: every block finds the bin b1
//     holding the K-th key from the histogram; elements above b1 are kept
//     (written as full 32-bit words of a per-row bitmap -- each word belongs
//     to exactly one wave, so no atomics), elements in b1 are appended to a
//     candidate list.  The last block of the row to finish (counted with a
//     device-scope atomic after a release fence) resolves the remaining
//     `need` entries by radix selection over the candidates (or over the
//     whole row when the candidate list overflowed, e.g. for tie storms),
//     merges them into the bitmap segment by segment in LDS and writes the
//     kept slots ascending.  It then clears the histogram and counters.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kSegWords = 4096;  // bitmap words merged per LDS segment

__global__ __launch_bounds__(256) void topk_hist_kernel(const float* __restrict__ scores,
                                                        int64_t n,
                                                        const int32_t* __restrict__ n_valid,
                                                        int32_t nv_add,
                                                        uint32_t* __restrict__ hist,
                                                        int64_t hist_stride, int32_t chunk) {
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  const int64_t start = (int64_t)blockIdx.x * chunk;
  if (start >= nv) return;
  const int64_t end = min(nv, start + chunk);
  for (int k = threadIdx.x; k < kHistBins; k += 256) lhist[k] = 0u;
  __syncthreads();
  const float* srow = scores + (int64_t)r * n;
  for (int64_t s = start + threadIdx.x; s < end; s += 256)
    atomicAdd(&lhist[score_key(srow[s]) >> kHistShift], 1u);
  __syncthreads();
  uint32_t* gh = hist + (int64_t)r * hist_stride;
  for (int k = threadIdx.x; k < kHistBins; k += 256)
    if (lhist[k]) atomicAdd(gh + k, lhist[k]);
}

// Find the bin holding the `need`-th largest element.  `bins` (nbins, a
// multiple of 256) are counts in ascending bin order.  Returns the bin and
// the number of elements in bins above it, through LDS broadcast slots.
template <typename LoadBin>
__device__ void find_cut(int nbins, uint32_t need, LoadBin load, uint32_t* tmp, int* cut_bin,
                         uint32_t* cut_above) {
  const int per = nbins / 256;
  const int tid = threadIdx.x;
  uint32_t sum = 0;
  for (int j = 0; j < per; ++j) sum += load(tid * per + j);
  uint32_t total;
  const uint32_t excl = block_exclusive_scan256(sum, tmp, &total);
  const uint32_t above = total - excl - sum;  // elements in bins of higher threads
  if (above < need && above + sum >= need) {
    uint32_t acc = above;
    for (int j = per - 1; j >= 0; --j) {
      const uint32_t c = load(tid * per + j);
      if (acc + c >= need) {
        *cut_bin = tid * per + j;
        *cut_above = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t ld_acquire_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_acquire_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void topk_select_kernel(
    const float* __restrict__ scores, int64_t n, const int32_t* __restrict__ n_valid,
    int32_t nv_add, const int32_t* __restrict__ slot_pos, int32_t k, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ count_out, uint32_t* __restrict__ hist, int64_t hist_stride,
    TopkCtl* __restrict__ ctl_base, int64_t ctl_stride, uint64_t* __restrict__ cand,
    int32_t cand_cap, uint32_t* __restrict__ bitmap, int64_t bm_words, int32_t chunk) {
  extern __shared__ uint32_t smem[];
  uint32_t* rhist = smem;                 // 2048 radix bins
  uint32_t* segw = smem + 2048;           // kSegWords bitmap words
  uint32_t* chosen = segw + kSegWords;    // k slots
  __shared__ uint32_t tmp[8];
  __shared__ int s_b1;
  __shared__ uint32_t s_above;
  __shared__ int s_last;
  __shared__ int s_dig;
  __shared__ uint32_t s_dig_above;
  __shared__ uint32_t s_nch;
  __shared__ uint32_t s_out;

  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nv = min((int64_t)n_valid[r] + nv_add, n);
  if (tid == 0) {
    s_b1 = 0x7FFFFFFF;  // replaced by find_cut; keeps an inconsistent histogram harmless
    s_above = 0;
    s_dig = 0;
    s_dig_above = 0;
  }
  __syncthreads();
  const float* srow = scores + (int64_t)r * n;
  uint32_t* bm = bitmap + (int64_t)r * bm_words;
  const uint32_t* rh = hist + (int64_t)r * hist_stride;
  TopkCtl* ctl = ctl_base + (int64_t)r * ctl_stride;

  if (nv > k) {
    find_cut(kHistBins, (uint32_t)k, [&](int j) { return rh[j]; }, tmp, &s_b1, &s_above);
    const uint32_t b1 = (uint32_t)s_b1;
    const int64_t start = (int64_t)blockIdx.x * chunk;
    const int64_t end = min(nv, start + chunk);
    for (int64_t base = start + 64 * wave; base < end; base += 256) {
      const int64_t s = base + lane;
      const bool valid = s < end;
      const uint32_t key = valid ? score_key(srow[s]) : 0u;
      const uint32_t bin = key >> kHistShift;
      const bool above = valid && bin > b1;
      const bool eq = valid && bin == b1;
      const uint64_t ma = __ballot(above);
      if (lane == 0) bm[base >> 5] = (uint32_t)ma;
      if (lane == 32 && base + 32 < end) bm[(base >> 5) + 1] = (uint32_t)(ma >> 32);
      const uint64_t me = __ballot(eq);
      if (me) {
        uint32_t cbase = 0;
        if (lane == 0) cbase = atomicAdd(&ctl->cand, (uint32_t)__popcll(me));
        cbase = __shfl(cbase, 0, kWave);
        if (eq) {
          const uint32_t pos = cbase + (uint32_t)__popcll(me & lanemask_lt());
          if (pos < (uint32_t)cand_cap)
            cand[(int64_t)r * cand_cap + pos] = rank_value(key, (uint32_t)s);
        }
      }
    }
  }

  // ---- last block of the row finishes the selection
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&ctl->done, 1u) == gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  int32_t* orow = idx_out + (int64_t)r * k;
  const int32_t* sp = slot_pos ? slot_pos + (int64_t)r * n : nullptr;
  if (nv <= k) {
    for (int j = tid; j < k; j += 256) orow[j] = (j < nv) ? (sp ? sp[j] : j) : -1;
    if (count_out && tid == 0) count_out[r] = (int32_t)nv;
  } else {
    const uint32_t b1 = (uint32_t)s_b1;
    const uint32_t need = (uint32_t)k - s_above;
    const uint32_t C = ld_acquire_u32(&ctl->cand);
    const bool from_cand = C <= (uint32_t)cand_cap;
    const uint64_t* crow = cand + (int64_t)r * cand_cap;
    // Visit every element of bin b1 with its 64-bit rank value.
    auto for_each = [&](auto&& f) {
      if (from_cand) {
        for (uint32_t j = tid; j < C; j += 256) f(ld_acquire_u64(crow + j));
      } else {
        for (int64_t s = tid; s < nv; s += 256) {
          const uint32_t key = score_key(srow[s]);
          if ((key >> kHistShift) == b1) f(rank_value(key, (uint32_t)s));
        }
      }
    };
    // Radix selection of the need-th largest rank value below the 12 known
    // top bits: digits of 11 bits at shifts 41, 30, 19, 8, then 8 bits at 0.
    uint64_t prefix = (uint64_t)b1 << 52;
    uint32_t rem = need;
    const int shifts[5] = {41, 30, 19, 8, 0};
    const int widths[5] = {11, 11, 11, 11, 8};
    for (int p = 0; p < 5; ++p) {
      const int sh = shifts[p], wd = widths[p];
      const int nb = 1 << wd;
      for (int j = tid; j < 2048; j += 256) rhist[j] = 0u;
      __syncthreads();
      const uint64_t hi_mask = ~0ull << (sh + wd);
      for_each([&](uint64_t v) {
        if ((v & hi_mask) == (prefix & hi_mask))
          atomicAdd(&rhist[(uint32_t)(v >> sh) & (uint32_t)(nb - 1)], 1u);
      });
      __syncthreads();
      find_cut(nb < 256 ? 256 : nb, rem, [&](int j) { return j < nb ? rhist[j] : 0u; }, tmp,
               &s_dig, &s_dig_above);
      const uint32_t d = (uint32_t)s_dig;
      rem -= s_dig_above;
      prefix |= (uint64_t)d << sh;
      const bool whole_bucket = rhist[d] == rem;
      __syncthreads();
      if (whole_bucket) break;
    }
    const uint64_t thr = prefix;  // keep every element of bin b1 with v >= thr
    if (tid == 0) s_nch = 0;
    __syncthreads();
    for_each([&](uint64_t v) {
      if (v >= thr) {
        const uint32_t c = atomicAdd(&s_nch, 1u);
        if (c < (uint32_t)k) chosen[c] = rank_slot(v);
      }
    });
    if (tid == 0) s_out = 0;
    __syncthreads();
    const uint32_t nch = min(s_nch, (uint32_t)k);
    const int64_t words = (nv + 31) >> 5;
    for (int64_t seg = 0; seg < words; seg += kSegWords) {
      const int nw = (int)min((int64_t)kSegWords, words - seg);
      for (int j = tid; j < nw; j += 256) segw[j] = ld_acquire_u32(bm + seg + j);
      __syncthreads();
      for (uint32_t c = tid; c < nch; c += 256) {
        const int64_t wi = (int64_t)(chosen[c] >> 5) - seg;
        if (wi >= 0 && wi < nw && chosen[c] < (uint32_t)nv)
          atomicOr(&segw[wi], 1u << (chosen[c] & 31));
      }
      __syncthreads();
      const int per = (nw + 255) / 256;
      const int lo = min(tid * per, nw), hi = min(lo + per, nw);
      uint32_t cnt = 0;
      for (int j = lo; j < hi; ++j) cnt += __popc(segw[j]);
      uint32_t tot;
      uint32_t o = s_out + block_exclusive_scan256(cnt, tmp, &tot);
      for (int j = lo; j < hi; ++j) {
        uint32_t bits = segw[j];
        while (bits) {
          const int bpos = __ffs(bits) - 1;
          bits &= bits - 1;
          const int64_t slot = ((seg + j) << 5) + bpos;
          if (o < (uint32_t)k && slot < nv) orow[o] = sp ? sp[slot] : (int32_t)slot;
          ++o;
        }
      }
      __syncthreads();
      if (tid == 0) s_out += tot;
      __syncthreads();
    }
    if (count_out && tid == 0) count_out[r] = k;
  }
  // leave the row's control words zero for the next call
  uint32_t* wh = hist + (int64_t)r * hist_stride;
  for (int j = tid; j < kHistBins; j += 256) wh[j] = 0u;
  if (tid == 0) {
    ctl->cand = 0u;
    ctl->done = 0u;
  }
}

size_t topk_lds_bytes(int32_t k) { return (size_t)(2048 + kSegWords + k) * sizeof(uint32_t); }

hipError_t launch_topk_hist(const float* scores, int32_t rows, int64_t n, const int32_t* n_valid,
                            int32_t nv_add, int64_t n_max, uint32_t* hist, int64_t hist_stride,
                            hipStream_t st) {
  const int32_t chunk = kTopkChunk;
  const int64_t nchunks = (n_max + chunk - 1) / chunk;
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_hist_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(256), 0, st,
                     scores, n, n_valid, nv_add, hist, hist_stride, chunk);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int32_t rows, int64_t n,
                              const int32_t* n_valid, int32_t nv_add, int64_t n_max,
                              const int32_t* slot_pos, int32_t k, int32_t* idx_out,
                              int32_t* count_out, const TopkWs& w, hipStream_t st) {
  const int32_t chunk = kTopkChunk;
  int64_t nchunks = (n_max + chunk - 1) / chunk;
  if (nchunks < 1) nchunks = 1;
  const size_t lds = topk_lds_bytes(k);
  static bool lds_raised = false;
  if (!lds_raised) {
    const hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)topk_lds_bytes(16384));
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(256), lds,
                     st, scores, n, n_valid, nv_add, slot_pos, k, idx_out, count_out, w.hist,
                     w.hist_stride, w.ctl, w.ctl_stride, w.cand, w.cand_cap, w.bitmap, w.bm_words,
                     chunk);
  return hipGetLastError();
}

}  // namespace csa2
