// misc.hip -- small helper kernels: workspace fill and pool score gather.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride) p[i] = 0u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  CSA2_KERNEL(true, true, fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)p,
                     words);
  return hipGetLastError();
}

// Scores of the pool members (slots s < count[r]) gathered into a dense row,
// with the 12-bit key histogram the Top-K select pass starts from.
__global__ __launch_bounds__(256) void gather_scores_kernel(
    const float* __restrict__ scores, int64_t n, const int32_t* __restrict__ pool, int32_t P,
    const int32_t* __restrict__ count, float* __restrict__ out, uint32_t* __restrict__ hist,
    int64_t hist_stride, int32_t hist_copies) {
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y;
  const int32_t c = min(count[r], P);
  const int32_t start = blockIdx.x * 4096;
  if (start >= c) return;
  const int32_t end = min(c, start + 4096);
  for (int k = threadIdx.x; k < kHistBins; k += 256) lhist[k] = 0u;
  __syncthreads();
  const float* srow = scores + (int64_t)r * n;
  const int32_t* prow = pool + (int64_t)r * P;
  float* orow = out + (int64_t)r * P;
  // 16 slots per thread, indices then scores all requested before use
  int32_t sl[16];
  float v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) sl[u] = prow[min(start + u * 256 + (int32_t)threadIdx.x, end - 1)];
#pragma unroll
  for (int u = 0; u < 16; ++u) v[u] = srow[sl[u]];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int32_t s = start + u * 256 + threadIdx.x;
    if (s < end) {
      orow[s] = v[u];
      atomicAdd(&lhist[score_key(v[u]) >> kHistShift], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)r * hist_stride + (blockIdx.x % hist_copies) * kHistBins;
  for (int k = threadIdx.x; k < kHistBins; k += 256)
    if (lhist[k]) atomicAdd(gh + k, lhist[k]);
}

hipError_t launch_gather_scores(const float* scores, int64_t n, const int32_t* pool, int32_t P,
                                const int32_t* count, int32_t rows, float* out, uint32_t* hist,
                                int64_t hist_stride, int32_t hist_copies, hipStream_t st) {
  const dim3 grid((unsigned)((P + 4095) / 4096), (unsigned)rows), block(256);
  CSA2_KERNEL(true, true, gather_scores_kernel, grid, block, 0, st, scores, n, pool, P, count, out, hist,
              hist_stride, hist_copies);
  return hipGetLastError();
}

}  // namespace csa2
