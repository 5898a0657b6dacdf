// quantize.hip -- quantize-on-write of KV rows into the FP4 cache.
//
// helmcode.com/deepseek-v41-flash, section "04 · FP4": the global KV is
// stored as E2M1 elements with one E4M3 scale per 16 channels and no extra
// global scale; quantisation is applied after RoPE.  Per block the scale is
// the E4M3 value nearest to amax/6 and each element takes the nearest E2M1
// grid value of x/scale.  Both roundings are decided by comparing against
// thresholds that are exact in fp32, so no division (and no double
// rounding) is involved.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"
#include "csa2_quant.hpp"

namespace csa2 {

// One thread per 16-channel block.
template <typename In>
__global__ __launch_bounds__(256) void quantize_kernel(const In* __restrict__ x, int64_t rows,
                                                       int32_t dim, int64_t stride,
                                                       const int64_t* __restrict__ dst_rows,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int32_t nb = dim >> 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * nb) return;
  const int64_t r = t / nb;
  const int32_t blk = (int32_t)(t - r * nb);
  const int64_t dr = dst_rows ? dst_rows[r] : r;
  quantize_block<In>(x + r * stride + (int64_t)blk * 16, codes + dr * (dim >> 1) + (int64_t)blk * 8,
                     scales + dr * nb + blk);
}

// FP8 main-cache rows (the E4M3 variant of the global KV, with one fp32
// scale per row): one wave per row.  scale = amax / 448 (1 for an all-zero
// row), byte = E4M3(clamp(x / scale, -448, 448)) rounded to nearest even by
// the hardware conversion; the divisions are IEEE fp32.
template <typename In>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const In* __restrict__ x, int64_t rows,
                                                           int32_t dim, int64_t stride,
                                                           const int64_t* __restrict__ dst_rows,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform per wave
  const In* src = x + r * stride;
  float amax = 0.0f;
  for (int c = lane; c < dim; c += 64) amax = fmaxf(amax, fabsf(load_elem<In>(src + c)));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  const float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
  const int64_t dr = dst_rows ? dst_rows[r] : r;
  uint8_t* dst = codes + dr * dim;
  // four channels per lane and step: lane l takes channels 4*(l + 64*k) ..
  for (int c = 4 * lane; c < dim; c += 256) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float y = load_elem<In>(src + c + j) / sc;
      v[j] = fminf(fmaxf(y, -448.0f), 448.0f);
    }
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
    *reinterpret_cast<uint32_t*>(dst + c) = (uint32_t)word;
  }
  if (lane == 0) scales[dr] = sc;
}

hipError_t launch_quantize_fp8(const void* x, bool bf16, int64_t rows, int32_t dim, int64_t stride,
                               const int64_t* dst_rows, uint8_t* codes, float* scales,
                               hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (bf16)
    CSA2_KERNEL(true, true, quantize_fp8_kernel<uint16_t>, grid, block, 0, st, (const uint16_t*)x,
                rows, dim, stride, dst_rows, codes, scales);
  else
    CSA2_KERNEL(true, true, quantize_fp8_kernel<float>, grid, block, 0, st, (const float*)x, rows,
                dim, stride, dst_rows, codes, scales);
  return hipGetLastError();
}

// Rotary embedding fused with the quantize-on-write (the quantisation is
// applied after RoPE).  The last rope_dim channels of a row form pairs
// (2i, 2i+1) of that region, rotated by the row's angle for pair i:
//   y0 = x0 c - x1 s,  y1 = x0 s + x1 c
// with c, s given per row and pair (cos_sin[row][i] = {c, s}); each product
// and each sum is rounded to fp32 separately (no fused multiply-add), so the
// rotated values, and hence the codes, are reproducible.  One thread per
// 16-channel block.
template <typename In>
__global__ __launch_bounds__(256) void rope_quantize_kernel(
    const In* __restrict__ x, int64_t rows, int32_t dim, int64_t stride, int32_t rope_dim,
    const float2* __restrict__ cos_sin, const int64_t* __restrict__ dst_rows,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int32_t nb = dim >> 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * nb) return;
  const int64_t r = t / nb;
  const int32_t blk = (int32_t)(t - r * nb);
  const int64_t dr = dst_rows ? dst_rows[r] : r;
  float v[16];
  const In* src = x + r * stride + (int64_t)blk * 16;
#pragma unroll
  for (int c = 0; c < 16; ++c) v[c] = load_elem<In>(src + c);
  const int32_t c0 = blk * 16 - (dim - rope_dim);  // channel offset inside the rope region
  if (c0 >= 0) {
    const float2* cs = cos_sin + r * (rope_dim >> 1) + (c0 >> 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 a = cs[j];
      const float x0 = v[2 * j], x1 = v[2 * j + 1];
      v[2 * j] = __fsub_rn(__fmul_rn(x0, a.x), __fmul_rn(x1, a.y));
      v[2 * j + 1] = __fadd_rn(__fmul_rn(x0, a.y), __fmul_rn(x1, a.x));
    }
  }
  quantize_values(v, codes + dr * (dim >> 1) + (int64_t)blk * 8, scales + dr * nb + blk);
}

hipError_t launch_rope_quantize(const void* x, bool bf16, int64_t rows, int32_t dim,
                                int64_t stride, int32_t rope_dim, const float* cos_sin,
                                const int64_t* dst_rows, uint8_t* codes, uint8_t* scales,
                                hipStream_t st) {
  const int64_t n = rows * (dim / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  const float2* cs = reinterpret_cast<const float2*>(cos_sin);
  if (bf16)
    CSA2_KERNEL(true, true, rope_quantize_kernel<uint16_t>, grid, block, 0, st,
                (const uint16_t*)x, rows, dim, stride, rope_dim, cs, dst_rows, codes, scales);
  else
    CSA2_KERNEL(true, true, rope_quantize_kernel<float>, grid, block, 0, st, (const float*)x,
                rows, dim, stride, rope_dim, cs, dst_rows, codes, scales);
  return hipGetLastError();
}

// The write of a decode or prefill step: query row r of x1 and x2 lands on
// cache row (r / T) * cap + q_pos[r] of each cache (one launch for both).
template <typename In>
__global__ __launch_bounds__(256) void quantize_step_kernel(
    const In* __restrict__ x1, const In* __restrict__ x2, int32_t rows, int32_t T,
    const int32_t* __restrict__ q_pos, int32_t dim1, int64_t cap1, uint8_t* __restrict__ codes1,
    uint8_t* __restrict__ scales1, int32_t dim2, int64_t cap2, uint8_t* __restrict__ codes2,
    uint8_t* __restrict__ scales2) {
  const int64_t n1 = (int64_t)rows * (dim1 >> 4);
  const int64_t n2 = (int64_t)rows * (dim2 >> 4);
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const In* x = x1;
  int32_t dim = dim1;
  int64_t cap = cap1;
  uint8_t* codes = codes1;
  uint8_t* scales = scales1;
  if (t >= n1) {
    t -= n1;
    if (t >= n2) return;
    x = x2;
    dim = dim2;
    cap = cap2;
    codes = codes2;
    scales = scales2;
  }
  const int32_t nb = dim >> 4;
  const int64_t r = t / nb;
  const int32_t blk = (int32_t)(t - r * nb);
  const int64_t dr = (r / T) * cap + q_pos[r];
  quantize_block<In>(x + r * dim + (int64_t)blk * 16, codes + dr * (dim >> 1) + (int64_t)blk * 8,
                     scales + dr * nb + blk);
}

hipError_t launch_quantize_step(const void* x1, const void* x2, bool bf16, int32_t rows,
                                int32_t T, const int32_t* q_pos, int32_t dim1, int64_t cap1,
                                uint8_t* codes1, uint8_t* scales1, int32_t dim2, int64_t cap2,
                                uint8_t* codes2, uint8_t* scales2, hipStream_t st) {
  const int64_t n = (int64_t)rows * (dim1 / 16 + dim2 / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (bf16)
    CSA2_KERNEL(true, true, quantize_step_kernel<uint16_t>, grid, block, 0, st, (const uint16_t*)x1,
                       (const uint16_t*)x2, rows, T, q_pos, dim1, cap1, codes1, scales1, dim2,
                       cap2, codes2, scales2);
  else
    CSA2_KERNEL(true, true, quantize_step_kernel<float>, grid, block, 0, st, (const float*)x1,
                       (const float*)x2, rows, T, q_pos, dim1, cap1, codes1, scales1, dim2, cap2,
                       codes2, scales2);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int32_t dim, int64_t stride,
                           const int64_t* dst_rows, uint8_t* codes, uint8_t* scales,
                           hipStream_t st) {
  const int64_t n = rows * (dim / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (bf16)
    CSA2_KERNEL(true, true, quantize_kernel<uint16_t>, grid, block, 0, st,
                       (const uint16_t*)x, rows, dim, stride, dst_rows, codes, scales);
  else
    CSA2_KERNEL(true, true, quantize_kernel<float>, grid, block, 0, st, (const float*)x, rows, dim,
                       stride, dst_rows, codes, scales);
  return hipGetLastError();
}

}  // namespace csa2
