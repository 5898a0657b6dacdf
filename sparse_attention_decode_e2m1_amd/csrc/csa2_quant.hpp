// csa2_quant.hpp -- the FP4 quantizer of one 16-channel block, shared by
// the quantize-on-write kernels and the decode scan (which writes a Full
// layer's new rows itself).
//
// helmcode.com/deepseek-v41-flash, section "04 · FP4": E2M1 elements with one
// E4M3 scale per 16 channels and no extra global scale.  The scale is the
// E4M3 value nearest to amax/6 and each element the nearest E2M1 grid value
// of x/scale; both roundings are decided by comparing against thresholds
// that are exact in fp32, so no division (and no double rounding) is involved.
#pragma once

#include "csa2_device.hpp"

namespace csa2 {

// Positive finite E4M3 value of byte b (0..126); exact in fp32.
__device__ __forceinline__ float e4m3_pos(int b) {
  const int e = b >> 3, m = b & 7;
  return (e == 0) ? (float)m * 0x1p-9f : ldexpf(1.0f + 0.125f * (float)m, e - 7);
}

// Scale byte = E4M3 value nearest to amax/6, ties to the even mantissa,
// saturating at 448.  Threshold b lies halfway between bytes b and b+1,
// times 6: 3*(v_b + v_{b+1}) has at most 8 significant bits, so it is exact;
// amax passes it when above it, or on it when byte b+1 has an even mantissa.
__device__ __forceinline__ bool scale_passes(float amax, int b) {
  const float t = 3.0f * (e4m3_pos(b) + e4m3_pos(b + 1));
  return amax > t || (amax == t && ((b + 1) & 1) == 0);
}
// The hardware conversion rounds the fp32 quotient amax/6 to its nearest
// E4M3 byte.  Every halfway point between E4M3 values is an fp32 number and
// rounding to fp32 is monotone, so the quotient never crosses one; it can
// only land on one, where the conversion's tie may pick the neighbour of the
// exact answer.  One comparison with the exact threshold on each side of
// the converted byte therefore gives the byte of the exact amax/6.
__device__ __forceinline__ int scale_byte(float amax) {
  const float qt = fminf(amax / 6.0f, 448.0f);
  int b = min(__builtin_amdgcn_cvt_pk_fp8_f32(qt, 0.0f, 0, false) & 0x7F, 126);
  if (b < 126 && scale_passes(amax, b))
    ++b;
  else if (b > 0 && !scale_passes(amax, b - 1))
    --b;
  return b;
}

// E2M1 magnitude code of |x| under scale s: nearest of {0,.5,1,1.5,2,3,4,6}*s
// with ties to the even code.  Midpoints t*s (t = .25,.75,1.25,1.75,2.5,3.5,5)
// are exact in fp32; ">=" at a midpoint rounds up onto an even code.
__device__ __forceinline__ uint32_t e2m1_mag(float a, float s) {
  if (s == 0.0f) return 0u;
  uint32_t c = 0;
  c += a > 0.25f * s;
  c += a >= 0.75f * s;
  c += a > 1.25f * s;
  c += a >= 1.75f * s;
  c += a > 2.5f * s;
  c += a >= 3.5f * s;
  c += a > 5.0f * s;
  return c;
}

template <typename In>
__device__ __forceinline__ float load_elem(const In* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(*p);
}

// Quantize one 16-channel block held in registers: 8 code bytes and one
// scale byte.
__device__ __forceinline__ void quantize_values(const float (&v)[16], uint8_t* code_dst,
                                                uint8_t* scale_dst) {
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(v[c]));
  const int sb = scale_byte(amax);
  const float s = e4m3_pos(sb);
  uint64_t packed = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint32_t sign = (__float_as_uint(v[c]) >> 31) << 3;
    const uint32_t code = sign | e2m1_mag(fabsf(v[c]), s);
    packed |= (uint64_t)code << (4 * c);
  }
  *reinterpret_cast<uint64_t*>(code_dst) = packed;
  *scale_dst = (uint8_t)sb;
}

// E2M1 magnitude code to its grid value (0, .5, 1, 1.5, 2, 3, 4, 6):
// mantissa bit over exponent bits (bias 1).
__device__ __forceinline__ float e2m1_grid(uint32_t mg) {
  return mg < 2u ? 0.5f * (float)mg : (1.0f + 0.5f * (float)(mg & 1u)) * (float)(1u << ((mg >> 1) - 1u));
}

// Element-parallel quantisation by one wave: each row of 16 lanes holds one
// 16-channel block (lane e holds channel e of it).  Every lane gets its
// exact dequantized value; lanes e = 0 and e = 8 get the 32-bit words of
// codes for channels 0..7 and 8..15 of their block, and every lane the
// block's scale byte.  Same codes and scale as quantize_values.
__device__ __forceinline__ void quantize_lane(float x, float* deq, uint32_t* word, uint32_t* sb) {
  const int e = threadIdx.x & 15;
  const float a = fabsf(x);
  const int b = scale_byte(row16_max(a));
  const float s = e4m3_pos(b);
  const uint32_t mg = e2m1_mag(a, s);
  const uint32_t code = ((__float_as_uint(x) >> 31) << 3) | mg;
  const float m = e2m1_grid(mg) * s;
  *deq = (code & 8u) ? -m : m;
  uint32_t v = code << (4 * (e & 7));
  v |= __shfl_xor(v, 1, 64);
  v |= __shfl_xor(v, 2, 64);
  v |= __shfl_xor(v, 4, 64);
  *word = v;
  *sb = (uint32_t)b;
}

// Quantize one 16-channel block read from memory.
template <typename In>
__device__ __forceinline__ void quantize_block(const In* __restrict__ src, uint8_t* code_dst,
                                               uint8_t* scale_dst) {
  float v[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) v[c] = load_elem<In>(src + c);
  quantize_values(v, code_dst, scale_dst);
}

}  // namespace csa2
