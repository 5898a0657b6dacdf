// csa2_device.hpp -- device helpers for the CSA2 kernels (gfx950 only).
//
// FP4 rows follow the cache layout declared in include/csa2.h: E2M1 codes
// (even channel in the low nibble) and one E4M3 scale byte per 16 channels
// (helmcode.com/deepseek-v41-flash, section "04 · FP4").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kHistBins = 4096;       // top 12 bits of the ordered score key
constexpr int kHistShift = 20;
// Most copies of each row's histogram; block b adds into copy b % copies.
// Device-scope atomics on one address serialise (about 11 ns each on
// MI355X), so the merge of many blocks is spread over the copies.
constexpr int kHistCopies = 8;

// Device-coherent accesses for data one block writes and another block of
// the same launch reads (agent scope: no full-cache write-back or invalidate).
template <typename T>
__device__ __forceinline__ void st_coh(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coh(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------------- FP8 / FP4
// E4M3 byte -> f32 (gfx950 converts the OCP "FN" encoding).  `sel` picks the
// byte of `word`.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}

// Eight E2M1 codes (one 32-bit word, channel 8i+j in nibble j) times a block
// scale, as fp16.  The hardware conversion applies only the exponent of its
// f32 scale operand, so it converts at scale 1 and the E4M3 scale (<= 4
// significant bits) is applied with a packed fp16 multiply; grid value times
// scale has at most 6 significant bits and lies in [2^-10, 2688], so every
// product is exact in fp16.
__device__ __forceinline__ f16x8 fp4x8_to_f16(uint32_t w, f16x2 s2) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Four E4M3 bytes -> four exact fp16 values (E4M3 has 4 significant bits and
// range [2^-9, 448], inside fp16's normal range).
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, _Float16* o) {
  o[0] = (_Float16)e4m3_to_f32<0>(w);
  o[1] = (_Float16)e4m3_to_f32<1>(w);
  o[2] = (_Float16)e4m3_to_f32<2>(w);
  o[3] = (_Float16)e4m3_to_f32<3>(w);
}

// Sixteen E4M3 bytes -> two fp16x8 vectors (channels 0..7 and 8..15).
__device__ __forceinline__ void e4m3x16_to_f16(uint4 v, f16x8& lo, f16x8& hi) {
  _Float16 t[16];
  e4m3x4_to_f16(v.x, t + 0);
  e4m3x4_to_f16(v.y, t + 4);
  e4m3x4_to_f16(v.z, t + 8);
  e4m3x4_to_f16(v.w, t + 12);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo[j] = t[j];
    hi[j] = t[8 + j];
  }
}

__device__ __forceinline__ f16x2 scale_pair(uint32_t byte) {
  _Float16 s = (_Float16)e4m3_to_f32<0>(byte);
  return f16x2{s, s};
}

// bf16 bit pattern -> f32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// Power-of-two exponent that brings a head's largest |value| into
// [2^14, 2^15): the query is then exact in fp16 for every element within
// 2^-31 of that maximum, and the scaling is undone exactly in fp32.
__device__ __forceinline__ int fp16_exponent_for(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  (void)frexpf(amax, &e);  // amax in [2^(e-1), 2^e)
  return 15 - e;
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// max(x, 0) in one integer instruction: a negative float (sign bit set)
// compares below 0 as a signed integer, and +0 is the integer 0.  (fmaxf
// would first quiet its operands, one more instruction each.)
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ------------------------------------------------------------ score keys
// Order-preserving unsigned key of an fp32 score: larger score -> larger
// key; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = __float_as_uint(x);
  if ((b << 1) == 0u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// 64-bit rank value: score key, then the lower slot wins a tie.
__device__ __forceinline__ uint64_t rank_value(uint32_t key, uint32_t slot) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - slot);
}
__device__ __forceinline__ uint32_t rank_slot(uint64_t v) {
  return 0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull);
}

// ----------------------------------------------------------- reductions
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

// DPP move inside each row of 16 lanes (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

// Maximum over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_move<kDppXor1>(v));
  v = fmaxf(v, dpp_move<kDppXor2>(v));
  v = fmaxf(v, dpp_move<kDppRor4>(v));
  v = fmaxf(v, dpp_move<kDppRor8>(v));
  return v;
}
// Sum over the 16 lanes of each row (every lane holds the sum; lanes of
// different quads may differ in the order of the additions).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_move<kDppXor1>(v);
  v += dpp_move<kDppXor2>(v);
  v += dpp_move<kDppRor4>(v);
  v += dpp_move<kDppRor8>(v);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive prefix sum over a 256-thread block; `tmp` holds 4 words of LDS.
__device__ __forceinline__ uint32_t block_exclusive_scan256(uint32_t v, uint32_t* tmp,
                                                            uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t t = tmp[w];
    off += (w < wave) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

}  // namespace csa2
