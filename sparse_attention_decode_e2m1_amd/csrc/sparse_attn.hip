// sparse_attn.hip -- attention over the Top-K FP4 rows plus the FP8 window.
//
// louisbouchard.ai/deepseek-v41-flash-kv-cache-writing-benchmark, "Share the
// cache and the search work": each query attends to the selected global
// entries alongside a local 128-token window; helmcode.com/
// deepseek-v41-flash, section "04 · FP4": the window KV stays in FP8.  One
// softmax runs over the union; values are the first dv channels of the same
// rows that give the keys.
//
// All 16 query heads share each KV row, so q.K and P.V are dense
// contractions with M = 16 heads: fp16 MFMA 16x16x32.  A block of 4 waves
// handles `tps` tiles of 16 entries of one query row (a "split"); each round
// every wave gathers one tile (lane (i, g) owns entry i and channels
// 64m + 16g + [0,16)), dequantizes it exactly to fp16 in registers, computes
// the tile's logits and stores the value channels in LDS.  The block then
// updates a running (max, sum) per head and accumulates P.V: wave w owns
// value channels [w*dv/4, (w+1)*dv/4).  Splits hold either global tiles or
// window tiles, never both, so window values enter as raw E4M3 and their
// scale multiplies the split's partial output once.  The last split of a row
// to finish (device-scope counter after a release fence) merges the
// partials.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

template <int D, int DV>
__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, int32_t T, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t cap, const int32_t* __restrict__ idx, int32_t K,
    const uint8_t* __restrict__ swa, const float* __restrict__ swa_scale,
    const int32_t* __restrict__ swa_pos0, int32_t S, int32_t W, const int32_t* __restrict__ q_pos,
    float sm_scale, float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part,
    uint32_t* __restrict__ cnt, int64_t cnt_stride, int32_t nsg, int32_t tps, int32_t nsplit,
    int32_t row0) {
  constexpr int NM = D / 64;        // 64-channel groups of a row
  constexpr int NMV = DV / 64;      // groups holding value channels
  constexpr int VST = DV + 8;       // LDS row stride of V (halves), padded
  constexpr int CPW = DV / 4;       // value channels per wave
  constexpr int NT = CPW / 16;      // P.V output tiles per wave
  constexpr int PSTRIDE = 16 * DV + 32;
  extern __shared__ _Float16 Vs[];  // [64 entries][VST]
  __shared__ _Float16 Ps[16 * 64];  // [head][entry of the round]
  __shared__ float red_max[4][16];
  __shared__ float red_sum[4][16];
  __shared__ int s_last;

  const int r = blockIdx.y, b = (row0 + r) / T, sidx = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;

  const int p = q_pos[r];
  const int pos0 = (W > 0) ? swa_pos0[b] : 0;  // window arrays may be NULL without a window
  const int wlo = max(p - W + 1, pos0);
  const int whi = min(p, pos0 + S - 1);
  const int nw = max(0, whi - wlo + 1);
  const bool is_win = sidx >= nsg;
  const int tile0 = (is_win ? sidx - nsg : sidx) * tps;
  const int ntile_kind = is_win ? (W + 15) / 16 : (K + 15) / 16;
  const int tile_end = min(tile0 + tps, ntile_kind);
  const float wscale = is_win ? swa_scale[b] : 1.0f;
  const float lscale = sm_scale * wscale;

  // ---- query fragments (head i), scaled per head into fp16 range
  f16x8 qa[NM][2];
  int qexp;
  {
    const uint16_t* qr = q + ((int64_t)r * 16 + i) * D;
    float amax = 0.0f;
    uint32_t raw[NM][8];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 a = *reinterpret_cast<const uint4*>(qr + 64 * m + 16 * g);
      const uint4 c = *reinterpret_cast<const uint4*>(qr + 64 * m + 16 * g + 8);
      raw[m][0] = a.x; raw[m][1] = a.y; raw[m][2] = a.z; raw[m][3] = a.w;
      raw[m][4] = c.x; raw[m][5] = c.y; raw[m][6] = c.z; raw[m][7] = c.w;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        amax = fmaxf(amax, fabsf(bf16_to_f32(raw[m][j] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(bf16_to_f32(raw[m][j] >> 16)));
      }
    }
    amax = fmaxf(amax, shfl_xor(amax, 16));
    amax = fmaxf(amax, shfl_xor(amax, 32));
    qexp = fp16_exponent_for(amax);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t wd = raw[m][4 * hf + j];
          qa[m][hf][2 * j] = (_Float16)ldexpf(bf16_to_f32(wd & 0xFFFFu), qexp);
          qa[m][hf][2 * j + 1] = (_Float16)ldexpf(bf16_to_f32(wd >> 16), qexp);
        }
  }
  int er[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) er[rr] = __shfl(qexp, 4 * g + rr, kWave);

  float m_run[4], l_run[4];
  f32x4 o[NT];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    m_run[rr] = -INFINITY;
    l_run[rr] = 0.0f;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int t0 = tile0; t0 < tile_end; t0 += 4) {
    const int tile = t0 + wave;
    const bool tvalid = tile < tile_end;
    const int e = tile * 16 + i;
    bool valid;
    f16x8 k0[NM], k1[NM];
    if (!is_win) {
      const int ix = (tvalid && e < K) ? idx[(int64_t)r * K + e] : -1;
      valid = ix >= 0 && ix < cap;
      const int64_t row = (int64_t)b * cap + (valid ? ix : 0);
      const uint8_t* cr = codes + row * (D / 2);
      const uint8_t* sr = scales + row * (D / 16);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint2 cw = *reinterpret_cast<const uint2*>(cr + 32 * m + 8 * g);
        const uint32_t s4 = *reinterpret_cast<const uint32_t*>(sr + 4 * m);
        const f16x2 s2 = scale_pair((s4 >> (8 * g)) & 0xFFu);
        k0[m] = fp4x8_to_f16(cw.x, s2);
        k1[m] = fp4x8_to_f16(cw.y, s2);
      }
    } else {
      valid = tvalid && e < nw;
      const int64_t row = (int64_t)b * S + (valid ? (wlo - pos0 + e) : 0);
      const uint8_t* wr = swa + row * D;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 v = *reinterpret_cast<const uint4*>(wr + 64 * m + 16 * g);
        e4m3x16_to_f16(v, k0[m], k1[m]);
      }
    }
    // logits of this tile: rows = heads 4g + rr, column = entry i
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      acc = mfma16x16x32(qa[m][0], k0[m], acc);
      acc = mfma16x16x32(qa[m][1], k1[m], acc);
    }
    // value channels to LDS: entry (wave*16 + i)
    {
      _Float16* vrow = Vs + (wave * 16 + i) * VST;
#pragma unroll
      for (int m = 0; m < NMV; ++m) {
        *reinterpret_cast<f16x8*>(vrow + 64 * m + 16 * g) = k0[m];
        *reinterpret_cast<f16x8*>(vrow + 64 * m + 16 * g + 8) = k1[m];
      }
    }
    float lg[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      lg[rr] = valid ? ldexpf(acc[rr], -er[rr]) * lscale : -INFINITY;
      float mx = lg[rr];
      mx = fmaxf(mx, shfl_xor(mx, 1));
      mx = fmaxf(mx, shfl_xor(mx, 2));
      mx = fmaxf(mx, shfl_xor(mx, 4));
      mx = fmaxf(mx, shfl_xor(mx, 8));
      if (i == 0) red_max[wave][4 * g + rr] = mx;
    }
    __syncthreads();
    float alpha[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = 4 * g + rr;
      const float mr = fmaxf(fmaxf(red_max[0][h], red_max[1][h]), fmaxf(red_max[2][h], red_max[3][h]));
      const float mnew = fmaxf(m_run[rr], mr);
      alpha[rr] = (mnew == -INFINITY) ? 1.0f : __expf(m_run[rr] - mnew);
      const float pr = (mnew == -INFINITY) ? 0.0f : __expf(lg[rr] - mnew);
      Ps[h * 64 + wave * 16 + i] = (_Float16)pr;
      float ps = pr;  // the normaliser sums the unrounded probabilities
      ps += shfl_xor(ps, 1);
      ps += shfl_xor(ps, 2);
      ps += shfl_xor(ps, 4);
      ps += shfl_xor(ps, 8);
      if (i == 0) red_sum[wave][h] = ps;
      m_run[rr] = mnew;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = 4 * g + rr;
      l_run[rr] = l_run[rr] * alpha[rr] + (red_sum[0][h] + red_sum[1][h] + red_sum[2][h] + red_sum[3][h]);
    }
    // P.V for this wave's channels
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) o[nt][rr] *= alpha[rr];
      const int ch = wave * CPW + nt * 16 + i;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f16x8 pa = *reinterpret_cast<const f16x8*>(Ps + i * 64 + 32 * ks + 8 * g);
        f16x8 vb;
#pragma unroll
        for (int j = 0; j < 8; ++j) vb[j] = Vs[(32 * ks + 8 * g + j) * VST + ch];
        o[nt] = mfma16x16x32(pa, vb, o[nt]);
      }
    }
    __syncthreads();
  }

  // ---- partial result of this split
  float* pb = part + ((int64_t)r * nsplit + sidx) * PSTRIDE;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      pb[(4 * g + rr) * DV + wave * CPW + nt * 16 + i] = o[nt][rr] * wscale;
  if (wave == 0 && i == 0) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      pb[16 * DV + 4 * g + rr] = m_run[rr];
      pb[16 * DV + 16 + 4 * g + rr] = l_run[rr];
    }
  }
  __threadfence();
  __syncthreads();
  uint32_t* c = cnt + (int64_t)r * cnt_stride;
  if (tid == 0) s_last = (atomicAdd(c, 1u) == (uint32_t)nsplit - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- merge the splits of row r
  const int h = tid >> 4, sub = tid & 15;
  const float* prow = part + (int64_t)r * nsplit * PSTRIDE;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, prow[s * PSTRIDE + 16 * DV + h]);
  float L = 0.0f;
  float4 acc4[DV / 64];
#pragma unroll
  for (int j = 0; j < DV / 64; ++j) acc4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float* ps = prow + s * PSTRIDE;
      const float ms = ps[16 * DV + h];
      if (ms == -INFINITY) continue;
      const float wgt = __expf(ms - M);
      L += wgt * ps[16 * DV + 16 + h];
#pragma unroll
      for (int j = 0; j < DV / 64; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(ps + h * DV + 64 * j + 4 * sub);
        acc4[j].x += wgt * v.x;
        acc4[j].y += wgt * v.y;
        acc4[j].z += wgt * v.z;
        acc4[j].w += wgt * v.w;
      }
    }
  }
  const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
  float* orow = out + ((int64_t)r * 16 + h) * DV;
#pragma unroll
  for (int j = 0; j < DV / 64; ++j) {
    float4 v = acc4[j];
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
    *reinterpret_cast<float4*>(orow + 64 * j + 4 * sub) = v;
  }
  if (lse && sub == 0) lse[(int64_t)r * 16 + h] = (L > 0.0f) ? M + logf(L) : -INFINITY;
  if (tid == 0) *c = 0u;
}

size_t attn_lds_bytes(int32_t dv) { return (size_t)64 * (dv + 8) * sizeof(_Float16); }

hipError_t launch_sparse_attn(const uint16_t* q, int32_t rows, int32_t T, int32_t D, int32_t dv,
                              const uint8_t* codes, const uint8_t* scales, int64_t cap,
                              const int32_t* idx, int32_t K, const uint8_t* swa,
                              const float* swa_scale, const int32_t* swa_pos0, int32_t S,
                              int32_t W, const int32_t* q_pos, float sm_scale, float* out,
                              float* lse, const AttnWs& w, hipStream_t st, int32_t row0) {
  const AttnSplit sp = attn_split(K, W);
  const dim3 grid((unsigned)sp.nsplit, (unsigned)rows), block(256);
  const size_t lds = attn_lds_bytes(dv);
  static bool lds_raised = false;
  if (!lds_raised) {
    hipError_t e = hipFuncSetAttribute((const void*)sparse_attn_kernel<576, 512>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)attn_lds_bytes(512));
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)sparse_attn_kernel<128, 128>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)attn_lds_bytes(128));
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  if (D == 576 && dv == 512) {
    hipLaunchKernelGGL((sparse_attn_kernel<576, 512>), grid, block, lds, st, q, T, codes, scales,
                       cap, idx, K, swa, swa_scale, swa_pos0, S, W, q_pos, sm_scale, out, lse,
                       w.part, w.cnt, w.cnt_stride, sp.nsg, sp.tps, sp.nsplit, row0);
  } else if (D == 128 && dv == 128) {
    hipLaunchKernelGGL((sparse_attn_kernel<128, 128>), grid, block, lds, st, q, T, codes, scales,
                       cap, idx, K, swa, swa_scale, swa_pos0, S, W, q_pos, sm_scale, out, lse,
                       w.part, w.cnt, w.cnt_stride, sp.nsg, sp.tps, sp.nsplit, row0);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa2
