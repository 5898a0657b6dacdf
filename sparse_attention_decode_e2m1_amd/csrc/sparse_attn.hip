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
// contractions with M = 16 heads: fp16 MFMA 16x16x32.  The entries of a query
// row are cut into splits of `tps` tiles of 16 entries; one block of 4 waves
// handles a split.  Each round every wave gathers one tile (lane (i, g) owns
// entry i and channels 64m + 16g + [0,16)), dequantizes it exactly to fp16 in
// registers, computes the tile's logits and stores the value channels in LDS;
// the block then updates a running (max, sum) per head and accumulates P.V
// (wave w owns value channels [w*dv/4, (w+1)*dv/4)).  The next round's
// gathers are issued before the current round is computed.  Splits hold
// either global tiles or window tiles, never both, so window values enter as
// raw E4M3 and their scale multiplies the split's partial output once.
//
// A second kernel merges the splits: one block per (query row, head) reads
// every split's (max, sum, partial output) for that head -- all splits in
// parallel -- and writes the normalised output and log-sum-exp.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

template <int NM>
struct TileRaw {
  uint32_t w0[NM], w1[NM];  // FP4 codes: channels 64m+16g+[0,8) and [8,16)
  uint32_t w2[NM], w3[NM];  // window rows only: E4M3 bytes 8..15 of the 16
  uint32_t sc[NM];          // FP4 scale byte (global rows)
};

template <int D, int DV>
__global__ __launch_bounds__(256) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, int32_t T, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int64_t cap, const int32_t* __restrict__ idx, int32_t K,
    const uint8_t* __restrict__ swa, const float* __restrict__ swa_scale,
    const int32_t* __restrict__ swa_pos0, int32_t S, int32_t W, const int32_t* __restrict__ q_pos,
    float sm_scale, float* __restrict__ part, int32_t nsg, int32_t tps, int32_t nsplit,
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

  // ---- gather of one tile into raw registers (no use of the data yet)
  auto load_tile = [&](int tile, TileRaw<NM>& raw) -> bool {
    const int e = tile * 16 + i;
    const bool tvalid = tile < tile_end;
    bool valid;
    if (!is_win) {
      const int ix = (tvalid && e < K) ? idx[(int64_t)r * K + e] : -1;
      valid = ix >= 0 && ix < cap;
      const int64_t row = (int64_t)b * cap + (valid ? ix : 0);
      const uint8_t* cr = codes + row * (D / 2);
      const uint8_t* sr = scales + row * (D / 16);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint2 cw = *reinterpret_cast<const uint2*>(cr + 32 * m + 8 * g);
        raw.w0[m] = cw.x;
        raw.w1[m] = cw.y;
        raw.sc[m] = sr[4 * m + g];
      }
    } else {
      valid = tvalid && e < nw;
      const int64_t row = (int64_t)b * S + (valid ? (wlo - pos0 + e) : 0);
      const uint8_t* wr = swa + row * D;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 v = *reinterpret_cast<const uint4*>(wr + 64 * m + 16 * g);
        raw.w0[m] = v.x;
        raw.w1[m] = v.y;
        raw.w2[m] = v.z;
        raw.w3[m] = v.w;
      }
    }
    return valid;
  };

  TileRaw<NM> cur, nxt;
  bool cur_valid = false, nxt_valid = false;
  if (tile0 < tile_end) cur_valid = load_tile(tile0 + wave, cur);

  // ---- query fragments (head i), scaled per head into fp16 range
  f16x8 qa[NM][2];
  int qexp;
  {
    const uint16_t* qr = q + ((int64_t)r * 16 + i) * D;
    float amax = 0.0f;
    uint32_t rq[NM][8];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 a = *reinterpret_cast<const uint4*>(qr + 64 * m + 16 * g);
      const uint4 c = *reinterpret_cast<const uint4*>(qr + 64 * m + 16 * g + 8);
      rq[m][0] = a.x; rq[m][1] = a.y; rq[m][2] = a.z; rq[m][3] = a.w;
      rq[m][4] = c.x; rq[m][5] = c.y; rq[m][6] = c.z; rq[m][7] = c.w;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        amax = fmaxf(amax, fabsf(bf16_to_f32(rq[m][j] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(bf16_to_f32(rq[m][j] >> 16)));
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
          const uint32_t wd = rq[m][4 * hf + j];
          qa[m][hf][2 * j] = (_Float16)ldexpf(bf16_to_f32(wd & 0xFFFFu), qexp);
          qa[m][hf][2 * j + 1] = (_Float16)ldexpf(bf16_to_f32(wd >> 16), qexp);
        }
  }
  int er[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) er[rr] = __shfl(qexp, 4 * g + rr, kWave);
  const float wscale = is_win ? swa_scale[b] : 1.0f;
  const float lscale = sm_scale * wscale;

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
    if (t0 + 4 < tile_end) nxt_valid = load_tile(t0 + 4 + wave, nxt);
    // dequantize this wave's tile
    f16x8 k0[NM], k1[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (!is_win) {
        const f16x2 s2 = scale_pair(cur.sc[m]);
        k0[m] = fp4x8_to_f16(cur.w0[m], s2);
        k1[m] = fp4x8_to_f16(cur.w1[m], s2);
      } else {
        uint4 v;
        v.x = cur.w0[m];
        v.y = cur.w1[m];
        v.z = cur.w2[m];
        v.w = cur.w3[m];
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
      lg[rr] = cur_valid ? ldexpf(acc[rr], -er[rr]) * lscale : -INFINITY;
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
    cur = nxt;
    cur_valid = nxt_valid;
  }

  // ---- partial result of this split: o[16][DV], m[16], l[16]
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
}

// Merge of the splits of query row r for head h (blockDim = DV/4 threads,
// four channels each).
template <int DV>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part,
                                                           int32_t nsplit, float* __restrict__ out,
                                                           float* __restrict__ lse) {
  constexpr int PSTRIDE = 16 * DV + 32;
  constexpr int NTH = DV / 4;
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[NTH];
  __shared__ float s_M, s_L;
  const int r = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const float* prow = part + (int64_t)r * nsplit * PSTRIDE;
  // split maxima and sums of this head
  float mloc = -INFINITY;
  for (int s = tid; s < nsplit; s += NTH) {
    const float ms = prow[(int64_t)s * PSTRIDE + 16 * DV + h];
    wgt[s] = ms;
    mloc = fmaxf(mloc, ms);
  }
  red[tid] = mloc;
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY;
    for (int j = 0; j < NTH; ++j) M = fmaxf(M, red[j]);
    s_M = M;
  }
  __syncthreads();
  const float M = s_M;
  float lloc = 0.0f;
  for (int s = tid; s < nsplit; s += NTH) {
    const float ms = wgt[s];
    const float wv = (M == -INFINITY || ms == -INFINITY) ? 0.0f : __expf(ms - M);
    wgt[s] = wv;
    lloc += wv * prow[(int64_t)s * PSTRIDE + 16 * DV + 16 + h];
  }
  red[tid] = lloc;
  __syncthreads();
  if (tid == 0) {
    float L = 0.0f;
    for (int j = 0; j < NTH; ++j) L += red[j];
    s_L = L;
  }
  __syncthreads();
  const float L = s_L;
  // weighted sum of the partial outputs: four splits' loads in flight at once
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* col = prow + h * DV + 4 * tid;
  int s = 0;
  for (; s + 4 <= nsplit; s += 4) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(col + (int64_t)(s + u) * PSTRIDE);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wv = wgt[s + u];
      acc.x += wv * v[u].x;
      acc.y += wv * v[u].y;
      acc.z += wv * v[u].z;
      acc.w += wv * v[u].w;
    }
  }
  for (; s < nsplit; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(col + (int64_t)s * PSTRIDE);
    const float wv = wgt[s];
    acc.x += wv * v.x;
    acc.y += wv * v.y;
    acc.z += wv * v.z;
    acc.w += wv * v.w;
  }
  const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
  acc.x *= inv;
  acc.y *= inv;
  acc.z *= inv;
  acc.w *= inv;
  *reinterpret_cast<float4*>(out + ((int64_t)r * 16 + h) * DV + 4 * tid) = acc;
  if (lse && tid == 0) lse[(int64_t)r * 16 + h] = (L > 0.0f) ? M + logf(L) : -INFINITY;
}

size_t attn_lds_bytes(int32_t dv) { return (size_t)64 * (dv + 8) * sizeof(_Float16); }

template <int D, int DV>
static hipError_t launch_attn_pair(const uint16_t* q, int32_t rows, int32_t T,
                                   const uint8_t* codes, const uint8_t* scales, int64_t cap,
                                   const int32_t* idx, int32_t K, const uint8_t* swa,
                                   const float* swa_scale, const int32_t* swa_pos0, int32_t S,
                                   int32_t W, const int32_t* q_pos, float sm_scale, float* out,
                                   float* lse, const AttnWs& w, hipStream_t st, int32_t row0) {
  static bool lds_raised = false;
  if (!lds_raised) {
    const hipError_t e = hipFuncSetAttribute((const void*)sparse_attn_kernel<D, DV>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)attn_lds_bytes(DV));
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  const AttnSplit sp = attn_split(K, W);
  hipLaunchKernelGGL((sparse_attn_kernel<D, DV>), dim3((unsigned)sp.nsplit, (unsigned)rows),
                     dim3(256), attn_lds_bytes(DV), st, q, T, codes, scales, cap, idx, K, swa,
                     swa_scale, swa_pos0, S, W, q_pos, sm_scale, w.part, sp.nsg, sp.tps, sp.nsplit,
                     row0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine_kernel<DV>), dim3((unsigned)rows, 16u), dim3(DV / 4), 0, st,
                     w.part, sp.nsplit, out, lse);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, int32_t rows, int32_t T, int32_t D, int32_t dv,
                              const uint8_t* codes, const uint8_t* scales, int64_t cap,
                              const int32_t* idx, int32_t K, const uint8_t* swa,
                              const float* swa_scale, const int32_t* swa_pos0, int32_t S,
                              int32_t W, const int32_t* q_pos, float sm_scale, float* out,
                              float* lse, const AttnWs& w, hipStream_t st, int32_t row0) {
  if (D == 576 && dv == 512)
    return launch_attn_pair<576, 512>(q, rows, T, codes, scales, cap, idx, K, swa, swa_scale,
                                      swa_pos0, S, W, q_pos, sm_scale, out, lse, w, st, row0);
  if (D == 128 && dv == 128)
    return launch_attn_pair<128, 128>(q, rows, T, codes, scales, cap, idx, K, swa, swa_scale,
                                      swa_pos0, S, W, q_pos, sm_scale, out, lse, w, st, row0);
  return hipErrorInvalidValue;
}

}  // namespace csa2
