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
// row are cut into splits of 64 (global entries or window entries, never
// both); one block of 4 waves takes a split, one tile of 16 entries per wave.
// Lane (i, g) owns entry i and channels 64m + 16g + [0,16): it gathers them,
// dequantizes exactly to fp16 in registers, and the wave computes the tile's
// logits.  The block finds each head's maximum and sum over its 64 entries
// (DPP reductions within a wave, LDS across waves), stores the value
// channels in LDS, and wave w accumulates P.V for value channels
// [w*dv/4, (w+1)*dv/4).  Window entries enter as raw E4M3 values and their
// scale multiplies the split's logits and partial output.
//
// Each split writes its partial (o, max, sum) per head, and a second kernel
// merges them:
//   out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s,  lse = M + log L.
// (Merging in the same launch, with the splits exchanging partials through
// device-coherent memory, measured slower on MI355X than the kernel boundary:
// partials written by one XCD and read by another make a slow round trip.)
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

// Partial values travel in pairs (64-bit accesses).
__device__ __forceinline__ void st_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ float2 ld_pair(const float* p) {
  return *reinterpret_cast<const float2*>(p);
}

// Layout of a split's partial output for one head: wave w, lane column i and
// output tile nt of P.V hold value channel w*dv/4 + 16*nt + i, stored at
// w*dv/4 + 32*(nt/2) + 2*i + nt%2, so a lane writes tiles nt, nt+1 as one
// pair and the 16 lanes of a row write 128 contiguous bytes.  Slot p of a
// head row therefore holds channel:
template <int DV>
__device__ __forceinline__ int partial_channel(int p) {
  constexpr int CPW = DV / 4;
  const int w = p / CPW, rem = p % CPW;
  return w * CPW + (2 * (rem / 32) + (rem & 1)) * 16 + (rem % 32) / 2;
}

// B operand of P.V straight from the row-major V tile: ds_read_b64_tr_b16
// hands lane t of each 16-lane group element t % 4 of the 64-bit word
// addressed by lane 4j + t / 4, as its element j.  With lane s addressing
// V[e0 + s / 4][c0 + 4 (s % 4)], lane t receives V[e0 + j][c0 + t], j < 4.
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
__device__ __forceinline__ f16x8 v_operand(const _Float16* lo, const _Float16* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(hi));
  return __builtin_bit_cast(f16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row stride (floats) of the round's logits: 64 entries + 4, so the 16 head
// rows of a 16-byte read fall on different banks.
constexpr int kLgStride = 68;
constexpr float kLog2e = 1.44269504088896341f;  // log2 e
constexpr float kLn2 = 0.693147180559945309f;   // ln 2

template <int DV>
constexpr int vs_stride() {
  // halves; a row stride of 8 banks mod 64 keeps the four rows of a
  // transposed read on distinct banks
  return DV + 16;
}

// The NW scale words of an FP4 row (one word per 64-channel group, byte j
// for channels 16j..16j+15 of the group), read with as few loads as the
// row's 4-byte alignment allows: every lane of the row takes the whole row
// (the same cache lines) and later shifts out its own byte, instead of one
// byte load per group.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
template <int NW>
__device__ __forceinline__ void load_scale_words(const uint8_t* sr, uint32_t (&out)[NW]) {
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(sr);
#pragma unroll
  for (int q = 0; q + 4 <= NW; q += 4) {
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(s32 + q);
    out[q] = v.x;
    out[q + 1] = v.y;
    out[q + 2] = v.z;
    out[q + 3] = v.w;
  }
  constexpr int R = NW & ~3;
  if constexpr (NW - R >= 2) {
    const u32x2_a4 v = *reinterpret_cast<const u32x2_a4*>(s32 + R);
    out[R] = v.x;
    out[R + 1] = v.y;
  }
  if constexpr ((NW - R) & 1) out[NW - 1] = s32[NW - 1];
}

struct AttnArgs {
  const uint16_t* q;
  int32_t T;
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t cap;
  const int32_t* idx;
  int32_t K;
  const uint8_t* swa;
  const float* swa_scale;
  const int32_t* swa_pos0;
  int32_t S, W;
  const int32_t* q_pos;
  float sm_scale;
  float* part;
  int32_t nsg, nsplit, rounds, row0;
  // FP8 main cache: codes holds D E4M3 bytes per row and row_scale one fp32
  // scale per row (null for the FP4 cache)
  const float* row_scale;
};

// One split of one query row.  WIN: the split holds window entries (raw
// E4M3 rows); MULTI: the split runs several rounds of 64 entries; KV8: the
// main cache holds E4M3 rows with one fp32 scale each (the per-entry scale
// multiplies the logit, and P.V uses p * s_j / s_max with s_max, the split's
// largest scale, applied to the partial output).  Each instantiation is
// straight-line code from the index load to the row loads, so the row loads
// issue as soon as the index arrives.  COH: the partial is stored with
// device-coherent stores, for blocks of the same launch to read.
template <int D, int DV, bool WIN, bool MULTI, bool KV8, bool COH = false>
__device__ __forceinline__ void split_body(const AttnArgs& a, int r, int sidx, _Float16* Vs,
                                           float* Lg, float* Sg) {
  static_assert(!(KV8 && MULTI), "FP8 main-cache splits take one round");
  constexpr int NM = D / 64;        // 64-channel groups of a row
  constexpr int NMV = DV / 64;      // groups holding value channels
  // FP4 main rows are read 16 bytes per lane: in each 128-channel group p
  // (NP of them) lane (i, g) holds channels 128p + 32g + [0, 32), which
  // feed the k-slots of MFMA pair (2p, 2p + 1); a last 64-channel group is
  // read 8 bytes per lane (channels 64m + 16g + [0, 16)), as are all groups
  // of the window and FP8 rows.  chan(m, hf) is the first of the 8 channels
  // lane (i, g) holds for operand half hf of group slot m; the query
  // fragments use the same channels.
  constexpr int NP = (!WIN && !KV8) ? D / 128 : 0;
  constexpr int VST = vs_stride<DV>();
  constexpr int CPW = DV / 4;       // value channels per wave
  constexpr int NT = CPW / 16;      // P.V output tiles per wave
  constexpr int PSTRIDE = 16 * DV + 32;
  const int b = (a.row0 + r) / a.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const uint32_t ghi = 0u - (uint32_t)(g >> 1);  // all ones for g = 2, 3
  auto chan = [&](int m, int hf) -> int {
    return (m < 2 * NP) ? 128 * (m >> 1) + 32 * g + 16 * (m & 1) + 8 * hf : 64 * m + 16 * g + 8 * hf;
  };
  const int rounds = MULTI ? a.rounds : 1;
  // entry of this lane in round rnd: e0 + 64 * rnd
  const int e0 = (WIN ? sidx - a.nsg : sidx) * 64 * rounds + wave * 16 + i;
  int nw = 0, wlo = 0, pos0 = 0;
  float wscale = 1.0f;
  if constexpr (WIN) {
    const int p = a.q_pos[r];
    pos0 = a.swa_pos0[b];
    wscale = a.swa_scale[b];
    wlo = max(p - a.W + 1, pos0);
    nw = max(0, min(p, pos0 + a.S - 1) - wlo + 1);
  }

  // ---- loads, in dependency order: the index, then the query, then the row
  // (a row with K == 0 still has one global split, and idx may be null)
  auto load_ix = [&](int e) -> int {
    return (WIN || a.K == 0) ? 0 : a.idx[(int64_t)r * a.K + min(e, a.K - 1)];
  };
  int ix = load_ix(e0);
  // the query row (16 heads x D bf16), loaded once by the whole block: the 16
  // threads 16h .. 16h + 15 (16 consecutive lanes of one wave) take head h,
  // thread 16h + c its 16-byte words c, c + 16, ... (the last clamped)
  constexpr int WPH = D / 8;                 // 16-byte words per head
  constexpr int QPT = (WPH + 15) / 16;       // words per thread
  const int qh = tid >> 4, qc = tid & 15;    // head and word column of this thread
  uint4 qraw[QPT];
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(a.q + ((int64_t)r * 16 + qh) * D);
#pragma unroll
    for (int k = 0; k < QPT; ++k) qraw[k] = qsrc[min(qc + 16 * k, WPH - 1)];
  }
  uint32_t w0[NM], w1[NM], w2[NM], w3[NM], sc[NM];
  bool valid;
  float sj = 0.0f;  // KV8: this lane's entry scale (0 for no entry)
  auto load_row = [&](int e) {
    if constexpr (!WIN && KV8) {
      valid = e < a.K && ix >= 0 && ix < a.cap;
      const int64_t row = (int64_t)b * a.cap + (valid ? ix : 0);
      const uint8_t* wr = a.codes + row * D;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 v = *reinterpret_cast<const uint4*>(wr + 64 * m + 16 * g);
        w0[m] = v.x;
        w1[m] = v.y;
        w2[m] = v.z;
        w3[m] = v.w;
      }
      const float sv = a.row_scale[row];
      sj = valid ? sv : 0.0f;
    } else if constexpr (!WIN) {
      valid = e < a.K && ix >= 0 && ix < a.cap;
      const int64_t row = (int64_t)b * a.cap + (valid ? ix : 0);
      const uint8_t* cr = a.codes + row * (D / 2);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const uint4 cw = *reinterpret_cast<const uint4*>(cr + 64 * q + 16 * g);
        w0[2 * q] = cw.x;
        w1[2 * q] = cw.y;
        w0[2 * q + 1] = cw.z;
        w1[2 * q + 1] = cw.w;
      }
#pragma unroll
      for (int m = 2 * NP; m < NM; ++m) {
        const uint2 cw = *reinterpret_cast<const uint2*>(cr + 32 * m + 8 * g);
        w0[m] = cw.x;
        w1[m] = cw.y;
      }
      load_scale_words<NM>(a.scales + row * (D / 16), sc);
    } else {
      valid = e < nw;
      const int64_t row = (int64_t)b * a.S + (valid ? (wlo - pos0 + e) : 0);
      const uint8_t* wr = a.swa + row * D;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 v = *reinterpret_cast<const uint4*>(wr + 64 * m + 16 * g);
        w0[m] = v.x;
        w1[m] = v.y;
        w2[m] = v.z;
        w3[m] = v.w;
      }
    }
  };
  // FP4 global splits of several rounds request the next round's rows into
  // a second set of registers once the current round's logits are done, so
  // they arrive during its softmax and P.V.
  constexpr bool PREF = MULTI && !WIN && !KV8;
  uint32_t p0[PREF ? NM : 1], p1[PREF ? NM : 1], psc[PREF ? NM : 1];
  bool pvalid = false;
  auto prefetch_row = [&](int e) {
    if constexpr (PREF) {
      pvalid = e < a.K && ix >= 0 && ix < a.cap;
      const int64_t row = (int64_t)b * a.cap + (pvalid ? ix : 0);
      const uint8_t* cr = a.codes + row * (D / 2);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const uint4 cw = *reinterpret_cast<const uint4*>(cr + 64 * q + 16 * g);
        p0[2 * q] = cw.x;
        p1[2 * q] = cw.y;
        p0[2 * q + 1] = cw.z;
        p1[2 * q + 1] = cw.w;
      }
#pragma unroll
      for (int m = 2 * NP; m < NM; ++m) {
        const uint2 cw = *reinterpret_cast<const uint2*>(cr + 32 * m + 8 * g);
        p0[m] = cw.x;
        p1[m] = cw.y;
      }
      load_scale_words<NM>(a.scales + row * (D / 16), psc);
    }
  };
  load_row(e0);
  // keep the row loads ahead of the query conversion (the scheduler would
  // otherwise sink them below it, after the query has arrived)
  __builtin_amdgcn_sched_barrier(0);

  // ---- query fragments (head i), scaled per head into fp16 range.  Each
  // head's largest magnitude comes from its 16 threads by a DPP row maximum;
  // they write the row as fp16 times the head's power of two into an LDS
  // copy (in the V tile's space, which is written only after every wave
  // holds its fragments); lane (i, g) then reads head i's channels
  // 64m + 16g + [0, 16).  Two barriers.
  f16x8 qa[NM][2];
  int er[4];
  {
    constexpr int QST = D + 8;      // fp16 row stride: the 16 heads' reads spread over banks
    __shared__ int s_qexp[16];
    _Float16* q16 = Vs;             // [16][QST], aliases the V tile
    static_assert(16 * QST <= 64 * vs_stride<DV>(), "query copy fits the V tile");
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      if (qc + 16 * k < WPH) {
        const uint32_t wd[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          am = fmaxf(am, fmaxf(fabsf(bf16_to_f32(wd[t] & 0xFFFFu)), fabsf(bf16_to_f32(wd[t] >> 16))));
      }
    }
    const int e = fp16_exponent_for(row16_max(am));
    if (qc == 0) s_qexp[qh] = e;
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int j = qc + 16 * k;
      if (j < WPH) {
        const uint32_t wd[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
        f16x8 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[2 * t] = (_Float16)ldexpf(bf16_to_f32(wd[t] & 0xFFFFu), e);
          v[2 * t + 1] = (_Float16)ldexpf(bf16_to_f32(wd[t] >> 16), e);
        }
        *reinterpret_cast<f16x8*>(q16 + qh * QST + 8 * j) = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qa[m][hf] = *reinterpret_cast<const f16x8*>(q16 + i * QST + chan(m, hf));
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) er[rr] = s_qexp[4 * g + rr];
    __syncthreads();  // every wave holds its fragments: the V tile may be written
  }
  // Logits are kept in base-2 units (natural logit x log2 e): the softmax
  // weights are then plain powers of two, 2^(l - m), one v_exp each, and the
  // partial's maximum is stored in the same units.  The query's power of two
  // folds into the per-head scale.
  const float lscale = a.sm_scale * wscale;
  float esc[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) esc[rr] = ldexpf(lscale * kLog2e, -er[rr]);

  // running softmax state of head i (every lane of the block holds its
  // head's), and this wave's P.V tiles
  float mrun = -INFINITY, lrun = 0.0f;
  float smax = 1.0f;  // KV8: the split's largest entry scale (one round)
  f32x4 o[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // this lane's transposed-read address in the V tile (see v_operand)
  const _Float16* vt = Vs + (8 * g + (i >> 2)) * VST + wave * CPW + 4 * (i & 3);

  for (int rnd = 0; rnd < rounds; ++rnd) {
    if (MULTI && rnd > 0) {
      __syncthreads();  // the previous round's reads of Vs and Lg are done
      if constexpr (PREF) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          w0[m] = p0[m];
          w1[m] = p1[m];
          sc[m] = psc[m];
        }
        valid = pvalid;
      } else {
        load_row(e0 + 64 * rnd);
      }
    }
    if (MULTI && rnd + 1 < rounds) ix = load_ix(e0 + 64 * (rnd + 1));  // next round's index
    // ---- dequantize this wave's tile, logits (rows = heads 4g + rr, column = entry i)
    f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
    {
      _Float16* vrow = Vs + (wave * 16 + i) * VST;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        f16x8 k0, k1;
        if constexpr (!WIN && KV8) {
          // E4M3 -> fp16 is exact; two bytes per conversion
          const uint32_t wv[4] = {w0[m], w1[m], w2[m], w3[m]};
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[q4], 1.0f, false);
            const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wv[q4], 1.0f, true);
            f16x8& k = (q4 < 2) ? k0 : k1;
            k[4 * (q4 & 1)] = lo[0];
            k[4 * (q4 & 1) + 1] = lo[1];
            k[4 * (q4 & 1) + 2] = hi[0];
            k[4 * (q4 & 1) + 3] = hi[1];
          }
        } else if constexpr (!WIN) {
          // the scale byte of this lane's 16 channels: byte 2 (g & 1) + (m & 1)
          // of word 2p + g / 2 in a 128-channel group, byte g of word m after
          // (a bitwise select: a conditional pick of the two words becomes
          // an indexed register read, which the compiler puts in scratch)
          uint32_t sb;
          if (m < 2 * NP) {
            const uint32_t lo = sc[m & ~1], hi = sc[(m & ~1) + 1];
            sb = (lo ^ ((lo ^ hi) & ghi)) >> (16 * (g & 1) + 8 * (m & 1));
          } else {
            sb = sc[m] >> (8 * g);
          }
          const f16x2 s2 = scale_pair(sb);
          k0 = fp4x8_to_f16(w0[m], s2);
          k1 = fp4x8_to_f16(w1[m], s2);
        } else {
          uint4 v;
          v.x = w0[m];
          v.y = w1[m];
          v.z = w2[m];
          v.w = w3[m];
          e4m3x16_to_f16(v, k0, k1);
        }
        acc0 = mfma16x16x32(qa[m][0], k0, acc0);
        acc1 = mfma16x16x32(qa[m][1], k1, acc1);
        if (m < NMV) {
          *reinterpret_cast<f16x8*>(vrow + chan(m, 0)) = k0;
          *reinterpret_cast<f16x8*>(vrow + chan(m, 1)) = k1;
        }
      }
    }
    if constexpr (PREF) {
      if (rnd + 1 < rounds) prefetch_row(e0 + 64 * (rnd + 1));
    }
    // ---- softmax: the tile's logits (heads 4g + rr, entry i) go to LDS; after
    // one barrier, lane (i, g) reads head i's logits at its P.V operand slots
    // (entries 32ks + 8g + [0, 8)), and the four lanes of head i agree on its
    // maximum and sum with lane exchanges.  Every wave thus builds P itself.
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float lg = (acc0[rr] + acc1[rr]) * esc[rr];
      if constexpr (!WIN && KV8) lg *= sj;
      Lg[(4 * g + rr) * kLgStride + wave * 16 + i] = valid ? lg : -INFINITY;
    }
    if constexpr (!WIN && KV8) {
      if (g == 0) Sg[wave * 16 + i] = sj;
      const float wm = row16_max(sj);
      if (lane == 0) Sg[64 + wave] = wm;
    }
    __syncthreads();  // every wave's logits and value rows are in LDS
    float lv[2][8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float4 x0 = *reinterpret_cast<const float4*>(Lg + i * kLgStride + 32 * ks + 8 * g);
      const float4 x1 = *reinterpret_cast<const float4*>(Lg + i * kLgStride + 32 * ks + 8 * g + 4);
      lv[ks][0] = x0.x; lv[ks][1] = x0.y; lv[ks][2] = x0.z; lv[ks][3] = x0.w;
      lv[ks][4] = x1.x; lv[ks][5] = x1.y; lv[ks][6] = x1.z; lv[ks][7] = x1.w;
    }
    float mr = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) mr = fmaxf(mr, lv[ks][j]);
    mr = fmaxf(mr, shfl_xor(mr, 16));
    mr = fmaxf(mr, shfl_xor(mr, 32));
    const float mnew = fmaxf(mrun, mr);
    const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mrun - mnew);
    // with no finite logit yet every lv is -inf, and 2^(-inf - 0) = 0
    const float msafe = (mnew == -INFINITY) ? 0.0f : mnew;
    f16x8 pa[2];
    float ps = 0.0f;  // the sum uses the unrounded probabilities
    float ew[2][8];   // KV8: s_j / s_max of the lane's entries
    if constexpr (!WIN && KV8) {
      smax = fmaxf(fmaxf(Sg[64], Sg[65]), fmaxf(Sg[66], Sg[67]));
      const float inv = (smax > 0.0f) ? 1.0f / smax : 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) ew[ks][j] = Sg[32 * ks + 8 * g + j] * inv;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pr = __builtin_amdgcn_exp2f(lv[ks][j] - msafe);
        ps += pr;
        if constexpr (!WIN && KV8)
          pa[ks][j] = (_Float16)(pr * ew[ks][j]);
        else
          pa[ks][j] = (_Float16)pr;
      }
    ps += shfl_xor(ps, 16);
    ps += shfl_xor(ps, 32);
    lrun = lrun * alpha + ps;
    mrun = mnew;
    // the P.V tiles hold heads 4g + rr: their rescale factors
    float alh[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) alh[rr] = __shfl(alpha, 4 * g + rr, kWave);
    // ---- P.V for this wave's channels
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) o[nt][rr] *= alh[rr];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const _Float16* vp = vt + 32 * ks * VST + 16 * nt;
        o[nt] = mfma16x16x32(pa[ks], v_operand(vp, vp + 4 * VST), o[nt]);
      }
    }
  }

  // ---- partial result of this split: o[16][DV], m[16], l[16]
  const float oscale = (!WIN && KV8) ? smax : wscale;
  float* pb = a.part + ((int64_t)r * a.nsplit + sidx) * PSTRIDE;
  static_assert(NT % 2 == 0, "tiles stored in pairs");
#pragma unroll
  for (int nt = 0; nt < NT; nt += 2)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float* dst = pb + (4 * g + rr) * DV + wave * CPW + 16 * nt + 2 * i;
      if constexpr (COH)
        st_coh(reinterpret_cast<uint64_t*>(dst),
               __builtin_bit_cast(uint64_t, make_float2(o[nt][rr] * oscale, o[nt + 1][rr] * oscale)));
      else
        st_pair(dst, o[nt][rr] * oscale, o[nt + 1][rr] * oscale);
    }
  // running max and sum of head i, written by lanes g == 0 of wave 0
  if (wave == 0 && g == 0) {
    if constexpr (COH) {
      st_coh(pb + 16 * DV + i, mrun);
      st_coh(pb + 16 * DV + 16 + i, lrun);
    } else {
      pb[16 * DV + i] = mrun;
      pb[16 * DV + 16 + i] = lrun;
    }
  }
}

// Block (s, r): split s of query row r (global entries for s < nsg, window
// entries after).
template <int D, int DV, bool MULTI, bool KV8>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(AttnArgs a) {
  // 16-byte aligned: the V tile is written and read with 16- and 8-byte LDS
  // accesses, so its base must not follow the static arrays unaligned
  extern __shared__ __attribute__((aligned(16))) _Float16 Vs[];  // [64 entries][vs_stride]
  __shared__ __attribute__((aligned(16))) float Lg[16 * kLgStride];  // [head][entry of the round]
  __shared__ float Sg[64 + 4];  // KV8: entry scales of the round, then each wave's largest
  const int r = blockIdx.y, sidx = blockIdx.x;
  if (sidx >= a.nsg)
    split_body<D, DV, true, MULTI, false>(a, r, sidx, Vs, Lg, Sg);
  else
    split_body<D, DV, false, MULTI, KV8>(a, r, sidx, Vs, Lg, Sg);
}

// Merge kernel.  Unit u of row r is the value-slot pair (2(u % (dv/2)), +1)
// of head u / (dv/2); SUB consecutive threads merge one unit, thread `sub`
// taking splits sub, sub + SUB, ...  Each thread loads, per split, its pair
// of the partial output, all requested before any is used, and the split's
// max and sum for the unit's head (staged once per block in LDS when the
// row has at most SUB * KB splits, else loaded by every thread); the SUB
// threads agree on the running maximum and add their shares with lane
// moves.  With the maxima m_s in base-2 units:
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  lse = M ln 2 + log L.
// One pass of 256 threads merges units [vb * 256 / SUB, (vb + 1) * 256 / SUB)
// of row r.  COH: the partials were written by blocks of the same launch.
template <int DV, int SUB, int KB, bool COH>  // KB: splits per thread per pass
__device__ __forceinline__ void merge_units(const float* __restrict__ part, int32_t nsplit, int r,
                                            int vb, float* __restrict__ out,
                                            float* __restrict__ lse) {
  static_assert(SUB == 4, "lane moves below cover groups of four lanes");
  constexpr int PSTRIDE = 16 * DV + 32;
  constexpr int UPH = DV / 2;          // units per head
  constexpr int UPB = 256 / SUB;       // units per pass
  static_assert(UPH % UPB == 0, "a pass lies inside one head");
  static_assert(2 * SUB * KB <= 256, "one staged value per thread");
  // Rows of at most SUB * KB splits (one group of splits per thread): the
  // maxima and sums of the pass's head (every unit of a pass belongs to one
  // head) are loaded once per block into LDS instead of by every thread.
  __shared__ float s_ml[2][SUB * KB];
  const bool staged = nsplit <= SUB * KB;  // the same for the whole block
  const int tid = threadIdx.x, sub = tid % SUB;
  const int u = vb * UPB + tid / SUB;  // the passes cover the units exactly
  const int h = u / UPH, pp = 2 * (u % UPH);
  const float* prow = part + (int64_t)r * nsplit * PSTRIDE;
  float Mrun = -INFINITY, L = 0.0f, nx = 0.0f, ny = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += SUB * KB) {
    float2 ov[KB];
    float mv[KB], lv[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int sc = min(s0 + sub + SUB * k, nsplit - 1);  // clamped: every load in bounds
      const float* ps = prow + (int64_t)sc * PSTRIDE;
      if constexpr (COH)
        ov[k] = __builtin_bit_cast(float2, ld_coh(reinterpret_cast<const uint64_t*>(ps + h * DV + pp)));
      else
        ov[k] = ld_pair(ps + h * DV + pp);
    }
    if (staged) {
      __syncthreads();  // an earlier pass's reads of s_ml are done
      if (tid < 2 * nsplit) {
        const float* pm = prow + (int64_t)(tid >> 1) * PSTRIDE + 16 * DV + 16 * (tid & 1) + h;
        s_ml[tid & 1][tid >> 1] = COH ? ld_coh(pm) : *pm;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int sc = min(sub + SUB * k, nsplit - 1);
        mv[k] = s_ml[0][sc];
        lv[k] = s_ml[1][sc];
      }
    } else {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int sc = min(s0 + sub + SUB * k, nsplit - 1);
        const float* ps = prow + (int64_t)sc * PSTRIDE;
        if constexpr (COH) {
          mv[k] = ld_coh(ps + 16 * DV + h);
          lv[k] = ld_coh(ps + 16 * DV + 16 + h);
        } else {
          mv[k] = ps[16 * DV + h];
          lv[k] = ps[16 * DV + 16 + h];
        }
      }
    }
    float cm = -INFINITY;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      if (s0 + sub + SUB * k >= nsplit) mv[k] = -INFINITY;
      cm = fmaxf(cm, mv[k]);
    }
    cm = fmaxf(cm, dpp_move<kDppXor1>(cm));
    cm = fmaxf(cm, dpp_move<kDppXor2>(cm));
    const float Mnew = fmaxf(Mrun, cm);
    const float a = (Mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(Mrun - Mnew);
    L *= a;
    nx *= a;
    ny *= a;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float wv = (mv[k] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mv[k] - Mnew);
      L += wv * lv[k];
      nx += wv * ov[k].x;
      ny += wv * ov[k].y;
    }
    Mrun = Mnew;
  }
  L += dpp_move<kDppXor1>(L);
  L += dpp_move<kDppXor2>(L);
  nx += dpp_move<kDppXor1>(nx);
  nx += dpp_move<kDppXor2>(nx);
  ny += dpp_move<kDppXor1>(ny);
  ny += dpp_move<kDppXor2>(ny);
  if (sub == 0) {
    const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
    const int ch = partial_channel<DV>(pp);  // slot pp + 1 holds channel ch + 16
    float* orow = out + (int64_t)r * 16 * DV + h * DV;
    orow[ch] = nx * inv;
    orow[ch + 16] = ny * inv;
    if (lse && pp == 0) lse[(int64_t)r * 16 + h] = (L > 0.0f) ? Mrun * kLn2 + logf(L) : -INFINITY;
  }
}

// Merge of whole rows, one block per row, for passes of many rows with few
// splits each (a prefill pass): thread t takes unit t + 256 k of the row
// (k < 16 DV / 512), with the splits' maxima and sums staged in LDS
// ([split][32]: the 16 maxima, then the 16 sums), and keeps KH units x SC
// splits of loads in flight.  Consecutive threads read consecutive pairs, so
// each load instruction covers 512 contiguous bytes of a partial; the merge
// kernel's groups of four threads per unit would load every split of a
// short list several times over.  Per unit the arithmetic is the merge
// kernel's, summed over the splits in order.
template <int DV>
__global__ __launch_bounds__(256) void attn_merge_rows_kernel(const float* __restrict__ part,
                                                              int32_t nsplit,
                                                              float* __restrict__ out,
                                                              float* __restrict__ lse) {
  extern __shared__ float s_ml[];  // nsplit x 32
  constexpr int PSTRIDE = 16 * DV + 32;
  constexpr int UPH = DV / 2;              // units per head
  constexpr int UPT = 16 * UPH / 256;      // units per thread
  constexpr int KH = UPT < 8 ? UPT : 8;    // units in flight
  constexpr int SC = 8;                    // splits in flight
  static_assert(UPT % KH == 0, "unit groups");
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* prow = part + (int64_t)r * nsplit * PSTRIDE;
  for (int x = tid; x < nsplit * 32; x += 256)
    s_ml[x] = prow[(int64_t)(x >> 5) * PSTRIDE + 16 * DV + (x & 31)];
  __syncthreads();
  for (int k0 = 0; k0 < UPT; k0 += KH) {
    float Mrun[KH], L[KH], nx[KH], ny[KH];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      Mrun[kh] = -INFINITY;
      L[kh] = nx[kh] = ny[kh] = 0.0f;
    }
    for (int s0 = 0; s0 < nsplit; s0 += SC) {
      float2 ov[SC][KH];
#pragma unroll
      for (int sc = 0; sc < SC; ++sc) {
        if (s0 + sc < nsplit) {  // the same for the whole block
#pragma unroll
          for (int kh = 0; kh < KH; ++kh) {
            const int u = tid + 256 * (k0 + kh);
            ov[sc][kh] = ld_pair(prow + (int64_t)(s0 + sc) * PSTRIDE + (u / UPH) * DV + 2 * (u % UPH));
          }
        }
      }
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        const int h = (tid + 256 * (k0 + kh)) / UPH;
        float cm = -INFINITY;
#pragma unroll
        for (int sc = 0; sc < SC; ++sc)
          if (s0 + sc < nsplit) cm = fmaxf(cm, s_ml[(s0 + sc) * 32 + h]);
        const float Mnew = fmaxf(Mrun[kh], cm);
        const float a = (Mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(Mrun[kh] - Mnew);
        L[kh] *= a;
        nx[kh] *= a;
        ny[kh] *= a;
#pragma unroll
        for (int sc = 0; sc < SC; ++sc) {
          if (s0 + sc < nsplit) {
            const float m = s_ml[(s0 + sc) * 32 + h];
            const float wv = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - Mnew);
            L[kh] += wv * s_ml[(s0 + sc) * 32 + 16 + h];
            nx[kh] += wv * ov[sc][kh].x;
            ny[kh] += wv * ov[sc][kh].y;
          }
        }
        Mrun[kh] = Mnew;
      }
    }
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      const int u = tid + 256 * (k0 + kh);
      const int h = u / UPH, pp = 2 * (u % UPH);
      const float inv = (L[kh] > 0.0f) ? 1.0f / L[kh] : 0.0f;
      const int ch = partial_channel<DV>(pp);  // slot pp + 1 holds channel ch + 16
      float* orow = out + (int64_t)r * 16 * DV + h * DV;
      orow[ch] = nx[kh] * inv;
      orow[ch + 16] = ny[kh] * inv;
      if (lse && pp == 0)
        lse[(int64_t)r * 16 + h] = (L[kh] > 0.0f) ? Mrun[kh] * kLn2 + logf(L[kh]) : -INFINITY;
    }
  }
}

template <int DV, int SUB, int KB>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part,
                                                           int32_t nsplit, float* __restrict__ out,
                                                           float* __restrict__ lse) {
  merge_units<DV, SUB, KB, false>(part, nsplit, blockIdx.y, blockIdx.x, out, lse);
}

// Split and merge in one launch, for grids whose blocks all fit on the
// device at once (the host checks).  Each block computes its split as the
// split kernel does, stores the partial with device-coherent stores, counts
// itself in its row's arrival word and waits (a bounded poll, the only wait
// on another block) until every split of the row has arrived; it then
// merges passes vb = split, split + nsplit, ... of the row's output with the
// merge kernel's arithmetic and split grouping, so the result is the same
// bit for bit.  Words of row r at ctl + r * ctl_stride: arrivals, departures,
// and a flag set if the wait ran out (after wait_limit polls; 0 gives up
// at once); the row's last block to leave zeroes the two counters.
template <int D, int DV, int KB>
__global__ __launch_bounds__(256, 2) void sparse_attn_one_launch_kernel(AttnArgs a, uint32_t* ctl,
                                                                        int64_t ctl_stride,
                                                                        float* out, float* lse,
                                                                        uint32_t wait_limit) {
  extern __shared__ __attribute__((aligned(16))) _Float16 Vs[];
  __shared__ __attribute__((aligned(16))) float Lg[16 * kLgStride];
  __shared__ float Sg[64 + 4];
  __shared__ uint32_t s_ok;
  const int r = blockIdx.y, sidx = blockIdx.x;
  if (sidx >= a.nsg)
    split_body<D, DV, true, false, false, true>(a, r, sidx, Vs, Lg, Sg);
  else
    split_body<D, DV, false, false, false, true>(a, r, sidx, Vs, Lg, Sg);
  // arrival: every thread's partial stores have completed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t* c = ctl + (int64_t)r * ctl_stride;
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t it = 0;
    bool ok = false;
    if (wait_limit > 0) {
      while (!(ok = ld_coh(c) >= (uint32_t)a.nsplit) && ++it < wait_limit)
        __builtin_amdgcn_s_sleep(2);
    }
    if (!ok) st_coh(c + 2, 1u);  // flagged in the control words; the output is not written
    s_ok = ok ? 1u : 0u;
  }
  __syncthreads();
  if (s_ok) {
    constexpr int NVB = 16 * DV / 2 / 64;  // passes of 64 units per row
    for (int vb = sidx; vb < NVB; vb += a.nsplit)
      merge_units<DV, 4, KB, true>(a.part, a.nsplit, r, vb, out, lse);
  }
  // departure: the row's last block leaves the counters zero
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(c + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)a.nsplit - 1u) {
      st_coh(c, 0u);
      st_coh(c + 1, 0u);
    }
  }
}

// Passes merged one block per row (at least this many rows, at most this
// many splits per row).
constexpr int32_t kMergeRowsMin = 128;
constexpr int32_t kMergeRowsMaxSplits = 64;

size_t attn_lds_bytes(int32_t dv) {
  return (size_t)64 * (dv == 512 ? vs_stride<512>() : vs_stride<128>()) * sizeof(_Float16);
}

// Launches the one-launch kernel if its grid fits the device at once
// (blocks per compute unit from the occupancy query, per device); sets
// *launched accordingly.
template <int D, int DV, int KB>
static hipError_t try_one_launch(const AttnArgs& args, int32_t rows, size_t lds, uint32_t* ctl,
                                 float* out, float* lse, hipStream_t st, bool* launched) {
  *launched = false;
  // raised once per process (thread-safe static initialisation)
  static const hipError_t raised =
      hipFuncSetAttribute((const void*)sparse_attn_one_launch_kernel<D, DV, KB>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (raised != hipSuccess) return raised;
  // unknown capacity (0): the split + merge kernels run instead
  const int64_t cap =
      device_resident_blocks((const void*)sparse_attn_one_launch_kernel<D, DV, KB>, 256, lds);
  if ((int64_t)args.nsplit * rows > cap) return hipSuccess;
  const dim3 grid((unsigned)args.nsplit, (unsigned)rows);
  CSA2_KERNEL(true, true, (sparse_attn_one_launch_kernel<D, DV, KB>), grid, dim3(256), lds, st,
              args, ctl, (int64_t)kCtlWordsPerRow, out, lse, wait_limit());
  *launched = true;
  return hipGetLastError();
}

template <int D, int DV>
static hipError_t launch_attn(const uint16_t* q, int32_t rows, int32_t T, const uint8_t* codes,
                              const uint8_t* scales, int64_t cap, const int32_t* idx, int32_t K,
                              const uint8_t* swa, const float* swa_scale,
                              const int32_t* swa_pos0, int32_t S, int32_t W,
                              const int32_t* q_pos, float sm_scale, float* out, float* lse,
                              const AttnWs& w, hipStream_t st, int32_t row0,
                              const float* row_scale, uint32_t* one_launch_ctl) {
  const size_t lds = attn_lds_bytes(DV);
  // raised once per process (thread-safe static initialisation)
  static const hipError_t raised = [lds]() {
    for (const void* k : {(const void*)sparse_attn_kernel<D, DV, false, false>,
                          (const void*)sparse_attn_kernel<D, DV, true, false>,
                          (const void*)sparse_attn_kernel<D, DV, false, true>}) {
      hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (raised != hipSuccess) return raised;
  // An empty window array contributes no entries (its pointers may be null).
  if (S == 0) W = 0;
  // Splits of several rounds (each prefetching the next round's rows) keep
  // the partials few when the grid would be large (attn_rounds).  For a
  // 256-row prefill pass 8 rounds took 115.8 us (split + merge) against
  // 120.4 (4 rounds), 127.9 (16) and 166 (2); a 4096-token chunk in passes
  // of 2048 rows took 2.66 ms with 8 rounds against 2.77 (4) and 2.72 (16).
  const bool kv8 = row_scale != nullptr;
  const int32_t rounds = attn_rounds(rows, K, W, kv8);
  const AttnSplit sp = attn_split(K, W, rounds);
  const AttnArgs args{q, T, codes, scales, cap, idx, K, swa, swa_scale, swa_pos0, S, W, q_pos,
                      sm_scale, w.part, sp.nsg, sp.nsplit, rounds, row0, row_scale};
  if (one_launch_ctl && !kv8 && rounds == 1) {
    bool launched = false;
    hipError_t e;
    if (sp.nsplit <= 16)
      e = try_one_launch<D, DV, 4>(args, rows, lds, one_launch_ctl, out, lse, st, &launched);
    else if (sp.nsplit <= 40)
      e = try_one_launch<D, DV, 10>(args, rows, lds, one_launch_ctl, out, lse, st, &launched);
    else
      e = try_one_launch<D, DV, 16>(args, rows, lds, one_launch_ctl, out, lse, st, &launched);
    if (e != hipSuccess || launched) return e;
  }
  const dim3 grid((unsigned)sp.nsplit, (unsigned)rows);
  if (kv8)
    CSA2_KERNEL(true, false, (sparse_attn_kernel<D, DV, false, true>), grid, dim3(256), lds, st,
                args);
  else if (rounds > 1)
    CSA2_KERNEL(true, false, (sparse_attn_kernel<D, DV, true, false>), grid, dim3(256), lds, st,
                args);
  else
    CSA2_KERNEL(true, false, (sparse_attn_kernel<D, DV, false, false>), grid, dim3(256), lds, st,
                args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // many rows of few splits: one block per row
  if (rows >= kMergeRowsMin && sp.nsplit <= kMergeRowsMaxSplits) {
    CSA2_KERNEL(false, true, attn_merge_rows_kernel<DV>, dim3((unsigned)rows), dim3(256),
                (size_t)sp.nsplit * 32 * sizeof(float), st, w.part, sp.nsplit, out, lse);
    return hipGetLastError();
  }
  // four threads per output unit; each pass takes 4 KB splits
  constexpr int NU = 16 * DV / 2;
  const dim3 cgrid(NU / 64, (unsigned)rows);
  if (sp.nsplit <= 16)
    CSA2_KERNEL(false, true, (attn_combine_kernel<DV, 4, 4>), cgrid, dim3(256), 0, st, w.part,
                sp.nsplit, out, lse);
  else if (sp.nsplit <= 40)
    CSA2_KERNEL(false, true, (attn_combine_kernel<DV, 4, 10>), cgrid, dim3(256), 0, st, w.part,
                sp.nsplit, out, lse);
  else
    CSA2_KERNEL(false, true, (attn_combine_kernel<DV, 4, 16>), cgrid, dim3(256), 0, st, w.part,
                sp.nsplit, out, lse);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, int32_t rows, int32_t T, int32_t D, int32_t dv,
                              const uint8_t* codes, const uint8_t* scales, int64_t cap,
                              const int32_t* idx, int32_t K, const uint8_t* swa,
                              const float* swa_scale, const int32_t* swa_pos0, int32_t S,
                              int32_t W, const int32_t* q_pos, float sm_scale, float* out,
                              float* lse, const AttnWs& w, hipStream_t st, int32_t row0,
                              const float* row_scale, uint32_t* one_launch_ctl) {
  if (D == 576 && dv == 512)
    return launch_attn<576, 512>(q, rows, T, codes, scales, cap, idx, K, swa, swa_scale, swa_pos0,
                                 S, W, q_pos, sm_scale, out, lse, w, st, row0, row_scale,
                                 one_launch_ctl);
  if (D == 128 && dv == 128)
    return launch_attn<128, 128>(q, rows, T, codes, scales, cap, idx, K, swa, swa_scale, swa_pos0,
                                 S, W, q_pos, sm_scale, out, lse, w, st, row0, row_scale,
                                 one_launch_ctl);
  return hipErrorInvalidValue;
}

}  // namespace csa2
