// One workgroup's rows of the cross-split log-sum-exp merge, as a device
// function of the workgroup index, so that the merge kernel and the launch
// that shares its grid with the chunk-importance kernel run the same code.
//
//   lse = ln sum_s exp(l_s)      out = sum_s exp(l_s - lse) * o_s
//
// o_s is each split's softmax-normalised output and l_s its natural-log
// normaliser (-inf for a split that saw no key of the row). A row is merged by
// WPR waves (1..16, chosen so that every lane covers its splits with one batch
// of loads): the lanes of a row form split groups of D/4 lanes (each lane owns
// 4 columns); a lane issues the loads of its splits before folding them into a
// running max/sum. Groups inside a wave combine by lane exchanges, the waves of
// a row through LDS.
#pragma once

#include "common.h"

namespace ts {

constexpr int kMergeBatch = 8;

__device__ __forceinline__ void lse_combine(float& m, float& ws, float4& acc, float m2, float w2,
                                            const float4& a2) {
  const float M = fmaxf(m, m2);
  const float f1 = M == -INFINITY ? 0.f : __expf(m - M);
  const float f2 = M == -INFINITY ? 0.f : __expf(m2 - M);
  ws = ws * f1 + w2 * f2;
  acc.x = acc.x * f1 + a2.x * f2; acc.y = acc.y * f1 + a2.y * f2;
  acc.z = acc.z * f1 + a2.z * f2; acc.w = acc.w * f1 + a2.w * f2;
  m = M;
}

template <int WPR> struct MergeShape {
  static constexpr int lanes = kWave * WPR;                    // lanes per row
  static constexpr int block = lanes < 256 ? 256 : lanes;      // threads per workgroup
  static constexpr int rows = block / lanes;                   // rows per workgroup
};

// 4 consecutive partial values: fp32, or bf16 widened exactly
__device__ __forceinline__ float4 load_part4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load_part4(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

template <typename Tout, int D, int WPR, typename Tin = float>
__device__ __forceinline__ void merge_block(const Tin* __restrict__ o_part, const float* __restrict__ l_part,
                                            int S, int rows, Tout* __restrict__ out, float* __restrict__ lse,
                                            int bx) {
  using Sh = MergeShape<WPR>;
  constexpr int C4 = D / 4;              // lanes per split group (one float4 each)
  constexpr int NG = Sh::lanes / C4;     // split groups per row
  __shared__ float4 acc_s[Sh::rows][WPR][C4];
  __shared__ float m_s[Sh::rows][WPR], w_s[Sh::rows][WPR];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int rr = tid / Sh::lanes, t = tid % Sh::lanes, wr = t / kWave;
  const int row = bx * Sh::rows + rr;
  const bool live = row < rows;
  const int gi = t / C4, c = t % C4;

  float m = -INFINITY, ws = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) {
    for (int s0 = gi; s0 < S; s0 += NG * kMergeBatch) {
      float lb[kMergeBatch];
      float4 ob[kMergeBatch];
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) {
        const int sp = s0 + b * NG;
        lb[b] = -INFINITY;
        ob[b] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (sp < S) {
          const int64_t pr = (int64_t)sp * rows + row;
          lb[b] = l_part[pr];
          ob[b] = load_part4(o_part + pr * D + 4 * c);
        }
      }
#pragma unroll
      for (int b = 0; b < kMergeBatch; ++b) {
        const float ls = lb[b];
        if (ls == -INFINITY) continue;   // empty split (or past S)
        const float mn = fmaxf(m, ls);
        const float a = __expf(m - mn);  // m = -inf: 0
        const float w = __expf(ls - mn);
        const float4 o = ob[b];
        ws = ws * a + w;
        acc.x = acc.x * a + w * o.x; acc.y = acc.y * a + w * o.y;
        acc.z = acc.z * a + w * o.z; acc.w = acc.w * a + w * o.w;
        m = mn;
      }
    }
  }
  // groups of one wave: lanes c, c + C4, ... hold the same columns
#pragma unroll
  for (int off = C4; off < kWave; off <<= 1) {
    float4 a2;
    const float m2 = __shfl_xor(m, off, kWave), w2 = __shfl_xor(ws, off, kWave);
    a2.x = __shfl_xor(acc.x, off, kWave); a2.y = __shfl_xor(acc.y, off, kWave);
    a2.z = __shfl_xor(acc.z, off, kWave); a2.w = __shfl_xor(acc.w, off, kWave);
    lse_combine(m, ws, acc, m2, w2, a2);
  }
  if constexpr (WPR > 1) {
    // waves of one row meet in LDS; the row's first wave finishes
    if (lane < C4) {
      acc_s[rr][wr][c] = acc;
      if (c == 0) { m_s[rr][wr] = m; w_s[rr][wr] = ws; }
    }
    __syncthreads();
    if (wr != 0) return;
#pragma unroll
    for (int w = 1; w < WPR; ++w) lse_combine(m, ws, acc, m_s[rr][w], w_s[rr][w], acc_s[rr][w][c]);
  }
  if (live && lane < C4) {
    const float inv = ws > 0.f ? 1.f / ws : 0.f;
    Tout* op = out + (int64_t)row * D + 4 * c;
    Elem<Tout>::store(op + 0, acc.x * inv);
    Elem<Tout>::store(op + 1, acc.y * inv);
    Elem<Tout>::store(op + 2, acc.z * inv);
    Elem<Tout>::store(op + 3, acc.w * inv);
    if (lse != nullptr && c == 0) lse[row] = ws > 0.f ? m + logf(ws) : -INFINITY;
  }
}

}  // namespace ts
