// Cross-split log-sum-exp merge of partial attention results.
//
//   lse = ln sum_s exp(l_s)      out = sum_s exp(l_s - lse) * o_s
//
// o_s is each split's softmax-normalised output and l_s its natural-log
// normaliser (-inf for a split that saw no key of the row).
//
// One wave per output row, four rows per 256-thread workgroup. The wave's
// lanes form 64/(D/4) split groups of D/4 lanes (each lane owns 4 columns);
// a lane first issues the loads of a batch of its splits, then folds them
// into a running max/sum, so several 16-byte loads are in flight per lane.
// The groups' partial results are combined with lane exchanges: no LDS and no
// barrier.
#include "common.h"

namespace ts {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;
constexpr int kBatch = 8;

template <typename Tout, int D>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(const float* __restrict__ o_part,
                                                              const float* __restrict__ l_part,
                                                              int S, int rows,
                                                              Tout* __restrict__ out,
                                                              float* __restrict__ lse) {
  constexpr int C4 = D / 4;              // lanes per split group (one float4 each)
  constexpr int NG = kWave / C4;         // split groups per wave
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;               // whole wave leaves; no barrier follows
  const int gi = lane / C4, c = lane % C4;

  float m = -INFINITY, ws = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = gi; s0 < S; s0 += NG * kBatch) {
    float lb[kBatch];
    float4 ob[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int s = s0 + b * NG;
      lb[b] = -INFINITY;
      ob[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < S) {
        const int64_t pr = (int64_t)s * rows + row;
        lb[b] = l_part[pr];
        ob[b] = *reinterpret_cast<const float4*>(o_part + pr * D + 4 * c);
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const float ls = lb[b];
      if (ls == -INFINITY) continue;     // empty split (or past S)
      const float mn = fmaxf(m, ls);
      const float a = __expf(m - mn);    // m = -inf: 0
      const float w = __expf(ls - mn);
      const float4 o = ob[b];
      ws = ws * a + w;
      acc.x = acc.x * a + w * o.x; acc.y = acc.y * a + w * o.y;
      acc.z = acc.z * a + w * o.z; acc.w = acc.w * a + w * o.w;
      m = mn;
    }
  }
  // combine the split groups: lanes c, c + C4, ... hold the same columns
#pragma unroll
  for (int off = C4; off < kWave; off <<= 1) {
    const float m2 = __shfl_xor(m, off, kWave), w2 = __shfl_xor(ws, off, kWave);
    float4 a2;
    a2.x = __shfl_xor(acc.x, off, kWave); a2.y = __shfl_xor(acc.y, off, kWave);
    a2.z = __shfl_xor(acc.z, off, kWave); a2.w = __shfl_xor(acc.w, off, kWave);
    const float M = fmaxf(m, m2);
    const float f1 = M == -INFINITY ? 0.f : __expf(m - M);
    const float f2 = M == -INFINITY ? 0.f : __expf(m2 - M);
    ws = ws * f1 + w2 * f2;
    acc.x = acc.x * f1 + a2.x * f2; acc.y = acc.y * f1 + a2.y * f2;
    acc.z = acc.z * f1 + a2.z * f2; acc.w = acc.w * f1 + a2.w * f2;
    m = M;
  }
  if (gi == 0) {
    const float inv = ws > 0.f ? 1.f / ws : 0.f;
    Tout* op = out + (int64_t)row * D + 4 * c;
    Elem<Tout>::store(op + 0, acc.x * inv);
    Elem<Tout>::store(op + 1, acc.y * inv);
    Elem<Tout>::store(op + 2, acc.z * inv);
    Elem<Tout>::store(op + 3, acc.w * inv);
    if (lse != nullptr && c == 0) lse[row] = ws > 0.f ? m + logf(ws) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_merge(const float* o_part, const float* l_part, int n_parts, int rows,
                             int D, void* out, float* lse, ts_dtype dtype, hipStream_t s) {
  const int grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (dtype == TS_BF16) {
    if (D == 128)
      attn_merge_kernel<bf16_t, 128><<<grid, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<bf16_t*>(out), lse);
    else
      attn_merge_kernel<bf16_t, 64><<<grid, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<bf16_t*>(out), lse);
  } else {
    if (D == 128)
      attn_merge_kernel<float, 128><<<grid, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<float*>(out), lse);
    else
      attn_merge_kernel<float, 64><<<grid, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<float*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace ts
