// Cross-split log-sum-exp merge of partial attention results.
//
//   lse = ln sum_s exp(l_s)      out = sum_s exp(l_s - lse) * o_s
//
// o_s is each split's softmax-normalised output and l_s its natural-log
// normaliser (-inf for a split that saw no key of the row).
//
// One workgroup per output row. The splits are spread over NG groups of D/4
// threads (each thread owns 4 columns), so every thread issues only S/NG
// independent 16-byte loads instead of walking all S splits one round trip at
// a time. Each group keeps its own running max; the groups' partial sums meet
// in LDS, rescaled to the common max.
#include "common.h"

namespace ts {
namespace {

constexpr int kThreads = 256;

template <typename Tout, int D>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(const float* __restrict__ o_part,
                                                              const float* __restrict__ l_part,
                                                              int S, int rows,
                                                              Tout* __restrict__ out,
                                                              float* __restrict__ lse) {
  constexpr int C4 = D / 4;              // threads per split group (one float4 each)
  constexpr int NG = kThreads / C4;      // split groups
  __shared__ float4 acc_s[NG][C4];
  __shared__ float m_s[NG], w_s[NG];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int gi = tid / C4, c = tid % C4;

  // each group merges its splits (s = gi, gi+NG, ...) with its own running max
  float m = -INFINITY, ws = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = gi; s < S; s += NG) {
    const int64_t pr = (int64_t)s * rows + row;
    const float ls = l_part[pr];
    const float4 o = *reinterpret_cast<const float4*>(o_part + pr * D + 4 * c);
    if (ls == -INFINITY) continue;
    const float mn = fmaxf(m, ls);
    const float a = __expf(m - mn);          // m = -inf: 0
    const float w = __expf(ls - mn);
    ws = ws * a + w;
    acc.x = acc.x * a + w * o.x; acc.y = acc.y * a + w * o.y;
    acc.z = acc.z * a + w * o.z; acc.w = acc.w * a + w * o.w;
    m = mn;
  }
  acc_s[gi][c] = acc;
  if (c == 0) { m_s[gi] = m; w_s[gi] = ws; }
  __syncthreads();
  if (gi == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < NG; ++k) M = fmaxf(M, m_s[k]);
    float wt = 0.f;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < NG; ++k) {
        if (m_s[k] == -INFINITY) continue;
        const float f = __expf(m_s[k] - M);
        wt += w_s[k] * f;
        const float4 a = acc_s[k][c];
        t.x += a.x * f; t.y += a.y * f; t.z += a.z * f; t.w += a.w * f;
      }
    }
    const float inv = wt > 0.f ? 1.f / wt : 0.f;
    Tout* op = out + (int64_t)row * D + 4 * c;
    Elem<Tout>::store(op + 0, t.x * inv);
    Elem<Tout>::store(op + 1, t.y * inv);
    Elem<Tout>::store(op + 2, t.z * inv);
    Elem<Tout>::store(op + 3, t.w * inv);
    if (lse != nullptr && c == 0) lse[row] = wt > 0.f ? M + logf(wt) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_merge(const float* o_part, const float* l_part, int n_parts, int rows,
                             int D, void* out, float* lse, ts_dtype dtype, hipStream_t s) {
  if (dtype == TS_BF16) {
    if (D == 128)
      attn_merge_kernel<bf16_t, 128><<<rows, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<bf16_t*>(out), lse);
    else
      attn_merge_kernel<bf16_t, 64><<<rows, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<bf16_t*>(out), lse);
  } else {
    if (D == 128)
      attn_merge_kernel<float, 128><<<rows, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<float*>(out), lse);
    else
      attn_merge_kernel<float, 64><<<rows, kThreads, 0, s>>>(o_part, l_part, n_parts, rows, static_cast<float*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace ts
