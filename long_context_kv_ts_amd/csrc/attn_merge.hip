// Cross-split log-sum-exp merge of partial attention results.
//
//   lse = ln sum_s exp(l_s)      out = sum_s exp(l_s - lse) * o_s
//
// o_s is each split's softmax-normalised output and l_s its natural-log
// normaliser (-inf for a split that saw no key of the row). One thread merges
// 4 consecutive columns of one row; loads are 16-byte and coalesced.
#include "common.h"

namespace ts {
namespace {

template <typename Tout>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ o_part,
                                                         const float* __restrict__ l_part,
                                                         int S, int rows, int D,
                                                         Tout* __restrict__ out,
                                                         float* __restrict__ lse) {
  const int per_row = D >> 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / per_row;
  const int c4 = (int)(gid % per_row);
  if (row >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, l_part[(int64_t)s * rows + row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = l_part[(int64_t)s * rows + row];
      if (ls == -INFINITY) continue;
      const float w = expf(ls - m);
      const float4 o = *reinterpret_cast<const float4*>(o_part + ((int64_t)s * rows + row) * D + c4 * 4);
      wsum += w;
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  Tout* op = out + row * D + c4 * 4;
  Elem<Tout>::store(op + 0, acc.x * inv);
  Elem<Tout>::store(op + 1, acc.y * inv);
  Elem<Tout>::store(op + 2, acc.z * inv);
  Elem<Tout>::store(op + 3, acc.w * inv);
  if (lse != nullptr && c4 == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(const float* o_part, const float* l_part, int n_parts, int rows,
                             int D, void* out, float* lse, ts_dtype dtype, hipStream_t s) {
  const int64_t threads = (int64_t)rows * (D / 4);
  const int blocks = (int)((threads + 255) / 256);
  if (dtype == TS_BF16)
    attn_merge_kernel<bf16_t><<<blocks, 256, 0, s>>>(o_part, l_part, n_parts, rows, D,
                                                     static_cast<bf16_t*>(out), lse);
  else
    attn_merge_kernel<float><<<blocks, 256, 0, s>>>(o_part, l_part, n_parts, rows, D,
                                                    static_cast<float*>(out), lse);
  return hipGetLastError();
}

}  // namespace ts
