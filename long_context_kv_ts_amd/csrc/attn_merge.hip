// Cross-split log-sum-exp merge of partial attention results (fp32 or bf16
// partials): the kernel and its launch shape; the per-workgroup body (and the
// formula) is in merge_block.h.
#include "merge_block.h"

namespace ts {
namespace {

template <typename Tout, int D, int WPR, typename Tin>
__global__ __launch_bounds__(MergeShape<WPR>::block) void attn_merge_kernel(
    const Tin* __restrict__ o_part, const float* __restrict__ l_part, int S, int rows,
    Tout* __restrict__ out, float* __restrict__ lse) {
  merge_block<Tout, D, WPR, Tin>(o_part, l_part, S, rows, out, lse, blockIdx.x);
}

template <typename Tout, int D, int WPR, typename Tin>
void launch_one(const Tin* o_part, const float* l_part, int S, int rows, void* out, float* lse,
                hipStream_t s) {
  using Sh = MergeShape<WPR>;
  const int grid = (rows + Sh::rows - 1) / Sh::rows;
  attn_merge_kernel<Tout, D, WPR, Tin><<<grid, Sh::block, 0, s>>>(o_part, l_part, S, rows,
                                                                  static_cast<Tout*>(out), lse);
}

template <typename Tout, int D, typename Tin>
void launch_d(const Tin* o_part, const float* l_part, int S, int rows, void* out, float* lse,
              hipStream_t s) {
  // lanes needed so that each lane holds at most one batch of splits
  const int need = ((S + kMergeBatch - 1) / kMergeBatch) * (D / 4);
  if (need <= 64) launch_one<Tout, D, 1>(o_part, l_part, S, rows, out, lse, s);
  else if (need <= 128) launch_one<Tout, D, 2>(o_part, l_part, S, rows, out, lse, s);
  else if (need <= 256) launch_one<Tout, D, 4>(o_part, l_part, S, rows, out, lse, s);
  else if (need <= 512) launch_one<Tout, D, 8>(o_part, l_part, S, rows, out, lse, s);
  else launch_one<Tout, D, 16>(o_part, l_part, S, rows, out, lse, s);
}

template <typename Tin>
hipError_t launch_t(const Tin* o_part, const float* l_part, int n_parts, int rows, int D, void* out,
                    float* lse, ts_dtype dtype, hipStream_t s) {
  if (dtype == TS_BF16) {
    if (D == 128) launch_d<bf16_t, 128>(o_part, l_part, n_parts, rows, out, lse, s);
    else launch_d<bf16_t, 64>(o_part, l_part, n_parts, rows, out, lse, s);
  } else {
    if (D == 128) launch_d<float, 128>(o_part, l_part, n_parts, rows, out, lse, s);
    else launch_d<float, 64>(o_part, l_part, n_parts, rows, out, lse, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_merge(const void* o_part, bool part_bf16, const float* l_part, int n_parts, int rows,
                             int D, void* out, float* lse, ts_dtype dtype, hipStream_t s) {
  return part_bf16 ? launch_t(static_cast<const bf16_t*>(o_part), l_part, n_parts, rows, D, out, lse, dtype, s)
                   : launch_t(static_cast<const float*>(o_part), l_part, n_parts, rows, D, out, lse, dtype, s);
}

}  // namespace ts
