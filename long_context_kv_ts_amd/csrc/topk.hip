// Top-k chunk selection per KV head: one 1024-thread workgroup per head; the
// selection itself is in topk_block.h.
#include "topk_block.h"

namespace ts {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = 4;                         // elements per thread per round
constexpr int kResidentMax = kThreads * kPer;   // n up to this stays in registers

template <bool kResident>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float* __restrict__ scores, int n, int k,
                                                               int32_t* __restrict__ idx_out,
                                                               float* __restrict__ val_out) {
  topk_block<kThreads, kPer, kResident>(scores, n, k, idx_out, val_out, blockIdx.x);
}

}  // namespace

hipError_t launch_topk(const float* scores, int Hkv, int n, int k, int32_t* idx, float* val,
                       hipStream_t s) {
  if (n <= kResidentMax) topk_select_kernel<true><<<Hkv, kThreads, 0, s>>>(scores, n, k, idx, val);
  else topk_select_kernel<false><<<Hkv, kThreads, 0, s>>>(scores, n, k, idx, val);
  return hipGetLastError();
}

}  // namespace ts
