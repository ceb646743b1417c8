// Gather of the selected chunks into the partial KV cache: bit-exact block
// copies. A chunk of one KV head is contiguous in both the cache
// ([Hkv][stride][D]) and the partial cache ([Hkv][k*chunk][D]), so every
// workgroup copies whole chunks with 16-byte loads and stores; K and V are
// handled by the same launch (blockIdx.z). An index outside [0, L/chunk)
// zero-fills its destination chunk instead of reading.
#include "common.h"

namespace ts {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 4;

__global__ __launch_bounds__(kThreads) void gather_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc, int64_t head_bytes,
    const int32_t* __restrict__ idx, int k, int64_t chunk_bytes, int n_chunks,
    uint8_t* __restrict__ kp, uint8_t* __restrict__ vp) {
  const int i = blockIdx.x, g = blockIdx.y;
  const uint8_t* src = blockIdx.z ? vc : kc;
  uint8_t* dst = (blockIdx.z ? vp : kp) + ((int64_t)g * k + i) * chunk_bytes;
  const int c = idx[(int64_t)g * k + i];
  const int64_t n16 = chunk_bytes >> 4;
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  if (c < 0 || c >= n_chunks) {
    for (int64_t j = threadIdx.x; j < n16; j += kThreads) d4[j] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const uint4* s4 = reinterpret_cast<const uint4*>(src + (int64_t)g * head_bytes + (int64_t)c * chunk_bytes);
  // full batches: all loads issued before the stores (a 64x128 bf16 chunk is
  // exactly one batch), then a plain tail
  const int n = (int)n16;
  int j = threadIdx.x;
  for (; j + (kBatch - 1) * kThreads < n; j += kBatch * kThreads) {
    uint4 b[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) b[u] = s4[j + u * kThreads];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) d4[j + u * kThreads] = b[u];
  }
  for (; j < n; j += kThreads) d4[j] = s4[j];
}

}  // namespace

hipError_t launch_gather(const void* kc, const void* vc, int64_t stride, const int32_t* idx,
                         int Hkv, int k, int chunk, int D, int64_t L, void* kp, void* vp,
                         int elem_bytes, hipStream_t s) {
  const int64_t row_bytes = (int64_t)D * elem_bytes;
  dim3 grid(k, Hkv, 2);
  gather_kernel<<<grid, kThreads, 0, s>>>(
      static_cast<const uint8_t*>(kc), static_cast<const uint8_t*>(vc), stride * row_bytes, idx, k,
      (int64_t)chunk * row_bytes, (int)(L / chunk), static_cast<uint8_t*>(kp),
      static_cast<uint8_t*>(vp));
  return hipGetLastError();
}

}  // namespace ts
