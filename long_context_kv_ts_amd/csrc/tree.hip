// Candidate tree of draft tokens from the per-position logits.
//
// Shape [k_0, .., k_{P-1}]: the candidates at depth d are the k_d highest
// logits of position d (equal logits: lower token id first); the tree is the
// product of the depths, numbered breadth-first and, inside a depth, in
// lexicographic order of the candidate ranks along the root path. Node q
// (0-based inside depth d) therefore has rank q % k_d at its own depth and
// parent q / k_d inside depth d-1, so every depth's nodes can be written
// knowing only that depth's candidates.
//
// One 1024-thread workgroup per depth: each thread keeps its own top-k of
// 64-bit keys (order-preserving logit key << 32 | ~token id, so larger is
// better and ties go to the lower id) while it strides over the vocabulary;
// the block then extracts the k best in k rounds of a block-wide max; finally
// the workgroup writes its depth's nodes.
#include "common.h"

namespace ts {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesT = kThreads / kWave;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;               // -0 and +0 rank together
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const uint64_t y = __shfl_xor(x, o, kWave);
    x = y > x ? y : x;
  }
  return x;
}

template <typename Tin>
__global__ __launch_bounds__(kThreads) void build_tree_kernel(const Tin* __restrict__ logits, int V,
                                                              TreeShape shape,
                                                              int32_t* __restrict__ parent,
                                                              int32_t* __restrict__ draft_tok,
                                                              int32_t* __restrict__ cand_out) {
  __shared__ uint64_t s_wmax[kWavesT];
  __shared__ int32_t s_cand[kTreeMaxK];
  const int d = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int k = shape.k[d];
  const Tin* row = logits + (int64_t)d * V;

  // per-thread top-kTreeMaxK, descending; 0 is below every real key
  uint64_t top[kTreeMaxK];
#pragma unroll
  for (int j = 0; j < kTreeMaxK; ++j) top[j] = 0ull;
  for (int i = tid; i < V; i += kThreads) {
    const uint64_t key = ((uint64_t)order_key(Elem<Tin>::load(row + i)) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
    if (key > top[kTreeMaxK - 1]) {
      uint64_t x = key;                  // insertion by compare-exchange down the list
#pragma unroll
      for (int j = 0; j < kTreeMaxK; ++j) {
        const uint64_t hi = x > top[j] ? x : top[j];
        x = x > top[j] ? top[j] : x;
        top[j] = hi;
      }
    }
  }
  // k rounds: the best remaining head wins and its owner pops it
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(top[0]);
    if (lane == 0) s_wmax[wave] = m;
    __syncthreads();
    uint64_t best = s_wmax[0];
#pragma unroll
    for (int w = 1; w < kWavesT; ++w) best = s_wmax[w] > best ? s_wmax[w] : best;
    if (top[0] == best && best != 0ull) {     // keys are unique: exactly one owner
#pragma unroll
      for (int j = 0; j < kTreeMaxK - 1; ++j) top[j] = top[j + 1];
      top[kTreeMaxK - 1] = 0ull;
    }
    if (tid == 0) s_cand[r] = (int32_t)(0xFFFFFFFFu - (uint32_t)best);
    __syncthreads();
  }
  if (cand_out != nullptr && tid < kTreeMaxK) cand_out[d * kTreeMaxK + tid] = tid < k ? s_cand[tid] : -1;

  // this depth's nodes
  const int off = shape.off[d], n = shape.n[d];
  const int poff = d > 0 ? shape.off[d - 1] : 0;
  for (int q = tid; q < n; q += kThreads) {
    parent[off + q] = d > 0 ? poff + q / k : -1;
    draft_tok[off + q] = s_cand[q % k];
  }
}

}  // namespace

hipError_t launch_build_tree(const void* logits, int V, const TreeShape& shape, int depth,
                             int32_t* parent, int32_t* draft_tok, int32_t* cand, ts_dtype dtype,
                             hipStream_t s) {
  if (dtype == TS_BF16)
    build_tree_kernel<bf16_t><<<depth, kThreads, 0, s>>>(static_cast<const bf16_t*>(logits), V, shape,
                                                        parent, draft_tok, cand);
  else
    build_tree_kernel<float><<<depth, kThreads, 0, s>>>(static_cast<const float*>(logits), V, shape,
                                                       parent, draft_tok, cand);
  return hipGetLastError();
}

}  // namespace ts
