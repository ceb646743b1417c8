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
// Candidates are ranked by 64-bit keys (order-preserving logit key << 32 |
// ~token id: larger is better, equal logits go to the lower id); keys are
// unique. Two launches:
//   1. grid (slices, depth): each 256-thread workgroup scans one slice of its
//      row (16-byte loads), keeps a per-thread top-KL list, and extracts its
//      slice's k best keys into the workspace in k rounds of a block max;
//   2. grid (depth): each workgroup merges its row's slice candidates the same
//      way and writes the ranked candidates and its depth's nodes.
#include "decode.h"

namespace ts {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesT = kThreads / kWave;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;               // -0 and +0 rank together
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float f, int i) {
  return ((uint64_t)order_key(f) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
}

__device__ __forceinline__ int key_token(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// Per-thread descending list of the KL largest keys seen (0 = empty slot).
template <int KL> struct TopList {
  uint64_t v[KL];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < KL; ++j) v[j] = 0ull;
  }
  __device__ void offer(uint64_t key) {
    if (key > v[KL - 1]) {
      uint64_t x = key;                  // insertion by compare-exchange down the list
#pragma unroll
      for (int j = 0; j < KL; ++j) {
        const uint64_t hi = x > v[j] ? x : v[j];
        x = x > v[j] ? v[j] : x;
        v[j] = hi;
      }
    }
  }
  __device__ void pop() {
#pragma unroll
    for (int j = 0; j < KL - 1; ++j) v[j] = v[j + 1];
    v[KL - 1] = 0ull;
  }
};

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) {
    const uint64_t y = __shfl_xor(x, o, kWave);
    x = y > x ? y : x;
  }
  return x;
}

// k rounds of a block-wide max over the threads' list heads; the owner of the
// winner pops it. Writes the k winners (0 when the block has run out) to out[].
template <int KL>
__device__ void block_extract(TopList<KL>& top, int k, uint64_t* s_wmax, uint64_t* out) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  for (int r = 0; r < k; ++r) {
    const uint64_t m = wave_max_u64(top.v[0]);
    if (lane == 0) s_wmax[wave] = m;
    __syncthreads();
    uint64_t best = s_wmax[0];
#pragma unroll
    for (int w = 1; w < kWavesT; ++w) best = s_wmax[w] > best ? s_wmax[w] : best;
    if (best != 0ull && top.v[0] == best) top.pop();   // keys are unique: one owner
    if (threadIdx.x == 0) out[r] = best;
    __syncthreads();
  }
}

template <typename Tin, int KL>
__global__ __launch_bounds__(kThreads) void tree_slice_kernel(const Tin* __restrict__ logits, int V,
                                                              int slice, TreeShape shape,
                                                              uint64_t* __restrict__ ws) {
  __shared__ uint64_t s_wmax[kWavesT];
  __shared__ uint64_t s_out[kTreeMaxK];
  const int b = blockIdx.x, d = blockIdx.y, nb = gridDim.x, tid = threadIdx.x;
  const int k = shape.k[d];
  const Tin* row = logits + (int64_t)d * V;
  const int i0 = b * slice, i1 = min(V, i0 + slice);
  TopList<KL> top;
  top.init();
  // 16-byte loads over the slice's aligned middle, element loads at its edges
  constexpr int kPer = 16 / sizeof(Tin);
  const uintptr_t base = reinterpret_cast<uintptr_t>(row + i0);
  const int head = min(i1 - i0, (int)(((16 - (base & 15)) & 15) / sizeof(Tin)));
  const bool vec = (base % sizeof(Tin)) == 0;
  const int a0 = vec ? i0 + head : i1;
  const int nvec = vec ? (i1 - a0) / kPer : 0;
  for (int v = tid; v < nvec; v += kThreads) {
    const uint4 u = reinterpret_cast<const uint4*>(row + a0)[v];
    Tin e[kPer];
    __builtin_memcpy(e, &u, 16);
#pragma unroll
    for (int q = 0; q < kPer; ++q) top.offer(make_key(Elem<Tin>::load(&e[q]), a0 + v * kPer + q));
  }
  for (int i = i0 + tid; i < a0; i += kThreads) top.offer(make_key(Elem<Tin>::load(row + i), i));
  for (int i = a0 + nvec * kPer + tid; i < i1; i += kThreads) top.offer(make_key(Elem<Tin>::load(row + i), i));
  block_extract<KL>(top, k, s_wmax, s_out);
  if (tid < k) ws[((int64_t)d * nb + b) * kTreeMaxK + tid] = s_out[tid];
}

template <int KL>
__global__ __launch_bounds__(kThreads) void tree_merge_kernel(const uint64_t* __restrict__ ws, int nb,
                                                              TreeShape shape,
                                                              int32_t* __restrict__ parent,
                                                              int32_t* __restrict__ draft_tok,
                                                              int32_t* __restrict__ cand_out) {
  __shared__ uint64_t s_wmax[kWavesT];
  __shared__ uint64_t s_out[kTreeMaxK];
  const int d = blockIdx.x, tid = threadIdx.x;
  const int k = shape.k[d];
  TopList<KL> top;
  top.init();
  const uint64_t* w = ws + (int64_t)d * nb * kTreeMaxK;
  for (int e = tid; e < nb * k; e += kThreads) top.offer(w[(e / k) * kTreeMaxK + (e % k)]);
  block_extract<KL>(top, k, s_wmax, s_out);
  if (cand_out != nullptr && tid < kTreeMaxK) cand_out[d * kTreeMaxK + tid] = tid < k ? key_token(s_out[tid]) : -1;
  const int off = shape.off[d], n = shape.n[d];
  const int poff = d > 0 ? shape.off[d - 1] : 0;
  for (int q = tid; q < n; q += kThreads) {
    parent[off + q] = d > 0 ? poff + q / k : -1;
    draft_tok[off + q] = key_token(s_out[q % k]);
  }
}

template <int KL>
void launch_kl(const void* logits, int V, const TreeShape& shape, int depth, int nb, int slice,
               uint64_t* ws, int32_t* parent, int32_t* draft_tok, int32_t* cand, ts_dtype dtype,
               hipStream_t s) {
  dim3 g1(nb, depth);
  if (dtype == TS_BF16)
    tree_slice_kernel<bf16_t, KL><<<g1, kThreads, 0, s>>>(static_cast<const bf16_t*>(logits), V, slice, shape, ws);
  else
    tree_slice_kernel<float, KL><<<g1, kThreads, 0, s>>>(static_cast<const float*>(logits), V, slice, shape, ws);
  tree_merge_kernel<KL><<<depth, kThreads, 0, s>>>(ws, nb, shape, parent, draft_tok, cand);
}

}  // namespace

int tree_slices(int V) {
  // about 4096 logits per workgroup, at most 64 slices per position
  int nb = (V + 4095) / 4096;
  return nb < 1 ? 1 : nb > 64 ? 64 : nb;
}

hipError_t launch_build_tree(const void* logits, int V, const TreeShape& shape, int depth,
                             int32_t* parent, int32_t* draft_tok, int32_t* cand, void* workspace,
                             ts_dtype dtype, hipStream_t s) {
  const int nb = tree_slices(V);
  const int slice = (V + nb - 1) / nb;
  int kmax = 1;
  for (int d = 0; d < depth; ++d) kmax = shape.k[d] > kmax ? shape.k[d] : kmax;
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  // a thread's list only needs the most keys one workgroup can extract
  if (kmax <= 4) launch_kl<4>(logits, V, shape, depth, nb, slice, ws, parent, draft_tok, cand, dtype, s);
  else if (kmax <= 8) launch_kl<8>(logits, V, shape, depth, nb, slice, ws, parent, draft_tok, cand, dtype, s);
  else launch_kl<16>(logits, V, shape, depth, nb, slice, ws, parent, draft_tok, cand, dtype, s);
  return hipGetLastError();
}

}  // namespace ts
