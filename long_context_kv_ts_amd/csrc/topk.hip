// Top-k chunk selection per KV head.
//
// Scores map to order-preserving 32-bit keys (larger score -> larger key; -0
// and +0 share a key). Ties go to the lower chunk index and the chosen chunks
// are written in ascending index order.
//
// n <= 4096 (the partial-KV workloads: 1600 chunks of 64 tokens at 100K):
//   one 1024-thread workgroup per KV head sorts the unique 64-bit keys
//   (score key << 32 | ~index) descending with a bitonic network in LDS; the
//   first k are the selection, which a second bitonic sort orders by index.
// larger n: four 8-bit radix passes over LDS histograms find the exact key of
//   the k-th largest element and how many of the elements equal to it are
//   kept; one exclusive prefix sum over the chunks in index order then both
//   breaks ties toward lower indices and writes the result in index order
//   (256 threads, each owning a contiguous run of chunk indices).
#include "common.h"

namespace ts {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;               // -0 and +0 compare equal: one key
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; returns this thread's prefix and
// writes the total to *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* buf, uint32_t* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const uint32_t add = tid >= off ? buf[tid - off] : 0u;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = buf[tid];
  *total = buf[kThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, int n,
                                                        int k, int32_t* __restrict__ idx_out,
                                                        float* __restrict__ val_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_buf[kThreads];
  __shared__ uint32_t sh_digit, sh_need;
  const int tid = threadIdx.x, g = blockIdx.x;
  const float* s = scores + (int64_t)g * n;
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);

  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    if (tid == 0) {
      sh_digit = 0u;
      sh_need = need;
    }
    __syncthreads();
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = order_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t looks at digit 255 - t: inclusive count of digits >= it
    const uint32_t c = hist[255 - tid];
    uint32_t total;
    const uint32_t above = block_exclusive_scan(c, scan_buf, &total);   // digits > 255-t
    if (above < need && above + c >= need) {
      sh_digit = 255u - tid;
      sh_need = need - above;
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    need = sh_need;
    __syncthreads();
  }
  const uint32_t thr = prefix;   // key of the k-th largest; keep `need` of the equal ones

  uint32_t n_eq = 0u;
  for (int i = i0; i < i1; ++i) n_eq += order_key(s[i]) == thr;
  uint32_t tot;
  uint32_t eq_before = block_exclusive_scan(n_eq, scan_buf, &tot);
  uint32_t n_sel = 0u;
  {
    uint32_t e = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = order_key(s[i]);
      if (key > thr) ++n_sel;
      else if (key == thr) { n_sel += e < need; ++e; }
    }
  }
  uint32_t pos = block_exclusive_scan(n_sel, scan_buf, &tot);
  uint32_t e = eq_before;
  for (int i = i0; i < i1; ++i) {
    const float f = s[i];
    const uint32_t key = order_key(f);
    bool keep = false;
    if (key > thr) keep = true;
    else if (key == thr) { keep = e < need; ++e; }
    if (keep && pos < (uint32_t)k) {
      idx_out[(int64_t)g * k + pos] = i;
      if (val_out) val_out[(int64_t)g * k + pos] = f;
      ++pos;
    }
  }
}

// Bitonic sort of N (power of two) 64-bit keys in LDS; descending if `desc`.
// Pair i of a stage is (lo, lo + stride) with lo = 2i - i % stride.
__device__ __forceinline__ void bitonic_sort(uint64_t* v, int N, bool desc, int tid, int nthreads) {
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (N >> 1); i += nthreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0) != desc;     // ascending run?
        const uint64_t a = v[lo], b = v[hi];
        if ((a > b) == up) {
          v[lo] = b;
          v[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

constexpr int kSortMax = 4096;
constexpr int kSortThreads = 1024;

__global__ __launch_bounds__(kSortThreads) void topk_sort_kernel(const float* __restrict__ scores,
                                                                 int n, int k,
                                                                 int32_t* __restrict__ idx_out,
                                                                 float* __restrict__ val_out) {
  __shared__ uint64_t v[kSortMax];
  const int tid = threadIdx.x, g = blockIdx.x;
  const float* s = scores + (int64_t)g * n;
  int N = 2;
  while (N < n) N <<= 1;
  // padding sorts last: every real key has a non-zero high word
  for (int i = tid; i < N; i += kSortThreads)
    v[i] = i < n ? ((uint64_t)order_key(s[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i) : 0ull;
  __syncthreads();
  bitonic_sort(v, N, true, tid, kSortThreads);
  // the first k, re-keyed by index (index << 32 | score key), sorted ascending
  int K = 2;
  while (K < k) K <<= 1;
  uint64_t w[kSortMax / kSortThreads];
  int cnt = 0;
  for (int i = tid; i < K; i += kSortThreads) {
    uint64_t x = ~0ull;
    if (i < k) {
      const uint64_t y = v[i];
      x = ((uint64_t)(0xFFFFFFFFu - (uint32_t)y) << 32) | (y >> 32);
    }
    w[cnt++] = x;
  }
  __syncthreads();
  cnt = 0;
  for (int i = tid; i < K; i += kSortThreads) v[i] = w[cnt++];
  __syncthreads();
  bitonic_sort(v, K, false, tid, kSortThreads);
  for (int i = tid; i < k; i += kSortThreads) {
    const uint64_t x = v[i];
    idx_out[(int64_t)g * k + i] = (int32_t)(x >> 32);
    if (val_out) {
      const uint32_t key = (uint32_t)x;
      const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
      val_out[(int64_t)g * k + i] = __uint_as_float(u);
    }
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int Hkv, int n, int k, int32_t* idx, float* val,
                       hipStream_t s) {
  if (n <= kSortMax) topk_sort_kernel<<<Hkv, kSortThreads, 0, s>>>(scores, n, k, idx, val);
  else topk_kernel<<<Hkv, kThreads, 0, s>>>(scores, n, k, idx, val);
  return hipGetLastError();
}

}  // namespace ts
