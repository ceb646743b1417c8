// Top-k chunk selection per KV head by radix select, then stream compaction.
//
// Scores map to order-preserving 32-bit keys (larger score -> larger key).
// Four 8-bit radix passes over LDS histograms find the exact key of the k-th
// largest element; `need` = how many elements equal to that key are kept.
// Among equal keys the lower chunk index wins, and the chosen chunks are
// written in ascending index order: both fall out of one exclusive prefix
// sum over the chunks in index order. One 256-thread workgroup per KV head;
// every thread owns a contiguous run of chunk indices.
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

}  // namespace

hipError_t launch_topk(const float* scores, int Hkv, int n, int k, int32_t* idx, float* val,
                       hipStream_t s) {
  topk_kernel<<<Hkv, kThreads, 0, s>>>(scores, n, k, idx, val);
  return hipGetLastError();
}

}  // namespace ts
