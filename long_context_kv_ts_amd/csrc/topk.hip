// Top-k chunk selection per KV head: one 1024-thread workgroup per head.
//
// Scores map to order-preserving 32-bit keys (larger score -> larger key; -0
// and +0 share a key). Ties go to the lower chunk index and the chosen chunks
// are written in ascending index order, so no sort is needed:
//   1. four 8-bit radix passes over an LDS histogram find the exact key `thr`
//      of the k-th largest element and how many (`need`) of the elements equal
//      to it are kept -- the lowest-indexed ones;
//   2. an exclusive count, in index order, of elements above `thr` and of
//      elements equal to it gives every kept element its output slot
//      (slot = above_before + min(equal_before, need)).
// Thread t owns elements t, t + 1024, t + 2048, ... (coalesced loads). With
// n <= 4096 the keys stay in registers across all passes; larger n re-reads
// the scores (L2-resident) in every pass. Per-wave counts come from ballots,
// the bin search and the cross-wave prefix from one 64-lane scan each.
#include "common.h"

namespace ts {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kPer = 4;                         // elements per thread per round
constexpr int kRound = kThreads * kPer;         // elements per round
constexpr int kResidentMax = kRound;            // n up to this stays in registers

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;               // -0 and +0 compare equal: one key
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ uint32_t popc_below(uint64_t ballot, int lane) {
  return (uint32_t)__popcll(ballot & ((1ull << lane) - 1ull));
}

template <bool kResident>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(const float* __restrict__ scores,
                                                               int n, int k,
                                                               int32_t* __restrict__ idx_out,
                                                               float* __restrict__ val_out) {
  __shared__ uint32_t hist[2][256];
  __shared__ uint32_t cnt_gt[kPer * kWaves], cnt_eq[kPer * kWaves];
  __shared__ uint32_t sh_digit, sh_need;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6, g = blockIdx.x;
  const float* s = scores + (int64_t)g * n;
  const int n_rounds = (n + kRound - 1) / kRound;

  uint32_t rk[kPer];
  if constexpr (kResident) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = j * kThreads + tid;
      rk[j] = i < n ? order_key(s[i]) : 0u;
    }
  }
  auto key_at = [&](int r, int j) -> uint32_t {
    if constexpr (kResident) return rk[j];
    const int i = (r * kPer + j) * kThreads + tid;
    return i < n ? order_key(s[i]) : 0u;
  };

  if (tid < 512) (&hist[0][0])[tid] = 0u;
  __syncthreads();

  // 1. radix select of the k-th largest key
  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* h = hist[pass & 1];
    for (int r = 0; r < n_rounds; ++r)
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = (r * kPer + j) * kThreads + tid;
        const uint32_t key = key_at(r, j);
        if (i < n && (key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
      }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 255-4l .. 252-4l, scanned from the top
      uint32_t c[4], tot = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = h[255 - 4 * lane - j];
        tot += c[j];
      }
      uint32_t above = wave_incl_scan(tot, lane) - tot;   // elements with larger digits
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < need && above + c[j] >= need) {
          sh_digit = 255u - 4u * lane - j;
          sh_need = need - above;
        }
        above += c[j];
      }
    } else if (wave == 4 && pass < 3) {
      // clear the other histogram for the next pass
      uint32_t* h2 = hist[(pass + 1) & 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) h2[lane * 4 + j] = 0u;
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    need = sh_need;
  }
  const uint32_t thr = prefix;

  // 2. index-order compaction
  uint32_t base_gt = 0u, base_eq = 0u;          // wave 0: counts of earlier rounds
  for (int r = 0; r < n_rounds; ++r) {
    uint32_t key[kPer], pg[kPer], pe[kPer];
    bool gt[kPer], eq[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = (r * kPer + j) * kThreads + tid;
      key[j] = key_at(r, j);
      gt[j] = i < n && key[j] > thr;
      eq[j] = i < n && key[j] == thr;
      const uint64_t bg = __ballot(gt[j]), be = __ballot(eq[j]);
      pg[j] = popc_below(bg, lane);
      pe[j] = popc_below(be, lane);
      if (lane == 0) {
        cnt_gt[j * kWaves + wave] = (uint32_t)__popcll(bg);
        cnt_eq[j * kWaves + wave] = (uint32_t)__popcll(be);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // entry e = j*16 + w covers elements (r*4 + j)*1024 + w*64 + [0, 64): index order
      const uint32_t a = cnt_gt[lane], b = cnt_eq[lane];
      const uint32_t ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
      cnt_gt[lane] = base_gt + ia - a;
      cnt_eq[lane] = base_eq + ib - b;
      base_gt += __shfl(ia, kWave - 1, kWave);
      base_eq += __shfl(ib, kWave - 1, kWave);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = (r * kPer + j) * kThreads + tid;
      const uint32_t gb = cnt_gt[j * kWaves + wave] + pg[j];
      const uint32_t eb = cnt_eq[j * kWaves + wave] + pe[j];
      const bool keep = gt[j] || (eq[j] && eb < need);
      const uint32_t pos = gb + min(eb, need);
      if (keep && pos < (uint32_t)k) {
        idx_out[(int64_t)g * k + pos] = i;
        if (val_out) val_out[(int64_t)g * k + pos] = s[i];
      }
    }
    if (r + 1 < n_rounds) __syncthreads();      // cnt_* is rewritten next round
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int Hkv, int n, int k, int32_t* idx, float* val,
                       hipStream_t s) {
  if (n <= kResidentMax) topk_select_kernel<true><<<Hkv, kThreads, 0, s>>>(scores, n, k, idx, val);
  else topk_select_kernel<false><<<Hkv, kThreads, 0, s>>>(scores, n, k, idx, val);
  return hipGetLastError();
}

}  // namespace ts
