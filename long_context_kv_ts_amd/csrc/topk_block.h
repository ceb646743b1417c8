#pragma once

#include "common.h"

// Top-k chunk selection per KV head, one workgroup's work as a device
// function, so that the top-k kernel (1024 threads a head) and the launch
// that shares its grid with the cross-split merge (256 threads a head) run the
// same selection.
//
// Scores map to order-preserving 32-bit keys (larger score -> larger key; -0
// and +0 share a key). Ties go to the lower chunk index and the chosen chunks
// are written in ascending index order, so no sort is needed:
//   1. up to four 8-bit radix passes over an LDS histogram find the prefix
//      `thr` (the bits `mask` covers) of the k-th largest element's offset
//      d = key - (smallest key) and how many (`need`) of the elements with
//      that prefix are kept -- the lowest-indexed ones. Digits are taken from
//      the top of d's range, so the first pass already spreads the keys over
//      the bins (scores of one magnitude share their top key bits, and would
//      crowd one bin's atomics). The passes stop early once the bin of the k-th
//      element holds exactly `need` elements: all of them are kept;
//   2. an exclusive count, in index order, of elements whose prefix is above
//      `thr` and of elements equal to it gives every kept element its output
//      slot (slot = above_before + min(equal_before, need)).
// Thread t of kNT owns elements t, t + kNT, t + 2 kNT, ... (coalesced loads).
// With n <= kNT * kPer the keys stay in registers across all passes; larger n
// re-reads the scores (L2-resident) in every pass. Per-wave counts come from ballots,
// the bin search and the cross-wave prefix from one 64-lane scan each.
namespace ts {

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;               // -0 and +0 compare equal: one key
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t popc_below(uint64_t ballot, int lane) {
  return (uint32_t)__popcll(ballot & ((1ull << lane) - 1ull));
}

// One KV head g's selection by a kNT-thread workgroup, kPer elements a thread
// per round (with kResident the keys of n <= kNT * kPer stay in registers).
template <int kNT, int kPer, bool kResident>
__device__ __forceinline__ void topk_block(const float* __restrict__ scores, int n, int k,
                                           int32_t* __restrict__ idx_out, float* __restrict__ val_out, int g) {
  constexpr int kThreads = kNT;
  constexpr int kWaves = kThreads / kWave;
  constexpr int kRound = kThreads * kPer;         // elements per round
  static_assert(kPer * kWaves <= kWave, "one scan lane per (round element, wave)");
  __shared__ uint32_t hist[2][256];
  __shared__ uint32_t cnt_gt[kPer * kWaves], cnt_eq[kPer * kWaves];
  __shared__ uint32_t sh_digit, sh_need, sh_whole, sh_kmin, sh_kmax;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const float* s = scores + (int64_t)g * n;
  const int n_rounds = (n + kRound - 1) / kRound;

  uint32_t rk[kPer];
  float rv[kPer];
  if constexpr (kResident) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = j * kThreads + tid;
      rv[j] = i < n ? s[i] : 0.f;
      rk[j] = order_key(rv[j]);
    }
  }
  auto key_at = [&](int r, int j) -> uint32_t {
    if constexpr (kResident) return rk[j];
    const int i = (r * kPer + j) * kThreads + tid;
    return i < n ? order_key(s[i]) : 0u;
  };

  if (tid < 512) (&hist[0][0])[tid] = 0u;
  if (tid == 0) {
    sh_kmin = 0xFFFFFFFFu;
    sh_kmax = 0u;
  }
  __syncthreads();

  // the keys' range
  {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int r = 0; r < n_rounds; ++r)
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = (r * kPer + j) * kThreads + tid;
        if (i < n) {
          lo = min(lo, key_at(r, j));
          hi = max(hi, key_at(r, j));
        }
      }
    lo = __float_as_uint(wave_reduce(__uint_as_float(lo), [](float a, float b) {
      return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
    }));
    hi = __float_as_uint(wave_reduce(__uint_as_float(hi), [](float a, float b) {
      return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
    }));
    if (lane == 0) {
      atomicMin(&sh_kmin, lo);
      atomicMax(&sh_kmax, hi);
    }
  }
  __syncthreads();
  const uint32_t kmin = sh_kmin;
  const int nbits = sh_kmax == kmin ? 0 : 32 - __clz((int)(sh_kmax - kmin));
  const int n_passes = (nbits + 7) / 8;  // 8-bit digits from the top of d's range

  // 1. radix select of the k-th largest offset
  uint32_t prefix = 0u, mask = 0u, need = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (pass >= n_passes || (pass > 0 && sh_whole)) break;   // uniform (read after the last barrier)
    // the next 8 bits below those already decided (the last pass may overlap
    // decided bits, which all candidates share)
    const int shift = max(nbits - 8 * (pass + 1), 0);
    uint32_t* h = hist[pass & 1];
    for (int r = 0; r < n_rounds; ++r)
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = (r * kPer + j) * kThreads + tid;
        const uint32_t d = key_at(r, j) - kmin;
        if (i < n && (d & mask) == prefix) atomicAdd(&h[(d >> shift) & 255u], 1u);
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
      uint32_t above = wave_incl_scan(tot) - tot;   // elements with larger digits
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < need && above + c[j] >= need) {
          sh_digit = 255u - 4u * lane - j;
          sh_need = need - above;
          sh_whole = above + c[j] == need;   // the whole bin is kept
        }
        above += c[j];
      }
    } else if (wave == (kWaves > 4 ? 4 : 1) && pass < 3) {
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
  const uint32_t thr = prefix;             // the k-th element's offset on the bits of `mask`

  // 2. index-order compaction
  uint32_t base_gt = 0u, base_eq = 0u;          // wave 0: counts of earlier rounds
  for (int r = 0; r < n_rounds; ++r) {
    uint32_t key[kPer], pg[kPer], pe[kPer];
    bool gt[kPer], eq[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = (r * kPer + j) * kThreads + tid;
      key[j] = key_at(r, j) - kmin;
      gt[j] = i < n && (key[j] & mask) > thr;
      eq[j] = i < n && (key[j] & mask) == thr;
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
      const uint32_t a = lane < kPer * kWaves ? cnt_gt[lane] : 0u;
      const uint32_t b = lane < kPer * kWaves ? cnt_eq[lane] : 0u;
      const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
      if (lane < kPer * kWaves) {
        cnt_gt[lane] = base_gt + ia - a;
        cnt_eq[lane] = base_eq + ib - b;
      }
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
        if (val_out) {
          if constexpr (kResident) val_out[(int64_t)g * k + pos] = rv[j];
          else val_out[(int64_t)g * k + pos] = s[i];
        }
      }
    }
    if (r + 1 < n_rounds) __syncthreads();      // cnt_* is rewritten next round
  }
}


}  // namespace ts
