// Target-token sampling over the logits of the verified positions.
//
// Row r's logits x (row 0: the position after the committed context; row t+1:
// the position after draft t) go through
//   1. the windowed repetition penalty: a token among the last W tokens of the
//      row's context (the committed tokens, then the drafts on the root path of
//      draft r-1) has x -> x / theta if x > 0, else x * theta (once, however
//      often it appears);
//   2. temperature tau and the min-p filter: with Z the row's largest
//      penalised logit z, token i is kept when z_i >= Z + tau * ln(min_p),
//      i.e. p_i >= min_p * max p, with weight w_i = 2^((z_i - Z) * log2(e)/tau);
//   3. the draw: the smallest token id whose cumulative weight exceeds
//      u[r] * sum(w). tau = 0 is greedy: the first token with z_i == Z.
//
// Rows are cut into sub-slices of 4096 logits. Two launches, one read of the
// logits:
//   A. grid (sub-slices / kSubPerWG, rows): a workgroup issues the window's
//      few loads, then the loads of all its sub-slices (16 logits a thread
//      each, held raw in registers), marks the windowed tokens of its range in
//      an LDS bitmap while they land, and for each sub-slice writes its
//      maximum m, its kept weight relative to m with
//      the sub-slice's own cut m + cut, and the kept tokens themselves while
//      there are at most 32 (a deterministic compaction in thread order).
//   B. grid (rows): the row maximum Z gives the row's cut Z + cut >= m + cut,
//      so a listed sub-slice's kept tokens are all in its list; with min-p off
//      (cut = -inf) the sub-slice sum rescales exactly by 2^((m - Z) s2). Only
//      a sub-slice with more than 32 kept tokens and min-p on is read again.
//      A scan of the sub-slice weights finds the one the draw falls in; its
//      list (sorted by id) or its logits give the token.
#include "decode.h"

namespace ts {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesS = kThreads / kWave;
constexpr int kSubPerWG = 1;
constexpr int kPT = kSampleSub / kThreads;              // logits per thread per sub-slice (16)
constexpr int kBitWords = kSubPerWG * kSampleSub / 32;  // bitmap of one workgroup's range

struct Lds {
  uint32_t bits[kBitWords];                 // windowed tokens of [i0, i1)
  int par[TS_MAX_DRAFT], dtok[TS_MAX_DRAFT];
  int path[TS_MAX_DRAFT];                   // draft tokens on the root path, leaf first
  int path_len;
  float red[kWavesS];
  int ired[kWavesS];
};

struct PickLds {
  float c[kSampleMaxSubs];                  // weight of each sub-slice at the row's cut
  int ovf[kSampleMaxSubs];                  // sub-slices that need their logits again
  int n_ovf;
  int bsel, win, last;
  float base;
  SampleCand sorted[kSampleList];
};

// The window loads of one thread, issued ahead of the logits: the forest
// entries tid + 256 k and up to 4 of the last min(n_hist, W) committed tokens.
constexpr int kHistRegs = 4;
constexpr int kDraftRegs = TS_MAX_DRAFT / kThreads;   // forest entries a thread stages
struct WindowRegs {
  int par[kDraftRegs], dtok[kDraftRegs];
  int hist[kHistRegs];
};

__device__ __forceinline__ void window_prefetch(const SampleArgs& a, int r, WindowRegs& w) {
  const int tid = threadIdx.x;
  const bool walk = r > 0 && a.window > 0;
#pragma unroll
  for (int k = 0; k < kDraftRegs; ++k) {
    const int t = tid + k * kThreads;
    w.par[k] = -1;
    w.dtok[k] = 0;
    if (walk && t < a.T) {
      w.par[k] = a.parent[t];
      w.dtok[k] = a.draft_tok[t];
    }
  }
  const int nh = min(a.n_hist, a.window);
  const int h0 = a.n_hist - nh;
#pragma unroll
  for (int k = 0; k < kHistRegs; ++k) {
    const int e = tid + k * kThreads;
    w.hist[k] = e < nh ? a.hist[h0 + e] : -1;
  }
}

// Marks, in s.bits, the tokens of [i0, i1) that lie in row r's window: the
// draft tokens on the root path of draft r-1 (at most W of them, leaf first)
// and the last W - (path length) committed tokens.
__device__ void mark_window(const SampleArgs& a, int r, int i0, int i1, Lds& s, const WindowRegs& w) {
  const int tid = threadIdx.x;
  const int nw = (i1 - i0 + 31) >> 5;
  for (int k = tid; k < nw; k += kThreads) s.bits[k] = 0u;
  const bool walk = r > 0 && a.window > 0;
#pragma unroll
  for (int k = 0; k < kDraftRegs; ++k) {
    const int t = tid + k * kThreads;
    if (walk && t < a.T) {
      s.par[t] = w.par[k];
      s.dtok[t] = w.dtok[k];
    }
  }
  __syncthreads();
  if (walk && tid == 0) {
    int n = 0, x = r - 1;
    while (x >= 0 && n < a.window) {           // parents outside [-1, x) end the path
      s.path[n++] = s.dtok[x];
      const int p = s.par[x];
      x = (p >= -1 && p < x) ? p : -1;
    }
    s.path_len = n;
  }
  __syncthreads();
  const int len = walk ? s.path_len : 0;
  auto mark = [&](int tk) {
    if (tk >= i0 && tk < i1) atomicOr(&s.bits[(tk - i0) >> 5], 1u << ((tk - i0) & 31));
  };
  for (int j = tid; j < len; j += kThreads) mark(s.path[j]);
  // committed tokens: of the last nh, those with index >= nh - h belong to this row
  const int nh = min(a.n_hist, a.window);
  const int h = max(0, min(a.n_hist, a.window - len));
#pragma unroll
  for (int k = 0; k < kHistRegs; ++k) {
    const int e = tid + k * kThreads;
    if (e < nh && e >= nh - h) mark(w.hist[k]);
  }
  for (int e = tid + kHistRegs * kThreads; e < nh; e += kThreads)   // windows above 1024 tokens
    if (e >= nh - h) mark(a.hist[a.n_hist - nh + e]);
  __syncthreads();
}

__device__ __forceinline__ float penalised(float x, const Lds& s, int rel, float theta) {
  if ((s.bits[rel >> 5] >> (rel & 31)) & 1u) return x > 0.0f ? x / theta : x * theta;
  return x;
}

// Token of element e of this thread in the sub-slice starting at `base`:
// groups of 16 bytes, consecutive threads on consecutive groups.
template <typename Tin>
__device__ __forceinline__ int token_of(int base, int e) {
  constexpr int kPer = 16 / sizeof(Tin);
  return base + ((e / kPer) * kThreads + (int)threadIdx.x) * kPer + (e % kPer);
}

// The thread's 16 logits of a sub-slice at `base`, -inf past V. Rows that are
// whole 16-byte groups from a 16-byte-aligned base (the host checks) take
// 16-byte loads, all issued back to back with no branch around them (a group
// past V is clamped onto the row's last group and masked afterwards); they
// stay raw in registers until used. Other rows take element loads.
template <typename Tin>
struct SubRaw {
  static constexpr int kPer = 16 / sizeof(Tin);
  static constexpr int kG = kPT / kPer;
  uint4 u[kG];
};

template <typename Tin, bool kVec>
__device__ __forceinline__ void fetch_sub(const Tin* row, int base, int V, SubRaw<Tin>& w) {
  if constexpr (kVec) {
    constexpr int kPer = SubRaw<Tin>::kPer;
#pragma unroll
    for (int g = 0; g < SubRaw<Tin>::kG; ++g) {
      const int t0 = min(token_of<Tin>(base, g * kPer), V - kPer);
      w.u[g] = *reinterpret_cast<const uint4*>(row + t0);
    }
  }
}

template <typename Tin, bool kVec>
__device__ __forceinline__ void unpack_sub(const Tin* row, int base, int V, SubRaw<Tin>& w,
                                           float (&x)[kPT]) {
  constexpr int kPer = SubRaw<Tin>::kPer;
  if constexpr (kVec) {
#pragma unroll
    for (int g = 0; g < SubRaw<Tin>::kG; ++g) {
      // the unpacking stays here: otherwise it is hoisted next to the loads,
      // whose wait would then precede the work meant to hide them
      asm volatile("" : "+v"(w.u[g].x), "+v"(w.u[g].y), "+v"(w.u[g].z), "+v"(w.u[g].w));
      Tin e[kPer];
      __builtin_memcpy(e, &w.u[g], 16);
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        x[g * kPer + q] = token_of<Tin>(base, g * kPer + q) < V ? Elem<Tin>::load(&e[q]) : -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPT; ++e) {
      const int t = token_of<Tin>(base, e);
      x[e] = t < V ? Elem<Tin>::load(row + t) : -INFINITY;
    }
  }
}

__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kWavesS; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < kWavesS; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Exclusive prefix over the threads in index order; total = the sum of all.
template <typename T>
__device__ T block_excl_scan(T v, T* red, T& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  T incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const T y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  T excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = T(0);
  if (lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  T off = T(0);
  total = T(0);
#pragma unroll
  for (int w = 0; w < kWavesS; ++w) {
    off += w < wave ? red[w] : T(0);
    total += red[w];
  }
  __syncthreads();
  return off + excl;
}

template <typename Tin, int kSPW, bool kVec>
__global__ __launch_bounds__(kThreads) void sample_scan_kernel(SampleArgs a) {
  __shared__ Lds s;
  const int r = blockIdx.y, tid = threadIdx.x;
  const int b0 = blockIdx.x * kSPW, b1 = min(a.nb, b0 + kSPW);
  const int i0 = b0 * kSampleSub, i1 = min(a.V, b1 * kSampleSub);
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  // the window's few loads first, then every logits load of the workgroup
  // (sub-slices past the row's last one reload it); the bitmap is built
  // while the logits are in flight
  WindowRegs wr;
  window_prefetch(a, r, wr);
  SubRaw<Tin> raw[kSPW];
#pragma unroll
  for (int k = 0; k < kSPW; ++k) fetch_sub<Tin, kVec>(row, min(b0 + k, b1 - 1) * kSampleSub, a.V, raw[k]);
  mark_window(a, r, i0, i1, s, wr);
#pragma unroll
  for (int k = 0; k < kSPW; ++k) {
    const int b = b0 + k;
    if (b >= b1) break;
    const int base = b * kSampleSub;
    float x[kPT];
    unpack_sub<Tin, kVec>(row, base, a.V, raw[k], x);
    float z[kPT];
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPT; ++e) {
      const int i = token_of<Tin>(base, e);
      z[e] = i < a.V ? penalised(x[e], s, i - i0, a.theta) : -INFINITY;
      m = fmaxf(m, z[e]);
    }
    m = block_max(m, s.red);
    const float thr = m + a.cut;
    float acc = 0.0f;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kPT; ++e) {
      if (z[e] > -INFINITY && z[e] >= thr) {
        acc += exp2f((z[e] - m) * a.s2);
        ++cnt;
      }
    }
    int n_all;
    int slot = block_excl_scan<int>(cnt, s.ired, n_all);
    if (n_all <= kSampleList) {
      SampleCand* list = a.cand + ((int64_t)r * a.nb + b) * kSampleList;
#pragma unroll
      for (int e = 0; e < kPT; ++e) {
        if (z[e] > -INFINITY && z[e] >= thr) list[slot++] = SampleCand{z[e], token_of<Tin>(base, e)};
      }
    }
    acc = block_sum(acc, s.red);
    if (tid == 0) a.sub[r * a.nb + b] = SampleSub{m, acc, n_all, 0};
  }
}

// Sum of the kept weights of sub-slice b at the row's cut, from its logits.
template <typename Tin>
__device__ float sub_weight(const SampleArgs& a, int r, int b, float Z, float thr, Lds& s) {
  const int base = b * kSampleSub;
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  WindowRegs wr;
  window_prefetch(a, r, wr);
  mark_window(a, r, base, min(a.V, base + kSampleSub), s, wr);
  SubRaw<Tin> raw;
  float x[kPT];
  unpack_sub<Tin, false>(row, base, a.V, raw, x);
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < kPT; ++e) {
    const int i = token_of<Tin>(base, e);
    if (i < a.V) {
      const float z = penalised(x[e], s, i - base, a.theta);
      if (z > -INFINITY && z >= thr) acc += exp2f((z - Z) * a.s2);
    }
  }
  return block_sum(acc, s.red);
}

template <typename Tin>
__global__ __launch_bounds__(kThreads) void sample_pick_kernel(SampleArgs a) {
  __shared__ Lds s;
  __shared__ PickLds p;
  const int r = blockIdx.x, tid = threadIdx.x;
  const bool greedy = a.s2 == 0.0f;
  SampleSub sb{-INFINITY, 0.0f, 0, 0};
  if (tid < a.nb) sb = a.sub[r * a.nb + tid];
  const float Z = block_max(sb.m, s.red);
  const float thr = Z + a.cut;
  if (tid == 0) {
    p.bsel = a.nb;
    p.win = INT32_MAX;
    p.last = -1;
    p.base = 0.0f;
    p.n_ovf = 0;
  }
  __syncthreads();
  float target = 0.0f;
  bool fallback = false;
  if (greedy) {
    if (tid < a.nb && sb.m == Z) atomicMin(&p.bsel, tid);
    __syncthreads();
  } else {
    // each sub-slice's weight at the row's cut (relative to Z)
    float c = 0.0f;
    if (tid < a.nb && sb.m > -INFINITY && sb.m >= thr) {
      if (a.cut == -INFINITY) {
        c = sb.s * exp2f((sb.m - Z) * a.s2);
      } else if (sb.n <= kSampleList) {
        const SampleCand* list = a.cand + ((int64_t)r * a.nb + tid) * kSampleList;
        for (int j = 0; j < sb.n; ++j) {
          const SampleCand e = list[j];
          if (e.z >= thr) c += exp2f((e.z - Z) * a.s2);
        }
      } else {
        p.ovf[atomicAdd(&p.n_ovf, 1)] = tid;
      }
    }
    p.c[tid] = c;                               // kThreads == kSampleMaxSubs
    __syncthreads();
    const int n_ovf = p.n_ovf;
    for (int k = 0; k < n_ovf; ++k) {           // rare: many kept tokens in one sub-slice
      const int b = p.ovf[k];
      const float w = sub_weight<Tin>(a, r, b, Z, thr, s);
      if (tid == 0) p.c[b] = w;
      __syncthreads();
    }
    c = p.c[tid];
    float total;
    const float excl = block_excl_scan<float>(c, s.red, total);
    target = a.u[r] * total;
    if (tid < a.nb && c > 0.0f && excl + c > target) atomicMin(&p.bsel, tid);
    __syncthreads();
    if (p.bsel == a.nb) {                       // u * total at or past the end: the last kept token
      fallback = true;
      __syncthreads();
      if (tid < a.nb && c > 0.0f) atomicMax(&p.last, tid);
      __syncthreads();
      if (tid == 0) {
        p.bsel = p.last;
        p.last = -1;
      }
    } else if (tid == p.bsel) {
      p.base = excl;
    }
    __syncthreads();
  }
  const int b = p.bsel;
  if (b < 0 || b >= a.nb) {                     // no finite logit in the row (outside the contract)
    if (tid == 0) a.tok[r] = -1;
    return;
  }
  const SampleSub chosen = a.sub[r * a.nb + b];
  const bool listed = chosen.n <= kSampleList && (greedy || a.cut > -INFINITY);
  if (listed) {
    // the sub-slice's kept tokens, in token order (greedy: its maxima)
    const SampleCand* list = a.cand + ((int64_t)r * a.nb + b) * kSampleList;
    if (tid < chosen.n) {
      const SampleCand e = list[tid];
      int rank = 0;
      for (int j = 0; j < chosen.n; ++j) rank += list[j].idx < e.idx;
      p.sorted[rank] = e;
    }
    __syncthreads();
    if (tid == 0) {
      int win = INT32_MAX, last = -1;
      float run = p.base;
      for (int j = 0; j < chosen.n; ++j) {
        const SampleCand e = p.sorted[j];
        if (greedy) {
          if (e.z == Z) {
            win = e.idx;
            break;
          }
        } else if (e.z >= thr) {
          run += exp2f((e.z - Z) * a.s2);
          last = e.idx;
          if (!fallback && win == INT32_MAX && run > target) win = e.idx;
        }
      }
      a.tok[r] = win != INT32_MAX ? win : last;
    }
    return;
  }
  // otherwise from the sub-slice's logits: thread tid owns tokens [c0, c1)
  const int base = b * kSampleSub, end = min(a.V, base + kSampleSub);
  {
    WindowRegs wr;
    window_prefetch(a, r, wr);
    mark_window(a, r, base, end, s, wr);
  }
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  const int c0 = min(end, base + tid * kPT), c1 = min(end, c0 + kPT);
  float w[kPT];
  float mine = 0.0f;
#pragma unroll
  for (int j = 0; j < kPT; ++j) {
    w[j] = 0.0f;
    if (c0 + j < c1) {
      const float z = penalised(Elem<Tin>::load(row + c0 + j), s, c0 + j - base, a.theta);
      if (greedy) {
        if (z == Z) atomicMin(&p.win, c0 + j);
      } else if (z > -INFINITY && z >= thr) {
        w[j] = exp2f((z - Z) * a.s2);
        mine += w[j];
      }
    }
  }
  if (!greedy) {
    float total;
    float run = p.base + block_excl_scan<float>(mine, s.red, total);
    int hit = INT32_MAX, last = -1;
#pragma unroll
    for (int j = 0; j < kPT; ++j) {
      if (w[j] > 0.0f) {
        run += w[j];
        last = c0 + j;
        if (hit == INT32_MAX && run > target) hit = c0 + j;
      }
    }
    if (!fallback && hit != INT32_MAX) atomicMin(&p.win, hit);
    if (last >= 0) atomicMax(&p.last, last);
  }
  __syncthreads();
  if (tid == 0) a.tok[r] = p.win != INT32_MAX ? p.win : p.last;
}

template <typename Tin>
hipError_t launch_t(const SampleArgs& a, hipStream_t st) {
  const dim3 grid((a.nb + kSubPerWG - 1) / kSubPerWG, a.R);
  constexpr int kPer = 16 / sizeof(Tin);
  // 16-byte loads when every row is whole 16-byte groups from an aligned base
  const bool vec = (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0 && a.V % kPer == 0;
  if (vec)
    sample_scan_kernel<Tin, kSubPerWG, true><<<grid, kThreads, 0, st>>>(a);
  else
    sample_scan_kernel<Tin, kSubPerWG, false><<<grid, kThreads, 0, st>>>(a);
  sample_pick_kernel<Tin><<<a.R, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

int sample_subslices(int V) { return V < 1 ? 1 : (V + kSampleSub - 1) / kSampleSub; }

size_t sample_workspace_bytes(int R, int V) {
  const size_t n = (size_t)R * sample_subslices(V);
  return n * sizeof(SampleSub) + n * kSampleList * sizeof(SampleCand);
}

hipError_t launch_sample(const SampleArgs& a, ts_dtype dtype, hipStream_t s) {
  static_assert(kThreads == kSampleMaxSubs, "the picking workgroup holds one sub-slice per thread");
  static_assert(kSampleList <= kThreads, "list entries are ranked one per thread");
  return dtype == TS_BF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace ts
