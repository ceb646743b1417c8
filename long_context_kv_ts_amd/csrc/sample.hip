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
//   3. top-p (when top_p < 1): with W the row's total weight, token i is also
//      required to have the weight of the tokens with a larger z below
//      top_p * W, i.e. z_i >= z*, the value at which the weight at or above
//      it first reaches top_p * W (tokens of equal z share the decision);
//   4. the draw: the smallest token id whose cumulative weight exceeds
//      u[r] * sum(w). tau = 0 is greedy: the first token with z_i == Z.
//
// Rows are cut into sub-slices of 1024 logits. Two launches, one read of the
// logits (a second only for sub-slices that keep many tokens under min-p):
//   A. grid (workgroups per row, rows), kNT threads, kPW sub-slices a wave: a
//      workgroup issues the window's few loads, then every logits load of its
//      waves (16 logits a lane per sub-slice, held raw in registers), and
//      marks the windowed tokens of its range in an LDS bitmap while they land
//      (its only barriers); the bitmap is also stored, 32 words a sub-slice.
//      Each wave then summarises its own sub-slices with DPP reductions and
//      ballots: the maximum m, the kept weight relative to m at the
//      sub-slice's own cut m + cut, and the kept tokens themselves while there
//      are at most 32 (weights and list entries only for those).
//   T. (top-p only) grid (rows): each row's z* by a weighted radix select over
//      the row's logits, written to the workspace;
//   B. grid (rows): the row maximum Z gives the row's cut Z + cut >= m + cut
//      (raised to z* under top-p),
//      so a listed sub-slice's kept tokens are all in its list; with min-p off
//      (cut = -inf) the sub-slice sum rescales exactly by 2^((m - Z) s2). A
//      sub-slice with more than 32 kept tokens and min-p on is read again, one
//      a wave, with its stored window bits. A scan of the sub-slice weights (up
//      to four a thread) finds the one the draw falls in; its list (sorted by
//      id) or its logits give the token.
#include <cfloat>

#include "decode.h"

namespace ts {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesS = kThreads / kWave;
constexpr int kPL = kSampleSub / kWave;                 // logits a lane per sub-slice (scan)
constexpr int kPT = kSampleSub / kThreads;              // logits a thread per sub-slice (pick)
constexpr int kMaxScanSubs = 64;                        // sub-slices a scanning workgroup, at most
constexpr int kPerT = kSampleMaxSubs / kThreads;        // sub-slices a picking thread, at most

template <int kWords>
struct Lds {
  uint32_t bits[kWords];                    // windowed tokens of [i0, i1)
  int par[TS_MAX_DRAFT], dtok[TS_MAX_DRAFT];
  int path[TS_MAX_DRAFT];                   // draft tokens on the root path, leaf first
  int path_len;
};

struct BlockRed {
  float red[kWavesS];
};

struct PickLds {
  float c[kSampleMaxSubs];                  // weight of each sub-slice at the row's cut
  int ovf[kSampleMaxSubs];                  // sub-slices that need their logits again
  int n_ovf;
  int bsel, win, last;
  float base;
  SampleCand sorted[kSampleList];
};

// The window loads of one thread of a kNT-thread workgroup, issued ahead of
// the logits: the forest entries tid + kNT k and the thread's share of the
// last min(n_hist, W, 1024) committed tokens.
template <int kNT>
struct WindowRegs {
  static constexpr int kDraftRegs = TS_MAX_DRAFT / kNT;
  static constexpr int kHistRegs = kNT >= 1024 ? 1 : 1024 / kNT;
  int par[kDraftRegs], dtok[kDraftRegs];
  int hist[kHistRegs];
};

template <int kNT>
__device__ __forceinline__ void window_prefetch(const SampleArgs& a, int r, WindowRegs<kNT>& w) {
  constexpr int kDraftRegs = WindowRegs<kNT>::kDraftRegs, kHistRegs = WindowRegs<kNT>::kHistRegs;
  const int tid = threadIdx.x;
  const bool walk = r > 0 && a.window > 0;
#pragma unroll
  for (int k = 0; k < kDraftRegs; ++k) {
    const int t = tid + k * kNT;
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
    const int e = tid + k * kNT;
    w.hist[k] = e < nh ? a.hist[h0 + e] : -1;
  }
}

// Marks, in s.bits (nw words, all cleared first), the tokens of [i0, i1)
// that lie in row r's window: the draft tokens on the root path of draft r-1
// (at most W of them, leaf first) and the last W - (path length) committed
// tokens.
template <int kNT, typename L>
__device__ void mark_window(const SampleArgs& a, int r, int i0, int i1, int nw, L& s, const WindowRegs<kNT>& w) {
  constexpr int kDraftRegs = WindowRegs<kNT>::kDraftRegs, kHistRegs = WindowRegs<kNT>::kHistRegs;
  const int tid = threadIdx.x;
  for (int k = tid; k < nw; k += kNT) s.bits[k] = 0u;
  const bool walk = r > 0 && a.window > 0;
#pragma unroll
  for (int k = 0; k < kDraftRegs; ++k) {
    const int t = tid + k * kNT;
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
  for (int j = tid; j < len; j += kNT) mark(s.path[j]);
  // committed tokens: of the last nh, those with index >= nh - h belong to this row
  const int nh = min(a.n_hist, a.window);
  const int h = max(0, min(a.n_hist, a.window - len));
#pragma unroll
  for (int k = 0; k < kHistRegs; ++k) {
    const int e = tid + k * kNT;
    if (e < nh && e >= nh - h) mark(w.hist[k]);
  }
  for (int e = tid + kHistRegs * kNT; e < nh; e += kNT)   // windows above 1024 tokens
    if (e >= nh - h) mark(a.hist[a.n_hist - nh + e]);
  __syncthreads();
}

// The penalty of a windowed token: x / theta above zero (as x times the
// reciprocal 1 / theta rounded once, on the host), x * theta otherwise.
__device__ __forceinline__ float penalty(float x, const SampleArgs& a) {
  return x > 0.0f ? x * a.inv_theta : x * a.theta;
}

__device__ __forceinline__ float penalised(float x, const uint32_t* bits, int rel, const SampleArgs& a) {
  return ((bits[rel >> 5] >> (rel & 31)) & 1u) ? penalty(x, a) : x;
}

// Token of element e of a lane in the sub-slice starting at `base`: groups of
// 16 bytes, consecutive lanes on consecutive groups.
template <typename Tin>
__device__ __forceinline__ int token_of(int base, int e, int lane) {
  constexpr int kPer = 16 / sizeof(Tin);
  return base + ((e / kPer) * kWave + lane) * kPer + (e % kPer);
}

// A lane's 16 logits of a sub-slice. Rows that are whole 16-byte groups from
// a 16-byte-aligned base (the host checks) take 16-byte loads, issued back to
// back with no branch around them (a group past V is clamped onto the row's
// last group and masked afterwards); they stay raw in registers until used.
// Other rows take element loads when the values are formed.
template <typename Tin>
struct SubRaw {
  static constexpr int kPer = 16 / sizeof(Tin);
  static constexpr int kG = kPL / kPer;
  uint4 u[kG];
};

template <typename Tin, bool kVec>
__device__ __forceinline__ void fetch_sub(const Tin* row, int base, int V, int lane, SubRaw<Tin>& w) {
  if constexpr (kVec) {
    constexpr int kPer = SubRaw<Tin>::kPer;
#pragma unroll
    for (int g = 0; g < SubRaw<Tin>::kG; ++g) {
      const int t0 = min(token_of<Tin>(base, g * kPer, lane), V - kPer);
      w.u[g] = *reinterpret_cast<const uint4*>(row + t0);
    }
  }
}

// The lane's penalised logits z of the sub-slice at `base` (-inf past V; a
// sub-slice wholly inside the row skips that test), with window bit t - i0 of
// `bits` (LDS or global) for token t. A group's kPer tokens start at a
// multiple of kPer from the 1024-aligned i0, so one word holds all their bits.
template <typename Tin, bool kVec, bool kFull>
__device__ __forceinline__ void sub_values(const Tin* row, int base, int i0, const SampleArgs& a, int lane,
                                           SubRaw<Tin>& w, const uint32_t* bitmap, float (&z)[kPL]) {
  constexpr int kPer = SubRaw<Tin>::kPer;
#pragma unroll
  for (int g = 0; g < SubRaw<Tin>::kG; ++g) {
    const int t0 = token_of<Tin>(base, g * kPer, lane);
    const uint32_t bits = bitmap[(t0 - i0) >> 5] >> ((t0 - i0) & 31);
    Tin e[kPer];
    if constexpr (kVec) {
      // the unpacking stays here: otherwise it is hoisted next to the loads,
      // whose wait would then precede the work meant to hide them
      asm volatile("" : "+v"(w.u[g].x), "+v"(w.u[g].y), "+v"(w.u[g].z), "+v"(w.u[g].w));
      __builtin_memcpy(e, &w.u[g], 16);
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const bool in = kFull || t0 + q < a.V;
      float x;
      if constexpr (kVec) x = Elem<Tin>::load(&e[q]);
      else x = in ? Elem<Tin>::load(row + t0 + q) : 0.0f;
      // the factor by bit selects, no compares: the sign picks theta or
      // 1 / theta (x = +-0 gives +-0 either way), the window bit picks it or 1
      const uint32_t sgn = (uint32_t)(__float_as_int(x) >> 31);
      const uint32_t f = (sgn & __float_as_uint(a.theta)) | (~sgn & __float_as_uint(a.inv_theta));
      const uint32_t w_q = (uint32_t)((int)(bits << (31 - q)) >> 31);
      x *= __uint_as_float((w_q & f) | (~w_q & 0x3f800000u));
      z[g * kPer + q] = in ? x : -INFINITY;
    }
  }
}

// All-lane reductions of a wave without LDS traffic: DPP exchanges within
// each row of 16 lanes (pairs, quads, half-row mirror, row mirror), then the
// four row results read out of lanes 0, 16, 32 and 48.
template <int kCtrl, typename T>
__device__ __forceinline__ T dpp(T x) {
  return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}
template <typename T>
__device__ __forceinline__ T readlane(T x, int l) {
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_all(T v, Op op) {
  v = op(v, dpp<0xB1>(v));                  // quad_perm [1,0,3,2]
  v = op(v, dpp<0x4E>(v));                  // quad_perm [2,3,0,1]
  v = op(v, dpp<0x141>(v));                 // row_half_mirror
  v = op(v, dpp<0x140>(v));                 // row_mirror
  return op(op(readlane(v, 0), readlane(v, 16)), op(readlane(v, 32), readlane(v, 48)));
}
__device__ __forceinline__ float wave_all_max(float v) { return wave_all(v, [](float x, float y) { return fmaxf(x, y); }); }
__device__ __forceinline__ float wave_all_sum(float v) { return wave_all(v, [](float x, float y) { return x + y; }); }

// Summary of sub-slice b (at `base`) by one wave: m, the kept weight relative
// to m at the cut m + cut, the count n, and the kept tokens when n <= 32.
template <typename Tin, bool kVec, bool kFull, typename L>
__device__ __forceinline__ void summarise(const SampleArgs& a, const Tin* row, int r, int b, int i0, int lane,
                                          SubRaw<Tin>& raw, const L& s) {
  const int base = b * kSampleSub;
  float z[kPL];
  sub_values<Tin, kVec, kFull>(row, base, i0, a, lane, raw, s.bits, z);
  float m = z[0];
#pragma unroll
  for (int e = 1; e < kPL; ++e) m = fmaxf(m, z[e]);
  m = wave_all_max(m);
  // kept: z >= m + cut, never -inf (the floor -FLT_MAX stands in for cut = -inf)
  const float thr = fmaxf(m + a.cut, -FLT_MAX);
  uint64_t kept[kPL];
  int n = 0;
#pragma unroll
  for (int e = 0; e < kPL; ++e) {
    kept[e] = __builtin_amdgcn_ballot_w64(z[e] >= thr);
    n += __popcll(kept[e]);
  }
  float acc = 0.0f;
  if (n <= kSampleList) {
    // few kept: their weights, and the tokens in (element, lane) order, the
    // slot being the ballot's count below this lane
    SampleCand* list = a.cand + ((int64_t)r * a.nb + b) * kSampleList;
    int off = 0;
#pragma unroll
    for (int e = 0; e < kPL; ++e) {
      const uint64_t k_e = kept[e];
      if (k_e == 0) continue;                   // a scalar test: no lane kept element e
      if ((k_e >> lane) & 1u) {
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(k_e >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)k_e, 0u));
        acc += __builtin_amdgcn_exp2f((z[e] - m) * a.s2);
        list[off + pos] = SampleCand{z[e], token_of<Tin>(base, e, lane)};
      }
      off += __popcll(k_e);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPL; ++e)
      acc += z[e] >= thr ? __builtin_amdgcn_exp2f((z[e] - m) * a.s2) : 0.0f;
  }
  acc = wave_all_sum(acc);
  // top-p needs the weight of every finite token; without min-p that is acc
  float wall = acc;
  if (a.topp_cut != nullptr && a.cut > -INFINITY) {
    wall = 0.0f;
#pragma unroll
    for (int e = 0; e < kPL; ++e)
      wall += z[e] > -INFINITY ? __builtin_amdgcn_exp2f((z[e] - m) * a.s2) : 0.0f;
    wall = wave_all_sum(wall);
  }
  if (lane == 0) a.sub[r * a.nb + b] = SampleSub{m, acc, n, wall};
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

template <typename Tin, int kNT, int kPW, bool kVec>
__global__ __launch_bounds__(kNT) void sample_scan_kernel(SampleArgs a) {
  constexpr int kW = kNT / kWave;
  static_assert(kW * kPW <= kMaxScanSubs, "sub-slices a workgroup");
  __shared__ Lds<kW * kPW * kSampleSub / 32> s;
  const int r = blockIdx.y, lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int b0 = blockIdx.x * (kW * kPW), b1 = min(a.nb, b0 + kW * kPW);
  const int i0 = b0 * kSampleSub, i1 = min(a.V, b1 * kSampleSub);
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  // wave w owns sub-slices b0 + w + kW k; the window's few loads go first,
  // then every logits load of the wave (a sub-slice past the row's last one
  // reloads it); the bitmap is built while the logits are in flight
  WindowRegs<kNT> wr;
  window_prefetch<kNT>(a, r, wr);
  SubRaw<Tin> raw[kPW];
#pragma unroll
  for (int k = 0; k < kPW; ++k)
    fetch_sub<Tin, kVec>(row, min(b0 + wave + kW * k, b1 - 1) * kSampleSub, a.V, lane, raw[k]);
  const int nw = (b1 - b0) * (kSampleSub / 32);
  mark_window<kNT>(a, r, i0, i1, nw, s, wr);
  // the bitmap also goes to the workspace, for the picking kernel's rereads
  for (int k = threadIdx.x; k < nw; k += kNT) a.wbits[((int64_t)r * a.nb + b0) * (kSampleSub / 32) + k] = s.bits[k];
#pragma unroll
  for (int k = 0; k < kPW; ++k) {
    const int b = b0 + wave + kW * k;
    if (b >= b1) break;
    if ((b + 1) * kSampleSub <= a.V)
      summarise<Tin, kVec, true>(a, row, r, b, i0, lane, raw[k], s);
    else
      summarise<Tin, kVec, false>(a, row, r, b, i0, lane, raw[k], s);
  }
}

// Sums of the kept weights of kU sub-slices b[u] at the row's cut thr
// (relative to the row maximum Z), from their logits and stored window bits;
// one wave, every load issued before the first sum.
template <typename Tin, bool kVec, int kU>
__device__ void reread_weights(const SampleArgs& a, int r, const int (&b)[kU], float Z, float thr, int lane,
                               float (&w)[kU]) {
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  SubRaw<Tin> raw[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) fetch_sub<Tin, kVec>(row, b[u] * kSampleSub, a.V, lane, raw[u]);
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int base = b[u] * kSampleSub;
    const uint32_t* bits = a.wbits + ((int64_t)r * a.nb + b[u]) * (kSampleSub / 32);
    float z[kPL];
    if (base + kSampleSub <= a.V)
      sub_values<Tin, kVec, true>(row, base, base, a, lane, raw[u], bits, z);
    else
      sub_values<Tin, kVec, false>(row, base, base, a, lane, raw[u], bits, z);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < kPL; ++e)
      if (z[e] > -INFINITY && z[e] >= thr) acc += exp2f((z[e] - Z) * a.s2);
    w[u] = wave_all_sum(acc);
  }
}

template <typename Tin, bool kVec>
__global__ __launch_bounds__(kThreads) void sample_pick_kernel(SampleArgs a) {
  __shared__ BlockRed s;
  __shared__ PickLds p;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const bool greedy = a.s2 == 0.0f;
  // thread tid owns sub-slices [q0, q0 + per), in row order
  const int per = (a.nb + kThreads - 1) / kThreads;
  const int q0 = tid * per;
  SampleSub sb[kPerT];
  float mloc = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPerT; ++k) {
    sb[k] = SampleSub{-INFINITY, 0.0f, 0, 0.0f};
    if (k < per && q0 + k < a.nb) sb[k] = a.sub[r * a.nb + q0 + k];
    mloc = fmaxf(mloc, sb[k].m);
  }
  const float Z = block_max(mloc, s.red);
  // the row's cut: min-p, raised to the row's top-p cut z* when top-p is on
  const float thr = fmaxf(Z + a.cut, a.topp_cut != nullptr && !greedy ? a.topp_cut[r] : -INFINITY);
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
#pragma unroll
    for (int k = 0; k < kPerT; ++k)
      if (k < per && q0 + k < a.nb && sb[k].m == Z) {
        atomicMin(&p.bsel, q0 + k);
        break;
      }
    __syncthreads();
  } else {
    // each sub-slice's weight at the row's cut (relative to Z)
#pragma unroll
    for (int k = 0; k < kPerT; ++k) {
      if (k >= per) break;
      const int q = q0 + k;
      float c = 0.0f;
      if (q < a.nb && sb[k].m > -INFINITY && sb[k].m >= thr) {
        if (thr == -INFINITY) {
          c = sb[k].s * exp2f((sb[k].m - Z) * a.s2);
        } else if (sb[k].n <= kSampleList) {
          const SampleCand* list = a.cand + ((int64_t)r * a.nb + q) * kSampleList;
          for (int j = 0; j < sb[k].n; ++j) {
            const SampleCand e = list[j];
            if (e.z >= thr) c += exp2f((e.z - Z) * a.s2);
          }
        } else {
          p.ovf[atomicAdd(&p.n_ovf, 1)] = q;
        }
      }
      p.c[q] = c;                               // q < kSampleMaxSubs: per <= kPerT
    }
    __syncthreads();
    // rare: sub-slices with more than 32 kept tokens are read again, one a
    // wave, four at a time (past the end the last one is repeated, unused)
    const int n_ovf = p.n_ovf;
    constexpr int kU = 4;
    for (int k = wave; k < n_ovf; k += kU * kWavesS) {
      int bs[kU];
      float w[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) bs[u] = p.ovf[min(k + u * kWavesS, n_ovf - 1)];
      reread_weights<Tin, kVec, kU>(a, r, bs, Z, thr, lane, w);
      if (lane == 0) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (k + u * kWavesS < n_ovf) p.c[bs[u]] = w[u];
      }
    }
    __syncthreads();
    float c[kPerT];
    float mine = 0.0f;
#pragma unroll
    for (int k = 0; k < kPerT; ++k) {
      c[k] = k < per ? p.c[q0 + k] : 0.0f;
      mine += c[k];
    }
    float total;
    const float excl = block_excl_scan<float>(mine, s.red, total);
    target = a.u[r] * total;
    // the first sub-slice whose cumulative weight passes the target
    float run = excl;
#pragma unroll
    for (int k = 0; k < kPerT; ++k) {
      if (c[k] > 0.0f && run + c[k] > target) {
        atomicMin(&p.bsel, q0 + k);
        break;
      }
      run += c[k];
    }
    __syncthreads();
    const int bs = p.bsel;
    if (bs == a.nb) {                           // u * total at or past the end: the last kept token
      fallback = true;
      __syncthreads();
#pragma unroll
      for (int k = kPerT - 1; k >= 0; --k)
        if (c[k] > 0.0f) {
          atomicMax(&p.last, q0 + k);
          break;
        }
      __syncthreads();
      if (tid == 0) {
        p.bsel = p.last;
        p.last = -1;
      }
    } else if (bs >= q0 && bs < q0 + per) {
      float pre = excl;
#pragma unroll
      for (int k = 0; k < kPerT; ++k) pre += k < bs - q0 ? c[k] : 0.0f;
      p.base = pre;
    }
    __syncthreads();
  }
  const int b = p.bsel;
  if (b < 0 || b >= a.nb) {                     // no finite logit in the row (outside the contract)
    if (tid == 0) a.tok[r] = -1;
    return;
  }
  const SampleSub chosen = a.sub[r * a.nb + b];
  const bool listed = chosen.n <= kSampleList && (greedy || thr > -INFINITY);
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
  const uint32_t* bits = a.wbits + ((int64_t)r * a.nb + b) * (kSampleSub / 32);
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  const int c0 = min(end, base + tid * kPT), c1 = min(end, c0 + kPT);
  float w[kPT];
  float mine = 0.0f;
#pragma unroll
  for (int j = 0; j < kPT; ++j) {
    w[j] = 0.0f;
    if (c0 + j < c1) {
      const float z = penalised(Elem<Tin>::load(row + c0 + j), bits, c0 + j - base, a);
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

// ---------------------------------------------------------------------------
// Top-p cut of each row: a weighted radix select over the row's penalised
// logits z, from the largest down, for the value z* at which the weight at or
// above it first reaches top_p * W (W: the row's total weight, from the
// scan's summaries). Pass 0 bins z by its weight, 1/8 of a power of two per
// bin below the row maximum (bin 255 takes everything further down), which
// spreads a row's tokens over the bins; passes 1..4 take the 8-bit digits of
// the order-preserving key of z inside the chosen bin, high to low. Each pass
// sums per bin the weight, the count and the smallest and largest key, and
// the search ends as soon as the chosen bin holds a single key. The weights
// are summed in fp32 in an unspecified order, so a z* whose cumulative weight
// is within rounding of top_p * W may come out one value either side.
constexpr int kToppThreads = 1024;

__device__ __forceinline__ uint32_t topp_key(float f) {
  if (f == 0.0f) f = 0.0f;               // -0 and +0: one key
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float topp_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <typename Tin>
__global__ __launch_bounds__(kToppThreads) void sample_topp_kernel(SampleArgs a) {
  constexpr int kW = kToppThreads / kWave;
  __shared__ float hw[256];
  __shared__ uint32_t hc[256], kmin[256], kmax[256];
  __shared__ float red[kW];
  __shared__ float s_m;                  // weight above the chosen bin
  __shared__ int s_sel;                  // chosen bin of the pass
  __shared__ uint32_t s_key;             // z*'s key once known
  __shared__ int s_done;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  const uint32_t* bits = a.wbits + (int64_t)r * a.nb * (kSampleSub / 32);

  // the row maximum and total weight from the sub-slice summaries (nb <= 1024)
  SampleSub sb = SampleSub{-INFINITY, 0.0f, 0, 0.0f};
  if (tid < a.nb) sb = a.sub[(int64_t)r * a.nb + tid];
  float v = wave_max(sb.m);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float Z = red[0];
#pragma unroll
  for (int w = 1; w < kW; ++w) Z = fmaxf(Z, red[w]);
  __syncthreads();
  v = wave_sum(sb.m > -INFINITY ? sb.wall * exp2f((sb.m - Z) * a.s2) : 0.0f);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float W = 0.0f;
#pragma unroll
  for (int w = 0; w < kW; ++w) W += red[w];
  const float target = a.top_p * W;
  if (tid == 0) {
    s_m = 0.0f;
    s_done = 0;
    s_key = 0u;
  }

  // pass 0: weight bins; passes 1..4: key digits inside bin b0
  int b0 = -1;
  uint32_t prefix = 0u, mask = 0u;
  for (int pass = 0; pass < 5; ++pass) {
    const int shift = 32 - 8 * pass;       // pass >= 1: digit (key >> shift) & 255
    if (tid < 256) {
      hw[tid] = 0.0f;
      hc[tid] = 0u;
      kmin[tid] = 0xFFFFFFFFu;
      kmax[tid] = 0u;
    }
    __syncthreads();
    for (int t = tid; t < a.V; t += kToppThreads) {
      float z = Elem<Tin>::load(row + t);
      if ((bits[t >> 5] >> (t & 31)) & 1u) z = penalty(z, a);
      if (!(z > -INFINITY)) continue;
      const int bin = (int)fminf((Z - z) * a.s2 * 8.0f, 255.0f);
      const uint32_t key = topp_key(z);
      int d;
      if (pass == 0) d = bin;
      else if (bin == b0 && (key & mask) == prefix) d = (int)((key >> shift) & 255u);
      else continue;
      atomicAdd(&hw[d], exp2f((z - Z) * a.s2));
      atomicAdd(&hc[d], 1u);
      atomicMin(&kmin[d], key);
      atomicMax(&kmax[d], key);
    }
    __syncthreads();
    if (wave == 0) {
      // bins in order of decreasing z: pass 0 ascending, key digits descending
      float c[4], tot = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = pass == 0 ? 4 * lane + j : 255 - 4 * lane - j;
        c[j] = hw[d];
        tot += c[j];
      }
      float incl = tot;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const float y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
      }
      float run = s_m + incl - tot;      // weight above this lane's first bin
      int sel = -1;
      float above = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = pass == 0 ? 4 * lane + j : 255 - 4 * lane - j;
        if (sel < 0 && hc[d] > 0u && run + c[j] >= target) {
          sel = d;
          above = run;
        }
        run += c[j];
      }
      // the first bin (in z order) that reaches the target; rounding can leave
      // the target past the total, and then the last non-empty bin is taken
      const uint64_t hit = __ballot(sel >= 0);
      int last = -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = pass == 0 ? 4 * lane + j : 255 - 4 * lane - j;
        if (hc[d] > 0u) last = d;
      }
      const uint64_t any = __ballot(last >= 0);
      if (hit != 0ull) {
        const int src = __ffsll((unsigned long long)hit) - 1;
        if (lane == src) {
          s_sel = sel;
          s_m = above;
        }
      } else if (any != 0ull) {
        const int src = 63 - __clzll((unsigned long long)any);
        if (lane == src) {
          // everything up to this bin lies above it
          float up = s_m + incl - tot;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = pass == 0 ? 4 * lane + j : 255 - 4 * lane - j;
            if (d == last) break;
            up += c[j];
          }
          s_sel = last;
          s_m = up;
        }
      } else if (lane == 0) {
        s_sel = -1;                      // no finite token (outside the contract)
      }
    }
    __syncthreads();
    const int sel = s_sel;
    if (sel < 0) {
      if (tid == 0) a.topp_cut[r] = -INFINITY;
      return;
    }
    if (kmin[sel] == kmax[sel] || pass == 4) {
      if (tid == 0) a.topp_cut[r] = topp_value(kmax[sel]);
      return;
    }
    if (pass == 0) {
      b0 = sel;
    } else {
      prefix |= (uint32_t)sel << shift;
      mask |= 255u << shift;
    }
    __syncthreads();                       // every thread has read this pass's bins
  }
}

template <typename Tin>
hipError_t launch_t(const SampleArgs& a, hipStream_t st) {
  // 256 threads, one sub-slice a wave: of 256/512/1024 threads and 1/2/4
  // sub-slices a wave, the fastest or within 2% of it for fp32 and bf16
  constexpr int kNT = 256, kPW = 1;
  constexpr int kSubs = kNT / kWave * kPW;
  const dim3 grid((a.nb + kSubs - 1) / kSubs, a.R);
  constexpr int kPer = 16 / sizeof(Tin);
  // 16-byte loads when every row is whole 16-byte groups from an aligned base
  const bool vec = (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0 && a.V % kPer == 0;
  if (vec)
    sample_scan_kernel<Tin, kNT, kPW, true><<<grid, kNT, 0, st>>>(a);
  else
    sample_scan_kernel<Tin, kNT, kPW, false><<<grid, kNT, 0, st>>>(a);
  if (a.topp_cut != nullptr) sample_topp_kernel<Tin><<<a.R, kToppThreads, 0, st>>>(a);
  if (vec)
    sample_pick_kernel<Tin, true><<<a.R, kThreads, 0, st>>>(a);
  else
    sample_pick_kernel<Tin, false><<<a.R, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

int sample_subslices(int V) { return V < 1 ? 1 : (V + kSampleSub - 1) / kSampleSub; }

size_t sample_workspace_bytes(int R, int V) {
  const size_t n = (size_t)R * sample_subslices(V);
  return n * sizeof(SampleSub) + n * kSampleList * sizeof(SampleCand) + n * (kSampleSub / 32) * sizeof(uint32_t) +
         (size_t)R * sizeof(float);
}

hipError_t launch_sample(const SampleArgs& a, ts_dtype dtype, hipStream_t s) {
  static_assert(kThreads * kPerT == kSampleMaxSubs, "a picking thread holds up to kPerT sub-slices");
  static_assert(kSampleList <= kThreads, "list entries are ranked one per thread");
  return dtype == TS_BF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace ts
