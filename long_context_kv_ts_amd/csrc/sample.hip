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
// Rows are cut into sub-slices of 1024 logits. Without top-p, two launches
// and one read of the logits (a second only for sub-slices that keep many
// tokens under min-p):
//   A. grid (workgroups per row, rows), kNT threads, kPW sub-slices a wave: a
//      workgroup issues the window's few loads, then every logits load of its
//      waves (16 logits a lane per sub-slice, held raw in registers), and
//      marks the windowed tokens of its range in an LDS bitmap while they land
//      (its only barriers); the bitmap is also stored, 32 words a sub-slice.
//      Each wave then summarises its own sub-slices with DPP reductions and
//      ballots: the maximum m, the kept weight relative to m at the
//      sub-slice's own cut m + cut, and the kept tokens themselves while there
//      are at most 32 (weights and list entries only for those).
//   (top-p rows: the scan also bins each sub-slice's weight into 32 coarse
//   bins on a fixed lattice of levels, powers of two of weight)
//   C. (top-p only) grid (rows): the bin totals in a fixed order, the bin where
//      the cumulative weight crosses top_p * W, and each sub-slice's weight
//      above it;
//   E. (top-p only) grid (workgroups per row, rows): the crossing bin's tokens
//      into a per-row list (sub-slices with no weight in it are not read);
//   T. (top-p only) grid (rows): z* by key passes over that list, the kept
//      weight of every sub-slice and the draw, in place of B;
//   B. grid (rows): the row maximum Z gives the row's cut Z + cut >= m + cut,
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

template <int kWords, int kBinWaves = 0>
struct Lds {
  uint32_t bits[kWords];                    // windowed tokens of [i0, i1)
  // the window's forest and path are dead once the bitmap is built (a barrier
  // ends the marking), so top-p rows' coarse bins reuse their space
  union {
    struct {
      int par[TS_MAX_DRAFT], dtok[TS_MAX_DRAFT];
      int path[TS_MAX_DRAFT];               // draft tokens on the root path, leaf first
      int path_len;
    };
    float bins[kBinWaves][kWave][kToppCoarseBins + 1];   // top-p: each lane's coarse bins (padded row)
  };
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

// Top-p coarse bins lie on a fixed lattice: token z is on level floor(-z s2)
// (clamped to +-2^29, so that differences fit an int), and its bin below a
// maximum on level l is min(level - l, 31) -- whole powers of two of weight,
// the last bin taking everything further down. A sub-slice bins its tokens
// below its own maximum; since levels are absolute, shifting its bins by the
// level difference to the row maximum gives exactly the row's binning.
__device__ __forceinline__ int topp_level(float z, float s2) {
  return (int)floorf(fminf(fmaxf(-z * s2, -536870912.0f), 536870912.0f));
}
__device__ __forceinline__ int topp_bin(float z, int top_level, float s2) {
  return min(topp_level(z, s2) - top_level, kToppCoarseBins - 1);
}

// Summary of sub-slice b (at `base`) by one wave: m, the kept weight relative
// to m at the cut m + cut, the count n, and the kept tokens when n <= 32.
// Top-p rows instead: m, the weight of every finite token relative to m, and
// the sub-slice's coarse bins (each lane adds its tokens' weights into its own
// LDS row; the wave adds the columns in a fixed order).
template <typename Tin, bool kVec, bool kFull, bool kTopp, typename L>
__device__ __forceinline__ void summarise(const SampleArgs& a, const Tin* row, int r, int b, int i0, int lane,
                                          SubRaw<Tin>& raw, L& s) {
  const int base = b * kSampleSub;
  float z[kPL];
  sub_values<Tin, kVec, kFull>(row, base, i0, a, lane, raw, s.bits, z);
  float m = z[0];
#pragma unroll
  for (int e = 1; e < kPL; ++e) m = fmaxf(m, z[e]);
  m = wave_all_max(m);
  if constexpr (kTopp) {
    float* mine = s.bins[threadIdx.x >> 6][lane];
#pragma unroll
    for (int c = 0; c < kToppCoarseBins; ++c) mine[c] = 0.0f;
    float wall = 0.0f;
    if (m > -INFINITY) {
      const int lm = topp_level(m, a.s2);
#pragma unroll
      for (int e = 0; e < kPL; ++e) {
        // no branch: -inf adds 0 to bin 0, which changes nothing
        const bool fin = z[e] > -INFINITY;
        const float w = fin ? __builtin_amdgcn_exp2f((z[e] - m) * a.s2) : 0.0f;
        wall += w;
        mine[fin ? topp_bin(z[e], lm, a.s2) : 0] += w;
      }
    }
    wall = wave_all_sum(wall);
    // the wave's own rows only: its LDS operations complete in order
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // column c = lane % 32 over rows 32h .. 32h + 31 (h = lane / 32), then the halves
    const int c = lane & (kToppCoarseBins - 1), h = lane >> 5;
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) t += s.bins[threadIdx.x >> 6][32 * h + j][c];
    t += __shfl_xor(t, 32, kWave);
    if (lane < kToppCoarseBins) a.topp_hist[((int64_t)r * a.nb + b) * kToppCoarseBins + lane] = t;
    if (lane == 0) a.sub[r * a.nb + b] = SampleSub{m, 0.0f, 0, wall};
    return;
  }
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
  const T incl = wave_incl_scan(v);
  const T excl = incl - v;
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

// (top-p: at most 128 VGPRs, so that four workgroups of 256 fit a CU, as their LDS does)
template <typename Tin, int kNT, int kPW, bool kVec, bool kTopp>
__global__ __launch_bounds__(kNT, kTopp ? 4 : 1) void sample_scan_kernel(SampleArgs a) {
  constexpr int kW = kNT / kWave;
  static_assert(kW * kPW <= kMaxScanSubs, "sub-slices a workgroup");
  __shared__ Lds<kW * kPW * kSampleSub / 32, kTopp ? kW : 0> s;
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
      summarise<Tin, kVec, true, kTopp>(a, row, r, b, i0, lane, raw[k], s);
    else
      summarise<Tin, kVec, false, kTopp>(a, row, r, b, i0, lane, raw[k], s);
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
        if (a.cut == -INFINITY) {
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
// Top-p rows (top_p < 1, tau > 0): three launches after the scan find each
// row's cut and draw the token, in place of the pick kernel.
//   * Z and the total weight W = sum 2^((z - Z) s2) come from the scan's
//     sub-slice summaries.
//   * The cut z* -- the value at which the weight at or above it first
//     reaches top_p * W -- by a weighted select from the largest z down.
//     The coarse step is spread over the grid: the scan bins every
//     sub-slice's weight into 32 bins, a power of two of weight each (on a
//     fixed lattice, so that sub-slice bins shift exactly into the row's; the
//     last bin takes everything further down). One workgroup a row adds
//     them up and finds the bin where the cumulative weight crosses
//     top_p * W, which is usually narrow; its tokens' keys and ids go to a
//     per-row list, again over the grid. Key passes over the list (in LDS)
//     cut its key range into 2048 sub-ranges until one key is left. A bin
//     with more tokens than the list holds (nearly flat logits) runs the key
//     passes over the row instead.
//   * The row's cut is the larger of z* and the min-p cut. The kept weight of
//     every 1024-logit sub-slice: when the cut is z* and the crossing bin's
//     tokens are all listed, its bins above the crossing one plus its listed
//     tokens at or above z*; else a pass over the row (four waves a
//     sub-slice, added in a fixed order). A scan finds the sub-slice the draw
//     u * (kept weight) falls in, and a scan over its 1024 tokens the token.
// Every pass over the row loads a thread's next eight 4-token groups before
// using any (a group past the row reloads the last one and is masked). The
// list's order follows the order in which its slot reservations land, but
// the key passes and the kept weights add the crossing bin's weights as
// integers, so the cut and the draw do not depend on it. All other sums run
// in a fixed order: every call gives the same tokens.
constexpr int kToppThreads = 1024;
constexpr int kToppWaves = kToppThreads / kWave;
constexpr int kToppBins = 2048;           // key-pass bins
constexpr int kToppCoarse = kToppCoarseBins;   // pass-0 bins: powers of two of weight
constexpr int kToppCand = kToppCandMax;   // keys (and token ids) of the crossing bin held in LDS
constexpr int kToppBatch = 8;             // 4-token groups a thread loads at once

__device__ __forceinline__ uint32_t topp_key(float f) {
  if (f == 0.0f) f = 0.0f;               // -0 and +0: one key
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float topp_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exclusive prefix over the workgroup's threads in index order; total = the sum.
__device__ float topp_scan(float v, float* red, float& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const float incl = wave_incl_scan(v);
  const float excl = incl - v;
  if (lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  float off = 0.0f, tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kToppWaves; ++w) {
    off += w < wave ? red[w] : 0.0f;
    tot += red[w];
  }
  __syncthreads();
  total = tot;
  return off + excl;
}

// Raw loads of a 4-token group from token t0 (a multiple of 4, t0 < V): one
// 16-byte (fp32) or 8-byte (bf16) load when the rows allow it, else four
// element loads clamped into the row; plus the group's window-bit word.
template <typename Tin, bool kVec>
struct ToppRaw {
  uint4 u;                               // fp32 bits, or bf16 pairs in x and y
  uint32_t w;
};
template <typename Tin, bool kVec>
__device__ __forceinline__ void topp_fetch(int V, const Tin* row, const uint32_t* bits, int t0, ToppRaw<Tin, kVec>& r) {
  if constexpr (kVec) {
    if constexpr (sizeof(Tin) == 4) {
      r.u = *reinterpret_cast<const uint4*>(row + t0);
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(row + t0);
      r.u = make_uint4(v.x, v.y, 0u, 0u);
    }
  } else {
    uint32_t e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Tin x = row[min(t0 + i, V - 1)];
      if constexpr (sizeof(Tin) == 4) e[i] = __builtin_bit_cast(uint32_t, x);
      else e[i] = (uint32_t)x << 16;
    }
    r.u = make_uint4(e[0], e[1], e[2], e[3]);
  }
  r.w = bits[t0 >> 5] >> (t0 & 31);
}
// The group's penalised logits (selects from the two factors held in
// registers, no branch); -inf past V or when `valid` is false.
template <typename Tin, bool kVec>
__device__ __forceinline__ void topp_values(int V, float theta, float inv_theta, int t0, bool valid,
                                            const ToppRaw<Tin, kVec>& r, float (&z)[4]) {
  float x[4];
  if constexpr (kVec && sizeof(Tin) == 2) {
    x[0] = __uint_as_float(r.u.x << 16); x[1] = __uint_as_float(r.u.x & 0xffff0000u);
    x[2] = __uint_as_float(r.u.y << 16); x[3] = __uint_as_float(r.u.y & 0xffff0000u);
  } else {
    x[0] = __uint_as_float(r.u.x); x[1] = __uint_as_float(r.u.y);
    x[2] = __uint_as_float(r.u.z); x[3] = __uint_as_float(r.u.w);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = x[i] * (x[i] > 0.0f ? inv_theta : theta);
    const float v = ((r.w >> i) & 1u) ? p : x[i];
    z[i] = valid && t0 + i < V ? v : -INFINITY;
  }
}

// f(k, z) for every 4-token group g = threadIdx.x + k * kToppThreads of the row
// (z = -inf past the row); the loop is uniform across the workgroup. Every
// load of a batch is issued before the first is used (a group past the row
// reloads the last one).
template <typename Tin, bool kVec, typename F>
__device__ __forceinline__ void topp_visit(int V, float theta, float inv_theta, const Tin* row, const uint32_t* bits,
                                           int ngroups, F&& f) {
  for (int k0 = 0; k0 * kToppThreads < ngroups; k0 += kToppBatch) {
    ToppRaw<Tin, kVec> raw[kToppBatch];
#pragma unroll
    for (int j = 0; j < kToppBatch; ++j) {
      const int g = threadIdx.x + (k0 + j) * kToppThreads;
      topp_fetch<Tin, kVec>(V, row, bits, 4 * min(g, ngroups - 1), raw[j]);
    }
#pragma unroll
    for (int j = 0; j < kToppBatch; ++j) {
      const int g = threadIdx.x + (k0 + j) * kToppThreads;
      float z[4];
      topp_values<Tin, kVec>(V, theta, inv_theta, 4 * g, g < ngroups, raw[j], z);
      f(k0 + j, z);
    }
  }
}

struct ToppLds {
  unsigned long long hw[kToppBins];      // key passes: weight per bin, fixed point
  uint32_t kmn[kToppBins], kmx[kToppBins];   // smallest and largest key per bin (none: ~0 and 0)
  uint32_t cand[kToppCand];              // keys of the crossing bin
  int32_t cid[kToppCand];                // and their token ids
  float part[4 * kSampleMaxSubs];        // kept weight of each sub-slice, in four parts
  unsigned long long partq[kSampleMaxSubs];   // its listed tokens' share, fixed point
  int32_t qlist[kSampleMaxSubs];         // sub-slices whose maximum reaches a binding min-p cut
  int nq;
  float red[kToppWaves];
  float above;                           // weight above the current range
  uint32_t lo, hi;                       // the crossing bin's key range
  int sel, last;
  int win, lastk;
};

// Among the 2048 key bins (in order of decreasing z), the first whose
// cumulative weight (after s.above) reaches `target`, else the last non-empty
// one; sets s.above to the weight before it and returns it.
__device__ int topp_select(ToppLds& s, float target, float inv_fx) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    s.sel = INT32_MAX;
    s.last = -1;
  }
  const float above0 = s.above;
  const int b0 = 2 * tid, b1 = 2 * tid + 1;
  const float c0 = (float)s.hw[b0] * inv_fx, c1 = (float)s.hw[b1] * inv_fx;
  // a bin holds tokens iff its smallest key is set (every token of the
  // crossing coarse bin has a positive weight: they are within a factor 2)
  const bool n0 = s.kmn[b0] != 0xFFFFFFFFu, n1 = s.kmn[b1] != 0xFFFFFFFFu;
  float tot;
  const float run = above0 + topp_scan(c0 + c1, s.red, tot);   // its barriers order the init above
  float my_above = 0.0f;
  int my_sel = INT32_MAX;
  if (n0 && run + c0 >= target) {
    my_sel = b0;
    my_above = run;
  } else if (n1 && run + c0 + c1 >= target) {
    my_sel = b1;
    my_above = run + c0;
  }
  if (my_sel != INT32_MAX) atomicMin(&s.sel, my_sel);
  const int my_last = n1 ? b1 : n0 ? b0 : -1;
  if (my_last >= 0) atomicMax(&s.last, my_last);
  __syncthreads();
  const bool hit = s.sel != INT32_MAX;
  const int sel = hit ? s.sel : s.last;
  __syncthreads();
  if (sel >= 0 && (sel == b0 || sel == b1)) s.above = hit ? my_above : (sel == b0 ? run : run + c0);
  __syncthreads();
  return sel;
}

__device__ __forceinline__ void topp_clear_keys(ToppLds& s) {
  for (int b = threadIdx.x; b < kToppBins; b += kToppThreads) {
    s.hw[b] = 0ull;
    s.kmn[b] = 0xFFFFFFFFu;
    s.kmx[b] = 0u;
  }
}

// Weights of the crossing bin's tokens are added as 64-bit integers, each
// the fp32 weight times fx = 2^(bc + 41): a token of coarse bin bc weighs
// less than 2^(1 - bc) (at most 1 in bin 0), so each term is below 2^42 and a
// row's sum below 2^62. Integer sums do not depend on the order in which the
// atomics land, so the cut and the draw are the same on every call.
__device__ __forceinline__ unsigned long long topp_fixed(float w, float fx) {
  return (unsigned long long)(w * fx);
}

// One key pass: the tokens with keys in [lo, hi] into bins of (key - lo) >> shift,
// in order of decreasing key.
__device__ __forceinline__ void topp_key_bin(ToppLds& s, uint32_t key, float Z, float s2, uint32_t lo, uint32_t hi,
                                             int shift, float fx) {
  if (key < lo || key > hi) return;
  const int b = kToppBins - 1 - (int)((key - lo) >> shift);
  atomicAdd(&s.hw[b], topp_fixed(__builtin_amdgcn_exp2f((topp_value(key) - Z) * s2), fx));
  atomicMin(&s.kmn[b], key);
  atomicMax(&s.kmx[b], key);
}

constexpr int kExtractWaves = 4;
// ToppRow::bc of a row whose min-p cut clearly binds: no crossing bin is sought
constexpr int kToppMinpBinds = -2;

// C: one workgroup a row. Z and the total weight W from the sub-slice
// summaries; each sub-slice's bins shifted by its level difference to Z and
// scaled by 2^((m - Z) s2) into the row's bins; the bin totals (each wave adds
// its 64 sub-slices, then the waves in order); the crossing bin bc, the first
// whose cumulative weight reaches top_p * W (else the last non-empty one), and
// the weight above it; each sub-slice's weight in the bins above bc. Also
// resets the row's candidate count for the extract kernel.
// Every token above the min-p cut Z + cut lies in the cut's bin or above it,
// so when those bins hold clearly less than top_p * W (by 2^-10 of it, far
// beyond the sums' rounding), the top-p cut z* lies below the min-p cut and
// the row's cut is the min-p one whatever z* is: bc = kToppMinpBinds, and the
// extract and the key passes are skipped.
__global__ __launch_bounds__(kToppThreads) void sample_topp_coarse_kernel(SampleArgs a) {
  __shared__ float ph[kToppThreads][kToppCoarse + 1];
  __shared__ float coarse[kToppWaves][kToppCoarse];
  __shared__ float red[kToppWaves];
  __shared__ int sel;
  __shared__ float above;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  // this thread's sub-slice: its summary and its bins (below its own maximum)
  SampleSub sb = SampleSub{-INFINITY, 0.0f, 0, 0.0f};
  float hb[kToppCoarse];
  if (tid < a.nb) {
    sb = a.sub[(int64_t)r * a.nb + tid];
    const float4* src = reinterpret_cast<const float4*>(a.topp_hist + ((int64_t)r * a.nb + tid) * kToppCoarse);
#pragma unroll
    for (int q = 0; q < kToppCoarse / 4; ++q) {
      const float4 v = src[q];
      hb[4 * q] = v.x; hb[4 * q + 1] = v.y; hb[4 * q + 2] = v.z; hb[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < kToppCoarse; ++q) hb[q] = 0.0f;
  }
  const float vmax = wave_max(sb.m);
  if (lane == 0) red[wave] = vmax;
  __syncthreads();
  float Z = red[0];
#pragma unroll
  for (int w = 1; w < kToppWaves; ++w) Z = fmaxf(Z, red[w]);
  __syncthreads();
  float W;
  topp_scan(sb.m > -INFINITY ? sb.wall * __builtin_amdgcn_exp2f((sb.m - Z) * a.s2) : 0.0f, red, W);
  ToppRow* row = a.topp_row + r;
  if (!(Z > -INFINITY)) {                // no finite logit in the row (outside the contract)
    if (tid == 0) *row = ToppRow{Z, 0.0f, 0.0f, -1, 0, {}};
    return;
  }
  const float target = a.top_p * W;
  // the bins scaled to Z, kept for the weight above bc; bin j is the row's
  // bin min(j + dl, 31)
  int dl = kToppCoarse;
  const float sc = sb.m > -INFINITY ? __builtin_amdgcn_exp2f((sb.m - Z) * a.s2) : 0.0f;
  if (sb.m > -INFINITY) dl = min(topp_level(sb.m, a.s2) - topp_level(Z, a.s2), kToppCoarse);
#pragma unroll
  for (int q = 0; q < kToppCoarse; ++q) hb[q] *= sc;
  float tail = 0.0f;
#pragma unroll
  for (int c = 0; c < kToppCoarse - 1; ++c)
    if (c < dl) ph[tid][c] = 0.0f;
#pragma unroll
  for (int q = 0; q < kToppCoarse; ++q) {
    if (q + dl < kToppCoarse - 1) ph[tid][q + dl] = hb[q];
    else tail += hb[q];
  }
  ph[tid][kToppCoarse - 1] = tail;
  if (tid == 0) above = 0.0f;
  __syncthreads();
  if (lane < kToppCoarse) {
    float t = 0.0f;
#pragma unroll 16
    for (int j = 0; j < kWave; ++j) t += ph[wave * kWave + j][lane];
    coarse[wave][lane] = t;
  }
  __syncthreads();
  if (wave == 0) {
    float c = 0.0f;
    if (lane < kToppCoarse)
      for (int w = 0; w < kToppWaves; ++w) c += coarse[w][lane];
    const float incl = wave_incl_scan(c);
    const float excl = incl - c;
    const uint64_t hit = __ballot(lane < kToppCoarse && c > 0.0f && incl >= target);
    const uint64_t any = __ballot(lane < kToppCoarse && c > 0.0f);
    const int src = hit ? __ffsll((unsigned long long)hit) - 1 : (any ? 63 - __clzll((unsigned long long)any) : -1);
    // (min-p off: cut = -inf sits in the last bin, whose inclusive sum is W)
    const int bm = topp_bin(Z + a.cut, topp_level(Z, a.s2), a.s2);
    const bool minp = __shfl(incl, bm, kWave) < target * (1.0f - 0x1p-10f);
    if (lane == 0) sel = minp ? kToppMinpBinds : src;
    if (src >= 0 && lane == src) above = excl;
  }
  __syncthreads();
  const int bc = sel;
  if (tid < a.nb) {
    float w = 0.0f;
#pragma unroll
    for (int q = 0; q < kToppCoarse; ++q) w += q + dl < bc ? hb[q] : 0.0f;
    a.topp_above[(int64_t)r * a.nb + tid] = w;
  }
  if (tid == 0) *row = ToppRow{Z, target, above, bc, 0, {}};
}

// E: the tokens of the crossing bin, one sub-slice a wave: their keys and ids
// into the row's candidate list (one slot reservation a wave, ballot-
// compacted; slots past the list's capacity are counted, not stored). A
// sub-slice with no weight in the crossing bin has none of its tokens (a bin
// above the last holds weights of at least 2^-32 of its maximum's) and is
// not read.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kExtractWaves * kWave) void sample_topp_extract_kernel(SampleArgs a) {
  const int r = blockIdx.y, lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int b = blockIdx.x * kExtractWaves + wave;
  ToppRow* row = a.topp_row + r;
  const int bc = row->bc;
  if (b >= a.nb || bc < 0) return;
  const float mb = a.sub[(int64_t)r * a.nb + b].m;
  if (!(mb > -INFINITY)) return;
  const int lz = topp_level(row->Z, a.s2);
  const int dl = topp_level(mb, a.s2) - lz;   // the sub-slice's bin j is the row's min(j + dl, 31)
  if (dl > bc) return;
  if (bc < kToppCoarse - 1 && !(a.topp_hist[((int64_t)r * a.nb + b) * kToppCoarse + (bc - dl)] > 0.0f)) return;
  float z[kPL];
  {
    const Tin* lrow = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
    const int base = b * kSampleSub;
    const uint32_t* bits = a.wbits + ((int64_t)r * a.nb + b) * (kSampleSub / 32);
    SubRaw<Tin> raw;
    fetch_sub<Tin, kVec>(lrow, base, a.V, lane, raw);
    if (base + kSampleSub <= a.V)
      sub_values<Tin, kVec, true>(lrow, base, base, a, lane, raw, bits, z);
    else
      sub_values<Tin, kVec, false>(lrow, base, base, a, lane, raw, bits, z);
  }
  uint64_t in[kPL];
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < kPL; ++e) {
    in[e] = __ballot(z[e] > -INFINITY && topp_bin(z[e], lz, a.s2) == bc);
    cnt += __popcll(in[e]);
  }
  if (cnt == 0) return;                  // uniform across the wave
  int base = 0;
  if (lane == 0) base = atomicAdd(&row->n, cnt);
  base = __builtin_amdgcn_readfirstlane(base);
  uint32_t* keys = a.topp_key + (int64_t)r * kToppCand;
  int32_t* ids = a.topp_id + (int64_t)r * kToppCand;
  int off = 0;
#pragma unroll
  for (int e = 0; e < kPL; ++e) {
    const uint64_t m = in[e];
    if (m == 0ull) continue;
    if ((m >> lane) & 1ull) {
      const int slot = base + off + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (slot < kToppCand) {
        keys[slot] = topp_key(z[e]);
        ids[slot] = token_of<Tin>(b * kSampleSub, e, lane);
      }
    }
    off += __popcll(m);
  }
}

// T: one 1024-thread workgroup a row: the crossing bin's candidates into LDS,
// the key passes down to z*, the kept weight of every sub-slice, the draw.
template <typename Tin, bool kVec>
__global__ __launch_bounds__(kToppThreads) void sample_topp_kernel(SampleArgs a) {
  __shared__ ToppLds s;
  const int r = blockIdx.x, tid = threadIdx.x;
  const Tin* row = static_cast<const Tin*>(a.logits) + (int64_t)r * a.V;
  const uint32_t* bits = a.wbits + (int64_t)r * a.nb * (kSampleSub / 32);
  const int V = a.V;
  const int ngroups = (V + 3) / 4;
  const float th = a.theta, ith = a.inv_theta;
  const ToppRow rw = a.topp_row[r];
  // loads that depend on nothing here: the draw's uniform, this thread's
  // sub-slice's weight above the crossing bin
  const float u_r = a.u[r];
  const float above_q = tid < a.nb ? a.topp_above[(int64_t)r * a.nb + tid] : 0.0f;
  // the min-p cut binds (the coarse kernel saw it): no crossing bin, no key passes
  const bool minp_only = rw.bc == kToppMinpBinds;
  // no finite logit, or (cannot happen: the crossing bin has weight) no token in it
  if (!minp_only && (rw.bc < 0 || rw.n == 0)) {
    if (tid == 0) a.tok[r] = -1;
    return;
  }
  const float Z = rw.Z, target = rw.target;
  const int bc = minp_only ? kToppCoarse - 1 : rw.bc, n = minp_only ? 0 : rw.n;
  const int lz = topp_level(Z, a.s2);
  const float fx = ldexpf(1.0f, bc + 41), inv_fx = ldexpf(1.0f, -(bc + 41));
  // the held candidates and their key range; a crowded bin starts from the
  // whole key range (three 11-bit passes still end on one key)
  if (tid == 0) {
    s.above = rw.above;
    s.lo = n <= kToppCand ? 0xFFFFFFFFu : 0u;
    s.hi = n <= kToppCand ? 0u : 0xFFFFFFFFu;
  }
  __syncthreads();
  if (n <= kToppCand) {
    const uint32_t* keys = a.topp_key + (int64_t)r * kToppCand;
    const int32_t* ids = a.topp_id + (int64_t)r * kToppCand;
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int i = tid; i < n; i += kToppThreads) {
      const uint32_t key = keys[i];
      s.cand[i] = key;
      s.cid[i] = ids[i];
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
    kmin = wave_all(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
    kmax = wave_all(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
    if ((tid & (kWave - 1)) == 0) {
      atomicMin(&s.lo, kmin);
      atomicMax(&s.hi, kmax);
    }
  }
  __syncthreads();
  uint32_t lo = s.lo, hi = s.hi;
  bool done = lo == hi || minp_only;
  for (int pass = 0; pass < 3 && !done; ++pass) {
    const int nbits = 32 - __clz((int)(hi - lo));
    const int shift = nbits > 11 ? nbits - 11 : 0;
    topp_clear_keys(s);
    __syncthreads();
    if (n <= kToppCand) {
      for (int i = tid; i < n; i += kToppThreads) topp_key_bin(s, s.cand[i], Z, a.s2, lo, hi, shift, fx);
    } else {
      // a crowded bin (nearly flat logits): the key passes read the row
      topp_visit<Tin, kVec>(V, th, ith, row, bits, ngroups, [&](int, const float (&z)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (z[i] > -INFINITY && topp_bin(z[i], lz, a.s2) == bc)
            topp_key_bin(s, topp_key(z[i]), Z, a.s2, lo, hi, shift, fx);
      });
    }
    __syncthreads();
    const int d = topp_select(s, target, inv_fx);
    lo = s.kmn[d];
    hi = s.kmx[d];
    done = lo == hi;
    __syncthreads();
  }
  const float zstar = minp_only ? -INFINITY : topp_value(lo);
  const float thr = fmaxf(Z + a.cut, zstar);
  if (tid == 0) a.topp_cut[r] = zstar;

  // ---- the kept weight of every sub-slice at the row's cut ------------------
  for (int q = tid; q < 4 * a.nb; q += kToppThreads) s.part[q] = 0.0f;
  for (int q = tid; q < a.nb; q += kToppThreads) s.partq[q] = 0ull;
  if (tid == 0) {
    s.win = INT32_MAX;
    s.lastk = -1;
    s.sel = INT32_MAX;
    s.last = -1;
  }
  __syncthreads();
  if (thr == zstar && n <= kToppCand) {
    // the cut is z* (min-p does not bind) and every token of the crossing bin
    // is a held candidate: a sub-slice keeps its weight in the bins above the
    // crossing one and its candidates at or above z* (keys are
    // order-preserving: key >= lo)
    for (int i = tid; i < n; i += kToppThreads) {
      const uint32_t key = s.cand[i];
      if (key >= lo)
        atomicAdd(&s.partq[s.cid[i] / kSampleSub], topp_fixed(__builtin_amdgcn_exp2f((topp_value(key) - Z) * a.s2), fx));
    }
    __syncthreads();
    if (tid < a.nb) {
      s.part[4 * tid] = above_q;
      s.part[4 * tid + 1] = (float)s.partq[tid] * inv_fx;
    }
  } else if (thr > zstar) {
    // min-p binds: a sub-slice whose maximum is below the cut keeps nothing,
    // so only the others are read, each as four 256-token quarters with the
    // lanes, sums and slots of the pass over the row below (the same weights)
    const int wave = tid >> 6, lane = tid & (kWave - 1);
    if (tid == 0) s.nq = 0;
    __syncthreads();
    if (tid < a.nb && a.sub[(int64_t)r * a.nb + tid].m >= thr) s.qlist[atomicAdd(&s.nq, 1)] = tid;
    __syncthreads();
    const int items = 4 * s.nq;
    for (int it = wave; it < items; it += kToppWaves) {
      const int q = s.qlist[it >> 2], j = it & 3;
      const int g = q * (kSampleSub / 4) + kWave * j + lane;
      ToppRaw<Tin, kVec> raw;
      topp_fetch<Tin, kVec>(V, row, bits, 4 * min(g, ngroups - 1), raw);
      float z[4];
      topp_values<Tin, kVec>(V, th, ith, 4 * g, g < ngroups, raw, z);
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (z[i] > -INFINITY && z[i] >= thr) acc += __builtin_amdgcn_exp2f((z[i] - Z) * a.s2);
      acc = wave_sum(acc);
      if (lane == 0) s.part[4 * q + j] = acc;
    }
  } else {
    // a crowded crossing bin at the cut z*: the pass over the row
    const int wave = tid >> 6, lane = tid & (kWave - 1);
    topp_visit<Tin, kVec>(V, th, ith, row, bits, ngroups, [&](int k, const float (&z)[4]) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (z[i] > -INFINITY && z[i] >= thr) acc += __builtin_amdgcn_exp2f((z[i] - Z) * a.s2);
      acc = wave_sum(acc);
      // a wave's 64 groups are 256 tokens of sub-slice 4k + wave/4
      const int q = 4 * k + (wave >> 2);
      if (lane == 0 && q < a.nb) s.part[4 * q + (wave & 3)] = acc;
    });
  }
  __syncthreads();
  float c = 0.0f;
  if (tid < a.nb) c = (s.part[4 * tid] + s.part[4 * tid + 1]) + (s.part[4 * tid + 2] + s.part[4 * tid + 3]);
  float total;
  const float excl = topp_scan(c, s.red, total);
  const float target2 = u_r * total;
  if (c > 0.0f && excl + c > target2) atomicMin(&s.sel, tid);
  if (c > 0.0f) atomicMax(&s.last, tid);
  __syncthreads();
  const bool fallback = s.sel == INT32_MAX;   // u * total at or past the end: the last kept token
  const int q = fallback ? s.last : s.sel;
  if (q < 0) {                           // nothing kept (cannot happen: the maximum always is)
    if (tid == 0) a.tok[r] = -1;
    return;
  }
  if (tid == q) s.above = excl;
  __syncthreads();
  const float base = s.above;
  const int t = q * kSampleSub + tid;
  float w = 0.0f;
  if (t < V) {
    const float x = Elem<Tin>::load(row + t);
    const float z = ((bits[t >> 5] >> (t & 31)) & 1u) ? x * (x > 0.0f ? ith : th) : x;
    if (z > -INFINITY && z >= thr) w = __builtin_amdgcn_exp2f((z - Z) * a.s2);
  }
  float tot_q;
  const float run = base + topp_scan(w, s.red, tot_q) + w;
  if (w > 0.0f) {
    if (!fallback && run > target2) atomicMin(&s.win, t);
    atomicMax(&s.lastk, t);
  }
  __syncthreads();
  if (tid == 0) a.tok[r] = s.win != INT32_MAX ? s.win : s.lastk;
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
  const bool topp = a.topp_cut != nullptr;
  if (vec && topp)
    sample_scan_kernel<Tin, kNT, kPW, true, true><<<grid, kNT, 0, st>>>(a);
  else if (vec)
    sample_scan_kernel<Tin, kNT, kPW, true, false><<<grid, kNT, 0, st>>>(a);
  else if (topp)
    sample_scan_kernel<Tin, kNT, kPW, false, true><<<grid, kNT, 0, st>>>(a);
  else
    sample_scan_kernel<Tin, kNT, kPW, false, false><<<grid, kNT, 0, st>>>(a);
  if (topp) {
    // top-p rows (the scan also binned them): the crossing bin per row, its
    // tokens over the grid, then the cut and the draw per row
    sample_topp_coarse_kernel<<<a.R, kToppThreads, 0, st>>>(a);
    const dim3 egrid((a.nb + kExtractWaves - 1) / kExtractWaves, a.R);
    if (vec)
      sample_topp_extract_kernel<Tin, true><<<egrid, kExtractWaves * kWave, 0, st>>>(a);
    else
      sample_topp_extract_kernel<Tin, false><<<egrid, kExtractWaves * kWave, 0, st>>>(a);
    if (vec)
      sample_topp_kernel<Tin, true><<<a.R, kToppThreads, 0, st>>>(a);
    else
      sample_topp_kernel<Tin, false><<<a.R, kToppThreads, 0, st>>>(a);
  } else if (vec) {
    sample_pick_kernel<Tin, true><<<a.R, kThreads, 0, st>>>(a);
  } else {
    sample_pick_kernel<Tin, false><<<a.R, kThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

int sample_subslices(int V) { return V < 1 ? 1 : (V + kSampleSub - 1) / kSampleSub; }

size_t sample_workspace_bytes(int R, int V) {
  const size_t n = (size_t)R * sample_subslices(V);
  return n * sizeof(SampleSub) + n * kSampleList * sizeof(SampleCand) + n * (kSampleSub / 32) * sizeof(uint32_t) +
         (size_t)R * sizeof(float) + n * (kToppCoarse + 1) * sizeof(float) +
         (size_t)R * kToppCand * (sizeof(uint32_t) + sizeof(int32_t)) + (size_t)R * sizeof(ToppRow);
}

hipError_t launch_sample(const SampleArgs& a, ts_dtype dtype, hipStream_t s) {
  static_assert(kThreads * kPerT == kSampleMaxSubs, "a picking thread holds up to kPerT sub-slices");
  static_assert(kSampleList <= kThreads, "list entries are ranked one per thread");
  return dtype == TS_BF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace ts
