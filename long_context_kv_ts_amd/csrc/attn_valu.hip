// Masked split-K attention on the vector ALUs (fp32 math), for fp32 inputs and
// for bf16 shapes whose grouped query rows per KV head are too few for a
// matrix-core tile (e.g. the 4-token draft pass of an MHA model).
//
// One workgroup = (row group of 16 query rows, split, KV head). A row is a
// (draft token t, query head h) pair of the KV head's group, row = t*G + h%G.
// The split walks its range of 64-key tiles -- cached tokens first, then the
// draft tokens under the ancestor-or-self mask -- staging each K/V tile in LDS
// as fp32, and keeps a running max / sum per row (online softmax in base 2).
// It writes the split's normalised output and natural-log LSE; the
// log-sum-exp merge combines splits (attn_merge.hip).
#include "common.h"

namespace ts {
namespace {

constexpr int kRows = 16;          // query rows per workgroup
constexpr int kThreads = 256;      // 4 waves, 4 rows each

template <typename Tin, int D>
__global__ __launch_bounds__(kThreads) void attn_split_valu_kernel(AttnArgs a) {
  constexpr int DL = D / kWave;    // output columns per lane
  __shared__ float Ks[kTile][D + 1];
  __shared__ float Vs[kTile][D];
  __shared__ float Qs[kRows][D];
  __shared__ float Ps[kRows][kTile];
  __shared__ uint32_t anc[kRows * (TS_MAX_DRAFT / 32)];   // this workgroup's drafts (<= kRows)
  __shared__ int32_t s_par[TS_MAX_DRAFT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = blockIdx.x, split = blockIdx.y, g = blockIdx.z;
  const AttnPlan& pl = a.plan;
  const int G = a.G, T = a.T, Hq = a.Hq;
  const int row0 = rg * kRows;
  const Tin* q = static_cast<const Tin*>(a.q);

  for (int i = tid; i < kRows * D; i += kThreads) {
    const int r = i / D, d = i % D, row = row0 + r;
    float v = 0.f;
    if (row < pl.rows_per_head) {
      const int t = row / G, h = g * G + row % G;
      v = Elem<Tin>::load(q + ((int64_t)t * Hq + h) * D + d) * a.scale_log2;
    }
    Qs[r][d] = v;
  }
  const int vt0 = split * pl.tiles_per_split;
  const int vt1 = min(vt0 + pl.tiles_per_split, pl.n_virtual);
  const int words = (T + 31) >> 5;
  int t_lo, t_hi;
  draft_rows_of(row0, min(pl.rows_per_head, row0 + kRows), G, T, t_lo, t_hi);
  if (vt1 > pl.n_cache_tiles) build_ancestor_rows(a.parent, words, t_lo, t_hi, anc, s_par, tid, kThreads);

  float m[4], l[4], acc[4][DL];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int k = 0; k < DL; ++k) acc[i][k] = 0.f;
  }

  for (int vt = vt0; vt < vt1; ++vt) {
    const bool draft = vt >= pl.n_cache_tiles;
    const int key0 = draft ? (vt - pl.n_cache_tiles) * kTile : vt * kTile;
    const int nvalid = draft ? min(kTile, T - key0) : (int)min((int64_t)kTile, a.L - key0);
    const Tin* kb = draft ? static_cast<const Tin*>(a.kd) + ((int64_t)g * T + key0) * D
                          : static_cast<const Tin*>(a.kc) + ((int64_t)g * a.cache_stride + key0) * D;
    const Tin* vb = draft ? static_cast<const Tin*>(a.vd) + ((int64_t)g * T + key0) * D
                          : static_cast<const Tin*>(a.vc) + ((int64_t)g * a.cache_stride + key0) * D;
    __syncthreads();
    for (int i = tid * 8; i < kTile * D; i += kThreads * 8) {
      const int key = i / D, d = i % D;
      float kv[8], vv[8];
      if (key < nvalid) {
        load8(kb + (int64_t)key * D + d, kv);
        load8(vb + (int64_t)key * D + d, vv);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) kv[j] = vv[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        Ks[key][d + j] = kv[j];
        Vs[key][d + j] = vv[j];
      }
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 4 + i, row = row0 + r;
      float s = 0.f;
#pragma unroll 16
      for (int d = 0; d < D; ++d) s += Qs[r][d] * Ks[lane][d];
      bool ok = lane < nvalid && row < pl.rows_per_head;
      if (draft && ok) {
        const int t = row / G, key = key0 + lane;
        ok = (anc[(t - t_lo) * words + (key >> 5)] >> (key & 31)) & 1u;
      }
      s = ok ? s : -INFINITY;
      const float mt = wave_max(s);
      const float mnew = fmaxf(m[i], mt);
      const float p = ok ? exp2f(s - mnew) : 0.f;
      const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m[i] - mnew);
      l[i] = l[i] * alpha + wave_sum(p);
      m[i] = mnew;
      Ps[r][lane] = p;
#pragma unroll
      for (int k = 0; k < DL; ++k) acc[i][k] *= alpha;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 4 + i;
#pragma unroll 8
      for (int j = 0; j < kTile; ++j) {
        const float p = Ps[r][j];
#pragma unroll
        for (int k = 0; k < DL; ++k) acc[i][k] += p * Vs[j][lane + kWave * k];
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + wave * 4 + i;
    if (row >= pl.rows_per_head) continue;
    const int t = row / G, h = g * G + row % G;
    const int64_t orow = ((int64_t)split * T + t) * Hq + h;
    const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;
#pragma unroll
    for (int k = 0; k < DL; ++k) a.o_part[orow * D + lane + kWave * k] = acc[i][k] * inv;
    if (lane == 0) a.l_part[orow] = l[i] > 0.f ? (m[i] + log2f(l[i])) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_split_valu(const AttnArgs& a, ts_dtype dtype, hipStream_t s) {
  dim3 grid(a.plan.n_rowgroups, a.plan.n_splits, a.Hkv);
  if (dtype == TS_BF16) {
    if (a.D == 128) attn_split_valu_kernel<bf16_t, 128><<<grid, kThreads, 0, s>>>(a);
    else attn_split_valu_kernel<bf16_t, 64><<<grid, kThreads, 0, s>>>(a);
  } else {
    if (a.D == 128) attn_split_valu_kernel<float, 128><<<grid, kThreads, 0, s>>>(a);
    else attn_split_valu_kernel<float, 64><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

int valu_rows_per_group() { return kRows; }

}  // namespace ts
