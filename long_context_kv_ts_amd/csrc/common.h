// Shared device helpers and the host-side launch interface of the kernels.
// gfx950 (CDNA4) only: 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ts.h"

namespace ts {

constexpr int kWave = 64;
constexpr int kTile = 64;          // keys per attention tile
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

typedef uint16_t bf16_t;           // bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, h);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};
// four values rounded to bf16 (to nearest even) and packed, lowest first
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2((uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16),
                    (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16));
}

template <> struct Elem<bf16_t> {
  __device__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Load 8 consecutive elements (16 B for bf16, 2x16 B for fp32) as floats.
__device__ __forceinline__ void load8(const bf16_t* p, float* o) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Reductions over the 64 lanes of a wave, the result in every lane, in lane
// moves that need no LDS: DPP within rows of 16 lanes (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror), then the row pairs and
// halves exchanged by v_permlane16_swap and v_permlane32_swap.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_f32<0xB1>(v));
  v = op(v, dpp_f32<0x4E>(v));
  v = op(v, dpp_f32<0x141>(v));
  v = op(v, dpp_f32<0x140>(v));
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
// Inclusive prefix sum over the 64 lanes of a wave in DPP lane moves: shifts
// by 1, 2, 4 and 8 within each row of 16 lanes, then each row's total
// broadcast into the rows above it (row_bcast:15 into rows 1 and 3,
// row_bcast:31 into rows 2 and 3). Lanes a move has no source for add zero.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_add_u32(uint32_t x) {
  return x + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xF, false);
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add_f32(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x = dpp_add_u32<0x111, 0xF>(x);
  x = dpp_add_u32<0x112, 0xF>(x);
  x = dpp_add_u32<0x114, 0xF>(x);
  x = dpp_add_u32<0x118, 0xF>(x);
  x = dpp_add_u32<0x142, 0xA>(x);
  x = dpp_add_u32<0x143, 0xC>(x);
  return x;
}
__device__ __forceinline__ float wave_incl_scan(float x) {
  x = dpp_add_f32<0x111, 0xF>(x);
  x = dpp_add_f32<0x112, 0xF>(x);
  x = dpp_add_f32<0x114, 0xF>(x);
  x = dpp_add_f32<0x118, 0xF>(x);
  x = dpp_add_f32<0x142, 0xA>(x);
  x = dpp_add_f32<0x143, 0xC>(x);
  return x;
}
__device__ __forceinline__ int wave_incl_scan(int x) { return (int)wave_incl_scan((uint32_t)x); }

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

// Ancestor-or-self bitmask rows of the drafts t in [t_lo, t_hi), built in LDS:
// bit a of anc[(t - t_lo) * words + a/32] is set iff a is t or an ancestor of
// t. parent[0 .. t_hi) is first staged in LDS (s_par), so each walk chases
// parents there. Entries of parent[] outside [-1, t) end the walk (treated as
// roots), so a walk takes at most t steps and never leaves [0, T). With
// parent == nullptr the drafts form one causal chain (parent[t] = t - 1) and
// s_par is not used. Rows a workgroup does not own are never built.
__device__ __forceinline__ void build_ancestor_rows(const int32_t* parent, int words, int t_lo, int t_hi,
                                                    uint32_t* anc, int32_t* s_par, int tid, int nthreads) {
  const int n = t_hi - t_lo;
  for (int i = tid; i < n * words; i += nthreads) anc[i] = 0u;
  if (parent != nullptr)
    for (int t = tid; t < t_hi; t += nthreads) s_par[t] = parent[t];
  __syncthreads();
  for (int t = t_lo + tid; t < t_hi; t += nthreads) {
    uint32_t* row = anc + (t - t_lo) * words;
    if (parent == nullptr) {
      for (int w = 0; w < words; ++w) {
        int lo = w * 32;
        uint32_t bits = 0u;
        if (t >= lo + 31) bits = 0xffffffffu;
        else if (t >= lo) bits = (t - lo == 31) ? 0xffffffffu : ((1u << (t - lo + 1)) - 1u);
        row[w] = bits;
      }
    } else {
      int a = t;
      while (a >= 0) {
        row[a >> 5] |= 1u << (a & 31);
        int p = s_par[a];
        a = (p >= 0 && p < a) ? p : -1;
      }
    }
  }
  __syncthreads();
}

// Draft rows [t_lo, t_hi) behind query rows [row0, row1) of one KV head (row = t * G + h).
__device__ __forceinline__ void draft_rows_of(int row0, int row1, int G, int T, int& t_lo, int& t_hi) {
  t_lo = row0 / G;
  t_hi = row1 > row0 ? min(T, (row1 - 1) / G + 1) : t_lo;
}

// ----------------------------------------------------------------------------
// Work decomposition of one masked split-K attention call.
// ----------------------------------------------------------------------------
enum AttnPath { kPathValu = 0, kPathMfma = 1, kPathSmall = 2 };

struct AttnPlan {
  int path;
  int tile;             // keys per tile of the chosen kernel
  int rows_per_head;    // T * G
  int rows_per_group;   // rows of one workgroup
  int n_rowgroups;
  int n_cache_tiles;    // ceil(L / tile)
  int n_draft_tiles;    // ceil(T / tile)
  int n_virtual;        // cache tiles then draft tiles
  int tiles_per_split;
  int n_splits;
};

struct AttnArgs {
  const void* q;            // [T][Hq][D]
  const void* kc;           // [Hkv][cache_stride][D]
  const void* vc;
  int64_t cache_stride;
  const void* kd;           // [Hkv][T][D]
  const void* vd;
  const int32_t* parent;    // [T] or nullptr = causal chain
  float* o_part;            // [S][T][Hq][D]
  bf16_t* o_part_h;         // or, when set, the same partials in bf16 (a call's own workspace)
  float* l_part;            // [S][T][Hq]
  int T, Hq, Hkv, G, D;
  int64_t L;
  float scale_log2;         // scale * log2(e)
  AttnPlan plan;
  // chunk importance over the same cache, computed by the split kernel's
  // all-padding wave (q_imp == nullptr: off; see attn_mfma_importance_fusable)
  const void* q_imp;        // [imp_R][Hq][D] the recent queries
  float* scores;            // [Hkv][L / 64]
  int imp_R;
  float imp_scale;
  // gather fused into the pass over a partial cache (small path only; gidx ==
  // nullptr: off): cache tile i of KV head g is chunk gidx[g][i] of the cache
  // kc/vc (cache_stride, g_chunks chunks of kTile tokens), and is also copied
  // to kp/vp [Hkv][L][D]; an index outside [0, g_chunks) is a zero tile
  const int32_t* gidx;      // [Hkv][L / kTile]
  int64_t g_chunks;
  void* kp;
  void* vp;
};

AttnPlan plan_attention(int T, int Hq, int Hkv, int D, int64_t L, ts_dtype dtype, int num_splits);

// Host-side pieces of the C ABI (api.cpp) that other entry points reuse: the
// shape checks of the attention calls, recording an error message for
// ts_last_error(), and ts_tree_verify_attn itself with a caller-chosen name
// for its messages.
ts_status check_attn_args(const char* fn, int T, int Hq, int Hkv, int D, int64_t L, ts_dtype dtype,
                          int num_splits);
ts_status set_error(ts_status st, const char* msg);
ts_status tree_verify_into(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                           int64_t cache_stride, const void* k_draft, const void* v_draft, const int32_t* parent,
                           void* out, float* lse, int T, int Hq, int Hkv, int D, int64_t L, float scale,
                           ts_dtype dtype, int num_splits, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

// Work decomposition of the matrix-core kernel (defined next to it).
int mfma_rows_per_group(int rows_per_head);   // 256, or 128 when a KV head has at most 128 rows
// Whether the matrix-core split kernel can score 64-token chunks of the cache
// for R recent queries of group size G in its last row group's all-padding wave.
bool attn_mfma_importance_fusable(const AttnPlan& p, int T, int G, int D, int64_t L, int R);
int mfma_groups_per_cu();
int mfma_tile_keys();

// Launchers (return the hipGetLastError() of the launch).
hipError_t launch_attn_split_valu(const AttnArgs& a, ts_dtype dtype, hipStream_t s);
hipError_t launch_attn_split_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_split_small(const AttnArgs& a, hipStream_t s);
// o_part: fp32, or bf16 when part_bf16
hipError_t launch_attn_merge(const void* o_part, bool part_bf16, const float* l_part, int n_parts, int rows,
                             int D, void* out, float* lse, ts_dtype dtype, hipStream_t s);
hipError_t launch_importance(const void* q, const void* kc, int64_t stride, float* scores,
                             int R, int Hq, int Hkv, int D, int64_t L, int chunk, float scale,
                             ts_dtype dtype, hipStream_t s);
// The merge and the 64-token chunk importance in one grid (fused.hip), for the
// shapes merge_importance_fusable accepts.
bool merge_importance_fusable(int n_parts, int Dm, int Di, int R, int Hq, int Hkv, int chunk, ts_dtype dtype);
hipError_t launch_merge_importance(const void* o_part, bool part_bf16, const float* l_part, int n_parts, int rows, void* out,
                                   float* lse, ts_dtype out_dtype, const void* q, const void* kc,
                                   int64_t stride, float* scores, int R, int Hq, int Hkv, int64_t L,
                                   float scale, hipStream_t s);
hipError_t launch_topk(const float* scores, int Hkv, int n, int k, int32_t* idx, float* val,
                       hipStream_t s);
// The merge and the top-k selection in one grid (fused.hip), for the merges
// merge_topk_fusable accepts.
bool merge_topk_fusable(int n_parts, int Dm);
hipError_t launch_merge_topk(const void* o_part, bool part_bf16, const float* l_part, int n_parts, int rows, void* out, float* lse,
                             ts_dtype out_dtype, const float* scores, int Hkv, int n, int k, int32_t* idx, float* val,
                             hipStream_t s);
hipError_t launch_gather(const void* kc, const void* vc, int64_t stride, const int32_t* idx,
                         int Hkv, int k, int chunk, int D, int64_t L, void* kp, void* vp,
                         int elem_bytes, hipStream_t s);

}  // namespace ts
