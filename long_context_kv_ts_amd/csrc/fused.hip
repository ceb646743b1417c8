// One launch for two independent steps of a decode step: the cross-split
// merge of the verify pass and the chunk importance of the partial-KV refresh.
// The first workgroups score chunks, the rest merge verify rows; each runs
// exactly the code of its own kernel (merge_block.h, importance_block.h), so
// the results are bit-identical to the two separate launches. Merging in the
// same grid saves one launch boundary and lets the merge's short workgroups
// fill the CUs as the importance read drains (chunk scoring comes first in
// the grid: merging first measured slower).
//
// Covered here: head_dim 128 for both, a merge that one wave per row covers
// (at most 16 splits), bf16 keys with 64-token chunks and at most 64 grouped
// query rows. Anything else takes the two separate launches.
#include "importance_block.h"
#include "merge_block.h"
#include "topk_block.h"

namespace ts {
namespace {

struct MergePart {
  const void* o_part;        // fp32, or bf16 (the kernels' Tin)
  const float* l_part;
  int S, rows;
  void* out;
  float* lse;
};

struct ImportancePart {
  const bf16_t* q;
  const bf16_t* kc;
  int64_t stride;
  float* scores;
  int R, Hq, Hkv, n_chunks;
  float scale;
};

template <typename Tout, typename Tin, int NRB, bool kPow2>
__global__ __launch_bounds__(256) void merge_importance_kernel(MergePart m, ImportancePart p, int imp_bx) {
  static_assert(MergeShape<1>::block == 256, "a merge workgroup is the launch's 256 threads");
  // chunk scoring first, merged rows last: the merge's short workgroups fill
  // the CUs as the importance read drains
  const int b = blockIdx.x, imp_blocks = imp_bx * p.Hkv;
  if (b < imp_blocks) {
    importance64_block<128, NRB, kPow2>(p.q, p.kc, p.stride, p.scores, p.R, p.Hq, p.Hkv, p.scale, p.n_chunks,
                                        b % imp_bx, b / imp_bx, imp_bx);
    return;
  }
  merge_block<Tout, 128, 1, Tin>(static_cast<const Tin*>(m.o_part), m.l_part, m.S, m.rows,
                                 static_cast<Tout*>(m.out), m.lse, b - imp_blocks);
}

template <typename Tout, typename Tin, bool kPow2>
hipError_t launch_rows(const MergePart& m, const ImportancePart& p, int imp_bx, int blocks, int rows_i,
                       hipStream_t s) {
  if (rows_i <= 16)
    merge_importance_kernel<Tout, Tin, 1, kPow2><<<blocks, 256, 0, s>>>(m, p, imp_bx);
  else if (rows_i <= 32)
    merge_importance_kernel<Tout, Tin, 2, kPow2><<<blocks, 256, 0, s>>>(m, p, imp_bx);
  else
    merge_importance_kernel<Tout, Tin, 4, kPow2><<<blocks, 256, 0, s>>>(m, p, imp_bx);
  return hipGetLastError();
}

template <typename Tout, typename Tin>
hipError_t launch_rows_t(const MergePart& m, const ImportancePart& p, int imp_bx, int blocks, int rows_i,
                         bool pow2, hipStream_t s) {
  return pow2 ? launch_rows<Tout, Tin, true>(m, p, imp_bx, blocks, rows_i, s)
              : launch_rows<Tout, Tin, false>(m, p, imp_bx, blocks, rows_i, s);
}

// The verify merge and the top-k chunk selection in one launch: the first Hkv
// workgroups select one KV head's chunks each (256 threads, eight scores a
// thread per round), the rest merge rows, each with its own kernel's code.
struct TopkPart {
  const float* scores;
  int n, k;
  int32_t* idx;
  float* val;
};

template <typename Tout, typename Tin, bool kResident>
__global__ __launch_bounds__(256) void merge_topk_kernel(MergePart m, TopkPart t, int Hkv) {
  const int b = blockIdx.x;
  if (b < Hkv) {
    topk_block<256, 8, kResident>(t.scores, t.n, t.k, t.idx, t.val, b);
    return;
  }
  merge_block<Tout, 128, 1, Tin>(static_cast<const Tin*>(m.o_part), m.l_part, m.S, m.rows,
                                 static_cast<Tout*>(m.out), m.lse, b - Hkv);
}

template <typename Tout, typename Tin>
void launch_merge_topk_t(const MergePart& m, const TopkPart& t, int Hkv, int blocks, bool resident, hipStream_t s) {
  if (resident) merge_topk_kernel<Tout, Tin, true><<<blocks, 256, 0, s>>>(m, t, Hkv);
  else merge_topk_kernel<Tout, Tin, false><<<blocks, 256, 0, s>>>(m, t, Hkv);
}

}  // namespace

bool merge_topk_fusable(int n_parts, int Dm) {
  const int need = ((n_parts + kMergeBatch - 1) / kMergeBatch) * (128 / 4);   // lanes a merged row needs
  return Dm == 128 && need <= kWave;
}

hipError_t launch_merge_topk(const void* o_part, bool part_bf16, const float* l_part, int n_parts, int rows, void* out,
                             float* lse, ts_dtype out_dtype, const float* scores, int Hkv, int n, int k, int32_t* idx,
                             float* val, hipStream_t s) {
  const int merge_blocks = (rows + MergeShape<1>::rows - 1) / MergeShape<1>::rows;
  const int64_t blocks = (int64_t)merge_blocks + Hkv;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const MergePart m{o_part, l_part, n_parts, rows, out, lse};
  const TopkPart t{scores, n, k, idx, val};
  const bool resident = n <= 256 * 8;
  if (out_dtype == TS_BF16) {
    if (part_bf16) launch_merge_topk_t<bf16_t, bf16_t>(m, t, Hkv, (int)blocks, resident, s);
    else launch_merge_topk_t<bf16_t, float>(m, t, Hkv, (int)blocks, resident, s);
  } else {
    if (part_bf16) launch_merge_topk_t<float, bf16_t>(m, t, Hkv, (int)blocks, resident, s);
    else launch_merge_topk_t<float, float>(m, t, Hkv, (int)blocks, resident, s);
  }
  return hipGetLastError();
}

bool merge_importance_fusable(int n_parts, int Dm, int Di, int R, int Hq, int Hkv, int chunk, ts_dtype dtype) {
  const int need = ((n_parts + kMergeBatch - 1) / kMergeBatch) * (128 / 4);   // lanes a merged row needs
  return Dm == 128 && Di == 128 && need <= kWave && dtype == TS_BF16 && chunk == 64 && R * (Hq / Hkv) <= 64;
}

hipError_t launch_merge_importance(const void* o_part, bool part_bf16, const float* l_part, int n_parts, int rows, void* out,
                                   float* lse, ts_dtype out_dtype, const void* q, const void* kc,
                                   int64_t stride, float* scores, int R, int Hq, int Hkv, int64_t L,
                                   float scale, hipStream_t s) {
  const int n_chunks = (int)(L / 64);
  const int merge_blocks = (rows + MergeShape<1>::rows - 1) / MergeShape<1>::rows;
  const int imp_bx = (n_chunks + 1) / 2;                 // two 64-token chunks a workgroup
  const int64_t blocks = (int64_t)merge_blocks + (int64_t)imp_bx * Hkv;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const MergePart m{o_part, l_part, n_parts, rows, out, lse};
  const ImportancePart p{static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(kc), stride, scores, R, Hq,
                         Hkv, n_chunks, scale};
  const int G = Hq / Hkv, rows_i = R * G;
  const bool pow2 = (G & (G - 1)) == 0;
  if (out_dtype == TS_BF16)
    return part_bf16 ? launch_rows_t<bf16_t, bf16_t>(m, p, imp_bx, (int)blocks, rows_i, pow2, s)
                     : launch_rows_t<bf16_t, float>(m, p, imp_bx, (int)blocks, rows_i, pow2, s);
  return part_bf16 ? launch_rows_t<float, bf16_t>(m, p, imp_bx, (int)blocks, rows_i, pow2, s)
                   : launch_rows_t<float, float>(m, p, imp_bx, (int)blocks, rows_i, pow2, s);
}

}  // namespace ts
