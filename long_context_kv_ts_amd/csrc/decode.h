// Host-side launch interface of the decode-step kernels that sit around the
// attention: the candidate tree, target-token sampling and the acceptance with
// its KV-cache commit.
#pragma once

#include "common.h"

namespace ts {

// Candidate tree of draft tokens (shape [k_0..k_{depth-1}]): per depth d the
// number of candidates k[d], the node count n[d] = k[0]*..*k[d] and the first
// node index off[d] (breadth-first numbering).
constexpr int kTreeMaxDepth = 8;
constexpr int kTreeMaxK = 16;
constexpr int kTreeMaxNodes = 1024;
struct TreeShape {
  int k[kTreeMaxDepth];
  int n[kTreeMaxDepth];
  int off[kTreeMaxDepth];
};
int tree_slices(int V);    // vocabulary slices per position (workspace rows)
hipError_t launch_build_tree(const void* logits, int V, const TreeShape& shape, int depth,
                             int32_t* parent, int32_t* draft_tok, int32_t* cand, void* workspace,
                             ts_dtype dtype, hipStream_t s);

hipError_t launch_accept_commit(const int32_t* parent, const int32_t* draft_tok,
                                const int32_t* target_tok, uint32_t rand_u32, int T, void* kc,
                                void* vc, int64_t stride, int64_t L, const void* kd, const void* vd,
                                int Hkv, int D, int elem_bytes, int32_t* n_out, int32_t* path_out,
                                int32_t* bonus_out, hipStream_t s);

// Target-token sampling: per row, the windowed repetition penalty, the
// temperature, the min-p filter and an inverse-CDF draw from u[row].
constexpr int kSampleSub = 4096;         // logits per sub-slice (the unit the draw is located in)
constexpr int kSampleMaxSubs = 256;      // sub-slices per row at most (V <= 1048576)
constexpr int kSampleList = 32;          // kept candidates remembered per sub-slice
struct SampleSub {                       // summary of one sub-slice
  float m;                               // largest penalised logit
  float s;                               // sum of 2^((z - m) * s2) over z >= m + cut
  int n;                                 // how many z >= m + cut (listed: the first kSampleList)
  int pad;
};
struct SampleCand {
  float z;                               // penalised logit
  int idx;                               // token id
};
struct SampleArgs {
  const void* logits;         // [R][V]
  int R, V;
  int nb;                     // sub-slices per row
  const int32_t* hist;        // the last n_hist committed tokens
  int n_hist;
  const int32_t* parent;      // [T] drafts; row t+1 follows draft t
  const int32_t* draft_tok;   // [T]
  int T;
  int window;                 // penalty window W (tokens)
  float theta;                // penalty
  float s2;                   // log2(e) / temperature (0: greedy)
  float cut;                  // temperature * ln(min_p) (<= 0; -inf keeps every token; greedy: 0)
  const float* u;             // [R] uniforms in [0, 1)
  int32_t* tok;               // [R]
  SampleSub* sub;             // [R][nb]
  SampleCand* cand;           // [R][nb][kSampleList]
};
int sample_subslices(int V);
size_t sample_workspace_bytes(int R, int V);
hipError_t launch_sample(const SampleArgs& a, ts_dtype dtype, hipStream_t s);

}  // namespace ts
