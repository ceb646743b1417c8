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
constexpr int kSampleSub = 1024;         // logits per sub-slice (the unit the draw is located in)
constexpr int kToppCoarseBins = 32;      // top-p coarse bins per sub-slice: powers of two of weight
constexpr int kToppCandMax = 8192;       // top-p: tokens of a row's crossing coarse bin held in a list
constexpr int kSampleMaxSubs = 1024;     // sub-slices per row at most (V <= 1048576)
constexpr int kSampleList = 32;          // kept candidates remembered per sub-slice
struct SampleSub {                       // summary of one sub-slice
  float m;                               // largest penalised logit
  float s;                               // sum of 2^((z - m) * s2) over z >= m + cut
  int n;                                 // how many z >= m + cut (listed: the first kSampleList)
  float wall;                            // sum of 2^((z - m) * s2) over every finite z (top-p only)
};
struct SampleCand {
  float z;                               // penalised logit
  int idx;                               // token id
};
struct ToppRow {                         // one top-p row's coarse result, a cache line of its own
  float Z;                               // largest penalised logit
  float target;                          // top_p times the row's total weight
  float above;                           // weight of the coarse bins above the crossing one
  int bc;                                // the crossing coarse bin (-1: no finite logit)
  int n;                                 // tokens in the crossing bin (counted by atomics)
  int pad[27];
};
static_assert(sizeof(ToppRow) == 128, "a row record fills one cache line");
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
  float inv_theta;            // 1 / theta, rounded once
  float s2;                   // log2(e) / temperature (0: greedy)
  float cut;                  // temperature * ln(min_p) (<= 0; -inf keeps every token; greedy: 0)
  const float* u;             // [R] uniforms in [0, 1)
  float top_p;                // nucleus mass (1: off)
  float* topp_cut;            // [R] each row's top-p cut on z (nullptr: top-p off)
  float* topp_hist;           // [R][nb][32] top-p: each sub-slice's weight per coarse bin
  float* topp_above;          // [R][nb] top-p: each sub-slice's weight above the crossing bin
  uint32_t* topp_key;         // [R][kToppCandMax] top-p: keys of the crossing bin's tokens
  int32_t* topp_id;           // [R][kToppCandMax] and their token ids
  ToppRow* topp_row;          // [R]
  int32_t* tok;               // [R]
  SampleSub* sub;             // [R][nb]
  SampleCand* cand;           // [R][nb][kSampleList]
  uint32_t* wbits;            // [R][nb][kSampleSub / 32] window bit of each token
};
int sample_subslices(int V);
size_t sample_workspace_bytes(int R, int V);
hipError_t launch_sample(const SampleArgs& a, ts_dtype dtype, hipStream_t s);

// 4-gram table of the committed text: header, slots (entry id or -1), entries.
struct NgramEntry {
  int32_t tok[4];
  int32_t count;                         // 0: an entry that was never published
  int32_t last;                          // last position at which the 4-gram ended
};
struct NgramHeader {                     // the first bytes of the table (same layout as ts_ngram_header)
  int32_t capacity_log2;
  int32_t max_entries;
  int32_t n_entries;                     // entries allocated (may pass max_entries: then dropped counts)
  int32_t dropped;                       // 4-grams that found no room
};
struct NgramView {
  NgramHeader* hdr;
  int32_t* slots;                        // [1 << capacity_log2]
  NgramEntry* entries;                   // [max_entries]
};
constexpr int kNgramHeaderBytes = 256;
constexpr int kNgramMaxCapacityLog2 = 24;
constexpr int kNgramMaxEntries = 262144; // 64 scan workgroups of 4096 entries
constexpr int kNgramMaxK = 64;
size_t ngram_table_bytes(int capacity_log2, int max_entries);
// The layout of a table of capacity 2^capacity_log2 (host and device).
__host__ __device__ inline NgramView ngram_view(void* table, int capacity_log2) {
  char* b = static_cast<char*>(table);
  NgramView v;
  v.hdr = reinterpret_cast<NgramHeader*>(b);
  v.slots = reinterpret_cast<int32_t*>(b + kNgramHeaderBytes);
  v.entries = reinterpret_cast<NgramEntry*>(b + kNgramHeaderBytes + ((size_t(4) << capacity_log2) + 255) / 256 * 256);
  return v;
}
size_t ngram_retrieve_workspace_bytes(int max_entries, int k);
hipError_t launch_ngram_init(NgramView t, int capacity_log2, int max_entries, hipStream_t s);
// These two read the table's layout from its header on the device.
hipError_t launch_ngram_update(void* table, const int32_t* tokens, int64_t from, int64_t to, hipStream_t s);
hipError_t launch_ngram_retrieve(void* table, int max_entries, const int32_t* first_tok, int k, int32_t* out_tok,
                                 int32_t* out_count, int32_t* n_found, void* workspace, hipStream_t s);

}  // namespace ts
