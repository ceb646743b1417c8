// Acceptance of the verified drafts and the KV-cache commit.
//
// Drafts form a forest (parent[t] in [-1, t); other values count as roots).
// target_tok[0] is the target model's token for the position after the
// committed context and target_tok[t+1] its token for the position after
// draft t. A draft path is valid when every node carries the token the target
// produced at the position before it. Among the valid paths of greatest
// length, ordered by their last node's index, number rand % count is accepted;
// its K/V rows move from the draft buffers into cache rows L .. L+n-1.
//
// One workgroup per (KV head, K or V). With at most 1024 drafts the acceptance
// is a few hundred integer operations, so every workgroup computes it itself
// (the forest and tokens are staged in LDS, thread t walks node t's ancestors
// there) and then copies its own head's rows:
// no workgroup waits for another. Workgroup (0, 0) also writes n, the path
// and the bonus token.
#include "decode.h"

namespace ts {
namespace {

constexpr int kThreads = TS_MAX_DRAFT;     // one thread per draft
constexpr int kWavesA = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void accept_commit_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ draft_tok,
    const int32_t* __restrict__ target_tok, int T, uint32_t rand_u32,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, int64_t head_bytes, int64_t L,
    const uint8_t* __restrict__ kd, const uint8_t* __restrict__ vd, int row_bytes,
    int32_t* __restrict__ n_out, int32_t* __restrict__ path_out, int32_t* __restrict__ bonus_out) {
  __shared__ int s_path[TS_MAX_DRAFT];
  __shared__ int s_par[TS_MAX_DRAFT], s_draft[TS_MAX_DRAFT], s_tgt[TS_MAX_DRAFT + 1];
  __shared__ int s_best[kWavesA], s_cnt[kWavesA];
  __shared__ int s_last;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t >> 6;

  // the forest and its tokens in LDS (the root walks below chase parents)
  if (t < T) {
    const int p = parent[t];
    s_par[t] = (p < -1 || p >= t) ? -1 : p;
    s_draft[t] = draft_tok[t];
  }
  if (t < T) s_tgt[t] = target_tok[t];
  if (t == 0) s_tgt[T] = target_tok[T];    // T may equal the block size
  __syncthreads();
  // depth of node t if its root path is valid, else -1 (the walk ends: parents decrease)
  int depth = -1;
  if (t < T) {
    bool ok = true;
    int d = 0, a = t;
    while (a >= 0) {
      const int p = s_par[a];
      ok = ok && s_draft[a] == s_tgt[p + 1];
      d += p >= 0;
      a = p;
    }
    depth = ok ? d : -1;
  }
  int m = depth;
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
  if (lane == 0) s_best[wave] = m;
  __syncthreads();
  int best = s_best[0];
#pragma unroll
  for (int w = 1; w < kWavesA; ++w) best = max(best, s_best[w]);

  // the (rand % count)-th deepest valid node in index order
  const bool cand = best >= 0 && depth == best;
  const uint64_t bal = __ballot(cand);
  if (lane == 0) s_cnt[wave] = (int)__popcll(bal);
  __syncthreads();
  int total = 0, before = 0;
#pragma unroll
  for (int w = 0; w < kWavesA; ++w) {
    total += s_cnt[w];
    before += w < wave ? s_cnt[w] : 0;
  }
  if (cand) {
    const int rank = before + (int)__popcll(bal & ((1ull << lane) - 1ull));
    if ((uint32_t)rank == rand_u32 % (uint32_t)total) s_last = t;
  }
  __syncthreads();
  const int n = best >= 0 ? best + 1 : 0;
  if (t == 0 && n > 0) {
    int a = s_last;
    for (int i = n - 1; i >= 0; --i) {
      s_path[i] = a;
      a = s_par[a];
    }
  }
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    if (t < T) path_out[t] = t < n ? s_path[t] : -1;
    if (t == 0) {
      *n_out = n;
      *bonus_out = n > 0 ? s_tgt[s_last + 1] : s_tgt[0];
    }
  }

  // commit: rows path[0..n) of this head's draft buffer -> cache rows L..L+n-1
  const int g = blockIdx.x;
  uint8_t* dst = (blockIdx.y ? vc : kc) + (int64_t)g * head_bytes + L * row_bytes;
  const uint8_t* src = (blockIdx.y ? vd : kd) + (int64_t)g * T * row_bytes;
  const int n16 = row_bytes >> 4;
  for (int e = t; e < n * n16; e += kThreads) {
    const int i = e / n16, cc = e - i * n16;
    reinterpret_cast<uint4*>(dst + (int64_t)i * row_bytes)[cc] =
        reinterpret_cast<const uint4*>(src + (int64_t)s_path[i] * row_bytes)[cc];
  }
}

}  // namespace

hipError_t launch_accept_commit(const int32_t* parent, const int32_t* draft_tok,
                                const int32_t* target_tok, uint32_t rand_u32, int T, void* kc,
                                void* vc, int64_t stride, int64_t L, const void* kd, const void* vd,
                                int Hkv, int D, int elem_bytes, int32_t* n_out, int32_t* path_out,
                                int32_t* bonus_out, hipStream_t s) {
  const int row_bytes = D * elem_bytes;
  dim3 grid(Hkv, 2);
  accept_commit_kernel<<<grid, kThreads, 0, s>>>(
      parent, draft_tok, target_tok, T, rand_u32, static_cast<uint8_t*>(kc),
      static_cast<uint8_t*>(vc), stride * row_bytes, L, static_cast<const uint8_t*>(kd),
      static_cast<const uint8_t*>(vd), row_bytes, n_out, path_out, bonus_out);
  return hipGetLastError();
}

}  // namespace ts
