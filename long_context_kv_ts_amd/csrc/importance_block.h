// Chunk importance over 64-token chunks on matrix cores, one workgroup's work
// as a device function of (workgroup index, KV head), so that the importance
// kernel and the launch that shares its grid with the cross-split merge run
// the same code. The score of chunk c of KV head g is the mean over the R
// recent queries and the chunk's tokens of the max over the G grouped query
// heads of scale * <q, k>.
#pragma once

#include "common.h"

namespace ts {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Rows x keys of one 16-key block, per wave (the padding column keeps the
// transposed writes off a single bank).
struct ScoreTile {
  float v[64][17];
};

// Sum over the R queries and the block's valid keys of the max over each
// query's G rows, from the tile (general G).
__device__ __forceinline__ float tile_group_max_sum(const ScoreTile& t, int R, int G, int nkeys, int lane) {
  float tot = 0.f;
  for (int p = lane; p < R * 16; p += kWave) {
    const int r = p >> 4, key = p & 15;
    if (key >= nkeys) continue;
    float v = -INFINITY;
    for (int h = 0; h < G; ++h) v = fmaxf(v, t.v[r * G + h][key]);
    tot += v;
  }
  return tot;
}

// ---------------------------------------------------------------------------
// matrix-core path (bf16)
//
// v_mfma_f32_16x16x32_bf16, A = K block (16 keys x 32 dims), B = Q^T (32 dims x
// 16 rows), C = S^T (16 keys x 16 rows). Lane l supplies A row l%16 and B
// column l%16, each with the 8 reduction elements 8*(l/16)..8*(l/16)+7 of the
// step; C lane l holds column l%16 (a query row) for keys 4*(l/16)+i, i<4.
// The reduction order over D is free, so reduction step ks of a lane takes
// dims 32*ks + 8*(l/16) .. +7, i.e. 64 contiguous bytes per key per step.

// 64-token chunks, two waves a chunk: each wave requests its 32 keys' K (8 KB)
// before any product; an 8 KB share a wave streams K faster than a 16 KB one.
// The query fragments are read from global memory once per workgroup and
// shared through LDS. The two halves' sums meet in LDS and are added in a
// fixed order, so the score is deterministic.
template <int D, int NRB, bool kPow2>
__device__ __forceinline__ void importance64_block(const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                                                   int64_t stride, float* __restrict__ scores, int R, int Hq,
                                                   int Hkv, float scale, int n_chunks, int bx, int g, int nbx) {
  constexpr int KS = D / 32, CHUNK = 64, NKB = CHUNK / 32;   // a wave's 16-key blocks
  ScoreTile* tiles = nullptr;                 // general G only: one tile per wave
  if constexpr (!kPow2) {
    __shared__ ScoreTile t[4];
    tiles = t;
  }
  const int G = Hq / Hkv, rows = R * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, quad = lane >> 4;

  __shared__ uint4 q_lds[NRB][KS][kWave];
  if (wave == 0) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int row = rb * 16 + col;
      const bool valid = row < rows;
      const int r = valid ? row / G : 0, h = g * G + (valid ? row % G : 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        q_lds[rb][ks][lane] = valid ? *reinterpret_cast<const uint4*>(q + ((int64_t)r * Hq + h) * D + ks * 32 + quad * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  bf16x8_t qb[NRB][KS];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[rb][ks] = __builtin_bit_cast(bf16x8_t, q_lds[rb][ks][lane]);
  const float inv = 1.f / (float)(CHUNK * R);
  __shared__ float half_sum[4];
  // workgroup iteration p covers chunks 2p and 2p + 1; every wave runs every
  // iteration (a wave past the last chunk only meets the barriers)
  const int n_pairs = (n_chunks + 1) / 2, half = wave & 1;
  for (int pr = bx; pr < n_pairs; pr += nbx) {
    const int c = 2 * pr + (wave >> 1);
    const bool live = c < n_chunks;
    const bf16_t* base = kc + ((int64_t)g * stride + (int64_t)min(c, n_chunks - 1) * CHUNK + half * 32) * D;
    bf16x8_t ka[NKB][KS];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[kb][ks] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(base + (int64_t)(kb * 16 + col) * D + ks * 32 + quad * 8));
    float tot = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][ks], qb[rb][ks], s, 0, 0, 0);
        // s[i]: key 16*kb + 4*quad + i, query row rb*16 + col
        if constexpr (kPow2) {
          // max over the G heads of a recent query = max over G adjacent columns (lanes)
          const int row = rb * 16 + col;
          const bool head0 = (row % G) == 0 && row < rows;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = s[i] * scale;
            for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
            tot += head0 ? v : 0.f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) tiles[wave].v[rb * 16 + col][4 * quad + i] = s[i] * scale;
        }
      }
      if constexpr (!kPow2) tot += tile_group_max_sum(tiles[wave], R, G, 16, lane);
    }
    tot = wave_sum(tot);
    if (lane == 0 && half == 1) half_sum[wave] = tot;
    __syncthreads();
    if (lane == 0 && half == 0 && live) scores[(int64_t)g * n_chunks + c] = (tot + half_sum[wave + 1]) * inv;
    __syncthreads();
  }
}

}  // namespace ts
