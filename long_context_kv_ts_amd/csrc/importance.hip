// Chunk importance for the dynamic partial KV cache.
//
// For KV head g and chunk c of `chunk` consecutive cached tokens:
//   u[r, j]  = max over the G query heads of group g of  scale * <q[r,h], k[g,j]>
//   score    = mean over recent queries r and tokens j of the chunk of u[r, j]
// Only K is read (V is never touched), once, in 16-byte coalesced loads.
//
// bf16, D = 128 or 64, R*G <= 64: matrix-core path. The scores of a 16-key block
// against all R*G query rows are one v_mfma_f32_16x16x32_bf16 chain per 16
// rows, computed transposed (S^T = K Q^T) so that the K operand is loaded
// straight from HBM into registers in the lane layout the instruction wants
// and never passes through LDS. A wave owns one chunk at a time (64-token
// chunks: half a chunk, 32 keys, with the query fragments shared through LDS
// by the workgroup). With G a
// power of two a query's G heads are G aligned adjacent columns and their max
// is a lane butterfly; other G (5, 6, 7 ... 15) pass the block's scores
// through a per-wave LDS tile and each lane takes the max over its query's G
// rows for one (query, key) pair.
// fp32 (or other shapes): vector-ALU path with the query rows in LDS.
#include "importance_block.h"

namespace ts {
namespace {


// ---------------------------------------------------------------------------
// vector-ALU path
// ---------------------------------------------------------------------------
template <typename Tin, int D>
__global__ __launch_bounds__(256) void importance_valu_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ kc, int64_t stride,
    float* __restrict__ scores, int R, int Hq, int Hkv, int chunk, float scale, int n_chunks) {
  __shared__ float Qs[64][D];
  const int g = blockIdx.y, G = Hq / Hkv, rows = R * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < rows * D; i += 256) {
    const int row = i / D, d = i % D, r = row / G, h = g * G + row % G;
    Qs[row][d] = Elem<Tin>::load(q + ((int64_t)r * Hq + h) * D + d) * scale;
  }
  __syncthreads();
  const int c = blockIdx.x * 4 + wave;
  if (c >= n_chunks) return;
  float tot = 0.f;
  for (int j = lane; j < chunk; j += kWave) {
    const Tin* kp = kc + ((int64_t)g * stride + (int64_t)c * chunk + j) * D;
    float kr[D];
#pragma unroll
    for (int d = 0; d < D; d += 8) load8(kp + d, kr + d);
    for (int r = 0; r < R; ++r) {
      float best = -INFINITY;
      for (int hl = 0; hl < G; ++hl) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s += Qs[r * G + hl][d] * kr[d];
        best = fmaxf(best, s);
      }
      tot += best;
    }
  }
  tot = wave_sum(tot);
  if (lane == 0) scores[(int64_t)g * n_chunks + c] = tot / (float)(chunk * R);
}

// ---------------------------------------------------------------------------
// matrix-core path (bf16); the operand layout is described in importance_block.h
// ---------------------------------------------------------------------------
template <int D, int NRB, bool kPow2>
__global__ __launch_bounds__(256) void importance_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, int64_t stride,
    float* __restrict__ scores, int R, int Hq, int Hkv, int chunk, float scale, int n_chunks) {
  constexpr int KS = D / 32;                  // reduction steps per 16x16 block
  ScoreTile* tiles = nullptr;                 // general G only: one tile per wave
  if constexpr (!kPow2) {
    __shared__ ScoreTile t[4];
    tiles = t;
  }
  const int g = blockIdx.y, G = Hq / Hkv, rows = R * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, quad = lane >> 4;

  // B operands: query rows (row = r*G + hl) scaled, rounded back to bf16.
  bf16x8_t qb[NRB][KS];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = rb * 16 + col;
    const bool valid = row < rows;
    const int r = valid ? row / G : 0, h = g * G + (valid ? row % G : 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t v;
      const bf16_t* p = q + ((int64_t)r * Hq + h) * D + ks * 32 + quad * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(valid ? bf16_to_f32(p[e]) : 0.f);
      qb[rb][ks] = v;
    }
  }

  const int waves_total = gridDim.x * 4;
  for (int c = blockIdx.x * 4 + wave; c < n_chunks; c += waves_total) {
    const bf16_t* base = kc + ((int64_t)g * stride + (int64_t)c * chunk) * D;
    float tot = 0.f;
    for (int kb = 0; kb < chunk; kb += 16) {
      // this lane's key of the block; keys past the chunk contribute nothing
      const int key = kb + col;
      bf16x8_t ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (key < chunk) {
          uint4 u = *reinterpret_cast<const uint4*>(base + (int64_t)key * D + ks * 32 + quad * 8);
          ka[ks] = __builtin_bit_cast(bf16x8_t, u);
        } else {
          ka[ks] = bf16x8_t{};
        }
      }
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[rb][ks], s, 0, 0, 0);
        // s[i]: key kb + 4*quad + i, query row rb*16 + col
        if constexpr (kPow2) {
          // max over the G heads of a recent query = max over G adjacent columns (lanes)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = s[i] * scale;
            for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
            const int row = rb * 16 + col;
            const bool head0 = (row % G) == 0 && row < rows && (kb + 4 * quad + i) < chunk;
            tot += head0 ? v : 0.f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) tiles[wave].v[rb * 16 + col][4 * quad + i] = s[i] * scale;
        }
      }
      if constexpr (!kPow2) tot += tile_group_max_sum(tiles[wave], R, G, min(16, chunk - kb), lane);
    }
    tot = wave_sum(tot);
    if (lane == 0) scores[(int64_t)g * n_chunks + c] = tot / (float)(chunk * R);
  }
}

template <int D, int NRB, bool kPow2>
__global__ __launch_bounds__(256) void importance_mfma64_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, int64_t stride,
    float* __restrict__ scores, int R, int Hq, int Hkv, float scale, int n_chunks) {
  importance64_block<D, NRB, kPow2>(q, kc, stride, scores, R, Hq, Hkv, scale, n_chunks, blockIdx.x, blockIdx.y,
                                    gridDim.x);
}

template <int D, bool kPow2>
hipError_t launch_mfma_g(const bf16_t* q, const bf16_t* kc, int64_t stride, float* scores, int R,
                         int Hq, int Hkv, int chunk, float scale, int n_chunks, hipStream_t s) {
  const int rows = R * (Hq / Hkv);
  // 64-token chunks: two chunks a workgroup; otherwise one chunk a wave
  // (workgroups stride over chunks only past 65535 of them)
  int blocks_x = chunk == 64 ? (n_chunks + 1) / 2 : (n_chunks + 3) / 4;
  if (blocks_x > 65535) blocks_x = 65535;
  dim3 grid(blocks_x, Hkv);
  if (chunk == 64) {
    if (rows <= 16)
      importance_mfma64_kernel<D, 1, kPow2><<<grid, 256, 0, s>>>(q, kc, stride, scores, R, Hq, Hkv, scale, n_chunks);
    else if (rows <= 32)
      importance_mfma64_kernel<D, 2, kPow2><<<grid, 256, 0, s>>>(q, kc, stride, scores, R, Hq, Hkv, scale, n_chunks);
    else
      importance_mfma64_kernel<D, 4, kPow2><<<grid, 256, 0, s>>>(q, kc, stride, scores, R, Hq, Hkv, scale, n_chunks);
    return hipGetLastError();
  }
  if (rows <= 16)
    importance_mfma_kernel<D, 1, kPow2><<<grid, 256, 0, s>>>(q, kc, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks);
  else if (rows <= 32)
    importance_mfma_kernel<D, 2, kPow2><<<grid, 256, 0, s>>>(q, kc, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks);
  else
    importance_mfma_kernel<D, 4, kPow2><<<grid, 256, 0, s>>>(q, kc, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const bf16_t* q, const bf16_t* kc, int64_t stride, float* scores, int R,
                       int Hq, int Hkv, int chunk, float scale, int n_chunks, hipStream_t s) {
  const int G = Hq / Hkv;
  if ((G & (G - 1)) == 0) return launch_mfma_g<D, true>(q, kc, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks, s);
  return launch_mfma_g<D, false>(q, kc, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks, s);
}

}  // namespace

hipError_t launch_importance(const void* q, const void* kc, int64_t stride, float* scores,
                             int R, int Hq, int Hkv, int D, int64_t L, int chunk, float scale,
                             ts_dtype dtype, hipStream_t s) {
  const int n_chunks = (int)(L / chunk);
  if (n_chunks == 0) return hipSuccess;
  if (dtype == TS_BF16) {
    const bf16_t* qb = static_cast<const bf16_t*>(q);
    const bf16_t* kb = static_cast<const bf16_t*>(kc);
    if (D == 128) return launch_mfma<128>(qb, kb, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks, s);
    return launch_mfma<64>(qb, kb, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks, s);
  }
  dim3 grid((n_chunks + 3) / 4, Hkv);
  const float* qf = static_cast<const float*>(q);
  const float* kf = static_cast<const float*>(kc);
  if (D == 128)
    importance_valu_kernel<float, 128><<<grid, 256, 0, s>>>(qf, kf, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks);
  else
    importance_valu_kernel<float, 64><<<grid, 256, 0, s>>>(qf, kf, stride, scores, R, Hq, Hkv, chunk, scale, n_chunks);
  return hipGetLastError();
}

}  // namespace ts
