// Matrix-core split-K masked attention for bf16 (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Work unit: (row group of 256 query rows, split, KV head). A row is a
// (draft token t, query head h) pair of the KV head's group, row = t*G + h%G,
// so the G grouped heads of one KV head share every K/V tile: 120 drafts x 4
// heads = 480 rows per KV head for a LLaMA3.1-8B layer. Eight waves (two per
// SIMD, so one wave's matrix products overlap the other's softmax), each owns
// one block of 32 rows; all eight read the same K/V tile from LDS.
//
// Scores are computed transposed, S^T = K . Q^T (A = K tile from LDS, B = Q
// held in registers), so each lane's accumulator values all belong to ONE
// query row (row = lane % 32 of the block, 16 keys per 32-key block, the other
// 16 in lane ^ 32). Row max/sum are then per-lane with one cross-half
// exchange, and the output O^T = V^T . P^T again gives every lane one row, so
// rescaling O is a per-lane multiply. P^T reuses the score registers
// directly as the B operand: the order of the reduction over keys is free, so
// the V^T operand is read in the matching key order. V^T is produced while
// staging (4x8 register transposes) into an LDS layout where that order is
// contiguous: column k' = 32*kb + 16*hh + 8*h + e holds key
// 32*kb + 16*hh + 8*(e/4) + 4*h + e%4.
//
// Softmax in base 2 on fp32 scores (exact bf16 products, fp32 sums); scale is
// applied in fp32 after the product. The running max is only raised when a new
// score exceeds it by more than 2^8 ("lazy rescale"), which keeps every
// probability <= 256 and makes rescaling of the accumulators rare. The
// probabilities are rounded to bf16 for the PV product; the row sum uses the
// unrounded values.
//
// K/V tiles of 64 keys are double-buffered in LDS: the global loads of tile
// i+1 are issued before the tile-i products and written to the other buffer
// after them; one barrier per tile. Tiles past the cache are the draft K/V,
// masked by the ancestor-or-self bitmask built in LDS from parent[].
#include "common.h"

namespace ts {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kWaves = 8;                    // 2 waves per SIMD: MFMA of one overlaps softmax of the other
constexpr int kNB = 1;                       // 32-row blocks per wave
constexpr int kRowsPerGroup = kWaves * kNB * 32;
constexpr float kLazy = 8.0f;                // log2 headroom before a rescale

template <int D> struct Layout {
  static constexpr int KS = D / 16;                  // k-steps of QK^T
  static constexpr int DB = D / 32;                  // 32-wide column blocks of O
  static constexpr int kRow = D + 8;                 // K tile row stride (bf16): +16 B
  static constexpr int vRow = kTile + 8;             // V^T row stride (bf16): 144 B
  static constexpr int kElems = kTile * kRow;
  static constexpr int vElems = D * vRow;
  static constexpr int vUnits = 2 * 8 * (D / 8);     // (key group, key half, 8-dim block) units of V
  static constexpr int kChunks = kTile * D / 8;      // 16-byte chunks of a K tile
  static constexpr int kThreadsK = kThreads - vUnits;
  static constexpr int kPer = (kChunks + kThreadsK - 1) / kThreadsK;
  static constexpr int nStage = kPer > 4 ? kPer : 4;
};

__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) {   // {a.lo, b.lo}
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) {   // {a.hi, b.hi}
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int D>
struct Stage {
  uint4 r[Layout<D>::nStage];   // V: 4 keys x 16 B  |  K: kPer chunks of 16 B
};

// V staging unit u: key group kg = u % 8 (= (kb, hh, h) of the V^T column
// order), key half eh = (u / 8) % 2, 8-dim block db = u / 16. It covers keys
// 32*kb + 16*hh + 4*h + 8*eh + i, i < 4, i.e. V^T columns kg*8 + eh*4 + i.
__device__ __forceinline__ int v_unit_key(int u, int i) {
  const int kg = u & 7, eh = (u >> 3) & 1;
  return 32 * (kg >> 2) + 16 * ((kg >> 1) & 1) + 4 * (kg & 1) + 8 * eh + i;
}

// Issue the global loads of one tile into registers (zeros past nvalid).
template <int D>
__device__ __forceinline__ void stage_load(Stage<D>& st, const bf16_t* kb, const bf16_t* vb,
                                           int nvalid, int tid) {
  using Ly = Layout<D>;
  if (tid < Ly::vUnits) {
    const int db = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = v_unit_key(tid, i);
      st.r[i] = key < nvalid ? *reinterpret_cast<const uint4*>(vb + (int64_t)key * D + db * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    const int kt = tid - Ly::vUnits;
#pragma unroll
    for (int n = 0; n < Ly::kPer; ++n) {
      const int j = kt + n * Ly::kThreadsK;          // chunk: key j/(D/8), 8-dim block j%(D/8)
      const int key = j / (D / 8), c8 = j % (D / 8);
      st.r[n] = (j < Ly::kChunks && key < nvalid)
                    ? *reinterpret_cast<const uint4*>(kb + (int64_t)key * D + c8 * 8)
                    : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Write staged registers into an LDS buffer: K row-major, V transposed
// (4x8 register transpose, 8-byte stores).
template <int D>
__device__ __forceinline__ void stage_store(const Stage<D>& st, bf16_t* Ks, bf16_t* Vt, int tid) {
  using Ly = Layout<D>;
  if (tid < Ly::vUnits) {
    const int kg = tid & 7, eh = (tid >> 3) & 1, db = tid >> 4;
    uint32_t w[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i][0] = st.r[i].x; w[i][1] = st.r[i].y; w[i][2] = st.r[i].z; w[i][3] = st.r[i].w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int src = j >> 1;
      uint2 o;
      if (j & 1) {
        o.x = perm_hi(w[0][src], w[1][src]); o.y = perm_hi(w[2][src], w[3][src]);
      } else {
        o.x = perm_lo(w[0][src], w[1][src]); o.y = perm_lo(w[2][src], w[3][src]);
      }
      *reinterpret_cast<uint2*>(Vt + (db * 8 + j) * Ly::vRow + kg * 8 + eh * 4) = o;
    }
  } else {
    const int kt = tid - Ly::vUnits;
#pragma unroll
    for (int n = 0; n < Ly::kPer; ++n) {
      const int j = kt + n * Ly::kThreadsK;
      if (j < Ly::kChunks) {
        const int key = j / (D / 8), c8 = j % (D / 8);
        *reinterpret_cast<uint4*>(Ks + key * Ly::kRow + c8 * 8) = st.r[n];
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_split_mfma_kernel(AttnArgs a) {
  using Ly = Layout<D>;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][Ly::kElems];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][Ly::vElems];
  __shared__ uint32_t anc[TS_MAX_DRAFT * (TS_MAX_DRAFT / 32)];

  const AttnPlan& pl = a.plan;
  // XCD-aware order: workgroups i and i+8 run on the same XCD (L2). The row
  // groups of one (split, head) unit -- which read the same K/V tiles -- are
  // placed 8 ids apart.
  const int R = pl.n_rowgroups;
  const int id = blockIdx.x;
  const int unit = (id / (8 * R)) * 8 + (id % 8);
  const int rg = (id % (8 * R)) / 8;
  const int n_units = pl.n_splits * a.Hkv;
  if (unit >= n_units) return;
  const int split = unit % pl.n_splits, g = unit / pl.n_splits;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.G, T = a.T, Hq = a.Hq;
  const float c = a.scale_log2;

  // ---- Q operand (B of S^T = K Q^T): lane holds row col of each block ------
  bf16x8_t qf[kNB][Ly::KS];
  bool row_ok[kNB];
  int row_t[kNB], row_h[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int row = rg * kRowsPerGroup + wave * (kNB * 32) + b * 32 + col;
    row_ok[b] = row < pl.rows_per_head;
    row_t[b] = row_ok[b] ? row / G : 0;
    row_h[b] = g * G + (row_ok[b] ? row % G : 0);
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + ((int64_t)row_t[b] * Hq + row_h[b]) * D;
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) {
      uint4 u = row_ok[b] ? *reinterpret_cast<const uint4*>(qp + ks * 16 + half * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
      qf[b][ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  // waves whose row blocks are all padding skip the products
  const bool wave_active = rg * kRowsPerGroup + wave * (kNB * 32) < pl.rows_per_head;

  const int vt0 = split * pl.tiles_per_split;
  const int vt1 = min(vt0 + pl.tiles_per_split, pl.n_virtual);
  const int words = (T + 31) >> 5;
  if (vt1 > pl.n_cache_tiles) build_ancestor_mask(a.parent, T, words, anc, tid, kThreads);

  auto tile_ptrs = [&](int vt, const bf16_t*& kb, const bf16_t*& vb, int& key0, int& nvalid) {
    const bool draft = vt >= pl.n_cache_tiles;
    key0 = draft ? (vt - pl.n_cache_tiles) * kTile : vt * kTile;
    nvalid = draft ? min(kTile, T - key0) : (int)min((int64_t)kTile, a.L - key0);
    kb = draft ? static_cast<const bf16_t*>(a.kd) + ((int64_t)g * T + key0) * D
               : static_cast<const bf16_t*>(a.kc) + ((int64_t)g * a.cache_stride + key0) * D;
    vb = draft ? static_cast<const bf16_t*>(a.vd) + ((int64_t)g * T + key0) * D
               : static_cast<const bf16_t*>(a.vc) + ((int64_t)g * a.cache_stride + key0) * D;
  };

  f32x16_t O[kNB][Ly::DB];
  float m[kNB], lsum[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    m[b] = -INFINITY;
    lsum[b] = 0.f;
#pragma unroll
    for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[b][db][i] = 0.f;
  }

  Stage<D> st;
  {
    const bf16_t *kb, *vb;
    int key0, nvalid;
    tile_ptrs(vt0, kb, vb, key0, nvalid);
    stage_load<D>(st, kb, vb, nvalid, tid);
    stage_store<D>(st, Ks[0], Vt[0], tid);
  }
  __syncthreads();

  for (int vt = vt0; vt < vt1; ++vt) {
    const int cur = (vt - vt0) & 1;
    if (vt + 1 < vt1) {
      const bf16_t *kb, *vb;
      int key0, nvalid;
      tile_ptrs(vt + 1, kb, vb, key0, nvalid);
      stage_load<D>(st, kb, vb, nvalid, tid);
    }
    if (wave_active) {
      const bool draft = vt >= pl.n_cache_tiles;
      const int key0 = draft ? (vt - pl.n_cache_tiles) * kTile : vt * kTile;
      const int nvalid = draft ? min(kTile, T - key0) : (int)min((int64_t)kTile, a.L - key0);
      const bf16_t* Kc = Ks[cur];
      const bf16_t* Vc = Vt[cur];

      // One 32-key block at a time: S^T block, mask, softmax update, PV.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16_t S[kNB];
#pragma unroll
        for (int b = 0; b < kNB; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) S[b][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < Ly::KS; ++ks) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
              Kc + (32 * kb + col) * Ly::kRow + ks * 16 + half * 8);
#pragma unroll
          for (int b = 0; b < kNB; ++b)
            S[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[b][ks], S[b], 0, 0, 0);
        }

        // mask: ragged cache tail, draft ancestor bits
        if (draft || nvalid < kTile) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
              bool ok = key < nvalid;
              if (draft) {
                const int kk = key0 + key;
                ok = ok && row_ok[b] && ((anc[row_t[b] * words + (kk >> 5)] >> (kk & 31)) & 1u);
              }
              if (!ok) S[b][i] = -INFINITY;
            }
          }
        }

        // online softmax (base 2, lazy rescale)
        bf16x8_t P[kNB][2];
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          float mx = S[b][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[b][i]);
          mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c;        // same for lanes l, l^32
          const bool need = mx > m[b] + kLazy;
          if (__builtin_amdgcn_ballot_w64(need) != 0) {
            // need implies mx finite; exp2(-inf) = 0 clears a row that had no key yet
            const float alpha = need ? __builtin_amdgcn_exp2f(m[b] - mx) : 1.f;
            m[b] = need ? mx : m[b];
            lsum[b] *= alpha;
#pragma unroll
            for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) O[b][db][i] *= alpha;
          }
          // finite stand-in for a row with no key yet: exp2(-inf) = 0 for masked scores
          const float nmb = -fmaxf(m[b], -3.0e38f);
          float ls = 0.f;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            bf16x8_t pv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              // v_exp_f32 directly: results below 2^-126 of the running max flush to 0
              const float p = __builtin_amdgcn_exp2f(fmaf(S[b][8 * hh + e], c, nmb));
              ls += p;
              pv[e] = static_cast<__bf16>(p);
            }
            P[b][hh] = pv;
          }
          lsum[b] += ls;
        }

        // O^T += V^T P^T over this block's 32 keys (two 16-key k-chunks)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int db = 0; db < Ly::DB; ++db) {
            const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(
                Vc + (32 * db + col) * Ly::vRow + 32 * kb + 16 * hh + half * 8);
#pragma unroll
            for (int b = 0; b < kNB; ++b)
              O[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, P[b][hh], O[b][db], 0, 0, 0);
          }
        }
      }
    }
    if (vt + 1 < vt1) stage_store<D>(st, Ks[cur ^ 1], Vt[cur ^ 1], tid);
    __syncthreads();
  }

  // ---- epilogue: normalise and write the split's partial ---------------------
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const float ltot = lsum[b] + __shfl_xor(lsum[b], 32, kWave);
    if (!row_ok[b]) continue;
    const int64_t orow = ((int64_t)split * T + row_t[b]) * Hq + row_h[b];
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float* op = a.o_part + orow * D;
#pragma unroll
    for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * half;
        float4 v = make_float4(O[b][db][4 * q4] * inv, O[b][db][4 * q4 + 1] * inv,
                               O[b][db][4 * q4 + 2] * inv, O[b][db][4 * q4 + 3] * inv);
        *reinterpret_cast<float4*>(op + d) = v;
      }
    if (half == 0) a.l_part[orow] = ltot > 0.f ? (m[b] + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

int mfma_rows_per_group() { return kRowsPerGroup; }

hipError_t launch_attn_split_mfma(const AttnArgs& a, hipStream_t s) {
  const int R = a.plan.n_rowgroups;
  const int n_units = a.plan.n_splits * a.Hkv;
  const int blocks = ((n_units + 7) / 8) * 8 * R;
  if (a.D == 128) attn_split_mfma_kernel<128><<<blocks, kThreads, 0, s>>>(a);
  else attn_split_mfma_kernel<64><<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ts
