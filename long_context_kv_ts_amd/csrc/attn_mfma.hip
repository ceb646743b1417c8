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
// query row (row = lane % 32, 16 keys of a 32-key block; the other 16 are in
// lane ^ 32). Row max/sum are then per-lane with one cross-half exchange, and
// the output O^T = V^T . P^T again gives every lane one row, so rescaling O is
// a per-lane multiply. P^T reuses the score registers directly as the B
// operand: the reduction order over keys is free, so the V^T operand is read
// in the key order the scores arrive in -- k-slot 8*h + 4*r + e of a 16-key
// chunk is key 16*hh + 8*r + 4*h + e.
//
// K and V tiles (64 keys) stream from HBM straight into LDS with 16-byte
// global_load_lds_dwordx4 (no staging registers) through a 3-stage ring, so
// two tiles are in flight while one is computed; one barrier per tile. Both
// tiles are stored row-major with 16-byte chunks XOR-swizzled per row (K:
// chunk ^ row%16, V: chunk ^ 4*(row%4)): the K operand reads (16 rows, one
// chunk) and the transposing ds_read_b64_tr_b16 reads of V^T (4 rows x 32
// bytes per 16 lanes) are both free of bank conflicts. Rows past the valid
// keys re-read the last valid row (finite data, masked scores).
//
// Softmax in base 2 on fp32 scores (exact bf16 products, fp32 sums); scale is
// applied in fp32 after the product. The running max is only raised when a new
// score exceeds it by more than 2^8 ("lazy rescale"), which keeps every
// probability <= 256 and makes rescaling of the accumulators rare. The
// probabilities are rounded to bf16 for the PV product; the row sum uses the
// unrounded values. Tiles past the cache are the draft K/V, masked by the
// ancestor-or-self bitmask built in LDS from parent[].
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

typedef short s16x4_t __attribute__((ext_vector_type(4)));
#define TS_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kStages = 3;

template <int D> struct Layout {
  static constexpr int KS = D / 16;                  // k-steps of QK^T
  static constexpr int DB = D / 32;                  // 32-wide column blocks of O
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int tileElems = kTile * D;        // one K or V tile, unpadded
  static constexpr int loadsPerTensor = kTile * D * 2 / 1024;   // 1 KB per wave-wide load
  static constexpr int loadsPerWave = 2 * loadsPerTensor / kWaves;
  static constexpr int rowsPerLoad = 1024 / (D * 2);
};

// Physical 16-byte chunk of logical chunk c in row r.
template <int D> __device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & (Layout<D>::CH - 1)); }
template <int D> __device__ __forceinline__ int v_chunk(int r, int c) {
  return c ^ ((4 * (r & 3)) & (Layout<D>::CH - 1));
}

// One wave-wide 16-byte-per-lane load from global memory straight into LDS:
// lane l reads base + voff (base uniform, in SGPRs) and its 16 bytes land at
// lds + 16*l (lds uniform, passed in M0). Written as asm with no outputs so
// that the compiler does not guard every later LDS read with a wait for ALL
// outstanding loads; completion is instead awaited explicitly (vmcnt) before
// the barrier that publishes a tile. Loads the compiler does not count only
// make its own waits stricter.
__device__ __forceinline__ void lds_dma16(const bf16_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

// Per-lane byte offset, within a tile, of the row/chunk that load n of wave w
// fills. Load q = w*loadsPerWave + n covers 1 KB block m = q % loadsPerTensor
// of K (waves in the first half) or of V (second half); lane l fills row
// m*rowsPerLoad + l/CH, physical chunk l%CH, so it reads the logical chunk
// that the row's swizzle maps there. Rows past nvalid re-read row nvalid-1.
template <int D>
__device__ __forceinline__ uint32_t dma_offset(int wave, int n, int lane, int nvalid) {
  using Ly = Layout<D>;
  const int q = wave * Ly::loadsPerWave + n;
  const bool isv = q >= Ly::loadsPerTensor;
  const int mblk = isv ? q - Ly::loadsPerTensor : q;
  const int r = mblk * Ly::rowsPerLoad + lane / Ly::CH;
  const int pc = lane % Ly::CH;
  const int c = isv ? v_chunk<D>(r, pc) : k_chunk<D>(r, pc);   // xor: its own inverse
  return (uint32_t)((min(r, nvalid - 1) * D + c * 8) * 2);
}

// v_permlane32_swap(x, x) returns (x[l], x[l+32]) in lanes 0-31 and (x[l-32], x[l])
// in lanes 32-63: combining the pair gives lane l and lane l^32 without LDS.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_split_mfma_kernel(AttnArgs a) {
  using Ly = Layout<D>;
  __shared__ __attribute__((aligned(1024))) bf16_t KVs[kStages][2][Ly::tileElems];
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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps wave math scalar
  const int col = lane & 31, half = lane >> 5;
  const int G = a.G, T = a.T, Hq = a.Hq;
  const float c = a.scale_log2;

  const int vt0 = split * pl.tiles_per_split;
  const int vt1 = min(vt0 + pl.tiles_per_split, pl.n_virtual);

  // This wave streams K (first half of the waves) or V (second half).
  const bool wave_v = wave * Ly::loadsPerWave >= Ly::loadsPerTensor;
  const bf16_t* cache_base =
      static_cast<const bf16_t*>(wave_v ? a.vc : a.kc) + (int64_t)g * a.cache_stride * D;
  const bf16_t* draft_base = static_cast<const bf16_t*>(wave_v ? a.vd : a.kd) + (int64_t)g * T * D;
  uint32_t off_full[Ly::loadsPerWave];
#pragma unroll
  for (int n = 0; n < Ly::loadsPerWave; ++n) off_full[n] = dma_offset<D>(wave, n, lane, kTile);
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TS_LDS(void, &KVs[0][0][0])));
  auto issue = [&](int vt, int stage) {
    const bool draft = vt >= pl.n_cache_tiles;
    const int key0 = draft ? (vt - pl.n_cache_tiles) * kTile : vt * kTile;
    const int nvalid = draft ? min(kTile, T - key0) : (int)min((int64_t)kTile, a.L - key0);
    const bf16_t* base = (draft ? draft_base : cache_base) + (int64_t)key0 * D;
    auto lds_of = [&](int n) {
      const int q = wave * Ly::loadsPerWave + n;
      const int mblk = q >= Ly::loadsPerTensor ? q - Ly::loadsPerTensor : q;
      return lds_base + (uint32_t)(((stage * 2 + (wave_v ? 1 : 0)) * Ly::tileElems + mblk * 512) * 2);
    };
    if (__builtin_expect(nvalid == kTile, 1)) {
#pragma unroll
      for (int n = 0; n < Ly::loadsPerWave; ++n) lds_dma16(base, off_full[n], lds_of(n));
    } else {
#pragma unroll
      for (int n = 0; n < Ly::loadsPerWave; ++n)
        lds_dma16(base, dma_offset<D>(wave, n, lane, nvalid), lds_of(n));
    }
  };
  // the first tile starts streaming before anything else
  issue(vt0, 0);

  // ---- Q operand (B of S^T = K Q^T): lane holds row `col` of the block -----
  bf16x8_t qf[Ly::KS];
  const int row = rg * kRowsPerGroup + wave * 32 + col;
  const bool row_ok = row < pl.rows_per_head;
  const int row_t = row_ok ? row / G : 0;
  const int row_h = g * G + (row_ok ? row % G : 0);
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + ((int64_t)row_t * Hq + row_h) * D;
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) {
      uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qp + ks * 16 + half * 8)
                       : make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
    // Wait for Q here, once: the compiler would otherwise place its wait at the
    // first use inside the tile loop, where it would run every iteration and
    // drain the prefetched tiles too.
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) asm volatile("" : : "v"(qf[ks]));
  }
  if (vt0 + 1 < vt1) issue(vt0 + 1, 1);
  // waves whose rows are all padding skip the products
  const bool wave_active = rg * kRowsPerGroup + wave * 32 < pl.rows_per_head;

  const int words = (T + 31) >> 5;
  if (vt1 > pl.n_cache_tiles) build_ancestor_mask(a.parent, T, words, anc, tid, kThreads);

  f32x16_t O[Ly::DB];
#pragma unroll
  for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[db][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  for (int vt = vt0; vt < vt1; ++vt) {
    const int i = vt - vt0;
    const int cur = i % kStages;
    // this wave's loads of tile vt are the oldest outstanding; the next tile's
    // (if issued) may stay in flight
    if (vt + 1 < vt1) __builtin_amdgcn_s_waitcnt(0x0F70 | Ly::loadsPerWave);   // vmcnt(loadsPerWave)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                                   // vmcnt(0)
    __syncthreads();   // tile vt visible to all; stage (i+2)%3 no longer read
    if (vt + 2 < vt1) issue(vt + 2, (i + 2) % kStages);

    if (wave_active) {
      const bool draft = vt >= pl.n_cache_tiles;
      const int key0 = draft ? (vt - pl.n_cache_tiles) * kTile : vt * kTile;
      const int nvalid = draft ? min(kTile, T - key0) : (int)min((int64_t)kTile, a.L - key0);
      const bf16_t* Kc = KVs[cur][0];
      const bf16_t* Vc = KVs[cur][1];

      // One 32-key block at a time: S^T block, mask, softmax update, PV.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16_t S;
#pragma unroll
        for (int e = 0; e < 16; ++e) S[e] = 0.f;
        const int kr = 32 * kb + col;                       // K row read by this lane
#pragma unroll
        for (int ks = 0; ks < Ly::KS; ++ks) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
              Kc + kr * D + k_chunk<D>(kr, 2 * ks + half) * 8);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], S, 0, 0, 0);
        }

        // mask: ragged cache tail, draft ancestor bits
        if (draft || nvalid < kTile) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = 32 * kb + 8 * (e >> 2) + 4 * half + (e & 3);
            bool ok = key < nvalid;
            if (draft) {
              const int kk = key0 + key;
              ok = ok && row_ok && ((anc[row_t * words + (kk >> 5)] >> (kk & 31)) & 1u);
            }
            if (!ok) S[e] = -INFINITY;
          }
        }

        // online softmax (base 2, lazy rescale)
        float mx = S[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[e]);
        mx = max_xor32(mx) * c;                                  // same for lanes l, l^32
        const bool need = mx > m + kLazy;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
          // need implies mx finite; exp2(-inf) = 0 clears a row that had no key yet
          const float alpha = need ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
          m = need ? mx : m;
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[db][e] *= alpha;
        }
        // finite stand-in for a row with no key yet: exp2(-inf) = 0 for masked scores
        const float nmb = -fmaxf(m, -3.0e38f);
        bf16x8_t P[2];
        float ls = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // v_exp_f32 directly: results below 2^-126 of the running max flush to 0
            const float p = __builtin_amdgcn_exp2f(fmaf(S[8 * hh + e], c, nmb));
            ls += p;
            P[hh][e] = static_cast<__bf16>(p);
          }
        }
        lsum += ls;

        // O^T += V^T P^T over this block's 32 keys (two 16-key chunks). The
        // V^T operand of lane l: dim 32*db + l%32, keys 16*hh + 8*r + 4*h + e,
        // fetched by two transposing reads (r = 0, 1) of 4 keys each.
        const int vrow0 = 32 * kb + 4 * half + ((lane & 15) >> 2);
        const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
          for (int db = 0; db < Ly::DB; ++db) {
            s16x4_t part[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
              const int vr = vrow0 + 16 * hh + 8 * r;
              const int d = 32 * db + vdim;
              const bf16_t* vp = Vc + vr * D + v_chunk<D>(vr, d >> 3) * 8 + (d & 7);
              part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TS_LDS(s16x4_t, vp));
            }
            const s16x4_t lo = part[0], hi = part[1];
            const bf16x8_t vf = __builtin_bit_cast(
                bf16x8_t, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                                      hi[0], hi[1], hi[2], hi[3]});
            O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, P[hh], O[db], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue: normalise and write the split's partial ---------------------
  const float ltot = sum_xor32(lsum);
  if (row_ok) {
    const int64_t orow = ((int64_t)split * T + row_t) * Hq + row_h;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    float* op = a.o_part + orow * D;
#pragma unroll
    for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * half;
        float4 v = make_float4(O[db][4 * q4] * inv, O[db][4 * q4 + 1] * inv,
                               O[db][4 * q4 + 2] * inv, O[db][4 * q4 + 3] * inv);
        *reinterpret_cast<float4*>(op + d) = v;
      }
    if (half == 0) a.l_part[orow] = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

int mfma_rows_per_group() { return kRowsPerGroup; }
int mfma_tile_keys() { return kTile; }
int mfma_groups_per_cu() { return 1; }

hipError_t launch_attn_split_mfma(const AttnArgs& a, hipStream_t s) {
  const int R = a.plan.n_rowgroups;
  const int n_units = a.plan.n_splits * a.Hkv;
  const int blocks = ((n_units + 7) / 8) * 8 * R;
  if (a.D == 128) attn_split_mfma_kernel<128><<<blocks, kThreads, 0, s>>>(a);
  else attn_split_mfma_kernel<64><<<blocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ts
