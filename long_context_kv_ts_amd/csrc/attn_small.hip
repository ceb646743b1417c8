// Split-K masked attention for KV heads with at most 16 grouped query rows
// (bf16, v_mfma_f32_16x16x32_bf16): the 4-token self-drafting pass over the
// partial cache (4 tokens x 4 grouped heads), single-token decode, short
// verification passes.
//
// Every wave is one split: it owns a range of 64-key tiles of one KV head and
// keeps its own online-softmax state, so there are no workgroup barriers. A
// row is a (token t, query head h) pair, row = t*G + h%G; 16 rows = one MFMA
// tile. Per tile:
//   * S^T = K . Q^T: the K operand (16 keys x 32 dims per instruction) is
//     loaded from HBM straight into registers in the lane layout the
//     instruction wants (lane l: key l%16, dims 8*(l/16)..+7 of the step);
//   * V streams into this wave's LDS slice with global_load_lds_dwordx4
//     (rows XOR-swizzled by 16-byte chunk) and is read back transposed with
//     ds_read_b64_tr_b16 as the V^T operand of O^T = V^T . P^T;
//   * the S^T accumulators hold, per lane, one query row (l%16) and keys
//     4*(l/16)+i of each 16-key block, so a 32-key chunk of P^T is exactly the
//     lane's 8 values of two blocks (k-slot 8*g + e is key 16*(e/4)+4*g+e%4).
// Softmax in base 2 with lazy rescaling (probabilities <= 2^8), scale applied
// in fp32 after the product, P rounded to bf16 for PV, row sums unrounded.
//
// With kGather the partial cache is gathered on the way: cache tile i of a KV
// head is the chosen 64-token chunk of the full cache, read from there, and the
// wave also writes it to the partial cache -- K from the operand registers, V
// read back from its LDS slice -- so the chunk crosses HBM once on each side.
#include "common.h"

namespace ts {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#define TS_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kBlockWaves = 1;     // independent waves (splits) per workgroup: one spreads the
                                   // splits over the most compute units
constexpr int kThreads = kBlockWaves * 64;
constexpr int kSmallMaxDrafts = 16;  // this path serves heads of at most 16 query rows
constexpr float kLazy = 8.0f;

template <int D> struct SLayout {
  static constexpr int KS = D / 32;          // k-steps of QK^T (32 dims each)
  static constexpr int DB = D / 16;          // 16-dim blocks of O^T
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int tileElems = kTile * D;
  static constexpr int loads = kTile * D * 2 / 1024;   // wave-wide 1 KB loads per V tile
  static constexpr int rowsPerLoad = 1024 / (D * 2);
};

// V tile row r, logical chunk c -> physical chunk (conflict-free transposed reads)
template <int D> __device__ __forceinline__ int vs_chunk(int r, int c) {
  return c ^ ((2 * (r & 7)) & (SLayout<D>::CH - 1));
}

// M0 carries the wave-uniform LDS destination, set right before its one
// reader; the compiler emits no M0 access of its own in this kernel, so the
// clobber it does not honour for a reserved register leaves nothing unsaved.
__device__ __forceinline__ void lds_dma16(const bf16_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}

template <int D, bool kGather>
__global__ __launch_bounds__(kThreads) void attn_split_small_kernel(AttnArgs a) {
  using Ly = SLayout<D>;
  __shared__ __attribute__((aligned(1024))) bf16_t Vs[kBlockWaves][Ly::tileElems];
  // at most 16 query rows per head reach this kernel, so at most 16 drafts: one mask word each
  __shared__ uint32_t anc[kSmallMaxDrafts];
  __shared__ int32_t s_par[kSmallMaxDrafts];

  const AttnPlan& pl = a.plan;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.y;
  const int split = blockIdx.x * kBlockWaves + wave;
  const int G = a.G, T = a.T, Hq = a.Hq;
  const float c = a.scale_log2;

  // the mask is needed by the wave(s) whose range reaches the drafts
  const int last_split = min(blockIdx.x * kBlockWaves + kBlockWaves - 1, pl.n_splits - 1);
  const bool block_has_draft = (last_split + 1) * pl.tiles_per_split > pl.n_cache_tiles;
  const int words = (T + 31) >> 5;                 // 1
  if (block_has_draft) build_ancestor_rows(a.parent, words, 0, T, anc, s_par, tid, kThreads);
  if (split >= pl.n_splits) return;

  const int vt0 = split * pl.tiles_per_split;
  const int vt1 = min(vt0 + pl.tiles_per_split, pl.n_virtual);

  // Q operand (B of S^T = K Q^T): lane l holds row l%16, dims 32*ks + 8*(l/16)..+7
  const int col = lane & 15, grp = lane >> 4;
  const bool row_ok = col < pl.rows_per_head;
  const int row_t = row_ok ? col / G : 0;
  const int row_h = g * G + (row_ok ? col % G : 0);
  bf16x8_t qf[Ly::KS];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + ((int64_t)row_t * Hq + row_h) * D;
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) {
      const uint4 u = row_ok ? *reinterpret_cast<const uint4*>(qp + ks * 32 + grp * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
  }

  f32x4_t O[Ly::DB];
#pragma unroll
  for (int db = 0; db < Ly::DB; ++db) O[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  const uint32_t vlds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TS_LDS(void, &Vs[wave][0])));

  for (int vt = vt0; vt < vt1; ++vt) {
    const bool draft = vt >= pl.n_cache_tiles;
    const int key0 = draft ? (vt - pl.n_cache_tiles) * kTile : vt * kTile;
    const int nvalid = draft ? min(kTile, T - key0) : (int)min((int64_t)kTile, a.L - key0);
    // source rows of the tile: with kGather a cache tile is the chosen chunk of
    // the full cache (a whole tile: the partial cache is whole chunks)
    int64_t src0 = (int64_t)g * a.cache_stride + key0;
    bool zero_tile = false;                     // an out-of-range chunk index (wave-uniform)
    if constexpr (kGather) {
      if (!draft) {
        const int ci = a.gidx[(int64_t)g * pl.n_cache_tiles + vt];
        zero_tile = ci < 0 || (int64_t)ci >= a.g_chunks;
        src0 = (int64_t)g * a.cache_stride + (zero_tile ? 0 : (int64_t)ci * kTile);
      }
    }
    const bf16_t* kb = draft ? static_cast<const bf16_t*>(a.kd) + ((int64_t)g * T + key0) * D
                             : static_cast<const bf16_t*>(a.kc) + src0 * D;
    const bf16_t* vb = draft ? static_cast<const bf16_t*>(a.vd) + ((int64_t)g * T + key0) * D
                             : static_cast<const bf16_t*>(a.vc) + src0 * D;

    // V tile -> this wave's LDS slice (rows past nvalid re-read row nvalid-1)
    if (!zero_tile) {
#pragma unroll
      for (int n = 0; n < Ly::loads; ++n) {
        const int r = n * Ly::rowsPerLoad + lane / Ly::CH;
        const int cc = vs_chunk<D>(r, lane % Ly::CH);
        lds_dma16(vb, (uint32_t)((min(r, nvalid - 1) * D + cc * 8) * 2), vlds + n * 1024);
      }
    } else {
#pragma unroll
      for (int n = 0; n < Ly::loads; ++n)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(vlds + n * 1024 + lane * 16) =
            u32x4_t{0u, 0u, 0u, 0u};
    }
    // K operands straight from HBM: block j, step ks -> key 16*j + l%16
    bf16x8_t kf[4][Ly::KS];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(16 * j + col, nvalid - 1);
#pragma unroll
      for (int ks = 0; ks < Ly::KS; ++ks)
        kf[j][ks] = zero_tile ? __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u))
                              : __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                                 kb + (int64_t)key * D + ks * 32 + grp * 8));
    }
    // the gathered K chunk -> the partial cache (every key of a cache tile is valid)
    if constexpr (kGather) {
      if (!draft) {
        bf16_t* kp = static_cast<bf16_t*>(a.kp) + ((int64_t)g * a.L + key0) * D;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int ks = 0; ks < Ly::KS; ++ks)
            *reinterpret_cast<uint4*>(kp + (int64_t)(16 * j + col) * D + ks * 32 + grp * 8) =
                __builtin_bit_cast(uint4, kf[j][ks]);
      }
    }
    f32x4_t S[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      S[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < Ly::KS; ++ks)
        S[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j][ks], qf[ks], S[j], 0, 0, 0);
    }
    // mask: ragged tail, padding rows, draft ancestor bits
    if (draft || nvalid < kTile) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * j + 4 * grp + i;
          bool ok = key < nvalid;
          if (draft) {
            const int kk = key0 + key;
            ok = ok && row_ok && ((anc[row_t * words + (kk >> 5)] >> (kk & 31)) & 1u);
          }
          if (!ok) S[j][i] = -INFINITY;
        }
    }
    // row max over the 4 lane groups holding the row's keys
    float mx = S[0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[j][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c;
    const bool need = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
      m = need ? mx : m;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < Ly::DB; ++db) O[db] *= alpha;
    }
    const float nmb = -fmaxf(m, -3.0e38f);
    bf16x8_t P[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[2 * h + (e >> 2)][e & 3], c, nmb));
        lsum += p;
        P[h][e] = static_cast<__bf16>(p);
      }

    // the wave's own V loads have landed
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // the gathered V chunk -> the partial cache: each lane stores the 16-byte
    // pieces it brought into LDS, at the offsets it read them from
    if constexpr (kGather) {
      if (!draft) {
        uint8_t* vp = static_cast<uint8_t*>(a.vp) + ((int64_t)g * a.L + key0) * D * 2;
#pragma unroll
        for (int n = 0; n < Ly::loads; ++n) {
          const int r = n * Ly::rowsPerLoad + lane / Ly::CH;
          const int cc = vs_chunk<D>(r, lane % Ly::CH);
          const u32x4_t v = *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(vlds + n * 1024 + lane * 16);
          *reinterpret_cast<u32x4_t*>(vp + (r * D + cc * 8) * 2) = v;
        }
      }
    }
    // O^T += V^T P^T: for chunk h (keys 32h..32h+31) lane l needs dim 16*db + l%16
    // of keys 32h + 16*(e/4) + 4*(l/16) + e%4: two transposing reads of 4 keys
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int db = 0; db < Ly::DB; ++db) {
        s16x4_t part[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int vr = 32 * h + 16 * r + 4 * grp + (col >> 2);
          const int d = 16 * db + 4 * (col & 3);
          const bf16_t* vp = &Vs[wave][vr * D + vs_chunk<D>(vr, d >> 3) * 8 + (d & 7)];
          part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TS_LDS(s16x4_t, vp));
        }
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, (short __attribute__((ext_vector_type(8)))){part[0][0], part[0][1], part[0][2], part[0][3],
                                                                  part[1][0], part[1][1], part[1][2], part[1][3]});
        O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, P[h], O[db], 0, 0, 0);
      }
    }
    // all lanes' transposing reads done before the next tile's loads overwrite the slice
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  }

  // row sum over the 4 lane groups, then write the split's partial
  float ltot = lsum + __shfl_xor(lsum, 16, kWave);
  ltot += __shfl_xor(ltot, 32, kWave);
  if (row_ok) {
    const int64_t orow = ((int64_t)split * T + row_t) * Hq + row_h;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (a.o_part_h != nullptr) {
      // a call's own bf16 partials: half the bytes for its merge to read
      bf16_t* op = a.o_part_h + orow * D;
#pragma unroll
      for (int db = 0; db < Ly::DB; ++db) {
        const f32x4_t v = O[db] * inv;
        *reinterpret_cast<uint2*>(op + 16 * db + 4 * grp) = pack_bf16x4(v[0], v[1], v[2], v[3]);
      }
    } else {
      float* op = a.o_part + orow * D;
#pragma unroll
      for (int db = 0; db < Ly::DB; ++db) {
        const f32x4_t v = O[db] * inv;
        *reinterpret_cast<float4*>(op + 16 * db + 4 * grp) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    if (grp == 0) a.l_part[orow] = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_split_small(const AttnArgs& a, hipStream_t s) {
  if (a.T > kSmallMaxDrafts || a.plan.rows_per_head > 16) return hipErrorInvalidValue;   // the plan never sends these
  dim3 grid((a.plan.n_splits + kBlockWaves - 1) / kBlockWaves, a.Hkv);
  if (a.gidx != nullptr) {
    // the gathered cache is whole 64-token chunks, one tile each
    if (a.L % kTile != 0 || a.plan.n_cache_tiles * (int64_t)kTile != a.L) return hipErrorInvalidValue;
    if (a.D == 128) attn_split_small_kernel<128, true><<<grid, kThreads, 0, s>>>(a);
    else attn_split_small_kernel<64, true><<<grid, kThreads, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.D == 128) attn_split_small_kernel<128, false><<<grid, kThreads, 0, s>>>(a);
  else attn_split_small_kernel<64, false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ts
