// Matrix-core split-K masked attention for bf16 (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Work unit: (row group of 256 query rows, split, KV head). A row is a
// (draft token t, query head h) pair of the KV head's group, row = t*G + h%G,
// so the G grouped heads of one KV head share every K/V tile: 120 drafts x 4
// heads = 480 rows per KV head for a LLaMA3.1-8B layer. Eight waves, two per
// SIMD, each own one block of 32 rows; all eight read the same K/V tile from
// LDS.
//
// Scores are computed transposed, S^T = K . Q^T (A = K tile from LDS, B = Q
// held in registers), so each lane's accumulator values all belong to ONE
// query row (row = lane % 32, 16 keys of a 32-key tile; the other 16 are in
// lane ^ 32). Row max/sum are then per-lane with one cross-half exchange
// (v_permlane32_swap), and O^T = V^T . P^T again gives every lane one row, so
// rescaling O is a per-lane multiply. P^T reuses the score registers directly
// as the B operand: the reduction order over keys is free, so the V^T operand
// is read in the key order the scores arrive in -- k-slot 8*h + 4*r + e of a
// 16-key chunk is key 16*hh + 8*r + 4*h + e.
//
// Schedule. A single wave can neither issue vector-ALU work nor matrix
// products at the SIMD's full rate, and the softmax of a 32x32 block costs
// about as many issue cycles as its 16 products, so each wave is
// software-pipelined over 32-key tiles: iteration j issues QK^T(j+1) and
// PV(j-1) on the matrix cores interleaved with the softmax of tile j on the
// vector ALUs, and the two waves of a SIMD fill each other's gaps. The K and
// V^T operands of the next iteration are read from LDS right after the
// products that last used their registers. The order of the products, the
// exponentials and the operand reads inside an iteration is the compiler's
// matrix/exponential interleave strategy (iglp_opt 2), which took the timed
// decode step 2-3% below a hand-placed pattern of scheduling groups, with
// the same instructions and bit-identical results.
//
// Tiles stream from HBM straight into LDS with 16-byte global_load_lds_dwordx4
// (no staging registers) through an 8-stage ring (7 when a head's mask of more
// than 256 drafts takes the LDS), tile j + stages - 2 issued while tile j is
// computed. K tiles of all stages come first, then the V tiles, so
// every operand read is a per-lane base plus an immediate offset. Rows are
// stored with 16-byte chunks XOR-swizzled per row (K: chunk ^ row%16, V:
// chunk ^ 4*(row%4)), which keeps the K operand reads (32 rows, one chunk)
// and the transposing ds_read_b64_tr_b16 reads of V^T free of bank conflicts.
// The ring's depth lets the steady-state barrier skip the LDS drain: the stage
// it hands to the next load was last read two iterations earlier, and those
// reads were consumed by products before the barrier. Tiles past the last
// full cache tile (a ragged tail, the drafts) are masked and form a suffix of
// the split; they run unpipelined after it.
//
// Softmax in base 2 on fp32 scores (exact bf16 products, fp32 sums); scale is
// applied in fp32 after the product. The running max m is only raised when a
// new score exceeds it by more than 2^8 ("lazy rescale"), which makes
// rescaling of the accumulators rare. In the steady state the probabilities
// are formed against the current m without a row maximum at all: a lane whose
// 16 probabilities of a tile sum to more than 2^12 (one of them is then above
// 2^8, or m is still -inf) flags the wave, which redoes that tile with the row
// maximum before its probabilities are used; otherwise every probability stays
// below 2^12. The probabilities are rounded to bf16 for the PV product; the
// row sum uses the unrounded values. Draft tiles are masked by the
// ancestor-or-self bitmask built in LDS from parent[] (a 32-key tile is one
// word of a row's mask).
//
// Chunk importance on the same reads (kImp). When the last row group of a KV
// head ends in a wave that holds no query row (480 rows = 256 + 224 for the
// LLaMA3.1-8B layer), that wave scores 64-token chunks of the cache for the R
// recent queries instead: its Q operand holds the R*G recent query rows and it
// runs S = Q . K^T (untransposed: the same register operands in the other
// order) on the K tiles already in LDS, skipping PV. A lane then holds one key
// and 16 query rows, a recent query's G heads being G consecutive registers,
// so the maximum over the heads and the sum over the queries are in-lane;
// every second tile completes a chunk, whose mean the wave reduces with DPP
// and writes. Splits then start on even tiles (64-token chunks).
#include "common.h"
#include <type_traits>

namespace ts {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
#define TS_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (vmcnt is split over bits 3:0 and 15:14; lgkmcnt and expcnt left
// at their maxima)
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kKeys = 32;
constexpr float kLazy = 8.0f;

template <int D, int kWaves> struct Layout {
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CH = D / 8;
  static constexpr int tileElems = kKeys * D;
  static constexpr int loadsPerTensor = kKeys * D * 2 / 1024;
  static constexpr int loadsPerWave = 2 * loadsPerTensor / kWaves;
  static constexpr int rowsPerLoad = 1024 / (D * 2);
};

template <int D> __device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & (D / 8 - 1)); }
template <int D> __device__ __forceinline__ int v_chunk(int r, int c) { return c ^ ((4 * (r & 3)) & (D / 8 - 1)); }

// The base address and the LDS destination are wave-uniform; they are passed
// through readfirstlane so that they stay scalar operands even where the
// compiler cannot prove it (free when they already live in scalar registers).
// M0 carries the LDS destination: the statement sets it right before its one
// reader. The compiler does not save a reserved register named as clobbered
// (it warns so); in these kernels it emits no M0 access of its own, so there
// is nothing of its to save. Written as asm, not as the compiler's builtin for
// this load, because the compiler would then put a wait for every DMA in
// flight before each LDS read it cannot tell apart from the ring's stages.
__device__ __forceinline__ void lds_dma16(const bf16_t* base, uint32_t voff, uint32_t lds) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(reinterpret_cast<const bf16_t*>(bs)), "s"(ls)
               : "memory", "m0");
}

template <int D, int kWaves>
__device__ __forceinline__ uint32_t dma_offset(int wave, int n, int lane, int nvalid) {
  using Ly = Layout<D, kWaves>;
  const int q = wave * Ly::loadsPerWave + n;
  const bool isv = q >= Ly::loadsPerTensor;
  const int mblk = isv ? q - Ly::loadsPerTensor : q;
  const int r = mblk * Ly::rowsPerLoad + lane / Ly::CH;
  const int pc = lane % Ly::CH;
  const int c = isv ? v_chunk<D>(r, pc) : k_chunk<D>(r, pc);
  return (uint32_t)((min(r, nvalid - 1) * D + c * 8) * 2);
}

__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool B> using Flag = std::integral_constant<bool, B>;

// Lane exchange within quads of lanes (DPP quad_perm).
template <int kCtrl>
__device__ __forceinline__ float quad_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// kStages-deep ring of K/V tiles; kMaxT drafts at most. Eight stages fit next to
// the mask of up to 256 drafts, seven next to the mask of up to 1024. kWaves
// waves of 32 rows each: 8 (two per SIMD), or 4 when a KV head has at most 128
// rows (one query head per KV head), which would leave half of 8 waves idle.
// Registers are budgeted for two waves per SIMD in both forms (8 / kWaves
// workgroups a CU): one wave per SIMD may take 512 registers, and the compiler
// then parks values in AGPRs and moves them back and forth in the loop.
template <int D, int kStages, int kMaxT, int kWaves, bool kImp>
__global__ __launch_bounds__(kWaves * 64, 8 / kWaves) void attn_split_mfma_kernel(AttnArgs a) {
  constexpr int kThreads = kWaves * 64;
  constexpr int kRowsPerGroup = kWaves * 32;
  using Ly = Layout<D, kWaves>;
  // tiles issued ahead of the one being computed: the ring minus the tile being
  // read and the one being published
  constexpr int kAhead = kStages - 2;
  // K tiles of every stage, then V tiles: operand reads are a per-lane base
  // plus an immediate (stage * tile bytes + row offsets), all below 64 KB
  static_assert((kStages - 1) * Ly::tileElems * 2 + 24 * D * 2 < 65536, "ds_read offset");
  __shared__ __attribute__((aligned(1024))) bf16_t Ks[kStages][Ly::tileElems];
  __shared__ __attribute__((aligned(1024))) bf16_t Vs[kStages][Ly::tileElems];
  // ancestor rows of this row group's drafts (at most 256 of them) and the staged forest
  __shared__ uint32_t anc[kRowsPerGroup * (kMaxT / 32)];
  __shared__ int32_t s_par[kMaxT];

  const AttnPlan& pl = a.plan;
  const int R = pl.n_rowgroups;
  const int id = blockIdx.x;
  const int unit = (id / (8 * R)) * 8 + (id % 8);
  const int rg = (id % (8 * R)) / 8;
  const int n_units = pl.n_splits * a.Hkv;
  if (unit >= n_units) return;
  const int split = unit % pl.n_splits, g = unit / pl.n_splits;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int G = a.G, T = a.T, Hq = a.Hq;
  const float c = a.scale_log2;

  const int vt0 = split * pl.tiles_per_split;
  const int vt1 = min(vt0 + pl.tiles_per_split, pl.n_virtual);
  const int nb = vt1 - vt0;

  const bool wave_v = wave * Ly::loadsPerWave >= Ly::loadsPerTensor;
  const bf16_t* cache_base =
      static_cast<const bf16_t*>(wave_v ? a.vc : a.kc) + (int64_t)g * a.cache_stride * D;
  const bf16_t* draft_base = static_cast<const bf16_t*>(wave_v ? a.vd : a.kd) + (int64_t)g * T * D;
  uint32_t off_full[Ly::loadsPerWave];
#pragma unroll
  for (int n = 0; n < Ly::loadsPerWave; ++n) off_full[n] = dma_offset<D, kWaves>(wave, n, lane, kKeys);
  const uint32_t k_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TS_LDS(void, &Ks[0][0])));
  const uint32_t v_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(TS_LDS(void, &Vs[0][0])));
  constexpr uint32_t kTileBytes = Ly::tileElems * 2;
  const uint32_t my_lds = wave_v ? v_lds : k_lds;     // this wave's DMA destination tensor
  auto tile_keys = [&](int vt, int& key0, int& nvalid) {
    const bool draft = vt >= pl.n_cache_tiles;
    key0 = draft ? (vt - pl.n_cache_tiles) * kKeys : vt * kKeys;
    nvalid = draft ? min(kKeys, T - key0) : (int)min((int64_t)kKeys, a.L - key0);
    return draft;
  };
  auto issue = [&](int j) {          // tile j of this split -> stage j % kStages
    int key0, nvalid;
    const bool draft = tile_keys(vt0 + j, key0, nvalid);
    const bf16_t* base = (draft ? draft_base : cache_base) + (int64_t)key0 * D;
    const uint32_t sb = my_lds + (uint32_t)(j % kStages) * kTileBytes;
    auto lds_of = [&](int n) {
      const int q = wave * Ly::loadsPerWave + n;
      const int mblk = q >= Ly::loadsPerTensor ? q - Ly::loadsPerTensor : q;
      return sb + (uint32_t)(mblk * 1024);
    };
    if (__builtin_expect(nvalid == kKeys, 1)) {
#pragma unroll
      for (int n = 0; n < Ly::loadsPerWave; ++n) lds_dma16(base, off_full[n], lds_of(n));
    } else {
#pragma unroll
      for (int n = 0; n < Ly::loadsPerWave; ++n)
        lds_dma16(base, dma_offset<D, kWaves>(wave, n, lane, nvalid), lds_of(n));
    }
  };
  // tiles [0, issued) of this split have been issued (uniform)
  int issued = 0;
  auto issue_upto = [&](int limit) {    // issue the next tile if it is <= limit
    if (issued < nb && issued <= limit) {
      issue(issued);
      ++issued;
    }
  };
  // wait until tile j has landed; younger tiles may stay in flight
  auto wait_for = [&](int j) {
    const int after = issued - 1 - j;
    if (after >= 5) __builtin_amdgcn_s_waitcnt(vm_wait(5 * Ly::loadsPerWave));
    else if (after == 4) __builtin_amdgcn_s_waitcnt(vm_wait(4 * Ly::loadsPerWave));
    else if (after == 3) __builtin_amdgcn_s_waitcnt(vm_wait(3 * Ly::loadsPerWave));
    else if (after == 2) __builtin_amdgcn_s_waitcnt(vm_wait(2 * Ly::loadsPerWave));
    else if (after == 1) __builtin_amdgcn_s_waitcnt(vm_wait(Ly::loadsPerWave));
    else __builtin_amdgcn_s_waitcnt(vm_wait(0));
  };

  // ---- Q operand: lane holds row `col` of this wave's 32-row block -----------
  bf16x8_t qf[Ly::KS];
  const int row = rg * kRowsPerGroup + wave * 32 + col;
  const bool row_ok = row < pl.rows_per_head;
  const int row_t = row_ok ? row / G : 0;
  const int row_h = g * G + (row_ok ? row % G : 0);
  // the importance wave: the last wave of the last row group, holding no query row
  bool imp = false;
  if constexpr (kImp) imp = rg == R - 1 && wave == kWaves - 1 && rg * kRowsPerGroup + wave * 32 >= pl.rows_per_head;
  if (imp) {
    // row col = (recent query col / G, head g*G + col % G); rows past R*G are zero
    const bool ok = col < a.imp_R * G;
    const bf16_t* qp = static_cast<const bf16_t*>(a.q_imp) + ((int64_t)(ok ? col / G : 0) * Hq + g * G + col % G) * D;
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks)
      qf[ks] = ok ? __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + ks * 16 + half * 8))
                  : __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
  } else {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + ((int64_t)row_t * Hq + row_h) * D;
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + ks * 16 + half * 8));
  }
#pragma unroll
  for (int ks = 0; ks < Ly::KS; ++ks) asm volatile("" : : "v"(qf[ks]));
  // tiles 0..kAhead-1 start streaming (Q has already landed)
  for (int j = 0; j < kAhead; ++j) issue_upto(j);

  const int words = (T + 31) >> 5;
  int t_lo, t_hi;
  draft_rows_of(rg * kRowsPerGroup, min(pl.rows_per_head, (rg + 1) * kRowsPerGroup), G, T, t_lo, t_hi);
  if (vt1 > pl.n_cache_tiles) build_ancestor_rows(a.parent, words, t_lo, t_hi, anc, s_par, tid, kThreads);

  // per-lane LDS addresses of the operand reads in stage 0
  uint32_t koff[Ly::KS], voff[Ly::DB];
  {
    const int vrow0 = 4 * half + ((lane & 15) >> 2);
    const int vdim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) koff[ks] = k_lds + (uint32_t)((col * D + k_chunk<D>(col, 2 * ks + half) * 8) * 2);
#pragma unroll
    for (int db = 0; db < Ly::DB; ++db) {
      const int d = 32 * db + vdim;
      voff[db] = v_lds + (uint32_t)((vrow0 * D + v_chunk<D>(vrow0, d >> 3) * 8 + (d & 7)) * 2);
    }
    // opaque to the compiler: the stage and row offsets then fold into the
    // instructions' immediate field instead of being added per read
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) asm volatile("" : "+v"(koff[ks]));
#pragma unroll
    for (int db = 0; db < Ly::DB; ++db) asm volatile("" : "+v"(voff[db]));
  }

  f32x16_t S;
  bf16x8_t Kf[Ly::KS];
  auto read_k_at = [&](uint32_t so) {          // so: stage offset in bytes
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks)
      Kf[ks] = *reinterpret_cast<__attribute__((address_space(3))) bf16x8_t*>(koff[ks] + so);
  };
  auto read_k = [&](int j) { read_k_at((uint32_t)(j % kStages) * kTileBytes); };
  auto qk = [&](f32x16_t& Sx) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Sx[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) Sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Kf[ks], qf[ks], Sx, 0, 0, 0);
  };
  // Chunk importance of tile j from S = Q . K^T (importance wave only): lane
  // holds key lane % 32 and query rows 8*(e/4) + 4*half + e%4 in register e, so
  // recent query r's G heads (rows r*G .. r*G + G-1) are G consecutive
  // registers. Per key, the maximum over the heads of each query, summed over
  // the queries; an odd tile completes a 64-token chunk.
  float imp_acc = 0.f;
  const int imp_rows = a.imp_R * G;
  const float imp_scale = a.imp_scale;
  auto imp_sum = [&](const f32x16_t& Sx, auto gc) {
    constexpr int GG = decltype(gc)::value;
    float sum = 0.f;
#pragma unroll
    for (int e0 = 0; e0 < 16; e0 += 4) {
      // registers e0..e0+3 are rows rb..rb+3
      const int rb = 8 * (e0 >> 2) + 4 * half;
#pragma unroll
      for (int q0 = 0; q0 < 4; q0 += GG) {
        // the query of rows rb+q0 .. rb+q0+GG-1
        float v = Sx[e0 + q0] * imp_scale;
#pragma unroll
        for (int h = 1; h < GG; ++h) v = fmaxf(v, Sx[e0 + q0 + h] * imp_scale);
        sum += rb + q0 < imp_rows ? v : 0.f;
      }
    }
    return sum;
  };
  auto imp_tile = [&](const f32x16_t& Sx, int j) {
    imp_acc += G == 4   ? imp_sum(Sx, std::integral_constant<int, 4>{})
               : G == 2 ? imp_sum(Sx, std::integral_constant<int, 2>{})
                        : imp_sum(Sx, std::integral_constant<int, 1>{});
    const int vt = vt0 + j;
    if (vt & 1) {
      // sum over the 64 lanes: DPP within rows of 16, then the four rows
      float x = imp_acc;
      x += quad_dpp<0xB1>(x);                        // quad_perm [1,0,3,2]
      x += quad_dpp<0x4E>(x);                        // quad_perm [2,3,0,1]
      x += quad_dpp<0x141>(x);                       // row_half_mirror
      x += quad_dpp<0x140>(x);                       // row_mirror
      const float tot = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16))) +
                        (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
      if (lane == 0) a.scores[(int64_t)g * (a.L >> 6) + (vt >> 1)] = tot * (1.f / (64.f * (float)a.imp_R));
      imp_acc = 0.f;
    }
  };
  // the importance wave's product: S = Q . K^T (operands of qk in the other order)
  auto qk_imp = [&](f32x16_t& Sx) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Sx[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < Ly::KS; ++ks) Sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], Kf[ks], Sx, 0, 0, 0);
  };

  // Tiles past the last full cache tile (ragged cache tail, drafts) are masked;
  // they form a suffix of the split and run after the pipelined prefix.
  const int full_tiles = (int)(a.L / kKeys);
  const int nb_u = max(0, min(nb, full_tiles - vt0));

  const bf16_t* cache_next = cache_base + (int64_t)(vt0 + kAhead) * kKeys * D;
  // the importance wave's steady-state iteration: the same barrier and loads, QK^T
  // and its chunk scores, no V
  auto fast_imp = [&](auto ust, int j) {
    constexpr int U = decltype(ust)::value;
    __builtin_amdgcn_s_waitcnt(vm_wait((kAhead - 3) * Ly::loadsPerWave));    // tile j+2 landed
    asm volatile("s_barrier" : : : "memory");
    {
      const bf16_t* base = cache_next + (int64_t)j * kKeys * D;         // tile j+kAhead
      const uint32_t sb = my_lds + (uint32_t)(((U + kAhead) % kStages) * kTileBytes);
#pragma unroll
      for (int n = 0; n < Ly::loadsPerWave; ++n) {
        const int q = wave * Ly::loadsPerWave + n;
        const int mblk = q >= Ly::loadsPerTensor ? q - Ly::loadsPerTensor : q;
        lds_dma16(base, off_full[n], sb + (uint32_t)(mblk * 1024));
      }
    }
    f32x16_t Sn;
    qk_imp(Sn);
    read_k_at((uint32_t)(((U + 2) % kStages) * kTileBytes));
    imp_tile(S, j);
    S = Sn;
  };
  auto steady = [&](auto&& body, int& j) {
    for (; j + kStages <= nb_u - kAhead; j += kStages) {  // j % kStages == 1
      body(std::integral_constant<int, 1 % kStages>{}, j);
      body(std::integral_constant<int, 2 % kStages>{}, j + 1);
      body(std::integral_constant<int, 3 % kStages>{}, j + 2);
      body(std::integral_constant<int, 4 % kStages>{}, j + 3);
      body(std::integral_constant<int, 5 % kStages>{}, j + 4);
      body(std::integral_constant<int, 6 % kStages>{}, j + 5);
      body(std::integral_constant<int, 7 % kStages>{}, j + 6);
      if constexpr (kStages == 8) body(std::integral_constant<int, 0>{}, j + 7);
      issued = j + kStages + kAhead;
    }
  };


  // ---- the importance wave: its own loop, with the same barriers and loads ----
  if constexpr (kImp) {
    if (imp) {
      // iteration j: publish tile j+2, start tile j+kAhead, QK^T(j+1), score tile j
      auto iter_imp = [&](auto next, int j) {
        constexpr bool kNext = decltype(next)::value;
        wait_for(j + 2);
        __syncthreads();
        issue_upto(j + kAhead);
        f32x16_t Sn;
        if constexpr (kNext) qk_imp(Sn);
        read_k(j + 2);
        imp_tile(S, j);
        if constexpr (kNext) S = Sn;
      };
      if (nb_u > 0) {
        wait_for(1);
        __syncthreads();
        read_k(0);
        qk_imp(S);
        if (nb_u > 1) read_k(1);
        if (nb_u == 1) {
          iter_imp(Flag<false>{}, 0);
        } else {
          iter_imp(Flag<true>{}, 0);
          int j = 1;
          steady(fast_imp, j);
          for (; j < nb_u - 1; ++j) iter_imp(Flag<true>{}, j);
          iter_imp(Flag<false>{}, nb_u - 1);
        }
      }
      // the masked suffix holds only draft tiles here: barriers and loads only
      for (int j = nb_u; j < nb; ++j) {
        wait_for(j);
        __syncthreads();
        issue_upto(j + kAhead - 1);
      }
      return;
    }
  }

  f32x16_t O[Ly::DB];
#pragma unroll
  for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[db][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  bf16x8_t P[2];
  bf16x8_t Vf[2][Ly::DB];

  auto read_v_at = [&](uint32_t so) {
#pragma unroll
    for (int db = 0; db < Ly::DB; ++db) {
      __attribute__((address_space(3))) s16x4_t* vp =
          reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(voff[db] + so);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vp + (16 * hh) * D / 4);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vp + (16 * hh + 8) * D / 4);
        Vf[hh][db] = __builtin_bit_cast(
            bf16x8_t, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                                  hi[0], hi[1], hi[2], hi[3]});
      }
    }
  };
  auto read_v = [&](int j) { read_v_at((uint32_t)(j % kStages) * kTileBytes); };
  auto pv = [&](const bf16x8_t* Px) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < Ly::DB; ++db)
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Vf[hh][db], Px[hh], O[db], 0, 0, 0);
  };
  // softmax of one 32x32 score block; returns whether O must be scaled by *alpha
  auto softmax = [&](auto masked, f32x16_t Sx, bf16x8_t* Px, float* alpha, int j) -> bool {
    if constexpr (decltype(masked)::value) {
      int key0, nvalid;
      const bool draft = tile_keys(vt0 + j, key0, nvalid);
      uint32_t bits = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
      if (draft) bits &= row_ok ? anc[(row_t - t_lo) * words + (key0 >> 5)] : 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 8 * (e >> 2) + 4 * half + (e & 3);
        Sx[e] = ((bits >> key) & 1u) ? Sx[e] : -INFINITY;
      }
    }
    float t2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float t = fmaxf(fmaxf(Sx[8 * i], Sx[8 * i + 1]), Sx[8 * i + 2]);
      t = fmaxf(fmaxf(t, Sx[8 * i + 3]), Sx[8 * i + 4]);
      t = fmaxf(fmaxf(t, Sx[8 * i + 5]), Sx[8 * i + 6]);
      t2[i] = fmaxf(t, Sx[8 * i + 7]);
    }
    float mx = fmaxf(t2[0], t2[1]);
    mx = max_xor32(mx) * c;
    const bool need = mx > m + kLazy;
    *alpha = need ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
    m = need ? mx : m;
    const float nmb = -fmaxf(m, -3.0e38f);
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(Sx[e], c, nmb));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) Px[hh][e] = static_cast<__bf16>(pe[8 * hh + e]);
    float s4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = (pe[4 * i] + pe[4 * i + 1]) + (pe[4 * i + 2] + pe[4 * i + 3]);
    lsum = lsum * *alpha + ((s4[0] + s4[1]) + (s4[2] + s4[3]));
    return __builtin_amdgcn_ballot_w64(need) != 0;
  };
  // Unmasked tiles: the probabilities against the current m, with no row
  // maximum. A lane whose 16 probabilities sum to more than 2^12 (so one
  // exceeds 2^8, or m is still -inf) flags the wave, which then redoes the
  // tile with the row maximum (softmax_fix) before the probabilities are used.
  auto softmax_fast = [&](f32x16_t Sx, bf16x8_t* Px, float& st) -> bool {
    const float nmb = -m;
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(Sx[e], c, nmb));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) Px[hh][e] = static_cast<__bf16>(pe[8 * hh + e]);
    float s4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = (pe[4 * i] + pe[4 * i + 1]) + (pe[4 * i + 2] + pe[4 * i + 3]);
    st = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    return st > 4096.0f;
  };
  auto softmax_fix = [&](f32x16_t Sx, bf16x8_t* Px, float* alpha) -> bool {
    float t2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float t = fmaxf(fmaxf(Sx[8 * i], Sx[8 * i + 1]), Sx[8 * i + 2]);
      t = fmaxf(fmaxf(t, Sx[8 * i + 3]), Sx[8 * i + 4]);
      t = fmaxf(fmaxf(t, Sx[8 * i + 5]), Sx[8 * i + 6]);
      t2[i] = fmaxf(t, Sx[8 * i + 7]);
    }
    float mx = fmaxf(t2[0], t2[1]);
    mx = max_xor32(mx) * c;
    const bool need = mx > m + kLazy;
    *alpha = need ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
    m = need ? mx : m;
    const float nmb = -fmaxf(m, -3.0e38f);
    float pe[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(Sx[e], c, nmb));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) Px[hh][e] = static_cast<__bf16>(pe[8 * hh + e]);
    float s4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = (pe[4 * i] + pe[4 * i + 1]) + (pe[4 * i + 2] + pe[4 * i + 3]);
    lsum = lsum * *alpha + ((s4[0] + s4[1]) + (s4[2] + s4[3]));
    return __builtin_amdgcn_ballot_w64(need) != 0;
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) O[db][e] *= alpha;
  };

  // Pipelined iteration j over unmasked tiles. On entry: S = S(j), Kf = K(j+1)
  // (if j+1 < nb_u), Vf = V(j-1) and P = P(j-1) (if j >= 1).
  auto iter = [&](auto prev, auto next, int j) {
    constexpr bool kPrev = decltype(prev)::value, kNext = decltype(next)::value;
    // publish tile j+2, start tile j+kAhead
    wait_for(j + 2);
    __syncthreads();                    // every wave is past iteration j-1: tile j-2 is free
    issue_upto(j + kAhead);
    f32x16_t Sn;
    if constexpr (kNext) qk(Sn);
    if constexpr (kPrev) pv(P);
    read_k(j + 2);                      // past the split's end this reads a stale stage: unused
    read_v(j);
    float al;
    bf16x8_t Pn[2];
    const bool rs = softmax(Flag<false>{}, S, Pn, &al, j);
    __builtin_amdgcn_iglp_opt(2);
    asm volatile("" : : "v"(Pn[0]), "v"(Pn[1]), "v"(lsum), "v"(m));
    if (rs) rescale(al);
    P[0] = Pn[0]; P[1] = Pn[1];
    if constexpr (kNext) S = Sn;
  };

  // Steady-state iteration j (1 <= j, j + kAhead < nb_u), stage U = j % kStages
  // known at compile time: tiles j+2..j+kAhead-1 are in flight, tile j+kAhead is
  // a full cache tile. The barrier needs no LDS drain: the stage it recycles
  // (tile j-2) was last read two iterations ago and those reads were consumed
  // by products.
  auto fast = [&](auto ust, int j) {
    constexpr int U = decltype(ust)::value;
    __builtin_amdgcn_s_waitcnt(vm_wait((kAhead - 3) * Ly::loadsPerWave));    // tile j+2 landed
    asm volatile("s_barrier" : : : "memory");
    {
      const bf16_t* base = cache_next + (int64_t)j * kKeys * D;         // tile j+kAhead
      const uint32_t sb = my_lds + (uint32_t)(((U + kAhead) % kStages) * kTileBytes);
#pragma unroll
      for (int n = 0; n < Ly::loadsPerWave; ++n) {
        const int q = wave * Ly::loadsPerWave + n;
        const int mblk = q >= Ly::loadsPerTensor ? q - Ly::loadsPerTensor : q;
        lds_dma16(base, off_full[n], sb + (uint32_t)(mblk * 1024));
      }
    }
    f32x16_t Sn;
    qk(Sn);
    pv(P);
    read_k_at((uint32_t)(((U + 2) % kStages) * kTileBytes));
    read_v_at((uint32_t)(U * kTileBytes));
    bf16x8_t Pn[2];
    float st;
    const bool bad = softmax_fast(S, Pn, st);
    const float lsum_fast = lsum + st;
    __builtin_amdgcn_iglp_opt(2);
    asm volatile("" : : "v"(Pn[0]), "v"(Pn[1]), "v"(lsum_fast));
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      float al;
      if (softmax_fix(S, Pn, &al)) rescale(al);
    } else {
      lsum = lsum_fast;
    }
    P[0] = Pn[0]; P[1] = Pn[1];
    S = Sn;
  };

  if (nb_u > 0) {
    // publish tiles 0 and 1 (tiles up to 4 are in flight)
    wait_for(1);
    __syncthreads();
    read_k(0);
    qk(S);
    if (nb_u > 1) read_k(1);
    if (nb_u == 1) iter(Flag<false>{}, Flag<false>{}, 0);
    else {
      iter(Flag<false>{}, Flag<true>{}, 0);
      int j = 1;
      steady(fast, j);
      for (; j < nb_u - 1; ++j) iter(Flag<true>{}, Flag<true>{}, j);
      iter(Flag<true>{}, Flag<false>{}, nb_u - 1);
    }
    pv(P);                              // PV of the last pipelined tile (Vf = V(nb_u - 1))
  }
  // masked suffix, one tile at a time
  for (int j = nb_u; j < nb; ++j) {
    wait_for(j);
    __syncthreads();                    // tile j visible; every wave is past tile j - 1
    issue_upto(j + kAhead - 1);
    read_k(j);
    qk(S);
    float al;
    if (softmax(Flag<true>{}, S, P, &al, j)) rescale(al);
    read_v(j);
    pv(P);
  }

  // ---- epilogue ---------------------------------------------------------------
  const float ltot = sum_xor32(lsum);
  if (row_ok) {
    const int64_t orow = ((int64_t)split * T + row_t) * Hq + row_h;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (a.o_part_h != nullptr) {
      // a call's own bf16 partials: half the bytes for its merge to read
      bf16_t* op = a.o_part_h + orow * D;
#pragma unroll
      for (int db = 0; db < Ly::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * db + 8 * q4 + 4 * half;
          *reinterpret_cast<uint2*>(op + d) =
              pack_bf16x4(O[db][4 * q4] * inv, O[db][4 * q4 + 1] * inv, O[db][4 * q4 + 2] * inv,
                          O[db][4 * q4 + 3] * inv);
        }
    } else {
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
    }
    if (half == 0) a.l_part[orow] = ltot > 0.f ? (m + log2f(ltot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

int mfma_rows_per_group(int rows_per_head) { return rows_per_head <= 128 ? 128 : 256; }

bool attn_mfma_importance_fusable(const AttnPlan& p, int T, int G, int D, int64_t L, int R) {
  // the 8-wave, 8-stage D = 128 kernel whose last row group ends in a wave with
  // no query row; R*G recent query rows fit that wave's 32 and a query's G heads
  // sit in one lane quad; the cache is whole 64-token chunks and the splits
  // start on even tiles
  const int last = p.rows_per_head - (p.n_rowgroups - 1) * p.rows_per_group;
  return p.path == kPathMfma && p.rows_per_group == 256 && D == 128 && T <= 256 && last <= 224 &&
         (G == 1 || G == 2 || G == 4) && R >= 1 && R * G <= 32 && L > 0 && L % 64 == 0 &&
         p.tiles_per_split % 2 == 0;
}
int mfma_tile_keys() { return kKeys; }
int mfma_groups_per_cu() { return 1; }

template <int kWaves>
hipError_t launch_waves(const AttnArgs& a, int blocks, hipStream_t s) {
  constexpr int kThreads = kWaves * 64;
  // up to 256 drafts: an 8-stage ring (tiles issued 6 ahead); more: 7 stages.
  // The 4-wave form serves at most 128 rows per KV head, so at most 128 drafts.
  if (kWaves == 4 && a.T > 128) return hipErrorInvalidValue;
  if (a.q_imp != nullptr) {
    // chunk importance in the all-padding wave (the caller checked the shape)
    if constexpr (kWaves == 8) {
      if (a.D != 128 || a.T > 256) return hipErrorInvalidValue;
      attn_split_mfma_kernel<128, 8, 256, 8, true><<<blocks, kThreads, 0, s>>>(a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (kWaves == 4 || a.T <= 256) {
    if (a.D == 128) attn_split_mfma_kernel<128, 8, 256, kWaves, false><<<blocks, kThreads, 0, s>>>(a);
    else attn_split_mfma_kernel<64, 8, 256, kWaves, false><<<blocks, kThreads, 0, s>>>(a);
  } else if constexpr (kWaves == 8) {
    if (a.D == 128) attn_split_mfma_kernel<128, 7, TS_MAX_DRAFT, kWaves, false><<<blocks, kThreads, 0, s>>>(a);
    else attn_split_mfma_kernel<64, 7, TS_MAX_DRAFT, kWaves, false><<<blocks, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_split_mfma(const AttnArgs& a, hipStream_t s) {
  const int R = a.plan.n_rowgroups;
  const int n_units = a.plan.n_splits * a.Hkv;
  const int blocks = ((n_units + 7) / 8) * 8 * R;
  return a.plan.rows_per_group == 128 ? launch_waves<4>(a, blocks, s) : launch_waves<8>(a, blocks, s);
}

}  // namespace ts
