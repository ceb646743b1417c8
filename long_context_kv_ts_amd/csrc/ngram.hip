// 4-gram table of the committed text and top-k retrieval by first token.
//
// The table is one device buffer: a header, an open-addressing array of slots
// (entry id or -1, linear probing) and a dense pool of entries {4 tokens,
// count, last position}. Entries are never removed, so a key's probe sequence
// only grows and "reached an empty slot" proves the key absent.
//
// Update (one 1024-thread workgroup, positions in chunks of 1024): thread q
// takes the 4-gram ending at position c+q and claims it in an LDS hash table
// of the chunk's 4-grams (2048 slots, linear probing, compare-and-swap): the
// thread that claims a 4-gram owns it, and every thread holding it adds one to
// the owner's multiplicity and raises its last position. Only owners insert,
// so keys inserted concurrently are distinct: an absent key's wave takes
// consecutive entry ids with one atomic, the entry is written and fenced
// before a compare-and-swap publishes its id in an empty slot, a lost swap
// means another key took the slot, and probing continues. No thread ever
// waits for another. Probing stops after `capacity` slots; an entry that
// cannot be placed is counted in the header and left with count 0.
//
// Retrieval: grid over the entry pool, 4096 entries a workgroup. A histogram
// of the matching entries' counts gives the smallest count that can still be
// among the workgroup's k best; the entries at or above it are ranked in LDS
// by (count, last position), both descending (last positions are distinct,
// so ranks are unique), and each workgroup keeps its k best; one workgroup
// then ranks those.
#include "decode.h"

namespace ts {
namespace {

constexpr int kUpdThreads = 1024;
constexpr int kUpdSlots = 2 * kUpdThreads;              // the chunk's LDS hash table, at most half full
constexpr int kRetThreads = 256;
constexpr int kRetPerThread = 16;
constexpr int kRetPerWG = kRetThreads * kRetPerThread;          // 4096 entries a scan workgroup
constexpr int kPickMax = (kNgramMaxEntries / kRetPerWG) * kNgramMaxK;   // candidates the pick ranks
static_assert(kPickMax <= kRetPerWG, "the pick holds every candidate, 16 a thread");
static_assert(kNgramMaxEntries / kRetPerWG <= kRetThreads, "the pick holds one scan workgroup per thread");

__device__ __forceinline__ uint32_t rotl(uint32_t x, int r) { return (x << r) | (x >> (32 - r)); }

// A mix of the four tokens (multiplicative hashing with odd 32-bit constants,
// then an xor-shift finaliser); only the slot order depends on it.
__device__ __forceinline__ uint32_t ngram_hash(int4 g) {
  uint32_t h = (uint32_t)g.x * 0x9E3779B1u;
  h ^= rotl((uint32_t)g.y * 0x85EBCA77u, 7);
  h ^= rotl((uint32_t)g.z * 0xC2B2AE3Du, 14);
  h ^= rotl((uint32_t)g.w * 0x27D4EB2Fu, 21);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return h;
}

__device__ __forceinline__ bool same(int4 a, int4 b) { return a.x == b.x && a.y == b.y && a.z == b.z && a.w == b.w; }

__device__ __forceinline__ int load_acq(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int load_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The key of an entry whose id was read with load_acq: that acquire orders these
// plain loads after the publisher's fence (entries are 8-byte aligned).
__device__ __forceinline__ int4 entry_key(const NgramEntry* e) {
  const int2 a = *reinterpret_cast<const int2*>(&e->tok[0]);
  const int2 b = *reinterpret_cast<const int2*>(&e->tok[2]);
  return make_int4(a.x, a.y, b.x, b.y);
}

__global__ __launch_bounds__(256) void ngram_init_kernel(NgramView t, int capacity_log2, int max_entries) {
  const int64_t cap = int64_t(1) << capacity_log2;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cap; i += (int64_t)gridDim.x * blockDim.x)
    t.slots[i] = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) *t.hdr = NgramHeader{capacity_log2, max_entries, 0, 0};
}

// Called by every thread of the update workgroup (`active` marks the owners of
// distinct 4-grams), so the entry allocation is one atomic per wave:
//   1. probe to the key (then add to its count and last position) or to the
//      first empty slot, which proves the key absent (no other thread of the
//      launch inserts the same key);
//   2. the wave's absent keys take consecutive entry ids with one atomicAdd;
//   3. each writes and fences its entry, then publishes its id with a
//      compare-and-swap at that slot or, if another key took it meanwhile, at
//      the next empty one.
__device__ void insert(NgramView t, int4 key, int m, int last, bool active) {
  const uint32_t cap = 1u << t.hdr->capacity_log2, mask = cap - 1u;
  const int max_entries = t.hdr->max_entries;
  uint32_t s = ngram_hash(key) & mask, probe = 0;
  bool absent = false;
  if (active) {
    for (; probe < cap; ++probe, s = (s + 1u) & mask) {
      const int cur = load_acq(&t.slots[s]);
      if (cur < 0) {
        absent = true;
        break;
      }
      NgramEntry* e = t.entries + cur;
      if (same(entry_key(e), key)) {
        atomicAdd(&e->count, m);
        atomicMax(&e->last, last);
        break;
      }
    }
    if (probe == cap) atomicAdd(&t.hdr->dropped, 1);     // full table, key absent
  }
  const uint64_t want = __ballot(absent);
  if (want == 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int leader = __ffsll((unsigned long long)want) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(&t.hdr->n_entries, __popcll(want));
  base = __shfl(base, leader, kWave);
  if (!absent) return;
  const int mine = base + __popcll(want & ((1ull << lane) - 1ull));
  if (mine >= max_entries) {
    atomicAdd(&t.hdr->dropped, 1);
    return;
  }
  NgramEntry* e = t.entries + mine;
  e->tok[0] = key.x;
  e->tok[1] = key.y;
  e->tok[2] = key.z;
  e->tok[3] = key.w;
  e->count = m;
  e->last = last;
  __threadfence();
  for (; probe < cap; ++probe, s = (s + 1u) & mask) {
    if (load_relaxed(&t.slots[s]) >= 0) continue;               // another key's slot
    if (atomicCAS(&t.slots[s], -1, mine) == -1) return;
  }
  e->count = 0;                                                 // never published; retrieval skips it
  atomicAdd(&t.hdr->dropped, 1);
}

__global__ __launch_bounds__(kUpdThreads) void ngram_update_kernel(void* table, const int32_t* __restrict__ tokens,
                                                                   int64_t from, int64_t to) {
  __shared__ int4 s_key[kUpdThreads];
  __shared__ int s_slot[kUpdSlots];            // owner thread of the 4-gram hashed there, or -1
  __shared__ int s_mult[kUpdThreads], s_last[kUpdThreads];
  const NgramView t = ngram_view(table, static_cast<const NgramHeader*>(table)->capacity_log2);
  const int q = threadIdx.x;
  for (int64_t c = from < 3 ? 3 : from; c < to; c += kUpdThreads) {
    const int n = (int)min((int64_t)kUpdThreads, to - c);
    int4 key = make_int4(0, 0, 0, 0);
    if (q < n) {
      const int32_t* w = tokens + (c + q - 3);
      key = make_int4(w[0], w[1], w[2], w[3]);
      s_key[q] = key;
    }
    for (int i = q; i < kUpdSlots; i += kUpdThreads) s_slot[i] = -1;
    s_mult[q] = 0;
    s_last[q] = -1;
    __syncthreads();
    int owner = -1;
    if (q < n) {
      // claim the 4-gram or find the thread that did: n <= half the slots, so an
      // empty slot is always reached
      for (uint32_t h = ngram_hash(key) & (kUpdSlots - 1);; h = (h + 1) & (kUpdSlots - 1)) {
        int cur = s_slot[h];
        if (cur < 0) {
          cur = atomicCAS(&s_slot[h], -1, q);
          if (cur < 0) {
            owner = q;
            break;
          }
        }
        if (same(s_key[cur], key)) {
          owner = cur;
          break;
        }
      }
      atomicAdd(&s_mult[owner], 1);
      atomicMax(&s_last[owner], q);
    }
    __syncthreads();
    const bool own = q < n && owner == q;
    insert(t, key, own ? s_mult[q] : 0, own ? (int)(c + s_last[q]) : 0, own);
    __syncthreads();                            // the next chunk reuses the LDS tables and sees these entries
  }
}

struct Cand {
  uint64_t key;                                 // count << 32 | last position
  int id;
  int pad;
};

// Exclusive prefix of v over the workgroup's threads (index order); total = the sum.
__device__ int block_excl_scan(int v, int* red, int& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  const int excl = incl - v;
  if (lane == kWave - 1) red[wave] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kRetThreads / kWave; ++w) {
    off += w < wave ? red[w] : 0;
    total += red[w];
  }
  __syncthreads();
  return off + excl;
}

constexpr int kCountBins = kRetThreads;          // counts >= 255 share the top bin

// How many of s[0..n) have a larger key: eight independent LDS reads at a time.
__device__ __forceinline__ int count_greater(const Cand* s, int n, uint64_t key) {
  int r = 0, j = 0;
  for (; j + 8 <= n; j += 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s[j + u].key;
#pragma unroll
    for (int u = 0; u < 8; ++u) r += v[u] > key;
  }
  for (; j < n; ++j) r += s[j].key > key;
  return r;
}

// The bin b of hist[0..kCountBins) (thread i holds bin kCountBins-1-i, so
// bins are visited from the top) where `before` plus the entries of the bins
// above b stay below k and reach k with bin b; -1 when they never reach k.
__device__ int cut_bin(const int* hist, int before, int k, int* red, int* s_cut) {
  const int tid = threadIdx.x;
  const int h = hist[kCountBins - 1 - tid];
  int total;
  const int above = before + block_excl_scan(h, red, total);
  if (tid == 0) *s_cut = -1;
  __syncthreads();
  if (h > 0 && above < k && above + h >= k) *s_cut = kCountBins - 1 - tid;
  __syncthreads();
  const int c = *s_cut;
  __syncthreads();
  return c;
}

struct SelectLds {
  Cand c[kRetPerWG];                            // the survivors of the cuts (at most every candidate)
  int hist[kCountBins];
  int red[kRetThreads / kWave];
  int cut;
};

// The k best of the candidates the workgroup holds, 16 a thread (valid[j]
// marks them), by (count, last) descending, written to out[0 .. min(n, k)) in
// rank order; returns min(n, k). A histogram of the counts gives the count bin
// that straddles the k-th best (higher bins are all in, lower bins all out:
// each of their candidates has k larger keys above it); inside that bin,
// where the counts tie, the same cut on the high bits of the last position;
// only the survivors are ranked against each other. All threads call it.
__device__ int select_best(const int (&cnt)[kRetPerThread], const int (&last)[kRetPerThread],
                           const int (&id)[kRetPerThread], const bool (&valid)[kRetPerThread], int k,
                           SelectLds& s, Cand* __restrict__ out) {
  const int tid = threadIdx.x;
  s.hist[tid] = 0;
  __syncthreads();
  int lmax = -1, nvalid = 0;
#pragma unroll
  for (int j = 0; j < kRetPerThread; ++j) {
    if (valid[j]) {
      atomicAdd(&s.hist[min(cnt[j], kCountBins - 1)], 1);
      lmax = max(lmax, last[j]);
      ++nvalid;
    }
  }
  __syncthreads();
  const int cut = cut_bin(s.hist, 0, k, s.red, &s.cut);
  int lcut = -1, shift = 0;
  if (cut >= 0 && cut < kCountBins - 1) {     // bins below the top hold one exact count
    int above_cut;
    block_excl_scan(tid > cut ? s.hist[tid] : 0, s.red, above_cut);
    int m = lmax;
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
    if ((tid & (kWave - 1)) == 0) s.red[tid >> 6] = m;
    __syncthreads();
    m = max(max(s.red[0], s.red[1]), max(s.red[2], s.red[3]));
    __syncthreads();
    shift = max(0, 32 - __clz(max(m, 1)) - 8);        // last >> shift < 256
    s.hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRetPerThread; ++j)
      if (valid[j] && cnt[j] == cut) atomicAdd(&s.hist[last[j] >> shift], 1);
    __syncthreads();
    lcut = cut_bin(s.hist, above_cut, k, s.red, &s.cut);
  }
  auto keep = [&](int j) {
    if (!valid[j]) return false;
    const int c = min(cnt[j], kCountBins - 1);
    if (cut < 0 || c > cut) return true;              // fewer than k candidates, or above the cut
    if (c < cut) return false;
    return lcut < 0 || (last[j] >> shift) >= lcut;
  };
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kRetPerThread; ++j) mine += keep(j);
  int nc;
  int slot = block_excl_scan(mine, s.red, nc);
#pragma unroll
  for (int j = 0; j < kRetPerThread; ++j)
    if (keep(j)) s.c[slot++] = Cand{((uint64_t)(uint32_t)cnt[j] << 32) | (uint32_t)last[j], id[j], 0};
  __syncthreads();
  for (int i = tid; i < nc; i += kRetThreads) {
    const int rank = count_greater(s.c, nc, s.c[i].key);
    if (rank < k) out[rank] = s.c[i];
  }
  int total;
  block_excl_scan(nvalid, s.red, total);
  return min(total, k);
}

__global__ __launch_bounds__(kRetThreads) void ngram_scan_kernel(void* table, const int32_t* __restrict__ first_tok,
                                                                 int k, int* __restrict__ ws_n, Cand* __restrict__ ws) {
  __shared__ SelectLds s;
  const NgramView t = ngram_view(table, static_cast<const NgramHeader*>(table)->capacity_log2);
  const int tid = threadIdx.x, b = blockIdx.x;
  const int n = min(load_acq(&t.hdr->n_entries), t.hdr->max_entries);
  const int e0 = b * kRetPerWG;
  if (e0 >= n) {                                // past the used entries: nothing to offer
    if (tid == 0) ws_n[b] = 0;
    return;
  }
  const int f = *first_tok;
  // the three fields that matter, every load issued before any is used (indices clamped in range)
  int tok0[kRetPerThread], cnt[kRetPerThread], last[kRetPerThread];
#pragma unroll
  for (int j = 0; j < kRetPerThread; ++j) {
    const NgramEntry* e = t.entries + min(e0 + tid + j * kRetThreads, n - 1);
    tok0[j] = e->tok[0];
    cnt[j] = e->count;
    last[j] = e->last;
  }
  bool hit[kRetPerThread];
  int id[kRetPerThread];
#pragma unroll
  for (int j = 0; j < kRetPerThread; ++j) {
    id[j] = e0 + tid + j * kRetThreads;
    hit[j] = id[j] < n && cnt[j] > 0 && tok0[j] == f;
  }
  const int nk = select_best(cnt, last, id, hit, k, s, ws + (int64_t)b * k);
  if (tid == 0) ws_n[b] = nk;
}

__global__ __launch_bounds__(kRetThreads) void ngram_pick_kernel(void* table, int nb, int k, const int* __restrict__ ws_n,
                                                                 const Cand* __restrict__ ws, int32_t* __restrict__ out_tok,
                                                                 int32_t* __restrict__ out_count, int32_t* __restrict__ n_found,
                                                                 Cand* __restrict__ best) {
  __shared__ SelectLds s;
  __shared__ int s_off[kNgramMaxEntries / kRetPerWG + 1];
  const NgramView t = ngram_view(table, static_cast<const NgramHeader*>(table)->capacity_log2);
  const int tid = threadIdx.x;
  {
    const int nbk = tid < nb ? ws_n[tid] : 0;   // nb <= kRetThreads
    int tot;
    const int off = block_excl_scan(nbk, s.red, tot);
    if (tid < nb) s_off[tid] = off;
    if (tid == 0) s_off[nb] = tot;
  }
  __syncthreads();
  const int total = s_off[nb];                  // <= kPickMax = kRetPerWG
  // candidate i (16 a thread) comes from the scan workgroup whose range holds it
  int cnt[kRetPerThread], last[kRetPerThread], id[kRetPerThread];
  bool valid[kRetPerThread];
#pragma unroll
  for (int j = 0; j < kRetPerThread; ++j) {
    const int i = tid + j * kRetThreads;
    valid[j] = i < total;
    cnt[j] = last[j] = id[j] = 0;
    if (valid[j]) {
      int b = 0;
      while (s_off[b + 1] <= i) ++b;
      const Cand c = ws[(int64_t)b * k + (i - s_off[b])];
      cnt[j] = (int)(c.key >> 32);
      last[j] = (int)(uint32_t)c.key;
      id[j] = c.id;
    }
  }
  const int nk = select_best(cnt, last, id, valid, k, s, best);
  __syncthreads();
  for (int i = tid; i < k; i += kRetThreads) {  // rows past the matches are empty
    if (i < nk) {
      const Cand c = best[i];
      const NgramEntry& e = t.entries[c.id];
#pragma unroll
      for (int x = 0; x < 4; ++x) out_tok[i * 4 + x] = e.tok[x];
      if (out_count) out_count[i] = (int32_t)(c.key >> 32);
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) out_tok[i * 4 + x] = -1;
      if (out_count) out_count[i] = 0;
    }
  }
  if (tid == 0 && n_found) *n_found = nk;
}

}  // namespace

static int scan_blocks(int max_entries) { return (max_entries + kRetPerWG - 1) / kRetPerWG; }
static size_t scan_counts_bytes(int max_entries) { return ((size_t)scan_blocks(max_entries) * sizeof(int) + 255) / 256 * 256; }

size_t ngram_table_bytes(int capacity_log2, int max_entries) {
  const size_t slots = ((size_t(4) << capacity_log2) + 255) / 256 * 256;
  return kNgramHeaderBytes + slots + (size_t)max_entries * sizeof(NgramEntry);
}

size_t ngram_retrieve_workspace_bytes(int max_entries, int k) {
  return scan_counts_bytes(max_entries) + (size_t)(scan_blocks(max_entries) + 1) * k * sizeof(Cand);
}

hipError_t launch_ngram_init(NgramView t, int capacity_log2, int max_entries, hipStream_t s) {
  const int64_t cap = int64_t(1) << capacity_log2;
  const int blocks = (int)std::min<int64_t>((cap + 255) / 256, 4096);
  ngram_init_kernel<<<blocks, 256, 0, s>>>(t, capacity_log2, max_entries);
  return hipGetLastError();
}

hipError_t launch_ngram_update(void* t, const int32_t* tokens, int64_t from, int64_t to, hipStream_t s) {
  if (to <= (from < 3 ? 3 : from)) return hipSuccess;
  ngram_update_kernel<<<1, kUpdThreads, 0, s>>>(t, tokens, from, to);
  return hipGetLastError();
}

hipError_t launch_ngram_retrieve(void* t, int max_entries, const int32_t* first_tok, int k, int32_t* out_tok,
                                 int32_t* out_count, int32_t* n_found, void* workspace, hipStream_t s) {
  const int nb = scan_blocks(max_entries);
  int* ws_n = static_cast<int*>(workspace);
  Cand* ws = reinterpret_cast<Cand*>(static_cast<char*>(workspace) + scan_counts_bytes(max_entries));
  ngram_scan_kernel<<<nb, kRetThreads, 0, s>>>(t, first_tok, k, ws_n, ws);
  ngram_pick_kernel<<<1, kRetThreads, 0, s>>>(t, nb, k, ws_n, ws, out_tok, out_count, n_found, ws + (int64_t)nb * k);
  return hipGetLastError();
}

}  // namespace ts
