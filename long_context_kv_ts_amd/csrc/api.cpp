// C ABI of the library: argument validation, work planning, launches.
// Nothing here allocates device memory or synchronises; every check runs on
// the host before the first HIP call, so a rejected call has no side effect.
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "decode.h"

namespace {

thread_local std::string g_last_error;

ts_status fail(ts_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ts_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return TS_OK;
  return fail(TS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(ts_dtype d) { return d == TS_BF16 ? 2 : 4; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int kValuRows = 16;
// MI355X: 256 compute units.
constexpr int kCUs = 256;

ts_status check_attn_shape(const char* fn, int T, int Hq, int Hkv, int D, int64_t L,
                           ts_dtype dtype, int num_splits) {
  if (dtype != TS_F32 && dtype != TS_BF16) return fail(TS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (T < 1 || T > TS_MAX_DRAFT) return fail(TS_ERR_UNSUPPORTED, "%s: T=%d outside [1, %d]", fn, T, TS_MAX_DRAFT);
  if (Hq < 1 || Hkv < 1) return fail(TS_ERR_INVALID_ARG, "%s: Hq=%d Hkv=%d must be >= 1", fn, Hq, Hkv);
  if (Hq % Hkv != 0) return fail(TS_ERR_INVALID_ARG, "%s: Hq=%d not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (Hq / Hkv > 16) return fail(TS_ERR_UNSUPPORTED, "%s: group size Hq/Hkv=%d > 16", fn, Hq / Hkv);
  if (Hq > 4096) return fail(TS_ERR_UNSUPPORTED, "%s: Hq=%d > 4096", fn, Hq);
  if (D != 64 && D != 128) return fail(TS_ERR_UNSUPPORTED, "%s: D=%d (supported: 64, 128)", fn, D);
  if (L < 0) return fail(TS_ERR_INVALID_ARG, "%s: L=%lld < 0", fn, (long long)L);
  if (L > (int64_t)1 << 30) return fail(TS_ERR_UNSUPPORTED, "%s: L=%lld > 2^30", fn, (long long)L);
  if (num_splits < 0 || num_splits > 65535) return fail(TS_ERR_INVALID_ARG, "%s: num_splits=%d", fn, num_splits);
  return TS_OK;
}

}  // namespace

namespace ts {

AttnPlan plan_attention(int T, int Hq, int Hkv, int D, int64_t L, ts_dtype dtype, int num_splits) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  p.rows_per_head = T * G;
  // bf16: matrix cores. KV heads with more than 16 grouped query rows use the
  // 256-row / 32-row-block kernel; up to 16 rows (one 16x16 MFMA tile) the
  // wave-per-split kernel. fp32: vector ALUs.
  if (dtype == TS_BF16) p.path = p.rows_per_head > 16 ? kPathMfma : kPathSmall;
  else p.path = kPathValu;
  (void)D;
  p.rows_per_group = p.path == kPathMfma ? mfma_rows_per_group(p.rows_per_head) : p.path == kPathSmall ? 16 : kValuRows;
  p.n_rowgroups = (p.rows_per_head + p.rows_per_group - 1) / p.rows_per_group;
  p.tile = p.path == kPathMfma ? mfma_tile_keys() : kTile;
  p.n_cache_tiles = (int)((L + p.tile - 1) / p.tile);
  p.n_draft_tiles = (T + p.tile - 1) / p.tile;
  p.n_virtual = p.n_cache_tiles + p.n_draft_tiles;
  int s = num_splits;
  if (s <= 0) {
    // workgroups per CU the launch aims for: as many matrix-core workgroups as
    // fit a CU, 8 waves of the small kernel (each wave a split), 4 vector-ALU
    const int per_cu = p.path == kPathMfma ? mfma_groups_per_cu() : p.path == kPathSmall ? 8 : 4;
    const int64_t groups = (int64_t)Hkv * p.n_rowgroups;
    s = (int)((kCUs * per_cu + groups - 1) / groups);
    if (s < 1) s = 1;
  }
  if (s > p.n_virtual) s = p.n_virtual;
  p.tiles_per_split = (p.n_virtual + s - 1) / s;
  // matrix-core splits start on even 32-key tiles, i.e. on 64-token chunk
  // boundaries (the split kernel can score chunks on the same reads)
  if (p.path == kPathMfma) p.tiles_per_split += p.tiles_per_split & 1;
  p.n_splits = (p.n_virtual + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

}  // namespace ts

using namespace ts;

extern "C" {

const char* ts_last_error(void) { return g_last_error.c_str(); }

int ts_abi_version(void) { return TS_ABI_VERSION; }

int ts_tree_verify_attn_num_splits(int T, int Hq, int Hkv, int D, int64_t L, ts_dtype dtype,
                                   int num_splits) {
  if (check_attn_shape("ts_tree_verify_attn_num_splits", T, Hq, Hkv, D, L, dtype, num_splits) != TS_OK)
    return -1;
  return plan_attention(T, Hq, Hkv, D, L, dtype, num_splits).n_splits;
}

// A call that merges its own splits keeps the O partials in its input dtype:
// bf16 for bf16 inputs (the output is bf16 too), half the bytes for the merge
// to read.
static size_t own_part_elem_bytes(ts_dtype dtype) { return dtype == TS_BF16 ? sizeof(bf16_t) : sizeof(float); }

size_t ts_tree_verify_attn_workspace(int T, int Hq, int Hkv, int D, int64_t L, ts_dtype dtype,
                                     int num_splits) {
  if (check_attn_shape("ts_tree_verify_attn_workspace", T, Hq, Hkv, D, L, dtype, num_splits) != TS_OK)
    return 0;
  const AttnPlan p = plan_attention(T, Hq, Hkv, D, L, dtype, num_splits);
  const size_t rows = (size_t)T * Hq;
  return align_up((size_t)p.n_splits * rows * D * own_part_elem_bytes(dtype)) +
         align_up((size_t)p.n_splits * rows * sizeof(float));
}

// chunk importance scored by the split kernel on the same reads of K
struct ImpFusion {
  const void* q_recent;
  float* scores;
  int R;
  float scale;
};

// The gather of the chosen chunks done by the pass over the partial cache
// (small path): the source cache and where the copies go.
struct GatherFusion {
  const int32_t* chunk_idx;
  int64_t n_chunks;          // chunks in the source cache
  void* k_part;
  void* v_part;
};

// Partials in fp32, or in bf16 for bf16 inputs (the split kernels of fp32
// inputs write fp32 only).
static ts_status check_part_dtype(const char* fn, ts_dtype part_dtype, ts_dtype dtype) {
  if (part_dtype != TS_F32 && part_dtype != TS_BF16)
    return fail(TS_ERR_INVALID_ARG, "%s: unknown part_dtype %d", fn, (int)part_dtype);
  if (part_dtype == TS_BF16 && dtype != TS_BF16)
    return fail(TS_ERR_UNSUPPORTED, "%s: bf16 partials need bf16 inputs", fn);
  return TS_OK;
}

static ts_status attn_common(const char* fn, const void* q, const void* kc, const void* vc,
                             int64_t cache_stride, const void* kd, const void* vd,
                             const int32_t* parent, bool need_parent, void* o_part, ts_dtype part_dtype,
                             float* l_part, int T, int Hq, int Hkv, int D, int64_t L, float scale,
                             ts_dtype dtype, int num_splits, hipStream_t stream,
                             const ImpFusion* imp = nullptr, const GatherFusion* gf = nullptr) {
  ts_status st = check_attn_shape(fn, T, Hq, Hkv, D, L, dtype, num_splits);
  if (st != TS_OK) return st;
  st = check_part_dtype(fn, part_dtype, dtype);
  if (st != TS_OK) return st;
  if (!q || !kd || !vd || !o_part || !l_part) return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (L > 0 && (!kc || !vc)) return fail(TS_ERR_INVALID_ARG, "%s: null cache pointer with L=%lld", fn, (long long)L);
  if (need_parent && !parent) return fail(TS_ERR_INVALID_ARG, "%s: parent is null", fn);
  if (!aligned16(q) || !aligned16(kd) || !aligned16(vd) || !aligned16(o_part) ||
      (L > 0 && (!aligned16(kc) || !aligned16(vc))))
    return fail(TS_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if (((uintptr_t)l_part & 3u) != 0) return fail(TS_ERR_INVALID_ARG, "%s: l_part misaligned", fn);
  if (!gf && cache_stride < L)
    return fail(TS_ERR_INVALID_ARG, "%s: cache_stride=%lld < L=%lld", fn, (long long)cache_stride, (long long)L);
  // The kernels take each row's maximum of the raw products and scale it
  // afterwards, which is the maximum of the scaled logits only for scale > 0.
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(TS_ERR_INVALID_ARG, "%s: scale must be finite and > 0 (got %g)", fn, (double)scale);

  const AttnPlan plan = plan_attention(T, Hq, Hkv, D, L, dtype, num_splits);
  // one workgroup per (split, KV head, row group), rounded up to a multiple of 8 per row group
  if (((int64_t)plan.n_splits * Hkv + 7) / 8 * 8 * plan.n_rowgroups > INT32_MAX)
    return fail(TS_ERR_UNSUPPORTED, "%s: %d splits x %d KV heads x %d row groups exceed one launch", fn,
                plan.n_splits, Hkv, plan.n_rowgroups);

  AttnArgs a{};
  a.q = q; a.kc = kc; a.vc = vc; a.cache_stride = cache_stride; a.kd = kd; a.vd = vd;
  a.parent = parent; a.l_part = l_part;
  if (part_dtype == TS_BF16) a.o_part_h = static_cast<bf16_t*>(o_part);
  else a.o_part = static_cast<float*>(o_part);
  a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D; a.L = L;
  a.scale_log2 = scale * kLog2e;
  a.plan = plan;
  if (imp != nullptr) {
    a.q_imp = imp->q_recent;
    a.scores = imp->scores;
    a.imp_R = imp->R;
    a.imp_scale = imp->scale;
  }
  if (gf != nullptr) {
    a.gidx = gf->chunk_idx;
    a.g_chunks = gf->n_chunks;
    a.kp = gf->k_part;
    a.vp = gf->v_part;
  }
  hipError_t e = a.plan.path == kPathMfma    ? launch_attn_split_mfma(a, stream)
                 : a.plan.path == kPathSmall ? launch_attn_split_small(a, stream)
                                             : launch_attn_split_valu(a, dtype, stream);
  return from_hip(e, fn);
}

ts_status ts_tree_verify_attn_partials(const void* q, const void* k_cache, const void* v_cache,
                                       int64_t cache_stride, const void* k_draft,
                                       const void* v_draft, const int32_t* parent,
                                       void* o_part, ts_dtype part_dtype, float* l_part, int T, int Hq,
                                       int Hkv, int D, int64_t L, float scale, ts_dtype dtype,
                                       int num_splits, hipStream_t stream) {
  return attn_common("ts_tree_verify_attn_partials", q, k_cache, v_cache, cache_stride, k_draft,
                     v_draft, parent, true, o_part, part_dtype, l_part, T, Hq, Hkv, D, L, scale, dtype,
                     num_splits, stream);
}

static ts_status check_importance(const char* fn, const void* q_recent, const void* k_cache,
                                  int64_t cache_stride, const float* scores, int R, int Hq, int Hkv, int D,
                                  int64_t L, int chunk, float scale, ts_dtype dtype);

ts_status ts_tree_verify_attn_partials_and_importance(
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_stride, const void* k_draft,
    const void* v_draft, const int32_t* parent, void* o_part, ts_dtype part_dtype, float* l_part, int T, int Hq,
    int Hkv, int D, int64_t L, float scale, ts_dtype dtype, int num_splits, const void* q_recent, int R, int chunk,
    float imp_scale, float* scores, hipStream_t stream) {
  const char* fn = "ts_tree_verify_attn_partials_and_importance";
  ts_status st = check_importance(fn, q_recent, k_cache, cache_stride, scores, R, Hq, Hkv, D, L, chunk,
                                  imp_scale, dtype);
  if (st != TS_OK) return st;
  st = check_attn_shape(fn, T, Hq, Hkv, D, L, dtype, num_splits);
  if (st != TS_OK) return st;
  st = check_part_dtype(fn, part_dtype, dtype);
  if (st != TS_OK) return st;
  const AttnPlan plan = plan_attention(T, Hq, Hkv, D, L, dtype, num_splits);
  const bool fused = dtype == TS_BF16 && chunk == 64 &&
                     attn_mfma_importance_fusable(plan, T, Hq / Hkv, D, L, R);
  if (!fused) {
    // two launches: the split kernel, then the importance kernel
    st = attn_common(fn, q, k_cache, v_cache, cache_stride, k_draft, v_draft, parent, true, o_part, part_dtype,
                     l_part, T, Hq, Hkv, D, L, scale, dtype, num_splits, stream);
    if (st != TS_OK) return st;
    return from_hip(launch_importance(q_recent, k_cache, cache_stride, scores, R, Hq, Hkv, D, L, chunk, imp_scale,
                                      dtype, stream), fn);
  }
  ImpFusion f{q_recent, scores, R, imp_scale};
  return attn_common(fn, q, k_cache, v_cache, cache_stride, k_draft, v_draft, parent, true, o_part, part_dtype,
                     l_part, T, Hq, Hkv, D, L, scale, dtype, num_splits, stream, &f);
}

static ts_status check_merge(const char* fn, const void* o_part, ts_dtype part_dtype, const float* l_part,
                             int n_parts, int rows, int D, const void* out, ts_dtype dtype) {
  if (dtype != TS_F32 && dtype != TS_BF16) return fail(TS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (part_dtype != TS_F32 && part_dtype != TS_BF16)
    return fail(TS_ERR_INVALID_ARG, "%s: unknown part_dtype %d", fn, (int)part_dtype);
  if (!o_part || !l_part || !out) return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (n_parts < 1 || rows < 1) return fail(TS_ERR_INVALID_ARG, "%s: n_parts=%d rows=%d must be >= 1", fn, n_parts, rows);
  if (D != 64 && D != 128) return fail(TS_ERR_UNSUPPORTED, "%s: D=%d (supported: 64, 128)", fn, D);
  if (!aligned16(o_part) || ((uintptr_t)out & 7u) != 0)
    return fail(TS_ERR_INVALID_ARG, "%s: o_part must be 16-byte and out 8-byte aligned", fn);
  return TS_OK;
}

ts_status ts_attn_merge(const void* o_part, ts_dtype part_dtype, const float* l_part, int n_parts, int rows, int D,
                        void* out, float* lse, ts_dtype dtype, hipStream_t stream) {
  const char* fn = "ts_attn_merge";
  const ts_status st = check_merge(fn, o_part, part_dtype, l_part, n_parts, rows, D, out, dtype);
  if (st != TS_OK) return st;
  return from_hip(launch_attn_merge(o_part, part_dtype == TS_BF16, l_part, n_parts, rows, D, out, lse, dtype, stream),
                  fn);
}

}  // extern "C"

namespace ts {
// The checks of the shape arguments of the attention calls (shared with the
// no-allocation entry point).
ts_status check_attn_args(const char* fn, int T, int Hq, int Hkv, int D, int64_t L, ts_dtype dtype,
                          int num_splits) {
  return check_attn_shape(fn, T, Hq, Hkv, D, L, dtype, num_splits);
}
ts_status set_error(ts_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace ts

extern "C" {

static ts_status verify_like(const char* fn, const void* q, const void* kc, const void* vc,
                             int64_t cache_stride, const void* kd, const void* vd,
                             const int32_t* parent, bool need_parent, void* out, float* lse,
                             int T, int Hq, int Hkv, int D, int64_t L, float scale,
                             ts_dtype dtype, int num_splits, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, const GatherFusion* gf = nullptr) {
  ts_status st = check_attn_shape(fn, T, Hq, Hkv, D, L, dtype, num_splits);
  if (st != TS_OK) return st;
  if (!out) return fail(TS_ERR_INVALID_ARG, "%s: out is null", fn);
  if (!aligned16(out)) return fail(TS_ERR_INVALID_ARG, "%s: out must be 16-byte aligned", fn);
  if (lse && ((uintptr_t)lse & 3u)) return fail(TS_ERR_INVALID_ARG, "%s: lse misaligned", fn);
  const size_t need = ts_tree_verify_attn_workspace(T, Hq, Hkv, D, L, dtype, num_splits);
  if (!workspace) return fail(TS_ERR_INVALID_ARG, "%s: workspace is null", fn);
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(TS_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  if (workspace_bytes < need)
    return fail(TS_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);
  const AttnPlan p = plan_attention(T, Hq, Hkv, D, L, dtype, num_splits);
  const size_t rows = (size_t)T * Hq;
  // the O partials at the front of the workspace (in the input dtype), then l_part
  void* o_part = workspace;
  float* l_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           align_up((size_t)p.n_splits * rows * D * own_part_elem_bytes(dtype)));
  st = attn_common(fn, q, kc, vc, cache_stride, kd, vd, parent, need_parent, o_part, dtype, l_part, T,
                   Hq, Hkv, D, L, scale, dtype, num_splits, stream, nullptr, gf);
  if (st != TS_OK) return st;
  return from_hip(launch_attn_merge(o_part, dtype == TS_BF16, l_part, p.n_splits, (int)rows, D, out, lse, dtype,
                                    stream), fn);
}

ts_status ts_tree_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                              int64_t cache_stride, const void* k_draft, const void* v_draft,
                              const int32_t* parent, void* out, float* lse, int T, int Hq,
                              int Hkv, int D, int64_t L, float scale, ts_dtype dtype,
                              int num_splits, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return verify_like("ts_tree_verify_attn", q, k_cache, v_cache, cache_stride, k_draft, v_draft,
                     parent, true, out, lse, T, Hq, Hkv, D, L, scale, dtype, num_splits,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace ts {
ts_status tree_verify_into(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                           int64_t cache_stride, const void* k_draft, const void* v_draft, const int32_t* parent,
                           void* out, float* lse, int T, int Hq, int Hkv, int D, int64_t L, float scale,
                           ts_dtype dtype, int num_splits, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return verify_like(fn, q, k_cache, v_cache, cache_stride, k_draft, v_draft, parent, true, out, lse, T, Hq,
                     Hkv, D, L, scale, dtype, num_splits, workspace, workspace_bytes, stream);
}
}  // namespace ts

extern "C" {

size_t ts_partial_draft_attn_workspace(int Tq, int Hq, int Hkv, int D, int64_t P, ts_dtype dtype,
                                       int num_splits) {
  return ts_tree_verify_attn_workspace(Tq, Hq, Hkv, D, P, dtype, num_splits);
}

ts_status ts_partial_draft_attn(const void* q, const void* k_part, const void* v_part,
                                const void* k_new, const void* v_new, void* out, float* lse,
                                int Tq, int Hq, int Hkv, int D, int64_t P, float scale,
                                ts_dtype dtype, int num_splits, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return verify_like("ts_partial_draft_attn", q, k_part, v_part, P, k_new, v_new, nullptr, false,
                     out, lse, Tq, Hq, Hkv, D, P, scale, dtype, num_splits, workspace,
                     workspace_bytes, stream);
}

static ts_status check_importance(const char* fn, const void* q_recent, const void* k_cache,
                                  int64_t cache_stride, const float* scores, int R, int Hq, int Hkv, int D,
                                  int64_t L, int chunk, float scale, ts_dtype dtype) {
  if (dtype != TS_F32 && dtype != TS_BF16) return fail(TS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (!q_recent || !k_cache || !scores) return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned16(q_recent) || !aligned16(k_cache) || ((uintptr_t)scores & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if (R < 1 || Hq < 1 || Hkv < 1) return fail(TS_ERR_INVALID_ARG, "%s: R, Hq, Hkv must be >= 1", fn);
  if (Hq % Hkv) return fail(TS_ERR_INVALID_ARG, "%s: Hq=%d not a multiple of Hkv=%d", fn, Hq, Hkv);
  const int G = Hq / Hkv;
  if (G > 16) return fail(TS_ERR_UNSUPPORTED, "%s: group size %d > 16", fn, G);
  if (R * G > 64) return fail(TS_ERR_UNSUPPORTED, "%s: R*G=%d > 64", fn, R * G);
  if (Hkv > 65535) return fail(TS_ERR_UNSUPPORTED, "%s: Hkv=%d > 65535", fn, Hkv);
  if (D != 64 && D != 128) return fail(TS_ERR_UNSUPPORTED, "%s: D=%d (supported: 64, 128)", fn, D);
  if (chunk < 1 || chunk > 4096) return fail(TS_ERR_UNSUPPORTED, "%s: chunk=%d outside [1, 4096]", fn, chunk);
  if (L < 0) return fail(TS_ERR_INVALID_ARG, "%s: L < 0", fn);
  if (L % chunk) return fail(TS_ERR_UNSUPPORTED, "%s: L=%lld not a multiple of chunk=%d", fn, (long long)L, chunk);
  if (L / chunk > (1 << 24)) return fail(TS_ERR_UNSUPPORTED, "%s: too many chunks", fn);
  if (cache_stride < L) return fail(TS_ERR_INVALID_ARG, "%s: cache_stride < L", fn);
  if (!std::isfinite(scale)) return fail(TS_ERR_INVALID_ARG, "%s: scale not finite", fn);
  return TS_OK;
}

ts_status ts_kv_importance_score(const void* q_recent, const void* k_cache, int64_t cache_stride,
                                 float* scores, int R, int Hq, int Hkv, int D, int64_t L,
                                 int chunk, float scale, ts_dtype dtype, hipStream_t stream) {
  const char* fn = "ts_kv_importance_score";
  const ts_status st = check_importance(fn, q_recent, k_cache, cache_stride, scores, R, Hq, Hkv, D, L, chunk,
                                        scale, dtype);
  if (st != TS_OK) return st;
  return from_hip(launch_importance(q_recent, k_cache, cache_stride, scores, R, Hq, Hkv, D, L,
                                    chunk, scale, dtype, stream), fn);
}

ts_status ts_attn_merge_and_importance(const void* o_part, ts_dtype part_dtype, const float* l_part, int n_parts,
                                       int rows, int Dv, void* out, float* lse, ts_dtype out_dtype,
                                       const void* q_recent, const void* k_cache, int64_t cache_stride, float* scores,
                                       int R, int Hq, int Hkv, int D, int64_t L, int chunk, float scale,
                                       ts_dtype dtype, hipStream_t stream) {
  const char* fn = "ts_attn_merge_and_importance";
  ts_status st = check_merge(fn, o_part, part_dtype, l_part, n_parts, rows, Dv, out, out_dtype);
  if (st != TS_OK) return st;
  st = check_importance(fn, q_recent, k_cache, cache_stride, scores, R, Hq, Hkv, D, L, chunk, scale, dtype);
  if (st != TS_OK) return st;
  if (L > 0 && merge_importance_fusable(n_parts, Dv, D, R, Hq, Hkv, chunk, dtype))
    return from_hip(launch_merge_importance(o_part, part_dtype == TS_BF16, l_part, n_parts, rows, out, lse, out_dtype,
                                            q_recent, k_cache, cache_stride, scores, R, Hq, Hkv, L, scale, stream),
                    fn);
  st = from_hip(launch_attn_merge(o_part, part_dtype == TS_BF16, l_part, n_parts, rows, Dv, out, lse, out_dtype,
                                  stream), fn);
  if (st != TS_OK) return st;
  return from_hip(launch_importance(q_recent, k_cache, cache_stride, scores, R, Hq, Hkv, D, L, chunk, scale, dtype,
                                    stream), fn);
}

static ts_status check_topk(const char* fn, const float* scores, int Hkv, int n_chunks, int k,
                            const int32_t* chunk_idx, const float* chunk_score) {
  if (!scores || !chunk_idx) return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (((uintptr_t)scores & 3u) || ((uintptr_t)chunk_idx & 3u) || ((uintptr_t)chunk_score & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (Hkv < 1 || Hkv > 65535) return fail(TS_ERR_INVALID_ARG, "%s: Hkv=%d", fn, Hkv);
  if (n_chunks < 1 || n_chunks > 65536) return fail(TS_ERR_UNSUPPORTED, "%s: n_chunks=%d outside [1, 65536]", fn, n_chunks);
  if (k < 1 || k > n_chunks) return fail(TS_ERR_INVALID_ARG, "%s: k=%d outside [1, n_chunks=%d]", fn, k, n_chunks);
  return TS_OK;
}

ts_status ts_kv_topk_select(const float* scores, int Hkv, int n_chunks, int k,
                            int32_t* chunk_idx, float* chunk_score, hipStream_t stream) {
  const char* fn = "ts_kv_topk_select";
  const ts_status st = check_topk(fn, scores, Hkv, n_chunks, k, chunk_idx, chunk_score);
  if (st != TS_OK) return st;
  return from_hip(launch_topk(scores, Hkv, n_chunks, k, chunk_idx, chunk_score, stream), fn);
}

ts_status ts_attn_merge_and_topk(const void* o_part, ts_dtype part_dtype, const float* l_part, int n_parts, int rows,
                                 int Dv, void* out, float* lse, ts_dtype out_dtype, const float* scores, int Hkv,
                                 int n_chunks, int k, int32_t* chunk_idx, float* chunk_score, hipStream_t stream) {
  const char* fn = "ts_attn_merge_and_topk";
  ts_status st = check_merge(fn, o_part, part_dtype, l_part, n_parts, rows, Dv, out, out_dtype);
  if (st != TS_OK) return st;
  st = check_topk(fn, scores, Hkv, n_chunks, k, chunk_idx, chunk_score);
  if (st != TS_OK) return st;
  if (merge_topk_fusable(n_parts, Dv))
    return from_hip(launch_merge_topk(o_part, part_dtype == TS_BF16, l_part, n_parts, rows, out, lse, out_dtype,
                                      scores, Hkv, n_chunks, k, chunk_idx, chunk_score, stream), fn);
  st = from_hip(launch_attn_merge(o_part, part_dtype == TS_BF16, l_part, n_parts, rows, Dv, out, lse, out_dtype,
                                  stream), fn);
  if (st != TS_OK) return st;
  return from_hip(launch_topk(scores, Hkv, n_chunks, k, chunk_idx, chunk_score, stream), fn);
}

static ts_status check_gather(const char* fn, const void* k_cache, const void* v_cache, int64_t cache_stride,
                              const int32_t* chunk_idx, int Hkv, int k, int chunk, int D, int64_t L,
                              const void* k_part, const void* v_part, ts_dtype dtype) {
  if (dtype != TS_F32 && dtype != TS_BF16) return fail(TS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (!k_cache || !v_cache || !chunk_idx || !k_part || !v_part)
    return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_part) || !aligned16(v_part) ||
      ((uintptr_t)chunk_idx & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if (Hkv < 1 || Hkv > 65535 || k < 1 || chunk < 1 || D < 1) return fail(TS_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (L < 0 || L % chunk) return fail(TS_ERR_UNSUPPORTED, "%s: L=%lld not a multiple of chunk=%d", fn, (long long)L, chunk);
  if (cache_stride < L) return fail(TS_ERR_INVALID_ARG, "%s: cache_stride < L", fn);
  if (((int64_t)chunk * D * elem_size(dtype)) % 16) return fail(TS_ERR_UNSUPPORTED, "%s: chunk*D*elem not a multiple of 16 bytes", fn);
  if (((int64_t)cache_stride * D * elem_size(dtype)) % 16) return fail(TS_ERR_UNSUPPORTED, "%s: cache head stride not a multiple of 16 bytes", fn);
  if (L / chunk > 2147483647LL) return fail(TS_ERR_UNSUPPORTED, "%s: too many chunks", fn);
  return TS_OK;
}

ts_status ts_kv_gather(const void* k_cache, const void* v_cache, int64_t cache_stride,
                       const int32_t* chunk_idx, int Hkv, int k, int chunk, int D, int64_t L,
                       void* k_part, void* v_part, ts_dtype dtype, hipStream_t stream) {
  const char* fn = "ts_kv_gather";
  const ts_status st = check_gather(fn, k_cache, v_cache, cache_stride, chunk_idx, Hkv, k, chunk, D, L, k_part,
                                    v_part, dtype);
  if (st != TS_OK) return st;
  return from_hip(launch_gather(k_cache, v_cache, cache_stride, chunk_idx, Hkv, k, chunk, D, L,
                                k_part, v_part, elem_size(dtype), stream), fn);
}

ts_status ts_kv_gather_and_draft_attn(const void* k_cache, const void* v_cache, int64_t cache_stride,
                                      const int32_t* chunk_idx, int k, int chunk, int64_t L, void* k_part,
                                      void* v_part, const void* q, const void* k_new, const void* v_new,
                                      void* out, float* lse, int Tq, int Hq, int Hkv, int D, float scale,
                                      ts_dtype dtype, int num_splits, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  const char* fn = "ts_kv_gather_and_draft_attn";
  ts_status st = check_gather(fn, k_cache, v_cache, cache_stride, chunk_idx, Hkv, k, chunk, D, L, k_part, v_part,
                              dtype);
  if (st != TS_OK) return st;
  if ((int64_t)k * chunk > (int64_t)INT32_MAX) return fail(TS_ERR_UNSUPPORTED, "%s: k*chunk too large", fn);
  const int64_t P = (int64_t)k * chunk;
  st = check_attn_shape(fn, Tq, Hq, Hkv, D, P, dtype, num_splits);
  if (st != TS_OK) return st;
  // every argument of the draft pass is checked before anything runs
  if (!q || !k_new || !v_new || !out || !workspace) return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) || ((uintptr_t)lse & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(TS_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  const size_t need = ts_tree_verify_attn_workspace(Tq, Hq, Hkv, D, P, dtype, num_splits);
  if (workspace_bytes < need)
    return fail(TS_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu required", fn, workspace_bytes, need);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(TS_ERR_INVALID_ARG, "%s: scale must be finite and > 0 (got %g)", fn, (double)scale);
  const AttnPlan p = plan_attention(Tq, Hq, Hkv, D, P, dtype, num_splits);
  if (((int64_t)p.n_splits * Hkv + 7) / 8 * 8 * p.n_rowgroups > INT32_MAX)
    return fail(TS_ERR_UNSUPPORTED, "%s: %d splits x %d KV heads exceed one launch", fn, p.n_splits, Hkv);
  if (dtype == TS_BF16 && chunk == kTile && p.path == kPathSmall) {
    const GatherFusion gf{chunk_idx, L / chunk, k_part, v_part};
    return verify_like(fn, q, k_cache, v_cache, cache_stride, k_new, v_new, nullptr, false, out, lse, Tq, Hq, Hkv,
                       D, P, scale, dtype, num_splits, workspace, workspace_bytes, stream, &gf);
  }
  st = from_hip(launch_gather(k_cache, v_cache, cache_stride, chunk_idx, Hkv, k, chunk, D, L, k_part, v_part,
                              elem_size(dtype), stream), fn);
  if (st != TS_OK) return st;
  return verify_like(fn, q, k_part, v_part, P, k_new, v_new, nullptr, false, out, lse, Tq, Hq, Hkv, D, P, scale,
                     dtype, num_splits, workspace, workspace_bytes, stream);
}

// Node count of a tree shape, or -1 (with ts_last_error) if the shape is not supported.
static int tree_shape(const char* fn, const int32_t* shape, int depth, TreeShape* out) {
  if (!shape) { fail(TS_ERR_INVALID_ARG, "%s: shape is null", fn); return -1; }
  if (depth < 1 || depth > kTreeMaxDepth) {
    fail(TS_ERR_UNSUPPORTED, "%s: depth=%d outside [1, %d]", fn, depth, kTreeMaxDepth);
    return -1;
  }
  TreeShape sh{};
  int64_t total = 0, n = 1;
  for (int d = 0; d < depth; ++d) {
    if (shape[d] < 1 || shape[d] > kTreeMaxK) {
      fail(TS_ERR_UNSUPPORTED, "%s: shape[%d]=%d outside [1, %d]", fn, d, shape[d], kTreeMaxK);
      return -1;
    }
    n *= shape[d];
    if (total + n > kTreeMaxNodes) {
      fail(TS_ERR_UNSUPPORTED, "%s: more than %d nodes", fn, kTreeMaxNodes);
      return -1;
    }
    sh.k[d] = shape[d];
    sh.n[d] = (int)n;
    sh.off[d] = (int)total;
    total += n;
  }
  if (out) *out = sh;
  return (int)total;
}

int ts_draft_tree_nodes(const int32_t* shape, int depth) {
  return tree_shape("ts_draft_tree_nodes", shape, depth, nullptr);
}

size_t ts_build_draft_tree_workspace(int V, int depth) {
  if (V < 1 || depth < 1 || depth > kTreeMaxDepth) return 0;
  return align_up((size_t)depth * tree_slices(V) * kTreeMaxK * sizeof(uint64_t));
}

ts_status ts_build_draft_tree(const void* logits, int P, int V, const int32_t* shape, int depth,
                              int32_t* parent, int32_t* draft_tok, int32_t* cand, ts_dtype dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "ts_build_draft_tree";
  if (dtype != TS_F32 && dtype != TS_BF16) return fail(TS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (!logits || !parent || !draft_tok) return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (((uintptr_t)logits % elem_size(dtype)) || ((uintptr_t)parent & 3u) || ((uintptr_t)draft_tok & 3u) ||
      ((uintptr_t)cand & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  TreeShape sh;
  if (tree_shape(fn, shape, depth, &sh) < 0) return TS_ERR_UNSUPPORTED;
  if (P < depth) return fail(TS_ERR_INVALID_ARG, "%s: P=%d positions for depth %d", fn, P, depth);
  if (V < 1) return fail(TS_ERR_INVALID_ARG, "%s: V=%d", fn, V);
  for (int d = 0; d < depth; ++d)
    if (shape[d] > V) return fail(TS_ERR_INVALID_ARG, "%s: shape[%d]=%d > V=%d", fn, d, shape[d], V);
  if (!workspace || ((uintptr_t)workspace & 255u)) return fail(TS_ERR_INVALID_ARG, "%s: workspace null or not 256-byte aligned", fn);
  if (workspace_bytes < ts_build_draft_tree_workspace(V, depth))
    return fail(TS_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                ts_build_draft_tree_workspace(V, depth));
  return from_hip(launch_build_tree(logits, V, sh, depth, parent, draft_tok, cand, workspace, dtype, stream), fn);
}

ts_status ts_accept_commit(const int32_t* parent, const int32_t* draft_tok, const int32_t* target_tok,
                           uint32_t rand_u32, int T, void* k_cache, void* v_cache, int64_t cache_stride,
                           int64_t L, const void* k_draft, const void* v_draft, int Hkv, int D,
                           ts_dtype dtype, int32_t* n_accepted, int32_t* path, int32_t* bonus,
                           hipStream_t stream) {
  const char* fn = "ts_accept_commit";
  if (dtype != TS_F32 && dtype != TS_BF16) return fail(TS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (!parent || !draft_tok || !target_tok || !k_cache || !v_cache || !k_draft || !v_draft ||
      !n_accepted || !path || !bonus)
    return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_draft) || !aligned16(v_draft) ||
      ((uintptr_t)parent & 3u) || ((uintptr_t)draft_tok & 3u) || ((uintptr_t)target_tok & 3u) ||
      ((uintptr_t)n_accepted & 3u) || ((uintptr_t)path & 3u) || ((uintptr_t)bonus & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned (int32 arrays 4-byte)", fn);
  if (T < 1 || T > TS_MAX_DRAFT) return fail(TS_ERR_INVALID_ARG, "%s: T=%d outside [1, %d]", fn, T, TS_MAX_DRAFT);
  if (Hkv < 1 || Hkv > 65535) return fail(TS_ERR_INVALID_ARG, "%s: Hkv=%d", fn, Hkv);
  if (D != 64 && D != 128) return fail(TS_ERR_UNSUPPORTED, "%s: D=%d (64 or 128)", fn, D);
  if (L < 0) return fail(TS_ERR_INVALID_ARG, "%s: L=%lld < 0", fn, (long long)L);
  if (cache_stride < L + T)
    return fail(TS_ERR_INVALID_ARG, "%s: cache_stride=%lld leaves no room for %d rows after L=%lld", fn,
                (long long)cache_stride, T, (long long)L);
  return from_hip(launch_accept_commit(parent, draft_tok, target_tok, rand_u32, T, k_cache, v_cache,
                                       cache_stride, L, k_draft, v_draft, Hkv, D, elem_size(dtype),
                                       n_accepted, path, bonus, stream), fn);
}

size_t ts_sample_workspace(int R, int V) {
  if (R < 1 || R > TS_MAX_DRAFT + 1 || V < 1 || V > kSampleSub * kSampleMaxSubs) return 0;
  return align_up(sample_workspace_bytes(R, V));
}

ts_status ts_sample_tokens(const void* logits, int R, int V, const int32_t* hist, int n_hist,
                           const int32_t* parent, const int32_t* draft_tok, int T, int window,
                           float penalty, float temperature, float min_p, float top_p, const float* u,
                           int32_t* tok, ts_dtype dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const char* fn = "ts_sample_tokens";
  if (dtype != TS_F32 && dtype != TS_BF16) return fail(TS_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (T < 0 || T > TS_MAX_DRAFT) return fail(TS_ERR_INVALID_ARG, "%s: T=%d outside [0, %d]", fn, T, TS_MAX_DRAFT);
  if (R != T + 1) return fail(TS_ERR_INVALID_ARG, "%s: R=%d rows for T=%d drafts (R = T + 1)", fn, R, T);
  if (V < 1 || V > kSampleSub * kSampleMaxSubs)
    return fail(TS_ERR_UNSUPPORTED, "%s: V=%d outside [1, %d]", fn, V, kSampleSub * kSampleMaxSubs);
  if (n_hist < 0 || window < 0) return fail(TS_ERR_INVALID_ARG, "%s: n_hist=%d window=%d", fn, n_hist, window);
  if (!logits || !tok || (n_hist > 0 && !hist) || (T > 0 && (!parent || !draft_tok)) ||
      (temperature > 0.0f && !u))
    return fail(TS_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (((uintptr_t)logits % elem_size(dtype)) || ((uintptr_t)hist & 3u) || ((uintptr_t)parent & 3u) ||
      ((uintptr_t)draft_tok & 3u) || ((uintptr_t)u & 3u) || ((uintptr_t)tok & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (!(penalty > 0.0f) || !std::isfinite(penalty)) return fail(TS_ERR_INVALID_ARG, "%s: penalty=%g", fn, penalty);
  if (!(temperature >= 0.0f) || !std::isfinite(temperature))
    return fail(TS_ERR_INVALID_ARG, "%s: temperature=%g", fn, temperature);
  if (!(min_p >= 0.0f && min_p <= 1.0f)) return fail(TS_ERR_INVALID_ARG, "%s: min_p=%g outside [0, 1]", fn, min_p);
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(TS_ERR_INVALID_ARG, "%s: top_p=%g outside (0, 1]", fn, top_p);
  if (!workspace || ((uintptr_t)workspace & 255u)) return fail(TS_ERR_INVALID_ARG, "%s: workspace null or not 256-byte aligned", fn);
  const size_t need = ts_sample_workspace(R, V);
  if (workspace_bytes < need) return fail(TS_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  SampleArgs a{};
  a.logits = logits;
  a.R = R;
  a.V = V;
  a.hist = hist;
  a.n_hist = n_hist;
  a.parent = parent;
  a.draft_tok = draft_tok;
  a.T = T;
  a.window = window;
  a.theta = penalty;
  a.inv_theta = (float)(1.0 / (double)penalty);
  // greedy keeps s2 = 0; a tiny temperature saturates at a finite scale so that 0 * s2 stays 0
  a.s2 = temperature > 0.0f ? (float)std::fmin(1.4426950408889634 / (double)temperature, 1e30) : 0.0f;
  // greedy: the cut sits at the maximum, so the kept tokens are the maxima
  a.cut = temperature == 0.0f ? 0.0f
          : min_p > 0.0f      ? (float)((double)temperature * std::log((double)min_p))
                              : -INFINITY;
  a.u = u;
  a.tok = tok;
  a.nb = sample_subslices(V);
  // the top-p row records first: each on a 128-byte line of its own
  a.topp_row = static_cast<ToppRow*>(workspace);
  a.sub = reinterpret_cast<SampleSub*>(a.topp_row + R);
  a.cand = reinterpret_cast<SampleCand*>(a.sub + (size_t)R * a.nb);
  a.wbits = reinterpret_cast<uint32_t*>(a.cand + (size_t)R * a.nb * kSampleList);
  // top-p is off at 1 (every token of non-zero weight has less than the whole
  // weight above it) and under greedy decoding (the maximum always survives)
  a.top_p = top_p;
  // (the per-sub-slice bins first: 16-byte aligned for their vector reads)
  const bool topp = top_p < 1.0f && temperature > 0.0f;
  a.topp_hist = topp ? reinterpret_cast<float*>(a.wbits + (size_t)R * a.nb * (kSampleSub / 32)) : nullptr;
  a.topp_above = topp ? a.topp_hist + (size_t)R * a.nb * kToppCoarseBins : nullptr;
  a.topp_key = topp ? reinterpret_cast<uint32_t*>(a.topp_above + (size_t)R * a.nb) : nullptr;
  a.topp_id = topp ? reinterpret_cast<int32_t*>(a.topp_key + (size_t)R * kToppCandMax) : nullptr;
  a.topp_cut = topp ? reinterpret_cast<float*>(a.topp_id + (size_t)R * kToppCandMax) : nullptr;
  if (!topp) a.topp_row = nullptr;
  return from_hip(launch_sample(a, dtype, stream), fn);
}

static_assert(sizeof(ts_ngram_header) == sizeof(NgramHeader), "header layouts agree");

size_t ts_ngram_table_bytes(int capacity_log2, int max_entries) {
  if (capacity_log2 < 4 || capacity_log2 > kNgramMaxCapacityLog2 || max_entries < 1 ||
      max_entries > kNgramMaxEntries || max_entries > (1 << capacity_log2))
    return 0;
  return align_up(ngram_table_bytes(capacity_log2, max_entries));
}

ts_status ts_ngram_init(void* table, size_t table_bytes, int capacity_log2, int max_entries, hipStream_t stream) {
  const char* fn = "ts_ngram_init";
  const size_t need = ts_ngram_table_bytes(capacity_log2, max_entries);
  if (need == 0)
    return fail(TS_ERR_UNSUPPORTED, "%s: capacity_log2=%d max_entries=%d (capacity_log2 in [4, %d], max_entries in "
                "[1, %d] and at most the capacity)", fn, capacity_log2, max_entries, kNgramMaxCapacityLog2,
                kNgramMaxEntries);
  if (!table || ((uintptr_t)table & 255u)) return fail(TS_ERR_INVALID_ARG, "%s: table null or not 256-byte aligned", fn);
  if (table_bytes < need) return fail(TS_ERR_WORKSPACE, "%s: table %zu < %zu bytes", fn, table_bytes, need);
  return from_hip(launch_ngram_init(ngram_view(table, capacity_log2), capacity_log2, max_entries, stream), fn);
}

ts_status ts_ngram_update(void* table, const int32_t* tokens, int64_t from, int64_t to, hipStream_t stream) {
  const char* fn = "ts_ngram_update";
  if (!table || ((uintptr_t)table & 255u)) return fail(TS_ERR_INVALID_ARG, "%s: table null or not 256-byte aligned", fn);
  if (from < 0 || to < from || to > 2147483647LL)
    return fail(TS_ERR_INVALID_ARG, "%s: from=%lld to=%lld", fn, (long long)from, (long long)to);
  if (to > 3 && (!tokens || ((uintptr_t)tokens & 3u)))
    return fail(TS_ERR_INVALID_ARG, "%s: tokens null or misaligned", fn);
  return from_hip(launch_ngram_update(table, tokens, from, to, stream), fn);
}

size_t ts_ngram_retrieve_workspace(int max_entries, int k) {
  if (max_entries < 1 || max_entries > kNgramMaxEntries || k < 1 || k > kNgramMaxK) return 0;
  return align_up(ngram_retrieve_workspace_bytes(max_entries, k));
}

ts_status ts_ngram_retrieve(const void* table, int max_entries, const int32_t* first_tok, int k,
                            int32_t* out_tok, int32_t* out_count, int32_t* n_found, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "ts_ngram_retrieve";
  if (max_entries < 1 || max_entries > kNgramMaxEntries || k < 1 || k > kNgramMaxK)
    return fail(TS_ERR_UNSUPPORTED, "%s: max_entries=%d k=%d (max_entries in [1, %d], k in [1, %d])", fn,
                max_entries, k, kNgramMaxEntries, kNgramMaxK);
  if (!table || ((uintptr_t)table & 255u)) return fail(TS_ERR_INVALID_ARG, "%s: table null or not 256-byte aligned", fn);
  if (!first_tok || !out_tok || ((uintptr_t)first_tok & 3u) || ((uintptr_t)out_tok & 3u) ||
      ((uintptr_t)out_count & 3u) || ((uintptr_t)n_found & 3u))
    return fail(TS_ERR_INVALID_ARG, "%s: null or misaligned pointer", fn);
  if (!workspace || ((uintptr_t)workspace & 255u)) return fail(TS_ERR_INVALID_ARG, "%s: workspace null or not 256-byte aligned", fn);
  const size_t need = ts_ngram_retrieve_workspace(max_entries, k);
  if (workspace_bytes < need) return fail(TS_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  return from_hip(launch_ngram_retrieve(const_cast<void*>(table), max_entries, first_tok, k, out_tok, out_count,
                                        n_found, workspace, stream), fn);
}

}  // extern "C"
