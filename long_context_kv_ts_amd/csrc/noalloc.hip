// ts_tree_verify_attn without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The split partials live in `scratch`, a file-scope device array of
// TS_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
// process ends. Host code never passes the array's name to a kernel (on the
// host it is only a stand-in, not a device address): at the first call on a
// device, with that device current, hipGetSymbolAddress gives this device's
// copy of the array, and that pointer is kept per device and handed to the
// kernels as the workspace of ts_tree_verify_attn. Nothing in the array needs
// to start at zero (every partial is written before it is read), and calls
// on one device share it: calls that overlap on one GPU race.
#include <cstdio>
#include <mutex>

#include "common.h"

namespace {

static __device__ __align__(256) unsigned char scratch[TS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];       // this library's scratch on each device, once looked up

}  // namespace

extern "C" ts_status ts_tree_verify_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                 int64_t cache_stride, const void* k_draft, const void* v_draft,
                                                 const int32_t* parent, void* out, float* lse, int T, int Hq,
                                                 int Hkv, int D, int64_t L, float scale, ts_dtype dtype,
                                                 int num_splits, hipStream_t stream) {
  const char* fn = "ts_tree_verify_attn_noalloc";
  // sizes first, on the host, before any HIP call
  const ts_status st = ts::check_attn_args(fn, T, Hq, Hkv, D, L, dtype, num_splits);
  if (st != TS_OK) return st;
  const size_t need = ts_tree_verify_attn_workspace(T, Hq, Hkv, D, L, dtype, num_splits);
  if (need > (size_t)TS_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "%s: the split partials of this call need %zu bytes, more than the %zu bytes of static scratch "
             "(use ts_tree_verify_attn with a workspace, or fewer splits)",
             fn, need, (size_t)TS_NOALLOC_SCRATCH_BYTES);
    return ts::set_error(TS_ERR_UNSUPPORTED, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof msg, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return ts::set_error(TS_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) return ts::set_error(TS_ERR_UNSUPPORTED, "ts_tree_verify_attn_noalloc: device id >= 64");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
      // this device's copy of the array (the current device is `dev`)
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || ptr == nullptr) {
        char msg[256];
        snprintf(msg, sizeof msg, "%s: hipGetSymbolAddress: %s", fn, hipGetErrorString(e));
        return ts::set_error(TS_ERR_HIP, msg);
      }
      g_scratch[dev] = ptr;
    }
    ptr = g_scratch[dev];
  }
  return ts::tree_verify_into(fn, q, k_cache, v_cache, cache_stride, k_draft, v_draft, parent, out, lse, T, Hq,
                              Hkv, D, L, scale, dtype, num_splits, ptr, (size_t)TS_NOALLOC_SCRATCH_BYTES, stream);
}
