// Measurement probes (libts_probe.so): the matrix-core bf16 rate, vector-ALU
// issue rates, LDS read bandwidth and a plain HBM streaming read, as this GPU
// sustains them. The
// benchmark states the hot-path kernels' fractions against these next to the
// published peaks. Nothing here is part of the hot path.
#include <hip/hip_runtime.h>

#include "../../include/ts_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kCUs = 256;
constexpr int kChains = 4;

// Operands differ per lane and are small, so the accumulators stay finite.
// With kToggle the A operand's mantissa bits flip every round (one vector
// xor per four products), so that the matrix cores see changing data as in a
// real kernel: the power drawn, and so the clock the chip settles at under
// load, depends on it.
template <int kThreads, bool kToggle>
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float* sink) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(((threadIdx.x * 7 + e * 3) & 15) * (1.0f / 4096.0f) - 0.001f);
    b[e] = static_cast<__bf16>(((threadIdx.x * 5 + e * 11) & 15) * (1.0f / 4096.0f) - 0.0015f);
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
    if constexpr (kToggle) {
      // flip the low 7 mantissa bits of every bf16 element of A
      uint4 u = __builtin_bit_cast(uint4, a);
      u.x ^= 0x007F007Fu; u.y ^= 0x007F007Fu; u.z ^= 0x007F007Fu; u.w ^= 0x007F007Fu;
      a = __builtin_bit_cast(bf16x8_t, u);
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[threadIdx.x & 255] = s;
}

template <int kOp>
__global__ __launch_bounds__(512) void valu_probe_kernel(int iters, float* sink) {
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = (threadIdx.x + j) * 1e-6f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (kOp == 0) v[j] = fmaf(v[j], 0.999f, 1e-7f);
      else v[j] = __builtin_amdgcn_exp2f(-v[j]);     // stays in [0.5, 1]; the negation is a source modifier
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += v[j];
  sink[threadIdx.x & 255] = s;
}

constexpr int kReadThreads = 256;
constexpr int kReadBatch = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                                   uint32_t* sink) {
  uint32_t acc = 0u;
  const size_t step = (size_t)gridDim.x * kReadThreads * kReadBatch;
  size_t i = (size_t)blockIdx.x * kReadThreads * kReadBatch + threadIdx.x;
  for (; i + (kReadBatch - 1) * kReadThreads < n16; i += step) {
    uint4 v[kReadBatch];
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) v[u] = p[i + u * kReadThreads];
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += kReadThreads) acc ^= p[i].x;
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;    // keeps the loads; practically never taken
}

// LDS read bandwidth: one 512-thread workgroup per CU over a 96 KB LDS array,
// every wave reading its own 1 KB (kTr: 512 B) slices, 16 reads a round, as
// ds_read_b128 (kTr false) or the transposing ds_read_b64_tr_b16 that feeds
// the V^T operand of the verify kernel's PV product (kTr true). The XOR of
// the results keeps the reads; the vector ALU work per read is below the LDS
// time.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kLdsVec = 6144;                    // 16-byte elements: 96 KB

template <bool kTr>
__global__ __launch_bounds__(512) void lds_read_probe_kernel(int iters, uint32_t* sink) {
  __shared__ u32x4_t buf[kLdsVec];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsVec; i += 512) buf[i] = u32x4_t{(uint32_t)i, (uint32_t)i + 1u, 7u, 9u};
  __syncthreads();
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(&buf[0]);
  uint32_t acc = 0u;
  if constexpr (kTr) {
    s16x4_t x = {0, 0, 0, 0};
    const uint32_t base = (uint32_t)(wave * 512 + lane * 8);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t off = (base + (uint32_t)r * 4096u + (uint32_t)it * 512u) % (uint32_t)(kLdsVec * 16);
        x ^= __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) s16x4_t*>(lds0 + off));
      }
    }
    // all 32 bits of acc depend on the reads (a 16-bit result could never equal
    // the test value below, and the reads would be dropped)
    acc = (((uint32_t)(uint16_t)x[0] << 16) | (uint16_t)x[1]) ^ (((uint32_t)(uint16_t)x[2] << 16) | (uint16_t)x[3]);
  } else {
    u32x4_t x = {0u, 0u, 0u, 0u};
    const int base = lane + wave * 64;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 16; ++r) x ^= buf[(base + r * 512 + it * 64) % kLdsVec];
    }
    acc = x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  if (acc == 0x9e3779b9u) sink[tid & 255] = acc;    // keeps the reads; practically never taken
}

}  // namespace

extern "C" {

int ts_probe_lds_read(int transposed, int iters, uint32_t* sink, hipStream_t stream) {
  if (!sink || iters < 1) return (int)hipErrorInvalidValue;
  if (transposed) lds_read_probe_kernel<true><<<kCUs, 512, 0, stream>>>(iters, sink);
  else lds_read_probe_kernel<false><<<kCUs, 512, 0, stream>>>(iters, sink);
  return (int)hipGetLastError();
}

double ts_probe_lds_read_bytes(int transposed, int iters) {
  // 256 workgroups x 8 waves x 16 reads a round; 1 KB (b128) or 512 B (tr_b64) a wave read
  return (double)kCUs * 8 * 16 * (double)iters * (transposed ? 512.0 : 1024.0);
}

int ts_probe_mfma_bf16(int waves_per_simd, int toggle, int iters, float* sink, hipStream_t stream) {
  if (!sink || iters < 1 || (waves_per_simd != 1 && waves_per_simd != 2)) return (int)hipErrorInvalidValue;
  if (waves_per_simd == 1) {
    if (toggle) mfma_probe_kernel<256, true><<<kCUs, 256, 0, stream>>>(iters, sink);
    else mfma_probe_kernel<256, false><<<kCUs, 256, 0, stream>>>(iters, sink);
  } else {
    if (toggle) mfma_probe_kernel<512, true><<<kCUs, 512, 0, stream>>>(iters, sink);
    else mfma_probe_kernel<512, false><<<kCUs, 512, 0, stream>>>(iters, sink);
  }
  return (int)hipGetLastError();
}

double ts_probe_mfma_bf16_flops(int waves_per_simd, int iters) {
  // 32 x 32 x 16 multiply-adds per instruction
  return (double)kCUs * 4 * waves_per_simd * (double)iters * kChains * (2.0 * 32 * 32 * 16);
}

int ts_probe_valu(int op, int iters, float* sink, hipStream_t stream) {
  if (!sink || iters < 1 || (op != 0 && op != 1)) return (int)hipErrorInvalidValue;
  if (op == 0) valu_probe_kernel<0><<<kCUs, 512, 0, stream>>>(iters, sink);
  else valu_probe_kernel<1><<<kCUs, 512, 0, stream>>>(iters, sink);
  return (int)hipGetLastError();
}

int ts_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || (bytes & 15u) || ((uintptr_t)buf & 15u)) return (int)hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const size_t per_block = (size_t)kReadThreads * kReadBatch;
  size_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > (size_t)kCUs * 16) blocks = (size_t)kCUs * 16;
  if (blocks < 1) blocks = 1;
  stream_read_kernel<<<(unsigned)blocks, kReadThreads, 0, stream>>>(static_cast<const uint4*>(buf), n16, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
