/*
 * ts_probe.h -- measurement probes of libts_probe.so (MI355X, gfx950).
 *
 * Not part of the hot path: these kernels measure what this GPU sustains
 * (matrix-core bf16 rate, vector-ALU issue rates, LDS read bandwidth, plain
 * streaming reads from HBM), so that the kernels' roofline fractions can also be stated against
 * measured ceilings next to the published peaks. The benchmark calls them.
 *
 * Every call enqueues one launch on `stream` and returns 0, or a hipError_t
 * code if the launch failed. `sink` is a device buffer of at least 1024 bytes
 * the kernels may write to (so that the compiler keeps their work); its
 * contents are meaningless.
 */
#ifndef TS_PROBE_H_
#define TS_PROBE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One workgroup per compute unit (256), `waves_per_simd` (1 or 2) waves on each
 * of a CU's 4 SIMDs, every wave issuing `iters` rounds of 4 independent
 * v_mfma_f32_32x32x16_bf16 chains. With `toggle` non-zero the A operand's
 * low mantissa bits flip every round (changing data, as in a real kernel,
 * draws more power than constant operands). Dense flops of one launch:
 * ts_probe_mfma_bf16_flops(waves_per_simd, iters). */
int ts_probe_mfma_bf16(int waves_per_simd, int toggle, int iters, float* sink, hipStream_t stream);
double ts_probe_mfma_bf16_flops(int waves_per_simd, int iters);

/* Vector-ALU issue: one workgroup per CU with 2 waves on each SIMD, every wave
 * issuing `iters` rounds of 16 independent dependency chains of v_fma_f32
 * (op 0) or v_exp_f32 (op 1). Wave instructions per SIMD of one launch:
 * 2 * 16 * iters. */
int ts_probe_valu(int op, int iters, float* sink, hipStream_t stream);

/* LDS read bandwidth: one 512-thread workgroup per CU, every wave issuing
 * `iters` rounds of 16 reads of its own slices of a 96 KB LDS array, as
 * ds_read_b128 (transposed = 0, 1 KB a wave read) or ds_read_b64_tr_b16
 * (transposed != 0, 512 B a wave read). Bytes of one launch:
 * ts_probe_lds_read_bytes(transposed, iters). */
int ts_probe_lds_read(int transposed, int iters, uint32_t* sink, hipStream_t stream);
double ts_probe_lds_read_bytes(int transposed, int iters);

/* A plain streaming read of `bytes` (a multiple of 16, 16-byte aligned) with
 * 16-byte loads, consecutive lanes on consecutive 16 bytes and eight loads in
 * flight per thread. */
int ts_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* TS_PROBE_H_ */
