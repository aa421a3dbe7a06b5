/*
 * moe_probe.h -- C ABI of libmoe_probe.so: measurement probes for the two device peaks the
 * layer's kernels are compared against on MI355X (gfx950): dense bf16 MFMA throughput and
 * HBM streaming bandwidth.  They compute nothing of the layer; bench.py times them with HIP
 * events and reports the measured peaks beside the published ones.
 *
 * Contract: pointers are DEVICE pointers owned by the caller; `stream` is a hipStream_t
 * passed as void* (NULL: the default stream); nothing is allocated, freed or synchronised.
 * Every call validates its arguments before queueing anything and returns 0 on success,
 * 1 for invalid arguments (nothing queued) and 4 for a launch error.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 MFMA probe.  `blocks` workgroups of 256 threads (four wavefronts); each
 * wavefront runs `iters` iterations of eight independent MFMAs on register operands:
 *   shape 0: v_mfma_f32_16x16x32_bf16 (16384 FLOP each)
 *   shape 1: v_mfma_f32_32x32x16_bf16 (32768 FLOP each; four per iteration, so the FLOPs
 *            per iteration match shape 0)
 * so one launch performs blocks * 4 * iters * 131072 FLOP.  sink: blocks * 256 floats, one
 * per thread (keeps the results live).  1 <= blocks <= 65536, 1 <= iters <= 1 << 24. */
int moe_probe_mfma_bf16(int shape, int blocks, int iters, float* sink, void* stream);

/* Streaming copy probe: dst[i] = src[i] for `bytes` bytes with 16-byte loads and stores,
 * `blocks` workgroups of 256 threads striding over the buffer.  bytes must be a multiple
 * of 16 and both pointers 16-byte aligned; 1 <= blocks <= 65536. */
int moe_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

/* Streaming read probe: reads `bytes` bytes of src with 16-byte loads and writes the XOR of
 * each thread's words to sink[blocks * 256] (uint32).  Same constraints as moe_probe_copy. */
int moe_probe_read(const void* src, size_t bytes, int blocks, uint32_t* sink, void* stream);

/* Lane-layout probe of the scaled fp8 matrix instruction (v_mfma_scale_f32_16x16x128_f8f6f4,
 * e4m3 operands): one wavefront per case runs one instruction with a zero accumulator.
 * For case c and lane L: a, b hold 32 bytes each at [(c*64 + L)*32] (the lane's operand
 * registers), sa, sb one dword each at [c*64 + L] (the lane's scale registers, byte 0
 * selected), and d receives the lane's four result floats at [(c*64 + L)*4].  1 <= cases <=
 * 4096; a, b, d 16-byte aligned. */
int moe_probe_mfma_fp8_layout(const uint8_t* a, const uint8_t* b, const uint32_t* sa, const uint32_t* sb,
                              int cases, float* d, void* stream);

/* fp32 -> fp8 e4m3 with the conversion instruction the fp8 kernels use (v_cvt_pk_fp8_f32):
 * dst[i] = code of src[i], i < n; n even, dst 2-byte aligned. */
int moe_probe_cvt_fp8(const float* src, int n, uint8_t* dst, void* stream);

/* Re-read probe: reads the `bytes` bytes of src (a multiple of 1024, at most 1 GiB, 16-byte
 * aligned) `passes` times over (1..4096) as kilobyte loads, one wavefront each, `blocks`
 * workgroups of 256 threads (1..65536).  mode 0 loads into registers and writes each
 * thread's XOR of the words it read to sink[blocks * 256]; mode 1 loads into LDS with
 * buffer_load_dwordx4 ... lds (the form the GEMM kernels use) and writes 0 there; mode 2 is
 * mode 1 with each kilobyte's 16-byte chunks taken in the lane order of the GEMMs' K-strided
 * stages. */
int moe_probe_reread(const void* src, size_t bytes, int passes, int mode, int blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
