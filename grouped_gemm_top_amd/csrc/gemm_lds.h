// gemm_lds.h -- building blocks shared by the bf16 grouped-GEMM kernels (internal, not part of
// the ABI): vector types, buffer descriptors, the direct-to-LDS loads, bf16 packing, the MFMA
// wrapper and the memory-counter waits.
#pragma once

#include "gemm_common.h"

namespace moe {
namespace gk {

using gg::rsrc_t;
using gg::ufl;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// LDS loads.  They are written as inline assembly on purpose: the compiler then does not
// track them as LDS writes and inserts no vmcnt waits of its own before LDS reads (it cannot
// tell the ring stages apart and would drain every load in flight).  Completion is ordered
// explicitly instead: every stage is read only after the vmcnt wait and barrier that follow
// its loads.  M0 holds the wavefront's LDS destination; lane L writes at M0 + 16 L (4 L for
// the 4-byte form).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 dmadesc(const void* p, long long bytes) {
  const uint64_t a = (uint64_t)p;
  const int n = bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes;
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), n, 0x00020000};
}
__device__ __forceinline__ i32x4 dmadesc_off(const void* p, long long off, long long bytes) {
  return dmadesc(static_cast<const char*>(p) + off, bytes);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p);
}
// The descriptor and the LDS address are wavefront-uniform; readfirstlane puts them in SGPRs.
// The compiler's hazard recognizer does not look inside inline assembly, so the required
// wait states are spelled out: a vector-memory instruction may read an SGPR only 5 wait
// states after a VALU instruction (such as readfirstlane) wrote it, and an LDS load needs 1
// after M0 was written.  s_nop 4 gives 5.
__device__ __forceinline__ i32x4 sgpr4(const i32x4& r) {
  return i32x4{ufl(r.x), ufl(r.y), ufl(r.z), ufl(r.w)};
}
// m0: LDS byte address of the wavefront's destination; voff: per-lane byte offset; soff: a
// wavefront-uniform byte offset added to every lane's address.  Every use below keeps each
// valid lane's voff + soff inside its tensor, and gives masked lanes a voff at or beyond the
// descriptor range, so both operands of a masked access fail the range check.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0)
               : "memory");
}
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t m0, uint32_t voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(sgpr4(r)), "{m0}"(m0)
               : "memory");
}
// the same with a wavefront-uniform byte offset soff (r already in SGPRs)
__device__ __forceinline__ void dma4s(const i32x4& r, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0)
               : "memory");
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two fp32 values to two bf16 (v_cvt_pk_bf16_f32: round to nearest even, the same bits as
// the scalar rounding for every finite value).
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wait until at most N vector-memory instructions of this wavefront are outstanding, then
// meet the other wavefronts.  The memory clobber keeps every LDS access on its side.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// K-strided operand rows in LDS: column chunk c (8 values) of k-row k sits at position c ^ f(k).
// f(k) takes 8 even values over k-rows 0-3 and 8-11 (and again over 16-19 and 24-27), so the
// 32-byte segments that one transposing read takes from 16 k-rows cover every bank once per
// half-wavefront for rows of 256 or 512 bytes.
__device__ __forceinline__ int mn_f(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

}  // namespace gk
}  // namespace moe
