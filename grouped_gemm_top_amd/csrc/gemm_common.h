// gemm_common.h -- definitions shared by the grouped-GEMM kernels (internal, not part of the ABI).
#pragma once

#include "common.h"

namespace moe {
namespace gg {

// The six grouped GEMMs of the layer and the two MX-FP8 forward GEMMs; the values equal their
// moe_kernel_id.
enum Kind {
  GATEUP = MOE_K_GATEUP, DOWN = MOE_K_DOWN, DH = MOE_K_DH, DX = MOE_K_DX, DWD = MOE_K_DWD, DW1 = MOE_K_DW1,
  GATEUP8 = MOE_K_GATEUP_FP8, DOWN8 = MOE_K_DOWN_FP8,
  DX8 = MOE_K_DX_FP8  // the dX product on MX-FP8 operands: DOWN8's GEMM with K = 2I
};

struct Args {
  const void* x;      // [N,H] activations (gathered)
  const void* wg;     // [E,I,H]
  const void* wu;     // [E,I,H]
  const void* wd;     // [E,H,I]
  const void* dout;   // [N,H]
  const void* hcache; // [M_cap, 2I]
  const void* act;    // [M_cap, I]   (DOWN: A;  DWD: A')
  const void* dh;     // [M_cap, 2I]  (DX, DW1)
  void* out0;         // GATEUP: hcache; DOWN: y; DH: dH; DX: dXe; DWD: dW_down; DW1: dW_gate
  void* out1;         // GATEUP: act;  DH: A';  DW1: dW_up
  float* dspart;      // DH: [M_cap, nTN] partial row-dots
  // MX-FP8 kinds: x, wg, wu, wd, act hold e4m3 codes and these their scale codes
  // ([rows, 4 ceil(K/128)] bytes, K the row length); GATEUP8 writes A's codes to out1 and its
  // scale codes to out2
  const void* xs;
  const void* wgs;
  const void* wus;
  const void* wds;
  const void* acts;
  void* out2;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* row_token;
  const float* row_w;
  int E, H, I;
  int N, M_cap;
};

// Raw buffer loads: an offset at or beyond the descriptor's byte range returns zeros and
// touches no memory, so masked rows, K tails and steps past the last tile cost nothing and
// need no branch.  Every pipeline step therefore issues the same instructions, which keeps
// the compiler's memory-counter waits static.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB = 0x80000000u;  // larger than every descriptor range (< 2^31 bytes)

__device__ __forceinline__ rsrc_t mkr(const void* p, long long bytes) {
  const int n = bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ int bld4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ int ufl(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ rsrc_t mkr_off(const void* p, long long byte_off, long long bytes) {
  return mkr(static_cast<const char*>(p) + byte_off, bytes);
}

}  // namespace gg

// bf16 grouped GEMM of kind KIND (gemm_bf16.hip); max_tiles bounds the tile count of the launch.
template <int KIND>
hipError_t run_gemm_bf16(const gg::Args& a, long long max_tiles, hipStream_t s);

}  // namespace moe
