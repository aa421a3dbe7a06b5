// common.h -- internal helpers shared by the HIP sources of libmoe.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef uint16_t bf16_t;  // storage type of bf16 values (bit pattern)

// Round-to-nearest-even fp32 -> bf16 (inputs are finite; a NaN stays a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Store 4 consecutive values (the 4 accumulator lanes of one MFMA output row segment).
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  uint2 v;
  v.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  v.y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ void load4(const float* p, float& a, float& b, float& c, float& d) {
  float4 v = *reinterpret_cast<const float4*>(p);
  a = v.x; b = v.y; c = v.z; d = v.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float& a, float& b, float& c, float& d) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  a = __uint_as_float(v.x << 16); b = __uint_as_float(v.x & 0xFFFF0000u);
  c = __uint_as_float(v.y << 16); d = __uint_as_float(v.y & 0xFFFF0000u);
}

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + expf(-g)); }

// MX-FP8 block scale: the exponent s of the smallest power of two with amax <= 448 2^s (448 is
// e4m3's largest value, so no value of the block clips), limited to [-127, 127].  With amax =
// 1.m 2^(E-127), E its exponent field, and 448 = 1.75 2^8: s = E - 135, plus one when 1.m >
// 1.75 (m > 0x600000); zero and fp32 subnormals give -127.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)((b >> 23) & 0xFF);
  if (ef == 0) return -127;
  const int s = ef - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// four values scaled by 2^-s (exact) and rounded to e4m3 codes (v_cvt_pk_fp8_f32: nearest,
// ties to even), byte j = value j
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, int s) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(a, -s), __builtin_amdgcn_ldexpf(b, -s), 0,
                                                false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(c, -s), __builtin_amdgcn_ldexpf(d, -s), w,
                                                    true);
}

// Device facts the launch shapes need (cached per device by the host side).
struct DevInfo {
  int cus;   // compute units
  int xcds;  // accelerator complex dies sharing the dispatcher's round-robin
};
DevInfo dev_info();

}  // namespace moe

// Measurement hook: records the registered start/stop event around a launch (no-op when unset).
namespace moe {
void kernel_event(int kid, int which, hipStream_t s);
}

// ---- launchers implemented in the .hip files and sequenced by api.hip ----
namespace moe {
hipError_t launch_route_topk(const float* logits, const float* bias, int N, int E, int k, int32_t* idx,
                             float* w, float* probs, float* tok_norm, hipStream_t s);
size_t permute_ws_bytes(int N, int E);
size_t permute_scratch_bytes();
hipError_t permute_scratch(void** out);  // device address of the no-alloc permute's scratch
hipError_t launch_permute(const int32_t* idx, const float* w, int N, int E, int k, const moe_plan& p,
                          void* ws, hipStream_t s);
size_t tr_ws_bytes(int N, int E);
float* tr_tok_norm(void* ws, int N, int E);  // where the plan's workspace holds the token normalisers
// cap = 0: token rounding with granule param; cap = 1: capacity plan with capacity param, keys with
// (use_p = 1) or without (0) the score, row weights from topk_w
hipError_t launch_token_round(const int32_t* idx, const float* probs, const float* tok_norm, const float* topk_w,
                              int N, int E, int k, int cap, int param, int use_p, const moe_plan& p, void* ws,
                              hipStream_t s);
hipError_t launch_combine(moe_dtype dt, const void* y, int H, const moe_plan& p, const float* row_w, void* out,
                          hipStream_t s, const float* dspart = nullptr, int nP = 0, float* ds = nullptr);
size_t gemm_fwd_ws_bytes(moe_dtype dt, int M_cap, int I);
hipError_t launch_quant_mxfp8(moe_dtype dt, const void* src, long long rows, int K, uint8_t* q, uint8_t* scales,
                              hipStream_t s);
size_t gemm_fwd_mxfp8_ws_bytes(int M_cap, int I);
hipError_t launch_gemm_fwd_mxfp8(const void* xq, const void* xs, const void* wgq, const void* wgs, const void* wuq,
                                 const void* wus, const void* wdq, const void* wds, int H, int I, const moe_plan& p,
                                 void* hcache, void* y, void* ws, hipStream_t s);
hipError_t launch_gemm_fwd(moe_dtype dt, const void* x, const void* wg, const void* wu, const void* wd, int H,
                           int I, const moe_plan& p, void* hcache, void* y, void* ws, hipStream_t s);
size_t router_bwd_ws_bytes(moe_dtype dt, int N, int H, int E);
size_t router_logits_ws_bytes(moe_dtype dt, int N, int H, int E);
// the router's products on the matrix cores (router_mm.hip)
size_t router_logits_mm_ws_bytes(moe_dtype dt, int N, int H, int E);
size_t router_bwd_mm_ws_bytes(moe_dtype dt, int N, int H, int E);
hipError_t launch_router_logits_mm(moe_dtype dt, const void* x, const float* wr, const float* bias, int N, int H,
                                   int E, float* logits, void* ws, float** part, int* S, hipStream_t s);
hipError_t launch_router_dx_mm(moe_dtype dt, const float* dlogits, const float* wr, int N, int H, int E,
                               const void* dx_in, void* dx_out, void* ws, hipStream_t s);
hipError_t launch_router_dw_mm(moe_dtype dt, const void* x, const float* dlogits, int N, int H, int E, void* ws,
                               float** part, int* S, hipStream_t s);
hipError_t launch_router_logits(moe_dtype dt, const void* x, const float* wr, const float* bias, int N, int H, int E,
                                float* logits, void* ws, hipStream_t s);
hipError_t launch_router_bwd(moe_dtype dt, const float* logits, const float* bias, const int32_t* idx,
                             const moe_plan& p, const float* ds, const void* x, const float* wr, int H,
                             const void* dx_in, void* dx_out, float* dlogits, float* dwr, float* dbias, void* ws,
                             hipStream_t s);
size_t layer_bwd_ws_bytes(moe_dtype dt, int N, int M_cap, int H, int I);
hipError_t launch_layer_bwd(moe_dtype dt, const void* dout, const void* x, const void* wg, const void* wu,
                            const void* wd, int H, int I, const moe_plan& p, const void* hcache, void* dx,
                            void* dwg, void* dwu, void* dwd, float* ds, void* ws, hipStream_t s);
// the backward with its dX product on MX-FP8 operands (bf16 layers)
hipError_t launch_quant_dx_weights(moe_dtype dt, const void* wg, const void* wu, int E, int H, int I, uint8_t* q,
                                   uint8_t* scales, hipStream_t s);
size_t layer_bwd_mxfp8_ws_bytes(int N, int M_cap, int H, int I);
hipError_t launch_layer_bwd_mxfp8(const void* dout, const void* x, const void* wg, const void* wu, const void* wd,
                                  const void* wtq, const void* wts, int H, int I, const moe_plan& p,
                                  const void* hcache, void* dx, void* dwg, void* dwu, void* dwd, float* ds, void* ws,
                                  hipStream_t s);
}  // namespace moe
