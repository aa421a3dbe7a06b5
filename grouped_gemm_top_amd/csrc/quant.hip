// quant.hip -- MX-FP8 quantization of a row-major matrix along its rows, and of the
// transposed gate/up weights for the backward's dX product.
//
// Pages cited (by title, then section):
//   [GG] "DeepSeek 계열 MoE 학습 가속: Python expert loop → grouped GEMM", section "한계"
//        (DeepSeek-V3's fine-grained FP8 grouped GEMM: FP8 operands with scales for small
//        blocks along the contraction dimension)
//
// Format (OCP microscaling FP8, the form gfx950's scaled matrix instructions consume): e4m3
// codes, one power-of-two scale X = 2^(c - 127) per 32 consecutive values of a row, c a byte.
// X is the smallest power of two with max |v| <= 448 X over the block (no value clips); each
// value is stored as v / X rounded to nearest e4m3, ties to even (v_cvt_pk_fp8_f32).
// Layout: codes [rows, K]; scale codes [rows, KS], KS = 4 ceil(K / 128) (four blocks per 128-wide
// k-step make one 32-bit word, the unit the GEMM loads per step), entries past K / 32 are 0.
//
// One thread per (row, scale entry): it reads its block's 32 values (64 bytes of bf16), takes
// the largest magnitude, derives the scale exponent from its bits, scales exactly with
// v_ldexp_f32 and converts four values per 32-bit store word.  Pure streaming: read once,
// write once.
#include "common.h"

namespace moe {

template <typename T>
__global__ __launch_bounds__(256) void k_quant_mxfp8(const T* __restrict__ src, long long rows, int K, int KS,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long r = gid / KS;
  const int b = (int)(gid - r * KS);
  if (r >= rows) return;
  if (b >= K / 32) {
    sc[r * KS + b] = 0;
    return;
  }
  const T* p = src + r * K + 32 * b;
  float v[32];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[8 * c + 2 * h] = __uint_as_float(w[h] << 16);
        v[8 * c + 2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 u = reinterpret_cast<const float4*>(p)[c];
      v[4 * c] = u.x; v[4 * c + 1] = u.y; v[4 * c + 2] = u.z; v[4 * c + 3] = u.w;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int s = mx_scale_exp(amax);
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = mx_pack4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], s);
  uint4* qo = reinterpret_cast<uint4*>(q + r * K + 32 * b);
  qo[0] = make_uint4(w[0], w[1], w[2], w[3]);
  qo[1] = make_uint4(w[4], w[5], w[6], w[7]);
  sc[r * KS + b] = (uint8_t)(s + 127);
}

// The weight operand of the backward's dX product: for expert e, row h of [W_gate[e]^T |
// W_up[e]^T] (2I values: W_gate[e][i][h] for i < I, then W_up[e][i - I][h]; I a multiple of 32,
// so a block lies in one of the two) quantized exactly as k_quant_mxfp8 quantizes a row, into
// codes [E, H, 2I] and scale codes [E, H, KS].  One thread per (e, scale entry b, h) with h
// fastest, so each of the block's 32 source rows is read 64 consecutive h at a time (128
// bytes of bf16 per wavefront load); a thread writes its block's 32 codes as two 16-byte stores.
template <typename T>
__global__ __launch_bounds__(256) void k_quant_dxw(const T* __restrict__ wg, const T* __restrict__ wu, int E, int H,
                                                  int I, int KS, uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)E * KS * H) return;
  const int h = (int)(gid % H);
  const long long eb = gid / H;
  const int b = (int)(eb % KS), e = (int)(eb / KS);
  const int K = 2 * I;
  const long long row = (long long)e * H + h;
  if (b >= K / 32) {
    sc[row * KS + b] = 0;
    return;
  }
  const int i0 = 32 * b;
  const T* src = i0 < I ? wg + ((long long)e * I + i0) * H + h : wu + ((long long)e * I + (i0 - I)) * H + h;
  float v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = to_f32<T>(src[(long long)j * H]);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int s = mx_scale_exp(amax);
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = mx_pack4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], s);
  uint4* qo = reinterpret_cast<uint4*>(q + row * K + i0);
  qo[0] = make_uint4(w[0], w[1], w[2], w[3]);
  qo[1] = make_uint4(w[4], w[5], w[6], w[7]);
  sc[row * KS + b] = (uint8_t)(s + 127);
}

hipError_t launch_quant_dx_weights(moe_dtype dt, const void* wg, const void* wu, int E, int H, int I, uint8_t* q,
                                   uint8_t* scales, hipStream_t s) {
  const int KS = 4 * ((2 * I + 127) / 128);
  const long long n = (long long)E * KS * H;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(k_quant_dxw<bf16_t>, dim3(grid), dim3(256), 0, s, (const bf16_t*)wg, (const bf16_t*)wu, E, H,
                       I, KS, q, scales);
  else
    hipLaunchKernelGGL(k_quant_dxw<float>, dim3(grid), dim3(256), 0, s, (const float*)wg, (const float*)wu, E, H, I,
                       KS, q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp8(moe_dtype dt, const void* src, long long rows, int K, uint8_t* q, uint8_t* scales,
                              hipStream_t s) {
  const int KS = 4 * ((K + 127) / 128);
  const long long n = rows * KS;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(k_quant_mxfp8<bf16_t>, dim3(grid), dim3(256), 0, s, (const bf16_t*)src, rows, K, KS, q, scales);
  else
    hipLaunchKernelGGL(k_quant_mxfp8<float>, dim3(grid), dim3(256), 0, s, (const float*)src, rows, K, KS, q, scales);
  return hipGetLastError();
}

}  // namespace moe
