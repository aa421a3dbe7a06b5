// router_mm.hip -- the router's three dense products on the matrix cores, at fp32 accuracy.
//
//   logits = x W_r (+ bias)        [N,H] x [H,E]
//   dx    += dlogits W_r^T         [N,E] x [E,H]
//   dW_r   = x^T dlogits           [H,N] x [N,E]   (and dbias from a row of ones)
//
// The products are fp32 (W_r and dlogits are fp32; x is bf16 or fp32), so each fp32 operand
// is split exactly into three bf16 parts, v = hi + mid + lo (hi = v rounded to bf16, mid =
// the rest rounded to bf16, lo = what remains, 24 significant bits in all), and the product
// is the sum of the part products with v_mfma_f32_16x16x32_bf16, which accumulates in fp32.
// A bf16 x is its own single part.  Part products whose two indices add up to more than 2
// (at most 2^-24 of the leading term each) are left out, so an fp32 x fp32 product takes six
// MFMA terms and a bf16 x fp32 one three; the error is then that of an fp32 dot product in
// another summation order.  The dx product of a bf16 layer, whose result is rounded to bf16,
// takes two parts a side and the three products of index sum <= 1.
//
// Operands reach the GEMM as "planes": bf16 parts [S][rows][ld], K-contiguous (row r holds
// the K values of output row / column r), made by two small passes that split and, where the
// source is laid out the other way, transpose.  The GEMM: a 64 x 64 output tile per 256-thread
// workgroup (four wavefronts, 32 x 32 each as 2 x 2 MFMA blocks), k in steps of 64 staged
// through LDS (16-byte chunk c of tile row r at position c ^ (r & 7)), the next step's global
// loads in registers during the MFMAs.  Long reductions are split over gridDim.z into fp32
// partial slices that a second kernel sums in slice order, so every result is bitwise
// reproducible.
#include "common.h"
#include "gemm_common.h"

namespace moe {
namespace rm {

using gg::OOB;
using gg::rsrc_t;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256, TM = 64, TN = 64, TK = 64;

__device__ __forceinline__ void split3(float v, bf16_t& h, bf16_t& m, bf16_t& l) {
  h = f32_to_bf16(v);
  float r = v - bf16_to_f32(h);  // exact: v and h agree in their leading 8 bits
  m = f32_to_bf16(r);
  r = r - bf16_to_f32(m);
  l = f32_to_bf16(r);
}

// Planes from a K-contiguous source: src[r * ld + k] (r < R, k < K) -> dst[s][r][k], row length
// Kp (a multiple of 8, >= K; entries k >= K are zero).  S = 1 copies (bf16 source), S = 3 splits,
// S = 2 keeps the first two parts (16 significant bits).
template <typename T, int S>
__global__ __launch_bounds__(NT) void k_plane_kc(const T* __restrict__ src, int R, int K, long long ld,
                                                 bf16_t* __restrict__ dst, long long pstride, int Kp) {
  const int nc = Kp / 8;
  const long long q = (long long)blockIdx.x * NT + threadIdx.x;
  if (q >= (long long)R * nc) return;
  const int r = (int)(q / nc), c = (int)(q - (long long)r * nc);
  bf16_t o[S][8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int k = 8 * c + u;
    const float v = k < K ? to_f32<T>(src[(long long)r * ld + k]) : 0.f;
    if constexpr (S == 1) {
      o[0][u] = f32_to_bf16(v);
    } else {
      bf16_t h, m, l;
      split3(v, h, m, l);
      o[0][u] = h;
      o[1][u] = m;
      if constexpr (S == 3) o[2][u] = l;
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
    *reinterpret_cast<uint4*>(dst + s * pstride + (long long)r * Kp + 8 * c) = *reinterpret_cast<const uint4*>(o[s]);
}

// Planes from a source laid out the other way: src[k * ld + r] (k < K, r < R) -> dst[s][r][k],
// row length Kp (zero for k >= K), through an LDS tile of 64 k x RT r (RT = 64 for bf16
// sources, 32 for fp32 ones: 8 KB of source either way): 16-byte loads along r (where ld and
// src allow them) and 16-byte stores along k.  ones: one more row, r = R, of ones (part 0; the
// other parts zero) for k < K.
template <typename T> constexpr int plane_rt() { return sizeof(T) == 2 ? 64 : 32; }
template <typename T, int S>
__global__ __launch_bounds__(NT) void k_plane_t(const T* __restrict__ src, int K, int R, long long ld,
                                                bf16_t* __restrict__ dst, long long pstride, int Kp, int ones) {
  constexpr int RT = plane_rt<T>();
  __shared__ float tile[64][RT + 1];
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = RT / EPC;             // chunks per tile row (8)
  constexpr int RPP = NT / CPR;             // tile rows per pass (32)
  const int k0 = blockIdx.x * 64, r0 = blockIdx.y * RT;
  const bool vec = (ld % EPC) == 0 && ((uintptr_t)src & 15u) == 0;
  const int c = threadIdx.x % CPR, kr = threadIdx.x / CPR;
  for (int p = 0; p < 64; p += RPP) {
    const int kl = p + kr, k = k0 + kl, r = r0 + c * EPC;
    float v[EPC];
    if (k < K && vec && r + EPC <= R) {
      const uint4 u = *reinterpret_cast<const uint4*>(src + (long long)k * ld + r);
      const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int q = 0; q < EPC; ++q) v[q] = to_f32<T>(e[q]);
    } else {
#pragma unroll
      for (int q = 0; q < EPC; ++q) {
        float x = 0.f;
        if (k < K) {
          if (r + q < R) x = to_f32<T>(src[(long long)k * ld + r + q]);
          else if (ones && r + q == R) x = 1.f;
        }
        v[q] = x;
      }
    }
#pragma unroll
    for (int q = 0; q < EPC; ++q) tile[kl][c * EPC + q] = v[q];
  }
  __syncthreads();
  const int Rout = R + (ones ? 1 : 0);
  const int ck = threadIdx.x & 7, rr = threadIdx.x >> 3;
  for (int p = 0; p < RT; p += 32) {
    const int rl = p + rr, r = r0 + rl, k = k0 + 8 * ck;
    if (r >= Rout || k >= Kp) continue;
    bf16_t o[S][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float v = tile[8 * ck + u][rl];
      if constexpr (S == 1) {
        o[0][u] = f32_to_bf16(v);
      } else {
        bf16_t h, m, l;
        split3(v, h, m, l);
        o[0][u] = h;
        o[1][u] = m;
        if constexpr (S == 3) o[2][u] = l;
      }
    }
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2)
      *reinterpret_cast<uint4*>(dst + s2 * pstride + (long long)r * Kp + k) = *reinterpret_cast<const uint4*>(o[s2]);
  }
}

enum Mode { PART = 0, LOGITS = 1, DX = 2 };

// C[M,Nn] = sum over k in slice blockIdx.z of A[m][k] B[n][k], A and B given as planes
// (SA, SB parts, leading dimensions lda, ldb, part strides pa, pb; rows past M / Nn and k past
// K read as zero); the part products whose indices add up to at most DMAX.
//  PART:   out fp32 [gridDim.z][M][Nn], slice blockIdx.z
//  LOGITS: out fp32 [M][Nn] = C + bias[n] (bias may be NULL; one slice)
//  DX:     out T [M][Nn] = cin + C (one slice), T = bf16 (cdt 1) or fp32 (cdt 0)
template <int SA, int SB, int MODE, int DMAX = 2>
__global__ __launch_bounds__(NT) void k_bmm(const bf16_t* __restrict__ A, long long pa, int lda,
                                            const bf16_t* __restrict__ B, long long pb, int ldb, int M, int Nn,
                                            int K, int kslice, const float* __restrict__ bias,
                                            const void* __restrict__ cin, void* __restrict__ cout, int cdt) {
  __shared__ __attribute__((aligned(16))) char sA[SA][TM * TK * 2];
  __shared__ __attribute__((aligned(16))) char sB[SB][TN * TK * 2];
  const int tid = threadIdx.x, L = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TN;
  const int kb0 = blockIdx.z * kslice;
  const int kb1 = min(K, kb0 + kslice);
  rsrc_t ra[SA], rb[SB];
#pragma unroll
  for (int s = 0; s < SA; ++s) ra[s] = gg::mkr(A + s * pa, (long long)M * lda * 2);
#pragma unroll
  for (int s = 0; s < SB; ++s) rb[s] = gg::mkr(B + s * pb, (long long)Nn * ldb * 2);
  // this thread's two 16-byte chunks of each tile: tile row q >> 3, chunk q & 7, q = tid, tid + 256
  int crow[2], cch[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    crow[i] = (tid + NT * i) >> 3;
    cch[i] = (tid + NT * i) & 7;
  }
  uint4 va[SA][2], vb[SB][2];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = k0 + 8 * cch[i];
      const bool kv = k < kb1;
      const uint32_t oa = kv ? ((uint32_t)(m0 + crow[i]) * (uint32_t)lda + (uint32_t)k) * 2u : OOB;
      const uint32_t ob = kv ? ((uint32_t)(n0 + crow[i]) * (uint32_t)ldb + (uint32_t)k) * 2u : OOB;
#pragma unroll
      for (int s = 0; s < SA; ++s) va[s][i] = gg::bld16(ra[s], oa);
#pragma unroll
      for (int s = 0; s < SB; ++s) vb[s][i] = gg::bld16(rb[s], ob);
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pos = crow[i] * 128 + ((cch[i] ^ (crow[i] & 7)) << 4);
#pragma unroll
      for (int s = 0; s < SA; ++s) *reinterpret_cast<uint4*>(sA[s] + pos) = va[s][i];
#pragma unroll
      for (int s = 0; s < SB; ++s) *reinterpret_cast<uint4*>(sB[s] + pos) = vb[s][i];
    }
  };
  // fragment of tile rows r0 .. r0 + 15, k-chunk 4 sub + (L >> 4)
  auto frag = [&](const char* t, int r0, int sub) __attribute__((always_inline)) {
    const int r = r0 + (L & 15), c = 4 * sub + (L >> 4);
    return *reinterpret_cast<const bf16x8*>(t + r * 128 + ((c ^ (r & 7)) << 4));
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kb0 < kb1) load(kb0);
  for (int k0 = kb0; k0 < kb1; k0 += TK) {
    store();
    __syncthreads();
    if (k0 + TK < kb1) load(k0 + TK);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      bf16x8 fa[SA][2], fb[SB][2];
#pragma unroll
      for (int s = 0; s < SA; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[s][i] = frag(sA[s], 32 * wm + 16 * i, sub);
#pragma unroll
      for (int s = 0; s < SB; ++s)
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[s][j] = frag(sB[s], 32 * wn + 16 * j, sub);
      // smallest terms first: part index sums DMAX .. 0
#pragma unroll
      for (int d = DMAX; d >= 0; --d)
#pragma unroll
        for (int sa = 0; sa < SA; ++sa) {
          const int sb = d - sa;
          if (sb < 0 || sb >= SB) continue;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[sb][j], fa[sa][i], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();
  }
  // lane L holds C[m][n .. n + 3], m = tile row 16 i + (L & 15), n = 16 j + 4 (L >> 4); four
  // columns at once when all four are inside (Nn a multiple of 4), else one by one
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 32 * wm + 16 * i + (L & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * wn + 16 * j + 4 * (L >> 4);
      if (n >= Nn) continue;
      const long long o = (long long)m * Nn + n;
      f32x4 c = acc[i][j];
      if (n + 4 <= Nn && (Nn & 3) == 0) {
        if constexpr (MODE == PART) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(cout) + (long long)blockIdx.z * M * Nn + o) = c;
        } else if constexpr (MODE == LOGITS) {
          if (bias) c += *reinterpret_cast<const f32x4*>(bias + n);
          *reinterpret_cast<f32x4*>(static_cast<float*>(cout) + o) = c;
        } else if (cdt) {
          const uint2 in = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(cin) + o);
          const uint32_t w0 = in.x, w1 = in.y;
          uint2 outv;
          outv.x = (uint32_t)f32_to_bf16(__uint_as_float(w0 << 16) + c[0]) |
                   ((uint32_t)f32_to_bf16(__uint_as_float(w0 & 0xFFFF0000u) + c[1]) << 16);
          outv.y = (uint32_t)f32_to_bf16(__uint_as_float(w1 << 16) + c[2]) |
                   ((uint32_t)f32_to_bf16(__uint_as_float(w1 & 0xFFFF0000u) + c[3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<bf16_t*>(cout) + o) = outv;
        } else {
          const f32x4 in = *reinterpret_cast<const f32x4*>(static_cast<const float*>(cin) + o);
          *reinterpret_cast<f32x4*>(static_cast<float*>(cout) + o) = in + c;
        }
        continue;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (n + v >= Nn) continue;
        if constexpr (MODE == PART) {
          static_cast<float*>(cout)[(long long)blockIdx.z * M * Nn + o + v] = c[v];
        } else if constexpr (MODE == LOGITS) {
          static_cast<float*>(cout)[o + v] = bias ? c[v] + bias[n + v] : c[v];
        } else if (cdt) {
          const bf16_t* ci = static_cast<const bf16_t*>(cin);
          static_cast<bf16_t*>(cout)[o + v] = f32_to_bf16(bf16_to_f32(ci[o + v]) + c[v]);
        } else {
          static_cast<float*>(cout)[o + v] = static_cast<const float*>(cin)[o + v] + c[v];
        }
      }
    }
  }
}

}  // namespace rm

// ---- host side ----
namespace {

size_t a256(size_t b) { return (b + 255) & ~(size_t)255; }
int r8(int v) { return (v + 7) / 8 * 8; }

template <typename T, int S>
hipError_t plane_kc(const T* src, int R, int K, long long ld, bf16_t* dst, long long pstride, int Kp,
                    hipStream_t s) {
  const long long n = (long long)R * (Kp / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((rm::k_plane_kc<T, S>), dim3((unsigned)((n + rm::NT - 1) / rm::NT)), dim3(rm::NT), 0, s, src, R,
                     K, ld, dst, pstride, Kp);
  return hipGetLastError();
}
template <typename T, int S>
hipError_t plane_t(const T* src, int K, int R, long long ld, bf16_t* dst, long long pstride, int Kp, int ones,
                   hipStream_t s) {
  const int Rout = R + (ones ? 1 : 0);
  if (Rout == 0 || Kp == 0) return hipSuccess;
  constexpr int RT = rm::plane_rt<T>();
  hipLaunchKernelGGL((rm::k_plane_t<T, S>), dim3((unsigned)((Kp + 63) / 64), (unsigned)((Rout + RT - 1) / RT)),
                     dim3(rm::NT), 0, s, src, K, R, ld, dst, pstride, Kp, ones);
  return hipGetLastError();
}
template <int SA, int SB, int MODE, int DMAX = 2>
hipError_t bmm(const bf16_t* A, long long pa, int lda, const bf16_t* B, long long pb, int ldb, int M, int Nn, int K,
               int S, const float* bias, const void* cin, void* cout, int cdt, hipStream_t s) {
  if (M <= 0 || Nn <= 0) return hipSuccess;
  const int kslice = ((K + S - 1) / S + rm::TK - 1) / rm::TK * rm::TK;
  const dim3 g((unsigned)((M + rm::TM - 1) / rm::TM), (unsigned)((Nn + rm::TN - 1) / rm::TN), (unsigned)S);
  hipLaunchKernelGGL((rm::k_bmm<SA, SB, MODE, DMAX>), g, dim3(rm::NT), 0, s, A, pa, lda, B, pb, ldb, M, Nn, K, kslice,
                     bias, cin, cout, cdt);
  return hipGetLastError();
}

// k-slices of a reduction over K with `tiles` output tiles: about 512 workgroups (two per CU,
// so that the loads of one overlap the MFMAs of the other, with fewer partial sums to add than
// at four), at least 128 k per slice, at most 16 slices
int slices(long long tiles, int K) {
  if (tiles <= 0) return 1;  // no rows: nothing to split
  long long S = (512 + tiles - 1) / tiles;
  const long long smax = K / 128;
  if (S > smax) S = smax;
  if (S > 16) S = 16;
  return S < 1 ? 1 : (int)S;
}

}  // namespace

// Workspace layouts (each part 256-byte aligned):
//  logits: W_r^T planes [3][E][H]; x planes [3][N][H] (fp32 x only); partial slices [S][N][E] (S > 1)
//  backward: dlogits planes [3][N][E8]; W_r planes [3][H][E8]; x^T planes [Sx][H + 1][N8] (the
//            last row ones, for dbias); dlogits^T planes [3][E][N8]; partial slices [S][H + 1][E]
//            (E8, N8: E, N rounded up to multiples of 8)
size_t router_logits_mm_ws_bytes(moe_dtype dt, int N, int H, int E) {
  const int S = slices((long long)((N + 63) / 64) * ((E + 63) / 64), H);
  size_t b = a256((size_t)3 * E * H * 2);
  if (dt != MOE_BF16) b += a256((size_t)3 * N * H * 2);
  if (S > 1) b += a256((size_t)S * N * E * 4);
  return b + 256;
}

size_t router_bwd_mm_ws_bytes(moe_dtype dt, int N, int H, int E) {
  const int E8 = r8(E), N8 = r8(N), Sx = dt == MOE_BF16 ? 1 : 3;
  const int S = slices((long long)((H + 1 + 63) / 64) * ((E + 63) / 64), N);
  return a256((size_t)3 * N * E8 * 2) + a256((size_t)3 * H * E8 * 2) + a256((size_t)Sx * (H + 1) * N8 * 2) +
         a256((size_t)3 * E * N8 * 2) + a256((size_t)S * (H + 1) * E * 4) + 256;
}

hipError_t launch_router_logits_mm(moe_dtype dt, const void* x, const float* wr, const float* bias, int N, int H,
                                   int E, float* logits, void* ws, float** part_out, int* S_out, hipStream_t s) {
  const int S = slices((long long)((N + 63) / 64) * ((E + 63) / 64), H);
  char* p = static_cast<char*>(ws);
  bf16_t* wt = reinterpret_cast<bf16_t*>(p);  // [3][E][H]
  p += a256((size_t)3 * E * H * 2);
  const long long pw = (long long)E * H;
  hipError_t e = plane_t<float, 3>(wr, H, E, E, wt, pw, H, 0, s);
  if (e != hipSuccess) return e;
  float* part = nullptr;
  const bf16_t* xa = static_cast<const bf16_t*>(x);
  long long px = 0;
  if (dt != MOE_BF16) {
    bf16_t* xp = reinterpret_cast<bf16_t*>(p);
    p += a256((size_t)3 * N * H * 2);
    px = (long long)N * H;
    if ((e = plane_kc<float, 3>(static_cast<const float*>(x), N, H, H, xp, px, H, s)) != hipSuccess) return e;
    xa = xp;
  }
  if (S > 1) part = reinterpret_cast<float*>(p);
  *S_out = S;
  *part_out = part;
  if (dt == MOE_BF16) {
    e = S > 1 ? bmm<1, 3, rm::PART>(xa, 0, H, wt, pw, H, N, E, H, S, nullptr, nullptr, part, 0, s)
              : bmm<1, 3, rm::LOGITS>(xa, 0, H, wt, pw, H, N, E, H, 1, bias, nullptr, logits, 0, s);
  } else {
    e = S > 1 ? bmm<3, 3, rm::PART>(xa, px, H, wt, pw, H, N, E, H, S, nullptr, nullptr, part, 0, s)
              : bmm<3, 3, rm::LOGITS>(xa, px, H, wt, pw, H, N, E, H, 1, bias, nullptr, logits, 0, s);
  }
  return e;
}

hipError_t launch_router_dx_mm(moe_dtype dt, const float* dlogits, const float* wr, int N, int H, int E,
                               const void* dx_in, void* dx_out, void* ws, hipStream_t s) {
  const int E8 = r8(E);
  char* p = static_cast<char*>(ws);
  bf16_t* dzp = reinterpret_cast<bf16_t*>(p);  // [3][N][E8]
  p += a256((size_t)3 * N * E8 * 2);
  bf16_t* wp = reinterpret_cast<bf16_t*>(p);  // [3][H][E8]
  const long long pz = (long long)N * E8, pw = (long long)H * E8;
  hipError_t e;
  if (dt == MOE_BF16) {
    // the result is rounded to bf16: two parts a side and the products of index sum <= 1
    // (16 significant bits each, about 2^-16 of each term) are far inside its precision
    e = plane_kc<float, 2>(dlogits, N, E, E, dzp, pz, E8, s);
    if (e == hipSuccess) e = plane_kc<float, 2>(wr, H, E, E, wp, pw, E8, s);
    if (e == hipSuccess) e = bmm<2, 2, rm::DX, 1>(dzp, pz, E8, wp, pw, E8, N, H, E8, 1, nullptr, dx_in, dx_out, 1, s);
    return e;
  }
  e = plane_kc<float, 3>(dlogits, N, E, E, dzp, pz, E8, s);
  if (e == hipSuccess) e = plane_kc<float, 3>(wr, H, E, E, wp, pw, E8, s);
  if (e == hipSuccess) e = bmm<3, 3, rm::DX>(dzp, pz, E8, wp, pw, E8, N, H, E8, 1, nullptr, dx_in, dx_out, 0, s);
  return e;
}

hipError_t launch_router_dw_mm(moe_dtype dt, const void* x, const float* dlogits, int N, int H, int E, void* ws,
                               float** part_out, int* S_out, hipStream_t s) {
  const int E8 = r8(E), N8 = r8(N), Sx = dt == MOE_BF16 ? 1 : 3;
  const int S = slices((long long)((H + 1 + 63) / 64) * ((E + 63) / 64), N);
  char* p = static_cast<char*>(ws);
  p += a256((size_t)3 * N * E8 * 2) + a256((size_t)3 * H * E8 * 2);  // the dX product's planes
  bf16_t* xt = reinterpret_cast<bf16_t*>(p);  // [Sx][H + 1][N8]
  p += a256((size_t)Sx * (H + 1) * N8 * 2);
  bf16_t* zt = reinterpret_cast<bf16_t*>(p);  // [3][E][N8]
  p += a256((size_t)3 * E * N8 * 2);
  float* part = reinterpret_cast<float*>(p);  // [S][H + 1][E]
  const long long pxt = (long long)(H + 1) * N8, pzt = (long long)E * N8;
  hipError_t e = dt == MOE_BF16 ? plane_t<bf16_t, 1>(static_cast<const bf16_t*>(x), N, H, H, xt, pxt, N8, 1, s)
                                : plane_t<float, 3>(static_cast<const float*>(x), N, H, H, xt, pxt, N8, 1, s);
  if (e == hipSuccess) e = plane_t<float, 3>(dlogits, N, E, E, zt, pzt, N8, 0, s);
  if (e == hipSuccess) {
    e = dt == MOE_BF16 ? bmm<1, 3, rm::PART>(xt, pxt, N8, zt, pzt, N8, H + 1, E, N8, S, nullptr, nullptr, part, 0, s)
                       : bmm<3, 3, rm::PART>(xt, pxt, N8, zt, pzt, N8, H + 1, E, N8, S, nullptr, nullptr, part, 0, s);
  }
  *part_out = part;
  *S_out = S;
  return e;
}

}  // namespace moe
