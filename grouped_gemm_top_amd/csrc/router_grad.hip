// router_grad.hip -- the router's logits product and its backward for gfx950.
//
//   logits[t,e] = sum_h x[t,h] W_r[h,e] (+ bias[e])                       (k_dense<LOGITS>)
//   dz[t,m]     = sum over final pairs f of t of dS_f w_f ([m == e_f] - q_m [m in K])
//                 with q_m = exp(z_m) / sum_{j in K} exp(z_j), K the token's top-k set  (k_router_dz)
//   dx_out[t,h] = dx_in[t,h] + sum_m dz[t,m] W_r[h,m]                        (k_dense<DXR>)
//   dW_r[h,m]   = sum_t x[t,h] dz[t,m],  dbias[m] = sum_t dz[t,m]            (k_dense<DWR> + k_dwr_reduce)
//
// The pages stop at dS, the gradient of the combine weights ("SonicMoE: IO·타일 인식 최적화로
// MoE 학습 가속하기", "3 기여 ①"); the rest follows from the weights' definition (the
// renormalised top-k softmax of "Deep EP", "1) Router", and, for token-rounding plans,
// P_e / S_t of "5 기여 ③ Token Rounding 라우팅", which is the same expression in z).
//
// These products are small next to the expert GEMMs (at E = 128 the three of them together
// are about 2 % of the layer's flops) and fp32 throughout, so they run on the vector ALUs:
// a 64 x 64 output tile per 256-thread workgroup, k in slices of 16 staged through LDS,
// 4 x 4 outputs per thread.  The weight gradient splits its long reduction (over tokens)
// into S slices written to the workspace and summed in a fixed order by a second kernel,
// so every result is bitwise reproducible.
#include <type_traits>

#include "common.h"

namespace moe {
namespace rg {

constexpr int TM = 64, TN = 64, TK = 16, NT = 256;

enum Mode { LOGITS = 0, DXR = 1, DWR = 2 };

// C[m,n] = sum_{k in [k0,k1)} A(m,k) B(k,n):
//  LOGITS: A(m,k) = x[m*lda + k] (TA), B(k,n) = wr[k*ldb + n];   out = logits (+ bias[n]), or with
//          several k-slices the partial slice blockIdx.z of [M, Nn]
//  DXR:    A(m,k) = dz[m*lda + k],     B(k,n) = wr[n*ldb + k];   out = dx_in + C (TA)
//  DWR:    A(m,k) = x[k*lda + m] (TA) for m < M - 1, 1 for m = M - 1 (the bias row);
//          B(k,n) = dz[k*ldb + n];     out = partial slice blockIdx.z of [M, Nn]
template <int MODE, typename TA>
__global__ __launch_bounds__(NT) void k_dense(const void* __restrict__ Ap, const float* __restrict__ Bp,
                                              int M, int Nn, int K, int lda, int ldb, int kslice,
                                              const float* __restrict__ bias, const void* __restrict__ cin,
                                              void* __restrict__ cout) {
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[TK][TN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.x * TM, n0 = blockIdx.y * TN;
  const int k0 = blockIdx.z * kslice;
  const int k1 = min(K, k0 + kslice);
  // the A operand is x (dtype TA) except for DXR, where it is dz (fp32); TA is then the
  // dtype of dx_in / dx_out
  using TOP = typename std::conditional<MODE == DXR, float, TA>::type;
  const TOP* A = static_cast<const TOP*>(Ap);
  float acc[4][4] = {};
  // the next k-slice is loaded into registers while the current one is multiplied
  float ra[4], rb[4];
  auto load_slice = [&](int kb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + NT * q;  // 1024 elements of each operand slice
      if constexpr (MODE == DWR) {
        const int kk = i >> 6, mm = i & 63, m = m0 + mm, k = kb + kk;  // x rows: m contiguous
        float v = 0.f;
        if (k < k1 && m < M) v = (m == M - 1) ? 1.f : to_f32<TOP>(A[(size_t)k * lda + m]);
        ra[q] = v;
      } else {
        const int mm = i >> 4, kk = i & 15, m = m0 + mm, k = kb + kk;  // rows: k contiguous
        ra[q] = (k < k1 && m < M) ? to_f32<TOP>(A[(size_t)m * lda + k]) : 0.f;
      }
      if constexpr (MODE == DXR) {
        const int nn = i >> 4, kk = i & 15, n = n0 + nn, k = kb + kk;  // W_r rows: k contiguous
        rb[q] = (k < k1 && n < Nn) ? Bp[(size_t)n * ldb + k] : 0.f;
      } else {
        const int kk = i >> 6, nn = i & 63, n = n0 + nn, k = kb + kk;  // n contiguous
        rb[q] = (k < k1 && n < Nn) ? Bp[(size_t)k * ldb + n] : 0.f;
      }
    }
  };
  auto store_slice = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + NT * q;
      if constexpr (MODE == DWR) As[i >> 6][i & 63] = ra[q];
      else As[i & 15][i >> 4] = ra[q];
      if constexpr (MODE == DXR) Bs[i & 15][i >> 4] = rb[q];
      else Bs[i >> 6][i & 63] = rb[q];
    }
  };
  if (k0 < k1) load_slice(k0);
  for (int kb = k0; kb < k1; kb += TK) {
    store_slice();
    __syncthreads();
    if (kb + TK < k1) load_slice(kb + TK);
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + ty * 4 + r;
    if (m >= M) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int n = n0 + tx * 4 + c;
      if (n >= Nn) continue;
      const size_t o = (size_t)m * Nn + n;
      if constexpr (MODE == LOGITS) {
        if (gridDim.z == 1) static_cast<float*>(cout)[o] = bias ? acc[r][c] + bias[n] : acc[r][c];
        else static_cast<float*>(cout)[(size_t)blockIdx.z * M * Nn + o] = acc[r][c];
      } else if constexpr (MODE == DXR) {
        const TA* ci = static_cast<const TA*>(cin);
        static_cast<TA*>(cout)[o] = from_f32<TA>(to_f32<TA>(ci[o]) + acc[r][c]);
      } else {
        static_cast<float*>(cout)[(size_t)blockIdx.z * M * Nn + o] = acc[r][c];
      }
    }
  }
}

// dW_r [H,E] and dbias [E] from S partial slices [S, H+1, E] (row H holds the bias sums),
// summed in slice order.
__global__ __launch_bounds__(NT) void k_dwr_reduce(const float* __restrict__ part, int S, int H, int E,
                                                   float* __restrict__ dwr, float* __restrict__ dbias) {
  const size_t n = (size_t)(H + 1) * E;
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n; i += (size_t)gridDim.x * NT) {
    float s = 0.f;
    for (int z = 0; z < S; ++z) s += part[(size_t)z * n + i];
    if (i < (size_t)H * E) {
      if (dwr) dwr[i] = s;
    } else if (dbias) {
      dbias[i - (size_t)H * E] = s;
    }
  }
}

// logits [N,E] from S partial slices [S, N, E], summed in slice order, plus the bias
__global__ __launch_bounds__(NT) void k_logits_reduce(const float* __restrict__ part, int S, int N, int E,
                                                      const float* __restrict__ bias, float* __restrict__ logits) {
  const size_t n = (size_t)N * E;
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n; i += (size_t)gridDim.x * NT) {
    float s = 0.f;
    for (int z = 0; z < S; ++z) s += part[(size_t)z * n + i];
    logits[i] = bias ? s + bias[i % E] : s;
  }
}

__global__ __launch_bounds__(NT) void k_zero(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n; i += (size_t)gridDim.x * NT) p[i] = 0.f;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wavefront per token; `row` is the wavefront's E floats of LDS.  The row is built in
// LDS (the pair terms, then the normaliser terms; an expert can be in both), then written.
__global__ __launch_bounds__(256) void k_router_dz(const float* __restrict__ logits, const float* __restrict__ bias,
                                                    const int32_t* __restrict__ idx, moe_plan p,
                                                    const float* __restrict__ ds, float* __restrict__ dz) {
  extern __shared__ float s_rows[];
  const int L = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  const int N = p.N, E = p.E, k = p.k;
  if (t >= N) return;
  float* row = s_rows + (size_t)wv * E;
  for (int m = L; m < E; m += 64) row[m] = 0.f;
  const float* lg = logits + (size_t)t * E;
  const int32_t* id = idx + (size_t)t * k;
  // q over the top-k set
  float zmax = -INFINITY;
  for (int j = L; j < k; j += 64) {
    const int e = id[j];
    zmax = fmaxf(zmax, bias ? lg[e] + bias[e] : lg[e]);
  }
  zmax = wave_max(zmax);
  float sk = 0.f;
  for (int j = L; j < k; j += 64) {
    const int e = id[j];
    sk += __expf((bias ? lg[e] + bias[e] : lg[e]) - zmax);
  }
  sk = wave_sum(sk);
  // c = sum over the final pairs of dS_f w_f, and the pair terms dS_f w_f at e_f
  const int r0 = p.tok_ptr[t], r1 = p.tok_ptr[t + 1];
  float c = 0.f;
  for (int q = r0 + L; q < r1; q += 64) {
    const int r = p.tok_rows[q];
    if (r < 0) continue;  // a slot of a pair the plan skipped
    // the expert owning row r: the last e with offsets[e] <= r
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.offsets[mid] <= r) lo = mid; else hi = mid;
    }
    const float d = p.kind == MOE_PLAN_TOPK ? ds[p.row_pair[r]] : ds[r];
    const float v = d * p.row_w[r];
    c += v;
    row[lo] = v;  // experts of one token's rows are distinct
  }
  c = wave_sum(c);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the pair terms are in LDS
  __builtin_amdgcn_wave_barrier();
  for (int j = L; j < k; j += 64) {
    const int e = id[j];
    const float qe = __expf((bias ? lg[e] + bias[e] : lg[e]) - zmax) / sk;
    row[e] = row[e] - qe * c;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  for (int m = L; m < E; m += 64) dz[(size_t)t * E + m] = row[m];
}

// k-slices of the long reductions: the weight gradient's over tokens, the logits' over H
int dw_slices(int N) {
  int S = N / 256;
  return S < 1 ? 1 : (S > 16 ? 16 : S);
}
int logit_slices(int N, int H) {
  if (N > 16384) return 1;  // enough tiles already
  int S = H / 256;
  return S < 1 ? 1 : (S > 8 ? 8 : S);
}

template <int MODE, typename TA>
hipError_t launch_dense(const void* A, const float* B, int M, int Nn, int K, int lda, int ldb, int S,
                        const float* bias, const void* cin, void* cout, hipStream_t s) {
  if (M <= 0 || Nn <= 0) return hipSuccess;
  const int kslice = ((K + S - 1) / S + TK - 1) / TK * TK;
  dim3 grid((unsigned)((M + TM - 1) / TM), (unsigned)((Nn + TN - 1) / TN), (unsigned)S);
  hipLaunchKernelGGL((k_dense<MODE, TA>), grid, dim3(NT), 0, s, A, B, M, Nn, K, lda, ldb, kslice, bias, cin, cout);
  return hipGetLastError();
}

}  // namespace rg

size_t router_bwd_ws_bytes(int N, int H, int E) {
  return (size_t)rg::dw_slices(N) * (size_t)(H + 1) * (size_t)E * 4;
}

size_t router_logits_ws_bytes(int N, int H, int E) {
  const int S = rg::logit_slices(N, H);
  return S > 1 ? (size_t)S * (size_t)N * (size_t)E * 4 : 256;
}

hipError_t launch_router_logits(moe_dtype dt, const void* x, const float* wr, const float* bias, int N, int H, int E,
                                float* logits, void* ws, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int S = rg::logit_slices(N, H);
  void* dst = S > 1 ? ws : static_cast<void*>(logits);
  kernel_event(MOE_K_ROUTER_LOGITS, 0, s);
  hipError_t e = dt == MOE_BF16
                     ? rg::launch_dense<rg::LOGITS, bf16_t>(x, wr, N, E, H, H, E, S, bias, nullptr, dst, s)
                     : rg::launch_dense<rg::LOGITS, float>(x, wr, N, E, H, H, E, S, bias, nullptr, dst, s);
  if (e == hipSuccess && S > 1) {
    const size_t n = (size_t)N * E;
    const unsigned g = (unsigned)((n + rg::NT - 1) / rg::NT < 2048 ? (n + rg::NT - 1) / rg::NT : 2048);
    hipLaunchKernelGGL(rg::k_logits_reduce, dim3(g), dim3(rg::NT), 0, s, static_cast<const float*>(ws), S, N, E,
                       bias, logits);
    e = hipGetLastError();
  }
  kernel_event(MOE_K_ROUTER_LOGITS, 1, s);
  return e;
}

hipError_t launch_router_bwd(moe_dtype dt, const float* logits, const float* bias, const int32_t* idx,
                             const moe_plan& p, const float* ds, const void* x, const float* wr, int H,
                             const void* dx_in, void* dx_out, float* dlogits, float* dwr, float* dbias, void* ws,
                             hipStream_t s) {
  const int N = p.N, E = p.E;
  if (N == 0) {
    // no tokens: the gradients of the parameters are zero (a fill kernel, so that the call
    // can be captured in a graph)
    if (dwr) hipLaunchKernelGGL(rg::k_zero, dim3(256), dim3(rg::NT), 0, s, dwr, (size_t)H * E);
    if (dbias) hipLaunchKernelGGL(rg::k_zero, dim3(1), dim3(rg::NT), 0, s, dbias, (size_t)E);
    return hipGetLastError();
  }
  kernel_event(MOE_K_ROUTER_DZ, 0, s);
  hipLaunchKernelGGL(rg::k_router_dz, dim3((unsigned)((N + 3) / 4)), dim3(256), (size_t)4 * E * 4, s, logits, bias,
                     idx, p, ds, dlogits);
  kernel_event(MOE_K_ROUTER_DZ, 1, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dx_out) {
    kernel_event(MOE_K_ROUTER_DX, 0, s);
    e = dt == MOE_BF16
            ? rg::launch_dense<rg::DXR, bf16_t>(dlogits, wr, N, H, E, E, E, 1, nullptr, dx_in, dx_out, s)
            : rg::launch_dense<rg::DXR, float>(dlogits, wr, N, H, E, E, E, 1, nullptr, dx_in, dx_out, s);
    kernel_event(MOE_K_ROUTER_DX, 1, s);
    if (e != hipSuccess) return e;
  }
  if (dwr || dbias) {
    const int S = rg::dw_slices(N);
    float* part = static_cast<float*>(ws);
    kernel_event(MOE_K_ROUTER_DW, 0, s);
    e = dt == MOE_BF16 ? rg::launch_dense<rg::DWR, bf16_t>(x, dlogits, H + 1, E, N, H, E, S, nullptr, nullptr, part, s)
                       : rg::launch_dense<rg::DWR, float>(x, dlogits, H + 1, E, N, H, E, S, nullptr, nullptr, part, s);
    if (e == hipSuccess) {
      const size_t n = (size_t)(H + 1) * E;
      const unsigned g = (unsigned)((n + rg::NT - 1) / rg::NT < 1024 ? (n + rg::NT - 1) / rg::NT : 1024);
      hipLaunchKernelGGL(rg::k_dwr_reduce, dim3(g), dim3(rg::NT), 0, s, part, S, H, E, dwr, dbias);
      e = hipGetLastError();
    }
    kernel_event(MOE_K_ROUTER_DW, 1, s);
  }
  return e;
}

}  // namespace moe
