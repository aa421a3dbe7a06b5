// router_grad.hip -- the router's logits product and its backward for gfx950.
//
//   logits[t,e] = sum_h x[t,h] W_r[h,e] (+ bias[e])                       (router_mm.hip)
//   dz[t,m]     = sum over final pairs f of t of dS_f w_f ([m == e_f] - q_m [m in K])
//                 with q_m = exp(z_m) / sum_{j in K} exp(z_j), K the token's top-k set  (k_router_dz)
//   dx_out[t,h] = dx_in[t,h] + sum_m dz[t,m] W_r[h,m]                        (router_mm.hip)
//   dW_r[h,m]   = sum_t x[t,h] dz[t,m],  dbias[m] = sum_t dz[t,m]            (router_mm.hip + k_dwr_reduce)
//
// The pages stop at dS, the gradient of the combine weights ("SonicMoE: IO·타일 인식 최적화로
// MoE 학습 가속하기", "3 기여 ①"); the rest follows from the weights' definition (the
// renormalised top-k softmax of "Deep EP", "1) Router", and, for token-rounding plans,
// P_e / S_t of "5 기여 ③ Token Rounding 라우팅", which is the same expression in z).
//
// The three products run on the matrix cores at fp32 accuracy (router_mm.hip); the long
// reductions (over H for the logits, over tokens for the weight gradient) are split into
// slices summed here in a fixed order, so every result is bitwise reproducible.
#include <type_traits>

#include "common.h"

namespace moe {
namespace rg {

constexpr int NT = 256;

// sum over z < S of part[z * n + i], added in slice order, eight loads in flight
__device__ __forceinline__ float slice_sum(const float* __restrict__ part, int S, size_t n, size_t i) {
  float s = 0.f;
  int z = 0;
  for (; z + 8 <= S; z += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(z + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; z < S; ++z) s += part[(size_t)z * n + i];
  return s;
}

// dW_r [H,E] and dbias [E] from S partial slices [S, H+1, E] (row H holds the bias sums),
// summed in slice order.
__global__ __launch_bounds__(NT) void k_dwr_reduce(const float* __restrict__ part, int S, int H, int E,
                                                   float* __restrict__ dwr, float* __restrict__ dbias) {
  const size_t n = (size_t)(H + 1) * E;
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n; i += (size_t)gridDim.x * NT) {
    const float s = slice_sum(part, S, n, i);
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
    const float s = slice_sum(part, S, n, i);
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
  extern __shared__ float s_rows[];  // four rows of E, then offsets[0 .. E]
  const int L = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  const int N = p.N, E = p.E, k = p.k;
  int* s_off = reinterpret_cast<int*>(s_rows + 4 * E);
  for (int q = threadIdx.x; q <= E; q += 256) s_off[q] = p.offsets[q];
  __syncthreads();
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
      if (s_off[mid] <= r) lo = mid; else hi = mid;
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

}  // namespace rg

size_t router_bwd_ws_bytes(moe_dtype dt, int N, int H, int E) { return router_bwd_mm_ws_bytes(dt, N, H, E); }

size_t router_logits_ws_bytes(moe_dtype dt, int N, int H, int E) { return router_logits_mm_ws_bytes(dt, N, H, E); }

hipError_t launch_router_logits(moe_dtype dt, const void* x, const float* wr, const float* bias, int N, int H, int E,
                                float* logits, void* ws, hipStream_t s) {
  if (N == 0) return hipSuccess;
  kernel_event(MOE_K_ROUTER_LOGITS, 0, s);
  float* part = nullptr;
  int S = 1;
  hipError_t e = launch_router_logits_mm(dt, x, wr, bias, N, H, E, logits, ws, &part, &S, s);
  if (e == hipSuccess && S > 1) {
    const size_t n = (size_t)N * E;
    const unsigned g = (unsigned)((n + rg::NT - 1) / rg::NT < 2048 ? (n + rg::NT - 1) / rg::NT : 2048);
    hipLaunchKernelGGL(rg::k_logits_reduce, dim3(g), dim3(rg::NT), 0, s, part, S, N, E, bias, logits);
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
  hipLaunchKernelGGL(rg::k_router_dz, dim3((unsigned)((N + 3) / 4)), dim3(256), (size_t)(5 * E + 1) * 4, s, logits, bias,
                     idx, p, ds, dlogits);
  kernel_event(MOE_K_ROUTER_DZ, 1, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dx_out) {
    kernel_event(MOE_K_ROUTER_DX, 0, s);
    e = launch_router_dx_mm(dt, dlogits, wr, N, H, E, dx_in, dx_out, ws, s);
    kernel_event(MOE_K_ROUTER_DX, 1, s);
    if (e != hipSuccess) return e;
  }
  if (dwr || dbias) {
    int S = 1;
    float* part = nullptr;
    kernel_event(MOE_K_ROUTER_DW, 0, s);
    e = launch_router_dw_mm(dt, x, dlogits, N, H, E, ws, &part, &S, s);
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
