// permute.hip -- routing plan: per-expert counts, offsets and the stable expert-sorted row order.
//
// Pages cited (by title, then section):
//   [GG]  "DeepSeek 계열 MoE 학습 가속: Python expert loop → grouped GEMM",
//         section "적용 — fused MoE training forward", steps (1)-(3): flatten the top-k ids,
//         sort by expert id so each expert's rows are one contiguous slice, bincount
//   [DEP] "Deep EP", section "2) Dispatch" (ragged layout needs offset/index metadata)
//
// A stable counting sort over the N*k (token, slot) pairs, never a comparison sort:
//   k_perm_hist     per block of 256 tokens: expert histogram in LDS -> bcnt[b][e]
//   k_perm_scan     counts[e] = sum_b bcnt[b][e]; offsets = exclusive scan over e;
//                   bbase[b][e] = offsets[e] + sum_{b'<b} bcnt[b'][e]
//   k_perm_scatter  rank of a pair inside (block, expert) = number of earlier tokens of the
//                   block routed to the same expert (LDS bitmask + popcount), so rows of an
//                   expert ascend by token; also writes the token-major row lists
// Integer counting only: the plan is bit-exact and independent of scheduling.
#include "common.h"

namespace moe {

constexpr int kPT = 256;  // tokens per block

__global__ __launch_bounds__(kPT) void k_perm_hist(const int32_t* __restrict__ idx, int N, int E, int k,
                                                   int32_t* __restrict__ bcnt) {
  __shared__ int s_cnt[1024];
  for (int e = threadIdx.x; e < E; e += kPT) s_cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kPT + threadIdx.x;
  if (t < N)
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPT) bcnt[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ bcnt, int nb, int N, int E, int k,
                                                    int32_t* __restrict__ bbase, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ tok_ptr) {
  __shared__ int s_wave[17];
  const int e = threadIdx.x, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int c = 0;
  if (e < E)
    for (int b = 0; b < nb; ++b) c += bcnt[(size_t)b * E + e];
  // block exclusive scan of c over the 1024 threads
  int x = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int q = 0; q < 16; ++q) {
      const int v = s_wave[q];
      s_wave[q] = run;
      run += v;
    }
    s_wave[16] = run;
  }
  __syncthreads();
  const int ex = s_wave[wv] + x - c;
  if (e < E) {
    counts[e] = c;
    offsets[e] = ex;
    int run = ex;
    for (int b = 0; b < nb; ++b) {
      const int v = bcnt[(size_t)b * E + e];
      bbase[(size_t)b * E + e] = run;
      run += v;
    }
  }
  if (threadIdx.x == 0) {
    offsets[E] = s_wave[16];
    tok_ptr[N] = N * k;
  }
}

__global__ __launch_bounds__(kPT) void k_perm_scatter(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      int N, int E, int k, const int32_t* __restrict__ bbase,
                                                      int32_t* __restrict__ row_token, float* __restrict__ row_w,
                                                      int32_t* __restrict__ row_pair, int32_t* __restrict__ tok_ptr,
                                                      int32_t* __restrict__ tok_rows) {
  constexpr int W = kPT / 32;  // bitmask words per expert
  __shared__ uint32_t s_bits[1024 * W];
  for (int q = threadIdx.x; q < E * W; q += kPT) s_bits[q] = 0u;
  __syncthreads();
  const int tl = threadIdx.x;
  const int t = blockIdx.x * kPT + tl;
  const int32_t* it = idx + (size_t)t * k;
  if (t < N)
    for (int j = 0; j < k; ++j) {
      const int e = it[j];
      if (e >= 0 && e < E) atomicOr(&s_bits[e * W + (tl >> 5)], 1u << (tl & 31));
    }
  __syncthreads();
  if (t >= N) return;
  tok_ptr[t] = t * k;
  const int32_t* bb = bbase + (size_t)blockIdx.x * E;
  for (int j = 0; j < k; ++j) {
    const int e = it[j];
    if (e < 0 || e >= E) continue;
    int rank = 0;
    const uint32_t* bits = s_bits + e * W;
    for (int q = 0; q < (tl >> 5); ++q) rank += __popc(bits[q]);
    rank += __popc(bits[tl >> 5] & ((1u << (tl & 31)) - 1u));
    const int row = bb[e] + rank;
    row_token[row] = t;
    row_w[row] = w[(size_t)t * k + j];
    row_pair[row] = t * k + j;
    // rows ascend with the expert id, so the token-major position is the number of this
    // token's experts with a smaller id
    int pos = 0;
    for (int q = 0; q < k; ++q) pos += (it[q] < e);
    tok_rows[(size_t)t * k + pos] = row;
  }
}

size_t permute_ws_bytes(int N, int E) {
  const size_t nb = ((size_t)N + kPT - 1) / kPT;
  return 2 * (((nb * E * 4) + 255) & ~(size_t)255) + 256;
}

hipError_t launch_perm_hist(const int32_t* idx, int N, int E, int k, int32_t* bcnt, hipStream_t s) {
  const int nb = (N + kPT - 1) / kPT;
  hipLaunchKernelGGL(k_perm_hist, dim3(nb), dim3(kPT), 0, s, idx, N, E, k, bcnt);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, const float* w, int N, int E, int k, const moe_plan& p, void* ws,
                          hipStream_t s) {
  const int nb = (N + kPT - 1) / kPT;
  int32_t* bcnt = (int32_t*)ws;
  int32_t* bbase = (int32_t*)((char*)ws + ((((size_t)nb * E * 4) + 255) & ~(size_t)255));
  hipError_t err;
  if (nb > 0) {
    if ((err = launch_perm_hist(idx, N, E, k, bcnt, s)) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, bcnt, nb, N, E, k, bbase, p.counts, p.offsets,
                     p.tok_ptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (nb > 0) {
    hipLaunchKernelGGL(k_perm_scatter, dim3(nb), dim3(kPT), 0, s, idx, w, N, E, k, bbase, p.row_token, p.row_w,
                       p.row_pair, p.tok_ptr, p.tok_rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
