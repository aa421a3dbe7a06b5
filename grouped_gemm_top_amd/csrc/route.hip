// route.hip -- router top-k and token-rounding plan kernels.
//
// Pages cited (by title, then section):
//   [DEP] "Deep EP", section "1) Router"
//   [SM]  "SonicMoE: IO·타일 인식 최적화로 MoE 학습 가속하기", section "5 기여 ③ Token Rounding 라우팅"
#include <limits.h>

#include "common.h"

namespace moe {

constexpr int kMaxE = 1024;
constexpr int kPerLane = kMaxE / 64;

// ---------------------------------------------------------------------------------------
// Top-k router ([DEP] "1) Router").  One 64-lane wavefront per token; lane l holds experts
// l, l+64, ...  Selection takes k rounds of a wave-wide arg-max under the total order
// (z descending, expert id ascending); IEEE compares only, so -0 and +0 tie.  Weights are
// the softmax over the chosen k (the full-E denominator cancels); probs is the full softmax.
// tok_norm (optional) is the sum of the chosen probs, the normaliser token rounding uses.
// ---------------------------------------------------------------------------------------
// Maximum over the wavefront, returned to every lane: xor-1 and xor-2 quad permutations, the
// half-row and row mirrors (each lane then holds its 16-lane row's maximum), then the four row
// maxima read out through SGPRs.  Exact: a maximum involves no rounding.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad permutation [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad permutation [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row half mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The routing of token t by one wavefront.  sz: the wavefront's LDS scratch (k floats, the
// chosen logits).
template <int PL>  // experts per lane: E <= 64 * PL
__device__ __forceinline__ void route_token(const float* __restrict__ logits, const float* __restrict__ bias, int t,
                                            int E, int k, int32_t* __restrict__ idx, float* __restrict__ w,
                                            float* __restrict__ probs, float* __restrict__ tok_norm, float* sz) {
  const int lane = threadIdx.x & 63;
  const float* lt = logits + (size_t)t * E;
  // all loads first (clamped index, masked afterwards), so they are in flight together
  float z[PL];
  uint32_t avail = 0;
#pragma unroll
  for (int q = 0; q < PL; ++q) {
    const int e = lane + 64 * q;
    const int ec = e < E ? e : 0;
    z[q] = lt[ec];
    if (bias) z[q] += bias[ec];
    if (e < E) avail |= 1u << q;
  }
  float zmax = 0.f;
  for (int j = 0; j < k; ++j) {
    // the largest available z: the lane's own maximum, then the wavefront's (row maxima with
    // DPP moves, then the four rows through SGPRs); a lane with nothing left offers -inf
    float lm = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < PL; ++q)
      if ((avail >> q) & 1u) lm = fmaxf(lm, z[q]);
    const float bz = wave_max(lm);
    // the lowest expert id holding it: the lowest q with a match, then the lowest lane (-0
    // and +0 compare equal)
    int be = INT_MAX;
#pragma unroll
    for (int q = PL - 1; q >= 0; --q) {
      const uint64_t m = __ballot(((avail >> q) & 1u) && z[q] == bz);
      if (m) be = 64 * q + __builtin_ctzll(m);
    }
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (lane == 0) {
      idx[(size_t)t * k + j] = be;
      sz[j] = bz;
    }
    if (j == 0) zmax = bz;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  // renormalised weights: softmax over the chosen k
  float sk = 0.f;
  for (int j = lane; j < k; j += 64) sk += expf(sz[j] - zmax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sk += __shfl_xor(sk, off);
  for (int j = lane; j < k; j += 64) w[(size_t)t * k + j] = expf(sz[j] - zmax) / sk;
  if (probs || tok_norm) {
    float ez[PL];
    float sa = 0.f;
#pragma unroll
    for (int q = 0; q < PL; ++q) {
      ez[q] = lane + 64 * q < E ? expf(z[q] - zmax) : 0.f;
      sa += ez[q];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sa += __shfl_xor(sa, off);
    if (probs) {
#pragma unroll
      for (int q = 0; q < PL; ++q)
        if (lane + 64 * q < E) probs[(size_t)t * E + lane + 64 * q] = ez[q] / sa;
    }
    if (tok_norm) {
      // sum of the chosen probabilities, in slot order, from the same fp32 values as probs
      if (lane == 0) {
        float s = 0.f;
        for (int j = 0; j < k; ++j) s += expf(sz[j] - zmax) / sa;
        tok_norm[t] = s;
      }
    }
  }
}

template <int PL>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int N, int E, int k,
                                                    int32_t* __restrict__ idx, float* __restrict__ w,
                                                    float* __restrict__ probs, float* __restrict__ tok_norm) {
  __shared__ float s_z[4][kMaxE];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N) return;  // whole wavefronts exit together; no block barrier below
  route_token<PL>(logits, bias, t, E, k, idx, w, probs, tok_norm, s_z[wave]);
}

hipError_t launch_route_topk(const float* logits, const float* bias, int N, int E, int k, int32_t* idx,
                             float* w, float* probs, float* tok_norm, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const dim3 g((N + 3) / 4), b(256);
  if (E <= 64) hipLaunchKernelGGL(k_route_topk<1>, g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else if (E <= 128) hipLaunchKernelGGL(k_route_topk<2>, g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else if (E <= 256) hipLaunchKernelGGL(k_route_topk<4>, g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else if (E <= 512) hipLaunchKernelGGL(k_route_topk<8>, g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else hipLaunchKernelGGL(k_route_topk<16>, g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Token rounding ([SM] "5 기여 ③ Token Rounding 라우팅").  After the top-k route and the
// per-block histogram of the permute step:
//   k_tr_sizes   c_e -> r_e = mtile*floor((c_e + mtile/2)/mtile) (<= largest multiple of
//                mtile <= N); plan counts = r_e, offsets = exclusive scan
//   k_tr_keys    key[e][t] = routed(t,e) << 63 | bits(P[t,e]) << 32 | ~t, so that the key
//                order is (routed first, score descending, token ascending)
//   k_tr_select  one block per expert: radix-select the r_e-th largest key, keep every key
//                >= it, compact in token order -> rows of expert e
//   k_tr_tokcount / scan / k_tr_tokfill   token-major row lists
// The capacity plan ([DEP] "Drop/Padding 방식": each expert's tokens lined up and cut at the
// capacity C, the rest dropped) runs the same kernels with r_e = min(c_e, C), the key's score
// left out for the position order, and each kept row taking its pair's top-k weight.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int block_excl_scan_1024(int v, int* s_wave, int* total) {
  // 1024 threads = 16 wavefronts; returns the exclusive prefix of v in thread order
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
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
      const int c = s_wave[q];
      s_wave[q] = run;
      run += c;
    }
    s_wave[16] = run;
  }
  __syncthreads();
  const int res = s_wave[wv] + x - v;
  *total = s_wave[16];
  __syncthreads();
  return res;
}

// cap = 0: token rounding, r_e = mtile-rounded c_e; cap = 1: capacity, r_e = min(c_e, param)
__global__ __launch_bounds__(1024) void k_tr_sizes(const int32_t* __restrict__ bcnt, int nb, int N, int E,
                                                   int param, int cap, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int s_wave[17];
  const int e = threadIdx.x;
  int r = 0;
  if (e < E) {
    // eight independent loads in flight (integer sums: the order is free)
    int cc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int b = 0;
    for (; b + 8 <= nb; b += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) cc[u] += bcnt[(size_t)(b + u) * E + e];
    }
    for (; b < nb; ++b) cc[0] += bcnt[(size_t)b * E + e];
    const int c = ((cc[0] + cc[1]) + (cc[2] + cc[3])) + ((cc[4] + cc[5]) + (cc[6] + cc[7]));
    if (cap) {
      r = c < param ? c : param;
    } else {
      const int mtile = param;
      const int rmax = mtile * (N / mtile);
      r = mtile * ((c + mtile / 2) / mtile);
      if (r > rmax) r = rmax;
    }
    counts[e] = r;
  }
  int total;
  const int ex = block_excl_scan_1024(r, s_wave, &total);
  if (e < E) offsets[e] = ex;
  if (e == 0) offsets[E] = total;
}

// use_p = 0 leaves the score out of the key (the capacity plan's position order)
__global__ __launch_bounds__(256) void k_tr_keys(const float* __restrict__ probs, const int32_t* __restrict__ idx,
                                                 int N, int E, int k, int use_p, uint64_t* __restrict__ keys) {
  __shared__ uint32_t s_p[64][65];
  __shared__ uint8_t s_r[64][64];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  for (int q = threadIdx.x; q < 64 * 64; q += 256) {
    const int tl = q >> 6, el = q & 63;
    const int t = t0 + tl, e = e0 + el;
    s_p[tl][el] = (use_p && t < N && e < E) ? (__float_as_uint(probs[(size_t)t * E + e]) & 0x7FFFFFFFu) : 0u;
    s_r[tl][el] = 0;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int t = t0 + threadIdx.x;
    if (t < N)
      for (int j = 0; j < k; ++j) {
        const int e = idx[(size_t)t * k + j];
        if (e >= e0 && e < e0 + 64) s_r[threadIdx.x][e - e0] = 1;
      }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * 64; q += 256) {
    const int el = q >> 6, tl = q & 63;
    const int t = t0 + tl, e = e0 + el;
    if (t < N && e < E)
      keys[(size_t)e * N + t] = ((uint64_t)s_r[tl][el] << 63) | ((uint64_t)s_p[tl][el] << 32) |
                                (uint64_t)(0xFFFFFFFFu - (uint32_t)t);
  }
}

// topk_w != NULL (capacity plans): a kept row takes its pair's top-k weight as it is
__global__ __launch_bounds__(1024) void k_tr_select(const uint64_t* __restrict__ keys, const float* __restrict__ probs,
                                                    const float* __restrict__ tok_norm, const float* __restrict__ topk_w,
                                                    const int32_t* __restrict__ idx, int N, int E, int k,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ row_of, int32_t* __restrict__ row_token,
                                                    float* __restrict__ row_w, int32_t* __restrict__ row_pair) {
  __shared__ int s_hist[256];
  __shared__ int s_whist[16][256];  // per-wavefront histograms: keys crowd into a few bins
  __shared__ int s_wave[17];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_remaining;
  __shared__ int s_done;
  const int e = blockIdx.x;
  const int r = counts[e];
  const int off = offsets[e];
  const uint64_t* ke = keys + (size_t)e * N;
  uint64_t thr = ~0ull;  // select nothing unless r > 0
  if (r > 0) {
    if (threadIdx.x == 0) { s_prefix = 0ull; s_remaining = r; s_done = 0; }
    uint64_t mask = 0ull;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      {
        int* wh = &s_whist[0][0];
        for (int q = threadIdx.x; q < 16 * 256; q += 1024) wh[q] = 0;
      }
      __syncthreads();
      const uint64_t prefix = s_prefix;
      int* myh = s_whist[threadIdx.x >> 6];
      for (int t = threadIdx.x; t < N; t += 1024) {
        const uint64_t key = ke[t];
        if ((key & mask) == prefix) atomicAdd(&myh[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (threadIdx.x < 256) {
        int h = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) h += s_whist[q][threadIdx.x];
        s_hist[threadIdx.x] = h;
      }
      __syncthreads();
      // the bin holding the rem-th largest key: thread q takes bin 255 - q, so its exclusive
      // prefix is the count of keys in the bins above; exactly one bin crosses rem
      const int rem = s_remaining;
      const int bq = 255 - (int)threadIdx.x;
      const int hq = threadIdx.x < 256 ? s_hist[bq] : 0;
      int tot;
      const int above = block_excl_scan_1024(hq, s_wave, &tot);
      if (threadIdx.x < 256 && above < rem && above + hq >= rem) {
        s_prefix = prefix | ((uint64_t)bq << shift);
        s_remaining = rem - above;
        // every key of the bin is needed: the threshold with zero low bits is already exact
        if (above + hq == rem) s_done = 1;
      }
      mask |= 0xFFull << shift;
      __syncthreads();
      if (s_done) break;
    }
    thr = s_prefix;
  }
  int run = 0;
  for (int base = 0; base < N; base += 1024) {
    const int t = base + threadIdx.x;
    const bool sel = (t < N) && (r > 0) && (ke[t] >= thr);
    int total;
    const int pos = block_excl_scan_1024(sel ? 1 : 0, s_wave, &total);
    if (t < N) {
      if (sel) {
        const int row = off + run + pos;
        row_of[(size_t)e * N + t] = row;
        row_token[row] = t;
        int pair = -1;
        for (int j = 0; j < k; ++j)
          if (idx[(size_t)t * k + j] == e) { pair = t * k + j; break; }
        row_w[row] = (topk_w && pair >= 0) ? topk_w[pair] : probs[(size_t)t * E + e] / tok_norm[t];
        row_pair[row] = pair;
      } else {
        row_of[(size_t)e * N + t] = -1;
      }
    }
    run += total;
  }
}

// the kept rows of token t among experts [e0, e1), eight loads in flight
__device__ __forceinline__ int tr_count_rows(const int32_t* __restrict__ row_of, int N, int t, int e0, int e1) {
  int cc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int e = e0;
  for (; e + 8 <= e1; e += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) cc[u] += row_of[(size_t)(e + u) * N + t] >= 0;
  }
  for (; e < e1; ++e) cc[0] += row_of[(size_t)e * N + t] >= 0;
  return ((cc[0] + cc[1]) + (cc[2] + cc[3])) + ((cc[4] + cc[5]) + (cc[6] + cc[7]));
}

// Token-major row lists from row_of [E, N].  One block per 64 tokens; thread (g, tl) covers
// token t0 + tl and the experts of quarter g (e in [g E/4, (g+1) E/4)), so every load reads 64
// consecutive tokens of one expert.
__global__ __launch_bounds__(256) void k_tr_tokcount(const int32_t* __restrict__ row_of, int N, int E,
                                                     int32_t* __restrict__ tcount) {
  __shared__ int s_c[4][64];
  const int tl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + tl;
  const int e0 = g * E / 4, e1 = (g + 1) * E / 4;
  s_c[g][tl] = t < N ? tr_count_rows(row_of, N, t, e0, e1) : 0;
  __syncthreads();
  if (g == 0 && t < N) tcount[t] = s_c[0][tl] + s_c[1][tl] + s_c[2][tl] + s_c[3][tl];
}

// exclusive scan of tcount[0..N) into tok_ptr[0..N]; one block of 1024 threads over segments of
// 16384 tokens: the segment goes through LDS (coalesced loads and stores), thread x scans its 16
// consecutive tokens x 16 .. x 16 + 15 there, and one block scan joins the threads
__global__ __launch_bounds__(1024) void k_scan_tokens(const int32_t* __restrict__ tcount, int N,
                                                      int32_t* __restrict__ tok_ptr) {
  __shared__ int s_seg[16384 + 1024];
  __shared__ int s_wave[17];
  int run = 0;
  for (int base = 0; base < N; base += 16384) {
    const int n = min(16384, N - base);
    // element q at q + q / 16, so that the 16 runs of a wavefront's lanes fall in distinct banks
    for (int q = threadIdx.x; q < 16384; q += 1024) s_seg[q + (q >> 4)] = q < n ? tcount[base + q] : 0;
    __syncthreads();
    int* my = s_seg + 17 * threadIdx.x;
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) sum += my[u];
    int total;
    int ex = run + block_excl_scan_1024(sum, s_wave, &total);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int v = my[u];
      my[u] = ex;
      ex += v;
    }
    __syncthreads();
    for (int q = threadIdx.x; q < n; q += 1024) tok_ptr[base + q] = s_seg[q + (q >> 4)];
    __syncthreads();
    run += total;
  }
  if (threadIdx.x == 0) tok_ptr[N] = run;
}

// the kept rows of each token in ascending expert order: quarter g writes after the rows of
// quarters 0 .. g-1
__global__ __launch_bounds__(256) void k_tr_tokfill(const int32_t* __restrict__ row_of, int N, int E,
                                                    const int32_t* __restrict__ tok_ptr,
                                                    int32_t* __restrict__ tok_rows) {
  __shared__ int s_c[4][64];
  const int tl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + tl;
  const int e0 = g * E / 4, e1 = (g + 1) * E / 4;
  s_c[g][tl] = t < N ? tr_count_rows(row_of, N, t, e0, e1) : 0;
  __syncthreads();
  if (t >= N) return;
  int p = tok_ptr[t];
  for (int q = 0; q < g; ++q) p += s_c[q][tl];
  int e = e0;
  for (; e + 8 <= e1; e += 8) {
    int r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = row_of[(size_t)(e + u) * N + t];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r[u] >= 0) tok_rows[p++] = r[u];
  }
  for (; e < e1; ++e) {
    const int r = row_of[(size_t)e * N + t];
    if (r >= 0) tok_rows[p++] = r;
  }
}

// defined in permute.hip
hipError_t launch_perm_hist(const int32_t* idx, int N, int E, int k, int32_t* bcnt, hipStream_t s);

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t tr_ws_bytes(int N, int E) {
  const size_t nb = ((size_t)N + 255) / 256;
  return align256(nb * E * 4) + align256((size_t)N * 4) + align256((size_t)E * N * 8) +
         align256((size_t)E * N * 4) + align256((size_t)N * 4) + 256;
}

hipError_t launch_token_round(const int32_t* idx, const float* probs, const float* tok_norm, const float* topk_w,
                              int N, int E, int k, int cap, int param, int use_p, const moe_plan& p, void* ws,
                              hipStream_t s) {
  const int nb = (N + 255) / 256;
  char* w = (char*)ws;
  int32_t* bcnt = (int32_t*)w;
  w += align256((size_t)nb * E * 4);
  w += align256((size_t)N * 4);  // tok_norm lives here (written by the route kernel)
  uint64_t* keys = (uint64_t*)w;
  w += align256((size_t)E * N * 8);
  int32_t* row_of = (int32_t*)w;
  w += align256((size_t)E * N * 4);
  int32_t* tcount = (int32_t*)w;
  hipError_t err;
  if (N > 0) {
    if ((err = launch_perm_hist(idx, N, E, k, bcnt, s)) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_tr_sizes, dim3(1), dim3(1024), 0, s, bcnt, nb, N, E, param, cap, p.counts, p.offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (N > 0) {
    hipLaunchKernelGGL(k_tr_keys, dim3((N + 63) / 64, (E + 63) / 64), dim3(256), 0, s, probs, idx, N, E, k, use_p,
                       keys);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_tr_select, dim3(E), dim3(1024), 0, s, keys, probs, tok_norm, topk_w, idx, N, E, k, p.counts,
                       p.offsets, row_of, p.row_token, p.row_w, p.row_pair);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_tr_tokcount, dim3((N + 63) / 64), dim3(256), 0, s, row_of, N, E, tcount);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_scan_tokens, dim3(1), dim3(1024), 0, s, tcount, N, p.tok_ptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (N > 0) {
    hipLaunchKernelGGL(k_tr_tokfill, dim3((N + 63) / 64), dim3(256), 0, s, row_of, N, E, p.tok_ptr, p.tok_rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
