// route.hip -- router top-k and token-rounding plan kernels.
//
// Pages cited (by title, then section):
//   [DEP] "Deep EP", section "1) Router"
//   [SM]  "SonicMoE: IO·타일 인식 최적화로 MoE 학습 가속하기", section "5 기여 ③ Token Rounding 라우팅"
#include <limits.h>

#include "common.h"

namespace moe {

constexpr int kMaxE = 1024;

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

// The routing of token t by one wavefront.  SMALLK (k <= 64): lane j keeps round j's logit and
// expert in registers and the wavefront writes them at the end; otherwise lane 0 writes each
// round's expert and sz (the wavefront's LDS scratch, k floats) holds the chosen logits.
template <int PL, bool SMALLK>  // experts per lane: E <= 64 * PL
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
  float myz = 0.f;  // SMALLK: lane j's round
  int myid = 0;
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
    if constexpr (SMALLK) {
      if (lane == j) {
        myz = bz;
        myid = be;
      }
    } else if (lane == 0) {
      idx[(size_t)t * k + j] = be;
      sz[j] = bz;
    }
    if (j == 0) zmax = bz;
  }
  // renormalised weights: softmax over the chosen k
  float sk = 0.f;
  if constexpr (SMALLK) {
    if (lane < k) {
      idx[(size_t)t * k + lane] = myid;
      sk = expf(myz - zmax);
    }
  } else {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int j = lane; j < k; j += 64) sk += expf(sz[j] - zmax);
  }
  const float ek = sk;  // SMALLK: this lane's term
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sk += __shfl_xor(sk, off);
  if constexpr (SMALLK) {
    if (lane < k) w[(size_t)t * k + lane] = ek / sk;
  } else {
    for (int j = lane; j < k; j += 64) w[(size_t)t * k + j] = expf(sz[j] - zmax) / sk;
  }
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
      if constexpr (SMALLK) {
        const float pj = ek / sa;  // lane j: round j's probability (lanes >= k: unused)
        float s = 0.f;
        for (int j = 0; j < k; ++j) s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), j));
        if (lane == 0) tok_norm[t] = s;
      } else if (lane == 0) {
        float s = 0.f;
        for (int j = 0; j < k; ++j) s += expf(sz[j] - zmax) / sa;
        tok_norm[t] = s;
      }
    }
  }
}

template <int PL, bool SMALLK>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int N, int E, int k,
                                                    int32_t* __restrict__ idx, float* __restrict__ w,
                                                    float* __restrict__ probs, float* __restrict__ tok_norm) {
  __shared__ float s_z[4][SMALLK ? 1 : kMaxE];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= N) return;  // whole wavefronts exit together; no block barrier below
  route_token<PL, SMALLK>(logits, bias, t, E, k, idx, w, probs, tok_norm, s_z[wave]);
}

template <bool SMALLK>
static void launch_route_pl(const float* logits, const float* bias, int N, int E, int k, int32_t* idx, float* w,
                            float* probs, float* tok_norm, hipStream_t s) {
  const dim3 g((N + 3) / 4), b(256);
  if (E <= 64)
    hipLaunchKernelGGL((k_route_topk<1, SMALLK>), g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else if (E <= 128)
    hipLaunchKernelGGL((k_route_topk<2, SMALLK>), g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else if (E <= 256)
    hipLaunchKernelGGL((k_route_topk<4, SMALLK>), g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else if (E <= 512)
    hipLaunchKernelGGL((k_route_topk<8, SMALLK>), g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
  else
    hipLaunchKernelGGL((k_route_topk<16, SMALLK>), g, b, 0, s, logits, bias, N, E, k, idx, w, probs, tok_norm);
}

hipError_t launch_route_topk(const float* logits, const float* bias, int N, int E, int k, int32_t* idx,
                             float* w, float* probs, float* tok_norm, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (k <= 64) launch_route_pl<true>(logits, bias, N, E, k, idx, w, probs, tok_norm, s);
  else launch_route_pl<false>(logits, bias, N, E, k, idx, w, probs, tok_norm, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Token rounding ([SM] "5 기여 ③ Token Rounding 라우팅").  After the top-k route and the
// per-block histogram of the permute step:
//   k_tr_sizes   c_e -> r_e = mtile*floor((c_e + mtile/2)/mtile) (<= largest multiple of
//                mtile <= N); plan counts = r_e, offsets = exclusive scan
//   k_tr_keys    key[e][t] = routed(t,e) << 63 | bits(P[t,e]) << 32 | ~t, so that the key
//                order is (routed first, score descending, token ascending)
//   k_tr_select  one block per expert: select the r_e-th largest key (a histogram of the
//                top bits, then radix passes over the threshold bin's keys in LDS), keep
//                every key >= it, compact in token order -> rows of expert e
//   k_tr_tokcount / k_tr_tokfill   token-major row lists (the fill scans the token counts
//                itself while the token blocks are few; else k_scan_tokens runs between)
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

// cap = 0: token rounding, r_e = mtile-rounded c_e; cap = 1: capacity, r_e = min(c_e, param).
// Thread (g, e) = g E + e, g < G = 1024 / E rounded down to a power of two: group g sums the
// histogram rows b = g, g + G, ... of expert e, then the G partial sums are added (integers:
// any order is exact).
__global__ __launch_bounds__(1024) void k_tr_sizes(const int32_t* __restrict__ bcnt, int nb, int N, int E,
                                                   int param, int cap, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int s_wave[17];
  __shared__ int s_part[1024];
  int G = 1;
  while (2 * G * E <= 1024) G *= 2;
  const int g = threadIdx.x / E, e = threadIdx.x - g * E;
  if (g < G) {
    // eight independent loads in flight
    int cc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int b = g;
    for (; b + 7 * G < nb; b += 8 * G) {
#pragma unroll
      for (int u = 0; u < 8; ++u) cc[u] += bcnt[(size_t)(b + u * G) * E + e];
    }
    for (; b < nb; b += G) cc[0] += bcnt[(size_t)b * E + e];
    s_part[threadIdx.x] = ((cc[0] + cc[1]) + (cc[2] + cc[3])) + ((cc[4] + cc[5]) + (cc[6] + cc[7]));
  }
  __syncthreads();
  int r = 0;
  const int et = threadIdx.x;  // from here on: thread e of the expert scan
  if (et < E) {
    int c = 0;
    for (int q = 0; q < G; ++q) c += s_part[q * E + et];
    if (cap) {
      r = c < param ? c : param;
    } else {
      const int mtile = param;
      const int rmax = mtile * (N / mtile);
      r = mtile * ((c + mtile / 2) / mtile);
      if (r > rmax) r = rmax;
    }
    counts[et] = r;
  }
  int total;
  const int ex = block_excl_scan_1024(r, s_wave, &total);
  if (et < E) offsets[et] = ex;
  if (et == 0) offsets[E] = total;
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

// Select: the r-th largest of an expert's N keys is the threshold; every key >= it is kept.
// A first pass counts the keys by their top 11 bits (the routed bit, P's exponent and two
// mantissa bits), which locates the bin holding the threshold; the keys of that bin (few, as a
// rule: the threshold sits where routed or unrouted scores thin out) are then gathered into
// LDS and the threshold is found among them by 8-bit radix passes.  Where the bin holds more
// than TR_CAP keys (many equal scores), the radix passes read the keys from memory instead.
constexpr int TR_HB = 11;            // first-pass digit: key bits 63 .. 53
constexpr int TR_NB = 1 << TR_HB;    // its bins
constexpr int TR_CAP = 4096;         // keys of the threshold bin held in LDS

// The rem-th largest (1-based) of the keys under `prefix` (their bits under `mask` equal it),
// given the count of keys under it is >= rem, by radix passes over the bits below `lo` + 1
// (8 bits a pass, the last pass narrower).  key(i), i < n, yields the keys.  whist: 16 x 256
// ints of LDS; all 1024 threads call it.  Returns the threshold with the bits below the
// last pass run at zero: the keys >= it are exactly the rem largest under the prefix and
// everything above the prefix.
template <typename KeyAt>
__device__ uint64_t tr_radix(KeyAt key, int n, uint64_t prefix, uint64_t mask, int rem, int lo, int* whist,
                             int* s_hist, int* s_wave, unsigned long long* s_prefix, int* s_rem, int* s_done) {
  const int tid = threadIdx.x;
  if (tid == 0) { *s_prefix = prefix; *s_rem = rem; *s_done = 0; }
  for (int hi = lo; hi >= 0; hi -= 8) {
    const int shift = hi >= 7 ? hi - 7 : 0;
    const uint64_t dmask = (1ull << (hi - shift + 1)) - 1ull;
    for (int q = tid; q < 16 * 256; q += 1024) whist[q] = 0;
    __syncthreads();
    const uint64_t pf = *s_prefix;
    int* myh = whist + (tid >> 6) * 256;
    for (int i = tid; i < n; i += 1024) {
      const uint64_t kv = key(i);
      if ((kv & mask) == pf) atomicAdd(&myh[(kv >> shift) & dmask], 1);
    }
    __syncthreads();
    if (tid < 256) {
      int h = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) h += whist[q * 256 + tid];
      s_hist[tid] = h;
    }
    __syncthreads();
    // thread q takes bin 255 - q: its exclusive prefix counts the keys in the bins above
    const int rm = *s_rem;
    const int bq = 255 - tid;
    const int hq = tid < 256 ? s_hist[bq] : 0;
    int tot;
    const int above = block_excl_scan_1024(hq, s_wave, &tot);
    if (tid < 256 && above < rm && above + hq >= rm) {
      *s_prefix = pf | ((uint64_t)bq << shift);
      *s_rem = rm - above;
      if (above + hq == rm) *s_done = 1;  // the whole bin is kept: zero low bits are exact
    }
    mask |= dmask << shift;
    __syncthreads();
    if (*s_done) break;
  }
  return *s_prefix;
}

// topk_w != NULL (capacity plans): a kept row takes its pair's top-k weight as it is.
// The kept tokens are written in token order: each wavefront owns a contiguous run of tokens,
// counts its kept keys, and after a scan of the sixteen counts writes its rows; then one
// thread per row looks up its weight and pair.
__global__ __launch_bounds__(1024) void k_tr_select(const uint64_t* __restrict__ keys, const float* __restrict__ probs,
                                                    const float* __restrict__ tok_norm, const float* __restrict__ topk_w,
                                                    const int32_t* __restrict__ idx, int N, int E, int k,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ row_of, int32_t* __restrict__ row_token,
                                                    float* __restrict__ row_w, int32_t* __restrict__ row_pair) {
  __shared__ int s_sub[8 * TR_NB];                   // first pass: one histogram per two wavefronts
  __shared__ unsigned long long s_cand[TR_CAP];      // the threshold bin's keys
  __shared__ int s_hist[256];
  __shared__ int s_wave[17];
  __shared__ int s_cnt[16];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_rem, s_done, s_nc, s_bin, s_above, s_hq;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;
  const int r = counts[e];
  const int off = offsets[e];
  const uint64_t* ke = keys + (size_t)e * N;
  uint64_t thr = ~0ull;  // no key reaches it: nothing kept
  if (r > 0) {
    for (int q = tid; q < 8 * TR_NB; q += 1024) s_sub[q] = 0;
    __syncthreads();
    {
      int* h = s_sub + (wv >> 1) * TR_NB;
#pragma unroll 4
      for (int t = tid; t < N; t += 1024) atomicAdd(&h[ke[t] >> (64 - TR_HB)], 1);
    }
    __syncthreads();
    // thread q owns bins TR_NB-1-2q and TR_NB-2-2q (from the top); r <= N, so exactly one
    // bin holds the r-th largest key
    {
      const int b0 = TR_NB - 1 - 2 * tid, b1 = b0 - 1;
      int h0 = 0, h1 = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        h0 += s_sub[u * TR_NB + b0];
        h1 += s_sub[u * TR_NB + b1];
      }
      int tot;
      const int above = block_excl_scan_1024(h0 + h1, s_wave, &tot);
      if (above < r && above + h0 >= r) {
        s_bin = b0; s_above = above; s_hq = h0;
      } else if (above + h0 < r && above + h0 + h1 >= r) {
        s_bin = b1; s_above = above + h0; s_hq = h1;
      }
      if (tid == 0) s_nc = 0;
      __syncthreads();
    }
    const int bin = s_bin, rem = r - s_above, hq = s_hq;
    const uint64_t prefix = (uint64_t)bin << (64 - TR_HB);
    const uint64_t mask = ~0ull << (64 - TR_HB);
    if (rem == hq) {
      thr = prefix;  // the whole bin is kept
    } else if (hq <= TR_CAP) {
      // gather the bin's keys (in any order: keys are distinct)
      for (int b = 0; b < N; b += 1024) {
        const int t = b + tid;
        const uint64_t kv = t < N ? ke[t] : 0ull;
        const bool in = t < N && (kv >> (64 - TR_HB)) == (uint64_t)bin;
        const unsigned long long m = __ballot(in);
        if (m) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&s_nc, __popcll(m));
          base = __builtin_amdgcn_readfirstlane(base);
          if (in) s_cand[base + __popcll(m & ((1ull << lane) - 1ull))] = kv;
        }
      }
      __syncthreads();
      thr = tr_radix([&](int i) { return (uint64_t)s_cand[i]; }, hq, prefix, mask, rem, 63 - TR_HB, s_sub, s_hist,
                     s_wave, &s_prefix, &s_rem, &s_done);
    } else {
      thr = tr_radix([&](int i) { return ke[i]; }, N, prefix, mask, rem, 63 - TR_HB, s_sub, s_hist, s_wave,
                     &s_prefix, &s_rem, &s_done);
    }
  }
  // kept keys, by wavefront runs of ch tokens (a multiple of 64): count, scan the sixteen
  // counts, then write row_of and row_token in token order
  const int ch = (((N + 15) / 16) + 63) & ~63;
  const int t0 = wv * ch, t1 = min(N, t0 + ch);
  int cnt = 0;
  for (int b = t0; b < t1; b += 256) {  // four groups of 64 tokens, their loads first
    uint64_t kv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = b + 64 * u + lane;
      kv[u] = t < t1 ? ke[t] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) cnt += __popcll(__ballot(b + 64 * u + lane < t1 && kv[u] >= thr));
  }
  if (lane == 0) s_cnt[wv] = cnt;
  __syncthreads();
  int run = off;
  for (int q = 0; q < wv; ++q) run += s_cnt[q];
  for (int b = t0; b < t1; b += 256) {
    uint64_t kv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = b + 64 * u + lane;
      kv[u] = t < t1 ? ke[t] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = b + 64 * u + lane;
      const bool sel = t < t1 && kv[u] >= thr;
      const unsigned long long m = __ballot(sel);
      if (t < t1) {
        int row = -1;
        if (sel) {
          row = run + __popcll(m & ((1ull << lane) - 1ull));
          row_token[row] = t;
        }
        row_of[(size_t)e * N + t] = row;
      }
      run += __popcll(m);
    }
  }
  // the expert's rows, one thread each: weight and pair (every load independent)
  __syncthreads();
  for (int i = tid; i < r; i += 1024) {
    const int row = off + i;
    const int t = row_token[row];
    int pair = -1;
    for (int j0 = 0; j0 < k; j0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = j0 + u < k ? idx[(size_t)t * k + j0 + u] : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (pair < 0 && v[u] == e) pair = t * k + j0 + u;
    }
    const float pv = probs[(size_t)t * E + e], tn = tok_norm[t];
    row_w[row] = (topk_w && pair >= 0) ? topk_w[pair] : pv / tn;
    row_pair[row] = pair;
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
// Writes each token's row count and each block's total.
__global__ __launch_bounds__(256) void k_tr_tokcount(const int32_t* __restrict__ row_of, int N, int E,
                                                     int32_t* __restrict__ tcount, int32_t* __restrict__ btot) {
  __shared__ int s_c[4][64];
  const int tl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + tl;
  const int e0 = g * E / 4, e1 = (g + 1) * E / 4;
  s_c[g][tl] = t < N ? tr_count_rows(row_of, N, t, e0, e1) : 0;
  __syncthreads();
  if (g == 0) {
    const int c = s_c[0][tl] + s_c[1][tl] + s_c[2][tl] + s_c[3][tl];
    if (t < N) tcount[t] = c;
    int v = c;  // integer sum over the wavefront (any order is exact)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (tl == 0) btot[blockIdx.x] = v;
  }
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
// quarters 0 .. g-1.  btot != NULL (few blocks): tok_ptr is not scanned yet; the block adds
// the totals of the blocks before it and scans its own 64 tokens' counts, and writes tok_ptr
// (the last block also tok_ptr[N]).
__global__ __launch_bounds__(256) void k_tr_tokfill(const int32_t* __restrict__ row_of, int N, int E,
                                                    const int32_t* __restrict__ btot,
                                                    int32_t* __restrict__ tok_ptr,
                                                    int32_t* __restrict__ tok_rows) {
  __shared__ int s_c[4][64];
  __shared__ int s_base[4];
  const int tl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + tl;
  const int e0 = g * E / 4, e1 = (g + 1) * E / 4;
  s_c[g][tl] = t < N ? tr_count_rows(row_of, N, t, e0, e1) : 0;
  if (btot) {
    int v = 0;  // the totals of blocks 0 .. blockIdx.x - 1 (integer sums: any order is exact)
    for (int q = threadIdx.x; q < (int)blockIdx.x; q += 256) v += btot[q];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (tl == 0) s_base[g] = v;
  }
  __syncthreads();
  int p;
  if (btot) {
    const int c = s_c[0][tl] + s_c[1][tl] + s_c[2][tl] + s_c[3][tl];
    int x = c;  // inclusive scan of the 64 counts over the wavefront
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (tl >= o) x += y;
    }
    p = s_base[0] + s_base[1] + s_base[2] + s_base[3] + x - c;
    if (g == 0 && t < N) {
      tok_ptr[t] = p;
      if (t == N - 1) tok_ptr[N] = p + c;
    }
  }
  if (t >= N) return;
  if (!btot) p = tok_ptr[t];
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

// histogram and token blocks of the plan: 64 tokens
constexpr int kTrTB = 64;

// the route kernel's token normalisers, in the plan's workspace after the histogram
float* tr_tok_norm(void* ws, int N, int E) {
  const size_t nb = ((size_t)N + kTrTB - 1) / kTrTB;
  return (float*)((char*)ws + align256(nb * E * 4));
}

size_t tr_ws_bytes(int N, int E) {
  const size_t nb = ((size_t)N + kTrTB - 1) / kTrTB;
  return align256(nb * E * 4) + align256((size_t)N * 4) + align256((size_t)E * N * 8) +
         align256((size_t)E * N * 4) + align256((size_t)N * 4) + align256(nb * 4) + 256;
}

hipError_t launch_token_round(const int32_t* idx, const float* probs, const float* tok_norm, const float* topk_w,
                              int N, int E, int k, int cap, int param, int use_p, const moe_plan& p, void* ws,
                              hipStream_t s) {
  const int nb = (N + kTrTB - 1) / kTrTB;
  char* w = (char*)ws;
  int32_t* bcnt = (int32_t*)w;
  w += align256((size_t)nb * E * 4);
  w += align256((size_t)N * 4);  // tok_norm lives here (written by the route kernel)
  uint64_t* keys = (uint64_t*)w;
  w += align256((size_t)E * N * 8);
  int32_t* row_of = (int32_t*)w;
  w += align256((size_t)E * N * 4);
  int32_t* tcount = (int32_t*)w;
  w += align256((size_t)N * 4);
  int32_t* btot = (int32_t*)w;
  // while the token blocks are few, the fill kernel scans the block totals itself
  const bool fused = nb <= 1024;
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
    hipLaunchKernelGGL(k_tr_tokcount, dim3(nb), dim3(256), 0, s, row_of, N, E, tcount, btot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (N == 0 || !fused) {
    hipLaunchKernelGGL(k_scan_tokens, dim3(1), dim3(1024), 0, s, tcount, N, p.tok_ptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (N > 0) {
    hipLaunchKernelGGL(k_tr_tokfill, dim3(nb), dim3(256), 0, s, row_of, N, E, fused ? btot : nullptr, p.tok_ptr,
                       p.tok_rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
