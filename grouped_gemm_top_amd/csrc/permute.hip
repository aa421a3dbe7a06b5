// permute.hip -- routing plan: per-expert counts, offsets and the stable expert-sorted row order.
//
// Pages cited (by title, then section):
//   [GG]  "DeepSeek 계열 MoE 학습 가속: Python expert loop → grouped GEMM",
//         section "적용 — fused MoE training forward", steps (1)-(3): flatten the top-k ids,
//         sort by expert id so each expert's rows are one contiguous slice, bincount
//   [DEP] "Deep EP", section "2) Dispatch" (ragged layout needs offset/index metadata)
//
// A stable counting sort over the N*k (token, slot) pairs, never a comparison sort, in two
// launches while the token blocks are few (k_perm_hist, then k_perm_scan_scatter: every block
// sums the whole histogram itself), else in three:
//   k_perm_hist     per block of TB tokens: expert histogram in LDS -> bcnt[b][e]
//   k_perm_scan     counts[e] = sum_b bcnt[b][e]; offsets = exclusive scan over e;
//                   bbase[b][e] = offsets[e] + sum_{b'<b} bcnt[b'][e]
//   k_perm_scatter  rank of a pair inside (block, expert) = number of earlier tokens of the
//                   block routed to the same expert (an LDS bitmask of the block's 64 tokens
//                   and one popcount), so rows of an expert ascend by token; also writes the
//                   token-major row lists
// Integer counting only: the plan is bit-exact and independent of scheduling.
//
// A pair (t, j) makes a row only if its expert id is in [0, E) and no earlier slot of the
// same token names the same expert; other pairs (which the router never produces) are
// skipped by every kernel here, so the plan stays consistent: counts and offsets count the
// rows made, token t's rows fill tok_rows[t k ..] in ascending row order and its remaining
// slots hold -1.
#include <mutex>

#include "common.h"

namespace moe {

constexpr int kPT = 256;  // threads per block
constexpr int kTB = 64;   // tokens per block of the top-k permute (one 64-bit mask per expert)

// per-block expert histogram; pair p of the block is (token p / k, slot p % k), read in order
// Pair j of a token (slots `it`) makes a row: its expert id is in range and is the first
// occurrence of that id among the token's slots.
__device__ __forceinline__ bool pair_makes_row(const int32_t* it, int j, int e, int E) {
  if (e < 0 || e >= E) return false;
  for (int x = 0; x < j; ++x)
    if (it[x] == e) return false;
  return true;
}

template <int TB>
__global__ __launch_bounds__(kPT) void k_perm_hist(const int32_t* __restrict__ idx, int N, int E, int k,
                                                   int32_t* __restrict__ bcnt) {
  __shared__ int s_cnt[1024];
  for (int e = threadIdx.x; e < E; e += kPT) s_cnt[e] = 0;
  __syncthreads();
  const long long t0 = (long long)blockIdx.x * TB;
  const int np = (int)(min((long long)TB, (long long)N - t0) * k);
  const int32_t* ib = idx + t0 * k;
  for (int q = threadIdx.x; q < np; q += kPT) {
    const int e = ib[q], tl = q / k;
    if (pair_makes_row(ib + (size_t)tl * k, q - tl * k, e, E)) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPT) bcnt[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// One block of 1024 threads.  Thread (part, e) owns the contiguous run of blocks
// [part * C, part * C + C) of expert e (P = 1024 / ES parts, ES = E rounded up to a power of
// two), so the per-expert sums and the block bases need one pass over short runs.
__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ bcnt, int nb, int N, int E, int k,
                                                    int32_t* __restrict__ bbase, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ tok_ptr) {
  __shared__ int s_part[1024];
  __shared__ int s_wave[17];
  int ES = 1;
  while (ES < E) ES <<= 1;
  const int P = 1024 / ES;
  const int e = threadIdx.x % ES, part = threadIdx.x / ES;
  const int C = (nb + P - 1) / P;
  const int b0 = part * C, b1 = min(nb, b0 + C);
  int c = 0;
  if (e < E) {
    for (int b = b0; b < b1; ++b) c += bcnt[(size_t)b * E + e];
  }
  s_part[threadIdx.x] = c;
  __syncthreads();
  // expert totals (thread e of part 0) and this thread's base within its expert
  int before = 0, total = 0;
  for (int q = 0; q < P; ++q) {
    const int v = s_part[q * ES + e];
    if (q < part) before += v;
    total += v;
  }
  // exclusive scan of the totals over e (threads of part 0 hold e = 0 .. ES-1 in order)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = (part == 0 && e < E) ? total : 0;
  const int xin = x;
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
  if (part == 0 && e < E) {
    const int ex = s_wave[wv] + x - xin;
    counts[e] = total;
    offsets[e] = ex;
    s_part[e] = ex;  // every thread of expert e has read its s_part values above
  }
  __syncthreads();
  if (e < E) {
    int run = s_part[e] + before;
    for (int b = b0; b < b1; ++b) {
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

// The scatter of block b's pairs (tokens 64 b .. 64 b + 63): bb[e] is the first row of expert
// e that this block fills.  Called by every thread of the block.
// The block's two LDS bitmaps: s_bits[2e ..] = which of the block's 64 tokens chose expert e,
// s_texp[tl EW ..] = which experts token tl chose.  Needs only the router's ids, so a caller
// can run it before its scan (the loads of the ids then overlap the scan's); the bitmaps are
// complete after the caller's next __syncthreads.
__device__ __forceinline__ void perm_block_bits(const int32_t* __restrict__ idx, int N, int E, int k,
                                                int32_t* __restrict__ tok_ptr, uint32_t* s_bits, uint32_t* s_texp) {
  const int EW = (E + 31) >> 5;
  for (int q = threadIdx.x; q < 2 * E; q += kPT) s_bits[q] = 0u;
  for (int q = threadIdx.x; q < kTB * EW; q += kPT) s_texp[q] = 0u;
  __syncthreads();
  const int t0 = blockIdx.x * kTB;
  const int nt = min(kTB, N - t0);
  const int np = nt * k;
  const int32_t* ib = idx + (size_t)t0 * k;
  for (int q = threadIdx.x; q < np; q += kPT) {
    const int e = ib[q], tl = q / k;
    if (e >= 0 && e < E) {  // (a repeated id sets the same bits again)
      atomicOr(&s_bits[2 * e + (tl >> 5)], 1u << (tl & 31));
      atomicOr(&s_texp[tl * EW + (e >> 5)], 1u << (e & 31));
    }
  }
  if (threadIdx.x < nt) tok_ptr[t0 + threadIdx.x] = (t0 + threadIdx.x) * k;
}

// The block's rows, from the bitmaps of perm_block_bits (complete: the caller synchronised
// after it) and the experts' row bases bb.
__device__ __forceinline__ void perm_block_rows(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                int N, int E, int k, const int* bb, int32_t* __restrict__ row_token,
                                                float* __restrict__ row_w, int32_t* __restrict__ row_pair,
                                                int32_t* __restrict__ tok_rows, const uint32_t* s_bits,
                                                const uint32_t* s_texp) {
  const int EW = (E + 31) >> 5;
  const int t0 = blockIdx.x * kTB;
  const int nt = min(kTB, N - t0);
  const int np = nt * k;
  const int32_t* ib = idx + (size_t)t0 * k;
  for (int q = threadIdx.x; q < np; q += kPT) {
    const int e = ib[q];
    const int tl = q / k, j = q - tl * k;
    const int t = t0 + tl;
    const uint32_t* tx = s_texp + tl * EW;
    if (!pair_makes_row(ib + (size_t)tl * k, j, e, E)) {
      // a skipped pair: the token's slots past its rows hold -1 (slot j is one of them when
      // j >= the number of distinct in-range experts of the token)
      int nrow = 0;
      for (int x = 0; x < EW; ++x) nrow += __popc(tx[x]);
      if (j >= nrow) tok_rows[(size_t)t * k + j] = -1;
      continue;
    }
    const uint32_t lo = s_bits[2 * e], hi = s_bits[2 * e + 1];
    const int rank = tl < 32 ? __popc(lo & ((1u << tl) - 1u)) : __popc(lo) + __popc(hi & ((1u << (tl - 32)) - 1u));
    const int row = bb[e] + rank;
    row_token[row] = t;
    row_w[row] = w[(size_t)t * k + j];
    row_pair[row] = t * k + j;
    // rows ascend with the expert id, so the token-major position is the number of this
    // token's distinct experts with a smaller id; slots past the token's rows are filled with
    // -1 above, and a token whose k experts are distinct and in range has exactly k rows
    int pos = __popc(tx[e >> 5] & ((1u << (e & 31)) - 1u));
    for (int x = 0; x < (e >> 5); ++x) pos += __popc(tx[x]);
    tok_rows[(size_t)t * k + pos] = row;
    int nrow = pos + __popc(tx[e >> 5] >> (e & 31));
    for (int x = (e >> 5) + 1; x < EW; ++x) nrow += __popc(tx[x]);
    if (j >= nrow) tok_rows[(size_t)t * k + j] = -1;
  }
}

__device__ __forceinline__ void perm_scatter_block(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                   int N, int E, int k, const int* bb, int32_t* __restrict__ row_token,
                                                   float* __restrict__ row_w, int32_t* __restrict__ row_pair,
                                                   int32_t* __restrict__ tok_ptr, int32_t* __restrict__ tok_rows,
                                                   uint32_t* s_bits, uint32_t* s_texp) {
  perm_block_bits(idx, N, E, k, tok_ptr, s_bits, s_texp);
  __syncthreads();
  perm_block_rows(idx, w, N, E, k, bb, row_token, row_w, row_pair, tok_rows, s_bits, s_texp);
}

__global__ __launch_bounds__(kPT) void k_perm_scatter(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      int N, int E, int k, const int32_t* __restrict__ bbase,
                                                      int32_t* __restrict__ row_token, float* __restrict__ row_w,
                                                      int32_t* __restrict__ row_pair, int32_t* __restrict__ tok_ptr,
                                                      int32_t* __restrict__ tok_rows) {
  __shared__ uint32_t s_bits[1024 * 2];         // expert e: tokens 0-31 and 32-63 of the block
  __shared__ uint32_t s_texp[kTB * (1024 / 32)];  // token tl: its experts, EW words of 32 ids
  perm_scatter_block(idx, w, N, E, k, bbase + (size_t)blockIdx.x * E, row_token, row_w, row_pair, tok_ptr, tok_rows,
                     s_bits, s_texp);
}

// The scan and the scatter in one launch, for plans with few blocks: every block sums the
// whole histogram itself (counts[e] over all nb blocks and its own base over the blocks before
// it, a pass over nb E integers), scans the counts over e, and scatters its pairs; block 0 also
// writes counts, offsets and tok_ptr[N].  The sums are integer, so every block derives the same
// offsets as k_perm_scan.
__global__ __launch_bounds__(kPT) void k_perm_scan_scatter(const int32_t* __restrict__ idx,
                                                           const float* __restrict__ w, int N, int E, int k,
                                                           const int32_t* __restrict__ bcnt, int nb,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ row_token, float* __restrict__ row_w,
                                                           int32_t* __restrict__ row_pair, int32_t* __restrict__ tok_ptr,
                                                           int32_t* __restrict__ tok_rows) {
  __shared__ int s_tot[1024];
  __shared__ int s_base[1024];
  __shared__ int s_wave[5];
  __shared__ uint32_t s_bits[1024 * 2];
  __shared__ uint32_t s_texp[kTB * (1024 / 32)];
  const int b = blockIdx.x;
  // the block's bitmaps first: their id loads overlap the histogram sums below (the sums'
  // __syncthreads completes them)
  perm_block_bits(idx, N, E, k, tok_ptr, s_bits, s_texp);
  // eight independent loads in flight per thread (the sums are integer, so their order is free)
  auto colsum = [&](int e, int q0, int q1) __attribute__((always_inline)) {
    int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int q = q0;
    for (; q + 8 <= q1; q += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += bcnt[(size_t)(q + u) * E + e];
    }
    for (; q < q1; ++q) acc[0] += bcnt[(size_t)q * E + e];
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  };
  if (2 * E <= kPT) {
    // G groups of E threads (G a power of two, G E <= kPT): group g sums the blocks g, g + G,
    // ... of expert e, those before b into the base and all into the total, eight loads in
    // flight; then the G partial sums are added
    __shared__ int s_pb[kPT], s_pt[kPT];
    int G = 2;
    while (2 * G * E <= kPT) G *= 2;
    const int g = threadIdx.x / E, e = threadIdx.x - g * E;
    int pb = 0, pt = 0;
    if (g < G) {
      int ab[8] = {0, 0, 0, 0, 0, 0, 0, 0}, at[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      int q = g;
      for (; q + 7 * G < nb; q += 8 * G) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = bcnt[(size_t)(q + u * G) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          at[u] += v[u];
          if (q + u * G < b) ab[u] += v[u];
        }
      }
      for (; q < nb; q += G) {
        const int v = bcnt[(size_t)q * E + e];
        at[0] += v;
        if (q < b) ab[0] += v;
      }
      pb = ((ab[0] + ab[1]) + (ab[2] + ab[3])) + ((ab[4] + ab[5]) + (ab[6] + ab[7]));
      pt = ((at[0] + at[1]) + (at[2] + at[3])) + ((at[4] + at[5]) + (at[6] + at[7]));
    }
    s_pb[threadIdx.x] = pb;
    s_pt[threadIdx.x] = pt;
    __syncthreads();
    if (threadIdx.x < E) {
      int sb = 0, st = 0;
      for (int q = 0; q < G; ++q) {
        sb += s_pb[q * E + threadIdx.x];
        st += s_pt[q * E + threadIdx.x];
      }
      s_base[threadIdx.x] = sb;
      s_tot[threadIdx.x] = st;
    }
  } else {
    for (int e = threadIdx.x; e < E; e += kPT) {
      const int bef = colsum(e, 0, b);
      s_tot[e] = bef + colsum(e, b, nb);
      s_base[e] = bef;
    }
  }
  __syncthreads();
  // exclusive scan of the totals: thread x owns experts 4x .. 4x + 3 (E <= 1024)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int v4[4], sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * threadIdx.x + u;
    v4[u] = e < E ? s_tot[e] : 0;
    sum += v4[u];
  }
  int x = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int q = 0; q < kPT / 64; ++q) {
      const int v = s_wave[q];
      s_wave[q] = run;
      run += v;
    }
    s_wave[kPT / 64] = run;
  }
  __syncthreads();
  int ex = s_wave[wv] + x - sum;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = 4 * threadIdx.x + u;
    if (e < E) {
      if (b == 0) {
        counts[e] = v4[u];
        offsets[e] = ex;
      }
      s_base[e] += ex;  // this thread alone touches entry e here
    }
    ex += v4[u];
  }
  if (b == 0 && threadIdx.x == 0) {
    offsets[E] = s_wave[kPT / 64];
    tok_ptr[N] = N * k;
  }
  __syncthreads();
  perm_block_rows(idx, w, N, E, k, s_base, row_token, row_w, row_pair, tok_rows, s_bits, s_texp);
}

// Scratch of moe_permute_noalloc: a fixed device array, one copy per GPU for the life of the
// process, holding what the workspace holds for moe_permute (the per-block histogram and the
// block bases, permute_ws_bytes(N, E) bytes).  Nothing in it needs clearing: k_perm_hist writes
// every histogram entry and k_perm_scan every block base.  Calls that overlap on one GPU share
// it and race.
constexpr size_t kPermuteScratchBytes = size_t(4) << 20;
static __device__ __attribute__((aligned(256))) char scratch[kPermuteScratchBytes];

size_t permute_scratch_bytes() { return kPermuteScratchBytes; }

// The device address of `scratch` on the current device, looked up once per device (the
// array's name in host code is a host-side stand-in, not a device address).
hipError_t permute_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

size_t permute_ws_bytes(int N, int E) {
  const size_t nb = ((size_t)N + kTB - 1) / kTB;
  return 2 * (((nb * E * 4) + 255) & ~(size_t)255) + 256;
}

// histogram over blocks of 64 tokens (the token-rounding plan's layout: bcnt[ceil(N/64)][E])
hipError_t launch_perm_hist(const int32_t* idx, int N, int E, int k, int32_t* bcnt, hipStream_t s) {
  const int nb = (N + kTB - 1) / kTB;
  hipLaunchKernelGGL(k_perm_hist<kTB>, dim3(nb), dim3(kPT), 0, s, idx, N, E, k, bcnt);
  return hipGetLastError();
}

// The histogram step is done (bcnt in the workspace, blocks of kTB tokens): the scan and the
// scatter, in one launch while the blocks are few enough for every block to sum the whole
// histogram (nb^2 E integers read in all), else in two.
static hipError_t launch_perm_finish(const int32_t* idx, const float* w, int N, int E, int k, const moe_plan& p,
                                     void* ws, hipStream_t s) {
  const int nb = (N + kTB - 1) / kTB;
  int32_t* bcnt = (int32_t*)ws;
  int32_t* bbase = (int32_t*)((char*)ws + ((((size_t)nb * E * 4) + 255) & ~(size_t)255));
  hipError_t err;
  if (nb > 0 && (long long)nb * nb * E <= (1LL << 25)) {
    hipLaunchKernelGGL(k_perm_scan_scatter, dim3(nb), dim3(kPT), 0, s, idx, w, N, E, k, bcnt, nb, p.counts,
                       p.offsets, p.row_token, p.row_w, p.row_pair, p.tok_ptr, p.tok_rows);
    return hipGetLastError();
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

hipError_t launch_permute(const int32_t* idx, const float* w, int N, int E, int k, const moe_plan& p, void* ws,
                          hipStream_t s) {
  const int nb = (N + kTB - 1) / kTB;
  if (nb > 0) {
    hipLaunchKernelGGL(k_perm_hist<kTB>, dim3(nb), dim3(kPT), 0, s, idx, N, E, k, (int32_t*)ws);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return launch_perm_finish(idx, w, N, E, k, p, ws, s);
}

}  // namespace moe
