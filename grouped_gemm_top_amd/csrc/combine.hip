// combine.hip -- weighted combine of expert rows back to token order.
//
// Pages cited (by title, then section):
//   [EP]  "EP: Expert를 나누고 토큰 보내기", section "여러 Expert의 결과도 같은 토큰으로 돌아오기"
//         (each token's expert outputs are summed with the combine weights, back at the token)
//   [DEP] "Deep EP", section "3) Combine" (weighted sum of the k expert outputs per token)
//
//   out[t] = sum over r in tok_rows[tok_ptr[t] .. tok_ptr[t+1]) of row_w[r] * y[r]
// (slots holding -1, pairs the plan skipped, add nothing)
// One workgroup per token, 16-byte vectors along H, fp32 accumulation in ascending row
// order (deterministic, no atomics).  Pure HBM streaming: each y row is read once.  A thread
// loads the vectors of up to RB rows before it accumulates any of them, so RB loads per lane
// are in flight instead of one (with one load at a time the kernel is bound by memory
// latency, not bandwidth), two such vectors at once on rows of 512 vectors or a multiple
// (NV below); the sum still runs row by row in ascending order.
//
// The dX combine also finishes dS ([SM] "3 기여 ①": the router-score gradient of each row,
// left by the dH GEMM's epilogue as nP partial sums per row): thread i of token t's
// workgroup adds the partials of the token's rows i, i + 256, ... in partial order and writes
// the pair's entry (top-k plans) or the row's (other plans, whose unused rows M .. M_cap get
// zeros from extra workgroups of 4096 rows each).
#include "common.h"

namespace moe {

struct DsSum {
  const float* part;  // [M_cap, nP]; NULL: no dS work
  int nP, by_pair;
  float* ds;
};

// NV: vectors per thread at a time (v0 + 256 h, h < NV), NV * RB loads in flight; NV = 2 for
// rows of 512 vectors or a multiple (H = 4096 in bf16), whose rows then come from HBM.  Other
// widths keep NV = 1 (with a partial second vector the workgroup's threads would carry unequal
// work, which measured slower), in a kernel of their own so that their register count, and
// with it the number of workgroups a CU holds, stays that of one vector.
template <typename T, int NV>
__global__ __launch_bounds__(256) void k_combine(const T* __restrict__ y, int H, const int32_t* __restrict__ tok_ptr,
                                                 const int32_t* __restrict__ tok_rows,
                                                 const float* __restrict__ row_w, T* __restrict__ out, moe_plan p,
                                                 DsSum d) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int RB = 8;
  const int t = blockIdx.x;
  if (t >= p.N) {  // zero the unused rows' dS (row-ordered plans)
    const int M = p.offsets[p.E];
    const int lo = max(M, (t - p.N) * 4096), hi = min(p.M_cap, (t - p.N + 1) * 4096);
    for (int r = lo + (int)threadIdx.x; r < hi; r += 256) d.ds[r] = 0.f;
    return;
  }
  const int q0 = tok_ptr[t], q1 = tok_ptr[t + 1];
  // dS of the token's first 256 rows: thread i loads row i's first DSP partials (and its pair)
  // before the row sums below and adds them after, so that their latency overlaps that work;
  // the sum runs in partial order either way
  constexpr int DSP = 4;
  int dr = -1, dpair = -1;
  float dp[DSP];
  if (d.part && (int)threadIdx.x < q1 - q0) {
    dr = tok_rows[q0 + threadIdx.x];
    if (dr >= 0) {
#pragma unroll
      for (int q = 0; q < DSP; ++q) dp[q] = q < d.nP ? d.part[(size_t)dr * d.nP + q] : 0.f;
      if (d.by_pair) dpair = p.row_pair[dr];
    }
  }
  auto ds_out = [&](int r, int pair, float sum) __attribute__((always_inline)) {
    if (d.by_pair) {
      if (pair >= 0) d.ds[pair] = sum;
    } else {
      d.ds[r] = sum;
    }
  };
  const int nv = H / VEC;
  for (int v0 = threadIdx.x; v0 < nv; v0 += 256 * NV) {
    float acc[NV][VEC];
#pragma unroll
    for (int h = 0; h < NV; ++h)
#pragma unroll
      for (int c = 0; c < VEC; ++c) acc[h][c] = 0.f;
    for (int qb = q0; qb < q1; qb += RB) {
      uint4 raw[NV][RB];
      float wr[RB];
      uint32_t live = 0u;  // bit u: slot qb + u is one of the token's rows
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        // past the token's last row the load repeats that row, and the sum below skips it; a
        // slot of -1 (a pair the plan skipped) loads row 0 and is skipped too
        const int r = tok_rows[min(qb + u, q1 - 1)];
        const int rr = r < 0 ? 0 : r;
        if (qb + u < q1 && r >= 0) live |= 1u << u;
        wr[u] = row_w ? row_w[rr] : 1.0f;
#pragma unroll
        for (int h = 0; h < NV; ++h)
          raw[h][u] = *reinterpret_cast<const uint4*>(y + (size_t)rr * H + (size_t)(v0 + 256 * h) * VEC);
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        if (live & (1u << u)) {  // uniform across the workgroup
#pragma unroll
          for (int h = 0; h < NV; ++h) {
            const T* vals = reinterpret_cast<const T*>(&raw[h][u]);
#pragma unroll
            for (int c = 0; c < VEC; ++c) acc[h][c] += wr[u] * to_f32<T>(vals[c]);
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < NV; ++h) {
      uint4 o;
      T* ov = reinterpret_cast<T*>(&o);
#pragma unroll
      for (int c = 0; c < VEC; ++c) ov[c] = from_f32<T>(acc[h][c]);
      *reinterpret_cast<uint4*>(out + (size_t)t * H + (size_t)(v0 + 256 * h) * VEC) = o;
    }
  }
  if (dr >= 0) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < DSP; ++q)
      if (q < d.nP) sum += dp[q];
    for (int q = DSP; q < d.nP; ++q) sum += d.part[(size_t)dr * d.nP + q];
    ds_out(dr, dpair, sum);
  }
  // rows past the first 256 of a token (plans that give a token more rows than that)
  for (int i = threadIdx.x + 256; d.part && i < q1 - q0; i += 256) {
    const int r = tok_rows[q0 + i];
    if (r >= 0) {
      float sum = 0.f;
      for (int q = 0; q < d.nP; ++q) sum += d.part[(size_t)r * d.nP + q];
      ds_out(r, d.by_pair ? p.row_pair[r] : -1, sum);
    }
  }
}

hipError_t launch_combine(moe_dtype dt, const void* y, int H, const moe_plan& p, const float* row_w, void* out,
                          hipStream_t s, const float* dspart, int nP, float* ds) {
  DsSum d{dspart, nP, p.kind == MOE_PLAN_TOPK ? 1 : 0, ds};
  const long long z = (dspart && !d.by_pair) ? ((long long)p.M_cap + 4095) / 4096 : 0;
  const long long g = (long long)p.N + z;
  if (g == 0) return hipSuccess;
  const bool two = (H / (dt == MOE_BF16 ? 8 : 4)) % 512 == 0;
  if (dt == MOE_BF16) {
    auto* k = two ? k_combine<bf16_t, 2> : k_combine<bf16_t, 1>;
    hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(256), 0, s, (const bf16_t*)y, H, p.tok_ptr, p.tok_rows, row_w,
                       (bf16_t*)out, p, d);
  } else {
    auto* k = two ? k_combine<float, 2> : k_combine<float, 1>;
    hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(256), 0, s, (const float*)y, H, p.tok_ptr, p.tok_rows, row_w,
                       (float*)out, p, d);
  }
  return hipGetLastError();
}

}  // namespace moe
