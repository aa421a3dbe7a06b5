// gemm.hip -- persistent grouped GEMMs over the ragged expert groups, forward and backward.
//
// Pages cited (by title, then section):
//   [GG] "DeepSeek 계열 MoE 학습 가속: Python expert loop → grouped GEMM",
//        sections "무엇이 필요한가 — Variable-M batched matmul" (a ragged-M grouped GEMM in one
//        launch instead of a per-expert loop) and "적용" step (6) (gate, up and down share one
//        set of group sizes)
//   [SM] "SonicMoE: IO·타일 인식 최적화로 MoE 학습 가속하기", sections
//        "3 기여 ①" (cache H=[G|U] only; dS from <dA', A> without Y),
//        "4 기여 ②" (varlen-M / varlen-K grouped GEMMs), "4.1 Gather 융합" (gather fused into
//        the global->shared load, backward too), "4.2 Epilogue 융합" (SwiGLU / dSwiGLU in the
//        epilogue; dH, dS and A' from one epilogue), "2 왜 fine-grained·sparse MoE는 느려지나"
//        (tile quantisation), "7 한계 & 의의" (no atomic-add reductions)
//
// Design (gfx950):
//  * One kernel template, six problems.  A workgroup of 256 threads (4 wavefronts, 2x2)
//    owns a 128x128 output tile; each wavefront owns 64x64 = 4x4 MFMA blocks of 16x16.
//    bf16: v_mfma_f32_16x16x32_bf16 (K=64 per LDS stage); fp32: v_mfma_f32_16x16x4f32 (K=32).
//  * Operands are staged global -> VGPR -> LDS with two LDS stages; the next stage's global
//    loads are in flight while the current stage feeds the MFMAs.  LDS holds both operands
//    K-contiguous ([row][k], rows padded by 16 bytes), so every MFMA fragment is one
//    16-byte LDS read.  Operands that are K-strided in memory (the backward's weight
//    operands and both varlen-K operands) are transposed in registers (4 k-rows x 8 values)
//    on their way into LDS.
//  * The MFMA is issued with the operands swapped (B fragment first), so each lane ends up
//    with 4 consecutive output columns of one row: the epilogue stores 8/16-byte vectors.
//  * Token gathers are fused into the A/B loads through row_token: permuted activations are
//    never materialised.
//  * Persistent grid (2 workgroups per CU, a multiple of the 8 XCDs).  Each workgroup
//    computes the tile space from the device-resident counts (no host sync): varlen-M tiles
//    are ordered (expert, n-tile, m-tile) so tiles sharing a weight slice are adjacent;
//    varlen-K tiles are ordered heaviest expert first.  Logical tile ranges are handed out
//    per XCD in contiguous chunks, so neighbouring tiles (same weights / same rows) run on
//    the same XCD and share its L2.
//  * No atomics anywhere; the dS row-dot is reduced across lanes and wavefronts in a fixed
//    order and across N-tiles by a separate ordered pass.
#include "common.h"

namespace moe {
namespace gg {

constexpr int BM = 128, BN = 128, NTHR = 256;

enum Kind { GATEUP = MOE_K_GATEUP, DOWN = MOE_K_DOWN, DH = MOE_K_DH, DX = MOE_K_DX, DWD = MOE_K_DWD, DW1 = MOE_K_DW1 };

template <int K> struct KindTraits;
template <> struct KindTraits<GATEUP> { static constexpr bool A_KC = true, B_KC = true, VK = false; };
template <> struct KindTraits<DOWN> { static constexpr bool A_KC = true, B_KC = true, VK = false; };
template <> struct KindTraits<DH> { static constexpr bool A_KC = true, B_KC = false, VK = false; };
template <> struct KindTraits<DX> { static constexpr bool A_KC = true, B_KC = false, VK = false; };
template <> struct KindTraits<DWD> { static constexpr bool A_KC = false, B_KC = false, VK = true; };
template <> struct KindTraits<DW1> { static constexpr bool A_KC = false, B_KC = false, VK = true; };

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <typename T> struct ElemCfg;
template <> struct ElemCfg<bf16_t> {
  static constexpr int VEC = 8;   // elements per 16-byte vector
  static constexpr int KPL = 8;   // k values per lane per MFMA
  static constexpr int BK = 64;   // k per LDS stage
  static constexpr int LDSW = BK + 8;
  typedef bf16x8 frag_t;
};
template <> struct ElemCfg<float> {
  static constexpr int VEC = 4;
  static constexpr int KPL = 1;
  static constexpr int BK = 32;
  static constexpr int LDSW = BK + 4;
  typedef float frag_t;
};

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Args {
  const void* x;      // [N,H] activations (gathered)
  const void* wg;     // [E,I,H]
  const void* wu;     // [E,I,H]
  const void* wd;     // [E,H,I]
  const void* dout;   // [N,H]
  const void* hcache; // [M_cap, 2I]
  const void* act;    // [M_cap, I]   (DOWN: A;  DWD: A')
  const void* dh;     // [M_cap, 2I]  (DX, DW1)
  void* out0;         // GATEUP: hcache; DOWN: y; DH: dH; DX: dXe; DWD: dW_down; DW1: dW_gate
  void* out1;         // GATEUP: act;  DH: A';  DW1: dW_up
  float* dspart;      // DH: [M_cap, nTN] partial row-dots
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* row_token;
  const float* row_w;
  int E, H, I;
};

struct Tile {
  int e;      // expert
  int roff;   // first plan row of the expert
  int m0;     // varlen-M: row offset inside the expert; varlen-K: first output row
  int n0;     // first output column (GATEUP: first i)
  int nt;     // n-tile index
  int mlen;   // varlen-M: valid rows in this tile
  int K;      // reduction length
};

template <typename T, int KIND>
struct Problem {
  using C = ElemCfg<T>;
  static constexpr int VEC = C::VEC, BK = C::BK;

  __device__ static int n_tiles(const Args& a) {
    switch (KIND) {
      case GATEUP: return (a.I + 63) / 64;
      case DOWN: return (a.H + BN - 1) / BN;
      case DH: return (a.I + BN - 1) / BN;
      case DX: return (a.H + BN - 1) / BN;
      case DWD: return (a.I + BN - 1) / BN;
      default: return (a.H + BN - 1) / BN;  // DW1
    }
  }
  __device__ static int m_tiles_k(const Args& a) {  // varlen-K: output rows
    return KIND == DWD ? (a.H + BM - 1) / BM : (2 * a.I + BM - 1) / BM;
  }
  __device__ static int k_len(const Args& a, int cnt) {
    switch (KIND) {
      case GATEUP: return a.H;
      case DOWN: return a.I;
      case DH: return a.H;
      case DX: return 2 * a.I;
      default: return cnt;
    }
  }

  // ---- K-contiguous operand: row `row` of the tile (tile-local), pointer to element k=0 ----
  __device__ static const T* a_row(const Args& a, const Tile& tl, int row) {
    if (row >= tl.mlen) return nullptr;
    const int r = tl.roff + tl.m0 + row;
    switch (KIND) {
      case GATEUP: return (const T*)a.x + (size_t)a.row_token[r] * a.H;
      case DOWN: return (const T*)a.act + (size_t)r * a.I;
      case DH: return (const T*)a.dout + (size_t)a.row_token[r] * a.H;
      default: return (const T*)a.dh + (size_t)r * (2 * a.I);  // DX
    }
  }
  __device__ static const T* b_row(const Args& a, const Tile& tl, int n) {  // GATEUP, DOWN
    if (KIND == GATEUP) {
      const int seg = (n >> 5) & 1;
      const int i = tl.n0 + (n >> 6) * 32 + (n & 31);
      if (i >= a.I) return nullptr;
      return (const T*)(seg ? a.wu : a.wg) + ((size_t)tl.e * a.I + i) * a.H;
    } else {
      const int h = tl.n0 + n;
      if (h >= a.H) return nullptr;
      return (const T*)a.wd + ((size_t)tl.e * a.H + h) * a.I;
    }
  }
  // ---- MN-contiguous operand: k-row `kk` (global k index), pointer to output column 0 of
  //      the tile's range, and the number of valid columns from there ----
  __device__ static const T* a_krow(const Args& a, const Tile& tl, int kk, int& lim) {  // DWD, DW1
    if (kk >= tl.K) return nullptr;
    const int r = tl.roff + kk;
    if (KIND == DWD) {
      lim = a.H - tl.m0;
      return (const T*)a.dout + (size_t)a.row_token[r] * a.H + tl.m0;
    } else {
      lim = 2 * a.I - tl.m0;
      return (const T*)a.dh + (size_t)r * (2 * a.I) + tl.m0;
    }
  }
  __device__ static const T* b_krow(const Args& a, const Tile& tl, int kk, int& lim) {  // DH, DX, DWD, DW1
    if (kk >= tl.K) return nullptr;
    switch (KIND) {
      case DH:
        lim = a.I - tl.n0;
        return (const T*)a.wd + ((size_t)tl.e * a.H + kk) * a.I + tl.n0;
      case DX:
        lim = a.H - tl.n0;
        return (kk < a.I ? (const T*)a.wg + ((size_t)tl.e * a.I + kk) * a.H
                         : (const T*)a.wu + ((size_t)tl.e * a.I + (kk - a.I)) * a.H) +
               tl.n0;
      case DWD:
        lim = a.I - tl.n0;
        return (const T*)a.act + (size_t)(tl.roff + kk) * a.I + tl.n0;
      default:  // DW1
        lim = a.H - tl.n0;
        return (const T*)a.x + (size_t)a.row_token[tl.roff + kk] * a.H + tl.n0;
    }
  }
};

// ------------------------------------------------------------------ operand staging
template <typename T>
struct Stage {
  using C = ElemCfg<T>;
  static constexpr int VEC = C::VEC, BK = C::BK, LDSW = C::LDSW;
  static constexpr int KG = BK / 4;          // k-groups of 4 for the transposing path
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// K-contiguous: thread -> chunk c = tid % 8 (VEC elements), rows tid/8 + 32v
template <typename T, class Src>
__device__ __forceinline__ void gload_kc(uint4 (&r)[4], const Src& src, int k0, int K) {
  constexpr int VEC = ElemCfg<T>::VEC;
  const int c = threadIdx.x & 7;
  const int kk = k0 + c * VEC;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const T* p = src.rows[v];
    r[v] = (p != nullptr && kk < K) ? ld16(p + kk) : make_uint4(0, 0, 0, 0);
  }
}
template <typename T>
__device__ __forceinline__ void sstore_kc(T* lds, const uint4 (&r)[4]) {
  constexpr int VEC = ElemCfg<T>::VEC, LDSW = ElemCfg<T>::LDSW;
  const int c = threadIdx.x & 7;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = (threadIdx.x >> 3) + 32 * v;
    *reinterpret_cast<uint4*>(lds + row * LDSW + c * VEC) = r[v];
  }
}
// MN-contiguous: thread -> k-group kg = tid % KG (k-rows 4kg..4kg+3), chunk ch = tid / KG
template <typename T>
__device__ __forceinline__ void sstore_mn(T* lds, const uint4 (&r)[4]);
template <>
__device__ __forceinline__ void sstore_mn<bf16_t>(bf16_t* lds, const uint4 (&r)[4]) {
  constexpr int KG = 16, LDSW = ElemCfg<bf16_t>::LDSW;
  const int kg = threadIdx.x % KG, ch = threadIdx.x / KG;
  const uint32_t* q0 = reinterpret_cast<const uint32_t*>(&r[0]);
  const uint32_t* q1 = reinterpret_cast<const uint32_t*>(&r[1]);
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(&r[2]);
  const uint32_t* q3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int h = j >> 1;
    uint2 o;
    if (j & 1) {
      o.x = (q0[h] >> 16) | (q1[h] & 0xFFFF0000u);
      o.y = (q2[h] >> 16) | (q3[h] & 0xFFFF0000u);
    } else {
      o.x = (q0[h] & 0xFFFFu) | (q1[h] << 16);
      o.y = (q2[h] & 0xFFFFu) | (q3[h] << 16);
    }
    *reinterpret_cast<uint2*>(lds + (ch * 8 + j) * LDSW + 4 * kg) = o;
  }
}
template <>
__device__ __forceinline__ void sstore_mn<float>(float* lds, const uint4 (&r)[4]) {
  constexpr int KG = 8, LDSW = ElemCfg<float>::LDSW;
  const int kg = threadIdx.x % KG, ch = threadIdx.x / KG;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint4 o;
    o.x = reinterpret_cast<const uint32_t*>(&r[0])[j];
    o.y = reinterpret_cast<const uint32_t*>(&r[1])[j];
    o.z = reinterpret_cast<const uint32_t*>(&r[2])[j];
    o.w = reinterpret_cast<const uint32_t*>(&r[3])[j];
    *reinterpret_cast<uint4*>(lds + (ch * 4 + j) * LDSW + 4 * kg) = o;
  }
}

template <typename T>
struct RowSrc {
  const T* rows[4];
};

// ------------------------------------------------------------------ the kernel
template <typename T, int KIND>
__global__ __launch_bounds__(NTHR, 2) void k_grouped_gemm(Args a) {
  using C = ElemCfg<T>;
  using P = Problem<T, KIND>;
  using TR = KindTraits<KIND>;
  constexpr int BK = C::BK, LDSW = C::LDSW, VEC = C::VEC, KPL = C::KPL;
  constexpr int KSTEP = 4 * KPL;
  constexpr int KG = BK / 4;
  constexpr int STAGE = (BM + BN) * LDSW;

  __shared__ __attribute__((aligned(16))) T s_tile[2 * STAGE];
  __shared__ int s_sched[1025];
  __shared__ int s_wave[5];
  __shared__ float s_red[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = a.E;
  const int nN = P::n_tiles(a);

  // ---- tile space from the device-resident counts ----
  int total;
  if constexpr (!TR::VK) {
    // per-expert tile count ceil(c/BM)*nN, exclusive prefix over experts (4 per thread)
    int loc[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      loc[q] = e < E ? ((a.counts[e] + BM - 1) / BM) * nN : 0;
      sum += loc[q];
    }
    int x = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int w = 0; w < 4; ++w) {
        const int v = s_wave[w];
        s_wave[w] = run;
        run += v;
      }
      s_wave[4] = run;
    }
    __syncthreads();
    int run = s_wave[wave] + x - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e <= E) s_sched[e] = run;
      run += loc[q];
    }
    total = s_wave[4];
    if (tid == 0) s_sched[E] = total;
    __syncthreads();
  } else {
    // heaviest expert first: rank_e = #{e' : c_e' > c_e or (c_e' == c_e and e' < e)}
    int* s_cnt = reinterpret_cast<int*>(s_tile);  // the operand stages are free until the first tile
    for (int e = tid; e < E; e += NTHR) s_cnt[e] = a.counts[e];
    __syncthreads();
    for (int e = tid; e < E; e += NTHR) {
      const int ce = s_cnt[e];
      int rank = 0;
      for (int f = 0; f < E; ++f) {
        const int cf = s_cnt[f];
        rank += (cf > ce) || (cf == ce && f < e);
      }
      s_sched[rank] = e;
    }
    __syncthreads();
    total = E * P::m_tiles_k(a) * nN;
  }

  const int G = gridDim.x;
  const int per = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  for (int it = 0;; ++it) {
    const long long tile_ll = (long long)it * G + (long long)xcd * per + slot;
    if (tile_ll >= total) break;
    const int tile = (int)tile_ll;

    // ---- decode ----
    Tile tl;
    if constexpr (!TR::VK) {
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_sched[mid] <= tile) lo = mid; else hi = mid;
      }
      const int e = lo;
      const int cnt = a.counts[e];
      const int mtiles = (cnt + BM - 1) / BM;
      const int local = tile - s_sched[e];
      const int mt = local % mtiles, nt = local / mtiles;
      tl.e = e;
      tl.roff = a.offsets[e];
      tl.m0 = mt * BM;
      tl.nt = nt;
      tl.n0 = (KIND == GATEUP) ? nt * 64 : nt * BN;
      tl.mlen = min(BM, cnt - tl.m0);
      tl.K = P::k_len(a, cnt);
    } else {
      const int per_e = P::m_tiles_k(a) * nN;
      const int rank = tile / per_e;
      const int local = tile - rank * per_e;
      const int e = s_sched[rank];
      tl.e = e;
      tl.roff = a.offsets[e];
      tl.m0 = (local / nN) * BM;
      tl.nt = local % nN;
      tl.n0 = tl.nt * BN;
      tl.mlen = BM;
      tl.K = a.counts[e];
    }

    // ---- per-thread operand row pointers (K-contiguous operands) ----
    RowSrc<T> asrc, bsrc;
    if constexpr (TR::A_KC) {
#pragma unroll
      for (int v = 0; v < 4; ++v) asrc.rows[v] = P::a_row(a, tl, (tid >> 3) + 32 * v);
    }
    if constexpr (TR::B_KC) {
#pragma unroll
      for (int v = 0; v < 4; ++v) bsrc.rows[v] = P::b_row(a, tl, (tid >> 3) + 32 * v);
    }

    auto gload = [&](uint4 (&ra)[4], uint4 (&rb)[4], int k0) {
      if constexpr (TR::A_KC) {
        gload_kc<T>(ra, asrc, k0, tl.K);
      } else {
        const int kg = tid % KG, ch = tid / KG;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int lim = 0;
          const T* p = P::a_krow(a, tl, k0 + 4 * kg + q, lim);
          ra[q] = (p != nullptr && ch * VEC < lim) ? ld16(p + ch * VEC) : make_uint4(0, 0, 0, 0);
        }
      }
      if constexpr (TR::B_KC) {
        gload_kc<T>(rb, bsrc, k0, tl.K);
      } else {
        const int kg = tid % KG, ch = tid / KG;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int lim = 0;
          const T* p = P::b_krow(a, tl, k0 + 4 * kg + q, lim);
          rb[q] = (p != nullptr && ch * VEC < lim) ? ld16(p + ch * VEC) : make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto sstore = [&](int s, const uint4 (&ra)[4], const uint4 (&rb)[4]) {
      T* la = s_tile + s * STAGE;
      T* lb = la + BM * LDSW;
      if constexpr (TR::A_KC) sstore_kc<T>(la, ra); else sstore_mn<T>(la, ra);
      if constexpr (TR::B_KC) sstore_kc<T>(lb, rb); else sstore_mn<T>(lb, rb);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (tl.K + BK - 1) / BK;
    uint4 ra[4], rb[4];
    if (nk > 0) {
      gload(ra, rb, 0);
      sstore(0, ra, rb);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int s = kt & 1;
      if (kt + 1 < nk) gload(ra, rb, (kt + 1) * BK);
      const T* la = s_tile + s * STAGE + (wm * 64 + (lane & 15)) * LDSW + (lane >> 4) * KPL;
      const T* lb = s_tile + s * STAGE + (BM + wn * 64 + (lane & 15)) * LDSW + (lane >> 4) * KPL;
#pragma unroll
      for (int ks = 0; ks < BK / KSTEP; ++ks) {
        typename C::frag_t fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fa[i] = *reinterpret_cast<const typename C::frag_t*>(la + i * 16 * LDSW + ks * KSTEP);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          fb[j] = *reinterpret_cast<const typename C::frag_t*>(lb + j * 16 * LDSW + ks * KSTEP);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mma(fb[j], fa[i], acc[i][j]);
      }
      if (kt + 1 < nk) sstore(s ^ 1, ra, rb);
      __syncthreads();
    }

    // ---- epilogue: acc[i][j][v] = C[m = wm*64 + i*16 + (lane&15)][n = wn*64 + j*16 + 4*(lane>>4) + v] ----
    const int mrow = wm * 64 + (lane & 15);
    const int ncol = wn * 64 + 4 * (lane >> 4);
    if constexpr (KIND == GATEUP) {
      T* hc = (T*)a.out0;
      T* ac = (T*)a.out1;
      const int I = a.I;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mrow + i * 16;
        if (m >= tl.mlen) continue;
        const size_t r = (size_t)(tl.roff + tl.m0 + m);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ii = tl.n0 + wn * 32 + j * 16 + 4 * (lane >> 4);
          if (ii >= I) continue;
          const f32x4 g = acc[i][j], u = acc[i][j + 2];
          store4(hc + r * (2 * I) + ii, g[0], g[1], g[2], g[3]);
          store4(hc + r * (2 * I) + I + ii, u[0], u[1], u[2], u[3]);
          float av[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) av[v] = g[v] * sigmoidf_(g[v]) * u[v];
          store4(ac + r * I + ii, av[0], av[1], av[2], av[3]);
        }
      }
    } else if constexpr (KIND == DOWN || KIND == DX) {
      T* out = (T*)a.out0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mrow + i * 16;
        if (m >= tl.mlen) continue;
        const size_t r = (size_t)(tl.roff + tl.m0 + m);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = tl.n0 + ncol + j * 16;
          if (h >= a.H) continue;
          store4(out + r * a.H + h, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    } else if constexpr (KIND == DH) {
      T* dh = (T*)a.out0;
      T* ap = (T*)a.out1;
      const T* hc = (const T*)a.hcache;
      const int I = a.I;
      float dsum[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dsum[i] = 0.f;
        const int m = mrow + i * 16;
        if (m >= tl.mlen) continue;
        const size_t r = (size_t)(tl.roff + tl.m0 + m);
        const float w = a.row_w[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ii = tl.n0 + ncol + j * 16;
          if (ii >= I) continue;
          float g[4], u[4], dg[4], du[4], av[4];
          load4(hc + r * (2 * I) + ii, g[0], g[1], g[2], g[3]);
          load4(hc + r * (2 * I) + I + ii, u[0], u[1], u[2], u[3]);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float sg = sigmoidf_(g[v]);
            const float silu = g[v] * sg;
            const float A = silu * u[v];
            const float dap = acc[i][j][v];
            dsum[i] += dap * A;
            const float da = w * dap;
            dg[v] = da * u[v] * sg * (1.0f + g[v] * (1.0f - sg));
            du[v] = da * silu;
            av[v] = w * A;
          }
          store4(dh + r * (2 * I) + ii, dg[0], dg[1], dg[2], dg[3]);
          store4(dh + r * (2 * I) + I + ii, du[0], du[1], du[2], du[3]);
          store4(ap + r * I + ii, av[0], av[1], av[2], av[3]);
        }
      }
      // row-dot partials: lanes l, l^16, l^32, l^48 hold the same row; then the two
      // wavefronts of a row block (wn = 0, 1), always in the same order
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dsum[i] += __shfl_xor(dsum[i], 16);
        dsum[i] += __shfl_xor(dsum[i], 32);
      }
      if (wn == 1 && lane < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[wm * 64 + i * 16 + lane] = dsum[i];
      }
      __syncthreads();
      if (wn == 0 && lane < 16) {
        const int nTN = (I + BN - 1) / BN;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mrow + i * 16;
          if (m < tl.mlen)
            a.dspart[(size_t)(tl.roff + tl.m0 + m) * nTN + tl.nt] = dsum[i] + s_red[m];
        }
      }
      __syncthreads();
    } else if constexpr (KIND == DWD) {
      T* dw = (T*)a.out0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = tl.m0 + mrow + i * 16;
        if (h >= a.H) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int ii = tl.n0 + ncol + j * 16;
          if (ii >= a.I) continue;
          store4(dw + ((size_t)tl.e * a.H + h) * a.I + ii, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    } else {  // DW1
      T* dwg = (T*)a.out0;
      T* dwu = (T*)a.out1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ip = tl.m0 + mrow + i * 16;
        if (ip >= 2 * a.I) continue;
        T* base = ip < a.I ? dwg + ((size_t)tl.e * a.I + ip) * a.H : dwu + ((size_t)tl.e * a.I + (ip - a.I)) * a.H;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = tl.n0 + ncol + j * 16;
          if (h >= a.H) continue;
          store4(base + h, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    }
  }
}

// dS: ordered sum of the N-tile partials; scattered to (t, j) order through row_pair for
// top-k plans, kept in row order for token-rounding plans.
__global__ __launch_bounds__(256) void k_ds_reduce(const float* __restrict__ dspart, int nTN,
                                                   const int32_t* __restrict__ offsets, int E,
                                                   const int32_t* __restrict__ row_pair, int by_pair, int M_cap,
                                                   float* __restrict__ ds) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= M_cap) return;
  const int M = offsets[E];
  if (r >= M) {
    if (!by_pair) ds[r] = 0.f;
    return;
  }
  float s = 0.f;
  for (int q = 0; q < nTN; ++q) s += dspart[(size_t)r * nTN + q];
  if (by_pair) {
    const int p = row_pair[r];
    if (p >= 0) ds[p] = s;
  } else {
    ds[r] = s;
  }
}

}  // namespace gg

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static int persistent_grid(long long max_tiles) {
  const DevInfo d = dev_info();
  long long g = 2LL * d.cus;
  if (max_tiles < g) g = max_tiles;
  if (g < 8) g = 8;
  return (int)((g + 7) / 8 * 8);
}

template <typename T, int KIND>
static hipError_t run(const gg::Args& a, long long max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  kernel_event(KIND, 0, s);  // gg::Kind values equal the moe_kernel_id of each GEMM
  hipLaunchKernelGGL((gg::k_grouped_gemm<T, KIND>), dim3(persistent_grid(max_tiles)), dim3(gg::NTHR), 0, s, a);
  kernel_event(KIND, 1, s);
  return hipGetLastError();
}

size_t gemm_fwd_ws_bytes(moe_dtype dt, int M_cap, int I) {
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  return align256((size_t)M_cap * I * es) + 256;
}

template <typename T>
static hipError_t gemm_fwd_t(const void* x, const void* wg, const void* wu, const void* wd, int H, int I,
                             const moe_plan& p, void* hcache, void* y, void* ws, hipStream_t s) {
  gg::Args a{};
  a.x = x; a.wg = wg; a.wu = wu; a.wd = wd;
  a.counts = p.counts; a.offsets = p.offsets; a.row_token = p.row_token; a.row_w = p.row_w;
  a.E = p.E; a.H = H; a.I = I;
  void* act = ws;
  const long long mt = (long long)(p.M_cap + gg::BM - 1) / gg::BM + p.E;
  a.out0 = hcache; a.out1 = act;
  hipError_t err = run<T, gg::GATEUP>(a, mt * ((I + 63) / 64), s);
  if (err != hipSuccess) return err;
  a.act = act; a.out0 = y; a.out1 = nullptr;
  return run<T, gg::DOWN>(a, mt * ((H + gg::BN - 1) / gg::BN), s);
}

hipError_t launch_gemm_fwd(moe_dtype dt, const void* x, const void* wg, const void* wu, const void* wd, int H,
                           int I, const moe_plan& p, void* hcache, void* y, void* ws, hipStream_t s) {
  if (dt == MOE_BF16) return gemm_fwd_t<bf16_t>(x, wg, wu, wd, H, I, p, hcache, y, ws, s);
  return gemm_fwd_t<float>(x, wg, wu, wd, H, I, p, hcache, y, ws, s);
}

size_t layer_bwd_ws_bytes(moe_dtype dt, int N, int M_cap, int H, int I) {
  (void)N;
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  const size_t nTN = (size_t)(I + gg::BN - 1) / gg::BN;
  return align256((size_t)M_cap * 2 * I * es) + align256((size_t)M_cap * I * es) +
         align256((size_t)M_cap * H * es) + align256((size_t)M_cap * nTN * 4) + 256;
}

template <typename T>
static hipError_t layer_bwd_t(const void* dout, const void* x, const void* wg, const void* wu, const void* wd,
                              int H, int I, const moe_plan& p, const void* hcache, void* dx, void* dwg,
                              void* dwu, void* dwd, float* ds, void* ws, hipStream_t s) {
  const size_t es = sizeof(T);
  const int nTN = (I + gg::BN - 1) / gg::BN;
  char* w = (char*)ws;
  void* dh = w;
  w += align256((size_t)p.M_cap * 2 * I * es);
  void* aprime = w;
  w += align256((size_t)p.M_cap * I * es);
  void* dxe = w;
  w += align256((size_t)p.M_cap * H * es);
  float* dspart = (float*)w;

  gg::Args a{};
  a.x = x; a.wg = wg; a.wu = wu; a.wd = wd; a.dout = dout; a.hcache = hcache;
  a.counts = p.counts; a.offsets = p.offsets; a.row_token = p.row_token; a.row_w = p.row_w;
  a.E = p.E; a.H = H; a.I = I;
  const long long mt = (long long)(p.M_cap + gg::BM - 1) / gg::BM + p.E;
  hipError_t err;

  // dH epilogue kernel: dH = [dG | dU], A' = w A, dS partials
  a.out0 = dh; a.out1 = aprime; a.dspart = dspart;
  if ((err = run<T, gg::DH>(a, mt * nTN, s)) != hipSuccess) return err;
  if (p.M_cap > 0) {
    kernel_event(MOE_K_DS_REDUCE, 0, s);
    hipLaunchKernelGGL(gg::k_ds_reduce, dim3((p.M_cap + 255) / 256), dim3(256), 0, s, dspart, nTN, p.offsets, p.E,
                       p.row_pair, p.kind == MOE_PLAN_TOPK ? 1 : 0, p.M_cap, ds);
    kernel_event(MOE_K_DS_REDUCE, 1, s);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // dW_down = sum_r dOut[t]^T A'   (varlen-K)
  a.act = aprime; a.out0 = dwd; a.out1 = nullptr;
  if ((err = run<T, gg::DWD>(a, (long long)p.E * ((H + 127) / 128) * nTN, s)) != hipSuccess) return err;
  // dXe = dH [W_gate; W_up]   (varlen-M), then the unweighted combine to token order
  a.dh = dh; a.out0 = dxe;
  if ((err = run<T, gg::DX>(a, mt * ((H + gg::BN - 1) / gg::BN), s)) != hipSuccess) return err;
  kernel_event(MOE_K_DX_COMBINE, 0, s);
  err = launch_combine(sizeof(T) == 2 ? MOE_BF16 : MOE_F32, dxe, H, p, nullptr, dx, s);
  kernel_event(MOE_K_DX_COMBINE, 1, s);
  if (err != hipSuccess) return err;
  // dW_gate, dW_up = sum_r dH^T x[t]   (varlen-K)
  a.out0 = dwg; a.out1 = dwu;
  return run<T, gg::DW1>(a, (long long)p.E * ((2 * I + 127) / 128) * ((H + 127) / 128), s);
}

hipError_t launch_layer_bwd(moe_dtype dt, const void* dout, const void* x, const void* wg, const void* wu,
                            const void* wd, int H, int I, const moe_plan& p, const void* hcache, void* dx,
                            void* dwg, void* dwu, void* dwd, float* ds, void* ws, hipStream_t s) {
  if (dt == MOE_BF16)
    return layer_bwd_t<bf16_t>(dout, x, wg, wu, wd, H, I, p, hcache, dx, dwg, dwu, dwd, ds, ws, s);
  return layer_bwd_t<float>(dout, x, wg, wu, wd, H, I, p, hcache, dx, dwg, dwu, dwd, ds, ws, s);
}

}  // namespace moe
