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
#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace gg {

constexpr int BM = 128, BN = 128, NTHR = 256;


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

// ------------------------------------------------------------------ tile schedule
// A cursor is a position (tile, k-step) in this workgroup's sequence of tiles.
struct Cur {
  int it;     // persistent iteration that produced the tile
  int valid;  // 0 once past the last tile
  int e, roff, m0, n0, nt, mlen, K, nk, kt;
};

template <typename T, int KIND>
struct Sched {
  using TR = KindTraits<KIND>;
  static constexpr int BK = ElemCfg<T>::BK;
  const int* s_sched;  // LDS: varlen-M tile prefix [E+1]; varlen-K expert order [E]
  int total, G, per, xcd, slot, E, nN, nM;

  // K (reduction length) and the number of k-steps of a tile of expert e with `cnt` rows
  __device__ __forceinline__ void klen(const Args& a, int cnt, int& K, int& nk) const {
    switch (KIND) {
      case GATEUP: K = a.H; break;
      case DOWN: K = a.I; break;
      case DH: K = a.H; break;
      case DX: K = a.I; break;  // two segments (gate rows, then up rows) of ceil(I/BK) steps
      default: K = cnt; break;
    }
    nk = (K + BK - 1) / BK;
    if (KIND == DX) nk *= 2;
  }

  __device__ __forceinline__ void decode(const Args& a, Cur& c, int it) const {
    c.it = it;
    c.kt = 0;
    const long long tile_ll = (long long)it * G + (long long)xcd * per + slot;
    c.valid = tile_ll < (long long)total;
    if (!c.valid) {
      c.e = 0; c.roff = 0; c.m0 = 0; c.n0 = 0; c.nt = 0; c.mlen = 0; c.K = 0; c.nk = 0;
      return;
    }
    const int tile = (int)tile_ll;
    if constexpr (!TR::VK) {
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_sched[mid] <= tile) lo = mid; else hi = mid;
      }
      const int e = ufl(lo);
      const int cnt = a.counts[e];
      const int mtiles = (cnt + BM - 1) / BM;
      const int local = tile - ufl(s_sched[e]);
      const int mt = local % mtiles, nt = local / mtiles;
      c.e = e;
      c.roff = a.offsets[e];
      c.m0 = mt * BM;
      c.nt = nt;
      c.n0 = (KIND == GATEUP) ? nt * 64 : nt * BN;
      c.mlen = min(BM, cnt - c.m0);
      klen(a, cnt, c.K, c.nk);
    } else {
      const int per_e = nM * nN;
      const int rank = tile / per_e;
      const int local = tile - rank * per_e;
      const int e = ufl(s_sched[rank]);
      c.e = e;
      c.roff = a.offsets[e];
      c.m0 = (local / nN) * BM;
      c.nt = local % nN;
      c.n0 = c.nt * BN;
      c.mlen = BM;
      klen(a, a.counts[e], c.K, c.nk);
    }
  }
  // the next tile after c's tile (tiles without k-steps are skipped when skip_empty)
  __device__ __forceinline__ void next_tile(const Args& a, Cur& c, bool skip_empty) const {
    int it = c.it + 1;
    for (;;) {
      decode(a, c, it);
      if (!c.valid || !skip_empty || c.nk > 0) return;
      ++it;
    }
  }
};

// ------------------------------------------------------------------ operand addressing
// K-contiguous operands (LDS rows = operand rows): thread t loads 16-byte chunk t % 8 of rows
// t/8 + 32v (v = 0..3), so 8 consecutive lanes read one full 128-byte row segment.
__device__ __forceinline__ int kc_row(int v, int w, int lane) { return 8 * w + (lane >> 3) + 32 * v; }
__device__ __forceinline__ int kc_chunk(int v, int w, int lane) { return lane & 7; }

// MN-contiguous operands (k-rows x columns in memory): thread -> k-group kg = tid % KG
// (k-rows 4kg .. 4kg+3 of the step) and column chunk ch = tid / KG.

template <typename T, int KIND>
struct Ops {
  using TR = KindTraits<KIND>;
  using C = ElemCfg<T>;
  static constexpr int VEC = C::VEC, BK = C::BK, LDSW = C::LDSW, KG = BK / 4;
  static constexpr uint32_t ES = sizeof(T);

  // per-tile state of the load cursor
  rsrc_t ra, rb0, rb1, rrt;
  uint32_t rowA[4];  // K-contiguous A: byte offset of each thread row (OOB if masked)
  uint32_t rowB[4];  // K-contiguous B
  int segB[4];       // GATEUP: 0 = gate rows, 1 = up rows (uniform per wavefront and load)

  __device__ __forceinline__ void setup_tile(const Args& a, const Cur& L, const int (&tok)[4], int w, int lane) {
    const int H = a.H, I = a.I;
    rrt = mkr(a.row_token, 4LL * (long long)a.M_cap);
    switch (KIND) {
      case GATEUP:
        ra = mkr(a.x, (long long)a.N * H * ES);
        rb0 = mkr((const T*)a.wg + (size_t)L.e * I * H, (long long)I * H * ES);
        rb1 = mkr((const T*)a.wu + (size_t)L.e * I * H, (long long)I * H * ES);
        break;
      case DOWN:
        ra = mkr(a.act, (long long)a.M_cap * I * ES);
        rb0 = rb1 = mkr((const T*)a.wd + (size_t)L.e * H * I, (long long)H * I * ES);
        break;
      case DH:
        ra = mkr(a.dout, (long long)a.N * H * ES);
        rb0 = rb1 = mkr((const T*)a.wd + (size_t)L.e * H * I, (long long)H * I * ES);
        break;
      case DX:
        ra = mkr(a.dh, (long long)a.M_cap * 2 * I * ES);
        rb0 = mkr((const T*)a.wg + (size_t)L.e * I * H, (long long)I * H * ES);
        rb1 = mkr((const T*)a.wu + (size_t)L.e * I * H, (long long)I * H * ES);
        break;
      case DWD:
        ra = mkr(a.dout, (long long)a.N * H * ES);
        rb0 = rb1 = mkr(a.act, (long long)a.M_cap * I * ES);
        break;
      default:  // DW1
        ra = mkr(a.dh, (long long)a.M_cap * 2 * I * ES);
        rb0 = rb1 = mkr(a.x, (long long)a.N * H * ES);
        break;
    }
    if constexpr (TR::A_KC) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = kc_row(v, w, lane);
        const bool ok = L.valid && row < L.mlen;
        const int r = L.roff + L.m0 + row;
        uint32_t off = OOB;
        if (ok) {
          switch (KIND) {
            case GATEUP:
            case DH: off = (uint32_t)tok[v] * (uint32_t)(H * ES); break;
            case DOWN: off = (uint32_t)r * (uint32_t)(I * ES); break;
            default: off = (uint32_t)r * (uint32_t)(2 * I * ES); break;  // DX
          }
        }
        rowA[v] = off;
      }
    }
    if constexpr (TR::B_KC) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = kc_row(v, w, lane);
        uint32_t off = OOB;
        if (KIND == GATEUP) {
          segB[v] = v & 1;  // = (n >> 5) & 1: rows 32v .. 32v+31 of the tile
          const int i = L.n0 + (n >> 6) * 32 + (n & 31);
          if (L.valid && i < I) off = (uint32_t)i * (uint32_t)(H * ES);
        } else {  // DOWN
          segB[v] = 0;
          const int h = L.n0 + n;
          if (L.valid && h < H) off = (uint32_t)h * (uint32_t)(I * ES);
        }
        rowB[v] = off;
      }
    }
  }

  // row tokens of the K-contiguous gathered rows of tile c (GATEUP, DH)
  __device__ __forceinline__ static void tile_tokens(const Args& a, rsrc_t rrt, const Cur& c, int (&tok)[4], int w, int lane) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = kc_row(v, w, lane);
      const bool ok = c.valid && row < c.mlen;
      tok[v] = bld4(rrt, ok ? (uint32_t)(c.roff + c.m0 + row) * 4u : OOB);
    }
  }
  // row tokens of the k-rows of step (c, kt) for varlen-K gathered operands (DWD, DW1)
  __device__ __forceinline__ static void step_tokens(rsrc_t rrt, const Cur& c, int kt, int (&tok)[4], int tid) {
    const int kg = tid % KG;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kk = kt * BK + 4 * kg + q;
      const bool ok = c.valid && kt < c.nk && kk < c.K;
      tok[q] = bld4(rrt, ok ? (uint32_t)(c.roff + kk) * 4u : OOB);
    }
  }

  // issue the 8 loads of step (L, L.kt): R[0..3] A, R[4..7] B
  __device__ __forceinline__ void issue(const Args& a, const Cur& L, uint4 (&R)[8], const int (&tok)[4], int w, int lane,
                        int tid) const {
    const int H = a.H, I = a.I;
    const bool live = L.valid && L.kt < L.nk;
    if constexpr (TR::A_KC) {
      int kofs, klim;
      if (KIND == DX) {
        const int half = L.nk / 2;
        const int seg = L.kt >= half;
        kofs = seg * I + (L.kt - seg * half) * BK;
        klim = seg * I + I;
      } else {
        kofs = L.kt * BK;
        klim = L.K;
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int k = kofs + kc_chunk(v, w, lane) * VEC;
        const uint32_t off = (live && rowA[v] != OOB && k < klim) ? rowA[v] + (uint32_t)k * ES : OOB;
        R[v] = bld16(ra, off);
      }
    } else {  // MN-contiguous A (DWD: gathered dout rows, DW1: dH rows)
      const int kg = tid % KG, ch = tid / KG;
      const int col = L.m0 + ch * VEC;
      const int lim = (KIND == DWD) ? H : 2 * I;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = L.kt * BK + 4 * kg + q;
        const bool ok = live && kk < L.K && col < lim;
        uint32_t off = OOB;
        if (ok) {
          if (KIND == DWD) off = ((uint32_t)tok[q] * (uint32_t)H + (uint32_t)col) * ES;
          else off = ((uint32_t)(L.roff + kk) * (uint32_t)(2 * I) + (uint32_t)col) * ES;
        }
        R[q] = bld16(ra, off);
      }
    }
    if constexpr (TR::B_KC) {
      const int k = L.kt * BK;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kk = k + kc_chunk(v, w, lane) * VEC;
        const uint32_t off = (live && rowB[v] != OOB && kk < L.K) ? rowB[v] + (uint32_t)kk * ES : OOB;
        R[4 + v] = bld16(segB[v] ? rb1 : rb0, off);
      }
    } else {  // MN-contiguous B
      const int kg = tid % KG, ch = tid / KG;
      const int col = L.n0 + ch * VEC;
      int seg = 0, kbase = L.kt * BK, klim = L.K;
      if (KIND == DX) {
        const int half = L.nk / 2;
        seg = L.kt >= half;
        kbase = (L.kt - seg * half) * BK;
        klim = I;
      }
      const int lim = (KIND == DH || KIND == DWD) ? I : H;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = kbase + 4 * kg + q;
        const bool ok = live && kk < klim && col < lim;
        uint32_t off = OOB;
        if (ok) {
          switch (KIND) {
            case DH: off = ((uint32_t)kk * (uint32_t)I + (uint32_t)col) * ES; break;
            case DX: off = ((uint32_t)kk * (uint32_t)H + (uint32_t)col) * ES; break;
            case DWD: off = ((uint32_t)(L.roff + kk) * (uint32_t)I + (uint32_t)col) * ES; break;
            default: off = ((uint32_t)tok[q] * (uint32_t)H + (uint32_t)col) * ES; break;  // DW1
          }
        }
        R[4 + q] = bld16(seg ? rb1 : rb0, off);
      }
    }
  }
};

// ------------------------------------------------------------------ LDS staging
// A stage holds 256 rows (A rows 0..127, B rows 128..255) of 128 bytes, K-contiguous: eight
// 16-byte chunks per row.  Chunk c of row r sits at position c ^ ((r >> 1) & 7).  Measured on
// gfx950 with the LDS bank-conflict counter, this placement is conflict-free for the full-row
// 16-byte writes, the transposing 8-byte writes and the 16-row (and 32-row) fragment reads,
// whereas 16-byte row padding and the swizzle c ^ (r & 7) ^ ((r >> 3) & 1) double the read time.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_byte(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

template <typename T>
__device__ __forceinline__ void sstore_kc(char* lds, const uint4* r, int w, int lane) {
#pragma unroll
  for (int v = 0; v < 4; ++v)
    *reinterpret_cast<uint4*>(lds + lds_byte(kc_row(v, w, lane), kc_chunk(v, w, lane))) = r[v];
}
// 4 k-rows x VEC columns in registers -> VEC LDS rows of 4 consecutive k values.  Threads of
// odd column chunks visit their rows in the order j ^ 1, so the two chunks written by one
// instruction land on rows of different parity (different bank halves).
template <typename T>
__device__ __forceinline__ void sstore_mn(char* lds, const uint4* r, int tid);
template <>
__device__ __forceinline__ void sstore_mn<bf16_t>(char* lds, const uint4* r, int tid) {
  const int kg = tid & 15, ch = tid >> 4;
  const uint32_t* q0 = reinterpret_cast<const uint32_t*>(&r[0]);
  const uint32_t* q1 = reinterpret_cast<const uint32_t*>(&r[1]);
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(&r[2]);
  const uint32_t* q3 = reinterpret_cast<const uint32_t*>(&r[3]);
  const int flip = ch & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int jj = j ^ flip;
    const int h = jj >> 1;
    uint2 o;
    if (jj & 1) {
      o.x = (q0[h] >> 16) | (q1[h] & 0xFFFF0000u);
      o.y = (q2[h] >> 16) | (q3[h] & 0xFFFF0000u);
    } else {
      o.x = (q0[h] & 0xFFFFu) | (q1[h] << 16);
      o.y = (q2[h] & 0xFFFFu) | (q3[h] << 16);
    }
    *reinterpret_cast<uint2*>(lds + lds_byte(ch * 8 + jj, kg >> 1) + ((kg & 1) << 3)) = o;
  }
}
template <>
__device__ __forceinline__ void sstore_mn<float>(char* lds, const uint4* r, int tid) {
  const int kg = tid & 7, ch = tid >> 3;
  const int flip = ch & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int jj = j ^ flip;
    uint4 o;
    o.x = reinterpret_cast<const uint32_t*>(&r[0])[jj];
    o.y = reinterpret_cast<const uint32_t*>(&r[1])[jj];
    o.z = reinterpret_cast<const uint32_t*>(&r[2])[jj];
    o.w = reinterpret_cast<const uint32_t*>(&r[3])[jj];
    *reinterpret_cast<uint4*>(lds + lds_byte(ch * 4 + jj, kg)) = o;
  }
}

// ------------------------------------------------------------------ epilogues
template <typename T, int KIND>
__device__ __forceinline__ void epilogue(const Args& a, const Cur& c, f32x4 (&acc)[4][4], float* s_red, int wm, int wn,
                                         int lane) {
  const int mrow = wm * 64 + (lane & 15);
  const int ncol = wn * 64 + 4 * (lane >> 4);
  if constexpr (KIND == GATEUP) {
    T* hc = (T*)a.out0;
    T* ac = (T*)a.out1;
    const int I = a.I;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mrow + i * 16;
      if (m >= c.mlen) continue;
      const size_t r = (size_t)(c.roff + c.m0 + m);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ii = c.n0 + wn * 32 + j * 16 + 4 * (lane >> 4);
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
      if (m >= c.mlen) continue;
      const size_t r = (size_t)(c.roff + c.m0 + m);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = c.n0 + ncol + j * 16;
        if (h >= a.H) continue;
        store4(out + r * a.H + h, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  } else if constexpr (KIND == DH) {
    T* dh = (T*)a.out0;
    T* ap = (T*)a.out1;
    const int I = a.I;
    constexpr uint32_t ES = sizeof(T);
    const rsrc_t rh = mkr(a.hcache, (long long)a.M_cap * 2 * I * ES);
    const rsrc_t rw = mkr(a.row_w, 4LL * a.M_cap);
    float dsum[4] = {0.f, 0.f, 0.f, 0.f};
    // two halves of the wavefront's rows: all loads of a half are issued before any use,
    // masked rows and columns read zeros (out-of-range buffer offsets)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 graw[2][4], uraw[2][4];
      float wrow[2];
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = half * 2 + ii;
        const int m = mrow + i * 16;
        const bool okr = m < c.mlen;
        const uint32_t r = (uint32_t)(c.roff + c.m0 + m);
        wrow[ii] = __int_as_float(bld4(rw, okr ? r * 4u : OOB));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = c.n0 + ncol + j * 16;
          const bool ok = okr && col < I;
          const uint32_t og = ok ? (r * (uint32_t)(2 * I) + (uint32_t)col) * ES : OOB;
          const uint32_t ou = ok ? og + (uint32_t)I * ES : OOB;
          if constexpr (sizeof(T) == 2) {
            graw[ii][j] = make_uint4(0, 0, 0, 0);
            uraw[ii][j] = make_uint4(0, 0, 0, 0);
            const auto g2 = __builtin_amdgcn_raw_buffer_load_b64(rh, og, 0, 0);
            const auto u2 = __builtin_amdgcn_raw_buffer_load_b64(rh, ou, 0, 0);
            graw[ii][j].x = g2[0]; graw[ii][j].y = g2[1];
            uraw[ii][j].x = u2[0]; uraw[ii][j].y = u2[1];
          } else {
            graw[ii][j] = bld16(rh, og);
            uraw[ii][j] = bld16(rh, ou);
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = half * 2 + ii;
        const int m = mrow + i * 16;
        const bool okr = m < c.mlen;
        const size_t r = (size_t)(c.roff + c.m0 + m);
        const float w = wrow[ii];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = c.n0 + ncol + j * 16;
          float g[4], u[4], dg[4], du[4], av[4];
          if constexpr (sizeof(T) == 2) {
            g[0] = __uint_as_float(graw[ii][j].x << 16); g[1] = __uint_as_float(graw[ii][j].x & 0xFFFF0000u);
            g[2] = __uint_as_float(graw[ii][j].y << 16); g[3] = __uint_as_float(graw[ii][j].y & 0xFFFF0000u);
            u[0] = __uint_as_float(uraw[ii][j].x << 16); u[1] = __uint_as_float(uraw[ii][j].x & 0xFFFF0000u);
            u[2] = __uint_as_float(uraw[ii][j].y << 16); u[3] = __uint_as_float(uraw[ii][j].y & 0xFFFF0000u);
          } else {
            g[0] = __uint_as_float(graw[ii][j].x); g[1] = __uint_as_float(graw[ii][j].y);
            g[2] = __uint_as_float(graw[ii][j].z); g[3] = __uint_as_float(graw[ii][j].w);
            u[0] = __uint_as_float(uraw[ii][j].x); u[1] = __uint_as_float(uraw[ii][j].y);
            u[2] = __uint_as_float(uraw[ii][j].z); u[3] = __uint_as_float(uraw[ii][j].w);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float sg = sigmoidf_(g[v]);
            const float silu = g[v] * sg;
            const float A = silu * u[v];
            const float dap = acc[i][j][v];
            dsum[i] += dap * A;  // masked rows/columns hold zeros in both factors
            const float da = w * dap;
            dg[v] = da * u[v] * sg * (1.0f + g[v] * (1.0f - sg));
            du[v] = da * silu;
            av[v] = w * A;
          }
          if (okr && col < I) {
            store4(dh + r * (2 * I) + col, dg[0], dg[1], dg[2], dg[3]);
            store4(dh + r * (2 * I) + I + col, du[0], du[1], du[2], du[3]);
            store4(ap + r * I + col, av[0], av[1], av[2], av[3]);
          }
        }
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
        if (m < c.mlen) a.dspart[(size_t)(c.roff + c.m0 + m) * nTN + c.nt] = dsum[i] + s_red[m];
      }
    }
    __syncthreads();
  } else if constexpr (KIND == DWD) {
    T* dw = (T*)a.out0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = c.m0 + mrow + i * 16;
      if (h >= a.H) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ii = c.n0 + ncol + j * 16;
        if (ii >= a.I) continue;
        store4(dw + ((size_t)c.e * a.H + h) * a.I + ii, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  } else {  // DW1
    T* dwg = (T*)a.out0;
    T* dwu = (T*)a.out1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ip = c.m0 + mrow + i * 16;
      if (ip >= 2 * a.I) continue;
      T* base = ip < a.I ? dwg + ((size_t)c.e * a.I + ip) * a.H : dwu + ((size_t)c.e * a.I + (ip - a.I)) * a.H;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = c.n0 + ncol + j * 16;
        if (h >= a.H) continue;
        store4(base + h, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
  }
}

// ------------------------------------------------------------------ the kernel
template <typename T, int KIND>
__global__ __launch_bounds__(NTHR, 2) void k_grouped_gemm(Args a, const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ offsets) {
  // The expert counts and offsets are read-only here; passing them as restrict kernel
  // arguments lets the compiler fetch them with scalar loads, which do not wait behind the
  // vector-memory prefetch queue.
  a.counts = counts;
  a.offsets = offsets;
  using C = ElemCfg<T>;
  using TR = KindTraits<KIND>;
  using O = Ops<T, KIND>;
  constexpr int BK = C::BK, LDSW = C::LDSW, KPL = C::KPL;
  constexpr int KSTEP = 4 * KPL;
  constexpr int STAGE = (BM + BN) * 128;  // bytes
  constexpr bool GATHER_KC = (KIND == GATEUP || KIND == DH);   // per-tile row tokens
  constexpr bool GATHER_MN = (KIND == DWD || KIND == DW1);     // per-step row tokens

  __shared__ __attribute__((aligned(16))) char s_tile[2 * STAGE];
  __shared__ int s_sched[1025];
  __shared__ int s_wave[5];
  __shared__ float s_red[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = ufl(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int E = a.E;

  Sched<T, KIND> S;
  S.s_sched = s_sched;
  S.E = E;
  S.G = gridDim.x;
  S.per = S.G >> 3;
  S.xcd = blockIdx.x & 7;
  S.slot = blockIdx.x >> 3;
  switch (KIND) {
    case GATEUP: S.nN = (a.I + 63) / 64; break;
    case DOWN: case DX: case DW1: S.nN = (a.H + BN - 1) / BN; break;
    default: S.nN = (a.I + BN - 1) / BN; break;  // DH, DWD
  }
  S.nM = KIND == DWD ? (a.H + BM - 1) / BM : (2 * a.I + BM - 1) / BM;

  // ---- tile space from the device-resident counts ----
  if constexpr (!TR::VK) {
    int loc[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      loc[q] = e < E ? ((a.counts[e] + BM - 1) / BM) * S.nN : 0;
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
      if (e < E) s_sched[e] = run;
      run += loc[q];
    }
    if (tid == 0) s_sched[E] = s_wave[4];
    S.total = ufl(s_wave[4]);
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
    S.total = E * S.nM * S.nN;
  }

  // ---- cursors: L = next step to load, Lx = the tile after L's, C = step being computed ----
  Cur L, Lx, Cc;
  S.decode(a, L, 0);
  if (L.valid && L.nk == 0) S.next_tile(a, L, true);
  Lx = L;
  S.next_tile(a, Lx, true);
  S.decode(a, Cc, 0);

  O ops;
  int tokA[4] = {0, 0, 0, 0}, tokN[4] = {0, 0, 0, 0};  // per-tile gathered rows (current / next tile)
  int rtE[4] = {0, 0, 0, 0}, rtO[4] = {0, 0, 0, 0};    // per-step gathered rows (even / odd steps)
  const rsrc_t rrt = mkr(a.row_token, 4LL * (long long)a.M_cap);
  if constexpr (GATHER_KC) {
    O::tile_tokens(a, rrt, L, tokA, wave, lane);
    O::tile_tokens(a, rrt, Lx, tokN, wave, lane);
  }
  ops.setup_tile(a, L, tokA, wave, lane);

  // advance L by one step; at a tile change the next tile's state becomes current
  auto advance_L = [&]() __attribute__((always_inline)) {
    if (L.valid && L.kt + 1 < L.nk) {
      ++L.kt;
      return;
    }
    L = Lx;
    Lx = L;
    S.next_tile(a, Lx, true);
    if constexpr (GATHER_KC) {
#pragma unroll
      for (int v = 0; v < 4; ++v) tokA[v] = tokN[v];
      O::tile_tokens(a, rrt, Lx, tokN, wave, lane);
    }
    ops.setup_tile(a, L, tokA, wave, lane);
  };
  // position one step after L (for the per-step token prefetch)
  auto peek_next = [&](Cur& p, int& kt) __attribute__((always_inline)) {
    if (L.valid && L.kt + 1 < L.nk) {
      p = L;
      kt = L.kt + 1;
    } else {
      p = Lx;
      kt = 0;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tiles without k-steps at the start of the sequence (empty experts, varlen-K only)
  if constexpr (TR::VK) {
    while (Cc.valid && Cc.nk == 0) {
      epilogue<T, KIND>(a, Cc, acc, s_red, wm, wn, lane);
      S.next_tile(a, Cc, false);
    }
  }
  if (!Cc.valid) return;

  // ---- prologue: steps 0 and 1 in flight, step 0 in LDS ----
  uint4 R0[8], R1[8];
  if constexpr (GATHER_MN) {
    O::step_tokens(rrt, L, L.kt, rtE, tid);
    Cur p;
    int pk;
    peek_next(p, pk);
    O::step_tokens(rrt, p, pk, rtO, tid);
  }
  ops.issue(a, L, R0, rtE, wave, lane, tid);
  advance_L();
  if constexpr (GATHER_MN) {
    Cur p;
    int pk;
    peek_next(p, pk);
    O::step_tokens(rrt, p, pk, rtE, tid);
  }
  ops.issue(a, L, R1, rtO, wave, lane, tid);
  advance_L();
  {
    char* la = s_tile;
    if constexpr (TR::A_KC) sstore_kc<T>(la, R0, wave, lane); else sstore_mn<T>(la, R0, tid);
    if constexpr (TR::B_KC) sstore_kc<T>(la + BM * 128, R0 + 4, wave, lane); else sstore_mn<T>(la + BM * 128, R0 + 4, tid);
  }
  __syncthreads();

  // one pipeline step: prefetch step s+2 into Rp, compute stage P, store Rq (step s+1) into stage 1-P
  auto step = [&](auto PP, uint4 (&Rp)[8], uint4 (&Rq)[8], int (&rt_use)[4], int (&rt_fill)[4])
                  __attribute__((always_inline)) {
    constexpr int P = decltype(PP)::value;
    if constexpr (GATHER_MN) {
      Cur p;
      int pk;
      peek_next(p, pk);
      O::step_tokens(rrt, p, pk, rt_fill, tid);  // tokens of step s+3, issued before the data of s+2
    }
    ops.issue(a, L, Rp, rt_use, wave, lane, tid);
    advance_L();

    // fragment rows: A rows wm*64 + i*16 + (lane & 15), B rows 128 + wn*64 + j*16 + (lane & 15);
    // the swizzle depends on row & 15 = lane & 15 only
    const char* sa = s_tile + P * STAGE + (wm * 64 + (lane & 15)) * 128;
    const char* sb = s_tile + P * STAGE + (BM + wn * 64 + (lane & 15)) * 128;
    const int fsw = swz(lane & 15);
    // a wavefront whose 64 rows all lie past the tile's valid rows has no work this step
    if (Cc.mlen > wm * 64) {
#pragma unroll
      for (int ks = 0; ks < BK / KSTEP; ++ks) {
        // byte offset of this lane's k values inside its row for k-step ks
        const int kbyte = (ks * KSTEP + (lane >> 4) * KPL) * (int)sizeof(T);
        const int off = (((kbyte >> 4) ^ fsw) << 4) + (kbyte & 15);
        typename C::frag_t fa[4], fb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          fb[j] = *reinterpret_cast<const typename C::frag_t*>(sb + j * 16 * 128 + off);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fa[i] = *reinterpret_cast<const typename C::frag_t*>(sa + i * 16 * 128 + off);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mma(fb[j], fa[i], acc[i][j]);
      }
    }
    {
      char* la = s_tile + (1 - P) * STAGE;
      if constexpr (TR::A_KC) sstore_kc<T>(la, Rq, wave, lane); else sstore_mn<T>(la, Rq, tid);
      if constexpr (TR::B_KC) sstore_kc<T>(la + BM * 128, Rq + 4, wave, lane);
      else sstore_mn<T>(la + BM * 128, Rq + 4, tid);
    }
    __syncthreads();
    // advance the compute cursor; finish the tile after its last step
    if (Cc.kt + 1 < Cc.nk) {
      ++Cc.kt;
    } else {
      epilogue<T, KIND>(a, Cc, acc, s_red, wm, wn, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      S.next_tile(a, Cc, false);
      if constexpr (TR::VK) {
        while (Cc.valid && Cc.nk == 0) {
          epilogue<T, KIND>(a, Cc, acc, s_red, wm, wn, lane);
          S.next_tile(a, Cc, false);
        }
      }
    }
  };

  for (;;) {
    step(std::integral_constant<int, 0>{}, R0, R1, rtE, rtO);
    if (!Cc.valid) break;
    step(std::integral_constant<int, 1>{}, R1, R0, rtO, rtE);
    if (!Cc.valid) break;
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
  hipLaunchKernelGGL((gg::k_grouped_gemm<T, KIND>), dim3(persistent_grid(max_tiles)), dim3(gg::NTHR), 0, s, a,
                     a.counts, a.offsets);
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
  a.E = p.E; a.H = H; a.I = I; a.N = p.N; a.M_cap = p.M_cap;
  void* act = ws;
  a.out0 = hcache; a.out1 = act;
  hipError_t err;
  if constexpr (std::is_same<T, bf16_t>::value) {
    const long long mt = (long long)(p.M_cap + 255) / 256 + p.E;
    if ((err = run_gemm_bf16<gg::GATEUP>(a, mt * ((I + 127) / 128), s)) != hipSuccess) return err;
    a.act = act; a.out0 = y; a.out1 = nullptr;
    return run_gemm_bf16<gg::DOWN>(a, mt * ((H + 255) / 256), s);
  } else {
    const long long mt = (long long)(p.M_cap + gg::BM - 1) / gg::BM + p.E;
    if ((err = run<T, gg::GATEUP>(a, mt * ((I + 63) / 64), s)) != hipSuccess) return err;
    a.act = act; a.out0 = y; a.out1 = nullptr;
    return run<T, gg::DOWN>(a, mt * ((H + gg::BN - 1) / gg::BN), s);
  }
}

hipError_t launch_gemm_fwd(moe_dtype dt, const void* x, const void* wg, const void* wu, const void* wd, int H,
                           int I, const moe_plan& p, void* hcache, void* y, void* ws, hipStream_t s) {
  if (dt == MOE_BF16) return gemm_fwd_t<bf16_t>(x, wg, wu, wd, H, I, p, hcache, y, ws, s);
  return gemm_fwd_t<float>(x, wg, wu, wd, H, I, p, hcache, y, ws, s);
}

// MX-FP8 forward: the workspace holds A's codes [M_cap, I] and its scale codes [M_cap, KS(I)].
size_t gemm_fwd_mxfp8_ws_bytes(int M_cap, int I) {
  const size_t ksi = 4 * (size_t)((I + 127) / 128);
  return align256((size_t)M_cap * I) + align256((size_t)M_cap * ksi) + 256;
}

hipError_t launch_gemm_fwd_mxfp8(const void* xq, const void* xs, const void* wgq, const void* wgs, const void* wuq,
                                 const void* wus, const void* wdq, const void* wds, int H, int I, const moe_plan& p,
                                 void* hcache, void* y, void* ws, hipStream_t s) {
  gg::Args a{};
  a.x = xq; a.xs = xs; a.wg = wgq; a.wgs = wgs; a.wu = wuq; a.wus = wus; a.wd = wdq; a.wds = wds;
  a.counts = p.counts; a.offsets = p.offsets; a.row_token = p.row_token; a.row_w = p.row_w;
  a.E = p.E; a.H = H; a.I = I; a.N = p.N; a.M_cap = p.M_cap;
  char* w = (char*)ws;
  void* aq = w;
  void* as = w + align256((size_t)p.M_cap * I);
  a.out0 = hcache; a.out1 = aq; a.out2 = as;
  const long long mt = (long long)(p.M_cap + 255) / 256 + p.E;
  hipError_t err = run_gemm_bf16<gg::GATEUP8>(a, mt * ((I + 127) / 128), s);
  if (err != hipSuccess) return err;
  a.act = aq; a.acts = as; a.out0 = y; a.out1 = nullptr; a.out2 = nullptr;
  return run_gemm_bf16<gg::DOWN8>(a, mt * ((H + 255) / 256), s);
}

size_t layer_bwd_ws_bytes(moe_dtype dt, int N, int M_cap, int H, int I) {
  (void)N;
  const size_t es = dt == MOE_BF16 ? 2 : 4;
  // the dH kernel's dS partials per row: fp32, one per 128-column N-tile; bf16, one per
  // wavefront half (128 columns) of each 256-column N-tile
  const size_t nP = dt == MOE_BF16 ? 2 * (size_t)((I + 255) / 256) : (size_t)((I + gg::BN - 1) / gg::BN);
  const size_t part = (size_t)M_cap * nP * 4;
  return align256((size_t)M_cap * 2 * I * es) + align256((size_t)M_cap * I * es) +
         align256((size_t)M_cap * H * es) + align256(part) + 256;
}

// MX-FP8 dX product: moe_layer_bwd's workspace, then the scale codes of the quantized dH
// [M_cap, KS(2I)] (its codes [M_cap, 2I] reuse the A' region, free once dW_down has run).
size_t layer_bwd_mxfp8_ws_bytes(int N, int M_cap, int H, int I) {
  return layer_bwd_ws_bytes(MOE_BF16, N, M_cap, H, I) + align256((size_t)M_cap * 4 * ((2 * I + 127) / 128));
}

// wtq / wts: the quantized [W_gate^T | W_up^T] of every expert for a dX product on MX-FP8
// operands (bf16 layers only), or NULL for the bf16 product.
template <typename T>
static hipError_t layer_bwd_t(const void* dout, const void* x, const void* wg, const void* wu, const void* wd,
                              int H, int I, const moe_plan& p, const void* hcache, void* dx, void* dwg,
                              void* dwu, void* dwd, float* ds, void* ws, hipStream_t s, const void* wtq = nullptr,
                              const void* wts = nullptr) {
  const size_t es = sizeof(T);
  constexpr bool BF = std::is_same<T, bf16_t>::value;
  const int tn = BF ? 256 : gg::BN;  // N-tile width of the dH kernel
  const int nTN = (I + tn - 1) / tn;
  const int nP = BF ? 2 * nTN : nTN;  // dS partials per row (bf16: one per 128-column half tile)
  char* w = (char*)ws;
  void* dh = w;
  w += align256((size_t)p.M_cap * 2 * I * es);
  void* aprime = w;
  w += align256((size_t)p.M_cap * I * es);
  void* dxe = w;
  w += align256((size_t)p.M_cap * H * es);
  float* dspart = (float*)w;  // dS partials [M_cap, nP]
  w += align256((size_t)p.M_cap * nP * 4);

  gg::Args a{};
  a.x = x; a.wg = wg; a.wu = wu; a.wd = wd; a.dout = dout; a.hcache = hcache;
  a.counts = p.counts; a.offsets = p.offsets; a.row_token = p.row_token; a.row_w = p.row_w;
  a.E = p.E; a.H = H; a.I = I; a.N = p.N; a.M_cap = p.M_cap;
  const int tm = BF ? 256 : gg::BM;
  const long long mt = (long long)(p.M_cap + tm - 1) / tm + p.E;
  // the launch of one grouped GEMM: the bf16 kernel or the fp32 one
  auto launch = [&](auto kind, long long tiles) -> hipError_t {
    constexpr int K = decltype(kind)::value;
    if constexpr (BF) return run_gemm_bf16<K>(a, tiles, s);
    else return run<T, K>(a, tiles, s);
  };
  using KDH = std::integral_constant<int, gg::DH>;
  using KDWD = std::integral_constant<int, gg::DWD>;
  using KDX = std::integral_constant<int, gg::DX>;
  using KDW1 = std::integral_constant<int, gg::DW1>;
  hipError_t err;

  // dA' = dOut[t] W_down^T (varlen-M GEMM) with the dSwiGLU epilogue: dH = [dG | dU],
  // A' = w A and the dS partials (their ordered sum runs in the dX combine below)
  a.out0 = dh; a.out1 = aprime; a.dspart = dspart;
  if ((err = launch(KDH{}, mt * nTN)) != hipSuccess) return err;
  // The two weight-gradient kernels run first and dX last.  The bf16 kernels store their dW
  // (805 MB in all at the headline shape) with the non-temporal policy, since no later kernel
  // of the step reads it; of the orders measured with those stores this one is the fastest
  // (with dW_g/u last, the write-back of its output had slowed the next step's gate/up GEMM).
  // dW_down = sum_r dOut[t]^T A'   (varlen-K)
  a.act = aprime; a.out0 = dwd; a.out1 = nullptr;
  if ((err = launch(KDWD{}, (long long)p.E * ((H + tm - 1) / tm) * nTN)) != hipSuccess) return err;
  // dW_gate, dW_up = sum_r dH^T x[t]   (varlen-K)
  a.dh = dh; a.out0 = dwg; a.out1 = dwu;
  const long long mtw = BF ? 2LL * ((I + 255) / 256) : (2LL * I + 127) / 128;
  if ((err = launch(KDW1{}, (long long)p.E * mtw * ((H + tn - 1) / tn))) != hipSuccess) return err;
  // dXe = dH [W_gate; W_up]   (varlen-M), then the unweighted combine to token order
  a.out0 = dxe; a.out1 = nullptr;
  if (BF && wtq != nullptr) {
    // on MX-FP8 operands: dH quantized along its 2I values (codes into the A' region, scale
    // codes after the workspace's other parts), then the product out[m][h] = sum_k dH~[m][k]
    // W~^T[e][h][k] as DOWN8's GEMM with K = 2I
    uint8_t* dhq = static_cast<uint8_t*>(aprime);
    uint8_t* dhs = reinterpret_cast<uint8_t*>(w);
    kernel_event(MOE_K_QUANT, 0, s);
    err = launch_quant_mxfp8(MOE_BF16, dh, p.M_cap, 2 * I, dhq, dhs, s);
    kernel_event(MOE_K_QUANT, 1, s);
    if (err != hipSuccess) return err;
    gg::Args a8 = a;
    a8.act = dhq; a8.acts = dhs; a8.wd = wtq; a8.wds = wts; a8.out0 = dxe; a8.out1 = nullptr;
    a8.I = 2 * I;
    if ((err = run_gemm_bf16<gg::DX8>(a8, mt * ((H + tn - 1) / tn), s)) != hipSuccess) return err;
  } else if ((err = launch(KDX{}, mt * ((H + tn - 1) / tn))) != hipSuccess) {
    return err;
  }
  kernel_event(MOE_K_DX_COMBINE, 0, s);
  err = launch_combine(sizeof(T) == 2 ? MOE_BF16 : MOE_F32, dxe, H, p, nullptr, dx, s, dspart, nP, ds);
  kernel_event(MOE_K_DX_COMBINE, 1, s);
  return err;
}

hipError_t launch_layer_bwd_mxfp8(const void* dout, const void* x, const void* wg, const void* wu, const void* wd,
                                  const void* wtq, const void* wts, int H, int I, const moe_plan& p,
                                  const void* hcache, void* dx, void* dwg, void* dwu, void* dwd, float* ds, void* ws,
                                  hipStream_t s) {
  return layer_bwd_t<bf16_t>(dout, x, wg, wu, wd, H, I, p, hcache, dx, dwg, dwu, dwd, ds, ws, s, wtq, wts);
}

hipError_t launch_layer_bwd(moe_dtype dt, const void* dout, const void* x, const void* wg, const void* wu,
                            const void* wd, int H, int I, const moe_plan& p, const void* hcache, void* dx,
                            void* dwg, void* dwu, void* dwd, float* ds, void* ws, hipStream_t s) {
  if (dt == MOE_BF16)
    return layer_bwd_t<bf16_t>(dout, x, wg, wu, wd, H, I, p, hcache, dx, dwg, dwu, dwd, ds, ws, s);
  return layer_bwd_t<float>(dout, x, wg, wu, wd, H, I, p, hcache, dx, dwg, dwu, dwd, ds, ws, s);
}

}  // namespace moe
