// gemm_bf16.hip -- the bf16 grouped GEMMs of the layer (forward and backward) for gfx950.
//
// Pages cited (by title, then section):
//   [GG] "DeepSeek 계열 MoE 학습 가속: Python expert loop → grouped GEMM",
//        "무엇이 필요한가 — Variable-M batched matmul" (one launch over ragged expert groups)
//        and "적용" step (6) (gate, up and down share one set of group sizes)
//   [SM] "SonicMoE: IO·타일 인식 최적화로 MoE 학습 가속하기": "3 기여 ①" (cache [G|U] only;
//        dS = <dA', A> without Y), "4 기여 ②" (varlen-M and varlen-K grouped GEMMs),
//        "4.1 Gather 융합" (the token gather happens inside the operand load, backward
//        included), "4.2 Epilogue 융합" (SwiGLU, dSwiGLU, dS and A' in the epilogue),
//        "4.3 MMA ↔ IO 오버랩" (hide the loads and the heavy epilogue behind the MMAs),
//        "7 한계 & 의의" (no atomic reductions)
//
// Design:
//  * One workgroup of 512 threads (8 wavefronts, 4 along M x 2 along N) per compute unit
//    owns a (64 MI) x 256 output tile (MI = 5 for the varlen-M kinds, so that a group of up
//    to 320 rows is one M-tile; MI = 4 for the varlen-K kinds); wavefront (wm, wn) computes
//    the 16-row blocks 16(4i + wm), i < MI, times 128 columns with v_mfma_f32_16x16x32_bf16
//    (MI x 8 blocks of 16x16).  Wavefront w runs on SIMD w % 4 = wm, so interleaving the row
//    blocks spreads a short tile's work over all four SIMDs; blocks at or past the tile's
//    row count are skipped.
//    The grid is persistent: one workgroup per CU walks its share of the tile list.
//  * Operands go from HBM straight into LDS with buffer_load ... lds (no VGPR staging).
//    Varlen-M kinds: two stages of k = 64 (every K-contiguous row of a stage is one whole
//    128-byte line); each tile runs its own loop, loads one step ahead of the MFMAs, and the
//    next tile's first step is issued before the finished tile's epilogue.  Varlen-K kinds
//    (many short tiles for small groups): four stages of k = 32 in one pipeline that runs
//    across tile boundaries, loads three steps ahead; only wavefronts 0-3 load and only
//    wavefronts 4-7 store (vk_epilogue1).
//  * K-contiguous operands are stored as 128-byte rows, chunk c of row r at c ^ ((r >> 1) & 7),
//    and read as one 16-byte fragment per lane.  K-strided operands (the backward's weights,
//    both varlen-K operands) are stored in their natural layout, k-rows of 512 bytes with
//    chunk c at c ^ f(k), and read with ds_read_b64_tr_b16, which transposes 4x16 blocks of
//    16-bit values across each group of 16 lanes; two such reads make one MFMA fragment.
//    Both placements spread every read over all LDS banks.
//  * Gathered rows (x and dOut through row_token) need the token of each row: per wavefront,
//    4-byte LDS loads fetch a varlen-M tile's tokens a whole tile ahead, and a varlen-K step's
//    six steps ahead, into small slots in LDS.
//  * Loads never branch: a buffer offset beyond the descriptor range returns zeros, which
//    masks rows past a group's end, K tails and steps past the last tile.  Every step issues
//    the same number of loads, and a wavefront's loads and stores complete in issue order, so
//    the wait for a step is an immediate vmcnt equal to the number of memory instructions
//    issued after that step's loads; a raw s_barrier then publishes the stage.
//  * Varlen-M tiles are ordered (expert, n-tile, m-tile) so tiles that share a weight slice
//    run together; varlen-K tiles are ordered heaviest expert first.  Each XCD gets
//    contiguous runs of the tile list, so neighbouring tiles share its L2.
//  * The schedule is static (round r of the grid takes the next G tiles); every tile is
//    computed by one workgroup in a fixed k order, so results are bitwise reproducible, and no
//    reduction uses atomics.  (A dynamic variant, where each XCD's workgroups drew their last
//    tiles from an XCD-local counter, measured slower on the ragged layers it was meant for.)
#include "gemm_lds.h"

namespace moe {
namespace g4 {

using namespace gk;

using gg::Args;
using gg::mkr;
using gg::OOB;
using gg::rsrc_t;
using gg::ufl;
using gg::GATEUP;
using gg::DOWN;
using gg::DH;
using gg::DX;
using gg::DWD;
using gg::DW1;
using gg::GATEUP8;
using gg::DOWN8;
using gg::DX8;

constexpr int NT = 512;        // threads per workgroup
constexpr int BM = 256, BN = 256, BK = 32;  // varlen-K tiles; k = 32 per stage
constexpr int NSTG = 4;        // varlen-K LDS ring depth (stages)
constexpr int AHEAD = NSTG - 1;
constexpr int TOKB = 256;      // bytes per token slot (64 row indices)

// A_KC / B_KC: operand is K-contiguous in memory; GA / GB: operand rows are gathered through
// row_token; VK: the reduction runs over an expert's rows (varlen-K); ST: a lower bound on the
// memory instructions one epilogue issues (used for the vmcnt immediates); MI: row blocks of 16
// per wavefront, so an M-tile has 64 MI rows (varlen-M: 320, which makes a group of up to 320
// rows a single M-tile; varlen-K: 256).
// F8: MX-FP8 operands (e4m3 codes with a scale per 32 values along K, v_mfma_scale_f32_16x16x128_f8f6f4).
template <int K> struct KT;
template <> struct KT<GATEUP> { static constexpr bool A_KC = true, B_KC = true, VK = false, GA = true, GB = false, F8 = false; static constexpr int ST = 32, MI = 5; };
template <> struct KT<DOWN> { static constexpr bool A_KC = true, B_KC = true, VK = false, GA = false, GB = false, F8 = false; static constexpr int ST = 16, MI = 5; };
template <> struct KT<DH> { static constexpr bool A_KC = true, B_KC = false, VK = false, GA = true, GB = false, F8 = false; static constexpr int ST = 40, MI = 5; };
template <> struct KT<DX> { static constexpr bool A_KC = true, B_KC = false, VK = false, GA = false, GB = false, F8 = false; static constexpr int ST = 16, MI = 5; };
template <> struct KT<DWD> { static constexpr bool A_KC = false, B_KC = false, VK = true, GA = true, GB = false, F8 = false; static constexpr int ST = 16, MI = 4; };
template <> struct KT<DW1> { static constexpr bool A_KC = false, B_KC = false, VK = true, GA = false, GB = true, F8 = false; static constexpr int ST = 16, MI = 4; };
template <> struct KT<GATEUP8> { static constexpr bool A_KC = true, B_KC = true, VK = false, GA = true, GB = false, F8 = true; static constexpr int ST = 32, MI = 5; };
template <> struct KT<DOWN8> { static constexpr bool A_KC = true, B_KC = true, VK = false, GA = false, GB = false, F8 = true; static constexpr int ST = 16, MI = 5; };
// DX8 is DOWN8's product out[m][h] = sum_k A[m][k] B[h][k] with A = the rows' quantized dH
// ([M, 2I]), B = expert e's quantized [W_gate^T | W_up^T] ([H, 2I]): launched with Args.I = 2I.
template <> struct KT<DX8> : KT<DOWN8> {};

// Per-kind tile geometry: BMK rows per M-tile; a stage covers BKS values of k and holds OPA
// bytes of A then OPB bytes of B; NST stages form the LDS ring.
//  varlen-M: k = 64 per stage, so a K-contiguous row of a stage is 128 bytes, one whole cache
//            line (with k = 32 every line was fetched twice, half of it each time); two stages
//            of 72 KB.  K-strided B: 64 k-rows of 512 bytes.
//  varlen-K: k = 32 per stage, both operands K-strided (32 k-rows of 512 bytes); four stages.
//            NA: A load instructions per stage (16 rows of 64 bytes each).
//  MX-FP8 (F8): k = 128 e4m3 codes per stage, so a row of a stage is again one 128-byte line and
//            the operand areas match the bf16 ones byte for byte; after them each stage holds
//            the block scales of its rows, one 32-bit word (four blocks of 32) per row: SCA
//            bytes for A (40 rows per wavefront) and SCB for B (32 rows per wavefront).
template <int KIND> struct Geo {
  static constexpr bool VK = KT<KIND>::VK, F8 = KT<KIND>::F8;
  static constexpr int ES = F8 ? 1 : 2;  // bytes per operand element
  static constexpr int MI = KT<KIND>::MI, BMK = 64 * MI;
  static constexpr int BKS = VK ? BK : (F8 ? 128 : 64), NST = VK ? NSTG : 2;
  static constexpr int OPA = BMK * ES * BKS, OPB = BN * ES * BKS, NA = BMK / 16;
  static constexpr int SCA = F8 ? 8 * 40 * 4 : 0, SCB = F8 ? 8 * 32 * 4 : 0;
  static constexpr int STGK = OPA + OPB + SCA + SCB;
  static constexpr int TOKSLOTS = VK ? NSTG : 2;  // token slots per wavefront
};

// sigmoid(g) = 1 / (1 + e^-g) with the hardware exponential and reciprocal (about 1 ulp each,
// far below the bf16 storage precision of every value it feeds)
__device__ __forceinline__ float sigm(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ void st4(rsrc_t r, uint32_t off, float a, float b, float c, float d) {
  u32x2 v;
  v.x = pk2(a, b);
  v.y = pk2(c, d);
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

// ------------------------------------------------------------------ tile list
struct Tile {
  int valid, it, e, roff, mt, nt, mlen, K, nk, kt;
};

template <int KIND>
struct Sched {
  using T = KT<KIND>;
  static constexpr int BMK = Geo<KIND>::BMK;
  const int* s_sched;  // LDS: varlen-M tile prefix [E+1]; varlen-K expert order [E]
  int total, G, per, xcd, slot, E, nN, nMg, nM;

  // Tile `it` of this workgroup: round it of the grid, where XCD x takes the run
  // [x per, (x + 1) per) of the round's G tiles and its workgroups one tile each.
  __device__ __forceinline__ void decode(const Args& a, Tile& c, int it) const {
    c.it = it;
    c.kt = 0;
    const long long tl = (long long)it * G + (long long)xcd * per + slot;
    c.valid = tl < (long long)total;
    if (!c.valid) {
      c.e = 0; c.roff = 0; c.mt = 0; c.nt = 0; c.mlen = 0; c.K = 0; c.nk = 0;
      return;
    }
    const int tile = (int)tl;
    if constexpr (!T::VK) {
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_sched[mid] <= tile) lo = mid; else hi = mid;
      }
      const int e = ufl(lo);
      const int cnt = a.counts[e];
      const int mtiles = (cnt + BMK - 1) / BMK;
      const int local = tile - ufl(s_sched[e]);
      c.e = e;
      c.roff = a.offsets[e];
      c.nt = local / mtiles;
      c.mt = local - c.nt * mtiles;
      c.mlen = min(BMK, cnt - c.mt * BMK);
      switch (KIND) {
        case GATEUP: case GATEUP8: case DH: c.K = a.H; break;
        case DOWN: case DOWN8: case DX8: c.K = a.I; break;
        default: c.K = 2 * a.I; break;  // DX
      }
    } else {
      const int per_e = nM * nN;
      const int rank = tile / per_e;
      const int local = tile - rank * per_e;
      const int e = ufl(s_sched[rank]);
      c.e = e;
      c.roff = a.offsets[e];
      c.mt = local / nN;
      c.nt = local - c.mt * nN;
      if (KIND == DWD) {
        c.mlen = min(BM, a.H - c.mt * BM);
      } else {
        const int seg = c.mt >= nMg;
        c.mlen = min(BM, a.I - (c.mt - seg * nMg) * BM);
      }
      c.K = a.counts[e];
    }
    c.nk = (c.K + Geo<KIND>::BKS - 1) / Geo<KIND>::BKS;
  }
  // Step forward; at a tile's end move to the next tile (skipping tiles without k-steps
  // when skip_empty is set).
  __device__ __forceinline__ void next(const Args& a, Tile& c, bool skip_empty) const {
    if (c.valid && c.kt + 1 < c.nk) {
      ++c.kt;
      return;
    }
    int it = c.it + 1;
    for (;;) {
      decode(a, c, it);
      if (!c.valid || !skip_empty || c.nk > 0) return;
      ++it;
    }
  }
};

// ------------------------------------------------------------------ operand loads
// A load instruction fills one kilobyte of an operand's stage area; lane L writes the 16
// bytes at offset 16 L of it (which kilobyte and which rows: Loader).  K-strided k-rows of
// 512 bytes hold column chunk c at position c ^ mn_f(k).

template <int KIND>
struct Loader {
  using T = KT<KIND>;
  using G = Geo<KIND>;
  i32x4 rA, rB, rB2;          // descriptors; rB2: the up-projection half (GATEUP rows, DX k-rows)
  uint32_t vA[5], vB[4];      // this lane's byte offsets at k = 0 (OOB when masked)
  i32x4 rSA, rSB, rSB2;       // MX-FP8: descriptors of the A and B scale codes (rSB2: up rows)
  uint32_t vSA, vSB;          // MX-FP8: this lane's scale-row byte offsets (OOB when masked)
  uint32_t colA[4], colB[4];  // K-strided: column byte offsets (OOB when masked)
  int kc_c;                   // k-chunk this lane loads (K-contiguous)
  int mn_k[4], mn_c[4];       // k-row and column chunk this lane loads (K-strided)

  // Varlen-M stages (k = 64): K-contiguous rows of 128 bytes, chunk c of row r at position
  // c ^ ((r >> 1) & 7); instruction q of wavefront w fills the kilobyte w + 8q of an operand:
  // rows 8(w + 8q) + (L >> 3) (lane position L & 7) or, K-strided, k-rows 2(w + 8q) + (L >> 5)
  // (lane position L & 31).  A has 5 such instructions per wavefront (BMK = 320 rows), B 4.
  // Varlen-K stages (k = 32): only wavefronts 0-3 load; instruction q (0..3) of wavefront w
  // fills kilobyte 4w + q of each operand, k-rows 2(4w + q) + (L >> 5); K-strided only.
  __device__ __forceinline__ void init(int w, int L) {
    if constexpr (!T::VK) {
      // row 8(w + 8q) + (L >> 3): (r >> 1) & 7 = (4 (w & 1) + (L >> 4)) & 7 for every q
      kc_c = (L & 7) ^ ((4 * (w & 1) + (L >> 4)) & 7);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mn_k[q] = 2 * (w + 8 * q) + (L >> 5);
        mn_c[q] = (L & 31) ^ mn_f(mn_k[q]);
      }
    } else {
      kc_c = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mn_k[q] = (4 * w + q) * 2 + (L >> 5);
        mn_c[q] = (L & 31) ^ mn_f(mn_k[q]);
      }
    }
  }

  // per-tile state; tok = this wavefront's token slot of the tile's first step
  __device__ __forceinline__ void setup(const Args& a, const Tile& c, const int* tok, int w, int L, int nMg) {
    const int H = a.H, I = a.I;
    constexpr uint32_t ES = (uint32_t)G::ES;
    constexpr bool GU = KIND == GATEUP || KIND == GATEUP8, DN = KIND == DOWN || KIND == DOWN8 || KIND == DX8;
    if constexpr (!T::VK) {
      uint32_t rowA[5], rowB[4];  // K-contiguous: row byte offsets (OOB when masked)
      const long long rb = (long long)c.roff + (long long)c.mt * G::BMK;  // first row of the M-tile
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        const int r = 8 * (w + 8 * q) + (L >> 3);  // < 320
        const bool ok = c.valid && r < c.mlen;
        if constexpr (GU || KIND == DH) {
          const int t = tok[8 * q + (L >> 3)];
          rowA[q] = ok ? (uint32_t)t * (uint32_t)H * ES : OOB;
        } else if constexpr (DN) {
          rowA[q] = ok ? (uint32_t)r * (uint32_t)I * ES : OOB;
        } else {  // DX: rows of dH = [dG | dU]
          rowA[q] = ok ? (uint32_t)r * (uint32_t)(2 * I) * 2u : OOB;
        }
      }
      if constexpr (GU || KIND == DH) rA = dmadesc(KIND == DH ? a.dout : a.x, (long long)a.N * H * ES);
      if constexpr (DN) rA = dmadesc_off(a.act, rb * I * ES, (long long)c.mlen * I * ES);
      if constexpr (KIND == DX) rA = dmadesc_off(a.dh, rb * 2 * I * 2, (long long)c.mlen * 2 * I * 2);
      if constexpr (GU) {
        // tile row n = 8w + 64q + (L >> 3): rows 64..127 of each 128-row half are up-projection
        // rows (q odd), for i = 128 nt + 64 (q >> 1) + (n & 63)
        const long long es = (long long)c.e * I * H * ES;
        rB = dmadesc_off(a.wg, es, (long long)I * H * ES);
        rB2 = dmadesc_off(a.wu, es, (long long)I * H * ES);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = c.nt * 128 + (q >> 1) * 64 + 8 * w + (L >> 3);
          rowB[q] = c.valid ? (uint32_t)i * (uint32_t)H * ES : OOB;  // i >= I lies past the range
        }
      } else if constexpr (DN) {
        rB = dmadesc_off(a.wd, (long long)c.e * H * I * ES, (long long)H * I * ES);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = c.nt * BN + 8 * (w + 8 * q) + (L >> 3);
          rowB[q] = (c.valid && n < H) ? (uint32_t)n * (uint32_t)I * ES : OOB;
        }
      } else if constexpr (KIND == DH) {
        rB = dmadesc_off(a.wd, (long long)c.e * H * I * 2, (long long)H * I * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c.nt * BN + 8 * mn_c[q];
          colB[q] = (c.valid && col < I) ? (uint32_t)col * 2u : OOB;
          vB[q] = colB[q] + (uint32_t)mn_k[q] * (uint32_t)I * 2u;
        }
      } else {  // DX
        const long long es = (long long)c.e * I * H * 2;
        rB = dmadesc_off(a.wg, es, (long long)I * H * 2);
        rB2 = dmadesc_off(a.wu, es, (long long)I * H * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c.nt * BN + 8 * mn_c[q];
          colB[q] = (c.valid && col < H) ? (uint32_t)col * 2u : OOB;
          vB[q] = colB[q] + (uint32_t)mn_k[q] * (uint32_t)H * 2u;
        }
      }
#pragma unroll
      for (int q = 0; q < 5; ++q) vA[q] = rowA[q] + 16u * (uint32_t)kc_c;  // OOB stays OOB: no wrap
      if constexpr (T::B_KC) {
#pragma unroll
        for (int q = 0; q < 4; ++q) vB[q] = rowB[q] + 16u * (uint32_t)kc_c;
      }
      if constexpr (G::F8) {
        // Scale words: lane l < 40 loads the word of A row 8(w + 8(l >> 3)) + (l & 7) (the rows
        // whose codes this wavefront loads; tok[l] is that row's token), lane l < 32 the word
        // of B row 8(w + 8(l >> 3)) + (l & 7); rows of a matrix hold 4 ceil(K / 128) bytes.
        const int KSH = 4 * ((H + 127) / 128), KSI = 4 * ((I + 127) / 128);
        const int r = 8 * (w + 8 * (L >> 3)) + (L & 7);
        const bool oka = c.valid && L < 40 && r < c.mlen;
        if constexpr (KIND == GATEUP8) {
          rSA = dmadesc(a.xs, (long long)a.N * KSH);
          vSA = oka ? (uint32_t)tok[L] * (uint32_t)KSH : OOB;
          const long long eo = (long long)c.e * I * KSH;
          rSB = dmadesc_off(a.wgs, eo, (long long)I * KSH);
          rSB2 = dmadesc_off(a.wus, eo, (long long)I * KSH);
          const int i = c.nt * 128 + ((L >> 4) & 1) * 64 + 8 * w + (L & 7);  // q = L >> 3: gate (even), up (odd)
          vSB = (c.valid && L < 32 && i < I) ? (uint32_t)i * (uint32_t)KSH : OOB;
          rSB2 = sgpr4(rSB2);
        } else {  // DOWN8 / DX8: A is the tile's rows of the quantized activation (dH), B is W_down[e] (W^T[e])
          rSA = dmadesc_off(a.acts, rb * KSI, (long long)c.mlen * KSI);
          vSA = oka ? (uint32_t)r * (uint32_t)KSI : OOB;
          rSB = dmadesc_off(a.wds, (long long)c.e * H * KSI, (long long)H * KSI);
          const int n = c.nt * BN + r;
          vSB = (c.valid && L < 32 && n < H) ? (uint32_t)n * (uint32_t)KSI : OOB;
        }
        rSA = sgpr4(rSA);
        rSB = sgpr4(rSB);
      }
      rA = sgpr4(rA);
      rB = sgpr4(rB);
      if constexpr (GU || KIND == DX) rB2 = sgpr4(rB2);
      return;
    }
    if constexpr (KIND == DWD) {
      rA = dmadesc(a.dout, (long long)a.N * H * 2);
      rB = dmadesc_off(a.act, (long long)c.roff * I * 2, (long long)c.K * I * 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ca = c.mt * BM + 8 * mn_c[q];
        colA[q] = (c.valid && ca < H) ? (uint32_t)ca * 2u : OOB;
        const int cb = c.nt * BN + 8 * mn_c[q];
        colB[q] = (c.valid && cb < I) ? (uint32_t)cb * 2u : OOB;
      }
    } else {  // DW1
      const int seg = c.mt >= nMg;
      const int m0 = (c.mt - seg * nMg) * BM;
      rA = dmadesc_off(a.dh, (long long)c.roff * 2 * I * 2, (long long)c.K * 2 * I * 2);
      rB = dmadesc(a.x, (long long)a.N * H * 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ma = m0 + 8 * mn_c[q];
        colA[q] = (c.valid && ma < I) ? (uint32_t)(seg * I + ma) * 2u : OOB;
        const int cb = c.nt * BN + 8 * mn_c[q];
        colB[q] = (c.valid && cb < H) ? (uint32_t)cb * 2u : OOB;
      }
    }
    // offsets at k = 0 for the steps without a K tail (OOB stays OOB: no 32-bit wrap)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (KIND == DWD) vB[q] = colB[q] + (uint32_t)mn_k[q] * (uint32_t)I * 2u;
      if constexpr (KIND == DW1) vA[q] = colA[q] + (uint32_t)mn_k[q] * (uint32_t)(2 * I) * 2u;
    }
    rA = sgpr4(rA);
    rB = sgpr4(rB);
  }

  // The operand loads of step c.kt.  mS: LDS address of the step's stage (see init for which
  // kilobytes this wavefront fills).  tok: the step's token slot (varlen-K gathers).
  // A step without a K tail adds the k advance as the uniform offset; the last step of a tile
  // whose K is not a multiple of the stage's k builds every lane's offset and masks k >= K.
  __device__ __forceinline__ void issue(const Args& a, const Tile& c, uint32_t mS, const int* tok, int w, int L) {
    const int H = a.H, I = a.I;
    // the descriptors in SGPRs once per step (the inline assembly takes them as scalar operands)
    const i32x4 rA = sgpr4(this->rA), rB = sgpr4(this->rB);
    const i32x4 rB2 = (KIND == GATEUP || KIND == GATEUP8 || KIND == DX) ? sgpr4(this->rB2) : rB;
    const int k0 = c.kt * G::BKS;
    constexpr uint32_t ES = (uint32_t)G::ES;
    if constexpr (G::F8) {
      // the step's scale words (word kt of each row: the four blocks of this k-step), lanes
      // outside the wavefront's rows inactive so they write no LDS
      const uint32_t msc = mS + (uint32_t)(G::OPA + G::OPB);
      const uint32_t so4 = (uint32_t)ufl(4 * c.kt);
      const i32x4 rSA_ = sgpr4(rSA), rSB_ = sgpr4(rSB);
      if (L < 40) dma4s(rSA_, msc + (uint32_t)(160 * w), vSA, so4);
      if constexpr (KIND == GATEUP8) {
        const i32x4 rSB2_ = sgpr4(rSB2);
        if (L < 32 && !(L & 8)) dma4s(rSB_, msc + (uint32_t)(G::SCA + 128 * w), vSB, so4);
        if (L < 32 && (L & 8)) dma4s(rSB2_, msc + (uint32_t)(G::SCA + 128 * w), vSB, so4);
      } else {
        if (L < 32) dma4s(rSB_, msc + (uint32_t)(G::SCA + 128 * w), vSB, so4);
      }
    }
    if constexpr (!T::VK) {
      const uint32_t mB = mS + (uint32_t)G::OPA;
      // the uniform advance is only used where it is non-negative and keeps every lane inside
      // its row: no K tail, and (dX) no stage that straddles the gate / up boundary at k = I
      bool fast = k0 + G::BKS <= c.K;
      if constexpr (KIND == DX) fast = fast && (k0 + G::BKS <= I || k0 >= I);
      if (fast) {
        const uint32_t so = (uint32_t)k0 * ES;
#pragma unroll
        for (int q = 0; q < 5; ++q) dma16(rA, mS + (uint32_t)(w + 8 * q) * 1024u, vA[q], so);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t m = mB + (uint32_t)(w + 8 * q) * 1024u;
          if constexpr (KIND == GATEUP || KIND == GATEUP8) dma16((q & 1) ? rB2 : rB, m, vB[q], so);
          if constexpr (KIND == DOWN || KIND == DOWN8 || KIND == DX8) dma16(rB, m, vB[q], so);
          if constexpr (KIND == DH) dma16(rB, m, vB[q], (uint32_t)k0 * (uint32_t)I * 2u);
          if constexpr (KIND == DX) {
            const bool up = k0 >= I;  // the whole stage lies in one half
            dma16(up ? rB2 : rB, m, vB[q], (uint32_t)(k0 - (up ? I : 0)) * (uint32_t)H * 2u);
          }
        }
        return;
      }
      // K tail (or a dX stage across k = I): full per-lane offsets, k >= K masked (a 16-byte
      // chunk holds 16 / ES values and K is a multiple of them, so a chunk is all in or all out)
      const bool kv = k0 + (16 / (int)ES) * kc_c < c.K;
#pragma unroll
      for (int q = 0; q < 5; ++q)
        dma16(rA, mS + (uint32_t)(w + 8 * q) * 1024u, kv ? vA[q] + (uint32_t)k0 * ES : OOB, 0u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t m = mB + (uint32_t)(w + 8 * q) * 1024u;
        if constexpr (KIND == GATEUP || KIND == GATEUP8)
          dma16((q & 1) ? rB2 : rB, m, kv ? vB[q] + (uint32_t)k0 * ES : OOB, 0u);
        if constexpr (KIND == DOWN || KIND == DOWN8 || KIND == DX8) dma16(rB, m, kv ? vB[q] + (uint32_t)k0 * ES : OOB, 0u);
        if constexpr (KIND == DH) {
          const uint32_t k = (uint32_t)(k0 + mn_k[q]);
          dma16(rB, m, colB[q] + k * (uint32_t)I * 2u, 0u);  // k >= H lies past the range
        }
        if constexpr (KIND == DX) {
          // both k-rows of an instruction lie in the same half (I is a multiple of 8), so the
          // half follows from the instruction's first k-row (wavefront-uniform)
          const bool up = k0 + 2 * (w + 8 * q) >= I;
          const uint32_t k = (uint32_t)(k0 + mn_k[q] - (up ? I : 0));
          dma16(up ? rB2 : rB, m, colB[q] + k * (uint32_t)H * 2u, 0u);  // k >= 2I: past the range
        }
      }
      return;
    } else {
      const uint32_t mA = mS + (uint32_t)(4 * w) * 1024u;
      const uint32_t mB = mS + (uint32_t)G::OPA + (uint32_t)(4 * w) * 1024u;
      if (k0 + BK <= c.K) {
        // (only wavefronts 0-3 issue loads: the uniform offset goes to an SGPR explicitly)
        if constexpr (KIND == DWD) {
          const uint32_t so = (uint32_t)ufl(k0 * I * 2);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t t = (uint32_t)tok[2 * q + (L >> 5)];
            dma16(rA, mA + q * 1024, t * (uint32_t)H * 2u + colA[q], 0u);
            dma16(rB, mB + q * 1024, vB[q], so);
          }
        } else {  // DW1
          const uint32_t so = (uint32_t)ufl(k0 * 2 * I * 2);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t t = (uint32_t)tok[2 * q + (L >> 5)];
            dma16(rA, mA + q * 1024, vA[q], so);
            dma16(rB, mB + q * 1024, t * (uint32_t)H * 2u + colB[q], 0u);
          }
        }
        return;
      }
      // K tail: every lane's own offset, k-rows >= K masked
      if constexpr (KIND == DWD) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = k0 + mn_k[q];
          const uint32_t t = (uint32_t)tok[2 * q + (L >> 5)];
          dma16(rA, mA + q * 1024, r < c.K ? t * (uint32_t)H * 2u + colA[q] : OOB, 0u);
          dma16(rB, mB + q * 1024, colB[q] + (uint32_t)r * (uint32_t)I * 2u, 0u);
        }
      } else {  // DW1
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = k0 + mn_k[q];
          const uint32_t t = (uint32_t)tok[2 * q + (L >> 5)];
          dma16(rA, mA + q * 1024, colA[q] + (uint32_t)r * (uint32_t)(2 * I) * 2u, 0u);
          dma16(rB, mB + q * 1024, r < c.K ? t * (uint32_t)H * 2u + colB[q] : OOB, 0u);
        }
      }
    }
  }
};

// ------------------------------------------------------------------ epilogues
// Stores go through LDS: a lane holds 4 consecutive columns of one row, which as a store would
// touch 16 rows x 32 bytes per instruction; staged through LDS, 16 lanes instead cover 256
// contiguous bytes of one row.  `st` is this wavefront's 4 KB of LDS.  A 16-row block of 128
// columns (blk[0..7], as acc[i][0..7]) is written as rows of 256 bytes, 16-byte chunk q of row
// r at position q ^ r, then read back 16 bytes per lane.
__device__ __forceinline__ void stage_write(char* st, const f32x4 (&blk)[8], int L) {
  const int c = L & 15, g = L >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = (2 * j + (g >> 1)) ^ c;
    u32x2 v;
    v.x = pk2(blk[j][0], blk[j][1]);
    v.y = pk2(blk[j][2], blk[j][3]);
    *reinterpret_cast<u32x2*>(st + c * 256 + pos * 16 + (g & 1) * 8) = v;
  }
}
// the same placement for a block already packed to bf16 pairs (blk[j] = columns 16j + 4(L>>4) + 0..3)
__device__ __forceinline__ void stage_write_pk(char* st, const u32x2 (&blk)[8], int L) {
  const int c = L & 15, g = L >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = (2 * j + (g >> 1)) ^ c;
    *reinterpret_cast<u32x2*>(st + c * 256 + pos * 16 + (g & 1) * 8) = blk[j];
  }
}
// fp32 columns 64h .. 64h+63 of a 16-row block (blk[4h .. 4h+3]) as rows of 256 bytes, 16-byte
// chunk q (columns 4q .. 4q+3 of the half) of row r at position q ^ r; read back with stage_read
__device__ __forceinline__ void stage_write_f32(char* st, const f32x4 (&blk)[8], int h, int L) {
  const int c = L & 15, g = L >> 4;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int pos = (4 * jj + g) ^ c;
    *reinterpret_cast<f32x4*>(st + c * 256 + pos * 16) = blk[4 * h + jj];
  }
}
// the 16 bytes (8 columns, chunk L & 15) of row 4p + (L >> 4) of the staged block
__device__ __forceinline__ uint4 stage_read(const char* st, int p, int L) {
  const int row = 4 * p + (L >> 4), q = L & 15;
  return *reinterpret_cast<const uint4*>(st + row * 256 + ((q ^ row) << 4));
}
__device__ __forceinline__ void st16(rsrc_t r, uint32_t off, const uint4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
// Non-temporal form (cache policy NT), for the weight gradients: no later kernel of the step
// reads them, and stored normally their dirty lines drain to HBM during the next kernels
// (the dX GEMM that follows them ran 24 us slower).
__device__ __forceinline__ void st16_nt(rsrc_t r, uint32_t off, const uint4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 2);
}

// acc[i][j][v] = C[m = 16(4i + wm) + (L & 15)][n = wn*128 + 16j + 4(L >> 4) + v]
// `st`: this wavefront's 4 KB of LDS staging, free for the duration of the epilogue.
template <int KIND>
__device__ __forceinline__ void epilogue(const Args& a, const Tile& c, f32x4 (&acc)[KT<KIND>::MI][8], int wm, int wn,
                                         int L_, int nMg, char* st) {
  // The lane's address arithmetic depends only on kernel constants; an opaque copy of the lane
  // index keeps the compiler from computing it once for the whole kernel and holding the
  // results in registers across the k-loop (where they would push the MFMA loop into spills).
  int L = L_;
  asm volatile("" : "+v"(L));
  const int H = a.H, I = a.I;
  constexpr int MI = KT<KIND>::MI;
  const long long rb = (long long)c.roff + (long long)c.mt * Geo<KIND>::BMK;
  if constexpr (KIND == GATEUP || KIND == GATEUP8) {
    const rsrc_t rh = gg::mkr_off(a.out0, rb * 2 * I * 2, (long long)c.mlen * 2 * I * 2);
    const rsrc_t ra = KIND == GATEUP ? gg::mkr_off(a.out1, rb * I * 2, (long long)c.mlen * I * 2)
                                     : gg::mkr_off(a.out1, rb * I, (long long)c.mlen * I);
    const int i0 = c.nt * 128 + wn * 64;  // first i of this wavefront's 64 gate and 64 up columns
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      // [G | U] block: staged columns 0..63 gate, 64..127 up, for i0 .. i0 + 63
      stage_write(st, acc[i], L);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 v = stage_read(st, p, L);
        const uint32_t m = (uint32_t)(16 * (4 * i + wm) + 4 * p + (L >> 4));  // rows >= mlen: past the range
        const int q = L & 15, ii = i0 + (q & 7) * 8;
        const uint32_t off = m * (uint32_t)(2 * I) * 2u + (uint32_t)((q >= 8 ? I : 0) + ii) * 2u;
        st16(rh, ii < I ? off : OOB, v);
      }
      if constexpr (KIND == GATEUP8) {
        // A = silu(G) * U quantized to MX-FP8 for the down GEMM: the wavefront's 64 columns are
        // two blocks of 32 (column blocks j = 0, 1 and 2, 3); a row's block lies in the four
        // lanes L & 15 + 16 g (eight values each), whose maximum gives the block's scale.
        // Columns >= I hold zeros (their weight rows loaded as zeros), so their blocks get
        // scale code 0, which also fills the scale row's padding entries.
        f32x4 av[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) av[j][v] = acc[i][j][v] * sigm(acc[i][j][v]) * acc[i][j + 4][v];
        int se[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float mx = 0.f;
#pragma unroll
          for (int j = 2 * b; j < 2 * b + 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) mx = fmaxf(mx, fabsf(av[j][v]));
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          se[b] = mx_scale_exp(mx);
        }
        const uint32_t m = (uint32_t)(16 * (4 * i + wm) + (L & 15));  // rows >= mlen: past the range
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t wq = mx_pack4(av[j][0], av[j][1], av[j][2], av[j][3], se[j >> 1]);
          const int ii = i0 + 16 * j + 4 * (L >> 4);
          __builtin_amdgcn_raw_buffer_store_b32(wq, ra, ii < I ? m * (uint32_t)I + (uint32_t)ii : OOB, 0, 0);
        }
        // the two scale codes of the row, by the lanes of column group 0 (i0 / 32 < KSI - 1)
        const int KSI = 4 * ((I + 127) / 128);
        const rsrc_t rs = gg::mkr_off(a.out2, rb * KSI, (long long)c.mlen * KSI);
        const uint16_t sc2 = (uint16_t)((se[0] + 127) | ((se[1] + 127) << 8));
        __builtin_amdgcn_raw_buffer_store_b16(sc2, rs, (L >> 4) == 0 ? m * (uint32_t)KSI + (uint32_t)(i0 / 32) : OOB,
                                              0, 0);
        continue;
      }
      // A = silu(G) * U, staged in the first 64 columns
      f32x4 ab[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int v = 0; v < 4; ++v) ab[j][v] = acc[i][j][v] * sigm(acc[i][j][v]) * acc[i][j + 4][v];
        ab[j + 4] = ab[j];
      }
      stage_write(st, ab, L);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 v = stage_read(st, p, L);
        const uint32_t m = (uint32_t)(16 * (4 * i + wm) + 4 * p + (L >> 4));
        const int q = L & 15, ii = i0 + q * 8;
        if (q < 8) st16(ra, ii < I ? m * (uint32_t)I * 2u + (uint32_t)ii * 2u : OOB, v);
      }
    }
  } else if constexpr (KIND == DOWN || KIND == DOWN8 || KIND == DX || KIND == DX8) {
    const rsrc_t ro = gg::mkr_off(a.out0, rb * H * 2, (long long)c.mlen * H * 2);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      stage_write(st, acc[i], L);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 v = stage_read(st, p, L);
        const uint32_t m = (uint32_t)(16 * (4 * i + wm) + 4 * p + (L >> 4));  // rows >= mlen: past the range
        const int n = c.nt * BN + wn * 128 + (L & 15) * 8;
        st16(ro, n < H ? m * (uint32_t)H * 2u + (uint32_t)n * 2u : OOB, v);
      }
    }
  } else if constexpr (KIND == DH) {
    // The dSwiGLU epilogue: acc holds dA' = dOut[t] W_down^T for 16-row blocks of 128 i columns.
    // With the cached [G | U] of the same rows and columns and the row's weight w:
    //   A = silu(G) U,  dA = w dA',  dG = dA U s (1 + G (1 - s)),  dU = dA silu(G)  (s = sigmoid(G)),
    //   A' = w A,  and this wavefront's part of dS = <dA', A> over its 128 columns.
    // G and U come in as rows of 256 contiguous bytes (16 lanes per row) through the
    // wavefront's 8 KB of staging (G in the first 4 KB, U in the second), are read back in the
    // accumulator layout, and dG / dU replace them in place; A' follows in the G half.  dH =
    // [dG | dU] and A' leave as rows of 256 bytes again.  dS partial q = 2 n-tile + wn of row r
    // goes to dspart[r nP + q] (nP = 2 ceil(I / 256)), summed in order by the next kernel.
    // Rows >= mlen and columns >= I lie past the descriptors' ranges: their loads read zeros
    // and their stores are dropped.
    const rsrc_t rhc = gg::mkr_off(a.hcache, rb * 2 * I * 2, (long long)c.mlen * 2 * I * 2);
    const rsrc_t rdh = gg::mkr_off(a.out0, rb * 2 * I * 2, (long long)c.mlen * 2 * I * 2);
    const rsrc_t rap = gg::mkr_off(a.out1, rb * I * 2, (long long)c.mlen * I * 2);
    const rsrc_t rw = gg::mkr_off(a.row_w, rb * 4, (long long)c.mlen * 4);
    const int nP = 2 * ((I + 255) / 256);
    const rsrc_t rds = gg::mkr_off(a.dspart, rb * nP * 4, (long long)c.mlen * nP * 4);
    const int c0 = c.nt * BN + wn * 128;
    char* sgu = st;         // G, then dG, then A'
    char* suu = st + 4096;  // U, then dU
    const int q = L & 15, g4 = L >> 4;
    const int col = c0 + 8 * q;  // the 8 columns this lane moves in row-contiguous form
    // (loading block i + 1's G and U during block i would keep 33 more registers live and
    // pushes them into scratch, which made the epilogue twice as slow)
    uint4 gv[4], uv[4];
    float w = 0.f;
    auto gu_load = [&](int i) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t m = (uint32_t)(16 * (4 * i + wm) + 4 * p + g4);
        const uint32_t off = m * (uint32_t)(2 * I) * 2u + (uint32_t)col * 2u;
        gv[p] = gg::bld16(rhc, col < I ? off : OOB);
        uv[p] = gg::bld16(rhc, col < I ? off + (uint32_t)I * 2u : OOB);
      }
      w = __int_as_float(gg::bld4(rw, (uint32_t)(16 * (4 * i + wm) + q) * 4u));
    };
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      gu_load(i);
      const float wi = w;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = 4 * p + g4;
        *reinterpret_cast<uint4*>(sgu + r * 256 + ((q ^ r) << 4)) = gv[p];
        *reinterpret_cast<uint4*>(suu + r * 256 + ((q ^ r) << 4)) = uv[p];
      }
      float ds = 0.f;
      u32x2 apk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int o = q * 256 + (((2 * j + (g4 >> 1)) ^ q) << 4) + (g4 & 1) * 8;
        const u32x2 G2 = *reinterpret_cast<const u32x2*>(sgu + o);
        const u32x2 U2 = *reinterpret_cast<const u32x2*>(suu + o);
        float rg[4], ru[4], ra[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t gw = v < 2 ? G2.x : G2.y, uw = v < 2 ? U2.x : U2.y;
          const float gg_ = __uint_as_float((v & 1) ? (gw & 0xFFFF0000u) : (gw << 16));
          const float u = __uint_as_float((v & 1) ? (uw & 0xFFFF0000u) : (uw << 16));
          const float sg = sigm(gg_);
          const float silu = gg_ * sg;
          const float act = silu * u;
          const float d = acc[i][j][v];
          ds += d * act;
          const float da = wi * d;
          rg[v] = da * u * sg * (1.0f + gg_ * (1.0f - sg));
          ru[v] = da * silu;
          ra[v] = wi * act;
        }
        *reinterpret_cast<u32x2*>(sgu + o) = u32x2{pk2(rg[0], rg[1]), pk2(rg[2], rg[3])};
        *reinterpret_cast<u32x2*>(suu + o) = u32x2{pk2(ru[0], ru[1]), pk2(ru[2], ru[3])};
        apk[j] = u32x2{pk2(ra[0], ra[1]), pk2(ra[2], ra[3])};
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t m = (uint32_t)(16 * (4 * i + wm) + 4 * p + g4);
        const uint32_t off = m * (uint32_t)(2 * I) * 2u + (uint32_t)col * 2u;
        st16(rdh, col < I ? off : OOB, stage_read(sgu, p, L));
        st16(rdh, col < I ? off + (uint32_t)I * 2u : OOB, stage_read(suu, p, L));
      }
      stage_write_pk(sgu, apk, L);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t m = (uint32_t)(16 * (4 * i + wm) + 4 * p + g4);
        st16(rap, col < I ? m * (uint32_t)I * 2u + (uint32_t)col * 2u : OOB, stage_read(sgu, p, L));
      }
      ds += __shfl_xor(ds, 16);
      ds += __shfl_xor(ds, 32);
      const uint32_t doff = ((uint32_t)(16 * (4 * i + wm) + q) * (uint32_t)nP + (uint32_t)(2 * c.nt + wn)) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ds), rds, g4 == 0 ? doff : OOB, 0, 0);
    }
  } else if constexpr (KIND == DWD) {
    const rsrc_t ro = gg::mkr_off(a.out0, (long long)c.e * H * I * 2, (long long)H * I * 2);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      stage_write(st, acc[i], L);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 v = stage_read(st, p, L);
        const int m = c.mt * BM + 16 * (4 * i + wm) + 4 * p + (L >> 4);  // h
        const int n = c.nt * BN + wn * 128 + (L & 15) * 8;                 // i
        st16(ro, (m < H && n < I) ? (uint32_t)m * (uint32_t)I * 2u + (uint32_t)n * 2u : OOB, v);
      }
    }
  } else {  // DW1
    const int seg = c.mt >= nMg;
    const int m0 = (c.mt - seg * nMg) * BM;
    const rsrc_t ro = gg::mkr_off(seg ? a.out1 : a.out0, (long long)c.e * I * H * 2, (long long)I * H * 2);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      stage_write(st, acc[i], L);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 v = stage_read(st, p, L);
        const int m = m0 + 16 * (4 * i + wm) + 4 * p + (L >> 4);  // i of dW_gate / dW_up
        const int n = c.nt * BN + wn * 128 + (L & 15) * 8;        // h
        st16(ro, (m < I && n < H) ? (uint32_t)m * (uint32_t)H * 2u + (uint32_t)n * 2u : OOB, v);
      }
    }
  }
}

// Varlen-K output addressing: row 4p + (L >> 4) and columns 8 (L & 15) .. + 7 of 16-row block
// i of wavefront (wm, wn) in tile c: the descriptor of the weight gradient it belongs to and
// the byte offset (OOB past the matrix).  DWD: rows h, columns i of dW_down[e]; DW1: rows i
// of dW_gate[e] (M-tiles below nMg) or dW_up[e], columns h.
template <int KIND>
__device__ __forceinline__ uint32_t vk_out(const Args& a, const Tile& c, int i, int p, int wm, int wn, int nMg,
                                           int L, rsrc_t& ro) {
  const int H = a.H, I = a.I;
  const int n = c.nt * BN + wn * 128 + (L & 15) * 8;
  if constexpr (KIND == DWD) {
    ro = gg::mkr_off(a.out0, (long long)c.e * H * I * 2, (long long)H * I * 2);
    const int m = c.mt * BM + 16 * (4 * i + wm) + 4 * p + (L >> 4);  // h
    return (m < H && n < I) ? (uint32_t)m * (uint32_t)I * 2u + (uint32_t)n * 2u : OOB;
  } else {
    const int seg = c.mt >= nMg;
    const int m = (c.mt - seg * nMg) * BM + 16 * (4 * i + wm) + 4 * p + (L >> 4);  // i
    ro = gg::mkr_off(seg ? a.out1 : a.out0, (long long)c.e * I * H * 2, (long long)I * H * 2);
    return (m < I && n < H) ? (uint32_t)m * (uint32_t)H * 2u + (uint32_t)n * 2u : OOB;
  }
}

// Varlen-K epilogue.  Wavefronts 0-3 (wn = 0) issue every operand load and no store;
// wavefronts 4-7 (wn = 1) issue every store.  Loads and stores of a wavefront complete in
// issue order on one counter, so a wavefront that stored a tile's results would have to wait
// for those stores to drain before it could wait for any load issued after them; split this
// way, the loaders' waits never include a store.
//  part 1 (every wavefront, after an LDS barrier): a loader writes its four blocks as bf16 to
//    `pst` (4 KB per block; stage_write placement); a storer stores its own blocks through
//    its 4 KB slot `own`.
//  part 2 (storers, after a second barrier): the partner loader's (w - 4) blocks from its `pst`.
template <int KIND>
__device__ __forceinline__ void vk_epilogue1(const Args& a, const Tile& c, f32x4 (&acc)[4][8], int wm, int wn,
                                             int L_, int nMg, char* pst, char* own) {
  int L = L_;
  asm volatile("" : "+v"(L));
  if (wn == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) stage_write(pst + i * 4096, acc[i], L);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      stage_write(own, acc[i], L);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint4 v = stage_read(own, p, L);
        rsrc_t ro;
        const uint32_t off = vk_out<KIND>(a, c, i, p, wm, 1, nMg, L, ro);
        st16_nt(ro, off, v);
      }
    }
  }
}
template <int KIND>
__device__ __forceinline__ void vk_epilogue2(const Args& a, const Tile& c, int wm, int L_, int nMg, const char* pst) {
  int L = L_;
  asm volatile("" : "+v"(L));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4 v = stage_read(pst + i * 4096, p, L);
      rsrc_t ro;
      const uint32_t off = vk_out<KIND>(a, c, i, p, wm, 0, nMg, L, ro);
      st16_nt(ro, off, v);
    }
}
// The zeros of an expert without rows.  Its weight gradient (DWD: dW_down[e], DW1: dW_gate[e]
// or dW_up[e]) is one contiguous region, so its tiles split the region into equal chunks of
// whole kilobytes, tile (mt, nt) taking chunk (mt - seg nMg) nN + nt, and write them as plain
// kilobyte rows (64 lanes x 16 bytes): the storers' wavefront wm the stores q = wm, wm + 4,
// ....
template <int KIND>
__device__ __forceinline__ void vk_zero(const Args& a, const Tile& c, int wm, int L_, int nN, int nMg) {
  int L = L_;
  asm volatile("" : "+v"(L));
  const uint4 z = {0u, 0u, 0u, 0u};
  const long long region = (long long)a.H * a.I * 2;
  const int seg = KIND == DW1 && c.mt >= nMg;
  const int ntl = (KIND == DWD ? (a.H + BM - 1) / BM : nMg) * nN;  // tiles per region
  const long long kb = (region + 1023) / 1024;
  const int ckb = (int)((kb + ntl - 1) / ntl);  // kilobytes per chunk
  const int lt = (c.mt - seg * nMg) * nN + c.nt;
  const rsrc_t ro = gg::mkr_off(seg ? a.out1 : a.out0, (long long)c.e * region, region);
  const uint32_t base = (uint32_t)lt * (uint32_t)ckb * 1024u + (uint32_t)L * 16u;
#pragma unroll 1
  for (int q = wm; q < ckb; q += 4) st16_nt(ro, base + (uint32_t)q * 1024u, z);
}

// ------------------------------------------------------------------ fragments
// K-contiguous fragment of rows r0 .. r0+15 (varlen-M stages, rows of 128 bytes): lane reads
// row r0 + (L & 15), k-chunk 4 sub + (L >> 4) of the stage's eight; kc_off: the lane's offset
// for sub = 0 (sub = 1 flips bit 2 of the chunk position, offset bit 6).
__device__ __forceinline__ bf16x8 frag_kc(const char* op, int r0, int sub, int kc_off) {
  return *reinterpret_cast<const bf16x8*>(op + r0 * 128 + (kc_off ^ (64 * sub)));
}
// K-strided fragment of columns x0 .. x0+15 (x0 a multiple of 16): two transposing reads of
// k-rows 8(L>>4) + 0..3 and + 4..7 (mn_k0 includes the 32-row offset of a second k-substep).
__device__ __forceinline__ bf16x8 frag_mn(const char* op, int x0, int mn_k0, int mn_f_, int mn_b) {
  const int pos = ((((x0 >> 3) ^ mn_f_) | mn_b) << 4);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(op + mn_k0 + pos));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(op + mn_k0 + 4 * 512 + pos));
  struct P { s16x4 a, b; } p{lo, hi};
  return __builtin_bit_cast(bf16x8, p);
}

// The wait before a varlen-M step: `later` of the tile's following steps (at most two, P
// memory instructions each) were issued after this step's loads.
template <int P>
__device__ __forceinline__ void mstep_wait(int later) {
  if (later >= 2) vm_wait_barrier<2 * P>();
  else if (later == 1) vm_wait_barrier<P>();
  else vm_wait_barrier<0>();
}

// ------------------------------------------------------------------ the kernel
template <int KIND>
__global__ __launch_bounds__(NT, 1) void k_gg_bf16(Args a, const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ offsets) {
  a.counts = counts;
  a.offsets = offsets;
  using T = KT<KIND>;
  using G = Geo<KIND>;
  constexpr bool GATHER = T::GA || T::GB;

  __shared__ __attribute__((aligned(1024))) char s_ring[G::NST * G::STGK];
  __shared__ __attribute__((aligned(256))) int s_tok[8 * G::TOKSLOTS * (TOKB / 4)];
  __shared__ int s_sched[1025];
  __shared__ int s_wsum[9];
  __shared__ __attribute__((aligned(256))) char s_stg[T::VK ? 4 * 4096 : 16];

  const int tid = threadIdx.x, L = tid & 63;
  const int w = ufl(tid >> 6);
  const int wm = w & 3, wn = w >> 2;
  const int E = a.E;

  Sched<KIND> S;
  S.s_sched = s_sched;
  S.E = E;
  S.G = gridDim.x;
  S.per = S.G >> 3;
  S.xcd = blockIdx.x & 7;
  S.slot = blockIdx.x >> 3;
  switch (KIND) {
    case GATEUP: case GATEUP8: S.nN = (a.I + 127) / 128; break;
    case DOWN: case DOWN8: case DX: case DX8: case DW1: S.nN = (a.H + BN - 1) / BN; break;
    default: S.nN = (a.I + BN - 1) / BN; break;  // DH, DWD
  }
  S.nMg = (a.I + BM - 1) / BM;
  S.nM = KIND == DWD ? (a.H + BM - 1) / BM : 2 * S.nMg;

  // ---- tile list from the device-resident counts ----
  if constexpr (!T::VK) {
    int loc[2], sum = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid * 2 + q;
      loc[q] = e < E ? ((a.counts[e] + G::BMK - 1) / G::BMK) * S.nN : 0;
      sum += loc[q];
    }
    int x = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (L >= off) x += y;
    }
    if (L == 63) s_wsum[w] = x;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int q = 0; q < 8; ++q) {
        const int v = s_wsum[q];
        s_wsum[q] = run;
        run += v;
      }
      s_wsum[8] = run;
    }
    __syncthreads();
    int run = s_wsum[w] + x - sum;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid * 2 + q;
      if (e < E) s_sched[e] = run;
      run += loc[q];
    }
    if (tid == 0) s_sched[E] = s_wsum[8];
    S.total = ufl(s_wsum[8]);
    __syncthreads();
  } else {
    // heaviest expert first: rank_e = #{f : c_f > c_e or (c_f == c_e and f < e)}
    int* s_cnt = reinterpret_cast<int*>(s_ring);  // the ring is free until the first load
    for (int e = tid; e < E; e += NT) s_cnt[e] = a.counts[e];
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
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

  f32x4 acc[G::MI][8];
#pragma unroll
  for (int i = 0; i < G::MI; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane fragment addressing (K-contiguous rows: chunk c of row r at c ^ ((r >> 1) & 7))
  const int kc_off = (L & 15) * 128 + ((((L >> 4) ^ ((L >> 1) & 7)) & 7) << 4);
  const int mn_m = L & 15, mn_g = L >> 4;
  const int mn_k0 = (8 * mn_g + (mn_m >> 2)) * 512 + 8 * (mn_m & 1);
  const int mn_ff = 2 * ((mn_m >> 2) | ((mn_g & 1) << 2));
  const int mn_b = (mn_m >> 1) & 1;

  // The MFMAs of one k-substep (k = 32; sub: which 32 of a varlen-M stage) from the stage at
  // `sa`: this wavefront's row blocks 16(4i + wm) that start below the tile's row count
  // (nb = mlen - 16 wm > 64 i; a block at or past it holds rows of no group and is skipped)
  // times its 128 columns.
  auto mma_stage = [&](const char* sa, int nb, int sub) __attribute__((always_inline)) {
    // opaque copies: the per-fragment LDS positions derived from these are recomputed each
    // step rather than held in registers across the loop
    int kco = kc_off, k0o = mn_k0 + sub * (32 * 512), ffo = mn_ff, bo = mn_b;
    asm volatile("" : "+v"(kco), "+v"(k0o), "+v"(ffo), "+v"(bo));
    const char* sb = sa + G::OPA;
    auto frag_a = [&](int i) __attribute__((always_inline)) {
      if constexpr (T::A_KC) return frag_kc(sa, 16 * (4 * i + wm), sub, kco);
      else return frag_mn(sa, 16 * (4 * i + wm), k0o, ffo, bo);
    };
    auto frag_b = [&](int j) __attribute__((always_inline)) {
      if constexpr (T::B_KC) return frag_kc(sb, wn * 128 + 16 * j, sub, kco);
      else return frag_mn(sb, wn * 128 + 16 * j, k0o, ffo, bo);
    };
    if constexpr (KIND == DH) {
      // (fewer live fragments, for the register budget of the dSwiGLU epilogue) all A
      // fragments first, then the B fragments one column block ahead.  Every row block is
      // computed, also those past the tile's rows (zeros, never stored): in this order the
      // row-block test becomes a branch around each MFMA, which costs more than the MFMAs
      // it saves.
      bf16x8 fa[G::MI];
#pragma unroll
      for (int i = 0; i < G::MI; ++i) fa[i] = frag_a(i);
      bf16x8 fb = frag_b(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 fn;
        if (j + 1 < 8) fn = frag_b(j + 1);
#pragma unroll
        for (int i = 0; i < G::MI; ++i) acc[i][j] = mma(fb, fa[i], acc[i][j]);
        if (j + 1 < 8) fb = fn;
      }
    } else {
      // all B fragments first, then the A fragments one row block ahead: block i + 1's read
      // is in flight during block i's MFMAs
      bf16x8 fb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[j] = frag_b(j);
      bf16x8 fa = frag_a(0);
#pragma unroll
      for (int i = 0; i < G::MI; ++i) {
        bf16x8 fn;
        if (i + 1 < G::MI) fn = frag_a(i + 1);
        if (i == 0 || nb > 64 * i) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = mma(fb[j], fa, acc[i][j]);
        }
        if (i + 1 < G::MI) fa = fn;
      }
    }
  };

  // MX-FP8 step, half h: the MFMAs of this wavefront's column blocks 4h .. 4h + 3 over the
  // stage's k = 128 (v_mfma_scale_f32_16x16x128_f8f6f4, e4m3 x e4m3).  The instruction takes
  // lane row (L & 15), bytes 16 (L >> 4) .. + 15 and 64 + 16 (L >> 4) .. + 15 of its 128: the two
  // chunks the bf16 step reads for its two k-substeps, so a fragment is those two reads.  The
  // scale of (row L & 15, block L >> 4) is byte L >> 4 of the row's scale word, which the lane
  // shifts down to byte 0 (the byte the instruction reads).  A's words sit in the stage at
  // 40 w + 8 q + r for row 8 (w + 8 q) + r, B's at 32 w + 8 q + r (the order of their loads).
  auto mma_stage8 = [&](const char* sa, int nb, int h) __attribute__((always_inline)) {
    int kco = kc_off, sho = 8 * (L >> 4), lro = L & 15;
    asm volatile("" : "+v"(kco), "+v"(sho), "+v"(lro));
    const char* sb = sa + G::OPA;
    const uint32_t* sca = reinterpret_cast<const uint32_t*>(sa + G::OPA + G::OPB);
    const uint32_t* scb = reinterpret_cast<const uint32_t*>(sa + G::OPA + G::OPB + G::SCA);
    auto frag8 = [&](const char* op, int r0) __attribute__((always_inline)) {
      struct P { bf16x8 lo, hi; } pr{frag_kc(op, r0, 0, kco), frag_kc(op, r0, 1, kco)};
      return __builtin_bit_cast(i32x8, pr);
    };
    auto scale_a = [&](int m) __attribute__((always_inline)) {
      return (int)(sca[40 * ((m >> 3) & 7) + 8 * (m >> 6) + (m & 7)] >> sho);
    };
    auto scale_b = [&](int n) __attribute__((always_inline)) {
      return (int)(scb[32 * ((n >> 3) & 7) + 8 * (n >> 6) + (n & 7)] >> sho);
    };
    i32x8 fb[4];
    int sbv[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int n0 = wn * 128 + 16 * (4 * h + jj);
      fb[jj] = frag8(sb, n0);
      sbv[jj] = scale_b(n0 + lro);
    }
    i32x8 fa = frag8(sa, 16 * wm);
    int sav = scale_a(16 * wm + lro);
#pragma unroll
    for (int i = 0; i < G::MI; ++i) {
      i32x8 fn;
      int sn = 0;
      if (i + 1 < G::MI) {
        fn = frag8(sa, 16 * (4 * (i + 1) + wm));
        sn = scale_a(16 * (4 * (i + 1) + wm) + lro);
      }
      if (i == 0 || nb > 64 * i) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          acc[i][4 * h + jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[jj], fa, acc[i][4 * h + jj], 0, 0,
                                                                                0, sbv[jj], 0, sav);
      }
      if (i + 1 < G::MI) {
        fa = fn;
        sav = sn;
      }
    }
  };

  // Varlen-K step: fa / fb hold this step's fragments, read during the previous step.  The
  // MFMAs go column block by column block; once a column's four MFMAs are issued its B
  // fragment is refilled with the next step's from the stage at `sn`, and after the last
  // column the A fragments are, so the next step's LDS reads overlap this step's MFMAs
  // instead of preceding them.  Every block is computed: a varlen-K tile's rows are weight
  // rows (h or i), ragged only in the last M-tile of a matrix, and the epilogue never stores
  // a row at or past the matrix's end, so what such blocks compute is discarded.
  auto mma_pf = [&](bf16x8 (&fa)[4], bf16x8 (&fb)[8], const char* sn) __attribute__((always_inline)) {
    int k0o = mn_k0, ffo = mn_ff, bo = mn_b;
    asm volatile("" : "+v"(k0o), "+v"(ffo), "+v"(bo));
    const char* sbn = sn + G::OPA;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = mma(fb[j], fa[i], acc[i][j]);
      fb[j] = frag_mn(sbn, wn * 128 + 16 * j, k0o, ffo, bo);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag_mn(sn, 16 * (4 * i + wm), k0o, ffo, bo);
  };

  Loader<KIND> ld;
  ld.init(w, L);
  const i32x4 rtok = dmadesc(a.row_token, 4LL * (long long)a.M_cap);
  int* my_tok = s_tok + w * G::TOKSLOTS * (TOKB / 4);  // this wavefront's token slots
  const uint32_t tok_m0 = lds_addr(my_tok);
  const uint32_t ring_m0 = lds_addr(s_ring);  // stage 0

  if constexpr (!T::VK) {
    // ---- varlen-M: this workgroup's tiles one after another ----
    // Two stages of k = 64: the loads of step kt + 1 are issued right after step kt's wait and
    // fill the stage that step kt - 1 used, during step kt's MFMAs.  Every tile has k-steps
    // (groups without rows have no tiles).  A tile's loader is set up and its first step
    // issued before the previous tile's epilogue, so those loads overlap the epilogue and the
    // epilogue's stores drain during the first step.  A tile's tokens (gathered A) are loaded
    // into LDS a tile earlier, before that earlier tile's first step, so they have landed by
    // its first wait; tokens alternate between two slots (tile it uses slot it & 1).
    static_assert(G::NST == 2, "varlen-M: two stages");
    auto tok_load = [&](const Tile& t) __attribute__((always_inline)) {
      if constexpr (T::GA) {
        // lane L: the token of row 8(w + 8(L >> 3)) + (L & 7), i.e. of A instruction L >> 3 of
        // this wavefront (instructions past the tile's five are never used)
        if (t.valid)
          dma4(rtok, tok_m0 + (uint32_t)(t.it & 1) * TOKB,
               (uint32_t)(t.roff + t.mt * G::BMK + 8 * w + 64 * (L >> 3) + (L & 7)) * 4u);
      }
    };
    auto issue_step = [&](const Tile& t, int kt, int stage) __attribute__((always_inline)) {
      Tile u = t;
      u.kt = kt;
      ld.issue(a, u, ring_m0 + (uint32_t)(stage & 1) * G::STGK, my_tok, w, L);
    };
    {
      Tile C0, C1;
      S.decode(a, C0, 0);
      if (!C0.valid) return;
      tok_load(C0);
      vm_drain();
      ld.setup(a, C0, my_tok, w, L, S.nMg);
      S.decode(a, C1, 1);
      tok_load(C1);
      issue_step(C0, 0, 0);
    }
    int gs = 0;  // ring sequence number of the current tile's first step
    int ep = 0;  // an epilogue's stores were issued after the current tile's first step
#pragma unroll 1
    for (int it = 0;; ++it) {
      // tile `it`: its loader is set up and its first step's loads are in flight
      Tile Cc;
      S.decode(a, Cc, it);
      if (!Cc.valid) break;
      const int nk = Cc.nk;
      const int nb = Cc.mlen - 16 * wm;
#pragma unroll 1
      for (int kt = 0; kt < nk; ++kt) {
        // step kt's loads have landed for every wavefront (at the first step, the previous
        // tile's epilogue stores, issued after them, may still be in flight: at least ST
        // instructions), and every wavefront is done with the stage that the loads below
        // refill (the stage of step kt - 1)
        if (kt == 0 && ep) vm_wait_barrier<T::ST>();
        else vm_wait_barrier<0>();
        // the two wavefronts of a SIMD issue the next step's loads at different points (before
        // and after their first k-substep), so one issues loads while the other runs MFMAs
        const char* sa = s_ring + ((gs + kt) & 1) * G::STGK;
        if (wn == 0 && kt + 1 < nk) issue_step(Cc, kt + 1, gs + kt + 1);
        if constexpr (G::F8) {
          if (nb > 0) mma_stage8(sa, nb, 0);
        } else {
          if (nb > 0) mma_stage(sa, nb, 0);
        }
        if (wn != 0 && kt + 1 < nk) issue_step(Cc, kt + 1, gs + kt + 1);
        if constexpr (G::F8) {
          if (nb > 0) mma_stage8(sa, nb, 1);
        } else {
          if (nb > 0) mma_stage(sa, nb, 1);
        }
      }
      // every wavefront is done with the ring: the last step's stage stages the epilogue, the
      // other takes the next tile's first step, issued before the epilogue so that its wait
      // does not include the epilogue's stores
      char* st = s_ring + ((gs + nk - 1) & 1) * G::STGK + w * (KIND == DH ? 8192 : 4096);
      lds_barrier();
      gs += nk;
      {
        Tile Cn;
        S.decode(a, Cn, it + 1);
        if (Cn.valid) {
          ld.setup(a, Cn, my_tok + ((it + 1) & 1) * (TOKB / 4), w, L, S.nMg);
          Tile Cnn;
          S.decode(a, Cnn, it + 2);
          tok_load(Cnn);
          issue_step(Cn, 0, gs);
        }
      }
      epilogue<KIND>(a, Cc, acc, wm, wn, L, S.nMg, st);
#pragma unroll
      for (int i = 0; i < G::MI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      ep = 1;
    }
    vm_drain();
  } else {
    // ---- varlen-K: one pipeline over the workgroup's tiles, three steps ahead ----
    // Wavefronts 0-3 (wn = 0) issue every load (operands and tokens), wavefronts 4-7 every
    // store (see vk_epilogue1); all eight compute.  Tiles without k-steps (empty groups) only
    // write zeros.
    const bool loader = wn == 0;
    char* s_own = s_stg + wm * 4096;  // a storer's staging slot
    Tile Cc;
    S.decode(a, Cc, 0);
    while (Cc.valid && Cc.nk == 0) {
      if (!loader) vk_zero<KIND>(a, Cc, wm, L, S.nN, S.nMg);
      S.decode(a, Cc, Cc.it + 1);
    }
    if (!Cc.valid) return;

    // the token load of cursor t at step index s (gathered kinds, every step): loader w takes
    // the rows 8w .. 8w + 63 of the step (its loads use rows 8w .. 8w + 7)
    auto tok_issue = [&](const Tile& t, int s) __attribute__((always_inline)) {
      const uint32_t m0 = tok_m0 + (uint32_t)(s & (NSTG - 1)) * TOKB;
      dma4(rtok, m0, t.valid ? (uint32_t)(t.roff + t.kt * BK + 8 * w + L) * 4u : OOB);
    };
    Tile Ld = Cc, Tk = Cc;
    auto load_issue = [&](int s) __attribute__((always_inline)) {
      const int* tk = my_tok + (s & (NSTG - 1)) * (TOKB / 4);
      if (Ld.kt == 0) ld.setup(a, Ld, tk, w, L, S.nMg);
      ld.issue(a, Ld, ring_m0 + (uint32_t)(s & (NSTG - 1)) * G::STGK, tk, w, L);
      S.next(a, Ld, true);
    };
    // memory instructions a loader issues per step: 8 operand loads and the token load
    constexpr int NLK = 8 + (GATHER ? 1 : 0);
    static_assert(G::NA == 16, "varlen-K: four loaders, eight loads each per step");

    // ---- prologue (loaders): tokens of steps 0..2 resident, loads of steps 0..2 in flight ----
    if (loader) {
      if constexpr (GATHER) {
#pragma unroll 1
        for (int s = 0; s < AHEAD; ++s) {
          tok_issue(Tk, s);
          S.next(a, Tk, true);
        }
        vm_drain();
      }
#pragma unroll 1
      for (int s = 0; s < AHEAD; ++s) {
        if constexpr (GATHER) {
          tok_issue(Tk, s + AHEAD);
          S.next(a, Tk, true);
        }
        load_issue(s);
      }
      // step 0's loads have landed (the loads of steps 1 and 2 and their token loads were
      // issued after them)
      vm_wait<2 * NLK>();
    }
    lds_barrier();
    bf16x8 fa[4], fb[8];
    {
#pragma unroll
      for (int j = 0; j < 8; ++j) fb[j] = frag_mn(s_ring + G::OPA, wn * 128 + 16 * j, mn_k0, mn_ff, mn_b);
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = frag_mn(s_ring, 16 * (4 * i + wm), mn_k0, mn_ff, mn_b);
    }

#pragma unroll 1
    for (int s = 0;; ++s) {
      // step s + 1's loads (issued two steps ago; only the next step's were issued after
      // them) have landed, and every wavefront's LDS reads are complete, in particular those
      // of the stage the loads below overwrite (step s - 1's)
      if (loader) vm_wait<NLK>();
      lds_barrier();

      // ---- this step's loads (three steps ahead), the MFMAs of step s and the fragment
      // reads of step s + 1 ----
      if (loader) {
        if constexpr (GATHER) {
          tok_issue(Tk, s + 2 * AHEAD);
          S.next(a, Tk, true);
        }
        load_issue(s + AHEAD);
      }
      mma_pf(fa, fb, s_ring + ((s + 1) & (NSTG - 1)) * G::STGK);

      // ---- advance the compute cursor; finish a tile after its last step ----
      if (Cc.kt + 1 < Cc.nk) {
        ++Cc.kt;
        continue;
      }
      // Stages s and s + 1 are free: every wavefront's reads of them are complete after the
      // barrier below, and the loads that refill them are issued after the barriers of steps
      // s + 1 and s + 2.  Loader w stages its blocks in the 16 KB at (w & 1) 16 KB of stage
      // s + (w >> 1).
      auto pst_of = [&](int v) __attribute__((always_inline)) {
        return s_ring + ((s + (v >> 1)) & (NSTG - 1)) * G::STGK + (v & 1) * 16384;
      };
      lds_barrier();
      vk_epilogue1<KIND>(a, Cc, acc, wm, wn, L, S.nMg, pst_of(wm), s_own);
      lds_barrier();
      if (!loader) vk_epilogue2<KIND>(a, Cc, wm, L, S.nMg, pst_of(wm));
#pragma unroll
      for (int i = 0; i < G::MI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      S.decode(a, Cc, Cc.it + 1);
      while (Cc.valid && Cc.nk == 0) {
        if (!loader) vk_zero<KIND>(a, Cc, wm, L, S.nN, S.nMg);
        S.decode(a, Cc, Cc.it + 1);
      }
      if (!Cc.valid) break;
    }
    // loads past the last tile (all masked) must land before the workgroup's LDS is released
    if (loader) vm_drain();
  }
}

}  // namespace g4

// ------------------------------------------------------------------ host side
template <int KIND>
hipError_t run_gemm_bf16(const gg::Args& a, long long max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const DevInfo d = dev_info();
  long long g = d.cus;
  if (max_tiles < g) g = max_tiles;
  g = (g + 7) / 8 * 8;
  kernel_event(KIND, 0, s);
  hipLaunchKernelGGL((g4::k_gg_bf16<KIND>), dim3((unsigned)g), dim3(g4::NT), 0, s, a, a.counts, a.offsets);
  kernel_event(KIND, 1, s);
  return hipGetLastError();
}

template hipError_t run_gemm_bf16<gg::GATEUP>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::DOWN>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::DH>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::DX>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::DWD>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::DW1>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::GATEUP8>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::DOWN8>(const gg::Args&, long long, hipStream_t);
template hipError_t run_gemm_bf16<gg::DX8>(const gg::Args&, long long, hipStream_t);

}  // namespace moe
