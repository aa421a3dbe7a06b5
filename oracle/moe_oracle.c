/*
 * moe_oracle.c -- plain, slow, CPU reference for the dropless MoE expert-MLP layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file; only the test-suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Every function computes the plain definition of one step, in the order the pages
 * state it, with explicit loops and no blocking, fusion or reordering.  Arithmetic is
 * carried in `real`, which is double unless the file is compiled with
 * -DORACLE_REAL=float (the fp32 variant is only used as a timing baseline).
 *
 * Pages cited (by title, then section):
 *   [GG]  "DeepSeek 계열 MoE 학습 가속: Python expert loop → grouped GEMM"
 *   [EP]  "EP: Expert를 나누고 토큰 보내기"
 *   [SM]  "SonicMoE: IO·타일 인식 최적화로 MoE 학습 가속하기"
 *   [DEP] "Deep EP"
 *
 * Conventions (all arrays row-major, all indices int32):
 *   x [N,H], w_gate/w_up [E,I,H], w_down [E,H,I]  (nn.Linear (out,in) stacked per expert,
 *   [GG] "적용 — fused MoE training forward", step (5)).
 *   A routing assignment ("pair") is (token t, expert e, combine weight w).
 *
 * Return value of every entry point: 0 on success, -1 on a bad argument, -2 on an
 * allocation failure.  No function keeps state between calls.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_REAL
#define ORACLE_REAL double
#endif
typedef ORACLE_REAL real;

#define ORACLE_EXPORT __attribute__((visibility("default")))

ORACLE_EXPORT int oracle_real_bytes(void) { return (int)sizeof(real); }

/* Number of OpenMP threads later parallel regions of this library use, when called from the
 * thread that calls the library (n >= 1); returns the resulting count. */
int oracle_threads(void);
ORACLE_EXPORT int oracle_set_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
  return oracle_threads();
}

/* Number of OpenMP threads a parallel region of this library uses. */
ORACLE_EXPORT int oracle_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

/* ------------------------------------------------------------------------------------
 * Router: top-k selection and combine weights.
 * [DEP] "1) Router": each token's k experts with the largest gate score, returned as an
 * index array and a score array, both [N,k].  The score is softmax(z); the combine
 * weights are the chosen scores renormalised to sum to one (the two weights of [EP]
 * "여러 Expert의 결과도 같은 토큰으로 돌아오기" sum to one).
 *
 *   z[t,e]   = logits[t,e] + bias[e]           (one fp32 add; bias may be NULL)
 *   order    : z descending, then expert id ascending (ties go to the lower id)
 *   P[t,e]   = exp(z[t,e]) / sum_e' exp(z[t,e'])        (full softmax, in real)
 *   w[t,j]   = P[t,idx[t,j]] / sum_j' P[t,idx[t,j']]
 *   probs    : P rounded to fp32 (may be NULL)
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_route_topk(const float* logits, const float* bias, int N, int E, int k,
                                    int32_t* idx, float* w, float* probs) {
  if (N < 0 || E < 1 || k < 1 || k > E || !logits || !idx || !w) return -1;
  float* z = (float*)malloc(sizeof(float) * (size_t)E);
  real* p = (real*)malloc(sizeof(real) * (size_t)E);
  char* taken = (char*)malloc((size_t)E);
  if (!z || !p || !taken) { free(z); free(p); free(taken); return -2; }
  for (int t = 0; t < N; ++t) {
    for (int e = 0; e < E; ++e) z[e] = bias ? logits[(size_t)t * E + e] + bias[e] : logits[(size_t)t * E + e];
    /* selection: k passes, each taking the best remaining expert under the total order */
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || z[e] > z[best]) best = e; /* strict '>' keeps the lower id on ties */
      }
      taken[best] = 1;
      idx[(size_t)t * k + j] = best;
    }
    /* full softmax over all E experts */
    real zmax = (real)z[0];
    for (int e = 1; e < E; ++e)
      if ((real)z[e] > zmax) zmax = (real)z[e];
    real s = 0;
    for (int e = 0; e < E; ++e) { p[e] = exp((real)z[e] - zmax); s += p[e]; }
    for (int e = 0; e < E; ++e) p[e] /= s;
    if (probs)
      for (int e = 0; e < E; ++e) probs[(size_t)t * E + e] = (float)p[e];
    /* renormalise over the chosen k */
    real sk = 0;
    for (int j = 0; j < k; ++j) sk += p[idx[(size_t)t * k + j]];
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = (float)(p[idx[(size_t)t * k + j]] / sk);
  }
  free(z); free(p); free(taken);
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Permute (routing plan).
 * [GG] "적용 — fused MoE training forward", steps (1)-(3): flatten the top-k ids, sort them
 * by expert so each expert's rows form one contiguous slice, and count rows per expert
 * (bincount).  [DEP] "2) Dispatch" (ragged vs padding table, row "추가 정보"): the ragged
 * layout carries offset and index metadata.  The sort is stable by token index.
 *
 *   rows are appended for e = 0..E-1, then t = 0..N-1, then j = 0..k-1 with idx[t,j] == e:
 *   row_token[r] = t, row_w[r] = w[t,j], row_pair[r] = t*k + j
 *   counts[e] = rows of expert e, offsets = exclusive prefix sum (offsets[E] = N*k)
 *   tok_ptr[t] = t*k; tok_rows[tok_ptr[t] ..] = rows of token t in ascending row order
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_permute(const int32_t* idx, const float* w, int N, int E, int k,
                                 int32_t* counts, int32_t* offsets, int32_t* row_token, float* row_w,
                                 int32_t* row_pair, int32_t* tok_ptr, int32_t* tok_rows) {
  if (N < 0 || E < 1 || k < 1 || k > E || !idx || !w || !counts || !offsets || !row_token ||
      !row_w || !row_pair || !tok_ptr || !tok_rows)
    return -1;
  int32_t r = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = r;
    for (int t = 0; t < N; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[(size_t)t * k + j] == e) {
          row_token[r] = t;
          row_w[r] = w[(size_t)t * k + j];
          row_pair[r] = t * k + j;
          ++r;
        }
    counts[e] = r - offsets[e];
  }
  offsets[E] = r;
  for (int t = 0; t <= N; ++t) tok_ptr[t] = t * k;
  int32_t* fill = (int32_t*)calloc((size_t)N + 1, sizeof(int32_t));
  if (!fill) return -2;
  for (int32_t q = 0; q < r; ++q) {
    int t = row_token[q];
    tok_rows[tok_ptr[t] + fill[t]++] = q;
  }
  free(fill);
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Token rounding.
 * [SM] "5 기여 ③ Token Rounding 라우팅": first the ordinary top-K token-choice routing; then,
 * per expert, order tokens by score and round the expert's count to the nearest multiple
 * of Mtile, padding with the best-scoring tokens when short and dropping the worst when
 * over.  Readings where the page is silent:
 *   score        = P[t,e], the full softmax probability (the router's score)
 *   target       r_e = Mtile * floor((c_e + Mtile/2) / Mtile)   (a half rounds up),
 *                clamped to the largest multiple of Mtile that is <= N
 *   keep/pad     order all N tokens by (routed to e first, P[t,e] descending, t ascending)
 *                and take the first r_e: this keeps the r_e best routed tokens when
 *                r_e <= c_e, and adds the best unrouted ones when r_e > c_e
 *   weight       P[t,e] / S_t with S_t = sum_j P[t,idx[t,j]] (the token's top-k
 *                normaliser); no renormalisation after rounding
 *   rows         ascending token index within an expert; row_pair = t*k+j for routed
 *                pairs and -1 for padded ones; tok_ptr/tok_rows as in the top-k plan
 * `probs` are the fp32 probabilities that the ordering uses (given, not recomputed), so the
 * plan is a pure function of (probs, idx).  Returns the row count M (>= 0) or < 0 on error.
 * ---------------------------------------------------------------------------------- */
typedef struct { int t; int routed; float p; } tr_cand;

static int tr_cmp(const void* a, const void* b) {
  const tr_cand* x = (const tr_cand*)a;
  const tr_cand* y = (const tr_cand*)b;
  if (x->routed != y->routed) return x->routed ? -1 : 1;
  if (x->p != y->p) return x->p > y->p ? -1 : 1;
  return x->t < y->t ? -1 : (x->t > y->t ? 1 : 0);
}

ORACLE_EXPORT int oracle_token_round(const float* probs, const int32_t* idx, int N, int E, int k, int mtile,
                                     int M_cap, int32_t* counts, int32_t* offsets, int32_t* row_token,
                                     float* row_w, int32_t* row_pair, int32_t* tok_ptr, int32_t* tok_rows) {
  if (N < 0 || E < 1 || k < 1 || k > E || mtile < 1 || !probs || !idx || !counts || !offsets ||
      !row_token || !row_w || !row_pair || !tok_ptr || !tok_rows)
    return -1;
  int32_t* c = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  tr_cand* cand = (tr_cand*)malloc(sizeof(tr_cand) * ((size_t)N + 1));
  char* sel = (char*)malloc((size_t)N + 1);
  int32_t* tcount = (int32_t*)calloc((size_t)N + 1, sizeof(int32_t));
  if (!c || !cand || !sel || !tcount) { free(c); free(cand); free(sel); free(tcount); return -2; }
  for (size_t q = 0; q < (size_t)N * k; ++q) c[idx[q]]++;
  const int rmax = mtile * (N / mtile);
  int32_t r = 0;
  for (int e = 0; e < E; ++e) {
    int re = mtile * ((c[e] + mtile / 2) / mtile);
    if (re > rmax) re = rmax;
    offsets[e] = r;
    if (r + re > M_cap) { free(c); free(cand); free(sel); free(tcount); return -1; }
    for (int t = 0; t < N; ++t) {
      int routed = 0;
      for (int j = 0; j < k; ++j) routed |= (idx[(size_t)t * k + j] == e);
      cand[t].t = t;
      cand[t].routed = routed;
      cand[t].p = probs[(size_t)t * E + e];
    }
    qsort(cand, (size_t)N, sizeof(tr_cand), tr_cmp);
    memset(sel, 0, (size_t)N);
    for (int q = 0; q < re; ++q) sel[cand[q].t] = 1;
    for (int t = 0; t < N; ++t) {
      if (!sel[t]) continue;
      real st = 0;
      int slot = -1;
      for (int j = 0; j < k; ++j) {
        st += (real)probs[(size_t)t * E + idx[(size_t)t * k + j]];
        if (idx[(size_t)t * k + j] == e) slot = j;
      }
      row_token[r] = t;
      row_w[r] = (float)((real)probs[(size_t)t * E + e] / st);
      row_pair[r] = slot >= 0 ? t * k + slot : -1;
      tcount[t]++;
      ++r;
    }
    counts[e] = r - offsets[e];
  }
  offsets[E] = r;
  tok_ptr[0] = 0;
  for (int t = 0; t < N; ++t) tok_ptr[t + 1] = tok_ptr[t] + tcount[t];
  memset(tcount, 0, sizeof(int32_t) * ((size_t)N + 1));
  for (int32_t q = 0; q < r; ++q) {
    int t = row_token[q];
    tok_rows[tok_ptr[t] + tcount[t]++] = q;
  }
  free(c); free(cand); free(sel); free(tcount);
  return (int)r;
}

/* ------------------------------------------------------------------------------------
 * Capacity plan (drop policy of the capacity-based layout).
 * [DEP] "Drop/Padding 방식": the tokens assigned to each expert are lined up and cut at the
 * expert's capacity C; the rest are dropped (padding up to C only matters for the dense
 * E x C x H layout; this plan keeps the ragged layout, so nothing is padded).  The line-up
 * order is the drop policy the same section names (Megatron-LM's "probs" or "position"):
 *   policy 0 (position): token index ascending
 *   policy 1 (probs)   : P[t,e] descending, then token index ascending
 * Kept pairs keep their top-k weight w[t,j] (no renormalisation); rows ascend by token within
 * an expert; row_pair = t*k + j; tok_ptr / tok_rows list each token's kept rows.  `probs` is
 * read only by policy 1.  Returns the row count M (>= 0) or < 0 on error.
 * ---------------------------------------------------------------------------------- */
typedef struct { int t; int j; float p; } cap_cand;
static int cap_policy;
static int cap_cmp(const void* a, const void* b) {
  const cap_cand* x = (const cap_cand*)a;
  const cap_cand* y = (const cap_cand*)b;
  if (cap_policy == 1 && x->p != y->p) return x->p > y->p ? -1 : 1;
  return x->t < y->t ? -1 : (x->t > y->t ? 1 : 0);
}
static int cap_tok_cmp(const void* a, const void* b) {
  const cap_cand* x = (const cap_cand*)a;
  const cap_cand* y = (const cap_cand*)b;
  return x->t < y->t ? -1 : (x->t > y->t ? 1 : 0);
}

ORACLE_EXPORT int oracle_capacity_plan(const float* probs, const int32_t* idx, const float* w, int N, int E, int k,
                                       int C, int policy, int M_cap, int32_t* counts, int32_t* offsets,
                                       int32_t* row_token, float* row_w, int32_t* row_pair, int32_t* tok_ptr,
                                       int32_t* tok_rows) {
  if (N < 0 || E < 1 || k < 1 || k > E || C < 0 || (policy != 0 && policy != 1) || !idx || !w || !counts ||
      !offsets || !row_token || !row_w || !row_pair || !tok_ptr || !tok_rows)
    return -1;
  if (policy == 1 && !probs) return -1;
  cap_cand* cand = (cap_cand*)malloc(sizeof(cap_cand) * ((size_t)N + 1));
  int32_t* tcount = (int32_t*)calloc((size_t)N + 1, sizeof(int32_t));
  if (!cand || !tcount) { free(cand); free(tcount); return -2; }
  cap_policy = policy;
  int32_t r = 0;
  for (int e = 0; e < E; ++e) {
    /* the tokens assigned to expert e, lined up by the policy */
    int n = 0;
    for (int t = 0; t < N; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[(size_t)t * k + j] == e) {
          cand[n].t = t;
          cand[n].j = j;
          cand[n].p = policy == 1 ? probs[(size_t)t * E + e] : 0.f;
          ++n;
        }
    qsort(cand, (size_t)n, sizeof(cap_cand), cap_cmp);
    const int keep = n < C ? n : C;
    /* the kept ones, in token order */
    qsort(cand, (size_t)keep, sizeof(cap_cand), cap_tok_cmp);
    offsets[e] = r;
    if (r + keep > M_cap) { free(cand); free(tcount); return -1; }
    for (int q = 0; q < keep; ++q) {
      const int t = cand[q].t, j = cand[q].j;
      row_token[r] = t;
      row_w[r] = w[(size_t)t * k + j];
      row_pair[r] = t * k + j;
      tcount[t]++;
      ++r;
    }
    counts[e] = keep;
  }
  offsets[E] = r;
  tok_ptr[0] = 0;
  for (int t = 0; t < N; ++t) tok_ptr[t + 1] = tok_ptr[t] + tcount[t];
  memset(tcount, 0, sizeof(int32_t) * ((size_t)N + 1));
  for (int32_t q = 0; q < r; ++q) {
    const int t = row_token[q];
    tok_rows[tok_ptr[t] + tcount[t]++] = q;
  }
  free(cand); free(tcount);
  return (int)r;
}

/* ------------------------------------------------------------------------------------
 * Expert MLP pieces shared by forward and backward (plain definitions).
 * The expert is the SwiGLU MLP named by [GG] "적용" step (6) (gate -> up -> down) and
 * [SM] "4.2 Epilogue 융합" (SwiGLU): a_i = silu(g_i) * u_i with silu(g) = g * sigmoid(g).
 * ---------------------------------------------------------------------------------- */
static real sigmoid_r(real g) { return (real)1 / ((real)1 + exp(-g)); }

/* g = W_gate[e] x, u = W_up[e] x, a = silu(g) * u   (vectors of length I) */
static void expert_hidden(const float* xt, const float* wg, const float* wu, int H, int I, int e,
                          real* g, real* u, real* a) {
  for (int i = 0; i < I; ++i) {
    const float* rg = wg + ((size_t)e * I + i) * H;
    const float* ru = wu + ((size_t)e * I + i) * H;
    real sg = 0, su = 0;
    for (int h = 0; h < H; ++h) {
      sg += (real)rg[h] * (real)xt[h];
      su += (real)ru[h] * (real)xt[h];
    }
    g[i] = sg;
    u[i] = su;
    a[i] = sg * sigmoid_r(sg) * su;
  }
}

/* y = W_down[e] a   (vector of length H) */
static void expert_out(const real* a, const float* wd, int H, int I, int e, real* y) {
  for (int h = 0; h < H; ++h) {
    const float* rd = wd + ((size_t)e * H + h) * I;
    real s = 0;
    for (int i = 0; i < I; ++i) s += (real)rd[i] * a[i];
    y[h] = s;
  }
}

/* CSR grouping of pairs by a key (token or expert); plain counting. */
static int group_pairs(int P, const int32_t* key, int nkeys, int32_t** ptr_out, int32_t** list_out) {
  int32_t* ptr = (int32_t*)calloc((size_t)nkeys + 1, sizeof(int32_t));
  int32_t* list = (int32_t*)malloc(sizeof(int32_t) * ((size_t)P + 1));
  int32_t* fill = (int32_t*)calloc((size_t)nkeys + 1, sizeof(int32_t));
  if (!ptr || !list || !fill) { free(ptr); free(list); free(fill); return -2; }
  for (int p = 0; p < P; ++p) ptr[key[p] + 1]++;
  for (int q = 0; q < nkeys; ++q) ptr[q + 1] += ptr[q];
  for (int p = 0; p < P; ++p) list[ptr[key[p]] + fill[key[p]]++] = p;
  free(fill);
  *ptr_out = ptr;
  *list_out = list;
  return 0;
}

static int check_pairs(int N, int E, int P, const int32_t* pt, const int32_t* pe) {
  for (int p = 0; p < P; ++p)
    if (pt[p] < 0 || pt[p] >= N || pe[p] < 0 || pe[p] >= E) return -1;
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Layer forward.
 * For every token t and each of its pairs (e, w):
 *   y = W_down[e] (silu(W_gate[e] x_t) * (W_up[e] x_t));   out[t] += w * y
 * [EP] "여러 Expert의 결과도 같은 토큰으로 돌아오기" (weighted sum of the experts' outputs back
 * at the token), [DEP] "3) Combine".  A token with no pairs gets out[t] = 0.
 * out is [N,H] in double.  Pairs need not cover every token (sampled checks pass a subset).
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_layer_fwd(const float* x, const float* wg, const float* wu, const float* wd, int N,
                                   int H, int I, int E, int P, const int32_t* pair_t, const int32_t* pair_e,
                                   const float* pair_w, double* out) {
  if (N < 0 || H < 1 || I < 1 || E < 1 || P < 0 || !x || !wg || !wu || !wd || !out) return -1;
  if (P > 0 && (!pair_t || !pair_e || !pair_w)) return -1;
  if (check_pairs(N, E, P, pair_t, pair_e)) return -1;
  memset(out, 0, sizeof(double) * (size_t)N * H);
  int32_t *tptr, *tlist;
  if (group_pairs(P, pair_t, N, &tptr, &tlist)) return -2;
  int fail = 0;
#pragma omp parallel
  {
    real* g = (real*)malloc(sizeof(real) * (size_t)I);
    real* u = (real*)malloc(sizeof(real) * (size_t)I);
    real* a = (real*)malloc(sizeof(real) * (size_t)I);
    real* y = (real*)malloc(sizeof(real) * (size_t)H);
    if (!g || !u || !a || !y) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int t = 0; t < N; ++t) {
        for (int q = tptr[t]; q < tptr[t + 1]; ++q) {
          int p = tlist[q];
          int e = pair_e[p];
          expert_hidden(x + (size_t)t * H, wg, wu, H, I, e, g, u, a);
          expert_out(a, wd, H, I, e, y);
          for (int h = 0; h < H; ++h) out[(size_t)t * H + h] += (double)((real)pair_w[p] * y[h]);
        }
      }
    }
    free(g); free(u); free(a); free(y);
  }
  free(tptr); free(tlist);
  return fail ? -2 : 0;
}

/* ------------------------------------------------------------------------------------
 * Layer backward, textbook chain rule per pair (it does not use the fused algebra of the
 * GPU path).  With dy = w * dOut[t]:
 *   dS[p]     = <dOut[t], y>              gradient w.r.t. the combine weight w of pair p
 *                                          ([SM] "3 기여 ①": router gradient dS)
 *   da        = W_down[e]^T dy,            dW_down[e] += dy (x) a
 *   dg_i      = da_i * u_i * s_i * (1 + g_i (1 - s_i)),  s = sigmoid(g)
 *   du_i      = da_i * silu(g_i)
 *   dW_gate[e] += dg (x) x_t,   dW_up[e] += du (x) x_t
 *   dx[t]     += W_gate[e]^T dg + W_up[e]^T du
 * Experts without pairs get dW = 0.  dx excludes the router path.  Any output pointer may
 * be NULL to skip that part.  dx [N,H], dW_gate/dW_up [E,I,H], dW_down [E,H,I], dS [P],
 * all double; dh [P, 2I] = [dg | du] of every pair, double.
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_layer_bwd(const float* dout, const float* x, const float* wg, const float* wu,
                                   const float* wd, int N, int H, int I, int E, int P, const int32_t* pair_t,
                                   const int32_t* pair_e, const float* pair_w, double* dx, double* dwg,
                                   double* dwu, double* dwd, double* ds, double* dh) {
  if (N < 0 || H < 1 || I < 1 || E < 1 || P < 0 || !dout || !x || !wg || !wu || !wd) return -1;
  if (P > 0 && (!pair_t || !pair_e || !pair_w)) return -1;
  if (check_pairs(N, E, P, pair_t, pair_e)) return -1;
  const size_t PI = (size_t)P * I;
  real* A = (real*)malloc(sizeof(real) * (PI + 1));
  real* DG = (real*)malloc(sizeof(real) * (PI + 1));
  real* DU = (real*)malloc(sizeof(real) * (PI + 1));
  if (!A || !DG || !DU) { free(A); free(DG); free(DU); return -2; }
  int fail = 0;

  /* phase 1, per pair: forward recompute, dS, da, dg, du */
#pragma omp parallel
  {
    real* g = (real*)malloc(sizeof(real) * (size_t)I);
    real* u = (real*)malloc(sizeof(real) * (size_t)I);
    real* y = (real*)malloc(sizeof(real) * (size_t)H);
    real* dy = (real*)malloc(sizeof(real) * (size_t)H);
    real* da = (real*)malloc(sizeof(real) * (size_t)I);
    if (!g || !u || !y || !dy || !da) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int p = 0; p < P; ++p) {
        const int t = pair_t[p], e = pair_e[p];
        const real w = (real)pair_w[p];
        const float* dot = dout + (size_t)t * H;
        real* a = A + (size_t)p * I;
        expert_hidden(x + (size_t)t * H, wg, wu, H, I, e, g, u, a);
        expert_out(a, wd, H, I, e, y);
        real s = 0;
        for (int h = 0; h < H; ++h) s += (real)dot[h] * y[h];
        if (ds) ds[p] = (double)s;
        for (int h = 0; h < H; ++h) dy[h] = w * (real)dot[h];
        for (int i = 0; i < I; ++i) da[i] = 0;
        for (int h = 0; h < H; ++h) {
          const float* rd = wd + ((size_t)e * H + h) * I;
          for (int i = 0; i < I; ++i) da[i] += (real)rd[i] * dy[h];
        }
        for (int i = 0; i < I; ++i) {
          const real sg = sigmoid_r(g[i]);
          DG[(size_t)p * I + i] = da[i] * u[i] * sg * ((real)1 + g[i] * ((real)1 - sg));
          DU[(size_t)p * I + i] = da[i] * g[i] * sg;
        }
      }
    }
    free(g); free(u); free(y); free(dy); free(da);
  }
  if (fail) { free(A); free(DG); free(DU); return -2; }
  if (dh)
    for (size_t p = 0; p < (size_t)P; ++p)
      for (int i = 0; i < I; ++i) {
        dh[p * 2 * I + i] = (double)DG[p * I + i];
        dh[p * 2 * I + I + i] = (double)DU[p * I + i];
      }

  /* phase 2, per token: dx */
  if (dx) {
    memset(dx, 0, sizeof(double) * (size_t)N * H);
    int32_t *tptr, *tlist;
    if (group_pairs(P, pair_t, N, &tptr, &tlist)) { free(A); free(DG); free(DU); return -2; }
#pragma omp parallel
    {
      real* acc = (real*)malloc(sizeof(real) * (size_t)H);
      if (!acc) {
#pragma omp atomic write
        fail = 1;
      } else {
#pragma omp for schedule(dynamic, 4)
        for (int t = 0; t < N; ++t) {
          for (int h = 0; h < H; ++h) acc[h] = 0;
          for (int q = tptr[t]; q < tptr[t + 1]; ++q) {
            const int p = tlist[q], e = pair_e[p];
            for (int i = 0; i < I; ++i) {
              const float* rg = wg + ((size_t)e * I + i) * H;
              const float* ru = wu + ((size_t)e * I + i) * H;
              const real dgi = DG[(size_t)p * I + i], dui = DU[(size_t)p * I + i];
              for (int h = 0; h < H; ++h) acc[h] += (real)rg[h] * dgi + (real)ru[h] * dui;
            }
          }
          for (int h = 0; h < H; ++h) dx[(size_t)t * H + h] = (double)acc[h];
        }
      }
      free(acc);
    }
    free(tptr); free(tlist);
  }

  /* phase 3, per expert and output row: weight gradients */
  if (dwg || dwu || dwd) {
    int32_t *eptr, *elist;
    if (group_pairs(P, pair_e, E, &eptr, &elist)) { free(A); free(DG); free(DU); return -2; }
#pragma omp parallel
    {
      real* acc = (real*)malloc(sizeof(real) * (size_t)(H > I ? H : I));
      if (!acc) {
#pragma omp atomic write
        fail = 1;
      } else {
/* one work item per output row: dW_down[e] row h (items 0 .. H-1 of expert e) or the
         * rows i of dW_gate[e] and dW_up[e] (items H .. H+I-1); each row is summed over the
         * expert's pairs in pair order */
#pragma omp for schedule(dynamic, 1)
        for (long wi = 0; wi < (long)E * (H + I); ++wi) {
          const int e = (int)(wi / (H + I)), r = (int)(wi % (H + I));
          if (r < H) {
            const int h = r;
            if (!dwd) continue;
            for (int i = 0; i < I; ++i) acc[i] = 0;
            for (int q = eptr[e]; q < eptr[e + 1]; ++q) {
              const int p = elist[q];
              const real dyh = (real)pair_w[p] * (real)dout[(size_t)pair_t[p] * H + h];
              const real* a = A + (size_t)p * I;
              for (int i = 0; i < I; ++i) acc[i] += dyh * a[i];
            }
            for (int i = 0; i < I; ++i) dwd[((size_t)e * H + h) * I + i] = (double)acc[i];
            continue;
          }
          const int i = r - H;
          if (dwg) {
            for (int h = 0; h < H; ++h) acc[h] = 0;
            for (int q = eptr[e]; q < eptr[e + 1]; ++q) {
              const int p = elist[q];
              const float* xt = x + (size_t)pair_t[p] * H;
              const real d = DG[(size_t)p * I + i];
              for (int h = 0; h < H; ++h) acc[h] += d * (real)xt[h];
            }
            for (int h = 0; h < H; ++h) dwg[((size_t)e * I + i) * H + h] = (double)acc[h];
          }
          if (dwu) {
            for (int h = 0; h < H; ++h) acc[h] = 0;
            for (int q = eptr[e]; q < eptr[e + 1]; ++q) {
              const int p = elist[q];
              const float* xt = x + (size_t)pair_t[p] * H;
              const real d = DU[(size_t)p * I + i];
              for (int h = 0; h < H; ++h) acc[h] += d * (real)xt[h];
            }
            for (int h = 0; h < H; ++h) dwu[((size_t)e * I + i) * H + h] = (double)acc[h];
          }
        }
      }
      free(acc);
    }
    free(eptr); free(elist);
  }
  free(A); free(DG); free(DU);
  return fail ? -2 : 0;
}

/* ------------------------------------------------------------------------------------
 * Router logits.
 * [DEP] "1) Router" maps the [N,H] hidden states to per-expert scores; the score of
 * expert e is a linear function of the token's hidden state:
 *   logits[t,e] = sum_h x[t,h] * W_r[h,e]   (+ bias[e] when bias is not NULL)
 * accumulated in real in ascending h, rounded once to fp32.  W_r is [H,E].
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_router_logits(const float* x, const float* wr, const float* bias, int N, int H, int E,
                                       float* logits) {
  if (N < 0 || H < 1 || E < 1 || !x || !wr || !logits) return -1;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < N; ++t)
    for (int e = 0; e < E; ++e) {
      real s = 0;
      for (int h = 0; h < H; ++h) s += (real)x[(size_t)t * H + h] * (real)wr[(size_t)h * E + e];
      if (bias) s += (real)bias[e];
      logits[(size_t)t * E + e] = (float)s;
    }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Router backward (the gradient of the combine weights back to the router's inputs).
 * The pages stop at dS, the gradient with respect to the combine weights ([SM] "3 기여 ①":
 * dS = <dA', A>); training the router needs the rest, written out here from the weights'
 * definition.  For token t with top-k set K (idx[t,0..k-1]) and z = logits[t,:] + bias:
 *   every final pair f = (t, e_f) has weight   w_f(z) = exp(z_{e_f}) / sum_{j in K} exp(z_j)
 * (the renormalised top-k softmax; for token-rounding plans the same expression, P_e / S_t,
 * also gives the padded pairs' weights, and dropped pairs simply have no f).  With
 * q_m = exp(z_m) / sum_{j in K} exp(z_j):
 *   dw_f / dz_m = w_f * ([m == e_f] - q_m * [m in K])
 *   dz[t,m]     = sum_f dS_f * dw_f / dz_m          (computed literally, f and m loops)
 * and, because z = x W_r + bias:
 *   dbias[m]    = sum_t dz[t,m]
 *   dW_r[h,m]   = sum_t x[t,h] * dz[t,m]
 *   dx[t,h]     = sum_m dz[t,m] * W_r[h,m]        (the router's share of dx only)
 * The pairs (pair_t, pair_e, pair_ds) list every final pair once; w_f is recomputed from z in
 * real (the plan's fp32 weight is that value rounded).  Outputs are double; dz [N,E],
 * dwr [H,E], dx [N,H], dbias [E]; any of dwr, dx, dbias may be NULL.
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_router_bwd(const float* logits, const float* bias, int N, int E, int k,
                                    const int32_t* idx, int P, const int32_t* pair_t, const int32_t* pair_e,
                                    const float* pair_ds, const float* x, const float* wr, int H, double* dz,
                                    double* dwr, double* dx, double* dbias) {
  if (N < 0 || E < 1 || k < 1 || k > E || P < 0 || H < 1 || !logits || !idx || !dz) return -1;
  if (P > 0 && (!pair_t || !pair_e || !pair_ds)) return -1;
  if ((dwr || dx) && (!x || !wr)) return -1;
  if (check_pairs(N, E, P, pair_t, pair_e)) return -1;
  int32_t *tptr, *tlist;
  if (group_pairs(P, pair_t, N, &tptr, &tlist)) return -2;
  int fail = 0;
#pragma omp parallel
  {
    real* z = (real*)malloc(sizeof(real) * (size_t)E);
    real* q = (real*)malloc(sizeof(real) * (size_t)E);  /* q_m, zero outside K */
    if (!z || !q) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(static)
      for (int t = 0; t < N; ++t) {
        for (int e = 0; e < E; ++e) {
          const float zf = bias ? logits[(size_t)t * E + e] + bias[e] : logits[(size_t)t * E + e];
          z[e] = (real)zf;
          q[e] = 0;
        }
        real zmax = z[idx[(size_t)t * k]];
        for (int j = 1; j < k; ++j)
          if (z[idx[(size_t)t * k + j]] > zmax) zmax = z[idx[(size_t)t * k + j]];
        real sk = 0;
        for (int j = 0; j < k; ++j) sk += exp(z[idx[(size_t)t * k + j]] - zmax);
        for (int j = 0; j < k; ++j) q[idx[(size_t)t * k + j]] = exp(z[idx[(size_t)t * k + j]] - zmax) / sk;
        for (int m = 0; m < E; ++m) {
          real s = 0;
          for (int c = tptr[t]; c < tptr[t + 1]; ++c) {
            const int f = tlist[c], ef = pair_e[f];
            const real wf = exp(z[ef] - zmax) / sk;
            const real dwdz = wf * ((m == ef ? (real)1 : (real)0) - q[m]);
            s += (real)pair_ds[f] * dwdz;
          }
          dz[(size_t)t * E + m] = (double)s;
        }
      }
    }
    free(z); free(q);
  }
  free(tptr); free(tlist);
  if (fail) return -2;
  if (dbias)
    for (int m = 0; m < E; ++m) {
      real s = 0;
      for (int t = 0; t < N; ++t) s += (real)dz[(size_t)t * E + m];
      dbias[m] = (double)s;
    }
  if (dwr) {
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h)
      for (int m = 0; m < E; ++m) {
        real s = 0;
        for (int t = 0; t < N; ++t) s += (real)x[(size_t)t * H + h] * (real)dz[(size_t)t * E + m];
        dwr[(size_t)h * E + m] = (double)s;
      }
  }
  if (dx) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < N; ++t)
      for (int h = 0; h < H; ++h) {
        real s = 0;
        for (int m = 0; m < E; ++m) s += (real)dz[(size_t)t * E + m] * (real)wr[(size_t)h * E + m];
        dx[(size_t)t * H + h] = (double)s;
      }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------
 * MX-FP8: the fine-grained FP8 grouped GEMM of [GG] "한계" (DeepSeek-V3's FP8 grouped GEMM:
 * FP8 operands with scales for small blocks along the contraction dimension).  The pages name
 * it but give no format; the reading here is the OCP microscaling (MX) FP8 layout:
 *   element : e4m3 -- sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field
 *             0 holds the subnormals (m/8) 2^-6; largest finite value 448; codes 0x7F and
 *             0xFF are NaN (never produced here)
 *   block   : 32 consecutive values along the contraction dimension (K) share one scale
 *             X = 2^(c - 127), c an unsigned byte code
 * Quantization rule (the pages give none): X is the smallest power of two with
 * max |v| <= 448 X over the block (no value clips), its code limited to 0..254; each value is
 * stored as v / X rounded to the nearest e4m3 value, ties to the even code.
 * Layout of a quantized [rows, K] matrix: codes q [rows, K] (row-major, one byte each) and
 * scale codes s [rows, KS] with KS = 4 ceil(K / 128): s[r, b] scales q[r, 32b .. 32b+31];
 * entries b >= K / 32 are 0.  K must be a multiple of 32.
 * ---------------------------------------------------------------------------------- */
static double e4m3_value(uint8_t c) {
  const int e = (c >> 3) & 0xF, m = c & 7;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return (c & 0x80) ? -v : v;
}

/* t rounded to the nearest e4m3 value, ties to the even code; requires |t| <= 448 */
static uint8_t e4m3_round(double t) {
  const uint8_t sign = signbit(t) ? 0x80 : 0;
  const double a = fabs(t);
  if (a < ldexp(1.0, -6)) {                 /* subnormal spacing 2^-9 (n = 8 is 2^-6, code 8) */
    const double n = nearbyint(a * 512.0);  /* exact scaling; nearbyint rounds ties to even */
    return sign | (uint8_t)n;
  }
  int ex;
  frexp(a, &ex);                            /* a in [2^(ex-1), 2^ex) */
  int e = ex - 1;
  double n = nearbyint(ldexp(a, 3 - e));    /* mantissa steps of 2^(e-3): n in [8, 16] */
  if (n == 16.0) { e += 1; n = 8.0; }
  return sign | (uint8_t)(((e + 7) << 3) | ((int)n - 8));
}

/* scale exponent of a block: the smallest s in [-127, 127] with amax <= 448 * 2^s */
static int mx_scale_exp(double amax) {
  if (amax == 0.0) return -127;
  int ex;
  const double f = frexp(amax, &ex);        /* amax = f 2^ex, f in [0.5, 1); 448 = 0.875 2^9 */
  int s = f <= 0.875 ? ex - 9 : ex - 8;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

static int mx_ks(int K) { return 4 * ((K + 127) / 128); }

/* quantize one row of K values (K multiple of 32) into codes q[K] and scale codes s[KS] */
static void mx_quantize_row(const float* v, int K, uint8_t* q, uint8_t* s) {
  const int KS = mx_ks(K);
  for (int b = 0; b < KS; ++b) s[b] = 0;
  for (int b = 0; b < K / 32; ++b) {
    double amax = 0;
    for (int j = 0; j < 32; ++j) amax = fmax(amax, fabs((double)v[32 * b + j]));
    const int se = mx_scale_exp(amax);
    s[b] = (uint8_t)(se + 127);
    for (int j = 0; j < 32; ++j) q[32 * b + j] = e4m3_round(ldexp((double)v[32 * b + j], -se));
  }
}

/* the values of the 256 element codes and of the 256 scale codes, from the definitions above
 * (filled once, before any parallel region) */
static double mx_elem_tab[256], mx_scale_tab[256];
static int mx_tab_ready = 0;
static void mx_tables(void) {
  if (mx_tab_ready) return;
  for (int c = 0; c < 256; ++c) {
    mx_elem_tab[c] = e4m3_value((uint8_t)c);
    mx_scale_tab[c] = ldexp(1.0, c - 127);
  }
  mx_tab_ready = 1;
}

/* value of element k of row r of a quantized matrix (mx_tables() called first) */
static double mx_value(const uint8_t* q, const uint8_t* s, int K, long r, int k) {
  return mx_elem_tab[q[(size_t)r * K + k]] * mx_scale_tab[s[(size_t)r * mx_ks(K) + k / 32]];
}

/* Quantize src [rows, K] (fp32 values) into q [rows, K] and s [rows, KS]. */
ORACLE_EXPORT int oracle_quantize_mxfp8(const float* src, long rows, int K, uint8_t* q, uint8_t* s) {
  if (rows < 0 || K < 32 || K % 32 != 0 || (rows > 0 && (!src || !q || !s))) return -1;
  const int KS = mx_ks(K);
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) mx_quantize_row(src + (size_t)r * K, K, q + (size_t)r * K, s + (size_t)r * KS);
  return 0;
}

/* ------------------------------------------------------------------------------------
 * Layer forward with MX-FP8 operands.  x (q, s) [N, H]; W_gate, W_up (q, s) [E*I, H]
 * (expert e's row i is row e*I + i); W_down (q, s) [E*H, I].  For every pair (t, e, w):
 *   g_i = sum_h W_gate[e,i,h] x[t,h],  u_i = sum_h W_up[e,i,h] x[t,h]   (dequantized values)
 *   a_i = silu(g_i) u_i, rounded to fp32, then quantized as one row of I values (MX-FP8)
 *   y_h = sum_i W_down[e,h,i] a~_i   (a~: the dequantized quantized a)
 *   out[t] += w y
 * The quantization of a is a decision taken in fp32 (the precision the layer's kernels hold
 * a in).  Optional per-pair outputs (NULL to skip): gu [P, 2I] = [g | u] in double, and the
 * quantized a: aq [P, I] codes and as [P, KS(I)] scale codes.  H and I multiples of 32.
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_layer_fwd_mxfp8(const uint8_t* xq, const uint8_t* xs, const uint8_t* gq, const uint8_t* gs,
                                         const uint8_t* uq, const uint8_t* us, const uint8_t* dq, const uint8_t* dsc,
                                         int N, int H, int I, int E, int P, const int32_t* pair_t,
                                         const int32_t* pair_e, const float* pair_w, double* out, double* gu,
                                         uint8_t* aq, uint8_t* as) {
  if (N < 0 || H < 32 || I < 32 || H % 32 || I % 32 || E < 1 || P < 0 || !out) return -1;
  if (N > 0 && (!xq || !xs)) return -1;
  if (!gq || !gs || !uq || !us || !dq || !dsc) return -1;
  if (P > 0 && (!pair_t || !pair_e || !pair_w)) return -1;
  if (check_pairs(N, E, P, pair_t, pair_e)) return -1;
  memset(out, 0, sizeof(double) * (size_t)N * H);
  mx_tables();
  int32_t *tptr, *tlist;
  if (group_pairs(P, pair_t, N, &tptr, &tlist)) return -2;
  const int KSI = mx_ks(I);
  int fail = 0;
#pragma omp parallel
  {
    real* xv = (real*)malloc(sizeof(real) * (size_t)H);
    real* g = (real*)malloc(sizeof(real) * (size_t)I);
    real* u = (real*)malloc(sizeof(real) * (size_t)I);
    float* a32 = (float*)malloc(sizeof(float) * (size_t)I);
    uint8_t* aqr = (uint8_t*)malloc((size_t)I);
    uint8_t* asr = (uint8_t*)malloc((size_t)KSI);
    if (!xv || !g || !u || !a32 || !aqr || !asr) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int t = 0; t < N; ++t) {
        if (tptr[t] == tptr[t + 1]) continue;
        for (int h = 0; h < H; ++h) xv[h] = (real)mx_value(xq, xs, H, t, h);
        for (int q = tptr[t]; q < tptr[t + 1]; ++q) {
          const int p = tlist[q], e = pair_e[p];
          for (int i = 0; i < I; ++i) {
            const long row = (long)e * I + i;
            real sg = 0, su = 0;
            for (int h = 0; h < H; ++h) {
              sg += (real)mx_value(gq, gs, H, row, h) * xv[h];
              su += (real)mx_value(uq, us, H, row, h) * xv[h];
            }
            g[i] = sg;
            u[i] = su;
            a32[i] = (float)(sg * sigmoid_r(sg) * su);
          }
          mx_quantize_row(a32, I, aqr, asr);
          for (int h = 0; h < H; ++h) {
            const long row = (long)e * H + h;
            real y = 0;
            for (int i = 0; i < I; ++i)
              y += (real)mx_value(dq, dsc, I, row, i) * (real)(mx_elem_tab[aqr[i]] * mx_scale_tab[asr[i / 32]]);
            out[(size_t)t * H + h] += (double)((real)pair_w[p] * y);
          }
          if (gu)
            for (int i = 0; i < I; ++i) {
              gu[(size_t)p * 2 * I + i] = (double)g[i];
              gu[(size_t)p * 2 * I + I + i] = (double)u[i];
            }
          if (aq) memcpy(aq + (size_t)p * I, aqr, (size_t)I);
          if (as) memcpy(as + (size_t)p * KSI, asr, (size_t)KSI);
        }
      }
    }
    free(xv); free(g); free(u); free(a32); free(aqr); free(asr);
  }
  free(tptr); free(tlist);
  return fail ? -2 : 0;
}


/* ------------------------------------------------------------------------------------
 * The backward's dX product on MX-FP8 operands (the FP8 grouped GEMM of [GG] "한계" applied
 * to dX = dH W).  For every pair p (token t, expert e):
 *   dh~ = the pair's row dh[p] = [dg | du] (2I fp32 values) quantized as one MX-FP8 row
 *   dx[t, h] += sum_k dh~[k] wt~[e, h, k]
 * where wt (q, s) [E*H, 2I] holds, as row e*H + h, expert e's [W_gate^T | W_up^T] row h
 * (W_gate[e][i][h] for k = i < I, then W_up[e][k - I][h]) quantized along its 2I values, and ~
 * marks dequantized values.  The quantization of dh is a decision taken on the fp32 values the
 * caller passes.  Optional dhq [P, 2I] / dhs [P, KS(2I)] (NULL to skip): the quantized rows.
 * dx [N, H] double.  H and I multiples of 32.
 * ---------------------------------------------------------------------------------- */
ORACLE_EXPORT int oracle_dx_mxfp8(const float* dh, const uint8_t* wq, const uint8_t* ws, int N, int H, int I, int E,
                                  int P, const int32_t* pair_t, const int32_t* pair_e, double* dx, uint8_t* dhq,
                                  uint8_t* dhs) {
  if (N < 0 || H < 32 || I < 32 || H % 32 || I % 32 || E < 1 || P < 0 || !dx || !wq || !ws) return -1;
  if (P > 0 && (!dh || !pair_t || !pair_e)) return -1;
  if (check_pairs(N, E, P, pair_t, pair_e)) return -1;
  memset(dx, 0, sizeof(double) * (size_t)N * H);
  mx_tables();
  int32_t *tptr, *tlist;
  if (group_pairs(P, pair_t, N, &tptr, &tlist)) return -2;
  const int K = 2 * I, KS = mx_ks(K);
  int fail = 0;
#pragma omp parallel
  {
    uint8_t* q = (uint8_t*)malloc((size_t)K);
    uint8_t* sc = (uint8_t*)malloc((size_t)KS);
    real* v = (real*)malloc(sizeof(real) * (size_t)K);
    if (!q || !sc || !v) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int t = 0; t < N; ++t) {
        for (int c = tptr[t]; c < tptr[t + 1]; ++c) {
          const int p = tlist[c], e = pair_e[p];
          mx_quantize_row(dh + (size_t)p * K, K, q, sc);
          for (int k = 0; k < K; ++k) v[k] = (real)(mx_elem_tab[q[k]] * mx_scale_tab[sc[k / 32]]);
          for (int h = 0; h < H; ++h) {
            const long row = (long)e * H + h;
            real acc = 0;
            for (int k = 0; k < K; ++k) acc += (real)mx_value(wq, ws, K, row, k) * v[k];
            dx[(size_t)t * H + h] += (double)acc;
          }
          if (dhq) memcpy(dhq + (size_t)p * K, q, (size_t)K);
          if (dhs) memcpy(dhs + (size_t)p * KS, sc, (size_t)KS);
        }
      }
    }
    free(q); free(sc); free(v);
  }
  free(tptr); free(tlist);
  return fail ? -2 : 0;
}
