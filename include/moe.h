/*
 * moe.h -- C ABI of libmoe.so: the dropless Mixture-of-Experts expert-MLP layer on one
 * MI355X (gfx950), forward and backward.
 *
 * Pages cited (by title, then section):
 *   [GG]  "DeepSeek 계열 MoE 학습 가속: Python expert loop → grouped GEMM"
 *   [EP]  "EP: Expert를 나누고 토큰 보내기"
 *   [SM]  "SonicMoE: IO·타일 인식 최적화로 MoE 학습 가속하기"
 *   [DEP] "Deep EP"
 *
 * General contract (applies to every entry point):
 *  - Array arguments are DEVICE pointers unless stated otherwise.  The caller allocates and
 *    owns every buffer, including the workspace, and keeps them alive until the work queued
 *    on `stream` has finished.  The library never allocates, frees or synchronises on these
 *    paths, and keeps no state between calls except a per-thread error string, a
 *    per-device cache of device properties and the optional kernel-event registry of
 *    moe_set_kernel_events().
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.  All work is
 *    queued on that stream in order; nothing is copied back to the host.
 *  - Layouts are row-major.  Expert weights are stacked nn.Linear (out, in) matrices,
 *    [GG] "적용 — fused MoE training forward" step (5):
 *        w_gate, w_up : [E, I, H]      w_down : [E, H, I]
 *  - Element type: x, weights, dout, hcache, y, out, dx and dW share one moe_dtype
 *    (MOE_F32 or MOE_BF16, bf16 values rounded to nearest even on every store).  Logits,
 *    bias, combine weights, probabilities and dS are always fp32; indices are int32.
 *    Contractions accumulate in fp32.
 *  - H and I must be multiples of 8 and every data pointer 16-byte aligned, else
 *    MOE_EUNSUPPORTED.  1 <= k <= E <= 1024; N >= 0 (N == 0 is a valid empty call).
 *  - Size limit of the grouped-GEMM calls (moe_grouped_gemm_fwd, moe_layer_bwd): their
 *    kernels address each of these tensors with 32-bit byte offsets, so each must be smaller
 *    than 2 GiB, else MOE_EUNSUPPORTED: x and dout (N*H elements), one expert's weight or
 *    weight-gradient matrix (I*H elements), the row activations hcache and dH (M_cap*2I
 *    elements) and the plan's row arrays (4*M_cap bytes).
 *  - Outputs are always overwritten, never accumulated into.
 *  - Errors: arguments are validated before anything is queued; on failure nothing is
 *    queued and moe_last_error() describes the problem.  MOE_EHIP reports a launch error
 *    seen right after a launch.  Faults inside kernels surface at the caller's next
 *    synchronisation, as with any stream-ordered HIP library.
 *  - Integer outputs (routing indices, counts, offsets, row lists) are deterministic; the
 *    floating-point outputs are deterministic too (no atomics; every reduction has a fixed
 *    order), so two identical calls give bitwise identical results.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null pointer, size out of range, inconsistent plan */
  MOE_EUNSUPPORTED = 2,  /* alignment, H/I not multiples of 8, unknown dtype */
  MOE_EWORKSPACE = 3,    /* workspace smaller than moe_workspace_bytes() */
  MOE_EHIP = 4           /* HIP runtime error while queueing work */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum moe_plan_kind {
  MOE_PLAN_TOPK = 0,     /* plain top-k: exactly N*k rows */
  MOE_PLAN_TR = 1,       /* token rounding: per-expert rows rounded to multiples of mtile */
  MOE_PLAN_CAP = 2       /* capacity: at most mtile (= the capacity C) rows per expert */
} moe_plan_kind;

typedef enum moe_cap_policy {
  MOE_CAP_POSITION = 0,  /* keep an expert's first C tokens in token order */
  MOE_CAP_PROBS = 1      /* keep its C tokens of largest probability P[t,e] (ties: lower token) */
} moe_cap_policy;

typedef enum moe_op {
  MOE_OP_PERMUTE = 0,
  MOE_OP_ROUTE_TR = 1,
  MOE_OP_GEMM_FWD = 2,
  MOE_OP_LAYER_BWD = 3,
  MOE_OP_ROUTER_BWD = 4,
  MOE_OP_ROUTER_LOGITS = 5,
  MOE_OP_GEMM_FWD_MXFP8 = 6,
  MOE_OP_LAYER_BWD_MXFP8 = 7
} moe_op;

/*
 * Routing plan: the ragged, expert-sorted layout with its offset and index metadata
 * ([DEP] "2) Dispatch", ragged-vs-padding table, row "추가 정보"; [GG] "적용" steps (1)-(3)).
 * A host struct of caller-owned device pointers.  Rows are grouped by expert (expert e
 * owns rows offsets[e] .. offsets[e+1]-1) and, inside an expert, ascend by token index.
 *
 *   counts    int32 [E]       rows per expert
 *   offsets   int32 [E+1]     exclusive prefix sum of counts; offsets[E] = M (rows in use)
 *   row_token int32 [M_cap]   token of each row
 *   row_w     fp32  [M_cap]   combine weight of each row
 *   row_pair  int32 [M_cap]   t*k + j for the row made from topk slot j of token t;
 *                             -1 for a row added by token rounding (padding)
 *   tok_ptr   int32 [N+1]     token t owns tok_rows[tok_ptr[t] .. tok_ptr[t+1]-1]
 *   tok_rows  int32 [M_cap]   rows of each token, ascending (then -1 in the slots of pairs
 *                             moe_permute skipped, see there)
 *
 * M_cap is the row capacity of the row arrays, of hcache/y and of the bwd row buffers;
 * use moe_plan_rows_cap().  For MOE_PLAN_TOPK tok_ptr[t] = t*k, and M = N*k exactly when
 * every pair is valid (always, for the router's own selection).
 */
typedef struct moe_plan {
  int32_t kind;      /* moe_plan_kind */
  int32_t N, E, k;
  int32_t M_cap;
  int32_t mtile;     /* MOE_PLAN_TR: rounding granule; MOE_PLAN_CAP: capacity C; 0 for top-k */
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  float* row_w;
  int32_t* row_pair;
  int32_t* tok_ptr;
  int32_t* tok_rows;
} moe_plan;

/* Row capacity a plan of this kind needs: N*k for top-k; N*k + E*(mtile/2) for token
 * rounding (rounding to the nearest multiple adds at most mtile/2 rows per expert);
 * min(N*k, E*C) for a capacity plan (mtile = C).  Returns -1 for invalid arguments.
 * Host-only, no GPU needed. */
int64_t moe_plan_rows_cap(int32_t kind, int32_t N, int32_t E, int32_t k, int32_t mtile);

/* Bytes of workspace an operation needs (host-only, no GPU needed).  M_cap is the plan's
 * row capacity (ignored for MOE_OP_PERMUTE).  Returns 0 if the arguments are invalid;
 * a valid operation may also need 0 bytes only if it has no workspace (none do). */
size_t moe_workspace_bytes(moe_op op, moe_dtype dt, int32_t N, int32_t E, int32_t k, int32_t H,
                           int32_t I, int32_t M_cap);

/* Human-readable description of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

/*
 * Router top-k.  [DEP] "1) Router": for each of N tokens, the k experts with the largest
 * score, returned as index and weight arrays [N,k].
 *   z[t,e] = logits[t,e] + bias[e]              (bias may be NULL; one fp32 add)
 *   slot j of token t = the j-th expert in the order (z descending, expert id ascending);
 *                       -0 and +0 compare equal and tie; inputs must be finite
 *   topk_w[t,j] = exp(z_j - z_max) / sum over the chosen k of exp(z - z_max)
 *                       (softmax over all E renormalised over the chosen k; the full
 *                        denominator cancels)
 *   probs[t,e]  = softmax over all E of z[t,:]  (optional: NULL skips it)
 * logits fp32 [N,E], bias fp32 [E] or NULL, topk_idx int32 [N,k], topk_w fp32 [N,k],
 * probs fp32 [N,E] or NULL.
 */
moe_status moe_route_topk(const float* logits, const float* bias, int32_t N, int32_t E, int32_t k,
                          int32_t* topk_idx, float* topk_w, float* probs, void* stream);

/*
 * Permute: build the top-k routing plan from topk_idx/topk_w without moving activations
 * ([GG] "적용" steps (1)-(3): flatten, sort by expert, bincount).  A stable counting sort:
 * rows of expert e appear in ascending token order.  Requires plan->kind == MOE_PLAN_TOPK,
 * plan->N/E/k equal to the arguments and plan->M_cap >= N*k.
 * Pairs that cannot make a row are skipped, so every plan this call writes is consistent and
 * safe to pass on: a pair (t, j) makes a row only if topk_idx[t,j] is in [0,E) and no slot
 * j' < j of token t names the same expert (moe_route_topk never produces another kind).  For
 * a skipped pair no row exists: counts and offsets count only the rows made (offsets[E] = M
 * <= N*k; plan rows M .. N*k-1 are not written), tok_ptr[t] = t*k still, token t's rows fill
 * tok_rows[t*k ..] in ascending row order and its remaining slots hold -1 (the combine skips
 * them), and moe_layer_bwd leaves ds[t*k+j] of that pair unwritten.  moe_router_bwd, which
 * reads topk_idx itself, still needs the router's own (valid) selection.
 * Workspace: moe_workspace_bytes(MOE_OP_PERMUTE, ...).
 */
moe_status moe_permute(const int32_t* topk_idx, const float* topk_w, int32_t N, int32_t E, int32_t k,
                       const moe_plan* plan, void* ws, size_t ws_bytes, void* stream);

/*
 * Permute without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same plan as
 * moe_permute, bit for bit, with the workspace replaced by a fixed 4 MiB scratch array that
 * the library holds on each GPU it runs on until the process ends.  Requires
 * moe_workspace_bytes(MOE_OP_PERMUTE, ...) <= 4 MiB (N*E up to about 2^25: N = 131008 tokens
 * at E = 256, 32704 at E = 1024), else MOE_EUNSUPPORTED and nothing is queued.  It calls no
 * allocating routine.
 * The scratch needs no clearing (every entry a call reads was written earlier in that call),
 * and all calls on one GPU share it: calls that overlap on one GPU (on different streams or
 * threads without ordering) race, so serialise them.  Arguments, plan and errors otherwise as
 * moe_permute.
 */
moe_status moe_permute_noalloc(const int32_t* topk_idx, const float* topk_w, int32_t N, int32_t E, int32_t k,
                               const moe_plan* plan, void* stream);

/*
 * Token-rounding route ([SM] "5 기여 ③ Token Rounding 라우팅"): ordinary top-k first (as
 * moe_route_topk, writing topk_idx, topk_w and probs, all required), then per expert the
 * row count c_e is rounded to r_e = mtile * floor((c_e + mtile/2) / mtile), clamped to the
 * largest multiple of mtile <= N; the r_e rows are the first r_e tokens in the order
 * (routed to e first, probs[t,e] descending, token ascending): surplus routed tokens with
 * the lowest scores are dropped, missing rows are padded with the best unrouted tokens.
 * Row weight = probs[t,e] / sum_j probs[t, topk_idx[t,j]] (kept pairs keep their top-k
 * weight up to rounding).  A token left with no rows contributes nothing.  The result is
 * written to `plan` (kind MOE_PLAN_TR, mtile as given, M_cap >= moe_plan_rows_cap()).
 * The number of rows M lives on the device in plan->offsets[E].
 */
moe_status moe_route_token_rounding(const float* logits, const float* bias, int32_t N, int32_t E,
                                    int32_t k, int32_t mtile, int32_t* topk_idx, float* topk_w,
                                    float* probs, const moe_plan* plan, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * Capacity routing: top-k (as moe_route_topk, writing topk_idx, topk_w and probs), then the
 * plan of the capacity-based layout of [DEP] "Drop/Padding 방식": the tokens assigned to each
 * expert are lined up and cut at the capacity C, the rest dropped.  The line-up order is the
 * drop policy that section names: MOE_CAP_POSITION (token order) or MOE_CAP_PROBS (P[t,e]
 * descending, then token order).  The plan stays ragged (rows ascending by token within an
 * expert, nothing padded: the dense E x C x H layout's padding is only a size), kept rows keep
 * their top-k weight (row_w = topk_w[t*k+j], no renormalisation), row_pair = t*k+j, and
 * tok_ptr / tok_rows list each token's kept rows (a token may keep fewer than k, or none).
 * moe_layer_bwd writes ds in row order for these plans, as for token rounding.  The plan
 * must have kind MOE_PLAN_CAP, mtile = capacity and M_cap >= moe_plan_rows_cap(); the row
 * count sits on the device in offsets[E].  Workspace: moe_workspace_bytes(MOE_OP_ROUTE_TR, ...).
 */
moe_status moe_route_capacity(const float* logits, const float* bias, int32_t N, int32_t E, int32_t k,
                              int32_t capacity, int32_t policy, int32_t* topk_idx, float* topk_w, float* probs,
                              const moe_plan* plan, void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped expert MLP forward: for every row r of expert e (token t = row_token[r]),
 *   G = x[t] W_gate[e]^T,  U = x[t] W_up[e]^T        (variable-M grouped GEMM, gate and up
 *                                                      share the group sizes, [GG] "적용" (6))
 *   hcache[r] = [G | U]                              (cached for the backward instead of
 *                                                      the O(TKd) activations, [SM] "3 기여 ①")
 *   A = silu(G) * U                                   (SwiGLU fused in the epilogue,
 *                                                      [SM] "4.2 Epilogue 융합")
 *   y[r] = A W_down[e]^T                              (variable-M grouped GEMM)
 * x rows are gathered inside the GEMM's global->LDS load ([SM] "4.1 Gather 융합"); the
 * permuted activations are never materialised.
 *   x [N,H], hcache [M_cap, 2I], y [M_cap, H]; rows >= M are not written.
 * Workspace: moe_workspace_bytes(MOE_OP_GEMM_FWD, ...) (holds A [M_cap, I]).
 */
moe_status moe_grouped_gemm_fwd(moe_dtype dt, const void* x, const void* w_gate, const void* w_up,
                                const void* w_down, int32_t H, int32_t I, const moe_plan* plan,
                                void* hcache, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * MX-FP8 (the fine-grained FP8 grouped GEMM of [GG] "한계": FP8 operands with a scale for each
 * small block along the contraction dimension, here in the OCP microscaling layout that
 * gfx950's scaled matrix instructions consume).  Element codes are e4m3 (sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, largest finite 448, no infinities); each block of 32
 * consecutive values along K has a scale code c, scale 2^(c - 127).
 * Layout of a quantized row-major [rows, K] matrix: codes q [rows, K] (one byte each) and
 * scale codes [rows, KS] with KS = 4 * ceil(K / 128) (the four blocks of a 128-wide k-step form
 * one 32-bit word): scales[r, b] scales q[r, 32b .. 32b + 31]; entries b >= K/32 are 0.
 *
 * moe_quantize_mxfp8: quantize src [rows, K] (dtype dt, row-major) into that layout.  Each
 * block's scale is the smallest power of two X with max |v| <= 448 X (no value clips), the code
 * limited to 0..254; each value is stored as v / X rounded to nearest e4m3, ties to even.
 * Deterministic, bit for bit.  K a positive multiple of 32; src and q 16-byte aligned.  A
 * weight tensor [E, out, in] is quantized as rows = E*out, K = in: W_gate and W_up along H,
 * W_down along I; activations x [N, H] along H.  Callers quantize the weights once per
 * update and reuse them over micro-batches.
 */
moe_status moe_quantize_mxfp8(moe_dtype dt, const void* src, int64_t rows, int32_t K, uint8_t* q, uint8_t* scales,
                              void* stream);

/*
 * Grouped expert MLP forward on MX-FP8 operands: the bf16 forward's computation with x,
 * W_gate, W_up (each quantized along H) and W_down (along I) given as codes and scale codes,
 * on gfx950's scaled fp8 matrix instructions (fp32 accumulation):
 *   [G | U] = x[t] [W_gate[e]; W_up[e]]^T  ->  hcache (bf16, as moe_grouped_gemm_fwd writes it,
 *                                               for the bf16 backward)
 *   A = silu(G) * U in fp32, quantized along I in the layout above into the workspace
 *   y[r] = A W_down[e]^T  ->  y (bf16)
 * x_q [N, H], x_s [N, KS(H)]; wg_q / wu_q [E, I, H], wg_s / wu_s [E, I, KS(H)]; wd_q [E, H, I],
 * wd_s [E, H, KS(I)]; hcache [M_cap, 2I] and y [M_cap, H] bf16.  H and I must be multiples of
 * 32.  Workspace: moe_workspace_bytes(MOE_OP_GEMM_FWD_MXFP8, MOE_BF16, N, E, k, H, I, M_cap);
 * after the call it holds A's codes [M_cap, I] at byte 0 and A's scale codes [M_cap, KS(I)] at
 * byte M_cap*I rounded up to a multiple of 256 (rows in plan order; rows >= M not written).
 * moe_unpermute_combine then sums y as in the bf16 path.
 */
moe_status moe_grouped_gemm_fwd_mxfp8(const uint8_t* x_q, const uint8_t* x_s, const uint8_t* wg_q,
                                      const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s,
                                      const uint8_t* wd_q, const uint8_t* wd_s, int32_t H, int32_t I,
                                      const moe_plan* plan, void* hcache, void* y, void* ws, size_t ws_bytes,
                                      void* stream);

/*
 * The backward's dX product on MX-FP8 operands: the FP8 grouped GEMM of [GG] "한계" applied to
 * dXe = dH [W_gate; W_up] of moe_layer_bwd, in the MX-FP8 layout of moe_quantize_mxfp8.
 *
 * moe_quantize_dx_weights_mxfp8: its weight operand.  For each expert e the matrix
 * [W_gate[e]^T | W_up[e]^T] ([H, 2I]: row h holds W_gate[e][i][h] for i < I, then
 * W_up[e][i][h]) quantized along its rows, 2I values in blocks of 32 (I a multiple of 32, so
 * no block mixes gate and up): codes wt_q [E, H, 2I], scale codes wt_s [E, H, 4 ceil(2I/128)].
 * Quantized once per weight update; bit for bit what moe_quantize_mxfp8 gives for that matrix.
 *   w_gate, w_up [E, I, H] (dtype dt); H, I multiples of 32; H * 2I bytes below 2 GiB.
 *
 * moe_layer_bwd_mxfp8: moe_layer_bwd for bf16 layers with its dX product on MX-FP8 operands:
 * each row's dH = [dG | dU] (stored in bf16, as in moe_layer_bwd) is quantized along its 2I
 * values, and dXe is taken from those codes and wt_q / wt_s, then combined per token in
 * ascending row order as before.  dW_gate, dW_up, dW_down and dS come from the same kernels
 * as in moe_layer_bwd, bit for bit; dx differs by the quantization of both operands.
 * H, I multiples of 32.  Workspace: moe_workspace_bytes(MOE_OP_LAYER_BWD_MXFP8, MOE_BF16, ...)
 * (moe_layer_bwd's plus the dH scale codes).
 */
moe_status moe_quantize_dx_weights_mxfp8(moe_dtype dt, const void* w_gate, const void* w_up, int32_t E, int32_t H,
                                         int32_t I, uint8_t* wt_q, uint8_t* wt_s, void* stream);
moe_status moe_layer_bwd_mxfp8(const void* dout, const void* x, const void* w_gate, const void* w_up,
                               const void* w_down, const uint8_t* wt_q, const uint8_t* wt_s, int32_t H, int32_t I,
                               const moe_plan* plan, const void* hcache, void* dx, void* dw_gate, void* dw_up,
                               void* dw_down, float* ds, void* ws, size_t ws_bytes, void* stream);

/*
 * Weighted combine back to token order ([EP] "여러 Expert의 결과도 같은 토큰으로
 * 돌아오기"; [DEP] "3) Combine"):
 *   out[t] = sum over r in tok_rows(t) of row_w[r] * y[r]     (row_w NULL: weights 1)
 * Rows are summed in ascending row order in fp32.  A token without rows gets 0.
 *   y [M_cap, H], row_w fp32 [M_cap] or NULL, out [N, H].
 */
moe_status moe_unpermute_combine(moe_dtype dt, const void* y, int32_t H, const moe_plan* plan,
                                 const float* row_w, void* out, void* stream);

/*
 * Layer backward given dOut (gradient of the combined output) and the forward's hcache.
 * For row r (expert e, token t, weight w) with G, U from hcache and A = silu(G) * U:
 *   dA'  = dOut[t] W_down[e]                  (varlen-M grouped GEMM, dOut gathered)
 *   dS_r = <dA', A>                           (= <dOut[t], y_r>: router-score gradient
 *                                              without loading Y, [SM] "3 기여 ①")
 *   dA   = w dA';  dG = dA U s (1 + G (1 - s)), s = sigmoid(G);  dU = dA silu(G)
 *   A'   = w A                                (dH, dS and A' from one epilogue,
 *                                              [SM] "4.2 Epilogue 융합"; dS leaves it as
 *                                              per-tile partials that the dX combine adds
 *                                              in a fixed order)
 *   dW_down[e] = sum_r dOut[t]^T A'           (varlen-K grouped GEMM, dOut gathered)
 *   dW_gate[e] = sum_r dG^T x[t],  dW_up[e] = sum_r dU^T x[t]   (varlen-K, x gathered)
 *   dx[t] = sum over rows of t of (dG W_gate[e] + dU W_up[e])  (varlen-M GEMM + combine)
 * ([SM] "4 기여 ②": varlen-M / varlen-K grouped GEMMs, gathers fused in the backward too.)
 *   dout, x [N,H]; hcache [M_cap,2I]; dx [N,H]; dw_gate, dw_up [E,I,H]; dw_down [E,H,I]
 *   (experts without rows get zeros); ds fp32: [N,k] in (t,j) order for top-k plans,
 *   [M_cap] in row order for token-rounding and capacity plans.  dx excludes the router's
 *   own path.
 * Workspace: moe_workspace_bytes(MOE_OP_LAYER_BWD, ...).
 */
moe_status moe_layer_bwd(moe_dtype dt, const void* dout, const void* x, const void* w_gate,
                         const void* w_up, const void* w_down, int32_t H, int32_t I,
                         const moe_plan* plan, const void* hcache, void* dx, void* dw_gate,
                         void* dw_up, void* dw_down, float* ds, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * Router logits.  [DEP] "1) Router" maps the [N,H] hidden states to per-expert scores; the
 * score is linear in the hidden state:
 *   logits[t,e] = sum_h x[t,h] * w_r[h,e]  (+ bias[e] when bias is not NULL)
 * accumulated in fp32 in a fixed order (the h range is cut into slices whose partial sums are
 * added in slice order; bitwise reproducible).  It runs on the bf16 matrix instructions with
 * each fp32 operand split exactly into three bf16 parts (v = hi + mid + lo), dropping only the
 * part products below 2^-24 of the leading one: fp32 accuracy.  x [N,H] of dtype dt; w_r fp32
 * [H,E]; bias fp32 [E] or NULL; logits fp32 [N,E] (written).  Requires 1 <= E <= 1024,
 * H >= 1, and (N+8)*H*2 and (H+1)*(N+8)*2 below 2 GiB (else MOE_EUNSUPPORTED).
 * Workspace: moe_workspace_bytes(MOE_OP_ROUTER_LOGITS, dt, N, E, 1, H, 0, 0).
 */
moe_status moe_router_logits(moe_dtype dt, const void* x, const float* w_r, const float* bias, int32_t N,
                             int32_t H, int32_t E, float* logits, void* ws, size_t ws_bytes, void* stream);

/*
 * Router backward: from dS, the gradient of the combine weights (moe_layer_bwd's ds), to
 * the router's logits, weight, bias and input.  The pages stop at dS ([SM] "3 기여 ①");
 * the rest follows from the weights' definition.  For token t with top-k set K
 * (topk_idx[t,:], the selection of the same logits and bias) and z = logits[t,:] + bias,
 * every final pair f = (t, e_f) of the plan has weight w_f = exp(z_{e_f}) / sum_{j in K}
 * exp(z_j): the renormalised top-k softmax ([DEP] "1) Router"), and for token-rounding
 * plans P_e / S_t ([SM] "5 기여 ③"), the same expression (padded pairs lie outside K,
 * dropped pairs have no row).  With q_m = exp(z_m) / sum_{j in K} exp(z_j):
 *   dlogits[t,m] = sum_f dS_f w_f ([m == e_f] - q_m [m in K])    (also d bias-shifted z)
 *   dx_out[t,h]  = dx_in[t,h] + sum_m dlogits[t,m] w_r[h,m]       (NULL dx_out skips it)
 *   dw_r[h,m]    = sum_t x[t,h] dlogits[t,m]                      (NULL skips it)
 *   dbias[m]     = sum_t dlogits[t,m]                             (NULL skips it)
 * w_f is the plan's row_w; dS_f is ds[t*k+j] (top-k plans, row_pair = t*k+j) or ds[r] (token
 * rounding and capacity plans, row order), the layout moe_layer_bwd writes.  logits, dlogits fp32 [N,E]; bias
 * fp32 [E] or NULL; topk_idx int32 [N,k]; x, dx_in, dx_out [N,H] of dtype dt (dx_out may be
 * dx_in: in place); w_r fp32 [H,E]; dw_r fp32 [H,E]; dbias fp32 [E].  Everything is written
 * fresh, in a fixed order (bitwise reproducible); the two products run like moe_router_logits'
 * (split bf16 parts, fp32 accuracy; the same size limit), except that the dx share of a bf16
 * layer, which is rounded to bf16, keeps 16 significant bits of each operand.  Workspace: moe_workspace_bytes(
 * MOE_OP_ROUTER_BWD, dt, N, E, k, H, 0, 0) when dx_out, dw_r or dbias is requested, else none.
 */
moe_status moe_router_bwd(moe_dtype dt, const float* logits, const float* bias, const int32_t* topk_idx,
                          const moe_plan* plan, const float* ds, const void* x, const float* w_r, int32_t H,
                          const void* dx_in, void* dx_out, float* dlogits, float* dw_r, float* dbias,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Measurement hook (for benchmarks and profilers, not needed for computing): kernels of
 * the library, identified by moe_kernel_id.  After moe_set_kernel_events(id, start, stop)
 * with two hipEvent_t handles (passed as void*), every later launch of that kernel records
 * `start` on the launch stream right before the launch and `stop` right after it; NULL
 * handles switch recording off.  The registry is process-global and not synchronised:
 * set it from one thread while no other thread calls the library.  Returns MOE_EINVAL for
 * an unknown id.  Ids that name a sequence (ROUTE_TR_PLAN, PERMUTE) bracket all of its
 * kernels.
 */
typedef enum moe_kernel_id {
  MOE_K_GATEUP = 0,      /* forward gate/up grouped GEMM + SwiGLU epilogue */
  MOE_K_DOWN = 1,        /* forward down grouped GEMM */
  MOE_K_DH = 2,          /* backward dH kernel: the dA' grouped GEMM with the dSwiGLU epilogue */
  MOE_K_DX = 3,          /* backward dX grouped GEMM (expert rows) */
  MOE_K_DWD = 4,         /* backward dW_down varlen-K GEMM */
  MOE_K_DW1 = 5,         /* backward dW_gate / dW_up varlen-K GEMM */
  MOE_K_COMBINE = 6,     /* weighted combine (moe_unpermute_combine) */
  MOE_K_DX_COMBINE = 7,  /* unweighted combine of dX rows inside moe_layer_bwd */
  MOE_K_ROUTE = 8,       /* top-k router kernel */
  MOE_K_PERMUTE = 9,     /* moe_permute: histogram, then scan + scatter (one kernel while the blocks are few) */
  MOE_K_ROUTE_TR_PLAN = 10, /* the token-rounding plan kernels after the router */
  MOE_K_DSWIGLU = 11,    /* not launched on its own any more: the dX combine sums the dS partials */
  MOE_K_ROUTER_LOGITS = 12, /* moe_router_logits */
  MOE_K_ROUTER_DZ = 13,  /* moe_router_bwd: dz from dS */
  MOE_K_ROUTER_DX = 14,  /* moe_router_bwd: dx_out = dx_in + dz W_r^T */
  MOE_K_ROUTER_DW = 15,  /* moe_router_bwd: dW_r and dbias (sliced product + ordered reduction) */
  MOE_K_GATEUP_FP8 = 16, /* moe_grouped_gemm_fwd_mxfp8: gate/up grouped GEMM + SwiGLU + A quantization */
  MOE_K_DOWN_FP8 = 17,   /* moe_grouped_gemm_fwd_mxfp8: down grouped GEMM */
  MOE_K_QUANT = 18,      /* moe_quantize_mxfp8, moe_quantize_dx_weights_mxfp8, and moe_layer_bwd_mxfp8's
                            quantization of dH */
  MOE_K_DX_FP8 = 19,     /* moe_layer_bwd_mxfp8: the dX grouped GEMM on MX-FP8 operands */
  MOE_K_COUNT = 20
} moe_kernel_id;

moe_status moe_set_kernel_events(int32_t kernel_id, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
