// api.hip -- the extern "C" entry points of libmoe.so: argument validation, workspace
// carving and launch sequencing on the caller's stream.  The operations themselves are
// documented in moe.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace {

thread_local char g_err[512];

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

moe_status check_dims(int32_t N, int32_t E, int32_t k) {
  REQUIRE(N >= 0, MOE_EINVAL, "N must be >= 0 (got %d)", N);
  REQUIRE(E >= 1 && E <= 1024, MOE_EINVAL, "E must be in [1, 1024] (got %d)", E);
  REQUIRE(k >= 1 && k <= E, MOE_EINVAL, "k must be in [1, E] (got k=%d, E=%d)", k, E);
  REQUIRE((int64_t)N * k <= INT32_MAX / 2, MOE_EINVAL, "N*k too large");
  return MOE_OK;
}

moe_status check_hi(int32_t H, int32_t I) {
  REQUIRE(H >= 8 && I >= 8, MOE_EINVAL, "H and I must be >= 8 (got H=%d, I=%d)", H, I);
  REQUIRE(H % 8 == 0 && I % 8 == 0, MOE_EUNSUPPORTED, "H and I must be multiples of 8 (got H=%d, I=%d)", H, I);
  return MOE_OK;
}

moe_status check_dtype(moe_dtype dt) {
  REQUIRE(dt == MOE_F32 || dt == MOE_BF16, MOE_EUNSUPPORTED, "unknown dtype %d", (int)dt);
  return MOE_OK;
}

moe_status check_plan(const moe_plan* p) {
  REQUIRE(p != nullptr, MOE_EINVAL, "plan is NULL");
  moe_status st = check_dims(p->N, p->E, p->k);
  if (st != MOE_OK) return st;
  REQUIRE(p->kind == MOE_PLAN_TOPK || p->kind == MOE_PLAN_TR || p->kind == MOE_PLAN_CAP, MOE_EINVAL,
          "unknown plan kind %d", p->kind);
  const int64_t need = moe_plan_rows_cap(p->kind, p->N, p->E, p->k, p->kind == MOE_PLAN_TOPK ? 0 : p->mtile);
  REQUIRE(need >= 0, MOE_EINVAL, "invalid plan dimensions");
  REQUIRE(p->M_cap >= need, MOE_EINVAL, "plan M_cap %d < required %lld", p->M_cap, (long long)need);
  REQUIRE(p->counts && p->offsets && p->tok_ptr, MOE_EINVAL, "plan has a NULL counts/offsets/tok_ptr array");
  REQUIRE(p->M_cap == 0 || (p->row_token && p->row_w && p->row_pair && p->tok_rows), MOE_EINVAL,
          "plan has a NULL row array");
  return MOE_OK;
}

int64_t mcap_of(const moe_plan* p) { return p->M_cap; }

// The GEMM kernels address a tensor through one buffer descriptor with 32-bit byte offsets
// (an offset of 2^31 or more marks a masked lane), so every tensor one descriptor covers must
// stay below 2 GiB: x and dOut [N,H], one expert's weight or weight-gradient matrix [I,H],
// the row-ordered activations (hcache and dH [M_cap, 2I], A and A' [M_cap, I]) and the plan's
// row arrays (4 M_cap bytes).
constexpr int64_t kDescBytes = 0x7FFFFFFF;
moe_status check_desc_sizes(moe_dtype dt, int64_t N, int64_t H, int64_t I, int64_t M_cap) {
  const int64_t es = dt == MOE_BF16 ? 2 : 4;
  REQUIRE(N * H * es <= kDescBytes, MOE_EUNSUPPORTED, "x/dout [N=%lld, H=%lld] must be < 2 GiB", (long long)N,
          (long long)H);
  REQUIRE(I * H * es <= kDescBytes, MOE_EUNSUPPORTED, "one expert's weight matrix [I=%lld, H=%lld] must be < 2 GiB",
          (long long)I, (long long)H);
  REQUIRE(M_cap * 2 * I * es <= kDescBytes, MOE_EUNSUPPORTED,
          "row activations [M_cap=%lld, 2I=%lld] must be < 2 GiB", (long long)M_cap, (long long)(2 * I));
  REQUIRE(M_cap * 4 <= kDescBytes, MOE_EUNSUPPORTED, "plan row arrays (M_cap=%lld) must be < 2 GiB",
          (long long)M_cap);
  return MOE_OK;
}

}  // namespace

namespace moe {
DevInfo dev_info() {
  static DevInfo cache[64];
  static bool have[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DevInfo{256, 8};
  if (!have[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cache[dev] = DevInfo{cus, 8};
    have[dev] = true;
  }
  return cache[dev];
}
}  // namespace moe

namespace {
hipEvent_t g_events[MOE_K_COUNT][2];
}

namespace moe {
void kernel_event(int kid, int which, hipStream_t s) {
  hipEvent_t ev = g_events[kid][which];
  if (ev) (void)hipEventRecord(ev, s);
}
}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_err; }

moe_status moe_set_kernel_events(int32_t kernel_id, void* start_event, void* stop_event) {
  g_err[0] = 0;
  REQUIRE(kernel_id >= 0 && kernel_id < MOE_K_COUNT, MOE_EINVAL, "unknown kernel id %d", kernel_id);
  g_events[kernel_id][0] = (hipEvent_t)start_event;
  g_events[kernel_id][1] = (hipEvent_t)stop_event;
  return MOE_OK;
}

int64_t moe_plan_rows_cap(int32_t kind, int32_t N, int32_t E, int32_t k, int32_t mtile) {
  if (N < 0 || E < 1 || E > 1024 || k < 1 || k > E) return -1;
  if (kind == MOE_PLAN_TOPK) return (int64_t)N * k;
  if (kind == MOE_PLAN_TR) {
    if (mtile < 1) return -1;
    return (int64_t)N * k + (int64_t)E * (mtile / 2);
  }
  if (kind == MOE_PLAN_CAP) {  // mtile holds the capacity
    if (mtile < 0) return -1;
    const int64_t a = (int64_t)N * k, b = (int64_t)E * mtile;
    return a < b ? a : b;
  }
  return -1;
}

size_t moe_workspace_bytes(moe_op op, moe_dtype dt, int32_t N, int32_t E, int32_t k, int32_t H, int32_t I,
                           int32_t M_cap) {
  if (check_dims(N, E, k) != MOE_OK) return 0;
  switch (op) {
    case MOE_OP_PERMUTE: return moe::permute_ws_bytes(N, E);
    case MOE_OP_ROUTE_TR: return moe::tr_ws_bytes(N, E);
    case MOE_OP_GEMM_FWD:
      if (check_dtype(dt) != MOE_OK || check_hi(H, I) != MOE_OK || M_cap < 0) return 0;
      return moe::gemm_fwd_ws_bytes(dt, M_cap, I);
    case MOE_OP_LAYER_BWD:
      if (check_dtype(dt) != MOE_OK || check_hi(H, I) != MOE_OK || M_cap < 0) return 0;
      return moe::layer_bwd_ws_bytes(dt, N, M_cap, H, I);
    case MOE_OP_ROUTER_BWD:
      if (check_dtype(dt) != MOE_OK || H < 1) return 0;
      return moe::router_bwd_ws_bytes(dt, N, H, E);
    case MOE_OP_ROUTER_LOGITS:
      if (check_dtype(dt) != MOE_OK || H < 1) return 0;
      return moe::router_logits_ws_bytes(dt, N, H, E);
    case MOE_OP_GEMM_FWD_MXFP8:
      if (H < 32 || I < 32 || H % 32 || I % 32 || M_cap < 0) return 0;
      return moe::gemm_fwd_mxfp8_ws_bytes(M_cap, I);
    case MOE_OP_LAYER_BWD_MXFP8:
      if (H < 32 || I < 32 || H % 32 || I % 32 || M_cap < 0) return 0;
      return moe::layer_bwd_mxfp8_ws_bytes(N, M_cap, H, I);
  }
  return 0;
}

moe_status moe_route_topk(const float* logits, const float* bias, int32_t N, int32_t E, int32_t k,
                          int32_t* topk_idx, float* topk_w, float* probs, void* stream) {
  g_err[0] = 0;
  moe_status st = check_dims(N, E, k);
  if (st != MOE_OK) return st;
  REQUIRE(N == 0 || (logits && topk_idx && topk_w), MOE_EINVAL, "NULL logits/topk_idx/topk_w");
  moe::kernel_event(MOE_K_ROUTE, 0, (hipStream_t)stream);
  hipError_t e = moe::launch_route_topk(logits, bias, N, E, k, topk_idx, topk_w, probs, nullptr, (hipStream_t)stream);
  moe::kernel_event(MOE_K_ROUTE, 1, (hipStream_t)stream);
  return hip_status(e, "moe_route_topk");
}

moe_status moe_permute(const int32_t* topk_idx, const float* topk_w, int32_t N, int32_t E, int32_t k,
                       const moe_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_dims(N, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(plan->kind == MOE_PLAN_TOPK, MOE_EINVAL, "moe_permute needs a top-k plan");
  REQUIRE(plan->N == N && plan->E == E && plan->k == k, MOE_EINVAL, "plan dimensions differ from the call");
  REQUIRE(N == 0 || (topk_idx && topk_w), MOE_EINVAL, "NULL topk_idx/topk_w");
  const size_t need = moe::permute_ws_bytes(N, E);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  moe::kernel_event(MOE_K_PERMUTE, 0, (hipStream_t)stream);
  hipError_t e = moe::launch_permute(topk_idx, topk_w, N, E, k, *plan, ws, (hipStream_t)stream);
  moe::kernel_event(MOE_K_PERMUTE, 1, (hipStream_t)stream);
  return hip_status(e, "moe_permute");
}

moe_status moe_permute_noalloc(const int32_t* topk_idx, const float* topk_w, int32_t N, int32_t E, int32_t k,
                               const moe_plan* plan, void* stream) {
  g_err[0] = 0;
  moe_status st = check_dims(N, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(plan->kind == MOE_PLAN_TOPK, MOE_EINVAL, "moe_permute_noalloc needs a top-k plan");
  REQUIRE(plan->N == N && plan->E == E && plan->k == k, MOE_EINVAL, "plan dimensions differ from the call");
  REQUIRE(N == 0 || (topk_idx && topk_w), MOE_EINVAL, "NULL topk_idx/topk_w");
  const size_t need = moe::permute_ws_bytes(N, E);
  REQUIRE(need <= moe::permute_scratch_bytes(), MOE_EUNSUPPORTED,
          "moe_permute_noalloc: N=%d, E=%d need %zu bytes of scratch, more than its fixed %zu", N, E, need,
          moe::permute_scratch_bytes());
  void* scratch = nullptr;
  hipError_t e = moe::permute_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "moe_permute_noalloc: scratch address");
  moe::kernel_event(MOE_K_PERMUTE, 0, (hipStream_t)stream);
  e = moe::launch_permute(topk_idx, topk_w, N, E, k, *plan, scratch, (hipStream_t)stream);
  moe::kernel_event(MOE_K_PERMUTE, 1, (hipStream_t)stream);
  return hip_status(e, "moe_permute_noalloc");
}

moe_status moe_route_token_rounding(const float* logits, const float* bias, int32_t N, int32_t E, int32_t k,
                                    int32_t mtile, int32_t* topk_idx, float* topk_w, float* probs,
                                    const moe_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_dims(N, E, k);
  if (st != MOE_OK) return st;
  REQUIRE(mtile >= 1 && mtile <= 65536, MOE_EINVAL, "mtile must be in [1, 65536] (got %d)", mtile);
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(plan->kind == MOE_PLAN_TR && plan->mtile == mtile, MOE_EINVAL,
          "token rounding needs a plan of kind MOE_PLAN_TR with the same mtile");
  REQUIRE(plan->N == N && plan->E == E && plan->k == k, MOE_EINVAL, "plan dimensions differ from the call");
  REQUIRE(N == 0 || (logits && topk_idx && topk_w && probs), MOE_EINVAL, "NULL logits/topk_idx/topk_w/probs");
  const size_t need = moe::tr_ws_bytes(N, E);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  // the token normaliser sits right after the block histogram in the workspace
  float* tok_norm = moe::tr_tok_norm(ws, N, E);
  hipStream_t s = (hipStream_t)stream;
  moe::kernel_event(MOE_K_ROUTE, 0, s);
  hipError_t e = moe::launch_route_topk(logits, bias, N, E, k, topk_idx, topk_w, probs, tok_norm, s);
  moe::kernel_event(MOE_K_ROUTE, 1, s);
  if (e != hipSuccess) return hip_status(e, "moe_route_token_rounding/route");
  moe::kernel_event(MOE_K_ROUTE_TR_PLAN, 0, s);
  e = moe::launch_token_round(topk_idx, probs, tok_norm, nullptr, N, E, k, 0, mtile, 1, *plan, ws, s);
  moe::kernel_event(MOE_K_ROUTE_TR_PLAN, 1, s);
  return hip_status(e, "moe_route_token_rounding");
}

moe_status moe_route_capacity(const float* logits, const float* bias, int32_t N, int32_t E, int32_t k,
                              int32_t capacity, int32_t policy, int32_t* topk_idx, float* topk_w, float* probs,
                              const moe_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st = check_dims(N, E, k);
  if (st != MOE_OK) return st;
  REQUIRE(capacity >= 0, MOE_EINVAL, "capacity must be >= 0 (got %d)", capacity);
  REQUIRE(policy == MOE_CAP_POSITION || policy == MOE_CAP_PROBS, MOE_EINVAL, "unknown capacity policy %d", policy);
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(plan->kind == MOE_PLAN_CAP && plan->mtile == capacity, MOE_EINVAL,
          "a capacity plan needs kind MOE_PLAN_CAP with the capacity in its mtile field");
  REQUIRE(plan->N == N && plan->E == E && plan->k == k, MOE_EINVAL, "plan dimensions differ from the call");
  REQUIRE(N == 0 || (logits && topk_idx && topk_w && probs), MOE_EINVAL, "NULL logits/topk_idx/topk_w/probs");
  const size_t need = moe::tr_ws_bytes(N, E);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  float* tok_norm = moe::tr_tok_norm(ws, N, E);
  hipStream_t s = (hipStream_t)stream;
  moe::kernel_event(MOE_K_ROUTE, 0, s);
  hipError_t e = moe::launch_route_topk(logits, bias, N, E, k, topk_idx, topk_w, probs, tok_norm, s);
  moe::kernel_event(MOE_K_ROUTE, 1, s);
  if (e != hipSuccess) return hip_status(e, "moe_route_capacity/route");
  moe::kernel_event(MOE_K_ROUTE_TR_PLAN, 0, s);
  e = moe::launch_token_round(topk_idx, probs, tok_norm, topk_w, N, E, k, 1, capacity,
                              policy == MOE_CAP_PROBS ? 1 : 0, *plan, ws, s);
  moe::kernel_event(MOE_K_ROUTE_TR_PLAN, 1, s);
  return hip_status(e, "moe_route_capacity");
}

moe_status moe_grouped_gemm_fwd(moe_dtype dt, const void* x, const void* w_gate, const void* w_up,
                                const void* w_down, int32_t H, int32_t I, const moe_plan* plan, void* hcache,
                                void* y, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st;
  if ((st = check_dtype(dt)) != MOE_OK) return st;
  if ((st = check_hi(H, I)) != MOE_OK) return st;
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(w_gate && w_up && w_down, MOE_EINVAL, "NULL weight argument");
  REQUIRE(plan->M_cap == 0 || (x && hcache && y), MOE_EINVAL, "NULL tensor argument");
  REQUIRE(aligned16(x) && aligned16(w_gate) && aligned16(w_up) && aligned16(w_down) && aligned16(hcache) &&
              aligned16(y) && aligned16(ws),
          MOE_EUNSUPPORTED, "tensors and workspace must be 16-byte aligned");
  if ((st = check_desc_sizes(dt, plan->N, H, I, plan->M_cap)) != MOE_OK) return st;
  const size_t need = moe::gemm_fwd_ws_bytes(dt, (int)mcap_of(plan), I);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  return hip_status(moe::launch_gemm_fwd(dt, x, w_gate, w_up, w_down, H, I, *plan, hcache, y, ws,
                                         (hipStream_t)stream),
                    "moe_grouped_gemm_fwd");
}

moe_status moe_quantize_mxfp8(moe_dtype dt, const void* src, int64_t rows, int32_t K, uint8_t* q, uint8_t* scales,
                              void* stream) {
  g_err[0] = 0;
  moe_status st;
  if ((st = check_dtype(dt)) != MOE_OK) return st;
  REQUIRE(rows >= 0, MOE_EINVAL, "rows must be >= 0 (got %lld)", (long long)rows);
  REQUIRE(K >= 32 && K % 32 == 0, MOE_EUNSUPPORTED, "K must be a positive multiple of 32 (got %d)", K);
  REQUIRE(rows == 0 || (src && q && scales), MOE_EINVAL, "NULL src/q/scales");
  REQUIRE(aligned16(src) && aligned16(q), MOE_EUNSUPPORTED, "src and q must be 16-byte aligned");
  REQUIRE(rows <= ((int64_t)1 << 40) / K, MOE_EINVAL, "rows too large");
  moe::kernel_event(MOE_K_QUANT, 0, (hipStream_t)stream);
  hipError_t e = moe::launch_quant_mxfp8(dt, src, rows, K, q, scales, (hipStream_t)stream);
  moe::kernel_event(MOE_K_QUANT, 1, (hipStream_t)stream);
  return hip_status(e, "moe_quantize_mxfp8");
}

moe_status moe_grouped_gemm_fwd_mxfp8(const uint8_t* x_q, const uint8_t* x_s, const uint8_t* wg_q,
                                      const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s,
                                      const uint8_t* wd_q, const uint8_t* wd_s, int32_t H, int32_t I,
                                      const moe_plan* plan, void* hcache, void* y, void* ws, size_t ws_bytes,
                                      void* stream) {
  g_err[0] = 0;
  moe_status st;
  REQUIRE(H >= 32 && I >= 32, MOE_EINVAL, "H and I must be >= 32 (got H=%d, I=%d)", H, I);
  REQUIRE(H % 32 == 0 && I % 32 == 0, MOE_EUNSUPPORTED, "H and I must be multiples of 32 (got H=%d, I=%d)", H, I);
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(wg_q && wg_s && wu_q && wu_s && wd_q && wd_s, MOE_EINVAL, "NULL weight argument");
  REQUIRE(plan->M_cap == 0 || (x_q && x_s && hcache && y), MOE_EINVAL, "NULL tensor argument");
  REQUIRE(aligned16(x_q) && aligned16(wg_q) && aligned16(wu_q) && aligned16(wd_q) && aligned16(hcache) &&
              aligned16(y) && aligned16(ws) && ((uintptr_t)x_s & 3u) == 0 && ((uintptr_t)wg_s & 3u) == 0 &&
              ((uintptr_t)wu_s & 3u) == 0 && ((uintptr_t)wd_s & 3u) == 0,
          MOE_EUNSUPPORTED, "codes, outputs and workspace must be 16-byte aligned, scale codes 4-byte aligned");
  // the bf16 outputs bound the sizes as in the bf16 forward; the codes are half as large
  if ((st = check_desc_sizes(MOE_BF16, plan->N, H, I, plan->M_cap)) != MOE_OK) return st;
  const size_t need = moe::gemm_fwd_mxfp8_ws_bytes((int)mcap_of(plan), I);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  return hip_status(moe::launch_gemm_fwd_mxfp8(x_q, x_s, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, H, I, *plan, hcache, y,
                                               ws, (hipStream_t)stream),
                    "moe_grouped_gemm_fwd_mxfp8");
}

moe_status moe_unpermute_combine(moe_dtype dt, const void* y, int32_t H, const moe_plan* plan, const float* row_w,
                                 void* out, void* stream) {
  g_err[0] = 0;
  moe_status st;
  if ((st = check_dtype(dt)) != MOE_OK) return st;
  REQUIRE(H >= 8, MOE_EINVAL, "H must be >= 8 (got %d)", H);
  REQUIRE(H % 8 == 0, MOE_EUNSUPPORTED, "H must be a multiple of 8 (got %d)", H);
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(plan->N == 0 || (out && (plan->M_cap == 0 || y)), MOE_EINVAL, "NULL tensor argument");
  REQUIRE(aligned16(y) && aligned16(out), MOE_EUNSUPPORTED, "tensors must be 16-byte aligned");
  moe::kernel_event(MOE_K_COMBINE, 0, (hipStream_t)stream);
  hipError_t e = moe::launch_combine(dt, y, H, *plan, row_w, out, (hipStream_t)stream);
  moe::kernel_event(MOE_K_COMBINE, 1, (hipStream_t)stream);
  return hip_status(e, "moe_unpermute_combine");
}

moe_status moe_layer_bwd(moe_dtype dt, const void* dout, const void* x, const void* w_gate, const void* w_up,
                         const void* w_down, int32_t H, int32_t I, const moe_plan* plan, const void* hcache,
                         void* dx, void* dw_gate, void* dw_up, void* dw_down, float* ds, void* ws, size_t ws_bytes,
                         void* stream) {
  g_err[0] = 0;
  moe_status st;
  if ((st = check_dtype(dt)) != MOE_OK) return st;
  if ((st = check_hi(H, I)) != MOE_OK) return st;
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(w_gate && w_up && w_down && dw_gate && dw_up && dw_down, MOE_EINVAL, "NULL weight/gradient argument");
  REQUIRE(plan->N == 0 || (dout && x && dx), MOE_EINVAL, "NULL activation argument");
  REQUIRE(plan->M_cap == 0 || (hcache && ds), MOE_EINVAL, "NULL hcache/ds argument");
  REQUIRE(aligned16(dout) && aligned16(x) && aligned16(w_gate) && aligned16(w_up) && aligned16(w_down) &&
              aligned16(hcache) && aligned16(dx) && aligned16(dw_gate) && aligned16(dw_up) && aligned16(dw_down) &&
              aligned16(ws),
          MOE_EUNSUPPORTED, "tensors and workspace must be 16-byte aligned");
  if ((st = check_desc_sizes(dt, plan->N, H, I, plan->M_cap)) != MOE_OK) return st;
  const size_t need = moe::layer_bwd_ws_bytes(dt, plan->N, (int)mcap_of(plan), H, I);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  return hip_status(moe::launch_layer_bwd(dt, dout, x, w_gate, w_up, w_down, H, I, *plan, hcache, dx, dw_gate,
                                          dw_up, dw_down, ds, ws, (hipStream_t)stream),
                    "moe_layer_bwd");
}

moe_status moe_quantize_dx_weights_mxfp8(moe_dtype dt, const void* w_gate, const void* w_up, int32_t E, int32_t H,
                                         int32_t I, uint8_t* wt_q, uint8_t* wt_s, void* stream) {
  g_err[0] = 0;
  moe_status st;
  if ((st = check_dtype(dt)) != MOE_OK) return st;
  REQUIRE(E >= 1 && E <= 1024, MOE_EINVAL, "E must be in [1, 1024] (got %d)", E);
  REQUIRE(H >= 32 && I >= 32, MOE_EINVAL, "H and I must be >= 32 (got H=%d, I=%d)", H, I);
  REQUIRE(H % 32 == 0 && I % 32 == 0, MOE_EUNSUPPORTED, "H and I must be multiples of 32 (got H=%d, I=%d)", H, I);
  REQUIRE(w_gate && w_up && wt_q && wt_s, MOE_EINVAL, "NULL argument");
  REQUIRE(aligned16(wt_q), MOE_EUNSUPPORTED, "wt_q must be 16-byte aligned");
  REQUIRE((int64_t)H * 2 * I <= kDescBytes, MOE_EUNSUPPORTED, "one expert's [H=%d, 2I=%d] codes must be < 2 GiB", H,
          2 * I);
  moe::kernel_event(MOE_K_QUANT, 0, (hipStream_t)stream);
  hipError_t e = moe::launch_quant_dx_weights(dt, w_gate, w_up, E, H, I, wt_q, wt_s, (hipStream_t)stream);
  moe::kernel_event(MOE_K_QUANT, 1, (hipStream_t)stream);
  return hip_status(e, "moe_quantize_dx_weights_mxfp8");
}

moe_status moe_layer_bwd_mxfp8(const void* dout, const void* x, const void* w_gate, const void* w_up,
                               const void* w_down, const uint8_t* wt_q, const uint8_t* wt_s, int32_t H, int32_t I,
                               const moe_plan* plan, const void* hcache, void* dx, void* dw_gate, void* dw_up,
                               void* dw_down, float* ds, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st;
  REQUIRE(H >= 32 && I >= 32, MOE_EINVAL, "H and I must be >= 32 (got H=%d, I=%d)", H, I);
  REQUIRE(H % 32 == 0 && I % 32 == 0, MOE_EUNSUPPORTED, "H and I must be multiples of 32 (got H=%d, I=%d)", H, I);
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(w_gate && w_up && w_down && dw_gate && dw_up && dw_down && wt_q && wt_s, MOE_EINVAL,
          "NULL weight/gradient argument");
  REQUIRE(plan->N == 0 || (dout && x && dx), MOE_EINVAL, "NULL activation argument");
  REQUIRE(plan->M_cap == 0 || (hcache && ds), MOE_EINVAL, "NULL hcache/ds argument");
  REQUIRE(aligned16(dout) && aligned16(x) && aligned16(w_gate) && aligned16(w_up) && aligned16(w_down) &&
              aligned16(hcache) && aligned16(dx) && aligned16(dw_gate) && aligned16(dw_up) && aligned16(dw_down) &&
              aligned16(ws) && aligned16(wt_q) && ((uintptr_t)wt_s & 3u) == 0,
          MOE_EUNSUPPORTED, "tensors and workspace must be 16-byte aligned, wt_s 4-byte aligned");
  if ((st = check_desc_sizes(MOE_BF16, plan->N, H, I, plan->M_cap)) != MOE_OK) return st;
  REQUIRE((int64_t)H * 2 * I <= kDescBytes, MOE_EUNSUPPORTED, "one expert's [H=%d, 2I=%d] codes must be < 2 GiB", H,
          2 * I);
  const size_t need = moe::layer_bwd_mxfp8_ws_bytes(plan->N, (int)mcap_of(plan), H, I);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  return hip_status(moe::launch_layer_bwd_mxfp8(dout, x, w_gate, w_up, w_down, wt_q, wt_s, H, I, *plan, hcache, dx,
                                                dw_gate, dw_up, dw_down, ds, ws, (hipStream_t)stream),
                    "moe_layer_bwd_mxfp8");
}

moe_status moe_router_logits(moe_dtype dt, const void* x, const float* w_r, const float* bias, int32_t N,
                             int32_t H, int32_t E, float* logits, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st;
  if ((st = check_dtype(dt)) != MOE_OK) return st;
  REQUIRE(N >= 0, MOE_EINVAL, "N must be >= 0 (got %d)", N);
  REQUIRE(E >= 1 && E <= 1024, MOE_EINVAL, "E must be in [1, 1024] (got %d)", E);
  REQUIRE(H >= 1, MOE_EINVAL, "H must be >= 1 (got %d)", H);
  REQUIRE((int64_t)N * (H + 8) * 2 <= kDescBytes && (int64_t)(H + 1) * (N + 8) * 2 <= kDescBytes, MOE_EUNSUPPORTED,
          "N*H too large for one router call (N=%d, H=%d: the operand planes exceed 2 GiB)", N, H);
  REQUIRE(N == 0 || (x && w_r && logits), MOE_EINVAL, "NULL x/w_r/logits");
  const size_t need = moe::router_logits_ws_bytes(dt, N, H, E);
  REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  return hip_status(moe::launch_router_logits(dt, x, w_r, bias, N, H, E, logits, ws, (hipStream_t)stream),
                    "moe_router_logits");
}

moe_status moe_router_bwd(moe_dtype dt, const float* logits, const float* bias, const int32_t* topk_idx,
                          const moe_plan* plan, const float* ds, const void* x, const float* w_r, int32_t H,
                          const void* dx_in, void* dx_out, float* dlogits, float* dw_r, float* dbias, void* ws,
                          size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe_status st;
  if ((st = check_dtype(dt)) != MOE_OK) return st;
  if ((st = check_plan(plan)) != MOE_OK) return st;
  REQUIRE(H >= 1, MOE_EINVAL, "H must be >= 1 (got %d)", H);
  const int32_t N = plan->N;
  REQUIRE(N == 0 || (logits && topk_idx && dlogits), MOE_EINVAL, "NULL logits/topk_idx/dlogits");
  REQUIRE(N == 0 || plan->M_cap == 0 || ds, MOE_EINVAL, "NULL ds");
  REQUIRE(!dx_out || (dx_in && w_r), MOE_EINVAL, "dx_out needs dx_in and w_r");
  REQUIRE(!(dw_r || dbias) || N == 0 || x, MOE_EINVAL, "dw_r / dbias need x");
  REQUIRE((int64_t)N * (H + 8) * 2 <= kDescBytes && (int64_t)(H + 1) * (N + 8) * 2 <= kDescBytes, MOE_EUNSUPPORTED,
          "N*H too large for one router call (N=%d, H=%d: the operand planes exceed 2 GiB)", N, H);
  if (dx_out || dw_r || dbias) {
    const size_t need = moe::router_bwd_ws_bytes(dt, N, H, plan->E);
    REQUIRE(ws_bytes >= need, MOE_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    REQUIRE(ws != nullptr, MOE_EINVAL, "NULL workspace");
  }
  return hip_status(moe::launch_router_bwd(dt, logits, bias, topk_idx, *plan, ds, x, w_r, H, dx_in, dx_out, dlogits,
                                           dw_r, dbias, ws, (hipStream_t)stream),
                    "moe_router_bwd");
}

}  // extern "C"
