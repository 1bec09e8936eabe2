// The extern "C" entry points of libmoe.so (declared in include/moe.h):
// argument validation on the host, then the kernel launches of each step.
#include <stdio.h>
#include <algorithm>
#include <string.h>

#include "internal.h"

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e) {
  strncpy(g_last_error, hipGetErrorString(e), sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = 0;
  return MOE_ERR_HIP;
}

int finish(hipError_t e) { return e == hipSuccess ? MOE_OK : hip_fail(e); }

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool need(const void* p) { return p != nullptr && aligned(p); }
bool opt(const void* p) { return p == nullptr || aligned(p); }

int check_desc(const moe_desc* d) {
  if (!d || d->struct_size != sizeof(moe_desc)) return MOE_ERR_INVALID_ARG;
  if (d->T < 1 || d->d < 1 || d->f < 1 || d->E < 1 || d->k < 1 || d->num_local < 1 || d->expert_begin < 0)
    return MOE_ERR_INVALID_ARG;
  if (d->k > d->E || (int64_t)d->expert_begin + d->num_local > d->E) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (d->tile_schedule != MOE_SCHEDULE_STATIC && d->tile_schedule != MOE_SCHEDULE_DYNAMIC)
    return MOE_ERR_INVALID_ARG;
  if (d->tile_schedule == MOE_SCHEDULE_DYNAMIC && !need(d->tile_counters)) return MOE_ERR_INVALID_ARG;
  if (d->wgrad_dtype != MOE_F32 && d->wgrad_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->wgrad_dtype == MOE_BF16 && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->d % 64 || d->f % 64 || d->E % 8 || d->E > 1024 || d->k > 32) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d->T * d->k >= (1ll << 31) || (int64_t)d->T * d->E >= (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int moe_workspace_size(const moe_desc* desc, int op, size_t* bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  switch (op) {
    case MOE_OP_ROUTER_LOGITS: *bytes = moe::router_logits_workspace(*desc); return MOE_OK;
    case MOE_OP_GROUPED_FFN:
    case MOE_OP_FFN_BWD_DX:
    case MOE_OP_FFN_BWD_DW: *bytes = 0; return MOE_OK;
    case MOE_OP_PERMUTE: *bytes = moe::permute_workspace(*desc); return MOE_OK;
    case MOE_OP_ROUTER_BWD: *bytes = moe::router_bwd_workspace(*desc); return MOE_OK;
    default: return MOE_ERR_INVALID_ARG;
  }
}

int moe_router_logits(const moe_desc* desc, const void* x, const void* Wr, const float* bias, float* logits,
                      void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(x) || !need(Wr) || !need(logits) || !opt(bias)) return MOE_ERR_INVALID_ARG;
  const size_t need_ws = moe::router_logits_workspace(*desc);
  if (need_ws && (!need(ws) || ws_bytes < need_ws)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return finish(moe::launch_router_logits(*desc, x, Wr, bias, logits, ws, S(stream)));
}

int moe_route(const moe_desc* desc, const float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(logits) || !need(topk_idx) || !need(topk_w)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_route(*desc, logits, 1, topk_idx, topk_w, S(stream)));
}

int moe_route_grouped(const moe_desc* desc, const float* logits, int n_groups, int32_t* topk_idx, float* topk_w,
                      void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(logits) || !need(topk_idx) || !need(topk_w)) return MOE_ERR_INVALID_ARG;
  if (n_groups < 1 || n_groups > 64 || desc->E % n_groups || desc->k % n_groups) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_route(*desc, logits, n_groups, topk_idx, topk_w, S(stream)));
}

int moe_permute(const moe_desc* desc, const int32_t* topk_idx, const void* x, int32_t* counts, int32_t* offsets,
                int32_t* row_token, int32_t* slot_row, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(topk_idx) || !need(counts) || !need(offsets) || !need(row_token) || !need(slot_row) || !opt(x))
    return MOE_ERR_INVALID_ARG;
  if (x && !need(x_perm)) return MOE_ERR_INVALID_ARG;
  if (!need(ws) || ws_bytes < moe::permute_workspace(*desc)) return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return finish(moe::launch_permute(*desc, topk_idx, x, counts, offsets, row_token, slot_row, x_perm, ws,
                                    S(stream)));
}

int moe_permute_noalloc(const moe_desc* desc, const int32_t* topk_idx, const void* x, int32_t* counts,
                        int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(topk_idx) || !need(counts) || !need(offsets) || !need(row_token) || !need(slot_row) || !opt(x))
    return MOE_ERR_INVALID_ARG;
  if (x && !need(x_perm)) return MOE_ERR_INVALID_ARG;
  const size_t want = moe::permute_workspace(*desc);
  if (want > moe::PERMUTE_SCRATCH_BYTES) {
    snprintf(g_last_error, sizeof(g_last_error),
             "moe_permute_noalloc: the shape needs %zu bytes of scratch, the fixed scratch holds %zu", want,
             moe::PERMUTE_SCRATCH_BYTES);
    return MOE_ERR_UNSUPPORTED;
  }
  return finish(moe::launch_permute_noalloc(*desc, topk_idx, x, counts, offsets, row_token, slot_row, x_perm,
                                            S(stream)));
}

int moe_grouped_ffn(const moe_desc* desc, const int32_t* offsets, const void* x_perm, const void* W1,
                    const void* W3, const void* W2, void* gu, void* h, void* y_perm, void* ws, size_t ws_bytes,
                    void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(x_perm) || !need(W1) || !need(W3) || !need(W2) || !opt(gu) || !need(h) ||
      !need(y_perm))
    return MOE_ERR_INVALID_ARG;
  hipError_t e = moe::launch_gate_up(*desc, offsets, x_perm, W1, W3, gu, h, S(stream));
  if (e == hipSuccess) e = moe::launch_down(*desc, offsets, h, W2, y_perm, S(stream));
  return finish(e);
}

int moe_expert_gate_up(const moe_desc* desc, const int32_t* offsets, const void* x_perm, const void* W1,
                       const void* W3, void* gu, void* h, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(x_perm) || !need(W1) || !need(W3) || !opt(gu) || !need(h)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_gate_up(*desc, offsets, x_perm, W1, W3, gu, h, S(stream)));
}

int moe_expert_down(const moe_desc* desc, const int32_t* offsets, const void* h, const void* W2, void* y_perm,
                    void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(h) || !need(W2) || !need(y_perm)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_down(*desc, offsets, h, W2, y_perm, S(stream)));
}

int moe_combine(const moe_desc* desc, const int32_t* slot_row, const float* topk_w, const void* y_perm, void* y,
                void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(slot_row) || !need(topk_w) || !need(y_perm) || !need(y)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_combine(*desc, slot_row, topk_w, y_perm, y, S(stream)));
}

int moe_combine_bwd(const moe_desc* desc, const int32_t* slot_row, const float* topk_w, const void* y_perm,
                    const void* dy, void* dy_perm, float* dtopk_w, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(slot_row) || !need(topk_w) || !need(y_perm) || !need(dy) || !need(dy_perm) || !need(dtopk_w))
    return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_combine_bwd(*desc, slot_row, topk_w, y_perm, dy, dy_perm, dtopk_w, S(stream)));
}

int moe_grouped_ffn_bwd_dx(const moe_desc* desc, const int32_t* offsets, const void* W1, const void* W3,
                           const void* W2, const void* gu, const void* dy_perm, void* dgu, void* dx_perm, void* ws,
                           size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(W1) || !need(W3) || !need(W2) || !need(gu) || !need(dy_perm) || !need(dgu) ||
      !need(dx_perm))
    return MOE_ERR_INVALID_ARG;
  hipError_t e = moe::launch_bwd_dh(*desc, offsets, W2, gu, dy_perm, dgu, S(stream));
  if (e == hipSuccess) e = moe::launch_bwd_dxp(*desc, offsets, W1, W3, dgu, dx_perm, S(stream));
  return finish(e);
}

int moe_expert_bwd_dh(const moe_desc* desc, const int32_t* offsets, const void* W2, const void* gu,
                      const void* dy_perm, void* dgu, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(W2) || !need(gu) || !need(dy_perm) || !need(dgu)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_bwd_dh(*desc, offsets, W2, gu, dy_perm, dgu, S(stream)));
}

int moe_expert_bwd_dx(const moe_desc* desc, const int32_t* offsets, const void* W1, const void* W3,
                      const void* dgu, void* dx_perm, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(W1) || !need(W3) || !need(dgu) || !need(dx_perm)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_bwd_dxp(*desc, offsets, W1, W3, dgu, dx_perm, S(stream)));
}

// The gathered operand x is addressed with 32-bit offsets.
static bool gather_ok(const moe_desc* d) {
  return d->dtype == MOE_BF16 && (int64_t)d->T * d->d * 2 < (1ll << 31);
}

int moe_expert_gate_up_gather(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token, const void* x,
                              const void* W1, const void* W3, void* gu, void* h, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(row_token) || !need(x) || !need(W1) || !need(W3) || !opt(gu) || !need(h))
    return MOE_ERR_INVALID_ARG;
  if (!gather_ok(desc)) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_gate_up(*desc, offsets, x, W1, W3, gu, h, S(stream), row_token));
}

int moe_grouped_ffn_bwd_dw_gather(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                                  const void* x, const void* h, const void* dgu, const void* dy_perm, void* dW1,
                                  void* dW3, void* dW2, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(row_token) || !need(x) || !need(h) || !need(dgu) || !need(dy_perm) || !need(dW1) ||
      !need(dW3) || !need(dW2))
    return MOE_ERR_INVALID_ARG;
  if (!gather_ok(desc)) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_ffn_bwd_dw(*desc, offsets, x, h, dgu, dy_perm, dW1, dW3, dW2, S(stream), row_token));
}

int moe_grouped_ffn_bwd_dw(const moe_desc* desc, const int32_t* offsets, const void* x_perm, const void* h,
                           const void* dgu, const void* dy_perm, void* dW1, void* dW3, void* dW2, void* ws,
                           size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(x_perm) || !need(h) || !need(dgu) || !need(dy_perm) || !need(dW1) || !need(dW3) ||
      !need(dW2))
    return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_ffn_bwd_dw(*desc, offsets, x_perm, h, dgu, dy_perm, dW1, dW3, dW2, S(stream)));
}

int moe_expert_bwd_dw_gate_up(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token, const void* a,
                              const void* dgu, void* dW1, void* dW3, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !opt(row_token) || !need(a) || !need(dgu) || !need(dW1) || !need(dW3))
    return MOE_ERR_INVALID_ARG;
  if (row_token && !gather_ok(desc)) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_dw_gate_up(*desc, offsets, a, dgu, dW1, dW3, S(stream), row_token));
}

int moe_expert_bwd_dw_down(const moe_desc* desc, const int32_t* offsets, const void* dy_perm, const void* h,
                           void* dW2, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(dy_perm) || !need(h) || !need(dW2)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_dw_down(*desc, offsets, dy_perm, h, dW2, S(stream)));
}

int moe_combine_bwd_gather(const moe_desc* desc, const int32_t* slot_row, const float* topk_w, const void* y_perm,
                           const void* dy, float* row_w, float* dtopk_w, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(slot_row) || !need(topk_w) || !need(y_perm) || !need(dy) || !need(row_w) || !need(dtopk_w))
    return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_combine_bwd(*desc, slot_row, topk_w, y_perm, dy, nullptr, dtopk_w, S(stream), row_w));
}

int moe_expert_bwd_dh_gather(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                             const float* row_w, const void* dy, const void* W2, const void* gu, void* dgu,
                             void* hw, float* dtopk_part, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(row_token) || !need(row_w) || !need(dy) || !need(W2) || !need(gu) || !need(dgu) ||
      !opt(hw) || !opt(dtopk_part))
    return MOE_ERR_INVALID_ARG;
  if (!gather_ok(desc)) return MOE_ERR_UNSUPPORTED;
  return finish(
      moe::launch_bwd_dh_gather(*desc, offsets, row_token, row_w, dy, W2, gu, dgu, hw, dtopk_part, S(stream)));
}

int moe_row_weights(const moe_desc* desc, const int32_t* slot_row, const float* topk_w, float* row_w,
                    void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(slot_row) || !need(topk_w) || !need(row_w)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_row_weights(*desc, slot_row, topk_w, row_w, S(stream)));
}

int moe_dtopk_w_from_parts(const moe_desc* desc, const int32_t* slot_row, const float* dtopk_part,
                           float* dtopk_w, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(slot_row) || !need(dtopk_part) || !need(dtopk_w)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_dtopk_from_parts(*desc, slot_row, dtopk_part, dtopk_w, S(stream)));
}

int moe_expert_bwd_dw_down_gather(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                                  const void* dy, const void* hw, void* dW2, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(row_token) || !need(dy) || !need(hw) || !need(dW2)) return MOE_ERR_INVALID_ARG;
  if (!gather_ok(desc)) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_dw_down_gather(*desc, offsets, row_token, dy, hw, dW2, S(stream)));
}

int moe_unpermute_bwd(const moe_desc* desc, const int32_t* slot_row, const void* dx_perm, const float* dx_add,
                      void* dx, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(slot_row) || !need(dx_perm) || !opt(dx_add) || !need(dx)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_unpermute_bwd(*desc, slot_row, dx_perm, dx_add, dx, S(stream)));
}

int moe_unpermute_router_bwd(const moe_desc* desc, const int32_t* slot_row, const void* dx_perm,
                             const int32_t* topk_idx, const float* dlogits, const void* Wr, void* dx,
                             void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(slot_row) || !need(dx_perm) || !need(topk_idx) || !need(dlogits) || !need(Wr) || !need(dx))
    return MOE_ERR_INVALID_ARG;
  if (desc->renormalize != 1) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_unpermute_router_bwd(*desc, slot_row, dx_perm, topk_idx, dlogits, Wr, dx, S(stream)));
}

int moe_route_bwd(const moe_desc* desc, const float* logits, const int32_t* topk_idx, const float* topk_w,
                  const float* dtopk_w, float* dlogits, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(topk_idx) || !need(topk_w) || !need(dtopk_w) || !need(dlogits)) return MOE_ERR_INVALID_ARG;
  if (desc->renormalize == 0 ? !need(logits) : !opt(logits)) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_route_bwd(*desc, logits, topk_idx, topk_w, dtopk_w, dlogits, S(stream)));
}

int moe_router_bwd(const moe_desc* desc, const void* x, const void* Wr, const float* dlogits, float* dx_router,
                   float* dWr, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(x) || !need(Wr) || !need(dlogits) || !opt(dx_router) || !opt(dWr)) return MOE_ERR_INVALID_ARG;
  if (dWr && (!need(ws) || ws_bytes < moe::router_bwd_workspace(*desc)))
    return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return finish(moe::launch_router_bwd(*desc, x, Wr, dlogits, dx_router, nullptr, dWr, ws, S(stream)));
}

int moe_router_bwd_acc(const moe_desc* desc, const void* x, const void* Wr, const float* dlogits, void* dx,
                       float* dWr, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(x) || !need(Wr) || !need(dlogits) || !opt(dx) || !opt(dWr)) return MOE_ERR_INVALID_ARG;
  if (dWr && (!need(ws) || ws_bytes < moe::router_bwd_workspace(*desc)))
    return ws ? MOE_ERR_WORKSPACE : MOE_ERR_INVALID_ARG;
  return finish(moe::launch_router_bwd(*desc, x, Wr, dlogits, nullptr, dx, dWr, ws, S(stream)));
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error; }

int moe_fp8_quantize(const void* w, int dtype, int64_t n, uint8_t* q, float* scales, void* stream) {
  if (!need(w) || !need(q) || !need(scales) || n < 0 || n % 128) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_fp8_quantize(w, dtype, n, q, scales, S(stream)));
}

int moe_fp8_quantize_pow2(const void* w, int dtype, int64_t n, uint8_t* q, uint8_t* e8, void* stream) {
  if (!need(w) || !need(q) || !need(e8) || n < 0 || n % 128) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_fp8_quantize_pow2(w, dtype, n, q, e8, S(stream)));
}

int moe_fp8_quantize_pow2_rows(const void* w, int dtype, int64_t rows, int64_t cols, const int32_t* nrows,
                               uint8_t* q, uint8_t* e8, int64_t e8_ld, void* stream) {
  if (!need(w) || !need(q) || !e8 || (reinterpret_cast<uintptr_t>(nrows) & 3u) || rows < 0 || cols < 128 || cols % 128 ||
      e8_ld < cols / 128 || e8_ld > cols / 128 + 15)
    return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_fp8_quantize_pow2_rows(w, dtype, rows, cols, nrows, q, e8, e8_ld, S(stream)));
}

int moe_fp8_dequantize(const uint8_t* q, const float* scales, int64_t n, void* w, void* stream) {
  if (!need(w) || !need(q) || !need(scales) || n < 0 || n % 128) return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_fp8_dequantize(q, scales, n, w, S(stream)));
}

// FP8 weights in the GEMMs: bf16 activations, and K (d for gate/up, f for
// down) in whole 128-value scale blocks.
static bool q8_ok(const moe_desc* d) { return d->dtype == MOE_BF16 && d->d % 128 == 0 && d->f % 128 == 0; }

int moe_expert_gate_up_fp8(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token, const void* a,
                           const uint8_t* W1q, const float* W1s, const uint8_t* W3q, const float* W3s, void* gu,
                           void* h, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !opt(row_token) || !need(a) || !need(W1q) || !need(W1s) || !need(W3q) || !need(W3s) ||
      !opt(gu) || !need(h))
    return MOE_ERR_INVALID_ARG;
  if (!q8_ok(desc) || (row_token && !gather_ok(desc))) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_gate_up_q8(*desc, offsets, a, row_token, W1q, W1s, W3q, W3s, gu, h, S(stream)));
}

int moe_expert_down_fp8(const moe_desc* desc, const int32_t* offsets, const void* h, const uint8_t* W2q,
                        const float* W2s, void* y_perm, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(h) || !need(W2q) || !need(W2s) || !need(y_perm)) return MOE_ERR_INVALID_ARG;
  if (!q8_ok(desc)) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_down_q8(*desc, offsets, h, W2q, W2s, y_perm, S(stream)));
}

int moe_expert_gate_up_fp8mm(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                             const uint8_t* xq, const uint8_t* xs, const uint8_t* W1q, const uint8_t* W1s,
                             const uint8_t* W3q, const uint8_t* W3s, void* gu, void* h, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(row_token) || !need(xq) || !need(xs) || !need(W1q) || !need(W1s) || !need(W3q) ||
      !need(W3s) || !opt(gu) || !need(h))
    return MOE_ERR_INVALID_ARG;
  // bf16 outputs; d in whole groups of four 128-code blocks (so a row's scale
  // bytes come as aligned dwords); the gathered codes addressed in 32 bits
  if (desc->dtype != MOE_BF16 || desc->d % 512 || (int64_t)desc->T * desc->d >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_gate_up_f8(*desc, offsets, row_token, xq, xs, W1q, W1s, W3q, W3s, gu, h, S(stream)));
}

int moe_expert_down_fp8mm(const moe_desc* desc, const int32_t* offsets, const uint8_t* hq, const uint8_t* hs,
                          const uint8_t* W2q, const uint8_t* W2s, void* y_perm, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!need(offsets) || !need(hq) || !need(hs) || !need(W2q) || !need(W2s) || !need(y_perm))
    return MOE_ERR_INVALID_ARG;
  // bf16 output; f in whole 128-code blocks; h's codes addressed in 32 bits
  const int64_t rc_rows = (int64_t)desc->T * std::min(desc->k, desc->num_local);
  if (desc->dtype != MOE_BF16 || desc->f % 128 || rc_rows * desc->f >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  return finish(moe::launch_down_f8(*desc, offsets, hq, hs, W2q, W2s, y_perm, S(stream)));
}

int moe_hold_cus(int workgroups, int lds_bytes, int microseconds, void* stream) {
  if (workgroups < 1 || workgroups > 4096 || lds_bytes < 4 || lds_bytes > 160 * 1024 || microseconds < 0 ||
      microseconds > 1000000)
    return MOE_ERR_INVALID_ARG;
  return finish(moe::launch_hold(workgroups, lds_bytes, microseconds, S(stream)));
}

}  // extern "C"
