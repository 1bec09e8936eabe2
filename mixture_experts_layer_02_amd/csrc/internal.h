// Host-side interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include "common.h"

namespace moe {

int num_cus();
hipError_t launch_hold(int workgroups, int lds_bytes, int microseconds, hipStream_t s);
hipError_t launch_gate_up_q8(const moe_desc& d, const int32_t* offsets, const void* a, const int32_t* row_token,
                             const uint8_t* W1q, const float* s1, const uint8_t* W3q, const float* s3, void* gu,
                             void* h, hipStream_t s);
hipError_t launch_gate_up_f8(const moe_desc& d, const int32_t* offsets, const int32_t* row_token, const uint8_t* xq,
                             const uint8_t* xs, const uint8_t* W1q, const uint8_t* W1s, const uint8_t* W3q,
                             const uint8_t* W3s, void* gu, void* h, hipStream_t s);
hipError_t launch_down_f8(const moe_desc& d, const int32_t* offsets, const uint8_t* hq, const uint8_t* hs,
                          const uint8_t* W2q, const uint8_t* W2s, void* y_perm, hipStream_t s);
// Bytes per row of power-of-two block scales for rows of n codes, as the FP8
// GEMMs read them: n/128, rounded up to a multiple of 4.
inline int fp8_scale_row_bytes(int64_t n) { return (int)(((n / 128) + 3) / 4 * 4); }
hipError_t launch_fp8_quantize_pow2_rows(const void* w, int dtype, int64_t rows, int64_t cols, const int32_t* nrows,
                                         uint8_t* q, uint8_t* e8, int64_t e8_ld, hipStream_t s);
hipError_t launch_down_q8(const moe_desc& d, const int32_t* offsets, const void* h, const uint8_t* W2q,
                          const float* s2, void* y_perm, hipStream_t s);
hipError_t launch_fp8_quantize(const void* w, int dtype, int64_t n, uint8_t* q, float* scales, hipStream_t s);
hipError_t launch_fp8_dequantize(const uint8_t* q, const float* scales, int64_t n, void* w, hipStream_t s);
hipError_t launch_fp8_quantize_pow2(const void* w, int dtype, int64_t n, uint8_t* q, uint8_t* e8, hipStream_t s);

size_t permute_workspace(const moe_desc& d);
// Size of the allocation-free permute's fixed device scratch (4 MiB per device).
constexpr size_t PERMUTE_SCRATCH_BYTES = (size_t)4 << 20;
hipError_t launch_permute_noalloc(const moe_desc& d, const int32_t* idx, const void* x, int32_t* counts,
                                  int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm,
                                  hipStream_t s);
size_t router_bwd_workspace(const moe_desc& d);

size_t router_logits_workspace(const moe_desc& d);
hipError_t launch_router_logits(const moe_desc& d, const void* x, const void* Wr, const float* bias,
                                float* logits, void* ws, hipStream_t s);
hipError_t launch_route(const moe_desc& d, const float* logits, int n_groups, int32_t* idx, float* w,
                        hipStream_t s);
hipError_t launch_route_bwd(const moe_desc& d, const float* logits, const int32_t* idx, const float* w,
                            const float* dw, float* dlogits, hipStream_t s);
hipError_t launch_permute(const moe_desc& d, const int32_t* idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm, void* ws,
                          hipStream_t s);
hipError_t launch_combine(const moe_desc& d, const int32_t* slot_row, const float* w, const void* y_perm,
                          void* y, hipStream_t s);
hipError_t launch_combine_bwd(const moe_desc& d, const int32_t* slot_row, const float* w, const void* y_perm,
                              const void* dy, void* dy_perm, float* dw, hipStream_t s, float* row_w = nullptr);
hipError_t launch_bwd_dh_gather(const moe_desc& d, const int32_t* offsets, const int32_t* row_token,
                                const float* row_w, const void* dy, const void* W2, const void* gu, void* dgu,
                                void* hw, float* dtopk_part, hipStream_t s);
hipError_t launch_row_weights(const moe_desc& d, const int32_t* slot_row, const float* w, float* row_w,
                              hipStream_t s);
hipError_t launch_dtopk_from_parts(const moe_desc& d, const int32_t* slot_row, const float* part, float* dtopk_w,
                                   hipStream_t s);
// Partial sums per row written by the dH product with dy read in place: two per
// 256-wide n-tile of f.
inline int dtopk_parts(const moe_desc& d) { return 2 * (int)((d.f + 255) / 256); }
hipError_t launch_dw_down_gather(const moe_desc& d, const int32_t* offsets, const int32_t* row_token,
                                 const void* dy, const void* hw, void* dW2, hipStream_t s);
hipError_t launch_unpermute_bwd(const moe_desc& d, const int32_t* slot_row, const void* dx_perm,
                                const float* dx_add, void* dx, hipStream_t s);
hipError_t launch_unpermute_router_bwd(const moe_desc& d, const int32_t* slot_row, const void* dx_perm,
                                       const int32_t* topk_idx, const float* dlogits, const void* Wr, void* dx,
                                       hipStream_t s);
hipError_t launch_gate_up(const moe_desc& d, const int32_t* offsets, const void* x_perm, const void* W1,
                          const void* W3, void* gu, void* h, hipStream_t s,
                          const int32_t* row_token = nullptr);
hipError_t launch_down(const moe_desc& d, const int32_t* offsets, const void* h, const void* W2, void* y_perm,
                       hipStream_t s);
hipError_t launch_bwd_dh(const moe_desc& d, const int32_t* offsets, const void* W2, const void* gu,
                         const void* dy_perm, void* dgu, hipStream_t s);
hipError_t launch_bwd_dxp(const moe_desc& d, const int32_t* offsets, const void* W1, const void* W3,
                          const void* dgu, void* dx_perm, hipStream_t s);
hipError_t launch_ffn_bwd_dw(const moe_desc& d, const int32_t* offsets, const void* x_perm, const void* h,
                             const void* dgu, const void* dy_perm, void* dW1, void* dW3, void* dW2,
                             hipStream_t s,
                             const int32_t* row_token = nullptr);
hipError_t launch_dw_gate_up(const moe_desc& d, const int32_t* offsets, const void* x_perm, const void* dgu,
                             void* dW1, void* dW3, hipStream_t s, const int32_t* row_token = nullptr);
hipError_t launch_dw_down(const moe_desc& d, const int32_t* offsets, const void* dy_perm, const void* h, void* dW2,
                          hipStream_t s);
hipError_t launch_router_bwd(const moe_desc& d, const void* x, const void* Wr, const float* dlogits,
                             float* dx_router, void* dx_acc, float* dWr, void* ws, hipStream_t s);

}  // namespace moe
