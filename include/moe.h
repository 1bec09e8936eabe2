/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE expert-layer library, libmoe.so.
 *
 * The layer is the sparse MoE block of one GPU's expert-parallel share, as
 * described by the Aurora page ("Scalable Pretraining of Large Mixture of
 * Experts Language Models on Aurora Super Computer", section 3.1
 * FastSparseMoE, Algorithm 1): router, softmax + top-k, per-expert token
 * counting with a prefix sum, index generation and gather, a grouped SwiGLU
 * expert MLP over all local experts, and the weighted output reduction; plus
 * the backward of each step.  Shapes of the 1T model come from the Domyn page
 * ("Training a 1T-Params MoE on EU public infrastructure", model table:
 * hidden 6144, 384 experts, top-8, expert hidden 1792).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except `desc` is a DEVICE pointer, owned by the
 *    caller, which allocates and frees it.  The library never allocates,
 *    frees or synchronises, keeps no per-call global state and is
 *    re-entrant; calls are asynchronous on `stream` (a hipStream_t, NULL =
 *    the default stream).
 *  - Matrices are row-major.  "dtype" tensors are float32 (MOE_F32) or
 *    bfloat16 bits (MOE_BF16) per desc->dtype; logits, routing weights,
 *    dlogits, dtopk_w and every weight gradient are always float32.
 *  - Weights use the layout of a linear layer (out x in), concatenated over
 *    the local experts (the page concatenates each expert's gate_proj,
 *    up_proj and down_proj weights per rank):  Wr [E][d],
 *    W1 = gate [NL][f][d], W3 = up [NL][f][d], W2 = down [NL][d][f].
 *  - NL = desc->num_local experts [expert_begin, expert_begin+NL) are local.
 *    R = offsets[NL] (on the device) is the number of routed rows; row
 *    buffers are sized R_cap = T * min(k, NL) rows and rows >= R are never
 *    written.  No entry point needs R on the host.
 *  - Every call validates its arguments on the host before any launch and
 *    returns MOE_OK or a negative error code; no exception crosses the ABI.
 *    Device inputs must hold finite values (not checked).
 *  - Pointers must be 16-byte aligned.  d and f must be multiples of 64,
 *    E a multiple of 8 and at most 1024, 1 <= k <= min(E, 32), T >= 1,
 *    0 <= expert_begin,
 *    1 <= num_local, expert_begin + num_local <= E.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad sizes, wrong struct_size */
  MOE_ERR_UNSUPPORTED = -2, /* dtype or shape outside the supported set above */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = -4          /* a HIP launch failed; see moe_last_error() */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

/* Order in which the persistent bf16 GEMM workgroups take output tiles
 * (Domyn page, section "Dynamic tile scheduling in SonicMoE").  STATIC: each
 * workgroup's list of tiles is fixed at launch.  DYNAMIC: workgroups take
 * the next tile from shared atomic counters when they are free (per-XCD
 * queues, then each other's), so workgroups that start late - their CUs
 * held by another kernel - do not delay the end of the product.  Outputs are
 * bitwise identical under both. */
enum moe_tile_schedule { MOE_SCHEDULE_STATIC = 0, MOE_SCHEDULE_DYNAMIC = 1 };

/* Which call a workspace size is asked for. */
enum moe_op {
  MOE_OP_ROUTER_LOGITS = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_GROUPED_FFN = 2,
  MOE_OP_FFN_BWD_DX = 3,
  MOE_OP_FFN_BWD_DW = 4,
  MOE_OP_ROUTER_BWD = 5
};

typedef struct moe_desc {
  uint32_t struct_size;     /* = sizeof(moe_desc) */
  int32_t T;                /* tokens on this GPU (Algorithm 1's T) */
  int32_t d;                /* hidden size (the page's H) */
  int32_t f;                /* expert hidden size */
  int32_t E;                /* router width: experts in the whole layer (the page's N) */
  int32_t k;                /* experts selected per token (the page's K) */
  int32_t expert_begin;     /* first local expert (the page's n_start) */
  int32_t num_local;        /* local experts (the page's NR) */
  int32_t dtype;            /* enum moe_dtype */
  int32_t renormalize;      /* 1: top-k probabilities divided by their sum; 0: raw softmax probabilities */
  int32_t tile_schedule;    /* enum moe_tile_schedule: order of the grouped GEMMs' output tiles */
  int32_t* tile_counters;   /* MOE_SCHEDULE_DYNAMIC: device int32[16], all zero before the first call;
                               every GEMM launch leaves them zero again.  Calls that share one array
                               must not run concurrently (same stream, or ordered by events).  Ignored
                               (may be NULL) for MOE_SCHEDULE_STATIC. */
  int32_t wgrad_dtype;      /* enum moe_dtype of the expert weight gradients dW1, dW3, dW2 written by
                               the B4 calls: MOE_F32 (0) float32, or MOE_BF16 (dtype MOE_BF16 only,
                               else MOE_ERR_UNSUPPORTED) bf16 - each sum accumulated in float32 and
                               rounded once to bf16 (nearest, ties to even) at the store, the
                               gradients computed in bf16 and reduced in fp32 of the Domyn page,
                               section "BF16 gradient all-to-all with FP32 accumulation" */
} moe_desc;

/* Host-only query: bytes of device workspace that call `op` needs for desc
 * (0 when it needs none).  Returns MOE_ERR_INVALID_ARG on a bad desc/op. */
int moe_workspace_size(const moe_desc* desc, int op, size_t* bytes);

/* A1, router scores (Aurora page, Algorithm 1 stage 1: the router is a linear
 * layer producing one logit per token and expert).
 *   x [T][d] dtype, Wr [E][d] dtype, bias [E] float32 or NULL (added to every
 *   token's logits), logits [T][E] float32 out.  Accumulation is float32.
 *   ws: moe_workspace_size(MOE_OP_ROUTER_LOGITS) bytes (may be NULL when that
 *   is 0).  For bf16 shapes with fewer 256x256 output tiles than 256, the
 *   product is split over d into whole 64-wide chunks whose float32 partial
 *   sums go to ws and are added in chunk order, then the bias; the split
 *   depends on the shape only, so results are the same on every call.
 *   Errors: MOE_ERR_WORKSPACE (ws too small), MOE_ERR_INVALID_ARG (ws NULL or
 *   misaligned when the query is not 0). */
int moe_router_logits(const moe_desc* desc, const void* x, const void* Wr, const float* bias,
                      float* logits, void* ws, size_t ws_bytes, void* stream);

/* A2, softmax + top-k (+ renormalisation) (Algorithm 1 stage 1).
 *   logits [T][E] float32 -> topk_idx [T][k] int32, topk_w [T][k] float32.
 *   Slot j holds the j-th largest logit; equal logits (and +0.0 / -0.0) go to
 *   the lower expert index.  renormalize=1: w_j = exp(L_j - L_0) / sum over
 *   the k selected of exp(L_i - L_0); renormalize=0: w_j = softmax over all
 *   E experts at the selected index. */
int moe_route(const moe_desc* desc, const float* logits, int32_t* topk_idx, float* topk_w,
              void* stream);

/* A2 with group-limited selection (Domyn page, section "Group-limited expert
 * routing": the experts form groups of consecutive experts, one per
 * expert-parallel rank, and the router takes the same number from each).
 *   Group g is experts [g*E/n_groups, (g+1)*E/n_groups); every token takes
 *   its k/n_groups best experts of every group, by the same order as
 *   moe_route (logit descending, lower index on ties), so every group
 *   receives exactly T*k/n_groups selections.  Slots hold the k taken
 *   experts in that order; weights as in moe_route (renormalize applies).
 *   n_groups = 1 is moe_route.  Errors: MOE_ERR_INVALID_ARG unless
 *   1 <= n_groups <= 64 divides both E and k.  Layouts and ownership as in
 *   moe_route. */
int moe_route_grouped(const moe_desc* desc, const float* logits, int n_groups, int32_t* topk_idx,
                      float* topk_w, void* stream);

/* A3 + A4, token counting, prefix sum, index generation and gather
 * (Algorithm 1 stages 2, 3 and the stage-4 gather).
 *   topk_idx [T][k] int32 (values in [0, E)), x [T][d] dtype (may be NULL:
 *   indices only).  A token's k experts must be distinct (moe_route and
 *   moe_route_grouped always give distinct experts; a routing supplied by
 *   the caller must too).  Not checked: a repeated expert is counted once
 *   and both of its slots get the same row, so counts no longer sum to T*k
 *   and the backward's per-row writes collide;
 *   counts [E] int32: selections of every expert, local or not;
 *   offsets [NL+1] int32: exclusive prefix sum of the local counts
 *     (offsets[NL] = R), the page's cum_token_counts;
 *   row_token [R_cap] int32: token of each routed row (the page's
 *     input_indices); rows of one expert are in ascending token order;
 *   slot_row [T][k] int32: row of each slot, or -1 when its expert is not
 *     local (the page's output_indices / selected_expert_indices);
 *   x_perm [R_cap][d] dtype: x_perm[r] = x[row_token[r]] (bit copy).
 *   ws: moe_workspace_size(MOE_OP_PERMUTE) bytes. */
int moe_permute(const moe_desc* desc, const int32_t* topk_idx, const void* x, int32_t* counts,
                int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm,
                void* ws, size_t ws_bytes, void* stream);

/* moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that
 * forbid it): the same kernels and bitwise the same outputs, with the
 * per-block counts and bases kept in a fixed scratch array of 4 MiB that the
 * library holds in each device's memory for the life of the process, instead
 * of a caller workspace.  The call allocates nothing: no hipMalloc, no
 * allocating library routine.  Arguments, layouts and ownership as in
 * moe_permute (the caller still passes every input and output).
 *   Limit: (E + num_local) * ceil(T / 256) * 4 bytes <= 4 MiB (e.g. E = 384,
 *   96 local: T up to 559,104 tokens); a larger shape returns
 *   MOE_ERR_UNSUPPORTED with the sizes in moe_last_error().
 *   The scratch is shared by every call on one device and keeps the last
 *   call's contents (each call rewrites all it reads): calls that may
 *   overlap on one device (different streams, or different host threads
 *   without ordering) race and must be serialised by the caller. */
int moe_permute_noalloc(const moe_desc* desc, const int32_t* topk_idx, const void* x,
                        int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                        void* x_perm, void* stream);

/* A5 + A6, the grouped SwiGLU expert MLP (Algorithm 1 stage 4: Grouped_mm of
 * gate and up, Silu(gate) * up, Grouped_mm of down, with segment boundaries
 * offsets).  For each local expert n and row r in [offsets[n], offsets[n+1]):
 *   G = x_perm[r] W1[n]^T, U = x_perm[r] W3[n]^T, h[r] = silu(G) * U,
 *   y_perm[r] = h[r] W2[n]^T.
 *   x_perm [R_cap][d], h [R_cap][f], y_perm [R_cap][d] dtype;
 *   gu [R_cap][2f] dtype or NULL: when given, G is saved in columns [0, f)
 *   and U in [f, 2f) for the backward.  Accumulation is float32; h, gu and
 *   y_perm are rounded to dtype. */
int moe_grouped_ffn(const moe_desc* desc, const int32_t* offsets, const void* x_perm,
                    const void* W1, const void* W3, const void* W2, void* gu, void* h,
                    void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* A5 alone: the gate/up grouped GEMM with the fused SwiGLU epilogue, i.e. the
 * first half of moe_grouped_ffn (h and, when gu != NULL, G | U as above). */
int moe_expert_gate_up(const moe_desc* desc, const int32_t* offsets, const void* x_perm, const void* W1,
                       const void* W3, void* gu, void* h, void* stream);

/* A4 + A5 fused (Domyn page, section "Dynamic tile scheduling in SonicMoE":
 * SonicMoE runs the expert GEMMs straight on the token-dispatch layout,
 * without a permuted copy of the tokens): moe_expert_gate_up with
 * x_perm[r] read as x[row_token[r]] inside the GEMM's operand loads, so that
 * x_perm is never written (moe_permute may then be called with x = NULL).
 *   row_token [R_cap] int32 from moe_permute; x [T][d] bf16.  Results are
 *   bitwise those of moe_expert_gate_up on x_perm.  MOE_ERR_UNSUPPORTED
 *   unless dtype is MOE_BF16 and T*d*2 < 2^31 (x is addressed with 32-bit
 *   offsets). */
int moe_expert_gate_up_gather(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                              const void* x, const void* W1, const void* W3, void* gu, void* h,
                              void* stream);

/* A6 alone: the down grouped GEMM, y_perm[r] = h[r] W2[n]^T (second half of
 * moe_grouped_ffn). */
int moe_expert_down(const moe_desc* desc, const int32_t* offsets, const void* h, const void* W2,
                    void* y_perm, void* stream);

/* A7, weighted output reduction (Algorithm 1 stage 5 forward):
 *   y[t] = sum over slots j = 0..k-1 with slot_row[t][j] >= 0 of
 *          topk_w[t][j] * y_perm[slot_row[t][j]], summed in float32 in slot
 *   order; y [T][d] dtype (0 for a token without a local slot). */
int moe_combine(const moe_desc* desc, const int32_t* slot_row, const float* topk_w,
                const void* y_perm, void* y, void* stream);

/* B1, backward of the output reduction (Algorithm 1 stage 5 backward):
 *   dy_perm[slot_row[t][j]] = topk_w[t][j] * dy[t]    ([R_cap][d] dtype),
 *   dtopk_w[t][j] = <y_perm[slot_row[t][j]], dy[t]>   ([T][k] float32; 0 for
 *   non-local slots).  dy [T][d] dtype. */
int moe_combine_bwd(const moe_desc* desc, const int32_t* slot_row, const float* topk_w,
                    const void* y_perm, const void* dy, void* dy_perm, float* dtopk_w,
                    void* stream);

/* B2 + B3, backward of the expert MLP with respect to its input (derived from
 * Algorithm 1 stage 4 by differentiation):
 *   dH = dy_perm W2[n], dU = dH * silu(G), dG = dH * U * silu'(G),
 *   dx_perm = dG W1[n] + dU W3[n].
 *   gu [R_cap][2f] dtype (as saved by moe_grouped_ffn), dy_perm [R_cap][d];
 *   dgu [R_cap][2f] dtype out (dG in [0, f), dU in [f, 2f)),
 *   dx_perm [R_cap][d] dtype out. */
int moe_grouped_ffn_bwd_dx(const moe_desc* desc, const int32_t* offsets, const void* W1,
                           const void* W3, const void* W2, const void* gu, const void* dy_perm,
                           void* dgu, void* dx_perm, void* ws, size_t ws_bytes, void* stream);

/* B2 alone: dH = dy_perm W2[n] with the SwiGLU backward fused into the
 * epilogue -> dgu (first half of moe_grouped_ffn_bwd_dx). */
int moe_expert_bwd_dh(const moe_desc* desc, const int32_t* offsets, const void* W2, const void* gu,
                      const void* dy_perm, void* dgu, void* stream);

/* B3 alone: dx_perm = dG W1[n] + dU W3[n], one grouped GEMM with K = 2f over
 * dgu (second half of moe_grouped_ffn_bwd_dx). */
int moe_expert_bwd_dx(const moe_desc* desc, const int32_t* offsets, const void* W1, const void* W3,
                      const void* dgu, void* dx_perm, void* stream);

/* B4, weight gradients of the expert MLP (variable-K grouped GEMMs):
 *   dW1[n] = dG_n^T x_perm_n, dW3[n] = dU_n^T x_perm_n  ([NL][f][d]),
 *   dW2[n] = dy_perm_n^T h_n                           ([NL][d][f]),
 *   where _n is the row segment of expert n, as float32 or bf16 by
 *   desc->wgrad_dtype (here and in every B4 call below).  They are
 *   overwritten, not accumulated; an expert with no rows gets exact zeros. */
int moe_grouped_ffn_bwd_dw(const moe_desc* desc, const int32_t* offsets, const void* x_perm,
                           const void* h, const void* dgu, const void* dy_perm, void* dW1,
                           void* dW3, void* dW2, void* ws, size_t ws_bytes, void* stream);

/* B4 with the gather fused (as moe_expert_gate_up_gather): dW1 and dW3 read
 * the rows of x_perm as x[row_token[r]] inside the GEMM's operand loads.
 *   Results are bitwise those of moe_grouped_ffn_bwd_dw on x_perm; same
 *   conditions as moe_expert_gate_up_gather. */
int moe_grouped_ffn_bwd_dw_gather(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                                  const void* x, const void* h, const void* dgu, const void* dy_perm,
                                  void* dW1, void* dW3, void* dW2, void* stream);

/* B4, first launch alone: dW1[n] = dG_n^T a_n and dW3[n] = dU_n^T a_n
 * ([NL][f][d], overwritten; exact zeros for an expert with no rows).
 *   row_token NULL: a is x_perm [R_cap][d]; else a is x [T][d] and k-row r
 *   of the product reads x[row_token[r]] (bf16 only, x under 2 GiB, else
 *   MOE_ERR_UNSUPPORTED).  dgu [R_cap][2f] as written by the dH step.
 *   Results are bitwise those of moe_grouped_ffn_bwd_dw's dW1 and dW3. */
int moe_expert_bwd_dw_gate_up(const moe_desc* desc, const int32_t* offsets,
                              const int32_t* row_token, const void* a, const void* dgu,
                              void* dW1, void* dW3, void* stream);

/* B4, second launch alone: dW2[n] = dy_perm_n^T h_n ([NL][d][f],
 * overwritten; exact zeros for an expert with no rows); bitwise
 * moe_grouped_ffn_bwd_dw's dW2. */
int moe_expert_bwd_dw_down(const moe_desc* desc, const int32_t* offsets, const void* dy_perm,
                           const void* h, void* dW2, void* stream);

/* The backward with dy read in place (Domyn page, section "Dynamic tile
 * scheduling in SonicMoE": the expert GEMMs run on the dispatch layout, with
 * no permuted copies).  dy_perm[r] = w_r dy[row_token[r]] is never stored;
 * its routing weight w_r is applied inside the products instead.  bf16 only,
 * x and dy under 2 GiB (else MOE_ERR_UNSUPPORTED).  In order:
 *
 * B1: dtopk_w [T][k] float32 as in moe_combine_bwd, and row_w [R_cap]
 *   float32, row_w[slot_row[t][j]] = topk_w[t][j] for every local slot (the
 *   weight row r carries).  No dy_perm is written. */
int moe_combine_bwd_gather(const moe_desc* desc, const int32_t* slot_row, const float* topk_w,
                           const void* y_perm, const void* dy, float* row_w, float* dtopk_w,
                           void* stream);

/* B1 without the dot products: row_w [R_cap] float32, row_w[slot_row[t][j]]
 *   = topk_w[t][j] for every local slot (the weight row r carries), for the
 *   dH product below; dtopk_w then comes from that product's partial sums
 *   (moe_dtopk_w_from_parts), since <dy[t], y_perm[r]> = <dy[t] W2[n], h[r]>
 *   for row r = slot_row[t][j] of expert n (y_perm[r] = h[r] W2[n]^T). */
int moe_row_weights(const moe_desc* desc, const int32_t* slot_row, const float* topk_w, float* row_w,
                    void* stream);

/* B2: dH[r] = row_w[r] * (dy[row_token[r]] W2[n]) with the SwiGLU backward
 *   fused as in moe_expert_bwd_dh -> dgu [R_cap][2f]; and, when hw is not
 *   NULL, hw[r] = row_w[r] * silu(G) * U [R_cap][f] bf16 from the saved
 *   G | U (gu), the operand of the dW2 product below; and, when dtopk_part
 *   is not NULL, dtopk_part [R_cap][P] float32, P = 2 * ceil(f / 256): the
 *   sums of (dy[row_token[r]] W2[n]) * silu(G) * U over consecutive 128-wide
 *   column blocks of f (with G, U the saved bf16 values).  dy [T][d]. */
int moe_expert_bwd_dh_gather(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                             const float* row_w, const void* dy, const void* W2, const void* gu,
                             void* dgu, void* hw, float* dtopk_part, void* stream);

/* B1's dot products from B2's partial sums: dtopk_w[t][j] = the sum, in
 *   order, of dtopk_part[slot_row[t][j]][0 .. P-1] for a local slot, 0 for a
 *   slot whose expert is not local (as moe_combine_bwd).  dtopk_w [T][k]
 *   float32. */
int moe_dtopk_w_from_parts(const moe_desc* desc, const int32_t* slot_row, const float* dtopk_part,
                           float* dtopk_w, void* stream);

/* B4, dW2 with dy read in place: dW2[n] = sum over rows r of expert n of
 *   dy[row_token[r]]^T hw[r]  ([NL][d][f], overwritten; exact zeros
 *   for an expert with no rows).  dW1 | dW3 come from
 *   moe_expert_bwd_dw_gate_up with row_token. */
int moe_expert_bwd_dw_down_gather(const moe_desc* desc, const int32_t* offsets,
                                  const int32_t* row_token, const void* dy, const void* hw,
                                  void* dW2, void* stream);

/* B5a, backward of the gather: dx[t] = dx_add[t] + sum over local slots j of
 *   dx_perm[slot_row[t][j]], summed in float32; dx [T][d] dtype out;
 *   dx_add [T][d] float32 or NULL (e.g. the router path's input gradient). */
int moe_unpermute_bwd(const moe_desc* desc, const int32_t* slot_row, const void* dx_perm,
                      const float* dx_add, void* dx, void* stream);

/* B5b, backward of softmax + top-k (+ renormalisation):
 *   renormalize=1: dlogits[t][m] = w_m (dw_m - sum_j w_j dw_j) for the k
 *   selected m (local or not), 0 elsewhere;
 *   renormalize=0: dlogits[t][e] = p_e (g_e - sum_j w_j dw_j) with p the
 *   softmax of logits over all E and g_e = dw_j at e = topk_idx[t][j], else
 *   0 (needs logits; it may be NULL when renormalize=1).
 *   dlogits [T][E] float32 out. */
int moe_route_bwd(const moe_desc* desc, const float* logits, const int32_t* topk_idx,
                  const float* topk_w, const float* dtopk_w, float* dlogits, void* stream);

/* B5c, backward of the router linear layer:
 *   dx_router = dlogits Wr   ([T][d] float32 out),
 *   dWr = dlogits^T x        ([E][d] float32 out, overwritten).
 *   On the bf16 path dlogits is rounded to bf16 for the matrix cores. */
int moe_router_bwd(const moe_desc* desc, const void* x, const void* Wr, const float* dlogits,
                   float* dx_router, float* dWr, void* ws, size_t ws_bytes, void* stream);

/* B5c with the router path added into the token gradient in place:
 *   dx += dlogits Wr  (dx [T][d] in the descriptor's dtype, in and out; on
 *                      the bf16 path the sum is rounded once to bf16),
 *   dWr = dlogits^T x ([E][d] float32 out, overwritten).
 * Either output may be NULL.  The layer's token gradient is the unpermute
 * sum of its expert rows plus this router term (Aurora page, Algorithm 1,
 * stage 1, differentiated); called after moe_unpermute_bwd with dx_add NULL,
 * it needs no float [T][d] intermediate.  Workspace and errors as for
 * moe_router_bwd. */
int moe_router_bwd_acc(const moe_desc* desc, const void* x, const void* Wr, const float* dlogits, void* dx,
                       float* dWr, void* ws, size_t ws_bytes, void* stream);

/* B5a and the dx half of B5c in one pass, for renormalised weights:
 *   dx[t] = sum over local slots j of dx_perm[slot_row[t][j]]
 *         + sum over all k slots j of dlogits[t][e_j] * Wr[e_j],  e_j = topk_idx[t][j].
 * With the weights renormalised over the selection (Aurora page, Algorithm
 * 1, stage 1, as read with renormalisation), dlogits is zero outside the k
 * selected experts (moe_route_bwd), so dlogits[t] Wr is that sum of k rows
 * of Wr; this replaces moe_unpermute_bwd followed by moe_router_bwd_acc
 * with dx (dWr still comes from moe_router_bwd_acc with dx NULL).
 *   slot_row [T][k] int32, dx_perm [R_cap][d], topk_idx [T][k] int32 (the
 *   selection moe_route wrote; entries outside [0, E) are clamped into it),
 *   dlogits [T][E] float32 (moe_route_bwd's output), Wr [E][d], dx [T][d]
 *   out, all but the index arrays and dlogits in the descriptor's dtype.
 *   float32 sums (expert rows in slot order, then router rows in slot
 *   order), one rounding at the store.
 * Errors: MOE_ERR_UNSUPPORTED when desc->renormalize is 0 (dlogits is then
 * dense: use moe_unpermute_bwd and moe_router_bwd_acc); MOE_ERR_INVALID_ARG
 * for a NULL pointer or a bad descriptor. */
int moe_unpermute_router_bwd(const moe_desc* desc, const int32_t* slot_row, const void* dx_perm,
                             const int32_t* topk_idx, const float* dlogits, const void* Wr, void* dx,
                             void* stream);

/* Static description of a status code. */
const char* moe_status_str(int status);

/* Text of the last HIP error seen by a failing call on this thread. */
const char* moe_last_error(void);

/* FP8 expert weights (Domyn page, section "FP8 expert weight all-gather":
 * the weights are cut into blocks of 128 values, each block is scaled to the
 * E4M3 range and cast, with one float32 scale per block, and the receivers
 * dequantise to bf16 before the expert GEMMs; the error is up to about 6% of
 * the block maximum per value).
 *   w [n] (MOE_BF16 or MOE_F32 as `dtype`), blocks of 128 consecutive values
 *   in memory order (the rows of W1/W3 [NL][f][d] and W2 [NL][d][f] when d
 *   and f are multiples of 128); q [n] uint8 E4M3 codes (OCP, no infinity,
 *   448 the largest); scales [n/128] float32.  Per block: amax = max |w|,
 *   scale = amax / 448, each code = the E4M3 value nearest to w * (448 / amax)
 *   (ties to even, after clamping to +-448); a block of zeros has scale 0 and
 *   codes 0.  Errors: MOE_ERR_INVALID_ARG if n is not a multiple of 128 or a
 *   pointer is NULL or not 16-byte aligned. */
int moe_fp8_quantize(const void* w, int dtype, int64_t n, uint8_t* q, float* scales, void* stream);

/* The inverse: w [n] bf16 = decode(q) * scale, in float32 rounded to nearest
 * even.  Same layouts and errors as moe_fp8_quantize. */
int moe_fp8_dequantize(const uint8_t* q, const float* scales, int64_t n, void* w, void* stream);

/* E4M3 blocks of 128 with power-of-two scales (Domyn page, section "FP8
 * expert weight all-gather", in the form a block-scaled FP8 matrix
 * instruction applies; used for the weights and the activations of the FP8
 * matrix-core GEMM below).  Per block: e = the least integer with
 * amax <= 448 * 2^e (so the block maximum lands in (224, 448]); each code =
 * the E4M3 value nearest to w * 2^-e (exact scaling; ties to even); the
 * scale leaves as its E8M0 byte e8 = e + 127.  A block of zeros gets
 * e8 = 127 and zero codes.
 *   w [n] (MOE_BF16 or MOE_F32 as `dtype`), blocks of 128 consecutive values
 *   (the rows of x [T][d] or W1/W3 [NL][f][d] when d is a multiple of 128);
 *   q [n] uint8 codes; e8 [n/128] uint8.  Errors as moe_fp8_quantize. */
int moe_fp8_quantize_pow2(const void* w, int dtype, int64_t n, uint8_t* q, uint8_t* e8,
                          void* stream);

/* moe_fp8_quantize_pow2 by rows, with the scales in rows of their own pitch
 * (the layout the FP8 matrix-core GEMMs read):
 *   w [rows][cols] (MOE_BF16 or MOE_F32), cols a multiple of 128; q
 *   [rows][cols] codes; e8 [rows][e8_ld] E8M0 bytes, block j of row r at
 *   e8[r * e8_ld + j], the bytes past cols/128 set to zero; e8_ld from
 *   cols/128 to cols/128 + 15.  nrows (device int32, or NULL): rows at or
 *   past *nrows are left alone (e.g. offsets + NL: the routed rows of a
 *   [R_cap] buffer).  Errors: MOE_ERR_INVALID_ARG for a NULL pointer, w or q
 *   not 16-byte aligned, nrows not 4-byte aligned, or sizes outside these
 *   rules; MOE_ERR_UNSUPPORTED for another dtype. */
int moe_fp8_quantize_pow2_rows(const void* w, int dtype, int64_t rows, int64_t cols, const int32_t* nrows,
                               uint8_t* q, uint8_t* e8, int64_t e8_ld, void* stream);

/* A5 and A6 on FP8 weights (the page's further step: the expert GEMMs take
 * the FP8 weights directly).  The weight tiles move as E4M3 codes - half the
 * bytes of bf16 - and are decoded to bf16 in the kernel where the MFMA
 * operands are read (decode * scale in float32, rounded to nearest even),
 * so the results are bitwise those of moe_expert_gate_up / moe_expert_down
 * on the weights moe_fp8_dequantize returns.
 *   W1q, W3q [NL][f][d] and W2q [NL][d][f] E4M3 codes with scales W1s, W3s
 *   [NL][f][d/128] and W2s [NL][d][f/128] as moe_fp8_quantize writes them;
 *   activations as in the bf16 calls; row_token NULL: `a` is x_perm, else `a`
 *   is x read through row_token (as moe_expert_gate_up_gather).
 *   MOE_ERR_UNSUPPORTED unless dtype is MOE_BF16 and d and f are multiples
 *   of 128 (and, with row_token, T*d*2 < 2^31). */
int moe_expert_gate_up_fp8(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                           const void* a, const uint8_t* W1q, const float* W1s, const uint8_t* W3q,
                           const float* W3s, void* gu, void* h, void* stream);
int moe_expert_down_fp8(const moe_desc* desc, const int32_t* offsets, const void* h, const uint8_t* W2q,
                        const float* W2s, void* y_perm, void* stream);

/* A5 on the FP8 matrix cores (Domyn page, section "FP8 expert weight
 * all-gather": the expert GEMMs in FP8 as the further step): the activations
 * and the weights are both E4M3 codes with power-of-two block scales, as
 * moe_fp8_quantize_pow2 writes them, and each 32 x 32 x 64 product applies
 * the row's and the column's scale itself, accumulating in float32:
 *   G[r] = sum over k of (xq * 2^xe)[row_token[r]][k] (W1q * 2^we)[n][k], U
 *   likewise with W3, h = silu(G) * U, as moe_expert_gate_up_gather.
 *   xq [T][d] codes, xs [T][d/128] E8M0 bytes (x quantised in blocks of 128
 *   along a row); W1q, W3q [NL][f][d] codes, W1s, W3s [NL][f][d/128] bytes;
 *   gu [R_cap][2f] (or NULL) and h [R_cap][f] bf16.  MOE_ERR_UNSUPPORTED
 *   unless dtype is bf16, d is a multiple of 512 and T * d < 2^31. */
int moe_expert_gate_up_fp8mm(const moe_desc* desc, const int32_t* offsets, const int32_t* row_token,
                             const uint8_t* xq, const uint8_t* xs, const uint8_t* W1q,
                             const uint8_t* W1s, const uint8_t* W3q, const uint8_t* W3s, void* gu,
                             void* h, void* stream);

/* A6 on the FP8 matrix cores (same passage): y_perm = h W2^T with h and W2
 * both E4M3 codes with power-of-two block scales along f, each 32 x 32 x 64
 * product applying the row's and the column's scale, float32 sums:
 *   y_perm[r][n] = sum over k of (hq * 2^hs)[r][k] (W2q * 2^ws)[g][n][k] for
 *   row r of expert g's segment (offsets, as moe_expert_down).
 *   hq [R_cap][f] codes and hs [R_cap][S] E8M0 bytes; W2q [NL][d][f] codes
 *   and W2s [NL][d][S] bytes, with S = f/128 rounded up to a multiple of 4
 *   (moe_fp8_quantize_pow2_rows with e8_ld = S writes both); y_perm
 *   [R_cap][d] bf16.  MOE_ERR_UNSUPPORTED unless dtype is bf16, f is a
 *   multiple of 128 and R_cap * f < 2^31. */
int moe_expert_down_fp8mm(const moe_desc* desc, const int32_t* offsets, const uint8_t* hq, const uint8_t* hs,
                          const uint8_t* W2q, const uint8_t* W2s, void* y_perm, void* stream);

/* Measurement aid (Domyn page, section "Dynamic tile scheduling in
 * SonicMoE": the two tile orders are compared with and without a dummy
 * kernel that occupies part of the GPU).  Launches `workgroups` one-wave
 * workgroups on `stream`, each reserving lds_bytes of LDS - so that a
 * grouped-GEMM workgroup cannot share its compute unit - and returning after
 * `microseconds` of the device's real-time clock.  No memory is touched.
 * MOE_ERR_INVALID_ARG unless 1 <= workgroups <= 4096,
 * 4 <= lds_bytes <= 163840 and 0 <= microseconds <= 1000000. */
int moe_hold_cus(int workgroups, int lds_bytes, int microseconds, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
