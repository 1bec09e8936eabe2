// Launchers of the grouped GEMMs: the SwiGLU expert MLP (Aurora page,
// section 3.1, Algorithm 1 stage 4: Grouped_mm of gate and up, Silu(gate) * up,
// Grouped_mm of down over the cum_token_counts segments), its backward, and
// the router's linear layer and its backward.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm.h"
#include "gemm_dma.h"
#include "internal.h"

namespace moe {

int num_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace {

GemmParams blank(const moe_desc& d) {
  GemmParams p{};
  p.dyn = d.tile_schedule == MOE_SCHEDULE_DYNAMIC ? d.tile_counters : nullptr;
  return p;
}

// Tile edge of the bf16 kernels: 256 x 256 (one workgroup per CU).
constexpr int MT = 256;

template <int ALAY, int BLAY, typename AT, int GRP, int EPI, bool DUAL>
hipError_t run_mfma(const GemmParams& p, int64_t ub_tiles, hipStream_t s) {
  int64_t grid = std::min<int64_t>(ub_tiles, (int64_t)num_cus());
  if (grid >= 8) grid -= grid % 8;  // whole XCD groups for the tile remap
  if (grid <= 0) return hipSuccess;
  gemm_mfma_kernel<MT, MT, ALAY, BLAY, AT, GRP, EPI, DUAL><<<(unsigned)grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

// k-slice width and ring depth of the LDS-DMA kernel (a 128 KB ring).
#ifndef MOE_DMA_BK
#define MOE_DMA_BK 64
#endif
constexpr int DMA_BK = MOE_DMA_BK;
constexpr int DMA_STAGES = DMA_BK == 64 ? 2 : 4;

// bf16 products: the LDS-DMA kernel when every K-contiguous operand has K a
// multiple of its 32-wide k-tile, else the register-staged kernel.
// KB16: a grouped-K product that may write bf16 (the weight gradients); the
// other grouped-K products (the router's split-K partials) write fp32 only,
// and no bf16-output kernel is built for them.
template <int ALAY, int BLAY, typename AT, int GRP, int EPI, bool DUAL, int GATH = GATH_NONE, bool BQ8 = false,
          bool F8 = false, bool KB16 = false>
hipError_t run_bf16(const GemmParams& p, int64_t ub_tiles, hipStream_t s) {
  // K-contiguous operands need whole 64-wide k-tiles: every K (GRP_M, plain)
  // or every K chunk (GRP_K split into kchunk pieces) a multiple of 64.
  const bool k_ok = (ALAY == LAY_MN && BLAY == LAY_MN) ||
                    (GRP != GRP_K && p.K % DMA_BK == 0) ||
                    (GRP == GRP_K && !p.offsets && p.kchunk % DMA_BK == 0 && p.K % DMA_BK == 0);
  if (!std::is_same<AT, uint16_t>::value || !k_ok) return run_mfma<ALAY, BLAY, AT, GRP, EPI, DUAL>(p, ub_tiles, s);
  int64_t grid = std::min<int64_t>(ub_tiles, (int64_t)num_cus());
  if (grid >= 8) grid -= grid % 8;
  if (grid <= 0) return hipSuccess;
  if constexpr (std::is_same<AT, uint16_t>::value) {
    constexpr bool F32_ONLY = GRP == GRP_K && !KB16;
    if (F32_ONLY && !p.c_f32) return hipErrorInvalidValue;
    const bool cf = (EPI == EPI_STORE || EPI == EPI_ADD) && p.c_f32;
    if (p.dyn) {
      if (cf) gemm_dma_kernel<DMA_BK, DMA_STAGES, ALAY, BLAY, GRP, EPI, DUAL, true, true, GATH, BQ8, F8><<<(unsigned)grid, 256, 0, s>>>(p);
      else if constexpr (!F32_ONLY)
        gemm_dma_kernel<DMA_BK, DMA_STAGES, ALAY, BLAY, GRP, EPI, DUAL, false, true, GATH, BQ8, F8><<<(unsigned)grid, 256, 0, s>>>(p);
    } else {
      if (cf) gemm_dma_kernel<DMA_BK, DMA_STAGES, ALAY, BLAY, GRP, EPI, DUAL, true, false, GATH, BQ8, F8><<<(unsigned)grid, 256, 0, s>>>(p);
      else if constexpr (!F32_ONLY)
        gemm_dma_kernel<DMA_BK, DMA_STAGES, ALAY, BLAY, GRP, EPI, DUAL, false, false, GATH, BQ8, F8><<<(unsigned)grid, 256, 0, s>>>(p);
    }
  }
  return hipGetLastError();
}

template <int ALAY, int BLAY, int GRP, int EPI, bool DUAL>
hipError_t run_f32(const GemmParams& p, int64_t ub_tiles, hipStream_t s) {
  const int64_t grid = std::min<int64_t>(ub_tiles, (int64_t)num_cus() * 4);
  if (grid <= 0) return hipSuccess;
  gemm_f32_kernel<ALAY, BLAY, GRP, EPI, DUAL><<<(unsigned)grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Band of the grouped-K tile order for a product of mtiles m-tiles: the
// divisor of mtiles nearest to the square root of an XCD's run of 32 tiles
// (6, then 5, 7, 4, 8), else 6; 0 (no bands) when M has 8 m-tiles or fewer.
int k_band(int64_t mtiles) {
  if (mtiles <= 8) return 0;
  for (int b : {6, 5, 7, 4, 8})
    if (mtiles % b == 0) return b;
  return 6;
}

int64_t r_cap(const moe_desc& d) { return (int64_t)d.T * std::min(d.k, d.num_local); }

// Upper bound on the m-tiles of a variable-M grouped product.
int64_t mtiles_ub(const moe_desc& d, int bm) { return cdiv(r_cap(d), bm) + d.num_local; }

// Split-K factor of the router-weight gradient (K = T is long, M x N small):
// the S that minimises a simple time model on a 256-CU part, rounds of
// output tiles times k-tiles per tile (~1.6 us per 64-wide k-tile of a
// 256 x 256 tile), plus writing and reading the S float32 partials at
// ~5 TB/s.  It depends on the shape only, so the summation order (and the
// result) is the same on every device and the workspace query needs no
// device.  Ties go to the smaller S.
int router_splits(const moe_desc& d) {
  const int64_t tiles = cdiv(d.E, MT) * cdiv(d.d, MT);
  int best = 1;
  int64_t best_cost = -1;
  for (int S = 1; S <= 64; ++S) {
    if (S > 1 && cdiv(d.T, S) < 64) break;  // chunks of at least one k-tile
    // cost in units of 1e-13 s: k-tile time 1.6 us = 16e6 units; a byte at 5 TB/s = 2 units
    const int64_t cost = cdiv((int64_t)S * tiles, 256) * cdiv(cdiv(d.T, S), 64) * 16000000 +
                         (int64_t)S * d.E * d.d * 8 * 2;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

// float32 -> bfloat16 (round to nearest even), 8 elements per thread; n % 8 == 0.
__global__ void __launch_bounds__(256) to_bf16_kernel(const float* __restrict__ in, int64_t n,
                                                      uint16_t* __restrict__ out) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (int64_t)gridDim.x * 256 * 8) {
    float v[8];
    const f32x4 a = *reinterpret_cast<const f32x4*>(in + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(in + i + 4);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    Vec16<uint16_t>::store(out + i, v);
  }
}

// out[i] = sum of the S partials in split order (+ bias[i % ncol] when given).
__global__ void __launch_bounds__(256) sum_splits_kernel(const float* __restrict__ part, int S, int64_t n,
                                                         float* __restrict__ out,
                                                         const float* __restrict__ bias = nullptr,
                                                         int ncol = 1) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc += part[(int64_t)s * n + i];
    if (bias) acc += bias[i % ncol];
    out[i] = acc;
  }
}

}  // namespace

// Router backward workspace: split-K partials of dWr, then (bf16 path) a
// bfloat16 copy of dlogits for the matrix cores.
size_t router_bwd_partials_bytes(const moe_desc& d) {
  return (((size_t)router_splits(d) * (size_t)d.E * (size_t)d.d * sizeof(float)) + 255) & ~(size_t)255;
}

size_t router_bwd_workspace(const moe_desc& d) {
  size_t b = router_bwd_partials_bytes(d);
  if (d.dtype == MOE_BF16) b += (size_t)d.T * (size_t)d.E * sizeof(uint16_t);
  return b;
}

// Router logits (bf16): with fewer output tiles than a 256-CU part has CUs
// (few tokens, or E small), the product is split over d into S chunks of
// whole 64-wide k-tiles, written as float32 partials [S][T][E] into the
// workspace and summed in chunk order (deterministic).  S depends on the
// shape only.
int router_logit_splits(const moe_desc& d) {
  if (d.dtype != MOE_BF16 || d.d % 64) return 1;
  const int64_t tiles = cdiv(d.T, MT) * cdiv(d.E, MT);
  const int64_t s = std::min<int64_t>(std::min<int64_t>(cdiv(256, tiles), d.d / 64), 16);
  if (s <= 1) return 1;
  const int64_t chunk = cdiv(d.d / 64, s) * 64;
  return (int)cdiv(d.d, chunk);
}

size_t router_logits_workspace(const moe_desc& d) {
  const int S = router_logit_splits(d);
  return S > 1 ? (size_t)S * (size_t)d.T * (size_t)d.E * sizeof(float) : 0;
}

hipError_t launch_router_logits(const moe_desc& d, const void* x, const void* Wr, const float* bias,
                                float* logits, void* ws, hipStream_t s) {
  const int S = router_logit_splits(d);
  if (S > 1) {
    float* part = reinterpret_cast<float*>(ws);
    GemmParams q = blank(d);
    q.A = x;
    q.lda = d.d;
    q.B = Wr;
    q.ldb = d.d;
    q.C = part;
    q.ldc = d.E;
    q.c_gstride = (int64_t)d.T * d.E;
    q.offsets = nullptr;
    q.ngroups = S;
    q.kchunk = (int)(cdiv(d.d / 64, S) * 64);
    q.M = d.T;
    q.N = d.E;
    q.K = d.d;
    q.c_f32 = 1;
    hipError_t e = run_bf16<LAY_K, LAY_K, uint16_t, GRP_K, EPI_STORE, false>(q, (int64_t)S * cdiv(d.T, MT) * cdiv(d.E, MT), s);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)d.T * d.E;
    const int64_t blocks = std::min<int64_t>(cdiv(n, 256), (int64_t)num_cus() * 8);
    sum_splits_kernel<<<(unsigned)blocks, 256, 0, s>>>(part, S, n, logits, bias, d.E);
    return hipGetLastError();
  }
  GemmParams p = blank(d);
  p.A = x;
  p.lda = d.d;
  p.B = Wr;
  p.ldb = d.d;
  p.C = logits;
  p.ldc = d.E;
  p.M = d.T;
  p.N = d.E;
  p.K = d.d;
  p.bias = bias;
  p.c_f32 = 1;
  if (d.dtype == MOE_BF16)
    return run_bf16<LAY_K, LAY_K, uint16_t, GRP_NONE, EPI_STORE, false>(p, cdiv(d.T, MT) * cdiv(d.E, MT), s);
  return run_f32<LAY_K, LAY_K, GRP_NONE, EPI_STORE, false>(p, cdiv(d.T, 64) * cdiv(d.E, 64), s);
}

// row_token != NULL: x_perm is x itself and row r of the product reads
// x[row_token[r]] (the gather fused into the A operand; bf16 only).
hipError_t launch_gate_up(const moe_desc& d, const int32_t* offsets, const void* x_perm, const void* W1,
                          const void* W3, void* gu, void* h, hipStream_t s, const int32_t* row_token) {
  const bool bf = d.dtype == MOE_BF16;
  GemmParams p = blank(d);
  p.A = x_perm;
  p.gather = row_token;
  p.gather_rows = d.T;
  p.lda = d.d;
  p.B = W1;
  p.B2 = W3;
  p.ldb = d.d;
  p.b_gstride = (int64_t)d.f * d.d;
  p.C = h;
  p.ldc = d.f;
  p.gu_out = gu;
  p.offsets = offsets;
  p.ngroups = d.num_local;
  p.N = d.f;
  p.K = d.d;
  p.c_f32 = bf ? 0 : 1;
  if (bf && row_token)
    return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_SWIGLU, true, GATH_A>(p, mtiles_ub(d, MT) * cdiv(d.f, MT / 2), s);
  if (row_token) return hipErrorNotSupported;
  if (bf) return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_SWIGLU, true>(p, mtiles_ub(d, MT) * cdiv(d.f, MT / 2), s);
  return run_f32<LAY_K, LAY_K, GRP_M, EPI_SWIGLU, true>(p, mtiles_ub(d, 64) * cdiv(d.f, 64), s);
}

// FP8 expert weights in the GEMMs (bf16 only): W1q/W3q [NL][f][d] and W2q
// [NL][d][f] E4M3 codes, s1/s3 [NL][f][d/128] and s2 [NL][d][f/128] block
// scales.  row_token != NULL: a is x, read through it (as launch_gate_up).
hipError_t launch_gate_up_q8(const moe_desc& d, const int32_t* offsets, const void* a, const int32_t* row_token,
                             const uint8_t* W1q, const float* s1, const uint8_t* W3q, const float* s3, void* gu,
                             void* h, hipStream_t s) {
  GemmParams p = blank(d);
  p.A = a;
  p.lda = d.d;
  p.gather = row_token;
  p.gather_rows = d.T;
  p.B = W1q;
  p.B2 = W3q;
  p.ldb = d.d;
  p.bs = s1;
  p.bs2 = s3;
  p.b_gstride = (int64_t)d.f * d.d;
  p.C = h;
  p.ldc = d.f;
  p.gu_out = gu;
  p.offsets = offsets;
  p.ngroups = d.num_local;
  p.N = d.f;
  p.K = d.d;
  const int64_t ub = mtiles_ub(d, MT) * cdiv(d.f, MT / 2);
  if (row_token) return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_SWIGLU, true, GATH_A, true>(p, ub, s);
  return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_SWIGLU, true, GATH_NONE, true>(p, ub, s);
}

// gate/up on the FP8 matrix cores: x and W1/W3 as E4M3 codes with power-of-two
// block scales (E8M0 bytes, one per 128 codes of a row), x read through
// row_token; the block-scaled MFMA applies both scales.  Codes count in
// pairs in the GEMM's units (a k-tile of 64 pairs is one scale block).
hipError_t launch_gate_up_f8(const moe_desc& d, const int32_t* offsets, const int32_t* row_token, const uint8_t* xq,
                             const uint8_t* xs, const uint8_t* W1q, const uint8_t* W1s, const uint8_t* W3q,
                             const uint8_t* W3s, void* gu, void* h, hipStream_t s) {
  GemmParams p = blank(d);
  p.A = xq;
  p.lda = d.d / 2;
  p.gather = row_token;
  p.gather_rows = d.T;
  p.B = W1q;
  p.B2 = W3q;
  p.ldb = d.d / 2;
  p.b_gstride = (int64_t)d.f * d.d / 2;
  p.a_scale = xs;
  p.b_scale = W1s;
  p.b2_scale = W3s;
  p.sbytes = d.d / 128;
  p.C = h;
  p.ldc = d.f;
  p.gu_out = gu;
  p.offsets = offsets;
  p.ngroups = d.num_local;
  p.N = d.f;
  p.K = d.d / 2;
  return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_SWIGLU, true, GATH_A, false, true>(
      p, mtiles_ub(d, MT) * cdiv(d.f, MT / 2), s);
}

// y_perm = h W2^T on the FP8 matrix cores: h [R_cap][f] and W2 [NL][d][f]
// as E4M3 codes, their power-of-two block scales in rows of sb bytes (f/128
// rounded up to a multiple of 4).
hipError_t launch_down_f8(const moe_desc& d, const int32_t* offsets, const uint8_t* hq, const uint8_t* hs,
                          const uint8_t* W2q, const uint8_t* W2s, void* y_perm, hipStream_t s) {
  GemmParams p = blank(d);
  p.A = hq;
  p.lda = d.f / 2;
  p.gather_rows = (int)r_cap(d);  // (the rows of A's scale array)
  p.B = W2q;
  p.ldb = d.f / 2;
  p.b_gstride = (int64_t)d.d * d.f / 2;
  p.a_scale = hs;
  p.b_scale = W2s;
  p.sbytes = fp8_scale_row_bytes(d.f);
  p.C = y_perm;
  p.ldc = d.d;
  p.offsets = offsets;
  p.ngroups = d.num_local;
  p.N = d.d;
  p.K = d.f / 2;
  return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_STORE, false, GATH_NONE, false, true>(
      p, mtiles_ub(d, MT) * cdiv(d.d, MT), s);
}

hipError_t launch_down_q8(const moe_desc& d, const int32_t* offsets, const void* h, const uint8_t* W2q,
                          const float* s2, void* y_perm, hipStream_t s) {
  GemmParams q = blank(d);
  q.A = h;
  q.lda = d.f;
  q.B = W2q;
  q.ldb = d.f;
  q.bs = s2;
  q.b_gstride = (int64_t)d.d * d.f;
  q.C = y_perm;
  q.ldc = d.d;
  q.offsets = offsets;
  q.ngroups = d.num_local;
  q.N = d.d;
  q.K = d.f;
  return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_STORE, false, GATH_NONE, true>(q, mtiles_ub(d, MT) * cdiv(d.d, MT), s);
}

hipError_t launch_down(const moe_desc& d, const int32_t* offsets, const void* h, const void* W2, void* y_perm,
                       hipStream_t s) {
  const bool bf = d.dtype == MOE_BF16;
  GemmParams q = blank(d);
  q.A = h;
  q.lda = d.f;
  q.B = W2;
  q.ldb = d.f;
  q.b_gstride = (int64_t)d.d * d.f;
  q.C = y_perm;
  q.ldc = d.d;
  q.offsets = offsets;
  q.ngroups = d.num_local;
  q.N = d.d;
  q.K = d.f;
  q.c_f32 = bf ? 0 : 1;
  if (bf) return run_bf16<LAY_K, LAY_K, uint16_t, GRP_M, EPI_STORE, false>(q, mtiles_ub(d, MT) * cdiv(d.d, MT), s);
  return run_f32<LAY_K, LAY_K, GRP_M, EPI_STORE, false>(q, mtiles_ub(d, 64) * cdiv(d.d, 64), s);
}

hipError_t launch_bwd_dh(const moe_desc& d, const int32_t* offsets, const void* W2, const void* gu,
                         const void* dy_perm, void* dgu, hipStream_t s) {
  const bool bf = d.dtype == MOE_BF16;
  // dH = dY W2 (W2 stored [d][f]: N-contiguous in k = d), SwiGLU backward epilogue -> dgu
  GemmParams p = blank(d);
  p.A = dy_perm;
  p.lda = d.d;
  p.B = W2;
  p.ldb = d.f;
  p.b_gstride = (int64_t)d.d * d.f;
  p.C = dgu;
  p.ldc = 2 * (int64_t)d.f;
  p.gu_in = gu;
  p.offsets = offsets;
  p.ngroups = d.num_local;
  p.N = d.f;
  p.K = d.d;
  p.c_f32 = bf ? 0 : 1;
  if (bf) return run_bf16<LAY_K, LAY_MN, uint16_t, GRP_M, EPI_SWIGLU_BWD, false>(p, mtiles_ub(d, MT) * cdiv(d.f, MT), s);
  return run_f32<LAY_K, LAY_MN, GRP_M, EPI_SWIGLU_BWD, false>(p, mtiles_ub(d, 64) * cdiv(d.f, 64), s);
}

// dH with dy read in place (bf16): row r of the product is dy[row_token[r]],
// scaled in the epilogue by row_w[r] (the routing weight the permuted copy
// would carry), then the SwiGLU backward -> dgu; hw[r] = row_w[r] silu(G) U
// (bf16) for the dW2 product.
hipError_t launch_bwd_dh_gather(const moe_desc& d, const int32_t* offsets, const int32_t* row_token,
                                const float* row_w, const void* dy, const void* W2, const void* gu, void* dgu,
                                void* hw, float* dtopk_part, hipStream_t s) {
  GemmParams p = blank(d);
  p.dw_part = dtopk_part;
  p.A = dy;
  p.lda = d.d;
  p.gather = row_token;
  p.gather_rows = d.T;
  p.row_scale = row_w;
  p.h_out = hw;
  p.B = W2;
  p.ldb = d.f;
  p.b_gstride = (int64_t)d.d * d.f;
  p.C = dgu;
  p.ldc = 2 * (int64_t)d.f;
  p.gu_in = gu;
  p.offsets = offsets;
  p.ngroups = d.num_local;
  p.N = d.f;
  p.K = d.d;
  p.c_f32 = 0;
  return run_bf16<LAY_K, LAY_MN, uint16_t, GRP_M, EPI_SWIGLU_BWD, false, GATH_A>(p, mtiles_ub(d, MT) * cdiv(d.f, MT), s);
}

// dW2 [d][f] = dy_perm^T hw with dy read in place: k-row r of the A operand
// is dy[row_token[r]] (bf16); hw carries the routing weight.
hipError_t launch_dw_down_gather(const moe_desc& d, const int32_t* offsets, const int32_t* row_token,
                                 const void* dy, const void* hw, void* dW2, hipStream_t s) {
  GemmParams q = blank(d);
  q.A = dy;
  q.lda = d.d;
  q.gather = row_token;
  q.gather_rows = d.T;
  q.B = hw;
  q.ldb = d.f;
  q.C = dW2;
  q.ldc = d.f;
  q.c_gstride = (int64_t)d.d * d.f;
  q.offsets = offsets;
  q.ngroups = d.num_local;
  q.M = d.d;
  q.N = d.f;
  q.c_f32 = d.wgrad_dtype == MOE_F32;
  q.band = k_band(cdiv(d.d, MT));
  return run_bf16<LAY_MN, LAY_MN, uint16_t, GRP_K, EPI_STORE, false, GATH_AK, false, false, true>(
      q, (int64_t)d.num_local * cdiv(d.d, MT) * cdiv(d.f, MT), s);
}

hipError_t launch_bwd_dxp(const moe_desc& d, const int32_t* offsets, const void* W1, const void* W3,
                          const void* dgu, void* dx_perm, hipStream_t s) {
  const bool bf = d.dtype == MOE_BF16;
  // dX = [dG | dU] [W1 ; W3]  (K = 2f; rows k < f of W1, k >= f of W3, both [f][d])
  GemmParams q = blank(d);
  q.A = dgu;
  q.lda = 2 * (int64_t)d.f;
  q.B = W1;
  q.B2 = W3;
  q.ksplit = d.f;
  q.ldb = d.d;
  q.b_gstride = (int64_t)d.f * d.d;
  q.C = dx_perm;
  q.ldc = d.d;
  q.offsets = offsets;
  q.ngroups = d.num_local;
  q.N = d.d;
  q.K = 2 * d.f;
  q.c_f32 = bf ? 0 : 1;
  if (bf) return run_bf16<LAY_K, LAY_MN, uint16_t, GRP_M, EPI_STORE, false>(q, mtiles_ub(d, MT) * cdiv(d.d, MT), s);
  return run_f32<LAY_K, LAY_MN, GRP_M, EPI_STORE, false>(q, mtiles_ub(d, 64) * cdiv(d.d, 64), s);
}

// dW1 | dW3 [f][d] = [dG | dU]^T x_perm over each expert's rows (one grouped-K
// product with M = 2f split at f).  row_token != NULL: x_perm is x itself and
// k-row r reads x[row_token[r]] (the gather fused into the B operand; bf16 only).
hipError_t launch_dw_gate_up(const moe_desc& d, const int32_t* offsets, const void* x_perm, const void* dgu,
                             void* dW1, void* dW3, hipStream_t s, const int32_t* row_token) {
  const bool bf = d.dtype == MOE_BF16;
  GemmParams p = blank(d);
  p.A = dgu;
  p.lda = 2 * (int64_t)d.f;
  p.B = x_perm;
  p.ldb = d.d;
  p.gather = row_token;
  p.gather_rows = d.T;
  p.C = dW1;
  p.C2 = dW3;
  p.msplit = d.f;
  p.ldc = d.d;
  p.c_gstride = (int64_t)d.f * d.d;
  p.offsets = offsets;
  p.ngroups = d.num_local;
  p.M = 2 * d.f;
  p.N = d.d;
  p.c_f32 = d.wgrad_dtype == MOE_F32;
  const int64_t tiles = (int64_t)d.num_local * cdiv(2 * d.f, MT) * cdiv(d.d, MT);
  if (bf) p.band = k_band(cdiv(2 * d.f, MT));
  if (bf && row_token)
    return run_bf16<LAY_MN, LAY_MN, uint16_t, GRP_K, EPI_STORE, false, GATH_B, false, false, true>(p, tiles, s);
  if (row_token) return hipErrorNotSupported;
  if (bf) return run_bf16<LAY_MN, LAY_MN, uint16_t, GRP_K, EPI_STORE, false, GATH_NONE, false, false, true>(p, tiles, s);
  return run_f32<LAY_MN, LAY_MN, GRP_K, EPI_STORE, false>(p, (int64_t)d.num_local * cdiv(2 * d.f, 64) * cdiv(d.d, 64), s);
}

// dW2 [d][f] = dy_perm^T h over each expert's rows.
hipError_t launch_dw_down(const moe_desc& d, const int32_t* offsets, const void* dy_perm, const void* h, void* dW2,
                          hipStream_t s) {
  const bool bf = d.dtype == MOE_BF16;
  GemmParams q = blank(d);
  q.A = dy_perm;
  q.lda = d.d;
  q.B = h;
  q.ldb = d.f;
  q.C = dW2;
  q.ldc = d.f;
  q.c_gstride = (int64_t)d.d * d.f;
  q.offsets = offsets;
  q.ngroups = d.num_local;
  q.M = d.d;
  q.N = d.f;
  q.c_f32 = d.wgrad_dtype == MOE_F32;
  if (bf) q.band = k_band(cdiv(d.d, MT));
  if (bf)
    return run_bf16<LAY_MN, LAY_MN, uint16_t, GRP_K, EPI_STORE, false, GATH_NONE, false, false, true>(
        q, (int64_t)d.num_local * cdiv(d.d, MT) * cdiv(d.f, MT), s);
  return run_f32<LAY_MN, LAY_MN, GRP_K, EPI_STORE, false>(q, (int64_t)d.num_local * cdiv(d.d, 64) * cdiv(d.f, 64), s);
}

hipError_t launch_ffn_bwd_dw(const moe_desc& d, const int32_t* offsets, const void* x_perm, const void* h,
                             const void* dgu, const void* dy_perm, void* dW1, void* dW3, void* dW2,
                             hipStream_t s, const int32_t* row_token) {
  hipError_t e = launch_dw_gate_up(d, offsets, x_perm, dgu, dW1, dW3, s, row_token);
  if (e != hipSuccess) return e;
  return launch_dw_down(d, offsets, dy_perm, h, dW2, s);
}

hipError_t launch_router_bwd(const moe_desc& d, const void* x, const void* Wr, const float* dlogits,
                             float* dx_router, void* dx_acc, float* dWr, void* ws, hipStream_t s) {
  const bool bf = d.dtype == MOE_BF16;
  hipError_t e = hipSuccess;
  float* part = reinterpret_cast<float*>(ws);
  // bf16 path: dlogits rounded once to bf16 (the matrix-core operand).
  const void* dl = dlogits;
  if (bf) {
    uint16_t* dl16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + router_bwd_partials_bytes(d));
    const int64_t n = (int64_t)d.T * d.E;
    const int64_t blocks = std::min<int64_t>(cdiv(n, 256 * 8), (int64_t)num_cus() * 8);
    to_bf16_kernel<<<(unsigned)blocks, 256, 0, s>>>(dlogits, n, dl16);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dl = dl16;
  }
  if (dx_router || dx_acc) {
    // dx_router [T][d] = dlogits [T][E] Wr [E][d] (float), or dx += dlogits Wr
    // in the layer's dtype
    GemmParams p = blank(d);
    p.A = dl;
    p.lda = d.E;
    p.B = Wr;
    p.ldb = d.d;
    p.C = dx_router ? static_cast<void*>(dx_router) : dx_acc;
    p.ldc = d.d;
    p.M = d.T;
    p.N = d.d;
    p.K = d.E;
    p.c_f32 = dx_router ? 1 : !bf;
    const int64_t tb = cdiv(d.T, MT) * cdiv(d.d, MT), tf = cdiv(d.T, 64) * cdiv(d.d, 64);
    if (dx_router) {
      if (bf) e = run_bf16<LAY_K, LAY_MN, uint16_t, GRP_NONE, EPI_STORE, false>(p, tb, s);
      else e = run_f32<LAY_K, LAY_MN, GRP_NONE, EPI_STORE, false>(p, tf, s);
    } else {
      if (bf) e = run_bf16<LAY_K, LAY_MN, uint16_t, GRP_NONE, EPI_ADD, false>(p, tb, s);
      else e = run_f32<LAY_K, LAY_MN, GRP_NONE, EPI_ADD, false>(p, tf, s);
    }
    if (e != hipSuccess) return e;
  }
  if (dWr) {
    // dWr [E][d] = dlogits^T x, split over T into S chunks, then summed in chunk order
    const int S = router_splits(d);
    GemmParams q = blank(d);
    q.A = dl;
    q.lda = d.E;
    q.B = x;
    q.ldb = d.d;
    q.C = part;
    q.ldc = d.d;
    q.c_gstride = (int64_t)d.E * d.d;
    q.offsets = nullptr;
    q.ngroups = S;
    q.kchunk = (int)cdiv(d.T, S);
    q.M = d.E;
    q.N = d.d;
    q.K = d.T;
    q.c_f32 = 1;
    if (bf) e = run_bf16<LAY_MN, LAY_MN, uint16_t, GRP_K, EPI_STORE, false>(q, (int64_t)S * cdiv(d.E, MT) * cdiv(d.d, MT), s);
    else e = run_f32<LAY_MN, LAY_MN, GRP_K, EPI_STORE, false>(q, (int64_t)S * cdiv(d.E, 64) * cdiv(d.d, 64), s);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)d.E * d.d;
    const int64_t blocks = std::min<int64_t>(cdiv(n, 256), (int64_t)num_cus() * 8);
    sum_splits_kernel<<<(unsigned)blocks, 256, 0, s>>>(part, S, n, dWr);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace moe
