// Token counting, prefix sums, index generation, gather, weighted combine and
// their backward (Aurora page, section 3.1, Algorithm 1 stages 2, 3, the
// stage-4 gather and stage 5).
//
// Counting and placement.  The page gives each GPU thread a block of 8 tokens,
// counts per (local expert, thread) into an expert-major array, prefix-sums it
// and places every selection at base + per-(expert, thread) counter, which
// makes every expert's rows ascend in token order.  Here a 256-thread
// workgroup owns a block of 256 tokens (one per lane): each wave builds, in
// LDS, a 64-bit mask per expert of the lanes that selected it (ds_or_b64, an
// order-free operation), the block count of an expert is the popcount of its
// four wave masks, and a selection's rank inside the block is the popcount of
// the masks of earlier waves plus the bits of lower lanes in its own wave.
// The result is the same stable, deterministic placement, without a global
// sort and without float or order-dependent atomics.
//
// Data movement (gather, combine and the backward scatter/sum) is token
// major: one wavefront per token reads the token's row once and writes or
// reads its routed rows with 16-byte vector accesses.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace moe {

constexpr int BLK_TOK = 256;

// counts per (expert, token block), expert-major: blk_counts[e * nblk + b].
__global__ void __launch_bounds__(256) count_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                    int32_t* __restrict__ blk_counts, int nblk) {
  extern __shared__ uint64_t masks[];  // [4][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * E; i += 256) masks[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * BLK_TOK + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(int64_t)t * k + j];
      if ((unsigned)e < (unsigned)E) atomicOr((unsigned long long*)&masks[wave * E + e], 1ull << lane);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    const int c = __popcll(masks[e]) + __popcll(masks[E + e]) + __popcll(masks[2 * E + e]) +
                  __popcll(masks[3 * E + e]);
    blk_counts[(int64_t)e * nblk + blockIdx.x] = c;
  }
}

// The page's partial_cum_token_counts (an exclusive prefix sum of the block
// counts in expert-major order) in two parallel steps.  expert_scan_kernel,
// one workgroup per expert: counts[e] = the expert's total over all blocks,
// and, for a local expert n, base_rel[n][b] = the exclusive prefix sum of its
// block counts.  offsets_kernel: offsets[n] = exclusive prefix sum of the
// local experts' counts, offsets[NL] = R.  A block's base is then
// offsets[n] + base_rel[n][b], which is the expert-major prefix sum.
__global__ void __launch_bounds__(256) expert_scan_kernel(const int32_t* __restrict__ blk_counts, int nblk, int e0,
                                                          int NL, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ base_rel) {
  __shared__ int wsum[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* src = blk_counts + (int64_t)e * nblk;
  const bool local = e >= e0 && e < e0 + NL;
  int32_t* dst = local ? base_rel + (int64_t)(e - e0) * nblk : base_rel;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + tid;
    const int v = b < nblk ? src[b] : 0;
    int inc = v;  // inclusive scan inside the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();  // wsum is rewritten by the next chunk
    if (local && b < nblk) dst[b] = before + inc - v;
    carry += total;
  }
  if (tid == 0) counts[e] = carry;
}

// One workgroup of 1024 threads (NL <= 1024).
__global__ void __launch_bounds__(1024) offsets_kernel(const int32_t* __restrict__ counts, int e0, int NL,
                                                       int32_t* __restrict__ offsets) {
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  const int v = tid < NL ? counts[e0 + tid] : 0;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int u = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += u;
    __syncthreads();
  }
  if (tid < NL) offsets[tid] = sh[tid] - v;
  if (tid == 0) offsets[NL] = sh[1023];
}

// row_token and slot_row from the block bases (the page's index generation).
__global__ void __launch_bounds__(256) place_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                    int e0, int NL, const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ base_rel, int nblk,
                                                    int32_t* __restrict__ row_token,
                                                    int32_t* __restrict__ slot_row) {
  extern __shared__ uint64_t masks[];  // [4][NL]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * NL; i += 256) masks[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * BLK_TOK + tid;
  const bool live = t < T;
  if (live) {
    for (int j = 0; j < k; ++j) {
      const int n = idx[(int64_t)t * k + j] - e0;
      if ((unsigned)n < (unsigned)NL) atomicOr((unsigned long long*)&masks[wave * NL + n], 1ull << lane);
    }
  }
  __syncthreads();
  if (!live) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int n = idx[(int64_t)t * k + j] - e0;
    int row = -1;
    if ((unsigned)n < (unsigned)NL) {
      int before = __popcll(masks[wave * NL + n] & below);
      for (int w = 0; w < wave; ++w) before += __popcll(masks[w * NL + n]);
      row = offsets[n] + base_rel[(int64_t)n * nblk + blockIdx.x] + before;
      row_token[row] = t;
    }
    slot_row[(int64_t)t * k + j] = row;
  }
}

// x_perm[slot_row[t][j]] = x[t] for every local slot: one wave per token,
// 16-byte vectors, the token's row read once.
__global__ void __launch_bounds__(256) gather_kernel(const uint8_t* __restrict__ x,
                                                     const int32_t* __restrict__ slot_row, int T, int k,
                                                     int64_t row_bytes, uint8_t* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const uint64_t live = __ballot(r >= 0);
  if (!live) return;
  const int64_t nvec = row_bytes / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)t * row_bytes);
  constexpr int U = 4;
  for (int64_t c0 = 0; c0 < nvec; c0 += 64 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * 64 + lane;
      if (c < nvec) v[u] = src[c];
    }
    uint64_t m = live;
    while (m) {
      const int j = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int row = __shfl(r, j, 64);
      u32x4* dst = reinterpret_cast<u32x4*>(x_perm + (int64_t)row * row_bytes);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * 64 + lane;
        if (c < nvec) dst[c] = v[u];
      }
    }
  }
}

// y[t] = sum_j w[t][j] y_perm[slot_row[t][j]] in slot order, float32 sums.
template <typename T>
__global__ void __launch_bounds__(256) combine_kernel(const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ w, const T* __restrict__ y_perm,
                                                      int Tn, int k, int d, T* __restrict__ y) {
  using V = Vec16<T>;
  constexpr int VN = V::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const float wl = lane < k ? w[(int64_t)t * k + lane] : 0.f;
  const uint64_t live = __ballot(r >= 0);
  constexpr int U = 2;
  for (int c0 = 0; c0 < d; c0 += 64 * VN * U) {
    float acc[U][VN];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[u][e] = 0.f;
    uint64_t m = live;
    while (m) {
      const int j = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int row = __shfl(r, j, 64);
      const float wj = __shfl(wl, j, 64);
      const T* src = y_perm + (int64_t)row * d;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + (u * 64 + lane) * VN;
        if (c < d) {
          float v[VN];
          V::load(src + c, v);
#pragma unroll
          for (int e = 0; e < VN; ++e) acc[u][e] = fmaf(wj, v[e], acc[u][e]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + (u * 64 + lane) * VN;
      if (c < d) V::store(y + (int64_t)t * d + c, acc[u]);
    }
  }
}

// dy_perm[row] = w dy[t] (when dy_perm is given);  dw[t][j] = <y_perm[row], dy[t]>
// (0 for non-local slots);  row_w[row] = w (when row_w is given: the weight
// each routed row carries, for a backward that reads dy in place).
template <typename T>
__global__ void __launch_bounds__(256) combine_bwd_kernel(const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ w,
                                                          const T* __restrict__ y_perm,
                                                          const T* __restrict__ dy, int Tn, int k, int d,
                                                          T* __restrict__ dy_perm, float* __restrict__ dw,
                                                          float* __restrict__ row_w) {
  using V = Vec16<T>;
  constexpr int VN = V::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const float wl = lane < k ? w[(int64_t)t * k + lane] : 0.f;
  const uint64_t live = __ballot(r >= 0);
  if (row_w && r >= 0) row_w[r] = wl;
  float mydot = 0.f;  // lane j ends with slot j's dot product
  uint64_t m = live;
  while (m) {
    const int j = __ffsll((unsigned long long)m) - 1;
    m &= m - 1;
    const int row = __shfl(r, j, 64);
    const float wj = __shfl(wl, j, 64);
    const T* yp = y_perm + (int64_t)row * d;
    const T* g = dy + (int64_t)t * d;
    T* out = dy_perm + (int64_t)row * d;
    float part = 0.f;
    for (int c = lane * VN; c < d; c += 64 * VN) {
      float gv[VN], yv[VN], ov[VN];
      V::load(g + c, gv);
      V::load(yp + c, yv);
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        part = fmaf(yv[e], gv[e], part);
        ov[e] = wj * gv[e];
      }
      if (dy_perm) V::store(out + c, ov);
    }
    part = wave_sum(part);
    if (lane == j) mydot = part;
  }
  if (lane < k) dw[(int64_t)t * k + lane] = mydot;
}

// dx[t] = dx_add[t] + sum_j dx_perm[slot_row[t][j]] (float32 sums).
template <typename T>
__global__ void __launch_bounds__(256) unpermute_bwd_kernel(const int32_t* __restrict__ slot_row,
                                                            const T* __restrict__ dx_perm,
                                                            const float* __restrict__ dx_add, int Tn, int k,
                                                            int d, T* __restrict__ dx) {
  using V = Vec16<T>;
  constexpr int VN = V::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const uint64_t live = __ballot(r >= 0);
  for (int c = lane * VN; c < d; c += 64 * VN) {
    float acc[VN];
    if (dx_add) {
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] = dx_add[(int64_t)t * d + c + e];
    } else {
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] = 0.f;
    }
    uint64_t m = live;
    while (m) {
      const int j = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int row = __shfl(r, j, 64);
      float v[VN];
      V::load(dx_perm + (int64_t)row * d + c, v);
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] += v[e];
    }
    V::store(dx + (int64_t)t * d + c, acc);
  }
}

// ---------------------------------------------------------------------------
size_t permute_workspace(const moe_desc& d) {
  const int64_t nblk = (d.T + BLK_TOK - 1) / BLK_TOK;
  // blk_counts [E][nblk] + base [NL][nblk]
  return (size_t)((int64_t)d.E * nblk + (int64_t)d.num_local * nblk) * sizeof(int32_t);
}

// Fixed device scratch of the allocation-free permute: the per-block counts
// and bases that moe_permute keeps in the caller's workspace.  Every kernel
// writes each entry it later reads, so nothing needs clearing between calls.
// Each device holds its own copy, at its own address, for the life of the
// process; host code uses only that address (from hipGetSymbolAddress),
// never the array's name.
static __device__ __align__(256) int32_t scratch[PERMUTE_SCRATCH_BYTES / sizeof(int32_t)];

namespace {
constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_addr[MAX_DEVICES];
std::mutex g_scratch_mu;
}  // namespace

// The current device's scratch address, resolved on the first call on that
// device (with it current) and kept.
hipError_t permute_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_permute_noalloc(const moe_desc& d, const int32_t* idx, const void* x, int32_t* counts,
                                  int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm,
                                  hipStream_t s) {
  if (permute_workspace(d) > PERMUTE_SCRATCH_BYTES) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = permute_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_permute(d, idx, x, counts, offsets, row_token, slot_row, x_perm, ws, s);
}

hipError_t launch_permute(const moe_desc& d, const int32_t* idx, const void* x, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm, void* ws,
                          hipStream_t s) {
  const int nblk = (d.T + BLK_TOK - 1) / BLK_TOK;
  int32_t* blk_counts = reinterpret_cast<int32_t*>(ws);
  int32_t* base = blk_counts + (int64_t)d.E * nblk;
  count_kernel<<<nblk, 256, 4 * d.E * sizeof(uint64_t), s>>>(idx, d.T, d.k, d.E, blk_counts, nblk);
  expert_scan_kernel<<<d.E, 256, 0, s>>>(blk_counts, nblk, d.expert_begin, d.num_local, counts, base);
  offsets_kernel<<<1, 1024, 0, s>>>(counts, d.expert_begin, d.num_local, offsets);
  place_kernel<<<nblk, 256, 4 * d.num_local * sizeof(uint64_t), s>>>(idx, d.T, d.k, d.E, d.expert_begin,
                                                                      d.num_local, offsets, base, nblk,
                                                                      row_token, slot_row);
  if (x) {
    const int64_t row_bytes = (int64_t)d.d * (d.dtype == MOE_BF16 ? 2 : 4);
    gather_kernel<<<(d.T + 3) / 4, 256, 0, s>>>(reinterpret_cast<const uint8_t*>(x), slot_row, d.T, d.k,
                                                row_bytes, reinterpret_cast<uint8_t*>(x_perm));
  }
  return hipGetLastError();
}

// Batched forms of the three slot loops above for k <= KB: per chunk of the
// row, every live slot's loads are issued before any of them is used, so a
// wave keeps up to KB row pieces in flight instead of one.  The sums run in
// the same slot order as above, so the results are bitwise the same.
namespace batched {
template <typename T> struct Raw;  // 16 bytes of a row, widened to float
template <> struct Raw<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void widen(const u32x4& q, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void widen(const u32x4& q, float (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(q[i]);
  }
};
template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) { return *reinterpret_cast<const u32x4*>(p); }
}  // namespace batched

template <typename T, int KB>
__global__ void __launch_bounds__(256) combine_kernel_b(const int32_t* __restrict__ slot_row,
                                                        const float* __restrict__ w, const T* __restrict__ y_perm,
                                                        int Tn, int k, int d, T* __restrict__ y) {
  using R = batched::Raw<T>;
  constexpr int VN = R::N, U = 1;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const float wl = lane < k ? w[(int64_t)t * k + lane] : 0.f;
  const uint64_t live = __ballot(r >= 0);
  int64_t rows[KB];
  float wj[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    rows[j] = (int64_t)__shfl(r, j, 64) * d;
    wj[j] = __shfl(wl, j, 64);
  }
  for (int c0 = 0; c0 < d; c0 += 64 * VN * U) {
    u32x4 q[KB][U];
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if ((live >> j) & 1)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + (u * 64 + lane) * VN;
          if (c < d) q[j][u] = batched::ld16(y_perm + rows[j] + c);
        }
    float acc[U][VN];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[u][e] = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if ((live >> j) & 1)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float v[VN];
          R::widen(q[j][u], v);
#pragma unroll
          for (int e = 0; e < VN; ++e) acc[u][e] = fmaf(wj[j], v[e], acc[u][e]);
        }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + (u * 64 + lane) * VN;
      if (c < d) Vec16<T>::store(y + (int64_t)t * d + c, acc[u]);
    }
  }
}

template <typename T, int KB>
__global__ void __launch_bounds__(256) combine_bwd_kernel_b(const int32_t* __restrict__ slot_row,
                                                            const float* __restrict__ w,
                                                            const T* __restrict__ y_perm,
                                                            const T* __restrict__ dy, int Tn, int k, int d,
                                                            T* __restrict__ dy_perm, float* __restrict__ dw,
                                                            float* __restrict__ row_w) {
  using R = batched::Raw<T>;
  constexpr int VN = R::N, U = 2;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const float wl = lane < k ? w[(int64_t)t * k + lane] : 0.f;
  const uint64_t live = __ballot(r >= 0);
  if (row_w && r >= 0) row_w[r] = wl;
  int64_t rows[KB];
  float wj[KB], part[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    rows[j] = (int64_t)__shfl(r, j, 64) * d;
    wj[j] = __shfl(wl, j, 64);
    part[j] = 0.f;
  }
  const T* g = dy + (int64_t)t * d;
  for (int c0 = 0; c0 < d; c0 += 64 * VN * U) {
    u32x4 gq[U], q[KB][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + (u * 64 + lane) * VN;
      if (c < d) gq[u] = batched::ld16(g + c);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if ((live >> j) & 1)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + (u * 64 + lane) * VN;
          if (c < d) q[j][u] = batched::ld16(y_perm + rows[j] + c);
        }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + (u * 64 + lane) * VN;
      if (c >= d) continue;
      float gv[VN];
      R::widen(gq[u], gv);
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if ((live >> j) & 1) {
          float yv[VN], ov[VN];
          R::widen(q[j][u], yv);
#pragma unroll
          for (int e = 0; e < VN; ++e) {
            part[j] = fmaf(yv[e], gv[e], part[j]);
            ov[e] = wj[j] * gv[e];
          }
          if (dy_perm) Vec16<T>::store(dy_perm + rows[j] + c, ov);
        }
    }
  }
  float mydot = 0.f;  // lane j ends with slot j's dot product
#pragma unroll
  for (int j = 0; j < KB; ++j)
    if ((live >> j) & 1) {
      const float sj = wave_sum(part[j]);
      if (lane == j) mydot = sj;
    }
  if (lane < k) dw[(int64_t)t * k + lane] = mydot;
}

template <typename T, int KB>
__global__ void __launch_bounds__(256) unpermute_bwd_kernel_b(const int32_t* __restrict__ slot_row,
                                                              const T* __restrict__ dx_perm,
                                                              const float* __restrict__ dx_add, int Tn, int k,
                                                              int d, T* __restrict__ dx) {
  using R = batched::Raw<T>;
  constexpr int VN = R::N, U = 2;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const uint64_t live = __ballot(r >= 0);
  int64_t rows[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) rows[j] = (int64_t)__shfl(r, j, 64) * d;
  for (int c0 = 0; c0 < d; c0 += 64 * VN * U) {
    float acc[U][VN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + (u * 64 + lane) * VN;
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[u][e] = 0.f;
      if (dx_add && c < d) {
#pragma unroll
        for (int e4 = 0; e4 < VN; e4 += 4) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(dx_add + (int64_t)t * d + c + e4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[u][e4 + e] = a[e];
        }
      }
    }
    u32x4 q[KB][U];
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if ((live >> j) & 1)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + (u * 64 + lane) * VN;
          if (c < d) q[j][u] = batched::ld16(dx_perm + rows[j] + c);
        }
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if ((live >> j) & 1)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float v[VN];
          R::widen(q[j][u], v);
#pragma unroll
          for (int e = 0; e < VN; ++e) acc[u][e] += v[e];
        }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + (u * 64 + lane) * VN;
      if (c < d) Vec16<T>::store(dx + (int64_t)t * d + c, acc[u]);
    }
  }
}

// dx[t] = sum_j dx_perm[slot_row[t][j]] + sum_j dL[t][e_j] W_r[e_j], e_j =
// topk_idx[t][j], dL the router-logit gradient.  With the weights
// renormalised over the selection, dL is zero outside it, so the router's
// share of dx, dlogits[t] W_r, is that sum of k rows of W_r: k multiply-adds
// per element here instead of a T x d x E product.  Sums in float32, the
// expert rows in slot order, then the router rows in slot order; one
// rounding at the store.
//
// W_r (E x d) is read by every token; at E = 384, d = 6144 it is 4.7 MB, more
// than one XCD's 4 MB L2.  So the columns are cut into 2^lg_s slices: block
// b takes slice b mod 2^lg_s of four tokens, and as consecutive blocks go to
// consecutive XCDs, each XCD reads only its slices' columns of W_r, which
// then fit in its L2.  The streamed operands (dx_perm in, dx out) carry the
// non-temporal hint so that they do not push W_r out.  Each wave takes one
// token's slice; per chunk of it every load (the live expert rows and the k
// router rows) is issued before any is used.
//
// With 96 of 384 experts local, about two of a token's eight slots have a
// local row, so the k rows of W_r are most of what a token reads (6.4 GB from
// L2 per pass at T = 65536, against 1.6 GB of dx_perm from HBM): the pass is
// bound by those L2 reads, not by HBM.  Measured at that shape: 0.747 ms with
// one slice, 0.691 with the hint, 0.672 with two slices and the hint, 0.695
// with four, 0.86 with eight.
constexpr bool kUnpermStreamHint = true;
namespace batched {
template <typename T>
__device__ __forceinline__ u32x4 ld16_stream(const T* p) {
  if constexpr (kUnpermStreamHint) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}
template <typename T, int N>
__device__ __forceinline__ void st16_stream(T* p, const float (&v)[N]) {
  u32x4 q;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = pack_bf2(v[2 * i], v[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = __float_as_uint(v[i]);
  }
  if constexpr (kUnpermStreamHint) __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = q;
}
}  // namespace batched

template <typename T, int KB>
__global__ void __launch_bounds__(256) unpermute_router_bwd_kernel_b(
    const int32_t* __restrict__ slot_row, const T* __restrict__ dx_perm, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dlogits, const T* __restrict__ wr, int Tn, int k, int E, int d, int lg_s,
    T* __restrict__ dx) {
  using R = batched::Raw<T>;
  constexpr int VN = R::N;
  const int lane = threadIdx.x & 63;
  const int t = (int)(blockIdx.x >> lg_s) * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int sw = d >> lg_s;  // a multiple of VN (d % 64 == 0, lg_s <= 3)
  const int c0 = (int)(blockIdx.x & ((1u << lg_s) - 1)) * sw, c1 = c0 + sw;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const int ex = lane < k ? min(max(topk_idx[(int64_t)t * k + lane], 0), E - 1) : 0;  // (clamped: no read outside W_r)
  const float g = lane < k ? dlogits[(int64_t)t * E + ex] : 0.f;
  const uint64_t live = __ballot(r >= 0);
  int64_t rows[KB], erows[KB];
  float gj[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    rows[j] = (int64_t)__shfl(r, j, 64) * d;
    erows[j] = (int64_t)__shfl(ex, j, 64) * d;
    gj[j] = __shfl(g, j, 64);
  }
  for (int c = c0 + lane * VN; c < c1; c += 64 * VN) {
    u32x4 q[KB], qw[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if ((live >> j) & 1) q[j] = batched::ld16_stream(dx_perm + rows[j] + c);
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (j < k) qw[j] = batched::ld16(wr + erows[j] + c);
    float acc[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if ((live >> j) & 1) {
        float v[VN];
        R::widen(q[j], v);
#pragma unroll
        for (int e = 0; e < VN; ++e) acc[e] += v[e];
      }
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (j < k) {
        float v[VN];
        R::widen(qw[j], v);
#pragma unroll
        for (int e = 0; e < VN; ++e) acc[e] = fmaf(gj[j], v[e], acc[e]);
      }
    batched::st16_stream<T, VN>(dx + (int64_t)t * d + c, acc);
  }
}

// The same for any k <= 64, one slot at a time.
template <typename T>
__global__ void __launch_bounds__(256) unpermute_router_bwd_kernel(
    const int32_t* __restrict__ slot_row, const T* __restrict__ dx_perm, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dlogits, const T* __restrict__ wr, int Tn, int k, int E, int d,
    T* __restrict__ dx) {
  using V = Vec16<T>;
  constexpr int VN = V::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  const int r = lane < k ? slot_row[(int64_t)t * k + lane] : -1;
  const int ex = lane < k ? min(max(topk_idx[(int64_t)t * k + lane], 0), E - 1) : 0;  // (clamped: no read outside W_r)
  const float g = lane < k ? dlogits[(int64_t)t * E + ex] : 0.f;
  const uint64_t live = __ballot(r >= 0);
  for (int c = lane * VN; c < d; c += 64 * VN) {
    float acc[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) acc[e] = 0.f;
    uint64_t m = live;
    while (m) {
      const int j = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      float v[VN];
      V::load(dx_perm + (int64_t)__shfl(r, j, 64) * d + c, v);
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] += v[e];
    }
    for (int j = 0; j < k; ++j) {
      const float gs = __shfl(g, j, 64);
      float v[VN];
      V::load(wr + (int64_t)__shfl(ex, j, 64) * d + c, v);
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] = fmaf(gs, v[e], acc[e]);
    }
    V::store(dx + (int64_t)t * d + c, acc);
  }
}

// row_w[slot_row[i]] = w[i] for every local slot i of the T x k selections.
__global__ void __launch_bounds__(256) row_weights_kernel(const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ w, int64_t n,
                                                          float* __restrict__ row_w) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int r = slot_row[i];
    if (r >= 0) row_w[r] = w[i];
  }
}

// dtopk_w[i] = the sum, in order, of the P partial sums of slot i's row (0
// for a slot whose expert is not local).
__global__ void __launch_bounds__(256) dtopk_parts_kernel(const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ part, int P, int64_t n,
                                                          float* __restrict__ dtopk_w) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int r = slot_row[i];
    float s = 0.f;
    if (r >= 0)
      for (int q = 0; q < P; ++q) s += part[(int64_t)r * P + q];
    dtopk_w[i] = s;
  }
}

hipError_t launch_combine(const moe_desc& d, const int32_t* slot_row, const float* w, const void* y_perm,
                          void* y, hipStream_t s) {
  const dim3 grid((d.T + 3) / 4), block(256);
  const bool b8 = d.k <= 8;
  if (d.dtype == MOE_BF16) {
    if (b8)
      combine_kernel_b<uint16_t, 8><<<grid, block, 0, s>>>(slot_row, w, (const uint16_t*)y_perm, d.T, d.k, d.d,
                                                           (uint16_t*)y);
    else
      combine_kernel<uint16_t><<<grid, block, 0, s>>>(slot_row, w, (const uint16_t*)y_perm, d.T, d.k, d.d,
                                                      (uint16_t*)y);
  } else {
    if (b8)
      combine_kernel_b<float, 8><<<grid, block, 0, s>>>(slot_row, w, (const float*)y_perm, d.T, d.k, d.d,
                                                        (float*)y);
    else
      combine_kernel<float><<<grid, block, 0, s>>>(slot_row, w, (const float*)y_perm, d.T, d.k, d.d, (float*)y);
  }
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const moe_desc& d, const int32_t* slot_row, const float* w, const void* y_perm,
                              const void* dy, void* dy_perm, float* dw, hipStream_t s, float* row_w) {
  const dim3 grid((d.T + 3) / 4), block(256);
  const bool b8 = d.k <= 8;
  if (d.dtype == MOE_BF16) {
    if (b8)
      combine_bwd_kernel_b<uint16_t, 8><<<grid, block, 0, s>>>(slot_row, w, (const uint16_t*)y_perm,
                                                               (const uint16_t*)dy, d.T, d.k, d.d,
                                                               (uint16_t*)dy_perm, dw, row_w);
    else
      combine_bwd_kernel<uint16_t><<<grid, block, 0, s>>>(slot_row, w, (const uint16_t*)y_perm,
                                                          (const uint16_t*)dy, d.T, d.k, d.d,
                                                          (uint16_t*)dy_perm, dw, row_w);
  } else {
    if (b8)
      combine_bwd_kernel_b<float, 8><<<grid, block, 0, s>>>(slot_row, w, (const float*)y_perm, (const float*)dy,
                                                            d.T, d.k, d.d, (float*)dy_perm, dw, row_w);
    else
      combine_bwd_kernel<float><<<grid, block, 0, s>>>(slot_row, w, (const float*)y_perm, (const float*)dy, d.T,
                                                       d.k, d.d, (float*)dy_perm, dw, row_w);
  }
  return hipGetLastError();
}

hipError_t launch_unpermute_bwd(const moe_desc& d, const int32_t* slot_row, const void* dx_perm,
                                const float* dx_add, void* dx, hipStream_t s) {
  const dim3 grid((d.T + 3) / 4), block(256);
  const bool b8 = d.k <= 8;
  if (d.dtype == MOE_BF16) {
    if (b8)
      unpermute_bwd_kernel_b<uint16_t, 8><<<grid, block, 0, s>>>(slot_row, (const uint16_t*)dx_perm, dx_add, d.T,
                                                                 d.k, d.d, (uint16_t*)dx);
    else
      unpermute_bwd_kernel<uint16_t><<<grid, block, 0, s>>>(slot_row, (const uint16_t*)dx_perm, dx_add, d.T,
                                                            d.k, d.d, (uint16_t*)dx);
  } else {
    if (b8)
      unpermute_bwd_kernel_b<float, 8><<<grid, block, 0, s>>>(slot_row, (const float*)dx_perm, dx_add, d.T, d.k,
                                                              d.d, (float*)dx);
    else
      unpermute_bwd_kernel<float><<<grid, block, 0, s>>>(slot_row, (const float*)dx_perm, dx_add, d.T, d.k, d.d,
                                                         (float*)dx);
  }
  return hipGetLastError();
}

// Column slices per token in the unpermute + router pass: up to 2, each at
// least one wave-wide chunk.
constexpr int kUnpermMaxLgSlices = 1;

hipError_t launch_unpermute_router_bwd(const moe_desc& d, const int32_t* slot_row, const void* dx_perm,
                                       const int32_t* topk_idx, const float* dlogits, const void* Wr, void* dx,
                                       hipStream_t s) {
  const dim3 block(256);
  const int vn = d.dtype == MOE_BF16 ? 8 : 4;
  int lg_s = 0;
  while (lg_s < kUnpermMaxLgSlices && (d.d >> (lg_s + 1)) >= 64 * vn) ++lg_s;
  const dim3 gridb((unsigned)((d.T + 3) / 4) << lg_s), grid((d.T + 3) / 4);
  const bool b8 = d.k <= 8;
  if (d.dtype == MOE_BF16) {
    if (b8)
      unpermute_router_bwd_kernel_b<uint16_t, 8><<<gridb, block, 0, s>>>(
          slot_row, (const uint16_t*)dx_perm, topk_idx, dlogits, (const uint16_t*)Wr, d.T, d.k, d.E, d.d, lg_s,
          (uint16_t*)dx);
    else
      unpermute_router_bwd_kernel<uint16_t><<<grid, block, 0, s>>>(slot_row, (const uint16_t*)dx_perm, topk_idx,
                                                                   dlogits, (const uint16_t*)Wr, d.T, d.k, d.E,
                                                                   d.d, (uint16_t*)dx);
  } else {
    if (b8)
      unpermute_router_bwd_kernel_b<float, 8><<<gridb, block, 0, s>>>(slot_row, (const float*)dx_perm, topk_idx,
                                                                      dlogits, (const float*)Wr, d.T, d.k, d.E,
                                                                      d.d, lg_s, (float*)dx);
    else
      unpermute_router_bwd_kernel<float><<<grid, block, 0, s>>>(slot_row, (const float*)dx_perm, topk_idx,
                                                                dlogits, (const float*)Wr, d.T, d.k, d.E, d.d,
                                                                (float*)dx);
  }
  return hipGetLastError();
}

hipError_t launch_row_weights(const moe_desc& d, const int32_t* slot_row, const float* w, float* row_w,
                              hipStream_t s) {
  const int64_t n = (int64_t)d.T * d.k;
  const int64_t g = std::min<int64_t>((n + 255) / 256, (int64_t)num_cus() * 8);
  row_weights_kernel<<<(unsigned)g, 256, 0, s>>>(slot_row, w, n, row_w);
  return hipGetLastError();
}

hipError_t launch_dtopk_from_parts(const moe_desc& d, const int32_t* slot_row, const float* part, float* dtopk_w,
                                   hipStream_t s) {
  const int64_t n = (int64_t)d.T * d.k;
  const int64_t g = std::min<int64_t>((n + 255) / 256, (int64_t)num_cus() * 8);
  dtopk_parts_kernel<<<(unsigned)g, 256, 0, s>>>(slot_row, part, dtopk_parts(d), n, dtopk_w);
  return hipGetLastError();
}

}  // namespace moe
