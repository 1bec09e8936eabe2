// FP8 (E4M3) blockwise weight quantisation and dequantisation (Domyn page,
// section "FP8 expert weight all-gather": blocks of 128 values are scaled to
// the E4M3 range and cast, one float32 scale per block, and dequantised to
// bf16 before the expert GEMMs).
//
// A block of 128 values is 16 lanes of 8 values: each lane loads its 8 values
// in one vector load, the block maximum is a 4-step butterfly inside the
// 16-lane group, and the codes leave as one 8-byte store.  Both kernels move
// about 3 bytes per value and are bound by HBM.  The conversions are gfx950's
// v_cvt_pk_fp8_f32 (round to nearest even) and v_cvt_f32_fp8.
#include <algorithm>

#include "internal.h"

namespace moe {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4_ w = *reinterpret_cast<const u32x4_*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// Scale = amax / 448 and inverse 448 / amax in float32 (both correctly
// rounded); each value is w * inverse, clamped to +-448 (the product may
// round past it) and cast.  An all-zero block has scale 0 and zero codes.
template <typename T>
__global__ void __launch_bounds__(256) fp8_quant_kernel(const T* __restrict__ w, int64_t nblk,
                                                        uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int sub = threadIdx.x & 15;
  for (int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4; blk < nblk;
       blk += ((int64_t)gridDim.x * 256) >> 4) {
    float v[8];
    load8(w + blk * 128 + sub * 8, v);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const bool nz = amax > 0.f;
    const float inv = nz ? 448.0f / amax : 0.f;
    uint32_t c[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = fminf(fmaxf(v[4 * h + i] * inv, -448.0f), 448.0f);
      int r = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      r = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], r, true);
      c[h] = nz ? (uint32_t)r : 0u;
    }
    const u32x2 out = {c[0], c[1]};
    *reinterpret_cast<u32x2*>(q + blk * 128 + sub * 8) = out;
    if (sub == 0) scales[blk] = nz ? amax / 448.0f : 0.f;
  }
}

// Power-of-two block scales (the scale a block-scaled FP8 matrix instruction
// applies): e = the least integer with amax <= 448 * 2^e, from amax = f 2^x
// (f in [0.5, 1)): x - 9 when f <= 0.875, else x - 8; each value w * 2^-e
// (exact) is cast; the scale leaves as its E8M0 byte e + 127.  An all-zero
// block gets e = 0.  One block per 16-lane group: src and dst its values and
// codes; returns the scale byte (in every lane of the group).
template <typename T>
__device__ __forceinline__ uint8_t quant_pow2_block(const T* src, uint8_t* dst, int sub) {
  float v[8];
  load8(src + sub * 8, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  int x = 0;
  const float f = frexpf(amax, &x);
  const int e = amax > 0.f ? (f <= 0.875f ? x - 9 : x - 8) : 0;
  uint32_t c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = ldexpf(v[4 * h + i], -e);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);
    c[h] = (uint32_t)r;
  }
  const u32x2 out = {c[0], c[1]};
  *reinterpret_cast<u32x2*>(dst + sub * 8) = out;
  return (uint8_t)(e + 127);
}

template <typename T>
__global__ void __launch_bounds__(256) fp8_quant_pow2_kernel(const T* __restrict__ w, int64_t nblk,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ e8) {
  const int sub = threadIdx.x & 15;
  for (int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4; blk < nblk;
       blk += ((int64_t)gridDim.x * 256) >> 4) {
    const uint8_t b = quant_pow2_block(w + blk * 128, q + blk * 128, sub);
    if (sub == 0) e8[blk] = b;
  }
}

// By rows: w [rows][cols], codes [rows][cols], scales [rows][e8_ld] (the
// bytes past cols/128 set to zero); rows at or past *nrows (if given) are
// left alone.
template <typename T>
__global__ void __launch_bounds__(256) fp8_quant_pow2_rows_kernel(const T* __restrict__ w, int64_t rows, int64_t cols,
                                                                  const int32_t* __restrict__ nrows,
                                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ e8,
                                                                  int64_t e8_ld) {
  const int sub = threadIdx.x & 15;
  const int64_t cb = cols / 128;
  const int64_t lim = nrows ? min(rows, (int64_t)*nrows) : rows;
  const int64_t nblk = lim * cb;
  for (int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4; blk < nblk;
       blk += ((int64_t)gridDim.x * 256) >> 4) {
    const int64_t r = blk / cb, j = blk - r * cb;
    const uint8_t b = quant_pow2_block(w + r * cols + j * 128, q + r * cols + j * 128, sub);
    if (sub == 0) e8[r * e8_ld + j] = b;
    if (j == cb - 1 && sub > 0 && cb + sub - 1 < e8_ld) e8[r * e8_ld + cb + sub - 1] = 0;
  }
}

// bf16 value = decode(code) * scale in float32, rounded to nearest even.
__global__ void __launch_bounds__(256) fp8_dequant_kernel(const uint8_t* __restrict__ q, const float* __restrict__ scales,
                                                          int64_t nblk, uint16_t* __restrict__ w) {
  const int sub = threadIdx.x & 15;
  for (int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4; blk < nblk;
       blk += ((int64_t)gridDim.x * 256) >> 4) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(q + blk * 128 + sub * 8);
    const float s = scales[blk];
    u32x4_ out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ch = (int)c[h];
      out[2 * h] = pack_bf2(__builtin_amdgcn_cvt_f32_fp8(ch, 0) * s, __builtin_amdgcn_cvt_f32_fp8(ch, 1) * s);
      out[2 * h + 1] = pack_bf2(__builtin_amdgcn_cvt_f32_fp8(ch, 2) * s, __builtin_amdgcn_cvt_f32_fp8(ch, 3) * s);
    }
    *reinterpret_cast<u32x4_*>(w + blk * 128 + sub * 8) = out;
  }
}

int64_t grid_for(int64_t nblk) {
  // 16 blocks per 256-thread workgroup; enough workgroups to fill the chip a few times over.
  return std::max<int64_t>(1, std::min<int64_t>((nblk + 15) / 16, (int64_t)num_cus() * 16));
}

}  // namespace

hipError_t launch_fp8_quantize(const void* w, int dtype, int64_t n, uint8_t* q, float* scales, hipStream_t s) {
  const int64_t nblk = n / 128;
  if (nblk == 0) return hipSuccess;
  if (dtype == MOE_BF16)
    fp8_quant_kernel<uint16_t><<<(unsigned)grid_for(nblk), 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w), nblk, q,
                                                                         scales);
  else
    fp8_quant_kernel<float><<<(unsigned)grid_for(nblk), 256, 0, s>>>(reinterpret_cast<const float*>(w), nblk, q, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_pow2(const void* w, int dtype, int64_t n, uint8_t* q, uint8_t* e8, hipStream_t s) {
  const int64_t nblk = n / 128;
  if (nblk == 0) return hipSuccess;
  if (dtype == MOE_BF16)
    fp8_quant_pow2_kernel<uint16_t><<<(unsigned)grid_for(nblk), 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w),
                                                                              nblk, q, e8);
  else
    fp8_quant_pow2_kernel<float><<<(unsigned)grid_for(nblk), 256, 0, s>>>(reinterpret_cast<const float*>(w), nblk, q,
                                                                           e8);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_pow2_rows(const void* w, int dtype, int64_t rows, int64_t cols, const int32_t* nrows,
                                         uint8_t* q, uint8_t* e8, int64_t e8_ld, hipStream_t s) {
  const int64_t nblk = rows * (cols / 128);
  if (nblk == 0) return hipSuccess;
  const unsigned g = (unsigned)grid_for(nblk);
  if (dtype == MOE_BF16)
    fp8_quant_pow2_rows_kernel<uint16_t><<<g, 256, 0, s>>>(reinterpret_cast<const uint16_t*>(w), rows, cols, nrows, q,
                                                           e8, e8_ld);
  else
    fp8_quant_pow2_rows_kernel<float><<<g, 256, 0, s>>>(reinterpret_cast<const float*>(w), rows, cols, nrows, q, e8,
                                                        e8_ld);
  return hipGetLastError();
}

hipError_t launch_fp8_dequantize(const uint8_t* q, const float* scales, int64_t n, void* w, hipStream_t s) {
  const int64_t nblk = n / 128;
  if (nblk == 0) return hipSuccess;
  fp8_dequant_kernel<<<(unsigned)grid_for(nblk), 256, 0, s>>>(q, scales, nblk, reinterpret_cast<uint16_t*>(w));
  return hipGetLastError();
}

}  // namespace moe
