// Softmax + top-k routing and its backward (Aurora page, section 3.1,
// Algorithm 1 stage 1: probs = Softmax(logits); weights, indices = TopK(probs),
// with the top-k probabilities renormalised over the selection by default).
//
// One wavefront owns one token: lane l holds logits l, l+64, l+128, ... of the
// token's row (coalesced 256-byte loads), and each of the k rounds is a
// lane-local arg-max followed by a 6-step butterfly over the wave.  The order
// is (logit descending, expert index ascending), so equal logits - including
// +0.0 against -0.0 - go to the lower expert.  The whole pass reads T*E*4
// bytes and writes T*k*8; it is bound by HBM.
#include "internal.h"

namespace moe {

// Group-limited selection (Domyn page, section "Group-limited expert
// routing"): with G > 1 groups of Eg = E/G consecutive experts, each group
// may give at most k/G experts.  The rounds still take the best remaining
// eligible expert, and once a group has given its quota its other experts
// leave the race, so the k picks are the union of every group's k/G best, in
// descending order (the eligible set only shrinks).  Lane g counts group g's
// picks.
//
// k rounds of a lane-local arg-max and a wave butterfly over the wave's
// token (v: the lane's logits, element i = expert i*64 + lane); writes the
// token's k selections and weights.
template <int MAXV, bool GROUPED>
__device__ __forceinline__ void topk_rounds(const float (&v)[MAXV], int lane, int t, int E, int k, int renorm,
                                            int G, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  uint32_t taken = 0;  // bit i: element i is selected already or absent
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (i * 64 + lane >= E) taken |= 1u << i;
  float my_v = 0.f, v0 = 0.f;
  int my_i = 0;
  const int Eg = GROUPED ? E / G : E, kg = GROUPED ? k / G : k;
  int group_picks = 0;  // lane g: experts taken from group g so far
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      if (!((taken >> i) & 1u) && (bi == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        bi = i * 64 + lane;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      const bool better = (oi != 0x7fffffff) && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi));
      if (better) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (GROUPED) {
      const int g = bi / Eg;
      if (lane == g) ++group_picks;
      if (__shfl(group_picks, g, 64) == kg) {  // the group is full: its other experts leave
#pragma unroll
        for (int i = 0; i < MAXV; ++i)
          if ((i * 64 + lane) / Eg == g) taken |= 1u << i;
      }
    }
    if (lane == j) {
      my_v = bv;
      my_i = bi;
    }
    if (j == 0) v0 = bv;
  }
  float w;
  if (renorm) {
    const float ex = lane < k ? expf(my_v - v0) : 0.f;
    w = ex / wave_sum(ex);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (i * 64 + lane < E) s += expf(v[i] - v0);
    s = wave_sum(s);
    w = expf(my_v - v0) / s;
  }
  if (lane < k) {
    idx_out[(int64_t)t * k + lane] = my_i;
    w_out[(int64_t)t * k + lane] = w;
  }
}

// Order-preserving unsigned key of a float (larger float, larger key), with
// -0.0 made equal to +0.0; 0 is below every finite float's key and marks an
// absent element.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);  // -0.0 + 0.0 = +0.0
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

template <int MAXV, bool GROUPED>
__global__ void __launch_bounds__(256) topk_route_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, int renorm, int G,
                                                         int32_t* __restrict__ idx_out,
                                                         float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;
  float v[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = i * 64 + lane;
    v[i] = e < E ? row[e] : 0.f;
  }
  if (GROUPED) {
    topk_rounds<MAXV, GROUPED>(v, lane, t, E, k, renorm, G, idx_out, w_out);
    return;
  }
  // Threshold selection.  theta = the k-th largest of the lanes' maximum keys
  // (a binary search over the key bits, counting lanes with ballots): at
  // least k elements have key >= theta, so every one of the k selections
  // does, and the candidates (key >= theta) are usually few.  They are
  // compacted through LDS, and a candidate's slot is the number of
  // candidates that come before it in the order (logit descending, expert
  // ascending).  With more than 64 candidates (heavy ties) the wave takes
  // the k rounds instead.
  uint32_t key[MAXV];
  uint32_t kmax = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    key[i] = i * 64 + lane < E ? order_key(v[i]) : 0u;
    kmax = max(kmax, key[i]);
  }
  uint32_t theta = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = theta | (1u << b);
    if ((int)__popcll(__ballot(kmax >= c)) >= k) theta = c;
  }
  uint64_t m[MAXV];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    m[i] = __ballot(key[i] != 0u && key[i] >= theta);
    cnt += (int)__popcll(m[i]);
  }
  if (cnt > 64) {  // uniform
    topk_rounds<MAXV, false>(v, lane, t, E, k, renorm, 1, idx_out, w_out);
    return;
  }
  __shared__ uint32_t s_key[4][64];
  __shared__ int32_t s_idx[4][64];
  __shared__ float s_val[4][64];
  const int wv = threadIdx.x >> 6;
  int base = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    if ((m[i] >> lane) & 1ull) {
      const int pos = base + (int)__popcll(m[i] & ((1ull << lane) - 1ull));
      s_key[wv][pos] = key[i];
      s_idx[wv][pos] = i * 64 + lane;
      s_val[wv][pos] = v[i];
    }
    base += (int)__popcll(m[i]);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const bool cand = lane < cnt;
  const uint32_t ck = cand ? s_key[wv][lane] : 0u;
  const int ci = cand ? s_idx[wv][lane] : 0x7fffffff;
  const float cv = cand ? s_val[wv][lane] : 0.f;
  int rank = 0;
  for (int j = 0; j < cnt; ++j) {
    const uint32_t kj = __builtin_amdgcn_readlane(ck, j);
    const int ij = __builtin_amdgcn_readlane(ci, j);
    rank += (kj > ck || (kj == ck && ij < ci)) ? 1 : 0;
  }
  const bool sel = cand && rank < k;
  // the largest selected logit (slot 0)
  const uint64_t top = __ballot(cand && rank == 0);
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cv), (int)__builtin_ctzll(top)));
  float w;
  if (renorm) {
    const float ex = sel ? expf(cv - v0) : 0.f;
    w = ex / wave_sum(ex);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (i * 64 + lane < E) s += expf(v[i] - v0);
    s = wave_sum(s);
    w = expf(cv - v0) / s;
  }
  if (sel) {
    idx_out[(int64_t)t * k + rank] = ci;
    w_out[(int64_t)t * k + rank] = w;
  }
}

// dlogits for one token per wave.  renorm: dL_m = w_m (dw_m - <w, dw>) on the
// selected experts (local or not), 0 elsewhere.  raw softmax: dL_e = p_e (g_e -
// <w, dw>) with g_e = dw_j at e = idx_j.  The k selections are read once into
// scalar registers (their lane is uniform) and scattered into the row held
// by the lanes: expert e is element e/64 of lane e%64.
template <int MAXV>
__global__ void __launch_bounds__(256) route_bwd_kernel(const float* __restrict__ logits,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ dw, int T, int E, int k,
                                                        int renorm, float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_i = -1;
  float my_w = 0.f, my_dw = 0.f;
  if (lane < k) {
    my_i = idx[(int64_t)t * k + lane];
    my_w = w[(int64_t)t * k + lane];
    my_dw = dw[(int64_t)t * k + lane];
  }
  const float s = wave_sum(my_w * my_dw);
  // g[i]: for renorm w_j (dw_j - s) at the selected experts, else dw_j
  float g[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) g[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int ij = __builtin_amdgcn_readlane(my_i, j);
    const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
    const float dwj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_dw), j));
    const float val = renorm ? wj * (dwj - s) : dwj;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (ij == i * 64 + lane) g[i] = val;
  }
  float* out = dlogits + (int64_t)t * E;
  if (renorm) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int e = i * 64 + lane;
      if (e < E) out[e] = g[i];
    }
  } else {
    const float* row = logits + (int64_t)t * E;
    float v[MAXV];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int e = i * 64 + lane;
      v[i] = e < E ? row[e] : -INFINITY;
      mx = fmaxf(mx, v[i]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (i * 64 + lane < E) z += expf(v[i] - mx);
    z = wave_sum(z);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int e = i * 64 + lane;
      if (e < E) out[e] = expf(v[i] - mx) / z * (g[i] - s);
    }
  }
}

template <bool GROUPED>
static void route_dispatch(const moe_desc& d, const float* logits, int G, int32_t* idx, float* w, hipStream_t s) {
  const dim3 grid((d.T + 3) / 4), block(256);
  const int nv = (d.E + 63) / 64;
  if (nv <= 1) topk_route_kernel<1, GROUPED><<<grid, block, 0, s>>>(logits, d.T, d.E, d.k, d.renormalize, G, idx, w);
  else if (nv <= 2) topk_route_kernel<2, GROUPED><<<grid, block, 0, s>>>(logits, d.T, d.E, d.k, d.renormalize, G, idx, w);
  else if (nv <= 4) topk_route_kernel<4, GROUPED><<<grid, block, 0, s>>>(logits, d.T, d.E, d.k, d.renormalize, G, idx, w);
  else if (nv <= 8) topk_route_kernel<8, GROUPED><<<grid, block, 0, s>>>(logits, d.T, d.E, d.k, d.renormalize, G, idx, w);
  else topk_route_kernel<16, GROUPED><<<grid, block, 0, s>>>(logits, d.T, d.E, d.k, d.renormalize, G, idx, w);
}

hipError_t launch_route(const moe_desc& d, const float* logits, int n_groups, int32_t* idx, float* w,
                        hipStream_t s) {
  if (n_groups > 1) route_dispatch<true>(d, logits, n_groups, idx, w, s);
  else route_dispatch<false>(d, logits, 1, idx, w, s);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const moe_desc& d, const float* logits, const int32_t* idx, const float* w,
                            const float* dw, float* dlogits, hipStream_t s) {
  const dim3 grid((d.T + 3) / 4), block(256);
  const int nv = (d.E + 63) / 64;
  if (nv <= 1) route_bwd_kernel<1><<<grid, block, 0, s>>>(logits, idx, w, dw, d.T, d.E, d.k, d.renormalize, dlogits);
  else if (nv <= 2) route_bwd_kernel<2><<<grid, block, 0, s>>>(logits, idx, w, dw, d.T, d.E, d.k, d.renormalize, dlogits);
  else if (nv <= 4) route_bwd_kernel<4><<<grid, block, 0, s>>>(logits, idx, w, dw, d.T, d.E, d.k, d.renormalize, dlogits);
  else if (nv <= 8) route_bwd_kernel<8><<<grid, block, 0, s>>>(logits, idx, w, dw, d.T, d.E, d.k, d.renormalize, dlogits);
  else route_bwd_kernel<16><<<grid, block, 0, s>>>(logits, idx, w, dw, d.T, d.E, d.k, d.renormalize, dlogits);
  return hipGetLastError();
}

}  // namespace moe
