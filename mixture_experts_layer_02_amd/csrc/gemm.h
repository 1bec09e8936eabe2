// Grouped GEMM kernels of the expert MLP, its backward and the router.
//
// One template covers every matrix product of the layer:
//   C[m][n] = sum_k A(m, k) B(k, n)
// with A stored K-contiguous (A[m*lda + k]) or M-contiguous (A[k*lda + m]),
// B stored K-contiguous (B[n*ldb + k]) or N-contiguous (B[k*ldb + n]), and
// three kinds of grouping:
//   GRP_NONE  one plain product (router);
//   GRP_M     variable-M groups: group g owns rows [offsets[g], offsets[g+1])
//             of A and C and its own B (the expert segments of the Aurora
//             page's Grouped_mm with cum_token_counts boundaries);
//   GRP_K     variable-K groups: group g reduces over k in [offsets[g],
//             offsets[g+1]) and owns its own C (expert weight gradients),
//             or uniform K chunks when offsets is NULL (split-K).
// The tile loop is persistent: the grid is sized to the machine and each
// workgroup walks tile ids blockIdx.x, blockIdx.x + gridDim.x, ...; the tile
// count is computed on the device from offsets, so no host sync is needed.
// Within an expert, tiles are ordered m-tile fastest so that the workgroups
// running together share one expert's weights and rows in L2 / MALL.
#pragma once

#include "common.h"

namespace moe {

enum { LAY_K = 0, LAY_MN = 1 };
enum { GRP_NONE = 0, GRP_M = 1, GRP_K = 2 };
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2, EPI_ADD = 3 };  // EPI_ADD: C += product
// Gathered operand of the LDS-DMA kernel: GATH_A the K-contiguous A of a
// GRP_M product, GATH_B the MN-contiguous B of a GRP_K product, GATH_AK the
// MN-contiguous A of a GRP_K product.
enum { GATH_NONE = 0, GATH_A = 1, GATH_B = 2, GATH_AK = 3 };

constexpr int MAXG = 1024;

struct GemmParams {
  const void* A;
  int64_t lda;
  const void* B;
  const void* B2;       // DUAL: second B (same layout); ksplit: B for k >= ksplit
  int64_t ldb;
  int64_t b_gstride;    // elements between groups' B (GRP_M)
  int ksplit;           // 0 = off; else k >= ksplit reads B2 at k - ksplit
  void* C;
  void* C2;             // msplit: rows >= msplit go to C2 at row - msplit
  int64_t ldc;
  int64_t c_gstride;    // elements between groups' C (GRP_K)
  int msplit;
  const int32_t* offsets;
  int ngroups;
  int M, N, K;
  int kchunk;           // GRP_K with offsets == NULL: group g = [g*kchunk, (g+1)*kchunk) of K
  const float* bias;    // EPI_STORE: C += bias[n] (NULL = none)
  const void* gu_in;    // EPI_SWIGLU_BWD: [rows][2N], G | U
  void* gu_out;         // EPI_SWIGLU: [rows][2N], G | U (NULL = not saved)
  int c_f32;            // 1: C is float, 0: C is bf16
  int* dyn;             // dynamic tile queues (int[16], zero on entry and on exit), NULL = static order
  const int32_t* gather;  // gathered operand (see gemm_dma_kernel's GATH): row r of it is row gather[r]
  int gather_rows;        //   of the source matrix, which has gather_rows rows
  const float* bs;        // BQ8: float32 scale of each 128-value block of B's rows (B2's in bs2)
  const float* bs2;
  int band;               // GRP_K: m-tiles per band of the tile order (0 = m-tile fastest over all of M)
  const uint8_t* a_scale;  // F8: E8M0 scale bytes of A's rows ([rows][sbytes], one per 128 codes of k)
  const uint8_t* b_scale;  //     ... of B's rows (B2's in b2_scale), [groups * N][sbytes]
  const uint8_t* b2_scale;
  int sbytes;              //     scale bytes per row (K codes / 128, a multiple of 4)
  const float* row_scale; // EPI_SWIGLU_BWD with a gathered A: dH of row r is scaled by row_scale[r]
  void* h_out;            //   and, when set, row_scale[r] * silu(G) * U is written here ([rows][N])
  float* dw_part;         //   and, when set, row r's partial sums of dH * silu(G) * U (unscaled dH)
                          //   over each wave's 128 columns: [rows][2 * n-tiles], entry 2 n-tile + wn
};

struct TileCtx {
  int g;
  int64_t m0;   // first row of the tile in C's row space (GRP_M: global row)
  int mlim;     // valid rows in the tile
  int n0;
  int nlim;     // valid columns in the tile
  int64_t k0, k1;  // K range of the tile
  int mtile;    // m-tile index within the group (GRP_K: within M, or within its band)
  int mtiles;   // m-tiles of the group (or of the band)
  bool nfast;   // tiles ordered n-tile fastest (else m-tile fastest)
  int ntile;    // n-tile index
};

// ---------------------------------------------------------------------------
// Tile scheduling (shared by the MFMA and the FMA kernels).
// ---------------------------------------------------------------------------
template <int GRP, int BM, int BN>
struct Scheduler {
  int total;
  int NT, MT;

  // Must be called by all threads of the block.
  __device__ void init(const GemmParams& p, int* s_pref, int* s_scan) {
    NT = (p.N + BN - 1) / BN;
    if (GRP == GRP_M) {
      const int tid = threadIdx.x;
      const int G = p.ngroups;
      int loc[4];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = tid * 4 + i;
        int c = 0;
        if (g < G) {
          const int m = p.offsets[g + 1] - p.offsets[g];
          c = (m + BM - 1) / BM * NT;
        }
        loc[i] = c;
        sum += c;
      }
      s_scan[tid] = sum;
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        const int v = tid >= off ? s_scan[tid - off] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
      }
      int ex = s_scan[tid] - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = tid * 4 + i;
        if (g < G) s_pref[g] = ex;
        ex += loc[i];
      }
      if (tid == 0) s_pref[G] = s_scan[255];
      __syncthreads();
      total = s_pref[G];
      MT = 0;
    } else {
      MT = (p.M + BM - 1) / BM;
      total = MT * NT * (GRP == GRP_K ? p.ngroups : 1);
    }
  }

  // BANDED = false compiles the banded order out (the dynamic-order
  // kernels, whose scalar registers are already at their limit).
  template <bool BANDED = true>
  __device__ TileCtx tile(const GemmParams& p, const int* s_pref, int id) const {
    TileCtx t;
    if (GRP == GRP_M) {
      int lo = 0, hi = p.ngroups;  // s_pref[lo] <= id < s_pref[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= id) lo = mid; else hi = mid;
      }
      const int g = lo;
      const int r0 = p.offsets[g], r1 = p.offsets[g + 1];
      const int mt_g = (r1 - r0 + BM - 1) / BM;
      const int local = id - s_pref[g];
      const int mt = local % mt_g, nt = local / mt_g;
      t.nfast = false;
      t.g = g;
      t.mtile = mt;
      t.mtiles = mt_g;
      t.ntile = nt;
      t.m0 = (int64_t)r0 + (int64_t)mt * BM;
      t.mlim = min(BM, r1 - (int)t.m0);
      t.n0 = nt * BN;
      t.nlim = min(BN, p.N - t.n0);
      t.k0 = 0;
      t.k1 = p.K;
    } else {
      const int per = MT * NT;
      const int g = GRP == GRP_K ? id / per : 0;
      const int local = id - g * per;
      // One plain product with fewer n-tiles than m-tiles (the router's, N =
      // E): n-tile fastest, so that the tiles sharing an A row block run
      // together and A (T x d) streams from memory once, not once per n-tile.
      const bool nf = GRP == GRP_NONE && MT >= NT;
      int mt = nf ? local / NT : local % MT, nt = nf ? local % NT : local / MT;
      // With two n-tiles (the second often narrower: E = 384 is 256 + 128)
      // a workgroup would take the same n-tile in every round of the static
      // order; swapping them in odd rounds gives each one both in turn.  (A
      // tile pair 2m, 2m + 1 lies in one round when the grid is even, so the
      // swap maps the round's tiles onto themselves.)
      if (GRP == GRP_NONE && BANDED && nf && NT == 2 && !(gridDim.x & 1u) && ((id / (int)gridDim.x) & 1)) nt ^= 1;
      t.mtile = mt;
      t.mtiles = MT;
      if (GRP == GRP_K && BANDED && p.band > 0 && p.band < MT) {
        // Banded order: bands of `band` m-tiles, m-tile fastest inside a band,
        // so that the consecutive tiles an XCD runs together form a block of
        // about band x (run / band) tiles, whose A and B k-slices they share,
        // instead of a column of all M.  (The last band may be shorter.)
        const int G = p.band;
        const int b = local / (G * NT);
        const int bm = min(G, MT - b * G);
        const int in = local - b * G * NT;
        mt = b * G + in % bm;
        nt = in / bm;
        t.mtile = in % bm;  // the sharers of a B k-slice are the band's m-tiles
        t.mtiles = bm;
      }
      t.nfast = nf;
      t.g = g;
      t.ntile = nt;
      t.m0 = (int64_t)mt * BM;
      t.mlim = min(BM, p.M - (int)t.m0);
      t.n0 = nt * BN;
      t.nlim = min(BN, p.N - t.n0);
      if (GRP == GRP_K) {
        if (p.offsets) {
          t.k0 = p.offsets[g];
          t.k1 = p.offsets[g + 1];
        } else {
          t.k0 = (int64_t)g * p.kchunk;
          t.k1 = max(t.k0, min((int64_t)p.K, t.k0 + p.kchunk));  // chunks past K are empty
        }
      } else {
        t.k0 = 0;
        t.k1 = p.K;
      }
    }
    return t;
  }
};

// ---------------------------------------------------------------------------
// Epilogue: one output element (and its DUAL partner) of a tile.
// r, c are tile-local; the caller has checked r < mlim, c < nlim.
// ---------------------------------------------------------------------------
template <int GRP, int EPI>
__device__ __forceinline__ void epi_store(const GemmParams& p, const TileCtx& t, int r, int c,
                                          float v, float v2) {
  const int64_t row = t.m0 + r;
  const int64_t col = (int64_t)t.n0 + c;
  if (EPI == EPI_STORE || EPI == EPI_ADD) {
    if (p.bias) v += p.bias[col];
    int64_t crow = row;
    void* Cb = p.C;
    if (p.msplit && row >= p.msplit) {
      crow = row - p.msplit;
      Cb = p.C2;
    }
    int64_t off = crow * p.ldc + col;
    if (GRP == GRP_K) off += (int64_t)t.g * p.c_gstride;
    if (EPI == EPI_ADD) v += p.c_f32 ? reinterpret_cast<const float*>(Cb)[off] : bf2f(reinterpret_cast<const uint16_t*>(Cb)[off]);
    if (p.c_f32) reinterpret_cast<float*>(Cb)[off] = v;
    else reinterpret_cast<uint16_t*>(Cb)[off] = f2bf(v);
  } else if (EPI == EPI_SWIGLU) {
    // v = gate (G), v2 = up (U); h = silu(G) * U
    const float h = v / (1.0f + __expf(-v)) * v2;
    if (p.c_f32) {
      reinterpret_cast<float*>(p.C)[row * p.ldc + col] = h;
      if (p.gu_out) {
        float* gu = reinterpret_cast<float*>(p.gu_out) + row * (2 * (int64_t)p.N);
        gu[col] = v;
        gu[p.N + col] = v2;
      }
    } else {
      reinterpret_cast<uint16_t*>(p.C)[row * p.ldc + col] = f2bf(h);
      if (p.gu_out) {
        uint16_t* gu = reinterpret_cast<uint16_t*>(p.gu_out) + row * (2 * (int64_t)p.N);
        gu[col] = f2bf(v);
        gu[p.N + col] = f2bf(v2);
      }
    }
  } else {  // EPI_SWIGLU_BWD: v = dH; C = dgu [rows][2N]
    float g, u;
    const int64_t gi = row * (2 * (int64_t)p.N) + col;
    if (p.c_f32) {
      g = reinterpret_cast<const float*>(p.gu_in)[gi];
      u = reinterpret_cast<const float*>(p.gu_in)[gi + p.N];
    } else {
      g = bf2f(reinterpret_cast<const uint16_t*>(p.gu_in)[gi]);
      u = bf2f(reinterpret_cast<const uint16_t*>(p.gu_in)[gi + p.N]);
    }
    const float s = sigmoidf_(g);
    const float du = v * g * s;
    const float dg = v * u * s * (1.0f + g * (1.0f - s));
    if (p.c_f32) {
      reinterpret_cast<float*>(p.C)[gi] = dg;
      reinterpret_cast<float*>(p.C)[gi + p.N] = du;
    } else {
      reinterpret_cast<uint16_t*>(p.C)[gi] = f2bf(dg);
      reinterpret_cast<uint16_t*>(p.C)[gi + p.N] = f2bf(du);
    }
  }
}

// Epilogue for 8 consecutive columns c .. c+7 of tile-local row r (the caller
// has checked r < mlim and c < nlim; N is a multiple of 8, so the whole
// vector is in range).  v / v2 hold the accumulators (v2: the DUAL partner).
template <int GRP, int EPI>
__device__ __forceinline__ void epi_store8(const GemmParams& p, const TileCtx& t, int r, int c,
                                           const float (&v)[8], const float (&v2)[8]) {
  const int64_t row = t.m0 + r;
  const int64_t col = (int64_t)t.n0 + c;
  if (EPI == EPI_STORE || EPI == EPI_ADD) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = v[e];
    if (p.bias) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += p.bias[col + e];
    }
    int64_t crow = row;
    void* Cb = p.C;
    if (p.msplit && row >= p.msplit) {
      crow = row - p.msplit;
      Cb = p.C2;
    }
    int64_t off = crow * p.ldc + col;
    if (GRP == GRP_K) off += (int64_t)t.g * p.c_gstride;
    if (EPI == EPI_ADD) {
      float old[8];
      if (p.c_f32) {
        Vec16<float>::load(reinterpret_cast<const float*>(Cb) + off, *reinterpret_cast<float(*)[4]>(&old[0]));
        Vec16<float>::load(reinterpret_cast<const float*>(Cb) + off + 4, *reinterpret_cast<float(*)[4]>(&old[4]));
      } else {
        Vec16<uint16_t>::load(reinterpret_cast<const uint16_t*>(Cb) + off, old);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += old[e];
    }
    if (p.c_f32) {
      float* d = reinterpret_cast<float*>(Cb) + off;
      *reinterpret_cast<f32x4*>(d) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(d + 4) = f32x4{o[4], o[5], o[6], o[7]};
    } else {
      Vec16<uint16_t>::store(reinterpret_cast<uint16_t*>(Cb) + off, o);
    }
  } else if (EPI == EPI_SWIGLU) {
    float h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = v[e] * sigmoidf_(v[e]) * v2[e];
    Vec16<uint16_t>::store(reinterpret_cast<uint16_t*>(p.C) + row * p.ldc + col, h);
    if (p.gu_out) {
      uint16_t* gu = reinterpret_cast<uint16_t*>(p.gu_out) + row * (2 * (int64_t)p.N);
      Vec16<uint16_t>::store(gu + col, v);
      Vec16<uint16_t>::store(gu + p.N + col, v2);
    }
  } else {  // EPI_SWIGLU_BWD
    const int64_t gi = row * (2 * (int64_t)p.N) + col;
    const uint16_t* gu = reinterpret_cast<const uint16_t*>(p.gu_in);
    float g[8], u[8], dg[8], du[8];
    Vec16<uint16_t>::load(gu + gi, g);
    Vec16<uint16_t>::load(gu + gi + p.N, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float s = sigmoidf_(g[e]);
      du[e] = v[e] * g[e] * s;
      dg[e] = v[e] * u[e] * s * (1.0f + g[e] * (1.0f - s));
    }
    uint16_t* out = reinterpret_cast<uint16_t*>(p.C);
    Vec16<uint16_t>::store(out + gi, dg);
    Vec16<uint16_t>::store(out + gi + p.N, du);
  }
}

// Plain float store of 4 columns (EPI_STORE with a float C).
template <int GRP>
__device__ __forceinline__ void epi_store4f(const GemmParams& p, const TileCtx& t, int r, int c,
                                            const float (&v)[4]) {
  const int64_t row = t.m0 + r;
  const int64_t col = (int64_t)t.n0 + c;
  f32x4 o = {v[0], v[1], v[2], v[3]};
  if (p.bias) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += p.bias[col + e];
  }
  int64_t crow = row;
  void* Cb = p.C;
  if (p.msplit && row >= p.msplit) {
    crow = row - p.msplit;
    Cb = p.C2;
  }
  int64_t off = crow * p.ldc + col;
  if (GRP == GRP_K) off += (int64_t)t.g * p.c_gstride;
  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Cb) + off) = o;
}

// Pointer to operand element (mn, k) for the current k-tile, honouring the
// group offset, the K split and the layout.  Returns the base such that
// element (mn_local, k_local) of the tile is base[mn_local*smn + k_local*sk].
template <typename T>
struct OpView {
  const T* base;
  int64_t smn, sk;
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  Block tile BM x BN (256 x 256 or 128 x 128), BK = 64,
// 4 waves in 2 x 2, each wave a (BM/2) x (BN/2) sub-tile of
// v_mfma_f32_32x32x16_bf16 blocks (4 x 4 of them at 256 x 256, with the 256
// float accumulators held in AccVGPRs).  Operand tiles are double buffered in
// LDS in the layout they have in HBM, so every global load and LDS store is a
// 16-byte vector:
//   K-contiguous operand   -> LDS [mn][k], row pitch BK + 8; a fragment is one
//                              ds_read_b128 (8 consecutive k of one row);
//   M/N-contiguous operand -> LDS [k][mn], row pitch MN + 32; a fragment is two
//                              ds_read_b64_tr_b16, the gfx950 transposing LDS
//                              read: within each 16-lane group, lane i receives
//                              element i%4 of the 8-byte chunk addressed by lane
//                              i/4 + 4j (j = 0..3), so 16 lanes pointing at a
//                              4 x 16 block of [k][mn] get one mn column each,
//                              four consecutive k deep.
// Both pitches keep the fragment reads free of bank conflicts.
// DUAL: the B tile's first BN/2 rows are columns n0.. of B and the last BN/2
// the same columns of B2; n-block ni of a wave pairs with ni + NI/2.
// ---------------------------------------------------------------------------
namespace mf {
constexpr int BK = 64, THREADS = 256;
template <int ROWS> struct Lds {
  static constexpr int KPITCH = BK + 8;        // K-contiguous: [ROWS][KPITCH]
  static constexpr int MNPITCH = ROWS + 32;    // MN-contiguous: [BK][MNPITCH]
  static constexpr int ELEMS = (ROWS * KPITCH > BK * MNPITCH) ? ROWS * KPITCH : BK * MNPITCH;
};
}  // namespace mf

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int LAY, typename ST, int ROWS>
struct MfLoader {
  static constexpr int NV = ROWS * mf::BK / 8 / mf::THREADS;  // 16-byte vectors per thread
  u32x4 v[NV];

  // Vector i of this thread: K-contig (mn, k) = (tid/8 + 32 i, (tid%8)*8);
  // MN-contig (k, mn) = (tid/(ROWS/8) + (THREADS/(ROWS/8)) i, (tid%(ROWS/8))*8).
  __device__ __forceinline__ void coords(int i, int& mn, int& k) const {
    const int tid = threadIdx.x;
    if (LAY == LAY_K) {
      mn = tid / 8 + 32 * i;
      k = (tid % 8) * 8;
    } else {
      constexpr int VPR = ROWS / 8;  // vectors per k row
      k = tid / VPR + (mf::THREADS / VPR) * i;
      mn = (tid % VPR) * 8;
    }
  }

  int klim_;

  // Element (mn, k) of the tile lives at K-contig base[mn*ld + k], MN-contig
  // base[k*ld + mn]; with dual, rows mn >= ROWS/2 come from base2 at mn - ROWS/2.
  // Vectors outside the tile's M/N range read a clamped in-range address: they
  // only feed output rows/columns that the epilogue never stores.  Vectors past
  // the tile's K extent are zeroed by store(), so the loads are branch-free and
  // nothing waits on them before the LDS store.
  __device__ __forceinline__ void load(const ST* base, const ST* base2, int64_t ld, int mnlim, int klim,
                                       bool dual) {
    klim_ = klim;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int mn, k;
      coords(i, mn, k);
      // K-contig rows of vector i are tid/8 + 32 i < 32 (i + 1): the DUAL half
      // is known at compile time from i.
      const bool second = (LAY == LAY_K) && dual && (32 * i >= ROWS / 2);
      const ST* b = second ? base2 : base;
      const int mn_eff = second ? mn - ROWS / 2 : mn;
      const int lim = dual ? min(mnlim, ROWS / 2) : mnlim;
      const int mc = mn_eff < lim ? mn_eff : 0, kc = k < klim ? k : 0;
      const ST* ptr = (LAY == LAY_K) ? b + (int64_t)mc * ld + kc : b + (int64_t)kc * ld + mc;
      if constexpr (sizeof(ST) == 2) {
        v[i] = *reinterpret_cast<const u32x4*>(ptr);
      } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(ptr);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(ptr + 4);
        v[i] = u32x4{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]),
                     pack_bf2(hi[2], hi[3])};
      }
    }
  }

  // Zero the vectors past the K extent (only a partial k-tile has any).
  __device__ __forceinline__ void zero_k_tail() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int mn, k;
      coords(i, mn, k);
      if (k >= klim_) v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  __device__ __forceinline__ void store(uint16_t* S) {
    if (__builtin_expect(klim_ < mf::BK, 0)) zero_k_tail();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int mn, k;
      coords(i, mn, k);
      if (LAY == LAY_K) *reinterpret_cast<u32x4*>(S + mn * mf::Lds<ROWS>::KPITCH + k) = v[i];
      else *reinterpret_cast<u32x4*>(S + k * mf::Lds<ROWS>::MNPITCH + mn) = v[i];
    }
  }
};

// MFMA fragment: 8 consecutive k (kk*16 + (lane/32)*8 ..) of row/column
// `row0 + lane%32` of an operand tile in LDS.
template <int LAY, int ROWS>
__device__ __forceinline__ bf16x8 mf_frag(const uint16_t* S, int row0, int kk, int lane) {
  if (LAY == LAY_K) {
    return *reinterpret_cast<const bf16x8*>(S + (row0 + (lane & 31)) * mf::Lds<ROWS>::KPITCH + kk * 16 +
                                            (lane >> 5) * 8);
  } else {
    constexpr int P = mf::Lds<ROWS>::MNPITCH;
    const int krow = kk * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);
    const int col = row0 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(S + krow * P + col));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(S + (krow + 4) * P + col));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  }
}

// Persistent tile ids are remapped so that the workgroups of one XCD (blocks
// b with the same b % 8 are dispatched to the same XCD) take a contiguous run
// of logical tiles: neighbouring tiles share operand tiles in that XCD's L2.
__device__ __forceinline__ int xcd_tile(int it, int grid) {
  const int b = blockIdx.x;
  if (grid % 8) return it * grid + b;
  return it * grid + (b % 8) * (grid / 8) + b / 8;
}

template <int BM, int BN, int ALAY, int BLAY, typename AT, int GRP, int EPI, bool DUAL>
__global__ void __launch_bounds__(256, (BM * BN > 128 * 128) ? 1 : 2) gemm_mfma_kernel(GemmParams p) {
  using namespace mf;
  static_assert(!DUAL || BLAY == LAY_K, "dual B is K-contiguous");
  constexpr int MI = BM / 64, NI = BN / 64;   // 32 x 32 blocks per wave
  constexpr int AE = Lds<BM>::ELEMS, BE = Lds<BN>::ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][AE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BE];
  __shared__ int s_pref[MAXG + 1];
  __shared__ int s_scan[256];

  Scheduler<GRP, BM, DUAL ? BN / 2 : BN> sched;
  sched.init(p, s_pref, s_scan);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const AT* Ag = reinterpret_cast<const AT*>(p.A);
  const uint16_t* Bg = reinterpret_cast<const uint16_t*>(p.B);
  const uint16_t* B2g = reinterpret_cast<const uint16_t*>(p.B2);

  for (int it = 0;; ++it) {
    const int id = xcd_tile(it, gridDim.x);
    if (it * (int)gridDim.x >= sched.total) break;
    if (id >= sched.total) continue;
    const TileCtx t = sched.tile(p, s_pref, id);
    const int64_t klen = t.k1 - t.k0;
    const int nk = (int)((klen + BK - 1) / BK);

    const AT* a_base = (ALAY == LAY_K) ? Ag + t.m0 * p.lda + t.k0 : Ag + t.k0 * p.lda + t.m0;
    const uint16_t* b_grp = Bg;
    const uint16_t* b2_grp = B2g;
    if (GRP == GRP_M) {
      b_grp += (int64_t)t.g * p.b_gstride;
      if (B2g) b2_grp += (int64_t)t.g * p.b_gstride;
    }

    MfLoader<ALAY, AT, BM> la;
    MfLoader<BLAY, uint16_t, BN> lb;

    auto b_ptrs = [&](int kt, const uint16_t*& b1, const uint16_t*& b2) {
      const int64_t kg = t.k0 + (int64_t)kt * BK;
      if (BLAY == LAY_K) {
        b1 = b_grp + (int64_t)t.n0 * p.ldb + kg;
        b2 = DUAL ? b2_grp + (int64_t)t.n0 * p.ldb + kg : nullptr;
      } else {
        if (p.ksplit && kg >= p.ksplit) b1 = b2_grp + (kg - p.ksplit) * p.ldb + t.n0;
        else b1 = b_grp + kg * p.ldb + t.n0;
        b2 = nullptr;
      }
    };
    auto a_ptr = [&](int kt) -> const AT* {
      const int64_t ko = (int64_t)kt * BK;
      return ALAY == LAY_K ? a_base + ko : a_base + ko * p.lda;
    };
    auto klim_of = [&](int kt) -> int { return (int)min((int64_t)BK, klen - (int64_t)kt * BK); };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
      const uint16_t *b1, *b2;
      b_ptrs(0, b1, b2);
      la.load(a_ptr(0), nullptr, p.lda, t.mlim, klim_of(0), false);
      lb.load(b1, b2, p.ldb, t.nlim, klim_of(0), DUAL);
      la.store(As[0]);
      lb.store(Bs[0]);
      __syncthreads();
    }
    // Main loop.  Global loads of k-tile kt+1 are issued first; the MFMA
    // fragments of k-step kk+1 are read from LDS while the 16 MFMAs of step kk
    // run; the staged k-tile kt+1 is written to the other LDS buffer inside
    // the last k-step, as late as possible after its loads were issued.
    auto read_frags = [&](const uint16_t* as, const uint16_t* bs, int kk, bf16x8 (&af)[MI], bf16x8 (&bfr)[NI]) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) af[mi] = mf_frag<ALAY, BM>(as, wm * (BM / 2) + mi * 32, kk, lane);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int brow = DUAL ? (ni / (NI / 2)) * (BN / 2) + wn * (BN / 4) + (ni % (NI / 2)) * 32
                              : wn * (BN / 2) + ni * 32;
        bfr[ni] = mf_frag<BLAY, BN>(bs, brow, kk, lane);
      }
    };
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        const uint16_t *b1, *b2;
        b_ptrs(kt + 1, b1, b2);
        la.load(a_ptr(kt + 1), nullptr, p.lda, t.mlim, klim_of(kt + 1), false);
        lb.load(b1, b2, p.ldb, t.nlim, klim_of(kt + 1), DUAL);
      }
      const uint16_t* as = As[cur];
      const uint16_t* bs = Bs[cur];
      bf16x8 af[2][MI], bfr[2][NI];
      read_frags(as, bs, 0, af[0], bfr[0]);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        if (kk + 1 < BK / 16) read_frags(as, bs, kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
        if (kk == BK / 16 - 1 && more) {
          la.store(As[cur ^ 1]);
          lb.store(Bs[cur ^ 1]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead above this step's MFMAs
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][mi], bfr[kk & 1][ni], acc[mi][ni], 0, 0, 0);
      }
      __syncthreads();
    }

    // Epilogue, staged through LDS (free after the last barrier of the k loop)
    // one 32-row block at a time: acc[mi][ni][r] is C[row][col] with
    //   row = wm*BM/2 + mi*32 + (r/4)*8 + (lane/32)*4 + r%4,
    //   col = n-block base + lane%32,
    // written to the wave's [32][WC] float staging area, then read back as
    // 8-column vectors for the vectorized epilogue.
    {
      constexpr int WC = NI * 32;        // staged columns per wave
      constexpr int SP = WC + 4;         // staging pitch (floats)
      float* stage = reinterpret_cast<float*>(&As[0][0]) + wave * 32 * SP;
      static_assert(4 * 32 * SP * 4 <= (int)sizeof(As), "staging fits in the A buffers");
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            stage[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * SP + ni * 32 + (lane & 31)] = acc[mi][ni][r];
        __syncthreads();
        constexpr int OC = DUAL ? WC / 2 : WC;   // output columns per wave
        constexpr int CPR = OC / 8;              // 8-column vectors per row
        for (int e = lane; e < 32 * CPR; e += 64) {
          const int rl = e / CPR, cv = (e % CPR) * 8;
          const int row = wm * (BM / 2) + mi * 32 + rl;
          const int col = (DUAL ? wn * (BN / 4) : wn * (BN / 2)) + cv;
          if (row < t.mlim && col < t.nlim) {
            float v[8], v2[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              v[q] = stage[rl * SP + cv + q];
              v2[q] = DUAL ? stage[rl * SP + OC + cv + q] : 0.f;
            }
            epi_store8<GRP, EPI>(p, t, row, col, v, v2);
          }
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 FMA kernel (the fp32 path): 64 x 64 tile, BK = 16, 256 threads with
// a 4 x 4 micro-tile each.  LDS holds both operands as [k][mn] rows.
// DUAL: the tile is 64 rows x 64 columns of B and the same columns of B2.
// ---------------------------------------------------------------------------
namespace ff {
constexpr int BM = 64, BN = 64, BK = 16, LDM = 64 + 4;
}

template <int LAY>
__device__ __forceinline__ void ff_load(float* S, const float* base, int64_t ld, int mnlim, int klim) {
  using namespace ff;
  const int tid = threadIdx.x;
  if (LAY == LAY_K) {
    const int mn = tid / 4, k = (tid % 4) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = mn < mnlim && k + e < klim;
      S[(k + e) * LDM + mn] = ok ? base[(int64_t)mn * ld + k + e] : 0.f;
    }
  } else {
    const int k = tid / 16, mn = (tid % 16) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = k < klim && mn + e < mnlim;
      S[k * LDM + mn + e] = ok ? base[(int64_t)k * ld + mn + e] : 0.f;
    }
  }
}

template <int ALAY, int BLAY, int GRP, int EPI, bool DUAL>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmParams p) {
  using namespace ff;
  __shared__ float As[BK * LDM];
  __shared__ float Bs[BK * LDM];
  __shared__ float B2s[DUAL ? BK * LDM : 1];
  __shared__ int s_pref[MAXG + 1];
  __shared__ int s_scan[256];

  Scheduler<GRP, BM, BN> sched;
  sched.init(p, s_pref, s_scan);
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const float* Ag = reinterpret_cast<const float*>(p.A);
  const float* Bg = reinterpret_cast<const float*>(p.B);
  const float* B2g = reinterpret_cast<const float*>(p.B2);

  for (int id = blockIdx.x; id < sched.total; id += gridDim.x) {
    const TileCtx t = sched.tile(p, s_pref, id);
    const int64_t klen = t.k1 - t.k0;
    float acc[4][4] = {}, acc2[4][4] = {};
    const float* b_grp = Bg;
    const float* b2_grp = B2g;
    if (GRP == GRP_M) {
      b_grp += (int64_t)t.g * p.b_gstride;
      if (B2g) b2_grp += (int64_t)t.g * p.b_gstride;
    }
    for (int64_t ko = 0; ko < klen; ko += BK) {
      const int klim = (int)min((int64_t)BK, klen - ko);
      const int64_t kg = t.k0 + ko;
      const float* a = ALAY == LAY_K ? Ag + t.m0 * p.lda + kg : Ag + kg * p.lda + t.m0;
      const float* b;
      const float* b2 = nullptr;
      if (BLAY == LAY_K) {
        b = b_grp + (int64_t)t.n0 * p.ldb + kg;
        if (DUAL) b2 = b2_grp + (int64_t)t.n0 * p.ldb + kg;
      } else {
        if (p.ksplit && kg >= p.ksplit) b = b2_grp + (kg - p.ksplit) * p.ldb + t.n0;
        else b = b_grp + kg * p.ldb + t.n0;
      }
      ff_load<ALAY>(As, a, p.lda, t.mlim, klim);
      ff_load<BLAY>(Bs, b, p.ldb, t.nlim, klim);
      if (DUAL) ff_load<BLAY>(B2s, b2, p.ldb, t.nlim, klim);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a4[4], b4[4], c4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a4[i] = As[kk * LDM + ty * 4 + i];
          b4[i] = Bs[kk * LDM + tx * 4 + i];
          if (DUAL) c4[i] = B2s[kk * LDM + tx * 4 + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[i][j] = fmaf(a4[i], b4[j], acc[i][j]);
            if (DUAL) acc2[i][j] = fmaf(a4[i], c4[j], acc2[i][j]);
          }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = ty * 4 + i, col = tx * 4 + j;
        if (row < t.mlim && col < t.nlim) epi_store<GRP, EPI>(p, t, row, col, acc[i][j], acc2[i][j]);
      }
  }
}

}  // namespace moe
