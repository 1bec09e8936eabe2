// Grouped GEMM with direct global->LDS loads (gfx950 global_load_lds_dwordx4).
//
// Same products, grouping modes, tile order and epilogues as gemm_mfma_kernel
// (gemm.h), but the operand tiles reach LDS through the gfx950 LDS DMA path:
// each wave instruction moves 64 x 16 bytes from HBM/L2 straight into 1 KB of
// contiguous LDS, without passing through VGPRs.  The k-slice width BK and
// the number of ring stages NST are template parameters (BK = 64 with 2
// stages is the 128 KB LDS ring used by default; BK = 32 with 4 stages keeps
// more, smaller k-tiles in flight).
//
// LDS layouts (no padding: a DMA instruction writes 1 KB contiguously, so bank
// conflicts are avoided by XOR-swizzling 16-byte chunks instead):
//   K-contiguous tile  [256 rows][BK k]: a row is BK/8 chunks; chunk c of
//     row r sits at position c ^ swz_k(r).  A fragment (8 k of one row) is
//     one ds_read_b128.
//   MN-contiguous tile [BK k][256 mn]: a k-row is 32 chunks; chunk c of
//     k-row r sits at position c ^ swz_mn(r).  A fragment is two
//     ds_read_b64_tr_b16.
// Both swizzles make the fragment reads of a wave conflict-free whether the
// LDS has 32 or 64 banks.
#pragma once

#include <type_traits>

#include "gemm.h"

namespace moe {

namespace dma {
constexpr int BM = 256, BN = 256;

// K-contiguous: row r's chunk position XOR.  The 16 (64 banks) or 8 (32
// banks) consecutive rows read by one LDS cycle land on distinct bank groups.
template <int BK>
__device__ __forceinline__ int swz_k(int r) {
  if (BK == 32) return ((r >> 1) ^ (r >> 3)) & 3;
  return (r ^ (r >> 3)) & 7;
}
// MN-contiguous: k-row r's chunk XOR, one of {0, 6, 12, 10} by r % 4, so the
// 4 k-rows x 2..4 chunks read by one LDS cycle use distinct banks.
__device__ __forceinline__ int swz_mn(int r) { return (0xAC60 >> ((r & 3) * 4)) & 0xF; }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero (range-checked per dword), which handles every tile edge: rows past a
// segment, k-rows past a variable-K group, and the last rows of a buffer.
// Word 3 is the gfx9 raw-buffer format word (32-bit data, no swizzle).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(bytes > 0xFFFFFFFFull ? 0xFFFFFFFFull : bytes));
  r[3] = 0x00020000;
  return r;
}

// One LDS-DMA instruction: lane i copies the 16 bytes at rsrc + voff + soff to
// LDS byte address lds_dst + 16 i.  Issued through inline asm so that the
// compiler neither waits for it before unrelated LDS reads nor before
// barriers: the kernel waits for it explicitly (wait_vm) where a ring stage
// is consumed.  M0 (the LDS base of the copy) is saved and restored around it.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint16_t* lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      // Wait states: one for the LDS DMA reading M0 after its SALU write, five
      // for a buffer instruction reading SGPRs a VALU op (readfirstlane,
      // readlane) may have written just before this block.
      "s_nop 3\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// L2 prefetch: lane i reads the 4 bytes at rsrc + voff + soff into the LDS
// word lds_junk + 4 i (a scratch area nobody reads).  Its only purpose is to
// start the L2 fill of that 64-byte sector well before the tile DMA needs
// it; an offset outside the resource reads nothing.
__device__ __forceinline__ void touch4(i32x4 rsrc, uint32_t voff, uint32_t soff, const uint32_t* lds_junk) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_junk);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 3\n\t"  // as in dma16
      "buffer_load_dword %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// Workgroup barrier for LDS hand-offs: this wave's LDS reads and writes are
// complete (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it does not
// wait for outstanding global memory operations (the DMA ring in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 256 x BK operand tile is BK/2 DMA instructions of 1 KB; wave w issues
// instructions j = w*BK/8 .. (w+1)*BK/8 - 1.  Per-lane byte offsets (fixed for
// the whole output tile; the k-tile advance goes in the scalar offset):
//   K-contig : j covers rows RPI*j .. RPI*j+RPI-1 (RPI = 512/BK rows of BK/8
//              chunks); lane i -> row RPI*j + i/(BK/8), LDS position i%(BK/8)
//              holding global chunk (i%(BK/8)) ^ swz_k(row); element (mn, k)
//              at base[mn * ld + k].  With dual, rows >= 128 are rows
//              row - 128 of the second resource.
//   MN-contig: j covers k-rows 2j, 2j+1; lane i -> k-row 2j + i/32, position
//              i%32 holding chunk (i%32) ^ swz_mn(krow); element (mn, k) at
//              base[k * ld + mn].
template <int BK, int LAY, bool DUAL_ROWS>
__device__ __forceinline__ uint32_t dma_voff(int j, int lane, int64_t ld) {
  if (LAY == LAY_K) {
    constexpr int CPR = BK / 8, RPI = 64 / CPR;  // chunks per row, rows per instruction
    const int row = RPI * j + lane / CPR;
    const int c = (lane % CPR) ^ swz_k<BK>(row);  // the swizzle follows the LDS row
    const int src_row = DUAL_ROWS ? (row & 127) : row;
    return (uint32_t)(src_row * ld * 2 + c * 16);
  } else {
    const int krow = 2 * j + (lane >> 5);
    const int c = (lane & 31) ^ swz_mn(krow);
    return (uint32_t)(krow * ld * 2 + c * 16);
  }
}

// MFMA fragment: k = kk*16 + (lane/32)*8 + 0..7 of row/column row0 + lane%32.
template <int BK, int LAY>
__device__ __forceinline__ bf16x8 frag(const uint16_t* S, int row0, int kk, int lane) {
  if (LAY == LAY_K) {
    const int r = row0 + (lane & 31);
    const int p = (2 * kk + (lane >> 5)) ^ swz_k<BK>(r);
    return *reinterpret_cast<const bf16x8*>(S + r * BK + p * 8);
  } else {
    const int krow = kk * 16 + (lane >> 5) * 8 + ((lane & 15) >> 2);
    const int col = row0 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
    const int p = (col >> 3) ^ swz_mn(krow);  // krow and krow + 4 share the swizzle
    const int off = p * 8 + (col & 7);
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(S + krow * 256 + off));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(S + (krow + 4) * 256 + off));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
  }
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most `later` stages of PER instructions each are outstanding.
template <int PER, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
  if (MAXL >= 3 && later >= 3) wait_vm<(MAXL >= 3 ? 3 * PER : 0)>();
  else if (MAXL >= 2 && later >= 2) wait_vm<(MAXL >= 2 ? 2 * PER : 0)>();
  else if (MAXL >= 1 && later >= 1) wait_vm<PER>();
  else wait_vm<0>();
}
}  // namespace dma

// Requirements (checked by the host before choosing this kernel): bf16
// operands, K-contiguous operands have K (or every k-tile) a multiple of 32.
template <int BK, int STAGES, int ALAY, int BLAY, int GRP, int EPI, bool DUAL>
__global__ void __launch_bounds__(256, 1) gemm_dma_kernel(GemmParams p) {
  using namespace dma;
  static_assert(!DUAL || BLAY == LAY_K, "dual B is K-contiguous");
  static_assert((BK == 32 && STAGES == 4) || (BK == 64 && STAGES == 2), "ring shapes of 128 KB");
  constexpr int MI = 4, NI = 4;          // 32 x 32 blocks per wave (128 x 128)
  constexpr int TILE_ELEMS = 256 * BK;   // one operand tile
  constexpr int STAGE_ELEMS = 2 * TILE_ELEMS;
  constexpr int NJ = BK / 8;             // DMA instructions per wave per operand tile
  constexpr int KS = BK / 16;            // MFMA k-steps per k-tile
  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES][STAGE_ELEMS];
  __shared__ int s_pref[MAXG + 1];
  __shared__ int s_scan[256];
  __shared__ __attribute__((aligned(256))) uint32_t lds_junk[64];

  Scheduler<GRP, BM, DUAL ? BN / 2 : BN> sched;
  sched.init(p, s_pref, s_scan);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps DMA operands scalar
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* Ag = reinterpret_cast<const uint16_t*>(p.A);
  const uint16_t* Bg = reinterpret_cast<const uint16_t*>(p.B);
  const uint16_t* B2g = reinterpret_cast<const uint16_t*>(p.B2);

  for (int it = 0;; ++it) {
    const int id = xcd_tile(it, gridDim.x);
    if (it * (int)gridDim.x >= sched.total) break;
    if (id >= sched.total) continue;
    const TileCtx t = sched.tile(p, s_pref, id);
    const int64_t klen = t.k1 - t.k0;
    const int nk = (int)((klen + BK - 1) / BK);

    const uint16_t* a_base = (ALAY == LAY_K) ? Ag + t.m0 * p.lda + t.k0 : Ag + t.k0 * p.lda + t.m0;
    const uint16_t* b_grp = Bg;
    const uint16_t* b2_grp = B2g;
    if (GRP == GRP_M) {
      b_grp += (int64_t)t.g * p.b_gstride;
      if (B2g) b2_grp += (int64_t)t.g * p.b_gstride;
    }
    // Buffer resources of this output tile.  K-contig: rows [0, lim) of the
    // tile's row block; MN-contig: k-rows [0, klen) from column m0/n0 (the
    // range ends with row k1-1, so it never runs past the allocation).
    const int nlim_b = DUAL ? min(t.nlim, BN / 2) : t.nlim;
    const i32x4 ra = (ALAY == LAY_K) ? make_rsrc(a_base, (uint64_t)t.mlim * p.lda * 2)
                                     : make_rsrc(a_base, (uint64_t)(klen * p.lda - t.m0) * 2);
    i32x4 rb, rb2;
    if (BLAY == LAY_K) {
      rb = make_rsrc(b_grp + (int64_t)t.n0 * p.ldb, (uint64_t)nlim_b * p.ldb * 2);
      rb2 = DUAL ? make_rsrc(b2_grp + (int64_t)t.n0 * p.ldb, (uint64_t)nlim_b * p.ldb * 2) : rb;
    } else if (p.ksplit) {  // k < ksplit from B, k >= ksplit from B2 (GRP_M: t.k0 = 0)
      rb = make_rsrc(b_grp + t.n0, (uint64_t)((int64_t)p.ksplit * p.ldb - t.n0) * 2);
      rb2 = make_rsrc(b2_grp + t.n0, (uint64_t)((klen - p.ksplit) * p.ldb - t.n0) * 2);
    } else {
      rb = make_rsrc(b_grp + t.k0 * p.ldb + t.n0, (uint64_t)(klen * p.ldb - t.n0) * 2);
      rb2 = rb;
    }
    uint32_t va[NJ], vb[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      va[jj] = dma_voff<BK, ALAY, false>(wave * NJ + jj, lane, p.lda);
      vb[jj] = dma_voff<BK, BLAY, DUAL>(wave * NJ + jj, lane, p.ldb);
    }
    // K-contig dual: instructions j >= BK/4 (waves 2, 3) read the second resource.
    const bool b_second = DUAL && wave >= 2;
    // DMA instruction q (0 .. 2*NJ-1) of k-tile kt: even q are A tiles, odd q B tiles.
    auto dma_one = [&](int kt, int q) {
      uint16_t* st = ring[kt % STAGES];
      const int jj = q >> 1;
      const int j = wave * NJ + jj;
      if ((q & 1) == 0) {
        const uint32_t so_a = (ALAY == LAY_K) ? (uint32_t)kt * BK * 2 : (uint32_t)((int64_t)kt * BK * p.lda * 2);
        dma16(ra, va[jj], so_a, st + j * 512);
      } else {
        i32x4 rbk = b_second ? rb2 : rb;
        uint32_t so_b;
        if (BLAY == LAY_K) {
          so_b = (uint32_t)kt * BK * 2;
        } else if (p.ksplit && (int64_t)kt * BK >= p.ksplit) {
          rbk = rb2;
          so_b = (uint32_t)(((int64_t)kt * BK - p.ksplit) * p.ldb * 2);
        } else {
          so_b = (uint32_t)((int64_t)kt * BK * p.ldb * 2);
        }
        dma16(rbk, vb[jj], so_b, st + TILE_ELEMS + j * 512);
      }
    };

    // L2 prefetch of k-tile pkt, one instruction per wave per operand, each
    // lane touching one 64-byte sector.  A tile is also loaded by the tiles
    // of the same XCD that run at the same time and share it: the tiles of
    // one n-tile and consecutive m-tiles share B, those of one m-tile and
    // consecutive n-tiles share A (tiles are ordered m-fastest and an XCD
    // takes RUN consecutive tiles per round).  The sectors of a shared tile
    // are dealt round-robin over its C sharers, so that each is prefetched
    // once per XCD: this tile takes sectors e = c + C*j, c = its own index
    // modulo C.  Unassigned lanes get an offset outside every resource.
    constexpr int NPF = 2;
    constexpr int ITEMS = 8 * BK;  // 64-byte sectors of a 256 x BK operand tile
    const int run = (gridDim.x % 8) ? 1 : (int)gridDim.x / 8;
    const int cB = max(1, min(t.mtiles, run));
    const int cA = max(1, min(sched.NT, run / max(t.mtiles, 1)));
    auto pf_voff = [&](int C, int c, int64_t ld, int lay, int parts) -> uint32_t {
      const int wl = wave % (4 / parts);
      const int e = c + C * (wl * 64 + lane);
      if (e >= ITEMS / parts) return 0x7FFFFFF0u;
      if (lay == LAY_K) {
        constexpr int SPR = BK / 32;  // sectors per row
        return (uint32_t)((e / SPR) * ld * 2 + (e % SPR) * 64);
      }
      return (uint32_t)((e >> 3) * ld * 2 + (e & 7) * 64);
    };
    const uint32_t pa = pf_voff(cA, t.ntile % cA, p.lda, ALAY, 1);
    const uint32_t pb = pf_voff(cB, t.mtile % cB, p.ldb, BLAY, DUAL ? 2 : 1);
    auto pf_one = [&](int kt, int o) {
      if (o == 0) {
        const uint32_t so_a = (ALAY == LAY_K) ? (uint32_t)kt * BK * 2 : (uint32_t)((int64_t)kt * BK * p.lda * 2);
        touch4(ra, pa, so_a, lds_junk);
      } else {
        i32x4 rbk = b_second ? rb2 : rb;
        uint32_t so_b;
        if (BLAY == LAY_K) {
          so_b = (uint32_t)kt * BK * 2;
        } else if (p.ksplit && (int64_t)kt * BK >= p.ksplit) {
          rbk = rb2;
          so_b = (uint32_t)(((int64_t)kt * BK - p.ksplit) * p.ldb * 2);
        } else {
          so_b = (uint32_t)((int64_t)kt * BK * p.ldb * 2);
        }
        touch4(rbk, pb, so_b, lds_junk);
      }
    };

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragment f (0 .. MI+NI-1) of k-step kk of a ring stage, in the order the
    // MFMAs (mi-major) first use them: A0, B0 .. B3, A1 .. A3.
    auto read_frag = [&](const uint16_t* st, int kk, int f, bf16x8(&a)[MI], bf16x8(&b)[NI]) {
      static_assert(MI == 4 && NI == 4, "fragment order");
      if (f == 0 || f > NI) {
        const int mi = f == 0 ? 0 : f - NI;
        a[mi] = frag<BK, ALAY>(st, wm * 128 + mi * 32, kk, lane);
      } else {
        const int ni = f - 1;
        const int brow = DUAL ? (ni / 2) * 128 + wn * 64 + (ni % 2) * 32 : wn * 128 + ni * 32;
        b[ni] = frag<BK, BLAY>(st + TILE_ELEMS, brow, kk, lane);
      }
    };

    // One k-step: the 16 MFMAs of fragments (a, b), with, in between, the
    // reads of the next k-step's fragments (stage rst, step rkk), ND DMA
    // instructions q0 .. q0+ND-1 of k-tile dkt and then NP L2 prefetches of
    // k-tile pkt, spread evenly.  The scheduling barriers pin this order, so
    // that the DMA issue never comes as a burst that would stall the wave's
    // MFMAs behind a full address queue.
    auto kstep = [&](auto nd_c, auto np_c, const bf16x8(&a)[MI], const bf16x8(&b)[NI], bf16x8(&na)[MI],
                     bf16x8(&nb)[NI], const uint16_t* rst, int rkk, int dkt, int q0, int pkt) {
      constexpr int ND = decltype(nd_c)::value;
      constexpr int NO = ND + decltype(np_c)::value;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int mi = i / NI, ni = i % NI;
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
        if ((i & 1) == 0 && (i >> 1) < MI + NI) read_frag(rst, rkk, i >> 1, na, nb);
#pragma unroll
        for (int o = (i * NO) / 16; o < ((i + 1) * NO) / 16; ++o) {
          if (o < ND) dma_one(dkt, q0 + o);
          else pf_one(pkt, o - ND);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Pipeline.  While k-tile kt is consumed, k-tiles kt+1 .. kt+STAGES-1
    // are in flight.  A k-tile is KS k-steps; each step's MFMAs overlap the
    // LDS reads of the next step.  Before the last step of k-tile kt,
    // k-tile kt+1 is waited for (one barrier per k-tile); the stage of
    // k-tile kt, now fully read, is then refilled with k-tile kt+STAGES,
    // whose PER DMA instructions per wave are spread over the last step of
    // kt and the first SPREAD-1 steps of kt+1 (all before the next barrier).
    // Right after the last of them, NPF prefetches start the L2 fill of
    // k-tile kt+STAGES+PFD, so that its DMA, PFD k-tiles later, hits in L2;
    // a barrier's wait leaves these prefetches in flight (they are the only
    // loads issued after the awaited k-tile), and they have until the next
    // barrier to land.
    // The schedule is the same for every k-tile: k-tiles past the end
    // (kt >= nk) are loaded too, as zero fills of a stage that is never read
    // again (their offsets lie outside the buffer resources, so they touch
    // no memory), which keeps the loop body free of branches.
    constexpr int PER = 2 * NJ;
    constexpr int SPREAD = KS >= 2 ? 2 : 1;
    constexpr int PART = PER / SPREAD;
    constexpr int PFD = 2;
    static_assert(PER % SPREAD == 0 && SPREAD <= KS, "a stage's DMA is issued before the next barrier");
    using N0 = std::integral_constant<int, 0>;
    using NDP = std::integral_constant<int, PART>;
    using NPP = std::integral_constant<int, NPF>;
    bf16x8 fa[2][MI], fb[2][NI];
    if (nk > 0) {
      // The same issue pattern as the loop: each stage's DMAs, then the
      // prefetches of the k-tile PFD further on.
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) {
#pragma unroll
        for (int q = 0; q < PER; ++q) dma_one(s, q);
#pragma unroll
        for (int o = 0; o < NPF; ++o) pf_one(s + PFD, o);
      }
#pragma unroll
      for (int q = 0; q < PART; ++q) dma_one(STAGES - 1, q);
      wait_vm<NPF + (STAGES - 2) * (PER + NPF) + PART>();  // k-tile 0 has landed
      lds_barrier();
#pragma unroll
      for (int f = 0; f < MI + NI; ++f) read_frag(ring[0], 0, f, fa[0], fb[0]);
    }
    for (int kt = 0; kt < nk; ++kt) {
      const uint16_t* st = ring[kt % STAGES];
#pragma unroll
      for (int s = 0; s < KS - 1; ++s) {
        if (s + 2 < SPREAD)
          kstep(NDP(), N0(), fa[s & 1], fb[s & 1], fa[(s + 1) & 1], fb[(s + 1) & 1], st, s + 1, kt - 1 + STAGES,
                (s + 1) * PART, 0);
        else if (s + 2 == SPREAD)
          kstep(NDP(), NPP(), fa[s & 1], fb[s & 1], fa[(s + 1) & 1], fb[(s + 1) & 1], st, s + 1,
                kt - 1 + STAGES, (s + 1) * PART, kt - 1 + STAGES + PFD);
        else
          kstep(N0(), N0(), fa[s & 1], fb[s & 1], fa[(s + 1) & 1], fb[(s + 1) & 1], st, s + 1, 0, 0, 0);
      }
      // k-tile kt+1 has landed: after its last DMA come only its prefetches
      // and the later stages (each PER DMAs and NPF prefetches).
      wait_vm<(STAGES - 2) * (PER + NPF) + NPF>();
      lds_barrier();
      // The last step also reads k-tile kt+1's first fragments (for the
      // last k-tile, from a stage it never uses).
      if (SPREAD == 1)
        kstep(NDP(), NPP(), fa[1], fb[1], fa[0], fb[0], ring[(kt + 1) % STAGES], 0, kt + STAGES, 0,
              kt + STAGES + PFD);
      else
        kstep(NDP(), N0(), fa[1], fb[1], fa[0], fb[0], ring[(kt + 1) % STAGES], 0, kt + STAGES, 0, 0);
    }
    wait_vm<0>();  // the zero fills past the end have landed before the ring is reused
    lds_barrier();  // every wave is done reading the ring (and no DMA is in flight) before staging

    // Epilogue, staged through the ring one 32-row block at a time: each
    // wave writes its 32 x 128 block of acc[mi] to its own staging area and
    // reads it back as row vectors of 8 columns.  The areas of the waves are
    // disjoint and a wave's LDS accesses complete in order, so only the ring
    // hand-offs need barriers (above, and after the last block).
    //   acc[mi][ni][r] is C[row][col] with
    //   row = wm*128 + mi*32 + (r/4)*8 + (lane/32)*4 + r%4, col = n-block base + lane%32.
    {
      constexpr int WC = NI * 32;
      constexpr int SP = WC + 4;
      float* stage = reinterpret_cast<float*>(&ring[0][0]) + wave * 32 * SP;
      static_assert(4 * 32 * SP * 4 <= (int)sizeof(ring), "staging fits in the ring");
      constexpr int OC = DUAL ? WC / 2 : WC;
      constexpr int CPR = OC / 8;                 // 8-column vectors per row
      constexpr int ITER = 32 * CPR / 64;         // vectors per lane per block
      static_assert(32 * CPR % 64 == 0, "whole vectors per lane");
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            stage[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * SP + ni * 32 + (lane & 31)] = acc[mi][ni][r];
        float v[ITER][8], v2[ITER][8];
#pragma unroll
        for (int it2 = 0; it2 < ITER; ++it2) {
          const int e = lane + it2 * 64;
          const int rl = e / CPR, cv = (e % CPR) * 8;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            v[it2][q] = stage[rl * SP + cv + q];
            v2[it2][q] = DUAL ? stage[rl * SP + OC + cv + q] : 0.f;
          }
        }
#pragma unroll
        for (int it2 = 0; it2 < ITER; ++it2) {
          const int e = lane + it2 * 64;
          const int rl = e / CPR, cv = (e % CPR) * 8;
          const int row = wm * 128 + mi * 32 + rl;
          const int col = (DUAL ? wn * 64 : wn * 128) + cv;
          if (row < t.mlim && col < t.nlim) epi_store8<GRP, EPI>(p, t, row, col, v[it2], v2[it2]);
        }
      }
      lds_barrier();  // all staging reads are done before the next tile's DMA refills the ring
    }
  }
}

}  // namespace moe
