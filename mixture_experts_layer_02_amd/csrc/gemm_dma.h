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
// FP8 K-contiguous rows of 64 bytes (four 16-byte chunks per k-tile).
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 3; }

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
// is consumed.  M0 (the LDS base of the copy) is an operand of the asm.
// lds: the destination's LDS byte address, already wave-uniform (the kernel
// derives it with scalar arithmetic from the ring's base, so that no vector
// instruction sits between the address and the copy).
//
// Wait states before it: one for the LDS DMA reading M0 after its SALU write,
// five for a buffer instruction reading SGPRs that a VALU op (readfirstlane,
// or the readlane of an SGPR spill reload) may have just written.  LIGHT
// issues one only; it is used in the steady k-loop alone, and the build checks
// the generated code of every kernel for a VALU write of a DMA's SGPR operand
// within five wait states before it (hazard_check.py). If the check finds one,
// the build compiles again with MOE_LIGHT_DMA=0, which gives every DMA five.
#ifndef MOE_LIGHT_DMA
#define MOE_LIGHT_DMA 1
#endif
template <bool LIGHT = false>
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  if (LIGHT)
    asm volatile(
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
        : "memory");
  else
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
        : "memory");
}

// L2 prefetch: lane i reads the 4 bytes at rsrc + voff + soff into the LDS
// word lds_junk + 4 i (a scratch area nobody reads).  Its only purpose is to
// start the L2 fill of that 64-byte sector well before the tile DMA needs
// it; an offset outside the resource reads nothing.
template <bool LIGHT = false>
__device__ __forceinline__ void touch4u(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  if (LIGHT)
    asm volatile(
        "s_nop 0\n\t"  // as in dma16
        "buffer_load_dword %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
        : "memory");
  else
    asm volatile(
        "s_nop 4\n\t"  // as in dma16
        "buffer_load_dword %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds)
        : "memory");
}
__device__ __forceinline__ void touch4(i32x4 rsrc, uint32_t voff, uint32_t soff, const uint32_t* lds_dst) {
  touch4u(rsrc, voff, soff, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst));
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

// FP8 B fragment (k = kk*16 + (lane/32)*8 + 0..7 of row row0 + lane%32) as
// bf16: the 8 codes are one 8-byte read, decoded to float32, multiplied by
// the row's block scale (16 KB past the codes) and rounded to nearest even.
typedef float f32x2_q8 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 frag_q8(const uint16_t* S, int row0, int kk, int lane) {
  const int r = row0 + (lane & 31);
  const uint8_t* Sb = reinterpret_cast<const uint8_t*>(S);
  const uint2 c = *reinterpret_cast<const uint2*>(Sb + r * 64 + ((kk ^ swz8(r)) << 4) + ((lane >> 5) << 3));
  const float sc = reinterpret_cast<const float*>(Sb + 16384)[r];
  const f32x2_q8 v0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false);
  const f32x2_q8 v1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
  const f32x2_q8 v2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false);
  const f32x2_q8 v3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
  typedef uint32_t u32x4q __attribute__((ext_vector_type(4)));
  const u32x4q w = {pack_bf2(v0[0] * sc, v0[1] * sc), pack_bf2(v1[0] * sc, v1[1] * sc),
                    pack_bf2(v2[0] * sc, v2[1] * sc), pack_bf2(v3[0] * sc, v3[1] * sc)};
  return __builtin_bit_cast(bf16x8, w);
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
// operands, K-contiguous operands have K (or every k-tile) a multiple of 32,
// msplit (if set) a multiple of 32.  CF32: C is float (EPI_STORE or EPI_ADD
// with p.c_f32 set); a compile-time choice, so that one kernel holds one
// epilogue.
//
// Tiles are pipelined across tile boundaries: the last k-tiles of a tile
// load the first k-tiles of the next one (positions past the end of a tile
// continue in the next), so that the next tile's operands are in flight
// while this tile's epilogue runs.  The epilogue stages through an LDS area
// of its own and writes C with unconditional buffer stores (rows and columns
// outside the tile fall outside the store resources), so that the number of
// memory instructions it issues is a compile-time constant and the next
// tile's first wait can let them stay in flight.
//
// GATH (the Domyn page's SonicMoE: expert GEMMs read the tokens in place,
// with no permuted copy): 0 none; GATH_A: the K-contiguous A of a GRP_M
// product is x[gather[r]] for row r (gate/up from x through row_token);
// GATH_B: the MN-contiguous B of a GRP_K product has k-row k equal to row
// gather[k] of x (dW1|dW3 from x through row_token); GATH_AK the same for the
// MN-contiguous A of a GRP_K product (dW2 from the layer's dy through
// row_token).  The gathered matrix has gather_rows rows of ldb (or lda)
// elements and must stay under 2 GiB.  With GATH_A and EPI_SWIGLU_BWD (dH
// from dy through row_token), row r's dH is scaled by row_scale[r] (the
// routing weight that the permuted copy of dy would carry), and
// row_scale[r] * silu(G) * U is written to h_out when it is set.
//
// BQ8 (FP8 expert weights, Domyn page section "FP8 expert weight
// all-gather"): the K-contiguous B of a GRP_M product holds E4M3 codes, one
// float32 scale per 128 consecutive values of a row (bs, bs2 for the second
// B).  The tiles move as bytes (half the traffic and LDS of bf16) and are
// decoded to bf16 when the MFMA fragments are read: decode * scale in
// float32, rounded to nearest even, which is exactly what moe_fp8_dequantize
// writes, so the product equals the bf16 product on dequantised weights.
//
// F8 (FP8 matrix cores): A and B hold E4M3 codes, two to a bf16 slot (K, lda,
// ldb and the strides count pairs of codes, so a 64-wide k-tile is 128 codes),
// with power-of-two block scales as E8M0 bytes, one per 128 codes of a row
// (a_scale, b_scale, b2_scale; sbytes per row).  A k-tile is then one scale
// block: each k-step is one v_mfma_scale_f32_32x32x64_f8f6f4 per 32 x 32
// block, which applies the row's A and the column's B scale itself.  The
// scale bytes of a k-tile's rows come with its operand tiles: one dword per
// row (the four blocks k-tile & ~3 .. | 3) into a 2 KB area of the stage,
// so sbytes is a multiple of 4 (a row's scales padded when K/128 is not).
// A is read through row_token (GATH_A) or in place (GATH_NONE).
template <int BK, int STAGES, int ALAY, int BLAY, int GRP, int EPI, bool DUAL, bool CF32, bool DYN, int GATH,
          bool BQ8, bool F8 = false>
__global__ void __launch_bounds__(256, 1) gemm_dma_kernel(GemmParams p) {
  using namespace dma;
  static_assert(!DUAL || BLAY == LAY_K, "dual B is K-contiguous");
  static_assert(GATH == 0 || (GATH == GATH_A && ALAY == LAY_K && GRP == GRP_M) ||
                    (GATH == GATH_B && BLAY == LAY_MN && GRP == GRP_K && !DUAL) ||
                    (GATH == GATH_AK && ALAY == LAY_MN && GRP == GRP_K && !DUAL),
                "gathered operands: K-contiguous A of GRP_M, MN-contiguous B of GRP_K");
  static_assert(!BQ8 || (BLAY == LAY_K && GRP == GRP_M && (GATH == GATH_NONE || GATH == GATH_A) && BK == 64),
                "FP8 B: K-contiguous B of GRP_M, 64-wide k-tiles (half a scale block)");
  static_assert(BK == 64 && STAGES == 2, "ring of two 64-wide k-tiles");
  static_assert(!F8 || (ALAY == LAY_K && BLAY == LAY_K && GRP == GRP_M && !BQ8 &&
                        (GATH == GATH_A || GATH == GATH_NONE)),
                "FP8 matrix cores: K-contiguous A (in place or read through row_token) and B of GRP_M");
  // GKB: the k-rows of an MN-contiguous operand of a grouped-K product are
  // gathered (B for GATH_B, A for GATH_AK), through a ring of token copies.
  constexpr bool GKB = GATH == GATH_B || GATH == GATH_AK;
  constexpr int MI = 4, NI = 4;          // 32 x 32 blocks per wave (128 x 128)
  typedef int i32x8f __attribute__((ext_vector_type(8)));
  using Frag = typename std::conditional<F8, i32x8f, bf16x8>::type;  // one operand fragment of a k-step
  constexpr int TILE_ELEMS = 256 * BK;   // one operand tile
  constexpr int STAGE_ELEMS = 2 * TILE_ELEMS + (F8 ? 1024 : 0);  // (F8: + A and B scale dwords, 1 KB each)
  constexpr int SCA = 2 * TILE_ELEMS * 2, SCB = SCA + 1024;        // their byte offsets in a stage
  constexpr int NJ = BK / 8;             // DMA instructions per wave per operand tile
  constexpr int NJB = BQ8 ? NJ / 2 : NJ;  // ... for B (FP8 B is half the bytes)
  constexpr int KS = F8 ? 2 : BK / 16;   // MFMA k-steps per k-tile (F8: 64 codes per step)
  constexpr int WC = NI * 32;            // columns of a wave's block
  constexpr int SP = WC + 4;             // staging row pitch (floats)
  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES][STAGE_ELEMS];
  __shared__ int s_pref[MAXG + 1];
  __shared__ int s_scan[256];
  __shared__ __attribute__((aligned(16))) float s_stage[4][8 * SP];
  __shared__ __attribute__((aligned(256))) uint32_t lds_junk[64];
  // Gathered operand: the source rows of a tile (GATH_A, two tiles) or of a
  // ring position (GATH_B and GATH_AK, eight positions).
  __shared__ __attribute__((aligned(256))) int32_t s_tok[GATH == GATH_A ? 2 : GKB ? 8 : 1]
                                                         [GATH == GATH_A ? 256 : 64];

  Scheduler<GRP, BM, DUAL ? BN / 2 : BN> sched;
  sched.init(p, s_pref, s_scan);
  // LDS byte address of the ring (the low half of its generic address).
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&ring[0][0]);
  const uint32_t junk_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&lds_junk[0]);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps DMA operands scalar
  const int wm = wave >> 1, wn = wave & 1;
  // Half tiles (row-grouped products in bf16): a tile with at most 128 valid
  // rows - an expert's last, partial m-tile - would spend wave row 1's
  // MFMAs on padding.  There wave row wm computes rows 64 wm .. 64 wm + 63
  // instead (arow, the A row base of its fragment reads), its row blocks 0
  // and 1 only: each wave then holds half the MFMAs of a full tile, and the
  // outputs stay disjoint.
  constexpr bool HALFM = GRP == GRP_M && !F8;
  // Likewise across columns for plain products (the router's logits, N = E =
  // 384): a tile with at most 128 valid columns has wave column wn compute
  // columns 64 wn .. 64 wn + 63 (bcol, the B row base of its fragment reads)
  // with its column blocks 0 and 1 only.
  constexpr bool HALFN = GRP == GRP_NONE && !DUAL && !F8 && !BQ8;
  // The steady k-loop's DMAs take one wait state (see dma16), except in the
  // gathered-B weight-gradient kernels, whose k-loop reloads spilled SGPRs
  // next to its DMAs: they take five.
  constexpr bool LIGHT_K = MOE_LIGHT_DMA && GATH != GATH_B;
  int arow = wm * 128, arow_next = wm * 128;
  int bcol = wn * 128, bcol_next = wn * 128;
  const uint16_t* Ag = reinterpret_cast<const uint16_t*>(p.A);
  const uint16_t* Bg = reinterpret_cast<const uint16_t*>(p.B);
  const uint16_t* B2g = reinterpret_cast<const uint16_t*>(p.B2);
  const int run = (gridDim.x % 8) ? 1 : (int)gridDim.x / 8;

  // Per-lane DMA offsets (the same for every tile: the tile moves the
  // resource bases) and the wave's B resource for dual K-contiguous B.
  uint32_t va[NJ], vb[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    va[jj] = dma_voff<BK, ALAY, false>(wave * NJ + jj, lane, p.lda);
    vb[jj] = dma_voff<BK, BLAY, DUAL>(wave * NJ + jj, lane, p.ldb);
  }
  // FP8 B: a k-tile row is 64 bytes, four 16-byte chunks; instruction j
  // covers rows 16j .. 16j+15, lane i row 16j + i/4 at LDS chunk i%4, which
  // holds global chunk (i%4) ^ swz8(row) (the swizzle spreads the 8-byte
  // fragment reads of consecutive rows over the banks).  The scale of a
  // lane's row (wave w copies rows 64w .. 64w+63) sits 16 KB into the stage.
  uint32_t vs = 0;
  if (BQ8) {
#pragma unroll
    for (int jj = 0; jj < NJB; ++jj) {
      const int row = 16 * (wave * NJB + jj) + lane / 4;
      const int src_row = DUAL ? (row & 127) : row;
      vb[jj] = (uint32_t)(src_row * p.K + (((lane & 3) ^ swz8(row)) << 4));
    }
    const int srow = DUAL ? ((wave * 64 + lane) & 127) : wave * 64 + lane;
    vs = (uint32_t)(srow * (p.K / 128) * 4);
  }
  const bool b_second = DUAL && wave >= 2;  // instructions j >= BK/4 read the second resource

  // Load state of one output tile: buffer resources over its operand tiles,
  // its k-tile count, and its L2 prefetch lane offsets.
  struct Ld {
    i32x4 ra, rb, rb2;
    int nk;
    uint32_t pa, pb;
    // Gathered operand: the resource over the tile's tokens (the source
    // rows of its A rows, GATH_A, or of its k-rows, GATH_B), how many are
    // valid and the lane's L2-prefetch sector of that operand (-1: none).
    i32x4 rt;
    int glim;
    int pfe;
    i32x4 rs;  // BQ8: the scales of the tile's B rows (of the second B for waves 2 and 3 with dual B)
    uint32_t sbo;    // F8: the lane's B-row scale offset (bit 31 set past the tile's valid rows)
    uint32_t sao;    // F8, A in place: the lane's A-row scale offset (bit 31 set past the valid rows)
  };
  // GATH_A: the A offsets of the current and the next tile's rows (filled
  // from their tokens once these are in LDS).
  uint32_t gcur[GATH == GATH_A ? NJ : 1], gnext[GATH == GATH_A ? NJ : 1];
  // F8: the lane's A-row scale offset (row 64 wave + lane of the tile) for
  // the current and the next tile, and its B-row scale offset.
  uint32_t gsc = 0x80000000u, gsn = 0x80000000u;
  // F8: one resource over all of A's scale rows, one over all of the wave's B
  // scale rows (B for waves 0 and 1, B2 for waves 2 and 3 with dual B).
  const i32x4 rsa = F8 ? make_rsrc(p.a_scale, (uint64_t)p.gather_rows * p.sbytes) : make_rsrc(Ag, 0);
  const i32x4 rsb = F8 ? make_rsrc(DUAL && wave >= 2 ? p.b2_scale : p.b_scale,
                                   (uint64_t)p.ngroups * p.N * p.sbytes)
                       : make_rsrc(Ag, 0);
  // L2 prefetch: one instruction per wave per operand, each lane touching one
  // 64-byte sector.  A tile is also loaded by the tiles of the same XCD that
  // run at the same time and share it: the tiles of one n-tile and
  // consecutive m-tiles share B, those of one m-tile and consecutive n-tiles
  // share A (tiles are ordered m-fastest and an XCD takes RUN consecutive
  // tiles per round).  The sectors of a shared tile are dealt round-robin
  // over its C sharers, so that each is prefetched once per XCD: this tile
  // takes sectors e = c + C*j, c = its own index modulo C.  Unassigned lanes
  // get an offset outside every resource.
  constexpr int NPF = 2;
  constexpr int ITEMS = 8 * BK;  // 64-byte sectors of a 256 x BK operand tile
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
  auto setup = [&](const TileCtx& t) -> Ld {
    Ld L;
    const int64_t klen = t.k1 - t.k0;
    L.nk = (int)((klen + BK - 1) / BK);
    const uint16_t* a_base = (ALAY == LAY_K) ? Ag + t.m0 * p.lda + t.k0 : Ag + t.k0 * p.lda + t.m0;
    const uint16_t* b_grp = Bg;
    const uint16_t* b2_grp = B2g;
    if (GRP == GRP_M) {
      b_grp += (int64_t)t.g * p.b_gstride;
      if (B2g) b2_grp += (int64_t)t.g * p.b_gstride;
    }
    // K-contig: rows [0, lim) of the tile's row block; MN-contig: k-rows
    // [0, klen) from column m0/n0 (the range ends with row k1-1, so it never
    // runs past the allocation).
    const int nlim_b = DUAL ? min(t.nlim, BN / 2) : t.nlim;
    L.ra = (ALAY == LAY_K) ? make_rsrc(a_base, (uint64_t)((int64_t)t.mlim * p.lda - t.k0) * 2)
                           : make_rsrc(a_base, (uint64_t)(klen * p.lda - t.m0) * 2);
    if (GATH == GATH_A) {  // rows come from anywhere in the source; row validity is in gv
      L.ra = make_rsrc(Ag, (uint64_t)p.gather_rows * p.lda * 2);
      L.rt = make_rsrc(p.gather + t.m0, (uint64_t)t.mlim * 4);
    }
    if (GATH == GATH_AK) {  // A's k-rows come from anywhere in the source; validity is in the offsets
      L.ra = make_rsrc(Ag + t.m0, (uint64_t)((int64_t)p.gather_rows * p.lda - t.m0) * 2);
      L.rt = make_rsrc(p.gather + t.k0, (uint64_t)klen * 4);
    }
    if (GATH == GATH_B) {  // k-rows come from anywhere in the source; k-row validity is in the offsets
      L.rb = L.rb2 = make_rsrc(Bg + t.n0, (uint64_t)((int64_t)p.gather_rows * p.ldb - t.n0) * 2);
      L.rt = make_rsrc(p.gather + t.k0, (uint64_t)klen * 4);
    } else if (BLAY == LAY_K) {
      // (a grouped-K product, split over K, starts at its chunk's k0)
      const int64_t bk0 = GRP == GRP_K ? t.k0 : 0;
      L.rb = make_rsrc(b_grp + (int64_t)t.n0 * p.ldb + bk0, (uint64_t)((int64_t)nlim_b * p.ldb - bk0) * 2);
      L.rb2 = DUAL ? make_rsrc(b2_grp + (int64_t)t.n0 * p.ldb + bk0, (uint64_t)((int64_t)nlim_b * p.ldb - bk0) * 2)
                   : L.rb;
    } else if (p.ksplit) {  // k < ksplit from B, k >= ksplit from B2 (GRP_M: t.k0 = 0)
      L.rb = make_rsrc(b_grp + t.n0, (uint64_t)((int64_t)p.ksplit * p.ldb - t.n0) * 2);
      L.rb2 = make_rsrc(b2_grp + t.n0, (uint64_t)((klen - p.ksplit) * p.ldb - t.n0) * 2);
    } else {
      L.rb = make_rsrc(b_grp + t.k0 * p.ldb + t.n0, (uint64_t)(klen * p.ldb - t.n0) * 2);
      L.rb2 = L.rb;
    }
    // Sharers within an XCD's run of consecutive tiles: m-tile fastest, the
    // run's m-tiles share B and, when a group has fewer m-tiles than the run,
    // its n-tiles share A; n-tile fastest, the other way round.
    const int cB = t.nfast ? max(1, min(t.mtiles, run / max(sched.NT, 1))) : max(1, min(t.mtiles, run));
    const int cA = t.nfast ? max(1, min(sched.NT, run)) : max(1, min(sched.NT, run / max(t.mtiles, 1)));
    L.pa = pf_voff(cA, t.ntile % cA, p.lda, ALAY, 1);
    L.pb = pf_voff(cB, t.mtile % cB, p.ldb, BLAY, DUAL ? 2 : 1);
    if (BQ8) {
      // FP8 B: bytes, and a k-tile row is one 64-byte sector.
      const uint8_t* q_grp = reinterpret_cast<const uint8_t*>(p.B) + (int64_t)t.g * p.b_gstride;
      const uint8_t* q2_grp = reinterpret_cast<const uint8_t*>(p.B2) + (int64_t)t.g * p.b_gstride;
      L.rb = make_rsrc(q_grp + (int64_t)t.n0 * p.K, (uint64_t)nlim_b * p.K);
      L.rb2 = DUAL ? make_rsrc(q2_grp + (int64_t)t.n0 * p.K, (uint64_t)nlim_b * p.K) : L.rb;
      const int kbl = p.K / 128;
      const int64_t srow0 = (int64_t)t.g * (p.b_gstride / p.K) + t.n0;
      const float* s_base = (DUAL && wave >= 2 ? p.bs2 : p.bs) + srow0 * kbl;
      L.rs = make_rsrc(s_base, (uint64_t)nlim_b * kbl * 4);
      const int parts = DUAL ? 2 : 1;
      const int e = t.mtile % cB + cB * ((wave % (4 / parts)) * 64 + lane);
      L.pb = e < 256 / parts ? (uint32_t)(e * p.K) : 0x7FFFFFF0u;
    }
    if (GATH == GATH_A) {
      const int e = t.ntile % cA + cA * (wave * 64 + lane);
      L.glim = t.mlim;
      L.pfe = e < ITEMS ? e : -1;
      L.pa = 0x7FFFFFF0u;
    }
    if (F8) {  // B row (64 wave + lane) mod the rows of one B is row g N + n0 + r of its scale array
      const int r = (wave * 64 + lane) & (DUAL ? 127 : 255);
      L.sbo = ((uint32_t)((int64_t)t.g * p.N + t.n0 + r) * (uint32_t)p.sbytes) | (r < nlim_b ? 0u : 0x80000000u);
      // A in place: tile row 64 wave + lane is A row m0 + that (read through
      // row_token instead, its offset comes from the tile's tokens)
      const int ra = wave * 64 + lane;
      L.sao = GATH == GATH_NONE ? ((uint32_t)(t.m0 + ra) * (uint32_t)p.sbytes) | (ra < t.mlim ? 0u : 0x80000000u)
                                : 0x80000000u;
    }
    if (GATH == GATH_B) {
      const int e = t.mtile % cB + cB * (wave * 64 + lane);
      L.glim = (int)klen;
      L.pfe = e < ITEMS ? e : -1;
    }
    if (GATH == GATH_AK) {
      const int e = t.ntile % cA + cA * (wave * 64 + lane);
      L.glim = (int)klen;
      L.pfe = e < ITEMS ? e : -1;
      L.pa = 0x7FFFFFF0u;
    }
    return L;
  };
  Ld null_ld;  // loads nothing: every offset is outside its resources
  null_ld.ra = null_ld.rb = null_ld.rb2 = null_ld.rt = null_ld.rs = make_rsrc(Ag, 0);
  null_ld.sbo = null_ld.sao = 0x80000000u;
  null_ld.nk = 0;
  null_ld.pa = null_ld.pb = 0x7FFFFFF0u;
  null_ld.glim = 0;
  null_ld.pfe = -1;

  // B resource and scalar offset of k-tile k of a tile.
  auto b_src = [&](const Ld& L, int k, i32x4& rbk, uint32_t& so_b) {
    rbk = b_second ? L.rb2 : L.rb;
    if (BQ8) {
      so_b = (uint32_t)k * BK;
    } else if (BLAY == LAY_K) {
      so_b = (uint32_t)k * BK * 2;
    } else if (p.ksplit && k * BK >= p.ksplit) {  // (32-bit scalar arithmetic: k * BK < K < 2^31, and the
      rbk = L.rb2;                                 //  offset is the 32-bit scalar offset of the buffer load)
      so_b = (uint32_t)(k * BK - p.ksplit) * (uint32_t)p.ldb * 2u;
    } else {
      so_b = (uint32_t)(k * BK) * (uint32_t)p.ldb * 2u;
    }
  };
  auto a_so = [&](int k) -> uint32_t {
    return (ALAY == LAY_K) ? (uint32_t)k * BK * 2 : (uint32_t)(k * BK) * (uint32_t)p.lda * 2u;
  };

  // Current and next tile.  A ring position is a k-tile of the current tile
  // (pos < cur.nk) or of the next one (pos - cur.nk); positions past both are
  // loads of nothing.  Ring stage of a position: (gbase + pos) % STAGES.
  // Tile order.  Static (p.dyn == NULL): workgroup b takes the ids
  // xcd_tile(0, grid), xcd_tile(1, grid), ... fixed at launch.  Dynamic
  // (the Domyn page's "Dynamic tile scheduling in SonicMoE": idle workgroups
  // take the next tile from a shared atomic counter, so that running ones
  // also take the tiles of workgroups that start late): the same per-XCD
  // sequences become eight queues, p.dyn[x] counting the tiles taken from
  // XCD x's sequence; a workgroup takes from its own XCD's queue and, once
  // that is empty, from the others.  Every tile is computed exactly as in
  // the static order, so the outputs are bitwise identical.  A workgroup
  // claims two tiles ahead (the next tile's operands load during this one);
  // a claim is issued at the top of a tile and its result published to LDS
  // after the wait of k-tile 1, when the atomic has long returned.  The last
  // workgroup to finish (p.dyn[8] counts them) zeroes the counters.
  __shared__ int s_q[2];
  constexpr bool dyn = DYN;  // a separate instantiation: the static one carries none of this
  const bool w0 = wave == 0;  // wave 0 runs the claims, all its lanes alike
  const int nq = (gridDim.x % 8) ? 1 : 8;
  const int x0 = (int)blockIdx.x % nq;
  // Wave 0 state (the same in all its lanes).  pend: the raw result of the
  // own-queue claim in flight (its lane 0 holds the claim's index), or
  // PEND_STEAL (the own queue is empty: take from the others).
  constexpr int PEND_NONE = -1, PEND_STEAL = -2;
  int exhausted = 0;  // bit x: queue x is known to be empty
  int pend = PEND_NONE;
  // What the tile's claim still needs: 0 nothing, 1 publishing the own-queue
  // claim in pend, 2 taking from the other queues.  Kept apart from pend so
  // that pend is not rewritten inside the k-loop: a rewrite there would
  // make the compiler copy it, and wait for the atomic, where the loop starts.
  int pstate = 0;
  auto q_tile = [&](int x, int n) __attribute__((always_inline)) -> int {
    return nq == 1 ? n : (n / run) * (int)gridDim.x + x * run + (n % run);
  };
  // A claim on counter x: lane 0 adds 1; its result is the claim's index.  The result is waited for only where it is
  // used (this file is built with LLVM's atomic optimizer off, which would
  // otherwise combine the wave's atomic into one lane's and wait for it at
  // once, stalling wave 0 behind every load in flight).
  auto claim = [&](int x) __attribute__((always_inline)) -> int {
    typedef __attribute__((address_space(1))) int gint;  // global: a flat atomic would also count on lgkmcnt
    int r = 0;
    if (lane == 0) r = __hip_atomic_fetch_add((gint*)(p.dyn + x), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return r;
  };
  // The tile of claim state n (see pend), taking from the other queues in
  // turn when the own one is empty; sched.total when every queue is.
  // Unrolled with no early exit, and all of wave 0 runs it, so that the
  // control flow stays uniform and the tile state stays in scalar registers.
  auto resolve = [&](int n) __attribute__((always_inline)) -> int {
    int found = sched.total;
    if (n >= 0) {
      const int c = q_tile(x0, n);
      if (c < sched.total) found = c;
      else exhausted |= 1 << x0;
    }
#pragma unroll
    for (int s = 1; s < 8; ++s) {
      const int x = (x0 + s) & 7;
      if (s < nq && found >= sched.total && !((exhausted >> x) & 1)) {
        const int c = q_tile(x, __builtin_amdgcn_readfirstlane(claim(x)));
        if (c < sched.total) found = c;
        else exhausted |= 1 << x;
      }
    }
    return found;
  };
  auto claim_own = [&]() __attribute__((always_inline)) -> int {
    return ((exhausted >> x0) & 1) ? PEND_STEAL : claim(x0);
  };
  auto dyn_finish = [&]() __attribute__((always_inline)) {
    if (dyn && w0) {
      const int done = __builtin_amdgcn_readfirstlane(claim(8));
      if (done == (int)gridDim.x - 1) {  // the last workgroup: every claim is over
#pragma unroll
        for (int x = 0; x < 9; ++x) atomicExch(p.dyn + x, 0);
      }
    }
  };

  int it = 0;
  int id;
  if (dyn) {
    if (w0) {
      const int i0 = resolve(__builtin_amdgcn_readfirstlane(claim_own()));
      const int i1 = i0 < sched.total ? resolve(__builtin_amdgcn_readfirstlane(claim_own())) : sched.total;
      s_q[0] = i0;
      s_q[1] = i1;
    }
    __syncthreads();
    id = __builtin_amdgcn_readfirstlane(s_q[0]);  // uniform: keeps the tile's resources scalar
  } else {
    id = xcd_tile(0, gridDim.x);
  }
  if (id >= sched.total) {
    dyn_finish();
    return;
  }
  TileCtx t = sched.template tile<!DYN>(p, s_pref, id);
  Ld cur = setup(t);
  Ld nxt = null_ld;
  int gbase = 0;
  bool primed = false;  // cur's k-tiles 0 and 1 are issued, k-tile 0 has landed and its first fragments are read

  // PURE: the position is known to be one of the current tile's.
  auto pick = [&](int pos, int& k, auto pure_c) -> Ld {
    if (decltype(pure_c)::value) {
      k = pos;
      return cur;
    }
    // (cur.nk is uniform; with a gathered operand the compiler may hold a
    // copy in a VGPR, so it is restated to keep k and the selects scalar.)
    const int cnk = (GATH != 0 || BQ8) ? __builtin_amdgcn_readfirstlane(cur.nk) : cur.nk;
    const bool c = pos < cnk;
    k = c ? pos : pos - cnk;
    Ld L;
    L.ra = c ? cur.ra : nxt.ra;
    L.rb = c ? cur.rb : nxt.rb;
    L.rb2 = c ? cur.rb2 : nxt.rb2;
    L.pa = c ? cur.pa : nxt.pa;
    L.pb = c ? cur.pb : nxt.pb;
    L.nk = 0;
    if (BQ8) L.rs = c ? cur.rs : nxt.rs;
    if (F8) {
      L.sbo = c ? cur.sbo : nxt.sbo;
      L.sao = c ? cur.sao : nxt.sao;
    }
    if (GATH != 0) {
      L.rt = c ? cur.rt : nxt.rt;
      L.glim = c ? cur.glim : nxt.glim;
      L.pfe = c ? cur.pfe : nxt.pfe;
    }
    return L;
  };
  // GATH_A: A offset jj of ring position pos (the current or the next tile's rows).
  // (A position past the current tile reads the next tile's rows; when the
  // next tile is not loaded ahead, its resource is empty and nothing loads.)
  auto a_gv = [&](int pos, int jj, auto pure_c) __attribute__((always_inline)) -> uint32_t {
    if (decltype(pure_c)::value) return gcur[GATH == GATH_A ? jj : 0];
    return pos < cur.nk ? gcur[GATH == GATH_A ? jj : 0] : gnext[GATH == GATH_A ? jj : 0];
  };
  auto a_gs = [&](int pos, auto pure_c) __attribute__((always_inline)) -> uint32_t {
    if (decltype(pure_c)::value) return gsc;
    return pos < cur.nk ? gsc : gsn;
  };
  // GATH_B (GATH_AK): the B (A) offsets of the position whose DMA is being
  // issued, and the L2-prefetch offset held for position kt+3 (see ktile).
  uint32_t gvb[GKB ? NJ : 1];
  uint32_t gpb = 0x7FFFFFF0u;
#pragma unroll
  for (int jj = 0; jj < (GKB ? NJ : 1); ++jj) gvb[jj] = 0x80000000u;
  // DMA instruction q (0 .. 2*NJ-1) of ring position pos: even q are A, odd q B.
  auto dma_one = [&](int pos, int q, auto pure_c) __attribute__((always_inline)) {
    int k;
    const Ld L = pick(pos, k, pure_c);
    uint16_t* st = ring[(uint32_t)(gbase + pos) % STAGES];
    // the stage's LDS byte address in scalar arithmetic; element offsets x2
    const uint32_t stb = ring_lds + ((uint32_t)(gbase + pos) % STAGES) * STAGE_ELEMS * 2;
    if (BQ8) {  // q < NJ: A; then NJB FP8 B instructions; then the B rows' scales
      constexpr bool LTQ = LIGHT_K && decltype(pure_c)::value;  // the steady k-loop: one wait state (checked at build)
      if (q < NJ) {
        dma16<LTQ>(L.ra, GATH == GATH_A ? a_gv(pos, q, pure_c) : va[q], a_so(k), stb + (wave * NJ + q) * 1024);
      } else if (q < NJ + NJB) {
        i32x4 rbk;
        uint32_t so_b;
        b_src(L, k, rbk, so_b);
        dma16<LTQ>(rbk, vb[q - NJ], so_b, stb + TILE_ELEMS * 2 + (wave * NJB + q - NJ) * 1024);
      } else {
        touch4(L.rs, vs, (uint32_t)(k >> 1) * 4u,
               reinterpret_cast<const uint32_t*>(st + TILE_ELEMS + 8192 + wave * 128));
      }
      return;
    }
    const int jj = q >> 1;
    const int j = wave * NJ + jj;
    constexpr bool LT = LIGHT_K && decltype(pure_c)::value;  // the steady k-loop: one wait state (checked at build)
    if (F8 && q >= 2 * NJ) {  // the scale dwords of the wave's 64 A rows, then of its 64 B rows
      // (always five wait states: the compiler spills these resources to
      // vector lanes and may reload one just before its use)
      const uint32_t so = (uint32_t)(k >> 2) * 4u;
      if (q == 2 * NJ) touch4u<false>(rsa, GATH == GATH_A ? a_gs(pos, pure_c) : L.sao, so, stb + SCA + wave * 256);
      else touch4u<false>(rsb, L.sbo, so, stb + SCB + wave * 256);
      return;
    }
    if ((q & 1) == 0 && GATH == GATH_AK) {
      dma16<LT>(L.ra, gvb[GKB ? jj : 0], 0u, stb + j * 1024);
    } else if ((q & 1) == 0) {
      dma16<LT>(L.ra, GATH == GATH_A ? a_gv(pos, jj, pure_c) : va[jj], a_so(k), stb + j * 1024);
    } else if (GATH == GATH_B) {
      dma16<LT>(L.rb, gvb[GKB ? jj : 0], 0u, stb + TILE_ELEMS * 2 + j * 1024);
    } else {
      i32x4 rbk;
      uint32_t so_b;
      b_src(L, k, rbk, so_b);
      dma16<LT>(rbk, vb[jj], so_b, stb + TILE_ELEMS * 2 + j * 1024);
    }
  };
  // L2 prefetch instruction o (0: A, 1: B) of ring position pos.
  auto pf_one = [&](int pos, int o, auto pure_c) __attribute__((always_inline)) {
    int k;
    const Ld L = pick(pos, k, pure_c);
    constexpr bool LT = LIGHT_K && decltype(pure_c)::value;  // as in dma_one
    if (o == 0 && GATH == GATH_AK) {
      touch4u(L.ra, gpb, __builtin_amdgcn_readfirstlane(0u), junk_lds);  // (a readfirstlane just before)
    } else if (o == 0) {
      touch4u<LT>(L.ra, L.pa, a_so(k), junk_lds);
    } else if (GATH == GATH_B) {
      touch4u(L.rb, gpb, __builtin_amdgcn_readfirstlane(0u), junk_lds);  // (a readfirstlane just before)
    } else {
      i32x4 rbk;
      uint32_t so_b;
      b_src(L, k, rbk, so_b);
      touch4u<LT>(rbk, L.pb, so_b, junk_lds);
    }
  };

  // ---- Gathered operands: token staging -------------------------------
  const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
  // GATH_A: tile it's tokens go to s_tok[it & 1]; wave w copies rows
  // 64w .. 64w+63 (rows past mlim read as 0 and are masked by glim).
  auto tok_dma_tile = [&](const Ld& L, int slot) __attribute__((always_inline)) {
    touch4(L.rt, (uint32_t)(wave * 64 + lane) * 4u, __builtin_amdgcn_readfirstlane(0u),
           reinterpret_cast<const uint32_t*>(&s_tok[slot & (GATH == GATH_A ? 1 : 0)][wave * 64]));
  };
  // GATH_A: the tile's A offsets and A prefetch offset from its tokens
  // (lane's rows 64w + 8jj + lane/8, and the prefetch sector's row pfe/2).
  auto tok_fill_tile = [&](Ld& L, int slot, uint32_t (&gv)[GATH == GATH_A ? NJ : 1], uint32_t& gs)
      __attribute__((always_inline)) {
    const int32_t* tk = s_tok[slot & (GATH == GATH_A ? 1 : 0)];
    if (F8) {  // the scale row of tile row 64 wave + lane
      const int row = wave * 64 + lane;
      gs = ((uint32_t)tk[row] * (uint32_t)p.sbytes) | (row < L.glim ? 0u : 0x80000000u);
    }
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
#pragma unroll
    for (int jj = 0; jj < (GATH == GATH_A ? NJ : 1); ++jj) {
      const int row = RPI * (wave * NJ + jj) + lane / CPR;
      const int c = (lane % CPR) ^ swz_k<BK>(row);
      // An invalid row gets bit 31 set, which puts it outside the resource
      // (the source is under 2 GiB); a select on the value instead would
      // make the compiler branch around the token read.
      gv[jj] = ((uint32_t)tk[row] * lda2 + c * 16) | (row < L.glim ? 0u : 0x80000000u);
    }
    constexpr int SPR = BK / 32;
    const int prow = L.pfe >= 0 ? L.pfe / SPR : 0;
    L.pa = ((uint32_t)tk[prow] * lda2 + (L.pfe % SPR) * 64) | (L.pfe >= 0 && prow < L.glim ? 0u : 0x80000000u);
  };
  // GATH_B, GATH_AK: ring position pos's 64 tokens go to s_tok[(gbase + pos) & 7];
  // every wave issues the copy (so that every wave counts the same memory
  // instructions) but only wave 0's lands in the ring.
  auto tok_dma_pos = [&](int pos) __attribute__((always_inline)) {
    int k;
    const Ld L = pick(pos, k, std::false_type());
    const uint32_t* dst = wave == 0 ? reinterpret_cast<const uint32_t*>(&s_tok[(gbase + pos) & 7][0]) : lds_junk;
    touch4(L.rt, (uint32_t)(k * BK + lane) * 4u, __builtin_amdgcn_readfirstlane(0u), dst);
  };
  // GATH_B, GATH_AK: the gathered operand's offsets of position pos into gvb, and the prefetch offset
  // of position ppos into gpb, from their tokens.
  auto tok_fill_pos = [&](int pos, int ppos) __attribute__((always_inline)) {
    int k;
    const Ld L = pick(pos, k, std::false_type());
    const int32_t* tk = s_tok[(gbase + pos) & 7];
    constexpr bool GA = GATH == GATH_AK;  // the gathered operand is A (its row pitch is lda)
#pragma unroll
    for (int jj = 0; jj < (GKB ? NJ : 1); ++jj) {
      const int krow = 2 * (wave * NJ + jj) + (lane >> 5);
      const int c = (lane & 31) ^ swz_mn(krow);
      gvb[jj] = ((uint32_t)tk[krow] * (GA ? lda2 : ldb2) + c * 16) | (k * BK + krow < L.glim ? 0u : 0x80000000u);
    }
    int kp;
    const Ld P = pick(ppos, kp, std::false_type());
    const int32_t* tp = s_tok[(gbase + ppos) & 7];
    const int pr = P.pfe >= 0 ? (P.pfe >> 3) : 0;
    gpb = ((uint32_t)tp[pr] * (GA ? lda2 : ldb2) + (P.pfe & 7) * 64) |
          (P.pfe >= 0 && kp * BK + pr < P.glim ? 0u : 0x80000000u);
  };

  f32x16 acc[MI][NI];
  // Fragment f (0 .. MI+NI-1) of k-step kk of a ring stage, in the order the
  // MFMAs (mi-major) first use them: A0, B0 .. B3, A1 .. A3.
  // F8 fragment (K-contiguous rows of codes): row row0 + lane%32, the 32
  // codes of 16-byte chunks 4 kk + 2 (lane/32) and the one after it, so that
  // the two lanes of a row cover the k-step's 64 codes (the two operands of
  // the instruction pair bytes the same way, measured on the MI355X).
  auto frag8 = [&](const uint16_t* S, int row0, int kk) __attribute__((always_inline)) -> i32x8f {
    const int r = row0 + (lane & 31);
    const int c0 = 4 * kk + 2 * (lane >> 5);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(S + r * BK + ((c0 ^ swz_k<BK>(r)) * 8));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(S + r * BK + (((c0 + 1) ^ swz_k<BK>(r)) * 8));
    const i32x8f v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return v;
  };
  auto read_frag = [&](const uint16_t* st, int kk, int f, Frag(&a)[MI], Frag(&b)[NI]) __attribute__((always_inline)) {
    static_assert(MI == 4 && NI == 4, "fragment order");
    if (f == 0 || f > NI) {
      const int mi = f == 0 ? 0 : f - NI;
      if constexpr (F8) a[mi] = frag8(st, wm * 128 + mi * 32, kk);
      else a[mi] = frag<BK, ALAY>(st, (HALFM ? arow : wm * 128) + mi * 32, kk, lane);
    } else {
      const int ni = f - 1;
      const int brow = DUAL ? (ni / 2) * 128 + wn * 64 + (ni % 2) * 32 : (HALFN ? bcol : wn * 128) + ni * 32;
      if constexpr (F8) b[ni] = frag8(st + TILE_ELEMS, brow, kk);
      else b[ni] = BQ8 ? frag_q8(st + TILE_ELEMS, brow, kk, lane) : frag<BK, BLAY>(st + TILE_ELEMS, brow, kk, lane);
    }
  };
  // F8: the E8M0 scale bytes of the wave's A rows and B columns for the k-tile
  // in use (sA, sB) and for the next one (nsA, nsB, read with its first
  // fragments): byte kb & 3 of each row's scale dword in stage st.  Byte mi
  // of sA is the scale of fragment row mi, byte ni of sB that of fragment
  // column ni; the instruction's op_sel picks the byte.
  uint32_t sA = 0, sB = 0, nsA = 0, nsB = 0;
  auto read_scales = [&](const uint16_t* st, int kb) __attribute__((always_inline)) {
    if constexpr (F8) {
      const uint8_t* sa = reinterpret_cast<const uint8_t*>(st) + SCA + (kb & 3);
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(st) + SCB + (kb & 3);
      uint32_t a = 0, b = 0;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) a |= (uint32_t)sa[(wm * 128 + mi * 32 + (lane & 31)) * 4] << (8 * mi);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int brow = DUAL ? (ni / 2) * 128 + wn * 64 + (ni % 2) * 32 : wn * 128 + ni * 32;
        b |= (uint32_t)sb[(brow + (lane & 31)) * 4] << (8 * ni);
      }
      nsA = a;
      nsB = b;
    }
  };
  // The block-scaled product of fragment row MI_ and column NI_ (op_sel must be a constant).
  auto mfma8 = [&](auto mi_c, auto ni_c, const Frag& a, const Frag& b, f32x16 c) __attribute__((always_inline)) {
    if constexpr (F8)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, decltype(mi_c)::value, (int)sA,
                                                            decltype(ni_c)::value, (int)sB);
    else
      return c;
  };
  // One k-step: the 16 MFMAs of fragments (a, b), with, in between, the
  // reads of the next k-step's fragments (stage rst, step rkk), ND DMA
  // instructions q0 .. q0+ND-1 of position dpos and then NP L2 prefetches of
  // position ppos, spread evenly.  The scheduling barriers pin this order, so
  // that the DMA issue never comes as a burst that would stall the wave's
  // MFMAs behind a full address queue.
  // (always_inline: out of line, the DMAs' scalar operands would arrive in
  // vector registers, which the instruction does not take)
  // (F8, NOREAD: the step reads no fragments - the last k-step of a tile,
  // whose successor reads its own after the epilogue)
  // (MIA, NIA: the wave's active row and column blocks - MI and NI, or 2 in
  // a half tile - whose MFMAs the step computes; RIA, RNIA: the blocks whose
  // next fragments it reads - the active ones, or all where the next step is
  // the next tile's)
  auto kstep = [&](auto nd_c, auto np_c, auto pure_c, const Frag(&a)[MI], const Frag(&b)[NI],
                   Frag(&na)[MI], Frag(&nb)[NI], const uint16_t* rst, int rkk, int dpos, int q0, int ppos,
                   auto noread_c, auto mia_c, auto ria_c, auto nia_c, auto rnia_c) __attribute__((always_inline)) {
    constexpr bool NOREAD = decltype(noread_c)::value;
    constexpr int MIA = decltype(mia_c)::value;
    constexpr int RIA = decltype(ria_c)::value;
    constexpr int NIA = decltype(nia_c)::value;
    constexpr int RNIA = decltype(rnia_c)::value;
    constexpr int ND = decltype(nd_c)::value;
    constexpr int NO = ND + decltype(np_c)::value;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mi = i / NI, ni = i % NI;
      if constexpr (F8) {
        switch (i) {  // (i is a constant once the loop is unrolled)
#define MOE_F8_CASE(I) \
  case I: acc[I / NI][I % NI] = mfma8(std::integral_constant<int, I / NI>(), std::integral_constant<int, I % NI>(), \
                                     a[I / NI], b[I % NI], acc[I / NI][I % NI]); break;
          MOE_F8_CASE(0) MOE_F8_CASE(1) MOE_F8_CASE(2) MOE_F8_CASE(3) MOE_F8_CASE(4) MOE_F8_CASE(5)
          MOE_F8_CASE(6) MOE_F8_CASE(7) MOE_F8_CASE(8) MOE_F8_CASE(9) MOE_F8_CASE(10) MOE_F8_CASE(11)
          MOE_F8_CASE(12) MOE_F8_CASE(13) MOE_F8_CASE(14) MOE_F8_CASE(15)
#undef MOE_F8_CASE
        }
        // The next step's fragment of a row once this step's row is done, of
        // a column after its last use (mi = 3): each then takes the registers
        // of the one it replaces, so that about 9 rather than 16 fragments of
        // 32 bytes are live at once.
        if (!NOREAD && ni == NI - 1) read_frag(rst, rkk, mi == 0 ? 0 : NI + mi, na, nb);
        if (!NOREAD && mi == MI - 1) read_frag(rst, rkk, 1 + ni, na, nb);
      } else {
        if (mi < MIA && ni < NIA)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
        // (fragment f: a[0], then b[0..NI-1], then a[1..MI-1])
        if ((i & 1) == 0 && (i >> 1) < MI + NI &&
            ((i >> 1) == 0 || ((i >> 1) <= NI ? (i >> 1) - 1 < RNIA : (i >> 1) - NI < RIA)))
          read_frag(rst, rkk, i >> 1, na, nb);
      }
#pragma unroll
      for (int o = (i * NO) / 16; o < ((i + 1) * NO) / 16; ++o) {
        if (o < ND) dma_one(dpos, q0 + o, pure_c);
        else pf_one(ppos, o - ND, pure_c);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Per k-tile kt: step 0 issues the second half of position kt+1 (except
  // for the first k-tile, whose position 1 is issued whole beforehand) and
  // the prefetch of position kt+1+PFD; steps 1 .. KS-2 only compute; then
  // position kt+1 is waited for (one barrier per k-tile); the last step reads
  // position kt+1's first fragments and issues the first half of position
  // kt+2 (the last k-tile issues it whole, before the epilogue).
  constexpr int PER = BQ8 ? NJ + NJB + 1 : 2 * NJ + (F8 ? 2 : 0);  // DMA instructions per wave per ring position
  constexpr int PART = PER / 2;                      // first part; the second has PER - PART
  constexpr int PFD = 1;  // (measured: 1 beats 2 and 3 by 1-2% on the 1T shapes; for F8, 2 is within noise)
  // Memory instructions per lane of one epilogue (the buffer stores and
  // loads below, all unconditional).
  // (ROWSC: dH scaled per row, with the scales loaded and h_out and the rows'
  // partial dot products stored: 32 more of each.)
  constexpr bool ROWSC = EPI == EPI_SWIGLU_BWD && GATH == GATH_A;
  constexpr int EPI_OPS = (EPI == EPI_SWIGLU) ? 48 : (EPI == EPI_SWIGLU_BWD) ? (ROWSC ? 224 : 128)
                          : (EPI == EPI_ADD ? 2 : 1) * (CF32 ? 64 : 32);
  // (+1: a gathered operand's token copy is issued between the epilogue and
  // the prefetches.)
  constexpr int FIRST_OPS = EPI_OPS + NPF + (GATH != 0 ? 1 : 0);
  constexpr int FIRST_N_PRIMED = FIRST_OPS > 63 ? 63 : FIRST_OPS;
  using N0 = std::integral_constant<int, 0>;
  using NDP = std::integral_constant<int, PART>;
  using NDP1 = std::integral_constant<int, PER - PART>;
  using NDF = std::integral_constant<int, PER>;
  using NPP = std::integral_constant<int, NPF>;
  Frag fa[2][MI], fb[2][NI];

  // Dynamic order: the claim issued at the top of tile it resolves to tile
  // it+2's id, stored where the top of tile it+1 reads it.  k-tile pub_kt
  // publishes an own-queue claim once its wait has passed (the atomic has long
  // returned by then); the tile's end publishes whatever is left (the tail,
  // or a tile without that k-tile).  pub_kt is opaque to the compiler, which
  // would otherwise peel that k-tile into a copy of its own.
  const int pub_kt = dyn ? __builtin_amdgcn_readfirstlane(p.ngroups >= 0 ? 1 : 2) : -1;
  auto publish_own = [&]() __attribute__((always_inline)) {
    if (w0 && pstate == 1) {
      const int c = q_tile(x0, __builtin_amdgcn_readfirstlane(pend));
      if (c < sched.total) {
        s_q[it & 1] = c;
        pstate = 0;
      } else {
        exhausted |= 1 << x0;
        pstate = 2;
      }
    }
  };
  auto publish = [&]() __attribute__((always_inline)) {
    if (w0 && pstate != 0) {
      s_q[it & 1] = resolve(pstate == 1 ? __builtin_amdgcn_readfirstlane(pend) : PEND_NONE);
      pstate = 0;
    }
  };

  // GATH_A: the next tile's load state (its A offsets are filled from its
  // tokens at k-tile gat_kt, opaque to the compiler for the reason above),
  // and whether that has happened.
  Ld lnext = null_ld;
  bool pipe = false, gat_done = true;
  const int gat_kt = GATH == GATH_A ? __builtin_amdgcn_readfirstlane(p.ngroups >= 0 ? 1 : 2) : -1;
  auto gat_fill_next = [&]() __attribute__((always_inline)) {
    if (!gat_done) {
      tok_fill_tile(lnext, it + 1, gnext, gsn);
      if (pipe) nxt.pa = lnext.pa;
      gat_done = true;
    }
  };

  // PURE: every position the k-tile loads (kt+1 .. kt+1+PFD) is the current tile's.
  auto ktile = [&](int kt, auto first_c, auto last_c, auto pure_c, auto mia_c, auto nia_c) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    using PU = decltype(pure_c);
    using MIA = decltype(mia_c);
    using NIA = decltype(nia_c);
    const uint16_t* st = ring[(uint32_t)(gbase + kt) % STAGES];
    if constexpr (F8) {  // this k-tile's scales, read with its first fragments
      sA = nsA;
      sB = nsB;
    }
    // GATH_B: the tokens of position kt+3+PFD (read two k-tiles later, after the
    // barriers that follow their wait).
    if (GKB) tok_dma_pos(kt + 3 + PFD);
#pragma unroll
    for (int s = 0; s < KS - 1; ++s) {
      if (s == 0) {
        if (FIRST)
          kstep(N0(), NPP(), PU(), fa[0], fb[0], fa[1], fb[1], st, 1, 0, 0, kt + 1 + PFD, std::false_type(), MIA(),
                MIA(), NIA(), NIA());
        else
          kstep(NDP1(), NPP(), PU(), fa[0], fb[0], fa[1], fb[1], st, 1, kt + 1, PART, kt + 1 + PFD,
                std::false_type(), MIA(), MIA(), NIA(), NIA());
        // GATH_B: position kt+1 is issued whole; its offsets make way for
        // those of kt+2 (issued at this k-tile's end and the next's start),
        // and the prefetch offset for kt+2+PFD (next k-tile's prefetch).
        if (GKB) tok_fill_pos(kt + 2, kt + 2 + PFD);
      } else {
        kstep(N0(), N0(), PU(), fa[s & 1], fb[s & 1], fa[(s + 1) & 1], fb[(s + 1) & 1], st, s + 1, 0, 0, 0,
              std::false_type(), MIA(), MIA(), NIA(), NIA());
      }
    }
    // Position kt+1 has landed: after its last DMA come only its prefetches,
    // or, for a first k-tile primed by the previous tile, that tile's
    // epilogue and then the prefetches.
    if (FIRST && primed) wait_vm<FIRST_N_PRIMED>();
    else wait_vm<NPF>();
    if (!FIRST && kt == pub_kt) publish_own();
    lds_barrier();
    // GATH_A: the next tile's tokens (copied at this tile's top, waited for
    // by now in every wave) give its A offsets.
    if (GATH == GATH_A && !FIRST && kt == gat_kt) gat_fill_next();
    const uint16_t* nst = ring[(uint32_t)(gbase + kt + 1) % STAGES];
    if (F8 && !LAST) {  // the scales of position kt+1 (its k-tile index picks the byte)
      int kn;
      pick(kt + 1, kn, PU());
      read_scales(nst, kn);
    }
    // (F8: the last k-tile leaves the next tile's first fragments and scales
    // to be read after the epilogue, so they are not live through it)
    using NR = std::integral_constant<bool, F8 && LAST>;
    if (LAST) {
      // (this step reads the next tile's first fragments: at that tile's A
      // rows, and all its row blocks, for a full tile may follow a half one)
      if constexpr (HALFM) arow = arow_next;
      if constexpr (HALFN) bcol = bcol_next;
      kstep(NDF(), N0(), PU(), fa[1], fb[1], fa[0], fb[0], nst, 0, kt + 2, 0, 0, NR(), MIA(),
            std::integral_constant<int, MI>(), NIA(), std::integral_constant<int, NI>());
    } else {
      kstep(NDP(), N0(), PU(), fa[1], fb[1], fa[0], fb[0], nst, 0, kt + 2, 0, 0, NR(), MIA(), MIA(), NIA(), NIA());
    }
  };

  // Epilogue resources: C (or C2 for rows past msplit) from the tile's
  // corner, with rows [0, mlim) in range; per-lane offsets of columns past
  // nlim lie outside.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  auto c_rsrc = [&](const void* base, int64_t ld_elems, int esz) -> __amdgpu_buffer_rsrc_t {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)((int64_t)t.mlim * ld_elems * esz), 0x00020000);
  };

  if (GATH == GATH_A) {  // the first tile's A offsets, from its tokens
    tok_dma_tile(cur, 0);
    wait_vm<0>();
    lds_barrier();
    tok_fill_tile(cur, 0, gcur, gsc);
  }
  for (;;) {
    // The next tile of this workgroup, loaded ahead if it is long enough.
    int idn;
    bool has_next;
    if (dyn) {
      lds_barrier();  // s_q[(it+1)&1] was published before it; s_q[it&1] has been read by every wave
      idn = __builtin_amdgcn_readfirstlane(s_q[(it + 1) & 1]);
      has_next = idn < sched.total;
      if (w0 && has_next) {  // tile it+2, published into s_q[it&1]
        pend = claim_own();
        pstate = ((exhausted >> x0) & 1) ? 2 : 1;
      }
    } else {
      idn = xcd_tile(it + 1, gridDim.x);
      has_next = (it + 1) * (int)gridDim.x < sched.total && idn < sched.total;
    }
    TileCtx tn = t;
    lnext = null_ld;
    if (has_next) {
      tn = sched.template tile<!DYN>(p, s_pref, idn);
      lnext = setup(tn);
      if (GATH == GATH_A) {
        tok_dma_tile(lnext, it + 1);
        gat_done = false;
      }
    }
    // (A gathered operand: the next tile's A offsets are ready at k-tile 1
    // (GATH_A), and token copies run five positions ahead (GATH_B), which
    // must not reach past the next tile; so only a tile of five k-tiles or
    // more hands over early.)
    pipe = has_next && lnext.nk >= STAGES && cur.nk >= (GATH != 0 ? 5 : 1);
    nxt = pipe ? lnext : null_ld;
    // Half tiles: this tile's A row base, and the next tile's, at which the
    // last k-step reads its first fragments when it is loaded ahead.  (When
    // this tile was loaded ahead, its first fragments were read at the
    // arow_next set here one tile earlier, for the same tile.)
    const bool half = HALFM && t.mlim <= 128;
    if constexpr (HALFM) {
      arow = half ? wm * 64 : wm * 128;
      arow_next = (pipe && tn.mlim <= 128) ? wm * 64 : wm * 128;
    }
    const bool halfn = HALFN && t.nlim <= 128;
    if constexpr (HALFN) {
      bcol = halfn ? wn * 64 : wn * 128;
      bcol_next = (pipe && tn.nlim <= 128) ? wn * 64 : wn * 128;
    }

#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (cur.nk > 0) {
      if (!primed) {
        if (GKB) {  // tokens of positions 0 .. 2+PFD
#pragma unroll
          for (int q = 0; q < 3 + PFD; ++q) tok_dma_pos(q);
          wait_vm<0>();
          lds_barrier();
          tok_fill_pos(0, PFD);
        }
        // Positions 0 and 1 whole, with position 0's prefetch in between.
#pragma unroll
        for (int q = 0; q < PER; ++q) dma_one(0, q, std::false_type());
#pragma unroll
        for (int o = 0; o < NPF; ++o) pf_one(PFD, o, std::false_type());
        if (GKB) tok_fill_pos(1, PFD + 1);
#pragma unroll
        for (int q = 0; q < PER; ++q) dma_one(1, q, std::false_type());
        wait_vm<PER + NPF>();  // position 0 has landed (then come its prefetch and position 1)
        lds_barrier();
#pragma unroll
        for (int f = 0; f < MI + NI; ++f) read_frag(ring[(uint32_t)gbase % STAGES], 0, f, fa[0], fb[0]);
        read_scales(ring[(uint32_t)gbase % STAGES], 0);
      } else if (F8) {  // primed: position 0 has landed (waited for before the previous tile's last step)
#pragma unroll
        for (int f = 0; f < MI + NI; ++f) read_frag(ring[(uint32_t)gbase % STAGES], 0, f, fa[0], fb[0]);
        read_scales(ring[(uint32_t)gbase % STAGES], 0);
      }
      using T_ = std::true_type;
      using F_ = std::false_type;
      auto kloop = [&](auto mia_c, auto nia_c) __attribute__((always_inline)) {
        if (cur.nk == 1) {
          ktile(0, T_(), T_(), F_(), mia_c, nia_c);
        } else {
          ktile(0, T_(), F_(), F_(), mia_c, nia_c);
          // k-tiles whose positions kt+1 .. kt+1+PFD are all the current tile's
          const int pure_end = max(1, cur.nk - 1 - PFD);
          for (int kt = 1; kt < pure_end; ++kt) ktile(kt, F_(), F_(), T_(), mia_c, nia_c);
          for (int kt = pure_end; kt < cur.nk - 1; ++kt) ktile(kt, F_(), F_(), F_(), mia_c, nia_c);
          ktile(cur.nk - 1, F_(), T_(), F_(), mia_c, nia_c);
        }
      };
      using IMI = std::integral_constant<int, MI>;
      using INI = std::integral_constant<int, NI>;
      using I2 = std::integral_constant<int, 2>;
      if (HALFM && half) kloop(I2(), INI());
      else if (HALFN && halfn) kloop(IMI(), I2());
      else kloop(IMI(), INI());
    }

    // Epilogue.  Each wave stages its 32 x 128 block acc[mi] eight rows at a
    // time (rows s*8 .. s*8+7 hold acc[mi][ni][4s .. 4s+3]) in its own LDS
    // area and reads them back as row vectors of W columns (16 bytes of
    // output: 8 bf16 or 4 float), so that consecutive lanes store
    // consecutive 16-byte pieces of a row.  A wave's LDS accesses complete
    // in order and the areas are disjoint, so no barrier is needed.
    //   acc[mi][ni][r] is C[row][col] with
    //   row = wm*128 + mi*32 + (r/4)*8 + (lane/32)*4 + r%4, col = n-block base + lane%32.
    {
      // The epilogue's lane-dependent offsets are recomputed here from an
      // opaque copy of the lane index: hoisted out of the tile loop they
      // would stay live across the k-loop and be spilled.
      int lane_e = lane;
      asm volatile("" : "+v"(lane_e));
      float* stage = s_stage[wave];
      constexpr int OC = DUAL ? WC / 2 : WC;
      constexpr bool PLAIN = EPI == EPI_STORE || EPI == EPI_ADD;
      // A bias is only taken by plain ungrouped products (the router's logits).
      constexpr bool HAS_BIAS = GRP == GRP_NONE && EPI == EPI_STORE;
      constexpr int W = (PLAIN && CF32) ? 4 : 8;
      constexpr int CPR = OC / W;               // vectors per row
      constexpr int VPL = 8 * CPR / 64;          // vectors per lane_e per slab
      static_assert(8 * CPR % 64 == 0, "whole vectors per lane_e");
      // (a half-N tile's wave column covers 64 columns; its vectors past them,
      // from the inactive column blocks, are masked below)
      const int col_base = DUAL ? wn * 64 : (HALFN && halfn) ? wn * 64 : wn * 128;
      const int cvlim = (HALFN && halfn) ? 64 : OC;
      // Resources (row 0 = the tile's first row, element 0 = its first column).
      const int64_t m0g = t.m0;
      __amdgpu_buffer_rsrc_t r0, r1;
      int64_t ldo = p.ldc;
      if (PLAIN) {
        const int esz = CF32 ? 4 : 2;
        char* cb = reinterpret_cast<char*>(p.C);
        char* cb2 = reinterpret_cast<char*>(p.C2);
        const int64_t gof = (GRP == GRP_K) ? (int64_t)t.g * p.c_gstride : 0;
        r0 = c_rsrc(cb + ((m0g * p.ldc + t.n0 + gof) * esz), p.ldc, esz);
        // C2 rows start at msplit: row r of the tile is C2 row m0 + r - msplit.
        r1 = p.msplit ? c_rsrc(cb2 + (((m0g - p.msplit) * p.ldc + t.n0 + gof) * esz), p.ldc, esz) : r0;
      } else if (EPI == EPI_SWIGLU) {
        // h [rows][N] in C; G | U [rows][2N] in gu_out (if saved).
        r0 = c_rsrc(reinterpret_cast<char*>(p.C) + (m0g * p.ldc + t.n0) * 2, p.ldc, 2);
        char* gub = reinterpret_cast<char*>(p.gu_out);
        const int64_t ld2 = 2 * (int64_t)p.N;
        r1 = gub ? c_rsrc(gub + (m0g * ld2 + t.n0) * 2, ld2, 2)
                 : __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(p.C), (short)0, 0, 0x00020000);
        ldo = ld2;
      } else {
        // dG | dU [rows][2N] in C, from dH and G | U [rows][2N] in gu_in.
        const int64_t ld2 = 2 * (int64_t)p.N;
        r0 = c_rsrc(reinterpret_cast<char*>(p.C) + (m0g * ld2 + t.n0) * 2, ld2, 2);
        r1 = c_rsrc(const_cast<char*>(reinterpret_cast<const char*>(p.gu_in)) + (m0g * ld2 + t.n0) * 2, ld2, 2);
        ldo = ld2;
      }
      // ROWSC: the rows' scales (float), h_out ([rows][N] bf16, or nothing) and
      // the rows' partial dot products ([rows][NP] float, or nothing).
      __amdgpu_buffer_rsrc_t rsc = r0, rho = r0, rdw = r0;
      const int NP = 2 * sched.NT;
      if (ROWSC) {
        rsc = c_rsrc(const_cast<float*>(p.row_scale) + m0g, 1, 4);
        rho = p.h_out ? c_rsrc(reinterpret_cast<char*>(p.h_out) + (m0g * p.N + t.n0) * 2, p.N, 2)
                      : __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(p.C), (short)0, 0, 0x00020000);
        rdw = p.dw_part ? c_rsrc(p.dw_part + m0g * NP, NP, 4)
                        : __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(p.C), (short)0, 0, 0x00020000);
      }
      // Values the epilogue reads are loaded in batches ahead of the stores
      // that use them: a load waits for every memory instruction issued
      // before it, so each batch costs one round trip after the previous
      // batch's stores. EPI_ADD: the old C values of two 32-row blocks (one
      // for fp32 C, whose two would not fit in registers). EPI_SWIGLU_BWD: G
      // and U (and the row scales) of one 8-row slab, two slabs ahead of its
      // use, in a window of three (load_gu below).
      constexpr int AB = VPL <= 2 ? 2 : 1;
      u32x4_t oldc[AB][4][VPL];
      u32x4_t gup[3][VPL][2];
      uint32_t rsv[3][VPL];
      // Rows 8 sl .. 8 sl + 7 of the wave's 32-row block mi, as fp32, into the
      // wave's staging area.
      auto stage_slab = [&](int mi_, int sl_) __attribute__((always_inline)) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            stage[((lane_e >> 5) * 4 + r4) * SP + ni * 32 + (lane_e & 31)] = acc[mi_][ni][sl_ * 4 + r4];
      };
      // EPI_SWIGLU_BWD: G and U (ROWSC: and the rows' scales) of slab j = 4 mi
      // + sl into gup[j % 3], issued two slabs before slab j is stored.  Their
      // wait then covers the stores of slab j - 2 and earlier, which have had
      // two slabs' time to drain, not those of slab j - 1 (with a batch per
      // 32-row block, each batch waited for the previous block's stores and
      // then made a round trip of its own).
      auto load_gu = [&](int j) __attribute__((always_inline)) {
        const int mi_ = j >> 2, sl_ = j & 3;
        const int rowb_ = (HALFM && half) ? (mi_ < 2 ? wm * 64 + mi_ * 32 : 256 + mi_ * 32) : wm * 128 + mi_ * 32;
#pragma unroll
        for (int vi = 0; vi < VPL; ++vi) {
          const int e = lane_e + vi * 64;
          const int rl = e / CPR, cv = (e % CPR) * W;
          const int row = rowb_ + sl_ * 8 + rl, col = col_base + cv;
          const int64_t eo = (int64_t)row * ldo + col;
          const bool ok = col < t.nlim;
          gup[j % 3][vi][0] = __builtin_amdgcn_raw_buffer_load_b128(r1, ok ? (uint32_t)(eo * 2) : 0x80000000u, 0, 0);
          gup[j % 3][vi][1] =
              __builtin_amdgcn_raw_buffer_load_b128(r1, ok ? (uint32_t)((eo + p.N) * 2) : 0x80000000u, 0, 0);
          if (ROWSC) rsv[j % 3][vi] = __builtin_amdgcn_raw_buffer_load_b32(rsc, (uint32_t)row * 4u, 0, 0);
        }
      };
      if (EPI == EPI_SWIGLU_BWD) {
        load_gu(0);
        load_gu(1);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        // the block's first row in the tile (a half tile's inactive blocks 2
        // and 3 are placed past its 256 rows, where every access is out of
        // range; arow already holds the next tile's base here)
        const int rowb = (HALFM && half) ? (mi < 2 ? wm * 64 + mi * 32 : 256 + mi * 32) : wm * 128 + mi * 32;
        // Rows of this block lie on one side of msplit (a multiple of 32).
        const bool side2 = PLAIN && p.msplit && m0g + rowb >= p.msplit;
        if (EPI == EPI_ADD && mi % AB == 0) {
#pragma unroll
          for (int m2 = 0; m2 < AB; ++m2) {
            const int rowb2 = rowb + m2 * 32;
            const bool side2b = p.msplit && m0g + rowb2 >= p.msplit;
#pragma unroll
            for (int sl = 0; sl < 4; ++sl)
#pragma unroll
              for (int vi = 0; vi < VPL; ++vi) {
                const int e = lane_e + vi * 64;
                const int rl = e / CPR, cv = (e % CPR) * W;
                const int row = rowb2 + sl * 8 + rl, col = col_base + cv;
                const int64_t eo = (int64_t)row * ldo + col;
                oldc[m2][sl][vi] = __builtin_amdgcn_raw_buffer_load_b128(
                    side2b ? r1 : r0, col < t.nlim && cv < cvlim ? (uint32_t)(eo * (CF32 ? 4 : 2)) : 0x80000000u, 0,
                    0);
              }
          }
        }
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          if (EPI == EPI_SWIGLU_BWD && mi * 4 + sl + 2 < MI * 4) load_gu(mi * 4 + sl + 2);
          if (mi == 0 && sl == 0) stage_slab(0, 0);  // later slabs are staged one ahead, below
          float vv[VPL][W], vv2[VPL][W];
#pragma unroll
          for (int vi = 0; vi < VPL; ++vi) {
            const int e = lane_e + vi * 64;
            const int rl = e / CPR, cv = (e % CPR) * W;
#pragma unroll
            for (int q = 0; q < W; ++q) {
              vv[vi][q] = stage[rl * SP + cv + q];
              vv2[vi][q] = DUAL ? stage[rl * SP + OC + cv + q] : 0.f;
            }
          }
          // Stage the next slab now: a wave's LDS operations run in order, so
          // these writes land after the reads above, and they issue while the
          // reads return and this slab is converted and stored.  The reads
          // and writes pass values between lanes, which the compiler does not
          // see as a dependence: empty asm with a memory clobber on both sides
          // keeps it from moving either across the other (a staging written by
          // half of the lanes has been reordered without it).
          asm volatile("" ::: "memory");
          if (sl < 3)
            stage_slab(mi, sl + 1);
          else if (mi + 1 < MI)
            stage_slab(mi + 1, 0);
          asm volatile("" ::: "memory");
#pragma unroll
          for (int vi = 0; vi < VPL; ++vi) {
            const int e = lane_e + vi * 64;
            const int rl = e / CPR, cv = (e % CPR) * W;
            float v[W], v2[W];
#pragma unroll
            for (int q = 0; q < W; ++q) {
              v[q] = vv[vi][q];
              v2[q] = vv2[vi][q];
            }
            const int row = rowb + sl * 8 + rl;  // row in the tile
            const int col = col_base + cv;       // column in the tile
            const bool ok = col < t.nlim && cv < cvlim;
            const int64_t eo = (int64_t)row * ldo + col;  // element offset from the corner
            if (PLAIN) {
              const __amdgpu_buffer_rsrc_t rc = side2 ? r1 : r0;
              if (CF32) {
                float o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = v[q];
                if (HAS_BIAS && p.bias) {
#pragma unroll
                  for (int q = 0; q < 4; ++q) o[q] += ok ? p.bias[t.n0 + col + q] : 0.f;
                }
                if (EPI == EPI_ADD) {
                  u32x4_t old = oldc[mi % AB][sl][vi];
                  asm volatile("" : "+v"(old));  // used here, not hoisted to its load
#pragma unroll
                  for (int q = 0; q < 4; ++q) o[q] += __uint_as_float(old[q]);
                }
                const u32x4_t d = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                   __float_as_uint(o[3])};
                // (weight gradients, written once and not read in this pass:
                // non-temporal stores)
                __builtin_amdgcn_raw_buffer_store_b128(d, rc, ok ? (uint32_t)(eo * 4) : 0x80000000u, 0,
                                                       GRP == GRP_K ? 2 : 0);
              } else {
                float o[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) o[q] = v[q];
                if (HAS_BIAS && p.bias) {
#pragma unroll
                  for (int q = 0; q < 8; ++q) o[q] += ok ? p.bias[t.n0 + col + q] : 0.f;
                }
                if (EPI == EPI_ADD) {
                  u32x4_t old = oldc[mi % AB][sl][vi];
                  asm volatile("" : "+v"(old));  // used here, not hoisted to its load
#pragma unroll
                  for (int q = 0; q < 8; ++q)
                    o[q] += __uint_as_float((q & 1) ? (old[q >> 1] & 0xffff0000u) : (old[q >> 1] << 16));
                }
                const u32x4_t d = {pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]),
                                   pack_bf2(o[6], o[7])};
                // (bf16 weight gradients: non-temporal as their fp32 form)
                __builtin_amdgcn_raw_buffer_store_b128(d, rc, ok ? (uint32_t)(eo * 2) : 0x80000000u, 0,
                                                       GRP == GRP_K ? 2 : 0);
              }
            } else if (EPI == EPI_SWIGLU) {
              float h[8];
#pragma unroll
              for (int q = 0; q < 8; ++q) h[q] = v[q] * sigmoidf_(v[q]) * v2[q];
              const u32x4_t dh = {pack_bf2(h[0], h[1]), pack_bf2(h[2], h[3]), pack_bf2(h[4], h[5]), pack_bf2(h[6], h[7])};
              const u32x4_t dg = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
              const u32x4_t du = {pack_bf2(v2[0], v2[1]), pack_bf2(v2[2], v2[3]), pack_bf2(v2[4], v2[5]),
                                  pack_bf2(v2[6], v2[7])};
              const int64_t eh = (int64_t)row * p.ldc + col;
              __builtin_amdgcn_raw_buffer_store_b128(dh, r0, ok ? (uint32_t)(eh * 2) : 0x80000000u, 0, 0);
              // (G | U is read back only by the backward: non-temporal stores)
              __builtin_amdgcn_raw_buffer_store_b128(dg, r1, ok ? (uint32_t)(eo * 2) : 0x80000000u, 0, 2);
              __builtin_amdgcn_raw_buffer_store_b128(du, r1, ok ? (uint32_t)((eo + p.N) * 2) : 0x80000000u, 0, 2);
            } else {  // EPI_SWIGLU_BWD: v = dH
              const uint32_t og = ok ? (uint32_t)(eo * 2) : 0x80000000u;
              const uint32_t ou = ok ? (uint32_t)((eo + p.N) * 2) : 0x80000000u;
              u32x4_t gq = gup[(mi * 4 + sl) % 3][vi][0];
              u32x4_t uq = gup[(mi * 4 + sl) % 3][vi][1];
              asm volatile("" : "+v"(gq), "+v"(uq));  // used here, not hoisted to their loads
              float sc = 1.0f;
              if (ROWSC) {
                uint32_t sw = rsv[(mi * 4 + sl) % 3][vi];
                asm volatile("" : "+v"(sw));
                sc = __uint_as_float(sw);
              }
              float dg[8], du[8], hs[8];
              float dot = 0.f;  // ROWSC: sum over the vector of unscaled dH * silu(G) U
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const uint32_t gw = gq[q >> 1], uw = uq[q >> 1];
                const float g = __uint_as_float((q & 1) ? (gw & 0xffff0000u) : (gw << 16));
                const float u = __uint_as_float((q & 1) ? (uw & 0xffff0000u) : (uw << 16));
                const float sg = sigmoidf_(g);
                const float dh = ROWSC ? v[q] * sc : v[q];
                du[q] = dh * g * sg;
                dg[q] = dh * u * sg * (1.0f + g * (1.0f - sg));
                hs[q] = g * sg * u * sc;
                if (ROWSC) dot = fmaf(v[q], g * sg * u, dot);
              }
              if (ROWSC) {
                // The row's CPR = 16 vectors are held by 16 consecutive lanes:
                // a butterfly over them, and the first of them writes the sum
                // over this wave's 128 columns (rows past mlim fall outside rdw).
                static_assert(!ROWSC || CPR == 16, "one row per 16 lanes");
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 16);
                // (issued by every lane, so the epilogue's store count stays fixed;
                // the other lanes' offsets lie outside rdw)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(dot), rdw,
                    (lane_e & 15) == 0 ? (uint32_t)(row * NP + 2 * t.ntile + wn) * 4u : 0x80000000u, 0, 0);
                const u32x4_t dhw = {pack_bf2(hs[0], hs[1]), pack_bf2(hs[2], hs[3]), pack_bf2(hs[4], hs[5]),
                                     pack_bf2(hs[6], hs[7])};
                const int64_t eh = (int64_t)row * p.N + col;
                __builtin_amdgcn_raw_buffer_store_b128(dhw, rho, ok ? (uint32_t)(eh * 2) : 0x80000000u, 0, 0);
              }
              const u32x4_t ddg = {pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]), pack_bf2(dg[4], dg[5]),
                                   pack_bf2(dg[6], dg[7])};
              const u32x4_t ddu = {pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]), pack_bf2(du[4], du[5]),
                                   pack_bf2(du[6], du[7])};
              __builtin_amdgcn_raw_buffer_store_b128(ddg, r0, og, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(ddu, r0, ou, 0, 0);
            }
          }
        }
      }
    }

    if (dyn) publish();  // a tile without a k-tile 1 publishes here
    if (GATH == GATH_A && !gat_done) {  // a tile without a k-tile 1: wait for the next tile's tokens here
      wait_vm<0>();
      lds_barrier();
      gat_fill_next();
    }
    // Advance to the next tile.
    gbase += cur.nk;
    ++it;
    if (!has_next) break;
    t = tn;
    cur = pipe ? nxt : lnext;
    if (GATH == GATH_A) {
#pragma unroll
      for (int jj = 0; jj < (GATH == GATH_A ? NJ : 1); ++jj) gcur[jj] = gnext[jj];
      gsc = gsn;
    }
    primed = pipe;
  }
  wait_vm<0>();  // no LDS DMA may land after the workgroup ends
  dyn_finish();
}

}  // namespace moe
