// Grouped expert GEMMs and the weighted combine of the sparse MoE layer
// (gfx950, wave64, bf16 MFMA with fp32 accumulation).
//
// "Optimizing on-device inference for Apple Silicon" (Perplexity 2026):
//  - section "Dequantize weights during matrix multiplication": the grouped
//    GEMM stages one small weight tile at a time in on-chip memory, multiplies
//    it with the routed activation rows, accumulates in fp32, writes bf16;
//  - section "Match tile size to expert load": output tiles map to
//    workgroups, and the tile height must suit the uneven rows per expert;
//  - section "Reduce intermediate and state traffic": the two input
//    projections go with their gated activation (one kernel here: gate and
//    up tiles share the A rows and SwiGLU runs on the accumulators), the
//    output projection goes with its routing score and the shared expert.
//
// Tile: up to 256 rows of one expert group (eight 32-row blocks), or 288
// for a group's last tile (a ninth block holding the group's last 1..32
// rows past a multiple of 256), x 256 weight rows, one 8-wave workgroup per CU (two waves per SIMD: the LDS
// serves one wave's operand reads about half as fast as two waves', and one
// wave's stalls hide behind the other's MFMAs).  Weights and the gathered
// activation rows (rows of a routed group through the scatter permutation,
// never copied) travel straight from global memory into LDS rings by
// global->LDS transfers, 8 rows x 128 bytes per instruction, each weight byte
// once per tile; a wave computes up to 128 rows x 64 columns (128 fp32
// accumulator registers).  With tiles of 256 rows (288 for a group's last)
// an expert's weights are read once whenever it has at most 288 rows (all
// experts at near-uniform routing, most of them on 8192-token chunks).  The
// number of 32-row blocks is a template parameter chosen per
// tile, so the inner loop has no branches and row blocks past the group's
// rows cost nothing.
//
// Launch order is XCD-aware: workgroup b runs on XCD b % 8; the tiles are
// dealt to the XCDs round-robin and the panels of a tile stay on one XCD,
// so its activation rows are re-read from that XCD's L2.  The gate/up launch
// takes the tiles in the order the routing scan lists them for it (most
// 32-row blocks first: the longest units start first and the short ones
// fill the end), the down launch the block map from its end.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 256;   // rows per tile (= kTileM)
constexpr int WN = 64;    // weight rows per wave
constexpr int NWR = 256;  // weight rows per workgroup
static_assert(BM == kTileM, "block map tile height");

struct GemmArgs {
  const uint16_t* a_x;    // gate/up: token rows [M][H]
  const uint16_t* a_r;    // down: routed h rows [A][I]
  const uint16_t* a_s;    // down: shared h rows [M][Is]
  const uint16_t* expert_w;
  const uint16_t* shared_w;
  const int32_t* perm;
  const Tile* tiles;
  const int32_t* ntiles;
  const uint32_t* ex_codes;   // 4-bit weights (Q4 kernels): codes, 8 per word
  const uint32_t* ex_groups;  // (scale, bias) per 64 elements
  const uint32_t* sh_codes;
  const uint32_t* sh_groups;
  uint16_t* out_r;
  uint16_t* out_s;
  const uint16_t* y_r;  // MODE 2: the routed experts' output rows (group order) to combine
  const float* w;       // MODE 2: routing weights [M][k]
  const int32_t* inv;   // MODE 2: group position of each assignment [M*k]
  uint16_t* out;        // MODE 2: the layer's output [M][H]
  int skip_tail;        // tiles at the end of the block map left out (the shared expert's, done elsewhere)
  int sgu_units;        // MODE 1: leading workgroups that run the shared expert's gate/up tiles
  int sgu_npan;         // MODE 1: gate/up panels of the shared expert
  int64_t M;
  int H, E, I, Is, k;
  int npan;
  int max_tiles;
  int tiled;  // weights in the tiled layout: a panel's K-step is one block (bf16: the stage image)
};

constexpr int BK = 64;        // K per pipeline step
constexpr int CPR = BK / 8;   // 16-byte chunks per row per step
constexpr int KK = BK / 16;   // MFMA sub-steps per step
constexpr int SA = BM * CPR;  // activation stage: BM rows x BK, 16-byte units (32 KB)
constexpr int SB = NWR * CPR; // weight stage: NWR rows x BK (32 KB); 4-bit: codes then group words
constexpr int DA = 2;         // activation stages in the LDS ring
constexpr int DW = 3;         // weight stages in the LDS ring (2 steps ahead)

// The LDS rings: distinct arrays per stage, so that the compiler can tell a
// read of one stage from the transfers still in flight into the others.
struct Ring {
  u32x4_t* a[DA];
  u32x4_t* w[DW];
};

// global -> LDS transfer of 16 (or 4) bytes per lane: lane i of the wave
// writes bytes [16 i, 16 i + 16) after the wave-uniform LDS address `dst`.
__device__ __forceinline__ void dma16(const void* src, u32x4_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
// The same with the non-temporal hint (streaming data read once: the weight
// panel of an expert whose rows fit one tile).
__device__ __forceinline__ void dma16_nt(const void* src, u32x4_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 2);
}
__device__ __forceinline__ void dma4(const void* src, uint32_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}
// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Workgroup barrier that orders nothing by itself: the waits before it are
// explicit, and the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Eight 4-bit codes (element j in bits 4j..4j+3) of one 64-element group
// with its (scale, bias) word -> eight bf16 weights s*q + b (fp32, then
// rounded to nearest even), as an MFMA operand fragment.
__device__ __forceinline__ u32x4_t dequant8(uint32_t c, uint32_t g) {
  const float s = bf16_lo(g), b = bf16_hi(g);
  uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 / 1,3,5,7
  // opaque to the compiler: each byte j then converts with one v_cvt_f32_ubyte<j>, instead of
  // a bit-field extract of the nibble from c and a conversion per element
  asm("" : "+v"(lo), "+v"(hi));
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = pack_bf16x2(s * (float)((lo >> (8 * j)) & 0xFFu) + b, s * (float)((hi >> (8 * j)) & 0xFFu) + b);
  return r;
}

// MODE 2 epilogue: the shared expert's down projection fused with the
// weighted combine ("Optimizing on-device inference for Apple Silicon",
// section "Reduce intermediate and state traffic": the output projection
// goes with its routing score and the shared expert's result).  The tile is
// <= 128 tokens (in order) x the panel's <= 256 columns.  Its shared-expert
// outputs S, rounded to bf16, are staged in the idle LDS rings (rows 0-63 in
// ring.a[0], 64-127 in ring.a[1], 512 bytes a row), the tile's inv / w
// entries beside them, then all 512 threads build out[t] = sum_j w[t,j] *
// y_r[inv[t,j]] (fp32, slot order) + S[t], rounded once to bf16, 8 columns
// (16-byte loads of each y row) per thread and step: the arithmetic of the
// stand-alone combine.
template <int NRH>
__device__ __forceinline__ void combine_epilogue(const GemmArgs& p, const Tile& tl, int panel, const Ring& ring,
                                                 const f32x16_t (&acc)[NRH][2], bool wave_cols, int cg, int rg,
                                                 int half, int l32) {
  const int tid = threadIdx.x, k = p.k;
  uint16_t* s_lo = (uint16_t*)ring.a[0];
  uint16_t* s_hi = (uint16_t*)ring.a[1];
  int32_t* s_pos = (int32_t*)ring.w[0];  // [128][k]
  float* s_w = (float*)ring.w[1];        // [128][k]
  if (wave_cols) {
#pragma unroll
    for (int j = 0; j < NRH; ++j) {
      const int rb = 2 * j + rg;
      if (32 * rb >= tl.rows) break;  // uniform
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
        uint16_t* srow = (row < 64 ? s_lo + row * 256 : s_hi + (row - 64) * 256);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) srow[64 * cg + 32 * cb + l32] = (uint16_t)f32_to_bf16(acc[j][cb][r]);
      }
    }
  }
  for (int e = tid; e < tl.rows * k; e += 512) {
    const int64_t a = ((int64_t)tl.pos0 + e / k) * k + e % k;
    s_pos[e] = p.inv[a];
    s_w[e] = p.w[a];
  }
  __syncthreads();
  const int c0 = panel * NWR;                                // first column of the panel
  const int nq = (p.H - c0 < NWR ? p.H - c0 : NWR) / 8;    // 8-column chunks in the panel
  for (int c = tid; c < tl.rows * 32; c += 512) {
    const int row = c >> 5, q = c & 31;
    if (q >= nq) continue;
    const int64_t t = (int64_t)tl.pos0 + row;
    const int col = c0 + 8 * q;
    float a8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int jb = 0; jb < k; jb += 8) {  // eight rows' loads in flight at a time
      u32x4_t v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (jb + jj < k)  // each y row is read once: non-temporal
          v[jj] = __builtin_nontemporal_load((const u32x4_t*)(p.y_r + (int64_t)s_pos[row * k + jb + jj] * p.H + col));
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (jb + jj >= k) break;
        const float wj = s_w[row * k + jb + jj];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          a8[2 * qq] += wj * bf16_lo(v[jj][qq]);
          a8[2 * qq + 1] += wj * bf16_hi(v[jj][qq]);
        }
      }
    }
    const uint16_t* srow = (row < 64 ? s_lo + row * 256 : s_hi + (row - 64) * 256) + 8 * q;
    const u32x4_t sv = *(const u32x4_t*)srow;
    u32x4_t o;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      a8[2 * qq] += bf16_lo(sv[qq]);
      a8[2 * qq + 1] += bf16_hi(sv[qq]);
      o[qq] = pack_bf16x2(a8[2 * qq], a8[2 * qq + 1]);
    }
    *(u32x4_t*)(p.out + t * p.H + col) = o;
  }
}

// One tile, eight waves (two per SIMD, so one wave's LDS and memory stalls
// overlap the other's MFMAs).  Wave w = 4 rg + cg: column group cg, row group
// rg.  MODE 0: h = silu(A Wg^T) * (A Wu^T) over a 128-column panel of I;
// column group cg owns gate rows [n0+32cg, +32) (col block 0) and the up rows
// of the same columns (col block 1), so SwiGLU is lane-local.  MODE 1:
// y = A Wd^T over a 256-column panel of H; column group cg owns columns
// [n0+64cg, +64).  Row group rg owns the 32-row blocks rb = rg, rg+2, ...
// below NRB (an odd NRB leaves row group 1 one block fewer; with NRB = 1 its
// waves only move their share of the transfers).
//
// K runs in steps of BK through two LDS rings filled by direct global->LDS
// transfers (no register staging): the weight tile (NWR rows x BK) in DW
// stages, DW - 1 steps ahead, and the gathered activation tile (rows of a
// routed group through the scatter permutation) in DA stages, one step
// ahead.  Every transfer moves 8 rows x 128 bytes (whole cache lines).  At
// step s each wave waits for its own transfers of step s (exact counts: the
// transfers issued after them are known), passes the barrier (then every
// wave's transfers of step s are done), refills the stages consumed at step
// s-1 and multiplies from the stages of step s.  Rows of a stage are 128
// bytes with the 16-byte chunks XOR-swizzled by the row (chunk q of row r at
// position q ^ ((r >> 1) & 7)), realised by choosing each lane's source
// chunk: the LDS serves a 16-byte read 16 lanes at a time, here 16
// consecutive rows, two per 256-byte line of its 64 banks, and the swizzle
// gives them 16 distinct bank groups (with q ^ (r & 7), rows r and r + 8
// collide and every operand read takes twice as long).  MFMA sub-step kk and lane half
// h take the 8 K-values 32h+8kk .. 32h+8kk+7 on both operands, a consistent
// permutation of K.
//
// Q4: a step's 64 K-values of a weight row are one group: the stage holds
// the rows' 32 bytes of codes and their group words, expanded to bf16
// operands in registers just before the MFMA.
template <int MODE, int NRB, bool Q4, bool NT = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const Tile& tl, int panel, const Ring& ring0) {
  // NRB = 9: a 288-row tile (a group's last 1..32 rows past 256 kept with
  // its 256).  Blocks 0..7 run as for NRB = 8; block 8 is split by column
  // block between the row groups (row group rg takes column block rg), its
  // activation rows in a stage of their own in the third weight stage, which
  // the tile gives up (weights one step ahead instead of two).
  constexpr bool X9 = NRB == 9;
  constexpr int NRBm = X9 ? 8 : NRB;   // blocks of the main stages
  constexpr int NRH = (NRBm + 1) / 2;  // row blocks of row group 0 (row group 1: NRBm / 2)
  constexpr int DWT = X9 ? 2 : DW;
  constexpr int U = DA * DWT;          // unroll: every ring stage index static
  // the K-step pipeline runs across steps (two sub-steps' operands live at
  // the step boundary) where the registers allow it without spilling
  constexpr bool XPIPE = NRB <= 8;
  struct RingT {
    u32x4_t* a[DA];
    u32x4_t* w[DW];
    u32x4_t* x[DA];
  } ring;
  ring.a[0] = ring0.a[0];
  ring.a[1] = ring0.a[1];
#pragma unroll
  for (int d = 0; d < DW; ++d) ring.w[d] = ring0.w[d];
  ring.x[0] = ring0.w[DW - 1];
  ring.x[1] = ring0.w[DW - 1] + 32 * CPR;  // 32 rows x 128 bytes further
  const bool is_shared = tl.g >= p.E;
  const int Ig = is_shared ? p.Is : p.I;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = wave & 3, rg = wave >> 2;
  const int lr = lane >> 3;  // transfers: row within 8
  // source chunk of this lane in a transfer that fills stage rows 8 blk .. +8
  auto srcq = [&](int blk) { return (lane & 7) ^ ((4 * (blk & 1) + (lr >> 1)) & 7); };

  int K, N, ncol0, ldw;
  if (MODE == 0) {  // gate/up; MODE 1 and 2: down
    K = p.H;
    N = Ig;
    ncol0 = panel * (NWR / 2) + 32 * cg;
    ldw = p.H;
  } else {
    K = Ig;
    N = p.H;
    ncol0 = panel * NWR + WN * cg;
    ldw = Ig;
  }
  // wave-uniform: does this wave own any output column (and, for one row
  // block, any row)?
  const bool wave_cols = ncol0 < N && (NRB > 1 || rg == 0);
  const int nsteps = K / BK;

  // ---- weight rows of column group cg: (col block cb, row l of 32) -> first element
  auto wrow_elem = [&](int cb, int l) -> int64_t {
    int wrow;
    int64_t rbase;
    if (MODE == 0) {
      wrow = ncol0 + l;
      rbase = cb == 0 ? 0 : (int64_t)Ig * p.H;  // gate, then up
    } else {
      wrow = ncol0 + 32 * cb + l;
      rbase = (int64_t)2 * Ig * p.H;  // down [H][Ig]
    }
    if (wrow >= N) wrow = 0;  // columns past N compute on row 0 and are never stored
    return rbase + (int64_t)wrow * ldw;
  };
  // stage row of (cg, cb, l): R = 64 cg + 32 cb + l; this wave moves cb = rg
  const char* wsrc;            // bf16 rows, or 4-bit codes
  const char* gsrc = nullptr;  // 4-bit group words
  uint32_t woff[4];            // byte offsets within the expert block
  uint32_t goff = 0;
  int wstep = 128;             // bytes from one weight step to the next
  int gstep = 4;               // 4-bit: group-word bytes from one step to the next
  if (Q4) {
    const int64_t eb = is_shared ? 0 : (int64_t)tl.g * 3 * p.I * p.H;  // expert block, elements
    wsrc = (const char*)(is_shared ? p.sh_codes : p.ex_codes) + eb / 2;
    gsrc = (const char*)(is_shared ? p.sh_groups : p.ex_groups) + eb / 16;
    // codes: stage rows 64cg + 32rg + lane/2, 16 bytes (half lane&1) each;
    // group words: stage rows 64cg + lane (moved by row group 0)
    if (p.tiled) {
      // tiled: step s of this panel is one block of trows x 32 bytes of codes
      // and one of trows group words, in stage row order (rows past a
      // partial panel re-read the first row: never stored)
      const int n = MODE == 0 ? (Ig - panel * (NWR / 2) < NWR / 2 ? Ig - panel * (NWR / 2) : NWR / 2)
                              : (p.H - panel * NWR < NWR ? p.H - panel * NWR : NWR);
      const int trows = MODE == 0 ? 2 * n : n;
      const int64_t pbase = MODE == 0 ? (int64_t)NWR * panel * p.H : (int64_t)2 * Ig * p.H + (int64_t)NWR * panel * Ig;
      wsrc += pbase / 2;
      gsrc += pbase / 16;
      wstep = trows * 32;
      gstep = trows * 4;
      const int R = 64 * cg + 32 * rg + (lane >> 1), gR = 64 * cg + lane;
      woff[0] = (uint32_t)((R < trows ? R : 0) * 32 + 16 * (lane & 1));
      goff = (uint32_t)((gR < trows ? gR : 0) * 4);
    } else {
      wstep = 32;
      woff[0] = (uint32_t)(wrow_elem(rg, lane >> 1) / 2 + 16 * (lane & 1));
      goff = (uint32_t)(wrow_elem(lane >> 5, lane & 31) / 64 * 4);
    }
    woff[1] = woff[2] = woff[3] = 0;
  } else {
    const uint16_t* W = is_shared ? p.shared_w : p.expert_w + (int64_t)tl.g * 3 * p.I * p.H;
    wsrc = (const char*)W;
    if (p.tiled) {
      // tiled layout: step s of this panel is one block of trows tile rows
      // x 128 bytes, already in stage order and swizzled, so transfer i
      // copies the 1 KB of stage rows 8 (8 cg + 4 rg + i) .. +8 verbatim
      // (rows past a partial panel re-read the first 1 KB: never stored)
      const int n = MODE == 0 ? (Ig - panel * (NWR / 2) < NWR / 2 ? Ig - panel * (NWR / 2) : NWR / 2)
                              : (p.H - panel * NWR < NWR ? p.H - panel * NWR : NWR);
      const int trows = MODE == 0 ? 2 * n : n;
      wstep = trows * 128;
      const int64_t pbase = MODE == 0 ? (int64_t)NWR * panel * p.H : (int64_t)2 * Ig * p.H + (int64_t)NWR * panel * Ig;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int blk = cg * 8 + rg * 4 + i;
        woff[i] = (uint32_t)(pbase * 2 + (8 * blk < trows ? blk : 0) * 1024 + lane * 16);
      }
    } else {
      // transfer i: rows 8i + lane/8 of col block rg (stage block 8 cg + 4 rg + i)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        woff[i] = (uint32_t)((wrow_elem(rg, 8 * i + lr) + 8 * srcq(cg * 8 + rg * 4 + i)) * 2);
    }
  }

  // ---- activation rows this wave moves: rows (wave*NRH + i)*8 + lane/8
  const char* asrc[NRH];
#pragma unroll
  for (int i = 0; i < NRH; ++i) {
    const int row = (wave * NRH + i) * 8 + lr;
    const int r = row < tl.rows ? row : 0;
    const uint16_t* rowp;
    if (MODE == 0) {
      const int64_t tok = is_shared ? (int64_t)tl.pos0 + r : (int64_t)(p.perm[tl.pos0 + r] / p.k);
      rowp = p.a_x + tok * p.H;
    } else {
      rowp = (is_shared ? p.a_s : p.a_r) + ((int64_t)tl.pos0 + r) * Ig;
    }
    asrc[i] = (const char*)(rowp + 8 * srcq(wave * NRH + i));
  }

  const char* xsrc = nullptr;  // NRB = 9: rows 256 + 8 wave + lane/8 (waves 0..3)
  if (X9) {
    const int row = 256 + 8 * (wave & 3) + lr;
    const int r = row < tl.rows ? row : 0;
    const uint16_t* rowp;
    if (MODE == 0) {
      const int64_t tok = is_shared ? (int64_t)tl.pos0 + r : (int64_t)(p.perm[tl.pos0 + r] / p.k);
      rowp = p.a_x + tok * p.H;
    } else {
      rowp = (is_shared ? p.a_s : p.a_r) + ((int64_t)tl.pos0 + r) * Ig;
    }
    xsrc = (const char*)(rowp + 8 * srcq(wave & 3));
  }
  auto load_a = [&](u32x4_t* st, u32x4_t* xst, int s) {
#pragma unroll
    for (int i = 0; i < NRH; ++i) dma16(asrc[i] + (int64_t)s * 128, st + (wave * NRH + i) * 64);
    if (X9 && wave < 4) dma16(xsrc + (int64_t)s * 128, xst + wave * 64);
  };
  auto load_w = [&](u32x4_t* st, int s) {
    if (Q4) {
      if (NT)
        dma16_nt(wsrc + woff[0] + (int64_t)s * wstep, st + (cg * 2 + rg) * 64);
      else
        dma16(wsrc + woff[0] + (int64_t)s * wstep, st + (cg * 2 + rg) * 64);
      if (rg == 0) dma4(gsrc + goff + (int64_t)s * gstep, (uint32_t*)(st + 2 * NWR) + cg * 64);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (NT)
          dma16_nt(wsrc + woff[i] + (int64_t)s * wstep, st + (cg * 8 + rg * 4 + i) * 64);
        else
          dma16(wsrc + woff[i] + (int64_t)s * wstep, st + (cg * 8 + rg * 4 + i) * 64);
      }
    }
  };

  f32x16_t acc[NRH][2];
#pragma unroll
  for (int j = 0; j < NRH; ++j)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[j][cb] = (f32x16_t){};
  f32x16_t accx = {};  // NRB = 9: block 8 x column block rg

  // operand reads: activation row 32 (2j + rg) + l32, weight row 64 cg + 32 cb
  // + l32, chunk 4 half + kk, swizzled by the row (both rows are = l32 mod 16)
  const int swr = (l32 >> 1) & 7;
  auto clampst = [&](int st) { return st < nsteps ? st : nsteps - 1; };

  // The K loop, one copy per kind of wave (a branch inside the loop would
  // merge the compiler's wait bookkeeping of both kinds at every step).
  //
  // Each step runs KK MFMA sub-steps; sub-step kk + 1's operands are read
  // from LDS while sub-step kk's MFMAs run.  The pipeline also runs across
  // steps: the barrier that opens step s + 1 and the reads of its first
  // sub-step's operands come before step s's last sub-step of MFMAs (whose
  // operands are already in registers), so the MFMA pipe keeps working
  // through every step's barrier and first LDS round trip.  Per accumulator
  // the MFMA order is that of the plain loop.  The step's transfers
  // (activation step s + 1 into the stage of step s - 1, weight step
  // s + DWT - 1 likewise) are issued between the MFMA sub-steps: a wave that
  // stalls issuing them leaves its SIMD to the other wave there, instead of
  // all transfers of a step queueing up front; the scheduling barriers keep
  // that order.  RG: the wave's row group, a constant, so that row group 1 of
  // an odd block count skips its last block (rows past the tile) without a
  // branch.
  auto kloop = [&](auto cols, auto nw, auto rgc) {
    constexpr bool XP = XPIPE;
    constexpr bool COLS = decltype(cols)::value;
    constexpr int NWC = decltype(nw)::value;
    constexpr int RG = decltype(rgc)::value;
    u32x4_t af[2][NRH], bf[2][2], ax[2];  // operands of sub-steps of parity 0 / 1
    u32x4_t bq[2];                        // 4-bit: the step's codes of the wave's two weight rows
    uint32_t bg[2] = {0, 0};              // 4-bit: their group words
    auto read_af = [&](const u32x4_t* sa, u32x4_t (&f)[NRH], int kk) {
      const int q = (4 * half + kk) ^ swr;
#pragma unroll
      for (int j = 0; j < NRH; ++j)
        if (2 * j + RG < NRBm) f[j] = sa[(32 * (2 * j + RG) + l32) * CPR + q];
    };
    auto read_bf = [&](const u32x4_t* sw, u32x4_t (&f)[2], int kk) {
      const int q = (4 * half + kk) ^ swr;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) f[cb] = sw[(64 * cg + 32 * cb + l32) * CPR + q];
    };
    auto read_ax = [&](const u32x4_t* sx, u32x4_t& f, int kk) { f = sx[l32 * CPR + ((4 * half + kk) ^ swr)]; };
    // the first sub-step's operands of the step held in stages (sa, sw, sx)
    auto pre = [&](const u32x4_t* sa, const u32x4_t* sw, const u32x4_t* sx) {
      if (!COLS) return;
      if (Q4) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int R = 64 * cg + 32 * cb + l32;
          bq[cb] = sw[2 * R + half];
          bg[cb] = ((const uint32_t*)(sw + 2 * NWR))[R];
        }
      } else {
        read_bf(sw, bf[0], 0);
      }
      read_af(sa, af[0], 0);
      if (X9) read_ax(sx, ax[0], 0);
    };

    // prologue: weight steps 0 .. DWT-2, then activation step 0; every
    // wave's transfers of step 0 done; step 0's first operands.  Transfers
    // are never conditional (a branch would merge the compiler's wait
    // bookkeeping into a full wait): steps past the end re-read the last step
    // into a stage nobody reads.
#pragma unroll
    for (int d = 0; d < DWT - 1; ++d) load_w(ring.w[d], clampst(d));
    load_a(ring.a[0], ring.x[0], 0);
    wait_vm_lgkm0<0>();
    barrier_only();
    pre(ring.a[0], ring.w[0], ring.x[0]);

    for (int s0 = 0; s0 < nsteps; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = s0 + u;
        if (s >= nsteps) break;  // uniform
        const u32x4_t* sa = ring.a[u % DA];
        const u32x4_t* sw = ring.w[u % DWT];
        const u32x4_t* sx = ring.x[u % DA];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          u32x4_t bw[2];
          if (COLS) {
            if (kk + 1 < KK) {
              read_af(sa, af[(kk + 1) & 1], kk + 1);
              if (!Q4) read_bf(sw, bf[(kk + 1) & 1], kk + 1);
              if (X9) read_ax(sx, ax[(kk + 1) & 1], kk + 1);
            }
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) bw[cb] = Q4 ? dequant8(bq[cb][kk], bg[cb]) : bf[kk & 1][cb];
          }
          if (kk == KK - 1 && XP) {
            // open step s + 1: own transfers of step s + 1 done (after them
            // only this step's weight transfers were issued, NWC of them; with
            // two weight stages those are step s + 1's own), own operand
            // reads of step s done (lgkmcnt 0), then the barrier: every
            // wave's transfers of step s + 1 have landed and no wave reads the
            // stages of step s any more (step s + 1 refills them).  Past the
            // last step this reads stale stages into registers nobody uses.
            __builtin_amdgcn_sched_barrier(0);
            if (DWT == 2)
              wait_vm_lgkm0<0>();
            else
              wait_vm_lgkm0<NWC>();
            barrier_only();
            pre(ring.a[(u + 1) % DA], ring.w[(u + 1) % DWT], ring.x[(u + 1) % DA]);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (COLS) {
#pragma unroll
            for (int j = 0; j < NRH; ++j)
              if (2 * j + RG < NRBm)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                  acc[j][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[kk & 1][j]),
                                                                       __builtin_bit_cast(bf16x8_t, bw[cb]),
                                                                       acc[j][cb], 0, 0, 0);
            if (X9)
              accx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ax[kk & 1]),
                                                             __builtin_bit_cast(bf16x8_t, bw[RG]), accx, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (kk == 0) load_a(ring.a[(u + 1) % DA], ring.x[(u + 1) % DA], clampst(s + 1));
          if (kk == 1) load_w(ring.w[(u + DWT - 1) % DWT], clampst(s + DWT - 1));
          __builtin_amdgcn_sched_barrier(0);
          if (kk == KK - 1 && !XP) {  // the same, after the step's last MFMAs
            if (DWT == 2)
              wait_vm_lgkm0<0>();
            else
              wait_vm_lgkm0<NWC>();
            barrier_only();
            pre(ring.a[(u + 1) % DA], ring.w[(u + 1) % DWT], ring.x[(u + 1) % DA]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  };
  // weight transfers per wave per step: bf16 4 (the row group's col block of
  // its column group); 4-bit 1 of codes, plus the group words in row group 0
  typedef std::integral_constant<int, Q4 ? 2 : 4> NW0;
  typedef std::integral_constant<int, Q4 ? 1 : 4> NW1;
  if (wave_cols) {
    if (rg == 0) kloop(std::true_type{}, NW0{}, std::integral_constant<int, 0>{});
    else kloop(std::true_type{}, NW1{}, std::integral_constant<int, 1>{});
  } else {
    if (rg == 0) kloop(std::false_type{}, NW0{}, std::integral_constant<int, 0>{});
    else kloop(std::false_type{}, NW1{}, std::integral_constant<int, 1>{});
  }
  // every wave's reads done before the activation stage is reused for staging
  wait_vm_lgkm0<0>();
  barrier_only();
  if (MODE == 2) {
    combine_epilogue<NRH>(p, tl, panel, ring0, acc, wave_cols, cg, rg, half, l32);
    return;
  }
  // NRB = 9, gate/up: block 8's up values (row group 1) go to the gate
  // waves (row group 0) of the column group through LDS; every wave passes
  // the barrier (none has left yet)
  float* xch = (float*)ring.w[0] + (cg * 64 + lane) * 16;
  if (X9 && MODE == 0) {
    if (wave_cols && rg == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[r] = accx[r];
    }
    wait_vm_lgkm0<0>();
    barrier_only();
  }
  if (!wave_cols) return;
  u32x4_t* smem = ring.a[0];

  // ---- epilogue: per 32-row block, round to bf16, stage through this wave's
  //      slice of the (now idle) LDS, write 16-byte chunks.
  //      32x32 block D layout: lane -> column lane%32, register r -> row
  //      8*(r/4) + 4*(lane/32) + r%4.
  constexpr int OC = MODE == 0 ? 32 : 64;  // output columns per wave
  constexpr int CPRO = OC / 8;             // 16-byte chunks per output row
  uint16_t* stage = (uint16_t*)smem + wave * (32 * OC);
  uint16_t* obase = is_shared ? p.out_s : p.out_r;
  const int ldo = MODE == 0 ? Ig : p.H;
#pragma unroll
  for (int j = 0; j < NRH; ++j) {
    const int rb = 2 * j + rg;
    if (32 * rb >= tl.rows) break;  // uniform; j stays a constant
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * half + (r & 3);
      if (MODE == 0) {
        stage[row * OC + l32] = (uint16_t)f32_to_bf16(silu(acc[j][0][r]) * acc[j][1][r]);
      } else {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) stage[row * OC + 32 * cb + l32] = (uint16_t)f32_to_bf16(acc[j][cb][r]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c = lane; c < 32 * CPRO; c += 64) {
      const int row = c / CPRO, q = c % CPRO;
      const int grow = 32 * rb + row;
      const int col = ncol0 + 8 * q;
      if (grow < tl.rows && col < N)
        *(u32x4_t*)(obase + ((int64_t)tl.pos0 + grow) * ldo + col) = *(const u32x4_t*)(stage + row * OC + 8 * q);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (X9) {
    // block 8 (rows 256..287): gate/up -> row group 0 writes h for its 32
    // columns; down -> each wave writes its column block's 32 columns
    if (MODE == 0 && rg == 1) return;
    constexpr int XC = 32;  // columns of block 8 per wave
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * half + (r & 3);
      const float v = MODE == 0 ? silu(accx[r]) * xch[r] : accx[r];
      stage[row * XC + l32] = (uint16_t)f32_to_bf16(v);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int xcol0 = MODE == 0 ? ncol0 : ncol0 + 32 * rg;
#pragma unroll
    for (int c = lane; c < 32 * (XC / 8); c += 64) {
      const int row = c / (XC / 8), q = c % (XC / 8);
      const int grow = 256 + row;
      const int col = xcol0 + 8 * q;
      if (grow < tl.rows && col < N)
        *(u32x4_t*)(obase + ((int64_t)tl.pos0 + grow) * ldo + col) = *(const u32x4_t*)(stage + row * XC + 8 * q);
    }
  }
}

// One routed tile, its inner loop specialised per count of 32-row blocks.
template <int MODE, bool Q4, bool NT>
__device__ __forceinline__ void routed_tile(const GemmArgs& p, const Tile& tl, int panel, const Ring& rg) {
  switch ((tl.rows + 31) >> 5) {
    case 1: gemm_tile<MODE, 1, Q4, NT>(p, tl, panel, rg); break;
    case 2: gemm_tile<MODE, 2, Q4, NT>(p, tl, panel, rg); break;
    case 3: gemm_tile<MODE, 3, Q4, NT>(p, tl, panel, rg); break;
    case 4: gemm_tile<MODE, 4, Q4, NT>(p, tl, panel, rg); break;
    case 5: gemm_tile<MODE, 5, Q4, NT>(p, tl, panel, rg); break;
    case 6: gemm_tile<MODE, 6, Q4, NT>(p, tl, panel, rg); break;
    case 7: gemm_tile<MODE, 7, Q4, NT>(p, tl, panel, rg); break;
    case 8: gemm_tile<MODE, 8, Q4, NT>(p, tl, panel, rg); break;
    default: gemm_tile<MODE, 9, Q4, NT>(p, tl, panel, rg); break;
  }
}

template <int MODE, bool Q4>
__global__ __launch_bounds__(512, 1) void k_grouped_gemm(GemmArgs p) {
  __shared__ u32x4_t sA0[SA], sA1[SA], sW0[SB], sW1[SB], sW2[SB];  // 160 KB
  const Ring rg{{sA0, sA1}, {sW0, sW1, sW2}};

  // ---- tile of this workgroup, XCD-aware: workgroup b runs on XCD b % 8;
  //      XCD x takes the tiles t = x (mod 8) of its list, all panels of a
  //      tile in a row (its activation rows are re-read from that XCD's L2)
  if (MODE == 2) {  // the shared expert's tokens in tiles of 128, panel-minor
    // tile t on XCD t % 8 with all its panels: the tile's shared-expert h
    // rows are fetched into that XCD's L2 once, not once per panel
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int tile = (local / p.npan) * 8 + xcd, panel = local % p.npan;
    const int64_t r0 = (int64_t)tile * 128;
    if (r0 >= p.M) return;
    const int rows = (int)(p.M - r0 < 128 ? p.M - r0 : 128);
    const Tile tl{p.E, (int)r0, rows, (int)r0};
    if (rows > 64)
      gemm_tile<2, 4, Q4>(p, tl, panel, rg);
    else
      gemm_tile<2, 2, Q4>(p, tl, panel, rg);
    return;
  }
  int b = blockIdx.x;
  if (MODE == 1 && p.sgu_units > 0) {
    // leading workgroups: the shared expert's gate/up tiles of 256 tokens (they
    // do not depend on the routing and their h is read only by the launch
    // after this one), dispatched first, as the longest units of the launch
    if (b < p.sgu_units) {
      const int tile = b / p.sgu_npan, panel = b % p.sgu_npan;
      const int64_t r0 = (int64_t)tile * BM;
      if (r0 >= p.M || panel * (NWR / 2) >= p.Is) return;
      const Tile tl{p.E, (int)r0, (int)(p.M - r0 < BM ? p.M - r0 : BM), (int)r0};
      switch (((tl.rows + 63) >> 6) << 1) {
        case 2: gemm_tile<0, 2, Q4>(p, tl, panel, rg); break;
        case 4: gemm_tile<0, 4, Q4>(p, tl, panel, rg); break;
        case 6: gemm_tile<0, 6, Q4>(p, tl, panel, rg); break;
        default: gemm_tile<0, 8, Q4>(p, tl, panel, rg); break;
      }
      return;
    }
    b -= p.sgu_units;  // a multiple of 8: the XCD of b is still b % 8
  }
  const int ntl = *p.ntiles - p.skip_tail;
  const int nt = ntl < p.max_tiles ? ntl : p.max_tiles;
  const int xcd = b & 7, local = b >> 3;
  const int j = local / p.npan, panel = local % p.npan;  // j-th tile of this XCD
  // gate/up: the launch-order list from its start; down: the block map from
  // its end (its short tiles, which mostly stream weights, then run among
  // the long ones, which mostly compute: the down tiles' weight panels are a
  // quarter of the gate/up ones', so there the mix pays more than the order)
  const int t = MODE == 0 ? 8 * j + xcd : nt - 1 - (8 * j + (7 - xcd));
  if (t < 0 || t >= nt) return;
  const Tile tl = p.tiles[t];
  if (MODE == 0) {
    const int Ig = tl.g >= p.E ? p.Is : p.I;
    if (panel * (NWR / 2) >= Ig) return;
  }
  // the weights of an expert whose rows fit one tile are read once in the
  // launch: fetched with the non-temporal hint, they leave the caches to the
  // activation rows (an expert split over several tiles is fetched by each of
  // them and keeps the default policy, as does the shared expert).  Not for
  // row-major 4-bit codes: a step takes a quarter of each row's cache line,
  // and the next three steps need the rest.
  if ((!Q4 || p.tiled) && tl.g < p.E && tl.r0 == 0 && tl.rows != BM)
    routed_tile<MODE, Q4, true>(p, tl, panel, rg);
  else
    routed_tile<MODE, Q4, false>(p, tl, panel, rg);
}

// out[t] = sum_j w[t,j] * y_r[inv[t*k+j]] + y_s[t]: fp32 sums in slot order,
// then the shared expert, rounded once to bf16.  One workgroup per token,
// eight columns (16 bytes) per thread per step.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y_r,
                                                 const uint16_t* __restrict__ y_s,
                                                 const float* __restrict__ w,
                                                 const int32_t* __restrict__ inv,
                                                 uint16_t* __restrict__ out, int H, int k) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t s_pos[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  if (threadIdx.x < k) {
    s_pos[threadIdx.x] = inv[t * k + threadIdx.x];
    s_w[threadIdx.x] = w[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)(y_r + (int64_t)s_pos[j] * H + c));
      const float wj = s_w[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wj * bf16_lo(v[q]);
        acc[2 * q + 1] += wj * bf16_hi(v[q]);
      }
    }
    if (y_s) {
      const u32x4_t v = *(const u32x4_t*)(y_s + t * H + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_lo(v[q]);
        acc[2 * q + 1] += bf16_hi(v[q]);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *(u32x4_t*)(out + t * H + c) = o;
  }
}

// 8 XCDs x (most tiles per XCD) x panels: every tile's panels have a workgroup
unsigned xcd_grid(int64_t max_tiles, int npan) { return (unsigned)(8 * ((max_tiles + 7) / 8) * npan); }

// The down launch's leading workgroups for the shared expert's gate/up tiles
// (x_shared_gu non-null: the gate/up launch left them out): one per (256-token
// tile, gate/up panel), rounded up to a multiple of 8 so that the down
// workgroups keep their XCD order.
void shared_gateup_units(GemmArgs* a, const uint16_t* x, uint16_t* h_s, const Plan& pl) {
  if (!x || !h_s || !pl.shared) return;
  a->a_x = x;
  a->out_s = h_s;
  a->sgu_npan = (pl.Is + NWR / 2 - 1) / (NWR / 2);
  const int64_t units = ((pl.M + BM - 1) / BM) * a->sgu_npan;
  a->sgu_units = (int)(8 * ((units + 7) / 8));
}

}  // namespace

hipError_t launch_gemm_gateup(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                              const int32_t* perm, const Tile* tiles, const int32_t* ntiles,
                              uint16_t* h_r, uint16_t* h_s, int skip_tail, const Plan& pl, const Launch& lc) {
  GemmArgs a{};
  a.skip_tail = skip_tail;
  a.a_x = x;
  a.expert_w = expert_w;
  a.shared_w = shared_w;
  a.perm = perm;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.out_r = h_r;
  a.out_s = h_s;
  a.M = pl.M;
  a.H = pl.H;
  a.E = pl.E;
  a.I = pl.I;
  a.Is = pl.Is;
  a.k = pl.k;
  const int maxI = pl.I > pl.Is ? pl.I : pl.Is;
  a.npan = (maxI + NWR / 2 - 1) / (NWR / 2);
  a.max_tiles = (int)pl.max_tiles;
  a.tiled = pl.tiled ? 1 : 0;
  return launch(lc, k_grouped_gemm<0, false>, dim3(xcd_grid(pl.max_tiles, a.npan)), dim3(512), a);
}

hipError_t launch_gemm_down(const uint16_t* h_r, uint16_t* h_s, const uint16_t* expert_w,
                            const uint16_t* shared_w, const Tile* tiles, const int32_t* ntiles,
                            uint16_t* y_r, uint16_t* y_s, int skip_tail, const uint16_t* x_shared_gu,
                            const Plan& pl, const Launch& lc) {
  GemmArgs a{};
  a.skip_tail = skip_tail;
  a.a_r = h_r;
  a.a_s = h_s;
  a.expert_w = expert_w;
  a.shared_w = shared_w;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.out_r = y_r;
  a.out_s = y_s;
  a.M = pl.M;
  a.H = pl.H;
  a.E = pl.E;
  a.I = pl.I;
  a.Is = pl.Is;
  a.k = pl.k;
  a.npan = (pl.H + NWR - 1) / NWR;
  a.max_tiles = (int)pl.max_tiles;
  a.tiled = pl.tiled ? 1 : 0;
  shared_gateup_units(&a, x_shared_gu, h_s, pl);  // last: it sets a_x and out_s
  return launch(lc, k_grouped_gemm<1, false>, dim3(a.sgu_units + xcd_grid(pl.max_tiles, a.npan)), dim3(512), a);
}

hipError_t launch_combine(const uint16_t* y_r, const uint16_t* y_s, const float* w, const int32_t* inv,
                          uint16_t* out, const Plan& pl, const Launch& lc) {
  return launch(lc, k_combine, dim3((unsigned)pl.M), dim3(256), y_r, pl.shared ? y_s : nullptr, w, inv, out, pl.H,
                pl.k);
}

hipError_t launch_gemm_gateup_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh, const int32_t* perm,
                                 const Tile* tiles, const int32_t* ntiles, uint16_t* h_r, uint16_t* h_s,
                                 int skip_tail, const Plan& pl, const Launch& lc) {
  GemmArgs a{};
  a.skip_tail = skip_tail;
  a.a_x = x;
  a.ex_codes = ex.codes;
  a.ex_groups = ex.groups;
  a.sh_codes = sh.codes;
  a.sh_groups = sh.groups;
  a.perm = perm;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.out_r = h_r;
  a.out_s = h_s;
  a.M = pl.M;
  a.H = pl.H;
  a.E = pl.E;
  a.I = pl.I;
  a.Is = pl.Is;
  a.k = pl.k;
  const int maxI = pl.I > pl.Is ? pl.I : pl.Is;
  a.npan = (maxI + NWR / 2 - 1) / (NWR / 2);
  a.max_tiles = (int)pl.max_tiles;
  a.tiled = pl.tiled ? 1 : 0;
  return launch(lc, k_grouped_gemm<0, true>, dim3(xcd_grid(pl.max_tiles, a.npan)), dim3(512), a);
}

hipError_t launch_gemm_down_q4(const uint16_t* h_r, uint16_t* h_s, const Q4Weights& ex, const Q4Weights& sh,
                               const Tile* tiles, const int32_t* ntiles, uint16_t* y_r, uint16_t* y_s, int skip_tail,
                               const uint16_t* x_shared_gu, const Plan& pl, const Launch& lc) {
  GemmArgs a{};
  a.skip_tail = skip_tail;
  a.a_r = h_r;
  a.a_s = h_s;
  a.ex_codes = ex.codes;
  a.ex_groups = ex.groups;
  a.sh_codes = sh.codes;
  a.sh_groups = sh.groups;
  a.tiles = tiles;
  a.ntiles = ntiles;
  a.out_r = y_r;
  a.out_s = y_s;
  a.M = pl.M;
  a.H = pl.H;
  a.E = pl.E;
  a.I = pl.I;
  a.Is = pl.Is;
  a.k = pl.k;
  a.npan = (pl.H + NWR - 1) / NWR;
  a.max_tiles = (int)pl.max_tiles;
  a.tiled = pl.tiled ? 1 : 0;
  shared_gateup_units(&a, x_shared_gu, h_s, pl);  // last: it sets a_x and out_s
  return launch(lc, k_grouped_gemm<1, true>, dim3(a.sgu_units + xcd_grid(pl.max_tiles, a.npan)), dim3(512), a);
}

namespace {

GemmArgs shared_combine_args(const uint16_t* h_s, const uint16_t* y_r, const float* w, const int32_t* inv,
                             uint16_t* out, const Plan& pl) {
  GemmArgs a{};
  a.a_s = h_s;
  a.y_r = y_r;
  a.w = w;
  a.inv = inv;
  a.out = out;
  a.M = pl.M;
  a.H = pl.H;
  a.E = pl.E;
  a.I = pl.I;
  a.Is = pl.Is;
  a.k = pl.k;
  a.npan = (pl.H + NWR - 1) / NWR;
  a.tiled = pl.tiled ? 1 : 0;
  return a;
}

// 8 XCDs x (most 128-token tiles per XCD) x panels
unsigned shared_combine_grid(const Plan& pl) {
  return (unsigned)(8 * (((pl.M + 127) / 128 + 7) / 8) * ((pl.H + NWR - 1) / NWR));
}

}  // namespace

hipError_t launch_shared_down_combine(const uint16_t* h_s, const uint16_t* shared_w, const uint16_t* y_r,
                                      const float* w, const int32_t* inv, uint16_t* out, const Plan& pl,
                                      const Launch& lc) {
  GemmArgs a = shared_combine_args(h_s, y_r, w, inv, out, pl);
  a.shared_w = shared_w;
  return launch(lc, k_grouped_gemm<2, false>, dim3(shared_combine_grid(pl)), dim3(512), a);
}

hipError_t launch_shared_down_combine_q4(const uint16_t* h_s, const Q4Weights& sh, const uint16_t* y_r,
                                         const float* w, const int32_t* inv, uint16_t* out, const Plan& pl,
                                         const Launch& lc) {
  GemmArgs a = shared_combine_args(h_s, y_r, w, inv, out, pl);
  a.sh_codes = sh.codes;
  a.sh_groups = sh.groups;
  return launch(lc, k_grouped_gemm<2, true>, dim3(shared_combine_grid(pl)), dim3(512), a);
}

}  // namespace moe
