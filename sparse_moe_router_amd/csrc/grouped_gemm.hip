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
// Tile: up to 256 rows of one expert group (eight 32-row blocks) x 256
// weight rows, one 4-wave workgroup per CU.  Every wave covers all rows of
// the tile and its own 64 weight rows (a 256x64 fp32 accumulator, 256
// registers, in AGPRs).  The weights -- the HBM stream -- go straight from
// global memory into MFMA operand registers, each byte loaded once per tile
// and never through LDS; the activation tile (rows of a routed group
// gathered through the scatter permutation, never copied) is staged once
// per K-step in LDS and read by all four waves.  With tiles of 256 rows an
// expert's weights are read once whenever it has at most 256 rows (all
// experts at near-uniform routing).  The number of 32-row blocks is a
// template parameter chosen per tile (rounded up to even), so the inner
// loop has no branches and row blocks past the group's rows cost nothing.
//
// Launch order is XCD-aware: workgroup b runs on XCD b % 8, and consecutive
// logical tiles (the panels of one row tile, then the next row tile of the
// same expert) are given to the same XCD so activation rows and weight
// panels are re-read from that XCD's L2 instead of HBM.
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
  int64_t M;
  int H, E, I, Is, k;
  int npan;
  int max_tiles;
};

constexpr int BK = 64;        // K per pipeline step
constexpr int CPR = BK / 8;   // 16-byte chunks per row per step
constexpr int KK = BK / 16;   // MFMA sub-steps per step
constexpr int DB2 = 2;        // weight steps in flight, bf16 weights (16 registers per step)
constexpr int DB4 = 4;        // weight steps in flight, 4-bit weights (5 registers per step)
constexpr int LDS_A = 2 * BM * CPR;  // two activation buffers, 16-byte units (64 KB)

__device__ __forceinline__ int swz(int row, int q) { return row * CPR + (q ^ (row & (CPR - 1))); }

// Eight 4-bit codes (element j in bits 4j..4j+3) of one 64-element group
// with its (scale, bias) word -> eight bf16 weights s*q + b (fp32, then
// rounded to nearest even), as an MFMA operand fragment.
__device__ __forceinline__ u32x4_t dequant8(uint32_t c, uint32_t g) {
  const float s = bf16_lo(g), b = bf16_hi(g);
  const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;  // elements 0,2,4,6 / 1,3,5,7
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = pack_bf16x2(s * (float)((lo >> (8 * j)) & 0xFFu) + b, s * (float)((hi >> (8 * j)) & 0xFFu) + b);
  return r;
}

// One tile.  MODE 0: h = silu(A Wg^T) * (A Wu^T) over a 128-column panel of
// I; wave w owns gate rows [n0+32w, +32) (col block 0) and the up rows of the
// same columns (col block 1), so SwiGLU is lane-local.  MODE 1: y = A Wd^T
// over a 256-column panel of H; wave w owns columns [n0+64w, +64).
//
// K runs in steps of BK with register pipelines.  Weights: DB ring slots;
// as soon as the MFMAs of sub-step kk have read their weight fragments, the
// slot's fragment kk is refilled with the same chunk DB steps ahead, so the
// weight loads spread through the MFMA phase and about DB steps of weights
// stay in flight.  Activations: the chunks of step s+1 are written to the
// other LDS buffer at the start of step s; they were loaded one step
// earlier, before that step's weight loads, so waiting for them (loads
// complete in issue order) never waits for the newer weight loads.  The
// activation fragments are double-buffered across MFMA sub-steps, so the
// LDS reads of sub-step kk+1 overlap the MFMAs of sub-step kk.  Within a
// step, MFMA sub-step kk and lane half h take the 8 K-values
// 32h+8kk .. 32h+8kk+7 on both operands, a consistent permutation of K that
// lets each lane read 16 contiguous bytes.  Loads past the last step
// re-read the last step (never out of bounds, never conditional), so no
// control flow surrounds memory operations.
//
// Q4: the weights are 4-bit codes with a (scale, bias) per 64-element group
// ("Dequantize weights during matrix multiplication").  A step's 64 K-values
// of a weight row are exactly one group, so per step and column block a
// lane loads 16 bytes of codes (its 32 K-values, the four sub-steps) and one
// group word, and expands each sub-step's eight codes to bf16 operands in
// registers just before the MFMA; the ring then holds DB4 steps.
template <int MODE, int NRB, bool Q4>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const Tile& tl, int panel, u32x4_t* smem) {
  constexpr int DB = Q4 ? DB4 : DB2;
  constexpr int U = DB;  // unroll: a multiple of DB and of the 2 LDS buffers
  constexpr int ACH = NRB * 32 * CPR / 256;  // activation chunks per thread per step
  const bool is_shared = tl.g >= p.E;
  const int Ig = is_shared ? p.Is : p.I;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  u32x4_t(*sA)[BM * CPR] = (u32x4_t(*)[BM * CPR])smem;

  const uint16_t* W = is_shared ? p.shared_w : p.expert_w + (int64_t)tl.g * 3 * p.I * p.H;
  int K, N, ncol0, ldw;
  if (MODE == 0) {
    K = p.H;
    N = Ig;
    ncol0 = panel * (NWR / 2) + 32 * wave;
    ldw = p.H;
  } else {
    K = Ig;
    N = p.H;
    ncol0 = panel * NWR + WN * wave;
    ldw = Ig;
  }
  const bool wave_cols = ncol0 < N;  // wave-uniform: does this wave own any output column?

  // ---- this wave's weight rows: col block cb -> one 16-byte chunk per lane per
  //      sub-step (bf16), or per step plus a group word (4-bit)
  const u32x4_t* bsrc[2];
  const u32x4_t* qsrc[2];
  const uint32_t* gsrc[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    int wrow;
    int64_t rbase;  // first element of the row set within the expert block
    if (MODE == 0) {
      wrow = ncol0 + l32;
      rbase = cb == 0 ? 0 : (int64_t)Ig * p.H;  // gate, then up
    } else {
      wrow = ncol0 + 32 * cb + l32;
      rbase = (int64_t)2 * Ig * p.H;  // down [H][Ig]
    }
    if (wrow >= N) wrow = 0;  // columns past N compute on row 0 and are never stored
    const int64_t e0 = rbase + (int64_t)wrow * ldw;  // the row's first element (a multiple of 64)
    if (Q4) {
      const uint32_t* cbase = is_shared ? p.sh_codes : p.ex_codes + (int64_t)tl.g * 3 * p.I * p.H / 8;
      const uint32_t* gbase = is_shared ? p.sh_groups : p.ex_groups + (int64_t)tl.g * 3 * p.I * p.H / 64;
      qsrc[cb] = (const u32x4_t*)(cbase + e0 / 8) + half;  // step st: element 2 st
      gsrc[cb] = gbase + e0 / 64;                          // step st: element st
      bsrc[cb] = nullptr;
    } else {
      bsrc[cb] = (const u32x4_t*)(W + e0) + (CPR / 2) * half;
      qsrc[cb] = nullptr;
      gsrc[cb] = nullptr;
    }
  }

  // ---- activation-tile loader: ACH chunks per thread per step (row-contiguous, coalesced)
  const u32x4_t* asrc[ACH];
  int adst[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + 256 * i, row = c / CPR, q = c % CPR;
    const int r = row < tl.rows ? row : 0;
    const uint16_t* rowp;
    if (MODE == 0) {
      const int64_t tok = is_shared ? (int64_t)tl.pos0 + r : (int64_t)(p.perm[tl.pos0 + r] / p.k);
      rowp = p.a_x + tok * p.H;
    } else {
      rowp = (is_shared ? p.a_s : p.a_r) + ((int64_t)tl.pos0 + r) * Ig;
    }
    asrc[i] = (const u32x4_t*)rowp + q;
    adst[i] = swz(row, q);
  }

  const int nsteps = K / BK;
  u32x4_t breg[Q4 ? 1 : DB][2][KK];
  u32x4_t qreg[Q4 ? DB : 1][2];
  uint32_t greg[Q4 ? DB : 1][2];
  u32x4_t areg[ACH];
  auto clampst = [&](int st) { return st < nsteps ? st : nsteps - 1; };
  auto chunk0 = [&](int st) { return clampst(st) * CPR; };
  // weights of step st into ring slot d (all sub-steps)
  auto load_b = [&](int st, int d) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (Q4) {
        qreg[d][cb] = qsrc[cb][2 * clampst(st)];
        greg[d][cb] = gsrc[cb][clampst(st)];
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) breg[d][cb][kk] = bsrc[cb][chunk0(st) + kk];
      }
    }
  };
  auto load_a = [&](int st) {
    const int c0 = chunk0(st);
#pragma unroll
    for (int i = 0; i < ACH; ++i) areg[i] = asrc[i][c0];
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) sA[buf][adst[i]] = areg[i];
  };

  f32x16_t acc[NRB][2];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[rb][cb] = (f32x16_t){};

  // prologue: activation step 0 -> LDS buffer 0, activation step 1 in
  // registers, then weight steps 0 .. DB-1 in flight.  Issuing the weights
  // after activation step 1, as in every later step, keeps the compiler's
  // wait counts at the loop head exact (it merges the entry state with the
  // back-edge state, and a shorter queue behind activation step 1 on entry
  // would make every step wait for weights issued one step earlier).
  load_a(0);
  store_a(0);
  load_a(1);
#pragma unroll
  for (int d = 0; d < DB; ++d) load_b(d, d);
  __syncthreads();

  // step s: weight slot s % DB, LDS buffer s % 2 (step s+1 goes to the other one)
  for (int s0 = 0; s0 < nsteps; s0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      const int ub = u % DB;
      store_a((u + 1) & 1);
      load_a(s + 2);
      const int cn = chunk0(s + DB);
      const int sn = clampst(s + DB);
      const bool active = wave_cols && s < nsteps;
      u32x4_t af[2][NRB];
      auto read_af = [&](u32x4_t (&f)[NRB], int kk) {
        const int q = (CPR / 2) * half + kk;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) f[rb] = sA[u & 1][swz(32 * rb + l32, q)];
      };
      if (active) read_af(af[0], 0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        // a step past the end (odd nsteps) only repeats the clamped loads and
        // the barrier, so every wave runs the same barriers
        if (active) {
          if (kk + 1 < KK) read_af(af[(kk + 1) & 1], kk + 1);
          u32x4_t bw[2];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) bw[cb] = Q4 ? dequant8(qreg[ub][cb][kk], greg[ub][cb]) : breg[Q4 ? 0 : ub][cb][kk];
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
              acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[kk & 1][rb]),
                                                                    __builtin_bit_cast(bf16x8_t, bw[cb]),
                                                                    acc[rb][cb], 0, 0, 0);
        }
        if (Q4) {
          if (kk == KK - 1) {  // the step's codes are consumed: refill the slot DB steps ahead
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              qreg[ub][cb] = qsrc[cb][2 * sn];
              greg[ub][cb] = gsrc[cb][sn];
            }
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) breg[Q4 ? 0 : ub][cb][kk] = bsrc[cb][cn + kk];
        }
      }
      __syncthreads();
    }
  }
  if (!wave_cols) return;

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
  for (int rb = 0; rb < NRB; ++rb) {
    if (32 * rb >= tl.rows) break;  // uniform; rb stays a constant
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * half + (r & 3);
      if (MODE == 0) {
        stage[row * OC + l32] = (uint16_t)f32_to_bf16(silu(acc[rb][0][r]) * acc[rb][1][r]);
      } else {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) stage[row * OC + 32 * cb + l32] = (uint16_t)f32_to_bf16(acc[rb][cb][r]);
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
}

template <int MODE, bool Q4>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm(GemmArgs p) {
  __shared__ u32x4_t smem[LDS_A];

  // ---- logical tile from the XCD-aware launch order
  const int nt = *p.ntiles;
  const int V = (nt < p.max_tiles ? nt : p.max_tiles) * p.npan;
  const int b = blockIdx.x, xcd = b & 7, local = b >> 3;
  const int per = (V + 7) >> 3;
  if (local >= per) return;
  const int lid = xcd * per + local;
  if (lid >= V) return;
  const Tile tl = p.tiles[lid / p.npan];
  const int panel = lid % p.npan;
  if (MODE == 0) {
    const int Ig = tl.g >= p.E ? p.Is : p.I;
    if (panel * (NWR / 2) >= Ig) return;
  }
  // row blocks of 32, rounded up to even: the inner loop is specialised per count
  const int nrb2 = ((tl.rows + 63) >> 6) << 1;
  switch (nrb2) {
    case 2: gemm_tile<MODE, 2, Q4>(p, tl, panel, smem); break;
    case 4: gemm_tile<MODE, 4, Q4>(p, tl, panel, smem); break;
    case 6: gemm_tile<MODE, 6, Q4>(p, tl, panel, smem); break;
    default: gemm_tile<MODE, 8, Q4>(p, tl, panel, smem); break;
  }
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
      const u32x4_t v = *(const u32x4_t*)(y_r + (int64_t)s_pos[j] * H + c);
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

unsigned xcd_grid(int64_t logical) { return (unsigned)(((logical + 7) / 8) * 8); }

}  // namespace

hipError_t launch_gemm_gateup(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                              const int32_t* perm, const Tile* tiles, const int32_t* ntiles,
                              uint16_t* h_r, uint16_t* h_s, const Plan& pl, const Launch& lc) {
  GemmArgs a{};
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
  return launch(lc, k_grouped_gemm<0, false>, dim3(xcd_grid(pl.max_tiles * a.npan)), dim3(256), a);
}

hipError_t launch_gemm_down(const uint16_t* h_r, const uint16_t* h_s, const uint16_t* expert_w,
                            const uint16_t* shared_w, const Tile* tiles, const int32_t* ntiles,
                            uint16_t* y_r, uint16_t* y_s, const Plan& pl, const Launch& lc) {
  GemmArgs a{};
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
  return launch(lc, k_grouped_gemm<1, false>, dim3(xcd_grid(pl.max_tiles * a.npan)), dim3(256), a);
}

hipError_t launch_combine(const uint16_t* y_r, const uint16_t* y_s, const float* w, const int32_t* inv,
                          uint16_t* out, const Plan& pl, const Launch& lc) {
  return launch(lc, k_combine, dim3((unsigned)pl.M), dim3(256), y_r, pl.shared ? y_s : nullptr, w, inv, out, pl.H,
                pl.k);
}

hipError_t launch_gemm_gateup_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh, const int32_t* perm,
                                 const Tile* tiles, const int32_t* ntiles, uint16_t* h_r, uint16_t* h_s,
                                 const Plan& pl, const Launch& lc) {
  GemmArgs a{};
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
  return launch(lc, k_grouped_gemm<0, true>, dim3(xcd_grid(pl.max_tiles * a.npan)), dim3(256), a);
}

hipError_t launch_gemm_down_q4(const uint16_t* h_r, const uint16_t* h_s, const Q4Weights& ex, const Q4Weights& sh,
                               const Tile* tiles, const int32_t* ntiles, uint16_t* y_r, uint16_t* y_s, const Plan& pl,
                               const Launch& lc) {
  GemmArgs a{};
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
  return launch(lc, k_grouped_gemm<1, true>, dim3(xcd_grid(pl.max_tiles * a.npan)), dim3(256), a);
}

}  // namespace moe
