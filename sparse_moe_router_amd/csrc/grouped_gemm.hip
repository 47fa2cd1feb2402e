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
// Tile: up to 256 rows of one expert group x 128 weight rows.  Four waves
// split the rows (64 each); each wave holds a 64x128 fp32 accumulator
// (2 x 4 blocks of 32x32) and needs all 128 weight rows, so the weight tile
// is shared through LDS while each wave loads its own activation rows
// straight into MFMA operand registers (the rows of a routed group are
// gathered through the scatter permutation, never copied).
//
// Launch order is XCD-aware: workgroup b runs on XCD b % 8, and consecutive
// logical tiles (the panels of one row tile, then the next row tile of the
// same expert) are given to the same XCD so activation rows and weight
// panels are re-read from that XCD's L2 instead of HBM.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BK = 32;   // K per pipeline step
constexpr int BNR = 128; // weight rows per tile

struct GemmArgs {
  const uint16_t* a_x;    // gate/up: token rows [M][H]
  const uint16_t* a_r;    // down: routed h rows [A][I]
  const uint16_t* a_s;    // down: shared h rows [M][Is]
  const uint16_t* expert_w;
  const uint16_t* shared_w;
  const int32_t* perm;
  const Tile* tiles;
  const int32_t* ntiles;
  uint16_t* out_r;
  uint16_t* out_s;
  int64_t M;
  int H, E, I, Is, k;
  int npan;
  int max_tiles;
};

// MODE 0: h = silu(A Wg^T) * (A Wu^T) over a 64-column panel of I (weight
//         rows 0..63 = gate rows, 64..127 = up rows of the same columns).
// MODE 1: y = A Wd^T over a 128-column panel of H.
template <int MODE>
__global__ __launch_bounds__(256, 2) void k_grouped_gemm(GemmArgs p) {
  __shared__ u32x4_t sB[2][BNR * (BK / 8)];  // 2 x 8 KB

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
  const bool is_shared = tl.g >= p.E;
  const int Ig = is_shared ? p.Is : p.I;

  const uint16_t* W = is_shared ? p.shared_w : p.expert_w + (int64_t)tl.g * 3 * p.I * p.H;
  int K, N, n0, ldw;
  const uint16_t* Wbase;
  if (MODE == 0) {
    n0 = panel * 64;
    if (n0 >= Ig) return;
    K = p.H;
    N = Ig;
    ldw = p.H;
    Wbase = W;  // gate [Ig][H], then up [Ig][H]
  } else {
    n0 = panel * BNR;
    K = Ig;
    N = p.H;
    ldw = Ig;
    Wbase = W + (int64_t)2 * Ig * p.H;  // down [H][Ig]
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;

  // ---- weight-tile loader: 512 chunks of 16 B per step, two per thread
  const u32x4_t* bsrc[2];
  bool bok[2];
  int bdst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, br = c >> 2, q = c & 3;
    int wrow;
    if (MODE == 0) {
      wrow = n0 + (br & 63);
      bok[i] = wrow < N;
      const uint16_t* base = br < 64 ? Wbase : Wbase + (int64_t)Ig * p.H;
      bsrc[i] = (const u32x4_t*)(base + (int64_t)(bok[i] ? wrow : 0) * ldw) + q;
    } else {
      wrow = n0 + br;
      bok[i] = wrow < N;
      bsrc[i] = (const u32x4_t*)(Wbase + (int64_t)(bok[i] ? wrow : 0) * ldw) + q;
    }
    bdst[i] = br * 4 + (q ^ ((br >> 1) & 3));
  }

  // ---- activation rows of this wave: rows 64*wave + 32*rb + lane%32
  const int wrow0 = 64 * wave;
  const bool wave_active = wrow0 < tl.rows;
  const u32x4_t* asrc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    int r = wrow0 + 32 * rb + (lane & 31);
    if (r >= tl.rows) r = 0;  // padding rows compute on row 0 and are never stored
    const uint16_t* rowp;
    if (MODE == 0) {
      const int64_t tok = is_shared ? (int64_t)tl.pos0 + r : (int64_t)(p.perm[tl.pos0 + r] / p.k);
      rowp = p.a_x + tok * p.H;
    } else {
      rowp = is_shared ? p.a_s + ((int64_t)tl.pos0 + r) * Ig : p.a_r + ((int64_t)tl.pos0 + r) * Ig;
    }
    asrc[rb] = (const u32x4_t*)rowp + half;
  }

  const u32x4_t zero = {0, 0, 0, 0};
  u32x4_t breg[2];
  u32x4_t acur[2][2], anxt[2][2];
  auto load_b = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) breg[i] = bok[i] ? bsrc[i][k0 >> 3] : zero;
  };
  auto store_b = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) sB[buf][bdst[i]] = breg[i];
  };
  auto load_a = [&](int k0, u32x4_t (&a)[2][2]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) a[rb][kk] = asrc[rb][(k0 >> 3) + 2 * kk];
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = (f32x16_t){};

  load_b(0);
  if (wave_active) load_a(0, acur);
  store_b(0);
  __syncthreads();
  const int nsteps = K / BK;
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) {
      load_b((s + 1) * BK);
      if (wave_active) load_a((s + 1) * BK, anxt);
    }
    if (wave_active) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4_t bf[4];
        const int q = 2 * kk + half;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int br = 32 * cb + (lane & 31);
          bf[cb] = sB[buf][br * 4 + (q ^ ((br >> 1) & 3))];
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, acur[rb][kk]), __builtin_bit_cast(bf16x8_t, bf[cb]),
                acc[rb][cb], 0, 0, 0);
      }
    }
    if (more) {
      store_b(buf ^ 1);
      if (wave_active) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) acur[rb][kk] = anxt[rb][kk];
      }
    }
    __syncthreads();
  }
  if (!wave_active) return;

  // ---- epilogue.  32x32 block D layout: lane -> column lane%32,
  //      register r -> row 8*(r/4) + 4*(lane/32) + r%4.
  const int col = lane & 31;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wrow0 + 32 * rb + 8 * (r >> 2) + 4 * half + (r & 3);
      if (row >= tl.rows) continue;
      if (MODE == 0) {
        uint16_t* orow = is_shared ? p.out_s + ((int64_t)tl.pos0 + row) * Ig
                                   : p.out_r + ((int64_t)tl.pos0 + row) * Ig;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int n = n0 + 32 * cb + col;
          const float g = acc[rb][cb][r], u = acc[rb][cb + 2][r];
          if (n < N) orow[n] = (uint16_t)f32_to_bf16(silu(g) * u);
        }
      } else {
        uint16_t* orow = is_shared ? p.out_s + ((int64_t)tl.pos0 + row) * p.H
                                   : p.out_r + ((int64_t)tl.pos0 + row) * p.H;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int n = n0 + 32 * cb + col;
          if (n < N) orow[n] = (uint16_t)f32_to_bf16(acc[rb][cb][r]);
        }
      }
    }
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
                              uint16_t* h_r, uint16_t* h_s, const Plan& pl, hipStream_t s) {
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
  a.npan = maxI / 64;
  a.max_tiles = (int)pl.max_tiles;
  hipLaunchKernelGGL(k_grouped_gemm<0>, dim3(xcd_grid(pl.max_tiles * a.npan)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const uint16_t* h_r, const uint16_t* h_s, const uint16_t* expert_w,
                            const uint16_t* shared_w, const Tile* tiles, const int32_t* ntiles,
                            uint16_t* y_r, uint16_t* y_s, const Plan& pl, hipStream_t s) {
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
  a.npan = (pl.H + BNR - 1) / BNR;
  a.max_tiles = (int)pl.max_tiles;
  hipLaunchKernelGGL(k_grouped_gemm<1>, dim3(xcd_grid(pl.max_tiles * a.npan)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y_r, const uint16_t* y_s, const float* w, const int32_t* inv,
                          uint16_t* out, const Plan& pl, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3((unsigned)pl.M), dim3(256), 0, s, y_r, pl.shared ? y_s : nullptr, w,
                     inv, out, pl.H, pl.k);
  return hipGetLastError();
}

}  // namespace moe
