// Routing kernels of the sparse MoE layer (gfx950, wave64).
//
// "Optimizing on-device inference for Apple Silicon" (Perplexity 2026),
// section "Keep expert routing on the GPU": after each token picks its
// experts, a histogram counts assignments per expert, a prefix scan turns
// counts into group offsets, a scatter places assignments in their expert's
// group and a block map lists the fixed-size tiles the grouped GEMM works
// on, all on the device with no host round trip.
//
// Design for CDNA4: tokens are handled in chunks of 64, one bit per token in
// a 64-bit mask per (chunk, expert).  The masks are built with LDS atomicOr
// (order-independent, so deterministic), counted with popcount, and a
// token's position inside its expert group is its chunk base plus the
// popcount of the mask bits below it -- a stable (ascending-token) scatter
// with no atomics on global memory.
#include "moe_internal.h"
#include "wave_topk.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ router scores

// L[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]); fp32 accumulate on MFMA.
// Tile 64 tokens x 64 experts (= one routing chunk), 4 waves in 2x2, each
// wave one 32x32 block, K in steps of 64 staged through LDS (double
// buffered, XOR-swizzled rows).  The tile also clears its chunk's bitmask
// words (cmask may be NULL on the decode path).
// Global loads run RD steps ahead in a register ring (loads past the end
// re-read the last step: never conditional, never out of bounds).
constexpr int RD = 4;
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ L,
                                                       uint64_t* __restrict__ cmask,
                                                       int32_t* __restrict__ status, int64_t M, int H, int E) {
  __shared__ u32x4_t sA[2][64 * 8];
  __shared__ u32x4_t sB[2][64 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int e0 = blockIdx.y * 64;
  const int wm = wave >> 1, wn = wave & 1;
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *status = 0;  // no waits on this path
  // this tile's (chunk, expert) bitmask words start empty; top-k sets their bits
  if (cmask && tid < 64 && e0 + tid < E) cmask[(int64_t)blockIdx.x * E + e0 + tid] = 0ull;

  // loader: 512 16-byte chunks per operand per step, two per thread.  Rows
  // past M (tokens) or E (experts) re-read row 0: they only reach output
  // rows / columns that are never stored, so the loaded registers go to LDS
  // untouched (a select on them would make every step wait for all loads).
  const u32x4_t* srcA[2];
  const u32x4_t* srcB[2];
  int dst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, row = c >> 3, q = c & 7;
    const int64_t t = t0 + row;
    const int e = e0 + row;
    srcA[i] = (const u32x4_t*)(x + (t < M ? t : 0) * (int64_t)H) + q;
    srcB[i] = (const u32x4_t*)(wr + (int64_t)(e < E ? e : 0) * H) + q;
    dst[i] = row * 8 + (q ^ ((row >> 1) & 7));
  }
  const int nsteps = H / 64;
  u32x4_t ra[RD][2], rb[RD][2];
  auto gload = [&](u32x4_t (&a)[2], u32x4_t (&b)[2], int st) {
    const int c0 = (st < nsteps ? st : nsteps - 1) * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = srcA[i][c0];
      b[i] = srcB[i][c0];
    }
  };
  auto lstore = [&](const u32x4_t (&a)[2], const u32x4_t (&b)[2], int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sA[buf][dst[i]] = a[i];
      sB[buf][dst[i]] = b[i];
    }
  };

  f32x16_t acc = {};
  const int arow = wm * 32 + (lane & 31), brow = wn * 32 + (lane & 31), half = lane >> 5;
#pragma unroll
  for (int st = 0; st < RD; ++st) gload(ra[st], rb[st], st);
  lstore(ra[0], rb[0], 0);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += RD) {
#pragma unroll
    for (int u = 0; u < RD; ++u) {
      const int s = s0 + u;
      const int buf = u & 1;
      if (s < nsteps) {
        u32x4_t a[4], b[4];  // all operand reads of the step first, then the MFMAs
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int q = 2 * kk + half;
          a[kk] = sA[buf][arow * 8 + (q ^ ((arow >> 1) & 7))];
          b[kk] = sB[buf][brow * 8 + (q ^ ((brow >> 1) & 7))];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[kk]),
                                                         __builtin_bit_cast(bf16x8_t, b[kk]), acc, 0, 0, 0);
      }
      gload(ra[u], rb[u], s + RD);
      lstore(ra[(u + 1) % RD], rb[(u + 1) % RD], buf ^ 1);
      __syncthreads();
    }
  }
  // D layout of the 32x32 block: lane -> column, register r -> row 8(r/4) + 4(lane/32) + r%4
  const int e = e0 + wn * 32 + (lane & 31);
  if (e < E) {
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t t = t0 + wm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (t < M) L[t * E + e] = acc[r] + bv;
    }
  }
}

// ------------------------------------------------------------------ top-k

// One wave per token (4 per workgroup): top-k, weights, and the token's bit
// in each selected expert's (chunk, expert) mask (64-bit atomicOr: the
// result does not depend on the order of the ORs).
template <int EPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ L, int32_t* __restrict__ ids,
                                              float* __restrict__ w, uint64_t* __restrict__ cmask,
                                              int64_t M, int E, int k) {
  __shared__ uint64_t s_keys[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= M) return;
  float f[EPL];
  load_scores<EPL>(L + t * E, E, lane, f);
  uint64_t top;
  const uint64_t mine = wave_topk<EPL>(f, E, k, lane, &top, s_keys[wave]);
  const float l0 = from_orderable((uint32_t)(top >> 32));
  const float lj = from_orderable((uint32_t)(mine >> 32));
  const int ej = (int)(0xFFFFFFFFu - (uint32_t)mine);
  const float ex = lane < k ? expf(lj - l0) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[t * k + lane] = ej;
    w[t * k + lane] = ex / sum;
    atomicOr((unsigned long long*)&cmask[(t / kChunk) * E + ej], 1ull << (t % kChunk));
  }
}

// ------------------------------------------------------------------ scan + block map

// Exclusive scan of one int per thread over a 1024-thread block.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int wv = lane < 16 ? s_wave[lane] : 0;
    int wi = wv;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int o = __shfl_up(wi, d, 64);
      if (lane >= d) wi += o;
    }
    if (lane < 16) s_wave[16 + lane] = wi - wv;  // exclusive prefix of wave totals
    if (lane == 15) s_wave[32] = wi;
  }
  __syncthreads();
  const int r = s_wave[16 + wave] + incl - v;
  *total = s_wave[32];
  __syncthreads();
  return r;
}

// Counts, offsets, the block map and its launch-order copy (tiles_lpt),
// from each expert's assignment count `total` (thread e < E; 0 elsewhere),
// its exclusive offset `off` and the routed total.  Every thread of the
// 1024-thread block calls it (it synchronises).
//
// Tiles of kTileM rows; a group's last 1..32 rows past a multiple of kTileM
// stay with the tile before (the last tile takes up to kTileM + 32 rows), so
// that group's weights are streamed once fewer.  The shared expert's tiles
// (all M tokens in order) follow the routed ones.  Launch order: class c =
// 32-row blocks of a tile (full tiles 8, a group's last tile 1..9), classes
// from 9 down, so that the longest units start first and the short ones fill
// the end of the launch; the order inside a class is that of the LDS atomics
// (it decides which workgroup runs a tile, not what is computed); the shared
// expert's tiles after them as in the block map.
__device__ void write_block_map(int total, int off, int routed_total, int32_t* __restrict__ counts,
                                int32_t* __restrict__ offsets, Tile* __restrict__ tiles,
                                int32_t* __restrict__ ntiles, Tile* __restrict__ tiles_lpt, int* s_wave,
                                int* s_cls, int64_t M, int E, int shared) {
  const int tid = threadIdx.x;
  const int nt = tid < E && total > 0 ? (total <= kTileM + 32 ? 1 : (total - 32 + kTileM - 1) / kTileM) : 0;
  int routed_tiles;
  const int tstart = block_exclusive_scan(nt, s_wave, &routed_tiles);
  if (tid < E) {
    counts[tid] = total;
    offsets[tid] = off;
    for (int i = 0; i < nt; ++i) {
      const int r0 = i * kTileM;
      Tile tl;
      tl.g = tid;
      tl.r0 = r0;
      tl.rows = i == nt - 1 ? total - r0 : kTileM;
      tl.pos0 = off + r0;
      tiles[tstart + i] = tl;
    }
  }
  if (tid == 0) offsets[E] = routed_total;
  const int nts = shared ? (int)((M + kTileM - 1) / kTileM) : 0;
  for (int i = tid; i < nts; i += 1024) {
    Tile tl;
    tl.g = E;
    tl.r0 = i * kTileM;
    tl.rows = (int)(M - tl.r0 < kTileM ? M - tl.r0 : kTileM);
    tl.pos0 = tl.r0;
    tiles[routed_tiles + i] = tl;
  }
  if (tid == 0) *ntiles = routed_tiles + nts;
  if (tid < 10) s_cls[tid] = 0;
  __syncthreads();
  const int last_rows = nt > 0 ? total - (nt - 1) * kTileM : 0;
  if (tid < E && nt > 0) {
    if (nt > 1) atomicAdd(&s_cls[8], nt - 1);
    atomicAdd(&s_cls[(last_rows + 31) >> 5], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = 9; c >= 1; --c) {
      const int v = s_cls[c];
      s_cls[c] = run;
      run += v;
    }
  }
  __syncthreads();
  if (tid < E && nt > 0) {
    const int f = nt > 1 ? atomicAdd(&s_cls[8], nt - 1) : 0;
    for (int i = 0; i < nt - 1; ++i) tiles_lpt[f + i] = Tile{tid, i * kTileM, kTileM, off + i * kTileM};
    const int r0 = (nt - 1) * kTileM;
    tiles_lpt[atomicAdd(&s_cls[(last_rows + 31) >> 5], 1)] = Tile{tid, r0, last_rows, off + r0};
  }
  for (int i = tid; i < nts; i += 1024) {
    Tile tl;
    tl.g = E;
    tl.r0 = i * kTileM;
    tl.rows = (int)(M - tl.r0 < kTileM ? M - tl.r0 : kTileM);
    tl.pos0 = tl.r0;
    tiles_lpt[routed_tiles + i] = tl;
  }
}

// Single workgroup (calls of more than kFusedScanChunks chunks; smaller ones
// take k_route_scan_scatter).  Reads the per-(chunk, expert) masks, writes counts,
// offsets, the block map, and cbase = the group position of the chunk's
// first assignment to each expert.  Also the same tiles in the order the
// gate/up launch takes them (tiles_lpt): the routed tiles by count of 32-row
// blocks, most first, so that the longest units start first and the short
// ones fill the end of the launch, then the shared expert's in order.
__global__ __launch_bounds__(1024) void k_route_scan(const uint64_t* __restrict__ cmask,
                                                     int32_t* __restrict__ cbase,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     Tile* __restrict__ tiles,
                                                     int32_t* __restrict__ ntiles,
                                                     Tile* __restrict__ tiles_lpt, int64_t M, int E,
                                                     int k, int shared) {
  __shared__ int s_part[1024];
  __shared__ int s_wave[40];
  __shared__ int s_cls[10];  // routed tiles per count of 32-row blocks (1..9), then each class's next slot
  const int tid = threadIdx.x;
  const int64_t nchunk = (M + kChunk - 1) / kChunk;
  const int P = 1024 / E;  // threads per expert (E <= 1024)
  const int e = tid % E, part = tid / E;
  const bool active = part < P;
  const int64_t cpp = (nchunk + P - 1) / P;
  const int64_t c0 = active ? (int64_t)part * cpp : 0;
  const int64_t c1 = active ? (c0 + cpp < nchunk ? c0 + cpp : nchunk) : 0;

  // pass 1: partial counts per (part, expert)
  int psum = 0;
  {
    int64_t c = c0;
    for (; c + 8 <= c1; c += 8) {  // eight independent loads in flight
      uint64_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = cmask[(c + j) * E + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) psum += __popcll(v[j]);
    }
    for (; c < c1; ++c) psum += __popcll(cmask[c * E + e]);
  }
  s_part[tid] = active ? psum : 0;
  __syncthreads();
  // expert totals (thread e < E), exclusive scan over experts
  int total = 0;
  if (tid < E)
    for (int p = 0; p < P; ++p) total += s_part[p * E + tid];
  int routed_total;
  const int off = block_exclusive_scan(tid < E ? total : 0, s_wave, &routed_total);
  write_block_map(tid < E ? total : 0, off, routed_total, counts, offsets, tiles, ntiles, tiles_lpt, s_wave, s_cls, M,
                  E, shared);
  // pass 2: chunk bases.  s_part[part*E + e] -> start of the part within expert e
  __syncthreads();
  if (tid < E) {
    int run = off;
    for (int p = 0; p < P; ++p) {
      const int v = s_part[p * E + tid];
      s_part[p * E + tid] = run;
      run += v;
    }
  }
  __syncthreads();
  if (active) {
    int run = s_part[tid];
    int64_t c = c0;
    for (; c + 8 <= c1; c += 8) {
      uint64_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = cmask[(c + j) * E + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cbase[(c + j) * E + e] = run;
        run += __popcll(v[j]);
      }
    }
    for (; c < c1; ++c) {
      cbase[c * E + e] = run;
      run += __popcll(cmask[c * E + e]);
    }
  }
}

// ------------------------------------------------------------------ scatter

// perm[p] = t*k + j and inv[t*k + j] = p for every assignment, where p is the
// chunk base of (chunk, expert) plus the number of earlier tokens of the chunk
// routed to that expert.
__global__ __launch_bounds__(256) void k_route_scatter(const int32_t* __restrict__ ids,
                                                       const uint64_t* __restrict__ cmask,
                                                       const int32_t* __restrict__ cbase,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv, int64_t M, int E,
                                                       int k) {
  const int64_t c = blockIdx.x;
  for (int idx = threadIdx.x; idx < kChunk * k; idx += 256) {
    const int tl = idx & (kChunk - 1), j = idx >> 6;
    const int64_t t = c * kChunk + tl;
    if (t >= M) continue;
    const int64_t a = t * k + j;
    const int e = ids[a];
    const uint64_t m = cmask[c * E + e];
    const int p = cbase[c * E + e] + __popcll(m & ((1ull << tl) - 1ull));
    perm[p] = (int32_t)a;
    inv[a] = p;
  }
}

// ------------------------------------------------------------------ scan + scatter in one launch

// One 1024-thread workgroup per 64-token chunk c, for calls of at most
// kFusedScanChunks chunks.  Every workgroup counts the assignments of every
// (chunk, expert) mask: the group offsets need all of them and chunk c's
// base in expert e's group is offset(e) plus the assignments to e of the
// chunks before c.  Then it scatters chunk c's assignments (the arithmetic
// of k_route_scatter); workgroup 0 also writes counts, offsets and the block
// map.  This replaces the single-workgroup scan and the scatter launch: the
// masks (128 KB at 4096 tokens) are read by every workgroup from the L2
// instead of twice by one workgroup.
constexpr int kFusedScanChunks = 128;
constexpr int kFusedScanBatch = 16;  // mask loads in flight per thread
__global__ __launch_bounds__(1024) void k_route_scan_scatter(const int32_t* __restrict__ ids,
                                                             const uint64_t* __restrict__ cmask,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             Tile* __restrict__ tiles,
                                                             int32_t* __restrict__ ntiles,
                                                             Tile* __restrict__ tiles_lpt,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv, int64_t M, int E, int k,
                                                             int shared) {
  __shared__ int s_tot[1024];       // per (part, expert): assignments in the part's chunks
  __shared__ int s_pre[1024];       // per (part, expert): the same, chunks before c only
  __shared__ uint64_t s_cm[kMaxE];  // chunk c's mask per expert
  __shared__ int s_base[kMaxE];     // chunk c's first position in each expert's group
  __shared__ int s_wave[40];
  __shared__ int s_cls[10];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int nchunk = (int)((M + kChunk - 1) / kChunk);
  const int P = 1024 / E;  // threads per expert (E <= 1024)
  const int e = tid % E, part = tid / E;
  const bool active = part < P;
  const int cpp = (nchunk + P - 1) / P;
  const int c0 = active ? part * cpp : 0;
  const int c1 = active ? (c0 + cpp < nchunk ? c0 + cpp : nchunk) : 0;

  // this thread's assignments of chunk c (at most two: 64 tokens x k <= 2048),
  // their experts loaded before the masks
  int my_a[2], my_e[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = tid + 1024 * r;
    const int tl = idx & (kChunk - 1), j = idx >> 6;
    const int64_t t = (int64_t)c * kChunk + tl;
    const bool ok = j < k && t < M;
    my_a[r] = ok ? (int)(t * k + j) : -1;
    my_e[r] = ok ? ids[t * k + j] : 0;
  }

  int tot = 0, pre = 0;
  for (int cc = c0; cc < c1; cc += kFusedScanBatch) {
    uint64_t v[kFusedScanBatch];
#pragma unroll
    for (int j = 0; j < kFusedScanBatch; ++j) {
      const int ch = cc + j < c1 ? cc + j : c1 - 1;  // clamped: never past the part
      v[j] = cmask[(int64_t)ch * E + e];
    }
#pragma unroll
    for (int j = 0; j < kFusedScanBatch; ++j) {
      if (cc + j >= c1) break;
      const int pc = __popcll(v[j]);
      tot += pc;
      if (cc + j < c) pre += pc;
      if (cc + j == c) s_cm[e] = v[j];
    }
  }
  s_tot[tid] = active ? tot : 0;
  s_pre[tid] = active ? pre : 0;
  __syncthreads();
  int total = 0, before = 0;
  if (tid < E)
    for (int p = 0; p < P; ++p) {
      total += s_tot[p * E + tid];
      before += s_pre[p * E + tid];
    }
  int routed_total;
  const int off = block_exclusive_scan(tid < E ? total : 0, s_wave, &routed_total);
  if (tid < E) s_base[tid] = off + before;
  if (blockIdx.x == 0)  // uniform in the workgroup
    write_block_map(tid < E ? total : 0, off, routed_total, counts, offsets, tiles, ntiles, tiles_lpt, s_wave, s_cls,
                    M, E, shared);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (my_a[r] < 0) continue;
    const int tl = (tid + 1024 * r) & (kChunk - 1);
    const int p = s_base[my_e[r]] + __popcll(s_cm[my_e[r]] & ((1ull << tl) - 1ull));
    perm[p] = my_a[r];
    inv[my_a[r]] = p;
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, float* L,
                                uint64_t* cmask, int32_t* status, int64_t M, int H, int E, const Launch& lc) {
  dim3 grid((unsigned)((M + 63) / 64), (unsigned)((E + 63) / 64));
  return launch(lc, k_router_logits, grid, dim3(256), x, wr, bias, L, cmask, status, M, H, E);
}

hipError_t launch_topk(const float* L, int32_t* ids, float* w, uint64_t* cmask, int64_t M, int E, int k,
                       const Launch& lc) {
  dim3 grid((unsigned)((M + 3) / 4));
  if (E <= 64) return launch(lc, k_topk<1>, grid, dim3(256), L, ids, w, cmask, M, E, k);
  if (E <= 128) return launch(lc, k_topk<2>, grid, dim3(256), L, ids, w, cmask, M, E, k);
  if (E <= 256) return launch(lc, k_topk<4>, grid, dim3(256), L, ids, w, cmask, M, E, k);
  if (E <= 512) return launch(lc, k_topk<8>, grid, dim3(256), L, ids, w, cmask, M, E, k);
  return launch(lc, k_topk<16>, grid, dim3(256), L, ids, w, cmask, M, E, k);
}

hipError_t launch_route_scan(const uint64_t* cmask, int32_t* cbase, int32_t* counts, int32_t* offsets,
                             Tile* tiles, int32_t* ntiles, Tile* tiles_lpt, int64_t M, int E, int k, bool shared,
                             const Launch& lc) {
  return launch(lc, k_route_scan, dim3(1), dim3(1024), cmask, cbase, counts, offsets, tiles, ntiles, tiles_lpt, M,
                E, k, shared ? 1 : 0);
}

bool route_scan_fused(int64_t M) { return (M + kChunk - 1) / kChunk <= kFusedScanChunks; }

hipError_t launch_route_scan_scatter(const int32_t* ids, const uint64_t* cmask, int32_t* counts, int32_t* offsets,
                                     Tile* tiles, int32_t* ntiles, Tile* tiles_lpt, int32_t* perm, int32_t* inv,
                                     int64_t M, int E, int k, bool shared, const Launch& lc) {
  dim3 grid((unsigned)((M + kChunk - 1) / kChunk));
  return launch(lc, k_route_scan_scatter, grid, dim3(1024), ids, cmask, counts, offsets, tiles, ntiles, tiles_lpt, perm,
                inv, M, E, k, shared ? 1 : 0);
}

hipError_t launch_route_scatter(const int32_t* ids, const uint64_t* cmask, const int32_t* cbase,
                                int32_t* perm, int32_t* inv, int64_t M, int E, int k, const Launch& lc) {
  dim3 grid((unsigned)((M + kChunk - 1) / kChunk));
  return launch(lc, k_route_scatter, grid, dim3(256), ids, cmask, cbase, perm, inv, M, E, k);
}

}  // namespace moe
