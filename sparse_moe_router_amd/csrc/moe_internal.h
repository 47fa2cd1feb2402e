// Internal declarations shared by the kernels and the C-ABI host code of the
// sparse MoE layer library (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ----------------------------------------------------------------- constants

constexpr int kChunk = 64;    // tokens per routing chunk: one bit per token in a 64-bit mask
constexpr int kTileM = 256;   // rows per grouped-GEMM tile (block-map granularity)
constexpr int kMaxE = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxSmallM = 64;  // most rows the matrix-vector paths take
constexpr int kSmallRows = 4;   // small-batch path: assignments per register batch / work unit
constexpr int kArriveStride = 64;  // decode, two launches: one arrival counter per 256-byte line

// ----------------------------------------------------------------- vector types

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// ----------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (the native conversion)
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// silu(z) = z * sigmoid(z), with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ----------------------------------------------------------------- workspace plan

// One tile of the block map: rows [r0, r0+rows) of group g.  pos0 is the
// first row's index into the group-ordered row space: for a routed group it
// is offsets[g] + r0 (a position in perm order), for the shared group (g == E)
// it is the token index r0.
struct Tile {
  int32_t g, r0, rows, pos0;
};

struct Plan {
  // shapes
  int64_t M;
  int32_t H, E, I, Is, k;
  bool shared;
  bool gemv;  // decode path
  bool tiled;  // bf16 expert weights in the tiled layout (WBf16T)
  int64_t A;  // assignments M*k
  int64_t nchunk;
  int64_t max_tiles;
  // byte offsets into the workspace (all 256-aligned)
  size_t logits, ids, w, cmask, cbase, counts, offsets, perm, inv, tiles, ntiles, h_r, h_s, y_r;
  size_t tiles_lpt;  // grouped path: the block map's tiles in launch order
  size_t un_count, un_exp, un_off, un_pair, un_unit;  // small-batch path: union of the selected experts
  size_t arrive;  // decode path, two launches: arrival counters of the gate/up workgroups, one per slot
  size_t total;
};

// Fills `p` for the given shapes; returns false on overflow.
bool make_plan(Plan* p, int64_t M, int H, int E, int I, int Is, int k, bool gemv);

// ----------------------------------------------------------------- launchers
// All launchers enqueue on L.s and return hipGetLastError() of the launch.
// When L carries events, the kernel is launched with hipExtLaunchKernelGGL,
// which stamps them with the kernel's own start and end (the same interval
// a kernel-trace profiler reports), for live per-kernel timing.

struct Launch {
  hipStream_t s;
  hipEvent_t start;
  hipEvent_t stop;
};

template <typename F, typename... Args>
inline hipError_t launch_shm(const Launch& L, F kernel, dim3 grid, dim3 block, size_t shm, Args... args) {
  if (L.start || L.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, shm, L.s, L.start, L.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, L.s, args...);
  return hipGetLastError();
}
template <typename F, typename... Args>
inline hipError_t launch(const Launch& L, F kernel, dim3 grid, dim3 block, Args... args) {
  return launch_shm(L, kernel, grid, block, 0, args...);
}

// 4-bit group-affine weights of one or E experts (packing as the bf16 blocks):
// codes, 8 per 32-bit word; one (scale, bias) word per 64 elements.
struct Q4Weights {
  const uint32_t* codes;
  const uint32_t* groups;
};

// Router scores L[M][E] = x Wr^T (+ bias), fp32 (MFMA); clears the chunk masks.
// *status (if given) = 0: this path has no in-kernel waits.
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, float* L,
                                uint64_t* cmask, int32_t* status, int64_t M, int H, int E, const Launch& lc);
// Top-k + weights per token, and the token's bits in the per-chunk expert masks.
hipError_t launch_topk(const float* L, int32_t* ids, float* w, uint64_t* cmask, int64_t M, int E, int k,
                       const Launch& lc);
// counts, offsets, per-chunk bases, block map; the same tiles in the gate/up
// launch's order (tiles_lpt: the routed tiles by count of 32-row blocks,
// most first, then the shared expert's in order).
hipError_t launch_route_scan(const uint64_t* cmask, int32_t* cbase, int32_t* counts, int32_t* offsets,
                             Tile* tiles, int32_t* ntiles, Tile* tiles_lpt, int64_t M, int E, int k, bool shared,
                             const Launch& lc);
// perm / inv from the chunk masks and bases.
hipError_t launch_route_scatter(const int32_t* ids, const uint64_t* cmask, const int32_t* cbase,
                                int32_t* perm, int32_t* inv, int64_t M, int E, int k, const Launch& lc);
// Scan, block map and scatter in one launch (one workgroup per 64-token
// chunk), for calls of at most 8192 tokens (route_scan_fused); the
// chunk-base table is not written.
bool route_scan_fused(int64_t M);
hipError_t launch_route_scan_scatter(const int32_t* ids, const uint64_t* cmask, int32_t* counts, int32_t* offsets,
                                     Tile* tiles, int32_t* ntiles, Tile* tiles_lpt, int32_t* perm, int32_t* inv,
                                     int64_t M, int E, int k, bool shared, const Launch& lc);
// Grouped gate/up GEMM + SwiGLU -> h (bf16) over the tiles in its launch
// order (tiles_lpt of launch_route_scan), leaving out the last skip_tail (the
// shared expert's, when the down launch runs them).
hipError_t launch_gemm_gateup(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                              const int32_t* perm, const Tile* tiles, const int32_t* ntiles,
                              uint16_t* h_r, uint16_t* h_s, int skip_tail, const Plan& p, const Launch& lc);
// Grouped down GEMM -> y (bf16) over the block map, leaving out its last
// skip_tail tiles (the shared expert's, when launch_shared_down_combine does
// them).  With x_shared_gu given, the launch first runs the shared expert's
// gate/up tiles (x -> h_s), which the gate/up launch then leaves out.
hipError_t launch_gemm_down(const uint16_t* h_r, uint16_t* h_s, const uint16_t* expert_w,
                            const uint16_t* shared_w, const Tile* tiles, const int32_t* ntiles,
                            uint16_t* y_r, uint16_t* y_s, int skip_tail, const uint16_t* x_shared_gu,
                            const Plan& p, const Launch& lc);
// The shared expert's down GEMM over the tokens in tiles of 128, with the
// weighted combine of the routed rows in its epilogue:
// out[t] = sum_j w[t,j] y_r[inv[t*k+j]] + (Sd h_s[t]) (bf16 out).
hipError_t launch_shared_down_combine(const uint16_t* h_s, const uint16_t* shared_w, const uint16_t* y_r,
                                      const float* w, const int32_t* inv, uint16_t* out, const Plan& p,
                                      const Launch& lc);
// The two grouped GEMMs reading 4-bit weights (same outputs and layouts).
hipError_t launch_gemm_gateup_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh, const int32_t* perm,
                                 const Tile* tiles, const int32_t* ntiles, uint16_t* h_r, uint16_t* h_s,
                                 int skip_tail, const Plan& p, const Launch& lc);
hipError_t launch_gemm_down_q4(const uint16_t* h_r, uint16_t* h_s, const Q4Weights& ex, const Q4Weights& sh,
                               const Tile* tiles, const int32_t* ntiles, uint16_t* y_r, uint16_t* y_s, int skip_tail,
                               const uint16_t* x_shared_gu, const Plan& p, const Launch& lc);
hipError_t launch_shared_down_combine_q4(const uint16_t* h_s, const Q4Weights& sh, const uint16_t* y_r,
                                         const float* w, const int32_t* inv, uint16_t* out, const Plan& p,
                                         const Launch& lc);
// out[t] = y_s[t] + sum_j w[t,j] y_r[inv[t*k+j]]  (bf16 out)
hipError_t launch_combine(const uint16_t* y_r, const uint16_t* y_s, const float* w, const int32_t* inv,
                          uint16_t* out, const Plan& p, const Launch& lc);

// Decode (M == 1) path.
// Router scores.
hipError_t launch_decode_router(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                                int32_t* status, const Plan& p, const Launch& lc);
// Shared and selected experts' gated activations (h_dec: fp32 [k][I] routed,
// then [Is] shared); top-k ids and weights.
hipError_t launch_decode_gateup(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                                const float* logits, int32_t* ids, float* w, float* h_dec, const Plan& p,
                                const Launch& lc);
hipError_t launch_decode_down(const uint16_t* expert_w, const uint16_t* shared_w, const int32_t* ids,
                              const float* w, const float* h_dec, uint16_t* out, const Plan& p,
                              const Launch& lc);

// The decode layer in two launches (MOE_FLAG_DECODE_TWO_LAUNCH, when
// decode_two_launch_fits(p): I, Is <= 512, H <= 4096, the h of all slots
// within 64 KB of LDS): launch 1
// writes the router scores and the shared expert's h and resets the
// arrival counters (and *status, if given); launch 2 selects, computes the
// routed h and the down projections + combine, the down workgroups waiting
// in the launch for the routed h (bounded; on giving up, NaN rows and
// *status = 1).  probe != 0 makes that wait one that never ends (test hook:
// the give-up path).  Same results as the three-launch path.
bool decode_two_launch_fits(const Plan& p);
hipError_t launch_decode_route(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                               const uint16_t* shared_w, float* h_dec, uint32_t* arrivals, int32_t* status,
                               const Plan& p, const Launch& lc);
hipError_t launch_decode_route_q4(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                                  const Q4Weights& sh, float* h_dec, uint32_t* arrivals, int32_t* status,
                                  const Plan& p, const Launch& lc);
hipError_t launch_decode_experts(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                                 const float* logits, int32_t* ids, float* w, float* h_dec, uint32_t* arrivals,
                                 int32_t* status, uint16_t* out, const Plan& p, int probe, const Launch& lc);
hipError_t launch_decode_experts_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh, const float* logits,
                                    int32_t* ids, float* w, float* h_dec, uint32_t* arrivals, int32_t* status,
                                    uint16_t* out, const Plan& p, int probe, const Launch& lc);

// The decode kernels above, reading 4-bit weights (same outputs and layout).
hipError_t launch_decode_gateup_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh,
                                   const float* logits, int32_t* ids, float* w, float* h_dec, const Plan& p,
                                   const Launch& lc);
hipError_t launch_decode_down_q4(const Q4Weights& ex, const Q4Weights& sh, const int32_t* ids, const float* w,
                                 const float* h_dec, uint16_t* out, const Plan& p, const Launch& lc);

// Small-batch path (2 <= M <= kMaxSmallM): matrix-vector products over the
// union of the experts the rows select.  h: fp32 [M*k][I] per assignment,
// then [M][Is] shared.
struct SmallUnion {
  int32_t* count;  // [2] distinct experts U, down-projection work units
  int32_t* exp;    // [min(E, M*k)] experts, ascending
  int32_t* off;    // [U+1] list offsets into pair
  int32_t* pair;   // [M*k] assignments t*k + j, grouped by expert
  int32_t* unit;   // [small_units(M, k, E)] down-projection work units
};
// Most work units: one per kSmallRows assignments of each expert, rounded
// up per expert (at most min(E, M*k) roundings), plus the shared expert's.
inline int64_t small_units(int64_t M, int k, int E) {
  const int64_t A = M * k;
  return (A < E ? A : E) + (A + kSmallRows - 1) / kSmallRows + (M + kSmallRows - 1) / kSmallRows;
}
hipError_t launch_small_router(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                               int32_t* status, const Plan& p, const Launch& lc);
hipError_t launch_small_topk(const float* logits, int32_t* ids, float* w, const SmallUnion& un, const Plan& p,
                             const Launch& lc);
hipError_t launch_small_gateup(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                               const SmallUnion& un, float* h, const Plan& p, const Launch& lc);
hipError_t launch_small_down(const uint16_t* expert_w, const uint16_t* shared_w, const float* w,
                             const SmallUnion& un, const float* h, uint16_t* out, const Plan& p, const Launch& lc);
hipError_t launch_small_gateup_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh, const SmallUnion& un,
                                  float* h, const Plan& p, const Launch& lc);
hipError_t launch_small_down_q4(const Q4Weights& ex, const Q4Weights& sh, const float* w, const SmallUnion& un,
                                const float* h, uint16_t* out, const Plan& p, const Launch& lc);

// nblocks bf16 expert blocks (hidden H, intermediate I) from the row-major
// packing to the tiled layout read with MOE_FLAG_TILED_WEIGHTS.
hipError_t launch_tile_weights(const uint16_t* src, uint16_t* dst, int64_t nblocks, int H, int I, hipStream_t s);
hipError_t launch_tile_weights_q4(const uint32_t* codes, const uint32_t* groups, uint32_t* codes_dst,
                                  uint32_t* groups_dst, int64_t nblocks, int H, int I, hipStream_t s);

}  // namespace moe
