// Batch-1 decode path of the sparse MoE layer (gfx950, wave64).
//
// "Optimizing on-device inference for Apple Silicon" (Perplexity 2026):
//  - section "Optimize the single-row weight path": with one activation row
//    the layer is matrix-vector work; a SIMD group cooperates on one output
//    while its lanes read different parts of the weight matrix;
//  - section "Reduce intermediate and state traffic": the two input expert
//    projections are fused with their gated activation, and the output
//    projection with its routing score and the shared expert's result;
//  - section "Limits of further optimization": the sparse GEMV is bound by
//    weight reads, not arithmetic.
//
// Three kernels per layer, all streaming bf16 weight rows with 16-byte loads
// (64 lanes x 16 B = 1 KB contiguous per load instruction) and fp32 wave
// reductions:
//   1. router scores (one wave per expert);
//   2. the shared expert's gate/up rows + SiLU gate, which stream while the
//      other workgroups select the top k from the scores (each workgroup
//      selects for itself), then the selected experts' gate/up rows + SiLU;
//   3. the down projection: one wave per (expert slot, 4 output rows), the
//      weighted slot partials summed in slot order through LDS.
#include "moe_internal.h"
#include "wave_topk.h"
#include "weights.h"

namespace moe {
namespace {

// Every wave issues all of its loads before using any of them (fixed-size
// register batches, addresses clamped in bounds, contributions masked), so
// a wave costs one memory round trip, not one per loop iteration.
constexpr int DB = 4;  // 16-byte chunks per lane per batch: 4 x 64 lanes x 8 = 2048 elements

// dot(x[0:n], w[0:n]) and dot(x, w2) for one wave (n % 8 == 0), fp32 in all
// lanes; w, w2 are weight rows of format W.
template <bool TWO, class W>
__device__ __forceinline__ void wave_dots(const uint16_t* __restrict__ x, const typename W::Row w,
                                          const typename W::Row w2, int n, int lane, float* d1, float* d2) {
  float a1 = 0.0f, a2 = 0.0f;
  for (int base = 0; base < n; base += DB * 512) {
    u32x4_t xa[DB];
    typename W::chunk_t wa[DB], wb[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      const int c = base + 512 * i + lane * 8;
      const int cc = c < n ? c : 0;
      xa[i] = *(const u32x4_t*)(x + cc);
      wa[i] = w.load(cc);
      if (TWO) wb[i] = w2.load(cc);
    }
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      if (base + 512 * i + lane * 8 >= n) continue;
      a1 += W::dot(wa[i], xa[i]);
      if (TWO) a2 += W::dot(wb[i], xa[i]);
    }
  }
  *d1 = wave_sum(a1);
  if (TWO) *d2 = wave_sum(a2);
}

// Router scores: one wave per expert; with ROWS, grid row r works on token row r.
template <bool ROWS>
__global__ __launch_bounds__(256) void k_dec_router(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wr,
                                                    const float* __restrict__ bias,
                                                    float* __restrict__ logits, int32_t* __restrict__ status,
                                                    int H, int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = 0;  // three launches: no waits
  if (ROWS) {
    x += (int64_t)blockIdx.y * H;
    logits += (int64_t)blockIdx.y * E;
  }
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  float v, unused;
  const WBf16::Row row{wr + (int64_t)e * H};
  wave_dots<false, WBf16>(x, row, row, H, lane, &v, &unused);
  if (lane == 0) logits[e] = v + (bias ? bias[e] : 0.0f);
}

// Gated activations of the shared and the selected experts, one wave per
// (gate, up) row pair.  Workgroups [0, nshared) take the shared expert's
// rows, which do not depend on the routing, so they stream while the other
// workgroups select: there wave 0 takes the top k of the E scores into LDS,
// then wave w computes row i = 4*(b % row_blocks) + w of slot j's expert.
// The first routed workgroup also publishes ids / weights.  With I == 0 only
// the selection runs.  With ROWS, grid row r works on token row r (h_r:
// [rows][k][I], h_s: [rows][Is]).
template <int EPL, class W, bool ROWS>
__global__ __launch_bounds__(256) void k_dec_gateup(const uint16_t* __restrict__ x, const W expert_w,
                                                    const W shared_w, const float* __restrict__ logits,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts,
                                                    float* __restrict__ h_r, float* __restrict__ h_s,
                                                    int H, int E, int I, int Is, int k, int nshared) {
  __shared__ int32_t s_ids[kMaxTopK];
  __shared__ uint64_t s_keys[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (ROWS) {
    const int64_t row = blockIdx.y;
    x += row * H;
    logits += row * E;
    ids += row * k;
    wts += row * k;
    h_r += row * k * I;
    h_s += row * Is;
  }
  if ((int)blockIdx.x < nshared) {
    const int i = blockIdx.x * 4 + wave;
    if (i >= Is) return;
    float g, u;
    wave_dots<true, W>(x, shared_w.gu(0, i, H, Is), shared_w.gu(1, i, H, Is), H, lane, &g, &u);
    if (lane == 0) h_s[i] = silu(g) * u;
    return;
  }
  const int b = blockIdx.x - nshared;
  if (wave == 0) {
    uint64_t top;
    float f[EPL];
    load_scores<EPL>(logits, E, lane, f);
    const uint64_t mine = wave_topk<EPL>(f, E, k, lane, &top, s_keys);
    const int ej = (int)(0xFFFFFFFFu - (uint32_t)mine);
    if (lane < k) s_ids[lane] = ej;
    if (b == 0) {
      const float l0 = from_orderable((uint32_t)(top >> 32));
      const float lj = from_orderable((uint32_t)(mine >> 32));
      const float ex = lane < k ? expf(lj - l0) : 0.0f;
      const float sum = wave_sum(ex);
      if (lane < k) {
        ids[lane] = ej;
        wts[lane] = ex / sum;
      }
    }
  }
  __syncthreads();
  if (I == 0) return;
  const int rblocks = (I + 3) / 4;
  const int j = b / rblocks;
  const int i = (b % rblocks) * 4 + wave;
  if (j >= k || i >= I) return;
  const W ew = expert_w.block((int64_t)s_ids[j] * 3 * I * H);
  float g, u;
  wave_dots<true, W>(x, ew.gu(0, i, H, I), ew.gu(1, i, H, I), H, lane, &g, &u);
  if (lane == 0) h_r[(int64_t)j * I + i] = silu(g) * u;
}

// out[c] = sum_j w_j * (Wd_{ids[j]}[c] . h_r[j]) + Sd[c] . h_s.
// Workgroup = one wave per expert slot (slot k = shared expert), DR output
// rows each; every wave loads its DR weight rows and its h slice at once,
// reduces, and the slot partials are summed in slot order through LDS.
// With ROWS, grid row r works on token row r.
constexpr int DR = 4;
template <class W, bool ROWS>
__global__ __launch_bounds__(1024) void k_dec_down(const W expert_w, const W shared_w,
                                                   const int32_t* __restrict__ ids,
                                                   const float* __restrict__ wts,
                                                   const float* __restrict__ h_r,
                                                   const float* __restrict__ h_s,
                                                   uint16_t* __restrict__ out, int H, int I, int Is,
                                                   int k, int nslot) {
  __shared__ float s_part[kMaxTopK + 1][DR];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = blockIdx.x * DR;
  if (ROWS) {
    const int64_t row = blockIdx.y;
    ids += row * k;
    wts += row * k;
    h_r += row * k * I;
    h_s += row * Is;
    out += row * H;
  }
  // slots wave, wave + nwaves, ... (one pass when k + 1 <= waves per workgroup)
  for (int j = wave; j < nslot; j += blockDim.x >> 6) {
    const bool sh = j == k;  // the shared expert
    const int n = sh ? Is : I;
    W wd;
    const float* hj;
    float wj = 1.0f;
    if (sh) {
      wd = shared_w;
      hj = h_s;
    } else {
      wd = expert_w.block((int64_t)ids[j] * 3 * I * H);
      hj = h_r + (int64_t)j * I;
      wj = wts[j];
    }
    float part[DR];
#pragma unroll
    for (int r = 0; r < DR; ++r) part[r] = 0.0f;
    for (int base = 0; base < n; base += 512) {
      const int q0 = base + lane * 8;
      const bool ok = q0 < n;
      const int qq = ok ? q0 : 0;
      typename W::chunk_t b[DR];
#pragma unroll
      for (int r = 0; r < DR; ++r) {
        const int c = c0 + r < H ? c0 + r : H - 1;
        b[r] = wd.dn(c, H, n).load(qq);
      }
      const f32x4_t h0 = *(const f32x4_t*)(hj + qq);
      const f32x4_t h1 = *(const f32x4_t*)(hj + qq + 4);
      if (ok) {
#pragma unroll
        for (int r = 0; r < DR; ++r) part[r] += W::dot(b[r], h0, h1);
      }
    }
#pragma unroll
    for (int r = 0; r < DR; ++r) {
      const float v = wave_sum(part[r]);
      if (lane == 0) s_part[j][r] = wj * v;
    }
  }
  __syncthreads();
  if (threadIdx.x < DR && c0 + (int)threadIdx.x < H) {
    float v = 0.0f;
    for (int j = 0; j < nslot; ++j) v += s_part[j][threadIdx.x];  // slot order, shared last
    out[c0 + threadIdx.x] = (uint16_t)f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------- the layer in two launches
//
// Launch 1 (k_dec_route): the router scores (one wave per expert), the
// shared expert's gated activations (one wave per (gate, up) row pair: they
// do not depend on the routing, so they stream beside the router rows), and
// the reset of the per-slot arrival counters and the status word.
//
// Launch 2 (k_dec_experts): every workgroup selects the top k from the
// scores.  The first k * ceil(I / kDW) workgroups compute the selected
// experts' gated activations, one wave per row pair (the arithmetic of
// k_dec_gateup).  The last ndown workgroups own kDRW output rows per wave:
// they issue the loads of those rows of the down projections of every
// selected expert and of the shared expert at once, before any h exists,
// then wait until every gate/up workgroup of every slot has arrived, read h,
// and sum the slots in slot order (shared last), the arithmetic of
// k_dec_down.  Publication: h is written with agent-scope stores (through
// the L2, which is not coherent between the XCDs); every wave waits until
// its store is complete, and after a workgroup barrier one thread adds the
// workgroup's arrival to its slot's counter.  A down workgroup polls the
// counters with agent-scope loads, then reads h with agent-scope loads,
// which return every value stored before the arrivals it saw.  Only down
// workgroups wait, and only for gate/up workgroups, which wait for nothing
// and come first in the grid: workgroups are dispatched in the order of
// their index, so every gate/up workgroup holds a compute unit before any
// down workgroup does, whatever the grid size and whatever else runs on the
// device.  The wait is also bounded: after kDecSpinLimit polls a down
// workgroup gives up, writes NaN to its output rows and 1 to the status
// word.
constexpr int kDW = 8;                 // waves per workgroup of the expert launch
constexpr int kDRW = 2;                // output rows per wave of a down workgroup
constexpr int kDSB = 9;                // slots whose down rows are loaded at once (top-8 + shared)
constexpr int kDecSpinLimit = 1 << 20;  // polls (each a memory round trip + a short sleep): about a second
constexpr int kDecProbeSpins = 64;      // polls of the wait probe (a condition that never occurs)

template <class W>
__global__ __launch_bounds__(256) void k_dec_route(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   const W shared_w, float* __restrict__ h_s,
                                                   uint32_t* __restrict__ arrivals, int32_t* __restrict__ status,
                                                   int H, int E, int Is, int k, int nrouter) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (blockIdx.x == 0) {
    if ((int)threadIdx.x < k)
      __hip_atomic_store(arrivals + threadIdx.x * kArriveStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0 && status) __hip_atomic_store(status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if ((int)blockIdx.x < nrouter) {
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    float v, unused;
    const WBf16::Row row{wr + (int64_t)e * H};
    wave_dots<false, WBf16>(x, row, row, H, lane, &v, &unused);
    if (lane == 0) logits[e] = v + (bias ? bias[e] : 0.0f);
    return;
  }
  const int i = (blockIdx.x - nrouter) * 4 + wave;
  if (i >= Is) return;
  float g, u;
  wave_dots<true, W>(x, shared_w.gu(0, i, H, Is), shared_w.gu(1, i, H, Is), H, lane, &g, &u);
  if (lane == 0) h_s[i] = silu(g) * u;
}

template <int EPL, class W>
__global__ __launch_bounds__(512) void k_dec_experts(const uint16_t* __restrict__ x, const W expert_w,
                                                     const W shared_w, const float* __restrict__ logits,
                                                     int32_t* __restrict__ ids, float* __restrict__ wts,
                                                     float* __restrict__ h_r, const float* __restrict__ h_s,
                                                     uint32_t* __restrict__ arrivals, int32_t* __restrict__ status,
                                                     uint16_t* __restrict__ out, int H, int E, int I, int Is, int k,
                                                     int probe) {
  extern __shared__ __attribute__((aligned(16))) float s_h[];  // down workgroups: h of slots 0 .. k-1 ([k][I]), then the shared expert's [Is]
  __shared__ int32_t s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ uint64_t s_keys[64];
  __shared__ int s_fail;
  __shared__ float s_hv[kDW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rblocks = (I + kDW - 1) / kDW;  // gate/up workgroups per slot
  if (wave == 0) {
    uint64_t top;
    float f[EPL];
    load_scores<EPL>(logits, E, lane, f);
    const uint64_t mine = wave_topk<EPL>(f, E, k, lane, &top, s_keys);
    const int ej = (int)(0xFFFFFFFFu - (uint32_t)mine);
    const float l0 = from_orderable((uint32_t)(top >> 32));
    const float lj = from_orderable((uint32_t)(mine >> 32));
    const float ex = lane < k ? expf(lj - l0) : 0.0f;
    const float sum = wave_sum(ex);
    if (lane < k) {
      s_ids[lane] = ej;
      s_w[lane] = ex / sum;
      if (blockIdx.x == 0) {  // one workgroup publishes the selection
        ids[lane] = ej;
        wts[lane] = ex / sum;
      }
    }
  }
  __syncthreads();

  const int ngu = k * rblocks;  // gate/up workgroups: the first ngu of the grid
  if ((int)blockIdx.x < ngu) {  // gated activations of slot j's expert, rows i0 .. i0 + kDW - 1
    const int b = blockIdx.x;
    const int j = b / rblocks, i0 = (b % rblocks) * kDW, i = i0 + wave;
    if (i < I) {
      const W ew = expert_w.block((int64_t)s_ids[j] * 3 * I * H);
      float g, u;
      wave_dots<true, W>(x, ew.gu(0, i, H, I), ew.gu(1, i, H, I), H, lane, &g, &u);
      if (lane == 0) s_hv[wave] = silu(g) * u;
    }
    __syncthreads();
    // one wave publishes the workgroup's kDW values: one store, then (once it is
    // complete) one arrival
    if (wave == 0) {
      if (lane < kDW && i0 + lane < I)
        __hip_atomic_store(h_r + (int64_t)j * I + i0 + lane, s_hv[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0)
        __hip_atomic_fetch_add(arrivals + j * kArriveStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // ---- down workgroup: output rows c0 .. c0 + kDRW - 1 of this wave
  const int db = (int)blockIdx.x - ngu;
  const int nslot = k + (Is > 0 ? 1 : 0);
  const int c0 = (db * kDW + wave) * kDRW;
  typename W::chunk_t wv[kDSB][kDRW];
  // loads of slots jb .. jb + kDSB - 1 (slot k = the shared expert); slots past
  // the last and lanes past a row's end re-read valid elements, never used
  auto issue = [&](int jb) {
#pragma unroll
    for (int s = 0; s < kDSB; ++s) {
      const int j = jb + s < nslot ? jb + s : 0;
      const bool sh = j == k;
      const int n = sh ? Is : I;
      const W wd = sh ? shared_w : expert_w.block((int64_t)s_ids[j] * 3 * I * H);
      const int q = lane * 8 < n ? lane * 8 : 0;
#pragma unroll
      for (int r = 0; r < kDRW; ++r) {
        const int c = c0 + r < H ? c0 + r : H - 1;
        wv[s][r] = wd.dn(c, H, n).load(q);
      }
    }
  };
  issue(0);

  // wait until every gate/up workgroup has arrived (bounded)
  if (wave == 0) {
    const uint32_t target = probe ? 0xFFFFFFFFu : (uint32_t)rblocks;
    const int limit = probe ? kDecProbeSpins : kDecSpinLimit;
    int spins = 0;
    bool ok = false;
    for (;;) {
      const uint32_t a = lane < k ? __hip_atomic_load(arrivals + lane * kArriveStride, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                  : target;
      if (__all(a >= target)) {
        ok = true;
        break;
      }
      if (++spins >= limit) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) s_fail = ok ? 0 : 1;
  }
  __syncthreads();
  if (s_fail) {  // gave up: NaN rows, status 1
    if (tid < kDW * kDRW) {
      const int c = db * kDW * kDRW + tid;
      if (c < H) out[c] = (uint16_t)0x7FC0u;
    }
    if (tid == 0 && status) __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // h of every slot into LDS: the routed slots with agent-scope loads, the
  // shared expert's from the previous launch
  {
    const uint64_t* hr64 = (const uint64_t*)h_r;
    const int n64 = k * I / 2;
    for (int q = tid; q < n64; q += kDW * 64) {
      const uint64_t v = __hip_atomic_load(hr64 + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_h[2 * q] = __uint_as_float((uint32_t)v);
      s_h[2 * q + 1] = __uint_as_float((uint32_t)(v >> 32));
    }
    for (int q = tid; q < Is; q += kDW * 64) s_h[k * I + q] = h_s[q];
  }
  __syncthreads();

  float acc[kDRW];
#pragma unroll
  for (int r = 0; r < kDRW; ++r) acc[r] = 0.0f;
  for (int jb = 0; jb < nslot; jb += kDSB) {
    if (jb > 0) issue(jb);
#pragma unroll
    for (int s = 0; s < kDSB; ++s) {
      const int j = jb + s;
      if (j >= nslot) break;  // uniform
      const bool sh = j == k;
      const int n = sh ? Is : I;
      const bool ok = lane * 8 < n;
      const float* hj = s_h + (int64_t)j * I + (ok ? lane * 8 : 0);
      const f32x4_t h0 = *(const f32x4_t*)hj;
      const f32x4_t h1 = *(const f32x4_t*)(hj + 4);
      const float wj = sh ? 1.0f : s_w[j];
#pragma unroll
      for (int r = 0; r < kDRW; ++r) {
        const float part = ok ? W::dot(wv[s][r], h0, h1) : 0.0f;
        const float d = wave_sum(part);
        {
          // slot order, shared last; the product rounded before the sum (no fused
          // multiply-add), as the three-launch and the small-batch paths compute it
#pragma clang fp contract(off)
          const float wd = wj * d;
          acc[r] = acc[r] + wd;
        }
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < kDRW; ++r)
      if (c0 + r < H) out[c0 + r] = (uint16_t)f32_to_bf16(acc[r]);
  }
}

}  // namespace

hipError_t launch_decode_router(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                                int32_t* status, const Plan& p, const Launch& lc) {
  const dim3 g((p.E + 3) / 4, (unsigned)p.M);
  if (p.M > 1) return launch(lc, k_dec_router<true>, g, dim3(256), x, wr, bias, logits, status, p.H, p.E);
  return launch(lc, k_dec_router<false>, g, dim3(256), x, wr, bias, logits, status, p.H, p.E);
}

namespace {

template <class W, bool ROWS>
hipError_t decode_gateup_launch(dim3 g, dim3 b, const uint16_t* x, const W ew, const W sw, const float* logits,
                                int32_t* ids, float* w, float* h_dec, float* h_s, int nshared, const Plan& p,
                                const Launch& lc) {
#define MOE_DEC_GATEUP(EPL) \
  launch(lc, k_dec_gateup<EPL, W, ROWS>, g, b, x, ew, sw, logits, ids, w, h_dec, h_s, p.H, p.E, p.I, p.Is, p.k, nshared)
  if (p.E <= 64) return MOE_DEC_GATEUP(1);
  if (p.E <= 128) return MOE_DEC_GATEUP(2);
  if (p.E <= 256) return MOE_DEC_GATEUP(4);
  if (p.E <= 512) return MOE_DEC_GATEUP(8);
  return MOE_DEC_GATEUP(16);
#undef MOE_DEC_GATEUP
}

template <class W>
hipError_t decode_gateup(const uint16_t* x, const W ew, const W sw, const float* logits, int32_t* ids, float* w,
                         float* h_dec, const Plan& p, const Launch& lc) {
  // p.I == 0 requests the selection only (routing without expert work)
  const int nshared = p.shared && p.I > 0 ? (p.Is + 3) / 4 : 0;
  const int blocks = nshared + (p.I > 0 ? p.k * ((p.I + 3) / 4) : 1);
  float* h_s = h_dec + p.M * p.k * p.I;
  const dim3 g(blocks, (unsigned)p.M), b(256);
  if (p.M > 1) return decode_gateup_launch<W, true>(g, b, x, ew, sw, logits, ids, w, h_dec, h_s, nshared, p, lc);
  return decode_gateup_launch<W, false>(g, b, x, ew, sw, logits, ids, w, h_dec, h_s, nshared, p, lc);
}

template <class W>
hipError_t decode_down(const W ew, const W sw, const int32_t* ids, const float* w, const float* h_dec,
                       uint16_t* out, const Plan& p, const Launch& lc) {
  const float* h_r = h_dec;
  const float* h_s = h_dec + p.M * p.k * p.I;
  const int nslot = p.k + (p.shared ? 1 : 0);
  const int waves = nslot < 16 ? nslot : 16;
  const dim3 g((p.H + DR - 1) / DR, (unsigned)p.M), b(64 * waves);
  if (p.M > 1) return launch(lc, k_dec_down<W, true>, g, b, ew, sw, ids, w, h_r, h_s, out, p.H, p.I, p.Is, p.k, nslot);
  return launch(lc, k_dec_down<W, false>, g, b, ew, sw, ids, w, h_r, h_s, out, p.H, p.I, p.Is, p.k, nslot);
}

}  // namespace

hipError_t launch_decode_gateup(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                                const float* logits, int32_t* ids, float* w, float* h_dec, const Plan& p,
                                const Launch& lc) {
  const uint16_t* sw = p.shared ? shared_w : nullptr;
  if (p.tiled) return decode_gateup(x, WBf16T{expert_w}, WBf16T{sw}, logits, ids, w, h_dec, p, lc);
  return decode_gateup(x, WBf16S{expert_w}, WBf16S{sw}, logits, ids, w, h_dec, p, lc);
}

hipError_t launch_decode_down(const uint16_t* expert_w, const uint16_t* shared_w, const int32_t* ids,
                              const float* w, const float* h_dec, uint16_t* out, const Plan& p,
                              const Launch& lc) {
  const uint16_t* sw = p.shared ? shared_w : nullptr;
  if (p.tiled) return decode_down(WBf16T{expert_w}, WBf16T{sw}, ids, w, h_dec, out, p, lc);
  return decode_down(WBf16S{expert_w}, WBf16S{sw}, ids, w, h_dec, out, p, lc);
}

namespace {

template <class W>
hipError_t decode_route(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits, const W sw,
                        float* h_dec, uint32_t* arrivals, int32_t* status, const Plan& p, const Launch& lc) {
  const int nrouter = (p.E + 3) / 4;
  const int nshared = p.shared ? (p.Is + 3) / 4 : 0;
  float* h_s = h_dec + (int64_t)p.k * p.I;
  return launch(lc, k_dec_route<W>, dim3(nrouter + nshared), dim3(256), x, wr, bias, logits, sw, h_s, arrivals,
                status, p.H, p.E, p.Is, p.k, nrouter);
}

template <class W>
hipError_t decode_experts(const uint16_t* x, const W ew, const W sw, const float* logits, int32_t* ids, float* w,
                          float* h_dec, uint32_t* arrivals, int32_t* status, uint16_t* out, const Plan& p, int probe,
                          const Launch& lc) {
  const int ndown = (p.H + kDW * kDRW - 1) / (kDW * kDRW);
  const int blocks = ndown + p.k * ((p.I + kDW - 1) / kDW);
  const size_t shm = ((size_t)p.k * p.I + p.Is) * 4;
  const float* h_s = h_dec + (int64_t)p.k * p.I;
  const dim3 g(blocks), b(kDW * 64);
#define MOE_DEC_EXPERTS(EPL) \
  launch_shm(lc, k_dec_experts<EPL, W>, g, b, shm, x, ew, sw, logits, ids, w, h_dec, h_s, arrivals, status, out, \
             p.H, p.E, p.I, p.Is, p.k, probe)
  if (p.E <= 64) return MOE_DEC_EXPERTS(1);
  if (p.E <= 128) return MOE_DEC_EXPERTS(2);
  if (p.E <= 256) return MOE_DEC_EXPERTS(4);
  if (p.E <= 512) return MOE_DEC_EXPERTS(8);
  return MOE_DEC_EXPERTS(16);
#undef MOE_DEC_EXPERTS
}

}  // namespace

bool decode_two_launch_fits(const Plan& p) {
  // one 8-element chunk per lane per down row; at most 256 down workgroups
  return p.I <= 512 && p.Is <= 512 && p.H <= 4096 && ((int64_t)p.k * p.I + p.Is) * 4 <= 64 * 1024;
}

hipError_t launch_decode_route(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                               const uint16_t* shared_w, float* h_dec, uint32_t* arrivals, int32_t* status,
                               const Plan& p, const Launch& lc) {
  const uint16_t* sw = p.shared ? shared_w : nullptr;
  if (p.tiled) return decode_route(x, wr, bias, logits, WBf16T{sw}, h_dec, arrivals, status, p, lc);
  return decode_route(x, wr, bias, logits, WBf16S{sw}, h_dec, arrivals, status, p, lc);
}

hipError_t launch_decode_route_q4(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                                  const Q4Weights& sh, float* h_dec, uint32_t* arrivals, int32_t* status,
                                  const Plan& p, const Launch& lc) {
  if (p.tiled) return decode_route(x, wr, bias, logits, WQ4T{sh.codes, sh.groups}, h_dec, arrivals, status, p, lc);
  return decode_route(x, wr, bias, logits, WQ4{sh.codes, sh.groups}, h_dec, arrivals, status, p, lc);
}

hipError_t launch_decode_experts(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                                 const float* logits, int32_t* ids, float* w, float* h_dec, uint32_t* arrivals,
                                 int32_t* status, uint16_t* out, const Plan& p, int probe, const Launch& lc) {
  const uint16_t* sw = p.shared ? shared_w : nullptr;
  if (p.tiled)
    return decode_experts(x, WBf16T{expert_w}, WBf16T{sw}, logits, ids, w, h_dec, arrivals, status, out, p, probe, lc);
  return decode_experts(x, WBf16S{expert_w}, WBf16S{sw}, logits, ids, w, h_dec, arrivals, status, out, p, probe, lc);
}

hipError_t launch_decode_experts_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh, const float* logits,
                                    int32_t* ids, float* w, float* h_dec, uint32_t* arrivals, int32_t* status,
                                    uint16_t* out, const Plan& p, int probe, const Launch& lc) {
  if (p.tiled)
    return decode_experts(x, WQ4T{ex.codes, ex.groups}, WQ4T{sh.codes, sh.groups}, logits, ids, w, h_dec, arrivals,
                          status, out, p, probe, lc);
  return decode_experts(x, WQ4{ex.codes, ex.groups}, WQ4{sh.codes, sh.groups}, logits, ids, w, h_dec, arrivals,
                        status, out, p, probe, lc);
}

hipError_t launch_decode_gateup_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh,
                                   const float* logits, int32_t* ids, float* w, float* h_dec, const Plan& p,
                                   const Launch& lc) {
  if (p.tiled) return decode_gateup(x, WQ4T{ex.codes, ex.groups}, WQ4T{sh.codes, sh.groups}, logits, ids, w, h_dec, p, lc);
  return decode_gateup(x, WQ4{ex.codes, ex.groups}, WQ4{sh.codes, sh.groups}, logits, ids, w, h_dec, p, lc);
}

hipError_t launch_decode_down_q4(const Q4Weights& ex, const Q4Weights& sh, const int32_t* ids, const float* w,
                                 const float* h_dec, uint16_t* out, const Plan& p, const Launch& lc) {
  if (p.tiled) return decode_down(WQ4T{ex.codes, ex.groups}, WQ4T{sh.codes, sh.groups}, ids, w, h_dec, out, p, lc);
  return decode_down(WQ4{ex.codes, ex.groups}, WQ4{sh.codes, sh.groups}, ids, w, h_dec, out, p, lc);
}

}  // namespace moe
