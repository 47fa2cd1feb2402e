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
// (one wave per output row: 64 lanes x 16 B = 1 KB per load instruction,
// contiguous) and fp32 wave reductions:
//   1. router scores (one wave per expert) and, independent of routing, the
//      shared expert's gate/up rows + SiLU gate (one wave per row);
//   2. top-k (recomputed by each workgroup from the scores) and the selected
//      experts' gate/up rows + SiLU gate;
//   3. the down projection of all selected experts and the shared expert,
//      weighted and summed in registers, one bf16 output per wave.
#include "moe_internal.h"
#include "wave_topk.h"

namespace moe {
namespace {

// dot(x[0:n], w[0:n]) for one wave, n % 8 == 0, both bf16 rows, fp32 result in all lanes
__device__ __forceinline__ float wave_dot_bf16(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ w, int n, int lane) {
  float acc = 0.0f;
  for (int c = lane * 8; c < n; c += 512) {
    const u32x4_t a = *(const u32x4_t*)(x + c);
    const u32x4_t b = *(const u32x4_t*)(w + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc += bf16_lo(a[q]) * bf16_lo(b[q]);
      acc += bf16_hi(a[q]) * bf16_hi(b[q]);
    }
  }
  return wave_sum(acc);
}

// Two rows (gate, up) against the same x, one pass over x.
__device__ __forceinline__ void wave_dot2_bf16(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ wg,
                                               const uint16_t* __restrict__ wu, int n, int lane,
                                               float* g, float* u) {
  float ag = 0.0f, au = 0.0f;
  for (int c = lane * 8; c < n; c += 512) {
    const u32x4_t a = *(const u32x4_t*)(x + c);
    const u32x4_t b = *(const u32x4_t*)(wg + c);
    const u32x4_t d = *(const u32x4_t*)(wu + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ag += bf16_lo(a[q]) * bf16_lo(b[q]);
      ag += bf16_hi(a[q]) * bf16_hi(b[q]);
      au += bf16_lo(a[q]) * bf16_lo(d[q]);
      au += bf16_hi(a[q]) * bf16_hi(d[q]);
    }
  }
  *g = wave_sum(ag);
  *u = wave_sum(au);
}

// Workgroups [0, nrouter) score experts, the rest compute the shared expert's gate.
__global__ __launch_bounds__(256) void k_dec_router_shared(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias,
                                                           const uint16_t* __restrict__ shared_w,
                                                           float* __restrict__ logits,
                                                           float* __restrict__ h_s, int H, int E,
                                                           int Is, int nrouter) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((int)blockIdx.x < nrouter) {
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    const float v = wave_dot_bf16(x, wr + (int64_t)e * H, H, lane);
    if (lane == 0) logits[e] = v + (bias ? bias[e] : 0.0f);
  } else {
    const int i = (blockIdx.x - nrouter) * 4 + wave;
    if (i >= Is) return;
    float g, u;
    wave_dot2_bf16(x, shared_w + (int64_t)i * H, shared_w + ((int64_t)Is + i) * H, H, lane, &g, &u);
    if (lane == 0) h_s[i] = silu(g) * u;
  }
}

// Each workgroup: wave 0 selects the top k from the E scores into LDS; then
// wave w computes row i = 4*(blockIdx % rows_blocks) + w of slot j's expert.
// Workgroup 0 also publishes ids / weights.  With I == 0 only the selection runs.
template <int EPL>
__global__ __launch_bounds__(256) void k_dec_gateup(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ expert_w,
                                                    const float* __restrict__ logits,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts,
                                                    float* __restrict__ h_r, int H, int E, int I,
                                                    int k) {
  __shared__ int32_t s_ids[kMaxTopK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    uint64_t top;
    const uint64_t mine = wave_topk<EPL>(logits, E, k, lane, &top);
    const int ej = (int)(0xFFFFFFFFu - (uint32_t)mine);
    if (lane < k) s_ids[lane] = ej;
    if (blockIdx.x == 0) {
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
  const int j = blockIdx.x / rblocks;
  const int i = (blockIdx.x % rblocks) * 4 + wave;
  if (j >= k || i >= I) return;
  const uint16_t* W = expert_w + (int64_t)s_ids[j] * 3 * I * H;
  float g, u;
  wave_dot2_bf16(x, W + (int64_t)i * H, W + ((int64_t)I + i) * H, H, lane, &g, &u);
  if (lane == 0) h_r[(int64_t)j * I + i] = silu(g) * u;
}

// out[c] = sum_j w_j * (Wd_{ids[j]}[c] . h_r[j]) + Sd[c] . h_s, one wave per c.
__global__ __launch_bounds__(256) void k_dec_down(const uint16_t* __restrict__ expert_w,
                                                  const uint16_t* __restrict__ shared_w,
                                                  const int32_t* __restrict__ ids,
                                                  const float* __restrict__ wts,
                                                  const float* __restrict__ h_r,
                                                  const float* __restrict__ h_s,
                                                  uint16_t* __restrict__ out, int H, int I, int Is,
                                                  int k) {
  __shared__ int32_t s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  if ((int)threadIdx.x < k) {
    s_ids[threadIdx.x] = ids[threadIdx.x];
    s_w[threadIdx.x] = wts[threadIdx.x];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + wave;
  if (c >= H) return;
  float total = 0.0f;
  for (int j = 0; j < k; ++j) {
    const uint16_t* wd = expert_w + (int64_t)s_ids[j] * 3 * I * H + (int64_t)2 * I * H + (int64_t)c * I;
    const float* hj = h_r + (int64_t)j * I;
    float acc = 0.0f;
    for (int q0 = lane * 8; q0 < I; q0 += 512) {
      const u32x4_t b = *(const u32x4_t*)(wd + q0);
      const f32x4_t h0 = *(const f32x4_t*)(hj + q0);
      const f32x4_t h1 = *(const f32x4_t*)(hj + q0 + 4);
      acc += bf16_lo(b[0]) * h0[0] + bf16_hi(b[0]) * h0[1] + bf16_lo(b[1]) * h0[2] +
             bf16_hi(b[1]) * h0[3];
      acc += bf16_lo(b[2]) * h1[0] + bf16_hi(b[2]) * h1[1] + bf16_lo(b[3]) * h1[2] +
             bf16_hi(b[3]) * h1[3];
    }
    total += s_w[j] * acc;
  }
  if (shared_w) {
    const uint16_t* wd = shared_w + (int64_t)2 * Is * H + (int64_t)c * Is;
    float acc = 0.0f;
    for (int q0 = lane * 8; q0 < Is; q0 += 512) {
      const u32x4_t b = *(const u32x4_t*)(wd + q0);
      const f32x4_t h0 = *(const f32x4_t*)(h_s + q0);
      const f32x4_t h1 = *(const f32x4_t*)(h_s + q0 + 4);
      acc += bf16_lo(b[0]) * h0[0] + bf16_hi(b[0]) * h0[1] + bf16_lo(b[1]) * h0[2] +
             bf16_hi(b[1]) * h0[3];
      acc += bf16_lo(b[2]) * h1[0] + bf16_hi(b[2]) * h1[1] + bf16_lo(b[3]) * h1[2] +
             bf16_hi(b[3]) * h1[3];
    }
    total += acc;
  }
  total = wave_sum(total);
  if (lane == 0) out[c] = (uint16_t)f32_to_bf16(total);
}

}  // namespace

hipError_t launch_decode_router_shared(const uint16_t* x, const uint16_t* wr, const float* bias,
                                       const uint16_t* shared_w, float* logits, float* h_s,
                                       const Plan& p, hipStream_t s) {
  const int nrouter = (p.E + 3) / 4;
  const int nshared = p.shared ? (p.Is + 3) / 4 : 0;
  hipLaunchKernelGGL(k_dec_router_shared, dim3(nrouter + nshared), dim3(256), 0, s, x, wr, bias,
                     shared_w, logits, h_s, p.H, p.E, p.shared ? p.Is : 0, nrouter);
  return hipGetLastError();
}

hipError_t launch_decode_gateup(const uint16_t* x, const uint16_t* expert_w, const float* logits,
                                int32_t* ids, float* w, float* h_r, const Plan& p, hipStream_t s) {
  // p.I == 0 requests the selection only (routing without expert work)
  const int blocks = p.I > 0 ? p.k * ((p.I + 3) / 4) : 1;
  dim3 g(blocks), b(256);
  if (p.E <= 64)
    hipLaunchKernelGGL(k_dec_gateup<1>, g, b, 0, s, x, expert_w, logits, ids, w, h_r, p.H, p.E, p.I, p.k);
  else if (p.E <= 128)
    hipLaunchKernelGGL(k_dec_gateup<2>, g, b, 0, s, x, expert_w, logits, ids, w, h_r, p.H, p.E, p.I, p.k);
  else if (p.E <= 256)
    hipLaunchKernelGGL(k_dec_gateup<4>, g, b, 0, s, x, expert_w, logits, ids, w, h_r, p.H, p.E, p.I, p.k);
  else if (p.E <= 512)
    hipLaunchKernelGGL(k_dec_gateup<8>, g, b, 0, s, x, expert_w, logits, ids, w, h_r, p.H, p.E, p.I, p.k);
  else
    hipLaunchKernelGGL(k_dec_gateup<16>, g, b, 0, s, x, expert_w, logits, ids, w, h_r, p.H, p.E, p.I, p.k);
  return hipGetLastError();
}

hipError_t launch_decode_down(const uint16_t* expert_w, const uint16_t* shared_w, const int32_t* ids,
                              const float* w, const float* h_dec, uint16_t* out, const Plan& p,
                              hipStream_t s) {
  const float* h_r = h_dec;
  const float* h_s = h_dec + (int64_t)p.k * p.I;
  hipLaunchKernelGGL(k_dec_down, dim3((p.H + 3) / 4), dim3(256), 0, s, expert_w,
                     p.shared ? shared_w : nullptr, ids, w, h_r, h_s, out, p.H, p.I, p.Is, p.k);
  return hipGetLastError();
}

}  // namespace moe
