// Small-batch path of the sparse MoE layer (up to 64 token rows; calls of up
// to 5 rows, 8 with 4-bit experts, run the decode kernels instead): matrix-
// vector work over the union of the experts the rows select (gfx950, wave64).
//
// "Optimizing on-device inference for Apple Silicon" (Perplexity 2026),
// section "Limits of further optimization": batches of a few rows (the
// verification step of speculative decoding) fit neither the one-row nor
// the many-row path, and their rows tend to pick different experts, so the
// expert bytes read grow with the row count.  "Ternary chunked prefill"
// (coreai-model-zoo knowledge page): a matrix-vector kernel widened to a few
// rows keeps those rows' activations close and reads every weight once for
// all of them.
//
// Here every expert in the union of the batch's selections is streamed from
// HBM once, and each weight chunk loaded is applied to all rows routed to
// that expert (up to four per register batch):
//   1. router scores: one wave per (expert, four token rows);
//   2. one workgroup: the top k and routing weights of every row, the union
//      as a compressed list (experts ascending, each with its assignments
//      t*k + j), and the down projection's work units;
//   3. gated activations: one wave per (union expert, gate/up row pair),
//      shared expert rows first (all rows use it);
//   4. down projection + combine: a workgroup per four output rows whose
//      waves share out the work units (up to four assignments of one
//      expert each); each assignment's weighted partial lands in its own
//      LDS slot, and the slots of a row are summed in slot order, shared
//      expert last.
// Results do not depend on the order of assignments inside an expert's list.
#include "moe_internal.h"
#include "wave_topk.h"
#include "weights.h"

namespace moe {
namespace {

constexpr int NP = kSmallRows;  // token rows per register batch
constexpr int DBS = 4;  // 16-byte chunks per lane per load batch: 4 x 64 lanes x 8 = 2048 elements
constexpr int DRS = 4;  // output rows per down-projection workgroup

// One wave: d1[p] = xs[p] . w and, with TWO, d2[p] = xs[p] . w2 over n
// elements (n % 8 == 0) for rows p < np <= NP, fp32, in every lane.  Each
// weight chunk is loaded once per batch and applied to all np rows; the
// caller points xs[p] for p >= np at a valid row (its results are unused).
template <bool TWO, class W>
__device__ __forceinline__ void wave_dots_rows(const uint16_t* const (&xs)[NP], int np, const typename W::Row w,
                                               const typename W::Row w2,
                                               int n, int lane, float (&d1)[NP], float (&d2)[NP]) {
  float a1[NP], a2[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) a1[p] = a2[p] = 0.0f;
  for (int base = 0; base < n; base += DBS * 512) {
    typename W::chunk_t wa[DBS], wb[DBS];
    u32x4_t xa[NP][DBS];
#pragma unroll
    for (int i = 0; i < DBS; ++i) {
      const int c = base + 512 * i + lane * 8;
      const int cc = c < n ? c : 0;
      wa[i] = w.load(cc);
      if (TWO) wb[i] = w2.load(cc);
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (p < np) xa[p][i] = *(const u32x4_t*)(xs[p] + cc);
    }
#pragma unroll
    for (int i = 0; i < DBS; ++i) {
      if (base + 512 * i + lane * 8 >= n) continue;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p >= np) continue;
        a1[p] += W::dot(wa[i], xa[p][i]);
        if (TWO) a2[p] += W::dot(wb[i], xa[p][i]);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p >= np) continue;
    d1[p] = wave_sum(a1[p]);
    if (TWO) d2[p] = wave_sum(a2[p]);
  }
}

// Exclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int s = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(s, d, 64);
    if (lane >= d) s += o;
  }
  return s - v;
}

// Router scores L[t][e] = x[t] . Wr[e] (+ bias[e]): one wave per (expert,
// group of NP token rows); workgroups of one token group are adjacent, so
// the groups after the first find the rows of Wr in cache.
__global__ __launch_bounds__(256) void k_sm_router(const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, int32_t* __restrict__ status,
                                                   int M, int H, int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *status = 0;  // no waits on this path
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  const WBf16::Row row{wr + (int64_t)e * H};
  const int t0 = blockIdx.y * NP;
  const int np = M - t0 < NP ? M - t0 : NP;
  const uint16_t* xs[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) xs[p] = x + (int64_t)(t0 + (p < np ? p : 0)) * H;
  float d[NP], unused[NP];
  wave_dots_rows<false, WBf16>(xs, np, row, row, H, lane, d, unused);
  if (lane == 0) {
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if (p < np) logits[(int64_t)(t0 + p) * E + e] = d[p] + b;
  }
}

// One workgroup (one wave per token row, up to 16 waves): top k of every
// row, routing weights = softmax over the selected scores, then the union
// of the selected experts as a compressed list:
//   un[0] = U (distinct experts), uexp[u] = u-th expert in ascending order,
//   uoff[u]..uoff[u+1]: its assignments in upair (values t*k + j);
// and the down projection's work units, each at most NP assignments of one
// item: un[1] = their number, unit[i] = (item << 16) | first, item 0 = the
// shared expert (first = token row), item u + 1 = union expert u (first =
// position in upair).  The shared expert's units come first.
template <int EPL>
__global__ __launch_bounds__(1024) void k_sm_topk(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                  float* __restrict__ wts, int32_t* __restrict__ un,
                                                  int32_t* __restrict__ uexp, int32_t* __restrict__ uoff,
                                                  int32_t* __restrict__ upair, int32_t* __restrict__ unit, int M,
                                                  int E, int k, int shared) {
  __shared__ uint64_t s_keys[16][64];
  __shared__ int32_t s_cnt[kMaxE];  // assignments per expert
  __shared__ int32_t s_pos[kMaxE];  // next free position of each expert's list
  __shared__ int16_t s_e[kMaxSmallM * kMaxTopK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int i = threadIdx.x; i < E; i += blockDim.x) s_cnt[i] = 0;
  __syncthreads();
  for (int t = wave; t < M; t += nw) {
    float f[EPL];
    load_scores<EPL>(logits + (int64_t)t * E, E, lane, f);
    uint64_t top;
    const uint64_t mine = wave_topk<EPL>(f, E, k, lane, &top, s_keys[wave]);
    const int ej = (int)(0xFFFFFFFFu - (uint32_t)mine);
    const float l0 = from_orderable((uint32_t)(top >> 32));
    const float lj = from_orderable((uint32_t)(mine >> 32));
    const float ex = lane < k ? expf(lj - l0) : 0.0f;
    const float sum = wave_sum(ex);
    if (lane < k) {
      ids[t * k + lane] = ej;
      wts[t * k + lane] = ex / sum;
      s_e[t * k + lane] = (int16_t)ej;
      atomicAdd(&s_cnt[ej], 1);
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane l owns experts [l*per, l*per + per), per = ceil(E / 64)
    const int per = (E + 63) >> 6;
    int tot = 0, nz = 0, nu = 0;
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      const int c = e < E ? s_cnt[e] : 0;
      tot += c;
      nz += c > 0;
      nu += (c + NP - 1) / NP;
    }
    const int sh_units = shared ? (M + NP - 1) / NP : 0;
    int pos = wave_excl_scan(tot, lane), u = wave_excl_scan(nz, lane);
    int ui = sh_units + wave_excl_scan(nu, lane);
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      const int c = e < E ? s_cnt[e] : 0;
      if (c > 0) {
        uexp[u] = e;
        uoff[u] = pos;
        s_pos[e] = pos;
        for (int f = 0; f < c; f += NP) unit[ui++] = ((u + 1) << 16) | (pos + f);
        pos += c;
        ++u;
      }
    }
    for (int i = lane; i < sh_units; i += 64) unit[i] = i * NP;  // item 0
    if (lane == 63) {  // the last lane ends with the totals
      uoff[u] = pos;
      un[0] = u;
      un[1] = ui;
    }
  }
  __syncthreads();
  for (int p = threadIdx.x; p < M * k; p += blockDim.x) upair[atomicAdd(&s_pos[s_e[p]], 1)] = p;
}

// Gated activations.  Workgroups [0, nsb): shared expert row i = 4*b + wave
// for every token row -> h_s[t][i].  Then workgroup b = nsb + u*rblocks + r:
// union expert u, row i = 4*r + wave, for each of its assignments a = t*k+j
// -> h_r[a][i] = silu(Wg[i] . x[t]) * (Wu[i] . x[t]).  Workgroups past the
// union's size exit at once.
template <class W>
__global__ __launch_bounds__(256) void k_sm_gateup(const uint16_t* __restrict__ x, const W expert_w,
                                                   const W shared_w, const int32_t* __restrict__ un,
                                                   const int32_t* __restrict__ uexp,
                                                   const int32_t* __restrict__ uoff,
                                                   const int32_t* __restrict__ upair, float* __restrict__ h_r,
                                                   float* __restrict__ h_s, int M, int H, int I, int Is, int k,
                                                   int nsb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* xs[NP];
  float dg[NP], du[NP];
  if ((int)blockIdx.x < nsb) {
    const int i = blockIdx.x * 4 + wave;
    if (i >= Is) return;
    const typename W::Row g = shared_w.gu(0, i, H, Is), u = shared_w.gu(1, i, H, Is);
    for (int t0 = 0; t0 < M; t0 += NP) {
      const int np = M - t0 < NP ? M - t0 : NP;
#pragma unroll
      for (int p = 0; p < NP; ++p) xs[p] = x + (int64_t)(t0 + (p < np ? p : 0)) * H;
      wave_dots_rows<true, W>(xs, np, g, u, H, lane, dg, du);
      if (lane == 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
          if (p < np) h_s[(int64_t)(t0 + p) * Is + i] = silu(dg[p]) * du[p];
      }
    }
    return;
  }
  const int rblocks = (I + 3) >> 2;
  const int b = blockIdx.x - nsb;
  const int ui = b / rblocks, i = (b - ui * rblocks) * 4 + wave;
  if (ui >= un[0] || i >= I) return;
  const W we = expert_w.block((int64_t)uexp[ui] * 3 * I * H);
  const typename W::Row g = we.gu(0, i, H, I), u = we.gu(1, i, H, I);
  const int a0 = uoff[ui], a1 = uoff[ui + 1];
  for (int q0 = a0; q0 < a1; q0 += NP) {
    const int np = a1 - q0 < NP ? a1 - q0 : NP;
    int as[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      as[p] = upair[q0 + (p < np ? p : 0)];
      xs[p] = x + (int64_t)(as[p] / k) * H;
    }
    wave_dots_rows<true, W>(xs, np, g, u, H, lane, dg, du);
    if (lane == 0) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (p < np) h_r[(int64_t)as[p] * I + i] = silu(dg[p]) * du[p];
    }
  }
}

// out[t][c] = sum_j w[t,j] * (Wd_{ids[t,j]}[c] . h_r[t*k+j]) + Sd[c] . h_s[t]
// for the DRS output rows c of this workgroup.  Wave w takes the work units
// w, w + waves, ... (at most NP assignments of one expert each, so a long
// list, e.g. the shared expert's, spreads over the waves): it loads the
// expert's DRS down rows and applies them to each assignment's h.  s_part
// (dynamic LDS): [M*k + M][DRS], assignment slots first, then one shared
// slot per token row.
template <class W>
__global__ __launch_bounds__(1024) void k_sm_down(const W expert_w, const W shared_w, const float* __restrict__ wts,
                                                  const int32_t* __restrict__ un, const int32_t* __restrict__ uexp,
                                                  const int32_t* __restrict__ uoff,
                                                  const int32_t* __restrict__ upair,
                                                  const int32_t* __restrict__ unit, const float* __restrict__ h_r,
                                                  const float* __restrict__ h_s, uint16_t* __restrict__ out, int M,
                                                  int H, int I, int Is, int k) {
  extern __shared__ float s_part[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int c0 = blockIdx.x * DRS;
  const bool shared = Is > 0;
  const int nunit = un[1];
  const int A = M * k;
  for (int it = wave; it < nunit; it += nw) {
    const int item = unit[it] >> 16, q0 = unit[it] & 0xFFFF;
    const bool sh = item == 0;
    int n, q1;
    W wd;
    if (sh) {
      n = Is;
      wd = shared_w;
      q1 = M;
    } else {
      n = I;
      wd = expert_w.block((int64_t)uexp[item - 1] * 3 * I * H);
      q1 = uoff[item];
    }
    const int np = q1 - q0 < NP ? q1 - q0 : NP;
    int slot[NP];
    const float* hp[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int q = q0 + (p < np ? p : 0);
      if (sh) {
        slot[p] = A + q;
        hp[p] = h_s + (int64_t)q * Is;
      } else {
        slot[p] = upair[q];
        hp[p] = h_r + (int64_t)slot[p] * I;
      }
    }
    float acc[NP][DRS];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < DRS; ++r) acc[p][r] = 0.0f;
    for (int base = 0; base < n; base += 512) {
      const int q = base + lane * 8;
      const bool ok = q < n;
      const int qq = ok ? q : 0;
      typename W::chunk_t b[DRS];
#pragma unroll
      for (int r = 0; r < DRS; ++r) {
        const int c = c0 + r < H ? c0 + r : H - 1;
        b[r] = wd.dn(c, H, n).load(qq);
      }
      f32x4_t h0[NP], h1[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (p >= np) continue;
        h0[p] = *(const f32x4_t*)(hp[p] + qq);
        h1[p] = *(const f32x4_t*)(hp[p] + qq + 4);
      }
      if (ok) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (p >= np) continue;
#pragma unroll
          for (int r = 0; r < DRS; ++r) acc[p][r] += W::dot(b[r], h0[p], h1[p]);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p >= np) continue;
      const float wj = sh ? 1.0f : wts[slot[p]];
#pragma unroll
      for (int r = 0; r < DRS; ++r) {
        const float v = wave_sum(acc[p][r]);
        if (lane == 0) s_part[slot[p] * DRS + r] = wj * v;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < M * DRS; idx += blockDim.x) {
    const int t = idx / DRS, r = idx - t * DRS;
    if (c0 + r >= H) continue;
    float v = 0.0f;
    for (int j = 0; j < k; ++j) v += s_part[(t * k + j) * DRS + r];  // slot order, shared last
    if (shared) v += s_part[(A + t) * DRS + r];
    out[(int64_t)t * H + c0 + r] = (uint16_t)f32_to_bf16(v);
  }
}

template <class W>
hipError_t small_gateup(const uint16_t* x, const W ew, const W sw, const SmallUnion& un, float* h, const Plan& p,
                        const Launch& lc) {
  const int nsb = p.shared ? (p.Is + 3) / 4 : 0;
  const int64_t umax = p.A < p.E ? p.A : p.E;
  const int64_t blocks = nsb + umax * ((p.I + 3) / 4);
  float* h_s = h + p.A * p.I;
  return launch(lc, k_sm_gateup<W>, dim3((unsigned)blocks), dim3(256), x, ew, sw, un.count, un.exp, un.off,
                un.pair, h, h_s, (int)p.M, p.H, p.I, p.Is, p.k, nsb);
}

template <class W>
hipError_t small_down(const W ew, const W sw, const float* w, const SmallUnion& un, const float* h, uint16_t* out,
                      const Plan& p, const Launch& lc) {
  const int64_t umax = p.A < p.E ? p.A : p.E;
  const int64_t units = umax + (p.shared ? 1 : 0);  // at least this many work units
  const int waves = units < 16 ? (int)units : 16;
  const size_t shm = (size_t)(p.A + p.M) * DRS * sizeof(float);
  const float* h_s = h + p.A * p.I;
  return launch_shm(lc, k_sm_down<W>, dim3((p.H + DRS - 1) / DRS), dim3(64 * waves), shm, ew, sw, w, un.count,
                    un.exp, un.off, un.pair, un.unit, h, h_s, out, (int)p.M, p.H, p.I, p.Is, p.k);
}

}  // namespace

hipError_t launch_small_router(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                               int32_t* status, const Plan& p, const Launch& lc) {
  return launch(lc, k_sm_router, dim3((p.E + 3) / 4, (unsigned)((p.M + NP - 1) / NP)), dim3(256), x, wr, bias,
                logits, status, (int)p.M, p.H, p.E);
}

hipError_t launch_small_topk(const float* logits, int32_t* ids, float* w, const SmallUnion& un, const Plan& p,
                             const Launch& lc) {
  const int waves = p.M < 16 ? (int)p.M : 16;
  const dim3 g(1), b(64 * waves);
  const int M = (int)p.M;
  const int sh = p.shared ? 1 : 0;
#define MOE_SM_TOPK(EPL) \
  launch(lc, k_sm_topk<EPL>, g, b, logits, ids, w, un.count, un.exp, un.off, un.pair, un.unit, M, p.E, p.k, sh)
  if (p.E <= 64) return MOE_SM_TOPK(1);
  if (p.E <= 128) return MOE_SM_TOPK(2);
  if (p.E <= 256) return MOE_SM_TOPK(4);
  if (p.E <= 512) return MOE_SM_TOPK(8);
  return MOE_SM_TOPK(16);
#undef MOE_SM_TOPK
}

hipError_t launch_small_gateup(const uint16_t* x, const uint16_t* expert_w, const uint16_t* shared_w,
                               const SmallUnion& un, float* h, const Plan& p, const Launch& lc) {
  const uint16_t* sw = p.shared ? shared_w : nullptr;
  if (p.tiled) return small_gateup(x, WBf16T{expert_w}, WBf16T{sw}, un, h, p, lc);
  return small_gateup(x, WBf16S{expert_w}, WBf16S{sw}, un, h, p, lc);
}

hipError_t launch_small_down(const uint16_t* expert_w, const uint16_t* shared_w, const float* w,
                             const SmallUnion& un, const float* h, uint16_t* out, const Plan& p, const Launch& lc) {
  const uint16_t* sw = p.shared ? shared_w : nullptr;
  if (p.tiled) return small_down(WBf16T{expert_w}, WBf16T{sw}, w, un, h, out, p, lc);
  return small_down(WBf16S{expert_w}, WBf16S{sw}, w, un, h, out, p, lc);
}

hipError_t launch_small_gateup_q4(const uint16_t* x, const Q4Weights& ex, const Q4Weights& sh, const SmallUnion& un,
                                  float* h, const Plan& p, const Launch& lc) {
  if (p.tiled) return small_gateup(x, WQ4T{ex.codes, ex.groups}, WQ4T{sh.codes, sh.groups}, un, h, p, lc);
  return small_gateup(x, WQ4{ex.codes, ex.groups}, WQ4{sh.codes, sh.groups}, un, h, p, lc);
}

hipError_t launch_small_down_q4(const Q4Weights& ex, const Q4Weights& sh, const float* w, const SmallUnion& un,
                                const float* h, uint16_t* out, const Plan& p, const Launch& lc) {
  if (p.tiled) return small_down(WQ4T{ex.codes, ex.groups}, WQ4T{sh.codes, sh.groups}, w, un, h, out, p, lc);
  return small_down(WQ4{ex.codes, ex.groups}, WQ4{sh.codes, sh.groups}, w, un, h, out, p, lc);
}

}  // namespace moe
