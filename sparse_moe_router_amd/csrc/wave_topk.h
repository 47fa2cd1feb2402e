// Wave-level top-k selection over one token's router scores (wave64).
// Ranking: descending score, equal scores -> lower expert index first.
#pragma once

#include "moe_internal.h"

namespace moe {

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0 is folded onto +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b << 1) == 0) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// Selection key: score first, then the LOWER expert index wins a tie.
__device__ __forceinline__ uint64_t sel_key(float f, int e) {
  return ((uint64_t)orderable(f) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

// DPP move of v (lanes whose source is outside the row or masked off read 0).
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                               BANK_MASK, true));
}

// Sum over the 64 lanes of a wave (all lanes active), in every lane.  Data
// parallel primitives on the VALU, no LDS round trips: shift-and-add within
// each 16-lane row (row_shr 1, 2, 4, 8 leave the row's sum in its lane 15),
// then row_bcast:15 adds row 0 into row 1 and row 2 into row 3, and
// row_bcast:31 adds lane 31 into rows 2 and 3, so lane 63 holds the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0x111>(v);       // row_shr:1
  v += dpp_move<0x112>(v);       // row_shr:2
  v += dpp_move<0x114>(v);       // row_shr:4
  v += dpp_move<0x118>(v);       // row_shr:8
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Loads lane's scores of one token (experts lane, lane+64, ...); padding
// (e >= E) is -inf, which sorts below every real score.
template <int EPL>
__device__ __forceinline__ void load_scores(const float* __restrict__ Lrow, int E, int lane, float (&f)[EPL]) {
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + 64 * q;
    f[q] = e < E ? Lrow[e] : -__builtin_inff();
  }
}

// wave_topk_radix: one wave selects the top k of E scores of one token; lane
// l holds the scores of experts l, l+64, ... in f.  Returns, in lane j < k,
// the rank-j key; every lane gets the rank-0 key in *top.  s_keys: 64
// wave-private LDS entries.
//
// Radix select with ballots: 32 rounds of compare + ballot + popcount find
// T, the k-th largest order-mapped score (count(v >= T) >= k, maximal).  The
// selection is every score above T plus the lowest-index experts scoring
// exactly T, as many as needed for k.  The k winners are compacted into LDS
// by ballot prefix counts, and each of lanes 0..k-1 ranks one winner against
// the others (keys are unique: score, then index) and stores it at its rank.
template <int EPL>
__device__ __forceinline__ uint64_t wave_topk_radix(const float (&f)[EPL], int E, int k, int lane, uint64_t* top,
                                                    uint64_t* s_keys) {
  uint32_t v[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) v[q] = lane + 64 * q < E ? orderable(f[q]) : 0u;
  uint32_t T = 0;
#pragma unroll 4
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < EPL; ++q) cnt += __popcll(__ballot(v[q] >= cand));
    if (cnt >= k) T = cand;
  }
  int gt = 0;
#pragma unroll
  for (int q = 0; q < EPL; ++q) gt += __popcll(__ballot(v[q] > T));
  const int need_eq = k - gt;
  const uint64_t below = (1ull << lane) - 1ull;  // lanes with a lower index
  int base_sel = 0, base_eq = 0;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const uint64_t beq = __ballot(v[q] == T);
    const int eq_rank = base_eq + __popcll(beq & below);
    const bool sel = v[q] > T || (v[q] == T && eq_rank < need_eq);
    const uint64_t bsel = __ballot(sel);
    if (sel)
      s_keys[base_sel + __popcll(bsel & below)] =
          ((uint64_t)v[q] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * q));
    base_sel += __popcll(bsel);
    base_eq += __popcll(beq);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t key = 0;
  int rank = 0;
  if (lane < k) {
    key = s_keys[lane];
    for (int i = 0; i < k; ++i) rank += s_keys[i] > key;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) s_keys[32 + rank] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t mine = lane < k ? s_keys[32 + lane] : 0ull;
  *top = s_keys[32];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return mine;
}

// The same selection (same results) with far fewer ballots, which dominate
// the cost: a radix select over the 64 lane maxima alone finds T, the
// k-th largest lane maximum T1 with its low 16 bits cleared (sign, exponent
// and 7 mantissa bits: 8 rounds of three independent ballots, two bits per
// round).  k distinct lanes hold a value >= T1 >= T, so every winner is
// among the candidates {values >= T}: the winners plus the few values
// within 2^-7 of T1, normally a dozen or so in all.  The candidates are
// compacted into LDS and each ranks itself among them by (score, lower
// index); ranks < k are the selection.  When more than 64 values lie at or
// above T (ties), the full radix select above takes over.
template <int EPL>
__device__ __forceinline__ uint64_t wave_topk(const float (&f)[EPL], int E, int k, int lane, uint64_t* top,
                                              uint64_t* s_keys) {
  uint32_t v[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) v[q] = lane + 64 * q < E ? orderable(f[q]) : 0u;
  uint32_t m = v[0];
#pragma unroll
  for (int q = 1; q < EPL; ++q) m = v[q] > m ? v[q] : m;
  uint32_t T = 0;
#pragma unroll
  for (int bit = 30; bit >= 16; bit -= 2) {
    const uint32_t c1 = T | (1u << bit), c2 = T | (2u << bit), c3 = T | (3u << bit);
    const int n1 = __popcll(__ballot(m >= c1)), n2 = __popcll(__ballot(m >= c2));
    const int n3 = __popcll(__ballot(m >= c3));
    T = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : T;
  }
  int C = 0;
#pragma unroll
  for (int q = 0; q < EPL; ++q) C += __popcll(__ballot(v[q] >= T));
  if (C > 64) return wave_topk_radix<EPL>(f, E, k, lane, top, s_keys);
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const bool c = v[q] >= T;
    const uint64_t b = __ballot(c);
    if (c)
      s_keys[base + __popcll(b & below)] =
          ((uint64_t)v[q] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * q));
    base += __popcll(b);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t key = 0;
  int rank = 0;
  if (lane < C) {
    key = s_keys[lane];
    for (int i = 0; i < C; ++i) rank += s_keys[i] > key;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < C && rank < k) s_keys[rank] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t mine = lane < k ? s_keys[lane] : 0ull;
  *top = s_keys[0];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return mine;
}

}  // namespace moe
