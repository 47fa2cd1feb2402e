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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// One wave selects the top k of E scores of one token; lanes own experts
// lane, lane+64, ...  Returns, in lane j < k, the rank-j key; all lanes get
// the rank-0 key in *top.
template <int EPL>
__device__ __forceinline__ uint64_t wave_topk(const float* __restrict__ Lrow, int E, int k, int lane,
                                              uint64_t* top) {
  uint64_t key[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + 64 * q;
    key[q] = e < E ? sel_key(Lrow[e], e) : 0ull;
  }
  // sort the lane's keys descending (insertion network, constant indices only)
#pragma unroll
  for (int i = 1; i < EPL; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const uint64_t a = key[j - 1], b = key[j];
      key[j - 1] = a > b ? a : b;
      key[j] = a > b ? b : a;
    }
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_u64(key[0]);
    if (j == 0) *top = best;
    if (lane == j) mine = best;
    if (key[0] == best) {  // keys are unique: exactly one owner lane pops its head
#pragma unroll
      for (int q = 0; q + 1 < EPL; ++q) key[q] = key[q + 1];
      key[EPL - 1] = 0ull;
    }
  }
  return mine;
}

}  // namespace moe
