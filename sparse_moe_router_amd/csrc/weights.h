// Expert weight formats read by the decode (matrix-vector) kernels.
//
// Both address an expert block by element index: expert e's block holds
// gate [I][H], up [I][H], down [H][I] (rows along the reduction dimension),
// and element offsets of rows and 8-element chunks are multiples of 8 (of
// 64 for row starts).
//
//  - WBf16: one bf16 per element.
//  - WQ4: the 4-bit group-affine format of "Optimizing on-device inference
//    for Apple Silicon", section "Dequantize weights during matrix
//    multiplication": each weight is an unsigned 4-bit code q, and each group
//    of 64 consecutive elements of a row shares one bf16 scale s and one bf16
//    bias b, w = s*q + b.  Codes: eight per 32-bit word, element 8i+j in bits
//    4j..4j+3 (two per byte, low nibble first); groups: one 32-bit word each,
//    s in the low half, b in the high half.
#pragma once

#include "moe_internal.h"

namespace moe {

struct WBf16 {
  const uint16_t* p;
  typedef u32x4_t chunk_t;  // 8 elements
  __device__ __forceinline__ WBf16 at(int64_t e) const { return {p + e}; }
  __device__ __forceinline__ chunk_t load(int64_t e) const { return *(const u32x4_t*)(p + e); }
  // sum_i w_i x_i over the 8 elements, x as 8 bf16
  __device__ __forceinline__ static float dot(const chunk_t& w, const u32x4_t& x) {
    float a = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) a += bf16_lo(x[q]) * bf16_lo(w[q]) + bf16_hi(x[q]) * bf16_hi(w[q]);
    return a;
  }
  // the same with x as 8 fp32
  __device__ __forceinline__ static float dot(const chunk_t& w, const f32x4_t& x0, const f32x4_t& x1) {
    return bf16_lo(w[0]) * x0[0] + bf16_hi(w[0]) * x0[1] + bf16_lo(w[1]) * x0[2] + bf16_hi(w[1]) * x0[3] +
           bf16_lo(w[2]) * x1[0] + bf16_hi(w[2]) * x1[1] + bf16_lo(w[3]) * x1[2] + bf16_hi(w[3]) * x1[3];
  }
};

struct WQ4 {
  const uint32_t* c;  // codes, 8 per word
  const uint32_t* g;  // (scale, bias) per 64 elements
  struct chunk_t {
    uint32_t c, g;
  };
  __device__ __forceinline__ WQ4 at(int64_t e) const { return {c + (e >> 3), g + (e >> 6)}; }
  __device__ __forceinline__ chunk_t load(int64_t e) const { return {c[e >> 3], g[e >> 6]}; }
  __device__ __forceinline__ static float code(uint32_t c, int j) {
    return (float)__builtin_amdgcn_ubfe(c, 4 * j, 4);
  }
  // sum_i (s q_i + b) x_i = s * sum_i q_i x_i + b * sum_i x_i
  __device__ __forceinline__ static float dot(const chunk_t& w, const u32x4_t& x) {
    float qx = 0.0f, sx = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float xl = bf16_lo(x[q]), xh = bf16_hi(x[q]);
      qx += code(w.c, 2 * q) * xl + code(w.c, 2 * q + 1) * xh;
      sx += xl + xh;
    }
    return bf16_lo(w.g) * qx + bf16_hi(w.g) * sx;
  }
  __device__ __forceinline__ static float dot(const chunk_t& w, const f32x4_t& x0, const f32x4_t& x1) {
    const float qx = code(w.c, 0) * x0[0] + code(w.c, 1) * x0[1] + code(w.c, 2) * x0[2] + code(w.c, 3) * x0[3] +
                     code(w.c, 4) * x1[0] + code(w.c, 5) * x1[1] + code(w.c, 6) * x1[2] + code(w.c, 7) * x1[3];
    const float sx = (x0[0] + x0[1]) + (x0[2] + x0[3]) + ((x1[0] + x1[1]) + (x1[2] + x1[3]));
    return bf16_lo(w.g) * qx + bf16_hi(w.g) * sx;
  }
};

}  // namespace moe
