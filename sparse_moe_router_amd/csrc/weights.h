// Expert weight formats read by the decode (matrix-vector) kernels.
//
// An expert block holds gate [I][H], up [I][H], down [H][I] (rows along the
// reduction dimension).  block(e) is the block at element offset e; gu(m, i)
// is row i of gate (m = 0) or up (m = 1), dn(c) row c of down; a row's
// load(k) returns its 8-element chunk k .. k+7 (k % 8 == 0).
//
//  - WBf16 / WBf16S: one bf16 per element, rows stored one after another.
//  - WBf16T: the same bf16 weights in the tiled layout the grouped GEMM
//    streams (each K-step of a weight tile one contiguous block): in the
//    gate/up part, panel p holds gate and up rows [128p, 128p + n) (n =
//    min(128, I - 128p)) as 2n tile rows, gate/up row 128p + 32c + l at tile
//    row 64c + 32m + l; in the down part, panel p holds rows [256p, 256p + n)
//    (n = min(256, H - 256p)) as tile rows 0 .. n-1.  A panel stores its
//    K-steps of 64 one after another, each as its tile rows of 64 elements,
//    whose eight 8-element chunks sit XOR-swizzled (chunk q of tile row R at
//    position q ^ ((R / 2) % 8)).  A row's chunk is found at
//    panel + step * (tile rows * 64) + R * 64 + 8 * (q ^ ((R / 2) % 8)); the eight
//    chunks of a step stay inside one 128-byte line, so loads that cover a
//    row's 64 elements stay coalesced.
//  - WQ4: the 4-bit group-affine format of "Optimizing on-device inference
//    for Apple Silicon", section "Dequantize weights during matrix
//    multiplication": each weight is an unsigned 4-bit code q, and each group
//    of 64 consecutive elements of a row shares one bf16 scale s and one bf16
//    bias b, w = s*q + b.  Codes: eight per 32-bit word, element 8i+j in bits
//    4j..4j+3 (two per byte, low nibble first); groups: one 32-bit word each,
//    s in the low half, b in the high half.
//  - WQ4T: the WQ4 codes and group words in the grouped GEMM's tiled order
//    (below).
//
// The expert formats (WBf16S, WBf16T, WQ4 codes) load with the non-temporal
// hint: a matrix-vector pass reads each expert weight once, and streamed with
// the default policy those bytes push the activations, scores and h out of
// the caches (the 40-layer decode graph: 18.6-19.0 -> 17.9-18.0 us per
// layer).  WBf16 keeps the default policy for the router rows.
#pragma once

#include "moe_internal.h"

namespace moe {

template <bool NT>
struct WBf16Rows {
  const uint16_t* p;
  typedef u32x4_t chunk_t;  // 8 elements
  struct Row {
    const uint16_t* p;
    __device__ __forceinline__ chunk_t load(int64_t k) const {
      return NT ? __builtin_nontemporal_load((const u32x4_t*)(p + k)) : *(const u32x4_t*)(p + k);
    }
  };
  __device__ __forceinline__ WBf16Rows block(int64_t e) const { return {p + e}; }
  __device__ __forceinline__ Row gu(int m, int i, int H, int I) const { return {p + ((int64_t)m * I + i) * H}; }
  __device__ __forceinline__ Row dn(int c, int H, int I) const { return {p + (int64_t)2 * I * H + (int64_t)c * I}; }
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

// Row-major bf16 rows with the default cache policy (router rows: the
// small-batch router re-reads them, and across decode steps the routers of
// all layers, 1 MB each, stay in the last-level cache; measured slower with
// the hint) and with the non-temporal hint (expert rows: read once per
// layer).
typedef WBf16Rows<false> WBf16;
typedef WBf16Rows<true> WBf16S;

struct WBf16T {
  const uint16_t* p;
  typedef u32x4_t chunk_t;
  struct Row {
    const uint16_t* p;  // tile row R of the row's first K-step
    int step;           // elements per K-step of its panel
    int swz;            // (R / 2) % 8
    __device__ __forceinline__ chunk_t load(int64_t k) const {
      return __builtin_nontemporal_load((const u32x4_t*)(p + (k >> 6) * step + 8 * (((int)(k >> 3) & 7) ^ swz)));
    }
  };
  __device__ __forceinline__ WBf16T block(int64_t e) const { return {p + e}; }
  __device__ __forceinline__ Row gu(int m, int i, int H, int I) const {
    const int pn = i >> 7, j = i & 127, n = I - 128 * pn < 128 ? I - 128 * pn : 128;
    const int R = 64 * (j >> 5) + 32 * m + (j & 31);
    return {p + (int64_t)256 * pn * H + 64 * R, 128 * n, (R >> 1) & 7};
  }
  __device__ __forceinline__ Row dn(int c, int H, int I) const {
    const int pn = c >> 8, R = c & 255, n = H - 256 * pn < 256 ? H - 256 * pn : 256;
    return {p + (int64_t)2 * I * H + (int64_t)256 * pn * I + 64 * R, 64 * n, (R >> 1) & 7};
  }
  __device__ __forceinline__ static float dot(const chunk_t& w, const u32x4_t& x) { return WBf16::dot(w, x); }
  __device__ __forceinline__ static float dot(const chunk_t& w, const f32x4_t& x0, const f32x4_t& x1) {
    return WBf16::dot(w, x0, x1);
  }
};

struct WQ4 {
  const uint32_t* c;  // codes, 8 per word
  const uint32_t* g;  // (scale, bias) per 64 elements
  struct chunk_t {
    uint32_t c, g;
  };
  struct Row {
    const uint32_t* c;
    const uint32_t* g;
    __device__ __forceinline__ chunk_t load(int64_t k) const {
      return {__builtin_nontemporal_load(c + (k >> 3)), g[k >> 6]};
    }
  };
  __device__ __forceinline__ WQ4 block(int64_t e) const { return {c + (e >> 3), g + (e >> 6)}; }
  __device__ __forceinline__ Row at_elem(int64_t e) const { return {c + (e >> 3), g + (e >> 6)}; }
  __device__ __forceinline__ Row gu(int m, int i, int H, int I) const { return at_elem(((int64_t)m * I + i) * H); }
  __device__ __forceinline__ Row dn(int c, int H, int I) const {
    return at_elem((int64_t)2 * I * H + (int64_t)c * I);
  }
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

// The 4-bit format in the tiled order of the grouped GEMM (moe_tile_weights_q4):
// the same panels and 64-element K-steps as WBf16T (no swizzle), a tile row's
// step being its 8 code words, and the group words in the same order, one
// per tile row and step.  A row's code word for elements k .. k+7 sits at
// panel + step * (tile rows * 8) + R * 8 + (k / 8) % 8, its group word at
// panel / 64 + step * (tile rows) + R.
struct WQ4T {
  const uint32_t* c;
  const uint32_t* g;
  typedef WQ4::chunk_t chunk_t;
  struct Row {
    const uint32_t* c;  // code words of tile row R at step 0
    const uint32_t* g;  // group word of tile row R at step 0
    int cst, gst;       // words per step: tile rows * 8, tile rows
    __device__ __forceinline__ chunk_t load(int64_t k) const {
      const int64_t s = k >> 6;
      return {__builtin_nontemporal_load(c + s * cst + ((k >> 3) & 7)), g[s * gst]};
    }
  };
  __device__ __forceinline__ WQ4T block(int64_t e) const { return {c + (e >> 3), g + (e >> 6)}; }
  __device__ __forceinline__ Row at(int64_t base, int R, int trows) const {
    return {c + (base >> 3) + 8 * R, g + (base >> 6) + R, 8 * trows, trows};
  }
  __device__ __forceinline__ Row gu(int m, int i, int H, int I) const {
    const int pn = i >> 7, j = i & 127, n = I - 128 * pn < 128 ? I - 128 * pn : 128;
    return at((int64_t)256 * pn * H, 64 * (j >> 5) + 32 * m + (j & 31), 2 * n);
  }
  __device__ __forceinline__ Row dn(int c, int H, int I) const {
    const int pn = c >> 8, n = H - 256 * pn < 256 ? H - 256 * pn : 256;
    return at((int64_t)2 * I * H + (int64_t)256 * pn * I, c & 255, n);
  }
  __device__ __forceinline__ static float dot(const chunk_t& w, const u32x4_t& x) { return WQ4::dot(w, x); }
  __device__ __forceinline__ static float dot(const chunk_t& w, const f32x4_t& x0, const f32x4_t& x1) {
    return WQ4::dot(w, x0, x1);
  }
};

}  // namespace moe
