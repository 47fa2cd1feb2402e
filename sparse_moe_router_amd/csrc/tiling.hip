// Tiled layout of bf16 expert weights (gfx950).
//
// "Optimizing on-device inference for Apple Silicon" (Perplexity 2026),
// section "Dequantize weights during matrix multiplication": the grouped
// GEMM stages one small weight tile at a time in on-chip memory.  With rows
// stored one after another, one K-step of a 256-row weight tile is 128 bytes
// from each of 256 rows 4 KB apart, and HBM delivers such scattered short
// runs at about three quarters of its rate for long ones.  The tiled layout
// stores each K-step of a weight tile as one contiguous block, in the order
// and XOR swizzle the GEMM's LDS stage uses, so the stage is filled by plain
// 1 KB copies.  The matrix-vector kernels read the same layout (a row's 64
// elements of one K-step still sit in one 128-byte line).
//
// Per expert block (same 3*I*H elements as the row-major packing):
//   gate/up part, 2*I*H elements: panel p (p = 0 .. ceil(I/128)-1) at
//     element 256*p*H holds n = min(128, I - 128p) gate and n up rows as 2n
//     tile rows: gate/up (m = 0/1) row 128p + 32c + l is tile row
//     64c + 32m + l;
//   down part, H*I elements at 2*I*H: panel p at 2*I*H + 256*p*I holds the n
//     = min(256, H - 256p) rows 256p .. as tile rows 0 .. n-1;
//   a panel is K/64 steps one after another (K = H for gate/up, I for
//   down), a step being its tile rows in order, 64 elements each, with the
//   8-element chunk q of tile row R at chunk position q ^ ((R / 2) % 8).
//
// The 4-bit format has the same tiled order without the swizzle: its code
// words (8 codes each) follow the element order above, and its group words
// (one per 64 elements) too, so a K-step of a 4-bit weight tile is one
// contiguous block of codes and one of group words.  In the row-major
// 4-bit packing one step is 32 bytes of each of 256 rows (a quarter of a
// 128-byte line) and 4 bytes of group words of each, 256 lines apiece.
#include "moe_internal.h"

namespace moe {
namespace {

// One thread per 8-element chunk of the destination: find its source chunk.
__global__ __launch_bounds__(256) void k_tile_bf16(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                   int64_t total, int64_t block_chunks, int H, int I) {
  const int64_t gu = (int64_t)2 * I * H;
  for (int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x; d < total; d += (int64_t)gridDim.x * 256) {
    const int64_t b = d / block_chunks;
    const int64_t e = (d - b * block_chunks) * 8;  // element of the tiled block
    int64_t from;
    if (e < gu) {
      const int64_t pn = e / ((int64_t)256 * H);
      const int64_t rem = e - pn * 256 * H;
      const int n = I - 128 * pn < 128 ? (int)(I - 128 * pn) : 128;
      const int64_t per = (int64_t)128 * n;  // elements per step: 2n tile rows x 64
      const int64_t s = rem / per;
      const int w = (int)(rem - s * per);
      const int R = w >> 6, q = ((w >> 3) & 7) ^ ((R >> 1) & 7);
      const int m = (R >> 5) & 1;
      const int64_t row = 128 * pn + 32 * (R >> 6) + (R & 31);
      from = ((int64_t)m * I + row) * H + 64 * s + 8 * q;
    } else {
      const int64_t e2 = e - gu;
      const int64_t pn = e2 / ((int64_t)256 * I);
      const int64_t rem = e2 - pn * 256 * I;
      const int n = H - 256 * pn < 256 ? (int)(H - 256 * pn) : 256;
      const int64_t per = (int64_t)64 * n;
      const int64_t s = rem / per;
      const int w = (int)(rem - s * per);
      const int R = w >> 6, q = ((w >> 3) & 7) ^ ((R >> 1) & 7);
      from = gu + (256 * pn + R) * (int64_t)I + 64 * s + 8 * q;
    }
    dst[d] = src[b * block_chunks + (from >> 3)];
  }
}

// Element e of a tiled block (the order above, without the swizzle) -> its
// element in the row-major block.
__device__ __forceinline__ int64_t tiled_to_rowmajor(int64_t e, int H, int I) {
  const int64_t gu = (int64_t)2 * I * H;
  if (e < gu) {
    const int64_t pn = e / ((int64_t)256 * H);
    const int64_t rem = e - pn * 256 * H;
    const int n = I - 128 * pn < 128 ? (int)(I - 128 * pn) : 128;
    const int64_t per = (int64_t)128 * n;
    const int64_t s = rem / per;
    const int w = (int)(rem - s * per);
    const int R = w >> 6;
    const int m = (R >> 5) & 1;
    const int64_t row = 128 * pn + 32 * (R >> 6) + (R & 31);
    return ((int64_t)m * I + row) * H + 64 * s + (w & 63);
  }
  const int64_t e2 = e - gu;
  const int64_t pn = e2 / ((int64_t)256 * I);
  const int64_t rem = e2 - pn * 256 * I;
  const int n = H - 256 * pn < 256 ? (int)(H - 256 * pn) : 256;
  const int64_t per = (int64_t)64 * n;
  const int64_t s = rem / per;
  const int w = (int)(rem - s * per);
  return gu + (256 * pn + (w >> 6)) * (int64_t)I + 64 * s + (w & 63);
}

// 4-bit: one thread per destination code word (8 elements), then per group
// word (64 elements).
__global__ __launch_bounds__(256) void k_tile_q4(const uint32_t* __restrict__ csrc, const uint32_t* __restrict__ gsrc,
                                                 uint32_t* __restrict__ cdst, uint32_t* __restrict__ gdst,
                                                 int64_t nblocks, int64_t block_words, int H, int I) {
  const int64_t block_groups = block_words / 8;
  const int64_t total = nblocks * (block_words + block_groups);
  for (int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x; d < total; d += (int64_t)gridDim.x * 256) {
    if (d < nblocks * block_words) {
      const int64_t b = d / block_words, w = d - b * block_words;
      cdst[d] = csrc[b * block_words + (tiled_to_rowmajor(8 * w, H, I) >> 3)];
    } else {
      const int64_t d2 = d - nblocks * block_words;
      const int64_t b = d2 / block_groups, w = d2 - b * block_groups;
      gdst[d2] = gsrc[b * block_groups + (tiled_to_rowmajor(64 * w, H, I) >> 6)];
    }
  }
}

}  // namespace

hipError_t launch_tile_weights_q4(const uint32_t* codes, const uint32_t* groups, uint32_t* codes_dst,
                                  uint32_t* groups_dst, int64_t nblocks, int H, int I, hipStream_t s) {
  const int64_t block_words = (int64_t)3 * I * H / 8;
  const int64_t total = nblocks * (block_words + block_words / 8);
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_tile_q4, dim3(grid), dim3(256), 0, s, codes, groups, codes_dst, groups_dst, nblocks,
                     block_words, H, I);
  return hipGetLastError();
}

hipError_t launch_tile_weights(const uint16_t* src, uint16_t* dst, int64_t nblocks, int H, int I, hipStream_t s) {
  const int64_t block_chunks = (int64_t)3 * I * H / 8;
  const int64_t total = nblocks * block_chunks;
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_tile_bf16, dim3(grid), dim3(256), 0, s, (const u32x4_t*)src, (u32x4_t*)dst, total,
                     block_chunks, H, I);
  return hipGetLastError();
}

}  // namespace moe
