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

}  // namespace

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
