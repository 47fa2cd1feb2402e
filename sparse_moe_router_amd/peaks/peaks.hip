// Measurement kernels: the sustainable HBM read rate and the sustainable
// dense bf16 MFMA rate of the device ("Optimizing on-device inference for
// Apple Silicon", section "Limits of further optimization": kernels are
// rated against the fastest sustainable rate of the resource they need).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_peaks.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kStreamBlocks = 2048;  // 8 per compute unit
constexpr int kStreamThreads = 512;
constexpr int kUnroll = 4;           // 16-byte loads in flight per thread per iteration

// Workgroup b reads the 16-byte chunks b*T + t, (b + B)*T + t, ... (T threads,
// B workgroups): each step of the grid covers one contiguous B*T*16-byte span.
__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const u32x4_t* __restrict__ buf, uint64_t n16,
                                                               uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_x[kStreamThreads / 64];
  const uint64_t span = (uint64_t)gridDim.x * blockDim.x;
  uint32_t x = 0;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kUnroll - 1) * span < n16; i += kUnroll * span) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * span);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += span) {
    const u32x4_t v = buf[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kStreamThreads / 64; ++w) r ^= s_x[w];
    sink[blockIdx.x] = r;
  }
}

// 8 waves per workgroup; each wave chains `iters` rounds of 8 independent
// MFMAs (independent accumulators, so the matrix pipe never waits on a result).
__global__ __launch_bounds__(512) void k_mfma_loop(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  f32x16_t acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = (f32x16_t){};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[m][r];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) sink[blockIdx.x * 8 + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

int moe_peak_stream_blocks(void) { return kStreamBlocks; }

int moe_peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15)) return 1;
  const uintptr_t b0 = (uintptr_t)buf, s0 = (uintptr_t)sink;
  if (s0 < b0 + bytes && b0 < s0 + (uintptr_t)kStreamBlocks * 4) return 1;
  hipLaunchKernelGGL(k_stream_read, dim3(kStreamBlocks), dim3(kStreamThreads), 0, stream, (const u32x4_t*)buf,
                     (uint64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int moe_peak_mfma_loop(int cus, int iters, float* sink, hipStream_t stream) {
  if (!sink || cus < 1 || cus > 4096 || iters < 1) return 1;
  hipLaunchKernelGGL(k_mfma_loop, dim3(cus), dim3(512), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
