// Device-side twin of synth/inputs.py: fills a buffer with elements of a
// counter-based SplitMix64 stream mapped to approximately normal variates
// (centred sum of eight 16-bit uniforms times one fp32 scale) and rounded
// to bfloat16 with round-to-nearest-even.  Bit-exact with the NumPy side.
//
// Synthetic-input plumbing only: none of the MoE layer's arithmetic is here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kM1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kM2 = 0x94D049BB133111EBull;
constexpr int64_t kMean = 262140;  // 8 * 65535 / 2

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kM1;
  z = (z ^ (z >> 27)) * kM2;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint16_t variate_bf16(uint64_t key, uint64_t i, float scale) {
  const uint64_t a = mix64(key + (2 * i + 1) * kGamma);
  const uint64_t b = mix64(key + (2 * i + 2) * kGamma);
  int64_t s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) s += (int64_t)((a >> (16 * q)) & 0xFFFF) + (int64_t)((b >> (16 * q)) & 0xFFFF);
  const float v = (float)(int32_t)(s - kMean) * scale;  // one IEEE multiply
  const uint32_t bits = __float_as_uint(v);
  return (uint16_t)((bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16);
}

__global__ void fill_kernel(uint16_t* __restrict__ dst, uint64_t key, uint64_t start, uint64_t n,
                            float scale) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = variate_bf16(key, start + i, scale);
}

}  // namespace

extern "C" {

// dst: device buffer of n uint16 (bf16 bits).  Element j receives stream
// element start+j.  Returns 0 or the hipError_t of the launch.
int synth_fill_normal_bf16(void* dst, uint64_t key, uint64_t start, uint64_t n, float scale,
                           void* stream) {
  if (n == 0) return 0;
  if (dst == nullptr) return (int)hipErrorInvalidValue;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint16_t*)dst, key, start, n, scale);
  return (int)hipGetLastError();
}

}  // extern "C"
