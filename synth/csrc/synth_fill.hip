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

__global__ void fill_words_kernel(uint64_t* __restrict__ dst, uint64_t key, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = mix64(key + (i + 1) * kGamma);
}

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  return (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
}

__global__ void fill_sb_kernel(uint32_t* __restrict__ dst, uint64_t key, uint64_t n, float s0) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t r = mix64(key + (i + 1) * kGamma);
    const float u = (float)(uint32_t)((r >> 9) & 0x7FFFFFu) * 0x1p-23f;
    const float v = (float)(uint32_t)(r >> 43) * 0x1p-21f;
    const float sm = 0.5f + u;  // exact
    const uint32_t sb = bf16_rne(s0 * sm);
    const float sv = __uint_as_float(sb << 16);
    const float m = 7.0f + v;  // exact
    const uint32_t bb = bf16_rne(-(sv * m));
    dst[i] = sb | (bb << 16);
  }
}

unsigned blocks_for(uint64_t n) {
  uint64_t b = (n + 255) / 256;
  return (unsigned)(b > 65536 ? 65536 : b);
}

}  // namespace

extern "C" {

// 4-bit codes: dst receives nbytes bytes of stream `key` (output n -> bytes
// 8(n-1) .. 8n-1, little-endian); nbytes must be a multiple of 8.
int synth_fill_q4_codes(void* dst, uint64_t key, uint64_t nbytes, void* stream) {
  if (nbytes == 0) return 0;
  if (dst == nullptr || nbytes % 8) return (int)hipErrorInvalidValue;
  const uint64_t n = nbytes / 8;
  hipLaunchKernelGGL(fill_words_kernel, dim3(blocks_for(n)), dim3(256), 0, (hipStream_t)stream, (uint64_t*)dst,
                     key, n);
  return (int)hipGetLastError();
}

// 4-bit scale/bias words of ngroups groups (s0 = sigma / 4.61 in fp32).
int synth_fill_q4_scale_bias(void* dst, uint64_t key, uint64_t ngroups, float s0, void* stream) {
  if (ngroups == 0) return 0;
  if (dst == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_sb_kernel, dim3(blocks_for(ngroups)), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)dst, key, ngroups, s0);
  return (int)hipGetLastError();
}

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
