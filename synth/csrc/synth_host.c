/* Host-side (CPU) twin of the seeded input generator in synth/inputs.py:
 * element i of stream `key` is the centred sum of the eight 16-bit fields of
 * SplitMix64 outputs 2i+1 and 2i+2, times one fp32 scale, rounded to
 * bfloat16 (round to nearest even).  Bit-exact with the NumPy definition
 * (tests/test_synth.py checks it); it exists only because regenerating the
 * full-size expert weights in NumPy takes about 0.3 s per expert.
 *
 * Synthetic-input plumbing only: none of the MoE layer's arithmetic is here.
 * Generator: SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) with Stafford's
 * Mix13 finaliser. */
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull
#define M1 0xBF58476D1CE4E5B9ull
#define M2 0x94D049BB133111EBull
#define IH_MEAN 262140

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * M1;
  z = (z ^ (z >> 27)) * M2;
  return z ^ (z >> 31);
}

/* dst[j] = bf16 bits of element start + j of stream key, for j < n */
void synth_host_normal_bf16(uint16_t* dst, uint64_t key, uint64_t start, uint64_t n, float scale) {
  for (uint64_t j = 0; j < n; ++j) {
    const uint64_t i = start + j;
    const uint64_t a = mix64(key + (2 * i + 1) * GAMMA);
    const uint64_t b = mix64(key + (2 * i + 2) * GAMMA);
    int64_t s = 0;
    for (int q = 0; q < 4; ++q) s += (int64_t)((a >> (16 * q)) & 0xFFFF) + (int64_t)((b >> (16 * q)) & 0xFFFF);
    const float v = (float)(int32_t)(s - IH_MEAN) * scale; /* one IEEE multiply */
    uint32_t bits;
    memcpy(&bits, &v, 4);
    dst[j] = (uint16_t)((bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16);
  }
}
