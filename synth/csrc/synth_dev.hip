// Device fill of the seeded synthetic inputs: the same counter-based generator as synth/gen.py
// (SplitMix64 output function over the counter key + G*(i+1); Irwin-Hall(4) sum of 16-bit fields
// times an fp32 scale; optional round-to-nearest-even storage in bf16). No step of the MoE method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t G = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float ih4(uint64_t w, float scale) {
  int s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += 2 * (int)((w >> (16 * j)) & 0xFFFFu) - 65535;
  return (float)s * scale;
}

__global__ void fill_normal(void* dst, long long n, uint64_t key, long long start, float scale, int out_bf16) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = ih4(mix64(key + G * (uint64_t)(start + i + 1)), scale);
  if (out_bf16) {
    const uint32_t b = __float_as_uint(v);
    static_cast<uint16_t*>(dst)[i] = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
  } else {
    static_cast<float*>(dst)[i] = v;
  }
}

}  // namespace

extern "C" int synth_fill_normal(void* dst, long long n, unsigned long long key, long long start, float scale,
                                 int out_bf16, hipStream_t stream) {
  if (n <= 0) return 0;
  const long long blocks = (n + 255) / 256;
  fill_normal<<<(unsigned)blocks, 256, 0, stream>>>(dst, n, key, start, scale, out_bf16);
  return (int)hipGetLastError();
}
