// Device filler for the synthetic inputs: the same SplitMix64 streams and value
// recipes as synth/__init__.py, bit for bit, so large workloads are generated
// where they are used and any slice can be regenerated on the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGolden); }

__device__ __forceinline__ float normal_f32(uint64_t key, uint64_t i) {
  int64_t acc = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const uint64_t d = draw(key, 3 * i + j);
#pragma unroll
    for (int f = 0; f < 4; ++f) acc += (int64_t)((d >> (16 * f)) & 0xFFFFull);
  }
  acc -= 6 * 65535;
  return (float)acc * 0x1p-16f;  // |acc| < 2^19: exact
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void k_fill(int kind, uint64_t key, uint64_t offset, int64_t n, int a, int emin, int emax,
                       void* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride) {
    const uint64_t i = offset + (uint64_t)t;
    switch (kind) {
      case 0: reinterpret_cast<float*>(out)[t] = normal_f32(key, i); break;
      case 1: reinterpret_cast<uint16_t*>(out)[t] = bf16_rne(normal_f32(key, i)); break;
      case 2: {
        const uint64_t hi = draw(key, i) >> 32;
        const int64_t v = (int64_t)((hi * (uint64_t)(2 * a + 1)) >> 32) - a;
        reinterpret_cast<uint16_t*>(out)[t] = bf16_rne((float)v);
        break;
      }
      case 3: reinterpret_cast<uint8_t*>(out)[t] = (uint8_t)(draw(key, i) & 0xFFu); break;
      case 4: {
        const uint64_t hi = draw(key, i) >> 32;
        const int64_t e = (int64_t)((hi * (uint64_t)(emax - emin + 1)) >> 32) + emin;
        reinterpret_cast<uint8_t*>(out)[t] = (uint8_t)((e + 7) << 3);
        break;
      }
      case 5: {
        const uint64_t d = draw(key, i);
        const uint64_t e = (((d >> 32) & 0xFFFFFFFFull) * 6ull >> 32) + 4;
        reinterpret_cast<uint8_t*>(out)[t] = (uint8_t)(((d >> 63) << 7) | (e << 3) | (d & 7ull));
        break;
      }
      case 6: {
        const float x = normal_f32(key, i);
        reinterpret_cast<float*>(out)[t] = (fabsf(x) + 0.5f) / 64.0f;
        break;
      }
      default: break;
    }
  }
}

}  // namespace

extern "C" int synth_fill(int kind, uint64_t key, uint64_t offset, int64_t n, int a, int emin, int emax,
                          void* out, void* stream) {
  if (kind < 0 || kind > 6 || n < 0 || (n > 0 && out == nullptr)) return -1;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     kind, key, offset, n, a, emin, emax, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
