// Standalone fp8-row and fp4-group codecs ([P1] quantisation paragraph: fp8
// attention cache, fp4 indexer cache; [P3] "Three mechanisms", third: E2M1
// values with one E4M3 scale per 16 channels). The compress and attend
// kernels run the same device routines fused into their loads and stores.
#include "kernels.h"

namespace cskv {

// One wave per row; each lane owns D/64 consecutive channels.
template <bool BF16_IN>
__global__ __launch_bounds__(256) void k_encode_fp8_rows(const void* __restrict__ x, int64_t rows,
                                                         int D, uint8_t* __restrict__ codes,
                                                         float* __restrict__ scale) {
  const int lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (row >= rows) return;
  const int cpl = D / kWave;
  float v[16];
  float amax = 0.0f;
  for (int i = 0; i < cpl; ++i) {
    const int64_t idx = row * D + lane * cpl + i;
    v[i] = BF16_IN ? bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[idx])
                   : reinterpret_cast<const float*>(x)[idx];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int i = 0; i < cpl; ++i) codes[row * D + lane * cpl + i] = (uint8_t)f32_to_e4m3(v[i] / sc);
  if (lane == 0) scale[row] = sc;
}

// One thread per code; the decode goes through the same converter the
// attention kernel uses on its loads (then exact to fp32, times the scale).
__global__ void k_decode_fp8_rows(const uint8_t* __restrict__ codes, const float* __restrict__ scale,
                                  int64_t rows, int D, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * D) return;
  const uint32_t bits = fp8x2_to_bf16x2<false>((uint32_t)codes[i]);
  out[i] = bf16_lo(bits) * scale[i / D];
}

// One thread per group of 16 channels.
template <bool BF16_IN>
__global__ void k_encode_fp4_g16(const void* __restrict__ x, int64_t groups,
                                 uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= groups) return;
  float v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = BF16_IN ? bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[gi * 16 + i])
                   : reinterpret_cast<const float*>(x)[gi * 16 + i];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  uint32_t sc = f32_to_e4m3(amax / 6.0f);
  if (e4m3_to_f32(sc) == 0.0f && amax > 0.0f) sc = 0x01u;
  const float sv = e4m3_to_f32(sc);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = sv == 0.0f ? 0u : f32_to_e2m1(v[i] / sv);
    if (i < 8) lo |= c << (4 * i);
    else hi |= c << (4 * (i - 8));
  }
  *reinterpret_cast<uint2*>(packed + gi * 8) = make_uint2(lo, hi);
  scales[gi] = (uint8_t)sc;
}

// One thread per packed byte (two channels); the decode goes through the
// same converter the indexer kernel uses.
__global__ void k_decode_fp4_g16(const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
                                 int64_t nbytes, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nbytes) return;
  const uint32_t word = *reinterpret_cast<const uint32_t*>(packed + (i & ~(int64_t)3));
  bf16x2_t p;
  switch (i & 3) {
    case 0: p = fp4x2_to_bf16x2<0>(word); break;
    case 1: p = fp4x2_to_bf16x2<1>(word); break;
    case 2: p = fp4x2_to_bf16x2<2>(word); break;
    default: p = fp4x2_to_bf16x2<3>(word); break;
  }
  const uint32_t bits = __builtin_bit_cast(uint32_t, p);
  const float s = e4m3_to_f32(scales[i / 8]);
  out[2 * i] = bf16_lo(bits) * s;
  out[2 * i + 1] = bf16_hi(bits) * s;
}

hipError_t launch_encode_fp8_rows(bool in_bf16, const void* x, int64_t rows, int D, uint8_t* codes,
                                  float* scale, hipStream_t stream) {
  dim3 grid((unsigned)((rows + 3) / 4));
  if (in_bf16) hipLaunchKernelGGL(k_encode_fp8_rows<true>, grid, dim3(256), 0, stream, x, rows, D, codes, scale);
  else hipLaunchKernelGGL(k_encode_fp8_rows<false>, grid, dim3(256), 0, stream, x, rows, D, codes, scale);
  return hipGetLastError();
}

hipError_t launch_decode_fp8_rows(const uint8_t* codes, const float* scale, int64_t rows, int D,
                                  float* out, hipStream_t stream) {
  const int64_t n = rows * D;
  hipLaunchKernelGGL(k_decode_fp8_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     codes, scale, rows, D, out);
  return hipGetLastError();
}

hipError_t launch_encode_fp4_g16(bool in_bf16, const void* x, int64_t rows, int Di, uint8_t* packed,
                                 uint8_t* scales, hipStream_t stream) {
  const int64_t groups = rows * (Di / 16);
  dim3 grid((unsigned)((groups + 255) / 256));
  if (in_bf16) hipLaunchKernelGGL(k_encode_fp4_g16<true>, grid, dim3(256), 0, stream, x, groups, packed, scales);
  else hipLaunchKernelGGL(k_encode_fp4_g16<false>, grid, dim3(256), 0, stream, x, groups, packed, scales);
  return hipGetLastError();
}

hipError_t launch_decode_fp4_g16(const uint8_t* packed, const uint8_t* scales, int64_t rows, int Di,
                                 float* out, hipStream_t stream) {
  const int64_t nbytes = rows * (Di / 2);
  hipLaunchKernelGGL(k_decode_fp4_g16, dim3((unsigned)((nbytes + 255) / 256)), dim3(256), 0, stream,
                     packed, scales, nbytes, out);
  return hipGetLastError();
}

}  // namespace cskv
