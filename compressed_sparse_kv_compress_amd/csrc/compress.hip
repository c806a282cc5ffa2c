// Compression of shared states into c4a / c128a cache entries.
//
// [P1] "c4a (the milder scheme)": each compressed token is a weighted sum of 8
// uncompressed tokens with stride 4. [P1] "c128a (the aggressive scheme)": a
// weighted sum of 128 tokens with stride 128. [P2] Step 4: the weights are a
// learned mix, not a plain average; here they are the softmax of the window's
// per-state gate logits.
//
// Both kernels stream S once from HBM (a c4a state feeds two entries but is
// loaded once per wave run) and fuse the output rounding / fp8 row encoding.
#include "kernels.h"

namespace cskv {

// Lane-owned slice of a D-wide row: CPL = D/64 channels per lane.
template <int D>
struct RowSlice {
  static constexpr int CPL = D / kWave;  // 8 (D=512) or 2 (D=128)
  float v[CPL];
};

template <int D>
__device__ __forceinline__ void load_row(const uint16_t* row, int lane, RowSlice<D>& r) {
  constexpr int CPL = RowSlice<D>::CPL;
  if constexpr (CPL == 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(row + lane * 8);
    r.v[0] = bf16_lo(q.x); r.v[1] = bf16_hi(q.x); r.v[2] = bf16_lo(q.y); r.v[3] = bf16_hi(q.y);
    r.v[4] = bf16_lo(q.z); r.v[5] = bf16_hi(q.z); r.v[6] = bf16_lo(q.w); r.v[7] = bf16_hi(q.w);
  } else {
    static_assert(CPL == 2, "D must be 128 or 512");
    const uint32_t q = *reinterpret_cast<const uint32_t*>(row + lane * 2);
    r.v[0] = bf16_lo(q); r.v[1] = bf16_hi(q);
  }
}

// Writes one finished entry row held as CPL fp32 values per lane: bf16 (RNE)
// or fp8 codes + one fp32 row scale (amax / 448 over the whole row).
template <int D, bool FP8>
__device__ __forceinline__ void store_entry(const float* acc, int lane, void* cache_row,
                                            float* scale_slot) {
  constexpr int CPL = D / kWave;
  if constexpr (!FP8) {
    uint16_t* out = reinterpret_cast<uint16_t*>(cache_row) + lane * CPL;
    if constexpr (CPL == 8) {
      uint4 q;
      q.x = pack_bf16x2(acc[0], acc[1]); q.y = pack_bf16x2(acc[2], acc[3]);
      q.z = pack_bf16x2(acc[4], acc[5]); q.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(out) = q;
    } else {
      *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(acc[0], acc[1]);
    }
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) amax = fmaxf(amax, fabsf(acc[i]));
    amax = wave_max(amax);
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint8_t* out = reinterpret_cast<uint8_t*>(cache_row) + lane * CPL;
    uint32_t c[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) c[i] = f32_to_e4m3(acc[i] / scale);
    if constexpr (CPL == 8) {
      uint2 q;
      q.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      q.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      *reinterpret_cast<uint2*>(out) = q;
    } else {
      *reinterpret_cast<uint16_t*>(out) = (uint16_t)(c[0] | (c[1] << 8));
    }
    if (lane == 0) *scale_slot = scale;
  }
}

// ---------------------------------------------------------------- c4a
// One wave owns a run of kC4aRun consecutive entries of one sequence. Entry c
// reads stride blocks c and c+1 (4 states each); the wave keeps the previous
// block in registers so every state of the run is loaded once.
constexpr int kC4aRun = 16;
constexpr int kCompressThreads = 256;

template <int D, bool FP8>
__global__ __launch_bounds__(kCompressThreads) void k_compress_c4a(
    const uint16_t* __restrict__ S, const float* __restrict__ gate, int64_t T, int64_t n_entries,
    int64_t first_entry, void* __restrict__ cache, float* __restrict__ cache_scale,
    int64_t cache_rows) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.y;
  const int64_t c0 = ((int64_t)blockIdx.x * (kCompressThreads / kWave) + wave) * kC4aRun;
  if (c0 >= n_entries) return;
  const int64_t c1 = c0 + kC4aRun < n_entries ? c0 + kC4aRun : n_entries;

  const uint16_t* Sb = S + b * T * D;
  const float* gb = gate + b * T;
  constexpr int ESZ = FP8 ? 1 : 2;
  uint8_t* cb = reinterpret_cast<uint8_t*>(cache) + (b * cache_rows + first_entry) * (int64_t)D * ESZ;
  float* sb = FP8 ? cache_scale + b * cache_rows + first_entry : nullptr;

  RowSlice<D> prev[4], cur[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) load_row<D>(Sb + (4 * c0 + j) * D, lane, prev[j]);

  for (int64_t c = c0; c < c1; ++c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) load_row<D>(Sb + (4 * c + 4 + j) * D, lane, cur[j]);
    // softmax of the window's 8 gate logits (fp32)
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = gb[4 * c + j];
    float m = g[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) m = fmaxf(m, g[j]);
    float e[8], z = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) { e[j] = expf(g[j] - m); z += e[j]; }
    float acc[RowSlice<D>::CPL];
#pragma unroll
    for (int i = 0; i < RowSlice<D>::CPL; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w = e[j] / z;
#pragma unroll
      for (int i = 0; i < RowSlice<D>::CPL; ++i) acc[i] = fmaf(w, prev[j].v[i], acc[i]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w = e[4 + j] / z;
#pragma unroll
      for (int i = 0; i < RowSlice<D>::CPL; ++i) acc[i] = fmaf(w, cur[j].v[i], acc[i]);
    }
    store_entry<D, FP8>(acc, lane, cb + c * (int64_t)D * ESZ, FP8 ? sb + c : nullptr);
#pragma unroll
    for (int j = 0; j < 4; ++j) prev[j] = cur[j];
  }
}

// ---------------------------------------------------------------- c128a
// One workgroup per entry: wave w folds states 32w .. 32w+31 of the window,
// then the four partial rows are added in wave order through LDS.
template <int D, bool FP8>
__global__ __launch_bounds__(kCompressThreads) void k_compress_c128a(
    const uint16_t* __restrict__ S, const float* __restrict__ gate, int64_t T, int64_t n_entries,
    int64_t first_entry, void* __restrict__ cache, float* __restrict__ cache_scale,
    int64_t cache_rows) {
  constexpr int CPL = D / kWave;
  constexpr int NW = kCompressThreads / kWave;
  __shared__ float part[NW][D];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.y;
  const int64_t c = blockIdx.x;
  const uint16_t* Sw = S + (b * T + 128 * c) * D;
  const float* gw = gate + b * T + 128 * c;

  // softmax over the 128 logits; every wave computes the same max and sum
  const float g0 = gw[lane], g1 = gw[lane + 64];
  const float m = wave_max(fmaxf(g0, g1));
  const float z = wave_sum(expf(g0 - m) + expf(g1 - m));

  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.0f;
  RowSlice<D> r[8];
  for (int j0 = 0; j0 < 32; j0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) load_row<D>(Sw + (int64_t)(32 * wave + j0 + u) * D, lane, r[u]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = expf(gw[32 * wave + j0 + u] - m) / z;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] = fmaf(w, r[u].v[i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) part[wave][lane * CPL + i] = acc[i];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    float s = part[0][lane * CPL + i];
#pragma unroll
    for (int w = 1; w < NW; ++w) s += part[w][lane * CPL + i];
    acc[i] = s;
  }
  constexpr int ESZ = FP8 ? 1 : 2;
  const int64_t row = b * cache_rows + first_entry + c;
  store_entry<D, FP8>(acc, lane, reinterpret_cast<uint8_t*>(cache) + row * (int64_t)D * ESZ,
                      FP8 ? cache_scale + row : nullptr);
}

// ---------------------------------------------------------------- launch

template <int D, bool FP8>
static hipError_t launch_compress_t(int kind, const uint16_t* S, const float* gate, int64_t B,
                                    int64_t T, int64_t n, int64_t first_entry, void* cache,
                                    float* cache_scale, int64_t cache_rows, hipStream_t stream) {
  if (kind == 0) {
    const int64_t per_block = (int64_t)kC4aRun * (kCompressThreads / kWave);
    dim3 grid((unsigned)((n + per_block - 1) / per_block), (unsigned)B);
    hipLaunchKernelGGL((k_compress_c4a<D, FP8>), grid, dim3(kCompressThreads), 0, stream, S, gate,
                       T, n, first_entry, cache, cache_scale, cache_rows);
  } else {
    dim3 grid((unsigned)n, (unsigned)B);
    hipLaunchKernelGGL((k_compress_c128a<D, FP8>), grid, dim3(kCompressThreads), 0, stream, S,
                       gate, T, n, first_entry, cache, cache_scale, cache_rows);
  }
  return hipGetLastError();
}

hipError_t launch_compress(int kind, const uint16_t* S, const float* gate, int64_t B, int64_t T,
                           int D, int64_t n, int64_t first_entry, bool fp8, void* cache,
                           float* cache_scale, int64_t cache_rows, hipStream_t stream) {
  if (D == 512)
    return fp8 ? launch_compress_t<512, true>(kind, S, gate, B, T, n, first_entry, cache, cache_scale, cache_rows, stream)
               : launch_compress_t<512, false>(kind, S, gate, B, T, n, first_entry, cache, cache_scale, cache_rows, stream);
  return fp8 ? launch_compress_t<128, true>(kind, S, gate, B, T, n, first_entry, cache, cache_scale, cache_rows, stream)
             : launch_compress_t<128, false>(kind, S, gate, B, T, n, first_entry, cache, cache_scale, cache_rows, stream);
}

}  // namespace cskv
