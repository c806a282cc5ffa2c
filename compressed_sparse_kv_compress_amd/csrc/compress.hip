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
//
// The append kernels serve streaming decode ([P1] cache-block paragraph: a
// constant-size compressor state per layer beside the entries and the
// window): each sequence appends one state to a ring of its newest W states
// (token p in slot p mod W), which is both the attention window and the
// compressor's carry, and an entry is written when its window completes. They
// fold an entry with the same routines as the span kernels, so a streamed
// entry is bit-identical to the one cskv_compress writes for the same states.
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

// Writes one finished entry row held as CPL fp32 values per lane: bf16 (RNE);
// or fp8 codes + one fp32 row scale (amax / 448 over the whole row); or a
// mixed row: the channels below D-64 as fp8 codes with a row scale over them
// alone, then the 64 rotary channels as bf16 (RNE); or an fp4 row: E2M1 codes
// with one E4M3 scale per 16 channels, encoded exactly as cskv_encode_fp4_g16
// does (a group is the 16 channels of a lane pair).
template <int D, int FMT>
__device__ __forceinline__ void store_entry(const float* acc, int lane, void* cache_row,
                                            float* scale_slot) {
  constexpr int CPL = D / kWave;
  if constexpr (FMT == kFmtFp4) {
    static_assert(D == 512, "fp4 rows: D = 512");
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) amax = fmaxf(amax, fabsf(acc[i]));
    amax = fmaxf(amax, dpp_f32<kDppQuadSwap1>(amax));       // the group's other 8 channels
    uint32_t sc = f32_to_e4m3(amax / 6.0f);
    if (e4m3_to_f32(sc) == 0.0f && amax > 0.0f) sc = 0x01u;
    const float sv = e4m3_to_f32(sc);
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) w |= (sv == 0.0f ? 0u : f32_to_e2m1(acc[i] / sv)) << (4 * i);
    uint8_t* row = reinterpret_cast<uint8_t*>(cache_row);
    *reinterpret_cast<uint32_t*>(row + lane * (CPL / 2)) = w;
    if ((lane & 1) == 0) row[D / 2 + lane / 2] = (uint8_t)sc;
    (void)scale_slot;
  } else if constexpr (FMT == kFmtMix) {
    static_assert(D == 512, "mixed rows: D = 512");
    const bool rope = lane * CPL >= D - kMixRope;          // lanes 56 .. 63
    float amax = 0.0f;
    if (!rope) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) amax = fmaxf(amax, fabsf(acc[i]));
    }
    amax = wave_max(amax);
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint8_t* row = reinterpret_cast<uint8_t*>(cache_row);
    if (!rope) {
      uint32_t c[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) c[i] = f32_to_e4m3(acc[i] / scale);
      uint2 q;
      q.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      q.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      *reinterpret_cast<uint2*>(row + lane * CPL) = q;
    } else {
      uint4 q;
      q.x = pack_bf16x2(acc[0], acc[1]); q.y = pack_bf16x2(acc[2], acc[3]);
      q.z = pack_bf16x2(acc[4], acc[5]); q.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(row + (D - kMixRope) + 2 * (lane * CPL - (D - kMixRope))) = q;
    }
    if (lane == 0) *scale_slot = scale;
  } else if constexpr (FMT == kFmtBf16) {
    uint16_t* out = reinterpret_cast<uint16_t*>(cache_row) + lane * CPL;
    if constexpr (CPL == 8) {
      uint4 q;
      q.x = pack_bf16x2(acc[0], acc[1]); q.y = pack_bf16x2(acc[2], acc[3]);
      q.z = pack_bf16x2(acc[4], acc[5]); q.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(out) = q;
    } else {
      *reinterpret_cast<uint32_t*>(out) = pack_bf16x2(acc[0], acc[1]);
    }
  } else {   // fp8
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
// One c4a entry from its 8 states (lo: states 0-3, hi: states 4-7) and their
// gate logits: softmax weights in fp32, then one fma per state in order.
template <int D>
__device__ __forceinline__ void fold_c4a(const RowSlice<D>* lo, const RowSlice<D>* hi, const float* g,
                                         float* acc) {
  float m = g[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) m = fmaxf(m, g[j]);
  // every lane holds the same 8 logits: lane j (mod 8) takes the exponential
  // and the weight of state j once, and the fold reads them with readlane
  // (the same operations on the same values, and the sum in the same order,
  // as 8 exponentials and 8 divisions in every lane)
  const int lane = lane_id();
  float gl = g[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) gl = (lane & 7) == j ? g[j] : gl;
  const float el = expf(gl - m);
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) z += lane_value(el, j);
  const float wl = el / z;
#pragma unroll
  for (int i = 0; i < RowSlice<D>::CPL; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float w = lane_value(wl, j);
#pragma unroll
    for (int i = 0; i < RowSlice<D>::CPL; ++i) acc[i] = fmaf(w, lo[j].v[i], acc[i]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float w = lane_value(wl, 4 + j);
#pragma unroll
    for (int i = 0; i < RowSlice<D>::CPL; ++i) acc[i] = fmaf(w, hi[j].v[i], acc[i]);
  }
}

// One wave owns a run of `run` consecutive entries of one sequence. Entry c
// reads stride blocks c and c+1 (4 states each); the wave keeps the previous
// block in registers so every state of the run is loaded once. Long spans use
// runs of 16; short decode-time spans shorter ones, down to one entry per wave,
// so that there are enough waves in flight (the entries do not depend on it).
constexpr int kC4aRunMax = 16;
constexpr int kCompressThreads = 256;

template <int D, int FMT>
__global__ __launch_bounds__(kCompressThreads) void k_compress_c4a(
    const uint16_t* __restrict__ S, const float* __restrict__ gate, int64_t T, int64_t n_entries,
    int64_t first_entry, void* __restrict__ cache, float* __restrict__ cache_scale,
    int64_t cache_rows, int run) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.y;
  const int64_t c0 = ((int64_t)blockIdx.x * (kCompressThreads / kWave) + wave) * run;
  if (c0 >= n_entries) return;
  const int64_t c1 = c0 + run < n_entries ? c0 + run : n_entries;

  const uint16_t* Sb = S + b * T * D;
  const float* gb = gate + b * T;
  constexpr int RB = row_bytes<D, FMT>();
  uint8_t* cb = reinterpret_cast<uint8_t*>(cache) + (b * cache_rows + first_entry) * (int64_t)RB;
  float* sb = FMT == kFmtFp8 || FMT == kFmtMix ? cache_scale + b * cache_rows + first_entry : nullptr;

  RowSlice<D> prev[4], cur[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) load_row<D>(Sb + (4 * c0 + j) * D, lane, prev[j]);

  for (int64_t c = c0; c < c1; ++c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) load_row<D>(Sb + (4 * c + 4 + j) * D, lane, cur[j]);
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = gb[4 * c + j];
    float acc[RowSlice<D>::CPL];
    fold_c4a<D>(prev, cur, g, acc);
    store_entry<D, FMT>(acc, lane, cb + c * (int64_t)RB, sb ? sb + c : nullptr);
#pragma unroll
    for (int j = 0; j < 4; ++j) prev[j] = cur[j];
  }
}

// ---------------------------------------------------------------- c128a
// One c128a entry from its 128 states (row_at(j): state j's row, gate_at(j):
// its logit), by the 4 waves of a workgroup: wave w folds states 32w .. 32w+31,
// then the four partial rows are added in wave order through LDS. The entry
// ends in wave 0's acc. Every thread of the workgroup must call it.
template <int D, class RowAt, class GateAt>
__device__ __forceinline__ void fold_c128a(RowAt row_at, GateAt gate_at, float (*part)[D], float* acc) {
  constexpr int CPL = D / kWave;
  constexpr int NW = kCompressThreads / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  // 4 batches of 8 states, the next batch's rows loaded while the current
  // one is folded
  RowSlice<D> r[8], nx[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) load_row<D>(row_at(32 * wave + u), lane, r[u]);
  // softmax over the 128 logits; every wave computes the same max and sum.
  // Lane l holds states l and l + 64 and takes their weights once; the fold
  // reads state s's weight from lane s mod 64 with readlane (the same
  // operations on the same values as one exponential and one division per
  // state in every lane)
  const float g0 = gate_at(lane), g1 = gate_at(lane + 64);
  const float m = wave_max(fmaxf(g0, g1));
  const float e0 = expf(g0 - m), e1 = expf(g1 - m);
  const float z = wave_sum(e0 + e1);
  const float w0 = e0 / z, w1 = e1 / z;
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j0 = 0; j0 < 32; j0 += 8) {
    if (j0 + 8 < 32) {
#pragma unroll
      for (int u = 0; u < 8; ++u) load_row<D>(row_at(32 * wave + j0 + 8 + u), lane, nx[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int st = 32 * wave + j0 + u;   // (wave-uniform)
      const float w = lane_value(st < 64 ? w0 : w1, st & 63);
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] = fmaf(w, r[u].v[i], acc[i]);
    }
    if (j0 + 8 < 32) {
#pragma unroll
      for (int u = 0; u < 8; ++u) r[u] = nx[u];
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
}

// One workgroup per entry.
template <int D, int FMT>
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
  float acc[CPL];
  fold_c128a<D>([&](int j) { return Sw + (int64_t)j * D; }, [&](int j) { return gw[j]; }, part, acc);
  if (wave != 0) return;
  const int64_t row = b * cache_rows + first_entry + c;
  store_entry<D, FMT>(acc, lane, reinterpret_cast<uint8_t*>(cache) + row * (int64_t)row_bytes<D, FMT>(),
                      FMT == kFmtFp8 || FMT == kFmtMix ? cache_scale + row : nullptr);
}

// bf16 rows when entries are fewer than compute units: workgroup (c, b, q)
// folds channels 128q .. 128q+127 of entry c. Every channel's fold (weights,
// order of the sums) is the whole-row kernel's, so the rows are bit-identical.
template <int D>
__global__ __launch_bounds__(kCompressThreads) void k_compress_c128a_slice(
    const uint16_t* __restrict__ S, const float* __restrict__ gate, int64_t T, int64_t first_entry,
    uint16_t* __restrict__ cache, int64_t cache_rows) {
  constexpr int DS = 128;
  constexpr int NW = kCompressThreads / kWave;
  __shared__ float part[NW][DS];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int q = blockIdx.z;
  const uint16_t* Sw = S + (b * T + 128 * c) * D + DS * q;
  const float* gw = gate + b * T + 128 * c;
  float acc[DS / kWave];
  fold_c128a<DS>([&](int j) { return Sw + (int64_t)j * D; }, [&](int j) { return gw[j]; }, part, acc);
  if (wave != 0) return;
  const int64_t row = b * cache_rows + first_entry + c;
  store_entry<DS, kFmtBf16>(acc, lane, cache + row * D + DS * q, nullptr);
}

// ---------------------------------------------------------------- append
// Sequence b appends state s_new[b] (gate logit g_new[b]) as token p = pos[b]
// (p < 0: the sequence is skipped). The state goes to ring slot p mod W; the
// entry whose window ends at p (c4a: p % 4 == 3 and p >= 7; c128a: p % 128 ==
// 127) is folded from the ring's older states plus the new one, read from the
// input, so no thread reads what this launch writes. The counts are the
// entries present in the cache and the window rows in the ring.

// The new state into its ring slot: lane l copies channels CPL*l .. CPL*l+CPL-1.
template <int D>
__device__ __forceinline__ void ring_put(const uint16_t* snew, uint16_t* dst, int lane) {
  constexpr int CPL = D / kWave;
  if constexpr (CPL == 8) {
    *reinterpret_cast<uint4*>(dst + lane * 8) = *reinterpret_cast<const uint4*>(snew + lane * 8);
  } else {
    *reinterpret_cast<uint32_t*>(dst + lane * 2) = *reinterpret_cast<const uint32_t*>(snew + lane * 2);
  }
}

__device__ __forceinline__ void append_counts(int64_t n, int64_t p, int W, int64_t cache_rows, int64_t b,
                                              int32_t* n_entries, int32_t* n_window) {
  if (n_entries) n_entries[b] = (int32_t)(n < cache_rows ? n : cache_rows);
  if (n_window) n_window[b] = (int32_t)(p + 1 < W ? p + 1 : W);
}

constexpr int kAppendC4aSeqs = kCompressThreads / kWave;   // c4a: one wave per sequence

template <int D, int FMT>
__global__ __launch_bounds__(kCompressThreads) void k_append_c4a(
    const uint16_t* __restrict__ s_new, const float* __restrict__ g_new, const int64_t* __restrict__ pos,
    int64_t B, uint16_t* __restrict__ ring, float* __restrict__ ring_gate, int W, void* __restrict__ cache,
    float* __restrict__ cache_scale, int64_t cache_rows, int32_t* __restrict__ n_entries,
    int32_t* __restrict__ n_window) {
  const int lane = lane_id();
  const int64_t b = (int64_t)blockIdx.x * kAppendC4aSeqs + threadIdx.x / kWave;
  if (b >= B) return;
  const int64_t p = pos[b];
  if (p < 0) return;
  const uint16_t* snew = s_new + b * D;
  uint16_t* rb = ring + b * (int64_t)W * D;
  float* gb = ring_gate + b * (int64_t)W;
  const int64_t slot = p % W;
  ring_put<D>(snew, rb + slot * D, lane);
  if (lane == 0) {
    gb[slot] = g_new[b];
    append_counts(p >= 7 ? (p - 7) / 4 + 1 : 0, p, W, cache_rows, b, n_entries, n_window);
  }
  if (p < 7 || (p & 3) != 3) return;
  const int64_t c = (p - 7) >> 2;
  if (c >= cache_rows) return;
  const int64_t s0 = (p - 7) % W;
  RowSlice<D> r[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const int64_t sl = s0 + j < W ? s0 + j : s0 + j - W;
    load_row<D>(rb + sl * D, lane, r[j]);
    g[j] = gb[sl];
  }
  load_row<D>(snew, lane, r[7]);
  g[7] = g_new[b];
  float acc[RowSlice<D>::CPL];
  fold_c4a<D>(r, r + 4, g, acc);
  const int64_t row = b * cache_rows + c;
  store_entry<D, FMT>(acc, lane, reinterpret_cast<uint8_t*>(cache) + row * (int64_t)row_bytes<D, FMT>(),
                      FMT == kFmtFp8 || FMT == kFmtMix ? cache_scale + row : nullptr);
}

template <int D, int FMT>
__global__ __launch_bounds__(kCompressThreads) void k_append_c128a(
    const uint16_t* __restrict__ s_new, const float* __restrict__ g_new, const int64_t* __restrict__ pos,
    uint16_t* __restrict__ ring, float* __restrict__ ring_gate, int W, void* __restrict__ cache,
    float* __restrict__ cache_scale, int64_t cache_rows, int32_t* __restrict__ n_entries,
    int32_t* __restrict__ n_window) {
  constexpr int CPL = D / kWave;
  constexpr int NW = kCompressThreads / kWave;
  __shared__ float part[NW][D];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t b = blockIdx.x;
  const int64_t p = pos[b];   // (every exit below is uniform over the workgroup)
  if (p < 0) return;
  const uint16_t* snew = s_new + b * D;
  uint16_t* rb = ring + b * (int64_t)W * D;
  float* gb = ring_gate + b * (int64_t)W;
  if (wave == 0) {
    const int64_t slot = p % W;
    ring_put<D>(snew, rb + slot * D, lane);
    if (lane == 0) {
      gb[slot] = g_new[b];
      append_counts((p + 1) / 128, p, W, cache_rows, b, n_entries, n_window);
    }
  }
  if ((p & 127) != 127) return;
  const int64_t c = p >> 7;
  if (c >= cache_rows) return;
  const int64_t s0 = (p - 127) % W;
  const float gn = g_new[b];
  auto slot_of = [&](int j) { return s0 + j < W ? s0 + j : s0 + j - W; };
  float acc[CPL];
  fold_c128a<D>([&](int j) { return j == 127 ? snew : rb + slot_of(j) * D; },
                [&](int j) { return j == 127 ? gn : gb[slot_of(j)]; }, part, acc);
  if (wave != 0) return;
  const int64_t row = b * cache_rows + c;
  store_entry<D, FMT>(acc, lane, reinterpret_cast<uint8_t*>(cache) + row * (int64_t)row_bytes<D, FMT>(),
                      FMT == kFmtFp8 || FMT == kFmtMix ? cache_scale + row : nullptr);
}

// ---------------------------------------------------------------- launch

template <int D, int FMT>
static hipError_t launch_compress_t(int kind, const uint16_t* S, const float* gate, int64_t B,
                                    int64_t T, int64_t n, int64_t first_entry, void* cache,
                                    float* cache_scale, int64_t cache_rows, hipStream_t stream) {
  if (kind == 0) {
    // about 4096 waves over the batch, or runs of kC4aRunMax when there are more
    int run = kC4aRunMax;
    while (run > 1 && B * ((n + run - 1) / run) < 4096) run /= 2;
    const int64_t per_block = (int64_t)run * (kCompressThreads / kWave);
    dim3 grid((unsigned)((n + per_block - 1) / per_block), (unsigned)B);
    hipLaunchKernelGGL((k_compress_c4a<D, FMT>), grid, dim3(kCompressThreads), 0, stream, S, gate,
                       T, n, first_entry, cache, cache_scale, cache_rows, run);
  } else {
    if constexpr (FMT == kFmtBf16 && D == 512) {
      if (n * B < 256) {
        // fewer entries than compute units: four channel slices per entry
        dim3 grid((unsigned)n, (unsigned)B, D / 128);
        hipLaunchKernelGGL((k_compress_c128a_slice<D>), grid, dim3(kCompressThreads), 0, stream, S, gate, T,
                           first_entry, reinterpret_cast<uint16_t*>(cache), cache_rows);
        return hipGetLastError();
      }
    }
    dim3 grid((unsigned)n, (unsigned)B);
    hipLaunchKernelGGL((k_compress_c128a<D, FMT>), grid, dim3(kCompressThreads), 0, stream, S,
                       gate, T, n, first_entry, cache, cache_scale, cache_rows);
  }
  return hipGetLastError();
}

template <int D, int FMT>
static hipError_t launch_append_t(int kind, const uint16_t* s_new, const float* g_new, const int64_t* pos,
                                  int64_t B, uint16_t* ring, float* ring_gate, int W, void* cache,
                                  float* cache_scale, int64_t cache_rows, int32_t* n_entries,
                                  int32_t* n_window, hipStream_t stream) {
  if (kind == 0) {
    dim3 grid((unsigned)((B + kAppendC4aSeqs - 1) / kAppendC4aSeqs));
    hipLaunchKernelGGL((k_append_c4a<D, FMT>), grid, dim3(kCompressThreads), 0, stream, s_new, g_new, pos, B,
                       ring, ring_gate, W, cache, cache_scale, cache_rows, n_entries, n_window);
  } else {
    hipLaunchKernelGGL((k_append_c128a<D, FMT>), dim3((unsigned)B), dim3(kCompressThreads), 0, stream, s_new,
                       g_new, pos, ring, ring_gate, W, cache, cache_scale, cache_rows, n_entries, n_window);
  }
  return hipGetLastError();
}

hipError_t launch_append(int kind, const uint16_t* s_new, const float* g_new, const int64_t* pos, int64_t B,
                         int D, uint16_t* ring, float* ring_gate, int W, int fmt, void* cache,
                         float* cache_scale, int64_t cache_rows, int32_t* n_entries, int32_t* n_window,
                         hipStream_t stream) {
#define CSKV_APPEND(DD, FF) launch_append_t<DD, FF>(kind, s_new, g_new, pos, B, ring, ring_gate, W, cache, \
                                                   cache_scale, cache_rows, n_entries, n_window, stream)
  if (D == 512) {
    if (fmt == kFmtFp4) return CSKV_APPEND(512, kFmtFp4);
    return fmt == kFmtMix ? CSKV_APPEND(512, kFmtMix) : (fmt == kFmtFp8 ? CSKV_APPEND(512, kFmtFp8) : CSKV_APPEND(512, kFmtBf16));
  }
  return fmt == kFmtFp8 ? CSKV_APPEND(128, kFmtFp8) : CSKV_APPEND(128, kFmtBf16);
#undef CSKV_APPEND
}

hipError_t launch_compress(int kind, const uint16_t* S, const float* gate, int64_t B, int64_t T,
                           int D, int64_t n, int64_t first_entry, int fmt, void* cache,
                           float* cache_scale, int64_t cache_rows, hipStream_t stream) {
#define CSKV_COMPRESS(DD, FF) launch_compress_t<DD, FF>(kind, S, gate, B, T, n, first_entry, cache, cache_scale, \
                                                       cache_rows, stream)
  if (D == 512) {
    if (fmt == kFmtFp4) return CSKV_COMPRESS(512, kFmtFp4);
    return fmt == kFmtMix ? CSKV_COMPRESS(512, kFmtMix) : (fmt == kFmtFp8 ? CSKV_COMPRESS(512, kFmtFp8) : CSKV_COMPRESS(512, kFmtBf16));
  }
  return fmt == kFmtFp8 ? CSKV_COMPRESS(128, kFmtFp8) : CSKV_COMPRESS(128, kFmtBf16);
#undef CSKV_COMPRESS
}

}  // namespace cskv
