// Indexer scores and exact top-k over c4a entries.
//
// [P1] "c4a (the milder scheme)": DeepSeek Sparse Attention keeps the top-k
// compressed entries per query (default k = 512). [P2] Step 5: a learned
// indexer scores every compressed block; the query reads only the chosen ones.
//
// Three kernels:
//   k_index_score  (grid: chunks x sequences) streams the indexer keys once
//     from HBM with 16-byte coalesced loads (bf16, or fp4 codes + E4M3 group
//     scales dequantised in registers), computes each entry's score as a GEMV
//     against the query's indexer vector, turns it into an order-preserving
//     32-bit key, writes the keys to the workspace (4 B per entry, coalesced)
//     and adds the chunk's histogram of the top 12 key bits into a
//     per-sequence histogram.
//   k_topk_filter  (grid: slices x sequences) finds, from that histogram, the
//     bin holding the k-th largest key and keeps the entries of its slice
//     whose bin is at or above it, in entry order (about k plus one bin's
//     worth per sequence). It also adds a histogram of the next 8 key bits of
//     the threshold bin's keys into a per-sequence 256-bin histogram, and the
//     first slice records the threshold bin and the count of keys above it.
//   k_topk_final   (grid: sequences) finds from the 256-bin histogram the
//     20-bit prefix of the k-th largest key, gathers the candidates, resolves
//     the remaining 12 key bits by radix select in LDS, writes the ids in
//     ascending entry order (ties go to the lower entry) and clears both
//     histograms for the next call.
// The selection is exact: every entry of a bin above the threshold bin is in
// the top k, and the threshold bin is resolved on full keys.
#include "kernels.h"

namespace cskv {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;   // per-sequence histogram of the top key bits
constexpr int kBinShift = 32 - kHistBits;
constexpr int kRadixPad = 257;              // per-wave radix histograms, bank-shifted
constexpr int kCandCap = 4096;              // candidates the final select holds in LDS
constexpr int kSliceUnit = 2048;            // keys a select workgroup filters per round
constexpr int kMaxSlices = 2048;
constexpr int kMisc = 16;
constexpr int kSubBits = 8;                 // key bits below the threshold bin resolved by the filter
constexpr int kSubBins = 1 << kSubBits;
constexpr int kLowBits = kBinShift - kSubBits;   // 12 bits left to the final select

// ------------------------------------------------------------- block helpers

// Exclusive prefix sum over the block in thread order; also returns the total.
__device__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int incl = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int s = scratch[w];
    if (w < wave) before += s;
    total += s;
  }
  __syncthreads();
  return before + incl - v;
}

// Radix select on the low `low_bits` bits: among keys[0..n) whose bits above
// `low_bits` equal those of `prefix`, finds the rem-th largest (1 <= rem <=
// their count). Returns the full key T and how many keys equal to T are
// needed. `keys` may be in LDS or global memory; `hist` is LDS.
__device__ void radix_select(const uint32_t* keys, int n, int rem, uint32_t prefix, int low_bits,
                             uint32_t* hist, int* misc, uint32_t& T_out, int& need_eq_out) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  int hi = low_bits;
  while (hi > 0) {
    const int w = hi < 8 ? hi : 8;
    const int shift = hi - w;
    const uint32_t dmask = (1u << w) - 1u;
    for (int i = t; i < kTopkWaves * kRadixPad; i += kTopkThreads) hist[i] = 0u;
    __syncthreads();
    uint32_t* h = hist + wave * kRadixPad;
    for (int i0 = 0; i0 < n; i0 += 4 * kTopkThreads) {
      uint32_t kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kTopkThreads + t;
        kv[u] = i < n ? keys[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kTopkThreads + t;
        const bool match = hi >= 32 || ((kv[u] ^ prefix) >> hi) == 0u;
        if (i < n && match) atomicAdd(&h[(kv[u] >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l covers digits 255-4l .. 252-4l: the scan runs from the top digit down
      int c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 255 - 4 * lane - j;
        int v = 0;
#pragma unroll
        for (int ww = 0; ww < kTopkWaves; ++ww) v += (int)hist[ww * kRadixPad + d];
        c[j] = v;
        s += v;
      }
      int above = wave_inclusive_scan(s) - s;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < rem && rem <= above + c[j]) {
          misc[0] = 255 - 4 * lane - j;
          misc[1] = above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    prefix = (prefix & ~(dmask << shift)) | ((uint32_t)misc[0] << shift);
    rem -= misc[1];
    hi = shift;
    __syncthreads();
  }
  T_out = prefix;
  need_eq_out = rem;
}

// Emits, in index order, every key > T plus the first need_eq keys == T (or
// every key when `all`): writes out_idx[p] = idx_map[i] (or idx_base + i).
// Returns the number emitted (same in all threads).
__device__ int block_emit(const uint32_t* keys, int n, bool all, uint32_t T, int need_eq, int* misc,
                          int32_t* out_idx, int out_cap, const int32_t* idx_map, int32_t idx_base) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int per = (((n + kTopkWaves - 1) / kTopkWaves) + kWave - 1) & ~(kWave - 1);
  const int lo = wave * per;
  const int hi = min(lo + per, n);
  int gt = 0, eq = 0;
  for (int base = lo; base < hi; base += kWave) {
    const int i = base + lane;
    const bool valid = i < hi;
    const uint32_t key = valid ? keys[i] : 0u;
    gt += __popcll(__ballot(valid && (all || key > T)));
    eq += __popcll(__ballot(valid && !all && key == T));
  }
  if (lane == 0) {
    misc[4 + wave] = gt;
    misc[4 + kTopkWaves + wave] = eq;
  }
  __syncthreads();
  int eq_before = 0, sel_before = 0, total = 0;
  {
    int eb = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const int e = misc[4 + kTopkWaves + w];
      const int take = min(max(need_eq - eb, 0), e);
      const int sel = misc[4 + w] + take;
      if (w < wave) {
        sel_before += sel;
        eq_before += e;
      }
      total += sel;
      eb += e;
    }
  }
  int eq_run = eq_before, pos = sel_before;
  for (int base = lo; base < hi; base += kWave) {
    const int i = base + lane;
    const bool valid = i < hi;
    const uint32_t key = valid ? keys[i] : 0u;
    const bool is_gt = valid && (all || key > T);
    const bool is_eq = valid && !all && key == T;
    const uint64_t eqm = __ballot(is_eq);
    const int eq_rank = eq_run + __popcll(eqm & lanemask_lt());
    const bool sel = is_gt || (is_eq && eq_rank < need_eq);
    const uint64_t selm = __ballot(sel);
    if (sel) {
      const int p = pos + __popcll(selm & lanemask_lt());
      if (p < out_cap) out_idx[p] = idx_map ? idx_map[i] : idx_base + i;
    }
    eq_run += __popcll(eqm);
    pos += __popcll(selm);
  }
  __syncthreads();  // misc is reused by the caller
  return total < out_cap ? total : out_cap;
}

// ------------------------------------------------------------- scoring

// Records one scored entry: its order key in LDS and in the chunk histogram.
__device__ __forceinline__ void put_key(uint32_t* keys, uint32_t* hist, int e, float score) {
  const uint32_t key = score_key(score);
  keys[e] = key;
  atomicAdd(&hist[key >> kBinShift], 1u);
}

// bf16 keys: LPE = DI/8 lanes read one 16-byte slice each of an entry; one
// wave-wide load covers 64/LPE consecutive entries (1 KiB contiguous).
template <int DI>
__device__ void score_chunk_bf16(const uint16_t* q, const uint16_t* keys_g, int n, uint32_t* keys,
                                 uint32_t* hist) {
  constexpr int LPE = DI / 8;
  constexpr int EPL = kWave / LPE;
  constexpr int U = 8;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane / LPE, cg = lane % LPE;
  const uint4 qv = *reinterpret_cast<const uint4*>(q + cg * 8);
  const bf16x2_t q0 = __builtin_bit_cast(bf16x2_t, qv.x), q1 = __builtin_bit_cast(bf16x2_t, qv.y);
  const bf16x2_t q2 = __builtin_bit_cast(bf16x2_t, qv.z), q3 = __builtin_bit_cast(bf16x2_t, qv.w);
  const uint4* kp = reinterpret_cast<const uint4*>(keys_g);
  const int n_groups = (n + EPL - 1) / EPL;
  for (int g0 = wave; g0 < n_groups; g0 += kTopkWaves * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = (g0 + kTopkWaves * u) * EPL + sub;
      v[u] = e < n ? load_stream(kp + (int64_t)e * LPE + cg) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v[u].x), q0, 0.0f, false);
      p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v[u].y), q1, p, false);
      p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v[u].z), q2, p, false);
      p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v[u].w), q3, p, false);
      if constexpr (LPE == 16) p = sum_row16(p);
      else if constexpr (LPE == 4) p = sum_quad(p);
      const int e = (g0 + kTopkWaves * u) * EPL + sub;
      if (cg == 0 && e < n) put_key(keys, hist, e, p);
    }
  }
}

// fp4 keys: each lane reads 16 code bytes (32 channels = two 16-channel groups)
// and the two matching E4M3 group scales; LPE = DI/32 lanes per entry. The
// E2M1 codes are widened to bf16 exactly by the gfx950 converter.
template <int DI>
__device__ void score_chunk_fp4(const uint16_t* q, const uint8_t* codes_g, const uint8_t* scales_g,
                                int n, uint32_t* keys, uint32_t* hist) {
  constexpr int LPE = DI / 32;
  constexpr int EPL = kWave / LPE;
  constexpr int U = 8;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane / LPE, part = lane % LPE;
  bf16x2_t qp[16];
  {
    const uint4* qq = reinterpret_cast<const uint4*>(q + part * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = qq[i];
      qp[4 * i + 0] = __builtin_bit_cast(bf16x2_t, x.x);
      qp[4 * i + 1] = __builtin_bit_cast(bf16x2_t, x.y);
      qp[4 * i + 2] = __builtin_bit_cast(bf16x2_t, x.z);
      qp[4 * i + 3] = __builtin_bit_cast(bf16x2_t, x.w);
    }
  }
  const uint4* cp = reinterpret_cast<const uint4*>(codes_g);
  const uint16_t* sp = reinterpret_cast<const uint16_t*>(scales_g);
  const int n_groups = (n + EPL - 1) / EPL;
  for (int g0 = wave; g0 < n_groups; g0 += kTopkWaves * U) {
    uint4 v[U];
    uint32_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = (g0 + kTopkWaves * u) * EPL + sub;
      v[u] = e < n ? load_stream(cp + (int64_t)e * LPE + part) : make_uint4(0, 0, 0, 0);
      s[u] = e < n ? load_stream(sp + (int64_t)e * LPE + part) : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float g0s = 0.0f, g1s = 0.0f;
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<0>(v[u].x), qp[0], g0s, false);
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<1>(v[u].x), qp[1], g0s, false);
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<2>(v[u].x), qp[2], g0s, false);
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<3>(v[u].x), qp[3], g0s, false);
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<0>(v[u].y), qp[4], g0s, false);
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<1>(v[u].y), qp[5], g0s, false);
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<2>(v[u].y), qp[6], g0s, false);
      g0s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<3>(v[u].y), qp[7], g0s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<0>(v[u].z), qp[8], g1s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<1>(v[u].z), qp[9], g1s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<2>(v[u].z), qp[10], g1s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<3>(v[u].z), qp[11], g1s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<0>(v[u].w), qp[12], g1s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<1>(v[u].w), qp[13], g1s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<2>(v[u].w), qp[14], g1s, false);
      g1s = __builtin_amdgcn_fdot2_f32_bf16(fp4x2_to_bf16x2<3>(v[u].w), qp[15], g1s, false);
      float p = fmaf(g1s, e4m3_to_f32(s[u] >> 8), g0s * e4m3_to_f32(s[u] & 0xFFu));
      if constexpr (LPE == 4) p = sum_quad(p);
      const int e = (g0 + kTopkWaves * u) * EPL + sub;
      if (part == 0 && e < n) put_key(keys, hist, e, p);
    }
  }
}

template <int DI, bool FP4>
__global__ __launch_bounds__(kTopkThreads) void k_index_score(
    const uint16_t* __restrict__ q_idx, const void* __restrict__ k_idx,
    const uint8_t* __restrict__ k_scale, const int32_t* __restrict__ n_entries, int64_t n_max,
    int chunk, int64_t key_stride, uint32_t* __restrict__ ws_keys, uint32_t* __restrict__ ws_hist) {
  extern __shared__ uint32_t lds[];
  uint32_t* hist = lds;
  uint32_t* keys = lds + kHistBins;
  const int t = threadIdx.x;
  const int64_t b = blockIdx.y;
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int64_t start = (int64_t)blockIdx.x * chunk;
  const int64_t rem = nv - start;
  if (rem <= 0) return;
  const int n = rem > chunk ? chunk : (int)rem;

  for (int i = t; i < kHistBins; i += kTopkThreads) hist[i] = 0u;
  __syncthreads();
  const uint16_t* q = q_idx + b * DI;
  if constexpr (FP4) {
    const uint8_t* codes = reinterpret_cast<const uint8_t*>(k_idx) + (b * n_max + start) * (DI / 2);
    const uint8_t* scales = k_scale + (b * n_max + start) * (DI / 16);
    score_chunk_fp4<DI>(q, codes, scales, n, keys, hist);
  } else {
    const uint16_t* kk = reinterpret_cast<const uint16_t*>(k_idx) + (b * n_max + start) * DI;
    score_chunk_bf16<DI>(q, kk, n, keys, hist);
  }
  __syncthreads();
  // keys -> workspace (start and key_stride are multiples of 4: 16-byte stores)
  uint32_t* dst = ws_keys + b * key_stride + start;
  for (int i = 4 * t; i < n; i += 4 * kTopkThreads) {
    if (i + 4 <= n) {
      *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(keys + i);
    } else {
      for (int j = i; j < n; ++j) dst[j] = keys[j];
    }
  }
  uint32_t* gh = ws_hist + b * kHistBins;
  for (int i = t; i < kHistBins; i += kTopkThreads) {
    const uint32_t h = hist[i];
    if (h) atomicAdd(&gh[i], h);
  }
}

// ------------------------------------------------------------- selection

struct SelectLds {
  uint32_t ckey[kCandCap];
  int32_t cidx[kCandCap];
  uint16_t slice_of[kCandCap];   // slice of each gathered candidate
  uint32_t rhist[kTopkWaves * kRadixPad];
  int pre[kMaxSlices + 1];
  int misc[kMisc];
  int scan[kTopkWaves];
};

// A thread's 16 bins of a sequence histogram, thread 0 holding the top ones
// (h[15] is the thread's highest bin).
constexpr int kBinsPerThread = kHistBins / kTopkThreads;
__device__ __forceinline__ void load_hist16(const uint32_t* gh, uint32_t (&h)[kBinsPerThread]) {
  const int top = kHistBins - 1 - kBinsPerThread * (int)threadIdx.x;
  const uint4* p = reinterpret_cast<const uint4*>(gh + top - (kBinsPerThread - 1));
#pragma unroll
  for (int i = 0; i < kBinsPerThread / 4; ++i) {
    const uint4 v = p[i];
    h[4 * i] = v.x; h[4 * i + 1] = v.y; h[4 * i + 2] = v.z; h[4 * i + 3] = v.w;
  }
}

// The bin of the k-th largest key of a sequence (1 <= k < total) and the
// number of keys in the bins above it, from the histogram slices of load_hist16.
__device__ void threshold_bin(const uint32_t (&h)[kBinsPerThread], int k, int* scan, int* misc, int& tbin,
                              int& above) {
  const int top = kHistBins - 1 - kBinsPerThread * (int)threadIdx.x;
  int s = 0;
#pragma unroll
  for (int i = 0; i < kBinsPerThread; ++i) s += (int)h[i];
  int total;
  int run = block_exclusive_scan(s, scan, total);
  if (run < k && k <= run + s) {
#pragma unroll
    for (int i = kBinsPerThread - 1; i >= 0; --i) {
      const int c = (int)h[i];
      if (run < k && k <= run + c) {
        misc[0] = top - (kBinsPerThread - 1 - i);
        misc[1] = run;
      }
      run += c;
    }
  }
  __syncthreads();
  tbin = misc[0];
  above = misc[1];
  __syncthreads();
}

// One workgroup per slice of a sequence: keeps the keys whose histogram bin
// is at or above the threshold bin, in entry order, with their entry numbers.
__global__ __launch_bounds__(kTopkThreads) void k_topk_filter(
    const uint32_t* __restrict__ ws_keys, int64_t key_stride, const int32_t* __restrict__ n_entries,
    int64_t n_max, int k, int slice, int n_slices, const uint32_t* __restrict__ ws_hist,
    uint32_t* __restrict__ ws_hist2, int2* __restrict__ ws_thr, uint32_t* __restrict__ ws_ckey,
    int32_t* __restrict__ ws_cidx, int32_t* __restrict__ ws_cnt) {
  __shared__ int scan[kTopkWaves];
  __shared__ int misc[kMisc];
  __shared__ uint32_t h2[kSubBins];       // next 8 bits of this slice's threshold-bin keys
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int64_t b = blockIdx.y;
  const int s = blockIdx.x;
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int n_here = (int)min((int64_t)slice, max((int64_t)0, nv - (int64_t)s * slice));
  int tbin = 0, above = 0;
  bool have_tbin = nv <= k;
  const bool take_all = have_tbin;
  for (int i = t; i < kSubBins; i += kTopkThreads) h2[i] = 0u;
  __syncthreads();

  const int64_t cand_base = (b * n_slices + s) * (int64_t)slice;
  const uint32_t* src = ws_keys + b * key_stride + (int64_t)s * slice;
  int written = 0;
  for (int r0 = 0; r0 < n_here; r0 += kSliceUnit) {
    const int rn = min(kSliceUnit, n_here - r0);
    // wave w owns keys [r0 + 512w, r0 + 512w + 512) of the round, lane-strided
    constexpr int PER = kSliceUnit / kTopkThreads;   // 8
    uint32_t kv[PER];
    bool keep[PER];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = wave * (PER * kWave) + u * kWave + lane;
      kv[u] = i < rn ? src[r0 + i] : 0u;
    }
    if (!have_tbin) {   // the histogram is read while the keys are in flight
      uint32_t h[kBinsPerThread];
      load_hist16(ws_hist + b * kHistBins, h);
      threshold_bin(h, k, scan, misc, tbin, above);
      have_tbin = true;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = wave * (PER * kWave) + u * kWave + lane;
      keep[u] = i < rn && (int)(kv[u] >> kBinShift) >= tbin;
      cnt += __popcll(__ballot(keep[u]));
      if (!take_all && i < rn && (int)(kv[u] >> kBinShift) == tbin)
        atomicAdd(&h2[(kv[u] >> kLowBits) & (kSubBins - 1)], 1u);
    }
    if (lane == 0) scan[wave] = cnt;
    __syncthreads();
    int pos = written, round_total = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const int c = scan[w];
      if (w < wave) pos += c;
      round_total += c;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const uint64_t m = __ballot(keep[u]);
      if (keep[u]) {
        const int p = pos + __popcll(m & lanemask_lt());
        const int i = wave * (PER * kWave) + u * kWave + lane;
        ws_ckey[cand_base + p] = kv[u];
        ws_cidx[cand_base + p] = (int32_t)((int64_t)s * slice + r0 + i);
      }
      pos += __popcll(m);
    }
    written += round_total;
  }
  if (t == 0) ws_cnt[b * n_slices + s] = written;
  if (!take_all) {
    if (s == 0 && t == 0) ws_thr[b] = make_int2(tbin, above);   // (nv > k: slice 0 holds keys)
    __syncthreads();
    for (int i = t; i < kSubBins; i += kTopkThreads) {
      const uint32_t c = h2[i];
      if (c) atomicAdd(&ws_hist2[b * kSubBins + i], c);
    }
  }
}

// One workgroup per sequence: finds the 20-bit prefix of the k-th largest key
// from the filter's threshold bin and 256-bin histogram, gathers the slices'
// candidates, resolves the remaining 12 bits on full keys, writes the ids
// (ascending, -1 padded) and clears both histograms for the next call.
__global__ __launch_bounds__(kTopkThreads) void k_topk_final(
    const int32_t* __restrict__ n_entries, int64_t n_max, int k, int slice, int n_slices,
    uint32_t* __restrict__ ws_hist, uint32_t* __restrict__ ws_hist2, const int2* __restrict__ ws_thr,
    uint32_t* __restrict__ ws_ckey, int32_t* __restrict__ ws_cidx, const int32_t* __restrict__ ws_cnt,
    int32_t* __restrict__ ids) {
  __shared__ SelectLds L;
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  uint32_t* gh = ws_hist + b * kHistBins;
  uint32_t* gh2 = ws_hist2 + b * kSubBins;
  const bool take_all = nv <= k;
  int32_t* out = ids + b * k;

  // slice counts (thread t owns slices 8t .. 8t+7), the threshold record and
  // the sub-bin histogram (thread t owns sub-bin 255 - t), loaded together
  constexpr int CPT = kMaxSlices / kTopkThreads;   // 8
  const int32_t* cnt_b = ws_cnt + b * n_slices;
  int c[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int si = CPT * t + j;
    c[j] = si < n_slices ? cnt_b[si] : 0;
  }
  int2 thr = make_int2(0, 0);
  uint32_t h2v = 0u;
  if (!take_all) {
    thr = ws_thr[b];
    h2v = gh2[kSubBins - 1 - t];
  }

  // slice offsets of the candidates
  int mine = 0;
#pragma unroll
  for (int j = 0; j < CPT; ++j) mine += c[j];
  int total;
  int run = block_exclusive_scan(mine, L.scan, total);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int si = CPT * t + j;
    if (si < n_slices) L.pre[si] = run;
    run += c[j];
  }
  if (t == 0) L.pre[n_slices] = total;

  // the sub-bin holding the k-th largest key: sub-bins from the top down
  uint32_t prefix = 0u;
  int rem = 0;
  if (!take_all) {
    const int need = k - thr.y;                  // keys still to take from the threshold bin
    int sub_total;
    const int above2 = block_exclusive_scan((int)h2v, L.scan, sub_total);   // keys in higher sub-bins
    if (above2 < need && need <= above2 + (int)h2v) {
      L.misc[0] = kSubBins - 1 - t;
      L.misc[1] = need - above2;
    }
  }
  __syncthreads();
  if (!take_all) {
    prefix = ((uint32_t)thr.x << kBinShift) | ((uint32_t)L.misc[0] << kLowBits);
    rem = L.misc[1];
  }

  const uint32_t* keys;
  const int32_t* idxs;
  if (total <= kCandCap) {
    // each candidate position's slice, then the gather into LDS
    for (int si = t; si < n_slices; si += kTopkThreads) {
      for (int j = L.pre[si]; j < L.pre[si + 1]; ++j) L.slice_of[j] = (uint16_t)si;
    }
    __syncthreads();
    for (int j0 = 0; j0 < total; j0 += 8 * kTopkThreads) {
      uint32_t kk[8];
      int32_t ii[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kTopkThreads + t;
        kk[u] = 0u;
        ii[u] = 0;
        if (j < total) {
          const int sl = L.slice_of[j];
          const int64_t off = (b * n_slices + sl) * (int64_t)slice + (j - L.pre[sl]);
          kk[u] = ws_ckey[off];
          ii[u] = ws_cidx[off];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kTopkThreads + t;
        if (j < total) {
          L.ckey[j] = kk[u];
          L.cidx[j] = ii[u];
        }
      }
    }
    __syncthreads();
    keys = L.ckey;
    idxs = L.cidx;
  } else {
    // more candidates than LDS holds (heavily tied scores): compact the slices
    // in place in global memory and select there (reads never overtake writes:
    // a slice's destination offset is at most its source offset)
    uint32_t* ck = ws_ckey + b * n_slices * (int64_t)slice;
    int32_t* ci = ws_cidx + b * n_slices * (int64_t)slice;
    for (int s1 = 1; s1 < n_slices; ++s1) {
      const int cs = L.pre[s1 + 1] - L.pre[s1];
      const int64_t from = (int64_t)s1 * slice, to = L.pre[s1];
      for (int j0 = 0; j0 < cs; j0 += kTopkThreads) {
        const int j = j0 + t;
        uint32_t kk = 0u;
        int32_t ii = 0;
        if (j < cs) { kk = ck[from + j]; ii = ci[from + j]; }
        __syncthreads();
        if (j < cs) { ck[to + j] = kk; ci[to + j] = ii; }
        __syncthreads();
      }
    }
    __threadfence_block();
    __syncthreads();
    keys = ck;
    idxs = ci;
  }

  int cnt = 0;
  if (total > 0) {
    if (take_all) {
      cnt = block_emit(keys, total, true, 0u, 0, L.misc, out, k, idxs, 0);
    } else {
      uint32_t T;
      int need_eq;
      radix_select(keys, total, rem, prefix, kLowBits, L.rhist, L.misc, T, need_eq);
      cnt = block_emit(keys, total, false, T, need_eq, L.misc, out, k, idxs, 0);
    }
  }
  for (int i = cnt + t; i < k; i += kTopkThreads) out[i] = -1;

  // leave the histograms clear for the next call
  if (!take_all) {
    for (int i = t; i < kHistBins; i += kTopkThreads) gh[i] = 0u;
    for (int i = t; i < kSubBins; i += kTopkThreads) gh2[i] = 0u;
  }
}

// ------------------------------------------------------------- planning / launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool plan_topk(int64_t B, int64_t n_max, int k, int chunk_hint, TopkPlan* p) {
  (void)k;
  int64_t chunk = chunk_hint;
  if (chunk == 0) {
    // about 1500 scoring workgroups over the batch, chunks of 512 .. 8192 entries
    const int64_t want = (B * n_max + 1535) / 1536;
    chunk = 512;
    while (chunk < want && chunk < 8192) chunk *= 2;
  }
  if (chunk < 256 || chunk > 16384 || chunk % 256 != 0) return false;
  p->chunk = chunk;
  p->n_chunks = n_max <= 0 ? 1 : (n_max + chunk - 1) / chunk;
  int64_t slice = kSliceUnit;
  while ((n_max + slice - 1) / slice > kMaxSlices) slice *= 2;
  if (slice > (int64_t)1 << 24) return false;
  p->slice = slice;
  p->n_slices = n_max <= 0 ? 1 : (n_max + slice - 1) / slice;
  p->key_stride = (n_max + 3) & ~(int64_t)3;
  const size_t nb = (size_t)B;
  size_t off = 0;
  p->off_hist = off; off = align256(off + nb * kHistBins * 4);
  p->off_hist2 = off; off = align256(off + nb * kSubBins * 4);
  p->zero_bytes = off;
  p->off_thr = off; off = align256(off + nb * 8);
  p->off_cnt = off; off = align256(off + nb * (size_t)p->n_slices * 4);
  p->off_keys = off; off = align256(off + nb * (size_t)p->key_stride * 4);
  p->off_ckey = off; off = align256(off + nb * (size_t)p->n_slices * (size_t)slice * 4);
  p->off_cidx = off; off = align256(off + nb * (size_t)p->n_slices * (size_t)slice * 4);
  p->bytes = off;
  return true;
}

template <int DI, bool FP4>
static hipError_t launch_score(const TopkPlan& p, const uint16_t* q_idx, const void* k_idx,
                               const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                               int64_t n_max, uint8_t* ws, hipStream_t stream) {
  const size_t shmem = (size_t)kHistBins * 4 + (size_t)p.chunk * 4;
  auto kern = k_index_score<DI, FP4>;
  if (shmem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)p.n_chunks, (unsigned)B);
  hipLaunchKernelGGL(kern, grid, dim3(kTopkThreads), shmem, stream, q_idx, k_idx, k_scale, n_entries,
                     n_max, (int)p.chunk, p.key_stride, reinterpret_cast<uint32_t*>(ws + p.off_keys),
                     reinterpret_cast<uint32_t*>(ws + p.off_hist));
  return hipGetLastError();
}

hipError_t launch_index_topk(const TopkPlan& p, const uint16_t* q_idx, bool fp4, const void* k_idx,
                             const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                             int64_t n_max, int Di, int k, int32_t* ids, void* workspace,
                             hipStream_t stream) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  hipError_t e = hipSuccess;
  if (n_max > 0) {
    if (fp4) {
      e = Di == 128 ? launch_score<128, true>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, ws, stream)
                    : launch_score<32, true>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, ws, stream);
    } else {
      e = Di == 128 ? launch_score<128, false>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, ws, stream)
                    : launch_score<32, false>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, ws, stream);
    }
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)p.n_slices, (unsigned)B);
  hipLaunchKernelGGL(k_topk_filter, grid, dim3(kTopkThreads), 0, stream,
                     reinterpret_cast<const uint32_t*>(ws + p.off_keys), p.key_stride, n_entries, n_max,
                     k, (int)p.slice, (int)p.n_slices, reinterpret_cast<const uint32_t*>(ws + p.off_hist),
                     reinterpret_cast<uint32_t*>(ws + p.off_hist2), reinterpret_cast<int2*>(ws + p.off_thr),
                     reinterpret_cast<uint32_t*>(ws + p.off_ckey), reinterpret_cast<int32_t*>(ws + p.off_cidx),
                     reinterpret_cast<int32_t*>(ws + p.off_cnt));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk_final, dim3((unsigned)B), dim3(kTopkThreads), 0, stream, n_entries, n_max, k,
                     (int)p.slice, (int)p.n_slices, reinterpret_cast<uint32_t*>(ws + p.off_hist),
                     reinterpret_cast<uint32_t*>(ws + p.off_hist2), reinterpret_cast<const int2*>(ws + p.off_thr),
                     reinterpret_cast<uint32_t*>(ws + p.off_ckey), reinterpret_cast<int32_t*>(ws + p.off_cidx),
                     reinterpret_cast<const int32_t*>(ws + p.off_cnt), ids);
  return hipGetLastError();
}

}  // namespace cskv
