// Indexer scores and exact top-k over c4a entries.
//
// [P1] "c4a (the milder scheme)": DeepSeek Sparse Attention keeps the top-k
// compressed entries per query (default k = 512). [P2] Step 5: a learned
// indexer scores every compressed block; the query reads only the chosen ones.
//
// Two kernels:
//   k_index_score  (grid: chunks x sequences) streams the indexer keys once
//     from HBM with 16-byte coalesced loads (bf16, or fp4 codes + E4M3 group
//     scales dequantised in registers), computes each entry's score as a GEMV
//     against the query's indexer vector and turns it into an order-preserving
//     32-bit key, kept in LDS. It adds the chunk's histogram of the top 12 key
//     bits into a per-sequence histogram with returning atomics. The counts
//     returned (plus the chunk's own) never exceed the final ones, so the bin
//     they place the k-th largest key in is at or below the true one. Each
//     wave keeps the entries of its quarter of the chunk in that bin or above
//     as candidates (key and entry number, in entry order) in a list of its
//     own: together a superset of the chunk's share of the top k.
//   k_topk_final   (grid: sequences, 1024 threads) finds the true threshold
//     bin from the complete histogram and gathers into LDS the candidates at
//     or above it, counting the next 8 key bits of the threshold bin's keys on
//     the way. That fixes the 20-bit prefix of the k-th largest key; the few
//     keys sharing it are ranked against each other (a radix select on the
//     last 12 bits when there are many). It writes the ids in ascending entry
//     order (ties go to the lower entry) and clears the histogram for the next
//     call.
// The selection is exact: every entry of a bin above the threshold bin is in
// the top k, and the threshold bin is resolved on full keys.
#include "kernels.h"

namespace cskv {

constexpr int kTopkThreads = 256;            // scoring workgroups
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kFinalThreads = 1024;          // selection workgroups (one per sequence)
constexpr int kFinalWaves = kFinalThreads / kWave;
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;   // per-sequence histogram of the top key bits
constexpr int kBinShift = 32 - kHistBits;
constexpr int kRadixPad = 257;              // per-wave radix histograms, bank-shifted
constexpr int kCandCap = 8192;              // candidates the final select holds in LDS
constexpr int kMaxChunks = 2048;            // scoring chunks per sequence
constexpr int kMaxLists = kMaxChunks * kTopkWaves;   // candidate lists per sequence (one per chunk and wave)
constexpr int kMisc = 4 + 2 * kFinalWaves;   // block_emit keeps two counts per wave after 4 words
constexpr int kSubBits = 8;                 // key bits below the threshold bin counted while gathering
constexpr int kSubBins = 1 << kSubBits;
constexpr int kLowBits = kBinShift - kSubBits;   // 12 bits below the 20-bit prefix
constexpr int kTieCap = 256;                // keys sharing the k-th key's 20-bit prefix ranked pairwise
constexpr int kTbCap = 2048;                // threshold-bin keys the final select lists apart

// ------------------------------------------------------------- block helpers

// Exclusive prefix sum over the block in thread order; also returns the total.
template <int NT>
__device__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int incl = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  // the waves' totals, scanned across the first NT / 64 lanes
  const int x = lane < NT / kWave ? scratch[lane] : 0;
  const int wincl = wave_inclusive_scan(x);
  total = __shfl(wincl, NT / kWave - 1);
  const int before = wave > 0 ? __shfl(wincl, wave - 1) : 0;
  __syncthreads();
  return before + incl - v;
}

// Radix select on the low `low_bits` bits: among keys[0..n) whose bits above
// `low_bits` equal those of `prefix`, finds the rem-th largest (1 <= rem <=
// their count). Returns the full key T and how many keys equal to T are
// needed. `keys` may be in LDS or global memory; `hist` is LDS.
template <int NT>
__device__ void radix_select(const uint32_t* keys, int n, int rem, uint32_t prefix, int low_bits,
                             uint32_t* hist, int* misc, uint32_t& T_out, int& need_eq_out) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  int hi = low_bits;
  while (hi > 0) {
    const int w = hi < 8 ? hi : 8;
    const int shift = hi - w;
    const uint32_t dmask = (1u << w) - 1u;
    for (int i = t; i < (NT / kWave) * kRadixPad; i += NT) hist[i] = 0u;
    __syncthreads();
    uint32_t* h = hist + wave * kRadixPad;
    for (int i0 = 0; i0 < n; i0 += 4 * NT) {
      uint32_t kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + t;
        kv[u] = i < n ? keys[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * NT + t;
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
        for (int ww = 0; ww < (NT / kWave); ++ww) v += (int)hist[ww * kRadixPad + d];
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
template <int NT>
__device__ int block_emit(const uint32_t* keys, int n, bool all, uint32_t T, int need_eq, int* misc,
                          int32_t* out_idx, int out_cap, const int32_t* idx_map, int32_t idx_base) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int per = (((n + (NT / kWave) - 1) / (NT / kWave)) + kWave - 1) & ~(kWave - 1);
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
    misc[4 + (NT / kWave) + wave] = eq;
  }
  __syncthreads();
  int eq_before = 0, sel_before = 0, total = 0;
  {
    int eb = 0;
#pragma unroll
    for (int w = 0; w < (NT / kWave); ++w) {
      const int e = misc[4 + (NT / kWave) + w];
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

// Entry groups [g_begin, g_end) of a chunk of n entries, a group being the
// 64/LPE consecutive entries one wave-wide load covers; g_end - g_begin is a
// multiple of 4 waves x 8 unrolled groups, or g_end is the chunk's last group.
//
// bf16 keys: LPE = DI/8 lanes read one 16-byte slice each of an entry; one
// wave-wide load covers 64/LPE consecutive entries (1 KiB contiguous).
template <int DI>
__device__ void score_chunk_bf16(const uint16_t* q, const uint16_t* keys_g, int n, int g_begin, int g_end,
                                 uint32_t* keys, uint32_t* hist) {
  constexpr int LPE = DI / 8;
  constexpr int EPL = kWave / LPE;
  constexpr int U = 8;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane / LPE, cg = lane % LPE;
  const uint4 qv = *reinterpret_cast<const uint4*>(q + cg * 8);
  const bf16x2_t q0 = __builtin_bit_cast(bf16x2_t, qv.x), q1 = __builtin_bit_cast(bf16x2_t, qv.y);
  const bf16x2_t q2 = __builtin_bit_cast(bf16x2_t, qv.z), q3 = __builtin_bit_cast(bf16x2_t, qv.w);
  const uint4* kp = reinterpret_cast<const uint4*>(keys_g);
  for (int g0 = g_begin + wave; g0 < g_end; g0 += kTopkWaves * U) {
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
                                int n, int g_begin, int g_end, uint32_t* keys, uint32_t* hist) {
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
  for (int g0 = g_begin + wave; g0 < g_end; g0 += kTopkWaves * U) {
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

constexpr int kBinsPerThread = kHistBins / kTopkThreads;

// The bin of the k-th largest key under the counts hist[0 .. 4096) in LDS, or
// 0 when they hold fewer than k keys, found by one wave alone: lane l sums the
// 64 bins of segment l (bins 4095 - 64l down to 4032 - 64l), a scan over the
// lanes finds the segment where the count from the top reaches k, and a scan
// over that segment's bins finds the bin. Also gives the number of keys in
// the bins above it and in the bin itself (both 0 with bin 0 when fewer than k).
__device__ int wave_threshold_bin(const uint32_t* hist, int k, int& above, int& count) {
  const int lane = lane_id();
  const uint4* seg = reinterpret_cast<const uint4*>(hist + kHistBins - 64 * (lane + 1));
  int s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint4 v = seg[(i + lane) & 15];   // rotated so that lanes spread over the banks
    s += (int)(v.x + v.y + v.z + v.w);
  }
  const int incl = wave_inclusive_scan(s);   // keys in segments 0 .. lane
  const uint64_t m = __ballot(incl - s < k && k <= incl);
  above = 0;
  count = 0;
  if (m == 0) return 0;
  const int L = __ffsll((unsigned long long)m) - 1;
  const int seg_above = __shfl(incl - s, L);
  const int top = kHistBins - 1 - 64 * L;
  const int cnt = (int)hist[top - lane];
  const int incl2 = wave_inclusive_scan(cnt) + seg_above;
  const uint64_t m2 = __ballot(incl2 - cnt < k && k <= incl2);
  const int F = __ffsll((unsigned long long)m2) - 1;
  above = __shfl(incl2 - cnt, F);
  count = __shfl(cnt, F);
  return top - F;
}

template <int DI, bool FP4>
__global__ __launch_bounds__(kTopkThreads) void k_index_score(
    const uint16_t* __restrict__ q_idx, const void* __restrict__ k_idx,
    const uint8_t* __restrict__ k_scale, const int32_t* __restrict__ n_entries, int64_t n_max,
    int chunk, int n_chunks, int k, uint32_t* __restrict__ ws_hist, uint32_t* __restrict__ ws_ckey,
    int32_t* __restrict__ ws_cidx, int32_t* __restrict__ ws_cnt) {
  extern __shared__ __align__(16) uint32_t lds[];
  uint32_t* hist = lds;
  uint32_t* keys = lds + kHistBins;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int64_t b = blockIdx.y;
  const int c = blockIdx.x;
  const int64_t list = ((int64_t)b * n_chunks + c) * kTopkWaves + wave;   // this wave's candidate list
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int64_t start = (int64_t)c * chunk;
  const int64_t rem = nv - start;
  if (rem <= 0) {
    if (lane == 0) ws_cnt[list] = 0;
    return;
  }
  const int n = rem > chunk ? chunk : (int)rem;

  for (int i = t; i < kHistBins; i += kTopkThreads) hist[i] = 0u;
  __syncthreads();
  const uint16_t* q = q_idx + b * DI;
  constexpr int EPL = FP4 ? kWave / (DI / 32) : kWave / (DI / 8);   // entries per wave-wide load
  const int n_groups = (n + EPL - 1) / EPL;
  if constexpr (FP4) {
    const uint8_t* codes = reinterpret_cast<const uint8_t*>(k_idx) + (b * n_max + start) * (DI / 2);
    const uint8_t* scales = k_scale + (b * n_max + start) * (DI / 16);
    score_chunk_fp4<DI>(q, codes, scales, n, 0, n_groups, keys, hist);
  } else {
    const uint16_t* kk = reinterpret_cast<const uint16_t*>(k_idx) + (b * n_max + start) * DI;
    score_chunk_bf16<DI>(q, kk, n, 0, n_groups, keys, hist);
  }
  __syncthreads();

  // Add the chunk histogram into the sequence's. A bin's returned count plus
  // the chunk's own is at most its final count; untouched bins count 0.
  uint32_t* gh = ws_hist + b * kHistBins;
  uint32_t now[kBinsPerThread];
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) {
    const uint32_t h = hist[t + u * kTopkThreads];
    now[u] = h ? atomicAdd(&gh[t + u * kTopkThreads], h) + h : 0u;
  }
#pragma unroll
  for (int u = 0; u < kBinsPerThread; ++u) hist[t + u * kTopkThreads] = now[u];
  __syncthreads();
  int tb_above, tb_count;
  const int tb = wave_threshold_bin(hist, k, tb_above, tb_count);   // at or below the final threshold bin

  // Wave w keeps the entries of its quarter of the chunk at or above that bin,
  // in entry order, in its own list.
  const int quarter = chunk / kTopkWaves;
  const int lo = wave * quarter, hi = min(lo + quarter, n);
  uint32_t* ck = ws_ckey + list * quarter;
  int32_t* ci = ws_cidx + list * quarter;
  int written = 0;
  for (int i0 = lo; i0 < hi; i0 += 4 * kWave) {
    uint32_t kv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kWave + lane;
      kv[u] = i < hi ? keys[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kWave + lane;
      const bool keep = i < hi && (int)(kv[u] >> kBinShift) >= tb;
      const uint64_t m = __ballot(keep);
      if (keep) {
        const int p = written + __popcll(m & lanemask_lt());
        ck[p] = kv[u];
        ci[p] = (int32_t)(start + i);
      }
      written += __popcll(m);
    }
  }
  if (lane == 0) ws_cnt[list] = written;
}

// ------------------------------------------------------------- selection

struct SelectLds {
  alignas(16) uint32_t ckey[kCandCap];
  int32_t cidx[kCandCap];
  uint8_t chosen[kCandCap];      // tie keys taken
  uint32_t rhist[kFinalWaves * kRadixPad];
  uint32_t h2[kSubBins];         // next 8 bits of the threshold bin's keys
  uint32_t tkey[kTieCap];        // keys sharing the k-th key's 20-bit prefix
  int tpos[kTieCap];             // ... and their candidate positions
  uint32_t bkey[kTbCap];         // the threshold bin's keys
  int bpos[kTbCap];              // ... and their candidate positions
  int pre[kMaxLists + 1];
  int misc[kMisc];
  int scan[kFinalWaves];
  int hscan[kFinalWaves];
};

// Writes, in candidate order, the ids of the candidates whose key's top 20
// bits exceed `pstar`, or equal it with `chosen` set (every candidate when
// `all`). Thread t handles one contiguous run of positions. Returns the number
// written (same in all threads).
template <int NT>
__device__ int ordered_emit(const uint32_t* keys, const int32_t* idxs, const uint8_t* chosen, int n, bool all,
                            uint32_t pstar, int* scan, int32_t* out, int out_cap) {
  const int t = threadIdx.x;
  const int per = (n + NT - 1) / NT;
  const int lo = min(t * per, n), hi = min(lo + per, n);
  auto taken = [&](int i) {
    const uint32_t p = keys[i] >> kLowBits;
    return all || p > pstar || (p == pstar && chosen[i]);
  };
  int cnt = 0;
  for (int i = lo; i < hi; ++i) cnt += taken(i) ? 1 : 0;
  int total;
  int pos = block_exclusive_scan<NT>(cnt, scan, total);
  for (int i = lo; i < hi; ++i) {
    if (taken(i)) {
      if (pos < out_cap) out[pos] = idxs[i];
      ++pos;
    }
  }
  return total < out_cap ? total : out_cap;
}

// Sum of per-wave counts cnt[0 .. wave) and of all kFinalWaves of them, by
// a scan over the first kFinalWaves lanes (same result in every lane).
__device__ __forceinline__ int waves_before(const int* cnt, int wave, int& all) {
  const int lane = lane_id();
  const int x = lane < kFinalWaves ? cnt[lane] : 0;
  const int incl = wave_inclusive_scan(x);
  all = __shfl(incl, kFinalWaves - 1);
  return wave > 0 ? __shfl(incl, wave - 1) : 0;
}

// One workgroup per sequence: finds the threshold bin from the complete
// histogram, gathers the candidates of the chunks' lists at or above it,
// resolves the remaining 20 bits on full keys, writes the ids (ascending, -1 padded) and
// clears the histogram for the next call.
__global__ __launch_bounds__(kFinalThreads) void k_topk_final(
    const int32_t* __restrict__ n_entries, int64_t n_max, int k, int list_cap, int n_lists,
    uint32_t* __restrict__ ws_hist, uint32_t* __restrict__ ws_ckey, int32_t* __restrict__ ws_cidx,
    const int32_t* __restrict__ ws_cnt, int32_t* __restrict__ ids) {
  __shared__ SelectLds L;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int64_t b = blockIdx.x;
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  uint32_t* gh = ws_hist + b * kHistBins;
  const bool take_all = nv <= k;
  int32_t* out = ids + b * k;
  if (nv == 0) {   // no entry was scored (the list counts may not even exist)
    for (int i = t; i < k; i += kFinalThreads) out[i] = -1;
    return;
  }

  // list counts (thread t owns lists CPT*t ..) and the histogram (thread t
  // owns bins 4095 - 4t down to 4092 - 4t), loaded together; one pair of
  // barriers serves the offsets of the lists and the threshold bin
  constexpr int CPT = kMaxLists / kFinalThreads;   // 8
  static_assert(kHistBins == 4 * kFinalThreads, "four histogram bins per thread");
  const int32_t* cnt_b = ws_cnt + b * n_lists;
  int c[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int si = CPT * t + j;
    c[j] = si < n_lists ? cnt_b[si] : 0;
  }
  const int top = kHistBins - 1 - 4 * t;
  const uint4 hv = *reinterpret_cast<const uint4*>(gh + top - 3);   // bins top-3 .. top
  for (int i = t; i < kSubBins; i += kFinalThreads) L.h2[i] = 0u;
  if (t == 0) L.misc[5] = 0;                        // threshold-bin list length
  int mine = 0;
#pragma unroll
  for (int j = 0; j < CPT; ++j) mine += c[j];
  const int hs = (int)(hv.x + hv.y + hv.z + hv.w);
  const int incl = wave_inclusive_scan(mine);
  const int hincl = wave_inclusive_scan(hs);
  if (lane == kWave - 1) {
    L.scan[wave] = incl;
    L.hscan[wave] = hincl;
  }
  __syncthreads();
  int total, htotal;
  int run = incl - mine + waves_before(L.scan, wave, total);
  int hrun = hincl - hs + waves_before(L.hscan, wave, htotal);
  // the thread whose bins hold the k-th largest key records the bin, the keys
  // above it and its count
  if (!take_all && hrun < k && k <= hrun + hs) {
    const int hb[4] = {(int)hv.w, (int)hv.z, (int)hv.y, (int)hv.x};   // from the top down
    int r = hrun;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (r < k && k <= r + hb[i]) {
        L.misc[0] = top - i;
        L.misc[1] = r;
        L.misc[2] = hb[i];
      }
      r += hb[i];
    }
  }
  // list offsets of the candidates
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int si = CPT * t + j;
    if (si < n_lists) L.pre[si] = run;
    run += c[j];
  }
  if (t == 0) L.pre[n_lists] = total;
  __syncthreads();
  const int tbin = take_all ? 0 : L.misc[0];
  const int above = take_all ? 0 : L.misc[1];
  const int tcount = take_all ? 0 : L.misc[2];
  // candidates at or above the threshold bin: every key there is one
  const int kept = take_all ? total : above + tcount;

  int cnt = 0;
  if (kept <= kCandCap) {
    // Gather into LDS, in candidate order, the ones at or above the threshold
    // bin, counting the next 8 bits of the threshold bin's keys on the way.
    // Each position's list comes from a search over the list offsets with
    // the same trip count in every lane; the loads follow all the searches.
    // (offsets within the sequence's lists fit 32 bits: at most 2048 chunks
    // of 16384 entries)
    constexpr int PER = 4;
    constexpr int ROUND = PER * kFinalThreads;
    const uint32_t* ck_b = ws_ckey + (int64_t)b * n_lists * list_cap;
    const int32_t* ci_b = ws_cidx + (int64_t)b * n_lists * list_cap;
    int n_sel = 0;
    for (int j0 = 0; j0 < total; j0 += ROUND) {
      int jj[PER], base[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        jj[u] = min(j0 + wave * (PER * kWave) + u * kWave + lane, total - 1);
        base[u] = 0;
      }
      for (int n = n_lists + 1; n > 1;) {
        const int half = n >> 1;
#pragma unroll
        for (int u = 0; u < PER; ++u) base[u] = L.pre[base[u] + half] <= jj[u] ? base[u] + half : base[u];
        n -= half;
      }
      uint32_t kk[PER];
      int32_t ii[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const uint32_t off = (uint32_t)base[u] * (uint32_t)list_cap + (uint32_t)(jj[u] - L.pre[base[u]]);
        kk[u] = ck_b[off];
        ii[u] = ci_b[off];
      }
      bool keep[PER];
      int cw = 0;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const bool valid = j0 + wave * (PER * kWave) + u * kWave + lane < total;
        const int bin = (int)(kk[u] >> kBinShift);
        keep[u] = valid && (take_all || bin >= tbin);
        cw += __popcll(__ballot(keep[u]));
        if (!take_all && valid && bin == tbin) atomicAdd(&L.h2[(kk[u] >> kLowBits) & (kSubBins - 1)], 1u);
      }
      if (lane == 0) L.scan[wave] = cw;
      __syncthreads();
      int round_total;
      int pos = n_sel + waves_before(L.scan, wave, round_total);
      // the threshold bin's keys also go to a list of their own (one slot
      // reservation per wave)
      uint64_t mb[PER];
      int nb_w = 0;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        mb[u] = __ballot(!take_all && keep[u] && (int)(kk[u] >> kBinShift) == tbin);
        nb_w += __popcll(mb[u]);
      }
      int slot = 0;
      if (nb_w > 0) {
        if (lane == 0) slot = atomicAdd(&L.misc[5], nb_w);
        slot = __shfl(slot, 0);
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const uint64_t m = __ballot(keep[u]);
        const int p = pos + __popcll(m & lanemask_lt());
        if (keep[u] && p < kCandCap) {   // (p < kept always holds for a zeroed workspace)
          L.ckey[p] = kk[u];
          L.cidx[p] = ii[u];
        }
        pos += __popcll(m);
        const int sl = slot + __popcll(mb[u] & lanemask_lt());
        if (((mb[u] >> lane) & 1u) && sl < kTbCap) {
          L.bkey[sl] = kk[u];
          L.bpos[sl] = p;
        }
        slot += __popcll(mb[u]);
      }
      n_sel += round_total;
      __syncthreads();
    }
    n_sel = min(n_sel, kCandCap);

    if (take_all) {
      cnt = ordered_emit<kFinalThreads>(L.ckey, L.cidx, L.chosen, n_sel, true, 0u, L.scan, out, k);
    } else {
      // the sub-bin holding the k-th largest key, found by every wave alone:
      // lane l holds sub-bins 255 - 4l .. 252 - 4l, scanned from the top down
      const int need = k - above;                  // keys still to take from the threshold bin
      int hc[4], hs = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hc[j] = (int)L.h2[kSubBins - 1 - 4 * lane - j];
        hs += hc[j];
      }
      int run2 = wave_inclusive_scan(hs) - hs;     // keys in higher sub-bins
      int sb = 0, rem = 0, m = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run2 < need && need <= run2 + hc[j]) {
          sb = kSubBins - 1 - 4 * lane - j;
          rem = need - run2;
          m = hc[j];
        }
        run2 += hc[j];
      }
      const int owner = __ffsll((unsigned long long)__ballot(m > 0 && rem > 0)) - 1;
      sb = __shfl(sb, owner);
      rem = __shfl(rem, owner);                    // keys to take among those sharing the prefix
      m = __shfl(m, owner);                        // keys sharing the prefix
      const uint32_t pstar = ((uint32_t)tbin << kSubBits) | (uint32_t)sb;   // 20-bit prefix
      const int nb = L.misc[5];
      if (m <= kTieCap && nb <= kTbCap) {
        // rank the keys sharing the prefix against each other (descending key,
        // then ascending entry, which candidate order gives)
        if (t == 0) L.misc[3] = 0;                 // tie counter (read after the barrier below)
        __syncthreads();
        for (int i0 = 0; i0 < nb; i0 += kFinalThreads) {   // (one slot reservation per wave)
          const int i = i0 + t;
          const uint32_t key = i < nb ? L.bkey[i] : 0u;
          const bool tie = i < nb && (key >> kLowBits) == pstar;
          const uint64_t mt = __ballot(tie);
          if (mt) {
            int slot = 0;
            if (lane == 0) slot = atomicAdd(&L.misc[3], __popcll(mt));
            slot = __shfl(slot, 0) + __popcll(mt & lanemask_lt());
            if (tie && slot < kTieCap) {   // (there are exactly m of them)
              L.tkey[slot] = key;
              L.tpos[slot] = L.bpos[i];
            }
          }
        }
        __syncthreads();
        if (t < m) {
          const uint32_t key = L.tkey[t];
          const int pos = L.tpos[t];
          int rank = 0;
          for (int s2 = 0; s2 < m; ++s2) {
            const uint32_t ks = L.tkey[s2];
            rank += (ks > key || (ks == key && L.tpos[s2] < pos)) ? 1 : 0;
          }
          if (pos < kCandCap) L.chosen[pos] = rank < rem ? 1 : 0;
        }
        __syncthreads();
        cnt = ordered_emit<kFinalThreads>(L.ckey, L.cidx, L.chosen, n_sel, false, pstar, L.scan, out, k);
      } else {
        uint32_t T;
        int need_eq;
        radix_select<kFinalThreads>(L.ckey, n_sel, rem, pstar << kLowBits, kLowBits, L.rhist, L.misc, T, need_eq);
        cnt = block_emit<kFinalThreads>(L.ckey, n_sel, false, T, need_eq, L.misc, out, k, L.cidx, 0);
      }
    }
  } else {
    // more keys at or above the threshold bin than LDS holds (heavily tied
    // scores): compact the lists in place in global memory and select
    // there (reads never overtake writes: a list's destination offset is at
    // most its source offset)
    uint32_t* ck = ws_ckey + b * n_lists * (int64_t)list_cap;
    int32_t* ci = ws_cidx + b * n_lists * (int64_t)list_cap;
    for (int s1 = 1; s1 < n_lists; ++s1) {
      const int cs = L.pre[s1 + 1] - L.pre[s1];
      const int64_t from = (int64_t)s1 * list_cap, to = L.pre[s1];
      for (int j0 = 0; j0 < cs; j0 += kFinalThreads) {
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
    uint32_t T;
    int need_eq;
    radix_select<kFinalThreads>(ck, total, k - above, (uint32_t)tbin << kBinShift, kBinShift, L.rhist, L.misc, T, need_eq);
    cnt = block_emit<kFinalThreads>(ck, total, false, T, need_eq, L.misc, out, k, ci, 0);
  }
  for (int i = cnt + t; i < k; i += kFinalThreads) out[i] = -1;

  // leave the histogram clear for the next call
  for (int i = t; i < kHistBins; i += kFinalThreads) gh[i] = 0u;
}

// ------------------------------------------------------------- planning / launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool plan_topk(int64_t B, int64_t n_max, int k, int chunk_hint, bool fp4, TopkPlan* p) {
  (void)k;
  int64_t chunk = chunk_hint;
  if (chunk == 0) {
    // bf16 keys (256 B per entry): about 768 scoring workgroups over the batch,
    // chunks of 512 .. 4096 entries; fp4 keys (72 B per entry): about 1536,
    // chunks of 512 .. 8192 (measured best on the c4a workloads); more when a
    // sequence would need more chunks than the final select tracks
    const int64_t groups = fp4 ? 1536 : 768;
    const int64_t cap = fp4 ? 8192 : 4096;
    const int64_t want = (B * n_max + groups - 1) / groups;
    chunk = 512;
    while (chunk < want && chunk < cap) chunk *= 2;
    while ((n_max + chunk - 1) / chunk > kMaxChunks && chunk < 16384) chunk *= 2;
  }
  if (chunk < 256 || chunk > 16384 || chunk % 256 != 0) return false;
  p->chunk = chunk;
  p->n_chunks = n_max <= 0 ? 1 : (n_max + chunk - 1) / chunk;
  if (p->n_chunks > kMaxChunks) return false;
  const size_t nb = (size_t)B;
  const size_t slots = nb * (size_t)p->n_chunks * (size_t)chunk;
  size_t off = 0;
  p->off_hist = off; off = align256(off + nb * kHistBins * 4);
  p->zero_bytes = off;
  p->off_cnt = off; off = align256(off + nb * (size_t)p->n_chunks * kTopkWaves * 4);
  p->off_ckey = off; off = align256(off + slots * 4);
  p->off_cidx = off; off = align256(off + slots * 4);
  p->bytes = off;
  return true;
}

template <int DI, bool FP4>
static hipError_t launch_score(const TopkPlan& p, const uint16_t* q_idx, const void* k_idx,
                               const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                               int64_t n_max, int k, uint8_t* ws, hipStream_t stream) {
  const size_t shmem = (size_t)kHistBins * 4 + (size_t)p.chunk * 4;
  auto kern = k_index_score<DI, FP4>;
  if (shmem > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)p.n_chunks, (unsigned)B);
  hipLaunchKernelGGL(kern, grid, dim3(kTopkThreads), shmem, stream, q_idx, k_idx, k_scale, n_entries,
                     n_max, (int)p.chunk, (int)p.n_chunks, k, reinterpret_cast<uint32_t*>(ws + p.off_hist),
                     reinterpret_cast<uint32_t*>(ws + p.off_ckey), reinterpret_cast<int32_t*>(ws + p.off_cidx),
                     reinterpret_cast<int32_t*>(ws + p.off_cnt));
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
      e = Di == 128 ? launch_score<128, true>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ws, stream)
                    : launch_score<32, true>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ws, stream);
    } else {
      e = Di == 128 ? launch_score<128, false>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ws, stream)
                    : launch_score<32, false>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ws, stream);
    }
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_topk_final, dim3((unsigned)B), dim3(kFinalThreads), 0, stream, n_entries, n_max, k,
                     (int)(p.chunk / kTopkWaves), (int)(p.n_chunks * kTopkWaves),
                     reinterpret_cast<uint32_t*>(ws + p.off_hist),
                     reinterpret_cast<uint32_t*>(ws + p.off_ckey), reinterpret_cast<int32_t*>(ws + p.off_cidx),
                     reinterpret_cast<const int32_t*>(ws + p.off_cnt), ids);
  return hipGetLastError();
}

}  // namespace cskv
