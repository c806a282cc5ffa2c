// Indexer scores and exact top-k over c4a entries.
//
// [P1] "c4a (the milder scheme)": DeepSeek Sparse Attention keeps the top-k
// compressed entries per query (default k = 512). [P2] Step 5: a learned
// indexer scores every compressed block; the query reads only the chosen ones.
//
// One launch, k_index_topk (grid: chunks x sequences, 1024 threads; one
// dimension with a sequence's chunks on one XCD when the batch is a multiple
// of 8):
//   Scoring. Each workgroup streams one chunk of a sequence's indexer keys
//     once from HBM with 16-byte non-temporal loads (bf16, or fp4 codes +
//     E4M3 group scales dequantised in registers), computes each entry's
//     score as a GEMV against the query's indexer vector and turns it into an
//     order-preserving 32-bit key, kept in LDS. It adds the chunk's histogram
//     of the top 12 key bits into the sequence's histogram with returning
//     atomics. The counts returned (plus the chunk's own) never exceed the
//     final ones, so the bin they place the k-th largest key in is at or below
//     the true one. The chunk's entries in that bin or above are written, in
//     entry order, to the chunk's candidate list: a superset of the chunk's
//     share of the top k.
//   Arrival. The lists and counts are stored with agent-scope atomics; once
//     every wave's stores have completed, one thread counts the chunk in on the
//     sequence's arrival counter. The workgroup that counts last knows every
//     chunk of its sequence is done; it reads their results with agent-scope
//     atomic loads and finishes the selection while the other sequences are
//     still being scored.
//   Selection. From the complete histogram it finds the true threshold bin
//     and gathers the candidates at or above it, in entry order, into
//     registers (a few per thread; LDS or global memory when there are more),
//     listing the threshold bin's keys in LDS, which fixes the 20-bit prefix
//     of the k-th largest key; the few keys sharing it are ranked against each
//     other (a radix select on the last 12 bits when there are many). One
//     block scan places every id in ascending entry order (ties go to the
//     lower entry); the histogram and the counter are cleared for the next
//     call.
// The selection is exact: every entry of a bin above the threshold bin is in
// the top k, and the threshold bin is resolved on full keys.
#include "kernels.h"

namespace cskv {

constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;   // per-sequence histogram of the top key bits
constexpr int kBinShift = 32 - kHistBits;
constexpr int kRadixPad = 257;              // per-wave radix histograms, bank-shifted
constexpr int kMaxChunks = 2048;            // scoring chunks (candidate lists) per sequence
constexpr int kSubBits = 8;                 // key bits below the threshold bin counted while gathering
constexpr int kSubBins = 1 << kSubBits;
constexpr int kLowBits = kBinShift - kSubBits;   // 12 bits below the 20-bit prefix
constexpr int kTieCap = 256;                // keys sharing the k-th key's 20-bit prefix ranked pairwise
constexpr int kTbCap = 1024;                // threshold-bin keys the selection lists apart
constexpr int kMisc = 40;                   // block_emit keeps two counts per wave after 4 words
// Workgroup size (scoring and selection). With 1024 threads and about one
// workgroup per compute unit every CU streams keys with 16 waves, and the
// selection that ends each sequence runs with 16 waves too (measured on the
// c4a 128K / 1M workloads: 59 / 48 us per call against 67 / 62 us with 256
// threads and three times the workgroups).
constexpr int kTopkThreads = 1024;
// Scoring workgroups when the selection runs as a launch of its own.
constexpr int kTopkScoreThreads = 256;
constexpr bool kTopkFused = true;
// candidate positions per thread and gather round of the selection
template <int NT>
constexpr int gather_per() { return NT >= 1024 ? 4 : 16; }

// Data that one workgroup hands to another within the launch (candidate
// lists, their counts, the histogram read back by the selection) is written
// and read with relaxed agent-scope atomics: gfx950 performs them at the
// device's coherence point, so no workgroup needs an agent-scope fence (which
// writes back and invalidates the whole L2 and costs far more than the data).
template <typename T>
__device__ __forceinline__ void put_shared(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T get_shared(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A selection in a launch of its own reads what the scoring launch wrote with
// plain loads (the launch boundary orders them); inside the scoring launch it
// reads through to the coherence point.
template <bool COH, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (COH) return get_shared(p);
  else return *p;
}

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
  total = lane_value(wincl, NT / kWave - 1);
  const int before = wave > 0 ? lane_value(wincl, wave - 1) : 0;
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
// multiple of NW waves x 8 unrolled groups, or g_end is the chunk's last group.
//
// bf16 keys: LPE = DI/8 lanes read one 16-byte slice each of an entry; one
// wave-wide load covers 64/LPE consecutive entries (1 KiB contiguous).
template <int DI, int NW>
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
  for (int g0 = g_begin + wave; g0 < g_end; g0 += NW * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = (g0 + NW * u) * EPL + sub;
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
      const int e = (g0 + NW * u) * EPL + sub;
      if (cg == 0 && e < n) put_key(keys, hist, e, p);
    }
  }
}

// fp4 keys: each lane reads 16 code bytes (32 channels = two 16-channel groups)
// and the two matching E4M3 group scales; LPE = DI/32 lanes per entry. The
// E2M1 codes are widened to bf16 exactly by the gfx950 converter.
template <int DI, int NW>
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
  for (int g0 = g_begin + wave; g0 < g_end; g0 += NW * U) {
    uint4 v[U];
    uint32_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = (g0 + NW * u) * EPL + sub;
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
      // the two E4M3 group scales, exactly, through the hardware converter
      // (byte 0 -> low half, byte 1 -> high half of a bf16 pair)
      const uint32_t sb = fp8x2_to_bf16x2<false>(s[u] & 0xFFFFu);
      float p = fmaf(g1s, __uint_as_float(sb & 0xFFFF0000u), g0s * __uint_as_float(sb << 16));
      if constexpr (LPE == 4) p = sum_quad(p);
      const int e = (g0 + NW * u) * EPL + sub;
      if (part == 0 && e < n) put_key(keys, hist, e, p);
    }
  }
}


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
  const int seg_above = lane_value(incl - s, L);
  const int top = kHistBins - 1 - 64 * L;
  const int cnt = (int)hist[top - lane];
  const int incl2 = wave_inclusive_scan(cnt) + seg_above;
  const uint64_t m2 = __ballot(incl2 - cnt < k && k <= incl2);
  const int F = __ffsll((unsigned long long)m2) - 1;
  above = lane_value(incl2 - cnt, F);
  count = lane_value(cnt, F);
  return top - F;
}

// ------------------------------------------------------------- selection

// Word offsets of the selection's arrays in the workgroup's dynamic LDS (the
// scoring arrays are dead by then). `cap` candidates at or above the
// threshold bin are gathered; `n_lists` candidate lists are offset.
struct SelectView {
  uint32_t* ckey;     // candidate keys, in entry order
  int32_t* cidx;      // ... and their entries
  uint32_t* rhist;    // one radix histogram of kRadixPad words per wave
  uint32_t* h2;       // next 8 bits of the threshold bin's keys
  uint32_t* tkey;     // keys sharing the k-th key's 20-bit prefix
  int* tpos;          // ... and their candidate positions
  uint32_t* bkey;     // the threshold bin's keys
  int* bpos;          // ... and their candidate positions
  int* misc;
  int* scan;
  int* hscan;
  int* pre;           // list offsets (n_lists + 1)
  uint8_t* chosen;    // tie keys taken
};

__host__ __device__ inline size_t select_lds_words(int cap, int tbcap, int n_lists, int nw) {
  return 2 * (size_t)cap + (size_t)nw * kRadixPad + kSubBins + 2 * kTieCap + 2 * (size_t)tbcap + kMisc +
         2 * (size_t)nw + (size_t)n_lists + 1 + ((size_t)cap + 3) / 4;
}

__device__ inline SelectView select_view(uint32_t* lds, int cap, int tbcap, int n_lists, int nw) {
  SelectView v;
  uint32_t* p = lds;
  v.ckey = p; p += cap;
  v.cidx = reinterpret_cast<int32_t*>(p); p += cap;
  v.rhist = p; p += nw * kRadixPad;
  v.h2 = p; p += kSubBins;
  v.tkey = p; p += kTieCap;
  v.tpos = reinterpret_cast<int*>(p); p += kTieCap;
  v.bkey = p; p += tbcap;
  v.bpos = reinterpret_cast<int*>(p); p += tbcap;
  v.misc = reinterpret_cast<int*>(p); p += kMisc;
  v.scan = reinterpret_cast<int*>(p); p += nw;
  v.hscan = reinterpret_cast<int*>(p); p += nw;
  v.pre = reinterpret_cast<int*>(p); p += n_lists + 1;
  v.chosen = reinterpret_cast<uint8_t*>(p);
  return v;
}

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

// Sum of per-wave counts cnt[0 .. wave) and of all NW of them, by a scan over
// the first NW lanes (same result in every lane).
template <int NW>
__device__ __forceinline__ int waves_before(const int* cnt, int wave, int& all) {
  const int lane = lane_id();
  const int x = lane < NW ? cnt[lane] : 0;
  const int incl = wave_inclusive_scan(x);
  all = lane_value(incl, NW - 1);
  return wave > 0 ? lane_value(incl, wave - 1) : 0;
}

// The common case of the selection, with the candidates kept in registers.
// After the list counts and the histogram (one round trip, done by the
// caller into L.pre and misc), thread t loads the PER consecutive candidate
// positions t*PER .. (one search over the list offsets finds the list of the
// first, later ones walk forward): threads in order hold the candidates in
// entry order. The threshold bin's keys are listed in LDS to find the 20-bit
// prefix of the k-th largest key and to rank the keys that share it (by key,
// then entry); one block scan over the per-thread selected counts then places
// every id. Returns false, before writing any id, when there are more
// candidates than PER * NT or the threshold bin or its ties exceed what LDS
// lists; the general path then runs. On success `cnt` is the number of ids
// written.
template <int NT, bool COH>
__device__ __forceinline__ bool select_registers(bool take_all, int k, int total, int tbin, int above,
                                                 int n_lists, int list_cap, int tbcap,
                                                 const uint32_t* __restrict__ ck_b, const int32_t* __restrict__ ci_b,
                                                 int32_t* __restrict__ out, const SelectView& L, int& cnt) {
  constexpr int PER = gather_per<NT>();
  const int t = threadIdx.x, lane = t % kWave;
  if (total > PER * NT) return false;
  const int p0 = t * PER;
  uint32_t kk[PER];
  int32_t ii[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    kk[u] = 0u;
    ii[u] = 0;
  }
  if (p0 < total) {
    int lst = 0;   // the largest list whose offset is <= p0
    for (int n = n_lists + 1; n > 1;) {
      const int half = n >> 1;
      lst = L.pre[lst + half] <= p0 ? lst + half : lst;
      n -= half;
    }
    int cur = L.pre[lst], next = L.pre[lst + 1];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int pp = p0 + u;
      if (pp < total) {
        while (pp >= next) {   // (ends: pre[n_lists] = total > pp)
          ++lst;
          cur = next;
          next = L.pre[lst + 1];
        }
        const int64_t off = (int64_t)lst * list_cap + (pp - cur);
        kk[u] = ld<COH>(ck_b + off);
        ii[u] = ld<COH>(ci_b + off);
      }
    }
  }
  // classify: above the threshold bin (taken), in it (listed apart), below
  uint32_t gtm = 0u, tbm = 0u;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const bool valid = p0 + u < total;
    const int bin = (int)(kk[u] >> kBinShift);
    const bool gt = valid && (take_all || bin > tbin);
    const bool tb = valid && !take_all && bin == tbin;
    gtm |= (gt ? 1u : 0u) << u;
    tbm |= (tb ? 1u : 0u) << u;
    if (tb) atomicAdd(&L.h2[(kk[u] >> kLowBits) & (kSubBins - 1)], 1u);
  }
  // the threshold bin's keys, listed apart: one slot reservation per wave
  const int ntb = __popc(tbm);
  const int wincl = wave_inclusive_scan(ntb);
  int slot = 0;
  if (lane == kWave - 1 && wincl > 0) slot = atomicAdd(&L.misc[5], wincl);
  slot = lane_value(slot, kWave - 1) + wincl - ntb;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if ((tbm >> u) & 1u) {
      if (slot < tbcap) {
        L.bkey[slot] = kk[u];
        L.bpos[slot] = ii[u];
      }
      ++slot;
    }
  }
  __syncthreads();

  uint32_t pstar = 0u;
  int rem = 0, m = 0;
  if (!take_all) {
    const int nb = L.misc[5];
    if (nb > tbcap) return false;
    // the sub-bin of the k-th largest key, found by every wave alone: lane l
    // holds sub-bins 255 - 4l .. 252 - 4l, scanned from the top down
    const int need = k - above;
    int hc[4], hsub = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hc[j] = (int)L.h2[kSubBins - 1 - 4 * lane - j];
      hsub += hc[j];
    }
    int run2 = wave_inclusive_scan(hsub) - hsub;
    int sb = 0;
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
    sb = lane_value(sb, owner);
    rem = lane_value(rem, owner);   // keys to take among those sharing the prefix
    m = lane_value(m, owner);       // keys sharing the prefix
    if (m > kTieCap) return false;
    pstar = ((uint32_t)tbin << kSubBits) | (uint32_t)sb;
    // the keys sharing the prefix, with their entries
    for (int i0 = 0; i0 < nb; i0 += NT) {
      const int i = i0 + t;
      const uint32_t key = i < nb ? L.bkey[i] : 0u;
      const bool tie = i < nb && (key >> kLowBits) == pstar;
      const uint64_t mt = __ballot(tie);
      if (mt) {
        int s2 = 0;
        if (lane == 0) s2 = atomicAdd(&L.misc[3], __popcll(mt));
        s2 = lane_value(s2, 0) + __popcll(mt & lanemask_lt());
        if (tie && s2 < kTieCap) {
          L.tkey[s2] = key;
          L.tpos[s2] = L.bpos[i];
        }
      }
    }
    __syncthreads();
  }

  // selected: above the threshold bin, or in it with a higher 20-bit prefix,
  // or sharing the prefix and ranked among the first rem (key, then entry)
  uint32_t selm = gtm;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if ((tbm >> u) & 1u) {
      const uint32_t pfx = kk[u] >> kLowBits;
      bool take = pfx > pstar;
      if (pfx == pstar) {
        int rank = 0;
        for (int s2 = 0; s2 < m; ++s2) {
          const uint32_t ks = L.tkey[s2];
          rank += (ks > kk[u] || (ks == kk[u] && L.tpos[s2] < ii[u])) ? 1 : 0;
        }
        take = rank < rem;
      }
      selm |= (take ? 1u : 0u) << u;
    }
  }
  int n_out;
  int pos = block_exclusive_scan<NT>(__popc(selm), L.scan, n_out);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    if ((selm >> u) & 1u) {
      if (pos < k) out[pos] = ii[u];
      ++pos;
    }
  }
  cnt = n_out < k ? n_out : k;
  return true;
}

// The selection of sequence b by the workgroup that scored its last chunk:
// finds the threshold bin from the complete histogram, gathers the
// candidates of the chunks' lists at or above it, resolves the remaining 20
// bits on full keys, writes the ids (ascending, -1 padded), then clears the
// histogram and the arrival counter for the next call.
template <int NT, bool COH>
__device__ __forceinline__ void select_sequence(int64_t nv, int k, int n_lists, int list_cap, int cap, int tbcap,
                                                uint32_t* __restrict__ gh, uint32_t* __restrict__ arrive,
                                                uint32_t* __restrict__ ck_b, int32_t* __restrict__ ci_b,
                                                const int32_t* __restrict__ cnt_b, int32_t* __restrict__ out,
                                                uint32_t* lds) {
  constexpr int NW = NT / kWave;
  constexpr int LPT = kMaxChunks / NT;        // lists per thread
  constexpr int BPT = kHistBins / NT;         // histogram bins per thread
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const SelectView L = select_view(lds, cap, tbcap, n_lists, NW);
  const bool take_all = nv <= k;
  if (nv == 0) {   // no entry was scored: no histogram counts to clear
    for (int i = t; i < k; i += NT) out[i] = -1;
    if (t == 0) *arrive = 0u;
    return;
  }

  // list counts (thread t owns lists LPT * t ..) and the histogram (thread t
  // owns bins 4095 - BPT t down to 4096 - BPT (t + 1)), loaded together; one
  // pair of barriers serves the offsets of the lists and the threshold bin
  int c[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int si = LPT * t + j;
    c[j] = si < n_lists ? ld<COH>(cnt_b + si) : 0;
  }
  const int top = kHistBins - 1 - BPT * t;
  int hb[BPT];   // hb[j]: bin top - j
#pragma unroll
  for (int j = 0; j < BPT; ++j) hb[j] = (int)ld<COH>(gh + top - j);
  for (int i = t; i < kSubBins; i += NT) L.h2[i] = 0u;
  if (t == 0) {
    L.misc[3] = 0;                                  // tie list length (register path)
    L.misc[5] = 0;                                  // threshold-bin list length
  }
  int mine = 0, hs = 0;
#pragma unroll
  for (int j = 0; j < LPT; ++j) mine += c[j];
#pragma unroll
  for (int j = 0; j < BPT; ++j) hs += hb[j];
  const int incl = wave_inclusive_scan(mine);
  const int hincl = wave_inclusive_scan(hs);
  if (lane == kWave - 1) {
    L.scan[wave] = incl;
    L.hscan[wave] = hincl;
  }
  __syncthreads();
  int total, htotal;
  int run = incl - mine + waves_before<NW>(L.scan, wave, total);
  const int hrun = hincl - hs + waves_before<NW>(L.hscan, wave, htotal);
  // the thread whose bins hold the k-th largest key records the bin, the keys
  // above it and its count
  if (!take_all && hrun < k && k <= hrun + hs) {
    int r = hrun;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
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
  for (int j = 0; j < LPT; ++j) {
    const int si = LPT * t + j;
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
  if (select_registers<NT, COH>(take_all, k, total, tbin, above, n_lists, list_cap, tbcap, ck_b, ci_b, out, L, cnt)) {
    // done
  } else if (kept <= cap) {
    // the general path reuses the LDS the register path may have filled
    __syncthreads();
    for (int i = t; i < kSubBins; i += NT) L.h2[i] = 0u;
    if (t == 0) L.misc[5] = 0;
    __syncthreads();
    // Gather into LDS, in candidate order, the ones at or above the threshold
    // bin, counting the next 8 bits of the threshold bin's keys on the way.
    // Thread t takes PER consecutive positions per round: one search over the
    // list offsets finds the list of the first, later ones walk forward, and
    // every load is issued before any is used. A block scan of the per-thread
    // counts places the kept ones. (Offsets within the sequence's lists fit
    // 32 bits: at most 2048 chunks of 16384 entries.)
    constexpr int PER = gather_per<NT>();
    constexpr int ROUND = PER * NT;
    int n_sel = 0;
    for (int j0 = 0; j0 < total; j0 += ROUND) {
      const int p0 = j0 + t * PER;
      uint32_t kk[PER];
      int32_t ii[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        kk[u] = 0u;
        ii[u] = 0;
      }
      if (p0 < total) {
        int lst = 0;   // the largest list whose offset is <= p0
        for (int n = n_lists + 1; n > 1;) {
          const int half = n >> 1;
          lst = L.pre[lst + half] <= p0 ? lst + half : lst;
          n -= half;
        }
        int cur = L.pre[lst], next = L.pre[lst + 1];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
          const int pp = p0 + u;
          if (pp < total) {
            while (pp >= next) {   // (ends: pre[n_lists] = total > pp)
              ++lst;
              cur = next;
              next = L.pre[lst + 1];
            }
            const uint32_t off = 4u * ((uint32_t)lst * (uint32_t)list_cap + (uint32_t)(pp - cur));
            kk[u] = get_shared(reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(ck_b) + off));
            ii[u] = get_shared(reinterpret_cast<const int32_t*>(reinterpret_cast<const uint8_t*>(ci_b) + off));
          }
        }
      }
      uint32_t keepm = 0u, tbm = 0u;   // bit u: position p0 + u is kept / in the threshold bin
      int nk = 0;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const bool valid = p0 + u < total;
        const int bin = (int)(kk[u] >> kBinShift);
        const bool keep = valid && (take_all || bin >= tbin);
        const bool tb = !take_all && valid && bin == tbin;
        keepm |= (keep ? 1u : 0u) << u;
        tbm |= (tb ? 1u : 0u) << u;
        nk += keep ? 1 : 0;
        if (tb) atomicAdd(&L.h2[(kk[u] >> kLowBits) & (kSubBins - 1)], 1u);
      }
      int round_total;
      int pos = n_sel + block_exclusive_scan<NT>(nk, L.scan, round_total);
      const int ntb = __popc(tbm);
      int slot = ntb ? atomicAdd(&L.misc[5], ntb) : 0;   // the threshold bin's keys, listed apart
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        if ((keepm >> u) & 1u) {
          if (pos < cap) {   // (pos < kept always holds for a zeroed workspace)
            L.ckey[pos] = kk[u];
            L.cidx[pos] = ii[u];
          }
          if ((tbm >> u) & 1u) {
            if (slot < tbcap) {
              L.bkey[slot] = kk[u];
              L.bpos[slot] = pos;
            }
            ++slot;
          }
          ++pos;
        }
      }
      n_sel += round_total;
      __syncthreads();
    }
    n_sel = min(n_sel, cap);

    if (take_all) {
      cnt = ordered_emit<NT>(L.ckey, L.cidx, L.chosen, n_sel, true, 0u, L.scan, out, k);
    } else {
      // the sub-bin holding the k-th largest key, found by every wave alone:
      // lane l holds sub-bins 255 - 4l .. 252 - 4l, scanned from the top down
      const int need = k - above;                  // keys still to take from the threshold bin
      int hc[4], hsub = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hc[j] = (int)L.h2[kSubBins - 1 - 4 * lane - j];
        hsub += hc[j];
      }
      int run2 = wave_inclusive_scan(hsub) - hsub;   // keys in higher sub-bins
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
      sb = lane_value(sb, owner);
      rem = lane_value(rem, owner);                    // keys to take among those sharing the prefix
      m = lane_value(m, owner);                        // keys sharing the prefix
      const uint32_t pstar = ((uint32_t)tbin << kSubBits) | (uint32_t)sb;   // 20-bit prefix
      const int nb = L.misc[5];
      if (m <= kTieCap && nb <= tbcap) {
        // rank the keys sharing the prefix against each other (descending key,
        // then ascending entry, which candidate order gives)
        if (t == 0) L.misc[3] = 0;                 // tie counter (read after the barrier below)
        __syncthreads();
        for (int i0 = 0; i0 < nb; i0 += NT) {      // (one slot reservation per wave)
          const int i = i0 + t;
          const uint32_t key = i < nb ? L.bkey[i] : 0u;
          const bool tie = i < nb && (key >> kLowBits) == pstar;
          const uint64_t mt = __ballot(tie);
          if (mt) {
            int slot2 = 0;
            if (lane == 0) slot2 = atomicAdd(&L.misc[3], __popcll(mt));
            slot2 = lane_value(slot2, 0) + __popcll(mt & lanemask_lt());
            if (tie && slot2 < kTieCap) {   // (there are exactly m of them)
              L.tkey[slot2] = key;
              L.tpos[slot2] = L.bpos[i];
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
          if (pos < cap) L.chosen[pos] = rank < rem ? 1 : 0;
        }
        __syncthreads();
        cnt = ordered_emit<NT>(L.ckey, L.cidx, L.chosen, n_sel, false, pstar, L.scan, out, k);
      } else {
        uint32_t T;
        int need_eq;
        radix_select<NT>(L.ckey, n_sel, rem, pstar << kLowBits, kLowBits, L.rhist, L.misc, T, need_eq);
        cnt = block_emit<NT>(L.ckey, n_sel, false, T, need_eq, L.misc, out, k, L.cidx, 0);
      }
    }
  } else {
    // more keys at or above the threshold bin than LDS holds (heavily tied
    // scores): compact the lists in place in global memory and select
    // there (reads never overtake writes: a list's destination offset is at
    // most its source offset; the lists of other workgroups are read through
    // to the coherence point, the compacted copy is this workgroup's own)
    for (int s1 = 1; s1 < n_lists; ++s1) {
      const int cs = L.pre[s1 + 1] - L.pre[s1];
      const int64_t from = (int64_t)s1 * list_cap, to = L.pre[s1];
      for (int j0 = 0; j0 < cs; j0 += NT) {
        const int j = j0 + t;
        uint32_t kk = 0u;
        int32_t ii = 0;
        if (j < cs) { kk = ld<COH>(ck_b + from + j); ii = ld<COH>(ci_b + from + j); }
        __syncthreads();
        if (j < cs) { ck_b[to + j] = kk; ci_b[to + j] = ii; }
        __syncthreads();
      }
    }
    __threadfence_block();
    __syncthreads();
    uint32_t T;
    int need_eq;
    radix_select<NT>(ck_b, total, k - above, (uint32_t)tbin << kBinShift, kBinShift, L.rhist, L.misc, T, need_eq);
    cnt = block_emit<NT>(ck_b, total, false, T, need_eq, L.misc, out, k, ci_b, 0);
  }
  for (int i = cnt + t; i < k; i += NT) out[i] = -1;

  // leave the histogram and the arrival counter clear for the next call
  for (int i = t; i < kHistBins; i += NT) gh[i] = 0u;
  if (t == 0) *arrive = 0u;
}

// ------------------------------------------------------------- the launch

template <int DI, bool FP4, int NT, bool FUSED>
__global__ __launch_bounds__(NT) void k_index_topk(
    const uint16_t* __restrict__ q_idx, const void* __restrict__ k_idx,
    const uint8_t* __restrict__ k_scale, const int32_t* __restrict__ n_entries, int64_t n_max,
    int chunk, int n_chunks, int k, int cand_cap, int tb_cap, uint32_t* __restrict__ ws_hist,
    uint32_t* __restrict__ ws_arrive, uint32_t* __restrict__ ws_ckey, int32_t* __restrict__ ws_cidx,
    int32_t* __restrict__ ws_cnt, int32_t* __restrict__ ids, int xcd) {
  constexpr int NW = NT / kWave;
  constexpr int BPT = kHistBins / NT;
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ int wcnt_l[NW];
  __shared__ int last_l, tb_l;
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  // workgroup -> (sequence, chunk). With `xcd` (a 1-D grid, the batch a
  // multiple of 8) a sequence's chunks get ids equal mod 8, and workgroups are
  // dealt to the 8 XCDs by id mod 8, so they run on one XCD: the sequence's
  // query and histogram lines stay in one L2, and its selection starts on the
  // XCD that scored its chunks.
  int64_t b;
  int c;
  if (xcd) {
    const int r = blockIdx.x >> 3;
    b = (int64_t)(r / n_chunks) * 8 + (blockIdx.x & 7);
    c = r % n_chunks;
  } else {
    b = blockIdx.y;
    c = blockIdx.x;
  }
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int64_t start = (int64_t)c * chunk;
  const int64_t rem = nv - start;
  uint32_t* ck = ws_ckey + ((int64_t)b * n_chunks + c) * chunk;   // this chunk's candidate list
  int32_t* ci = ws_cidx + ((int64_t)b * n_chunks + c) * chunk;
  uint32_t* gh = ws_hist + b * kHistBins;

  if (rem > 0) {
    const int n = rem > chunk ? chunk : (int)rem;
    uint32_t* hist = lds;
    uint32_t* keys = lds + kHistBins;
    for (int i = t; i < kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
    const uint16_t* q = q_idx + b * DI;
    constexpr int EPL = FP4 ? kWave / (DI / 32) : kWave / (DI / 8);   // entries per wave-wide load
    const int n_groups = (n + EPL - 1) / EPL;
    if constexpr (FP4) {
      const uint8_t* codes = reinterpret_cast<const uint8_t*>(k_idx) + (b * n_max + start) * (DI / 2);
      const uint8_t* scales = k_scale + (b * n_max + start) * (DI / 16);
      score_chunk_fp4<DI, NW>(q, codes, scales, n, 0, n_groups, keys, hist);
    } else {
      const uint16_t* kk = reinterpret_cast<const uint16_t*>(k_idx) + (b * n_max + start) * DI;
      score_chunk_bf16<DI, NW>(q, kk, n, 0, n_groups, keys, hist);
    }
    __syncthreads();

    // Add the chunk histogram into the sequence's. A bin's returned count plus
    // the chunk's own is at most its final count; untouched bins count 0.
    // (all of a thread's returning atomics are in flight at once)
    uint32_t hv[BPT], now[BPT];
#pragma unroll
    for (int u = 0; u < BPT; ++u) hv[u] = hist[t + u * NT];
#pragma unroll
    for (int u = 0; u < BPT; ++u) now[u] = hv[u] ? atomicAdd(&gh[t + u * NT], hv[u]) : 0u;
#pragma unroll
    for (int u = 0; u < BPT; ++u) hist[t + u * NT] = hv[u] ? now[u] + hv[u] : 0u;
    __syncthreads();
    // the bin at or below the final threshold bin: found by wave 0 alone (16
    // waves reading the whole histogram would queue 256 KiB of LDS reads)
    if (wave == 0) {
      int tb_above, tb_count;
      const int tb0 = wave_threshold_bin(hist, k, tb_above, tb_count);
      if (lane == 0) tb_l = tb0;
    }
    __syncthreads();
    const int tb = tb_l;

    // The chunk's entries at or above that bin go to its list in entry order:
    // wave w counts those of its share of the chunk, then writes them after
    // the lower shares' ones.
    const int share = chunk / NW;
    const int lo = wave * share, hi = min(lo + share, n);
    auto kept = [&](int i, uint32_t& kv) __attribute__((always_inline)) {
      kv = i < hi ? keys[i] : 0u;
      return i < hi && (int)(kv >> kBinShift) >= tb;
    };
    int mine = 0;
    for (int i0 = lo; i0 < hi; i0 += 4 * kWave) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t kv;
        mine += __popcll(__ballot(kept(i0 + u * kWave + lane, kv)));
      }
    }
    if (lane == 0) wcnt_l[wave] = mine;
    __syncthreads();
    int written = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      written += w < wave ? wcnt_l[w] : 0;
      total += wcnt_l[w];
    }
    for (int i0 = lo; i0 < hi; i0 += 4 * kWave) {
      uint32_t kv[4];
      bool keep[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) keep[u] = kept(i0 + u * kWave + lane, kv[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint64_t m = __ballot(keep[u]);
        if (keep[u]) {
          const int p = written + __popcll(m & lanemask_lt());
          if constexpr (FUSED) {
            put_shared(ck + p, kv[u]);
            put_shared(ci + p, (int32_t)(start + i0 + u * kWave + lane));
          } else {
            ck[p] = kv[u];
            ci[p] = (int32_t)(start + i0 + u * kWave + lane);
          }
        }
        written += __popcll(m);
      }
    }
    if (t == 0) put_shared(ws_cnt + b * n_chunks + c, total);
  } else if (t == 0) {
    put_shared(ws_cnt + b * n_chunks + c, 0);
  }
  if constexpr (!FUSED) return;   // the selection runs in a launch of its own

  // Arrival: every wave waits until its list stores and histogram atomics
  // have completed at the coherence point, then the chunk counts in; the
  // workgroup that counts the sequence's last chunk reads every chunk's
  // results through to that point and runs the selection.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (t == 0) {
    const uint32_t before = __hip_atomic_fetch_add(ws_arrive + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_l = before == (uint32_t)(n_chunks - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!last_l) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  select_sequence<NT, true>(nv, k, n_chunks, chunk, cand_cap, tb_cap, gh, ws_arrive + b,
                      ws_ckey + (int64_t)b * n_chunks * chunk, ws_cidx + (int64_t)b * n_chunks * chunk,
                      ws_cnt + b * n_chunks, ids + b * k, lds);
}

// The selection as a launch of its own (grid: sequences), after a scoring
// launch that only wrote the candidate lists and the histogram.
template <int NT>
__global__ __launch_bounds__(NT) void k_topk_select(const int32_t* __restrict__ n_entries, int64_t n_max, int k,
                                                   int chunk, int n_chunks, int cand_cap, int tb_cap,
                                                   uint32_t* __restrict__ ws_hist, uint32_t* __restrict__ ws_arrive,
                                                   uint32_t* __restrict__ ws_ckey, int32_t* __restrict__ ws_cidx,
                                                   const int32_t* __restrict__ ws_cnt, int32_t* __restrict__ ids) {
  extern __shared__ __align__(16) uint32_t lds[];
  const int64_t b = blockIdx.x;
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  select_sequence<NT, false>(nv, k, n_chunks, chunk, cand_cap, tb_cap, ws_hist + b * kHistBins, ws_arrive + b,
                             ws_ckey + (int64_t)b * n_chunks * chunk, ws_cidx + (int64_t)b * n_chunks * chunk,
                             ws_cnt + b * n_chunks, ids + b * k, lds);
}

// ------------------------------------------------------------- planning / launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool plan_topk(int64_t B, int64_t n_max, int k, int chunk_hint, bool fp4, TopkPlan* p) {
  // Workgroups of 1024 threads, about one per compute unit: every CU streams
  // with 16 waves, and the selection that ends each sequence runs with 16.
  p->fused = kTopkFused;
  p->threads = kTopkFused ? kTopkThreads : kTopkScoreThreads;
  int64_t chunk = chunk_hint;
  if (chunk == 0) {
    // fused: at most about 256 workgroups of 1024 threads over the batch,
    // chunks of 1024 .. 16384 entries; separate selection: about 768 (bf16
    // keys) or 1536 (fp4 keys) workgroups of 256, chunks of 512 .. 4096 or
    // 8192. A sequence gets groups / B chunks, each a multiple of 256 entries,
    // so that an entry count just past a power of two (a growing context)
    // neither doubles the chunk (idling CUs) nor adds a chunk per sequence
    // (a second round of workgroups); more chunks when a sequence would need
    // more than the selection tracks
    const int64_t groups = p->fused ? 256 : (fp4 ? 1536 : 768);
    const int64_t cap = p->fused ? 16384 : (fp4 ? 8192 : 4096);
    const int64_t per_seq = groups / B > 1 ? groups / B : 1;
    chunk = ((n_max + per_seq - 1) / per_seq + 255) / 256 * 256;
    const int64_t floor_chunk = p->fused ? 1024 : 512;
    chunk = chunk < floor_chunk ? floor_chunk : (chunk > cap ? cap : chunk);
    while ((n_max + chunk - 1) / chunk > kMaxChunks && chunk < 16384) chunk = chunk * 2 > 16384 ? 16384 : chunk * 2;
  }
  if (chunk < 256 || chunk > 16384 || chunk % 256 != 0) return false;
  // (a chunk smaller than one round of the 1024-thread score loop leaves
  // waves idle but stays correct)
  p->chunk = chunk;
  p->n_chunks = n_max <= 0 ? 1 : (n_max + chunk - 1) / chunk;
  if (p->n_chunks > kMaxChunks) return false;
  // candidates the selection gathers into LDS: the k keys at or above the
  // threshold bin plus that bin's other keys (a few hundred on the c4a
  // workloads); more go through the global-memory path
  p->cand_cap = k <= 1024 ? 2048 : 4096;
  p->tb_cap = kTbCap;
  const size_t score_words = (size_t)kHistBins + (size_t)chunk;
  const size_t select_words = select_lds_words(p->cand_cap, p->tb_cap, (int)p->n_chunks, kTopkThreads / kWave);
  p->lds_bytes = 4 * (p->fused && select_words > score_words ? select_words : score_words);
  p->select_lds_bytes = 4 * select_words;
  const size_t nb = (size_t)B;
  const size_t slots = nb * (size_t)p->n_chunks * (size_t)chunk;
  size_t off = 0;
  p->off_hist = off; off = align256(off + nb * kHistBins * 4);
  p->off_arrive = off; off = align256(off + nb * 4);
  p->zero_bytes = off;
  p->off_cnt = off; off = align256(off + nb * (size_t)p->n_chunks * 4);
  p->off_ckey = off; off = align256(off + slots * 4);
  p->off_cidx = off; off = align256(off + slots * 4);
  p->bytes = off;
  return true;
}

template <int DI, bool FP4, int NT, bool FUSED>
static hipError_t launch_t(const TopkPlan& p, const uint16_t* q_idx, const void* k_idx,
                           const uint8_t* k_scale, const int32_t* n_entries, int64_t B, int64_t n_max,
                           int k, int32_t* ids, uint8_t* ws, hipStream_t stream) {
  auto kern = k_index_topk<DI, FP4, NT, FUSED>;
  if (p.lds_bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds_bytes);
    if (e != hipSuccess) return e;
  }
  // a sequence's chunks on one XCD when the batch fills whole XCD rounds
  const bool xcd = FUSED && B % 8 == 0 && B * p.n_chunks <= 0x7FFFFFFF;
  const dim3 grid = xcd ? dim3((unsigned)(B * p.n_chunks)) : dim3((unsigned)p.n_chunks, (unsigned)B);
  hipLaunchKernelGGL(kern, grid, dim3(NT), p.lds_bytes, stream, q_idx, k_idx, k_scale, n_entries,
                     n_max, (int)p.chunk, (int)p.n_chunks, k, p.cand_cap, p.tb_cap,
                     reinterpret_cast<uint32_t*>(ws + p.off_hist), reinterpret_cast<uint32_t*>(ws + p.off_arrive),
                     reinterpret_cast<uint32_t*>(ws + p.off_ckey), reinterpret_cast<int32_t*>(ws + p.off_cidx),
                     reinterpret_cast<int32_t*>(ws + p.off_cnt), ids, xcd ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (FUSED || e != hipSuccess) return e;
  auto sel = k_topk_select<kTopkThreads>;
  if (p.select_lds_bytes > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(sel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)p.select_lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sel, dim3((unsigned)B), dim3(kTopkThreads), p.select_lds_bytes, stream, n_entries, n_max, k,
                     (int)p.chunk, (int)p.n_chunks, p.cand_cap, p.tb_cap,
                     reinterpret_cast<uint32_t*>(ws + p.off_hist), reinterpret_cast<uint32_t*>(ws + p.off_arrive),
                     reinterpret_cast<uint32_t*>(ws + p.off_ckey), reinterpret_cast<int32_t*>(ws + p.off_cidx),
                     reinterpret_cast<const int32_t*>(ws + p.off_cnt), ids);
  return hipGetLastError();
}

template <int NT, bool FUSED>
static hipError_t launch_nt(const TopkPlan& p, const uint16_t* q_idx, bool fp4, const void* k_idx,
                            const uint8_t* k_scale, const int32_t* n_entries, int64_t B, int64_t n_max,
                            int Di, int k, int32_t* ids, uint8_t* ws, hipStream_t stream) {
  if (fp4) {
    return Di == 128 ? launch_t<128, true, NT, FUSED>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream)
                     : launch_t<32, true, NT, FUSED>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream);
  }
  return Di == 128 ? launch_t<128, false, NT, FUSED>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream)
                   : launch_t<32, false, NT, FUSED>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream);
}

hipError_t launch_index_topk(const TopkPlan& p, const uint16_t* q_idx, bool fp4, const void* k_idx,
                             const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                             int64_t n_max, int Di, int k, int32_t* ids, void* workspace,
                             hipStream_t stream) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  if (p.fused) return launch_nt<kTopkThreads, true>(p, q_idx, fp4, k_idx, k_scale, n_entries, B, n_max, Di, k, ids, ws, stream);
  return launch_nt<kTopkScoreThreads, false>(p, q_idx, fp4, k_idx, k_scale, n_entries, B, n_max, Di, k, ids, ws, stream);
}

}  // namespace cskv
