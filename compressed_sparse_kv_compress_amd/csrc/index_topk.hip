// Indexer scores and exact top-k over c4a entries.
//
// [P1] "c4a (the milder scheme)": DeepSeek Sparse Attention keeps the top-k
// compressed entries per query (default k = 512). [P2] Step 5: a learned
// indexer scores every compressed block; the query reads only the chosen ones.
//
// Level 0 (k_index_chunk): one workgroup scores a chunk of entries - a GEMV of
// the query's indexer vector against bf16 or fp4 keys streamed from HBM with
// 16-byte coalesced loads, reduced across lanes with DPP - writes each score's
// orderable 32-bit key to LDS, then selects the chunk's k best with a radix
// select in LDS and writes them in entry order.
// Levels >= 1 (k_topk_merge): one workgroup merges up to `fanin` lists of one
// sequence into its k best, again in entry order. The global top-k under the
// total order (score desc, entry asc) is contained in the union of the chunks'
// top-k, so every level is exact; the last level writes the ids, -1 padded.
#include "kernels.h"

namespace cskv {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kHistPad = 257;               // per-wave histogram copies, bank-shifted
constexpr int kMaxChunk = 16384;            // LDS keys of one chunk
constexpr int kMaxMerge = 16384;            // candidates one merge workgroup holds
constexpr int kAutoChunkMax = 8192;
constexpr int kMisc = 16;

// ------------------------------------------------------------- selection core

// k-th largest of keys[0..n) (1 <= k <= n) by 4 passes of 8-bit radix select.
// Returns the key T and how many keys equal to T belong to the top k.
__device__ void block_kth(const uint32_t* keys, int n, int k, uint32_t* hist, int* misc,
                          uint32_t& T_out, int& need_eq_out) {
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  uint32_t prefix = 0;
  int remaining = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = t; i < kTopkWaves * kHistPad; i += kTopkThreads) hist[i] = 0u;
    __syncthreads();
    uint32_t* h = hist + wave * kHistPad;
    for (int i = t; i < n; i += kTopkThreads) {
      const uint32_t key = keys[i];
      const bool match = (pass == 0) || (((key ^ prefix) >> (shift + 8)) == 0u);
      if (match) atomicAdd(&h[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l covers digits 255-4l .. 252-4l, so the scan runs from the top digit down
      int c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 255 - 4 * lane - j;
        int v = 0;
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) v += (int)hist[w * kHistPad + d];
        c[j] = v;
        s += v;
      }
      int above = wave_inclusive_scan(s) - s;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < remaining && remaining <= above + c[j]) {
          misc[0] = 255 - 4 * lane - j;
          misc[1] = above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)misc[0] << shift;
    remaining -= misc[1];
    __syncthreads();
  }
  T_out = prefix;
  need_eq_out = remaining;
}

// Emits, in index order, every key > T plus the first need_eq keys == T (or
// every key when `all`). Writes key (if out_key) and id = idx_map[i] (if
// idx_map) else idx_base + i. Returns the number emitted (same in all threads).
__device__ int block_emit(const uint32_t* keys, int n, bool all, uint32_t T, int need_eq,
                          int* misc, uint32_t* out_key, int32_t* out_idx, int out_cap,
                          const int32_t* idx_map, int32_t idx_base) {
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
      if (p < out_cap) {   // always true when the selection is consistent; guards the store
        if (out_key) out_key[p] = key;
        out_idx[p] = idx_map ? idx_map[i] : idx_base + i;
      }
    }
    eq_run += __popcll(eqm);
    pos += __popcll(selm);
  }
  __syncthreads();  // misc is reused by the caller
  return total < out_cap ? total : out_cap;
}

// ------------------------------------------------------------- level 0

// bf16 keys: LPE = DI/8 lanes read one 16-byte slice each of an entry; a
// wave-wide load covers 64/LPE consecutive entries (1 KiB contiguous).
template <int DI>
__device__ void score_chunk_bf16(const uint16_t* q, const uint16_t* keys_g, int n, uint32_t* keys) {
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
      v[u] = e < n ? kp[(int64_t)e * LPE + cg] : make_uint4(0, 0, 0, 0);
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
      if (cg == 0 && e < n) keys[e] = score_key(p);
    }
  }
}

// fp4 keys: each lane reads 16 code bytes (32 channels = two 16-channel groups)
// and the two matching E4M3 group scales; LPE = DI/32 lanes per entry.
template <int DI>
__device__ void score_chunk_fp4(const uint16_t* q, const uint8_t* codes_g, const uint8_t* scales_g,
                                int n, uint32_t* keys) {
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
      v[u] = e < n ? cp[(int64_t)e * LPE + part] : make_uint4(0, 0, 0, 0);
      s[u] = e < n ? (uint32_t)sp[(int64_t)e * LPE + part] : 0u;
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
      if (part == 0 && e < n) keys[e] = score_key(p);
    }
  }
}

template <int DI, bool FP4>
__global__ __launch_bounds__(kTopkThreads) void k_index_chunk(
    const uint16_t* __restrict__ q_idx, const void* __restrict__ k_idx,
    const uint8_t* __restrict__ k_scale, const int32_t* __restrict__ n_entries, int64_t n_max,
    int chunk, int k, int64_t n_lists, uint32_t* __restrict__ out_key,
    int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt, int32_t* __restrict__ final_ids) {
  extern __shared__ uint32_t lds[];
  uint32_t* keys = lds;
  uint32_t* hist = lds + chunk;
  int* misc = reinterpret_cast<int*>(hist + kTopkWaves * kHistPad);
  const int64_t b = blockIdx.y;
  const int64_t c = blockIdx.x;
  int64_t nv = n_entries ? (int64_t)n_entries[b] : n_max;
  nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
  const int64_t start = c * chunk;
  const int64_t rem = nv - start;
  const int n = rem <= 0 ? 0 : (rem > chunk ? chunk : (int)rem);
  const int64_t list = b * n_lists + c;

  if (n > 0) {
    const uint16_t* q = q_idx + b * DI;
    if constexpr (FP4) {
      const uint8_t* codes = reinterpret_cast<const uint8_t*>(k_idx) + (b * n_max + start) * (DI / 2);
      const uint8_t* scales = k_scale + (b * n_max + start) * (DI / 16);
      score_chunk_fp4<DI>(q, codes, scales, n, keys);
    } else {
      const uint16_t* kk = reinterpret_cast<const uint16_t*>(k_idx) + (b * n_max + start) * DI;
      score_chunk_bf16<DI>(q, kk, n, keys);
    }
  }
  __syncthreads();
  const bool all = n <= k;
  uint32_t T = 0u;
  int need = 0;
  if (!all) block_kth(keys, n, k, hist, misc, T, need);
  int cnt = 0;
  if (final_ids) {
    int32_t* ids = final_ids + b * k;
    if (n > 0) cnt = block_emit(keys, n, all, T, need, misc, nullptr, ids, k, nullptr, (int32_t)start);
    for (int i = cnt + threadIdx.x; i < k; i += kTopkThreads) ids[i] = -1;
  } else {
    if (n > 0)
      cnt = block_emit(keys, n, all, T, need, misc, out_key + list * k, out_idx + list * k, k, nullptr,
                       (int32_t)start);
    if (threadIdx.x == 0) out_cnt[list] = cnt;
  }
}

// ------------------------------------------------------------- levels >= 1

__global__ __launch_bounds__(kTopkThreads) void k_topk_merge(
    const uint32_t* __restrict__ in_key, const int32_t* __restrict__ in_idx,
    const int32_t* __restrict__ in_cnt, int64_t in_lists, int fanin, int k,
    uint32_t* __restrict__ out_key, int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt,
    int64_t out_lists, int32_t* __restrict__ final_ids) {
  extern __shared__ uint32_t lds[];
  const int cap = fanin * k;
  uint32_t* keys = lds;
  int32_t* idx = reinterpret_cast<int32_t*>(lds + cap);
  uint32_t* hist = lds + 2 * cap;
  int* misc = reinterpret_cast<int*>(hist + kTopkWaves * kHistPad);
  int* offs = misc + kMisc;  // [fanin + 1]
  const int64_t b = blockIdx.y;
  const int64_t node = blockIdx.x;
  const int64_t l0 = node * fanin;
  const int m = (int)((l0 + fanin <= in_lists ? l0 + fanin : in_lists) - l0);
  const int t = threadIdx.x;
  if (t < kWave) {
    const int cnt = t < m ? in_cnt[b * in_lists + l0 + t] : 0;
    const int incl = wave_inclusive_scan(cnt);
    if (t < m) offs[t + 1] = incl;
    if (t == 0) offs[0] = 0;
  }
  __syncthreads();
  const int total = offs[m];
  for (int i = t; i < m * k; i += kTopkThreads) {
    const int j = i / k, s = i - j * k;
    if (s < offs[j + 1] - offs[j] && offs[j] + s < cap) {
      const int64_t src = (b * in_lists + l0 + j) * k + s;
      keys[offs[j] + s] = in_key[src];
      idx[offs[j] + s] = in_idx[src];
    }
  }
  __syncthreads();
  const bool all = total <= k;
  uint32_t T = 0u;
  int need = 0;
  if (!all) block_kth(keys, total, k, hist, misc, T, need);
  int cnt = 0;
  if (final_ids) {
    int32_t* ids = final_ids + b * k;
    if (total > 0) cnt = block_emit(keys, total, all, T, need, misc, nullptr, ids, k, idx, 0);
    for (int i = cnt + t; i < k; i += kTopkThreads) ids[i] = -1;
  } else {
    const int64_t list = b * out_lists + node;
    if (total > 0)
      cnt = block_emit(keys, total, all, T, need, misc, out_key + list * k, out_idx + list * k, k, idx, 0);
    if (t == 0) out_cnt[list] = cnt;
  }
}

// ------------------------------------------------------------- planning / launch

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool plan_topk(int64_t B, int64_t n_max, int k, int chunk_hint, TopkPlan* p) {
  int64_t chunk = chunk_hint;
  if (chunk == 0) {
    // aim at ~512 level-0 workgroups over the whole batch
    int64_t want = (B * n_max + 511) / 512;
    chunk = 1024;
    while (chunk < want && chunk < kAutoChunkMax) chunk *= 2;
  }
  if (chunk < 256 || chunk > kMaxChunk || chunk % 256 != 0) return false;
  p->chunk = chunk;
  p->fanin = kMaxMerge / k < 64 ? kMaxMerge / k : 64;
  if (p->fanin < 2) return false;
  int64_t lists = n_max <= 0 ? 1 : (n_max + chunk - 1) / chunk;
  int lv = 0;
  p->lists[lv++] = lists;
  while (lists > 1) {
    if (lv >= 8) return false;
    lists = (lists + p->fanin - 1) / p->fanin;
    p->lists[lv++] = lists;
  }
  p->levels = lv;
  size_t off = 0;
  for (int i = 0; i < lv; ++i) {
    p->off_key[i] = p->off_idx[i] = p->off_cnt[i] = 0;
    if (i == lv - 1) break;  // the last level writes the caller's ids
    const size_t n = (size_t)B * (size_t)p->lists[i];
    p->off_key[i] = off; off = align256(off + n * (size_t)k * 4);
    p->off_idx[i] = off; off = align256(off + n * (size_t)k * 4);
    p->off_cnt[i] = off; off = align256(off + n * 4);
  }
  p->bytes = off;
  return true;
}

template <int DI, bool FP4>
static hipError_t launch_level0(const TopkPlan& p, const uint16_t* q_idx, const void* k_idx,
                                const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                                int64_t n_max, int k, int32_t* ids, uint8_t* ws,
                                hipStream_t stream) {
  const size_t shmem = (size_t)p.chunk * 4 + kTopkWaves * kHistPad * 4 + kMisc * 4;
  auto kern = k_index_chunk<DI, FP4>;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const bool final_level = p.levels == 1;
  dim3 grid((unsigned)p.lists[0], (unsigned)B);
  hipLaunchKernelGGL(kern, grid, dim3(kTopkThreads), shmem, stream, q_idx, k_idx, k_scale,
                     n_entries, n_max, (int)p.chunk, k, p.lists[0],
                     final_level ? nullptr : reinterpret_cast<uint32_t*>(ws + p.off_key[0]),
                     final_level ? nullptr : reinterpret_cast<int32_t*>(ws + p.off_idx[0]),
                     final_level ? nullptr : reinterpret_cast<int32_t*>(ws + p.off_cnt[0]),
                     final_level ? ids : nullptr);
  return hipGetLastError();
}

hipError_t launch_index_topk(const TopkPlan& p, const uint16_t* q_idx, bool fp4, const void* k_idx,
                             const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                             int64_t n_max, int Di, int k, int32_t* ids, void* workspace,
                             hipStream_t stream) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  hipError_t e;
  if (fp4) {
    e = Di == 128 ? launch_level0<128, true>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream)
                  : launch_level0<32, true>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream);
  } else {
    e = Di == 128 ? launch_level0<128, false>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream)
                  : launch_level0<32, false>(p, q_idx, k_idx, k_scale, n_entries, B, n_max, k, ids, ws, stream);
  }
  if (e != hipSuccess) return e;
  const size_t shmem = (size_t)p.fanin * k * 8 + kTopkWaves * kHistPad * 4 + kMisc * 4 +
                       ((size_t)p.fanin + 1) * 4;
  if (p.levels > 1 && shmem > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_merge),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  for (int lv = 1; lv < p.levels; ++lv) {
    const bool final_level = lv == p.levels - 1;
    dim3 grid((unsigned)p.lists[lv], (unsigned)B);
    hipLaunchKernelGGL(k_topk_merge, grid, dim3(kTopkThreads), shmem, stream,
                       reinterpret_cast<const uint32_t*>(ws + p.off_key[lv - 1]),
                       reinterpret_cast<const int32_t*>(ws + p.off_idx[lv - 1]),
                       reinterpret_cast<const int32_t*>(ws + p.off_cnt[lv - 1]), p.lists[lv - 1],
                       p.fanin, k,
                       final_level ? nullptr : reinterpret_cast<uint32_t*>(ws + p.off_key[lv]),
                       final_level ? nullptr : reinterpret_cast<int32_t*>(ws + p.off_idx[lv]),
                       final_level ? nullptr : reinterpret_cast<int32_t*>(ws + p.off_cnt[lv]),
                       p.lists[lv], final_level ? ids : nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace cskv
