// Shared-K/V multi-query attention over gathered cache entries plus the
// uncompressed window, with inverse RoPE on the output.
//
// [P2] Step 3: one shared state S_j is compared with the query (score =
// Q.S_j) and mixed into the output as content. [P2] Step 5: the query reads
// the selected c4a entries, or every c128a entry. [P2] Step 6 and [P1] "The
// sliding window": the newest 128 states are read exactly, in the same
// softmax. [P1] "Shared key and value": inverse RoPE on the attention output.
//
// All heads of a sequence share the key rows, so both contractions are dense
// and run on 16x16x32 bf16 MFMA. A workgroup (4 waves, one per compute unit)
// owns one sequence and a contiguous split of its key slots; wave w owns heads
// 16w .. 16w+15. Key rows move in tiles of 32 slots through a ring of four LDS
// buffers, two (bf16 rows: the step that runs QK^T on a tile also runs PV on
// the one before, so that slot is still in use) or three tiles ahead of
// their use:
//   - bf16 rows of 1 KiB go by direct HBM->LDS DMA (non-temporal, one wave
//     instruction per row, no registers); fp8 rows go by DMA into a staging
//     ring and one cooperative pass widens the codes to bf16 exactly, and the
//     row scales travel by DMA too (folded into logits and probabilities);
//     mixed and fp4 rows land raw in their tile rows and are widened in place,
//     tile i+1 under tile i's PV products (see raw_read / raw_write);
//     other shapes go through registers. Empty slots (an id out of range, or
//     past the last key) load a zero row, so every wave issues the same number
//     of DMA instructions per tile and the wait for a tile is an exact count of
//     the younger DMAs still in flight. The entry ids of a split are staged in
//     LDS once. Each ring buffer is its own LDS object and the tile loop is
//     unrolled over the ring, so the compiler can tell the DMA into one buffer
//     from the reads of another and never serialises them;
//   - S^T[32 keys x 16 heads] = K Q^T with Q held in registers;
//   - softmax per head in the exp2 domain against a reference maximum that is
//     fixed for the whole split (0 at first). Each lane also tracks the largest
//     logit it saw; if at the end a head's true maximum lies more than 64
//     (log2 units) above or below the reference, the split is run a second time
//     with the true maximum as reference. Probabilities therefore stay within
//     [2^-64, 2^64] of the largest one (inside bf16 and fp32 range) and the
//     accumulators are never rescaled, so the loop holds them in the MFMA
//     accumulator registers without moving them;
//   - the probabilities of all 64 heads meet in a 4 KiB LDS buffer (each lane
//     writes its 8 values as one 16-byte store, already in the key order the
//     next product consumes), and wave w computes O^T[D/4 channels x 64 heads]
//     += K^T P^T for its quarter of the channels, so each K element is read
//     from LDS once by QK^T's wave and once, transposed, for PV; K^T comes from
//     the row-major tile through gfx950's transposing LDS reads.
// Tile rows are padded to a stride of 8 (mod 64) dwords and their 16-byte
// chunks are XOR-swizzled by (row / 4) mod 4. Of the swizzles and strides
// measured on the QK^T row reads and the PV transposing reads of a resident
// tile, this one was the fastest for both (QK^T reads: 553 ns a tile per CU,
// against 737 ns with (row / 8) mod 4 and 558 ns with none).
// Each lane ends with 4 consecutive channels of one head: rotary pairs sit in
// one lane. With one split the epilogue normalises, applies inverse RoPE and
// stores O; otherwise partials (reference maximum, sum, unnormalised O, the
// latter in the accumulators' register order so that every store writes 1 KiB
// contiguously) go to the workspace and k_attend_merge combines them with a
// log-sum-exp merge.
#include <type_traits>

#include "kernels.h"

namespace cskv {

constexpr int kAttThreads = 256;
constexpr int kTK = 32;          // key slots per tile
constexpr int kNStage = 4;       // tiles in the LDS ring
constexpr int kHMax = 64;        // heads per workgroup (4 waves x 16)
constexpr int kMaxSplitIds = 2048;   // entry ids of a sparse split staged in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 64.0f;       // log2 distance allowed between reference and true maximum
constexpr int kCachePolicyStream = 2;    // non-temporal loads for rows read once

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// DMA sources of empty slots: a zero row and a zero row scale (file-local, so
// their addresses are PC-relative constants rather than loads).
static __device__ __attribute__((aligned(16))) uint8_t g_zero_row[1024];
static __device__ float g_empty_scale = 0.0f;
static __device__ float g_one_scale = 1.0f;
static __device__ int32_t g_no_count = 0;   // read in place of an absent count

// Swizzle of a tile row's 16-byte chunks.
__device__ __forceinline__ int chunk_swz(int row) { return (row >> 2) & 3; }

// CF: cache row format (kFmtBf16, kFmtFp8 or kFmtMix); WFP8: fp8 window rows.
template <int D, int CF, bool WFP8>
struct AttCfg {
  static constexpr bool kDma = D == 512 && CF == kFmtBf16 && !WFP8;   // bf16 rows by DMA
  static constexpr bool kDmaFp8 = D == 512 && CF == kFmtFp8 && WFP8;  // fp8 rows by DMA + widening pass
  // mixed cache rows by DMA into their tile rows as raw bytes + an in-place
  // widening pass; bf16 window rows by DMA as in the bf16 path
  static constexpr bool kDmaMix = D == 512 && CF == kFmtMix && !WFP8;
  static constexpr bool kDmaFp4 = D == 512 && CF == kFmtFp4 && !WFP8;  // fp4 rows: likewise
  static constexpr bool kDmaRaw = kDmaMix || kDmaFp4;                 // raw rows widened in place
  static constexpr int kRawChunks = kDmaMix ? kMixRowChunks : kFp4RowChunks;
  static constexpr bool kReg = !kDma && !kDmaFp8 && !kDmaRaw;         // register-staged fill
  // rows carry a value scale (mixed rows are widened with theirs applied)
  static constexpr bool kScaled = CF == kFmtFp8 || WFP8;
  static constexpr int KROW = D + 16;                           // bf16 per tile row
  static constexpr int kTileElems = kTK * KROW;                 // bf16 per tile
  // fp8 staging tile: the rows' codes, then their 32 scales (one DMA target per slot)
  static constexpr int kStageBytes = kDmaFp8 ? kTK * D + kTK * 4 : 16;
  // DMA instructions per wave and tile: 8 rows (+ their scales for fp8 / mixed rows)
  static constexpr int kOpsPerTile = kDma ? 8 : (kDmaFp8 ? 5 : (kDmaRaw ? 9 : 0));
};

// vmcnt(n) with the other counters left alone (n <= 63).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until the oldest in-flight tile has landed, `younger` tiles (0 .. 2)
// having been issued after it.
template <int OPS>
__device__ __forceinline__ void wait_tile(int younger) {
  if (younger >= 2) wait_vm<2 * OPS>();
  else if (younger == 1) wait_vm<OPS>();
  else wait_vm<0>();
}

// Workgroup barrier for LDS traffic only: LDS writes are complete before it,
// in-flight DMA is left alone (tile arrival is waited for by count). The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ uint64_t lane_u64(uint64_t p, int lane) {
  const uint32_t lo32 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)p, lane);
  const uint32_t hi32 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(p >> 32), lane);
  return ((uint64_t)hi32 << 32) | lo32;
}

// Window rows of sequence b that are keys: the first n_window[b] (clamped to
// [0, W]), or all W.
__device__ __forceinline__ int64_t window_rows(const AttendArgs& a, int64_t b) {
  if (!a.n_window) return a.W;
  const int64_t n = a.n_window[b];
  return n < 0 ? 0 : (n > a.W ? a.W : n);
}

// Kernel-uniform sources of key rows (held in scalar registers, so choosing
// between cache and window selects values instead of loading an argument).
struct RowSrc {
  const uint8_t* cache;      // row 0 of this sequence's cache
  const float* cache_scale;  // fp8 cache: row scales of this sequence
  const uint8_t* window;     // window row 0 of this sequence
  const float* window_scale;
  int64_t cache_rows;
};

template <int D, int CF, bool WFP8>
__device__ __forceinline__ RowSrc row_src(const AttendArgs& a, int64_t b) {
  RowSrc r;
  r.cache = reinterpret_cast<const uint8_t*>(a.cache) + b * a.cache_rows * row_bytes<D, CF>();
  r.cache_scale = CF == kFmtFp8 || CF == kFmtMix ? a.cache_scale + b * a.cache_rows : nullptr;
  r.window = reinterpret_cast<const uint8_t*>(a.window) + b * a.win_bstride * D * (WFP8 ? 1 : 2);
  r.window_scale = WFP8 ? a.window_scale + b * a.win_bstride : nullptr;
  r.cache_rows = a.cache_rows;
  return r;
}

// The row a slot reads: pointer (nullptr for an empty slot) and fp8 scale
// pointer (nullptr for bf16). Sparse ids come from the split's LDS copy.
template <int D, int CF, bool WFP8>
__device__ __forceinline__ void slot_source(const RowSrc& rs, int64_t slot, int64_t lo, int64_t n_sel,
                                            int64_t n_keys, bool dense, const int32_t* ids_l,
                                            const uint8_t*& ptr, const float*& scale) {
  ptr = nullptr;
  scale = nullptr;
  if (slot >= n_keys) return;
  const bool in_cache = slot < n_sel;
  const int64_t id = in_cache ? (dense ? slot : (int64_t)ids_l[slot - lo]) : slot - n_sel;
  if (in_cache && (id < 0 || id >= rs.cache_rows)) return;
  const uint8_t* base = in_cache ? rs.cache : rs.window;
  const float* sbase = in_cache ? rs.cache_scale : rs.window_scale;
  ptr = base + id * (in_cache ? row_bytes<D, CF>() : (WFP8 ? D : 2 * D));
  scale = sbase ? sbase + id : nullptr;
}

// Issues the fill of one tile (slots tile0 .. tile0+31): wave w handles rows
// 8w .. 8w+7, lane j < 8 resolving row 8w + j. `tile` is the bf16 buffer
// (DMA and register paths), `stage` the fp8 staging buffer; per slot, `pb` is
// the logit bias (0, or -inf for an empty slot) and `vs` the row's value scale
// (fp8 rows: the row scale; bf16 rows: 1; empty slots: 0).
template <int D, int CF, bool WFP8>
__device__ __forceinline__ void issue_tile(const RowSrc& rsrc, int64_t tile0, int64_t lo,
                                           int64_t n_sel, int64_t n_keys, bool dense, const int32_t* ids_l,
                                           uint16_t* tile, uint8_t* stage, float* pb, float* vs, int wave,
                                           int lane) {
  using C = AttCfg<D, CF, WFP8>;
  if constexpr (C::kReg) {
    // thread (kb, cb): rows 8kb .. 8kb+7, logical chunk cb (8 channels)
    const int t = threadIdx.x, kb = t >> 6, cb = t & 63;
    const bool active_c = cb * 8 < D;
    uint4 r[8];
    float sc[8], bias[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint8_t* p;
      const float* sp;
      slot_source<D, CF, WFP8>(rsrc, tile0 + 8 * kb + i, lo, n_sel, n_keys, dense, ids_l, p, sp);
      // a cache row of the mixed format: codes widened with the row scale applied,
      // the rotary channels copied (value scale 1)
      const bool mix = CF == kFmtMix && tile0 + 8 * kb + i < n_sel;
      const bool f4 = CF == kFmtFp4 && tile0 + 8 * kb + i < n_sel;   // fp4 cache row: exact widening
      r[i] = make_uint4(0, 0, 0, 0);
      sc[i] = p ? (sp && !mix ? *sp : 1.0f) : 0.0f;
      bias[i] = p ? 0.0f : -INFINITY;
      if (p && active_c) {
        if (f4) {
          r[i] = fp4x8_to_bf16x8_scaled(*reinterpret_cast<const uint32_t*>(p + cb * 4), e4m3_to_f32(p[D / 2 + cb / 2]));
        } else if (mix) {
          if (cb * 8 < D - kMixRope) r[i] = fp8x8_to_bf16x8_scaled(*reinterpret_cast<const uint2*>(p + cb * 8), *sp);
          else r[i] = *reinterpret_cast<const uint4*>(p + (D - kMixRope) + 2 * (cb * 8 - (D - kMixRope)));
        } else if (sp) {
          r[i] = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(p + cb * 8));
        } else {
          r[i] = *reinterpret_cast<const uint4*>(p + cb * 16);
        }
      }
    }
    if (active_c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * kb + i;
        *reinterpret_cast<uint4*>(tile + row * C::KROW + 8 * (cb ^ chunk_swz(row))) = r[i];
      }
    }
    if (cb == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (C::kScaled) vs[8 * kb + i] = sc[i];   // vs has kTK slots only for scaled rows
        pb[8 * kb + i] = bias[i];
      }
    }
  } else {
    if constexpr (C::kDma) {
      // dense rows that all come from the cache: contiguous, so the row
      // addresses are scalar arithmetic and the swizzle (which depends on
      // row / 4 only) is one lane offset for each half of the wave's 8 rows
      const int wv = __builtin_amdgcn_readfirstlane(wave);   // scalar, so LDS targets are too
      const int64_t row0 = tile0 + 8 * wv;
      if (dense && row0 + 8 <= n_sel) {
        if (lane < 8) pb[8 * wv + lane] = 0.0f;
        const uint8_t* src0 = rsrc.cache + row0 * (D * 2) + 16 * (lane ^ chunk_swz(8 * wv));
        const uint8_t* src1 = rsrc.cache + row0 * (D * 2) + 16 * (lane ^ chunk_swz(8 * wv + 4));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)((i < 4 ? src0 : src1) + i * (D * 2)),
                                           (__attribute__((address_space(3))) void*)(tile + (8 * wv + i) * C::KROW),
                                           16, 0, kCachePolicyStream);
        }
        return;
      }
      if (!dense && row0 + 8 <= n_sel) {
        // selected entries only: each lane < 8 reads one id, each row takes it
        // with one readlane; rows of invalid ids read the zero row
        const int myid = lane < 8 ? ids_l[row0 - lo + lane] : 0;
        const bool ok = myid >= 0 && (int64_t)myid < rsrc.cache_rows;
        if (lane < 8) pb[8 * wv + lane] = ok ? 0.0f : -INFINITY;
        const int lane_off0 = 16 * (lane ^ chunk_swz(8 * wv)), lane_off1 = 16 * (lane ^ chunk_swz(8 * wv + 4));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int id = __builtin_amdgcn_readlane(myid, i);
          const uint8_t* rowp = id >= 0 && (int64_t)id < rsrc.cache_rows ? rsrc.cache + (int64_t)id * (D * 2) : g_zero_row;
          __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(rowp + (i < 4 ? lane_off0 : lane_off1)),
                                           (__attribute__((address_space(3))) void*)(tile + (8 * wv + i) * C::KROW),
                                           16, 0, kCachePolicyStream);
        }
        return;
      }
    }
    if constexpr (C::kDmaRaw) {
      // dense rows that all come from the cache: contiguous raw rows, scalar
      // row addresses; only the lanes of a row's bytes move data (the other
      // chunks are written by the widening), and every DMA has active lanes,
      // so each still counts once in the wave's vmcnt
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const int64_t row0 = tile0 + 8 * wv;
      if (dense && row0 + 8 <= n_sel) {
        if (lane < 8) {
          pb[8 * wv + lane] = 0.0f;
          const float* s = C::kDmaMix ? rsrc.cache_scale + row0 + lane : &g_one_scale;
          __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)s,
                                           (__attribute__((address_space(3))) void*)(tile + 8 * wv * C::KROW + D),
                                           4, 0, 0);
        }
        constexpr int RBY = row_bytes<D, CF>();
        const uint8_t* src = rsrc.cache + row0 * RBY + 16 * lane;
        if (lane < C::kRawChunks) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src + i * RBY),
                                             (__attribute__((address_space(3))) void*)(tile + (8 * wv + i) * C::KROW),
                                             16, 0, kCachePolicyStream);
          }
        }
        return;
      }
    }
    const uint8_t* p = nullptr;
    const float* sp = nullptr;
    if (lane < 8) slot_source<D, CF, WFP8>(rsrc, tile0 + 8 * wave + lane, lo, n_sel, n_keys, dense, ids_l, p, sp);
    const uint64_t src_l = reinterpret_cast<uint64_t>(p ? p : g_zero_row);
    if (lane < 8) pb[8 * wave + lane] = p ? 0.0f : -INFINITY;
    if constexpr (C::kDmaRaw) {
      // per row a scale that marks raw rows for the widening pass (mixed rows:
      // their row scale; fp4 rows: 1; window and empty rows: 0), the wave's 8
      // of them in the 32 pad bytes of its first row (the tile buffers stay the
      // only DMA targets besides the first dummy one)
      const bool mix_l = lane < 8 && p && tile0 + 8 * wave + lane < n_sel;
      if (lane < 8) {
        const float* s = mix_l ? (C::kDmaMix ? sp : &g_one_scale) : &g_empty_scale;
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)s,
                                         (__attribute__((address_space(3))) void*)(tile + 8 * wave * C::KROW + D),
                                         4, 0, 0);
      }
      const uint64_t mix_m = __ballot(mix_l);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * wave + i;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(lane_u64(src_l, i));
        // raw row: its bytes land at chunk positions 0 .. kRawChunks-1, moved
        // by those lanes only (the widening writes the other chunks); bf16 row:
        // swizzled chunks as in the bf16 path. Every DMA has active lanes.
        const bool raw_row = (mix_m >> i) & 1;
        const uint8_t* a = raw_row ? src + 16 * lane : src + 16 * (lane ^ chunk_swz(row));
        if (!raw_row || lane < C::kRawChunks) {
          __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)a,
                                           (__attribute__((address_space(3))) void*)(tile + row * C::KROW), 16, 0,
                                           kCachePolicyStream);
        }
      }
      return;
    }
    if constexpr (C::kDma) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * wave + i;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(lane_u64(src_l, i));
        // lane l fills chunk position l, which holds logical chunk l ^ swz(row)
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(src + 16 * (lane ^ chunk_swz(row))),
            (__attribute__((address_space(3))) void*)(tile + row * C::KROW), 16, 0, kCachePolicyStream);
      }
    } else {
      // row scales: lanes 0-7 move one dword each into vs[8w .. 8w+7]
      if (lane < 8) {
        const float* s = p ? sp : &g_empty_scale;
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)s,
                                         (__attribute__((address_space(3))) void*)(vs + 8 * wave), 4, 0, 0);
      }
      // fp8 rows of 512 B: lanes 0-31 move row 2i, lanes 32-63 row 2i+1
      const int half = lane >> 5, hl = lane & 31;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t even = lane_u64(src_l, 2 * i), odd = lane_u64(src_l, 2 * i + 1);
        const uint8_t* src = reinterpret_cast<const uint8_t*>(half ? odd : even);
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src + 16 * hl),
                                         (__attribute__((address_space(3))) void*)(stage + (8 * wave + 2 * i) * D),
                                         16, 0, kCachePolicyStream);
      }
    }
  }
}

// A 16-byte LDS store the compiler does not see as one: it would otherwise
// wait for every LDS DMA in flight first (it cannot tell the DMA targets from
// this address). Used only for stores into a tile whose DMA has landed; the
// next lds_barrier() waits for the store (lgkmcnt(0)).
__device__ __forceinline__ void lds_store_b128_unordered(void* p, uint4 v) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  const uint32_t addr = (uint32_t)reinterpret_cast<uintptr_t>(p);   // LDS offset
  const u32x4v d = {v.x, v.y, v.z, v.w};
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(d) : "memory");
}

// Widens a staged fp8 tile into a bf16 tile: thread t converts the 64 codes
// of row t/8, logical chunks 8(t%8) .. 8(t%8)+7 (empty rows hold zero codes).
template <int D>
__device__ __forceinline__ void widen_tile(const uint8_t* stage, uint16_t* tile) {
  using C = AttCfg<D, true, true>;
  const int t = threadIdx.x;
  const int r = t >> 3, part = t & 7;
  const uint8_t* src = stage + r * D + part * 64;
  // the staged codes are read in one asm block that waits for its own reads:
  // as ordinary LDS reads the compiler would first wait for every DMA in
  // flight (it cannot tell this staging slot from the ones still landing),
  // which empties the ring on every tile
  uint4 c[4];
  {
    const uint32_t a0 = (uint32_t)reinterpret_cast<uintptr_t>(src);
    asm volatile(
        "ds_read_b128 %0, %4\n"
        "ds_read_b128 %1, %4 offset:16\n"
        "ds_read_b128 %2, %4 offset:32\n"
        "ds_read_b128 %3, %4 offset:48\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3])
        : "v"(a0)
        : "memory");
  }
  uint16_t* row = tile + r * C::KROW;
  const int swz = chunk_swz(r);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch0 = 8 * part + 2 * j;          // logical chunks ch0, ch0 + 1
    lds_store_b128_unordered(row + 8 * (ch0 ^ swz), fp8x8_to_bf16x8(make_uint2(c[j].x, c[j].y)));
    lds_store_b128_unordered(row + 8 * ((ch0 + 1) ^ swz), fp8x8_to_bf16x8(make_uint2(c[j].z, c[j].w)));
  }
}


// Raw rows (mixed or fp4) are widened in place in two phases: a read phase
// that takes one thread's share of the tile's raw bytes into registers, then
// eight write slices. Thread t takes row t/8 (rows 8w .. 8w+7 are the ones
// wave w's own DMA brought, so the wave's own tile wait covers them), and
// writes 8 of the row's 64 output chunks (16 bytes, 8 channels each, in the
// swizzled chunk layout). A row's reads are all issued before any of its
// writes, by the lanes of one wave, and LDS runs one wave's accesses in
// order; the stores' memory clobber keeps the compiler from moving a read
// past them. Rows whose scale (mixed) or flag (fp4) is 0 are bf16 already;
// the values of rows 8w .. 8w+7 sit in the pad of row 8w. A thread with
// nothing to write (such a row, or no next tile) stores into its row's pad
// instead, which nothing reads after the read phase: the stores need no
// branch.
//
// Mixed rows: part p = t % 8 turns codes 8c .. 8c+7 (raw bytes 8c ..) of
// chunks c = p + 8s, s < 7, into channels 8c .. 8c+7 times the row scale, and
// moves rotary chunk 56 + p (raw bytes 448 + 16p ..) to its place: every part
// does the same work.
struct MixRaw {
  uint2 code[7];
  uint4 rope;
  float sc;
};

template <int D>
__device__ __forceinline__ void raw_read(const uint16_t* tile, MixRaw& m) {
  using C = AttCfg<D, kFmtMix, false>;
  const int t = threadIdx.x, r = t >> 3, p = t & 7;
  const uint16_t* row = tile + r * C::KROW;
  m.sc = reinterpret_cast<const float*>(tile + (r & ~7) * C::KROW + D)[r & 7];
#pragma unroll
  for (int s = 0; s < 7; ++s) m.code[s] = reinterpret_cast<const uint2*>(row)[p + 8 * s];
  m.rope = reinterpret_cast<const uint4*>(row + (D - kMixRope) / 2)[p];
}

template <int D>
__device__ __forceinline__ void raw_write(uint16_t* tile, const MixRaw& m, int s, bool on) {
  using C = AttCfg<D, kFmtMix, false>;
  static_assert(D - kMixRope == 7 * 64, "mixed rows: 7 code chunks per part");
  const int t = threadIdx.x, r = t >> 3, p = t & 7;
  uint16_t* row = tile + r * C::KROW;
  const int chunk = (s < 7 ? p + 8 * s : 56 + p) ^ chunk_swz(r);
  const uint4 v = s < 7 ? fp8x8_to_bf16x8_scaled(m.code[s], m.sc) : m.rope;
  lds_store_b128_unordered(row + (on && m.sc > 0.0f ? 8 * chunk : D), v);
}

// fp4 rows: part p takes chunks c = p + 8s: the code word at raw byte 4c
// (channels 8c .. 8c+7) times the scale of group c/2 (raw byte 256 + c/2),
// exactly. The strided chunks keep the word reads and the widened stores of a
// wave's 64 lanes on distinct LDS banks.
struct Fp4Raw {
  uint32_t code[8];
  uint4 sc0, sc1;   // the row's 32 group scales
  float flag;
};

template <int D>
__device__ __forceinline__ void raw_read(const uint16_t* tile, Fp4Raw& m) {
  using C = AttCfg<D, kFmtFp4, false>;
  static_assert(D == 512, "fp4 rows: 8 chunks per part");
  const int t = threadIdx.x, r = t >> 3, p = t & 7;
  const uint16_t* row = tile + r * C::KROW;
  m.flag = reinterpret_cast<const float*>(tile + (r & ~7) * C::KROW + D)[r & 7];
#pragma unroll
  for (int s = 0; s < 8; ++s) m.code[s] = reinterpret_cast<const uint32_t*>(row)[p + 8 * s];
  m.sc0 = reinterpret_cast<const uint4*>(row + D / 4)[0];
  m.sc1 = reinterpret_cast<const uint4*>(row + D / 4)[1];
}

template <int D>
__device__ __forceinline__ void raw_write(uint16_t* tile, const Fp4Raw& m, int s, bool on) {
  using C = AttCfg<D, kFmtFp4, false>;
  const int t = threadIdx.x, r = t >> 3, p = t & 7;
  uint16_t* row = tile + r * C::KROW;
  const uint32_t sw[8] = {m.sc0.x, m.sc0.y, m.sc0.z, m.sc0.w, m.sc1.x, m.sc1.y, m.sc1.z, m.sc1.w};
  // group 4s + p/2: byte p/2 of scale word s, exactly, through the hardware
  // E4M3 converter
  const uint32_t code = (sw[s] >> (8 * (p >> 1))) & 0xFFu;
  const float gs = __uint_as_float(fp8x2_to_bf16x2<false>(code) << 16);
  const uint4 v = fp4x8_to_bf16x8_scaled(m.code[s], gs);
  lds_store_b128_unordered(row + (on && m.flag > 0.0f ? 8 * ((p + 8 * s) ^ chunk_swz(r)) : D), v);
}

// The register share of a raw tile for row format CF (an empty type for others).
struct NoRaw {};
template <int D>
__device__ __forceinline__ void raw_read(const uint16_t*, NoRaw&) {}
template <int D>
__device__ __forceinline__ void raw_write(uint16_t*, const NoRaw&, int, bool) {}
template <int CF> struct RawOf { using type = NoRaw; };
template <> struct RawOf<kFmtMix> { using type = MixRaw; };
template <> struct RawOf<kFmtFp4> { using type = Fp4Raw; };

// The whole widening of a tile's rows, waiting for the reads before the writes.
template <int D, typename R>
__device__ __forceinline__ void widen_raw_tile(uint16_t* tile) {
  R m;
  raw_read<D>(tile, m);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
#pragma unroll
  for (int s = 0; s < 8; ++s) raw_write<D>(tile, m, s, true);
}

template <int D, int CF, bool WFP8>
__global__ __launch_bounds__(kAttThreads, 1) void k_attend(int splits, int64_t keys_per_split,
                                                          uint16_t* __restrict__ ws_acc, float* __restrict__ ws_ml,
                                                          AttendArgs a) {
  using C = AttCfg<D, CF, WFP8>;
  constexpr int KS = D / 32;          // k-steps of QK^T
  constexpr int CTW = D / 64;         // 16-channel tiles of O^T per wave (a quarter of D)
  constexpr int KROW = C::KROW;
  // ring buffers: separate LDS objects so DMA targets and reads never alias
  __shared__ __attribute__((aligned(16))) uint16_t tile0[C::kTileElems], tile1[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile2[C::kDmaFp8 ? 8 : C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile3[C::kDmaFp8 ? 8 : C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint8_t stage0[C::kStageBytes], stage1[C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage2[C::kStageBytes], stage3[C::kStageBytes];
  // per slot: logit bias (0 or -inf) and value scale (scaled rows only)
  __shared__ __attribute__((aligned(16))) float pb0[kTK], pb1[kTK], pb2[kTK], pb3[kTK];
  constexpr int kVsLen = C::kScaled && !C::kDmaFp8 ? kTK : 4;   // the fp8 DMA path keeps them in stage
  __shared__ __attribute__((aligned(16))) float vs0[kVsLen], vs1[kVsLen], vs2[kVsLen], vs3[kVsLen];
  __shared__ int32_t ids_l[kMaxSplitIds];
  // probabilities of the tile, row h: key slots in the k order of the PV product
  // (bf16 rows alternate two buffers: tile i's are written while tile i-1's are read)
  __shared__ __attribute__((aligned(16))) uint16_t p_l[kHMax * kTK];
  __shared__ __attribute__((aligned(16))) uint16_t p_l1[C::kDma ? kHMax * kTK : 8];
  __shared__ float mref_l[kHMax], lsum_l[kHMax];
  __shared__ int redo_l;
  // target of one DMA issued before any tile: the compiler's bookkeeping of
  // LDS DMA targets treats the first target it meets as aliasing later DMA,
  // so that role goes to a buffer the loop never reads
  __shared__ __attribute__((aligned(16))) uint8_t dma_first_l[16 * kWave];
  __shared__ float cos_l[D / 2], sin_l[D / 2];

  // The argument block is fresh memory at every launch: its scalar fields fill
  // its first four cache lines, fetched here together (one round trip rather
  // than one per line at first use).
  asm volatile("" ::"s"(splits), "s"(a.Q), "s"(a.k), "s"(a.rope_dims), "s"(a.part_in));
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int l16 = lane & 15, g = lane >> 4;
  // workgroup id -> (sequence, split): the splits of a sequence get ids that
  // are equal mod 8, and workgroups are dealt to the 8 XCDs by id mod 8, so a
  // sequence's Q is fetched into one L2 once and its other splits hit it
  const int r = blockIdx.x >> 3;
  const int64_t b = (int64_t)(r / splits) * 8 + (blockIdx.x & 7);
  const int s = r % splits;
  if (b >= a.B) return;
  const bool dense = a.ids == nullptr;
  // the sequence's entry and window counts, loaded alongside Q (from a dummy
  // when absent, so that no load waits behind a branch)
  const int32_t* ne_p = dense && a.n_entries ? a.n_entries + b : &g_no_count;
  const int32_t* nw_p = a.n_window ? a.n_window + b : &g_no_count;
  const int32_t ne_v = *ne_p, nw_v = *nw_p;
  const int h = 16 * wave + l16;            // this lane's head
  const bool wave_on = 16 * wave < a.H;     // wave-uniform
  // Q fragment: B operand of S^T = K Q^T; lane holds Q[h][32ks + 8g .. +7]
  bf16x8_t qf[KS];
  {
    // (every lane loads, from row 0 when it has no head, so that the loads
    // are one straight run ahead of the counts' first use)
    const bool qok = wave_on && h < a.H;
    const uint16_t* qrow = a.Q + (b * a.H + (qok ? h : 0)) * D;
    uint4 qv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qv[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8_t, qok ? qv[ks] : make_uint4(0, 0, 0, 0));
  }
  int64_t n_sel;
  if (dense) {
    n_sel = a.n_entries ? (int64_t)ne_v : a.cache_rows;
    n_sel = n_sel < 0 ? 0 : (n_sel > a.cache_rows ? a.cache_rows : n_sel);
  } else {
    n_sel = a.k;
  }
  const int64_t n_win = !a.n_window ? (int64_t)a.W : (nw_v < 0 ? 0 : (nw_v > a.W ? (int64_t)a.W : (int64_t)nw_v));
  const int64_t n_keys = n_sel + n_win;
  const int64_t lo = (int64_t)s * keys_per_split;
  const int64_t hi = lo + keys_per_split < n_keys ? lo + keys_per_split : n_keys;
  const int n_tiles = hi > lo ? (int)((hi - lo + kTK - 1) / kTK) : 0;
  const float tau_log2e = a.softmax_scale * kLog2e;
  // the split's entry ids (sparse)
  if (!dense) {
    const int64_t n_ids = min(hi, n_sel) - lo;
    for (int64_t j = t; j < n_ids; j += kAttThreads) ids_l[j] = a.ids[b * a.k + lo + j];
  }
  if (t == 0) redo_l = 0;
  // rows of heads without a computing wave stay zero
  for (int j = t; j < kHMax * kTK / 8; j += kAttThreads) {
    reinterpret_cast<uint4*>(p_l)[j] = make_uint4(0, 0, 0, 0);
    if constexpr (C::kDma) reinterpret_cast<uint4*>(p_l1)[j] = make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // LDS read offsets (bf16 elements) that do not depend on the tile.
  // QK^T A operand: row l16 (and 16 + l16), logical chunk 4ks + g.
  const int qk_off0 = l16 * KROW + 8 * (g ^ chunk_swz(l16));
  const int qk_off1 = (16 + l16) * KROW + 8 * (g ^ chunk_swz(16 + l16));
  // PV A operand by transposing reads: lane l16 of group g supplies 4 channels
  // c0 + 4(l16 % 4) .. +3 of row kbase + l16/4, so that lane l16 receives
  // channel c0 + l16 of rows kbase .. kbase+3 (kbase = 4g, then 16 + 4g). The
  // logical chunk of channel 16ct + 4tq is 2ct + (tq >> 1); with ct = 2m + e
  // the swizzled chunk is 4m + ((2e + (tq >> 1)) ^ swz(row)).
  const int tq = l16 & 3, tr_r = l16 >> 2;
  const int tr_row0 = 4 * g + tr_r, tr_row1 = 16 + 4 * g + tr_r;
  // this wave's channel tiles are ct = CTW * wave + j, j < CTW
  int tr_base0[2], tr_base1[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    tr_base0[e] = tr_row0 * KROW + 8 * ((2 * e + (tq >> 1)) ^ chunk_swz(tr_row0)) + 4 * (tq & 1) + 16 * CTW * wave;
    tr_base1[e] = tr_row1 * KROW + 8 * ((2 * e + (tq >> 1)) ^ chunk_swz(tr_row1)) + 4 * (tq & 1) + 16 * CTW * wave;
  }
  // P^T B operand of head tile ht: lane (l16, g) reads row 16 ht + l16, slots 8g .. 8g+7
  const int p_off = l16 * kTK + 8 * g;

  const RowSrc rsrc = row_src<D, CF, WFP8>(a, b);

  // ring slot S: bf16 tile, staging tile, slot scales
  auto tile_of = [&](auto sc) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (C::kDmaFp8) return (S & 1) ? tile1 : tile0;
    else return S == 0 ? tile0 : (S == 1 ? tile1 : (S == 2 ? tile2 : tile3));
  };
  auto stage_of = [&](auto sc) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(sc)::value;
    return S == 0 ? stage0 : (S == 1 ? stage1 : (S == 2 ? stage2 : stage3));
  };
  auto pb_of = [&](auto sc) __attribute__((always_inline)) -> float* {
    constexpr int S = decltype(sc)::value;
    return S == 0 ? pb0 : (S == 1 ? pb1 : (S == 2 ? pb2 : pb3));
  };
  auto vs_of = [&](auto sc) __attribute__((always_inline)) -> float* {
    constexpr int S = decltype(sc)::value;
    if constexpr (C::kDmaFp8) return reinterpret_cast<float*>(stage_of(sc) + kTK * D);
    else return S == 0 ? vs0 : (S == 1 ? vs1 : (S == 2 ? vs2 : vs3));
  };
  auto issue = [&](auto sc, int i) __attribute__((always_inline)) {
    issue_tile<D, CF, WFP8>(rsrc, lo + (int64_t)i * kTK, lo, n_sel, n_keys, dense, ids_l, tile_of(sc),
                              stage_of(sc), pb_of(sc), vs_of(sc), wave, lane);
  };
  // Softmax state of head h: probabilities are exp2(logit - m_ref) with m_ref
  // fixed for a pass; m_seen is the largest logit this lane saw and l_run the
  // sum of this lane's probabilities (the four lanes of a head are summed at
  // the end).
  float m_ref = 0.0f, m_seen, l_run;
  f32x4_t acc[CTW][4];   // O^T[16 (CTW wave + j) + 4g + i][16 ht + l16]

  // QK^T and softmax of this wave's 16 heads on a ready bf16 tile with its slot
  // biases and value scales; the probabilities go to p_l
  auto qk_softmax = [&](const uint16_t* kt, const float* pbv, const float* vsv, uint16_t* pw) __attribute__((always_inline)) {
    // slot metadata of keys 4g .. 4g+3 and 16+4g .. 16+4g+3 (same for all heads)
    const float4 b_lo = *reinterpret_cast<const float4*>(pbv + 4 * g);
    const float4 b_hi = *reinterpret_cast<const float4*>(pbv + 16 + 4 * g);
    float4 v_lo = make_float4(1.0f, 1.0f, 1.0f, 1.0f), v_hi = v_lo;
    if constexpr (C::kScaled) {
      v_lo = *reinterpret_cast<const float4*>(vsv + 4 * g);
      v_hi = *reinterpret_cast<const float4*>(vsv + 16 + 4 * g);
    }
    // S^T = K Q^T, with the LDS reads of the key rows kQD k-steps ahead of use
    constexpr int kQD = 4;
    bf16x8_t ka0[KS], ka1[KS];
#pragma unroll
    for (int ks = 0; ks < kQD; ++ks) {
      ka0[ks] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off0 + 32 * ks);
      ka1[ks] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off1 + 32 * ks);
    }
    f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + kQD < KS) {
        ka0[ks + kQD] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off0 + 32 * (ks + kQD));
        ka1[ks + kQD] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off1 + 32 * (ks + kQD));
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[ks], qf[ks], s1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds the logits of head h for key slots 4g+i (s0) and 16+4g+i (s1)
    const float bb[8] = {b_lo.x, b_lo.y, b_lo.z, b_lo.w, b_hi.x, b_hi.y, b_hi.z, b_hi.w};
    const float vv[8] = {v_lo.x, v_lo.y, v_lo.z, v_lo.w, v_hi.x, v_hi.y, v_hi.z, v_hi.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = C::kScaled ? fmaf(s0[i] * vv[i], tau_log2e, bb[i]) : fmaf(s0[i], tau_log2e, bb[i]);
      x[4 + i] = C::kScaled ? fmaf(s1[i] * vv[4 + i], tau_log2e, bb[4 + i]) : fmaf(s1[i], tau_log2e, bb[4 + i]);
    }
    m_seen = fmaxf(m_seen, fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                 fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);   // exp2(-inf) = 0 for empty slots
      l_run += p[i];
      if constexpr (C::kScaled) p[i] *= vv[i];
    }
    // k slot j of group g is key 4g+j (j < 4) or 16+4g+j-4: the lane's 8 values in order
    uint4 pq;
    pq.x = pack_bf16x2(p[0], p[1]);
    pq.y = pack_bf16x2(p[2], p[3]);
    pq.z = pack_bf16x2(p[4], p[5]);
    pq.w = pack_bf16x2(p[6], p[7]);
    *reinterpret_cast<uint4*>(pw + 16 * wave * kTK + p_off) = pq;
  };

  // raw rows: this thread's share of the next tile, read before this tile's
  // PV products and written back widened between them
  typename RawOf<CF>::type raw;

  // O^T[this wave's channels x 64 heads] += K^T P^T on a ready tile whose
  // probabilities are in p_l; with WIDEN, write slice j of the next raw tile
  // (held in `raw`, at nt) after the products of channel tile j if `on`
  auto pv = [&](const uint16_t* kt, auto widen, uint16_t* nt, bool on) __attribute__((always_inline)) {
    constexpr bool WIDEN = decltype(widen)::value;
    bf16x8_t pb[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) pb[ht] = *reinterpret_cast<const bf16x8_t*>(p_l + 16 * ht * kTK + p_off);
    constexpr int kPD = CTW < 3 ? CTW : 3;   // channel tiles read ahead
    v4i16_t kr0[CTW], kr1[CTW];
    auto read_kt = [&](int j) __attribute__((always_inline)) {
      const int e = j & 1, m = j >> 1;
      kr0[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kt + tr_base0[e] + 32 * m));
      kr1[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kt + tr_base1[e] + 32 * m));
    };
#pragma unroll
    for (int j = 0; j < kPD; ++j) read_kt(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      if (j + kPD < CTW) read_kt(j + kPD);
      const v4i16_t kk[2] = {kr0[j], kr1[j]};
      const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, kk);
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[j][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, pb[ht], acc[j][ht], 0, 0, 0);
      if constexpr (WIDEN) {
        static_assert(CTW == 8, "one widening slice per channel tile");
        raw_write<D>(nt, raw, j, on);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // one ring step: tile i sits in ring slot S = i mod 4
  auto step = [&](auto sc, int i) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    if (i >= n_tiles) return;
    // (raw rows: tile i was waited for and widened in the previous step)
    wait_tile<C::kOpsPerTile>(min(kNStage - 2, n_tiles - 1 - i));
    lds_barrier();   // tile i visible to all waves; ring slot S-1 free again
    if (i + kNStage - 1 < n_tiles) issue(std::integral_constant<int, (S + kNStage - 1) % kNStage>{}, i + kNStage - 1);
    if constexpr (C::kDmaFp8) {
      widen_tile<D>(stage_of(sc), tile_of(sc));
      lds_barrier();
    }
    // raw rows: wave w widens rows 8w .. 8w+7 of tile i+1, the ones its own
    // DMA brought (tiles i+2, i+3 may still be in flight behind it): it reads
    // them before this tile's QK^T and writes them back under its PV
    // products; the next step's barrier shows them. One PV body either way
    // (the last tile reads its successor's slot and writes nothing), so the
    // accumulators keep their registers.
    constexpr int SN = (S + 1) % kNStage;
    const bool nxt = i + 1 < n_tiles;
    if constexpr (C::kDmaRaw) {
      if (nxt) wait_tile<C::kOpsPerTile>(min(kNStage - 2, n_tiles - 2 - i));
      raw_read<D>(tile_of(std::integral_constant<int, SN>{}), raw);
    }
    if (wave_on) qk_softmax(tile_of(sc), pb_of(sc), vs_of(sc), p_l);
    lds_barrier();   // probabilities of all heads visible
    if constexpr (C::kDmaRaw) {
      pv(tile_of(sc), std::true_type{}, tile_of(std::integral_constant<int, SN>{}), nxt);
    } else {
      pv(tile_of(sc), std::false_type{}, nullptr, false);
    }
  };

  // bf16 rows, software-pipelined: step i runs QK^T and the softmax of tile i
  // with the PV products of tile i-1 interleaved (the matrix cores take PV while
  // LDS serves QK^T's row reads), one barrier a step. Tiles move two ahead: the
  // slot of tile i-2, whose PV ended in step i-1, takes tile i+2. Step i writes
  // its probabilities to buffer i % 2 and reads tile i-1's from the other.
  auto p_buf = [&](auto par) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(par)::value == 0) return p_l;
    else return p_l1;
  };
  auto qk_pv = [&](const uint16_t* kt, const float* pbv, const uint16_t* kp, const uint16_t* pr,
                   uint16_t* pw) __attribute__((always_inline)) {
    const float4 b_lo = *reinterpret_cast<const float4*>(pbv + 4 * g);
    const float4 b_hi = *reinterpret_cast<const float4*>(pbv + 16 + 4 * g);
    bf16x8_t pbo[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) pbo[ht] = *reinterpret_cast<const bf16x8_t*>(pr + 16 * ht * kTK + p_off);
    constexpr int kQD = 4;
    constexpr int kPD = 2;
    bf16x8_t ka0[KS], ka1[KS];
    v4i16_t kr0[CTW], kr1[CTW];
    auto read_kt = [&](int j) __attribute__((always_inline)) {
      const int e = j & 1, m = j >> 1;
      kr0[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kp + tr_base0[e] + 32 * m));
      kr1[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kp + tr_base1[e] + 32 * m));
    };
#pragma unroll
    for (int ks = 0; ks < kQD; ++ks) {
      ka0[ks] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off0 + 32 * ks);
      ka1[ks] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off1 + 32 * ks);
    }
#pragma unroll
    for (int j = 0; j < kPD; ++j) read_kt(j);
    f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
    static_assert(KS == 2 * CTW, "one PV channel tile per two QK^T k-steps");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + kQD < KS) {
        ka0[ks + kQD] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off0 + 32 * (ks + kQD));
        ka1[ks + kQD] = *reinterpret_cast<const bf16x8_t*>(kt + qk_off1 + 32 * (ks + kQD));
      }
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[ks], qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[ks], qf[ks], s1, 0, 0, 0);
      if (ks & 1) {
        const int j = ks >> 1;
        if (j + kPD < CTW) read_kt(j + kPD);
        const v4i16_t kk[2] = {kr0[j], kr1[j]};
        const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, kk);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) acc[j][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, pbo[ht], acc[j][ht], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const float bb[8] = {b_lo.x, b_lo.y, b_lo.z, b_lo.w, b_hi.x, b_hi.y, b_hi.z, b_hi.w};
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = fmaf(s0[i], tau_log2e, bb[i]);
      x[4 + i] = fmaf(s1[i], tau_log2e, bb[4 + i]);
    }
    m_seen = fmaxf(m_seen, fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                 fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);
      l_run += p[i];
    }
    uint4 pq;
    pq.x = pack_bf16x2(p[0], p[1]);
    pq.y = pack_bf16x2(p[2], p[3]);
    pq.z = pack_bf16x2(p[4], p[5]);
    pq.w = pack_bf16x2(p[6], p[7]);
    *reinterpret_cast<uint4*>(pw + 16 * wave * kTK + p_off) = pq;
  };
  // the PV products of the last tile alone, from probability buffer pr
  auto pv_only = [&](const uint16_t* kp, const uint16_t* pr) __attribute__((always_inline)) {
    bf16x8_t pbo[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) pbo[ht] = *reinterpret_cast<const bf16x8_t*>(pr + 16 * ht * kTK + p_off);
    v4i16_t kr0[CTW], kr1[CTW];
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const int e = j & 1, m = j >> 1;
      kr0[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kp + tr_base0[e] + 32 * m));
      kr1[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kp + tr_base1[e] + 32 * m));
    }
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const v4i16_t kk[2] = {kr0[j], kr1[j]};
      const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, kk);
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[j][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, pbo[ht], acc[j][ht], 0, 0, 0);
    }
  };
  // step i (i % 4 == S): tile i in slot S, tile i-1 in slot S-1. The first
  // step (FIRST, i = 0: QK^T and softmax alone) runs ahead of the loop, so
  // that the loop's four steps have one shape: with the first tile's path
  // inside step 0 the compiler gave that step a second accumulator bank and
  // copied 120 accumulators back after it, every fourth tile.
  auto pstep = [&](auto sc, auto first, int i) __attribute__((always_inline)) {
    constexpr int S = decltype(sc)::value;
    constexpr int SP = (S + kNStage - 1) % kNStage;
    constexpr bool FIRST = decltype(first)::value;
    if (i > n_tiles) return;
    if (i < n_tiles) wait_tile<C::kOpsPerTile>(i + 1 < n_tiles ? 1 : 0);
    lds_barrier();   // tile i and probabilities i-1 visible; slot S+2 (tile i-2) free
    if (i + 2 < n_tiles) issue(std::integral_constant<int, (S + 2) % kNStage>{}, i + 2);
    uint16_t* pw = p_buf(std::integral_constant<int, S & 1>{});
    const uint16_t* pr = p_buf(std::integral_constant<int, (S & 1) ^ 1>{});
    if constexpr (FIRST) {
      if (i < n_tiles && wave_on) qk_softmax(tile_of(sc), pb_of(sc), vs_of(sc), pw);
    } else if (i < n_tiles && wave_on) {
      qk_pv(tile_of(sc), pb_of(sc), tile_of(std::integral_constant<int, SP>{}), pr, pw);
    } else {
      pv_only(tile_of(std::integral_constant<int, SP>{}), pr);
    }
  };

  // At most two passes over the split: the second only when some head's true
  // maximum lies too far from the reference maximum of the first.
  // (still in flight when the first tile wait retires it with everything older)
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(g_zero_row + 16 * lane),
                                   (__attribute__((address_space(3))) void*)dma_first_l, 16, 0, 0);
#pragma nounroll
  for (int pass = 0;; ++pass) {
    // prologue: the first tiles (two for bf16 rows, three otherwise), then the
    // accumulators are cleared while they land
    if (n_tiles > 0) issue(std::integral_constant<int, 0>{}, 0);
    if (n_tiles > 1) issue(std::integral_constant<int, 1>{}, 1);
    if (!C::kDma && n_tiles > 2) issue(std::integral_constant<int, 2>{}, 2);
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[j][ht] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    m_seen = -INFINITY;
    l_run = 0.0f;
    if constexpr (C::kDmaRaw) {
      // raw rows: the first tile is widened here, later ones under the
      // previous tile's PV products
      if (n_tiles > 0) {
        wait_tile<C::kOpsPerTile>(min(kNStage - 2, n_tiles - 1));
        widen_raw_tile<D, typename RawOf<CF>::type>(tile0);
      }
    }
    if (pass == 0 && splits == 1 && t < a.rope_dims / 2) {
      // the rotary table of a single split, while the first tiles are in flight
      sincos_rad(-(double)a.q_pos[b] * a.inv_freq[t], &sin_l[t], &cos_l[t]);
    }
    if constexpr (C::kDma) {
      pstep(std::integral_constant<int, 0>{}, std::true_type{}, 0);
      for (int i = 1; i <= n_tiles; i += kNStage) {
        pstep(std::integral_constant<int, 1>{}, std::false_type{}, i);
        pstep(std::integral_constant<int, 2>{}, std::false_type{}, i + 1);
        pstep(std::integral_constant<int, 3>{}, std::false_type{}, i + 2);
        pstep(std::integral_constant<int, 0>{}, std::false_type{}, i + 3);
      }
    } else {
      for (int i = 0; i < n_tiles; i += kNStage) {
        step(std::integral_constant<int, 0>{}, i);
        step(std::integral_constant<int, 1>{}, i + 1);
        step(std::integral_constant<int, 2>{}, i + 2);
        step(std::integral_constant<int, 3>{}, i + 3);
      }
    }
    // the head's largest logit over the split (every tile has landed: no DMA in flight)
    const float mh = max_xor32(max_xor16(m_seen));
    const bool redo = pass == 0 && wave_on && mh != -INFINITY &&
                      (mh > m_ref + kHeadroom || mh < m_ref - kHeadroom);
    if (__ballot(redo) && lane == 0) redo_l = 1;
    lds_barrier();   // votes visible; every wave is done with the ring
    if (redo_l == 0 || pass > 0) break;
    m_ref = mh != -INFINITY ? mh : 0.0f;
  }
  l_run = add_xor32(add_xor16(l_run));
  // every wave holds channels of all heads: share each head's reference and sum
  if (g == 0) {
    mref_l[h] = m_ref;
    lsum_l[h] = wave_on ? l_run : 0.0f;
  }
  __syncthreads();
  // for head tile ht, the lane holds channels 16 (CTW wave + j) + 4g .. +3 of
  // head 16 ht + l16
  if (splits == 1 && a.part_out) {
    // the call's partial in the public layout: values normalised by their own
    // sum, no rotation, then (reference maximum, sum) per head
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int hh = 16 * ht + l16;
      if (hh >= a.H) continue;
      const float L = lsum_l[hh];
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      float* prow = a.part_out + (b * a.H + hh) * D;
#pragma unroll
      for (int j = 0; j < CTW; ++j) {
        const f32x4_t v = acc[j][ht];
        *reinterpret_cast<float4*>(prow + 16 * (CTW * wave + j) + 4 * g) =
            make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      }
    }
    if (t < a.H) {
      reinterpret_cast<float2*>(a.part_out + a.B * a.H * D)[b * a.H + t] = make_float2(mref_l[t], lsum_l[t]);
    }
  } else if (splits == 1) {
    const int R = a.rope_dims;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int hh = 16 * ht + l16;
      if (hh >= a.H) continue;
      // with a partial over other keys: log-sum-exp weights of this call's
      // keys (wi) and of the partial (we, which also undoes its normalisation);
      // a side with sum 0 saw no key and takes no part
      float L = lsum_l[hh], wi = 1.0f, we = 0.0f;
      const float* erow = nullptr;
      if (a.part_in) {
        const float2 e = reinterpret_cast<const float2*>(a.part_in + a.B * a.H * D)[b * a.H + hh];
        if (e.y > 0.0f) {
          const float mi = mref_l[hh];
          const float M = L > 0.0f ? fmaxf(mi, e.x) : e.x;
          wi = L > 0.0f ? exp2f(mi - M) : 0.0f;
          we = exp2f(e.x - M) * e.y;
          L = L * wi + we;
          erow = a.part_in + (b * a.H + hh) * D;
        }
      }
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      wi *= inv;
      we *= inv;
      float* orow = a.O + (b * a.H + hh) * D;
#pragma unroll
      for (int j = 0; j < CTW; ++j) {
        const int c = 16 * (CTW * wave + j) + 4 * g;
        const f32x4_t v = acc[j][ht];
        float4 o = make_float4(v[0] * wi, v[1] * wi, v[2] * wi, v[3] * wi);
        if (erow) {
          const float4 ev = *reinterpret_cast<const float4*>(erow + c);
          o = make_float4(fmaf(ev.x, we, o.x), fmaf(ev.y, we, o.y), fmaf(ev.z, we, o.z), fmaf(ev.w, we, o.w));
        }
        if (c >= D - R) {
          const int q = (c - (D - R)) >> 1;
          const float c0 = cos_l[q], s0 = sin_l[q];
          o = make_float4(o.x * c0 - o.y * s0, o.x * s0 + o.y * c0, o.z, o.w);
        }
        if (c + 2 >= D - R) {
          const int q = (c + 2 - (D - R)) >> 1;
          const float c1 = cos_l[q], s1 = sin_l[q];
          o = make_float4(o.x, o.y, o.z * c1 - o.w * s1, o.z * s1 + o.w * c1);
        }
        *reinterpret_cast<float4*>(orow + c) = o;
      }
    }
  } else {
    // partial of (sequence, split), normalised by its own sum (a convex
    // combination of key rows) and rounded to bf16: 4-channel blocks
    // [wave][j][ht][lane] of 8 bytes, each store 512 B contiguous
    const int64_t part = b * splits + s;
    uint2* dst = reinterpret_cast<uint2*>(ws_acc) + (part * 4 + wave) * (CTW * 4 * kWave) + lane;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const float L = lsum_l[16 * ht + l16];
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
      for (int j = 0; j < CTW; ++j) {
        const f32x4_t v = acc[j][ht];
        dst[(j * 4 + ht) * kWave] = make_uint2(pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv));
      }
    }
    if (t < kHMax) reinterpret_cast<float2*>(ws_ml)[part * kHMax + t] = make_float2(mref_l[t], lsum_l[t]);
  }
}

// Log-sum-exp merge of a sequence's splits, then inverse RoPE. Workgroup
// (q, b) combines partial block q (a 16-channel tile of every head: 256
// blocks of 4 channels): thread t owns block t, i.e. head 16 (t / 64) + t % 16
// and channels 16q + 4 ((t % 64) / 16) .. +3. First, per head, the splits'
// reference maxima and sums are reduced to (M, L) by four groups of 64
// threads and each split's weight exp2(m_s - M) l_s / L is stored in LDS (the
// partials are normalised by their own sums l_s); then every thread loads its
// block of all splits at once and sums them weighted.
constexpr int kMergeMaxSplits = 256;

// U: partial blocks a thread loads at once (4, 8 or 16: the smallest that
// holds every split when there are at most 16, so that no load repeats another)
template <int D, int U>
__global__ __launch_bounds__(256) void k_attend_merge(int splits, const uint16_t* __restrict__ ws_acc,
                                                      const float* __restrict__ ws_ml, AttendArgs a) {
  constexpr int CTW = D / 64;
  extern __shared__ float w_l[];            // [splits][kHMax] weights
  __shared__ float mq_l[4][kHMax], lq_l[4][kHMax];
  __shared__ float cs_l[2][8];              // rotary cos/sin of this tile's (up to 8) pairs
  __shared__ float we_l[kHMax];             // weight of a partial over other keys (a.part_in)
  // workgroup id -> (sequence, channel tile) with a sequence's tiles on one
  // XCD (ids equal mod 8), the one whose L2 its splits' partials went through
  constexpr int NQ = D / 16;
  // the argument block's scalar lines, fetched together
  asm volatile("" ::"s"(splits), "s"(a.Q), "s"(a.k), "s"(a.rope_dims), "s"(a.part_in));
  const int rq = blockIdx.x >> 3;
  const int64_t b = (int64_t)(rq / NQ) * 8 + (blockIdx.x & 7);
  const int q = rq % NQ;                    // 16-channel tile: wave slice q / CTW, j = q % CTW
  if (b >= a.B) return;
  const int t = threadIdx.x;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + b * splits * kHMax;
  const int R = a.rope_dims;
  // rotary pairs of channels 16q .. 16q+15 that lie in the last R channels:
  // thread t < 8 takes pair t; its frequency and position load with the rest,
  // the angle's sine and cosine are taken once the weights are stored
  const int c_rot = 16 * q + 2 * t;
  const bool rot = t < 8 && c_rot >= D - R;
  double f_rot = 0.0;
  int64_t p_rot = 0;
  if (rot) {
    f_rot = a.inv_freq[(c_rot - (D - R)) >> 1];
    p_rot = a.q_pos[b];
  }
  // thread (grp, hh0) folds the (reference maximum, sum) pairs of head hh0
  // over splits grp, grp + 4, ..; the first kMlU of them (every split when
  // there are at most U) are loaded at once, ahead of the partials, and kept
  // for the weights
  const int hh0 = t & 63, grp = t >> 6;
  constexpr int kMlU = U / 4;
  float2 mlr[kMlU];
#pragma unroll
  for (int u = 0; u < kMlU; ++u) {
    const int sp = grp + 4 * u;
    mlr[u] = ml[(int64_t)(sp < splits ? sp : 0) * kHMax + hh0];
  }
  // the first U splits' blocks are loaded before the weights are known
  const int ht = t >> 6, lane = t & 63;
  const int hh = 16 * ht + (lane & 15);
  const int w = q / CTW, j = q % CTW;
  const uint2* src = reinterpret_cast<const uint2*>(ws_acc) + (((b * splits) * 4 + w) * CTW + j) * (4 * kWave) + t;
  const int64_t pstride = 4 * CTW * 4 * kWave;   // 4-channel blocks per partial
  uint2 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = src[(int64_t)(u < splits ? u : splits - 1) * pstride];
  {
    // A split that saw no key (ragged counts, -1 ids, an empty range) has sum
    // 0 and a reference maximum that says nothing about the logits: it takes
    // no part in M, L or the weights.
    float M = -INFINITY, L = 0.0f;
    auto fold = [&](float2 v) {
      if (!(v.y > 0.0f)) return;
      if (v.x > M) {
        L = (M == -INFINITY ? 0.0f : L * exp2f(M - v.x)) + v.y;
        M = v.x;
      } else {
        L += v.y * exp2f(v.x - M);
      }
    };
#pragma unroll
    for (int u = 0; u < kMlU; ++u) {
      if (grp + 4 * u < splits) fold(mlr[u]);
    }
    for (int sp = grp + 4 * kMlU; sp < splits; sp += 4) fold(ml[(int64_t)sp * kHMax + hh0]);
    // a partial over other keys counts as one more split (group 0 folds it)
    if (a.part_in && grp == 0 && hh0 < a.H) fold(reinterpret_cast<const float2*>(a.part_in + a.B * a.H * D)[b * a.H + hh0]);
    mq_l[grp][hh0] = M;
    lq_l[grp][hh0] = L;
  }
  __syncthreads();
  {
    float M = -INFINITY;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) M = fmaxf(M, mq_l[gg][hh0]);
    float L = 0.0f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const float mg = mq_l[gg][hh0];
      if (mg != -INFINITY) L += lq_l[gg][hh0] * exp2f(mg - M);
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    auto weight = [&](float2 v) { return v.y > 0.0f ? exp2f(v.x - M) * v.y * inv : 0.0f; };
#pragma unroll
    for (int u = 0; u < kMlU; ++u) {
      const int sp = grp + 4 * u;
      if (sp < splits) w_l[sp * kHMax + hh0] = weight(mlr[u]);
    }
    for (int sp = grp + 4 * kMlU; sp < splits; sp += 4) w_l[sp * kHMax + hh0] = weight(ml[(int64_t)sp * kHMax + hh0]);
    if (a.part_in && grp == 0) {
      we_l[hh0] = hh0 < a.H ? weight(reinterpret_cast<const float2*>(a.part_in + a.B * a.H * D)[b * a.H + hh0]) : 0.0f;
    }
  }
  if (rot) {
    // (opaque until here, so that no use of the two loads moves up to them)
    asm volatile("" : "+v"(p_rot), "+v"(f_rot));
    sincos_rad(-(double)p_rot * f_rot, &cs_l[1][t], &cs_l[0][t]);
  }
  __syncthreads();
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < splits; s0 += U) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sp = s0 + u < splits ? s0 + u : splits - 1;
        v[u] = src[(int64_t)sp * pstride];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wgt = s0 + u < splits ? w_l[(s0 + u) * kHMax + hh] : 0.0f;
      o.x = fmaf(__uint_as_float(v[u].x << 16), wgt, o.x);
      o.y = fmaf(__uint_as_float(v[u].x & 0xFFFF0000u), wgt, o.y);
      o.z = fmaf(__uint_as_float(v[u].y << 16), wgt, o.z);
      o.w = fmaf(__uint_as_float(v[u].y & 0xFFFF0000u), wgt, o.w);
    }
  }
  if (hh >= a.H) return;
  const int c = 16 * q + 4 * (lane >> 4);
  if (a.part_in) {
    const float we = we_l[hh];
    if (we > 0.0f) {
      const float4 ev = *reinterpret_cast<const float4*>(a.part_in + (b * a.H + hh) * D + c);
      o = make_float4(fmaf(ev.x, we, o.x), fmaf(ev.y, we, o.y), fmaf(ev.z, we, o.z), fmaf(ev.w, we, o.w));
    }
  }
  // (the weights already divide by L)
  if (c >= D - R) {
    const int pr = (c - 16 * q) >> 1;
    const float c0 = cs_l[0][pr], s0 = cs_l[1][pr];
    o = make_float4(o.x * c0 - o.y * s0, o.x * s0 + o.y * c0, o.z, o.w);
  }
  if (c + 2 >= D - R) {
    const int pr = (c + 2 - 16 * q) >> 1;
    const float c1 = cs_l[0][pr], s1 = cs_l[1][pr];
    o = make_float4(o.x, o.y, o.z * c1 - o.w * s1, o.z * s1 + o.w * c1);
  }
  *reinterpret_cast<float4*>(a.O + (b * a.H + hh) * D + c) = o;
}

// ------------------------------------------------------------- planning / launch

bool plan_attend(int64_t B, int H, int D, int64_t max_keys, bool sparse, int splits_hint, AttendPlan* p) {
  const int64_t tiles = max_keys <= 0 ? 1 : (max_keys + kTK - 1) / kTK;
  int64_t splits = splits_hint;
  if (splits <= 0) {
    // about one workgroup per compute unit
    splits = (256 + B - 1) / B;
    if (splits > 64) splits = 64;
  }
  if (sparse) {
    // a sparse split stages at most kMaxSplitIds entry ids in LDS
    const int64_t min_splits = (tiles + kMaxSplitIds / kTK - 1) / (kMaxSplitIds / kTK);
    if (min_splits > kMergeMaxSplits) return false;
    if (splits < min_splits) splits = min_splits;
  }
  if (splits > kMergeMaxSplits) splits = kMergeMaxSplits;
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int64_t tiles_per = (tiles + splits - 1) / splits;
  splits = (tiles + tiles_per - 1) / tiles_per;
  p->splits = (int)splits;
  p->keys_per_split = tiles_per * kTK;
  // workspace: bf16 partials, then an fp32 (reference maximum, sum) pair per head
  p->bytes = splits > 1 ? (size_t)B * splits * kHMax * ((size_t)D * 2 + 8) : 0;
  return true;
}

template <int D, int CF, bool WFP8>
static hipError_t launch_attend_t(const AttendPlan& p, const AttendArgs& a, void* workspace,
                                  hipStream_t stream) {
  auto kern = k_attend<D, CF, WFP8>;
  uint16_t* ws_acc = reinterpret_cast<uint16_t*>(workspace);
  float* ws_ml = p.splits > 1 ? reinterpret_cast<float*>(ws_acc + (size_t)a.B * p.splits * kHMax * D) : nullptr;
  const int64_t b8 = 8 * ((a.B + 7) / 8);   // sequences padded to whole XCD rounds
  hipLaunchKernelGGL(kern, dim3((unsigned)(b8 * p.splits)), dim3(kAttThreads), 0, stream, p.splits,
                     p.keys_per_split, ws_acc, ws_ml, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const dim3 mgrid((unsigned)(b8 * (D / 16)));
  const size_t mlds = (size_t)p.splits * kHMax * sizeof(float);
  if (p.splits <= 4)
    hipLaunchKernelGGL((k_attend_merge<D, 4>), mgrid, dim3(256), mlds, stream, p.splits, ws_acc, ws_ml, a);
  else if (p.splits <= 8)
    hipLaunchKernelGGL((k_attend_merge<D, 8>), mgrid, dim3(256), mlds, stream, p.splits, ws_acc, ws_ml, a);
  else
    hipLaunchKernelGGL((k_attend_merge<D, 16>), mgrid, dim3(256), mlds, stream, p.splits, ws_acc, ws_ml, a);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendPlan& p, const AttendArgs& a, void* workspace,
                         hipStream_t stream) {
  if (a.D == 512) {
    // The variant follows the rows the call reads: without cache rows (a
    // window-only partial) the cache's format is moot, and without window rows
    // (entries only) the window's, so such calls take the DMA variant of the
    // one format they read rather than a mixed one that fills tiles through
    // registers.
    const bool no_cache = a.ids ? a.k == 0 : a.cache_rows == 0;
    if (no_cache) return a.win_fp8 && a.W > 0 ? launch_attend_t<512, kFmtFp8, true>(p, a, workspace, stream)
                                              : launch_attend_t<512, kFmtBf16, false>(p, a, workspace, stream);
    if (a.W == 0 && a.cache_fp8) return launch_attend_t<512, kFmtFp8, true>(p, a, workspace, stream);
    if (a.cache_mix) return a.win_fp8 ? launch_attend_t<512, kFmtMix, true>(p, a, workspace, stream)
                                      : launch_attend_t<512, kFmtMix, false>(p, a, workspace, stream);
    if (a.cache_fp4) return a.win_fp8 ? launch_attend_t<512, kFmtFp4, true>(p, a, workspace, stream)
                                      : launch_attend_t<512, kFmtFp4, false>(p, a, workspace, stream);
    if (a.cache_fp8) return a.win_fp8 ? launch_attend_t<512, kFmtFp8, true>(p, a, workspace, stream)
                                      : launch_attend_t<512, kFmtFp8, false>(p, a, workspace, stream);
    return a.win_fp8 ? launch_attend_t<512, kFmtBf16, true>(p, a, workspace, stream)
                     : launch_attend_t<512, kFmtBf16, false>(p, a, workspace, stream);
  }
  if (a.cache_fp8) return a.win_fp8 ? launch_attend_t<128, kFmtFp8, true>(p, a, workspace, stream)
                                    : launch_attend_t<128, kFmtFp8, false>(p, a, workspace, stream);
  return a.win_fp8 ? launch_attend_t<128, kFmtBf16, true>(p, a, workspace, stream)
                   : launch_attend_t<128, kFmtBf16, false>(p, a, workspace, stream);
}

}  // namespace cskv
