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
// and run on 16x16x32 bf16 MFMA. A workgroup (4 waves) owns one sequence and a
// contiguous split of its key slots; wave w owns heads 16w .. 16w+15. Per tile
// of 32 key slots:
//   1. the rows reach LDS one tile ahead of their use: bf16 rows of 1 KiB by
//      direct HBM->LDS DMA (non-temporal, no registers), fp8 rows by DMA into
//      a staging buffer and one cooperative pass that widens the codes to bf16
//      exactly (an fp8 row's scale is folded into its logits and
//      probabilities); other shapes through registers. Entry ids of sparse
//      reads are fetched one tile earlier still, so no DMA waits on an id;
//   2. S^T[32 keys x 16 heads] = K Q^T with Q held in registers;
//   3. online softmax per head in the exp2 domain; the running maximum is
//      raised only when a logit exceeds it by more than 2^8, so the
//      accumulators are rescaled rarely;
//   4. O^T[D x 16 heads] += K^T P^T: the probabilities stay in the registers
//      the QK^T product left them in (they are exactly the B operand, for a
//      matching order of the 32 keys), and K^T comes from the row-major tile
//      through gfx950's transposing LDS reads.
// Tile rows are padded to a stride of 8 (mod 64) dwords and their 16-byte
// chunks are XOR-swizzled by (row / 8) mod 4, which keeps both the row reads of
// QK^T and the transposing reads of PV free of LDS bank conflicts.
// Each lane ends with 4 consecutive channels of one head: rotary pairs sit in
// one lane. With one split the epilogue normalises, applies inverse RoPE and
// stores O; otherwise partials (max, sum, unnormalised O) go to the workspace
// and k_attend_merge combines them with a log-sum-exp merge.
#include <type_traits>

#include "kernels.h"

namespace cskv {

constexpr int kAttThreads = 256;
constexpr int kTK = 32;        // key slots per tile
constexpr int kHMax = 64;      // heads per workgroup (4 waves x 16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescale = 8.0f;   // log2 headroom before the running max is raised
constexpr int kCachePolicyStream = 2;  // non-temporal loads for rows read once

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Swizzle of a tile row's 16-byte chunks.
__device__ __forceinline__ int chunk_swz(int row) { return (row >> 3) & 3; }

template <int D, bool CFP8, bool WFP8>
struct AttLayout {
  static constexpr bool kAllFp8 = CFP8 && WFP8;
  static constexpr bool kDma = D == 512 && !CFP8 && !WFP8;      // bf16 rows by DMA
  static constexpr bool kDmaFp8 = D == 512 && kAllFp8;          // fp8 rows by DMA + widening pass
  static constexpr int KROW = D + 16;                           // bf16 per tile row
  static constexpr int NBUF = kDmaFp8 ? 1 : 2;                  // bf16 tiles
  static constexpr size_t tile_bytes = (size_t)kTK * KROW * 2;
  static constexpr size_t stage_bytes = kDmaFp8 ? (size_t)kTK * D : 0;   // fp8 rows, unpadded
  static constexpr size_t off_tile = 0;
  static constexpr size_t off_stage = NBUF * tile_bytes;                 // [2] staging tiles
  static constexpr size_t off_rs = off_stage + 2 * stage_bytes;          // [2][kTK] logit factor per slot
  static constexpr size_t off_ps = off_rs + 2 * kTK * 4;                 // [2][kTK] value scale (-inf: empty)
  static constexpr size_t off_cos = off_ps + 2 * kTK * 4;
  static constexpr size_t off_sin = off_cos + (D / 2) * 4;
  static constexpr size_t bytes = off_sin + (D / 2) * 4;
};

// Where a slot's row lives: pointer (nullptr for an empty slot - an id out of
// range, or past the last key) and its fp8 row scale (nullptr for bf16).
struct SlotRow {
  const uint8_t* ptr;
  const float* scale;
};

template <int D, bool CFP8, bool WFP8>
__device__ __forceinline__ SlotRow slot_row(const AttendArgs& a, int64_t b, int64_t slot, int64_t row_id,
                                            int64_t n_sel, int64_t n_keys) {
  SlotRow sr{nullptr, nullptr};
  if (slot >= n_keys) return sr;
  if (slot < n_sel) {
    if (row_id < 0 || row_id >= a.cache_rows) return sr;
    const int64_t r = b * a.cache_rows + row_id;
    sr.ptr = reinterpret_cast<const uint8_t*>(a.cache) + r * D * (CFP8 ? 1 : 2);
    sr.scale = CFP8 ? a.cache_scale + r : nullptr;
  } else {
    const int64_t r = b * a.win_bstride + (slot - n_sel);
    sr.ptr = reinterpret_cast<const uint8_t*>(a.window) + r * D * (WFP8 ? 1 : 2);
    sr.scale = WFP8 ? a.window_scale + r : nullptr;
  }
  return sr;
}

// Entry id of a slot (sparse: from ids; dense: the slot itself).
__device__ __forceinline__ int64_t slot_id(const AttendArgs& a, int64_t b, int64_t slot, int64_t n_sel,
                                           bool dense) {
  if (dense || slot >= n_sel || slot < 0) return slot;
  return (int64_t)a.ids[b * a.k + slot];
}

__device__ __forceinline__ void put_slot(uint8_t* lds, size_t off_rs, size_t off_ps, int buf, int j,
                                         float vs, float tau_log2e) {
  float* rs = reinterpret_cast<float*>(lds + off_rs) + buf * kTK;
  float* ps = reinterpret_cast<float*>(lds + off_ps) + buf * kTK;
  rs[j] = vs != -INFINITY ? vs * tau_log2e : 0.0f;
  ps[j] = vs;
}

__device__ __forceinline__ const uint8_t* lane_ptr(uint64_t p, int lane) {
  const uint32_t lo32 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)p, lane);
  const uint32_t hi32 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(p >> 32), lane);
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi32 << 32) | lo32);
}

// A tile row as lane j < 8 of wave w holds it for row 8w + j: its address and
// value scale (-inf for an empty slot), resolved one tile before its DMA so that
// issuing the DMA never waits on an id or scale load.
struct RowRef {
  uint64_t ptr;
  float vs;
};

template <int D, bool CFP8, bool WFP8>
__device__ __forceinline__ RowRef resolve_row(const AttendArgs& a, int64_t b, int64_t slot, int64_t row_id,
                                              int64_t n_sel, int64_t n_keys) {
  const SlotRow sr = slot_row<D, CFP8, WFP8>(a, b, slot, row_id, n_sel, n_keys);
  RowRef r;
  r.ptr = reinterpret_cast<uint64_t>(sr.ptr);
  r.vs = !sr.ptr ? -INFINITY : (sr.scale ? *sr.scale : 1.0f);
  return r;
}

// DMA fill of one tile: wave w moves rows 8w .. 8w+7 whose references lanes
// 0-7 hold. bf16 rows (1 KiB) go straight into their swizzled LDS row; fp8
// rows (512 B, two per wave instruction) go into the staging tile. Empty bf16
// rows are zeroed here, empty fp8 rows by the widening pass.
template <int D, bool CFP8, bool WFP8>
__device__ __forceinline__ void dma_tile(const RowRef& ref, uint8_t* lds, int buf, float tau_log2e, int wave,
                                         int lane) {
  using L = AttLayout<D, CFP8, WFP8>;
  const uint64_t p = lane < 8 ? ref.ptr : 0;
  if (lane < 8) put_slot(lds, L::off_rs, L::off_ps, buf, 8 * wave + lane, ref.vs, tau_log2e);
  if constexpr (L::kDma) {
    uint8_t* tile = lds + L::off_tile + buf * L::tile_bytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * wave + i;
      const uint8_t* src = lane_ptr(p, i);
      uint8_t* row = tile + (size_t)r * L::KROW * 2;
      // lane l fills chunk position l, which holds logical chunk l ^ swz(r)
      if (src) {
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(src + 16 * (lane ^ chunk_swz(r))),
            (__attribute__((address_space(3))) void*)row, 16, 0, kCachePolicyStream);
      } else {
        *reinterpret_cast<uint4*>(row + 16 * lane) = make_uint4(0, 0, 0, 0);
      }
    }
  } else {
    static_assert(L::kDmaFp8, "DMA fill needs bf16 or fp8 rows of D = 512");
    uint8_t* stage = lds + L::off_stage + buf * L::stage_bytes;
    const int half = lane >> 5, hl = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // lanes 0-31 move row 2i, lanes 32-63 row 2i+1 (readlane needs a uniform lane)
      const uint8_t* src_even = lane_ptr(p, 2 * i);
      const uint8_t* src_odd = lane_ptr(p, 2 * i + 1);
      const uint8_t* src = half ? src_odd : src_even;
      if (src) {
        __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src + 16 * hl),
                                         (__attribute__((address_space(3))) void*)(stage + (8 * wave + 2 * i) * D),
                                         16, 0, kCachePolicyStream);
      }
    }
  }
}

// Widens a staged fp8 tile into the bf16 tile: thread t converts 64 codes of
// row t/8 (logical chunks 8(t%8) .. 8(t%8)+7); empty slots become zeros.
template <int D>
__device__ __forceinline__ void widen_tile(uint8_t* lds, int buf) {
  using L = AttLayout<D, true, true>;
  const int t = threadIdx.x;
  const int r = t >> 3, part = t & 7;
  const uint8_t* stage = lds + L::off_stage + buf * L::stage_bytes + r * D + part * 64;
  const float* ps = reinterpret_cast<const float*>(lds + L::off_ps) + buf * kTK;
  const bool empty = ps[r] == -INFINITY;
  uint4 c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = *reinterpret_cast<const uint4*>(stage + 16 * j);
  uint16_t* row = reinterpret_cast<uint16_t*>(lds + L::off_tile) + r * L::KROW;
  const int swz = chunk_swz(r);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint4 lo = fp8x8_to_bf16x8(make_uint2(c[j].x, c[j].y));
    uint4 hi = fp8x8_to_bf16x8(make_uint2(c[j].z, c[j].w));
    if (empty) lo = hi = make_uint4(0, 0, 0, 0);
    const int ch0 = 8 * part + 2 * j;          // logical chunks ch0, ch0 + 1
    *reinterpret_cast<uint4*>(row + 8 * (ch0 ^ swz)) = lo;
    *reinterpret_cast<uint4*>(row + 8 * ((ch0 + 1) ^ swz)) = hi;
  }
}

// Register-staged fill (mixed cache/window dtypes, or D = 128): one thread's
// share is rows 8*kb .. 8*kb+7, logical chunk cb (8 channels), held as bf16.
struct TileRegs {
  uint4 r[8];
  float vs[8];     // value scale of the row (1 for bf16), or -inf for an empty slot
};

template <int D, bool CFP8, bool WFP8>
__device__ __forceinline__ void load_tile(const AttendArgs& a, int64_t b, int64_t slot0, int64_t n_sel,
                                          int64_t n_keys, bool dense, int kb, int cb, TileRegs& t) {
  const bool active_c = cb * 8 < D;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    t.r[i] = make_uint4(0, 0, 0, 0);
    t.vs[i] = -INFINITY;
    const int64_t slot = slot0 + 8 * kb + i;
    const SlotRow sr = slot_row<D, CFP8, WFP8>(a, b, slot, slot_id(a, b, slot, n_sel, dense), n_sel, n_keys);
    if (!sr.ptr) continue;
    t.vs[i] = sr.scale ? *sr.scale : 1.0f;
    if (!active_c) continue;
    if (sr.scale) t.r[i] = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(sr.ptr + cb * 8));
    else t.r[i] = *reinterpret_cast<const uint4*>(sr.ptr + cb * 16);
  }
}

template <int D, bool CFP8, bool WFP8>
__device__ __forceinline__ void store_tile(uint8_t* lds, int buf, int kb, int cb, const TileRegs& t,
                                           float tau_log2e) {
  using L = AttLayout<D, CFP8, WFP8>;
  uint16_t* tile = reinterpret_cast<uint16_t*>(lds + L::off_tile + buf * L::tile_bytes);
  if (cb * 8 < D) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * kb + i;
      *reinterpret_cast<uint4*>(tile + r * L::KROW + 8 * (cb ^ chunk_swz(r))) = t.r[i];
    }
  }
  if (cb == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) put_slot(lds, L::off_rs, L::off_ps, buf, 8 * kb + i, t.vs[i], tau_log2e);
  }
}

template <int D, bool CFP8, bool WFP8>
__global__ __launch_bounds__(kAttThreads, 2) void k_attend(AttendArgs a, int splits,
                                                          int64_t keys_per_split,
                                                          float* __restrict__ ws_acc,
                                                          float* __restrict__ ws_ml) {
  using L = AttLayout<D, CFP8, WFP8>;
  constexpr bool kAnyDma = L::kDma || L::kDmaFp8;
  constexpr int KS = D / 32;          // k-steps of QK^T
  constexpr int CT = D / 16;          // 16-channel tiles of O^T
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  float* cos_l = reinterpret_cast<float*>(lds + L::off_cos);
  float* sin_l = reinterpret_cast<float*>(lds + L::off_sin);

  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.y;
  const int s = blockIdx.x;
  const bool dense = a.ids == nullptr;
  int64_t n_sel;
  if (dense) {
    n_sel = a.n_entries ? (int64_t)a.n_entries[b] : a.cache_rows;
    n_sel = n_sel < 0 ? 0 : (n_sel > a.cache_rows ? a.cache_rows : n_sel);
  } else {
    n_sel = a.k;
  }
  const int64_t n_keys = n_sel + a.W;
  const int64_t lo = (int64_t)s * keys_per_split;
  const int64_t hi = lo + keys_per_split < n_keys ? lo + keys_per_split : n_keys;
  const float tau_log2e = a.softmax_scale * kLog2e;
  const int h = 16 * wave + l16;            // this lane's head
  const bool wave_on = 16 * wave < a.H;     // wave-uniform

  // rotary tables (fp64 angles), used by the single-split epilogue
  if (splits == 1 && t < a.rope_dims / 2) {
    const double theta = pow((double)a.rope_base, -2.0 * (double)t / (double)a.rope_dims);
    const double ang = -(double)a.q_pos[b] * theta;
    cos_l[t] = (float)cos(ang);
    sin_l[t] = (float)sin(ang);
  }

  // DMA paths: lane j < 8 of wave w tracks row 8w + j of the coming tiles:
  // ref1 (address and scale) for the next tile to fill, id2 for the one after.
  RowRef ref1{0, -INFINITY};
  int64_t id2 = 0;
  auto row_slot = [&](int64_t tile0) { return tile0 + 8 * wave + lane; };
  if (kAnyDma && lane < 8) {
    ref1 = resolve_row<D, CFP8, WFP8>(a, b, row_slot(lo), slot_id(a, b, row_slot(lo), n_sel, dense), n_sel,
                                      n_keys);
    id2 = slot_id(a, b, row_slot(lo + kTK), n_sel, dense);
  }
  // after a DMA of tile0 + kTK's predecessor: resolve tile0 + kTK, fetch the id of tile0 + 2 kTK
  auto advance = [&](int64_t tile0) {
    if (lane < 8) {
      ref1 = resolve_row<D, CFP8, WFP8>(a, b, row_slot(tile0 + kTK), id2, n_sel, n_keys);
      id2 = slot_id(a, b, row_slot(tile0 + 2 * kTK), n_sel, dense);
    }
  };

  // Q fragment: B operand of S^T = K Q^T; lane holds Q[h][32ks + 8g .. +7]
  bf16x8_t qf[KS];
  {
    const bool qok = wave_on && h < a.H;
    const uint16_t* qrow = a.Q + (b * a.H + (qok ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = qok ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  // LDS read offsets (bf16 elements) that do not depend on the tile.
  // QK^T A operand: row l16 (and 16 + l16), logical chunk 4ks + g.
  const int qk_off0 = l16 * L::KROW + 8 * (g ^ chunk_swz(l16));
  const int qk_off1 = (16 + l16) * L::KROW + 8 * (g ^ chunk_swz(16 + l16));
  // PV A operand by transposing reads: lane l16 of group g supplies 4 channels
  // c0 + 4(l16 % 4) .. +3 of row kbase + l16/4, so that lane l16 receives
  // channel c0 + l16 of rows kbase .. kbase+3 (kbase = 4g, then 16 + 4g).
  const int tq = l16 & 3, tr_r = l16 >> 2;
  const int tr_row0 = 4 * g + tr_r, tr_row1 = 16 + 4 * g + tr_r;
  // logical chunk of channel 16ct + 4tq is 2ct + (tq >> 1); with ct = 2m + e the
  // swizzled chunk is 4m + ((2e + (tq >> 1)) ^ swz(row))
  int tr_base0[2], tr_base1[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    tr_base0[e] = tr_row0 * L::KROW + 8 * ((2 * e + (tq >> 1)) ^ chunk_swz(tr_row0)) + 4 * (tq & 1);
    tr_base1[e] = tr_row1 * L::KROW + 8 * ((2 * e + (tq >> 1)) ^ chunk_swz(tr_row1)) + 4 * (tq & 1);
  }

  const int kb = t >> 6, cb = t & 63;
  TileRegs tr;
  if (lo < hi) {
    if constexpr (kAnyDma) {
      dma_tile<D, CFP8, WFP8>(ref1, lds, 0, tau_log2e, wave, lane);
      advance(lo);
    } else {
      load_tile<D, CFP8, WFP8>(a, b, lo, n_sel, n_keys, dense, kb, cb, tr);
      store_tile<D, CFP8, WFP8>(lds, 0, kb, cb, tr, tau_log2e);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (L::kDmaFp8) {
    if (lo < hi) widen_tile<D>(lds, 0);
    __syncthreads();
  }

  int buf = 0;
  for (int64_t tile = lo; tile < hi; tile += kTK) {
    const bool more = tile + kTK < hi;
    if (more) {
      // the other buffer was last read before the previous barrier
      if constexpr (kAnyDma) {
        dma_tile<D, CFP8, WFP8>(ref1, lds, buf ^ 1, tau_log2e, wave, lane);
        advance(tile + kTK);
      } else {
        load_tile<D, CFP8, WFP8>(a, b, tile + kTK, n_sel, n_keys, dense, kb, cb, tr);
      }
    }

    if (wave_on) {
      const int cur = L::kDmaFp8 ? 0 : buf;
      const uint16_t* kt = reinterpret_cast<const uint16_t*>(lds + L::off_tile + cur * L::tile_bytes);
      const float* rs = reinterpret_cast<const float*>(lds + L::off_rs) + buf * kTK;
      const float* ps = reinterpret_cast<const float*>(lds + L::off_ps) + buf * kTK;
      f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kt + qk_off0 + 32 * ks);
        const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kt + qk_off1 + 32 * ks);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
        if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // bound the loads kept in flight
      }
      // lane holds the logits of head h for key slots 4g+i (s0) and 16+4g+i (s1)
      float x[8], vsc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j0 = 4 * g + i, j1 = 16 + 4 * g + i;
        vsc[i] = ps[j0];
        vsc[4 + i] = ps[j1];
        x[i] = vsc[i] != -INFINITY ? s0[i] * rs[j0] : -INFINITY;
        x[4 + i] = vsc[4 + i] != -INFINITY ? s1[i] * rs[j1] : -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const bool raise = mx > m_run + kLazyRescale || (m_run == -INFINITY && mx != -INFINITY);
      if (__ballot(raise)) {
        const float alpha = raise ? (m_run == -INFINITY ? 0.0f : exp2f(m_run - mx)) : 1.0f;
        if (raise) m_run = mx;
        l_run *= alpha;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[ct][i] *= alpha;
        }
      }
      float p[8], lsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = x[i] == -INFINITY ? 0.0f : exp2f(x[i] - m_run);
        lsum += p[i];
      }
      lsum += __shfl_xor(lsum, 16, kWave);
      lsum += __shfl_xor(lsum, 32, kWave);
      l_run += lsum;
      // P^T as the B operand: k-slot j of group g is key 4g+j (j < 4) or 16+4g+j-4
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = p[i] == 0.0f ? 0.0f : p[i] * vsc[i];
      uint4 pw;
      pw.x = pack_bf16x2(pv[0], pv[1]);
      pw.y = pack_bf16x2(pv[2], pv[3]);
      pw.z = pack_bf16x2(pv[4], pv[5]);
      pw.w = pack_bf16x2(pv[6], pv[7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int e = ct & 1, m = ct >> 1;
        const v4i16_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kt + tr_base0[e] + 32 * m));
        const v4i16_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kt + tr_base1[e] + 32 * m));
        const v4i16_t kk[2] = {r0, r1};
        const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, kk);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, pb, acc[ct], 0, 0, 0);
        if ((ct & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!kAnyDma) {
      if (more) store_tile<D, CFP8, WFP8>(lds, buf ^ 1, kb, cb, tr, tau_log2e);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the next tile's rows have landed in LDS
    __syncthreads();
    if constexpr (L::kDmaFp8) {
      if (more) widen_tile<D>(lds, buf ^ 1);
      __syncthreads();
    }
    buf ^= 1;
  }

  if (!wave_on) return;
  // lane holds O^T[16ct + 4g + i][h]: channels 16ct+4g .. 16ct+4g+3 of head h
  if (splits == 1) {
    const int R = a.rope_dims;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    if (h < a.H) {
      float* orow = a.O + (b * a.H + h) * D;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + 4 * g;
        float4 o = make_float4(acc[ct][0] * inv, acc[ct][1] * inv, acc[ct][2] * inv, acc[ct][3] * inv);
        if (c >= D - R) {
          const int j = (c - (D - R)) >> 1;
          const float c0 = cos_l[j], s0 = sin_l[j];
          o = make_float4(o.x * c0 - o.y * s0, o.x * s0 + o.y * c0, o.z, o.w);
        }
        if (c + 2 >= D - R) {
          const int j = (c + 2 - (D - R)) >> 1;
          const float c1 = cos_l[j], s1 = sin_l[j];
          o = make_float4(o.x, o.y, o.z * c1 - o.w * s1, o.z * s1 + o.w * c1);
        }
        *reinterpret_cast<float4*>(orow + c) = o;
      }
    }
  } else {
    const int64_t part = b * splits + s;
    if (h < a.H) {
      float* arow = ws_acc + (part * kHMax + h) * D;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c = 16 * ct + 4 * g;
        *reinterpret_cast<float4*>(arow + c) = make_float4(acc[ct][0], acc[ct][1], acc[ct][2], acc[ct][3]);
      }
      if (g == 0) *reinterpret_cast<float2*>(ws_ml + (part * kHMax + h) * 2) = make_float2(m_run, l_run);
    }
  }
}

// Log-sum-exp merge of the splits of one (sequence, head), then inverse RoPE.
// Thread t owns channels 4t .. 4t+3.
template <int D>
__global__ __launch_bounds__(128) void k_attend_merge(AttendArgs a, int splits,
                                                      const float* __restrict__ ws_acc,
                                                      const float* __restrict__ ws_ml) {
  const int64_t b = blockIdx.y;
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  if (4 * t >= D) return;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml) + (b * splits) * kHMax + h;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[(int64_t)s * kHMax].x);
  float Lsum = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (M != -INFINITY) {
    const float* base = ws_acc + ((b * splits) * kHMax + h) * D + 4 * t;
    constexpr int U = 8;
    for (int s0 = 0; s0 < splits; s0 += U) {
      float4 v[U];
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = s0 + u;
        w[u] = 0.0f;
        v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (s < splits) {
          const float2 p = ml[(int64_t)s * kHMax];
          if (p.x != -INFINITY) {
            w[u] = exp2f(p.x - M);
            Lsum += p.y * w[u];
            v[u] = *reinterpret_cast<const float4*>(base + (int64_t)s * kHMax * D);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        o.x = fmaf(v[u].x, w[u], o.x);
        o.y = fmaf(v[u].y, w[u], o.y);
        o.z = fmaf(v[u].z, w[u], o.z);
        o.w = fmaf(v[u].w, w[u], o.w);
      }
    }
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  o = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  const int R = a.rope_dims;
  const int c = 4 * t;
  if (c >= D - R) {
    const int j = (c - (D - R)) >> 1;
    const double th = pow((double)a.rope_base, -2.0 * (double)j / (double)R);
    const double ang = -(double)a.q_pos[b] * th;
    const float c0 = (float)cos(ang), s0 = (float)sin(ang);
    o = make_float4(o.x * c0 - o.y * s0, o.x * s0 + o.y * c0, o.z, o.w);
  }
  if (c + 2 >= D - R) {
    const int j = (c + 2 - (D - R)) >> 1;
    const double th = pow((double)a.rope_base, -2.0 * (double)j / (double)R);
    const double ang = -(double)a.q_pos[b] * th;
    const float c1 = (float)cos(ang), s1 = (float)sin(ang);
    o = make_float4(o.x, o.y, o.z * c1 - o.w * s1, o.z * s1 + o.w * c1);
  }
  *reinterpret_cast<float4*>(a.O + (b * a.H + h) * D + c) = o;
}

// ------------------------------------------------------------- planning / launch

bool plan_attend(int64_t B, int H, int D, int64_t max_keys, int splits_hint, AttendPlan* p) {
  (void)H;
  (void)D;
  const int64_t tiles = max_keys <= 0 ? 1 : (max_keys + kTK - 1) / kTK;
  int64_t splits = splits_hint;
  if (splits <= 0) {
    // about two workgroups per compute unit, at least 4 tiles per split
    const int64_t want = (512 + B - 1) / B;
    const int64_t cap = tiles / 4;
    splits = want < cap ? want : cap;
    if (splits < 1) splits = 1;
    if (splits > 64) splits = 64;
  }
  if (splits > tiles) splits = tiles;
  if (splits < 1) splits = 1;
  const int64_t tiles_per = (tiles + splits - 1) / splits;
  splits = (tiles + tiles_per - 1) / tiles_per;
  p->splits = (int)splits;
  p->keys_per_split = tiles_per * kTK;
  p->bytes = splits > 1 ? (size_t)B * splits * kHMax * ((size_t)D + 2) * 4 : 0;
  return true;
}

template <int D, bool CFP8, bool WFP8>
static hipError_t launch_attend_t(const AttendPlan& p, const AttendArgs& a, void* workspace,
                                  hipStream_t stream) {
  using L = AttLayout<D, CFP8, WFP8>;
  auto kern = k_attend<D, CFP8, WFP8>;
  if (L::bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
    if (e != hipSuccess) return e;
  }
  float* ws_acc = reinterpret_cast<float*>(workspace);
  float* ws_ml = p.splits > 1 ? ws_acc + (size_t)a.B * p.splits * kHMax * D : nullptr;
  dim3 grid((unsigned)p.splits, (unsigned)a.B);
  hipLaunchKernelGGL(kern, grid, dim3(kAttThreads), L::bytes, stream, a, p.splits,
                     p.keys_per_split, ws_acc, ws_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL((k_attend_merge<D>), dim3((unsigned)a.H, (unsigned)a.B), dim3(128), 0, stream,
                     a, p.splits, ws_acc, ws_ml);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendPlan& p, const AttendArgs& a, void* workspace,
                         hipStream_t stream) {
  if (a.D == 512) {
    if (a.cache_fp8) return a.win_fp8 ? launch_attend_t<512, true, true>(p, a, workspace, stream)
                                      : launch_attend_t<512, true, false>(p, a, workspace, stream);
    return a.win_fp8 ? launch_attend_t<512, false, true>(p, a, workspace, stream)
                     : launch_attend_t<512, false, false>(p, a, workspace, stream);
  }
  if (a.cache_fp8) return a.win_fp8 ? launch_attend_t<128, true, true>(p, a, workspace, stream)
                                    : launch_attend_t<128, true, false>(p, a, workspace, stream);
  return a.win_fp8 ? launch_attend_t<128, false, true>(p, a, workspace, stream)
                   : launch_attend_t<128, false, false>(p, a, workspace, stream);
}

}  // namespace cskv
