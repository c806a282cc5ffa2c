// Shared-K/V multi-query attention over gathered cache entries plus the
// uncompressed window, with inverse RoPE on the output.
//
// [P2] Step 3: one shared state S_j is compared with the query (score =
// Q.S_j) and mixed into the output as content. [P2] Step 5: the query reads
// the selected c4a entries, or every c128a entry. [P2] Step 6 and [P1] "The
// sliding window": the newest 128 states are read exactly, in the same
// softmax. [P1] "Shared key and value": inverse RoPE on the attention output.
//
// All heads of a sequence share the key rows, so QK^T and PV are dense
// contractions of [heads x D] against [keys x D]: they run on 16x16x32 bf16
// MFMA. A workgroup (4 waves) owns one sequence and a contiguous split of its
// key slots; per 32-slot tile it
//   1. gathers the rows (bf16, or fp8 codes decoded exactly to bf16 with the
//      row scale folded into logits and probabilities) from HBM into
//      registers one tile ahead, then stores them to LDS twice: row-major for
//      QK^T and channel-major (8x8 register transposes) for PV;
//   2. QK^T: wave w computes S^T[32 keys x 16 heads] for heads 16w..16w+15
//      with its Q fragment held in registers;
//   3. online softmax (exp2 domain) per head, P to LDS as bf16;
//   4. PV: wave w accumulates O[heads x D/4 channels] for its channel quarter.
// With one split the epilogue normalises, applies inverse RoPE and stores O;
// otherwise partial (max, sum, unnormalised O) go to the workspace and
// k_attend_merge combines them (log-sum-exp) and applies inverse RoPE.
#include "kernels.h"

namespace cskv {

constexpr int kAttThreads = 256;
constexpr int kTK = 32;        // key slots per tile
constexpr int kHMax = 64;      // heads per workgroup (padded to 16s)
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct AttLayout {
  static constexpr int KROW = D + 8;        // bf16 per row-major key row (padding vs bank conflicts)
  static constexpr int KCOL = kTK + 8;      // bf16 per channel-major row
  static constexpr int PST = kTK + 8;       // bf16 per P row
  static constexpr size_t off_krow = 0;
  static constexpr size_t off_kcol = off_krow + (size_t)kTK * KROW * 2;
  static constexpr size_t off_p = off_kcol + (size_t)D * KCOL * 2;
  static constexpr size_t off_alpha = off_p + (size_t)kHMax * PST * 2;
  static constexpr size_t off_rs = off_alpha + kHMax * 4;      // per-slot logit factor
  static constexpr size_t off_ps = off_rs + kTK * 4;           // per-slot value scale (< 0 = masked)
  static constexpr size_t off_m = off_ps + kTK * 4;
  static constexpr size_t off_l = off_m + kHMax * 4;
  static constexpr size_t off_cos = off_l + kHMax * 4;
  static constexpr size_t off_sin = off_cos + (D / 2) * 4;
  static constexpr size_t bytes = off_sin + (D / 2) * 4;
};

// 8 fp8 codes -> 8 bf16 (exact), packed like a bf16 row load.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 c) {
  uint4 r;
  r.x = e4m3_to_bf16_bits(c.x & 0xFFu) | (e4m3_to_bf16_bits((c.x >> 8) & 0xFFu) << 16);
  r.y = e4m3_to_bf16_bits((c.x >> 16) & 0xFFu) | (e4m3_to_bf16_bits(c.x >> 24) << 16);
  r.z = e4m3_to_bf16_bits(c.y & 0xFFu) | (e4m3_to_bf16_bits((c.y >> 8) & 0xFFu) << 16);
  r.w = e4m3_to_bf16_bits((c.y >> 16) & 0xFFu) | (e4m3_to_bf16_bits(c.y >> 24) << 16);
  return r;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// One thread's share of a tile: rows 8*kb .. 8*kb+7, channels 8*cb .. 8*cb+7.
struct TileRegs {
  uint4 r[8];
  float vs[8];     // value scale of the row (1 for bf16)
  bool ok[8];      // slot holds a real key row
};

template <int D, bool CFP8, bool WFP8>
__device__ __forceinline__ void load_tile(const AttendArgs& a, int64_t b, int64_t slot0, int64_t n_sel,
                                          int64_t n_keys, bool dense, int kb, int cb, TileRegs& t) {
  const bool active_c = cb * 8 < D;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t slot = slot0 + 8 * kb + i;
    t.r[i] = make_uint4(0, 0, 0, 0);
    t.vs[i] = 0.0f;
    t.ok[i] = false;
    if (slot >= n_keys) continue;
    if (slot < n_sel) {
      const int64_t row = dense ? slot : (int64_t)a.ids[b * a.k + slot];
      if (row < 0 || row >= a.cache_rows) continue;
      const int64_t r = b * a.cache_rows + row;
      t.ok[i] = true;
      if constexpr (CFP8) {
        t.vs[i] = a.cache_scale[r];
        if (active_c) t.r[i] = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(
                          reinterpret_cast<const uint8_t*>(a.cache) + r * D + cb * 8));
      } else {
        t.vs[i] = 1.0f;
        if (active_c) t.r[i] = *reinterpret_cast<const uint4*>(
                          reinterpret_cast<const uint16_t*>(a.cache) + r * D + cb * 8);
      }
    } else {
      const int64_t r = b * a.win_bstride + (slot - n_sel);
      t.ok[i] = true;
      if constexpr (WFP8) {
        t.vs[i] = a.window_scale[r];
        if (active_c) t.r[i] = fp8x8_to_bf16x8(*reinterpret_cast<const uint2*>(
                          reinterpret_cast<const uint8_t*>(a.window) + r * D + cb * 8));
      } else {
        t.vs[i] = 1.0f;
        if (active_c) t.r[i] = *reinterpret_cast<const uint4*>(
                          reinterpret_cast<const uint16_t*>(a.window) + r * D + cb * 8);
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(uint8_t* lds, int kb, int cb, const TileRegs& t,
                                           float tau_log2e) {
  using L = AttLayout<D>;
  uint16_t* krow = reinterpret_cast<uint16_t*>(lds + L::off_krow);
  uint16_t* kcol = reinterpret_cast<uint16_t*>(lds + L::off_kcol);
  if (cb * 8 < D) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(krow + (8 * kb + i) * L::KROW + 8 * cb) = t.r[i];
    // transpose the 8x8 bf16 block: channel c of keys 0..7
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = word_of(t.r[i], c >> 1);
      uint4 o;
      if ((c & 1) == 0) {
        o.x = lo_pair(w[0], w[1]); o.y = lo_pair(w[2], w[3]);
        o.z = lo_pair(w[4], w[5]); o.w = lo_pair(w[6], w[7]);
      } else {
        o.x = hi_pair(w[0], w[1]); o.y = hi_pair(w[2], w[3]);
        o.z = hi_pair(w[4], w[5]); o.w = hi_pair(w[6], w[7]);
      }
      *reinterpret_cast<uint4*>(kcol + (8 * cb + c) * L::KCOL + 8 * kb) = o;
    }
  }
  if (cb == 0) {
    float* rs = reinterpret_cast<float*>(lds + L::off_rs);
    float* ps = reinterpret_cast<float*>(lds + L::off_ps);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rs[8 * kb + i] = t.ok[i] ? t.vs[i] * tau_log2e : 0.0f;
      ps[8 * kb + i] = t.ok[i] ? t.vs[i] : -1.0f;   // < 0 marks a masked slot
    }
  }
}

template <int D, bool CFP8, bool WFP8>
__global__ __launch_bounds__(kAttThreads) void k_attend(AttendArgs a, int splits, int64_t keys_per_split,
                                                       float* __restrict__ ws_acc,
                                                       float* __restrict__ ws_ml) {
  using L = AttLayout<D>;
  constexpr int KS = D / 32;          // k-steps of QK^T
  constexpr int CTW = D / 64;         // 16-channel tiles per wave in PV
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint16_t* krow = reinterpret_cast<uint16_t*>(lds + L::off_krow);
  uint16_t* kcol = reinterpret_cast<uint16_t*>(lds + L::off_kcol);
  uint16_t* pl = reinterpret_cast<uint16_t*>(lds + L::off_p);
  float* alpha_l = reinterpret_cast<float*>(lds + L::off_alpha);
  float* rs_l = reinterpret_cast<float*>(lds + L::off_rs);
  float* ps_l = reinterpret_cast<float*>(lds + L::off_ps);
  float* m_l = reinterpret_cast<float*>(lds + L::off_m);
  float* l_l = reinterpret_cast<float*>(lds + L::off_l);
  float* cos_l = reinterpret_cast<float*>(lds + L::off_cos);
  float* sin_l = reinterpret_cast<float*>(lds + L::off_sin);

  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.y;
  const int s = blockIdx.x;
  const int HT = (a.H + 15) / 16;
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

  // rotary tables (fp64 angles), used by the single-split epilogue
  if (splits == 1 && t < a.rope_dims / 2) {
    const double theta = pow((double)a.rope_base, -2.0 * (double)t / (double)a.rope_dims);
    const double ang = -(double)a.q_pos[b] * theta;
    cos_l[t] = (float)cos(ang);
    sin_l[t] = (float)sin(ang);
  }

  // Q fragment: B operand of S^T = K Q^T; lane holds Q[16w + l16][32ks + 8g .. +7]
  bf16x8_t qf[KS];
  {
    const int h = 16 * wave + l16;
    const bool qok = wave < HT && h < a.H;
    const uint16_t* qrow = a.Q + (b * a.H + (qok ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = qok ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t acc[4][CTW];
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) acc[ht][ct] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  const int kb = t >> 6, cb = t & 63;
  TileRegs tr;
  if (lo < hi) load_tile<D, CFP8, WFP8>(a, b, lo, n_sel, n_keys, dense, kb, cb, tr);

  for (int64_t tile = lo; tile < hi; tile += kTK) {
    __syncthreads();                        // previous tile fully consumed
    store_tile<D>(lds, kb, cb, tr, tau_log2e);
    __syncthreads();
    if (tile + kTK < hi) load_tile<D, CFP8, WFP8>(a, b, tile + kTK, n_sel, n_keys, dense, kb, cb, tr);

    if (wave < HT) {
      f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(krow + l16 * L::KROW + 32 * ks + 8 * g);
        const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(krow + (16 + l16) * L::KROW + 32 * ks + 8 * g);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
      }
      // lane holds logits of head 16w + l16 for slots 4g+i and 16+4g+i
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j0 = 4 * g + i, j1 = 16 + 4 * g + i;
        x[i] = ps_l[j0] >= 0.0f ? s0[i] * rs_l[j0] : -INFINITY;
        x[4 + i] = ps_l[j1] >= 0.0f ? s1[i] * rs_l[j1] : -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
      float p[8], lsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = (x[i] == -INFINITY) ? 0.0f : exp2f(x[i] - m_new);
        lsum += p[i];
      }
      lsum += __shfl_xor(lsum, 16, kWave);
      lsum += __shfl_xor(lsum, 32, kWave);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      const int h = 16 * wave + l16;
      uint16_t* prow = pl + h * L::PST;
      uint2 w0, w1;
      {
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = p[i] * fmaxf(ps_l[4 * g + i], 0.0f);
          v[4 + i] = p[4 + i] * fmaxf(ps_l[16 + 4 * g + i], 0.0f);
        }
        w0.x = pack_bf16x2(v[0], v[1]); w0.y = pack_bf16x2(v[2], v[3]);
        w1.x = pack_bf16x2(v[4], v[5]); w1.y = pack_bf16x2(v[6], v[7]);
      }
      *reinterpret_cast<uint2*>(prow + 4 * g) = w0;
      *reinterpret_cast<uint2*>(prow + 16 + 4 * g) = w1;
      if (g == 0) alpha_l[h] = alpha;
    }
    __syncthreads();

    // PV: O[heads][channels of this wave] += P[heads][32 slots] x K[32 slots][channels]
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      if (ht < HT) {
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = alpha_l[16 * ht + 4 * g + i];
        const bf16x8_t pa = *reinterpret_cast<const bf16x8_t*>(pl + (16 * ht + l16) * L::PST + 8 * g);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const int ch = wave * (D / 4) + 16 * ct + l16;
          const bf16x8_t kv = *reinterpret_cast<const bf16x8_t*>(kcol + ch * L::KCOL + 8 * g);
          f32x4_t c = acc[ht][ct];
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] *= al[i];
          acc[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, kv, c, 0, 0, 0);
        }
      }
    }
  }

  // per-head softmax state -> LDS
  if (wave < HT && g == 0) {
    m_l[16 * wave + l16] = m_run;
    l_l[16 * wave + l16] = l_run;
  }
  __syncthreads();

  if (splits == 1) {
    const int R = a.rope_dims;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      if (ht >= HT) continue;
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int ch = wave * (D / 4) + 16 * ct + l16;
        const bool rot = ch >= D - R;
        const int j = (ch - (D - R)) >> 1;
        const float cs = rot ? cos_l[j] : 1.0f, sn = rot ? sin_l[j] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 16 * ht + 4 * g + i;
          const float lh = l_l[h];
          const float v = lh > 0.0f ? acc[ht][ct][i] / lh : 0.0f;
          const float pv = __shfl_xor(v, 1, kWave);
          float o = v;
          if (rot) o = (ch & 1) == 0 ? v * cs - pv * sn : pv * sn + v * cs;
          if (h < a.H) a.O[(b * a.H + h) * D + ch] = o;
        }
      }
    }
  } else {
    const int64_t part = b * splits + s;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      if (ht >= HT) continue;
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int ch = wave * (D / 4) + 16 * ct + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 16 * ht + 4 * g + i;
          if (h < a.H) ws_acc[(part * kHMax + h) * D + ch] = acc[ht][ct][i];
        }
      }
    }
    if (t < a.H) {
      ws_ml[(part * kHMax + t) * 2 + 0] = m_l[t];
      ws_ml[(part * kHMax + t) * 2 + 1] = l_l[t];
    }
  }
}

// Log-sum-exp merge of the splits of one (sequence, head), then inverse RoPE.
template <int D>
__global__ __launch_bounds__(128) void k_attend_merge(AttendArgs a, int splits,
                                                      const float* __restrict__ ws_acc,
                                                      const float* __restrict__ ws_ml) {
  const int64_t b = blockIdx.y;
  const int h = blockIdx.x;
  const int t = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ws_ml[((b * splits + s) * kHMax + h) * 2]);
  float Lsum = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float* ml = ws_ml + ((b * splits + s) * kHMax + h) * 2;
      if (ml[0] != -INFINITY) Lsum += ml[1] * exp2f(ml[0] - M);
    }
  }
  const int R = a.rope_dims;
  for (int pr = t; pr < D / 2; pr += 128) {
    const int c0 = 2 * pr;
    float x = 0.0f, y = 0.0f;
    if (Lsum > 0.0f) {
      for (int s = 0; s < splits; ++s) {
        const float* ml = ws_ml + ((b * splits + s) * kHMax + h) * 2;
        if (ml[0] == -INFINITY) continue;
        const float w = exp2f(ml[0] - M);
        const float* acc = ws_acc + ((b * splits + s) * kHMax + h) * D;
        x = fmaf(acc[c0], w, x);
        y = fmaf(acc[c0 + 1], w, y);
      }
      x /= Lsum;
      y /= Lsum;
    }
    if (c0 >= D - R) {
      const int j = (c0 - (D - R)) >> 1;
      const double theta = pow((double)a.rope_base, -2.0 * (double)j / (double)R);
      const double ang = -(double)a.q_pos[b] * theta;
      const float cs = (float)cos(ang), sn = (float)sin(ang);
      const float xr = x * cs - y * sn, yr = x * sn + y * cs;
      x = xr;
      y = yr;
    }
    float* o = a.O + (b * a.H + h) * D + c0;
    o[0] = x;
    o[1] = y;
  }
}

// ------------------------------------------------------------- planning / launch

bool plan_attend(int64_t B, int H, int D, int64_t max_keys, int splits_hint, AttendPlan* p) {
  (void)H;
  const int64_t tiles = max_keys <= 0 ? 1 : (max_keys + kTK - 1) / kTK;
  int64_t splits = splits_hint;
  if (splits <= 0) {
    int64_t want = (512 + B - 1) / B;
    int64_t cap = tiles / 4;
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
  using L = AttLayout<D>;
  auto kern = k_attend<D, CFP8, WFP8>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)L::bytes);
  if (e != hipSuccess) return e;
  float* ws_acc = reinterpret_cast<float*>(workspace);
  float* ws_ml = p.splits > 1 ? ws_acc + (size_t)a.B * p.splits * kHMax * D : nullptr;
  dim3 grid((unsigned)p.splits, (unsigned)a.B);
  hipLaunchKernelGGL(kern, grid, dim3(kAttThreads), L::bytes, stream, a, p.splits,
                     p.keys_per_split, ws_acc, ws_ml);
  e = hipGetLastError();
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
