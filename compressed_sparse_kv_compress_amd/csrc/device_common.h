// Device-side helpers shared by the gfx950 kernels: number formats, wave
// reductions, MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cskv {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values to a bf16 pair (round to nearest even), one gfx950
// conversion instruction; the first value lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- E4M3 (OCP, "FN")
// sign | 4-bit exponent (bias 7) | 3-bit mantissa; exponent 0 is subnormal;
// S.1111.111 is NaN; largest finite 448.

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
  float mag = (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 0xFu && m == 7u) mag = __uint_as_float(0x7FC00000u);
  return __uint_as_float(__float_as_uint(mag) | ((code & 0x80u) << 24));
}

// bf16 bit pattern of an E4M3 value (exact: 3 mantissa bits, exponents -9..8).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t code) {
  return __float_as_uint(e4m3_to_f32(code)) >> 16;
}

// Nearest E4M3 code, ties to even mantissa, saturating at 448; NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  if (a != a) return 0x7Fu;
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0x1p-6f) {
    // subnormal range: value = m * 2^-9, m = nearest-even integer of a * 2^9
    // (m == 8 is the smallest normal, which is also code 8)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // keep 3 of the 23 fp32 mantissa bits, rounding to nearest even
    const uint32_t ua = __float_as_uint(a);
    const uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
  }
  return code | sign;
}

// ---------------------------------------------------------------- E2M1 (OCP MX FP4)
// sign | 2-bit exponent (bias 1) | 1-bit mantissa; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.

__device__ __forceinline__ float e2m1_to_f32(uint32_t code) {
  // (e,m) placed as a tiny float whose exponent field is e: times 2^126 this is
  // exactly the E2M1 value, subnormal (e = 0) included.
  const float mag = __uint_as_float((code & 7u) << 22) * 0x1p126f;
  return __uint_as_float(__float_as_uint(mag) | ((code & 8u) << 28));
}

// Nearest E2M1 code, ties to even, saturating at 6; NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  const uint32_t u = __float_as_uint(x);
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  if (a != a) return 0u;
  const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
  return mag | ((u >> 28) & 8u);
}

// Two packed E2M1 codes (one byte of `word`, selected by SEL) to a bf16 pair;
// the low nibble lands in the low half. Uses the gfx950 scaled converter with
// scale 1.
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// Two E4M3 codes (one 16-bit half of `word`, selected by HI) to a bf16 pair,
// exactly (3 mantissa bits and exponents 2^-9 .. 2^8 fit bf16), through the
// gfx950 scaled converter with scale 1; the lower code lands in the low half.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI));
}

// 8 E4M3 codes -> 8 bf16, packed like a 16-byte bf16 row load.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 c) {
  return make_uint4(fp8x2_to_bf16x2<false>(c.x), fp8x2_to_bf16x2<true>(c.x), fp8x2_to_bf16x2<false>(c.y),
                    fp8x2_to_bf16x2<true>(c.y));
}

// Cache row formats shared by the compressor and the attention kernels.
constexpr int kFmtBf16 = 0;   // D bf16 channels
constexpr int kFmtFp8 = 1;    // D E4M3 codes + one fp32 scale per row (separate array)
constexpr int kFmtMix = 2;    // D-64 E4M3 codes, then the 64 rotary channels in bf16; fp32 row scale of the codes
constexpr int kFmtFp4 = 3;    // D/2 bytes of E2M1 codes (channel 2j in the low nibble), then D/16 E4M3 group scales
constexpr int kMixRope = 64;  // rotary channels a mixed row keeps in bf16
constexpr int kMixRowChunks = (512 - kMixRope + 2 * kMixRope) / 16;   // 16-byte chunks of a D = 512 mixed row
template <int D, int FMT>
constexpr int row_bytes() {
  return FMT == kFmtBf16 ? 2 * D : (FMT == kFmtFp8 ? D : (FMT == kFmtMix ? D - kMixRope + 2 * kMixRope : D / 2 + D / 16));
}
constexpr int kFp4RowChunks = (512 / 2 + 512 / 16) / 16;   // 16-byte chunks of a D = 512 fp4 row

// 8 E2M1 codes (one 32-bit word, channel 2j in the low nibble of byte j) times
// their group's E4M3 scale value, as 8 bf16 (exact: at most 5 significant bits).
__device__ __forceinline__ uint4 fp4x8_to_bf16x8_scaled(uint32_t w, float s) {
  const uint32_t b0 = __builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<0>(w));
  const uint32_t b1 = __builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<1>(w));
  const uint32_t b2 = __builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<2>(w));
  const uint32_t b3 = __builtin_bit_cast(uint32_t, fp4x2_to_bf16x2<3>(w));
  return make_uint4(pack_bf16x2(bf16_lo(b0) * s, bf16_hi(b0) * s), pack_bf16x2(bf16_lo(b1) * s, bf16_hi(b1) * s),
                    pack_bf16x2(bf16_lo(b2) * s, bf16_hi(b2) * s), pack_bf16x2(bf16_lo(b3) * s, bf16_hi(b3) * s));
}

// 8 E4M3 codes times the row scale, rounded to bf16 (mixed rows enter the
// tile already scaled, so their value scale is 1): exact bf16 of each code by
// the hardware converter, then one fp32 multiply and one rounding.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8_scaled(uint2 c, float s) {
  const uint4 v = fp8x8_to_bf16x8(c);
  return make_uint4(pack_bf16x2(bf16_lo(v.x) * s, bf16_hi(v.x) * s), pack_bf16x2(bf16_lo(v.y) * s, bf16_hi(v.y) * s),
                    pack_bf16x2(bf16_lo(v.z) * s, bf16_hi(v.z) * s), pack_bf16x2(bf16_lo(v.w) * s, bf16_hi(v.w) * s));
}

// ---------------------------------------------------------------- streaming loads
// Data read exactly once (indexer keys, cache rows) is loaded non-temporally so
// that it does not displace reusable lines from the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(p);
}

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// DPP controls (GFX9): quad permutations and rotations within a row of 16 lanes.
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;   // row_ror:4
constexpr int kDppRowRor8 = 0x128;   // row_ror:8

// Sum over each aligned group of 4 lanes (every lane of the group gets it).
__device__ __forceinline__ float sum_quad(float v) {
  v += dpp_f32<kDppQuadSwap1>(v);
  v += dpp_f32<kDppQuadSwap2>(v);
  return v;
}

// Sum over each row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ float sum_row16(float v) {
  v = sum_quad(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  return v;
}

// Row broadcasts (GFX9): lane 15 of each row into rows 1 and 3, lane 31 into
// rows 2 and 3. Lanes of the rows left out get `old`.
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows_f32(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}

// cos and sin of an angle in radians (fp64, any size; rotary angles reach
// ~1e6): reduced to [-pi, pi] in fp64, then evaluated in fp32. The reduction
// error is ~1e-10 rad at 1e6, so the results are within ~1.5 ulp of the fp64
// functions rounded to fp32, which cost a slow large-argument reduction.
__device__ __forceinline__ void sincos_rad(double a, float* s, float* c) {
  const double r = a - 6.283185307179586 * rint(a * 0.15915494309189535);
  sincosf((float)r, s, c);
}

// v combined with lane l ^ 16 and with lane l ^ 32 (gfx950 lane swaps: for a
// register swapped with itself, the two results hold v and v[l ^ 16] (or
// v[l ^ 32]) in some order, so their sum or maximum is the pair's).
__device__ __forceinline__ float add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum and sum over the wave, in every lane: DPP within each row of 16
// lanes, the rows folded into lane 63 by row broadcasts, then read back as a
// scalar (no LDS shuffles).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  v = fmaxf(v, dpp_rows_f32<kDppRowBcast15, 0xA>(v, v));
  v = fmaxf(v, dpp_rows_f32<kDppRowBcast31, 0xC>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = sum_row16(v);
  v += dpp_rows_f32<kDppRowBcast15, 0xA>(0.0f, v);
  v += dpp_rows_f32<kDppRowBcast31, 0xC>(0.0f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Inclusive prefix sum over the wave (lane 0 first).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  // DPP: sums within each row of 16 lanes by shifts of 1, 2, 4 and 8 (lanes
  // shifted in from outside the row add 0), then lane 15's row total into
  // rows 1 and 3 and lane 31's running total into rows 2 and 3. Each step is
  // one VALU add (a shuffle would be an LDS round trip).
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return v;
}
// The value of lane `src` (the same in every lane of the wave): a scalar read
// instead of a shuffle through LDS.
__device__ __forceinline__ int lane_value(int v, int src) {
  return __builtin_amdgcn_readlane(v, __builtin_amdgcn_readfirstlane(src));
}
// (the float's bits, not a conversion of its value)
__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(lane_value(__float_as_int(v), src));
}

// Orderable key of a score: larger score -> larger key; -0 equals +0; NaN -> 0
// (below every number, -inf included).
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 0u;
  s = s + 0.0f;  // -0 + +0 = +0 under round-to-nearest
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace cskv
