// C ABI of libcskv: argument validation, launch planning, error reporting.
// Everything is checked on the host before any kernel is enqueued.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/cskv.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

cskv_status fail(cskv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

cskv_status ok() {
  g_err[0] = '\0';
  return CSKV_OK;
}

cskv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int row_format(int32_t cache_dtype) {
  switch (cache_dtype) {
    case CSKV_FP8_ROPE64: return cskv::kFmtMix;
    case CSKV_FP8_E4M3: return cskv::kFmtFp8;
    case CSKV_FP4_E2M1: return cskv::kFmtFp4;
    default: return cskv::kFmtBf16;
  }
}

// Cache formats: bf16, fp8 rows, mixed rows and fp4 rows (the last two D = 512).
bool cache_format_ok(int32_t dt) {
  return dt == CSKV_BF16 || dt == CSKV_FP8_E4M3 || dt == CSKV_FP8_ROPE64 || dt == CSKV_FP4_E2M1;
}
// Formats with a separate fp32 scale per row.
bool needs_row_scale(int32_t dt) { return dt == CSKV_FP8_E4M3 || dt == CSKV_FP8_ROPE64; }

#define CHECK(cond, status, ...) \
  do {                           \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

}  // namespace

extern "C" {

const char* cskv_status_string(cskv_status s) {
  switch (s) {
    case CSKV_OK: return "ok";
    case CSKV_EINVAL: return "invalid argument";
    case CSKV_EUNSUPPORTED: return "unsupported";
    case CSKV_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* cskv_last_error(void) { return g_err; }

int32_t cskv_version(void) { return 100; }

// ------------------------------------------------------------------ compress

cskv_status cskv_compress(int32_t kind, const void* S, const float* gate, int64_t B, int64_t T,
                          int32_t D, int64_t first_entry, int32_t cache_dtype, void* cache,
                          float* cache_scale, int64_t cache_rows, void* stream) {
  CHECK(kind == CSKV_C4A || kind == CSKV_C128A, CSKV_EINVAL, "compress: unknown kind %d", kind);
  CHECK(B >= 0 && T >= 0 && first_entry >= 0 && cache_rows >= 0, CSKV_EINVAL,
        "compress: negative size (B=%lld T=%lld first_entry=%lld cache_rows=%lld)", (long long)B,
        (long long)T, (long long)first_entry, (long long)cache_rows);
  CHECK(D == 128 || D == 512, CSKV_EUNSUPPORTED, "compress: D=%d (supported: 128, 512)", D);
  CHECK(cache_format_ok(cache_dtype), CSKV_EUNSUPPORTED,
        "compress: cache dtype %d (supported: bf16, fp8, fp8 + bf16 rotary, fp4)", cache_dtype);
  CHECK((cache_dtype != CSKV_FP8_ROPE64 && cache_dtype != CSKV_FP4_E2M1) || D == 512, CSKV_EUNSUPPORTED,
        "compress: fp8 + bf16 rotary and fp4 rows need D = 512");
  const int64_t w = kind == CSKV_C4A ? 8 : 128, s = kind == CSKV_C4A ? 4 : 128;
  const int64_t n = T < w ? 0 : (T - w) / s + 1;
  CHECK(first_entry + n <= cache_rows, CSKV_EINVAL,
        "compress: entries %lld..%lld do not fit cache_rows=%lld", (long long)first_entry,
        (long long)(first_entry + n - 1), (long long)cache_rows);
  if (B == 0 || n == 0) return ok();
  CHECK(S && gate && cache, CSKV_EINVAL, "compress: null S, gate or cache");
  CHECK(!needs_row_scale(cache_dtype) || cache_scale, CSKV_EINVAL, "compress: fp8 cache needs cache_scale");
  CHECK(aligned(S, 16) && aligned(cache, 16) && aligned(gate, 4), CSKV_EINVAL,
        "compress: S and cache must be 16-byte aligned");
  CHECK(B <= 65535, CSKV_EUNSUPPORTED, "compress: B=%lld > 65535", (long long)B);
  CHECK(kind == CSKV_C4A || n <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "compress: too many entries");
  return hip_status(cskv::launch_compress(kind, reinterpret_cast<const uint16_t*>(S), gate, B, T, D,
                                          n, first_entry, row_format(cache_dtype), cache,
                                          cache_scale, cache_rows,
                                          reinterpret_cast<hipStream_t>(stream)),
                    "compress launch");
}

// ------------------------------------------------------------------ append

cskv_status cskv_append(int32_t kind, const void* s_new, const float* g_new, const int64_t* pos,
                        int64_t B, int32_t D, void* ring, float* ring_gate, int32_t W,
                        int32_t cache_dtype, void* cache, float* cache_scale, int64_t cache_rows,
                        int32_t* n_entries, int32_t* n_window, void* stream) {
  CHECK(kind == CSKV_C4A || kind == CSKV_C128A, CSKV_EINVAL, "append: unknown kind %d", kind);
  CHECK(B >= 0 && cache_rows >= 0, CSKV_EINVAL, "append: negative size (B=%lld cache_rows=%lld)",
        (long long)B, (long long)cache_rows);
  CHECK(D == 128 || D == 512, CSKV_EUNSUPPORTED, "append: D=%d (supported: 128, 512)", D);
  CHECK(cache_format_ok(cache_dtype), CSKV_EUNSUPPORTED,
        "append: cache dtype %d (supported: bf16, fp8, fp8 + bf16 rotary, fp4)", cache_dtype);
  CHECK((cache_dtype != CSKV_FP8_ROPE64 && cache_dtype != CSKV_FP4_E2M1) || D == 512, CSKV_EUNSUPPORTED,
        "append: fp8 + bf16 rotary and fp4 rows need D = 512");
  const int32_t w = kind == CSKV_C4A ? 8 : 128;
  CHECK(W >= w, CSKV_EINVAL, "append: W=%d must be >= %d, the states of one entry", W, w);
  CHECK(cache_rows <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "append: cache_rows too large for int32 counts");
  if (B == 0) return ok();
  CHECK(s_new && g_new && pos && ring && ring_gate, CSKV_EINVAL, "append: null s_new, g_new, pos or ring");
  CHECK(cache_rows == 0 || cache, CSKV_EINVAL, "append: null cache");
  CHECK(!needs_row_scale(cache_dtype) || cache_rows == 0 || cache_scale, CSKV_EINVAL,
        "append: fp8 cache needs cache_scale");
  CHECK(aligned(s_new, 16) && aligned(ring, 16) && (!cache || aligned(cache, 16)) && aligned(g_new, 4) &&
            aligned(ring_gate, 4) && aligned(pos, 8),
        CSKV_EINVAL, "append: s_new, ring and cache must be 16-byte aligned");
  CHECK(B <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "append: B=%lld too large", (long long)B);
  return hip_status(cskv::launch_append(kind, reinterpret_cast<const uint16_t*>(s_new), g_new, pos, B, D,
                                        reinterpret_cast<uint16_t*>(ring), ring_gate, W,
                                        row_format(cache_dtype), cache, cache_scale, cache_rows,
                                        n_entries, n_window, reinterpret_cast<hipStream_t>(stream)),
                    "append launch");
}

// ------------------------------------------------------------------ index / top-k

static cskv_status topk_common(int64_t B, int64_t n_max, int32_t Di, int32_t k, int32_t key_dtype,
                               int32_t chunk, cskv::TopkPlan* plan) {
  CHECK(B >= 0 && n_max >= 0, CSKV_EINVAL, "index_topk: negative size");
  CHECK(k >= 1, CSKV_EINVAL, "index_topk: k=%d must be >= 1", k);
  CHECK(k <= 2048, CSKV_EUNSUPPORTED, "index_topk: k=%d > 2048", k);
  CHECK(Di == 32 || Di == 128, CSKV_EUNSUPPORTED, "index_topk: Di=%d (supported: 32, 128)", Di);
  CHECK(key_dtype == CSKV_BF16 || key_dtype == CSKV_FP4_E2M1, CSKV_EUNSUPPORTED,
        "index_topk: key dtype %d (supported: bf16, fp4)", key_dtype);
  CHECK(chunk == 0 || (chunk >= 256 && chunk <= 16384 && chunk % 256 == 0), CSKV_EINVAL,
        "index_topk: chunk=%d must be 0 or a multiple of 256 in [256, 16384]", chunk);
  CHECK(B <= 65535, CSKV_EUNSUPPORTED, "index_topk: B=%lld > 65535", (long long)B);
  CHECK(n_max <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "index_topk: n_max too large for int32 ids");
  CHECK(cskv::plan_topk(B, n_max, k, chunk, key_dtype == CSKV_FP4_E2M1, plan), CSKV_EUNSUPPORTED,
        "index_topk: no selection plan for n_max=%lld k=%d chunk=%d", (long long)n_max, k, chunk);
  return ok();
}

size_t cskv_index_topk_workspace(int64_t B, int64_t n_max, int32_t Di, int32_t k, int32_t key_dtype,
                                 int32_t chunk) {
  cskv::TopkPlan plan;
  if (topk_common(B, n_max, Di, k, key_dtype, chunk, &plan) != CSKV_OK) return 0;
  return plan.bytes;
}

cskv_status cskv_index_topk(const void* q_idx, int32_t key_dtype, const void* k_idx,
                            const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                            int64_t n_max, int32_t Di, int32_t k, int32_t* ids, int32_t chunk,
                            void* workspace, size_t workspace_bytes, void* stream) {
  cskv::TopkPlan plan;
  cskv_status st = topk_common(B, n_max, Di, k, key_dtype, chunk, &plan);
  if (st != CSKV_OK) return st;
  if (B == 0) return ok();
  CHECK(q_idx && ids, CSKV_EINVAL, "index_topk: null q_idx or ids");
  CHECK(n_max == 0 || k_idx, CSKV_EINVAL, "index_topk: null k_idx");
  CHECK(key_dtype != CSKV_FP4_E2M1 || n_max == 0 || k_scale, CSKV_EINVAL,
        "index_topk: fp4 keys need k_scale");
  CHECK(aligned(q_idx, 16) && (k_idx == nullptr || aligned(k_idx, 16)), CSKV_EINVAL,
        "index_topk: q_idx and k_idx must be 16-byte aligned");
  CHECK(k_scale == nullptr || aligned(k_scale, 2), CSKV_EINVAL, "index_topk: k_scale must be 2-byte aligned");
  CHECK(workspace_bytes >= plan.bytes, CSKV_EINVAL,
        "index_topk: workspace %zu bytes < %zu required", workspace_bytes, plan.bytes);
  CHECK(plan.bytes == 0 || (workspace && aligned(workspace, 256)), CSKV_EINVAL,
        "index_topk: workspace must be non-null and 256-byte aligned");
  return hip_status(cskv::launch_index_topk(plan, reinterpret_cast<const uint16_t*>(q_idx),
                                            key_dtype == CSKV_FP4_E2M1, k_idx, k_scale, n_entries,
                                            B, n_max, Di, k, ids, workspace,
                                            reinterpret_cast<hipStream_t>(stream)),
                    "index_topk launch");
}

// ------------------------------------------------------------------ attend

size_t cskv_attend_workspace(int64_t B, int32_t H, int32_t D, int64_t max_keys, int32_t splits) {
  cskv::AttendPlan plan;
  if (B < 0 || H < 1 || H > 64 || !(D == 128 || D == 512) || max_keys < 0 || splits < 0) return 0;
  // the larger of the dense and the sparse plan, whichever the call will use
  size_t bytes = 0;
  if (cskv::plan_attend(B, H, D, max_keys, false, splits, &plan)) bytes = plan.bytes;
  if (cskv::plan_attend(B, H, D, max_keys, true, splits, &plan) && plan.bytes > bytes) bytes = plan.bytes;
  return bytes;
}

}  // extern "C"

// Validation and planning shared by cskv_attend and cskv_attend_noalloc.
static cskv_status attend_prepare(const void* Q, int64_t B, int32_t H, int32_t D, int32_t cache_dtype,
                                  const void* cache, const float* cache_scale, int64_t cache_rows,
                                  const int32_t* ids, int32_t k, const int32_t* n_entries, int32_t window_dtype,
                                  const void* window, const float* window_scale, int32_t W,
                                  int64_t window_batch_stride, const int32_t* n_window, int32_t rope_dims,
                                  float rope_base, const int64_t* q_pos, float softmax_scale, float* O,
                                  int32_t splits, cskv::AttendPlan* plan, cskv::AttendArgs* a) {
  CHECK(B >= 0 && cache_rows >= 0 && W >= 0, CSKV_EINVAL, "attend: negative size");
  CHECK(H >= 1 && H <= 64, CSKV_EUNSUPPORTED, "attend: H=%d (supported: 1..64)", H);
  CHECK(D == 128 || D == 512, CSKV_EUNSUPPORTED, "attend: D=%d (supported: 128, 512)", D);
  CHECK(cache_format_ok(cache_dtype), CSKV_EUNSUPPORTED,
        "attend: cache dtype %d (supported: bf16, fp8, fp8 + bf16 rotary, fp4)", cache_dtype);
  CHECK((cache_dtype != CSKV_FP8_ROPE64 && cache_dtype != CSKV_FP4_E2M1) || D == 512, CSKV_EUNSUPPORTED,
        "attend: fp8 + bf16 rotary and fp4 rows need D = 512");
  CHECK(window_dtype == CSKV_BF16 || window_dtype == CSKV_FP8_E4M3, CSKV_EUNSUPPORTED,
        "attend: window dtype %d (supported: bf16, fp8)", window_dtype);
  CHECK(ids == nullptr || k >= 0, CSKV_EINVAL, "attend: k=%d must be >= 0", k);
  CHECK(rope_dims >= 0 && rope_dims <= D && rope_dims % 2 == 0, CSKV_EINVAL,
        "attend: rope_dims=%d must be even and <= D", rope_dims);
  CHECK(rope_dims == 0 || rope_base > 0.0f, CSKV_EINVAL, "attend: rope_base must be > 0");
  CHECK(splits >= 0, CSKV_EINVAL, "attend: splits=%d must be >= 0", splits);
  CHECK(W == 0 || window_batch_stride >= W, CSKV_EINVAL,
        "attend: window_batch_stride=%lld < W=%d", (long long)window_batch_stride, W);
  CHECK(B <= 65535, CSKV_EUNSUPPORTED, "attend: B=%lld > 65535", (long long)B);
  if (B == 0) return ok();
  CHECK(Q && O, CSKV_EINVAL, "attend: null Q or O");
  CHECK(rope_dims == 0 || q_pos, CSKV_EINVAL, "attend: rope_dims > 0 needs q_pos");
  const int64_t n_sel_max = ids ? (int64_t)k : cache_rows;
  CHECK(n_sel_max == 0 || cache, CSKV_EINVAL, "attend: null cache");
  CHECK(!needs_row_scale(cache_dtype) || n_sel_max == 0 || cache_scale, CSKV_EINVAL,
        "attend: fp8 cache needs cache_scale");
  CHECK(W == 0 || window, CSKV_EINVAL, "attend: null window");
  CHECK(window_dtype != CSKV_FP8_E4M3 || W == 0 || window_scale, CSKV_EINVAL,
        "attend: fp8 window needs window_scale");
  CHECK(aligned(Q, 16) && aligned(O, 4) && (!cache || aligned(cache, 16)) &&
            (!window || aligned(window, 16)),
        CSKV_EINVAL, "attend: Q, cache and window must be 16-byte aligned");
  const int64_t max_keys = n_sel_max + W;
  CHECK(cskv::plan_attend(B, H, D, max_keys, ids != nullptr, splits, plan), CSKV_EUNSUPPORTED,
        "attend: no plan for %lld key slots (sparse reads support at most 524288)", (long long)max_keys);
  a->Q = reinterpret_cast<const uint16_t*>(Q);
  a->B = B;
  a->H = H;
  a->D = D;
  a->cache_fp8 = cache_dtype == CSKV_FP8_E4M3;
  a->cache_mix = cache_dtype == CSKV_FP8_ROPE64;
  a->cache_fp4 = cache_dtype == CSKV_FP4_E2M1;
  a->cache = cache;
  a->cache_scale = cache_scale;
  a->cache_rows = cache_rows;
  a->ids = ids;
  a->k = ids ? k : 0;
  a->n_entries = ids ? nullptr : n_entries;
  a->win_fp8 = window_dtype == CSKV_FP8_E4M3;
  a->window = window;
  a->window_scale = window_scale;
  a->W = W;
  a->n_window = W > 0 ? n_window : nullptr;
  a->win_bstride = window_batch_stride;
  a->rope_dims = rope_dims;
  a->rope_base = rope_base;
  for (int i = 0; i < rope_dims / 2; ++i) a->inv_freq[i] = std::pow((double)rope_base, -2.0 * i / rope_dims);
  a->q_pos = q_pos;
  a->softmax_scale = softmax_scale;
  a->O = O;
  a->part_out = nullptr;
  a->part_in = nullptr;
  return ok();
}

// Scratch of cskv_attend_noalloc: the split partials of an attend call, in a
// file-scope device array instead of a caller workspace. Host code must not
// use this name as an address (on the host it is a stand-in); the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[CSKV_ATTEND_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array (looked up the
// first time a call runs on that device).
cskv_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CSKV_EHIP, "attend_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  CHECK(dev >= 0 && dev < kMaxDevices, CSKV_EUNSUPPORTED, "attend_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(CSKV_EHIP, "attend_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}
}  // namespace

extern "C" {

cskv_status cskv_attend(const void* Q, int64_t B, int32_t H, int32_t D, int32_t cache_dtype,
                        const void* cache, const float* cache_scale, int64_t cache_rows,
                        const int32_t* ids, int32_t k, const int32_t* n_entries,
                        int32_t window_dtype, const void* window, const float* window_scale,
                        int32_t W, int64_t window_batch_stride, const int32_t* n_window,
                        int32_t rope_dims, float rope_base, const int64_t* q_pos,
                        float softmax_scale, float* O,
                        int32_t splits, void* workspace, size_t workspace_bytes, void* stream) {
  cskv::AttendPlan plan;
  cskv::AttendArgs a;
  const cskv_status st = attend_prepare(Q, B, H, D, cache_dtype, cache, cache_scale, cache_rows, ids, k, n_entries,
                                        window_dtype, window, window_scale, W, window_batch_stride, n_window,
                                        rope_dims, rope_base, q_pos, softmax_scale, O, splits, &plan, &a);
  if (st != CSKV_OK || B == 0) return st;
  CHECK(workspace_bytes >= plan.bytes, CSKV_EINVAL, "attend: workspace %zu bytes < %zu required",
        workspace_bytes, plan.bytes);
  CHECK(plan.bytes == 0 || (workspace && aligned(workspace, 256)), CSKV_EINVAL,
        "attend: workspace must be non-null and 256-byte aligned");
  return hip_status(cskv::launch_attend(plan, a, workspace, reinterpret_cast<hipStream_t>(stream)),
                    "attend launch");
}

cskv_status cskv_attend_with_partial(const void* Q, int64_t B, int32_t H, int32_t D, int32_t cache_dtype,
                                     const void* cache, const float* cache_scale, int64_t cache_rows,
                                     const int32_t* ids, int32_t k, const int32_t* n_entries,
                                     int32_t window_dtype, const void* window, const float* window_scale,
                                     int32_t W, int64_t window_batch_stride, const int32_t* n_window,
                                     int32_t rope_dims, float rope_base, const int64_t* q_pos,
                                     float softmax_scale, const float* partial, float* O,
                                     int32_t splits, void* workspace, size_t workspace_bytes, void* stream) {
  cskv::AttendPlan plan;
  cskv::AttendArgs a;
  const cskv_status st = attend_prepare(Q, B, H, D, cache_dtype, cache, cache_scale, cache_rows, ids, k, n_entries,
                                        window_dtype, window, window_scale, W, window_batch_stride, n_window,
                                        rope_dims, rope_base, q_pos, softmax_scale, O, splits, &plan, &a);
  if (st != CSKV_OK || B == 0) return st;
  CHECK(partial && aligned(partial, 16), CSKV_EINVAL, "attend_with_partial: partial must be non-null and 16-byte aligned");
  CHECK(workspace_bytes >= plan.bytes, CSKV_EINVAL, "attend_with_partial: workspace %zu bytes < %zu required",
        workspace_bytes, plan.bytes);
  CHECK(plan.bytes == 0 || (workspace && aligned(workspace, 256)), CSKV_EINVAL,
        "attend_with_partial: workspace must be non-null and 256-byte aligned");
  a.part_in = partial;
  return hip_status(cskv::launch_attend(plan, a, workspace, reinterpret_cast<hipStream_t>(stream)),
                    "attend_with_partial launch");
}

size_t cskv_attend_partial_bytes(int64_t B, int32_t H, int32_t D) {
  if (B < 0 || H < 1 || H > 64 || (D != 128 && D != 512)) return 0;
  return (size_t)B * H * ((size_t)D + 2) * sizeof(float);
}

cskv_status cskv_attend_window_partial(const void* Q, int64_t B, int32_t H, int32_t D, int32_t window_dtype,
                                       const void* window, const float* window_scale, int32_t W,
                                       int64_t window_batch_stride, const int32_t* n_window, float softmax_scale,
                                       float* partial, void* stream) {
  cskv::AttendPlan plan;
  cskv::AttendArgs a;
  // dense reads of no cache rows: the keys are the window rows alone, in one split
  const cskv_status st = attend_prepare(Q, B, H, D, CSKV_BF16, nullptr, nullptr, 0, nullptr, 0, nullptr,
                                        window_dtype, window, window_scale, W, window_batch_stride, n_window,
                                        0, 1.0f, nullptr, softmax_scale, partial, 1, &plan, &a);
  if (st != CSKV_OK || B == 0) return st;
  CHECK(aligned(partial, 16), CSKV_EINVAL, "attend_window_partial: partial must be 16-byte aligned");
  CHECK(plan.splits == 1 && plan.bytes == 0, CSKV_EUNSUPPORTED, "attend_window_partial: no one-split plan");
  a.O = nullptr;
  a.part_out = partial;
  return hip_status(cskv::launch_attend(plan, a, nullptr, reinterpret_cast<hipStream_t>(stream)),
                    "attend_window_partial launch");
}

cskv_status cskv_attend_noalloc(const void* Q, int64_t B, int32_t H, int32_t D, int32_t cache_dtype,
                                const void* cache, const float* cache_scale, int64_t cache_rows,
                                const int32_t* ids, int32_t k, const int32_t* n_entries,
                                int32_t window_dtype, const void* window, const float* window_scale,
                                int32_t W, int64_t window_batch_stride, const int32_t* n_window,
                                int32_t rope_dims, float rope_base, const int64_t* q_pos,
                                float softmax_scale, float* O, int32_t splits, void* stream) {
  cskv::AttendPlan plan;
  cskv::AttendArgs a;
  const cskv_status st = attend_prepare(Q, B, H, D, cache_dtype, cache, cache_scale, cache_rows, ids, k, n_entries,
                                        window_dtype, window, window_scale, W, window_batch_stride, n_window,
                                        rope_dims, rope_base, q_pos, softmax_scale, O, splits, &plan, &a);
  if (st != CSKV_OK || B == 0) return st;
  CHECK(plan.bytes <= (size_t)CSKV_ATTEND_NOALLOC_SCRATCH_BYTES, CSKV_EUNSUPPORTED,
        "attend_noalloc: the call needs %zu bytes of scratch, more than the %d the library holds per device "
        "(use cskv_attend with a workspace, or fewer splits or sequences per call)",
        plan.bytes, CSKV_ATTEND_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (plan.bytes > 0) {
    const cskv_status s2 = scratch_of_current_device(&ws);
    if (s2 != CSKV_OK) return s2;
  }
  return hip_status(cskv::launch_attend(plan, a, ws, reinterpret_cast<hipStream_t>(stream)),
                    "attend_noalloc launch");
}

// ------------------------------------------------------------------ codecs

cskv_status cskv_encode_fp8_rows(int32_t in_dtype, const void* x, int64_t rows, int32_t D,
                                 uint8_t* codes, float* scale, void* stream) {
  CHECK(in_dtype == CSKV_BF16 || in_dtype == CSKV_F32, CSKV_EUNSUPPORTED,
        "encode_fp8_rows: input dtype %d (supported: bf16, f32)", in_dtype);
  CHECK(rows >= 0, CSKV_EINVAL, "encode_fp8_rows: negative rows");
  CHECK(D >= 64 && D <= 1024 && D % 64 == 0, CSKV_EUNSUPPORTED,
        "encode_fp8_rows: D=%d must be a multiple of 64 in [64, 1024]", D);
  if (rows == 0) return ok();
  CHECK(x && codes && scale, CSKV_EINVAL, "encode_fp8_rows: null pointer");
  CHECK((rows + 3) / 4 <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "encode_fp8_rows: too many rows");
  return hip_status(cskv::launch_encode_fp8_rows(in_dtype == CSKV_BF16, x, rows, D, codes, scale,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    "encode_fp8_rows launch");
}

cskv_status cskv_decode_fp8_rows(const uint8_t* codes, const float* scale, int64_t rows, int32_t D,
                                 float* out, void* stream) {
  CHECK(rows >= 0 && D >= 1, CSKV_EINVAL, "decode_fp8_rows: bad size");
  if (rows == 0) return ok();
  CHECK(codes && scale && out, CSKV_EINVAL, "decode_fp8_rows: null pointer");
  CHECK((rows * D + 255) / 256 <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "decode_fp8_rows: too large");
  return hip_status(cskv::launch_decode_fp8_rows(codes, scale, rows, D, out,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    "decode_fp8_rows launch");
}

cskv_status cskv_encode_fp4_g16(int32_t in_dtype, const void* x, int64_t rows, int32_t Di,
                                uint8_t* packed, uint8_t* scales, void* stream) {
  CHECK(in_dtype == CSKV_BF16 || in_dtype == CSKV_F32, CSKV_EUNSUPPORTED,
        "encode_fp4_g16: input dtype %d (supported: bf16, f32)", in_dtype);
  CHECK(rows >= 0 && Di >= 16 && Di % 16 == 0, CSKV_EINVAL,
        "encode_fp4_g16: Di=%d must be a positive multiple of 16", Di);
  if (rows == 0) return ok();
  CHECK(x && packed && scales, CSKV_EINVAL, "encode_fp4_g16: null pointer");
  CHECK(aligned(packed, 8), CSKV_EINVAL, "encode_fp4_g16: packed must be 8-byte aligned");
  CHECK((rows * (Di / 16) + 255) / 256 <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "encode_fp4_g16: too large");
  return hip_status(cskv::launch_encode_fp4_g16(in_dtype == CSKV_BF16, x, rows, Di, packed, scales,
                                                reinterpret_cast<hipStream_t>(stream)),
                    "encode_fp4_g16 launch");
}

cskv_status cskv_decode_fp4_g16(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                                int32_t Di, float* out, void* stream) {
  CHECK(rows >= 0 && Di >= 16 && Di % 16 == 0, CSKV_EINVAL,
        "decode_fp4_g16: Di=%d must be a positive multiple of 16", Di);
  if (rows == 0) return ok();
  CHECK(packed && scales && out, CSKV_EINVAL, "decode_fp4_g16: null pointer");
  CHECK(aligned(packed, 4), CSKV_EINVAL, "decode_fp4_g16: packed must be 4-byte aligned");
  CHECK((rows * (Di / 2) + 255) / 256 <= 0x7FFFFFFF, CSKV_EUNSUPPORTED, "decode_fp4_g16: too large");
  return hip_status(cskv::launch_decode_fp4_g16(packed, scales, rows, Di, out,
                                                reinterpret_cast<hipStream_t>(stream)),
                    "decode_fp4_g16 launch");
}

}  // extern "C"
