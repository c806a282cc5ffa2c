// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
// Every launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace cskv {

// ---- compress.hip
hipError_t launch_compress(int kind, const uint16_t* S, const float* gate, int64_t B, int64_t T,
                           int D, int64_t n, int64_t first_entry, int fmt, void* cache,
                           float* cache_scale, int64_t cache_rows, hipStream_t stream);
hipError_t launch_append(int kind, const uint16_t* s_new, const float* g_new, const int64_t* pos, int64_t B,
                         int D, uint16_t* ring, float* ring_gate, int W, int fmt, void* cache,
                         float* cache_scale, int64_t cache_rows, int32_t* n_entries, int32_t* n_window,
                         hipStream_t stream);

// ---- index_topk.hip
// Plan of the indexer: k_index_topk scores `chunk` entries per workgroup and
// writes the chunk's candidates as one list; the workgroup that scores a
// sequence's last chunk runs its selection. Workspace regions (byte offsets):
// the per-sequence histograms and arrival counters come first (they must be
// zero when a call starts and every call leaves them zero), then the lists'
// candidate counts and their candidate keys / entry numbers (room for every
// entry).
struct TopkPlan {
  int64_t chunk, n_chunks;     // entries per scoring workgroup, workgroups per sequence
  bool fused;                  // selection by the scoring launch's last chunk per sequence
  int threads;                 // scoring workgroup size
  int cand_cap, tb_cap;        // selection: candidates gathered in LDS, threshold-bin keys listed
  size_t lds_bytes;            // dynamic LDS per scoring workgroup
  size_t select_lds_bytes;     // dynamic LDS of a selection workgroup (separate launch)
  size_t off_hist, off_arrive, off_cnt, off_ckey, off_cidx;
  size_t zero_bytes;           // leading bytes that must be zero between calls
  size_t bytes;                // workspace bytes
};
bool plan_topk(int64_t B, int64_t n_max, int k, int chunk_hint, bool fp4, TopkPlan* plan);
hipError_t launch_index_topk(const TopkPlan& plan, const uint16_t* q_idx, bool fp4,
                             const void* k_idx, const uint8_t* k_scale, const int32_t* n_entries,
                             int64_t B, int64_t n_max, int Di, int k, int32_t* ids,
                             void* workspace, hipStream_t stream);

// ---- attend.hip
struct AttendPlan {
  int splits;            // key-row splits per sequence
  int64_t keys_per_split;
  size_t bytes;          // workspace bytes: the splits' partials (none with one split)
};
// Plans the key-slot splits of an attend call; sparse calls stage their entry
// ids in LDS, which bounds a split's length. False if no plan exists.
bool plan_attend(int64_t B, int H, int D, int64_t max_keys, bool sparse, int splits_hint, AttendPlan* plan);
struct AttendArgs {
  const uint16_t* Q;
  int64_t B;
  int H, D;
  bool cache_fp8;
  bool cache_mix;            // mixed rows (kFmtMix); cache_fp8 is false then
  bool cache_fp4;            // fp4 rows (kFmtFp4), group scales inside the row
  const void* cache;
  const float* cache_scale;
  int64_t cache_rows;
  const int32_t* ids;
  int k;
  const int32_t* n_entries;
  bool win_fp8;
  const void* window;
  const float* window_scale;
  int W;
  const int32_t* n_window;   // per-sequence window rows that are keys, or NULL for W
  int64_t win_bstride;
  int rope_dims;
  float rope_base;
  const int64_t* q_pos;
  float softmax_scale;
  float* O;
  // partials in the public layout: values [B][H][D] fp32 (normalised by their
  // own sum, not rotated), then (reference maximum in log2 units, sum) [B][H]
  float* part_out;           // one split: write this call's partial there instead of O
  const float* part_in;      // a partial over other keys, merged into O (or NULL)
  // rotary frequencies theta_i = rope_base^(-2i / rope_dims), i < rope_dims / 2,
  // in fp64, computed on the host (they depend on no device data). Last, so
  // that the scalar fields above share the argument block's first cache lines.
  double inv_freq[256];
};
hipError_t launch_attend(const AttendPlan& plan, const AttendArgs& a, void* workspace,
                         hipStream_t stream);

// ---- codec.hip
hipError_t launch_encode_fp8_rows(bool in_bf16, const void* x, int64_t rows, int D,
                                  uint8_t* codes, float* scale, hipStream_t stream);
hipError_t launch_decode_fp8_rows(const uint8_t* codes, const float* scale, int64_t rows, int D,
                                  float* out, hipStream_t stream);
hipError_t launch_encode_fp4_g16(bool in_bf16, const void* x, int64_t rows, int Di,
                                 uint8_t* packed, uint8_t* scales, hipStream_t stream);
hipError_t launch_decode_fp4_g16(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                                 int Di, float* out, hipStream_t stream);

}  // namespace cskv
