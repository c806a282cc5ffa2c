/*
 * cskv.h - decode-step attention over compressed shared-K/V caches, for
 * AMD Instinct MI355X (gfx950). C ABI of libcskv.so.
 *
 * Sources (cited by page title and section):
 *   [P1] "How DeepSeek V4 Uses Less Memory: KV Cache Explained"
 *   [P2] "DeepSeek V4 KV Cache" visual walkthrough, Steps 1-7
 *   [P3] "KV cache at 890 bytes per token: how DeepSeek squeezed attention memory"
 *
 * Conventions shared by every call
 *   - Every tensor argument is a plain pointer to caller-owned DEVICE memory,
 *     dense and row-major in the layout stated at the call; sizes are passed
 *     explicitly. The library never allocates or frees device memory and keeps
 *     no state between calls except a thread-local error string.
 *   - bf16 tensors are arrays of uint16 bit patterns.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     kernels on it and return; results are ready when the stream reaches them.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued, outputs are untouched and cskv_last_error()
 *     describes the problem. A fault inside a kernel is reported by the HIP
 *     runtime at the caller's next synchronisation, not by these calls.
 *   - Workspaces are caller-provided device buffers of at least the size the
 *     matching *_workspace() query returns (for the same arguments), 256-byte
 *     aligned. Two calls that share a workspace must be stream-ordered. The
 *     index_topk workspace carries state between calls (see there); the
 *     attend workspace does not.
 */
#ifndef CSKV_H
#define CSKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t cskv_status;
#define CSKV_OK             0
#define CSKV_EINVAL        (-1)  /* null pointer, bad size, inconsistent arguments */
#define CSKV_EUNSUPPORTED  (-2)  /* valid request this build has no kernel for */
#define CSKV_EHIP          (-3)  /* the HIP runtime refused a launch or query */

/* Element formats. */
#define CSKV_BF16      0  /* 2 bytes per channel */
#define CSKV_F32       1  /* 4 bytes per channel */
#define CSKV_FP8_E4M3  2  /* 1 byte per channel (OCP E4M3, max 448) + one fp32 scale per row */
#define CSKV_FP4_E2M1  3  /* 2 channels per byte (channel 2j in the low nibble) + one E4M3
                             scale byte per 16 channels */
#define CSKV_FP8_ROPE64 4 /* mixed attention-cache row ([P1] mixed-precision bullet and
                             quantisation paragraph: bf16 kept for the rotary channels, fp8 for
                             the rest): D-64 E4M3 codes, then the last 64 channels as bf16, i.e.
                             D+64 bytes per row (576 for D = 512), plus one fp32 scale per row
                             for the codes (max |x| over the D-64 channels / 448); D = 512 only */

/* Compression kinds ([P1] paragraphs "c4a" and "c128a"; [P2] Step 4). */
#define CSKV_C4A    0  /* an entry folds 8 consecutive states; entries start every 4 states */
#define CSKV_C128A  1  /* an entry folds 128 consecutive states; entries start every 128 */

const char* cskv_status_string(cskv_status s);
/* Text of the last error raised on the calling thread ("" if none). */
const char* cskv_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int32_t cskv_version(void);

/* ------------------------------------------------------------------------
 * Compression ([P1] "c4a (the milder scheme)", "c128a (the aggressive
 * scheme)"; [P2] Step 4 "Older shared states are compressed").
 *
 * Entry c of a sequence is  sum_j w_{c,j} * S[s*c + j],  j = 0..w-1, where
 * (w, s) = (8, 4) for C4A and (128, 128) for C128A and the weights are the
 * softmax of the window's own gate logits: w_{c,.} = softmax(gate[s*c .. s*c+w-1]).
 * Accumulation is fp32; the entry is rounded to bf16 (nearest even) or encoded
 * to fp8 rows exactly as cskv_encode_fp8_rows does.
 *
 *   S         [B, T, D] bf16   states of a span; row 0 is state first_entry*s
 *                              (for C4A, a span that continues an earlier one
 *                              therefore starts with the w-s = 4 carried states)
 *   gate      [B, T] fp32      one gate logit per state
 *   D         128 or 512
 *   cache     [B, cache_rows, D] bf16, or fp8 codes [B, cache_rows, D] plus
 *             cache_scale [B, cache_rows] fp32 (cache_dtype CSKV_FP8_E4M3), or mixed
 *             rows [B, cache_rows, D+64] bytes plus cache_scale (CSKV_FP8_ROPE64), or fp4
 *             rows [B, cache_rows, D/2 + D/16] bytes (CSKV_FP4_E2M1, D = 512: the
 *             packed E2M1 codes, then one E4M3 scale byte per 16 channels, encoded as
 *             cskv_encode_fp4_g16 does; [P3] "Three mechanisms", third; no cache_scale)
 *
 * Writes rows first_entry .. first_entry+n-1 of every sequence's cache, where
 * n = floor((T-w)/s)+1 complete windows (n = 0 when T < w: nothing is written).
 * EINVAL if first_entry+n > cache_rows.
 */
cskv_status cskv_compress(int32_t kind, const void* S, const float* gate, int64_t B, int64_t T,
                          int32_t D, int64_t first_entry, int32_t cache_dtype, void* cache,
                          float* cache_scale, int64_t cache_rows, void* stream);

/* ------------------------------------------------------------------------
 * Streaming decode append ([P1] paragraph on cache block types: besides the
 * compressed entries each layer keeps a constant-size compressor state and the
 * sliding window; [P1] "c4a" / "c128a" and [P2] Step 4: an entry exists once
 * its window of w states is complete, i.e. every 4 (C4A) or 128 (C128A)
 * decode steps; [P2] Step 6: the window holds the newest states).
 *
 * Sequence b appends state s_new[b] with gate logit g_new[b] as its token
 * pos[b] (absolute, 0-based; positions may differ between sequences; a
 * negative position skips the sequence). The caller-owned ring keeps each
 * sequence's newest W states and gate logits, token p in slot p mod W; it is
 * both the compressor's carry and the attention window (pass it to cskv_attend
 * as the window with n_window). The call stores the new state and logit in
 * their slot and, when token pos[b] completes an entry (C4A: pos % 4 == 3 and
 * pos >= 7, entry (pos-7)/4 from tokens pos-7 .. pos; C128A: pos % 128 == 127,
 * entry pos/128 from tokens pos-127 .. pos), writes that entry to its cache
 * row with exactly the arithmetic of cskv_compress (bit-identical to what
 * cskv_compress writes from the same states). Entries at rows >= cache_rows
 * are not written. The ring must already hold the entry's older states: append
 * each token of a sequence once, in order.
 *
 *   s_new      [B, D] bf16;  g_new [B] fp32;  pos [B] int64 device array
 *   ring       [B, W, D] bf16;  ring_gate [B, W] fp32;  W >= 8 (C4A), >= 128 (C128A)
 *   cache      any cache format of cskv_compress (bf16; fp8 rows or mixed rows with
 *              cache_scale; fp4 rows), cache_rows rows per sequence
 *   n_entries  [B] int32 or NULL: set to the sequence's entries in the cache,
 *              min(complete entries, cache_rows) (C4A: pos >= 7 ? (pos-7)/4+1
 *              : 0; C128A: (pos+1)/128), for cskv_index_topk / cskv_attend
 *   n_window   [B] int32 or NULL: set to min(pos+1, W), the ring rows that
 *              hold states (the leading ones until the ring has wrapped)
 * Sequences with a negative position keep their counts.
 * EINVAL for W below the entry's w, a null or misaligned pointer (s_new, ring
 * and cache 16-byte aligned) or a missing cache_scale; EUNSUPPORTED for D not
 * in {128, 512}, mixed or fp4 rows with D != 512, or an unknown cache format.
 * Positions are device data: the host cannot check them, so a position whose
 * older states were never appended folds whatever the ring holds.
 */
cskv_status cskv_append(int32_t kind, const void* s_new, const float* g_new, const int64_t* pos,
                        int64_t B, int32_t D, void* ring, float* ring_gate, int32_t W,
                        int32_t cache_dtype, void* cache, float* cache_scale, int64_t cache_rows,
                        int32_t* n_entries, int32_t* n_window, void* stream);

/* ------------------------------------------------------------------------
 * Indexer scores and exact top-k ([P1] "c4a": top-k selection, default
 * k = 512; [P2] Step 5 "The query now reads a mixed memory map": a learned
 * indexer scores the compressed blocks and the query reads only the chosen
 * ones).
 *
 * score[b, c] = sum_d q_idx[b, d] * key[b, c, d] with fp32 accumulation over
 * the entries c < n_entries[b]; ids[b] receives the k best entries under the
 * order (score descending, entry ascending on ties; NaN below every number),
 * listed in ascending entry order and padded with -1 when fewer than k exist.
 * Whenever every partial sum is exact in fp32 (e.g. small integers times
 * dyadic keys), the ids are bit-exact against any exact evaluation.
 *
 *   q_idx     [B, Di] bf16
 *   key_dtype CSKV_BF16: k_idx [B, n_max, Di] bf16, k_scale NULL
 *             CSKV_FP4_E2M1: k_idx [B, n_max, Di/2] packed codes,
 *                            k_scale [B, n_max, Di/16] E4M3 scale codes
 *   n_entries [B] int32 device array of valid entry counts (clamped to
 *             [0, n_max]), or NULL for n_max everywhere
 *   Di        32 or 128;  1 <= k <= 2048
 *   ids       [B, k] int32
 *   chunk     entries scored per workgroup: 0 = automatic, else a multiple
 *             of 256 in [256, 16384]
 *   workspace cskv_index_topk_workspace() bytes. Its leading region holds
 *             per-sequence histograms and chunk arrival counters that must be
 *             zero when a call starts: zero-fill the workspace before the first
 *             call, and again before a call with different B, n_max, k or chunk
 *             or after the buffer served another purpose. Every completed call
 *             leaves that region zero (whatever n_entries held), so calls with
 *             the same arguments can reuse the workspace as it is. The call is
 *             one kernel launch: the workgroup that scores a sequence's last
 *             chunk also selects that sequence's ids. Two calls in flight at
 *             once on one workspace (two streams) corrupt each other.
 * EUNSUPPORTED if a sequence would need more than 2048 chunks (n_max > 2048 *
 * chunk; with automatic chunking, n_max > 33554432).
 */
size_t cskv_index_topk_workspace(int64_t B, int64_t n_max, int32_t Di, int32_t k,
                                 int32_t key_dtype, int32_t chunk);
cskv_status cskv_index_topk(const void* q_idx, int32_t key_dtype, const void* k_idx,
                            const uint8_t* k_scale, const int32_t* n_entries, int64_t B,
                            int64_t n_max, int32_t Di, int32_t k, int32_t* ids, int32_t chunk,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Shared-K/V attention with inverse RoPE ([P2] Step 3 "DeepSeek V4 makes one
 * vector do both jobs": the same cached state is the key and the value;
 * [P2] Step 6 "The newest tokens stay uncompressed": the window; [P1]
 * "Shared key and value": inverse RoPE on the output).
 *
 * For each sequence b and head h, over the key rows K_j = the selected cache
 * entries followed by the window rows:
 *   O[b,h] = invrope( sum_j softmax_j(softmax_scale * Q[b,h].K_j) * K_j )
 * with one softmax over entries and window together; fp8 rows are
 * value(code) * row scale. invrope turns each pair (2i, 2i+1) of the last
 * rope_dims channels by -q_pos[b] * rope_base^(-2i/rope_dims) (angles in
 * fp64). A sequence with no key rows gets O = 0.
 *
 *   Q            [B, H, D] bf16;  1 <= H <= 64;  D 128 or 512
 *   cache        [B, cache_rows, D] bf16, or fp8 codes + cache_scale [B, cache_rows] fp32,
 *                or mixed rows (CSKV_FP8_ROPE64, D = 512) + cache_scale, or fp4 rows
 *                (CSKV_FP4_E2M1, D = 512, layout as in cskv_compress); the scale of a
 *                mixed row must be positive and finite, as cskv_compress writes it (an
 *                all-zero row gets 1): a row read with another scale has undefined values
 *   ids          [B, k] int32 entry ids (ids < 0 or >= cache_rows are skipped),
 *                or NULL for dense attention over entries 0 .. n_entries[b]-1
 *   n_entries    dense mode only: [B] int32 device counts, or NULL for cache_rows
 *   window       rows at window + b*window_batch_stride*D (elements), W of them
 *                (W may be 0); window_dtype CSKV_BF16 or CSKV_FP8_E4M3 (then
 *                window_scale at window_scale + b*window_batch_stride)
 *   n_window     [B] int32 device counts or NULL: only the first n_window[b]
 *                window rows of sequence b (clamped to [0, W]) are keys; NULL
 *                = all W (a ring from cskv_append that has not wrapped yet)
 *   rope_dims    even, <= D (0 = no rotation);  q_pos [B] int64 device positions
 *   O            [B, H, D] fp32
 *   splits       key-row splits per sequence: 0 = automatic, else >= 1 (sparse
 *                reads split further so that a split covers at most 2048 ids)
 *   workspace    cskv_attend_workspace() bytes (the query covers both dense and
 *                sparse use of the same sizes); no state is kept in it
 * EUNSUPPORTED for sparse reads of more than 524288 key slots.
 */
size_t cskv_attend_workspace(int64_t B, int32_t H, int32_t D, int64_t max_keys, int32_t splits);
cskv_status cskv_attend(const void* Q, int64_t B, int32_t H, int32_t D, int32_t cache_dtype,
                        const void* cache, const float* cache_scale, int64_t cache_rows,
                        const int32_t* ids, int32_t k, const int32_t* n_entries,
                        int32_t window_dtype, const void* window, const float* window_scale,
                        int32_t W, int64_t window_batch_stride, const int32_t* n_window,
                        int32_t rope_dims, float rope_base, const int64_t* q_pos,
                        float softmax_scale, float* O,
                        int32_t splits, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Attention in two parts that can overlap ([P3] "Three mechanisms instead of
 * one trick": the extra bookkeeping must not eat the saving; [P2] Step 6
 * "The newest tokens stay uncompressed": the window rows do not depend on
 * the indexer). The window-only part runs while the indexer selects entries
 * (on another stream); the attend over the selected entries then merges it
 * with log-sum-exp weights, so that both parts together give cskv_attend's O
 * over entries and window in one softmax.
 *
 * A partial of B sequences and H heads (caller-owned device memory of
 * cskv_attend_partial_bytes(B, H, D) bytes, 16-byte aligned):
 *   values [B, H, D] fp32:  sum_j p_j K_j / sum_j p_j over the partial's keys
 *                           (no rotation), with p_j = exp2(x_j - m)
 *   stats  [B, H] x (m, l) fp32 pairs, after the values:  x_j = softmax_scale
 *          * log2(e) * Q[b,h].K_j, m a reference (the largest x_j, or a value
 *          within 64 of it), l = sum_j exp2(x_j - m); l = 0 when there was
 *          no key (then the values are 0 and m means nothing)
 *
 * cskv_attend_window_partial: the partial over the window rows alone
 * (arguments as in cskv_attend; W may be 0, n_window may be NULL). It needs
 * no workspace.
 *
 * cskv_attend_with_partial: cskv_attend (same arguments, results and
 * workspace) whose O also covers the keys of `partial` (typically the call
 * passes W = 0 and the window partial of the same Q). The partial must be
 * complete before the call starts on `stream` (record an event after the
 * partial's call and wait for it on `stream`).
 * EINVAL for a null or misaligned partial; cskv_attend_partial_bytes returns
 * 0 for unsupported sizes.
 */
size_t cskv_attend_partial_bytes(int64_t B, int32_t H, int32_t D);
cskv_status cskv_attend_window_partial(const void* Q, int64_t B, int32_t H, int32_t D, int32_t window_dtype,
                                       const void* window, const float* window_scale, int32_t W,
                                       int64_t window_batch_stride, const int32_t* n_window, float softmax_scale,
                                       float* partial, void* stream);
cskv_status cskv_attend_with_partial(const void* Q, int64_t B, int32_t H, int32_t D, int32_t cache_dtype,
                                     const void* cache, const float* cache_scale, int64_t cache_rows,
                                     const int32_t* ids, int32_t k, const int32_t* n_entries,
                                     int32_t window_dtype, const void* window, const float* window_scale,
                                     int32_t W, int64_t window_batch_stride, const int32_t* n_window,
                                     int32_t rope_dims, float rope_base, const int64_t* q_pos,
                                     float softmax_scale, const float* partial, float* O,
                                     int32_t splits, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * cskv_attend without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).
 *
 * Arguments, results and errors are those of cskv_attend; the split partials
 * that cskv_attend keeps in the caller's workspace live instead in a scratch
 * array of CSKV_ATTEND_NOALLOC_SCRATCH_BYTES that the library holds in each
 * GPU's memory for the life of the process (its device address is looked up
 * on the first call on a device). The call allocates nothing. A call whose
 * plan needs more scratch than that returns CSKV_EUNSUPPORTED with a message
 * naming both sizes (the plan needs B * splits * 64 * (2 D + 8) bytes; e.g.
 * 16.9 MB for 16 sequences of 16 splits at D = 512). Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two streams,
 * or two threads with their own streams) race and give wrong results; calls
 * ordered on one stream do not. The scratch keeps no state between calls.
 */
#define CSKV_ATTEND_NOALLOC_SCRATCH_BYTES (32 << 20)
cskv_status cskv_attend_noalloc(const void* Q, int64_t B, int32_t H, int32_t D, int32_t cache_dtype,
                                const void* cache, const float* cache_scale, int64_t cache_rows,
                                const int32_t* ids, int32_t k, const int32_t* n_entries,
                                int32_t window_dtype, const void* window, const float* window_scale,
                                int32_t W, int64_t window_batch_stride, const int32_t* n_window,
                                int32_t rope_dims, float rope_base, const int64_t* q_pos,
                                float softmax_scale, float* O, int32_t splits, void* stream);

/* ------------------------------------------------------------------------
 * Cache codecs ([P1] quantisation paragraph: fp8 attention cache, "partly
 * token-wise"; fp4 indexer cache. [P3] "Three mechanisms", third: E2M1 values
 * with one E4M3 scale per 16 channels). The same device routines run fused
 * inside the kernels above.
 *
 * fp8 rows: scale = max|x| / 448 (fp32), code = E4M3 nearest of x / scale,
 *   ties to even, saturating at 448; an all-zero row gets scale 1.
 * fp4 groups of 16: scale code = E4M3 nearest of max|x| / 6, raised to the
 *   smallest subnormal if it rounds to zero while max|x| > 0; code = E2M1
 *   nearest of x / scale, ties to even, saturating at 6; zero scale -> zero codes.
 *
 *   x: [rows, D] in_dtype CSKV_BF16 or CSKV_F32; D a multiple of 16 (fp4) or
 *   of 64 (fp8, D <= 1024). Decoders write fp32.
 */
cskv_status cskv_encode_fp8_rows(int32_t in_dtype, const void* x, int64_t rows, int32_t D,
                                 uint8_t* codes, float* scale, void* stream);
cskv_status cskv_decode_fp8_rows(const uint8_t* codes, const float* scale, int64_t rows,
                                 int32_t D, float* out, void* stream);
cskv_status cskv_encode_fp4_g16(int32_t in_dtype, const void* x, int64_t rows, int32_t Di,
                                uint8_t* packed, uint8_t* scales, void* stream);
cskv_status cskv_decode_fp4_g16(const uint8_t* packed, const uint8_t* scales, int64_t rows,
                                int32_t Di, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSKV_H */
