/*
 * pkd.h - C ABI of the paged KV decode library (MI355X / gfx950).
 *
 * Paged decode attention over a block-table KV cache: one query token per
 * sequence, grouped-query heads, split-KV partials that carry the softmax
 * state (max, sum), a combine pass into BF16, and BF16 / FP8-E4M3 / NVFP4
 * caches filled through a slot mapping. The calls and their argument order
 * follow the launchers of the metrale API page
 * "metrale_model_layers/layers/ops/prefill_attn_b.rs" (the GPU-backend and
 * kernel-handle arguments dropped, the stream passed as a hipStream_t).
 *
 * Conventions for every call
 *  - Buffers are device pointers owned by the caller. The library never
 *    allocates, frees or synchronizes; every call only enqueues kernels on
 *    `stream` (0 = the null stream) and returns. No call reads device data
 *    back to the host, so a sequence of calls can be captured in a HIP graph.
 *  - BF16 data is passed as its 16-bit patterns (uint16_t). Counts are
 *    uint32_t, byte sizes uint64_t, indices int32_t (page ids, sequence
 *    lengths, slots), scales float.
 *  - Return value: PKD_OK (0), or a negative status, in which case nothing
 *    was enqueued (except PKD_ERR_LAUNCH, reported after a launch failed).
 *    Only host-side arguments are validated; values that live in device
 *    memory (sequence lengths, block-table entries, slots) are the caller's
 *    contract as stated on each call.
 *  - A call with no work (num_tokens, num_seqs or n_elems equal to 0) is a
 *    valid no-op and may pass null buffers.
 *  - Supported shapes: head_dim in {64, 128, 256, 512}; block_size in
 *    {16, 32, 64, 128, 256}; num_q_heads a multiple of num_kv_heads (any
 *    group size); 1 <= num_splits <= PKD_MAX_SPLITS.
 *  - Alignment: every buffer is 16-byte aligned; element strides (q_stride,
 *    key_stride, value_stride) are multiples of 8 elements; byte strides and
 *    section sizes of the FP8 / NVFP4 caches are multiples of 16.
 *
 * Cache layouts (K and V are two separate pools with the same layout):
 *  - BF16:  [num_pages][block_size][num_kv_heads][head_dim] elements; page p
 *           starts at element p * block_size * num_kv_heads * head_dim (the
 *           order stated for the BF16 split-K launcher on the metrale page).
 *  - FP8:   the same index order, one E4M3FN byte per element, page p starts
 *           at byte p * cache_stride.
 *  - NVFP4: page p starts at byte p * block_stride_bytes. Its first
 *           data_section_bytes hold E2M1 codes, the E4M3FN scales follow
 *           (reshape_and_cache_nvfp4 on the metrale page). Element d of
 *           (offset o, kv head h) is a nibble of byte (o*Hkv + h)*D/2 + d/2,
 *           the low nibble holding the even element; its group scale is byte
 *           data_section_bytes + (o*Hkv + h)*D/16 + d/16.
 *  A slot s names page s / block_size, offset s % block_size.
 */
#ifndef PKD_H
#define PKD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKD_OK 0
#define PKD_ERR_INVALID_ARG (-1) /* null buffer with work to do, bad count, stride or alignment */
#define PKD_ERR_UNSUPPORTED (-2) /* head_dim / block_size / num_splits outside the supported set,
                                  or a split-K launch of more than 2^30 16-key tiles (sequences x
                                  kv heads x the tiles a block-table row or window can hold) */
#define PKD_ERR_LAUNCH (-3)      /* the HIP runtime reported an error after the launch */
#define PKD_ERR_SCRATCH (-4)     /* paged_decode_attn_bf16_noalloc: the call needs more than
                                    PKD_SCRATCH_BYTES of split-K workspace */

#define PKD_MAX_SPLITS 4096u

#if defined(__GNUC__)
#define PKD_API __attribute__((visibility("default")))
#else
#define PKD_API
#endif

/* ---------------------------------------------------------------- cache writes
 * Write each token's K and V rows into the paged cache at its slot_mapping
 * slot; one workgroup per token (reshape_and_cache_nvfp4 on the metrale page).
 *   key, value    BF16 [num_tokens] rows; token t, kv head h starts at element
 *                 t*key_stride + h*head_dim (resp. value_stride).
 *   k_cache, v_cache  the pools described above.
 *   slot_mapping  int32 [num_tokens]. A negative slot skips the token. Valid
 *                 slots must lie inside the pools and be distinct (two tokens
 *                 writing one slot race). Bytes of slots not written, padding
 *                 between sections and after a page's scales keep their value.
 * Encoding (exact, bit for bit the same as the CPU oracle):
 *   FP8:   code = E4M3FN(x / scale): IEEE float32 division, round to nearest
 *          with ties to the even code, |y| >= 448 saturates to +-448, NaN ->
 *          0x7F, the sign of y kept (a negative value that rounds to zero is
 *          0x80); scale == 0 writes code 0.
 *   NVFP4: per group of 16 consecutive elements of a row: amax = max |x|;
 *          scale code = E4M3FN(amax / 6) with the same rounding; S its value;
 *          S == 0 -> all 16 codes 0; else code_i = E2M1(x_i / S) (float32
 *          division, ties to the even code, |y| >= 6 saturates, sign kept).
 *          Non-finite inputs are outside the contract.
 */
PKD_API int reshape_and_cache_bf16(const uint16_t* key, const uint16_t* value,
                                   uint16_t* k_cache, uint16_t* v_cache,
                                   const int32_t* slot_mapping, uint32_t num_tokens,
                                   uint32_t num_kv_heads, uint32_t head_dim,
                                   uint32_t block_size, uint32_t key_stride,
                                   uint32_t value_stride, hipStream_t stream);

/* cache_stride: bytes between consecutive pages, >= block_size*num_kv_heads*head_dim. */
PKD_API int reshape_and_cache_fp8(const uint16_t* key, const uint16_t* value,
                                  uint8_t* k_cache, uint8_t* v_cache,
                                  const int32_t* slot_mapping, uint32_t num_tokens,
                                  uint32_t num_kv_heads, uint32_t head_dim,
                                  uint32_t block_size, uint32_t key_stride,
                                  uint32_t value_stride, float k_scale, float v_scale,
                                  uint64_t cache_stride, hipStream_t stream);

/* data_section_bytes >= block_size*num_kv_heads*head_dim/2;
 * block_stride_bytes >= data_section_bytes + block_size*num_kv_heads*head_dim/16. */
PKD_API int reshape_and_cache_nvfp4(const uint16_t* key, const uint16_t* value,
                                    uint8_t* k_cache, uint8_t* v_cache,
                                    const int32_t* slot_mapping, uint32_t num_tokens,
                                    uint32_t num_kv_heads, uint32_t head_dim,
                                    uint32_t block_size, uint32_t key_stride,
                                    uint32_t value_stride, uint64_t block_stride_bytes,
                                    uint64_t data_section_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- FP8 calibration
 * *out_max = max(*out_max, max_i |data[i]|) over n_elems BF16 values, folded in
 * with an atomic max (bf16_absmax on the metrale page). NaN inputs are
 * ignored. *out_max must hold a non-negative float on entry: the caller zeroes
 * it before a new tensor. The FP8 scale of a tensor is then absmax / 448. */
PKD_API int bf16_absmax(const uint16_t* data, float* out_max, uint64_t n_elems,
                        hipStream_t stream);

/* ---------------------------------------------------------------- split-K decode
 * Paged decode attention, split-KV pass (paged_decode_attn_splitk_* on the
 * metrale page). For sequence b and q head h:
 *   kv head g = h / (num_q_heads / num_kv_heads);
 *   L = seq_lens[b]; lo = (sliding_window > 0 && L > sliding_window)
 *                         ? L - sliding_window : 0;
 *   keys j in [lo, L), row j at page block_tables[b*max_blocks_per_seq + j/bs],
 *   offset j % bs; logit s_j = (q . k_j) * scale (the scale applied after the
 *   dot); output = softmax(s) . V.
 * Splits: the keys of every (b, h) are divided into at most num_splits
 *   pieces, each a set of 16-key tiles (a contiguous range over a batch; for
 *   one sequence without a window, every Q-th tile); how the launch's work is
 *   divided among waves is internal (equal key counts across the waves it
 *   launches, whatever the batch's length mix).
 * Workspace: float32 [num_seqs][num_q_heads][num_splits][head_dim + 2]; slot i
 *   of (b, h) holds a piece's o (head_dim values, its softmax-normalized
 *   output), m and l = sum of exp(s_j - m), where m is a reference logit at
 *   most 8*ln(2) below the piece's largest logit (and never above it). A
 *   slot that holds no keys has l = 0; a slot with l < 0 is an end marker:
 *   it and every later slot of (b, h) hold no keys, whatever they contain.
 *   The o of a slot without keys is unspecified. Size:
 *   paged_decode_workspace_bytes(). Any contents on entry are fine.
 *   q:            BF16; row of (b, h) at element b*q_stride + h*head_dim,
 *                 q_stride >= num_q_heads*head_dim.
 *   block_tables: int32 [num_seqs][max_blocks_per_seq]; the entries of the
 *                 first ceil(L/bs) columns of row b must be valid pages.
 *   seq_lens:     int32 [num_seqs], 0 <= L <= max_blocks_per_seq*block_size
 *                 (a longer L is read as max_blocks_per_seq*block_size, so
 *                 no read passes the sequence's block-table row).
 *   scale:        softmax scale (1/sqrt(head_dim) typically), used as given.
 *   sliding_window: 0 = attend to every key.
 * Follow with paged_decode_attn_reduce() on the same stream. */
PKD_API int paged_decode_attn_splitk_bf16(const uint16_t* q, const uint16_t* k_cache,
                                          const uint16_t* v_cache, float* workspace,
                                          const int32_t* block_tables, const int32_t* seq_lens,
                                          uint32_t max_blocks_per_seq, uint32_t num_q_heads,
                                          uint32_t num_kv_heads, uint32_t head_dim,
                                          uint32_t block_size, float scale, uint32_t num_splits,
                                          uint32_t q_stride, uint32_t num_seqs,
                                          uint32_t sliding_window, hipStream_t stream);

/* FP8-E4M3FN cache: k_j = code * k_scale, v_j = code * v_scale; cache_stride
 * as for reshape_and_cache_fp8. */
PKD_API int paged_decode_attn_splitk_fp8(const uint16_t* q, const uint8_t* k_cache,
                                         const uint8_t* v_cache, float* workspace,
                                         const int32_t* block_tables, const int32_t* seq_lens,
                                         uint32_t max_blocks_per_seq, uint32_t num_q_heads,
                                         uint32_t num_kv_heads, uint32_t head_dim,
                                         uint32_t block_size, float scale, uint32_t num_splits,
                                         float k_scale, float v_scale, uint32_t q_stride,
                                         uint64_t cache_stride, uint32_t num_seqs,
                                         uint32_t sliding_window, hipStream_t stream);

/* NVFP4 cache: element = E2M1 value * E4M3 group scale. The sliding_window
 * argument is an extension of the metrale NVFP4 launcher (0 = off). */
PKD_API int paged_decode_attn_splitk_nvfp4(const uint16_t* q, const uint8_t* k_cache,
                                           const uint8_t* v_cache, float* workspace,
                                           const int32_t* block_tables, const int32_t* seq_lens,
                                           uint32_t max_blocks_per_seq, uint32_t num_q_heads,
                                           uint32_t num_kv_heads, uint32_t head_dim,
                                           uint32_t block_size, float scale, uint32_t num_splits,
                                           uint32_t q_stride, uint64_t block_stride_bytes,
                                           uint64_t data_section_bytes, uint32_t num_seqs,
                                           uint32_t sliding_window, hipStream_t stream);

/* ---------------------------------------------------------------- split-K with append
 * The decode step's cache write and split-K pass in one launch, for the usual
 * decode case where every sequence appends one token at its last position:
 * the new token of sequence b (row b of `key` / `value`: num_kv_heads *
 * head_dim BF16 values at key + b * key_stride) is written to position
 * seq_lens[b] - 1, i.e. page block_tables[b][(L-1) / block_size], offset
 * (L-1) % block_size, encoded exactly as reshape_and_cache_{bf16,fp8,nvfp4}
 * encode it; then the same pass as paged_decode_attn_splitk_* runs over keys
 * [lo, L), the new one included. Equivalent to reshape_and_cache_* of those
 * tokens (slot_mapping[b] = that position's slot) followed by
 * paged_decode_attn_splitk_*. Sequences with seq_lens[b] == 0 append
 * nothing. Follow with paged_decode_attn_reduce. */
PKD_API int paged_decode_attn_splitk_append_bf16(
    const uint16_t* q, const uint16_t* key, const uint16_t* value, uint16_t* k_cache,
    uint16_t* v_cache, float* workspace, const int32_t* block_tables, const int32_t* seq_lens,
    uint32_t max_blocks_per_seq, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t num_splits, uint32_t q_stride, uint32_t key_stride,
    uint32_t value_stride, uint32_t num_seqs, uint32_t sliding_window, hipStream_t stream);

/* FP8-E4M3FN cache: codes of x / k_scale and x / v_scale. */
PKD_API int paged_decode_attn_splitk_append_fp8(
    const uint16_t* q, const uint16_t* key, const uint16_t* value, uint8_t* k_cache,
    uint8_t* v_cache, float* workspace, const int32_t* block_tables, const int32_t* seq_lens,
    uint32_t max_blocks_per_seq, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t num_splits, float k_scale, float v_scale,
    uint32_t q_stride, uint32_t key_stride, uint32_t value_stride, uint64_t cache_stride,
    uint32_t num_seqs, uint32_t sliding_window, hipStream_t stream);

/* NVFP4 cache: E2M1 codes with one E4M3 scale per 16 values. */
PKD_API int paged_decode_attn_splitk_append_nvfp4(
    const uint16_t* q, const uint16_t* key, const uint16_t* value, uint8_t* k_cache,
    uint8_t* v_cache, float* workspace, const int32_t* block_tables, const int32_t* seq_lens,
    uint32_t max_blocks_per_seq, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t num_splits, uint32_t q_stride, uint32_t key_stride,
    uint32_t value_stride, uint64_t block_stride_bytes, uint64_t data_section_bytes,
    uint32_t num_seqs, uint32_t sliding_window, hipStream_t stream);

/* ---------------------------------------------------------------- combine
 * Merge the split partials of every (b, h) into output BF16
 * [num_seqs][num_q_heads][head_dim] (contiguous), one combine for every cache
 * type (paged_decode_attn_reduce_fp8 on the metrale page): over the slots
 * before the first end marker that have l_i > 0, M = max m_i;
 * w_i = l_i * exp(m_i - M); out = sum w_i o_i / max(sum w_i, 1e-20), rounded
 * to BF16 (nearest even). A
 * sequence with seq_lens[b] == 0 gets zeros. Deterministic: a fixed
 * summation order. */
PKD_API int paged_decode_attn_reduce(const float* workspace, uint16_t* output,
                                     const int32_t* seq_lens, uint32_t num_q_heads,
                                     uint32_t head_dim, uint32_t num_splits, uint32_t num_seqs,
                                     hipStream_t stream);

/* ---------------------------------------------------------------- whole decode
 * The whole decode into BF16 output [num_seqs][num_q_heads][head_dim]
 * (contiguous), in one call: the same attention as a split-K call followed by
 * paged_decode_attn_reduce. The argument order follows the non-split launcher
 * paged_decode_attn_nvfp4 of the metrale page (q, caches, output,
 * block_tables, seq_lens, max_blocks_per_seq, num_seqs, head counts,
 * head_dim, block_size, scale, q_stride, cache layout); sliding_window,
 * workspace and num_splits are extensions.
 *   num_splits == 1: one workgroup per (sequence, kv head, 16 q heads) row
 *     writes the output, as the non-split launcher does (BF16 and FP8 rows
 *     up to head_dim 256: four waves that take the row's tiles in turn and
 *     merge in LDS); workspace is not used (may be null). Only
 *     num_seqs x num_kv_heads workgroups then read the whole cache: slow
 *     for few, long sequences (one sequence of 32K keys, 8 kv heads: some
 *     50x the split path).
 *   num_splits > 1: the split-K pass and the combine, as two launches on
 *     `stream`; workspace as for the split-K calls
 *     (paged_decode_workspace_bytes). paged_decode_num_splits() gives the
 *     split count to use. Short rows are the exception: when every
 *     sequence's keys fit 12 tiles of 16 (by max_blocks_per_seq x
 *     block_size, or by the window) and all num_seqs x num_kv_heads rows
 *     are resident at once (BF16 and FP8 rows up to head_dim 256, G <= 16),
 *     the call runs the num_splits == 1 form in one launch, which is faster
 *     there (one sequence of 128 keys, 8 kv heads: 6.2 against 7.6 us), and
 *     leaves the workspace untouched.
 * Sequences with seq_lens[b] == 0 get zeros. Other arguments and errors as
 * for the split-K calls; output must be 16-byte aligned. */
PKD_API int paged_decode_attn_bf16(const uint16_t* q, const uint16_t* k_cache,
                                   const uint16_t* v_cache, uint16_t* output,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   uint32_t max_blocks_per_seq, uint32_t num_seqs,
                                   uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                                   uint32_t block_size, float scale, uint32_t q_stride,
                                   uint32_t sliding_window, float* workspace, uint32_t num_splits,
                                   hipStream_t stream);

/* FP8-E4M3FN cache, as paged_decode_attn_splitk_fp8. */
PKD_API int paged_decode_attn_fp8(const uint16_t* q, const uint8_t* k_cache,
                                  const uint8_t* v_cache, uint16_t* output,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  uint32_t max_blocks_per_seq, uint32_t num_seqs,
                                  uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                                  uint32_t block_size, float scale, float k_scale, float v_scale,
                                  uint32_t q_stride, uint64_t cache_stride,
                                  uint32_t sliding_window, float* workspace, uint32_t num_splits,
                                  hipStream_t stream);

/* NVFP4 cache (paged_decode_attn_nvfp4 on the metrale page, extended). */
PKD_API int paged_decode_attn_nvfp4(const uint16_t* q, const uint8_t* k_cache,
                                    const uint8_t* v_cache, uint16_t* output,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    uint32_t max_blocks_per_seq, uint32_t num_seqs,
                                    uint32_t num_q_heads, uint32_t num_kv_heads,
                                    uint32_t head_dim, uint32_t block_size, float scale,
                                    uint32_t q_stride, uint64_t block_stride_bytes,
                                    uint64_t data_section_bytes, uint32_t sliding_window,
                                    float* workspace, uint32_t num_splits, hipStream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): paged_decode_attn_bf16
 * without the workspace argument. Its split-K partials go to a static device
 * array of PKD_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call allocates and frees nothing. num_splits
 * > 1 needs paged_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 * num_splits) <= PKD_SCRATCH_BYTES, else PKD_ERR_SCRATCH (nothing enqueued);
 * num_splits == 1 uses no scratch. Calls on one GPU share the array: calls
 * that overlap on one GPU (different streams, not ordered) race, calls in
 * one stream do not. Other arguments, results and errors as for
 * paged_decode_attn_bf16. */
#define PKD_SCRATCH_BYTES (16u << 20)
PKD_API int paged_decode_attn_bf16_noalloc(const uint16_t* q, const uint16_t* k_cache,
                                           const uint16_t* v_cache, uint16_t* output,
                                           const int32_t* block_tables, const int32_t* seq_lens,
                                           uint32_t max_blocks_per_seq, uint32_t num_seqs,
                                           uint32_t num_q_heads, uint32_t num_kv_heads,
                                           uint32_t head_dim, uint32_t block_size, float scale,
                                           uint32_t q_stride, uint32_t sliding_window,
                                           uint32_t num_splits, hipStream_t stream);

/* ---------------------------------------------------------------- query blocks
 * Multi-token paged attention over the same block table: q_len query tokens
 * per sequence (chunked prefill, speculative verify), each attending the
 * sequence's paged keys (pegainfer issue #1008, the paged prefill launch body
 * of its Description; AstrAI csrc/tests commit log, the causal_offset,
 * stride-addressing and layout bullets). The block is the sequence's newest
 * q_len tokens, already written to the cache (a reshape_and_cache call
 * first), so token i of sequence b sits at position p = seq_lens[b] - q_len
 * + i, the per-sequence form of a causal offset that names the first query
 * position.
 *   causal != 0: token i attends keys max(0, p + 1 - W) .. p, W =
 *     sliding_window (0: from key 0). A token with p < 0 gets zeros.
 *   causal == 0 (the causal offset -1): every token attends what a
 *     one-token decode would, keys [max(0, L - W), L).
 * q: BF16, token i of sequence b at q + b*q_stride + i*q_token_stride
 *   (elements, multiples of 8; q_token_stride >= num_q_heads*head_dim when
 *   q_len > 1), heads head_dim apart, 16-byte aligned.
 * output: BF16 [num_seqs][q_len][num_q_heads][head_dim], contiguous.
 * num_splits == 1: one pass writes the output (workspace unused, may be
 *   null; one workgroup per row, slow for long contexts, see
 *   paged_prefill_num_splits). num_splits > 1: the split-K pass and the
 *   combine, two launches;
 *   workspace of paged_decode_workspace_bytes(num_seqs, num_q_heads * q_len,
 *   head_dim, num_splits) bytes, laid out [num_seqs][q_len][num_q_heads]
 *   [num_splits][head_dim + 2] (the combine is paged_decode_attn_reduce with
 *   num_q_heads * q_len query rows per sequence).
 * The q heads of one kv head and the block's tokens share the kv head's one
 * pass over its pages, group * q_len query rows per 16-column tile; blocks
 * with group * q_len > 16 take ceil(group * q_len / 16) passes.
 * Errors: as for the whole-decode calls; PKD_ERR_INVALID_ARG for q_len == 0 or a
 * query stride too small, PKD_ERR_UNSUPPORTED for q_len > 4096. */
PKD_API int paged_prefill_attn_bf16(const uint16_t* q, const uint16_t* k_cache,
                                    const uint16_t* v_cache, uint16_t* output,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    uint32_t max_blocks_per_seq, uint32_t num_seqs,
                                    uint32_t q_len, uint32_t num_q_heads, uint32_t num_kv_heads,
                                    uint32_t head_dim, uint32_t block_size, float scale,
                                    uint32_t q_stride, uint32_t q_token_stride, uint32_t causal,
                                    uint32_t sliding_window, float* workspace,
                                    uint32_t num_splits, hipStream_t stream);

/* FP8-E4M3FN cache: k_scale, v_scale and cache_stride as for
 * paged_decode_attn_splitk_fp8. */
PKD_API int paged_prefill_attn_fp8(const uint16_t* q, const uint8_t* k_cache,
                                   const uint8_t* v_cache, uint16_t* output,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   uint32_t max_blocks_per_seq, uint32_t num_seqs,
                                   uint32_t q_len, uint32_t num_q_heads, uint32_t num_kv_heads,
                                   uint32_t head_dim, uint32_t block_size, float scale,
                                   float k_scale, float v_scale, uint32_t q_stride,
                                   uint32_t q_token_stride, uint64_t cache_stride,
                                   uint32_t causal, uint32_t sliding_window, float* workspace,
                                   uint32_t num_splits, hipStream_t stream);

/* NVFP4 cache: block_stride_bytes and data_section_bytes as for
 * paged_decode_attn_splitk_nvfp4. */
PKD_API int paged_prefill_attn_nvfp4(const uint16_t* q, const uint8_t* k_cache,
                                     const uint8_t* v_cache, uint16_t* output,
                                     const int32_t* block_tables, const int32_t* seq_lens,
                                     uint32_t max_blocks_per_seq, uint32_t num_seqs,
                                     uint32_t q_len, uint32_t num_q_heads, uint32_t num_kv_heads,
                                     uint32_t head_dim, uint32_t block_size, float scale,
                                     uint32_t q_stride, uint32_t q_token_stride,
                                     uint64_t block_stride_bytes, uint64_t data_section_bytes,
                                     uint32_t causal, uint32_t sliding_window, float* workspace,
                                     uint32_t num_splits, hipStream_t stream);

/* A split count for the query-block calls: as paged_decode_num_splits, with
 * rows of up to 16 query columns (group x tokens) for blocks of at most 32
 * columns and of up to 128 columns for wider ones (BF16 blocks that wide are
 * streamed by four waves sharing each K/V tile), and, for a causal window W,
 * a window of W + q_len - 1 keys (the keys one row of the block can touch).
 * Returns 1 for q_len outside 1 .. 4096. */
PKD_API uint32_t paged_prefill_num_splits(uint32_t num_seqs, uint32_t q_len,
                                          uint32_t num_q_heads, uint32_t num_kv_heads,
                                          uint32_t max_blocks_per_seq, uint32_t block_size,
                                          uint32_t causal, uint32_t sliding_window,
                                          uint32_t num_cus);

/* ---------------------------------------------------------------- contiguous K/V
 * The multi-token attention above over contiguous K/V tensors instead of a
 * paged cache (AstrAI csrc/tests commit log: the ContigKV / PagedKV source
 * policy, stride-based Q/KV/O addressing, the bhld / blhd layouts): key j of
 * sequence b, kv head h is the row at element
 *   b*strides[3] + j*strides[4] + h*strides[5]   of k  (BF16, or E4M3FN codes)
 *   b*strides[6] + j*strides[7] + h*strides[8]   of v
 * q token i, head h at b*strides[0] + i*strides[1] + h*strides[2]; the output
 * row at b*strides[9] + i*strides[10] + h*strides[11] (BF16). strides: a host
 * array of 12 element strides, each a multiple of 16 bytes. So (b, l, h, d)
 * and (b, h, l, d) tensors, padded rows and views are all read in place.
 * Keys j < seq_lens[b] <= max_seq_len are read; causal, sliding_window,
 * num_splits and workspace as for paged_prefill_attn_bf16 (workspace of
 * paged_decode_workspace_bytes(num_seqs, num_q_heads * q_len, head_dim,
 * num_splits) bytes). q_len = 1 is plain decode.
 * The paged kernels run with the block-table lookup replaced by the strides:
 * the same tiles, order and arithmetic, so a paged cache holding the same
 * rows gives bit-identical outputs.
 * Errors: PKD_ERR_INVALID_ARG for a null or misaligned buffer, a stride not
 * a multiple of 16 bytes, max_seq_len == 0 or q_len == 0;
 * PKD_ERR_UNSUPPORTED for head_dim / num_splits outside the supported set,
 * q_len > 4096 or a K/V token stride so large that 16 rows pass 2^31 bytes. */
PKD_API int contig_kv_attn_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                uint16_t* output, const int32_t* seq_lens, uint32_t num_seqs,
                                uint32_t q_len, uint32_t max_seq_len, uint32_t num_q_heads,
                                uint32_t num_kv_heads, uint32_t head_dim, float scale,
                                const uint64_t* strides, uint32_t causal,
                                uint32_t sliding_window, float* workspace, uint32_t num_splits,
                                hipStream_t stream);

/* FP8-E4M3FN K/V codes with per-tensor k_scale, v_scale (values are
 * code * scale, as in the paged FP8 cache). */
PKD_API int contig_kv_attn_fp8(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                               uint16_t* output, const int32_t* seq_lens, uint32_t num_seqs,
                               uint32_t q_len, uint32_t max_seq_len, uint32_t num_q_heads,
                               uint32_t num_kv_heads, uint32_t head_dim, float scale,
                               float k_scale, float v_scale, const uint64_t* strides,
                               uint32_t causal, uint32_t sliding_window, float* workspace,
                               uint32_t num_splits, hipStream_t stream);

/* ---------------------------------------------------------------- host helpers
 * Bytes of the split-K workspace: num_seqs*num_q_heads*num_splits*(head_dim+2)*4. */
PKD_API size_t paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_q_heads,
                                            uint32_t head_dim, uint32_t num_splits);

/* A split count for the split-K calls: 1 + 4 * (4 * num_cus) / rows, rows =
 * num_seqs * num_kv_heads * ceil(group / 16), capped at the row's tile bound
 * (16-key tiles within max_blocks_per_seq pages, or the window) and at
 * PKD_MAX_SPLITS. The split-K pass launches about four waves per CU and spreads
 * the batch's tiles evenly over them, so this count only needs to exceed the
 * pieces a row is cut into. Pure host arithmetic; num_cus = compute-unit
 * count. */
PKD_API uint32_t paged_decode_num_splits(uint32_t num_seqs, uint32_t num_q_heads,
                                         uint32_t num_kv_heads, uint32_t max_blocks_per_seq,
                                         uint32_t block_size, uint32_t sliding_window,
                                         uint32_t num_cus);

/* Static description of a status code. */
PKD_API const char* pkd_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PKD_H */
