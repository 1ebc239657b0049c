// Host-side argument checks and launch arithmetic shared by the entry points.
// Plain C++ (no HIP), so the checks can be built and exercised without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pkd {

constexpr int kOk = 0;
constexpr int kInvalid = -1;
constexpr int kUnsupported = -2;
constexpr int kLaunch = -3;
constexpr int kScratch = -4;       // the call needs more workspace than the static scratch
constexpr uint32_t kMaxSplits = 4096;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool supported_head_dim(uint32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

inline bool supported_block_size(uint32_t bs) {
  return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256;
}

// Shape checks common to the three cache writes.
inline int check_cache_write(const void* key, const void* value, const void* kc, const void* vc,
                             const void* slots, uint32_t num_kv_heads, uint32_t head_dim,
                             uint32_t block_size, uint32_t key_stride, uint32_t value_stride) {
  if (num_kv_heads == 0) return kInvalid;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return kUnsupported;
  const uint64_t row = uint64_t(num_kv_heads) * head_dim;
  if (key_stride < row || value_stride < row) return kInvalid;
  if ((key_stride % 8) || (value_stride % 8)) return kInvalid;
  if (!key || !value || !kc || !vc || !slots) return kInvalid;
  if (!aligned16(key) || !aligned16(value) || !aligned16(kc) || !aligned16(vc)) return kInvalid;
  return kOk;
}

inline int check_fp8_stride(uint32_t num_kv_heads, uint32_t head_dim, uint32_t block_size,
                            uint64_t cache_stride) {
  const uint64_t page = uint64_t(block_size) * num_kv_heads * head_dim;
  if (cache_stride < page || (cache_stride % 16)) return kInvalid;
  return kOk;
}

inline int check_nvfp4_sections(uint32_t num_kv_heads, uint32_t head_dim, uint32_t block_size,
                                uint64_t block_stride_bytes, uint64_t data_section_bytes) {
  const uint64_t elems = uint64_t(block_size) * num_kv_heads * head_dim;
  if (data_section_bytes < elems / 2 || (data_section_bytes % 16)) return kInvalid;
  if (block_stride_bytes < data_section_bytes + elems / 16 || (block_stride_bytes % 16))
    return kInvalid;
  return kOk;
}

// Checks common to the three split-K decode calls.
inline int check_decode(const void* q, const void* kc, const void* vc, const void* ws,
                        const void* bt, const void* lens, uint32_t max_blocks_per_seq,
                        uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                        uint32_t block_size, uint32_t num_splits, uint32_t q_stride) {
  if (num_kv_heads == 0 || num_q_heads == 0 || num_q_heads % num_kv_heads) return kInvalid;
  if (max_blocks_per_seq == 0) return kInvalid;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return kUnsupported;
  if (num_splits == 0 || num_splits > kMaxSplits) return kUnsupported;
  if (q_stride < uint64_t(num_q_heads) * head_dim || (q_stride % 8)) return kInvalid;
  if (!q || !kc || !vc || !ws || !bt || !lens) return kInvalid;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(ws)) return kInvalid;
  return kOk;
}

// Checks of the whole-decode calls: the split-K checks (the workspace only
// when num_splits > 1), then the output.
inline int check_single(const void* q, const void* kc, const void* vc, const void* out,
                        const void* ws, const void* bt, const void* lens,
                        uint32_t max_blocks_per_seq, uint32_t num_q_heads, uint32_t num_kv_heads,
                        uint32_t head_dim, uint32_t block_size, uint32_t num_splits,
                        uint32_t q_stride) {
  static const uint64_t kAligned = 16;   // stands in for a workspace the call does not use
  const void* ws_or = num_splits > 1 ? ws : reinterpret_cast<const void*>(kAligned);
  const int st = check_decode(q, kc, vc, ws_or, bt, lens, max_blocks_per_seq, num_q_heads,
                              num_kv_heads, head_dim, block_size, num_splits, q_stride);
  if (st) return st;
  if (!out || !aligned16(out)) return kInvalid;
  return kOk;
}

// The new-token rows of the append calls.
inline int check_append(const void* key, const void* value, uint32_t num_kv_heads,
                        uint32_t head_dim, uint32_t key_stride, uint32_t value_stride) {
  const uint64_t row = uint64_t(num_kv_heads) * head_dim;
  if (!key || !value || !aligned16(key) || !aligned16(value)) return kInvalid;
  if (key_stride < row || value_stride < row || (key_stride % 8) || (value_stride % 8))
    return kInvalid;
  return kOk;
}

// The query block of the multi-token calls: q_len >= 1 tokens per sequence,
// token rows q_token_stride elements apart inside a sequence's q_stride.
constexpr uint32_t kMaxQueryLen = 4096;
inline int check_prefill(uint32_t q_len, uint32_t num_q_heads, uint32_t head_dim,
                         uint32_t q_stride, uint32_t q_token_stride) {
  if (q_len == 0) return kInvalid;
  if (q_len > kMaxQueryLen || uint64_t(num_q_heads) * q_len > 0x7FFFFFFFull) return kUnsupported;
  const uint64_t row = uint64_t(num_q_heads) * head_dim;
  if (q_token_stride % 8) return kInvalid;
  if (q_len > 1 && q_token_stride < row) return kInvalid;
  if (uint64_t(q_stride) < uint64_t(q_len - 1) * q_token_stride + row) return kInvalid;
  return kOk;
}

// Keys one row of a query block may touch: with a causal window W the first
// token's W keys plus the q_len - 1 after it; 0 (no bound) if that overflows.
inline uint32_t prefill_row_window(uint32_t q_len, uint32_t causal, uint32_t sliding_window) {
  if (!causal || sliding_window == 0) return sliding_window;
  const uint64_t w = uint64_t(sliding_window) + q_len - 1;
  return w > 0xFFFFFFFFull ? 0u : uint32_t(w);
}

// The contiguous-K/V calls. strides: 12 element strides, q (seq, token,
// head), k, v, output; every one a multiple of 16 bytes, so that rows stay
// 16-byte aligned; a K/V token stride small enough that 16 rows stay within
// 32-bit buffer offsets.
inline int check_contig(const void* q, const void* k, const void* v, const void* out,
                        const void* ws, const void* lens, const uint64_t* strides,
                        uint32_t num_seqs, uint32_t q_len, uint32_t max_seq_len,
                        uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
                        uint32_t kv_elem_bytes, uint32_t num_splits) {
  if (num_kv_heads == 0 || num_q_heads == 0 || num_q_heads % num_kv_heads) return kInvalid;
  if (!supported_head_dim(head_dim)) return kUnsupported;
  if (num_splits == 0 || num_splits > kMaxSplits) return kUnsupported;
  if (q_len == 0) return kInvalid;
  if (q_len > kMaxQueryLen || uint64_t(num_q_heads) * q_len > 0x7FFFFFFFull) return kUnsupported;
  if (max_seq_len == 0 || max_seq_len > 0x7FFFFFF0u) return kInvalid;
  if (!strides || !q || !k || !v || !out || !lens || (num_splits > 1 && !ws)) return kInvalid;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return kInvalid;
  if (num_splits > 1 && !aligned16(ws)) return kInvalid;
  for (int i = 0; i < 12; ++i) {
    const uint64_t bytes = (i >= 3 && i < 9) ? kv_elem_bytes : 2;
    if ((strides[i] * bytes) % 16) return kInvalid;
  }
  // q / output strides fit the kernel's 32-bit q fields; K/V tiles of 16 rows
  // stay within 32-bit buffer offsets
  if (strides[0] > 0xFFFFFFFFull || strides[1] > 0xFFFFFFFFull || strides[2] > 0xFFFFFFFFull)
    return kUnsupported;
  const uint64_t row = uint64_t(head_dim) * kv_elem_bytes;
  for (int i : {4, 7})
    if (strides[i] * kv_elem_bytes * 15 + row > 0x7FFFFFF0ull) return kUnsupported;
  (void)num_seqs;
  return kOk;
}

inline int check_reduce(const void* ws, const void* out, const void* lens, uint32_t num_q_heads,
                        uint32_t head_dim, uint32_t num_splits) {
  if (num_q_heads == 0) return kInvalid;
  if (!supported_head_dim(head_dim)) return kUnsupported;
  if (num_splits == 0 || num_splits > kMaxSplits) return kUnsupported;
  if (!ws || !out || !lens) return kInvalid;
  if (!aligned16(ws) || !aligned16(out)) return kInvalid;
  return kOk;
}

// Most pages one sequence's attended key range can touch.
inline uint32_t split_page_bound(uint32_t max_blocks_per_seq, uint32_t block_size,
                                 uint32_t sliding_window) {
  uint32_t bound = max_blocks_per_seq;
  if (sliding_window > 0) {
    const uint64_t w = (uint64_t(sliding_window) + block_size - 2) / block_size + 1;
    if (w < bound) bound = uint32_t(w);
  }
  return bound ? bound : 1;
}

inline uint32_t head_chunks(uint32_t group) { return (group + 15) / 16; }

inline size_t workspace_bytes(uint32_t num_seqs, uint32_t num_q_heads, uint32_t head_dim,
                              uint32_t num_splits) {
  return size_t(num_seqs) * num_q_heads * num_splits * (size_t(head_dim) + 2) * sizeof(float);
}

// Split-count heuristic. The split-K pass launches about 4 waves per CU and
// balances the batch's tiles evenly over them; num_splits only bounds how many
// pieces one (sequence, kv head) row may be cut into. It is chosen so that this
// bound does not force pieces longer than an even share, with room for batches
// whose sequences are shorter than the block-table width (4x).
// rows: (sequence, kv head, column group) rows the split pass will stream.
inline uint32_t num_splits_for_rows(uint64_t rows, uint32_t max_blocks_per_seq,
                                    uint32_t block_size, uint32_t sliding_window,
                                    uint32_t num_cus) {
  if (rows == 0 || block_size == 0) return 1;
  const uint64_t waves = uint64_t(num_cus ? num_cus : 256) * 4;
  const uint32_t bound = split_page_bound(max_blocks_per_seq, block_size, sliding_window);
  const uint64_t tiles = uint64_t(bound) * (block_size / 16);
  uint64_t s = 1 + (4 * waves + rows - 1) / rows;
  if (s > tiles) s = tiles;                    // a piece holds at least one tile
  if (s < 2) s = tiles >= 2 ? 2 : 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return uint32_t(s);
}

inline uint32_t num_splits_heuristic(uint32_t num_seqs, uint32_t num_q_heads,
                                     uint32_t num_kv_heads, uint32_t max_blocks_per_seq,
                                     uint32_t block_size, uint32_t sliding_window,
                                     uint32_t num_cus) {
  if (num_seqs == 0 || num_kv_heads == 0 || num_q_heads < num_kv_heads || block_size == 0)
    return 1;
  const uint64_t rows =
      uint64_t(num_seqs) * num_kv_heads * head_chunks(num_q_heads / num_kv_heads);
  return num_splits_for_rows(rows, max_blocks_per_seq, block_size, sliding_window, num_cus);
}

// Query blocks: rows hold up to 128 query columns (group x tokens) when a
// block is wider than 32 (a workgroup of waves shares each tile), else 16.
// Fewer, wider rows need more pieces per row to fill the chip.
inline uint32_t prefill_num_splits(uint32_t num_seqs, uint32_t q_len, uint32_t num_q_heads,
                                   uint32_t num_kv_heads, uint32_t max_blocks_per_seq,
                                   uint32_t block_size, uint32_t row_window, uint32_t num_cus) {
  if (num_seqs == 0 || num_kv_heads == 0 || num_q_heads < num_kv_heads || q_len == 0)
    return 1;
  const uint64_t cols = uint64_t(num_q_heads / num_kv_heads) * q_len;
  const uint64_t per_row = cols > 32 ? 128 : 16;
  const uint64_t rows = uint64_t(num_seqs) * num_kv_heads * ((cols + per_row - 1) / per_row);
  return num_splits_for_rows(rows, max_blocks_per_seq, block_size, row_window, num_cus);
}

}  // namespace pkd
