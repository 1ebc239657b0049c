// Paged decode attention: split-KV pass and combine, for BF16, FP8-E4M3FN and
// NVFP4 caches, written for gfx950 (wave64, MFMA, 160 KB LDS per CU).
//
// Method (metrale API page "metrale_model_layers/layers/ops/prefill_attn_b.rs",
// the paged_decode_attn_splitk_{nvfp4,fp8,bf16} and paged_decode_attn_reduce_*
// launchers; AstrAI csrc/tests commit log, the split-KV decode, combine and
// numerics bullets): every split of a sequence writes its partial output and
// softmax state (m, l) to a float32 workspace [head_dim values, m, l]; one
// combine merges them into BF16 with a 1e-20 guard on the denominator.
//
// Work unit: a piece of a (sequence, kv head, chunk of up to 16 query
// columns) row, streamed by one wavefront (by two that split a head_dim of
// 512, or by four that take its tiles in turn and merge in LDS for one
// sequence and for the one-launch decode). A kv head's columns are its
// group's q heads, times
// the q_len tokens of a query block (pegainfer issue #1008, the paged prefill
// launch; AstrAI log, the unified causal offset): all of them are served by
// the one pass over its pages, so each K/V byte leaves HBM once per step
// while group * q_len <= 16. A causal column masks the keys after its token.
//
// Per 16-token tile (a page holds block_size/16 tiles):
//  * K and V tiles stream from HBM into an LDS ring with direct-to-LDS buffer
//    loads, one block-table lookup per tile.
//  * S = K . Q^T on v_mfma_f32_16x16x32_bf16 (M = keys, N = query columns,
//    K = head_dim; columns beyond the group's are zero). FP8 K codes are
//    dequantized to BF16 and NVFP4 codes to FP16 (whose MFMAs that format
//    uses) in registers on their way from LDS to the MFMA (exact: every E4M3
//    value is a BF16 value, every E2M1 x E4M3 product an FP16 value).
//  * Online softmax in fp32 on the MFMA output layout (lane l: head l%16,
//    tokens 4g..4g+3), exp2 with log2(e) folded into the logit scale.
//  * O^T[dim][head] += V^T . P on v_mfma_f32_16x16x16_bf16, V^T read from
//    LDS with transposed reads, P rounded to BF16 in registers (FP16 for
//    NVFP4). A quantized V tile is first dequantized into a 16-bit copy in
//    LDS.
#include <atomic>
#include <mutex>

#include "../../include/pkd.h"
#include "device_common.hpp"
#include "validate.hpp"

namespace pkd {

enum Fmt { kBf16 = 0, kFp8 = 1, kNvfp4 = 2 };

// Largest growth of a head's max (log2 units) absorbed without rescaling.
constexpr float kLazyMax = 8.0f;
// Starting reference max (log2 units): below any finite scaled logit that
// matters, yet finite.
constexpr float kMaxFloor = -3.0e38f;


struct DecodeArgs {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  float* ws;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  uint32_t max_blocks;
  uint32_t num_q_heads;
  uint32_t num_kv_heads;
  uint32_t group;          // q heads per kv head
  uint32_t col_chunks;     // ceil(group * q_len / 16): 16-column chunks of a kv head's queries
  uint32_t head_chunks;    // rows per kv head: col_chunks / (chunks per wave), rounded up
  uint32_t block_size;
  float logit_scale;       // scale * log2(e) (* k_scale for FP8)
  float out_scale;         // v_scale for FP8, 1 otherwise
  uint32_t num_splits;
  uint32_t q_stride;
  uint64_t page_bytes;     // bytes per page of one pool
  uint64_t data_section;   // NVFP4: byte offset of the scales within a page
  uint32_t window;         // keys of a row: the last `window` (0: all)
  uint32_t num_seqs;
  uint32_t chunk_min;      // least tiles per wave (at most S pieces per row)
  uint32_t row_lead;       // most start-up tiles counted ahead of each row (split-K only)
  uint32_t max_len;        // keys a sequence can hold (block-table width x block, or the
                           // contiguous tensors' length): longer seq_lens are clamped
  uint32_t static_q;       // one sequence: Q units per row, unit u streams row u % R, tiles
                           // u / R + Q k (0: the stream partition)
  uint32_t head_group;     // split-K over a batch: kv heads that share each partition unit's
                           // tiles, one workgroup each, placed on one XCD (1: none)
  uint16_t* out;           // non-split decode (num_splits 1): BF16 output, else null
  // append: each sequence's new token, written to position L - 1 by the
  // piece that ends the row, before that piece loads its last tile
  const uint16_t* new_k;   // null: no append
  const uint16_t* new_v;
  uint32_t new_k_stride;   // elements between the rows of consecutive sequences
  uint32_t new_v_stride;
  float enc_k_scale;       // FP8 cache encode scales
  float enc_v_scale;
  // query blocks: q_len tokens per sequence, column c of a kv head's row is
  // token c / group, q head c % group of the group
  uint32_t q_len;          // 1 for decode
  uint32_t q_tok_stride;   // elements between the rows of consecutive tokens
  uint32_t causal;         // token i sits at L - q_len + i and sees keys up to it
  uint32_t q_window;       // keys a token sees with causal: the last q_window up to it
  uint32_t q_head_stride;  // elements between the q rows of consecutive heads (D by default)
  uint64_t o_seq, o_tok, o_head;   // output element strides (sequence, token, head)
  // contiguous K/V (no block table): byte strides of sequence, token, kv head
  uint64_t k_strides[3];
  uint64_t v_strides[3];
};

// Two FP8-E4M3FN codes (bytes 0/1 or 2/3 of w) -> packed BF16 pair, in one
// gfx950 convert at unit scale (exact: every E4M3FN value is a BF16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Eight FP8 codes (little-endian in w) -> eight BF16 values.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0),
               fp8x2_to_bf16x2<false>(w1), fp8x2_to_bf16x2<true>(w1)};
}

// NVFP4 runs its MFMAs in FP16: every E2M1 x E4M3 product is an FP16 value
// (at most 6 significant bits, magnitude 2^-10 .. 2688), so the group scale
// is applied with one packed FP16 multiply per pair, and P keeps 11 bits.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t w, f16x2 S) {
  const f16x2 x = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, x * S);
}

// Eight E2M1 codes (one 32-bit word) of one scale group -> eight FP16 values.
__device__ __forceinline__ u32x4 fp4x8_to_f16x8(uint32_t w, _Float16 s) {
  const f16x2 S = {s, s};
  return u32x4{fp4x2_to_f16x2<0>(w, S), fp4x2_to_f16x2<1>(w, S), fp4x2_to_f16x2<2>(w, S),
               fp4x2_to_f16x2<3>(w, S)};
}

// The two MFMAs on raw 16-bit operands: FP16 for NVFP4, BF16 otherwise.
template <int FMT>
__device__ __forceinline__ f32x4 mfma_qk(u32x4 k, u32x4 q, f32x4 acc) {
  if constexpr (FMT == kNvfp4)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), acc, 0, 0, 0);
}
template <int FMT>
__device__ __forceinline__ f32x4 mfma_pv(u32x2 v, u32x2 p, f32x4 acc) {
  if constexpr (FMT == kNvfp4)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, v),
                                                 __builtin_bit_cast(f16x4, p), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v),
                                                     __builtin_bit_cast(s16x4, p), acc, 0, 0, 0);
}

// A softmax weight in the MFMA's 16-bit type (round to nearest even) and the
// value it holds.
template <int FMT>
__device__ __forceinline__ uint32_t p_bits(float p) {
  if constexpr (FMT == kNvfp4) return __builtin_bit_cast(uint16_t, _Float16(p));
  else return f32_to_bf16_bits(p);
}
template <int FMT>
__device__ __forceinline__ float p_value(uint32_t bits) {
  if constexpr (FMT == kNvfp4) return float(__builtin_bit_cast(_Float16, uint16_t(bits)));
  else return __uint_as_float(bits << 16);
}

// Orders this wave's LDS accesses for the compiler; a wave's LDS operations
// execute in issue order, so no wait is needed.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// K and V tiles stream into an LDS ring with direct-to-LDS buffer loads
// (gfx950 LDS DMA, 16 bytes per lane). Each load instruction moves whole rows
// of the tile: lane l of instruction i fetches row i*RPI + l/CPR and the
// 16-byte chunk (l % CPR) ^ swz(row) of it, so the tile lands in LDS
// row-major with the chunks of each row XOR-permuted. swz(row) counts the
// rows that start at the same bank (the 64 banks span 256 bytes), so the K
// reads that feed the MFMA (16 rows, one chunk each) and the transposed V
// reads hit 16 different bank groups whatever the row length. NVFP4 tiles carry their group-scale rows behind the
// codes, fetched by one more load instruction. No VGPRs hold data in flight,
// so the ring depth is set by LDS alone; the waits on the DMA are explicit
// (the compiler does not track LDS-DMA writes).
template <int FMT, int D, int DS = 1>
struct LdsTraits {
  static constexpr int RB = FMT == kBf16 ? 2 * D : (FMT == kFp8 ? D : D / 2);  // row bytes
  static constexpr int CPR = RB / 16;            // 16-byte chunks per row (2 .. 64)
  static constexpr int RPI = 64 / CPR;           // rows per load instruction
  static constexpr int NI = RPI >= 16 ? 1 : 16 / RPI;   // load instructions per tile
  static constexpr int TILE = NI * 1024;         // LDS bytes of the codes of a tile
  // NVFP4 group scales: 16 rows of D/16 bytes in one load, of 4-byte pieces
  // for rows up to 16 bytes (the wave's 64 lanes then write no more LDS than
  // the 256 bytes of scales: 2.4% off the NVFP4 batch's split pass against
  // 16-byte pieces, 48 of whose lanes wrote zeros), else 16-byte pieces
  static constexpr int SC_ROW = D / 16;
  static constexpr int SC_SIZE = SC_ROW > 16 ? 16 : 4;
  static constexpr int SC_LPR = SC_ROW / SC_SIZE;       // lanes per scale row
  static_assert(FMT != kNvfp4 || 16 * SC_LPR <= 64, "one load covers the 16 scale rows");
  static constexpr int SC_TILE = FMT == kNvfp4 ? 64 * SC_SIZE : 0;
  static constexpr int KV = TILE + SC_TILE;      // LDS bytes of one K or V tile
  static constexpr int NDMA = NI + (FMT == kNvfp4 ? 1 : 0);   // load instructions per tile
  static constexpr int SLOT = 2 * KV;            // K tile + V tile
#ifndef PKD_LDS_NBUF128
#define PKD_LDS_NBUF128 1
#endif
#ifndef PKD_EARLY_K
#define PKD_EARLY_K 1
#endif
#ifndef PKD_LDS_NBUF_Q
#define PKD_LDS_NBUF_Q 1
#endif
  // ring depth in tiles: measured best at one 4 KB tile pair per wave with
  // four waves per CU; small tiles get more slots
  // (a wave holding half of a split head dim keeps one slot, so that four
  // two-wave workgroups fit a CU's LDS)
#ifndef PKD_LDS_NBUF_SPLIT
#define PKD_LDS_NBUF_SPLIT 1
#endif
  static constexpr int NBUF =
      DS > 1 ? PKD_LDS_NBUF_SPLIT
             : FMT == kBf16 ? (D <= 64 ? 4 : (D == 128 ? PKD_LDS_NBUF128 : (D == 256 ? 2 : 1)))
                            : (TILE <= 1024 ? 4 : (TILE <= 2048 ? 2 : PKD_LDS_NBUF_Q));
  static constexpr int WAIT = (2 * NBUF - 1) * NDMA;    // loads allowed in flight at a read
  static constexpr int BRB = 2 * D;              // bytes of a BF16 row (V read transposed)
  static constexpr int BCPR = D / 8;             // 16-byte chunks of a BF16 row
  // rows sharing a bank base: RB >= 256 bytes puts every row at the same one
  static constexpr int SWZ_DIV = RB >= 256 ? 1 : 256 / RB;
  static constexpr int BSWZ_DIV = BRB >= 256 ? 1 : 256 / BRB;
  // chunk permutation of row r of a raw tile / of a BF16 V tile
  __device__ static constexpr int swz(int r) { return (r / SWZ_DIV) % CPR; }
  __device__ static constexpr int bswz(int r) { return (r / BSWZ_DIV) % BCPR; }
  static constexpr int STAGE = FMT == kBf16 ? 16 : 16 * BRB;   // BF16 copy of a quantized V tile
  static_assert(WAIT < 64, "vmcnt range");
};

// s_waitcnt that waits for vmcnt <= N only (expcnt / lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Accesses to the LDS the tile DMA writes (the ring, and the stage of a
// quantized V tile beside it), as inline asm. With several waves' rings in
// one workgroup the compiler cannot tell which LDS bytes a DMA load in flight
// writes, and would wait for every one of them (the V tile's included) before
// each such access; the waits on the DMA are explicit instead. Reads wait for
// their own results in the same statement, so no consumer is scheduled before
// the data is there; writes need no wait (a wave's LDS operations execute in
// issue order).
template <int N>
__device__ __forceinline__ void lds_read_b128(u32x4 (&v)[N], const uint32_t (&ad)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "read count");
  if constexpr (N == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(ad[0]) : "memory");
  } else if constexpr (N == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(ad[0]), "v"(ad[1]) : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\tds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7])
        : "memory");
  }
}

template <int N>
__device__ __forceinline__ void lds_read_b64(u32x2 (&v)[N], const uint32_t (&ad)[N]) {
  static_assert(N == 2 || N == 4 || N == 8, "read count");
  if constexpr (N == 2) {
    asm volatile("ds_read_b64 %0, %2\n\tds_read_b64 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(ad[0]), "v"(ad[1]) : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\t"
        "ds_read_b64 %3, %7\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64 %0, %8\n\tds_read_b64 %1, %9\n\tds_read_b64 %2, %10\n\t"
        "ds_read_b64 %3, %11\n\tds_read_b64 %4, %12\n\tds_read_b64 %5, %13\n\t"
        "ds_read_b64 %6, %14\n\tds_read_b64 %7, %15\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7])
        : "memory");
  }
}

// NVFP4 K: N chunks of 32 codes (16 bytes) and their two scale bytes (a
// 16-bit read each).
template <int N>
__device__ __forceinline__ void lds_read_fp4_chunks(u32x4 (&v)[N], uint32_t (&sc)[N],
                                                    const uint32_t (&ad)[N],
                                                    const uint32_t (&sad)[N]) {
  static_assert(N == 1 || N == 2, "read count");
  if constexpr (N == 1) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_u16 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(sc[0]) : "v"(ad[0]), "v"(sad[0]) : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_u16 %2, %6\n\t"
        "ds_read_u16 %3, %7\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(sc[0]), "=&v"(sc[1])
        : "v"(ad[0]), "v"(ad[1]), "v"(sad[0]), "v"(sad[1])
        : "memory");
  }
}

// NVFP4 V staging: N words of 8 codes and the scale byte of each.
template <int N>
__device__ __forceinline__ void lds_read_fp4_words(uint32_t (&w)[N], uint32_t (&sc)[N],
                                                   const uint32_t (&ad)[N],
                                                   const uint32_t (&sad)[N]) {
  static_assert(N == 2 || N == 4 || N == 8, "read count");
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_u8 %2, %6\n\t"
        "ds_read_u8 %3, %7\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(sc[0]), "=&v"(sc[1])
        : "v"(ad[0]), "v"(ad[1]), "v"(sad[0]), "v"(sad[1])
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b32 %0, %8\n\tds_read_b32 %1, %9\n\tds_read_b32 %2, %10\n\t"
        "ds_read_b32 %3, %11\n\tds_read_u8 %4, %12\n\tds_read_u8 %5, %13\n\t"
        "ds_read_u8 %6, %14\n\tds_read_u8 %7, %15\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(sc[0]), "=&v"(sc[1]),
          "=&v"(sc[2]), "=&v"(sc[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(sad[0]), "v"(sad[1]),
          "v"(sad[2]), "v"(sad[3])
        : "memory");
  } else {
    lds_read_fp4_words<4>(*reinterpret_cast<uint32_t(*)[4]>(&w[0]),
                          *reinterpret_cast<uint32_t(*)[4]>(&sc[0]),
                          *reinterpret_cast<const uint32_t(*)[4]>(&ad[0]),
                          *reinterpret_cast<const uint32_t(*)[4]>(&sad[0]));
    lds_read_fp4_words<4>(*reinterpret_cast<uint32_t(*)[4]>(&w[4]),
                          *reinterpret_cast<uint32_t(*)[4]>(&sc[4]),
                          *reinterpret_cast<const uint32_t(*)[4]>(&ad[4]),
                          *reinterpret_cast<const uint32_t(*)[4]>(&sad[4]));
  }
}

__device__ __forceinline__ void lds_write_b128(uint32_t ad, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(ad), "v"(v) : "memory");
}

// Balanced ("stream") partition of one launch's work. A row is a (sequence,
// kv head, chunk of up to 16 q heads) triple; row (b, k) has n_b tiles, the
// 16-key tiles overlapping the sequence's attended keys. The rows are laid end
// to end, sequence-major, into one index space, each row with keys behind
// `lead` empty start-up positions (see for_each_piece); wave w of the P
// launched waves takes positions [w*c, (w+1)*c) with c = max(ceil(T/P), c_min)
// (or one more when that buys the whole lead) and c_min = ceil(n_bound / (S -
// 1)) for the host's bound n_bound on n_b. A wave thus covers one or more row
// pieces, each a contiguous key range; the piece of row r starting at flat
// position f goes to workspace slot floor(f/c) - floor(first(r)/c) <= S - 1,
// first(r) being the position of the row's first tile. The wave that ends a
// row marks the row's later slots empty. With S == 1, wave w takes row w
// whole. Every wave gets the same number of positions whatever the length mix
// of the batch. ("Wave" here is the partition unit: one workgroup, whose
// waves may split the head dim or interleave a piece's tiles.) Adjacent kv
// heads whose rows share cache lines may be partitioned as one row group,
// each member streaming the same tiles of its own row (head_group). One
// sequence without a window skips this partition for a fixed one that does
// not depend on the length (static_q).

__device__ __forceinline__ uint32_t row_tiles(uint32_t L, uint32_t window) {
  if (L == 0) return 0;
  const uint32_t lo = (window > 0 && L > window) ? L - window : 0u;
  return (L + 15) / 16 - lo / 16;
}

// Keys of a sequence: its length, never past what its block-table row (or
// contiguous tensor) holds, so a length beyond the table cannot send a read
// past the row.
__device__ __forceinline__ uint32_t seq_len(const DecodeArgs& a, int32_t Ls) {
  return Ls > 0 ? min(uint32_t(Ls), a.max_len) : 0u;
}

// Inclusive prefix sum over the 64 lanes, in DPP moves: shifts by 1, 2, 4
// and 8 within each row of 16 lanes (lanes shifted in from outside the row
// add 0), then lane 15 of rows 0 and 2 is added to rows 1 and 3, and lane 31
// (the sum of rows 0 and 1) to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xF, 0xF, false));   // row_shr:1
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xF, 0xF, false));   // row_shr:2
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xF, 0xF, false));   // row_shr:4
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xF, 0xF, false));   // row_shr:8
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x142, 0xA, 0xF, false));   // row_bcast:15
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x143, 0xC, 0xF, false));   // row_bcast:31
  return x;
}

struct RowLoc {
  uint32_t b, kh, n, start;     // sequence, kv-head/chunk index, tiles, flat start of the row
};

// Total tiles T of the launch (all rows of all sequences), and the rows
// that have any.
__device__ __forceinline__ uint32_t total_tiles(const DecodeArgs& a, uint32_t rows_per_seq,
                                                uint32_t& live_rows) {
  uint32_t tot = 0;
  live_rows = 0;
  for (uint32_t b0 = 0; b0 < a.num_seqs; b0 += 64) {
    const uint32_t bb = b0 + (threadIdx.x & 63);
    const int32_t Ls = bb < a.num_seqs ? a.seq_lens[bb] : 0;
    const uint32_t n = row_tiles(seq_len(a, Ls), a.window);
    tot += uint32_t(__builtin_amdgcn_readlane(int(wave_scan(n * rows_per_seq)), 63));
    live_rows += uint32_t(__builtin_popcountll(__builtin_amdgcn_ballot_w64(n > 0))) * rows_per_seq;
  }
  return tot;
}

// The row holding flat position `pos` (pos < T + lead * live rows), each row
// taking its `lead` start-up positions and then its tiles.
__device__ __forceinline__ RowLoc find_row(const DecodeArgs& a, uint32_t pos,
                                           uint32_t rows_per_seq, uint32_t lead) {
  uint32_t base = 0;
  for (uint32_t b0 = 0; b0 < a.num_seqs; b0 += 64) {
    const uint32_t bb = b0 + (threadIdx.x & 63);
    const int32_t Ls = bb < a.num_seqs ? a.seq_lens[bb] : 0;
    const uint32_t nt = row_tiles(seq_len(a, Ls), a.window);
    const uint32_t n = nt > 0 ? nt + lead : 0u;
    const uint32_t incl = wave_scan(n * rows_per_seq);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > pos);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const uint32_t nl = uint32_t(__builtin_amdgcn_readlane(int(n), l));
      const uint32_t excl = uint32_t(__builtin_amdgcn_readlane(int(incl), l)) - nl * rows_per_seq;
      const uint32_t kh = (pos - base - excl) / nl;
      return RowLoc{b0 + l, kh, nl, base + excl + kh * nl};
    }
    base += uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
  }
  return RowLoc{a.num_seqs, 0, 0, base};
}


// LDS of one wave: the tile ring and the BF16 copy of a quantized V tile.
template <int FMT, int DW, int DS>
struct StreamLds {
  __attribute__((aligned(1024))) uint8_t ring[LdsTraits<FMT, DW, DS>::NBUF *
                                              LdsTraits<FMT, DW, DS>::SLOT];
  __attribute__((aligned(16))) uint8_t stage[LdsTraits<FMT, DW, DS>::STAGE];
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// A quantized V tile (raw codes in the ring) -> 16-bit rows in the stage
// (BF16 for FP8, FP16 for NVFP4), laid out as a BF16 tile would be (chunk c
// of row r at c ^ bswz(r)). Lane l makes
// BF16 chunks k*64 + l (8 values each), so 16 consecutive lanes write 16
// consecutive chunks of one row: no bank conflicts. Rows of keys outside
// [lo, khi) become zeros for FP8 (selected when MASK: its codes may be NaN);
// NVFP4 rows only have NaN scales cleared (their weight is zero).
template <int FMT, int D, bool MASK, typename AfterRead>
__device__ __forceinline__ void stage_v(lds_u8* vt, lds_u8* stage, int lane, uint32_t tok0,
                                        uint32_t lo, uint32_t khi, AfterRead&& after_read) {
  using T = LdsTraits<FMT, D>;
  constexpr int NQ = 16 * T::BCPR / 64;          // BF16 chunks per lane
  const uint32_t vta = uint32_t(uintptr_t(vt)), sta = uint32_t(uintptr_t(stage));
  u32x4 h[NQ];
  if constexpr (FMT == kFp8) {
    // codes 8c .. 8c+7: half of raw chunk c/2
    u32x2 w[NQ];
    uint32_t ad[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int q = k * 64 + lane;
      const int row = q / T::BCPR, c = q % T::BCPR;
      ad[k] = vta + row * T::RB + ((c >> 1) ^ T::swz(row)) * 16 + 8 * (c & 1);
    }
    lds_read_b64<NQ>(w, ad);
    after_read();
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const uint32_t tok = tok0 + (k * 64 + lane) / T::BCPR;
      h[k] = fp8x8_to_bf16x8(w[k][0], w[k][1]);
      if (MASK && !(tok >= lo && tok < khi)) h[k] = u32x4{0u, 0u, 0u, 0u};
    }
  } else {
    // codes 8c .. 8c+7: a quarter of raw chunk c/4; scale group c/2. E2M1
    // codes are always finite, so only the scale can poison a row past the
    // keys: in a partial tile (MASK) a NaN scale code (0x7F / 0xFF) becomes
    // 0, every row decodes to finite values, and the zero weight of a masked
    // key removes it (a key's own scale, as the cache write encodes it, is
    // never NaN). No per-row test, so the LDS reads of all chunks issue
    // together.
    (void)tok0;
    (void)lo;
    (void)khi;
    uint32_t w[NQ], sraw[NQ], ad[NQ], sad[NQ];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int q = k * 64 + lane;
      const int row = q / T::BCPR, c = q % T::BCPR;
      ad[k] = vta + row * T::RB + ((c >> 2) ^ T::swz(row)) * 16 + 4 * (c & 3);
      sad[k] = vta + T::TILE + row * T::SC_ROW + (c >> 1);
    }
    lds_read_fp4_words<NQ>(w, sraw, ad, sad);
    after_read();
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const uint32_t sb = (MASK && (sraw[k] & 0x7Fu) == 0x7Fu) ? 0u : sraw[k];
      h[k] = fp4x8_to_f16x8(w[k], _Float16(__builtin_amdgcn_cvt_f32_fp8(sb, 0)));
    }
  }
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int q = k * 64 + lane;
    const int row = q / T::BCPR, c = q % T::BCPR;
    lds_write_b128(sta + row * T::BRB + (c ^ T::bswz(row)) * 16, h[k]);
  }
}

// Append: this wave's half of the head dims (all of them when DS = 1) of
// sequence b's new token, kv head kvh, into position L - 1 of its K and V
// pages, encoded as reshape_and_cache_{bf16,fp8,nvfp4} encode it. Lanes 0-31
// write K and lanes 32-63 write V. The caller waits for the stores before it
// requests the tile that holds position L - 1.
template <int FMT, int D, int DS>
__device__ __forceinline__ void append_token(const DecodeArgs& a, uint32_t b, uint32_t kvh,
                                             uint32_t L, int w, int lane) {
  constexpr int DW = D / DS;
  constexpr int PER = FMT == kNvfp4 ? 16 : 8;     // values a lane encodes
  static_assert(DW / PER <= 32, "one lane half covers a row");
  const int kv = lane >> 5, j = lane & 31;
  if (j >= DW / PER) return;
  const uint32_t pos = L - 1;
  const uint32_t phys = uint32_t(a.block_tables[uint64_t(b) * a.max_blocks + pos / a.block_size]);
  const uint64_t row = uint64_t(pos % a.block_size) * a.num_kv_heads + kvh;   // (offset, head)
  const uint16_t* src = (kv ? a.new_v + uint64_t(b) * a.new_v_stride
                            : a.new_k + uint64_t(b) * a.new_k_stride) + kvh * D + w * DW + PER * j;
  uint8_t* const pool = const_cast<uint8_t*>(kv ? a.v_cache : a.k_cache) + uint64_t(phys) * a.page_bytes;
  if constexpr (FMT == kBf16) {
    *reinterpret_cast<u32x4*>(pool + (row * D + w * DW + 8 * j) * 2) =
        *reinterpret_cast<const u32x4*>(src);
  } else if constexpr (FMT == kFp8) {
    *reinterpret_cast<u32x2*>(pool + row * D + w * DW + 8 * j) =
        fp8_encode8(*reinterpret_cast<const u32x4*>(src), kv ? a.enc_v_scale : a.enc_k_scale);
  } else {
    uint32_t sc;
    const u32x2 codes = nvfp4_encode16(*reinterpret_cast<const u32x4*>(src),
                                       *reinterpret_cast<const u32x4*>(src + 8), sc);
    *reinterpret_cast<u32x2*>(pool + row * (D / 2) + (w * DW) / 2 + 8 * j) = codes;
    pool[a.data_section + row * (D / 16) + (w * DW) / 16 + j] = uint8_t(sc);
  }
}

// Query column col of kv head kvh: token qi = col / group and q head qh of
// that token; false past the group * q_len columns (then qi = 0).
__device__ __forceinline__ bool column_of(const DecodeArgs& a, uint32_t kvh, uint32_t col,
                                          uint32_t& qi, uint32_t& qh) {
  const bool ok = col < a.group * a.q_len;
  qi = ok ? col / a.group : 0u;
  qh = kvh * a.group + (col - qi * a.group);
  return ok;
}

// First of the eight head dims (within this wave's share) that lane group g
// feeds to QK MFMA c. The dot product sums over all dims, so any order works
// as long as K and q agree. A lane reads whole 16-byte K chunks: BF16 tiles
// (8 dims a chunk) take dims 32c + 8g .. +8; FP8 takes half c % 2 of chunk
// 4 (c / 2) + g (16 dims a chunk); NVFP4 from 128 dims takes word c % 4
// of chunk 4 (c / 4) + g (32 dims a chunk); narrower NVFP4 tiles keep the
// BF16 order.
template <int FMT, int DW>
__device__ __forceinline__ constexpr int qk_dim(int c, int g) {
  if constexpr (FMT == kNvfp4 && DW >= 128) return 32 * (4 * (c / 4) + g) + 8 * (c % 4);
  if constexpr (FMT == kFp8) return 16 * (4 * (c / 2) + g) + 8 * (c % 2);
  return 32 * c + 8 * g;
}

// The state a wave leaves after streaming its tiles: O^T (unnormalized,
// lane (g, n) holding dims 16 mt + 4 g .. +4 of column n), the reference max
// m_run (log2 units, at most kLazyMax below the largest logit seen) and the
// lane's part of the weight sum l_run.
template <int FMT, int D, int DS, int NC>
struct WaveState {
  f32x4 acc[NC][D / DS / 16];
  float m_run[NC], l_run[NC];
};

// One wave streams the key tiles first + k * step, k < count, of row (b, kh)
// (tile t holds keys 16t .. 16t + 15; keys outside [lo, L) are masked), with
// count the tiles below `tend`. The row's NC chunks of 16 query columns share
// every K/V tile: each K or V read from LDS feeds NC MFMAs.
// With DS = 2 the workgroup's two waves split the head dim: wave w loads and
// accumulates dims [w D/2, (w+1) D/2) of K, V, q and o, and the two halves of
// every tile's logits are added through LDS (`xg`, two buffers used in turn,
// `xturn` counting the exchanges of the launch).
// q and the first 64 block-table entries are requested before anything that
// depends on the length, so that when `first` and `step` do not depend on it
// (a single sequence, see splitk_stream) those loads share its round trip.
// can_append: the length is within the block table, so the new token (if
// any) is written to position L - 1 by the wave holding that tile, which
// waits for its stores only right before it requests the tile.
template <int FMT, int D, int DS, int NC, bool CONTIG>
__device__ __forceinline__ void stream_tiles(const DecodeArgs& a, StreamLds<FMT, D / DS, DS>& sh,
                                             lds_u8* xg, uint32_t& xturn, uint32_t b,
                                             uint32_t kh, uint32_t first, uint32_t step,
                                             uint32_t tend, uint32_t L, bool can_append,
                                             WaveState<FMT, D, DS, NC>& st) {
  static_assert(DS == 1 || NC == 1, "a split head dim carries one column chunk");
  static_assert(!CONTIG || FMT != kNvfp4, "contiguous K/V: BF16 and FP8 rows only");
  // The tile sequence is the same for every lane; saying so keeps the tile
  // loop, the block-table walk and the load descriptors in scalar registers
  // (a descriptor the compiler cannot prove uniform costs a loop per load).
  b = __builtin_amdgcn_readfirstlane(b);
  kh = __builtin_amdgcn_readfirstlane(kh);
  first = __builtin_amdgcn_readfirstlane(first);
  step = __builtin_amdgcn_readfirstlane(step);
  constexpr int DW = D / DS;                     // head dims of this wave
  using T = LdsTraits<FMT, DW, DS>;              // tile geometry of this wave's half rows
  using TF = LdsTraits<FMT, D>;                  // full rows (strides in the pools)
  constexpr int NBUF = T::NBUF;
  const int lane = threadIdx.x & 63;
  const int w = DS > 1 ? int(threadIdx.x >> 6) : 0;
  const int g = lane >> 4;
  const int n = lane & 15;
  const uint32_t kvh = kh / a.head_chunks, hc = kh % a.head_chunks;
  const uint32_t tpp = a.block_size / 16;
  const int32_t* bt = a.block_tables + uint64_t(b) * a.max_blocks;

  // block-table entries of the first 64 tiles (entry per tile; any entry of
  // the row may be read, those past the length are never used)
  int32_t bt_first = 0;
  if constexpr (!CONTIG) {
    const uint64_t t = uint64_t(first) + uint64_t(lane) * step;
    if (t < uint64_t(a.max_blocks) * tpp) bt_first = bt[t / tpp];
  }

  // q as the B operand of the QK MFMAs: column n, dims qk_dim(c, g) .. +8
  bool head_ok[NC];
  uint32_t qi_of[NC];
  u32x4 qf[NC][DW / 32];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    uint32_t qi, qh;
    head_ok[k] = column_of(a, kvh, (hc * NC + k) * 16 + n, qi, qh);
    qi_of[k] = qi;
    const uint16_t* qsrc = a.q + uint64_t(b) * a.q_stride + uint64_t(qi) * a.q_tok_stride +
                           uint64_t(qh) * a.q_head_stride + w * DW;
#pragma unroll
    for (int c = 0; c < DW / 32; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head_ok[k]) v = *reinterpret_cast<const u32x4*>(qsrc + qk_dim<FMT, DW>(c, g));
      qf[k][c] = v;
    }
  }

  L = __builtin_amdgcn_readfirstlane(L);
  tend = __builtin_amdgcn_readfirstlane(tend);
  const uint32_t count = tend > first ? (tend - first + step - 1) / step : 0u;
  const uint32_t lo = (a.window > 0 && L > a.window) ? L - a.window : 0u;

  // the keys [c_lo, c_hi) column n of chunk k attends: the row's range, or
  // with causal the keys up to its token's position (the last q_window)
  uint32_t c_lo[NC], c_hi[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    c_lo[k] = lo;
    c_hi[k] = L;
    if (a.causal && head_ok[k]) {
      const int p1 = int(L) - int(a.q_len) + int(qi_of[k]) + 1;     // position + 1
      c_hi[k] = p1 > 0 ? uint32_t(p1) : 0u;
      c_lo[k] = (a.q_window > 0 && c_hi[k] > a.q_window) ? c_hi[k] - a.q_window : 0u;
    }
  }

  // append: the wave whose tiles include the one holding position L - 1
  const uint32_t t_last = L > 0 ? (L - 1) / 16 : 0u;
  const uint32_t k_last = t_last >= first ? (t_last - first) / step : 0xFFFFFFFFu;
  bool pend = !CONTIG && a.new_k != nullptr && can_append && L > 0 && t_last >= first &&
              (t_last - first) % step == 0 && k_last < count;
  if constexpr (!CONTIG) {
    if (pend) append_token<FMT, D, DS>(a, b, kvh, L, w, lane);
  }

  float qup[NC];               // NVFP4: logits of this column's dims are scaled by qup
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    qup[k] = 1.0f;
    if constexpr (FMT == kNvfp4) {
      // q in FP16 for the FP16 MFMA: shifted down by 2^e so that the
      // column's largest |q| stays below 2^15 (exact for every BF16 value in range)
      uint32_t mlo = 0, mhi = 0;     // largest magnitudes (BF16 bits order as values)
#pragma unroll
      for (int c = 0; c < DW / 32; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          mlo = max(mlo, qf[k][c][j] & 0x7FFFu);
          mhi = max(mhi, qf[k][c][j] & 0x7FFF0000u);
        }
      float m = fmaxf(bf16_lo(mlo), bf16_hi(mhi));
      m = max_over_rows(m);
      const int e = int((__float_as_uint(m) >> 23) & 255u) - 127;
      const int sh2 = e > 14 ? e - 14 : 0;
      const float down = __uint_as_float(uint32_t(127 - sh2) << 23);
      qup[k] = __uint_as_float(uint32_t(127 + sh2) << 23);
#pragma unroll
      for (int c = 0; c < DW / 32; ++c) {
        u32x4 h;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 f = {bf16_lo(qf[k][c][j]) * down, bf16_hi(qf[k][c][j]) * down};
          h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
        }
        qf[k][c] = h;
      }
    }
  }
  // logit scale of each column: the call's (times log2 e) and, for NVFP4, the
  // power of two the column's q was shifted down by (exact either way)
  float lscale[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) lscale[k] = a.logit_scale * qup[k];

  lds_u8* const ring3 = (lds_u8*)(sh.ring);
  lds_u8* const stage3 = (lds_u8*)(sh.stage);
  const int ld_row = lane / T::CPR;                  // + i * RPI
  const int ld_pos = lane % T::CPR;

#pragma unroll
  for (int k = 0; k < NC; ++k)
#pragma unroll
    for (int mt = 0; mt < DW / 16; ++mt) st.acc[k][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The reference max starts at a finite floor rather than -inf, so that a
  // column whose keys in this piece are all masked keeps weights exp2(-inf -
  // floor) = 0 and rescale factors 1 (never exp2(-inf + inf)).
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    st.m_run[k] = kMaxFloor;
    st.l_run[k] = 0.0f;
  }

  // Segments of up to 64 tiles: the block-table entries of a segment's tiles
  // sit in one VGPR (entry per lane); the DMA ring restarts at every segment.
  for (uint32_t k0 = 0; k0 < count; k0 += 64) {
    const uint32_t kend = min(k0 + 64, count);
    int32_t bt_reg = 0;
    if constexpr (!CONTIG) {
      if (k0 == 0) {
        bt_reg = bt_first;
      } else {
        const uint64_t t = uint64_t(first) + uint64_t(k0 + lane) * step;
        bt_reg = (k0 + lane < kend) ? bt[t / tpp] : 0;
      }
    }

    // Tile k of the sequence, kind kv (0 = K, 1 = V), into ring slot s. A
    // tile past the segment's end gets a zero-length descriptor: zeros land
    // in LDS and no memory is read. Lanes without a row to fetch use an
    // offset past any page, which reads nothing either.
    auto issue = [&](int s, int kv, uint32_t k) {
      const bool live = k < kend;
      if (pend && live && k == k_last) {
        // the tile with the appended token: its stores must have landed
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        wait_vmcnt<0>();
        pend = false;
      }
      const uint8_t* pool = kv ? a.v_cache : a.k_cache;
      __amdgpu_buffer_rsrc_t rsrc;
      uint32_t off0 = 0, rstride = 0;       // paged: first row of the tile; contiguous: row bytes
      if constexpr (CONTIG) {
        // keys 16t .. 16t + 15 of sequence b, kv head kvh: the descriptor
        // spans the tile's rows below L only
        const uint64_t* stv = kv ? a.v_strides : a.k_strides;
        const uint32_t tok0 = (first + k * step) * 16;
        const uint32_t nv = live ? min(16u, L - tok0) : 0u;
        rstride = uint32_t(stv[1]);
        rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(pool + uint64_t(b) * stv[0] + uint64_t(live ? tok0 : 0u) * stv[1] +
                                 uint64_t(kvh) * stv[2]),
            0, nv ? int((nv - 1) * rstride + TF::RB) : 0, 0x00020000);
      } else {
        const uint32_t kk = min(k, kend - 1);
        const uint32_t phys = uint32_t(__builtin_amdgcn_readlane(bt_reg, int(kk - k0)));
        rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(pool + uint64_t(phys) * a.page_bytes), 0,
            live ? int(a.page_bytes) : 0, 0x00020000);
        off0 = ((first + kk * step) % tpp) * 16;
      }
      lds_u8* const dst = ring3 + s * T::SLOT + kv * T::KV;
#pragma unroll
      for (int i = 0; i < T::NI; ++i) {
        const int row = i * T::RPI + ld_row;
        const int chunk = ld_pos ^ T::swz(row);
        int voff = CONTIG ? int(row * rstride + w * T::RB + chunk * 16)
                          : int(((off0 + row) * a.num_kv_heads + kvh) * TF::RB + w * T::RB +
                                chunk * 16);
        if constexpr (T::RPI > 16) voff = row < 16 ? voff : 0x7FFFFFF0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + i * 1024), 16, voff,
                                                 0, 0, 2);
      }
      if constexpr (FMT == kNvfp4) {
        const int srow = lane / T::SC_LPR;
        const int part = lane % T::SC_LPR;
        const int voff = srow < 16 ? int(a.data_section) +
                                         int(((off0 + srow) * a.num_kv_heads + kvh) * TF::SC_ROW +
                                             w * T::SC_ROW + part * T::SC_SIZE)
                                   : 0x7FFFFFF0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + T::TILE), T::SC_SIZE,
                                                 voff, 0, 0, 2);
      }
    };

#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      issue(s, 0, k0 + s);
      issue(s, 1, k0 + s);
    }

    for (uint32_t kb = k0; kb < kend; kb += NBUF) {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        const uint32_t k = kb + s;               // k >= kend: phantom tile, all keys masked
        const uint32_t tok0 = (first + k * step) * 16;
        const uint32_t khi = k < kend ? L : 0u;
        lds_u8* const kt = ring3 + s * T::SLOT;
        lds_u8* const vt = kt + T::KV;

        // ---- S = K Q^T from the LDS tile (row n, dims 32c + 8g .. +8)
        wait_vmcnt<T::WAIT>();
        wave_lds_fence();
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sc[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint32_t kta = uint32_t(uintptr_t(kt));
        // The K slot is free once its rows are in registers (the reads wait
        // for themselves): for NVFP4 tiles, whose K decode is long, the next K
        // tile is requested before the decode and the MFMAs (measured: 3% on
        // the NVFP4 batch, within noise for BF16 and FP8).
        bool k_issued = false;
        auto issue_k_early = [&]() {
          if constexpr (PKD_EARLY_K && FMT == kNvfp4) {
            __builtin_amdgcn_sched_barrier(0);
            issue(s, 0, k + NBUF);
            __builtin_amdgcn_sched_barrier(0);
            k_issued = true;
          }
        };
        if constexpr (FMT == kBf16) {
          u32x4 kv[DW / 32];
          uint32_t ka[DW / 32];
#pragma unroll
          for (int c = 0; c < DW / 32; ++c) ka[c] = kta + n * T::RB + (((4 * c + g) ^ T::swz(n)) * 16);
          lds_read_b128<DW / 32>(kv, ka);
          issue_k_early();
#pragma unroll
          for (int c = 0; c < DW / 32; ++c)
#pragma unroll
            for (int j = 0; j < NC; ++j) sc[j] = mfma_qk<FMT>(kv[c], qf[j][c], sc[j]);
        } else if constexpr (FMT == kFp8) {
          // lane group g takes whole 16-byte chunks 4h + g (16 codes): MFMA
          // 2h + u uses its half u (q is loaded in the same dim order, qk_dim)
          u32x4 cw[DW / 64];
          uint32_t ka[DW / 64];
#pragma unroll
          for (int h = 0; h < DW / 64; ++h) ka[h] = kta + n * T::RB + (((4 * h + g) ^ T::swz(n)) * 16);
          lds_read_b128<DW / 64>(cw, ka);
          issue_k_early();
#pragma unroll
          for (int h = 0; h < DW / 64; ++h) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const u32x4 kv = fp8x8_to_bf16x8(cw[h][2 * u], cw[h][2 * u + 1]);
#pragma unroll
              for (int j = 0; j < NC; ++j) sc[j] = mfma_qk<FMT>(kv, qf[j][2 * h + u], sc[j]);
            }
          }
        } else {
          if constexpr (DW >= 128) {
            // lane group g takes whole 16-byte chunks 4h + g (32 codes, the
            // dims of two scale groups): MFMA 4h + u uses its word u, so a
            // lane makes one 16-byte and one 2-byte read per chunk (q is
            // loaded in the same dim order, qk_dim)
            u32x4 cw[DW / 128];
            uint32_t s2[DW / 128], ka[DW / 128], sa[DW / 128];
#pragma unroll
            for (int h = 0; h < DW / 128; ++h) {
              const int j = 4 * h + g;
              ka[h] = kta + n * T::RB + ((j ^ T::swz(n)) * 16);
              sa[h] = kta + T::TILE + n * T::SC_ROW + 2 * j;
            }
            lds_read_fp4_chunks<DW / 128>(cw, s2, ka, sa);
            issue_k_early();
#pragma unroll
            for (int h = 0; h < DW / 128; ++h) {
              const _Float16 S0 = _Float16(__builtin_amdgcn_cvt_f32_fp8(s2[h], 0));
              const _Float16 S1 = _Float16(__builtin_amdgcn_cvt_f32_fp8(s2[h], 1));
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const u32x4 kv = fp4x8_to_f16x8(cw[h][u], u < 2 ? S0 : S1);
#pragma unroll
                for (int q = 0; q < NC; ++q) sc[q] = mfma_qk<FMT>(kv, qf[q][4 * h + u], sc[q]);
              }
            }
          } else {
            // group of dims 32c + 8g is 2c + g/2: byte 2(c & 1) of scale word
            // c/2 once the words are shifted down by g/2 bytes
            uint32_t sw[(T::SC_ROW + 3) / 4];
#pragma unroll
            for (int i = 0; i < (T::SC_ROW + 3) / 4; ++i)
              sw[i] = *(lds_u32*)(kt + T::TILE + n * T::SC_ROW + 4 * i) >> (8 * (g >> 1));
#pragma unroll
            for (int c = 0; c < DW / 32; ++c) {
              const int chunk = c ^ T::swz(n);
              const uint32_t wd = *(lds_u32*)(kt + n * T::RB + chunk * 16 + 4 * g);
              const float S = (c & 1) ? __builtin_amdgcn_cvt_f32_fp8(sw[c / 2], 2)
                                      : __builtin_amdgcn_cvt_f32_fp8(sw[c / 2], 0);
              const u32x4 kv = fp4x8_to_f16x8(wd, _Float16(S));
#pragma unroll
              for (int q = 0; q < NC; ++q) sc[q] = mfma_qk<FMT>(kv, qf[q][c], sc[q]);
            }
          }
        }
        if constexpr (DS > 1) {
          // the other parts of the head dim: partial logits through LDS,
          // summed in wave order so that every wave gets the same sum
          typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
          lds_f32x4* const xs = (lds_f32x4*)xg + (xturn++ & 1) * (DS * 64);
          xs[w * 64 + lane] = sc[0];
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          f32x4 part[DS];
#pragma unroll
          for (int u = 0; u < DS; ++u) part[u] = u == w ? sc[0] : xs[u * 64 + lane];
          f32x4 sum = part[0];
#pragma unroll
          for (int u = 1; u < DS; ++u) sum += part[u];
          sc[0] = sum;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!k_issued) issue(s, 0, k + NBUF);

        // ---- online softmax (lane: column n, tokens tok0 + 4g + j)
        // The reference m_run follows the running max lazily: it moves only
        // when some column's max exceeds it by more than kLazyMax (log2
        // units), and only then is the accumulator rescaled. The weights stay
        // below 2^kLazyMax; (m, l, o) is exact for any reference, so only the
        // amount of rescaling work changes.
        bool rescale[NC];
        float alpha[NC];
        u32x2 pf[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const uint32_t c_khi = k < kend ? c_hi[j] : 0u;
          float sv[4];
          float mx = -__builtin_inff();
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t tok = tok0 + 4 * g + r;
            sv[r] = (tok >= c_lo[j] && tok < c_khi) ? sc[j][r] * lscale[j] : -__builtin_inff();
            mx = fmaxf(mx, sv[r]);
          }
          mx = max_over_rows(mx);
          rescale[j] = __builtin_amdgcn_ballot_w64(mx > st.m_run[j] + kLazyMax) != 0;
          alpha[j] = 1.0f;
          if (rescale[j]) {
            const float m_new = fmaxf(st.m_run[j], mx);
            alpha[j] = __builtin_amdgcn_exp2f(st.m_run[j] - m_new);
            st.m_run[j] = m_new;
          }
          uint32_t pbits[4];
          float psum = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(sv[r] - st.m_run[j]);
            pbits[r] = p_bits<FMT>(p);
            psum += p_value<FMT>(pbits[r]);
          }
          st.l_run[j] = st.l_run[j] * alpha[j] + psum;
          pf[j] = u32x2{pbits[0] | (pbits[1] << 16), pbits[2] | (pbits[3] << 16)};
        }

        // ---- V tile as BF16 rows with masked tokens zeroed: in place for a
        // BF16 cache (partial tiles only), else dequantized into the stage
        wait_vmcnt<T::WAIT>();
        wave_lds_fence();
        __builtin_amdgcn_sched_barrier(0);
        lds_u8* vsrc;
        if constexpr (FMT == kBf16) {
          vsrc = vt;
          if (tok0 < lo || tok0 + 16 > khi) {
#pragma unroll
            for (int i = 0; i < T::NI; ++i) {
              const uint32_t tok = tok0 + i * T::RPI + ld_row;
              if (tok < lo || tok >= khi)
                *(lds_u32x4*)(vt + i * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
            }
            wave_lds_fence();
          }
        } else {
          vsrc = stage3;
          // FP8 codes of masked tokens may be anything (NaN included), so
          // partial tiles select zeros; E2M1 codes are always finite, so a
          // masked NVFP4 row just takes a zero scale. The raw V slot is free
          // once its codes are in registers: the next V tile is requested
          // then, before the dequant and the stage writes.
          auto next_v = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            issue(s, 1, k + NBUF);
            __builtin_amdgcn_sched_barrier(0);
          };
          if (tok0 < lo || tok0 + 16 > khi)
            stage_v<FMT, DW, true>(vt, stage3, lane, tok0, lo, khi, next_v);
          else
            stage_v<FMT, DW, false>(vt, stage3, lane, tok0, lo, khi, next_v);
          wave_lds_fence();
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- O^T += V^T P: lane supplies V[4g + n/4][16mt + 4(n%4) .. +4]. The
        // transposed reads are issued as inline asm: the compiler would otherwise
        // wait for every pending LDS-DMA load before each of them. Four reads,
        // then their MFMAs, which run while the next reads are in flight.
#pragma unroll
        for (int j = 0; j < NC; ++j)
          if (rescale[j]) {
#pragma unroll
            for (int mt = 0; mt < DW / 16; ++mt) st.acc[j][mt] *= alpha[j];
          }
        const int vtok = 4 * g + (n >> 2);
        const uint32_t vrow = uint32_t(uintptr_t(vsrc)) + vtok * T::BRB + (n & 1) * 8;
#pragma unroll
        for (int q4 = 0; q4 < DW / 64; ++q4) {
          uint32_t ad[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int mt = 4 * q4 + u;
            ad[u] = vrow + (((2 * mt + ((n & 3) >> 1)) ^ T::bswz(vtok)) * 16);
          }
          // four transposed reads and their wait in one statement: the outputs
          // exist only after the wait, so no consumer can be scheduled earlier
          u32x2 vv[4];
          asm volatile(
              "ds_read_b64_tr_b16 %0, %4\n\t"
              "ds_read_b64_tr_b16 %1, %5\n\t"
              "ds_read_b64_tr_b16 %2, %6\n\t"
              "ds_read_b64_tr_b16 %3, %7\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(vv[0]), "=&v"(vv[1]), "=&v"(vv[2]), "=&v"(vv[3])
              : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
              : "memory");
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < NC; ++j)
              st.acc[j][4 * q4 + u] = mfma_pv<FMT>(vv[u], pf[j], st.acc[j][4 * q4 + u]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (FMT == kBf16) issue(s, 1, k + NBUF);
      }
    }
    wait_vmcnt<0>();                               // the ring restarts with the next segment
    wave_lds_fence();
  }
}

// No marker slot.
constexpr uint32_t kNoSlot = 0xFFFFFFFFu;

typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;

// The end of a piece. With WI > 1 the workgroup's WI waves streamed
// interleaved tiles of the same piece; their states merge through LDS: each
// wave puts its O^T into its own (drained) ring and its (m, l) per column
// into `mlx`; then every wave takes M = max m_i and the weights exp2(m_i -
// M) in wave order, and sums the O^T blocks 16 mt .. of its share of the
// head dims in wave order (deterministic). The piece then writes o = O / l
// (times the FP8 v scale), m = M ln 2 and l to workspace slot `slot` of its
// query columns, or BF16 output when the call has no split (a.out), and an end
// marker (l = -1) in slot `marker` when that is not kNoSlot.
template <int FMT, int D, int DS, int NC, int WI>
__device__ __forceinline__ void finish_piece(const DecodeArgs& a, StreamLds<FMT, D / DS, DS>* shs,
                                             lds_f32x2* mlx, WaveState<FMT, D, DS, NC>& st,
                                             uint32_t b, uint32_t kh, uint32_t slot,
                                             uint32_t marker) {
  constexpr int DW = D / DS;
  constexpr int MT = DW / 16;                    // 16-dim blocks of a wave's share
  static_assert(WI == 1 || DS == 1, "waves interleave tiles of whole rows only");
  static_assert(MT % WI == 0, "the merged blocks split evenly over the waves");
  constexpr int MW = MT / WI;                    // blocks each wave merges and writes
  const int lane = threadIdx.x & 63;
  const int wv = int(threadIdx.x >> 6);
  const int w = DS > 1 ? wv : 0;                 // head-dim part
  const int wi = WI > 1 ? wv : 0;                // interleaved wave
  // the wave that writes the piece's (m, l) and end marker: the first of the
  // waves sharing the piece
  const bool lead = (DS > 1 ? w : wi) == 0;
  const int g = lane >> 4, n = lane & 15;
  const uint32_t kvh = kh / a.head_chunks, hc = kh % a.head_chunks;

  float M[NC], lsum[NC];
  f32x4 o[NC][MW];
  if constexpr (WI > 1) {
    static_assert(sizeof(StreamLds<FMT, DW, DS>) >= size_t(NC) * MT * 64 * 16,
                  "a wave's ring holds its O^T for the merge");
    lds_f32x4* const mine = (lds_f32x4*)(lds_u8*)(shs[wi].ring);
#pragma unroll
    for (int k = 0; k < NC; ++k) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) mine[(k * MT + mt) * 64 + lane] = st.acc[k][mt];
      const float lw = sum_over_rows(st.l_run[k]);
      if (g == 0) mlx[(wi * NC + k) * 16 + n] = f32x2{st.m_run[k], lw};
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      f32x2 ml[WI];
      M[k] = kMaxFloor;
#pragma unroll
      for (int i = 0; i < WI; ++i) {
        ml[i] = mlx[(i * NC + k) * 16 + n];
        M[k] = fmaxf(M[k], ml[i][0]);
      }
      float wgt[WI];
      lsum[k] = 0.0f;
#pragma unroll
      for (int i = 0; i < WI; ++i) {
        wgt[i] = __builtin_amdgcn_exp2f(ml[i][0] - M[k]);
        lsum[k] += wgt[i] * ml[i][1];
      }
      // every wave's blocks come back from LDS, its own included: indexing
      // the register array by the wave number would move it to scratch
#pragma unroll
      for (int u = 0; u < MW; ++u) {
        const int mt = wi * MW + u;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < WI; ++i)
          s += wgt[i] * ((lds_f32x4*)(lds_u8*)(shs[i].ring))[(k * MT + mt) * 64 + lane];
        o[k][u] = s;
      }
    }
    // the rings are refilled by the next piece only once every wave has read them
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    (void)shs;
    (void)mlx;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      M[k] = st.m_run[k];
      lsum[k] = sum_over_rows(st.l_run[k]);
#pragma unroll
      for (int u = 0; u < MW; ++u) o[k][u] = st.acc[k][u];
    }
  }

#pragma unroll
  for (int k = 0; k < NC; ++k) {
    // a column without keys (l = 0) writes zeros
    const float inv = lsum[k] > 0.0f ? a.out_scale / lsum[k] : 0.0f;
    uint32_t qi, qh;
    if (!column_of(a, kvh, (hc * NC + k) * 16 + n, qi, qh)) continue;
    if (a.out) {
      // non-split: the whole row in one piece, the normalized output
      // straight to BF16
      uint16_t* orow = a.out + uint64_t(b) * a.o_seq + uint64_t(qi) * a.o_tok +
                       uint64_t(qh) * a.o_head + w * DW;
#pragma unroll
      for (int u = 0; u < MW; ++u) {
        const int mt = wi * MW + u;
        *reinterpret_cast<u32x2*>(orow + 16 * mt + 4 * g) =
            u32x2{pack_bf16x2(o[k][u][0] * inv, o[k][u][1] * inv),
                  pack_bf16x2(o[k][u][2] * inv, o[k][u][3] * inv)};
      }
      continue;
    }
    // workspace row of the column: [B][q_len][Hq] order
    const uint64_t qrow = (uint64_t(b) * a.q_len + qi) * a.num_q_heads + qh;
    float* const wbase = a.ws + qrow * a.num_splits * (D + 2);
    float* wrow = wbase + uint64_t(slot) * (D + 2);
#pragma unroll
    for (int u = 0; u < MW; ++u) {
      const int mt = wi * MW + u;
      f32x2 lo2 = {o[k][u][0] * inv, o[k][u][1] * inv};
      f32x2 hi2 = {o[k][u][2] * inv, o[k][u][3] * inv};
      *reinterpret_cast<f32x2*>(wrow + w * DW + mt * 16 + 4 * g) = lo2;
      *reinterpret_cast<f32x2*>(wrow + w * DW + mt * 16 + 4 * g + 2) = hi2;
    }
    if (g == 0 && lead) {
      wrow[D] = M[k] * kLn2;
      wrow[D + 1] = lsum[k];
      // the row ends in this piece: an end marker (l = -1) tells the combine
      // to ignore that slot and all later ones
      if (marker != kNoSlot) {
        float* e = wbase + uint64_t(marker) * (D + 2);
        e[D] = -__builtin_inff();
        e[D + 1] = -1.0f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Query blocks wider than one wave (BF16 tiles): WQ waves of a workgroup
// share every K/V tile of the row's pages through one LDS ring, each wave
// owning NC chunks of 16 query columns, so the pages are read once per
// WQ * NC * 16 columns instead of once per NC * 16. Each wave issues its
// share of a tile's DMA loads; rows at or past the sequence length get an
// offset past the page and read as zeros, so no wave ever writes the shared
// tiles. One workgroup barrier per tile makes the tile visible to all waves
// and frees the slot of the previous tile, which is refilled right after it.
#ifndef PKD_SHARED_NB
#define PKD_SHARED_NB 3
#endif
template <int D>
struct SharedLds {
  static constexpr int NB = PKD_SHARED_NB;       // tile-pair slots of the ring
  __attribute__((aligned(1024))) uint8_t ring[NB * LdsTraits<kBf16, D>::SLOT];
};

template <int D, int NC, int WQ>
__device__ __forceinline__ void run_piece_shared(const DecodeArgs& a, SharedLds<D>& sh,
                                                 uint32_t b, uint32_t kh, uint32_t tau0,
                                                 uint32_t tau1, uint32_t slot, bool last,
                                                 uint32_t L) {
  using T = LdsTraits<kBf16, D>;
  constexpr int NB = SharedLds<D>::NB;
  constexpr int NLD = 2 * T::NI;                 // load instructions of a K + V tile pair
  static_assert(NLD % WQ == 0, "the tile loads split evenly over the waves");
  constexpr int LPW = NLD / WQ;                  // load instructions per wave and tile
  b = __builtin_amdgcn_readfirstlane(b);
  kh = __builtin_amdgcn_readfirstlane(kh);
  tau0 = __builtin_amdgcn_readfirstlane(tau0);
  tau1 = __builtin_amdgcn_readfirstlane(tau1);
  slot = __builtin_amdgcn_readfirstlane(slot);
  L = __builtin_amdgcn_readfirstlane(L);
  if (slot >= a.num_splits) return;      // the same for every wave of the workgroup
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int g = lane >> 4;
  const int n = lane & 15;
  const uint32_t kvh = kh / a.head_chunks, hc = kh % a.head_chunks;
  const uint32_t lo = (a.window > 0 && L > a.window) ? L - a.window : 0u;
  const uint32_t tpp = a.block_size / 16;
  const uint32_t t0 = lo / 16 + tau0, t1 = lo / 16 + tau1;
  const uint32_t pa = t0 / tpp, pb = (t1 + tpp - 1) / tpp;
  const uint32_t chunk0 = (hc * WQ + w) * NC;    // this wave's first column chunk

  bool head_ok[NC];
  uint64_t qoff[NC];
  uint32_t c_lo[NC], c_hi[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    uint32_t qi, qh;
    head_ok[k] = column_of(a, kvh, (chunk0 + k) * 16 + n, qi, qh);
    qoff[k] = uint64_t(b) * a.q_stride + uint64_t(qi) * a.q_tok_stride +
              uint64_t(qh) * a.q_head_stride;
    c_lo[k] = lo;
    c_hi[k] = L;
    if (a.causal && head_ok[k]) {
      const int p1 = int(L) - int(a.q_len) + int(qi) + 1;
      c_hi[k] = p1 > 0 ? uint32_t(p1) : 0u;
      c_lo[k] = (a.q_window > 0 && c_hi[k] > a.q_window) ? c_hi[k] - a.q_window : 0u;
    }
  }
  const int32_t* bt = a.block_tables + uint64_t(b) * a.max_blocks;
  u32x4 qf[NC][D / 32];
#pragma unroll
  for (int k = 0; k < NC; ++k)
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head_ok[k]) v = *reinterpret_cast<const u32x4*>(a.q + qoff[k] + qk_dim<kBf16, D>(c, g));
      qf[k][c] = v;
    }

  lds_u8* const ring3 = (lds_u8*)(sh.ring);
  const int ld_row = lane / T::CPR;
  const int ld_pos = lane % T::CPR;
  f32x4 acc[NC][D / 16];
  float m_run[NC], l_run[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) acc[k][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[k] = kMaxFloor;
    l_run[k] = 0.0f;
  }

  for (uint32_t cp = pa; cp < pb;) {
    const uint32_t cpe = min(cp + 64, pb);
    const int32_t bt_reg = (cp + lane < cpe) ? bt[cp + lane] : 0;
    const uint32_t ct0 = max(cp * tpp, t0);
    const uint32_t ct1 = min(cpe * tpp, t1);

    // this wave's share of tile t (K and V) into ring slot s; a tile past the
    // segment gets zero-length descriptors
    auto issue = [&](int s, uint32_t t) {
      const bool live = t < ct1;
      const uint32_t page = min(t / tpp, cpe - 1);
      const uint32_t phys = uint32_t(__builtin_amdgcn_readlane(bt_reg, int(page - cp)));
      const uint32_t off0 = (t % tpp) * 16;
#pragma unroll
      for (int m = 0; m < LPW; ++m) {
        const int mi = w + m * WQ;                 // load instruction of the tile pair
        const int kv = mi / T::NI, i = mi % T::NI;
        const uint8_t* pool = kv ? a.v_cache : a.k_cache;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(pool + uint64_t(phys) * a.page_bytes), 0,
            live ? int(a.page_bytes) : 0, 0x00020000);
        const int row = i * T::RPI + ld_row;
        const int chunk = ld_pos ^ T::swz(row);
        const bool keep = row < 16 && t * 16 + row < L;
        const int voff = keep ? int(((off0 + row) * a.num_kv_heads + kvh) * T::RB + chunk * 16)
                              : 0x7FFFFFF0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (lds_void*)(ring3 + s * T::SLOT + kv * T::KV + i * 1024), 16, voff, 0, 0, 2);
      }
    };

#pragma unroll
    for (int s = 0; s < NB - 1; ++s) issue(s, ct0 + s);
    int s = 0;                                     // slot of tile t
    for (uint32_t t = ct0; t < ct1; ++t) {
      const uint32_t tok0 = t * 16;
      // tile t is in LDS once every wave's share has landed
      wait_vmcnt<(NB - 2) * LPW>();
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      issue(s == 0 ? NB - 1 : s - 1, t + NB - 1);  // the slot of tile t - 1 is free now
      lds_u8* const kt = ring3 + s * T::SLOT;
      lds_u8* const vt = kt + T::KV;

      f32x4 sc[NC];
#pragma unroll
      for (int k = 0; k < NC; ++k) sc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 kv = *(lds_u32x4*)(kt + n * T::RB + ((4 * c + g) ^ T::swz(n)) * 16);
#pragma unroll
        for (int k = 0; k < NC; ++k) sc[k] = mfma_qk<kBf16>(kv, qf[k][c], sc[k]);
      }

      bool rescale[NC];
      float alpha[NC];
      u32x2 pf[NC];
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        float sv[4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t tok = tok0 + 4 * g + j;
          sv[j] = (tok >= c_lo[k] && tok < c_hi[k]) ? sc[k][j] * a.logit_scale : -__builtin_inff();
          mx = fmaxf(mx, sv[j]);
        }
        mx = max_over_rows(mx);
        rescale[k] = __builtin_amdgcn_ballot_w64(mx > m_run[k] + kLazyMax) != 0;
        alpha[k] = 1.0f;
        if (rescale[k]) {
          const float m_new = fmaxf(m_run[k], mx);
          alpha[k] = __builtin_amdgcn_exp2f(m_run[k] - m_new);
          m_run[k] = m_new;
        }
        uint32_t pbits[4];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(sv[j] - m_run[k]);
          pbits[j] = p_bits<kBf16>(p);
          psum += p_value<kBf16>(pbits[j]);
        }
        l_run[k] = l_run[k] * alpha[k] + psum;
        pf[k] = u32x2{pbits[0] | (pbits[1] << 16), pbits[2] | (pbits[3] << 16)};
      }
#pragma unroll
      for (int k = 0; k < NC; ++k)
        if (rescale[k]) {
#pragma unroll
          for (int mt = 0; mt < D / 16; ++mt) acc[k][mt] *= alpha[k];
        }
      {
        const int vtok = 4 * g + (n >> 2);
        const uint32_t vrow = uint32_t(uintptr_t(vt)) + vtok * T::BRB + (n & 1) * 8;
#pragma unroll
        for (int q4 = 0; q4 < D / 64; ++q4) {
          uint32_t ad[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int mt = 4 * q4 + u;
            ad[u] = vrow + (((2 * mt + ((n & 3) >> 1)) ^ T::bswz(vtok)) * 16);
          }
          u32x2 vv[4];
          asm volatile(
              "ds_read_b64_tr_b16 %0, %4\n\t"
              "ds_read_b64_tr_b16 %1, %5\n\t"
              "ds_read_b64_tr_b16 %2, %6\n\t"
              "ds_read_b64_tr_b16 %3, %7\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(vv[0]), "=&v"(vv[1]), "=&v"(vv[2]), "=&v"(vv[3])
              : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
              : "memory");
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < NC; ++k)
              acc[k][4 * q4 + u] = mfma_pv<kBf16>(vv[u], pf[k], acc[k][4 * q4 + u]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      s = s == NB - 1 ? 0 : s + 1;
    }
    // the ring restarts with the next segment once every wave is done with it
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    cp = cpe;
  }

#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const float l_tot = sum_over_rows(l_run[k]);
    const float inv = l_tot > 0.0f ? a.out_scale / l_tot : 0.0f;
    if (!head_ok[k]) continue;
    uint32_t qi, qh;
    column_of(a, kvh, (chunk0 + k) * 16 + n, qi, qh);
    if (a.out) {
      uint16_t* orow = a.out + uint64_t(b) * a.o_seq + uint64_t(qi) * a.o_tok +
                       uint64_t(qh) * a.o_head;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
        *reinterpret_cast<u32x2*>(orow + 16 * mt + 4 * g) =
            u32x2{pack_bf16x2(acc[k][mt][0] * inv, acc[k][mt][1] * inv),
                  pack_bf16x2(acc[k][mt][2] * inv, acc[k][mt][3] * inv)};
      continue;
    }
    const uint64_t qrow = (uint64_t(b) * a.q_len + qi) * a.num_q_heads + qh;
    float* const wbase = a.ws + qrow * a.num_splits * (D + 2);
    float* wrow = wbase + uint64_t(slot) * (D + 2);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      *reinterpret_cast<f32x2*>(wrow + mt * 16 + 4 * g) = f32x2{acc[k][mt][0] * inv, acc[k][mt][1] * inv};
      *reinterpret_cast<f32x2*>(wrow + mt * 16 + 4 * g + 2) = f32x2{acc[k][mt][2] * inv, acc[k][mt][3] * inv};
    }
    if (g == 0) {
      wrow[D] = m_run[k] * kLn2;
      wrow[D + 1] = l_tot;
    }
    if (last && g == 0 && slot + 1 < a.num_splits) {
      float* e = wbase + uint64_t(slot + 1) * (D + 2);
      e[D] = -__builtin_inff();
      e[D + 1] = -1.0f;
    }
  }
}

// Zeros for the query columns of row (b, kh) of a sequence without keys.
// With WQ waves sharing a row, wave w zeros its own chunks.
template <int D, int NC, int WQ>
__device__ __forceinline__ void zero_row(const DecodeArgs& a, uint32_t b, uint32_t kh) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  const uint32_t w = WQ > 1 ? threadIdx.x >> 6 : 0u;
  const uint32_t kvh = kh / a.head_chunks, hc = kh % a.head_chunks;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    uint32_t qi, qh;
    if (!column_of(a, kvh, ((hc * WQ + w) * NC + k) * 16 + n, qi, qh)) continue;
    uint16_t* orow = a.out + uint64_t(b) * a.o_seq + uint64_t(qi) * a.o_tok + uint64_t(qh) * a.o_head;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
      *reinterpret_cast<u32x2*>(orow + 16 * mt + 4 * g) = u32x2{0u, 0u};
  }
}

// Head-dim split: at head_dim 512 a workgroup of DS waves shares each row
// piece, each wave holding D/DS of the dims (the accumulator alone would
// otherwise take 128 registers of one wave): two waves, or four for NVFP4
// tiles (PKD_NVFP4_DSPLIT), whose dequant work wants more waves per CU than
// half-dim registers allow.
#ifndef PKD_NVFP4_DSPLIT
#define PKD_NVFP4_DSPLIT 2
#endif
template <int FMT, int D>
constexpr int kDSplit = D == 512 ? (FMT == kNvfp4 ? PKD_NVFP4_DSPLIT : 2) : 1;

// Waves per SIMD the register budget is held to: quantized tiles up to
// head_dim 256 and split head dims run two (their ALU work hides behind the
// other wave's loads).
template <int FMT, int D>
constexpr int kWavesPerSimd =
    kDSplit<FMT, D> > 2 ? 3 : (((FMT != kBf16 && D <= 256) || kDSplit<FMT, D> > 1) ? 2 : 1);

// Column chunks one wave can carry: two for BF16 tiles up to head_dim 128
// (a second accumulator and q fit the registers), else one.
template <int FMT, int D>
constexpr int kMaxChunks = (FMT == kBf16 && D <= 128) ? 2 : 1;

// The pieces of partition unit `unit` of the P units of a launch (one
// workgroup) under the stream partition (rows of R per sequence; with kv-head
// groups, a row stands for the group's head_group rows and kh is the group's
// row index), in order: piece(b, kh, tau0, tau1, slot, last, L, can_append)
// for each (can_append: the sequence's length is within its block-table row,
// so its new token has a position to go to); with num_splits 1 the unit takes
// row `unit` whole, and for a sequence without keys writes zeros if
// `zero_lead` (the unit's lead wave).
template <int D, int NC, int WQ, typename Piece>
__device__ __forceinline__ void for_each_piece(const DecodeArgs& a, uint32_t unit, uint32_t P,
                                               bool zero_lead, Piece&& piece) {
  // rows per sequence; kv heads in groups of head_group share one row's
  // pieces, each head its own workgroup
  const uint32_t R = a.num_kv_heads / a.head_group * a.head_chunks;
  const bool whole = a.num_splits == 1;                       // one unit per row
  // With at most 64 sequences, one length per lane, loaded once: the tile
  // counts, their prefix sums and every row lookup come from these registers.
  const bool cached = a.num_seqs <= 64;
  uint32_t L_l = 0, n_l = 0, T = 0, live = 0, incl = 0, live_le = 0;
  uint64_t over = 0;                        // sequences longer than their block-table row
  if (cached && !whole) {
    const uint32_t lane = threadIdx.x & 63;
    const int32_t Ls = lane < a.num_seqs ? a.seq_lens[lane] : 0;
    over = __builtin_amdgcn_ballot_w64(Ls > 0 && uint32_t(Ls) > a.max_len);
    L_l = seq_len(a, Ls);
    n_l = row_tiles(L_l, a.window);
    incl = wave_scan(n_l * R);
    T = uint32_t(__builtin_amdgcn_readlane(int(incl), 63));
    // sequences with keys: in the wave, and up to this lane
    const uint64_t has = __builtin_amdgcn_ballot_w64(n_l > 0);
    live = uint32_t(__builtin_popcountll(has)) * R;
    live_le = __builtin_amdgcn_mbcnt_hi(uint32_t(has >> 32),
                                        __builtin_amdgcn_mbcnt_lo(uint32_t(has), 0u)) +
              (n_l > 0 ? 1u : 0u);
  } else if (!whole) {
    T = total_tiles(a, R, live);
  }
  // Start-up positions: each row with keys is laid out behind `lead` empty
  // positions, paid by the wave that starts the row for that row's first
  // round trips (length, block table and q, first tile, with its ring
  // empty). They fill only the slack that rounding c up left (P*c >= T +
  // lead*live), so no wave gets more positions than c, unless c is long
  // enough that one more tile costs little. When c is the least chunk
  // instead, waves are idle anyway and the rows stay aligned.
  uint32_t c = 1, lead = 0, pos = unit, end = unit + 1;
  if (!whole) {
    const uint32_t c0 = (T + P - 1) / P;
    c = max(c0, a.chunk_min);
    if (live > 0 && c == c0) {
      uint32_t slack = P * c - T;                  // < P: c rounds T / P up
      // Chunks of 32 tiles or more: one more tile per wave (at most 3%) when
      // that buys every row its whole lead.
      if (c >= 32 && live * a.row_lead > slack && live * a.row_lead <= slack + P) {
        ++c;
        slack += P;
      }
      lead = live * a.row_lead <= slack ? a.row_lead : slack / live;
    }
    incl += lead * R * live_le;                  // inclusive prefix of the laid-out spans
    const uint32_t flat = T + lead * live;
    pos = uint32_t(min(uint64_t(unit) * c, uint64_t(flat)));
    end = uint32_t(min(uint64_t(pos) + c, uint64_t(flat)));
  }
  while (pos < end) {
    // the row holding flat position pos: sequence b, row kh, its n tiles
    // from flat position rs (behind `lead` start-up positions)
    uint32_t b, kh, n, rs, L;
    bool fits = true;
    if (whole) {
      b = unit / R;
      kh = unit % R;
      if (b >= a.num_seqs) break;                  // a unit past the rows of the launch
      const int32_t Ls = a.seq_lens[b];
      fits = !(Ls > 0 && uint32_t(Ls) > a.max_len);
      L = seq_len(a, Ls);
      n = row_tiles(L, a.window);
      rs = pos;
      if (n == 0) {
        if (a.out && zero_lead) zero_row<D, NC, WQ>(a, b, kh);
        break;
      }
    } else if (cached) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > pos);
      const int l = hit ? __builtin_ctzll(hit) : 64;
      if (uint32_t(l) >= a.num_seqs) break;        // pos < T + lead * live: never taken
      n = uint32_t(__builtin_amdgcn_readlane(int(n_l), l));
      const uint32_t span = n + lead;
      const uint32_t excl = uint32_t(__builtin_amdgcn_readlane(int(incl), l)) - span * R;
      L = uint32_t(__builtin_amdgcn_readlane(int(L_l), l));
      fits = ((over >> l) & 1) == 0;
      b = uint32_t(l);
      kh = (pos - excl) / span;
      rs = excl + kh * span + lead;
    } else {
      const RowLoc r = find_row(a, pos, R, lead);
      if (r.b >= a.num_seqs) break;                // as above: never taken
      b = r.b;
      kh = r.kh;
      n = r.n - lead;
      rs = r.start + lead;
      const int32_t Ls = a.seq_lens[b];
      fits = !(Ls > 0 && uint32_t(Ls) > a.max_len);
      L = seq_len(a, Ls);
    }
    if (n == 0 || kh >= R) break;                  // as above: never taken
    const uint32_t f0 = max(pos, rs);
    const uint32_t f1 = whole ? rs + n : min(rs + n, end);
    if (f1 > f0) {
      // slot: waves from the one holding the row's first tile
      piece(b, kh, f0 - rs, f1 - rs, whole ? 0u : f0 / c - rs / c, whole || rs + n <= end, L,
            fits);
    }
    if (whole) break;
    pos = max(f1, min(rs, end));
  }
}

// Waves of a workgroup that share a piece by interleaving its tiles (wave i
// takes tiles i, i + WI, ...) and merge their states in LDS before one
// workspace write: four, one per SIMD of a CU, for BF16 and FP8 rows of one
// column chunk up to head_dim 256 (a wave's ring then holds its O^T for the
// merge). A launch then writes a quarter of the partials and the combine
// reads a quarter of the slots.
template <int FMT, int D, int NC>
constexpr int kMergeWaves = (kDSplit<FMT, D> == 1 && FMT != kNvfp4 && NC == 1) ? 4 : 1;

// Waves of a stream workgroup: WI interleaving waves, or the DS waves of a
// split head dim, or one.
template <int FMT, int D, int WI>
constexpr int kGroupWaves = kDSplit<FMT, D> > 1 ? kDSplit<FMT, D> : WI;

// The stream kernel, one partition unit per workgroup. WI = 1: a unit is one
// wave (two sharing a split head dim), which may cross rows (split-K passes
// over a batch). WI > 1: the WI waves of a workgroup take the tiles of one
// piece in turn (wave i tiles i, i + WI, ...) and merge their states in LDS
// before one write (a single sequence, one piece per workgroup; or a whole
// row per workgroup with no split), so the launch writes a WI-th of the
// partials.
template <int FMT, int D, int NC, bool CONTIG, int WI>
__global__ __launch_bounds__((64 * kGroupWaves<FMT, D, WI>), (kWavesPerSimd<FMT, D>)) void splitk_stream(
    DecodeArgs a) {
  constexpr int DS = kDSplit<FMT, D>;
  constexpr int GW = kGroupWaves<FMT, D, WI>;
  static_assert(WI == 1 || WI == kMergeWaves<FMT, D, NC>, "interleaved waves merge in LDS");
  __shared__ StreamLds<FMT, D / DS, DS> sh[GW];
  __shared__ __attribute__((aligned(16))) uint8_t xg[DS > 1 ? 2 * DS * 64 * 16 : 16];
  __shared__ f32x2 mlx[WI > 1 ? WI * NC * 16 : 1];
  const uint32_t wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  StreamLds<FMT, D / DS, DS>& mine = sh[GW > 1 ? wv : 0];
  const uint32_t wi = WI > 1 ? wv : 0;
  uint32_t unit = blockIdx.x, P = gridDim.x;
  lds_u8* const xg3 = (lds_u8*)xg;
  lds_f32x2* const mlx3 = (lds_f32x2*)mlx;
  uint32_t xturn = 0;
  if (a.static_q) {
    // One sequence, no window: unit u takes row u % R and, as j = u / R of
    // the row's Q units, its tiles j + Q m (wave i of an interleaving group
    // the m = i mod WI). Which tiles a wave streams does not depend on the
    // length, so its q and block-table entries are requested in the same
    // round trip as the length.
    const uint32_t R = a.num_kv_heads * a.head_chunks;
    const uint32_t Q = a.static_q;                 // <= num_splits
    const uint32_t kh = unit % R, j = unit / R;
    if (j >= Q) return;                            // a unit past the R * Q of the launch
    const int32_t Ls = a.seq_lens[0];
    const uint32_t L = seq_len(a, Ls);
    WaveState<FMT, D, DS, NC> st;
    stream_tiles<FMT, D, DS, NC, CONTIG>(a, mine, xg3, xturn, 0, kh, j + Q * wi, Q * WI,
                                         (L + 15) / 16, L, !(Ls > 0 && uint32_t(Ls) > a.max_len),
                                         st);
    finish_piece<FMT, D, DS, NC, WI>(a, sh, mlx3, st, 0, kh, j,
                                     (j == 0 && Q < a.num_splits) ? Q : kNoSlot);
    return;
  }
  // Kv heads grouped by head_group: the group's workgroups of one unit are 8
  // apart in the grid (units in runs of 8), so the dispatcher, which deals
  // workgroups to the 8 XCDs in turn, puts them on one XCD, where the cache
  // lines their rows share (NVFP4 scale rows, rows shorter than a line) are
  // fetched from HBM once. The grid is a multiple of 8 * head_group.
  const uint32_t hg = a.head_group;
  uint32_t member = 0;
  if (hg > 1) {
    member = (unit / 8) % hg;
    unit = unit / (8 * hg) * 8 + unit % 8;
    P /= hg;
  }
  for_each_piece<D, NC, 1>(a, unit, P, wv == 0,
                           [&](uint32_t b, uint32_t kg, uint32_t tau0, uint32_t tau1,
                               uint32_t slot, bool last, uint32_t L, bool fits) {
    if (slot >= a.num_splits) return;      // only if a sequence outgrows its block table
    // the row of kv head (head group, member), column chunk kg % head_chunks
    const uint32_t kh =
        hg > 1 ? ((kg / a.head_chunks) * hg + member) * a.head_chunks + kg % a.head_chunks : kg;
    const uint32_t lo = (a.window > 0 && L > a.window) ? L - a.window : 0u;
    const uint32_t t0 = lo / 16 + tau0, t1 = lo / 16 + tau1;   // tiles of the sequence
    WaveState<FMT, D, DS, NC> st;
    stream_tiles<FMT, D, DS, NC, CONTIG>(a, mine, xg3, xturn, b, kh, t0 + wi, WI, t1, L, fits,
                                         st);
    finish_piece<FMT, D, DS, NC, WI>(a, sh, mlx3, st, b, kh, slot,
                                     (last && slot + 1 < a.num_splits) ? slot + 1 : kNoSlot);
  });
}

// WQ waves sharing the K/V tiles of each piece (BF16 query blocks).
template <int D, int NC, int WQ>
__global__ __launch_bounds__(64 * WQ, 1) void splitk_shared(DecodeArgs a) {
  __shared__ SharedLds<D> sh;
  for_each_piece<D, NC, WQ>(a, blockIdx.x, gridDim.x, true,
                            [&](uint32_t b, uint32_t kh, uint32_t tau0, uint32_t tau1,
                                uint32_t slot, bool last, uint32_t L, bool) {
    run_piece_shared<D, NC, WQ>(a, sh, b, kh, tau0, tau1, slot, last, L);
  });
}

// Slots whose values each combine lane requests before the weights are known
// (a multiple of 8; clamped to the slot count at run time).
#ifndef PKD_COMBINE_U
#define PKD_COMBINE_U 8
#endif
#ifndef PKD_COMBINE_WAVE_R
#define PKD_COMBINE_WAVE_R 8
#endif
// Most workgroups a combine launch splits rows' columns up to.
#ifndef PKD_COMBINE_MAX_WG
#define PKD_COMBINE_MAX_WG 256
#endif

// Where the combine writes query row bh (sequence-major: per_seq rows per
// sequence, heads rows per token): element strides of sequence, token, head.
struct OutMap {
  uint64_t seq, tok, head;
  uint32_t per_seq, heads;
};

__device__ __forceinline__ uint16_t* out_row(uint16_t* out, const OutMap& om, uint32_t bh) {
  const uint32_t b = bh / om.per_seq, r = bh - b * om.per_seq;
  const uint32_t i = r / om.heads, h = r - i * om.heads;
  return out + uint64_t(b) * om.seq + uint64_t(i) * om.tok + uint64_t(h) * om.head;
}

// Combine: CW workgroups of NT lanes per (sequence, q head), workgroup c
// taking CC = D / (2 CW) of the float2 columns. Lane t owns column t % CC of
// its share and the slots i = t / CC (mod KS). It requests its first U slots'
// values at the start, in the same round trip as the first NT slots' (m, l);
// further (m, l) are read in chunks of NT only while no end marker has shown
// up. The (m, l) go to LDS and become weights. A value enters the sum only
// where its slot's weight is nonzero, so slots past the end marker, whose
// contents are stale, never reach it. Further slots follow in rounds of eight
// loads, and the KS partial sums are added in a fixed order (deterministic).
template <int D, int NT, int CW>
__global__ __launch_bounds__(NT) void reduce_kernel(const float* ws, uint16_t* out,
                                                    const int32_t* seq_lens, OutMap om,
                                                    uint32_t num_splits) {
  constexpr int CC = D / 2 / CW;              // float2 columns of one workgroup
  constexpr int KS = NT / CC;                 // split lanes
  constexpr int NW = NT / 64;                 // waves
  constexpr int U = PKD_COMBINE_U;            // slots per lane requested up front
  static_assert(CC * CW == D / 2 && CC * KS == NT, "combine lane split");
  extern __shared__ float wsh[];              // l (then weights) and m of every slot
  __shared__ float red[NW], red2[NW];
  __shared__ uint32_t stops[NW];
  __shared__ f32x2 part[KS][CC];
  const int tid = threadIdx.x;
  const uint32_t bh = blockIdx.x / CW;
  const int col = int(blockIdx.x % CW) * CC + tid % CC, ks = tid / CC;
  const uint32_t b = bh / om.per_seq;
  uint16_t* o = out_row(out, om, bh);
  const float* base = ws + uint64_t(bh) * num_splits * (D + 2);

  // unconditional loads (the slot index clamped into the workspace), so that
  // no branch sits between them and all are in flight at once
  f32x2 v0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t i = min(uint32_t(ks + u * KS), num_splits - 1);
    v0[u] = *reinterpret_cast<const f32x2*>(base + uint64_t(i) * (D + 2) + 2 * col);
  }
  // slot i counts if l_i > 0 and no earlier slot holds an end marker (l < 0).
  // One pass per NT slots finds each wave's first marker and the largest m
  // of the wave's live slots before it; the block then takes the first
  // marker (stop) and the largest m of the waves that start before it.
  const int32_t L = seq_lens[b];
  const int wv = tid >> 6;
  uint32_t stop = num_splits;
  float M = -__builtin_inff();
  for (uint32_t c0 = 0; c0 < num_splits; c0 += NT) {
    const uint32_t i = c0 + tid;
    f32x2 ml = {-__builtin_inff(), 0.0f};
    if (i < num_splits) {
      ml = *reinterpret_cast<const f32x2*>(base + uint64_t(i) * (D + 2) + D);
      wsh[i] = ml[1];
      wsh[num_splits + i] = ml[0];
    }
    const uint64_t marks = __builtin_amdgcn_ballot_w64(i < num_splits && ml[1] < 0.0f);
    const uint32_t mark = marks ? c0 + uint32_t(tid & ~63) + uint32_t(__builtin_ctzll(marks))
                                : num_splits;
    const float mw = wave_max(ml[1] > 0.0f && i < mark ? ml[0] : -__builtin_inff());
    if ((tid & 63) == 0) {
      stops[wv] = mark;
      red[wv] = mw;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NW; ++k) stop = min(stop, stops[k]);
#pragma unroll
    for (int k = 0; k < NW; ++k)
      if (c0 + 64u * k < stop) M = fmaxf(M, red[k]);
    if (stop < num_splits || c0 + NT >= num_splits) break;   // the same for every lane
    __syncthreads();                            // stops and red are written again
  }
  if (L <= 0) {                               // empty sequence: zeros
    stop = 0;
    M = -__builtin_inff();
  }
  if (M == -__builtin_inff()) {               // no slot holds a key
    if (tid < CC) reinterpret_cast<uint32_t*>(o)[col] = 0u;
    return;
  }
  // weights, each lane for the slots it read above (no barrier needed)
  float wsum = 0.0f;
  for (uint32_t i = tid; i < stop; i += NT) {
    const float l = wsh[i];
    const float w = l > 0.0f ? l * __builtin_amdgcn_exp2f((wsh[num_splits + i] - M) * kLog2e)
                             : 0.0f;
    wsh[i] = w;
    wsum += w;
  }
  wsum = wave_sum(wsum);
  if ((tid & 63) == 0) red2[wv] = wsum;
  __syncthreads();
  wsum = 0.0f;
#pragma unroll
  for (int k = 0; k < NW; ++k) wsum += red2[k];

  f32x2 acc = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t i = ks + u * KS;
    const float w = i < stop ? wsh[i] : 0.0f;
    if (w != 0.0f) {
      acc[0] = fmaf(w, v0[u][0], acc[0]);
      acc[1] = fmaf(w, v0[u][1], acc[1]);
    }
  }
  for (uint32_t i0 = ks + U * KS; i0 < stop; i0 += 8 * KS) {
    // eight slots per round; a slot without keys is not read
    float w[8];
    f32x2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = i0 + u * KS;
      w[u] = i < stop ? wsh[i] : 0.0f;
      v[u] = f32x2{0.0f, 0.0f};
      if (w[u] != 0.0f)
        v[u] = *reinterpret_cast<const f32x2*>(base + uint64_t(i) * (D + 2) + 2 * col);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc[0] = fmaf(w[u], v[u][0], acc[0]);
      acc[1] = fmaf(w[u], v[u][1], acc[1]);
    }
  }
  part[ks][tid % CC] = acc;
  __syncthreads();
  if (tid < CC) {
    f32x2 sum = part[0][tid];
#pragma unroll
    for (int k = 1; k < KS; ++k) sum += part[k][tid];
    const float inv = 1.0f / fmaxf(wsum, 1e-20f);
    reinterpret_cast<uint32_t*>(o)[col] = pack_bf16x2(sum[0] * inv, sum[1] * inv);
  }
}

// Combine with at most 64 slots and many rows: one wave per (sequence, q
// head), every reduction in registers. Lane i reads slot i's (m, l); the end
// marker and the largest m come from a ballot and a cross-lane max, the sum of
// the weights is taken in slot order. Lane c then sums float2 column c (and
// c + 64, ...) over the slots in slot order, R loads in flight; a slot whose
// weight is 0 is not read, so no bytes beyond the live slots leave memory.
template <int D>
__global__ __launch_bounds__(64) void reduce_wave_kernel(const float* ws, uint16_t* out,
                                                         const int32_t* seq_lens, OutMap om,
                                                         uint32_t num_splits) {
  constexpr int COLS = D / 2;                      // float2 columns of a slot
  constexpr int NC = COLS >= 64 ? COLS / 64 : 1;   // columns per lane
  constexpr int R = NC >= 4 ? 8 : PKD_COMBINE_WAVE_R;   // loads in flight per column
  const int lane = threadIdx.x;
  const uint32_t bh = blockIdx.x;
  const float* base = ws + uint64_t(bh) * num_splits * (D + 2);
  uint16_t* o = out_row(out, om, bh);
  f32x2 ml = {-__builtin_inff(), 0.0f};
  if (uint32_t(lane) < num_splits) ml = *reinterpret_cast<const f32x2*>(base + lane * (D + 2) + D);
  const int32_t L = seq_lens[bh / om.per_seq];
  const uint64_t marks = __builtin_amdgcn_ballot_w64(uint32_t(lane) < num_splits && ml[1] < 0.0f);
  uint32_t stop = marks ? uint32_t(__builtin_ctzll(marks)) : num_splits;
  if (L <= 0) stop = 0;
  const bool live = uint32_t(lane) < stop && ml[1] > 0.0f;
  const float M = wave_max(live ? ml[0] : -__builtin_inff());
  if (M == -__builtin_inff()) {                    // no slot holds a key
    for (int d = lane; d < D / 2; d += 64) reinterpret_cast<uint32_t*>(o)[d] = 0u;
    return;
  }
  const float w = live ? ml[1] * __builtin_amdgcn_exp2f((ml[0] - M) * kLog2e) : 0.0f;
  float wsum = 0.0f;
  for (uint32_t i = 0; i < stop; ++i)
    wsum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), int(i)));
  f32x2 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x2{0.0f, 0.0f};
  for (uint32_t i0 = 0; i0 < stop; i0 += R) {
    f32x2 v[R][NC];
    float wi[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const uint32_t i = i0 + u;
      // the slot's weight from its lane (a slot holding no keys weighs 0)
      wi[u] = i < stop ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                       __builtin_bit_cast(int, w), int(i)))
                       : 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        v[u][c] = f32x2{0.0f, 0.0f};
        if (wi[u] != 0.0f && lane + 64 * c < COLS)
          v[u][c] = *reinterpret_cast<const f32x2*>(base + i * (D + 2) + 2 * (lane + 64 * c));
      }
    }
#pragma unroll
    for (int u = 0; u < R; ++u)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc[c][0] = fmaf(wi[u], v[u][c][0], acc[c][0]);
        acc[c][1] = fmaf(wi[u], v[u][c][1], acc[c][1]);
      }
  }
  const float inv = 1.0f / fmaxf(wsum, 1e-20f);
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (lane + 64 * c < COLS)
      reinterpret_cast<uint32_t*>(o)[lane + 64 * c] = pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv);
}

static int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : kLaunch;
}

// Resident waves per CU of a stream kernel (workgroups x waves per workgroup).
template <int FMT, int D, int NC, bool CONTIG, int WI>
static int stream_occupancy() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, splitk_stream<FMT, D, NC, CONTIG, WI>,
                                                   64 * kGroupWaves<FMT, D, WI>, 0) != hipSuccess)
    return 0;
  return per_cu * kGroupWaves<FMT, D, WI>;
}

// Waves a stream kernel launches on the current device: all resident at
// once (at most the occupancy), cached per device and kernel instance. The
// cache entries are atomics: host threads that launch at the same time may
// both compute an entry, and store the same value.
template <int FMT, int D, int NC, bool CONTIG, int WI>
static uint64_t stream_capacity() {
  static std::atomic<uint64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const uint64_t known = cache[dev].load(std::memory_order_relaxed);
  if (known) return known;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int per_cu = stream_occupancy<FMT, D, NC, CONTIG, WI>();
  if (per_cu <= 0 || cus <= 0) return 0;
#ifndef PKD_STREAM_WAVES_PER_CU
#define PKD_STREAM_WAVES_PER_CU 4
#endif
#ifndef PKD_STREAM_WAVES_PER_CU_Q
#define PKD_STREAM_WAVES_PER_CU_Q 8
#endif
  // BF16: four long waves per CU stream better than more, shorter ones;
  // quantized tiles carry more ALU work per byte and gain from a second wave
  // per SIMD where the registers allow it. The count is a multiple of the CU
  // count so that every CU gets the same work.
#ifndef PKD_STREAM_WAVES_PER_CU_NC
#define PKD_STREAM_WAVES_PER_CU_NC 4
#endif
#ifndef PKD_STREAM_WAVES_PER_CU_FP8
#define PKD_STREAM_WAVES_PER_CU_FP8 4
#endif
#ifndef PKD_STREAM_WAVES_PER_CU_Q4
#define PKD_STREAM_WAVES_PER_CU_Q4 12
#endif
  const int cap = FMT == kBf16 && D < 512
                      ? (NC > 1 ? PKD_STREAM_WAVES_PER_CU_NC : PKD_STREAM_WAVES_PER_CU)
                      : (FMT == kFp8 && D < 512 ? PKD_STREAM_WAVES_PER_CU_FP8
                         : kDSplit<FMT, D> > 2  ? PKD_STREAM_WAVES_PER_CU_Q4
                                                : PKD_STREAM_WAVES_PER_CU_Q);
  if (per_cu > cap) per_cu = cap;
  const uint64_t waves = uint64_t(per_cu) * uint64_t(cus);
  cache[dev].store(waves, std::memory_order_relaxed);
  return waves;
}

// Start-up positions counted ahead of each row by the stream partition: a
// row's first round trips and its ring fill cost about three tiles' time.
#ifndef PKD_ROW_LEAD
#define PKD_ROW_LEAD 3
#endif
constexpr uint32_t kRowLead = PKD_ROW_LEAD;

// The partition counts tiles, start-up positions and wave ranges in 32 bits:
// T + 3 * rows + 2 * waves stays below 2^32 for T up to 2^30 tiles.
constexpr uint64_t kMaxLaunchTiles = 1ull << 30;

// Kv heads per head group of a batch's split-K pass: the adjacent heads
// whose rows share a 128-byte line in their shortest section (the NVFP4
// scale rows of D/16 bytes; any row shorter than a line), at most 8 and a
// divisor of the kv heads.
#ifndef PKD_HEAD_GROUP
#define PKD_HEAD_GROUP 0
#endif
template <int FMT, int D>
static uint32_t head_group_of(uint32_t num_kv_heads) {
  constexpr uint32_t row = FMT == kNvfp4 ? D / 16 : (FMT == kFp8 ? D : 2 * D);
  uint32_t hg = PKD_HEAD_GROUP > 0 ? PKD_HEAD_GROUP : (row >= 128 ? 1u : min(128u / row, 8u));
  while (hg > 1 && num_kv_heads % hg != 0) hg /= 2;
  return hg;
}

// One launch of the stream kernel with NC column chunks per wave, WI
// interleaving waves per piece (or 1: independent waves).
template <int FMT, int D, int NC, bool CONTIG, int WI>
static int launch_stream_wi(DecodeArgs a, uint64_t rows, hipStream_t stream) {
  constexpr uint32_t gw = kGroupWaves<FMT, D, WI>;    // waves of a workgroup, one unit
  // a unit of WI interleaving waves takes WI positions in one tile's time
  a.row_lead = kRowLead * WI;
  uint64_t units = rows;
  if (a.num_splits > 1) {
    const uint64_t cap = stream_capacity<FMT, D, NC, CONTIG, WI>() / gw;
    units = rows * a.num_splits;
    if (cap && units > cap) units = cap;
    // One sequence without a window: Q units per row, each taking every Q-th
    // tile, fill the same resident capacity and start without waiting for the
    // length (at most num_splits slots per row).
    if (a.static_q) {
      a.static_q = uint32_t(max(uint64_t(1), min(cap / rows, uint64_t(a.num_splits))));
      units = rows * a.static_q;
    } else if (a.head_group > 1) {
      // partition units in whole runs of 8, head_group workgroups each
      const uint64_t hg = a.head_group;
      units = max(uint64_t(8), units / hg / 8 * 8) * hg;
    }
  }
  const uint64_t groups = units;
  if (groups > 0x7FFFFFFFull) return kUnsupported;
  hipLaunchKernelGGL((splitk_stream<FMT, D, NC, CONTIG, WI>), dim3(uint32_t(groups)),
                     dim3(uint32_t(64 * gw)), 0, stream, a);
  return launch_status();
}

// One launch of the stream kernel with NC column chunks per wave: a batch's
// split-K pass on independent waves; one sequence without a window, and the
// non-split call, on waves that interleave each piece's tiles where the rows
// allow it.
template <int FMT, int D, int NC, bool CONTIG>
static int launch_stream(DecodeArgs a, hipStream_t stream) {
  a.head_chunks = (a.col_chunks + NC - 1) / NC;
  const uint64_t rows = uint64_t(a.num_seqs) * a.num_kv_heads * a.head_chunks;
  uint64_t tile_bound = uint64_t(a.max_blocks) * (a.block_size / 16);
  if (a.window > 0) tile_bound = min(tile_bound, uint64_t((a.window + 14) / 16 + 1));
  if (rows * tile_bound > kMaxLaunchTiles) return kUnsupported;
  a.chunk_min = a.num_splits > 1
                    ? uint32_t((tile_bound + a.num_splits - 2) / (a.num_splits - 1))
                    : 1u;
  constexpr int wis = kMergeWaves<FMT, D, NC>;            // the single-piece form
  constexpr uint32_t unit_waves = kGroupWaves<FMT, D, wis>;
  a.static_q = 0;                               // set to Q by launch_stream_wi
  if (a.num_splits > 1 && a.num_seqs == 1 && a.window == 0)
    a.static_q = stream_capacity<FMT, D, NC, CONTIG, wis>() / unit_waves >= rows ? 1u : 0u;
  if (a.num_splits == 1 || a.static_q)
    return launch_stream_wi<FMT, D, NC, CONTIG, wis>(a, rows, stream);
  a.head_group = head_group_of<FMT, D>(a.num_kv_heads);
  return launch_stream_wi<FMT, D, NC, CONTIG, 1>(a, rows, stream);
}


// One launch of the shared-tile kernel: rows of WQ * NC column chunks.
template <int D, int NC, int WQ>
static int launch_shared(DecodeArgs a, hipStream_t stream) {
  static std::atomic<uint64_t> cache[64];
  a.head_chunks = (a.col_chunks + NC * WQ - 1) / (NC * WQ);
  const uint64_t rows = uint64_t(a.num_seqs) * a.num_kv_heads * a.head_chunks;
  uint64_t tile_bound = uint64_t(a.max_blocks) * (a.block_size / 16);
  if (a.window > 0) tile_bound = min(tile_bound, uint64_t((a.window + 14) / 16 + 1));
  if (rows * tile_bound > kMaxLaunchTiles) return kUnsupported;
  a.chunk_min = a.num_splits > 1
                    ? uint32_t((tile_bound + a.num_splits - 2) / (a.num_splits - 1))
                    : 1u;
  a.row_lead = kRowLead;
  uint64_t groups = rows;
  if (a.num_splits > 1) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kLaunch;
    uint64_t cap = cache[dev].load(std::memory_order_relaxed);
    if (!cap) {
      int cus = 0, per_cu = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, splitk_shared<D, NC, WQ>,
                                                       64 * WQ, 0) != hipSuccess)
        return kLaunch;
#ifndef PKD_SHARED_WAVES_PER_CU
#define PKD_SHARED_WAVES_PER_CU 8
#endif
      if (per_cu > PKD_SHARED_WAVES_PER_CU / WQ) per_cu = PKD_SHARED_WAVES_PER_CU / WQ;
      cap = uint64_t(per_cu > 0 ? per_cu : 1) * uint64_t(cus > 0 ? cus : 1);
      cache[dev].store(cap, std::memory_order_relaxed);
    }
    groups = rows * a.num_splits;
    if (groups > cap) groups = cap;
  }
  if (groups > 0x7FFFFFFFull) return kUnsupported;
  hipLaunchKernelGGL((splitk_shared<D, NC, WQ>), dim3(uint32_t(groups)), dim3(64 * WQ), 0,
                     stream, a);
  return launch_status();
}

// Two chunks per wave when the row has them and the registers allow it; a
// BF16 block wider than one wave's chunks (and no append) shares each tile
// among two waves, or four when it fills more than two.
template <int FMT, int D, bool CONTIG>
static int launch_stream_nc(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (FMT == kBf16 && !CONTIG && D <= 256) {
    constexpr uint32_t nc = kMaxChunks<FMT, D>;
    if (a.col_chunks > nc && a.new_k == nullptr) {
      if (a.col_chunks <= 2 * nc) return launch_shared<D, nc, 2>(a, stream);
      return launch_shared<D, nc, 4>(a, stream);
    }
  }
  if constexpr (kMaxChunks<FMT, D> >= 2) {
    if (a.col_chunks >= 2) return launch_stream<FMT, D, 2, CONTIG>(a, stream);
  }
  return launch_stream<FMT, D, 1, CONTIG>(a, stream);
}

template <int FMT, bool CONTIG = false>
static int launch_splitk(DecodeArgs a, uint32_t num_seqs, uint32_t head_dim,
                         hipStream_t stream) {
  // one page must stay addressable by 32-bit buffer offsets
  if (a.page_bytes > 0x7FFF0000ull) return kUnsupported;
  a.num_seqs = num_seqs;
  switch (head_dim) {
    case 64: return launch_stream_nc<FMT, 64, CONTIG>(a, stream);
    case 128: return launch_stream_nc<FMT, 128, CONTIG>(a, stream);
    case 256: return launch_stream_nc<FMT, 256, CONTIG>(a, stream);
    case 512: return launch_stream_nc<FMT, 512, CONTIG>(a, stream);
    default: return kUnsupported;
  }
}

static DecodeArgs make_args(const uint16_t* q, const void* kc, const void* vc, float* ws,
                            const int32_t* bt, const int32_t* lens, uint32_t max_blocks,
                            uint32_t Hq, uint32_t Hkv, uint32_t bs, float logit_scale,
                            float out_scale, uint32_t S, uint32_t q_stride, uint64_t page_bytes,
                            uint64_t data_section, uint32_t window, uint32_t head_dim) {
  DecodeArgs a;
  a.q = q;
  a.k_cache = static_cast<const uint8_t*>(kc);
  a.v_cache = static_cast<const uint8_t*>(vc);
  a.ws = ws;
  a.block_tables = bt;
  a.seq_lens = lens;
  a.max_blocks = max_blocks;
  a.num_q_heads = Hq;
  a.num_kv_heads = Hkv;
  a.group = Hq / Hkv;
  a.col_chunks = head_chunks(a.group);
  a.head_chunks = a.col_chunks;
  a.block_size = bs;
  a.logit_scale = logit_scale;
  a.out_scale = out_scale;
  a.num_splits = S;
  a.q_stride = q_stride;
  a.page_bytes = page_bytes;
  a.data_section = data_section;
  a.window = window;
  a.num_seqs = 0;
  a.chunk_min = 1;
  a.row_lead = 0;
  a.max_len = uint32_t(min(uint64_t(max_blocks) * bs, uint64_t(0x7FFFFFFF)));
  a.static_q = 0;
  a.head_group = 1;
  a.out = nullptr;
  a.new_k = nullptr;
  a.new_v = nullptr;
  a.new_k_stride = 0;
  a.new_v_stride = 0;
  a.enc_k_scale = 1.0f;
  a.enc_v_scale = 1.0f;
  a.q_len = 1;
  a.q_tok_stride = 0;
  a.causal = 0;
  a.q_window = window;
  a.q_head_stride = head_dim;
  a.o_head = head_dim;                        // output [B][q_len][Hq][D], contiguous
  a.o_tok = uint64_t(Hq) * head_dim;
  a.o_seq = a.o_tok;
  for (int i = 0; i < 3; ++i) a.k_strides[i] = a.v_strides[i] = 0;
  return a;
}

template <int D, int CW>
static void launch_reduce_cols(uint64_t rows, size_t lds, const float* workspace,
                               uint16_t* output, const int32_t* seq_lens, const OutMap& om,
                               uint32_t num_splits, hipStream_t stream) {
  constexpr int NT = CW == 1 ? 1024 : 256;
  hipLaunchKernelGGL((reduce_kernel<D, NT, CW>), dim3(uint32_t(rows * CW)), dim3(NT), lds, stream,
                     workspace, output, seq_lens, om, num_splits);
}

template <int D>
static void launch_reduce_d(uint64_t rows, uint32_t cw, const float* workspace, uint16_t* output,
                            const int32_t* seq_lens, const OutMap& om, uint32_t num_splits,
                            hipStream_t stream) {
  if (cw == 1 && num_splits <= 64) {           // one wave per (b, h), registers only
    hipLaunchKernelGGL((reduce_wave_kernel<D>), dim3(uint32_t(rows)), dim3(64), 0, stream,
                       workspace, output, seq_lens, om, num_splits);
    return;
  }
  const size_t lds = 2 * size_t(num_splits) * sizeof(float);
  switch (cw) {
    case 1: launch_reduce_cols<D, 1>(rows, lds, workspace, output, seq_lens, om, num_splits, stream); break;
    case 2: if constexpr (D >= 64) launch_reduce_cols<D, 2>(rows, lds, workspace, output, seq_lens, om, num_splits, stream); break;
    case 4: if constexpr (D >= 128) launch_reduce_cols<D, 4>(rows, lds, workspace, output, seq_lens, om, num_splits, stream); break;
    case 8: if constexpr (D >= 256) launch_reduce_cols<D, 8>(rows, lds, workspace, output, seq_lens, om, num_splits, stream); break;
    case 16: if constexpr (D >= 512) launch_reduce_cols<D, 16>(rows, lds, workspace, output, seq_lens, om, num_splits, stream); break;
  }
}

// Rows of the combine are (sequence, q head) pairs. Few rows (a small batch)
// leave most CUs idle, so each row's columns are split over CW workgroups:
// the largest power of two up to D / 32 with rows * CW <= 256 (by default).
// Each of them reads every slot's (m, l), which is why CW stays 1 for many
// rows.
static int launch_reduce(const float* workspace, uint16_t* output, const int32_t* seq_lens,
                         const OutMap& om, uint32_t head_dim, uint32_t num_splits,
                         uint32_t num_seqs, hipStream_t stream) {
  const uint64_t rows = uint64_t(num_seqs) * om.per_seq;
  if (rows > 0x7FFFFFFFull / 16) return kUnsupported;
  uint32_t cw = 1;
  while (cw * 2 <= head_dim / 32 && rows * cw * 2 <= PKD_COMBINE_MAX_WG) cw *= 2;
  switch (head_dim) {
    case 64: launch_reduce_d<64>(rows, cw, workspace, output, seq_lens, om, num_splits, stream); break;
    case 128: launch_reduce_d<128>(rows, cw, workspace, output, seq_lens, om, num_splits, stream); break;
    case 256: launch_reduce_d<256>(rows, cw, workspace, output, seq_lens, om, num_splits, stream); break;
    case 512: launch_reduce_d<512>(rows, cw, workspace, output, seq_lens, om, num_splits, stream); break;
    default: return kUnsupported;
  }
  return launch_status();
}

// Rows of at most this many 16-key tiles (by the block-table width, or the
// window) are decoded in one launch whatever the split count.
#ifndef PKD_ONE_LAUNCH_TILES
#define PKD_ONE_LAUNCH_TILES 12
#endif

// Whether a decode (one query token) runs faster as the one-launch form:
// one workgroup of interleaving waves per row, merging in LDS, where the
// rows are short and all of them are resident at once. The split pass and
// the combine are two launches of a few dependent round trips each; at one
// sequence of 8 kv heads they take 7.6 us at 128 keys, the one-launch form
// 6.2 us, and the two are even at 256 keys (0.8 us per further tile of a
// wave).
template <int FMT, int D, bool CONTIG>
static bool one_launch_fits(const DecodeArgs& a, uint32_t num_seqs) {
  if constexpr (kMergeWaves<FMT, D, 1> > 1) {
    constexpr int wi = kMergeWaves<FMT, D, 1>;
    if (a.q_len != 1 || a.col_chunks != 1) return false;
    uint64_t tile_bound = uint64_t(a.max_blocks) * (a.block_size / 16);
    if (a.window > 0) tile_bound = min(tile_bound, uint64_t((a.window + 14) / 16 + 1));
    const uint64_t rows = uint64_t(num_seqs) * a.num_kv_heads;
    const uint64_t resident = stream_capacity<FMT, D, 1, CONTIG, wi>() / kGroupWaves<FMT, D, wi>;
    return tile_bound <= PKD_ONE_LAUNCH_TILES && rows <= resident;
  }
  return false;
}

// Non-split decode (num_splits 1), or a decode of short rows: one workgroup
// per row writes the output. Otherwise the split-K pass and the combine, as
// two launches.
template <int FMT, bool CONTIG = false>
static int launch_decode(DecodeArgs a, uint16_t* output, uint32_t num_seqs, uint32_t head_dim,
                         hipStream_t stream) {
  bool one = a.num_splits == 1;
  if (!one) {
    switch (head_dim) {
      case 64: one = one_launch_fits<FMT, 64, CONTIG>(a, num_seqs); break;
      case 128: one = one_launch_fits<FMT, 128, CONTIG>(a, num_seqs); break;
      case 256: one = one_launch_fits<FMT, 256, CONTIG>(a, num_seqs); break;
      default: break;
    }
  }
  if (!one) {
    const int st = launch_splitk<FMT, CONTIG>(a, num_seqs, head_dim, stream);
    if (st) return st;
    const OutMap om = {a.o_seq, a.o_tok, a.o_head, a.num_q_heads * a.q_len, a.num_q_heads};
    return launch_reduce(a.ws, output, a.seq_lens, om, head_dim, a.num_splits, num_seqs, stream);
  }
  a.out = output;
  a.num_splits = 1;
  return launch_splitk<FMT, CONTIG>(a, num_seqs, head_dim, stream);
}

}  // namespace pkd

using namespace pkd;

extern "C" PKD_API int paged_decode_attn_splitk_bf16(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, float* workspace,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim, uint32_t block_size,
    float scale, uint32_t num_splits, uint32_t q_stride, uint32_t num_seqs,
    uint32_t sliding_window, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_decode(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  const uint64_t page_bytes = uint64_t(block_size) * num_kv_heads * head_dim * 2;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, page_bytes, 0,
                           sliding_window, head_dim);
  return launch_splitk<kBf16>(a, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_splitk_fp8(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, float* workspace,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim, uint32_t block_size,
    float scale, uint32_t num_splits, float k_scale, float v_scale, uint32_t q_stride,
    uint64_t cache_stride, uint32_t num_seqs, uint32_t sliding_window, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_decode(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_fp8_stride(num_kv_heads, head_dim, block_size, cache_stride);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * k_scale * kLog2e, v_scale, num_splits, q_stride, cache_stride,
                           0, sliding_window, head_dim);
  return launch_splitk<kFp8>(a, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_splitk_nvfp4(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, float* workspace,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim, uint32_t block_size,
    float scale, uint32_t num_splits, uint32_t q_stride, uint64_t block_stride_bytes,
    uint64_t data_section_bytes, uint32_t num_seqs, uint32_t sliding_window,
    hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_decode(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_nvfp4_sections(num_kv_heads, head_dim, block_size, block_stride_bytes,
                            data_section_bytes);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, block_stride_bytes,
                           data_section_bytes, sliding_window, head_dim);
  return launch_splitk<kNvfp4>(a, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_splitk_append_bf16(
    const uint16_t* q, const uint16_t* key, const uint16_t* value, uint16_t* k_cache,
    uint16_t* v_cache, float* workspace, const int32_t* block_tables, const int32_t* seq_lens,
    uint32_t max_blocks_per_seq, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t num_splits, uint32_t q_stride, uint32_t key_stride,
    uint32_t value_stride, uint32_t num_seqs, uint32_t sliding_window, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_decode(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_append(key, value, num_kv_heads, head_dim, key_stride, value_stride);
  if (st) return st;
  const uint64_t page_bytes = uint64_t(block_size) * num_kv_heads * head_dim * 2;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, page_bytes, 0,
                           sliding_window, head_dim);
  a.new_k = key; a.new_v = value; a.new_k_stride = key_stride; a.new_v_stride = value_stride;
  return launch_splitk<kBf16>(a, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_splitk_append_fp8(
    const uint16_t* q, const uint16_t* key, const uint16_t* value, uint8_t* k_cache,
    uint8_t* v_cache, float* workspace, const int32_t* block_tables, const int32_t* seq_lens,
    uint32_t max_blocks_per_seq, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t num_splits, float k_scale, float v_scale,
    uint32_t q_stride, uint32_t key_stride, uint32_t value_stride, uint64_t cache_stride,
    uint32_t num_seqs, uint32_t sliding_window, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_decode(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_fp8_stride(num_kv_heads, head_dim, block_size, cache_stride);
  if (st) return st;
  st = check_append(key, value, num_kv_heads, head_dim, key_stride, value_stride);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * k_scale * kLog2e, v_scale, num_splits, q_stride, cache_stride,
                           0, sliding_window, head_dim);
  a.new_k = key; a.new_v = value; a.new_k_stride = key_stride; a.new_v_stride = value_stride;
  a.enc_k_scale = k_scale; a.enc_v_scale = v_scale;
  return launch_splitk<kFp8>(a, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_splitk_append_nvfp4(
    const uint16_t* q, const uint16_t* key, const uint16_t* value, uint8_t* k_cache,
    uint8_t* v_cache, float* workspace, const int32_t* block_tables, const int32_t* seq_lens,
    uint32_t max_blocks_per_seq, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t num_splits, uint32_t q_stride, uint32_t key_stride,
    uint32_t value_stride, uint64_t block_stride_bytes, uint64_t data_section_bytes,
    uint32_t num_seqs, uint32_t sliding_window, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_decode(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_nvfp4_sections(num_kv_heads, head_dim, block_size, block_stride_bytes,
                            data_section_bytes);
  if (st) return st;
  st = check_append(key, value, num_kv_heads, head_dim, key_stride, value_stride);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, block_stride_bytes,
                           data_section_bytes, sliding_window, head_dim);
  a.new_k = key; a.new_v = value; a.new_k_stride = key_stride; a.new_v_stride = value_stride;
  return launch_splitk<kNvfp4>(a, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_bf16(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* output,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_seqs, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t q_stride, uint32_t sliding_window,
    float* workspace, uint32_t num_splits, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_single(q, k_cache, v_cache, output, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  const uint64_t page_bytes = uint64_t(block_size) * num_kv_heads * head_dim * 2;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, page_bytes, 0,
                           sliding_window, head_dim);
  return launch_decode<kBf16>(a, output, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_fp8(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, uint16_t* output,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_seqs, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, float k_scale, float v_scale, uint32_t q_stride,
    uint64_t cache_stride, uint32_t sliding_window, float* workspace, uint32_t num_splits,
    hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_single(q, k_cache, v_cache, output, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_fp8_stride(num_kv_heads, head_dim, block_size, cache_stride);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * k_scale * kLog2e, v_scale, num_splits, q_stride, cache_stride,
                           0, sliding_window, head_dim);
  return launch_decode<kFp8>(a, output, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_nvfp4(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, uint16_t* output,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_seqs, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t q_stride, uint64_t block_stride_bytes,
    uint64_t data_section_bytes, uint32_t sliding_window, float* workspace, uint32_t num_splits,
    hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_single(q, k_cache, v_cache, output, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_nvfp4_sections(num_kv_heads, head_dim, block_size, block_stride_bytes,
                            data_section_bytes);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, block_stride_bytes,
                           data_section_bytes, sliding_window, head_dim);
  return launch_decode<kNvfp4>(a, output, num_seqs, head_dim, stream);
}

// ---------------------------------------------------------------------------
// The BF16 whole decode without a caller workspace. The split-K partials go
// to `scratch`, a file-scope device array of kScratchBytes that every GPU the
// library runs on holds until the process ends. In host code the array's
// name stands for a host-side shadow, not device memory: its device address
// comes from hipGetSymbolAddress, taken once per device (with that device
// current) on the first call there, and only that address reaches the
// kernels. Calls on one GPU share the array; calls that overlap on one GPU
// (different streams) race. The split-K pass leaves no requirement on the
// array's contents (the combine reads only slots written in the same call),
// so nothing is cleared.
constexpr size_t kScratchBytes = PKD_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

static float* scratch_on_device(int& status) {
  static std::once_flag once[64];
  static float* ptr[64];
  static hipError_t err[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    status = kLaunch;
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    ptr[dev] = static_cast<float*>(p);
  });
  if (err[dev] != hipSuccess || ptr[dev] == nullptr) {
    status = kLaunch;
    return nullptr;
  }
  return ptr[dev];
}

extern "C" PKD_API int paged_decode_attn_bf16_noalloc(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* output,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_seqs, uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim,
    uint32_t block_size, float scale, uint32_t q_stride, uint32_t sliding_window,
    uint32_t num_splits, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  // the checks of the whole decode, the scratch standing in for the workspace
  static const uint64_t kAligned = 16;
  int st = check_single(q, k_cache, v_cache, output, reinterpret_cast<const void*>(kAligned),
                        block_tables, seq_lens, max_blocks_per_seq, num_q_heads, num_kv_heads,
                        head_dim, block_size, num_splits, q_stride);
  if (st) return st;
  float* ws = nullptr;
  if (num_splits > 1) {
    const uint64_t rows = uint64_t(num_seqs) * num_q_heads;     // both factors < 2^32
    if (rows > kScratchBytes ||
        rows * num_splits * (uint64_t(head_dim) + 2) * sizeof(float) > kScratchBytes)
      return kScratch;
    ws = scratch_on_device(st);
    if (!ws) return st;
  }
  const uint64_t page_bytes = uint64_t(block_size) * num_kv_heads * head_dim * 2;
  DecodeArgs a = make_args(q, k_cache, v_cache, ws, block_tables, seq_lens, max_blocks_per_seq,
                           num_q_heads, num_kv_heads, block_size, scale * kLog2e, 1.0f,
                           num_splits, q_stride, page_bytes, 0, sliding_window, head_dim);
  return launch_decode<kBf16>(a, output, num_seqs, head_dim, stream);
}

// Query-block arguments on top of the decode arguments: column chunks over
// the group's q_len x group columns, the row window widened for a causal
// window (the first token's keys through the last token's).
static void set_query_block(DecodeArgs& a, uint32_t q_len, uint32_t q_token_stride,
                            uint32_t causal, uint32_t sliding_window) {
  a.q_len = q_len;
  a.q_tok_stride = q_token_stride;
  a.causal = causal ? 1u : 0u;
  a.q_window = sliding_window;
  a.window = prefill_row_window(q_len, a.causal, sliding_window);
  a.col_chunks = head_chunks(a.group * q_len);
  a.o_seq = uint64_t(q_len) * a.o_tok;
}

extern "C" PKD_API int paged_prefill_attn_bf16(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* output,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_seqs, uint32_t q_len, uint32_t num_q_heads, uint32_t num_kv_heads,
    uint32_t head_dim, uint32_t block_size, float scale, uint32_t q_stride,
    uint32_t q_token_stride, uint32_t causal, uint32_t sliding_window, float* workspace,
    uint32_t num_splits, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_single(q, k_cache, v_cache, output, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_prefill(q_len, num_q_heads, head_dim, q_stride, q_token_stride);
  if (st) return st;
  const uint64_t page_bytes = uint64_t(block_size) * num_kv_heads * head_dim * 2;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, page_bytes, 0,
                           sliding_window, head_dim);
  set_query_block(a, q_len, q_token_stride, causal, sliding_window);
  return launch_decode<kBf16>(a, output, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_prefill_attn_fp8(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, uint16_t* output,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_seqs, uint32_t q_len, uint32_t num_q_heads, uint32_t num_kv_heads,
    uint32_t head_dim, uint32_t block_size, float scale, float k_scale, float v_scale,
    uint32_t q_stride, uint32_t q_token_stride, uint64_t cache_stride, uint32_t causal,
    uint32_t sliding_window, float* workspace, uint32_t num_splits, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_single(q, k_cache, v_cache, output, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_prefill(q_len, num_q_heads, head_dim, q_stride, q_token_stride);
  if (st) return st;
  st = check_fp8_stride(num_kv_heads, head_dim, block_size, cache_stride);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * k_scale * kLog2e, v_scale, num_splits, q_stride, cache_stride,
                           0, sliding_window, head_dim);
  set_query_block(a, q_len, q_token_stride, causal, sliding_window);
  return launch_decode<kFp8>(a, output, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_prefill_attn_nvfp4(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, uint16_t* output,
    const int32_t* block_tables, const int32_t* seq_lens, uint32_t max_blocks_per_seq,
    uint32_t num_seqs, uint32_t q_len, uint32_t num_q_heads, uint32_t num_kv_heads,
    uint32_t head_dim, uint32_t block_size, float scale, uint32_t q_stride,
    uint32_t q_token_stride, uint64_t block_stride_bytes, uint64_t data_section_bytes,
    uint32_t causal, uint32_t sliding_window, float* workspace, uint32_t num_splits,
    hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_single(q, k_cache, v_cache, output, workspace, block_tables, seq_lens,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_splits, q_stride);
  if (st) return st;
  st = check_prefill(q_len, num_q_heads, head_dim, q_stride, q_token_stride);
  if (st) return st;
  st = check_nvfp4_sections(num_kv_heads, head_dim, block_size, block_stride_bytes,
                            data_section_bytes);
  if (st) return st;
  DecodeArgs a = make_args(q, k_cache, v_cache, workspace, block_tables, seq_lens,
                           max_blocks_per_seq, num_q_heads, num_kv_heads, block_size,
                           scale * kLog2e, 1.0f, num_splits, q_stride, block_stride_bytes,
                           data_section_bytes, sliding_window, head_dim);
  set_query_block(a, q_len, q_token_stride, causal, sliding_window);
  return launch_decode<kNvfp4>(a, output, num_seqs, head_dim, stream);
}

// Contiguous K/V: 16-key tiles addressed through the caller's strides; the
// tile bound comes from max_seq_len. Strides: q (seq, token, head), k, v,
// output, in elements.
template <int FMT>
static int contig_attn(const uint16_t* q, const void* k, const void* v, uint16_t* output,
                       const int32_t* seq_lens, uint32_t num_seqs, uint32_t q_len,
                       uint32_t max_seq_len, uint32_t num_q_heads, uint32_t num_kv_heads,
                       uint32_t head_dim, float logit_scale, float out_scale,
                       const uint64_t* strides, uint32_t causal, uint32_t sliding_window,
                       float* workspace, uint32_t num_splits, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  const uint32_t esize = FMT == kBf16 ? 2 : 1;
  int st = check_contig(q, k, v, output, workspace, seq_lens, strides, num_seqs, q_len,
                        max_seq_len, num_q_heads, num_kv_heads, head_dim, esize, num_splits);
  if (st) return st;
  DecodeArgs a = make_args(q, k, v, workspace, nullptr, seq_lens, (max_seq_len + 15) / 16,
                           num_q_heads, num_kv_heads, 16, logit_scale, out_scale, num_splits,
                           uint32_t(strides[0]), 0, 0, sliding_window, head_dim);
  set_query_block(a, q_len, uint32_t(strides[1]), causal, sliding_window);
  a.max_len = max_seq_len;
  a.q_head_stride = uint32_t(strides[2]);
  for (int i = 0; i < 3; ++i) {
    a.k_strides[i] = strides[3 + i] * esize;
    a.v_strides[i] = strides[6 + i] * esize;
  }
  a.o_seq = strides[9];
  a.o_tok = strides[10];
  a.o_head = strides[11];
  return launch_decode<FMT, true>(a, output, num_seqs, head_dim, stream);
}

extern "C" PKD_API int contig_kv_attn_bf16(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* output,
    const int32_t* seq_lens, uint32_t num_seqs, uint32_t q_len, uint32_t max_seq_len,
    uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim, float scale,
    const uint64_t* strides, uint32_t causal, uint32_t sliding_window, float* workspace,
    uint32_t num_splits, hipStream_t stream) {
  return contig_attn<kBf16>(q, k, v, output, seq_lens, num_seqs, q_len, max_seq_len,
                            num_q_heads, num_kv_heads, head_dim, scale * kLog2e, 1.0f, strides,
                            causal, sliding_window, workspace, num_splits, stream);
}

extern "C" PKD_API int contig_kv_attn_fp8(
    const uint16_t* q, const uint8_t* k, const uint8_t* v, uint16_t* output,
    const int32_t* seq_lens, uint32_t num_seqs, uint32_t q_len, uint32_t max_seq_len,
    uint32_t num_q_heads, uint32_t num_kv_heads, uint32_t head_dim, float scale, float k_scale,
    float v_scale, const uint64_t* strides, uint32_t causal, uint32_t sliding_window,
    float* workspace, uint32_t num_splits, hipStream_t stream) {
  return contig_attn<kFp8>(q, k, v, output, seq_lens, num_seqs, q_len, max_seq_len, num_q_heads,
                           num_kv_heads, head_dim, scale * k_scale * kLog2e, v_scale, strides,
                           causal, sliding_window, workspace, num_splits, stream);
}

extern "C" PKD_API uint32_t paged_prefill_num_splits(uint32_t num_seqs, uint32_t q_len,
                                                     uint32_t num_q_heads, uint32_t num_kv_heads,
                                                     uint32_t max_blocks_per_seq,
                                                     uint32_t block_size, uint32_t causal,
                                                     uint32_t sliding_window, uint32_t num_cus) {
  if (q_len == 0 || q_len > kMaxQueryLen || uint64_t(num_q_heads) * q_len > 0x7FFFFFFFull)
    return 1;
  return prefill_num_splits(num_seqs, q_len, num_q_heads, num_kv_heads, max_blocks_per_seq,
                            block_size, prefill_row_window(q_len, causal, sliding_window),
                            num_cus);
}

extern "C" PKD_API int paged_decode_attn_reduce(const float* workspace, uint16_t* output,
                                                const int32_t* seq_lens, uint32_t num_q_heads,
                                                uint32_t head_dim, uint32_t num_splits,
                                                uint32_t num_seqs, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_reduce(workspace, output, seq_lens, num_q_heads, head_dim, num_splits);
  if (st) return st;
  const OutMap om = {uint64_t(num_q_heads) * head_dim, 0, head_dim, num_q_heads, num_q_heads};
  return launch_reduce(workspace, output, seq_lens, om, head_dim, num_splits, num_seqs, stream);
}

extern "C" PKD_API size_t paged_decode_workspace_bytes(uint32_t num_seqs, uint32_t num_q_heads,
                                                       uint32_t head_dim, uint32_t num_splits) {
  return workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits);
}

extern "C" PKD_API uint32_t paged_decode_num_splits(uint32_t num_seqs, uint32_t num_q_heads,
                                                    uint32_t num_kv_heads,
                                                    uint32_t max_blocks_per_seq,
                                                    uint32_t block_size, uint32_t sliding_window,
                                                    uint32_t num_cus) {
  return num_splits_heuristic(num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq,
                              block_size, sliding_window, num_cus);
}

extern "C" PKD_API const char* pkd_status_string(int status) {
  switch (status) {
    case kOk: return "ok";
    case kInvalid: return "invalid argument";
    case kUnsupported: return "unsupported shape";
    case kLaunch: return "kernel launch failed";
    case kScratch: return "workspace larger than the static scratch";
    default: return "unknown status";
  }
}
