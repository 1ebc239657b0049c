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
// Work unit: one wavefront per (sequence, kv head, chunk of up to 16 q heads
// of that kv head's group, split). All q heads sharing a kv head are served by
// the one pass over its pages, so each K/V byte leaves HBM once per step.
//
// Per 16-token tile (a page holds block_size/16 tiles):
//  * K tile -> MFMA A operand straight from 16-byte global loads: lane l owns
//    token l%16 and a contiguous run of E elements of its row per load
//    (lane group g = l/16 takes the g-th run of every 4E-element stripe).
//    FP8 / NVFP4 codes are dequantized to BF16 in registers (exact).
//  * S = K . Q^T on v_mfma_f32_16x16x32_bf16 (M = tokens, N = q heads, K =
//    head_dim; q heads beyond the group are zero columns).
//  * Online softmax in fp32 on the MFMA output layout (lane l: head l%16,
//    tokens 4g..4g+3), exp2 with log2(e) folded into the logit scale.
//  * V tile -> BF16 rows in LDS (masked tokens written as zeros), read back
//    transposed as the A operand of v_mfma_f32_16x16x16_bf16 computing
//    O^T[dim][head] += V^T . P, P rounded to BF16 in registers.
#include "../../include/pkd.h"
#include "device_common.hpp"
#include "validate.hpp"

namespace pkd {

enum Fmt { kBf16 = 0, kFp8 = 1, kNvfp4 = 2 };

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
  uint32_t head_chunks;    // ceil(group / 16)
  uint32_t block_size;
  float logit_scale;       // scale * log2(e) (* k_scale for FP8)
  float out_scale;         // v_scale for FP8, 1 otherwise
  uint32_t num_splits;
  uint32_t pages_per_split;
  uint32_t q_stride;
  uint64_t page_bytes;     // bytes per page of one pool
  uint64_t data_section;   // NVFP4: byte offset of the scales within a page
  uint32_t window;
  uint32_t num_seqs;
  uint32_t chunk_min;      // stream partition: least tiles per wave (S - 1 pieces per row at most)
};

template <int FMT, int D>
struct Traits {
  // elements of one row a lane loads per instruction (at most 16 bytes)
  static constexpr int kElemBits = FMT == kBf16 ? 16 : (FMT == kFp8 ? 8 : 4);
  static constexpr int kE0 = 128 / kElemBits;               // 16 bytes worth
  static constexpr int E = kE0 < D / 4 ? kE0 : D / 4;
  static constexpr int kLoadBytes = E * kElemBits / 8;      // 16 or 8
  static constexpr int NLOAD = D / (4 * E);                 // loads per tile per lane
  static constexpr int MPER = E / 8;                        // bf16x8 fragments per load
  static constexpr int NFRAG = D / 32;                      // QK MFMAs per tile
  static constexpr int RS = D + 16;                         // LDS row stride (elements)
  static constexpr int ROW_BYTES = D * kElemBits / 8;       // bytes of one (token, head) row
  // tiles in flight per wave: about 128 VGPRs of raw K+V bytes, 1 to 4 tiles
  static constexpr int kTileRegs = 2 * NLOAD * (kLoadBytes / 4 + (FMT == kNvfp4 ? 1 : 0));
  static constexpr int kRing = 128 / kTileRegs;
  static constexpr int NBUF = kRing < 1 ? 1 : (kRing > 4 ? 4 : kRing);
};

// Raw bytes of one lane's share of a K or V tile.
template <int FMT, int D>
struct RawTile {
  u32x4 d[Traits<FMT, D>::NLOAD];
  uint32_t s[Traits<FMT, D>::NLOAD];     // NVFP4 group-scale bytes
};

// Loads one lane's share of a K or V tile with buffer instructions. The
// descriptor covers one page; live == false gives it zero records, so the
// loads return zeros without touching memory (phantom tiles past the end of a
// split keep the loop's load count uniform).
template <int FMT, int D>
__device__ __forceinline__ void load_tile(RawTile<FMT, D>& t, const uint8_t* pool,
                                          const DecodeArgs& a, uint32_t phys, bool live,
                                          uint32_t off, uint32_t kvh, int g) {
  using T = Traits<FMT, D>;
  const uint8_t* page = pool + uint64_t(phys) * a.page_bytes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(page), 0, live ? int(a.page_bytes) : 0, 0x00020000);
  const uint32_t rowidx = off * a.num_kv_heads + kvh;               // (offset, head) row
#pragma unroll
  for (int r = 0; r < T::NLOAD; ++r) {
    const int e0 = r * 4 * T::E + g * T::E;                        // first element
    const int voff = int(rowidx * T::ROW_BYTES + (e0 * T::kElemBits) / 8);
    if constexpr (T::kLoadBytes == 16) {
      t.d[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, 0, 2));
    } else {
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, 0, 2));
      t.d[r][0] = v[0];
      t.d[r][1] = v[1];
    }
    if constexpr (FMT == kNvfp4) {
      const int soff = int(a.data_section) + int(rowidx * (D / 16) + e0 / 16);
      if constexpr (T::E == 32) t.s[r] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, soff, 0, 2);
      else t.s[r] = __builtin_amdgcn_raw_buffer_load_b8(rsrc, soff, 0, 2);
    }
  }
}

// Two FP8-E4M3FN codes (bytes `hi` selects 0/1 or 2/3 of w) -> packed BF16 pair.
// gfx950 converts E4M3FN exactly; every value fits BF16.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  return pack_bf16x2(f[0], f[1]);
}

// Two E2M1 codes (byte `sel` of w) times scale S -> packed BF16 pair (exact).
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, int sel, float S) {
  f32x2 f;
  switch (sel) {
    case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
    case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
    case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
    default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
  }
  return pack_bf16x2(f[0] * S, f[1] * S);
}

// Fragment f (8 consecutive elements) of a lane's load r, as BF16.
template <int FMT, int D>
__device__ __forceinline__ bf16x8 dequant_frag(const RawTile<FMT, D>& t, int r, int f) {
  if constexpr (FMT == kBf16) {
    return __builtin_bit_cast(bf16x8, t.d[r]);
  } else if constexpr (FMT == kFp8) {
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t word = t.d[r][2 * f + w];
      out[2 * w] = fp8x2_to_bf16x2<false>(word);
      out[2 * w + 1] = fp8x2_to_bf16x2<true>(word);
    }
    return __builtin_bit_cast(bf16x8, out);
  } else {
    // 8 codes = one 32-bit word; group scale = byte f/2 of the lane's scales
    const uint32_t word = t.d[r][f];
    const float S = (f >> 1) ? __builtin_amdgcn_cvt_f32_fp8(t.s[r], 1)
                             : __builtin_amdgcn_cvt_f32_fp8(t.s[r], 0);
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = fp4x2_to_bf16x2(word, i, S);
    return __builtin_bit_cast(bf16x8, out);
  }
}

// Orders this wave's LDS accesses around the V transpose for the compiler; a
// wave's LDS operations execute in issue order, so no wait is needed.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int FMT, int D>
__global__ __launch_bounds__(64) void splitk_kernel(DecodeArgs a) {
  using T = Traits<FMT, D>;
  constexpr int NBUF = T::NBUF;
  const int lane = threadIdx.x;
  const int g = lane >> 4;          // lane group: k-run for loads, token quad for outputs
  const int n = lane & 15;          // head column / token row / dim column

  uint32_t wg = blockIdx.x;
  const uint32_t split = wg % a.num_splits;
  wg /= a.num_splits;
  const uint32_t hc = wg % a.head_chunks;
  wg /= a.head_chunks;
  const uint32_t kvh = wg % a.num_kv_heads;
  const uint32_t b = wg / a.num_kv_heads;

  const int32_t Ls = a.seq_lens[b];
  const uint32_t L = Ls > 0 ? uint32_t(Ls) : 0u;
  const uint32_t lo = (a.window > 0 && L > a.window) ? L - a.window : 0u;
  const uint32_t bs = a.block_size;
  const uint32_t p0 = lo / bs, pend = (L + bs - 1) / bs;
  const uint32_t pa = p0 + split * a.pages_per_split;
  const uint32_t pb = min(pa + a.pages_per_split, pend);

  const uint32_t head_in_group = hc * 16 + n;
  const bool head_ok = head_in_group < a.group;
  const uint32_t qh = kvh * a.group + head_in_group;        // q head of this lane's column
  float* wrow = a.ws + ((uint64_t(b) * a.num_q_heads + qh) * a.num_splits + split) * (D + 2);

  if (pa >= pb) {                                           // empty split
    if (head_ok) {
      for (int d = g; d < D + 2; d += 4)
        wrow[d] = d == D ? -__builtin_inff() : 0.0f;
    }
    return;
  }

  const uint32_t tpp = bs / 16;                              // tiles per page
  const uint32_t t0 = max(pa * tpp, lo / 16);
  const uint32_t t1 = min(pb * tpp, (L + 15) / 16);
  const int32_t* bt = a.block_tables + uint64_t(b) * a.max_blocks;

  // q as the B operand of the QK MFMAs: column n = head, k-run of group g.
  bf16x8 qf[T::NFRAG];
  {
    const uint16_t* qrow = a.q + uint64_t(b) * a.q_stride + uint64_t(qh) * D;
#pragma unroll
    for (int c = 0; c < T::NFRAG; ++c) {
      const int r = c / T::MPER, f = c % T::MPER;
      const int e0 = r * 4 * T::E + g * T::E + 8 * f;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head_ok) v = *reinterpret_cast<const u32x4*>(qrow + e0);
      qf[c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  __shared__ __attribute__((aligned(16))) uint16_t vlds[16 * T::RS];
  // transposed-read address of this lane: row 4g + n/4, column 4*(n%4) (+16 per M tile)
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  lds_u16* const tr_base = (lds_u16*)(vlds) + (4 * g + (n >> 2)) * T::RS + 4 * (n & 3);

  f32x4 acc[D / 16];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  RawTile<FMT, D> kb[NBUF], vb[NBUF];

  // Pages in chunks of 64 (one block-table entry per lane); within a chunk the
  // NBUF-deep register ring keeps NBUF tiles of K and V in flight.
  for (uint32_t cp = pa; cp < pb; cp += 64) {
    const uint32_t cpe = min(cp + 64, pb);
    const int32_t bt_reg = (cp + lane < cpe) ? bt[cp + lane] : 0;
    const uint32_t ct0 = max(cp * tpp, t0);
    const uint32_t ct1 = min(cpe * tpp, t1);
    auto issue = [&](RawTile<FMT, D>& dst, const uint8_t* pool, uint32_t t) {
      const bool live = t < ct1;
      const uint32_t page = min(t / tpp, cpe - 1);
      const uint32_t phys = uint32_t(__builtin_amdgcn_readlane(bt_reg, int(page - cp)));
      load_tile<FMT, D>(dst, pool, a, phys, live, (t % tpp) * 16 + n, kvh, g);
    };
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      issue(kb[s], a.k_cache, ct0 + s);
      issue(vb[s], a.v_cache, ct0 + s);
    }

    for (uint32_t tb = ct0; tb < ct1; tb += NBUF) {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        const uint32_t t = tb + s;                 // t >= ct1: phantom tile, all keys masked
        const uint32_t tok0 = t * 16;
        const uint32_t klo = lo, khi = t < ct1 ? L : 0u;

        // ---- S = K Q^T, then the slot's K registers take the tile NBUF ahead
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < T::NFRAG; ++c) {
          const bf16x8 kf = dequant_frag<FMT, D>(kb[s], c / T::MPER, c % T::MPER);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sc, 0, 0, 0);
        }
        // the refill reuses the slot's registers only if it stays after their last use
        __builtin_amdgcn_sched_barrier(0);
        issue(kb[s], a.k_cache, t + NBUF);

        // ---- V tile -> LDS rows (token n of the tile), masked tokens as zeros
        {
          const uint32_t tok = tok0 + n;
          const bool ok = tok >= klo && tok < khi;
          uint16_t* dst = vlds + n * T::RS;
#pragma unroll
          for (int r = 0; r < T::NLOAD; ++r) {
#pragma unroll
            for (int f = 0; f < T::MPER; ++f) {
              u32x4 v = __builtin_bit_cast(u32x4, dequant_frag<FMT, D>(vb[s], r, f));
              if (!ok) v = u32x4{0u, 0u, 0u, 0u};
              *reinterpret_cast<u32x4*>(dst + r * 4 * T::E + g * T::E + 8 * f) = v;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(vb[s], a.v_cache, t + NBUF);

        // ---- online softmax (lane: head n, tokens tok0 + 4g + j)
        float sv[4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t tok = tok0 + 4 * g + j;
          sv[j] = (tok >= klo && tok < khi) ? sc[j] * a.logit_scale : -__builtin_inff();
          mx = fmaxf(mx, sv[j]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // finite: the first tile of a split holds a key, phantom tiles come after it
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        uint32_t pbits[4];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(sv[j] - m_new);
          pbits[j] = f32_to_bf16_bits(p);
          psum += __uint_as_float(pbits[j] << 16);
        }
        l_run = l_run * alpha + psum;
        s16x4 pf;
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[j] = short(pbits[j]);

        wave_lds_fence();
        // ---- O^T += V^T P  (A: V^T rows = dims of M tile mt, k = tokens 4g..4g+3)
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
          const bf16x4 vt =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tr_base + mt * 16));
          f32x4 c = acc[mt] * alpha;
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vt), pf,
                                                              c, 0, 0, 0);
        }
        wave_lds_fence();
      }
    }
  }

  // ---- partial state out: o = acc / l, m in natural-log units
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (head_ok) {
    const float inv = a.out_scale / l_tot;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      f32x2 lo2 = {acc[mt][0] * inv, acc[mt][1] * inv};
      f32x2 hi2 = {acc[mt][2] * inv, acc[mt][3] * inv};
      *reinterpret_cast<f32x2*>(wrow + mt * 16 + 4 * g) = lo2;
      *reinterpret_cast<f32x2*>(wrow + mt * 16 + 4 * g + 2) = hi2;
    }
    if (g == 0) {
      wrow[D] = m_run * kLn2;
      wrow[D + 1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// BF16 cache: K and V tiles stream into an LDS ring with direct-to-LDS buffer
// loads (gfx950 16-byte LDS DMA). Each load instruction moves whole rows:
// lane l of instruction i fetches row i*RPI + l/CPR of the tile, and the
// 16-byte chunk (l % CPR) ^ row of it, so the tile lands in LDS row-major
// with the chunks of row r XOR-permuted by r. Reading K as the MFMA A
// operand (16 rows, one chunk each) then hits 16 different bank groups, and
// V is read transposed with ds_read_b64_tr_b16. No VGPRs hold data in
// flight, so the ring depth is set by LDS alone; the waits on the DMA are
// explicit (the compiler does not track LDS-DMA writes).
template <int D>
struct LdsTraits {
  static constexpr int RB = 2 * D;              // bytes of one (token, head) row
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;          // rows per load instruction (1..8)
  static constexpr int NI = 16 / RPI;           // load instructions per 16-token tile
  static constexpr int TILE = 16 * RB;          // bytes of one K or V tile
#ifndef PKD_LDS_NBUF128
#define PKD_LDS_NBUF128 1
#endif
  static constexpr int NBUF = D <= 64 ? 4 : (D == 128 ? PKD_LDS_NBUF128 : (D == 256 ? 2 : 1));
  static constexpr int SLOT = 2 * TILE;         // K tile + V tile
  static constexpr int WAIT = (2 * NBUF - 1) * NI;   // DMA loads allowed in flight at a read
};

// s_waitcnt that waits for vmcnt <= N only (expcnt / lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Balanced ("stream") partition of one launch's work. A row is a (sequence,
// kv head, chunk of up to 16 q heads) triple; row (b, k) has n_b tiles, the
// 16-key tiles overlapping the sequence's attended keys. The rows are laid end
// to end, sequence-major, into one index space of T tiles; wave w of the P
// launched waves takes tiles [w*c, (w+1)*c) with c = max(ceil(T/P), c_min) and
// c_min = ceil(n_bound / (S - 1)) for the host's bound n_bound on n_b. A wave
// thus covers one or more row pieces, each a contiguous key range; the piece
// of row r starting at flat tile f goes to workspace slot
// floor(f/c) - floor(start(r)/c) <= S - 1. The wave that ends a row marks the
// row's later slots empty. With S == 1, wave w takes row w whole. Every wave
// gets the same number of tiles whatever the length mix of the batch.

__device__ __forceinline__ uint32_t row_tiles(uint32_t L, uint32_t window) {
  if (L == 0) return 0;
  const uint32_t lo = (window > 0 && L > window) ? L - window : 0u;
  return (L + 15) / 16 - lo / 16;
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

struct RowLoc {
  uint32_t b, kh, n, start;     // sequence, kv-head/chunk index, tiles, flat start of the row
};

// Total tiles T of the launch (all rows of all sequences).
__device__ __forceinline__ uint32_t total_tiles(const DecodeArgs& a, uint32_t rows_per_seq) {
  uint32_t tot = 0;
  for (uint32_t b0 = 0; b0 < a.num_seqs; b0 += 64) {
    const uint32_t bb = b0 + threadIdx.x;
    const int32_t Ls = bb < a.num_seqs ? a.seq_lens[bb] : 0;
    const uint32_t t = row_tiles(Ls > 0 ? uint32_t(Ls) : 0u, a.window) * rows_per_seq;
    tot += __shfl(wave_scan(t), 63, 64);
  }
  return tot;
}

// The row holding flat tile `pos` (pos < T).
__device__ __forceinline__ RowLoc find_row(const DecodeArgs& a, uint32_t pos,
                                           uint32_t rows_per_seq) {
  uint32_t base = 0;
  for (uint32_t b0 = 0; b0 < a.num_seqs; b0 += 64) {
    const uint32_t bb = b0 + threadIdx.x;
    const int32_t Ls = bb < a.num_seqs ? a.seq_lens[bb] : 0;
    const uint32_t n = row_tiles(Ls > 0 ? uint32_t(Ls) : 0u, a.window);
    const uint32_t incl = wave_scan(n * rows_per_seq);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(base + incl > pos);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const uint32_t nl = __shfl(n, l, 64);
      const uint32_t excl = __shfl(incl - n * rows_per_seq, l, 64);
      const uint32_t kh = (pos - base - excl) / nl;
      return RowLoc{b0 + l, kh, nl, base + excl + kh * nl};
    }
    base += __shfl(incl, 63, 64);
  }
  return RowLoc{a.num_seqs, 0, 0, base};
}

template <int D>
struct StreamLds {
  __attribute__((aligned(1024))) uint8_t ring[LdsTraits<D>::NBUF * LdsTraits<D>::SLOT];
};

// One row piece: tiles [tau0, tau1) of row (b, kh), partial state to `slot`.
template <int D>
__device__ __forceinline__ void run_piece(const DecodeArgs& a, StreamLds<D>& sh, uint32_t b,
                                          uint32_t kh, uint32_t tau0, uint32_t tau1,
                                          uint32_t slot, bool last, uint32_t L) {
  using T = LdsTraits<D>;
  constexpr int NBUF = T::NBUF;
  const int lane = threadIdx.x;
  const int g = lane >> 4;
  const int n = lane & 15;
  const uint32_t kvh = kh / a.head_chunks, hc = kh % a.head_chunks;

  const uint32_t lo = (a.window > 0 && L > a.window) ? L - a.window : 0u;
  const uint32_t tpp = a.block_size / 16;
  const uint32_t t0 = lo / 16 + tau0, t1 = lo / 16 + tau1;   // tiles of the sequence
  const uint32_t pa = t0 / tpp, pb = (t1 + tpp - 1) / tpp;

  const uint32_t head_in_group = hc * 16 + n;
  const bool head_ok = head_in_group < a.group;
  const uint32_t qh = kvh * a.group + head_in_group;
  float* const wbase = a.ws + (uint64_t(b) * a.num_q_heads + qh) * a.num_splits * (D + 2);
  const int32_t* bt = a.block_tables + uint64_t(b) * a.max_blocks;

  // q as the B operand of the QK MFMAs: column n = head, dims 32c + 8g .. +8;
  // issued ahead of the tile loads, which only ever wait for later loads.
  bf16x8 qf[D / 32];
  {
    const uint16_t* qrow = a.q + uint64_t(b) * a.q_stride + uint64_t(qh) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head_ok) v = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * g);
      qf[c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  typedef __attribute__((address_space(3))) void lds_void;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_u8* const ring3 = (lds_u8*)(sh.ring);
  const int ld_row = lane / T::CPR;                  // + i * RPI
  const int ld_pos = lane % T::CPR;

  f32x4 acc[D / 16];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  // Segments of up to 64 pages: the block-table entries of a segment sit in
  // one VGPR (entry per lane); the DMA ring restarts at every segment.
  for (uint32_t cp = pa; cp < pb; cp += 64) {
    const uint32_t cpe = min(cp + 64, pb);
    const int32_t bt_reg = (cp + lane < cpe) ? bt[cp + lane] : 0;
    const uint32_t ct0 = max(cp * tpp, t0);
    const uint32_t ct1 = min(cpe * tpp, t1);

    auto issue = [&](int s, int kv, uint32_t t) {
      const bool live = t < ct1;
      const uint32_t page = min(t / tpp, cpe - 1);
      const uint32_t phys = uint32_t(__builtin_amdgcn_readlane(bt_reg, int(page - cp)));
      const uint8_t* pool = kv ? a.v_cache : a.k_cache;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(pool + uint64_t(phys) * a.page_bytes), 0,
          live ? int(a.page_bytes) : 0, 0x00020000);
      const uint32_t off0 = (t % tpp) * 16;
#pragma unroll
      for (int i = 0; i < T::NI; ++i) {
        const int row = i * T::RPI + ld_row;
        const int chunk = ld_pos ^ (row % T::CPR);
        const int voff = int(((off0 + row) * a.num_kv_heads + kvh) * T::RB + chunk * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (lds_void*)(ring3 + s * T::SLOT + kv * T::TILE + i * 1024), 16, voff, 0, 0, 2);
      }
    };

#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      issue(s, 0, ct0 + s);
      issue(s, 1, ct0 + s);
    }

    for (uint32_t tb = ct0; tb < ct1; tb += NBUF) {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        const uint32_t t = tb + s;               // t >= ct1: phantom tile, all keys masked
        const uint32_t tok0 = t * 16;
        const uint32_t khi = t < ct1 ? L : 0u;
        lds_u8* const kt = ring3 + s * T::SLOT;
        lds_u8* const vt = kt + T::TILE;

        // ---- S = K Q^T from the LDS tile (row n, chunk 4c+g swizzled by n)
        wait_vmcnt<T::WAIT>();
        wave_lds_fence();
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const int chunk = (4 * c + g) ^ (n % T::CPR);
          const u32x4 kv = *(lds_u32x4*)(kt + n * T::RB + chunk * 16);
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qf[c], sc,
                                                       0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(s, 0, t + NBUF);

        // ---- online softmax (lane: head n, tokens tok0 + 4g + j)
        float sv[4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t tok = tok0 + 4 * g + j;
          sv[j] = (tok >= lo && tok < khi) ? sc[j] * a.logit_scale : -__builtin_inff();
          mx = fmaxf(mx, sv[j]);
        }
        mx = max_over_rows(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        // the accumulator is rescaled only when some head's running max moved
        const bool rescale = __builtin_amdgcn_ballot_w64(m_new != m_run) != 0;
        m_run = m_new;
        uint32_t pbits[4];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(sv[j] - m_new);
          pbits[j] = f32_to_bf16_bits(p);
          psum += __uint_as_float(pbits[j] << 16);
        }
        l_run = l_run * alpha + psum;
        s16x4 pf;
#pragma unroll
        for (int j = 0; j < 4; ++j) pf[j] = short(pbits[j]);

        // ---- V tile: wait, zero the rows of masked tokens (partial tiles only)
        wait_vmcnt<T::WAIT>();
        wave_lds_fence();
        __builtin_amdgcn_sched_barrier(0);
        if (tok0 < lo || tok0 + 16 > khi) {
#pragma unroll
          for (int i = 0; i < T::NI; ++i) {
            const uint32_t tok = tok0 + i * T::RPI + ld_row;
            if (tok < lo || tok >= khi)
              *(lds_u32x4*)(vt + i * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
          }
          wave_lds_fence();
        }
        // ---- O^T += V^T P: lane supplies V[4g + n/4][16mt + 4(n%4) .. +4]. The
        // transposed reads are issued as inline asm: the compiler would otherwise
        // wait for every pending LDS-DMA load before each of them.
        {
          const int vtok = 4 * g + (n >> 2);
          const uint32_t vrow = uint32_t(uintptr_t(vt)) + vtok * T::RB + (n & 1) * 8;
          u32x2 vv[D / 16];
#pragma unroll
          for (int q4 = 0; q4 < D / 64; ++q4) {
            uint32_t ad[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int mt = 4 * q4 + u;
              ad[u] = vrow + (((2 * mt + ((n & 3) >> 1)) ^ (vtok % T::CPR)) * 16);
            }
            // four transposed reads and their wait in one statement: the outputs
            // exist only after the wait, so no consumer can be scheduled earlier
            asm volatile(
                "ds_read_b64_tr_b16 %0, %4\n\t"
                "ds_read_b64_tr_b16 %1, %5\n\t"
                "ds_read_b64_tr_b16 %2, %6\n\t"
                "ds_read_b64_tr_b16 %3, %7\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(vv[4 * q4]), "=&v"(vv[4 * q4 + 1]), "=&v"(vv[4 * q4 + 2]), "=&v"(vv[4 * q4 + 3])
                : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
                : "memory");
          }
          if (rescale) {
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) acc[mt] *= alpha;
          }
#pragma unroll
          for (int mt = 0; mt < D / 16; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv[mt]),
                                                                pf, acc[mt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(s, 1, t + NBUF);
      }
    }
    wait_vmcnt<0>();                               // the ring restarts with the next segment
    wave_lds_fence();
  }

  const float l_tot = sum_over_rows(l_run);
  if (head_ok) {
    float* wrow = wbase + uint64_t(slot) * (D + 2);
    const float inv = a.out_scale / l_tot;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      f32x2 lo2 = {acc[mt][0] * inv, acc[mt][1] * inv};
      f32x2 hi2 = {acc[mt][2] * inv, acc[mt][3] * inv};
      *reinterpret_cast<f32x2*>(wrow + mt * 16 + 4 * g) = lo2;
      *reinterpret_cast<f32x2*>(wrow + mt * 16 + 4 * g + 2) = hi2;
    }
    if (g == 0) {
      wrow[D] = m_run * kLn2;
      wrow[D + 1] = l_tot;
    }
    // the row ends in this piece: an end marker (l = -1) in the next slot
    // tells the combine to ignore that slot and all later ones
    if (last && g == 0 && slot + 1 < a.num_splits) {
      float* e = wbase + uint64_t(slot + 1) * (D + 2);
      e[D] = -__builtin_inff();
      e[D + 1] = -1.0f;
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void splitk_bf16_stream(DecodeArgs a) {
  __shared__ StreamLds<D> sh;
  const uint32_t R = a.num_kv_heads * a.head_chunks;          // rows per sequence
  if (a.num_splits == 1) {                                    // one wave per row
    const uint32_t b = blockIdx.x / R, kh = blockIdx.x % R;
    const int32_t Ls = a.seq_lens[b];
    const uint32_t L = Ls > 0 ? uint32_t(Ls) : 0u;
    const uint32_t n = row_tiles(L, a.window);
    if (n) run_piece<D>(a, sh, b, kh, 0, n, 0, true, L);
    return;
  }
  const uint32_t P = gridDim.x;
  if (a.num_seqs <= 64) {
    // one length per lane, loaded once: the tile counts, their prefix sums and
    // every row lookup come from these registers
    const uint32_t lane = threadIdx.x;
    const int32_t Ls = lane < a.num_seqs ? a.seq_lens[lane] : 0;
    const uint32_t L_l = Ls > 0 ? uint32_t(Ls) : 0u;
    const uint32_t n_l = row_tiles(L_l, a.window);
    const uint32_t incl = wave_scan(n_l * R);
    const uint32_t T = __shfl(incl, 63, 64);
    const uint32_t c = max((T + P - 1) / P, a.chunk_min);
    uint32_t pos = blockIdx.x * c;
    const uint32_t end = min(pos + c, T);
    while (pos < end) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(incl > pos);
      const int l = __builtin_ctzll(hit);
      const uint32_t n = __shfl(n_l, l, 64);
      const uint32_t excl = __shfl(incl, l, 64) - n * R;
      const uint32_t L = __shfl(L_l, l, 64);
      const uint32_t kh = (pos - excl) / n;
      const uint32_t start = excl + kh * n;
      const uint32_t tau1 = min(n, end - start);
      run_piece<D>(a, sh, uint32_t(l), kh, pos - start, tau1, pos / c - start / c,
                   start + n <= end, L);
      pos = start + tau1;
    }
    return;
  }
  const uint32_t T = total_tiles(a, R);
  const uint32_t c = max((T + P - 1) / P, a.chunk_min);
  uint32_t pos = blockIdx.x * c;
  const uint32_t end = min(pos + c, T);
  while (pos < end) {
    const RowLoc r = find_row(a, pos, R);
    const uint32_t tau0 = pos - r.start;
    const uint32_t tau1 = min(r.n, end - r.start);
    const uint32_t slot = pos / c - r.start / c;
    const int32_t Ls = a.seq_lens[r.b];
    run_piece<D>(a, sh, r.b, r.kh, tau0, tau1, slot, r.start + r.n <= end,
                 Ls > 0 ? uint32_t(Ls) : 0u);
    pos = r.start + tau1;
  }
}

// Combine: one workgroup of NT lanes per (sequence, q head); NT = 1024 when
// there are many slots. The (m, l) of all slots are read once into LDS (with
// the sequence length alongside) and turned into weights; then lane t
// accumulates the float2 column t % (D/2) over the slots i = t / (D/2)
// (mod KS), eight loads in flight, slots without keys not read, and the KS
// partial sums are added in a fixed order (deterministic).
template <int D, int NT>
__global__ __launch_bounds__(NT) void reduce_kernel(const float* ws, uint16_t* out,
                                                    const int32_t* seq_lens,
                                                    uint32_t num_q_heads, uint32_t num_splits) {
  constexpr int COLS = D / 2;                 // float2 columns of one split row
  constexpr int KS = NT / COLS;               // split lanes
  constexpr int NW = NT / 64;                 // waves
  extern __shared__ float wsh[];              // l (then weights) and m of every slot
  __shared__ float red[NW];
  __shared__ uint32_t stops[NW];
  __shared__ f32x2 part[KS][COLS];
  const int tid = threadIdx.x;
  const uint32_t bh = blockIdx.x;
  const uint32_t b = bh / num_q_heads;
  uint16_t* o = out + uint64_t(bh) * D;
  const float* base = ws + uint64_t(bh) * num_splits * (D + 2);

  // slot i counts if l_i > 0 and no earlier slot holds an end marker (l < 0)
  const int32_t L = seq_lens[b];
  uint32_t stop = num_splits;
  for (uint32_t i = tid; i < num_splits; i += NT) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(base + uint64_t(i) * (D + 2) + D);
    wsh[i] = ml[1];
    wsh[num_splits + i] = ml[0];
    if (ml[1] < 0.0f) stop = min(stop, i);
  }
  if (L <= 0) stop = 0;                       // empty sequence: zeros
#pragma unroll
  for (int of = 32; of >= 1; of >>= 1) stop = min(stop, uint32_t(__shfl_xor(int(stop), of, 64)));
  if ((tid & 63) == 0) stops[tid >> 6] = stop;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NW; ++k) stop = min(stop, stops[k]);
  float M = -__builtin_inff();
  for (uint32_t i = tid; i < stop; i += NT)
    if (wsh[i] > 0.0f) M = fmaxf(M, wsh[num_splits + i]);
  M = wave_max(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) M = fmaxf(M, red[k]);
  __syncthreads();
  if (M == -__builtin_inff()) {               // no slot holds a key
    for (int d = tid; d < D; d += NT) o[d] = 0;
    return;
  }
  float wsum = 0.0f;
  for (uint32_t i = tid; i < num_splits; i += NT) {
    const float l = wsh[i];
    const float w = (i < stop && l > 0.0f)
                        ? l * __builtin_amdgcn_exp2f((wsh[num_splits + i] - M) * kLog2e) : 0.0f;
    wsh[i] = w;
    wsum += w;
  }
  wsum = wave_sum(wsum);
  if ((tid & 63) == 0) red[tid >> 6] = wsum;
  __syncthreads();
  wsum = 0.0f;
#pragma unroll
  for (int k = 0; k < NW; ++k) wsum += red[k];

  const int col = tid % COLS, ks = tid / COLS;
  f32x2 acc = {0.0f, 0.0f};
  for (uint32_t i0 = ks; i0 < stop; i0 += 8 * KS) {
    // eight slots per round; a slot without keys is not read (the weight is
    // the same for every lane of a wave when D >= 128)
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
  part[ks][col] = acc;
  __syncthreads();
  if (tid < COLS) {
    f32x2 sum = part[0][tid];
#pragma unroll
    for (int k = 1; k < KS; ++k) sum += part[k][tid];
    const float inv = 1.0f / fmaxf(wsum, 1e-20f);
    const uint32_t packed = pack_bf16x2(sum[0] * inv, sum[1] * inv);
    *reinterpret_cast<uint32_t*>(o + 2 * tid) = packed;
  }
}

static int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : kLaunch;
}

// Waves the stream kernel launches on the current device: all resident at
// once (at most the occupancy), cached per device and head_dim.
static uint64_t stream_capacity(uint32_t head_dim) {
  static uint64_t cache[64][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int di = head_dim == 64 ? 0 : head_dim == 128 ? 1 : head_dim == 256 ? 2 : 3;
  if (cache[dev][di]) return cache[dev][di];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  hipError_t e = hipErrorInvalidValue;
  switch (head_dim) {
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, splitk_bf16_stream<64>, 64, 0); break;
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, splitk_bf16_stream<128>, 64, 0); break;
    case 256: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, splitk_bf16_stream<256>, 64, 0); break;
    case 512: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, splitk_bf16_stream<512>, 64, 0); break;
  }
  if (e != hipSuccess || per_cu <= 0 || cus <= 0) return 0;
#ifndef PKD_STREAM_WAVES_PER_CU
#define PKD_STREAM_WAVES_PER_CU 4
#endif
  // four long waves per CU stream better than more, shorter ones; the count is
  // a multiple of the CU count so that every CU gets the same work
  if (per_cu > PKD_STREAM_WAVES_PER_CU) per_cu = PKD_STREAM_WAVES_PER_CU;
  cache[dev][di] = uint64_t(per_cu) * uint64_t(cus);
  return cache[dev][di];
}

template <int FMT>
static int launch_splitk(DecodeArgs a, uint32_t num_seqs, uint32_t head_dim,
                         hipStream_t stream) {
  a.num_seqs = num_seqs;
  const uint64_t grid = uint64_t(num_seqs) * a.num_kv_heads * a.head_chunks * a.num_splits;
  if (grid > 0x7FFFFFFFull) return kUnsupported;
  const dim3 gd = dim3(uint32_t(grid)), bd = dim3(64);
  if (FMT == kBf16) {
    const uint32_t rows = num_seqs * a.num_kv_heads * a.head_chunks;
    uint32_t tile_bound = a.max_blocks * (a.block_size / 16);
    if (a.window > 0) tile_bound = min(tile_bound, (a.window + 14) / 16 + 1);
    a.chunk_min = a.num_splits > 1 ? (tile_bound + a.num_splits - 2) / (a.num_splits - 1) : 1;
    uint64_t waves = rows;
    if (a.num_splits > 1) {
      waves = uint64_t(rows) * a.num_splits;
      const uint64_t cap = stream_capacity(head_dim);
      if (cap && waves > cap) waves = cap;
    }
    const dim3 sgd = dim3(uint32_t(waves));
    switch (head_dim) {
      case 64: hipLaunchKernelGGL(splitk_bf16_stream<64>, sgd, bd, 0, stream, a); break;
      case 128: hipLaunchKernelGGL(splitk_bf16_stream<128>, sgd, bd, 0, stream, a); break;
      case 256: hipLaunchKernelGGL(splitk_bf16_stream<256>, sgd, bd, 0, stream, a); break;
      case 512: hipLaunchKernelGGL(splitk_bf16_stream<512>, sgd, bd, 0, stream, a); break;
      default: return kUnsupported;
    }
    return launch_status();
  }
  switch (head_dim) {
    case 64: hipLaunchKernelGGL((splitk_kernel<FMT, 64>), gd, bd, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((splitk_kernel<FMT, 128>), gd, bd, 0, stream, a); break;
    case 256: hipLaunchKernelGGL((splitk_kernel<FMT, 256>), gd, bd, 0, stream, a); break;
    case 512: hipLaunchKernelGGL((splitk_kernel<FMT, 512>), gd, bd, 0, stream, a); break;
    default: return kUnsupported;
  }
  return launch_status();
}

static DecodeArgs make_args(const uint16_t* q, const void* kc, const void* vc, float* ws,
                            const int32_t* bt, const int32_t* lens, uint32_t max_blocks,
                            uint32_t Hq, uint32_t Hkv, uint32_t bs, float logit_scale,
                            float out_scale, uint32_t S, uint32_t q_stride, uint64_t page_bytes,
                            uint64_t data_section, uint32_t window) {
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
  a.head_chunks = head_chunks(a.group);
  a.block_size = bs;
  a.logit_scale = logit_scale;
  a.out_scale = out_scale;
  a.num_splits = S;
  a.pages_per_split = pages_per_split(max_blocks, bs, window, S);
  a.q_stride = q_stride;
  a.page_bytes = page_bytes;
  a.data_section = data_section;
  a.window = window;
  a.num_seqs = 0;
  a.chunk_min = 1;
  return a;
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
                           sliding_window);
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
                           0, sliding_window);
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
                           data_section_bytes, sliding_window);
  return launch_splitk<kNvfp4>(a, num_seqs, head_dim, stream);
}

extern "C" PKD_API int paged_decode_attn_reduce(const float* workspace, uint16_t* output,
                                                const int32_t* seq_lens, uint32_t num_q_heads,
                                                uint32_t head_dim, uint32_t num_splits,
                                                uint32_t num_seqs, hipStream_t stream) {
  if (num_seqs == 0) return kOk;
  int st = check_reduce(workspace, output, seq_lens, num_q_heads, head_dim, num_splits);
  if (st) return st;
  const uint64_t grid = uint64_t(num_seqs) * num_q_heads;
  if (grid > 0x7FFFFFFFull) return kUnsupported;
  const size_t lds = 2 * size_t(num_splits) * sizeof(float);
  const bool wide = num_splits >= 64;          // many slots: more lanes per (b, h)
  const dim3 gd = dim3(uint32_t(grid)), bd = dim3(wide ? 1024 : 256);
#define PKD_REDUCE(DD) \
  if (wide) hipLaunchKernelGGL((reduce_kernel<DD, 1024>), gd, bd, lds, stream, workspace, output, seq_lens, num_q_heads, num_splits); \
  else hipLaunchKernelGGL((reduce_kernel<DD, 256>), gd, bd, lds, stream, workspace, output, seq_lens, num_q_heads, num_splits);
  switch (head_dim) {
    case 64: PKD_REDUCE(64) break;
    case 128: PKD_REDUCE(128) break;
    case 256: PKD_REDUCE(256) break;
    case 512: PKD_REDUCE(512) break;
    default: return kUnsupported;
  }
#undef PKD_REDUCE
  return launch_status();
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
    default: return "unknown status";
  }
}
