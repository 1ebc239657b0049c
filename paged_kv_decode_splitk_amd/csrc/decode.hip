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
  static constexpr int RS = D + 8;                          // LDS row stride (elements)
  static constexpr int ROW_BYTES = D * kElemBits / 8;       // bytes of one (token, head) row
};

// Raw bytes of one lane's share of a K or V tile.
template <int FMT, int D>
struct RawTile {
  u32x4 d[Traits<FMT, D>::NLOAD];
  uint32_t s[Traits<FMT, D>::NLOAD];     // NVFP4 group-scale bytes
};

template <int FMT, int D>
__device__ __forceinline__ void load_tile(RawTile<FMT, D>& t, const uint8_t* pool,
                                          const DecodeArgs& a, uint32_t phys, uint32_t off,
                                          uint32_t kvh, int g) {
  using T = Traits<FMT, D>;
  const uint64_t page = uint64_t(phys) * a.page_bytes;
  const uint64_t rowidx = uint64_t(off) * a.num_kv_heads + kvh;   // (offset, head) row
  const uint8_t* row = pool + page + rowidx * T::ROW_BYTES;
#pragma unroll
  for (int r = 0; r < T::NLOAD; ++r) {
    const int e0 = r * 4 * T::E + g * T::E;                        // first element
    const uint8_t* p = row + (e0 * T::kElemBits) / 8;
    if constexpr (T::kLoadBytes == 16) {
      t.d[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    } else {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
      t.d[r][0] = v[0];
      t.d[r][1] = v[1];
    }
    if constexpr (FMT == kNvfp4) {
      const uint8_t* sp = pool + page + a.data_section + rowidx * (D / 16) + e0 / 16;
      if constexpr (T::E == 32) t.s[r] = *reinterpret_cast<const uint16_t*>(sp);
      else t.s[r] = *sp;
    }
  }
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 from the exponent / mantissa bits
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
  bits |= (c & 8u) << 28;
  return __uint_as_float(bits);
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
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float lo = e4m3_to_f32((word >> (16 * h)) & 0xFFu);
        const float hi = e4m3_to_f32((word >> (16 * h + 8)) & 0xFFu);
        out[2 * w + h] = pack_bf16x2(lo, hi);      // exact: codes fit BF16
      }
    }
    return __builtin_bit_cast(bf16x8, out);
  } else {
    // 8 codes = one 32-bit word; group scale = byte f/2 of the lane's scales
    const uint32_t word = t.d[r][f];
    const float S = e4m3_to_f32((t.s[r] >> (8 * (f >> 1))) & 0xFFu);
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = e2m1_value((word >> (8 * i)) & 0xFu) * S;
      const float hi = e2m1_value((word >> (8 * i + 4)) & 0xFu) * S;
      out[i] = pack_bf16x2(lo, hi);                // exact: <= 6 significant bits
    }
    return __builtin_bit_cast(bf16x8, out);
  }
}

template <int FMT, int D>
__global__ __launch_bounds__(64) void splitk_kernel(DecodeArgs a) {
  using T = Traits<FMT, D>;
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

  const uint32_t tpp = bs / 16;                              // tiles per page
  const uint32_t t0 = max(pa * tpp, lo / 16);
  const uint32_t t1 = min(pb * tpp, (L + 15) / 16);
  const int32_t* bt = a.block_tables + uint64_t(b) * a.max_blocks;

  // block-table entries of the split, 64 at a time, one per lane
  uint32_t bt_base = pa;
  int32_t bt_reg = (pa + lane < pb) ? bt[pa + lane] : 0;
  auto phys_of = [&](uint32_t page) -> uint32_t {
    if (page >= bt_base + 64) {
      bt_base = page;
      bt_reg = (page + lane < pb) ? bt[page + lane] : 0;
    }
    return uint32_t(__builtin_amdgcn_readlane(bt_reg, int(page - bt_base)));
  };

  f32x4 acc[D / 16];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  RawTile<FMT, D> kn, vn;
  {
    const uint32_t page = t0 / tpp, off = (t0 % tpp) * 16 + n;
    const uint32_t phys = phys_of(page);
    load_tile<FMT, D>(kn, a.k_cache, a, phys, off, kvh, g);
    load_tile<FMT, D>(vn, a.v_cache, a, phys, off, kvh, g);
  }

  for (uint32_t t = t0; t < t1; ++t) {
    RawTile<FMT, D> kt = kn, vt = vn;
    if (t + 1 < t1) {
      const uint32_t page = (t + 1) / tpp, off = ((t + 1) % tpp) * 16 + n;
      const uint32_t phys = phys_of(page);
      load_tile<FMT, D>(kn, a.k_cache, a, phys, off, kvh, g);
      load_tile<FMT, D>(vn, a.v_cache, a, phys, off, kvh, g);
    }
    const uint32_t tok0 = t * 16;

    // ---- S = K Q^T
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < T::NFRAG; ++c) {
      const bf16x8 kf = dequant_frag<FMT, D>(kt, c / T::MPER, c % T::MPER);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], s, 0, 0, 0);
    }

    // ---- online softmax (lane: head n, tokens tok0 + 4g + j)
    float sv[4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t tok = tok0 + 4 * g + j;
      sv[j] = (tok >= lo && tok < L) ? s[j] * a.logit_scale : -__builtin_inff();
      mx = fmaxf(mx, sv[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);                   // finite: the tile holds a key
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

    // ---- V tile -> LDS rows (token n of the tile), masked tokens as zeros
    {
      const uint32_t tok = tok0 + n;
      const bool ok = tok >= lo && tok < L;
      uint16_t* dst = vlds + n * T::RS;
#pragma unroll
      for (int r = 0; r < T::NLOAD; ++r) {
#pragma unroll
        for (int f = 0; f < T::MPER; ++f) {
          u32x4 v = __builtin_bit_cast(u32x4, dequant_frag<FMT, D>(vt, r, f));
          if (!ok) v = u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(dst + r * 4 * T::E + g * T::E + 8 * f) = v;
        }
      }
    }
    __syncthreads();

    // ---- O^T += V^T P  (A: V^T rows = dims, k = tokens 4g..4g+3)
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      s16x4 vf;
#pragma unroll
      for (int j = 0; j < 4; ++j) vf[j] = short(vlds[(4 * g + j) * T::RS + mt * 16 + n]);
      f32x4 c = acc[mt] * alpha;
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, c, 0, 0, 0);
    }
    __syncthreads();
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

// Combine: one wavefront per (sequence, q head).
template <int D>
__global__ __launch_bounds__(64) void reduce_kernel(const float* ws, uint16_t* out,
                                                    const int32_t* seq_lens, uint32_t num_q_heads,
                                                    uint32_t num_splits) {
  extern __shared__ float wsh[];                    // num_splits weights
  const int lane = threadIdx.x;
  const uint32_t bh = blockIdx.x;
  const uint32_t b = bh / num_q_heads;
  uint16_t* o = out + uint64_t(bh) * D;
  const float* base = ws + uint64_t(bh) * num_splits * (D + 2);
  constexpr int PER = D / 64;

  float M = -__builtin_inff();
  if (seq_lens[b] > 0) {
    for (uint32_t i = lane; i < num_splits; i += 64) {
      const float l = base[uint64_t(i) * (D + 2) + D + 1];
      if (l > 0.0f) M = fmaxf(M, base[uint64_t(i) * (D + 2) + D]);
    }
    M = wave_max(M);
  }
  if (M == -__builtin_inff()) {                     // empty sequence: zeros
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k * 64 + lane] = 0;
    return;
  }
  float wsum = 0.0f;
  for (uint32_t i = lane; i < num_splits; i += 64) {
    const float l = base[uint64_t(i) * (D + 2) + D + 1];
    const float m = base[uint64_t(i) * (D + 2) + D];
    const float w = l > 0.0f ? l * __builtin_amdgcn_exp2f((m - M) * kLog2e) : 0.0f;
    wsh[i] = w;
    wsum += w;
  }
  wsum = wave_sum(wsum);
  __syncthreads();
  float accv[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) accv[k] = 0.0f;
  for (uint32_t i = 0; i < num_splits; ++i) {
    const float w = wsh[i];
    if (w == 0.0f) continue;
    const float* oi = base + uint64_t(i) * (D + 2);
#pragma unroll
    for (int k = 0; k < PER; ++k) accv[k] = fmaf(w, oi[k * 64 + lane], accv[k]);
  }
  const float inv = 1.0f / fmaxf(wsum, 1e-20f);
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k * 64 + lane] = f32_to_bf16_bits(accv[k] * inv);
}

static int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? kOk : kLaunch;
}

template <int FMT>
static int launch_splitk(const DecodeArgs& a, uint32_t num_seqs, uint32_t head_dim,
                         hipStream_t stream) {
  const uint64_t grid = uint64_t(num_seqs) * a.num_kv_heads * a.head_chunks * a.num_splits;
  if (grid > 0x7FFFFFFFull) return kUnsupported;
  const dim3 gd = dim3(uint32_t(grid)), bd = dim3(64);
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
  const size_t lds = size_t(num_splits) * sizeof(float);
  const dim3 gd = dim3(uint32_t(grid)), bd = dim3(64);
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(reduce_kernel<64>, gd, bd, lds, stream, workspace, output, seq_lens, num_q_heads, num_splits); break;
    case 128: hipLaunchKernelGGL(reduce_kernel<128>, gd, bd, lds, stream, workspace, output, seq_lens, num_q_heads, num_splits); break;
    case 256: hipLaunchKernelGGL(reduce_kernel<256>, gd, bd, lds, stream, workspace, output, seq_lens, num_q_heads, num_splits); break;
    case 512: hipLaunchKernelGGL(reduce_kernel<512>, gd, bd, lds, stream, workspace, output, seq_lens, num_q_heads, num_splits); break;
    default: return kUnsupported;
  }
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
